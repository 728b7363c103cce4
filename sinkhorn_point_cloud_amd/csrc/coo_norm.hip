// coo_norm.hip -- Sinkhorn normalisation of a sparse plan on its stored
// support (CUDA-APML page, Abstract and Innovation: Sinkhorn normalisation run
// directly in COO form).
//
// Per pair, with lv_k = log vals_k over the stored entries, row scalings alpha
// and column scalings beta start at 0 and each round sets
//     alpha_i = log a_i - LSE_{k in row i}(lv_k + beta_{col k})
//     beta_j  = log b_j - LSE_{k in col j}(lv_k + alpha_{row k})
// (a row or column with no finite term keeps 0); the values become
// exp(lv_k + alpha_i + beta_j), whose column sums are b exactly after every
// round and whose row sums approach a.
//
// Rows are runs of the row-sorted plan; columns are runs of its transpose (the
// plan extracted with the roles of the clouds exchanged, which the symmetric
// evaluation of log P makes entry-for-entry identical, values included).  Row
// updates read the plan, column updates read the transpose, and both are
// rescaled in place with the same arithmetic, so they stay each other's
// transpose bit for bit.  The transpose is checked first: per pair, the entry
// counts and a checksum (the sum mod 2^64 of a 64-bit mix of each entry's row,
// column and value bits, independent of the order) must agree.  One wave
// reduces one row or one column in a fixed order: no atomics on values,
// deterministic results.
#include "common.h"

namespace sk {
namespace {

constexpr int kSegsPerGroup = 4;   // one wave per row or column

// SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", 2014): a bijective 64-bit mix
__device__ __forceinline__ uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

// sums[b] += sum over the pair's entries of mix(row, col, value bits), where
// (ri, ci) are the entry's row and column in the plan's orientation
__global__ __launch_bounds__(256) void checksum_kernel(const int32_t *__restrict__ ri,
                                                       const int32_t *__restrict__ ci,
                                                       const float *__restrict__ v,
                                                       const int64_t *__restrict__ offs,
                                                       uint64_t *__restrict__ sums)
{
    __shared__ uint64_t part[256 / kWave];
    const int b = blockIdx.y;
    const int64_t lo = offs[b], hi = offs[b + 1];
    uint64_t acc = 0;
    for (int64_t k = lo + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < hi;
         k += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t rc = ((uint64_t)(uint32_t)ri[k] << 32) | (uint32_t)ci[k];
        acc += mix64(rc ^ mix64((uint64_t)__float_as_uint(v[k]) + 0x9e3779b97f4a7c15ull));
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        acc += __shfl_xor(acc, off, kWave);
    if (lane_id() == 0)
        part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t t = 0;
        for (int w = 0; w < 256 / kWave; ++w)
            t += part[w];
        atomicAdd((unsigned long long *)&sums[b], (unsigned long long)t);
    }
}

// *bad = number of pairs whose entry counts or checksums differ
__global__ __launch_bounds__(256) void compare_kernel(const int64_t *__restrict__ offs,
                                                      const int64_t *__restrict__ t_offs,
                                                      const uint64_t *__restrict__ sums, int B,
                                                      int *__restrict__ bad)
{
    __shared__ int cnt;
    if (threadIdx.x == 0)
        cnt = 0;
    __syncthreads();
    int mine = 0;
    for (int b = threadIdx.x; b < B; b += 256)
        mine += (offs[b + 1] - offs[b] != t_offs[b + 1] - t_offs[b]) || (sums[b] != sums[B + b]);
    if (mine)
        atomicAdd(&cnt, mine);
    __syncthreads();
    if (threadIdx.x == 0)
        *bad = cnt;
}

__global__ void zero_u64(uint64_t *__restrict__ p, int count)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count)
        p[i] = 0;
}

// lv = log vals, four entries per thread: with 16-byte accesses when both
// arrays are 16-byte aligned (vec), the last nnz % 4 entries one at a time
__global__ void log_kernel(const float *__restrict__ vals, int64_t nnz, float *__restrict__ lv,
                           bool vec)
{
    const int64_t k = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
    if (vec && k + 4 <= nnz) {
        const float4 v = *reinterpret_cast<const float4 *>(vals + k);
        *reinterpret_cast<float4 *>(lv + k) = make_float4(logf(v.x), logf(v.y), logf(v.z),
                                                          logf(v.w));
    } else {
        for (int64_t q = k; q < k + 4 && q < nnz; ++q)
            lv[q] = logf(vals[q]);
    }
}

// One scaling update per segment (a row of the plan or a row of the transpose,
// i.e. a column of the plan): out_s = lw_s - LSE over the segment's entries k
// of (lv_k + other_{partner_k}).
// Two segments per wave, kSegLanes lanes each: a row holds a few hundred
// entries, so the per-segment work (the shift, the reductions, the logarithm)
// is a large share, and two segments share those instructions.
constexpr int kSegLanes = 32;

// Sum and maximum over the kSegLanes lanes of a segment (butterfly, fixed order).
__device__ __forceinline__ double seg_sum(double v)
{
#pragma unroll
    for (int off = kSegLanes / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ double seg_max(double v)
{
#pragma unroll
    for (int off = kSegLanes / 2; off > 0; off >>= 1)
        v = fmax(v, __shfl_xor(v, off, kWave));
    return v;
}

__global__ __launch_bounds__(kSegsPerGroup *kWave) void scale_pass(
    const int64_t *__restrict__ sb, const int64_t *__restrict__ se,
    const int32_t *__restrict__ partner, const float *__restrict__ lv,
    const double *__restrict__ other, int count, int other_count, const double *__restrict__ lw,
    double *__restrict__ out)
{
    const int b = blockIdx.y;
    const int lane = lane_id();
    const int sl = lane % kSegLanes;   // lane within the segment
    const int s = (blockIdx.x * kSegsPerGroup + wave_id_uniform()) * (kWave / kSegLanes) +
                  lane / kSegLanes;
    if (s >= count)
        return;   // whole segments: the shuffles below stay inside a segment's lanes
    const size_t si = (size_t)b * count + s;
    const int64_t lo = sb[si], hi = se[si];
    const double *ob = other + (size_t)b * other_count;
    auto term = [&](int64_t q) -> double {
        const int p = partner[q];
        if (p < 0 || p >= other_count)
            return -INFINITY;
        return (double)lv[q] + ob[p];
    };
    // Shifted pass: the segment's previous scaling puts its log-sum-exp near
    // M = lw - out (every scaling starts at 0), so the terms are summed against
    // that fixed shift, with no maximum per entry.  A sum outside [2^-40, 2^60]
    // (the shift was stale), a segment of zero weight or an empty one takes
    // the online form below instead.
    const double Msh = lw[si] - out[si];
    if (isfinite(Msh)) {   // uniform over the segment
        double Ssh = 0.0;
        int64_t q = lo + sl;
        // four entries per lane and step: their indices and values, then their
        // partners' scalings, are all in flight before the first is used
        for (; q + 3 * kSegLanes < hi; q += 4 * kSegLanes) {
            int pp[4];
            float lq[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                pp[u] = partner[q + u * kSegLanes];
                lq[u] = lv[q + u * kSegLanes];
            }
            double z[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                z[u] = pp[u] < 0 || pp[u] >= other_count ? -INFINITY : (double)lq[u] + ob[pp[u]];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                Ssh += (double)expf((float)(z[u] - Msh));
        }
        if (q + kSegLanes < hi) {   // two more, loaded together
            const double z0 = term(q), z1 = term(q + kSegLanes);
            Ssh += (double)expf((float)(z0 - Msh));
            Ssh += (double)expf((float)(z1 - Msh));
            q += 2 * kSegLanes;
        }
        for (; q < hi; q += kSegLanes)
            Ssh += (double)expf((float)(term(q) - Msh));
        Ssh = seg_sum(Ssh);
        if (Ssh >= 0x1p-40 && Ssh <= 0x1p60) {
            if (sl == 0)
                out[si] = lw[si] - (Msh + log(Ssh));
            return;
        }
    }
    // online form: each lane keeps (M, S) meaning S e^M over its entries, raising
    // M when a larger term arrives
    double M = -INFINITY, S = 0.0;
    auto add = [&](double z) {
        if (z > M) {
            S = S * (double)expf((float)(M - z)) + 1.0;
            M = z;
        } else if (z > -INFINITY) {
            S += (double)expf((float)(z - M));
        }
    };
    // two entries per lane and step (loaded before either is used), in order
    int64_t q = lo + sl;
    for (; q + kSegLanes < hi; q += 2 * kSegLanes) {
        const double z0 = term(q), z1 = term(q + kSegLanes);
        add(z0);
        add(z1);
    }
    if (q < hi)
        add(term(q));
    // merge the lanes: the segment's maximum, each lane's sum rescaled to it once,
    // then one sum (fixed order)
    const double Mw = seg_max(M);
    S = M > -INFINITY ? S * (double)expf((float)(M - Mw)) : 0.0;
    S = seg_sum(S);
    if (sl == 0)
        out[si] = Mw > -INFINITY ? lw[si] - (Mw + log(S)) : 0.0;
}

// vals_k <- exp(lv_k + alpha_{ri_k} + beta_{ci_k}) with (ri, ci) the entry's row
// and column in the plan's orientation (the same sum, in the same order, for
// the plan and for its transpose)
__global__ void apply_kernel(const int32_t *__restrict__ ri, const int32_t *__restrict__ ci,
                             const int64_t *__restrict__ offs, int n, int m,
                             const float *__restrict__ lv, const double *__restrict__ al,
                             const double *__restrict__ be, float *__restrict__ vals)
{
    const int b = blockIdx.y;
    const int64_t lo = offs[b], hi = offs[b + 1];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const double *alb = al + (size_t)b * n, *beb = be + (size_t)b * m;
    auto one = [&](int64_t k, int i, int j, float l) {
        if (i < 0 || i >= n || j < 0 || j >= m)
            return;
        vals[k] = expf((float)((double)l + alb[i] + beb[j]));
    };
    int64_t k = lo + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // four entries per thread and step, their loads in flight together
    for (; k + 3 * stride < hi; k += 4 * stride) {
        int i[4], j[4];
        float l[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            i[u] = ri[k + u * stride];
            j[u] = ci[k + u * stride];
            l[u] = lv[k + u * stride];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            one(k + u * stride, i[u], j[u], l[u]);
    }
    for (; k < hi; k += stride)
        one(k, ri[k], ci[k], lv[k]);
}

// |sum of the segment's values - weight| per row (of the plan or of the transpose)
__global__ __launch_bounds__(kSegsPerGroup *kWave) void marginal_pass(
    const int64_t *__restrict__ sb, const int64_t *__restrict__ se, const float *__restrict__ vals,
    int count, const float *__restrict__ w, double *__restrict__ part)
{
    const int b = blockIdx.y;
    const int s = blockIdx.x * kSegsPerGroup + wave_id_uniform();
    if (s >= count)
        return;
    const int lane = lane_id();
    const size_t si = (size_t)b * count + s;
    double acc = 0.0;
    for (int64_t q = sb[si] + lane; q < se[si]; q += kWave)
        acc += (double)vals[q];
    acc = wave_sum(acc);
    if (lane == 0)
        part[si] = fabs(acc - (w ? (double)w[si] : 1.0 / (double)count));
}

__global__ __launch_bounds__(256) void pair_err(const double *__restrict__ part, int count,
                                                float *__restrict__ err, int slot)
{
    __shared__ double sm[256];
    const int b = blockIdx.x;
    double acc = 0.0;
    for (int i = threadIdx.x; i < count; i += 256)
        acc += part[(size_t)b * count + i];
    sm[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < s)
            sm[threadIdx.x] += sm[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        err[2 * b + slot] = (float)sm[0];
}

__global__ void zero_f64(double *__restrict__ p, size_t count)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count)
        p[i] = 0.0;
}

}  // namespace

hipError_t launch_coo_check(const int32_t *rows, const int32_t *cols, const float *vals,
                            const int64_t *offs, const int32_t *t_rows, const int32_t *t_cols,
                            const float *t_vals, const int64_t *t_offs, int B, const CooNormWs &w,
                            hipStream_t st)
{
    hipLaunchKernelGGL(zero_u64, dim3(ceil_div(2 * B, 256)), dim3(256), 0, st, w.sums, 2 * B);
    hipLaunchKernelGGL(checksum_kernel, dim3(64, B), dim3(256), 0, st, rows, cols, vals, offs,
                       w.sums);
    // the transpose's entry (row j, column i) is the plan's (i, j)
    hipLaunchKernelGGL(checksum_kernel, dim3(64, B), dim3(256), 0, st, t_cols, t_rows, t_vals,
                       t_offs, w.sums + B);
    hipLaunchKernelGGL(compare_kernel, dim3(1), dim3(256), 0, st, offs, t_offs,
                       (const uint64_t *)w.sums, B, w.bad);
    return hipGetLastError();
}

hipError_t launch_coo_normalize(const int32_t *rows, const int32_t *cols, float *vals,
                                const int64_t *offs, const int32_t *t_rows, const int32_t *t_cols,
                                float *t_vals, const int64_t *t_offs, int B, int n, int m,
                                int64_t nnz, int iters, float *err, const float *a,
                                const float *b, const CooNormWs &w, hipStream_t st)
{
    const unsigned nb = (unsigned)((nnz + 1023) / 1024);   // log_kernel: 4 entries a thread
    if (nnz > 0) {
        auto a16 = [](const void *q1, const void *q2) {
            return (((uintptr_t)q1 | (uintptr_t)q2) & 15) == 0;
        };
        hipLaunchKernelGGL(log_kernel, dim3(nb), dim3(256), 0, st, (const float *)vals, nnz, w.lv,
                           a16(vals, w.lv));
        hipLaunchKernelGGL(log_kernel, dim3(nb), dim3(256), 0, st, (const float *)t_vals, nnz,
                           w.lvt, a16(t_vals, w.lvt));
    }
    const size_t cn = (size_t)B * m;
    const size_t rn = (size_t)B * n;
    hipLaunchKernelGGL(zero_f64, dim3((unsigned)((cn + 255) / 256)), dim3(256), 0, st, w.be, cn);
    hipLaunchKernelGGL(zero_f64, dim3((unsigned)((rn + 255) / 256)), dim3(256), 0, st, w.al, rn);
    const dim3 gr(ceil_div(n, kSegsPerGroup), B), gc(ceil_div(m, kSegsPerGroup), B);
    constexpr int kScaleSegs = kSegsPerGroup * (kWave / kSegLanes);   // segments per group
    const dim3 grs(ceil_div(n, kScaleSegs), B), gcs(ceil_div(m, kScaleSegs), B);
    const dim3 blk(kSegsPerGroup * kWave);
    for (int it = 0; it < iters; ++it) {
        hipLaunchKernelGGL(scale_pass, grs, blk, 0, st, (const int64_t *)w.rb, (const int64_t *)w.re,
                           cols, (const float *)w.lv, (const double *)w.be, n, m,
                           (const double *)w.la, w.al);
        hipLaunchKernelGGL(scale_pass, gcs, blk, 0, st, (const int64_t *)w.cb, (const int64_t *)w.ce,
                           t_cols, (const float *)w.lvt, (const double *)w.al, m, n,
                           (const double *)w.lb, w.be);
    }
    if (iters > 0) {
        hipLaunchKernelGGL(apply_kernel, dim3(256, B), dim3(256), 0, st, rows, cols, offs, n, m,
                           (const float *)w.lv, (const double *)w.al, (const double *)w.be, vals);
        hipLaunchKernelGGL(apply_kernel, dim3(256, B), dim3(256), 0, st, t_cols, t_rows, t_offs, n,
                           m, (const float *)w.lvt, (const double *)w.al, (const double *)w.be,
                           t_vals);
    }
    if (err) {
        hipLaunchKernelGGL(marginal_pass, gr, blk, 0, st, (const int64_t *)w.rb,
                           (const int64_t *)w.re, (const float *)vals, n, a, w.row_part);
        hipLaunchKernelGGL(marginal_pass, gc, blk, 0, st, (const int64_t *)w.cb,
                           (const int64_t *)w.ce, (const float *)t_vals, m, b, w.col_part);
        hipLaunchKernelGGL(pair_err, dim3(B), dim3(256), 0, st, (const double *)w.row_part, n,
                           err, 0);
        hipLaunchKernelGGL(pair_err, dim3(B), dim3(256), 0, st, (const double *)w.col_part, m,
                           err, 1);
    }
    return hipGetLastError();
}

}  // namespace sk

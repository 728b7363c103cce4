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
// evaluation of log P makes entry-for-entry identical), mapped back to plan
// entries once by binary search inside each row.  One wave reduces one row or
// one column in a fixed order: no atomics on values, deterministic results.
#include "common.h"

namespace sk {
namespace {

constexpr int kSegsPerGroup = 4;   // one wave per row or column

__device__ __forceinline__ double wave_sum_d(double v)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

// perm[q] = plan entry holding (t_cols[q], t_rows[q]), or -1 (counted in *bad)
__global__ void perm_kernel(const int32_t *__restrict__ cols, const int32_t *__restrict__ t_rows,
                            const int32_t *__restrict__ t_cols, const int64_t *__restrict__ t_offs,
                            int n, int m, const int64_t *__restrict__ rb,
                            const int64_t *__restrict__ re, int64_t *__restrict__ perm,
                            int *__restrict__ bad)
{
    const int b = blockIdx.y;
    const int64_t lo = t_offs[b], hi = t_offs[b + 1];
    for (int64_t q = lo + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < hi;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int j = t_rows[q], i = t_cols[q];
        int64_t found = -1;
        if (i >= 0 && i < n && j >= 0 && j < m) {
            int64_t l = rb[(size_t)b * n + i], h = re[(size_t)b * n + i];
            while (l < h) {   // first entry of row i with column >= j
                const int64_t mid = l + (h - l) / 2;
                if (cols[mid] < j)
                    l = mid + 1;
                else
                    h = mid;
            }
            if (l < re[(size_t)b * n + i] && cols[l] == j)
                found = l;
        }
        perm[q] = found;
        if (found < 0)
            atomicAdd(bad, 1);
    }
}

__global__ void log_kernel(const float *__restrict__ vals, int64_t nnz, float *__restrict__ lv)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k < nnz)
        lv[k] = logf(vals[k]);
}

// One scaling update per segment (row of the plan or column of its transpose):
// out_s = lw_s - LSE over the segment of (lv_k + other_{partner}).
// ROW: entries k = begin..end of the plan, partner = cols[k];
// COL: entries q = begin..end of the transpose, k = perm[q], partner = t_cols[q].
template <bool ROW>
__global__ __launch_bounds__(kSegsPerGroup *kWave) void scale_pass(
    const int64_t *__restrict__ sb, const int64_t *__restrict__ se,
    const int32_t *__restrict__ partner, const int64_t *__restrict__ perm,
    const float *__restrict__ lv, const double *__restrict__ other, int count,
    int other_count, const double *__restrict__ lw, double *__restrict__ out)
{
    const int b = blockIdx.y;
    const int s = blockIdx.x * kSegsPerGroup + wave_id_uniform();
    if (s >= count)
        return;
    const int lane = lane_id();
    const size_t si = (size_t)b * count + s;
    const int64_t lo = sb[si], hi = se[si];
    const double *ob = other + (size_t)b * other_count;
    auto term = [&](int64_t q) -> double {
        const int64_t k = ROW ? q : perm[q];
        const int p = partner[q];
        if (k < 0 || p < 0 || p >= other_count)
            return -INFINITY;
        return (double)lv[k] + ob[p];
    };
    // one pass: each lane keeps (M, S) meaning S e^M over its entries, raising M
    // when a larger term arrives; lanes merge in a fixed order
    double M = -INFINITY, S = 0.0;
    for (int64_t q = lo + lane; q < hi; q += kWave) {
        const double z = term(q);
        if (z > M) {
            S = S * (double)expf((float)(M - z)) + 1.0;
            M = z;
        } else if (z > -INFINITY) {
            S += (double)expf((float)(z - M));
        }
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const double M2 = __shfl_xor(M, off, kWave), S2 = __shfl_xor(S, off, kWave);
        const double Mn = fmax(M, M2);
        if (Mn > -INFINITY)
            S = (M > -INFINITY ? S * (double)expf((float)(M - Mn)) : 0.0) +
                (M2 > -INFINITY ? S2 * (double)expf((float)(M2 - Mn)) : 0.0);
        M = Mn;
    }
    if (lane == 0)
        out[si] = M > -INFINITY ? lw[si] - (M + log(S)) : 0.0;
}

__global__ void apply_kernel(const int32_t *__restrict__ rows, const int32_t *__restrict__ cols,
                             const int64_t *__restrict__ offs, int n, int m,
                             const float *__restrict__ lv, const double *__restrict__ al,
                             const double *__restrict__ be, float *__restrict__ vals)
{
    const int b = blockIdx.y;
    const int64_t lo = offs[b], hi = offs[b + 1];
    for (int64_t k = lo + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < hi;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int i = rows[k], j = cols[k];
        if (i < 0 || i >= n || j < 0 || j >= m)
            continue;
        const double z = (double)lv[k] + al[(size_t)b * n + i] + be[(size_t)b * m + j];
        vals[k] = expf((float)z);
    }
}

// |sum of the segment's values - weight| per row or column
template <bool ROW>
__global__ __launch_bounds__(kSegsPerGroup *kWave) void marginal_pass(
    const int64_t *__restrict__ sb, const int64_t *__restrict__ se,
    const int64_t *__restrict__ perm, const float *__restrict__ vals, int count,
    const float *__restrict__ w, double *__restrict__ part)
{
    const int b = blockIdx.y;
    const int s = blockIdx.x * kSegsPerGroup + wave_id_uniform();
    if (s >= count)
        return;
    const int lane = lane_id();
    const size_t si = (size_t)b * count + s;
    double acc = 0.0;
    for (int64_t q = sb[si] + lane; q < se[si]; q += kWave) {
        const int64_t k = ROW ? q : perm[q];
        if (k >= 0)
            acc += (double)vals[k];
    }
    acc = wave_sum_d(acc);
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

__global__ void zero_i32(int *__restrict__ p)
{
    if (threadIdx.x == 0 && blockIdx.x == 0)
        *p = 0;
}

}  // namespace

hipError_t launch_coo_perm(const int32_t *cols, const int32_t *t_rows, const int32_t *t_cols,
                           const int64_t *t_offs, int B, int n, int m, const CooNormWs &w,
                           hipStream_t st)
{
    hipLaunchKernelGGL(zero_i32, dim3(1), dim3(64), 0, st, w.bad);
    hipLaunchKernelGGL(perm_kernel, dim3(256, B), dim3(256), 0, st, cols, t_rows, t_cols, t_offs,
                       n, m, (const int64_t *)w.rb, (const int64_t *)w.re, w.perm, w.bad);
    return hipGetLastError();
}

hipError_t launch_coo_normalize(const int32_t *rows, const int32_t *cols, float *vals,
                                const int64_t *offs, const int32_t *t_cols, int B, int n, int m,
                                int64_t nnz, int iters, float *err, const float *a,
                                const float *b, const CooNormWs &w, hipStream_t st)
{
    const unsigned nb = (unsigned)((nnz + 255) / 256);
    if (nnz > 0)
        hipLaunchKernelGGL(log_kernel, dim3(nb), dim3(256), 0, st, (const float *)vals, nnz, w.lv);
    const size_t cn = (size_t)B * m;
    hipLaunchKernelGGL(zero_f64, dim3((unsigned)((cn + 255) / 256)), dim3(256), 0, st, w.be, cn);
    const dim3 gr(ceil_div(n, kSegsPerGroup), B), gc(ceil_div(m, kSegsPerGroup), B);
    const dim3 blk(kSegsPerGroup * kWave);
    for (int it = 0; it < iters; ++it) {
        hipLaunchKernelGGL(scale_pass<true>, gr, blk, 0, st, (const int64_t *)w.rb,
                           (const int64_t *)w.re, cols, (const int64_t *)nullptr,
                           (const float *)w.lv, (const double *)w.be, n, m,
                           (const double *)w.la, w.al);
        hipLaunchKernelGGL(scale_pass<false>, gc, blk, 0, st, (const int64_t *)w.cb,
                           (const int64_t *)w.ce, t_cols, (const int64_t *)w.perm,
                           (const float *)w.lv, (const double *)w.al, m, n,
                           (const double *)w.lb, w.be);
    }
    if (iters > 0)
        hipLaunchKernelGGL(apply_kernel, dim3(256, B), dim3(256), 0, st, rows, cols, offs, n, m,
                           (const float *)w.lv, (const double *)w.al, (const double *)w.be, vals);
    if (err) {
        hipLaunchKernelGGL(marginal_pass<true>, gr, blk, 0, st, (const int64_t *)w.rb,
                           (const int64_t *)w.re, (const int64_t *)nullptr, (const float *)vals, n,
                           a, w.row_part);
        hipLaunchKernelGGL(marginal_pass<false>, gc, blk, 0, st, (const int64_t *)w.cb,
                           (const int64_t *)w.ce, (const int64_t *)w.perm, (const float *)vals, m,
                           b, w.col_part);
        hipLaunchKernelGGL(pair_err, dim3(B), dim3(256), 0, st, (const double *)w.row_part, n,
                           err, 0);
        hipLaunchKernelGGL(pair_err, dim3(B), dim3(256), 0, st, (const double *)w.col_part, m,
                           err, 1);
    }
    return hipGetLastError();
}

}  // namespace sk

// plan.hip -- passes over the transport plan at the final eps, never stored:
//     log P_ij = (f_i + g_j - C_ij)/eps + log a_i + log b_j,  C_ij = ||x_i - y_j||^2
// (the plan of the stabilised log-domain Sinkhorn solution, FlashSinkhorn
// summary, Methodologie 1), used for
//   - the transport cost   sum_ij P_ij C_ij;
//   - the thresholded sparse plan of the CUDA-APML page (Abstract, Innovation):
//     per pair the maximum of log P, a count of the entries at or above
//     max + log(rel_threshold) per row, a scan of the counts into offsets, and
//     the emission of (row, col, P) in row-major order.
//
// log P is evaluated in fp64 from the fp32 potentials and weights (fp64 FMA
// runs at the fp32 rate on this chip, and these passes run once per solve),
// so the threshold decision does not add fp32 rounding of the large
// potentials; P itself is returned as fp32.  The count and emit passes call the
// same evaluation on the same inputs, so their decisions agree bit for bit.
//
// Layout: one wave per row, lanes across columns (64 consecutive columns per
// step), so every wave reads contiguous keys and writes contiguous COO slices.
#include "common.h"

namespace sk {
namespace {

constexpr int kRowsPerGroup = 4;  // one wave per row

template <int DP> struct RowCtx {
    float x[DP];   // row point (exact fp32 value of the fp32 / bf16 input)
    double f, la;
};

template <typename T, int DP>
__device__ __forceinline__ double sq_dist(const float (&x)[DP], const T *y, int d)
{
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < DP; ++k) {
        if (k < d) {
            const double t = (double)x[k] - (double)Elem<T>::get(y, k);
            s = fma(t, t, s);
        }
    }
    return s;
}

__global__ void log_weights_kernel(const float *__restrict__ w, int count, size_t total,
                                   double *__restrict__ out)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total)
        return;
    if (!w) {
        out[i] = -log((double)count);
        return;
    }
    const float v = w[i];
    out[i] = v > 0.f ? log((double)v) : -INFINITY;
}

// log P_ij (nats) and C_ij for a row context and column j of one pair.  Written
// with explicit fma so that every pass evaluates it with the same roundings.
template <typename T, int DP>
__device__ __forceinline__ double log_plan(const RowCtx<DP> &r, const PlanArgs &p,
                                           const T *Yb, const float *gb, double lbj, int j,
                                           double *C)
{
    const double c = sq_dist<T, DP>(r.x, Yb + (size_t)j * p.d, p.d);
    *C = c;
    return fma((r.f + (double)gb[j]) - c, p.inv_eps, r.la) + lbj;
}

template <typename T, int DP>
__device__ void load_row(RowCtx<DP> &r, const PlanArgs &p, int b, int i)
{
    const T *x = (const T *)p.X + ((size_t)b * p.n + i) * p.d;
#pragma unroll
    for (int k = 0; k < DP; ++k)
        r.x[k] = k < p.d ? Elem<T>::get(x, k) : 0.f;
    r.f = (double)p.f[(size_t)b * p.n + i];
    r.la = p.la[(size_t)b * p.n + i];
}

// mode 0: cost  (row sum of P C, double)   -> outd[row]
// mode 1: max   (row max of log P, double) -> outd[row]
// mode 2: count (entries >= thr, int32)    -> outi[row]
template <typename T, int DP, int MODE>
__global__ __launch_bounds__(kRowsPerGroup *kWave) void row_pass(PlanArgs p,
                                                                 const double *__restrict__ thr,
                                                                 double *__restrict__ outd,
                                                                 int32_t *__restrict__ outi)
{
    const int b = blockIdx.y;
    const int i = blockIdx.x * kRowsPerGroup + wave_id_uniform();
    if (i >= p.n)
        return;
    const int lane = lane_id();
    RowCtx<DP> r;
    load_row<T, DP>(r, p, b, i);
    const T *Yb = (const T *)p.Y + (size_t)b * p.m * p.d;
    const float *gb = p.g + (size_t)b * p.m;
    const double t = MODE == 2 ? thr[b] : 0.0;
    double acc = MODE == 1 ? -INFINITY : 0.0;
    int cnt = 0;
    for (int j0 = 0; j0 < p.m; j0 += kWave) {
        const int j = j0 + lane;
        if (j < p.m) {
            double C;
            const double lbj = p.lb[(size_t)b * p.m + j];
            const double lp = log_plan<T, DP>(r, p, Yb, gb, lbj, j, &C);
            if (MODE == 0) {
                const double P = (double)ex2((float)(lp * 1.4426950408889634));
                acc = fma(P, C, acc);
            } else if (MODE == 1) {
                acc = fmax(acc, lp);
            } else {
                cnt += lp >= t ? 1 : 0;
            }
        }
    }
    if (MODE == 0) {
        acc = wave_sum(acc);
        if (lane == 0)
            outd[(size_t)b * p.n + i] = acc;
    } else if (MODE == 1) {
        acc = wave_max(acc);
        if (lane == 0)
            outd[(size_t)b * p.n + i] = acc;
    } else {
        cnt = wave_sum(cnt);
        if (lane == 0)
            outi[(size_t)b * p.n + i] = cnt;
    }
}

// Per-pair reduction of row values in a fixed order (deterministic).
// mode 0: sum -> float out[b];  mode 1: max + add -> double out[b]
template <int MODE>
__global__ __launch_bounds__(256) void pair_reduce(const double *__restrict__ rowv, int n,
                                                   float *__restrict__ outf,
                                                   double *__restrict__ outd, double add)
{
    __shared__ double sm[256];
    const int b = blockIdx.x;
    double acc = MODE == 0 ? 0.0 : -INFINITY;
    for (int i = threadIdx.x; i < n; i += 256) {
        const double v = rowv[(size_t)b * n + i];
        acc = MODE == 0 ? acc + v : fmax(acc, v);
    }
    sm[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < s)
            sm[threadIdx.x] = MODE == 0 ? sm[threadIdx.x] + sm[threadIdx.x + s]
                                        : fmax(sm[threadIdx.x], sm[threadIdx.x + s]);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        if (MODE == 0)
            outf[b] = (float)sm[0];
        else
            outd[b] = sm[0] + add;
    }
}

// Sum of the row counts of each pair.
__global__ __launch_bounds__(256) void pair_totals(const int32_t *__restrict__ cnt, int n,
                                                   int64_t *__restrict__ tot)
{
    __shared__ int64_t sm[256];
    const int b = blockIdx.x;
    int64_t acc = 0;
    for (int i = threadIdx.x; i < n; i += 256)
        acc += cnt[(size_t)b * n + i];
    sm[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < s)
            sm[threadIdx.x] += sm[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        tot[b] = sm[0];
}

// Exclusive scan of a block-sized chunk in LDS; returns the chunk total.
__device__ int64_t block_exclusive_scan(int64_t *sm, int64_t v)
{
    const int t = threadIdx.x;
    sm[t] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int64_t add = t >= off ? sm[t - off] : 0;
        __syncthreads();
        sm[t] += add;
        __syncthreads();
    }
    const int64_t incl = sm[t];
    const int64_t total = sm[255];
    __syncthreads();
    sm[t] = incl - v;
    return total;
}

// Single group: pair_offsets[0..B] from the pair totals.
__global__ __launch_bounds__(256) void pair_offsets_scan(const int64_t *__restrict__ tot, int B,
                                                         int64_t *__restrict__ offs)
{
    __shared__ int64_t sm[256];
    int64_t carry = 0;
    for (int base = 0; base < B; base += 256) {
        const int b = base + threadIdx.x;
        const int64_t v = b < B ? tot[b] : 0;
        const int64_t total = block_exclusive_scan(sm, v);
        if (b < B)
            offs[b] = carry + sm[threadIdx.x];
        carry += total;
        __syncthreads();
    }
    if (threadIdx.x == 0)
        offs[B] = carry;
}

// One group per pair: global offset of every row.
__global__ __launch_bounds__(256) void row_offsets_scan(const int32_t *__restrict__ cnt, int n,
                                                        const int64_t *__restrict__ offs,
                                                        int64_t *__restrict__ row_off)
{
    __shared__ int64_t sm[256];
    const int b = blockIdx.x;
    int64_t carry = offs[b];
    for (int base = 0; base < n; base += 256) {
        const int i = base + threadIdx.x;
        const int64_t v = i < n ? cnt[(size_t)b * n + i] : 0;
        const int64_t total = block_exclusive_scan(sm, v);
        if (i < n)
            row_off[(size_t)b * n + i] = carry + sm[threadIdx.x];
        carry += total;
        __syncthreads();
    }
}

template <typename T, int DP>
__global__ __launch_bounds__(kRowsPerGroup *kWave) void emit_pass(
    PlanArgs p, const double *__restrict__ thr, const int64_t *__restrict__ row_off,
    const int32_t *__restrict__ row_cnt, int32_t *__restrict__ rows, int32_t *__restrict__ cols,
    float *__restrict__ vals)
{
    const int b = blockIdx.y;
    const int i = blockIdx.x * kRowsPerGroup + wave_id_uniform();
    if (i >= p.n)
        return;
    const int lane = lane_id();
    RowCtx<DP> r;
    load_row<T, DP>(r, p, b, i);
    const T *Yb = (const T *)p.Y + (size_t)b * p.m * p.d;
    const float *gb = p.g + (size_t)b * p.m;
    const double t = thr[b];
    int64_t pos = row_off[(size_t)b * p.n + i];
    const int64_t end = pos + row_cnt[(size_t)b * p.n + i];
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int j0 = 0; j0 < p.m; j0 += kWave) {
        const int j = j0 + lane;
        bool keep = false;
        double lp = 0.0;
        if (j < p.m) {
            double C;
            const double lbj = p.lb[(size_t)b * p.m + j];
            lp = log_plan<T, DP>(r, p, Yb, gb, lbj, j, &C);
            keep = lp >= t;
        }
        const uint64_t mask = __ballot(keep);
        if (keep) {
            const int64_t k = pos + __popcll(mask & below);
            if (k < end) {   // always true: count and emit make identical decisions
                rows[k] = i;
                cols[k] = j;
                vals[k] = ex2((float)(lp * 1.4426950408889634));
            }
        }
        pos += __popcll(mask);
    }
}

template <typename F>
void with_dp(int d, F fn)
{
    if (d <= 4) fn.template operator()<4>();
    else if (d <= 8) fn.template operator()<8>();
    else if (d <= 16) fn.template operator()<16>();
    else if (d <= 32) fn.template operator()<32>();
    else if (d <= 64) fn.template operator()<64>();
    else fn.template operator()<128>();
}

template <int MODE>
void row_dispatch(const PlanArgs &p, const double *thr, double *outd, int32_t *outi,
                  hipStream_t st)
{
    dim3 grid(ceil_div(p.n, kRowsPerGroup), p.B);
    dim3 block(kRowsPerGroup * kWave);
    with_dp(p.d, [&]<int DP>() {
        if (p.dtype == 1)
            hipLaunchKernelGGL((row_pass<uint16_t, DP, MODE>), grid, block, 0, st, p, thr, outd,
                               outi);
        else
            hipLaunchKernelGGL((row_pass<float, DP, MODE>), grid, block, 0, st, p, thr, outd,
                               outi);
    });
}

}  // namespace

hipError_t launch_log_weights(const float *w, int B, int count, double *out, hipStream_t st)
{
    const size_t total = (size_t)B * count;
    hipLaunchKernelGGL(log_weights_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       st, w, count, total, out);
    return hipGetLastError();
}

hipError_t launch_cost(const PlanArgs &p, double *row_part, float *cost, hipStream_t st)
{
    row_dispatch<0>(p, nullptr, row_part, nullptr, st);
    hipLaunchKernelGGL(pair_reduce<0>, dim3(p.B), dim3(256), 0, st, (const double *)row_part,
                       p.n, cost, (double *)nullptr, 0.0);
    return hipGetLastError();
}

hipError_t launch_row_sums(const double *row_part, int B, int n, float *out, hipStream_t st)
{
    hipLaunchKernelGGL(pair_reduce<0>, dim3(B), dim3(256), 0, st, row_part, n, out,
                       (double *)nullptr, 0.0);
    return hipGetLastError();
}

hipError_t launch_plan_max(const PlanArgs &p, double *row_max, double *pair_thr,
                           double log_rel_thr, hipStream_t st)
{
    row_dispatch<1>(p, nullptr, row_max, nullptr, st);
    hipLaunchKernelGGL(pair_reduce<1>, dim3(p.B), dim3(256), 0, st, (const double *)row_max,
                       p.n, (float *)nullptr, pair_thr, log_rel_thr);
    return hipGetLastError();
}

hipError_t launch_plan_count(const PlanArgs &p, const double *pair_thr, int32_t *row_count,
                             hipStream_t st)
{
    row_dispatch<2>(p, pair_thr, nullptr, row_count, st);
    return hipGetLastError();
}

hipError_t launch_plan_scan(const int32_t *row_count, int B, int n, int64_t *row_off,
                            int64_t *pair_offsets, int64_t *pair_tot, hipStream_t st)
{
    hipLaunchKernelGGL(pair_totals, dim3(B), dim3(256), 0, st, row_count, n, pair_tot);
    hipLaunchKernelGGL(pair_offsets_scan, dim3(1), dim3(256), 0, st, (const int64_t *)pair_tot,
                       B, pair_offsets);
    hipLaunchKernelGGL(row_offsets_scan, dim3(B), dim3(256), 0, st, row_count, n,
                       (const int64_t *)pair_offsets, row_off);
    return hipGetLastError();
}

hipError_t launch_plan_emit(const PlanArgs &p, const double *pair_thr, const int64_t *row_off,
                            const int32_t *row_count, int32_t *rows, int32_t *cols,
                            float *vals, hipStream_t st)
{
    dim3 grid(ceil_div(p.n, kRowsPerGroup), p.B);
    dim3 block(kRowsPerGroup * kWave);
    with_dp(p.d, [&]<int DP>() {
        if (p.dtype == 1)
            hipLaunchKernelGGL((emit_pass<uint16_t, DP>), grid, block, 0, st, p, pair_thr,
                               row_off, row_count, rows, cols, vals);
        else
            hipLaunchKernelGGL((emit_pass<float, DP>), grid, block, 0, st, p, pair_thr, row_off,
                               row_count, rows, cols, vals);
    });
    return hipGetLastError();
}

}  // namespace sk

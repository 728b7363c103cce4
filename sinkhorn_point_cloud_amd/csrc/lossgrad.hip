// lossgrad.hip -- transport loss and its gradient with respect to X on the
// stored support of a sparse (COO) plan, the plan held fixed (CUDA-APML page,
// Abstract: gradients preserved on the stored support):
//     loss[p]  = sum_{k in pair p} P_k ||x_{r_k} - y_{c_k}||^2
//     dX[p][i] = sum_{k in pair p, r_k = i} 2 P_k (x_i - y_{c_k})
//
// The COO comes sorted by row within each pair (the order the plan extraction
// writes).  Each row's run of entries is found by binary search; then one wave
// reduces one row (lanes across its entries), so every row is summed without
// atomics and in a fixed order.  Column indices outside the pair's range are
// skipped rather than followed.  For d <= 4 and a pair's Y of at most 32 KiB
// the points are gathered from an LDS copy shared by 32 rows.
#include "plan_eval.h"

namespace sk {
namespace {

constexpr int kRowsPerGroup = 4;

// Row runs of a row-sorted COO by binary search: row i of pair b runs from the
// first entry of the pair with row >= i to the first with row >= i + 1.  Work
// item i (0 <= i <= n) finds the first entry with row >= i once and writes it
// as the begin of row i and the end of row i - 1; rows outside [0, n) end up
// in no run.
__global__ void row_bounds_search(const int32_t *__restrict__ rows,
                                  const int64_t *__restrict__ offs, int n,
                                  int64_t *__restrict__ begin, int64_t *__restrict__ end)
{
    const int b = blockIdx.y;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i > n)
        return;
    int64_t l = offs[b], h = offs[b + 1];
    while (l < h) {
        const int64_t mid = l + (h - l) / 2;
        if (rows[mid] < i)
            l = mid + 1;
        else
            h = mid;
    }
    if (i < n)
        begin[(size_t)b * n + i] = l;
    if (i > 0)
        end[(size_t)b * n + i - 1] = l;
}

template <typename T, int DP>
__global__ __launch_bounds__(kRowsPerGroup *kWave) void loss_grad_rows(
    const T *__restrict__ X, const T *__restrict__ Y, int d, int n, int m,
    const int32_t *__restrict__ cols, const float *__restrict__ vals,
    const int64_t *__restrict__ begin, const int64_t *__restrict__ end,
    double *__restrict__ row_loss, float *__restrict__ dX)
{
    const int b = blockIdx.y;
    const int i = blockIdx.x * kRowsPerGroup + wave_id_uniform();
    if (i >= n)
        return;
    const int lane = lane_id();
    const size_t ri = (size_t)b * n + i;
    // the DP = 3 instantiation serves d == 3 only: no per-component test
    auto has = [&](int c) { return has_dim<DP>(c, d); };
    float x[DP];
#pragma unroll
    for (int k = 0; k < DP; ++k)
        x[k] = has(k) ? Elem<T>::get(X, ri * d + k) : 0.f;
    const T *Yb = Y + (size_t)b * m * d;
    const int64_t k0 = begin[ri], k1 = end[ri];
    double loss = 0.0;
    float gr[DP];
#pragma unroll
    for (int k = 0; k < DP; ++k)
        gr[k] = 0.f;
    auto entry = [&](int64_t k) {
        const int j = cols[k];
        if (j < 0 || j >= m)
            return;
        loss_term_at<T, DP>(x, Yb + (size_t)j * d, d, vals[k], loss, gr);
    };
    // two entries per lane and step keep more loads in flight
    int64_t k = k0 + lane;
    for (; k + kWave < k1; k += 2 * kWave) {
        entry(k);
        entry(k + kWave);
    }
    if (k < k1)
        entry(k);
    loss = wave_sum(loss);
    if (lane == 0)
        row_loss[ri] = loss;
    if (dX) {
#pragma unroll
        for (int c = 0; c < DP; ++c) {
            if (has(c)) {
                const float v = wave_sum(gr[c]);
                if (lane == 0)
                    dX[ri * d + c] = v;
            }
        }
    }
}

// The same reduction with the pair's Y staged in LDS (component-major fp32,
// exact for both input types) when it fits: a work-group of kStagedWaves waves
// takes kStagedRows consecutive rows of one pair, a wave per row at a time, and
// gathers y_j from LDS instead of memory.  Same arithmetic, same order.
constexpr int kStagedWaves = 8, kStagedRows = 32;
constexpr size_t kStagedBytes = 32 * 1024;   // largest staged Y of one pair

template <typename T, int DP>
__global__ __launch_bounds__(kStagedWaves *kWave) void loss_grad_staged(
    const T *__restrict__ X, const T *__restrict__ Y, int d, int n, int m,
    const int32_t *__restrict__ cols, const float *__restrict__ vals,
    const int64_t *__restrict__ begin, const int64_t *__restrict__ end,
    double *__restrict__ row_loss, float *__restrict__ dX)
{
    static_assert(DP <= 4, "staged Y holds at most 4 components per point");
    extern __shared__ float ys[];   // [DP][m]
    const int b = blockIdx.y;
    const T *Yb = Y + (size_t)b * m * d;
    for (int j = threadIdx.x; j < m; j += kStagedWaves * kWave) {
#pragma unroll
        for (int c = 0; c < DP; ++c)
            ys[(size_t)c * m + j] = has_dim<DP>(c, d) ? Elem<T>::get(Yb, (size_t)j * d + c) : 0.f;
    }
    __syncthreads();
    const int lane = lane_id();
    auto has = [&](int c) { return has_dim<DP>(c, d); };
    constexpr int kRowsPerWave = kStagedRows / kStagedWaves;
    for (int q = 0; q < kRowsPerWave; ++q) {
        const int i = blockIdx.x * kStagedRows + wave_id_uniform() * kRowsPerWave + q;
        if (i >= n)
            break;
        const size_t ri = (size_t)b * n + i;
        float x[DP], gr[DP];
#pragma unroll
        for (int c = 0; c < DP; ++c) {
            x[c] = has(c) ? Elem<T>::get(X, ri * d + c) : 0.f;
            gr[c] = 0.f;
        }
        const int64_t k0 = begin[ri], k1 = end[ri];
        double loss = 0.0;
        auto entry = [&](int j, float v) {
            if (j < 0 || j >= m)
                return;
            float y[DP];
#pragma unroll
            for (int c = 0; c < DP; ++c)
                y[c] = ys[(size_t)c * m + j];
            loss_term_xy<DP>(x, y, d, v, loss, gr);
        };
        // a lane takes the row's entries lane, lane + 64, ... in order, four per
        // step with their loads in flight together
        int64_t k = k0 + lane;
        for (; k + 3 * kWave < k1; k += 4 * kWave) {
            int j[4];
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                j[u] = cols[k + u * kWave];
                v[u] = vals[k + u * kWave];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                entry(j[u], v[u]);
        }
        for (; k < k1; k += kWave)
            entry(cols[k], vals[k]);
        loss = wave_sum(loss);
        if (lane == 0)
            row_loss[ri] = loss;
        if (dX) {
#pragma unroll
            for (int c = 0; c < DP; ++c) {
                if (has(c)) {
                    const float v = wave_sum(gr[c]);
                    if (lane == 0)
                        dX[ri * d + c] = v;
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void pair_sum(const double *__restrict__ rowv, int n,
                                                float *__restrict__ out)
{
    __shared__ double sm[256];
    const int b = blockIdx.x;
    double acc = 0.0;
    for (int i = threadIdx.x; i < n; i += 256)
        acc += rowv[(size_t)b * n + i];
    sm[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < s)
            sm[threadIdx.x] += sm[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        out[b] = (float)sm[0];
}

template <typename T, int DP>
void launch_rows(const void *X, const void *Y, int d, int B, int n, int m, const int32_t *cols,
                 const float *vals, const int64_t *begin, const int64_t *end,
                 double *row_loss, float *dX, hipStream_t st)
{
    dim3 grid(ceil_div(n, kRowsPerGroup), B);
    hipLaunchKernelGGL((loss_grad_rows<T, DP>), grid, dim3(kRowsPerGroup * kWave), 0, st,
                       (const T *)X, (const T *)Y, d, n, m, cols, vals, begin, end, row_loss,
                       dX);
}

template <typename T>
void rows_dispatch(const void *X, const void *Y, int d, int B, int n, int m,
                   const int32_t *cols, const float *vals, const int64_t *begin,
                   const int64_t *end, double *row_loss, float *dX, hipStream_t st)
{
    if (d <= 4 && (size_t)m * 4 * sizeof(float) <= kStagedBytes) {
        const dim3 grid(ceil_div(n, kStagedRows), B), block(kStagedWaves * kWave);
        if (d == 3)
            hipLaunchKernelGGL((loss_grad_staged<T, 3>), grid, block, (size_t)m * 3 * sizeof(float),
                               st, (const T *)X, (const T *)Y, d, n, m, cols, vals, begin, end,
                               row_loss, dX);
        else
            hipLaunchKernelGGL((loss_grad_staged<T, 4>), grid, block, (size_t)m * 4 * sizeof(float),
                               st, (const T *)X, (const T *)Y, d, n, m, cols, vals, begin, end,
                               row_loss, dX);
        return;
    }
    if (d == 3) launch_rows<T, 3>(X, Y, d, B, n, m, cols, vals, begin, end, row_loss, dX, st);
    else if (d <= 4) launch_rows<T, 4>(X, Y, d, B, n, m, cols, vals, begin, end, row_loss, dX, st);
    else if (d <= 8) launch_rows<T, 8>(X, Y, d, B, n, m, cols, vals, begin, end, row_loss, dX, st);
    else if (d <= 16) launch_rows<T, 16>(X, Y, d, B, n, m, cols, vals, begin, end, row_loss, dX, st);
    else if (d <= 32) launch_rows<T, 32>(X, Y, d, B, n, m, cols, vals, begin, end, row_loss, dX, st);
    else if (d <= 64) launch_rows<T, 64>(X, Y, d, B, n, m, cols, vals, begin, end, row_loss, dX, st);
    else launch_rows<T, 128>(X, Y, d, B, n, m, cols, vals, begin, end, row_loss, dX, st);
}

}  // namespace

hipError_t launch_segment_bounds(const int32_t *keys, const int64_t *pair_offsets, int B, int count,
                                 int64_t *begin, int64_t *end, hipStream_t st)
{
    hipLaunchKernelGGL(row_bounds_search, dim3(ceil_div(count + 1, 256), B), dim3(256), 0, st, keys,
                       pair_offsets, count, begin, end);
    return hipGetLastError();
}

hipError_t launch_loss_grad(const void *X, const void *Y, int dtype, int d, int B, int n,
                            int m, const int32_t *rows, const int32_t *cols, const float *vals,
                            const int64_t *pair_offsets, int64_t *row_begin,
                            int64_t *row_end, double *row_loss, float *loss, float *dX,
                            hipStream_t st)
{
    hipLaunchKernelGGL(row_bounds_search, dim3(ceil_div(n + 1, 256), B), dim3(256), 0, st, rows,
                       pair_offsets, n, row_begin, row_end);
    if (dtype == 1)
        rows_dispatch<uint16_t>(X, Y, d, B, n, m, cols, vals, row_begin, row_end, row_loss, dX,
                                st);
    else
        rows_dispatch<float>(X, Y, d, B, n, m, cols, vals, row_begin, row_end, row_loss, dX, st);
    hipLaunchKernelGGL(pair_sum, dim3(B), dim3(256), 0, st, (const double *)row_loss, n, loss);
    return hipGetLastError();
}

}  // namespace sk

// lossgrad.hip -- transport loss and its gradient with respect to X on the
// stored support of a sparse (COO) plan, the plan held fixed (CUDA-APML page,
// Abstract: gradients preserved on the stored support):
//     loss[p]  = sum_{k in pair p} P_k ||x_{r_k} - y_{c_k}||^2
//     dX[p][i] = sum_{k in pair p, r_k = i} 2 P_k (x_i - y_{c_k})
//
// The COO comes sorted by row within each pair (the order the plan extraction
// writes).  A first pass marks where each row's run of entries begins and
// ends; then one wave reduces one row (lanes across its entries), so every
// row is summed without atomics and in a fixed order.  Indices outside the
// pair's range are skipped rather than followed.
#include "common.h"

namespace sk {
namespace {

constexpr int kRowsPerGroup = 4;

__global__ void fill_i64(int64_t *__restrict__ p, size_t count)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count)
        p[i] = 0;
}

__global__ void row_bounds(const int32_t *__restrict__ rows, const int64_t *__restrict__ offs,
                           int n, int64_t *__restrict__ begin, int64_t *__restrict__ end)
{
    const int b = blockIdx.y;
    const int64_t lo = offs[b], hi = offs[b + 1];
    for (int64_t k = lo + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < hi;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int r = rows[k];
        if (r < 0 || r >= n)
            continue;
        if (k == lo || rows[k - 1] != r)
            begin[(size_t)b * n + r] = k;
        if (k == hi - 1 || rows[k + 1] != r)
            end[(size_t)b * n + r] = k + 1;
    }
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
    float x[DP];
#pragma unroll
    for (int k = 0; k < DP; ++k)
        x[k] = k < d ? Elem<T>::get(X, ri * d + k) : 0.f;
    const T *Yb = Y + (size_t)b * m * d;
    const int64_t k0 = begin[ri], k1 = end[ri];
    double loss = 0.0;
    float gr[DP];
#pragma unroll
    for (int k = 0; k < DP; ++k)
        gr[k] = 0.f;
    for (int64_t k = k0 + lane; k < k1; k += kWave) {
        const int j = cols[k];
        if (j < 0 || j >= m)
            continue;
        const float P = vals[k];
        double C = 0.0;
#pragma unroll
        for (int c = 0; c < DP; ++c) {
            if (c < d) {
                const float t = x[c] - Elem<T>::get(Yb, (size_t)j * d + c);
                C = fma((double)t, (double)t, C);
                gr[c] = fmaf(2.0f * P, t, gr[c]);
            }
        }
        loss = fma((double)P, C, loss);
    }
    loss = wave_sum(loss);
    if (lane == 0)
        row_loss[ri] = loss;
    if (dX) {
#pragma unroll
        for (int c = 0; c < DP; ++c) {
            if (c < d) {
                const float v = wave_sum(gr[c]);
                if (lane == 0)
                    dX[ri * d + c] = v;
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
    if (d <= 4) launch_rows<T, 4>(X, Y, d, B, n, m, cols, vals, begin, end, row_loss, dX, st);
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
    const size_t cnt = (size_t)B * count;
    hipLaunchKernelGGL(fill_i64, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st, begin,
                       cnt);
    hipLaunchKernelGGL(fill_i64, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st, end, cnt);
    hipLaunchKernelGGL(row_bounds, dim3(256, B), dim3(256), 0, st, keys, pair_offsets, count,
                       begin, end);
    return hipGetLastError();
}

hipError_t launch_loss_grad(const void *X, const void *Y, int dtype, int d, int B, int n,
                            int m, const int32_t *rows, const int32_t *cols, const float *vals,
                            const int64_t *pair_offsets, int64_t *row_begin,
                            int64_t *row_end, double *row_loss, float *loss, float *dX,
                            hipStream_t st)
{
    const size_t cnt = (size_t)B * n;
    hipLaunchKernelGGL(fill_i64, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st,
                       row_begin, cnt);
    hipLaunchKernelGGL(fill_i64, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st,
                       row_end, cnt);
    hipLaunchKernelGGL(row_bounds, dim3(256, B), dim3(256), 0, st, rows, pair_offsets, n,
                       row_begin, row_end);
    if (dtype == 1)
        rows_dispatch<uint16_t>(X, Y, d, B, n, m, cols, vals, row_begin, row_end, row_loss, dX,
                                st);
    else
        rows_dispatch<float>(X, Y, d, B, n, m, cols, vals, row_begin, row_end, row_loss, dX, st);
    hipLaunchKernelGGL(pair_sum, dim3(B), dim3(256), 0, st, (const double *)row_loss, n, loss);
    return hipGetLastError();
}

}  // namespace sk

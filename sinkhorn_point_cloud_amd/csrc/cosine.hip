// cosine.hip -- normalisation for the cosine cost and its backward.
//
// The FlashSinkhorn summary (Betekenis en Claims) notes that the attention
// form holds for the cosine distance after normalisation: for unit vectors
// ||x^ - y^||^2 = 2 - 2 x^ . y^, the cosine cost, so the squared-Euclidean
// path solves the cosine-cost problem on the normalised points.  These two
// kernels map points to unit length and carry a gradient with respect to the
// normalised points back to the raw ones:
//     x^ = x / ||x||,   dX = (G - x^ (x^ . G)) / ||x||   (Jacobian (I - x^ x^T) / ||x||).
// A zero vector maps to 0 with norm 0 and gets a zero gradient.  The norm and
// the quotient are formed in fp64 and rounded once.
//
// One wave per point, lanes across the dimensions (coalesced rows for any d).
#include "common.h"

namespace sk {
namespace {

constexpr int kPointsPerGroup = 4;   // one wave per point

__device__ __forceinline__ double wave_sum_d(double v)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

template <typename T>
__global__ __launch_bounds__(kPointsPerGroup *kWave) void normalize_kernel(
    const T *__restrict__ X, long count, int d, float *__restrict__ Xh, float *__restrict__ norms)
{
    const long i = (long)blockIdx.x * kPointsPerGroup + wave_id_uniform();
    if (i >= count)
        return;
    const int lane = lane_id();
    const T *x = X + i * d;
    double s = 0.0;
    for (int k = lane; k < d; k += kWave) {
        const double v = (double)Elem<T>::get(x, k);
        s = fma(v, v, s);
    }
    const double r = sqrt(wave_sum_d(s));
    for (int k = lane; k < d; k += kWave)
        Xh[i * d + k] = r > 0.0 ? (float)((double)Elem<T>::get(x, k) / r) : 0.f;
    if (lane == 0)
        norms[i] = (float)r;
}

__global__ __launch_bounds__(kPointsPerGroup *kWave) void normalize_backward_kernel(
    const float *__restrict__ Xh, const float *__restrict__ norms, const float *__restrict__ G,
    long count, int d, float *__restrict__ dX)
{
    const long i = (long)blockIdx.x * kPointsPerGroup + wave_id_uniform();
    if (i >= count)
        return;
    const int lane = lane_id();
    double dot = 0.0;
    for (int k = lane; k < d; k += kWave)
        dot = fma((double)Xh[i * d + k], (double)G[i * d + k], dot);
    dot = wave_sum_d(dot);
    const double r = (double)norms[i];
    for (int k = lane; k < d; k += kWave)
        dX[i * d + k] =
            r > 0.0 ? (float)(((double)G[i * d + k] - (double)Xh[i * d + k] * dot) / r) : 0.f;
}

}  // namespace

hipError_t launch_normalize(const void *X, int dtype, long count, int d, float *Xh,
                            float *norms, hipStream_t st)
{
    const unsigned groups = (unsigned)((count + kPointsPerGroup - 1) / kPointsPerGroup);
    if (dtype == 1)
        hipLaunchKernelGGL(normalize_kernel<uint16_t>, dim3(groups),
                           dim3(kPointsPerGroup * kWave), 0, st, (const uint16_t *)X, count, d,
                           Xh, norms);
    else
        hipLaunchKernelGGL(normalize_kernel<float>, dim3(groups), dim3(kPointsPerGroup * kWave),
                           0, st, (const float *)X, count, d, Xh, norms);
    return hipGetLastError();
}

hipError_t launch_normalize_backward(const float *Xh, const float *norms, const float *G,
                                     long count, int d, float *dX, hipStream_t st)
{
    const unsigned groups = (unsigned)((count + kPointsPerGroup - 1) / kPointsPerGroup);
    hipLaunchKernelGGL(normalize_backward_kernel, dim3(groups), dim3(kPointsPerGroup * kWave), 0,
                       st, Xh, norms, G, count, d, dX);
    return hipGetLastError();
}

}  // namespace sk

// rates.hip -- instruction-rate probe behind the roofline figures of the
// streaming kernels (the FlashSinkhorn summary, Probleemstelling: the update is
// bound by compute and by instruction efficiency once HBM traffic is gone).
//
// Each work-group's waves run `iters` iterations of one fixed instruction mix
// on independent register chains (enough chains, and enough waves per SIMD,
// that latency is hidden and the issue rate is what is measured).  Wave 0 of
// every work-group records the shader-clock counter (s_memtime, core clock)
// and the constant-rate wall-clock counter (s_memrealtime) at its start and at
// its end, after the work-group's barrier, so the host can compute the
// clock the chip ran at and the issue rate per compute unit per clock.
//
// Mixes (per iteration and lane):
//   0  16 v_exp_f32                       (8 chains x 2)
//   1  16 v_fma_f32                       (8 chains x 2, packed forms disabled)
//   2  16 v_exp_f32 + 16 v_add_f32        (the exponential-and-accumulate pair)
//   3  4 v_mfma_f32_16x16x32_bf16         (4 independent accumulators)
//   4  one d = 3 score tile of the streaming LSE: 4 MFMAs (one per 16-row group,
//      the shift in the accumulator input), then S += 2^D for their 16 outputs
//   5  16 v_fma_f64                       (8 chains x 2)
//   6  one d = 64 bf16 feature tile: per group two chained MFMAs, then
//      S += 2^(2c D + beta) for their 4 outputs (16 fma, 16 exp, 16 add)
//   7  2 v_mfma_f32_32x32x16_bf16         (2 independent accumulators)
//   8  the d = 64 feature tile with 32 x 32 blocks: four chained 32x32x16 MFMAs
//      (the same 1024 entries and products), then 16 fma, 16 exp, 16 add
// In 4 and 6 the key operand and the accumulator inputs pass through empty asm
// statements every iteration, so the products are recomputed as in the kernels.
#include "common.h"
#include "sinkhorn.h"
#include "sinkhorn_probe.h"

namespace sk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int Kind>
__global__ __launch_bounds__(256) void rate_kernel(float *__restrict__ sink,
                                                   unsigned long long *__restrict__ clocks,
                                                   int iters, float seed)
{
    unsigned long long t0 = 0, w0 = 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        t0 = clock64();
        w0 = wall_clock64();
    }
    const float x0 = seed * (float)(threadIdx.x + 1) * 1e-3f;
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        v[k] = x0 + 0.01f * k;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    double dv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        dv[k] = (double)v[k];
    f32x4 D[4];
    bf16x8 A, Bm;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        A[e] = (__bf16)(0.01f * (x0 + 0.125f * e));
        Bm[e] = (__bf16)(0.05f - 0.00625f * e);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
        D[g] = f32x4{-x0 - g, -1.f - g, -2.f - g, -3.f - g};
    f32x16 W[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            W[h][e] = -x0 - 0.25f * e - h;

    for (int it = 0; it < iters; ++it) {
        if constexpr (Kind == 0) {
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    v[k] = ex2(-v[k]);   // stays in (0, 1]
        } else if constexpr (Kind == 1) {
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    v[k] = fmaf(v[k], 0.999f, 1e-3f);
        } else if constexpr (Kind == 2) {
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    v[k] = ex2(-v[k]);
                    acc[k] += v[k];
                }
        } else if constexpr (Kind == 3) {
#pragma unroll
            for (int g = 0; g < 4; ++g)
                D[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bm, D[g], 0, 0, 0);
        } else if constexpr (Kind == 4) {
            asm volatile("" : "+v"(Bm));
#pragma unroll
            for (int g = 0; g < 4; ++g)
                asm volatile("" : "+v"(D[g]));
            f32x4 E[4];
#pragma unroll
            for (int g = 0; g < 4; ++g)
                E[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bm, D[g], 0, 0, 0);
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[2 * g + (r >> 1)] += ex2(E[g][r]);
        } else if constexpr (Kind == 6) {
            asm volatile("" : "+v"(Bm));
#pragma unroll
            for (int g = 0; g < 4; ++g)
                asm volatile("" : "+v"(D[g]));
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 E = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bm, D[g], 0, 0, 0);
                E = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Bm, A, E, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[2 * g + (r >> 1)] += ex2(fmaf(v[0], E[r], v[1]));
            }
        } else if constexpr (Kind == 5) {
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    dv[k] = fma(dv[k], 0.999, 1e-3);
        } else if constexpr (Kind == 7) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
                W[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bm, W[h], 0, 0, 0);
        } else {
            asm volatile("" : "+v"(Bm));
            asm volatile("" : "+v"(W[0]));
            f32x16 E = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bm, W[0], 0, 0, 0);
            E = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Bm, A, E, 0, 0, 0);
            E = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bm, E, 0, 0, 0);
            E = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Bm, A, E, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[r >> 1] += ex2(fmaf(v[0], E[r], v[1]));
        }
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        s += v[k] + acc[k] + (float)dv[k];
#pragma unroll
    for (int g = 0; g < 4; ++g)
        s += D[g][0] + D[g][1] + D[g][2] + D[g][3];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        s += W[h][0] + W[h][15];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;   // keeps every chain live
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned long long t1 = clock64(), w1 = wall_clock64();
        unsigned long long *c = clocks + 4 * (size_t)blockIdx.x;
        c[0] = t0;
        c[1] = t1;
        c[2] = w0;
        c[3] = w1;
    }
}

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" int sinkhorn_probe_rates(int kind, int blocks, int iters, float *sink,
                                    unsigned long long *clocks, double *wall_clock_hz,
                                    void *stream)
{
    if (kind < 0 || kind > 8 || blocks < 1 || blocks > (1 << 20) || iters < 1 || !sink ||
        !clocks || !wall_clock_hz)
        return SK_ERR_INVALID_ARG;
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
        return SK_ERR_HIP;
    *wall_clock_hz = 1e3 * (double)khz;
    hipStream_t st = (hipStream_t)stream;
    const float seed = 1.0f + 0.5f * kind;
    switch (kind) {
    case 0: hipLaunchKernelGGL(rate_kernel<0>, dim3(blocks), dim3(256), 0, st, sink, clocks, iters, seed); break;
    case 1: hipLaunchKernelGGL(rate_kernel<1>, dim3(blocks), dim3(256), 0, st, sink, clocks, iters, seed); break;
    case 2: hipLaunchKernelGGL(rate_kernel<2>, dim3(blocks), dim3(256), 0, st, sink, clocks, iters, seed); break;
    case 3: hipLaunchKernelGGL(rate_kernel<3>, dim3(blocks), dim3(256), 0, st, sink, clocks, iters, seed); break;
    case 4: hipLaunchKernelGGL(rate_kernel<4>, dim3(blocks), dim3(256), 0, st, sink, clocks, iters, seed); break;
    case 5: hipLaunchKernelGGL(rate_kernel<5>, dim3(blocks), dim3(256), 0, st, sink, clocks, iters, seed); break;
    case 6: hipLaunchKernelGGL(rate_kernel<6>, dim3(blocks), dim3(256), 0, st, sink, clocks, iters, seed); break;
    case 7: hipLaunchKernelGGL(rate_kernel<7>, dim3(blocks), dim3(256), 0, st, sink, clocks, iters, seed); break;
    default: hipLaunchKernelGGL(rate_kernel<8>, dim3(blocks), dim3(256), 0, st, sink, clocks, iters, seed); break;
    }
    return hipGetLastError() == hipSuccess ? SK_OK : SK_ERR_HIP;
}

extern "C" long long sinkhorn_probe_wait_limit(long long microseconds)
{
    return lse3_split_set_wait_us(microseconds);
}

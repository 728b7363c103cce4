// lse_feat.hip -- fused streaming half-iteration for feature clouds of
// dimension d <= 128 (fp32 or bf16 points), computed on the vector ALUs.
//
// Same update as lse_d3.hip (FlashSinkhorn summary, Methodologie 1,
// Propositie 1; streaming per Methodologie 2), in base 2:
//     s_ij = 2c (x_i . y_j) + beta_j,  beta_j = c (g_j - ||y_j||^2) + log2 w_j,
//     f_i  = ||x_i||^2 - (eps ln2) * log2 sum_j 2^(s_ij),   c = log2(e)/eps,
// with beta in a separate bias array and the true potentials as the state
// (row results and biases formed in fp64 and rounded once).
//
// Each lane owns one query row, held in registers as fp32.  A work-group of
// 4 waves shares 64 rows; per step the group stages 4 tiles of kKeys keys in
// LDS (bf16 widened to fp32 on the way), each wave then streams its own tile
// with broadcast LDS reads.  The online (M, S) state with a lazy maximum is
// the one described in lse_d3.hip.
#include "common.h"

namespace sk {
namespace {

constexpr int kKeys = 16;
constexpr int kWaves = 4;
constexpr float kLazy = 32.0f;

__device__ __forceinline__ float bias_of(double c, float pot, float sq, float l2w)
{
    return l2w == kNeg ? kNeg : (float)fma(c, (double)pot - (double)sq, (double)l2w);
}

template <typename T>
__global__ void packF_kernel(const T *__restrict__ X, int d, const float *__restrict__ w,
                             int warm, int n, int n_pad, float *__restrict__ bias,
                             float *__restrict__ pot, float *__restrict__ l2w, double c0)
{
    const int b = blockIdx.y;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_pad)
        return;
    if (i >= n) {
        bias[(size_t)b * n_pad + i] = kNeg;
        return;
    }
    const T *x = X + ((size_t)b * n + i) * d;
    float sq = 0.f;
    for (int k = 0; k < d; ++k) {
        const float v = Elem<T>::get(x, k);
        sq = fmaf(v, v, sq);
    }
    float lw;
    if (w) {
        const float wi = w[(size_t)b * n + i];
        lw = wi > 0.f ? log2f(wi) : kNeg;
    } else {
        lw = -log2f((float)n);
    }
    const size_t k = (size_t)b * n + i;
    if (!warm)
        pot[k] = 0.f;
    l2w[k] = lw;
    bias[(size_t)b * n_pad + i] = bias_of(c0, pot[k], sq, lw);
}

// squared norm of a row held in registers, summed in the order of packF_kernel
template <int DP>
__device__ __forceinline__ float row_sq(const float (&q)[DP], int d)
{
    float sq = 0.f;
#pragma unroll
    for (int k = 0; k < DP; ++k)
        if (k < d)
            sq = fmaf(q[k], q[k], sq);
    return sq;
}

__device__ __forceinline__ void finish_row(float *qbias, float *qpot, const float *ql2w,
                                           size_t pt, size_t k, float sq, float M, float S,
                                           double eps_ln2, double c_next)
{
    const double lse2 = (double)M + (double)lg2(S);
    const float f = (float)((double)sq - lse2 * eps_ln2);
    qpot[k] = f;
    qbias[pt] = bias_of(c_next, f, sq, ql2w[k]);
}

template <typename T, int DP>
__global__ __launch_bounds__(kWaves *kWave) void lseF_kernel(
    const T *__restrict__ qx_, float *__restrict__ qbias, float *__restrict__ qpot,
    const float *__restrict__ ql2w, const T *__restrict__ ky_, const float *__restrict__ kbias,
    float2 *__restrict__ part, int d, int nq, int nq_pad, int nk, int nk_pad,
    int tiles_per_split, float two_c, double eps_ln2, double c_next)
{
    __shared__ float4 tile[kWaves][kKeys][DP / 4];
    __shared__ float2 red[kWaves][kWave];
    const int b = blockIdx.z;
    const int split = blockIdx.y;
    const int lane = lane_id();
    const int w = wave_id_uniform();
    const int row = blockIdx.x * kWave + lane;

    float q[DP];
    {
        const T *x = qx_ + ((size_t)b * nq + (row < nq ? row : 0)) * d;
#pragma unroll
        for (int k = 0; k < DP; ++k)
            q[k] = (k < d && row < nq) ? Elem<T>::get(x, k) : 0.f;
    }
    const T *ky = ky_ + (size_t)b * nk * d;
    const float *kb = kbias + (size_t)b * nk_pad;
    const int n_tiles = nk_pad / kKeys;
    const int t_begin = split * tiles_per_split;
    const int t_end = min(t_begin + tiles_per_split, n_tiles);

    float M = kNeg, S = 0.f;
    for (int t0 = t_begin; t0 < t_end; t0 += kWaves) {
        // stage kWaves tiles (kWaves * kKeys keys) cooperatively
        __syncthreads();
        float *flat = &tile[0][0][0].x;
        const int total = kWaves * kKeys * DP;
        for (int e = threadIdx.x; e < total; e += kWaves * kWave) {
            const int key = e / DP, k = e % DP;
            const int j = t0 * kKeys + key;
            float v = 0.f;
            if (k < d && j < nk && t0 + key / kKeys < t_end)
                v = Elem<T>::get(ky, (size_t)j * d + k);
            flat[e] = v;
        }
        __syncthreads();
        const int t = t0 + w;
        if (t >= t_end)
            continue;
        float dot[kKeys];
#pragma unroll
        for (int u = 0; u < kKeys; ++u) {
            float acc = 0.f;
#pragma unroll
            for (int k4 = 0; k4 < DP / 4; ++k4) {
                const float4 y = tile[w][u][k4];
                acc = fmaf(q[4 * k4 + 0], y.x, acc);
                acc = fmaf(q[4 * k4 + 1], y.y, acc);
                acc = fmaf(q[4 * k4 + 2], y.z, acc);
                acc = fmaf(q[4 * k4 + 3], y.w, acc);
            }
            dot[u] = acc;
        }
        float r[kKeys];
        float cm = kNeg;
#pragma unroll
        for (int u = 0; u < kKeys; ++u) {
            r[u] = fmaf(two_c, dot[u], kb[t * kKeys + u] - M);
            cm = fmaxf(cm, r[u]);
        }
        if (cm > kLazy) {
            float Mn = M;
#pragma unroll
            for (int u = 0; u < kKeys; ++u) {
                r[u] = fmaf(two_c, dot[u], kb[t * kKeys + u]);
                Mn = fmaxf(Mn, r[u]);
            }
            S *= ex2(M - Mn);
#pragma unroll
            for (int u = 0; u < kKeys; ++u)
                r[u] -= Mn;
            M = Mn;
        }
#pragma unroll
        for (int u = 0; u < kKeys; ++u)
            S += ex2(r[u]);
    }

    red[w][lane] = make_float2(M, S);
    __syncthreads();
    if (w != 0)
        return;
#pragma unroll
    for (int v = 1; v < kWaves; ++v) {
        const float2 o = red[v][lane];
        lse_merge(M, S, o.x, o.y);
    }
    if (part) {
        part[((size_t)split * gridDim.z + b) * nq_pad + row] = make_float2(M, S);
        return;
    }
    if (row < nq)
        finish_row(qbias, qpot, ql2w, (size_t)b * nq_pad + row, (size_t)b * nq + row,
                   row_sq(q, d), M, S, eps_ln2, c_next);
}

template <typename T>
__global__ void lseF_finalize(const T *__restrict__ qx_, int d, float *__restrict__ qbias,
                              float *__restrict__ qpot, const float *__restrict__ ql2w,
                              const float2 *__restrict__ part, int B, int nq, int nq_pad,
                              int splits, double eps_ln2, double c_next)
{
    const int b = blockIdx.y;
    const int row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= nq)
        return;
    float2 s0 = part[(size_t)b * nq_pad + row];
    float M = s0.x, S = s0.y;
    for (int s = 1; s < splits; ++s) {
        const float2 o = part[((size_t)s * B + b) * nq_pad + row];
        lse_merge(M, S, o.x, o.y);
    }
    const T *x = qx_ + ((size_t)b * nq + row) * d;
    float sq = 0.f;
    for (int k = 0; k < d; ++k) {
        const float v = Elem<T>::get(x, k);
        sq = fmaf(v, v, sq);
    }
    finish_row(qbias, qpot, ql2w, (size_t)b * nq_pad + row, (size_t)b * nq + row, sq, M, S,
               eps_ln2, c_next);
}

int padded_dim(int d)
{
    if (d <= 8) return 8;
    if (d <= 16) return 16;
    if (d <= 32) return 32;
    if (d <= 64) return 64;
    if (d <= 128) return 128;
    return 0;
}

int lseF_splits(int B, int nq_pad, int nk_pad)
{
    const long groups = (long)B * (nq_pad / kWave);
    const int tiles = nk_pad / kKeys;
    int splits = (int)((1024 + groups - 1) / groups);
    const int max_splits = tiles / (2 * kWaves);
    if (splits > max_splits)
        splits = max_splits;
    return splits < 1 ? 1 : splits;
}

template <typename T, int DP>
void launch_lseF_t(SideF q, SideF k, int d, int B, float two_c, double eps_ln2,
                   double c_next, float2 *part, hipStream_t st)
{
    const int splits = lseF_splits(B, q.n_pad, k.n_pad);
    const int tiles = k.n_pad / kKeys;
    const int tps = ceil_div(tiles, splits);
    dim3 grid(q.n_pad / kWave, splits, B);
    hipLaunchKernelGGL((lseF_kernel<T, DP>), grid, dim3(kWaves * kWave), 0, st,
                       (const T *)q.pts, q.bias, q.pot, (const float *)q.l2w,
                       (const T *)k.pts, (const float *)k.bias, splits > 1 ? part : nullptr, d,
                       q.n, q.n_pad, k.n, k.n_pad, tps, two_c, eps_ln2, c_next);
    if (splits > 1) {
        dim3 g2(ceil_div(q.n, 256), B);
        hipLaunchKernelGGL(lseF_finalize<T>, g2, dim3(256), 0, st, (const T *)q.pts, d, q.bias,
                           q.pot, (const float *)q.l2w, (const float2 *)part, B, q.n, q.n_pad,
                           splits, eps_ln2, c_next);
    }
}

template <typename T>
void dispatch(SideF q, SideF k, int d, int B, float two_c, double ne, double cn, float2 *part,
              hipStream_t st)
{
    switch (padded_dim(d)) {
    case 8: launch_lseF_t<T, 8>(q, k, d, B, two_c, ne, cn, part, st); break;
    case 16: launch_lseF_t<T, 16>(q, k, d, B, two_c, ne, cn, part, st); break;
    case 32: launch_lseF_t<T, 32>(q, k, d, B, two_c, ne, cn, part, st); break;
    case 64: launch_lseF_t<T, 64>(q, k, d, B, two_c, ne, cn, part, st); break;
    default: launch_lseF_t<T, 128>(q, k, d, B, two_c, ne, cn, part, st); break;
    }
}

}  // namespace

bool lseF_supported(int dtype, int d) { return (dtype == 0 || dtype == 1) && padded_dim(d) > 0; }

size_t lseF_partial_floats2(int B, int nq_pad, int nk_pad)
{
    const int s = lseF_splits(B, nq_pad, nk_pad);
    return s > 1 ? (size_t)s * B * nq_pad : 0;
}

hipError_t launch_packF(const void *X, int dtype, int d, const float *w, int warm, int B,
                        SideF s, double c0, hipStream_t st)
{
    dim3 grid(ceil_div(s.n_pad, 256), B);
    if (dtype == 1)
        hipLaunchKernelGGL(packF_kernel<uint16_t>, grid, dim3(256), 0, st,
                           (const uint16_t *)X, d, w, warm, s.n, s.n_pad, s.bias, s.pot, s.l2w,
                           c0);
    else
        hipLaunchKernelGGL(packF_kernel<float>, grid, dim3(256), 0, st, (const float *)X, d, w,
                           warm, s.n, s.n_pad, s.bias, s.pot, s.l2w, c0);
    return hipGetLastError();
}

hipError_t launch_lseF(SideF q, SideF k, int dtype, int d, int B, float eps, float eps_next,
                       float2 *part, hipStream_t st)
{
    const float c = scale_of(eps);
    const double c_next = (double)scale_of(eps_next);
    const double eps_ln2 = 1.0 / (double)c;
    if (dtype == 1)
        dispatch<uint16_t>(q, k, d, B, 2.0f * c, eps_ln2, c_next, part, st);
    else
        dispatch<float>(q, k, d, B, 2.0f * c, eps_ln2, c_next, part, st);
    return hipGetLastError();
}

}  // namespace sk

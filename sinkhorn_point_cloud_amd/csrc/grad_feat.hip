// grad_feat.hip -- dense gradient and barycentric projection for bf16 feature
// clouds on the matrix cores (d = 32 or 64).
//
// The transport application of the FlashSinkhorn summary (Methodologie 3,
// "Toepassing van Transportmatrix": the gradient and the barycentric
// projection are weighted averages over the plan, streamed like the update
// without storing the plan).  With c = log2(e)/eps and the potentials f, g of
// the solution,
//     P_ij / a_i = E_ij = 2^(2c x_i.y_j + alpha_i + beta_j),
//     alpha_i = c (f_i - ||x_i||^2),   beta_j = c (g_j - ||y_j||^2) + log2 b_j,
// and per row the kernel accumulates the mass m_i = sum_j E_ij and
// O_i = sum_j E_ij y_j, then writes
//     dX_i = 2 a_i (m_i x_i - O_i)   (= sum_j 2 P_ij (x_i - y_j)),
//     T_i  = O_i / m_i               (= sum_j P_ij y_j / sum_j P_ij).
// E is the plan divided by the row weight, so m_i is near 1 for potentials
// that solve the problem, whatever the sizes.
//
// Two contractions per key tile of 16 keys, both on the matrix cores:
//   - scores, transposed: D' = Y_tile X_group^T on v_mfma_f32_16x16x32_bf16
//     (exact bf16 products, fp32 sums), keys in the rows of D', so lane l
//     holds E for row l % 16 and keys 4 (l / 16) + r;
//   - O += E Y_tile on v_mfma_f32_16x16x16_bf16: those four values are exactly
//     the lane's A operand (A[row = l % 16][key = 4 (l / 16) + e]); E enters as
//     two bf16 pieces, hi + lo, which keep 16 of its bits.  The B operand
//     (keys 4 (l / 16) + e, dim l % 16 of a 16-dim block) is one 8-byte load
//     from a transposed copy of the keys, Yt[d][m_pad].
//
// A work-group is 4 waves on 64 rows, each wave taking every 4th key tile; the
// waves merge in LDS in a fixed order.  A row block with a row whose mass
// falls outside [2^-64, 2^100] (potentials far from solving these weights) is
// flagged; the fp64 plan pass redoes it.
#include "mfma_bf16.h"

namespace sk {
namespace {

constexpr int kWavesG = 4;
constexpr int kKeysG = 16;
constexpr int kGroupsG = 4;
constexpr float kMassLo = 5.421010862e-20f;  // 2^-64
constexpr float kMassHi = 1.2676506e30f;     // 2^100

template <int DK>
__global__ __launch_bounds__(kWavesG *kWave) void gradFm_kernel(
    const uint16_t *__restrict__ X, const float *__restrict__ xpot, const float *__restrict__ xsq,
    const float *__restrict__ xw, int n, const uint16_t *__restrict__ Y,
    const uint16_t *__restrict__ Yt, const float *__restrict__ ybias, int m, int m_pad,
    float c, float *__restrict__ grad, float *__restrict__ proj, int *__restrict__ redo)
{
    constexpr int d = 32 * DK;
    constexpr int NB = d / 16;   // 16-dim blocks of the output
    __shared__ float osum[kWave][d + 1];
    __shared__ float msum[kWave];
    __shared__ int flag;
    const int b = blockIdx.z;
    const int lane = lane_id();
    const int w = wave_id_uniform();
    const int row0 = blockIdx.x * kWave;
    const int kq = lane >> 4;
    const int c16 = lane & 15;
    const float two_c = 2.0f * c;

    // rows as the B operand of the transposed score; alpha / 2c rides in the
    // accumulator input: 2c (x.y + (f - ||x||^2) / 2) = 2c x.y + alpha
    bf16x8 Xo[kGroupsG][DK];
    f32x4 Cin[kGroupsG];
#pragma unroll
    for (int g = 0; g < kGroupsG; ++g) {
        const int ra = row0 + 16 * g + c16;
        const int rc = min(ra, n - 1);
#pragma unroll
        for (int kb = 0; kb < DK; ++kb) {
            bf16x8 v = load8(X + ((size_t)b * n + rc) * d + 32 * kb + 8 * kq);
            if (ra >= n)
                v = bf16x8{};
            Xo[g][kb] = v;
        }
        const size_t k = (size_t)b * n + rc;
        const float h = ra < n ? (float)(0.5 * ((double)xpot[k] - (double)xsq[k])) : 0.f;
        Cin[g] = f32x4{h, h, h, h};
    }
    f32x4 O[kGroupsG][NB];
    float mass[kGroupsG];
#pragma unroll
    for (int g = 0; g < kGroupsG; ++g) {
        mass[g] = 0.f;
#pragma unroll
        for (int q = 0; q < NB; ++q)
            O[g][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const uint16_t *yb = Y + (size_t)b * m * d;
    const uint16_t *ytb = Yt + (size_t)b * d * m_pad;
    const float *beb = ybias + (size_t)b * m_pad;
    const int n_tiles = m_pad / kKeysG;
    for (int t = w; t < n_tiles; t += kWavesG) {
        const int j = min(t * kKeysG + c16, m - 1);   // padding keys: bias -1e30, E = 0
        bf16x8 Ka[DK];
#pragma unroll
        for (int kb = 0; kb < DK; ++kb)
            Ka[kb] = load8(yb + (size_t)j * d + 32 * kb + 8 * kq);
        const float4 be = *reinterpret_cast<const float4 *>(beb + t * kKeysG + 4 * kq);
        i16x4 Bt[NB];
#pragma unroll
        for (int q = 0; q < NB; ++q)
            Bt[q] = load4(ytb + (size_t)(16 * q + c16) * m_pad + t * kKeysG + 4 * kq);
#pragma unroll
        for (int g = 0; g < kGroupsG; ++g) {
            f32x4 D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ka[0], Xo[g][0], Cin[g], 0, 0, 0);
#pragma unroll
            for (int kb = 1; kb < DK; ++kb)
                D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ka[kb], Xo[g][kb], D, 0, 0, 0);
            const float E[4] = {ex2(fmaf(two_c, D[0], be.x)), ex2(fmaf(two_c, D[1], be.y)),
                                ex2(fmaf(two_c, D[2], be.z)), ex2(fmaf(two_c, D[3], be.w))};
            mass[g] += (E[0] + E[1]) + (E[2] + E[3]);
            i16x4 hi, lo;
            split2(E, hi, lo);
#pragma unroll
            for (int q = 0; q < NB; ++q) {
                O[g][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, Bt[q], O[g][q], 0, 0, 0);
                O[g][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, Bt[q], O[g][q], 0, 0, 0);
            }
        }
    }
    // a row's mass is spread over the four lanes sharing l % 16
#pragma unroll
    for (int g = 0; g < kGroupsG; ++g) {
        mass[g] += __shfl_xor(mass[g], 16, kWave);
        mass[g] += __shfl_xor(mass[g], 32, kWave);
    }
    // waves add their partials into LDS one after another (fixed order)
    for (int v = 0; v < kWavesG; ++v) {
        if (w == v) {
#pragma unroll
            for (int g = 0; g < kGroupsG; ++g) {
#pragma unroll
                for (int q = 0; q < NB; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float &o = osum[16 * g + 4 * kq + r][16 * q + c16];
                        o = v == 0 ? O[g][q][r] : o + O[g][q][r];
                    }
                if (kq == 0) {
                    float &s = msum[16 * g + c16];
                    s = v == 0 ? mass[g] : s + mass[g];
                }
            }
        }
        __syncthreads();
    }
    if (w == 0) {
        const int row = row0 + lane;
        const float ms = msum[lane];
        const bool live = row < n && (xw ? xw[(size_t)b * n + row] > 0.f : true);
        const bool bad = live && !(ms >= kMassLo && ms <= kMassHi);
        const int f = __ballot(bad) != 0 ? 1 : 0;
        if (lane == 0) {
            flag = f;
            redo[b * gridDim.x + blockIdx.x] = f;
        }
    }
    __syncthreads();
    if (flag)
        return;
    const float inv_n = 1.0f / (float)n;
    for (int e = threadIdx.x; e < kWave * d; e += kWavesG * kWave) {
        const int r = e / d, k = e % d;
        const int row = row0 + r;
        if (row >= n)
            continue;
        const size_t o = ((size_t)b * n + row) * d + k;
        const float wi = xw ? xw[(size_t)b * n + row] : inv_n;
        const float ms = msum[r], Ok = osum[r][k];
        const float x = bf16_to_float(X[o]);
        const bool live = wi > 0.f;
        if (grad)
            grad[o] = live ? 2.0f * wi * fmaf(ms, x, -Ok) : 0.f;
        if (proj)
            proj[o] = live ? Ok / ms : 0.f;
    }
}

// Xt[b][k][j] = X[b][j][k] for j < n, 0 for the padding up to n_pad.
__global__ void transpose_bf16_kernel(const uint16_t *__restrict__ X, int n, int n_pad, int d,
                                      uint16_t *__restrict__ Xt)
{
    __shared__ uint16_t tile[64][65];
    const int b = blockIdx.z;
    const int j0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;   // 256 threads: 4 rows a pass
    for (int jj = ty; jj < 64; jj += 4) {
        const int j = j0 + jj, k = k0 + tx;
        tile[jj][tx] = (j < n && k < d) ? X[((size_t)b * n + j) * d + k] : (uint16_t)0;
    }
    __syncthreads();
    for (int kk = ty; kk < 64; kk += 4) {
        const int k = k0 + kk, j = j0 + tx;
        if (k < d && j < n_pad)
            Xt[((size_t)b * d + k) * n_pad + j] = tile[tx][kk];
    }
}

}  // namespace

bool gradF_matrix_cores(int dtype, int d) { return dtype == 1 && (d == 32 || d == 64); }

hipError_t launch_transpose_bf16(const void *X, int B, int n, int n_pad, int d, uint16_t *Xt,
                                 hipStream_t st)
{
    dim3 grid(n_pad / 64, ceil_div(d, 64), B);
    hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, st, (const uint16_t *)X, n,
                       n_pad, d, Xt);
    return hipGetLastError();
}

hipError_t launch_gradFm(const SideF &rows, const float *row_w, const SideF &keys,
                         const uint16_t *keys_t, int d, int B, float eps, float *grad,
                         float *proj, hipStream_t st)
{
    const float c = scale_of(eps);
    dim3 grid(rows.n_pad / kWave, 1, B);
    if (d == 32)
        hipLaunchKernelGGL((gradFm_kernel<1>), grid, dim3(kWavesG * kWave), 0, st,
                           (const uint16_t *)rows.pts, (const float *)rows.pot,
                           (const float *)rows.sq, row_w, rows.n, (const uint16_t *)keys.pts,
                           keys_t, (const float *)keys.bias, keys.n, keys.n_pad, c, grad, proj,
                           rows.redo);
    else
        hipLaunchKernelGGL((gradFm_kernel<2>), grid, dim3(kWavesG * kWave), 0, st,
                           (const uint16_t *)rows.pts, (const float *)rows.pot,
                           (const float *)rows.sq, row_w, rows.n, (const uint16_t *)keys.pts,
                           keys_t, (const float *)keys.bias, keys.n, keys.n_pad, c, grad, proj,
                           rows.redo);
    return hipGetLastError();
}

}  // namespace sk

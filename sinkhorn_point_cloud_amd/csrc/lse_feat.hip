// lse_feat.hip -- fused streaming half-iteration for feature clouds of
// dimension d <= 128 (fp32 or bf16 points): a vector-ALU kernel for any such d,
// and, for bf16 points with d a multiple of 32, a matrix-core kernel (below).
//
// Same update as lse_d3.hip (FlashSinkhorn summary, Methodologie 1,
// Propositie 1; streaming per Methodologie 2), in base 2:
//     s_ij = 2c (x_i . y_j) + beta_j,  beta_j = c (g_j - ||y_j||^2) + log2 w_j,
//     f_i  = ||x_i||^2 - (eps ln2) * log2 sum_j 2^(s_ij),   c = log2(e)/eps,
// with beta in a separate bias array and the true potentials as the state
// (row results and biases formed in fp64 and rounded once).
//
// Vector kernel: each lane owns one query row, held in registers as fp32.  A
// work-group of 4 waves shares 64 rows; per step the group stages 4 tiles of kKeys keys in
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
                             float *__restrict__ pot, float *__restrict__ l2w,
                             float *__restrict__ sqo, double c0)
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
    sqo[k] = sq;
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

// One 64-row block rb of pair b (of B), the keys of split `split`, with the
// kWaves waves of the calling work-group (every one must call it).
template <typename T, int DP>
__device__ __forceinline__ void lseF_block(
    const T *__restrict__ qx_, float *__restrict__ qbias, float *__restrict__ qpot,
    const float *__restrict__ ql2w, const T *__restrict__ ky_, const float *__restrict__ kbias,
    float2 *__restrict__ part, int rb, int split, int b, int B, int d, int nq, int nq_pad,
    int nk, int nk_pad, int tiles_per_split, float two_c, double eps_ln2, double c_next)
{
    __shared__ float4 tile[kWaves][kKeys][DP / 4];
    __shared__ float2 red[kWaves][kWave];
    const int lane = lane_id();
    const int w = wave_id_uniform();
    const int row = rb * kWave + lane;

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
        part[((size_t)split * B + b) * nq_pad + row] = make_float2(M, S);
        return;
    }
    if (row < nq)
        finish_row(qbias, qpot, ql2w, (size_t)b * nq_pad + row, (size_t)b * nq + row,
                   row_sq(q, d), M, S, eps_ln2, c_next);
}

template <typename T, int DP>
__global__ __launch_bounds__(kWaves *kWave) void lseF_kernel(
    const T *__restrict__ qx_, float *__restrict__ qbias, float *__restrict__ qpot,
    const float *__restrict__ ql2w, const T *__restrict__ ky_, const float *__restrict__ kbias,
    float2 *__restrict__ part, int d, int nq, int nq_pad, int nk, int nk_pad,
    int tiles_per_split, float two_c, double eps_ln2, double c_next)
{
    lseF_block<T, DP>(qx_, qbias, qpot, ql2w, ky_, kbias, part, blockIdx.x, blockIdx.y,
                      blockIdx.z, gridDim.z, d, nq, nq_pad, nk, nk_pad, tiles_per_split, two_c,
                      eps_ln2, c_next);
}

// ---------------------------------------------------------------------------
// Matrix-core variant for bf16 features with d a multiple of 32 (the
// high-dimensional workload).  The score's dot product x_i . y_j is a real
// dense contraction: v_mfma_f32_16x16x32_bf16 multiplies bf16 inputs exactly
// and accumulates in fp32, one instruction per 16 x 16 block and 32 dims.
// Lane l supplies A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16],
// e = 0..7, and receives D[4 (l / 16) + r][l % 16] (layout checked with an
// in-bounds probe).  The factor 2c is applied in fp32 after the product, never
// to the bf16 inputs.  (32 x 32 x 16 blocks, half the matrix instructions per
// entry, were measured slower: 495 against 466 us per feat-50k half-iteration;
// a wave then covers 32 rows, which doubles the LDS reads per entry.)
//
// Shifted streaming as in lse_d3.hip: row i streams against
// M_i = c (||x_i||^2 - f_i), carried in the accumulator input as
// -M_i / (2c) = -(||x_i||^2 - f_i) / 2, so one fma with the column bias gives
// s_ij - M_i = 2c D_ij + beta_j.  With one shift per row, partial sums over
// key ranges simply add.
//
// Work partition (stream-K): a work-group of 16 waves owns 1024 consecutive rows
// (a row group; each wave 64 rows as four 16-row groups), and the key tiles of every row group are
// laid end to end, pair by pair, into one range of units (row group, 16-key
// tile).  A launch has a fixed number of work-groups (one per compute unit, 4
// waves per SIMD, or one per row group when there are more row groups), and
// work-group w takes
// the units [w U / P, (w + 1) U / P): equal shares, so every compute unit
// finishes together, whatever the row and key counts.  A share spans at most
// two row groups; for each it writes the partial sums of its rows to slot
// (w, 0) or (w, 1).  The keys of a share stream through LDS (double buffered,
// 256 keys a stage, loaded cooperatively with 16-byte accesses) and the 16
// waves read them from there, so each key tile is fetched once per 1024 rows
// (16 waves: 1% faster than two work-groups of 8 per compute unit).  The finalize kernel adds, for every row, the
// partials of the work-groups that cover its row group in increasing order
// (a fixed order: the result does not depend on timing), turns the sums into
// potentials and biases, and recomputes on the vector ALUs, in the same
// launch, a 64-row block whose sum left [2^-64, 2^100] (a stale shift).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int kGroups = 4;
constexpr float kSumLo = 5.421010862e-20f;  // 2^-64
constexpr float kSumHi = 1.2676506e30f;     // 2^100

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t *p)
{
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    return __builtin_bit_cast(bf16x8, v);
}

constexpr int kSWaves = 16;                     // waves per work-group
constexpr int kSRows = 16 * kGroups;            // rows per wave
constexpr int kSGroupRows = kSWaves * kSRows;   // rows per row group (work-group)
constexpr int kSKeys = 16;                      // keys per tile
constexpr int kSStageTiles = 16;                // tiles per LDS stage (256 keys)
constexpr int kSSlots = 256;                    // work-groups per launch: 1 per compute unit

// The stream-K partition of one pass: G row groups (B pairs x RG each), T
// tiles per row, U = G T units, P work-groups.
struct Part {
    int RG, T, P;
    long long U;
};

// First unit of work-group w (w = P gives U).  When P T == U (one work-group
// per row group) the shares are whole row groups.
__device__ __forceinline__ long long share_lo(int w, const Part &pt)
{
    return pt.U == (long long)pt.P * pt.T ? (long long)w * pt.T : (long long)w * pt.U / pt.P;
}

// The work-group whose share holds unit u (the largest w with share_lo(w) <= u).
__device__ __forceinline__ int share_of(long long u, const Part &pt)
{
    if (pt.U == (long long)pt.P * pt.T)
        return (int)(u / pt.T);
    return (int)(((u + 1) * pt.P - 1) / pt.U);
}

template <int DK>
__global__ __launch_bounds__(kSWaves *kWave) void lseFs_kernel(
    const uint16_t *__restrict__ qx_, const float *__restrict__ qpot,
    const float *__restrict__ qsq, const uint16_t *__restrict__ ky_,
    const float *__restrict__ kbias, float *__restrict__ part, int nq, int nk, int nk_pad,
    Part pt, float two_c)
{
    constexpr int d = 32 * DK;
    constexpr int kStageKeys = kSStageTiles * kSKeys;   // 256
    constexpr int kChunks = d / 8;                      // 16-byte chunks per key
    constexpr int kStride = kChunks + 1;                // padded key stride in LDS (bank spread)
    constexpr int kTotal = kStageKeys * kChunks;        // 16-byte chunks per stage
    constexpr int kThreads = kSWaves * kWave;
    constexpr int kLoads = kTotal / kThreads;        // 16-byte chunks per thread and stage
    static_assert(kTotal % kThreads == 0 && kLoads <= 4, "whole chunks per thread");
    __shared__ uint4 kbuf[2][kStageKeys * kStride];
    __shared__ float bbuf[2][kStageKeys];
    const int wg = blockIdx.x;
    const int lane = lane_id();
    const int w = wave_id_uniform();
    const int kq = lane >> 4;      // operand k index this lane supplies / row quad it receives
    const int c16 = lane & 15;     // operand row (A) or column (B) within a 16-block
    const int e0 = threadIdx.x;

    const long long u_end = share_lo(wg + 1, pt);
    long long u = share_lo(wg, pt);
    for (int seg = 0; u < u_end && seg < 2; ++seg) {   // a share spans <= 2 row groups
        const long long gb = u / pt.T;                    // pair-major row group
        const long long g_end = (gb + 1) * pt.T;
        const int t0 = (int)(u - gb * pt.T);
        const int t1 = (int)((u_end < g_end ? u_end : g_end) - gb * pt.T);
        u = u_end < g_end ? u_end : g_end;
        const int b = (int)(gb / pt.RG);
        const int row0 = (int)(gb % pt.RG) * kSGroupRows + w * kSRows;   // this wave's rows
        const bool live = row0 < nq;   // wave-uniform: a wave past the last row only loads

        bf16x8 A[kGroups][DK];
        f32x4 Cn[kGroups], S[kGroups];
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            const int ra = row0 + 16 * g + c16;      // row whose operand this lane supplies
            const int rc = min(ra, nq - 1);
#pragma unroll
            for (int kb = 0; kb < DK; ++kb) {
                bf16x8 v = load_bf16x8(qx_ + ((size_t)b * nq + rc) * d + 32 * kb + 8 * kq);
                if (ra >= nq)
                    v = bf16x8{};
                A[g][kb] = v;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rr = row0 + 16 * g + 4 * kq + r;   // row whose results this lane holds
                float sh = 0.f;
                if (rr < nq) {
                    const size_t k = (size_t)b * nq + rr;
                    sh = -0.5f * (qsq[k] - qpot[k]);
                }
                Cn[g][r] = sh;
                S[g][r] = 0.f;
            }
        }
        const uint4 *ky = reinterpret_cast<const uint4 *>(ky_ + (size_t)b * nk * d);
        const float *kb_ = kbias + (size_t)b * nk_pad;
        const int n_stages = (t1 - t0 + kSStageTiles - 1) / kSStageTiles;

        // cooperative stage load: chunk e of the stage is part e % kChunks of its
        // key e / kChunks; keys past the share's last tile get bias -1e30 (they
        // add exactly 0) and their point index is clamped inside the pair.  A
        // thread's chunks of the next stage are loaded into registers while the
        // current stage is consumed, then written to the other LDS buffer.
        uint4 ld0, ld1, ld2, ld3;   // the first kLoads of them are used
        float lb = kNeg;
        auto fetch = [&](int s) {
            const int key0 = (t0 + s * kSStageTiles) * kSKeys;
            auto one = [&](int i) {
                const int e = e0 + i * kThreads;
                return ky[(size_t)min(key0 + e / kChunks, nk - 1) * kChunks + e % kChunks];
            };
            ld0 = one(0);
            if constexpr (kLoads > 1)
                ld1 = one(1);
            if constexpr (kLoads > 2)
                ld2 = one(2);
            if constexpr (kLoads > 3)
                ld3 = one(3);
            if (e0 < kStageKeys)
                lb = key0 + e0 < t1 * kSKeys ? kb_[key0 + e0] : kNeg;
        };
        auto stash = [&](int buf) {
            auto one = [&](int i, const uint4 &v) {
                const int e = e0 + i * kThreads;
                kbuf[buf][(e / kChunks) * kStride + e % kChunks] = v;
            };
            one(0, ld0);
            if constexpr (kLoads > 1)
                one(1, ld1);
            if constexpr (kLoads > 2)
                one(2, ld2);
            if constexpr (kLoads > 3)
                one(3, ld3);
            if (e0 < kStageKeys)
                bbuf[buf][e0] = lb;
        };
        fetch(0);
        stash(0);
        __syncthreads();
        for (int s = 0; s < n_stages; ++s) {
            const int buf = s & 1;
            if (s + 1 < n_stages)
                fetch(s + 1);   // in flight while this stage is consumed
            if (live) {
#pragma unroll 1
                for (int tt = 0; tt < kSStageTiles; ++tt) {
                    bf16x8 Bv[DK];
#pragma unroll
                    for (int kb = 0; kb < DK; ++kb)
                        Bv[kb] = __builtin_bit_cast(
                            bf16x8, kbuf[buf][(tt * kSKeys + c16) * kStride + 4 * kb + kq]);
                    const float be = bbuf[buf][tt * kSKeys + c16];
#pragma unroll
                    for (int g = 0; g < kGroups; ++g) {
                        f32x4 D =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][0], Bv[0], Cn[g], 0, 0, 0);
#pragma unroll
                        for (int kb = 1; kb < DK; ++kb)
                            D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][kb], Bv[kb], D, 0, 0,
                                                                        0);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            S[g][r] += ex2(fmaf(two_c, D[r], be));
                    }
                }
            }
            if (s + 1 < n_stages)
                stash(buf ^ 1);
            __syncthreads();
        }
        // row sums: each of the 16 lanes of a row holds one key column
        float *out = part + ((size_t)wg * 2 + seg) * kSGroupRows + w * kSRows;
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = row16_sum(S[g][r]);
                if (c16 == 0 && live)
                    out[16 * g + 4 * kq + r] = v;
            }
    }
}

// Sum of the partials of every row (fixed order), potentials and biases; a
// 64-row block with a sum out of range is recomputed by the work-group's waves
// on the vector ALUs with an online maximum over all keys.
template <int DP>
__global__ __launch_bounds__(kWaves *kWave) void lseFs_finalize(
    const uint16_t *__restrict__ qx_, float *__restrict__ qbias, float *__restrict__ qpot,
    const float *__restrict__ ql2w, const float *__restrict__ qsq,
    const uint16_t *__restrict__ ky_, const float *__restrict__ kbias,
    const float *__restrict__ part, int B, int d, int nq, int nq_pad, int nk, int nk_pad,
    Part pt, float two_c, double eps_ln2, double c_next)
{
    __shared__ int stale;
    const int b = blockIdx.y;
    const int row = blockIdx.x * kWave + lane_id();
    const int w = wave_id_uniform();
    float Ssum = 0.f;
    if (w == 0) {
        if (row < nq) {
            const long long gb = (long long)b * pt.RG + row / kSGroupRows;
            const int rr = row % kSGroupRows;
            const int w0 = share_of(gb * pt.T, pt), w1 = share_of(gb * pt.T + pt.T - 1, pt);
            for (int v = w0; v <= w1; ++v) {
                const int seg = share_lo(v, pt) / pt.T == gb ? 0 : 1;
                Ssum += part[((size_t)v * 2 + seg) * kSGroupRows + rr];
            }
        }
        const bool bad = row < nq && !(Ssum >= kSumLo && Ssum <= kSumHi);
        const int flag = __builtin_amdgcn_readfirstlane(__ballot(bad) != 0 ? 1 : 0);
        if (lane_id() == 0)
            stale = flag;
    }
    __syncthreads();
    if (stale) {
        lseF_block<uint16_t, DP>(qx_, qbias, qpot, ql2w, ky_, kbias, nullptr, blockIdx.x, 0, b,
                                 B, d, nq, nq_pad, nk, nk_pad, nk_pad / kKeys, two_c, eps_ln2,
                                 c_next);
        return;
    }
    if (w != 0 || row >= nq)
        return;
    const size_t k = (size_t)b * nq + row;
    const float sqf = qsq[k];
    const double sq = (double)sqf;
    // the shift the partial kernels used: s - M = 2c (x.y + Cn) + beta, M = -2c Cn
    const float Cn = -0.5f * (sqf - qpot[k]);
    const double M = -2.0 * (0.5 * (double)two_c) * (double)Cn;
    const double lse2 = M + (double)lg2(Ssum);
    const float f = (float)(sq - lse2 * eps_ln2);
    qpot[k] = f;
    qbias[(size_t)b * nq_pad + row] = bias_of(c_next, f, sqf, ql2w[k]);
}

// Transport cost for the bf16 matrix-core path, streamed like a half-
// iteration: with both biases of the final passes (c (f - ||x||^2) + log2 a and
// c (g - ||y||^2) + log2 b at the last eps),
//     log2 P_ij = 2c x_i . y_j + beta_j + alpha_i,
//     C_ij = ||x_i||^2 + ||y_j||^2 - 2 x_i . y_j,
// and each row's sum_j P_ij C_ij goes to row_out (fp64) for a fixed-order
// per-pair reduction.  No n x m quantity is stored.
template <int DK>
__global__ __launch_bounds__(kWaves *kWave) void costFm_kernel(
    const uint16_t *__restrict__ X, const float *__restrict__ xbias, const float *__restrict__ xsq,
    const uint16_t *__restrict__ Y, const float *__restrict__ ybias, const float *__restrict__ ysq,
    int n, int n_pad, int m, int m_pad, float two_c, double *__restrict__ row_out)
{
    constexpr int d = 32 * DK;
    __shared__ float red[kWaves][kWave];
    const int b = blockIdx.z;
    const int lane = lane_id();
    const int w = wave_id_uniform();
    const int row0 = blockIdx.x * kWave;
    const int kq = lane >> 4;
    const int c16 = lane & 15;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    bf16x8 A[kGroups][DK];
    f32x4 al[kGroups], sqx[kGroups], acc[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        const int ra = row0 + 16 * g + c16;
        const int rc = min(ra, n - 1);
#pragma unroll
        for (int kb = 0; kb < DK; ++kb) {
            bf16x8 v = load_bf16x8(X + ((size_t)b * n + rc) * d + 32 * kb + 8 * kq);
            if (ra >= n)
                v = bf16x8{};
            A[g][kb] = v;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = row0 + 16 * g + 4 * kq + r;
            al[g][r] = rr < n ? xbias[(size_t)b * n_pad + rr] : kNeg;
            sqx[g][r] = rr < n ? xsq[(size_t)b * n + rr] : 0.f;
            acc[g][r] = 0.f;
        }
    }
    const uint16_t *yb = Y + (size_t)b * m * d;
    const int n_tiles = m_pad / kKeys;
    for (int t = w; t < n_tiles; t += kWaves) {
        const int jr = t * kKeys + c16;
        const int j = min(jr, m - 1);
        bf16x8 Bv[DK];
#pragma unroll
        for (int kb = 0; kb < DK; ++kb)
            Bv[kb] = load_bf16x8(yb + (size_t)j * d + 32 * kb + 8 * kq);
        const float be = jr < m ? ybias[(size_t)b * m_pad + jr] : kNeg;
        const float sy = ysq[(size_t)b * m + j];
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            f32x4 D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][0], Bv[0], zero, 0, 0, 0);
#pragma unroll
            for (int kb = 1; kb < DK; ++kb)
                D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][kb], Bv[kb], D, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float P = ex2(fmaf(two_c, D[r], be) + al[g][r]);
                const float C = fmaf(-2.f, D[r], sqx[g][r] + sy);
                acc[g][r] = fmaf(P, C, acc[g][r]);
            }
        }
    }
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = row16_sum(acc[g][r]);
            if (c16 == 0)
                red[w][16 * g + 4 * kq + r] = v;
        }
    __syncthreads();
    if (w != 0)
        return;
    double tot = 0.0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v)
        tot += (double)red[v][lane];
    const int row = row0 + lane;
    if (row < n)
        row_out[(size_t)b * n + row] = tot;
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

// Stream-K partition of a matrix-core pass: 1024-row groups of every pair,
// 16-key tiles; one work-group per compute unit, or one per row group when
// there are more row groups (then a share never spans more than two groups:
// every share is at most one row group long).  At least 16 tiles per share.
Part lseFs_part(int B, int nq_pad, int nk_pad)
{
    Part pt;
    pt.RG = ceil_div(nq_pad, kSGroupRows);
    pt.T = nk_pad / kSKeys;
    const long long G = (long long)B * pt.RG;
    pt.U = G * pt.T;
    long long P = pt.U / 16;
    if (P > kSSlots)
        P = kSSlots;
    if (P < G)
        P = G;
    pt.P = (int)P;
    return pt;
}

template <int DK>
void launch_lseFs_t(SideF q, SideF k, int B, float two_c, double eps_ln2, double c_next,
                    float *part, hipStream_t st)
{
    const Part pt = lseFs_part(B, q.n_pad, k.n_pad);
    hipLaunchKernelGGL((lseFs_kernel<DK>), dim3(pt.P), dim3(kSWaves * kWave), 0, st,
                       (const uint16_t *)q.pts, (const float *)q.pot, (const float *)q.sq,
                       (const uint16_t *)k.pts, (const float *)k.bias, part, q.n, k.n, k.n_pad,
                       pt, two_c);
    constexpr int DP = 32 * DK;
    hipLaunchKernelGGL((lseFs_finalize<DP>), dim3(q.n_pad / kWave, B), dim3(kWaves * kWave), 0,
                       st, (const uint16_t *)q.pts, q.bias, q.pot, (const float *)q.l2w,
                       (const float *)q.sq, (const uint16_t *)k.pts, (const float *)k.bias,
                       (const float *)part, B, DP, q.n, q.n_pad, k.n, k.n_pad, pt, two_c,
                       eps_ln2, c_next);
}

// Matrix cores for bf16 with whole 32-dim blocks, 16-byte aligned rows (the
// operands are read as 16-byte vectors) and at least 128 row blocks.
bool use_matrix_cores(SideF q, SideF k, int dtype, int d, int B)
{
    const bool aligned = ((uintptr_t)q.pts % 16 == 0) && ((uintptr_t)k.pts % 16 == 0);
    return dtype == 1 && d % 32 == 0 && d <= 128 && aligned && (long)B * (q.n_pad / kWave) >= 128;
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

bool lseF_matrix_cores(SideF q, SideF k, int dtype, int d, int B)
{
    return use_matrix_cores(q, k, dtype, d, B) && use_matrix_cores(k, q, dtype, d, B);
}

hipError_t launch_costFm(SideF x, SideF y, int d, int B, float eps, double *row_part,
                         hipStream_t st)
{
    const float two_c = 2.0f * scale_of(eps);
    dim3 grid(x.n_pad / kWave, 1, B);
#define SK_COSTFM(DK)                                                                      \
    hipLaunchKernelGGL((costFm_kernel<DK>), grid, dim3(kWaves * kWave), 0, st,                 \
                       (const uint16_t *)x.pts, (const float *)x.bias, (const float *)x.sq,     \
                       (const uint16_t *)y.pts, (const float *)y.bias, (const float *)y.sq, x.n, \
                       x.n_pad, y.n, y.n_pad, two_c, row_part)
    switch (d / 32) {
    case 1: SK_COSTFM(1); break;
    case 2: SK_COSTFM(2); break;
    case 3: SK_COSTFM(3); break;
    default: SK_COSTFM(4); break;
    }
#undef SK_COSTFM
    return hipGetLastError();
}

// float2 slots of partial-state workspace: the vector path's split (M, S) states
// or the matrix-core path's split sums (one float each), whichever is larger
size_t lseF_partial_floats2(int B, int nq_pad, int nk_pad)
{
    const int s = lseF_splits(B, nq_pad, nk_pad);
    const size_t vec = s > 1 ? (size_t)s * B * nq_pad : 0;
    const size_t mat = (size_t)lseFs_part(B, nq_pad, nk_pad).P * kSGroupRows;   // 2 floats each
    return vec > mat ? vec : mat;
}

hipError_t launch_packF(const void *X, int dtype, int d, const float *w, int warm, int B,
                        SideF s, double c0, hipStream_t st)
{
    dim3 grid(ceil_div(s.n_pad, 256), B);
    if (dtype == 1)
        hipLaunchKernelGGL(packF_kernel<uint16_t>, grid, dim3(256), 0, st,
                           (const uint16_t *)X, d, w, warm, s.n, s.n_pad, s.bias, s.pot, s.l2w,
                           s.sq, c0);
    else
        hipLaunchKernelGGL(packF_kernel<float>, grid, dim3(256), 0, st, (const float *)X, d, w,
                           warm, s.n, s.n_pad, s.bias, s.pot, s.l2w, s.sq, c0);
    return hipGetLastError();
}

hipError_t launch_lseF(SideF q, SideF k, int dtype, int d, int B, float eps, float eps_next,
                       float2 *part, hipStream_t st)
{
    const float c = scale_of(eps);
    const double c_next = (double)scale_of(eps_next);
    const double eps_ln2 = 1.0 / (double)c;
    if (use_matrix_cores(q, k, dtype, d, B)) {
        switch (d / 32) {
        case 1: launch_lseFs_t<1>(q, k, B, 2.0f * c, eps_ln2, c_next, (float *)part, st); break;
        case 2: launch_lseFs_t<2>(q, k, B, 2.0f * c, eps_ln2, c_next, (float *)part, st); break;
        case 3: launch_lseFs_t<3>(q, k, B, 2.0f * c, eps_ln2, c_next, (float *)part, st); break;
        default: launch_lseFs_t<4>(q, k, B, 2.0f * c, eps_ln2, c_next, (float *)part, st); break;
        }
    } else if (dtype == 1)
        dispatch<uint16_t>(q, k, d, B, 2.0f * c, eps_ln2, c_next, part, st);
    else
        dispatch<float>(q, k, d, B, 2.0f * c, eps_ln2, c_next, part, st);
    return hipGetLastError();
}

}  // namespace sk

// plan_rows_mc.h -- the matrix-core row pass over a transport plan for bf16
// feature clouds (d = 32 or 64), shared by the dense gradient (grad_feat.hip)
// and the Hessian-vector product (hvp_feat.hip).
//
// The plan is written as P_ij = a_i E_ij with
//     E_ij = 2^(2c (x_i.y_j + h_i) + beta_j),   h_i = (f_i - ||x_i||^2) / 2,
//     beta_j = c (g_j - ||y_j||^2) + log2 b_j,   c = log2(e)/eps
// (FlashSinkhorn summary, Methodologie 3, Toepassing van Transportmatrix: sums
// over the plan streamed like the update, the plan never stored).  Per 16-key
// tile the scores come out of v_mfma_f32_16x16x32_bf16 with the keys as A and a
// 16-row group as B (h_i rides in the accumulator input), so a lane holds E for
// row l % 16 and keys 4 (l / 16) + r: exactly the A operand of the
// v_mfma_f32_16x16x16_bf16 that forms E Y against the transposed keys, with E in
// two bf16 pieces (hi + lo, 16 bits).  Row pass modes:
//     mass:   m_i = sum_j E_ij,  O_i = sum_j E_ij y_j;
//     first:  the same and Q_i = sum_j E_ij (v_i.y_j) y_j (v_i as a third B operand);
//     CG:     e_i = sum_j E_ij u_j;
//     final:  e_i and W_i = sum_j E_ij u_j y_j.
#pragma once

#include "mfma_bf16.h"

#include <algorithm>

namespace sk {
namespace mc {

constexpr int kWaves = 8;    // waves per work-group
constexpr int kTile = 16;    // keys (or rows) per streamed tile
constexpr int kMaxSplits = 64;

enum : int { kRowsCg = 0, kRowsFirst = 1, kRowsFinal = 2, kRowsMass = 3 };

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

__device__ __forceinline__ f32x4 score(const bf16x8 (&A)[2], const bf16x8 (&Bm)[2], f32x4 C,
                                       int dk)
{
    f32x4 D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0], Bm[0], C, 0, 0, 0);
    if (dk == 2)
        D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1], Bm[1], D, 0, 0, 0);
    return D;
}

// S splits of tps tiles for `blocks` work-groups' worth of points (all pairs)
// against `tiles` streamed tiles, aiming at `target` work-groups.  When the
// points alone give enough work-groups there is one split; otherwise S is a
// multiple of the 8 XCDs where the tiles allow: work-groups are dealt to them
// round-robin by linear index, split fastest, so each XCD keeps to the same
// key ranges.
struct Split {
    int S, tps;
};
inline Split split_of(int blocks, int tiles, int target)
{
    const int need = ceil_div(target, std::max(1, blocks));
    const int want = need <= 1 ? 1 : std::min(round_up(need, 8), kMaxSplits);
    Split sp;
    sp.tps = ceil_div(tiles, want);
    sp.S = ceil_div(tiles, sp.tps);
    return sp;
}

// Rows pass.  Work-group blockIdx.y holds kWaves G groups of 16 rows, G per
// wave; pair blockIdx.z; the key tiles of split blockIdx.x stream through LDS
// NT tiles a stage (double buffered: every thread loads its share of the next
// stage into registers while the current one is used, then writes it to the
// other buffer), and every wave reads its operands from there, so a key tile
// is fetched once per work-group.  part_s [S][B][n_pad]: m_i (first, mass) or
// e_i; part_v [S][B][n_pad][d]: O_i (first, mass) or W_i (final); part_q: Q_i
// (first).
template <int DK, int G, int NT, int MODE>
__global__ __launch_bounds__(kWaves *kWave) void rows_kernel(
    const uint16_t *__restrict__ X, const float *__restrict__ h, int n, int n_pad,
    const uint16_t *__restrict__ Y, const uint16_t *__restrict__ Yt,
    const float *__restrict__ ybias, int m, int m_pad, const uint16_t *__restrict__ vh,
    const uint16_t *__restrict__ vl, const float *__restrict__ u, float two_c, int tps,
    float *__restrict__ part_s, float *__restrict__ part_v, float *__restrict__ part_q)
{
    constexpr int d = 32 * DK;
    constexpr int NB = d / 16;
    constexpr int R = 16 * G;   // rows per wave
    constexpr bool kVec = MODE != kRowsCg;
    constexpr bool kQ = MODE == kRowsFirst;
    constexpr bool kU = MODE == kRowsCg || MODE == kRowsFinal;
    constexpr int SK = NT * kTile;                        // keys per stage
    constexpr int kCh = d / 8;                             // 16-byte chunks per key
    constexpr int kStr = kCh + 1;                          // padded key stride (bank spread)
    constexpr int kThr = kWaves * kWave;
    constexpr int kKL = (SK * kCh + kThr - 1) / kThr;      // key chunks per thread
    constexpr int kTCh = SK / 8;                           // chunks of one dim row of Yt
    constexpr int kTStr = SK + 8;                          // padded dim row (bf16)
    constexpr int kTL = kVec ? (d * kTCh + kThr - 1) / kThr : 1;
    static_assert(SK <= kThr && kKL <= 2 && kTL <= 2, "a stage in at most two chunks a thread");
    __shared__ uint4 kbuf[2][SK * kStr];
    __shared__ __align__(16) float bbuf[2][SK];
    __shared__ __align__(16) float ubuf[2][kU ? SK : 4];
    __shared__ __align__(16) uint16_t tbuf[2][kVec ? d * kTStr : 8];
    const int split = blockIdx.x, b = blockIdx.z, B = gridDim.z;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id_uniform();
    const int kq = lane >> 4, c16 = lane & 15;
    const int row0 = (blockIdx.y * kWaves + w) * R;   // + R <= n_pad

    // the rows as the B operand of the transposed score, h_i in the accumulator
    bf16x8 Xo[G][2], Vh[kQ ? G : 1][2], Vl[kQ ? G : 1][2];
    f32x4 Cin[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int ra = row0 + 16 * g + c16;
        const int rc = min(ra, n - 1);
#pragma unroll
        for (int kb = 0; kb < DK; ++kb)
            Xo[g][kb] = load8(X + ((size_t)b * n + rc) * d + 32 * kb + 8 * kq);
        const float hv = h[(size_t)b * n_pad + ra];
        Cin[g] = f32x4{hv, hv, hv, hv};
        if constexpr (kQ) {
#pragma unroll
            for (int kb = 0; kb < DK; ++kb) {
                const size_t o = ((size_t)b * n_pad + ra) * d + 32 * kb + 8 * kq;
                Vh[g][kb] = load8(vh + o);
                Vl[g][kb] = load8(vl + o);
            }
        }
    }
    float acc[G];
    f32x4 O[kVec ? G : 1][NB], Q[kQ ? G : 1][NB];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        acc[g] = 0.f;
        if constexpr (kVec) {
#pragma unroll
            for (int q = 0; q < NB; ++q)
                O[g][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if constexpr (kQ) {
#pragma unroll
            for (int q = 0; q < NB; ++q)
                Q[g][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    const uint4 *yk = reinterpret_cast<const uint4 *>(Y + (size_t)b * m * d);
    const uint16_t *ytb = Yt + (size_t)b * d * m_pad;
    const float *beb = ybias + (size_t)b * m_pad;
    const float *ub = kU ? u + (size_t)b * m_pad : nullptr;
    const int n_tiles = m_pad / kTile;
    const int t0 = split * tps, t1 = min(n_tiles, t0 + tps);
    const int n_st = t0 < t1 ? (t1 - t0 + NT - 1) / NT : 0;   // uniform per work-group
    // A stage's values: key chunk e is chunk e % kCh of key e / kCh (keys past
    // the pair clamped inside it; their bias is kNeg), bias and u of key tid,
    // and chunk e of the transposed keys (dim e / kTCh, 8 keys from 8 (e % kTCh)).
    // (named registers, not arrays: an array written in one lambda and read in
    // the other stays in scratch memory)
    uint4 kr0 = zero4(), kr1 = zero4(), tr0 = zero4(), tr1 = zero4();
    float br = kNeg, ur = 0.f;
    const int kend = t1 * kTile;
    auto key_chunk = [&](int key0, int e) {
        return e < SK * kCh ? yk[(size_t)min(key0 + e / kCh, m - 1) * kCh + e % kCh] : zero4();
    };
    auto yt_chunk = [&](int key0, int e) {
        const int kk = key0 + 8 * (e % kTCh);   // a multiple of 8, as is m_pad
        return e < d * kTCh && kk < m_pad
                   ? *reinterpret_cast<const uint4 *>(ytb + (size_t)(e / kTCh) * m_pad + kk)
                   : zero4();
    };
    auto fetch = [&](int st) {
        const int key0 = (t0 + st * NT) * kTile;
        kr0 = key_chunk(key0, tid);
        if constexpr (kKL > 1)
            kr1 = key_chunk(key0, tid + kThr);
        if (tid < SK) {
            const int kk = key0 + tid;
            br = kk < kend ? beb[kk] : kNeg;
            if constexpr (kU)
                ur = kk < kend ? ub[kk] : 0.f;
        }
        if constexpr (kVec) {
            tr0 = yt_chunk(key0, tid);
            if constexpr (kTL > 1)
                tr1 = yt_chunk(key0, tid + kThr);
        }
    };
    auto put_key = [&](int bf, int e, uint4 v) {
        if (e < SK * kCh)
            kbuf[bf][(e / kCh) * kStr + e % kCh] = v;
    };
    auto put_yt = [&](int bf, int e, uint4 v) {
        if (e < d * kTCh)
            *reinterpret_cast<uint4 *>(&tbuf[bf][(e / kTCh) * kTStr + 8 * (e % kTCh)]) = v;
    };
    auto stash = [&](int bf) {
        put_key(bf, tid, kr0);
        if constexpr (kKL > 1)
            put_key(bf, tid + kThr, kr1);
        if (tid < SK) {
            bbuf[bf][tid] = br;
            if constexpr (kU)
                ubuf[bf][tid] = ur;
        }
        if constexpr (kVec) {
            put_yt(bf, tid, tr0);
            if constexpr (kTL > 1)
                put_yt(bf, tid + kThr, tr1);
        }
    };
    if (n_st > 0) {
        fetch(0);
        stash(0);
        __syncthreads();
    }
    for (int st = 0; st < n_st; ++st) {
        const int bf = st & 1;
        if (st + 1 < n_st)
            fetch(st + 1);   // in flight while this stage is used
        const int nt = min(NT, t1 - (t0 + st * NT));
        for (int tt = 0; tt < nt; ++tt) {
            bf16x8 Ka[2];
#pragma unroll
            for (int kb = 0; kb < DK; ++kb)
                Ka[kb] = __builtin_bit_cast(bf16x8,
                                            kbuf[bf][(tt * kTile + c16) * kStr + 4 * kb + kq]);
            const float4 be = *reinterpret_cast<const float4 *>(&bbuf[bf][tt * kTile + 4 * kq]);
            float4 uu = make_float4(0.f, 0.f, 0.f, 0.f);
            if constexpr (kU)
                uu = *reinterpret_cast<const float4 *>(&ubuf[bf][tt * kTile + 4 * kq]);
            i16x4 Bt[kVec ? NB : 1];
            if constexpr (kVec) {
#pragma unroll
                for (int q = 0; q < NB; ++q)
                    Bt[q] = *reinterpret_cast<const i16x4 *>(
                        &tbuf[bf][(16 * q + c16) * kTStr + tt * kTile + 4 * kq]);
            }
            // every group's scores first, so the exponentials do not wait on the
            // matrix cores
            f32x4 D[G];
#pragma unroll
            for (int g = 0; g < G; ++g)
                D[g] = score(Ka, Xo[g], Cin[g], DK);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float E[4] = {ex2(fmaf(two_c, D[g][0], be.x)),
                                    ex2(fmaf(two_c, D[g][1], be.y)),
                                    ex2(fmaf(two_c, D[g][2], be.z)),
                                    ex2(fmaf(two_c, D[g][3], be.w))};
                if constexpr (MODE == kRowsCg) {
                    float s = fmaf(E[0], uu.x, acc[g]);
                    s = fmaf(E[1], uu.y, s);
                    s = fmaf(E[2], uu.z, s);
                    acc[g] = fmaf(E[3], uu.w, s);
                } else if constexpr (MODE == kRowsFirst) {
                    acc[g] += (E[0] + E[1]) + (E[2] + E[3]);
                    f32x4 Sv = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < DK; ++kb) {
                        Sv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ka[kb], Vh[g][kb], Sv, 0, 0, 0);
                        Sv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ka[kb], Vl[g][kb], Sv, 0, 0, 0);
                    }
                    const float es[4] = {E[0] * Sv[0], E[1] * Sv[1], E[2] * Sv[2], E[3] * Sv[3]};
                    i16x4 hi, lo;
                    split2(E, hi, lo);
#pragma unroll
                    for (int q = 0; q < NB; ++q) {
                        O[g][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, Bt[q], O[g][q], 0, 0, 0);
                        O[g][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, Bt[q], O[g][q], 0, 0, 0);
                    }
                    split2(es, hi, lo);
#pragma unroll
                    for (int q = 0; q < NB; ++q) {
                        Q[g][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, Bt[q], Q[g][q], 0, 0, 0);
                        Q[g][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, Bt[q], Q[g][q], 0, 0, 0);
                    }
                } else if constexpr (MODE == kRowsMass) {
                    acc[g] += (E[0] + E[1]) + (E[2] + E[3]);
                    i16x4 hi, lo;
                    split2(E, hi, lo);
#pragma unroll
                    for (int q = 0; q < NB; ++q) {
                        O[g][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, Bt[q], O[g][q], 0, 0, 0);
                        O[g][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, Bt[q], O[g][q], 0, 0, 0);
                    }
                } else {
                    const float eu[4] = {E[0] * uu.x, E[1] * uu.y, E[2] * uu.z, E[3] * uu.w};
                    acc[g] += (eu[0] + eu[1]) + (eu[2] + eu[3]);
                    i16x4 hi, lo;
                    split2(eu, hi, lo);
#pragma unroll
                    for (int q = 0; q < NB; ++q) {
                        O[g][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, Bt[q], O[g][q], 0, 0, 0);
                        O[g][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, Bt[q], O[g][q], 0, 0, 0);
                    }
                }
            }
        }
        if (st + 1 < n_st)
            stash(bf ^ 1);
        __syncthreads();
    }
    // a row's scalar is spread over the four lanes sharing l % 16
    const size_t base = ((size_t)split * B + b) * n_pad + row0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float s = acc[g] + __shfl_xor(acc[g], 16, kWave);
        s += __shfl_xor(s, 32, kWave);
        if (kq == 0)
            part_s[base + 16 * g + c16] = s;
        if constexpr (kVec) {
#pragma unroll
            for (int q = 0; q < NB; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const size_t o = (base + 16 * g + 4 * kq + r) * d + 16 * q + c16;
                    part_v[o] = O[g][q][r];
                    if constexpr (kQ)
                        part_q[o] = Q[g][q][r];
                }
        }
    }
}

}  // namespace mc
}  // namespace sk

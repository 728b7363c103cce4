// lse_d3.hip -- fused streaming half-iteration for 3-D point clouds (fp32 or bf16
// coordinates, computed in fp32).
//
// One launch computes, for every row i of the "query" side and every pair b,
//     f_i = -eps * LSE_j[(g_j - ||x_i - y_j||^2)/eps + log w_j]
// as the stabilised log-domain update in its biased dot-product form
// (FlashSinkhorn summary, Methodologie 1, Propositie 1: Q = sqrt2 X, K = sqrt2 Y,
// the row-broadcast bias is the opposite hat potential g - ||y||^2 plus
// eps log w; the row's own ||x_i||^2 leaves the LSE and is added back).  With
// rows = X this is the f-update, with rows = Y the g-update (the same kernel,
// roles swapped).  The score matrix only exists tile by tile in registers
// (Methodologie 2: no n x m matrix in memory, online max / sum-exp on chip,
// one fused pass per update, query rows held stationary).
//
// Work is done in base 2: with c = log2(e)/eps,
//     s_ij = (2c x_i) . y_j + beta_j,   beta_j = c (g_j - ||y_j||^2) + log2 w_j,
//     f_i  = ||x_i||^2 - (eps ln2) * log2 sum_j 2^(s_ij)
// Two kernels compute it.  The default one (lse3m_kernel, below) forms s on
// the matrix cores from exact bf16 splits of the fp32 operands and streams each
// row against a fixed shift; the vector one (lse3_kernel, behind
// SK_VALU_SCORES) forms s with fp32 FMAs from packed keys (x, y, z, beta) read
// with wave-uniform addresses, one query row per lane, and keeps a lazy online
// maximum.  Both give the exact LSE up to fp32 rounding.
//
// The state carried between passes is the true potential (f, g), not the hat
// potential f - ||x||^2: when the clouds are far from the origin compared with
// the size of the potentials, an fp32 hat potential would lose an ulp of
// ||x||^2 on every pass.  Each row's result and the bias it hands to the
// other pass are formed in fp64 (a few operations per row) and rounded once.
//
// Online log-sum-exp with a lazy maximum: each state keeps (M, S) meaning
// S * 2^M.  Scores are formed relative to M; only when a tile holds a value
// more than kLazy above M is the tile re-evaluated against the new maximum
// and S rescaled.  The result is the exact LSE up to fp32 rounding, because
// LSE(z) = M + log2 sum 2^(z - M) for any M and no term exceeds 2^kLazy.
//
// A work-group holds W waves on the same 64 rows, each streaming every W-th key
// tile; their states merge at the end.  When a batch has too few rows to fill
// the chip the key range is also split across work-groups and a second small
// kernel merges the partial states; on the matrix-core path a third launch
// recomputes, with exact shifts, the row blocks whose merged sums left the
// range (it returns at once for every other block).
//
// Two stage kernels run every iteration of an eps stage in one launch, for
// batches where a launch per half-iteration would cost more than its work:
// lse3p_kernel (one work-group per pair, for batches of at least one pair per
// compute unit) and lse3s_kernel (a small batch of clouds of at most 1024
// points, each pair spread over work-groups of 16 rows that hand their new
// biases to one another between half-iterations).
#include "common.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace sk {
namespace {

constexpr int kTile = 16;      // keys per tile (64 SGPRs)
constexpr int kWaves = 8;      // waves per work-group, sharing rows
constexpr float kLazy = 32.0f; // terms may reach 2^kLazy before a rescale

__device__ __forceinline__ float score(float qx, float qy, float qz, float4 k, float base)
{
    return fmaf(qz, k.z, fmaf(qy, k.y, fmaf(qx, k.x, base)));
}

__device__ __forceinline__ float sq3(float x0, float x1, float x2)
{
    return fmaf(x2, x2, fmaf(x1, x1, x0 * x0));
}

// bias handed to the other pass: c (pot - ||x||^2) + log2 w, rounded once
__device__ __forceinline__ float bias_of(double c, float pot, float sq, float l2w)
{
    return (float)fma(c, (double)pot - (double)sq, (double)l2w);
}

// ---- bf16 records for the matrix-core path --------------------------------
// An fp32 value is the exact sum of three bf16 pieces (8 + 8 + 8 significant
// bits, fp32's exponent range): v = v0 + v1 + v2.  Products of two bf16 pieces
// are exact in the MFMA's fp32 accumulator, so
//     q . y = sum_u sum_(a,b) q_u,a y_u,b     over (a,b) in kPairs
// reproduces the fp32 dot product up to the accumulator's fp32 rounding and
// the dropped products of pieces (a, b) with a + b > 2.  With round-to-nearest
// pieces |v1| <= 2^-8 |v| and |v2| <= 2^-16 |v|, so (1, 2) and (2, 1) are each
// at most 2^-24 |q_u y_u| and (2, 2) 2^-32 |q_u y_u|: a score error of at most
// about 2^-23 sum_u |q_u y_u|, the size of one fp32 rounding of the products
// (the vector path's fp32 FMAs round at 2^-24 per operation).  Record slots (one 16x16x32 MFMA
// k-range): 6u + p holds piece kPairs[p] of coordinate u (query: q's piece a,
// key: y's piece b); slots 20..22 hold the bias pieces (key) or 1 (query);
// the rest are zero.
__device__ __forceinline__ uint32_t bf16_bits(float v)   // round to nearest even
{
    const uint32_t u = __float_as_uint(v);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_value(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ void split3(float v, uint32_t (&h)[3])
{
    h[0] = bf16_bits(v);
    const float r1 = v - bf16_value(h[0]);
    h[1] = bf16_bits(r1);
    const float r2 = r1 - bf16_value(h[1]);
    h[2] = bf16_bits(r2);
}

constexpr int kPairA[6] = {0, 0, 1, 0, 1, 2};   // query piece of pair p
constexpr int kPairB[6] = {0, 1, 0, 2, 1, 0};   // key piece of pair p
constexpr int kBiasSlot = 20;
constexpr uint32_t kBf16One = 0x3F80u;

__device__ __forceinline__ void store_record(uint16_t *rec, const uint32_t (&slot)[kRec])
{
    uint4 *dst = reinterpret_cast<uint4 *>(rec);
#pragma unroll
    for (int c = 0; c < 4; ++c)
        dst[c] = make_uint4(slot[8 * c] | slot[8 * c + 1] << 16, slot[8 * c + 2] | slot[8 * c + 3] << 16,
                            slot[8 * c + 4] | slot[8 * c + 5] << 16, slot[8 * c + 6] | slot[8 * c + 7] << 16);
}

// bias pieces of a key record: one 8-byte store of slots 20..23
__device__ __forceinline__ void store_key_bias(uint16_t *rec, float beta)
{
    uint32_t h[3];
    split3(beta, h);
    *reinterpret_cast<uint2 *>(rec + kBiasSlot) = make_uint2(h[0] | h[1] << 16, h[2]);
}

__device__ __forceinline__ void store_key_record(uint16_t *rec, float x0, float x1, float x2,
                                                 float beta)
{
    uint32_t h[3][3], slot[kRec];
    split3(x0, h[0]);
    split3(x1, h[1]);
    split3(x2, h[2]);
#pragma unroll
    for (int k = 0; k < kRec; ++k)
        slot[k] = 0;
#pragma unroll
    for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int p = 0; p < 6; ++p)
            slot[6 * u + p] = h[u][kPairB[p]];
    uint32_t hb[3];
    split3(beta, hb);
    slot[kBiasSlot] = hb[0];
    slot[kBiasSlot + 1] = hb[1];
    slot[kBiasSlot + 2] = hb[2];
    store_record(rec, slot);
}

__device__ __forceinline__ void store_query_record(uint16_t *rec, float q0, float q1, float q2)
{
    uint32_t h[3][3], slot[kRec];
    split3(q0, h[0]);
    split3(q1, h[1]);
    split3(q2, h[2]);
#pragma unroll
    for (int k = 0; k < kRec; ++k)
        slot[k] = 0;
#pragma unroll
    for (int u = 0; u < 3; ++u)
#pragma unroll
        for (int p = 0; p < 6; ++p)
            slot[6 * u + p] = h[u][kPairA[p]];
    slot[kBiasSlot] = slot[kBiasSlot + 1] = slot[kBiasSlot + 2] = kBf16One;
    store_record(rec, slot);
}

// Center of each pair: midpoint of the bounding box of both clouds.  The
// squared-Euclidean cost is unchanged by a common translation, so the packed
// points are stored relative to it; this keeps ||x||^2 and 2 x . y, whose fp32
// rounding the expanded score carries, as small as the clouds allow.
constexpr int kCenterChunk = 8192;   // points per work-group of the partial boxes

__device__ __forceinline__ void box_reduce(float (&mn)[3], float (&mx)[3])
{
    __shared__ float lo[3][256], hi[3][256];
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        lo[k][t] = mn[k];
        hi[k][t] = mx[k];
    }
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (t < s)
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                lo[k][t] = fminf(lo[k][t], lo[k][t + s]);
                hi[k][t] = fmaxf(hi[k][t], hi[k][t + s]);
            }
        __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        mn[k] = lo[k][0];
        mx[k] = hi[k][0];
    }
}

// Partial bounding boxes: work-group (c, b) covers points c*kCenterChunk ...
// of the concatenation X_b, Y_b.  part[2 (b parts + c)] = (min, max).
template <typename T>
__global__ __launch_bounds__(256) void center3_parts_kernel(const T *__restrict__ X, int n,
                                                            const T *__restrict__ Y, int m,
                                                            float4 *__restrict__ part)
{
    const int b = blockIdx.y, c = blockIdx.x;
    float mn[3] = {INFINITY, INFINITY, INFINITY}, mx[3] = {-INFINITY, -INFINITY, -INFINITY};
    const int end = min(n + m, (c + 1) * kCenterChunk);
    for (int i = c * kCenterChunk + threadIdx.x; i < end; i += 256) {
        const T *p = i < n ? X + ((size_t)b * n + i) * 3 : Y + ((size_t)b * m + i - n) * 3;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const float v = Elem<T>::get(p, k);
            mn[k] = fminf(mn[k], v);
            mx[k] = fmaxf(mx[k], v);
        }
    }
    box_reduce(mn, mx);
    if (threadIdx.x == 0) {
        const size_t o = 2 * ((size_t)b * gridDim.x + c);
        part[o] = make_float4(mn[0], mn[1], mn[2], 0.f);
        part[o + 1] = make_float4(mx[0], mx[1], mx[2], 0.f);
    }
}

// Merge of the partial boxes of each pair into its center.
__global__ __launch_bounds__(256) void center3_kernel(const float4 *__restrict__ part, int parts,
                                                     float4 *__restrict__ center)
{
    const int b = blockIdx.x;
    float mn[3] = {INFINITY, INFINITY, INFINITY}, mx[3] = {-INFINITY, -INFINITY, -INFINITY};
    for (int c = threadIdx.x; c < parts; c += 256) {
        const float4 lo = part[2 * ((size_t)b * parts + c)];
        const float4 hi = part[2 * ((size_t)b * parts + c) + 1];
        mn[0] = fminf(mn[0], lo.x); mn[1] = fminf(mn[1], lo.y); mn[2] = fminf(mn[2], lo.z);
        mx[0] = fmaxf(mx[0], hi.x); mx[1] = fmaxf(mx[1], hi.y); mx[2] = fmaxf(mx[2], hi.z);
    }
    box_reduce(mn, mx);
    if (threadIdx.x == 0) {
        float c[3];
#pragma unroll
        for (int k = 0; k < 3; ++k)
            c[k] = isfinite(mn[k]) && isfinite(mx[k]) ? 0.5f * (mn[k] + mx[k]) : 0.f;
        center[b] = make_float4(c[0], c[1], c[2], 0.f);
    }
}

template <typename T>
__global__ void pack3_kernel(const T *__restrict__ X, const float *__restrict__ w, int warm,
                             int n, int n_pad, const float4 *__restrict__ center,
                             float4 *__restrict__ pts, float *__restrict__ pot,
                             float *__restrict__ l2w, uint16_t *__restrict__ krec, double c0)
{
    const int b = blockIdx.y;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_pad)
        return;
    float4 out = make_float4(0.f, 0.f, 0.f, kNeg);
    if (i < n) {
        const T *x = X + ((size_t)b * n + i) * 3;
        const float4 o = center[b];
        const float x0 = Elem<T>::get(x, 0) - o.x, x1 = Elem<T>::get(x, 1) - o.y,
                    x2 = Elem<T>::get(x, 2) - o.z;
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
        out = make_float4(x0, x1, x2, lw == kNeg ? kNeg : bias_of(c0, pot[k], sq3(x0, x1, x2), lw));
    }
    pts[(size_t)b * n_pad + i] = out;
    store_key_record(krec + ((size_t)b * n_pad + i) * kRec, out.x, out.y, out.z, out.w);
}

// Query records at the scale c of the current eps: q = 2c (x, y, z).
// With xch set, the side's (tag, bias) words of the split stage launch are
// zeroed as well.
__global__ void qrec3_kernel(const float4 *__restrict__ pts, int n_pad, float two_c,
                             uint16_t *__restrict__ qrec, uint64_t *__restrict__ xch)
{
    const int b = blockIdx.y;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_pad)
        return;
    const size_t k = (size_t)b * n_pad + i;
    const float4 p = pts[k];
    store_query_record(qrec + k * kRec, two_c * p.x, two_c * p.y, two_c * p.z);
    if (xch)
        xch[k] = 0;
}

// Row result: true potential from the (M, S) state, and the bias of this row
// for the other pass (lw: the row's log2 weight), which is returned.
__device__ __forceinline__ float finish_row(float4 *qpts, uint16_t *qkrec, float *qpot, float lw,
                                            size_t pt, size_t k, float4 p, float M, float S,
                                            double eps_ln2, double c_next)
{
    const float sq = sq3(p.x, p.y, p.z);
    const double lse2 = (double)M + (double)lg2(S);
    const float f = (float)((double)sq - lse2 * eps_ln2);
    qpot[k] = f;
    const float beta = lw == kNeg ? kNeg : bias_of(c_next, f, sq, lw);
    qpts[pt].w = beta;
    store_key_bias(qkrec + pt * kRec, beta);
    return beta;
}

// part == nullptr: single split, finalise in place.
__global__ __launch_bounds__(kWaves *kWave) void lse3_kernel(
    float4 *__restrict__ qpts, uint16_t *__restrict__ qkrec, const float4 *__restrict__ kpts,
    float *__restrict__ qpot, const float *__restrict__ ql2w, float2 *__restrict__ part, int nq,
    int nq_pad, int nk_pad, int tiles_per_split, float two_c, double eps_ln2, double c_next)
{
    __shared__ float2 red[kWaves][kWave];
    const int b = blockIdx.z;
    const int split = blockIdx.y;
    const int lane = lane_id();
    const int w = wave_id_uniform();
    const int row = blockIdx.x * kWave + lane;

    const float4 p = qpts[(size_t)b * nq_pad + row];
    const float qx = two_c * p.x, qy = two_c * p.y, qz = two_c * p.z;
    const float4 *kp = kpts + (size_t)b * nk_pad;
    const int n_tiles = nk_pad / kTile;
    const int t_begin = split * tiles_per_split;
    const int t_end = min(t_begin + tiles_per_split, n_tiles);

    float M = kNeg, S0 = 0.f, S1 = 0.f;
    for (int t = t_begin + w; t < t_end; t += kWaves) {
        const float4 *kt = kp + (size_t)t * kTile;
        float4 kk[kTile];
#pragma unroll
        for (int u = 0; u < kTile; ++u)
            kk[u] = kt[u];
        float r[kTile];
#pragma unroll
        for (int u = 0; u < kTile; ++u)
            r[u] = score(qx, qy, qz, kk[u], kk[u].w - M);
        float cm = r[0];
#pragma unroll
        for (int u = 1; u < kTile; ++u)
            cm = fmaxf(cm, r[u]);
        if (cm > kLazy) {
            // re-evaluate the tile against its own maximum, then rescale
            float Mn = M;
#pragma unroll
            for (int u = 0; u < kTile; ++u) {
                r[u] = score(qx, qy, qz, kk[u], kk[u].w);
                Mn = fmaxf(Mn, r[u]);
            }
            const float scale = ex2(M - Mn);
            S0 *= scale;
            S1 *= scale;
#pragma unroll
            for (int u = 0; u < kTile; ++u)
                r[u] -= Mn;
            M = Mn;
        }
#pragma unroll
        for (int u = 0; u < kTile; u += 2) {
            S0 += ex2(r[u]);
            S1 += ex2(r[u + 1]);
        }
    }
    float S = S0 + S1;

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
        finish_row(qpts, qkrec, qpot, ql2w[(size_t)b * nq + row], (size_t)b * nq_pad + row,
                   (size_t)b * nq + row, p, M, S, eps_ln2, c_next);
}

// ---------------------------------------------------------------------------
// Matrix-core variant.  Score and bias are one contraction over the 32-slot
// records: s_ij - M = qrec_i . krec_j + (-M), the bf16 pieces of 2c x_i against
// those of y_j plus 1 against the pieces of beta_j.  One
// v_mfma_f32_16x16x32_bf16 per 16 x 16 block produces s - M, with -M riding in
// the accumulator input; the vector ALUs are left with the exponential and the
// accumulation.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (wave64): lane l supplies
// A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16] for e = 0..7 and
// receives D[4 (l / 16) + r][l % 16] in register r.  A wave covers 64 query
// rows as 4 groups of 16; per key tile of 16 columns it issues 4 MFMAs.  Each
// (lane, group, register) keeps its own (M, S) over the columns l % 16 + 16 t;
// the 16 lanes of a row merge at the end with DPP moves, then the W waves of
// the work-group (each streaming every W-th tile) merge through LDS.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kGroups = 4;        // 16-row groups per wave
constexpr unsigned kXcds = 8;     // XCDs (each with its own L2) the dispatcher deals to in turn

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t *p)
{
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

// D = A B + C over one 32-slot record range: the augmented score from the
// bf16 pieces (exact products, fp32 accumulation)
__device__ __forceinline__ f32x4 mfma4(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Shifted pass: every row streams against a fixed shift, the log-sum-exp of
// its previous pass, M_i = c (||x_i||^2 - f_i).  Between passes potentials
// move little, so 2^(s - M) stays in range and the loop is exponential plus
// accumulation only.  The merged sum of each row is checked at the end: if any
// row of a 64-row block left [2^-64, 2^100] (the shift was stale, e.g. on the
// first pass or after a large change of eps), the block's shifts are made
// exact: a pass over the same keys takes every row's maximum of s - M, M moves
// up by it, and the shifted pass runs again, now with terms of at most 1 and a
// sum in [1, keys].  Either way the result is the exact log-sum-exp to fp32
// rounding.
constexpr float kSumLo = 5.421010862e-20f;  // 2^-64
constexpr float kSumHi = 1.2676506e30f;     // 2^100

// LDS copy of a side's key records (per-pair launch, clouds of at most
// kLdsMaxPoints points): record r's four 16-byte chunks at 16-byte index 4 r
// + (c ^ ((r >> 1) & 3)).  A tile read has lane (kq, c16) take chunk kq of
// record 16 t + c16; the XOR spreads the 8 lanes that share kq over all banks
// (record stride 64 bytes alone would map pairs of them onto the same banks).
constexpr int kLdsMaxPoints = 1024;
__device__ __forceinline__ int lds_chunk(int r, int c) { return 4 * r + (c ^ ((r >> 1) & 3)); }

// Bias pieces of record r in the LDS copy (slots 20..23 = chunk 2, bytes 8..15).
__device__ __forceinline__ void store_key_bias_lds(uint4 *lds, int r, float beta)
{
    uint32_t h[3];
    split3(beta, h);
    reinterpret_cast<uint2 *>(&lds[lds_chunk(r, 2)])[1] = make_uint2(h[0] | h[1] << 16, h[2]);
}

// Stream of one wave: key tiles first, first + W, ... (cnt of them) against the
// wave's 64 rows with the shift in Cn, accumulated into S as a sum of 2^(s - M)
// (the shifted pass) or as the maximum of s - M (kMax, the pass that makes a
// stale shift exact; the same tiles, operands and MFMAs, so the maximum is
// taken over exactly the values the following shifted pass exponentiates).  The
// first cnt % 3 tiles go one by one, the rest in groups of three with no
// branch inside a group, so every key operand is loaded two tiles ahead of its
// use (the scheduling barriers keep each load in place; indices are clamped to
// the wave's last tile so that loads past the end stay inside the pair).  Three
// register sets take turns, so no operand is copied.  Key operands come through
// a buffer resource: the tile offset rides in an SGPR (soffset), the lane's
// offset is a constant VGPR, so there is no vector address arithmetic per tile.
// With kLds the key records come from a copy in LDS instead (lds: the pair's
// records in the layout of lds_chunk), the same operands in the same order.
template <int W, bool kMax, int G = kGroups, bool kLds = false>
__device__ __forceinline__ void key_stream(const bf16x8 (&A)[G], const f32x4 (&Cn)[G],
                                           f32x4 (&S)[G], const uint16_t *kb, int nk_pad,
                                           int lane_off, int first, int cnt,
                                           const uint4 *lds = nullptr)
{
    const int last = first + (cnt > 0 ? cnt - 1 : 0) * W;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)kb, (short)0, nk_pad * kRec * (int)sizeof(uint16_t), 0x00020000);
    const int voff = lane_off * (int)sizeof(uint16_t);
    // the lane's chunk of record t kTile + (l & 15) sits at 4 kTile t + lane_lds:
    // the swizzle (r >> 1) & 3 of lds_chunk depends on the low bits of r only
    static_assert(kTile % 8 == 0, "tile starts keep the swizzle");
    const int lane_rec = lane_id() & 15, lane_chunk = lane_id() >> 4;
    const int lane_lds = lds_chunk(lane_rec, lane_chunk);
    auto key = [&](int k) {
        const int t = min(first + k * W, last);
        if constexpr (kLds)
            return __builtin_bit_cast(bf16x8, lds[4 * kTile * t + lane_lds]);
        else
            return __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                            krs, voff, t * (kTile * kRec * (int)sizeof(uint16_t)), 0));
    };
    // With W > 1 the four MFMAs of a tile are issued together ahead of its
    // exponentials (one wait on the first result instead of one per group;
    // gmm-64k 1.3% faster).  The per-pair launch (W = 1) keeps the interleaved
    // order: at its 128-register limit the grouped one spills.
    auto tile = [&](const bf16x8 &Bt) {
        f32x4 D[G];
#pragma unroll
        for (int g = 0; g < G; ++g)
            D[g] = mfma4(A[g], Bt, Cn[g]);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[g][r] = kMax ? fmaxf(S[g][r], D[g][r]) : S[g][r] + ex2(D[g][r]);
        if constexpr (W > 1) {
            __builtin_amdgcn_sched_group_barrier(0x008, G, 0);       // the MFMAs
            __builtin_amdgcn_sched_group_barrier(0x002, 8 * G, 0);   // then the vector work
        }
    };
    // From LDS, the tiles of the groups whose loads all stay below cnt are read
    // unclamped (the index affine in k: one address add per group of three, the
    // rest immediate offsets), the last group with the clamp.
    auto key_in = [&](int k) {
        return __builtin_bit_cast(bf16x8, lds[4 * kTile * (first + k * W) + lane_lds]);
    };
    int k = 0;
    for (; k < cnt % 3; ++k)
        tile(key(k));
    if (k < cnt) {
        bf16x8 Ra = key(k), Rb = key(k + 1), Rc;
        if constexpr (kLds) {
            for (; k + 4 < cnt; k += 3) {
                Rc = key_in(k + 2);
                __builtin_amdgcn_sched_barrier(0);
                tile(Ra);
                __builtin_amdgcn_sched_barrier(0);
                Ra = key_in(k + 3);
                __builtin_amdgcn_sched_barrier(0);
                tile(Rb);
                __builtin_amdgcn_sched_barrier(0);
                Rb = key_in(k + 4);
                __builtin_amdgcn_sched_barrier(0);
                tile(Rc);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        for (; k < cnt; k += 3) {
            Rc = key(k + 2);
            __builtin_amdgcn_sched_barrier(0);
            tile(Ra);
            __builtin_amdgcn_sched_barrier(0);
            Ra = key(k + 3);
            __builtin_amdgcn_sched_barrier(0);
            tile(Rb);
            __builtin_amdgcn_sched_barrier(0);
            Rb = key(k + 4);
            __builtin_amdgcn_sched_barrier(0);
            tile(Rc);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Lazy-maximum stream of one wave: key tiles t0, t0 + W, ... below t_end into
// the (M, S) states, M carried as -Cn (+1e30 marks a state that has seen no key
// yet).  The key operand of the next tile is loaded one tile ahead; the clamped
// index keeps that load inside the pair's keys on the last tile.
template <int W, int G = kGroups, bool kLds = false>
__device__ __forceinline__ void shifted_stream(const bf16x8 (&A)[G], const f32x4 (&Cn)[G],
                                               f32x4 (&S)[G], const uint16_t *kb, int nk_pad,
                                               int lane_off, int first, int cnt,
                                               const uint4 *lds = nullptr)
{
    key_stream<W, false, G, kLds>(A, Cn, S, kb, nk_pad, lane_off, first, cnt, lds);
}

// Query operands of a wave's 16 G rows.
template <int G = kGroups>
__device__ __forceinline__ void load_rows(bf16x8 (&A)[G], const uint16_t *qrec_rows, int lane_off)
{
#pragma unroll
    for (int g = 0; g < G; ++g)
        A[g] = load_bf16x8(qrec_rows + (size_t)(16 * g) * kRec + lane_off);
}

// Their shifts M_i = c (||x_i||^2 - f_i), carried as -M in the accumulator
// input, and empty sums.  Each lane loads one row's point and potential and
// forms its shift; the wave hands the shifts through shv (64 floats of LDS,
// 16-byte aligned, the wave's own) to the lanes whose results hold the row:
// two loads a lane instead of one per (row group, result register).
template <int G = kGroups>
__device__ __forceinline__ void load_shifts(f32x4 (&Cn)[G], f32x4 (&S)[G], const float4 *qrow,
                                            const float *qpot_b, int nq, int row0, int kq, float c,
                                            float *shv)
{
    const int lane = lane_id();
    if (lane < 16 * G) {
        const float4 p = qrow[lane];
        const float f = row0 + lane < nq ? qpot_b[row0 + lane] : 0.f;
        shv[lane] = -(c * (sq3(p.x, p.y, p.z) - f));
    }
    __builtin_amdgcn_wave_barrier();   // a wave's LDS accesses complete in order
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float4 v = *reinterpret_cast<const float4 *>(shv + 16 * g + 4 * kq);
        Cn[g] = f32x4{v.x, v.y, v.z, v.w};
        S[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __builtin_amdgcn_wave_barrier();   // shv is written again later
}

__device__ __forceinline__ float row16_max(float v)
{
    v = fmaxf(v, dpp_move<kDppXor1>(v));
    v = fmaxf(v, dpp_move<kDppXor2>(v));
    v = fmaxf(v, dpp_move<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_move<kDppMirror>(v));
    return v;
}

// Row sums of one wave's states, with the row's shift, into red_w[row].  The
// 16 lanes of a DPP row hold the same rows (16 G of them) for different key
// columns.  With G = 4 the sums are a reduce-scatter over those 16 lanes: four
// pairings (lanes i and 15 - i, then i and 7 - i within each half row, then
// i ^ 1, then i ^ 2) each halve the values a lane carries, the lane keeping
// the half its bit of the pairing selects and adding the partner's copy of it,
// so that every lane ends with one row's sum (and selects that row's shift)
// and writes it: 45 selects and 15 adds instead of 64 adds, 16 negations and
// 16 masked stores.  It pays where a wave's rows are short (sphere-2k's 32
// tiles per wave: 3% off the half-iteration); with 8 waves on long rows
// (gmm-64k) the sum is a rounding error of the launch and that kernel keeps
// the all-lane sums (kScatter false), which measured 0.9% faster there.  With
// G = 1 every lane sums all 16 lanes of each row.
template <int G = kGroups, bool kScatter = true>
__device__ __forceinline__ void wave_sums(const f32x4 (&Cn)[G], const f32x4 (&S)[G],
                                          float2 *red_w, int kq, int c16)
{
    if constexpr (G == 4 && kScatter) {
        float x[16], m[16];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[4 * g + r] = S[g][r];
                m[4 * g + r] = -Cn[g][r];
            }
        const bool b3 = c16 & 8, b2 = c16 & 4, b1 = c16 & 2, b0 = c16 & 1;
        auto step = [&](auto ctrl, int half, bool hi) {
            constexpr int kCtrl = decltype(ctrl)::value;
#pragma unroll
            for (int v = 0; v < half; ++v) {
                const float keep = hi ? x[v + half] : x[v];
                const float send = hi ? x[v] : x[v + half];
                x[v] = keep + dpp_move<kCtrl>(send);
                m[v] = hi ? m[v + half] : m[v];
            }
        };
        step(std::integral_constant<int, kDppMirror>{}, 8, b3);
        step(std::integral_constant<int, kDppHalfMirror>{}, 4, b2);
        step(std::integral_constant<int, kDppXor1>{}, 2, b0);
        step(std::integral_constant<int, kDppXor2>{}, 1, b1);
        const int v = 8 * b3 + 4 * b2 + 2 * b0 + b1;   // the row value this lane holds
        red_w[16 * (v >> 2) + 4 * kq + (v & 3)] = make_float2(m[0], x[0]);
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float Sr = row16_sum(S[g][r]);
                if (c16 == 0)
                    red_w[16 * g + 4 * kq + r] = make_float2(-Cn[g][r], Sr);
            }
    }
}

// Makes the shifts of a 64-row block exact: the maximum of s - M over the
// block's keys (each wave its tiles, merged over the W waves through red) is
// added to every row's M, and S is emptied for the shifted pass that follows.
// With W > 1 every wave of the work-group must call it.
template <int W, int G = kGroups, bool kLds = false>
__device__ __forceinline__ void exact_shifts(const bf16x8 (&A)[G], f32x4 (&Cn)[G], f32x4 (&S)[G],
                                             const uint16_t *kb, int nk_pad, int lane_off,
                                             int first, int cnt, float2 (*red)[kWave], int w,
                                             int kq, int c16, const uint4 *lds = nullptr)
{
#pragma unroll
    for (int g = 0; g < G; ++g)
        S[g] = f32x4{kNeg, kNeg, kNeg, kNeg};
    key_stream<W, true, G, kLds>(A, Cn, S, kb, nk_pad, lane_off, first, cnt, lds);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[g][r] = row16_max(S[g][r]);
    if constexpr (W > 1) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (c16 == 0)
                    red[w][16 * g + 4 * kq + r].x = S[g][r];
        __syncthreads();
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int lr = 16 * g + 4 * kq + r;
                float mx = red[0][lr].x;
#pragma unroll
                for (int v = 1; v < W; ++v)
                    mx = fmaxf(mx, red[v][lr].x);
                S[g][r] = mx;
            }
        __syncthreads();   // red is written again by the caller
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            Cn[g][r] -= S[g][r];
            S[g][r] = 0.f;
        }
}

// One work-group: 16 G query rows of pair b (G = 4: one 64-row block; G = 1:
// 16 rows, for launches with too few 64-row blocks to spread over the chip),
// W waves, key tiles of split blockIdx.y.  Three uses (the last two with
// G = 4 only):
//   part == nullptr, redo == nullptr: all keys; shifted pass, made exact where
//     a row left the range; finishes the rows.
//   part != nullptr: the split's keys with the rows' shifts; writes the partial
//     (M, S) of every row (no range check: the merge checks the whole row).
//   redo != nullptr (repair, after the merge of split partials): only blocks
//     marked in redo; exact shifts over all keys, then the shifted pass.
template <int W, int G>
__global__ __launch_bounds__(W *kWave) void lse3m_kernel(
    float4 *__restrict__ qpts, uint16_t *__restrict__ qkrec, const uint16_t *__restrict__ qrec,
    const uint16_t *__restrict__ krec, float *__restrict__ qpot, const float *__restrict__ ql2w,
    float2 *__restrict__ part, const int *__restrict__ redo, int nq, int nq_pad, int nk_pad,
    int tiles_per_split, float two_c, double eps_ln2, double c_next)
{
    __shared__ __align__(16) float2 red[W][kWave];
    __shared__ int stale;
    // XCD-aware placement for batches: the dispatcher deals work-groups to the
    // XCDs in turn, so the linear id is remapped to give each XCD a contiguous
    // run of (row block, split, pair) and keep a pair's key records in one L2
    // (one pair: every XCD needs its keys anyway, and the launch stays as is)
    int bx = blockIdx.x, split = blockIdx.y, b = blockIdx.z;
    {
        const unsigned gx = gridDim.x, gy = gridDim.y;
        const unsigned total = gx * gy * gridDim.z;   // B n_pad / 64 * splits < 2^31
        if (gridDim.z > 1 && total % kXcds == 0) {
            unsigned L = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
            L = (L % kXcds) * (total / kXcds) + L / kXcds;
            bx = (int)(L % gx);
            L /= gx;
            split = (int)(L % gy);
            b = (int)(L / gy);
        }
    }
    if (redo && !redo[(size_t)b * (nq_pad / kWave) + bx])
        return;   // the whole work-group: this block was finished by the merge
    static_assert(G == kGroups || G == 1, "a work-group holds 64 or 16 rows");
    constexpr int R = 16 * G;      // rows of the work-group
    const int lane = lane_id();
    const int w = wave_id_uniform();
    const int row0 = bx * R;
    const int kq = lane >> 4;      // operand k index this lane supplies / row quad it receives
    const int c16 = lane & 15;     // operand row (A) or column (B) within a 16-block

    const float4 *qrow = qpts + (size_t)b * nq_pad + row0;
    const int lane_off = c16 * kRec + 8 * kq;   // this lane's 8 slots of a record
    const uint16_t *qrec_rows = qrec + ((size_t)b * nq_pad + row0) * kRec;
    const uint16_t *kb = krec + (size_t)b * nk_pad * kRec;
    const int n_tiles = nk_pad / kTile;
    const int t_begin = split * tiles_per_split;
    const int t_end = min(t_begin + tiles_per_split, n_tiles);
    const int first = t_begin + w;   // this wave takes tiles first + k W
    const int cnt = first < t_end ? (t_end - first + W - 1) / W : 0;
    bf16x8 A[G];
    f32x4 Cn[G], S[G];
    load_rows<G>(A, qrec_rows, lane_off);
    load_shifts<G>(Cn, S, qrow, qpot + (size_t)b * nq, nq, row0, kq, 0.5f * two_c,
                   reinterpret_cast<float *>(red[w]));
    const int row = row0 + lane;
    const bool mine = lane < R && row < nq;   // lane of wave 0 that finishes a row
    // the finishing lanes fetch their row's point and log2 weight now, off the
    // path that follows the merge
    float4 prow = make_float4(0.f, 0.f, 0.f, 0.f);
    float lw = 0.f;
    if (w == 0 && mine) {
        prow = qpts[(size_t)b * nq_pad + row];
        lw = ql2w[(size_t)b * nq + row];
    }

    if (redo == nullptr) {
        shifted_stream<W, G>(A, Cn, S, kb, nk_pad, lane_off, first, cnt);
        // every partial of a row has the same shift: the merge is a sum
        wave_sums<G, (W < 8)>(Cn, S, red[w], kq, c16);
        if (threadIdx.x == 0)
            stale = 0;
        __syncthreads();
        float Ssum = 0.f;
        const float M = red[0][lane].x;
        if (w == 0) {
#pragma unroll
            for (int v = 0; v < W; ++v)
                Ssum += red[v][lane].y;
            if (part)
                part[((size_t)split * gridDim.z + b) * nq_pad + row] = make_float2(M, Ssum);
            else if (mine && !(Ssum >= kSumLo && Ssum <= kSumHi))
                stale = 1;   // benign race: every writer stores 1 (padding rows never do)
        }
        if (part)
            return;
        __syncthreads();
        if (!stale) {
            if (w == 0 && mine)
                finish_row(qpts, qkrec, qpot, lw, (size_t)b * nq_pad + row, (size_t)b * nq + row,
                           prow, M, Ssum, eps_ln2, c_next);
            return;
        }
    }

    exact_shifts<W, G>(A, Cn, S, kb, nk_pad, lane_off, first, cnt, red, w, kq, c16);
    shifted_stream<W, G>(A, Cn, S, kb, nk_pad, lane_off, first, cnt);
    wave_sums<G, (W < 8)>(Cn, S, red[w], kq, c16);
    __syncthreads();
    if (w != 0 || !mine)
        return;
    float Ssum = 0.f;
#pragma unroll
    for (int v = 0; v < W; ++v)
        Ssum += red[v][lane].y;
    finish_row(qpts, qkrec, qpot, lw, (size_t)b * nq_pad + row, (size_t)b * nq + row, prow,
               red[0][lane].x, Ssum, eps_ln2, c_next);
}

// ---------------------------------------------------------------------------
// Persistent pass per pair, for batches of at least as many pairs as the chip
// has compute units: one work-group of kPairWaves waves owns one pair and runs
// every iteration of a stage in one launch.  Each wave takes whole 64-row
// blocks (all keys, the shifted stream, made exact and streamed again when a
// row's sum leaves the range), finishes its rows, and the
// work-group synchronises between the f- and the g-update.  Everything a pass
// reads from the other side was written by this work-group, so the barrier is
// the only synchronisation; the per-launch cost of the other path (a launch
// and the fill and drain of the chip for every half-iteration) is paid once
// per stage.  The arithmetic per row is that of lse3m_kernel<1, 4>.
constexpr int kPairWaves = 16;

// One wave: rows row0 .. row0 + 63 of pair b on side q against all keys of side k.
// With stale set (the first updates of a cold start, where the potentials
// are zeros and most pairs' shifts are far off) the shifts are made exact
// before the first shifted pass instead of after a failed one.  With kLds the
// keys' records are read from their LDS copy k_lds, and each finished row
// writes its new bias pieces to the LDS copy of its own side, q_lds, as well.
template <bool kLds>
__device__ __forceinline__ void wave_rows(const Side3 &q, const Side3 &k, int b, int row0,
                                          float two_c, double eps_ln2, double c_next,
                                          float2 *red, bool stale, const uint4 *k_lds,
                                          uint4 *q_lds, const float *q_sq, float *q_pot,
                                          const float *q_lw, bool last,
                                          const bf16x8 (&A)[kGroups],
                                          const uint16_t *next_rows, bf16x8 (&An)[kGroups])
{
    const int lane = lane_id();
    const int kq = lane >> 4, c16 = lane & 15;
    const int lane_off = c16 * kRec + 8 * kq;
    const float4 *qrow = q.pts + (size_t)b * q.n_pad + row0;
    const uint16_t *kb = k.krec + (size_t)b * k.n_pad * kRec;
    const int n_tiles = k.n_pad / kTile;
    f32x4 Cn[kGroups], S[kGroups];
    const int row = row0 + lane;
    float4 prow = make_float4(0.f, 0.f, 0.f, 0.f);
    float lw = 0.f;
    if constexpr (kLds) {
        // squared norms and potentials from the stage's LDS copy (the same values
        // the global arrays would give: written by this work-group)
        const float sh = -(0.5f * two_c * (q_sq[row] - q_pot[row]));
        float *shv = reinterpret_cast<float *>(red);
        shv[lane] = sh;
        __builtin_amdgcn_wave_barrier();   // a wave's LDS accesses complete in order
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            const float4 v = *reinterpret_cast<const float4 *>(shv + 16 * g + 4 * kq);
            Cn[g] = f32x4{v.x, v.y, v.z, v.w};
            S[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __builtin_amdgcn_wave_barrier();
        lw = q_lw[row];
    } else {
        load_shifts(Cn, S, qrow, q.pot + (size_t)b * q.n, q.n, row0, kq, 0.5f * two_c,
                    reinterpret_cast<float *>(red));
        // the row this lane finishes: its point and log2 weight, fetched now, off
        // the path that follows the stream
        if (row < q.n) {
            prow = qrow[lane];
            lw = q.l2w[(size_t)b * q.n + row];
        }
    }
    float M = 0.f, Sf = 0.f;
    if (!stale) {
        shifted_stream<1, kGroups, kLds>(A, Cn, S, kb, k.n_pad, lane_off, 0, n_tiles, k_lds);
        wave_sums(Cn, S, red, kq, c16);
        __builtin_amdgcn_wave_barrier();
        M = red[lane].x;
        Sf = red[lane].y;
        // the whole wave decides: it owns every row of the block
        stale = __ballot(row < q.n && !(Sf >= kSumLo && Sf <= kSumHi)) != 0;
        __builtin_amdgcn_wave_barrier();   // red is written again below
    }
    if (stale) {
        exact_shifts<1, kGroups, kLds>(A, Cn, S, kb, k.n_pad, lane_off, 0, n_tiles, nullptr, 0,
                                       kq, c16, k_lds);
        shifted_stream<1, kGroups, kLds>(A, Cn, S, kb, k.n_pad, lane_off, 0, n_tiles, k_lds);
        __builtin_amdgcn_wave_barrier();
        wave_sums(Cn, S, red, kq, c16);
        __builtin_amdgcn_wave_barrier();
        M = red[lane].x;
        Sf = red[lane].y;
    }
    // the next block's query operands (records fixed for the stage: no
    // dependency on this pass) load now, while the rows finish and the
    // work-group meets at the barrier
    if (next_rows)
        load_rows(An, next_rows, lane_off);
    if (row < q.n) {
        if constexpr (kLds) {
            // the arithmetic of finish_row, the state kept in LDS; the global
            // arrays are written by the stage's last iteration only
            const float sq = q_sq[row];
            const double lse2 = (double)M + (double)lg2(Sf);
            const float f = (float)((double)sq - lse2 * eps_ln2);
            q_pot[row] = f;
            const float beta = lw == kNeg ? kNeg : bias_of(c_next, f, sq, lw);
            store_key_bias_lds(q_lds, row, beta);
            if (last) {
                const size_t pt = (size_t)b * q.n_pad + row;
                q.pot[(size_t)b * q.n + row] = f;
                q.pts[pt].w = beta;
                store_key_bias(q.krec + pt * kRec, beta);
            }
        } else {
            finish_row(q.pts, q.krec, q.pot, lw, (size_t)b * q.n_pad + row, (size_t)b * q.n + row,
                       prow, M, Sf, eps_ln2, c_next);
        }
    }
    __builtin_amdgcn_wave_barrier();   // red is reused by the next block
}

// kLds (both clouds of at most kLdsMaxPoints points): the key records of both
// sides are copied into LDS once per launch (128 KB), and the passes read
// their keys from there; between passes only the bias pieces of the records
// change, and the rows that produce them write them to the copy as well.
template <bool kLds>
__global__ __launch_bounds__(kPairWaves *kWave) void lse3p_kernel(Side3 x, Side3 y, int iters,
                                                                  float two_c, double eps_ln2,
                                                                  double c_next_last, int cold)
{
    __shared__ __align__(16) float2 red[kPairWaves][kWave];
    __shared__ uint4 recs[2][kLds ? kLdsMaxPoints * kRec / 8 : 1];   // unused without kLds
    // with kLds also every point's squared norm, potential and log2 weight, both
    // sides (the stage's state)
    __shared__ float sqs[2][kLds ? kLdsMaxPoints : 1], pots[2][kLds ? kLdsMaxPoints : 1];
    __shared__ float lws[2][kLds ? kLdsMaxPoints : 1];   // log2 weights
    const int b = blockIdx.x;
    const int w = wave_id_uniform();
    const double c_same = 0.5 * (double)two_c;
    if constexpr (kLds) {
        const Side3 *side[2] = {&x, &y};
#pragma unroll
        for (int sd = 0; sd < 2; ++sd) {
            const uint4 *src =
                reinterpret_cast<const uint4 *>(side[sd]->krec + (size_t)b * side[sd]->n_pad * kRec);
            const int chunks = side[sd]->n_pad * (kRec / 8);   // n_pad <= kLdsMaxPoints
            for (int e = threadIdx.x; e < chunks; e += kPairWaves * kWave)
                recs[sd][lds_chunk(e >> 2, e & 3)] = src[e];
            const float4 *pts = side[sd]->pts + (size_t)b * side[sd]->n_pad;
            const float *pot = side[sd]->pot + (size_t)b * side[sd]->n;
            for (int i = threadIdx.x; i < side[sd]->n_pad; i += kPairWaves * kWave) {
                const float4 p = pts[i];
                sqs[sd][i] = sq3(p.x, p.y, p.z);
                pots[sd][i] = i < side[sd]->n ? pot[i] : 0.f;
                lws[sd][i] = i < side[sd]->n ? side[sd]->l2w[(size_t)b * side[sd]->n + i] : 0.f;
            }
        }
        __syncthreads();
    }
    // Query operands of a wave's row blocks: the records are fixed for the
    // stage, so each block's are loaded during the finish of the block before
    // (pre: the records An holds)
    const int lane = lane_id();
    const int lane_off = (lane & 15) * kRec + 8 * (lane >> 4);
    const int nbx = x.n_pad / kWave, nby = y.n_pad / kWave;
    auto rec_of = [&](const Side3 &s, int rb) {
        return s.qrec + ((size_t)b * s.n_pad + (size_t)rb * kWave) * kRec;
    };
    bf16x8 An[kGroups];
    const uint16_t *pre = nullptr;
    for (int it = 0; it < iters; ++it) {
        const bool stale = cold && it == 0;
        const bool last = it + 1 == iters;
        for (int rb = w; rb < nbx; rb += kPairWaves) {
            const uint16_t *need = rec_of(x, rb);
            if (pre != need)
                load_rows(An, need, lane_off);
            bf16x8 A[kGroups];
#pragma unroll
            for (int g = 0; g < kGroups; ++g)
                A[g] = An[g];
            pre = rb + kPairWaves < nbx ? rec_of(x, rb + kPairWaves)
                                        : (w < nby ? rec_of(y, w) : nullptr);
            wave_rows<kLds>(x, y, b, rb * kWave, two_c, eps_ln2, c_same, red[w], stale, recs[1],
                            recs[0], sqs[0], pots[0], lws[0], last, A, pre, An);
        }
        __syncthreads();   // f and the X-side biases are complete
        const double cn = it + 1 < iters ? c_same : c_next_last;
        for (int rb = w; rb < nby; rb += kPairWaves) {
            const uint16_t *need = rec_of(y, rb);
            if (pre != need)
                load_rows(An, need, lane_off);
            bf16x8 A[kGroups];
#pragma unroll
            for (int g = 0; g < kGroups; ++g)
                A[g] = An[g];
            pre = rb + kPairWaves < nby ? rec_of(y, rb + kPairWaves)
                                        : (w < nbx && !last ? rec_of(x, w) : nullptr);
            wave_rows<kLds>(y, x, b, rb * kWave, two_c, eps_ln2, cn, red[w], stale, recs[0],
                            recs[1], sqs[1], pots[1], lws[1], last, A, pre, An);
        }
        __syncthreads();   // g and the Y-side biases are complete
    }
}

// ---------------------------------------------------------------------------
// Whole stages of a small batch of small pairs in one launch, each pair split
// over work-groups (a single pair of 1024 points: 64 of them).  A launch per
// half-iteration costs more than the half-iteration's own work there (a
// separate launch took 4.5 us for a pair of 1024 points, of which the stream
// itself is under 1 us on 64 compute units), so the stage runs in one launch
// instead:
// work-group (b, part) owns rows 16 part .. 16 part + 15 of both sides of pair
// b, keeps both sides' key records in LDS (as the per-pair launch does) and,
// per half-iteration, streams all keys against its 16 rows, W waves each
// taking every W-th key tile.  The rows' new biases are what the other
// work-groups need next: each finished row publishes (tag, bias) as one 64-bit
// word in `xch`, and in the next half-iteration each wave reads the words of
// the keys of its own tiles until they carry that half-iteration's tag,
// writing the bias pieces into the LDS copy of the records, and streams them
// at once: the waves meet only to merge their sums.  The words are read and
// written with device-scope (relaxed atomic) loads and stores, which are
// coherent across the XCDs' L2 caches; no other memory is shared within the
// launch.  A word holds one value of one half-iteration: the producer of the
// next value for the same row first needs this half-iteration's results of
// every work-group, each of which has read the word by then, so no value is
// overwritten before it is read.  Tags count half-iterations from 1 within the
// launch and the words are zeroed before it (by the query-record kernel of the
// stage), so a word from an earlier launch never matches.
//
// Every wait is bounded by a wall-clock limit (wait_ticks of the constant
// 100 MHz counter; below 0, every wait fails at once): a work-group whose wait
// runs out stops waiting for the rest of the launch, publishes NaN biases and,
// at its end, writes NaN as the potentials of its rows, so every row that
// depends on the failed wait comes back NaN instead of the launch hanging.
// The launch needs all of its work-groups resident at once: it takes at most
// one work-group per two compute units, so that it fits beside other work.  Per row the arithmetic is that of the
// other matrix-core kernels (shifted stream, merged over the waves, made
// exact and streamed again when a row's sum leaves the range).
constexpr int kSplitRows = 16;   // rows of each side per work-group

// Key biases of half-iteration tag - 1 for the keys that wave w streams (the 16
// keys of each of its tiles w, w + W, ...; cnt tiles), from the words that
// every work-group publishes, into the LDS records recs (keys 0 .. nk-1; the
// padding keys' records keep their bias).  Each lane reads its keys' words
// together and polls again only those that do not yet carry the tag.
template <int W>
__device__ __forceinline__ void split_refresh(uint4 *recs, const uint64_t *xk, int nk, int w,
                                              int cnt, unsigned tag, long long wait_ticks,
                                              bool &dead)
{
    constexpr int kMaxTiles = (kLdsMaxPoints / kTile + W - 1) / W;   // tiles of one wave
    constexpr int kPer = kMaxTiles * kTile / kWave;                  // keys of one lane
    static_assert(kPer >= 1 && kPer * kWave == kMaxTiles * kTile, "lanes divide the keys");
    const int lane = lane_id();
    uint64_t v[kPer];
    int key[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const int i = lane + e * kWave;   // the wave's i-th key: tile i / 16 of its list
        const int j = (w + (i / kTile) * W) * kTile + i % kTile;
        key[e] = i / kTile < cnt && j < nk ? j : -1;
        v[e] = key[e] >= 0 ? __hip_atomic_load(xk + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : (uint64_t)tag << 32;
    }
    auto ready = [&]() {
        bool ok = true;
#pragma unroll
        for (int e = 0; e < kPer; ++e)
            ok = ok && (unsigned)(v[e] >> 32) == tag;
        return ok;
    };
    if (!dead && !ready()) {
        const long long t0 = (long long)wall_clock64();
        while (true) {
            if (wait_ticks < 0 || (long long)wall_clock64() - t0 > wait_ticks) {
                dead = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int e = 0; e < kPer; ++e)
                if ((unsigned)(v[e] >> 32) != tag)
                    v[e] = __hip_atomic_load(xk + key[e], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
            if (ready())
                break;
        }
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e)
        if (key[e] >= 0)
            store_key_bias_lds(recs, key[e], __uint_as_float((unsigned)v[e]));
}

// One half-iteration of a work-group: its 16 rows of side q against all keys of
// side k (records in k_lds).  h: the half-iteration's index in the launch
// (its results carry tag h + 1; for h > 0 the keys' biases are those of tag h).
// The rows' state (squared norm, potential, log2 weight) is in LDS (q_sq,
// q_pot, q_lw), the potentials written by wave 0 as it finishes the rows.
// Each wave refreshes the biases of its own tiles' keys and forms the shifts
// itself, so the only barrier is the one before the merge of the waves' sums
// (red: this half-iteration's buffer of two, so that the waves may start the
// next half-iteration while wave 0 merges).  A row whose merged sum leaves the
// range after a shifted pass is recomputed by wave 0 alone over all keys with
// exact shifts (the records stay in place until every wave has passed the next
// half-iteration's barrier, which wave 0 reaches only after this).
template <int W>
__device__ __forceinline__ void split_half(const Side3 &q, const Side3 &k, int b, int row0,
                                           bool has_rows, const bf16x8 (&A)[1],
                                           const float *q_sq, float *q_pot, const float *q_lw,
                                           uint4 *k_lds, float2 (*red)[kWave],
                                           float (*shv)[kSplitRows], float2 *redo_red,
                                           int *dead_any, int h, bool stale, bool last,
                                           bool publish, float two_c, double eps_ln2,
                                           double c_next, long long wait_ticks, bool &dead)
{
    if (!has_rows)
        return;   // the whole work-group: it holds no row of side q
    const int lane = lane_id();
    const int w = wave_id_uniform();
    const int kq = lane >> 4, c16 = lane & 15;
    const int lane_off = c16 * kRec + 8 * kq;
    const int row = row0 + lane;
    const int n_tiles = k.n_pad / kTile;
    const int cnt = w < n_tiles ? (n_tiles - w + W - 1) / W : 0;
    if (h > 0) {
        if (*dead_any)   // a wait of this work-group already ran out
            dead = true;
        split_refresh<W>(k_lds, k.xch + (size_t)b * k.n_pad, k.n, w, cnt, (unsigned)h,
                         wait_ticks, dead);
        if (dead)
            *dead_any = 1;
    }
    if (lane < kSplitRows)
        shv[w][lane] = -(0.5f * two_c * (q_sq[lane] - q_pot[lane]));
    __builtin_amdgcn_wave_barrier();   // a wave's LDS accesses complete in order
    f32x4 Cn[1], S[1];
    const float4 sh = *reinterpret_cast<const float4 *>(&shv[w][4 * kq]);
    Cn[0] = f32x4{sh.x, sh.y, sh.z, sh.w};
    S[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t *kb = k.krec + (size_t)b * k.n_pad * kRec;
    if (stale)
        exact_shifts<W, 1, true>(A, Cn, S, kb, k.n_pad, lane_off, w, cnt, red, w, kq, c16, k_lds);
    shifted_stream<W, 1, true>(A, Cn, S, kb, k.n_pad, lane_off, w, cnt, k_lds);
    wave_sums<1>(Cn, S, red[w], kq, c16);
    __syncthreads();   // every wave's sums are in red
    if (w != 0)
        return;
    float M = 0.f, Ssum = 0.f;
    bool bad = false;
    if (lane < kSplitRows) {
        M = red[0][lane].x;
#pragma unroll
        for (int v = 0; v < W; ++v)
            Ssum += red[v][lane].y;
        bad = row < q.n && !(Ssum >= kSumLo && Ssum <= kSumHi);
    }
    if (!stale && __ballot(bad) != 0) {
        Cn[0] = f32x4{sh.x, sh.y, sh.z, sh.w};
        S[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        exact_shifts<1, 1, true>(A, Cn, S, kb, k.n_pad, lane_off, 0, n_tiles, nullptr, 0, kq, c16,
                                 k_lds);
        shifted_stream<1, 1, true>(A, Cn, S, kb, k.n_pad, lane_off, 0, n_tiles, k_lds);
        wave_sums<1>(Cn, S, redo_red, kq, c16);
        __builtin_amdgcn_wave_barrier();
        if (lane < kSplitRows) {
            M = redo_red[lane].x;
            Ssum = redo_red[lane].y;
        }
        __builtin_amdgcn_wave_barrier();   // redo_red is written again later
    }
    if (lane < kSplitRows && row < q.n) {
        // the arithmetic of finish_row, the state in LDS
        const float sq = q_sq[lane], lw = q_lw[lane];
        const double lse2 = (double)M + (double)lg2(Ssum);
        const float f = (float)((double)sq - lse2 * eps_ln2);
        q_pot[lane] = f;
        const float beta = lw == kNeg ? kNeg : bias_of(c_next, f, sq, lw);
        // after a failed wait the row's bias goes out as NaN, so that every
        // row computed from it is NaN as well
        const float out = dead || *dead_any ? __builtin_nanf("") : beta;
        if (publish)
            __hip_atomic_store(q.xch + (size_t)b * q.n_pad + row,
                               (uint64_t)(unsigned)(h + 1) << 32 | __float_as_uint(out),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (last) {
            const size_t pt = (size_t)b * q.n_pad + row;
            q.pot[(size_t)b * q.n + row] = f;
            q.pts[pt].w = beta;
            store_key_bias(q.krec + pt * kRec, beta);
        }
    }
}

template <int W>
__global__ __launch_bounds__(W *kWave) void lse3s_kernel(Side3 x, Side3 y, int parts, int iters,
                                                         float two_c, double eps_ln2,
                                                         double c_next_last, int cold,
                                                         long long wait_ticks)
{
    __shared__ uint4 recs[2][kLdsMaxPoints * kRec / 8];
    __shared__ __align__(16) float2 red[2][W][kWave];
    __shared__ __align__(16) float shv[W][kSplitRows];
    __shared__ __align__(16) float2 redo_red[kWave];
    // the rows' state, per side: squared norm, potential, log2 weight
    __shared__ float sqs[2][kSplitRows], pots[2][kSplitRows], lws[2][kSplitRows];
    __shared__ int dead_any;
    const int b = blockIdx.x / parts;
    const int row0 = (blockIdx.x - b * parts) * kSplitRows;
    const int lane = lane_id();
    const int w = wave_id_uniform();
    const Side3 *side[2] = {&x, &y};
    if (threadIdx.x == 0)
        dead_any = 0;
#pragma unroll
    for (int sd = 0; sd < 2; ++sd) {
        const uint4 *src =
            reinterpret_cast<const uint4 *>(side[sd]->krec + (size_t)b * side[sd]->n_pad * kRec);
        const int chunks = side[sd]->n_pad * (kRec / 8);   // n_pad <= kLdsMaxPoints
        for (int e = threadIdx.x; e < chunks; e += W * kWave)
            recs[sd][lds_chunk(e >> 2, e & 3)] = src[e];
        if (threadIdx.x < kSplitRows) {
            const int row = row0 + threadIdx.x;
            float sq = 0.f, pot = 0.f, lw = 0.f;
            if (row < side[sd]->n_pad) {
                const float4 p = side[sd]->pts[(size_t)b * side[sd]->n_pad + row];
                sq = sq3(p.x, p.y, p.z);
                if (row < side[sd]->n) {
                    pot = side[sd]->pot[(size_t)b * side[sd]->n + row];
                    lw = side[sd]->l2w[(size_t)b * side[sd]->n + row];
                }
            }
            sqs[sd][threadIdx.x] = sq;
            pots[sd][threadIdx.x] = pot;
            lws[sd][threadIdx.x] = lw;
        }
    }
    // the rows' query operands (fixed for the stage), in every wave
    const bool has_x = row0 < x.n_pad, has_y = row0 < y.n_pad;
    const int lane_off = (lane & 15) * kRec + 8 * (lane >> 4);
    bf16x8 Ax[1], Ay[1];
    if (has_x)
        load_rows<1>(Ax, x.qrec + ((size_t)b * x.n_pad + row0) * kRec, lane_off);
    if (has_y)
        load_rows<1>(Ay, y.qrec + ((size_t)b * y.n_pad + row0) * kRec, lane_off);
    __syncthreads();   // records and row state are in LDS
    bool dead = false;
    const double c_same = 0.5 * (double)two_c;
    for (int it = 0; it < iters; ++it) {
        const bool stale = cold && it == 0;
        const bool last = it + 1 == iters;
        split_half<W>(x, y, b, row0, has_x, Ax, sqs[0], pots[0], lws[0], recs[1], red[0], shv,
                      redo_red, &dead_any, 2 * it, stale, last, true, two_c, eps_ln2, c_same,
                      wait_ticks, dead);
        split_half<W>(y, x, b, row0, has_y, Ay, sqs[1], pots[1], lws[1], recs[0], red[1], shv,
                      redo_red, &dead_any, 2 * it + 1, stale, last, !last, two_c, eps_ln2,
                      last ? c_next_last : c_same, wait_ticks, dead);
    }
    __syncthreads();
    if (dead_any && w == 0 && lane < kSplitRows) {
        const int row = row0 + lane;
        if (has_x && row < x.n)
            x.pot[(size_t)b * x.n + row] = __builtin_nanf("");
        if (has_y && row < y.n)
            y.pot[(size_t)b * y.n + row] = __builtin_nanf("");
    }
}

// Merge of the split partials of every row.  Matrix-core partials of a row
// share one shift (vector-pass partials are exact states), so the merge is a
// sum.  With redo, a row whose merged sum left [2^-64, 2^100] is not finished;
// its 64-row block is marked (every block's mark is written on every pass) and
// the repair launch of lse3m_kernel recomputes it with exact shifts.
__global__ void lse3_finalize(float4 *__restrict__ qpts, uint16_t *__restrict__ qkrec,
                              float *__restrict__ qpot,
                              const float *__restrict__ ql2w, const float2 *__restrict__ part,
                              int *__restrict__ redo, int B, int nq, int nq_pad, int splits,
                              double eps_ln2, double c_next)
{
    const int b = blockIdx.y;
    const int row = blockIdx.x * blockDim.x + threadIdx.x;   // blockDim: whole waves
    bool bad = false;
    if (row < nq) {
        float2 s0 = part[(size_t)b * nq_pad + row];
        float M = s0.x, S = s0.y;
        for (int s = 1; s < splits; ++s) {
            const float2 o = part[((size_t)s * B + b) * nq_pad + row];
            lse_merge(M, S, o.x, o.y);
        }
        bad = redo && !(S >= kSumLo && S <= kSumHi);
        const size_t pt = (size_t)b * nq_pad + row;
        if (!bad)
            finish_row(qpts, qkrec, qpot, ql2w[(size_t)b * nq + row], pt, (size_t)b * nq + row,
                       qpts[pt], M, S, eps_ln2, c_next);
    }
    if (redo) {
        const bool any = __ballot(bad) != 0;
        const int rb = row / kWave;
        if (lane_id() == 0 && rb < nq_pad / kWave)
            redo[(size_t)b * (nq_pad / kWave) + rb] = any ? 1 : 0;
    }
}

// Column splits so that a launch has about 4 work-groups per CU.  A split costs
// two more launches (the merge and the repair of stale blocks), so rows of at
// most 64 tiles per wave are never split: there the launch is latency-bound and
// one kernel is as fast or faster (one pair of 4096 points: 8% slower split;
// four pairs of 8192: 13% slower; one pair of 8192: 5% faster).
int lse3_splits(int B, int nq_pad, int nk_pad)
{
    const long groups = (long)B * (nq_pad / kWave);
    const int tiles = nk_pad / kTile;
    if (tiles <= 64 * kWaves)
        return 1;
    int splits = (int)((1024 + groups - 1) / groups);
    const int max_splits = tiles / (2 * kWaves);  // keep >= 2 tiles per wave
    if (splits > max_splits)
        splits = max_splits;
    return splits < 1 ? 1 : splits;
}


// Waves per work-group of the matrix-core pass.  Every wave pays a fixed cost
// (query operands, shift, merge) besides its key tiles.  Long rows (512 tiles
// or more per split) take 8 waves; shorter rows take at most 4, and the fewest
// that still give about 4096 waves per launch (4 per SIMD), which spreads that
// fixed cost over the most tiles.  Every wave gets at least 2 tiles.
int lse3m_waves(long groups, int tiles_per_split)
{
    int w = tiles_per_split >= 512 ? 8 : 4;
    if (tiles_per_split < 512)
        while (w > 1 && groups * (w / 2) >= 4096)
            w /= 2;
    while (w > 1 && tiles_per_split < 2 * w)
        w /= 2;
    return w;
}

// A launch of fewer 64-row blocks than a quarter of the compute units (a single
// small pair: 16 blocks for 1024 points) uses 16-row work-groups of
// kSmallWaves waves instead, four times as many, so that more compute units
// share the pass; every wave keeps at least 2 tiles.
constexpr int kSmallWaves = 8;
bool lse3m_small(long groups, int tiles_per_split)
{
    return groups * 4 <= 256 && tiles_per_split >= 2 * kSmallWaves;
}

template <int W, int G>
void launch_lse3m_w(dim3 grid, hipStream_t st, Side3 q, Side3 k, float2 *part, const int *redo,
                    int tiles_per_split, float two_c, double eps_ln2, double c_next)
{
    hipLaunchKernelGGL((lse3m_kernel<W, G>), grid, dim3(W * kWave), 0, st, q.pts, q.krec,
                       (const uint16_t *)q.qrec, (const uint16_t *)k.krec, q.pot,
                       (const float *)q.l2w, part, redo, q.n, q.n_pad, k.n_pad, tiles_per_split,
                       two_c, eps_ln2, c_next);
}

// grid.x counts 64-row blocks; with 16-row work-groups it is multiplied by 4
void launch_lse3m(dim3 grid, hipStream_t st, Side3 q, Side3 k, float2 *part, const int *redo,
                  int tiles_per_split, float two_c, double eps_ln2, double c_next)
{
    const long groups = (long)grid.x * grid.y * grid.z;
    if (!part && !redo && lse3m_small(groups, tiles_per_split)) {
        const dim3 g16(grid.x * 4, grid.y, grid.z);
        launch_lse3m_w<kSmallWaves, 1>(g16, st, q, k, part, redo, tiles_per_split, two_c,
                                        eps_ln2, c_next);
        return;
    }
    switch (lse3m_waves(groups, tiles_per_split)) {
    case 1: launch_lse3m_w<1, kGroups>(grid, st, q, k, part, redo, tiles_per_split, two_c, eps_ln2, c_next); break;
    case 2: launch_lse3m_w<2, kGroups>(grid, st, q, k, part, redo, tiles_per_split, two_c, eps_ln2, c_next); break;
    case 4: launch_lse3m_w<4, kGroups>(grid, st, q, k, part, redo, tiles_per_split, two_c, eps_ln2, c_next); break;
    default: launch_lse3m_w<8, kGroups>(grid, st, q, k, part, redo, tiles_per_split, two_c, eps_ln2, c_next); break;
    }
}
}  // namespace

size_t lse3_partial_floats2(int B, int nq_pad, int nk_pad)
{
    const int s = lse3_splits(B, nq_pad, nk_pad);
    return s > 1 ? (size_t)s * B * nq_pad : 0;
}

int center3_parts(int n, int m) { return ceil_div(n + m, kCenterChunk); }

hipError_t launch_center3(const void *X, int dtype, int n, const void *Y, int m, int B,
                          float4 *part,
                          float4 *center, hipStream_t st)
{
    const int parts = center3_parts(n, m);
    if (dtype == 1)
        hipLaunchKernelGGL(center3_parts_kernel<uint16_t>, dim3(parts, B), dim3(256), 0, st,
                           (const uint16_t *)X, n, (const uint16_t *)Y, m, part);
    else
        hipLaunchKernelGGL(center3_parts_kernel<float>, dim3(parts, B), dim3(256), 0, st,
                           (const float *)X, n, (const float *)Y, m, part);
    hipLaunchKernelGGL(center3_kernel, dim3(B), dim3(256), 0, st, (const float4 *)part, parts,
                       center);
    return hipGetLastError();
}

hipError_t launch_pack3(const void *X, int dtype, const float *w, int warm, int B, Side3 s,
                        const float4 *center, double c0, hipStream_t st)
{
    dim3 grid(ceil_div(s.n_pad, 256), B);
    if (dtype == 1)
        hipLaunchKernelGGL(pack3_kernel<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)X, w,
                           warm, s.n, s.n_pad, center, s.pts, s.pot, s.l2w, s.krec, c0);
    else
        hipLaunchKernelGGL(pack3_kernel<float>, grid, dim3(256), 0, st, (const float *)X, w, warm,
                           s.n, s.n_pad, center, s.pts, s.pot, s.l2w, s.krec, c0);
    return hipGetLastError();
}

hipError_t launch_qrec3(Side3 s, int B, float eps, hipStream_t st)
{
    dim3 grid(ceil_div(s.n_pad, 256), B);
    hipLaunchKernelGGL(qrec3_kernel, grid, dim3(256), 0, st, (const float4 *)s.pts, s.n_pad,
                       2.0f * scale_of(eps), s.qrec, s.xch);
    return hipGetLastError();
}

bool lse3_pairwise(int B, int n_pad, int m_pad)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return false;
    return B >= cus && n_pad <= kPairMaxPoints && m_pad <= kPairMaxPoints;
}

hipError_t launch_lse3_pairwise(Side3 x, Side3 y, int B, float eps, int iters, float eps_next,
                                bool cold, hipStream_t st)
{
    const float c = scale_of(eps);
    if (x.n_pad <= kLdsMaxPoints && y.n_pad <= kLdsMaxPoints)
        hipLaunchKernelGGL(lse3p_kernel<true>, dim3(B), dim3(kPairWaves * kWave), 0, st, x, y,
                           iters, 2.0f * c, 1.0 / (double)c, (double)scale_of(eps_next),
                           cold ? 1 : 0);
    else
        hipLaunchKernelGGL(lse3p_kernel<false>, dim3(B), dim3(kPairWaves * kWave), 0, st, x, y,
                           iters, 2.0f * c, 1.0 / (double)c, (double)scale_of(eps_next),
                           cold ? 1 : 0);
    return hipGetLastError();
}

constexpr int kSplitWaves = 8;   // waves per work-group of the split stage launch
std::atomic<long long> g_split_wait_us{1000000};

long long lse3_split_set_wait_us(long long us) { return g_split_wait_us.exchange(us); }

int lse3_split_parts(int B, int n_pad, int m_pad)
{
    if (n_pad > kLdsMaxPoints || m_pad > kLdsMaxPoints)
        return 0;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    const int parts = std::max(n_pad, m_pad) / kSplitRows;
    return 2L * B * parts <= cus ? parts : 0;
}

hipError_t launch_lse3_split(Side3 x, Side3 y, int B, int parts, float eps, int iters,
                             float eps_next, bool cold, hipStream_t st)
{
    if (!x.xch || !y.xch || x.n_pad > kLdsMaxPoints || y.n_pad > kLdsMaxPoints ||
        parts * kSplitRows < std::max(x.n_pad, y.n_pad))
        return hipErrorInvalidValue;
    int dev = 0, khz = 0;
    hipError_t e;
    if ((e = hipGetDevice(&dev)) != hipSuccess ||
        (e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess)
        return e;
    const long long us = g_split_wait_us.load();
    const long long ticks = us < 0 ? -1 : us * (long long)khz / 1000;
    const float c = scale_of(eps);
    hipLaunchKernelGGL(lse3s_kernel<kSplitWaves>, dim3(B * parts), dim3(kSplitWaves * kWave), 0,
                       st, x, y, parts, iters, 2.0f * c, 1.0 / (double)c,
                       (double)scale_of(eps_next), cold ? 1 : 0, ticks);
    return hipGetLastError();
}

hipError_t launch_lse3(Side3 q, Side3 k, int B, float eps, float eps_next, float2 *part,
                       bool mfma, hipStream_t st)
{
    // one fp32 value of c = log2(e)/eps is used everywhere (scores, bias, result)
    const float c = scale_of(eps);
    const double c_next = (double)scale_of(eps_next);
    const double eps_ln2 = 1.0 / (double)c;
    const int splits = lse3_splits(B, q.n_pad, k.n_pad);
    const int tiles = k.n_pad / kTile;
    const int tiles_per_split = ceil_div(tiles, splits);
    dim3 grid(q.n_pad / kWave, splits, B);
    if (mfma)
        launch_lse3m(grid, st, q, k, splits > 1 ? part : nullptr, nullptr, tiles_per_split,
                     2.0f * c, eps_ln2, c_next);
    else
        hipLaunchKernelGGL(lse3_kernel, grid, dim3(kWaves * kWave), 0, st, q.pts, q.krec,
                           (const float4 *)k.pts, q.pot, (const float *)q.l2w,
                           splits > 1 ? part : nullptr, q.n, q.n_pad, k.n_pad, tiles_per_split,
                           2.0f * c, eps_ln2, c_next);
    if (splits > 1) {
        int *redo = mfma ? q.redo : nullptr;
        dim3 g2(ceil_div(q.n, 256), B);
        hipLaunchKernelGGL(lse3_finalize, g2, dim3(256), 0, st, q.pts, q.krec, q.pot,
                           (const float *)q.l2w, (const float2 *)part, redo, B, q.n, q.n_pad,
                           splits, eps_ln2, c_next);
        if (redo)   // rows whose merged sum left the range, with exact shifts over all keys
            launch_lse3m(dim3(q.n_pad / kWave, 1, B), st, q, k, nullptr, redo, tiles, 2.0f * c,
                         eps_ln2, c_next);
    }
    return hipGetLastError();
}

}  // namespace sk

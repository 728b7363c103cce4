// hvp_feat.hip -- Hessian-vector product for bf16 feature clouds with d = 32
// or 64, every sum over the plan on the matrix cores.
//
// FlashSinkhorn summary, Methodologie 3 (Hessiaan-Vector Producten): the HVP
// as transport-vector and transport-matrix products, nothing of size n x m
// stored.  The quantities and the conjugate-gradient solve are those of the
// fp64 path (hvp.hip); here the plan is written, as in the dense gradient, as
//     P_ij = a_i E_ij,   E_ij = 2^(2c (x_i.y_j + h_i) + beta_j),
//     c = log2(e)/eps,   h_i = (f_i - ||x_i||^2) / 2,   beta_j = c (g_j - ||y_j||^2) + log2 b_j,
// and every pass is a sum of E against vectors or matrices.
//
// Row passes (16-row groups held as the B operand, key tiles streaming as A):
//     first:  m_i = sum_j E_ij,  O_i = sum_j E_ij y_j,  Q_i = sum_j E_ij s_ij y_j,
//             s_ij = v_i.y_j (a third contraction, v_i as B in two bf16 pieces);
//     CG:     e_i = sum_j E_ij u_j;
//     final:  e_i and W_i = sum_j E_ij u_j y_j  (u = dg).
// Column passes (16-key groups held as B, row tiles streaming as A):
//     first:  sum_i a_i E_ij = mb_j,  sum_i a_i ur_i E_ij,  sum_i a_i t_i E_ij,
//             PV_j = sum_i a_i E_ij v_i;
//     CG:     sum_i w_i E_ij.
// With t_i = v_i.x_i and sigma_i = v_i.O_i (= sum_j E_ij s_ij):
//     ma_i = a_i m_i,   D1_i = a_i (m_i x_i - O_i),   tv_i = v_i.D1_i,
//     Tv_i = t_i D1_i - a_i (sigma_i x_i - Q_i),
//     tw_j = y_j.PV_j - sum_i a_i t_i E_ij,   rhs_j = -2 tw_j - (P^T ur)_j,
//     (P u)_i = a_i e_i,   Du_i = a_i (e_i x_i - W_i).
//
// Both orientations feed the same operands to the same instruction -- the
// rows' bf16 points, the keys' bf16 points and h_i in the accumulator input,
// with A and B exchanged -- and add beta_j in the same fma, so a column pass
// sees the row passes' E bit for bit (the instruction gives identical results
// with A and B exchanged: an in-bounds probe over 2^20 random entries found no
// bit different).
// E, E u and E s enter the transport-matrix products as hi + lo bf16 pieces
// (16 bits); v enters as two bf16 pieces, and every sum that v enters uses
// those pieces, so the plan sums are exact for that rounded direction.  Sums
// are fp32; the work-group's waves merge in LDS in wave order and the key (or
// row) splits are added in split order in fp64, so results are deterministic.
//
// The potentials are meant to solve the problem at eps: a live row whose mass
// m_i falls outside [2^-64, 2^100] marks its pair, whose output (HV and the
// residual) is then NaN.
#include "hvp.h"
#include "plan_rows_mc.h"

#include <algorithm>

namespace sk {
namespace {

using mc::kRowsCg;
using mc::kRowsFinal;
using mc::kRowsFirst;
using mc::score;
using mc::zero4;
constexpr int kWavesH = mc::kWaves;   // waves per work-group of the plan passes
constexpr int kKeysH = mc::kTile;     // keys (or rows) per streamed tile
constexpr float kMassLoH = 5.421010862e-20f;   // 2^-64
constexpr float kMassHiH = 1.2676506e30f;      // 2^100
constexpr int kGroupsCg = 4;      // 16-point groups per wave, CG passes
constexpr int kGroupsRows1 = 2;   // the first row pass (three products)
constexpr int kGroupsOther = 4;   // the first column pass and the final row pass
constexpr int kTilesCg = 8;       // 16-point tiles per LDS stage, CG passes
constexpr int kTilesVec = 4;      // the same, passes with d-vector sums
// work-groups a pass aims for: the CG passes (scalar partials) split finely, the
// passes with d-vector partials less so
constexpr int kTargetCg = 4096;
constexpr int kTargetVec = 1024;
// Relative CG residual at which the solve stops: the plan products carry fp32
// rounding (2^-24 relative), and past about 2^-20 further steps only move the
// iterate along that rounding.
constexpr double kCgStop = 9.5367431640625e-07;   // 2^-20
// every work-group's points lie inside the padded arrays
static_assert(kHvpPad % (kWavesH * 16 * kGroupsCg) == 0 &&
                  kHvpPad % (kWavesH * 16 * kGroupsRows1) == 0 &&
                  kHvpPad % (kWavesH * 16 * kGroupsOther) == 0,
              "padding must hold whole work-groups");

enum : int { kColsCg = 0, kColsFirst = 1 };

// Columns pass.  Work-group blockIdx.y holds kWavesH G groups of 16 keys, G per
// wave; pair blockIdx.z; the row tiles of split blockIdx.x stream through LDS as
// in the rows pass.  part_s [NS][S][B][m_pad] with NS = 3 (first: sums against
// w0 = a, w1 = a ur, w2 = a t) or 1 (CG: against w0); part_v [S][B][m_pad][d]:
// PV_j (first).
template <int DK, int G, int NT, int MODE>
__global__ __launch_bounds__(kWavesH *kWave) void hvp_cols_kernel(
    const uint16_t *__restrict__ X, const float *__restrict__ h, int n, int n_pad,
    const uint16_t *__restrict__ Y, const float *__restrict__ ybias, int m, int m_pad,
    const float *__restrict__ w0, const float *__restrict__ w1, const float *__restrict__ w2,
    const uint16_t *__restrict__ vth, const uint16_t *__restrict__ vtl, float two_c, int tps,
    float *__restrict__ part_s, float *__restrict__ part_v)
{
    constexpr int d = 32 * DK;
    constexpr int NB = d / 16;
    constexpr int R = 16 * G;   // keys per wave
    constexpr bool kFirst = MODE == kColsFirst;
    constexpr int NS = kFirst ? 3 : 1;
    constexpr int SR = NT * kKeysH;                        // rows per stage
    constexpr int kCh = d / 8;
    constexpr int kStr = kCh + 1;
    constexpr int kThr = kWavesH * kWave;
    constexpr int kXL = (SR * kCh + kThr - 1) / kThr;      // row chunks per thread
    constexpr int kTCh = SR / 8;
    constexpr int kTStr = SR + 8;
    constexpr int kTL = kFirst ? (d * kTCh + kThr - 1) / kThr : 1;
    static_assert(SR <= kThr && kXL <= 2 && kTL <= 1, "a stage in few chunks a thread");
    __shared__ uint4 xbuf[2][SR * kStr];
    __shared__ __align__(16) float hbuf[2][SR];
    __shared__ __align__(16) float wbuf[2][NS][SR];
    __shared__ __align__(16) uint16_t vhbuf[2][kFirst ? d * kTStr : 8];
    __shared__ __align__(16) uint16_t vlbuf[2][kFirst ? d * kTStr : 8];
    const int split = blockIdx.x, S = gridDim.x, b = blockIdx.z, B = gridDim.z;
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id_uniform();
    const int kq = lane >> 4, c16 = lane & 15;
    const int key0 = (blockIdx.y * kWavesH + w) * R;   // + R <= m_pad

    // the keys as the B operand (the rows pass's A), beta_j added after the sum
    bf16x8 Yo[G][2];
    float bk[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int ka = key0 + 16 * g + c16;
        const int kc = min(ka, m - 1);
#pragma unroll
        for (int kb = 0; kb < DK; ++kb)
            Yo[g][kb] = load8(Y + ((size_t)b * m + kc) * d + 32 * kb + 8 * kq);
        bk[g] = ybias[(size_t)b * m_pad + ka];
    }
    float acc[NS][G];
    f32x4 PV[kFirst ? G : 1][NB];
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
            acc[s][g] = 0.f;
        if constexpr (kFirst) {
#pragma unroll
            for (int q = 0; q < NB; ++q)
                PV[g][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    const uint4 *xk = reinterpret_cast<const uint4 *>(X + (size_t)b * n * d);
    const size_t wo = (size_t)b * n_pad;
    const float *const ws[3] = {w0 + wo, w1 + wo, w2 + wo};
    const uint16_t *vhb = vth + (size_t)b * d * n_pad;
    const uint16_t *vlb = vtl + (size_t)b * d * n_pad;
    const int n_tiles = n_pad / kKeysH;
    const int t0 = split * tps, t1 = min(n_tiles, t0 + tps);
    const int n_st = t0 < t1 ? (t1 - t0 + NT - 1) / NT : 0;
    // a stage's values: row chunks (rows clamped inside the pair; rows past the
    // pair have h = kNeg, rows past the split are not read), h and the row
    // values of row tid, and the transposed direction's chunks
    // (named registers, not arrays: see the rows pass)
    uint4 xr0 = zero4(), xr1 = zero4(), vhr = zero4(), vlr = zero4();
    float hr = kNeg, wr0 = 0.f, wr1 = 0.f, wr2 = 0.f;
    const int rend = t1 * kKeysH;
    auto row_chunk = [&](int r0, int e) {
        return e < SR * kCh ? xk[(size_t)min(r0 + e / kCh, n - 1) * kCh + e % kCh] : zero4();
    };
    auto fetch = [&](int st) {
        const int r0 = (t0 + st * NT) * kKeysH;
        xr0 = row_chunk(r0, tid);
        if constexpr (kXL > 1)
            xr1 = row_chunk(r0, tid + kThr);
        if (tid < SR) {
            const int rr = r0 + tid;
            const bool in = rr < rend;
            hr = in ? h[wo + rr] : kNeg;
            wr0 = in ? ws[0][rr] : 0.f;
            if constexpr (kFirst) {
                wr1 = in ? ws[1][rr] : 0.f;
                wr2 = in ? ws[2][rr] : 0.f;
            }
        }
        if constexpr (kFirst) {
            const int e = tid;
            const int rr = r0 + 8 * (e % kTCh);   // a multiple of 8, as is n_pad
            const size_t o = (size_t)(e / kTCh) * n_pad + rr;
            const bool in = e < d * kTCh && rr < n_pad;
            vhr = in ? *reinterpret_cast<const uint4 *>(vhb + o) : zero4();
            vlr = in ? *reinterpret_cast<const uint4 *>(vlb + o) : zero4();
        }
    };
    auto put_row = [&](int bf, int e, uint4 v) {
        if (e < SR * kCh)
            xbuf[bf][(e / kCh) * kStr + e % kCh] = v;
    };
    auto stash = [&](int bf) {
        put_row(bf, tid, xr0);
        if constexpr (kXL > 1)
            put_row(bf, tid + kThr, xr1);
        if (tid < SR) {
            hbuf[bf][tid] = hr;
            wbuf[bf][0][tid] = wr0;
            if constexpr (kFirst) {
                wbuf[bf][1][tid] = wr1;
                wbuf[bf][2][tid] = wr2;
            }
        }
        if constexpr (kFirst) {
            const int e = tid;
            if (e < d * kTCh) {
                const int o = (e / kTCh) * kTStr + 8 * (e % kTCh);
                *reinterpret_cast<uint4 *>(&vhbuf[bf][o]) = vhr;
                *reinterpret_cast<uint4 *>(&vlbuf[bf][o]) = vlr;
            }
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
            fetch(st + 1);
        const int nt = min(NT, t1 - (t0 + st * NT));
        for (int tt = 0; tt < nt; ++tt) {
            bf16x8 Xa[2];
#pragma unroll
            for (int kb = 0; kb < DK; ++kb)
                Xa[kb] = __builtin_bit_cast(bf16x8,
                                            xbuf[bf][(tt * kKeysH + c16) * kStr + 4 * kb + kq]);
            const int r4 = tt * kKeysH + 4 * kq;
            const float4 h4 = *reinterpret_cast<const float4 *>(&hbuf[bf][r4]);
            const f32x4 Cin = f32x4{h4.x, h4.y, h4.z, h4.w};
            const float4 a4 = *reinterpret_cast<const float4 *>(&wbuf[bf][0][r4]);
            float4 u4 = make_float4(0.f, 0.f, 0.f, 0.f), t4 = u4;
            i16x4 Bh[kFirst ? NB : 1], Bl[kFirst ? NB : 1];
            if constexpr (kFirst) {
                u4 = *reinterpret_cast<const float4 *>(&wbuf[bf][1][r4]);
                t4 = *reinterpret_cast<const float4 *>(&wbuf[bf][2][r4]);
#pragma unroll
                for (int q = 0; q < NB; ++q) {
                    const int o = (16 * q + c16) * kTStr + r4;
                    Bh[q] = *reinterpret_cast<const i16x4 *>(&vhbuf[bf][o]);
                    Bl[q] = *reinterpret_cast<const i16x4 *>(&vlbuf[bf][o]);
                }
            }
            f32x4 D[G];
#pragma unroll
            for (int g = 0; g < G; ++g)
                D[g] = score(Xa, Yo[g], Cin, DK);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float E[4] = {ex2(fmaf(two_c, D[g][0], bk[g])),
                                    ex2(fmaf(two_c, D[g][1], bk[g])),
                                    ex2(fmaf(two_c, D[g][2], bk[g])),
                                    ex2(fmaf(two_c, D[g][3], bk[g]))};
                {
                    float s = fmaf(E[0], a4.x, acc[0][g]);
                    s = fmaf(E[1], a4.y, s);
                    s = fmaf(E[2], a4.z, s);
                    acc[0][g] = fmaf(E[3], a4.w, s);
                }
                if constexpr (kFirst) {
                    float s = fmaf(E[0], u4.x, acc[1][g]);
                    s = fmaf(E[1], u4.y, s);
                    s = fmaf(E[2], u4.z, s);
                    acc[1][g] = fmaf(E[3], u4.w, s);
                    s = fmaf(E[0], t4.x, acc[2][g]);
                    s = fmaf(E[1], t4.y, s);
                    s = fmaf(E[2], t4.z, s);
                    acc[2][g] = fmaf(E[3], t4.w, s);
                    const float aE[4] = {E[0] * a4.x, E[1] * a4.y, E[2] * a4.z, E[3] * a4.w};
                    i16x4 hi, lo;
                    split2(aE, hi, lo);
#pragma unroll
                    for (int q = 0; q < NB; ++q) {
                        PV[g][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, Bh[q], PV[g][q], 0, 0, 0);
                        PV[g][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, Bl[q], PV[g][q], 0, 0, 0);
                        PV[g][q] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, Bh[q], PV[g][q], 0, 0, 0);
                    }
                }
            }
        }
        if (st + 1 < n_st)
            stash(bf ^ 1);
        __syncthreads();
    }
    // a key's scalars are spread over the four lanes sharing l % 16
    const size_t base = ((size_t)split * B + b) * m_pad + key0;
    const size_t plane = (size_t)S * B * m_pad;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            float v = acc[s][g] + __shfl_xor(acc[s][g], 16, kWave);
            v += __shfl_xor(v, 32, kWave);
            if (kq == 0)
                part_s[s * plane + base + 16 * g + c16] = v;
        }
        if constexpr (kFirst) {
#pragma unroll
            for (int q = 0; q < NB; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    part_v[(base + 16 * g + 4 * kq + r) * d + 16 * q + c16] = PV[g][q][r];
        }
    }
}

__device__ __forceinline__ double row_weight(const float *a, size_t ri, int n)
{
    return a ? (double)a[ri] : 1.0 / (double)n;
}

// One wave per row (lane = dimension): h_i, the row weights for the column
// passes, and v in two bf16 pieces; padding rows get h = kNeg and zeros.
__global__ __launch_bounds__(256) void hvp_prep_rows(const uint16_t *__restrict__ X,
                                                     const float *__restrict__ a,
                                                     const float *__restrict__ f,
                                                     const float *__restrict__ V, int n, int n_pad,
                                                     int d, float *__restrict__ h,
                                                     float *__restrict__ wa, float *__restrict__ wu,
                                                     float *__restrict__ wt,
                                                     uint16_t *__restrict__ vh,
                                                     uint16_t *__restrict__ vl)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int k = lane_id();
    const int b = blockIdx.y;
    if (row >= n_pad)
        return;
    const size_t rp = (size_t)b * n_pad + row;
    const bool real = row < n;
    const size_t ri = (size_t)b * n + (real ? row : 0);
    double x = 0.0;
    float v = 0.f;
    if (real && k < d) {
        x = (double)bf16_to_float(X[ri * d + k]);
        v = V[ri * d + k];
    }
    const double sq = wave_sum(x * x);
    if (k < d) {
        const __bf16 hi = (__bf16)v;
        const __bf16 lo = (__bf16)(v - (float)hi);
        vh[rp * d + k] = __builtin_bit_cast(uint16_t, hi);
        vl[rp * d + k] = __builtin_bit_cast(uint16_t, lo);
    }
    if (k == 0) {
        const double ai = real ? row_weight(a, ri, n) : 0.0;
        h[rp] = ai > 0.0 ? (float)(0.5 * ((double)f[ri] - (double)(float)sq)) : kNeg;
        wa[rp] = (float)ai;
        wu[rp] = 0.f;
        wt[rp] = 0.f;
    }
}

// One wave per row: the first row pass's splits added in order (fp64), then
// ma, D1, tv, Tv, the row mass, the column pass's row values a ur and a t, and
// the range flag of the pair.
__global__ __launch_bounds__(256) void hvp_rows_first_combine(
    const float *__restrict__ part_s, const float *__restrict__ part_v,
    const float *__restrict__ part_q, int S, int B, int n, int n_pad, int d,
    const uint16_t *__restrict__ X, const float *__restrict__ a, const uint16_t *__restrict__ vh,
    const uint16_t *__restrict__ vl, double *__restrict__ mrow, double *__restrict__ ma,
    double *__restrict__ tv, double *__restrict__ D1, double *__restrict__ Tv,
    float *__restrict__ wu, float *__restrict__ wt, int *__restrict__ bad)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int k = lane_id();
    const int b = blockIdx.y;
    if (row >= n)
        return;
    const size_t ri = (size_t)b * n + row, rp = (size_t)b * n_pad + row;
    const bool on = k < d;
    double ms = 0.0, O = 0.0, Q = 0.0;
    for (int s = 0; s < S; ++s) {
        const size_t o = ((size_t)s * B + b) * n_pad + row;
        ms += (double)part_s[o];
        if (on) {
            O += (double)part_v[o * d + k];
            Q += (double)part_q[o * d + k];
        }
    }
    const double ai = row_weight(a, ri, n);
    const double x = on ? (double)bf16_to_float(X[ri * d + k]) : 0.0;
    const double v = on ? (double)bf16_to_float(vh[rp * d + k]) +
                              (double)bf16_to_float(vl[rp * d + k])
                        : 0.0;
    const double d1 = ai * (ms * x - O);
    const double t = wave_sum(v * x);
    const double sig = wave_sum(v * O);
    const double tvi = wave_sum(v * d1);
    const double mai = ai * ms;
    if (on) {
        D1[ri * d + k] = d1;
        Tv[ri * d + k] = t * d1 - ai * (sig * x - Q);
    }
    if (k == 0) {
        mrow[ri] = ms;
        ma[ri] = mai;
        tv[ri] = tvi;
        const double ur = mai > 0.0 ? 2.0 * tvi / mai : 0.0;
        wu[rp] = (float)(ai * ur);
        wt[rp] = (float)(ai * t);
        if (ai > 0.0 && !(ms >= (double)kMassLoH && ms <= (double)kMassHiH))
            bad[b] = 1;
    }
}

// One wave per key: the first column pass's splits added in order, then mb
// and rhs_j = -2 (y_j.PV_j - tau_j) - muc_j.
__global__ __launch_bounds__(256) void hvp_cols_first_combine(
    const float *__restrict__ part_s, const float *__restrict__ part_v, int S, int B, int m,
    int m_pad, int d, const uint16_t *__restrict__ Y, double *__restrict__ mb,
    double *__restrict__ rhs)
{
    const int key = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int k = lane_id();
    const int b = blockIdx.y;
    if (key >= m)
        return;
    const size_t kj = (size_t)b * m + key;
    const size_t plane = (size_t)S * B * m_pad;
    double mbs = 0.0, muc = 0.0, tau = 0.0, pv = 0.0;
    for (int s = 0; s < S; ++s) {
        const size_t o = ((size_t)s * B + b) * m_pad + key;
        mbs += (double)part_s[o];
        muc += (double)part_s[plane + o];
        tau += (double)part_s[2 * plane + o];
        if (k < d)
            pv += (double)part_v[o * d + k];
    }
    const double y = k < d ? (double)bf16_to_float(Y[kj * d + k]) : 0.0;
    const double tw = wave_sum(y * pv) - tau;
    if (k == 0) {
        mb[kj] = mbs;
        rhs[kj] = -2.0 * tw - muc;
    }
}

// The row values of a CG column pass: w_i = a_i (P u)_i / ma_i = a_i e_i / m_i.
__global__ void hvp_rows_cg_combine(const float *__restrict__ part_s, int S, int B, int n,
                                    int n_pad, const double *__restrict__ mrow,
                                    const float *__restrict__ a, float *__restrict__ wu)
{
    const int row = blockIdx.x * blockDim.x + threadIdx.x;
    const int b = blockIdx.y;
    if (row >= n)
        return;
    const size_t ri = (size_t)b * n + row;
    double e = 0.0;
    for (int s = 0; s < S; ++s)
        e += (double)part_s[((size_t)s * B + b) * n_pad + row];
    const double mr = mrow[ri];
    wu[(size_t)b * n_pad + row] = mr > 0.0 ? (float)(row_weight(a, ri, n) * e / mr) : 0.f;
}

// One wave per row: HV_i = (2/eps)(df_i D1_i + Du_i - 2 Tv_i) + 2 ma_i v_i with
// P dg = a e, Du = a (e x - W), df = (2 tv - P dg) / ma; NaN for a marked pair.
__global__ __launch_bounds__(256) void hvp_final_combine(
    const float *__restrict__ part_s, const float *__restrict__ part_v, int S, int B, int n,
    int n_pad, int d, const uint16_t *__restrict__ X, const float *__restrict__ a,
    const double *__restrict__ ma, const double *__restrict__ tv, const double *__restrict__ D1,
    const double *__restrict__ Tv, const float *__restrict__ V, const int *__restrict__ bad,
    double inv_eps, float *__restrict__ HV)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int k = lane_id();
    const int b = blockIdx.y;
    if (row >= n || k >= d)
        return;
    const size_t ri = (size_t)b * n + row;
    double e = 0.0, W = 0.0;
    for (int s = 0; s < S; ++s) {
        const size_t o = ((size_t)s * B + b) * n_pad + row;
        e += (double)part_s[o];
        W += (double)part_v[o * d + k];
    }
    const double ai = row_weight(a, ri, n);
    const double x = (double)bf16_to_float(X[ri * d + k]);
    const double pdg = ai * e;
    const double du = ai * (e * x - W);
    const double mai = ma[ri];
    const double df = mai > 0.0 ? (2.0 * tv[ri] - pdg) / mai : 0.0;
    const size_t o = ri * d + k;
    const double hv =
        2.0 * inv_eps * (df * D1[o] + du - 2.0 * Tv[o]) + 2.0 * mai * (double)V[o];
    HV[o] = bad[b] ? __builtin_nanf("") : (float)hv;
}

__global__ void zero_words(uint32_t *__restrict__ p, size_t count)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count)
        p[i] = 0u;
}

hipError_t zero(void *p, size_t bytes, hipStream_t st)
{
    const size_t words = bytes / 4;
    hipLaunchKernelGGL(zero_words, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st,
                       (uint32_t *)p, words);
    return hipGetLastError();
}

// the split of each pass; launches and combines take these
mc::Split rows_split(int G, int target, int B, int np, int mp)
{
    return mc::split_of(np / (kWavesH * 16 * G) * B, mp / kKeysH, target);
}

mc::Split cols_split(int G, int target, int B, int np, int mp)
{
    return mc::split_of(mp / (kWavesH * 16 * G) * B, np / kKeysH, target);
}

template <int MODE>
void rows_pass(const uint16_t *X, const uint16_t *Y, const HvpFeatWs &w, int d, int B, int n,
               int n_pad, int m, int m_pad, float two_c, const float *u, hipStream_t st)
{
    constexpr int G = MODE == kRowsCg ? kGroupsCg : MODE == kRowsFirst ? kGroupsRows1
                                                                       : kGroupsOther;
    const mc::Split sp = rows_split(G, MODE == kRowsCg ? kTargetCg : kTargetVec, B, n_pad, m_pad);
    dim3 grid(sp.S, n_pad / (kWavesH * 16 * G), B), block(kWavesH * kWave);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, st, X, (const float *)w.h, n, n_pad, Y,
                           (const uint16_t *)w.yt, (const float *)w.y.bias, m, m_pad,
                           (const uint16_t *)w.vh, (const uint16_t *)w.vl, u, two_c, sp.tps,
                           w.part_r, w.part_rv, w.part_rq);
    };
    constexpr int NT = MODE == kRowsCg ? kTilesCg : kTilesVec;
    if (d == 32)
        go(mc::rows_kernel<1, G, NT, MODE>);
    else
        go(mc::rows_kernel<2, G, NT, MODE>);
}

template <int MODE>
void cols_pass(const uint16_t *X, const uint16_t *Y, const HvpFeatWs &w, int d, int B, int n,
               int n_pad, int m, int m_pad, float two_c, const float *w0, hipStream_t st)
{
    constexpr int G = MODE == kColsCg ? kGroupsCg : kGroupsOther;
    const mc::Split sp = cols_split(G, MODE == kColsCg ? kTargetCg : kTargetVec, B, n_pad, m_pad);
    dim3 grid(sp.S, m_pad / (kWavesH * 16 * G), B), block(kWavesH * kWave);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, st, X, (const float *)w.h, n, n_pad, Y,
                           (const float *)w.y.bias, m, m_pad, w0, (const float *)w.wu,
                           (const float *)w.wt, (const uint16_t *)w.vth, (const uint16_t *)w.vtl,
                           two_c, sp.tps, w.part_c, w.part_cv);
    };
    constexpr int NT = MODE == kColsCg ? kTilesCg : kTilesVec;
    if (d == 32)
        go(hvp_cols_kernel<1, G, NT, MODE>);
    else
        go(hvp_cols_kernel<2, G, NT, MODE>);
}

}  // namespace

bool hvp_matrix_cores(int dtype, int d) { return dtype == 1 && (d == 32 || d == 64); }

HvpFeatSizes hvp_feat_sizes(int B, int n, int m, int d)
{
    const int np = round_up(n, kHvpPad), mp = round_up(m, kHvpPad);
    const int r_cg = rows_split(kGroupsCg, kTargetCg, B, np, mp).S;
    const int r_1 = rows_split(kGroupsRows1, kTargetVec, B, np, mp).S;
    const int r_f = rows_split(kGroupsOther, kTargetVec, B, np, mp).S;
    const int c_cg = cols_split(kGroupsCg, kTargetCg, B, np, mp).S;
    const int c_1 = cols_split(kGroupsOther, kTargetVec, B, np, mp).S;
    HvpFeatSizes z;
    z.part_r = (size_t)std::max({r_cg, r_1, r_f}) * B * np;
    z.part_rv = (size_t)std::max(r_1, r_f) * B * np * d;
    z.part_c = (size_t)std::max(c_cg, 3 * c_1) * B * mp;
    z.part_cv = (size_t)c_1 * B * mp * d;
    return z;
}

hipError_t launch_hvp_feat(const void *X_, const void *Y_, const float *a, const float *b,
                           const float *f, const float *g, const float *V, int B, int n, int m,
                           int d, float eps, int cg_iters, float *HV, float *cg_residual,
                           const HvpFeatWs &w, hipStream_t st)
{
    const uint16_t *X = (const uint16_t *)X_, *Y = (const uint16_t *)Y_;
    const int np = round_up(n, kHvpPad), mp = round_up(m, kHvpPad);
    const float c = scale_of(eps);
    const float two_c = 2.0f * c;
    hipError_t e;
    // keys: beta_j at eps (the potentials are only read) and the transposed points
    SideF sy = w.y;
    sy.pot = const_cast<float *>(g);
    if ((e = launch_packF(Y, 1, d, b, 1, B, sy, (double)c, st)) ||
        (e = launch_transpose_bf16(Y, B, m, mp, d, w.yt, st)))
        return e;
    if ((e = zero(w.u32, (size_t)B * mp * sizeof(float), st)) ||
        (e = zero(w.x32, (size_t)B * mp * sizeof(float), st)) ||
        (e = zero(w.bad, (size_t)B * sizeof(int), st)))
        return e;
    hipLaunchKernelGGL(hvp_prep_rows, dim3(np / 4, B), dim3(256), 0, st, X, a, f, V, n, np, d,
                       w.h, w.wa, w.wu, w.wt, w.vh, w.vl);
    if ((e = hipGetLastError()) || (e = launch_transpose_bf16(w.vh, B, np, np, d, w.vth, st)) ||
        (e = launch_transpose_bf16(w.vl, B, np, np, d, w.vtl, st)))
        return e;

    // first row pass: m, O, Q -> ma, D1, tv, Tv, and the column pass's row values
    rows_pass<kRowsFirst>(X, Y, w, d, B, n, np, m, mp, two_c, nullptr, st);
    {
        const int S = rows_split(kGroupsRows1, kTargetVec, B, np, mp).S;
        hipLaunchKernelGGL(hvp_rows_first_combine, dim3(ceil_div(n, 4), B), dim3(256), 0, st,
                           (const float *)w.part_r, (const float *)w.part_rv,
                           (const float *)w.part_rq, S, B, n, np, d, X, a,
                           (const uint16_t *)w.vh, (const uint16_t *)w.vl, w.mrow, w.ma, w.tv,
                           w.D1, w.Tv, w.wu, w.wt, w.bad);
    }
    // first column pass: mb, P^T ur, sum a t E, PV -> rhs
    cols_pass<kColsFirst>(X, Y, w, d, B, n, np, m, mp, two_c, w.wa, st);
    {
        const int S = cols_split(kGroupsOther, kTargetVec, B, np, mp).S;
        hipLaunchKernelGGL(hvp_cols_first_combine, dim3(ceil_div(m, 4), B), dim3(256), 0, st,
                           (const float *)w.part_c, (const float *)w.part_cv, S, B, m, mp, d, Y,
                           w.mb, w.rhs);
    }
    if ((e = hipGetLastError()) ||
        (e = launch_cg_start(w.rhs, B, m, w.x, w.res, w.dir, w.rr, w.rr0, w.x32, w.u32, mp, true,
                             st)))
        return e;
    const int s_rows = rows_split(kGroupsCg, kTargetCg, B, np, mp).S;
    const int s_cols = cols_split(kGroupsCg, kTargetCg, B, np, mp).S;
    for (int it = 0; it < cg_iters; ++it) {
        // q2 = P^T ((P dir) / ma): e = sum_j E dir_j, w = a e / m, then sum_i w_i E_ij
        rows_pass<kRowsCg>(X, Y, w, d, B, n, np, m, mp, two_c, w.u32, st);
        hipLaunchKernelGGL(hvp_rows_cg_combine, dim3(ceil_div(n, 256), B), dim3(256), 0, st,
                           (const float *)w.part_r, s_rows, B, n, np, (const double *)w.mrow, a,
                           w.wu);
        cols_pass<kColsCg>(X, Y, w, d, B, n, np, m, mp, two_c, w.wu, st);
        const double *rr_cur = w.rr + (size_t)(it & 1) * B;
        double *rr_next = w.rr + (size_t)((it + 1) & 1) * B;
        if ((e = launch_cg_step_wide(w.mb, w.part_c, s_cols, mp, B, m, w.x, w.res, w.dir, w.rhs,
                                     rr_cur, rr_next, w.rr0, kCgStop * kCgStop, true, w.red_pq,
                                     w.red_s, w.red_q, w.x32, w.u32, st)))
            return e;
    }
    // final row pass with u = dg: P dg and Du -> HV
    rows_pass<kRowsFinal>(X, Y, w, d, B, n, np, m, mp, two_c, w.x32, st);
    {
        const int S = rows_split(kGroupsOther, kTargetVec, B, np, mp).S;
        hipLaunchKernelGGL(hvp_final_combine, dim3(ceil_div(n, 4), B), dim3(256), 0, st,
                           (const float *)w.part_r, (const float *)w.part_rv, S, B, n, np, d, X,
                           a, (const double *)w.ma, (const double *)w.tv, (const double *)w.D1,
                           (const double *)w.Tv, V, (const int *)w.bad, 1.0 / (double)eps, HV);
    }
    if ((e = hipGetLastError()))
        return e;
    if (cg_residual)
        return launch_cg_report(w.rr + (size_t)(cg_iters & 1) * B, w.rr0, w.bad, B, cg_residual,
                                st);
    return hipSuccess;
}

}  // namespace sk

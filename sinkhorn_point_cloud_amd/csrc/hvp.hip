// hvp.hip -- streaming Hessian-vector product of the entropic OT value in X
// (FlashSinkhorn summary, Methodologie 3, Hessiaan-Vector Producten: the HVP
// as a sequence of transport-vector and transport-matrix products, working
// memory O((n + m) d), neither the Hessian nor the plan stored).
//
// With the plan P of potentials f, g at eps (row sums ma, column sums mb) and a
// direction V [n][d], dC_ij = 2 (x_i - y_j) . v_i and
//     r_i = sum_j P_ij dC_ij = 2 tv_i,       c_j = sum_i P_ij dC_ij,
// the potentials' derivatives solve (marginals held fixed)
//     ma_i df_i + (P dg)_i = r_i,   (P^T df)_j + mb_j dg_j = c_j,
// i.e. S dg = rhs with S = diag(mb) - P^T diag(1/ma) P (symmetric, positive
// semidefinite, null space the constants) and rhs = c - P^T (r / ma), solved by
// conjugate gradients from dg = 0 (which stays orthogonal to the null space);
// then df = (r - P dg) / ma and
//     HV_i = (2/eps) (df_i D1_i + Du_i - 2 Tv_i) + 2 ma_i v_i,
// with D1_i = sum_j P_ij (x_i - y_j), Du_i = sum_j P_ij dg_j (x_i - y_j) and
// Tv_i = sum_j P_ij ((x_i - y_j) . v_i)(x_i - y_j).
//
// Every sum over the plan is one streaming pass (transport_pass): one row per
// lane, keys read with wave-uniform loads, log P in fp64 as in the other plan
// passes; the four waves of a work-group split the keys and merge in LDS in a
// fixed order.  Conjugate-gradient vectors and dot products are fp64; one
// work-group per pair reduces in a fixed order.  Deterministic throughout.
// bf16 clouds with d = 32 or 64 take the matrix-core passes of hvp_feat.hip,
// which share the conjugate-gradient kernels below.
#include "hvp.h"
#include "plan_eval.h"

namespace sk {
namespace {

constexpr int kHvpWaves = 4;
constexpr int kHvpStage = 512;   // d = 3 key-side values staged in LDS per step
enum : int { F_V = 1, F_U = 2, F_W = 4, F_D = 8, F_M = 16 };

// Per row i of p.X against the keys of p.Y:
//   m0 = sum P (F_M);  mu = sum P u_j (F_U);  D1 = sum P (x - y), Du = sum P u_j (x - y) (F_D);
//   tv = sum P (x - y).v_i, Tv = sum P ((x - y).v_i)(x - y) (F_V);  tw = sum P (x - y).w_j (F_W).
template <typename T, int DP, int FL, bool KD>
__global__ __launch_bounds__(kHvpWaves *kWave) void transport_pass(
    PlanArgs p, const float *__restrict__ v, const double *__restrict__ u,
    const float *__restrict__ wk, double *__restrict__ o_m0, double *__restrict__ o_mu,
    double *__restrict__ o_tv, double *__restrict__ o_tw, double *__restrict__ o_D1,
    double *__restrict__ o_Du, double *__restrict__ o_Tv)
{
    __shared__ double red[kHvpWaves][kWave];
    const int b = blockIdx.y;
    const int w = wave_id_uniform();
    const int lane = lane_id();
    const int i = blockIdx.x * kWave + lane;
    const bool live = i < p.n;
    const int ic = live ? i : p.n - 1;
    RowCtx<DP> r;
    load_row<T, DP>(r, p, b, ic);
    double vi[DP];
#pragma unroll
    for (int k = 0; k < DP; ++k)
        vi[k] = (FL & F_V) && has_dim<DP>(k, p.d) ? (double)v[((size_t)b * p.n + ic) * p.d + k]
                                                  : 0.0;
    const T *Yb = (const T *)p.Y + (size_t)b * p.m * p.d;
    const float *gb = p.g + (size_t)b * p.m;
    const double *lbb = p.lb + (size_t)b * p.m;
    // d = 3: log P in the expanded form from KeyB records and the row's A_i
    const KeyB *kbb = KD ? p.kb + (size_t)b * p.m : nullptr;
    double xd[3] = {0.0, 0.0, 0.0}, A = 0.0;
    if constexpr (KD) {
#pragma unroll
        for (int k = 0; k < 3; ++k)
            xd[k] = (double)r.x[k];
        // base 2, as the records: log2 P ready for the exponential
        A = kLog2eD * side_term_d3(xd[0], xd[1], xd[2], r.f, r.la, p.inv_eps);
    }
    const double two_inv_eps = 2.0 * p.inv_eps * kLog2eD;
    double m0 = 0.0, mu = 0.0, tv = 0.0, tw = 0.0;
    double D1[DP], Du[DP], Tv[DP];
#pragma unroll
    for (int k = 0; k < DP; ++k)
        D1[k] = Du[k] = Tv[k] = 0.0;
    // d = 3: the key side's values (fp64 record, u_j, w_j) pass through LDS a
    // stage at a time and every lane of a wave reads the same key
    __shared__ KeyB kst[KD ? kHvpStage : 1];
    __shared__ double ust[KD && (FL & F_U) ? kHvpStage : 1];
    __shared__ float wst[KD && (FL & F_W) ? 3 * kHvpStage : 1];
    constexpr bool kNeedDiff = (FL & (F_D | F_V | F_W)) != 0;
    auto visit = [&](int j, int js) {
        double diff[DP];
        double lp;
        if constexpr (KD) {
            const KeyB kr = kst[js];
            const double y[3] = {kr.y[0], kr.y[1], kr.y[2]};
            lp = log_plan_b3(xd, A, y, kr.B, two_inv_eps);
            if constexpr (kNeedDiff) {
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    diff[k] = xd[k] - y[k];
            }
        } else {
            KeyVals<DP> kv;
            double C;
            load_key<T, DP, false>(kv, p, Yb, gb, nullptr, j);
            lp = log_plan_kv<DP>(r, kv, lbb[j], p.inv_eps, p.d, &C, diff);
        }
        const double P = (double)ex2((float)(KD ? lp : lp * kLog2eD));
        if (FL & F_M)
            m0 += P;
        double uj = 0.0;
        if (FL & F_U) {
            if constexpr (KD)
                uj = ust[js];
            else
                uj = u[(size_t)b * p.m + j];
            mu = fma(P, uj, mu);
        }
        if (FL & F_D) {
#pragma unroll
            for (int k = 0; k < DP; ++k) {
                D1[k] = fma(P, diff[k], D1[k]);
                if (FL & F_U)
                    Du[k] = fma(P * uj, diff[k], Du[k]);
            }
        }
        if (FL & F_V) {
            double dv = 0.0;
#pragma unroll
            for (int k = 0; k < DP; ++k)
                dv = fma(diff[k], vi[k], dv);
            tv = fma(P, dv, tv);
#pragma unroll
            for (int k = 0; k < DP; ++k)
                Tv[k] = fma(P * dv, diff[k], Tv[k]);
        }
        if (FL & F_W) {
            const float *wj = KD ? wst + 3 * js : wk + ((size_t)b * p.m + j) * p.d;
            double dw = 0.0;
#pragma unroll
            for (int k = 0; k < DP; ++k)
                if (has_dim<DP>(k, p.d))
                    dw = fma(diff[k], (double)wj[k], dw);
            tw = fma(P, dw, tw);
        }
    };
    if constexpr (KD) {
        for (int c0 = 0; c0 < p.m; c0 += kHvpStage) {
            const int kc = min(kHvpStage, p.m - c0);
            __syncthreads();   // the previous stage is no longer read
            for (int e = threadIdx.x; e < kc; e += kHvpWaves * kWave) {
                kst[e] = kbb[c0 + e];
                if constexpr ((FL & F_U) != 0)
                    ust[e] = u[(size_t)b * p.m + c0 + e];
                if constexpr ((FL & F_W) != 0) {
                    const float *wj = wk + ((size_t)b * p.m + c0 + e) * 3;
                    wst[3 * e] = wj[0];
                    wst[3 * e + 1] = wj[1];
                    wst[3 * e + 2] = wj[2];
                }
            }
            __syncthreads();
            int js = w;
            // four keys per step; the sums still take the keys in order
            for (; js + 3 * kHvpWaves < kc; js += 4 * kHvpWaves) {
                visit(c0 + js, js);
                visit(c0 + js + kHvpWaves, js + kHvpWaves);
                visit(c0 + js + 2 * kHvpWaves, js + 2 * kHvpWaves);
                visit(c0 + js + 3 * kHvpWaves, js + 3 * kHvpWaves);
            }
            for (; js < kc; js += kHvpWaves)
                visit(c0 + js, js);
        }
    } else {
        int j = w;
        if constexpr (DP <= 4) {
            // four keys per step, so that their loads are in flight together (the
            // sums still take the keys in order)
            for (; j + 3 * kHvpWaves < p.m; j += 4 * kHvpWaves) {
                visit(j, 0);
                visit(j + kHvpWaves, 0);
                visit(j + 2 * kHvpWaves, 0);
                visit(j + 3 * kHvpWaves, 0);
            }
        }
        for (; j < p.m; j += kHvpWaves)
            visit(j, 0);
    }
    // merge the waves' partial sums in a fixed order, one quantity at a time
    auto merged = [&](double val) {
        __syncthreads();
        red[w][lane] = val;
        __syncthreads();
        double s = red[0][lane];
#pragma unroll
        for (int v2 = 1; v2 < kHvpWaves; ++v2)
            s += red[v2][lane];
        return s;
    };
    const size_t ri = (size_t)b * p.n + i;
    if (FL & F_M) {
        const double s = merged(m0);
        if (w == 0 && live && o_m0)
            o_m0[ri] = s;
    }
    if (FL & F_U) {
        const double s = merged(mu);
        if (w == 0 && live && o_mu)
            o_mu[ri] = s;
    }
    if (FL & F_V) {
        const double s = merged(tv);
        if (w == 0 && live && o_tv)
            o_tv[ri] = s;
    }
    if (FL & F_W) {
        const double s = merged(tw);
        if (w == 0 && live && o_tw)
            o_tw[ri] = s;
    }
#pragma unroll
    for (int k = 0; k < DP; ++k) {
        if (!has_dim<DP>(k, p.d))   // uniform: every thread skips alike
            continue;
        if (FL & F_D) {
            const double s = merged(D1[k]);
            if (w == 0 && live && o_D1)
                o_D1[ri * p.d + k] = s;
            if (FL & F_U) {
                const double s2 = merged(Du[k]);
                if (w == 0 && live && o_Du)
                    o_Du[ri * p.d + k] = s2;
            }
        }
        if (FL & F_V) {
            const double s = merged(Tv[k]);
            if (w == 0 && live && o_Tv)
                o_Tv[ri * p.d + k] = s;
        }
    }
}

// out_i = num_i / den_i (0 where den_i = 0), times scale
__global__ void ratio_kernel(const double *__restrict__ num, const double *__restrict__ den,
                             size_t count, double scale, double *__restrict__ out)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count)
        out[i] = den[i] > 0.0 ? scale * num[i] / den[i] : 0.0;
}

// rhs_j = -2 tw_j - mu_j  (c_j = -2 tw_j when the pass ran with rows Y, keys X)
__global__ void rhs_kernel(const double *__restrict__ tw, const double *__restrict__ mu,
                           size_t count, double *__restrict__ rhs)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count)
        rhs[i] = -2.0 * tw[i] - mu[i];
}

__device__ double block_sum(double v, double *sm)
{
    const int t = threadIdx.x;
    sm[t] = v;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (t < s)
            sm[t] += sm[t + s];
        __syncthreads();
    }
    const double r = sm[0];
    __syncthreads();
    return r;
}

// x = 0, res = rhs, dir = rhs, rr = rr0 = |rhs|^2 (one work-group per pair);
// x32 / dir32 (if given, [B][m_pad]) receive fp32 copies of x and dir.  With
// project, rhs is first taken orthogonal to the constants (S's null space).
__global__ __launch_bounds__(256) void cg_start(const double *__restrict__ rhs, int m,
                                                double *__restrict__ x, double *__restrict__ res,
                                                double *__restrict__ dir, double *__restrict__ rr,
                                                double *__restrict__ rr0, float *__restrict__ x32,
                                                float *__restrict__ dir32, int m_pad, int project)
{
    __shared__ double sm[256];
    const int b = blockIdx.x;
    double mean = 0.0;
    if (project) {
        double acc = 0.0;
        for (int j = threadIdx.x; j < m; j += 256)
            acc += rhs[(size_t)b * m + j];
        mean = block_sum(acc, sm) / (double)m;
    }
    double acc = 0.0;
    for (int j = threadIdx.x; j < m; j += 256) {
        const size_t k = (size_t)b * m + j;
        const double v = rhs[k] - mean;
        x[k] = 0.0;
        res[k] = v;
        dir[k] = v;
        if (dir32) {
            x32[(size_t)b * m_pad + j] = 0.f;
            dir32[(size_t)b * m_pad + j] = (float)v;
        }
        acc = fma(v, v, acc);
    }
    const double s = block_sum(acc, sm);
    if (threadIdx.x == 0) {
        rr[b] = s;
        rr0[b] = s;
    }
}

// One conjugate-gradient step, with S dir = mb o dir - q2 (q2 = P^T((P dir)/ma)).
__global__ __launch_bounds__(256) void cg_step(const double *__restrict__ mb,
                                               const double *__restrict__ q2, int m,
                                               double *__restrict__ x, double *__restrict__ res,
                                               double *__restrict__ dir, double *__restrict__ rr)
{
    __shared__ double sm[256];
    const int b = blockIdx.x;
    double acc = 0.0;
    for (int j = threadIdx.x; j < m; j += 256) {
        const size_t k = (size_t)b * m + j;
        const double q = fma(mb[k], dir[k], -q2[k]);
        acc = fma(dir[k], q, acc);
    }
    const double pq = block_sum(acc, sm);
    const double rr_old = rr[b];
    const double alpha = pq > 0.0 ? rr_old / pq : 0.0;
    acc = 0.0;
    for (int j = threadIdx.x; j < m; j += 256) {
        const size_t k = (size_t)b * m + j;
        const double q = fma(mb[k], dir[k], -q2[k]);
        x[k] = fma(alpha, dir[k], x[k]);
        res[k] = fma(-alpha, q, res[k]);
        acc = fma(res[k], res[k], acc);
    }
    const double rr_new = block_sum(acc, sm);
    const double beta = rr_old > 0.0 ? rr_new / rr_old : 0.0;
    for (int j = threadIdx.x; j < m; j += 256) {
        const size_t k = (size_t)b * m + j;
        dir[k] = fma(beta, dir[k], res[k]);
    }
    if (threadIdx.x == 0)
        rr[b] = rr_new;
}

// Wide conjugate-gradient step: many work-groups per pair, kCgChunk entries each,
// three launches.  A work-group adds the others' partial sums itself, in block
// order, so every work-group holds the same value and results are
// deterministic.  rr holds two slots per pair: step k reads slot k % 2 and
// writes the other; a pair whose residual has reached stop2 rr0 is left alone
// (its slot is carried over).
constexpr int kCgChunk = 1024;

__device__ double sum_parts(const double *__restrict__ p, int count, double *sm)
{
    double a = 0.0;
    for (int k = threadIdx.x; k < count; k += 256)
        a += p[k];
    return block_sum(a, sm);
}

__device__ __forceinline__ bool cg_active(const double *rr_cur, const double *rr0, double stop2,
                                          int b)
{
    return rr_cur[b] > stop2 * rr0[b];
}

// q = mb o dir - q2 (q2 from S fp32 partials), and the blocks' dir.q
__global__ __launch_bounds__(256) void cg_wide_q(const double *__restrict__ mb,
                                                 const float *__restrict__ part, int S, int B,
                                                 int m, int m_pad, const double *__restrict__ dir,
                                                 double *__restrict__ q,
                                                 const double *__restrict__ rr_cur,
                                                 const double *__restrict__ rr0, double stop2,
                                                 double *__restrict__ red_pq)
{
    __shared__ double sm[256];
    const int b = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
    if (!cg_active(rr_cur, rr0, stop2, b))
        return;
    const int j1 = min(m, (blk + 1) * kCgChunk);
    double acc = 0.0;
    for (int j = blk * kCgChunk + threadIdx.x; j < j1; j += 256) {
        const size_t k = (size_t)b * m + j;
        double q2 = 0.0;
        for (int p = 0; p < S; ++p)
            q2 += (double)part[((size_t)p * B + b) * m_pad + j];
        const double v = fma(mb[k], dir[k], -q2);
        q[k] = v;
        acc = fma(dir[k], v, acc);
    }
    const double s = block_sum(acc, sm);
    if (threadIdx.x == 0)
        red_pq[(size_t)b * nblk + blk] = s;
}

// x += alpha dir, res -= alpha q; the blocks' sum and sum of squares of res
__global__ __launch_bounds__(256) void cg_wide_x(int m, double *__restrict__ x,
                                                 double *__restrict__ res,
                                                 const double *__restrict__ dir,
                                                 const double *__restrict__ q,
                                                 const double *__restrict__ rr_cur,
                                                 const double *__restrict__ rr0, double stop2,
                                                 const double *__restrict__ red_pq,
                                                 double *__restrict__ red_s,
                                                 double *__restrict__ red_q)
{
    __shared__ double sm[256];
    const int b = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
    if (!cg_active(rr_cur, rr0, stop2, b))
        return;
    const double pq = sum_parts(red_pq + (size_t)b * nblk, nblk, sm);
    const double alpha = pq > 0.0 ? rr_cur[b] / pq : 0.0;
    const int j1 = min(m, (blk + 1) * kCgChunk);
    double rs = 0.0, rq = 0.0;
    for (int j = blk * kCgChunk + threadIdx.x; j < j1; j += 256) {
        const size_t k = (size_t)b * m + j;
        x[k] = fma(alpha, dir[k], x[k]);
        const double r = fma(-alpha, q[k], res[k]);
        res[k] = r;
        rs += r;
        rq = fma(r, r, rq);
    }
    const double s1 = block_sum(rs, sm);
    const double s2 = block_sum(rq, sm);
    if (threadIdx.x == 0) {
        red_s[(size_t)b * nblk + blk] = s1;
        red_q[(size_t)b * nblk + blk] = s2;
    }
}

// res taken orthogonal to the constants (project), beta, dir = res + beta dir,
// fp32 copies of x and dir, and the next residual slot
__global__ __launch_bounds__(256) void cg_wide_dir(int m, int m_pad, int project,
                                                   const double *__restrict__ x,
                                                   double *__restrict__ res,
                                                   double *__restrict__ dir,
                                                   const double *__restrict__ rr_cur,
                                                   double *__restrict__ rr_next,
                                                   const double *__restrict__ rr0, double stop2,
                                                   const double *__restrict__ red_s,
                                                   const double *__restrict__ red_q,
                                                   float *__restrict__ x32,
                                                   float *__restrict__ dir32)
{
    __shared__ double sm[256];
    const int b = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
    const bool lead = blk == 0 && threadIdx.x == 0;
    if (!cg_active(rr_cur, rr0, stop2, b)) {
        if (lead)
            rr_next[b] = rr_cur[b];
        return;
    }
    const double rs = sum_parts(red_s + (size_t)b * nblk, nblk, sm);
    const double rq = sum_parts(red_q + (size_t)b * nblk, nblk, sm);
    const double mean = project ? rs / (double)m : 0.0;
    // sum (r - mean)^2 = sum r^2 - m mean^2
    const double rr_new = fmax(rq - (double)m * mean * mean, 0.0);
    const double beta = rr_cur[b] > 0.0 ? rr_new / rr_cur[b] : 0.0;
    const int j1 = min(m, (blk + 1) * kCgChunk);
    for (int j = blk * kCgChunk + threadIdx.x; j < j1; j += 256) {
        const size_t k = (size_t)b * m + j;
        const double r = res[k] - mean;
        res[k] = r;
        const double dn = fma(beta, dir[k], r);
        dir[k] = dn;
        x32[(size_t)b * m_pad + j] = (float)x[k];
        dir32[(size_t)b * m_pad + j] = (float)dn;
    }
    if (lead)
        rr_next[b] = rr_new;
}

// HV_i = (2/eps)(df_i D1_i + Du_i - 2 Tv_i) + 2 ma_i v_i,  df_i = (2 tv_i - (P dg)_i) / ma_i
__global__ void hv_kernel(const double *__restrict__ ma, const double *__restrict__ tv,
                          const double *__restrict__ pdg, const double *__restrict__ D1,
                          const double *__restrict__ Du, const double *__restrict__ Tv,
                          const float *__restrict__ V, size_t rows, int d, double inv_eps,
                          float *__restrict__ HV)
{
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= rows * d)
        return;
    const size_t i = e / d;
    const double df = ma[i] > 0.0 ? (2.0 * tv[i] - pdg[i]) / ma[i] : 0.0;
    const double h = 2.0 * inv_eps * (df * D1[e] + Du[e] - 2.0 * Tv[e]) + 2.0 * ma[i] * (double)V[e];
    HV[e] = (float)h;
}

// sqrt(rr / rr0) per pair; NaN for a pair marked in bad (if given)
__global__ void cg_report(const double *__restrict__ rr, const double *__restrict__ rr0,
                          const int *__restrict__ bad, int B, float *__restrict__ out)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B)
        out[b] = bad && bad[b] ? __builtin_nanf("")
                               : rr0[b] > 0.0 ? (float)sqrt(rr[b] / rr0[b]) : 0.f;
}

template <int FL>
void pass(const PlanArgs &p, const float *v, const double *u, const float *wk, double *m0,
          double *mu, double *tv, double *tw, double *D1, double *Du, double *Tv, hipStream_t st)
{
    dim3 grid(ceil_div(p.n, kWave), p.B), block(kHvpWaves * kWave);
    auto go = [&]<int DP, bool KD = false>() {
        if (p.dtype == 1)
            hipLaunchKernelGGL((transport_pass<uint16_t, DP, FL, KD>), grid, block, 0, st, p, v, u,
                               wk, m0, mu, tv, tw, D1, Du, Tv);
        else
            hipLaunchKernelGGL((transport_pass<float, DP, FL, KD>), grid, block, 0, st, p, v, u, wk,
                               m0, mu, tv, tw, D1, Du, Tv);
    };
    if (p.d == 3 && p.kb) go.template operator()<3, true>();
    else if (p.d == 3) go.template operator()<3>();
    else if (p.d <= 4) go.template operator()<4>();
    else if (p.d <= 8) go.template operator()<8>();
    else go.template operator()<16>();
}

unsigned blocks_for(size_t count) { return (unsigned)((count + 255) / 256); }

}  // namespace

hipError_t launch_hvp(const PlanArgs &px, const PlanArgs &py, const float *V, int cg_iters,
                      float *HV, float *cg_residual, const HvpWs &w, hipStream_t st)
{
    const int B = px.B, n = px.n, m = px.m, d = px.d;
    const size_t Bn = (size_t)B * n, Bm = (size_t)B * m;
    // rows X: ma, D1, tv, Tv
    pass<F_M | F_V | F_D>(px, V, nullptr, nullptr, w.ma, nullptr, w.tv, nullptr, w.D1, nullptr,
                          w.Tv, st);
    // u_i = r_i / ma_i = 2 tv_i / ma_i; rows Y (keys X carry v): mb, P^T u, tw
    hipLaunchKernelGGL(ratio_kernel, dim3(blocks_for(Bn)), dim3(256), 0, st,
                       (const double *)w.tv, (const double *)w.ma, Bn, 2.0, w.ur);
    pass<F_M | F_U | F_W>(py, nullptr, w.ur, V, w.mb, w.muc, nullptr, w.tw, nullptr, nullptr,
                          nullptr, st);
    hipLaunchKernelGGL(rhs_kernel, dim3(blocks_for(Bm)), dim3(256), 0, st, (const double *)w.tw,
                       (const double *)w.muc, Bm, w.rhs);
    hipLaunchKernelGGL(cg_start, dim3(B), dim3(256), 0, st, (const double *)w.rhs, m, w.x, w.res,
                       w.dir, w.rr, w.rr0, nullptr, nullptr, m, 0);
    for (int it = 0; it < cg_iters; ++it) {
        // q2 = P^T ((P dir) / ma)
        pass<F_U>(px, nullptr, w.dir, nullptr, nullptr, w.mur, nullptr, nullptr, nullptr,
                  nullptr, nullptr, st);
        hipLaunchKernelGGL(ratio_kernel, dim3(blocks_for(Bn)), dim3(256), 0, st,
                           (const double *)w.mur, (const double *)w.ma, Bn, 1.0, w.ur);
        pass<F_U>(py, nullptr, w.ur, nullptr, nullptr, w.muc, nullptr, nullptr, nullptr, nullptr,
                  nullptr, st);
        hipLaunchKernelGGL(cg_step, dim3(B), dim3(256), 0, st, (const double *)w.mb,
                           (const double *)w.muc, m, w.x, w.res, w.dir, w.rr);
    }
    // rows X with u = dg: P dg and Du
    // (D1 comes out bit-identical to the first pass's and is simply rewritten)
    pass<F_U | F_D>(px, nullptr, w.x, nullptr, nullptr, w.mur, nullptr, nullptr, w.D1, w.Du,
                    nullptr, st);
    hipLaunchKernelGGL(hv_kernel, dim3(blocks_for(Bn * d)), dim3(256), 0, st,
                       (const double *)w.ma, (const double *)w.tv, (const double *)w.mur,
                       (const double *)w.D1, (const double *)w.Du, (const double *)w.Tv, V, Bn, d,
                       px.inv_eps, HV);
    if (cg_residual)
        hipLaunchKernelGGL(cg_report, dim3(blocks_for(B)), dim3(256), 0, st, (const double *)w.rr,
                           (const double *)w.rr0, nullptr, B, cg_residual);
    return hipGetLastError();
}

hipError_t launch_cg_start(const double *rhs, int B, int m, double *x, double *res, double *dir,
                           double *rr, double *rr0, float *x32, float *dir32, int m_pad,
                           bool project, hipStream_t st)
{
    hipLaunchKernelGGL(cg_start, dim3(B), dim3(256), 0, st, rhs, m, x, res, dir, rr, rr0, x32,
                       dir32, m_pad, project ? 1 : 0);
    return hipGetLastError();
}

int cg_wide_blocks(int m) { return ceil_div(m, kCgChunk); }

hipError_t launch_cg_step_wide(const double *mb, const float *q2_part, int S, int m_pad, int B,
                               int m, double *x, double *res, double *dir, double *q,
                               const double *rr_cur, double *rr_next, const double *rr0,
                               double stop2, bool project, double *red_pq, double *red_s,
                               double *red_q, float *x32, float *dir32, hipStream_t st)
{
    const dim3 grid(cg_wide_blocks(m), B), block(256);
    hipLaunchKernelGGL(cg_wide_q, grid, block, 0, st, mb, q2_part, S, B, m, m_pad,
                       (const double *)dir, q, rr_cur, rr0, stop2, red_pq);
    hipLaunchKernelGGL(cg_wide_x, grid, block, 0, st, m, x, res, (const double *)dir,
                       (const double *)q, rr_cur, rr0, stop2, (const double *)red_pq, red_s,
                       red_q);
    hipLaunchKernelGGL(cg_wide_dir, grid, block, 0, st, m, m_pad, project ? 1 : 0,
                       (const double *)x, res, dir, rr_cur, rr_next, rr0, stop2,
                       (const double *)red_s, (const double *)red_q, x32, dir32);
    return hipGetLastError();
}

hipError_t launch_cg_report(const double *rr, const double *rr0, const int *bad, int B,
                            float *out, hipStream_t st)
{
    hipLaunchKernelGGL(cg_report, dim3(blocks_for(B)), dim3(256), 0, st, rr, rr0, bad, B, out);
    return hipGetLastError();
}

}  // namespace sk

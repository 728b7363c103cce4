// plan_eval.h -- per-entry evaluation of the transport plan at the final eps,
//     log P_ij = (f_i + g_j - C_ij)/eps + log a_i + log b_j,  C_ij = ||x_i - y_j||^2,
// in fp64 from the fp32 (or bf16) inputs, shared by the passes over the plan
// (cost, sparse plan, dense gradient, transport products of the Hessian-vector
// product) so that all of them see the same values; and the per-entry loss
// term shared by the loss pass and the emission of the sparse plan.
//
// Every pass reads a key (column j) as fp64 values: its point components and
// g_j, exact conversions of the inputs.  For d = 3 they come precomputed
// (KeyD, one 32-byte record per key, written by launch_keys_d3), so that a pass
// whose lanes share the key reads them whole (staged in LDS, or with scalar
// loads) and spends no vector instruction on conversions; otherwise they are
// converted where they are read.
// The values, and so every result, are the same either way.  For d = 3 the
// sparse plan's passes (max, count, emit), the dense gradient and the
// Hessian-vector product's transport passes instead take the expanded form of
// log P from KeyB records (log_plan_b3 below); only the cost pass, which needs
// C_ij itself, keeps the form above.
#pragma once
#include "common.h"

namespace sk {
namespace {

template <int DP> struct RowCtx {
    float x[DP];   // row point (exact fp32 value of the fp32 / bf16 input)
    double f, la;
};

// Whether component k exists: the DP = 3 instantiations serve d == 3 only, so
// their loops carry no run-time test; wider ones pad d up to DP.
template <int DP>
__device__ __forceinline__ bool has_dim(int k, int d)
{
    return DP == 3 || k < d;
}

// A key's point components and potential as fp64 (components past d are 0).
template <int DP> struct KeyVals {
    double y[DP];
    double g;
};

// Key j of one pair: from its KeyD record (KD: DP = 3 with records present; a
// compile-time choice, so that the loop around it has no branch) or converted
// from the inputs.
template <typename T, int DP, bool KD>
__device__ __forceinline__ void load_key(KeyVals<DP> &kv, const PlanArgs &p, const T *Yb,
                                         const float *gb, const KeyD *kdb, int j)
{
    if constexpr (KD) {
        static_assert(DP == 3, "KeyD records hold three components");
        const KeyD k = kdb[j];
        kv.y[0] = k.y[0];
        kv.y[1] = k.y[1];
        kv.y[2] = k.y[2];
        kv.g = k.g;
        return;
    }
    const T *yp = Yb + (size_t)j * p.d;
#pragma unroll
    for (int k = 0; k < DP; ++k)
        kv.y[k] = has_dim<DP>(k, p.d) ? (double)Elem<T>::get(yp, k) : 0.0;
    kv.g = (double)gb[j];
}

// log P_ij (nats) from the row context and the key's values; *C receives
// C_ij = sum_k (x_k - y_k)^2 (differences exact in fp64, summed with fma in
// component order).  Written with explicit fma so that every pass evaluates it
// with the same roundings, and symmetric in the two sides (f_i + g_j,
// (x - y)^2 = (y - x)^2 and log a_i + log b_j all round the same either way),
// so a pass over the plan with the roles of X and Y exchanged sees
// bit-identical values: the sparse plan of (Y, X) is exactly the transpose of
// that of (X, Y).  With diff != nullptr the differences x_k - y_k are returned
// too (callers with DP <= 16 only: they live in registers).
template <int DP>
__device__ __forceinline__ double log_plan_kv(const RowCtx<DP> &r, const KeyVals<DP> &kv,
                                              double lbj, double inv_eps, int d, double *C,
                                              double *diff = nullptr)
{
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < DP; ++k) {
        if (has_dim<DP>(k, d)) {
            const double t = (double)r.x[k] - kv.y[k];
            s = fma(t, t, s);
            if (diff)
                diff[k] = t;
        } else if (diff) {
            diff[k] = 0.0;
        }
    }
    *C = s;
    return fma((r.f + kv.g) - s, inv_eps, r.la + lbj);
}

// the same for column j of one pair, its components read from global memory
// one at a time (no per-entry array: for wide points)
template <typename T, int DP>
__device__ __forceinline__ double log_plan(const RowCtx<DP> &r, const PlanArgs &p,
                                           const T *Yb, const float *gb, double lbj, int j,
                                           double *C)
{
    const T *yp = Yb + (size_t)j * p.d;
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < DP; ++k) {
        if (has_dim<DP>(k, p.d)) {
            const double t = (double)r.x[k] - (double)Elem<T>::get(yp, k);
            s = fma(t, t, s);
        }
    }
    *C = s;
    return fma((r.f + (double)gb[j]) - s, p.inv_eps, r.la + lbj);
}

// log P for d = 3 in the expanded form
//     log P_ij = (2/eps) x_i . y_j + A_i + B_j,
//     A_i = (f_i - ||x_i||^2)/eps + log a_i,   B_j = (g_j - ||y_j||^2)/eps + log b_j,
// five fp64 operations per entry instead of the ten of log_plan_kv.  Both
// sides' constant terms come from side_term_d3 and the three products of the
// dot product are exact in fp64 and summed with fma in component order, so the
// value is the same with the roles of X and Y exchanged (the plan of (Y, X) is
// exactly the transpose).  Its rounding differs from log_plan_kv's by a few
// units in the last place of the larger terms, which only moves threshold
// decisions of entries at the threshold to within that.
__device__ __forceinline__ double side_term_d3(double v0, double v1, double v2, double pot,
                                               double lw, double inv_eps)
{
    const double sq = fma(v0, v0, fma(v1, v1, v2 * v2));
    return fma(pot - sq, inv_eps, lw);
}

__device__ __forceinline__ double log_plan_b3(const double (&x)[3], double A,
                                              const double (&y)[3], double B, double two_inv_eps)
{
    const double dot = fma(x[0], y[0], fma(x[1], y[1], x[2] * y[2]));
    return fma(dot, two_inv_eps, A + B);
}

// Points up to this width keep a key's values (and differences) in registers;
// wider ones stream their components.
constexpr int kKeyRegDims = 16;

// One stored entry's share of the transport loss and of its gradient in x:
//     loss += P ||x - y||^2,   gr += 2 P (x - y)
// from the exact fp64 differences diff = x - y and their squared norm C (as
// log_plan_kv returns them); the gradient accumulates in fp32.  The loss pass
// over a stored plan and the emission that computes the loss on the fly both
// call this, so they agree per entry (only the summation order differs).
template <int DP>
__device__ __forceinline__ void loss_term(const double (&diff)[DP], double C, int d, float P,
                                          double &loss, float (&gr)[DP])
{
#pragma unroll
    for (int c = 0; c < DP; ++c)
        if (has_dim<DP>(c, d))
            gr[c] = fmaf(2.0f * P, (float)diff[c], gr[c]);
    loss = fma((double)P, C, loss);
}

// The same from the row point and the key's point components (fp32 values),
// for callers without the differences at hand: identical per-entry arithmetic
// (each difference exact in fp64, squares summed with fma in component order).
template <int DP>
__device__ __forceinline__ void loss_term_xy(const float (&x)[DP], const float (&y)[DP], int d,
                                             float P, double &loss, float (&gr)[DP])
{
    double s = 0.0;
#pragma unroll
    for (int c = 0; c < DP; ++c) {
        if (has_dim<DP>(c, d)) {
            const double t = (double)x[c] - (double)y[c];
            s = fma(t, t, s);
            gr[c] = fmaf(2.0f * P, (float)t, gr[c]);
        }
    }
    loss = fma((double)P, s, loss);
}

// The same with the key's components read from memory one at a time (no
// per-entry array, for wide points).
template <typename T, int DP>
__device__ __forceinline__ void loss_term_at(const float (&x)[DP], const T *yp, int d, float P,
                                             double &loss, float (&gr)[DP])
{
    double s = 0.0;
#pragma unroll
    for (int c = 0; c < DP; ++c) {
        if (has_dim<DP>(c, d)) {
            const double t = (double)x[c] - (double)Elem<T>::get(yp, c);
            s = fma(t, t, s);
            gr[c] = fmaf(2.0f * P, (float)t, gr[c]);
        }
    }
    loss = fma((double)P, s, loss);
}

template <typename T, int DP>
__device__ void load_row(RowCtx<DP> &r, const PlanArgs &p, int b, int i)
{
    const T *x = (const T *)p.X + ((size_t)b * p.n + i) * p.d;
#pragma unroll
    for (int k = 0; k < DP; ++k)
        r.x[k] = has_dim<DP>(k, p.d) ? Elem<T>::get(x, k) : 0.f;
    r.f = (double)p.f[(size_t)b * p.n + i];
    r.la = p.la[(size_t)b * p.n + i];
}

}  // namespace
}  // namespace sk

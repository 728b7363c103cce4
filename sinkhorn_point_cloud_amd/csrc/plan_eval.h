// plan_eval.h -- per-entry evaluation of the transport plan at the final eps,
//     log P_ij = (f_i + g_j - C_ij)/eps + log a_i + log b_j,  C_ij = ||x_i - y_j||^2,
// in fp64 from the fp32 (or bf16) inputs, shared by the passes over the plan
// (cost, sparse plan, dense gradient, transport products of the Hessian-vector
// product) so that all of them see the same values; and the per-entry loss
// term shared by the loss pass and the emission of the sparse plan.
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

// ||x - y||^2 in fp64 from the fp32 components (exact conversions), in
// component order
template <int DP>
__device__ __forceinline__ double sq_dist(const float (&x)[DP], const float (&y)[DP], int d)
{
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < DP; ++k) {
        if (has_dim<DP>(k, d)) {
            const double t = (double)x[k] - (double)y[k];
            s = fma(t, t, s);
        }
    }
    return s;
}

// log P_ij (nats) and C_ij from the row context and the column's values (its
// point's components as fp32, g_j, log b_j).  Written with explicit fma so
// that every pass evaluates it with the same roundings, and symmetric in the
// two sides (f_i + g_j, (x - y)^2 = (y - x)^2 and log a_i + log b_j all round
// the same either way), so a pass over the plan with the roles of X and Y
// exchanged sees bit-identical values: the sparse plan of (Y, X) is exactly
// the transpose of that of (X, Y).
template <int DP>
__device__ __forceinline__ double log_plan_at(const RowCtx<DP> &r, const float (&y)[DP], float gj,
                                              double lbj, double inv_eps, int d, double *C)
{
    const double c = sq_dist<DP>(r.x, y, d);
    *C = c;
    return fma((r.f + (double)gj) - c, inv_eps, r.la + lbj);
}

// the same for column j of one pair, read from global memory
template <typename T, int DP>
__device__ __forceinline__ double log_plan(const RowCtx<DP> &r, const PlanArgs &p,
                                           const T *Yb, const float *gb, double lbj, int j,
                                           double *C)
{
    const T *yp = Yb + (size_t)j * p.d;
    float y[DP];
#pragma unroll
    for (int k = 0; k < DP; ++k)
        y[k] = has_dim<DP>(k, p.d) ? Elem<T>::get(yp, k) : 0.f;
    return log_plan_at<DP>(r, y, gb[j], lbj, p.inv_eps, p.d, C);
}

// One stored entry's share of the transport loss and of its gradient in x:
//     loss += P ||x - y||^2,   gr += 2 P (x - y)
// with x - y formed in fp32 and the squared distance summed in fp64.  The loss
// pass over a stored plan and the emission that computes the loss on the fly
// both call this, so they agree per entry (only the summation order differs).
template <int DP>
__device__ __forceinline__ void loss_term(const float (&x)[DP], const float (&y)[DP], int d,
                                          float P, double &loss, float (&gr)[DP])
{
    double C = 0.0;
#pragma unroll
    for (int c = 0; c < DP; ++c) {
        if (has_dim<DP>(c, d)) {
            const float t = x[c] - y[c];
            C = fma((double)t, (double)t, C);
            gr[c] = fmaf(2.0f * P, t, gr[c]);
        }
    }
    loss = fma((double)P, C, loss);
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

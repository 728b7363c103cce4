// plan_eval.h -- per-entry evaluation of the transport plan at the final eps,
//     log P_ij = (f_i + g_j - C_ij)/eps + log a_i + log b_j,  C_ij = ||x_i - y_j||^2,
// in fp64 from the fp32 (or bf16) inputs, shared by the passes over the plan
// (cost, sparse plan, dense gradient, transport products of the Hessian-vector
// product) so that all of them see the same values.
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

template <typename T, int DP>
__device__ __forceinline__ double sq_dist(const float (&x)[DP], const T *y, int d)
{
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < DP; ++k) {
        if (has_dim<DP>(k, d)) {
            const double t = (double)x[k] - (double)Elem<T>::get(y, k);
            s = fma(t, t, s);
        }
    }
    return s;
}

// log P_ij (nats) and C_ij for a row context and column j of one pair.  Written
// with explicit fma so that every pass evaluates it with the same roundings,
// and symmetric in the two sides (f_i + g_j, (x - y)^2 = (y - x)^2 and
// log a_i + log b_j all round the same either way), so a pass over the plan
// with the roles of X and Y exchanged sees bit-identical values: the sparse
// plan of (Y, X) is exactly the transpose of that of (X, Y).
template <typename T, int DP>
__device__ __forceinline__ double log_plan(const RowCtx<DP> &r, const PlanArgs &p,
                                           const T *Yb, const float *gb, double lbj, int j,
                                           double *C)
{
    const double c = sq_dist<T, DP>(r.x, Yb + (size_t)j * p.d, p.d);
    *C = c;
    return fma((r.f + (double)gb[j]) - c, p.inv_eps, r.la + lbj);
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

// hvp.h -- launchers of the Hessian-vector product's matrix-core path and the
// conjugate-gradient kernels it shares with the fp64 path (hvp.hip).
#pragma once

#include "common.h"

namespace sk {

// Conjugate-gradient start (one work-group per pair, fp64): with x32 / dir32
// ([B][m_pad]) it also writes fp32 copies of x and dir, and with project it takes
// the right-hand side orthogonal to the constants.  cg_report gives sqrt(rr/rr0)
// per pair, NaN for a pair marked in bad (if given).
hipError_t launch_cg_start(const double *rhs, int B, int m, double *x, double *res, double *dir,
                           double *rr, double *rr0, float *x32, float *dir32, int m_pad,
                           bool project, hipStream_t st);
hipError_t launch_cg_report(const double *rr, const double *rr0, const int *bad, int B,
                            float *out, hipStream_t st);
// The CG step spread over cg_wide_blocks(m) work-groups per pair (three
// launches), for q2 as S fp32 partials: q [B][m] scratch, red_* [B][blocks]
// scratch; reads rr_cur [B], writes rr_next [B].
int cg_wide_blocks(int m);
hipError_t launch_cg_step_wide(const double *mb, const float *q2_part, int S, int m_pad, int B,
                               int m, double *x, double *res, double *dir, double *q,
                               const double *rr_cur, double *rr_next, const double *rr0,
                               double stop2, bool project, double *red_pq, double *red_s,
                               double *red_q, float *x32, float *dir32, hipStream_t st);
// The same product on the matrix cores for bf16 with d = 32 or 64 (X, Y 16-byte
// aligned).  Point counts are padded to kHvpPad there.
constexpr int kHvpPad = 512;
bool hvp_matrix_cores(int dtype, int d);
struct HvpFeatSizes {
    size_t part_r, part_rv, part_c, part_cv;   // floats of the partial-sum buffers
};
HvpFeatSizes hvp_feat_sizes(int B, int n, int m, int d);
struct HvpFeatWs {
    SideF y;                          // keys: biases at eps, squared norms, log weights
    uint16_t *yt;                     // [B][d][m_pad] transposed key points
    float *h, *wa, *wu, *wt;          // [B][n_pad] row offsets and row values
    uint16_t *vh, *vl;                // [B][n_pad][d] the direction in two bf16 pieces
    uint16_t *vth, *vtl;              // [B][d][n_pad] the same, transposed
    float *u32, *x32;                 // [B][m_pad] fp32 key vectors (dir, dg)
    float *part_r, *part_rv, *part_rq;   // row-pass partial sums
    float *part_c, *part_cv;             // column-pass partial sums
    double *mrow, *ma, *tv, *D1, *Tv;    // [B][n], [B][n][d]
    double *mb, *rhs, *x, *res, *dir;    // [B][m] (rhs doubles as the CG step's q)
    double *rr, *rr0;                    // [2][B], [B]
    double *red_pq, *red_s, *red_q;      // [B][cg_wide_blocks(m)]
    int *bad;                            // [B] pairs outside the path's range
};
hipError_t launch_hvp_feat(const void *X, const void *Y, const float *a, const float *b,
                           const float *f, const float *g, const float *V, int B, int n, int m,
                           int d, float eps, int cg_iters, float *HV, float *cg_residual,
                           const HvpFeatWs &w, hipStream_t st);
}  // namespace sk

// common.h -- device helpers and launcher declarations shared by the HIP
// sources of the streaming Sinkhorn library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sk {

constexpr int kWave = 64;

// Stand-in for log 0 = -inf.  A finite value keeps every subtraction of two
// "minus infinities" finite (no NaN), while 2^(kNeg + anything sane) is 0.
constexpr float kNeg = -1.0e30f;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr double kLog2eD = 1.4426950408889634;
constexpr double kLn2D = 0.6931471805599453;

// c = log2(e)/eps rounded to fp32 once; every use of c (scores, biases, the
// conversion of a row's log-sum-exp back to a potential) takes this value.
inline float scale_of(float eps) { return (float)(kLog2eD / (double)eps); }

// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ int wave_id_uniform()
{
    return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ double wave_max(double v)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        v = fmax(v, __shfl_xor(v, off, kWave));
    return v;
}

// Merge of two partial log-sum-exp states (M, S), meaning S * 2^M.
__device__ __forceinline__ void lse_merge(float &M, float &S, float M2, float S2)
{
    float Mn = fmaxf(M, M2);
    S = S * ex2(M - Mn) + S2 * ex2(M2 - Mn);
    M = Mn;
}

// Reductions over each row of 16 lanes with DPP lane moves (no LDS traffic).
// The four moves pair lanes i^1, i^2 (quad permutes), then 7-i within each
// half row and 15-i within the row; after the four steps every lane of a row
// holds the row's result.  All 64 lanes must be active.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

template <int Ctrl>
__device__ __forceinline__ float dpp_move(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), Ctrl, 0xF, 0xF, true));
}

__device__ __forceinline__ float row16_sum(float v)
{
    v += dpp_move<kDppXor1>(v);
    v += dpp_move<kDppXor2>(v);
    v += dpp_move<kDppHalfMirror>(v);
    v += dpp_move<kDppMirror>(v);
    return v;
}

__device__ __forceinline__ void row16_merge(float &M, float &S)
{
    lse_merge(M, S, dpp_move<kDppXor1>(M), dpp_move<kDppXor1>(S));
    lse_merge(M, S, dpp_move<kDppXor2>(M), dpp_move<kDppXor2>(S));
    lse_merge(M, S, dpp_move<kDppHalfMirror>(M), dpp_move<kDppHalfMirror>(S));
    lse_merge(M, S, dpp_move<kDppMirror>(M), dpp_move<kDppMirror>(S));
}

__device__ __forceinline__ float bf16_to_float(uint16_t h)
{
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Element access for the two point dtypes.
template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float get(const float *p, size_t i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
    __device__ __forceinline__ static float get(const uint16_t *p, size_t i)
    {
        return bf16_to_float(p[i]);
    }
};

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline int round_up(int a, int b) { return ceil_div(a, b) * b; }

// ---------------------------------------------------------------- launchers
// Every launcher enqueues on `stream` and returns hipGetLastError().

// Points of one side packed for the d = 3 streaming kernel: (x, y, z, bias).
struct Side3 {
    float4 *pts;      // [B][n_pad] (x, y, z, bias for the opposite pass)
    float *pot;       // [B][n]     potential of this side (the state; in/out)
    float *l2w;       // [B][n]     log2 of the weights (kNeg for 0)
    uint16_t *krec;   // [B][n_pad][32] bf16 key records (matrix-core path)
    uint16_t *qrec;   // [B][n_pad][32] bf16 query records at the current eps
    int n, n_pad;
    int *redo = nullptr;   // [B][n_pad / 64] row blocks to recompute after a split merge
    // [B][n_pad] (tag, bias) words of the split stage launch, zeroed by the
    // query-record kernel of each stage (nullptr: that path is not used)
    uint64_t *xch = nullptr;
};
constexpr int kRec = 32;  // bf16 slots per record (one 16x16x32 MFMA k-range)

// Query records of one side for the scale of eps (rebuilt when eps changes);
// also zeroes s.xch when it is set.
hipError_t launch_qrec3(Side3 s, int B, float eps, hipStream_t st);
// Whole stages per pair in one launch (matrix-core scores): used when the batch
// has at least as many pairs as the device has compute units and each cloud has
// at most kPairMaxPoints points (padded).  Runs `iters` iterations at eps; the
// last g-update hands the f-update biases at eps_next.  cold: the potentials
// are the zeros of a cold start (the first f- and g-update take exact shifts).
constexpr int kPairMaxPoints = 8192;
bool lse3_pairwise(int B, int n_pad, int m_pad);
hipError_t launch_lse3_pairwise(Side3 x, Side3 y, int B, float eps, int iters, float eps_next,
                                bool cold, hipStream_t st);
// Whole stages of a small batch of pairs of at most 1024 points (padded), each
// pair split over work-groups of 16 rows per side, in one launch: used when the
// batch's work-groups fit on half of the compute units.  Returns the
// work-groups per pair, or 0 where the path does not apply.  The launch needs
// x.xch and y.xch, zeroed since the last launch (launch_qrec3 does it).  Its
// waits are bounded: a pair whose wait ran out gets NaN potentials.
int lse3_split_parts(int B, int n_pad, int m_pad);
hipError_t launch_lse3_split(Side3 x, Side3 y, int B, int parts, float eps, int iters,
                             float eps_next, bool cold, hipStream_t st);
// Wall-clock limit of each wait of the split stage launch, in microseconds, for
// the launches that follow (process-wide; below 0: every wait fails at once);
// returns the previous limit.
long long lse3_split_set_wait_us(long long us);

// Per-pair center (bounding-box midpoint of both clouds) for the d = 3 path;
// part holds center3_parts(n, m) * B partial boxes.
int center3_parts(int n, int m);
hipError_t launch_center3(const void *X, int dtype, int n, const void *Y, int m, int B,
                          float4 *part, float4 *center, hipStream_t st);
// Packs points relative to the pair's center, and the initial bias; without
// warm start the potential is set to 0.
hipError_t launch_pack3(const void *X, int dtype, const float *w, int warm, int B, Side3 s,
                        const float4 *center, double c0, hipStream_t st);
// One half-iteration, d = 3: q side rows, k side columns; scores on the matrix
// cores (mfma) or on the vector ALUs.
hipError_t launch_lse3(Side3 q, Side3 k, int B, float eps, float eps_next, float2 *part,
                       bool mfma, hipStream_t st);
size_t lse3_partial_floats2(int B, int nq_pad, int nk_pad);

// Generic-d feature path (fp32 or bf16 points, VALU).
struct SideF {
    const void *pts;  // [B][n][d] original points (fp32 or bf16)
    float *bias;      // [B][n_pad] bias for the opposite pass
    float *pot;       // [B][n] potential of this side (the state; in/out)
    float *l2w;       // [B][n]
    float *sq;        // [B][n] squared norms of the points
    int *redo;        // [B][n_pad / 64] per-row-block fallback flags (matrix-core path)
    int n, n_pad;
};
hipError_t launch_packF(const void *X, int dtype, int d, const float *w, int warm, int B,
                        SideF s, double c0, hipStream_t st);
hipError_t launch_lseF(SideF q, SideF k, int dtype, int d, int B, float eps, float eps_next,
                       float2 *part, hipStream_t st);
size_t lseF_partial_floats2(int B, int nq_pad, int nk_pad);
bool lseF_supported(int dtype, int d);
// true when both passes of this shape run on the matrix-core kernel
bool lseF_matrix_cores(SideF q, SideF k, int dtype, int d, int B);
// transport cost rows for the matrix-core feature path, from the biases of the
// final passes (which must have run at eps)
hipError_t launch_costFm(SideF x, SideF y, int d, int B, float eps, double *row_part,
                         hipStream_t st);
hipError_t launch_row_sums(const double *row_part, int B, int n, float *out, hipStream_t st);

// One key of a d = 3 plan pass as fp64: point components and potential (exact
// conversions of the inputs), 32 bytes.
struct alignas(32) KeyD {
    double y[3];
    double g;
};

// One key of the d = 3 passes that evaluate log P in the expanded form (sparse
// plan, dense gradient, Hessian-vector product) as fp64: point components and
// B_j = (g_j - ||y_j||^2)/eps + log b_j, 32 bytes.  With the row's
// A_i = (f_i - ||x_i||^2)/eps + log a_i they give
//     log P_ij = (2/eps) x_i . y_j + A_i + B_j.
// The dense gradient's and the Hessian-vector product's records (and row terms)
// carry these in base 2, ready for the exponential: B_j log2 e.
struct alignas(32) KeyB {
    double y[3];
    double B;
};

// Plan evaluation passes, shared by the cost, max, count and emit steps.
struct PlanArgs {
    const void *X, *Y;
    int dtype, d, B, n, m;
    const float *f, *g;      // true potentials
    const double *la, *lb;   // natural log of the weights, [B][n] and [B][m] (-inf for 0)
    double inv_eps;
    const KeyD *kd = nullptr;   // d = 3: the keys (Y, g) as KeyD [B][m], or NULL
    const KeyB *kb = nullptr;   // d = 3 (all but the cost pass): the keys as KeyB [B][m]
};
// KeyD records of the keys (Y [B][m][3], g [B][m]) of a d = 3 pass.
hipError_t launch_keys_d3(const void *Y, int dtype, const float *g, int B, int m, KeyD *out,
                          hipStream_t st);
// log a, log b (fp64, as launch_log_weights) and, for d = 3, the KeyB records of
// X (kx, from f and log a) and of Y (ky, from g and log b) where not NULL, in one
// launch.
hipError_t launch_plan_prep(const float *a, const float *b, int B, int n, int m, double *la,
                            double *lb, const void *X, const void *Y, int dtype, const float *f,
                            const float *g, double inv_eps, double scale, KeyB *kx, KeyB *ky,
                            hipStream_t st);
// log of the weights in fp64 (w == NULL: uniform 1/count)
hipError_t launch_log_weights(const float *w, int B, int count, double *out, hipStream_t st);
hipError_t launch_cost(const PlanArgs &p, double *row_part, float *cost, hipStream_t st);
hipError_t launch_plan_max(const PlanArgs &p, double *row_max, double *pair_thr,
                           double log_rel_thr, hipStream_t st);
hipError_t launch_plan_count(const PlanArgs &p, const double *pair_thr, int32_t *row_count,
                             hipStream_t st);
// total_copy != NULL: the entry count is also written there (device int64).
hipError_t launch_plan_scan(const int32_t *row_count, int B, int n, int64_t *row_off,
                            int64_t *pair_offsets, int64_t *pair_tot, int64_t *total_copy,
                            hipStream_t st);
// Emission of the counted entries; with loss / dX (either may be NULL) also the
// loss per pair and its gradient in X on the emitted support (row_loss: [B][n]
// scratch, needed with loss).
// gate != NULL: every kernel first reads *gate (the plan's entry count, on the
// device) and writes nothing if it exceeds gate_cap.
hipError_t launch_plan_emit(const PlanArgs &p, const double *pair_thr, const int64_t *row_off,
                            const int32_t *row_count, int32_t *rows, int32_t *cols,
                            float *vals, double *row_loss, float *loss, float *dX,
                            const int64_t *gate, int64_t gate_cap, hipStream_t st);
// Dense gradient 2 sum_j P_ij (x_i - y_j) and barycentric projection
// sum_j P_ij y_j / sum_j P_ij of every row of p.X (either output may be NULL),
// log P in fp64.  only != NULL: just the 64-row blocks flagged there.
hipError_t launch_dense_grad(const PlanArgs &p, float *grad, float *proj, const int *only,
                             hipStream_t st);
// The same on the matrix cores for bf16 with d = 32 or 64, one side: the rows'
// side (points, potential, squared norms; n_pad a multiple of kGradPad; its redo
// array [B][ceil(n / 64)] receives the 64-row blocks left to the fp64 pass), row
// weights (NULL: uniform), the key side's points, biases at eps (launch_packF
// with warm start, n_pad a multiple of kGradPad) and transposed points
// [B][d][n_pad], and scratch sized by gradF_sizes.
constexpr int kGradPad = 512;
bool gradF_matrix_cores(int dtype, int d);
struct GradFSizes {
    size_t h, part_s, part_v;   // floats
};
GradFSizes gradF_sizes(int B, int n, int m, int d);
struct GradFWs {
    float *h, *part_s, *part_v;
};
hipError_t launch_gradF(const SideF &rows, const float *row_w, const SideF &keys,
                        const uint16_t *keys_t, int d, int B, float eps, const GradFWs &w,
                        float *grad, float *proj, hipStream_t st);
hipError_t launch_transpose_bf16(const void *X, int B, int n, int n_pad, int d, uint16_t *Xt,
                                 hipStream_t st);
// Runs of equal keys in a key-sorted COO (per pair), by binary search:
// begin/end [B][count]; a key with no entries gets an empty run.
hipError_t launch_segment_bounds(const int32_t *keys, const int64_t *pair_offsets, int B, int count,
                                 int64_t *begin, int64_t *end, hipStream_t st);
// Sinkhorn normalisation of a row-sorted COO plan on its support, given its
// transpose (column-sorted, the same entries and values).  Workspace pieces as
// carved by the ABI.
struct CooNormWs {
    int64_t *rb, *re, *cb, *ce;   // row runs of the plan, column runs of the transpose
    float *lv, *lvt;              // log of the values of the plan and of the transpose
    double *al, *be, *la, *lb;    // scalings and log weights
    double *row_part, *col_part;  // per-row / per-column marginal errors
    uint64_t *sums;               // [2][B] entry checksums of the plan and the transpose
    int *bad;                     // pairs whose transpose does not match the plan
};
// Checks the transpose against the plan (per pair: entry counts and a checksum
// of every entry's (row, column, value bits)); *w.bad = mismatching pairs.
hipError_t launch_coo_check(const int32_t *rows, const int32_t *cols, const float *vals,
                            const int64_t *offs, const int32_t *t_rows, const int32_t *t_cols,
                            const float *t_vals, const int64_t *t_offs, int B, const CooNormWs &w,
                            hipStream_t st);
hipError_t launch_coo_normalize(const int32_t *rows, const int32_t *cols, float *vals,
                                const int64_t *offs, const int32_t *t_rows, const int32_t *t_cols,
                                float *t_vals, const int64_t *t_offs, int B, int n, int m,
                                int64_t nnz, int iters, float *err, const float *a,
                                const float *b, const CooNormWs &w, hipStream_t st);
// Hessian-vector product of the entropic OT value in X (d <= 16): px = plan
// arguments with rows X, py the same with the roles exchanged.
struct HvpWs {
    double *la, *lb;                    // log weights
    double *ma, *tv, *ur, *mur;         // [B][n]
    double *D1, *Tv, *Du;               // [B][n][d]
    double *mb, *muc, *tw, *rhs;        // [B][m]
    double *x, *res, *dir;              // conjugate-gradient vectors [B][m]
    double *rr, *rr0;                   // [B]
    KeyB *kbx = nullptr, *kby = nullptr;   // d = 3: fp64 keys of the two sides
};
hipError_t launch_hvp(const PlanArgs &px, const PlanArgs &py, const float *V, int cg_iters,
                      float *HV, float *cg_residual, const HvpWs &w, hipStream_t st);
// Cosine cost support: points to unit length (fp32 out, norms kept), and the
// gradient through that map.
hipError_t launch_normalize(const void *X, int dtype, long count, int d, float *Xh,
                            float *norms, hipStream_t st);
hipError_t launch_normalize_backward(const float *Xh, const float *norms, const float *G,
                                     long count, int d, float *dX, hipStream_t st);

hipError_t launch_loss_grad(const void *X, const void *Y, int dtype, int d, int B, int n,
                            int m, const int32_t *rows, const int32_t *cols, const float *vals,
                            const int64_t *pair_offsets, int64_t *row_begin,
                            int64_t *row_end, double *row_loss, float *loss, float *dX,
                            hipStream_t st);

}  // namespace sk

// plan.hip -- passes over the transport plan at the final eps, never stored:
//     log P_ij = (f_i + g_j - C_ij)/eps + log a_i + log b_j,  C_ij = ||x_i - y_j||^2
// (the plan of the stabilised log-domain Sinkhorn solution, FlashSinkhorn
// summary, Methodologie 1), used for
//   - the transport cost   sum_ij P_ij C_ij;
//   - the thresholded sparse plan of the CUDA-APML page (Abstract, Innovation):
//     per pair the maximum of log P, a count of the entries at or above
//     max + log(rel_threshold) per row, a scan of the counts into offsets, and
//     the emission of (row, col, P) in row-major order.
//
// log P is evaluated in fp64 from the fp32 potentials and weights (fp64 FMA
// runs at the fp32 rate on this chip, and these passes run once per solve),
// so the threshold decision does not add fp32 rounding of the large
// potentials; P itself is returned as fp32.  The count and emit passes call the
// same evaluation on the same inputs, so their decisions agree bit for bit.
//
//   - the dense transport application (FlashSinkhorn summary, Methodologie 3,
//     "Toepassing van Transportmatrix": the gradient and the barycentric
//     projection are weighted averages over the plan, streamed like the
//     update): per row r_i = sum_j P_ij, G_i = sum_j P_ij (x_i - y_j), giving
//     dX_i = 2 G_i and T_i = sum_j P_ij y_j / r_i = x_i - G_i / r_i.
//
// Two traversals.  Passes that reduce each row to a few numbers (cost, max,
// count, dense gradient) hold one row per lane, 64 rows per wave, and take the
// keys one at a time, the same key in every lane: for d = 3 the work-group
// stages the keys' fp64 records in LDS and the lanes read them with broadcast
// loads, otherwise they read them with wave-uniform (scalar) loads; the 4
// waves of a work-group take every 4th key and merge in LDS.  The emit
// pass holds one row per wave with lanes across 64 consecutive columns, so
// each wave writes contiguous slices of the COO arrays; for d <= 4 the
// columns are staged in LDS once per work-group of 32 rows.
#include "plan_eval.h"

namespace sk {
namespace {

constexpr int kRowsPerGroup = 4;  // emit pass: one wave per row

__global__ void log_weights_kernel(const float *__restrict__ w, int count, size_t total,
                                   double *__restrict__ out)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total)
        return;
    if (!w) {
        out[i] = -log((double)count);
        return;
    }
    const float v = w[i];
    out[i] = v > 0.f ? log((double)v) : -INFINITY;
}


constexpr int kTileWaves = 4;   // waves of a tile_pass work-group, splitting the keys
constexpr int kKeyStage = 512;  // d = 3 key records staged in LDS per step (20 KB)
constexpr int kGradDims = 16;   // gradient components accumulated per launch (no spills)

// mode 0: cost  (row sum of P C, double)          -> outd[row]
// mode 1: max   (row max of log P, double)        -> outd[row]
// mode 2: count (entries >= thr, int32)           -> outi[row]
// mode 3: dense gradient for dims k0 .. k0+KC-1   -> grad, proj (fp32, [B][n][d])
template <typename T, int DP, int MODE, bool KD>
__global__ __launch_bounds__(kTileWaves *kWave) void tile_pass(
    PlanArgs p, const double *__restrict__ thr, double *__restrict__ outd,
    int32_t *__restrict__ outi, float *__restrict__ grad, float *__restrict__ proj, int k0,
    const int *__restrict__ only)
{
    // only != nullptr: redo just the row blocks flagged there
    if (only && !only[blockIdx.y * gridDim.x + blockIdx.x])
        return;
    constexpr int KC = MODE == 3 ? (DP < kGradDims ? DP : kGradDims) : 1;
    __shared__ double red[kTileWaves][kWave];
    const int b = blockIdx.y;
    const int w = wave_id_uniform();
    const int lane = lane_id();
    const int i = blockIdx.x * kWave + lane;
    const bool live = i < p.n;
    RowCtx<DP> r;
    load_row<T, DP>(r, p, b, live ? i : p.n - 1);
    const T *Yb = (const T *)p.Y + (size_t)b * p.m * p.d;
    const float *gb = p.g + (size_t)b * p.m;
    const double *lbb = p.lb + (size_t)b * p.m;
    const KeyD *kdb = p.kd ? p.kd + (size_t)b * p.m : nullptr;
    // the sparse plan's max and count passes and the dense gradient over staged
    // d = 3 keys take the expanded form of log P (KeyB records, the row's A_i);
    // the cost pass (which needs C_ij) takes KeyD records
    constexpr bool kPB = MODE != 0 && KD;
    const KeyB *kbb = kPB ? p.kb + (size_t)b * p.m : nullptr;
    double xd[3] = {0.0, 0.0, 0.0}, A = 0.0;
    if constexpr (kPB) {
#pragma unroll
        for (int k = 0; k < 3; ++k)
            xd[k] = (double)r.x[k];
        A = side_term_d3(xd[0], xd[1], xd[2], r.f, r.la, p.inv_eps);
    }
    // the dense gradient's records and A_i carry log P in base 2
    constexpr double kLs = kPB && MODE == 3 ? kLog2eD : 1.0;
    if constexpr (kLs != 1.0)
        A *= kLs;
    const double two_inv_eps = 2.0 * p.inv_eps * kLs;
    const double t = MODE == 2 ? thr[b] : 0.0;
    double acc = MODE == 1 ? -INFINITY : 0.0;
    int cnt = 0;
    double G[KC], xc[KC];   // gradient sums and this chunk's row coordinates
    {
        const T *x = (const T *)p.X + ((size_t)b * p.n + (live ? i : p.n - 1)) * p.d;
#pragma unroll
        for (int k = 0; k < KC; ++k) {
            G[k] = 0.0;
            xc[k] = MODE == 3 && has_dim<DP>(k0 + k, p.d) ? (double)Elem<T>::get(x, k0 + k) : 0.0;
        }
    }
    // narrow points: the key's values in registers (from the staged KeyD records
    // for d = 3), and whole-row gradients (one chunk) reuse the evaluation's
    // differences
    constexpr bool kRegs = DP <= kKeyRegDims;
    constexpr bool kDiff = kRegs && MODE == 3 && KC == DP;
    __shared__ KeyD kst[KD && !kPB ? kKeyStage : 1];
    __shared__ double lbst[KD && !kPB ? kKeyStage : 1];
    __shared__ KeyB kbst[kPB ? kKeyStage : 1];
    auto visit = [&](int j, int js) {
        double C, lp;
        double diff[kDiff ? DP : 1];
        if constexpr (kPB) {
            // staged in LDS: every lane of the wave reads the same record
            const KeyB kr = kbst[js];
            const double y[3] = {kr.y[0], kr.y[1], kr.y[2]};
            lp = log_plan_b3(xd, A, y, kr.B, two_inv_eps);
            if constexpr (kDiff) {
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    diff[k] = xd[k] - y[k];
            }
        } else if constexpr (KD) {
            // staged in LDS: every lane of the wave reads the same record
            const KeyD kr = kst[js];
            KeyVals<DP> kv;
#pragma unroll
            for (int k = 0; k < DP; ++k)
                kv.y[k] = kr.y[k];
            kv.g = kr.g;
            lp = log_plan_kv<DP>(r, kv, lbst[js], p.inv_eps, p.d, &C, kDiff ? diff : nullptr);
        } else if constexpr (kRegs) {
            KeyVals<DP> kv;
            load_key<T, DP, KD>(kv, p, Yb, gb, kdb, j);
            lp = log_plan_kv<DP>(r, kv, lbb[j], p.inv_eps, p.d, &C, kDiff ? diff : nullptr);
        } else {
            lp = log_plan<T, DP>(r, p, Yb, gb, lbb[j], j, &C);
        }
        if (MODE == 0) {
            const double P = (double)ex2((float)(lp * 1.4426950408889634));
            acc = fma(P, C, acc);
        } else if (MODE == 1) {
            acc = fmax(acc, lp);
        } else if (MODE == 2) {
            cnt += lp >= t ? 1 : 0;
        } else {
            const double P = (double)ex2((float)(kLs != 1.0 ? lp : lp * kLog2eD));
            acc += P;
            if constexpr (kDiff) {
#pragma unroll
                for (int k = 0; k < KC; ++k)
                    if (has_dim<DP>(k, p.d))
                        G[k] = fma(P, diff[k], G[k]);
            } else {
                const T *y = Yb + (size_t)j * p.d;
#pragma unroll
                for (int k = 0; k < KC; ++k)
                    if (has_dim<DP>(k0 + k, p.d))
                        G[k] = fma(P, xc[k] - (double)Elem<T>::get(y, k0 + k), G[k]);
            }
        }
    };
    if constexpr (KD) {
        // d = 3: the pair's fp64 key records pass through LDS a stage at a time
        for (int c0 = 0; c0 < p.m; c0 += kKeyStage) {
            const int kc = min(kKeyStage, p.m - c0);
            __syncthreads();   // the previous stage is no longer read
            for (int e = threadIdx.x; e < kc; e += kTileWaves * kWave) {
                if constexpr (kPB) {
                    kbst[e] = kbb[c0 + e];
                } else {
                    kst[e] = kdb[c0 + e];
                    lbst[e] = lbb[c0 + e];
                }
            }
            __syncthreads();
            int js = w;
            for (; js + 3 * kTileWaves < kc; js += 4 * kTileWaves) {
                visit(c0 + js, js);
                visit(c0 + js + kTileWaves, js + kTileWaves);
                visit(c0 + js + 2 * kTileWaves, js + 2 * kTileWaves);
                visit(c0 + js + 3 * kTileWaves, js + 3 * kTileWaves);
            }
            for (; js < kc; js += kTileWaves)
                visit(c0 + js, js);
        }
    } else {
        int j = w;
        if constexpr (DP <= 4) {
            // four keys per step, so that their loads are in flight together
            for (; j + 3 * kTileWaves < p.m; j += 4 * kTileWaves) {
                visit(j, 0);
                visit(j + kTileWaves, 0);
                visit(j + 2 * kTileWaves, 0);
                visit(j + 3 * kTileWaves, 0);
            }
        }
        for (; j < p.m; j += kTileWaves)
            visit(j, 0);
    }
    // merge the waves in a fixed order
    auto merged = [&](double v, bool is_max) {
        __syncthreads();
        red[w][lane] = v;
        __syncthreads();
        double s = red[0][lane];
#pragma unroll
        for (int v2 = 1; v2 < kTileWaves; ++v2)
            s = is_max ? fmax(s, red[v2][lane]) : s + red[v2][lane];
        return s;
    };
    if (MODE == 2) {
        const double tot = merged((double)cnt, false);
        if (w == 0 && live)
            outi[(size_t)b * p.n + i] = (int32_t)tot;
    } else if (MODE != 3) {
        const double tot = merged(acc, MODE == 1);
        if (w == 0 && live)
            outd[(size_t)b * p.n + i] = tot;
    } else {
        const double mass = merged(acc, false);
        const size_t o = ((size_t)b * p.n + i) * p.d;
#pragma unroll
        for (int k = 0; k < KC; ++k) {
            if (!has_dim<DP>(k0 + k, p.d))   // uniform: every thread skips alike
                continue;
            const double Gk = merged(G[k], false);
            if (w == 0 && live) {
                if (grad)
                    grad[o + k0 + k] = (float)(2.0 * Gk);
                if (proj)
                    proj[o + k0 + k] = mass > 0.0 ? (float)(xc[k] - Gk / mass) : 0.f;
            }
        }
    }
}

// Per-pair reduction of row values in a fixed order (deterministic).
// mode 0: sum -> float out[b];  mode 1: max + add -> double out[b]
// gate != nullptr: write nothing unless *gate <= gate_cap (a plan that fit)
template <int MODE>
__global__ __launch_bounds__(256) void pair_reduce(const double *__restrict__ rowv, int n,
                                                   float *__restrict__ outf,
                                                   double *__restrict__ outd, double add,
                                                   const int64_t *__restrict__ gate,
                                                   int64_t gate_cap)
{
    __shared__ double sm[256];
    if (gate && *gate > gate_cap)
        return;
    const int b = blockIdx.x;
    double acc = MODE == 0 ? 0.0 : -INFINITY;
    for (int i = threadIdx.x; i < n; i += 256) {
        const double v = rowv[(size_t)b * n + i];
        acc = MODE == 0 ? acc + v : fmax(acc, v);
    }
    sm[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < s)
            sm[threadIdx.x] = MODE == 0 ? sm[threadIdx.x] + sm[threadIdx.x + s]
                                        : fmax(sm[threadIdx.x], sm[threadIdx.x + s]);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        if (MODE == 0)
            outf[b] = (float)sm[0];
        else
            outd[b] = sm[0] + add;
    }
}

// Sum of the row counts of each pair.
__global__ __launch_bounds__(256) void pair_totals(const int32_t *__restrict__ cnt, int n,
                                                   int64_t *__restrict__ tot)
{
    __shared__ int64_t sm[256];
    const int b = blockIdx.x;
    int64_t acc = 0;
    for (int i = threadIdx.x; i < n; i += 256)
        acc += cnt[(size_t)b * n + i];
    sm[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < s)
            sm[threadIdx.x] += sm[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        tot[b] = sm[0];
}

// Exclusive scan of a block-sized chunk in LDS; returns the chunk total.
__device__ int64_t block_exclusive_scan(int64_t *sm, int64_t v)
{
    const int t = threadIdx.x;
    sm[t] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int64_t add = t >= off ? sm[t - off] : 0;
        __syncthreads();
        sm[t] += add;
        __syncthreads();
    }
    const int64_t incl = sm[t];
    const int64_t total = sm[255];
    __syncthreads();
    sm[t] = incl - v;
    return total;
}

// Single group: pair_offsets[0..B] from the pair totals.
// (total != NULL: the plan's entry count is also written there)
__global__ __launch_bounds__(256) void pair_offsets_scan(const int64_t *__restrict__ tot, int B,
                                                         int64_t *__restrict__ offs,
                                                         int64_t *__restrict__ total_out)
{
    __shared__ int64_t sm[256];
    int64_t carry = 0;
    for (int base = 0; base < B; base += 256) {
        const int b = base + threadIdx.x;
        const int64_t v = b < B ? tot[b] : 0;
        const int64_t total = block_exclusive_scan(sm, v);
        if (b < B)
            offs[b] = carry + sm[threadIdx.x];
        carry += total;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        offs[B] = carry;
        if (total_out)
            *total_out = carry;
    }
}

// One group per pair: global offset of every row.
__global__ __launch_bounds__(256) void row_offsets_scan(const int32_t *__restrict__ cnt, int n,
                                                        const int64_t *__restrict__ offs,
                                                        int64_t *__restrict__ row_off)
{
    __shared__ int64_t sm[256];
    const int b = blockIdx.x;
    int64_t carry = offs[b];
    for (int base = 0; base < n; base += 256) {
        const int i = base + threadIdx.x;
        const int64_t v = i < n ? cnt[(size_t)b * n + i] : 0;
        const int64_t total = block_exclusive_scan(sm, v);
        if (i < n)
            row_off[(size_t)b * n + i] = carry + sm[threadIdx.x];
        carry += total;
        __syncthreads();
    }
}

// LG: also accumulate the loss and its gradient in x over the emitted entries
// (loss_term on the value as stored), one row per wave: row_loss [B][n] and
// dX [B][n][d] (either may be NULL).
template <typename T, int DP, bool LG>
__global__ __launch_bounds__(kRowsPerGroup *kWave) void emit_pass(
    PlanArgs p, const double *__restrict__ thr, const int64_t *__restrict__ row_off,
    const int32_t *__restrict__ row_cnt, int32_t *__restrict__ rows, int32_t *__restrict__ cols,
    float *__restrict__ vals, double *__restrict__ row_loss, float *__restrict__ dX,
    const int64_t *__restrict__ gate, int64_t gate_cap)
{
    if (gate && *gate > gate_cap)
        return;   // the plan does not fit: nothing is written
    const int b = blockIdx.y;
    const int i = blockIdx.x * kRowsPerGroup + wave_id_uniform();
    if (i >= p.n)
        return;
    const int lane = lane_id();
    RowCtx<DP> r;
    load_row<T, DP>(r, p, b, i);
    const T *Yb = (const T *)p.Y + (size_t)b * p.m * p.d;
    const float *gb = p.g + (size_t)b * p.m;
    const double t = thr[b];
    int64_t pos = row_off[(size_t)b * p.n + i];
    const int64_t end = pos + row_cnt[(size_t)b * p.n + i];
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    double loss = 0.0;
    float gr[DP];
#pragma unroll
    for (int c = 0; c < DP; ++c)
        gr[c] = 0.f;
    for (int j0 = 0; j0 < p.m && pos < end; j0 += kWave) {
        const int j = j0 + lane;
        bool keep = false;
        double lp = 0.0, C = 0.0;
        if (j < p.m) {
            lp = log_plan<T, DP>(r, p, Yb, gb, p.lb[(size_t)b * p.m + j], j, &C);
            keep = lp >= t;
        }
        const uint64_t mask = __ballot(keep);
        if (keep) {
            const int64_t k = pos + __popcll(mask & below);
            if (k < end) {   // always true: count and emit make identical decisions
                const float P = ex2((float)(lp * 1.4426950408889634));
                rows[k] = i;
                cols[k] = j;
                vals[k] = P;
                if constexpr (LG)   // differences recomputed: no per-entry array for wide rows
                    loss_term_at<T, DP>(r.x, Yb + (size_t)j * p.d, p.d, P, loss, gr);
            }
        }
        pos += __popcll(mask);
    }
    if (LG) {
        const size_t ri = (size_t)b * p.n + i;
        loss = wave_sum(loss);
        if (row_loss && lane == 0)
            row_loss[ri] = loss;
        if (dX) {
#pragma unroll
            for (int c = 0; c < DP; ++c) {
                if (has_dim<DP>(c, p.d)) {
                    const float v = wave_sum(gr[c]);
                    if (lane == 0)
                        dX[ri * p.d + c] = v;
                }
            }
        }
    }
}

// Emit pass for small d with the keys staged in LDS: a work-group of
// kEmitWaves waves takes kEmitRows consecutive rows of one pair (a wave per row
// at a time, lanes across 64 consecutive columns, as above) and shares one
// staged copy of each chunk of kEmitChunk columns (d = 3: the KeyB records'
// point components and B_j; d = 4: point components and g_j as fp64, log b_j),
// so the column data is read and converted once per work-group instead of once
// per row.  The evaluation is the count pass's (log_plan_b3 for d = 3,
// log_plan_kv otherwise) on the same values, so the decisions agree bit for bit.
constexpr int kEmitWaves = 8, kEmitRows = 32, kEmitChunk = 1024;

template <typename T, int DP, bool LG>
__global__ __launch_bounds__(kEmitWaves *kWave) void emit_staged(
    PlanArgs p, const double *__restrict__ thr, const int64_t *__restrict__ row_off,
    const int32_t *__restrict__ row_cnt, int32_t *__restrict__ rows, int32_t *__restrict__ cols,
    float *__restrict__ vals, double *__restrict__ row_loss, float *__restrict__ dX,
    const int64_t *__restrict__ gate, int64_t gate_cap)
{
    if (gate && *gate > gate_cap)
        return;   // the plan does not fit: nothing is written
    static_assert(DP <= 4, "staged emit holds at most 4 components per column");
    constexpr int kRowsPerWave = kEmitRows / kEmitWaves;
    // d = 3: the expanded log P from KeyB records (the count pass's values);
    // gs then holds B_j and lbs is not used
    constexpr bool kPB = DP == 3;
    __shared__ double ys[DP][kEmitChunk];
    __shared__ double gs[kEmitChunk];
    __shared__ double lbs[kPB ? 1 : kEmitChunk];
    const int b = blockIdx.y;
    const int wave = wave_id_uniform(), lane = lane_id();
    const int i0 = blockIdx.x * kEmitRows + wave * kRowsPerWave;
    const T *Yb = (const T *)p.Y + (size_t)b * p.m * p.d;
    const float *gb = p.g + (size_t)b * p.m;
    const double *lbb = p.lb + (size_t)b * p.m;
    const KeyB *kbb = kPB ? p.kb + (size_t)b * p.m : nullptr;
    const double t = thr[b];
    const double two_inv_eps = 2.0 * p.inv_eps;
    RowCtx<DP> r[kRowsPerWave];
    double xd[kRowsPerWave][3], A[kRowsPerWave];   // kPB: the rows as fp64 and their A_i
    int64_t pos[kRowsPerWave];   // the row's next entry
    int rem[kRowsPerWave];       // and how many are still to come (wave-uniform)
    double loss[kRowsPerWave];
    float gr[kRowsPerWave][DP];
#pragma unroll
    for (int q = 0; q < kRowsPerWave; ++q) {
        const int i = min(i0 + q, p.n - 1);   // rows past n are loaded but never emitted
        load_row<T, DP>(r[q], p, b, i);
        if constexpr (kPB) {
#pragma unroll
            for (int k = 0; k < 3; ++k)
                xd[q][k] = (double)r[q].x[k];
            A[q] = side_term_d3(xd[q][0], xd[q][1], xd[q][2], r[q].f, r[q].la, p.inv_eps);
        }
        pos[q] = row_off[(size_t)b * p.n + i];
        rem[q] = i0 + q < p.n ? row_cnt[(size_t)b * p.n + i] : 0;
        loss[q] = 0.0;
#pragma unroll
        for (int c = 0; c < DP; ++c)
            gr[q][c] = 0.f;
    }
    for (int c0 = 0; c0 < p.m; c0 += kEmitChunk) {
        const int kc = min(kEmitChunk, p.m - c0);
        __syncthreads();   // the previous chunk is no longer read
        for (int j = threadIdx.x; j < kc; j += kEmitWaves * kWave) {
            if constexpr (kPB) {
                const KeyB kr = kbb[c0 + j];
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    ys[k][j] = kr.y[k];
                gs[j] = kr.B;
            } else {
                KeyVals<DP> kv;
                load_key<T, DP, false>(kv, p, Yb, gb, nullptr, c0 + j);
#pragma unroll
                for (int k = 0; k < DP; ++k)
                    ys[k][j] = kv.y[k];
                gs[j] = kv.g;
                lbs[j] = lbb[c0 + j];
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kRowsPerWave; ++q) {
            // wave-uniform bases at the row's next entry; a lane stores at its
            // 32-bit rank among the step's kept entries
            int32_t *rq = rows + pos[q];
            int32_t *cq = cols + pos[q];
            float *vq = vals + pos[q];
            int left = rem[q];
            for (int j0 = 0; j0 < kc && left > 0; j0 += kWave) {
                const int j = j0 + lane;
                const int jc = min(j, kc - 1);   // lanes past the chunk evaluate its last column
                KeyVals<DP> kv;
#pragma unroll
                for (int k = 0; k < DP; ++k)
                    kv.y[k] = ys[k][jc];
                kv.g = gs[jc];
                double C = 0.0, lp;
                double diff[LG ? DP : 1];
                if constexpr (kPB) {
                    const double y[3] = {kv.y[0], kv.y[1], kv.y[2]};
                    lp = log_plan_b3(xd[q], A[q], y, kv.g, two_inv_eps);
                    if constexpr (LG) {   // the loss term's differences and C as log_plan_kv
#pragma unroll
                        for (int k = 0; k < 3; ++k) {
                            diff[k] = xd[q][k] - y[k];
                            C = fma(diff[k], diff[k], C);
                        }
                    }
                } else {
                    lp = log_plan_kv<DP>(r[q], kv, lbs[jc], p.inv_eps, p.d, &C,
                                         LG ? diff : nullptr);
                }
                const bool keep = j < kc && lp >= t;
                const uint64_t mask = __builtin_amdgcn_ballot_w64(keep);
                // kept lanes below this one
                const uint32_t idx = __builtin_amdgcn_mbcnt_hi(
                    (uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                if (keep && idx < (uint32_t)left) {   // always: count and emit agree
                    const float P = ex2((float)(lp * 1.4426950408889634));
                    const uint32_t at = idx * 4u;   // 32-bit byte offset from the bases
                    *(int32_t *)((char *)rq + at) = i0 + q;
                    *(int32_t *)((char *)cq + at) = c0 + j;
                    *(float *)((char *)vq + at) = P;
                    if constexpr (LG)
                        loss_term<DP>(diff, C, p.d, P, loss[q], gr[q]);
                }
                const int nk = __popcll(mask);
                rq += nk;
                cq += nk;
                vq += nk;
                left -= nk;
            }
            pos[q] += rem[q] - left;
            rem[q] = left;
        }
    }
    if (LG) {
#pragma unroll
        for (int q = 0; q < kRowsPerWave; ++q) {
            if (i0 + q >= p.n)
                break;
            const size_t ri = (size_t)b * p.n + i0 + q;
            const double l = wave_sum(loss[q]);
            if (row_loss && lane == 0)
                row_loss[ri] = l;
            if (dX) {
#pragma unroll
                for (int c = 0; c < DP; ++c) {
                    if (has_dim<DP>(c, p.d)) {
                        const float v = wave_sum(gr[q][c]);
                        if (lane == 0)
                            dX[ri * p.d + c] = v;
                    }
                }
            }
        }
    }
}

template <typename T>
__global__ void keys_d3_kernel(const T *__restrict__ Y, const float *__restrict__ g, size_t count,
                               KeyD *__restrict__ out)
{
    const size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= count)
        return;
    KeyD r;
#pragma unroll
    for (int c = 0; c < 3; ++c)
        r.y[c] = (double)Elem<T>::get(Y, 3 * k + c);
    r.g = (double)g[k];
    out[k] = r;
}

// The plan passes' per-point inputs in one launch: la = log a [B][n] and
// lb = log b [B][m] (as log_weights_kernel), and for d = 3 the KeyB records of
// either side, from the point, its potential and the log weight just computed,
// B times scale: kx from (X, f, la) when not NULL, ky from (Y, g, lb) when not
// NULL.
template <typename T>
__global__ void plan_prep_kernel(const float *__restrict__ a, const float *__restrict__ b,
                                 int B, int n, int m, double *__restrict__ la,
                                 double *__restrict__ lb, const T *__restrict__ X,
                                 const T *__restrict__ Y, const float *__restrict__ f,
                                 const float *__restrict__ g, double inv_eps, double scale,
                                 KeyB *__restrict__ kx, KeyB *__restrict__ ky)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t bn = (size_t)B * n, bm = (size_t)B * m;
    const bool xs = i < bn;
    if (!xs && i >= bn + bm)
        return;
    const size_t k = xs ? i : i - bn;
    const float *w = xs ? a : b;
    const int count = xs ? n : m;
    double lw;
    if (!w) {
        lw = -log((double)count);
    } else {
        const float v = w[k];
        lw = v > 0.f ? log((double)v) : -INFINITY;
    }
    (xs ? la : lb)[k] = lw;
    KeyB *out = xs ? kx : ky;
    if (out) {
        const T *P = xs ? X : Y;
        KeyB r;
#pragma unroll
        for (int c = 0; c < 3; ++c)
            r.y[c] = (double)Elem<T>::get(P, 3 * k + c);
        r.B = scale * side_term_d3(r.y[0], r.y[1], r.y[2], (double)(xs ? f : g)[k], lw, inv_eps);
        out[k] = r;
    }
}

template <typename F>
void with_dp(int d, F fn)
{
    if (d == 3) fn.template operator()<3>();
    else if (d <= 4) fn.template operator()<4>();
    else if (d <= 8) fn.template operator()<8>();
    else if (d <= 16) fn.template operator()<16>();
    else if (d <= 32) fn.template operator()<32>();
    else if (d <= 64) fn.template operator()<64>();
    else fn.template operator()<128>();
}

template <int MODE>
void tile_dispatch(const PlanArgs &p, const double *thr, double *outd, int32_t *outi,
                   float *grad, float *proj, hipStream_t st, const int *only = nullptr)
{
    dim3 grid(ceil_div(p.n, kWave), p.B);
    dim3 block(kTileWaves * kWave);
    with_dp(p.d, [&]<int DP>() {
        const int chunks = MODE == 3 ? ceil_div(p.d, kGradDims) : 1;
        auto go = [&]<bool KD>() {
            for (int c = 0; c < chunks; ++c) {
                if (p.dtype == 1)
                    hipLaunchKernelGGL((tile_pass<uint16_t, DP, MODE, KD>), grid, block, 0, st, p,
                                       thr, outd, outi, grad, proj, c * kGradDims, only);
                else
                    hipLaunchKernelGGL((tile_pass<float, DP, MODE, KD>), grid, block, 0, st, p,
                                       thr, outd, outi, grad, proj, c * kGradDims, only);
            }
        };
        if constexpr (DP == 3) {
            if (MODE != 0 ? p.kb != nullptr : p.kd != nullptr) {
                go.template operator()<true>();
                return;
            }
        }
        go.template operator()<false>();
    });
}

}  // namespace

hipError_t launch_keys_d3(const void *Y, int dtype, const float *g, int B, int m, KeyD *out,
                          hipStream_t st)
{
    const size_t count = (size_t)B * m;
    const dim3 grid((unsigned)((count + 255) / 256));
    if (dtype == 1)
        hipLaunchKernelGGL(keys_d3_kernel<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)Y,
                           g, count, out);
    else
        hipLaunchKernelGGL(keys_d3_kernel<float>, grid, dim3(256), 0, st, (const float *)Y, g,
                           count, out);
    return hipGetLastError();
}

hipError_t launch_plan_prep(const float *a, const float *b, int B, int n, int m, double *la,
                            double *lb, const void *X, const void *Y, int dtype, const float *f,
                            const float *g, double inv_eps, double scale, KeyB *kx, KeyB *ky,
                            hipStream_t st)
{
    const size_t total = (size_t)B * n + (size_t)B * m;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (dtype == 1)
        hipLaunchKernelGGL(plan_prep_kernel<uint16_t>, grid, dim3(256), 0, st, a, b, B, n, m, la,
                           lb, (const uint16_t *)X, (const uint16_t *)Y, f, g, inv_eps, scale, kx,
                           ky);
    else
        hipLaunchKernelGGL(plan_prep_kernel<float>, grid, dim3(256), 0, st, a, b, B, n, m, la, lb,
                           (const float *)X, (const float *)Y, f, g, inv_eps, scale, kx, ky);
    return hipGetLastError();
}

hipError_t launch_log_weights(const float *w, int B, int count, double *out, hipStream_t st)
{
    const size_t total = (size_t)B * count;
    hipLaunchKernelGGL(log_weights_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       st, w, count, total, out);
    return hipGetLastError();
}

hipError_t launch_cost(const PlanArgs &p, double *row_part, float *cost, hipStream_t st)
{
    tile_dispatch<0>(p, nullptr, row_part, nullptr, nullptr, nullptr, st);
    hipLaunchKernelGGL(pair_reduce<0>, dim3(p.B), dim3(256), 0, st, (const double *)row_part,
                       p.n, cost, (double *)nullptr, 0.0, (const int64_t *)nullptr, (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_row_sums(const double *row_part, int B, int n, float *out, hipStream_t st)
{
    hipLaunchKernelGGL(pair_reduce<0>, dim3(B), dim3(256), 0, st, row_part, n, out,
                       (double *)nullptr, 0.0, (const int64_t *)nullptr, (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_plan_max(const PlanArgs &p, double *row_max, double *pair_thr,
                           double log_rel_thr, hipStream_t st)
{
    if (p.d == 3 && !p.kb)
        return hipErrorInvalidValue;   // d = 3 plans take KeyB records in every pass
    tile_dispatch<1>(p, nullptr, row_max, nullptr, nullptr, nullptr, st);
    hipLaunchKernelGGL(pair_reduce<1>, dim3(p.B), dim3(256), 0, st, (const double *)row_max,
                       p.n, (float *)nullptr, pair_thr, log_rel_thr, (const int64_t *)nullptr,
                       (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_plan_count(const PlanArgs &p, const double *pair_thr, int32_t *row_count,
                             hipStream_t st)
{
    if (p.d == 3 && !p.kb)
        return hipErrorInvalidValue;
    tile_dispatch<2>(p, pair_thr, nullptr, row_count, nullptr, nullptr, st);
    return hipGetLastError();
}

hipError_t launch_plan_scan(const int32_t *row_count, int B, int n, int64_t *row_off,
                            int64_t *pair_offsets, int64_t *pair_tot, int64_t *total_copy,
                            hipStream_t st)
{
    hipLaunchKernelGGL(pair_totals, dim3(B), dim3(256), 0, st, row_count, n, pair_tot);
    hipLaunchKernelGGL(pair_offsets_scan, dim3(1), dim3(256), 0, st, (const int64_t *)pair_tot,
                       B, pair_offsets, total_copy);
    hipLaunchKernelGGL(row_offsets_scan, dim3(B), dim3(256), 0, st, row_count, n,
                       (const int64_t *)pair_offsets, row_off);
    return hipGetLastError();
}

hipError_t launch_plan_emit(const PlanArgs &p, const double *pair_thr, const int64_t *row_off,
                            const int32_t *row_count, int32_t *rows, int32_t *cols,
                            float *vals, double *row_loss, float *loss, float *dX,
                            const int64_t *gate, int64_t gate_cap, hipStream_t st)
{
    const bool lg = loss || dX;
    double *rl = loss ? row_loss : nullptr;
    if (p.d == 3 && !p.kb)
        return hipErrorInvalidValue;
    if (p.d <= 4) {
        const dim3 grid(ceil_div(p.n, kEmitRows), p.B), block(kEmitWaves * kWave);
        auto go = [&]<int DP, bool LG>() {
            if (p.dtype == 1)
                hipLaunchKernelGGL((emit_staged<uint16_t, DP, LG>), grid, block, 0, st, p,
                                   pair_thr, row_off, row_count, rows, cols, vals, rl, dX, gate, gate_cap);
            else
                hipLaunchKernelGGL((emit_staged<float, DP, LG>), grid, block, 0, st, p, pair_thr,
                                   row_off, row_count, rows, cols, vals, rl, dX, gate, gate_cap);
        };
        if (p.d == 3)
            lg ? go.template operator()<3, true>() : go.template operator()<3, false>();
        else
            lg ? go.template operator()<4, true>() : go.template operator()<4, false>();
    } else {
        const dim3 grid(ceil_div(p.n, kRowsPerGroup), p.B), block(kRowsPerGroup * kWave);
        auto go = [&]<int DP, bool LG>() {
            if (p.dtype == 1)
                hipLaunchKernelGGL((emit_pass<uint16_t, DP, LG>), grid, block, 0, st, p, pair_thr,
                                   row_off, row_count, rows, cols, vals, rl, dX, gate, gate_cap);
            else
                hipLaunchKernelGGL((emit_pass<float, DP, LG>), grid, block, 0, st, p, pair_thr,
                                   row_off, row_count, rows, cols, vals, rl, dX, gate, gate_cap);
        };
        with_dp(p.d, [&]<int DP>() {
            lg ? go.template operator()<DP, true>() : go.template operator()<DP, false>();
        });
    }
    if (loss)
        hipLaunchKernelGGL(pair_reduce<0>, dim3(p.B), dim3(256), 0, st, (const double *)row_loss,
                           p.n, loss, (double *)nullptr, 0.0, gate, gate_cap);
    return hipGetLastError();
}

hipError_t launch_dense_grad(const PlanArgs &p, float *grad, float *proj, const int *only,
                             hipStream_t st)
{
    tile_dispatch<3>(p, nullptr, nullptr, nullptr, grad, proj, st, only);
    return hipGetLastError();
}

}  // namespace sk

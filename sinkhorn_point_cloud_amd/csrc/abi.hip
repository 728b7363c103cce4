// abi.hip -- the C ABI declared in include/sinkhorn.h: argument checks,
// workspace carve-up, the eps-annealing driver and kernel launches.
#include "common.h"
#include "hvp.h"
#include "sinkhorn.h"
#include "sinkhorn_probe.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

namespace sk {
namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char *where)
{
    return fail(SK_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int kPad = 64;
constexpr int kMaxPoints = 1 << 24;
constexpr int kMaxPairs = 65535;     // pairs index a grid dimension (y or z), at most 65535
constexpr int kMaxNormDim = 4096;   // dimensions accepted by the normalisation

// Bump allocator over the caller's workspace (256-byte aligned pieces).
// Pieces of the caller's workspace, each at a 256-byte aligned address (the
// sizes add 256 bytes of slack for a workspace that starts unaligned).
struct Carve {
    char *base;
    size_t off = 0;
    template <typename T> T *take(size_t count)
    {
        const uintptr_t at = (uintptr_t)base + off;
        off += (((at + 255) & ~(uintptr_t)255) - at);
        T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
};

bool shape_ok(int B, int n, int m, int d)
{
    return B >= 1 && B <= kMaxPairs && n >= 1 && m >= 1 && d >= 1 && n <= kMaxPoints &&
           m <= kMaxPoints && (long long)B * n <= (1ll << 31) && (long long)B * m <= (1ll << 31);
}

bool path3(int dtype, int d) { return (dtype == SK_F32 || dtype == SK_BF16) && d == 3; }

bool supported(int dtype, int d) { return path3(dtype, d) || lseF_supported(dtype, d); }

// How the iterations of a d = 3 solve run on the current device (the value of
// sinkhorn_probe_potentials_path): 0 one launch per half-iteration on the
// matrix cores, 1 one launch per stage with a work-group per pair, 2 one
// launch per stage with each pair over 16-row work-groups, 3 one launch per
// half-iteration with vector scores.
int d3_launch_shape(int B, int n_pad, int m_pad, bool mfma)
{
    if (!mfma)
        return 3;
    if (lse3_pairwise(B, n_pad, m_pad))
        return 1;
    return lse3_split_parts(B, n_pad, m_pad) ? 2 : 0;
}

struct PotWs {
    // d = 3 path
    float4 *px = nullptr, *py = nullptr, *center = nullptr, *boxes = nullptr;
    uint16_t *kxrec = nullptr, *kyrec = nullptr, *qxrec = nullptr, *qyrec = nullptr;
    // feature path
    float *xbias = nullptr, *ybias = nullptr, *xsq = nullptr, *ysq = nullptr;
    // both: per 64-row block marks of rows to recompute
    int *xredo = nullptr, *yredo = nullptr;
    // d = 3: (tag, bias) words of the split stage launch
    uint64_t *xxch = nullptr, *yxch = nullptr;
    // both
    float *l2a, *l2b;
    float2 *part;
    double *row_part;
    double *la, *lb;   // fp64 log-weights for the cost pass
    KeyD *kd = nullptr;   // d = 3: fp64 keys of the cost pass
};

PotWs carve_potentials(Carve &c, int B, int n, int m, int d, int dtype)
{
    PotWs w;
    const int np = round_up(n, kPad), mp = round_up(m, kPad);
    size_t parts;
    if (path3(dtype, d)) {
        w.px = c.take<float4>((size_t)B * np);
        w.py = c.take<float4>((size_t)B * mp);
        w.center = c.take<float4>(B);
        w.kxrec = c.take<uint16_t>((size_t)B * np * kRec);
        w.kyrec = c.take<uint16_t>((size_t)B * mp * kRec);
        w.qxrec = c.take<uint16_t>((size_t)B * np * kRec);
        w.qyrec = c.take<uint16_t>((size_t)B * mp * kRec);
        w.boxes = c.take<float4>((size_t)2 * B * center3_parts(n, m));
        w.xredo = c.take<int>((size_t)B * (np / kPad));
        w.yredo = c.take<int>((size_t)B * (mp / kPad));
        w.xxch = c.take<uint64_t>((size_t)B * np);
        w.yxch = c.take<uint64_t>((size_t)B * mp);
        parts = std::max(lse3_partial_floats2(B, np, mp), lse3_partial_floats2(B, mp, np));
    } else {
        w.xbias = c.take<float>((size_t)B * np);
        w.ybias = c.take<float>((size_t)B * mp);
        w.xsq = c.take<float>((size_t)B * n);
        w.ysq = c.take<float>((size_t)B * m);
        w.xredo = c.take<int>((size_t)B * (np / kPad));
        w.yredo = c.take<int>((size_t)B * (mp / kPad));
        parts = std::max(lseF_partial_floats2(B, np, mp), lseF_partial_floats2(B, mp, np));
    }
    w.l2a = c.take<float>((size_t)B * n);
    w.l2b = c.take<float>((size_t)B * m);
    w.part = c.take<float2>(parts > 0 ? parts : 1);
    w.row_part = c.take<double>((size_t)B * n);
    w.la = c.take<double>((size_t)B * n);
    w.lb = c.take<double>((size_t)B * m);
    if (d == 3)
        w.kd = c.take<KeyD>((size_t)B * m);
    return w;
}

struct CooWs {
    double *la, *lb;
    double *row_max, *pair_thr;
    int32_t *row_count;
    int64_t *row_off, *pair_tot;
    KeyB *kb = nullptr;   // d = 3: fp64 keys of the max, count and emit passes
};

CooWs carve_coo(Carve &c, int B, int n, int m, int d)
{
    CooWs w;
    w.la = c.take<double>((size_t)B * n);
    w.lb = c.take<double>((size_t)B * m);
    w.row_max = c.take<double>((size_t)B * n);
    w.pair_thr = c.take<double>(B);
    w.row_count = c.take<int32_t>((size_t)B * n);
    w.row_off = c.take<int64_t>((size_t)B * n);
    w.pair_tot = c.take<int64_t>(B);
    if (d == 3)
        w.kb = c.take<KeyB>((size_t)B * m);
    return w;
}

struct LossWs {
    int64_t *begin, *end;
    double *row_loss;
};

LossWs carve_loss(Carve &c, int B, int n)
{
    LossWs w;
    w.begin = c.take<int64_t>((size_t)B * n);
    w.end = c.take<int64_t>((size_t)B * n);
    w.row_loss = c.take<double>((size_t)B * n);
    return w;
}

struct GradWs {
    double *la, *lb;
    KeyB *kbx = nullptr, *kby = nullptr;   // d = 3: fp64 keys of the two sides
    // matrix-core path (bf16, d = 32 or 64)
    float *xbias = nullptr, *ybias = nullptr, *xsq = nullptr, *ysq = nullptr;
    float *l2a = nullptr, *l2b = nullptr;
    uint16_t *xt = nullptr, *yt = nullptr;
    int *xredo = nullptr, *yredo = nullptr;
    GradFWs mc{nullptr, nullptr, nullptr};
};

GradWs carve_grad(Carve &c, int B, int n, int m, int d, int dtype)
{
    GradWs w;
    w.la = c.take<double>((size_t)B * n);
    w.lb = c.take<double>((size_t)B * m);
    if (d == 3) {
        w.kbx = c.take<KeyB>((size_t)B * n);
        w.kby = c.take<KeyB>((size_t)B * m);
    }
    if (gradF_matrix_cores(dtype, d)) {
        const int np = round_up(n, kGradPad), mp = round_up(m, kGradPad);
        w.xbias = c.take<float>((size_t)B * np);
        w.ybias = c.take<float>((size_t)B * mp);
        w.xsq = c.take<float>((size_t)B * n);
        w.ysq = c.take<float>((size_t)B * m);
        w.l2a = c.take<float>((size_t)B * n);
        w.l2b = c.take<float>((size_t)B * m);
        w.xt = c.take<uint16_t>((size_t)B * d * np);
        w.yt = c.take<uint16_t>((size_t)B * d * mp);
        w.xredo = c.take<int>((size_t)B * ceil_div(n, kPad));
        w.yredo = c.take<int>((size_t)B * ceil_div(m, kPad));
        const GradFSizes z = gradF_sizes(B, n, m, d);
        w.mc.h = c.take<float>(z.h);
        w.mc.part_s = c.take<float>(z.part_s);
        w.mc.part_v = c.take<float>(z.part_v);
    }
    return w;
}

CooNormWs carve_coo_norm(Carve &c, int B, int n, int m, int64_t nnz)
{
    CooNormWs w;
    w.rb = c.take<int64_t>((size_t)B * n);
    w.re = c.take<int64_t>((size_t)B * n);
    w.cb = c.take<int64_t>((size_t)B * m);
    w.ce = c.take<int64_t>((size_t)B * m);
    w.lv = c.take<float>(nnz > 0 ? (size_t)nnz : 1);
    w.lvt = c.take<float>(nnz > 0 ? (size_t)nnz : 1);
    w.al = c.take<double>((size_t)B * n);
    w.la = c.take<double>((size_t)B * n);
    w.be = c.take<double>((size_t)B * m);
    w.lb = c.take<double>((size_t)B * m);
    w.row_part = c.take<double>((size_t)B * n);
    w.col_part = c.take<double>((size_t)B * m);
    w.sums = c.take<uint64_t>((size_t)2 * B);
    w.bad = c.take<int>(1);
    return w;
}

constexpr int kMaxHvpDim = 16;

HvpWs carve_hvp(Carve &c, int B, int n, int m, int d)
{
    HvpWs w;
    const size_t Bn = (size_t)B * n, Bm = (size_t)B * m;
    w.la = c.take<double>(Bn);
    w.lb = c.take<double>(Bm);
    w.ma = c.take<double>(Bn);
    w.tv = c.take<double>(Bn);
    w.ur = c.take<double>(Bn);
    w.mur = c.take<double>(Bn);
    w.D1 = c.take<double>(Bn * d);
    w.Tv = c.take<double>(Bn * d);
    w.Du = c.take<double>(Bn * d);
    w.mb = c.take<double>(Bm);
    w.muc = c.take<double>(Bm);
    w.tw = c.take<double>(Bm);
    w.rhs = c.take<double>(Bm);
    w.x = c.take<double>(Bm);
    w.res = c.take<double>(Bm);
    w.dir = c.take<double>(Bm);
    w.rr = c.take<double>(B);
    w.rr0 = c.take<double>(B);
    if (d == 3) {
        w.kbx = c.take<KeyB>(Bn);
        w.kby = c.take<KeyB>(Bm);
    }
    return w;
}

HvpFeatWs carve_hvp_feat(Carve &c, int B, int n, int m, int d)
{
    HvpFeatWs w;
    const int np = round_up(n, kHvpPad), mp = round_up(m, kHvpPad);
    const size_t Bn = (size_t)B * n, Bm = (size_t)B * m, Bnp = (size_t)B * np,
                 Bmp = (size_t)B * mp;
    const HvpFeatSizes z = hvp_feat_sizes(B, n, m, d);
    w.y.pts = nullptr;
    w.y.bias = c.take<float>(Bmp);
    w.y.pot = nullptr;
    w.y.l2w = c.take<float>(Bm);
    w.y.sq = c.take<float>(Bm);
    w.y.redo = nullptr;
    w.y.n = m;
    w.y.n_pad = mp;
    w.yt = c.take<uint16_t>(Bmp * d);
    w.h = c.take<float>(Bnp);
    w.wa = c.take<float>(Bnp);
    w.wu = c.take<float>(Bnp);
    w.wt = c.take<float>(Bnp);
    w.vh = c.take<uint16_t>(Bnp * d);
    w.vl = c.take<uint16_t>(Bnp * d);
    w.vth = c.take<uint16_t>(Bnp * d);
    w.vtl = c.take<uint16_t>(Bnp * d);
    w.u32 = c.take<float>(Bmp);
    w.x32 = c.take<float>(Bmp);
    w.part_r = c.take<float>(z.part_r);
    w.part_rv = c.take<float>(z.part_rv);
    w.part_rq = c.take<float>(z.part_rv);
    w.part_c = c.take<float>(z.part_c);
    w.part_cv = c.take<float>(z.part_cv);
    w.mrow = c.take<double>(Bn);
    w.ma = c.take<double>(Bn);
    w.tv = c.take<double>(Bn);
    w.D1 = c.take<double>(Bn * d);
    w.Tv = c.take<double>(Bn * d);
    w.mb = c.take<double>(Bm);
    w.rhs = c.take<double>(Bm);
    w.x = c.take<double>(Bm);
    w.res = c.take<double>(Bm);
    w.dir = c.take<double>(Bm);
    w.rr = c.take<double>((size_t)2 * B);
    w.rr0 = c.take<double>(B);
    const size_t nred = (size_t)B * cg_wide_blocks(m);
    w.red_pq = c.take<double>(nred);
    w.red_s = c.take<double>(nred);
    w.red_q = c.take<double>(nred);
    w.bad = c.take<int>(B);
    return w;
}

size_t ws_size(int op, int B, int n, int m, int d, int dtype)
{
    Carve c{nullptr};
    if (op == SK_OP_POTENTIALS)
        carve_potentials(c, B, n, m, d, dtype);
    else if (op == SK_OP_PLAN_COO)
        carve_coo(c, B, n, m, d);
    else if (op == SK_OP_LOSS_GRAD)
        carve_loss(c, B, n);
    else if (op == SK_OP_DENSE_GRAD)
        carve_grad(c, B, n, m, d, dtype);
    else if (hvp_matrix_cores(dtype, d))
        carve_hvp_feat(c, B, n, m, d);
    else
        carve_hvp(c, B, n, m, d);
    return c.off + 256;
}

int check_ws(void *ws, size_t ws_bytes, size_t need)
{
    if (!ws || ws_bytes < need)
        return fail(SK_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need,
                    ws_bytes, ws ? "" : " (ws is NULL)");
    return SK_OK;
}

int check_common(const void *X, const void *Y, int dtype, int B, int n, int m, int d)
{
    if (!X || !Y)
        return fail(SK_ERR_INVALID_ARG, "X and Y must be non-NULL device pointers");
    if (dtype != SK_F32 && dtype != SK_BF16)
        return fail(SK_ERR_INVALID_ARG, "dtype %d is neither SK_F32 nor SK_BF16", dtype);
    if (!shape_ok(B, n, m, d))
        return fail(SK_ERR_INVALID_ARG, "bad sizes B=%d n=%d m=%d d=%d", B, n, m, d);
    if (!supported(dtype, d))
        return fail(SK_ERR_UNSUPPORTED, "no kernel for dtype %d with d=%d", dtype, d);
    return SK_OK;
}

// Argument checks of the potentials entry points (no HIP call).
int check_potentials(const void *X, const void *Y, int dtype, int B, int n, int m, int d,
                     const float *eps, const int *iters, int n_stages, unsigned flags,
                     const float *f, const float *g, const float *cost)
{
    int rc = check_common(X, Y, dtype, B, n, m, d);
    if (rc)
        return rc;
    if (!f || !g)
        return fail(SK_ERR_INVALID_ARG, "f and g must be non-NULL device pointers");
    if (n_stages < 0 || (n_stages > 0 && (!eps || !iters)))
        return fail(SK_ERR_INVALID_ARG, "n_stages=%d needs host arrays eps and iters", n_stages);
    if (flags & ~(SK_WARM_START | SK_VALU_SCORES))
        return fail(SK_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    for (int s = 0; s < n_stages; ++s) {
        if (!(eps[s] > 0.f) || !isfinite(eps[s]))
            return fail(SK_ERR_INVALID_ARG, "eps[%d]=%g must be finite and > 0", s, eps[s]);
        if (iters[s] < 0)
            return fail(SK_ERR_INVALID_ARG, "iters[%d]=%d must be >= 0", s, iters[s]);
    }
    if (cost && n_stages == 0)
        return fail(SK_ERR_INVALID_ARG, "cost needs an eps (n_stages >= 1)");
    return SK_OK;
}

// The eps-annealing driver over a workspace of ws_size(SK_OP_POTENTIALS, ...) bytes.
int run_potentials(const void *X, const void *Y, int dtype, const float *a, const float *b,
                   int B, int n, int m, int d, const float *eps, const int *iters, int n_stages,
                   unsigned flags, float *f, float *g, float *cost, void *ws, void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    Carve c{(char *)ws};
    PotWs w = carve_potentials(c, B, n, m, d, dtype);
    const int warm = (flags & SK_WARM_START) ? 1 : 0;
    const bool mfma = !(flags & SK_VALU_SCORES);
    const int np = round_up(n, kPad), mp = round_up(m, kPad);

    // eps of every half-iteration, in order
    int first = -1;
    for (int s = 0; s < n_stages; ++s)
        if (iters[s] > 0) {
            first = s;
            break;
        }
    const double c0 = (double)scale_of(first >= 0 ? eps[first] : 1.0f);
    hipError_t e;
    const bool p3 = path3(dtype, d);
    const int shape = p3 ? d3_launch_shape(B, np, mp, mfma) : -1;
    const bool pairwise = shape == 1;
    // work-groups per pair of the split stage launch (0: not used)
    const int split = shape == 2 ? lse3_split_parts(B, np, mp) : 0;
    // the caller's f and g are the state of the iteration
    Side3 sx3{w.px, f, w.l2a, w.kxrec, w.qxrec, n, np, w.xredo, split ? w.xxch : nullptr};
    Side3 sy3{w.py, g, w.l2b, w.kyrec, w.qyrec, m, mp, w.yredo, split ? w.yxch : nullptr};
    SideF sxf{X, w.xbias, f, w.l2a, w.xsq, w.xredo, n, np};
    SideF syf{Y, w.ybias, g, w.l2b, w.ysq, w.yredo, m, mp};
    if (p3) {
        if ((e = launch_center3(X, dtype, n, Y, m, B, w.boxes, w.center, st)))
            return hip_fail(e, "center");
        if ((e = launch_pack3(X, dtype, a, warm, B, sx3, w.center, c0, st)))
            return hip_fail(e, "pack X");
        if ((e = launch_pack3(Y, dtype, b, warm, B, sy3, w.center, c0, st)))
            return hip_fail(e, "pack Y");
    } else {
        if ((e = launch_packF(X, dtype, d, a, warm, B, sxf, c0, st)))
            return hip_fail(e, "pack X");
        if ((e = launch_packF(Y, dtype, d, b, warm, B, syf, c0, st)))
            return hip_fail(e, "pack Y");
    }
    for (int s = 0; s < n_stages; ++s) {
        if (p3 && mfma && iters[s] > 0) {
            // query records carry 2c x, so they follow eps
            if ((e = launch_qrec3(sx3, B, eps[s], st)) || (e = launch_qrec3(sy3, B, eps[s], st)))
                return hip_fail(e, "query records");
        }
        if (p3 && mfma && iters[s] > 0 && (pairwise || split)) {
            float eps_next = eps[s];   // eps of the f-update after the stage's last g-update
            for (int t = s + 1; t < n_stages; ++t)
                if (iters[t] > 0) {
                    eps_next = eps[t];
                    break;
                }
            const bool cold = !warm && s == first;
            if ((e = pairwise ? launch_lse3_pairwise(sx3, sy3, B, eps[s], iters[s], eps_next,
                                                     cold, st)
                              : launch_lse3_split(sx3, sy3, B, split, eps[s], iters[s], eps_next,
                                                  cold, st)))
                return hip_fail(e, "iterations");
            continue;
        }
        for (int it = 0; it < iters[s]; ++it) {
            // eps of the f-update that follows this g-update
            float eps_next = eps[s];
            if (it == iters[s] - 1)
                for (int t = s + 1; t < n_stages; ++t)
                    if (iters[t] > 0) {
                        eps_next = eps[t];
                        break;
                    }
            if (p3) {
                if ((e = launch_lse3(sx3, sy3, B, eps[s], eps[s], w.part, mfma, st)))
                    return hip_fail(e, "f-update");
                if ((e = launch_lse3(sy3, sx3, B, eps[s], eps_next, w.part, mfma, st)))
                    return hip_fail(e, "g-update");
            } else {
                if ((e = launch_lseF(sxf, syf, dtype, d, B, eps[s], eps[s], w.part, st)))
                    return hip_fail(e, "f-update");
                if ((e = launch_lseF(syf, sxf, dtype, d, B, eps[s], eps_next, w.part, st)))
                    return hip_fail(e, "g-update");
            }
        }
    }
    if (cost && !p3 && iters[n_stages - 1] > 0 && lseF_matrix_cores(sxf, syf, dtype, d, B)) {
        // the final passes left both biases at the last eps: stream the cost on the
        // matrix cores like a half-iteration
        if ((e = launch_costFm(sxf, syf, d, B, eps[n_stages - 1], w.row_part, st)) ||
            (e = launch_row_sums(w.row_part, B, n, cost, st)))
            return hip_fail(e, "cost");
    } else if (cost) {
        PlanArgs p{X, Y, dtype, d, B, n, m, f, g, w.la, w.lb, 1.0 / (double)eps[n_stages - 1], w.kd};
        if ((e = launch_log_weights(a, B, n, w.la, st)) ||
            (e = launch_log_weights(b, B, m, w.lb, st)) ||
            (w.kd && (e = launch_keys_d3(Y, dtype, g, B, m, w.kd, st))))
            return hip_fail(e, "log weights");
        if ((e = launch_cost(p, w.row_part, cost, st)))
            return hip_fail(e, "cost");
    }
    return SK_OK;
}

// Workspace of sinkhorn_potentials_noalloc: a device array that lives in the
// library's code object, one copy per GPU the library runs on, held until the
// process ends.  Host code never uses the name `scratch` as an address (on the
// host it is only a stand-in for the symbol): the device address of each GPU's
// copy is resolved once, with that GPU current, and kept in g_scratch.
constexpr size_t kScratchBytes = SK_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of the current GPU's copy of `scratch`.
int scratch_address(void *stream, void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (stream) {
        hipDevice_t sdev = 0;
        if ((e = hipStreamGetDevice((hipStream_t)stream, &sdev)) != hipSuccess)
            return hip_fail(e, "hipStreamGetDevice");
        if ((int)sdev != dev)
            return fail(SK_ERR_INVALID_ARG, "stream belongs to device %d, the current device is %d",
                        (int)sdev, dev);
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SK_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p)
            return fail(SK_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SK_OK;
}

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" {

size_t sinkhorn_workspace_bytes(int op, int B, int n, int m, int d, int dtype)
{
    if (op < SK_OP_POTENTIALS || op > SK_OP_HVP || !shape_ok(B, n, m, d) ||
        (op == SK_OP_HVP && d > kMaxHvpDim && !hvp_matrix_cores(dtype, d)) ||
        (dtype != SK_F32 && dtype != SK_BF16) || !supported(dtype, d))
        return 0;
    return ws_size(op, B, n, m, d, dtype);
}

const char *sinkhorn_status_string(int s)
{
    switch (s) {
    case SK_OK: return "ok";
    case SK_ERR_INVALID_ARG: return "invalid argument";
    case SK_ERR_UNSUPPORTED: return "unsupported dtype/dimension";
    case SK_ERR_WORKSPACE: return "workspace missing or too small";
    case SK_ERR_CAPACITY: return "sparse plan exceeds capacity";
    case SK_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *sinkhorn_last_error(void) { return g_err; }

int sinkhorn_probe_potentials_path(int B, int n, int m, int d, int dtype, unsigned flags)
{
    if (!shape_ok(B, n, m, d) || !supported(dtype, d))
        return -1;
    if (!path3(dtype, d))
        return 4;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return -2;
    return d3_launch_shape(B, round_up(n, kPad), round_up(m, kPad), !(flags & SK_VALU_SCORES));
}

int sinkhorn_potentials(const void *X, const void *Y, int dtype, const float *a, const float *b,
                        int B, int n, int m, int d, const float *eps, const int *iters,
                        int n_stages, unsigned flags, float *f, float *g, float *cost, void *ws,
                        size_t ws_bytes, void *stream)
{
    g_err[0] = '\0';
    int rc = check_potentials(X, Y, dtype, B, n, m, d, eps, iters, n_stages, flags, f, g, cost);
    if (rc)
        return rc;
    rc = check_ws(ws, ws_bytes, ws_size(SK_OP_POTENTIALS, B, n, m, d, dtype));
    if (rc)
        return rc;
    return run_potentials(X, Y, dtype, a, b, B, n, m, d, eps, iters, n_stages, flags, f, g, cost,
                          ws, stream);
}

int sinkhorn_potentials_noalloc(const void *X, const void *Y, int dtype, const float *a,
                                const float *b, int B, int n, int m, int d, const float *eps,
                                const int *iters, int n_stages, unsigned flags, float *f,
                                float *g, float *cost, void *stream)
{
    g_err[0] = '\0';
    int rc = check_potentials(X, Y, dtype, B, n, m, d, eps, iters, n_stages, flags, f, g, cost);
    if (rc)
        return rc;
    const size_t need = ws_size(SK_OP_POTENTIALS, B, n, m, d, dtype);
    if (need > kScratchBytes)
        return fail(SK_ERR_WORKSPACE,
                    "these sizes need %zu bytes of scratch, the static scratch holds %zu "
                    "(use sinkhorn_potentials with a workspace)",
                    need, kScratchBytes);
    void *ws = nullptr;
    if ((rc = scratch_address(stream, &ws)))
        return rc;
    return run_potentials(X, Y, dtype, a, b, B, n, m, d, eps, iters, n_stages, flags, f, g, cost,
                          ws, stream);
}

int sinkhorn_plan_coo(const void *X, const void *Y, int dtype, const float *a, const float *b,
                      int B, int n, int m, int d, float eps, const float *f, const float *g,
                      float rel_threshold, int64_t capacity, int32_t *rows, int32_t *cols,
                      float *vals, int64_t *pair_offsets, float *loss, float *dX,
                      int64_t *nnz_total, void *ws, size_t ws_bytes, void *stream)
{
    g_err[0] = '\0';
    int rc = check_common(X, Y, dtype, B, n, m, d);
    if (rc)
        return rc;
    if (!f || !g || !pair_offsets || !nnz_total)
        return fail(SK_ERR_INVALID_ARG, "f, g, pair_offsets and nnz_total must be non-NULL");
    if (!(eps > 0.f) || !isfinite(eps))
        return fail(SK_ERR_INVALID_ARG, "eps=%g must be finite and > 0", eps);
    if (!(rel_threshold > 0.f && rel_threshold <= 1.f))
        return fail(SK_ERR_INVALID_ARG, "rel_threshold=%g must be in (0, 1]", rel_threshold);
    if (capacity < 0 || (capacity > 0 && (!rows || !cols || !vals)))
        return fail(SK_ERR_INVALID_ARG, "capacity=%lld needs rows, cols and vals",
                    (long long)capacity);
    rc = check_ws(ws, ws_bytes, ws_size(SK_OP_PLAN_COO, B, n, m, d, dtype));
    if (rc)
        return rc;

    hipStream_t st = (hipStream_t)stream;
    Carve c{(char *)ws};
    CooWs w = carve_coo(c, B, n, m, d);
    PlanArgs p{X, Y, dtype, d, B, n, m, f, g, w.la, w.lb, 1.0 / (double)eps};
    p.kb = w.kb;
    hipError_t e;
    if ((e = launch_plan_prep(a, b, B, n, m, w.la, w.lb, X, Y, dtype, f, g, p.inv_eps, 1.0,
                              nullptr, w.kb, st)))
        return hip_fail(e, "log weights");
    if ((e = launch_plan_max(p, w.row_max, w.pair_thr, log((double)rel_threshold), st)))
        return hip_fail(e, "plan max");
    if ((e = launch_plan_count(p, w.pair_thr, w.row_count, st)))
        return hip_fail(e, "plan count");
    if ((e = launch_plan_scan(w.row_count, B, n, w.row_off, pair_offsets, w.pair_tot, nullptr,
                              st)))
        return hip_fail(e, "plan scan");
    int64_t total = 0;
    if ((e = hipMemcpyAsync(&total, pair_offsets + B, sizeof total, hipMemcpyDeviceToHost, st)))
        return hip_fail(e, "read nnz");
    if ((e = hipStreamSynchronize(st)))
        return hip_fail(e, "sync for nnz");
    *nnz_total = total;
    if (total > capacity)
        return fail(SK_ERR_CAPACITY, "sparse plan has %lld entries, capacity is %lld",
                    (long long)total, (long long)capacity);
    // row_max is free once the threshold is known: it takes the per-row loss
    if ((total > 0 || loss || dX) &&
        (e = launch_plan_emit(p, w.pair_thr, w.row_off, w.row_count, rows, cols, vals, w.row_max,
                              loss, dX, nullptr, 0, st)))
        return hip_fail(e, "plan emit");
    return SK_OK;
}

int sinkhorn_plan_coo_async(const void *X, const void *Y, int dtype, const float *a,
                            const float *b, int B, int n, int m, int d, float eps, const float *f,
                            const float *g, float rel_threshold, int64_t capacity, int32_t *rows,
                            int32_t *cols, float *vals, int64_t *pair_offsets, float *loss,
                            float *dX, int64_t *nnz_device, void *ws, size_t ws_bytes,
                            void *stream)
{
    g_err[0] = '\0';
    int rc = check_common(X, Y, dtype, B, n, m, d);
    if (rc)
        return rc;
    if (!f || !g || !pair_offsets || !nnz_device)
        return fail(SK_ERR_INVALID_ARG, "f, g, pair_offsets and nnz_device must be non-NULL");
    if (!(eps > 0.f) || !isfinite(eps))
        return fail(SK_ERR_INVALID_ARG, "eps=%g must be finite and > 0", eps);
    if (!(rel_threshold > 0.f && rel_threshold <= 1.f))
        return fail(SK_ERR_INVALID_ARG, "rel_threshold=%g must be in (0, 1]", rel_threshold);
    if (capacity < 1 || !rows || !cols || !vals)
        return fail(SK_ERR_INVALID_ARG, "capacity=%lld must be >= 1 with rows, cols and vals",
                    (long long)capacity);
    rc = check_ws(ws, ws_bytes, ws_size(SK_OP_PLAN_COO, B, n, m, d, dtype));
    if (rc)
        return rc;

    hipStream_t st = (hipStream_t)stream;
    Carve c{(char *)ws};
    CooWs w = carve_coo(c, B, n, m, d);
    PlanArgs p{X, Y, dtype, d, B, n, m, f, g, w.la, w.lb, 1.0 / (double)eps};
    p.kb = w.kb;
    hipError_t e;
    if ((e = launch_plan_prep(a, b, B, n, m, w.la, w.lb, X, Y, dtype, f, g, p.inv_eps, 1.0,
                              nullptr, w.kb, st)))
        return hip_fail(e, "log weights");
    if ((e = launch_plan_max(p, w.row_max, w.pair_thr, log((double)rel_threshold), st)) ||
        (e = launch_plan_count(p, w.pair_thr, w.row_count, st)) ||
        (e = launch_plan_scan(w.row_count, B, n, w.row_off, pair_offsets, w.pair_tot,
                              nnz_device, st)))
        return hip_fail(e, "plan count");
    if ((e = launch_plan_emit(p, w.pair_thr, w.row_off, w.row_count, rows, cols, vals, w.row_max,
                              loss, dX, pair_offsets + B, capacity, st)))
        return hip_fail(e, "plan emit");
    return SK_OK;
}

int sinkhorn_loss_grad(const void *X, const void *Y, int dtype, int B, int n, int m, int d,
                       const int32_t *rows, const int32_t *cols, const float *vals,
                       const int64_t *pair_offsets, float *loss, float *dX, void *ws,
                       size_t ws_bytes, void *stream)
{
    g_err[0] = '\0';
    int rc = check_common(X, Y, dtype, B, n, m, d);
    if (rc)
        return rc;
    if (!rows || !cols || !vals || !pair_offsets || !loss)
        return fail(SK_ERR_INVALID_ARG, "rows, cols, vals, pair_offsets and loss must be non-NULL");
    rc = check_ws(ws, ws_bytes, ws_size(SK_OP_LOSS_GRAD, B, n, m, d, dtype));
    if (rc)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    Carve c{(char *)ws};
    LossWs w = carve_loss(c, B, n);
    hipError_t e = launch_loss_grad(X, Y, dtype, d, B, n, m, rows, cols, vals, pair_offsets,
                                    w.begin, w.end, w.row_loss, loss, dX, st);
    if (e)
        return hip_fail(e, "loss/grad");
    return SK_OK;
}

int sinkhorn_dense_grad(const void *X, const void *Y, int dtype, const float *a, const float *b,
                        int B, int n, int m, int d, float eps, const float *f, const float *g,
                        float *dX, float *TX, float *dY, float *TY, void *ws, size_t ws_bytes,
                        void *stream)
{
    g_err[0] = '\0';
    int rc = check_common(X, Y, dtype, B, n, m, d);
    if (rc)
        return rc;
    if (!f || !g)
        return fail(SK_ERR_INVALID_ARG, "f and g must be non-NULL device pointers");
    if (!(eps > 0.f) || !isfinite(eps))
        return fail(SK_ERR_INVALID_ARG, "eps=%g must be finite and > 0", eps);
    rc = check_ws(ws, ws_bytes, ws_size(SK_OP_DENSE_GRAD, B, n, m, d, dtype));
    if (rc)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    Carve c{(char *)ws};
    GradWs w = carve_grad(c, B, n, m, d, dtype);
    hipError_t e;
    const double inv_eps = 1.0 / (double)eps;
    const bool want_x = dX || TX, want_y = dY || TY;
    // log weights and, for d = 3, the key records of the sides in use
    if ((e = launch_plan_prep(a, b, B, n, m, w.la, w.lb, X, Y, dtype, f, g, inv_eps, kLog2eD,
                              want_y ? w.kbx : nullptr, want_x ? w.kby : nullptr, st)))
        return hip_fail(e, "log weights");
    // log P is symmetric in (X, a, f) and (Y, b, g): the Y side is the same pass
    PlanArgs px{X, Y, dtype, d, B, n, m, f, g, w.la, w.lb, inv_eps};
    PlanArgs py{Y, X, dtype, d, B, m, n, g, f, w.lb, w.la, inv_eps};
    px.kb = w.kby;
    py.kb = w.kbx;
    const bool aligned = (uintptr_t)X % 16 == 0 && (uintptr_t)Y % 16 == 0;
    if (gradF_matrix_cores(dtype, d) && aligned) {
        const int np = round_up(n, kGradPad), mp = round_up(m, kGradPad);
        // potentials are only read (warm start): biases c (pot - ||.||^2) + log2 w at eps
        SideF sx{X, w.xbias, const_cast<float *>(f), w.l2a, w.xsq, w.xredo, n, np};
        SideF sy{Y, w.ybias, const_cast<float *>(g), w.l2b, w.ysq, w.yredo, m, mp};
        const double c0 = (double)scale_of(eps);
        if ((e = launch_packF(X, dtype, d, a, 1, B, sx, c0, st)) ||
            (e = launch_packF(Y, dtype, d, b, 1, B, sy, c0, st)))
            return hip_fail(e, "dense gradient: biases");
        if (want_x) {
            if ((e = launch_transpose_bf16(Y, B, m, mp, d, w.yt, st)) ||
                (e = launch_gradF(sx, a, sy, w.yt, d, B, eps, w.mc, dX, TX, st)) ||
                (e = launch_dense_grad(px, dX, TX, w.xredo, st)))
                return hip_fail(e, "dense gradient (X side)");
        }
        if (want_y) {
            if ((e = launch_transpose_bf16(X, B, n, np, d, w.xt, st)) ||
                (e = launch_gradF(sy, b, sx, w.xt, d, B, eps, w.mc, dY, TY, st)) ||
                (e = launch_dense_grad(py, dY, TY, w.yredo, st)))
                return hip_fail(e, "dense gradient (Y side)");
        }
        return SK_OK;
    }
    if (want_x && (e = launch_dense_grad(px, dX, TX, nullptr, st)))
        return hip_fail(e, "dense gradient (X side)");
    if (want_y && (e = launch_dense_grad(py, dY, TY, nullptr, st)))
        return hip_fail(e, "dense gradient (Y side)");
    return SK_OK;
}

int sinkhorn_hvp(const void *X, const void *Y, int dtype, const float *a, const float *b, int B,
                 int n, int m, int d, float eps, const float *f, const float *g, const float *V,
                 int cg_iters, float *HV, float *cg_residual, void *ws, size_t ws_bytes,
                 void *stream)
{
    g_err[0] = '\0';
    int rc = check_common(X, Y, dtype, B, n, m, d);
    if (rc)
        return rc;
    const bool mfma = hvp_matrix_cores(dtype, d);
    if (d > kMaxHvpDim && !mfma)
        return fail(SK_ERR_UNSUPPORTED,
                    "Hessian-vector products need d <= %d, or bf16 points with d = 32 or 64 "
                    "(d=%d)",
                    kMaxHvpDim, d);
    if (mfma && ((uintptr_t)X % 16 != 0 || (uintptr_t)Y % 16 != 0))
        return fail(SK_ERR_INVALID_ARG,
                    "Hessian-vector products of bf16 points with d = %d need X and Y at "
                    "16-byte aligned addresses",
                    d);
    if (!f || !g || !V || !HV)
        return fail(SK_ERR_INVALID_ARG, "f, g, V and HV must be non-NULL device pointers");
    if (!(eps > 0.f) || !isfinite(eps))
        return fail(SK_ERR_INVALID_ARG, "eps=%g must be finite and > 0", eps);
    if (cg_iters < 0)
        return fail(SK_ERR_INVALID_ARG, "cg_iters=%d must be >= 0", cg_iters);
    rc = check_ws(ws, ws_bytes, ws_size(SK_OP_HVP, B, n, m, d, dtype));
    if (rc)
        return rc;
    hipStream_t st = (hipStream_t)stream;
    Carve c{(char *)ws};
    hipError_t e;
    if (mfma) {
        HvpFeatWs w = carve_hvp_feat(c, B, n, m, d);
        if ((e = launch_hvp_feat(X, Y, a, b, f, g, V, B, n, m, d, eps, cg_iters, HV, cg_residual,
                                 w, st)))
            return hip_fail(e, "Hessian-vector product (matrix cores)");
        return SK_OK;
    }
    HvpWs w = carve_hvp(c, B, n, m, d);
    const double inv_eps = 1.0 / (double)eps;
    if ((e = launch_plan_prep(a, b, B, n, m, w.la, w.lb, X, Y, dtype, f, g, inv_eps, kLog2eD,
                              w.kbx, w.kby, st)))
        return hip_fail(e, "log weights");
    PlanArgs px{X, Y, dtype, d, B, n, m, f, g, w.la, w.lb, inv_eps};
    PlanArgs py{Y, X, dtype, d, B, m, n, g, f, w.lb, w.la, inv_eps};
    px.kb = w.kby;
    py.kb = w.kbx;
    if ((e = launch_hvp(px, py, V, cg_iters, HV, cg_residual, w, st)))
        return hip_fail(e, "Hessian-vector product");
    return SK_OK;
}

size_t sinkhorn_coo_workspace_bytes(int B, int n, int m, int64_t nnz)
{
    if (B < 1 || B > kMaxPairs || n < 1 || m < 1 || nnz < 0 || n > kMaxPoints || m > kMaxPoints ||
        (long long)B * n > (1ll << 31) || (long long)B * m > (1ll << 31))
        return 0;
    Carve c{nullptr};
    carve_coo_norm(c, B, n, m, nnz);
    return c.off + 256;
}

int sinkhorn_coo_normalize(int B, int n, int m, const int32_t *rows, const int32_t *cols,
                           float *vals, const int64_t *pair_offsets, const int32_t *t_rows,
                           const int32_t *t_cols, float *t_vals, const int64_t *t_pair_offsets,
                           const float *a, const float *b, int iters, float *err, void *ws,
                           size_t ws_bytes, void *stream)
{
    g_err[0] = '\0';
    if (B < 1 || B > kMaxPairs || n < 1 || m < 1 || n > kMaxPoints || m > kMaxPoints ||
        (long long)B * n > (1ll << 31) || (long long)B * m > (1ll << 31))
        return fail(SK_ERR_INVALID_ARG, "bad sizes B=%d n=%d m=%d", B, n, m);
    if (!rows || !cols || !vals || !pair_offsets || !t_rows || !t_cols || !t_vals ||
        !t_pair_offsets)
        return fail(SK_ERR_INVALID_ARG, "the plan, its transpose and both offset arrays must be "
                                        "non-NULL device pointers");
    if (iters < 0)
        return fail(SK_ERR_INVALID_ARG, "iters=%d must be >= 0", iters);
    hipStream_t st = (hipStream_t)stream;
    int64_t tot[2] = {0, 0};
    hipError_t e;
    if ((e = hipMemcpyAsync(&tot[0], pair_offsets + B, sizeof(int64_t), hipMemcpyDeviceToHost,
                            st)) ||
        (e = hipMemcpyAsync(&tot[1], t_pair_offsets + B, sizeof(int64_t), hipMemcpyDeviceToHost,
                            st)) ||
        (e = hipStreamSynchronize(st)))
        return hip_fail(e, "read entry counts");
    if (tot[0] != tot[1] || tot[0] < 0)
        return fail(SK_ERR_INVALID_ARG, "plan has %lld entries, its transpose %lld",
                    (long long)tot[0], (long long)tot[1]);
    const int64_t nnz = tot[0];
    if (!ws || ws_bytes < sinkhorn_coo_workspace_bytes(B, n, m, nnz))
        return fail(SK_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
                    sinkhorn_coo_workspace_bytes(B, n, m, nnz), ws_bytes);
    Carve c{(char *)ws};
    CooNormWs w = carve_coo_norm(c, B, n, m, nnz);
    if ((e = launch_log_weights(a, B, n, w.la, st)) || (e = launch_log_weights(b, B, m, w.lb, st)) ||
        (e = launch_segment_bounds(rows, pair_offsets, B, n, w.rb, w.re, st)) ||
        (e = launch_segment_bounds(t_rows, t_pair_offsets, B, m, w.cb, w.ce, st)) ||
        (e = launch_coo_check(rows, cols, vals, pair_offsets, t_rows, t_cols, t_vals,
                              t_pair_offsets, B, w, st)))
        return hip_fail(e, "coo normalisation set-up");
    int bad = 0;
    if ((e = hipMemcpyAsync(&bad, w.bad, sizeof bad, hipMemcpyDeviceToHost, st)) ||
        (e = hipStreamSynchronize(st)))
        return hip_fail(e, "read transpose check");
    if (bad)
        return fail(SK_ERR_INVALID_ARG,
                    "the transpose does not hold the plan's entries and values in %d pair(s)", bad);
    if ((e = launch_coo_normalize(rows, cols, vals, pair_offsets, t_rows, t_cols, t_vals,
                                  t_pair_offsets, B, n, m, nnz, iters, err, a, b, w, st)))
        return hip_fail(e, "coo normalisation");
    return SK_OK;
}

int sinkhorn_normalize(const void *X, int dtype, int B, int n, int d, float *Xh, float *norms,
                       void *stream)
{
    g_err[0] = '\0';
    if (!X || !Xh || !norms)
        return fail(SK_ERR_INVALID_ARG, "X, Xh and norms must be non-NULL device pointers");
    if (dtype != SK_F32 && dtype != SK_BF16)
        return fail(SK_ERR_INVALID_ARG, "dtype %d is neither SK_F32 nor SK_BF16", dtype);
    if (B < 1 || n < 1 || d < 1 || d > kMaxNormDim || (long long)B * n > (1ll << 31))
        return fail(SK_ERR_INVALID_ARG, "bad sizes B=%d n=%d d=%d", B, n, d);
    hipError_t e = launch_normalize(X, dtype, (long)B * n, d, Xh, norms, (hipStream_t)stream);
    return e ? hip_fail(e, "normalize") : SK_OK;
}

int sinkhorn_normalize_backward(const float *Xh, const float *norms, const float *G, int B, int n,
                                int d, float *dX, void *stream)
{
    g_err[0] = '\0';
    if (!Xh || !norms || !G || !dX)
        return fail(SK_ERR_INVALID_ARG, "Xh, norms, G and dX must be non-NULL device pointers");
    if (B < 1 || n < 1 || d < 1 || d > kMaxNormDim || (long long)B * n > (1ll << 31))
        return fail(SK_ERR_INVALID_ARG, "bad sizes B=%d n=%d d=%d", B, n, d);
    hipError_t e = launch_normalize_backward(Xh, norms, G, (long)B * n, d, dX, (hipStream_t)stream);
    return e ? hip_fail(e, "normalize backward") : SK_OK;
}

}  // extern "C"

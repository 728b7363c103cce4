// grad_feat.hip -- dense gradient and barycentric projection for bf16 feature
// clouds on the matrix cores (d = 32 or 64).
//
// The transport application of the FlashSinkhorn summary (Methodologie 3,
// "Toepassing van Transportmatrix": the gradient and the barycentric
// projection are weighted averages over the plan, streamed like the update
// without storing the plan).  With c = log2(e)/eps and the potentials f, g of
// the solution,
//     P_ij / a_i = E_ij = 2^(2c (x_i.y_j + h_i) + beta_j),
//     h_i = (f_i - ||x_i||^2) / 2,   beta_j = c (g_j - ||y_j||^2) + log2 b_j,
// the mass pass of plan_rows_mc.h accumulates per row m_i = sum_j E_ij and
// O_i = sum_j E_ij y_j (keys streamed through LDS, both sums on the matrix
// cores and in fp32, key ranges split over work-groups), and the combine adds
// the splits in order in fp64 and writes
//     dX_i = 2 a_i (m_i x_i - O_i)   (= sum_j 2 P_ij (x_i - y_j)),
//     T_i  = O_i / m_i               (= sum_j P_ij y_j / sum_j P_ij).
// E is the plan divided by the row weight, so m_i is near 1 for potentials
// that solve the problem, whatever the sizes.  A 64-row block with a live row
// whose mass falls outside [2^-64, 2^100] (potentials far from solving these
// weights) is flagged and left unwritten; the fp64 plan pass redoes it.
#include "plan_rows_mc.h"

namespace sk {
namespace {

constexpr int kGroupsG = 4;                          // 16-row groups per wave
constexpr int kTilesG = 4;                           // 16-key tiles per LDS stage
constexpr int kTargetG = 512;                        // work-groups a pass aims for
constexpr int kRowsPerWg = mc::kWaves * 16 * kGroupsG;
constexpr double kMassLoG = 5.421010862427522e-20;   // 2^-64
constexpr double kMassHiG = 1.2676506002282294e30;   // 2^100
static_assert(kGradPad % kRowsPerWg == 0, "padding must hold whole work-groups");

mc::Split grad_split(int B, int n_pad, int m_pad)
{
    return mc::split_of(n_pad / kRowsPerWg * B, m_pad / mc::kTile, kTargetG);
}

// h_i for the rows of one side ([B][n_pad]); rows of weight 0 and padding rows
// get kNeg, so their E is 0 and they add nothing
__global__ void grad_h_kernel(const float *__restrict__ pot, const float *__restrict__ sq,
                              const float *__restrict__ w, int n, int n_pad, float *__restrict__ h)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int b = blockIdx.y;
    if (i >= n_pad)
        return;
    const size_t k = (size_t)b * n + i;
    const bool live = i < n && (w ? w[k] > 0.f : true);
    h[(size_t)b * n_pad + i] = live ? (float)(0.5 * ((double)pot[k] - (double)sq[k])) : kNeg;
}

// One work-group per 64-row block: the splits of m and O added in order (fp64),
// the block's range check, then dX and T (left to the fp64 pass when flagged).
__global__ __launch_bounds__(256) void grad_combine(const float *__restrict__ part_s,
                                                    const float *__restrict__ part_v, int S,
                                                    int B, int n, int n_pad, int d,
                                                    const uint16_t *__restrict__ X,
                                                    const float *__restrict__ w,
                                                    float *__restrict__ grad,
                                                    float *__restrict__ proj,
                                                    int *__restrict__ redo)
{
    __shared__ double ms[kWave];
    __shared__ int flag;
    const int blk = blockIdx.x, b = blockIdx.y, nb = gridDim.x;
    const int tid = threadIdx.x;
    if (tid < kWave) {   // wave 0: a row per lane
        const int row = blk * kWave + tid;
        double s = 0.0;
        bool bad = false;
        if (row < n) {
            for (int p = 0; p < S; ++p)
                s += (double)part_s[((size_t)p * B + b) * n_pad + row];
            const bool live = w ? w[(size_t)b * n + row] > 0.f : true;
            bad = live && !(s >= kMassLoG && s <= kMassHiG);
        }
        ms[tid] = s;
        const bool any = __ballot(bad) != 0;
        if (tid == 0) {
            flag = any ? 1 : 0;
            redo[(size_t)b * nb + blk] = any ? 1 : 0;
        }
    }
    __syncthreads();
    if (flag)
        return;
    const double inv_n = 1.0 / (double)n;
    for (int e = tid; e < kWave * d; e += 256) {
        const int r = e / d, k = e % d;
        const int row = blk * kWave + r;
        if (row >= n)
            continue;
        double O = 0.0;
        for (int p = 0; p < S; ++p)
            O += (double)part_v[(((size_t)p * B + b) * n_pad + row) * d + k];
        const size_t o = ((size_t)b * n + row) * d + k;
        const double wi = w ? (double)w[(size_t)b * n + row] : inv_n;
        const double m = ms[r];
        const bool live = wi > 0.0;
        const double x = (double)bf16_to_float(X[o]);
        if (grad)
            grad[o] = live ? (float)(2.0 * wi * (m * x - O)) : 0.f;
        if (proj)
            proj[o] = live && m > 0.0 ? (float)(O / m) : 0.f;
    }
}

// Xt[b][k][j] = X[b][j][k] for j < n, 0 for the padding up to n_pad.
__global__ void transpose_bf16_kernel(const uint16_t *__restrict__ X, int n, int n_pad, int d,
                                      uint16_t *__restrict__ Xt)
{
    __shared__ uint16_t tile[64][65];
    const int b = blockIdx.z;
    const int j0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;   // 256 threads: 4 rows a pass
    for (int jj = ty; jj < 64; jj += 4) {
        const int j = j0 + jj, k = k0 + tx;
        tile[jj][tx] = (j < n && k < d) ? X[((size_t)b * n + j) * d + k] : (uint16_t)0;
    }
    __syncthreads();
    for (int kk = ty; kk < 64; kk += 4) {
        const int k = k0 + kk, j = j0 + tx;
        if (k < d && j < n_pad)
            Xt[((size_t)b * d + k) * n_pad + j] = tile[tx][kk];
    }
}

}  // namespace

bool gradF_matrix_cores(int dtype, int d) { return dtype == 1 && (d == 32 || d == 64); }

hipError_t launch_transpose_bf16(const void *X, int B, int n, int n_pad, int d, uint16_t *Xt,
                                 hipStream_t st)
{
    dim3 grid(n_pad / 64, ceil_div(d, 64), B);
    hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, st, (const uint16_t *)X, n,
                       n_pad, d, Xt);
    return hipGetLastError();
}

GradFSizes gradF_sizes(int B, int n, int m, int d)
{
    // one side at a time: X rows against Y keys, then Y rows against X keys
    const int np = round_up(n, kGradPad), mp = round_up(m, kGradPad);
    const size_t px = (size_t)grad_split(B, np, mp).S * np;
    const size_t py = (size_t)grad_split(B, mp, np).S * mp;
    GradFSizes z;
    z.h = (size_t)B * std::max(np, mp);
    z.part_s = (size_t)B * std::max(px, py);
    z.part_v = z.part_s * d;
    return z;
}

hipError_t launch_gradF(const SideF &rows, const float *row_w, const SideF &keys,
                        const uint16_t *keys_t, int d, int B, float eps, const GradFWs &w,
                        float *grad, float *proj, hipStream_t st)
{
    const float two_c = 2.0f * scale_of(eps);
    const int np = rows.n_pad, mp = keys.n_pad;
    hipLaunchKernelGGL(grad_h_kernel, dim3(ceil_div(np, 256), B), dim3(256), 0, st,
                       (const float *)rows.pot, (const float *)rows.sq, row_w, rows.n, np, w.h);
    const mc::Split sp = grad_split(B, np, mp);
    const dim3 grid(sp.S, np / kRowsPerWg, B), block(mc::kWaves * kWave);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, st, (const uint16_t *)rows.pts,
                           (const float *)w.h, rows.n, np, (const uint16_t *)keys.pts, keys_t,
                           (const float *)keys.bias, keys.n, mp, nullptr, nullptr, nullptr,
                           two_c, sp.tps, w.part_s, w.part_v, nullptr);
    };
    if (d == 32)
        go(mc::rows_kernel<1, kGroupsG, kTilesG, mc::kRowsMass>);
    else
        go(mc::rows_kernel<2, kGroupsG, kTilesG, mc::kRowsMass>);
    hipLaunchKernelGGL(grad_combine, dim3(ceil_div(rows.n, kWave), B), dim3(256), 0, st,
                       (const float *)w.part_s, (const float *)w.part_v, sp.S, B, rows.n, np, d,
                       (const uint16_t *)rows.pts, row_w, grad, proj, rows.redo);
    return hipGetLastError();
}

}  // namespace sk

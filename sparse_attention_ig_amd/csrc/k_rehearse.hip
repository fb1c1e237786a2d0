// Speculation kernels (InfiniGen, arXiv 2406.19707, paper-graph-ui summary,
// section 3.4 "Decoding Stage", step 1 partial query projection and step 2
// speculated attention scores).
//
// k_rehearse_proj: q_part = x W~_Q^partial, a dense contraction with M = B
//   batch rows, run on the matrix cores: the partial weight is stored with one
//   row of D inputs per partial column, so both MFMA operands come straight
//   from HBM as 16-byte loads along k.  Workgroups split the D reduction;
//   partial sums go to the workspace in a fixed order (no float atomics), so
//   results are deterministic.
// k_rehearse_score: one workgroup per (b, h, row chunk).  It sums the D-slice
//   partials of its (b, h) (and the bias), then streams its chunk of the
//   partial key cache Kp[b][h][j][0..r) with coalesced 16-byte loads, LPR lanes
//   per row, and reduces each row's dot product across those lanes.
#include "ig_device.h"
#include "ig_internal.h"

namespace ig {

constexpr int kProjThreads = 256;
constexpr int kScoreThreads = 256;
constexpr int kScoreUnroll = 8;  // partial-key rows per lane group per batch

// part[s][b][c] = sum over k in split s of x[b][k] * WT[c][k].  Workgroup (64-column tile, D split,
// 16-row batch block); each wave owns 16 columns.  Every load of a chunk is issued before the first
// MFMA (one memory round trip per chunk; a split of 256 bf16 rows is one chunk).
template <typename T>
__global__ __launch_bounds__(kProjThreads) void k_rehearse_proj(const T* __restrict__ x, const T* __restrict__ WT,
                                                               int B, int D, int N, int ks,
                                                               float* __restrict__ part) {
    using M = ProjMma<T>;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int col = blockIdx.x * 64 + wave * 16 + lane % 16;
    const int kg = lane / 16;
    const int b = blockIdx.z * 16 + lane % 16;
    const int k0 = blockIdx.y * ks, k1 = min(D, k0 + ks);
    const bool col_ok = col < N, b_ok = b < B;
    const T* wrow = WT + static_cast<size_t>(col_ok ? col : 0) * D;
    const T* xrow = x + static_cast<size_t>(b_ok ? b : 0) * D;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int kc = k0; kc < k1; kc += M::CHUNK * M::K) {
        typename M::vec w[M::CHUNK], xv[M::CHUNK];
#pragma unroll
        for (int u = 0; u < M::CHUNK; ++u) {
            const int k = kc + u * M::K + kg * M::E;  // D % E == 0, so a group is wholly in or out
            const bool in = k < k1;
            w[u] = (col_ok && in) ? M::load(wrow + k) : M::zero();
            xv[u] = (b_ok && in) ? M::load(xrow + k) : M::zero();
        }
#pragma unroll
        for (int u = 0; u < M::CHUNK; ++u) acc = M::mma(xv[u], w[u], acc);
    }
    if (!col_ok) return;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int bb = blockIdx.z * 16 + 4 * kg + q;
        if (bb < B) part[(static_cast<size_t>(blockIdx.y) * B + bb) * N + col] = acc[q];
    }
}

template <typename T, int LPR>
__global__ __launch_bounds__(kScoreThreads) void k_rehearse_score(
    const float* __restrict__ part, int splits, const float* __restrict__ bias,
    const T* __restrict__ Kp, int B, int H, int r, int n, int n_cap, int chunk, float scale,
    float* __restrict__ q_part, float* __restrict__ scores, int ld) {
    constexpr int VEC = Vec<T>::N;
    constexpr int RPI = kScoreThreads / LPR;  // rows per workgroup step
    __shared__ float qs[LPR * VEC];
    __shared__ float s_part[kScoreThreads];

    const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
    const int N = H * r;
    const int tid = threadIdx.x;
    const int li = tid % LPR, ri = tid / LPR;
    const T* base = Kp + static_cast<size_t>(bh) * n_cap * r + li * VEC;
    float* srow = scores + static_cast<size_t>(bh) * ld;
    const int j0 = blockIdx.x * chunk, j1 = min(n, j0 + chunk);
    // kScoreUnroll rows per lane group per batch, two batches in flight (double buffering); the first
    // batch goes out before the partial sums are read
    constexpr int STEP = RPI * kScoreUnroll;
    uint4 cur[kScoreUnroll], nxt[kScoreUnroll];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
        const int j = j0 + u * RPI + ri;
        cur[u] = j < j1 ? load_raw16(base + static_cast<size_t>(j) * r) : make_uint4(0, 0, 0, 0);
    }
    sum_partials<kScoreThreads>(part, splits, B, N, b, h * r, r, bias, qs, s_part,
                                (blockIdx.x == 0 && q_part) ? q_part + static_cast<size_t>(bh) * r : nullptr);
    float q[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) q[v] = qs[li * VEC + v] * scale;

    for (int jb = j0; jb < j1; jb += STEP) {
        const bool more = jb + STEP < j1;
        if (more) {
#pragma unroll
            for (int u = 0; u < kScoreUnroll; ++u) {
                const int j = jb + STEP + u * RPI + ri;
                nxt[u] = j < j1 ? load_raw16(base + static_cast<size_t>(j) * r) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            float kv[VEC];
            unpack_raw(cur[u], kv);
            float sc = 0.f;
#pragma unroll
            for (int v = 0; v < VEC; ++v) sc = fmaf(q[v], kv[v], sc);
            sc = group_sum<LPR>(sc);
            const int j = jb + u * RPI + ri;
            if (li == 0 && j < j1) srow[j] = sc;
        }
        if (more) {
#pragma unroll
            for (int u = 0; u < kScoreUnroll; ++u) cur[u] = nxt[u];
        }
    }
}

RehearsePlan plan_rehearse(int B, int H, int D, int r, int n, int dtype) {
    (void)dtype;  // the same split for both element types, so the workspace size is dtype-free
    RehearsePlan p{};
    const int N = H * r;
    p.tiles = (N + 63) / 64;
    p.bb = 16;
    p.bblocks = (B + 15) / 16;
    // D splits of 256 rows (512 when that leaves more than 1024 workgroups)
    int ks = 256;
    if (static_cast<int64_t>(p.tiles) * p.bblocks * ((D + 255) / 256) > 1024) ks = 512;
    p.rows_per_split = ks;
    p.splits = (D + ks - 1) / ks;
    p.ws_bytes = static_cast<size_t>(p.splits) * B * N * sizeof(float);
    // score chunks: ~1024 workgroups over B*H*n rows, 256..4096 rows each
    const int64_t rows = static_cast<int64_t>(n) * B * H;
    int64_t c = (rows + 1023) / 1024;
    c = ((c + 255) / 256) * 256;
    c = std::max<int64_t>(256, std::min<int64_t>(4096, c));
    p.chunk = static_cast<int>(c);
    p.chunks = (n + p.chunk - 1) / p.chunk;
    return p;
}

template <typename T>
static int launch_proj_t(const T* x, const T* W, int B, int D, int N, const RehearsePlan& p, float* part,
                         hipStream_t s) {
    hipLaunchKernelGGL(k_rehearse_proj<T>, dim3(p.tiles, p.splits, p.bblocks), dim3(kProjThreads), 0, s, x, W, B, D,
                       N, p.rows_per_split, part);
    return static_cast<int>(hipGetLastError());
}

int launch_proj(const void* x, const void* W, int B, int D, int N, int dtype, const RehearsePlan& p, float* part,
                hipStream_t s) {
    if (dtype == IG_BF16)
        return launch_proj_t(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(W), B, D, N, p, part, s);
    return launch_proj_t(static_cast<const float*>(x), static_cast<const float*>(W), B, D, N, p, part, s);
}

template <typename T>
static int launch_score_t(const float* part, const float* bias, const T* Kp, int B, int H, int r, int n,
                          int n_cap, float scale, float* q_part, float* scores, int ld,
                          const RehearsePlan& p, hipStream_t s) {
    constexpr int VEC = Vec<T>::N;
    dim3 grid(p.chunks, B * H);
    const int lpr = r / VEC;
#define IG_SCORE_CASE(L)                                                                               \
    case L:                                                                                            \
        hipLaunchKernelGGL((k_rehearse_score<T, L>), grid, dim3(kScoreThreads), 0, s, part, p.splits, \
                           bias, Kp, B, H, r, n, n_cap, p.chunk, scale, q_part, scores, ld);          \
        break;
    switch (lpr) {
        IG_SCORE_CASE(1)
        IG_SCORE_CASE(2)
        IG_SCORE_CASE(4)
        IG_SCORE_CASE(8)
        IG_SCORE_CASE(16)
        IG_SCORE_CASE(32)
        default: return static_cast<int>(hipErrorInvalidValue);
    }
#undef IG_SCORE_CASE
    return static_cast<int>(hipGetLastError());
}

int launch_score(const float* part, const float* bias, const void* Kp, int B, int H, int r, int n, int n_cap,
                 int dtype, float scale, float* q_part, float* scores, int ld, const RehearsePlan& p, hipStream_t s) {
    if (dtype == IG_BF16)
        return launch_score_t(part, bias, static_cast<const uint16_t*>(Kp), B, H, r, n, n_cap, scale, q_part, scores,
                              ld, p, s);
    return launch_score_t(part, bias, static_cast<const float*>(Kp), B, H, r, n, n_cap, scale, q_part, scores, ld, p,
                          s);
}

int launch_rehearse(const void* x, const void* Wq_part, const float* bq_part, const void* Kp, int B, int D,
                    int H, int r, int n, int n_cap, int dtype, float scale, float* q_part, float* scores,
                    int ld, void* ws, hipStream_t s) {
    const RehearsePlan p = plan_rehearse(B, H, D, r, n, dtype);
    float* part = static_cast<float*>(ws);
    int e;
    if (dtype == IG_BF16) {
        e = launch_proj_t(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(Wq_part), B, D, H * r, p, part, s);
        if (e) return e;
        return launch_score_t(part, bq_part, static_cast<const uint16_t*>(Kp), B, H, r, n, n_cap, scale, q_part,
                              scores, ld, p, s);
    }
    e = launch_proj_t(static_cast<const float*>(x), static_cast<const float*>(Wq_part), B, D, H * r, p, part, s);
    if (e) return e;
    return launch_score_t(part, bq_part, static_cast<const float*>(Kp), B, H, r, n, n_cap, scale, q_part, scores,
                          ld, p, s);
}

}  // namespace ig

// Speculation kernels (InfiniGen, arXiv 2406.19707, paper-graph-ui summary,
// section 3.4 "Decoding Stage", step 1 partial query projection and step 2
// speculated attention scores).
//
// k_rehearse_proj: q_part = x W~_Q^partial.  M = B is tiny, so this is a
//   bandwidth-bound pass over the [D][H*r] weight: each 256-thread workgroup
//   owns a 64-column tile and a slice of the D rows; every lane streams 16-byte
//   rows of its 8 (bf16) or 4 (f32) columns and multiplies them with x from LDS
//   for up to 16 batch rows at once.  Partial sums of the D slices go to the
//   workspace in a fixed order (no float atomics), so results are
//   deterministic.
// k_rehearse_score: one workgroup per (b, h, row chunk).  It sums the D-slice
//   partials of its (b, h) (and the bias), then streams its chunk of the
//   partial key cache Kp[b][h][j][0..r) with coalesced 16-byte loads, LPR lanes
//   per row, and reduces each row's dot product across those lanes.
#include "ig_device.h"
#include "ig_internal.h"

namespace ig {

constexpr int kProjThreads = 256;
constexpr int kScoreThreads = 256;
constexpr int kScoreUnroll = 4;

template <typename T, int BB>
__global__ __launch_bounds__(kProjThreads) void k_rehearse_proj(
    const T* __restrict__ x, const T* __restrict__ W, int B, int D, int N, int rows_per_split,
    float* __restrict__ part) {
    constexpr int VEC = Vec<T>::N;
    constexpr int CPT = 64 / VEC;            // lanes across the 64-column tile
    constexpr int RSUB = kProjThreads / CPT; // rows in flight per workgroup step
    extern __shared__ __align__(16) float smem[];  // x slice [BB][rows_per_split], later the reduction buffer

    const int tid = threadIdx.x;
    const int cg = tid % CPT, rs = tid / CPT;
    const int col = blockIdx.x * 64 + cg * VEC;
    const int k0 = blockIdx.y * rows_per_split;
    const int kn = min(rows_per_split, D - k0);
    const int b0 = blockIdx.z * BB;

    // every weight row of this lane is put in flight before anything waits (one HBM round trip);
    // rows_per_split <= 256, so a lane owns at most 256 / RSUB rows
    constexpr int UMAX = 256 / RSUB;
    uint4 w[UMAX];
    const bool col_ok = col < N;
    const T* wp = W + static_cast<size_t>(k0) * N + col;
#pragma unroll
    for (int u = 0; u < UMAX; ++u) {
        const int kk = rs + u * RSUB;
        w[u] = (col_ok && kk < kn) ? load_raw16(wp + static_cast<size_t>(kk) * N) : make_uint4(0, 0, 0, 0);
    }
    // x slice [BB][rows_per_split] into LDS; all of a lane's loads are issued before any store
    {
        constexpr int UX = (16 * 256 + kProjThreads - 1) / kProjThreads;  // BB <= 16, rows_per_split <= 256
        float xv[UX];
#pragma unroll
        for (int u = 0; u < UX; ++u) {
            const int i = tid + u * kProjThreads;
            const int bb = i / rows_per_split, kk = i - bb * rows_per_split;
            xv[u] = (i < BB * rows_per_split && b0 + bb < B && kk < kn)
                        ? to_f32(x[static_cast<size_t>(b0 + bb) * D + k0 + kk]) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < UX; ++u) {
            const int i = tid + u * kProjThreads;
            if (i < BB * rows_per_split) smem[i] = xv[u];
        }
    }
    __syncthreads();

    float acc[BB][VEC];
#pragma unroll
    for (int bb = 0; bb < BB; ++bb)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[bb][v] = 0.f;
#pragma unroll
    for (int u = 0; u < UMAX; ++u) {
        const int kk = rs + u * RSUB;
        if (kk < kn) {
            float wv[VEC];
            unpack_raw(w[u], wv);
#pragma unroll
            for (int bb = 0; bb < BB; ++bb) {
                const float xv = smem[bb * rows_per_split + kk];
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[bb][v] = fmaf(xv, wv[v], acc[bb][v]);
            }
        }
    }
    // reduction over the RSUB row groups through LDS (cross-lane shuffles of 64 values per lane cost
    // more than the whole weight stream): red[rs][bb][64 columns], then each output sums RSUB terms
    __syncthreads();  // x slice no longer needed
    float* red = smem;
#pragma unroll
    for (int bb = 0; bb < BB; ++bb)
#pragma unroll
        for (int v = 0; v < VEC; ++v) red[(rs * BB + bb) * 64 + cg * VEC + v] = acc[bb][v];
    __syncthreads();
    for (int i = tid; i < BB * 64; i += kProjThreads) {
        const int bb = i / 64, c = i % 64;
        float s = 0.f;
#pragma unroll 8
        for (int g = 0; g < RSUB; ++g) s += red[(g * BB + bb) * 64 + c];
        const int b = b0 + bb, cc = blockIdx.x * 64 + c;
        if (b < B && cc < N) part[(static_cast<size_t>(blockIdx.y) * B + b) * N + cc] = s;
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
    sum_partials<kScoreThreads>(part, splits, B, N, b, h * r, r, bias, qs, s_part,
                                blockIdx.x == 0 ? q_part + static_cast<size_t>(bh) * r : nullptr);

    const int li = tid % LPR, ri = tid / LPR;
    float q[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) q[v] = qs[li * VEC + v] * scale;

    const T* base = Kp + static_cast<size_t>(bh) * n_cap * r + li * VEC;
    float* srow = scores + static_cast<size_t>(bh) * ld;
    const int j0 = blockIdx.x * chunk, j1 = min(n, j0 + chunk);
    for (int jb = j0; jb < j1; jb += RPI * kScoreUnroll) {
        float kv[kScoreUnroll][VEC];
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            const int j = jb + u * RPI + ri;
            if (j < j1) {
                load_vec(base + static_cast<size_t>(j) * r, kv[u]);
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v) kv[u][v] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < kScoreUnroll; ++u) {
            float s = 0.f;
#pragma unroll
            for (int v = 0; v < VEC; ++v) s = fmaf(q[v], kv[u][v], s);
            s = group_sum<LPR>(s);
            const int j = jb + u * RPI + ri;
            if (li == 0 && j < j1) srow[j] = s;
        }
    }
}

RehearsePlan plan_rehearse(int B, int H, int D, int r, int n, int dtype) {
    (void)dtype;
    RehearsePlan p{};
    const int N = H * r;
    p.tiles = (N + 63) / 64;
    int bb = 1;
    while (bb < B && bb < 16) bb <<= 1;
    p.bb = bb;
    p.bblocks = (B + bb - 1) / bb;
    // aim for ~256 workgroups over the weight; D slices are multiples of 32 rows, at most 256
    int splits = (256 + p.tiles * p.bblocks - 1) / (p.tiles * p.bblocks);
    splits = std::max(1, std::min(splits, (D + 31) / 32));
    int rps = (D + splits - 1) / splits;
    rps = ((rps + 31) / 32) * 32;
    if (rps > 256) rps = 256;
    p.rows_per_split = rps;
    p.splits = (D + rps - 1) / rps;
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

template <typename T, int BB>
static int launch_proj_bb(dim3 grid, size_t smem, hipStream_t s, const T* x, const T* W, int B, int D, int N, int rps,
                          float* part) {
    static bool attr_set = false;  // dynamic LDS above 64 KB needs the per-function limit raised once
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_rehearse_proj<T, BB>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return static_cast<int>(e);
        attr_set = true;
    }
    hipLaunchKernelGGL((k_rehearse_proj<T, BB>), grid, dim3(kProjThreads), smem, s, x, W, B, D, N, rps, part);
    return static_cast<int>(hipGetLastError());
}

template <typename T>
static int launch_proj_t(const T* x, const T* W, int B, int D, int N, const RehearsePlan& p, float* part,
                         hipStream_t s) {
    dim3 grid(p.tiles, p.splits, p.bblocks);
    // x slice [bb][rows_per_split], then the reduction buffer [row groups][bb][64]
    const int rsub = kProjThreads / (64 / Vec<T>::N);
    const size_t smem = static_cast<size_t>(p.bb) * std::max(p.rows_per_split, rsub * 64) * sizeof(float);
    switch (p.bb) {
        case 1: return launch_proj_bb<T, 1>(grid, smem, s, x, W, B, D, N, p.rows_per_split, part);
        case 2: return launch_proj_bb<T, 2>(grid, smem, s, x, W, B, D, N, p.rows_per_split, part);
        case 4: return launch_proj_bb<T, 4>(grid, smem, s, x, W, B, D, N, p.rows_per_split, part);
        case 8: return launch_proj_bb<T, 8>(grid, smem, s, x, W, B, D, N, p.rows_per_split, part);
        default: return launch_proj_bb<T, 16>(grid, smem, s, x, W, B, D, N, p.rows_per_split, part);
    }
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

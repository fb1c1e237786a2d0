// Per-head token selection (InfiniGen, arXiv 2406.19707, paper-graph-ui summary,
// section 3.4 "Decoding Stage": step 3 threshold max - alpha, step 4 head
// averaging, step 5 per-layer cap; the fixed-budget top-k is the comparator of
// section 2, challenge C1).
//
// One 1024-thread workgroup per (b, h) row.  Scores are mapped to
// order-preserving uint32 keys (kept in LDS when the row fits).
//  - Threshold: block max of the keys, cut = max - alpha in float32, count of
//    keys >= key(cut).  If that count fits the cap, those rows are the answer.
//  - Otherwise (and for top-k): exact radix select of the k-th largest key,
//    MSB first, 8 bits per pass with a 256-bin LDS histogram.  It yields the
//    k-th key T and how many rows equal to T must be kept (the lowest indices).
//  - Ordered compaction: every thread takes 8 consecutive rows; a block-wide
//    exclusive scan of per-thread counts (wave shuffles + per-wave totals in
//    LDS) gives each selected row its output slot, so idx comes out ascending
//    without any sort and the result is deterministic.
#include <climits>

#include "ig_device.h"
#include "ig_internal.h"

namespace ig {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelLdsKeys = 8192;   // rows per (b, h) held in LDS (32 KB)
constexpr int kSelPerThread = 8;    // consecutive rows per thread in the compaction

// mode values beyond the public ones: count-only pass of the head average
constexpr int kSelCountOnly = 100;

struct SelScratch {
    int hist[256];
    int wtot[kSelWaves];
    uint32_t wmax[kSelWaves];
    int bc[4];
};

__device__ __forceinline__ int block_sum(int v, SelScratch& sh) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    v = wave_sum_i32(v);
    if (lane == 0) sh.wtot[wave] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) t += sh.wtot[w];
    __syncthreads();
    return t;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, SelScratch& sh) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    v = wave_max_u32(v);
    if (lane == 0) sh.wmax[wave] = v;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) t = sh.wmax[w] > t ? sh.wmax[w] : t;
    __syncthreads();
    return t;
}

// exclusive prefix of v over the block in thread order; *total = block sum
__device__ __forceinline__ int block_excl_scan(int v, SelScratch& sh, int* total) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    int inc = v;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        const int t = __shfl_up(inc, m, kWave);
        if (lane >= m) inc += t;
    }
    if (lane == kWave - 1) sh.wtot[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const int t = sh.wtot[w];
        base += (w < wave) ? t : 0;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return base + inc - v;
}

template <bool IN_LDS>
__device__ __forceinline__ uint32_t row_key(const float* __restrict__ srow, const uint32_t* lk, int j) {
    if (IN_LDS) return lk[j];
    return score_key(srow[j]);
}

// Radix select: the kk-th largest key (1 <= kk <= n) and how many keys equal
// to it belong to the top kk.
template <bool IN_LDS>
__device__ void radix_kth(const float* __restrict__ srow, const uint32_t* lk, int n, int kk, SelScratch& sh,
                          uint32_t* T_out, int* need_eq) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, pmask = 0;
    int remaining = kk;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kSelThreads) sh.hist[i] = 0;
        __syncthreads();
        for (int j = tid; j < n; j += kSelThreads) {
            const uint32_t key = row_key<IN_LDS>(srow, lk, j);
            if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        if (tid < kWave) {
            const int lane = tid;
            const int b0 = lane * 4;
            const int h0 = sh.hist[b0], h1 = sh.hist[b0 + 1], h2 = sh.hist[b0 + 2], h3 = sh.hist[b0 + 3];
            const int s = h0 + h1 + h2 + h3;
            int suf = s;  // sum over this lane and all higher lanes (higher bins)
#pragma unroll
            for (int m = 1; m < kWave; m <<= 1) {
                const int t = __shfl_down(suf, m, kWave);
                if (lane + m < kWave) suf += t;
            }
            int cum = suf - s;  // rows in bins above this lane's four
            const int hv[4] = {h3, h2, h1, h0};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (cum < remaining && cum + hv[q] >= remaining) {
                    sh.bc[0] = b0 + 3 - q;
                    sh.bc[1] = cum;
                }
                cum += hv[q];
            }
        }
        __syncthreads();
        const uint32_t digit = static_cast<uint32_t>(sh.bc[0]);
        remaining -= sh.bc[1];
        prefix |= digit << shift;
        pmask |= 255u << shift;
        __syncthreads();
    }
    *T_out = prefix;
    *need_eq = remaining;
}

// Write ascending indices of rows with key > T, plus the first need_eq rows
// with key == T.  Returns the number written (block-uniform).
template <bool IN_LDS>
__device__ int ordered_compact(const float* __restrict__ srow, const uint32_t* lk, int n, uint32_t T,
                               int need_eq, int32_t* __restrict__ out, int max_out, SelScratch& sh) {
    const int tid = threadIdx.x;
    int written = 0, eq_seen = 0;
    constexpr int TILE = kSelThreads * kSelPerThread;
    for (int base = 0; base < n; base += TILE) {
        const int j0 = base + tid * kSelPerThread;
        uint32_t keys[kSelPerThread];
        int n_eq = 0;
#pragma unroll
        for (int e = 0; e < kSelPerThread; ++e) {
            const int j = j0 + e;
            keys[e] = (j < n) ? row_key<IN_LDS>(srow, lk, j) : 0u;
            n_eq += (j < n && keys[e] == T) ? 1 : 0;
        }
        int tot_eq;
        int eq_rank = eq_seen + block_excl_scan(n_eq, sh, &tot_eq);
        bool sel[kSelPerThread];
        int n_sel = 0;
#pragma unroll
        for (int e = 0; e < kSelPerThread; ++e) {
            const int j = j0 + e;
            bool s = false;
            if (j < n) {
                if (keys[e] > T) {
                    s = true;
                } else if (keys[e] == T) {
                    s = eq_rank < need_eq;
                    ++eq_rank;
                }
            }
            sel[e] = s;
            n_sel += s ? 1 : 0;
        }
        int tot_sel;
        int pos = written + block_excl_scan(n_sel, sh, &tot_sel);
#pragma unroll
        for (int e = 0; e < kSelPerThread; ++e) {
            if (sel[e]) {
                if (pos < max_out) out[pos] = j0 + e;
                ++pos;
            }
        }
        written += tot_sel;
        eq_seen += tot_eq;
    }
    return written;
}

template <bool IN_LDS>
__global__ __launch_bounds__(kSelThreads) void k_select(
    const float* __restrict__ scores, int H, int n, int ld, int mode, float alpha, int k, int max_sel,
    int32_t* __restrict__ idx, int32_t* __restrict__ count, int max_out, int32_t* __restrict__ head_counts) {
    __shared__ uint32_t lk[IN_LDS ? kSelLdsKeys : 1];
    __shared__ SelScratch sh;
    const int bh = blockIdx.x, tid = threadIdx.x;
    const float* srow = scores + static_cast<size_t>(bh) * ld;

    uint32_t kmax = 0;
    for (int j = tid; j < n; j += kSelThreads) {
        const uint32_t key = score_key(srow[j]);
        if (IN_LDS) lk[j] = key;
        kmax = key > kmax ? key : kmax;
    }
    // block_max_u32 synchronises, which also publishes the LDS keys
    const uint32_t kmax_all = block_max_u32(kmax, sh);

    int limit = min(n, max_out);
    int kk;
    if (mode == IG_SEL_THRESHOLD || mode == kSelCountOnly) {
        const float cut = key_score(kmax_all) - alpha;
        const uint32_t kc = score_key(cut);
        int c = 0;
        for (int j = tid; j < n; j += kSelThreads) c += row_key<IN_LDS>(srow, lk, j) >= kc ? 1 : 0;
        const int cnt = block_sum(c, sh);
        if (mode == kSelCountOnly) {
            if (tid == 0) head_counts[bh] = cnt;
            return;
        }
        if (max_sel > 0) limit = min(limit, max_sel);
        if (cnt <= limit) {
            const int w = ordered_compact<IN_LDS>(srow, lk, n, kc, INT_MAX,
                                                  idx + static_cast<size_t>(bh) * max_out, max_out, sh);
            if (tid == 0) count[bh] = w;
            return;
        }
        kk = limit;
    } else if (mode == IG_SEL_HEADAVG) {
        // every head of sequence b takes ceil(mean_h count_h), capped
        const int b = bh / H;
        int tot = 0;
        for (int h = 0; h < H; ++h) tot += head_counts[b * H + h];
        kk = (tot + H - 1) / H;
        if (max_sel > 0) kk = min(kk, max_sel);
        kk = max(1, min(kk, limit));
    } else {
        kk = min(k, limit);
    }
    uint32_t T;
    int need_eq;
    radix_kth<IN_LDS>(srow, lk, n, kk, sh, &T, &need_eq);
    const int w = ordered_compact<IN_LDS>(srow, lk, n, T, need_eq, idx + static_cast<size_t>(bh) * max_out,
                                          max_out, sh);
    if (tid == 0) count[bh] = w;
}

size_t select_ws_bytes(int B, int H, int n, int max_out) {
    (void)n;
    (void)max_out;
    return static_cast<size_t>(B) * H * sizeof(int32_t);  // per-head counts of the head-average mode
}

int launch_select(const float* scores, int B, int H, int n, int ld, int mode, float alpha, int k, int max_sel,
                  int32_t* idx, int32_t* count, int max_out, void* ws, hipStream_t s) {
    const dim3 grid(B * H), block(kSelThreads);
    int32_t* hc = static_cast<int32_t*>(ws);
    const bool lds = n <= kSelLdsKeys;
    if (mode == IG_SEL_HEADAVG) {
        if (lds)
            hipLaunchKernelGGL((k_select<true>), grid, block, 0, s, scores, H, n, ld, kSelCountOnly, alpha, k,
                               max_sel, idx, count, max_out, hc);
        else
            hipLaunchKernelGGL((k_select<false>), grid, block, 0, s, scores, H, n, ld, kSelCountOnly, alpha, k,
                               max_sel, idx, count, max_out, hc);
        const int e = static_cast<int>(hipGetLastError());
        if (e) return e;
    }
    if (lds)
        hipLaunchKernelGGL((k_select<true>), grid, block, 0, s, scores, H, n, ld, mode, alpha, k, max_sel, idx,
                           count, max_out, hc);
    else
        hipLaunchKernelGGL((k_select<false>), grid, block, 0, s, scores, H, n, ld, mode, alpha, k, max_sel, idx,
                           count, max_out, hc);
    return static_cast<int>(hipGetLastError());
}

}  // namespace ig

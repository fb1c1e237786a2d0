// Block-level selection primitives (InfiniGen, arXiv 2406.19707, paper-graph-ui
// summary, section 3.4 "Decoding Stage" steps 3-5): block reductions and scans
// for 1024-thread workgroups, an exact MSB-first radix select of the k-th
// largest order-preserving key, and the ordered compaction that writes the
// selected indices ascending.  Used by the standalone selection kernel and by
// the fused speculation kernel.
#pragma once

#include <climits>

#include "ig_device.h"

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

// f(j, key) for every row j < n owned by this thread (j = tid mod kSelThreads).  Rows in HBM are
// read 8 per lane at a time, all loads issued before any is used.
template <bool IN_LDS, typename F>
__device__ __forceinline__ void for_each_key(const float* __restrict__ srow, const uint32_t* lk, int n, F f) {
    const int tid = threadIdx.x;
    if (IN_LDS) {
        for (int j = tid; j < n; j += kSelThreads) f(j, lk[j]);
        return;
    }
    constexpr int U = 8;
    for (int j0 = tid; j0 < n; j0 += kSelThreads * U) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * kSelThreads;
            v[u] = j < n ? srow[j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * kSelThreads;
            if (j < n) f(j, score_key(v[u]));
        }
    }
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
        for_each_key<IN_LDS>(srow, lk, n, [&](int, uint32_t key) {
            if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1);
        });
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

// Per-row action of a compaction (no-op by default): visit(pos, j) for the
// row j written at output slot pos.
struct NoVisit {
    __device__ __forceinline__ void operator()(int, int) const {}
};

// Write ascending indices of rows with key > T, plus the first need_eq rows
// with key == T; visit(pos, j) is called for every row written.  Returns the
// number written (block-uniform).  Each tile's keys are read into registers
// before the tile's first barrier and pos <= j, so a visitor may overwrite
// lk[pos] (the slots of rows already consumed) with the selected index.
template <bool IN_LDS, typename Visit = NoVisit>
__device__ int ordered_compact(const float* __restrict__ srow, const uint32_t* lk, int n, uint32_t T,
                               int need_eq, int32_t* __restrict__ out, int max_out, SelScratch& sh,
                               Visit visit = Visit()) {
    const int tid = threadIdx.x;
    int written = 0, eq_seen = 0;
    constexpr int TILE = kSelThreads * kSelPerThread;
    for (int base = 0; base < n; base += TILE) {
        const int j0 = base + tid * kSelPerThread;
        uint32_t keys[kSelPerThread];
        int n_eq = 0;
        if (IN_LDS && j0 + kSelPerThread <= n) {
            // two 16-byte LDS reads instead of eight strided words
            const uint4 a = *reinterpret_cast<const uint4*>(lk + j0);
            const uint4 b = *reinterpret_cast<const uint4*>(lk + j0 + 4);
            keys[0] = a.x; keys[1] = a.y; keys[2] = a.z; keys[3] = a.w;
            keys[4] = b.x; keys[5] = b.y; keys[6] = b.z; keys[7] = b.w;
        } else {
#pragma unroll
            for (int e = 0; e < kSelPerThread; ++e) {
                const int j = j0 + e;
                keys[e] = (j < n) ? row_key<IN_LDS>(srow, lk, j) : 0u;
            }
        }
#pragma unroll
        for (int e = 0; e < kSelPerThread; ++e) n_eq += (j0 + e < n && keys[e] == T) ? 1 : 0;
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
                if (pos < max_out) {
                    out[pos] = j0 + e;
                    visit(pos, j0 + e);
                }
                ++pos;
            }
        }
        written += tot_sel;
        eq_seen += tot_eq;
    }
    return written;
}

}  // namespace ig

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
// Threshold and top-k rows longer than the LDS holds are cut into slices, as in
// the fused speculation: each slice workgroup keeps its slice's keys in LDS and
// hands on a superset of its own selection as candidates, and a merge
// workgroup per row applies the row's rules to them (a key among the row's top
// k is among its slice's top k, and a key at or above the row's cut is at or
// above its slice's, whose maximum is at most the row's).  The head-average
// mode, and rows beyond 16 slices, stream the row from HBM in every pass.
#include <algorithm>
#include <type_traits>

#include "ig_internal.h"
#include "ig_select_dev.h"
#include "ig_spec_dev.h"

namespace ig {

template <bool IN_LDS>
__global__ __launch_bounds__(kSelThreads) void k_select(
    const float* __restrict__ scores, int H, int n, int ld, int mode, float alpha, int k, int max_sel,
    int32_t* __restrict__ idx, int32_t* __restrict__ count, int max_out, int32_t* __restrict__ head_counts) {
    extern __shared__ __align__(16) uint32_t lk[];  // IN_LDS: the row's n keys (dynamic, n <= 32768)
    __shared__ SelScratch sh;
    __shared__ std::conditional_t<IN_LDS, FastSel, int> fs;
    const int bh = blockIdx.x, tid = threadIdx.x;
    const float* srow = scores + static_cast<size_t>(bh) * ld;

    if constexpr (IN_LDS) fast_sel_init(fs);  // published by the barriers of block_max_u32
    uint32_t kmax = 0;
    for_each_key<false>(srow, nullptr, n, [&](int j, uint32_t key) {
        if (IN_LDS) lk[j] = key;
        kmax = key > kmax ? key : kmax;
    });
    // block_max_u32 synchronises, which also publishes the LDS keys
    const uint32_t kmax_all = block_max_u32(kmax, sh);

    int limit = min(n, max_out);
    int kk;
    if (mode == IG_SEL_THRESHOLD || mode == kSelCountOnly) {
        const float cut = key_score(kmax_all) - alpha;
        const uint32_t kc = score_key(cut);
        int cnt;
        if constexpr (IN_LDS) {
            cnt = count_ge_lds(lk, n, kc, sh);
        } else {
            int c = 0;
            for_each_key<IN_LDS>(srow, lk, n, [&](int, uint32_t key) { c += key >= kc ? 1 : 0; });
            cnt = block_sum(c, sh);
        }
        if (mode == kSelCountOnly) {
            if (tid == 0) head_counts[bh] = cnt;
            return;
        }
        if (max_sel > 0) limit = min(limit, max_sel);
        if (cnt <= limit) {
            int w;
            if constexpr (IN_LDS)
                w = compact_lds(lk, n, kc, INT_MAX, INT_MAX, idx + static_cast<size_t>(bh) * max_out, max_out, fs,
                                NoVisit());
            else
                w = ordered_compact<IN_LDS>(srow, lk, n, kc, INT_MAX, idx + static_cast<size_t>(bh) * max_out,
                                            max_out, sh);
            if (tid == 0) count[bh] = min(w, max_out);
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
    int need_eq, w;
    if constexpr (IN_LDS) {
        int eq_total;
        if (!sampled_kth_lds(lk, n, kk, fs, sh, &T, &need_eq, &eq_total))
            radix_kth_lds(lk, n, kk, fs, &T, &need_eq, &eq_total);
        w = compact_lds(lk, n, T, need_eq, eq_total, idx + static_cast<size_t>(bh) * max_out, max_out, fs,
                        NoVisit());
    } else {
        radix_kth<IN_LDS>(srow, lk, n, kk, sh, &T, &need_eq);
        w = ordered_compact<IN_LDS>(srow, lk, n, T, need_eq, idx + static_cast<size_t>(bh) * max_out, max_out, sh);
    }
    if (tid == 0) count[bh] = min(w, max_out);
}

// Slice workgroup (slice, row) of a long row: the slice's keys in LDS, then its candidates.
__global__ __launch_bounds__(kSpecThreads) void k_select_slice(SpecParams p, const float* __restrict__ scores,
                                                               int ld) {
    extern __shared__ __align__(16) uint32_t keys[];  // the slice's keys (slice_rows <= kSpecMaxRows)
    __shared__ SpecShared<kSpecMaxSlices + 1> sm;
    const int tid = threadIdx.x;
    const int nrow = p.B * p.H;
    const int slice = blockIdx.x / nrow, bh = blockIdx.x - slice * nrow;
    const int r0 = slice * p.slice_rows;
    const int m = min(p.n - r0, p.slice_rows);
    const float* __restrict__ srow = scores + static_cast<size_t>(bh) * ld + r0;
    fast_sel_init(sm.fs);  // published by the barriers of block_max_u32
    constexpr int U = 8;   // loads per lane in flight
    uint32_t kmax = 0;
    for (int j0 = tid; j0 < m; j0 += kSpecThreads * U) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = j0 + u * kSpecThreads < m ? srow[j0 + u * kSpecThreads] : 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * kSpecThreads;
            if (j < m) {
                const uint32_t key = score_key(v[u]);
                keys[j] = key;
                kmax = key > kmax ? key : kmax;
            }
        }
    }
    const uint32_t kmax_all = block_max_u32(kmax, sm.sh);  // also publishes the LDS keys
    spec_select<true>(p, bh / p.H, bh, slice, m, m, kmax_all, LdsKeys{keys}, keys, sm.sh, sm.fs, sm.last,
                      [&](int j) { return r0 + j; });
}

// Workspace of a select call: the head-average mode's per-head counts, then (rows longer than the LDS
// holds) the slices' candidate counts, keys and row indices.
struct SelectPlan {
    SlicePlan sl;
    bool sliced;
    size_t off_cnt, off_key, off_idx, bytes;
};

static size_t align256s(size_t v) { return (v + 255) / 256 * 256; }

static SelectPlan plan_select(int B, int H, int n, int max_out) {
    SelectPlan sp{};
    const int64_t rows = static_cast<int64_t>(B) * H;
    sp.off_cnt = align256s(static_cast<size_t>(rows) * sizeof(int32_t));
    sp.bytes = static_cast<size_t>(rows) * sizeof(int32_t);
    if (n > kSelLdsKeys) {
        sp.sl = plan_slices(rows, n, std::min(n, max_out));
        sp.sliced = sp.sl.ok && sp.sl.slices > 1;
    }
    if (sp.sliced) {
        const size_t cands = static_cast<size_t>(rows) * sp.sl.slices * sp.sl.cap;
        sp.off_key = sp.off_cnt + align256s(static_cast<size_t>(rows) * sp.sl.slices * sizeof(int32_t));
        sp.off_idx = sp.off_key + align256s(cands * sizeof(uint32_t));
        sp.bytes = sp.off_idx + cands * sizeof(int32_t);
    }
    return sp;
}

size_t select_ws_bytes(int B, int H, int n, int max_out) { return plan_select(B, H, n, max_out).bytes; }

bool select_needs_ws(int B, int H, int n, int max_out, int mode) {
    return mode == IG_SEL_HEADAVG || plan_select(B, H, n, max_out).sliced;
}

static int launch_select_sliced(const SelectPlan& sp, const float* scores, int B, int H, int n, int ld, int mode,
                                float alpha, int k, int max_sel, int32_t* idx, int32_t* count, int max_out,
                                void* ws, hipStream_t s) {
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_select_slice),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(speculate_lds_bytes(kSpecMaxRows)));
        if (e != hipSuccess) return static_cast<int>(e);
        attr_set = true;
    }
    char* w = static_cast<char*>(ws);
    SpecParams p{};
    p.B = B;
    p.H = H;
    p.n = n;
    p.n_cap = n;
    p.ld = ld;
    p.scale = 1.f;
    p.mode = mode;
    p.alpha = alpha;
    p.k = k;
    p.max_sel = max_sel;
    p.max_out = max_out;
    p.idx = idx;
    p.count = count;
    p.xcd_heads = 0;  // merge workgroup wg is row wg: b = wg / H
    p.slices = sp.sl.slices;
    p.slice_rows = sp.sl.slice_rows;
    p.cand_cap = sp.sl.cap;
    p.cand_key = reinterpret_cast<uint32_t*>(w + sp.off_key);
    p.cand_idx = reinterpret_cast<int32_t*>(w + sp.off_idx);
    p.cand_cnt = reinterpret_cast<int32_t*>(w + sp.off_cnt);
    hipLaunchKernelGGL(k_select_slice, dim3(B * H * sp.sl.slices), dim3(kSpecThreads),
                       speculate_lds_bytes(sp.sl.slice_rows), s, p, scores, ld);
    const int e = static_cast<int>(hipGetLastError());
    return e ? e : launch_spec_merge(p, IG_F32, s);
}

int launch_select(const float* scores, int B, int H, int n, int ld, int mode, float alpha, int k, int max_sel,
                  int32_t* idx, int32_t* count, int max_out, void* ws, hipStream_t s) {
    if (mode != IG_SEL_HEADAVG) {
        const SelectPlan sp = plan_select(B, H, n, max_out);
        if (sp.sliced)
            return launch_select_sliced(sp, scores, B, H, n, ld, mode, alpha, k, max_sel, idx, count, max_out, ws, s);
    }
    const dim3 grid(B * H), block(kSelThreads);
    int32_t* hc = static_cast<int32_t*>(ws);
    const bool lds = n <= kSelLdsKeys;
    static bool attr_set = false;  // dynamic LDS above 64 KB needs the per-function limit raised once
    if (lds && !attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_select<true>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(kSelLdsKeys * sizeof(uint32_t)));
        if (e != hipSuccess) return static_cast<int>(e);
        attr_set = true;
    }
    const size_t dyn = lds ? static_cast<size_t>(n) * sizeof(uint32_t) : 0;
    for (int pass = mode == IG_SEL_HEADAVG ? 0 : 1; pass < 2; ++pass) {
        const int m = pass == 0 ? kSelCountOnly : mode;  // the head average counts every head first
        if (lds)
            hipLaunchKernelGGL((k_select<true>), grid, block, dyn, s, scores, H, n, ld, m, alpha, k, max_sel, idx,
                               count, max_out, hc);
        else
            hipLaunchKernelGGL((k_select<false>), grid, block, 0, s, scores, H, n, ld, m, alpha, k, max_sel, idx,
                               count, max_out, hc);
        const int e = static_cast<int>(hipGetLastError());
        if (e) return e;
    }
    return 0;
}

}  // namespace ig

// Fused speculation for one (b, h) row as a device function (InfiniGen, arXiv 2406.19707,
// paper-graph-ui summary, section 3.4 "Decoding Stage" steps 1-3 and 5, and
// "KV Cache Pool Management Under Memory Pressure"): partial query, speculated
// scores, threshold or top-k selection, and the access-counter update.
//
// A speculation launch has two kinds of workgroups:
//  0. Projection workgroups (the lowest workgroup indices of the launch, never
//     waiting on anything): each multiplies the attention input x by one block
//     of columns of the partial weight over one split of 512 inputs of D for
//     every batch row, reading its weight rows once from HBM, and stores the
//     split partial sums [splits][B][H*r].
//  1. One 1024-thread row workgroup per (b, h) (or per slice of a row): it
//     issues its first partial-key loads, polls its head's split partials
//     until all are stored, adds them in a fixed order (its partial query),
//     then:
//  2. Scores of every cached row go to LDS as order-preserving keys (and to
//     HBM only if the caller asks for them), streaming the partial-key rows in
//     double-buffered batches of 16 bytes per lane.
//  3. Selection runs on the LDS keys with the same rules as ig_select; the
//     compaction leaves the selected indices in LDS.
//  4. Every selected slot's counter gets an integer atomic increment, all
//     issued together; the last workgroup of a sequence to arrive (one arrival
//     word per sequence in the workspace) applies the halving and picks the
//     victim, then returns the word to zero.
//
// The waits are safe without co-residency guarantees: a row workgroup only
// waits on workgroups with lower indices, which the hardware dispatches first
// and which run to completion unconditionally; every wait is also bounded.
//
// The workgroup index `wg` of the row is passed in (the fused decode kernel
// runs rows after other roles' workgroups); the caller provides the LDS:
// `keys` holds max(n, kProjLdsWords) words, `sm` the fixed scratch.
#pragma once

#include <climits>
#include <type_traits>

#include "ig_attn_dev.h"
#include "ig_internal.h"
#include "ig_pool_dev.h"
#include "ig_select_dev.h"

namespace ig {

constexpr int kSpecThreads = 1024;
constexpr int kRowSelThreads = 512;  // threads that select a whole row once its keys are in LDS
constexpr int kSpecBatch = 8;  // default partial-key rows per lane per batch

struct SpecParams {
    const void* x;       // [B][D] attention input
    const void* W;       // [H*r][D] partial query weight (one row per partial column)
    int D;
    float* part;         // split partial sums [splits][B][H*r] of the launch's projection workgroups
    int splits;          //   (splits of kProjSplit inputs), added by each row in split order
    const float* bias;
    const void* Kp;
    int B, H, r, n, n_cap, ld;
    float scale;
    int mode;
    float alpha;
    int k, max_sel, max_out;
    int32_t* idx;
    int32_t* count;
    float* q_part;
    float* scores;
    uint32_t* counters;
    uint32_t cmax;
    int32_t* victim;
    uint32_t* arrive;  // [B] words: (arrivals << 16) + saturated workgroups; zero between calls
    int xcd_heads;
    // sliced rows (few rows, or rows longer than one workgroup's LDS): workgroup (slice, row) selects
    // within rows [slice * slice_rows, +slice_rows) and leaves its candidates; a merge workgroup per
    // row selects among them.  slices == 1: the row's own workgroup does everything.
    int slices, slice_rows, cand_cap;
    uint32_t* cand_key;      // [B*H][slices][cand_cap]
    int32_t* cand_idx;       // [B*H][slices][cand_cap] row indices
    int32_t* cand_cnt;       // [B*H][slices]
    // large merges: the merge leaves each row's selection as a bitmap [B*H][ceil(n / 32)] and a counter
    // kernel adds the heads' bits per slot (no atomics per selected slot); NULL: atomics in the merge
    uint32_t* bits;
    // projection workgroups: the first proj_wgs workgroups of the launch (proj_blocks column blocks x
    // splits); row_wgs: the row workgroups
    int proj_wgs, proj_blocks, row_wgs;
    // workspace status word (sticky failure bits) and shape stamp (the (B, H, D, r) key of the calls the
    // workspace serves; 0 until the first call claims it).  NULL: no checks (the standalone selection).
    uint32_t* status;
    unsigned long long* stamp;
    unsigned long long key;
    uint32_t spin_limit;  // polls of a row workgroup before it stops waiting for its partial query
    int withhold;         // failure-path testing: the projection workgroups store no partial sums
    // top-k slices with tight candidates: a slice hands on about its share of the row's budget (plus a
    // margin) and records in cand_lo [B*H][slices] the bound it used (every key of the slice at or above
    // it was handed on); the first slice of a row stores the row's scaled partial query in q_rows
    // [B*H][r], from which a merge whose candidates turn out too few recomputes the row's scores.
    int tight;
    uint32_t* cand_lo;
    float* q_rows;
    // head average (whole rows): each row's threshold count [B*H], summed per sequence by the merge
    int32_t* hcount;
};

// Sticky status bits of a speculation workspace (the public IG_WS_* values).
constexpr uint32_t kWsTimeout = IG_WS_TIMEOUT;
constexpr uint32_t kWsShape = IG_WS_SHAPE;

// Fills the launch parameters of a speculation call (projection and row workgroups).
int begin_speculate(const SpecCall& c, SpecParams* p);
// The merge launch of sliced rows: one workgroup per row over the slices' candidate slots.
int launch_spec_merge(const SpecParams& p, int dtype, hipStream_t s, const CombineArgs& cb = CombineArgs{});
// After the launch of sliced rows: the merge (with the attention combine cb, if any), and the counter
// kernels when the merge leaves bitmaps.
int finish_speculate(const SpecParams& p, int dtype, void* ws, hipStream_t s, const CombineArgs& cb = CombineArgs{});

template <int R>
struct SpecShared {
    SelScratch sh;
    FastSel fs;
    float q[R < kSpecMaxSlices + 1 ? kSpecMaxSlices + 1 : R];  // partial query; slice offsets in a merge
    int last;
};

// Projection workgroups (summary section 3.4 "Decoding Stage" step 1, the partial query
// x . W~_Q^partial, a dense contraction: M = batch rows, N = H*r partial columns, K = D).  Workgroup
// pw takes column block pw / splits (kProjCols columns) and split pw % splits of the D inputs
// (kProjSplit of them).  Wave w owns 16-column tile w % kProjTiles and input slice
// w / kProjTiles (kProjSplit / kProjSlices inputs) and runs it on the matrix cores (16x16x32 bf16 or
// 16x16x4 f32 MFMA, x rows as A in blocks of 16 batch rows, weight columns as B, both loaded 16 bytes
// (bf16) along k: the weight straight from HBM, x from L2); the slices' 16x16 results meet in LDS and
// are added in slice order.
//
// Hand-over without flags: a partial-sum slot holds 0 (all bits clear) while it is empty.  A
// producer never writes those bits (a sum of +0.0 is stored as -0.0, which adds the same in the
// readers' sums, all started from +0.0), so a reader polls its slots until none is 0, then returns
// them to 0 for the next call (the last reader of a sliced row does, counted per row).  Slots and
// counts travel through device-coherent stores and loads (agent scope: written through to the
// level all XCDs share, read from there); no fence is needed (on this chip an agent-scope fence
// writes back the XCD's whole L2).  The workspace starts zero-filled.
constexpr int kProjSplit = 512;   // inputs per split partial
constexpr int kProjTiles = 2;     // 16-column tiles per projection workgroup
constexpr int kProjCols = 16 * kProjTiles;
constexpr int kProjSlices = kSpecThreads / kWave / kProjTiles;  // input slices (one wave per tile and slice)
constexpr int kProjLdsWords = kProjSlices * kProjTiles * 256;   // the slices' results (also the least `keys` size)
constexpr uint32_t kProjSpinLimit = 1u << 22;  // default polls before a row workgroup stops waiting

__device__ __forceinline__ void coherent_store(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ void proj_role(const SpecParams& p, int pw, uint32_t* lds) {
    using M = ProjMma<T>;
    constexpr int KPS = kProjSplit / kProjSlices;  // inputs per slice
    constexpr int STEPS = KPS / M::K;              // MFMA steps per slice
    constexpr int CH = STEPS < 8 ? STEPS : 8;      // steps whose loads are in flight together
    static_assert(KPS % M::K == 0 && STEPS % CH == 0, "projection tiling");
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int tile = wave % kProjTiles, slice = wave / kProjTiles;
    const int kg = lane / 16;
    const int N = p.H * p.r, D = p.D, B = p.B;
    // head-major: the splits of a column block are dispatched together, so the first blocks' partial
    // queries are complete early and their rows start streaming while later blocks are projected
    const int blk = pw / p.splits, s = pw - blk * p.splits;
    const int col = blk * kProjCols + tile * 16 + lane % 16;
    const bool col_ok = col < N;
    const int k0 = s * kProjSplit + slice * KPS + kg * M::E;  // this lane's first input (D % E == 0)
    const T* __restrict__ x = static_cast<const T*>(p.x);
    const T* __restrict__ wrow = static_cast<const T*>(p.W) + static_cast<size_t>(col_ok ? col : 0) * D;
    float* red = reinterpret_cast<float*>(lds);  // [slice][tile][16 rows][16 columns]
    for (int b0 = 0; b0 < B; b0 += 16) {
        const int b = b0 + lane % 16;
        const T* __restrict__ xrow = x + static_cast<size_t>(b < B ? b : 0) * D;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c0 = 0; c0 < STEPS; c0 += CH) {
            typename M::vec w[CH], xv[CH];
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                const int k = k0 + (c0 + u) * M::K;
                w[u] = (col_ok && k < D) ? M::load(wrow + k) : M::zero();
                xv[u] = (b < B && k < D) ? M::load(xrow + k) : M::zero();
            }
#pragma unroll
            for (int u = 0; u < CH; ++u) acc = M::mma(xv[u], w[u], acc);
        }
        // lane l holds rows 4 (l / 16) .. + 3 of column l % 16
#pragma unroll
        for (int q = 0; q < 4; ++q) red[((slice * kProjTiles + tile) * 16 + 4 * kg + q) * 16 + lane % 16] = acc[q];
        __syncthreads();
        const int t = threadIdx.x;
        if (t < kProjTiles * 256) {
            const int tl = t / 256, row = (t / 16) % 16, c = blk * kProjCols + tl * 16 + t % 16;
            if (b0 + row < B && c < N && !p.withhold) {
                float v = 0.f;
#pragma unroll
                for (int sl = 0; sl < kProjSlices; ++sl) v += red[(sl * kProjTiles + tl) * 256 + row * 16 + t % 16];
                coherent_store(p.part + (static_cast<size_t>(s) * B + b0 + row) * N + c,
                               __float_as_uint(v) == 0u ? -0.f : v);  // never the empty bits
            }
        }
        __syncthreads();  // red is reused by the next block of batch rows
    }
}

// Admission of a row workgroup to the workspace (thread 0; the caller makes the result block-wide):
// the status word must be clear (a failure of an earlier call poisons the workspace until it is
// zero-filled again) and the shape stamp must be this call's key -- a zero stamp is claimed with a
// compare-and-swap (the first call after the zero-fill).  A stamp of another shape sets kWsShape.
// Returns true when the row may proceed.  Both words are read with device-coherent loads, issued
// together.
__device__ __forceinline__ bool ws_admit(const SpecParams& p) {
    if (!p.status) return true;
    const uint32_t st = __hip_atomic_load(p.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned long long s = __hip_atomic_load(p.stamp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (s == 0ull) {
        unsigned long long e = 0ull;
        __hip_atomic_compare_exchange_strong(p.stamp, &e, p.key, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        s = e == 0ull ? p.key : e;
    }
    if (s != p.key) {
        atomicOr(p.status, kWsShape);
        return false;
    }
    return st == 0u;
}

// Row workgroup: the partial query q[c] (c < R) of row b, columns [col0, col0 + R): poll the split
// partials until every slot is filled, add them in a fixed order (thread (c, i) adds splits i, i + P,
// .. in turn, then the P threads of column c are added by DPP; bias last), and return the slots to
// empty (a whole row; the slices of a row leave that to the row's merge).  Writes q (and q_out when not
// NULL); s_flag: one word of LDS scratch; ends with a barrier.  Returns false (block-uniform) when the
// row may not use the workspace (ws_admit) or when some slot is still empty after spin_limit polls:
// then nothing is added and no slot is touched (a producer may still be about to store into one), the
// timeout sets kWsTimeout, and the workspace stays unusable until it is zero-filled again.
template <int R>
__device__ __forceinline__ bool wait_partial_query(const SpecParams& p, int b, int col0, float* q, float* q_out,
                                                   int* s_flag) {
    constexpr int P = kSpecThreads / R < 64 ? kSpecThreads / R : 64;  // threads per column
    const int tid = threadIdx.x;
    const bool on = tid < R * P;
    const int c = tid / P, i = tid % P;
    const int N = p.H * p.r;
    const bool sole = p.slices == 1;  // the only reader of these slots
    bool admitted = false;            // (block-uniform)
    float acc = 0.f;
    for (int s0 = 0; s0 < p.splits; s0 += P) {
        const int s = s0 + i;
        const bool mine = on && s < p.splits;
        float* src = p.part + (static_cast<size_t>(s) * p.B + b) * N + col0 + c;
        float v = 0.f;
        uint32_t polls = 0;
        for (;;) {
            if (mine) v = coherent_load(src);
            // the admission's loads travel with the first poll's (one round trip for both)
            if (!admitted && tid == 0) *s_flag = ws_admit(p) ? 0 : 1;
            const bool empty = __syncthreads_or(mine && __float_as_uint(v) == 0u);
            if (!admitted) {
                admitted = true;
                if (*s_flag) return false;  // (published by the barrier above)
            }
            if (!empty) break;
            if (++polls >= p.spin_limit) {  // block-uniform: every thread counts the same polls
                if (tid == 0 && p.status) atomicOr(p.status, kWsTimeout);
                __syncthreads();
                return false;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        // every slot of this round is filled: add them all at once, then return them to empty
        if (mine) acc += v;
    }
    if (sole) {
        for (int s0 = 0; s0 < p.splits; s0 += P) {
            const int s = s0 + i;
            if (on && s < p.splits) coherent_store(p.part + (static_cast<size_t>(s) * p.B + b) * N + col0 + c, 0.f);
        }
    }
    acc = group_sum<P>(acc);
    if (on && i == 0) {
        const float v = p.bias ? acc + p.bias[col0 + c] : acc;
        q[c] = v;
        if (q_out) q_out[c] = v;
    }
    // (the slices of a row all read the same slots: the row's merge, a launch after them, empties them)
    __syncthreads();
    return true;
}

// (b, h) of a row workgroup index: with xcd_heads, groups of adjacent heads go to one XCD with all
// their batch rows (workgroups are dealt to the 8 XCDs round robin)
__device__ __forceinline__ void spec_bh(const SpecParams& p, int row_wg, int* b, int* h) {
    if (p.xcd_heads) {
        const int G = p.xcd_heads;
        const int xcd = row_wg % 8, slot = row_wg / 8;
        const int grp = xcd + 8 * (slot / (p.B * G));
        const int rem = slot % (p.B * G);
        *h = grp * G + rem % G;
        *b = rem / G;
    } else {
        *b = row_wg / p.H;
        *h = row_wg - *b * p.H;
    }
}

template <int NT = kSpecThreads>
__device__ __forceinline__ void seq_arrive(const SpecParams& p, int b, bool sat, uint32_t* lds, SelScratch& sh,
                                           int& s_last);

// Row index of key j for a whole row (the key's own position).
struct IdentityIdx {
    __device__ __forceinline__ int operator()(int j) const { return j; }
};
// Row index of key j from an array in LDS (a merge's candidates copied there with their row indices).
struct LdsIdx {
    const int32_t* p;
    __device__ __forceinline__ int operator()(int j) const { return p[j]; }
};

constexpr int kSampledMin = 16384;  // keys from which a selection first tries the sampled bracket

// The cut of a selection.  Selecting every key above kth and the first need_eq keys equal to it (of
// eq_total equal keys; every key >= kth when need_eq >= eq_total) gives the selection.  A slice's cut
// from a sampled bound (win_lo > 0) is good only when it selects between win_lo (its kk) and cand_cap
// keys; the compaction checks that count before it places anything.
struct SelCut {
    uint32_t kth;
    int need_eq, eq_total;
    int kk, win_lo;
};

// Keys a slice of `rows` of a row's n rows hands on for a top-kk selection of the row with tight
// candidates: its expected share of the row's kk plus five standard deviations and 8 (a slice holding
// more of the row's top kk than that makes the merge recompute the row), at most cap.
__device__ __forceinline__ int tight_slice_k(int kk_row, int rows, int n, int cap) {
    const float e = static_cast<float>(kk_row) * static_cast<float>(rows) / static_cast<float>(n);
    const int want = static_cast<int>(ceilf(e + 5.f * sqrtf(e) + 8.f));
    return min(min(want, rows), cap);
}

// The exact cut of the top kk of ks[0..m) (fast_sel_init and a barrier before): the sampled bracket
// pays off on long rows; below kSampledMin keys the radix over every key is faster.
template <int NT = kSpecThreads, class KS>
__device__ __forceinline__ void exact_cut(KS keys, int m, int kk, FastSel& fs, SelScratch& sh, SelCut& c) {
    if (m < kSampledMin || !sampled_kth<NT>(keys, m, kk, fs, sh, &c.kth, &c.need_eq, &c.eq_total))
        radix_kth_keys<NT>(keys, m, kk, fs, &c.kth, &c.need_eq, &c.eq_total);
}

// The cut of the selection over the keys ks[0..m) (held in LDS, a merge's candidates in global memory,
// or a row recomputed from its partial keys).  `rows`: the row count the limit refers to (the slice's
// length in a slice workgroup, n otherwise).  TO_CANDS (a slice): the cut of a superset of the slice's
// selection of at most cand_cap keys -- every key at or above a sampled lower bound of the slice's cut,
// to be checked by the compaction (win_lo); with tight top-k candidates, of the slice's share of the
// row's budget.
template <bool TO_CANDS, int NT = kSpecThreads, class KS>
__device__ __forceinline__ SelCut spec_cut(const SpecParams& p, int b, int bh, int m, int rows, uint32_t kmax_all,
                                           KS keys, SelScratch& sh, FastSel& fs) {
    int limit = min(rows, p.max_out);
    bool done = false;
    int kk = 0;
    SelCut c{0u, INT_MAX, INT_MAX, 0, 0};
    if (p.mode == IG_SEL_HEADAVG) {
        if constexpr (TO_CANDS) {
            // a whole row of a head-average call: its threshold count for the sequence's average, and as
            // candidates every key an averaged count could take, the row's top min(n, max_out, max_sel)
            const uint32_t kc = score_key(key_score(kmax_all) - p.alpha);
            const int cnt = count_ge<NT>(keys, m, kc, sh);
            if (threadIdx.x == 0) p.hcount[bh] = cnt;
            kk = p.max_sel > 0 ? min(limit, p.max_sel) : limit;
        } else {
            // the merge: every head of sequence b takes ceil(mean_h count_h), then the cap and the output
            if (threadIdx.x == 0) {
                long long tot = 0;
                for (int h = 0; h < p.H; ++h) tot += p.hcount[static_cast<size_t>(b) * p.H + h];
                long long cb = (tot + p.H - 1) / p.H;
                if (p.max_sel > 0) cb = min(cb, static_cast<long long>(p.max_sel));
                sh.bc[0] = static_cast<int>(max(1ll, min(cb, static_cast<long long>(min(limit, m)))));
            }
            __syncthreads();
            kk = sh.bc[0];
            __syncthreads();
        }
    } else if (p.mode == IG_SEL_THRESHOLD) {
        const uint32_t kc = score_key(key_score(kmax_all) - p.alpha);
        const int cnt = count_ge<NT>(keys, m, kc, sh);
        if (p.max_sel > 0) limit = min(limit, p.max_sel);
        if (cnt <= limit) {
            c.kth = kc;
            done = true;
        } else {
            kk = limit;
        }
    } else {
        kk = min(p.k, limit);
        if constexpr (TO_CANDS) {
            if (p.tight) kk = tight_slice_k(min(p.k, min(p.n, p.max_out)), rows, p.n, p.cand_cap);
        }
    }
    c.kk = kk;
    if constexpr (TO_CANDS) {
        if (!done && p.cand_cap > kk + kk / 8 && sampled_bound<NT>(keys, m, kk, p.cand_cap, fs, &c.kth)) {
            c.win_lo = kk;  // every key >= the bound, when there are kk to cand_cap of them
            return c;
        }
    }
    if (!done) exact_cut<NT>(keys, m, kk, fs, sh, c);
    return c;
}

// The results of a selection with cut c over ks[0..m): gidx(j) is the row index of key j; lds: at least
// 1024 words of LDS scratch (may be the keys' own storage).  TO_CANDS: write the selected keys and row
// indices as this slice's candidates (at most cand_cap keys; when the merge may read the candidate
// arrays whole, the slice's unused slots get key 0, below every score key) and, with tight candidates,
// the slice's bound; returns false, having written nothing, when a sampled cut selects a count outside
// its window.  Otherwise write idx / count and update the counters (one integer atomic per selected
// slot, all in flight together; the last workgroup of sequence b halves if any slot saturated and picks
// the victim).
template <bool TO_CANDS, int NT = kSpecThreads, class KS, typename GIdx>
__device__ __forceinline__ bool spec_emit(const SpecParams& p, int b, int bh, int slice, int m, const SelCut& c,
                                          KS keys, uint32_t* lds, SelScratch& sh, FastSel& fs, int& s_last,
                                          GIdx gidx) {
    const int tid = threadIdx.x;
    const uint32_t kth = c.kth;
    const int need_eq = c.need_eq, eq_total = c.eq_total;
    if constexpr (TO_CANDS) {
        const size_t base = (static_cast<size_t>(bh) * p.slices + slice) * p.cand_cap;
        uint32_t* ck = p.cand_key + base;
        int32_t* ci = p.cand_idx + base;
        // the candidates are staged in LDS (the select's scratch words are free by the compaction's
        // placing pass) and written out coalesced, when they fit there
        const bool staged = 2 * p.cand_cap <= kFastStage;
        uint32_t* sk = fs.stage();
        int32_t* si = reinterpret_cast<int32_t*>(sk + p.cand_cap);
        auto put = [&](int pos, int j) {
            if (staged) {
                sk[pos] = keys.at(j);
                si[pos] = gidx(j);
            } else {
                ck[pos] = keys.at(j);
                ci[pos] = gidx(j);
            }
        };
        const int got = compact_keys<NT>(keys, m, kth, need_eq, eq_total, nullptr, p.cand_cap, fs, put, c.win_lo,
                                     c.win_lo > 0 ? p.cand_cap : INT_MAX);
        if (got < 0) return false;
        const int written = min(got, p.cand_cap);
        if (staged) {
            __syncthreads();
            for (int i = tid; i < written; i += NT) {
                ck[i] = sk[i];
                ci[i] = si[i];
            }
        }
        // (a merge reads the candidate arrays whole only when they exceed its LDS)
        if (static_cast<int64_t>(p.slices) * p.cand_cap > kSpecMaxRows)
            for (int i = written + tid; i < p.cand_cap; i += NT) ck[i] = 0u;
        if (tid == 0) {
            p.cand_cnt[static_cast<size_t>(bh) * p.slices + slice] = written;
            // every key above kth was handed on, and every key equal to it unless only some of the ties
            // were taken: the keys are integers, so the bound is kth or kth + 1
            if (p.cand_lo) p.cand_lo[static_cast<size_t>(bh) * p.slices + slice] = need_eq >= eq_total ? kth : kth + 1u;
        }
        return true;
    } else {
        const int n = p.n;
        uint32_t* crow = p.counters ? p.counters + static_cast<size_t>(b) * p.n_cap : nullptr;
        const uint32_t cmax = p.cmax;
        uint32_t* stage = fs.stage();  // the select's scratch words are free by now
        int32_t* out = p.idx + static_cast<size_t>(bh) * p.max_out;
        int written;
        if constexpr (std::is_same<GIdx, IdentityIdx>::value || std::is_same<GIdx, LdsIdx>::value) {
            // the row index of each selected key is at hand: staged in LDS as the key is placed (beyond
            // the staging words, written straight out), then written out coalesced
            auto keep = [&](int pos, int j) {
                const int g = gidx(j);
                if (pos < kFastStage)
                    stage[pos] = static_cast<uint32_t>(g);
                else
                    out[pos] = g;
            };
            written = compact_keys<NT>(keys, m, kth, need_eq, eq_total, nullptr, p.max_out, fs, keep);
            __syncthreads();
            const int ws = min(min(written, p.max_out), kFastStage);
            for (int i = tid; i < ws; i += NT) out[i] = static_cast<int32_t>(stage[i]);
        } else {
            // key positions first, then every position mapped to its row index with batched loads
            written = compact_keys<NT>(keys, m, kth, need_eq, eq_total, out, p.max_out, fs, NoVisit());
            __syncthreads();
            const int w = min(written, p.max_out);
            constexpr int U = 8;
            for (int i0 = tid; i0 < w; i0 += NT * U) {
                int pos[U];
#pragma unroll
                for (int u = 0; u < U; ++u) pos[u] = i0 + u * NT < w ? out[i0 + u * NT] : 0;
                int g[U];
#pragma unroll
                for (int u = 0; u < U; ++u) g[u] = i0 + u * NT < w ? gidx(pos[u]) : 0;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = i0 + u * NT;
                    if (i < w) {
                        out[i] = g[u];
                        if (i < kFastStage) stage[i] = static_cast<uint32_t>(g[u]);
                    }
                }
            }
            __syncthreads();
        }
        if (tid == 0) p.count[bh] = min(written, p.max_out);
        if (!crow) return true;
        if (p.bits) {
            // the row's selection as a bitmap of its n slots, built in LDS and written out whole
            const int nw = (n + 31) / 32;
            const int w = min(written, p.max_out);
            for (int i = tid; i < nw; i += NT) lds[i] = 0u;
            __syncthreads();
            for (int i = tid; i < w; i += NT) {
                const uint32_t j = i < kFastStage ? stage[i] : static_cast<uint32_t>(out[i]);
                if (j < static_cast<uint32_t>(n)) atomicOr(&lds[j >> 5], 1u << (j & 31u));
            }
            __syncthreads();
            uint32_t* dst = p.bits + static_cast<size_t>(bh) * nw;
            for (int i = tid; i < nw; i += NT) dst[i] = lds[i];
            return true;
        }
        int sat = 0;
        // (written <= max_out and every staged index is < n by construction; both are re-checked so
        // that no counter update can land outside the row)
        // at most one atomic per lane when the selection is small, else 8 per lane in flight at a time,
        // their returns checked afterwards
        const int touched = min(written, p.max_out);
        if (touched <= NT) {
            if (tid < touched) {
                const uint32_t j = tid < kFastStage ? stage[tid] : static_cast<uint32_t>(out[tid]);
                if (j < static_cast<uint32_t>(n) && atomicAdd(&crow[j], 1u) + 1u >= cmax) sat = 1;
            }
        } else {
        constexpr int U = 8;
        for (int i0 = tid; i0 < touched; i0 += NT * U) {
            uint32_t old[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * NT;
                uint32_t j = 0xFFFFFFFFu;
                if (i < touched) j = i < kFastStage ? stage[i] : static_cast<uint32_t>(out[i]);
                old[u] = j < static_cast<uint32_t>(n) ? atomicAdd(&crow[j], 1u) : 0u;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + u * NT;
                if (i < touched && old[u] + 1u >= cmax) sat = 1;
            }
        }
        }
        seq_arrive<NT>(p, b, __syncthreads_or(sat) != 0, lds, sh, s_last);
        return true;
    }
}

// Selection over ks[0..m) and its results (spec_cut, then spec_emit).
template <bool TO_CANDS, int NT = kSpecThreads, class KS, typename GIdx>
__device__ __forceinline__ void spec_select(const SpecParams& p, int b, int bh, int slice, int m, int rows,
                                            uint32_t kmax_all, KS keys, uint32_t* lds, SelScratch& sh, FastSel& fs,
                                            int& s_last, GIdx gidx) {
    const SelCut c = spec_cut<TO_CANDS, NT>(p, b, bh, m, rows, kmax_all, keys, sh, fs);
    if (spec_emit<TO_CANDS, NT>(p, b, bh, slice, m, c, keys, lds, sh, fs, s_last, gidx)) return;
    // a sampled bound whose superset held too few or too many keys: the exact cut of the slice's kk
    __syncthreads();  // every wave is done with the sample's histograms
    fast_sel_init<NT>(fs);
    __syncthreads();
    SelCut e{0u, INT_MAX, INT_MAX, c.kk, 0};
    exact_cut<NT>(keys, m, c.kk, fs, sh, e);
    spec_emit<TO_CANDS, NT>(p, b, bh, slice, m, e, keys, lds, sh, fs, s_last, gidx);
}

// Score keys of a whole row recomputed from its partial keys (the exact fallback of a merge whose tight
// candidates turn out too few): the same float32 products in the same order as the row workgroups'
// stream -- per lane group member the fused multiply-adds over its VEC channels, then the members'
// partial sums added pairwise as the cross-lane reduction adds them -- so every key equals the one the
// slice held.  q: the scaled partial query [R] in LDS.
template <typename T, int LPR>
struct RowKeys {
    static constexpr int kE = LPR >= 8 ? 1 : 4;  // keys per lane per step (each a row of LPR 16-byte loads)
    static constexpr int VEC = Vec<T>::N;
    static constexpr int R = LPR * VEC;
    const T* kp;     // the row's partial keys [n][R]
    const float* q;
    __device__ __forceinline__ uint32_t at(int j) const {
        const T* row = kp + static_cast<size_t>(j) * R;
        float part[LPR];
#pragma unroll
        for (int l = 0; l < LPR; ++l) {
            float kv[VEC];
            unpack_raw(load_raw16(row + l * VEC), kv);
            float s = 0.f;
#pragma unroll
            for (int v = 0; v < VEC; ++v) s = fmaf(q[l * VEC + v], kv[v], s);
            part[l] = s;
        }
#pragma unroll
        for (int w = 1; w < LPR; w *= 2) {
#pragma unroll
            for (int i = 0; i < LPR; i += 2 * w) part[i] = part[i] + part[i + w];
        }
        return score_key(part[0]);
    }
    template <int E>
    __device__ __forceinline__ void load(int j, int end, uint32_t (&k)[E]) const {
#pragma unroll
        for (int e = 0; e < E; ++e) k[e] = j + e < end ? at(j + e) : 0u;
    }
};

// The arrival of a row of sequence b after its counter updates (sat: some increment of this workgroup
// reached cmax).  Every counter atomic of this workgroup has returned (its value was used) before the
// barrier inside __syncthreads_or that produced `sat`, so it is performed before thread 0's arrival
// atomic below; atomics are coherent across XCDs, so no fence (an agent-scope fence writes back the
// XCD's whole L2) is needed.  One word per sequence carries the arrivals (high half) and the workgroups
// that saw a saturation (low half); the last of the H rows halves the sequence's counters if any row
// saturated, picks the victim and returns the word to zero.
template <int NT>
__device__ __forceinline__ void seq_arrive(const SpecParams& p, int b, bool sat, uint32_t* lds, SelScratch& sh,
                                           int& s_last) {
    const int tid = threadIdx.x;
    if (tid == 0) {
        const uint32_t old = atomicAdd(&p.arrive[b], 0x10000u + (sat ? 1u : 0u));
        const bool last = (old >> 16) == static_cast<uint32_t>(p.H - 1);
        s_last = last ? (1 + (((old & 0xFFFFu) + (sat ? 1u : 0u)) != 0u ? 1 : 0)) : 0;
    }
    __syncthreads();
    if (!s_last) return;
    const bool halve = s_last == 2;
    uint32_t* crow = p.counters + static_cast<size_t>(b) * p.n_cap;
    const int v = pool_finish<NT>(crow, p.n, p.cmax, halve, p.victim != nullptr, lds, &sh.wtot[0]);
    if (tid == 0) {
        if (p.victim) p.victim[b] = v;
        __hip_atomic_store(&p.arrive[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// A whole row (or a merged row) that could not be computed: count = -1 marks it; its counters are not
// touched, but the row still arrives so that the sequence's last row finishes as usual (with bitmaps,
// the row's bitmap is all zero instead).
__device__ __forceinline__ void spec_fail_row(const SpecParams& p, int b, int bh, uint32_t* lds, SelScratch& sh,
                                              int& s_last) {
    const int tid = threadIdx.x;
    if (tid == 0) p.count[bh] = -1;
    if (!p.counters) return;
    if (p.bits) {
        const int nw = (p.n + 31) / 32;
        uint32_t* dst = p.bits + static_cast<size_t>(bh) * nw;
        for (int i = tid; i < nw; i += kSpecThreads) dst[i] = 0u;
        return;
    }
    __syncthreads();
    seq_arrive(p, b, false, lds, sh, s_last);
}

// Row workgroup wg of the speculation launch (counted from the first row workgroup): one (b, h) row,
// or (slices > 1) one slice of one row (wg = slice * B*H + row).  The first partial-key batch is
// issued, the partial query is read from the projection workgroups' partial sums, the slice's scores
// go to LDS keys from its partial-key rows, then the selection.
template <typename T, int LPR, int BATCH = kSpecBatch, bool PRE = true>
__device__ __forceinline__ void spec_row(const SpecParams& p, int wg, uint32_t* keys, SpecShared<LPR * Vec<T>::N>& sm) {
    constexpr int VEC = Vec<T>::N;
    constexpr int R = LPR * VEC;               // partial channels per head
    constexpr int RPP = kSpecThreads / LPR;    // rows per pass
    constexpr int STEP = RPP * BATCH;          // rows per batch
    SelScratch& sh = sm.sh;
    FastSel& fs = sm.fs;
    float* s_q = sm.q;

    const int tid = threadIdx.x, li = tid % LPR, ri = tid / LPR;
    const int nrow = p.B * p.H;
    const int slice = p.slices > 1 ? wg / nrow : 0;
    int b, h;
    spec_bh(p, p.slices > 1 ? wg - slice * nrow : wg, &b, &h);
    const int bh = b * p.H + h;
    const int r0 = slice * p.slice_rows;
    const int n = p.slices > 1 ? min(p.n - r0, p.slice_rows) : p.n;  // this workgroup's rows
    const T* kp = static_cast<const T*>(p.Kp) + (static_cast<size_t>(bh) * p.n_cap + r0) * R + li * VEC;

    fast_sel_init(fs);  // the barriers of the partial-query wait publish the cleared histograms

    // 1. the partial query of this (b, h), with the first partial-key batch in flight (PRE) or after
    uint4 cur[BATCH], nxt[BATCH];
    if constexpr (PRE) {
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int j = u * RPP + ri;
            cur[u] = j < n ? load_raw16(kp + static_cast<size_t>(j) * R) : make_uint4(0, 0, 0, 0);
        }
    }
    float* q_out = (p.q_part && slice == 0) ? p.q_part + static_cast<size_t>(bh) * R : nullptr;
    if (!wait_partial_query<R>(p, b, h * R, s_q, q_out, &sm.last)) {
        // no partial query: a slice marks its candidates invalid for the merge, a whole row fails
        if (p.slices > 1) {
            if (tid == 0) p.cand_cnt[static_cast<size_t>(bh) * p.slices + slice] = -1;
        } else {
            spec_fail_row(p, b, bh, keys, sh, sm.last);
        }
        return;
    }
    if constexpr (!PRE) {
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int j = u * RPP + ri;
            cur[u] = j < n ? load_raw16(kp + static_cast<size_t>(j) * R) : make_uint4(0, 0, 0, 0);
        }
    }
    float q[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) q[v] = s_q[li * VEC + v] * p.scale;
    // the scaled partial query, for a merge that may have to recompute this row's scores
    if (p.q_rows && slice == 0 && tid < R) p.q_rows[static_cast<size_t>(bh) * R + tid] = s_q[tid] * p.scale;

    // 2. scores -> LDS keys, double-buffered row batches (the first batch is already in flight)
    float* srow = p.scores ? p.scores + static_cast<size_t>(bh) * p.ld + r0 : nullptr;
    uint32_t kmax = 0;
    for (int jb = 0; jb < n; jb += STEP) {
        const bool more = jb + STEP < n;
        if (more) {
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int j = jb + STEP + u * RPP + ri;
                nxt[u] = j < n ? load_raw16(kp + static_cast<size_t>(j) * R) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            float kv[VEC];
            unpack_raw(cur[u], kv);
            float s = 0.f;
#pragma unroll
            for (int v = 0; v < VEC; ++v) s = fmaf(q[v], kv[v], s);
            s = group_sum<LPR>(s);
            const int j = jb + u * RPP + ri;
            if (li == 0 && j < n) {
                const uint32_t key = score_key(s);
                keys[j] = key;
                kmax = key > kmax ? key : kmax;
                if (srow) srow[j] = s;
            }
        }
        if (more) {
#pragma unroll
            for (int u = 0; u < BATCH; ++u) cur[u] = nxt[u];
        }
    }
    const uint32_t kmax_all = block_max_u32(kmax, sh);  // also publishes the LDS keys

    // 3. selection (and, for a whole row, counters; a slice, or a row of a head-average call, hands on
    // candidates to the merge instead)
    if (p.slices > 1 || p.mode == IG_SEL_HEADAVG) {
        spec_select<true>(p, b, bh, slice, n, n, kmax_all, LdsKeys{keys}, keys, sh, fs, sm.last,
                          [&](int j) { return r0 + j; });
        return;
    }
    // A whole row is selected by its first kRowSelThreads threads; the other waves end here (a barrier
    // waits only for the waves still running).  Every wave that takes part repeats the radix digit
    // search and the compaction's scans, which cost issue slots on SIMDs shared with the workgroup
    // beside it: eight waves finish sooner than sixteen (measured at 2048 keys); four expose too much
    // LDS latency and are slower.
    if (__builtin_amdgcn_readfirstlane(tid / kWave) >= kRowSelThreads / kWave) return;  // wave-uniform
    spec_select<false, kRowSelThreads>(p, b, bh, 0, n, n, kmax_all, LdsKeys{keys}, keys, sh, fs, sm.last,
                                       IdentityIdx());
}

// The partial-sum slots of row (b, h): every slice of the row read them in the launch before, so the
// merge returns them to empty for the next call.
__device__ __forceinline__ void merge_empty_part(const SpecParams& p, int b, int h) {
    if (!p.part) return;
    const int N = p.H * p.r;
    for (int k = threadIdx.x; k < p.splits * p.r; k += kSpecThreads)
        coherent_store(p.part + (static_cast<size_t>(k / p.r) * p.B + b) * N + h * p.r + k % p.r, 0.f);
}

// A merge whose candidate slots fit in LDS twice over (keys and row indices) with at most one slot per
// thread and slice.  One round trip reads every slot of every slice (an unused slot is read, then
// dropped) together with the slices' counts and bounds; the used slots go to LDS in row order.
// With tight candidates the row's cut is searched among the keys at or above E = the largest slice
// bound only: the merge is exact exactly when at least kk candidates reach E (then the kk-th largest
// key T' >= E), and those keys lie in [E, the largest key].  Returns false when the row must be
// recomputed (fewer than kk candidates reach E).
template <int R>
__device__ __forceinline__ bool merge_small(const SpecParams& p, int b, int h, int m, int cnt, uint32_t lo,
                                            bool checked, uint32_t* keys, SpecShared<R>& sm) {
    SelScratch& sh = sm.sh;
    FastSel& fs = sm.fs;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int bh = b * p.H + h;
    const size_t base = static_cast<size_t>(bh) * m;
    const uint32_t* ck = p.cand_key + base;
    const int32_t* ci = p.cand_idx + base;
    uint32_t v[kSpecMaxSlices];
    int32_t x[kSpecMaxSlices];
#pragma unroll
    for (int sl = 0; sl < kSpecMaxSlices; ++sl) {
        const bool on = sl < p.slices && tid < p.cand_cap;
        const size_t g = static_cast<size_t>(sl) * p.cand_cap + tid;
        v[sl] = on ? ck[g] : 0u;
        x[sl] = on ? ci[g] : 0;
    }
    merge_empty_part(p, b, h);
    // wave 0: where each slice's used slots go (a prefix sum over the slices), whether a slice failed,
    // and E
    int* s_off = reinterpret_cast<int*>(sm.q);  // (kSpecMaxSlices + 1 words, free until a recompute)
    if (wave == 0) {
        const int c = tid < p.slices ? min(max(cnt, 0), p.cand_cap) : 0;
        const int inc = wave_incl_scan(c);
        if (tid < p.slices) s_off[tid + 1] = inc;
        const bool bad = __ballot(tid < p.slices && cnt < 0) != 0;
        const uint32_t em = wave_max_u32(lo);
        if (tid == 0) {
            s_off[0] = 0;
            sh.bc[1] = bad ? 1 : 0;
            sh.bc[2] = static_cast<int>(em);
        }
    }
    fast_sel_init(fs);
    __syncthreads();
    if (sh.bc[1]) {
        spec_fail_row(p, b, bh, keys, sh, sm.last);
        return true;
    }
    const uint32_t emax = static_cast<uint32_t>(sh.bc[2]);
    const int mu = s_off[p.slices];  // used candidate slots, in row order slice by slice
    int32_t* lidx = reinterpret_cast<int32_t*>(keys + mu);
    uint32_t kmax = 0;
    int ge = 0;
#pragma unroll
    for (int sl = 0; sl < kSpecMaxSlices; ++sl) {
        if (sl < p.slices) {
            const int o = s_off[sl];
            if (tid < s_off[sl + 1] - o) {
                keys[o + tid] = v[sl];
                lidx[o + tid] = x[sl];
                kmax = max_u32(kmax, v[sl]);
                ge += v[sl] >= emax ? 1 : 0;
            }
        }
    }
    // the largest key and the count at or above E in one barrier (which also publishes the LDS copy)
    kmax = wave_max_u32(kmax);
    ge = wave_sum_i32(ge);
    if (lane == 0) {
        fs.wtot[wave] = static_cast<int>(kmax);
        fs.wtot2[wave] = ge;
    }
    __syncthreads();
    uint32_t kmax_all = 0;
    int ge_all = 0;
#pragma unroll
    for (int w = 0; w < kSpecThreads / kWave; ++w) {
        kmax_all = max_u32(kmax_all, static_cast<uint32_t>(fs.wtot[w]));
        ge_all += fs.wtot2[w];
    }
    SelCut c{0u, INT_MAX, INT_MAX};
    if (checked) {
        const int kk = min(p.k, min(p.n, p.max_out));
        if (ge_all < kk) return false;
        radix_kth_keys(LdsKeys{keys}, mu, kk, fs, &c.kth, &c.need_eq, &c.eq_total, emax, kmax_all);
        if (c.kth == 0u) return false;
    } else {
        c = spec_cut<false>(p, b, bh, mu, p.n, kmax_all, LdsKeys{keys}, sh, fs);
    }
    spec_emit<false>(p, b, bh, 0, mu, c, LdsKeys{keys}, keys, sh, fs, sm.last, LdsIdx{lidx});
    return true;
}

// Any other merge: the used slots are copied to LDS once the counts are known (keys, and row indices
// when they fit too), or the selection runs straight on the candidate arrays.  Returns false when the
// row must be recomputed (tight candidates whose cut T' is below a slice's bound).
template <int R>
__device__ __forceinline__ bool merge_large(const SpecParams& p, int b, int h, int m, int cnt, uint32_t lo,
                                            bool checked, uint32_t* keys, SpecShared<R>& sm) {
    SelScratch& sh = sm.sh;
    FastSel& fs = sm.fs;
    const int tid = threadIdx.x;
    const int bh = b * p.H + h;
    const size_t base = static_cast<size_t>(bh) * m;
    const uint32_t* ck = p.cand_key + base;
    const int32_t* ci = p.cand_idx + base;
    auto gidx = [&](int j) { return static_cast<int>(ci[j]); };
    merge_empty_part(p, b, h);
    if (__syncthreads_or(cnt < 0)) {
        spec_fail_row(p, b, bh, keys, sh, sm.last);
        return true;
    }
    // where each slice's candidates go when only the used slots are copied: a prefix sum over the slices
    int* s_off = reinterpret_cast<int*>(sm.q);  // (kSpecMaxSlices + 1 words, free until a recompute)
    if (tid < p.slices) s_off[tid + 1] = min(cnt, p.cand_cap);
    const uint32_t emax = checked ? block_max_u32(lo, sh) : 0u;
    __syncthreads();
    if (tid == 0) {
        s_off[0] = 0;
        for (int sl = 1; sl <= p.slices; ++sl) s_off[sl] += s_off[sl - 1];
    }
    fast_sel_init(fs);
    __syncthreads();
    const int mu = s_off[p.slices];  // used candidate slots, in row order slice by slice
    uint32_t kmax = 0;
    constexpr int U = 8;  // loads per lane in flight
    if (mu <= kSpecMaxRows) {
        // the used slots' keys to LDS [0, mu), and their row indices to [mu, 2 mu) when they fit too
        const bool with_idx = 2 * mu <= kSpecMaxRows;
        int32_t* lidx = reinterpret_cast<int32_t*>(keys + mu);
        // thread t copies used slot t (t + 1024, ..) of every slice, the loads of all the slices in flight
        // together: slot i of slice sl goes to s_off[sl] + i
        for (int i = tid; i < p.cand_cap; i += kSpecThreads) {
            uint32_t v[kSpecMaxSlices];
            int32_t x[kSpecMaxSlices];
#pragma unroll
            for (int sl = 0; sl < kSpecMaxSlices; ++sl) {
                const bool on = sl < p.slices && i < s_off[sl + 1] - s_off[sl];
                const size_t g = static_cast<size_t>(sl) * p.cand_cap + i;
                v[sl] = on ? ck[g] : 0u;
                x[sl] = on && with_idx ? ci[g] : 0;
            }
#pragma unroll
            for (int sl = 0; sl < kSpecMaxSlices; ++sl) {
                if (sl < p.slices && i < s_off[sl + 1] - s_off[sl]) {
                    keys[s_off[sl] + i] = v[sl];
                    if (with_idx) lidx[s_off[sl] + i] = x[sl];
                    kmax = v[sl] > kmax ? v[sl] : kmax;
                }
            }
        }
        const uint32_t kmax_all = block_max_u32(kmax, sh);  // also publishes the LDS keys
        const SelCut c = spec_cut<false>(p, b, bh, mu, p.n, kmax_all, LdsKeys{keys}, sh, fs);
        if (checked && !(c.kth != 0u && c.kth >= emax)) return false;
        if (with_idx) {
            spec_emit<false>(p, b, bh, 0, mu, c, LdsKeys{keys}, keys, sh, fs, sm.last, LdsIdx{lidx});
        } else {
            // the row index of used slot j: slot j - s_off[sl] of the slice sl holding it
            auto used_idx = [&](int j) {
                int sl = 0;
                while (sl + 1 < p.slices && s_off[sl + 1] <= j) ++sl;
                return static_cast<int>(ci[static_cast<size_t>(sl) * p.cand_cap + (j - s_off[sl])]);
            };
            spec_emit<false>(p, b, bh, 0, mu, c, LdsKeys{keys}, keys, sh, fs, sm.last, used_idx);
        }
        return true;
    }
    if (p.mode == IG_SEL_THRESHOLD) {
        for (int i0 = tid; i0 < m; i0 += kSpecThreads * U) {
            uint32_t v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = i0 + u * kSpecThreads < m ? ck[i0 + u * kSpecThreads] : 0u;
#pragma unroll
            for (int u = 0; u < U; ++u) kmax = v[u] > kmax ? v[u] : kmax;
        }
    }
    const uint32_t kmax_all = block_max_u32(kmax, sh);  // (also the barrier after fast_sel_init)
    const SelCut c = spec_cut<false>(p, b, bh, m, p.n, kmax_all, GlobalKeys{ck}, sh, fs);
    if (checked && !(c.kth != 0u && c.kth >= emax)) return false;
    spec_emit<false>(p, b, bh, 0, m, c, GlobalKeys{ck}, keys, sh, fs, sm.last, gidx);
    return true;
}

// The exact fallback of a tight top-k merge: the row's n keys recomputed from its partial keys and the
// scaled partial query, and the selection over them; the workspace counts the rows recomputed (word 4
// of the status region).
template <typename T, int LPR, int R>
__device__ __forceinline__ void merge_recompute(const SpecParams& p, int b, int bh, uint32_t* keys, SpecShared<R>& sm) {
    const int tid = threadIdx.x;
    if (tid == 0 && p.status) atomicAdd(p.status + 4, 1u);
    __syncthreads();  // every wave is done with the candidate cut's scratch
    if (tid < R) sm.q[tid] = p.q_rows[static_cast<size_t>(bh) * R + tid];
    fast_sel_init(sm.fs);
    __syncthreads();
    const RowKeys<T, LPR> rk{static_cast<const T*>(p.Kp) + static_cast<size_t>(bh) * p.n_cap * R, sm.q};
    spec_select<false>(p, b, bh, 0, p.n, p.n, 0u, rk, keys, sm.sh, sm.fs, sm.last, IdentityIdx());
}

// Merge workgroup of a sliced row.  Slice sl left its candidates in slots [sl * cap, +cap) of the row
// (when the slots exceed the merge's LDS, unused ones hold key 0, below every score key), so the
// m = slices * cap slots are in row order.
// Without tight candidates they hold the row's selection: a key among the row's top c is among its
// slice's top c, and a key at or above the row's threshold cut is at or above its slice's.  The
// selection runs again over them with the row's rules.
//
// With tight top-k candidates a slice handed on only about its share of the row's budget, every key of
// it at or above its bound E_s.  The row's kk-th largest candidate T' is then checked: when T' >= E_s for
// every slice, every key of the row at or above T' is a candidate, so the kk-th largest key of the row is
// T' and the row's top kk (ties to the lower index) are the candidates' top kk -- the selection is exact.
// Otherwise (a slice held more of the row's top kk than its share) the row's scores are recomputed from
// its partial keys (RowKeys, the same float32 arithmetic as the slices) and the selection runs over
// them: exact as well, only slower.
template <typename T, int LPR, int R>
__device__ __forceinline__ void spec_merge(const SpecParams& p, int wg, uint32_t* keys, SpecShared<R>& sm) {
    const int tid = threadIdx.x;
    int b, h;
    spec_bh(p, wg, &b, &h);
    const int bh = b * p.H + h;
    const int m = p.slices * p.cand_cap;
    // the slices' candidate counts (a slice that could not compute its scores marks its count -1: the row
    // fails) and, with tight candidates, their bounds
    const bool checked = p.tight && p.mode == IG_SEL_TOPK;
    int cnt = 0;
    uint32_t lo = 0;
    if (tid < p.slices) {
        cnt = p.cand_cnt[static_cast<size_t>(bh) * p.slices + tid];
        if (checked) lo = p.cand_lo[static_cast<size_t>(bh) * p.slices + tid];
    }
    const bool done = 2 * m <= kSpecMaxRows && p.cand_cap <= kSpecThreads
                          ? merge_small(p, b, h, m, cnt, lo, checked, keys, sm)
                          : merge_large(p, b, h, m, cnt, lo, checked, keys, sm);
    if (!done) merge_recompute<T, LPR>(p, b, bh, keys, sm);
}

}  // namespace ig

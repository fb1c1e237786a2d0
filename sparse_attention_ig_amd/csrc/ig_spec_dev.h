// Fused speculation for one (b, h) row as a device function (InfiniGen, arXiv 2406.19707,
// paper-graph-ui summary, section 3.4 "Decoding Stage" steps 1-3 and 5, and
// "KV Cache Pool Management Under Memory Pressure"): partial query, speculated
// scores, threshold or top-k selection, and the access-counter update.
//
// One 1024-thread workgroup per (b, h); scores never leave the chip.
//  0. A projection kernel (k_rehearse_proj, shared with ig_rehearse) reads the
//     partial query weight once and leaves fixed-order split partials.
//  1. The workgroup sums its (b, h) partials into the partial query.
//  2. Scores of every cached row go to LDS as order-preserving keys (and to
//     HBM only if the caller asks for them), streaming the partial-key rows in
//     double-buffered batches of 8 rows x 16 bytes per lane.
//  3. Selection runs on the LDS keys with the same rules as ig_select; the
//     compaction leaves the selected indices in LDS.
//  4. Every selected slot's counter gets an integer atomic increment, all
//     issued together; the last workgroup of a sequence to arrive (one arrival
//     word per sequence in the workspace) applies the halving and picks the
//     victim, then returns the word to zero.
//
// The workgroup index `wg` of the row is passed in (the fused decode kernel
// runs rows after other roles' workgroups); the caller provides the LDS:
// `keys` holds max(n, 1024) words, `sm` the fixed scratch.
#pragma once

#include <climits>

#include "ig_internal.h"
#include "ig_pool_dev.h"
#include "ig_select_dev.h"

namespace ig {

constexpr int kSpecThreads = 1024;
constexpr int kSpecBatch = 8;  // default partial-key rows per lane per batch

struct SpecParams {
    const float* part;   // [splits][B][H*r] partial sums of the projection kernel
    int splits;
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
};

// Launches the partial-query projection of a speculation call and fills the row kernel's parameters.
int begin_speculate(const SpecCall& c, SpecParams* p, hipStream_t s);

template <int R>
struct SpecShared {
    SelScratch sh;
    FastSel fs;
    float q[R];
    int last;
};

template <typename T, int LPR, int BATCH = kSpecBatch>
__device__ __forceinline__ void spec_row(const SpecParams& p, int wg, uint32_t* keys, SpecShared<LPR * Vec<T>::N>& sm) {
    constexpr int VEC = Vec<T>::N;
    constexpr int R = LPR * VEC;               // partial channels per head
    constexpr int RPP = kSpecThreads / LPR;    // rows per pass
    constexpr int STEP = RPP * BATCH;     // rows per batch
    SelScratch& sh = sm.sh;
    FastSel& fs = sm.fs;
    float* s_q = sm.q;
    int& s_last = sm.last;

    const int tid = threadIdx.x, li = tid % LPR, ri = tid / LPR;
    const int lane = tid % kWave, wave = tid / kWave;
    int b, h;
    if (p.xcd_heads) {
        // groups of G adjacent heads (G = xcd_heads) go to one XCD with all their batch rows, so the
        // weight lines those heads share are fetched into a single L2
        const int G = p.xcd_heads;
        const int xcd = wg % 8, slot = wg / 8;
        const int grp = xcd + 8 * (slot / (p.B * G));
        const int rem = slot % (p.B * G);
        h = grp * G + rem % G;
        b = rem / G;
    } else {
        b = wg / p.H;
        h = wg - b * p.H;
    }
    const int bh = b * p.H + h, n = p.n;
    const T* kp = static_cast<const T*>(p.Kp) + static_cast<size_t>(bh) * p.n_cap * R + li * VEC;

    fast_sel_init(fs);  // the barriers of the partial-query sum below publish the cleared histograms

    // 1. partial query of this (b, h): sum of the projection kernel's D-slice partials (fixed order),
    //    then the first partial-key batch goes in flight
    uint4 cur[BATCH], nxt[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
        const int j = u * RPP + ri;
        cur[u] = j < n ? load_raw16(kp + static_cast<size_t>(j) * R) : make_uint4(0, 0, 0, 0);
    }
    sum_partials<kSpecThreads>(p.part, p.splits, p.B, p.H * R, b, h * R, R, p.bias, s_q, reinterpret_cast<float*>(keys),
                               p.q_part ? p.q_part + static_cast<size_t>(bh) * R : nullptr);
    float q[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) q[v] = s_q[li * VEC + v] * p.scale;

    // 2. scores -> LDS keys, double-buffered row batches (the first batch is already in flight)
    float* srow = p.scores ? p.scores + static_cast<size_t>(bh) * p.ld : nullptr;
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

    // 3. selection; the compaction also stages the selected indices in LDS (the freed histograms)
    uint32_t* crow = p.counters ? p.counters + static_cast<size_t>(b) * p.n_cap : nullptr;
    const uint32_t cmax = p.cmax;
    uint32_t* stage = fs.stage();
    auto keep = [&](int pos, int j) {
        if (pos < kFastStage) stage[pos] = static_cast<uint32_t>(j);
    };
    int32_t* out = p.idx + static_cast<size_t>(bh) * p.max_out;
    int limit = min(n, p.max_out);
    int written;
    bool done = false;
    int kk = 0;
    uint32_t kth = 0;
    int need_eq = INT_MAX;
    if (p.mode == IG_SEL_THRESHOLD) {
        const uint32_t kc = score_key(key_score(kmax_all) - p.alpha);
        int c = 0;
        for (int j = tid; j < n; j += kSpecThreads) c += keys[j] >= kc ? 1 : 0;
        const int cnt = block_sum(c, sh);
        if (p.max_sel > 0) limit = min(limit, p.max_sel);
        if (cnt <= limit) {
            kth = kc;
            done = true;
        } else {
            kk = limit;
        }
    } else {
        kk = min(p.k, limit);
    }
    int eq_total = INT_MAX;
    if (!done) radix_kth_lds(keys, n, kk, fs, &kth, &need_eq, &eq_total);
    written = compact_lds(keys, n, kth, need_eq, eq_total, out, p.max_out, fs, keep);
    if (tid == 0) p.count[bh] = min(written, p.max_out);

    // 4. counters: one integer atomic per selected slot, all in flight together; the last workgroup
    //    of sequence b halves (if any slot saturated) and picks the victim
    if (!crow) return;
    __syncthreads();
    int sat = 0;
    // (written <= max_out and every staged index is < n by construction; both are re-checked so
    // that no counter update can land outside the row)
    const int touched = min(written, p.max_out);
    for (int i = tid; i < touched; i += kSpecThreads) {
        const uint32_t j = i < kFastStage ? stage[i] : static_cast<uint32_t>(out[i]);
        if (j >= static_cast<uint32_t>(n)) continue;
        const uint32_t old = atomicAdd(&crow[j], 1u);
        if (old + 1u >= cmax) sat = 1;
    }
    sat = __syncthreads_or(sat);
    // Every counter atomic of this workgroup has returned (its value was used) before the barrier, so
    // it is performed before thread 0's arrival atomic below; atomics are coherent across XCDs, so no
    // fence (an agent-scope fence writes back the XCD's whole L2) is needed.  One word per sequence
    // carries the arrivals (high half) and the number of workgroups that saw a saturation (low half).
    if (tid == 0) {
        const uint32_t old = atomicAdd(&p.arrive[b], 0x10000u + (sat ? 1u : 0u));
        const bool last = (old >> 16) == static_cast<uint32_t>(p.H - 1);
        s_last = last ? (1 + (((old & 0xFFFFu) + (sat ? 1u : 0u)) != 0u ? 1 : 0)) : 0;
    }
    __syncthreads();
    if (!s_last) return;
    const bool halve = s_last == 2;
    // reuse the key storage for the argmin scratch
    const int v = pool_finish<kSpecThreads>(crow, n, cmax, halve, p.victim != nullptr, keys, &sh.wtot[0]);
    if (tid == 0) {
        if (p.victim) p.victim[b] = v;
        __hip_atomic_store(&p.arrive[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace ig

// Fused speculation for one layer in one launch (InfiniGen, arXiv 2406.19707,
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
#include "ig_internal.h"
#include "ig_pool_dev.h"
#include "ig_select_dev.h"

namespace ig {

constexpr int kSpecThreads = 1024;
constexpr int kSpecWaves = kSpecThreads / kWave;
constexpr int kSpecBatch = 8;  // partial-key rows per lane per batch

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


template <typename T, int LPR>
__global__ __launch_bounds__(kSpecThreads) void k_speculate(SpecParams p) {
    constexpr int VEC = Vec<T>::N;
    constexpr int R = LPR * VEC;               // partial channels per head
    constexpr int RPP = kSpecThreads / LPR;    // rows per pass
    constexpr int STEP = RPP * kSpecBatch;     // rows per batch
    extern __shared__ __align__(16) uint32_t keys[];  // n order-preserving score keys
    __shared__ SelScratch sh;
    __shared__ FastSel fs;
    __shared__ float s_q[R];
    __shared__ int s_last;

    const int tid = threadIdx.x, li = tid % LPR, ri = tid / LPR;
    const int lane = tid % kWave, wave = tid / kWave;
    int b, h;
    if (p.xcd_heads) {
        // groups of G adjacent heads (G = xcd_heads) go to one XCD with all their batch rows, so the
        // weight lines those heads share are fetched into a single L2
        const int G = p.xcd_heads;
        const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
        const int grp = xcd + 8 * (slot / (p.B * G));
        const int rem = slot % (p.B * G);
        h = grp * G + rem % G;
        b = rem / G;
    } else {
        b = blockIdx.x / p.H;
        h = blockIdx.x - b * p.H;
    }
    const int bh = b * p.H + h, n = p.n;
    const T* kp = static_cast<const T*>(p.Kp) + static_cast<size_t>(bh) * p.n_cap * R + li * VEC;

    fast_sel_init(fs);  // the barriers of the partial-query sum below publish the cleared histograms

    // 1. partial query of this (b, h): sum of the projection kernel's D-slice partials (fixed order),
    //    then the first partial-key batch goes in flight
    uint4 cur[kSpecBatch], nxt[kSpecBatch];
#pragma unroll
    for (int u = 0; u < kSpecBatch; ++u) {
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
            for (int u = 0; u < kSpecBatch; ++u) {
                const int j = jb + STEP + u * RPP + ri;
                nxt[u] = j < n ? load_raw16(kp + static_cast<size_t>(j) * R) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < kSpecBatch; ++u) {
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
            for (int u = 0; u < kSpecBatch; ++u) cur[u] = nxt[u];
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

size_t speculate_ws_bytes(int B, int H, int D, int r, int n, int dtype) {
    const size_t part = (plan_rehearse(B, H, D, r, n, dtype).ws_bytes + 255) / 256 * 256;
    return part + (static_cast<size_t>(B) * sizeof(uint32_t) + 255) / 256 * 256;
}

// keys for the n rows; at least one word per thread (the same storage first holds the split-partial
// staging of the partial query, and last the argmin scratch of the pool finish)
size_t speculate_lds_bytes(int n) { return static_cast<size_t>(n < kSpecThreads ? kSpecThreads : n) * sizeof(uint32_t); }

template <typename T, int L>
static int launch_spec_tl(const SpecParams& p, hipStream_t s) {
    const size_t lds = speculate_lds_bytes(p.n);
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_speculate<T, L>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(speculate_lds_bytes(kSpecMaxRows)));
        if (e != hipSuccess) return static_cast<int>(e);
        attr_set = true;
    }
    hipLaunchKernelGGL((k_speculate<T, L>), dim3(p.B * p.H), dim3(kSpecThreads), lds, s, p);
    return static_cast<int>(hipGetLastError());
}

template <typename T>
static int launch_spec_t(const SpecParams& p, hipStream_t s) {
    switch (p.r / Vec<T>::N) {
        case 1: return launch_spec_tl<T, 1>(p, s);
        case 2: return launch_spec_tl<T, 2>(p, s);
        case 4: return launch_spec_tl<T, 4>(p, s);
        case 8: return launch_spec_tl<T, 8>(p, s);
        case 16: return launch_spec_tl<T, 16>(p, s);
        case 32: return launch_spec_tl<T, 32>(p, s);
        default: return static_cast<int>(hipErrorInvalidValue);
    }
}

int launch_speculate(const void* x, const void* Wq_part, const float* bq_part, const void* Kp, int B, int D, int H,
                     int r, int n, int n_cap, int dtype, float scale, int mode, float alpha, int k, int max_sel,
                     int32_t* idx, int32_t* count, int max_out, uint32_t* counters, uint32_t cmax, int32_t* victim,
                     float* q_part, float* scores, int ld, void* ws, hipStream_t s) {
    const RehearsePlan rp = plan_rehearse(B, H, D, r, n, dtype);
    float* part = static_cast<float*>(ws);
    uint32_t* arrive = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + (rp.ws_bytes + 255) / 256 * 256);
    const int e = launch_proj(x, Wq_part, B, D, H * r, dtype, rp, part, s);
    if (e) return e;
    // heads sharing a 128-byte line of the partial-key rows' neighbours are irrelevant here; group the
    // batch rows of a head on one XCD when the heads split evenly over the 8 XCDs
    SpecParams p{part, rp.splits, bq_part, Kp, B, H, r, n, n_cap, ld, scale, mode, alpha, k, max_sel, max_out, idx,
                 count, q_part, scores, counters, cmax, victim, arrive, H % 8 == 0 ? 1 : 0};
    return dtype == IG_BF16 ? launch_spec_t<uint16_t>(p, s) : launch_spec_t<float>(p, s);
}

__global__ void k_zero_words(uint32_t* p, size_t n) {
    const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

int launch_zero(void* ws, size_t bytes, hipStream_t s) {
    const size_t n = bytes / sizeof(uint32_t);
    if (n == 0) return 0;
    hipLaunchKernelGGL(k_zero_words, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<uint32_t*>(ws), n);
    return static_cast<int>(hipGetLastError());
}

}  // namespace ig

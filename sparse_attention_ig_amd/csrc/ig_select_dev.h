// Block-level selection primitives (InfiniGen, arXiv 2406.19707, paper-graph-ui
// summary, section 3.4 "Decoding Stage" steps 3-5): block reductions for
// 1024-thread workgroups, an exact MSB-first radix select of the k-th largest
// order-preserving key (and a sampled bracket that narrows it), and the
// ordered compaction that writes the selected indices ascending.  The keys
// come from LDS or from global memory (a key source).  Used by the standalone
// selection kernel and by the fused speculation kernel.
#pragma once

#include <climits>
#include <cmath>

#include "ig_device.h"

namespace ig {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelLdsKeys = 32768;  // rows per (b, h) held in LDS (up to 128 KB of dynamic LDS)
constexpr int kSelPerThread = 8;    // consecutive rows per thread in the compaction of rows in HBM

// mode values beyond the public ones: count-only pass of the head average
constexpr int kSelCountOnly = 100;

struct SelScratch {
    int hist[256];
    int wtot[kSelWaves];
    uint32_t wmax[kSelWaves];
    int bc[4];
};

// Sum over the first NT threads of the block (the ones still running).
template <int NT = kSelThreads>
__device__ __forceinline__ int block_sum(int v, SelScratch& sh) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    v = wave_sum_i32(v);
    if (lane == 0) sh.wtot[wave] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) t += sh.wtot[w];
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

// ------------------------------------------------------------------ rows streamed from HBM
// (the standalone selection of rows longer than the LDS key store: each pass streams the scores with
// coalesced loads, several in flight per lane)
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


// ------------------------------------------------------------------ radix select and compaction
// One 256-bin histogram per radix pass, three of them in rotation: pass p adds into buffer p % 3 and,
// after its barrier, clears buffer (p + 2) % 3 (last read in pass p - 1), so a pass needs a single
// barrier and every wave derives the digit on its own.  The histogram words are free after the
// select and stage the selected indices (kFastStage of them).
constexpr int kFastStage = 6144;
constexpr int kSampleBase = 1024;             // words[1024, 2048): one sampled key per thread
constexpr int kCandBase = 2048;               // words[2048, 6144): candidate keys of the sampled select
constexpr int kMaxCand = kFastStage - kCandBase;

struct __align__(16) FastSel {  // 16-byte aligned: the histograms are read 4 bins at a time
    uint32_t words[kFastStage];  // hist[3][256], samples and candidates during the select, then staging
    int wtot[kSelWaves];
    int wtot2[kSelWaves];
    __device__ uint32_t* hist(int i) { return words + 256 * i; }
    __device__ uint32_t* stage() { return words; }
};

// Clears histograms 0 and 1 (the first NT threads of the block); a barrier must follow before
// radix_kth_lds.
template <int NT = kSelThreads>
__device__ __forceinline__ void fast_sel_init(FastSel& fs) {
    for (int i = threadIdx.x; i < 512; i += NT) fs.words[i] = 0u;
}

// E consecutive keys of lk from j (j % E == 0, lk 16-byte aligned); positions at or past `end` read 0.
template <int E>
__device__ __forceinline__ void load_keys(const uint32_t* lk, int j, int end, uint32_t (&k)[E]) {
    if constexpr (E == 4) {
        if (j + 3 < end) {
            const uint4 v = *reinterpret_cast<const uint4*>(lk + j);
            k[0] = v.x; k[1] = v.y; k[2] = v.z; k[3] = v.w;
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) k[e] = j + e < end ? lk[j + e] : 0u;
}

// Key sources of the selection primitives: keys held in LDS (16-byte aligned), or a row of keys in
// global memory (any alignment, scalar loads).
struct LdsKeys {
    static constexpr int kE = 4;  // keys per lane per step on long rows (one 16-byte LDS read)
    const uint32_t* p;
    __device__ __forceinline__ uint32_t at(int j) const { return p[j]; }
    template <int E>
    __device__ __forceinline__ void load(int j, int end, uint32_t (&k)[E]) const { load_keys<E>(p, j, end, k); }
};
struct GlobalKeys {
    static constexpr int kE = 8;  // keys per lane per step on long rows (loads in flight together)
    const uint32_t* __restrict__ p;
    __device__ __forceinline__ uint32_t at(int j) const { return p[j]; }
    template <int E>
    __device__ __forceinline__ void load(int j, int end, uint32_t (&k)[E]) const {
#pragma unroll
        for (int e = 0; e < E; ++e) k[e] = j + e < end ? p[j + e] : 0u;
    }
};

// One radix pass: hist[digit] counts of the keys k >= base whose offset k - base has the bits above
// `shift + 8` equal to `prefix` (base 0: the keys themselves).
template <int NT, int E, class KS>
__device__ __forceinline__ void radix_hist(KS lk, int n, uint32_t* h, int shift, uint32_t prefix, uint32_t pmask,
                                           bool first, uint32_t base) {
    const int lane = threadIdx.x % kWave;
    for (int j0 = E * static_cast<int>(threadIdx.x); j0 < n; j0 += E * NT) {
        uint32_t k[E];
        lk.template load<E>(j0, n, k);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t kb = k[e] - base;
            const uint32_t bin = (kb >> shift) & 255u;
            bool on = j0 + e < n && k[e] >= base && (kb & pmask) == prefix;
            if (first) {
                // the first pass's keys crowd into the few bins of their sign and exponent bits, and
                // LDS atomics to one address serialise: the bin of the first active lane is counted
                // with one ballot and a single atomic
                const uint64_t act = __ballot(on);
                if (act != 0) {
                    const int leader = __ffsll(static_cast<unsigned long long>(act)) - 1;
                    const uint32_t b0 = static_cast<uint32_t>(read_lane(static_cast<int>(bin), leader));
                    const uint64_t m = __ballot(on && bin == b0);
                    if (lane == leader) atomicAdd(&h[b0], static_cast<uint32_t>(__popcll(m)));
                    on = on && bin != b0;
                }
            }
            if (on) atomicAdd(&h[bin], 1u);
        }
    }
}

// Exact kk-th largest key T of lk[0..n) (1 <= kk <= n; the first NT threads of the block take part,
// the others have exited; fast_sel_init and a barrier before).  Selecting every key above T and the
// first *need_eq keys equal to T gives the top kk; *eq_total keys equal T.  When a digit's whole bin
// belongs to the top kk the search stops early: T is then the bin's lowest key value (its low bits
// zero) and every key >= T is selected (*need_eq == *eq_total).  Ends after a barrier.
//
// With a known range base <= T <= hi (at least kk keys >= base, none above hi), only the keys >= base
// take part, as offsets k - base, and the passes start at the digit of the highest bit of hi - base:
// every offset of a key in range has the bits above it zero.  (base 0, hi ~0: every key, four passes.)
//
// Per pass: LDS atomics into that pass's histogram, one barrier, then every wave finds the digit on
// its own: lane L holds bins 255-4L .. 252-4L, a DPP prefix sum over the lanes gives the keys above
// each bin, and the lane holding the bin where the count reaches rem broadcasts it.
template <int NT = kSelThreads, class KS>
__device__ __forceinline__ void radix_kth_keys(KS lk, int n, int kk, FastSel& fs, uint32_t* T_out, int* need_eq_out,
                                               int* eq_total_out, uint32_t base = 0u, uint32_t hi = ~0u) {
    static_assert(NT >= 256, "a pass clears a 256-bin histogram with one thread per bin");
    const int tid = threadIdx.x, lane = tid % kWave;
    constexpr int E = KS::kE;
    const bool wide = n >= E * NT;
    const uint32_t span = hi - base;
    const int top = span ? (31 - __clz(static_cast<int>(span))) / 8 * 8 : 0;  // shift of the first pass
    uint32_t prefix = 0, pmask = top < 24 ? ~0u << (top + 8) : 0u;
    int rem = kk, dcount = 0;
    for (int pass = 0, shift = top; shift >= 0; ++pass, shift -= 8) {
        uint32_t* h = fs.hist(pass % 3);
        if (wide)
            radix_hist<NT, E>(lk, n, h, shift, prefix, pmask, pass == 0, base);
        else
            radix_hist<NT, 1>(lk, n, h, shift, prefix, pmask, pass == 0, base);
        __syncthreads();
        if (tid < 256) fs.hist((pass + 2) % 3)[tid] = 0u;
        const uint4 c4 = *reinterpret_cast<const uint4*>(h + 252 - 4 * lane);
        const int c[4] = {static_cast<int>(c4.w), static_cast<int>(c4.z), static_cast<int>(c4.y),
                          static_cast<int>(c4.x)};  // bins 255-4L, 254-4L, 253-4L, 252-4L
        const int s = c[0] + c[1] + c[2] + c[3];
        int cum = wave_incl_scan(s) - s;  // keys in the bins above 255-4L
        int digit = -1, above = 0, cnt = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (digit < 0 && cum < rem && cum + c[q] >= rem) {
                digit = 255 - 4 * lane - q;
                above = cum;
                cnt = c[q];
            }
            cum += c[q];
        }
        const uint64_t found = __ballot(digit >= 0);
        const int src = found ? __ffsll(static_cast<unsigned long long>(found)) - 1 : 0;
        digit = read_lane(digit, src) & 255;
        above = read_lane(above, src);
        dcount = read_lane(cnt, src);
        rem -= above;
        prefix |= static_cast<uint32_t>(digit) << shift;
        pmask |= 255u << shift;
        if (dcount == rem) break;  // the whole bin is taken
    }
    *T_out = base + prefix;
    *need_eq_out = rem;
    *eq_total_out = dcount;
}

template <int NT = kSelThreads>
__device__ __forceinline__ void radix_kth_lds(const uint32_t* lk, int n, int kk, FastSel& fs, uint32_t* T_out,
                                              int* need_eq_out, int* eq_total_out) {
    radix_kth_keys<NT>(LdsKeys{lk}, n, kk, fs, T_out, need_eq_out, eq_total_out);
}

// Keys >= kc among lk[0..n), summed over the first NT threads (ends after barriers).
template <int NT = kSelThreads, class KS>
__device__ __forceinline__ int count_ge(KS lk, int n, uint32_t kc, SelScratch& sh) {
    constexpr int E = KS::kE;
    int c = 0;
    if (n >= E * NT) {
        for (int j0 = E * static_cast<int>(threadIdx.x); j0 < n; j0 += E * NT) {
            uint32_t k[E];
            lk.template load<E>(j0, n, k);
#pragma unroll
            for (int e = 0; e < E; ++e) c += (j0 + e < n && k[e] >= kc) ? 1 : 0;
        }
    } else {
        for (int j = threadIdx.x; j < n; j += NT) c += lk.at(j) >= kc ? 1 : 0;
    }
    return block_sum<NT>(c, sh);
}

template <int NT = kSelThreads>
__device__ __forceinline__ int count_ge_lds(const uint32_t* lk, int n, uint32_t kc, SelScratch& sh) {
    return count_ge<NT>(LdsKeys{lk}, n, kc, sh);
}

// Ordered compaction of lk[0..n): the rows with key > T and the first need_eq rows with key == T (every
// row >= T when need_eq >= eq_total), ascending.  Each wave owns a contiguous chunk of whole groups of
// 64*E keys (E consecutive keys per lane): it counts its rows in registers, one barrier shares the
// per-wave counts, and a second pass places each group with DPP prefix sums over the lanes' counts,
// writing out[pos] = j and calling visit(pos, j).  Returns the number selected (block-uniform), or -1
// without placing anything when that number lies outside [win_lo, win_hi].  lk is read by other waves
// while visit runs, so a visitor must not write lk.
template <int NT, int E, class KS, typename Visit>
__device__ int compact_e(KS lk, int n, uint32_t T, int need_eq, int eq_total, int32_t* __restrict__ out, int max_out,
                         FastSel& fs, Visit visit, int win_lo = 0, int win_hi = INT_MAX) {
    constexpr int NW = NT / kWave, G = kWave * E;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const bool all_eq = need_eq >= eq_total;
    const int chunk = (n + NW * G - 1) / (NW * G) * G;
    const int lo = min(n, wave * chunk), hi = min(n, lo + chunk);
    int c_gt = 0, c_eq = 0;
    for (int j0 = lo + lane * E; j0 < hi; j0 += G) {
        uint32_t k[E];
        lk.template load<E>(j0, hi, k);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            c_gt += (j0 + e < hi && k[e] > T) ? 1 : 0;
            c_eq += (j0 + e < hi && k[e] == T) ? 1 : 0;
        }
    }
    // per-wave counts, prefix-summed over the waves
    const int w_gt = wave_sum_i32(c_gt), w_eq = wave_sum_i32(c_eq);
    if (lane == 0) {
        fs.wtot[wave] = w_gt;
        fs.wtot2[wave] = w_eq;
    }
    __syncthreads();
    const int incl_gt = wave_incl_scan(lane < NW ? fs.wtot[lane] : 0);
    const int incl_eq = wave_incl_scan(lane < NW ? fs.wtot2[lane] : 0);
    const int gt_before = wave > 0 ? read_lane(incl_gt, wave - 1) : 0;
    int eq_before = wave > 0 ? read_lane(incl_eq, wave - 1) : 0;
    const int gt_tot = read_lane(incl_gt, NW - 1), eq_tot = read_lane(incl_eq, NW - 1);
    const int take = all_eq ? eq_tot : min(eq_tot, need_eq);
    if (gt_tot + take < win_lo || gt_tot + take > win_hi) return -1;  // uniform: block-wide counts
    int pos = gt_before + min(eq_before, take);
    for (int g0 = lo; g0 < hi; g0 += G) {  // whole wave in step: the DPP scans need every lane
        const int j0 = g0 + lane * E;
        uint32_t k[E];
        lk.template load<E>(j0, hi, k);
        bool sel[E];
        int cs = 0;
        if (all_eq) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                sel[e] = j0 + e < hi && k[e] >= T;
                cs += sel[e] ? 1 : 0;
            }
        } else {
            int ce = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) ce += (j0 + e < hi && k[e] == T) ? 1 : 0;
            const int ie = wave_incl_scan(ce);
            int er = eq_before + ie - ce;  // rank among the equal keys of this lane's first equal key
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool valid = j0 + e < hi;
                const bool eq = valid && k[e] == T;
                sel[e] = (valid && k[e] > T) || (eq && er < need_eq);
                er += eq ? 1 : 0;
                cs += sel[e] ? 1 : 0;
            }
            eq_before += read_lane(ie, kWave - 1);
        }
        if (__ballot(cs != 0) == 0) continue;  // nothing selected in this group (uniform)
        const int is = wave_incl_scan(cs);
        int p = pos + is - cs;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (sel[e]) {
                if (p < max_out) {
                    if (out) out[p] = j0 + e;
                    visit(p, j0 + e);
                }
                ++p;
            }
        }
        pos += read_lane(is, kWave - 1);
    }
    return gt_tot + take;
}

template <int NT = kSelThreads, class KS, typename Visit = NoVisit>
__device__ int compact_keys(KS lk, int n, uint32_t T, int need_eq, int eq_total, int32_t* __restrict__ out,
                            int max_out, FastSel& fs, Visit visit, int win_lo = 0, int win_hi = INT_MAX) {
    if (n >= KS::kE * NT)
        return compact_e<NT, KS::kE>(lk, n, T, need_eq, eq_total, out, max_out, fs, visit, win_lo, win_hi);
    return compact_e<NT, 1>(lk, n, T, need_eq, eq_total, out, max_out, fs, visit, win_lo, win_hi);
}

template <int NT = kSelThreads, typename Visit = NoVisit>
__device__ int compact_lds(const uint32_t* lk, int n, uint32_t T, int need_eq, int eq_total,
                           int32_t* __restrict__ out, int max_out, FastSel& fs, Visit visit) {
    return compact_keys<NT>(LdsKeys{lk}, n, T, need_eq, eq_total, out, max_out, fs, visit);
}

// Top-kk cut of a long row through a sampled bracket.  One key per thread at a fixed stride gives a
// sample of NT keys; with e the expected sample count above the cut and m = 2.5 sqrt(e) + 4, the
// sample's (e + m)-th largest key L bounds the cut from below and, when e - m >= 1, its (e - m)-th
// largest key U bounds it from above (taken only when the keys >= L would not fit).  One pass over the row counts the keys >= U (c_hi) and copies the
// keys in [L, U) (the band) to LDS in any order.  When c_hi < kk <= c_hi + |band| and the band holds at
// most kMaxCand keys, the row's kk-th largest key is the band's (kk - c_hi)-th largest, found by the
// exact radix select on the band, and keys equal to it all lie in the band, so the counts it returns
// are the row's.  Without an upper bound the band is every key >= L.  Returns false (nothing decided;
// run the full radix) when a bound fails.  The selection is then every key above *T plus the first
// *need_eq keys equal to *T, *eq_total keys being equal to it.  Ends after a barrier.
template <int NT = kSelThreads, class KS>
__device__ bool sampled_kth(KS lk, int n, int kk, FastSel& fs, SelScratch& sh, uint32_t* T_out, int* need_eq_out,
                            int* eq_total_out, uint32_t* band = nullptr, int band_cap = kMaxCand) {
    const int tid = threadIdx.x, lane = tid % kWave;
    constexpr int E = KS::kE;
    if (n < 8 * NT) return false;
    const double expect = static_cast<double>(kk) * NT / n;
    const double margin = 2.5 * sqrt(expect) + 4.0;
    const int r_lo = static_cast<int>(expect + margin);
    const int r_hi = static_cast<int>(expect - margin);
    if (r_lo >= NT) return false;
    uint32_t* sample = fs.words + kSampleBase;
    uint32_t* cand = band ? band : fs.words + kCandBase;  // (a caller's band store: at least band_cap words)
    sample[tid] = lk.at(static_cast<int>(static_cast<int64_t>(tid) * n / NT));
    __syncthreads();
    uint32_t L, U = 0;
    int ne, et;
    // (an early exit gives a lower value: L is still a lower bound, and U is checked by the count)
    radix_kth_lds<NT>(sample, NT, r_lo, fs, &L, &ne, &et);
    // the upper bound only when the keys >= L are expected to overflow the candidate space
    const bool want_hi = r_hi >= 1 && static_cast<double>(r_lo) * n / NT > 0.75 * band_cap;
    if (want_hi) {
        __syncthreads();  // every wave has read the last histogram before it is cleared
        fast_sel_init<NT>(fs);
        __syncthreads();
        radix_kth_lds<NT>(sample, NT, r_hi, fs, &U, &ne, &et);
    }
    const bool has_hi = want_hi && U > L;
    if (tid == 0) fs.wtot[0] = 0;  // band keys placed so far
    __syncthreads();
    int c_hi = 0;
    for (int j0 = E * tid; j0 < n; j0 += E * NT) {  // E keys per lane
        uint32_t k[E];
        lk.template load<E>(j0, n, k);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool valid = j0 + e < n;
            const bool hi = valid && has_hi && k[e] >= U;
            const bool in = valid && !hi && k[e] >= L;
            c_hi += hi ? 1 : 0;
            // lane 0 holds the wave's lowest j0, so it is active whenever any lane is
            const uint64_t m = __ballot(in);
            if (m != 0) {
                int base = 0;
                if (lane == 0) base = atomicAdd(&fs.wtot[0], __popcll(m));
                base = read_lane(base, 0);
                const int pos = base + __popcll(m & lanemask_lt());
                if (in && pos < band_cap) cand[pos] = k[e];
            }
        }
    }
    __syncthreads();
    const int c_band = fs.wtot[0];
    c_hi = block_sum<NT>(c_hi, sh);
    if (c_hi >= kk || c_hi + c_band < kk || c_band > band_cap) {  // uniform: block-wide counts
        // the sample's passes left counts in the histograms: the full radix starts from clean ones
        fast_sel_init<NT>(fs);
        __syncthreads();
        return false;
    }
    fast_sel_init<NT>(fs);  // fresh histograms for the band select
    __syncthreads();
    uint32_t T;
    radix_kth_lds<NT>(cand, c_band, kk - c_hi, fs, &T, need_eq_out, eq_total_out);
    // an early exit leaves T at its bin's lowest value, which may lie below L: every band key at or
    // above it is selected, and those with the keys >= U are exactly the row's keys >= max(T, L)
    *T_out = T < L ? L : T;
    __syncthreads();
    return true;
}

// A bound for a superset of the top kk of ks[0..n) of at most `cap` keys: L = the sample's r-th
// largest key (r as in sampled_kth), so that about kk plus a margin keys are >= L.  Whether their count
// really lies in [kk, cap] (the top kk are then among them) is for the caller to check, e.g. with the
// window of compact_keys.  Returns false (nothing decided) when the row is too short to sample.  The
// sample's passes leave counts in the histograms (waves may still be reading the last one): a select
// that follows needs a barrier, then fast_sel_init and another barrier.
template <int NT = kSelThreads, class KS>
__device__ bool sampled_bound(KS lk, int n, int kk, int cap, FastSel& fs, uint32_t* L_out) {
    const int tid = threadIdx.x;
    if (n < 8 * NT || cap < kk) return false;
    const double expect = static_cast<double>(kk) * NT / n;
    const int r_lo = static_cast<int>(expect + 2.5 * sqrt(expect) + 4.0);
    if (r_lo >= NT) return false;
    uint32_t* sample = fs.words + kSampleBase;
    sample[tid] = lk.at(static_cast<int>(static_cast<int64_t>(tid) * n / NT));
    __syncthreads();
    int ne, et;
    radix_kth_lds<NT>(sample, NT, r_lo, fs, L_out, &ne, &et);
    return true;
}

template <int NT = kSelThreads>
__device__ bool sampled_kth_lds(const uint32_t* lk, int n, int kk, FastSel& fs, SelScratch& sh, uint32_t* T_out,
                                int* need_eq_out, int* eq_total_out) {
    return sampled_kth<NT>(LdsKeys{lk}, n, kk, fs, sh, T_out, need_eq_out, eq_total_out);
}

}  // namespace ig

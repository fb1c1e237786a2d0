// Fused speculation entry point: projection workgroups for the partial query,
// then one 1024-thread workgroup per (b, h) running spec_row (scores, selection
// and counters with the scores kept on chip), all in one launch.  Few rows, or
// rows longer than one workgroup's LDS: each row is cut into slices, one
// workgroup each, that leave their local selection as candidates, and a merge
// workgroup per row selects among them.  InfiniGen, arXiv 2406.19707,
// paper-graph-ui summary, section 3.4 "Decoding Stage" steps 1-3 and 5.
#include <algorithm>
#include <mutex>

#include "ig_spec_dev.h"

namespace ig {

template <typename T, int LPR>
__global__ __launch_bounds__(kSpecThreads, 8) void k_speculate(SpecParams p) {
    extern __shared__ __align__(16) uint32_t keys[];  // staged x (projection), or the slice's score keys
    __shared__ SpecShared<LPR * Vec<T>::N> sm;
    const int wg = blockIdx.x;
    if (wg < p.proj_wgs)
        proj_role<T>(p, wg, keys);
    else
        spec_row<T, LPR, 4>(p, wg - p.proj_wgs, keys, sm);
}

// One workgroup per row: the merge of the row's slices; in a decode layer whose attention is split, the
// same workgroup index also combines that attention's splits of (b, h) = blockIdx.x (B and H are shared).
template <typename T, int LPR>
__global__ __launch_bounds__(kSpecThreads) void k_spec_merge(SpecParams p, CombineArgs cb) {
    extern __shared__ __align__(16) uint32_t keys[];  // the candidates' keys (up to kSpecMaxRows), or scratch
    __shared__ SpecShared<LPR * Vec<T>::N> sm;
    // the combine's loads go out with the merge's first reads; its sums are formed after the merge
    CombinePre pre;
    const bool ahead = cb.part && cb.nsplit <= kCombinePre;
    if (ahead) combine_load(cb, blockIdx.x, pre);
    spec_merge<T, LPR>(p, blockIdx.x, keys, sm);
    if (ahead)
        combine_store(cb, blockIdx.x, pre);
    else if (cb.part)
        combine_item(cb, blockIdx.x);
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Candidate slots of a slice of `rows` of a row's n rows for a top-k selection of up to max_out rows
// with tight candidates: twice the slice's share of the budget with its margin (tight_slice_k on the
// device), and 64 more, so that a sampled bound of the slice's cut usually fits.
static int tight_cap(int max_out, int rows, int n) {
    const double e = static_cast<double>(max_out) * rows / n;
    const int want = static_cast<int>(std::ceil(e + 5.0 * std::sqrt(e) + 8.0));
    return std::min(rows, 2 * want + 64);
}

SlicePlan plan_slices(int64_t rows, int n, int max_out, bool topk) {
    // slices per row: enough for every row to fit in LDS, more (up to 16, at least 2048 rows each) when
    // there are too few rows to fill the chip; fewer while the merge's candidates would not fit its LDS,
    // down to what the occupancy needs (a merge over more candidates reads them from global memory).
    // Top-k rows that are sliced at all get slices of at most kTopkSliceRows rows (two workgroups per
    // CU, also beside attention workgroups) with tight candidates, whose merge stays small.
    const int s_min = (n + kSpecMaxRows - 1) / kSpecMaxRows;
    int S = static_cast<int>(std::min<int64_t>(kSpecMaxSlices, (256 + rows - 1) / rows));
    S = std::min(S, std::max(1, n / 2048));
    S = std::max(S, s_min);
    int slice_rows = 0, cap = 0;
    if (topk && S > 1) {
        S = std::max(S, std::min(kSpecMaxSlices, (n + kTopkSliceRows - 1) / kTopkSliceRows));
        slice_rows = (n + S - 1) / S;
        cap = tight_cap(max_out, slice_rows, n);
    } else {
        // candidate slots per slice: for large selections max_out and half again, so that a slice can hand
        // on every key above a sampled bound of its cut instead of finding the exact cut (small selections
        // find the exact cut cheaply, and more slots would only grow the merge)
        const int slack = max_out >= kSliceSlackMin
                              ? static_cast<int>(std::min<int64_t>(static_cast<int64_t>(max_out) + max_out / 2 + 64,
                                                                   INT32_MAX))
                              : max_out;
        for (;;) {
            slice_rows = (n + S - 1) / S;
            cap = std::min(slice_rows, slack);
            if (S == 1 || static_cast<int64_t>(S) * cap <= kSpecMaxRows || S == s_min) break;
            --S;
        }
    }
    SlicePlan pl{};
    pl.slices = (n + slice_rows - 1) / slice_rows;
    pl.ok = pl.slices <= kSpecMaxSlices;
    pl.slice_rows = pl.slices > 1 ? slice_rows : n;
    pl.cap = pl.slices > 1 ? cap : 0;
    return pl;
}

SpecPlan plan_speculate(int B, int H, int D, int r, int n, int max_out, int dtype, int mode) {
    SpecPlan sp{};
    const int64_t rows = static_cast<int64_t>(B) * H;
    // the workspace serves both modes (its size query knows no mode): regions sized for the larger plan
    const SlicePlan thr = plan_slices(rows, n, max_out, false);
    const SlicePlan tk = plan_slices(rows, n, max_out, true);
    // the head average: whole rows only (the threshold count needs the row's maximum), each handing on its
    // top min(n, max_out) as candidates
    SlicePlan ha = thr;
    ha.ok = thr.slices == 1;
    ha.cap = std::min(n, max_out);
    const SlicePlan& pl = mode == IG_SEL_TOPK ? tk : mode == IG_SEL_HEADAVG ? ha : thr;
    sp.ok = pl.ok;
    sp.slices = pl.slices;
    sp.slice_rows = pl.slice_rows;
    sp.cand_cap = pl.cap;
    sp.tight = mode == IG_SEL_TOPK && pl.slices > 1;
    sp.headavg = mode == IG_SEL_HEADAVG;
    const int s_max = std::max(thr.slices, tk.slices);
    const size_t ha_cands = ha.ok ? static_cast<size_t>(rows) * ha.cap : 0;
    const size_t cands = std::max(static_cast<size_t>(rows) * std::max(static_cast<size_t>(thr.slices) * thr.cap,
                                                                       static_cast<size_t>(tk.slices) * tk.cap),
                                  ha_cands);
    // projection workgroups: column blocks x splits of the D inputs
    sp.proj_blocks = (H * r + kProjCols - 1) / kProjCols;
    sp.splits = (D + kProjSplit - 1) / kProjSplit;
    sp.proj_wgs = sp.proj_blocks * sp.splits;
    sp.off_status = 0;  // status word at 0, shape stamp at 8 (one 256-byte region)
    // the rows' arrival words [B], then the bitmap counter kernels' per-sequence saturation flags [B]: both
    // must be zero on entry, so they sit where no other region reaches whatever n is
    sp.off_arrive = 256;
    sp.off_part = sp.off_arrive + align256(2 * static_cast<size_t>(B) * sizeof(uint32_t));
    sp.off_cnt = sp.off_part + align256(static_cast<size_t>(sp.splits) * B * H * r * sizeof(float));
    const bool sliced = s_max > 1 || ha.ok;  // (candidate regions: slices, or head-average rows)
    sp.off_lo = sp.off_cnt + (sliced ? align256(static_cast<size_t>(rows) * s_max * sizeof(int32_t)) : 0);
    sp.off_q = sp.off_lo + (sliced ? align256(static_cast<size_t>(rows) * s_max * sizeof(uint32_t)) : 0);
    sp.off_key = sp.off_q + (tk.slices > 1 ? align256(static_cast<size_t>(rows) * r * sizeof(float)) : 0);
    sp.off_idx = sp.off_key + (sliced ? align256(cands * sizeof(uint32_t)) : 0);
    // many selected slots per sequence: counter atomics in the merge would be throughput-bound
    auto uses_bits = [&](const SlicePlan& q) {
        return q.slices > 1 && H <= 128 && rows * std::min(max_out, n) >= kBitsTouchMin;
    };
    sp.bits = uses_bits(pl);
    const bool any_bits = uses_bits(thr) || uses_bits(tk);
    const size_t nw = (static_cast<size_t>(n) + 31) / 32;
    sp.off_bits = sp.off_idx + (sliced ? align256(cands * sizeof(int32_t)) : 0);
    sp.off_hcount = sp.off_bits + (any_bits ? align256(static_cast<size_t>(rows) * nw * sizeof(uint32_t)) : 0);
    sp.ws_bytes = sp.off_hcount + (ha.ok ? align256(static_cast<size_t>(rows) * sizeof(int32_t)) : 0);
    return sp;
}

size_t speculate_ws_bytes(int B, int H, int D, int r, int n, int max_out, int dtype) {
    return plan_speculate(B, H, D, r, n, max_out, dtype, IG_SEL_TOPK).ws_bytes;  // the same for every mode
}

// keys for the rows of a workgroup; at least the projection workgroups' slice results (which also
// covers the pool finish's argmin scratch of one word per thread)
size_t speculate_lds_bytes(int n) {
    const size_t w = static_cast<size_t>(std::max(n, kProjLdsWords));
    return w * sizeof(uint32_t);
}

template <typename T, int L>
static int launch_spec_tl(const SpecParams& p, hipStream_t s) {
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_speculate<T, L>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(speculate_lds_bytes(kSpecMaxRows)));
        if (e != hipSuccess) return static_cast<int>(e);
        attr_set = true;
    }
    hipLaunchKernelGGL((k_speculate<T, L>), dim3(p.proj_wgs + p.row_wgs), dim3(kSpecThreads),
                       speculate_lds_bytes(p.slice_rows), s, p);
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

template <typename T, int L>
static int launch_merge_tl(const SpecParams& p, const CombineArgs& cb, hipStream_t s) {
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_spec_merge<T, L>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(speculate_lds_bytes(kSpecMaxRows)));
        if (e != hipSuccess) return static_cast<int>(e);
        attr_set = true;
    }
    // the used candidates' keys and row indices (at most twice the slots, at most the LDS key store), or
    // the bitmap
    const int64_t m = static_cast<int64_t>(p.slices) * p.cand_cap;
    const int words = static_cast<int>(std::max<int64_t>(std::min<int64_t>(2 * m, kSpecMaxRows),
                                                         p.bits ? (p.n + 31) / 32 : 0));
    hipLaunchKernelGGL((k_spec_merge<T, L>), dim3(p.B * p.H), dim3(kSpecThreads), speculate_lds_bytes(words), s, p,
                       cb);
    return static_cast<int>(hipGetLastError());
}

template <typename T>
static int launch_merge_t(const SpecParams& p, const CombineArgs& cb, hipStream_t s) {
    switch (p.r / Vec<T>::N) {
        case 1: return launch_merge_tl<T, 1>(p, cb, s);
        case 2: return launch_merge_tl<T, 2>(p, cb, s);
        case 4: return launch_merge_tl<T, 4>(p, cb, s);
        case 8: return launch_merge_tl<T, 8>(p, cb, s);
        case 16: return launch_merge_tl<T, 16>(p, cb, s);
        case 32: return launch_merge_tl<T, 32>(p, cb, s);
        default: return static_cast<int>(hipErrorInvalidValue);
    }
}

// The merge launch of sliced rows; dtype and p.r pick the instance whose recompute reads the partial keys
// (a merge without tight candidates never recomputes: any instance serves it).  cb: an attention split
// combine to run in the same workgroups (part NULL: none).
int launch_spec_merge(const SpecParams& p, int dtype, hipStream_t s, const CombineArgs& cb) {
    if (!p.tight) return launch_merge_tl<float, 1>(p, cb, s);
    return dtype == IG_BF16 ? launch_merge_t<uint16_t>(p, cb, s) : launch_merge_t<float>(p, cb, s);
}

// Failure-path testing (ig_set_handover_test_mode): the row workgroups' poll limit, and whether the
// projection workgroups withhold their partial sums.  Process-wide; read when a call is launched.
static uint32_t g_spin_limit = kProjSpinLimit;
static int g_withhold = 0;

void set_handover_test_mode(uint32_t spin_limit, int withhold) {
    g_spin_limit = spin_limit ? spin_limit : kProjSpinLimit;
    g_withhold = withhold ? 1 : 0;
}

unsigned long long spec_shape_key(int B, int H, int D, int r) {
    // B < 2^16, H < 2^16, D < 2^22, r <= 256 (checked by the callers); the top bit keeps it nonzero
    return (1ull << 63) | (static_cast<unsigned long long>(B) << 47) | (static_cast<unsigned long long>(H) << 31) |
           (static_cast<unsigned long long>(D) << 9) | static_cast<unsigned long long>(r - 1);
}

int begin_speculate(const SpecCall& c, SpecParams* p) {
    const SpecPlan sp = plan_speculate(c.B, c.H, c.D, c.r, c.n, c.max_out, c.dtype, c.mode);
    char* ws = static_cast<char*>(c.ws);
    // all batch rows of a head on one XCD when the heads split evenly over the 8 XCDs
    *p = SpecParams{c.x, c.Wq_part, c.D, reinterpret_cast<float*>(ws + sp.off_part), sp.splits, c.bq_part, c.Kp, c.B,
                    c.H, c.r, c.n, c.n_cap, c.ld, c.scale, c.mode, c.alpha,
                    c.k, c.max_sel, c.max_out, c.idx, c.count, c.q_part, c.scores, c.counters, c.cmax, c.victim,
                    reinterpret_cast<uint32_t*>(ws + sp.off_arrive), c.H % 8 == 0 ? 1 : 0, sp.slices, sp.slice_rows,
                    sp.cand_cap, reinterpret_cast<uint32_t*>(ws + sp.off_key), reinterpret_cast<int32_t*>(ws + sp.off_idx),
                    reinterpret_cast<int32_t*>(ws + sp.off_cnt)};
    if (sp.bits && c.counters) p->bits = reinterpret_cast<uint32_t*>(ws + sp.off_bits);
    p->proj_wgs = sp.proj_wgs;
    p->proj_blocks = sp.proj_blocks;
    p->row_wgs = c.B * c.H * sp.slices;
    p->status = reinterpret_cast<uint32_t*>(ws + sp.off_status);
    p->stamp = reinterpret_cast<unsigned long long*>(ws + sp.off_status + 8);
    p->key = spec_shape_key(c.B, c.H, c.D, c.r);
    p->spin_limit = g_spin_limit;
    p->withhold = g_withhold;
    p->tight = sp.tight ? 1 : 0;
    if (sp.slices > 1) p->cand_lo = reinterpret_cast<uint32_t*>(ws + sp.off_lo);
    if (sp.tight) p->q_rows = reinterpret_cast<float*>(ws + sp.off_q);
    if (sp.headavg) p->hcount = reinterpret_cast<int32_t*>(ws + sp.off_hcount);
    return 0;
}

int launch_speculate(const void* x, const void* Wq_part, const float* bq_part, const void* Kp, int B, int D, int H,
                     int r, int n, int n_cap, int dtype, float scale, int mode, float alpha, int k, int max_sel,
                     int32_t* idx, int32_t* count, int max_out, uint32_t* counters, uint32_t cmax, int32_t* victim,
                     float* q_part, float* scores, int ld, void* ws, hipStream_t s) {
    const SpecCall c{x, Wq_part, bq_part, Kp, B, D, H, r, n, n_cap, dtype, scale, mode, alpha, k, max_sel, idx, count,
                     max_out, counters, cmax, victim, q_part, scores, ld, ws};
    SpecParams p;
    int e = begin_speculate(c, &p);
    if (e) return e;
    e = dtype == IG_BF16 ? launch_spec_t<uint16_t>(p, s) : launch_spec_t<float>(p, s);
    if (e || (p.slices == 1 && p.mode != IG_SEL_HEADAVG)) return e;
    return finish_speculate(p, dtype, ws, s);
}

// After the launch of sliced rows: the merge, and the counter kernels when the merge leaves bitmaps.
int finish_speculate(const SpecParams& p, int dtype, void* ws, hipStream_t s, const CombineArgs& cb) {
    int e = launch_spec_merge(p, dtype, s, cb);
    if (e || !p.bits) return e;
    const SpecPlan sp = plan_speculate(p.B, p.H, p.D, p.r, p.n, p.max_out, dtype, p.mode);
    return launch_touch_bits(p.counters, p.bits, p.B, p.H, p.n, p.n_cap, p.cmax,
                             reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + sp.off_arrive) + p.B, p.victim, s);
}

// ------------------------------------------------------------------ ig_speculate_noalloc
// The speculation workspace of callers that cannot allocate: a file-scope device array, one copy per
// GPU (each GPU the library runs on holds it until the process ends).  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol): the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (hipError_t as int).
static int noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return static_cast<int>(e);
    if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return static_cast<int>(e);
        if (!ptr) return static_cast<int>(hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return 0;
}

// Start of a no-allocation call: every word of [0, words) to zero except the shape stamp (words 2-3),
// which gets this call's key.
__global__ void k_scratch_reset(uint32_t* ws, size_t words, unsigned long long key) {
    const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < words) ws[i] = i == 2 ? static_cast<uint32_t>(key) : i == 3 ? static_cast<uint32_t>(key >> 32) : 0u;
}

int launch_speculate_noalloc(const SpecCall& c, hipStream_t s) {
    const SpecPlan sp = plan_speculate(c.B, c.H, c.D, c.r, c.n, c.max_out, c.dtype, c.mode);
    if (sp.ws_bytes > kNoAllocScratchBytes) return static_cast<int>(hipErrorInvalidValue);  // checked before
    void* ws = nullptr;
    int e = noalloc_scratch(&ws);
    if (e) return e;
    // the status word, the stamp, the arrival words and flags and the partial-sum slots come first
    // (off_cnt is where the candidates start); the candidates and bitmaps are written before they are
    // read in every call
    const size_t words = sp.off_cnt / sizeof(uint32_t);
    hipLaunchKernelGGL(k_scratch_reset, dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256), 0, s,
                       static_cast<uint32_t*>(ws), words, spec_shape_key(c.B, c.H, c.D, c.r));
    if ((e = static_cast<int>(hipGetLastError()))) return e;
    return launch_speculate(c.x, c.Wq_part, c.bq_part, c.Kp, c.B, c.D, c.H, c.r, c.n, c.n_cap, c.dtype, c.scale,
                            c.mode, c.alpha, c.k, c.max_sel, c.idx, c.count, c.max_out, c.counters, c.cmax, c.victim,
                            c.q_part, c.scores, c.ld, ws, s);
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

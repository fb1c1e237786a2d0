// One decode layer in one launch (InfiniGen, arXiv 2406.19707, paper-graph-ui
// summary, section 3.2 "Big-Picture Architecture", KV Selection Controller:
// the speculation for the next layer runs while the current layer computes,
// from the current layer's attention input; section 3.4 "Decoding Stage"):
// the attention of layer l over the rows its speculation selected, beside the
// speculation for layer l+1 (scores, selection and counters).
//
// One grid holds three roles: the partial-query projection workgroups for
// layer l+1 first, then one spec_row workgroup per (b, h) (or per slice of a
// long row) for layer l+1, which waits only for the projection workgroups
// (lower indices, never waiting themselves), then the attention items of
// layer l (one (b, h, split) each, all 1024 threads of the workgroup on it).
// The attention items take the slots the rows leave as they finish, so the
// two roles overlap where the speculation's rows end and are in their
// latency-bound selection.  (With long rows cut into slices, placing the
// attention items among the slices instead measured slower: their scattered
// K/V row reads and the slices' partial-key streams share the memory system
// worse than the two phases do one after the other.)  The attention and the
// speculation touch disjoint buffers; a CU holds two workgroups.  Sliced rows
// are merged by a launch of their own, which also combines the attention's
// splits; otherwise the usual combine kernel follows.
#include "ig_attn_dev.h"
#include "ig_spec_dev.h"

namespace ig {

constexpr int kDecodeThreads = 1024;

template <int R, int LPR_A, int VEC>
union DecodeShared {
    SpecShared<R> spec;
    AttnShared<kDecodeThreads, LPR_A, VEC> attn;
};

// Two 1024-thread workgroups per CU (8 waves per SIMD, at most 64 VGPRs each), so that one workgroup
// of each role fits on a CU at once (the second launch bound is the minimum number of waves per SIMD).
// Rows in flight per lane: 4 partial-key rows (double buffered; the most that keep the registers
// without spills) and ROWS K/V rows per attention lane group: 1 when an attention item's rows fit
// two passes of one row per lane group (the attention then takes less of the memory system while
// the rows stream their partial keys: measured faster at 128 rows per item), else 2 (measured
// faster at 205-218 rows per item).
constexpr int kDecodeSpecBatch = 4;

template <typename T, int LPR_S, int LPR_A, int ROWS>
__global__ __launch_bounds__(kDecodeThreads, 8) void k_decode_layer(SpecParams p, AttnArgs a, int bh_attn) {
    extern __shared__ __align__(16) uint32_t keys[];  // staged x (projection) or the speculation's score keys
    __shared__ DecodeShared<LPR_S * Vec<T>::N, LPR_A, Vec<T>::N> sm;
    const int wg = blockIdx.x;
    if (wg < p.proj_wgs) {
        proj_role<T>(p, wg, keys);
        return;
    }
    // every row workgroup (or slice) first, then the attention items
    const int c = wg - p.proj_wgs;
    if (c < p.row_wgs) {
        spec_row<T, LPR_S, kDecodeSpecBatch>(p, c, keys, sm.spec);
    } else {
        const int item = c - p.row_wgs;
        attn_item<T, LPR_A, kDecodeThreads, ROWS>(a, item % bh_attn, item / bh_attn, sm.attn);
    }
}

template <typename T, int LPR_S, int LPR_A, int ROWS>
static int launch_fused(const SpecParams& p, const AttnArgs& a, int bh_attn, hipStream_t s) {
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_decode_layer<T, LPR_S, LPR_A, ROWS>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(speculate_lds_bytes(kDecodeMaxRows)));
        if (e != hipSuccess) return static_cast<int>(e);
        attr_set = true;
    }
    const int items = a.nsplit * bh_attn;
    const int grid = p.proj_wgs + p.row_wgs + items;
    hipLaunchKernelGGL((k_decode_layer<T, LPR_S, LPR_A, ROWS>), dim3(grid), dim3(kDecodeThreads),
                       speculate_lds_bytes(p.slice_rows), s, p, a, bh_attn);
    return static_cast<int>(hipGetLastError());
}

// lanes per partial-key row (r / elements per 16 bytes) and per K/V row (d / elements per 16 bytes)
static int lpr_of(int len, int dtype) { return len / (dtype == IG_BF16 ? 8 : 4); }

bool decode_fusable(const AttnCall& a, const SpecCall& s) {
    const int ls = lpr_of(s.r, s.dtype), la = lpr_of(a.d, a.dtype);
    const SpecPlan sp = plan_speculate(s.B, s.H, s.D, s.r, s.n, s.max_out, s.dtype, s.mode);
    // whole rows up to kDecodeMaxRows keys, or slices small enough for two workgroups per CU
    const bool rows_ok = sp.slices == 1 ? s.n <= kDecodeMaxRows : sp.slice_rows <= kTopkSliceRows;
    return a.dtype == s.dtype && sp.ok && rows_ok && (ls == 2 || ls == 4 || ls == 8) &&
           (la == 8 || la == 16 || la == 32);
}

template <typename T, int LPR_S, int LPR_A>
static int launch_fused_r(const SpecParams& p, const AttnArgs& a, int bh_attn, hipStream_t s) {
    // one K/V row per lane group when an item's rows fit two passes of that, else two
    if (a.rows_per_split <= 2 * (kDecodeThreads / LPR_A)) return launch_fused<T, LPR_S, LPR_A, 1>(p, a, bh_attn, s);
    return launch_fused<T, LPR_S, LPR_A, 2>(p, a, bh_attn, s);
}

template <typename T, int LPR_S>
static int launch_fused_s(const SpecParams& p, const AttnArgs& a, int la, int bh_attn, hipStream_t s) {
    switch (la) {
        case 8: return launch_fused_r<T, LPR_S, 8>(p, a, bh_attn, s);
        case 16: return launch_fused_r<T, LPR_S, 16>(p, a, bh_attn, s);
        case 32: return launch_fused_r<T, LPR_S, 32>(p, a, bh_attn, s);
        default: return static_cast<int>(hipErrorInvalidValue);
    }
}

template <typename T>
static int launch_fused_t(const SpecParams& p, const AttnArgs& a, int ls, int la, int bh_attn, hipStream_t s) {
    switch (ls) {
        case 2: return launch_fused_s<T, 2>(p, a, la, bh_attn, s);
        case 4: return launch_fused_s<T, 4>(p, a, la, bh_attn, s);
        case 8: return launch_fused_s<T, 8>(p, a, la, bh_attn, s);
        default: return static_cast<int>(hipErrorInvalidValue);
    }
}

static int launch_attn_call(const AttnCall& c, hipStream_t s) {
    return launch_attn(c.q, c.K, c.V, c.ld_rows, c.idx, c.count, c.B, c.H, c.d, c.max_out, c.dtype, c.scale, c.out,
                       c.lse, c.ws, s);
}

static int launch_spec_call(const SpecCall& c, hipStream_t s) {
    return launch_speculate(c.x, c.Wq_part, c.bq_part, c.Kp, c.B, c.D, c.H, c.r, c.n, c.n_cap, c.dtype, c.scale,
                            c.mode, c.alpha, c.k, c.max_sel, c.idx, c.count, c.max_out, c.counters, c.cmax, c.victim,
                            c.q_part, c.scores, c.ld, c.ws, s);
}

int launch_decode_layer(const AttnCall* a, const SpecCall* sc, hipStream_t s) {
    if (!a) return launch_spec_call(*sc, s);
    if (!sc) return launch_attn_call(*a, s);
    if (!decode_fusable(*a, *sc)) {
        const int e = launch_spec_call(*sc, s);
        return e ? e : launch_attn_call(*a, s);
    }
    SpecParams p;
    int e = begin_speculate(*sc, &p);
    if (e) return e;
    const AttnPlan ap = plan_attn(a->B, a->H, a->d, a->max_out);
    const AttnArgs aa{a->q, a->K, a->V, a->ld_rows, a->idx, a->count, a->d, a->max_out, ap.rows_per_split, ap.nsplit,
                      a->scale, a->out, a->lse, static_cast<float*>(a->ws)};
    const int bh = a->B * a->H;
    e = a->dtype == IG_BF16 ? launch_fused_t<uint16_t>(p, aa, lpr_of(sc->r, sc->dtype), lpr_of(a->d, a->dtype), bh, s)
                            : launch_fused_t<float>(p, aa, lpr_of(sc->r, sc->dtype), lpr_of(a->d, a->dtype), bh, s);
    if (e) return e;
    if (p.slices > 1 || p.mode == IG_SEL_HEADAVG) {
        // the merge (whose workgroups also combine the attention's splits), then the counters
        const CombineArgs cb{ap.nsplit > 1 ? aa.part : nullptr, ap.nsplit, a->d, a->out, a->lse};
        return finish_speculate(p, sc->dtype, sc->ws, s, cb);
    }
    if (ap.nsplit == 1) return 0;
    return launch_attn_combine(aa.part, ap.nsplit, a->d, bh, a->out, a->lse, s);
}

}  // namespace ig

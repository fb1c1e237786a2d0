// C ABI of the InfiniGen decode hot path (include/ig.h): argument validation,
// error reporting and dispatch to the kernel launchers.  Every check happens
// on the host before anything is enqueued, so an IG_EINVAL call writes
// nothing.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include <hip/hip_runtime.h>

#include "ig_internal.h"

namespace ig {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return IG_OK;
}

static int hip_status(int e, const char* what) {
    if (e == 0) return ok();
    return fail(IG_EHIP, "%s: HIP error %d (%s)", what, e, hipGetErrorString(static_cast<hipError_t>(e)));
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int elem_size(int dtype) { return dtype == IG_BF16 ? 2 : 4; }

static bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// d / (16 / element size) must be 4, 8, 16 or 32 lanes per row
static bool head_dim_ok(int d, int dtype) {
    const int vec = 16 / elem_size(dtype);
    if (d % vec) return false;
    const int lpr = d / vec;
    return pow2(lpr) && lpr >= 4 && lpr <= 32;
}

#define IG_REQUIRE(cond, ...)                                  \
    do {                                                       \
        if (!(cond)) return fail(IG_EINVAL, __VA_ARGS__);      \
    } while (0)

#define IG_REQUIRE_DTYPE(fn, dtype) IG_REQUIRE((dtype) == IG_F32 || (dtype) == IG_BF16, fn ": unknown dtype %d", dtype)

}  // namespace ig

using namespace ig;

extern "C" {

const char* ig_last_error(void) { return g_err; }

int ig_version(void) { return 11; }

int ig_skew_weights(const ig_skew_args* args) { return skew_weights(args); }

int ig_skew_apply(const double* A, int H, int d, const double* M, int64_t rows, double* out, int nthreads) {
    return skew_apply(A, H, d, M, rows, out, nthreads);
}

int ig_store(const double* vals, int64_t count, int dtype, void* out) { return store(vals, count, dtype, out); }

int ig_partial_weight_index(const void* Wq_s, int D, int H, int d, int r, const void* K_s, int B, int n_cap, int n,
                            int dtype, int32_t* chan, void* Wq_part, int nthreads) {
    return partial_weight_index(Wq_s, D, H, d, r, K_s, B, n_cap, n, dtype, chan, Wq_part, nthreads);
}

size_t ig_workspace_size(int op, int B, int H, int D, int d, int r, int n, int max_out) {
    if (B < 1 || H < 1) return 0;
    switch (op) {
        case IG_OP_REHEARSE:
            if (D < 1 || r < 1 || n < 1) return 0;
            return plan_rehearse(B, H, D, r, n, IG_BF16).ws_bytes;
        case IG_OP_SELECT:
            return select_ws_bytes(B, H, n, max_out);
        case IG_OP_ATTN:
            if (d < 1 || max_out < 1) return 0;
            return plan_attn(B, H, d, max_out).ws_bytes;
        case IG_OP_TOUCH:
            if (max_out < 1) return 0;
            return touch_single_kernel(H, max_out) ? 0 : touch_ws_bytes(B);
        case IG_OP_SPECULATE:
            if (D < 1 || r < 1 || n < 1) return 0;
            return speculate_ws_bytes(B, H, D, r, n, max_out, IG_BF16);
        case IG_OP_SETUP:
            if (D < 1 || d < 1 || n < 1) return 0;
            return plan_setup(B, H, d, D, n).ws_bytes;
        default:
            return 0;
    }
}

int ig_rehearse(const void* x, const void* Wq_part, const float* bq_part, const void* Kp, int B, int D, int H, int r,
                int n, int n_cap, int dtype, float scale, float* q_part, float* scores, int ld, void* ws,
                size_t ws_bytes, hipStream_t stream) {
    IG_REQUIRE_DTYPE("ig_rehearse", dtype);
    IG_REQUIRE(x && Wq_part && Kp && q_part && scores, "ig_rehearse: NULL required pointer");
    IG_REQUIRE(B >= 1 && D >= 1 && H >= 1 && r >= 1 && n >= 1 && n <= n_cap && ld >= n,
               "ig_rehearse: bad sizes (B=%d D=%d H=%d r=%d n=%d n_cap=%d ld=%d)", B, D, H, r, n, n_cap, ld);
    IG_REQUIRE(r % 8 == 0 && pow2(r / (16 / elem_size(dtype))) && r / (16 / elem_size(dtype)) <= 32,
               "ig_rehearse: r / (16 / element size) must be a power of two <= 32 (got r=%d)", r);
    IG_REQUIRE(std::isfinite(scale), "ig_rehearse: scale must be finite");
    IG_REQUIRE(aligned16(x) && aligned16(Wq_part) && aligned16(Kp), "ig_rehearse: x, Wq_part and Kp must be 16-byte aligned");
    IG_REQUIRE(D % (16 / elem_size(dtype)) == 0, "ig_rehearse: D must be a multiple of 16 / element size (got D=%d)", D);
    const RehearsePlan p = plan_rehearse(B, H, D, r, n, dtype);
    IG_REQUIRE(ws && ws_bytes >= p.ws_bytes, "ig_rehearse: workspace of %zu bytes needed (got %zu)", p.ws_bytes,
               ws ? ws_bytes : static_cast<size_t>(0));
    return hip_status(launch_rehearse(x, Wq_part, bq_part, Kp, B, D, H, r, n, n_cap, dtype, scale, q_part, scores,
                                      ld, ws, stream),
                      "ig_rehearse");
}

int ig_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
    IG_REQUIRE(ws || ws_bytes == 0, "ig_workspace_init: NULL workspace");
    IG_REQUIRE(aligned16(ws), "ig_workspace_init: workspace must be 16-byte aligned");
    return hip_status(launch_zero(ws, ws_bytes, stream), "ig_workspace_init");
}

int ig_workspace_status(const void* ws, size_t ws_bytes, uint32_t* status, uint32_t* recomputed,
                        hipStream_t stream) {
    IG_REQUIRE(ws && status && ws_bytes >= 256, "ig_workspace_status: NULL workspace or status, or fewer than 256 "
               "bytes");
    uint32_t v[5] = {0, 0, 0, 0, 0};
    hipError_t e = hipMemcpyAsync(v, ws, sizeof(v), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_status(static_cast<int>(e), "ig_workspace_status");
    *status = v[0];
    if (recomputed) *recomputed = v[4];
    return ok();
}

int ig_set_handover_test_mode(uint32_t spin_limit, int withhold) {
    set_handover_test_mode(spin_limit, withhold);
    return ok();
}

// Validation of a speculation call (ig_speculate, and the speculation half of ig_decode_layer).
// noalloc: the workspace is the library's static scratch (ig_speculate_noalloc).
static int check_spec(const char* fn, const SpecCall& c, size_t ws_bytes, bool noalloc = false) {
    const int dtype = c.dtype, B = c.B, D = c.D, H = c.H, r = c.r, n = c.n, n_cap = c.n_cap, max_out = c.max_out;
    IG_REQUIRE(dtype == IG_F32 || dtype == IG_BF16, "%s: unknown dtype %d", fn, dtype);
    IG_REQUIRE(c.x && c.Wq_part && c.Kp && c.idx && c.count, "%s: NULL required pointer", fn);
    IG_REQUIRE(B >= 1 && D >= 1 && H >= 1 && r >= 1 && n >= 1 && n <= n_cap && max_out >= 1,
               "%s: bad sizes (B=%d D=%d H=%d r=%d n=%d n_cap=%d max_out=%d)", fn, B, D, H, r, n, n_cap, max_out);
    IG_REQUIRE(r % 8 == 0 && pow2(r / (16 / elem_size(dtype))) && r / (16 / elem_size(dtype)) <= 32,
               "%s: r / (16 / element size) must be a power of two <= 32 (got r=%d)", fn, r);
    IG_REQUIRE(!c.scores || c.ld >= n, "%s: ld must be >= n when scores are written", fn);
    IG_REQUIRE(std::isfinite(c.scale), "%s: scale must be finite", fn);
    IG_REQUIRE(aligned16(c.x) && aligned16(c.Wq_part) && aligned16(c.Kp), "%s: x, Wq_part and Kp must be 16-byte aligned",
               fn);
    IG_REQUIRE(D % (16 / elem_size(dtype)) == 0, "%s: D must be a multiple of 16 / element size (got D=%d)", fn, D);
    if (c.mode == IG_SEL_THRESHOLD)
        IG_REQUIRE(c.alpha >= 0.f && !std::isnan(c.alpha) && c.max_sel >= 0, "%s: alpha must be >= 0", fn);
    else if (c.mode == IG_SEL_TOPK)
        IG_REQUIRE(c.k >= 1, "%s: k must be >= 1", fn);
    else if (c.mode == IG_SEL_HEADAVG)
        IG_REQUIRE(c.alpha >= 0.f && !std::isnan(c.alpha) && c.max_sel >= 0, "%s: alpha must be >= 0", fn);
    else
        return fail(IG_EINVAL, "%s: unknown mode %d", fn, c.mode);
    const SpecPlan plan = plan_speculate(B, H, D, r, n, max_out, dtype, c.mode);
    if (!plan.ok && c.mode == IG_SEL_HEADAVG)
        return fail(IG_EUNSUPPORTED, "%s: the head-average mode needs rows held whole by one workgroup (n <= %d "
                    "and enough rows to fill the chip); use ig_rehearse + ig_select", fn, kSpecMaxRows);
    if (!plan.ok)
        return fail(IG_EUNSUPPORTED, "%s: n = %d needs more than %d slices of %d rows; use ig_rehearse + "
                    "ig_select", fn, n, kSpecMaxSlices, kSpecMaxRows);
    IG_REQUIRE(!c.counters || c.cmax >= 2, "%s: cmax must be >= 2", fn);
    IG_REQUIRE(H <= 0xFFFF && B <= 0xFFFF && D < (1 << 22), "%s: at most 65535 heads and batch rows and "
               "D < 2^22 (the workspace stamp)", fn);
    const size_t need = plan.ws_bytes;
    if (noalloc) {
        IG_REQUIRE(need <= kNoAllocScratchBytes, "%s: the call needs %zu bytes of scratch, more than the %zu "
                   "bytes of the static scratch; use ig_speculate with a workspace", fn, need, kNoAllocScratchBytes);
        return IG_OK;
    }
    IG_REQUIRE(c.ws && ws_bytes >= need, "%s: workspace of %zu bytes needed", fn, need);
    IG_REQUIRE(aligned16(c.ws), "%s: workspace must be 16-byte aligned", fn);
    return IG_OK;
}

int ig_speculate(const void* x, const void* Wq_part, const float* bq_part, const void* Kp, int B, int D, int H, int r,
                 int n, int n_cap, int dtype, float scale, int mode, float alpha, int k, int max_sel, int32_t* idx,
                 int32_t* count, int max_out, uint32_t* counters, uint32_t cmax, int32_t* victim, float* q_part,
                 float* scores, int ld, void* ws, size_t ws_bytes, hipStream_t stream) {
    const SpecCall c{x, Wq_part, bq_part, Kp, B, D, H, r, n, n_cap, dtype, scale, mode, alpha, k, max_sel, idx, count,
                     max_out, counters, cmax, victim, q_part, scores, ld, ws};
    if (const int e = check_spec("ig_speculate", c, ws_bytes)) return e;
    return hip_status(launch_decode_layer(nullptr, &c, stream), "ig_speculate");
}

int ig_speculate_noalloc(const void* x, const void* Wq_part, const float* bq_part, const void* Kp, int B, int D,
                         int H, int r, int n, int n_cap, int dtype, float scale, int mode, float alpha, int k,
                         int max_sel, int32_t* idx, int32_t* count, int max_out, uint32_t* counters, uint32_t cmax,
                         int32_t* victim, float* q_part, float* scores, int ld, hipStream_t stream) {
    const SpecCall c{x, Wq_part, bq_part, Kp, B, D, H, r, n, n_cap, dtype, scale, mode, alpha, k, max_sel, idx, count,
                     max_out, counters, cmax, victim, q_part, scores, ld, nullptr};
    if (const int e = check_spec("ig_speculate_noalloc", c, 0, true)) return e;
    return hip_status(launch_speculate_noalloc(c, stream), "ig_speculate_noalloc");
}

int ig_select(const float* scores, int B, int H, int n, int ld, int mode, float alpha, int k, int max_sel,
              int32_t* idx, int32_t* count, int max_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    IG_REQUIRE(scores && idx && count, "ig_select: NULL required pointer");
    IG_REQUIRE(B >= 1 && H >= 1 && n >= 1 && ld >= n && max_out >= 1,
               "ig_select: bad sizes (B=%d H=%d n=%d ld=%d max_out=%d)", B, H, n, ld, max_out);
    IG_REQUIRE(mode == IG_SEL_THRESHOLD || mode == IG_SEL_TOPK || mode == IG_SEL_HEADAVG,
               "ig_select: unknown mode %d", mode);
    IG_REQUIRE(max_sel >= 0, "ig_select: max_sel must be >= 0");
    if (mode != IG_SEL_TOPK)
        IG_REQUIRE(alpha >= 0.f && !std::isnan(alpha), "ig_select: alpha must be >= 0 (inf allowed)");
    else
        IG_REQUIRE(k >= 1, "ig_select: k must be >= 1");
    const size_t need = select_needs_ws(B, H, n, max_out, mode) ? select_ws_bytes(B, H, n, max_out) : 0;
    IG_REQUIRE(need == 0 || (ws && ws_bytes >= need), "ig_select: workspace of %zu bytes needed", need);
    return hip_status(launch_select(scores, B, H, n, ld, mode, alpha, k, max_sel, idx, count, max_out, ws, stream),
                      "ig_select");
}

int ig_gather_kv(const void* K, const void* V, const int32_t* idx, const int32_t* count, int B, int H, int d,
                 int n_cap, int max_out, int dtype, void* Kc, void* Vc, hipStream_t stream) {
    IG_REQUIRE_DTYPE("ig_gather_kv", dtype);
    IG_REQUIRE(K && V && idx && count && Kc && Vc, "ig_gather_kv: NULL required pointer");
    IG_REQUIRE(B >= 1 && H >= 1 && n_cap >= 1 && max_out >= 1, "ig_gather_kv: bad sizes");
    IG_REQUIRE(head_dim_ok(d, dtype), "ig_gather_kv: unsupported head dim %d", d);
    IG_REQUIRE(aligned16(K) && aligned16(V) && aligned16(Kc) && aligned16(Vc),
               "ig_gather_kv: K, V, Kc, Vc must be 16-byte aligned");
    return hip_status(launch_gather(K, V, idx, count, B, H, d, n_cap, max_out, dtype, Kc, Vc, stream),
                      "ig_gather_kv");
}

// Validation of an attention call (ig_sparse_decode_attn, and the attention half of ig_decode_layer).
static int check_attn(const char* fn, const AttnCall& c, size_t ws_bytes) {
    const int dtype = c.dtype, B = c.B, H = c.H, d = c.d, max_out = c.max_out;
    IG_REQUIRE(dtype == IG_F32 || dtype == IG_BF16, "%s: unknown dtype %d", fn, dtype);
    IG_REQUIRE(c.q && c.K && c.V && c.count && c.out, "%s: NULL required pointer", fn);
    IG_REQUIRE(B >= 1 && H >= 1 && c.ld_rows >= 1 && max_out >= 1, "%s: bad sizes (B=%d H=%d ld_rows=%d max_out=%d)",
               fn, B, H, c.ld_rows, max_out);
    IG_REQUIRE(head_dim_ok(d, dtype), "%s: unsupported head dim %d", fn, d);
    IG_REQUIRE(std::isfinite(c.scale), "%s: scale must be finite", fn);
    IG_REQUIRE(aligned16(c.q) && aligned16(c.K) && aligned16(c.V), "%s: q, K, V must be 16-byte aligned", fn);
    const AttnPlan p = plan_attn(B, H, d, max_out);
    IG_REQUIRE(p.ws_bytes == 0 || (c.ws && ws_bytes >= p.ws_bytes), "%s: workspace of %zu bytes needed", fn,
               p.ws_bytes);
    return IG_OK;
}

int ig_sparse_decode_attn(const void* q, const void* K, const void* V, int ld_rows, const int32_t* idx,
                          const int32_t* count, int B, int H, int d, int max_out, int dtype, float scale, float* out,
                          float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
    const AttnCall c{q, K, V, ld_rows, idx, count, B, H, d, max_out, dtype, scale, out, lse, ws};
    if (const int e = check_attn("ig_sparse_decode_attn", c, ws_bytes)) return e;
    return hip_status(launch_decode_layer(&c, nullptr, stream), "ig_sparse_decode_attn");
}

int ig_partial_weight_index_dev(const void* Wq_s, int D, int H, int d, int r, const void* K_s, int B, int n_cap,
                                int n, int dtype, int32_t* chan, void* Wq_part, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
    IG_REQUIRE_DTYPE("ig_partial_weight_index_dev", dtype);
    IG_REQUIRE(Wq_s && K_s && chan && Wq_part, "ig_partial_weight_index_dev: NULL required pointer");
    IG_REQUIRE(D >= 1 && H >= 1 && B >= 1 && r >= 1 && r <= d && n >= 1 && n <= n_cap,
               "ig_partial_weight_index_dev: bad sizes (D=%d H=%d d=%d r=%d B=%d n=%d n_cap=%d)", D, H, d, r, B, n,
               n_cap);
    IG_REQUIRE(head_dim_ok(d, dtype), "ig_partial_weight_index_dev: unsupported head dim %d", d);
    const size_t need = plan_setup(B, H, d, D, n).ws_bytes;
    IG_REQUIRE(ws && ws_bytes >= need && aligned16(ws),
               "ig_partial_weight_index_dev: workspace of %zu bytes needed (16-byte aligned)", need);
    return hip_status(launch_setup(Wq_s, D, H, d, r, K_s, B, n_cap, n, dtype, chan, Wq_part, ws, stream),
                      "ig_partial_weight_index_dev");
}

int ig_decode_layer(int B, int H, int d, int dtype, const ig_attn_call* attn, const ig_spec_call* spec,
                    hipStream_t stream) {
    IG_REQUIRE(attn || spec, "ig_decode_layer: nothing to do (attn and spec both NULL)");
    AttnCall ac{};
    SpecCall sc{};
    if (attn) {
        ac = AttnCall{attn->q, attn->K, attn->V, attn->ld_rows, attn->idx, attn->count, B, H, d, attn->max_out, dtype,
                      attn->scale, attn->out, attn->lse, attn->ws};
        if (const int e = check_attn("ig_decode_layer (attn)", ac, attn->ws_bytes)) return e;
    }
    if (spec) {
        sc = SpecCall{spec->x, spec->Wq_part, spec->bq_part, spec->Kp, B, spec->D, H, spec->r, spec->n, spec->n_cap,
                      dtype, spec->scale, spec->mode, spec->alpha, spec->k, spec->max_sel, spec->idx, spec->count,
                      spec->max_out, spec->counters, spec->cmax, spec->victim, spec->q_part, spec->scores, spec->ld,
                      spec->ws};
        if (const int e = check_spec("ig_decode_layer (spec)", sc, spec->ws_bytes)) return e;
    }
    if (attn && spec) {
        // the halves run concurrently: what the speculation writes must not be what the attention reads
        IG_REQUIRE(static_cast<const void*>(sc.idx) != static_cast<const void*>(ac.idx) &&
                       static_cast<const void*>(sc.count) != static_cast<const void*>(ac.count),
                   "ig_decode_layer: the speculation's idx/count must not be the attention's");
        IG_REQUIRE(ac.ws == nullptr || ac.ws != sc.ws, "ig_decode_layer: the two halves need distinct workspaces");
    }
    return hip_status(launch_decode_layer(attn ? &ac : nullptr, spec ? &sc : nullptr, stream), "ig_decode_layer");
}

int ig_pool_touch(uint32_t* counters, const int32_t* idx, const int32_t* count, int B, int H, int n, int n_cap,
                  int max_out, uint32_t cmax, int32_t* victim, void* ws, size_t ws_bytes, hipStream_t stream) {
    IG_REQUIRE(counters && idx && count, "ig_pool_touch: NULL required pointer");
    IG_REQUIRE(B >= 1 && H >= 1 && n >= 1 && n <= n_cap && max_out >= 1,
               "ig_pool_touch: bad sizes (B=%d H=%d n=%d n_cap=%d max_out=%d)", B, H, n, n_cap, max_out);
    IG_REQUIRE(cmax >= 2, "ig_pool_touch: cmax must be >= 2");
    IG_REQUIRE(H <= 1024, "ig_pool_touch: at most 1024 heads");
    if (!touch_single_kernel(H, max_out))
        IG_REQUIRE(ws && ws_bytes >= touch_ws_bytes(B) && aligned16(ws),
                   "ig_pool_touch: workspace of %zu bytes needed (16-byte aligned)", touch_ws_bytes(B));
    return hip_status(launch_touch(counters, idx, count, B, H, n, n_cap, max_out, cmax, victim, ws, stream),
                      "ig_pool_touch");
}

int ig_build_partial_cache(const void* K, const int32_t* chan, void* Kp, int B, int H, int d, int r, int n_cap,
                           int row0, int row1, int dtype, hipStream_t stream) {
    IG_REQUIRE_DTYPE("ig_build_partial_cache", dtype);
    IG_REQUIRE(K && chan && Kp, "ig_build_partial_cache: NULL required pointer");
    IG_REQUIRE(B >= 1 && H >= 1 && d >= 1 && r >= 1 && r <= d && 0 <= row0 && row0 <= row1 && row1 <= n_cap,
               "ig_build_partial_cache: bad sizes");
    if (row0 == row1) return ok();
    return hip_status(launch_build_partial(K, chan, Kp, B, H, d, r, n_cap, row0, row1, dtype, stream),
                      "ig_build_partial_cache");
}

int ig_append_kv(void* K, void* V, void* Kp, uint32_t* counters, const int32_t* chan, const void* k_new,
                 const void* v_new, const int32_t* victim, int B, int H, int d, int r, int n_cap, int n, int dtype,
                 int32_t* slot_out, hipStream_t stream) {
    IG_REQUIRE_DTYPE("ig_append_kv", dtype);
    IG_REQUIRE(Kp && chan && k_new && v_new && (K != nullptr) == (V != nullptr), "ig_append_kv: NULL required pointer");
    IG_REQUIRE(B >= 1 && H >= 1 && d >= 1 && r >= 1 && r <= d && 0 <= n && n <= n_cap && n_cap >= 1,
               "ig_append_kv: bad sizes");
    IG_REQUIRE(n < n_cap || victim, "ig_append_kv: the pool is full (n == n_cap): victim is required");
    return hip_status(launch_append(K, V, Kp, counters, chan, k_new, v_new, victim, B, H, d, r, n_cap, n, dtype,
                                    slot_out, stream),
                      "ig_append_kv");
}

size_t ig_int4_record_bytes(int d) { return d >= 32 && d % 32 == 0 ? int4_record_bytes(d) : 0; }

int ig_quantize_kv(const void* K, const void* V, int B, int H, int d, int ld_rows, int dtype, int row0, int nrows,
                   const int32_t* slot, void* KVq, int q_rows, hipStream_t stream) {
    IG_REQUIRE_DTYPE("ig_quantize_kv", dtype);
    IG_REQUIRE(K && V && KVq, "ig_quantize_kv: NULL required pointer");
    IG_REQUIRE(B >= 1 && H >= 1 && d >= 32 && d % 32 == 0 && d <= 4096, "ig_quantize_kv: d must be a multiple of 32 "
               "(got %d)", d);
    IG_REQUIRE(0 <= row0 && nrows >= 0 && row0 + nrows <= ld_rows && q_rows >= 1,
               "ig_quantize_kv: bad rows (row0=%d nrows=%d ld_rows=%d q_rows=%d)", row0, nrows, ld_rows, q_rows);
    IG_REQUIRE(slot || row0 + nrows <= q_rows, "ig_quantize_kv: rows beyond the record array");
    IG_REQUIRE(aligned16(K) && aligned16(V) && aligned16(KVq), "ig_quantize_kv: K, V and KVq must be 16-byte aligned");
    return hip_status(launch_quantize(K, V, B, H, d, ld_rows, dtype, row0, nrows, slot, KVq, q_rows, stream),
                      "ig_quantize_kv");
}

int ig_gather_kv_int4(const void* KVq, const int32_t* idx, const int32_t* count, int B, int H, int d, int q_rows,
                      int max_out, int dtype_out, void* Kc, void* Vc, hipStream_t stream) {
    IG_REQUIRE_DTYPE("ig_gather_kv_int4", dtype_out);
    IG_REQUIRE(KVq && idx && count && Kc && Vc, "ig_gather_kv_int4: NULL required pointer");
    IG_REQUIRE(B >= 1 && H >= 1 && q_rows >= 1 && max_out >= 1, "ig_gather_kv_int4: bad sizes");
    IG_REQUIRE(d >= 32 && d % 32 == 0 && d <= 4096, "ig_gather_kv_int4: d must be a multiple of 32 (got %d)", d);
    IG_REQUIRE(aligned16(KVq) && aligned16(Kc) && aligned16(Vc), "ig_gather_kv_int4: KVq, Kc, Vc must be 16-byte "
               "aligned");
    return hip_status(launch_gather_q4(KVq, idx, count, B, H, d, q_rows, max_out, dtype_out, Kc, Vc, stream),
                      "ig_gather_kv_int4");
}

}  // extern "C"

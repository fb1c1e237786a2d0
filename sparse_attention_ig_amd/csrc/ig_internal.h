// Internal declarations shared by the C-ABI layer, the host setup and the
// kernel launchers.  Not part of the public interface (include/ig.h).
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/ig.h"

namespace ig {

// Record an error message for ig_last_error() (thread-local) and return code.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int ok();

// host setup (ig_setup.cpp)
int skew_weights(const ig_skew_args* a);
int skew_apply(const double* A, int H, int d, const double* M, int64_t rows, double* out, int nthreads);
int store(const double* vals, int64_t count, int dtype, void* out);
int partial_weight_index(const void* Wq_s, int D, int H, int d, int r, const void* K_s, int B,
                         int n_cap, int n, int dtype, int32_t* chan, void* Wq_part, int nthreads);

// Launch plans: every workspace size and grid is derived from these, so the
// size query and the launch always agree.
struct RehearsePlan {
    int tiles;       // 64-column tiles of H*r
    int splits;      // split of the D reduction
    int rows_per_split;
    int bblocks;     // batch blocks
    int bb;          // batch rows per block (1, 2, 4, 8 or 16)
    int chunk;       // Kp rows per score workgroup
    int chunks;
    size_t ws_bytes; // split partials [splits][B][H*r] float
};
RehearsePlan plan_rehearse(int B, int H, int D, int r, int n, int dtype);

struct AttnPlan {
    int rows_per_split;
    int nsplit;
    size_t ws_bytes; // [B*H][nsplit][2 + d] float when nsplit > 1
};
AttnPlan plan_attn(int B, int H, int d, int max_out);

size_t select_ws_bytes(int B, int H, int n, int max_out);
bool select_needs_ws(int B, int H, int n, int max_out, int mode);  // head average, or sliced long rows

constexpr int kSpecMaxRows = 32768;   // rows (or candidates) one speculation workgroup holds in LDS
constexpr int kSpecMaxSlices = 16;    // slices per row of the fused speculation
constexpr int64_t kBitsTouchMin = 262144;  // selected slots per call from which sliced rows use bitmaps
constexpr int kSliceSlackMin = 2048;       // max_out from which slices get spare candidate slots
// Slices of rows too long for one workgroup's LDS, or too few to fill the chip: `slices` workgroups
// per row of `slice_rows` rows each, handing on up to `cap` candidates each to a merge workgroup per
// row (the fused speculation and ig_select's long rows).  ok is false when a row would need more than
// kSpecMaxSlices slices.
struct SlicePlan {
    int slices, slice_rows, cap;
    bool ok;
};
SlicePlan plan_slices(int64_t rows, int n, int max_out, bool topk = false);
constexpr int kTopkSliceRows = 8192;  // rows per slice of a sliced top-k row

struct SpecPlan {
    int slices, slice_rows, cand_cap;
    int proj_blocks, splits, proj_wgs;  // projection workgroups: column blocks x splits of the D inputs
    bool bits;                        // the merge leaves bitmaps and a counter kernel applies them
    bool tight;                       // top-k slices with tight candidates (the merge checks, or recomputes)
    bool headavg;                     // head average: whole rows hand on candidates, the merge averages
    bool ok;                          // false: rows too long for the candidates to fit one merge
    size_t off_status, off_arrive, off_part, off_cnt, off_lo, off_q, off_key, off_idx, off_bits, off_hcount,
        ws_bytes;
};
SpecPlan plan_speculate(int B, int H, int D, int r, int n, int max_out, int dtype, int mode);
size_t speculate_ws_bytes(int B, int H, int D, int r, int n, int max_out, int dtype);
size_t speculate_lds_bytes(int n);
void set_handover_test_mode(uint32_t spin_limit, int withhold);
// ig_speculate_noalloc: the speculation workspace in a static device array of this size per GPU
constexpr size_t kNoAllocScratchBytes = static_cast<size_t>(64) << 20;
unsigned long long spec_shape_key(int B, int H, int D, int r);

// kernel launchers (return hipError_t as int)
int launch_rehearse(const void* x, const void* Wq_part, const float* bq_part, const void* Kp,
                    int B, int D, int H, int r, int n, int n_cap, int dtype, float scale,
                    float* q_part, float* scores, int ld, void* ws, hipStream_t s);
int launch_proj(const void* x, const void* W, int B, int D, int N, int dtype, const RehearsePlan& p, float* part,
                hipStream_t s);
int launch_score(const float* part, const float* bias, const void* Kp, int B, int H, int r, int n, int n_cap,
                 int dtype, float scale, float* q_part, float* scores, int ld, const RehearsePlan& p, hipStream_t s);

int launch_select(const float* scores, int B, int H, int n, int ld, int mode, float alpha, int k,
                  int max_sel, int32_t* idx, int32_t* count, int max_out, void* ws, hipStream_t s);
int launch_attn(const void* q, const void* K, const void* V, int ld_rows, const int32_t* idx,
                const int32_t* count, int B, int H, int d, int max_out, int dtype, float scale,
                float* out, float* lse, void* ws, hipStream_t s);
bool host_resident(const void* p);  // host memory (pinned, device-mapped), or a pointer the runtime does not know
int launch_gather(const void* K, const void* V, const int32_t* idx, const int32_t* count, int B, int H,
                  int d, int n_cap, int max_out, int dtype, void* Kc, void* Vc, hipStream_t s);
int launch_touch(uint32_t* counters, const int32_t* idx, const int32_t* count, int B, int H, int n,
                 int n_cap, int max_out, uint32_t cmax, int32_t* victim, void* ws, hipStream_t s);
size_t touch_ws_bytes(int B);
int launch_touch_bits(uint32_t* counters, const uint32_t* bits, int B, int H, int n, int n_cap, uint32_t cmax,
                      uint32_t* flags, int32_t* victim, hipStream_t s);
bool touch_single_kernel(int H, int max_out);
int launch_speculate(const void* x, const void* Wq_part, const float* bq_part, const void* Kp, int B, int D, int H,
                     int r, int n, int n_cap, int dtype, float scale, int mode, float alpha, int k, int max_sel,
                     int32_t* idx, int32_t* count, int max_out, uint32_t* counters, uint32_t cmax, int32_t* victim,
                     float* q_part, float* scores, int ld, void* ws, hipStream_t s);
int launch_zero(void* ws, size_t bytes, hipStream_t s);
int launch_attn_combine(const float* part, int nsplit, int d, int BH, float* out, float* lse, hipStream_t s);

// device-side partial weight index: float64 column-sum partials of |W~_Q| ([wslices][H*d]) and |K~|
// ([B*kchunks][H][d]) in the workspace
struct SetupPlan {
    int wslices, kchunks;
    size_t off_k, ws_bytes;
};
SetupPlan plan_setup(int B, int H, int d, int D, int n);
int launch_setup(const void* Wq_s, int D, int H, int d, int r, const void* K_s, int B, int n_cap, int n, int dtype,
                 int32_t* chan, void* Wq_part, void* ws, hipStream_t s);

// host-side descriptors of the two halves of a decode layer (the arguments of launch_attn and
// launch_speculate)
struct AttnCall {
    const void* q;
    const void* K;
    const void* V;
    int ld_rows;
    const int32_t* idx;
    const int32_t* count;
    int B, H, d, max_out, dtype;
    float scale;
    float* out;
    float* lse;
    void* ws;
};
struct SpecCall {
    const void* x;
    const void* Wq_part;
    const float* bq_part;
    const void* Kp;
    int B, D, H, r, n, n_cap, dtype;
    float scale;
    int mode;
    float alpha;
    int k, max_sel;
    int32_t* idx;
    int32_t* count;
    int max_out;
    uint32_t* counters;
    uint32_t cmax;
    int32_t* victim;
    float* q_part;
    float* scores;
    int ld;
    void* ws;
};
constexpr int kDecodeMaxRows = 16384;  // rows per (b, h) for the fused decode launch (LDS with two roles)
bool decode_fusable(const AttnCall& a, const SpecCall& s);
int launch_decode_layer(const AttnCall* a, const SpecCall* s, hipStream_t st);
int launch_speculate_noalloc(const SpecCall& c, hipStream_t s);
size_t int4_record_bytes(int d);
int launch_quantize(const void* K, const void* V, int B, int H, int d, int ld_rows, int dtype, int row0, int nrows,
                    const int32_t* slot, void* KVq, int q_rows, hipStream_t s);
int launch_gather_q4(const void* KVq, const int32_t* idx, const int32_t* count, int B, int H, int d, int q_rows,
                     int max_out, int dtype_out, void* Kc, void* Vc, hipStream_t s);
int launch_build_partial(const void* K, const int32_t* chan, void* Kp, int B, int H, int d, int r,
                         int n_cap, int row0, int row1, int dtype, hipStream_t s);
int launch_append(void* K, void* V, void* Kp, uint32_t* counters, const int32_t* chan,
                  const void* k_new, const void* v_new, const int32_t* victim, int B, int H, int d,
                  int r, int n_cap, int n, int dtype, int32_t* slot_out, hipStream_t s);

}  // namespace ig

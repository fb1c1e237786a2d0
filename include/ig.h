/*
 * ig.h -- C ABI of the MI355X (gfx950) InfiniGen decode hot path.
 *
 * Method: "InfiniGen: Efficient Generative Inference of Large Language Models
 * with Dynamic KV Cache Management" (arXiv 2406.19707), as summarised on the
 * paper-graph-ui page for that paper, section 3.4 ("Detailed, Sentence-Based
 * Technical Breakdown") and section 2 ("Context and Motivation").
 *
 * Conventions for every call
 *  - Return value: IG_OK, or an error code.  IG_EINVAL: an argument is
 *    invalid; detected on the host before anything is launched, nothing is
 *    written.  IG_EHIP: the HIP runtime reported an error.  IG_EUNSUPPORTED:
 *    a valid but unimplemented shape.  ig_last_error() returns the message of
 *    the last failing call on the calling thread.  No C++ exception crosses
 *    this boundary.
 *  - Ownership: the caller owns every buffer.  The library keeps no state and
 *    allocates no device memory; scratch comes from the caller through
 *    `ws` / `ws_bytes`, sized by ig_workspace_size().  Workspace contents on
 *    entry are ignored.
 *  - Device calls are asynchronous on `stream`; they never synchronise and
 *    never read device buffers on the host.  Device pointers must be 16-byte
 *    aligned.  Host calls (ig_skew_*, ig_store, ig_partial_weight_index) are
 *    synchronous and touch no GPU.
 *  - Layouts are row-major.  B = batch, H = heads, d = head dim, D = hidden
 *    (the attention input width), r = partial channels per head, n = valid
 *    cached rows (N + i), n_cap = allocated rows per (b, h).  Element dtype is
 *    IG_F32 (float) or IG_BF16 (bfloat16 bits in uint16_t); accumulation and
 *    every produced score, logit and output is float32.
 *  - Constraints checked: all sizes >= 1; r <= d; r / (16 / sizeof(element))
 *    a power of two <= 32 (r in {8, 16, 32, 64, 128, 256} for bf16,
 *    {8, 16, 32, 64, 128} for f32); d / (16 / sizeof(element)) a power of two
 *    between 4 and 32 (d in {32, 64, 128, 256} for bf16, {16, 32, 64, 128} for
 *    f32); D a multiple of 16 / sizeof(element) for the speculation calls;
 *    n <= n_cap.
 */
#ifndef IG_H_
#define IG_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { IG_OK = 0, IG_EINVAL = 1, IG_EHIP = 2, IG_EUNSUPPORTED = 3 };
enum { IG_F32 = 0, IG_BF16 = 1 };
enum { IG_SEL_THRESHOLD = 0, IG_SEL_TOPK = 1, IG_SEL_HEADAVG = 2 };
enum { IG_OP_REHEARSE = 0, IG_OP_SELECT = 1, IG_OP_ATTN = 2, IG_OP_SPECULATE = 3, IG_OP_TOUCH = 4,
       IG_OP_SETUP = 5 };
/* Sticky status bits of a speculation workspace (ig_workspace_status). */
enum { IG_WS_TIMEOUT = 1,   /* a row's partial query did not arrive within the poll limit */
       IG_WS_SHAPE = 2 };   /* a call's (B, H, D, r) differs from the one the workspace was claimed for */

/* Message of the last failing call on this thread ("" if none). */
const char* ig_last_error(void);
/* ABI version: bumped on any signature or layout change (2: ig_pool_touch takes a
 * workspace; 3: Wq_part is stored one row per partial column, [H*r][D];
 * 4: ig_decode_layer; 5: ig_partial_weight_index_dev; 6: the speculation
 * workspace starts with its arrival words; 7: the INT4 pool calls; 8: the
 * speculation's partial query comes from projection workgroups of the same
 * launch, whose split partial sums follow the sequences' arrival words in
 * the workspace; 9: ig_select takes a workspace for rows longer than 32768 keys;
 * 10: the speculation workspace starts with a status word and a shape stamp,
 * ig_workspace_status, ig_set_handover_test_mode; 11: the bitmap counter
 * kernels' flags follow the arrival words, at a place that does not depend on
 * n). */
int ig_version(void);

/* ------------------------------------------------------------------ host, offline setup */

/* Arguments of ig_skew_weights.  All host memory, float64. */
typedef struct {
    int D, H, d;                /* hidden, heads, head dim (weights are [D][H*d]) */
    int m;                      /* rows of each head's skew source, m >= d */
    const double* skew_src;     /* [H][m][d]: the sample query of each head (or any matrix whose
                                   right singular vectors define that head's rotation) */
    const double* Wq;           /* [D][H*d] or NULL */
    const double* Wk;           /* [D][H*d] or NULL */
    const double* bq;           /* [H*d] or NULL */
    const double* bk;           /* [H*d] or NULL */
    double* A;                  /* out [H][d][d]; column j = j-th right singular vector */
    double* sigma;              /* out [H][d] singular values, descending; may be NULL */
    double* Wq_s;               /* out [D][H*d] = Wq A (per head block); NULL iff Wq is NULL */
    double* Wk_s;               /* out, NULL iff Wk is NULL */
    double* bq_s;               /* out [H*d], NULL iff bq is NULL */
    double* bk_s;               /* out, NULL iff bk is NULL */
    int nthreads;               /* host threads (<= 0: all hardware threads) */
} ig_skew_args;

/*
 * Offline skewing (section 3.4, "Skewed Partial Weights"): for each head,
 * A_h = V_h from the SVD skew_src_h = U S V^T (one-sided Jacobi in float64),
 * columns ordered by descending singular value, each column signed so that its
 * largest-magnitude entry is positive (lowest row index on equal magnitudes).
 * Then W~ = W A and b~ = b A per head block, so that Q~ K~^T = Q K^T.
 * The rotation is unique up to those signs only when the singular values are
 * distinct and m >= d.  IG_EINVAL on NULL required pointers, m < d, d < 1.
 */
int ig_skew_weights(const ig_skew_args* args);

/*
 * Rotate every head block of a row-major [rows][H*d] float64 matrix by that
 * head's A_h: out[:, h*d:(h+1)*d] = M[:, h*d:(h+1)*d] A_h (queries or keys
 * given in the unrotated basis; same section).  out must not alias M.
 */
int ig_skew_apply(const double* A, int H, int d, const double* M, int64_t rows,
                  double* out, int nthreads);

/*
 * Store float64 setup results in the element dtype: round to float32
 * (nearest-even); for IG_BF16 round that float32 to bfloat16 (nearest-even).
 */
int ig_store(const double* vals, int64_t count, int dtype, void* out);

/*
 * Partial weight index generation (section 3.4, "Prefill Stage: Partial
 * Weight Index Generation", steps 2-3).  Per head h, channel score
 *   score[c] = sum_i |Wq_s[i][h*d+c]| + sum_{b, j<n} |K_s[b][h][j][c]|
 * (float64 sums of the stored values); chan[h] = the r highest-scoring
 * channels (ties: lower channel), ascending.  Wq_part[h*r+k][i] =
 * Wq_s[i][h*d + chan[h][k]] (a copy of the stored elements, one row of D
 * inputs per partial column: the transpose of the column selection).
 * Host pointers: Wq_s [D][H*d] dtype; K_s [B][H][n_cap][d] dtype (rows < n
 * used); chan [H][r] int32 out; Wq_part [H*r][D] dtype out.
 */
int ig_partial_weight_index(const void* Wq_s, int D, int H, int d, int r,
                            const void* K_s, int B, int n_cap, int n, int dtype,
                            int32_t* chan, void* Wq_part, int nthreads);

/* ------------------------------------------------------------------ device calls */

/*
 * ig_partial_weight_index on the GPU (section 3.4, "Prefill Stage: Partial
 * Weight Index Generation", steps 2-3), so that the prefill setup and the
 * cache growth (ig_build_partial_cache, ig_append_kv) never leave the device.
 * Same definition and outputs: per head, score[c] = sum_i |Wq_s[i][h*d+c]| +
 * sum_{b, j<n} |K_s[b][h][j][c]| in float64 (partial sums over fixed slices,
 * added in a fixed order, so the result is deterministic; it can differ from
 * the host routine only where two channel scores agree to rounding), the r
 * largest (ties: lower channel) in ascending order to chan [H][r], and
 * Wq_part [H*r][D] = the chosen columns, one row per channel.  Device
 * pointers; workspace IG_OP_SETUP bytes (B, H, D, d, n used).
 */
int ig_partial_weight_index_dev(const void* Wq_s, int D, int H, int d, int r, const void* K_s, int B, int n_cap,
                                int n, int dtype, int32_t* chan, void* Wq_part, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * Bytes of scratch a call needs (0 if none).  op = IG_OP_REHEARSE: B, H, D,
 * r used.  IG_OP_SELECT: B, H, n, max_out used.  IG_OP_ATTN: B, H, d,
 * max_out used.  IG_OP_SPECULATE: B, H, D, r, n, max_out used.  IG_OP_TOUCH:
 * B, H, max_out used.  Unused arguments are ignored.
 */
size_t ig_workspace_size(int op, int B, int H, int D, int d, int r, int n, int max_out);

/*
 * Zero-fill a workspace on `stream` (a fill kernel, so it may be captured in a
 * graph).  Required once after allocating the workspace of ig_speculate, whose
 * calls then leave it zero-filled (status and stamp aside); required again
 * before a speculation call of another (B, H, D, r), and after a failure (a
 * nonzero status).  Harmless for the other calls' workspaces.
 */
int ig_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Status word of a speculation workspace (ig_speculate, the speculation half
 * of ig_decode_layer): 0, or IG_WS_* bits set by a call that ran on it.  The
 * bits are sticky: a workspace with a nonzero status gives count = -1 for
 * every row of later calls until ig_workspace_init clears it.  *recomputed
 * (when not NULL) receives the number of sliced top-k rows, summed over the
 * calls since ig_workspace_init (modulo 2^32), whose merge found the slices'
 * tight candidates too few and recomputed the row's scores (exact, slower;
 * see ig_speculate).  Waits for the work enqueued on `stream`
 * (hipStreamSynchronize) and copies the words; not for use under graph
 * capture.  IG_EINVAL when ws or status is NULL or ws_bytes is below 256.
 */
int ig_workspace_status(const void* ws, size_t ws_bytes, uint32_t* status, uint32_t* recomputed,
                        hipStream_t stream);

/*
 * Failure-path testing of the speculation's in-launch hand-over, process-wide,
 * read when a call is launched: spin_limit = polls of a row workgroup before it
 * stops waiting for its partial query (0: the default, 2^22 polls of a few
 * hundred ns each); withhold != 0 makes the projection workgroups store no
 * partial sums, so that every row reaches its poll limit and fails as
 * ig_speculate describes.  ig_set_handover_test_mode(0, 0) restores normal
 * operation.  Returns IG_OK.
 */
int ig_set_handover_test_mode(uint32_t spin_limit, int withhold);

/*
 * Speculation for the next layer (section 3.4, "Decoding Stage", steps 1-2):
 *   q_part[b][h][c]  = sum_i x[b][i] Wq_part[h*r+c][i] (+ bq_part[h*r+c])
 *   scores[b][h][j]  = scale * sum_c q_part[b][h][c] Kp[b][h][j][c],  j < n
 * x [B][D] dtype (this layer's attention input); Wq_part [H*r][D] dtype (the
 * next layer's partial query weight, one row per partial column, as
 * ig_partial_weight_index writes it); bq_part [H*r] float or NULL;
 * Kp [B][H][n_cap][r] dtype (the next layer's partial key cache);
 * q_part [B][H][r] float out; scores [B][H][ld] float out (ld >= n; columns
 * >= n untouched).  scale: the softmax scale of the attention (e.g. 1/sqrt(d)).
 */
int ig_rehearse(const void* x, const void* Wq_part, const float* bq_part, const void* Kp,
                int B, int D, int H, int r, int n, int n_cap, int dtype, float scale,
                float* q_part, float* scores, int ld,
                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Fused speculation for one layer in one launch: the partial query, speculated
 * scores, selection and counter update of ig_rehearse + ig_select +
 * ig_pool_touch (section 3.4, "Decoding Stage" steps 1-3 and 5, and the pool
 * paragraph), with the scores kept on chip.  Same arguments and results as
 * those calls, in all three modes.  A row's scores live in LDS: when there are
 * too few rows to fill the GPU, or n > 32768, each row is cut into up to 16
 * slices that select locally, and a merge launch selects among their
 * candidates; IG_EUNSUPPORTED when n > 16 x 32768, or in IG_SEL_HEADAVG when
 * rows would have to be sliced (each whole row hands on its top candidates
 * and its threshold count, and the merge launch gives every head of a
 * sequence the averaged count).  When a sliced call selects many slots, the
 * counters are updated from per-row bitmaps by two small kernels after the
 * merge.
 * q_part [B][H][r] and scores [B][H][ld] are written only when not NULL.
 * counters (not NULL) are updated as by ig_pool_touch, victim [B] (not NULL)
 * receives the victim.  One launch: projection workgroups (each one block of
 * partial columns over one split of 512 inputs of D, for every batch row) and
 * one workgroup per (b, h) (or per slice), which adds its head's split
 * partial sums in split order, then scores, selects and updates the counters;
 * with slices, a merge launch follows.  The workspace (IG_OP_SPECULATE bytes,
 * required) starts with a 256-byte region holding the status word (uint32 at
 * offset 0, see ig_workspace_status) and the shape stamp (uint64 at offset 8),
 * then two uint32 words per sequence at offset 256 (the rows' arrivals [B],
 * then the bitmap counter kernels' saturation flags [B]) and the projection's
 * split partial sums, then the slices' candidates (when there are slices)
 * and the counter kernels' bitmaps; it must have been zero-filled once with
 * ig_workspace_init, and every call returns the per-sequence words and the
 * partial-sum slots to zero.  The first call after the zero-fill stamps
 * the workspace with its (B, H, D, r) (the places of those regions depend on
 * them; n, max_out and the mode may change from call to call); a call of
 * another (B, H, D, r) sets IG_WS_SHAPE instead of running: run
 * ig_workspace_init before it.  Calls sharing a workspace must not overlap.
 * Failures (not reported by the return value, which covers the launch only):
 * a row workgroup that finds a nonzero status or a foreign stamp, or whose
 * partial query is still missing after the poll limit (IG_WS_TIMEOUT; it then
 * leaves every partial-sum slot as it is, since a late producer may still
 * store into one), writes count = -1 for its row (idx, q_part and scores of
 * that row unspecified) and touches no counter of it; the rows that completed
 * are valid.  H <= 65535, B <= 65535, D < 2^22.
 */
int ig_speculate(const void* x, const void* Wq_part, const float* bq_part, const void* Kp,
                 int B, int D, int H, int r, int n, int n_cap, int dtype, float scale,
                 int mode, float alpha, int k, int max_sel,
                 int32_t* idx, int32_t* count, int max_out,
                 uint32_t* counters, uint32_t cmax, int32_t* victim,
                 float* q_part, float* scores, int ld,
                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ig_speculate without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments (minus ws, ws_bytes), results and
 * failure rule (count = -1) as ig_speculate; this call allocates nothing.  Its
 * workspace is a static device array of 64 MiB (IG_NOALLOC_SCRATCH_BYTES) that
 * each GPU the library runs on holds until the process ends; IG_EINVAL when
 * ig_workspace_size(IG_OP_SPECULATE, ...) of the call exceeds it (B4 H32
 * D4096 r32 n131072 top-5243 needs 33 MiB).  Every call first clears the
 * regions that must start at zero (a fill kernel on `stream`, capturable) and
 * stamps them with its shape, so shapes may change freely from call to call
 * and a failed call leaves nothing behind.  All calls on one GPU share that
 * GPU's array: calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race and give unspecified results.
 */
#define IG_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ig_speculate_noalloc(const void* x, const void* Wq_part, const float* bq_part, const void* Kp,
                         int B, int D, int H, int r, int n, int n_cap, int dtype, float scale,
                         int mode, float alpha, int k, int max_sel,
                         int32_t* idx, int32_t* count, int max_out,
                         uint32_t* counters, uint32_t cmax, int32_t* victim,
                         float* q_part, float* scores, int ld, hipStream_t stream);

/*
 * One decode layer (section 3.2, "Big-Picture Architecture": the KV Selection
 * Controller speculates layer i's tokens from layer i-1's attention input
 * while layer i-1 computes; section 3.4, "Decoding Stage"): the attention of
 * layer l over the rows selected for it, and the speculation for layer l+1.
 * `attn` holds the arguments of ig_sparse_decode_attn for layer l, `spec` those
 * of ig_speculate for layer l+1 (B, H, dtype shared; d is the attention's head
 * dim); either may be NULL (then this is that one call).  With both: one
 * launch in which the speculation's projection and (b, h) workgroups and the
 * attention's run side by side (no ordering between the two halves, so
 * spec->idx, count, counters,
 * victim, q_part, scores must not
 * alias anything attn reads), then the split combine of the attention if it
 * splits.  Results: those of the two calls (the attention's float sums may
 * associate differently).  Falls back to the two calls in sequence for shapes
 * outside the fused set (spec r / (16 / element size) in {2, 4, 8}, attn d /
 * (16 / element size) in {8, 16, 32}, spec n <= 16384 without slices).
 */
typedef struct {
    const void* q;
    const void* K;
    const void* V;
    int ld_rows;
    const int32_t* idx;
    const int32_t* count;
    int max_out;
    float scale;
    float* out;
    float* lse;
    void* ws;
    size_t ws_bytes;
} ig_attn_call;

typedef struct {
    const void* x;
    const void* Wq_part;
    const float* bq_part;
    const void* Kp;
    int D, r, n, n_cap;
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
    size_t ws_bytes;
} ig_spec_call;

int ig_decode_layer(int B, int H, int d, int dtype, const ig_attn_call* attn, const ig_spec_call* spec,
                    hipStream_t stream);

/*
 * Per-head token selection (section 3.4, "Decoding Stage", steps 3-5).
 *  IG_SEL_THRESHOLD: S = {j < n : s_j >= max_j s_j - alpha} (alpha >= 0,
 *    +inf allowed); if |S| exceeds max_sel (> 0) or max_out, S keeps its
 *    largest scores (the per-layer cap).
 *  IG_SEL_TOPK: S = the min(k, n, max_out) largest scores (k >= 1).
 *  IG_SEL_HEADAVG: every head of a sequence takes the same count, the mean
 *    over heads of its threshold counts rounded up (then limited by max_sel
 *    and max_out); each head keeps its largest scores.
 * Ties go to the lower index; the comparison is in float32.  Output:
 * idx [B][H][max_out] int32 ascending (entries >= count unspecified),
 * count [B][H] int32 in [1, max_out].  Scores must not be NaN.
 * One workgroup per (b, h) row with the row's keys in LDS up to n = 32768.
 * Longer threshold and top-k rows are cut into slices that select locally and
 * hand on candidates to a merge launch (up to 16 slices of 32768 rows; longer
 * rows, and the head-average mode, are streamed from HBM in every pass).  The
 * workspace (IG_OP_SELECT bytes) is required in the head-average mode and for
 * sliced rows (ws may be NULL otherwise); it needs no initialisation.
 */
int ig_select(const float* scores, int B, int H, int n, int ld, int mode,
              float alpha, int k, int max_sel,
              int32_t* idx, int32_t* count, int max_out,
              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Fetch the full key and value rows of the selected tokens into compact
 * buffers (section 3.4, "Decoding Stage", step 5):
 *   Kc[b][h][i][:] = K[b][h][idx[b][h][i]][:],  i < count[b][h]  (same for V)
 * K, V [B][H][n_cap][d] dtype, in device memory or in pinned host memory
 * mapped into the device address space (zero-copy reads over the host link);
 * Kc, Vc [B][H][max_out][d] device.  Rows >= count are untouched.  Index
 * values outside [0, n_cap) are clamped into it.
 */
int ig_gather_kv(const void* K, const void* V, const int32_t* idx, const int32_t* count,
                 int B, int H, int d, int n_cap, int max_out, int dtype,
                 void* Kc, void* Vc, hipStream_t stream);

/*
 * Attention over the selected rows only (section 3.2, Inference Controller;
 * section 2, softmax(QK^T)V):
 *   o[b][h] = sum_{i<c} p_i V[b][h][row_i],  p = softmax_i(scale q[b][h].K[b][h][row_i])
 *   lse[b][h] = log sum_i exp(scale q.K_row_i)     (natural log)
 * with c = min(count[b][h], max_out) and row_i = idx[b][h][i], or row_i = i
 * when idx is NULL (dense over the first count rows, or a compact buffer).
 * q [B][H][d] dtype; K, V [B][H][ld_rows][d] dtype; out [B][H][d] float;
 * lse [B][H] float or NULL.  c = 0 gives o = 0, lse = -inf.  Index values
 * outside [0, ld_rows) are clamped into it.
 */
int ig_sparse_decode_attn(const void* q, const void* K, const void* V, int ld_rows,
                          const int32_t* idx, const int32_t* count,
                          int B, int H, int d, int max_out, int dtype, float scale,
                          float* out, float* lse,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Counter-based pool policy (section 3.4, "KV Cache Pool Management Under
 * Memory Pressure"): every (head, selected slot) adds 1 to the slot's counter;
 * C <- min(C + inc, cmax); if any slot j < n of a sequence then holds cmax,
 * all its slots j < n are halved (floor).  victim[b] (if not NULL) = the
 * lowest index among the minima of C[b][0..n).  counters [B][n_cap] uint32,
 * updated in place; precondition C[b][j] < cmax for j < n.  Indices of one
 * head must be distinct; values outside [0, n) are ignored.  cmax >= 2,
 * H <= 1024.  When H * max_out <= 32768 one workgroup per sequence does the
 * whole update (workspace unused, may be NULL); otherwise three launches
 * (zero the per-sequence flags, increments over (b, h, chunk) workgroups,
 * per-sequence finish) with IG_OP_TOUCH workspace bytes.
 */
int ig_pool_touch(uint32_t* counters, const int32_t* idx, const int32_t* count,
                  int B, int H, int n, int n_cap, int max_out, uint32_t cmax,
                  int32_t* victim, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Build rows [row0, row1) of the partial key cache from the skewed key cache
 * (section 3.4, prefill step 3): Kp[b][h][j][c] = K[b][h][j][chan[h][c]].
 * K [B][H][n_cap][d], Kp [B][H][n_cap][r] dtype; chan [H][r] int32 device.
 */
int ig_build_partial_cache(const void* K, const int32_t* chan, void* Kp,
                           int B, int H, int d, int r, int n_cap, int row0, int row1,
                           int dtype, hipStream_t stream);

/*
 * Append one decoded token per sequence (section 3.4, "Partial Key Cache
 * Updates During Decoding" and the pool paragraph): slot = n if n < n_cap,
 * else victim[b] (victim required then); K[b][h][slot] = k_new[b][h],
 * V[b][h][slot] = v_new[b][h], Kp[b][h][slot][c] = k_new[b][h][chan[h][c]],
 * counters[b][slot] = 0 (if counters not NULL); slot_out[b] = slot (if not
 * NULL).  k_new, v_new [B][H][d] dtype.  K and V may both be NULL (a pool kept
 * as INT4 records, see ig_quantize_kv): then only the partial key row, the
 * counter and slot_out are written.
 */
int ig_append_kv(void* K, void* V, void* Kp, uint32_t* counters, const int32_t* chan,
                 const void* k_new, const void* v_new, const int32_t* victim,
                 int B, int H, int d, int r, int n_cap, int n, int dtype,
                 int32_t* slot_out, hipStream_t stream);

/* ------------------------------------------------------------------ INT4 pool */

/*
 * A KV pool stored at 4 bits per element, of which only the speculated rows
 * are fetched: the combination the summary proposes under "Follow-Up
 * Research" (speculative prefetching of a quantised pool), with the 4-bit
 * group-wise asymmetric quantisation of its section 5 baselines.  The partial
 * key cache (Kp) stays at full precision in HBM, so the speculation is
 * unchanged.
 *
 * Record of one token's key and value rows of d elements each (d a multiple
 * of 32), of ig_int4_record_bytes(d) bytes (160 for d = 128): K codes in
 * bytes [0, d/2), V codes in [d/2, d) (element i in byte i/2 of its half, low
 * nibble for even i); then for each group g of 32 elements, the K groups
 * first, a float16 step s16 and a float16 minimum m16 (bytes d + 4g and
 * d + 4g + 2, little endian); zero padding to a multiple of 32 bytes.  A
 * fetched token costs three 64-byte reads over the host link (a bf16 K and V
 * row, eight).  Record arrays are [B][H][q_rows][record bytes].
 */
size_t ig_int4_record_bytes(int d);   /* 0 if d is not a positive multiple of 32 */

/*
 * Quantise rows [row0, row0 + nrows) of every (b, h) of K and V
 * [B][H][ld_rows][d] (dtype bf16 or f32, device memory) into the records of
 * KVq (device or host-mapped memory; writes over the host link are zero-copy).  Per group of
 * 32 values: mn, mx; s16 = half((mx - mn) / 15) and m16 = half(mn), nearest
 * even; code = clamp(rint((v - m16) / s16), 0, 15) in float32 (correctly
 * rounded division, halves to even), 0 when s16 is 0.  Values must lie in
 * float16's range.  Destination row = the source row, or, with slot [B] (not
 * NULL), slot[b] + (row - row0): the append of a new token, with K, V = the
 * new rows [B][H][1][d], row0 = 0, nrows = 1 and the slot_out of ig_append_kv
 * (called with K = V = NULL, which then writes only the partial key row and
 * the counter).  Destination rows are clamped into [0, q_rows).
 */
int ig_quantize_kv(const void* K, const void* V, int B, int H, int d, int ld_rows, int dtype, int row0, int nrows,
                   const int32_t* slot, void* KVq, int q_rows, hipStream_t stream);

/*
 * Step 5 on a quantised pool: for i < min(count[b][h], max_out) and
 * j = idx[b][h][i] (clamped into [0, q_rows)), Kc[b][h][i] and Vc[b][h][i]
 * = the dequantised rows, v = m16 + code * s16 in float32, stored as
 * dtype_out (bf16, nearest even, or f32).  KVq: the record array in device
 * or host-mapped memory (zero-copy reads over the host link); Kc, Vc
 * [B][H][max_out][d] device.
 */
int ig_gather_kv_int4(const void* KVq, const int32_t* idx, const int32_t* count,
                      int B, int H, int d, int q_rows, int max_out, int dtype_out,
                      void* Kc, void* Vc, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* IG_H_ */

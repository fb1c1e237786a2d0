"""Plain, slow CPU oracle of InfiniGen's decode-time hot path (fp64 NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constant tables); it reads the same
stored input bits and decodes them itself.

Source: "InfiniGen: Efficient Generative Inference of Large Language Models with
Dynamic KV Cache Management" (arXiv 2406.19707), as summarised on the
paper-graph-ui page for that paper ("the pages" below), section 3.4 "Detailed,
Sentence-Based Technical Breakdown" and section 2 "Context and Motivation".

Each function follows one step of that section, in the pages' order and
notation.  Arithmetic is float64 on the decoded inputs; selection decisions use
the float64 scores.  Readings of points the pages leave open are stated where
they are used (softmax scale, >= at the cut, tie order, cap rounding, counter
width and halving, victim ties).

Parity status: every function here is pinned by a ``-m "not gpu"`` test
(closed forms, brute force, hand-computed fixtures under ``tests/golden/``);
none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

F32, BF16 = "f32", "bf16"


# ---------------------------------------------------------------- storage
def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values of stored inputs: float32 arrays as is; bfloat16 bits widened to float32."""
    if dtype == F32:
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def store(vals: np.ndarray, dtype: str) -> np.ndarray:
    """Store float64 setup results: round to float32 (nearest-even); for bfloat16 round the
    float32 value again to the top 16 bits (nearest-even), as a float32-accumulating model would."""
    with np.errstate(over="ignore"):
        f = np.asarray(vals, dtype=np.float64).astype(np.float32)
    if dtype == F32:
        return f
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


# ---------------------------------------------------------------- offline skewing
def skew_rotation(src: np.ndarray) -> np.ndarray:
    """Per-head orthogonal skew matrix A_h = V_h, the right singular vectors of the sample
    query matrix Q_h = U_h S_h V_h^T, columns in descending singular-value order
    (section 3.4, "Skewed Partial Weights": A is set to V so that Q~ = Q V = U S).

    Singular vectors are fixed only up to sign; reading: each column is signed so that its
    largest-magnitude entry is positive (the lowest row index among equal magnitudes).
    src: [H][m][d] -> A: [H][d][d]
    """
    src = np.asarray(src, dtype=np.float64)
    H, _, d = src.shape
    A = np.zeros((H, d, d))
    for h in range(H):
        _, _, vt = np.linalg.svd(src[h], full_matrices=True)
        v = vt.T.copy()                      # column j = j-th right singular vector
        for j in range(d):
            col = v[:, j]
            piv = int(np.argmax(np.abs(col)))  # first index of the largest magnitude
            if col[piv] < 0:
                v[:, j] = -col
        A[h] = v
    return A


def skew_apply(A: np.ndarray, M: np.ndarray) -> np.ndarray:
    """Rotate every head's d-column block of M (..., H*d) by that head's A_h:
    M~[..., h*d:(h+1)*d] = M[..., h*d:(h+1)*d] A_h  (section 3.4, "Skewed Partial Weights":
    W~_Q = W_Q A, W~_K = W_K A; a query or key row given in the original basis rotates the same way)."""
    A = np.asarray(A, dtype=np.float64)
    H, d, _ = A.shape
    M = np.asarray(M, dtype=np.float64)
    out = np.empty_like(M)
    for h in range(H):
        out[..., h * d:(h + 1) * d] = M[..., h * d:(h + 1) * d] @ A[h]
    return out


def skew_weights(Wq, Wk, src, bq=None, bk=None):
    """Offline skewing of one layer: A from the sample query, W~_Q = W_Q A, W~_K = W_K A,
    biases rotated the same way (q = xW + b  =>  q~ = x W A + b A).
    Returns (A, Wq_s, Wk_s, bq_s, bk_s) in float64."""
    A = skew_rotation(src)
    Wq_s = skew_apply(A, Wq)
    Wk_s = None if Wk is None else skew_apply(A, Wk)
    bq_s = None if bq is None else skew_apply(A, bq)
    bk_s = None if bk is None else skew_apply(A, bk)
    return A, Wq_s, Wk_s, bq_s, bk_s


# ---------------------------------------------------------------- prefill: partial weight index generation
def partial_weight_index(Wq_s: np.ndarray, K_s: np.ndarray, H: int, d: int, r: int,
                         n: Optional[int] = None, dtype: Optional[str] = None) -> np.ndarray:
    """Channel pick of section 3.4, "Prefill Stage: Partial Weight Index Generation", step 2:
    take element-wise absolute values of the skewed query weight and of the skewed key cache,
    sum each over its rows, add the two column-sum vectors, keep the top r columns.

    Readings: r columns per head (the pages' "k" read per head); the element-wise sum of the
    two differently shaped matrices is read as the sum of their column-sum vectors; ties go to
    the lower channel index; indices are returned ascending.
    Wq_s: [D][H*d]; K_s: [B][H][rows][d] (first n rows used); values, or stored bits when dtype
    is given (decoded one head at a time) -> chan [H][r] int32.
    """
    dec = (lambda a: np.asarray(a, dtype=np.float64)) if dtype is None else (lambda a: decode(a, dtype))
    if n is None:
        n = K_s.shape[2]
    chan = np.zeros((H, r), dtype=np.int32)
    for h in range(H):
        score = np.abs(dec(Wq_s[:, h * d:(h + 1) * d])).sum(axis=0) \
            + np.abs(dec(K_s[:, h, :n, :])).sum(axis=(0, 1))
        order = sorted(range(d), key=lambda c: (-score[c], c))
        chan[h] = np.sort(np.asarray(order[:r], dtype=np.int32))
    return chan


def pack_partial_weight(Wq_s_bits: np.ndarray, chan: np.ndarray, d: int) -> np.ndarray:
    """W~_Q^partial: the chosen columns of the skewed query weight, head-major
    (column h*r + c holds channel chan[h][c] of head h) -- step 3 "Extract partial matrices"."""
    H, r = chan.shape
    cols = [h * d + int(c) for h in range(H) for c in chan[h]]
    return np.ascontiguousarray(np.asarray(Wq_s_bits)[:, cols])


def partial_key_cache(K_bits: np.ndarray, chan: np.ndarray) -> np.ndarray:
    """Partial key cache: the same chosen channels of every cached skewed key row
    ([B][H][rows][d] -> [B][H][rows][r]); same indices as the query, step 3 and the
    "same column indices for query and key" paragraph."""
    B, H, rows, d = K_bits.shape
    out = np.empty((B, H, rows, chan.shape[1]), dtype=np.asarray(K_bits).dtype)
    for h in range(H):
        out[:, h] = np.asarray(K_bits)[:, h][:, :, chan[h]]
    return out


# ---------------------------------------------------------------- decoding: speculation
def rehearse(x: np.ndarray, Wq_part: np.ndarray, Kp: np.ndarray, n: int, H: int, r: int,
             scale: float, bq_part: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Decoding stage, step 1 (partial query projection) and step 2 (speculated scores).

    q_part[b, h, :] = x[b] W~_Q^partial[:, h*r:(h+1)*r]  (+ bias), one query row per sequence;
    score[b, h, j]  = scale * q_part[b, h] . Kp[b, h, j]  for the n cached rows.
    Reading: the scores carry the same softmax scale as the attention logits (default 1/sqrt(d)),
    so that alpha is measured in logit units as the pages' e^-alpha argument requires.
    x: [B][D], Wq_part: [D][H*r], Kp: [B][H][rows][r] (all float64 values).
    """
    x = np.asarray(x, dtype=np.float64)
    Wq_part = np.asarray(Wq_part, dtype=np.float64)
    Kp = np.asarray(Kp, dtype=np.float64)
    B = x.shape[0]
    qp = (x @ Wq_part).reshape(B, H, r)
    if bq_part is not None:
        qp = qp + np.asarray(bq_part, dtype=np.float64).reshape(1, H, r)
    s = np.empty((B, H, n))
    for b in range(B):
        for h in range(H):
            s[b, h] = scale * (Kp[b, h, :n, :] @ qp[b, h])
    return qp, s


def order_by_score(s: np.ndarray) -> np.ndarray:
    """Row indices by descending score, lower index first among equal scores."""
    n = len(s)
    return np.lexsort((np.arange(n), -np.asarray(s, dtype=np.float64)))


def select_threshold(s: np.ndarray, alpha: float, max_sel: int = 0, max_out: int = 0) -> np.ndarray:
    """Decoding stage, step 3: keep {j : s_j >= max(s) - alpha}; with the per-layer cap of step 5
    ("up to 20% of the KV cache") keep at most max_sel of them, by descending score.

    Readings: ">=" at the cut (so the maximum is always kept, even for alpha = 0); alpha = +inf
    keeps every row; a set larger than max_sel (or the output capacity max_out) keeps its top rows
    by (score desc, index asc); the result is ascending.  max_sel = 0 or max_out = 0: no limit.
    """
    s = np.asarray(s, dtype=np.float64)
    if len(s) == 0:
        return np.zeros(0, dtype=np.int32)
    m = s.max()
    cut = m - alpha
    S = np.nonzero(s >= cut)[0]
    limit = len(s)
    if max_sel > 0:
        limit = min(limit, max_sel)
    if max_out > 0:
        limit = min(limit, max_out)
    if len(S) > limit:
        S = order_by_score(s)[:limit]
    return np.sort(S).astype(np.int32)


def select_topk(s: np.ndarray, k: int, max_out: int = 0) -> np.ndarray:
    """Fixed-budget mode: the k largest scores (all rows if k >= n), ties to the lower index,
    clamped to the output capacity; ascending.  (The pages' "Optimal" comparator in
    section 2, challenge C1, is this rule applied to exact attention scores.)"""
    s = np.asarray(s, dtype=np.float64)
    kk = min(k, len(s))
    if max_out > 0:
        kk = min(kk, max_out)
    return np.sort(order_by_score(s)[:kk]).astype(np.int32)


def select(scores: np.ndarray, mode: str, alpha: float = math.inf, k: int = 0,
           max_sel: int = 0, max_out: int = 0):
    """Apply the per-head rule to every (b, h) row; returns idx [B][H][max_out] (ascending,
    zero padded) and count [B][H]."""
    scores = np.asarray(scores, dtype=np.float64)
    B, H, n = scores.shape
    cap = max_out if max_out > 0 else n
    idx = np.zeros((B, H, cap), dtype=np.int32)
    cnt = np.zeros((B, H), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            if mode == "threshold":
                S = select_threshold(scores[b, h], alpha, max_sel, cap)
            elif mode == "topk":
                S = select_topk(scores[b, h], k, cap)
            else:
                raise ValueError(mode)
            idx[b, h, :len(S)] = S
            cnt[b, h] = len(S)
    return idx, cnt


def select_head_average(scores: np.ndarray, alpha: float, max_sel: int = 0, max_out: int = 0):
    """Decoding stage, step 4 (multi-head averaging): every head of a sequence takes the same
    count, the mean over heads of the per-head threshold counts; each head then keeps its top
    rows by score.  Readings: the mean is rounded up; the 20% cap and the output capacity
    apply to the averaged count."""
    scores = np.asarray(scores, dtype=np.float64)
    B, H, n = scores.shape
    cap = max_out if max_out > 0 else n
    idx = np.zeros((B, H, cap), dtype=np.int32)
    cnt = np.zeros((B, H), dtype=np.int32)
    for b in range(B):
        counts = [len(select_threshold(scores[b, h], alpha)) for h in range(H)]
        cbar = int(math.ceil(sum(counts) / H))
        if max_sel > 0:
            cbar = min(cbar, max_sel)
        cbar = min(cbar, cap)
        for h in range(H):
            S = select_topk(scores[b, h], cbar)
            idx[b, h, :len(S)] = S
            cnt[b, h] = len(S)
    return idx, cnt


# ---------------------------------------------------------------- decoding: attention on the selection
def gather_kv(K: np.ndarray, V: np.ndarray, idx: np.ndarray, count: np.ndarray, max_out: int):
    """Fetch the full key and value rows of the selected tokens into compact buffers
    (decoding stage, step 5: the full rows, all channels, of the chosen tokens)."""
    B, H, _, d = K.shape
    Kc = np.zeros((B, H, max_out, d), dtype=K.dtype)
    Vc = np.zeros((B, H, max_out, d), dtype=V.dtype)
    for b in range(B):
        for h in range(H):
            c = int(count[b, h])
            Kc[b, h, :c] = K[b, h, idx[b, h, :c]]
            Vc[b, h, :c] = V[b, h, idx[b, h, :c]]
    return Kc, Vc


def attention_rows(q: np.ndarray, K_rows: np.ndarray, V_rows: np.ndarray, scale: float):
    """softmax(scale q K^T) V over the given rows (section 2, the attention definition), with the
    natural-log partition value lse = log sum_j exp(scale q.K_j).  No rows: o = 0, lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    K_rows = np.asarray(K_rows, dtype=np.float64)
    V_rows = np.asarray(V_rows, dtype=np.float64)
    if K_rows.shape[0] == 0:
        return np.zeros(V_rows.shape[1]), -math.inf
    logits = scale * (K_rows @ q)
    m = logits.max()
    w = np.exp(logits - m)
    z = w.sum()
    return (w @ V_rows) / z, m + math.log(z)


def sparse_decode_attn(q: np.ndarray, K: np.ndarray, V: np.ndarray, idx: Optional[np.ndarray],
                       count: np.ndarray, scale: float):
    """Attention of each (b, h) query over the selected cached rows only (Inference Controller,
    section 3.2; the rest of the cache is dropped for this layer and step).  idx None: the first
    count rows.  q [B][H][d], K/V [B][H][rows][d] values -> o [B][H][d], lse [B][H]."""
    q = np.asarray(q, dtype=np.float64)
    B, H, d = q.shape
    o = np.zeros((B, H, d))
    lse = np.zeros((B, H))
    for b in range(B):
        for h in range(H):
            c = int(count[b, h])
            rows = np.arange(c) if idx is None else np.asarray(idx[b, h, :c], dtype=np.int64)
            o[b, h], lse[b, h] = attention_rows(q[b, h], K[b, h, rows], V[b, h, rows], scale)
    return o, lse


def dense_decode_attn(q, K, V, n: int, scale: float):
    """Dense decode attention over all n cached rows (section 2: softmax(QK^T)V over the
    H x (N+i) x d cache)."""
    q = np.asarray(q, dtype=np.float64)
    B, H, _ = q.shape
    return sparse_decode_attn(q, K, V, None, np.full((B, H), n, dtype=np.int32), scale)


# ---------------------------------------------------------------- KV pool management
def pool_touch(C: np.ndarray, idx: np.ndarray, count: np.ndarray, n: int, cmax: int,
               want_victim: bool = False):
    """Counter-based pool policy (section 3.4, "KV Cache Pool Management Under Memory Pressure"):
    a slot's counter rises each time the token is selected; when a counter saturates all counters
    of the pool are halved; the victim is the slot with the smallest counter.

    Readings: +1 per (head, selected slot) per step; storage uint32 with saturation value cmax:
    C <- min(C + inc, cmax), then if any slot j < n holds cmax, every slot j < n is halved (floor);
    victim = lowest index among the minima over j < n.  Precondition: C[b, j] < cmax for j < n.
    Returns (C_new, victim [B] int32 or None).
    """
    C = np.array(C, dtype=np.int64)
    B = C.shape[0]
    H = count.shape[1]
    assert (C[:, :n] < cmax).all(), "counters must be below cmax on entry"
    inc = np.zeros_like(C)
    for b in range(B):
        for h in range(H):
            for j in idx[b, h, :int(count[b, h])]:
                inc[b, int(j)] += 1
    C = np.minimum(C + inc, cmax)
    victim = np.zeros(B, dtype=np.int32) if want_victim else None
    for b in range(B):
        if (C[b, :n] == cmax).any():
            C[b, :n] //= 2
        if want_victim:
            victim[b] = int(np.argmin(C[b, :n]))
    return C.astype(np.uint32), victim


def pool_append(K_bits, V_bits, Kp_bits, C, chan, k_new, v_new, n: int, victim=None):
    """Append the new token of each sequence (section 3.4, "Partial Key Cache Updates During
    Decoding" and the pool paragraph): slot n while the pool has room, else the victim slot;
    the full key and value rows go to the slot, the chosen channels of the key to the partial
    key cache row, and the slot's counter restarts at 0.  Returns (slots [B], new n)."""
    B, H, cap, d = K_bits.shape
    slots = np.zeros(B, dtype=np.int64)
    for b in range(B):
        slot = n if n < cap else int(victim[b])
        slots[b] = slot
        K_bits[b, :, slot] = k_new[b]
        V_bits[b, :, slot] = v_new[b]
        for h in range(H):
            Kp_bits[b, h, slot] = k_new[b, h, chan[h]]
        C[b, slot] = 0
    return slots, min(n + 1, cap)


# ---------------------------------------------------------------- INT4 host pool (follow-up)
INT4_GROUP = 32   # elements per quantisation group (along the head dimension)


def quantize_int4(X_bits: np.ndarray, dtype: str, group: int = INT4_GROUP):
    """Group-wise asymmetric 4-bit quantisation of stored key or value rows: the INT4 scheme the
    pages name among the baselines (section 5 "Evaluation Methodology", the quantised-KV baseline)
    and propose to combine with the speculative selection (the "Follow-Up Research" paragraph on
    combining prefetching with KV cache quantisation).

    Per group of `group` consecutive elements v of a row: mn = min v, mx = max v; the group keeps
    its minimum and step s = (mx - mn) / 15 as float16 (nearest-even), m16 and s16, and one code per
    element, q = clamp(rint((v - m16) / s16), 0, 15) (q = 0 when s16 is 0).
    Readings: the pages give neither the group size nor the storage of the group constants; groups
    run along the head dimension and the constants are float16.  A code is an integer decided by
    floating-point arithmetic, so it is decided in float32 (the precision the kernel computes in),
    with rint rounding half to even; the values must lie in float16's range.
    Returns codes uint8 [..., d] (0..15, one per element), s16 and m16 float16 [..., d / group]."""
    v = decode(X_bits, dtype).astype(np.float32)
    d = v.shape[-1]
    assert d % group == 0
    g = v.reshape(v.shape[:-1] + (d // group, group))
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    s = (mx - mn) / np.float32(15.0)
    s16 = s.astype(np.float16)
    m16 = mn.astype(np.float16)
    sf = s16.astype(np.float32)[..., None]
    mf = m16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g - mf) / sf
    q = np.where(sf > 0, np.clip(np.rint(t), 0, 15), 0).astype(np.uint8)
    return q.reshape(v.shape), s16, m16


def dequantize_int4(q: np.ndarray, s16: np.ndarray, m16: np.ndarray, group: int = INT4_GROUP) -> np.ndarray:
    """Values of quantised rows, float64: v = m16 + q * s16 for each element of a group."""
    d = q.shape[-1]
    qg = q.astype(np.float64).reshape(q.shape[:-1] + (d // group, group))
    v = m16.astype(np.float64)[..., None] + qg * s16.astype(np.float64)[..., None]
    return v.reshape(q.shape)


def gather_kv_int4(Kq, Ks, Km, Vq, Vs, Vm, idx: np.ndarray, count: np.ndarray, max_out: int, dtype: str,
                   group: int = INT4_GROUP):
    """Step 5 on a quantised pool: the selected rows, dequantised (float64, then stored in `dtype`
    as a float32-computing kernel stores them), in compact buffers [B][H][max_out][d]."""
    B, H, _, d = Kq.shape
    Kc = np.zeros((B, H, max_out, d))
    Vc = np.zeros((B, H, max_out, d))
    for b in range(B):
        for h in range(H):
            rows = idx[b, h, :int(count[b, h])]
            Kc[b, h, :len(rows)] = dequantize_int4(Kq[b, h, rows], Ks[b, h, rows], Km[b, h, rows], group)
            Vc[b, h, :len(rows)] = dequantize_int4(Vq[b, h, rows], Vs[b, h, rows], Vm[b, h, rows], group)
    return store(Kc, dtype), store(Vc, dtype)


# ---------------------------------------------------------------- one decode layer-step
def decode_step(x, Wq_part, Kp, q, K, V, C, *, n, H, r, scale, mode, alpha=math.inf, k=0,
                max_sel=0, max_out=0, cmax=65535, bq_part=None, want_victim=False):
    """One layer-step of the hot path, in the pages' order (section 3.4, "Decoding Stage" steps 1-5
    and the pool paragraph): partial query, speculated scores, selection (mode "threshold" or "topk"
    per head, or "headavg": step 4's multi-head averaging of the threshold counts), attention over
    the selected rows, counter update.  Inputs are float64 values, except the counters C (uint32,
    left unchanged when None: then no counters or victim are returned)."""
    qp, s = rehearse(x, Wq_part, Kp, n, H, r, scale, bq_part)
    if mode == "headavg":
        idx, cnt = select_head_average(s, alpha, max_sel=max_sel, max_out=max_out)
    else:
        idx, cnt = select(s, mode, alpha=alpha, k=k, max_sel=max_sel, max_out=max_out)
    o, lse = sparse_decode_attn(q, K, V, idx, cnt, scale)
    C2 = victim = None
    if C is not None:
        C2, victim = pool_touch(C, idx, cnt, n, cmax, want_victim)
    return dict(q_part=qp, scores=s, idx=idx, count=cnt, out=o, lse=lse, counters=C2, victim=victim)

"""Two independent routes from the same raw draws to the decode-path inputs.

``lib_inputs`` runs the library's own host setup (libig.so: Jacobi skew,
rotation, storage rounding, channel pick) and ``oracle_inputs`` runs the
oracle's (numpy SVD, ...).  Only ``gen`` is shared.  The two routes agree to
float64 rounding, so the stored bits they produce coincide; ``compare_inputs``
checks that as a setup-parity result.  Comparison helpers implement the parity
rules: scores within 1e-3 (row-normwise), index sets and counters exact except
rows whose oracle score lies within 1e-4 of the cut, attention within 1e-2
(bf16 inputs) or 1e-5 (float32 inputs).
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from sparse_attention_ig_amd import gen
from sparse_attention_ig_amd.runtime import HostLayer, heads_layout, prepare_layer, rows_layout

SCORE_RTOL = 1e-3
BAND = 1e-4
ATTN_TOL = {"bf16": 1e-2, "f32": 1e-5}


Inputs = HostLayer
_rows_layout = rows_layout
_heads_layout = heads_layout


def lib_inputs(spec: gen.Spec, layer: int = 0, lay: Optional[gen.Layer] = None) -> Inputs:
    return prepare_layer(spec, layer, lay)


def oracle_inputs(spec: gen.Spec, layer: int = 0, lay: Optional[gen.Layer] = None) -> Inputs:
    from oracle import oracle as O
    B, H, d, r = spec.B, spec.H, spec.d, spec.r
    lay = lay or gen.draw_layer(spec, layer, with_wk=False)
    A, Wq_s64, _, _, _ = O.skew_weights(lay.Wq, None, lay.skew_src)
    Wq_s = O.store(Wq_s64, spec.dtype)
    q = O.store(O.skew_apply(A, lay.q_raw), spec.dtype)
    if spec.frame == "raw":
        K = O.store(_heads_layout(O.skew_apply(A, _rows_layout(lay.K_raw)), B, H, spec.cap, d), spec.dtype)
        V, heavy = lay.V, lay.heavy_pos
    else:
        K, V, heavy = gen.draw_cache(spec, layer, O.decode(q, spec.dtype))
    chan = O.partial_weight_index(Wq_s, K, H, d, r, spec.n, dtype=spec.dtype)
    Wq_part = O.pack_partial_weight(Wq_s, chan, d)
    return Inputs(spec, lay.x, Wq_part, chan, q.reshape(B, H, d), K, V,
                  extra={"A": A, "heavy": heavy, "Kp": O.partial_key_cache(K, chan), "Wq_s": Wq_s})


def ulp_mismatch(a: np.ndarray, b: np.ndarray) -> int:
    """Number of stored elements whose bits differ (float32 / bf16 arrays)."""
    return int(np.count_nonzero(a.view(np.uint32 if a.dtype == np.float32 else np.uint16)
                                != b.view(np.uint32 if b.dtype == np.float32 else np.uint16)))


def assert_setup_routes_agree(a: Inputs, b: Inputs) -> Dict[str, int]:
    """The two setup routes give the same channel sets, x and V bit for bit, and the rotated K, q and
    Wq_part bit for bit up to a handful of elements (a float64 rotation by the Jacobi and by the LAPACK
    SVD may round an element to the neighbouring bfloat16 value); returns the mismatch counts."""
    mism = compare_inputs(a, b)
    assert mism["chan"] == 0 and mism["x"] == 0 and mism["V"] == 0, mism
    total = a.K.size + a.q.size + a.Wq_part.size
    assert mism["K"] + mism["q"] + mism["Wq_part"] <= max(2, total * 1e-5), mism
    return mism


def compare_inputs(a: Inputs, b: Inputs) -> Dict[str, int]:
    """Setup parity: bits of every derived input, and the channel sets."""
    return {
        "chan": int(np.count_nonzero(a.chan != b.chan)),
        "Wq_part": ulp_mismatch(a.Wq_part, np.ascontiguousarray(b.Wq_part.T)),  # library layout: [H*r][D]
        "q": ulp_mismatch(a.q, b.q),
        "K": ulp_mismatch(a.K, b.K),
        "V": ulp_mismatch(a.V, b.V),
        "x": ulp_mismatch(a.x, b.x),
    }


# ---------------------------------------------------------------- oracle side of a step
def oracle_step(inp: Inputs, *, mode: str, alpha: float = math.inf, k: int = 0, max_sel: int = 0,
                max_out: int = 0, cmax: int = 65535, counters: Optional[np.ndarray] = None,
                want_victim: bool = False, heads=None):
    """The oracle's decode layer-step on its own inputs.  ``heads``: optional list of (b, h) to
    evaluate (sampled parity at large sizes); counters are then not computed."""
    from oracle import oracle as O
    s = inp.spec
    dt = s.dtype
    x = O.decode(inp.x, dt)
    Wp = O.decode(inp.Wq_part, dt)
    Kp = inp.extra.get("Kp")
    if Kp is None:
        Kp = O.partial_key_cache(inp.K, inp.chan)
    if heads is None:
        return O.decode_step(x, Wp, O.decode(Kp, dt), O.decode(inp.q, dt), O.decode(inp.K, dt), O.decode(inp.V, dt),
                             counters, n=s.n, H=s.H, r=s.r, scale=s.softmax_scale, mode=mode, alpha=alpha, k=k,
                             max_sel=max_sel, max_out=max_out, cmax=cmax, want_victim=want_victim)
    return oracle_heads(inp, mode=mode, alpha=alpha, k=k, max_sel=max_sel, max_out=max_out, heads=heads)[0]


def oracle_heads(inp: Inputs, *, mode: str, alpha: float = math.inf, k: int = 0, max_sel: int = 0,
                 max_out: int = 0, n: Optional[int] = None, x_bits=None, heads=None, attn: bool = True,
                 Kp=None, q_layer: Optional[Inputs] = None):
    """The oracle's layer-step one (b, h) at a time, decoding only that head's rows (the whole cache in
    float64 would not fit at the long-context sizes): partial query, scores, selection and (attn) the
    attention over the selected rows.  ``heads``: list of (b, h), default every head; ``x_bits``: the
    attention input driving the speculation (default the layer's own x); ``n``: rows (default the
    spec's); ``Kp``: partial key cache bits (default the layer's); ``q_layer``: the layer whose query,
    K and V the attention uses (default ``inp``).  Returns (records per (b, h), idx [B][H][cap]
    ascending, count [B][H]) -- the last two for the counters of every head."""
    from oracle import oracle as O
    s = inp.spec
    dt = s.dtype
    n = s.n if n is None else n
    x = O.decode(inp.x if x_bits is None else x_bits, dt)
    Wp = O.decode(inp.Wq_part, dt)
    if Kp is None:
        Kp = inp.extra.get("Kp")
        if Kp is None:
            Kp = O.partial_key_cache(inp.K, inp.chan)
    ql = inp if q_layer is None else q_layer
    if heads is None:
        heads = [(b, h) for b in range(s.B) for h in range(s.H)]
    cap = max_out if max_out > 0 else n
    idx_all = np.zeros((s.B, s.H, cap), dtype=np.int32)
    cnt_all = np.zeros((s.B, s.H), dtype=np.int32)
    out = {}
    for (b, h) in heads:
        qp, sc = O.rehearse(x[b:b + 1], Wp[:, h * s.r:(h + 1) * s.r], O.decode(Kp[b:b + 1, h:h + 1, :n], dt), n, 1,
                            s.r, s.softmax_scale)
        idx, cnt = _oracle_select(sc, mode, alpha, k, max_sel, max_out)
        c = int(cnt[0, 0])
        rows = idx[0, 0, :c].astype(np.int64)
        rec = dict(q_part=qp[0, 0], scores=sc[0, 0], idx=rows)
        if attn:
            rec["out"], rec["lse"] = O.attention_rows(O.decode(ql.q[b, h], dt), O.decode(ql.K[b, h, rows], dt),
                                                      O.decode(ql.V[b, h, rows], dt), s.softmax_scale)
        out[(b, h)] = rec
        idx_all[b, h, :c] = rows
        cnt_all[b, h] = c
    return out, idx_all, cnt_all


def _oracle_select(sc, mode, alpha, k, max_sel, max_out):
    from oracle import oracle as O
    if mode == "headavg":
        return O.select_head_average(sc, alpha, max_sel, max_out)
    return O.select(sc, mode, alpha=alpha, k=k, max_sel=max_sel, max_out=max_out)


# ---------------------------------------------------------------- comparisons
def score_error(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max_j |gpu - ref| / max_j |ref| (row-normwise)."""
    g = gpu.reshape(-1, gpu.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1])
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((np.abs(g - r).max(axis=1) / den).max())


def cut_of(ref_scores: np.ndarray, ref_sel: np.ndarray, mode: str, alpha: float) -> float:
    """The value the selection was cut at: max - alpha, or the smallest kept score when the
    set was cut by count (top-k, head average, or a threshold set hitting its cap)."""
    if mode == "threshold":
        cut = ref_scores.max() - alpha
        kept_all = np.count_nonzero(ref_scores >= cut)
        if kept_all == len(ref_sel):
            return cut
    return float(ref_scores[ref_sel].min()) if len(ref_sel) else math.inf


def check_heads(g_idx, g_cnt, ref: dict, mode: str, alpha: float, g_q_part=None, g_scores=None, g_out=None,
                g_lse=None, tol: Optional[float] = None, n: Optional[int] = None):
    """Every (b, h) of ``ref`` (oracle_heads records) against the GPU's arrays: q_part and scores within
    1e-3 row-normwise, the index set equal outside the 1e-4 band (ascending, distinct), and where the
    sets are equal the attention within ``tol``.  Returns the heads whose sets differ inside the band."""
    inexact = []
    for (b, h), r in ref.items():
        if g_q_part is not None:
            assert score_error(g_q_part[b, h], r["q_part"]) <= SCORE_RTOL, ("q_part", b, h)
        if g_scores is not None:
            sc = g_scores[b, h, :len(r["scores"])]
            assert score_error(sc, r["scores"]) <= SCORE_RTOL, ("scores", b, h)
        gs = g_idx[b, h, :g_cnt[b, h]]
        assert np.all(np.diff(gs) > 0), ("not ascending", b, h)
        ok, exact, band = compare_sets(gs, r["idx"], r["scores"], mode, alpha)
        assert ok, ("set", b, h, sorted(set(gs.tolist()) ^ set(r["idx"].tolist())))
        if not exact:
            inexact.append((b, h))
            continue
        if g_out is not None and "out" in r:
            err = np.abs(g_out[b, h] - r["out"]).max()
            assert err <= tol, ("attention", b, h, err)
            if g_lse is not None:
                assert abs(g_lse[b, h] - r["lse"]) <= max(tol, 1e-5 * abs(r["lse"])), ("lse", b, h)
    return inexact


def check_counters(g_C, ref_C, g_idx, g_cnt, ref_idx, ref_cnt, n: int, g_victim=None, ref_victim=None):
    """Counters slot by slot.  A head whose set differs from the oracle's inside the 1e-4 band moves the
    counters of exactly those slots, by at most the number of such heads: every other slot must be equal,
    and the victim too where no slot moved.  (No halving may differ: callers keep counters below cmax.)
    Returns the sequences with moved slots."""
    B = g_C.shape[0]
    H = g_cnt.shape[1]
    moved = []
    for b in range(B):
        diff = np.zeros(n, dtype=np.int64)
        for h in range(H):
            gs = set(int(v) for v in g_idx[b, h, :g_cnt[b, h]])
            rs = set(int(v) for v in ref_idx[b, h, :ref_cnt[b, h]])
            for j in gs ^ rs:
                diff[j] += 1
        free = diff == 0
        assert np.array_equal(g_C[b, n:], ref_C[b, n:]), ("counters past n", b)
        assert np.array_equal(g_C[b, :n][free], ref_C[b, :n][free]), ("counters", b)
        gd = np.abs(g_C[b, :n].astype(np.int64) - ref_C[b, :n].astype(np.int64))
        assert (gd[~free] <= diff[~free]).all(), ("counters in the band", b)
        if (~free).any():
            moved.append(b)
        elif g_victim is not None:
            assert g_victim[b] == ref_victim[b], ("victim", b)
    return moved


def band_rows(ref_scores: np.ndarray, cut: float) -> np.ndarray:
    return np.flatnonzero(np.abs(ref_scores - cut) <= BAND)


def compare_sets(gpu_sel: np.ndarray, ref_sel: np.ndarray, ref_scores: np.ndarray, mode: str, alpha: float):
    """Returns (ok, exact, band) -- ok: sets equal outside the band; exact: equal outright."""
    g = set(int(v) for v in gpu_sel)
    r = set(int(v) for v in ref_sel)
    cut = cut_of(ref_scores, np.asarray(sorted(r), dtype=np.int64), mode, alpha)
    band = set(int(v) for v in band_rows(ref_scores, cut))
    ok = (g - band) == (r - band)
    return ok, g == r, band


# ---------------------------------------------------------------- multi-layer pipeline
def pipeline_setup(spec: gen.Spec, layers: int, steps: int, route):
    """Per-layer inputs through ``route`` (lib_inputs or oracle_inputs) from the shared pipeline draws:
    x_l(0) drives each layer's own query, x_l(t) drives the speculation for layer l+1."""
    xs = gen.pipeline_x(spec, layers, steps)
    ins = [route(spec, l, lay=gen.draw_layer(spec, l, x_bits=xs[0, l], with_wk=False)) for l in range(layers)]
    new = [[gen.draw_new_rows(spec, l, t) for l in range(layers)] for t in range(steps)]
    return xs, ins, new


def oracle_pipeline(spec: gen.Spec, xs, ins, new, max_out: int, cmax: int = 65535):
    """The oracle's decode loop: per step, per layer l, attention over idx_l (layer 0 dense), then the
    speculation for layer l+1 from x_l; after the last layer every layer appends the new token."""
    from oracle import oracle as O
    dt = spec.dtype
    L = len(ins)
    K = [i.K.copy() for i in ins]
    V = [i.V.copy() for i in ins]
    Kp = [O.partial_key_cache(i.K, i.chan) for i in ins]
    C = [np.zeros((spec.B, spec.cap), np.uint32) for _ in ins]
    idx = [None] * L
    cnt = [None] * L
    victim = [None] * L
    n = spec.n
    trace = []
    for t in range(xs.shape[0]):
        rec = {"n": n, "out": [], "idx": [None] * L, "count": [None] * L, "scores": [None] * L}
        k = min(max_out, int(math.ceil(0.05 * n)))
        for l in range(L):
            q = O.decode(ins[l].q, dt)
            if l == 0:
                o, _ = O.dense_decode_attn(q, O.decode(K[l], dt), O.decode(V[l], dt), n, spec.softmax_scale)
            else:
                o, _ = O.sparse_decode_attn(q, O.decode(K[l], dt), O.decode(V[l], dt), idx[l], cnt[l],
                                            spec.softmax_scale)
            rec["out"].append(o)
            if l + 1 < L:
                _, sc = O.rehearse(O.decode(xs[t, l], dt), O.decode(ins[l + 1].Wq_part, dt),
                                   O.decode(Kp[l + 1], dt), n, spec.H, spec.r, spec.softmax_scale)
                idx[l + 1], cnt[l + 1] = O.select(sc, "topk", k=k, max_out=max_out)
                C[l + 1], victim[l + 1] = O.pool_touch(C[l + 1], idx[l + 1], cnt[l + 1], n, cmax, want_victim=True)
                rec["idx"][l + 1], rec["count"][l + 1], rec["scores"][l + 1] = idx[l + 1], cnt[l + 1], sc
        full = n == spec.cap
        if full:
            # layer 0 attends to every row and no speculation selects for it: its victim is the lowest
            # slot among the minima of counters that only appends reset
            _, victim[0] = O.pool_touch(C[0], np.zeros((spec.B, spec.H, 1), np.int32),
                                        np.zeros((spec.B, spec.H), np.int32), n, cmax, want_victim=True)
        rec["victims"] = [None if v is None else v.copy() for v in victim] if full else None
        for l in range(L):
            kn, vn = new[t][l]
            _, n2 = O.pool_append(K[l], V[l], Kp[l], C[l], ins[l].chan, kn, vn, n,
                                  victim=victim[l] if full else None)
        n = n2
        trace.append(rec)
    trace[-1]["K"] = K   # the caches after the last append
    return trace, C

"""Seeded synthetic inputs for the InfiniGen decode hot path.

This module only draws random numbers and encodes them in the storage dtype.
It holds none of the method's arithmetic (no skewing, no channel pick, no
scores, no selection, no attention, no counters): the library and the oracle
each run those on what is drawn here.  Both sides import this module; it
imports neither of them.

Workload shapes follow the OPT / Llama-2 decode layers the InfiniGen paper
evaluates (paper-graph-ui summary of arXiv 2406.19707, section 5 "Evaluation
Methodology": OPT 6.7B-30B, Llama-2 7B/13B; partial ratio, alpha and the 20%
cap from the same section).  The pages' datasets are not used; these draws
stand in for their shapes only.

Two stages:

* ``draw_layer`` -- everything that does not depend on the skew rotation:
  the attention input x, the raw query weight W_Q (and W_K), the matrix whose
  right singular vectors define the rotation, the raw query q = x W_Q (the
  model's own query projection, which the method takes as given), and for the
  "raw frame" workloads the raw key / value cache.
* ``draw_cache`` -- for the "skewed frame" workloads, the key cache drawn
  directly in the rotated basis (per-channel log-normal scales, so that a few
  channels dominate after skewing) with heavy hitters pushed along the unit
  skewed query that the caller passes in, and the value cache.

Every random stream is keyed by (base seed, layer, purpose, b, h) through
numpy's SeedSequence, so any (b, h) slice can be re-drawn alone.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os
from typing import Optional

import numpy as np

# purpose codes for keyed sub-streams
_P_X, _P_WQ, _P_WK, _P_SKEW, _P_XS, _P_K, _P_V, _P_HEAVY, _P_KSCALE, _P_VSCALE, \
    _P_NEWKV, _P_CNT, _P_DRIFT, _P_IDX = range(14)


@dataclasses.dataclass(frozen=True)
class Spec:
    """One synthetic decode-layer workload."""
    name: str
    B: int
    H: int
    d: int
    n: int                 # current rows N+i
    r: int                 # partial channels per head
    dtype: str             # "f32" | "bf16"
    wstd: float            # std of W_Q / W_K entries
    heavy: int             # heavy-hitter rows per (b, h)
    gamma: float           # heavy-hitter key boost
    frame: str             # "raw": K given unskewed, rotated by the setup; "skewed": K drawn rotated
    skew: str              # "query_svd": A from sample query X_s W_Q; "gauss_block": A from random d x d block
    heavy_shared: bool = False   # same heavy positions for every head (tiny workload)
    heavy_span: int = 0          # > 0: heavy positions drawn from the first heavy_span rows only
    lognormal: bool = True       # per-channel log-normal K / V scales
    n_cap: int = 0               # allocated rows (0 -> n)
    seed: int = 1000
    alpha: float = 5.0
    topk: int = 128
    cap_frac: float = 0.2
    scale: float = 0.0           # 0 -> 1/sqrt(d)
    xs_rows: int = 256           # rows of the sample input for "query_svd"

    @property
    def D(self) -> int:
        return self.H * self.d

    @property
    def cap(self) -> int:
        return self.n_cap if self.n_cap else self.n

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.d)

    @property
    def max_sel(self) -> int:
        """Per-head cap on a threshold selection: 20% of the current rows, at least 1."""
        return max(1, int(math.floor(self.cap_frac * self.n)))


def tiny_fp32() -> Spec:
    """Tiny single layer: B1 H4 d64 hidden 256 N256 r16 fp32, 8 shared heavy tokens x4."""
    return Spec("tiny-fp32", B=1, H=4, d=64, n=256, r=16, dtype="f32", wstd=1.0 / 16,
                heavy=8, gamma=4.0, frame="raw", skew="query_svd", heavy_shared=True,
                lognormal=False, seed=1001, alpha=4.0, topk=32, scale=1.0 / 8)


def opt_6_7b(n: int = 2048, B: int = 8) -> Spec:
    """OPT-6.7B-shaped decode layer: hidden 4096, H32 d128, B8, N2048, r32, bf16, 2% heavy."""
    return Spec("opt-6.7b", B=B, H=32, d=128, n=n, r=32, dtype="bf16", wstd=1.0 / 64,
                heavy=int(round(0.02 * n)), gamma=3.0, frame="skewed", skew="gauss_block",
                seed=1002, alpha=5.0, topk=128)


def llama2_13b(n: int = 4096, B: int = 16, n_cap: int = 4352) -> Spec:
    """Llama-2-13B-shaped layer of the 40-layer pipeline: hidden 5120, H40 d128, B16, r32."""
    return Spec("llama2-13b", B=B, H=40, d=128, n=n, r=32, dtype="bf16", wstd=1.0 / math.sqrt(5120),
                heavy=int(round(0.02 * n)), gamma=3.0, frame="skewed", skew="gauss_block",
                n_cap=n_cap, seed=1003, alpha=5.0, topk=int(math.ceil(0.05 * n)))


def opt_30b(n: int = 2048, B: int = 16, n_cap: int = 4096) -> Spec:
    """OPT-30B-shaped offloaded-pool layer: hidden 7168, H56 d128, B16, r32, alpha 5, cap 20%."""
    return Spec("opt-30b", B=B, H=56, d=128, n=n, r=32, dtype="bf16", wstd=1.0 / math.sqrt(7168),
                heavy=int(round(0.02 * n)), gamma=3.0, frame="skewed", skew="gauss_block",
                n_cap=n_cap, seed=1004, alpha=5.0, topk=0)


def llama2_7b_long(n: int = 32768, B: int = 1, frac: float = 0.01) -> Spec:
    """Long-context Llama-2-7B-shaped layer: hidden 4096, H32 d128, 1% heavy, top-k frac of n."""
    return Spec("llama2-7b-long", B=B, H=32, d=128, n=n, r=32, dtype="bf16", wstd=1.0 / 64,
                heavy=int(round(0.01 * n)), gamma=3.0, frame="skewed", skew="gauss_block",
                seed=1005, alpha=5.0, topk=int(math.ceil(frac * n)))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(spec: Spec, layer: int, purpose: int, *keys: int) -> np.random.Generator:
    ss = np.random.SeedSequence([spec.seed, layer, purpose, *keys])
    return np.random.Generator(np.random.PCG64(ss))


# ---------------------------------------------------------------- encoding
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    if nan.any():
        out[nan] = 0x7FC0
    return out


def encode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage encoding of drawn values: float32 array, or bf16 bits as uint16."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits(np.asarray(a, dtype=np.float32))
    raise ValueError(dtype)


def values(bits: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values of an encoded array (used to build follow-on draws, not by the method)."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float64)
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- stage 1
@dataclasses.dataclass
class Layer:
    spec: Spec
    layer: int
    x: np.ndarray            # [B][D] encoded
    Wq: np.ndarray           # [D][H*d] float64 (values of float32 draws)
    Wk: np.ndarray           # [D][H*d] float64
    skew_src: np.ndarray     # [H][m][d] float64
    q_raw: np.ndarray        # [B][H*d] float64 = x W_Q (unskewed query)
    K_raw: Optional[np.ndarray] = None   # [B][H][n_cap][d] float64, raw frame only
    V: Optional[np.ndarray] = None       # [B][H][n_cap][d] encoded, raw frame only
    heavy_pos: Optional[np.ndarray] = None


def draw_x(spec: Spec, layer: int = 0) -> np.ndarray:
    g = _rng(spec, layer, _P_X)
    return encode(g.standard_normal((spec.B, spec.D), dtype=np.float32), spec.dtype)


def draw_layer(spec: Spec, layer: int = 0, x_bits: Optional[np.ndarray] = None,
               with_wk: bool = True) -> Layer:
    """Stage-1 draws for one layer.  ``x_bits`` overrides the attention input (pipelines)."""
    B, H, d, D = spec.B, spec.H, spec.d, spec.D
    x = draw_x(spec, layer) if x_bits is None else x_bits
    Wq = (_rng(spec, layer, _P_WQ).standard_normal((D, D), dtype=np.float32) * np.float32(spec.wstd)).astype(np.float64)
    Wk = None
    if with_wk:
        Wk = (_rng(spec, layer, _P_WK).standard_normal((D, D), dtype=np.float32) * np.float32(spec.wstd)).astype(np.float64)
    # the model's own query projection of the (encoded) attention input
    q_raw = values(x, spec.dtype) @ Wq
    if spec.skew == "query_svd":
        # sample forward pass: Q_h = X_s W_Q,h over a Gaussian sample input
        Xs = _rng(spec, layer, _P_XS).standard_normal((spec.xs_rows, D)).astype(np.float64)
        Qs = Xs @ Wq
        skew_src = np.stack([Qs[:, h * d:(h + 1) * d] for h in range(H)])
    elif spec.skew == "gauss_block":
        skew_src = np.stack([_rng(spec, layer, _P_SKEW, h).standard_normal((d, d)) for h in range(H)])
    else:
        raise ValueError(spec.skew)
    lay = Layer(spec, layer, x, Wq, Wk, np.ascontiguousarray(skew_src), q_raw)
    if spec.frame == "raw":
        lay.K_raw, lay.V, lay.heavy_pos = _raw_cache(spec, layer, q_raw)
    return lay


def _heavy_positions(spec: Spec, layer: int, b: int, h: int) -> np.ndarray:
    if spec.heavy <= 0:
        return np.zeros(0, dtype=np.int64)
    key = (0, 0) if spec.heavy_shared else (b, h)
    g = _rng(spec, layer, _P_HEAVY, *key)
    span = min(spec.heavy_span, spec.n) if spec.heavy_span > 0 else spec.n
    assert spec.heavy_span <= 0 or spec.heavy <= span, "heavy rows must fit their span"
    return np.sort(g.choice(span, size=min(spec.heavy, span), replace=False))


def _raw_cache(spec: Spec, layer: int, q_raw: np.ndarray):
    """Unit-scale Gaussian K (unskewed frame) with heavy keys pushed along the raw query; V."""
    B, H, d, n, cap = spec.B, spec.H, spec.d, spec.n, spec.cap
    K = np.zeros((B, H, cap, d))
    V = np.zeros((B, H, cap, d), dtype=np.float32)
    heavy = np.zeros((B, H, max(spec.heavy, 0)), dtype=np.int64)
    rho = math.sqrt(d)          # expected key norm for unit-variance channels
    for b in range(B):
        for h in range(H):
            K[b, h, :n] = _rng(spec, layer, _P_K, b, h).standard_normal((n, d))
            V[b, h, :n] = _rng(spec, layer, _P_V, b, h).standard_normal((n, d), dtype=np.float32)
            qh = q_raw[b, h * d:(h + 1) * d]
            qhat = qh / np.linalg.norm(qh)
            pos = _heavy_positions(spec, layer, b, h)
            heavy[b, h, :len(pos)] = pos
            K[b, h, pos] += (spec.gamma - 1.0) * rho * qhat
    return K, encode(V, spec.dtype), heavy


# ---------------------------------------------------------------- stage 2
def channel_scales(spec: Spec, layer: int, purpose: int) -> np.ndarray:
    """Per-(head, channel) log-normal scales exp(N(0,1)), shared over the batch."""
    if not spec.lognormal:
        return np.ones((spec.H, spec.d))
    return np.exp(_rng(spec, layer, purpose).standard_normal((spec.H, spec.d)))


def draw_cache_slice(spec: Spec, layer: int, b: int, h: int, qdir: np.ndarray,
                     rows: Optional[int] = None):
    """Skewed-frame K (float64, before encoding) and V (float32) of one (b, h), ``rows`` rows.

    K~[j, c] = s_c z_jc, heavy rows get (gamma-1) * rho_h * qhat added, rho_h = sqrt(sum_c s_c^2),
    qhat = qdir / |qdir| (the unit skewed query of that (b, h)).
    """
    d = spec.d
    rows = spec.n if rows is None else rows
    sk = channel_scales(spec, layer, _P_KSCALE)[h]
    sv = channel_scales(spec, layer, _P_VSCALE)[h]
    K = _rng(spec, layer, _P_K, b, h).standard_normal((rows, d), dtype=np.float32).astype(np.float64) * sk
    V = _rng(spec, layer, _P_V, b, h).standard_normal((rows, d), dtype=np.float32) * sv.astype(np.float32)
    pos = _heavy_positions(spec, layer, b, h)
    pos = pos[pos < rows]
    if len(pos):
        rho = math.sqrt(float(np.sum(sk * sk)))
        qhat = qdir / np.linalg.norm(qdir)
        K[pos] += (spec.gamma - 1.0) * rho * qhat
    return K, V, pos


def draw_cache(spec: Spec, layer: int, q_skewed: np.ndarray):
    """Skewed-frame caches for every (b, h).

    ``q_skewed`` is the skewed full query [B][H*d] (float64 values of its encoded bits), computed
    by whichever side runs the setup.  Returns K~ and V encoded as [B][H][n_cap][d] (rows >= n
    are zero) and the heavy positions.
    """
    B, H, d, n, cap = spec.B, spec.H, spec.d, spec.n, spec.cap
    enc = np.float32 if spec.dtype == "f32" else np.uint16
    Kb = np.zeros((B, H, cap, d), dtype=enc)
    Vb = np.zeros((B, H, cap, d), dtype=enc)
    heavy = np.zeros((B, H, max(spec.heavy, 0)), dtype=np.int64)

    def one(bh):
        b, h = divmod(bh, H)
        K, V, pos = draw_cache_slice(spec, layer, b, h, q_skewed[b, h * d:(h + 1) * d])
        Kb[b, h, :n] = encode(K.astype(np.float32), spec.dtype)
        Vb[b, h, :n] = encode(V, spec.dtype)
        heavy[b, h, :len(pos)] = pos

    # numpy's generators release the GIL while filling, so slices draw in parallel
    with cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(B * H)))
    return Kb, Vb, heavy


def draw_new_rows(spec: Spec, layer: int, step: int):
    """New token's skewed key and value rows [B][H][d] (non-heavy draws) for an append step."""
    B, H, d = spec.B, spec.H, spec.d
    g = _rng(spec, layer, _P_NEWKV, step)
    sk = channel_scales(spec, layer, _P_KSCALE)
    sv = channel_scales(spec, layer, _P_VSCALE)
    K = g.standard_normal((B, H, d), dtype=np.float32) * sk.astype(np.float32)[None]
    V = g.standard_normal((B, H, d), dtype=np.float32) * sv.astype(np.float32)[None]
    return encode(K, spec.dtype), encode(V, spec.dtype)


def draw_counters(spec: Spec, cmax: int, layer: int = 0) -> np.ndarray:
    """Access counters [B][n_cap] uint32, uniform in [0, cmax) for the first n slots, 0 beyond."""
    g = _rng(spec, layer, _P_CNT)
    c = np.zeros((spec.B, spec.cap), dtype=np.uint32)
    c[:, :spec.n] = g.integers(0, cmax, size=(spec.B, spec.n), dtype=np.uint32)
    return c


def draw_index_sets(spec: Spec, max_out: int, layer: int = 0):
    """Random ascending distinct row-index sets per (b, h) with random counts in [0, max_out]."""
    g = _rng(spec, layer, _P_IDX)
    idx = np.zeros((spec.B, spec.H, max_out), dtype=np.int32)
    cnt = np.zeros((spec.B, spec.H), dtype=np.int32)
    for b in range(spec.B):
        for h in range(spec.H):
            c = int(g.integers(0, min(max_out, spec.n) + 1))
            sel = np.sort(g.choice(spec.n, size=c, replace=False))
            idx[b, h, :c] = sel
            cnt[b, h] = c
    return idx, cnt


def drift(spec: Spec, x_bits: np.ndarray, layer: int, std: float, purpose_key: int = 0) -> np.ndarray:
    """Residual-stream stand-in for the next layer's input: x + N(0, std^2), re-encoded."""
    g = _rng(spec, layer, _P_DRIFT, purpose_key)
    x = values(x_bits, spec.dtype) + g.standard_normal(x_bits.shape) * std
    return encode(x.astype(np.float32), spec.dtype)


# ---------------------------------------------------------------- multi-layer decode pipeline
PIPE_LAYER_STD = 0.395   # x_{l+1} = x_l + N(0, 0.395^2): cosine ~0.93 between consecutive layer inputs
PIPE_STEP_STD = 0.14     # x_0(t) = x_0(t-1) + N(0, 0.14^2): cosine ~0.99 between consecutive steps


def pipeline_x(spec: Spec, layers: int, steps: int) -> np.ndarray:
    """Attention inputs x_l(t) [steps][layers][B][D] (stored dtype) of a decode pipeline.

    Stand-in for the residual stream: the first layer's input drifts slowly from step to step and
    each layer adds an independent perturbation to the previous layer's input, so consecutive layers
    see similar inputs (the summary's Table 1 reports cosine 0.89-0.97 between consecutive block
    inputs; 0.395 per layer gives about 0.93 for unit-variance channels)."""
    out = np.empty((steps, layers, spec.B, spec.D), dtype=np.float32 if spec.dtype == "f32" else np.uint16)
    x0 = draw_x(spec, 0)
    for t in range(steps):
        if t > 0:
            x0 = drift(spec, x0, 0, PIPE_STEP_STD, purpose_key=100000 + t)
        out[t, 0] = x0
        for l in range(1, layers):
            out[t, l] = drift(spec, out[t, l - 1], l, PIPE_LAYER_STD, purpose_key=t)
    return out

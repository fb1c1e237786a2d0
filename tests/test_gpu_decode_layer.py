"""GPU: ig_decode_layer (layer l's attention beside the speculation for layer l+1, one fused launch).

The InfiniGen summary (arXiv 2406.19707, paper-graph-ui, section 3.2 "Big-Picture Architecture")
runs the speculation for the next layer while the current layer computes.  The fused call must give
what the two separate calls give:
  speculation half   idx, count, counters, q_part bit-exact against ig_speculate on a copy of the layer
                     (same arithmetic per row; only the number of rows in flight differs), and against
                     the oracle on its own inputs (q_part within 1e-3, every head's set outside the
                     1e-4 band, counters slot by slot);
  attention half     within 1e-5 relative of ig_sparse_decode_attn on a copy (the lane groups
                     associate the float sums differently), and within the bf16/f32 attention tolerance
                     of the oracle on the selected rows.
Covered: the fused shapes (bf16 and f32, more than 16 batch rows), the benchmark's OPT-6.7B shape, an
attention with two K/V rows per lane group in flight (256 items of 218 rows), an attention split into
several workgroups with the combine, a shape outside the fused set (two launches), either half alone,
and the aliasing check.
"""

import numpy as np
import pytest

from oracle import oracle as O
from sparse_attention_ig_amd import gen
from tests import harness
from tests.gpu_util import DeviceLayer, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_ig_amd import _lib as L
    L.load()
    yield


def _spec(base: gen.Spec, **kw) -> gen.Spec:
    return gen.Spec(**{**base.__dict__, **kw})


CASES = [
    # name, attention-layer spec, speculation-layer spec, step kwargs
    ("bf16-topk", lambda: _spec(gen.opt_6_7b(n=1500, B=2), H=3, topk=100),
     lambda: _spec(gen.opt_6_7b(n=1800, B=2), H=3, topk=100, seed=2002), dict(mode="topk", k=100, max_out=100)),
    ("bf16-split-threshold", lambda: _spec(gen.opt_6_7b(n=6000, B=1), H=3),
     lambda: _spec(gen.opt_6_7b(n=6000, B=1), H=3, seed=2003),
     dict(mode="threshold", alpha=5.0, max_sel=1200, max_out=1200)),
    ("f32-tiny", lambda: gen.tiny_fp32(), lambda: _spec(gen.tiny_fp32(), seed=2004), dict(mode="topk", k=32, max_out=32)),
    ("bf16-head64-fallback", lambda: _spec(gen.opt_6_7b(n=700, B=2), H=4, d=32, r=8),
     lambda: _spec(gen.opt_6_7b(n=700, B=2), H=4, d=32, r=8, seed=2005), dict(mode="topk", k=40, max_out=40)),
    ("opt6.7b-full", lambda: gen.opt_6_7b(), lambda: _spec(gen.opt_6_7b(), seed=2006),
     dict(mode="topk", k=128, max_out=128)),
    # more than 16 batch rows (two 16-row blocks in the projection workgroups) and r = 16 (a 32-column
    # block spans two heads)
    ("bf16-batch20-r16", lambda: _spec(gen.opt_6_7b(n=600, B=20), H=3, r=16, heavy=12, topk=50),
     lambda: _spec(gen.opt_6_7b(n=640, B=20), H=3, r=16, heavy=12, topk=50, seed=2007),
     dict(mode="topk", k=50, max_out=50)),
    # 256 (b, h) items of 218 rows (the Llama-2-13B 5% budget): the attention role keeps two K/V rows
    # per lane group in flight
    ("bf16-rows2-218", lambda: _spec(gen.opt_6_7b(n=4352, B=8), topk=218),
     lambda: _spec(gen.opt_6_7b(n=4352, B=8), topk=218, seed=2008), dict(mode="topk", k=218, max_out=218)),
    # a long speculated row cut into 16 slices of 2500 rows (tight top-k candidates, a merge launch),
    # its slice workgroups before the attention items in the one launch
    ("bf16-sliced-topk", lambda: _spec(gen.opt_6_7b(n=3000, B=1), H=4, topk=400),
     lambda: _spec(gen.llama2_7b_long(n=40000, B=1), H=4, topk=400, seed=2009), dict(mode="topk", k=400, max_out=400)),
    # the head average (every head of a sequence takes the mean threshold count): whole rows hand on
    # candidates, a merge launch after the fused one averages and selects
    ("bf16-headavg", lambda: _spec(gen.opt_6_7b(n=1500, B=2), H=3, topk=100),
     lambda: _spec(gen.opt_6_7b(n=1800, B=2), H=3, seed=2011), dict(mode="headavg", alpha=5.0, max_sel=300, max_out=300)),
    # 128 rows of 65536 keys, top 2048: slices of 8192, counters from the merge's bitmaps
    ("bf16-sliced-bitmaps", lambda: _spec(gen.opt_6_7b(n=4000, B=4), topk=2048),
     lambda: _spec(gen.llama2_7b_long(n=65536, B=4), topk=2048, seed=2010), dict(mode="topk", k=2048, max_out=2048)),
]


def _layers(spec_fn, step_kw):
    spec = spec_fn()
    li = harness.lib_inputs(spec)
    a = DeviceLayer(li, max_out=step_kw["max_out"])
    return spec, li, a, a.clone()


@pytest.mark.parametrize("name,attn_fn,spec_fn,kw", CASES, ids=[c[0] for c in CASES])
def test_decode_layer_matches_separate_calls(name, attn_fn, spec_fn, kw):
    from sparse_attention_ig_amd.runtime import decode_layer
    sa, li_a, A, A2 = _layers(attn_fn, kw)
    sb, li_b, Bl, B2 = _layers(spec_fn, kw)
    say(f"[decode layer {name}] attn B{sa.B} H{sa.H} d{sa.d} n{sa.n}; spec r{sb.r} n{sb.n} {sb.dtype} {kw}")
    # layer l's own selection first (identical on both copies)
    for layer in (A, A2):
        layer.step(**kw, parts=("speculate",))
    # separate calls on the copies, the fused call on the originals
    A2.step(**kw, parts=("attn",))
    B2.step(**kw, parts=("speculate",))
    decode_layer(A, Bl, kw)
    g_a = to_host(dict(out=A.out, lse=A.lse, idx=A.idx, count=A.count))
    r_a = to_host(dict(out=A2.out, lse=A2.lse))
    g_b = to_host(dict(idx=Bl.idx, count=Bl.count, counters=Bl.counters, q_part=Bl.q_part))
    r_b = to_host(dict(idx=B2.idx, count=B2.count, counters=B2.counters, q_part=B2.q_part))
    say(f"[decode layer {name}] gpu done")

    # speculation half: bit-exact against ig_speculate
    assert np.array_equal(g_b["count"], r_b["count"])
    for b in range(sb.B):
        for h in range(sb.H):
            c = r_b["count"][b, h]
            assert np.array_equal(g_b["idx"][b, h, :c], r_b["idx"][b, h, :c]), (b, h)
    assert np.array_equal(g_b["counters"], r_b["counters"])
    assert np.array_equal(g_b["q_part"].view(np.uint32), r_b["q_part"].view(np.uint32))
    # ... and against the oracle on its own inputs: q_part, every head's set, the counters slot by slot
    oi_b = harness.oracle_inputs(sb)
    harness.assert_setup_routes_agree(li_b, oi_b)
    mode = kw["mode"]
    if mode == "headavg":
        # the average couples a sequence's heads: the oracle runs the whole layer-step
        full = harness.oracle_step(oi_b, mode=mode, alpha=kw["alpha"], max_sel=kw.get("max_sel", 0),
                                   max_out=kw["max_out"], counters=np.zeros((sb.B, sb.cap), np.uint32))
        ri, rc = full["idx"], full["count"]
        ref = {(b, h): dict(q_part=full["q_part"][b, h], scores=full["scores"][b, h],
                            idx=ri[b, h, :rc[b, h]].astype(np.int64))
               for b in range(sb.B) for h in range(sb.H)}
        assert np.array_equal(g_b["count"], rc), (g_b["count"], rc)
    else:
        ref, ri, rc = harness.oracle_heads(oi_b, mode=mode, alpha=kw.get("alpha", np.inf), k=kw.get("k", 0),
                                           max_sel=kw.get("max_sel", 0), max_out=kw["max_out"], attn=False)
    inexact = harness.check_heads(g_b["idx"], g_b["count"], ref, mode, kw.get("alpha", np.inf),
                                  g_q_part=g_b["q_part"])
    assert len(inexact) <= max(1, sb.B * sb.H // 50), inexact
    rC, _ = O.pool_touch(np.zeros((sb.B, sb.cap), np.uint32), ri, rc, sb.n, 65535)
    harness.check_counters(g_b["counters"].view(np.uint32), rC, g_b["idx"], g_b["count"], ri, rc, sb.n)

    # attention half: against ig_sparse_decode_attn and against the oracle on the selected rows
    scale = np.abs(r_a["out"]).max(axis=-1, keepdims=True) + 1e-30
    assert (np.abs(g_a["out"] - r_a["out"]) / scale).max() <= 1e-5
    assert np.abs(g_a["lse"] - r_a["lse"]).max() <= 1e-5 * max(1.0, np.abs(r_a["lse"]).max())
    tol = harness.ATTN_TOL[sa.dtype]
    q = O.decode(li_a.q, sa.dtype)
    K, V = O.decode(li_a.K, sa.dtype), O.decode(li_a.V, sa.dtype)
    for b in range(sa.B):
        for h in range(sa.H):
            rows = g_a["idx"][b, h, :g_a["count"][b, h]].astype(np.int64)
            o, lse = O.attention_rows(q[b, h], K[b, h, rows], V[b, h, rows], sa.softmax_scale)
            assert np.abs(g_a["out"][b, h] - o).max() <= tol, (b, h)
            assert abs(g_a["lse"][b, h] - lse) <= max(tol, 1e-5 * abs(lse)), (b, h)


def test_decode_layer_single_halves_and_aliasing():
    """attn alone is ig_sparse_decode_attn, spec alone is ig_speculate; aliased outputs are rejected."""
    from sparse_attention_ig_amd import _lib as L
    from sparse_attention_ig_amd.runtime import attn_call, spec_call
    kw = dict(mode="topk", k=64, max_out=64)
    spec = _spec(gen.opt_6_7b(n=900, B=2), H=3, topk=64)
    A = DeviceLayer(harness.lib_inputs(spec), max_out=64)
    A2 = A.clone()
    for layer in (A, A2):
        layer.step(**kw, parts=("speculate",))
    L.ig_decode_layer(attn_call(A), None)
    A2.step(**kw, parts=("attn",))
    g, r = to_host(dict(out=A.out, lse=A.lse)), to_host(dict(out=A2.out, lse=A2.lse))
    assert np.array_equal(g["out"].view(np.uint32), r["out"].view(np.uint32))   # the same kernel
    S = A.clone()
    L.ig_decode_layer(None, spec_call(S, mode="topk", k=64, max_out=64))
    S2 = A.clone()
    S2.step(**kw, parts=("speculate",))
    gs, rs = to_host(dict(idx=S.idx, count=S.count)), to_host(dict(idx=S2.idx, count=S2.count))
    assert np.array_equal(gs["count"], rs["count"])
    # the speculation may not write the index list the attention reads
    with pytest.raises(RuntimeError, match="must not be the attention's"):
        L.ig_decode_layer(attn_call(A), spec_call(A, mode="topk", k=64, max_out=64))


def test_sliced_merge_recomputes_concentrated_rows():
    """Tight top-k candidates: each slice hands on about its share of the row's top k.  With every heavy
    key of a row inside its first slice, that slice holds far more of the top k than it hands on, so
    the merge finds fewer than k candidates at or above the slices' largest bound and recomputes the
    row's scores from its partial keys.  The selection must still be the oracle's and the counters
    exact, and the workspace counts the rows recomputed."""
    from sparse_attention_ig_amd import _lib as L
    kw = dict(mode="topk", k=400, max_out=400)
    spec_fn = lambda: _spec(gen.llama2_7b_long(n=40000, B=1), H=4, topk=400, heavy=400, heavy_span=2400,
                            gamma=6.0, seed=2012)
    sb, li_b, Bl, _ = _layers(spec_fn, kw)
    say(f"[sliced recompute] B{sb.B} H{sb.H} n{sb.n} {kw}")
    Bl.step(**kw, parts=("speculate",))
    st, rec = L.ig_workspace_status(Bl.ws_spec, recomputed=True)
    say(f"[sliced recompute] status {st}, rows recomputed {rec}")
    assert st == 0
    assert rec == sb.B * sb.H, "every row's heavy keys sit in one slice: every merge must recompute"
    g = to_host(dict(idx=Bl.idx, count=Bl.count, counters=Bl.counters, q_part=Bl.q_part))
    oi = harness.oracle_inputs(sb)
    ref, ri, rc = harness.oracle_heads(oi, mode="topk", alpha=np.inf, k=kw["k"], max_sel=0,
                                       max_out=kw["max_out"], attn=False)
    inexact = harness.check_heads(g["idx"], g["count"], ref, "topk", np.inf, g_q_part=g["q_part"])
    assert len(inexact) <= max(1, sb.B * sb.H // 50), inexact
    rC, _ = O.pool_touch(np.zeros((sb.B, sb.cap), np.uint32), ri, rc, sb.n, 65535)
    harness.check_counters(g["counters"].view(np.uint32), rC, g["idx"], g["count"], ri, rc, sb.n)

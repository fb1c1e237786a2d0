"""GPU parity at the full sizes the benchmarks time, on every (b, h) head (the oracle computes each head
on its own, decoding only that head's rows):

  * the 40-layer Llama-2-13B pipeline's layer pair (B16 H40 d128 D5120 r32, n = 4096, top 5%): layer 0
    dense attention, layer 0's ig_decode_layer (the projection and speculation for layer 1 beside
    layer 0's attention, one launch), layer 1's attention over the speculated rows, layer 1's counters;
  * the OPT-30B pinned host pool (B16 H56 d128 D7168 r32, alpha 5, 20% cap, 4096 slots), with bf16
    rows and with INT4 records, at the sampled layers {0, 1, 24, 47} and the sampled steps of the growth
    from 2048 to 4096 rows {first, middle, last} = n in {2048, 3072, 4096} (the first n rows of one
    4096-row draw per layer; counters accumulate over the three steps): speculation in HBM, zero-copy
    gather, attention;
  * the long-context Llama-2-7B layer at its largest size (B4, n = 131072, top 4%, the benchmark's
    workload): the fused speculation, and ig_decode_layer as the benchmark calls it (the speculation's
    slices beside the attention of the layer before, in one launch).

Selections must match outside the 1e-4 band; attention within 1e-2 (bf16) where the sets are equal;
counters slot by slot (only slots of band-differing heads may move, by at most that many).
"""
import math

import numpy as np
import pytest

from oracle import oracle as O
from sparse_attention_ig_amd import gen
from tests import harness
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_ig_amd import _lib as L
    L.load()
    yield


def test_pipeline_layer_pair_full_size():
    import torch
    from sparse_attention_ig_amd.pipeline import DecodePipeline
    from sparse_attention_ig_amd.runtime import to_device
    spec = gen.llama2_13b(n=4096, B=16, n_cap=4352)
    max_out = int(math.ceil(0.05 * spec.cap))
    say(f"[full pipeline] B={spec.B} H={spec.H} n={spec.n} 2 layers")
    xs, lib_in, _ = harness.pipeline_setup(spec, 2, 1, harness.lib_inputs)
    _, ora_in, _ = harness.pipeline_setup(spec, 2, 1, harness.oracle_inputs)
    for a, b in zip(lib_in, ora_in):
        harness.assert_setup_routes_agree(a, b)
    pipe = DecodePipeline(lib_in, max_out=max_out)
    k = pipe.topk()
    pipe.step([to_device(xs[0, l]) for l in range(2)], append=False)
    torch.cuda.synchronize()
    say("[full pipeline] gpu step done")
    out0, out1 = host(pipe.layers[0].out), host(pipe.layers[1].out)
    gi, gc = host(pipe.layers[1].idx), host(pipe.layers[1].count)
    gC = host(pipe.layers[1].counters).view(np.uint32)
    dt = spec.dtype
    tol = harness.ATTN_TOL[dt]
    L0 = ora_in[0]
    for b in range(spec.B):
        for h in range(spec.H):
            o, _ = O.attention_rows(O.decode(L0.q[b, h], dt), O.decode(L0.K[b, h, :spec.n], dt),
                                    O.decode(L0.V[b, h, :spec.n], dt), spec.softmax_scale)
            assert np.abs(out0[b, h] - o).max() <= tol, ("layer 0", b, h)
    say("[full pipeline] layer 0 dense attention: every head within tolerance")
    ref, ri, rc = harness.oracle_heads(ora_in[1], mode="topk", k=k, max_out=max_out, x_bits=xs[0, 0])
    inexact = harness.check_heads(gi, gc, ref, "topk", 0.0, g_out=out1, tol=tol)
    assert len(inexact) <= spec.B * spec.H // 50, inexact
    rC, _ = O.pool_touch(np.zeros((spec.B, spec.cap), np.uint32), ri, rc, spec.n, 65535)
    moved = harness.check_counters(gC, rC, gi, gc, ri, rc, spec.n)
    say(f"[full pipeline] layer 1: {spec.B * spec.H} heads checked, {len(inexact)} band-affected, "
        f"counters moved in {len(moved)} sequences")


@pytest.mark.parametrize("layer", [0, 1, 24, 47])
def test_pool_full_size_sampled_layers_and_steps(layer):
    import torch
    from sparse_attention_ig_amd.runtime import PoolLayer
    spec = gen.opt_30b(n=4096, B=16, n_cap=4096)
    say(f"[full pool layer {layer}] B={spec.B} H={spec.H} cap={spec.cap}: setup")
    lay = gen.draw_layer(spec, layer, with_wk=False)
    li, oi = harness.lib_inputs(spec, layer, lay=lay), harness.oracle_inputs(spec, layer, lay=lay)
    harness.assert_setup_routes_agree(li, oi)
    max_out = spec.max_sel                    # 20% of the largest n
    pools = {"bf16": PoolLayer(li, max_out=max_out), "int4": PoolLayer(li, max_out=max_out, int4=True)}
    dt = spec.dtype
    tol = harness.ATTN_TOL[dt]
    rC = np.zeros((spec.B, spec.cap), np.uint32)
    diverged = set()
    for n in (2048, 3072, 4096):
        max_sel = max(1, int(math.floor(0.2 * n)))
        for kind, pool in pools.items():
            pool.speculate(alpha=spec.alpha, max_sel=max_sel, n=n, want_victim=True)
            pool.gather()
            pool.attend()
        torch.cuda.synchronize()
        say(f"[full pool layer {layer}] n={n} gpu done")
        ref, ri, rc = harness.oracle_heads(oi, mode="threshold", alpha=spec.alpha, max_sel=max_sel, max_out=max_out,
                                           n=n, attn=False)
        rC, rv = O.pool_touch(rC, ri, rc, n, 65535, want_victim=True)
        for kind, pool in pools.items():
            gi, gc, out = host(pool.idx), host(pool.count), host(pool.out)
            inexact = harness.check_heads(gi, gc, ref, "threshold", spec.alpha)
            assert len(inexact) <= spec.B * spec.H // 50, (kind, inexact)
            for (b, h), r in ref.items():
                if (b, h) in inexact:
                    continue
                rows = r["idx"]
                K, V = oi.K[b, h, rows], oi.V[b, h, rows]
                if kind == "int4":
                    K = O.store(O.dequantize_int4(*O.quantize_int4(K, dt)), dt)
                    V = O.store(O.dequantize_int4(*O.quantize_int4(V, dt)), dt)
                o, _ = O.attention_rows(O.decode(oi.q[b, h], dt), O.decode(K, dt), O.decode(V, dt),
                                        spec.softmax_scale)
                assert np.abs(out[b, h] - o).max() <= tol, (kind, n, b, h)
            gC = host(pool.counters).view(np.uint32)
            keep = [b for b in range(spec.B) if b not in diverged]
            moved = harness.check_counters(gC[keep], rC[keep], gi[keep], gc[keep], ri[keep], rc[keep], n,
                                           host(pool.victim)[keep], rv[keep])
            diverged.update(keep[i] for i in moved)
            say(f"[full pool layer {layer}] n={n} {kind}: {spec.B * spec.H} heads, {len(inexact)} band-affected, "
                f"mean count {gc.mean():.1f}")
    assert len(diverged) <= 2, diverged


def test_long_context_b4_full_size():
    """Llama-2-7B-shaped layer at 131072 rows, batch 4, top 4% (5243 rows per head), the fused path:
    the projection workgroups, 16 slices of 8192 rows per row handing on tight candidates, a merge per
    row, counters from the rows' bitmaps; then the attention split over the selected rows.  Every head
    against the oracle, counters slot by slot."""
    from sparse_attention_ig_amd.runtime import DeviceLayer
    from tests.gpu_util import to_host
    spec = gen.llama2_7b_long(n=131072, B=4, frac=0.04)
    say(f"[long b4 full] n={spec.n} k={spec.topk}")
    li, oi = harness.lib_inputs(spec), harness.oracle_inputs(spec)
    harness.assert_setup_routes_agree(li, oi)
    layer = DeviceLayer(li, max_out=spec.topk)
    g = to_host(layer.step(mode="topk", k=spec.topk, max_out=spec.topk, want_victim=True, parts=DeviceLayer.FUSED))
    say("[long b4 full] gpu step done")
    ref, ri, rc = harness.oracle_heads(oi, mode="topk", k=spec.topk, max_out=spec.topk)
    inexact = harness.check_heads(g["idx"], g["count"], ref, "topk", 0.0, g_q_part=g["q_part"], g_scores=g["scores"],
                                  g_out=g["out"], g_lse=g["lse"], tol=harness.ATTN_TOL["bf16"])
    assert len(inexact) <= 3, inexact
    assert (g["count"] == spec.topk).all()
    rC, rv = O.pool_touch(np.zeros((spec.B, spec.cap), np.uint32), ri, rc, spec.n, 65535, want_victim=True)
    moved = harness.check_counters(g["counters"], rC, g["idx"], g["count"], ri, rc, spec.n, g["victim"], rv)
    say(f"[long b4 full] {spec.B * spec.H} heads, {len(inexact)} band-affected, counters moved in {len(moved)}")


def test_long_context_b4_decode_layer_full_size():
    """ig_decode_layer at the benchmark's workload (B4, n = 131072, top 4%): the attention of a layer
    over its own speculated rows beside the speculation of a copy of it (16 slices of 8192 rows per row,
    then the attention items, in one launch; a merge and the bitmap counter kernels after).  Every head of
    both halves against the oracle (one layer's draws serve both: a copy has the same caches)."""
    import torch
    from sparse_attention_ig_amd.runtime import DeviceLayer, decode_layer
    from tests.gpu_util import to_host
    spec = gen.llama2_7b_long(n=131072, B=4, frac=0.04)
    kw = dict(mode="topk", k=spec.topk, max_out=spec.topk)
    say(f"[long b4 decode layer] n={spec.n} k={spec.topk}")
    li, oi = harness.lib_inputs(spec), harness.oracle_inputs(spec)
    harness.assert_setup_routes_agree(li, oi)
    A = DeviceLayer(li, max_out=spec.topk)
    del li
    A.keep_scores = False
    A.step(**kw, parts=("speculate",))          # layer l's own selection, which its attention reads
    S = A.clone()
    S.counters.zero_()
    S.idx.fill_(-1)
    decode_layer(A, S, kw)
    torch.cuda.synchronize()
    say("[long b4 decode layer] gpu step done")
    from sparse_attention_ig_amd import _lib as L
    assert L.ig_workspace_status(S.ws_spec) == 0
    ga = to_host(dict(idx=A.idx, count=A.count, out=A.out, lse=A.lse))
    gs = to_host(dict(idx=S.idx, count=S.count, counters=S.counters, q_part=S.q_part))
    ref, ri, rc = harness.oracle_heads(oi, mode="topk", k=spec.topk, max_out=spec.topk)
    # the speculation half: every head's set, q_part, counters slot by slot
    inexact = harness.check_heads(gs["idx"], gs["count"], ref, "topk", 0.0, g_q_part=gs["q_part"])
    assert len(inexact) <= 3, inexact
    rC, _ = O.pool_touch(np.zeros((spec.B, spec.cap), np.uint32), ri, rc, spec.n, 65535)
    harness.check_counters(gs["counters"].view(np.uint32), rC, gs["idx"], gs["count"], ri, rc, spec.n)
    # the attention half, over layer l's own selection (the same rule on the same layer)
    inexact_a = harness.check_heads(ga["idx"], ga["count"], ref, "topk", 0.0, g_out=ga["out"], g_lse=ga["lse"],
                                    tol=harness.ATTN_TOL["bf16"])
    assert len(inexact_a) <= 3, inexact_a
    say(f"[long b4 decode layer] {spec.B * spec.H} heads per half, band-affected {len(inexact)} / {len(inexact_a)}")

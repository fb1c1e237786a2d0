"""GPU parity at the full sizes the benchmarks time, on sampled heads (the oracle computes those heads
one by one on its own inputs):

  * the 40-layer Llama-2-13B pipeline's layer pair (B16 H40 d128 D5120 r32, n = 4096, top 5%): layer 0
    dense attention, layer 0's ig_decode_layer (the projection and speculation for layer 1 beside
    layer 0's attention, one launch), layer 1's attention over the speculated rows;
  * the OPT-30B pinned host pool (B16 H56 d128 D7168 r32, n = 2048 of 4096 slots, alpha 5, 20% cap),
    with bf16 rows and with INT4 records: speculation in HBM, zero-copy gather, attention;
  * the long-context Llama-2-7B layer at its largest benchmark size (B4, n = 131072, top 4%).

Selections must match outside the 1e-4 band; attention within 1e-2 (bf16) where the sets are equal.
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


def _spec_head(ins, x_bits, b, h, n, mode, **kw):
    """Oracle speculation for head (b, h) of the layer `ins` from the attention input x_bits[b]."""
    s = ins.spec
    dt = s.dtype
    Wp = O.decode(ins.Wq_part, dt)[:, h * s.r:(h + 1) * s.r]
    Kp = O.decode(ins.extra["Kp"][b:b + 1, h:h + 1], dt)
    _, sc = O.rehearse(O.decode(x_bits[b:b + 1], dt), Wp, Kp, n, 1, s.r, s.softmax_scale)
    idx, cnt = O.select(sc, mode, **kw)
    return sc[0, 0], idx[0, 0, :cnt[0, 0]].astype(np.int64)


def test_pipeline_layer_pair_full_size_sampled():
    import torch
    from sparse_attention_ig_amd.pipeline import DecodePipeline
    from sparse_attention_ig_amd.runtime import to_device
    spec = gen.llama2_13b(n=4096, B=16, n_cap=4352)
    max_out = int(math.ceil(0.05 * spec.cap))
    say(f"[full pipeline] B={spec.B} H={spec.H} n={spec.n} 2 layers")
    xs, lib_in, _ = harness.pipeline_setup(spec, 2, 1, harness.lib_inputs)
    _, ora_in, _ = harness.pipeline_setup(spec, 2, 1, harness.oracle_inputs)
    for a, b in zip(lib_in, ora_in):
        assert harness.compare_inputs(a, b)["chan"] == 0
    pipe = DecodePipeline(lib_in, max_out=max_out)
    k = pipe.topk()
    pipe.step([to_device(xs[0, l]) for l in range(2)], append=False)
    torch.cuda.synchronize()
    say("[full pipeline] gpu step done")
    out0, out1 = host(pipe.layers[0].out), host(pipe.layers[1].out)
    gi, gc = host(pipe.layers[1].idx), host(pipe.layers[1].count)
    dt = spec.dtype
    tol = harness.ATTN_TOL[dt]
    exact_heads = 0
    for (b, h) in [(0, 0), (7, 13), (15, 39)]:
        L0 = ora_in[0]
        o, _ = O.attention_rows(O.decode(L0.q[b, h], dt), O.decode(L0.K[b, h, :spec.n], dt),
                                O.decode(L0.V[b, h, :spec.n], dt), spec.softmax_scale)
        assert np.abs(out0[b, h] - o).max() <= tol, ("layer 0", b, h)
        sc, rows = _spec_head(ora_in[1], xs[0, 0], b, h, spec.n, "topk", k=k, max_out=max_out)
        ok, exact, _ = harness.compare_sets(gi[b, h, :gc[b, h]], rows, sc, "topk", 0.0)
        assert ok and gc[b, h] == len(rows), ("layer 1 set", b, h)
        if exact:
            exact_heads += 1
            L1 = ora_in[1]
            o, _ = O.attention_rows(O.decode(L1.q[b, h], dt), O.decode(L1.K[b, h, rows], dt),
                                    O.decode(L1.V[b, h, rows], dt), spec.softmax_scale)
            assert np.abs(out1[b, h] - o).max() <= tol, ("layer 1", b, h)
    assert exact_heads >= 1


@pytest.mark.parametrize("int4", [False, True], ids=["bf16-rows", "int4-records"])
def test_pool_full_size_sampled(int4):
    import torch
    from sparse_attention_ig_amd.runtime import PoolLayer
    spec = gen.opt_30b(n=2048, B=16, n_cap=4096)
    say(f"[full pool int4={int4}] B={spec.B} H={spec.H} n={spec.n} cap={spec.cap}")
    li, oi = harness.lib_inputs(spec), harness.oracle_inputs(spec)
    assert harness.compare_inputs(li, oi)["chan"] == 0
    lay = PoolLayer(li, max_out=spec.max_sel, int4=int4)
    lay.speculate(alpha=spec.alpha, max_sel=spec.max_sel)
    lay.gather()
    lay.attend()
    torch.cuda.synchronize()
    say("[full pool] gpu step done")
    gi, gc, out = host(lay.idx), host(lay.count), host(lay.out)
    dt = spec.dtype
    exact_heads = 0
    for (b, h) in [(0, 0), (9, 27), (15, 55)]:
        sc, rows = _spec_head(oi, oi.x, b, h, spec.n, "threshold", alpha=spec.alpha, max_sel=spec.max_sel,
                              max_out=spec.max_sel)
        ok, exact, _ = harness.compare_sets(gi[b, h, :gc[b, h]], rows, sc, "threshold", spec.alpha)
        assert ok, (b, h)
        if not exact:
            continue
        exact_heads += 1
        K, V = oi.K[b, h, rows], oi.V[b, h, rows]
        if int4:
            K = O.store(O.dequantize_int4(*O.quantize_int4(K, dt)), dt)
            V = O.store(O.dequantize_int4(*O.quantize_int4(V, dt)), dt)
        o, _ = O.attention_rows(O.decode(oi.q[b, h], dt), O.decode(K, dt), O.decode(V, dt), spec.softmax_scale)
        assert np.abs(out[b, h] - o).max() <= harness.ATTN_TOL[dt], (b, h)
    assert exact_heads >= 1


def test_long_context_b4_full_size_sampled():
    """Llama-2-7B-shaped layer at 131072 rows, batch 4, top 4% (5243 rows per head), the fused path:
    the projection workgroups, 4 slices of 32768 rows per row, a merge of 20972 candidates per row; then the
    attention split over the selected rows.  Sampled heads against the oracle, every head's counters."""
    from sparse_attention_ig_amd.runtime import DeviceLayer
    from tests.gpu_util import to_host
    spec = gen.llama2_7b_long(n=131072, B=4, frac=0.04)
    say(f"[long b4 full] n={spec.n} k={spec.topk}")
    li, oi = harness.lib_inputs(spec), harness.oracle_inputs(spec)
    assert harness.compare_inputs(li, oi)["chan"] == 0
    layer = DeviceLayer(li, max_out=spec.topk)
    g = to_host(layer.step(mode="topk", k=spec.topk, max_out=spec.topk, parts=DeviceLayer.FUSED))
    say("[long b4 full] gpu step done")
    heads = [(0, 0), (1, 17), (3, 31)]
    ref = harness.oracle_step(oi, mode="topk", k=spec.topk, max_out=spec.topk, heads=heads)
    exact_heads = 0
    for (b, h), r in ref.items():
        assert harness.score_error(g["scores"][b, h, :spec.n], r["scores"]) <= harness.SCORE_RTOL
        ok, exact, _ = harness.compare_sets(g["idx"][b, h, :g["count"][b, h]], r["idx"], r["scores"], "topk", 0.0)
        assert ok and g["count"][b, h] == len(r["idx"]), (b, h)
        if exact:
            exact_heads += 1
            assert np.abs(g["out"][b, h] - r["out"]).max() <= harness.ATTN_TOL["bf16"], (b, h)
    assert exact_heads >= 1
    assert int(g["counters"].sum()) == spec.B * spec.H * spec.topk

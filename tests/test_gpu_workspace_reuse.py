"""Speculation workspaces reused across calls, as the ABI allows: calls on one workspace agree on B,
H, D and r while n, max_out and the mode change (whole rows, sliced rows whose slices all read each
row's partial query, the fused decode layer); a call of another (B, H, D, r) follows
ig_workspace_init.  Every call must leave the workspace as it found it (the projection's partial-sum
slots empty, the arrival words at zero, the status word clear), so each
result equals, bit for bit, that of the same call on a fresh workspace."""
import numpy as np
import pytest

from sparse_attention_ig_amd import gen
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _spec(base, **kw):
    return gen.Spec(**{**base.__dict__, **kw})


def _outputs(layer, res):
    from tests.gpu_util import to_host
    return to_host(dict(count=res["count"], idx=res["idx"], counters=layer.counters, q_part=layer.q_part))


def _same(a, b, tag):
    assert np.array_equal(a["count"], b["count"]), tag
    B, H = a["count"].shape
    for bb in range(B):
        for hh in range(H):
            c = int(a["count"][bb, hh])
            assert np.array_equal(a["idx"][bb, hh, :c], b["idx"][bb, hh, :c]), (tag, bb, hh)
    assert np.array_equal(a["counters"].view(np.uint32), b["counters"].view(np.uint32)), tag
    assert np.array_equal(a["q_part"].view(np.uint32), b["q_part"].view(np.uint32)), tag


def _run(layer, kw, ws=None):
    run = layer.clone()
    run.keep_scores = False
    if ws is not None:
        run.ws_spec = ws
    return _outputs(run, run.step(**kw, parts=("speculate",)))


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_ig_amd import _lib as L
    L.load()
    return L


def test_whole_row_calls_of_different_shapes(lib):
    """Calls of one (B, H, D, r) share a workspace with no re-initialisation; a call of another shape
    needs ig_workspace_init first (the workspace is stamped with the shape of its first call), after
    which every result equals, bit for bit, the same call on a fresh workspace."""
    import torch
    from sparse_attention_ig_amd.runtime import DeviceLayer, decode_layer, prepare_layer
    specs = [_spec(gen.opt_6_7b(n=1500, B=4), H=8, topk=100),
             _spec(gen.opt_6_7b(n=600, B=20), H=3, r=16, heavy=12, topk=50)]  # two 16-row blocks
    layers = [DeviceLayer(prepare_layer(s), max_out=s.topk) for s in specs]
    kws = [dict(mode="topk", k=s.topk, max_out=s.topk) for s in specs]
    ref = [_run(l, kw) for l, kw in zip(layers, kws)]
    shared = lib.ig_workspace_init(torch.empty(max(int(l.ws_spec.numel()) for l in layers), dtype=torch.uint8,
                                               device="cuda"))
    prev = None
    for i in (0, 0, 1, 1, 1, 0, 1, 0, 0):
        if prev is not None and prev != i:
            lib.ig_workspace_init(shared)   # another (B, H, D, r): the stamp must be cleared first
        prev = i
        say(f"[shared workspace] ig_speculate B={specs[i].B} H={specs[i].H} r={specs[i].r} n={specs[i].n}")
        _same(_run(layers[i], kws[i], shared), ref[i], f"speculate {i}")
        assert lib.ig_workspace_status(shared) == 0
    say("[shared workspace] ig_decode_layer")
    attn = layers[0].clone()
    attn.keep_scores = False
    attn.step(**kws[0], parts=("speculate",))  # its own selection first: the attention reads idx and count
    spec = layers[0].clone()
    spec.keep_scores = False
    spec.ws_spec = shared
    decode_layer(attn, spec, kws[0])
    _same(_outputs(spec, dict(count=spec.count, idx=spec.idx)), ref[0], "decode layer")
    _same(_run(layers[0], kws[0], shared), ref[0], "speculate after the decode layer")
    assert lib.ig_workspace_status(shared) == 0


def test_sliced_rows_changing_n_and_mode(lib):
    """Sliced rows (several slice workgroups read each row's partial query), with n, max_out and the
    mode changing from call to call on one workspace."""
    from sparse_attention_ig_amd.runtime import DeviceLayer, prepare_layer
    spec = _spec(gen.llama2_7b_long(n=20000), H=2, topk=200)
    layer = DeviceLayer(prepare_layer(spec), max_out=4000)
    calls = [dict(mode="topk", k=200, max_out=200),
             dict(mode="threshold", alpha=5.0, max_sel=4000, max_out=4000, n=18000),
             dict(mode="topk", k=1000, max_out=1000, n=12000),
             dict(mode="topk", k=200, max_out=200)]
    ref = [_run(layer, kw) for kw in calls]
    shared = layer.ws_spec  # (zero: this layer has not run yet)
    for rep in range(2):
        for i, kw in enumerate(calls):
            say(f"[shared workspace] sliced rows, call {i} {kw}")
            _same(_run(layer, kw, shared), ref[i], f"sliced call {i} rep {rep}")
            assert lib.ig_workspace_status(shared) == 0


def test_bitmap_counters_changing_n(lib):
    """Sliced rows whose selections are large enough for the bitmap counter kernels (32 rows x 8192
    selected slots), with n changing from call to call on one workspace: the kernels' per-sequence
    saturation flags must start every call at zero, so they sit at a place that does not move with n
    (the bitmaps and candidates that do move hold nonzero words after a call)."""
    import torch
    from sparse_attention_ig_amd.runtime import DeviceLayer, prepare_layer
    spec = _spec(gen.llama2_7b_long(n=16384), topk=8192)
    layer = DeviceLayer(prepare_layer(spec), max_out=8192)
    calls = [dict(mode="topk", k=8192, max_out=8192),
             dict(mode="topk", k=8192, max_out=8192, n=12000),
             dict(mode="topk", k=6000, max_out=8192, n=14000),
             dict(mode="topk", k=8192, max_out=8192)]
    ref = [_run(layer, kw) for kw in calls]
    shared = layer.ws_spec
    B = spec.B
    for i, kw in enumerate(calls):
        say(f"[shared workspace] bitmap counters, call {i} {kw}")
        _same(_run(layer, kw, shared), ref[i], f"bitmap call {i}")
        assert lib.ig_workspace_status(shared) == 0
        torch.cuda.synchronize()
        words = shared[256:256 + 8 * B].cpu().numpy()
        assert not words.any(), f"per-sequence words must return to zero after call {i}"

"""GPU: ig_speculate_noalloc (the speculation with the library's static device scratch as its workspace,
for callers that cannot allocate) gives what ig_speculate gives on a fresh workspace, bit for bit, on
two calls in a row on one GPU, the second with a smaller input (the scratch keeps the first call's
contents; the second call must not see them).  The first call is a long row cut into slices whose merge
leaves bitmaps for the counter kernel (the largest use of the scratch here); the second has whole rows.
A call needing more than the scratch is rejected on the host."""
import numpy as np
import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_ig_amd import _lib as L
    L.load()
    return L


def _inputs(B, H, D, r, n, max_out, seed):
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    dv = "cuda"
    t = dict(x=torch.randn((B, D), generator=g, device=dv).to(torch.bfloat16),
             W=(torch.randn((H * r, D), generator=g, device=dv) / 64).to(torch.bfloat16),
             Kp=torch.randn((B, H, n, r), generator=g, device=dv).to(torch.bfloat16),
             C0=torch.randint(0, 50, (B, n), generator=g, device=dv, dtype=torch.int32))
    t.update(B=B, H=H, D=D, r=r, n=n, max_out=max_out)
    return t


def _outputs(t):
    import torch
    dv = "cuda"
    B, H, r, n = t["B"], t["H"], t["r"], t["n"]
    return dict(idx=torch.full((B, H, t["max_out"]), -5, dtype=torch.int32, device=dv),
                count=torch.full((B, H), -5, dtype=torch.int32, device=dv),
                counters=t["C0"].clone(), victim=torch.full((B,), -5, dtype=torch.int32, device=dv),
                q_part=torch.zeros((B, H, r), dtype=torch.float32, device=dv),
                scores=torch.zeros((B, H, n), dtype=torch.float32, device=dv))


def _call(L, t, o, kw, noalloc):
    fn = L.ig_speculate_noalloc if noalloc else L.ig_speculate
    fn(t["x"], t["W"], t["Kp"], t["n"], 0.125, kw["mode"], t["max_out"], alpha=kw.get("alpha", float("inf")),
       k=kw.get("k", 0), max_sel=kw.get("max_sel", 0), idx=o["idx"], count=o["count"], counters=o["counters"],
       victim=o["victim"], q_part=o["q_part"], scores=o["scores"])


def _host(o):
    from sparse_attention_ig_amd.runtime import to_host
    return {k: to_host(v).copy() for k, v in o.items()}


def _same(a, b, tag):
    assert np.array_equal(a["count"], b["count"]), tag
    assert (a["count"] >= 1).all(), tag
    B, H = a["count"].shape
    for bb in range(B):
        for hh in range(H):
            c = int(a["count"][bb, hh])
            assert np.array_equal(a["idx"][bb, hh, :c], b["idx"][bb, hh, :c]), (tag, bb, hh)
    for key in ("counters", "victim", "q_part", "scores"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (tag, key)


CALLS = [
    # 128 rows of 65536 keys, top 2048: two slices per row, candidates merged, counters from bitmaps
    (dict(B=4, H=32, D=4096, r=32, n=65536, max_out=2048), dict(mode="topk", k=2048)),
    # then a smaller call: 6 whole rows, threshold with the cap
    (dict(B=2, H=3, D=1024, r=32, n=1500, max_out=300), dict(mode="threshold", alpha=1.5, max_sel=300)),
]


def test_noalloc_matches_workspace_call_twice(lib):
    import torch
    L = lib
    for i, (shape, kw) in enumerate(CALLS):
        t = _inputs(**shape, seed=40 + i)
        nb = L.ig_workspace_size(L.IG_OP_SPECULATE, t["B"], t["H"], t["D"], 0, t["r"], t["n"], t["max_out"])
        assert 0 < nb <= L.IG_NOALLOC_SCRATCH_BYTES
        say(f"[noalloc call {i}] {shape} {kw}: workspace call ({nb} bytes)")
        ref = _outputs(t)
        _call(L, t, ref, kw, noalloc=False)
        say(f"[noalloc call {i}] static scratch call")
        got = _outputs(t)
        _call(L, t, got, kw, noalloc=True)
        torch.cuda.synchronize()
        _same(_host(got), _host(ref), f"call {i}")
        say(f"[noalloc call {i}] equal")


def test_noalloc_rejects_calls_beyond_the_scratch(lib):
    """A call whose workspace would exceed the static scratch returns IG_EINVAL before any launch."""
    import ctypes
    L = lib
    lib_ = L.load()
    B, H, D, r, n, max_out = 64, 32, 4096, 32, 131072, 20000
    need = L.ig_workspace_size(L.IG_OP_SPECULATE, B, H, D, 0, r, n, max_out)
    assert need > L.IG_NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    st = lib_.ig_speculate_noalloc(p, p, None, p, B, D, H, r, n, n, L.IG_BF16, ctypes.c_float(0.125), L.IG_SEL_TOPK,
                                   ctypes.c_float(0.0), max_out, 0, p, p, max_out, None, 15, None, None, None, n, None)
    assert st == L.IG_EINVAL and "static scratch" in L.ig_last_error()

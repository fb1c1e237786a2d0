"""GPU: failures of the speculation's in-launch hand-over are reported, never silent.

A row workgroup of ig_speculate (and of the speculation half of ig_decode_layer) waits for the partial
query that projection workgroups of the same launch store into the workspace.  Its wait is bounded;
when the bound is reached, or when the workspace was claimed for another (B, H, D, r), or when an
earlier call left a failure behind, the row writes count = -1, touches no counter, still arrives for
its sequence's finish, and the workspace's sticky status word says why (ig_workspace_status) until
ig_workspace_init clears it.

The failures are forced from the host so that every kernel still exits normally: the test mode makes
the projection workgroups withhold their partial sums and gives the rows a short poll limit (64
polls), so each row stops waiting after a few microseconds.  Inputs are random device tensors: these
tests check the failure protocol, and compare the calls after ig_workspace_init bit for bit with the
same calls on a fresh workspace (the parity tests compare those with the oracle)."""
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
    yield L
    L.ig_set_handover_test_mode(0, False)


class Layer:
    """Random bf16 speculation inputs of one shape, with its outputs and a speculation workspace."""

    def __init__(self, L, B, H, D, r, n, max_out, seed):
        import torch
        g = torch.Generator(device="cuda").manual_seed(seed)
        dv = "cuda"
        self.B, self.H, self.D, self.r, self.n, self.max_out = B, H, D, r, n, max_out
        self.x = torch.randn((B, D), generator=g, device=dv).to(torch.bfloat16)
        self.W = (torch.randn((H * r, D), generator=g, device=dv) / 64).to(torch.bfloat16)
        self.Kp = torch.randn((B, H, n, r), generator=g, device=dv).to(torch.bfloat16)
        self.C0 = torch.randint(0, 50, (B, n), generator=g, device=dv, dtype=torch.int32)
        self.counters = self.C0.clone()
        self.idx = torch.zeros((B, H, max_out), dtype=torch.int32, device=dv)
        self.count = torch.zeros((B, H), dtype=torch.int32, device=dv)
        self.victim = torch.full((B,), -7, dtype=torch.int32, device=dv)
        self.q_part = torch.zeros((B, H, r), dtype=torch.float32, device=dv)
        self.ws = self.new_ws(L)

    def new_ws(self, L):
        import torch
        nb = L.ig_workspace_size(L.IG_OP_SPECULATE, self.B, self.H, self.D, 0, self.r, self.n, self.max_out)
        return L.ig_workspace_init(torch.empty(nb, dtype=torch.uint8, device="cuda"))

    def call(self, L, k, ws=None):
        self.counters.copy_(self.C0)
        L.ig_speculate(self.x, self.W, self.Kp, self.n, 0.125, "topk", self.max_out, k=k, idx=self.idx,
                       count=self.count, counters=self.counters, victim=self.victim, q_part=self.q_part,
                       ws=self.ws if ws is None else ws)

    def results(self):
        from sparse_attention_ig_amd.runtime import to_host
        return {name: to_host(getattr(self, name)).copy() for name in ("idx", "count", "counters", "victim", "q_part")}


def _arrivals_zero(ws, B):
    from sparse_attention_ig_amd.runtime import to_host
    return not to_host(ws)[256:256 + 4 * B].any()


def _same(a, b, tag):
    assert np.array_equal(a["count"], b["count"]), tag
    B, H = a["count"].shape
    for bb in range(B):
        for hh in range(H):
            c = int(a["count"][bb, hh])
            assert np.array_equal(a["idx"][bb, hh, :c], b["idx"][bb, hh, :c]), (tag, bb, hh)
    for key in ("counters", "victim", "q_part"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (tag, key)


def _failed(L, lay, res, bits, tag):
    """Every row failed: count -1, counters as before, the victim picked from them, arrivals back to 0."""
    from sparse_attention_ig_amd.runtime import to_host
    assert (res["count"] == -1).all(), (tag, res["count"])
    C0 = to_host(lay.C0)
    assert np.array_equal(res["counters"], C0), tag
    assert np.array_equal(res["victim"], np.argmin(C0[:, :lay.n], axis=1).astype(np.int32)), tag
    assert _arrivals_zero(lay.ws, lay.B), tag
    assert L.ig_workspace_status(lay.ws) & bits == bits, (tag, L.ig_workspace_status(lay.ws))


# whole rows; sliced rows merged per row; sliced rows whose merge leaves bitmaps for the counter kernel
SHAPES = [
    ("whole-rows", dict(B=2, H=3, D=1024, r=32, n=1500, max_out=100), 100),
    ("sliced-rows", dict(B=1, H=2, D=1024, r=32, n=20000, max_out=200), 200),
    ("sliced-bitmaps", dict(B=4, H=32, D=4096, r=32, n=65536, max_out=2048), 2048),
]


@pytest.mark.parametrize("name,shape,k", SHAPES, ids=[s[0] for s in SHAPES])
def test_timeout_is_reported_and_sticky(lib, name, shape, k):
    L = lib
    lay = Layer(L, **shape, seed=11)
    say(f"[handover {name}] reference call on a fresh workspace")
    lay.call(L, k)
    ref = lay.results()
    assert L.ig_workspace_status(lay.ws) == 0
    assert (ref["count"] == k).all()

    say(f"[handover {name}] partial sums withheld, 64 polls per row")
    ws = lay.new_ws(L)
    L.ig_set_handover_test_mode(64, True)
    try:
        lay.call(L, k, ws)
        res = lay.results()
    finally:
        L.ig_set_handover_test_mode(0, False)
    lay.ws, ref_ws = ws, lay.ws
    _failed(L, lay, res, L.IG_WS_TIMEOUT, f"{name} timeout")

    say(f"[handover {name}] normal mode again, same workspace: still failing (sticky)")
    lay.call(L, k)
    _failed(L, lay, lay.results(), L.IG_WS_TIMEOUT, f"{name} sticky")

    say(f"[handover {name}] after ig_workspace_init")
    L.ig_workspace_init(lay.ws)
    lay.call(L, k)
    assert L.ig_workspace_status(lay.ws) == 0
    _same(lay.results(), ref, f"{name} after init")
    lay.ws = ref_ws


def test_shape_stamp_mismatch(lib):
    """A workspace stamped by one (B, H, D, r) rejects a call of another until ig_workspace_init."""
    import torch
    L = lib
    a = Layer(L, B=2, H=4, D=1024, r=32, n=1200, max_out=64, seed=21)
    b = Layer(L, B=4, H=2, D=1024, r=32, n=1200, max_out=64, seed=22)
    say("[stamp] references on fresh workspaces")
    a.call(L, 64)
    ref_a = a.results()
    b.call(L, 64)
    ref_b = b.results()
    shared = L.ig_workspace_init(torch.empty(max(a.ws.numel(), b.ws.numel()), dtype=torch.uint8, device="cuda"))
    a.call(L, 64, shared)
    _same(a.results(), ref_a, "a on the shared workspace")
    assert L.ig_workspace_status(shared) == 0
    say("[stamp] b on a's workspace")
    b.ws = shared
    b.call(L, 64)
    _failed(L, b, b.results(), L.IG_WS_SHAPE, "b on a's stamp")
    say("[stamp] a again without init: sticky")
    a.ws = shared
    a.call(L, 64)
    _failed(L, a, a.results(), L.IG_WS_SHAPE, "a after the mismatch")
    say("[stamp] init, then b claims the workspace")
    L.ig_workspace_init(shared)
    b.call(L, 64)
    _same(b.results(), ref_b, "b after init")
    assert L.ig_workspace_status(shared) == 0


def test_decode_layer_speculation_fails_attention_runs(lib):
    """In the fused decode layer a failed speculation half leaves the attention half untouched."""
    import torch
    L = lib
    dv = "cuda"
    lay = Layer(L, B=2, H=4, D=512, r=32, n=1000, max_out=64, seed=31)
    g = torch.Generator(device=dv).manual_seed(32)
    q = torch.randn((2, 4, 128), generator=g, device=dv).to(torch.bfloat16)
    K = torch.randn((2, 4, 1000, 128), generator=g, device=dv).to(torch.bfloat16)
    V = torch.randn((2, 4, 1000, 128), generator=g, device=dv).to(torch.bfloat16)
    aidx = torch.sort(torch.randperm(1000, generator=g, device=dv)[:64]).values.to(torch.int32)
    aidx = aidx.repeat(2, 4, 1).contiguous()
    acnt = torch.full((2, 4), 64, dtype=torch.int32, device=dv)
    out_ref = torch.zeros((2, 4, 128), dtype=torch.float32, device=dv)
    L.ig_sparse_decode_attn(q, K, V, aidx, acnt, 0.088, out=out_ref)
    out = torch.zeros_like(out_ref)
    attn = dict(q=q, K=K, V=V, idx=aidx, count=acnt, scale=0.088, out=out)
    spec = dict(x=lay.x, Wq_part=lay.W, Kp=lay.Kp, n=lay.n, scale=0.125, mode="topk", k=64, idx=lay.idx,
                count=lay.count, counters=lay.counters, victim=lay.victim, q_part=lay.q_part, ws=lay.ws)
    say("[decode layer] partial sums withheld")
    lay.counters.copy_(lay.C0)
    L.ig_set_handover_test_mode(64, True)
    try:
        L.ig_decode_layer(attn, spec)
        torch.cuda.synchronize()
    finally:
        L.ig_set_handover_test_mode(0, False)
    _failed(L, lay, lay.results(), L.IG_WS_TIMEOUT, "decode layer")
    scale = out_ref.abs().amax(dim=-1, keepdim=True) + 1e-30
    assert float(((out - out_ref).abs() / scale).max()) <= 1e-5

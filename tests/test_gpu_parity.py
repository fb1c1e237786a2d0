"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Each side builds its inputs from the shared raw draws with its own setup (library vs oracle);
the setup routes are first checked to agree bit for bit.  Then:
  scores / q_part  within 1e-3, row-normwise;
  index sets       exactly equal except rows whose oracle score is within 1e-4 of the cut;
  attention        within 1e-2 max-abs (bf16 inputs) or 1e-5 (float32), on heads whose sets match;
  counters         bit-exact (sequences whose sets differ only in the band are adjusted first).
"""
import math

import numpy as np
import pytest

from oracle import oracle as O
from sparse_attention_ig_amd import gen
from tests import harness
from tests.gpu_util import DeviceLayer, dev, host, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_ig_amd import _lib as L
    L.load()
    say("device:", torch.cuda.get_device_name(0))
    yield


def _spec(base: gen.Spec, **kw) -> gen.Spec:
    return gen.Spec(**{**base.__dict__, **kw})


def small_bf16():
    return _spec(gen.opt_6_7b(n=1500, B=2), H=3, heavy=30, topk=100)


def long_global():
    return _spec(gen.llama2_7b_long(n=20000), H=2, topk=200)


def batch20_r16():
    # two 16-row batch blocks in the projection; a 32-column block spans two heads; D = 384 is not a
    # whole number of 512-input splits
    return _spec(gen.opt_6_7b(n=600, B=20), H=3, r=16, heavy=12, topk=50)


def tiny_batch17():
    return _spec(gen.tiny_fp32(), B=17)


CASES = [
    # name, spec factory, mode, kwargs
    ("tiny-threshold", gen.tiny_fp32, "threshold", dict(alpha=4.0)),
    ("tiny-topk32", gen.tiny_fp32, "topk", dict(k=32)),
    ("tiny-cap", gen.tiny_fp32, "threshold", dict(alpha=4.0, max_sel=51, cap=True)),
    ("tiny-halving", gen.tiny_fp32, "topk", dict(k=32, cmax=15, counters="random")),
    ("small-bf16-threshold", small_bf16, "threshold", dict(alpha=5.0, max_sel=300)),
    ("small-bf16-topk", small_bf16, "topk", dict(k=100)),
    ("small-bf16-headavg", small_bf16, "headavg", dict(alpha=5.0, max_sel=300)),
    ("opt6.7b-threshold-cap", gen.opt_6_7b, "threshold", dict(alpha=5.0, max_sel=409, cap=True)),
    ("opt6.7b-threshold-nocap", gen.opt_6_7b, "threshold", dict(alpha=5.0)),
    ("opt6.7b-topk128", gen.opt_6_7b, "topk", dict(k=128, counters="random", victim=True)),
    ("long-global-topk", long_global, "topk", dict(k=200)),
    ("long-global-threshold", long_global, "threshold", dict(alpha=5.0, max_sel=4000, cap=True)),
    ("batch20-r16-topk", batch20_r16, "topk", dict(k=50)),
    ("tiny-batch17-threshold", tiny_batch17, "threshold", dict(alpha=4.0)),
]


def _max_out(spec, mode, kw):
    if mode == "topk":
        return min(kw["k"], spec.n)
    if kw.get("cap"):
        return kw["max_sel"]
    return spec.n


def check_step(name, spec, mode, kw, lib_in=None, ora_in=None, path="unfused"):
    say(f"[case {name}] {path} B={spec.B} H={spec.H} d={spec.d} n={spec.n} r={spec.r} {spec.dtype} mode={mode} {kw}")
    lib_in = lib_in or harness.lib_inputs(spec)
    ora_in = ora_in or harness.oracle_inputs(spec)
    harness.assert_setup_routes_agree(lib_in, ora_in)
    cmax = kw.get("cmax", 65535)
    C0 = gen.draw_counters(spec, cmax) if kw.get("counters") == "random" else np.zeros((spec.B, spec.cap), np.uint32)
    max_out = _max_out(spec, mode, kw)
    alpha = kw.get("alpha", math.inf)
    k = kw.get("k", 0)
    max_sel = kw.get("max_sel", 0)
    want_victim = bool(kw.get("victim"))

    layer = DeviceLayer(lib_in, C0)
    parts = DeviceLayer.FUSED if path == "fused" else DeviceLayer.PARTS
    g = to_host(layer.step(mode=mode, alpha=alpha, k=k, max_sel=max_sel, max_out=max_out, cmax=cmax,
                           want_victim=want_victim, parts=parts))
    if path == "fused":
        # the arrival words (B words from byte 256 of the workspace) are back to zero, the status is clear
        from sparse_attention_ig_amd import _lib as L
        assert not host(layer.ws_spec)[256:256 + 8 * spec.B].any(), "per-sequence words must return to zero"
        assert L.ig_workspace_status(layer.ws_spec) == 0
    say(f"[case {name}] gpu step done")
    ref = harness.oracle_step(ora_in, mode=mode, alpha=alpha, k=k, max_sel=max_sel, max_out=max_out, cmax=cmax,
                              counters=C0, want_victim=want_victim)

    assert harness.score_error(g["q_part"], ref["q_part"]) <= harness.SCORE_RTOL
    serr = harness.score_error(g["scores"][..., :spec.n], ref["scores"])
    assert serr <= harness.SCORE_RTOL, serr

    tol = harness.ATTN_TOL[spec.dtype]
    inexact = []
    shifted = set()
    if mode == "headavg":
        # the shared count of a sequence may move only if some head's threshold count has a band row
        for b in range(spec.B):
            if not np.array_equal(g["count"][b], ref["count"][b]):
                assert any(len(harness.band_rows(ref["scores"][b, h], ref["scores"][b, h].max() - alpha))
                           for h in range(spec.H)), b
                shifted.add(b)
    for b in range(spec.B):
        for h in range(spec.H):
            if b in shifted:
                inexact.append((b, h))
                continue
            gs = g["idx"][b, h, :g["count"][b, h]]
            rs = ref["idx"][b, h, :ref["count"][b, h]]
            assert np.all(np.diff(gs) > 0), "gpu indices not ascending"
            ok, exact, band = harness.compare_sets(gs, rs, ref["scores"][b, h], mode, alpha)
            assert ok, (b, h, sorted(set(gs.tolist()) ^ set(rs.tolist())), band)
            if not exact:
                inexact.append((b, h))
                continue
            err = np.abs(g["out"][b, h] - ref["out"][b, h]).max()
            assert err <= tol, (b, h, err)
            assert abs(g["lse"][b, h] - ref["lse"][b, h]) <= max(tol, 1e-5 * abs(ref["lse"][b, h])), (b, h)
    assert len(inexact) <= max(spec.H if shifted else 1, spec.B * spec.H // 50), inexact
    bad_b = {b for b, _ in inexact}
    for b in range(spec.B):
        if b in bad_b:
            continue
        assert np.array_equal(g["counters"][b], ref["counters"][b]), b
        if want_victim:
            assert g["victim"][b] == ref["victim"][b]
    counts = g["count"]
    say(f"[case {name}] ok: score err {serr:.2e}, counts min/mean/max {counts.min()}/{counts.mean():.1f}/"
        f"{counts.max()}, band-affected heads {len(inexact)}")
    return g, ref


@pytest.mark.parametrize("name,factory,mode,kw", CASES, ids=[c[0] for c in CASES])
def test_decode_step_parity(name, factory, mode, kw):
    check_step(name, factory(), mode, kw)


FUSED_CASES = CASES


@pytest.mark.parametrize("name,factory,mode,kw", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_speculation_parity(name, factory, mode, kw):
    """ig_speculate (partial query, scores, selection and counters in one launch; the head average with
    a merge launch after the rows) + attention."""
    check_step(name, factory(), mode, kw, path="fused")


# ---------------------------------------------------------------- per-kernel parity on generator inputs
def _kv(spec):
    q = np.random.default_rng(spec.seed).standard_normal((spec.B, spec.D))
    K, V, _ = gen.draw_cache(spec, 0, q)
    qb = gen.encode(q.astype(np.float32), spec.dtype).reshape(spec.B, spec.H, spec.d)
    return qb, K, V


@pytest.mark.parametrize("spec_fn,max_out", [
    (lambda: _spec(gen.opt_6_7b(n=700, B=2), H=4), 300),       # single split, empty heads included
    (lambda: _spec(gen.opt_6_7b(n=6000, B=1), H=3), 5000),     # many splits + combine
    (lambda: _spec(gen.tiny_fp32(), frame="skewed", lognormal=True, B=2), 200),
])
def test_attention_kernel_parity(spec_fn, max_out):
    from sparse_attention_ig_amd import _lib as L
    spec = spec_fn()
    say(f"[attn] B={spec.B} H={spec.H} n={spec.n} {spec.dtype} max_out={max_out}")
    q, K, V = _kv(spec)
    idx, cnt = gen.draw_index_sets(spec, max_out)
    cnt[0, 0] = 0                       # an empty selection
    o, lse = L.ig_sparse_decode_attn(dev(q), dev(K), dev(V), dev(idx), dev(cnt), spec.softmax_scale)
    o, lse = host(o), host(lse)
    ro, rl = O.sparse_decode_attn(O.decode(q, spec.dtype), O.decode(K, spec.dtype), O.decode(V, spec.dtype), idx,
                                  cnt, spec.softmax_scale)
    tol = harness.ATTN_TOL[spec.dtype]
    assert np.abs(o - ro).max() <= tol
    assert np.all(o[0, 0] == 0) and lse[0, 0] == -np.inf
    fin = np.isfinite(rl)
    assert np.abs(lse[fin] - rl[fin]).max() <= max(tol, 1e-5 * np.abs(rl[fin]).max())
    # idx = NULL: dense over the first count rows
    dense_cnt = np.minimum(cnt + 1, spec.n).astype(np.int32)
    o2, _ = L.ig_sparse_decode_attn(dev(q), dev(K), dev(V), None, dev(dense_cnt), spec.softmax_scale,
                                    max_out=spec.cap)
    ro2, _ = O.sparse_decode_attn(O.decode(q, spec.dtype), O.decode(K, spec.dtype), O.decode(V, spec.dtype), None,
                                  dense_cnt, spec.softmax_scale)
    assert np.abs(host(o2) - ro2).max() <= tol


def test_gather_and_partial_cache_bit_exact():
    from sparse_attention_ig_amd import _lib as L
    import torch
    spec = _spec(gen.opt_6_7b(n=900, B=2), H=3)
    say("[gather/build] ", spec.B, spec.H, spec.n)
    q, K, V = _kv(spec)
    idx, cnt = gen.draw_index_sets(spec, 128)
    Kc, Vc = L.ig_gather_kv(dev(K), dev(V), dev(idx), dev(cnt))
    rK, rV = O.gather_kv(K, V, idx, cnt, 128)
    Kc, Vc = host(Kc), host(Vc)
    for b in range(spec.B):
        for h in range(spec.H):
            c = cnt[b, h]
            assert np.array_equal(Kc[b, h, :c], rK[b, h, :c]) and np.array_equal(Vc[b, h, :c], rV[b, h, :c])
    chan = np.sort(np.random.default_rng(0).permuted(np.tile(np.arange(spec.d), (spec.H, 1)), axis=1)[:, :spec.r],
                   axis=1).astype(np.int32)
    Kd = dev(K)
    Kp = torch.zeros((spec.B, spec.H, spec.cap, spec.r), dtype=Kd.dtype, device="cuda")
    L.ig_build_partial_cache(Kd, dev(chan), Kp, 0, 500)
    L.ig_build_partial_cache(Kd, dev(chan), Kp, 500, spec.n)
    assert np.array_equal(host(Kp), O.partial_key_cache(K, chan))


@pytest.mark.parametrize("cmax,H,max_out", [(15, 8, 400), (65535, 8, 400), (15, 64, 1000), (65535, 64, 1000)])
def test_pool_touch_bit_exact(cmax, H, max_out):
    """Single-workgroup path (H * max_out <= 32768) and the three-launch path for large selections."""
    from sparse_attention_ig_amd import _lib as L
    spec = _spec(gen.opt_6_7b(n=3000, B=3), H=H)
    say(f"[touch] cmax={cmax} H={H} max_out={max_out}")
    C = gen.draw_counters(spec, cmax)
    idx, cnt = gen.draw_index_sets(spec, max_out)
    Cd = dev(C)
    rC = C
    for step in range(3):
        _, victim = L.ig_pool_touch(Cd, dev(idx), dev(cnt), spec.n, cmax, want_victim=True)
        rC, rv = O.pool_touch(rC, idx, cnt, spec.n, cmax, want_victim=True)
        assert np.array_equal(host(Cd).view(np.uint32), rC), step
        assert np.array_equal(host(victim), rv), step


def test_append_matches_oracle():
    from sparse_attention_ig_amd import _lib as L
    import torch
    spec = _spec(gen.opt_6_7b(n=64, B=2), H=2, n_cap=66)
    say("[append]")
    q, K, V = _kv(spec)
    chan = np.tile(np.arange(0, spec.d, spec.d // spec.r, dtype=np.int32), (spec.H, 1))
    Kp = O.partial_key_cache(K, chan)
    C = gen.draw_counters(spec, 100)
    Kd, Vd, Kpd, Cd, chd = dev(K), dev(V), dev(Kp), dev(C), dev(chan)
    rK, rV, rKp, rC = K.copy(), V.copy(), Kp.copy(), C.copy()
    n = spec.n
    slot = torch.empty(spec.B, dtype=torch.int32, device="cuda")
    for step in range(4):
        kn, vn = gen.draw_new_rows(spec, 0, step)
        victim = np.array([5 + step, 60 - step], dtype=np.int32)
        L.ig_append_kv(Kd, Vd, Kpd, Cd, chd, dev(kn), dev(vn), n, victim=dev(victim), slot_out=slot)
        slots, n2 = O.pool_append(rK, rV, rKp, rC, chan, kn, vn, n, victim=victim)
        assert np.array_equal(host(slot), slots)
        n = n2
    assert np.array_equal(host(Kd), rK) and np.array_equal(host(Vd), rV)
    assert np.array_equal(host(Kpd), rKp) and np.array_equal(host(Cd).view(np.uint32), rC)


def test_edge_cases():
    from sparse_attention_ig_amd import _lib as L
    spec = _spec(gen.opt_6_7b(n=1, B=1), H=2, heavy=0)
    # n = 1: every rule selects the single row
    for mode, kw in [("threshold", dict(alpha=0.0)), ("topk", dict(k=5)), ("headavg", dict(alpha=3.0))]:
        check_step(f"n1-{mode}", spec, mode, kw)
    s2 = small_bf16()
    li, oi = harness.lib_inputs(s2), harness.oracle_inputs(s2)
    check_step("alpha0", s2, "threshold", dict(alpha=0.0), li, oi)
    check_step("alpha-inf", s2, "threshold", dict(alpha=math.inf), li, oi)
    check_step("k-above-n", s2, "topk", dict(k=5000), li, oi)
    check_step("k-equals-n", s2, "topk", dict(k=s2.n), li, oi)
    # output capacity below the selection: clamped by score
    g, ref = check_step("max-out-clamp", s2, "threshold", dict(alpha=8.0, max_sel=7, cap=True), li, oi)
    assert g["count"].max() <= 7
    # r = d: speculated scores are the exact logits
    s3 = _spec(gen.opt_6_7b(n=257, B=1), H=2, r=128, heavy=5)
    g, ref = check_step("r-equals-d", s3, "topk", dict(k=20))
    lay = gen.draw_layer(s3, with_wk=False)
    inp = harness.oracle_inputs(s3, lay=lay)
    exact = np.einsum("bhd,bhnd->bhn", O.decode(inp.q, "bf16"), O.decode(inp.K[:, :, :s3.n], "bf16")) * s3.softmax_scale
    # q_part is x W~ over all channels, the full skewed query before its own rounding
    assert harness.score_error(g["scores"][..., :s3.n], exact) <= 2e-2


def test_determinism():
    spec = gen.opt_6_7b()
    say("[determinism]")
    li = harness.lib_inputs(spec)
    runs = []
    for _ in range(2):
        layer = DeviceLayer(li)
        runs.append(to_host(layer.step(mode="threshold", alpha=5.0, max_sel=409, max_out=409)))
    assert np.array_equal(runs[0]["count"], runs[1]["count"])
    for key in ("q_part", "scores", "out", "lse", "counters"):
        a, b = runs[0][key], runs[1][key]
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), key
    cnt = runs[0]["count"]
    for b in range(spec.B):
        for h in range(spec.H):
            c = cnt[b, h]     # entries past count are unspecified
            assert np.array_equal(runs[0]["idx"][b, h, :c], runs[1]["idx"][b, h, :c])


@pytest.mark.parametrize("path", ["unfused", "fused"])
def test_long_context_full_size(path):
    """Llama-2-7B-shaped layer at 131072 rows, top 1%: every head's scores, selection and attention
    against the oracle, counters slot by slot.  The fused speculation cuts each row into slices (one
    workgroup each, candidates merged per row)."""
    spec = gen.llama2_7b_long(n=131072, B=1, frac=0.01)
    say(f"[long full {path}] n={spec.n} k={spec.topk}")
    li, oi = harness.lib_inputs(spec), harness.oracle_inputs(spec)
    harness.assert_setup_routes_agree(li, oi)
    layer = DeviceLayer(li, max_out=spec.topk)
    parts = DeviceLayer.FUSED if path == "fused" else DeviceLayer.PARTS
    g = to_host(layer.step(mode="topk", k=spec.topk, max_out=spec.topk, want_victim=True, parts=parts))
    say("[long full] gpu step done")
    ref, ri, rc = harness.oracle_heads(oi, mode="topk", k=spec.topk, max_out=spec.topk)
    inexact = harness.check_heads(g["idx"], g["count"], ref, "topk", 0.0, g_q_part=g["q_part"], g_scores=g["scores"],
                                  g_out=g["out"], g_lse=g["lse"], tol=harness.ATTN_TOL["bf16"])
    assert len(inexact) <= 1, inexact
    assert (g["count"] == spec.topk).all()
    rC, rv = O.pool_touch(np.zeros((spec.B, spec.cap), np.uint32), ri, rc, spec.n, 65535, want_victim=True)
    harness.check_counters(g["counters"], rC, g["idx"], g["count"], ri, rc, spec.n, g["victim"], rv)


def test_graph_replay_matches_eager():
    """The layer-step captured once in a HIP graph and replayed (with eager work and
    synchronisations between replays) gives the eager results on every replay."""
    import torch
    spec = gen.opt_6_7b()
    say("[graph replay]")
    li = harness.lib_inputs(spec)
    layer = DeviceLayer(li, max_out=128)
    kw = dict(mode="topk", k=128, max_out=128)
    C0 = layer.counters.clone()
    eager = to_host(layer.step(**kw))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.counters.copy_(C0)
        layer.step(**kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.step(**kw)
    for rep in range(3):
        layer.counters.copy_(C0)
        layer.scores.fill_(-1.0)
        layer.out.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = to_host(dict(scores=layer.scores, count=layer.count, idx=layer.idx, out=layer.out, lse=layer.lse,
                           counters=layer.counters))
        for key in ("scores", "count", "out", "lse", "counters"):
            assert np.array_equal(got[key].view(np.uint8), eager[key].view(np.uint8)), (rep, key)
        assert np.array_equal(got["idx"], eager["idx"]), rep


def test_long_context_32k_fused():
    """Llama-2-7B-shaped layer at 32768 rows (the fused path's LDS limit), batch 4, top 4%: every head's
    scores, selection and attention against the oracle, counters slot by slot."""
    spec = gen.llama2_7b_long(n=32768, B=4, frac=0.04)
    say(f"[long 32k fused] n={spec.n} k={spec.topk}")
    li, oi = harness.lib_inputs(spec), harness.oracle_inputs(spec)
    harness.assert_setup_routes_agree(li, oi)
    layer = DeviceLayer(li, max_out=spec.topk)
    g = to_host(layer.step(mode="topk", k=spec.topk, max_out=spec.topk, want_victim=True, parts=DeviceLayer.FUSED))
    say("[long 32k fused] gpu step done")
    ref, ri, rc = harness.oracle_heads(oi, mode="topk", k=spec.topk, max_out=spec.topk)
    inexact = harness.check_heads(g["idx"], g["count"], ref, "topk", 0.0, g_q_part=g["q_part"], g_scores=g["scores"],
                                  g_out=g["out"], g_lse=g["lse"], tol=harness.ATTN_TOL["bf16"])
    assert len(inexact) <= 3, inexact
    rC, rv = O.pool_touch(np.zeros((spec.B, spec.cap), np.uint32), ri, rc, spec.n, 65535, want_victim=True)
    harness.check_counters(g["counters"], rC, g["idx"], g["count"], ri, rc, spec.n, g["victim"], rv)

"""GPU: the INT4 pool (records of 4-bit group-wise asymmetric codes, float16 step and minimum per group of
32; only the speculated rows fetched and dequantised) against the oracle.

The summary proposes this combination under "Follow-Up Research" (prefetch only the selected tokens of a
quantised pool) and names the 4-bit group-wise asymmetric scheme among its section 5 baselines.  Codes,
steps and minima are integer or float16 decisions that both sides take in float32: bit-exact.  The
dequantised rows are m16 + code * s16 rounded once to float32 then stored: bit-exact.  The pool step
(speculation in HBM, gather of the selected records from pinned host memory, attention) matches the
oracle's attention over its own dequantised rows within the bf16 attention tolerance.
"""
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


def unpack(rec: np.ndarray, d: int):
    """(K codes, K steps, K minima), (V codes, V steps, V minima) and the padding of records
    [.., record bytes], read by the documented layout: K codes in bytes [0, d/2), V codes in [d/2, d),
    low nibble first; then (step, minimum) float16 pairs per group of 32, K groups first."""
    g = d // 32
    out = []
    for half in range(2):
        b = rec[..., half * d // 2:(half + 1) * d // 2]
        codes = np.empty(rec.shape[:-1] + (d,), np.uint8)
        codes[..., 0::2] = b & 15
        codes[..., 1::2] = b >> 4
        sm = np.ascontiguousarray(rec[..., d + 4 * g * half:d + 4 * g * (half + 1)]).view(np.float16)
        out.append((codes, sm[..., 0::2], sm[..., 1::2]))
    return out[0], out[1], rec[..., d + 8 * g:]


def _same(got, ref):
    (q, s, m), (rq, rs, rm) = got, ref
    return np.array_equal(q, rq) and np.array_equal(s.view(np.uint16), rs.view(np.uint16)) and \
        np.array_equal(m.view(np.uint16), rm.view(np.uint16))


def _cache(g, B, H, n, d, dtype):
    scale = np.exp(g.standard_normal((1, H, 1, d)))
    return gen.encode((g.standard_normal((B, H, n, d)) * scale).astype(np.float32), dtype)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 128), ("bf16", 64)])
def test_quantize_matches_oracle(dtype, d):
    import torch
    from sparse_attention_ig_amd import _lib as L
    g = np.random.default_rng(11 + d)
    B, H, n = 2, 3, 150
    K, V = _cache(g, B, H, n, d, dtype), _cache(g, B, H, n, d, dtype)
    K[0, 0, 7] = K[0, 0, 7, :1]                      # a constant row: step 0, codes 0
    rec = L.ig_int4_record_bytes(d)
    Xq = torch.full((B, H, n, rec), 0xAB, dtype=torch.uint8, device="cuda")
    say(f"[int4 quantize] {dtype} d={d}")
    L.ig_quantize_kv(dev(K), dev(V), Xq, 0, n)
    gk, gv, pad = unpack(host(Xq), d)
    assert _same(gk, O.quantize_int4(K, dtype)) and _same(gv, O.quantize_int4(V, dtype))
    assert not pad.any()


def test_quantize_append_at_slots():
    import torch
    from sparse_attention_ig_amd import _lib as L
    g = np.random.default_rng(5)
    B, H, d, q_rows = 2, 4, 128, 40
    kn, vn = _cache(g, B, H, 1, d, "bf16"), _cache(g, B, H, 1, d, "bf16")
    rec = L.ig_int4_record_bytes(d)
    Xq = torch.full((B, H, q_rows, rec), 0x5A, dtype=torch.uint8, device="cuda")
    slot = torch.tensor([7, 39], dtype=torch.int32, device="cuda")
    say("[int4 append slots]")
    L.ig_quantize_kv(dev(kn), dev(vn), Xq, 0, 1, slot=slot)
    got = host(Xq)
    rk, rv = O.quantize_int4(kn[:, :, 0], "bf16"), O.quantize_int4(vn[:, :, 0], "bf16")
    for b, sl in enumerate((7, 39)):
        gk, gv, _ = unpack(got[b, :, sl], d)
        assert _same(gk, tuple(a[b] for a in rk)) and _same(gv, tuple(a[b] for a in rv))
        others = np.delete(got[b], sl, axis=1)
        assert np.all(others == 0x5A)


@pytest.mark.parametrize("where,dtype_out", [("device", "bf16"), ("host", "bf16"), ("device", "f32")])
def test_gather_int4_matches_oracle(where, dtype_out):
    import torch
    from sparse_attention_ig_amd import _lib as L
    from sparse_attention_ig_amd.runtime import MappedHost
    g = np.random.default_rng(21)
    B, H, n, d, max_out = 2, 3, 300, 128, 40
    K, V = _cache(g, B, H, n, d, "bf16"), _cache(g, B, H, n, d, "bf16")
    rec = L.ig_int4_record_bytes(d)
    Xq = torch.empty((B, H, n, rec), dtype=torch.uint8, device="cuda")
    L.ig_quantize_kv(dev(K), dev(V), Xq, 0, n)
    if where == "host":
        Xh = Xq.cpu().pin_memory()
        src = MappedHost(Xh)
    else:
        src = Xq
    idx = np.sort(g.permuted(np.tile(np.arange(n), (B, H, 1)), axis=-1)[..., :max_out], axis=-1).astype(np.int32)
    count = g.integers(0, max_out + 1, (B, H)).astype(np.int32)
    count[0, 0] = max_out
    Kc = torch.zeros((B, H, max_out, d), dtype=torch.bfloat16 if dtype_out == "bf16" else torch.float32,
                     device="cuda")
    Vc = torch.zeros_like(Kc)
    say(f"[int4 gather] {where} {dtype_out}")
    L.ig_gather_kv_int4(src, dev(idx), dev(count), d, Kc=Kc, Vc=Vc)
    gk, gv = host(Kc), host(Vc)
    Kq, Ks, Km = O.quantize_int4(K, "bf16")
    Vq, Vs, Vm = O.quantize_int4(V, "bf16")
    rk, rv = O.gather_kv_int4(Kq, Ks, Km, Vq, Vs, Vm, idx, count, max_out, dtype_out)
    for b in range(B):
        for h in range(H):
            c = count[b, h]
            assert np.array_equal(gk[b, h, :c].view(np.uint8), rk[b, h, :c].view(np.uint8)), (b, h)
            assert np.array_equal(gv[b, h, :c].view(np.uint8), rv[b, h, :c].view(np.uint8)), (b, h)


def test_int4_pool_step_matches_oracle():
    """PoolLayer with INT4 records: threshold speculation in HBM, gather of the selected records from
    pinned host memory, attention on the dequantised rows; then an append at slot n."""
    import torch
    from sparse_attention_ig_amd.runtime import PoolLayer, prepare_layer
    base = gen.opt_30b(n=600, B=2, n_cap=640)
    spec = gen.Spec(**{**base.__dict__, "H": 4})
    li, oi = harness.lib_inputs(spec), harness.oracle_inputs(spec)
    max_out = spec.max_sel
    say(f"[int4 pool] B={spec.B} H={spec.H} n={spec.n} cap={spec.cap} max_out={max_out}")
    lay = PoolLayer(li, max_out=max_out, int4=True)
    lay.speculate(alpha=spec.alpha, max_sel=spec.max_sel)
    lay.gather()
    lay.attend()
    torch.cuda.synchronize()
    gi, gc, out = host(lay.idx), host(lay.count), host(lay.out)
    dt = spec.dtype
    _, sc = O.rehearse(O.decode(oi.x, dt), O.decode(oi.Wq_part, dt), O.decode(oi.extra["Kp"], dt), spec.n, spec.H,
                       spec.r, spec.softmax_scale)
    ridx, rcnt = O.select(sc, "threshold", alpha=spec.alpha, max_sel=spec.max_sel, max_out=max_out)
    Kq, Ks, Km = O.quantize_int4(oi.K, dt)
    Vq, Vs, Vm = O.quantize_int4(oi.V, dt)
    # the gather leaves the dequantised rows in bf16 compact buffers: the attention reads those values
    Kd = O.decode(O.store(O.dequantize_int4(Kq, Ks, Km), dt), dt)
    Vd = O.decode(O.store(O.dequantize_int4(Vq, Vs, Vm), dt), dt)
    q = O.decode(oi.q, dt)
    exact = 0
    for b in range(spec.B):
        for h in range(spec.H):
            gs, rs = gi[b, h, :gc[b, h]], ridx[b, h, :rcnt[b, h]]
            ok, same, _ = harness.compare_sets(gs, rs, sc[b, h], "threshold", spec.alpha)
            assert ok, (b, h)
            if same:
                exact += 1
                rows = rs.astype(np.int64)
                o, _ = O.attention_rows(q[b, h], Kd[b, h, rows], Vd[b, h, rows], spec.softmax_scale)
                assert np.abs(out[b, h] - o).max() <= harness.ATTN_TOL["bf16"], (b, h)
    assert exact >= spec.B * spec.H // 2
    # append the next token: its records land at slot n, its partial key row in HBM
    kn, vn = gen.draw_new_rows(spec, 0, 0)
    slot = host(lay.append(dev(kn), dev(vn), spec.n))
    assert np.all(slot == spec.n)
    torch.cuda.synchronize()
    gk, gv, _ = unpack(lay.KVq_host.numpy()[:, :, spec.n], spec.d)
    assert _same(gk, O.quantize_int4(kn, dt)) and _same(gv, O.quantize_int4(vn, dt))
    assert np.array_equal(host(lay.Kp)[:, :, spec.n], np.take_along_axis(kn, li.chan[None, :, :].repeat(spec.B, 0), 2))

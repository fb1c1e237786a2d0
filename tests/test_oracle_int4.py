"""Pins of the oracle's INT4 pool functions (group-wise asymmetric 4-bit quantisation of key and value
rows, dequantisation, gather of the dequantised selected rows) against hand-computed groups
(tests/golden/int4_cases.json), the defining optimality of each code, the error bound it implies, and
special cases."""
import json
import os

import numpy as np
import pytest

from oracle import oracle as O
from sparse_attention_ig_amd import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int4_cases.json")


def _check_golden():
    doc = json.load(open(GOLDEN))
    G = doc["group"]
    for case in doc["cases"]:
        x = gen.encode(np.asarray(case["values"], np.float32)[None, :], "bf16")
        q, s16, m16 = O.quantize_int4(x, "bf16", G)
        assert list(q[0]) == case["expect_codes"], case["note"]
        assert float(s16[0, 0]) == case["expect_step"] and float(m16[0, 0]) == case["expect_min"], case["note"]
        assert list(O.dequantize_int4(q, s16, m16, G)[0]) == case["expect_dequant"], case["note"]


def test_golden_groups():
    _check_golden()


def test_planted_rounding_mistake_fails_the_fixture(monkeypatch):
    """Truncating instead of rounding to nearest (a plausible slip) must fail the hand-computed groups."""
    monkeypatch.setattr(O.np, "rint", np.floor)
    with pytest.raises(AssertionError):
        _check_golden()


def _groups(seed, rows=64, d=128, scale=3.0):
    g = np.random.default_rng(seed)
    v = g.standard_normal((rows, d)).astype(np.float32) * np.float32(scale) * np.exp(g.standard_normal((rows, 1)))
    return gen.encode(v.astype(np.float32), "bf16")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_each_code_is_the_nearest_level(seed):
    """q minimises |v - (m16 + q s16)| over the 16 levels (up to float32 rounding of the quotient)."""
    x = _groups(seed)
    q, s16, m16 = O.quantize_int4(x, "bf16")
    v = O.decode(x, "bf16").reshape(q.shape[0], -1, O.INT4_GROUP)
    sf = s16.astype(np.float64)[..., None]
    mf = m16.astype(np.float64)[..., None]
    levels = mf[..., None] + np.arange(16)[None, None, None, :] * sf[..., None]
    err = np.abs(v[..., None] - levels)                       # [rows][groups][G][16]
    chosen = np.take_along_axis(err, q.reshape(v.shape)[..., None].astype(np.int64), axis=-1)[..., 0]
    assert np.all(chosen <= err.min(axis=-1) + 1e-6 * sf)


@pytest.mark.parametrize("seed", [4, 5])
def test_round_trip_error_bound(seed):
    """|v - dequant| <= s16 / 2 plus the float16 rounding of the step (x 15) and of the minimum."""
    x = _groups(seed)
    q, s16, m16 = O.quantize_int4(x, "bf16")
    v = O.decode(x, "bf16")
    vg = v.reshape(v.shape[0], -1, O.INT4_GROUP)
    mn, mx = vg.min(-1), vg.max(-1)
    s = (mx - mn) / 15.0
    bound = 0.5 * s16.astype(np.float64) + 15 * np.abs(s - s16.astype(np.float64)) + \
        np.abs(mn - m16.astype(np.float64)) + 1e-6 * np.maximum(s, 1e-30)
    err = np.abs(v - O.dequantize_int4(q, s16, m16)).reshape(vg.shape).max(-1)
    assert np.all(err <= bound)
    # the extremes of a group: its minimum maps to level 0 or 1 and its maximum to level 14 or 15
    qg = q.reshape(vg.shape)
    assert np.all(np.take_along_axis(qg, vg.argmin(-1)[..., None], -1) <= 1)
    assert np.all(np.take_along_axis(qg, vg.argmax(-1)[..., None], -1) >= 14)


def test_gather_of_quantised_rows():
    """The gather of the dequantised selected rows equals the plain gather of the dequantised cache."""
    g = np.random.default_rng(9)
    B, H, n, d = 2, 3, 40, 64
    K = gen.encode(g.standard_normal((B, H, n, d)).astype(np.float32), "bf16")
    V = gen.encode(g.standard_normal((B, H, n, d)).astype(np.float32), "bf16")
    Kq, Ks, Km = O.quantize_int4(K, "bf16")
    Vq, Vs, Vm = O.quantize_int4(V, "bf16")
    max_out = 10
    idx = np.sort(g.permuted(np.tile(np.arange(n), (B, H, 1)), axis=-1)[..., :max_out], axis=-1).astype(np.int32)
    count = g.integers(1, max_out + 1, (B, H)).astype(np.int32)
    Kc, Vc = O.gather_kv_int4(Kq, Ks, Km, Vq, Vs, Vm, idx, count, max_out, "bf16")
    Kd = O.store(O.dequantize_int4(Kq, Ks, Km), "bf16")
    Vd = O.store(O.dequantize_int4(Vq, Vs, Vm), "bf16")
    Kr, Vr = O.gather_kv(Kd, Vd, idx, count, max_out)
    for b in range(B):
        for h in range(H):
            c = count[b, h]
            assert np.array_equal(Kc[b, h, :c], Kr[b, h, :c]) and np.array_equal(Vc[b, h, :c], Vr[b, h, :c])

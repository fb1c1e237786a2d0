"""The shared input generator: determinism, keyed slices, encoding round trip, shapes."""
import numpy as np

from sparse_attention_ig_amd import gen
from oracle import oracle as O


def test_bf16_encoding_round_trip():
    g = np.random.default_rng(0)
    a = (g.standard_normal(10000) * 100).astype(np.float32)
    bits = gen.bf16_bits(a)
    back = O.decode(bits, "bf16")
    # within half an ulp of bf16 (8 significant bits)
    assert np.all(np.abs(back - a) <= np.abs(a) * 2.0 ** -8 + 1e-38)
    # agrees with the oracle's own float32 -> bf16 rounding
    assert np.array_equal(bits, O.store(a.astype(np.float64), "bf16"))


def test_draws_are_deterministic_and_keyed():
    spec = gen.opt_6_7b(n=64, B=2)
    spec = gen.Spec(**{**spec.__dict__, "H": 4, "d": 16})
    l1 = gen.draw_layer(spec, 3)
    l2 = gen.draw_layer(spec, 3)
    assert np.array_equal(l1.x, l2.x) and np.array_equal(l1.Wq, l2.Wq)
    assert np.array_equal(l1.skew_src, l2.skew_src)
    q = np.random.default_rng(1).standard_normal((spec.B, spec.D))
    K, V, heavy = gen.draw_cache(spec, 3, q)
    Ks, Vs, pos = gen.draw_cache_slice(spec, 3, 1, 2, q[1, 32:48])
    assert np.array_equal(K[1, 2, :spec.n], gen.encode(Ks.astype(np.float32), "bf16"))
    assert np.array_equal(V[1, 2, :spec.n], gen.encode(Vs, "bf16"))
    assert len(pos) == spec.heavy and len(set(pos.tolist())) == len(pos)
    assert K.shape == (2, 4, 64, 16) and K.dtype == np.uint16


def test_heavy_rows_align_with_query():
    spec = gen.opt_6_7b(n=512, B=1)
    spec = gen.Spec(**{**spec.__dict__, "H": 2})
    q = np.random.default_rng(2).standard_normal((1, spec.D))
    K, V, pos = gen.draw_cache_slice(spec, 0, 0, 1, q[0, 128:256])
    qh = q[0, 128:256] / np.linalg.norm(q[0, 128:256])
    proj = K @ qh
    heavy = np.zeros(spec.n, bool)
    heavy[pos] = True
    assert proj[heavy].min() > np.percentile(proj[~heavy], 99)


def test_tiny_raw_frame_shapes():
    spec = gen.tiny_fp32()
    lay = gen.draw_layer(spec)
    assert lay.x.dtype == np.float32 and lay.x.shape == (1, 256)
    assert lay.skew_src.shape == (4, 256, 64)
    assert lay.K_raw.shape == (1, 4, 256, 64) and lay.V.shape == (1, 4, 256, 64)
    assert np.array_equal(lay.heavy_pos[0, 0], lay.heavy_pos[0, 3])   # shared positions

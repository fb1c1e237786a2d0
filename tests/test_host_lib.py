"""Host-side checks of libig.so that need no GPU: exported symbols, the offline setup against the
oracle, storage rounding, and argument validation (every rejection happens before a launch)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from oracle import oracle as O
from sparse_attention_ig_amd import gen
from tests import harness
from tests.conftest import ROOT

L = pytest.importorskip("sparse_attention_ig_amd._lib")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libig.so not built")
    return L.load()


def test_exports_every_declared_symbol(lib):
    with open(os.path.join(ROOT, "include", "ig.h")) as f:
        header = f.read()
    declared = set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(ig_\w+)\s*\(", header, re.M))
    assert declared, "no declarations parsed"
    assert declared == set(L.exported_symbols())
    for name in declared:
        assert hasattr(lib, name)
    assert L.ig_version() == 11


@pytest.mark.parametrize("m,d", [(256, 64), (128, 128), (64, 16)])
def test_skew_weights_match_oracle(lib, m, d):
    g = np.random.default_rng(m + d)
    H, D = 3, 3 * d
    src = g.standard_normal((H, m, d))
    Wq = g.standard_normal((D, D)) / math.sqrt(D)
    Wk = g.standard_normal((D, D)) / math.sqrt(D)
    bq = g.standard_normal(D)
    out = L.ig_skew_weights(src, Wq=Wq, Wk=Wk, bq=bq)
    A_ref, Wq_ref, Wk_ref, bq_ref, _ = O.skew_weights(Wq, Wk, src, bq=bq)
    np.testing.assert_allclose(out["A"], A_ref, atol=1e-9)
    np.testing.assert_allclose(out["Wq_s"], Wq_ref, atol=1e-9)
    np.testing.assert_allclose(out["Wk_s"], Wk_ref, atol=1e-9)
    np.testing.assert_allclose(out["bq_s"], bq_ref, atol=1e-9)
    for h in range(H):
        A = out["A"][h]
        np.testing.assert_allclose(A.T @ A, np.eye(d), atol=1e-12)
        assert np.all(np.diff(out["sigma"][h]) <= 0)
        np.testing.assert_allclose(np.linalg.norm(src[h] @ A, axis=0), out["sigma"][h], rtol=1e-10)


def test_skew_apply_matches_oracle(lib):
    g = np.random.default_rng(1)
    A = O.skew_rotation(g.standard_normal((2, 40, 16)))
    M = g.standard_normal((7, 32))
    np.testing.assert_allclose(L.ig_skew_apply(A, M), O.skew_apply(A, M), atol=1e-12)


def test_store_matches_oracle_bits(lib):
    g = np.random.default_rng(2)
    vals = np.concatenate([g.standard_normal(5000) * 10, [1 + 2 ** -8, 1 + 3 * 2 ** -8, -0.0, 0.0, 1e39, -1e39,
                                                            1e-45, 3.4e38]])
    assert np.array_equal(L.ig_store(vals, "bf16"), O.store(vals, "bf16"))
    assert np.array_equal(L.ig_store(vals, "f32").view(np.uint32), O.store(vals, "f32").view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_partial_weight_index_matches_oracle(lib, dtype):
    g = np.random.default_rng(3)
    B, H, d, n, cap, r, D = 2, 3, 32, 50, 60, 8, 64
    Wq_s = gen.encode(g.standard_normal((D, H * d)).astype(np.float32), dtype)
    K = gen.encode((g.standard_normal((B, H, cap, d)) * np.exp(g.standard_normal(d))).astype(np.float32), dtype)
    chan, Wp = L.ig_partial_weight_index(Wq_s, K, r, n, dtype)
    chan_ref = O.partial_weight_index(Wq_s, K, H, d, r, n, dtype=dtype)
    assert np.array_equal(chan, chan_ref)
    # the library stores the selection transposed: one row of D inputs per partial column
    assert np.array_equal(Wp, O.pack_partial_weight(Wq_s, chan_ref, d).T)


def _small_bf16():
    base = gen.opt_6_7b(n=300, B=2)
    return gen.Spec(**{**base.__dict__, "H": 3, "topk": 16})


@pytest.mark.parametrize("spec_fn", [gen.tiny_fp32, _small_bf16])
def test_setup_routes_agree(lib, spec_fn):
    """Library route and oracle route from the same raw draws give the same stored inputs."""
    spec = spec_fn()
    a = harness.lib_inputs(spec)
    b = harness.oracle_inputs(spec)
    mism = harness.compare_inputs(a, b)
    assert mism["chan"] == 0 and mism["x"] == 0 and mism["V"] == 0
    total = a.K.size + a.q.size + a.Wq_part.size
    assert mism["K"] + mism["q"] + mism["Wq_part"] <= max(2, total * 1e-5), mism


def test_device_calls_reject_bad_arguments_before_launch(lib):
    """Invalid arguments return IG_EINVAL on the host; nothing reaches the GPU."""
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    f = ctypes.c_float
    # NULL inputs
    assert lib.ig_rehearse(None, p, None, p, 1, 64, 1, 8, 4, 4, L.IG_BF16, f(1.0), p, p, 4, p, 1 << 20, None) == L.IG_EINVAL
    # n > n_cap
    assert lib.ig_rehearse(p, p, None, p, 1, 64, 1, 8, 9, 4, L.IG_BF16, f(1.0), p, p, 9, p, 1 << 20, None) == L.IG_EINVAL
    assert "bad sizes" in L.ig_last_error()
    # r not a multiple of 8
    assert lib.ig_rehearse(p, p, None, p, 1, 64, 1, 12, 4, 4, L.IG_BF16, f(1.0), p, p, 4, p, 1 << 20, None) == L.IG_EINVAL
    # workspace too small
    assert lib.ig_rehearse(p, p, None, p, 8, 4096, 32, 32, 2048, 2048, L.IG_BF16, f(1.0), p, p, 2048, p, 16, None) == L.IG_EINVAL
    # negative alpha, NaN alpha, k = 0, unknown mode
    assert lib.ig_select(p, 1, 1, 4, 4, L.IG_SEL_THRESHOLD, f(-1.0), 0, 0, p, p, 4, None, 0, None) == L.IG_EINVAL
    assert lib.ig_select(p, 1, 1, 4, 4, L.IG_SEL_THRESHOLD, f(math.nan), 0, 0, p, p, 4, None, 0, None) == L.IG_EINVAL
    assert lib.ig_select(p, 1, 1, 4, 4, L.IG_SEL_TOPK, f(0.0), 0, 0, p, p, 4, None, 0, None) == L.IG_EINVAL
    assert lib.ig_select(p, 1, 1, 4, 4, 7, f(0.0), 1, 0, p, p, 4, None, 0, None) == L.IG_EINVAL
    assert lib.ig_select(p, 1, 1, 0, 4, L.IG_SEL_TOPK, f(0.0), 1, 0, p, p, 4, None, 0, None) == L.IG_EINVAL
    # head dim not supported; misaligned pointer
    assert lib.ig_sparse_decode_attn(p, p, p, 8, None, p, 1, 1, 24, 4, L.IG_BF16, f(1.0), p, None, None, 0, None) == L.IG_EINVAL
    assert lib.ig_sparse_decode_attn(ctypes.c_void_p(18), p, p, 8, None, p, 1, 1, 128, 4, L.IG_BF16, f(1.0), p, None,
                                     None, 0, None) == L.IG_EINVAL
    # cmax < 2, n > n_cap
    assert lib.ig_pool_touch(p, p, p, 1, 1, 4, 4, 4, 1, None, None, 0, None) == L.IG_EINVAL
    assert lib.ig_pool_touch(p, p, p, 1, 1, 5, 4, 4, 15, None, None, 0, None) == L.IG_EINVAL
    # a large selection needs the flag workspace
    assert lib.ig_pool_touch(p, p, p, 1, 64, 5000, 5000, 1000, 15, None, None, 0, None) == L.IG_EINVAL
    # full pool without a victim
    assert lib.ig_append_kv(p, p, p, p, p, p, p, None, 1, 1, 64, 8, 4, 4, L.IG_BF16, None, None) == L.IG_EINVAL
    # fused speculation: rows beyond 16 slices of 32768, or the head-average mode, are unsupported
    assert lib.ig_speculate(p, p, None, p, 1, 64, 1, 8, 600000, 600000, L.IG_BF16, f(1.0), L.IG_SEL_TOPK, f(0.0), 4,
                            0, p, p, 20000, None, 15, None, None, None, 600000, None, 0, None) == L.IG_EUNSUPPORTED
    # (the head average needs whole rows: a 100000-key row is sliced)
    assert lib.ig_speculate(p, p, None, p, 1, 64, 1, 8, 100000, 100000, L.IG_BF16, f(1.0), L.IG_SEL_HEADAVG, f(1.0), 4,
                            0, p, p, 4, None, 15, None, None, None, 100000, None, 0, None) == L.IG_EUNSUPPORTED
    # no workspace
    assert lib.ig_speculate(p, p, None, p, 1, 64, 1, 8, 40, 40, L.IG_BF16, f(1.0), L.IG_SEL_TOPK, f(0.0), 4, 0,
                            p, p, 4, p, 15, None, None, None, 40, None, 0, None) == L.IG_EINVAL
    # batch beyond the workspace stamp's range
    assert lib.ig_speculate(p, p, None, p, 70000, 64, 1, 8, 40, 40, L.IG_BF16, f(1.0), L.IG_SEL_TOPK, f(0.0), 4, 0,
                            p, p, 4, None, 15, None, None, None, 40, p, 1 << 30, None) == L.IG_EINVAL
    # the status query needs a workspace and somewhere to put the word
    assert lib.ig_workspace_status(None, 256, ctypes.byref(ctypes.c_uint32()), None, None) == L.IG_EINVAL
    assert lib.ig_workspace_status(p, 8, ctypes.byref(ctypes.c_uint32()), None, None) == L.IG_EINVAL
    # INT4 pool: d not a multiple of 32, rows past the record array, NULL records
    assert L.ig_int4_record_bytes(128) == 160 and L.ig_int4_record_bytes(64) == 96 and L.ig_int4_record_bytes(48) == 0
    assert lib.ig_quantize_kv(p, p, 1, 1, 48, 8, L.IG_BF16, 0, 8, None, p, 8, None) == L.IG_EINVAL
    assert lib.ig_quantize_kv(p, p, 1, 1, 64, 8, L.IG_BF16, 0, 8, None, p, 4, None) == L.IG_EINVAL
    assert lib.ig_quantize_kv(p, p, 1, 1, 64, 8, L.IG_BF16, 4, 8, None, p, 16, None) == L.IG_EINVAL
    assert lib.ig_quantize_kv(p, None, 1, 1, 64, 8, L.IG_BF16, 0, 8, None, p, 8, None) == L.IG_EINVAL
    assert lib.ig_gather_kv_int4(None, p, p, 1, 1, 64, 8, 4, L.IG_BF16, p, p, None) == L.IG_EINVAL
    assert lib.ig_gather_kv_int4(p, p, p, 1, 1, 40, 8, 4, L.IG_BF16, p, p, None) == L.IG_EINVAL
    # append: K without V
    assert lib.ig_append_kv(p, None, p, p, p, p, p, None, 1, 1, 64, 8, 4, 1, L.IG_BF16, None, None) == L.IG_EINVAL
    # host setup: m < d
    args = L.SkewArgs(0, 1, 8, 4, 16, None, None, None, None, 16, None, None, None, None, None, 1)
    assert lib.ig_skew_weights(ctypes.byref(args)) == L.IG_EINVAL


def test_workspace_sizes(lib):
    assert L.ig_workspace_size(L.IG_OP_REHEARSE, 8, 32, 4096, 128, 32, 2048, 0) > 0
    assert L.ig_workspace_size(L.IG_OP_ATTN, 1, 1, 0, 128, 0, 0, 16) == 0   # a single split needs none
    assert L.ig_workspace_size(L.IG_OP_ATTN, 1, 32, 0, 128, 0, 0, 5243) > 0
    assert L.ig_workspace_size(L.IG_OP_SELECT, 2, 3, 0, 0, 0, 100, 10) == 2 * 3 * 4


def test_speculation_workspace_holds_its_documented_regions(lib):
    """The speculation workspace holds (in this order, each 256-byte aligned) the status word and the
    shape stamp (256 bytes), two words per sequence (the rows' arrivals, then the counter flags) and
    the projection's split partial sums [ceil(D/512)][B][H*r] float32, then the slices' candidates when
    rows are sliced; its size only grows with n."""
    a256 = lambda v: (v + 255) // 256 * 256
    for B, H, D, r, n, max_out in [(8, 32, 4096, 32, 2048, 128), (16, 40, 5120, 32, 4352, 218),
                                   (1, 4, 256, 16, 256, 32), (20, 3, 384, 16, 600, 50), (4, 32, 4096, 32, 131072, 5243)]:
        need = 256 + a256(8 * B) + a256(-(-D // 512) * B * H * r * 4)
        sizes = [L.ig_workspace_size(L.IG_OP_SPECULATE, B, H, D, 128, r, nn, max_out) for nn in (max(1, n // 4), n)]
        assert sizes[1] >= need, (B, H, D, r, n)
        assert sizes[1] >= sizes[0], (B, H, D, r, n)

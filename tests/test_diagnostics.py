"""Host statistics of the speculation-fidelity diagnostic (recall@c, softmax mass, rank correlation),
pinned to their definitions by special cases and by a library routine (scipy's Spearman)."""
import numpy as np
import pytest

from sparse_attention_ig_amd.diagnostics import set_fidelity, spearman_rows


def test_spearman_matches_scipy_with_ties():
    st = pytest.importorskip("scipy.stats")
    g = np.random.default_rng(5)
    a = g.standard_normal((6, 80))
    b = a + g.standard_normal((6, 80)) * 0.7
    a[0, :20] = 0.25                       # a run of ties
    b[1] = np.round(b[1])                  # many ties on the other side
    r = spearman_rows(a, b)
    ref = np.array([st.spearmanr(a[i], b[i]).statistic for i in range(6)])
    assert np.abs(r - ref).max() < 1e-12


def test_spearman_monotone_and_reversed():
    x = np.linspace(-3, 3, 41)[None, :]
    assert spearman_rows(x, np.exp(x))[0] == pytest.approx(1.0)
    assert spearman_rows(x, -x ** 3)[0] == pytest.approx(-1.0)
    assert spearman_rows(x, np.zeros_like(x))[0] == 0.0     # constant row: no correlation defined -> 0


def _sets(sel, B=1, H=1, cap=8):
    idx = np.zeros((B, H, cap), np.int32)
    cnt = np.zeros((B, H), np.int32)
    idx[0, 0, :len(sel)] = sel
    cnt[0, 0] = len(sel)
    return idx, cnt


def test_set_fidelity_special_cases():
    n = 10
    logits = np.log(np.arange(1, n + 1, dtype=np.float64))[None, None, :]   # softmax weights j / 55
    best = [7, 8, 9]
    ti, tc = _sets(best)
    same = set_fidelity(*_sets([7, 8, 9]), ti, tc, logits, logits, n)
    assert same["recall"][0, 0] == 1.0
    assert same["mass_exact"][0, 0] == pytest.approx((8 + 9 + 10) / 55)
    assert same["mass_spec"][0, 0] == same["mass_exact"][0, 0]
    assert same["rho"][0, 0] == pytest.approx(1.0)
    disjoint = set_fidelity(*_sets([0, 1, 2]), ti, tc, -logits, logits, n)
    assert disjoint["recall"][0, 0] == 0.0
    assert disjoint["mass_spec"][0, 0] == pytest.approx((1 + 2 + 3) / 55)
    assert disjoint["rho"][0, 0] == pytest.approx(-1.0)
    part = set_fidelity(*_sets([1, 8, 9]), ti, tc, logits, logits, n)
    assert part["recall"][0, 0] == pytest.approx(2 / 3)
    every = set_fidelity(*_sets(list(range(n)), cap=n), *_sets(list(range(n)), cap=n), logits, logits, n)
    assert every["mass_spec"][0, 0] == pytest.approx(1.0)

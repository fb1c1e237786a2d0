"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own formula: hand-computed fixtures
(tests/golden, each citing its passage), closed forms (orthogonal-skew invariance, r = d
exactness, alpha = inf / k = n equal to dense attention), invariants (nesting in alpha, the
score separation of a top-k set, the e^-alpha mass bound, permutation invariance, counter sums),
a textbook library routine (torch scaled_dot_product_attention on CPU for dense attention) and
brute force over all subsets on tiny inputs.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as O
from tests.conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- storage decode / encode
def test_decode_known_bf16_patterns():
    # IEEE bfloat16 = top 16 bits of binary32
    bits = np.array([0x3F80, 0xC040, 0x3F81, 0x0000, 0x8000, 0x7F80, 0x4049], dtype=np.uint16)
    want = [1.0, -3.0, 1.0 + 2 ** -7, 0.0, -0.0, math.inf, 3.140625]
    got = O.decode(bits, "bf16")
    assert list(got) == want


def test_store_rounds_to_nearest_even():
    vals = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 3.0e38 * 10])
    got = O.store(vals, "bf16")
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 tie -> even (1+2^-6); just above a tie rounds up;
    # -2.5 exact; overflow of float32 -> inf
    assert list(got) == [0x3F80, 0x3F82, 0x3F81, 0xC020, 0x7F80]
    assert O.store(np.array([1.0 / 3.0]), "f32")[0] == np.float32(1.0 / 3.0)


# ---------------------------------------------------------------- skewing
def test_skew_rotation_hand_cases():
    for case in _load("skew_cases.json")["svd"]:
        A = O.skew_rotation(np.array([case["Q"]]))[0]
        np.testing.assert_allclose(A, np.array(case["expect_A"]), atol=1e-12)
        Qt = np.array(case["Q"]) @ A
        np.testing.assert_allclose(np.linalg.norm(Qt, axis=0), case["sigma"], atol=1e-12)


def test_skew_apply_hand_case():
    c = _load("skew_cases.json")["apply"]
    got = O.skew_apply(np.array(c["A"]), np.array(c["M"]))
    np.testing.assert_allclose(got, np.array(c["expect"]), atol=0)


def _power_sigma1(Q, iters=3000):
    v = np.ones(Q.shape[1]) / math.sqrt(Q.shape[1])
    for _ in range(iters):
        w = Q.T @ (Q @ v)
        v = w / np.linalg.norm(w)
    return float(np.linalg.norm(Q @ v))


@pytest.mark.parametrize("m,d", [(256, 64), (128, 128), (40, 16)])
def test_skew_rotation_is_the_svd_basis(m, d):
    """A orthogonal; Q~ = Q A = U Sigma: orthogonal columns with descending norms; the first norm
    is the spectral norm (power iteration); Frobenius norm preserved; canonical signs."""
    g = np.random.default_rng(7 + m + d)
    Q = g.standard_normal((m, d)) @ np.diag(np.linspace(3.0, 0.2, d)) @ np.linalg.qr(g.standard_normal((d, d)))[0]
    A = O.skew_rotation(Q[None])[0]
    np.testing.assert_allclose(A.T @ A, np.eye(d), atol=1e-12)
    Qt = Q @ A
    G = Qt.T @ Qt
    off = G - np.diag(np.diag(G))
    assert np.abs(off).max() <= 1e-9 * np.abs(G).max()
    norms = np.linalg.norm(Qt, axis=0)
    assert np.all(np.diff(norms) <= 1e-12)
    assert abs(norms[0] - _power_sigma1(Q)) <= 1e-9 * norms[0]
    assert abs(np.sum(norms ** 2) - np.sum(Q ** 2)) <= 1e-9 * np.sum(Q ** 2)
    piv = np.argmax(np.abs(A), axis=0)
    assert np.all(A[piv, np.arange(d)] > 0)


def test_skew_invariance_QK():
    """Closed form (a): skewing W_Q and W_K by the same orthogonal A leaves Q K^T unchanged
    (section 3.4, 'Skewed Partial Weights': A A^T = I)."""
    g = np.random.default_rng(11)
    H, d, D, N = 4, 64, 256, 50
    X = g.standard_normal((N, D))
    Wq = g.standard_normal((D, D)) / 16
    Wk = g.standard_normal((D, D)) / 16
    Xs = g.standard_normal((256, D))
    src = np.stack([(Xs @ Wq)[:, h * d:(h + 1) * d] for h in range(H)])
    A, Wq_s, Wk_s, _, _ = O.skew_weights(Wq, Wk, src)
    for h in range(H):
        sl = slice(h * d, (h + 1) * d)
        ref = (X @ Wq[:, sl]) @ (X @ Wk[:, sl]).T
        got = (X @ Wq_s[:, sl]) @ (X @ Wk_s[:, sl]).T
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10 * np.abs(ref).max())
    # skewing concentrates magnitude: the first skewed column of Q~ outweighs the last
    Qs = X @ Wq_s
    assert np.abs(Qs[:, 0]).sum() > np.abs(Qs[:, d - 1]).sum()


def test_bias_rotates_with_the_weight():
    g = np.random.default_rng(3)
    H, d, D = 2, 8, 16
    W = g.standard_normal((D, D))
    b = g.standard_normal(D)
    src = g.standard_normal((H, 20, d))
    A, Ws, _, bs, _ = O.skew_weights(W, None, src, bq=b)
    x = g.standard_normal(D)
    # (x W + b) A == x W~ + b~, per head
    np.testing.assert_allclose(O.skew_apply(A, x @ W + b), x @ Ws + bs, atol=1e-12)


# ---------------------------------------------------------------- channel pick
def test_partial_weight_index_hand_cases():
    for c in _load("channel_pick_cases.json")["cases"]:
        chan = O.partial_weight_index(np.array(c["Wq"]), np.array(c["K"]), c["H"], c["d"], c["r"])
        assert chan.tolist() == c["expect"], c.get("note")


def test_partial_weight_index_brute_force():
    """The picked set maximises the summed column score over all r-subsets (tiny, no ties)."""
    g = np.random.default_rng(5)
    H, d, r, D = 3, 7, 3, 5
    Wq = g.standard_normal((D, H * d))
    K = g.standard_normal((2, H, 4, d))
    chan = O.partial_weight_index(Wq, K, H, d, r)
    for h in range(H):
        colscore = [sum(abs(Wq[i, h * d + c]) for i in range(D))
                    + sum(abs(K[b, h, j, c]) for b in range(2) for j in range(4)) for c in range(d)]
        best = max(itertools.combinations(range(d), r), key=lambda S: sum(colscore[c] for c in S))
        assert tuple(chan[h]) == best


def test_partial_sizes_printed_ratio():
    """Printed pin: with a partial ratio of 0.3 the partial key cache is 0.3 x 0.5 = 15% of the
    KV cache (section 3.4, step 3 "Extract partial matrices")."""
    B, H, n, d, r = 1, 2, 5, 10, 3
    K = np.zeros((B, H, n, d), dtype=np.uint16)
    chan = np.array([[0, 4, 9], [1, 2, 3]], dtype=np.int32)
    Kp = O.partial_key_cache(K, chan)
    assert Kp.nbytes / (2 * K.nbytes) == pytest.approx(0.15)


# ---------------------------------------------------------------- rehearsal
def _tiny_setup(seed=0, B=2, H=3, d=8, D=None, n=11, r=3):
    g = np.random.default_rng(seed)
    D = D or H * d
    x = g.standard_normal((B, D))
    Wq = g.standard_normal((D, H * d)) / math.sqrt(D)
    K = g.standard_normal((B, H, n, d))
    return g, x, Wq, K


def test_rehearse_brute_force_loops():
    g, x, Wq, K = _tiny_setup()
    B, H, n, d = K.shape
    r = 3
    chan = np.array([sorted(g.choice(d, r, replace=False)) for _ in range(H)], dtype=np.int32)
    Wp = O.pack_partial_weight(Wq, chan, d)
    Kp = O.partial_key_cache(K, chan)
    bias = g.standard_normal(H * r)
    qp, s = O.rehearse(x, Wp, Kp, n, H, r, 0.5, bq_part=bias)
    for b in range(B):
        for h in range(H):
            for c in range(r):
                ch = h * d + int(chan[h][c])
                want = sum(x[b, i] * Wq[i, ch] for i in range(x.shape[1])) + bias[h * r + c]
                assert qp[b, h, c] == pytest.approx(want, rel=1e-12, abs=1e-12)
            for j in range(n):
                want = 0.5 * sum(qp[b, h, c] * K[b, h, j, int(chan[h][c])] for c in range(r))
                assert s[b, h, j] == pytest.approx(want, rel=1e-12, abs=1e-12)


def test_rehearse_partial_is_subsum_of_full_dot():
    """Same channel indices for query and key make the partial score a sub-sum of the full
    product q~ . k~ (section 3.4, 'same column indices' paragraph)."""
    g, x, Wq, K = _tiny_setup(seed=1)
    B, H, n, d = K.shape
    chan = np.array([[0, 2, 5], [1, 3, 7], [4, 5, 6]], dtype=np.int32)
    _, s = O.rehearse(x, O.pack_partial_weight(Wq, chan, d), O.partial_key_cache(K, chan), n, H, 3, 1.0)
    q = (x @ Wq).reshape(B, H, d)
    for b in range(B):
        for h in range(H):
            terms = q[b, h][None, :] * K[b, h]           # [n][d] per-channel products
            np.testing.assert_allclose(s[b, h], terms[:, chan[h]].sum(axis=1), atol=1e-12)


def test_rehearse_r_equals_d_gives_exact_logits():
    """Closed form (b): with every channel kept, the speculated score is the exact scaled logit,
    and through the skew invariance it equals the unskewed q . k."""
    g = np.random.default_rng(2)
    B, H, d, n = 2, 2, 16, 9
    D = H * d
    x = g.standard_normal((B, D))
    Wq = g.standard_normal((D, D)) / math.sqrt(D)
    Kraw = g.standard_normal((B, H, n, d))
    A, Wq_s, _, _, _ = O.skew_weights(Wq, None, g.standard_normal((H, 30, d)))
    Ks = np.stack([np.stack([Kraw[b, h] @ A[h] for h in range(H)]) for b in range(B)])
    chan = np.tile(np.arange(d, dtype=np.int32), (H, 1))
    _, s = O.rehearse(x, O.pack_partial_weight(Wq_s, chan, d), O.partial_key_cache(Ks, chan), n, H, d, 0.25)
    q = (x @ Wq).reshape(B, H, d)
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(s[b, h], 0.25 * Kraw[b, h] @ q[b, h], atol=1e-12)


# ---------------------------------------------------------------- selection
def test_select_hand_cases():
    cases = _load("select_cases.json")
    for c in cases["threshold"]:
        a = math.inf if c["alpha"] == "inf" else c["alpha"]
        got = O.select_threshold(np.array(c["scores"]), a, c["max_sel"])
        assert got.tolist() == c["expect"], c.get("note")
    for c in cases["topk"]:
        assert O.select_topk(np.array(c["scores"]), c["k"]).tolist() == c["expect"]
    for c in cases["head_average"]:
        idx, cnt = O.select_head_average(np.array([c["scores"]]), c["alpha"], c["max_sel"])
        got = [idx[0, h, :cnt[0, h]].tolist() for h in range(len(c["scores"]))]
        assert got == c["expect"], c.get("note")


def _brute_threshold(s, alpha):
    m = max(s)
    return [j for j in range(len(s)) if s[j] >= m - alpha]


@pytest.mark.parametrize("seed", range(6))
def test_select_brute_force_and_invariants(seed):
    g = np.random.default_rng(100 + seed)
    n = int(g.integers(1, 300))
    s = np.round(g.standard_normal(n) * 3, 1)        # rounding makes ties common
    alphas = [0.0, 0.3, 1.0, 4.0, 5.0, 9.0, math.inf]
    prev = set()
    for a in alphas:
        S = O.select_threshold(s, a).tolist()
        assert S == _brute_threshold(list(s), a)
        assert prev <= set(S)                          # nested, monotone in alpha
        prev = set(S)
    assert O.select_threshold(s, math.inf).tolist() == list(range(n))
    assert O.select_threshold(s, 0.0).tolist() == [j for j in range(n) if s[j] == s.max()]
    for k in [1, 2, 5, n // 2 + 1, n, n + 3]:
        S = O.select_topk(s, k).tolist()
        assert len(S) == min(k, n)
        inside = set(S)
        # separation: every kept row beats every dropped row, ties broken towards the lower index
        for i in inside:
            for j in range(n):
                if j not in inside:
                    assert s[i] > s[j] or (s[i] == s[j] and i < j)
    assert O.select_topk(s, 1).tolist() == [int(np.flatnonzero(s == s.max())[0])]


def test_select_cap_keeps_top_of_threshold_set():
    g = np.random.default_rng(9)
    s = g.standard_normal(200)
    full = set(O.select_threshold(s, 2.5).tolist())
    capped = O.select_threshold(s, 2.5, max_sel=10).tolist()
    assert len(full) > 10 and len(capped) == 10 and set(capped) <= full
    assert set(capped) == set(O.select_topk(s, 10).tolist())
    # the output capacity clamps the same way
    assert O.select_threshold(s, 2.5, max_out=7).tolist() == O.select_topk(s, 7).tolist()


def test_topk_brute_force_subsets():
    """Tiny rows: the top-k set is the lexicographically best k-subset by (score sum desc, indices)."""
    g = np.random.default_rng(4)
    for _ in range(20):
        n = int(g.integers(1, 8))
        s = np.round(g.standard_normal(n), 0)
        for k in range(1, n + 1):
            best = max(itertools.combinations(range(n), k),
                       key=lambda S: (sorted((s[j] for j in S), reverse=True), [-j for j in S]))
            assert tuple(O.select_topk(s, k).tolist()) == best


# ---------------------------------------------------------------- attention
def test_attention_hand_cases():
    cases = _load("attention_cases.json")
    for c in cases["cases"]:
        o, lse = O.attention_rows(np.array(c["q"]), np.array(c["K"]), np.array(c["V"]), c["scale"])
        np.testing.assert_allclose(o, c["expect_out"], atol=1e-14)
        assert lse == pytest.approx(c["expect_lse"], abs=1e-14)
    pr = cases["printed_ratio"]
    # two tokens, logits m and m - alpha: the second weighs e^-alpha of the first
    q = np.array([1.0])
    K = np.array([[3.0], [3.0 - pr["alpha"]]])
    V = np.array([[1.0], [0.0]])
    o, _ = O.attention_rows(q, K, V, 1.0)
    p1 = o[0]
    ratio = (1 - p1) / p1
    assert ratio == pytest.approx(pr["ratio_printed"], abs=5e-5)
    assert 1 / ratio == pytest.approx(pr["inverse_printed"], abs=0.05)


def test_dense_attention_matches_torch_sdpa():
    """Dense attention agrees with a textbook library routine (torch SDPA on CPU, float64)."""
    import torch
    g = np.random.default_rng(8)
    B, H, n, d = 2, 3, 37, 16
    q = g.standard_normal((B, H, d))
    K = g.standard_normal((B, H, n, d))
    V = g.standard_normal((B, H, n, d))
    o, _ = O.dense_decode_attn(q, K, V, n, 0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[:, :, None, :], torch.tensor(K), torch.tensor(V), scale=0.3)[:, :, 0, :]
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)


def test_sparse_equals_dense_when_everything_selected():
    """Closed form (c): alpha = inf or k = n selects every row, and the sparse output is the
    dense softmax(qK^T)V."""
    g = np.random.default_rng(12)
    B, H, n, d = 2, 2, 50, 8
    q = g.standard_normal((B, H, d))
    K = g.standard_normal((B, H, n, d))
    V = g.standard_normal((B, H, n, d))
    s = np.einsum("bhd,bhnd->bhn", q, K)
    dense = O.dense_decode_attn(q, K, V, n, 0.5)
    for idx, cnt in [O.select(s, "threshold", alpha=math.inf), O.select(s, "topk", k=n)]:
        o, lse = O.sparse_decode_attn(q, K, V, idx, cnt, 0.5)
        np.testing.assert_allclose(o, dense[0], atol=1e-13)
        np.testing.assert_allclose(lse, dense[1], atol=1e-13)


def test_attention_permutation_invariance():
    """Order of cache rows is free if K and V of a token stay together (section 3.4, pool
    paragraph): permuting rows and remapping indices leaves the output unchanged."""
    g = np.random.default_rng(13)
    B, H, n, d = 1, 2, 30, 8
    q = g.standard_normal((B, H, d))
    K = g.standard_normal((B, H, n, d))
    V = g.standard_normal((B, H, n, d))
    idx, cnt = O.select(np.einsum("bhd,bhnd->bhn", q, K), "topk", k=9)
    perm = g.permutation(n)
    inv = np.argsort(perm)
    o1, _ = O.sparse_decode_attn(q, K, V, idx, cnt, 1.0)
    o2, _ = O.sparse_decode_attn(q, K[:, :, perm], V[:, :, perm], inv[idx], cnt, 1.0)
    np.testing.assert_allclose(o1, o2, atol=1e-13)


def test_threshold_dropped_mass_bound():
    """With exact scores (r = d) and threshold alpha, every dropped token weighs at most e^-alpha
    of the maximum, so |o_dense - o_sparse|_inf <= 2 * m_d * max|V| with the dropped mass
    m_d <= (n - c) e^-alpha p_max (section 3.4 step 3)."""
    g = np.random.default_rng(14)
    B, H, n, d = 1, 4, 400, 16
    q = g.standard_normal((B, H, d)) * 2
    K = g.standard_normal((B, H, n, d))
    V = g.standard_normal((B, H, n, d))
    scale, alpha = 0.5, 4.0
    s = scale * np.einsum("bhd,bhnd->bhn", q, K)
    idx, cnt = O.select(s, "threshold", alpha=alpha)
    od, _ = O.dense_decode_attn(q, K, V, n, scale)
    os_, _ = O.sparse_decode_attn(q, K, V, idx, cnt, scale)
    for h in range(H):
        p = np.exp(s[0, h] - s[0, h].max())
        p /= p.sum()
        md_bound = (n - cnt[0, h]) * math.exp(-alpha) * p.max()
        assert np.abs(od[0, h] - os_[0, h]).max() <= 2 * md_bound * np.abs(V[0, h]).max() + 1e-12


def test_gather_kv_rows():
    K = np.arange(2 * 1 * 5 * 2).reshape(2, 1, 5, 2)
    V = -K
    idx = np.array([[[4, 1, 0]], [[2, 0, 0]]], dtype=np.int32)
    cnt = np.array([[2], [1]], dtype=np.int32)
    Kc, Vc = O.gather_kv(K, V, idx, cnt, 3)
    assert Kc[0, 0].tolist() == [[8, 9], [2, 3], [0, 0]]
    assert Kc[1, 0].tolist() == [[14, 15], [0, 0], [0, 0]]
    assert (Vc == -Kc).all()


# ---------------------------------------------------------------- counters / pool
def test_counter_hand_cases():
    for c in _load("counter_cases.json")["cases"]:
        C = np.array(c["C"], dtype=np.uint32)
        idx = np.array(c["idx"], dtype=np.int32)
        cnt = np.array(c["count"], dtype=np.int32)
        C2, v = O.pool_touch(C, idx, cnt, c["n"], c["cmax"], want_victim=True)
        assert C2.tolist() == c["expect_C"], c.get("note")
        assert v.tolist() == c["expect_victim"], c.get("note")


def test_counter_sums_and_halving():
    g = np.random.default_rng(15)
    B, H, n, cmax = 3, 4, 60, 1000
    s = g.standard_normal((B, H, n))
    idx, cnt = O.select(s, "topk", k=7)
    C = np.zeros((B, n), dtype=np.uint32)
    C2, _ = O.pool_touch(C, idx, cnt, n, cmax)
    assert C2.sum() == cnt.sum()                       # sum of increments = sum of counts
    # forced saturation: cmax small, repeated steps keep every counter below cmax and >= 0
    C = np.zeros((B, n), dtype=np.uint32)
    for _ in range(12):
        C, v = O.pool_touch(C, idx, cnt, n, 15, want_victim=True)
        assert (C < 15).all()
        for b in range(B):
            assert C[b, v[b]] == C[b, :n].min() and (C[b, :v[b]] > C[b, v[b]]).all()


def test_pool_append_slots():
    B, H, cap, d, r = 2, 1, 3, 2, 1
    K = np.zeros((B, H, cap, d), dtype=np.uint16)
    V = np.zeros_like(K)
    Kp = np.zeros((B, H, cap, r), dtype=np.uint16)
    C = np.full((B, cap), 9, dtype=np.uint32)
    chan = np.array([[1]], dtype=np.int32)
    kn = np.array([[[5, 6]], [[7, 8]]], dtype=np.uint16)
    slots, n2 = O.pool_append(K, V, Kp, C, chan, kn, kn, n=2)
    assert slots.tolist() == [2, 2] and n2 == 3 and C[:, 2].tolist() == [0, 0]
    assert Kp[0, 0, 2].tolist() == [6] and K[1, 0, 2].tolist() == [7, 8]
    slots, n3 = O.pool_append(K, V, Kp, C, chan, kn, kn, n=3, victim=np.array([0, 1]))
    assert slots.tolist() == [0, 1] and n3 == 3 and C[0, 0] == 0 and C[1, 1] == 0


# ---------------------------------------------------------------- one whole layer-step
def _step_inputs(case, common):
    """Arrays of a decode_step golden case: x [1][D], Wq_part [D][H*r], Kp [1][H][n][r], q [1][H][d],
    K, V [1][H][n][d], counters [1][n]."""
    H = case["H"]
    heads = ["head0", "head1"][:H]
    def per_head(key):
        return np.array([[case.get(f"{key}_{hd}", common.get(f"{key}_{hd}")) for hd in heads]], dtype=float)
    x = np.array(common["x"], dtype=float)
    W = np.array(case["Wq_part"], dtype=float)
    bq = None if case["bq_part"] is None else np.array(case["bq_part"], dtype=float)
    return x, W, bq, per_head("Kp"), per_head("q"), per_head("K"), per_head("V"), np.array(case["C"], dtype=np.uint32)


def test_decode_step_golden_cases():
    """decode_step chains the steps and forwards every argument (bias, cap, output capacity, mode,
    cmax, victim): hand-computed layer-steps (tests/golden/decode_step_cases.json)."""
    g = _load("decode_step_cases.json")
    common = g["common"]
    for case in g["cases"]:
        x, W, bq, Kp, q, K, V, C = _step_inputs(case, common)
        res = O.decode_step(x, W, Kp, q, K, V, C, n=common["n"], H=case["H"], r=2, scale=common["scale"],
                            mode=case["mode"], alpha=case.get("alpha", math.inf), k=case.get("k", 0),
                            max_sel=case["max_sel"], max_out=case["max_out"], cmax=case["cmax"], bq_part=bq,
                            want_victim=True)
        e = case["expect"]
        name = case["name"]
        for key in ("q_part", "scores", "out", "lse"):
            assert np.allclose(res[key], np.array(e[key]), rtol=0, atol=1e-12), (name, key, res[key])
        assert res["count"].tolist() == e["count"], (name, res["count"])
        for h in range(case["H"]):
            c = int(res["count"][0, h])
            assert res["idx"][0, h, :c].tolist() == e["idx"][0][h], (name, h)
        assert res["counters"].tolist() == e["counters"], (name, res["counters"])
        assert res["victim"].tolist() == e["victim"], (name, res["victim"])


# ---------------------------------------------------------------- the pins catch planted mistakes
def test_pins_catch_planted_mistakes(monkeypatch):
    """Each planted mistake in a copy of an oracle step makes one of the pins above fail."""
    import oracle.oracle as mod
    real_rehearse, real_thr, real_att, real_touch = mod.rehearse, mod.select_threshold, mod.attention_rows, mod.pool_touch

    def no_scale(x, Wp, Kp, n, H, r, scale, bq_part=None):
        return real_rehearse(x, Wp, Kp, n, H, r, 1.0, bq_part)

    def strict_cut(s, alpha, max_sel=0, max_out=0):  # sign error: cut at max + alpha
        s = np.asarray(s, dtype=float)
        return np.flatnonzero(s >= s.max() + alpha).astype(np.int32)

    def no_value_weighting(q, K, V, scale):
        o, l = real_att(q, K, V, scale)
        return np.asarray(V, dtype=float).mean(axis=0) if len(V) else o, l

    def no_halving(C, idx, count, n, cmax, want_victim=False):
        C = np.array(C, dtype=np.int64)
        for b in range(C.shape[0]):
            for h in range(count.shape[1]):
                for j in idx[b, h, :int(count[b, h])]:
                    C[b, int(j)] += 1
        v = np.argmin(C[:, :n], axis=1).astype(np.int32) if want_victim else None
        return np.minimum(C, cmax).astype(np.uint32), v

    real_step = mod.decode_step

    def bias_dropped(*a, **kw):  # the bias is not forwarded to the partial query
        return real_step(*a, **{**kw, "bq_part": None})

    def cap_dropped(*a, **kw):  # the per-layer cap is not forwarded to the selection
        return real_step(*a, **{**kw, "max_sel": 0})

    def capacity_dropped(*a, **kw):  # the output capacity is not forwarded
        return real_step(*a, **{**kw, "max_out": 0})

    real_avg = mod.select_head_average

    def avg_rounded_down(scores, alpha, max_sel=0, max_out=0):  # head average rounded down
        B, H, n = scores.shape
        counts = [len(mod.select_threshold(scores[0, h], alpha)) for h in range(H)]
        if sum(counts) % H == 0:
            return real_avg(scores, alpha, max_sel, max_out)
        return real_avg(scores, alpha, max(1, sum(counts) // H), max_out)

    planted = [("rehearse", no_scale, test_rehearse_brute_force_loops),
               ("select_threshold", strict_cut, test_select_hand_cases),
               ("attention_rows", no_value_weighting, test_attention_hand_cases),
               ("pool_touch", no_halving, test_counter_hand_cases),
               ("rehearse", no_scale, test_decode_step_golden_cases),
               ("pool_touch", no_halving, test_decode_step_golden_cases),
               ("decode_step", bias_dropped, test_decode_step_golden_cases),
               ("decode_step", cap_dropped, test_decode_step_golden_cases),
               ("decode_step", capacity_dropped, test_decode_step_golden_cases),
               ("select_head_average", avg_rounded_down, test_select_hand_cases)]
    for name, fake, pin in planted:
        monkeypatch.setattr(mod, name, fake)
        with pytest.raises(AssertionError):
            pin()
        monkeypatch.undo()

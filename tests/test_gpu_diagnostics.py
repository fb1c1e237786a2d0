"""GPU: the speculation-fidelity diagnostic against the same statistics computed from the oracle's own
pipeline (its speculated sets and scores) and the oracle's exact logits (the whole skewed query weight
against the whole key cache, InfiniGen summary, arXiv 2406.19707, paper-graph-ui, section 3.4).

Rows whose c-th and (c+1)-th score (speculated or exact, oracle's float64) lie within 1e-4 of each
other may pick either row on either side; there only the rank correlation is compared."""
import math

import numpy as np
import pytest

from oracle import oracle as O
from sparse_attention_ig_amd import gen
from sparse_attention_ig_amd.diagnostics import set_fidelity
from tests import harness
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_ig_amd import _lib as L
    L.load()
    yield


def _clear_cut(s: np.ndarray, c: int) -> bool:
    v = np.sort(s)[::-1]
    return c >= len(v) or v[c - 1] - v[c] > 1e-4 * max(1.0, abs(v[c - 1]))


def test_fidelity_matches_oracle_statistics():
    from sparse_attention_ig_amd.diagnostics import speculation_fidelity
    base = gen.llama2_13b(n=300, B=2, n_cap=306)
    spec = gen.Spec(**{**base.__dict__, "H": 8, "heavy": 6})
    layers, steps = 3, 3
    max_out = int(math.ceil(0.05 * spec.cap))
    say(f"[fidelity] layers={layers} steps={steps} B={spec.B} H={spec.H} n0={spec.n}")
    xs, lib_in, new = harness.pipeline_setup(spec, layers, steps, harness.lib_inputs)
    _, ora_in, _ = harness.pipeline_setup(spec, layers, steps, harness.oracle_inputs)
    res = speculation_fidelity(lib_in, xs, max_out, new_rows=new)
    say("[fidelity] gpu done")
    trace, _ = harness.oracle_pipeline(spec, xs, ora_in, new, max_out)
    dt = spec.dtype
    compared = 0
    for t in range(steps):
        n = trace[t]["n"]
        c = min(max_out, int(math.ceil(0.05 * n)))
        for l in range(1, layers):
            K = ora_in[l].K.copy()
            for i in range(t):                      # the rows appended before step t (no eviction here)
                K[:, :, spec.n + i] = new[i][l][0]
            _, ex = O.rehearse(O.decode(xs[t, l], dt), O.decode(ora_in[l].extra["Wq_s"], dt), O.decode(K, dt),
                               n, spec.H, spec.d, spec.softmax_scale)
            ti, tc = O.select(ex, "topk", k=c, max_out=max_out)
            ref = set_fidelity(trace[t]["idx"][l], trace[t]["count"][l], ti, tc, trace[t]["scores"][l], ex, n)
            got = {k: v[t] for k, v in res["raw"][l].items()}
            assert np.abs(got["rho"] - ref["rho"]).max() <= 1e-3, (t, l)
            for b in range(spec.B):
                for h in range(spec.H):
                    if _clear_cut(trace[t]["scores"][l][b, h, :n], c) and _clear_cut(ex[b, h, :n], c):
                        compared += 1
                        assert got["recall"][b, h] == ref["recall"][b, h], (t, l, b, h)
                        assert abs(got["mass_spec"][b, h] - ref["mass_spec"][b, h]) <= 1e-4, (t, l, b, h)
                        assert abs(got["mass_exact"][b, h] - ref["mass_exact"][b, h]) <= 1e-4, (t, l, b, h)
    assert compared >= steps * (layers - 1) * spec.B * spec.H // 2
    assert 0.0 <= res["recall_mean"] <= 1.0 and res["mass_spec"] <= res["mass_exact"] + 1e-6

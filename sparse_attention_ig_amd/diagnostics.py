"""Speculation fidelity: how much of each layer's exact top-c set the speculation recovers.

The InfiniGen summary (arXiv 2406.19707, paper-graph-ui) names the accuracy of the speculated
attention pattern as the method's weak point (section 6 "Limitations") and its direct measurement
as a next step (section 7 "Implications").  This diagnostic measures it on the cross-layer decode
pipeline.  At every decode step t and layer l >= 1:

  speculated set S   the pipeline's selection for layer l, taken at layer l-1 from x_{l-1}(t) with
                     layer l's partial weight (r channels) and partial key cache, with its scores;
  exact logits       scale * q . K over the same n rows for layer l's own query q = x_l(t) W~_Q
                     (every channel), computed by the library's kernels: ig_rehearse with the whole
                     skewed query weight as the "partial" weight and the whole key cache as the
                     "partial" cache (r = d), then ig_select top-c for the exact set T;
  recall@c           |S intersect T| / |T| per (b, h);
  attention mass     sum of the exact softmax weights over S, beside the same sum over T (the most
                     any c rows can hold);
  rank correlation   Spearman correlation of the speculated and the exact logits over the n rows.

The statistics (set intersection, ranks, softmax mass) are host-side bookkeeping of the diagnostic;
they are not steps of the decode path.  The pipeline's attention half keeps each layer's step-0 query
(a property of the synthetic workload); the exact logits use x_l(t), the query a model would form.
"""
from __future__ import annotations

import argparse
import json
import math
import sys
from typing import Dict, List, Sequence

import numpy as np

from . import _lib as L
from . import gen


def spearman_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Spearman rank correlation of each row of a with the same row of b (ties get average ranks)."""
    def ranks(m):
        m = np.asarray(m, dtype=np.float64)
        order = np.argsort(m, axis=1, kind="stable")
        srt = np.take_along_axis(m, order, axis=1)
        r = np.empty_like(m)
        for i in range(m.shape[0]):
            # average rank over each run of equal values
            v = srt[i]
            starts = np.flatnonzero(np.r_[True, v[1:] != v[:-1]])
            ends = np.r_[starts[1:], len(v)]
            avg = (starts + ends - 1) / 2.0
            r[i, order[i]] = np.repeat(avg, ends - starts)
        return r
    ra, rb = ranks(a), ranks(b)
    ra -= ra.mean(axis=1, keepdims=True)
    rb -= rb.mean(axis=1, keepdims=True)
    den = np.sqrt((ra * ra).sum(1) * (rb * rb).sum(1))
    return np.where(den > 0, (ra * rb).sum(1) / np.where(den > 0, den, 1.0), 0.0)


def set_fidelity(spec_idx, spec_cnt, true_idx, true_cnt, spec_logits, exact_logits, n: int) -> Dict[str, np.ndarray]:
    """Per-(b, h) recall@c, softmax mass of the speculated and of the exact set, and rank correlation.
    idx [B][H][>=count], count [B][H], logits [B][H][>=n] (host arrays)."""
    B, H = spec_cnt.shape
    e = exact_logits[..., :n].astype(np.float64)
    p = np.exp(e - e.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    recall = np.zeros((B, H))
    mass_s = np.zeros((B, H))
    mass_t = np.zeros((B, H))
    for b in range(B):
        for h in range(H):
            t = true_idx[b, h, :true_cnt[b, h]].astype(np.int64)
            s = spec_idx[b, h, :spec_cnt[b, h]].astype(np.int64)
            recall[b, h] = len(np.intersect1d(t, s)) / max(1, len(t))
            mass_s[b, h] = p[b, h, s].sum()
            mass_t[b, h] = p[b, h, t].sum()
    rho = spearman_rows(spec_logits[..., :n].reshape(B * H, n), e.reshape(B * H, n)).reshape(B, H)
    return {"recall": recall, "mass_spec": mass_s, "mass_exact": mass_t, "rho": rho}


class ExactTopk:
    """Exact logits and top-c of one layer's full query against its whole key cache (GPU)."""

    def __init__(self, host, max_out: int):
        import torch
        from .runtime import to_device
        s = host.spec
        self.spec = s
        self.W = to_device(np.ascontiguousarray(host.extra["Wq_s"].T))   # [H*d][D]: every channel
        dv = "cuda"
        self.q = torch.empty((s.B, s.H, s.d), dtype=torch.float32, device=dv)
        self.logits = torch.empty((s.B, s.H, s.cap), dtype=torch.float32, device=dv)
        self.idx = torch.empty((s.B, s.H, max_out), dtype=torch.int32, device=dv)
        self.count = torch.empty((s.B, s.H), dtype=torch.int32, device=dv)
        self.ws = torch.empty(max(16, L.ig_workspace_size(L.IG_OP_REHEARSE, s.B, s.H, s.D, s.d, s.d, s.cap, 0)),
                              dtype=torch.uint8, device=dv)
        self.max_out = max_out

    def __call__(self, x, K, n: int, c: int):
        s = self.spec
        L.ig_rehearse(x, self.W, K, n, s.softmax_scale, q_part=self.q, scores=self.logits, ld=s.cap, ws=self.ws)
        L.ig_select(self.logits, "topk", self.max_out, n=n, k=c, idx=self.idx, count=self.count)
        return self.idx, self.count, self.logits


def speculation_fidelity(hosts: Sequence, xs: np.ndarray, max_out: int, *, new_rows=None,
                         same_input: bool = False) -> Dict:
    """Runs the decode pipeline over xs [steps][layers][B][D] and measures every layer l >= 1 at every
    step, before the step's new token is appended.  ``new_rows[t][l]`` = (k, v) rows to append
    (default: the generator's draws).  ``same_input``: the speculation for layer l uses layer l's own
    input x_l(t) instead of x_{l-1}(t), which isolates the error of the partial channels from that of
    the cross-layer input."""
    import torch
    from .pipeline import DecodePipeline
    from .runtime import to_device, to_host
    spec = hosts[0].spec
    nl, steps = len(hosts), xs.shape[0]
    pipe = DecodePipeline(list(hosts), max_out=max_out)
    for lay in pipe.layers[1:]:
        lay.keep_scores = True
    exact = [None] + [ExactTopk(h, max_out) for h in hosts[1:]]
    rec: List[Dict[str, List[np.ndarray]]] = [dict() for _ in range(nl)]
    for t in range(steps):
        n, c = pipe.n, pipe.topk()
        xd = [to_device(xs[t, l]) for l in range(nl)]
        pipe.step(xd[1:] + xd[-1:] if same_input else xd, append=False)
        for l in range(1, nl):
            lay = pipe.layers[l]
            ti, tc, tl = exact[l](xd[l], lay.K, n, c)
            torch.cuda.synchronize()
            f = set_fidelity(to_host(lay.idx), to_host(lay.count), to_host(ti), to_host(tc), to_host(lay.scores),
                             to_host(tl), n)
            for k, v in f.items():
                rec[l].setdefault(k, []).append(v)
        rows = new_rows[t] if new_rows is not None else [gen.draw_new_rows(spec, l, t) for l in range(nl)]
        pipe.append([to_device(r[0]) for r in rows], [to_device(r[1]) for r in rows])
    per_layer = {}
    for l in range(1, nl):
        st = {k: np.stack(v) for k, v in rec[l].items()}   # [steps][B][H]
        per_layer[l] = {"recall_mean": float(st["recall"].mean()), "recall_p10": float(np.percentile(st["recall"], 10)),
                        "mass_spec": float(st["mass_spec"].mean()), "mass_exact": float(st["mass_exact"].mean()),
                        "rho_mean": float(st["rho"].mean())}
    agg = {k: float(np.mean([v[k] for v in per_layer.values()])) for k in next(iter(per_layer.values()))}
    return {"per_layer": per_layer, **agg, "raw": rec}


def main() -> int:
    ap = argparse.ArgumentParser(description="speculation fidelity of the cross-layer decode pipeline")
    ap.add_argument("--layers", type=int, default=6)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--n", type=int, default=4096)
    ap.add_argument("--r", type=int, default=32, help="partial channels per head (8, 16, 32, 64 or 128)")
    ap.add_argument("--same-input", action="store_true",
                    help="speculate each layer from its own input instead of the previous layer's")
    args = ap.parse_args()
    import torch
    if not torch.cuda.is_available():
        print("the diagnostic runs the decode pipeline on the GPU", file=sys.stderr)
        return 1
    L.load()
    from .runtime import prepare_layer
    base = gen.llama2_13b(n=args.n, B=args.batch, n_cap=args.n + max(256, args.steps))
    spec = gen.Spec(**{**base.__dict__, "r": args.r})
    xs = gen.pipeline_x(spec, args.layers, args.steps)
    hosts = []
    for l in range(args.layers):
        print(f"[fidelity] preparing layer {l}", file=sys.stderr, flush=True)
        hosts.append(prepare_layer(spec, l, lay=gen.draw_layer(spec, l, x_bits=xs[0, l], with_wk=False)))
    res = speculation_fidelity(hosts, xs, int(math.ceil(0.05 * spec.cap)), same_input=args.same_input)
    res.pop("raw")
    r4 = lambda v: round(v, 4)
    src = "x_l (same layer)" if args.same_input else "x_{l-1} (previous layer)"
    out = {"workload": f"llama2-13b-shaped pipeline B{spec.B} H{spec.H} d{spec.d} r{spec.r} n{spec.n} top-5%",
           "speculation_input": src,
           "layers": args.layers, "steps": args.steps,
           **{k: r4(v) for k, v in res.items() if k != "per_layer"},
           "per_layer": {l: {k: r4(v) for k, v in d.items()} for l, d in res["per_layer"].items()}}
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

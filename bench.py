#!/usr/bin/env python3
"""Decode-step benchmark of the InfiniGen hot path on one MI355X.

Default workload: the long-context Llama-2-7B-shaped decode layer (hidden 4096, 32 heads of 128,
batch 4, context 131072, 32 partial channels, bf16 storage, fp32 accumulation), top 4% of the
context (5243 rows) per head, all KV resident in HBM -- the largest of the single-GPU workloads.
One step = one decode step through ``--layers`` distinct layer buffers (distinct HBM buffers with
the same contents, so that the 256 MB Infinity Cache cannot serve the working set; by default the
model's 32 layers, as many as fit in 96 GB: 9 at the default workload), each running the whole hot
path: partial query, speculated scores, selection, counters (the speculation for layer l+1) and the
sparse attention of layer l, one ig_decode_layer call per layer (the first layer's speculation and
the last layer's attention run alone).

Prints one JSON line: tokens/s per layer (= batch x layers x steps / time), the roofline of the
dominant call (algorithmic bytes per call over its average duration from HIP events, against
8 TB/s), the CPU oracle timed on a bounded sample of the same workload on the host's cores, and
as extra keys the OPT-6.7B-shaped layer (B8, n2048, top-128), the 40-layer Llama-2-13B pipeline
and the OPT-30B host-pool figures (host-link GB/s, overlap ratio, eviction at the 80% pool limit).
"""
from __future__ import annotations

import argparse
import faulthandler
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode step tokens/s per layer (rehearse+select+sparse attn) + % HBM peak"


def alg_bytes(spec, c: float) -> dict:
    """Algorithmic bytes of one layer-step by call (c = mean selected rows per head).  Per layer-step:
    Wq_part D*H*r*s + x B*D*s + Kp B*H*n*r*s + selected K and V B*H*c*2*d*s + q B*H*d*s + o B*H*d*4
    + idx and counters 2*B*H*c*4; the scores' float32 round trip of the six-call path is an
    implementation cost, not algorithmic."""
    s = 2 if spec.dtype == "bf16" else 4
    B, H, D, d, r, n = spec.B, spec.H, spec.D, spec.d, spec.r, spec.n
    parts = {
        "rehearse": D * H * r * s + B * D * s + B * H * n * r * s,
        "select": B * H * c * 4,                            # idx written
        "touch": B * H * c * 4,                             # counters
        "attn": B * H * c * 2 * d * s + B * H * d * s + B * H * d * 4,
    }
    parts["speculate"] = parts["rehearse"] + parts["select"] + parts["touch"]
    parts["decode_layer"] = parts["speculate"] + parts["attn"]
    return parts


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=0,
                    help="distinct layer buffers per step (default: the model's 32 layers, as many as fit in 96 GB, "
                         "at least 2)")
    ap.add_argument("--mode", choices=["topk", "threshold"], default="topk")
    ap.add_argument("--path", choices=["fused", "unfused"], default="fused",
                    help="fused: ig_speculate + ig_sparse_decode_attn; unfused: the six-call path")
    ap.add_argument("--schedule", choices=["layer", "serial"], default="layer",
                    help="layer: ig_decode_layer runs layer l's attention beside the speculation for layer l+1 "
                         "in one launch; serial: call after call on one stream")
    ap.add_argument("--workload", choices=["llama2-7b-long", "opt-6.7b", "llama2-13b-pipeline", "opt-30b-pool",
                                          "opt-30b-pool-int4"],
                    default="llama2-7b-long",
                    help="llama2-7b-long: the headline layer (B4, n 131072, top 4%% by default); the others are "
                         "extra measurements")
    ap.add_argument("--n", type=int, default=0, help="context rows (llama2-7b-long; default 131072)")
    ap.add_argument("--batch", type=int, default=0, help="batch (llama2-7b-long; default 4)")
    ap.add_argument("--frac", type=float, default=0.04, help="top-k budget as a fraction of n (llama2-7b-long)")
    ap.add_argument("--extras", default="all",
                    help="extra measurements after the headline: all, none, or a comma list of opt-6.7b, "
                         "pipeline, pool")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="run this many eager steps of the schedule and exit (for hardware-counter passes)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="copy MB megabytes device to device three times and exit (counter calibration)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 counter_collection files of a --profile-steps run and of a "
                         "--copy-calibration run into the traffic record (no GPU needed)")
    args = ap.parse_args()
    if args.record_traffic:
        return record_traffic(args)
    faulthandler.enable()   # a fatal signal prints the Python stack of every thread

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this path has no multi-GPU "
              f"mode: the path would shard over (batch, head) with no exchange)", file=sys.stderr)
        return 2

    import torch
    from sparse_attention_ig_amd import _lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        return 1
    if args.copy_calibration:
        # a plain copy kernel of known size: reads and writes exactly MB megabytes per launch
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copied {nbytes} bytes x 3", file=sys.stderr, flush=True)
        return 0
    _lib.load()

    if args.workload == "llama2-13b-pipeline":
        return emit(pipeline_line(args, bench_pipeline(args)))
    if args.workload in ("opt-30b-pool", "opt-30b-pool-int4"):
        return emit(pool_line(args, bench_pool(args, int4=args.workload.endswith("int4"))))
    spec, step_kw, wl = layer_workload(args.workload, args.mode, n=args.n, batch=args.batch, frac=args.frac)
    res = bench_layer(args, spec, step_kw, wl)
    if res is None:   # --profile-steps
        return 0
    out = {
        "metric": METRIC,
        "value": res["tokens_s_layer"],
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded {spec.name}-shaped draws, no weights or datasets)",
        "config": res["config"],
    }
    out.update({k: v for k, v in res.items() if k not in ("config", "tokens_s_layer", "ms_per_step")})
    extras = [] if args.extras == "none" else (["opt-6.7b", "pipeline", "pool"] if args.extras == "all"
                                                 else [e.strip() for e in args.extras.split(",") if e.strip()])
    if "opt-6.7b" in extras and args.workload != "opt-6.7b":
        s2, kw2, wl2 = layer_workload("opt-6.7b", args.mode)
        sub = argparse.Namespace(**{**vars(args), "workload": "opt-6.7b", "layers": 0})
        r2 = bench_layer(sub, s2, kw2, wl2, quiet=True)
        out["opt_6_7b"] = {"workload": wl2, **{k: r2[k] for k in (
            "tokens_s_layer", "t_layer_us", "step_hbm_GBs", "step_hbm_frac", "per_call_us", "roofline",
            "ms_per_step_p10_p50_p90")}}
    if "pipeline" in extras:
        out["llama2_13b_pipeline"] = bench_pipeline(args)
    if "pool" in extras:
        sub = argparse.Namespace(**{**vars(args), "layers": 4})
        out["opt_30b_pool"] = bench_pool(sub, int4=False, ns=(4096,))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(spec, step_kw, args.cpu_seconds)
    return emit(out)


def emit(out: dict) -> int:
    print(json.dumps(out), flush=True)
    return 0


MODEL_LAYERS = 32            # decoder layers of OPT-6.7B and Llama-2-7B
LAYER_BUDGET_BYTES = 96e9    # HBM given to a step's distinct layer buffers


def layer_workload(name: str, mode: str, n: int = 0, batch: int = 0, frac: float = 0.04):
    """(spec, step kwargs, workload name) of a single-layer workload."""
    from sparse_attention_ig_amd import gen
    if name == "llama2-7b-long":
        spec = gen.llama2_7b_long(n=n or 131072, B=batch or 4, frac=frac)
    else:
        spec = gen.opt_6_7b()
    if mode == "topk":
        step_kw = dict(mode="topk", k=spec.topk, max_out=spec.topk)
        wl = f"{spec.name} decode layer B{spec.B} H{spec.H} d{spec.d} D{spec.D} n{spec.n} r{spec.r} bf16 top-{spec.topk}"
    else:
        step_kw = dict(mode="threshold", alpha=spec.alpha, max_sel=spec.max_sel, max_out=spec.max_sel)
        wl = (f"{spec.name} decode layer B{spec.B} H{spec.H} d{spec.d} D{spec.D} n{spec.n} r{spec.r} bf16 "
              f"alpha={spec.alpha} cap={spec.max_sel}")
    return spec, step_kw, wl


def bench_layer(args, spec, step_kw, wl, quiet: bool = False):
    """Time one decode step through distinct layer buffers of one single-layer workload.  Returns the
    measured figures (None after --profile-steps)."""
    import numpy as np
    import torch
    from sparse_attention_ig_amd import _lib
    from sparse_attention_ig_amd.runtime import DeviceLayer, decode_layer, prepare_layer, to_host

    print(f"[bench] preparing {wl}", file=sys.stderr, flush=True)
    host = prepare_layer(spec)
    base = DeviceLayer(host, max_out=step_kw["max_out"])
    # a decode step through as many distinct layer buffers as the model has (32 for OPT-6.7B and
    # Llama-2-7B), as far as 96 GB of them fit (a third of the HBM), at least 2
    n_layers = args.layers or max(2, min(MODEL_LAYERS, int(LAYER_BUDGET_BYTES // base.nbytes())))
    base.keep_scores = args.path == "unfused"   # the fused path keeps the scores on chip
    layers = [base] + [base.clone() for _ in range(n_layers - 1)]
    del host
    torch.cuda.synchronize()
    footprint = sum(l.nbytes() for l in layers)
    PARTS = DeviceLayer.FUSED if args.path == "fused" else DeviceLayer.PARTS
    schedule = args.schedule if args.path == "fused" else "serial"   # the fused decode layer needs the fused
    #                                                                  speculation

    def run_layer():
        """One ig_decode_layer call per layer: layer l's attention beside the speculation for layer l+1
        (the first layer's speculation and the last layer's attention are the plain calls)."""
        layers[0].step(**step_kw, parts=("speculate",))
        for i in range(len(layers)):
            decode_layer(layers[i], layers[i + 1] if i + 1 < len(layers) else None, step_kw)

    def run(parts=PARTS):
        if parts == PARTS and schedule == "layer":
            return run_layer()
        # stream=None: torch's current stream, which is the capture stream inside a graph capture
        for l in layers:
            l.step(**step_kw, parts=parts)

    def capture(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    def timed_ms(fn, reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    if args.profile_steps:
        for _ in range(args.profile_steps):
            run()
        torch.cuda.synchronize()
        print(f"[bench] {args.profile_steps} profiled steps done", file=sys.stderr, flush=True)
        return None

    # eager launches (every call goes through Python and ctypes)
    for _ in range(args.warmup):
        run()
    ms_eager = timed_ms(run, args.steps) / args.steps

    # the whole step captured once as a HIP graph; the timed region is exactly --steps replays
    graph = capture(run)
    for _ in range(args.warmup):
        graph.replay()
    # one event between consecutive replays: the steps' own durations give the percentiles
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        graph.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = evs[0].elapsed_time(evs[-1])
    step_ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    ms_step = ms_total / args.steps
    tok_s_layer = spec.B * n_layers * args.steps / (ms_total / 1e3)
    # no hand-over failed in any call (the workspaces' status words are clear); rows whose merge recomputed
    recomputed = 0
    for l in layers:
        st, rc = _lib.ig_workspace_status(l.ws_spec, recomputed=True)
        if st:
            raise RuntimeError(f"speculation workspace status {st}: a row's partial query did not arrive")
        recomputed += rc

    # per-call durations: each call alone over every layer in its own graph, HIP events on the stream
    # the kernels run on, averaged over --steps replays
    per_us = {}
    for part in PARTS:
        gp = capture(lambda: run((part,)))
        for _ in range(3):
            gp.replay()
        per_us[part] = 1e3 * timed_ms(gp.replay, args.steps) / (args.steps * n_layers)
    if schedule == "layer":
        # the fused call alone: attention of layer i beside the speculation for layer i+1, every layer
        def run_fused_calls():
            for i in range(len(layers)):
                decode_layer(layers[i], layers[(i + 1) % len(layers)], step_kw)
        gl = capture(run_fused_calls)
        for _ in range(3):
            gl.replay()
        per_us["decode_layer"] = 1e3 * timed_ms(gl.replay, args.steps) / (args.steps * n_layers)

    # dense decode attention over all n rows of the same caches (informative comparison)
    dense_count = torch.full((spec.B, spec.H), spec.n, dtype=torch.int32, device="cuda")

    def run_dense():
        for l in layers:
            _lib.ig_sparse_decode_attn(l.q, l.K, l.V, None, dense_count, spec.softmax_scale, max_out=spec.n,
                                       out=l.out, lse=l.lse, ws=l.ws)
    gd = capture(run_dense)
    for _ in range(3):
        gd.replay()
    dense_reps = max(3, min(args.steps, int(2e3 / max(1e-3, timed_ms(gd.replay, 1)))))
    dense_us = 1e3 * timed_ms(gd.replay, dense_reps) / (dense_reps * n_layers)
    dense_bytes = spec.B * spec.H * spec.n * 2 * spec.d * (2 if spec.dtype == "bf16" else 4)

    res = to_host(layers[0].count)
    c_mean = float(res.mean())
    ab = alg_bytes(spec, c_mean)
    step_bytes = sum(ab[p] for p in PARTS)
    t_layer_s = ms_step / 1e3 / n_layers
    dominant = max(per_us, key=per_us.get)
    dom_bytes = ab[dominant]
    dom_gbs = dom_bytes / (per_us[dominant] * 1e-6) / 1e9 if dom_bytes else 0.0
    key = f"{wl}/{args.path}/{schedule}/ig_{dominant}"
    if not quiet:
        print(f"[bench] {wl}: {t_layer_s * 1e6:.1f} us/layer", file=sys.stderr, flush=True)
    return {
        "tokens_s_layer": round(tok_s_layer, 1),
        "ms_per_step": round(ms_step, 4),
        "config": {"workload": wl, "layers_per_step": n_layers, "footprint_GB": round(footprint / 1e9, 2),
                   "mean_selected_per_head": round(c_mean, 1), "path": args.path, "schedule": schedule,
                   "calls_per_layer": ["decode_layer"] if schedule == "layer" else list(PARTS)},
        "t_layer_us": round(t_layer_s * 1e6, 3),
        "step_alg_bytes_per_layer": int(step_bytes),
        "step_hbm_GBs": round(step_bytes / t_layer_s / 1e9, 1),
        "step_hbm_frac": round(step_bytes / t_layer_s / 1e9 / HBM_PEAK_GBS, 4),
        "per_call_us": {k: round(v, 3) for k, v in per_us.items()},
        "eager_ms_per_step": round(ms_eager, 4),
        "eager_tokens_s_layer": round(spec.B * n_layers / (ms_eager / 1e3), 1),
        "ms_per_step_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 4) for q in (10, 50, 90)],
        "dense_attn_us": round(dense_us, 3),
        "dense_attn_GBs": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
        "roofline": {"kernel": f"ig_{dominant}", "bound": "hbm", "achieved": round(dom_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(key), "alg_bytes_per_launch": int(dom_bytes),
                     "us_per_call": round(per_us[dominant], 3)},
        "wall_s_timed": round(wall, 3),
        "merge_recomputed_rows": recomputed,
    }


def bench_pipeline(args) -> dict:
    """40-layer Llama-2-13B-shaped decode pipeline (speculation for layer l+1 at layer l, layer 0 dense,
    one appended token per step), measured at the first step (n = 4096) and at the last one
    (n = 4351) of a 256-token generation.  One layer's draws are cloned into 40 distinct buffers."""
    import torch
    from sparse_attention_ig_amd import gen
    from sparse_attention_ig_amd.pipeline import DecodePipeline
    from sparse_attention_ig_amd.runtime import prepare_layer, to_device

    L_ = 40
    steps = min(args.steps, 20)
    res = {}
    for n0 in (4096, 4351):
        spec = gen.llama2_13b(n=n0, B=16, n_cap=4352)
        print(f"[bench] preparing llama2-13b pipeline n={n0}", file=sys.stderr, flush=True)
        host = prepare_layer(spec)
        max_out = int(math.ceil(0.05 * spec.cap))
        pipe = DecodePipeline([host], max_out=max_out)
        del host
        base = pipe.layers[0]
        pipe.layers = [base] + [base.clone() for _ in range(L_ - 1)]
        xs = gen.pipeline_x(spec, L_, 1)
        xd = [to_device(xs[0, l]) for l in range(L_)]
        kn, vn = gen.draw_new_rows(spec, 0, 0)
        knd, vnd = [to_device(kn)] * L_, [to_device(vn)] * L_

        def run():
            pipe.n = n0
            pipe.step(xd, knd, vnd)

        for _ in range(3):
            run()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        for _ in range(min(args.warmup, 5)):
            g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        k = min(max_out, int(math.ceil(0.05 * n0)))
        s_ = 2
        per_layer = (spec.D * spec.H * spec.r * s_ + spec.B * spec.D * s_ + spec.B * spec.H * n0 * spec.r * s_
                     + spec.B * spec.H * k * (2 * spec.d * s_ + 8) + spec.B * spec.H * spec.d * (s_ + 4))
        res[n0] = {"ms_per_step": round(ms, 4), "tokens_s_layer": round(spec.B * L_ / (ms / 1e3), 1),
                   "alg_GBs_layers_1_to_39": round(per_layer * (L_ - 1) / (ms / 1e3) / 1e9, 1), "k": k}
        del pipe, base, g
        torch.cuda.empty_cache()
    return {"workload": "llama2-13b 40-layer decode pipeline B16 H40 d128 D5120 r32 top-5%, n 4096 and 4351",
            "steps": steps, "per_step": res}


def pipeline_line(args, res: dict) -> dict:
    first = res["per_step"][4096]
    return {"metric": METRIC, "value": first["tokens_s_layer"], "unit": "tokens/s/layer", "n_gpus": 1,
            "steps": res["steps"], "warmup": min(args.warmup, 5), "ms_per_step": first["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded Llama-2-13B-shaped draws, one layer cloned into 40 buffers)",
            "config": {"workload": res["workload"], "per_step": res["per_step"]}}


def bench_pool(args, int4: bool = False, ns=(2048, 4096)) -> dict:
    """OPT-30B-shaped layers with the full KV cache in a pinned host pool (threshold alpha 5, 20% cap):
    bf16 rows, or (int4) records of 4-bit group-wise codes with a float16 step and minimum per group of 32.
    Per layer: speculation in HBM on the main stream; the selected rows gathered over the host link
    (zero-copy, dequantised on the way for int4) on a side stream; attention on the compact rows once the
    gather is done.  The gather of layer l overlaps the speculation of layer l+1 and the attention of
    layer l-1.  The same work run call after call on one stream gives the overlap ratio: the gather time
    hidden by the two-stream schedule over the gather time.  Then the eviction run: OPT-6.7B-shaped
    layers whose pool holds 80% of the 2048 tokens of a full cache (the summary's Table 2 limit), full,
    so that every decode step evicts each sequence's victim."""
    import numpy as np
    import torch
    from sparse_attention_ig_amd import gen
    from sparse_attention_ig_amd.runtime import PoolLayer, prepare_layer

    nl = args.layers or 8
    steps = min(args.steps, 20)
    res = {}
    main_s = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    for n in ns:
        spec = gen.opt_30b(n=n, B=16, n_cap=4096)
        print(f"[bench] preparing opt-30b pool n={n} x {nl} host-resident layers", file=sys.stderr, flush=True)
        host = prepare_layer(spec)
        layers = [PoolLayer(host, max_out=spec.max_sel, int4=int4) for _ in range(nl)]
        del host

        def step(timing=None):
            E = [ev() for _ in layers]
            F = [ev() for _ in layers]
            G0 = [ev() for _ in layers]
            for l, lay in enumerate(layers):
                lay.speculate(alpha=spec.alpha, max_sel=spec.max_sel, stream=main_s)
                E[l].record(main_s)
                side.wait_event(E[l])
                G0[l].record(side)
                lay.gather(stream=side)
                F[l].record(side)
                if l > 0:
                    main_s.wait_event(F[l - 1])
                    layers[l - 1].attend(stream=main_s)
            main_s.wait_event(F[-1])
            layers[-1].attend(stream=main_s)
            if timing is not None:
                timing.append((G0, F))

        def serial(timing=None):
            G0 = [ev() for _ in layers]
            F = [ev() for _ in layers]
            for l, lay in enumerate(layers):
                lay.speculate(alpha=spec.alpha, max_sel=spec.max_sel, stream=main_s)
                G0[l].record(main_s)
                lay.gather(stream=main_s)
                F[l].record(main_s)
                lay.attend(stream=main_s)
            if timing is not None:
                timing.append((G0, F))

        def timed(fn, reps):
            recs = []
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record(main_s)
            for _ in range(reps):
                fn(recs)
            b.record(main_s)
            torch.cuda.synchronize()
            g_ms = float(np.mean([s0.elapsed_time(f) for G0, F in recs for s0, f in zip(G0, F)]))
            return a.elapsed_time(b) / reps, g_ms

        ms, g_ms = timed(step, steps)
        ms_serial, g_ms_serial = timed(serial, steps)
        cnt = sum(int(l.count.sum().item()) for l in layers) / nl
        link_bytes = cnt * layers[0].record_bytes   # K and V rows (or the token's record) per selected row
        hidden = max(0.0, ms_serial - ms)
        res[n] = {"ms_per_step": round(ms, 3), "layers": nl, "t_layer_us": round(ms * 1e3 / nl, 1),
                  "tokens_s_layer": round(spec.B * nl / (ms / 1e3), 1),
                  "selected_rows_per_layer": int(cnt), "gather_us": round(g_ms * 1e3, 1),
                  "host_link_GBs": round(link_bytes / (g_ms / 1e3) / 1e9, 2),
                  "serial_t_layer_us": round(ms_serial * 1e3 / nl, 1),
                  "serial_gather_us": round(g_ms_serial * 1e3, 1),
                  "overlap_ratio": round(min(1.0, hidden / (g_ms_serial * nl)), 3)}
        del layers
        torch.cuda.empty_cache()
    # the pinned host -> device copy ceiling over the same link
    src = torch.empty(1 << 30, dtype=torch.uint8).pin_memory()
    dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        dst.copy_(src, non_blocking=True)
    a, b = ev(), ev()
    torch.cuda.synchronize()
    a.record()
    for _ in range(5):
        dst.copy_(src, non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    h2d = 5 * (1 << 30) / (a.elapsed_time(b) / 1e3) / 1e9
    del src, dst
    return {"workload": f"opt-30b pinned host KV pool{' (INT4 records, 160 B per token)' if int4 else ''} "
                        f"B16 H56 d128 D7168 r32 alpha 5 cap 20%, {nl} layers",
            "steps": steps, "per_n": res, "pinned_h2d_copy_GBs": round(h2d, 2),
            "eviction_80pct": bench_eviction(args, int4=int4)}


def bench_eviction(args, int4: bool = False) -> dict:
    """OPT-6.7B-shaped layers (B8 H32 d128 D4096 r32, threshold alpha 5, cap 20%) whose host pool has
    1638 slots, 80% of the 2048 tokens of the full cache, all filled: each decode step speculates (with
    the victim), gathers the selected rows over the host link, attends, and appends the new token over
    each sequence's victim slot."""
    import torch
    from sparse_attention_ig_amd import gen
    from sparse_attention_ig_amd.runtime import PoolLayer, prepare_layer, to_device

    nl = 4
    steps = min(args.steps, 20)
    cap = int(0.8 * 2048)
    spec = gen.Spec(**{**gen.opt_6_7b(n=cap, B=8).__dict__, "n_cap": cap})
    print(f"[bench] preparing the eviction run: {nl} pools of {cap} slots (80% of 2048)", file=sys.stderr,
          flush=True)
    host = prepare_layer(spec)
    layers = [PoolLayer(host, max_out=spec.max_sel, int4=int4) for _ in range(nl)]
    del host
    kn, vn = gen.draw_new_rows(spec, 0, 0)
    knd, vnd = to_device(kn), to_device(vn)
    slot = torch.empty(spec.B, dtype=torch.int32, device="cuda")

    def step():
        for lay in layers:
            lay.speculate(alpha=spec.alpha, max_sel=spec.max_sel, want_victim=True)
            lay.gather()
            lay.attend()
            lay.append(knd, vnd, cap, victim=lay.victim, slot_out=slot)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    cnt = sum(int(l.count.sum().item()) for l in layers) / nl
    out = {"workload": f"opt-6.7b pinned host pool of {cap} slots (80% of 2048) B8 H32 d128 D4096 r32 alpha 5 "
                       f"cap 20%, full, {nl} layers", "steps": steps, "t_layer_us": round(ms * 1e3 / nl, 1),
           "tokens_s_layer": round(spec.B * nl / (ms / 1e3), 1), "evictions_per_layer_step": spec.B,
           "selected_rows_per_layer": int(cnt)}
    del layers
    torch.cuda.empty_cache()
    return out


def pool_line(args, res: dict) -> dict:
    last = res["per_n"][max(res["per_n"])]
    return {"metric": METRIC, "value": last["tokens_s_layer"], "unit": "tokens/s/layer", "n_gpus": 1,
            "steps": res["steps"], "warmup": 2, "ms_per_step": last["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded OPT-30B-shaped draws; one layer's pool copied into each pinned buffer)",
            "config": {"workload": res["workload"], "per_n": res["per_n"],
                       "pinned_h2d_copy_GBs": res["pinned_h2d_copy_GBs"]},
            "eviction_80pct": res["eviction_80pct"]}


def _oracle_rate(spec, oi, step_kw, seconds: float, threads: int):
    import numpy as np
    from threadpoolctl import threadpool_limits
    from tests import harness

    with threadpool_limits(threads):
        C0 = np.zeros((spec.B, spec.cap), np.uint32)
        reps = 0
        t0 = time.perf_counter()
        while True:
            harness.oracle_step(oi, counters=C0, **step_kw)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return spec.B * reps / el, reps, el


def _oracle_head_rate(spec, oi, step_kw, seconds: float, threads: int):
    """Oracle layer-step one (b, h) head at a time (partial query, scores, selection, attention, that
    head's counter increments), cycling over the heads for ~seconds; returns tokens/s/layer scaled
    from the time per head (a layer-step is B x H heads)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import oracle as O
    from tests import harness

    heads = [(b, h) for b in range(spec.B) for h in range(spec.H)]
    sel = {k: v for k, v in step_kw.items() if k in ("mode", "alpha", "k", "max_sel", "max_out")}
    C0 = np.zeros((1, spec.cap), np.uint32)
    with threadpool_limits(threads):
        done = 0
        t0 = time.perf_counter()
        while True:
            b, h = heads[done % len(heads)]
            _, idx, cnt = harness.oracle_heads(oi, heads=[(b, h)], **sel)
            O.pool_touch(C0, idx[b:b + 1], cnt[b:b + 1], spec.n, 65535)
            done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    t_layer = el / done * len(heads)
    return spec.B / t_layer, done, el


def cpu_baseline(spec, step_kw, seconds: float) -> dict:
    """The CPU oracle (float64 NumPy) on the same layer-step for ~seconds: with BLAS on the cores this
    process may use (its affinity, capped by OMP_NUM_THREADS when set), and with one thread.  Small
    layers run whole layer-steps; the long-context layer (whose float64 cache would not fit) runs one
    head at a time, over as many heads as the time allows, scaled to the layer's B x H heads."""
    from tests import harness

    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        cores = max(1, min(cores, int(os.environ["OMP_NUM_THREADS"])))
    print("[bench] cpu baseline: the oracle's own setup of the same inputs", file=sys.stderr, flush=True)
    oi = harness.oracle_inputs(spec)
    if spec.B * spec.H * spec.n <= (1 << 21):
        rate, reps, el = _oracle_rate(spec, oi, step_kw, seconds, cores)
        rate1, reps1, el1 = _oracle_rate(spec, oi, step_kw, seconds / 2, 1)
        what = f"full layer-steps of the same workload (1 layer, all {spec.B}x{spec.H} heads)"
        what1 = "layer-steps"
    else:
        rate, reps, el = _oracle_head_rate(spec, oi, step_kw, seconds, cores)
        rate1, reps1, el1 = _oracle_head_rate(spec, oi, step_kw, seconds / 2, 1)
        what = (f"(b, h) heads of the same layer-step ({spec.n} rows each: partial query, scores, selection, "
                f"attention, counters), scaled to the layer's {spec.B}x{spec.H} heads")
        what1 = "heads"
    return {"value": round(rate, 2), "unit": "tokens/s/layer", "cores": cores, "kind": "oracle",
            "sample": f"{reps} {what}, {el:.1f} s, BLAS threads = {cores}",
            "value_1thread": round(rate1, 2),
            "sample_1thread": f"{reps1} {what1}, {el1:.1f} s, BLAS limited to 1 thread"}


# ---------------------------------------------------------------- HBM traffic from hardware counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = ("ig_attn_dev.h", "ig_device.h", "ig_pool_dev.h", "ig_select_dev.h", "ig_spec_dev.h",
                  "k_decode.hip", "k_rehearse.hip", "k_speculate.hip", "k_attn.hip", "k_select.hip", "k_pool.hip")


def kernel_sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_attention_ig_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


# the kernels of a call (rocprofv3 kernel names start with these): ig_decode_layer is one fused launch plus,
# for sliced rows, the merge (which also combines a split attention) and the counter kernels; where the
# two halves are not fused it is the speculation's kernels and the attention's
CALL_KERNELS = {
    "ig_decode_layer": ("void ig::k_decode_layer<", "void ig::k_spec_merge<", "ig::k_touch_bits(",
                        "ig::k_touch_finish("),
    "ig_decode_layer/unfused": ("void ig::k_speculate<", "void ig::k_spec_merge<", "ig::k_touch_bits(",
                                "ig::k_touch_finish(", "void ig::k_attn_split<", "ig::k_attn_combine("),
    "ig_speculate": ("void ig::k_speculate<", "void ig::k_spec_merge<", "ig::k_touch_bits(",
                     "ig::k_touch_finish("),
}


def _counter_means(path: str) -> dict:
    """Mean counter value (KiB) per kernel name of a rocprofv3 counter_collection CSV."""
    import csv
    acc = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            acc.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def record_traffic(args) -> int:
    """Per-call HBM bytes of the bench's dominant call from FETCH_SIZE and WRITE_SIZE passes, each scaled
    by what the same counter reads for a plain device copy of --copy-calibration MB (default 512)."""
    fetch, write, cfetch, cwrite = (_counter_means(p) for p in args.record_traffic)
    copy_kib = (args.copy_calibration or 512) * 1024.0
    cname = [k for k in cfetch if "copyBuffer" in k]
    if not cname:
        print("no copy kernel in the calibration files", file=sys.stderr)
        return 1
    f_fac = copy_kib / cfetch[cname[0]]
    w_fac = copy_kib / cwrite[cname[0]]
    call = "ig_decode_layer" if args.schedule == "layer" else "ig_speculate"
    kset = call
    if call == "ig_decode_layer" and not any(k.startswith("void ig::k_decode_layer<") for k in fetch):
        kset = "ig_decode_layer/unfused"
    per_kernel = {}
    total = 0.0
    for prefix in CALL_KERNELS[kset]:
        names = [k for k in fetch if k.startswith(prefix)]
        if len(names) > 1:
            print(f"expected at most one kernel named {prefix}*, found {names}", file=sys.stderr)
            return 1
        if not names:
            continue
        nm = names[0]
        b = (fetch[nm] * f_fac + write[nm] * w_fac) * 1024.0
        per_kernel[nm] = {"fetch_KiB": round(fetch[nm], 1), "write_KiB": round(write[nm], 1),
                          "bytes": int(round(b))}
        total += b
    if not per_kernel:
        print(f"no kernel of {call} in the counter files", file=sys.stderr)
        return 1
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec["note"] = ("HBM bytes per call: rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean over the "
                   "dispatches of a --profile-steps run), each scaled by copy MB / counter reading of a plain "
                   "device copy; 'sources' is the digest of the kernel sources the counters were taken with")
    _, _, wl = layer_workload(args.workload, args.mode, n=args.n, batch=args.batch, frac=args.frac)
    key = f"{wl}/{args.path}/{args.schedule}/{call}"
    rec.setdefault("entries", {})[key] = {
        "sources": kernel_sources_digest(), "bytes_per_call": int(round(total)),
        "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4), "kernels": per_kernel}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec["entries"][key]))
    return 0


def measured_traffic(key: str):
    """HBM bytes per call from the committed FETCH_SIZE / WRITE_SIZE counter passes, scaled by the copy
    calibration; None when there is no record for this workload and call (key: workload name / path /
    schedule / call), or when the kernel sources have changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("entries", {}).get(key)
    if not entry or entry.get("sources") != kernel_sources_digest():
        return None
    return entry.get("bytes_per_call")


if __name__ == "__main__":
    sys.exit(main())

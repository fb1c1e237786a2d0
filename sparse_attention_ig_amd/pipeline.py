"""Cross-layer decode pipeline on one GPU, through libig.so only.

The speculation for layer l+1 runs at layer l from layer l's attention input
(the summary of InfiniGen, arXiv 2406.19707, section 3.2 and section 3.4
"Decoding Stage"): per decode step and layer l,

    attention(l)          over idx_l selected at layer l-1 (layer 0: dense over every row)
    ig_speculate(l + 1)   from x_l with layer l+1's partial weight and partial key cache
                          -> idx_{l+1}, counters of layer l+1

and after the last layer every layer appends the new token's key and value (ig_append_kv), which
also writes the partial-key row and restarts the slot's counter.
"""
from __future__ import annotations

import math
from typing import List, Optional

from . import _lib as L
from .runtime import DeviceLayer, HostLayer


class DecodePipeline:
    def __init__(self, hosts: List[HostLayer], max_out: int, cmax: int = 65535):
        import torch
        self.layers = [DeviceLayer(h, max_out=max_out) for h in hosts]
        for lay in self.layers:
            lay.keep_scores = False
        s = hosts[0].spec
        self.spec = s
        self.n = s.n
        self.cmax = cmax
        self.max_out = max_out
        self.dense_count = torch.full((s.B, s.H), s.n, dtype=torch.int32, device="cuda")
        self.slot = torch.empty((s.B,), dtype=torch.int32, device="cuda")

    def topk(self) -> int:
        """Fixed budget of the pipeline workload: 5% of the current context."""
        return min(self.max_out, int(math.ceil(0.05 * self.n)))

    def step(self, x_layers, k_new=None, v_new=None, *, mode: str = "topk", k: Optional[int] = None,
             alpha: float = math.inf, max_sel: int = 0, stream=None, append: bool = True):
        """One decode step through every layer.  x_layers: per-layer attention inputs [B][D];
        k_new / v_new: per-layer new key / value rows [B][H][d] (appended when ``append``)."""
        s = self.spec
        n = self.n
        k = self.topk() if k is None else k
        self.dense_count.fill_(n)
        nl = len(self.layers)
        for l, lay in enumerate(self.layers):
            if l == 0:
                L.ig_sparse_decode_attn(lay.q, lay.K, lay.V, None, self.dense_count, s.softmax_scale,
                                        max_out=s.cap, out=lay.out, lse=lay.lse, ws=lay.ws, stream=stream)
            else:
                L.ig_sparse_decode_attn(lay.q, lay.K, lay.V, lay.idx, lay.count, s.softmax_scale, out=lay.out,
                                        lse=lay.lse, ws=lay.ws, stream=stream)
            if l + 1 < nl:
                nxt = self.layers[l + 1]
                L.ig_speculate(x_layers[l], nxt.Wq_part, nxt.Kp, n, s.softmax_scale, mode, self.max_out,
                               alpha=alpha, k=k, max_sel=max_sel, idx=nxt.idx, count=nxt.count,
                               counters=nxt.counters, cmax=self.cmax, q_part=nxt.q_part, ws=nxt.ws_spec,
                               stream=stream)
        if append:
            for l, lay in enumerate(self.layers):
                L.ig_append_kv(lay.K, lay.V, lay.Kp, lay.counters, lay.chan, k_new[l], v_new[l], n,
                               slot_out=self.slot, stream=stream)
            self.n = min(n + 1, s.cap)

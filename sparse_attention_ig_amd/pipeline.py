"""Cross-layer decode pipeline on one GPU, through libig.so only.

The speculation for layer l+1 runs at layer l from layer l's attention input
(the summary of InfiniGen, arXiv 2406.19707, section 3.2 and section 3.4
"Decoding Stage"): per decode step and layer l,

    attention(l)          over idx_l selected at layer l-1 (layer 0: dense over every row)
    speculation(l + 1)    from x_l with layer l+1's partial weight and partial key cache
                          -> idx_{l+1}, counters of layer l+1

both in one ig_decode_layer call (the two run side by side on the GPU),
and after the last layer every layer appends the new token's key and value (ig_append_kv), which
also writes the partial-key row and restarts the slot's counter.

Once the cache is full (n = n_cap) an append overwrites each sequence's victim, the slot with the
smallest access counter (the summary's counter-based eviction, section 3.4 "KV Cache Pool Management
Under Memory Pressure"): layers 1.. take it from their speculation (which then asks for it); layer 0,
which no speculation selects for (it attends to every row), takes the lowest slot among the minima of
its counters, which only appends reset (ig_pool_touch with empty selections).
"""
from __future__ import annotations

import math
from typing import List, Optional

from . import _lib as L
from .runtime import DeviceLayer, HostLayer, attn_call, spec_call


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
        self.no_count = torch.zeros((s.B, s.H), dtype=torch.int32, device="cuda")

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
            # attention of layer l (layer 0: dense over every row) beside the speculation for layer l+1
            attn = attn_call(lay)
            if l == 0:
                attn.update(idx=None, count=self.dense_count, max_out=s.cap)
            spec = None
            if l + 1 < nl:
                spec = spec_call(self.layers[l + 1], mode=mode, alpha=alpha, k=k, max_sel=max_sel, cmax=self.cmax,
                                 n=n, x=x_layers[l], want_victim=n == s.cap)
            L.ig_decode_layer(attn, spec, stream=stream)
        if append:
            self.append(k_new, v_new, stream=stream)

    def append(self, k_new, v_new, *, stream=None):
        """Every layer appends the new token's key and value rows (slot n, or the victim when full)."""
        n = self.n
        full = n == self.spec.cap
        for l, lay in enumerate(self.layers):
            if full and l == 0:
                L.ig_pool_touch(lay.counters, lay.idx, self.no_count, n, self.cmax, victim=lay.victim, ws=lay.ws,
                                stream=stream)
            L.ig_append_kv(lay.K, lay.V, lay.Kp, lay.counters, lay.chan, k_new[l], v_new[l], n,
                           victim=lay.victim if full else None, slot_out=self.slot, stream=stream)
        self.n = min(n + 1, self.spec.cap)

"""Layer preparation and the decode layer-step on the GPU, through libig.so only.

``prepare_layer`` runs the library's host setup on one layer's raw draws:
skew rotation (ig_skew_weights), rotation of the raw query / keys
(ig_skew_apply), storage rounding (ig_store) and the channel pick with the
partial query weight (ig_partial_weight_index).  ``DeviceLayer`` holds a
layer's decode-path tensors in HBM and builds the partial key cache with
ig_build_partial_cache.  ``DeviceLayer.step`` is one layer-step of the hot
path: ig_rehearse -> ig_select -> ig_sparse_decode_attn -> ig_pool_touch, all
enqueued on one stream with no host synchronisation.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

from . import gen


@dataclass
class HostLayer:
    spec: gen.Spec
    x: np.ndarray          # [B][D] stored
    Wq_part: np.ndarray    # [H*r][D] stored (one row per partial column)
    chan: np.ndarray       # [H][r] int32
    q: np.ndarray          # [B][H][d] stored (skewed full query)
    K: np.ndarray          # [B][H][n_cap][d] stored (skewed keys)
    V: np.ndarray          # [B][H][n_cap][d] stored
    extra: Dict = field(default_factory=dict)


def rows_layout(K: np.ndarray) -> np.ndarray:
    """[B][H][n][d] -> [B*n][H*d] (head blocks side by side), for per-head rotation."""
    B, H, n, d = K.shape
    return np.ascontiguousarray(K.transpose(0, 2, 1, 3).reshape(B * n, H * d))


def heads_layout(M: np.ndarray, B: int, H: int, n: int, d: int) -> np.ndarray:
    return np.ascontiguousarray(M.reshape(B, n, H, d).transpose(0, 2, 1, 3))


def prepare_layer(spec: gen.Spec, layer: int = 0, lay: Optional[gen.Layer] = None) -> HostLayer:
    """Library route from the raw draws of one layer to its stored decode-path inputs."""
    from . import _lib as L
    B, H, d, r = spec.B, spec.H, spec.d, spec.r
    lay = lay or gen.draw_layer(spec, layer, with_wk=False)
    sk = L.ig_skew_weights(lay.skew_src, Wq=lay.Wq)
    Wq_s = L.ig_store(sk["Wq_s"], spec.dtype)
    q = L.ig_store(L.ig_skew_apply(sk["A"], lay.q_raw), spec.dtype)
    if spec.frame == "raw":
        Kr = L.ig_skew_apply(sk["A"], rows_layout(lay.K_raw))
        K = L.ig_store(heads_layout(Kr, B, H, spec.cap, d), spec.dtype)
        V, heavy = lay.V, lay.heavy_pos
    else:
        K, V, heavy = gen.draw_cache(spec, layer, gen.values(q, spec.dtype))
    chan, Wq_part = L.ig_partial_weight_index(Wq_s, K, r, spec.n, spec.dtype)
    return HostLayer(spec, lay.x, Wq_part, chan, q.reshape(B, H, d), K, V,
                     extra={"A": sk["A"], "sigma": sk["sigma"], "heavy": heavy, "Wq_s": Wq_s})


def to_device(a: np.ndarray):
    """numpy -> cuda tensor; uint16 arrays are bf16 bits, uint32 counters ride as int32."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).cuda()
    return torch.from_numpy(a).cuda()


def to_host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class DeviceLayer:
    """One layer's decode-path inputs resident in HBM, plus preallocated outputs and workspaces."""

    def __init__(self, host: HostLayer, counters: Optional[np.ndarray] = None, max_out: Optional[int] = None):
        import torch
        from . import _lib as L
        s = host.spec
        self.spec = s
        self.x = to_device(host.x)
        self.Wq_part = to_device(host.Wq_part)
        self.chan = to_device(host.chan)
        self.q = to_device(host.q)
        self.K = to_device(host.K)
        self.V = to_device(host.V)
        self.Kp = torch.zeros((s.B, s.H, s.cap, s.r), dtype=self.K.dtype, device="cuda")
        L.ig_build_partial_cache(self.K, self.chan, self.Kp, 0, s.n)
        self.counters = to_device(counters if counters is not None else np.zeros((s.B, s.cap), dtype=np.uint32))
        self.max_out = max_out or s.cap
        self.keep_scores = True   # the fused path writes the scores to HBM only when asked
        dv = "cuda"
        self.q_part = torch.empty((s.B, s.H, s.r), dtype=torch.float32, device=dv)
        self.scores = torch.empty((s.B, s.H, s.cap), dtype=torch.float32, device=dv)
        self.idx = torch.empty((s.B, s.H, self.max_out), dtype=torch.int32, device=dv)
        self.count = torch.empty((s.B, s.H), dtype=torch.int32, device=dv)
        self.out = torch.empty((s.B, s.H, s.d), dtype=torch.float32, device=dv)
        self.lse = torch.empty((s.B, s.H), dtype=torch.float32, device=dv)
        self.victim = torch.empty((s.B,), dtype=torch.int32, device=dv)
        nb = max(L.ig_workspace_size(L.IG_OP_REHEARSE, s.B, s.H, s.D, s.d, s.r, s.cap, self.max_out),
                 L.ig_workspace_size(L.IG_OP_SELECT, s.B, s.H, s.D, s.d, s.r, s.cap, self.max_out),
                 L.ig_workspace_size(L.IG_OP_ATTN, s.B, s.H, s.D, s.d, s.r, s.cap, self.max_out),
                 L.ig_workspace_size(L.IG_OP_ATTN, s.B, s.H, s.D, s.d, s.r, s.cap, s.cap),
                 L.ig_workspace_size(L.IG_OP_TOUCH, s.B, s.H, s.D, s.d, s.r, s.cap, self.max_out), 16)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=dv)
        # the fused speculation keeps its arrival words in its own workspace, zero between calls
        self.ws_spec = L.ig_workspace_init(torch.empty(
            L.ig_workspace_size(L.IG_OP_SPECULATE, s.B, s.H, s.D, s.d, s.r, s.cap, self.max_out),
            dtype=torch.uint8, device=dv))

    def clone(self) -> "DeviceLayer":
        """A copy in distinct HBM buffers (device-to-device copies of every tensor)."""
        import copy
        other = copy.copy(self)
        for name, v in vars(self).items():
            if hasattr(v, "is_cuda") and v.is_cuda:
                setattr(other, name, v.clone())
        return other

    def nbytes(self) -> int:
        return sum(v.numel() * v.element_size() for v in vars(self).values() if hasattr(v, "is_cuda"))

    PARTS = ("rehearse", "select", "attn", "touch")      # the six-call path
    FUSED = ("speculate", "attn")                        # fused speculation, then attention

    def step(self, *, mode: str, alpha: float = math.inf, k: int = 0, max_sel: int = 0,
             max_out: Optional[int] = None, cmax: int = 65535, want_victim: bool = False,
             n: Optional[int] = None, stream=None, events=None, parts=PARTS) -> Dict:
        """One layer-step (or the listed ``parts`` of it), enqueued on ``stream`` (default: the
        current stream).  ``events``: optional dict part -> (start, end) torch events recorded
        around each call."""
        from . import _lib as L
        s = self.spec
        n = s.n if n is None else n
        max_out = self.max_out if max_out is None else max_out
        idx = self.idx if max_out == self.max_out else self.idx.view(-1)[:s.B * s.H * max_out].view(s.B, s.H, max_out)
        ev = events or {}

        for part in parts:
            if part in ev:
                ev[part][0].record(stream)
            if part == "rehearse":
                L.ig_rehearse(self.x, self.Wq_part, self.Kp, n, s.softmax_scale, q_part=self.q_part,
                              scores=self.scores, ld=s.cap, ws=self.ws, stream=stream)
            elif part == "select":
                L.ig_select(self.scores, mode, max_out, n=n, alpha=alpha, k=k, max_sel=max_sel, idx=idx,
                            count=self.count, ws=self.ws, stream=stream)
            elif part == "attn":
                L.ig_sparse_decode_attn(self.q, self.K, self.V, idx, self.count, s.softmax_scale, out=self.out,
                                        lse=self.lse, ws=self.ws, stream=stream)
            elif part == "speculate":
                L.ig_speculate(self.x, self.Wq_part, self.Kp, n, s.softmax_scale, mode, max_out, alpha=alpha, k=k,
                               max_sel=max_sel, idx=idx, count=self.count, counters=self.counters, cmax=cmax,
                               victim=self.victim if want_victim else None, q_part=self.q_part,
                               scores=self.scores if self.keep_scores else None, ld=s.cap, ws=self.ws_spec,
                               stream=stream)
            elif part == "touch":
                L.ig_pool_touch(self.counters, idx, self.count, n, cmax,
                                victim=self.victim if want_victim else None, ws=self.ws, stream=stream)
            else:
                raise ValueError(part)
            if part in ev:
                ev[part][1].record(stream)
        return dict(q_part=self.q_part, scores=self.scores, idx=idx, count=self.count, out=self.out, lse=self.lse,
                    counters=self.counters, victim=self.victim if want_victim else None)


def attn_call(layer: "DeviceLayer", max_out: Optional[int] = None) -> Dict:
    """The attention half of ig_decode_layer for ``layer`` (its q, cache and current selection)."""
    s = layer.spec
    max_out = layer.max_out if max_out is None else max_out
    idx = layer.idx if max_out == layer.max_out else layer.idx.view(-1)[:s.B * s.H * max_out].view(s.B, s.H, max_out)
    return dict(q=layer.q, K=layer.K, V=layer.V, idx=idx, count=layer.count, scale=s.softmax_scale, out=layer.out,
                lse=layer.lse, ws=layer.ws)


def spec_call(layer: "DeviceLayer", *, mode: str, alpha: float = math.inf, k: int = 0, max_sel: int = 0,
              max_out: Optional[int] = None, cmax: int = 65535, want_victim: bool = False,
              n: Optional[int] = None, x=None) -> Dict:
    """The speculation half of ig_decode_layer for ``layer`` (from its own x unless ``x`` is given)."""
    s = layer.spec
    max_out = layer.max_out if max_out is None else max_out
    idx = layer.idx if max_out == layer.max_out else layer.idx.view(-1)[:s.B * s.H * max_out].view(s.B, s.H, max_out)
    return dict(x=layer.x if x is None else x, Wq_part=layer.Wq_part, Kp=layer.Kp, n=s.n if n is None else n,
                scale=s.softmax_scale, mode=mode, alpha=alpha, k=k, max_sel=max_sel, idx=idx, count=layer.count,
                counters=layer.counters, cmax=cmax, victim=layer.victim if want_victim else None,
                q_part=layer.q_part, scores=layer.scores if layer.keep_scores else None, ld=s.cap, ws=layer.ws_spec)


def decode_layer(attn_layer: Optional["DeviceLayer"], spec_layer: Optional["DeviceLayer"], step_kw: Dict,
                 stream=None):
    """Layer l's attention (attn_layer) beside the speculation for layer l+1 (spec_layer), one fused launch."""
    from . import _lib as L
    kw = {k: v for k, v in step_kw.items() if k in ("mode", "alpha", "k", "max_sel", "max_out", "cmax",
                                                     "want_victim", "n")}
    L.ig_decode_layer(attn_call(attn_layer, step_kw.get("max_out")) if attn_layer is not None else None,
                      spec_call(spec_layer, **kw) if spec_layer is not None else None, stream=stream)


class MappedHost:
    """Device-side view of a pinned host tensor: the address kernels must use, from
    hipHostGetDevicePointer (fails cleanly if the memory is not pinned and mapped), with the shape and
    dtype the binding reads."""

    _hip = None

    def __init__(self, t):
        import ctypes
        if not t.is_pinned():
            raise ValueError("tensor is not in pinned host memory")
        if MappedHost._hip is None:
            MappedHost._hip = ctypes.CDLL("libamdhip64.so")
        dptr = ctypes.c_void_p()
        err = MappedHost._hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(t.data_ptr()), 0)
        if err != 0 or not dptr.value:
            raise RuntimeError(f"hipHostGetDevicePointer failed ({err}): host pool not mapped into the device")
        self._t = t
        self._dptr = dptr.value
        self.shape, self.dtype = t.shape, t.dtype

    def data_ptr(self) -> int:
        return self._dptr

    def is_contiguous(self) -> bool:
        return self._t.is_contiguous()


class PoolLayer:
    """A layer whose full key / value cache lives in pinned host memory (the KV pool: bf16 rows, or INT4
    records with ``int4``), with the partial key cache, weights, query and counters in HBM.  The selected rows are fetched over the host link by
    ig_gather_kv (zero-copy reads of the pinned pool) into compact HBM buffers, and the attention runs on
    those (the summary's section 3.2 Pool Manager and section 3.4 "Decoding Stage" step 5)."""

    def __init__(self, host: HostLayer, max_out: int, int4: bool = False):
        import torch
        from . import _lib as L
        s = host.spec
        self.spec = s
        self.max_out = max_out
        self.int4 = int4
        self.x = to_device(host.x)
        self.Wq_part = to_device(host.Wq_part)
        self.chan = to_device(host.chan)
        self.q = to_device(host.q)
        dv = "cuda"
        self.Kp = torch.zeros((s.B, s.H, s.cap, s.r), dtype=torch.bfloat16, device=dv)
        if int4:
            # the pool as INT4 records (ig_quantize_kv writes them over the host link from a transient
            # device copy of the prefilled cache); the partial key cache keeps full precision in HBM
            rec = L.ig_int4_record_bytes(s.d)
            self.KVq_host = torch.zeros((s.B, s.H, s.cap, rec), dtype=torch.uint8).pin_memory()
            self.KVq = MappedHost(self.KVq_host)
            Kd, Vd = to_device(host.K), to_device(host.V)
            L.ig_quantize_kv(Kd, Vd, self.KVq, 0, s.n)
            L.ig_build_partial_cache(Kd, self.chan, self.Kp, 0, s.n)
            torch.cuda.synchronize()
            del Kd, Vd
            self.record_bytes = rec
        else:
            self.Kh_host = torch.from_numpy(host.K.view(np.int16)).view(torch.bfloat16).pin_memory()
            self.Vh_host = torch.from_numpy(host.V.view(np.int16)).view(torch.bfloat16).pin_memory()
            self.Kh, self.Vh = MappedHost(self.Kh_host), MappedHost(self.Vh_host)
            L.ig_build_partial_cache(self.Kh, self.chan, self.Kp, 0, s.n)   # reads the pinned pool directly
            self.record_bytes = 2 * s.d * 2   # a K and a V row
        self.counters = torch.zeros((s.B, s.cap), dtype=torch.int32, device=dv)
        self.idx = torch.empty((s.B, s.H, max_out), dtype=torch.int32, device=dv)
        self.count = torch.empty((s.B, s.H), dtype=torch.int32, device=dv)
        self.victim = torch.empty((s.B,), dtype=torch.int32, device=dv)
        self.Kc = torch.empty((s.B, s.H, max_out, s.d), dtype=torch.bfloat16, device=dv)
        self.Vc = torch.empty_like(self.Kc)
        self.out = torch.empty((s.B, s.H, s.d), dtype=torch.float32, device=dv)
        self.lse = torch.empty((s.B, s.H), dtype=torch.float32, device=dv)
        self.ws_spec = L.ig_workspace_init(torch.empty(
            L.ig_workspace_size(L.IG_OP_SPECULATE, s.B, s.H, s.D, s.d, s.r, s.cap, max_out),
            dtype=torch.uint8, device=dv))
        self.ws = torch.empty(max(L.ig_workspace_size(L.IG_OP_ATTN, s.B, s.H, s.D, s.d, s.r, s.cap, max_out), 16),
                              dtype=torch.uint8, device=dv)

    def speculate(self, *, alpha: float, max_sel: int, cmax: int = 65535, n: Optional[int] = None,
                  want_victim: bool = False, stream=None):
        from . import _lib as L
        s = self.spec
        L.ig_speculate(self.x, self.Wq_part, self.Kp, s.n if n is None else n, s.softmax_scale, "threshold",
                       self.max_out, alpha=alpha, max_sel=max_sel, idx=self.idx, count=self.count,
                       counters=self.counters, cmax=cmax, victim=self.victim if want_victim else None,
                       ws=self.ws_spec, stream=stream)

    def gather(self, stream=None):
        from . import _lib as L
        if self.int4:
            L.ig_gather_kv_int4(self.KVq, self.idx, self.count, self.spec.d, Kc=self.Kc, Vc=self.Vc, stream=stream)
        else:
            L.ig_gather_kv(self.Kh, self.Vh, self.idx, self.count, Kc=self.Kc, Vc=self.Vc, stream=stream)

    def append(self, k_new, v_new, n: int, *, victim=None, slot_out=None, stream=None):
        """The new token's rows into the pool (slot n, or the victim when full): full rows, or INT4 records
        written at the slot ig_append_kv picked; the partial key row and the counter in HBM."""
        import torch
        from . import _lib as L
        s = self.spec
        if slot_out is None:
            slot_out = torch.empty((s.B,), dtype=torch.int32, device="cuda")
        if self.int4:
            L.ig_append_kv(None, None, self.Kp, self.counters, self.chan, k_new, v_new, n, victim=victim,
                           slot_out=slot_out, stream=stream)
            L.ig_quantize_kv(k_new.view(s.B, s.H, 1, s.d), v_new.view(s.B, s.H, 1, s.d), self.KVq, 0, 1, slot=slot_out,
                             stream=stream)
        else:
            L.ig_append_kv(self.Kh, self.Vh, self.Kp, self.counters, self.chan, k_new, v_new, n, victim=victim,
                           slot_out=slot_out, stream=stream)
        return slot_out

    def attend(self, stream=None):
        from . import _lib as L
        L.ig_sparse_decode_attn(self.q, self.Kc, self.Vc, None, self.count, self.spec.softmax_scale,
                                max_out=self.max_out, out=self.out, lse=self.lse, ws=self.ws, stream=stream)

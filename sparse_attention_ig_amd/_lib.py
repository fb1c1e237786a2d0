"""Python binding of libig.so (include/ig.h): argument marshalling only.

Each ``ig_*`` function here calls the C function of the same name.  Device
arguments are torch tensors on the GPU (bfloat16 or float32 elements, int32
indices, uint32 counters held as int32 tensors); host setup arguments are numpy
arrays.  Sizes are read off the tensor shapes; every check on values and sizes
is the library's.  Work is enqueued on ``stream`` (default: torch's current
stream).  There is no fallback: if libig.so is missing or a call fails, a
RuntimeError is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libig.so")

IG_OK, IG_EINVAL, IG_EHIP, IG_EUNSUPPORTED = 0, 1, 2, 3
IG_F32, IG_BF16 = 0, 1
IG_SEL_THRESHOLD, IG_SEL_TOPK, IG_SEL_HEADAVG = 0, 1, 2
IG_OP_REHEARSE, IG_OP_SELECT, IG_OP_ATTN, IG_OP_SPECULATE, IG_OP_TOUCH, IG_OP_SETUP = 0, 1, 2, 3, 4, 5

_MODES = {"threshold": IG_SEL_THRESHOLD, "topk": IG_SEL_TOPK, "headavg": IG_SEL_HEADAVG}

_vp, _i, _i64, _f, _u32, _sz, _d = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                   ctypes.c_uint32, ctypes.c_size_t, ctypes.c_double)


class SkewArgs(ctypes.Structure):
    _fields_ = [("D", _i), ("H", _i), ("d", _i), ("m", _i),
                ("skew_src", _vp), ("Wq", _vp), ("Wk", _vp), ("bq", _vp), ("bk", _vp),
                ("A", _vp), ("sigma", _vp), ("Wq_s", _vp), ("Wk_s", _vp), ("bq_s", _vp), ("bk_s", _vp),
                ("nthreads", _i)]


class AttnCall(ctypes.Structure):
    """ig_attn_call: the attention half of ig_decode_layer."""
    _fields_ = [("q", _vp), ("K", _vp), ("V", _vp), ("ld_rows", _i), ("idx", _vp), ("count", _vp),
                ("max_out", _i), ("scale", _f), ("out", _vp), ("lse", _vp), ("ws", _vp), ("ws_bytes", _sz)]


class SpecCall(ctypes.Structure):
    """ig_spec_call: the speculation half of ig_decode_layer."""
    _fields_ = [("x", _vp), ("Wq_part", _vp), ("bq_part", _vp), ("Kp", _vp), ("D", _i), ("r", _i), ("n", _i),
                ("n_cap", _i), ("scale", _f), ("mode", _i), ("alpha", _f), ("k", _i), ("max_sel", _i),
                ("idx", _vp), ("count", _vp), ("max_out", _i), ("counters", _vp), ("cmax", _u32), ("victim", _vp),
                ("q_part", _vp), ("scores", _vp), ("ld", _i), ("ws", _vp), ("ws_bytes", _sz)]


_SIGS = {
    "ig_last_error": (ctypes.c_char_p, []),
    "ig_version": (_i, []),
    "ig_skew_weights": (_i, [ctypes.POINTER(SkewArgs)]),
    "ig_skew_apply": (_i, [_vp, _i, _i, _vp, _i64, _vp, _i]),
    "ig_store": (_i, [_vp, _i64, _i, _vp]),
    "ig_partial_weight_index": (_i, [_vp, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _vp, _vp, _i]),
    "ig_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "ig_workspace_init": (_i, [_vp, _sz, _vp]),
    "ig_workspace_status": (_i, [_vp, _sz, ctypes.POINTER(_u32), ctypes.POINTER(_u32), _vp]),
    "ig_set_handover_test_mode": (_i, [_u32, _i]),
    "ig_speculate": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _f, _i, _i, _vp, _vp, _i,
                          _vp, _u32, _vp, _vp, _vp, _i, _vp, _sz, _vp]),
    "ig_speculate_noalloc": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _f, _i, _i, _vp, _vp, _i,
                                  _vp, _u32, _vp, _vp, _vp, _i, _vp]),
    "ig_rehearse": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _i, _vp, _sz, _vp]),
    "ig_select": (_i, [_vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp, _vp, _i, _vp, _sz, _vp]),
    "ig_gather_kv": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "ig_sparse_decode_attn": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _sz, _vp]),
    "ig_pool_touch": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _u32, _vp, _vp, _sz, _vp]),
    "ig_decode_layer": (_i, [_i, _i, _i, _i, ctypes.POINTER(AttnCall), ctypes.POINTER(SpecCall), _vp]),
    "ig_partial_weight_index_dev": (_i, [_vp, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "ig_build_partial_cache": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "ig_append_kv": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "ig_int4_record_bytes": (_sz, [_i]),
    "ig_quantize_kv": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _i, _vp]),
    "ig_gather_kv_int4": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libig.so (once); raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_attention_ig_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols():
    return list(_SIGS)


def _check(status: int, name: str):
    if status != IG_OK:
        msg = load().ig_last_error().decode(errors="replace")
        raise RuntimeError(f"{name} failed with status {status}: {msg}")


# ---------------------------------------------------------------- marshalling helpers
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        if not t.flags["C_CONTIGUOUS"]:
            raise ValueError("array must be C-contiguous")
        return t.ctypes.data
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _dtype_of(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return IG_BF16
    if t.dtype == torch.float32:
        return IG_F32
    raise ValueError(f"element dtype must be bfloat16 or float32, got {t.dtype}")


def _np_dtype(dtype: str) -> int:
    return {"f32": IG_F32, "bf16": IG_BF16}[dtype]


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ws(ws, nbytes: int, device):
    if nbytes == 0:
        return ws, 0
    if ws is None:
        ws = _torch().empty(nbytes, dtype=_torch().uint8, device=device)
    return ws, ws.numel() * ws.element_size()


# ---------------------------------------------------------------- host setup
def ig_version() -> int:
    return load().ig_version()


def ig_last_error() -> str:
    return load().ig_last_error().decode(errors="replace")


def ig_workspace_size(op: int, B: int, H: int, D: int = 0, d: int = 0, r: int = 0, n: int = 0,
                      max_out: int = 0) -> int:
    return int(load().ig_workspace_size(op, B, H, D, d, r, n, max_out))


def ig_skew_weights(skew_src: np.ndarray, Wq=None, Wk=None, bq=None, bk=None, nthreads: int = 0) -> dict:
    """A [H][d][d], sigma [H][d] and the rotated weights / biases (float64 numpy)."""
    src = np.ascontiguousarray(skew_src, dtype=np.float64)
    H, m, d = src.shape
    f64 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float64)
    Wq, Wk, bq, bk = f64(Wq), f64(Wk), f64(bq), f64(bk)
    D = (Wq if Wq is not None else Wk).shape[0] if (Wq is not None or Wk is not None) else 0
    out = {"A": np.empty((H, d, d)), "sigma": np.empty((H, d))}
    for name, a in (("Wq_s", Wq), ("Wk_s", Wk), ("bq_s", bq), ("bk_s", bk)):
        out[name] = None if a is None else np.empty_like(a)
    args = SkewArgs(D, H, d, m, _ptr(src), _ptr(Wq), _ptr(Wk), _ptr(bq), _ptr(bk), _ptr(out["A"]),
                    _ptr(out["sigma"]), _ptr(out["Wq_s"]), _ptr(out["Wk_s"]), _ptr(out["bq_s"]),
                    _ptr(out["bk_s"]), int(nthreads))
    _check(load().ig_skew_weights(ctypes.byref(args)), "ig_skew_weights")
    return out


def ig_skew_apply(A: np.ndarray, M: np.ndarray, nthreads: int = 0) -> np.ndarray:
    A = np.ascontiguousarray(A, dtype=np.float64)
    M = np.ascontiguousarray(M, dtype=np.float64)
    H, d, _ = A.shape
    out = np.empty_like(M)
    rows = M.size // (H * d)
    _check(load().ig_skew_apply(_ptr(A), H, d, _ptr(M), rows, _ptr(out), int(nthreads)), "ig_skew_apply")
    return out


def ig_store(vals: np.ndarray, dtype: str) -> np.ndarray:
    vals = np.ascontiguousarray(vals, dtype=np.float64)
    out = np.empty(vals.shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    _check(load().ig_store(_ptr(vals), vals.size, _np_dtype(dtype), _ptr(out)), "ig_store")
    return out


def ig_partial_weight_index(Wq_s: np.ndarray, K_s: np.ndarray, r: int, n: int, dtype: str, nthreads: int = 0):
    """chan [H][r] int32 and the packed partial query weight [D][H*r] (stored dtype)."""
    Wq_s = np.ascontiguousarray(Wq_s)
    K_s = np.ascontiguousarray(K_s)
    B, H, n_cap, d = K_s.shape
    D = Wq_s.shape[0]
    chan = np.empty((H, r), dtype=np.int32)
    Wp = np.empty((H * r, D), dtype=Wq_s.dtype)   # one row of D inputs per partial column
    _check(load().ig_partial_weight_index(_ptr(Wq_s), D, H, d, r, _ptr(K_s), B, n_cap, n, _np_dtype(dtype),
                                          _ptr(chan), _ptr(Wp), int(nthreads)), "ig_partial_weight_index")
    return chan, Wp


# ---------------------------------------------------------------- device calls
def ig_rehearse(x, Wq_part, Kp, n: int, scale: float, *, bq_part=None, q_part=None, scores=None, ld=None,
                ws=None, stream=None):
    torch = _torch()
    B, D = x.shape
    Bk, H, n_cap, r = Kp.shape
    ld = n if ld is None else ld
    if q_part is None:
        q_part = torch.empty((B, H, r), dtype=torch.float32, device=x.device)
    if scores is None:
        scores = torch.empty((B, H, ld), dtype=torch.float32, device=x.device)
    ws, wsb = _ws(ws, ig_workspace_size(IG_OP_REHEARSE, B, H, D, 0, r, n, 0), x.device)
    _check(load().ig_rehearse(_ptr(x), _ptr(Wq_part), _ptr(bq_part), _ptr(Kp), B, D, H, r, n, n_cap, _dtype_of(x),
                              float(scale), _ptr(q_part), _ptr(scores), ld, _ptr(ws), wsb, _stream(stream)),
           "ig_rehearse")
    return q_part, scores


def ig_workspace_init(ws, *, stream=None):
    _check(load().ig_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "ig_workspace_init")
    return ws


def ig_workspace_status(ws, *, stream=None, recomputed: bool = False):
    """The status word of a speculation workspace (0, or IG_WS_* bits); with ``recomputed``, also the
    number of sliced top-k rows whose merge recomputed the row's scores.  Waits for ``stream``."""
    v = ctypes.c_uint32(0)
    r = ctypes.c_uint32(0)
    _check(load().ig_workspace_status(_ptr(ws), ws.numel() * ws.element_size(), ctypes.byref(v), ctypes.byref(r),
                                      _stream(stream)), "ig_workspace_status")
    return (int(v.value), int(r.value)) if recomputed else int(v.value)


def ig_set_handover_test_mode(spin_limit: int = 0, withhold: bool = False):
    """Failure-path testing of the speculation hand-over (0, False: normal operation)."""
    _check(load().ig_set_handover_test_mode(spin_limit, 1 if withhold else 0), "ig_set_handover_test_mode")


IG_WS_TIMEOUT, IG_WS_SHAPE = 1, 2


def ig_speculate(x, Wq_part, Kp, n: int, scale: float, mode: str, max_out: int, *, alpha: float = math.inf,
                 k: int = 0, max_sel: int = 0, bq_part=None, idx=None, count=None, counters=None, cmax: int = 65535,
                 victim=None, q_part=None, scores=None, ld=None, ws=None, stream=None):
    """Fused partial query + scores + selection (+ counter update when ``counters`` is given).
    ``ws`` (IG_OP_SPECULATE bytes) must have been zero-filled once by ig_workspace_init."""
    torch = _torch()
    B, D = x.shape
    Bk, H, n_cap, r = Kp.shape
    if idx is None:
        idx = torch.empty((B, H, max_out), dtype=torch.int32, device=x.device)
    if count is None:
        count = torch.empty((B, H), dtype=torch.int32, device=x.device)
    if ld is None:
        ld = scores.shape[2] if scores is not None else n
    if ws is None:
        ws = ig_workspace_init(torch.empty(ig_workspace_size(IG_OP_SPECULATE, B, H, D, 0, r, n, max_out),
                                           dtype=torch.uint8, device=x.device), stream=stream)
    wsb = ws.numel() * ws.element_size()
    _check(load().ig_speculate(_ptr(x), _ptr(Wq_part), _ptr(bq_part), _ptr(Kp), B, D, H, r, n, n_cap, _dtype_of(x),
                               float(scale), _MODES[mode], float(alpha), int(k), int(max_sel), _ptr(idx), _ptr(count),
                               max_out, _ptr(counters), int(cmax), _ptr(victim), _ptr(q_part), _ptr(scores), ld,
                               _ptr(ws), wsb, _stream(stream)), "ig_speculate")
    return idx, count


def ig_speculate_noalloc(x, Wq_part, Kp, n: int, scale: float, mode: str, max_out: int, *, alpha: float = math.inf,
                         k: int = 0, max_sel: int = 0, bq_part=None, idx=None, count=None, counters=None,
                         cmax: int = 65535, victim=None, q_part=None, scores=None, ld=None, stream=None):
    """ig_speculate with the library's static device scratch as its workspace (allocates nothing;
    ``idx`` and ``count`` must be given)."""
    B, D = x.shape
    Bk, H, n_cap, r = Kp.shape
    if idx is None or count is None:
        raise ValueError("ig_speculate_noalloc: idx and count must be preallocated")
    if ld is None:
        ld = scores.shape[2] if scores is not None else n
    _check(load().ig_speculate_noalloc(_ptr(x), _ptr(Wq_part), _ptr(bq_part), _ptr(Kp), B, D, H, r, n, n_cap,
                                       _dtype_of(x), float(scale), _MODES[mode], float(alpha), int(k), int(max_sel),
                                       _ptr(idx), _ptr(count), max_out, _ptr(counters), int(cmax), _ptr(victim),
                                       _ptr(q_part), _ptr(scores), ld, _stream(stream)), "ig_speculate_noalloc")
    return idx, count


IG_NOALLOC_SCRATCH_BYTES = 64 << 20


def ig_select(scores, mode: str, max_out: int, *, n=None, alpha: float = math.inf, k: int = 0, max_sel: int = 0,
              idx=None, count=None, ws=None, stream=None):
    torch = _torch()
    B, H, ld = scores.shape
    n = ld if n is None else n
    if idx is None:
        idx = torch.empty((B, H, max_out), dtype=torch.int32, device=scores.device)
    if count is None:
        count = torch.empty((B, H), dtype=torch.int32, device=scores.device)
    m = _MODES[mode]
    need = ig_workspace_size(IG_OP_SELECT, B, H, 0, 0, 0, n, max_out)  # head average, sliced long rows
    ws, wsb = _ws(ws, need, scores.device)
    _check(load().ig_select(_ptr(scores), B, H, n, ld, m, float(alpha), int(k), int(max_sel), _ptr(idx),
                            _ptr(count), max_out, _ptr(ws), wsb, _stream(stream)), "ig_select")
    return idx, count


def ig_gather_kv(K, V, idx, count, *, Kc=None, Vc=None, stream=None):
    torch = _torch()
    B, H, n_cap, d = K.shape
    max_out = idx.shape[2]
    if Kc is None:
        Kc = torch.empty((B, H, max_out, d), dtype=K.dtype, device=idx.device)
    if Vc is None:
        Vc = torch.empty((B, H, max_out, d), dtype=V.dtype, device=idx.device)
    _check(load().ig_gather_kv(_ptr(K), _ptr(V), _ptr(idx), _ptr(count), B, H, d, n_cap, max_out, _dtype_of(K),
                               _ptr(Kc), _ptr(Vc), _stream(stream)), "ig_gather_kv")
    return Kc, Vc


def ig_sparse_decode_attn(q, K, V, idx, count, scale: float, *, max_out=None, out=None, lse=None, want_lse=True,
                          ws=None, stream=None):
    torch = _torch()
    B, H, ld_rows, d = K.shape
    if max_out is None:
        max_out = idx.shape[2] if idx is not None else ld_rows
    if out is None:
        out = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    ws, wsb = _ws(ws, ig_workspace_size(IG_OP_ATTN, B, H, 0, d, 0, 0, max_out), q.device)
    _check(load().ig_sparse_decode_attn(_ptr(q), _ptr(K), _ptr(V), ld_rows, _ptr(idx), _ptr(count), B, H, d, max_out,
                                        _dtype_of(q), float(scale), _ptr(out), _ptr(lse), _ptr(ws), wsb,
                                        _stream(stream)), "ig_sparse_decode_attn")
    return out, lse


def ig_partial_weight_index_dev(Wq_s, K_s, r: int, n: int, *, chan=None, Wq_part=None, ws=None, stream=None):
    """Device tensors: Wq_s [D][H*d], K_s [B][H][n_cap][d]; returns chan [H][r] int32 and
    Wq_part [H*r][D] (device)."""
    torch = _torch()
    D = Wq_s.shape[0]
    B, H, n_cap, d = K_s.shape
    if chan is None:
        chan = torch.empty((H, r), dtype=torch.int32, device=Wq_s.device)
    if Wq_part is None:
        Wq_part = torch.empty((H * r, D), dtype=Wq_s.dtype, device=Wq_s.device)
    ws, wsb = _ws(ws, ig_workspace_size(IG_OP_SETUP, B, H, D, d, r, n, 0), Wq_s.device)
    _check(load().ig_partial_weight_index_dev(_ptr(Wq_s), D, H, d, r, _ptr(K_s), B, n_cap, int(n), _dtype_of(Wq_s),
                                              _ptr(chan), _ptr(Wq_part), _ptr(ws), wsb, _stream(stream)),
           "ig_partial_weight_index_dev")
    return chan, Wq_part


def ig_decode_layer(attn: Optional[dict] = None, spec: Optional[dict] = None, *, stream=None):
    """Attention of layer l and speculation for layer l+1 in one fused launch (after the projection).

    ``attn``: dict with q, K, V, idx, count, scale, out, and optionally lse, max_out, ws (the arguments
    of ig_sparse_decode_attn).  ``spec``: dict with x, Wq_part, Kp, n, scale, mode, idx, count, ws and
    optionally alpha, k, max_sel, bq_part, counters, cmax, victim, q_part, scores, ld (the arguments of
    ig_speculate; ws zero-filled once).  Output tensors must be preallocated.  Either may be None."""
    a_ref = s_ref = None
    if attn is None and spec is None:
        raise ValueError("nothing to do")
    ref = attn["K"] if attn is not None else spec["Kp"]
    B, H = ref.shape[0], ref.shape[1]
    dtype = _dtype_of(ref)
    d = attn["K"].shape[3] if attn is not None else 0
    if attn is not None:
        K = attn["K"]
        idx = attn.get("idx")
        max_out = attn.get("max_out") or (idx.shape[2] if idx is not None else K.shape[2])
        ws = attn.get("ws")
        a_ref = AttnCall(_ptr(attn["q"]), _ptr(K), _ptr(attn["V"]), K.shape[2], _ptr(idx), _ptr(attn["count"]),
                         max_out, float(attn["scale"]), _ptr(attn["out"]), _ptr(attn.get("lse")), _ptr(ws),
                         ws.numel() * ws.element_size() if ws is not None else 0)
    if spec is not None:
        x, Kp, ws = spec["x"], spec["Kp"], spec["ws"]
        scores = spec.get("scores")
        ld = spec.get("ld") or (scores.shape[2] if scores is not None else spec["n"])
        s_ref = SpecCall(_ptr(x), _ptr(spec["Wq_part"]), _ptr(spec.get("bq_part")), _ptr(Kp), x.shape[1], Kp.shape[3],
                         int(spec["n"]), Kp.shape[2], float(spec["scale"]), _MODES[spec["mode"]],
                         float(spec.get("alpha", math.inf)), int(spec.get("k", 0)), int(spec.get("max_sel", 0)),
                         _ptr(spec["idx"]), _ptr(spec["count"]), spec["idx"].shape[2], _ptr(spec.get("counters")),
                         int(spec.get("cmax", 65535)), _ptr(spec.get("victim")), _ptr(spec.get("q_part")),
                         _ptr(scores), ld, _ptr(ws), ws.numel() * ws.element_size())
    _check(load().ig_decode_layer(B, H, d, dtype, ctypes.byref(a_ref) if a_ref is not None else None,
                                  ctypes.byref(s_ref) if s_ref is not None else None, _stream(stream)),
           "ig_decode_layer")


def ig_pool_touch(counters, idx, count, n: int, cmax: int, *, victim=None, want_victim=False, ws=None, stream=None):
    torch = _torch()
    B, n_cap = counters.shape
    H, max_out = idx.shape[1], idx.shape[2]
    if victim is None and want_victim:
        victim = torch.empty((B,), dtype=torch.int32, device=counters.device)
    ws, wsb = _ws(ws, ig_workspace_size(IG_OP_TOUCH, B, H, 0, 0, 0, n, max_out), counters.device)
    _check(load().ig_pool_touch(_ptr(counters), _ptr(idx), _ptr(count), B, H, n, n_cap, max_out, int(cmax),
                                _ptr(victim), _ptr(ws), wsb, _stream(stream)), "ig_pool_touch")
    return counters, victim


def ig_build_partial_cache(K, chan, Kp, row0: int, row1: int, *, stream=None):
    B, H, n_cap, d = K.shape
    r = Kp.shape[3]
    _check(load().ig_build_partial_cache(_ptr(K), _ptr(chan), _ptr(Kp), B, H, d, r, n_cap, row0, row1,
                                         _dtype_of(K), _stream(stream)), "ig_build_partial_cache")
    return Kp


def ig_append_kv(K, V, Kp, counters, chan, k_new, v_new, n: int, *, victim=None, slot_out=None, stream=None):
    """K = V = None: a pool kept as INT4 records (only the partial key row, counter and slot are written)."""
    B, H, n_cap, r = Kp.shape
    d = k_new.shape[2]
    _check(load().ig_append_kv(_ptr(K), _ptr(V), _ptr(Kp), _ptr(counters), _ptr(chan), _ptr(k_new), _ptr(v_new),
                               _ptr(victim), B, H, d, r, n_cap, n, _dtype_of(k_new), _ptr(slot_out),
                               _stream(stream)),
           "ig_append_kv")
    return slot_out


# ---------------------------------------------------------------- INT4 pool
def ig_int4_record_bytes(d: int) -> int:
    return int(load().ig_int4_record_bytes(int(d)))


def ig_quantize_kv(K, V, KVq, row0: int = 0, nrows: Optional[int] = None, *, slot=None, stream=None):
    """Records of rows [row0, row0 + nrows) of K, V [B][H][ld_rows][d] into KVq [B][H][q_rows][record bytes]
    (a uint8 device tensor or a MappedHost view); slot [B] int32: destination slot[b] + row - row0."""
    B, H, ld_rows, d = K.shape
    q_rows = KVq.shape[2]
    nrows = ld_rows - row0 if nrows is None else nrows
    _check(load().ig_quantize_kv(_ptr(K), _ptr(V), B, H, d, ld_rows, _dtype_of(K), int(row0), int(nrows), _ptr(slot),
                                 _ptr(KVq), q_rows, _stream(stream)), "ig_quantize_kv")
    return KVq


def ig_gather_kv_int4(KVq, idx, count, d: int, *, Kc=None, Vc=None, dtype_out=None, stream=None):
    """Selected records of KVq [B][H][q_rows][record bytes], dequantised into compact Kc, Vc
    [B][H][max_out][d] (bf16 unless Kc is given as float32)."""
    torch = _torch()
    B, H, q_rows, _ = KVq.shape
    max_out = idx.shape[2]
    if Kc is None:
        dt = torch.bfloat16 if dtype_out in (None, "bf16") else torch.float32
        Kc = torch.empty((B, H, max_out, d), dtype=dt, device=idx.device)
        Vc = torch.empty_like(Kc)
    _check(load().ig_gather_kv_int4(_ptr(KVq), _ptr(idx), _ptr(count), B, H, d, q_rows, max_out,
                                    _dtype_of(Kc), _ptr(Kc), _ptr(Vc), _stream(stream)), "ig_gather_kv_int4")
    return Kc, Vc

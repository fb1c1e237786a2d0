"""Device-side helpers for the GPU tests: upload stored arrays, run the library's decode step."""
from __future__ import annotations

import math
import sys
from typing import Optional

import numpy as np


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


from sparse_attention_ig_amd.runtime import DeviceLayer, to_device as dev, to_host as host  # noqa: E402


def to_host(res: dict) -> dict:
    import torch
    torch.cuda.synchronize()
    out = {}
    for k, v in res.items():
        if v is None:
            out[k] = None
        elif k == "counters":
            out[k] = host(v).view(np.uint32).copy()
        else:
            out[k] = host(v).copy()
    return out

"""Shared test helpers (no method arithmetic here)."""
import sys

import numpy as np
import torch


def f64(t):
    """Exact fp64 copy of a torch tensor (bf16/fp32 values are all representable)."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").double().numpy()


def relF(x, ref):
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (n if n > 0 else 1.0))


def eye_off(T):
    """T - I for a stack of square blocks (reports the error of the non-trivial part)."""
    C = T.shape[-1]
    return T - np.eye(C)


def say(msg):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(msg, flush=True)
    sys.stdout.flush()


def cuda(t):
    return t.to("cuda").contiguous()

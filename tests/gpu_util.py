"""Helpers shared by the GPU tests: move seeded numpy inputs to the device and run
the C ABI through the thin binding.  Holds no quantisation arithmetic."""
import sys

import numpy as np


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.float16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_np(t, dtype=None):
    a = t.detach().cpu().numpy()
    return a.view(dtype) if dtype is not None else a


def announce(msg: str):
    """Name the case before any GPU step, flushed, so a failing run says where it was."""
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def oracle_codec(K, O, c):
    """Binding codec -> oracle codec (same fields, separate classes)."""
    return O.Codec(c.codebook, c.bits, c.group, rot=c.rot_width, aux_bits=c.aux_bits)

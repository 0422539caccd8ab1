"""Binary16/binary32 rounding helpers of the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def rn16(x) -> np.ndarray:
    """fp32 -> fp16 scale: saturate to +-65504, RN16, and store -0 as +0."""
    x = np.clip(np.asarray(x, dtype=F32), F32(-65504.0), F32(65504.0))
    h = x.astype(np.float16)
    return np.where(h == 0, np.float16(0.0), h)


def inv32(s16: np.ndarray) -> np.ndarray:
    """RN32(1 / f32(s)); a zero scale gives a zero reciprocal (all codes at 0)."""
    s = np.asarray(s16).astype(F32)
    out = np.zeros_like(s)
    nz = s != 0
    out[nz] = F32(1.0) / s[nz]
    return out



"""Oracle bit accounting (bits per stored value, scales included).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Group scales count in the totals ([E21W, Result]: 3.5 bits per value for 3-bit
at group 32, 4.5 for 4-bit; [E22L, What I tested]: 3.125 / 3.25 / 3.5 / 3.625
for the four arms, averaged over keys and values); NF4 or int4 at group 64 is
4.25 ([FMAG-6, Milestone]); fp16 anchor layers count 16 bits ([FMAG-6, Minimal
recipe]).  The rFFT codecs count the exact bits stored per row divided by
head_dim; [FMAG-R] gives the payload-only figure (4 + 8) * 33 / 64 = 6.1875 at
head_dim 64, tending to 6 as head_dim grows.
"""
from __future__ import annotations

from .codec import FP16, INT_MINMAX, RFFT_CART, RFFT_POLAR, Codec


def bits_per_value(codec: Codec, D: int) -> float:
    cb = codec.codebook
    if cb == FP16:
        return 16.0
    if cb in (RFFT_POLAR, RFFT_CART):
        F = D // 2 + 1
        ng = -(-F // codec.group)
        if cb == RFFT_POLAR:
            bits = F * (codec.bits + codec.aux_bits) + 16 * ng
        else:
            bits = 2 * F * codec.bits + 16 * 2 * ng
        return bits / D
    n_params = 2 if cb == INT_MINMAX else 1
    return codec.code_bits() + 16.0 * n_params / codec.group


def kv_bits_per_value(k: Codec, v: Codec, D: int, anchor_layers: int = 0, layers: int = 1) -> float:
    """Mean of K and V bits per value over `layers` layers, of which
    `anchor_layers` are stored as fp16."""
    q = (bits_per_value(k, D) + bits_per_value(v, D)) / 2.0
    return (anchor_layers * 16.0 + (layers - anchor_layers) * q) / layers


def rfft_payload_bits_per_value(mag_bits: int, phase_bits: int, D: int) -> float:
    """Payload only (no scales): (mag + phase) bits on D/2 + 1 bins per D reals."""
    return (mag_bits + phase_bits) * (D // 2 + 1) / D

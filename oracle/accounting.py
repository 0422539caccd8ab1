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

import numpy as np

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


def tiles(segments, layers: int, tokens: int, heads: int = 1) -> bool:
    """True when the segments (layer0, n_layers, token0, n_tokens[, head0, n_heads])
    cover every (layer, head, token) of a layers x heads x tokens cache exactly
    once (a segment without a head range holds every head)."""
    cover = np.zeros((layers, heads, tokens), dtype=np.int64)
    for sg in segments:
        l0, nl, t0, nt = sg[:4]
        h0, nh = (sg[4], sg[5]) if len(sg) > 4 else (0, heads)
        if min(nl, nt, nh) < 1 or min(l0, t0, h0) < 0 or l0 + nl > layers or t0 + nt > tokens or h0 + nh > heads:
            return False
        cover[l0:l0 + nl, h0:h0 + nh, t0:t0 + nt] += 1
    return bool(np.all(cover == 1))


def effective_bits(segments, layers: int, tokens: int, D: int, heads: int = 1) -> float:
    """Bits per cached value of a cache tiled by segments (k_codec, v_codec,
    layer0, n_layers, token0, n_tokens[, head0, n_heads]): each segment's K/V mean
    bits per value weighted by the layers x heads x tokens it holds.

    [FMAG-6, Milestone / Minimal recipe / Best results]: anchored rows count at
    their own precision in the "effective bits"; decode anchors kept for the
    prompt (L tokens) and the first D decoded tokens cost L + D rows on each
    anchored layer, so the figure tends to the anchor precision as the prompt
    grows, while a single fp16 anchor layer adds (16 - b) / n_layers.
    """
    assert tiles([sg[2:] for sg in segments], layers, tokens, heads)
    tot = 0.0
    for sg in segments:
        kc, vc, l0, nl, t0, nt = sg[:6]
        nh = sg[7] if len(sg) > 6 else heads
        tot += (bits_per_value(kc, D) + bits_per_value(vc, D)) / 2.0 * nl * nt * nh
    return tot / (layers * tokens * heads)

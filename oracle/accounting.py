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


def tiles(segments, layers: int, tokens: int) -> bool:
    """True when the segments (layer0, n_layers, token0, n_tokens) cover every
    (layer, token) of a layers x tokens cache exactly once."""
    cover = [[0] * tokens for _ in range(layers)]
    for (l0, nl, t0, nt) in segments:
        if nl < 1 or nt < 1 or l0 < 0 or t0 < 0 or l0 + nl > layers or t0 + nt > tokens:
            return False
        for l in range(l0, l0 + nl):
            for t in range(t0, t0 + nt):
                cover[l][t] += 1
    return all(c == 1 for row in cover for c in row)


def effective_bits(segments, layers: int, tokens: int, D: int) -> float:
    """Bits per cached value of a cache tiled by segments (k_codec, v_codec,
    layer0, n_layers, token0, n_tokens): each segment's K/V mean bits per value
    weighted by the layers x tokens it holds.

    [FMAG-6, Milestone / Minimal recipe / Best results]: anchored rows count at
    their own precision in the "effective bits"; decode anchors kept for the
    prompt (L tokens) and the first D decoded tokens cost L + D rows on each
    anchored layer, so the figure tends to the anchor precision as the prompt
    grows, while a single fp16 anchor layer adds (16 - b) / n_layers.
    """
    assert tiles([(l0, nl, t0, nt) for (_, _, l0, nl, t0, nt) in segments], layers, tokens)
    tot = 0.0
    for (kc, vc, l0, nl, t0, nt) in segments:
        tot += (bits_per_value(kc, D) + bits_per_value(vc, D)) / 2.0 * nl * nt
    return tot / (layers * tokens)

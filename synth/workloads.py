"""Seeded synthetic stand-ins for the KV caches the pages measure on.

The pages measure on real captured caches that are not available here (the
E21W post "PROVISIONAL: known 3-bit KV cache methods on the 4B fall well short
of 4-bit quality (proxy queries)", sections "Benchmark" and "What I tested":
8 full-attention layers x 4 KV heads, head_dim 256, 6,000 tokens, proxy
queries; the E22L post "Can 4-bit keys and 2-bit values hit a 1M-token memory
budget?", section "What I tested": 64K-token spans).  Each workload below draws
fp16 K/V of the same shape and structure (outlier channels, RoPE-rotated keys,
causal proxy queries) from a seeded generator.

Seeding: every (batch b, layer l, KV head h, tensor) unit has its own
``numpy.random.default_rng`` stream, so any unit can be regenerated on its own
(the oracle samples units of the full-size workloads) and units can be drawn in
parallel.  Values are float32 standard normals, scaled, then rounded to fp16
(round-to-nearest-even).

Nothing in this module computes a quantiser, transform or attention.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_K, _V = 0, 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    B: int            # batch (sequences)
    L: int            # layers
    H: int            # KV heads
    T: int            # tokens
    D: int            # head_dim
    Hq: int           # query heads (GQA: Hq % H == 0)
    n_q: int          # queries per (batch, layer)
    k_sigma: float
    v_sigma: float
    n_outlier: int    # outlier K channels per (layer, head)
    outlier_mult: float
    outlier_layers: tuple | None  # None: every layer
    rope: bool        # keys (and queries) RoPE-rotated by position, base 1e4
    query_kind: str   # "normal" | "keys" (queries are keys at sampled positions)
    pos_range: tuple | None       # query positions [lo, hi) for causal probes
    causal_inclusive: bool        # keys [0, p] (True) or [0, p) (False)
    description: str
    k_mean_share: float = 0.0     # share of expected key energy in a shared per-(layer, head) mean
    k_head_scales: tuple | None = None   # per KV head key multipliers (head h uses [h % len]); None: 1

    def with_sizes(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def rows(self) -> int:
        return self.B * self.L * self.H * self.T


WORKLOADS = {
    # Tiny reference: one layer, one KV head, min-max 4-bit g32, causal queries.
    "c1": Workload("c1", 1, B=1, L=1, H=1, T=512, D=128, Hq=1, n_q=16,
                   k_sigma=1.0, v_sigma=1.0, n_outlier=4, outlier_mult=8.0,
                   outlier_layers=None, rope=False, query_kind="normal",
                   pos_range=(256, 512), causal_inclusive=True,
                   description="1x1x1x512x128, K 4 channels x8, 16 causal queries in [256,512)"),
    # Proxy-query probe (E21W): 3 sequences, seq 0 calibrates per-channel K scales.
    "c2": Workload("c2", 2, B=3, L=8, H=4, T=6000, D=256, Hq=4, n_q=128,
                   k_sigma=1.0, v_sigma=0.5, n_outlier=8, outlier_mult=10.0,
                   outlier_layers=None, rope=False, query_kind="keys",
                   pos_range=(3000, 6000), causal_inclusive=False,
                   description="3 seq x 8 x 4 x 6000 x 256, K 8 ch x10, V sd 0.5, proxy queries = keys"),
    # Long-context decode at 64K (E22L arm A shape): the timed workload.
    "c3": Workload("c3", 3, B=1, L=8, H=4, T=65536, D=256, Hq=16, n_q=256,
                   k_sigma=1.0, v_sigma=1.0, n_outlier=8, outlier_mult=10.0,
                   outlier_layers=None, rope=False, query_kind="normal",
                   pos_range=None, causal_inclusive=False,
                   description="1 x 8 x 4 x 65536 x 256, GQA 16:4, 256 decode queries"),
    # Extreme low-bit codebooks with an fp16 anchor layer 0.
    "c4": Workload("c4", 4, B=4, L=32, H=8, T=16384, D=128, Hq=32, n_q=64,
                   k_sigma=1.0, v_sigma=1.0, n_outlier=4, outlier_mult=8.0,
                   outlier_layers=(0,), rope=False, query_kind="normal",
                   pos_range=None, causal_inclusive=False,
                   description="4 x 32 x 8 x 16384 x 128, layer-0 K 4 ch x8, 64 decode steps"),
    # Transform ablation: RoPE-rotated keys, head_dim 128.
    "c5": Workload("c5", 5, B=4, L=16, H=8, T=32768, D=128, Hq=32, n_q=64,
                   k_sigma=1.0, v_sigma=1.0, n_outlier=0, outlier_mult=1.0,
                   outlier_layers=None, rope=True, query_kind="normal",
                   pos_range=None, causal_inclusive=False,
                   description="4 x 16 x 8 x 32768 x 128, RoPE keys (base 1e4), 64 decode steps"),
}


def get(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.with_sizes(**overrides) if overrides else w


def unit_rng(w: Workload, *key: int) -> np.random.Generator:
    """Independent stream for one unit; `key` identifies what is drawn."""
    return np.random.default_rng([w.cfg_id, *key])


def _outlier_channels(w: Workload, l: int, h: int) -> np.ndarray:
    # A property of the (synthetic) model: the same for every sequence.
    if w.n_outlier == 0:
        return np.zeros(0, dtype=np.int64)
    if w.outlier_layers is not None and l not in w.outlier_layers:
        return np.zeros(0, dtype=np.int64)
    rng = unit_rng(w, 100, l, h)
    return np.sort(rng.choice(w.D, size=w.n_outlier, replace=False))


def _shared_key_mean(w: Workload, l: int, h: int, n_out: int) -> np.ndarray:
    """A per-(layer, head) vector added to every key row (a property of the
    synthetic model, the same for every sequence), scaled so that it carries
    k_mean_share of the expected key energy."""
    m = unit_rng(w, 200, l, h).standard_normal(w.D)
    e_row = w.k_sigma ** 2 * ((w.D - n_out) + n_out * w.outlier_mult ** 2)
    target = w.k_mean_share / (1.0 - w.k_mean_share) * e_row
    return (m * np.sqrt(target / float(m @ m))).astype(np.float32)


def _rope_fp64(x: np.ndarray, pos: np.ndarray, D: int) -> np.ndarray:
    """Rotate-half RoPE (pairs (i, i + D/2), theta_i = 1e4^(-2i/D)) in fp64."""
    half = D // 2
    inv_freq = 10000.0 ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    ang = pos.astype(np.float64)[:, None] * inv_freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1 = x[..., :half].astype(np.float64)
    x2 = x[..., half:].astype(np.float64)
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def gen_unit(w: Workload, b: int, l: int, h: int, tensor: str) -> np.ndarray:
    """fp16 [T, D] rows of one (batch, layer, KV head) unit; tensor 'K' or 'V'."""
    tid = _K if tensor == "K" else _V
    rng = unit_rng(w, 1, b, l, h, tid)
    x = rng.standard_normal((w.T, w.D), dtype=np.float32)
    if tid == _K:
        if w.k_sigma != 1.0:
            x *= np.float32(w.k_sigma)
        ch = _outlier_channels(w, l, h)
        if ch.size:
            x[:, ch] *= np.float32(w.outlier_mult)
        if w.k_head_scales is not None:
            x *= np.float32(w.k_head_scales[h % len(w.k_head_scales)])
        if w.k_mean_share > 0.0:
            x += _shared_key_mean(w, l, h, ch.size)[None, :]
        if w.rope:
            return _rope_fp64(x, np.arange(w.T), w.D).astype(np.float16)
    else:
        if w.v_sigma != 1.0:
            x *= np.float32(w.v_sigma)
    return x.astype(np.float16)


def _threads() -> int:
    return max(1, min(8, len(os.sched_getaffinity(0))))


def gen_kv(w: Workload, layers: range | None = None, threads: int | None = None):
    """Full fp16 K and V arrays [B][L'][H][T][D] for the given layers (default all)."""
    layers = range(w.L) if layers is None else layers
    Ls = len(layers)
    K = np.empty((w.B, Ls, w.H, w.T, w.D), dtype=np.float16)
    V = np.empty_like(K)
    jobs = [(b, li, l, h) for b in range(w.B) for li, l in enumerate(layers) for h in range(w.H)]

    def fill(job):
        b, li, l, h = job
        K[b, li, h] = gen_unit(w, b, l, h, "K")
        V[b, li, h] = gen_unit(w, b, l, h, "V")

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(fill, jobs))
    return K, V


def query_positions(w: Workload, b: int) -> np.ndarray:
    """Distinct causal probe positions for sequence b (None for decode workloads)."""
    lo, hi = w.pos_range
    rng = unit_rng(w, 200, b)
    return np.sort(rng.choice(np.arange(lo, hi), size=w.n_q, replace=False))


def gen_queries(w: Workload, K: np.ndarray | None = None, layers: range | None = None):
    """Queries fp16 [B][L'][n_q][Hq][D] and causal key counts int32 [B][L'][n_q].

    * "normal": q ~ N(0,1); decode workloads attend all T keys, causal probes
      attend keys [0, p] for a sampled position p.
    * "keys": proxy queries are the fp16 keys at sampled positions, each
      attending the keys strictly before it (E21W "Benchmark" row); needs K.
    """
    layers = range(w.L) if layers is None else layers
    Ls = len(layers)
    q = np.empty((w.B, Ls, w.n_q, w.Hq, w.D), dtype=np.float16)
    kv_len = np.empty((w.B, Ls, w.n_q), dtype=np.int32)
    for b in range(w.B):
        pos = query_positions(w, b) if w.pos_range is not None else None
        for li, l in enumerate(layers):
            if w.query_kind == "keys":
                assert K is not None and w.Hq == w.H
                q[b, li] = np.transpose(K[b, li][:, pos, :], (1, 0, 2))
                kv_len[b, li] = pos
                continue
            rng = unit_rng(w, 300, b, l)
            x = rng.standard_normal((w.n_q, w.Hq, w.D), dtype=np.float32)
            if w.rope:
                xr = _rope_fp64(x.reshape(-1, w.D), np.full(w.n_q * w.Hq, w.T), w.D)
                q[b, li] = xr.reshape(w.n_q, w.Hq, w.D).astype(np.float16)
            else:
                q[b, li] = x.astype(np.float16)
            if pos is not None:
                kv_len[b, li] = pos + 1 if w.causal_inclusive else pos
            else:
                kv_len[b, li] = w.T
    return q, kv_len

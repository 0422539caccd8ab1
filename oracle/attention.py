"""Oracle attention and error metrics in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definitions ([E21W, Benchmark]: attention output and the attention
distribution are compared against fp16; K/V error is squared error over signal
energy; attention error is the relative error of the attention output; KL is
the divergence of the attention distribution from the fp16 one):

* logits l_t = sigma * (q . k_t) over keys t < n, sigma = 1/sqrt(D) unless given;
* p = softmax(l) (max-subtracted), o = sum_t p_t v_t;
* KL_r = sum_t p_t (ln p_t - ln phat_t) with p from fp16 K/V and phat from the
  dequantised K/V, in nats; terms with p_t = 0 contribute 0;
* eps_r = ||ohat - o||_2 / ||o||_2;
* E_u = sum (xhat - x)^2 / sum x^2 per (batch, layer, KV head) unit.

GQA: query head j reads KV head floor(j / (Hq/H)) (the pages never say; this is
the repeat-kv convention of the Hugging Face simulation in [E22L, Result]).
"""
from __future__ import annotations

import numpy as np


def _lse(x: np.ndarray) -> np.ndarray:
    m = x.max(-1, keepdims=True)
    return (m + np.log(np.exp(x - m).sum(-1, keepdims=True)))[..., 0]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, n: int, sm_scale: float):
    """q [G, D], K/V [T, D] (any float, used in fp64), keys [0, n) ->
    (out [G, D], lse [G], logits [G, n])."""
    q = np.asarray(q, dtype=np.float64)
    if n == 0:
        G, D = q.shape
        return np.zeros((G, V.shape[1])), np.full(G, -np.inf), np.zeros((G, 0))
    k = np.asarray(K[:n], dtype=np.float64)
    v = np.asarray(V[:n], dtype=np.float64)
    logits = sm_scale * (q @ k.T)
    m = logits.max(-1, keepdims=True)
    e = np.exp(logits - m)
    Z = e.sum(-1, keepdims=True)
    p = e / Z
    return p @ v, (m + np.log(Z))[..., 0], logits


def attend_unit(q, K, V, kv_len, sm_scale):
    """All queries of one (batch, layer, KV head) unit: q [nq, G, D] ->
    (out [nq, G, D], lse [nq, G])."""
    nq, G, D = q.shape
    out = np.zeros((nq, G, V.shape[1]))
    lse = np.zeros((nq, G))
    for i in range(nq):
        out[i], lse[i], _ = attend(q[i], K, V, int(kv_len[i]), sm_scale)
    return out, lse


def _scale(D, sm_scale):
    return 1.0 / np.sqrt(D) if not sm_scale else float(sm_scale)


def decode_attn(q16, Kd, Vd, kv_len=None, sm_scale=0.0):
    """q16 [B][L][nq][Hq][D] fp16, Kd/Vd [B][L][H][T][D] dequantised (or fp16)
    -> (out float64 [B][L][nq][Hq][D], lse [B][L][nq][Hq])."""
    B, L, nq, Hq, D = q16.shape
    H, T = Kd.shape[2], Kd.shape[3]
    G = Hq // H
    s = _scale(D, sm_scale)
    out = np.zeros((B, L, nq, Hq, Vd.shape[-1]))
    lse = np.zeros((B, L, nq, Hq))
    q = q16.astype(np.float64)
    for b in range(B):
        for l in range(L):
            n = np.full(nq, T) if kv_len is None else kv_len[b, l]
            for h in range(H):
                o, z = attend_unit(q[b, l, :, h * G:(h + 1) * G], Kd[b, l, h], Vd[b, l, h], n, s)
                out[b, l, :, h * G:(h + 1) * G] = o
                lse[b, l, :, h * G:(h + 1) * G] = z
    return out, lse


def kl_div(logits_ref: np.ndarray, logits_q: np.ndarray) -> np.ndarray:
    """KL(p_ref || p_q) in nats over the last axis of two logit arrays."""
    if logits_ref.shape[-1] == 0:
        return np.zeros(logits_ref.shape[:-1])
    lp = logits_ref - _lse(logits_ref)[..., None]
    lq = logits_q - _lse(logits_q)[..., None]
    p = np.exp(lp)
    return np.where(p > 0, p * (lp - lq), 0.0).sum(-1)


def rel_err(o_hat: np.ndarray, o: np.ndarray) -> np.ndarray:
    num = np.linalg.norm(o_hat - o, axis=-1)
    den = np.linalg.norm(o, axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)


def kv_err_unit(x16: np.ndarray, x_hat: np.ndarray):
    """(sum (xhat - x)^2, sum x^2) in fp64 for one unit's rows."""
    x = x16.astype(np.float64)
    d = np.asarray(x_hat, dtype=np.float64) - x
    return float((d * d).sum()), float((x * x).sum())


def renyi2(logits: np.ndarray) -> np.ndarray:
    """Renyi entropy of order 2 of softmax(logits), -ln sum_t p_t^2, in nats
    ([LCPP] Finding 2: H_2(h) of a head's attention distribution); 0 for no keys."""
    if logits.shape[-1] == 0:
        return np.zeros(logits.shape[:-1])
    lp = logits - _lse(logits)[..., None]
    return -np.log(np.exp(2.0 * lp).sum(-1))


def js_div(logits_ref: np.ndarray, logits_q: np.ndarray) -> np.ndarray:
    """Jensen-Shannon divergence of the two attention distributions in nats:
    (KL(p || m) + KL(phat || m)) / 2 with m = (p + phat) / 2, 0 ln 0 = 0
    ([FMAG-R] reply's diagnostic ladder: attention KL / JS); 0 for no keys."""
    if logits_ref.shape[-1] == 0:
        return np.zeros(logits_ref.shape[:-1])
    p = np.exp(logits_ref - _lse(logits_ref)[..., None])
    r = np.exp(logits_q - _lse(logits_q)[..., None])
    m = 0.5 * (p + r)
    a = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0) / np.where(m > 0, m, 1.0)), 0.0).sum(-1)
    b = np.where(r > 0, r * np.log(np.where(r > 0, r, 1.0) / np.where(m > 0, m, 1.0)), 0.0).sum(-1)
    return 0.5 * (a + b)


def logit_relerr(logits_ref: np.ndarray, logits_q: np.ndarray) -> np.ndarray:
    """||lhat - l||_2 / ||l||_2 over the attended keys (the ladder's QK-logit error);
    0 for no keys or an all-zero reference."""
    num = np.sqrt(((logits_q - logits_ref) ** 2).sum(-1))
    den = np.sqrt((logits_ref ** 2).sum(-1))
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)


def top1_flip(logits_ref: np.ndarray, logits_q: np.ndarray) -> np.ndarray:
    """1 where the most-attended key differs (first index on ties), else 0 (the
    ladder's top-attended-token flips); 0 for no keys."""
    if logits_ref.shape[-1] == 0:
        return np.zeros(logits_ref.shape[:-1])
    return (np.argmax(logits_ref, -1) != np.argmax(logits_q, -1)).astype(np.float64)


def entropy_adaptive_bits(h2: np.ndarray, b_avg: float) -> np.ndarray:
    """Per-head bits b_h = b_avg + 0.25 (H_avg - H_2(h)) ([LCPP] Finding 2), with
    H_avg the mean of H_2 over the heads given (the plain reading); the mean of
    b_h is b_avg."""
    h2 = np.asarray(h2, dtype=np.float64)
    return b_avg + 0.25 * (h2.mean() - h2)


def attn_error_ex(q16, K16, V16, Kd, Vd, kv_len=None, sm_scale=0.0, units=None):
    """attn_error plus the other rungs of the diagnostic ladder, per row: Renyi-2
    entropy of the fp16 distribution, JS divergence, QK-logit relative error and
    top-1 flips (dict of arrays [B][L][nq][Hq]; 'kv_err' [B][L][H][4])."""
    B, L, nq, Hq, D = q16.shape
    H, T = K16.shape[2], K16.shape[3]
    G = Hq // H
    s = _scale(D, sm_scale)
    names = ("kl", "relerr", "renyi2", "js", "logit_relerr", "top1_flip")
    res = {k: np.full((B, L, nq, Hq), np.nan) for k in names}
    res["kv_err"] = np.full((B, L, H, 4), np.nan)
    q = q16.astype(np.float64)
    todo = units if units is not None else [(b, l, h) for b in range(B) for l in range(L) for h in range(H)]
    for (b, l, h) in todo:
        n = np.full(nq, T) if kv_len is None else kv_len[b, l]
        for i in range(nq):
            o, _, lr = attend(q[b, l, i, h * G:(h + 1) * G], K16[b, l, h], V16[b, l, h], int(n[i]), s)
            oh, _, lq = attend(q[b, l, i, h * G:(h + 1) * G], Kd[b, l, h], Vd[b, l, h], int(n[i]), s)
            sl = (b, l, i, slice(h * G, (h + 1) * G))
            res["kl"][sl] = kl_div(lr, lq)
            res["relerr"][sl] = rel_err(oh, o)
            res["renyi2"][sl] = renyi2(lr)
            res["js"][sl] = js_div(lr, lq)
            res["logit_relerr"][sl] = logit_relerr(lr, lq)
            res["top1_flip"][sl] = top1_flip(lr, lq)
        res["kv_err"][b, l, h, 0:2] = kv_err_unit(K16[b, l, h], Kd[b, l, h])
        res["kv_err"][b, l, h, 2:4] = kv_err_unit(V16[b, l, h], Vd[b, l, h])
    return res


def attn_error(q16, K16, V16, Kd, Vd, kv_len=None, sm_scale=0.0, units=None):
    """Per-row KL and relative output error of attention through (Kd, Vd) vs
    fp16 (K16, V16), plus per-unit K/V error sums.

    Returns kl [B][L][nq][Hq], relerr [B][L][nq][Hq], kv_err [B][L][H][4] with
    (sum dK^2, sum K^2, sum dV^2, sum V^2).  `units`, if given, is a list of
    (b, l, h) to evaluate (others are left as NaN).
    """
    B, L, nq, Hq, D = q16.shape
    H, T = K16.shape[2], K16.shape[3]
    G = Hq // H
    s = _scale(D, sm_scale)
    kl = np.full((B, L, nq, Hq), np.nan)
    re = np.full((B, L, nq, Hq), np.nan)
    kv = np.full((B, L, H, 4), np.nan)
    q = q16.astype(np.float64)
    todo = units if units is not None else [(b, l, h) for b in range(B) for l in range(L) for h in range(H)]
    for (b, l, h) in todo:
        n = np.full(nq, T) if kv_len is None else kv_len[b, l]
        for i in range(nq):
            o, _, lr = attend(q[b, l, i, h * G:(h + 1) * G], K16[b, l, h], V16[b, l, h], int(n[i]), s)
            oh, _, lq = attend(q[b, l, i, h * G:(h + 1) * G], Kd[b, l, h], Vd[b, l, h], int(n[i]), s)
            kl[b, l, i, h * G:(h + 1) * G] = kl_div(lr, lq)
            re[b, l, i, h * G:(h + 1) * G] = rel_err(oh, o)
        kv[b, l, h, 0:2] = kv_err_unit(K16[b, l, h], Kd[b, l, h])
        kv[b, l, h, 2:4] = kv_err_unit(V16[b, l, h], Vd[b, l, h])
    return kl, re, kv


def assemble_segments(segments, B: int, L: int, H: int, T: int, D: int):
    """The logical [B][L][H][T][D] cache from dequantised segments (Kd_s, Vd_s,
    layer0, token0[, head0]), each [B][L_s][H_s][T_s][D]: every segment placed at
    its layers, heads and tokens.  Decoding over segments is, by definition,
    decoding over this assembled cache."""
    Kd = np.full((B, L, H, T, D), np.nan, dtype=np.float32)
    Vd = np.full((B, L, H, T, D), np.nan, dtype=np.float32)
    for sg in segments:
        ks, vs, l0, t0 = sg[:4]
        h0 = sg[4] if len(sg) > 4 else 0
        nl, nh, nt = ks.shape[1], ks.shape[2], ks.shape[3]
        Kd[:, l0:l0 + nl, h0:h0 + nh, t0:t0 + nt] = ks
        Vd[:, l0:l0 + nl, h0:h0 + nh, t0:t0 + nt] = vs
    assert not np.isnan(Kd).any() and not np.isnan(Vd).any(), "segments do not cover the cache"
    return Kd, Vd

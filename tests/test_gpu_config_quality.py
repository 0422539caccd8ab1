"""The quality reports of the configurations at full size (the launches bench.py's c1,
c2 and c5 workloads run): the error kernel's per-row KL and output error and per-unit
K/V squared error against the oracle, on every row of the tiny reference and on
sampled (sequence, layer, head) units of the proxy-query probe's arms A-D at 3 and 4
bits ([E21W] What I tested, Result) and of the transform ablation's arms ([FMAG-R] the
Colab-probe reply: rFFT polar and Cartesian codes against a Hadamard control).

Bars: KL and output error within 1e-4 absolute per row, K/V error sums within 1e-9
relative (fp64 sums of the same dequantised values in another order)."""
import functools

import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import announce, oracle_codec, to_dev, to_np

pytestmark = pytest.mark.gpu

KL_TOL = 1e-4
RE_TOL = 1e-4


@functools.lru_cache(maxsize=1)
def _data(name):
    w = synth.get(name)
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w, Kx)
    if name == "c5":                                  # 16 decode queries, as bench.py reports
        q = np.ascontiguousarray(q[:, :, :16])
        kv_len = np.ascontiguousarray(kv_len[:, :, :16])
    return w, Kx, Vx, q, kv_len


def _gpu_error(K, Kx, Vx, kp, vp, q, kv_len, shape, Hq):
    import torch
    B, L, nq = q.shape[0], q.shape[1], q.shape[2]
    kl = torch.empty((B, L, nq, Hq), dtype=torch.float32, device="cuda:0")
    re = torch.empty_like(kl)
    kv = torch.empty((B, L, shape.heads, 4), dtype=torch.float64, device="cuda:0")
    wb = K.kvq_attn_error_workspace(shape, Hq, nq)
    ws = torch.empty(max(wb, 16), dtype=torch.uint8, device="cuda:0")
    K.kvq_attn_error(Kx, Vx, kp, vp, Hq, nq, to_dev(q), to_dev(kv_len), 0.0, kl, re, kv, ws, wb)
    torch.cuda.synchronize()
    return to_np(kl), to_np(re), to_np(kv)


def _compare_units(K, w, Kx, Vx, q, kv_len, kc, vc, chan, units, kl, re, kv):
    """Oracle attention error of each sampled unit (its K, V, channel scales and
    queries sliced out) against the GPU rows of that unit."""
    G = w.Hq // w.H
    okc, ovc = oracle_codec(K, O, kc), oracle_codec(K, O, vc)
    for (b, l, h) in units:
        ku = Kx[b:b + 1, l:l + 1, h:h + 1]
        vu = Vx[b:b + 1, l:l + 1, h:h + 1]
        cu = chan[l:l + 1, h:h + 1] if chan is not None else None
        wk, sk, zk = O.quantize_pack(ku, okc, cu)
        Kd = O.dequant(wk, sk, zk, okc, ku.shape, cu)
        if vc.codebook == K.FP16:
            Vd = vu.astype(np.float32)
        else:
            wv, sv, zv = O.quantize_pack(vu, ovc)
            Vd = O.dequant(wv, sv, zv, ovc, vu.shape)
        qu = np.ascontiguousarray(q[b:b + 1, l:l + 1, :, h * G:(h + 1) * G])
        klo, reo, kvo = O.attn_error(qu, ku, vu, Kd, Vd, kv_len[b:b + 1, l:l + 1])
        rows = (b, l, slice(None), slice(h * G, (h + 1) * G))
        assert np.abs(kl[rows] - klo[0, 0]).max() < KL_TOL, f"unit {(b, l, h)} KL"
        assert np.abs(re[rows] - reo[0, 0]).max() < RE_TOL, f"unit {(b, l, h)} output error"
        got = kv[b, l, h]
        ref = kvo[0, 0, 0]
        assert np.all(np.abs(got - ref) <= 1e-9 * np.abs(ref) + 1e-12), f"unit {(b, l, h)} K/V error sums"


def test_c1_tiny_reference_every_row():
    import kv_cache_bit_fwht_amd as K
    w, Kx, Vx, q, kv_len = _data("c1")
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    codec = K.Codec(K.INT_MINMAX, 4, 32, 0)
    kp, vp = K.alloc_packed(codec, shape), K.alloc_packed(codec, shape)
    kd, vd = to_dev(Kx), to_dev(Vx)
    announce("c1 full: int4 min-max g32")
    K.kvq_quantize_pack_kv(kd, vd, kp, vp)
    kl, re, kv = _gpu_error(K, kd, vd, kp, vp, q, kv_len, shape, w.Hq)
    _compare_units(K, w, Kx, Vx, q, kv_len, codec, codec, None, [(0, 0, 0)], kl, re, kv)


C2_ARMS = [(arm, b) for b in (3, 4) for arm in "ABCD"]


@pytest.mark.parametrize("arm,b", C2_ARMS)
def test_c2_arms_full_size_sampled_units(arm, b):
    import torch
    import kv_cache_bit_fwht_amd as K
    w, Kx, Vx, q, kv_len = _data("c2")
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    rot = 256 if arm in "BD" else 0
    cb = K.INT_ABSMAX if arm in "BD" else K.INT_MINMAX
    kc = vc = K.Codec(cb, b, 32, rot)
    chan = O.calibrate_chan_scale(Kx[0]) if arm in "CD" else None
    announce(f"c2 full: arm {arm}, {b} bits")
    kd, vd = to_dev(Kx), to_dev(Vx)
    if chan is not None:
        cd = torch.empty((w.L, w.H, w.D), dtype=torch.float32, device="cuda:0")
        K.kvq_calibrate_chan_scale(kd[:1].contiguous(), K.Shape(1, w.L, w.H, w.T, w.D), cd)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(cd), chan)
    kp = K.alloc_packed(kc, shape, chan_scale=cd if chan is not None else None)
    vp = K.alloc_packed(vc, shape)
    K.kvq_quantize_pack_kv(kd, vd, kp, vp)
    kl, re, kv = _gpu_error(K, kd, vd, kp, vp, q, kv_len, shape, w.Hq)
    _compare_units(K, w, Kx, Vx, q, kv_len, kc, vc, chan, [(0, 0, 0), (1, 4, 2), (2, 7, 3)], kl, re, kv)


@pytest.mark.parametrize("arm", ["polar", "cart", "fwht"])
def test_c5_arms_full_size_sampled_units(arm):
    import kv_cache_bit_fwht_amd as K
    w, Kx, Vx, q, kv_len = _data("c5")
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    kc = {"polar": K.Codec(K.RFFT_POLAR, 5, 32, 0, 7), "cart": K.Codec(K.RFFT_CART, 6, 32, 0),
          "fwht": K.Codec(K.INT_ABSMAX, 6, 32, 128)}[arm]
    announce(f"c5 full: {arm}")
    kd, vd = to_dev(Kx), to_dev(Vx)
    kp = K.alloc_packed(kc, shape)
    K.kvq_quantize_pack(kd, kp)
    vp = K.packed_from_fp16(vd, shape)
    kl, re, kv = _gpu_error(K, kd, vd, kp, vp, q, kv_len, shape, w.Hq)
    _compare_units(K, w, Kx, Vx, q, kv_len, kc, K.Codec(K.FP16), None, [(0, 0, 0), (3, 15, 7)], kl, re, kv)

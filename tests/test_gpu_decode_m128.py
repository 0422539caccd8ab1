"""GPU parity of the head_dim-128 MFMA decode (kvq_decode_attn_ex path 2 at head_dim
128) against the CPU oracle: keys ternary or sign at group 8, int8 rows, fp16 or NF4
at group 64, values ternary or sign at group 8, int8 rows, fp16 or 4-bit signed absmax
at group 64, in every combination ([FMAG-6] Milestone and Best results: the extreme
low-bit arms, NF4 keys with 4-bit values, the int8 reference row and the fp16 anchor
layer); and 6-bit signed absmax keys at group 32, unrotated or rotated by the
normalised Hadamard-128, rFFT keys with 6-bit real and imaginary parts at group 32,
and rFFT keys with 5-bit magnitudes at group 32 and 7-bit phases (the Hadamard,
real/imaginary and polar arms of the matched-rate transform control in the Fourier
Magnitude thread's Colab-probe reply).

Bars: attention outputs within 2e-3 relative L2 per row and lse within 1e-4 of the
oracle's fp64 attention over the oracle's dequantised cache; path 0 takes the same
kernel as path 2 (same bits); a cache whose rows past the attended keys hold garbage
(NaN scales, all-ones codes) decodes as a clean one."""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import announce, oracle_codec, to_dev, to_np
from tests.test_gpu_attn import _check_decode, _gpu_decode

pytestmark = pytest.mark.gpu

K_CODECS = ["ter", "sign", "int8", "f16", "nf4", "i6", "i6h", "rc", "rp"]
V_CODECS = ["ter", "sign", "int8", "f16", "i4"]


def _codec(K, name):
    return {"ter": K.Codec(K.TERNARY, 2, 8, 0), "sign": K.Codec(K.SIGN, 1, 8, 0),
            "int8": K.Codec(K.INT8_SYM, 8, 128, 0), "f16": K.Codec(K.FP16),
            "nf4": K.Codec(K.NF4, 4, 64, 0), "i4": K.Codec(K.INT_ABSMAX, 4, 64, 0),
            "i6": K.Codec(K.INT_ABSMAX, 6, 32, 0), "i6h": K.Codec(K.INT_ABSMAX, 6, 32, 128),
            "rc": K.Codec(K.RFFT_CART, 6, 32, 0), "rp": K.Codec(K.RFFT_POLAR, 5, 32, 0, 7)}[name]


def _pack(K, x, codec, shape):
    xd = to_dev(x)
    if codec.codebook == K.FP16:
        return K.packed_from_fp16(xd, shape), x.astype(np.float32)
    p = K.alloc_packed(codec, shape)
    K.kvq_quantize_pack(xd, p)
    oc = oracle_codec(K, O, codec)
    w, s, z = O.quantize_pack(x, oc)
    return p, O.dequant(w, s, z, oc, x.shape)


def _inputs(B=2, L=2, T=333, n_q=2, Hq=32):
    w = synth.get("c4", B=B, L=L, T=T, n_q=n_q, Hq=Hq)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    return w, Kx, Vx, q


@pytest.mark.parametrize("kname", K_CODECS)
@pytest.mark.parametrize("vname", V_CODECS)
def test_codec_pairs(kname, vname):
    """T = 333 (ragged last step), two queries per row with lengths T and 200."""
    import kv_cache_bit_fwht_amd as K
    w, Kx, Vx, q, = _inputs()
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    kc, vc = _codec(K, kname), _codec(K, vname)
    kp, Kd = _pack(K, Kx, kc, shape)
    vp, Vd = _pack(K, Vx, vc, shape)
    kv_len = np.zeros((w.B, w.L, 2), np.int32)
    kv_len[..., 0] = w.T
    kv_len[..., 1] = 200
    announce(f"m128 decode K={kname} V={vname}")
    out, lse = _gpu_decode(K, kp, vp, q, kv_len, path=2)
    ref_out, ref_lse = O.decode_attn(q, Kd, Vd, kv_len)
    _check_decode(out, lse, ref_out, ref_lse, kv_len)
    out0, lse0 = _gpu_decode(K, kp, vp, q, kv_len, path=0)
    assert np.array_equal(out0, out) and np.array_equal(lse0, lse), "path 0 should take the same kernel"


@pytest.mark.parametrize("G", [1, 2, 3, 4])
def test_query_heads_per_kv_head(G):
    """1-4 query heads per KV head; lengths 0, 1, 31, 32, 33, T-1, T across rows."""
    import kv_cache_bit_fwht_amd as K
    H = 8
    w, Kx, Vx, q = _inputs(B=1, L=2, T=1000, n_q=4, Hq=G * H)
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    kp, Kd = _pack(K, Kx, _codec(K, "ter"), shape)
    vp, Vd = _pack(K, Vx, _codec(K, "int8"), shape)
    kv_len = np.array([[[0, 1, 31, 32], [33, 999, 1000, 517]]], np.int32)
    announce(f"m128 decode G={G}")
    out, lse = _gpu_decode(K, kp, vp, q, kv_len, path=2)
    ref_out, ref_lse = O.decode_attn(q, Kd, Vd, kv_len)
    _check_decode(out, lse, ref_out, ref_lse, kv_len)


@pytest.mark.parametrize("kname", ["i6h", "rc", "rp"])
@pytest.mark.parametrize("G", [1, 2, 3])
def test_query_heads_per_kv_head_transform_keys(G, kname):
    """The 6-bit and rFFT keys (query rotated or transformed in the prologue, high part
    and remainder in alternate columns) with 1-3 query heads per KV head: the columns of
    absent heads carry a zero query; lengths 0, 1, 31, 32, 33, T-1, T across rows."""
    import kv_cache_bit_fwht_amd as K
    H = 8
    w, Kx, Vx, q = _inputs(B=1, L=2, T=1000, n_q=4, Hq=G * H)
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    kp, Kd = _pack(K, Kx, _codec(K, kname), shape)
    vp, Vd = _pack(K, Vx, _codec(K, "i4"), shape)
    kv_len = np.array([[[0, 1, 31, 32], [33, 999, 1000, 517]]], np.int32)
    announce(f"m128 decode {kname} G={G}")
    out, lse = _gpu_decode(K, kp, vp, q, kv_len, path=2)
    ref_out, ref_lse = O.decode_attn(q, Kd, Vd, kv_len)
    _check_decode(out, lse, ref_out, ref_lse, kv_len)


@pytest.mark.parametrize("T", [32, 100, 4096])
def test_cache_lengths(T):
    import kv_cache_bit_fwht_amd as K
    w, Kx, Vx, q = _inputs(B=1, L=1, T=T, n_q=1)
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    kp, Kd = _pack(K, Kx, _codec(K, "sign"), shape)
    vp, Vd = _pack(K, Vx, _codec(K, "ter"), shape)
    announce(f"m128 decode T={T}")
    out, lse = _gpu_decode(K, kp, vp, q, None, path=2)
    ref_out, ref_lse = O.decode_attn(q, Kd, Vd, None)
    _check_decode(out, lse, ref_out, ref_lse, None)


@pytest.mark.parametrize("kname,vname", [("ter", "ter"), ("sign", "sign"), ("int8", "int8"), ("f16", "f16"),
                                         ("nf4", "i4"), ("i6h", "f16"), ("i6", "int8"),
                                         ("rc", "f16"), ("rc", "i4"), ("rp", "f16"), ("rp", "sign")])
def test_garbage_rows_past_the_keys(kname, vname):
    """Rows at and past each query's length hold NaN scales and all-ones codes (fp16: NaN
    values); the outputs equal those of a clean cache within the bars."""
    import torch
    import kv_cache_bit_fwht_amd as K
    w, Kx, Vx, q = _inputs(B=1, L=2, T=333, n_q=1)
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    kp, Kd = _pack(K, Kx, _codec(K, kname), shape)
    vp, Vd = _pack(K, Vx, _codec(K, vname), shape)
    n = 250
    kv_len = np.full((w.B, w.L, 1), n, np.int32)
    rows = torch.arange(w.B * w.L * w.H * w.T, device="cuda:0") % w.T >= n
    for p in (kp, vp):
        if p.codec.codebook == K.FP16:
            p.codes.view(-1, w.D)[rows] = 0x7E00       # fp16 NaN
        else:
            p.codes[rows] = -1                         # every code bit set
            p.scales[rows] = 0x7E00                    # fp16 NaN
    torch.cuda.synchronize()
    announce(f"m128 decode garbage rows K={kname} V={vname}")
    out, lse = _gpu_decode(K, kp, vp, q, kv_len, path=2)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    ref_out, ref_lse = O.decode_attn(q, Kd, Vd, kv_len)
    _check_decode(out, lse, ref_out, ref_lse, kv_len)


@pytest.mark.parametrize("kname,vname", [("ter", "ter"), ("nf4", "i4")])
def test_full_size_c4_sampled_units(kname, vname):
    """The extreme low-bit configuration at its full unit size (4 sequences x 8 KV heads x
    16,384 tokens x 128, 32 query heads; 3 of its layers), one decode query per sequence;
    sampled units against the oracle."""
    import torch
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c4", L=3, n_q=1)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    kc, vc = _codec(K, kname), _codec(K, vname)
    kp, vp = K.alloc_packed(kc, shape), K.alloc_packed(vc, shape)
    K.kvq_quantize_pack_kv(to_dev(Kx), to_dev(Vx), kp, vp)
    announce(f"m128 decode full-size c4 K={kname} V={vname}")
    out, lse = _gpu_decode(K, kp, vp, q, None, path=2)
    G = w.Hq // w.H
    okc, ovc = oracle_codec(K, O, kc), oracle_codec(K, O, vc)
    for (b, l, h) in [(0, 0, 0), (3, 2, 7), (1, 1, 4)]:
        ku, vu = Kx[b, l, h][None, None, None], Vx[b, l, h][None, None, None]
        wk, sk, zk = O.quantize_pack(ku, okc)
        wv, sv, zv = O.quantize_pack(vu, ovc)
        Kd = O.dequant(wk, sk, zk, okc, ku.shape)[0, 0, 0]
        Vd = O.dequant(wv, sv, zv, ovc, vu.shape)[0, 0, 0]
        ro, rl, _ = O.attention.attend(q[b, l, 0, h * G:(h + 1) * G].astype(np.float64), Kd, Vd, w.T,
                                       1.0 / np.sqrt(w.D))
        go = out[b, l, 0, h * G:(h + 1) * G].astype(np.float64)
        assert (np.linalg.norm(go - ro, axis=-1) / np.linalg.norm(ro, axis=-1)).max() < 2e-3
        assert np.abs(lse[b, l, 0, h * G:(h + 1) * G] - rl).max() < 1e-4


@pytest.mark.parametrize("kname", ["i6h", "rc", "rp"])
@pytest.mark.parametrize("qmag", [1e-3, 3e3])
def test_i6_query_range(qmag, kname):
    """Rotated 6-bit or rFFT keys with queries scaled by 1e-3 and 3e3 (fp16 inputs up to
    ~1.4e4, whose rotation or spectrum reaches past what an unscaled fp16 operand holds),
    G = 4 and 2."""
    import kv_cache_bit_fwht_amd as K
    for Hq in (32, 16):
        w, Kx, Vx, q = _inputs(B=1, L=2, T=700, n_q=2, Hq=Hq)
        q = (q.astype(np.float32) * qmag).astype(np.float16)
        shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
        kp, Kd = _pack(K, Kx, _codec(K, kname), shape)
        vp, Vd = _pack(K, Vx, _codec(K, "f16"), shape)
        announce(f"m128 decode {kname} query x{qmag} Hq={Hq}")
        # the logit scale is shrunk with large queries so the softmax stays comparable
        sm = 1.0 / np.sqrt(w.D) / max(qmag, 1.0)
        out, lse = _gpu_decode(K, kp, vp, q, None, path=2, sm_scale=sm)
        ref_out, ref_lse = O.decode_attn(q, Kd, Vd, None, sm_scale=sm)
        _check_decode(out, lse, ref_out, ref_lse, None)


@pytest.mark.parametrize("kname", ["i6h", "rc", "rp"])
def test_full_size_c5_sampled_units(kname):
    """The transform-ablation configuration's three arms at their full unit size (4 sequences x 8 KV heads x 32,768 tokens x 128, 32 query heads; 2 of
    its 16 layers; keys RoPE-rotated, then FWHT-128 + 6-bit absmax at group 32, rFFT with
    6-bit real and imaginary parts at group 32, or rFFT with 5-bit magnitudes at group 32
    and 7-bit phases; fp16 values), one decode query per sequence; sampled units against
    the oracle."""
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c5", L=2, n_q=1)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    kc = _codec(K, kname)
    kp = K.alloc_packed(kc, shape)
    K.kvq_quantize_pack(to_dev(Kx), kp)
    vp = K.packed_from_fp16(to_dev(Vx), shape)
    announce(f"m128 decode full-size c5 {kname}")
    out, lse = _gpu_decode(K, kp, vp, q, None, path=2)
    out0, lse0 = _gpu_decode(K, kp, vp, q, None, path=0)
    assert np.array_equal(out0, out) and np.array_equal(lse0, lse), "path 0 should take the MFMA kernel"
    G = w.Hq // w.H
    okc = oracle_codec(K, O, kc)
    for (b, l, h) in [(0, 0, 0), (3, 1, 7), (2, 1, 3)]:
        ku = Kx[b, l, h][None, None, None]
        wk, sk, zk = O.quantize_pack(ku, okc)
        Kd = O.dequant(wk, sk, zk, okc, ku.shape)[0, 0, 0]
        ro, rl, _ = O.attention.attend(q[b, l, 0, h * G:(h + 1) * G].astype(np.float64), Kd,
                                       Vx[b, l, h].astype(np.float64), w.T, 1.0 / np.sqrt(w.D))
        go = out[b, l, 0, h * G:(h + 1) * G].astype(np.float64)
        assert (np.linalg.norm(go - ro, axis=-1) / np.linalg.norm(ro, axis=-1)).max() < 2e-3
        assert np.abs(lse[b, l, 0, h * G:(h + 1) * G] - rl).max() < 1e-4

"""GPU parity of the shared key-mean subtraction ([LCPP] llama.cpp issue
"Per-head adaptive KV cache quantization", the later comment measuring the failure
mode): kvq_key_mean bit-exact against the oracle; quantize+pack and dequant with a
mean (and with a mean and channel scales) bit-exact for every kernel family; decode
with a key mean (out unchanged by the constant logit shift, lse shifted by
sm * q.mean) and the error reduction (K error with the mean restored) within the
attention bars."""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import announce, oracle_codec, to_dev, to_np
from tests.test_gpu_attn import KL_TOL, _check_decode, _gpu_decode, _gpu_error

pytestmark = pytest.mark.gpu


def _gpu_mean(K, x):
    import torch
    B, L, H, T, D = x.shape
    shape = K.Shape(B, L, H, T, D)
    mean = torch.full((L, H, D), float("nan"), dtype=torch.float32, device="cuda:0")
    wsb = K.kvq_key_mean_workspace(shape)
    ws = torch.full((max(wsb, 16),), 0x5a, dtype=torch.uint8, device="cuda:0")   # stale contents
    K.kvq_key_mean(to_dev(x) if x.size else torch.empty(8, dtype=torch.int16, device="cuda:0"), shape, mean, ws, wsb)
    torch.cuda.synchronize()
    return mean


@pytest.mark.parametrize("shape", [(2, 2, 2, 777, 256), (3, 1, 3, 1001, 128), (1, 2, 1, 5, 64), (2, 1, 2, 0, 128)])
def test_key_mean_bit_exact(shape):
    import kv_cache_bit_fwht_amd as K
    B, L, H, T, D = shape
    rng = np.random.default_rng([21, *shape])
    x = rng.standard_normal(shape) * 3 + rng.standard_normal((1, L, H, 1, D)) * 5
    x = x.astype(np.float16)
    if T:
        x[0, 0, 0, :, :4] = np.float16(65504.0)
        x[..., 5] = np.float16(6e-8)
    announce(f"key mean {shape}")
    m = _gpu_mean(K, x)
    assert np.array_equal(to_np(m), O.key_mean(x))


CODECS = [((1, 4, 128, 256), 256), ((1, 3, 128, 256), 256), ((1, 2, 128, 0), 256), ((2, 3, 32, 0), 128),
          ((5, 4, 64, 0), 64), ((7, 5, 32, 0, 7), 128), ((8, 6, 16, 0), 128), ((9, 2, 64, 0), 128),
          ((10, 3, 32, 128), 128)]


@pytest.mark.parametrize("T", [203, 204])
@pytest.mark.parametrize("with_chan", [False, True])
@pytest.mark.parametrize("cspec,D", CODECS)
def test_quantize_dequant_with_mean_bit_exact(cspec, D, with_chan, T):
    """T = 204 (a multiple of 4) takes the 256-wide absmax kernel's mean/scale variant
    for the head_dim-256 absmax codecs; T = 203 the general kernel."""
    import torch
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", B=2, L=2, H=2, T=T, D=D, k_mean_share=0.53)
    Kx, _ = synth.gen_kv(w)
    mu = O.key_mean(Kx)
    chan = np.random.default_rng(D).uniform(0.5, 2.0, (2, 2, D)).astype(np.float32) if with_chan else None
    codec = K.Codec(*cspec)
    oc = oracle_codec(K, O, codec)
    shape = K.Shape(*Kx.shape)
    announce(f"quantize with mean codec={codec} D={D} chan={with_chan}")
    p = K.alloc_packed(codec, shape, chan_scale=to_dev(chan) if chan is not None else None, mean=to_dev(mu))
    K.kvq_quantize_pack(to_dev(Kx), p)
    xh = torch.empty(Kx.shape, dtype=torch.float32, device="cuda:0")
    K.kvq_dequant(p, xh)
    torch.cuda.synchronize()
    wr, sr, zr = O.quantize_pack(Kx, oc, chan, mu)
    assert np.array_equal(to_np(p.codes, np.uint32), wr), "codes differ"
    if sr.shape[1]:
        assert np.array_equal(to_np(p.scales, np.uint16), sr.view(np.uint16)), "scales differ"
    if zr.shape[1]:
        assert np.array_equal(to_np(p.mins, np.uint16), zr.view(np.uint16)), "mins differ"
    ref = O.dequant(wr, sr, zr, oc, Kx.shape, chan, mu)
    assert np.array_equal(to_np(xh), ref), f"dequant max diff {np.abs(to_np(xh) - ref).max()}"


@pytest.mark.parametrize("case", [("mfma", (1, 4, 128, 256), 2), ("auto", (1, 4, 128, 256), None),
                                  ("general", (1, 4, 128, 256), 1), ("general", (1, 3, 128, 256), 1),
                                  ("general", (2, 3, 32, 0), 1), ("general", (7, 5, 32, 0, 7), 1),
                                  ("map_pair", (1, 5, 64, 256), 1), ("mfma_k3", (1, 3, 128, 256), 2)])
def test_decode_and_error_with_key_mean(case):
    import kv_cache_bit_fwht_amd as K
    name, kspec, path = case
    w = synth.get("c3", L=2, T=704, n_q=3, k_mean_share=0.53)
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w)
    kv_len = np.array(kv_len) if kv_len is not None else None
    mu = O.key_mean(Kx)
    kc, vc = K.Codec(*kspec), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    okc, ovc = oracle_codec(K, O, kc), oracle_codec(K, O, vc)
    shape = K.Shape(*Kx.shape)
    announce(f"decode with key mean {name} kc={kc}")
    kp = K.alloc_packed(kc, shape, mean=to_dev(mu))
    vp = K.alloc_packed(vc, shape)
    K.kvq_quantize_pack(to_dev(Kx), kp)
    K.kvq_quantize_pack(to_dev(Vx), vp)
    wk, sk, zk = O.quantize_pack(Kx, okc, None, mu)
    wv, sv, zv = O.quantize_pack(Vx, ovc)
    Kd = O.dequant(wk, sk, zk, okc, Kx.shape, None, mu)
    Vd = O.dequant(wv, sv, zv, ovc, Vx.shape)
    out, lse = _gpu_decode(K, kp, vp, q, kv_len, path)
    ref_out, ref_lse = O.decode_attn(q, Kd, Vd, kv_len)
    _check_decode(out, lse, ref_out, ref_lse, kv_len)
    # the shift is real: without the correction lse would be off by sm * q.mean
    sm = 1.0 / np.sqrt(Kx.shape[-1])
    G = q.shape[3] // Kx.shape[2]
    qm = np.einsum("blihd,lhd->blih", q.astype(np.float64), np.repeat(mu.astype(np.float64), G, axis=1)) * sm
    assert np.abs(qm).max() > 0.1
    kl, re, kv = _gpu_error(K, Kx, Vx, kp, vp, q, kv_len)
    rkl, rre, rkv = O.attn_error(q, Kx, Vx, Kd, Vd, kv_len)
    assert np.abs(kl - rkl).max() < KL_TOL, f"KL diff {np.abs(kl - rkl).max():.3g}"
    assert np.abs(re - rre).max() < 1e-4
    assert np.allclose(kv, rkv, rtol=1e-9, atol=1e-12), "kv_err differs"

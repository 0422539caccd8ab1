"""GPU parity of kvq_quantize_pack_kv and kvq_quantize_pack_tokens_kv (keys and
values coded in one call) against the CPU oracle: codes and scales bit-exact, on the
one-launch route (both tensors 256-wide signed absmax without a mean or channel
scales) and on the fallback routes."""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import announce, oracle_codec, to_dev, to_np
from tests.test_gpu_quant import _inputs

pytestmark = pytest.mark.gpu


def _check(K, x, p, codec, chan=None, mean=None):
    oc = oracle_codec(K, O, codec)
    w, s, z = O.quantize_pack(x, oc, chan, mean=mean) if mean is not None else O.quantize_pack(x, oc, chan)
    codes = to_np(p.codes, np.uint32)
    bad = np.nonzero((codes != w).any(1))[0]
    assert bad.size == 0, f"{bad.size} rows with code mismatches, first rows {bad[:3]}"
    if s.shape[1]:
        assert np.array_equal(to_np(p.scales, np.uint16), s.view(np.uint16)), "scales differ"
    if z.shape[1]:
        assert np.array_equal(to_np(p.mins, np.uint16), z.view(np.uint16)), "mins differ"


# (K codec, V codec) as (codebook, bits, group, rot); the first six take the one-launch route
PAIRS = [((1, 4, 128, 256), (1, 2, 128, 0)), ((1, 2, 32, 256), (1, 4, 64, 256)), ((1, 8, 256, 0), (1, 8, 16, 256)),
         ((1, 4, 16, 0), (1, 2, 256, 0)), ((1, 2, 128, 0), (1, 2, 128, 0)), ((1, 8, 64, 256), (1, 4, 32, 0)),
         # symmetric-grid or Lloyd-Max values: two launches of the quad coder
         ((1, 4, 128, 256), (9, 2, 128, 256)), ((1, 4, 128, 256), (10, 2, 128, 256)), ((1, 4, 64, 0), (9, 4, 32, 0)),
         ((1, 4, 256, 256), (10, 4, 16, 0)),
         # fallbacks: another codebook or bit width on one side
         ((1, 3, 128, 256), (1, 2, 128, 0)), ((5, 4, 64, 0), (1, 4, 64, 0)), ((2, 4, 32, 0), (2, 4, 32, 0)),
         ((7, 5, 32, 0), (0, 16, 0, 0))]


@pytest.mark.parametrize("kspec,vspec", PAIRS)
@pytest.mark.parametrize("dims", [(1, 2, 3, 37), (2, 1, 2, 64)])
def test_quantize_pack_kv_bit_exact(kspec, vspec, dims):
    """222 rows (a ragged last quad) or 256 rows, with the special rows of the
    single-tensor test (zeros, -0, subnormals, saturation, +-A ties, a constant row)."""
    import kv_cache_bit_fwht_amd as K
    import torch
    B, L, H, T = dims
    D = 256
    kc = K.Codec(kspec[0], kspec[1], kspec[2], kspec[3], 7 if kspec[0] == K.RFFT_POLAR else 0)
    vc = K.Codec(*vspec)
    xk = _inputs(B, L, H, T, D, seed=31 + sum(kspec))
    xv = _inputs(B, L, H, T, D, seed=57 + sum(vspec))
    shape = K.Shape(B, L, H, T, D)
    kp = K.alloc_packed(kc, shape)
    kdev, vdev = to_dev(xk), to_dev(xv)
    vp = K.packed_from_fp16(vdev, shape) if vc.codebook == K.FP16 else K.alloc_packed(vc, shape)
    announce(f"quantize_pack_kv dims={dims} K={kc} V={vc}")
    K.kvq_quantize_pack_kv(kdev, vdev, kp, vp)
    torch.cuda.synchronize()
    _check(K, xk, kp, kc)
    if vc.codebook != K.FP16:
        _check(K, xv, vp, vc)


def test_quantize_pack_kv_with_key_mean_falls_back():
    """A key mean takes the single-tensor kernels; the results are the oracle's."""
    import kv_cache_bit_fwht_amd as K
    import torch
    B, L, H, T, D = 1, 2, 2, 64, 256
    xk = _inputs(B, L, H, T, D, seed=5, specials=False)
    xv = _inputs(B, L, H, T, D, seed=6, specials=False)
    mean = O.key_mean(xk)
    kc, vc = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    shape = K.Shape(B, L, H, T, D)
    kp = K.alloc_packed(kc, shape, mean=to_dev(mean))
    vp = K.alloc_packed(vc, shape)
    announce("quantize_pack_kv with a key mean")
    K.kvq_quantize_pack_kv(to_dev(xk), to_dev(xv), kp, vp)
    torch.cuda.synchronize()
    _check(K, xk, kp, kc, mean=mean)
    _check(K, xv, vp, vc)


@pytest.mark.parametrize("t0,n", [(0, 1), (63, 1), (17, 5), (0, 64), (40, 24)])
def test_quantize_pack_tokens_kv_window(t0, n):
    """Append windows: the window's rows equal the oracle's codes of those tokens;
    rows outside the window keep their previous contents."""
    import kv_cache_bit_fwht_amd as K
    import torch
    B, L, H, T, D = 2, 2, 3, 64, 256
    xk = _inputs(B, L, H, T, D, seed=71, specials=False)
    xv = _inputs(B, L, H, T, D, seed=72, specials=False)
    kc, vc = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    shape = K.Shape(B, L, H, T, D)
    kp, vp = K.alloc_packed(kc, shape), K.alloc_packed(vc, shape)
    for p in (kp, vp):
        p.codes.fill_(0x5A5A5A5A)
        p.scales.fill_(0x1234)
    wk = np.ascontiguousarray(xk[:, :, :, t0:t0 + n])
    wv = np.ascontiguousarray(xv[:, :, :, t0:t0 + n])
    announce(f"quantize_pack_tokens_kv t0={t0} n={n}")
    K.kvq_quantize_pack_tokens_kv(to_dev(wk), to_dev(wv), t0, n, kp, vp)
    torch.cuda.synchronize()
    for x, p, c in ((xk, kp, kc), (xv, vp, vc)):
        w, s, _ = O.quantize_pack(x, oracle_codec(K, O, c))
        codes = to_np(p.codes, np.uint32).reshape(B, L, H, T, -1)
        scales = to_np(p.scales, np.uint16).reshape(B, L, H, T, -1)
        w = w.reshape(B, L, H, T, -1)
        s = s.view(np.uint16).reshape(B, L, H, T, -1)
        assert np.array_equal(codes[:, :, :, t0:t0 + n], w[:, :, :, t0:t0 + n])
        assert np.array_equal(scales[:, :, :, t0:t0 + n], s[:, :, :, t0:t0 + n])
        outside = np.ones(T, bool)
        outside[t0:t0 + n] = False
        assert np.all(codes[:, :, :, outside] == 0x5A5A5A5A)
        assert np.all(scales[:, :, :, outside] == 0x1234)


def test_quantize_pack_kv_invalid_arguments_write_nothing():
    import kv_cache_bit_fwht_amd as K
    import torch
    shape = K.Shape(1, 1, 2, 16, 256)
    kc, vc = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    kp, vp = K.alloc_packed(kc, shape), K.alloc_packed(vc, shape)
    kp.codes.fill_(-1)
    vp.codes.fill_(-1)
    x = to_dev(np.zeros((1, 1, 2, 16, 256), np.float16))
    other = K.alloc_packed(vc, K.Shape(1, 1, 2, 8, 256))
    announce("quantize_pack_kv invalid arguments")
    with pytest.raises(K.KvqError):
        K.kvq_quantize_pack_kv(x, x, kp, other)                      # shapes differ
    with pytest.raises(K.KvqError):
        K.kvq_quantize_pack_kv(x, x, kp, kp)                         # one output for both
    with pytest.raises(K.KvqError):
        K.kvq_quantize_pack_tokens_kv(x, x, 10, 7, kp, vp)           # window past the end
    torch.cuda.synchronize()
    assert bool((kp.codes == -1).all()) and bool((vp.codes == -1).all())


def test_full_size_64k_kv_sampled_units():
    """The 64K decode workload at full size (8 x 4 x 65536 x 256) coded by one
    kvq_quantize_pack_kv call, the launch the benchmark times; sampled units against
    the oracle."""
    import kv_cache_bit_fwht_amd as K
    import torch
    w = synth.get("c3")
    announce("full-size 64K quantize_pack_kv")
    Kx, Vx = synth.gen_kv(w)
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    kc, vc = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    kp, vp = K.alloc_packed(kc, shape), K.alloc_packed(vc, shape)
    K.kvq_quantize_pack_kv(to_dev(Kx), to_dev(Vx), kp, vp)
    torch.cuda.synchronize()
    for (l, h) in [(0, 0), (3, 2), (7, 3)]:
        rows = slice((l * w.H + h) * w.T, (l * w.H + h + 1) * w.T)
        for x, p, c in ((Kx, kp, kc), (Vx, vp, vc)):
            wo, so, _ = O.quantize_pack(x[0, l, h][None, None, None], oracle_codec(K, O, c))
            assert np.array_equal(to_np(p.codes[rows], np.uint32), wo), f"unit {(l, h)} codes"
            assert np.array_equal(to_np(p.scales[rows], np.uint16), so.view(np.uint16)), f"unit {(l, h)} scales"

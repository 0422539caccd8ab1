"""GPU parity of kvq_quantize_pack / kvq_dequant / kvq_calibrate_chan_scale
against the CPU oracle: codes, scales and mins bit-exact; dequantised values
equal to the oracle's (same binary32 operation order)."""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import announce, oracle_codec, to_dev, to_np

pytestmark = pytest.mark.gpu


def _inputs(B, L, H, T, D, seed, specials=True):
    rng = np.random.default_rng([7, seed, D, T])
    x = rng.standard_normal((B, L, H, T, D), dtype=np.float32)
    ch = rng.choice(D, size=max(1, D // 32), replace=False)
    x[..., ch] *= 10.0
    if specials and T >= 6:
        x[0, 0, 0, 0] = 0.0                                 # zero row
        x[0, 0, 0, 1, : D // 2] = -0.0                      # -0 half row
        x[0, 0, 0, 2] *= 1e-6                               # fp16 subnormals
        x[0, 0, 0, 3] = np.sign(x[0, 0, 0, 3]) * 60000.0    # saturation after rotation
        x[0, 0, 0, 4, ::2] = 3.0
        x[0, 0, 0, 4, 1::2] = -3.0                          # +-A ties
        x[0, 0, 0, 5] = 1.0                                 # constant row
    return x.astype(np.float16)


def _run(K, x, codec, chan=None):
    B, L, H, T, D = x.shape
    shape = K.Shape(B, L, H, T, D)
    chan_d = to_dev(chan) if chan is not None else None
    p = K.alloc_packed(codec, shape, chan_scale=chan_d)
    K.kvq_quantize_pack(to_dev(x), p)
    import torch
    xh = torch.empty((B, L, H, T, D), dtype=torch.float32, device="cuda:0")
    K.kvq_dequant(p, xh)
    torch.cuda.synchronize()
    return p, to_np(xh)


def _compare(K, x, codec, chan=None):
    oc = oracle_codec(K, O, codec)
    p, xh = _run(K, x, codec, chan)
    w, s, z = O.quantize_pack(x, oc, chan)
    codes = to_np(p.codes, np.uint32)
    assert codes.shape == w.shape
    bad = np.nonzero((codes != w).any(1))[0]
    assert bad.size == 0, f"{bad.size} rows with code mismatches, first row {bad[:3]}"
    if s.shape[1]:
        assert np.array_equal(to_np(p.scales, np.uint16), s.view(np.uint16)), "scales differ"
    if z.shape[1]:
        assert np.array_equal(to_np(p.mins, np.uint16), z.view(np.uint16)), "mins differ"
    ref = O.dequant(w, s, z, oc, x.shape, chan)
    assert np.array_equal(xh, ref), f"dequant max abs diff {np.abs(xh - ref).max()}"


CASES = []
for D in (64, 128, 256):
    for b in (2, 3, 4, 5, 6, 7, 8):
        for g in (8, 32, 128):
            if g <= D:
                CASES.append((D, (1, b, g, 0)))
        CASES.append((D, (1, b, 32, D)))
    CASES += [(D, (2, 4, 32, 0)), (D, (2, 3, 8, 0)), (D, (2, 2, 64, D)), (D, (3, 2, 8, 0)), (D, (4, 1, 8, 0)),
              (D, (4, 1, 32, 0)), (D, (5, 4, 64, 0)), (D, (6, 8, D, 0)), (D, (0, 16, 0, 0)), (D, (1, 4, 16, 0)),
              (D, (1, 4, 64, D // 2)), (D, (1, 6, 32, 16)), (D, (1, 4, 8, 8)), (D, (3, 2, 8, D))]
CASES.append((256, (1, 4, 256, 256)))
# the symmetric grid and the Gaussian Lloyd-Max codebook (value codecs the 64K experiment names next)
for D in (64, 128, 256):
    CASES += [(D, (9, 2, 8, 0)), (D, (9, 3, 32, D)), (D, (9, 4, 64, 0)), (D, (9, 8, 32, 0)),
              (D, (10, 2, 8, 0)), (D, (10, 2, 64, D)), (D, (10, 3, 32, 0)), (D, (10, 4, 16, D))]
# at head_dim 256 (2-, 4- and 8-bit, groups of 16 or more) these run on the one-quad-per-
# wavefront row coder: more groups, rotations and the 64K experiment's value arms
CASES += [(256, (9, 2, 128, 256)), (256, (9, 2, 16, 0)), (256, (9, 4, 256, 256)), (256, (9, 8, 128, 256)),
          (256, (10, 2, 128, 256)), (256, (10, 2, 256, 0)), (256, (10, 4, 32, 0)), (256, (10, 2, 16, 256))]


@pytest.mark.parametrize("D,cspec", CASES)
def test_quantize_pack_bit_exact(D, cspec):
    import kv_cache_bit_fwht_amd as K
    cb, b, g, rot = cspec
    codec = K.Codec(cb, b, g, rot)
    x = _inputs(1, 2, 3, 37, D, seed=cb * 100 + b * 10 + g + rot)
    announce(f"quantize D={D} codec={codec}")
    _compare(K, x, codec)


# rFFT codecs: magnitude/phase (bits, phase bits, group) and real/imaginary (bits, group)
RFFT_CASES = []
for D in (64, 128, 256):
    RFFT_CASES += [(D, "polar", b, pb, g) for (b, pb, g) in
                   [(5, 7, 32), (4, 8, 16), (6, 6, 8), (2, 3, 128), (8, 8, 64), (3, 5, 8), (7, 4, 128)]]
    RFFT_CASES += [(D, "cart", b, 0, g) for (b, g) in [(6, 32), (8, 8), (2, 128), (3, 16), (5, 64), (4, 8)]]


def _rfft_codec(K, kind, b, pb, g):
    return K.Codec(K.RFFT_POLAR, b, g, 0, pb) if kind == "polar" else K.Codec(K.RFFT_CART, b, g, 0)


@pytest.mark.parametrize("D,kind,b,pb,g", RFFT_CASES)
def test_rfft_quantize_bit_exact(D, kind, b, pb, g):
    """222 rows (a ragged last wavefront at every head_dim) with the special rows of
    _inputs; codes, scales and the dequantised rows against the oracle."""
    import kv_cache_bit_fwht_amd as K
    codec = _rfft_codec(K, kind, b, pb, g)
    x = _inputs(1, 2, 3, 37, D, seed=1000 + 10 * b + pb + g)
    announce(f"rfft quantize D={D} codec={codec}")
    _compare(K, x, codec)


@pytest.mark.parametrize("D,kind", [(64, "polar"), (128, "polar"), (256, "polar"), (128, "cart"), (256, "cart")])
def test_rfft_quantize_channel_scales_extreme_magnitudes(D, kind):
    """Per-unit channel multipliers of 1e-33, 1e-26, 1e30 and about 1 put spectrum
    values below 2^-96 (products in the side tests underflow), above 2^96 (squares
    overflow to infinity) and in the ordinary range; 3 x 401 rows per unit."""
    import kv_cache_bit_fwht_amd as K
    codec = _rfft_codec(K, kind, 5, 7, 32) if kind == "polar" else _rfft_codec(K, kind, 6, 0, 32)
    x = _inputs(1, 2, 2, 401, D, seed=77 + D)
    rng = np.random.default_rng([13, D])
    chan = rng.uniform(0.5, 2.0, (2, 2, D)).astype(np.float32)
    chan[0, 0] *= np.float32(1e-33)
    chan[0, 1] *= np.float32(1e-26)
    chan[1, 0] *= np.float32(1e30)
    announce(f"rfft quantize channel scales D={D} codec={codec}")
    _compare(K, x, codec, chan)


def test_rfft_quantize_many_passes():
    """70,001 rows at head_dim 256 (4 rows per wavefront): every wavefront of the
    capped grid encodes several row groups and the last group is ragged."""
    import kv_cache_bit_fwht_amd as K
    codec = _rfft_codec(K, "polar", 5, 7, 32)
    x = _inputs(1, 1, 1, 70001, 256, seed=4242)
    announce(f"rfft quantize 70001 rows codec={codec}")
    _compare(K, x, codec)


@pytest.mark.parametrize("cspec", [(1, 4, 128, 256), (1, 2, 128, 0), (10, 2, 32, 256), (10, 3, 128, 0)])
def test_quantize_many_passes_ragged(cspec):
    """90,003 rows at head_dim 256: every wavefront encodes several row quads, and
    the last quad is ragged (3 of 4 rows); all rows checked.  The Lloyd-Max arms
    check the RMS scale (a square root) over ~0.4-0.7M groups, where a last-ulp error
    of the root would move some fp16 scale."""
    import kv_cache_bit_fwht_amd as K
    codec = K.Codec(*cspec)
    x = _inputs(1, 1, 3, 30001, 256, seed=911 + cspec[1])
    announce(f"quantize 90003 rows codec={codec}")
    _compare(K, x, codec)


@pytest.mark.parametrize("arm", ["C", "D", "D4"])
def test_prescaled_keys_bit_exact(arm):
    """E21W arms C/D: per-channel K scaling calibrated on sequence 0."""
    import kv_cache_bit_fwht_amd as K
    import torch
    w = synth.get("c2", B=2, L=2, H=2, Hq=2, T=300, pos_range=(100, 300), n_q=4)
    Kx, _ = synth.gen_kv(w)
    announce(f"calibrate + quantize arm {arm}")
    cal = torch.empty((w.L, w.H, w.D), dtype=torch.float32, device="cuda:0")
    K.kvq_calibrate_chan_scale(to_dev(np.ascontiguousarray(Kx[:1])), K.Shape(1, w.L, w.H, w.T, w.D), cal)
    torch.cuda.synchronize()
    c_ref = O.calibrate_chan_scale(Kx[0])
    assert np.array_equal(to_np(cal), c_ref)
    codec = {"C": K.Codec(K.INT_MINMAX, 3, 32, 0), "D": K.Codec(K.INT_ABSMAX, 3, 32, 256),
             "D4": K.Codec(K.INT_ABSMAX, 4, 32, 256)}[arm]
    _compare(K, Kx, codec, c_ref)


def test_full_size_64k_sampled_rows():
    """The 64K decode workload at full size (8 x 4 x 65536 x 256) in the launch
    configuration the benchmark times; the oracle checks sampled units."""
    import kv_cache_bit_fwht_amd as K
    import torch
    w = synth.get("c3")
    announce("full-size 64K quantize")
    Kx, Vx = synth.gen_kv(w)
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    kc, vc = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    kp, vp = K.alloc_packed(kc, shape), K.alloc_packed(vc, shape)
    K.kvq_quantize_pack(to_dev(Kx), kp)
    K.kvq_quantize_pack(to_dev(Vx), vp)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    for (l, h) in [(0, 0), (7, 3), (int(rng.integers(8)), int(rng.integers(4)))]:
        rows = slice(((0 * w.L + l) * w.H + h) * w.T, ((0 * w.L + l) * w.H + h + 1) * w.T)
        for x, p, c in ((Kx, kp, kc), (Vx, vp, vc)):
            unit = x[0, l, h][None, None, None]
            wo, so, _ = O.quantize_pack(unit, oracle_codec(K, O, c))
            assert np.array_equal(to_np(p.codes[rows], np.uint32), wo), f"unit {(l, h)} codes"
            assert np.array_equal(to_np(p.scales[rows], np.uint16), so.view(np.uint16)), f"unit {(l, h)} scales"


def test_invalid_arguments_write_nothing():
    import kv_cache_bit_fwht_amd as K
    import torch
    shape = K.Shape(1, 1, 1, 16, 128)
    p = K.alloc_packed(K.Codec(K.INT_ABSMAX, 4, 32, 0), shape)
    p.codes.fill_(-1)
    x = to_dev(np.zeros((1, 1, 1, 16, 128), np.float16))
    bad = K.Packed(K.Codec(K.INT_ABSMAX, 4, 48, 0), shape, p.codes, p.scales, None)
    with pytest.raises(K.KvqError):
        K.kvq_quantize_pack(x, bad)
    with pytest.raises(K.KvqError):
        K.kvq_quantize_pack(x[..., 1:].contiguous().view(-1)[1:], p)   # misaligned input
    torch.cuda.synchronize()
    assert bool((p.codes == -1).all())

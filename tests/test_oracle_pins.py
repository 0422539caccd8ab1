"""More pins of the oracle codec (CPU only): the published NF4 table, brute-force
nearest-grid checks of the min-max and rFFT encoders, and the binary16 limits of
the scale rounding.

Every pin here is a function that reports violations.  Each is run twice: on the
oracle (no violations) and on a deliberately wrong variant written in this file
(a plausible slip in the same encoder), which it must catch.  The wrong variants
live only here; the oracle itself is never modified.
"""
import json
import os

import numpy as np
import pytest

import oracle as O
from oracle import rfft as R

F32 = np.float32
GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ NF4

def _published_nf4():
    with open(os.path.join(GOLD, "nf4_qlora.json")) as f:
        return np.array(json.load(f)["levels"], dtype=np.float64)


def _nf4_fp64_construction():
    """A plausible slip: the exact offset 1 - (1/30 + 1/32)/2 and every step in fp64,
    rounded to binary32 once at the end."""
    from scipy.stats import norm
    off = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    pos = norm.ppf(np.linspace(off, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(off, 0.5, 8)[:-1])
    v = np.sort(np.concatenate([pos, [0.0], neg]))
    return (v / v.max()).astype(F32)


def test_nf4_levels_are_the_published_table():
    pub = _published_nf4()
    assert np.all(pub.astype(F32).astype(np.float64) == pub)          # printed values are binary32
    assert np.array_equal(O.nf4_levels().astype(np.float64), pub)
    # the pin distinguishes the construction details: an all-fp64 variant differs by a few ulp
    assert not np.array_equal(_nf4_fp64_construction().astype(np.float64), pub)


def test_nf4_midpoints_from_published_levels():
    L = _published_nf4().astype(F32)
    M = O.nf4_midpoints()
    assert np.array_equal(M, (L[:-1] + L[1:]) * F32(0.5))
    assert np.all((M > L[:-1]) & (M < L[1:]))


# ------------------------------------------------------------------ brute-force nearest grid point

def nearest_violations(vals, codes, grid, tol):
    """Entries whose code is not the nearest grid point to the exact value.

    vals: float array of the values coded; codes: int array (same shape); grid:
    [..., n_levels] exact grid values per element (fp64); tol: per-element slack in
    value units, covering the binary32 roundings the encoder takes before its
    decision.  An element passes when the chosen level is at most `tol` farther
    than the nearest one."""
    v = np.asarray(vals, dtype=np.float64)[..., None]
    d = np.abs(grid - v)
    dmin = d.min(-1)
    dc = np.take_along_axis(d, codes[..., None], -1)[..., 0]
    return np.count_nonzero(dc > dmin + tol)


def _minmax_encode_with_lo(y, b):
    """A plausible slip in the min-max encoder: codes taken relative to the fp32
    minimum instead of the stored fp16 one."""
    lo = y.min(-1)
    hi = y.max(-1)
    s16 = O.rn16((hi - lo) / F32(2 ** b - 1))
    z16 = O.rn16(lo)
    inv = O.inv32(s16)
    t = (y - lo[..., None]) * inv[..., None]
    return np.clip(np.rint(t), 0, 2 ** b - 1).astype(np.int64), s16, z16


def _minmax_groups():
    """Groups of fp32 values (after a rotation or channel scale they need not be
    fp16) whose minimum is far from its fp16 rounding, in units of the step: a
    level near 1000 has an fp16 spacing of 0.5, the same as the 4-bit step."""
    rng = np.random.default_rng(11)
    a = F32(1000.0) + F32(0.2) + (rng.random((64, 32)) * 7.5).astype(F32)
    b = (rng.standard_normal((64, 32)) * 3).astype(F32)
    return np.concatenate([a, b])


def _minmax_violations(enc, b):
    y = _minmax_groups()
    codes, s16, z16 = enc(y, b)
    s = s16.astype(np.float64)[:, None, None]
    z = z16.astype(np.float64)[:, None, None]
    q = np.arange(2 ** b, dtype=np.float64)
    grid = q * s + z
    # three binary32 roundings before the decision (y - z, 1/s, the product)
    tol = 4 * 2.0 ** -24 * (2 ** b) * np.abs(s16.astype(np.float64))[:, None] + \
        2 * 2.0 ** -24 * np.abs(y.astype(np.float64))
    return nearest_violations(y, codes, grid, tol)


@pytest.mark.parametrize("b", [3, 4])
def test_minmax_codes_are_nearest_on_stored_grid(b):
    assert _minmax_violations(O.codec._enc_minmax, b) == 0
    assert _minmax_violations(_minmax_encode_with_lo, b) > 0


def test_minmax_minimum_element_decodes_to_stored_min():
    """Where the fp16 rounding of the minimum is under half a step away, the
    minimum element gets code 0, whose level is exactly the stored minimum."""
    rng = np.random.default_rng(12)
    y = (rng.standard_normal((200, 32)) * 2).astype(np.float16)
    c = O.Codec(O.INT_MINMAX, 4, 32)
    f, s, z = O.quantize_rows(y, c)
    codes = f[0][0]
    arg = y.astype(F32).argmin(-1)
    assert np.all(codes[np.arange(200), arg] == 0)
    xh = O.dequant_rows(f, s, z, c, 32)
    assert np.array_equal(xh[np.arange(200), arg], z[:, 0].astype(F32))


# ------------------------------------------------------------------ rFFT codes

def _spectra():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((48, 128)) * 2).astype(np.float16).astype(F32)
    return x, R.rfft(x)


def _polar_trunc(x, codec):
    """A plausible slip: magnitudes truncated to the grid instead of rounded."""
    re, im = R.rfft(x)
    mu = R.magnitude(re, im)
    F = mu.shape[1]
    qm = np.zeros(mu.shape, np.int64)
    sc = []
    for a, e in R._groups(F, codec.group):
        s16 = O.rn16(mu[:, a:e].max(-1) / F32(2 ** codec.bits - 1))
        inv = O.inv32(s16)
        qm[:, a:e] = np.clip(np.floor(mu[:, a:e] * inv[:, None]), 0, 2 ** codec.bits - 1)
        sc.append(s16)
    return qm, np.stack(sc, 1)


def _polar_magnitude_violations(enc):
    x, (re, im) = _spectra()
    codec = O.Codec(O.RFFT_POLAR, 5, 32, aux_bits=7)
    qm, sc = enc(x, codec)
    mu = R.magnitude(re, im)
    F = mu.shape[1]
    bad = 0
    for gi, (a, e) in enumerate(R._groups(F, codec.group)):
        s = sc[:, gi].astype(np.float64)
        grid = np.arange(32, dtype=np.float64)[None, None, :] * s[:, None, None]
        tol = 3 * 2.0 ** -24 * 32 * s[:, None]
        bad += nearest_violations(mu[:, a:e], qm[:, a:e], grid, tol)
    return bad


def _polar_oracle(x, codec):
    codes, sc, _ = R.encode(x, codec)
    return codes[0][0], sc


def test_polar_magnitude_codes_are_nearest_and_scale_is_max_over_31():
    assert _polar_magnitude_violations(_polar_oracle) == 0
    assert _polar_magnitude_violations(_polar_trunc) > 0
    # the scale puts the group's largest magnitude on the top level (to fp16 rounding)
    x, (re, im) = _spectra()
    mu = R.magnitude(re, im).astype(np.float64)
    _, sc = _polar_oracle(x, O.Codec(O.RFFT_POLAR, 5, 32, aux_bits=7))
    for gi, (a, e) in enumerate(R._groups(mu.shape[1], 32)):
        ref = mu[:, a:e].max(-1) / 31
        assert np.all(np.abs(sc[:, gi].astype(np.float64) - ref) <= 2.0 ** -11 * ref + 1e-30)


def _cart_off_by_one(x, codec):
    """A plausible slip: codes stored with offset 2^(b-1) - 1 instead of 2^(b-1)."""
    codes, sc, _ = R.encode(x, codec)
    return [(np.clip(c - 1, 0, 2 ** b - 1), b) for c, b in codes], sc


def _cart_violations(enc):
    x, (re, im) = _spectra()
    codec = O.Codec(O.RFFT_CART, 6, 32)
    codes, sc = enc(x, codec)
    F = re.shape[1]
    grp = R._groups(F, codec.group)
    b = codec.bits
    q = np.arange(2 ** b, dtype=np.float64) - 2 ** (b - 1)
    bad = 0
    for part, comp in enumerate((re, im)):
        for gi, (a, e) in enumerate(grp):
            s = sc[:, part * len(grp) + gi].astype(np.float64)
            grid = q[None, None, :] * s[:, None, None]
            tol = 3 * 2.0 ** -24 * 2 ** b * np.abs(s)[:, None]
            bad += nearest_violations(comp[:, a:e], codes[part][0][:, a:e], grid, tol)
    return bad


def _cart_oracle(x, codec):
    codes, sc, _ = R.encode(x, codec)
    return codes, sc


def test_cartesian_codes_are_nearest_and_extreme_is_exact():
    assert _cart_violations(_cart_oracle) == 0
    assert _cart_violations(_cart_off_by_one) > 0
    # the group's signed extreme sits on the long end of the grid, -2^(b-1) * s
    x, (re, im) = _spectra()
    codes, sc, _ = R.encode(x, O.Codec(O.RFFT_CART, 6, 32))
    for gi, (a, e) in enumerate(R._groups(re.shape[1], 32)):
        v = re[:, a:e].astype(np.float64)
        ext = np.where(-v.min(-1) >= v.max(-1), v.min(-1), v.max(-1))
        lvl = -32 * sc[:, gi].astype(np.float64)
        assert np.all(np.abs(lvl - ext) <= 2.0 ** -11 * np.abs(ext) * 33 / 32 + 1e-30)


# ------------------------------------------------------------------ binary16 limits of the scales

def test_rn16_saturates_at_largest_finite_binary16_and_drops_negative_zero():
    big = (2 - 2.0 ** -10) * 2.0 ** 15                     # 65504, largest finite binary16
    x = np.array([big, 65519.0, 65520.0, 1e6, 3e38, -65520.0, -1e9, -0.0, 0.0, 1e-9, -1e-9], F32)
    h = O.rn16(x)
    bits = h.view(np.uint16)
    assert h.dtype == np.float16
    assert list(bits[:5]) == [0x7BFF] * 5                 # no infinity: saturation
    assert list(bits[5:7]) == [0xFBFF] * 2
    assert list(bits[7:]) == [0, 0, 0, 0]                  # -0 and values below half the
    #                                                        smallest subnormal store +0
    # the smallest subnormal 2^-24 and rounding to it from above half of it
    assert O.rn16(np.array([2.0 ** -24, 0.51 * 2.0 ** -24], F32)).view(np.uint16).tolist() == [1, 1]


def test_saturated_scale_codes_clip_to_the_grid_ends():
    """A group whose extreme exceeds the binary16 range keeps the saturated scale,
    and values beyond the grid clip to its ends (the reading for fp16 overflow)."""
    y = np.array([[-8.0e5, -1.0e5, 0.0, 1.0e5, 5.0e5, 7.9e5, 3.0, -3.0]], F32)
    codes, s16, _ = O.codec._enc_int_absmax(y.reshape(1, 1, 8), 4)
    assert s16.view(np.uint16)[0, 0] == 0x7BFF               # -8e5 * -1/8 saturates to +65504
    q = codes[0, 0] - 8
    assert q[0] == -8 and q[5] == 7 and q[4] == 7 and q[2] == 0

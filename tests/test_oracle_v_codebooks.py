"""Pins of the two value codebooks the 64K experiment names as its next test
("Can 4-bit keys and 2-bit values hit a 1M-token memory budget?", Result: a
symmetric grid, or Gaussian Lloyd-Max levels on rotated values): the symmetric
b-bit grid (INT_SYM) and the Lloyd-Max levels of a unit normal (LLOYD).

The pages print neither table, so the pins are mathematical: the Lloyd-Max
optimality conditions checked by numerical integration (not the closed form the
oracle iterates), symmetry, the classical published levels and distortions,
brute-force nearest-level codes, and the exact grids of the symmetric codec.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy import integrate
from scipy.stats import norm

import oracle as O

F32 = np.float32

# Max (1960), "Quantizing for minimum distortion", Table I: positive output
# levels and mean-squared error of the optimum quantiser of a unit normal.
MAX_LEVELS = {2: [0.4528, 1.510], 3: [0.2451, 0.7560, 1.344, 2.152],
              4: [0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733]}
MAX_MSE = {2: 0.1175, 3: 0.03454, 4: 0.009497}


@pytest.mark.parametrize("b", [2, 3, 4])
def test_lloyd_levels_are_optimal_for_the_unit_normal(b):
    L = O.lloyd_levels(b).astype(np.float64)
    n = 2 ** b
    assert L.shape == (n,) and np.all(np.diff(L) > 0)
    assert np.allclose(L, -L[::-1], atol=1e-7)                 # symmetric
    edges = np.concatenate([[-np.inf], 0.5 * (L[:-1] + L[1:]), [np.inf]])
    mse = 0.0
    for k in range(n):
        a, c = edges[k], edges[k + 1]
        p, _ = integrate.quad(norm.pdf, a, c, epsabs=1e-13, epsrel=1e-12)
        m, _ = integrate.quad(lambda x: x * norm.pdf(x), a, c, epsabs=1e-13, epsrel=1e-12)
        assert abs(m / p - L[k]) < 2e-6                           # each level is its cell's centroid
        e, _ = integrate.quad(lambda x: (x - L[k]) ** 2 * norm.pdf(x), a, c, epsabs=1e-13, epsrel=1e-12)
        mse += e
    assert np.allclose(L[n // 2:], MAX_LEVELS[b], atol=1e-3)
    assert abs(mse - MAX_MSE[b]) < 2e-4 * max(1.0, MAX_MSE[b] * 10)


@pytest.mark.parametrize("b", [2, 3, 4])
def test_lloyd_codes_are_the_nearest_level_and_scale_is_rms(b):
    rng = np.random.default_rng(40 + b)
    y = rng.standard_normal((60, 64)).astype(np.float16)
    y[0] = 0.0                                                    # zero group
    c = O.Codec(O.LLOYD, b, 32)
    f, s, z = O.quantize_rows(y, c)
    assert z is None
    codes = f[0][0]
    L = O.lloyd_levels(b)
    yy = y.astype(np.float64).reshape(60, 2, 32)
    rms = np.sqrt((yy ** 2).mean(-1))
    s64 = s.astype(np.float64)
    assert np.all(np.abs(s64 - rms) <= rms * 2.0 ** -11 + 1e-12)  # fp16 rounding of the RMS
    t = (y.astype(F32).reshape(60, 2, 32) * O.inv32(s)[..., None]).reshape(60, 64)
    ref = np.argmin(np.abs(t.astype(np.float64)[..., None] - L.astype(np.float64)), axis=-1)
    diff = codes != ref
    if diff.any():   # only within binary32 rounding of a midpoint
        M = O.lloyd_midpoints(b).astype(np.float64)
        assert np.all(np.min(np.abs(t[diff][:, None].astype(np.float64) - M), axis=-1) < 1e-6)
    xh = O.dequant_rows(f, s, None, c, 64)
    assert np.array_equal(xh, (L[codes].reshape(60, 2, 32) * s.astype(F32)[..., None]).reshape(60, 64))
    assert np.all(xh[0] == 0)


def _nearest_half_grid(t, b):
    """Nearest level k - h (h = (2^b-1)/2) to each t, exactly; ties to the even k."""
    h = Fraction(2 ** b - 1, 2)
    out = []
    for v in t.ravel().tolist():
        cands = list(range(2 ** b))
        d = [abs(Fraction(v) - (k - h)) for k in cands]
        m = min(d)
        ks = [k for k, dk in zip(cands, d) if dk == m]
        out.append(ks[0] if len(ks) == 1 else [k for k in ks if k % 2 == 0][0])
    return np.array(out).reshape(t.shape)


@pytest.mark.parametrize("b", [2, 3])
def test_int_sym_grid_is_symmetric_and_codes_are_nearest(b):
    rng = np.random.default_rng(50 + b)
    y = (rng.standard_normal((40, 32)) * 2).astype(np.float16)
    y[1] = 0.0
    c = O.Codec(O.INT_SYM, b, 32)
    f, s, _ = O.quantize_rows(y, c)
    codes = f[0][0]
    h = (2 ** b - 1) / 2
    xh = O.dequant_rows(f, s, None, c, 32)
    # every value is on the half-integer grid (k - h) * s, as many levels below 0 as above
    assert np.array_equal(xh, ((codes.astype(F32) - F32(h)) * s.astype(F32)))
    lv = np.arange(2 ** b) - h
    assert np.array_equal(lv, -lv[::-1])
    if b == 2:
        assert list(lv) == [-1.5, -0.5, 0.5, 1.5]
    # the group's extreme lands on an outermost level
    i = np.argmax(np.abs(y.astype(np.float64)), axis=-1)
    ext = codes[np.arange(40), i]
    nz = np.abs(y).max(-1) > 0
    assert np.all((ext[nz] == 0) | (ext[nz] == 2 ** b - 1))
    # codes: nearest level of t = RN32(y * RN32(1/s)), ties to the even code, except where
    # binary32 rounding of t + h moved it across a half
    t = y.astype(F32) * O.inv32(s)
    ref = _nearest_half_grid(t, b)
    frac = np.abs((t.astype(np.float64) + h) - np.floor(t.astype(np.float64) + h) - 0.5)
    assert np.all((codes == ref) | (frac < 1e-6) | (t.astype(np.float64) + h > 2 ** b - 1) | (t + h < 0))
    assert np.all(xh[1] == 0)


def test_v_codebook_bits_per_value():
    assert O.bits_per_value(O.Codec(O.INT_SYM, 2, 128), 256) == 2.125
    assert O.bits_per_value(O.Codec(O.LLOYD, 3, 32), 128) == 3.5
    assert O.kv_bits_per_value(O.Codec(O.INT_ABSMAX, 4, 128, rot=256), O.Codec(O.LLOYD, 2, 128, rot=256), 256) == 3.125


def test_lloyd_beats_the_one_sided_grid_on_rotated_gaussian_values():
    """A property, not a number from the pages: on rotated Gaussian values at 2
    bits and group 128, the Lloyd-Max codebook (MSE-optimal for a normal of
    known spread) has lower squared error than the one-sided absmax grid."""
    rng = np.random.default_rng(77)
    v = rng.standard_normal((256, 256)).astype(np.float16)

    def rel_mse(c):
        f, s, z = O.quantize_rows(v, c)
        xh = O.dequant_rows(f, s, z, c, 256).astype(np.float64)
        x = v.astype(np.float64)
        return ((xh - x) ** 2).sum() / (x ** 2).sum()

    e_abs = rel_mse(O.Codec(O.INT_ABSMAX, 2, 128, rot=256))
    e_sym = rel_mse(O.Codec(O.INT_SYM, 2, 128, rot=256))
    e_ll = rel_mse(O.Codec(O.LLOYD, 2, 128, rot=256))
    assert e_ll < e_abs and e_ll < e_sym
    assert abs(e_ll - MAX_MSE[2]) < 0.03                        # close to the known-spread optimum

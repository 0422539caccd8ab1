"""Pins of the oracle codec against what the pages and mathematics fix (CPU only).

Each test pins the oracle to something other than itself: the pages' printed
grids and bit totals (golden JSON files, each entry cited), explicit Sylvester
matrices, brute-force nearest-level search, hand-worked examples of the
readings, and closed forms.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle as O
from oracle import rfft as R

GOLD = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ FWHT

@pytest.mark.parametrize("W", [2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_matches_sylvester_matrix(W):
    rng = np.random.default_rng(W)
    x = rng.standard_normal((64, W)).astype(F32)
    H = hadamard(W).astype(np.float64) / np.sqrt(W)   # Sylvester order, symmetric
    ref = x.astype(np.float64) @ H.T
    got = O.fwht(x, W).astype(np.float64)
    # log2(W) rounded adds plus one multiply, each relative 2^-24 of a partial sum
    tol = (np.log2(W) + 2) * 2.0 ** -24 * np.sqrt(W) * np.abs(x).max()
    assert np.abs(got - ref).max() <= tol


@pytest.mark.parametrize("W", [64, 128, 256])
def test_fwht_orthonormal_involution_energy(W):
    I = np.eye(W, dtype=F32)
    Hn = O.fwht(I, W).astype(np.float64)      # rows of H / sqrt(W)
    assert np.allclose(Hn @ Hn.T, np.eye(W), atol=2e-6)
    assert np.allclose(Hn, Hn.T, atol=0)        # symmetric, computed bitwise
    rng = np.random.default_rng(1)
    x = rng.standard_normal((32, W)).astype(F32)
    y = O.fwht(x, W)
    assert np.allclose((y.astype(np.float64) ** 2).sum(1), (x.astype(np.float64) ** 2).sum(1), rtol=1e-5)
    assert np.allclose(O.fwht(y, W), x, atol=1e-5)


def test_fwht_2x2_and_kappa():
    # H_2 = [[1, 1], [1, -1]] / sqrt 2
    y = O.fwht(np.array([[1.0, 0.0], [0.0, 1.0]], F32), 2)
    k2 = F32(1 / np.sqrt(2.0))
    assert np.array_equal(y, np.array([[k2, k2], [k2, -k2]], F32))
    # 1/sqrt(128) is the nearest binary32: 0x3DB504F3 (checked with exact rationals)
    k = O.fwht_kappa(128)
    assert k.view(np.uint32) == 0x3DB504F3
    kf = Fraction(float(k))
    ulp = Fraction(2) ** (-4 - 23)
    # |k - 1/sqrt(128)| <= ulp/2  <=>  (k -+ ulp/2)^2 brackets 1/128
    assert (kf - ulp / 2) ** 2 <= Fraction(1, 128) <= (kf + ulp / 2) ** 2
    assert O.fwht_kappa(256) == F32(0.0625) and O.fwht_kappa(64) == F32(0.125)


def test_fwht_butterfly_order_worked_example():
    ex = _gold("worked_examples.json")["fwht4_order"]
    y = O.fwht(np.array([ex["x"]], F32), 4)[0]
    assert np.array_equal(y, np.array(ex["y"], F32))


def test_fwht_blocks_when_width_below_head_dim():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 256)).astype(F32)
    y = O.fwht(x, 128)
    assert np.array_equal(y[:, :128], O.fwht(x[:, :128], 128))
    assert np.array_equal(y[:, 128:], O.fwht(x[:, 128:], 128))


# ------------------------------------------------------------------ grids

def _rows(n=257, D=256, seed=0, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, D)).astype(F32)
    if outliers:
        x[:, [3, 77, 200]] *= 10
    x[0] = 0.0                     # an all-zero row: zero scales
    x[1, :64] = -0.0
    return x.astype(np.float16)


def _deq(x16, c):
    f, s, z = O.quantize_rows(x16, c)
    return f, s, z, O.dequant_rows(f, s, z, c, x16.shape[1])


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("g", [8, 32, 128])
def test_int_absmax_grid_membership_and_extreme(b, g):
    x16 = _rows()
    c = O.Codec(O.INT_ABSMAX, b, g)
    f, s, _, xh = _deq(x16, c)
    codes = f[0][0]
    N, D = x16.shape
    q = codes.reshape(N, D // g, g) - 2 ** (b - 1)
    assert q.min() >= -(2 ** (b - 1)) and q.max() <= 2 ** (b - 1) - 1
    sf = s.astype(np.float64)
    # dequantised value / scale is exactly the integer grid point
    ratio = xh.reshape(N, D // g, g).astype(np.float64)
    nz = sf != 0
    assert np.array_equal(ratio[nz] / sf[nz][:, None], q[nz].astype(np.float64))
    # the group's extreme element takes the long side -2^(b-1)
    y = x16.astype(F32).reshape(N, D // g, g)
    mx, mn = y.max(-1), y.min(-1)
    m = np.where(-mn >= mx, mn, mx)               # +-A tie: the negative extreme
    at_ext = (y == m[..., None]) & nz[..., None]
    assert at_ext.any() and np.all(q[at_ext] == -(2 ** (b - 1)))
    # scales are never -0
    assert not np.any(np.signbit(s[s == 0]))


def test_int_absmax_2bit_grid_is_pages_grid():
    # E22L Result: the 2-bit grid is {-2, -1, 0, 1} x scale
    x16 = _rows()
    f, s, _, xh = _deq(x16, O.Codec(O.INT_ABSMAX, 2, 128))
    N = x16.shape[0]
    r = xh.reshape(N, 2, 128).astype(np.float64)
    sf = s.astype(np.float64)
    nz = sf != 0
    assert set(np.unique(r[nz] / sf[nz][:, None])) <= {-2.0, -1.0, 0.0, 1.0}


def _brute_nearest_int(t, lo, hi):
    """Nearest integer in [lo, hi] to binary32 t, ties to even, by exhaustive search."""
    best = []
    for v in t.ravel().tolist():
        cands = list(range(lo, hi + 1))
        d = [abs(Fraction(v) - k) for k in cands]
        m = min(d)
        ks = [k for k, dk in zip(cands, d) if dk == m]
        best.append(ks[0] if len(ks) == 1 else [k for k in ks if k % 2 == 0][0])
    return np.array(best).reshape(t.shape)


@pytest.mark.parametrize("cb,b", [(O.INT_ABSMAX, 3), (O.INT_ABSMAX, 4), (O.INT8_SYM, 8), (O.TERNARY, 2)])
def test_codes_are_brute_force_nearest(cb, b):
    rng = np.random.default_rng(5)
    y = (rng.standard_normal((40, 32)) * 3).astype(np.float16)
    y[0, 5] = 0.5   # exact ties appear after scaling below
    c = O.Codec(cb, b, 32)
    f, s, _ = O.quantize_rows(y, c)
    inv = O.inv32(s)
    t = (y.astype(F32).reshape(40, 1, 32) * inv[..., None]).reshape(40, 32)
    if cb == O.INT_ABSMAX:
        lo, hi, off = -(2 ** (b - 1)), 2 ** (b - 1) - 1, 2 ** (b - 1)
    elif cb == O.INT8_SYM:
        lo, hi, off = -127, 127, 127
    else:
        lo, hi, off = -1, 1, 1
    assert np.array_equal(f[0][0] - off, _brute_nearest_int(t, lo, hi))


def test_nf4_table_and_nearest_level():
    L = O.nf4_levels()
    assert L.shape == (16,) and np.all(np.diff(L) > 0)
    assert L[0] == -1 and L[-1] == 1 and L[7] == 0          # exact zero, 7 negative, 8 positive
    # the construction is from normal quantiles: symmetric extremes, mean of
    # the positive part equals the published NF4 property (levels in [-1, 1])
    rng = np.random.default_rng(6)
    y = rng.standard_normal((50, 64)).astype(np.float16)
    c = O.Codec(O.NF4, 4, 64)
    f, s, _ = O.quantize_rows(y, c)
    t = y.astype(F32) * O.inv32(s)[:, 0][:, None]
    codes = f[0][0]
    # brute force: nearest level, ties to the lower one
    d = np.abs(t.astype(np.float64)[..., None] - L.astype(np.float64))
    # midpoints are rounded to binary32 in the rule; compare against exact nearest
    ref = np.argmin(d, axis=-1)
    diff = codes != ref
    # disagreement only possible within binary32 rounding of a midpoint
    M = O.nf4_midpoints()
    if diff.any():
        near = np.min(np.abs(t[diff][:, None].astype(np.float64) - M), axis=-1)
        assert np.all(near < 1e-6)
    xh = O.dequant_rows(f, s, None, c, 64)
    assert np.array_equal(xh, (L[codes] * s.astype(F32)))


def test_ternary_sign_grids():
    x16 = _rows()
    f, s, _, xh = _deq(x16, O.Codec(O.TERNARY, 2, 8))
    N = x16.shape[0]
    r = xh.reshape(N, 32, 8).astype(np.float64)
    sf = s.astype(np.float64)
    nz = sf != 0
    assert set(np.unique(r[nz] / sf[nz][:, None])) <= {-1.0, 0.0, 1.0}
    f, s, _, xh = _deq(x16, O.Codec(O.SIGN, 1, 8))
    r = xh.reshape(N, 32, 8).astype(np.float64)
    sf = s.astype(np.float64)
    nz = sf != 0
    assert set(np.unique(r[nz] / sf[nz][:, None])) <= {-1.0, 1.0}
    # sign scale = mean |y| (within fp32 summation and fp16 rounding)
    y = np.abs(x16.astype(np.float64)).reshape(N, 32, 8).mean(-1)
    assert np.allclose(sf, y, rtol=2 ** -10, atol=1e-7)


def test_grid_error_bound_and_minmax_endpoints():
    x16 = _rows(outliers=False)
    for c in [O.Codec(O.INT_ABSMAX, 4, 32), O.Codec(O.INT_MINMAX, 4, 32), O.Codec(O.INT_MINMAX, 3, 32)]:
        f, s, z, xh = _deq(x16, c)
        N = x16.shape[0]
        y = x16.astype(np.float64).reshape(N, 8, 32)
        e = np.abs(xh.astype(np.float64).reshape(N, 8, 32) - y)
        sf = np.abs(s.astype(np.float64))[..., None]
        # half a step, plus fp16 rounding of the scale/min stretching the grid
        slack = 2 ** -10 * np.abs(y).max(-1, keepdims=True) * (2 ** c.bits)
        ok = e <= sf / 2 + slack + 1e-7
        if c.codebook == O.INT_ABSMAX:
            # values beyond the short side of the asymmetric grid are clipped
            t = y / s.astype(np.float64)[..., None]
            ok |= t > 2 ** (c.bits - 1) - 0.5
        assert np.all(ok)
        if c.codebook == O.INT_MINMAX:
            lo = y.min(-1)
            zf = z.astype(np.float64)
            assert np.all(np.abs(zf - lo) <= 2 ** -11 * np.abs(lo) + 1e-7)


@pytest.mark.parametrize("key", ["absmax_b2_grid", "minmax_b2", "ternary", "sign"])
def test_worked_grid_examples(key):
    ex = _gold("worked_examples.json")[key]
    g = np.array([ex["group"]], np.float16)
    n = g.shape[1]
    if key == "absmax_b2_grid":
        c = O.Codec(O.INT_ABSMAX, ex["bits"], n)
    elif key == "minmax_b2":
        c = O.Codec(O.INT_MINMAX, ex["bits"], n)
    elif key == "ternary":
        c = O.Codec(O.TERNARY, 2, n)
    else:
        c = O.Codec(O.SIGN, 1, n)
    f, s, z = O.quantize_rows(g, c)
    assert list(f[0][0][0]) == ex["codes"]
    assert float(s[0, 0]) == ex["scale"]
    if "min" in ex:
        assert float(z[0, 0]) == ex["min"]
    if "dequant" in ex:
        xh = O.dequant_rows(f, s, z, c, n)
        assert list(xh[0]) == ex["dequant"]


def test_zero_groups_and_negative_zero():
    x = np.zeros((2, 32), np.float16)
    x[1] = -0.0
    for c in [O.Codec(O.INT_ABSMAX, 4, 32), O.Codec(O.INT_MINMAX, 4, 32), O.Codec(O.TERNARY, 2, 32),
              O.Codec(O.SIGN, 1, 32), O.Codec(O.NF4, 4, 32), O.Codec(O.INT8_SYM, 8, 32)]:
        f, s, z, xh = _deq(x, c)
        assert np.all(s == 0) and not np.any(np.signbit(s))
        assert np.all(xh == 0)
        if z is not None:
            assert not np.any(np.signbit(z))


# ------------------------------------------------------------------ packing

@pytest.mark.parametrize("key", ["pack_b2", "pack_b3_straddle", "pack_b4_nibbles"])
def test_pack_worked_examples(key):
    ex = _gold("worked_examples.json")[key]
    w = O.pack_bits([(np.array([ex["codes"]]), ex["bits"])])
    assert list(w[0]) == ex["words"]


@pytest.mark.parametrize("b", [1, 2, 3, 4, 5, 6, 7, 8, 16])
def test_pack_roundtrip(b):
    rng = np.random.default_rng(b)
    codes = rng.integers(0, 2 ** b, size=(9, 256))
    w = O.pack_bits([(codes, b)])
    assert w.shape == (9, (256 * b + 31) // 32)
    assert np.array_equal(O.unpack_bits(w, [(256, b)])[0], codes)
    # stream bit k is bit k % 32 of word k // 32 (check every code bit directly)
    for j in (0, 7, 100, 255):
        for i in range(b):
            k = j * b + i
            assert ((int(w[3, k // 32]) >> (k % 32)) & 1) == ((int(codes[3, j]) >> i) & 1)


def test_fp16_codec_is_identity():
    x16 = _rows()
    c = O.Codec(O.FP16)
    w, s, z = O.quantize_pack(x16.reshape(1, 1, 1, *x16.shape), c)
    assert w.tobytes() == x16.tobytes()
    xh = O.dequant(w, s, z, c, (1, 1, 1) + x16.shape)
    assert np.array_equal(xh[0, 0, 0], x16.astype(F32))


# ------------------------------------------------------------------ accounting

def _codec(spec):
    name, b, g = spec
    cb = {"int_absmax": O.INT_ABSMAX, "nf4": O.NF4}[name]
    return O.Codec(cb, b, g)


def test_bits_per_value_pages():
    gold = _gold("accounting.json")
    for case in gold["cases"]:
        got = O.kv_bits_per_value(_codec(case["k"]), _codec(case["v"]), case["D"])
        assert got == case["bpv"], case["cite"]
    p = gold["rfft_payload"]
    assert O.rfft_payload_bits_per_value(p[0]["mag"], p[0]["phase"], p[0]["D"]) == p[0]["bpv"]
    assert p[0]["D"] // 2 + 1 == p[0]["bins"]
    lim = O.rfft_payload_bits_per_value(p[1]["mag"], p[1]["phase"], p[1]["D"])
    assert abs(lim - p[1]["bpv_limit"]) < 1e-3


def test_bits_per_value_minmax_and_anchor():
    # two fp16 parameters per min-max group; an fp16 anchor layer counts 16
    assert O.bits_per_value(O.Codec(O.INT_MINMAX, 4, 32), 128) == 5.0
    assert O.bits_per_value(O.Codec(O.INT_MINMAX, 3, 32), 256) == 4.0
    t = O.Codec(O.TERNARY, 2, 8)
    assert O.kv_bits_per_value(t, t, 128, anchor_layers=1, layers=32) == (16 + 31 * 4.0) / 32
    # the packed row length agrees with the accounting
    for c in [O.Codec(O.INT_ABSMAX, 3, 32), O.Codec(O.RFFT_POLAR, 5, 32, aux_bits=7),
              O.Codec(O.RFFT_CART, 6, 32), O.Codec(O.SIGN, 1, 8)]:
        nw, ns, nm = O.layout(c, 128)
        payload = O.bits_per_value(c, 128) * 128 - 16 * (ns + nm)
        assert nw == -(-int(round(payload)) // 32)


# ------------------------------------------------------------------ calibration

def test_chan_scale_calibration_roundtrip():
    rng = np.random.default_rng(9)
    k = (rng.standard_normal((2, 3, 100, 64)) * np.linspace(0.1, 10, 64)).astype(np.float16)
    k[0, 0, :, 5] = 0
    c = O.calibrate_chan_scale(k)
    lam = np.abs(k.astype(np.float64)).max(axis=2)
    assert c.shape == (2, 3, 64)
    assert c[0, 0, 5] == 1.0
    nz = lam != 0
    assert np.allclose(c[nz] * lam[nz], 1.0, rtol=2 ** -23)
    # pre-scale then divide back out after dequantising: values come back
    x = k[None]                                   # [1][L][H][T][D]
    cc = O.Codec(O.INT_ABSMAX, 8, 64)
    w, s, z = O.quantize_pack(x, cc, c)
    xh = O.dequant(w, s, z, cc, x.shape, c)
    rel = np.abs(xh - x.astype(F32)).max() / np.abs(x.astype(F32)).max()
    assert rel < 0.01

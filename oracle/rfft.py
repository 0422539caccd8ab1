"""Oracle rFFT physical codecs along head_dim (polar and Cartesian).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[FMAG-R] describes a physical codec: real K -> rFFT (one-sided spectrum of
D/2 + 1 bins) -> packed magnitude index + packed phase-angle index -> inverse
rFFT, with a fixed payload per complex coefficient (e.g. 4 + 8 bits, or the
matched-rate splits 5 + 7 and 6 + 6), and a real/imaginary control at the same
payload.  The pages fix neither the FFT algorithm, the grouping of magnitude
scales, nor the phase rule; the readings taken here:

* FFT: iterative radix-2 decimation in time on bit-reversed input, spans
  2, 4, ..., N; twiddle w_k = (RN32(cos 2 pi k/N), RN32(-sin 2 pi k/N)) from fp64;
  complex product (a+bi)(c+di) = (RN32(RN32(ac) - RN32(bd)), RN32(RN32(ad) +
  RN32(bc))); butterflies (x_top + t, x_top - t).  Forward unnormalised; the
  inverse rebuilds the Hermitian spectrum, uses conjugate twiddles, keeps the
  real part and multiplies by 1/N (exact).
* Polar: |z| = RN32(sqrt(RN32(RN32(re^2) + RN32(im^2)))) on an unsigned
  (2^b - 1)-step grid with one fp16 scale per `group` consecutive bins (last
  group ragged); phase = nearest of 2^p sectors centred on 2 pi k / 2^p, decided
  by exact sign flips/swaps into the first octant and binary32 side tests
  against the sector boundaries (no atan2), z = 0 -> sector 0.
* Cartesian: real parts and imaginary parts as two rows of bins, each coded on
  the signed absmax grid with b bits and the same ragged bin groups.
* Stream per row: all magnitude (or real) codes, then all phase (or imaginary)
  codes.
"""
from __future__ import annotations

import numpy as np

from .rounding import inv32, rn16

F32 = np.float32


def _bitrev(N: int) -> np.ndarray:
    nb = N.bit_length() - 1
    return np.array([int(format(i, f"0{nb}b")[::-1], 2) for i in range(N)], dtype=np.int64)


def twiddles(N: int):
    k = np.arange(N // 2, dtype=np.float64)
    ang = 2.0 * np.pi * k / N
    return np.cos(ang).astype(F32), (-np.sin(ang)).astype(F32)


def directions(P: int):
    """Sector centre directions (RN32 cos, RN32 sin) of 2 pi k / P."""
    k = np.arange(P, dtype=np.float64)
    ang = 2.0 * np.pi * k / P
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def boundaries(P: int):
    """First-octant sector boundaries beta_j = (2j+1) pi / P, j < P/8."""
    j = np.arange(P // 8, dtype=np.float64)
    ang = (2.0 * j + 1.0) * np.pi / P
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def fft(re: np.ndarray, im: np.ndarray, inverse: bool = False):
    """Radix-2 DIT FFT of complex rows (float32 [N_rows, N]) as described above."""
    N = re.shape[-1]
    wr_t, wi_t = twiddles(N)
    if inverse:
        wi_t = -wi_t
    r = _bitrev(N)
    ar = re[:, r].astype(F32, copy=True)
    ai = im[:, r].astype(F32, copy=True)
    span = 2
    while span <= N:
        half = span // 2
        step = N // span
        for j in range(half):
            wr = wr_t[j * step]
            wi = wi_t[j * step]
            top = np.arange(j, N, span)
            bot = top + half
            br = ar[:, bot]
            bi = ai[:, bot]
            tr = br * wr - bi * wi
            ti = br * wi + bi * wr
            xt_r = ar[:, top]
            xt_i = ai[:, top]
            ar[:, bot] = xt_r - tr
            ai[:, bot] = xt_i - ti
            ar[:, top] = xt_r + tr
            ai[:, top] = xt_i + ti
        span *= 2
    return ar, ai


def rfft(x: np.ndarray):
    """One-sided spectrum (bins 0..N/2) of real float32 rows [N_rows, N]."""
    N = x.shape[-1]
    ar, ai = fft(x.astype(F32), np.zeros_like(x, dtype=F32))
    return ar[:, : N // 2 + 1], ai[:, : N // 2 + 1]


def irfft(zr: np.ndarray, zi: np.ndarray, N: int) -> np.ndarray:
    """Real rows from a one-sided spectrum: Hermitian extension, inverse FFT,
    real part times 1/N."""
    F = N // 2 + 1
    fr = np.zeros((zr.shape[0], N), dtype=F32)
    fi = np.zeros((zr.shape[0], N), dtype=F32)
    fr[:, :F] = zr
    fi[:, :F] = zi
    idx = np.arange(1, N // 2)
    fr[:, N - idx] = zr[:, idx]
    fi[:, N - idx] = -zi[:, idx]
    ar, _ = fft(fr, fi, inverse=True)
    return ar * F32(1.0 / N)


def magnitude(re, im):
    return np.sqrt(re * re + im * im)


def phase_sector(re: np.ndarray, im: np.ndarray, P: int) -> np.ndarray:
    """Nearest phase sector k in [0, P) without atan2 (P = 2^p, p >= 3)."""
    neg_im = im < 0
    ai = np.where(neg_im, -im, im)
    neg_re = re < 0
    ar = np.where(neg_re, -re, re)
    swap = ai > ar
    x = np.where(swap, ai, ar)
    y = np.where(swap, ar, ai)          # now 0 <= y <= x: first octant
    bc, bs = boundaries(P)
    k0 = np.zeros(re.shape, dtype=np.int64)
    for j in range(P // 8):
        side = bc[j] * y - bs[j] * x    # >= 0: on or counter-clockwise of beta_j
        k0 += (side >= 0).astype(np.int64)
    k0 = np.where(x == 0, 0, k0)
    k = np.where(swap, P // 4 - k0, k0)
    k = np.where(neg_re, P // 2 - k, k)
    k = np.where(neg_im, P - k, k)
    return np.mod(k, P)


def _groups(F: int, g: int):
    return [(a, min(a + g, F)) for a in range(0, F, g)]


def _absmax_code(v, b):
    """Signed absmax grid (same rule as the int codebook) on a [N, n] slice."""
    mx = v.max(-1)
    mn = v.min(-1)
    m = np.where(-mn >= mx, mn, mx)
    s16 = rn16(m * F32(-(2.0 ** -(b - 1))))
    inv = inv32(s16)
    q = np.clip(np.rint(v * inv[:, None]), -(2 ** (b - 1)), 2 ** (b - 1) - 1)
    return (q + 2 ** (b - 1)).astype(np.int64), s16


def encode(x: np.ndarray, codec):
    """x float32 [N_rows, D] -> ([(codes, bits), ...], scales fp16 [N_rows, ns], None)."""
    from .codec import RFFT_POLAR
    N, D = x.shape
    F = D // 2 + 1
    re, im = rfft(x)
    grp = _groups(F, codec.group)
    if codec.codebook == RFFT_POLAR:
        mb = codec.bits
        mu = magnitude(re, im)
        qm = np.zeros((N, F), dtype=np.int64)
        sc = np.zeros((N, len(grp)), dtype=np.float16)
        for gi, (a, e) in enumerate(grp):
            s16 = rn16(mu[:, a:e].max(-1) / F32(2 ** mb - 1))
            inv = inv32(s16)
            qm[:, a:e] = np.clip(np.rint(mu[:, a:e] * inv[:, None]), 0, 2 ** mb - 1)
            sc[:, gi] = s16
        ph = phase_sector(re, im, 2 ** codec.aux_bits)
        return [(qm, mb), (ph, codec.aux_bits)], sc, None
    b = codec.bits
    qr = np.zeros((N, F), dtype=np.int64)
    qi = np.zeros((N, F), dtype=np.int64)
    sc = np.zeros((N, 2 * len(grp)), dtype=np.float16)
    for gi, (a, e) in enumerate(grp):
        qr[:, a:e], sc[:, gi] = _absmax_code(re[:, a:e], b)
        qi[:, a:e], sc[:, len(grp) + gi] = _absmax_code(im[:, a:e], b)
    return [(qr, b), (qi, b)], sc, None


def decode_spectrum(codes_list, scales, codec, D: int):
    """Dequantised one-sided spectrum (re, im) float32 [N_rows, D/2 + 1]."""
    from .codec import RFFT_POLAR
    F = D // 2 + 1
    grp = _groups(F, codec.group)
    N = codes_list[0][0].shape[0]
    scales = np.asarray(scales).reshape(N, -1)
    if codec.codebook == RFFT_POLAR:
        qm = codes_list[0][0]
        ph = codes_list[1][0]
        mu = np.zeros((N, F), dtype=F32)
        for gi, (a, e) in enumerate(grp):
            mu[:, a:e] = qm[:, a:e].astype(F32) * scales[:, gi].astype(F32)[:, None]
        dc, ds = directions(2 ** codec.aux_bits)
        return mu * dc[ph], mu * ds[ph]
    b = codec.bits
    qr, qi = codes_list[0][0], codes_list[1][0]
    zr = np.zeros((N, F), dtype=F32)
    zi = np.zeros((N, F), dtype=F32)
    for gi, (a, e) in enumerate(grp):
        zr[:, a:e] = (qr[:, a:e] - 2 ** (b - 1)).astype(F32) * scales[:, gi].astype(F32)[:, None]
        zi[:, a:e] = (qi[:, a:e] - 2 ** (b - 1)).astype(F32) * \
            scales[:, len(grp) + gi].astype(F32)[:, None]
    return zr, zi


def decode(codes_list, scales, codec, D: int) -> np.ndarray:
    zr, zi = decode_spectrum(codes_list, scales, codec, D)
    return irfft(zr, zi, D)

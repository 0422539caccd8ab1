"""Oracle codec: rotation, group scales, codebooks, bit packing, dequantisation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Every arithmetic step is one IEEE binary32 operation on NumPy float32 arrays
(never fused), scales are rounded to IEEE binary16 with round-to-nearest-even.
Notation: RN32/RN16 = round-to-nearest-even to binary32/binary16; rne(t) =
nearest integer, ties to even.  Citation tags are defined in
``oracle/__init__.py``.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import rfft as _rfft
from .rounding import inv32, rn16  # noqa: F401

F32 = np.float32

FP16, INT_ABSMAX, INT_MINMAX, TERNARY, SIGN, NF4, INT8_SYM, RFFT_POLAR, RFFT_CART, INT_SYM, LLOYD = range(11)
_NAMES = {FP16: "fp16", INT_ABSMAX: "int_absmax", INT_MINMAX: "int_minmax", TERNARY: "ternary",
          SIGN: "sign", NF4: "nf4", INT8_SYM: "int8_sym", RFFT_POLAR: "rfft_polar",
          RFFT_CART: "rfft_cart", INT_SYM: "int_sym", LLOYD: "lloyd"}


@dataclasses.dataclass(frozen=True)
class Codec:
    """One tensor's codec.

    codebook  one of the constants above
    bits      code bits (INT_ABSMAX/INT_MINMAX 2..8; fixed for the others; for
              the rFFT codecs: magnitude bits (polar) or per-component bits
              (Cartesian))
    group     values per fp16 scale (rFFT: frequency bins per scale)
    rot       Walsh-Hadamard width (0 = none); must divide head_dim
    aux_bits  phase bits of RFFT_POLAR (2**aux_bits sectors)
    """
    codebook: int
    bits: int = 0
    group: int = 0
    rot: int = 0
    aux_bits: int = 0

    @property
    def name(self) -> str:
        return _NAMES[self.codebook]

    def code_bits(self) -> int:
        return {FP16: 16, TERNARY: 2, SIGN: 1, NF4: 4, INT8_SYM: 8}.get(self.codebook, self.bits)


# ---------------------------------------------------------------- Walsh-Hadamard

def fwht_kappa(W: int) -> np.float32:
    """Normalisation 1/sqrt(W): exact power of two for even log2 W, else RN32."""
    e = W.bit_length() - 1
    if e % 2 == 0:
        return F32(2.0 ** (-(e // 2)))
    return F32(1.0 / np.sqrt(float(W)))


def fwht(x: np.ndarray, W: int) -> np.ndarray:
    """Normalised Walsh-Hadamard transform over each W-wide block of the last axis.

    Rotation of post-RoPE K/V before quantising, undone after dequantising
    ([E22L, What I tested]: 256-wide Hadamard rotation; [E21W, What I tested]
    arm B; [FMAG-R] Hadamard control at head_dim width).  Sylvester (natural)
    order; butterfly stages with strides 1, 2, 4, ..., W/2, each pair (i, i+s)
    becoming (RN32(u_i + u_{i+s}), RN32(u_i - u_{i+s})); then one RN32 multiply
    by 1/sqrt(W).  The transform is its own inverse (H/sqrt(W) is symmetric and
    orthogonal).
    """
    x = np.asarray(x, dtype=F32)
    shp = x.shape
    u = x.reshape(-1, W).copy()
    n = u.shape[0]
    s = 1
    while s < W:
        v = u.reshape(n, W // (2 * s), 2, s)
        a = v[:, :, 0, :]
        b = v[:, :, 1, :]
        u = np.stack((a + b, a - b), axis=2).reshape(n, W)
        s *= 2
    return (u * fwht_kappa(W)).reshape(shp)


# ---------------------------------------------------------------- per-channel K scale

def calibrate_chan_scale(k_cal: np.ndarray) -> np.ndarray:
    """Per-channel K multipliers c[l][h][d] = RN32(1/lambda), lambda = max_t |K|.

    [E21W, What I tested] arm C: per-channel key scaling calibrated offline on
    one text; the statistic is not given, the plain reading (absmax over the
    calibration tokens, SmoothAttention exponent 1) is taken.  k_cal is fp16
    [L][H][T][D] (one calibration sequence); a zero channel gets c = 1.
    """
    lam = np.abs(k_cal.astype(F32)).max(axis=-2)
    c = np.ones_like(lam)
    nz = lam != 0
    c[nz] = F32(1.0) / lam[nz]
    return c


# ---------------------------------------------------------------- shared key mean

def key_mean(k16: np.ndarray) -> np.ndarray:
    """Per-(layer, head) key mean mu[l][h][d] over every sequence and token.

    [LCPP] (llama.cpp issue "Per-head adaptive KV cache quantization", the later
    comment measuring the failure mode): a shared per-head key mean carries about
    half of the key energy; subtracting the running mean before quantising and
    restoring it afterwards removes the failure.  The pages give no estimator;
    the reading taken: the plain mean over the B*T rows present, from the exact
    sum of the fp16 values (an integer in units of 2^-24), divided by B*T in fp64
    and rounded to binary32 (the fp64 conversion of the sum, the fp64 quotient
    and the binary32 rounding are the only roundings).  k16: fp16 [B][L][H][T][D].
    """
    B, L, H, T, D = k16.shape
    ints = (k16.astype(np.float64) * 2.0 ** 24).astype(np.int64)   # exact: fp16 are multiples of 2^-24
    S = ints.sum(axis=(0, 3))                                       # exact int64 [L][H][D]
    n = B * T
    mu = (S.astype(np.float64) / float(n)) * 2.0 ** -24 if n else np.zeros(S.shape)
    return mu.astype(F32)


# ---------------------------------------------------------------- codebooks
# All encoders take y: float32 [..., G, g] (G groups of g values) and return
# (codes int64 [..., G, g], scale fp16 [..., G], min fp16 [..., G] or None).

def _enc_int_absmax(y, b):
    """Signed absmax grid [-2^(b-1), 2^(b-1)-1] * s, ggml style ([E22L, Result]:
    the 2-bit grid is {-2,-1,0,1}*s, one side has fewer levels).

    The scale carries the sign of the group's extreme element so that element
    lands on the long side: m = (-min >= max) ? min : max, s = RN16(m * -2^-(b-1)).
    q = clamp(rne(RN32(y * RN32(1/s))), -2^(b-1), 2^(b-1)-1); stored q + 2^(b-1).
    """
    mx = y.max(-1)
    mn = y.min(-1)
    m = np.where(-mn >= mx, mn, mx)
    s16 = rn16(m * F32(-(2.0 ** -(b - 1))))
    inv = inv32(s16)
    t = y * inv[..., None]
    q = np.clip(np.rint(t), -(2 ** (b - 1)), 2 ** (b - 1) - 1)
    return (q + 2 ** (b - 1)).astype(np.int64), s16, None


def _dec_int_absmax(codes, s16, b):
    q = (codes - 2 ** (b - 1)).astype(F32)
    return q * s16.astype(F32)[..., None]


def _enc_minmax(y, b):
    """Unsigned min-max grid [0, 2^b-1]*s + z ([E21W, What I tested] arm A, plain
    per-token min-max along head_dim).

    s = RN16(RN32(RN32(max - min) / (2^b - 1))), z = RN16(min);
    q = clamp(rne(RN32(RN32(y - z) * RN32(1/s))), 0, 2^b - 1).
    """
    lo = y.min(-1)
    hi = y.max(-1)
    s16 = rn16((hi - lo) / F32(2 ** b - 1))
    z16 = rn16(lo)
    inv = inv32(s16)
    t = (y - z16.astype(F32)[..., None]) * inv[..., None]
    q = np.clip(np.rint(t), 0, 2 ** b - 1)
    return q.astype(np.int64), s16, z16


def _dec_minmax(codes, s16, z16):
    # q*s is exact in binary32, so this is one rounding: RN32(q*s + z)
    return codes.astype(F32) * s16.astype(F32)[..., None] + z16.astype(F32)[..., None]


def _enc_ternary(y):
    """Ternary {-s, 0, +s} ([FMAG-6, Milestone], [FMAG-6, Best results]).
    Scale = group absmax (tails kept intact, [FMAG-6, Mechanism findings]);
    q = clamp(rne(RN32(y * RN32(1/s))), -1, 1); stored q + 1 in 2 bits."""
    s16 = rn16(np.abs(y).max(-1))
    inv = inv32(s16)
    q = np.clip(np.rint(y * inv[..., None]), -1, 1)
    return (q + 1).astype(np.int64), s16, None


def _dec_ternary(codes, s16):
    return (codes - 1).astype(F32) * s16.astype(F32)[..., None]


def _pairwise_sum(a):
    """Pairwise tree sum along the last axis: adjacent pairs first."""
    while a.shape[-1] > 1:
        a = a[..., 0::2] + a[..., 1::2]
    return a[..., 0]


def _enc_sign(y):
    """Binary sign {-s, +s} ([FMAG-6, Minimal recipe], [FMAG-6, Best results]).
    The pages give no scale; s = mean |y| (the L2-best scale for a fixed sign
    pattern), summed as a pairwise tree then scaled by 1/g (exact).  Code 1 for
    y >= 0 (including -0), 0 otherwise."""
    g = y.shape[-1]
    S = _pairwise_sum(np.abs(y))
    s16 = rn16(S * F32(1.0 / g))
    return (y >= 0).astype(np.int64), s16, None


def _dec_sign(codes, s16):
    s = s16.astype(F32)[..., None]
    return np.where(codes == 1, s, -s)


def nf4_levels() -> np.ndarray:
    """NormalFloat-4 levels as published with QLoRA (Dettmers et al. 2023: the
    construction of section 3, the table of Appendix E).

    Steps, in this order:
    - o = RN32(0.9677083), the offset to seven decimals, halfway between 1 - 1/30
      and 1 - 1/32 (so the outermost quantiles are finite);
    - positive side: the 9 probabilities p_i = RN32(o + i * (1/2 - o) / 8),
      i = 0..8, each formed in fp64 then rounded to binary32, last one dropped;
    - negative side: the same with 8 probabilities (divisor 7), last dropped,
      and the sign flipped;
    - each level = RN32 of the fp64 standard-normal quantile of its binary32
      probability; an exact zero is added and the 16 values are sorted;
    - every level is divided by the largest, in binary32.

    This reproduces the 16 values printed in the paper's Appendix E bit for bit
    (pinned by ``tests/golden/nf4_qlora.json``).  The pages name NF4 keys
    ([FMAG-6, Milestone]; fixed non-uniform codebooks win, [FMAG-6, Mechanism
    findings]) without printing levels, so the published table is the reading.
    """
    from scipy.stats import norm
    o = float(F32(0.9677083))
    pos = [F32(o + i * (0.5 - o) / 8.0) for i in range(8)]
    neg = [F32(o + i * (0.5 - o) / 7.0) for i in range(7)]
    v = [F32(norm.ppf(float(p))) for p in pos] + [F32(0.0)] + [F32(-norm.ppf(float(p))) for p in neg]
    v = np.sort(np.array(v, dtype=F32))
    return (v / v[-1]).astype(F32)


def nf4_midpoints(levels=None) -> np.ndarray:
    L = nf4_levels() if levels is None else levels
    return (L[:-1] + L[1:]) * F32(0.5)


def _enc_nf4(y):
    """NF4: s = RN16(absmax); t = RN32(y * RN32(1/s)); code = number of
    midpoints M_k = RN32(L_k + L_{k+1}) / 2 strictly below t (a tie goes to the
    lower level)."""
    s16 = rn16(np.abs(y).max(-1))
    inv = inv32(s16)
    t = y * inv[..., None]
    M = nf4_midpoints()
    codes = (t[..., None] > M).sum(-1)
    return codes.astype(np.int64), s16, None


def _dec_nf4(codes, s16):
    return nf4_levels()[codes] * s16.astype(F32)[..., None]


def _enc_int_sym(y, b):
    """Symmetric b-bit grid: levels k - h for k = 0 .. 2^b - 1, h = (2^b - 1)/2,
    i.e. half-integers with as many levels on each side ([E22L, Result]: the
    symmetric value grid is the next test after the one-sided {-2,-1,0,1}).  The
    pages fix no scale; reading: s = RN16(RN32(A / h)) with A = max |y| of the
    group (the extreme lands on the outermost level), t = RN32(y * RN32(1/s)),
    k = rne(RN32(t + h)) clipped to [0, 2^b - 1]."""
    h = F32((2 ** b - 1) / 2)
    A = np.abs(y).max(-1)
    s16 = rn16(A / h)
    inv = inv32(s16)
    t = y * inv[..., None]
    k = np.clip(np.rint(t + h), 0, 2 ** b - 1)
    return k.astype(np.int64), s16, None


def _dec_int_sym(codes, s16, b):
    h = F32((2 ** b - 1) / 2)
    return (codes.astype(F32) - h) * s16.astype(F32)[..., None]


def lloyd_levels(b: int) -> np.ndarray:
    """Lloyd-Max levels of the standard normal for 2^b levels ([E22L, Result]:
    Gaussian Lloyd-Max levels on rotated values as the next test).  The fixed
    point of Lloyd's two conditions in fp64: each cell boundary halfway between
    its neighbouring levels, each level the mean of N(0, 1) over its cell,
    (pdf(a) - pdf(b)) / (cdf(b) - cdf(a)); started from the cell-centre
    quantiles, stopped when no level moves by 1e-14; rounded to binary32.

    The pages print no levels: parity unpinned by the pages; pinned by the two
    optimality conditions (checked by numerical integration) and symmetry."""
    from scipy.stats import norm
    n = 2 ** b
    L = norm.ppf((np.arange(n) + 0.5) / n)
    for _ in range(100000):
        t = np.concatenate([[-np.inf], 0.5 * (L[:-1] + L[1:]), [np.inf]])
        m = (norm.pdf(t[:-1]) - norm.pdf(t[1:])) / (norm.cdf(t[1:]) - norm.cdf(t[:-1]))
        moved = np.abs(m - L).max()
        L = m
        if moved < 1e-14:
            break
    return L.astype(F32)


def lloyd_midpoints(b: int) -> np.ndarray:
    L = lloyd_levels(b)
    return (L[:-1] + L[1:]) * F32(0.5)


def _enc_lloyd(y, b):
    """Gaussian Lloyd-Max codebook.  Reading: the levels are those of a unit
    normal scaled by the group's root mean square s = RN16(sqrt(RN32(S * 1/g)))
    with S the fixed pairwise-tree sum of RN32(y^2) (the tree of the sign
    codec); t = RN32(y * RN32(1/s)); code = number of midpoints strictly below t
    (a tie goes to the lower level)."""
    g = y.shape[-1]
    S = _pairwise_sum(y * y)
    s16 = rn16(np.sqrt(S * F32(1.0 / g)))
    inv = inv32(s16)
    t = y * inv[..., None]
    M = lloyd_midpoints(b)
    return (t[..., None] > M).sum(-1).astype(np.int64), s16, None


def _dec_lloyd(codes, s16, b):
    return lloyd_levels(b)[codes] * s16.astype(F32)[..., None]


def _enc_int8_sym(y):
    """int8 per-token reference ([FMAG-6, Milestone] int8 KV row): symmetric
    +-127 grid, s = RN16(RN32(absmax / 127)); stored q + 127."""
    s16 = rn16(np.abs(y).max(-1) / F32(127.0))
    inv = inv32(s16)
    q = np.clip(np.rint(y * inv[..., None]), -127, 127)
    return (q + 127).astype(np.int64), s16, None


def _dec_int8_sym(codes, s16):
    return (codes - 127).astype(F32) * s16.astype(F32)[..., None]


# ---------------------------------------------------------------- packing

def pack_bits(fields) -> np.ndarray:
    """Row bitstreams: fields = [(codes int [N, n_i], b_i), ...] concatenated in
    order; code j of a field occupies stream bits [j*b, (j+1)*b); stream bit k
    is bit k%32 of uint32 word k//32; the last word is zero-padded.

    The pages only say the codes are packed ([FMAG-R] physical codec of packed
    magnitude and angle indices); this layout is the plain reading.
    """
    bit_rows = []
    for codes, b in fields:
        codes = np.asarray(codes, dtype=np.uint64)
        bits = (codes[..., None] >> np.arange(b, dtype=np.uint64)) & np.uint64(1)
        bit_rows.append(bits.reshape(codes.shape[0], -1).astype(np.uint8))
    bits = np.concatenate(bit_rows, axis=1)
    n = bits.shape[1]
    nw = (n + 31) // 32
    padded = np.zeros((bits.shape[0], nw * 32), dtype=np.uint8)
    padded[:, :n] = bits
    by = np.packbits(padded, axis=1, bitorder="little")
    return np.ascontiguousarray(by).view("<u4")


def unpack_bits(words: np.ndarray, widths) -> list:
    """Inverse of pack_bits: widths = [(n_i, b_i), ...] -> list of int64 [N, n_i]."""
    words = np.ascontiguousarray(words, dtype="<u4")
    bits = np.unpackbits(words.view(np.uint8), axis=1, bitorder="little").astype(np.int64)
    out, pos = [], 0
    for n, b in widths:
        f = bits[:, pos:pos + n * b].reshape(bits.shape[0], n, b)
        out.append((f << np.arange(b)).sum(-1))
        pos += n * b
    return out


def layout(codec: Codec, D: int):
    """(uint32 words per row, scales per row, mins per row)."""
    if codec.codebook in (RFFT_POLAR, RFFT_CART):
        F = D // 2 + 1
        ng = -(-F // codec.group)
        if codec.codebook == RFFT_POLAR:
            nbits = F * (codec.bits + codec.aux_bits)
            return (nbits + 31) // 32, ng, 0
        return (2 * F * codec.bits + 31) // 32, 2 * ng, 0
    b = codec.code_bits()
    if codec.codebook == FP16:
        return D * 16 // 32, 0, 0
    ng = D // codec.group
    return (D * b + 31) // 32, ng, ng if codec.codebook == INT_MINMAX else 0


# ---------------------------------------------------------------- rows

def quantize_rows(x16: np.ndarray, codec: Codec, cscale: np.ndarray | None = None,
                  mean: np.ndarray | None = None):
    """Quantise fp16 rows [N, D] -> (codes list of (int64 [N, n], bits), scales
    fp16 [N, ns] or None, mins fp16 [N, nm] or None).

    Steps ([E22L, What I tested]; [E21W, What I tested]): fp16 -> fp32 (exact);
    optional shared-mean subtraction RN32(x - mu) ([LCPP], the shared key-mean comment);
    optional per-channel multiply RN32(x * c) (arms C/D); optional FWHT over
    each `rot`-wide block; groups of `group` consecutive values; codebook.
    """
    N, D = x16.shape
    cb = codec.codebook
    if cb == FP16:
        return [(x16.view(np.uint16).astype(np.int64), 16)], None, None
    x = x16.astype(F32)
    if mean is not None:
        x = x - mean.astype(F32)
    if cscale is not None:
        x = x * cscale.astype(F32)
    if cb in (RFFT_POLAR, RFFT_CART):
        return _rfft.encode(x, codec)
    if codec.rot:
        x = fwht(x, codec.rot)
    g = codec.group
    y = x.reshape(N, D // g, g)
    if cb == INT_ABSMAX:
        codes, s, z = _enc_int_absmax(y, codec.bits)
    elif cb == INT_MINMAX:
        codes, s, z = _enc_minmax(y, codec.bits)
    elif cb == TERNARY:
        codes, s, z = _enc_ternary(y)
    elif cb == SIGN:
        codes, s, z = _enc_sign(y)
    elif cb == NF4:
        codes, s, z = _enc_nf4(y)
    elif cb == INT8_SYM:
        codes, s, z = _enc_int8_sym(y)
    elif cb == INT_SYM:
        codes, s, z = _enc_int_sym(y, codec.bits)
    elif cb == LLOYD:
        codes, s, z = _enc_lloyd(y, codec.bits)
    else:
        raise ValueError(f"unknown codebook {cb}")
    return [(codes.reshape(N, D), codec.code_bits())], s, z


def dequant_rows(codes_list, scales, mins, codec: Codec, D: int,
                 cscale: np.ndarray | None = None, mean: np.ndarray | None = None) -> np.ndarray:
    """Invert quantize_rows: fp32 [N, D] in the original coordinates (inverse
    codebook, inverse FWHT, then RN32(x / c) for pre-scaled keys, then RN32(x + mu)
    where a shared mean was subtracted)."""
    cb = codec.codebook
    if cb == FP16:
        return codes_list[0][0].astype(np.uint16).view(np.float16).astype(F32)
    if cb in (RFFT_POLAR, RFFT_CART):
        x = _rfft.decode(codes_list, scales, codec, D)
    else:
        codes = codes_list[0][0]
        N = codes.shape[0]
        g = codec.group
        c3 = codes.reshape(N, D // g, g)
        if cb == INT_ABSMAX:
            y = _dec_int_absmax(c3, scales, codec.bits)
        elif cb == INT_MINMAX:
            y = _dec_minmax(c3, scales, mins)
        elif cb == TERNARY:
            y = _dec_ternary(c3, scales)
        elif cb == SIGN:
            y = _dec_sign(c3, scales)
        elif cb == NF4:
            y = _dec_nf4(c3, scales)
        elif cb == INT8_SYM:
            y = _dec_int8_sym(c3, scales)
        elif cb == INT_SYM:
            y = _dec_int_sym(c3, scales, codec.bits)
        elif cb == LLOYD:
            y = _dec_lloyd(c3, scales, codec.bits)
        else:
            raise ValueError(f"unknown codebook {cb}")
        x = y.reshape(N, D)
        if codec.rot:
            x = fwht(x, codec.rot)
    if cscale is not None:
        x = x / cscale.astype(F32)
    if mean is not None:
        x = x + mean.astype(F32)
    return x


# ---------------------------------------------------------------- whole tensors

def _row_cscale(chan_scale, shape):
    """Broadcast a [L][H][D] vector (channel scale or shared mean) to rows of a
    [B][L][H][T][D] tensor."""
    if chan_scale is None:
        return None
    B, L, H, T, D = shape
    c = np.broadcast_to(chan_scale[None, :, :, None, :], (B, L, H, T, D))
    return c.reshape(-1, D)


def _field_widths(codec: Codec, D: int):
    if codec.codebook == RFFT_POLAR:
        F = D // 2 + 1
        return [(F, codec.bits), (F, codec.aux_bits)]
    if codec.codebook == RFFT_CART:
        F = D // 2 + 1
        return [(2 * F, codec.bits)]
    return [(D, codec.code_bits())]


def quantize_pack(x16: np.ndarray, codec: Codec, chan_scale: np.ndarray | None = None,
                  mean: np.ndarray | None = None):
    """fp16 [B][L][H][T][D] -> (words uint32 [rows][nw], scales fp16 [rows][ns],
    mins fp16 [rows][nm]); rows in [B][L][H][T] order.  chan_scale and mean are
    [L][H][D] fp32 or None."""
    shape = x16.shape
    D = shape[-1]
    rows = x16.reshape(-1, D)
    fields, s, z = quantize_rows(rows, codec, _row_cscale(chan_scale, shape), _row_cscale(mean, shape))
    if codec.codebook == RFFT_CART:
        fields = [(np.concatenate([fields[0][0], fields[1][0]], axis=1), codec.bits)]
    words = pack_bits(fields)
    N = rows.shape[0]
    scales = s.reshape(N, -1) if s is not None else np.zeros((N, 0), np.float16)
    mins = z.reshape(N, -1) if z is not None else np.zeros((N, 0), np.float16)
    return words, scales, mins


def dequant(words, scales, mins, codec: Codec, shape, chan_scale=None, mean=None) -> np.ndarray:
    """Packed rows -> fp32 [B][L][H][T][D] in the original coordinates."""
    D = shape[-1]
    widths = _field_widths(codec, D)
    fields = unpack_bits(words, widths)
    if codec.codebook == RFFT_CART:
        F = D // 2 + 1
        fields = [fields[0][:, :F], fields[0][:, F:]]
    if codec.codebook not in (RFFT_POLAR, RFFT_CART):
        N = words.shape[0]
        if codec.codebook != FP16:
            ng = D // codec.group
            scales = np.asarray(scales).reshape(N, ng)
            mins = np.asarray(mins).reshape(N, ng) if codec.codebook == INT_MINMAX else None
    fl = [(f, b) for f, (_, b) in zip(fields, widths)] if codec.codebook != RFFT_CART else \
        [(fields[0], codec.bits), (fields[1], codec.bits)]
    x = dequant_rows(fl, scales, mins, codec, D, _row_cscale(chan_scale, shape), _row_cscale(mean, shape))
    return x.reshape(shape)

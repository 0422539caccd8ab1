"""Pins of the shared key-mean subtraction ([LCPP], llama.cpp issue "Per-head
adaptive KV cache quantization", the later comment measuring the failure mode: a
per-head shared key mean carries about half of the key energy; subtracting the
running mean before quantising and restoring it after removes the failure).

The pages print no numbers that a CPU run could reproduce (their figures are
perplexities of real models), so the pins are mathematical: the mean against
exact rational arithmetic, closed forms, exact shift invariance of the codes, and
the restore in dequantisation."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth

F32 = np.float32


def test_key_mean_is_the_rounded_exact_mean():
    rng = np.random.default_rng(3)
    k = (rng.standard_normal((2, 2, 3, 7, 8)) * np.exp(rng.uniform(-14, 10, (2, 2, 3, 7, 8)))).astype(np.float16)
    k[0, 0, 0, :, 0] = np.float16(6e-8)          # fp16 subnormals
    k[:, 1, 2, :, 3] = np.float16(65504.0)       # largest fp16
    mu = O.key_mean(k)
    assert mu.shape == (2, 3, 8) and mu.dtype == np.float32
    for l in range(2):
        for h in range(3):
            for d in range(8):
                vals = [Fraction(float(v)) for v in k[:, l, h, :, d].ravel()]
                exact = sum(vals, Fraction(0)) / len(vals)
                r32 = F32(float(exact))                            # RN64 then RN32 of the exact mean
                got = Fraction(float(mu[l, h, d]))
                ulp = Fraction(float(np.spacing(np.abs(r32)))) if r32 != 0 else Fraction(1, 2 ** 149)
                assert abs(got - exact) <= ulp, (l, h, d)
                # equal to the once-rounded exact mean unless the fp64 quotient sat on a binary32 tie
                assert mu[l, h, d] == r32 or abs(exact - (Fraction(float(r32)) + got) / 2) < exact * Fraction(1, 2 ** 50)
    assert mu[1, 2, 3] == F32(65504.0)


def test_key_mean_closed_forms():
    x = np.zeros((3, 1, 2, 5, 16), np.float16)
    x[:, 0, 0] = np.float16(1.25)                                 # constant rows
    x[:, 0, 1, :, :8] = np.float16(3.0)
    x[:, 0, 1, :, 8:] = np.float16(-3.0)
    mu = O.key_mean(x)
    assert np.all(mu[0, 0] == F32(1.25))
    assert np.all(mu[0, 1, :8] == F32(3.0)) and np.all(mu[0, 1, 8:] == F32(-3.0))
    y = np.concatenate([x, -x], axis=3)                           # +r and -r rows: mean 0
    assert np.all(O.key_mean(y) == 0)


def _exact_pair(rng, shape):
    """fp16 rows x and a mean m on grids coarse enough that x + m is exact in
    fp16 and (x + m) - m == x exactly in binary32."""
    x = (rng.integers(-512, 512, shape) / 16.0).astype(np.float16)
    m = (rng.integers(-64, 64, shape[:-2] + shape[-1:]) / 4.0).astype(np.float32)   # [L][H][D]
    xm = (x.astype(np.float32) + m[:, :, None, :]).astype(np.float16)
    assert np.array_equal(xm.astype(np.float32) - m[:, :, None, :], x.astype(np.float32))
    return x, m, xm


@pytest.mark.parametrize("cspec", [(O.INT_ABSMAX, 4, 32, 0), (O.INT_ABSMAX, 3, 128, 256), (O.INT_MINMAX, 3, 32, 0),
                                   (O.NF4, 4, 64, 0), (O.RFFT_POLAR, 5, 32, 0, 7), (O.RFFT_CART, 6, 16, 0)])
def test_mean_subtraction_codes_are_shift_invariant(cspec):
    """Coding x + m with mean m gives exactly the codes and scales of coding x."""
    rng = np.random.default_rng(17)
    c = O.Codec(*cspec)
    x, m, xm = _exact_pair(rng, (2, 3, 11, 128))
    ref = O.quantize_pack(x[None], c)
    got = O.quantize_pack(xm[None], c, None, m)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    # the restore: dequant with the mean is dequant without it, plus the mean (one rounding)
    d0 = O.dequant(*ref, c, (1,) + x.shape)
    d1 = O.dequant(*got, c, (1,) + x.shape, None, m)
    assert np.array_equal(d1, (d0 + m[None, :, :, None, :]).astype(np.float32))


def test_mean_then_channel_scale_order():
    """The mean is subtracted before the per-channel multiply and added after the
    division: x -> RN32(RN32(x - m) * c), restored as RN32(RN32(y / c) + m)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 1, 2, 9, 64)).astype(np.float16)
    m = rng.standard_normal((1, 2, 64)).astype(np.float32)
    cs = rng.uniform(0.5, 2.0, (1, 2, 64)).astype(np.float32)
    c = O.Codec(O.INT_ABSMAX, 8, 16, 0)
    rows = x.reshape(-1, 64)
    mr = np.repeat(m.reshape(2, 64), 9, axis=0)
    cr = np.repeat(cs.reshape(2, 64), 9, axis=0)
    y = (rows.astype(np.float32) - mr) * cr
    w, s, z = O.quantize_pack(x, c, cs, m)
    f, s2, _ = O.quantize_rows(rows, c, cr, mr)
    yq = O.dequant_rows(f, s2, None, c, 64)                        # coded y, no restore
    back = O.dequant(w, s, z, c, x.shape, cs, m).reshape(-1, 64)
    assert np.array_equal(back, (yq / cr + mr).astype(np.float32))
    assert np.abs(yq - y).max() <= np.abs(y).max() / 127 * 0.5 + 1e-6   # 8-bit grid around y, not x


def test_synthetic_mean_share_and_estimate():
    w = synth.get("c3", L=2, T=3000, n_q=2, k_mean_share=0.53)
    K, _ = synth.gen_kv(w)
    k = K.astype(np.float64)
    mu = O.key_mean(K).astype(np.float64)
    share = (mu ** 2).sum(-1).mean() / (k ** 2).sum(-1).mean()
    assert abs(share - 0.53) < 0.02
    res = k - mu[None, :, :, None, :]
    assert np.abs(res.mean(axis=(0, 3))).max() < 1e-5              # the residual rows have mean ~0
    w0 = synth.get("c3", L=2, T=3000, n_q=2)
    K0, _ = synth.gen_kv(w0)
    assert (O.key_mean(K0).astype(np.float64) ** 2).sum(-1).mean() < 0.02 * (K0.astype(np.float64) ** 2).sum(-1).mean()


def test_mean_subtraction_lowers_attention_kl_with_a_shared_mean():
    """A property, not a number from the pages: with a shared mean carrying 53% of
    the key energy, 3-bit rotated absmax keys give a clearly lower attention KL
    once the mean is subtracted (the direction of the pages' 3-bit result)."""
    w = synth.get("c3", L=1, T=1500, n_q=3, k_mean_share=0.53)
    Kx, Vx = synth.gen_kv(w)
    q, kvl = synth.gen_queries(w)
    mu = O.key_mean(Kx)
    kc = O.Codec(O.INT_ABSMAX, 3, 128, 256)
    Vd = Vx.astype(np.float32)
    kl = []
    for m in (None, mu):
        wk, sk, zk = O.quantize_pack(Kx, kc, None, m)
        Kd = O.dequant(wk, sk, zk, kc, Kx.shape, None, m)
        kl.append(O.attn_error(q, Kx, Vx, Kd, Vd, kvl)[0].mean())
    assert kl[1] < 0.7 * kl[0]

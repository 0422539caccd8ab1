"""Pins of the attention-visible error ladder ([FMAG-R], the Colab-probe reply:
QK-logit error, attention KL / JS, top-attended-token flips, attention-output
error) and of the entropy-adaptive bit rule ([LCPP], llama.cpp issue "Per-head
adaptive KV cache quantization", Finding 2: b_h = b_avg + 0.25 (H_avg - H_2(h)),
H_2 the Renyi entropy of the head's attention).  Closed forms, bounds and brute
force; the pages print no values for synthetic inputs."""
import math

import numpy as np
import pytest

import oracle as O
import synth


def test_renyi2_closed_forms():
    assert O.renyi2(np.zeros(7)) == pytest.approx(math.log(7))          # uniform over n keys
    assert O.renyi2(np.array([0.0, -1e4, -1e4])) == pytest.approx(0.0, abs=1e-12)   # one key
    for a in (0.1, 0.3, 0.5, 0.9):
        lg = np.log(np.array([a, 1 - a]))
        assert O.renyi2(lg) == pytest.approx(-math.log(a * a + (1 - a) ** 2), rel=1e-12)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 33)) * 3
    p = np.exp(x - x.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    shannon = -(p * np.log(p)).sum(-1)
    h2 = O.renyi2(x)
    assert np.all(h2 <= shannon + 1e-12) and np.all(h2 >= 0) and np.all(h2 <= math.log(33) + 1e-12)
    assert np.allclose(O.renyi2(x + 5.0), h2)                            # softmax shift invariance
    assert O.renyi2(np.zeros((2, 0))).shape == (2,)


def test_js_closed_forms_and_bounds():
    p, r = np.array([0.5, 0.5]), np.array([0.25, 0.75])
    m = (p + r) / 2
    ref = 0.5 * sum(pi * math.log(pi / mi) for pi, mi in zip(p, m)) + 0.5 * sum(ri * math.log(ri / mi)
                                                                              for ri, mi in zip(r, m))
    assert O.js_div(np.log(p), np.log(r)) == pytest.approx(ref, rel=1e-12)
    assert O.js_div(np.log(r), np.log(p)) == pytest.approx(ref, rel=1e-12)   # symmetric
    rng = np.random.default_rng(1)
    a, b = rng.standard_normal((40, 17)) * 2, rng.standard_normal((40, 17)) * 2
    js = O.js_div(a, b)
    assert np.all(js >= 0) and np.all(js <= math.log(2) + 1e-12)
    assert np.allclose(O.js_div(a, a), 0.0, atol=1e-15)
    jeff = O.kl_div(a, b) + O.kl_div(b, a)
    assert np.all(js <= 0.25 * jeff + 1e-12)                              # JS <= Jeffreys / 4
    far = O.js_div(np.array([0.0, -200.0]), np.array([-200.0, 0.0]))    # disjoint mass: ln 2
    assert far == pytest.approx(math.log(2), rel=1e-9)


def test_logit_error_and_top1():
    l = np.array([1.0, -2.0, 0.5, 3.0])
    assert O.logit_relerr(l, l) == 0.0
    assert O.logit_relerr(l, 2 * l) == pytest.approx(1.0)
    assert O.logit_relerr(l, l + np.array([0, 0, 0, 1.0])) == pytest.approx(1.0 / np.linalg.norm(l))
    assert O.top1_flip(l, l) == 0.0
    assert O.top1_flip(l, np.array([1.0, -2.0, 3.5, 3.0])) == 1.0
    assert O.top1_flip(np.array([2.0, 2.0, 1.0]), np.array([2.0, 1.0, 2.0])) == 0.0   # first index on ties


def test_entropy_adaptive_bits_rule():
    h2 = np.array([0.2, 2.0, 3.0, 3.4, 4.1, 1.0])
    b = O.entropy_adaptive_bits(h2, 4.0)
    assert b.mean() == pytest.approx(4.0, abs=1e-12)                     # the average is kept
    assert np.all(np.diff(b[np.argsort(h2)]) <= 0)                       # sharper heads get more bits
    assert b[0] - b[4] == pytest.approx(0.25 * (4.1 - 0.2))


def test_attn_error_ex_agrees_and_vanishes_on_exact_caches():
    w = synth.get("c1", T=200, n_q=4)
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w, Kx)
    c = O.Codec(O.INT_MINMAX, 3, 32, 0)
    wk, sk, zk = O.quantize_pack(Kx, c)
    wv, sv, zv = O.quantize_pack(Vx, c)
    Kd, Vd = O.dequant(wk, sk, zk, c, Kx.shape), O.dequant(wv, sv, zv, c, Vx.shape)
    kl, re, kv = O.attn_error(q, Kx, Vx, Kd, Vd, kv_len)
    r = O.attn_error_ex(q, Kx, Vx, Kd, Vd, kv_len)
    assert np.array_equal(r["kl"], kl) and np.array_equal(r["relerr"], re) and np.array_equal(r["kv_err"], kv)
    assert np.all(r["js"] > 0) and np.all(r["js"] <= np.log(2)) and np.all(r["logit_relerr"] > 0)
    e = O.attn_error_ex(q, Kx, Vx, Kx.astype(np.float32), Vx.astype(np.float32), kv_len)
    assert np.all(e["js"] == 0) and np.all(e["logit_relerr"] == 0) and np.all(e["top1_flip"] == 0)
    assert np.allclose(e["renyi2"], r["renyi2"])                         # the fp16 side only

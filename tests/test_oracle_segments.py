"""Pins of the segment machinery around the path ([FMAG-6] The winning recipe,
Selective-Layer Decode Anchoring; Minimal recipe; Milestone): the effective-bits
accounting against the figure the pages print, the tiling rule, the assembly of a
logical cache from segments, and the row independence the append path relies on."""
import json
import os

import numpy as np
import pytest

import oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")

_CB = {"fp16": O.FP16, "nf4": O.NF4, "int_absmax": O.INT_ABSMAX}


def _codec(spec):
    return O.Codec(_CB[spec[0]], *spec[1:])


def test_effective_bits_of_the_pages_figures():
    gold = json.load(open(os.path.join(GOLD, "effective_bits.json")))
    for c in gold["cases"]:
        if c.get("payload_only"):
            # payload-only figure: a 1-bit code with no scales, the anchor layer at 16
            bits = {"fp16": 16.0, "sign_payload": 1.0}
            tot = sum(bits[k[0]] * nl * nt for (k, v, l0, nl, t0, nt) in c["segments"])
            e = tot / (c["layers"] * c["tokens"])
        else:
            segs = [(_codec(k), _codec(v), l0, nl, t0, nt) for (k, v, l0, nl, t0, nt) in c["segments"]]
            e = O.effective_bits(segs, c["layers"], c["tokens"], c["D"])
        assert abs(e - c["effective_bits"]) <= c["tolerance"], c["cite"]


def test_effective_bits_closed_forms():
    nf4 = (O.Codec(O.NF4, 4, 64), O.Codec(O.INT_ABSMAX, 4, 64))
    f16 = (O.Codec(O.FP16), O.Codec(O.FP16))
    # one fp16 anchor layer adds (16 - b) / layers
    for L in (2, 8, 26, 32):
        segs = [(*f16, 0, 1, 0, 10), (*nf4, 1, L - 1, 0, 10)]
        assert O.effective_bits(segs, L, 10, 128) == pytest.approx(4.25 + (16 - 4.25) / L, abs=1e-12)
    # prompt + decode anchors on every layer (A = L + D rows at fp16): ((A) 16 + (T - A) b) / T,
    # tending to 16 as the prompt grows
    prev = 0.0
    for P in (16, 64, 256, 1024, 4000):
        T, D = 4096, 32
        segs = [(*f16, 0, 4, 0, P + D), (*nf4, 0, 4, P + D, T - P - D)]
        e = O.effective_bits(segs, 4, T, 128)
        assert e == pytest.approx(((P + D) * 16 + (T - P - D) * 4.25) / T, abs=1e-12)
        assert e > prev
        prev = e
    assert prev > 15.4


@pytest.mark.parametrize("segs,ok", [
    ([(0, 2, 0, 8)], True),
    ([(0, 2, 0, 5), (0, 2, 5, 3)], True),
    ([(0, 1, 0, 8), (1, 1, 0, 2), (1, 1, 2, 6)], True),
    ([(0, 2, 0, 5), (0, 2, 6, 2)], False),          # gap at token 5
    ([(0, 2, 0, 5), (0, 2, 4, 4)], False),          # overlap at token 4
    ([(0, 1, 0, 8)], False),                        # layer 1 uncovered
    ([(0, 2, 0, 9)], False),                        # past the end
    ([(0, 2, 0, 8), (1, 1, 3, 1)], False),          # double cover
])
def test_tiling_rule(segs, ok):
    assert O.tiles(segs, 2, 8) == ok


def test_assembly_places_each_segment_and_decode_is_the_whole_cache():
    w = synth.get("c3", L=3, T=90, n_q=2)
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w)
    Kf, Vf = Kx.astype(np.float32), Vx.astype(np.float32)
    cuts = [(0, 1, 0, 90), (1, 2, 0, 40), (1, 2, 40, 50)]
    segs = [(Kf[:, l0:l0 + nl, :, t0:t0 + nt], Vf[:, l0:l0 + nl, :, t0:t0 + nt], l0, t0) for (l0, nl, t0, nt) in cuts]
    Kd, Vd = O.assemble_segments(segs, *Kx.shape)
    assert np.array_equal(Kd, Kf) and np.array_equal(Vd, Vf)
    o1, l1 = O.decode_attn(q, Kd, Vd, kv_len)
    o2, l2 = O.decode_attn(q, Kf, Vf, kv_len)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    with pytest.raises(AssertionError):
        O.assemble_segments(segs[:2], *Kx.shape)


@pytest.mark.parametrize("cspec", [(O.INT_ABSMAX, 4, 128, 128), (O.INT_MINMAX, 3, 32, 0), (O.NF4, 4, 64, 0),
                                   (O.RFFT_POLAR, 5, 32, 0, 7), (O.SIGN, 1, 8, 0)])
def test_rows_code_independently(cspec):
    """The append path writes a token window; its codes are the rows of coding the
    whole tensor, because no codec step mixes rows."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((2, 2, 3, 20, 128)).astype(np.float16)
    c = O.Codec(*cspec)
    w, s, z = O.quantize_pack(x, c)
    ww, sw, zw = O.quantize_pack(np.ascontiguousarray(x[:, :, :, 7:12]), c)
    rows = np.arange(w.shape[0]).reshape(2, 2, 3, 20)[:, :, :, 7:12].ravel()
    assert np.array_equal(w[rows], ww) and np.array_equal(s[rows], sw) and np.array_equal(z[rows], zw)


def test_head_ranges_tile_and_weigh():
    """Per-head codec maps ([LCPP] the per-head KV-type request): segments over head
    ranges tile (layer, head, token) cells; a sink head at fp16 among 4-bit heads
    weighs 1 / heads of the cache."""
    assert O.tiles([(0, 2, 0, 8, 0, 1), (0, 2, 0, 8, 1, 3)], 2, 8, heads=4)
    assert not O.tiles([(0, 2, 0, 8, 0, 1), (0, 2, 0, 8, 2, 2)], 2, 8, heads=4)          # head 1 missing
    assert not O.tiles([(0, 2, 0, 8, 0, 2), (0, 2, 0, 8, 1, 3)], 2, 8, heads=4)          # head 1 twice
    i4 = O.Codec(O.INT_ABSMAX, 4, 64)
    f16 = O.Codec(O.FP16)
    e = O.effective_bits([(f16, f16, 0, 3, 0, 50, 0, 1), (i4, i4, 0, 3, 0, 50, 1, 7)], 3, 50, 128, heads=8)
    assert e == pytest.approx((16 + 7 * 4.25) / 8, abs=1e-12)
    rng = np.random.default_rng(3)
    K = rng.standard_normal((1, 2, 4, 6, 8)).astype(np.float32)
    segs = [(K[:, :, :1], K[:, :, :1], 0, 0, 0), (K[:, :, 1:, :4], K[:, :, 1:, :4], 0, 0, 1),
            (K[:, :, 1:, 4:], K[:, :, 1:, 4:], 0, 4, 1)]
    Kd, _ = O.assemble_segments(segs, 1, 2, 4, 6, 8)
    assert np.array_equal(Kd, K)

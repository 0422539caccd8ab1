"""The C ABI without a GPU: the library loads, exports every entry point that
include/kvq.h declares, and its host-only calls (layouts, bit accounting,
constant tables, argument validation) agree with the oracle and the header.

Every call here either is host-only or is rejected by argument validation
before anything is launched; no kernel runs.  Some calls pass FAKE, a made-up device
address, relying on host validation to reject them first; so the whole module skips
itself wherever a GPU is visible, and a gap in validation can never turn into a
device access.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O

def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


pytestmark = pytest.mark.skipif(_gpu_visible(), reason="passes made-up device addresses: CPU-only host test")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

OK, ERR_ARG, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE = 0, -1, -2, -3, -4
FAKE = 0x10000            # a 16-byte-aligned non-null address; never dereferenced (validation fails first)
FAKE_ODD = FAKE + 8       # 8-byte aligned only


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def K():
    import kv_cache_bit_fwht_amd as K
    return K


def test_library_exports_every_declared_entry_point(K):
    declared = _declared()
    assert len(declared) >= 13
    lib = ctypes.CDLL(K.LIB_PATH)
    missing = [n for n in declared if not hasattr(lib, n)]
    assert not missing, f"declared in kvq.h but not exported: {missing}"
    assert sorted(K.EXPORTS) == declared, "the Python binding must mirror the header one to one"


def test_timeline_entry_point_only_in_the_profiling_build(K):
    """kvq_timeline_read is declared in its own header and exported only by the
    profiling build (libkvq_timeline.so); the default library keeps the stamps out."""
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "kvq_timeline.h")).read(), flags=re.S)
    assert re.findall(r"\b(kvq_[a-z_0-9]+)\s*\(", text) == ["kvq_timeline_read"]
    assert not hasattr(ctypes.CDLL(os.path.join(os.path.dirname(K.LIB_PATH), "libkvq.so")), "kvq_timeline_read")
    tl = os.path.join(os.path.dirname(K.LIB_PATH), "libkvq_timeline.so")
    if os.path.exists(tl):
        assert hasattr(ctypes.CDLL(tl), "kvq_timeline_read")


def test_status_strings_and_version(K):
    assert K.kvq_version().startswith("kvq")
    for st in (OK, ERR_ARG, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, -5):
        s = K.kvq_status_string(st)
        assert s and s != K.kvq_status_string(12345)


CODECS = [
    O.Codec(O.FP16),
    O.Codec(O.INT_ABSMAX, 2, 128),
    O.Codec(O.INT_ABSMAX, 3, 32),
    O.Codec(O.INT_ABSMAX, 4, 128, rot=256),
    O.Codec(O.INT_ABSMAX, 4, 256, rot=128),
    O.Codec(O.INT_MINMAX, 4, 64),
    O.Codec(O.INT_MINMAX, 8, 16),
    O.Codec(O.TERNARY, 0, 32),
    O.Codec(O.SIGN, 0, 8),
    O.Codec(O.NF4, 0, 64),
    O.Codec(O.INT8_SYM, 0, 128),
    O.Codec(O.RFFT_POLAR, 4, 32, aux_bits=8),
    O.Codec(O.RFFT_CART, 3, 16),
    O.Codec(O.INT_SYM, 2, 128, rot=256),
    O.Codec(O.INT_SYM, 3, 32),
    O.Codec(O.LLOYD, 2, 128, rot=256),
    O.Codec(O.LLOYD, 4, 16),
]


def _valid_dims(c):
    if c.codebook in (O.FP16, O.RFFT_POLAR, O.RFFT_CART):
        return (64, 128, 256)
    return tuple(D for D in (64, 128, 256) if c.group <= D and c.rot <= D)


def _kcodec(K, c):
    return K.Codec(c.codebook, c.bits, c.group, c.rot, c.aux_bits)


@pytest.mark.parametrize("ci", range(len(CODECS)))
def test_layout_and_bits_match_the_oracle(K, ci):
    oc = CODECS[ci]
    dims = _valid_dims(oc)
    assert dims
    for D in dims:
        shape = K.Shape(1, 2, 3, 5, D)
        assert K.kvq_packed_layout(shape, _kcodec(K, oc)) == O.layout(oc, D)
        assert K.kvq_bits_per_value(_kcodec(K, oc), D) == pytest.approx(O.accounting.bits_per_value(oc, D), abs=0)


def test_bits_per_value_of_the_pages_figures(K):
    """The library's accounting against the figures the pages print (cited per
    case in tests/golden/accounting.json)."""
    import json
    cases = json.load(open(os.path.join(ROOT, "tests", "golden", "accounting.json")))["cases"]
    names = {"int_absmax": K.INT_ABSMAX, "nf4": K.NF4}
    for c in cases:
        kc = K.Codec(names[c["k"][0]], c["k"][1], c["k"][2], 0)
        vc = K.Codec(names[c["v"][0]], c["v"][1], c["v"][2], 0)
        got = (K.kvq_bits_per_value(kc, c["D"]) + K.kvq_bits_per_value(vc, c["D"])) / 2
        assert got == pytest.approx(c["bpv"]), c["cite"]


def test_constant_tables_match_the_oracle(K):
    np.testing.assert_array_equal(K.kvq_constant_table(0, 16), O.codec.nf4_levels().astype(np.float32))
    np.testing.assert_array_equal(K.kvq_constant_table(1, 15), O.codec.nf4_midpoints().astype(np.float32))
    for D in (64, 128, 256):
        c, s = O.rfft.twiddles(D)
        np.testing.assert_array_equal(K.kvq_constant_table(2, D // 2), c)
        np.testing.assert_array_equal(K.kvq_constant_table(3, D // 2), s)
    for P in (8, 16, 64, 256):
        c, s = O.rfft.directions(P)
        np.testing.assert_array_equal(K.kvq_constant_table(4, P), c)
        np.testing.assert_array_equal(K.kvq_constant_table(5, P), s)
        bc, bs = O.rfft.boundaries(P)
        np.testing.assert_array_equal(K.kvq_constant_table(6, P // 8), bc)
        np.testing.assert_array_equal(K.kvq_constant_table(7, P // 8), bs)
    for b in (2, 3, 4):
        np.testing.assert_array_equal(K.kvq_constant_table(6 + b, 2 ** b), O.lloyd_levels(b))


@pytest.mark.parametrize("which,n", [(0, 15), (1, 16), (2, 3), (2, 256), (4, 4), (4, 512), (6, 0), (8, 5), (10, 8),
                                     (11, 4), (-1, 4)])
def test_constant_table_rejects_bad_sizes(K, which, n):
    out = np.zeros(max(n, 1), dtype=np.float32)
    assert K._lib.kvq_constant_table(which, n, out.ctypes.data) == ERR_ARG


@pytest.mark.parametrize("codec,D,status", [
    ((1, 4, 96, 0, 0), 128, ERR_UNSUPPORTED),       # group not a power of two
    ((1, 4, 4, 0, 0), 128, ERR_UNSUPPORTED),        # group below 8
    ((1, 4, 256, 0, 0), 128, ERR_UNSUPPORTED),      # group above head_dim
    ((1, 1, 32, 0, 0), 128, ERR_UNSUPPORTED),       # 1-bit INT_ABSMAX
    ((2, 9, 32, 0, 0), 128, ERR_UNSUPPORTED),       # 9-bit INT_MINMAX
    ((1, 4, 32, 48, 0), 128, ERR_UNSUPPORTED),      # rotation width not a power of two
    ((1, 4, 32, 512, 0), 256, ERR_UNSUPPORTED),     # rotation wider than head_dim
    ((7, 4, 32, 0, 2), 128, ERR_UNSUPPORTED),       # polar rFFT with 4 phase sectors
    ((8, 4, 32, 64, 0), 128, ERR_UNSUPPORTED),      # rFFT codecs take no rotation
    ((11, 4, 32, 0, 0), 128, ERR_UNSUPPORTED),      # no such codebook
    ((9, 1, 32, 0, 0), 128, ERR_UNSUPPORTED),       # 1-bit INT_SYM
    ((9, 9, 32, 0, 0), 128, ERR_UNSUPPORTED),       # 9-bit INT_SYM
    ((10, 5, 32, 0, 0), 128, ERR_UNSUPPORTED),      # 5-bit LLOYD (tables for 2..4 bits)
    ((10, 1, 32, 0, 0), 128, ERR_UNSUPPORTED),      # 1-bit LLOYD
])
def test_layout_rejects_invalid_codecs(K, codec, D, status):
    c = K.kvq_codec(*codec)
    s = K.kvq_shape(1, 1, 1, 4, D)
    w, ns, nm = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert K._lib.kvq_packed_layout(ctypes.byref(s), ctypes.byref(c), ctypes.byref(w), ctypes.byref(ns),
                                    ctypes.byref(nm)) == status
    assert K._lib.kvq_bits_per_value(ctypes.byref(c), D) < 0


@pytest.mark.parametrize("shape,status", [
    ((1, 1, 1, 4, 96), ERR_UNSUPPORTED),   # head_dim must be 64, 128 or 256
    ((0, 1, 1, 4, 128), ERR_ARG),
    ((1, 1, 1, -1, 128), ERR_ARG),
])
def test_layout_rejects_invalid_shapes(K, shape, status):
    c = K.kvq_codec(1, 4, 32, 0, 0)
    s = K.kvq_shape(*shape)
    w, ns, nm = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert K._lib.kvq_packed_layout(ctypes.byref(s), ctypes.byref(c), ctypes.byref(w), ctypes.byref(ns),
                                    ctypes.byref(nm)) == status


def _packed(K, codec=(1, 4, 128, 256, 0), shape=(1, 2, 4, 64, 256), codes=FAKE, scales=FAKE, mins=None):
    return K.kvq_packed(K.kvq_codec(*codec), K.kvq_shape(*shape), codes, scales, mins, None)


def test_quantize_and_dequant_validate_before_launching(K):
    L = K._lib
    p = _packed(K)
    assert L.kvq_quantize_pack(None, ctypes.byref(p), None) == ERR_ARG
    assert L.kvq_quantize_pack(FAKE_ODD, ctypes.byref(p), None) == ERR_ALIGN
    assert L.kvq_dequant(ctypes.byref(p), None, None) == ERR_ARG
    assert L.kvq_dequant(ctypes.byref(p), FAKE_ODD, None) == ERR_ALIGN
    assert L.kvq_quantize_pack(FAKE, ctypes.byref(_packed(K, codes=FAKE_ODD)), None) == ERR_ALIGN
    assert L.kvq_quantize_pack(FAKE, ctypes.byref(_packed(K, codes=None)), None) == ERR_ARG
    assert L.kvq_quantize_pack(FAKE, ctypes.byref(_packed(K, scales=None)), None) == ERR_ARG
    # INT_MINMAX needs its mins array
    assert L.kvq_quantize_pack(FAKE, ctypes.byref(_packed(K, codec=(2, 4, 64, 0, 0))), None) == ERR_ARG
    assert L.kvq_quantize_pack(FAKE, None, None) == ERR_ARG
    # per-channel key calibration takes batch 1 only
    s2 = K.kvq_shape(2, 1, 1, 8, 128)
    assert L.kvq_calibrate_chan_scale(FAKE, ctypes.byref(s2), FAKE, None) == ERR_ARG


def _decode(K, k, v, q_heads=16, n_q=1, q=FAKE, out=FAKE, ws=FAKE, ws_bytes=None, path=0, sm=0.0, lse=None):
    if ws_bytes is None:
        ws_bytes = K._lib.kvq_decode_attn_workspace(ctypes.byref(k.shape), q_heads, n_q)
    return K._lib.kvq_decode_attn_ex(ctypes.byref(k), ctypes.byref(v), q_heads, n_q, q, None, sm, out, lse,
                                     ws, ws_bytes, path, None)


def test_decode_validates_before_launching(K):
    k = _packed(K)
    v = _packed(K, codec=(1, 2, 128, 0, 0))
    need = K._lib.kvq_decode_attn_workspace(ctypes.byref(k.shape), 16, 1)
    assert need > 0
    assert _decode(K, k, v, ws_bytes=need - 1) == ERR_WORKSPACE
    assert _decode(K, k, v, ws=None) == ERR_WORKSPACE
    assert _decode(K, k, v, q=None) == ERR_ARG
    assert _decode(K, k, v, q=FAKE_ODD) == ERR_ALIGN
    assert _decode(K, k, v, out=None) == ERR_ARG
    assert _decode(K, k, v, lse=FAKE_ODD) == ERR_ALIGN
    assert _decode(K, k, v, ws=FAKE_ODD) == ERR_ALIGN
    assert _decode(K, k, v, path=3) == ERR_ARG
    assert _decode(K, k, v, sm=-1.0) == ERR_ARG
    assert _decode(K, k, v, sm=float("nan")) == ERR_ARG
    assert _decode(K, k, v, q_heads=6) == ERR_UNSUPPORTED          # not a multiple of the 4 KV heads
    assert _decode(K, k, v, q_heads=36) == ERR_UNSUPPORTED         # 9 query heads per KV head
    assert _decode(K, k, v, n_q=0) == ERR_ARG
    # K and V must have the same shape; V may not use an rFFT codec
    v_other = _packed(K, codec=(1, 2, 128, 0, 0), shape=(1, 2, 4, 32, 256))
    assert _decode(K, k, v_other) == ERR_ARG
    v_rfft = _packed(K, codec=(7, 4, 32, 0, 8))
    assert _decode(K, k, v_rfft) == ERR_UNSUPPORTED


@pytest.mark.parametrize("case", ["tokens_below_32", "head_dim_128", "k_6bit", "v_5bit", "v_group_32",
                                  "k_minmax", "v_chan_scale", "g8", "v_lloyd_4bit", "d128_k_6bit_g64",
                                  "d128_k_cart_5bit", "d128_k_polar_6bit", "d128_k_6bit_rot64"])
def test_mfma_path_rejects_what_it_does_not_cover(K, case):
    kc, vc, shape, q_heads = (1, 4, 128, 256, 0), (1, 2, 128, 0, 0), (1, 2, 4, 64, 256), 16
    v_chan = None
    if case == "tokens_below_32":
        shape = (1, 2, 4, 20, 256)
    elif case == "head_dim_128":
        shape = (1, 2, 4, 64, 128)
        kc = (1, 4, 128, 128, 0)
    elif case == "k_6bit":
        kc = (1, 6, 128, 256, 0)
    elif case == "v_5bit":
        vc = (1, 5, 128, 0, 0)
    elif case == "v_lloyd_4bit":
        vc = (10, 4, 128, 0, 0)
    elif case.startswith("d128_"):
        # head_dim 128: 6-bit keys only at group 32 and rotation 0 or 128, rFFT keys only
        # 6+6-bit Cartesian or 5+7-bit polar at group 32
        shape = (1, 2, 4, 64, 128)
        vc = (1, 4, 64, 0, 0)
        kc = {"d128_k_6bit_g64": (1, 6, 64, 128, 0), "d128_k_cart_5bit": (8, 5, 32, 0, 0),
              "d128_k_polar_6bit": (7, 6, 32, 0, 7), "d128_k_6bit_rot64": (1, 6, 32, 64, 0)}[case]
    elif case == "v_group_32":
        vc = (1, 2, 32, 0, 0)
    elif case == "k_minmax":
        kc = (2, 4, 128, 0, 0)
    elif case == "v_chan_scale":
        v_chan = FAKE
    elif case == "g8":
        q_heads = 32
    k = _packed(K, codec=kc, shape=shape, mins=FAKE if kc[0] == 2 else None)
    v = _packed(K, codec=vc, shape=shape)
    if v_chan is not None:
        v.chan_scale = v_chan
    assert _decode(K, k, v, q_heads=q_heads, path=2) == ERR_UNSUPPORTED


def test_workspace_sizes_cover_the_decode_partials(K):
    # one fp32 partial of head_dim + 2 values per (row, query head, split) at least
    s = K.kvq_shape(1, 8, 4, 65536, 256)
    ws = K._lib.kvq_decode_attn_workspace(ctypes.byref(s), 16, 1)
    assert ws >= 8 * 16 * 2 * 258 * 4
    assert ws % 256 == 0 or ws > 0
    assert K._lib.kvq_decode_attn_workspace(ctypes.byref(s), 0, 1) == 0
    assert K._lib.kvq_attn_error_workspace(ctypes.byref(s), 16, 1) > 0


def test_key_mean_validates_before_launching(K):
    L = K._lib
    s = K.kvq_shape(2, 2, 4, 64, 128)
    need = L.kvq_key_mean_workspace(ctypes.byref(s))
    assert need == 8 * 2 * 4 * 128
    assert L.kvq_key_mean(None, ctypes.byref(s), FAKE, FAKE, need, None) == ERR_ARG
    assert L.kvq_key_mean(FAKE, ctypes.byref(s), None, FAKE, need, None) == ERR_ARG
    assert L.kvq_key_mean(FAKE, ctypes.byref(s), FAKE, FAKE, need - 1, None) == ERR_WORKSPACE
    assert L.kvq_key_mean(FAKE, ctypes.byref(s), FAKE, None, need, None) == ERR_WORKSPACE
    assert L.kvq_key_mean(FAKE_ODD, ctypes.byref(s), FAKE, FAKE, need, None) == ERR_ALIGN
    assert L.kvq_key_mean(FAKE, ctypes.byref(s), FAKE, FAKE_ODD, need, None) == ERR_ALIGN
    big = K.kvq_shape(2, 1, 1, 2 ** 22 + 1, 64)          # batch * tokens above 2^23
    assert L.kvq_key_mean(FAKE, ctypes.byref(big), FAKE, FAKE, 8 * 64, None) == ERR_ARG


def test_mean_field_is_validated(K):
    L = K._lib
    p = _packed(K)
    p.mean = FAKE_ODD
    assert L.kvq_quantize_pack(FAKE, ctypes.byref(p), None) == ERR_ALIGN
    p16 = _packed(K, codec=(0, 0, 0, 0, 0), scales=None)
    p16.mean = FAKE
    assert L.kvq_quantize_pack(FAKE, ctypes.byref(p16), None) == ERR_UNSUPPORTED
    k = _packed(K)
    k.mean = FAKE                                          # a key mean is fine for decode ...
    v = _packed(K, codec=(1, 2, 128, 0, 0))
    v.mean = FAKE                                          # ... a value mean is not
    assert _decode(K, k, v) == ERR_UNSUPPORTED


def _seg_pair(K, codec_k, codec_v, shape):
    k = K.kvq_packed(K.kvq_codec(*codec_k), K.kvq_shape(*shape), FAKE, FAKE if codec_k[0] else None, None, None)
    v = K.kvq_packed(K.kvq_codec(*codec_v), K.kvq_shape(*shape), FAKE, FAKE if codec_v[0] else None, None, None)
    return k, v


def _segs(K, parts):
    keep, arr = [], (K.kvq_segment * len(parts))()
    for i, (ck, cv, shape, l0, t0) in enumerate(parts):
        k, v = _seg_pair(K, ck, cv, shape)
        keep += [k, v]
        arr[i] = K.kvq_segment(ctypes.pointer(k), ctypes.pointer(v), l0, t0)
    return arr, keep


F16 = (0, 0, 0, 0, 0)
NF4 = (5, 4, 64, 0, 0)
I4 = (1, 4, 64, 0, 0)


def test_effective_bits_match_the_oracle(K):
    """Layer-0 fp16 anchors with NF4/int4 elsewhere, and prompt + decode anchors on two
    of four layers, against the oracle's accounting."""
    L = K._lib
    arr, keep = _segs(K, [(F16, F16, (1, 1, 4, 100, 128), 0, 0), (NF4, I4, (1, 25, 4, 100, 128), 1, 0)])
    e = L.kvq_effective_bits(arr, 2, 26, 4, 100)
    ref = O.effective_bits([(O.Codec(O.FP16), O.Codec(O.FP16), 0, 1, 0, 100),
                            (O.Codec(O.NF4, 4, 64), O.Codec(O.INT_ABSMAX, 4, 64), 1, 25, 0, 100)], 26, 100, 128)
    assert e == pytest.approx(ref, abs=1e-12) and round(e, 2) == 4.70
    parts = [(F16, F16, (1, 2, 4, 80, 128), 0, 0), (NF4, I4, (1, 2, 4, 176, 128), 0, 80),
             (NF4, I4, (1, 2, 4, 256, 128), 2, 0)]
    arr, keep = _segs(K, parts)
    ref = O.effective_bits([(O.Codec(O.FP16), O.Codec(O.FP16), 0, 2, 0, 80),
                            (O.Codec(O.NF4, 4, 64), O.Codec(O.INT_ABSMAX, 4, 64), 0, 2, 80, 176),
                            (O.Codec(O.NF4, 4, 64), O.Codec(O.INT_ABSMAX, 4, 64), 2, 2, 0, 256)], 4, 256, 128)
    assert L.kvq_effective_bits(arr, 3, 4, 4, 256) == pytest.approx(ref, abs=1e-12)


@pytest.mark.parametrize("case", ["gap", "overlap", "uncovered_layer", "past_end", "batch_mismatch", "zero_segments",
                                  "seventeen"])
def test_segments_reject_bad_tilings(K, case):
    L = K._lib
    sh = (1, 2, 4, 64, 128)
    parts = [(I4, I4, sh, 0, 0), (I4, I4, (1, 2, 4, 36, 128), 0, 64)]        # 2 layers x 100 tokens
    n, layers, tokens = 2, 2, 100
    if case == "gap":
        parts[1] = (I4, I4, (1, 2, 4, 30, 128), 0, 65)
        tokens = 95
    elif case == "overlap":
        parts[1] = (I4, I4, (1, 2, 4, 37, 128), 0, 63)
    elif case == "uncovered_layer":
        layers = 3
    elif case == "past_end":
        tokens = 90
    elif case == "batch_mismatch":
        parts[1] = (I4, I4, (2, 2, 4, 36, 128), 0, 64)
    elif case == "zero_segments":
        n = 0
    elif case == "seventeen":
        parts = [(I4, I4, (1, 2, 4, 4, 128), 0, 4 * i) for i in range(17)]
        n, tokens = 17, 68
    arr, keep = _segs(K, parts)
    assert L.kvq_effective_bits(arr, n, layers, 4, tokens) < 0
    st = L.kvq_decode_attn_segments(arr, n, layers, 4, tokens, 16, 1, FAKE, None, 0.0, FAKE, None, FAKE, 1 << 30,
                                    None)
    assert st == ERR_ARG


def test_segments_validate_before_launching(K):
    L = K._lib
    arr, keep = _segs(K, [(I4, I4, (1, 2, 4, 64, 128), 0, 0)])
    need = L.kvq_decode_attn_segments_workspace(arr, 1, 2, 4, 16, 1)
    assert need > 65536
    args = dict(q=FAKE, out=FAKE, ws=FAKE, wsb=need)

    def call(**kw):
        a = dict(args, **kw)
        return L.kvq_decode_attn_segments(arr, 1, 2, 4, 64, 16, 1, a["q"], None, 0.0, a["out"], None, a["ws"],
                                          a["wsb"], None)
    assert call(wsb=need - 1) == ERR_WORKSPACE
    assert call(ws=None) == ERR_WORKSPACE
    assert call(q=None) == ERR_ARG
    assert call(out=FAKE_ODD) == ERR_ALIGN


def test_append_validates_before_launching(K):
    L = K._lib
    p = _packed(K)                                         # 64 tokens
    assert L.kvq_quantize_pack_tokens(FAKE, 60, 5, ctypes.byref(p), None) == ERR_ARG
    assert L.kvq_quantize_pack_tokens(FAKE, -1, 2, ctypes.byref(p), None) == ERR_ARG
    assert L.kvq_quantize_pack_tokens(FAKE, 0, 0, ctypes.byref(p), None) == ERR_ARG
    assert L.kvq_quantize_pack_tokens(None, 0, 1, ctypes.byref(p), None) == ERR_ARG
    assert L.kvq_quantize_pack_tokens(FAKE_ODD, 0, 1, ctypes.byref(p), None) == ERR_ALIGN


def test_segments_reject_a_missing_head(K):
    L = K._lib
    parts = [(I4, I4, (1, 2, 1, 64, 128), 0, 0), (I4, I4, (1, 2, 2, 64, 128), 0, 0)]
    arr, keep = _segs(K, parts)
    arr[1].head0 = 2                                       # head 1 of 4 uncovered, head 3 too
    assert L.kvq_effective_bits(arr, 2, 2, 4, 64) < 0
    arr[1].head0 = 1
    parts.append((I4, I4, (1, 2, 1, 64, 128), 0, 0))
    arr2, keep2 = _segs(K, parts)
    arr2[1].head0, arr2[2].head0 = 1, 3
    assert L.kvq_effective_bits(arr2, 3, 2, 4, 64) == pytest.approx(4.25)


def test_segments_path_is_validated_before_launching(K):
    """kvq_decode_attn_segments_ex: a path outside 0..2 is an argument error, and the
    one-launch path refuses segments that are not whole-token tiles, or whose codec
    pair the mixed kernel does not compile, before any launch."""
    L = K._lib
    whole = [(I4, I4, (1, 1, 4, 100, 128), 0, 0), ((1, 3, 64, 0, 0), I4, (1, 1, 4, 100, 128), 1, 0)]
    arr, keep = _segs(K, whole)
    need = L.kvq_decode_attn_segments_workspace(arr, 2, 2, 4, 16, 1)
    assert need > 65536

    def call(a, n, tokens, path, wsb=need):
        return L.kvq_decode_attn_segments_ex(a, n, 2, 4, tokens, 16, 1, FAKE, None, 0.0, FAKE, None, FAKE, wsb, path,
                                             None)
    for bad in (-1, 3, 7):
        assert call(arr, 2, 100, bad) == ERR_ARG
    assert call(arr, 2, 100, 2, wsb=need - 1) == ERR_WORKSPACE
    ranges = [(I4, I4, (1, 2, 4, 64, 128), 0, 0), (I4, I4, (1, 2, 4, 36, 128), 0, 64)]   # token ranges
    arr2, keep2 = _segs(K, ranges)
    need2 = L.kvq_decode_attn_segments_workspace(arr2, 2, 2, 4, 16, 1)
    assert L.kvq_decode_attn_segments_ex(arr2, 2, 2, 4, 100, 16, 1, FAKE, None, 0.0, FAKE, None, FAKE, need2, 2,
                                         None) == ERR_UNSUPPORTED
    sym = [(I4, I4, (1, 1, 4, 100, 128), 0, 0), (I4, (9, 2, 64, 0, 0), (1, 1, 4, 100, 128), 1, 0)]
    arr3, keep3 = _segs(K, sym)                             # 4-bit keys, 2-bit symmetric values: not compiled
    need3 = L.kvq_decode_attn_segments_workspace(arr3, 2, 2, 4, 16, 1)
    assert L.kvq_decode_attn_segments_ex(arr3, 2, 2, 4, 100, 16, 1, FAKE, None, 0.0, FAKE, None, FAKE, need3, 2,
                                         None) == ERR_UNSUPPORTED


def test_one_launch_codec_map_respects_the_launch_grid(K):
    """Three one-layer tiles of 30,000 sequences each: every tile alone fits a launch
    grid, the whole map in one launch would not (90,000 rows), so path 2 is refused
    before anything is launched."""
    L = K._lib
    parts = [(I4, I4, (30000, 1, 4, 64, 128), l, 0) for l in range(3)]
    arr, keep = _segs(K, parts)
    need = L.kvq_decode_attn_segments_workspace(arr, 3, 3, 4, 16, 1)
    assert need > 0
    assert L.kvq_decode_attn_segments_ex(arr, 3, 3, 4, 64, 16, 1, FAKE, None, 0.0, FAKE, None, FAKE, need, 2,
                                         None) == ERR_UNSUPPORTED

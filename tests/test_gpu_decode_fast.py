"""GPU parity of the MFMA decode-attention kernel (2-, 3-, 4- or 5-bit keys, 2-, 3- or
4-bit affine values or 2-bit Lloyd-Max values, head_dim 256) against the CPU oracle,
and against the general kernel.

Bar: outputs within 2e-3 relative L2 per row, lse within 1e-4 absolute.  The
rotated query enters the int8 matrix cores as an integer (four 7-bit digits, the
fp32 query exactly) against the key codes as bytes, so QK is exact up to the
query's fp32 rotation; the P.V weights enter as fp16 (2^-11 relative per
weight), which sets the output error (a few 1e-4 at most).
"""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import announce, oracle_codec, to_dev, to_np
from tests.test_gpu_attn import _check_decode, _gpu_decode, _gpu_pack, _oracle

pytestmark = pytest.mark.gpu


def _case(K, w, kc, vc, kv_len=None, compare_general=True):
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    kp, vp = _gpu_pack(K, Kx, kc), _gpu_pack(K, Vx, vc)
    _, Kd, Vd = _oracle(Kx, Vx, oracle_codec(K, O, kc), oracle_codec(K, O, vc), q, kv_len)
    out, lse = _gpu_decode(K, kp, vp, q, kv_len, path=2)
    ref_out, ref_lse = O.decode_attn(q, Kd, Vd, kv_len)
    rel = _check_decode(out, lse, ref_out, ref_lse, kv_len, lse_tol=1e-4)
    if compare_general:
        out1, lse1 = _gpu_decode(K, kp, vp, q, kv_len, path=1)
        rel1 = np.linalg.norm(out1 - out, axis=-1) / np.maximum(np.linalg.norm(out1, axis=-1), 1e-30)
        assert rel1.max() < 2e-3
    return rel


def test_fast_c3_shape_shrunk():
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=2, T=2048, n_q=3)
    announce("mfma c3 shrunk")
    rel = _case(K, w, K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0))
    print(f"max rel err {rel:.2e}")


@pytest.mark.parametrize("variant", ["kgroup256", "vgroup64", "vgroup256", "rot128", "norot", "G2", "G1",
                                     "vrot", "vsym", "vsym_rot", "v4", "v4_g64", "v4_g256_k256", "v4_rot",
                                     "v4_sym", "v4_sym_rot", "v4_G1", "k3", "k5", "k3_v4", "k5_v4",
                                     "k5_v4_g64", "k3_kg256_rot128", "k5_norot_G2", "k3_v4_rot", "k2", "k2_v4",
                                     "k2_norot_G2", "k2_kg256_rot128", "k2_v4_rot", "vlloyd", "vlloyd_rot",
                                     "vlloyd_g64", "vlloyd_g256_k256", "vlloyd_k3_G1", "vlloyd_k2_rot128",
                                     "vlloyd_k5_G2", "v3", "v3_sym_rot", "v3_g64", "v3_g256_k2", "v3_k3_G1",
                                     "v3_sym_k5_G2", "vlloyd3", "vlloyd3_rot", "vlloyd3_g64", "vlloyd3_g256_k2",
                                     "vlloyd3_k3_G1", "vlloyd3_k5_G2"])
def test_fast_variants(variant):
    import kv_cache_bit_fwht_amd as K
    kc, vc = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    w = synth.get("c3", L=1, T=640, n_q=2)
    if variant == "kgroup256":
        kc = K.Codec(K.INT_ABSMAX, 4, 256, 256)
    elif variant == "vgroup64":
        vc = K.Codec(K.INT_ABSMAX, 2, 64, 0)
    elif variant == "vgroup256":
        vc = K.Codec(K.INT_ABSMAX, 2, 256, 0)
    elif variant == "rot128":
        kc = K.Codec(K.INT_ABSMAX, 4, 128, 128)
    elif variant == "norot":
        kc = K.Codec(K.INT_ABSMAX, 4, 128, 0)
    elif variant == "G2":
        w = w.with_sizes(Hq=8)
    elif variant == "G1":
        w = w.with_sizes(Hq=4)
    elif variant == "vrot":
        vc = K.Codec(K.INT_ABSMAX, 2, 128, 256)
    elif variant == "vsym":
        vc = K.Codec(K.INT_SYM, 2, 128, 0)
    elif variant == "vsym_rot":
        vc = K.Codec(K.INT_SYM, 2, 128, 256)
    elif variant == "v4":
        vc = K.Codec(K.INT_ABSMAX, 4, 128, 0)
    elif variant == "v4_g64":
        vc = K.Codec(K.INT_ABSMAX, 4, 64, 0)
    elif variant == "v4_g256_k256":
        kc, vc = K.Codec(K.INT_ABSMAX, 4, 256, 256), K.Codec(K.INT_ABSMAX, 4, 256, 0)
    elif variant == "v4_rot":
        vc = K.Codec(K.INT_ABSMAX, 4, 128, 256)
    elif variant == "v4_sym":
        vc = K.Codec(K.INT_SYM, 4, 128, 0)
    elif variant == "v4_sym_rot":
        vc = K.Codec(K.INT_SYM, 4, 64, 128)
    elif variant == "v4_G1":
        w = w.with_sizes(Hq=4)
        vc = K.Codec(K.INT_ABSMAX, 4, 128, 0)
    elif variant in ("k3", "k5"):
        kc = K.Codec(K.INT_ABSMAX, int(variant[1]), 128, 256)
    elif variant in ("k3_v4", "k5_v4"):
        kc, vc = K.Codec(K.INT_ABSMAX, int(variant[1]), 128, 256), K.Codec(K.INT_ABSMAX, 4, 128, 0)
    elif variant == "k5_v4_g64":
        kc, vc = K.Codec(K.INT_ABSMAX, 5, 128, 256), K.Codec(K.INT_ABSMAX, 4, 64, 0)
    elif variant == "k3_kg256_rot128":
        kc = K.Codec(K.INT_ABSMAX, 3, 256, 128)
    elif variant == "k5_norot_G2":
        w = w.with_sizes(Hq=8)
        kc = K.Codec(K.INT_ABSMAX, 5, 128, 0)
    elif variant == "k3_v4_rot":
        kc, vc = K.Codec(K.INT_ABSMAX, 3, 256, 256), K.Codec(K.INT_ABSMAX, 4, 128, 256)
    elif variant == "k2":
        kc = K.Codec(K.INT_ABSMAX, 2, 128, 256)
    elif variant == "k2_v4":
        kc, vc = K.Codec(K.INT_ABSMAX, 2, 128, 256), K.Codec(K.INT_ABSMAX, 4, 128, 0)
    elif variant == "k2_norot_G2":
        w = w.with_sizes(Hq=8)
        kc = K.Codec(K.INT_ABSMAX, 2, 128, 0)
    elif variant == "k2_kg256_rot128":
        kc = K.Codec(K.INT_ABSMAX, 2, 256, 128)
    elif variant == "k2_v4_rot":
        kc, vc = K.Codec(K.INT_ABSMAX, 2, 128, 256), K.Codec(K.INT_ABSMAX, 4, 64, 256)
    elif variant == "vlloyd":
        vc = K.Codec(K.LLOYD, 2, 128, 0)
    elif variant == "vlloyd_rot":
        vc = K.Codec(K.LLOYD, 2, 128, 256)
    elif variant == "vlloyd_g64":
        vc = K.Codec(K.LLOYD, 2, 64, 256)
    elif variant == "vlloyd_g256_k256":
        kc, vc = K.Codec(K.INT_ABSMAX, 4, 256, 256), K.Codec(K.LLOYD, 2, 256, 256)
    elif variant == "vlloyd_k3_G1":
        w = w.with_sizes(Hq=4)
        kc, vc = K.Codec(K.INT_ABSMAX, 3, 128, 256), K.Codec(K.LLOYD, 2, 128, 256)
    elif variant == "vlloyd_k2_rot128":
        kc, vc = K.Codec(K.INT_ABSMAX, 2, 128, 128), K.Codec(K.LLOYD, 2, 128, 128)
    elif variant == "vlloyd_k5_G2":
        w = w.with_sizes(Hq=8)
        kc, vc = K.Codec(K.INT_ABSMAX, 5, 128, 0), K.Codec(K.LLOYD, 2, 128, 0)
    elif variant == "v3":
        vc = K.Codec(K.INT_ABSMAX, 3, 128, 0)
    elif variant == "v3_sym_rot":
        vc = K.Codec(K.INT_SYM, 3, 128, 256)
    elif variant == "v3_g64":
        vc = K.Codec(K.INT_ABSMAX, 3, 64, 256)
    elif variant == "v3_g256_k2":
        kc, vc = K.Codec(K.INT_ABSMAX, 2, 256, 256), K.Codec(K.INT_SYM, 3, 256, 0)
    elif variant == "v3_k3_G1":
        w = w.with_sizes(Hq=4)
        kc, vc = K.Codec(K.INT_ABSMAX, 3, 128, 256), K.Codec(K.INT_ABSMAX, 3, 128, 0)
    elif variant == "v3_sym_k5_G2":
        w = w.with_sizes(Hq=8)
        kc, vc = K.Codec(K.INT_ABSMAX, 5, 128, 0), K.Codec(K.INT_SYM, 3, 64, 128)
    elif variant == "vlloyd3":
        vc = K.Codec(K.LLOYD, 3, 128, 0)
    elif variant == "vlloyd3_rot":
        vc = K.Codec(K.LLOYD, 3, 128, 256)
    elif variant == "vlloyd3_g64":
        vc = K.Codec(K.LLOYD, 3, 64, 256)
    elif variant == "vlloyd3_g256_k2":
        kc, vc = K.Codec(K.INT_ABSMAX, 2, 256, 256), K.Codec(K.LLOYD, 3, 256, 0)
    elif variant == "vlloyd3_k3_G1":
        w = w.with_sizes(Hq=4)
        kc, vc = K.Codec(K.INT_ABSMAX, 3, 128, 256), K.Codec(K.LLOYD, 3, 128, 256)
    elif variant == "vlloyd3_k5_G2":
        w = w.with_sizes(Hq=8)
        kc, vc = K.Codec(K.INT_ABSMAX, 5, 128, 0), K.Codec(K.LLOYD, 3, 64, 128)
    announce(f"mfma variant {variant}")
    _case(K, w, kc, vc)


def test_fast_causal_lengths():
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=1, T=1024, n_q=8)
    kv_len = np.array([[[0, 1, 31, 32, 33, 500, 1023, 1024]]], dtype=np.int32)
    announce("mfma causal lengths")
    _case(K, w, K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0), kv_len)


def test_fast_many_blocks_per_unit():
    """Few (row, KV head) units over 16K tokens: 32 blocks share each unit's chunk
    counter and the last of them merges the unit; causal lengths end chunks early."""
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=1, T=16384, n_q=2)
    kv_len = np.array([[[16384, 9000]]], dtype=np.int32)
    announce("mfma many blocks per unit")
    _case(K, w, K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0), kv_len)


@pytest.mark.parametrize("vb", [2, 3])
def test_fast_lloyd_values_many_blocks_and_lengths(vb):
    """2- and 3-bit Lloyd-Max values (rotated, [E22L] Result's next test): 32 blocks per
    unit on a counter, causal lengths ending mid-step."""
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=1, T=16384, n_q=3)
    kv_len = np.array([[[16384, 9001, 31]]], dtype=np.int32)
    announce(f"mfma {vb}-bit Lloyd-Max values, many blocks per unit")
    _case(K, w, K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.LLOYD, vb, 128, 256), kv_len)


def test_fast_3bit_values_many_blocks_and_lengths():
    """3-bit values (the symmetric grid, rotated: [E22L] Result's next test at 3 bits): 32
    blocks per unit on a counter, causal lengths ending mid-step."""
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=1, T=16384, n_q=3)
    kv_len = np.array([[[16384, 9001, 31]]], dtype=np.int32)
    announce("mfma 3-bit values, many blocks per unit")
    _case(K, w, K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_SYM, 3, 128, 256), kv_len)


def test_fast_4bit_values_many_blocks_and_lengths():
    """4-bit values: 32 blocks per unit on a counter, causal lengths ending mid-step."""
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=1, T=16384, n_q=3)
    kv_len = np.array([[[16384, 9001, 31]]], dtype=np.int32)
    announce("mfma 4-bit values, many blocks per unit")
    _case(K, w, K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 4, 128, 0), kv_len)


def test_fast_2_3_and_5_bit_keys_many_blocks_and_lengths():
    """2-, 3- and 5-bit keys (3 and 5: fields cut across word boundaries): 32 blocks per
    unit on a counter, causal lengths ending mid-step."""
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=1, T=16384, n_q=3)
    kv_len = np.array([[[16384, 9001, 31]]], dtype=np.int32)
    for kb in (2, 3, 5):
        announce(f"mfma {kb}-bit keys, many blocks per unit")
        _case(K, w, K.Codec(K.INT_ABSMAX, kb, 128, 256), K.Codec(K.INT_ABSMAX, 4, 128, 0), kv_len)


@pytest.mark.parametrize("T", [32, 33, 48, 100, 333, 1000])
def test_fast_token_counts_not_a_multiple_of_32(T):
    """The last step of a cache whose length is not a multiple of 32 reads the unit's last
    32 rows and masks the tokens before the step; with causal lengths too."""
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", B=2, L=1, T=T, n_q=3)
    kv_len = np.array([[[T, T - 1, 1]], [[max(T - 17, 0), 0, T // 2]]], dtype=np.int32)
    announce(f"mfma {T} tokens")
    _case(K, w, K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0), kv_len)
    _case(K, w, K.Codec(K.INT_ABSMAX, 3, 128, 256), K.Codec(K.INT_ABSMAX, 4, 128, 0), None)


def test_fast_static_chunks_many_rows():
    """More (query row, KV head) units than the workspace has counters for: blocks take
    fixed chunks and a separate kernel merges the partials."""
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=2, T=64, n_q=1030)             # 2 * 1030 * 4 = 8240 units
    announce("mfma static chunks, 8240 units")
    _case(K, w, K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0))


@pytest.mark.parametrize("kb", [2, 3, 4, 5])
@pytest.mark.parametrize("rot", [0, 256])
def test_fast_single_token_logits(kb, rot):
    """With one attended key the lse is that key's logit: the QK product on the int8
    matrix cores (query as an exact integer, codes as bytes) leaves only the query's
    rotation in fp32 and the final scaling, so single logits sit well inside the lse
    bar (3e-6 here; the fp16 matrix cores with fp16 subnormal codes left up to 2e-4)."""
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=1, T=640, n_q=8)
    kv_len = np.tile(np.array([1, 1, 2, 3, 5, 8, 1, 1], np.int32), (w.B, w.L, 1))
    kc, vc = K.Codec(K.INT_ABSMAX, kb, 128, rot), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    kp, vp = _gpu_pack(K, Kx, kc), _gpu_pack(K, Vx, vc)
    _, Kd, Vd = _oracle(Kx, Vx, oracle_codec(K, O, kc), oracle_codec(K, O, vc), q, kv_len)
    announce(f"mfma single-token logits kb={kb} rot={rot}")
    _, lse = _gpu_decode(K, kp, vp, q, kv_len, path=2)
    _, ref_lse = O.decode_attn(q, Kd, Vd, kv_len)
    err = np.abs(lse - ref_lse).max()
    print(f"max lse error {err:.2e}")
    assert err < 3e-6


def test_fast_rejects_unsupported_and_auto_falls_back():
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=1, T=20, n_q=1)                  # fewer than 32 tokens
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    kp = _gpu_pack(K, Kx, K.Codec(K.INT_ABSMAX, 4, 128, 256))
    vp = _gpu_pack(K, Vx, K.Codec(K.INT_ABSMAX, 2, 128, 0))
    announce("mfma unsupported shape")
    with pytest.raises(K.KvqError):
        _gpu_decode(K, kp, vp, q, None, path=2)
    out, _ = _gpu_decode(K, kp, vp, q, None, path=None)   # automatic: general kernel
    assert np.isfinite(out).all()


def test_fast_repeat_calls_agree_to_rounding():
    """The MFMA kernel hands steps out dynamically, so the order in which a block's
    wavefronts sum their tokens varies from call to call: repeated calls agree to fp32
    rounding, not bit for bit.  The calls share one workspace, whose counters each
    call must leave at zero (checked after the last call, and through the results)."""
    import torch
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=2, T=4096, n_q=2)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    announce("mfma repeat calls")
    kp = _gpu_pack(K, Kx, K.Codec(K.INT_ABSMAX, 4, 128, 256))
    vp = _gpu_pack(K, Vx, K.Codec(K.INT_ABSMAX, 2, 128, 0))
    wsb = K.kvq_decode_attn_workspace(kp.shape, w.Hq, w.n_q)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda:0")
    runs = [_gpu_decode(K, kp, vp, q, None, path=2, ws=ws) for _ in range(4)]
    for out, lse in runs[1:]:
        rel = np.linalg.norm(out - runs[0][0], axis=-1) / np.linalg.norm(runs[0][0], axis=-1)
        assert rel.max() < 1e-5
        assert np.abs(lse - runs[0][1]).max() < 1e-5
    assert int(ws[:65536].count_nonzero()) == 0
    _, Kd, Vd = _oracle(Kx, Vx, oracle_codec(K, O, K.Codec(K.INT_ABSMAX, 4, 128, 256)),
                        oracle_codec(K, O, K.Codec(K.INT_ABSMAX, 2, 128, 0)), q, None)
    ref_out, ref_lse = O.decode_attn(q, Kd, Vd, None)
    _check_decode(runs[-1][0], runs[-1][1], ref_out, ref_lse, None, lse_tol=1e-4)


def test_fast_full_size_64k_sampled():
    """The 64K-token decode workload at full size, one decode query per call as
    the benchmark times it, checked on sampled (layer, KV head) units."""
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3")
    announce("mfma full-size 64K")
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    kc, vc = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    kp, vp = _gpu_pack(K, Kx, kc), _gpu_pack(K, Vx, vc)
    okc, ovc = oracle_codec(K, O, kc), oracle_codec(K, O, vc)
    for i in (0, 137):
        qi = np.ascontiguousarray(q[:, :, i:i + 1])
        out, lse = _gpu_decode(K, kp, vp, qi, None)
        for (l, h) in ((0, 0), (5, 2), (7, 3)):
            ku = Kx[0, l, h][None, None, None]
            vu = Vx[0, l, h][None, None, None]
            wk, sk, zk = O.quantize_pack(ku, okc)
            wv, sv, zv = O.quantize_pack(vu, ovc)
            Kd = O.dequant(wk, sk, zk, okc, ku.shape)[0, 0, 0]
            Vd = O.dequant(wv, sv, zv, ovc, vu.shape)[0, 0, 0]
            G = w.Hq // w.H
            ro, rl, _ = O.attention.attend(qi[0, l, 0, h * G:(h + 1) * G].astype(np.float64), Kd, Vd, w.T,
                                           1.0 / 16.0)
            go = out[0, l, 0, h * G:(h + 1) * G].astype(np.float64)
            rel = np.linalg.norm(go - ro, axis=-1) / np.linalg.norm(ro, axis=-1)
            assert rel.max() < 2e-3, f"query {i} unit {(l, h)} rel {rel.max():.3g}"
            assert np.abs(lse[0, l, 0, h * G:(h + 1) * G] - rl).max() < 1e-4


# (tokens, key counts [layer][query], first unwritten token): tokens that are and are not
# a multiple of 32 (the MFMA kernel's last step then re-reads the unit's last 32 rows and
# masks those before its start), with a key count of T - 1 (only the last row unwritten)
DIRTY = [(352, [[300, 289], [1, 299]], 300), (333, [[332, 289], [1, 299]], 332),
         (333, [[300, 33], [1, 299]], 300), (1000, [[999, 640], [31, 977]], 999),
         (1000, [[700, 33], [32, 699]], 700)]


@pytest.mark.parametrize("vname", ["absmax2", "lloyd2", "sym3", "lloyd3"])
@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("T,lens,dirty_from", DIRTY)
def test_unwritten_rows_past_the_lengths_do_not_matter(path, T, lens, dirty_from, vname):
    """A cache filled by appends has rows past every query's key count that nothing has
    written: NaN scales and all-ones codes there leave the decode of keys [0, kv_len)
    as on a clean cache (MFMA kernel and general kernel)."""
    import torch
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", B=1, L=2, T=T, n_q=2)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    kc = K.Codec(K.INT_ABSMAX, 4, 128, 256)
    vc = {"absmax2": K.Codec(K.INT_ABSMAX, 2, 128, 0), "lloyd2": K.Codec(K.LLOYD, 2, 128, 256),
          "sym3": K.Codec(K.INT_SYM, 3, 128, 0), "lloyd3": K.Codec(K.LLOYD, 3, 128, 256)}[vname]
    kv_len = np.array([lens], dtype=np.int32)
    assert kv_len.max() <= dirty_from
    announce(f"unwritten rows past the lengths, path {path}, T={T}, from {dirty_from}, V {vname}")
    clean = (_gpu_pack(K, Kx, kc), _gpu_pack(K, Vx, vc))
    dirty = (_gpu_pack(K, Kx, kc), _gpu_pack(K, Vx, vc))
    B, L, H, T, D = Kx.shape
    t = torch.arange(B * L * H * T, device="cuda:0") % T
    for p in dirty:
        p.scales[t >= dirty_from] = 0x7E00              # fp16 NaN
        p.codes[t >= dirty_from] = -1                   # every code bit set
    torch.cuda.synchronize()
    o1, l1 = _gpu_decode(K, clean[0], clean[1], q, kv_len, path=path)
    o2, l2 = _gpu_decode(K, dirty[0], dirty[1], q, kv_len, path=path)
    assert np.isfinite(o2).all() and np.isfinite(l2).all()
    if path == 1:
        # the general kernel is bit-reproducible
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    else:
        # the MFMA kernel hands out steps dynamically: equal to fp32 rounding order
        rel = np.linalg.norm(o1 - o2, axis=-1) / np.linalg.norm(o1, axis=-1)
        assert rel.max() < 1e-5 and np.abs(l1 - l2).max() < 1e-5
    Kd = O.dequant(*O.quantize_pack(Kx, oracle_codec(K, O, kc)), oracle_codec(K, O, kc), Kx.shape)
    Vd = O.dequant(*O.quantize_pack(Vx, oracle_codec(K, O, vc)), oracle_codec(K, O, vc), Vx.shape)
    ref_out, ref_lse = O.decode_attn(q, Kd, Vd, kv_len)
    _check_decode(o2, l2, ref_out, ref_lse, kv_len)


@pytest.mark.parametrize("mult", [1.0e3, 1.4e4])
@pytest.mark.parametrize("rot", [0, 256])
def test_calibrated_channel_scales_with_large_channels(mult, rot):
    """Keys with 8 channels per head scaled so their absmax is about 4.5e3 or 6e4,
    channel scales calibrated on the same keys (arm C/D of [E21W] What I tested).  The
    query enters the key coordinates as q / c = q * absmax, up to ~2e5 and past the fp16
    range: the MFMA kernel normalises each head's query by a power of two before its
    fp16 operands, so the outputs stay within the 2e-3 bar of the oracle.  The logits
    reach ~1e3 here, so lse is held relative to its size: the MFMA kernel's unsigned
    codes fold their offset out as a query sum, so each logit is the difference of two
    fp32 sums about ten times its size, good to ~2e-5 of it (at ordinary logit sizes the
    other tests hold lse to 1e-4 absolute)."""
    import kv_cache_bit_fwht_amd as K
    B, L, H, T, D, Hq, nq = 1, 1, 2, 640, 256, 8, 2
    rng = np.random.default_rng([23, int(mult), rot])
    k = rng.standard_normal((B, L, H, T, D), dtype=np.float32)
    for h in range(H):
        k[:, :, h, :, rng.choice(D, 8, replace=False)] *= mult
    Kx = np.clip(k, -65000, 65000).astype(np.float16)
    Vx = rng.standard_normal((B, L, H, T, D), dtype=np.float32).astype(np.float16)
    q = rng.standard_normal((B, L, nq, Hq, D), dtype=np.float32).astype(np.float16)
    chan = O.calibrate_chan_scale(Kx[0])
    kc, vc = K.Codec(K.INT_ABSMAX, 4, 128, rot), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    announce(f"calibrated channel scales, channel mult {mult}, rot {rot}")
    kp, vp = _gpu_pack(K, Kx, kc, to_dev(chan)), _gpu_pack(K, Vx, vc)
    okc, ovc = oracle_codec(K, O, kc), oracle_codec(K, O, vc)
    wk, sk, zk = O.quantize_pack(Kx, okc, chan)
    wv, sv, zv = O.quantize_pack(Vx, ovc)
    ref_out, ref_lse = O.decode_attn(q, O.dequant(wk, sk, zk, okc, Kx.shape, chan), O.dequant(wv, sv, zv, ovc, Vx.shape),
                                     None)
    for path in (2, 1):
        out, lse = _gpu_decode(K, kp, vp, q, None, path=path)
        assert np.isfinite(out).all() and np.isfinite(lse).all(), f"path {path}"
        rel = np.linalg.norm(out - ref_out, axis=-1) / np.linalg.norm(ref_out, axis=-1)
        assert rel.max() < 2e-3, f"path {path} rel {rel.max():.3g}"
        err = np.abs(lse - ref_lse)
        assert np.all(err <= 1e-4 + 5e-5 * np.abs(ref_lse)), f"path {path} lse err {err.max():.3g}"

"""GPU parity of kvq_decode_attn and kvq_attn_error against the CPU oracle.

Bars (from the arithmetic): attention outputs within 2e-3 relative L2 per row,
KL within 1e-4 absolute, relative-error rows within 1e-4 absolute, per-unit K/V
squared-error sums within 1e-9 relative (same dequantised values, fp64 sums in a
different order), rFFT codes bit-exact.  Each workload is shrunk in tokens (and
layers/batch) so the oracle finishes in seconds while several 16-token tiles and
a ragged tail remain.
"""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import announce, oracle_codec, to_dev, to_np

pytestmark = pytest.mark.gpu

REL_OUT = 2e-3
KL_TOL = 1e-4


def _gpu_pack(K, x, codec, chan=None):
    B, L, H, T, D = x.shape
    p = K.alloc_packed(codec, K.Shape(B, L, H, T, D), chan_scale=chan)
    K.kvq_quantize_pack(to_dev(x), p)
    return p


def _gpu_decode(K, kp, vp, q, kv_len, path=None, ws=None, sm_scale=0.0):
    """One decode call; `ws` (a zero-filled device byte tensor) is reused when given."""
    import torch
    B, L, nq, Hq, D = q.shape
    out = torch.empty((B, L, nq, Hq, D), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, L, nq, Hq), dtype=torch.float32, device="cuda:0")
    wsb = K.kvq_decode_attn_workspace(kp.shape, Hq, nq)
    if ws is None:
        ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda:0")
    assert ws.numel() >= wsb
    kl = to_dev(kv_len) if kv_len is not None else None
    K.kvq_decode_attn(kp, vp, Hq, nq, to_dev(q), kl, sm_scale, out, lse, ws, wsb, path=path)
    torch.cuda.synchronize()
    return to_np(out), to_np(lse)


def _gpu_error(K, Kx, Vx, kp, vp, q, kv_len):
    import torch
    B, L, nq, Hq, D = q.shape
    H = Kx.shape[2]
    kl = torch.empty((B, L, nq, Hq), dtype=torch.float32, device="cuda:0")
    re = torch.empty_like(kl)
    kv = torch.empty((B, L, H, 4), dtype=torch.float64, device="cuda:0")
    wsb = K.kvq_attn_error_workspace(kp.shape, Hq, nq)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda:0")
    kvl = to_dev(kv_len) if kv_len is not None else None
    K.kvq_attn_error(to_dev(Kx), to_dev(Vx), kp, vp, Hq, nq, to_dev(q), kvl, 0.0, kl, re, kv, ws, wsb)
    torch.cuda.synchronize()
    return to_np(kl), to_np(re), to_np(kv)


def _oracle(Kx, Vx, kc, vc, q, kv_len, chan=None):
    wk, sk, zk = O.quantize_pack(Kx, kc, chan)
    wv, sv, zv = O.quantize_pack(Vx, vc)
    Kd = O.dequant(wk, sk, zk, kc, Kx.shape, chan)
    Vd = O.dequant(wv, sv, zv, vc, Vx.shape)
    return (wk, sk, zk), Kd, Vd


def _check_decode(out, lse, ref_out, ref_lse, kv_len, lse_tol=1e-4):
    num = np.linalg.norm(out.astype(np.float64) - ref_out, axis=-1)
    den = np.linalg.norm(ref_out, axis=-1)
    empty = den == 0
    rel = np.where(empty, num, num / np.where(empty, 1, den))
    assert rel.max() < REL_OUT, f"max rel err {rel.max():.3g}"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - ref_lse[fin]).max(initial=0) < lse_tol
    return rel.max()


def _run_case(K, Kx, Vx, q, kv_len, kcodec, vcodec, chan=None, check_error=True, path=None):
    okc, ovc = oracle_codec(K, O, kcodec), oracle_codec(K, O, vcodec)
    chan_d = to_dev(chan) if chan is not None else None
    kp = _gpu_pack(K, Kx, kcodec, chan_d)
    vp = _gpu_pack(K, Vx, vcodec)
    (wk, sk, zk), Kd, Vd = _oracle(Kx, Vx, okc, ovc, q, kv_len, chan)
    assert np.array_equal(to_np(kp.codes, np.uint32), wk), "K codes differ from the oracle"
    out, lse = _gpu_decode(K, kp, vp, q, kv_len, path)
    ref_out, ref_lse = O.decode_attn(q, Kd, Vd, kv_len)
    rel = _check_decode(out, lse, ref_out, ref_lse, kv_len)
    if not check_error:
        return rel
    kl, re, kv = _gpu_error(K, Kx, Vx, kp, vp, q, kv_len)
    rkl, rre, rkv = O.attn_error(q, Kx, Vx, Kd, Vd, kv_len)
    assert np.abs(kl - rkl).max() < KL_TOL, f"KL diff {np.abs(kl - rkl).max():.3g}"
    assert np.abs(re - rre).max() < 1e-4, f"relerr diff {np.abs(re - rre).max():.3g}"
    assert np.allclose(kv, rkv, rtol=1e-9, atol=1e-12), "kv_err differs"
    return rel


# ------------------------------------------------------------------ the five workloads (shrunk)

def test_c1_tiny_reference_full_size():
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c1")
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w, Kx)
    c = K.Codec(K.INT_MINMAX, 4, 32, 0)
    announce("c1 minmax4 g32 decode+error")
    _run_case(K, Kx, Vx, q, kv_len, c, c)


@pytest.mark.parametrize("arm", ["A", "B", "C", "D"])
@pytest.mark.parametrize("bits", [3, 4])
def test_c2_proxy_probe_arms(arm, bits):
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c2", L=2, T=700, pos_range=(350, 700), n_q=12)
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w, Kx)
    chan = None
    if arm == "A":
        kc = vc = K.Codec(K.INT_MINMAX, bits, 32, 0)
    elif arm == "B":
        kc = vc = K.Codec(K.INT_ABSMAX, bits, 32, 256)
    elif arm == "C":
        kc = vc = K.Codec(K.INT_MINMAX, bits, 32, 0)
        chan = O.calibrate_chan_scale(Kx[0])
    else:
        kc = vc = K.Codec(K.INT_ABSMAX, bits, 32, 256)
        chan = O.calibrate_chan_scale(Kx[0])
    announce(f"c2 arm {arm} bits {bits}")
    _run_case(K, Kx[1:], Vx[1:], q[1:], kv_len[1:], kc, vc, chan)


def test_c3_shape_generic_kernel():
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=2, T=1000, n_q=3)
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w)
    announce("c3 shrunk, general kernel")
    _run_case(K, Kx, Vx, q, None, K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0), path=1)


@pytest.mark.parametrize("arm", ["ternary", "sign", "nf4_int4", "int8"])
def test_c4_low_bit_arms_with_fp16_anchor(arm):
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c4", B=2, L=3, H=2, Hq=8, T=500, n_q=3)
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w)
    if arm == "ternary":
        kc = vc = K.Codec(K.TERNARY, 2, 8, 0)
    elif arm == "sign":
        kc = vc = K.Codec(K.SIGN, 1, 8, 0)
    elif arm == "nf4_int4":
        kc, vc = K.Codec(K.NF4, 4, 64, 0), K.Codec(K.INT_ABSMAX, 4, 64, 0)
    else:
        kc = vc = K.Codec(K.INT8_SYM, 8, 128, 0)
    announce(f"c4 {arm}")
    # layer 0: fp16 anchor (identity codec) ; layers 1..: the arm
    A = lambda x: np.ascontiguousarray(x[:, :1])
    R = lambda x: np.ascontiguousarray(x[:, 1:])
    f = K.Codec(K.FP16)
    _run_case(K, A(Kx), A(Vx), A(q), None, f, f)
    _run_case(K, R(Kx), R(Vx), R(q), None, kc, vc)


@pytest.mark.parametrize("arm", ["sym2", "sym2_rot", "lloyd2_rot", "lloyd3_rot", "sym3_rot"])
def test_c3_value_codebooks_decode_and_error(arm):
    """Rotated 4-bit keys with the value grids the 64K experiment names as its next
    test: the symmetric grid and Gaussian Lloyd-Max levels, rotated or not."""
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=2, T=700, n_q=3)
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w)
    kc = K.Codec(K.INT_ABSMAX, 4, 128, 256)
    vc = {"sym2": K.Codec(K.INT_SYM, 2, 128, 0), "sym2_rot": K.Codec(K.INT_SYM, 2, 128, 256),
          "lloyd2_rot": K.Codec(K.LLOYD, 2, 128, 256), "lloyd3_rot": K.Codec(K.LLOYD, 3, 128, 256),
          "sym3_rot": K.Codec(K.INT_SYM, 3, 128, 256)}[arm]
    announce(f"c3 values {arm}")
    _run_case(K, Kx, Vx, q, None, kc, vc)


@pytest.mark.parametrize("arm", ["map_pair", "map_pair_rot_v", "runtime"])
def test_single_codec_routes_of_the_general_kernel(arm):
    """Codec pairs without an instance of their own: one the codec-map kernel compiles
    (decoded as a one-tile map) and one it does not (the runtime-codec instance)."""
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", B=2, L=2, T=610, n_q=2)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    kv_len = np.random.default_rng(41).integers(0, 611, (2, 2, 2)).astype(np.int32)
    if arm == "map_pair":
        kc, vc = K.Codec(K.INT_ABSMAX, 2, 64, 256), K.Codec(K.INT_ABSMAX, 3, 32, 0)
    elif arm == "map_pair_rot_v":
        kc, vc = K.Codec(K.INT_ABSMAX, 6, 128, 0), K.Codec(K.INT_ABSMAX, 2, 128, 256)
    else:
        kc, vc = K.Codec(K.INT_MINMAX, 4, 32, 0), K.Codec(K.INT_SYM, 3, 64, 0)
    announce(f"single codec route {arm}")
    _run_case(K, Kx, Vx, q, kv_len, kc, vc, path=1)


@pytest.mark.parametrize("G,n_q", [(1, 5), (1, 4), (2, 3), (2, 1), (1, 1)])
def test_general_kernel_packs_query_rows(G, n_q):
    """With one or two query heads per KV head, the general kernel's four query slots
    take the heads of several query rows (a group of rows may be partly filled); each
    row keeps its own key count, including none."""
    import kv_cache_bit_fwht_amd as K
    H = 3
    w = synth.get("c3", B=2, L=2, H=H, Hq=G * H, T=333, n_q=n_q)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    kv_len = np.random.default_rng(51 + G * 10 + n_q).integers(0, 334, (2, 2, n_q)).astype(np.int32)
    kv_len[0, 0, 0] = 0
    kv_len[1, 1, -1] = 333
    announce(f"general kernel, {G} query heads per KV head, {n_q} query rows")
    for kc, vc in ((K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)),
                   (K.Codec(K.TERNARY, 2, 8, 0), K.Codec(K.TERNARY, 2, 8, 0))):
        _run_case(K, Kx, Vx, q, kv_len, kc, vc, check_error=False, path=1)


@pytest.mark.parametrize("arm", ["polar", "cart", "fwht6"])
def test_c5_transform_arms(arm):
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c5", B=2, L=2, H=2, Hq=8, T=400, n_q=2)
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w)
    if arm == "polar":
        kc = K.Codec(K.RFFT_POLAR, 5, 32, 0, 7)
    elif arm == "cart":
        kc = K.Codec(K.RFFT_CART, 6, 32, 0)
    else:
        kc = K.Codec(K.INT_ABSMAX, 6, 32, 128)
    announce(f"c5 {arm}")
    _run_case(K, Kx, Vx, q, None, kc, K.Codec(K.FP16))


@pytest.mark.parametrize("spec", [(K_, D) for K_ in ("polar", "cart") for D in (64, 128, 256)])
def test_rfft_codecs_bit_exact_and_dequant(spec):
    import kv_cache_bit_fwht_amd as K
    import torch
    kind, D = spec
    rng = np.random.default_rng([5, D])
    x = rng.standard_normal((1, 2, 2, 41, D), dtype=np.float32)
    x[0, 0, 0, 0] = 0.0
    x[0, 0, 0, 1] = 1.0
    x = x.astype(np.float16)
    if kind == "polar":
        c = K.Codec(K.RFFT_POLAR, 5, 32, 0, 7) if D != 256 else K.Codec(K.RFFT_POLAR, 4, 16, 0, 8)
    else:
        c = K.Codec(K.RFFT_CART, 6, 32, 0) if D != 64 else K.Codec(K.RFFT_CART, 8, 8, 0)
    announce(f"rfft {kind} D={D}")
    p = _gpu_pack(K, x, c)
    xh = torch.empty(x.shape, dtype=torch.float32, device="cuda:0")
    K.kvq_dequant(p, xh)
    torch.cuda.synchronize()
    oc = oracle_codec(K, O, c)
    w, s, z = O.quantize_pack(x, oc)
    assert np.array_equal(to_np(p.codes, np.uint32), w)
    assert np.array_equal(to_np(p.scales, np.uint16), s.view(np.uint16))
    ref = O.dequant(w, s, z, oc, x.shape)
    assert np.array_equal(to_np(xh), ref), f"max diff {np.abs(to_np(xh) - ref).max()}"


# ------------------------------------------------------------------ edge cases

def test_causal_lengths_zero_one_full_and_ragged():
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=1, T=77, n_q=5)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    kv_len = np.array([[[0, 1, 16, 17, 77]]], dtype=np.int32)
    announce("edge causal lengths")
    kc, vc = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    okc, ovc = oracle_codec(K, O, kc), oracle_codec(K, O, vc)
    kp, vp = _gpu_pack(K, Kx, kc), _gpu_pack(K, Vx, vc)
    _, Kd, Vd = _oracle(Kx, Vx, okc, ovc, q, kv_len)
    for path in (None, 1):
        out, lse = _gpu_decode(K, kp, vp, q, kv_len, path)
        ref_out, ref_lse = O.decode_attn(q, Kd, Vd, kv_len)
        assert np.all(out[0, 0, 0] == 0) and np.all(np.isneginf(lse[0, 0, 0]))
        _check_decode(out, lse, ref_out, ref_lse, kv_len)
    kl, re, kv = _gpu_error(K, Kx, Vx, kp, vp, q, kv_len)
    rkl, rre, _ = O.attn_error(q, Kx, Vx, Kd, Vd, kv_len)
    assert np.abs(kl - rkl).max() < KL_TOL and np.abs(re - rre).max() < 1e-4


def test_fp16_cache_has_zero_error_and_kl():
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c4", B=1, L=1, H=2, Hq=8, T=100, n_q=2)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    announce("fp16 identity error")
    f = K.Codec(K.FP16)
    kp, vp = _gpu_pack(K, Kx, f), _gpu_pack(K, Vx, f)
    kl, re, kv = _gpu_error(K, Kx, Vx, kp, vp, q, None)
    assert np.abs(kl).max() < 1e-6 and np.abs(re).max() == 0.0
    assert np.all(kv[..., 0] == 0) and np.all(kv[..., 2] == 0)


def test_general_decode_is_deterministic():
    """The general kernel's summation order is fixed: repeated calls agree bit for bit."""
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=1, T=3000, n_q=1)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    announce("determinism")
    kp = _gpu_pack(K, Kx, K.Codec(K.INT_ABSMAX, 4, 128, 256))
    vp = _gpu_pack(K, Vx, K.Codec(K.INT_ABSMAX, 2, 128, 0))
    a, la = _gpu_decode(K, kp, vp, q, None, path=1)
    b, lb = _gpu_decode(K, kp, vp, q, None, path=1)
    assert a.tobytes() == b.tobytes() and la.tobytes() == lb.tobytes()

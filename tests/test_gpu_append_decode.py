"""GPU parity of kvq_append_decode_attn ([FMAG-6] The winning recipe: each decode step
writes its token's K and V into the quantised cache, then attends over it) against the
oracle: an append-then-decode loop over a cache whose rows past the written tokens hold
garbage (NaN scales, all-ones codes), on the one-launch route (4-bit keys, the MFMA
decode codes the new rows itself) and on the two-launch fallback.

Per step: the new rows' codes and scales are bit-exact to the oracle's, rows outside
the window keep their contents, and the decode output is within 2e-3 relative L2 (lse
1e-4) of the oracle's attention over the oracle's cache."""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import announce, oracle_codec, to_dev, to_np
from tests.test_gpu_attn import _check_decode

pytestmark = pytest.mark.gpu


def _setup(K, kc, vc, T, P, n_q=1, L=2, Hq=16):
    import torch
    w = synth.get("c3", B=1, L=L, T=T, n_q=n_q, Hq=Hq)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    kp, vp = K.alloc_packed(kc, shape), K.alloc_packed(vc, shape)
    for p in (kp, vp):
        p.codes.fill_(-1)                               # every code bit set
        p.scales.fill_(0x7E00)                          # fp16 NaN
    # tokens [0, P) written before the loop
    K.kvq_quantize_pack_tokens_kv(to_dev(np.ascontiguousarray(Kx[:, :, :, :P])),
                                  to_dev(np.ascontiguousarray(Vx[:, :, :, :P])), 0, P, kp, vp)
    torch.cuda.synchronize()
    okc, ovc = oracle_codec(K, O, kc), oracle_codec(K, O, vc)
    wk, sk, zk = O.quantize_pack(Kx, okc)
    wv, sv, zv = O.quantize_pack(Vx, ovc)
    ref = dict(wk=wk, sk=sk, wv=wv, sv=sv, Kd=O.dequant(wk, sk, zk, okc, Kx.shape),
               Vd=O.dequant(wv, sv, zv, ovc, Vx.shape))
    return w, Kx, Vx, q, shape, kp, vp, ref


def _step(K, w, Kx, Vx, q, shape, kp, vp, ref, t0, n, kv_len):
    import torch
    B, L, H, T, D, Hq = w.B, w.L, w.H, w.T, w.D, w.Hq
    nq = q.shape[2]
    kn = to_dev(np.ascontiguousarray(Kx[:, :, :, t0:t0 + n]))
    vn = to_dev(np.ascontiguousarray(Vx[:, :, :, t0:t0 + n]))
    out = torch.empty((B, L, nq, Hq, D), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, L, nq, Hq), dtype=torch.float32, device="cuda:0")
    wsb = K.kvq_decode_attn_workspace(shape, Hq, nq)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda:0")
    before_k = to_np(kp.codes, np.uint32).copy()
    K.kvq_append_decode_attn(kn, vn, t0, n, kp, vp, Hq, nq, to_dev(q), to_dev(kv_len), 0.0, out, lse, ws, wsb)
    torch.cuda.synchronize()
    rows = np.zeros((B, L, H, T), bool)
    rows[:, :, :, t0:t0 + n] = True
    rows = rows.ravel()
    kc_now = to_np(kp.codes, np.uint32)
    assert np.array_equal(kc_now[rows], ref["wk"][rows]), "new key codes"
    assert np.array_equal(to_np(kp.scales, np.uint16)[rows], ref["sk"].view(np.uint16)[rows]), "new key scales"
    assert np.array_equal(to_np(vp.codes, np.uint32)[rows], ref["wv"][rows]), "new value codes"
    assert np.array_equal(to_np(vp.scales, np.uint16)[rows], ref["sv"].view(np.uint16)[rows]), "new value scales"
    assert np.array_equal(kc_now[~rows], before_k[~rows]), "rows outside the window changed"
    assert np.all(to_np(ws[:65536]) == 0), "counters left non-zero"
    ref_out, ref_lse = O.decode_attn(q, ref["Kd"], ref["Vd"], kv_len)
    _check_decode(to_np(out), to_np(lse), ref_out, ref_lse, kv_len)


FUSED = ((1, 4, 128, 256), (1, 2, 128, 0))


@pytest.mark.parametrize("kspec,vspec", [FUSED, ((1, 4, 256, 0), (1, 4, 64, 256)),
                                         # fallback routes: 3-bit keys, symmetric-grid values
                                         ((1, 3, 128, 256), (1, 2, 128, 0)), ((1, 4, 128, 256), (9, 2, 128, 0))])
def test_append_then_decode_loop(kspec, vspec):
    """T = 1000 (not a multiple of 32), tokens [0, 980) present; 10 single-token steps
    crossing the step boundary at token 992, each query attending every written token."""
    import kv_cache_bit_fwht_amd as K
    kc, vc = K.Codec(*kspec), K.Codec(*vspec)
    T, P = 1000, 980
    w, Kx, Vx, q, shape, kp, vp, ref = _setup(K, kc, vc, T, P)
    for t in range(P, P + 10):
        announce(f"append+decode K={kc} V={vc} token {t}")
        kv_len = np.full((w.B, w.L, q.shape[2]), t + 1, np.int32)
        _step(K, w, Kx, Vx, q, shape, kp, vp, ref, t, 1, kv_len)


@pytest.mark.parametrize("t0,n", [(985, 3), (988, 8), (992, 8), (968, 1)])
def test_append_windows_and_lengths(t0, n):
    """Windows of up to 8 tokens, across a step boundary; two queries per row, one
    attending through the window, one stopping inside it (and for t0 = 968 one before it:
    the new rows are written but not attended)."""
    import kv_cache_bit_fwht_amd as K
    kc, vc = K.Codec(*FUSED[0]), K.Codec(*FUSED[1])
    w, Kx, Vx, q, shape, kp, vp, ref = _setup(K, kc, vc, 1000, t0, n_q=2)
    kv_len = np.array([[[t0 + n, t0 + (n + 1) // 2], [t0 + n, max(t0 - 5, 1)]]], np.int32)
    announce(f"append window t0={t0} n={n}")
    _step(K, w, Kx, Vx, q, shape, kp, vp, ref, t0, n, kv_len)


def test_append_decode_64k_shape():
    """The 64K workload's shape (8 x 4 x 65,536 x 256, Hq 16) with its last token
    appended by the one-launch route; sampled units against the oracle."""
    import torch
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", n_q=1)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    B, L, H, T, D, Hq = w.B, w.L, w.H, w.T, w.D, w.Hq
    kc, vc = K.Codec(*FUSED[0]), K.Codec(*FUSED[1])
    shape = K.Shape(B, L, H, T, D)
    kp, vp = K.alloc_packed(kc, shape), K.alloc_packed(vc, shape)
    kd, vd = to_dev(Kx), to_dev(Vx)
    K.kvq_quantize_pack_kv(kd, vd, kp, vp)
    t = T - 1
    for p in (kp, vp):                                 # the last token not written yet
        rows = torch.arange(B * L * H * T, device="cuda:0") % T == t
        p.codes[rows] = -1
        p.scales[rows] = 0x7E00
    out = torch.empty((B, L, 1, Hq, D), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, L, 1, Hq), dtype=torch.float32, device="cuda:0")
    wsb = K.kvq_decode_attn_workspace(shape, Hq, 1)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda:0")
    announce("append+decode at 64K")
    K.kvq_append_decode_attn(kd[:, :, :, t:t + 1].contiguous(), vd[:, :, :, t:t + 1].contiguous(), t, 1, kp, vp,
                             Hq, 1, to_dev(q[:, :, :1]), None, 0.0, out, lse, ws, wsb)
    torch.cuda.synchronize()
    G = Hq // H
    okc, ovc = oracle_codec(K, O, kc), oracle_codec(K, O, vc)
    for (l, h) in [(0, 0), (7, 3)]:
        ku, vu = Kx[0, l, h][None, None, None], Vx[0, l, h][None, None, None]
        wk, sk, zk = O.quantize_pack(ku, okc)
        wv, sv, zv = O.quantize_pack(vu, ovc)
        unit = slice((l * H + h) * T, (l * H + h + 1) * T)
        assert np.array_equal(to_np(kp.codes[unit], np.uint32), wk)
        assert np.array_equal(to_np(vp.codes[unit], np.uint32), wv)
        Kd, Vd = O.dequant(wk, sk, zk, okc, ku.shape)[0, 0, 0], O.dequant(wv, sv, zv, ovc, vu.shape)[0, 0, 0]
        ro, rl, _ = O.attention.attend(q[0, l, 0, h * G:(h + 1) * G].astype(np.float64), Kd, Vd, T, 1.0 / 16.0)
        go = to_np(out)[0, l, 0, h * G:(h + 1) * G].astype(np.float64)
        assert (np.linalg.norm(go - ro, axis=-1) / np.linalg.norm(ro, axis=-1)).max() < 2e-3
        assert np.abs(to_np(lse)[0, l, 0, h * G:(h + 1) * G] - rl).max() < 1e-4


def test_append_decode_invalid_arguments_write_nothing():
    import torch
    import kv_cache_bit_fwht_amd as K
    shape = K.Shape(1, 1, 2, 64, 256)
    kc, vc = K.Codec(*FUSED[0]), K.Codec(*FUSED[1])
    kp, vp = K.alloc_packed(kc, shape), K.alloc_packed(vc, shape)
    kp.codes.fill_(-1)
    new = to_dev(np.zeros((1, 1, 2, 2, 256), np.float16))
    q = to_dev(np.zeros((1, 1, 1, 8, 256), np.float16))
    out = torch.full((1, 1, 1, 8, 256), -7.0, dtype=torch.float32, device="cuda:0")
    wsb = K.kvq_decode_attn_workspace(shape, 8, 1)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda:0")
    announce("append+decode invalid arguments")
    with pytest.raises(K.KvqError):                   # window past the end
        K.kvq_append_decode_attn(new, new, 63, 2, kp, vp, 8, 1, q, None, 0.0, out, None, ws, wsb)
    with pytest.raises(K.KvqError):                   # workspace too small
        K.kvq_append_decode_attn(new, new, 10, 2, kp, vp, 8, 1, q, None, 0.0, out, None, ws, wsb - 1024)
    torch.cuda.synchronize()
    assert bool((kp.codes == -1).all()) and bool((out == -7.0).all())

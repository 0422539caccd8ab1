"""The allocation-free decode entry point, kvq_decode_attn_static, against
kvq_decode_attn with a caller workspace (both through the C ABI), on calls in a
row: a 64K-style MFMA-path cache, then two smaller head_dim-128 caches (NF4 keys; rFFT
keys, whose query spectra share the scratch), then the first size again (the shared
device scratch must have been left ready).  Also checks the
size limit, which is enforced before anything is launched."""
import numpy as np
import pytest

import oracle as O
from tests.gpu_util import announce, oracle_codec, to_dev, to_np

pytestmark = pytest.mark.gpu


def _cache(K, dims, kc, vc, n_q, Hq, seed):
    import torch
    B, L, H, T, D = dims
    rng = np.random.default_rng([seed, T, D])
    k = rng.standard_normal((B, L, H, T, D), dtype=np.float32)
    k[..., rng.choice(D, 8, replace=False)] *= 10.0
    k = k.astype(np.float16)
    v = rng.standard_normal((B, L, H, T, D), dtype=np.float32).astype(np.float16)
    q = rng.standard_normal((B, L, n_q, Hq, D), dtype=np.float32).astype(np.float16)
    kv_len = rng.integers(max(T // 2, 1), T + 1, (B, L, n_q)).astype(np.int32)
    kv_len[0, 0, 0] = T
    shape = K.Shape(B, L, H, T, D)
    kp, vp = K.alloc_packed(kc, shape), K.alloc_packed(vc, shape)
    K.kvq_quantize_pack_kv(to_dev(k), to_dev(v), kp, vp)
    torch.cuda.synchronize()
    return k, v, q, kv_len, shape, kp, vp


def _both(K, kp, vp, shape, q, kv_len, Hq, n_q):
    import torch
    B, L, D = shape.batch, shape.layers, shape.head_dim
    qd, kl = to_dev(q), to_dev(kv_len)
    out_s = torch.full((B, L, n_q, Hq, D), float("nan"), dtype=torch.float32, device="cuda:0")
    lse_s = torch.full((B, L, n_q, Hq), float("nan"), dtype=torch.float32, device="cuda:0")
    out_w, lse_w = torch.empty_like(out_s), torch.empty_like(lse_s)
    K.kvq_decode_attn_static(kp, vp, Hq, n_q, qd, kl, 0.0, out_s, lse_s)
    wsb = K.kvq_decode_attn_workspace(shape, Hq, n_q)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda:0")
    K.kvq_decode_attn(kp, vp, Hq, n_q, qd, kl, 0.0, out_w, lse_w, ws, wsb)
    torch.cuda.synchronize()
    return to_np(out_s), to_np(lse_s), to_np(out_w), to_np(lse_w)


def _oracle(K, k, v, q, kv_len, kc, vc):
    okc, ovc = oracle_codec(K, O, kc), oracle_codec(K, O, vc)
    wk, sk, zk = O.quantize_pack(k, okc)
    wv, sv, zv = O.quantize_pack(v, ovc)
    Kd = O.dequant(wk, sk, zk, okc, k.shape)
    Vd = O.dequant(wv, sv, zv, ovc, v.shape)
    return O.decode_attn(q, Kd, Vd, kv_len)


def _rel(a, b):
    return np.linalg.norm(a - b, axis=-1) / np.linalg.norm(b, axis=-1)


def test_static_decode_matches_workspace_decode_on_consecutive_calls():
    import kv_cache_bit_fwht_amd as K
    big = ((1, 2, 4, 1000, 256), K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0), 16, 2)
    small = ((1, 1, 2, 300, 128), K.Codec(K.NF4, 4, 64, 0), K.Codec(K.INT_ABSMAX, 4, 64, 0), 4, 1)
    # rFFT keys keep their query spectra in the scratch after the partials
    spec = ((2, 1, 2, 700, 128), K.Codec(K.RFFT_CART, 6, 32, 0), K.Codec(K.INT_ABSMAX, 4, 64, 0), 8, 2)
    for step, (dims, kc, vc, Hq, n_q) in enumerate((big, small, spec, big)):
        announce(f"kvq_decode_attn_static call {step}: dims={dims} K={kc} V={vc} Hq={Hq} n_q={n_q}")
        k, v, q, kv_len, shape, kp, vp = _cache(K, dims, kc, vc, n_q, Hq, seed=100 + step)
        out_s, lse_s, out_w, lse_w = _both(K, kp, vp, shape, q, kv_len, Hq, n_q)
        assert np.all(np.isfinite(out_s)) and np.all(np.isfinite(lse_s))
        if kc.codebook == K.NF4:
            # the general kernel is bit-reproducible: the same kernels give the same bits
            assert np.array_equal(out_s, out_w) and np.array_equal(lse_s, lse_w)
        else:
            # the MFMA kernel hands out its steps dynamically: fp32 rounding order differs
            assert _rel(out_s.astype(np.float64), out_w.astype(np.float64)).max() < 1e-5
            assert np.abs(lse_s - lse_w).max() < 1e-5
        ref, ref_lse = _oracle(K, k, v, q, kv_len, kc, vc)
        assert _rel(out_s.astype(np.float64), ref).max() < 2e-3
        assert np.abs(lse_s - ref_lse).max() < 1e-4


def test_static_decode_rejects_sizes_beyond_the_scratch():
    """n_q = 256 decode queries of the 64K cache need about 34 MB of partials: the
    call returns KVQ_ERR_WORKSPACE before launching (every buffer is real and of its
    full size, so nothing could read out of bounds even if it launched)."""
    import kv_cache_bit_fwht_amd as K
    import torch
    B, L, H, T, D, Hq, n_q = 1, 8, 4, 65536, 256, 16, 256
    shape = K.Shape(B, L, H, T, D)
    need = K.kvq_decode_attn_workspace(shape, Hq, n_q)
    assert need > K.STATIC_SCRATCH_BYTES
    kp = K.alloc_packed(K.Codec(K.INT_ABSMAX, 4, 128, 256), shape)
    vp = K.alloc_packed(K.Codec(K.INT_ABSMAX, 2, 128, 0), shape)
    q = torch.zeros((B, L, n_q, Hq, D), dtype=torch.int16, device="cuda:0")
    out = torch.full((B, L, n_q, Hq, D), -7.0, dtype=torch.float32, device="cuda:0")
    announce("kvq_decode_attn_static over the size limit")
    with pytest.raises(K.KvqError) as e:
        K.kvq_decode_attn_static(kp, vp, Hq, n_q, q, None, 0.0, out, None)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert bool((out == -7.0).all())

"""The general decode kernel at the split counts it uses on long caches: 512 splits
(its maximum) for one (layer, KV head) unit of 65,536 tokens, directly and as the
per-head segments of a codec map decoded by per-segment launches; outputs against
the oracle's decode at full length ([E22L] What I tested: 64K-token spans)."""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import announce, oracle_codec, to_dev, to_np
from tests.test_gpu_attn import _check_decode, _gpu_decode, _gpu_pack

pytestmark = pytest.mark.gpu

T64 = 65536


def _deq(K, x, codec):
    oc = oracle_codec(K, O, codec)
    w, s, z = O.quantize_pack(x, oc)
    return O.dequant(w, s, z, oc, x.shape)


def test_general_kernel_512_splits_one_unit_64k():
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=1, H=1, Hq=4, n_q=2)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    kv_len = np.array([[[T64, 40001]]], dtype=np.int32)
    kc, vc = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    shape = K.Shape(1, 1, 1, T64, 256)
    # the workspace holds 512 splits' partials: [rows][Hq][512][D + 2] fp32
    assert K.kvq_decode_attn_workspace(shape, 4, 2) >= 65536 + 2 * 4 * 512 * 258 * 4
    announce("general kernel, one 64K unit, 512 splits")
    kp, vp = _gpu_pack(K, Kx, kc), _gpu_pack(K, Vx, vc)
    out, lse = _gpu_decode(K, kp, vp, q, kv_len, path=1)
    ref_out, ref_lse = O.decode_attn(q, _deq(K, Kx, kc), _deq(K, Vx, vc), kv_len)
    _check_decode(out, lse, ref_out, ref_lse, kv_len)


def test_general_kernel_per_head_64k_segments_route1():
    """Two one-head segments of 65,536 tokens with codecs the MFMA kernel does not take
    (6-bit keys with 3-bit values; NF4 keys with 4-bit values), each decoded by its own
    general-kernel launch at 512 splits, merged by log-sum-exp."""
    import torch
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=1, H=2, Hq=8, n_q=2)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    kv_len = np.array([[[T64, 12345]]], dtype=np.int32)
    codecs = [(K.Codec(K.INT_ABSMAX, 6, 128, 256), K.Codec(K.INT_ABSMAX, 3, 128, 0)),
              (K.Codec(K.NF4, 4, 64, 0), K.Codec(K.INT_ABSMAX, 4, 64, 0))]
    announce("general kernel, per-head 64K segments, route 1")
    segs, ref = [], []
    for h, (kc, vc) in enumerate(codecs):
        ks = np.ascontiguousarray(Kx[:, :, h:h + 1])
        vs = np.ascontiguousarray(Vx[:, :, h:h + 1])
        segs.append(K.Segment(_gpu_pack(K, ks, kc), _gpu_pack(K, vs, vc), 0, 0, h))
        ref.append((_deq(K, ks, kc), _deq(K, vs, vc), 0, 0, h))
    Kd, Vd = O.assemble_segments(ref, 1, 1, 2, T64, 256)
    out = torch.empty((1, 1, 2, 8, 256), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((1, 1, 2, 8), dtype=torch.float32, device="cuda:0")
    wsb = K.kvq_decode_attn_segments_workspace(segs, 1, 2, 8, 2)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda:0")
    K.kvq_decode_attn_segments(segs, 1, 2, T64, 8, 2, to_dev(q), to_dev(kv_len), 0.0, out, lse, ws, wsb, path=1)
    torch.cuda.synchronize()
    ref_out, ref_lse = O.decode_attn(q, Kd, Vd, kv_len)
    _check_decode(to_np(out), to_np(lse), ref_out, ref_lse, kv_len)

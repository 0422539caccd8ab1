"""GPU parity of the pieces around the path in real decoding ([FMAG-6] The winning
recipe, Selective-Layer Decode Anchoring):

* the append path (kvq_quantize_pack_tokens) writes exactly the codes of quantising
  the whole tensor, window by window, and touches no other row;
* decode over segments (anchors at other precisions on chosen layers and tokens,
  per-layer codecs, a key mean on one segment) against the oracle's decode of the
  assembled cache, within the attention bars;
* codec maps (per-layer and per-head codec pairs over whole-token tiles) decoded by
  one launch, by per-segment launches and by the default route;
* an append-then-decode loop gives, step by step, the decode of the fully quantised
  cache at the same lengths."""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import announce, oracle_codec, to_dev, to_np
from tests.test_gpu_attn import _check_decode

pytestmark = pytest.mark.gpu


def _packed_arrays(p):
    out = [to_np(p.codes, np.uint32)]
    if p.scales is not None and p.scales.numel():
        out.append(to_np(p.scales, np.uint16))
    if p.mins is not None:
        out.append(to_np(p.mins, np.uint16))
    return out


APPEND = [((1, 4, 128, 256), 256, False), ((1, 2, 128, 0), 256, False), ((2, 3, 32, 0), 128, False),
          ((5, 4, 64, 0), 64, False), ((7, 5, 32, 0, 7), 128, False), ((8, 6, 16, 0), 256, False),
          ((0,), 128, False), ((1, 4, 128, 256), 256, True), ((10, 3, 32, 128), 128, True)]


@pytest.mark.parametrize("cspec,D,with_mean", APPEND)
def test_append_windows_equal_the_whole_tensor(cspec, D, with_mean):
    import torch
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", B=2, L=2, H=2, T=90, D=D, k_mean_share=0.5 if with_mean else 0.0)
    Kx, _ = synth.gen_kv(w)
    shape = K.Shape(*Kx.shape)
    codec = K.Codec(*cspec)
    mean = to_dev(O.key_mean(Kx)) if with_mean else None
    announce(f"append windows codec={codec} D={D} mean={with_mean}")
    full = K.alloc_packed(codec, shape, mean=mean)
    K.kvq_quantize_pack(to_dev(Kx), full)
    win = K.alloc_packed(codec, shape, mean=mean)
    for t in (win.codes, win.scales, win.mins):
        if t is not None and t.numel():
            t.fill_(0x5a5a)
    for (t0, n) in ((0, 50), (50, 1), (51, 39)):
        K.kvq_quantize_pack_tokens(to_dev(np.ascontiguousarray(Kx[:, :, :, t0:t0 + n])), t0, n, win)
    torch.cuda.synchronize()
    for a, b in zip(_packed_arrays(full), _packed_arrays(win)):
        assert np.array_equal(a, b)
    # a middle window alone: only its rows change
    mid = K.alloc_packed(codec, shape, mean=mean)
    for t in (mid.codes, mid.scales, mid.mins):
        if t is not None and t.numel():
            t.fill_(0x5a5a)
    before = _packed_arrays(mid)
    K.kvq_quantize_pack_tokens(to_dev(np.ascontiguousarray(Kx[:, :, :, 30:37])), 30, 7, mid)
    torch.cuda.synchronize()
    rows = np.zeros((2, 2, 2, 90), bool)
    rows[:, :, :, 30:37] = True
    rows = rows.ravel()
    for a, b, f in zip(_packed_arrays(full), _packed_arrays(mid), before):
        assert np.array_equal(b[rows], a[rows]) and np.array_equal(b[~rows], f[~rows])


def _oracle_seg(K, x, codec, mean=None, chan=None):
    oc = oracle_codec(K, O, codec)
    w, s, z = O.quantize_pack(x, oc, chan, mean)
    return O.dequant(w, s, z, oc, x.shape, chan, mean)


def _gpu_seg(K, x, codec, mean=None, chan=None):
    p = K.alloc_packed(codec, K.Shape(*x.shape), mean=to_dev(mean) if mean is not None else None,
                       chan_scale=to_dev(chan) if chan is not None else None)
    if codec.codebook == K.FP16:
        return K.packed_from_fp16(to_dev(x), K.Shape(*x.shape))
    K.kvq_quantize_pack(to_dev(x), p)
    return p


def _run_segments(K, Kx, Vx, q, kv_len, layout, mean_seg=None, path=None, chan_seg=None):
    """layout: list of (kcodec, vcodec, layer0, n_layers, token0, n_tokens[, head0, n_heads]);
    segment mean_seg carries a key mean, segment chan_seg per-channel key scales
    (calibrated on its sequence 0); path as for kvq_decode_attn_segments_ex."""
    import torch
    B, L, H, T, D = Kx.shape
    nq, Hq = q.shape[2], q.shape[3]
    segs, ref = [], []
    for i, sg in enumerate(layout):
        kc, vc, l0, nl, t0, nt = sg[:6]
        h0, nh = (sg[6], sg[7]) if len(sg) > 6 else (0, H)
        ks = np.ascontiguousarray(Kx[:, l0:l0 + nl, h0:h0 + nh, t0:t0 + nt])
        vs = np.ascontiguousarray(Vx[:, l0:l0 + nl, h0:h0 + nh, t0:t0 + nt])
        mean = O.key_mean(ks) if i == mean_seg else None
        chan = O.calibrate_chan_scale(ks[0]) if i == chan_seg else None
        segs.append(K.Segment(_gpu_seg(K, ks, kc, mean, chan), _gpu_seg(K, vs, vc), l0, t0, h0))
        ref.append((_oracle_seg(K, ks, kc, mean, chan), _oracle_seg(K, vs, vc), l0, t0, h0))
    Kd, Vd = O.assemble_segments(ref, B, L, H, T, D)
    out = torch.empty((B, L, nq, Hq, D), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((B, L, nq, Hq), dtype=torch.float32, device="cuda:0")
    wsb = K.kvq_decode_attn_segments_workspace(segs, L, H, Hq, nq)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda:0")
    K.kvq_decode_attn_segments(segs, L, H, T, Hq, nq, to_dev(q), to_dev(kv_len) if kv_len is not None else None, 0.0,
                               out, lse, ws, wsb, path=path)
    torch.cuda.synchronize()
    ref_out, ref_lse = O.decode_attn(q, Kd, Vd, kv_len)
    _check_decode(to_np(out), to_np(lse), ref_out, ref_lse, kv_len)
    assert np.all(to_np(ws[:65536]) == 0)                 # counters left zero
    return segs


@pytest.mark.parametrize("variant", ["anchors", "per_layer", "causal_mean", "window", "per_head", "per_head_b2"])
def test_decode_over_segments(variant):
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=4, T=704, n_q=3)
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w)
    k4, v2 = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    f16, i8 = K.Codec(K.FP16), K.Codec(K.INT8_SYM, 8, 256, 0)
    mean_seg = None
    if variant == "anchors":
        # prompt [0, 640) in 4/2 bits; the first 48 decoded tokens at fp16 on layers 0-1
        # and in 4/2 bits on layers 2-3; the last 16 tokens int8 on every layer
        layout = [(k4, v2, 0, 4, 0, 640), (f16, f16, 0, 2, 640, 48), (k4, v2, 2, 2, 640, 48), (i8, i8, 0, 4, 688, 16)]
    elif variant == "per_layer":
        layout = [(f16, f16, 0, 1, 0, 704), (k4, v2, 1, 3, 0, 704)]
    elif variant == "causal_mean":
        kv_len = np.array([[[704, 650, 17], [0, 640, 700], [1, 688, 689], [300, 301, 704]]], dtype=np.int32)
        layout = [(k4, v2, 0, 4, 0, 640), (K.Codec(K.INT_ABSMAX, 4, 64, 0), K.Codec(K.INT_ABSMAX, 4, 64, 0), 0, 4, 640, 64)]
        mean_seg = 0
    elif variant == "window":
        layout = [(K.Codec(K.SIGN, 1, 8, 0), K.Codec(K.SIGN, 1, 8, 0), 0, 4, 0, 640), (f16, f16, 0, 4, 640, 64)]
    else:
        # per-head KV types: a sink head at fp16, two heads in 4/2 bits, a diffuse head in
        # 3-bit keys; layers 2-3 of head 0 back in 4/2 bits for the first 352 tokens
        if variant == "per_head_b2":
            w = synth.get("c3", B=2, L=4, T=704, n_q=2)
            Kx, Vx = synth.gen_kv(w)
            q, kv_len = synth.gen_queries(w)
            kv_len = np.random.default_rng(2).integers(0, 705, (2, 4, 2)).astype(np.int32)
        k3 = K.Codec(K.INT_ABSMAX, 3, 128, 256)
        layout = [(f16, f16, 0, 2, 0, 704, 0, 1), (k4, v2, 2, 2, 0, 352, 0, 1), (f16, f16, 2, 2, 352, 352, 0, 1),
                  (k4, v2, 0, 4, 0, 704, 1, 2), (k3, v2, 0, 4, 0, 704, 3, 1)]
    announce(f"segments {variant}")
    _run_segments(K, Kx, Vx, q, kv_len, layout, mean_seg)


MAPS = ["alloc_319", "heads_entropy", "anchor_layer", "g8_heads", "mfma_tile", "mfma_map_heads", "mfma_map_layers",
        "mfma_map_g2", "mfma_map_k2", "wave_map_g1"]


@pytest.mark.parametrize("path", [None, 1, 2])
@pytest.mark.parametrize("variant", MAPS)
def test_codec_map_in_one_launch(variant, path):
    """Codec maps (every segment a whole-token tile of layers x KV heads) decoded by one
    launch (path 2), by per-segment launches (path 1) and by the default choice, each
    against the oracle's decode of the assembled cache."""
    import kv_cache_bit_fwht_amd as K
    A = K.INT_ABSMAX
    mean_seg = chan_seg = None
    if variant == "alloc_319":
        # per-layer bits of [E21W] Result's 3.19-bit allocation (rotated, groups of 128):
        # 2-bit keys on layers 2 and 7, 4-bit values on layers 1, 3 and 4, 3 bits elsewhere
        w = synth.get("c3", L=8, T=600, n_q=2)
        Kx, Vx = synth.gen_kv(w)
        q, _ = synth.gen_queries(w)
        kv_len = np.random.default_rng(31).integers(0, 601, (1, 8, 2)).astype(np.int32)
        k2, k3 = K.Codec(A, 2, 128, 256), K.Codec(A, 3, 128, 256)
        v3, v4 = K.Codec(A, 3, 128, 256), K.Codec(A, 4, 128, 256)
        layout = [(k3, v3, 0, 1, 0, 600), (k3, v4, 1, 1, 0, 600), (k2, v3, 2, 1, 0, 600), (k3, v4, 3, 2, 0, 600),
                  (k3, v3, 5, 2, 0, 600), (k2, v3, 7, 1, 0, 600)]
        chan_seg = 3
    elif variant == "heads_entropy":
        # per-head key bits [5, 4, 4, 3] over 4-bit values, a key mean on head 0
        w = synth.get("c3", B=2, L=3, T=520, n_q=2, k_head_scales=(3.0, 1.0, 1.0, 0.5), k_mean_share=0.3)
        Kx, Vx = synth.gen_kv(w)
        q, _ = synth.gen_queries(w)
        kv_len = np.random.default_rng(32).integers(0, 521, (2, 3, 2)).astype(np.int32)
        kv_len[1, 2, 1] = 0
        v4 = K.Codec(A, 4, 128, 0)
        layout = [(K.Codec(A, 5, 128, 256), v4, 0, 3, 0, 520, 0, 1), (K.Codec(A, 4, 128, 256), v4, 0, 3, 0, 520, 1, 2),
                  (K.Codec(A, 3, 128, 256), v4, 0, 3, 0, 520, 3, 1)]
        mean_seg = 0
    elif variant == "anchor_layer":
        # head_dim 128: an fp16 layer, then ternary / NF4+int4 / int8 / sign tiles
        w = synth.get("c4", B=1, L=4, H=4, Hq=16, T=300, n_q=2)
        Kx, Vx = synth.gen_kv(w)
        q, kv_len = synth.gen_queries(w)
        f16, tern = K.Codec(K.FP16), K.Codec(K.TERNARY, 2, 8, 0)
        nf4, a4, i8 = K.Codec(K.NF4, 4, 64, 0), K.Codec(A, 4, 64, 0), K.Codec(K.INT8_SYM, 8, 128, 0)
        sgn = K.Codec(K.SIGN, 1, 8, 0)
        layout = [(f16, f16, 0, 1, 0, 300), (tern, tern, 1, 2, 0, 300, 0, 2), (nf4, a4, 1, 1, 0, 300, 2, 2),
                  (i8, i8, 2, 1, 0, 300, 2, 2), (sgn, sgn, 3, 1, 0, 300)]
    elif variant == "g8_heads":
        # 8 query heads per KV head (two head groups per block row), rotated 2-bit values on head 0
        w = synth.get("c3", L=2, H=2, Hq=16, T=400, n_q=2)
        Kx, Vx = synth.gen_kv(w)
        q, _ = synth.gen_queries(w)
        kv_len = np.array([[[400, 0], [1, 333]]], dtype=np.int32)
        layout = [(K.Codec(A, 2, 128, 0), K.Codec(A, 2, 128, 256), 0, 2, 0, 400, 0, 1),
                  (K.Codec(A, 6, 64, 128), K.Codec(A, 3, 32, 0), 0, 2, 0, 400, 1, 1)]
    elif variant == "mfma_map_heads":
        # per-head key bits [5, 4, 4, 3] over 4-bit values at group 128: every tile an MFMA
        # pair, so the default and path 2 run the map in one MFMA launch
        w = synth.get("c3", B=2, L=3, T=512, n_q=2, k_head_scales=(3.0, 1.0, 1.0, 0.5))
        Kx, Vx = synth.gen_kv(w)
        q, _ = synth.gen_queries(w)
        kv_len = np.random.default_rng(33).integers(0, 513, (2, 3, 2)).astype(np.int32)
        kv_len[0, 1, 0] = 0
        v4 = K.Codec(A, 4, 128, 0)
        layout = [(K.Codec(A, 5, 128, 256), v4, 0, 3, 0, 512, 0, 1), (K.Codec(A, 4, 128, 256), v4, 0, 3, 0, 512, 1, 2),
                  (K.Codec(A, 3, 128, 256), v4, 0, 3, 0, 512, 3, 1)]
    elif variant == "mfma_map_layers":
        # per-layer pairs with 2- and 4-bit values, a rotated-value tile and a tile with key
        # channel scales, 4 query heads per KV head
        w = synth.get("c3", L=4, T=448, n_q=3)
        Kx, Vx = synth.gen_kv(w)
        q, _ = synth.gen_queries(w)
        kv_len = np.array([[[448, 31, 200], [1, 447, 448], [0, 64, 65], [300, 301, 96]]], dtype=np.int32)
        layout = [(K.Codec(A, 3, 128, 256), K.Codec(A, 2, 128, 0), 0, 1, 0, 448),
                  (K.Codec(A, 4, 128, 256), K.Codec(A, 4, 128, 256), 1, 2, 0, 448),
                  (K.Codec(A, 5, 128, 128), K.Codec(K.INT_SYM, 2, 128, 0), 3, 1, 0, 448)]
        chan_seg = 2
    elif variant == "mfma_map_g2":
        # two query heads per KV head on the MFMA codec map, a key mean on one tile
        w = synth.get("c3", L=2, Hq=8, T=384, n_q=2, k_mean_share=0.3)
        Kx, Vx = synth.gen_kv(w)
        q, _ = synth.gen_queries(w)
        kv_len = np.array([[[384, 100], [33, 0]]], dtype=np.int32)
        layout = [(K.Codec(A, 5, 128, 256), K.Codec(A, 2, 128, 0), 0, 2, 0, 384, 0, 3),
                  (K.Codec(A, 3, 128, 256), K.Codec(A, 4, 128, 256), 0, 2, 0, 384, 3, 1)]
        mean_seg = 1
    elif variant == "mfma_map_k2":
        # 2-bit keys (over 2- and 4-bit values) beside 4-bit keys, all MFMA pairs: one launch
        w = synth.get("c3", L=3, T=352, n_q=2)
        Kx, Vx = synth.gen_kv(w)
        q, _ = synth.gen_queries(w)
        kv_len = np.array([[[352, 33], [0, 351], [200, 1]]], dtype=np.int32)
        layout = [(K.Codec(A, 2, 128, 256), K.Codec(A, 2, 128, 0), 0, 1, 0, 352),
                  (K.Codec(A, 2, 128, 0), K.Codec(A, 4, 128, 256), 1, 1, 0, 352),
                  (K.Codec(A, 4, 128, 256), K.Codec(A, 2, 128, 0), 2, 1, 0, 352)]
    elif variant == "wave_map_g1":
        # one query head per KV head on the general codec map: four query rows share a
        # wavefront, each with its own key count
        w = synth.get("c3", L=2, Hq=4, T=300, n_q=5)
        Kx, Vx = synth.gen_kv(w)
        q, _ = synth.gen_queries(w)
        kv_len = np.random.default_rng(34).integers(0, 301, (1, 2, 5)).astype(np.int32)
        kv_len[0, 1, 4] = 0
        layout = [(K.Codec(A, 2, 128, 256), K.Codec(A, 3, 128, 0), 0, 1, 0, 300),
                  (K.Codec(K.SIGN, 1, 8, 0), K.Codec(K.SIGN, 1, 8, 0), 1, 1, 0, 300)]
    else:
        # a tile the MFMA kernel would take (4-bit rotated keys, 2-bit values) beside an fp16 layer
        w = synth.get("c3", L=3, T=448, n_q=2)
        Kx, Vx = synth.gen_kv(w)
        q, kv_len = synth.gen_queries(w)
        layout = [(K.Codec(K.FP16), K.Codec(K.FP16), 0, 1, 0, 448),
                  (K.Codec(A, 4, 128, 256), K.Codec(A, 2, 128, 0), 1, 2, 0, 448)]
    announce(f"codec map {variant} path={path}")
    _run_segments(K, Kx, Vx, q, kv_len, layout, mean_seg, path, chan_seg)


def test_append_then_decode_loop_matches_the_whole_cache():
    """Tokens appended one by one (the last 8 of 520) with a decode after each, against
    the same decode on the cache quantised in one call."""
    import torch
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=2, T=520, n_q=1)
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    B, L, H, T, D = Kx.shape
    Hq = q.shape[3]
    shape = K.Shape(B, L, H, T, D)
    kc, vc = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    announce("append + decode loop")
    kf, vf = K.alloc_packed(kc, shape), K.alloc_packed(vc, shape)
    K.kvq_quantize_pack(to_dev(Kx), kf)
    K.kvq_quantize_pack(to_dev(Vx), vf)
    ka, va = K.alloc_packed(kc, shape), K.alloc_packed(vc, shape)
    K.kvq_quantize_pack_tokens(to_dev(np.ascontiguousarray(Kx[:, :, :, :512])), 0, 512, ka)
    K.kvq_quantize_pack_tokens(to_dev(np.ascontiguousarray(Vx[:, :, :, :512])), 0, 512, va)
    wsb = K.kvq_decode_attn_workspace(shape, Hq, 1)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda:0")
    qd = to_dev(q)
    for t in range(512, 520):
        K.kvq_quantize_pack_tokens(to_dev(np.ascontiguousarray(Kx[:, :, :, t:t + 1])), t, 1, ka)
        K.kvq_quantize_pack_tokens(to_dev(np.ascontiguousarray(Vx[:, :, :, t:t + 1])), t, 1, va)
        kvl = to_dev(np.full((B, L, 1), t + 1, dtype=np.int32))
        o1 = torch.empty((B, L, 1, Hq, D), dtype=torch.float32, device="cuda:0")
        o2, l1, l2 = torch.empty_like(o1), torch.empty((B, L, 1, Hq), dtype=torch.float32, device="cuda:0"), \
            torch.empty((B, L, 1, Hq), dtype=torch.float32, device="cuda:0")
        K.kvq_decode_attn(ka, va, Hq, 1, qd, kvl, 0.0, o1, l1, ws, wsb)
        K.kvq_decode_attn(kf, vf, Hq, 1, qd, kvl, 0.0, o2, l2, ws, wsb)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"step {t}"
    for a, b in zip(_packed_arrays(kf) + _packed_arrays(vf), _packed_arrays(ka) + _packed_arrays(va)):
        assert np.array_equal(a, b)

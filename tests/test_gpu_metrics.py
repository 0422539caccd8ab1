"""GPU parity of kvq_attn_error_ex: the diagnostic ladder's rungs ([FMAG-R], the
Colab-probe reply: QK-logit error, attention KL / JS, top-attended-token flips,
attention-output error) and the Renyi-2 entropy of [LCPP] Finding 2, against the
oracle's fp64 definitions.  Bars: KL and relative error as for kvq_attn_error;
H_2, JS and the logit error within 1e-5 (both sides fp64 over the same dequantised
values, summed in different orders); top-1 flips equal except where the oracle's
two largest logits lie within 1e-9 of each other."""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_util import announce, oracle_codec, to_dev, to_np
from tests.test_gpu_attn import KL_TOL

pytestmark = pytest.mark.gpu


def _run(K, Kx, Vx, q, kv_len, kc, vc, mean=None, subset=None):
    import torch
    B, L, nq, Hq, D = q.shape
    H = Kx.shape[2]
    shape = K.Shape(*Kx.shape)
    kp = K.alloc_packed(kc, shape, mean=to_dev(mean) if mean is not None else None)
    vp = K.alloc_packed(vc, shape)
    K.kvq_quantize_pack(to_dev(Kx), kp)
    K.kvq_quantize_pack(to_dev(Vx), vp)
    names = subset or ("kl", "relerr", "renyi2", "js", "logit_relerr", "top1")
    outs = {n: torch.full((B, L, nq, Hq), float("nan"), dtype=torch.float32, device="cuda:0") for n in names}
    kv = torch.empty((B, L, H, 4), dtype=torch.float64, device="cuda:0") if subset is None else None
    wsb = K.kvq_attn_error_workspace(shape, Hq, nq)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda:0")
    K.kvq_attn_error_ex(to_dev(Kx), to_dev(Vx), kp, vp, Hq, nq, to_dev(q),
                        to_dev(kv_len) if kv_len is not None else None, 0.0, ws, wsb, kv_err=kv, **outs)
    torch.cuda.synchronize()
    okc, ovc = oracle_codec(K, O, kc), oracle_codec(K, O, vc)
    wk, sk, zk = O.quantize_pack(Kx, okc, None, mean)
    wv, sv, zv = O.quantize_pack(Vx, ovc)
    Kd = O.dequant(wk, sk, zk, okc, Kx.shape, None, mean)
    Vd = O.dequant(wv, sv, zv, ovc, Vx.shape)
    ref = O.attn_error_ex(q, Kx, Vx, Kd, Vd, kv_len)
    got = {n: to_np(t) for n, t in outs.items()}
    if "kl" in got:
        assert np.abs(got["kl"] - ref["kl"]).max() < KL_TOL
    if "relerr" in got:
        assert np.abs(got["relerr"] - ref["relerr"]).max() < 1e-4
    for n in ("renyi2", "js", "logit_relerr"):
        if n in got:
            d = np.abs(got[n] - ref[n])
            assert d.max() < 1e-5 + 1e-4 * np.abs(ref[n]).max(), f"{n}: max diff {d.max():.3g}"
    if "top1" in got:
        bad = got["top1"] != ref["top1_flip"]
        if bad.any():   # only where the reference's top-2 logits nearly tie
            s = 1.0 / np.sqrt(D)
            qq = q.astype(np.float64)
            G = Hq // H
            for (b, l, i, j) in zip(*np.nonzero(bad)):
                n = Kx.shape[3] if kv_len is None else int(kv_len[b, l, i])
                for kk in (Kx.astype(np.float64), Kd.astype(np.float64)):
                    lg = np.sort(s * kk[b, l, j // G, :n] @ qq[b, l, i, j])[::-1]
                    assert n > 1 and lg[0] - lg[1] < 1e-9, f"top-1 differs at {(b, l, i, j)}"
    if kv is not None:
        assert np.allclose(to_np(kv), ref["kv_err"], rtol=1e-9, atol=1e-12)
    return got, ref


@pytest.mark.parametrize("case", ["c1_minmax3", "c3_k4rot_v2", "c3_k3rot_v2_mean", "c5_rfft_polar", "c4_ternary"])
def test_error_ladder_matches_the_oracle(case):
    import kv_cache_bit_fwht_amd as K
    mean = None
    if case == "c1_minmax3":
        w = synth.get("c1", T=300, n_q=5)
        Kx, Vx = synth.gen_kv(w)
        q, kv_len = synth.gen_queries(w, Kx)
        kc = vc = K.Codec(K.INT_MINMAX, 3, 32, 0)
    elif case.startswith("c3"):
        w = synth.get("c3", L=2, T=600, n_q=3, k_mean_share=0.53 if "mean" in case else 0.0)
        Kx, Vx = synth.gen_kv(w)
        q, kv_len = synth.gen_queries(w)
        kv_len = np.array([[[600, 17, 0], [1, 599, 300]]], dtype=np.int32)
        kc = K.Codec(K.INT_ABSMAX, 4 if "k4" in case else 3, 128, 256)
        vc = K.Codec(K.INT_ABSMAX, 2, 128, 0)
        if "mean" in case:
            mean = O.key_mean(Kx)
    elif case == "c5_rfft_polar":
        w = synth.get("c5", B=1, L=2, H=2, Hq=8, T=300, n_q=2)
        Kx, Vx = synth.gen_kv(w)
        q, kv_len = synth.gen_queries(w)
        kc, vc = K.Codec(K.RFFT_POLAR, 5, 32, 0, 7), K.Codec(K.FP16)
    else:
        w = synth.get("c4", B=1, L=2, H=2, Hq=8, T=300, n_q=2)
        Kx, Vx = synth.gen_kv(w)
        q, kv_len = synth.gen_queries(w)
        kc = vc = K.Codec(K.TERNARY, 2, 8, 0)
    announce(f"error ladder {case}")
    got, ref = _run(K, Kx, Vx, q, kv_len, kc, vc, mean)
    assert np.all(got["js"] >= -1e-7) and np.all(got["js"] <= np.log(2) + 1e-6)
    assert np.all(np.isfinite(got["renyi2"]))


def test_error_outputs_subset_and_js_alone():
    import kv_cache_bit_fwht_amd as K
    w = synth.get("c3", L=1, T=333, n_q=2)
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w)
    announce("error ladder subset")
    kc, vc = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    _run(K, Kx, Vx, q, kv_len, kc, vc, subset=("js",))
    _run(K, Kx, Vx, q, kv_len, kc, vc, subset=("renyi2", "top1"))

"""Benchmark of the hot path on the 64K-token decode workload (one GPU).

Workload: 8 layers x 4 KV heads x 65,536 tokens x head_dim 256, batch 1, 16
query heads (GQA 4:1); keys Walsh-Hadamard-rotated (256) 4-bit signed absmax at
group 128, values 2-bit signed absmax at group 128 (3.125 bits per value with
the fp16 scales); 256 decode queries ~ N(0,1).  Seeded synthetic fp16 K/V stand
in for the real 64K-span caches the pages measure on.

One step = quantise+pack K and V of the whole cache (kvq_quantize_pack_kv, one
launch) + 256 decode-attention calls (kvq_decode_attn, one per decode query,
each reading the whole packed cache).  Inputs are resident in HBM before the
timed region; three copies of the packed cache are rotated so the 256 MB
Infinity Cache cannot serve repeats.

Prints one JSON line: value = decode tokens per second of the whole step
(quantise included); the split rates, the roofline of the dominant kernel
(decode) measured with HIP events on the launch stream, and the CPU oracle
timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X published HBM3E bandwidth
KERNEL_SRC = {"decode": ["kv_cache_bit_fwht_amd/csrc/kvq_attn_fast.hip", "kv_cache_bit_fwht_amd/csrc/kvq_mfma_body.inc",
                         "kv_cache_bit_fwht_amd/csrc/kvq_attn.hip", "kv_cache_bit_fwht_amd/csrc/kvq_quant256.hpp",
                         "kv_cache_bit_fwht_amd/csrc/kvq_internal.hpp"],
              "quantize": ["kv_cache_bit_fwht_amd/csrc/kvq_quant.hip", "kv_cache_bit_fwht_amd/csrc/kvq_codec.hpp",
                           "kv_cache_bit_fwht_amd/csrc/kvq_quant256.hpp", "kv_cache_bit_fwht_amd/csrc/kvq_internal.hpp"]}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def src_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kind, per_launch_units):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f).get(kind)
    if not d or d.get("src_hash") != src_hash(KERNEL_SRC[kind]):
        return None
    return d.get("bytes_per_launch")


def measure_ceilings(torch, dev):
    """Achievable-bandwidth reference measured with a library kernel (not this
    package's): a 1 GiB device-to-device copy (1 GiB read + 1 GiB written).
    Median of 5 after 2 warm-ups."""
    n = 1 << 28
    src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)

    def med(fn):
        for _ in range(2):
            fn()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    t_copy = med(lambda: dst.copy_(src))
    del src, dst
    torch.cuda.empty_cache()
    nbytes = n * 4
    return {"copy_GBps": round(2 * nbytes / t_copy / 1e9, 1),
            "how": "1 GiB device-to-device copy (1 GiB read + 1 GiB written), median of 5"}


def cpu_baseline(Kx, Vx, q, units_sample=2, queries_sample=4):
    """The oracle as it stands, timed on this host's cores on a bounded sample of
    the same workload and extrapolated to the whole step (the full step would take
    about an hour of CPU time).

    - quantise+pack: `units_sample` whole (layer, head) units of K and V (65,536
      rows each) through the oracle's binary32 codec (NumPy elementwise: 1 core);
    - decode attention: `queries_sample` decode queries against those units in
      fp64 on the oracle's dequantised cache, once with BLAS held to 1 thread and
      once with every core in this process's affinity mask.
    value = decode tokens per second of the whole step (all units quantised, every
    query attended over all units) with the all-cores attention leg."""
    from threadpoolctl import threadpool_limits
    import oracle as O
    B, L, H, T, D = Kx.shape
    nq = q.shape[2]
    G = q.shape[3] // H
    kc = O.Codec(O.INT_ABSMAX, 4, 128, rot=256)
    vc = O.Codec(O.INT_ABSMAX, 2, 128)
    ncores = len(os.sched_getaffinity(0))
    deq = []
    t_q = 0.0
    with threadpool_limits(limits=1):
        for u in range(units_sample):
            l, h = u // H, u % H
            ku = Kx[0, l, h][None, None, None]
            vu = Vx[0, l, h][None, None, None]
            t0 = time.perf_counter()
            wk, sk, zk = O.quantize_pack(ku, kc)
            wv, sv, zv = O.quantize_pack(vu, vc)
            t_q += time.perf_counter() - t0
            deq.append((O.dequant(wk, sk, zk, kc, ku.shape)[0, 0, 0], O.dequant(wv, sv, zv, vc, vu.shape)[0, 0, 0]))
    t_q /= units_sample

    def attend_all():
        t0 = time.perf_counter()
        for u in range(units_sample):
            l, h = u // H, u % H
            Kd, Vd = deq[u]
            for i in range(queries_sample):
                O.attention.attend(q[0, l, i, h * G:(h + 1) * G].astype(np.float64), Kd, Vd, T, 1.0 / np.sqrt(D))
        return (time.perf_counter() - t0) / (units_sample * queries_sample)

    with threadpool_limits(limits=1):
        t_att1 = attend_all()
    with threadpool_limits(limits=ncores):
        t_attn = attend_all()
    units = B * L * H
    unit_bytes = T * (2 * D * 2 + D * 4 // 8 + 4 + D * 2 // 8 + 4)
    step1 = units * t_q + nq * units * t_att1
    stepn = units * t_q + nq * units * t_attn
    return {
        "value": round(nq * B / stepn, 6), "unit": "tok/s", "cores": ncores, "kind": "oracle",
        "sample": (f"extrapolated: {units_sample} of {units} (layer, head) units quantised+packed (K and V, "
                   f"{T} rows each) and {queries_sample} of {nq} decode queries attended over them in fp64, "
                   f"scaled to the whole step ({units} units, {nq} queries); quantise on 1 core (NumPy "
                   f"elementwise), attention with BLAS on all {ncores} affinity cores"),
        "value_1core": round(nq * B / step1, 6),
        "quantize_pack_GBps_1core": round(unit_bytes / t_q / 1e9, 5),
        "seconds_per_unit_quantize_pack": round(t_q, 3),
        "seconds_per_query_unit_attention": {"1 core": round(t_att1, 5), f"{ncores} cores": round(t_attn, 5)},
        "cpu": _cpu_name(),
    }


def _cpu_name():
    """CPU model string and family/model numbers from /proc/cpuinfo."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" in line:
                    k, v = (x.strip() for x in line.split(":", 1))
                    if k in ("model name", "cpu family", "model", "stepping") and k not in fields:
                        fields[k] = v
                if not line.strip() and fields:
                    break
    except OSError:
        pass
    if not fields:
        return "unknown"
    return (f"{fields.get('model name', 'unknown')} (family {fields.get('cpu family', '?')}, "
            f"model {fields.get('model', '?')}, stepping {fields.get('stepping', '?')})")


def _median_time(torch, fn, reps):
    fn()                                             # warm: code loaded, clocks up
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    return float(np.median(ts))


def secondary(workload, reps):
    """The other decode configurations (not the headline line): c4, extreme low-bit
    codecs at head_dim 128 with layer 0 kept in fp16; c5, transformed keys at
    head_dim 128 with fp16 values; c3v, the 64K cache with rotated 4-bit keys and
    each value codebook (the one-sided 2-bit grid, and the symmetric and Gaussian
    Lloyd-Max grids named as the next test), with the attention KL and output
    error of 16 queries; c3m, the 64K cache whose keys carry a shared per-(layer,
    head) mean (53% of key energy), 4- and 3-bit rotated keys coded with and
    without the mean subtracted, with the same error figures and the time of
    kvq_key_mean.  One JSON line per arm: quantize+pack of the arm's K and V, and
    one decode step (every layer, every query head, B queries)."""
    import torch
    import kv_cache_bit_fwht_amd as K
    import synth
    dev = torch.device("cuda:0")
    w = synth.get("c3" if workload == "c3v" else workload) if workload != "c3m" else synth.get("c3", k_mean_share=0.53)
    log(f"generating {w.description}")
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    kd = torch.from_numpy(Kx.view(np.int16)).to(dev)
    vd = torch.from_numpy(Vx.view(np.int16)).to(dev)
    qd = torch.from_numpy(np.ascontiguousarray(q[:, :, :1]).view(np.int16)).to(dev)
    del Kx, Vx
    f16 = K.Codec(K.FP16)
    mean_d, mean_us = None, 0.0
    if workload == "c3m":
        # keys with a shared per-(layer, head) mean carrying 53% of their energy; each key
        # codec with and without the mean subtracted (value codec fixed)
        shape_all = K.Shape(w.B, w.L, w.H, w.T, w.D)
        mean_d = torch.empty((w.L, w.H, w.D), dtype=torch.float32, device=dev)
        wmb = K.kvq_key_mean_workspace(shape_all)
        wm = torch.empty(wmb, dtype=torch.uint8, device=dev)
        K.kvq_key_mean(kd, shape_all, mean_d, wm, wmb)
        torch.cuda.synchronize()
        mean_us = _median_time(torch, lambda: K.kvq_key_mean(kd, shape_all, mean_d, wm, wmb), reps) * 1e6
        v2 = K.Codec(K.INT_ABSMAX, 2, 128, 0)
        arms = {}
        for kb_ in (4, 3):
            kcm = K.Codec(K.INT_ABSMAX, kb_, 128, 256)
            arms[f"K int{kb_} FWHT-256 g128, no mean"] = (kcm, v2)
            arms[f"K int{kb_} FWHT-256 g128, key mean subtracted"] = (kcm, v2, True)
        lo = 0
    elif workload == "c3v":
        kc3 = K.Codec(K.INT_ABSMAX, 4, 128, 256)
        arms = {"V int2 absmax g128 (one-sided grid)": (kc3, K.Codec(K.INT_ABSMAX, 2, 128, 0)),
                "V int2 symmetric g128, rotated": (kc3, K.Codec(K.INT_SYM, 2, 128, 256)),
                "V Lloyd-Max 2-bit g128, rotated": (kc3, K.Codec(K.LLOYD, 2, 128, 256)),
                "V int3 symmetric g128, rotated": (kc3, K.Codec(K.INT_SYM, 3, 128, 256)),
                "V Lloyd-Max 3-bit g128, rotated": (kc3, K.Codec(K.LLOYD, 3, 128, 256))}
        lo = 0
    elif workload == "c4":
        arms = {"ternary g8": (K.Codec(K.TERNARY, 2, 8, 0),) * 2, "sign g8": (K.Codec(K.SIGN, 1, 8, 0),) * 2,
                "NF4 K g64 + int4 V g64": (K.Codec(K.NF4, 4, 64, 0), K.Codec(K.INT_ABSMAX, 4, 64, 0)),
                "int8 g128": (K.Codec(K.INT8_SYM, 8, 128, 0),) * 2}
        lo = 1                                       # layer 0 is the fp16 anchor
    else:
        arms = {"rFFT polar 5+7 g32": (K.Codec(K.RFFT_POLAR, 5, 32, 0, 7), f16),
                "rFFT Cartesian 6+6 g32": (K.Codec(K.RFFT_CART, 6, 32, 0), f16),
                "FWHT-128 int6 absmax g32": (K.Codec(K.INT_ABSMAX, 6, 32, 128), f16)}
        lo = 0
    B, L, H, T, D, Hq = w.B, w.L, w.H, w.T, w.D, w.Hq
    shape = K.Shape(B, L - lo, H, T, D)
    kq, vq = kd[:, lo:].contiguous() if lo else kd, vd[:, lo:].contiguous() if lo else vd
    qq = qd[:, lo:].contiguous() if lo else qd
    out = torch.empty((B, L - lo, 1, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, L - lo, 1, Hq), dtype=torch.float32, device=dev)
    wsb = K.kvq_decode_attn_workspace(shape, Hq, 1)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
    anchor_s = 0.0
    if lo:
        ashape = K.Shape(B, 1, H, T, D)
        ka, va = K.packed_from_fp16(kd[:, :1].contiguous(), ashape), K.packed_from_fp16(vd[:, :1].contiguous(), ashape)
        qa = qd[:, :1].contiguous()
        oa = torch.empty((B, 1, 1, Hq, D), dtype=torch.float32, device=dev)
        la = torch.empty((B, 1, 1, Hq), dtype=torch.float32, device=dev)
        wsa_b = K.kvq_decode_attn_workspace(ashape, Hq, 1)
        wsa = torch.zeros(max(wsa_b, 16), dtype=torch.uint8, device=dev)
        anchor_s = _median_time(torch, lambda: K.kvq_decode_attn(ka, va, Hq, 1, qa, None, 0.0, oa, la, wsa, wsa_b),
                                reps)
    rows = B * (L - lo) * H * T
    for name, arm in arms.items():
        kc, vc = arm[0], arm[1]
        use_mean = len(arm) > 2 and arm[2]
        kp = K.alloc_packed(kc, shape, dev, mean=mean_d if use_mean else None)
        vp = K.packed_from_fp16(vq, shape) if vc.codebook == K.FP16 else K.alloc_packed(vc, shape, dev)

        def quant():
            if vc.codebook != K.FP16:
                K.kvq_quantize_pack_kv(kq, vq, kp, vp)
            else:
                K.kvq_quantize_pack(kq, kp)

        quant()
        torch.cuda.synchronize()
        t_q = _median_time(torch, quant, reps)
        K.kvq_decode_attn(kp, vp, Hq, 1, qq, None, 0.0, out, lse, ws, wsb)
        torch.cuda.synchronize()
        t_d = _median_time(torch, lambda: K.kvq_decode_attn(kp, vp, Hq, 1, qq, None, 0.0, out, lse, ws, wsb), reps)
        quality = None
        if workload in ("c4", "c5"):                 # attention-visible error of 16 decode queries
            nqe = 16
            qe = torch.from_numpy(np.ascontiguousarray(q[:, lo:, :nqe]).view(np.int16)).to(dev)
            quality, _ = _quality(K, torch, dev, kq, vq, kp, vp, qe, None, Hq, nqe, shape)
            quality["queries"] = nqe
        if workload in ("c3v", "c3m"):               # attention-visible error of 16 queries
            nqe = 16
            qe = torch.from_numpy(np.ascontiguousarray(q[:, :, :nqe]).view(np.int16)).to(dev)
            kl = torch.empty((B, L, nqe, Hq), dtype=torch.float32, device=dev)
            re = torch.empty_like(kl)
            kv = torch.empty((B, L, H, 4), dtype=torch.float64, device=dev)
            web = K.kvq_attn_error_workspace(shape, Hq, nqe)
            we = torch.empty(max(web, 16), dtype=torch.uint8, device=dev)
            K.kvq_attn_error(kd, vd, kp, vp, Hq, nqe, qe, None, 0.0, kl, re, kv, we, web)
            torch.cuda.synchronize()
            kvn = kv.double().sum(dim=(0, 1, 2)).cpu().numpy()
            quality = {"mean_KL": float(kl.double().mean()), "p99_KL": float(torch.quantile(kl.double().flatten(), 0.99)),
                       "mean_out_relerr": float(re.double().mean()), "K_rel_sq_err": float(kvn[0] / kvn[1]),
                       "V_rel_sq_err": float(kvn[2] / kvn[3]), "queries": nqe}
            del we, kl, re, kv
        kw, ks, km = K.kvq_packed_layout(shape, kc)
        vw, vs, vm = K.kvq_packed_layout(shape, vc)
        kb = rows * (4 * kw + 2 * (ks + km))
        vb = rows * (D * 2 if vc.codebook == K.FP16 else 4 * vw + 2 * (vs + vm))
        q_bytes = rows * D * 2 * (1 if vc.codebook == K.FP16 else 2) + kb + (0 if vc.codebook == K.FP16 else vb)
        d_bytes = kb + vb
        anchor_bytes = (B * H * T * D * 2 * 2) if lo else 0
        step = t_d + anchor_s
        rec = {
            "workload": f"{workload}: B={B} L={L} H={H} T={T} D={D} Hq={Hq}" + (", layer 0 fp16" if lo else ""),
            "arm": name,
            "bits_per_value": round((K.kvq_bits_per_value(kc, D) + K.kvq_bits_per_value(vc, D)) / 2, 4),
            "quantize_pack": {"us": round(t_q * 1e6, 1), "GB/s": round(q_bytes / t_q / 1e9, 1),
                              "frac_hbm": round(q_bytes / t_q / 1e9 / HBM_PEAK_GBS, 4), "bytes": q_bytes},
            "decode_step": {"us": round(step * 1e6, 1), "tok/s": round(B / step, 1),
                            "GB/s": round((d_bytes + anchor_bytes) / step / 1e9, 1),
                            "frac_hbm": round((d_bytes + anchor_bytes) / step / 1e9 / HBM_PEAK_GBS, 4),
                            "bytes": d_bytes + anchor_bytes, "anchor_us": round(anchor_s * 1e6, 1)},
        }
        if quality:
            rec["quality"] = quality
        if workload == "c3m":
            rec["key_mean"] = {"subtracted": bool(use_mean), "kvq_key_mean_us": round(mean_us, 1),
                               "share_of_key_energy": w.k_mean_share}
        print(json.dumps(rec), flush=True)
        del kp, vp
        torch.cuda.empty_cache()


def _quality(K, torch, dev, k16, v16, kp, vp, qq, kv_len, Hq, nq, shape):
    """Attention-visible error of a packed cache against fp16 ([E21W] Benchmark): per-row
    KL and output error, per-unit K/V squared error over energy, and the ladder's other
    rungs, from kvq_attn_error_ex on the GPU; summaries as in the pages (means over rows
    and units, pooled energies)."""
    B, L = shape.batch, shape.layers
    rows = (B, L, nq, Hq)
    o = {k: torch.empty(rows, dtype=torch.float32, device=dev) for k in ("kl", "relerr", "renyi2", "js",
                                                                       "logit_relerr", "top1")}
    kv = torch.empty((B, L, shape.heads, 4), dtype=torch.float64, device=dev)
    wb = K.kvq_attn_error_workspace(shape, Hq, nq)
    ws = torch.empty(max(wb, 16), dtype=torch.uint8, device=dev)
    K.kvq_attn_error_ex(k16, v16, kp, vp, Hq, nq, qq, kv_len, 0.0, ws, wb, kv_err=kv, **o)
    torch.cuda.synchronize()
    a = {k: v.double().cpu().numpy() for k, v in o.items()}
    kvn = kv.double().cpu().numpy()
    unit = lambda i: np.where(kvn[..., i + 1] > 0, kvn[..., i] / np.maximum(kvn[..., i + 1], 1e-300), 0.0)
    return {"mean_KL": float(a["kl"].mean()), "p99_KL": float(np.quantile(a["kl"], 0.99)),
            "mean_out_relerr": float(a["relerr"].mean()), "mean_JS": float(a["js"].mean()),
            "mean_logit_relerr": float(a["logit_relerr"].mean()), "top1_flip_rate": float(a["top1"].mean()),
            "mean_renyi2_fp16": float(a["renyi2"].mean()),
            "K_rel_sq_err": float(kvn[..., 0].sum() / kvn[..., 1].sum()),
            "V_rel_sq_err": float(kvn[..., 2].sum() / kvn[..., 3].sum()) if kvn[..., 3].sum() > 0 else 0.0,
            "K_rel_sq_err_unit_mean": float(unit(0).mean()), "V_rel_sq_err_unit_mean": float(unit(2).mean()),
            "rows": int(np.prod(rows))}, a


def config_quality(workload):
    """c1 and c2: the quality reports these configurations ask for, at full size, from
    the GPU error kernel.

    c1 (tiny reference): K and V int4 min-max at group 32 with an fp16 scale and an fp16
    minimum per group, no rotation; 16 causal queries at positions in [256, 512), keys
    [0, p]; K/V squared error over signal energy, attention output error, KL.
    c2 (proxy-query probe, [E21W] What I tested and Result): arms A (min-max), B
    (Hadamard-256 then signed absmax), C (per-channel key scales calibrated on sequence
    0, then min-max) and D (the scales, then Hadamard then absmax; values Hadamard then
    absmax), each at 3 and 4 bits, group 32, on K and V; 128 proxy queries per sequence
    and layer (the keys at positions in [3000, 6000)) attending the keys before them;
    attention error and KL per sequence."""
    import torch
    import kv_cache_bit_fwht_amd as K
    import synth
    dev = torch.device("cuda:0")
    w = synth.get(workload)
    log(f"generating {w.description}")
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w, Kx)
    B, L, H, T, D, Hq, nq = w.B, w.L, w.H, w.T, w.D, w.Hq, w.n_q
    shape = K.Shape(B, L, H, T, D)
    kd = torch.from_numpy(Kx.view(np.int16)).to(dev)
    vd = torch.from_numpy(Vx.view(np.int16)).to(dev)
    qd = torch.from_numpy(q.view(np.int16)).to(dev)
    kvl = torch.from_numpy(kv_len).to(dev)
    A, MM = K.INT_ABSMAX, K.INT_MINMAX
    if workload == "c1":
        arms = {"K, V int4 min-max g32 (fp16 scale and min), no rotation": (K.Codec(MM, 4, 32, 0),
                                                                            K.Codec(MM, 4, 32, 0), False)}
    else:
        arms = {}
        for b in (3, 4):
            arms[f"A: min-max, {b}-bit g32"] = (K.Codec(MM, b, 32, 0), K.Codec(MM, b, 32, 0), False)
            arms[f"B: Hadamard-256 + signed absmax, {b}-bit g32"] = (K.Codec(A, b, 32, 256), K.Codec(A, b, 32, 256),
                                                                    False)
            arms[f"C: K channel scales + min-max, {b}-bit g32"] = (K.Codec(MM, b, 32, 0), K.Codec(MM, b, 32, 0), True)
            arms[f"D: K channel scales + Hadamard-256 + absmax, {b}-bit g32"] = (K.Codec(A, b, 32, 256),
                                                                             K.Codec(A, b, 32, 256), True)
    chan = None
    if any(a[2] for a in arms.values()):
        chan = torch.empty((L, H, D), dtype=torch.float32, device=dev)
        K.kvq_calibrate_chan_scale(kd[:1].contiguous(), K.Shape(1, L, H, T, D), chan)
    for name, (kc, vc, pre) in arms.items():
        kp = K.alloc_packed(kc, shape, dev, chan_scale=chan if pre else None)
        vp = K.alloc_packed(vc, shape, dev)
        K.kvq_quantize_pack_kv(kd, vd, kp, vp)
        summ, a = _quality(K, torch, dev, kd, vd, kp, vp, qd, kvl, Hq, nq, shape)
        rec = {"workload": f"{workload}: B={B} L={L} H={H} T={T} D={D} Hq={Hq}, {nq} queries per sequence and layer"
                           + (" (proxy queries: the keys at positions in [3000, 6000), keys before them)"
                              if workload == "c2" else " at positions in [256, 512), keys [0, p]"),
               "arm": name,
               "bits_per_value": round((K.kvq_bits_per_value(kc, D) + K.kvq_bits_per_value(vc, D)) / 2, 4),
               "quality": summ}
        if B > 1:
            rec["per_sequence"] = {"mean_out_relerr": [round(float(a["relerr"][b].mean()), 5) for b in range(B)],
                                   "mean_KL": [round(float(a["kl"][b].mean()), 6) for b in range(B)]}
            if workload == "c2":
                rec["per_sequence"]["note"] = "sequence 0 is the channel-scale calibration sequence"
        print(json.dumps(rec), flush=True)
        del kp, vp
        torch.cuda.empty_cache()


def anchors_workload(reps):
    """c3a: the 64K cache in a decoding loop ([FMAG-6] The winning recipe, Selective-Layer
    Decode Anchoring).  Tokens [0, 65472) of every layer in the 4-bit-key / 2-bit-value
    codec; the next 48 (the first decoded tokens) at fp16 on layers 0-3 and in the
    same 4/2 codec on layers 4-7; the last 16 in 4/2 everywhere.  Times the append of
    one decoded token (K and V of every layer and head into the packed cache) and one
    decode step over the four segments, against the decode of the same cache held as
    one packed tensor; the append followed by the decode, as two launches and as one
    (kvq_append_decode_attn); reports the effective bits.  Times are per call over 100
    back-to-back calls."""
    import torch
    import kv_cache_bit_fwht_amd as K
    import synth
    dev = torch.device("cuda:0")
    w = synth.get("c3")
    log(f"generating {w.description}")
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    B, L, H, T, D, Hq = w.B, w.L, w.H, w.T, w.D, w.Hq
    P, A = 65472, 48
    kc, vc, f16 = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0), K.Codec(K.FP16)
    qd = torch.from_numpy(np.ascontiguousarray(q[:, :, :1]).view(np.int16)).to(dev)

    def part(x, l0, nl, t0, nt, codec):
        sub = torch.from_numpy(np.ascontiguousarray(x[:, l0:l0 + nl, :, t0:t0 + nt]).view(np.int16)).to(dev)
        shape = K.Shape(B, nl, H, nt, D)
        if codec.codebook == K.FP16:
            return K.packed_from_fp16(sub, shape)
        p = K.alloc_packed(codec, shape, dev)
        K.kvq_quantize_pack(sub, p)
        return p

    layout = [(0, L, 0, P, kc, vc), (0, 4, P, A, f16, f16), (0, 4, P + A, T - P - A, kc, vc),
              (4, L - 4, P, T - P, kc, vc)]
    segs = [K.Segment(part(Kx, l0, nl, t0, nt, ck), part(Vx, l0, nl, t0, nt, cv), l0, t0)
            for (l0, nl, t0, nt, ck, cv) in layout]
    shape = K.Shape(B, L, H, T, D)
    kfull, vfull = K.alloc_packed(kc, shape, dev), K.alloc_packed(vc, shape, dev)
    K.kvq_quantize_pack(torch.from_numpy(Kx.view(np.int16)).to(dev), kfull)
    K.kvq_quantize_pack(torch.from_numpy(Vx.view(np.int16)).to(dev), vfull)
    newk = torch.from_numpy(np.ascontiguousarray(Kx[:, :, :, T - 1:T]).view(np.int16)).to(dev)
    newv = torch.from_numpy(np.ascontiguousarray(Vx[:, :, :, T - 1:T]).view(np.int16)).to(dev)
    del Kx, Vx
    out = torch.empty((B, L, 1, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, L, 1, Hq), dtype=torch.float32, device=dev)
    wsb = K.kvq_decode_attn_segments_workspace(segs, L, H, Hq, 1)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    wsb1 = K.kvq_decode_attn_workspace(shape, Hq, 1)
    ws1 = torch.zeros(wsb1, dtype=torch.uint8, device=dev)

    def seg_step():
        K.kvq_decode_attn_segments(segs, L, H, T, Hq, 1, qd, None, 0.0, out, lse, ws, wsb)

    def one_step():
        K.kvq_decode_attn(kfull, vfull, Hq, 1, qd, None, 0.0, out, lse, ws1, wsb1)

    def append():
        K.kvq_quantize_pack_tokens_kv(newk, newv, T - 1, 1, kfull, vfull)

    def append_then_decode():
        append()
        one_step()

    def append_decode():
        K.kvq_append_decode_attn(newk, newv, T - 1, 1, kfull, vfull, Hq, 1, qd, None, 0.0, out, lse, ws1, wsb1)

    for f in (seg_step, one_step, append, append_decode):
        f()
    torch.cuda.synchronize()
    # per call, over 100 back-to-back calls (a decoding loop issues its steps that way);
    # the median of the passes
    t_seg = _median_time(torch, lambda: [seg_step() for _ in range(100)], reps) / 100
    t_one = _median_time(torch, lambda: [one_step() for _ in range(100)], reps) / 100
    t_app = _median_time(torch, lambda: [append() for _ in range(100)], reps) / 100
    t_atd = _median_time(torch, lambda: [append_then_decode() for _ in range(100)], reps) / 100
    t_ad = _median_time(torch, lambda: [append_decode() for _ in range(100)], reps) / 100
    eff = K.kvq_effective_bits(segs, L, H, T)
    d_bytes = sum(s.k.codes.numel() * 4 + (s.k.scales.numel() * 2 if s.k.scales is not None else 0) +
                  s.v.codes.numel() * 4 + (s.v.scales.numel() * 2 if s.v.scales is not None else 0) for s in segs)
    rec = {"workload": f"c3a: B={B} L={L} H={H} T={T} D={D} Hq={Hq}, prompt {P} + {A} decode anchors fp16 on "
                       f"layers 0-3 + {T - P - A} tokens, K int4 FWHT-256 g128 / V int2 g128 elsewhere",
           "segments": len(segs), "effective_bits": round(eff, 4),
           "decode_step_segments": {"us": round(t_seg * 1e6, 1), "tok/s": round(B / t_seg, 1),
                                    "GB/s": round(d_bytes / t_seg / 1e9, 1),
                                    "frac_hbm": round(d_bytes / t_seg / 1e9 / HBM_PEAK_GBS, 4), "bytes": d_bytes},
           "decode_step_one_tensor": {"us": round(t_one * 1e6, 1)},
           "append_one_token_kv": {"us": round(t_app * 1e6, 1), "rows": 2 * B * L * H},
           "append_then_decode_two_launches": {"us": round(t_atd * 1e6, 1)},
           "append_decode_one_launch": {"us": round(t_ad * 1e6, 1),
                                        "over_decode_alone": round(t_ad / t_one - 1.0, 4)}}
    print(json.dumps(rec), flush=True)


def _round_keep_sum(b, lo=2, hi=8):
    """Integer bits from fractional ones, keeping their sum (largest remainders first)."""
    fl = np.clip(np.floor(b), lo, hi).astype(int)
    need = int(round(float(np.sum(b)))) - int(fl.sum())
    order = np.argsort(-(b - np.floor(b)), kind="stable")
    for h in order[:max(need, 0)]:
        fl[h] = min(fl[h] + 1, hi)
    return fl


def entropy_workload(reps):
    """c3h: per-head key bits from attention entropy ([LCPP] Finding 2: b_h = b_avg +
    0.25 (H_avg - H_2(h)), and the per-head KV-type request).  The 64K cache with
    per-head key scales (3, 1, 1, 0.5), so one head attends sharply and one diffusely;
    H_2 per KV head from 8 calibration queries (kvq_attn_error_ex on the fp16 cache);
    bits by the rule at an average of 4, rounded keeping the sum; keys of each head
    coded at its bits (FWHT-256, g128) as head segments, values int4 g128.  Compared
    with uniform 4-bit keys: attention KL of 16 queries, and one decode step (the
    head segments decoded as one codec-map launch and as a launch per segment)."""
    import torch
    import kv_cache_bit_fwht_amd as K
    import synth
    dev = torch.device("cuda:0")
    w = synth.get("c3", k_head_scales=(3.0, 1.0, 1.0, 0.5))
    log(f"generating {w.description} with per-head key scales {w.k_head_scales}")
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    B, L, H, T, D, Hq = w.B, w.L, w.H, w.T, w.D, w.Hq
    G = Hq // H
    shape = K.Shape(B, L, H, T, D)
    kd = torch.from_numpy(Kx.view(np.int16)).to(dev)
    vd = torch.from_numpy(Vx.view(np.int16)).to(dev)
    nqc, nqe = 8, 16
    qc = torch.from_numpy(np.ascontiguousarray(q[:, :, nqe:nqe + nqc]).view(np.int16)).to(dev)
    qe = torch.from_numpy(np.ascontiguousarray(q[:, :, :nqe]).view(np.int16)).to(dev)
    # calibration: Renyi-2 entropy of the fp16 attention of each head
    f16k, f16v = K.packed_from_fp16(kd, shape), K.packed_from_fp16(vd, shape)
    h2 = torch.empty((B, L, nqc, Hq), dtype=torch.float32, device=dev)
    web = K.kvq_attn_error_workspace(shape, Hq, nqc)
    we = torch.empty(web, dtype=torch.uint8, device=dev)
    K.kvq_attn_error_ex(kd, vd, f16k, f16v, Hq, nqc, qc, None, 0.0, we, web, renyi2=h2)
    torch.cuda.synchronize()
    del we
    h2_head = h2.double().cpu().numpy().reshape(B, L, nqc, H, G).mean(axis=(0, 1, 2, 4))
    b_avg = 4.0
    frac = b_avg + 0.25 * (h2_head.mean() - h2_head)
    bits = _round_keep_sum(frac)
    vc = K.Codec(K.INT_ABSMAX, 4, 128, 0)

    def quality(kp, vp, k16, v16, qq, hq):
        kl = torch.empty((B, L, nqe, hq), dtype=torch.float32, device=dev)
        js = torch.empty_like(kl)
        sh = kp.shape
        wb = K.kvq_attn_error_workspace(sh, hq, nqe)
        wsp = torch.empty(wb, dtype=torch.uint8, device=dev)
        K.kvq_attn_error_ex(k16, v16, kp, vp, hq, nqe, qq, None, 0.0, wsp, wb, kl=kl, js=js)
        torch.cuda.synchronize()
        return kl.double().cpu().numpy(), js.double().cpu().numpy()

    out = torch.empty((B, L, 1, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, L, 1, Hq), dtype=torch.float32, device=dev)
    q1 = qe[:, :, :1].contiguous()
    recs = []
    # uniform 4-bit keys
    ku = K.alloc_packed(K.Codec(K.INT_ABSMAX, 4, 128, 256), shape, dev)
    vu = K.alloc_packed(vc, shape, dev)
    K.kvq_quantize_pack(kd, ku)
    K.kvq_quantize_pack(vd, vu)
    klu, jsu = quality(ku, vu, kd, vd, qe, Hq)
    wsb = K.kvq_decode_attn_workspace(shape, Hq, 1)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    fn = lambda: K.kvq_decode_attn(ku, vu, Hq, 1, q1, None, 0.0, out, lse, ws, wsb)
    fn()
    tu = _median_time(torch, fn, reps)
    recs.append(("K int4 FWHT-256 g128, every head", [4] * H, klu, jsu, tu,
                 K.kvq_bits_per_value(K.Codec(K.INT_ABSMAX, 4, 128, 256), D)))
    del ku
    # entropy-adaptive keys: one segment per head
    segs, kls, jss = [], np.zeros_like(klu), np.zeros_like(jsu)
    for h in range(H):
        sub = K.Shape(B, L, 1, T, D)
        k16 = kd[:, :, h:h + 1].contiguous()
        v16 = vd[:, :, h:h + 1].contiguous()
        kp = K.alloc_packed(K.Codec(K.INT_ABSMAX, int(bits[h]), 128, 256), sub, dev)
        vp = K.alloc_packed(vc, sub, dev)
        K.kvq_quantize_pack(k16, kp)
        K.kvq_quantize_pack(v16, vp)
        klh, jsh = quality(kp, vp, k16, v16, qe[:, :, :, h * G:(h + 1) * G].contiguous(), G)
        kls[..., h * G:(h + 1) * G] = klh
        jss[..., h * G:(h + 1) * G] = jsh
        segs.append(K.Segment(kp, vp, 0, 0, h))
    wsb = K.kvq_decode_attn_segments_workspace(segs, L, H, Hq, 1)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    kb = sum(K.kvq_bits_per_value(sg.k.codec, D) for sg in segs) / H
    for path, how in ((2, "one launch for the codec map"), (1, "a launch per head segment")):
        fn = lambda: K.kvq_decode_attn_segments(segs, L, H, T, Hq, 1, q1, None, 0.0, out, lse, ws, wsb, path=path)
        fn()
        ta = _median_time(torch, fn, reps)
        recs.append((f"K bits per head by b_h = 4 + 0.25 (H_avg - H_2(h)), head segments, {how}",
                     [int(b) for b in bits], kls, jss, ta, kb))
    for name, bh, kl, js, t, kbits in recs:
        print(json.dumps({
            "workload": f"c3h: B={B} L={L} H={H} T={T} D={D} Hq={Hq}, per-head key scales {list(w.k_head_scales)}, "
                        f"V int4 g128",
            "arm": name, "H2_per_kv_head": [round(float(x), 3) for x in h2_head],
            "rule_bits": [round(float(x), 3) for x in frac], "key_bits_per_head": bh,
            "key_bits_per_value": round(kbits, 4),
            "quality": {"mean_KL": float(kl.mean()), "p99_KL": float(np.quantile(kl, 0.99)),
                        "mean_KL_per_kv_head": [float(kl[..., h * G:(h + 1) * G].mean()) for h in range(H)],
                        "mean_JS": float(js.mean()), "queries": nqe},
            "decode_step_us": round(t * 1e6, 1)}), flush=True)


# [E21W] Result: the 3.19-bit allocation (rotated, groups of 128): 2-bit keys on layers
# 2 and 7, 4-bit values on layers 1, 3 and 4, 3 bits everywhere else
ALLOC_K_BITS = (3, 3, 2, 3, 3, 3, 3, 2)
ALLOC_V_BITS = (3, 4, 3, 4, 4, 3, 3, 3)


def allocation_workload(reps):
    """c2a: the per-layer K/V bit allocation of [E21W] Result against rotated 4-bit and
    3-bit caches at group 32 ([E21W] What I tested, variant B at 3 and 4 bits), on the
    proxy-query probe shape (3 sequences x 8 layers x 4 KV heads x 6,000 tokens x 256;
    queries are the keys at 128 positions in [3,000, 6,000), each attending the keys
    before it).  Per sequence: mean attention output error and attention KL
    (kvq_attn_error_ex).  Decode: one call over all 3 x 128 queries, the allocation as one
    codec-map launch and as a launch per layer segment."""
    import torch
    import kv_cache_bit_fwht_amd as K
    import synth
    dev = torch.device("cuda:0")
    w = synth.get("c2")
    log(f"generating {w.description}")
    Kx, Vx = synth.gen_kv(w)
    q, kv_len = synth.gen_queries(w, Kx)
    B, L, H, T, D, Hq, nq = w.B, w.L, w.H, w.T, w.D, w.Hq, w.n_q
    kd = torch.from_numpy(Kx.view(np.int16)).to(dev)
    vd = torch.from_numpy(Vx.view(np.int16)).to(dev)
    qd = torch.from_numpy(q.view(np.int16)).to(dev)
    kvl = torch.from_numpy(kv_len).to(dev)
    A = K.INT_ABSMAX

    def errors(kp, vp, k16, v16, qq, kl_len, nl):
        kl = torch.empty((B, nl, nq, Hq), dtype=torch.float32, device=dev)
        re = torch.empty_like(kl)
        wb = K.kvq_attn_error_workspace(kp.shape, Hq, nq)
        wsp = torch.empty(wb, dtype=torch.uint8, device=dev)
        K.kvq_attn_error_ex(k16, v16, kp, vp, Hq, nq, qq, kl_len, 0.0, wsp, wb, kl=kl, relerr=re)
        torch.cuda.synchronize()
        return kl.double().cpu().numpy(), re.double().cpu().numpy()

    out = torch.empty((B, L, nq, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, L, nq, Hq), dtype=torch.float32, device=dev)
    recs = []
    shape = K.Shape(B, L, H, T, D)
    for name, bits in (("rotated 4-bit g32 (variant B, q4_0-like)", 4), ("rotated 3-bit g32 (variant B)", 3)):
        c = K.Codec(A, bits, 32, 256)
        kp, vp = K.alloc_packed(c, shape, dev), K.alloc_packed(c, shape, dev)
        K.kvq_quantize_pack(kd, kp)
        K.kvq_quantize_pack(vd, vp)
        kl, re = errors(kp, vp, kd, vd, qd, kvl, L)
        wsb = K.kvq_decode_attn_workspace(shape, Hq, nq)
        ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
        fn = lambda: K.kvq_decode_attn(kp, vp, Hq, nq, qd, kvl, 0.0, out, lse, ws, wsb)
        fn()
        t = _median_time(torch, fn, reps)
        recs.append((name, [bits] * L, [bits] * L, K.kvq_bits_per_value(c, D), kl, re, {"decode_us": t}))
        del kp, vp, ws
    # the allocation: one segment per run of layers with the same (key bits, value bits)
    runs, l0 = [], 0
    for l in range(1, L + 1):
        if l == L or (ALLOC_K_BITS[l], ALLOC_V_BITS[l]) != (ALLOC_K_BITS[l0], ALLOC_V_BITS[l0]):
            runs.append((l0, l - l0))
            l0 = l
    segs, kl, re = [], np.zeros((B, L, nq, Hq)), np.zeros((B, L, nq, Hq))
    bpv = 0.0
    for l0, nl in runs:
        sub = K.Shape(B, nl, H, T, D)
        kc, vc = K.Codec(A, ALLOC_K_BITS[l0], 128, 256), K.Codec(A, ALLOC_V_BITS[l0], 128, 256)
        k16 = kd[:, l0:l0 + nl].contiguous()
        v16 = vd[:, l0:l0 + nl].contiguous()
        kp, vp = K.alloc_packed(kc, sub, dev), K.alloc_packed(vc, sub, dev)
        K.kvq_quantize_pack(k16, kp)
        K.kvq_quantize_pack(v16, vp)
        kls, res = errors(kp, vp, k16, v16, qd[:, l0:l0 + nl].contiguous(), kvl[:, l0:l0 + nl].contiguous(), nl)
        kl[:, l0:l0 + nl], re[:, l0:l0 + nl] = kls, res
        bpv += nl * (K.kvq_bits_per_value(kc, D) + K.kvq_bits_per_value(vc, D)) / 2
        segs.append(K.Segment(kp, vp, l0, 0, 0))
    wsb = K.kvq_decode_attn_segments_workspace(segs, L, H, Hq, nq)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    times = {}
    for path, key in ((2, "decode_us"), (1, "decode_us_per_segment_launches")):
        fn = lambda: K.kvq_decode_attn_segments(segs, L, H, T, Hq, nq, qd, kvl, 0.0, out, lse, ws, wsb, path=path)
        fn()
        times[key] = _median_time(torch, fn, reps)
    recs.append((f"3.19-bit allocation, {len(runs)} layer segments", list(ALLOC_K_BITS), list(ALLOC_V_BITS), bpv / L,
                 kl, re, times))
    for name, kb, vb, bpv, kl, re, t in recs:
        print(json.dumps({
            "workload": f"c2a: B={B} L={L} H={H} T={T} D={D} Hq={Hq}, {nq} proxy queries per sequence and layer "
                        f"(keys at positions in [3000, 6000), causal)",
            "arm": name, "key_bits_per_layer": kb, "value_bits_per_layer": vb, "bits_per_value": round(bpv, 4),
            "attention_error_per_sequence": [round(float(re[b].mean()), 4) for b in range(B)],
            "KL_per_sequence": [round(float(kl[b].mean()), 5) for b in range(B)],
            **{k: round(v * 1e6, 1) for k, v in t.items()}}), flush=True)


TIMELINE_SLOTS = ["entry", "query prologue done", "after prologue barrier", "loop end", "wavefront reduced",
                  "after block barrier", "partial stores issued", "partial stores complete", "block counted",
                  "last block: merge tables in", "merge end"]


def decode_timeline(K, torch, call, w):
    """One decode call on the profiling build: the clock stamps of every wavefront
    ([block][wave][slot], 100 MHz), as percentiles per slot from the first entry, and the
    spreads that make the fixed cost of a call."""
    n = 4096 * 8 * 16
    K.kvq_timeline_read(n)                             # clears what the warm-up left
    call()
    torch.cuda.synchronize()
    ts = K.kvq_timeline_read(n).reshape(4096, 8, 16).astype(np.int64)
    used = ts[:, :, 0] > 0
    nblk = int(used.any(axis=1).sum())
    if nblk == 0:
        raise RuntimeError("no stamps: the call did not take the MFMA decode")
    ts = ts[:nblk]
    t0 = ts[:, :, 0][ts[:, :, 0] > 0].min()
    us = lambda x: (x - t0) * 0.01                     # 100 MHz clock
    units = int((ts[:, 0, 10] > 0).sum())             # one merging block per unit
    bpu = nblk // max(units, 1)
    pct = lambda v: {"min": round(float(np.min(v)), 2), "p10": round(float(np.percentile(v, 10)), 2),
                     "p50": round(float(np.percentile(v, 50)), 2), "p90": round(float(np.percentile(v, 90)), 2),
                     "max": round(float(np.max(v)), 2)}
    slots = {}
    for i, name in enumerate(TIMELINE_SLOTS):
        v = ts[:, :, i][ts[:, :, i] > 0]
        if v.size:
            slots[name] = dict(pct(us(v)), n=int(v.size))
    loop_end = us(ts[:, :, 3])                         # [block][wave]
    wave_spread = loop_end.max(axis=1) - loop_end.min(axis=1)
    blk_end = loop_end.max(axis=1).reshape(units, bpu)
    merge_end = us(ts[:, :, 10].max(axis=1)).reshape(units, bpu).max(axis=1)
    rec = {"timeline": "64K decode, one call, per-wavefront s_memrealtime stamps (us from the first entry)",
           "blocks": nblk, "units": units, "blocks_per_unit": bpu, "slots": slots,
           "wave_loop_end_spread_in_block_us": pct(wave_spread),
           "block_loop_end_spread_in_unit_us": pct(blk_end.max(axis=1) - blk_end.min(axis=1)),
           "merge_end_after_unit_last_loop_end_us": pct(merge_end - blk_end.max(axis=1)),
           "kernel_span_us": round(float(us(ts[ts > 0].max())), 2)}
    for name, v in slots.items():
        log(f"{name:30s} n={v['n']:5d} min {v['min']:7.2f} p10 {v['p10']:7.2f} p50 {v['p50']:7.2f} "
            f"p90 {v['p90']:7.2f} max {v['max']:7.2f} us")
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--decode-queries", type=int, default=256)
    ap.add_argument("--path", type=int, default=0, help="decode kernel: 0 auto, 1 general, 2 MFMA")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--profile", action="store_true",
                    help="short run for hardware-counter passes: a known-size copy (the counters' "
                         "calibration), one quantize+pack pair and --decode-queries decode calls")
    ap.add_argument("--workload", default="c3", choices=["c3", "c1", "c2", "c4", "c5", "c3v", "c3m", "c3a", "c3h", "c2a"],
                    help="c3: the headline line (default); c1/c2: the quality reports of the tiny reference and "
                         "of the proxy-query probe's arms A-D at 3 and 4 bits; c4/c5: one line per codec arm of "
                         "those configs, with throughput and the attention error and KL of 16 decode queries; "
                         "c3v: the 64K cache with each value codebook, with attention KL; "
                         "c3m: the 64K cache with a shared key mean, keys coded with and without it; "
                         "c3a: the 64K cache as decode segments with fp16 anchors, and the append path; "
                         "c3h: per-head key bits from attention entropy, as head segments; "
                         "c2a: the per-layer 3.19-bit allocation on the proxy-query probe")
    ap.add_argument("--reps", type=int, default=5, help="timed repetitions per arm (c4/c5)")
    ap.add_argument("--timeline", action="store_true",
                    help="c3 only: load the profiling build (libkvq_timeline.so, from build.py --timeline), "
                         "run one 64K decode call and print its per-wavefront clock timeline instead of the "
                         "bench line")
    ap.add_argument("--tokens", type=int, default=None,
                    help="c3 only: tokens per (layer, KV head) instead of 65,536 (a multiple of 32), to see how "
                         "the per-call fixed costs amortise; the headline line is the default")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(see DESIGN.md for how the path would shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.workload in ("c1", "c2"):
        config_quality(args.workload)
        return
    if args.workload == "c3a":
        anchors_workload(args.reps)
        return
    if args.workload == "c3h":
        entropy_workload(args.reps)
        return
    if args.workload == "c2a":
        allocation_workload(args.reps)
        return
    if args.workload != "c3":
        secondary(args.workload, args.reps)
        return

    if args.timeline:
        os.environ["KVQ_TIMELINE"] = "1"
    import torch
    import kv_cache_bit_fwht_amd as K
    import synth

    dev = torch.device("cuda:0")
    w = synth.get("c3") if args.tokens is None else synth.get("c3", T=args.tokens)
    nq = min(args.decode_queries, w.n_q)
    log(f"generating {w.description}")
    Kx, Vx = synth.gen_kv(w)
    q, _ = synth.gen_queries(w)
    shape = K.Shape(w.B, w.L, w.H, w.T, w.D)
    kc, vc = K.Codec(K.INT_ABSMAX, 4, 128, 256), K.Codec(K.INT_ABSMAX, 2, 128, 0)
    kd = torch.from_numpy(Kx.view(np.int16)).to(dev)
    vd = torch.from_numpy(Vx.view(np.int16)).to(dev)
    # one contiguous [B][L][1][Hq][D] query per decode step
    qs = np.ascontiguousarray(q.transpose(2, 0, 1, 3, 4)[:nq, :, :, None])
    qd = torch.from_numpy(qs.view(np.int16)).to(dev)
    copies = [(K.alloc_packed(kc, shape, dev), K.alloc_packed(vc, shape, dev)) for _ in range(args.copies)]
    out = torch.empty((w.B, w.L, 1, w.Hq, w.D), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.L, 1, w.Hq), dtype=torch.float32, device=dev)
    wsb = K.kvq_decode_attn_workspace(shape, w.Hq, 1)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    for kp, vp in copies:
        K.kvq_quantize_pack_kv(kd, vd, kp, vp)
    torch.cuda.synchronize()

    if args.profile:
        # 1 GiB device-to-device copy of known size: FETCH_SIZE / WRITE_SIZE of this kernel
        # calibrate the counters (expected 1 GiB read and 1 GiB written)
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        kp, vp = copies[0]
        K.kvq_quantize_pack_kv(kd, vd, kp, vp)
        for i in range(nq):
            kp2, vp2 = copies[i % len(copies)]
            K.kvq_decode_attn(kp2, vp2, w.Hq, 1, qd[i], None, 0.0, out, lse, ws, wsb, None,
                              args.path or None)
        torch.cuda.synchronize()
        log("profile run done")
        return

    rows = w.B * w.L * w.H * w.T
    q_bytes = rows * (w.D * 2) * 2 + rows * (w.D * 4 // 8 + 2 * 2) + rows * (w.D * 2 // 8 + 2 * 2)
    d_bytes = rows * (w.D * 4 // 8 + 2 * 2 + w.D * 2 // 8 + 2 * 2)
    step_idx = [0]

    sh = stream.cuda_stream
    path = args.path or None
    # raw device addresses, so the per-call host work is only argument marshalling
    q_ptrs = [qd[i].data_ptr() for i in range(nq)]
    out_p, lse_p, ws_p = out.data_ptr(), lse.data_ptr(), ws.data_ptr()

    def step(ev):
        """One step; ev = (start, after quantise, after the decode calls) events or None."""
        c = step_idx[0] % len(copies)
        step_idx[0] += 1
        kp, vp = copies[c]
        if ev:
            ev[0].record(stream)
        K.kvq_quantize_pack_kv(kd, vd, kp, vp, sh)
        if ev:
            ev[1].record(stream)
        for i in range(nq):
            kp2, vp2 = copies[(c + i) % len(copies)]
            K.kvq_decode_attn(kp2, vp2, w.Hq, 1, q_ptrs[i], None, 0.0, out_p, lse_p, ws_p, wsb, sh, path)
        if ev:
            ev[2].record(stream)

    log(f"warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    if args.timeline:
        decode_timeline(K, torch, lambda: K.kvq_decode_attn(copies[0][0], copies[0][1], w.Hq, 1, q_ptrs[0], None,
                                                           0.0, out_p, lse_p, ws_p, wsb, sh, path), w)
        return
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"timing {args.steps} step(s) of quantize+pack + {nq} decode calls")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for s_ in range(args.steps):
        step(evs[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = evs[0][0].elapsed_time(evs[-1][2])
    ms_step = total_ms / args.steps
    qz_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dc_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) / nq
    log(f"step {ms_step:.3f} ms (wall {wall / args.steps * 1e3:.1f} ms); quantize {qz_ms * 1e3:.1f} us; "
        f"decode {dc_ms * 1e3:.1f} us per call")

    ceil = measure_ceilings(torch, dev)
    value = nq * w.B / (ms_step * 1e-3)
    dec_gbs = d_bytes / (dc_ms * 1e-3) / 1e9
    qz_gbs = q_bytes / (qz_ms * 1e-3) / 1e9
    rec_line = {
        "metric": "quantize+pack GB/s and packed decode-attn tok/s @64K; % of HBM peak",
        "value": round(value, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "decode: int8 MFMA for QK (exact integer sums), fp16 MFMA for PV with fp32 accumulation; codec: fp32",
        "data": "synthetic (seeded fp16 K/V with outlier channels, N(0,1) queries)",
        "config": {"workload": f"{'64K' if w.T == 65536 else str(w.T)} decode: B=1 L=8 H=4 T={w.T} D=256, Hq=16 (GQA 4:1), "
                               "K FWHT-256 int4 absmax g128, V int2 absmax g128 (3.125 bpv), "
                               f"{nq} decode queries per step",
                   "decode_calls_per_step": nq, "packed_cache_copies": len(copies),
                   "decode_path": {0: "auto", 1: "general", 2: "mfma"}[args.path]},
        "quantize_pack": {"GB/s": round(qz_gbs, 1), "frac_hbm": round(qz_gbs / HBM_PEAK_GBS, 4),
                          "frac_copy_ceiling": round(qz_gbs / ceil["copy_GBps"], 4),
                          "us_per_call_pair": round(qz_ms * 1e3, 2), "bytes": q_bytes},
        "decode": {"tok/s": round(1e3 / dc_ms, 1), "us_per_token": round(dc_ms * 1e3, 2),
                   "GB/s": round(dec_gbs, 1), "frac_hbm": round(dec_gbs / HBM_PEAK_GBS, 4),
                   "frac_copy_ceiling": round(dec_gbs / ceil["copy_GBps"], 4),
                   "bytes_per_launch": d_bytes},
        "ceilings": ceil,
        "roofline": {"bound": "hbm", "kernel": "kvq_decode_attn", "achieved": round(dec_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     # the counters were read on the 64K workload
                     "traffic": traffic_for("decode", 1) if w.T == 65536 else None},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        rec_line["cpu_baseline"] = cpu_baseline(Kx, Vx, q)
    print(json.dumps(rec_line), flush=True)


if __name__ == "__main__":
    main()

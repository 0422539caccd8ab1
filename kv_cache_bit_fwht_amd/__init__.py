"""Python binding of libkvq (MI355X / gfx950 group-wise low-bit KV-cache codec and
packed decode attention).

Argument marshalling only: every function here forwards to the C entry point of
the same name in ``libkvq.so`` (declared in ``include/kvq.h``); all computation
runs in the HIP kernels.  PyTorch supplies device memory (``tensor.data_ptr()``)
and the current stream.  Importing this package fails loudly if the library has
not been built; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_TIMELINE=1 selects the profiling build (per-wavefront clock stamps in the MFMA
# decode, kvq_timeline_read); the results are the same
LIB_PATH = os.path.join(_HERE, "libkvq_timeline.so" if os.environ.get("KVQ_TIMELINE") == "1" else "libkvq.so")

# codebooks (kvq_codebook)
FP16, INT_ABSMAX, INT_MINMAX, TERNARY, SIGN, NF4, INT8_SYM, RFFT_POLAR, RFFT_CART, INT_SYM, LLOYD = range(11)

STATUS = {0: "KVQ_OK", -1: "KVQ_ERR_ARG", -2: "KVQ_ERR_UNSUPPORTED", -3: "KVQ_ERR_ALIGN",
          -4: "KVQ_ERR_WORKSPACE", -5: "KVQ_ERR_HIP"}

EXPORTS = [
    "kvq_status_string", "kvq_version", "kvq_packed_layout", "kvq_bits_per_value",
    "kvq_constant_table", "kvq_calibrate_chan_scale", "kvq_key_mean_workspace", "kvq_key_mean",
    "kvq_quantize_pack", "kvq_dequant",
    "kvq_decode_attn_workspace", "kvq_decode_attn", "kvq_decode_attn_ex",
    "kvq_attn_error_workspace", "kvq_attn_error", "kvq_quantize_pack_tokens",
    "kvq_decode_attn_segments_workspace", "kvq_decode_attn_segments", "kvq_decode_attn_segments_ex",
    "kvq_effective_bits",
    "kvq_attn_error_ex", "kvq_quantize_pack_kv", "kvq_quantize_pack_tokens_kv", "kvq_decode_attn_static",
    "kvq_append_decode_attn",
]


class KvqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")


class kvq_codec(ctypes.Structure):
    _fields_ = [("codebook", ctypes.c_int32), ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("rot_width", ctypes.c_int32), ("aux_bits", ctypes.c_int32)]


class kvq_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("layers", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("tokens", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class kvq_packed(ctypes.Structure):
    _fields_ = [("codec", kvq_codec), ("shape", kvq_shape), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("mins", ctypes.c_void_p), ("chan_scale", ctypes.c_void_p),
                ("mean", ctypes.c_void_p)]


class kvq_error_outputs(ctypes.Structure):
    _fields_ = [("kl", ctypes.c_void_p), ("relerr", ctypes.c_void_p), ("kv_err", ctypes.c_void_p),
                ("renyi2", ctypes.c_void_p), ("js", ctypes.c_void_p), ("logit_relerr", ctypes.c_void_p),
                ("top1", ctypes.c_void_p)]


class kvq_segment(ctypes.Structure):
    _fields_ = [("k", ctypes.POINTER(kvq_packed)), ("v", ctypes.POINTER(kvq_packed)),
                ("layer0", ctypes.c_int32), ("token0", ctypes.c_int32), ("head0", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m kv_cache_bit_fwht_amd.build` "
                          "(or __graft_entry__.build()); there is no CPU fallback")
    # torch (the device-memory and stream provider) ships its own HIP runtime; loading it
    # first makes this library bind to that same runtime instead of a second copy from
    # the ROCm install, whose kernels could not use torch's allocations
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, F, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float, ctypes.c_double
    sig = {
        "kvq_status_string": ([I32], ctypes.c_char_p),
        "kvq_version": ([], ctypes.c_char_p),
        "kvq_packed_layout": ([P, P, P, P, P], I32),
        "kvq_bits_per_value": ([P, I32], D),
        "kvq_constant_table": ([I32, I32, P], I32),
        "kvq_calibrate_chan_scale": ([P, P, P, P], I32),
        "kvq_key_mean_workspace": ([P], SZ),
        "kvq_key_mean": ([P, P, P, P, SZ, P], I32),
        "kvq_quantize_pack": ([P, P, P], I32),
        "kvq_dequant": ([P, P, P], I32),
        "kvq_decode_attn_workspace": ([P, I32, I32], SZ),
        "kvq_decode_attn": ([P, P, I32, I32, P, P, F, P, P, P, SZ, P], I32),
        "kvq_decode_attn_ex": ([P, P, I32, I32, P, P, F, P, P, P, SZ, I32, P], I32),
        "kvq_attn_error_workspace": ([P, I32, I32], SZ),
        "kvq_attn_error": ([P, P, P, P, I32, I32, P, P, F, P, P, P, P, SZ, P], I32),
        "kvq_quantize_pack_tokens": ([P, I32, I32, P, P], I32),
        "kvq_decode_attn_segments_workspace": ([P, I32, I32, I32, I32, I32], SZ),
        "kvq_decode_attn_segments": ([P, I32, I32, I32, I32, I32, I32, P, P, F, P, P, P, SZ, P], I32),
        "kvq_decode_attn_segments_ex": ([P, I32, I32, I32, I32, I32, I32, P, P, F, P, P, P, SZ, I32, P], I32),
        "kvq_effective_bits": ([P, I32, I32, I32, I32], D),
        "kvq_attn_error_ex": ([P, P, P, P, I32, I32, P, P, F, P, P, SZ, P], I32),
        "kvq_quantize_pack_kv": ([P, P, P, P, P], I32),
        "kvq_quantize_pack_tokens_kv": ([P, P, I32, I32, P, P, P], I32),
        "kvq_decode_attn_static": ([P, P, I32, I32, P, P, F, P, P, P], I32),
        "kvq_append_decode_attn": ([P, P, I32, I32, P, P, I32, I32, P, P, F, P, P, P, SZ, P], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if hasattr(lib, "kvq_timeline_read"):              # the profiling build only
        lib.kvq_timeline_read.argtypes = [P, SZ]
        lib.kvq_timeline_read.restype = I32
    return lib


_lib = _load()


# ------------------------------------------------------------------ python-side descriptions

@dataclasses.dataclass(frozen=True)
class Codec:
    codebook: int
    bits: int = 0
    group: int = 0
    rot_width: int = 0
    aux_bits: int = 0

    def c(self) -> kvq_codec:
        return kvq_codec(self.codebook, self.bits, self.group, self.rot_width, self.aux_bits)


@dataclasses.dataclass(frozen=True)
class Shape:
    batch: int
    layers: int
    heads: int
    tokens: int
    head_dim: int

    def c(self) -> kvq_shape:
        return kvq_shape(self.batch, self.layers, self.heads, self.tokens, self.head_dim)

    @property
    def rows(self) -> int:
        return self.batch * self.layers * self.heads * self.tokens


@dataclasses.dataclass
class Packed:
    """A packed tensor: torch tensors on the device plus its codec and shape."""
    codec: Codec
    shape: Shape
    codes: object           # torch.int32 [rows][words]  (uint32 bit pattern)
    scales: object          # torch.int16 [rows][ns]     (fp16 bit pattern)
    mins: object            # torch.int16 [rows][nm] or None
    chan_scale: object = None  # torch.float32 [L][H][D] or None
    mean: object = None        # torch.float32 [L][H][D] or None (shared key mean)

    def c(self) -> kvq_packed:
        # cached: the tensors of a Packed are fixed once it is built
        cs = self.__dict__.get("_cstruct")
        if cs is None:
            cs = kvq_packed(self.codec.c(), self.shape.c(), _ptr(self.codes), _ptr(self.scales),
                            _ptr(self.mins), _ptr(self.chan_scale), _ptr(self.mean))
            self.__dict__["_cstruct"] = cs
        return cs


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr() if t.numel() else None


def _check(fn, st):
    if st != 0:
        raise KvqError(fn, st)


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------------ entry points

def kvq_status_string(status: int) -> str:
    return _lib.kvq_status_string(status).decode()


def kvq_version() -> str:
    return _lib.kvq_version().decode()


def kvq_packed_layout(shape: Shape, codec: Codec):
    w, s, m = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    sc, cc = shape.c(), codec.c()
    _check("kvq_packed_layout", _lib.kvq_packed_layout(ctypes.byref(sc), ctypes.byref(cc), ctypes.byref(w),
                                                       ctypes.byref(s), ctypes.byref(m)))
    return w.value, s.value, m.value


def kvq_bits_per_value(codec: Codec, head_dim: int) -> float:
    cc = codec.c()
    return _lib.kvq_bits_per_value(ctypes.byref(cc), head_dim)


def kvq_constant_table(which: int, n: int):
    import numpy as np
    out = np.zeros(n, dtype=np.float32)
    _check("kvq_constant_table", _lib.kvq_constant_table(which, n, out.ctypes.data))
    return out


def kvq_calibrate_chan_scale(k_fp16, shape: Shape, chan_scale, stream=None):
    sc = shape.c()
    _check("kvq_calibrate_chan_scale",
           _lib.kvq_calibrate_chan_scale(_ptr(k_fp16), ctypes.byref(sc), _ptr(chan_scale), _stream(stream)))


def kvq_key_mean_workspace(shape: Shape) -> int:
    sc = shape.c()
    return _lib.kvq_key_mean_workspace(ctypes.byref(sc))


def kvq_key_mean(k_fp16, shape: Shape, mean, ws, ws_bytes: int, stream=None):
    sc = shape.c()
    _check("kvq_key_mean", _lib.kvq_key_mean(_ptr(k_fp16), ctypes.byref(sc), _ptr(mean), _ptr(ws), ws_bytes,
                                             _stream(stream)))


def kvq_quantize_pack(x_fp16, out: Packed, stream=None):
    pc = out.c()
    _check("kvq_quantize_pack", _lib.kvq_quantize_pack(_ptr(x_fp16), ctypes.byref(pc), _stream(stream)))


def kvq_quantize_pack_tokens(x_fp16, token0: int, n_tokens: int, out: Packed, stream=None):
    """Append path: code x_fp16 [B][L][H][n_tokens][D] into tokens [token0, token0 + n_tokens) of `out`."""
    pc = out.c()
    _check("kvq_quantize_pack_tokens",
           _lib.kvq_quantize_pack_tokens(_ptr(x_fp16), token0, n_tokens, ctypes.byref(pc), _stream(stream)))


def kvq_quantize_pack_kv(k_fp16, v_fp16, k: Packed, v: Packed, stream=None):
    """Keys and values of one cache in one call (one launch where both codecs allow)."""
    kc, vc = k.c(), v.c()
    _check("kvq_quantize_pack_kv", _lib.kvq_quantize_pack_kv(_ptr(k_fp16), _ptr(v_fp16), ctypes.byref(kc),
                                                             ctypes.byref(vc), _stream(stream)))


def kvq_quantize_pack_tokens_kv(k_fp16, v_fp16, token0: int, n_tokens: int, k: Packed, v: Packed, stream=None):
    """Append path for K and V together: tokens [token0, token0 + n_tokens) of both."""
    kc, vc = k.c(), v.c()
    _check("kvq_quantize_pack_tokens_kv",
           _lib.kvq_quantize_pack_tokens_kv(_ptr(k_fp16), _ptr(v_fp16), token0, n_tokens, ctypes.byref(kc),
                                            ctypes.byref(vc), _stream(stream)))


@dataclasses.dataclass
class Segment:
    """Packed K and V holding layers [layer0, layer0 + k.shape.layers), KV heads
    [head0, head0 + k.shape.heads) and tokens [token0, token0 + k.shape.tokens) of
    a logical cache."""
    k: Packed
    v: Packed
    layer0: int = 0
    token0: int = 0
    head0: int = 0


def _segments_c(segs):
    arr = (kvq_segment * len(segs))()
    keep = []
    for i, sg in enumerate(segs):
        kc, vc = sg.k.c(), sg.v.c()
        keep += [kc, vc]
        arr[i] = kvq_segment(ctypes.pointer(kc), ctypes.pointer(vc), sg.layer0, sg.token0, sg.head0)
    return arr, keep


def kvq_decode_attn_segments_workspace(segs, layers: int, heads: int, q_heads: int, n_q: int) -> int:
    arr, _keep = _segments_c(segs)
    return _lib.kvq_decode_attn_segments_workspace(arr, len(segs), layers, heads, q_heads, n_q)


def kvq_decode_attn_segments(segs, layers: int, heads: int, tokens: int, q_heads: int, n_q: int, q, kv_len,
                             sm_scale: float, out, lse, ws, ws_bytes: int, stream=None, path: int | None = None):
    arr, _keep = _segments_c(segs)
    if path is None:
        _check("kvq_decode_attn_segments",
               _lib.kvq_decode_attn_segments(arr, len(segs), layers, heads, tokens, q_heads, n_q, _ptr(q),
                                             _ptr(kv_len), sm_scale, _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
                                             _stream(stream)))
    else:
        _check("kvq_decode_attn_segments_ex",
               _lib.kvq_decode_attn_segments_ex(arr, len(segs), layers, heads, tokens, q_heads, n_q, _ptr(q),
                                                _ptr(kv_len), sm_scale, _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
                                                path, _stream(stream)))


def kvq_decode_attn_segments_ex(segs, layers, heads, tokens, q_heads, n_q, q, kv_len, sm_scale, out, lse, ws,
                                ws_bytes, path: int, stream=None):
    kvq_decode_attn_segments(segs, layers, heads, tokens, q_heads, n_q, q, kv_len, sm_scale, out, lse, ws, ws_bytes,
                             stream, path)


def kvq_effective_bits(segs, layers: int, heads: int, tokens: int) -> float:
    arr, _keep = _segments_c(segs)
    return _lib.kvq_effective_bits(arr, len(segs), layers, heads, tokens)


def kvq_dequant(inp: Packed, x_hat, stream=None):
    pc = inp.c()
    _check("kvq_dequant", _lib.kvq_dequant(ctypes.byref(pc), _ptr(x_hat), _stream(stream)))


def kvq_decode_attn_workspace(shape: Shape, q_heads: int, n_q: int) -> int:
    sc = shape.c()
    return _lib.kvq_decode_attn_workspace(ctypes.byref(sc), q_heads, n_q)


def kvq_decode_attn(k: Packed, v: Packed, q_heads: int, n_q: int, q, kv_len, sm_scale: float, out, lse,
                    ws, ws_bytes: int, stream=None, path: int | None = None):
    kc, vc = k.c(), v.c()
    if path is None:
        st = _lib.kvq_decode_attn(ctypes.byref(kc), ctypes.byref(vc), q_heads, n_q, _ptr(q), _ptr(kv_len),
                                  sm_scale, _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream))
        _check("kvq_decode_attn", st)
    else:
        st = _lib.kvq_decode_attn_ex(ctypes.byref(kc), ctypes.byref(vc), q_heads, n_q, _ptr(q), _ptr(kv_len),
                                     sm_scale, _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, path, _stream(stream))
        _check("kvq_decode_attn_ex", st)


def kvq_decode_attn_ex(k: Packed, v: Packed, q_heads, n_q, q, kv_len, sm_scale, out, lse, ws, ws_bytes,
                       path: int, stream=None):
    kvq_decode_attn(k, v, q_heads, n_q, q, kv_len, sm_scale, out, lse, ws, ws_bytes, stream, path)


def kvq_append_decode_attn(k_new, v_new, token0: int, n_new: int, k: Packed, v: Packed, q_heads: int, n_q: int,
                           q, kv_len, sm_scale: float, out, lse, ws, ws_bytes: int, stream=None):
    """Append n_new tokens' K and V at token0, then decode (one launch where the codecs allow)."""
    kc, vc = k.c(), v.c()
    _check("kvq_append_decode_attn",
           _lib.kvq_append_decode_attn(_ptr(k_new), _ptr(v_new), token0, n_new, ctypes.byref(kc), ctypes.byref(vc),
                                       q_heads, n_q, _ptr(q), _ptr(kv_len), sm_scale, _ptr(out), _ptr(lse),
                                       _ptr(ws), ws_bytes, _stream(stream)))


STATIC_SCRATCH_BYTES = 16 << 20      # KVQ_STATIC_SCRATCH_BYTES of kvq.h


def kvq_timeline_read(count: int):
    """The MFMA decode's clock stamps ([block][wave][slot], uint64), then cleared; only in
    the profiling build (KVQ_TIMELINE=1 with libkvq_timeline.so)."""
    import numpy as np
    if not hasattr(_lib, "kvq_timeline_read"):
        raise RuntimeError(f"{LIB_PATH} is not the timeline build (build it with `build.py --timeline`, "
                           "load it with KVQ_TIMELINE=1)")
    dst = np.zeros(count, dtype=np.uint64)
    _check("kvq_timeline_read", _lib.kvq_timeline_read(dst.ctypes.data, count))
    return dst


def kvq_decode_attn_static(k: Packed, v: Packed, q_heads: int, n_q: int, q, kv_len, sm_scale: float, out, lse,
                           stream=None):
    """kvq_decode_attn on the library's own device scratch: no workspace, nothing allocated."""
    kc, vc = k.c(), v.c()
    _check("kvq_decode_attn_static",
           _lib.kvq_decode_attn_static(ctypes.byref(kc), ctypes.byref(vc), q_heads, n_q, _ptr(q), _ptr(kv_len),
                                       sm_scale, _ptr(out), _ptr(lse), _stream(stream)))


def kvq_attn_error_workspace(shape: Shape, q_heads: int, n_q: int) -> int:
    sc = shape.c()
    return _lib.kvq_attn_error_workspace(ctypes.byref(sc), q_heads, n_q)


def kvq_attn_error(k_fp16, v_fp16, k: Packed, v: Packed, q_heads: int, n_q: int, q, kv_len, sm_scale: float,
                   kl_rows, relerr_rows, kv_err, ws, ws_bytes: int, stream=None):
    kc, vc = k.c(), v.c()
    st = _lib.kvq_attn_error(_ptr(k_fp16), _ptr(v_fp16), ctypes.byref(kc), ctypes.byref(vc), q_heads, n_q,
                             _ptr(q), _ptr(kv_len), sm_scale, _ptr(kl_rows), _ptr(relerr_rows), _ptr(kv_err),
                             _ptr(ws), ws_bytes, _stream(stream))
    _check("kvq_attn_error", st)


def kvq_attn_error_ex(k_fp16, v_fp16, k: Packed, v: Packed, q_heads: int, n_q: int, q, kv_len, sm_scale: float,
                      ws, ws_bytes: int, stream=None, kl=None, relerr=None, kv_err=None, renyi2=None, js=None,
                      logit_relerr=None, top1=None):
    """The error reduction with any subset of its outputs (torch tensors or None)."""
    kc, vc = k.c(), v.c()
    o = kvq_error_outputs(_ptr(kl), _ptr(relerr), _ptr(kv_err), _ptr(renyi2), _ptr(js), _ptr(logit_relerr),
                          _ptr(top1))
    st = _lib.kvq_attn_error_ex(_ptr(k_fp16), _ptr(v_fp16), ctypes.byref(kc), ctypes.byref(vc), q_heads, n_q,
                                _ptr(q), _ptr(kv_len), sm_scale, ctypes.byref(o), _ptr(ws), ws_bytes, _stream(stream))
    _check("kvq_attn_error_ex", st)


# ------------------------------------------------------------------ device-memory plumbing

def alloc_packed(codec: Codec, shape: Shape, device="cuda", chan_scale=None, mean=None) -> Packed:
    """Allocate the device buffers of a packed tensor (sizes from kvq_packed_layout)."""
    import torch
    w, s, m = kvq_packed_layout(shape, codec)
    rows = shape.rows
    codes = torch.empty((rows, w), dtype=torch.int32, device=device)
    scales = torch.empty((rows, s), dtype=torch.int16, device=device)
    mins = torch.empty((rows, m), dtype=torch.int16, device=device) if m else None
    return Packed(codec, shape, codes, scales, mins, chan_scale, mean)


def packed_from_fp16(x_fp16, shape: Shape) -> Packed:
    """View fp16 rows as an FP16-codebook packed tensor (anchor layers): no copy."""
    return Packed(Codec(FP16), shape, x_fp16, None, None, None)

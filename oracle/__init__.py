"""CPU oracle for group-wise low-bit KV-cache quantisation and packed decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.  The
product path (``kv_cache_bit_fwht_amd``) never imports, calls or links it, and
this package never imports the product path.  The two share no code: the only
common dependency is the seeded input generator in ``synth/``, which holds no
quantisation or attention arithmetic.

What it computes, and the pages it follows (citation tags used throughout):

* [FMAG-6]  HF forum thread "Fourier Magnitude KV Cache Quantization", post #6
            (sections "Minimal recipe (post-debunk)", "Milestone", "Best
            results", "The winning recipe", "Mechanism findings").
* [FMAG-R]  Same thread, the reply with a small Colab probe (the parts on the
            rFFT physical codec, real/imag control, matched-rate allocation and
            attention-visible error).
* [LCPP]    llama.cpp issue #21385 "Per-head adaptive KV cache quantization:
            lossless q4_0 on hybrid models, +8% quality on standard models".
* [E21W]    "PROVISIONAL: known 3-bit KV cache methods on the 4B fall well short
            of 4-bit quality (proxy queries)" (sections "Benchmark", "What I
            tested", "Result").
* [E22L]    "Can 4-bit keys and 2-bit values hit a 1M-token memory budget?
            Simulated KV cache, 4B model, 64K" (sections "What I tested",
            "Result").

Precision: wherever floating point decides an integer code, the oracle takes the
decision in IEEE binary32 (NumPy float32: every elementwise op is one correctly
rounded operation and is never fused), the precision the HIP kernels compute
in; stored scales are IEEE binary16 as the pages fix (fp16 group scales,
[E22L, What I tested]).  Attention and error metrics are computed in fp64 on the
oracle's own dequantised values.

Functions whose results the pages do not pin are marked "parity unpinned" in
their docstrings: the Gaussian Lloyd-Max levels (named, not printed; pinned by
the Lloyd-Max optimality conditions instead).  The NF4 levels (the pages name NF4
but print no table) follow the QLoRA construction and are pinned to the table
printed in that paper's Appendix E.
"""
from .codec import (  # noqa: F401
    Codec,
    FP16, INT_ABSMAX, INT_MINMAX, TERNARY, SIGN, NF4, INT8_SYM, RFFT_POLAR, RFFT_CART, INT_SYM, LLOYD,
    rn16, inv32, fwht, fwht_kappa, calibrate_chan_scale, key_mean, nf4_levels, nf4_midpoints, lloyd_levels, lloyd_midpoints,
    quantize_rows, dequant_rows, layout, pack_bits, unpack_bits,
    quantize_pack, dequant,
)
from .attention import (  # noqa: F401
    attend_unit, decode_attn, attn_error, kl_div, rel_err, kv_err_unit, assemble_segments,
    renyi2, js_div, logit_relerr, top1_flip, entropy_adaptive_bits, attn_error_ex,
)
from .accounting import bits_per_value, kv_bits_per_value, rfft_payload_bits_per_value, tiles, effective_bits  # noqa: F401

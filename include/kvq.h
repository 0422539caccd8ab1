/*
 * kvq.h - C ABI of libkvq: group-wise low-bit KV-cache quantisation and decode
 * attention read back through the packed cache, for AMD MI355X (gfx950).
 *
 * Sources of the operations (web pages; cited by title and section):
 *  [E22L]  "Can 4-bit keys and 2-bit values hit a 1M-token memory budget?
 *          Simulated KV cache, 4B model, 64K" - What I tested, Result.
 *  [E21W]  "PROVISIONAL: known 3-bit KV cache methods on the 4B fall well short
 *          of 4-bit quality (proxy queries)" - Benchmark, What I tested, Result.
 *  [FMAG-6] HF forum "Fourier Magnitude KV Cache Quantization", post #6 -
 *          Minimal recipe, Milestone, Best results, Mechanism findings.
 *  [FMAG-R] same thread, the Colab-probe reply - the rFFT physical codec
 *          (packed magnitude index + packed phase-angle index), real/imag control.
 *  [LCPP]  llama.cpp issue #21385 - independent K and V cache types (-ctk/-ctv).
 *
 * Conventions for every entry point
 *  - Tensors are dense, row-major [batch][layers][heads][tokens][head_dim]; a
 *    "row" is one head_dim vector.  Device pointers must be 16-byte aligned.
 *  - The caller owns every buffer (allocate with the sizes the layout and
 *    workspace queries return).  The library never allocates, frees or
 *    synchronises; all device work is enqueued on `stream` (a hipStream_t; NULL
 *    = the null stream) and returns before it completes.
 *  - Arguments are validated on the host before anything is launched; on any
 *    error nothing is written.  A failed launch returns KVQ_ERR_HIP.
 *  - Inputs must be finite; results for NaN/Inf inputs are unspecified (but
 *    every access stays in bounds).
 *  - Calls on one stream are ordered; calls that write the same buffers on
 *    different streams race.  No C++ exception crosses this interface.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_ARG = -1,          /* null pointer, bad shape, inconsistent K/V shapes */
  KVQ_ERR_UNSUPPORTED = -2,  /* codec/bits/group/rotation not supported */
  KVQ_ERR_ALIGN = -3,        /* device pointer not 16-byte aligned */
  KVQ_ERR_WORKSPACE = -4,    /* workspace smaller than the query returned */
  KVQ_ERR_HIP = -5           /* HIP launch or runtime error */
} kvq_status;

/* Codebooks.  Dequantised values (before the inverse rotation) per group with
 * fp16 scale s (and fp16 minimum z):
 *  FP16        identity; the "codes" are the fp16 rows (anchor layers, [FMAG-6]
 *              Minimal recipe: layer 0 kept fp16).
 *  INT_ABSMAX  {-2^(b-1), ..., 2^(b-1)-1} * s, ggml-style signed absmax; the
 *              scale takes the sign of the group's extreme value ([E22L] Result:
 *              the 2-bit grid {-2,-1,0,1}*s).  bits 2..8.
 *  INT_MINMAX  {0, ..., 2^b-1} * s + z ([E21W] What I tested, arm A).  bits 2..8.
 *  TERNARY     {-s, 0, +s}, s = group absmax, 2 stored bits ([FMAG-6] Milestone).
 *  SIGN        {-s, +s}, s = mean |y|, 1 bit ([FMAG-6] Minimal recipe).
 *  NF4         NormalFloat-4 levels * s, s = group absmax, 4 bits ([FMAG-6]
 *              Milestone "NF4-K").
 *  INT8_SYM    {-127..127} * s, s = absmax/127, 8 bits ([FMAG-6] int8 KV row).
 *  RFFT_POLAR  rFFT along head_dim (D/2+1 bins); per bin an unsigned `bits`
 *              magnitude code (fp16 scale per `group` bins) and an `aux_bits`
 *              phase-sector code ([FMAG-R] physical codec).  Keys only.
 *  RFFT_CART   rFFT; real and imaginary parts each INT_ABSMAX with `bits` bits
 *              per `group` bins ([FMAG-R] real/imag control).  Keys only.
 *  INT_SYM     symmetric grid {-(2^b-1)/2, ..., (2^b-1)/2} * s (half-integer
 *              levels, as many on each side), s = absmax / ((2^b-1)/2); bits
 *              2..8.  The symmetric value grid [E22L] Result names as the next
 *              test after the one-sided {-2,-1,0,1} grid.
 *  LLOYD       Lloyd-Max levels of a unit Gaussian (2^b of them) * s, s = the
 *              group's root mean square; bits 2..4 ([E22L] Result: Gaussian
 *              Lloyd-Max levels on rotated values; use rot_width for the
 *              rotation).
 * Scalar rules (rounding, ties, zero groups) are those of the CPU oracle:
 * binary32 arithmetic, round-to-nearest-even, fp16 scales saturated to
 * +-65504 and never -0. */
typedef enum {
  KVQ_FP16 = 0,
  KVQ_INT_ABSMAX = 1,
  KVQ_INT_MINMAX = 2,
  KVQ_TERNARY = 3,
  KVQ_SIGN = 4,
  KVQ_NF4 = 5,
  KVQ_INT8_SYM = 6,
  KVQ_RFFT_POLAR = 7,
  KVQ_RFFT_CART = 8,
  KVQ_INT_SYM = 9,
  KVQ_LLOYD = 10
} kvq_codebook;

typedef struct {
  int32_t codebook;   /* kvq_codebook */
  int32_t bits;       /* INT_ABSMAX/INT_MINMAX/INT_SYM: 2..8; LLOYD: 2..4; RFFT_*:
                         2..8 magnitude/component bits; ignored (implied) for the
                         other codebooks */
  int32_t group;      /* values per scale: 8, 16, 32, 64, 128 or 256 (<= head_dim);
                         RFFT_*: bins per scale (8..128) */
  int32_t rot_width;  /* Walsh-Hadamard width: 0 (none) or a power of two in
                         [2, head_dim]; applied per rot_width block of each row
                         ([E22L] What I tested: 256-wide Hadamard rotation) */
  int32_t aux_bits;   /* RFFT_POLAR phase bits: 3..8; else 0 */
} kvq_codec;

typedef struct {
  int32_t batch, layers, heads, tokens, head_dim;  /* head_dim in {64, 128, 256} */
} kvq_shape;

/* A packed tensor.  codes: uint32 [rows][code_words_per_row] (FP16: the fp16
 * rows themselves); scales: fp16 [rows][scales_per_row]; mins: fp16
 * [rows][mins_per_row] (INT_MINMAX only, else NULL); chan_scale: optional fp32
 * [layers][heads][head_dim] per-channel multipliers applied before the rotation
 * and divided back out after dequantising ([E21W] What I tested, arms C/D),
 * NULL for none; mean: optional fp32 [layers][heads][head_dim] shared mean
 * subtracted from every row before the channel multiply and added back after
 * dequantising (the shared key-mean subtraction of [LCPP], the later comment
 * measuring the failure mode; see kvq_key_mean), NULL for none.  Bit layout: per
 * row, code j occupies bits [j*b, (j+1)*b) of a little-endian stream of uint32
 * words (RFFT_POLAR: all magnitude codes, then all phase codes; RFFT_CART: all
 * real codes, then all imaginary codes).  The per-row operations are, in order:
 * x -> x - mean -> (x - mean) * chan_scale -> rotation -> codebook, each rounded
 * to binary32. */
typedef struct {
  kvq_codec codec;
  kvq_shape shape;
  uint32_t* codes;
  uint16_t* scales;
  uint16_t* mins;
  const float* chan_scale;
  const float* mean;
} kvq_packed;

/* Human-readable status. */
const char* kvq_status_string(kvq_status s);

/* Library version string. */
const char* kvq_version(void);

/* Host only (no device needed).  Per-row sizes of a packed tensor. */
kvq_status kvq_packed_layout(const kvq_shape* shape, const kvq_codec* codec,
                             size_t* code_words_per_row, size_t* scales_per_row,
                             size_t* mins_per_row);

/* Host only.  Stored bits per value including fp16 scales (and mins): b + 16 *
 * n_params / group; FP16 = 16; rFFT codecs: exact bits per row / head_dim
 * ([E21W] Result: 3.5 / 4.5 bits at group 32; [E22L] What I tested: 3.125 ...
 * 3.625 for the K+V arms).  Returns a negative value for an invalid codec. */
double kvq_bits_per_value(const kvq_codec* codec, int32_t head_dim);

/* Host only.  Copies a constant table the kernels use into `out` (n floats):
 * which = 0 NF4 levels (16), 1 NF4 midpoints (15), 2/3 FFT twiddle cos/-sin
 * for head_dim n*2 (n = D/2 entries), 4/5 phase-sector direction cos/sin for
 * 2^aux sectors (n = 2^aux), 6/7 first-octant sector boundary cos/sin (n =
 * 2^aux / 8), 8/9/10 LLOYD levels for 2/3/4 bits (n = 2^bits). */
kvq_status kvq_constant_table(int32_t which, int32_t n, float* out);

/* Per-channel key multipliers from a calibration sequence ([E21W] What I
 * tested, arm C: per-channel K scaling calibrated offline): chan_scale[l][h][d]
 * = RN32(1 / max_t |k[0][l][h][t][d]|), or 1 for an all-zero channel.  k_fp16
 * is [1][layers][heads][tokens][head_dim] (batch must be 1); chan_scale is
 * fp32 [layers][heads][head_dim]. */
kvq_status kvq_calibrate_chan_scale(const uint16_t* k_fp16, const kvq_shape* shape,
                                    float* chan_scale, void* stream);

/* Bytes of workspace kvq_key_mean needs: 8 * layers * heads * head_dim. */
size_t kvq_key_mean_workspace(const kvq_shape* shape);

/* Shared per-(layer, head) key mean ([LCPP] llama.cpp issue "Per-head adaptive
 * KV cache quantization", the later comment measuring the failure mode: a shared
 * key mean carries about half of the key energy, and subtracting the running
 * mean before quantising and restoring it after removes the failure).
 * mean[l][h][d] = binary32 rounding of (fp64(S) / (batch * tokens)) * 2^-24,
 * where S is the exact integer sum over every sequence and token of the fp16
 * values times 2^24 (so the result does not depend on summation order).
 * k_fp16: [B][L][H][T][D]; mean: fp32 [L][H][D]; ws: device scratch of
 * kvq_key_mean_workspace() bytes (no initial contents needed).  batch * tokens
 * must be at most 2^23 (the exact sum then fits 64 bits); tokens = 0 gives
 * zeros.  Pass the result as kvq_packed.mean of the key cache. */
kvq_status kvq_key_mean(const uint16_t* k_fp16, const kvq_shape* shape, float* mean, void* ws,
                        size_t ws_bytes, void* stream);

/* Quantise and pack fp16 rows x_fp16 [B][L][H][T][D] into `out` (codes,
 * scales, mins; shape and codec taken from `out`).  One fused kernel per call:
 * load, optional mean subtraction, optional per-channel multiply, optional
 * Walsh-Hadamard rotation, group
 * statistic, fp16 scale, code, bit-pack ([E22L] What I tested; [E21W] What I
 * tested).  Codes and scales are bit-identical to the CPU oracle. */
kvq_status kvq_quantize_pack(const uint16_t* x_fp16, const kvq_packed* out, void* stream);

/* Append path: quantise and pack fp16 rows x_fp16 [B][L][H][n_tokens][D] into
 * token positions [token0, token0 + n_tokens) of every (sequence, layer, head)
 * unit of `out` (shape and codec from `out`; rows outside the window are not
 * touched).  The codes of a row do not depend on any other row, so appending
 * tokens one step at a time gives exactly the codes of quantising them all at
 * once ([FMAG-6] The winning recipe: decode steps write the cache as they go).
 * 0 <= token0, n_tokens >= 1, token0 + n_tokens <= out->shape.tokens. */
kvq_status kvq_quantize_pack_tokens(const uint16_t* x_fp16, int32_t token0, int32_t n_tokens,
                                    const kvq_packed* out, void* stream);

/* The keys and values of one cache in one call: the same results as
 * kvq_quantize_pack(k_fp16, k) followed by kvq_quantize_pack(v_fp16, v) ([E22L]
 * What I tested: 4-bit rotated keys with 2-bit values; [LCPP] independent K and V
 * cache types).  When both are signed-absmax codecs at head_dim 256 (2, 4 or 8
 * bits, rotation 0 or 256, group >= 16) without a mean or channel scales, one
 * kernel codes both tensors (each wavefront a quad of key rows and the same quad
 * of value rows); otherwise the two tensors are coded by their own launches.
 * k and v must have the same shape and distinct outputs; k_fp16 and v_fp16 are
 * [B][L][H][T][D] fp16.  Errors as for kvq_quantize_pack; nothing is launched on
 * an error.  A cache with no tokens is a no-op. */
kvq_status kvq_quantize_pack_kv(const uint16_t* k_fp16, const uint16_t* v_fp16, const kvq_packed* k,
                                const kvq_packed* v, void* stream);

/* Append path for keys and values together: kvq_quantize_pack_tokens on k and on
 * v with the same window, in one launch where kvq_quantize_pack_kv would use one
 * ([FMAG-6] The winning recipe: each decode step writes its token's K and V into
 * the cache).  k_fp16 and v_fp16 are [B][L][H][n_tokens][D]. */
kvq_status kvq_quantize_pack_tokens_kv(const uint16_t* k_fp16, const uint16_t* v_fp16, int32_t token0,
                                       int32_t n_tokens, const kvq_packed* k, const kvq_packed* v,
                                       void* stream);

/* Dequantise `in` to fp32 x_hat [B][L][H][T][D] in the original coordinates
 * (inverse codebook, inverse rotation, division by chan_scale, addition of the
 * mean): the reconstructed K and V whose error against fp16 is the squared error
 * over signal energy of [E21W] Benchmark, and the values read back by the
 * simulations of [E22L] What I tested (quantise, then dequantise post-RoPE K/V).
 * Every element is written; results are bit-identical to the CPU oracle. */
kvq_status kvq_dequant(const kvq_packed* in, float* x_hat, void* stream);

/* Bytes of workspace kvq_decode_attn needs for these sizes.  Its first 65536
 * bytes hold the MFMA kernel's work counters: they must be zero before the
 * first call that uses the workspace (fill it with zeros once after
 * allocating it), and every call leaves them zero again.  The rest holds
 * split-K partials and needs no initial contents.  Calls that share a
 * workspace must not overlap in time. */
size_t kvq_decode_attn_workspace(const kvq_shape* kv, int32_t q_heads, int32_t n_q);

/* Decode attention read back through packed K and V ([E22L] What I tested:
 * attention over the quantised post-RoPE cache; [E21W] Benchmark: causal
 * proxy queries).  q: fp16 [B][L][n_q][q_heads][D]; query head j reads KV head
 * j / (q_heads / heads).  kv_len: int32 [B][L][n_q] keys attended per query
 * (keys [0, kv_len)), NULL = all tokens; values are clamped to [0, tokens].
 * sm_scale: logit scale, 0 = 1/sqrt(head_dim).  out: fp32 [B][L][n_q][q_heads][D];
 * lse: fp32 [B][L][n_q][q_heads] natural-log partition (-inf for no keys),
 * nullable.  K and V must have the same shape; V's codebook may not be an rFFT
 * codec.  ws: device workspace of at least kvq_decode_attn_workspace() bytes.
 * K dequantisation happens in registers/LDS: rotated keys are read by rotating
 * the query instead, rotated values by rotating the output once per query.
 * Supported: every codebook for K, every non-rFFT codebook for V, head_dim
 * 64/128/256, up to 8 query heads per KV head, kv_len batch*layers*n_q rows of
 * at most 65535 per launch grid dimension.  A key mean (k->mean) shifts every
 * logit of a query by the same q.mean, which leaves the attention weights and
 * out unchanged; lse gets sm_scale * q.mean added.  V may not carry a mean. */
kvq_status kvq_decode_attn(const kvq_packed* k, const kvq_packed* v, int32_t q_heads,
                           int32_t n_q, const uint16_t* q, const int32_t* kv_len,
                           float sm_scale, float* out, float* lse, void* ws,
                           size_t ws_bytes, void* stream);

/* As kvq_decode_attn, choosing the kernel: path 0 = automatic (the MFMA kernel
 * where it applies, else the general one), 1 = the general kernel (every codec
 * above), 2 = the MFMA kernel, KVQ_ERR_UNSUPPORTED unless: head_dim 256, at least
 * 32 tokens, at most 4 query heads per KV head, K INT_ABSMAX
 * 2-, 3-, 4- or 5-bit at group 128 or 256 (any rotation, optional chan_scale), V
 * INT_ABSMAX or INT_SYM, 2-, 3- or 4-bit, or LLOYD 2- or 3-bit, at group 64..256
 * without chan_scale (any rotation) -- the 4-bit-key / 2-bit-value arms of [E22L] What I
 * tested, the Gaussian Lloyd-Max values on rotated values of [E22L] Result, the
 * 2-bit keys of the per-layer allocation of [E21W] Result, the
 * symmetric value grid of [E22L] Result, 4-bit values ([LCPP] Finding 1) and the
 * per-head key widths of [LCPP] Finding 2; or head_dim 128, at least 32 tokens, at
 * most 4 query heads per KV head, K TERNARY or SIGN at group 8, INT8_SYM at group
 * 128, FP16 or NF4 at group 64, V TERNARY or SIGN at group 8, INT8_SYM at group 128,
 * FP16 or 4-bit INT_ABSMAX at group 64, without rotation, chan_scale or mean -- the
 * extreme low-bit arms, NF4 keys with 4-bit values, the int8 reference row and the
 * fp16 anchor layer of [FMAG-6] Milestone and Best results -- and also K 6-bit
 * INT_ABSMAX at group 32 (unrotated or rot_width 128), RFFT_CART 6-bit at group 32 or
 * RFFT_POLAR 5-bit magnitude + 7-bit phase at group 32 (the Hadamard, real/imaginary
 * and polar arms of the matched-rate transform control, [FMAG-R] Colab-probe reply)
 * with any of those values.  With rFFT keys the weighted query spectra are kept in
 * the workspace after the partials (the call then uses fewer splits). */
kvq_status kvq_decode_attn_ex(const kvq_packed* k, const kvq_packed* v, int32_t q_heads,
                              int32_t n_q, const uint16_t* q, const int32_t* kv_len,
                              float sm_scale, float* out, float* lse, void* ws,
                              size_t ws_bytes, int32_t path, void* stream);

/* One decode step of a growing cache ([FMAG-6] The winning recipe: each decode step
 * writes its token's K and V into the quantised cache, then attends over it):
 * kvq_quantize_pack_tokens_kv(k_new, v_new, token0, n_new, k, v) followed by
 * kvq_decode_attn(k, v, ...), with the same results.  k_new, v_new: fp16
 * [B][L][H][n_new][D].  When the MFMA decode applies (see kvq_decode_attn_ex) with
 * 4-bit signed-absmax keys, signed-absmax values, rotation 0 or 256, no channel
 * scales or mean, and n_new <= 8, one launch does both: the first block of each
 * (query row, KV head) codes the new rows before it reads them, and the steps holding
 * them are decoded by that block.  Otherwise an append launch precedes the decode.
 * The workspace is kvq_decode_attn's (same size query).  Arguments are validated
 * before anything is launched; errors as for the two calls. */
kvq_status kvq_append_decode_attn(const uint16_t* k_new, const uint16_t* v_new, int32_t token0,
                                  int32_t n_new, const kvq_packed* k, const kvq_packed* v,
                                  int32_t q_heads, int32_t n_q, const uint16_t* q,
                                  const int32_t* kv_len, float sm_scale, float* out, float* lse,
                                  void* ws, size_t ws_bytes, void* stream);

/* Bytes of the library's own device scratch used by kvq_decode_attn_static (one
 * copy on every GPU the library runs on, held until the process ends). */
#define KVQ_STATIC_SCRATCH_BYTES (16u << 20)

/* kvq_decode_attn without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The split-K partials and work counters live in a static device
 * array of KVQ_STATIC_SCRATCH_BYTES per GPU instead of `ws`; nothing is allocated
 * or freed, by the library or by anything it calls.  Runs on the current device
 * (`stream` must belong to it); the first call on a device takes the array's
 * device address and clears its counter region with a kernel on `stream`.  Every
 * call on a GPU shares that GPU's array and leaves its counters zero (the partials
 * keep the last call's contents): calls on one GPU that overlap in time (other
 * streams, other threads) race and must be serialised by the caller.  Returns
 * KVQ_ERR_WORKSPACE, launching nothing, when kvq_decode_attn_workspace() for these
 * sizes exceeds KVQ_STATIC_SCRATCH_BYTES (the 64K workload with one decode query
 * needs about 1.1 MB).  Arguments, results and other errors as kvq_decode_attn. */
kvq_status kvq_decode_attn_static(const kvq_packed* k, const kvq_packed* v, int32_t q_heads,
                                  int32_t n_q, const uint16_t* q, const int32_t* kv_len,
                                  float sm_scale, float* out, float* lse, void* stream);

/* One piece of a logical cache of `layers` x `heads` x `tokens`: packed K and V
 * (same shape; batch and head_dim equal to the other segments') holding layers
 * [layer0, layer0 + k->shape.layers), KV heads [head0, head0 + k->shape.heads)
 * and tokens [token0, token0 + k->shape.tokens) of every sequence.  Segments
 * describe decode anchors ([FMAG-6] The winning recipe, Selective-Layer Decode
 * Anchoring: the KV of the first decoded tokens kept at fp16/int8/int4 on chosen
 * layers), fp16 anchor layers ([FMAG-6] Minimal recipe), sliding windows, and
 * per-layer and per-head codec choices ([LCPP] the per-head KV-type request: sink
 * heads at f16 or q8_0, standard heads at q4_0, diffuse heads lower). */
typedef struct {
  const kvq_packed* k;
  const kvq_packed* v;
  int32_t layer0;
  int32_t token0;
  int32_t head0;
} kvq_segment;

/* Bytes of workspace kvq_decode_attn_segments needs (0 for invalid arguments).
 * Its first 65536 bytes are the decode counters (zero before first use, left
 * zero by every call), as for kvq_decode_attn. */
size_t kvq_decode_attn_segments_workspace(const kvq_segment* segs, int32_t n_seg, int32_t layers,
                                          int32_t heads, int32_t q_heads, int32_t n_q);

/* Decode attention over a logical cache [B][layers][heads][tokens][D] given as
 * 1..16 segments that tile it: for every (layer, KV head), the segments covering
 * it cover tokens [0, tokens) exactly, without overlap.  q_heads is a multiple of
 * heads (query head j reads KV head j / (q_heads / heads), as for
 * kvq_decode_attn).  q: fp16 [B][layers][n_q][q_heads][D];
 * kv_len: int32 [B][layers][n_q] over the logical token axis (NULL = all);
 * out/lse as for kvq_decode_attn over the whole logical cache.  Each segment is
 * decoded by the kvq_decode_attn kernels (the MFMA kernel where it applies) and
 * its (out, lse) merged into the running result by log-sum-exp weights; a
 * segment's key mean shifts only its own lse, as the whole cache's would.
 * A codec map (every segment holding all tokens of its layer range x head range,
 * as for a per-layer bit allocation, [E21W] Result, or per-head bit widths,
 * [LCPP] Finding 2) with two or more segments is decoded by one launch when its
 * tiles qualify: see kvq_decode_attn_segments_ex. */
kvq_status kvq_decode_attn_segments(const kvq_segment* segs, int32_t n_seg, int32_t layers,
                                    int32_t heads, int32_t tokens, int32_t q_heads, int32_t n_q,
                                    const uint16_t* q,
                                    const int32_t* kv_len, float sm_scale, float* out, float* lse,
                                    void* ws, size_t ws_bytes, void* stream);

/* kvq_decode_attn_segments with the route chosen: path 0 = as
 * kvq_decode_attn_segments; 1 = each segment by its own launches and a
 * log-sum-exp merge; 2 = one decode launch for the whole codec map (every block
 * looks up the segment of its (layer, KV head) and decodes with that segment's
 * codecs).  Path 2 needs every segment to hold tokens [0, tokens) of its tile.  It
 * runs on the MFMA kernel (which merges in the kernel) when every tile is one the
 * MFMA decode takes at groups of 128 (head_dim 256, 3-5-bit signed absmax keys, 2- or
 * 4-bit signed absmax or symmetric-grid values, no value channel scales) and the
 * rows fit the workspace counters; otherwise on the general kernel plus one split
 * combine, when every key/value codec pair is among: signed absmax keys of 2-6 bits
 * with signed absmax values of 2, 3 or 4 bits (any group, rotation and channel
 * scale), fp16/fp16, int8/int8, ternary/ternary, sign/sign, NF4 keys with 4-bit
 * signed absmax values; else KVQ_ERR_UNSUPPORTED (nothing launched).  Path 0 takes
 * the MFMA one-launch route whenever it applies and there are several segments.
 * Segment key means are applied by every route.  Same workspace query; any other
 * path value is KVQ_ERR_ARG. */
kvq_status kvq_decode_attn_segments_ex(const kvq_segment* segs, int32_t n_seg, int32_t layers,
                                       int32_t heads, int32_t tokens, int32_t q_heads, int32_t n_q,
                                       const uint16_t* q,
                                       const int32_t* kv_len, float sm_scale, float* out, float* lse,
                                       void* ws, size_t ws_bytes, int32_t path, void* stream);

/* Host only.  Effective bits per cached value of a tiled logical cache: the
 * segments' K/V bits per value (kvq_bits_per_value, averaged over K and V)
 * weighted by the layers x heads x tokens each holds ([FMAG-6] Milestone and
 * Minimal recipe: anchored rows count at their own precision, so anchors kept for
 * the prompt and the first D decoded tokens cost (L + D) rows per anchored layer).
 * Returns a negative value for segments that do not tile the cache. */
double kvq_effective_bits(const kvq_segment* segs, int32_t n_seg, int32_t layers, int32_t heads,
                          int32_t tokens);

/* Bytes of workspace kvq_attn_error needs. */
size_t kvq_attn_error_workspace(const kvq_shape* kv, int32_t q_heads, int32_t n_q);

/* Attention-visible error of the packed cache against fp16 ([E21W] Benchmark:
 * K/V error is squared error over signal energy, attention error is the
 * relative error of the attention output, KL is the divergence of the
 * attention distribution from f16).  One pass over fp16 K/V and packed K/V per
 * query: kl_rows [B][L][n_q][q_heads] = KL(p_fp16 || p_quant) in nats,
 * relerr_rows = ||o_quant - o_fp16|| / ||o_fp16||; kv_err [B][L][H][4] fp64 =
 * (sum dK^2, sum K^2, sum dV^2, sum V^2) over the unit's rows, with dK the
 * dequantised minus fp16 value in original coordinates (mean restored).  Other
 * arguments as for kvq_decode_attn. */
kvq_status kvq_attn_error(const uint16_t* k_fp16, const uint16_t* v_fp16,
                          const kvq_packed* k, const kvq_packed* v, int32_t q_heads,
                          int32_t n_q, const uint16_t* q, const int32_t* kv_len,
                          float sm_scale, float* kl_rows, float* relerr_rows,
                          double* kv_err, void* ws, size_t ws_bytes, void* stream);

/* Outputs of kvq_attn_error_ex, each nullable; row arrays are fp32
 * [B][L][n_q][q_heads] over the attended keys of the row.  The rungs of the
 * diagnostic ladder ([FMAG-R] the Colab-probe reply: QK-logit error, attention
 * KL / JS, top-attended-token flips, attention-output error) and the Renyi
 * entropy that sizes per-head bits ([LCPP] Finding 2). */
typedef struct {
  float* kl;            /* KL(p_fp16 || p_quant), nats */
  float* relerr;        /* ||o_quant - o_fp16|| / ||o_fp16|| */
  double* kv_err;       /* [B][L][H][4] as for kvq_attn_error */
  float* renyi2;        /* H_2(p_fp16) = -ln sum_t p_t^2, nats (0 without keys) */
  float* js;            /* Jensen-Shannon divergence of p_fp16 and p_quant, nats
                           (one more pass over the keys) */
  float* logit_relerr;  /* ||l_quant - l_fp16|| / ||l_fp16|| of the logits sm * q.k */
  float* top1;          /* 1 where the most-attended key differs (first index on
                           ties), else 0 */
} kvq_error_outputs;

/* kvq_attn_error with the outputs chosen by `outs` (any subset; the same
 * workspace size).  A key mean is restored in every output (the quantised
 * logits include q.mean). */
kvq_status kvq_attn_error_ex(const uint16_t* k_fp16, const uint16_t* v_fp16,
                             const kvq_packed* k, const kvq_packed* v, int32_t q_heads,
                             int32_t n_q, const uint16_t* q, const int32_t* kv_len,
                             float sm_scale, const kvq_error_outputs* outs, void* ws,
                             size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */

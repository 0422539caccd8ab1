// libkvq C ABI: argument validation, layout and workspace queries, constant
// tables, and dispatch to the kernels.  Every check runs on the host before any
// launch, so an invalid call writes nothing.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "kvq_internal.hpp"

namespace kvq {

// ------------------------------------------------------------------ constant tables

// Standard normal quantile by bisection on Phi(x) = erfc(-x/sqrt 2)/2 in fp64.
static double norm_ppf(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 2000; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    const double c = 0.5 * std::erfc(-mid / std::sqrt(2.0));
    if (c < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

// Lloyd-Max quantiser of the standard normal with n levels (fp64 fixed point,
// rounded to binary32): boundaries halfway between neighbouring levels, each
// level the mean of the normal over its cell, (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
// Started from the cell-centre quantiles and iterated to convergence.
static void lloyd_max_levels(int n, float* out) {
  double L[16], t[17];
  for (int k = 0; k < n; ++k) L[k] = norm_ppf((k + 0.5) / n);
  auto pdf = [](double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); };
  auto cdf = [](double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); };
  for (int it = 0; it < 100000; ++it) {
    t[0] = -INFINITY;
    t[n] = INFINITY;
    for (int k = 1; k < n; ++k) t[k] = 0.5 * (L[k - 1] + L[k]);
    double change = 0.0;
    for (int k = 0; k < n; ++k) {
      const double m = (pdf(t[k]) - pdf(t[k + 1])) / (cdf(t[k + 1]) - cdf(t[k]));
      change = std::max(change, std::fabs(m - L[k]));
      L[k] = m;
    }
    if (change < 1e-14) break;
  }
  for (int k = 0; k < n; ++k) out[k] = (float)L[k];
  for (int k = n; k < 16; ++k) out[k] = INFINITY;
}

// NormalFloat-4 levels as published with QLoRA (Dettmers et al. 2023: the
// construction of section 3, the table of Appendix E): offset o = RN32(0.9677083);
// 8 positive levels at probabilities RN32(o + i (1/2 - o) / 8), i < 8, and 7
// negative ones at RN32(o + i (1/2 - o) / 7), i < 7 (each probability formed in
// fp64, rounded to binary32); each level the fp64 normal quantile of its binary32
// probability, rounded to binary32; an exact zero; all divided by the largest in
// binary32.  This gives the paper's printed table bit for bit.  The pages name NF4
// ([FMAG-6] Milestone) without printing levels.
static Tables build_tables() {
  Tables t{};
  const double o = (double)(float)0.9677083;
  float v[16];
  int n = 0;
  for (int i = 0; i < 8; ++i) v[n++] = (float)norm_ppf((double)(float)(o + i * (0.5 - o) / 8.0));
  v[n++] = 0.0f;
  for (int i = 0; i < 7; ++i) v[n++] = (float)(-norm_ppf((double)(float)(o + i * (0.5 - o) / 7.0)));
  // sort ascending (insertion sort: 16 values)
  for (int i = 1; i < 16; ++i)
    for (int k = i; k > 0 && v[k - 1] > v[k]; --k) { float tmp = v[k]; v[k] = v[k - 1]; v[k - 1] = tmp; }
  for (int i = 0; i < 16; ++i) t.nf4_lv[i] = v[i] / v[15];
  for (int i = 0; i < 15; ++i) {
    const float s = t.nf4_lv[i] + t.nf4_lv[i + 1];
    t.nf4_mid[i] = s * 0.5f;
  }
  t.nf4_mid[15] = INFINITY;
  for (int b = 2; b <= 4; ++b) lloyd_max_levels(1 << b, t.lloyd_lv[b - 2]);
  return t;
}

const Tables& host_tables() {
  static const Tables t = build_tables();
  return t;
}

void host_fft_tables(int N, FftTables* t) {
  std::memset(t, 0, sizeof(*t));
  for (int k = 0; k < N / 2; ++k) {
    const double ang = 2.0 * M_PI * k / N;
    t->tw_c[k] = (float)std::cos(ang);
    t->tw_s[k] = (float)(-std::sin(ang));
  }
}

void host_phase_tables(int P, PhaseTables* t) {
  std::memset(t, 0, sizeof(*t));
  for (int k = 0; k < P; ++k) {
    const double ang = 2.0 * M_PI * k / P;
    t->dir_c[k] = (float)std::cos(ang);
    t->dir_s[k] = (float)std::sin(ang);
  }
  for (int j = 0; j < P / 8; ++j) {
    const double ang = (2.0 * j + 1.0) * M_PI / P;
    t->bnd_c[j] = (float)std::cos(ang);
    t->bnd_s[j] = (float)std::sin(ang);
  }
}

// ------------------------------------------------------------------ validation

static bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static kvq_status check_shape(const kvq_shape* s) {
  if (!s) return KVQ_ERR_ARG;
  if (s->batch < 1 || s->layers < 1 || s->heads < 1 || s->tokens < 0) return KVQ_ERR_ARG;
  if (s->head_dim != 64 && s->head_dim != 128 && s->head_dim != 256) return KVQ_ERR_UNSUPPORTED;
  const double rows = (double)s->batch * s->layers * s->heads * s->tokens;
  if (rows * s->head_dim > 9.0e15) return KVQ_ERR_ARG;
  return KVQ_OK;
}

static bool is_rfft(int cb) { return cb == KVQ_RFFT_POLAR || cb == KVQ_RFFT_CART; }

static kvq_status check_codec(const kvq_codec* c, int D) {
  if (!c) return KVQ_ERR_ARG;
  const int cb = c->codebook;
  if (cb < KVQ_FP16 || cb > KVQ_LLOYD) return KVQ_ERR_UNSUPPORTED;
  if (cb == KVQ_FP16) return KVQ_OK;
  if (is_rfft(cb)) {
    if (c->bits < 2 || c->bits > 8) return KVQ_ERR_UNSUPPORTED;
    if (c->group < 8 || c->group > 128 || !pow2(c->group)) return KVQ_ERR_UNSUPPORTED;
    if (c->rot_width != 0) return KVQ_ERR_UNSUPPORTED;
    if (cb == KVQ_RFFT_POLAR && (c->aux_bits < 3 || c->aux_bits > 8)) return KVQ_ERR_UNSUPPORTED;
    return KVQ_OK;
  }
  if (cb == KVQ_INT_ABSMAX || cb == KVQ_INT_MINMAX || cb == KVQ_INT_SYM) {
    if (c->bits < 2 || c->bits > 8) return KVQ_ERR_UNSUPPORTED;
  }
  if (cb == KVQ_LLOYD && (c->bits < 2 || c->bits > 4)) return KVQ_ERR_UNSUPPORTED;
  if (!pow2(c->group) || c->group < 8 || c->group > 256 || c->group > D) return KVQ_ERR_UNSUPPORTED;
  if (c->rot_width != 0 && (!pow2(c->rot_width) || c->rot_width < 2 || c->rot_width > D))
    return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

static int code_bits(const kvq_codec& c) {
  switch (c.codebook) {
    case KVQ_FP16: return 16;
    case KVQ_TERNARY: return 2;
    case KVQ_SIGN: return 1;
    case KVQ_NF4: return 4;
    case KVQ_INT8_SYM: return 8;
    default: return c.bits;
  }
}

static void layout_of(const kvq_codec& c, int D, size_t* words, size_t* ns, size_t* nm) {
  if (is_rfft(c.codebook)) {
    const int F = D / 2 + 1, ng = (F + c.group - 1) / c.group;
    const long bits = (c.codebook == KVQ_RFFT_POLAR) ? (long)F * (c.bits + c.aux_bits) : 2L * F * c.bits;
    *words = (size_t)((bits + 31) / 32);
    *ns = (size_t)((c.codebook == KVQ_RFFT_POLAR) ? ng : 2 * ng);
    *nm = 0;
    return;
  }
  *words = (size_t)D * code_bits(c) / 32;
  *ns = (c.codebook == KVQ_FP16) ? 0 : (size_t)(D / c.group);
  *nm = (c.codebook == KVQ_INT_MINMAX) ? *ns : 0;
}

static kvq_status check_packed(const kvq_packed* p, bool need_write) {
  (void)need_write;
  if (!p) return KVQ_ERR_ARG;
  kvq_status st = check_shape(&p->shape);
  if (st != KVQ_OK) return st;
  st = check_codec(&p->codec, p->shape.head_dim);
  if (st != KVQ_OK) return st;
  size_t w, ns, nm;
  layout_of(p->codec, p->shape.head_dim, &w, &ns, &nm);
  if (!p->codes) return KVQ_ERR_ARG;
  if (ns && !p->scales) return KVQ_ERR_ARG;
  if (nm && !p->mins) return KVQ_ERR_ARG;
  if (!aligned16(p->codes) || (p->scales && !aligned16(p->scales)) || (p->mins && !aligned16(p->mins)) ||
      (p->chan_scale && !aligned16(p->chan_scale)) || (p->mean && !aligned16(p->mean)))
    return KVQ_ERR_ALIGN;
  if ((p->chan_scale || p->mean) && p->codec.codebook == KVQ_FP16) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

static bool same_shape(const kvq_shape& a, const kvq_shape& b) {
  return a.batch == b.batch && a.layers == b.layers && a.heads == b.heads && a.tokens == b.tokens &&
         a.head_dim == b.head_dim;
}

static kvq_status hip_status(hipError_t e) {
  if (e == hipSuccess) return KVQ_OK;
  return KVQ_ERR_HIP;
}

// Allocation-free decode: the workspace is the library's own device array `scratch`
// (KVQ_STATIC_SCRATCH_BYTES, one copy per GPU, alive until the process ends).  Host
// code never passes the array's name to a kernel: on the first call on a device (that
// device current) its device address is taken with hipGetSymbolAddress and kept per
// device, and the counter region is cleared once by a fill kernel on the caller's
// stream (a kernel rather than a memset, so a first call inside graph capture records
// a kernel node).  Every decode leaves the counters zero again.
static __device__ __align__(256) unsigned char scratch[KVQ_STATIC_SCRATCH_BYTES];

__global__ void k_zero_words(uint32_t* p, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static kvq_status static_scratch(void** out, hipStream_t st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return KVQ_ERR_HIP;
    const long long words = (long long)(kWsCounterBytes / sizeof(uint32_t));
    k_zero_words<<<(unsigned)((words + kBlock - 1) / kBlock), kBlock, 0, st>>>(static_cast<uint32_t*>(ptr), words);
    if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KVQ_OK;
}

}  // namespace kvq

using namespace kvq;

extern "C" {

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported codec or shape";
    case KVQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case KVQ_ERR_WORKSPACE: return "workspace too small";
    case KVQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* kvq_version(void) { return "kvq 0.1 gfx950"; }

kvq_status kvq_packed_layout(const kvq_shape* shape, const kvq_codec* codec, size_t* code_words_per_row,
                             size_t* scales_per_row, size_t* mins_per_row) {
  kvq_status st = check_shape(shape);
  if (st != KVQ_OK) return st;
  st = check_codec(codec, shape->head_dim);
  if (st != KVQ_OK) return st;
  if (!code_words_per_row || !scales_per_row || !mins_per_row) return KVQ_ERR_ARG;
  layout_of(*codec, shape->head_dim, code_words_per_row, scales_per_row, mins_per_row);
  return KVQ_OK;
}

double kvq_bits_per_value(const kvq_codec* codec, int32_t head_dim) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return -1.0;
  if (check_codec(codec, head_dim) != KVQ_OK) return -1.0;
  if (codec->codebook == KVQ_FP16) return 16.0;
  size_t w, ns, nm;
  layout_of(*codec, head_dim, &w, &ns, &nm);
  if (is_rfft(codec->codebook)) {
    const int F = head_dim / 2 + 1;
    const double payload = (codec->codebook == KVQ_RFFT_POLAR) ? (double)F * (codec->bits + codec->aux_bits)
                                                              : 2.0 * F * codec->bits;
    return (payload + 16.0 * (double)ns) / head_dim;
  }
  const double nparams = (codec->codebook == KVQ_INT_MINMAX) ? 2.0 : 1.0;
  return code_bits(*codec) + 16.0 * nparams / codec->group;
}

kvq_status kvq_constant_table(int32_t which, int32_t n, float* out) {
  if (!out || n < 1) return KVQ_ERR_ARG;
  if (which == 0 || which == 1) {
    const Tables& t = host_tables();
    const int len = which == 0 ? 16 : 15;
    if (n != len) return KVQ_ERR_ARG;
    std::memcpy(out, which == 0 ? t.nf4_lv : t.nf4_mid, sizeof(float) * len);
    return KVQ_OK;
  }
  if (which == 2 || which == 3) {
    if (n > 128 || !pow2(n)) return KVQ_ERR_ARG;
    FftTables t;
    host_fft_tables(2 * n, &t);
    std::memcpy(out, which == 2 ? t.tw_c : t.tw_s, sizeof(float) * n);
    return KVQ_OK;
  }
  if (which >= 8 && which <= 10) {
    const int b = which - 6;
    if (n != (1 << b)) return KVQ_ERR_ARG;
    std::memcpy(out, host_tables().lloyd_lv[b - 2], sizeof(float) * n);
    return KVQ_OK;
  }
  if (which >= 4 && which <= 7) {
    const int P = which <= 5 ? n : 8 * n;
    if (P < 8 || P > 256 || !pow2(P)) return KVQ_ERR_ARG;
    PhaseTables t;
    host_phase_tables(P, &t);
    const float* src = which == 4 ? t.dir_c : which == 5 ? t.dir_s : which == 6 ? t.bnd_c : t.bnd_s;
    std::memcpy(out, src, sizeof(float) * n);
    return KVQ_OK;
  }
  return KVQ_ERR_ARG;
}

kvq_status kvq_calibrate_chan_scale(const uint16_t* k_fp16, const kvq_shape* shape, float* chan_scale,
                                    void* stream) {
  kvq_status st = check_shape(shape);
  if (st != KVQ_OK) return st;
  if (shape->batch != 1) return KVQ_ERR_ARG;
  if (!k_fp16 || !chan_scale) return KVQ_ERR_ARG;
  if (!aligned16(k_fp16) || !aligned16(chan_scale)) return KVQ_ERR_ALIGN;
  return hip_status(launch_calibrate(k_fp16, *shape, chan_scale, (hipStream_t)stream));
}

size_t kvq_key_mean_workspace(const kvq_shape* shape) {
  if (check_shape(shape) != KVQ_OK) return 0;
  return (size_t)8 * shape->layers * shape->heads * shape->head_dim;
}

kvq_status kvq_key_mean(const uint16_t* k_fp16, const kvq_shape* shape, float* mean, void* ws, size_t ws_bytes,
                        void* stream) {
  kvq_status st = check_shape(shape);
  if (st != KVQ_OK) return st;
  if (!k_fp16 || !mean) return KVQ_ERR_ARG;
  if ((double)shape->batch * shape->tokens > (double)(1 << 23)) return KVQ_ERR_ARG;
  if (!aligned16(k_fp16) || !aligned16(mean)) return KVQ_ERR_ALIGN;
  const size_t need = (size_t)8 * shape->layers * shape->heads * shape->head_dim;
  if (ws_bytes < need || !ws) return KVQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return KVQ_ERR_ALIGN;
  return hip_status(launch_key_mean(k_fp16, *shape, mean, static_cast<long long*>(ws), (hipStream_t)stream));
}

kvq_status kvq_quantize_pack(const uint16_t* x_fp16, const kvq_packed* out, void* stream) {
  kvq_status st = check_packed(out, true);
  if (st != KVQ_OK) return st;
  if (!x_fp16) return KVQ_ERR_ARG;
  if (!aligned16(x_fp16)) return KVQ_ERR_ALIGN;
  if (is_rfft(out->codec.codebook)) return hip_status(launch_rfft_quantize(x_fp16, *out, (hipStream_t)stream));
  return hip_status(launch_quantize(x_fp16, *out, (hipStream_t)stream));
}

kvq_status kvq_quantize_pack_tokens(const uint16_t* x_fp16, int32_t token0, int32_t n_tokens, const kvq_packed* out,
                                    void* stream) {
  kvq_status st = check_packed(out, true);
  if (st != KVQ_OK) return st;
  if (!x_fp16) return KVQ_ERR_ARG;
  if (!aligned16(x_fp16)) return KVQ_ERR_ALIGN;
  if (token0 < 0 || n_tokens < 1 || (long long)token0 + n_tokens > out->shape.tokens) return KVQ_ERR_ARG;
  if (is_rfft(out->codec.codebook))
    return hip_status(launch_rfft_quantize_tokens(x_fp16, *out, token0, n_tokens, (hipStream_t)stream));
  return hip_status(launch_quantize_tokens(x_fp16, *out, token0, n_tokens, (hipStream_t)stream));
}

// K and V of one cache: the two kvq_quantize_pack_tokens calls in one, sharing a
// launch when both codecs allow it.
static kvq_status quantize_kv(const uint16_t* k_fp16, const uint16_t* v_fp16, bool whole, int32_t token0,
                              int32_t n_tokens, const kvq_packed* k, const kvq_packed* v, void* stream) {
  kvq_status st = check_packed(k, true);
  if (st != KVQ_OK) return st;
  st = check_packed(v, true);
  if (st != KVQ_OK) return st;
  if (!same_shape(k->shape, v->shape)) return KVQ_ERR_ARG;
  if (!k_fp16 || !v_fp16) return KVQ_ERR_ARG;
  if (!aligned16(k_fp16) || !aligned16(v_fp16)) return KVQ_ERR_ALIGN;
  if (k->codes == v->codes || (k->scales && k->scales == v->scales)) return KVQ_ERR_ARG;
  if (whole) {
    token0 = 0;
    n_tokens = k->shape.tokens;
    if (n_tokens == 0) return KVQ_OK;
  } else if (token0 < 0 || n_tokens < 1 || (long long)token0 + n_tokens > k->shape.tokens) {
    return KVQ_ERR_ARG;
  }
  const hipStream_t s = (hipStream_t)stream;
  const bool window = !whole && n_tokens != k->shape.tokens;
  if (is_rfft(k->codec.codebook) || is_rfft(v->codec.codebook)) {
    auto one = [&](const uint16_t* x, const kvq_packed& p) {
      if (is_rfft(p.codec.codebook))
        return window ? launch_rfft_quantize_tokens(x, p, token0, n_tokens, s) : launch_rfft_quantize(x, p, s);
      return window ? launch_quantize_tokens(x, p, token0, n_tokens, s) : launch_quantize(x, p, s);
    };
    const hipError_t e = one(k_fp16, *k);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(one(v_fp16, *v));
  }
  return hip_status(launch_quantize_kv(k_fp16, v_fp16, *k, *v, token0, n_tokens, s));
}

kvq_status kvq_quantize_pack_kv(const uint16_t* k_fp16, const uint16_t* v_fp16, const kvq_packed* k,
                                const kvq_packed* v, void* stream) {
  return quantize_kv(k_fp16, v_fp16, true, 0, 0, k, v, stream);
}

kvq_status kvq_quantize_pack_tokens_kv(const uint16_t* k_fp16, const uint16_t* v_fp16, int32_t token0,
                                       int32_t n_tokens, const kvq_packed* k, const kvq_packed* v, void* stream) {
  return quantize_kv(k_fp16, v_fp16, false, token0, n_tokens, k, v, stream);
}

kvq_status kvq_dequant(const kvq_packed* in, float* x_hat, void* stream) {
  kvq_status st = check_packed(in, false);
  if (st != KVQ_OK) return st;
  if (!x_hat) return KVQ_ERR_ARG;
  if (!aligned16(x_hat)) return KVQ_ERR_ALIGN;
  if (is_rfft(in->codec.codebook)) return hip_status(launch_rfft_dequant(*in, x_hat, (hipStream_t)stream));
  return hip_status(launch_dequant(*in, x_hat, (hipStream_t)stream));
}

static kvq_status check_kv(const kvq_packed* k, const kvq_packed* v, int32_t q_heads, int32_t n_q) {
  kvq_status st = check_packed(k, false);
  if (st != KVQ_OK) return st;
  st = check_packed(v, false);
  if (st != KVQ_OK) return st;
  if (!same_shape(k->shape, v->shape)) return KVQ_ERR_ARG;
  if (is_rfft(v->codec.codebook) || v->mean) return KVQ_ERR_UNSUPPORTED;
  if (q_heads < 1 || q_heads % k->shape.heads != 0 || q_heads / k->shape.heads > 8) return KVQ_ERR_UNSUPPORTED;
  if (n_q < 1) return KVQ_ERR_ARG;
  return KVQ_OK;
}

static kvq_status check_attn(const kvq_packed* k, const kvq_packed* v, int32_t q_heads, int32_t n_q,
                             const uint16_t* q) {
  kvq_status st = check_kv(k, v, q_heads, n_q);
  if (st != KVQ_OK) return st;
  if (!q) return KVQ_ERR_ARG;
  if (!aligned16(q)) return KVQ_ERR_ALIGN;
  return KVQ_OK;
}

// Segments of a logical layers x heads x tokens cache: each valid on its own (with its
// own KV-head count, q_heads / heads query heads per KV head), all with the same batch
// and head_dim, inside the cache, and tiling every (layer, head)'s tokens exactly.
static kvq_status check_segments(const kvq_segment* segs, int32_t n_seg, int32_t layers, int32_t heads,
                                 int32_t tokens, int32_t q_heads, int32_t n_q) {
  if (!segs || n_seg < 1 || n_seg > kMaxSegments || layers < 1 || heads < 1 || tokens < 1) return KVQ_ERR_ARG;
  if (q_heads < 1 || q_heads % heads != 0) return KVQ_ERR_UNSUPPORTED;
  const int G = q_heads / heads;
  const kvq_packed* k0 = segs[0].k;
  if (!k0) return KVQ_ERR_ARG;
  for (int i = 0; i < n_seg; ++i) {
    const kvq_segment& sg = segs[i];
    if (!sg.k || !sg.v) return KVQ_ERR_ARG;
    const kvq_shape& sh = sg.k->shape;
    if (sh.heads < 1) return KVQ_ERR_ARG;
    kvq_status st = check_kv(sg.k, sg.v, sh.heads * G, n_q);
    if (st != KVQ_OK) return st;
    if (sh.batch != k0->shape.batch || sh.head_dim != k0->shape.head_dim) return KVQ_ERR_ARG;
    if (sh.tokens < 1 || sg.layer0 < 0 || sg.token0 < 0 || sg.head0 < 0 ||
        (long long)sg.layer0 + sh.layers > layers || (long long)sg.head0 + sh.heads > heads ||
        (long long)sg.token0 + sh.tokens > tokens)
      return KVQ_ERR_ARG;
  }
  for (int l = 0; l < layers; ++l) {
    for (int h = 0; h < heads; ++h) {
      std::vector<std::pair<int, int>> r;
      for (int i = 0; i < n_seg; ++i) {
        const kvq_shape& sh = segs[i].k->shape;
        if (l >= segs[i].layer0 && l < segs[i].layer0 + sh.layers && h >= segs[i].head0 &&
            h < segs[i].head0 + sh.heads)
          r.emplace_back(segs[i].token0, sh.tokens);
      }
      std::sort(r.begin(), r.end());
      long long next = 0;
      for (const auto& [t0, n] : r) {
        if (t0 != next) return KVQ_ERR_ARG;
        next = (long long)t0 + n;
      }
      if (next != tokens) return KVQ_ERR_ARG;
    }
  }
  return KVQ_OK;
}

// How kvq_decode_attn_segments runs (byte offsets into its workspace).  With batch 1,
// a segment none of whose layers an earlier segment covered decodes straight into the
// output (its query and length rows are contiguous there); every other segment decodes
// into partials of its own, merged into the output by one kernel at the end.  Rows that
// no direct segment writes start at (0, -inf).
struct SegPlan {
  size_t dec, dec_bytes, q, kvl, lacc, total;
  size_t out_off[kMaxSegments], lse_off[kMaxSegments];
  bool direct[kMaxSegments];
  bool need_init;
  size_t mixed_bytes;
};

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

static SegPlan seg_plan(const kvq_segment* segs, int32_t n_seg, int32_t layers, int32_t heads, int32_t q_heads,
                        int32_t n_q) {
  SegPlan p{};
  const kvq_shape& s0 = segs[0].k->shape;
  const int G = q_heads / heads;
  std::vector<char> touched(layers, 0), direct_layer(layers, 0);
  size_t dec = 0, q = 0, kvl = 0;
  for (int i = 0; i < n_seg; ++i) {
    const kvq_shape& sh = segs[i].k->shape;
    const int l0 = segs[i].layer0, l1 = l0 + sh.layers;
    const bool inside = l0 >= 0 && l1 <= layers;
    // direct: batch 1, every head, and no earlier segment on these layers
    bool fresh = inside && s0.batch == 1 && sh.heads == heads && segs[i].head0 == 0;
    for (int l = l0; fresh && l < l1; ++l) fresh = !touched[l];
    p.direct[i] = fresh;
    for (int l = std::max(l0, 0); l < std::min(l1, (int)layers); ++l) {
      touched[l] = 1;
      if (fresh) direct_layer[l] = 1;
    }
    const int hq = sh.heads * G;
    const size_t rows = (size_t)sh.batch * sh.layers * n_q;
    dec = std::max(dec, decode_ws_bytes(sh, hq, n_q));
    q = std::max(q, rows * hq * sh.head_dim * 2);
    kvl = std::max(kvl, rows * 4);
  }
  for (int l = 0; l < layers; ++l) p.need_init |= !direct_layer[l];
  p.dec_bytes = dec;
  p.dec = kWsCounterBytes;
  p.q = p.dec + round256(dec);
  p.kvl = p.q + round256(q);
  size_t off = p.kvl + round256(kvl);
  for (int i = 0; i < n_seg; ++i) {
    if (p.direct[i]) continue;
    const kvq_shape& sh = segs[i].k->shape;
    const size_t rows = (size_t)sh.batch * sh.layers * n_q * sh.heads * G;
    p.out_off[i] = off;
    off += round256(rows * sh.head_dim * 4);
    p.lse_off[i] = off;
    off += round256(rows * 4);
  }
  p.lacc = off;
  p.total = p.lacc + round256((size_t)s0.batch * layers * n_q * q_heads * 4);
  // the one-launch path of a codec map: counters, then its split partials
  int tokens = 0;
  for (int i = 0; i < n_seg; ++i) tokens = std::max(tokens, segs[i].token0 + segs[i].k->shape.tokens);
  p.mixed_bytes = mixed_ws_bytes(segs, layers, heads, tokens, q_heads, n_q);
  p.total = std::max(p.total, kWsCounterBytes + p.mixed_bytes);
  p.total = std::max(p.total, kWsCounterBytes + mixed_fast_ws_bytes(segs, layers, heads, tokens, q_heads, n_q));
  return p;
}

// One decode of a packed K/V pair: counters at ctr (kWsCounterBytes, zero and left zero),
// split-K partials at part.
// app_n > 0: the MFMA kernel also codes app_k / app_v into tokens [app_t0, app_t0 + app_n)
// (the caller has checked fused_append_supported).
static hipError_t decode_packed(const kvq_packed* k, const kvq_packed* v, int32_t q_heads, int32_t n_q,
                                const uint16_t* q, const int32_t* kv_len, float sm_scale, float* out, float* lse,
                                void* ctr, void* part, size_t part_bytes, int32_t path, hipStream_t st,
                                const uint16_t* app_k = nullptr, const uint16_t* app_v = nullptr, int app_t0 = 0,
                                int app_n = 0) {
  const bool fast_ok = fast_decode_supported(*k, *v, q_heads);
  const bool m128_ok = app_n == 0 && m128_decode_supported(*k, *v, q_heads);
  AttnProblem pr{};
  pr.k = k; pr.v = v; pr.Hq = q_heads; pr.n_q = n_q; pr.q = q; pr.kv_len = kv_len;
  pr.app_k = app_k; pr.app_v = app_v; pr.app_t0 = app_t0; pr.app_n = app_n;
  if (app_n > 0) path = 2;
  pr.sm_scale = sm_scale > 0.0f ? sm_scale : (float)(1.0 / std::sqrt((double)k->shape.head_dim));
  pr.out = out; pr.lse = lse;
  pr.ctr = static_cast<int*>(ctr);
  pr.ws = part;
  pr.ws_bytes = part_bytes;
  const bool use_fast = (path == 2) || (path == 0 && (fast_ok || m128_ok));
  bool mean_done = false;
  hipError_t e = !use_fast ? launch_decode_generic(pr, st)
                 : (m128_ok && !fast_ok) ? launch_decode_m128(pr, st)
                                         : launch_decode_fast(pr, st, &mean_done);
  // a key mean adds q.mean to every logit of a query: weights unchanged, lse shifted (by
  // the MFMA kernel's own merge when it merges, else here)
  if (e == hipSuccess && k->mean && lse && !mean_done) e = launch_lse_mean(pr, st);
  return e;
}

size_t kvq_decode_attn_workspace(const kvq_shape* kv, int32_t q_heads, int32_t n_q) {
  if (check_shape(kv) != KVQ_OK || q_heads < 1 || n_q < 1) return 0;
  return kWsCounterBytes + decode_ws_bytes(*kv, q_heads, n_q);
}

kvq_status kvq_decode_attn_ex(const kvq_packed* k, const kvq_packed* v, int32_t q_heads, int32_t n_q,
                              const uint16_t* q, const int32_t* kv_len, float sm_scale, float* out, float* lse,
                              void* ws, size_t ws_bytes, int32_t path, void* stream) {
  kvq_status st = check_attn(k, v, q_heads, n_q, q);
  if (st != KVQ_OK) return st;
  if (!out) return KVQ_ERR_ARG;
  if (!aligned16(out) || (lse && !aligned16(lse)) || (kv_len && !aligned16(kv_len))) return KVQ_ERR_ALIGN;
  if (!(sm_scale >= 0.0f) || !std::isfinite(sm_scale)) return KVQ_ERR_ARG;
  if (path < 0 || path > 2) return KVQ_ERR_ARG;
  const size_t need = kWsCounterBytes + decode_ws_bytes(k->shape, q_heads, n_q);
  if (ws_bytes < need || (need && !ws)) return KVQ_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return KVQ_ERR_ALIGN;
  if (path == 2 && !fast_decode_supported(*k, *v, q_heads) && !m128_decode_supported(*k, *v, q_heads))
    return KVQ_ERR_UNSUPPORTED;
  // no keys (tokens = 0): zero output, lse = -inf (the generic kernel's combine)
  return hip_status(decode_packed(k, v, q_heads, n_q, q, kv_len, sm_scale, out, lse, ws,
                                  static_cast<char*>(ws) + kWsCounterBytes, ws_bytes - kWsCounterBytes, path,
                                  (hipStream_t)stream));
}

kvq_status kvq_decode_attn(const kvq_packed* k, const kvq_packed* v, int32_t q_heads, int32_t n_q,
                           const uint16_t* q, const int32_t* kv_len, float sm_scale, float* out, float* lse,
                           void* ws, size_t ws_bytes, void* stream) {
  return kvq_decode_attn_ex(k, v, q_heads, n_q, q, kv_len, sm_scale, out, lse, ws, ws_bytes, 0, stream);
}

kvq_status kvq_decode_attn_static(const kvq_packed* k, const kvq_packed* v, int32_t q_heads, int32_t n_q,
                                  const uint16_t* q, const int32_t* kv_len, float sm_scale, float* out, float* lse,
                                  void* stream) {
  kvq_status st = check_attn(k, v, q_heads, n_q, q);
  if (st != KVQ_OK) return st;
  if (!out) return KVQ_ERR_ARG;
  if (!aligned16(out) || (lse && !aligned16(lse)) || (kv_len && !aligned16(kv_len))) return KVQ_ERR_ALIGN;
  if (!(sm_scale >= 0.0f) || !std::isfinite(sm_scale)) return KVQ_ERR_ARG;
  const size_t need = kWsCounterBytes + decode_ws_bytes(k->shape, q_heads, n_q);
  if (need > (size_t)KVQ_STATIC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
  void* ws = nullptr;
  st = static_scratch(&ws, (hipStream_t)stream);
  if (st != KVQ_OK) return st;
  return kvq_decode_attn_ex(k, v, q_heads, n_q, q, kv_len, sm_scale, out, lse, ws, (size_t)KVQ_STATIC_SCRATCH_BYTES,
                            0, stream);
}

kvq_status kvq_append_decode_attn(const uint16_t* k_new, const uint16_t* v_new, int32_t token0, int32_t n_new,
                                  const kvq_packed* k, const kvq_packed* v, int32_t q_heads, int32_t n_q,
                                  const uint16_t* q, const int32_t* kv_len, float sm_scale, float* out, float* lse,
                                  void* ws, size_t ws_bytes, void* stream) {
  // every check before anything is launched
  kvq_status st = check_attn(k, v, q_heads, n_q, q);
  if (st != KVQ_OK) return st;
  if (!out || !k_new || !v_new) return KVQ_ERR_ARG;
  if (!aligned16(out) || (lse && !aligned16(lse)) || (kv_len && !aligned16(kv_len)) || !aligned16(k_new) ||
      !aligned16(v_new))
    return KVQ_ERR_ALIGN;
  if (!(sm_scale >= 0.0f) || !std::isfinite(sm_scale)) return KVQ_ERR_ARG;
  if (token0 < 0 || n_new < 1 || (long long)token0 + n_new > k->shape.tokens) return KVQ_ERR_ARG;
  if (k->codes == v->codes || (k->scales && k->scales == v->scales)) return KVQ_ERR_ARG;
  if (is_rfft(v->codec.codebook)) return KVQ_ERR_UNSUPPORTED;
  const size_t need = kWsCounterBytes + decode_ws_bytes(k->shape, q_heads, n_q);
  if (ws_bytes < need || (need && !ws)) return KVQ_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return KVQ_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  char* part = static_cast<char*>(ws) + kWsCounterBytes;
  if (fused_append_supported(*k, *v, q_heads, n_new))
    return hip_status(decode_packed(k, v, q_heads, n_q, q, kv_len, sm_scale, out, lse, ws, part,
                                    ws_bytes - kWsCounterBytes, 2, s, k_new, v_new, token0, n_new));
  hipError_t e;
  if (is_rfft(k->codec.codebook)) {
    e = launch_rfft_quantize_tokens(k_new, *k, token0, n_new, s);
    if (e == hipSuccess) e = launch_quantize_tokens(v_new, *v, token0, n_new, s);
  } else {
    e = launch_quantize_kv(k_new, v_new, *k, *v, token0, n_new, s);
  }
  if (e != hipSuccess) return hip_status(e);
  return hip_status(decode_packed(k, v, q_heads, n_q, q, kv_len, sm_scale, out, lse, ws, part,
                                  ws_bytes - kWsCounterBytes, 0, s));
}

size_t kvq_decode_attn_segments_workspace(const kvq_segment* segs, int32_t n_seg, int32_t layers, int32_t heads,
                                          int32_t q_heads, int32_t n_q) {
  if (!segs || n_seg < 1 || n_seg > kMaxSegments || layers < 1 || heads < 1 || q_heads < 1 || q_heads % heads)
    return 0;
  const int G = q_heads / heads;
  for (int i = 0; i < n_seg; ++i) {
    if (!segs[i].k || !segs[i].v || segs[i].k->shape.heads < 1) return 0;
    if (check_kv(segs[i].k, segs[i].v, segs[i].k->shape.heads * G, n_q) != KVQ_OK) return 0;
  }
  return seg_plan(segs, n_seg, layers, heads, q_heads, n_q).total;
}

kvq_status kvq_decode_attn_segments_ex(const kvq_segment* segs, int32_t n_seg, int32_t layers, int32_t heads,
                                       int32_t tokens, int32_t q_heads, int32_t n_q, const uint16_t* q,
                                       const int32_t* kv_len, float sm_scale, float* out, float* lse, void* ws,
                                       size_t ws_bytes, int32_t path, void* stream) {
  kvq_status st = check_segments(segs, n_seg, layers, heads, tokens, q_heads, n_q);
  if (st != KVQ_OK) return st;
  if (!q || !out) return KVQ_ERR_ARG;
  if (!aligned16(q) || !aligned16(out) || (lse && !aligned16(lse)) || (kv_len && !aligned16(kv_len)))
    return KVQ_ERR_ALIGN;
  if (!(sm_scale >= 0.0f) || !std::isfinite(sm_scale)) return KVQ_ERR_ARG;
  if (path < 0 || path > 2) return KVQ_ERR_ARG;
  const SegPlan pl = seg_plan(segs, n_seg, layers, heads, q_heads, n_q);
  if (ws_bytes < pl.total || !ws) return KVQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return KVQ_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* w = static_cast<char*>(ws);
  const int B = segs[0].k->shape.batch, D = segs[0].k->shape.head_dim, G = q_heads / heads;
  // a codec map (every segment a whole-token tile) in one launch, asked for or by default
  // with several tiles: on the MFMA kernel when every tile is one of its pairs at group
  // 128, else on the general kernel when no tile would take the MFMA kernel
  const bool mixf_ok = mixed_fast_supported(segs, n_seg, layers, heads, tokens, q_heads, n_q);
  const bool mix_ok = mixed_decode_supported(segs, n_seg, layers, heads, tokens, q_heads, n_q);
  if (path == 2 && !mixf_ok && !mix_ok) return KVQ_ERR_UNSUPPORTED;
  const float sm = sm_scale > 0.0f ? sm_scale : (float)(1.0 / std::sqrt((double)D));
  if (mixf_ok && (path == 2 || (path == 0 && n_seg > 1)))
    return hip_status(launch_decode_fast_mixed(segs, n_seg, layers, heads, tokens, q_heads, n_q, q, kv_len, sm, out,
                                               lse, reinterpret_cast<int*>(w), w + kWsCounterBytes, s));
  bool use_mix = path == 2;
  if (path == 0 && mix_ok && n_seg > 1) {
    use_mix = true;
    for (int i = 0; i < n_seg; ++i)
      if (fast_decode_supported(*segs[i].k, *segs[i].v, segs[i].k->shape.heads * G)) use_mix = false;
  }
  if (use_mix)
    return hip_status(launch_decode_mixed(segs, n_seg, layers, heads, tokens, q_heads, n_q, q, kv_len, sm, out, lse,
                                          w + kWsCounterBytes, true, s));
  const size_t rpl = (size_t)n_q * q_heads;                     // output rows per (sequence, layer)
  float* lacc = lse ? lse : reinterpret_cast<float*>(w + pl.lacc);
  hipError_t e = hipSuccess;
  if (pl.need_init) e = launch_seg_init(out, lacc, (long long)B * layers * rpl, D, s);
  int nm = 0, ml0[kMaxSegments], mls[kMaxSegments], mj0[kMaxSegments], mhq[kMaxSegments];
  float* mos[kMaxSegments];
  float* mlse[kMaxSegments];
  for (int i = 0; i < n_seg && e == hipSuccess; ++i) {
    const kvq_segment& sg = segs[i];
    const kvq_shape& sh = sg.k->shape;
    const int hq = sh.heads * G, j0 = sg.head0 * G;              // the segment's query heads
    const bool all_heads = hq == q_heads;
    const uint16_t* qs = q;
    const int32_t* kvls = kv_len;
    uint16_t* qbuf = nullptr;
    int32_t* kbuf = nullptr;
    if (B == 1 && all_heads) {
      qs = q + (size_t)sg.layer0 * rpl * D;                     // contiguous layer slice
      if (kv_len) kvls = kv_len + (size_t)sg.layer0 * n_q;
      if (kv_len && sg.token0 != 0) kbuf = reinterpret_cast<int32_t*>(w + pl.kvl);
    } else {
      qbuf = reinterpret_cast<uint16_t*>(w + pl.q);
      if (kv_len) {
        if (B == 1 && sg.token0 == 0) kvls = kv_len + (size_t)sg.layer0 * n_q;
        else kbuf = reinterpret_cast<int32_t*>(w + pl.kvl);
      }
    }
    if (qbuf || kbuf)
      e = launch_seg_prepare(q, kv_len, qbuf, kbuf, B, layers, sh.layers, sg.layer0, n_q, q_heads, j0, hq, D,
                             sg.token0, sh.tokens, s);
    if (qbuf) qs = qbuf;
    if (kbuf) kvls = kbuf;
    // (keys [0, kv_len) clamp to [0, tokens] inside the decode, so a segment at token 0
    // needs no adjusted lengths)
    float* os;
    float* ls;
    if (pl.direct[i]) {
      os = out + (size_t)sg.layer0 * rpl * D;
      ls = lacc + (size_t)sg.layer0 * rpl;
    } else {
      os = reinterpret_cast<float*>(w + pl.out_off[i]);
      ls = reinterpret_cast<float*>(w + pl.lse_off[i]);
      ml0[nm] = sg.layer0;
      mls[nm] = sh.layers;
      mj0[nm] = j0;
      mhq[nm] = hq;
      mos[nm] = os;
      mlse[nm] = ls;
      ++nm;
    }
    if (e == hipSuccess)
      e = decode_packed(sg.k, sg.v, hq, n_q, qs, kvls, sm_scale, os, ls, w, w + pl.dec, pl.dec_bytes, 0, s);
  }
  if (e == hipSuccess)
    e = launch_seg_merge(nm, ml0, mls, mj0, mhq, mos, mlse, out, lacc, B, layers, n_q, q_heads, D, s);
  return hip_status(e);
}

kvq_status kvq_decode_attn_segments(const kvq_segment* segs, int32_t n_seg, int32_t layers, int32_t heads,
                                    int32_t tokens, int32_t q_heads, int32_t n_q, const uint16_t* q,
                                    const int32_t* kv_len, float sm_scale, float* out, float* lse, void* ws,
                                    size_t ws_bytes, void* stream) {
  return kvq_decode_attn_segments_ex(segs, n_seg, layers, heads, tokens, q_heads, n_q, q, kv_len, sm_scale, out, lse,
                                     ws, ws_bytes, 0, stream);
}

double kvq_effective_bits(const kvq_segment* segs, int32_t n_seg, int32_t layers, int32_t heads, int32_t tokens) {
  if (check_segments(segs, n_seg, layers, heads, tokens, heads, 1) != KVQ_OK) return -1.0;
  double tot = 0.0;
  for (int i = 0; i < n_seg; ++i) {
    const kvq_packed& k = *segs[i].k;
    const kvq_packed& v = *segs[i].v;
    const double b = 0.5 * (kvq_bits_per_value(&k.codec, k.shape.head_dim) +
                            kvq_bits_per_value(&v.codec, v.shape.head_dim));
    tot += b * k.shape.layers * k.shape.heads * k.shape.tokens;
  }
  return tot / ((double)layers * heads * tokens);
}

size_t kvq_attn_error_workspace(const kvq_shape* kv, int32_t q_heads, int32_t n_q) {
  if (check_shape(kv) != KVQ_OK || q_heads < 1 || n_q < 1) return 0;
  return kWsCounterBytes + error_ws_bytes(*kv, q_heads, n_q);
}

kvq_status kvq_attn_error_ex(const uint16_t* k_fp16, const uint16_t* v_fp16, const kvq_packed* k,
                             const kvq_packed* v, int32_t q_heads, int32_t n_q, const uint16_t* q,
                             const int32_t* kv_len, float sm_scale, const kvq_error_outputs* outs, void* ws,
                             size_t ws_bytes, void* stream) {
  kvq_status st = check_attn(k, v, q_heads, n_q, q);
  if (st != KVQ_OK) return st;
  if (!k_fp16 || !v_fp16 || !outs) return KVQ_ERR_ARG;
  const void* ptrs[] = {outs->kl, outs->relerr, outs->kv_err, outs->renyi2, outs->js, outs->logit_relerr, outs->top1};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KVQ_ERR_ALIGN;
  if (!aligned16(k_fp16) || !aligned16(v_fp16) || (kv_len && !aligned16(kv_len))) return KVQ_ERR_ALIGN;
  if (!(sm_scale >= 0.0f) || !std::isfinite(sm_scale)) return KVQ_ERR_ARG;
  const size_t need = kWsCounterBytes + error_ws_bytes(k->shape, q_heads, n_q);
  if (ws_bytes < need || (need && !ws)) return KVQ_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return KVQ_ERR_ALIGN;
  AttnProblem pr{};
  pr.k = k; pr.v = v; pr.Hq = q_heads; pr.n_q = n_q; pr.q = q; pr.kv_len = kv_len;
  pr.sm_scale = sm_scale > 0.0f ? sm_scale : (float)(1.0 / std::sqrt((double)k->shape.head_dim));
  pr.k16 = k_fp16; pr.v16 = v_fp16;
  pr.kl = outs->kl; pr.relerr = outs->relerr; pr.kv_err = outs->kv_err;
  pr.renyi2 = outs->renyi2; pr.js = outs->js; pr.logit_relerr = outs->logit_relerr; pr.top1 = outs->top1;
  pr.ctr = nullptr;                                  // same layout as decode; no counters used
  pr.ws = static_cast<char*>(ws) + kWsCounterBytes;
  pr.ws_bytes = ws_bytes - kWsCounterBytes;
  return hip_status(launch_attn_error(pr, (hipStream_t)stream));
}

kvq_status kvq_attn_error(const uint16_t* k_fp16, const uint16_t* v_fp16, const kvq_packed* k,
                          const kvq_packed* v, int32_t q_heads, int32_t n_q, const uint16_t* q,
                          const int32_t* kv_len, float sm_scale, float* kl_rows, float* relerr_rows,
                          double* kv_err, void* ws, size_t ws_bytes, void* stream) {
  if (!kl_rows || !relerr_rows || !kv_err) return KVQ_ERR_ARG;
  kvq_error_outputs o{};
  o.kl = kl_rows;
  o.relerr = relerr_rows;
  o.kv_err = kv_err;
  return kvq_attn_error_ex(k_fp16, v_fp16, k, v, q_heads, n_q, q, kv_len, sm_scale, &o, ws, ws_bytes, stream);
}

}  // extern "C"

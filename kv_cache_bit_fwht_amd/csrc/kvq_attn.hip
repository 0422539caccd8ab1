// Decode attention read back through the packed cache, and the attention-error
// reduction ([E22L] "Can 4-bit keys and 2-bit values hit a 1M-token memory
// budget?", What I tested: attention through the quantised post-RoPE cache;
// [E21W] "PROVISIONAL: known 3-bit KV cache methods ...", Benchmark: attention
// output relative error, KL of the attention distribution from f16, K/V squared
// error over signal energy).
//
// General kernel (every codec): split-K over tokens ("flash decoding").  Block
// (split s, KV head h, query row r) streams TB-token tiles: the K and V rows
// are dequantised by the same per-lane decode as kvq_dequant into padded LDS
// tiles, in the codec's own coordinates (rotated keys are met by a rotated
// query, rotated values are rotated back once per query in the combine; rFFT
// keys by the query's spectrum), then logits, online softmax and P.V for the
// G = Hq/H query heads that share the KV head.  Each block writes (m, l, o)
// partials; the combine kernel merges them with log-sum-exp weights.
#include <cmath>
#include <type_traits>

#include "kvq_codec.hpp"
#include "kvq_rfft.hpp"

namespace kvq {

constexpr int TB = 16;          // tokens per tile
constexpr int kMaxG = 8;
constexpr int kMaxSplits = 1024;   // split partials merged per query head

struct DevCodec {
  int cb, bits, g, W, ng;
  float kappa;
  size_t row_bytes;
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* mins;
  const float* chan;
  const float* mean;
  RfftCodec rc;
};

struct DirTables {
  float dir_c[256], dir_s[256];
};

struct AArgs {
  DevCodec k, v;
  const uint16_t* q;
  const int32_t* kv_len;
  const uint16_t* k16;
  const uint16_t* v16;
  float sm_scale;
  int B, L, H, T, D, Hq, G, n_q, S, chunk;
  int qp, nqg;         // wavefront decode: query rows per wavefront, row groups per (b, l)
  int lpt_log2;
  int Dc;              // coded key length (D, or 2*(D/2+1) for rFFT keys)
  float* ws;           // split partials
  float* dout;         // wavefront decode with one block per row: the output, written by the
  float* dlse;         // block merge itself (no combine launch); else null.  lse nullable
  const double* js_rowz;  // error kernel, JS pass: per row (ln Z of fp16, ln Z of quant), else null
  Tables tab;
  FftTables tw;        // twiddles of head_dim (rFFT keys: the query's DFT)
  DirTables dirs;      // phase-sector directions (rFFT polar keys)
};

// The problem-wide fields the wavefront body reads, as scalars (and the level tables by
// reference), so that the codec-map kernel hands its body values rather than the address
// of its large argument block (which the compiler would then copy to scratch).
struct WaveView {
  const uint16_t* q;
  const int32_t* kv_len;
  float* ws;
  float* dout;
  float* dlse;
  float sm_scale;
  int B, L, H, T, D, Hq, G, n_q, S, chunk, lpt_log2, qp, nqg;
  const Tables& tab;
};

// Error-kernel split partials: [2*D floats (o_quant, o_fp16)][kErrDoubles doubles]:
// m, l, m2, l2, A, S2 (sum e^{2(l - m2)}), LE (sum (lhat - l)^2), LL (sum l^2),
// argmax fp16, argmax quant, JS (second pass).
constexpr int kErrDoubles = 11;

// ------------------------------------------------------------------ tile dequantisation

template <int CB, int BITS>
__device__ __forceinline__ void dq_row(const DevCodec& c, long long row, int j, const Tables& tab, float v[16]) {
  uint32_t w[8], cc[16];
  uint16_t s16[2] = {0, 0}, z16[2] = {0, 0};
  load_chunk<BITS>(c.codes, (size_t)row * c.row_bytes + (size_t)j * 2 * BITS, w);
  if constexpr (CB != KVQ_FP16) {
    const size_t sbase = (size_t)row * c.ng;
    if (c.g == 8) {
      s16[0] = c.scales[sbase + 2 * j];
      s16[1] = c.scales[sbase + 2 * j + 1];
      if constexpr (CB == KVQ_INT_MINMAX) { z16[0] = c.mins[sbase + 2 * j]; z16[1] = c.mins[sbase + 2 * j + 1]; }
    } else {
      const int gi = (16 * j) / c.g;
      s16[0] = s16[1] = c.scales[sbase + gi];
      if constexpr (CB == KVQ_INT_MINMAX) z16[0] = z16[1] = c.mins[sbase + gi];
    }
  }
  unpack16<BITS>(w, cc);
  decode16<CB, BITS>(cc, s16, z16, tab, v);
}

__device__ __noinline__ void dq_row_any(const DevCodec& c, long long row, int j, const Tables& tab, float v[16]) {
  switch (c.cb) {
    case KVQ_FP16: dq_row<KVQ_FP16, 16>(c, row, j, tab, v); return;
    case KVQ_TERNARY: dq_row<KVQ_TERNARY, 2>(c, row, j, tab, v); return;
    case KVQ_SIGN: dq_row<KVQ_SIGN, 1>(c, row, j, tab, v); return;
    case KVQ_NF4: dq_row<KVQ_NF4, 4>(c, row, j, tab, v); return;
    case KVQ_INT8_SYM: dq_row<KVQ_INT8_SYM, 8>(c, row, j, tab, v); return;
    case KVQ_INT_ABSMAX:
      switch (c.bits) {
        case 2: dq_row<KVQ_INT_ABSMAX, 2>(c, row, j, tab, v); return;
        case 3: dq_row<KVQ_INT_ABSMAX, 3>(c, row, j, tab, v); return;
        case 4: dq_row<KVQ_INT_ABSMAX, 4>(c, row, j, tab, v); return;
        case 5: dq_row<KVQ_INT_ABSMAX, 5>(c, row, j, tab, v); return;
        case 6: dq_row<KVQ_INT_ABSMAX, 6>(c, row, j, tab, v); return;
        case 7: dq_row<KVQ_INT_ABSMAX, 7>(c, row, j, tab, v); return;
        default: dq_row<KVQ_INT_ABSMAX, 8>(c, row, j, tab, v); return;
      }
    case KVQ_INT_SYM:
      switch (c.bits) {
        case 2: dq_row<KVQ_INT_SYM, 2>(c, row, j, tab, v); return;
        case 3: dq_row<KVQ_INT_SYM, 3>(c, row, j, tab, v); return;
        case 4: dq_row<KVQ_INT_SYM, 4>(c, row, j, tab, v); return;
        case 5: dq_row<KVQ_INT_SYM, 5>(c, row, j, tab, v); return;
        case 6: dq_row<KVQ_INT_SYM, 6>(c, row, j, tab, v); return;
        case 7: dq_row<KVQ_INT_SYM, 7>(c, row, j, tab, v); return;
        default: dq_row<KVQ_INT_SYM, 8>(c, row, j, tab, v); return;
      }
    case KVQ_LLOYD:
      switch (c.bits) {
        case 2: dq_row<KVQ_LLOYD, 2>(c, row, j, tab, v); return;
        case 3: dq_row<KVQ_LLOYD, 3>(c, row, j, tab, v); return;
        default: dq_row<KVQ_LLOYD, 4>(c, row, j, tab, v); return;
      }
    default:
      switch (c.bits) {
        case 2: dq_row<KVQ_INT_MINMAX, 2>(c, row, j, tab, v); return;
        case 3: dq_row<KVQ_INT_MINMAX, 3>(c, row, j, tab, v); return;
        case 4: dq_row<KVQ_INT_MINMAX, 4>(c, row, j, tab, v); return;
        case 5: dq_row<KVQ_INT_MINMAX, 5>(c, row, j, tab, v); return;
        case 6: dq_row<KVQ_INT_MINMAX, 6>(c, row, j, tab, v); return;
        case 7: dq_row<KVQ_INT_MINMAX, 7>(c, row, j, tab, v); return;
        default: dq_row<KVQ_INT_MINMAX, 8>(c, row, j, tab, v); return;
      }
  }
}

// Rows [t0, t0+TB) of one unit (first row urow0) into tile[TB][RS] at pidx
// positions, in coded coordinates; rows at or beyond tend are zero.
__device__ void tile_dequant(const AArgs& a, const DevCodec& c, long long urow0, int t0, int tend, float* tile,
                             int RS) {
  const int tid = threadIdx.x;
  if (c.cb == KVQ_RFFT_POLAR || c.cb == KVQ_RFFT_CART) {
    const int F = c.rc.F;
    for (int it = tid; it < TB * F; it += kBlock) {
      const int r = it / F, f = it - r * F, t = t0 + r;
      float zr = 0.0f, zi = 0.0f;
      if (t < tend) {
        const long long row = urow0 + t;
        rfft_bin_value(c.rc, reinterpret_cast<const uint32_t*>(c.codes) + (size_t)row * c.rc.words,
                       c.scales + (size_t)row * c.rc.nscales, f, a.dirs.dir_c, a.dirs.dir_s, zr, zi);
      }
      tile[r * RS + pidx(f)] = zr;
      tile[r * RS + pidx(F + f)] = zi;
    }
    return;
  }
  const int LPT = 1 << a.lpt_log2, j = tid & (LPT - 1), rloc = tid >> a.lpt_log2, RPB = kBlock >> a.lpt_log2;
  for (int r0 = 0; r0 < TB; r0 += RPB) {
    const int r = r0 + rloc;
    if (r < TB) {
      const int t = t0 + r;
      float v[16];
      if (t < tend) {
        dq_row_any(c, urow0 + t, j, a.tab, v);
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = 0.0f;
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) tile[r * RS + pidx(16 * j + k)] = v[k];
    }
  }
}

// fp16 rows [t0, t0+TB) of one unit into tile (original coordinates).
__device__ void tile_fp16(const AArgs& a, const uint16_t* x, long long urow0, int t0, int tend, float* tile,
                          int RS) {
  for (int it = threadIdx.x; it < TB * a.D; it += kBlock) {
    const int r = it / a.D, d = it - r * a.D, t = t0 + r;
    tile[r * RS + pidx(d)] = (t < tend) ? h2f(x[(size_t)(urow0 + t) * a.D + d]) : 0.0f;
  }
}

// Normalised Walsh-Hadamard transform (width W) of `rows` LDS rows of D values
// (pidx layout, row stride RS); all threads call it.
__device__ void fwht_lds_rows(float* base, int rows, int RS, int D, int W, float kappa) {
  for (int s = 1; s < W; s <<= 1) {
    for (int p = threadIdx.x; p < rows * (D / 2); p += kBlock) {
      const int r = p / (D / 2), pp = p - r * (D / 2);
      const int i = (pp / s) * 2 * s + (pp % s);
      float* row = base + r * RS;
      const float x = row[pidx(i)], y = row[pidx(i + s)];
      row[pidx(i)] = x + y;
      row[pidx(i + s)] = x - y;
    }
    __syncthreads();
  }
  for (int p = threadIdx.x; p < rows * D; p += kBlock) {
    const int r = p / D, d = p - r * D;
    base[r * RS + pidx(d)] *= kappa;
  }
  __syncthreads();
}

// Query prologue: qc[g] = the query in the key codec's coordinates times the
// logit scale; optionally qr[g] = sigma * q in original coordinates.
__device__ void query_prologue(const AArgs& a, int b, int l, int i, int h, float* qc, float* qr, int RS) {
  const int D = a.D, G = a.G;
  const uint16_t* qsrc = a.q + ((((size_t)b * a.L + l) * a.n_q + i) * a.Hq + (size_t)h * G) * D;
  const float* kch = a.k.chan ? a.k.chan + ((size_t)l * a.H + h) * D : nullptr;
  for (int p = threadIdx.x; p < G * D; p += kBlock) {
    const int g = p / D, d = p - g * D;
    const float x = h2f(qsrc[(size_t)g * D + d]);
    if (qr) qr[g * RS + pidx(d)] = x * a.sm_scale;
    qc[g * RS + pidx(d)] = kch ? x / kch[d] : x;
  }
  __syncthreads();
  if (a.k.cb == KVQ_RFFT_POLAR || a.k.cb == KVQ_RFFT_CART) {
    // logit = sigma * sum_f w_f (Re Z_f Re Q_f + Im Z_f Im Q_f), Q = DFT(q), w = 1/N at f = 0, N/2 else 2/N
    const int N = D, F = N / 2 + 1;
    float* tmp = qc + G * RS;   // scratch row block (caller provides 2*G rows)
    for (int p = threadIdx.x; p < G * F; p += kBlock) {
      const int g = p / F, f = p - g * F;
      float sr = 0.0f, si = 0.0f;
      for (int n = 0; n < N; ++n) {
        const int m = (f * n) & (N - 1);
        const float cs = (m < N / 2) ? a.tw.tw_c[m] : -a.tw.tw_c[m - N / 2];
        const float sn = (m < N / 2) ? -a.tw.tw_s[m] : a.tw.tw_s[m - N / 2];   // sin(2 pi m / N)
        const float x = qc[g * RS + pidx(n)];
        sr += x * cs;
        si -= x * sn;
      }
      const float wf = ((f == 0 || f == N / 2) ? 1.0f : 2.0f) / (float)N * a.sm_scale;
      tmp[g * RS + pidx(f)] = sr * wf;
      tmp[g * RS + pidx(F + f)] = si * wf;
    }
    __syncthreads();
    for (int p = threadIdx.x; p < G * 2 * F; p += kBlock) {
      const int g = p / (2 * F), e = p - g * 2 * F;
      qc[g * RS + pidx(e)] = tmp[g * RS + pidx(e)];
    }
    __syncthreads();
    return;
  }
  if (a.k.W > 1) fwht_lds_rows(qc, G, RS, D, a.k.W, a.k.kappa);
  for (int p = threadIdx.x; p < G * D; p += kBlock) {
    const int g = p / D, d = p - g * D;
    qc[g * RS + pidx(d)] *= a.sm_scale;
  }
  __syncthreads();
}

template <typename T>
__device__ __forceinline__ T grp_max16(T v) {
#pragma unroll
  for (int m = 1; m < TB; m <<= 1) { const T o = __shfl_xor(v, m); v = v > o ? v : o; }
  return v;
}
template <typename T>
__device__ __forceinline__ T grp_min16(T v) {
#pragma unroll
  for (int m = 1; m < TB; m <<= 1) { const T o = __shfl_xor(v, m); v = v < o ? v : o; }
  return v;
}
template <typename T>
__device__ __forceinline__ T grp_sum16(T v) {
#pragma unroll
  for (int m = 1; m < TB; m <<= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float exp_t(float x) { return expf(x); }
__device__ __forceinline__ double exp_t(double x) { return exp(x); }

// ------------------------------------------------------------------ split kernel
//
// ERR = false: decode.  ERR = true: attention-error pass over fp16 and packed
// K/V together; its logits and softmax statistics are accumulated in fp64 (the
// error of a KL that is a small difference of large log-partition terms).

template <bool ERR>
__global__ __launch_bounds__(kBlock) void k_attn_split(AArgs a) {
  using acc_t = typename std::conditional<ERR, double, float>::type;
  extern __shared__ float smem[];
  const int RS = 17 * (a.D / 16) + 17;           // row stride of LDS rows (odd)
  float* qc = smem;                              // [2*G][RS] (second half: rFFT scratch)
  float* qr = qc + 2 * kMaxG * RS;               // [G][RS] (ERR)
  float* kt = qr + (ERR ? kMaxG * RS : 0);       // [TB][RS]
  float* vt = kt + TB * RS;                      // [TB][RS]
  float* kt2 = vt + TB * RS;                     // [TB][RS] fp16 K (ERR)
  float* vt2 = kt2 + (ERR ? TB * RS : 0);        // [TB][RS] fp16 V (ERR)
  float* pb = vt2 + (ERR ? TB * RS : 0);         // [G][TB] weights (quant)
  float* pb2 = pb + kMaxG * TB;                  // [G][TB] weights (fp16)
  acc_t* sc = reinterpret_cast<acc_t*>(pb2 + kMaxG * TB);   // [G][TB] logits (quant)
  acc_t* sc2 = sc + kMaxG * TB;                  // [G][TB] logits (fp16)
  acc_t* st = sc2 + kMaxG * TB;                  // stats [16][kMaxG]

  const int s = blockIdx.x, h = blockIdx.y;
  const long long rq = blockIdx.z;                // (b*L + l)*n_q + i
  const int i = (int)(rq % a.n_q);
  const int l = (int)((rq / a.n_q) % a.L);
  const int b = (int)(rq / ((long long)a.n_q * a.L));
  const int G = a.G, D = a.D, tid = threadIdx.x;
  const long long urow0 = (((long long)b * a.L + l) * a.H + h) * a.T;
  int n = a.T;
  if (a.kv_len) n = min(max(a.kv_len[rq], 0), a.T);
  const int tb0 = s * a.chunk, tb1 = min(tb0 + a.chunk, n);
  const acc_t NEG_INF = -(acc_t)INFINITY;

  query_prologue(a, b, l, i, h, qc, ERR ? qr : nullptr, RS);
  // stats: 0 m, 1 l, 2 alpha, 3 A, 4 m2, 5 l2, 6 alpha2, 7 S2, 8 LE, 9 LL, 10 argmax fp16,
  // 11 argmax quant, 12 JS, 13 q.mean (the quantised logits' shift when keys carry a mean)
  const bool jsp = ERR && a.js_rowz != nullptr;  // second pass: JS only
  if (tid < kMaxG) {
    st[0 * kMaxG + tid] = NEG_INF; st[1 * kMaxG + tid] = 0; st[2 * kMaxG + tid] = 1;
    st[3 * kMaxG + tid] = 0; st[4 * kMaxG + tid] = NEG_INF; st[5 * kMaxG + tid] = 0;
    st[6 * kMaxG + tid] = 1;
    if (ERR) {
      st[7 * kMaxG + tid] = 0; st[8 * kMaxG + tid] = 0; st[9 * kMaxG + tid] = 0;
      st[10 * kMaxG + tid] = -1; st[11 * kMaxG + tid] = -1; st[12 * kMaxG + tid] = 0;
      acc_t qm = 0;
      if (a.k.mean && tid < G) {
        const float* mp = a.k.mean + ((size_t)l * a.H + h) * D;
        for (int d = 0; d < D; ++d) qm += (acc_t)qr[tid * RS + pidx(d)] * (acc_t)mp[d];
      }
      st[13 * kMaxG + tid] = qm;
    }
  }
  float acc[kMaxG], acc2[kMaxG];
#pragma unroll
  for (int g = 0; g < kMaxG; ++g) { acc[g] = 0.0f; acc2[g] = 0.0f; }
  __syncthreads();

  for (int t0 = tb0; t0 < tb1; t0 += TB) {
    tile_dequant(a, a.k, urow0, t0, tb1, kt, RS);
    if (!jsp) tile_dequant(a, a.v, urow0, t0, tb1, vt, RS);
    if (ERR) {
      tile_fp16(a, a.k16, urow0, t0, tb1, kt2, RS);
      if (!jsp) tile_fp16(a, a.v16, urow0, t0, tb1, vt2, RS);
    }
    __syncthreads();
    if (tid < TB * G) {
      const int t = tid % TB, g = tid / TB;
      const bool valid = t0 + t < tb1;
      acc_t sq = 0;
      for (int e = 0; e < a.Dc; ++e) sq += (acc_t)qc[g * RS + pidx(e)] * (acc_t)kt[t * RS + pidx(e)];
      if (ERR) sq += st[13 * kMaxG + g];
      sc[g * TB + t] = valid ? sq : NEG_INF;
      if (ERR) {
        acc_t sr = 0;
        for (int d = 0; d < D; ++d) sr += (acc_t)qr[g * RS + pidx(d)] * (acc_t)kt2[t * RS + pidx(d)];
        sc2[g * TB + t] = valid ? sr : NEG_INF;
      }
    }
    __syncthreads();
    if (jsp) {   // JS terms with the final normalisers of both distributions
      if (tid < TB * G) {
        const int t = tid % TB, g = tid / TB;
        const acc_t x = sc2[g * TB + t], xq = sc[g * TB + t];
        const double* rz = a.js_rowz + ((size_t)rq * a.Hq + (size_t)h * G + g) * 2;
        const acc_t pp = (x == NEG_INF || rz[0] == NEG_INF) ? (acc_t)0 : exp_t(x - rz[0]);
        const acc_t rr = (xq == NEG_INF || rz[1] == NEG_INF) ? (acc_t)0 : exp_t(xq - rz[1]);
        const acc_t mm = (acc_t)0.5 * (pp + rr);
        acc_t term = 0;
        if (pp > 0) term += pp * log(pp / mm);
        if (rr > 0) term += rr * log(rr / mm);
        const acc_t js = grp_sum16(term);
        if (t == 0) st[12 * kMaxG + g] += (acc_t)0.5 * js;
      }
      __syncthreads();
      continue;
    }
    if (tid < TB * G) {
      const int t = tid % TB, g = tid / TB;
      {  // packed cache: online softmax
        const acc_t x = sc[g * TB + t];
        const acc_t mo = st[0 * kMaxG + g];
        const acc_t mt = grp_max16(x);
        if (ERR) {  // first index of the running maximum
          const acc_t cand = (x == mt && x != NEG_INF) ? (acc_t)(t0 + t) : (acc_t)INFINITY;
          const acc_t at = grp_min16(cand);
          if (t == 0 && mt > mo) st[11 * kMaxG + g] = at;
        }
        const acc_t M = mo > mt ? mo : mt;
        const acc_t p = (x == NEG_INF) ? (acc_t)0 : exp_t(x - M);
        const acc_t ps = grp_sum16(p);
        pb[g * TB + t] = (float)p;
        if (t == 0) {
          const acc_t al = (M == NEG_INF) ? (acc_t)1 : exp_t(mo - M);
          st[2 * kMaxG + g] = al;
          st[1 * kMaxG + g] = st[1 * kMaxG + g] * al + ps;
          st[0 * kMaxG + g] = M;
        }
      }
      if (ERR) {  // fp16 cache, and A = sum_t e^{l_t - m} (l_t - lhat_t)
        const acc_t x = sc2[g * TB + t], xq = sc[g * TB + t];
        const acc_t mo = st[4 * kMaxG + g];
        const acc_t mt = grp_max16(x);
        const acc_t M = mo > mt ? mo : mt;
        const acc_t p = (x == NEG_INF) ? (acc_t)0 : exp_t(x - M);
        const acc_t ps = grp_sum16(p);
        const acc_t pa = grp_sum16((x == NEG_INF) ? (acc_t)0 : p * (x - xq));
        const acc_t p2 = grp_sum16(p * p);
        const acc_t le = grp_sum16((x == NEG_INF) ? (acc_t)0 : (xq - x) * (xq - x));
        const acc_t ll = grp_sum16((x == NEG_INF) ? (acc_t)0 : x * x);
        const acc_t cand = (x == mt && x != NEG_INF) ? (acc_t)(t0 + t) : (acc_t)INFINITY;
        const acc_t at = grp_min16(cand);
        pb2[g * TB + t] = (float)p;
        if (t == 0) {
          const acc_t al = (M == NEG_INF) ? (acc_t)1 : exp_t(mo - M);
          st[6 * kMaxG + g] = al;
          st[5 * kMaxG + g] = st[5 * kMaxG + g] * al + ps;
          st[3 * kMaxG + g] = st[3 * kMaxG + g] * al + pa;
          st[7 * kMaxG + g] = st[7 * kMaxG + g] * al * al + p2;
          st[8 * kMaxG + g] += le;
          st[9 * kMaxG + g] += ll;
          if (mt > mo) st[10 * kMaxG + g] = at;
          st[4 * kMaxG + g] = M;
        }
      }
    }
    __syncthreads();
    if (tid < D) {
#pragma unroll
      for (int g = 0; g < kMaxG; ++g) {
        if (g >= G) break;
        float o = acc[g] * (float)st[2 * kMaxG + g];
#pragma unroll
        for (int t = 0; t < TB; ++t) o += pb[g * TB + t] * vt[t * RS + pidx(tid)];
        acc[g] = o;
        if (ERR) {
          float o2 = acc2[g] * (float)st[6 * kMaxG + g];
#pragma unroll
          for (int t = 0; t < TB; ++t) o2 += pb2[g * TB + t] * vt2[t * RS + pidx(tid)];
          acc2[g] = o2;
        }
      }
    }
    __syncthreads();
  }

  // partials: decode [rq][Hq][S][D+2 floats] = (o[D], m, l); error
  // [rq][Hq][S][2D floats + kErrDoubles doubles] (see kErrDoubles)
  const int P = ERR ? 2 * D + 2 * kErrDoubles : D + 2;
#pragma unroll
  for (int g = 0; g < kMaxG; ++g) {
    if (g >= G) break;
    float* dst = a.ws + ((rq * a.Hq + (size_t)h * G + g) * a.S + s) * P;
    if (tid < D) {
      dst[tid] = acc[g];
      if (ERR) dst[D + tid] = acc2[g];
    }
    if (tid == 0) {
      if (ERR) {
        double* dd = reinterpret_cast<double*>(dst + 2 * D);
        dd[0] = (double)st[0 * kMaxG + g];
        dd[1] = (double)st[1 * kMaxG + g];
        dd[2] = (double)st[4 * kMaxG + g];
        dd[3] = (double)st[5 * kMaxG + g];
        dd[4] = (double)st[3 * kMaxG + g];
#pragma unroll
        for (int k = 5; k < kErrDoubles; ++k) dd[k] = (double)st[(k + 2) * kMaxG + g];
      } else {
        dst[D] = (float)st[0 * kMaxG + g];
        dst[D + 1] = (float)st[1 * kMaxG + g];
      }
    }
  }
}

// ------------------------------------------------------------------ wavefront decode kernel
//
// The decode path of every codec except the rFFT keys.  Each wavefront owns one
// split (a token range) of one (query row, KV head) and runs on its own: lane
// (r, j) dequantises the 16 values j of row slot r straight into registers (the
// codec's per-lane decode, as kvq_dequant), the logits of up to 4 query heads are
// dot products against the query held in registers, reduced across the D/16
// lanes of the row, and the online softmax (log2 units, a reference maximum that
// moves only when a logit exceeds it by more than 8) and P.V accumulate per lane.
// No barrier in the loop; three iterations of code and scale loads are in flight.
// The wavefront's (o, m, l) partial is merged by the combine kernel.

constexpr int kWaveHeads = 4;     // query heads per wavefront (G > 4: several head groups)

template <int CB, int BITS>
struct RawChunk {                 // a lane's undecoded 16 values of one row
  uint32_t w[8];
  uint16_t s[2], z[2];            // fp16 scale (and min-max min) of values 0-7 and 8-15
};
template <int BITS>
struct RawChunk<-1, BITS> {       // the runtime-codec fallback loads as it decodes
  long long row;
};

template <int CB, int BITS>
__device__ __forceinline__ void raw_load(const DevCodec& c, long long row, int j, int glog2, RawChunk<CB, BITS>& r) {
  if constexpr (CB < 0) {
    r.row = row;
  } else {
    load_chunk<BITS>(c.codes, (size_t)row * c.row_bytes + (size_t)j * 2 * BITS, r.w);
    if constexpr (CB != KVQ_FP16) {
      // groups of values 0-7 and 8-15 of the lane (the same group unless g = 8)
      const size_t i0 = (size_t)row * c.ng + ((16 * j) >> glog2), i1 = (size_t)row * c.ng + ((16 * j + 8) >> glog2);
      r.s[0] = c.scales[i0];
      r.s[1] = c.scales[i1];
      if constexpr (CB == KVQ_INT_MINMAX) {
        r.z[0] = c.mins[i0];
        r.z[1] = c.mins[i1];
      }
    }
  }
}

template <int CB, int BITS>
__device__ __forceinline__ void raw_decode(const DevCodec& c, const RawChunk<CB, BITS>& r, int j, const Tables& tab,
                                           const float* nf4_lds, float v[16]) {
  if constexpr (CB < 0) {
    dq_row_any(c, r.row, j, tab, v);
  } else if constexpr (CB == KVQ_NF4 || CB == KVQ_LLOYD) {   // levels from LDS (a per-lane index)
    uint32_t cc[16];
    unpack16<BITS>(r.w, cc);
    const float s0 = h2f(r.s[0]), s1 = h2f(r.s[1]);
    const float* lv = (CB == KVQ_NF4) ? nf4_lds : nf4_lds + 16 * (BITS - 1);   // LLOYD b: after NF4's 16
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = lv[cc[i] & 15u] * (i < 8 ? s0 : s1);
  } else {
    uint32_t cc[16];
    unpack16<BITS>(r.w, cc);
    const uint16_t z0[2] = {0, 0};
    decode16<CB, BITS>(cc, r.s, CB == KVQ_INT_MINMAX ? r.z : z0, tab, v);
  }
}

// Sum over the lanes of a row (lpt = 4, 8 or 16 consecutive lanes) with DPP: quad
// swaps, then the half-row and row mirrors.  Every lane must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_lanes_sum(float x, int lpt) {
  x += dpp_mov<0xB1>(x);                             // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);                             // quad_perm [2,3,0,1]
  if (lpt >= 8) x += dpp_mov<0x141>(x);              // row_half_mirror
  if (lpt >= 16) x += dpp_mov<0x140>(x);             // row_mirror
  return x;
}

// rFFT keys: lane j of a row owns bins 8j .. 8j+7, whose first fields (magnitude or real
// codes) form one run of at most 64 bits and whose second fields (phase or imaginary
// codes) another, so three words hold each run; the last lane also takes the Nyquist
// bin.  A lane's 8 bins share one scale group (group >= 8).
struct RawRfft {
  uint32_t a[3], b[3];            // words holding the lane's first / second field runs
  uint32_t na[2], nb[2];          // words holding the Nyquist bin's fields
  uint16_t sa, sb, nsa, nsb;      // scales (Cartesian: real, imaginary) of the lane's group and the Nyquist bin
};

__device__ __forceinline__ uint32_t rfft_word(const uint32_t* w, int i, int words) { return w[min(i, words - 1)]; }

// nb bits at bit o (< 96, and o + nb <= 96) of the 3-word window w
// (selects between shifted values, not array elements, so the window stays in registers)
__device__ __forceinline__ uint32_t field3(const uint32_t w[3], int o, int nb) {
  const int wi = o >> 5, sh = o & 31;
  const uint32_t r0 = __builtin_amdgcn_alignbit(w[1], w[0], sh);
  const uint32_t r1 = __builtin_amdgcn_alignbit(w[2], w[1], sh);
  const uint32_t r2 = w[2] >> sh;
  return (wi == 0 ? r0 : (wi == 1 ? r1 : r2)) & ((1u << nb) - 1u);
}

__device__ __forceinline__ void rfft_raw_load(const DevCodec& c, long long row, int j, int lpt, RawRfft& r) {
  const RfftCodec& rc = c.rc;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(c.codes) + (size_t)row * rc.words;
  const uint16_t* sc = c.scales + (size_t)row * rc.nscales;
  const int ab = rc.bits, bb = (rc.cb == KVQ_RFFT_POLAR) ? rc.pbits : rc.bits;
  const int f0 = 8 * j, fN = rc.F - 1;
  const int wa = (f0 * ab) >> 5, wb = (rc.F * ab + f0 * bb) >> 5;
  const int wna = (fN * ab) >> 5, wnb = (rc.F * ab + fN * bb) >> 5;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    r.a[k] = rfft_word(w, wa + k, rc.words);
    r.b[k] = rfft_word(w, wb + k, rc.words);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    r.na[k] = rfft_word(w, wna + k, rc.words);
    r.nb[k] = rfft_word(w, wnb + k, rc.words);
  }
  const int gi = f0 / rc.g, gN = fN / rc.g;
  const int second = (rc.cb == KVQ_RFFT_POLAR) ? 0 : rc.ngroups;   // imaginary scales follow the real ones
  r.sa = sc[gi];
  r.sb = sc[second + gi];
  r.nsa = sc[gN];
  r.nsb = sc[second + gN];
  (void)lpt;
}

// The lane's spectrum values (bins 8j .. 8j+7, then the Nyquist bin) of one row.
__device__ __forceinline__ void rfft_raw_decode(const DevCodec& c, const RawRfft& r, int j, const float* dirc,
                                                const float* dirs, float zr[9], float zi[9]) {
  const RfftCodec& rc = c.rc;
  const bool polar = rc.cb == KVQ_RFFT_POLAR;
  const int ab = rc.bits, bb = polar ? rc.pbits : rc.bits;
  const int f0 = 8 * j, fN = rc.F - 1;
  const int oa = (f0 * ab) & 31, ob = (rc.F * ab + f0 * bb) & 31;
  const float off = (float)(1 << (ab - 1));
  const float sa = h2f(r.sa), sb = h2f(r.sb);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t A = field3(r.a, oa + k * ab, ab), B = field3(r.b, ob + k * bb, bb);
    if (polar) {
      const float mu = (float)A * sa;
      zr[k] = mu * dirc[B];
      zi[k] = mu * dirs[B];
    } else {
      zr[k] = ((float)A - off) * sa;
      zi[k] = ((float)B - off) * sb;
    }
  }
  const uint32_t wa3[3] = {r.na[0], r.na[1], 0u}, wb3[3] = {r.nb[0], r.nb[1], 0u};
  const uint32_t A = field3(wa3, (fN * ab) & 31, ab), B = field3(wb3, (rc.F * ab + fN * bb) & 31, bb);
  if (polar) {
    const float mu = (float)A * h2f(r.nsa);
    zr[8] = mu * dirc[B];
    zi[8] = mu * dirs[B];
  } else {
    zr[8] = ((float)A - off) * h2f(r.nsa);
    zi[8] = ((float)B - off) * h2f(r.nsb);
  }
}

// One block's work: the (query row, KV head h, head group, 4 splits) of blockIdx, with
// key codec kc and value codec vc whose rows of this unit start at urow0, and the key
// channel scales of the unit at kch (or null).  `a` holds the problem-wide fields.
template <int KCB, int KB, int VCB, int VB, typename A>
__device__ __forceinline__ void wave_unit(const A& a, const DevCodec& kc, const DevCodec& vc, float* smem,
                                          long long urow0, const float* kch) {
  constexpr bool KR = (KCB == KVQ_RFFT_POLAR || KCB == KVQ_RFFT_CART);
  using KRaw = typename std::conditional<KR, RawRfft, RawChunk<KCB, KB>>::type;
  const int D = a.D, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int RS = 17 * (D / 16) + 17;
  float* qc = smem;                                  // [kWaveHeads][RS] query rows
  const int lg = a.lpt_log2, LPT = 1 << lg, RPW = 64 >> lg;   // lanes per row, rows per wavefront step
  const int j = lane & (LPT - 1), r = lane >> lg;
  const int HG = (a.G + kWaveHeads - 1) / kWaveHeads;
  const int h = blockIdx.y / HG, hg = blockIdx.y - h * HG;
  const int GH = min(kWaveHeads, a.G - kWaveHeads * hg);      // query heads of this head group
  // The 4 slots of a wavefront: with qp == 1, query heads 4hg.. of one query row; with
  // qp > 1 (fewer than 4 query heads per KV head), the G heads of qp consecutive rows.
  const long long bl = (long long)blockIdx.z / a.nqg;         // b*L + l
  const int qg = (int)(blockIdx.z - bl * a.nqg);
  // slot g -> its query row ((b*L + l)*n_q + i) and query head, or row -1 (absent)
  const int qp = a.qp, Gq = a.G, nq = a.n_q;
  auto slot = [qp, Gq, nq, qg, bl, h, hg, GH](int g, long long& row, int& head) __attribute__((always_inline)) {
    int i;
    if (qp > 1) {
      i = qg * qp + g / Gq;
      head = h * Gq + g % Gq;
    } else {
      i = qg;
      head = h * Gq + kWaveHeads * hg + g;
    }
    const bool ok = (qp > 1) ? (i < nq) : (g < GH);
    row = ok ? bl * nq + i : -1;
  };
  const int split = blockIdx.x * (kBlock / 64) + wave;
  const int t_begin = split * a.chunk;
  int t_end_s[kWaveHeads];                           // per slot: end of its keys in this split
  int t_end = t_begin;                               // the furthest of them
#pragma unroll
  for (int g = 0; g < kWaveHeads; ++g) {
    long long row;
    int head;
    slot(g, row, head);
    int n = a.T;
    if (row >= 0 && a.kv_len) n = min(max(a.kv_len[row], 0), a.T);
    t_end_s[g] = row >= 0 ? min(t_begin + a.chunk, n) : t_begin;
    t_end = max(t_end, t_end_s[g]);
  }
  const int glog2k = 31 - __builtin_clz(kc.g > 0 ? kc.g : 1), glog2v = 31 - __builtin_clz(vc.g > 0 ? vc.g : 1);

  // ---- query prologue: the slots' query rows in the key codec's coordinates, times the
  // logit scale in log2 units; rows of absent slots are zero
  for (int p = tid; p < kWaveHeads * D; p += kBlock) {
    const int g = p / D, d = p - g * D;
    long long row;
    int head;
    slot(g, row, head);
    float x = (row >= 0) ? h2f(a.q[((size_t)row * a.Hq + head) * D + d]) : 0.0f;
    if (kch) x = x / kch[d];
    qc[g * RS + pidx(d)] = x;
  }
  if (tid < 64)                                      // NF4 levels, then the Lloyd-Max levels of 2, 3, 4 bits
    qc[2 * kWaveHeads * RS + 512 + kWaveHeads * 16 * 20 + tid] = tid < 16 ? a.tab.nf4_lv[tid]
                                                                          : a.tab.lloyd_lv[(tid >> 4) - 1][tid & 15];
  __syncthreads();
  const float lsc = a.sm_scale * 1.4426950408889634f;
  float q[kWaveHeads][16];                           // the query chunk (codec coordinates)
  float* dirc = qc + 2 * kWaveHeads * RS;            // rFFT polar keys: sector directions
  float* dirs = dirc + 256;
  // rFFT keys: per (head, lane j) the query spectrum of bins 8j .. 8j+7 and the Nyquist
  // bin: Re[0..7], Im[0..7], Re, Im, 2 pad (16-byte rows)
  float* qsp = dirs + 256;
  float* const nf4l = qsp + kWaveHeads * 16 * 20;    // NF4 and Lloyd-Max levels (written before the first barrier)
  if constexpr (KR) {
    // logit = sigma * sum_f w_f (Re Z_f Re Q_f + Im Z_f Im Q_f), Q = DFT(q), w = 1/N at f = 0, N/2, else 2/N
    const int N = D, F = N / 2 + 1;
    float* tmp = qc + kWaveHeads * RS;
    for (int p = tid; p < kWaveHeads * F; p += kBlock) {
      const int g = p / F, f = p - g * F;
      float sr = 0.0f, si = 0.0f;
      for (int nn = 0; nn < N; ++nn) {
        const int m = (f * nn) & (N - 1);
        const float cs = (m < N / 2) ? a.tw.tw_c[m] : -a.tw.tw_c[m - N / 2];
        const float sn = (m < N / 2) ? -a.tw.tw_s[m] : a.tw.tw_s[m - N / 2];   // sin(2 pi m / N)
        const float x = qc[g * RS + pidx(nn)];
        sr = __builtin_fmaf(x, cs, sr);
        si = __builtin_fmaf(-x, sn, si);
      }
      const float wf = ((f == 0 || f == N / 2) ? 1.0f : 2.0f) / (float)N * lsc;
      tmp[g * RS + pidx(f)] = sr * wf;
      tmp[g * RS + pidx(F + f)] = si * wf;
    }
    if (KCB == KVQ_RFFT_POLAR)
      for (int p = tid; p < (1 << kc.rc.pbits); p += kBlock) {
        dirc[p] = a.dirs.dir_c[p];
        dirs[p] = a.dirs.dir_s[p];
      }
    __syncthreads();
    for (int p = tid; p < kWaveHeads * LPT * 20; p += kBlock) {
      const int g = p / (LPT * 20), jj = (p / 20) % LPT, e = p % 20;
      float v = 0.0f;
      if (e < 16) v = tmp[g * RS + pidx((e < 8 ? 0 : F) + 8 * jj + (e & 7))];
      else if (jj == LPT - 1 && e == 16) v = tmp[g * RS + pidx(F - 1)];        // Nyquist bin (last lane)
      else if (jj == LPT - 1 && e == 17) v = tmp[g * RS + pidx(2 * F - 1)];
      qsp[p] = v;
    }
    __syncthreads();
  } else {
    if (kc.W > 1) fwht_lds_rows(qc, kWaveHeads, RS, D, kc.W, kc.kappa);
#pragma unroll
    for (int g = 0; g < kWaveHeads; ++g)
#pragma unroll
      for (int k = 0; k < 16; ++k) q[g][k] = qc[g * RS + pidx(16 * j + k)] * lsc;
  }

  float acc[kWaveHeads][16];
  float mref[kWaveHeads], lsum[kWaveHeads];
#pragma unroll
  for (int g = 0; g < kWaveHeads; ++g) {
    mref[g] = -INFINITY;
    lsum[g] = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[g][k] = 0.0f;
  }
  // rows past the split's last attended key re-read that key's row (weight 0, nothing
  // stored): rows at or past the keys attended may never have been written (a cache
  // filled by appends), and a weight of 0 times a code decoded from garbage can be NaN
  const int last_row = min(max(t_end, t_begin + 1) - 1, a.T - 1);
  auto load = [&](int it, KRaw& kr, RawChunk<VCB, VB>& vr) __attribute__((always_inline)) {
    const long long row = urow0 + min(t_begin + it * RPW + r, last_row);
    if constexpr (KR) rfft_raw_load(kc, row, j, LPT, kr);
    else raw_load<KCB, KB>(kc, row, j, glog2k, kr);
    raw_load<VCB, VB>(vc, row, j, glog2v, vr);
  };
  auto step = [&](int it, const KRaw& kr, const RawChunk<VCB, VB>& vr) __attribute__((always_inline)) {
    const int trow = t_begin + it * RPW + r;
    float kv[16], zr[9], zi[9];
    if constexpr (KR) rfft_raw_decode(kc, kr, j, dirc, dirs, zr, zi);
    else raw_decode<KCB, KB>(kc, kr, j, a.tab, nf4l, kv);
    float sc[kWaveHeads];
    bool grow = false;
#pragma unroll
    for (int g = 0; g < kWaveHeads; ++g) {
      float x = 0.0f;
      if constexpr (KR) {
        // the LDS offset is opaque per step, so the query spectrum is re-read here rather
        // than hoisted out of the loop into 80 loop-carried registers
        int qo = (g * LPT + j) * 20;
        asm volatile("" : "+v"(qo));
        const float4* qv = reinterpret_cast<const float4*>(qsp + qo);
        const float4 r0 = qv[0], r1 = qv[1], i0 = qv[2], i1 = qv[3], ny = qv[4];
        const float qr8[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
        const float qi8[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) x = __builtin_fmaf(qi8[k], zi[k], __builtin_fmaf(qr8[k], zr[k], x));
        x = __builtin_fmaf(ny.y, zi[8], __builtin_fmaf(ny.x, zr[8], x));
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) x = __builtin_fmaf(q[g][k], kv[k], x);
      }
      x = row_lanes_sum(x, LPT);
      sc[g] = (trow < t_end_s[g]) ? x : -INFINITY;
      grow |= sc[g] > mref[g] + 8.0f;
    }
    // the wavefront's maximum is only needed when some logit passes the reference by 8
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int g = 0; g < kWaveHeads; ++g) {
        float mt = sc[g];
        for (int m = LPT; m < 64; m <<= 1) mt = fmaxf(mt, __shfl_xor(mt, m));   // the same in every lane
        if (mt > mref[g] + 8.0f) {
          const float al = (mref[g] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mref[g] - mt);
          mref[g] = mt;
          lsum[g] *= al;
#pragma unroll
          for (int k = 0; k < 16; ++k) acc[g][k] *= al;
        }
      }
    }
    float vv[16];
    raw_decode<VCB, VB>(vc, vr, j, a.tab, nf4l, vv);
#pragma unroll
    for (int g = 0; g < kWaveHeads; ++g) {
      const float pw = (sc[g] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sc[g] - mref[g]);
      lsum[g] += pw;
#pragma unroll
      for (int k = 0; k < 16; ++k) acc[g][k] = __builtin_fmaf(pw, vv[k], acc[g][k]);
    }
  };
  const int n_it = (t_end > t_begin) ? (t_end - t_begin + RPW - 1) / RPW : 0;
  if constexpr (KR) {                                // two iterations in flight (registers)
    KRaw k0, k1;
    RawChunk<VCB, VB> v0, v1;
    load(0, k0, v0);
    load(1, k1, v1);
    for (int it = 0; it < n_it; it += 2) {
      step(it, k0, v0);
      load(it + 2, k0, v0);
      if (it + 1 >= n_it) break;
      step(it + 1, k1, v1);
      load(it + 3, k1, v1);
    }
  } else {
    KRaw k0, k1, k2;
    RawChunk<VCB, VB> v0, v1, v2;
    load(0, k0, v0);
    load(1, k1, v1);
    load(2, k2, v2);
    for (int it = 0; it < n_it; it += 3) {
      step(it, k0, v0);
      load(it + 3, k0, v0);
      if (it + 1 >= n_it) break;
      step(it + 1, k1, v1);
      load(it + 4, k1, v1);
      if (it + 2 >= n_it) break;
      step(it + 2, k2, v2);
      load(it + 5, k2, v2);
    }
  }
  // ---- sum the row slots, then merge the block's 4 wavefronts (4 consecutive splits)
  // through LDS into one partial per query head: o in the codec's value coordinates,
  // m in natural-log units, l.  Partial index: blockIdx.x of gridDim.x per row.
#pragma unroll
  for (int g = 0; g < kWaveHeads; ++g) {
    for (int m = LPT; m < 64; m <<= 1) lsum[g] += __shfl_xor(lsum[g], m);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      for (int m = LPT; m < 64; m <<= 1) acc[g][k] += __shfl_xor(acc[g][k], m);
  }
  constexpr int NW = kBlock / 64;
  __syncthreads();                                   // every wavefront is past its last LDS read
  float* mo = smem;                                  // [NW][kWaveHeads][D] wavefront outputs
  float* mm = mo + NW * kWaveHeads * D;              // [NW][kWaveHeads] reference maxima (log2 units)
  float* ml = mm + NW * kWaveHeads;                  // [NW][kWaveHeads] sums
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < kWaveHeads; ++g) {
#pragma unroll
      for (int k = 0; k < 16; ++k) mo[(wave * kWaveHeads + g) * D + 16 * j + k] = acc[g][k];
      if (j == 0) {
        mm[wave * kWaveHeads + g] = mref[g];
        ml[wave * kWaveHeads + g] = lsum[g];
      }
    }
  }
  __syncthreads();
  constexpr float kLn2 = 0.6931471805599453f;
  const int P = D + 2;
  for (int p = tid; p < kWaveHeads * D; p += kBlock) {
    const int g = p / D, d = p - g * D;
    long long row;
    int head;
    slot(g, row, head);
    if (row < 0) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mm[w * kWaveHeads + g]);
    float o = 0.0f, lw = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float m = mm[w * kWaveHeads + g];
      const float wt = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
      o = __builtin_fmaf(wt, mo[(w * kWaveHeads + g) * D + d], o);
      lw = __builtin_fmaf(wt, ml[w * kWaveHeads + g], lw);
    }
    if (a.dout) {
      // the only partial of its row: what the combine would make of it (its fp64 steps)
      const double lq = (double)lw;
      a.dout[((size_t)row * a.Hq + head) * D + d] = lq > 0.0 ? (float)((double)o / lq) : 0.0f;
      if (d == 0 && a.dlse)
        a.dlse[(size_t)row * a.Hq + head] = lq > 0.0 ? (float)((double)(M * kLn2) + log(lq)) : -INFINITY;
      continue;
    }
    float* dst = a.ws + (((size_t)row * a.Hq + head) * gridDim.x + blockIdx.x) * P;
    dst[d] = o;
    if (d == 0) {
      dst[D] = (M == -INFINITY) ? -INFINITY : M * kLn2;
      dst[D + 1] = lw;
    }
  }
}

template <int KCB, int KB, int VCB, int VB>
__global__ __launch_bounds__(kBlock) void k_decode_wave(AArgs a) {
  extern __shared__ float smem[];
  const int HG = (a.G + kWaveHeads - 1) / kWaveHeads;
  const int h = blockIdx.y / HG;
  const long long bl = (long long)blockIdx.z / a.nqg;          // b*L + l
  const int l = (int)(bl % a.L);
  const int b = (int)(bl / a.L);
  const long long urow0 = (((long long)b * a.L + l) * a.H + h) * a.T;
  const float* kch = a.k.chan ? a.k.chan + ((size_t)l * a.H + h) * a.D : nullptr;
  wave_unit<KCB, KB, VCB, VB>(a, a.k, a.v, smem, urow0, kch);
}

// ------------------------------------------------------------------ codec maps in one launch
//
// A cache tiled into (layer range x KV-head range) tiles, each stored with its own key
// and value codecs over every token: per-layer bit allocations ([E21W] Result, the
// 3.19-bit allocation) and per-head bit widths ([LCPP] Finding 2).  One launch decodes
// all of it: each block finds the tile of its (layer, KV head) and runs the compiled
// decode of that tile's codec pair, so blocks of different pairs share the launch.
// The pairs compiled in (id, key codebook, key bits, value codebook, value bits):
#define KVQ_MIX_PAIRS(X)                                                                        \
  X(0, KVQ_INT_ABSMAX, 2, KVQ_INT_ABSMAX, 2) X(1, KVQ_INT_ABSMAX, 2, KVQ_INT_ABSMAX, 3)         \
  X(2, KVQ_INT_ABSMAX, 2, KVQ_INT_ABSMAX, 4) X(3, KVQ_INT_ABSMAX, 3, KVQ_INT_ABSMAX, 2)         \
  X(4, KVQ_INT_ABSMAX, 3, KVQ_INT_ABSMAX, 3) X(5, KVQ_INT_ABSMAX, 3, KVQ_INT_ABSMAX, 4)         \
  X(6, KVQ_INT_ABSMAX, 4, KVQ_INT_ABSMAX, 2) X(7, KVQ_INT_ABSMAX, 4, KVQ_INT_ABSMAX, 3)         \
  X(8, KVQ_INT_ABSMAX, 4, KVQ_INT_ABSMAX, 4) X(9, KVQ_INT_ABSMAX, 5, KVQ_INT_ABSMAX, 2)         \
  X(10, KVQ_INT_ABSMAX, 5, KVQ_INT_ABSMAX, 3) X(11, KVQ_INT_ABSMAX, 5, KVQ_INT_ABSMAX, 4)       \
  X(12, KVQ_INT_ABSMAX, 6, KVQ_INT_ABSMAX, 2) X(13, KVQ_INT_ABSMAX, 6, KVQ_INT_ABSMAX, 3)       \
  X(14, KVQ_INT_ABSMAX, 6, KVQ_INT_ABSMAX, 4) X(15, KVQ_FP16, 16, KVQ_FP16, 16)                 \
  X(16, KVQ_INT8_SYM, 8, KVQ_INT8_SYM, 8) X(17, KVQ_TERNARY, 2, KVQ_TERNARY, 2)                 \
  X(18, KVQ_SIGN, 1, KVQ_SIGN, 1) X(19, KVQ_NF4, 4, KVQ_INT_ABSMAX, 4)

struct MixCodec {        // the fields of DevCodec the wavefront decode reads
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* mins;
  const float* chan;
  int row_bytes, ng, g, W;
  float kappa;
  int cb, bits;
};

struct MixTile {         // layers [l0, l0 + ls) x KV heads [h0, h0 + hs), all tokens
  MixCodec k, v;
  int l0, ls, h0, hs;
  int pair;              // index into KVQ_MIX_PAIRS
};

struct MArgs {
  const uint16_t* q;
  const int32_t* kv_len;
  float* ws;             // split partials, as the single-codec kernel writes them
  float sm_scale;
  int B, L, H, T, D, Hq, G, n_q, S, chunk, lpt_log2;
  int qp, nqg;           // query rows per wavefront, row groups per (b, l)
  int ntiles;
  Tables tab;
  MixTile tile[kMaxSegments];
};

__device__ __forceinline__ DevCodec mix_codec(const MixCodec& m) {
  DevCodec c{};
  c.cb = m.cb;
  c.bits = m.bits;
  c.g = m.g;
  c.W = m.W;
  c.ng = m.ng;
  c.kappa = m.kappa;
  c.row_bytes = (size_t)m.row_bytes;
  c.codes = m.codes;
  c.scales = m.scales;
  c.mins = m.mins;
  c.chan = m.chan;
  return c;
}

__global__ __launch_bounds__(kBlock) void k_decode_wave_mix(MArgs a) {
  extern __shared__ float smem[];
  const int HG = (a.G + kWaveHeads - 1) / kWaveHeads;
  const int h = blockIdx.y / HG;
  const long long bl = (long long)blockIdx.z / a.nqg;          // b*L + l
  const int l = (int)(bl % a.L);
  const int b = (int)(bl / a.L);
  int ti = 0;                                        // the tiles cover every (layer, head) once
  while (ti + 1 < a.ntiles) {
    const MixTile& t = a.tile[ti];
    if (l >= t.l0 && l < t.l0 + t.ls && h >= t.h0 && h < t.h0 + t.hs) break;
    ++ti;
  }
  const MixTile& t = a.tile[ti];
  const int ll = l - t.l0, hl = h - t.h0;            // the unit inside its tile's arrays
  const long long urow0 = (((long long)b * t.ls + ll) * t.hs + hl) * a.T;
  const DevCodec kc = mix_codec(t.k), vc = mix_codec(t.v);
  const float* kch = kc.chan ? kc.chan + ((size_t)ll * t.hs + hl) * a.D : nullptr;
  const WaveView v{a.q, a.kv_len, a.ws, nullptr, nullptr, a.sm_scale, a.B, a.L, a.H, a.T, a.D, a.Hq, a.G, a.n_q, a.S, a.chunk,
                   a.lpt_log2, a.qp, a.nqg, a.tab};
  switch (t.pair) {
#define KVQ_MIX_CASE(id, KCB, KB, VCB, VB) \
  case id: wave_unit<KCB, KB, VCB, VB>(v, kc, vc, smem, urow0, kch); break;
    KVQ_MIX_PAIRS(KVQ_MIX_CASE)
#undef KVQ_MIX_CASE
    default: break;
  }
}

// ------------------------------------------------------------------ combine

// One block per (query row, query head).  Merges the S split partials:
// M = max m_s, L = sum l_s e^{m_s - M}, o = sum o_s e^{m_s - M} / L; then
// rotates o back if V was rotated and divides V's per-channel scale.
struct MixV {            // a tile of a codec map: its value rotation and channel scales, its key mean
  int l0, ls, h0, hs, vW;
  float vkappa;
  const float* vchan;    // [ls][hs][D] or null
  const float* kmean;    // [ls][hs][D] or null
};

struct CArgs {
  const float* ws;
  int S, D, Hq, G, H, L, n_q;
  int vW;
  float vkappa;
  const float* vchan;
  int* ctr;             // decode chunk counters to set back to zero, or null
  int ntiles;           // > 0: a codec map; the tile of (layer, KV head) gives vW, vkappa, vchan
  const uint16_t* q;    // codec map: the queries, for the lse shift of a tile's key mean
  float sm;             // codec map: the logit scale
  MixV tile[kMaxSegments];
};

struct ErrOut {          // error outputs beyond KL / relative error (each nullable)
  float* renyi2;
  float* logit_relerr;
  float* top1;
  double* rowz;          // per row (ln Z fp16, ln Z quant) for the JS pass
};

template <bool ERR>
__global__ __launch_bounds__(kBlock) void k_attn_combine(CArgs a, float* out, float* lse, float* kl,
                                                         float* relerr, ErrOut eo) {
  __shared__ float orow[17 * 16 + 17];
  __shared__ double wq[kMaxSplits], w2[kMaxSplits];   // per-split weights e^{m_s - M}
  __shared__ double red[6][kBlock];
  const long long rh = blockIdx.x;               // rq * Hq + j
  const int j = (int)(rh % a.Hq);
  const long long rq = rh / a.Hq;
  const int l = (int)((rq / a.n_q) % a.L);
  const int h = j / a.G;
  const int D = a.D, tid = threadIdx.x;
  const int P = ERR ? 2 * D + 2 * kErrDoubles : D + 2;
  const float* src = a.ws + (size_t)rh * a.S * P;
  // per split: m, l (packed cache) and m2, l2, A (fp16 cache)
  auto stat = [&](int s, int k) -> double {
    const float* p = src + (size_t)s * P;
    if (ERR) return reinterpret_cast<const double*>(p + 2 * D)[k];
    return (double)p[D + k];
  };
  // 1. maxima over splits
  double mx = -INFINITY, mx2 = -INFINITY;
  for (int s = tid; s < a.S; s += kBlock) {
    mx = fmax(mx, stat(s, 0));
    if (ERR) mx2 = fmax(mx2, stat(s, 2));
  }
  red[0][tid] = mx;
  red[1][tid] = mx2;
  __syncthreads();
  for (int st = kBlock / 2; st > 0; st >>= 1) {
    if (tid < st) {
      red[0][tid] = fmax(red[0][tid], red[0][tid + st]);
      red[1][tid] = fmax(red[1][tid], red[1][tid + st]);
    }
    __syncthreads();
  }
  const double M = red[0][0], M2 = red[1][0];
  __syncthreads();
  // 2. split weights and the normalisers
  double lq = 0.0, l2 = 0.0, aa = 0.0, s2 = 0.0, le = 0.0, ll = 0.0;
  for (int s = tid; s < a.S; s += kBlock) {
    const double ms = stat(s, 0);
    const double w = (M == -INFINITY || ms == -INFINITY) ? 0.0 : exp(ms - M);
    wq[s] = w;
    lq += stat(s, 1) * w;
    if (ERR) {
      const double m2s = stat(s, 2);
      const double v = (M2 == -INFINITY || m2s == -INFINITY) ? 0.0 : exp(m2s - M2);
      w2[s] = v;
      l2 += stat(s, 3) * v;
      aa += stat(s, 4) * v;
      s2 += stat(s, 5) * v * v;
      le += stat(s, 6);
      ll += stat(s, 7);
    }
  }
  red[0][tid] = lq;
  red[1][tid] = l2;
  red[2][tid] = aa;
  red[3][tid] = s2;
  red[4][tid] = le;
  red[5][tid] = ll;
  __syncthreads();
  for (int st = kBlock / 2; st > 0; st >>= 1) {
    if (tid < st) {
#pragma unroll
      for (int k = 0; k < 6; ++k) red[k][tid] += red[k][tid + st];
    }
    __syncthreads();
  }
  const double Lq = red[0][0], L2 = red[1][0], A = red[2][0], S2 = red[3][0], LE = red[4][0], LL = red[5][0];
  // 3. outputs, one dimension per thread (coalesced over the partial rows)
  float o = 0.0f, o2 = 0.0f;
  if (tid < D) {
    double acc = 0.0, acc2 = 0.0;
    int s = 0;
    // eight splits' loads in flight at a time; the sums keep split order
    for (; s + 8 <= a.S; s += 8) {
      float v[8], v2[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* p = src + (size_t)(s + u) * P;
        v[u] = p[tid];
        if (ERR) v2[u] = p[D + tid];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc += (double)v[u] * wq[s + u];
        if (ERR) acc2 += (double)v2[u] * w2[s + u];
      }
    }
    for (; s < a.S; ++s) {
      const float* p = src + (size_t)s * P;
      acc += (double)p[tid] * wq[s];
      if (ERR) acc2 += (double)p[D + tid] * w2[s];
    }
    o = Lq > 0.0 ? (float)(acc / Lq) : 0.0f;
    if (ERR) o2 = L2 > 0.0 ? (float)(acc2 / L2) : 0.0f;
    orow[pidx(tid)] = o;
  }
  __syncthreads();
  int vW = a.vW;
  float vkappa = a.vkappa;
  const float* vchan = a.vchan ? a.vchan + ((size_t)l * a.H + h) * D : nullptr;
  const float* kmean = nullptr;
  if (a.ntiles > 0) {                            // the tile of (l, h); the tiles cover each once
    int ti = 0;
    while (ti + 1 < a.ntiles) {
      const MixV& t = a.tile[ti];
      if (l >= t.l0 && l < t.l0 + t.ls && h >= t.h0 && h < t.h0 + t.hs) break;
      ++ti;
    }
    const MixV& t = a.tile[ti];
    const size_t u = ((size_t)(l - t.l0) * t.hs + (h - t.h0)) * D;
    vW = t.vW;
    vkappa = t.vkappa;
    vchan = t.vchan ? t.vchan + u : nullptr;
    kmean = t.kmean ? t.kmean + u : nullptr;
  }
  if (vW > 1) fwht_lds_rows(orow, 1, 0, D, vW, vkappa);
  if (tid < D) {
    o = orow[pidx(tid)];
    if (vchan) o = o / vchan[tid];
  }
  if (!ERR) {
    // a tile whose keys carry a mean: every logit of the row is larger by q.mean, so the
    // weights stay and the lse moves by sm * q.mean
    float shift = 0.0f;
    if (kmean && lse) {
      red[0][tid] = (tid < D) ? (double)h2f(a.q[(size_t)rh * D + tid]) * (double)kmean[tid] : 0.0;
      __syncthreads();
      for (int st = kBlock / 2; st > 0; st >>= 1) {
        if (tid < st) red[0][tid] += red[0][tid + st];
        __syncthreads();
      }
      shift = a.sm * (float)red[0][0];
    }
    if (tid < D) out[(size_t)rh * D + tid] = o;
    if (tid == 0 && lse) lse[rh] = (Lq > 0.0) ? (float)(M + log(Lq)) + shift : -INFINITY;
    if (tid == 0 && a.ctr && j % a.G == 0) a.ctr[rq * a.H + h] = 0;   // ready for the next call
    return;
  }
  // relative error of the quantised output against the fp16 one, and KL
  __syncthreads();
  const float dlt = (tid < D) ? (o - o2) : 0.0f;
  red[0][tid] = (double)dlt * dlt;
  red[1][tid] = (tid < D) ? (double)o2 * o2 : 0.0;
  __syncthreads();
  for (int st = kBlock / 2; st > 0; st >>= 1) {
    if (tid < st) {
      red[0][tid] += red[0][tid + st];
      red[1][tid] += red[1][tid + st];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double num = red[0][0], den = red[1][0];
    if (relerr) relerr[rh] = den > 0.0 ? (float)(sqrt(num) / sqrt(den)) : 0.0f;
    double k = 0.0;
    if (L2 > 0.0 && Lq > 0.0) k = A / L2 - (M2 + log(L2)) + (M + log(Lq));
    if (kl) kl[rh] = (float)k;
    if (eo.renyi2) eo.renyi2[rh] = L2 > 0.0 ? (float)(2.0 * log(L2) - log(S2)) : 0.0f;
    if (eo.logit_relerr) eo.logit_relerr[rh] = LL > 0.0 ? (float)(sqrt(LE) / sqrt(LL)) : 0.0f;
    if (eo.top1) {
      // the first key holding the maximum: the earliest split reaching it, then its first index
      double a2 = -1.0, aq = -1.0;
      for (int s = 0; s < a.S && a2 < 0.0; ++s)
        if (stat(s, 2) == M2 && M2 != -INFINITY) a2 = stat(s, 8);
      for (int s = 0; s < a.S && aq < 0.0; ++s)
        if (stat(s, 0) == M && M != -INFINITY) aq = stat(s, 9);
      eo.top1[rh] = (L2 > 0.0 && a2 != aq) ? 1.0f : 0.0f;
    }
    if (eo.rowz) {
      eo.rowz[rh * 2 + 0] = L2 > 0.0 ? M2 + log(L2) : -INFINITY;
      eo.rowz[rh * 2 + 1] = Lq > 0.0 ? M + log(Lq) : -INFINITY;
    }
  }
}

// JS of a row: the second pass's split partials summed in split order.
__global__ void k_js_final(const float* __restrict__ ws, int S, int P, int D, long long rows, float* __restrict__ js) {
  const long long rh = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (rh >= rows) return;
  double t = 0.0;
  for (int s = 0; s < S; ++s) t += reinterpret_cast<const double*>(ws + ((size_t)rh * S + s) * P + 2 * D)[10];
  js[rh] = (float)t;
}

// ------------------------------------------------------------------ K/V squared error

struct EArgs {
  DevCodec c;
  const uint16_t* x;
  int T, H, L, D, lpt_log2, chunks;
  double* part;     // [units][chunks][2]
  Tables tab;
};

__global__ __launch_bounds__(kBlock) void k_kverr(EArgs a) {
  __shared__ double red[2][kBlock];
  const int tid = threadIdx.x;
  const int LPT = 1 << a.lpt_log2, j = tid & (LPT - 1), rloc = tid >> a.lpt_log2, RPB = kBlock >> a.lpt_log2;
  const long long unit = blockIdx.y;
  const int per = (a.T + a.chunks - 1) / a.chunks;
  const int t0 = blockIdx.x * per, t1 = min(a.T, t0 + per);
  const float* cp = nullptr;
  const float* mp = nullptr;
  {
    const int h = (int)(unit % a.H), l = (int)((unit / a.H) % a.L);
    if (a.c.chan) cp = a.c.chan + ((size_t)l * a.H + h) * a.D + 16 * j;
    if (a.c.mean) mp = a.c.mean + ((size_t)l * a.H + h) * a.D + 16 * j;
  }
  double se = 0.0, sx = 0.0;
  for (int tb = t0; tb < t1; tb += RPB) {
    const int t = tb + rloc;
    const bool active = t < t1;
    const long long row = unit * a.T + t;
    float v[16];
    if (active) {
      dq_row_any(a.c, row, j, a.tab, v);
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = 0.0f;
    }
    if (a.c.W > 1) fwht_rows(v, j, a.c.W, a.c.kappa);
    if (active) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        float y = cp ? __fdiv_rn(v[k], cp[k]) : v[k];
        if (mp) y = y + mp[k];
        const double x = (double)h2f(a.x[(size_t)row * a.D + 16 * j + k]);
        const double d = (double)y - x;
        se += d * d;
        sx += x * x;
      }
    }
  }
  red[0][tid] = se;
  red[1][tid] = sx;
  __syncthreads();
  for (int st = kBlock / 2; st > 0; st >>= 1) {
    if (tid < st) { red[0][tid] += red[0][tid + st]; red[1][tid] += red[1][tid + st]; }
    __syncthreads();
  }
  if (tid == 0) {
    a.part[(unit * a.chunks + blockIdx.x) * 2 + 0] = red[0][0];
    a.part[(unit * a.chunks + blockIdx.x) * 2 + 1] = red[1][0];
  }
}

// Fixed-order sum of the chunk partials: kv_err[unit] = (dK^2, K^2, dV^2, V^2).
__global__ void k_kverr_final(const double* pk, const double* pv, int chunks, long long units, double* out) {
  const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;
  double a0 = 0, a1 = 0, b0 = 0, b1 = 0;
  for (int c = 0; c < chunks; ++c) {
    a0 += pk[(u * chunks + c) * 2]; a1 += pk[(u * chunks + c) * 2 + 1];
    b0 += pv[(u * chunks + c) * 2]; b1 += pv[(u * chunks + c) * 2 + 1];
  }
  out[u * 4 + 0] = a0; out[u * 4 + 1] = a1; out[u * 4 + 2] = b0; out[u * 4 + 3] = b1;
}

// A shared key mean adds q.mean to every logit of a query (a constant per row, so
// the attention weights do not move): lse[row] += sm * q.mean[l][kv head].  One
// wavefront per (b, l, query, query head) row.
__global__ __launch_bounds__(kBlock) void k_lse_mean(const uint16_t* __restrict__ q, const float* __restrict__ mean,
                                                     float* __restrict__ lse, long long rows, int L, int n_q, int Hq,
                                                     int H, int D, float sm) {
  const long long row = (long long)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;                       // the whole wavefront shares the row
  const int jq = (int)(row % Hq);
  const int l = (int)((row / ((long long)Hq * n_q)) % L);
  const int kvh = jq / (Hq / H);
  const uint16_t* qp = q + row * D;
  const float* mp = mean + ((size_t)l * H + kvh) * D;
  float s = 0.0f;
  for (int d = lane; d < D; d += 64) s += h2f(qp[d]) * mp[d];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if (lane == 0) lse[row] = lse[row] + sm * s;   // -inf (no keys) stays -inf
}

// ------------------------------------------------------------------ host side

static int lpt_log2_of(int D) { return D == 64 ? 2 : D == 128 ? 3 : 4; }

static float kappa_of(int W) {
  if (W <= 1) return 1.0f;
  int e = 0;
  while ((1 << e) < W) ++e;
  return (e % 2 == 0) ? ldexpf(1.0f, -e / 2) : (float)(1.0 / std::sqrt((double)W));
}

static DevCodec dev_codec(const kvq_packed& p) {
  DevCodec c{};
  c.cb = p.codec.codebook;
  c.bits = p.codec.bits;
  c.g = p.codec.group;
  c.W = p.codec.rot_width > 1 ? p.codec.rot_width : 0;
  c.kappa = kappa_of(c.W);
  const int D = p.shape.head_dim;
  int b = p.codec.bits;
  switch (c.cb) {
    case KVQ_FP16: b = 16; break;
    case KVQ_TERNARY: b = 2; break;
    case KVQ_SIGN: b = 1; break;
    case KVQ_NF4: b = 4; break;
    case KVQ_INT8_SYM: b = 8; break;
    default: break;
  }
  c.row_bytes = (size_t)D * b / 8;
  c.ng = (c.cb == KVQ_FP16 || c.g == 0) ? 0 : D / c.g;
  c.codes = reinterpret_cast<const uint8_t*>(p.codes);
  c.scales = p.scales;
  c.mins = p.mins;
  c.chan = p.chan_scale;
  c.mean = p.mean;
  if (c.cb == KVQ_RFFT_POLAR || c.cb == KVQ_RFFT_CART) {
    RfftCodec& r = c.rc;
    r.cb = c.cb;
    r.N = D;
    r.F = D / 2 + 1;
    r.bits = p.codec.bits;
    r.pbits = (c.cb == KVQ_RFFT_POLAR) ? p.codec.aux_bits : 0;
    r.g = p.codec.group;
    r.ngroups = (r.F + r.g - 1) / r.g;
    r.nscales = (c.cb == KVQ_RFFT_POLAR) ? r.ngroups : 2 * r.ngroups;
    const long bits = (c.cb == KVQ_RFFT_POLAR) ? (long)r.F * (r.bits + r.pbits) : 2L * r.F * r.bits;
    r.words = (int)((bits + 31) / 32);
  }
  return c;
}

int decode_splits(const kvq_shape& s, int Hq, int n_q) {
  (void)Hq;
  const long long pairs = (long long)s.batch * s.layers * n_q * s.heads;
  const int max_s = std::max(1, (s.tokens + TB - 1) / TB);
  long long S = (2048 + pairs - 1) / pairs;
  if (S < 1) S = 1;
  if (S > max_s) S = max_s;
  if (S > kMaxSplits) S = kMaxSplits;
  // equalise: chunk is a multiple of TB; recompute S so no split is empty
  const int chunk = (int)(((s.tokens + S - 1) / S + TB - 1) / TB * TB);
  return chunk > 0 ? std::max(1, (s.tokens + chunk - 1) / chunk) : 1;
}

static int split_chunk(const kvq_shape& s, int S) {
  const int c = ((s.tokens + S - 1) / S + TB - 1) / TB * TB;
  return c > 0 ? c : TB;
}

// Splits (one wavefront each) of the wavefront decode kernel: about 8192 wavefronts
// in all, a multiple of the 4 wavefronts of a block, at least 4 steps each.
static int wave_rows_per_step(int D) { return 64 / (D / 16); }
// Query rows per wavefront: with 1 or 2 query heads per KV head, the wavefront's 4 query
// slots take the heads of 4 or 2 consecutive query rows (rows attend the same keys).
static int wave_qp(int G, int n_q) { return (n_q > 1 && (G == 1 || G == 2)) ? kWaveHeads / G : 1; }
static int wave_nqg(int G, int n_q) { const int qp = wave_qp(G, n_q); return (n_q + qp - 1) / qp; }
static int decode_wave_splits(const kvq_shape& s, int Hq, int n_q) {
  const int G = Hq / s.heads, HG = (G + kWaveHeads - 1) / kWaveHeads;
  const long long units = (long long)s.batch * s.layers * wave_nqg(G, n_q) * s.heads * HG;
  long long S = (8192 + units - 1) / units;
  const long long max_s = std::max(1, s.tokens / (4 * wave_rows_per_step(s.head_dim)));
  S = std::min(S, max_s);
  S = (S + 3) / 4 * 4;
  // at most 512 splits: past that the combine's per-row merge costs more than the extra
  // wavefronts gain (a one-head cache still gets 4096 wavefronts)
  return (int)std::max(4LL, std::min(S, 512LL));
}

int decode_wave_split_count(const kvq_shape& s, int Hq, int n_q) { return decode_wave_splits(s, Hq, n_q); }

// Workspace of kvq_decode_attn: split partials of whichever kernel runs.
size_t decode_ws_bytes(const kvq_shape& s, int Hq, int n_q) {
  const int S = std::max(decode_splits(s, Hq, n_q), decode_wave_splits(s, Hq, n_q));
  const size_t gen = (size_t)s.batch * s.layers * n_q * Hq * S * (s.head_dim + 2) * sizeof(float);
  const size_t fast = fast_part_bytes(s, Hq, n_q);
  return gen > fast ? gen : fast;
}

static int kverr_chunks(const kvq_shape& s) {
  const long long units = (long long)s.batch * s.layers * s.heads;
  long long c = (4096 + units - 1) / units;
  if (c > 64) c = 64;
  if (c > s.tokens) c = s.tokens;
  return (int)(c < 1 ? 1 : c);
}

size_t error_ws_bytes(const kvq_shape& s, int Hq, int n_q) {
  const int S = decode_splits(s, Hq, n_q);
  const size_t part = (size_t)s.batch * s.layers * n_q * Hq * S * (2 * s.head_dim + 2 * kErrDoubles) * sizeof(float);
  const size_t units = (size_t)s.batch * s.layers * s.heads;
  const size_t kv = 2 * units * kverr_chunks(s) * 2 * sizeof(double);
  const size_t rowz = (size_t)s.batch * s.layers * n_q * Hq * 2 * sizeof(double);   // JS pass normalisers
  return ((part + 255) / 256) * 256 + kv + rowz;
}

static AArgs make_aargs(const AttnProblem& pr) {
  AArgs a{};
  a.k = dev_codec(*pr.k);
  a.v = dev_codec(*pr.v);
  a.q = pr.q;
  a.kv_len = pr.kv_len;
  a.k16 = pr.k16;
  a.v16 = pr.v16;
  a.sm_scale = pr.sm_scale;
  const kvq_shape& s = pr.k->shape;
  a.B = s.batch; a.L = s.layers; a.H = s.heads; a.T = s.tokens; a.D = s.head_dim;
  a.Hq = pr.Hq; a.G = pr.Hq / s.heads; a.n_q = pr.n_q;
  a.S = decode_splits(s, pr.Hq, pr.n_q);
  a.chunk = split_chunk(s, a.S);
  a.qp = 1;
  a.nqg = a.n_q;
  a.lpt_log2 = lpt_log2_of(a.D);
  a.Dc = (a.k.cb == KVQ_RFFT_POLAR || a.k.cb == KVQ_RFFT_CART) ? 2 * (a.D / 2 + 1) : a.D;
  a.ws = static_cast<float*>(pr.ws);
  a.tab = host_tables();
  host_fft_tables(a.D, &a.tw);
  if (a.k.cb == KVQ_RFFT_POLAR) {
    PhaseTables pt;
    host_phase_tables(1 << a.k.rc.pbits, &pt);
    for (int k = 0; k < 256; ++k) { a.dirs.dir_c[k] = pt.dir_c[k]; a.dirs.dir_s[k] = pt.dir_s[k]; }
  }
  return a;
}

static size_t split_smem(const AArgs& a, bool err) {
  const int RS = 17 * (a.D / 16) + 17;
  size_t f = (size_t)2 * kMaxG * RS + 2 * TB * RS + 2 * kMaxG * TB;
  if (err) f += (size_t)kMaxG * RS + 2 * TB * RS;
  f = (f + 3) / 4 * 4;                                   // 16-byte align the logit/stat arrays
  const size_t acc_bytes = err ? sizeof(double) : sizeof(float);
  return f * sizeof(float) + (2 * kMaxG * TB + 16 * kMaxG) * acc_bytes;
}

// Dynamic LDS of the wavefront kernels: query rows, rFFT tables and levels during the
// loop, then the 4 wavefronts' outputs for the block merge.
static size_t wave_smem_bytes(int D) {
  const size_t loop = (size_t)2 * kWaveHeads * (17 * (D / 16) + 17) + 512 + kWaveHeads * 16 * 20 + 64;
  const size_t merge = (size_t)(kBlock / 64) * kWaveHeads * (D + 2);
  return std::max(loop, merge) * sizeof(float);
}

template <int KCB, int KB, int VCB, int VB>
static hipError_t launch_wave(const AArgs& a, long long R, hipStream_t st) {
  const int HG = (a.G + kWaveHeads - 1) / kWaveHeads;
  const size_t smem = wave_smem_bytes(a.D);
  k_decode_wave<KCB, KB, VCB, VB><<<dim3(a.S / 4, a.H * HG, (unsigned)R), kBlock, smem, st>>>(a);
  return hipGetLastError();
}

// The codec pairs of the five workloads get their own instantiation (codes decoded
// with compile-time widths).  For any other pair nothing is launched and *compiled is
// set false: the caller takes the codec-map kernel if it compiles the pair, else the
// runtime-codec instance.
static hipError_t dispatch_wave(const AArgs& a, long long R, hipStream_t st, bool* compiled) {
  *compiled = true;
  const int kc = a.k.cb, kb = a.k.bits, vc = a.v.cb, vb = a.v.bits;
  auto is = [](int cb, int bits, int c2, int b2) { return cb == c2 && (bits == b2 || b2 < 0); };
  if (is(kc, kb, KVQ_INT_ABSMAX, 4) && is(vc, vb, KVQ_INT_ABSMAX, 2))
    return launch_wave<KVQ_INT_ABSMAX, 4, KVQ_INT_ABSMAX, 2>(a, R, st);
  if (is(kc, kb, KVQ_INT_ABSMAX, 4) && is(vc, vb, KVQ_INT_ABSMAX, 4))
    return launch_wave<KVQ_INT_ABSMAX, 4, KVQ_INT_ABSMAX, 4>(a, R, st);
  if (is(kc, kb, KVQ_INT_ABSMAX, 3) && is(vc, vb, KVQ_INT_ABSMAX, 3))
    return launch_wave<KVQ_INT_ABSMAX, 3, KVQ_INT_ABSMAX, 3>(a, R, st);
  if (is(kc, kb, KVQ_INT_ABSMAX, 3) && is(vc, vb, KVQ_INT_ABSMAX, 2))
    return launch_wave<KVQ_INT_ABSMAX, 3, KVQ_INT_ABSMAX, 2>(a, R, st);
  if (is(kc, kb, KVQ_INT_ABSMAX, 3) && is(vc, vb, KVQ_INT_ABSMAX, 4))
    return launch_wave<KVQ_INT_ABSMAX, 3, KVQ_INT_ABSMAX, 4>(a, R, st);
  if (is(kc, kb, KVQ_INT_ABSMAX, 5) && is(vc, vb, KVQ_INT_ABSMAX, 4))
    return launch_wave<KVQ_INT_ABSMAX, 5, KVQ_INT_ABSMAX, 4>(a, R, st);
  if (is(kc, kb, KVQ_INT_MINMAX, 4) && is(vc, vb, KVQ_INT_MINMAX, 4))
    return launch_wave<KVQ_INT_MINMAX, 4, KVQ_INT_MINMAX, 4>(a, R, st);
  if (is(kc, kb, KVQ_INT_MINMAX, 3) && is(vc, vb, KVQ_INT_MINMAX, 3))
    return launch_wave<KVQ_INT_MINMAX, 3, KVQ_INT_MINMAX, 3>(a, R, st);
  if (is(kc, kb, KVQ_TERNARY, -1) && is(vc, vb, KVQ_TERNARY, -1))
    return launch_wave<KVQ_TERNARY, 2, KVQ_TERNARY, 2>(a, R, st);
  if (is(kc, kb, KVQ_SIGN, -1) && is(vc, vb, KVQ_SIGN, -1))
    return launch_wave<KVQ_SIGN, 1, KVQ_SIGN, 1>(a, R, st);
  if (is(kc, kb, KVQ_NF4, -1) && is(vc, vb, KVQ_INT_ABSMAX, 4))
    return launch_wave<KVQ_NF4, 4, KVQ_INT_ABSMAX, 4>(a, R, st);
  if (is(kc, kb, KVQ_INT8_SYM, -1) && is(vc, vb, KVQ_INT8_SYM, -1))
    return launch_wave<KVQ_INT8_SYM, 8, KVQ_INT8_SYM, 8>(a, R, st);
  if (is(kc, kb, KVQ_FP16, -1) && is(vc, vb, KVQ_FP16, -1))
    return launch_wave<KVQ_FP16, 16, KVQ_FP16, 16>(a, R, st);
  if (is(kc, kb, KVQ_INT_ABSMAX, 6) && is(vc, vb, KVQ_FP16, -1))
    return launch_wave<KVQ_INT_ABSMAX, 6, KVQ_FP16, 16>(a, R, st);
  // rotated 4-bit keys with the 2- and 3-bit value grids [E22L] Result names for the next test
  if (is(kc, kb, KVQ_INT_ABSMAX, 4) && is(vc, vb, KVQ_INT_SYM, 2))
    return launch_wave<KVQ_INT_ABSMAX, 4, KVQ_INT_SYM, 2>(a, R, st);
  if (is(kc, kb, KVQ_INT_ABSMAX, 4) && is(vc, vb, KVQ_INT_SYM, 3))
    return launch_wave<KVQ_INT_ABSMAX, 4, KVQ_INT_SYM, 3>(a, R, st);
  if (is(kc, kb, KVQ_INT_ABSMAX, 4) && is(vc, vb, KVQ_LLOYD, 2))
    return launch_wave<KVQ_INT_ABSMAX, 4, KVQ_LLOYD, 2>(a, R, st);
  if (is(kc, kb, KVQ_INT_ABSMAX, 4) && is(vc, vb, KVQ_LLOYD, 3))
    return launch_wave<KVQ_INT_ABSMAX, 4, KVQ_LLOYD, 3>(a, R, st);
  if (kc == KVQ_RFFT_POLAR && vc == KVQ_FP16) return launch_wave<KVQ_RFFT_POLAR, 0, KVQ_FP16, 16>(a, R, st);
  if (kc == KVQ_RFFT_CART && vc == KVQ_FP16) return launch_wave<KVQ_RFFT_CART, 0, KVQ_FP16, 16>(a, R, st);
  *compiled = false;
  return hipSuccess;
}

static int mix_pair(const kvq_packed& k, const kvq_packed& v);

hipError_t launch_decode_generic(const AttnProblem& pr, hipStream_t st) {
  AArgs a = make_aargs(pr);
  // rFFT keys on the wavefront kernel: fp16 values, and a lane's 8 bins in one scale group
  const bool rk = a.k.cb == KVQ_RFFT_POLAR || a.k.cb == KVQ_RFFT_CART;
  const bool rk_wave = rk && a.v.cb == KVQ_FP16 && a.k.rc.g >= 8 && (a.k.rc.g & 7) == 0;
  if (!rk || rk_wave) {
    const kvq_shape& s = pr.k->shape;
    a.S = decode_wave_splits(s, pr.Hq, pr.n_q);
    const int rpw = wave_rows_per_step(a.D);
    a.chunk = ((s.tokens + a.S - 1) / a.S + rpw - 1) / rpw * rpw;
    a.qp = wave_qp(a.G, a.n_q);
    a.nqg = wave_nqg(a.G, a.n_q);
    const long long R = (long long)a.B * a.L * a.nqg;
    // one block (4 splits) per row, no value rotation, channel scale or key mean: the
    // block merge writes the output (the combine would only divide by l)
    const bool direct = a.S == 4 && pr.v->codec.rot_width <= 1 && !pr.v->chan_scale && !pr.k->mean;
    if (direct) {
      a.dout = pr.out;
      a.dlse = pr.lse;
    }
    bool compiled = false;
    hipError_t e = dispatch_wave(a, R, st, &compiled);
    if (e != hipSuccess) return e;
    if (!compiled) {
      if (!rk && mix_pair(*pr.k, *pr.v) >= 0) {      // a pair the codec-map kernel compiles: one tile
        const kvq_segment sg{pr.k, pr.v, 0, 0, 0};
        const kvq_shape& s = pr.k->shape;
        return launch_decode_mixed(&sg, 1, s.layers, s.heads, s.tokens, pr.Hq, pr.n_q, pr.q, pr.kv_len,
                                   pr.sm_scale, pr.out, pr.lse, pr.ws, false, st);
      }
      e = launch_wave<-1, 0, -1, 0>(a, R, st);
      if (e != hipSuccess) return e;
    }
    if (direct) return hipSuccess;
    return launch_combine_partials(pr, a.S / 4, nullptr, st);   // one partial per block of 4 splits
  }
  const long long R = (long long)a.B * a.L * a.n_q;
  const size_t smem = split_smem(a, false);
  hipError_t e0 = hipFuncSetAttribute((const void*)k_attn_split<false>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e0 != hipSuccess) return e0;
  k_attn_split<false><<<dim3(a.S, a.H, (unsigned)R), kBlock, smem, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine_partials(pr, a.S, nullptr, st);
}

static CArgs make_cargs(const AttnProblem& pr, int S, float* ws) {
  CArgs c{};
  const kvq_shape& s = pr.k->shape;
  c.ws = ws;
  c.S = S;
  c.D = s.head_dim;
  c.Hq = pr.Hq;
  c.G = pr.Hq / s.heads;
  c.H = s.heads;
  c.L = s.layers;
  c.n_q = pr.n_q;
  c.vW = pr.v->codec.rot_width > 1 ? pr.v->codec.rot_width : 0;
  c.vkappa = kappa_of(c.vW);
  c.vchan = pr.v->chan_scale;
  return c;
}

hipError_t launch_combine_partials(const AttnProblem& pr, int S, int* ctr, hipStream_t st) {
  const kvq_shape& s = pr.k->shape;
  const long long R = (long long)s.batch * s.layers * pr.n_q;
  CArgs c = make_cargs(pr, S, static_cast<float*>(pr.ws));
  c.ctr = ctr;
  k_attn_combine<false><<<(unsigned)(R * pr.Hq), kBlock, 0, st>>>(c, pr.out, pr.lse, nullptr, nullptr, ErrOut{});
  return hipGetLastError();
}

hipError_t launch_attn_error(const AttnProblem& pr, hipStream_t st) {
  AArgs a = make_aargs(pr);
  const kvq_shape& s = pr.k->shape;
  const long long R = (long long)a.B * a.L * a.n_q;
  const size_t smem = split_smem(a, true);
  hipError_t e0 = hipFuncSetAttribute((const void*)k_attn_split<true>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e0 != hipSuccess) return e0;
  k_attn_split<true><<<dim3(a.S, a.H, (unsigned)R), kBlock, smem, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // workspace: split partials | per-unit K/V error partials | per-row normalisers (JS pass)
  const long long units = (long long)s.batch * s.layers * s.heads;
  const int chunks = kverr_chunks(s);
  const int P = 2 * a.D + 2 * kErrDoubles;
  const size_t part_bytes = (size_t)R * a.Hq * a.S * P * sizeof(float);
  double* pk = reinterpret_cast<double*>(static_cast<char*>(pr.ws) + ((part_bytes + 255) / 256) * 256);
  double* pv = pk + units * chunks * 2;
  double* rowz = pv + units * chunks * 2;
  ErrOut eo{pr.renyi2, pr.logit_relerr, pr.top1, pr.js ? rowz : nullptr};
  k_attn_combine<true><<<(unsigned)(R * a.Hq), kBlock, 0, st>>>(make_cargs(pr, a.S, a.ws), nullptr, nullptr,
                                                                pr.kl, pr.relerr, eo);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (pr.js) {   // second pass: JS needs both distributions' final normalisers
    AArgs aj = a;
    aj.js_rowz = rowz;
    k_attn_split<true><<<dim3(a.S, a.H, (unsigned)R), kBlock, smem, st>>>(aj);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long rows = R * a.Hq;
    k_js_final<<<(unsigned)((rows + 255) / 256), 256, 0, st>>>(a.ws, a.S, P, a.D, rows, pr.js);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!pr.kv_err) return hipSuccess;
  // per-unit K/V squared error
  if (units == 0 || s.tokens == 0) {
    return hipMemsetAsync(pr.kv_err, 0, sizeof(double) * 4 * units, st);
  }
  const kvq_packed* tens[2] = {pr.k, pr.v};
  const uint16_t* xs[2] = {pr.k16, pr.v16};
  double* parts[2] = {pk, pv};
  for (int w = 0; w < 2; ++w) {
    const kvq_packed& p = *tens[w];
    if (p.codec.codebook == KVQ_RFFT_POLAR || p.codec.codebook == KVQ_RFFT_CART) {
      e = launch_rfft_kverr(xs[w], p, parts[w], chunks, st);
    } else {
      EArgs ea{};
      ea.c = dev_codec(p);
      ea.x = xs[w];
      ea.T = s.tokens; ea.H = s.heads; ea.L = s.layers; ea.D = s.head_dim;
      ea.lpt_log2 = lpt_log2_of(s.head_dim);
      ea.chunks = chunks;
      ea.part = parts[w];
      ea.tab = host_tables();
      k_kverr<<<dim3(chunks, (unsigned)units), kBlock, 0, st>>>(ea);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
  }
  k_kverr_final<<<(unsigned)((units + 255) / 256), 256, 0, st>>>(pk, pv, chunks, units, pr.kv_err);
  return hipGetLastError();
}

}  // namespace kvq

namespace kvq {

static int code_bits(int cb, int bits) {
  switch (cb) {
    case KVQ_FP16: return 16;
    case KVQ_TERNARY: return 2;
    case KVQ_SIGN: return 1;
    case KVQ_NF4: return 4;
    case KVQ_INT8_SYM: return 8;
    default: return bits;
  }
}

static int mix_pair(const kvq_packed& k, const kvq_packed& v) {
  const int kcb = k.codec.codebook, kb = code_bits(kcb, k.codec.bits);
  const int vcb = v.codec.codebook, vb = code_bits(vcb, v.codec.bits);
#define KVQ_MIX_ID(id, KCB, KB, VCB, VB) \
  if (kcb == KCB && kb == KB && vcb == VCB && vb == VB) return id;
  KVQ_MIX_PAIRS(KVQ_MIX_ID)
#undef KVQ_MIX_ID
  return -1;
}

bool mixed_decode_supported(const kvq_segment* segs, int n, int layers, int heads, int tokens, int Hq, int n_q) {
  if (n < 1 || n > kMaxSegments || heads < 1 || Hq % heads != 0) return false;
  // the launch grids over the whole map: (splits, heads x head groups, rows x row groups)
  const int G = Hq / heads;
  const long long gy = (long long)heads * ((G + kWaveHeads - 1) / kWaveHeads);
  const long long gz = (long long)segs[0].k->shape.batch * layers * wave_nqg(G, n_q);
  if (gy > 65535 || gz > 65535 || (long long)segs[0].k->shape.batch * layers * n_q * Hq > 0x7fffffffLL) return false;
  for (int i = 0; i < n; ++i) {
    if (segs[i].token0 != 0 || segs[i].k->shape.tokens != tokens) return false;
    if (mix_pair(*segs[i].k, *segs[i].v) < 0) return false;
  }
  return true;
}

static kvq_shape mixed_shape(const kvq_segment* segs, int layers, int heads, int tokens) {
  kvq_shape s = segs[0].k->shape;
  s.layers = layers;
  s.heads = heads;
  s.tokens = tokens;
  return s;
}

size_t mixed_ws_bytes(const kvq_segment* segs, int layers, int heads, int tokens, int Hq, int n_q) {
  const kvq_shape s = mixed_shape(segs, layers, heads, tokens);
  const int S = decode_wave_splits(s, Hq, n_q);
  return (size_t)s.batch * s.layers * n_q * Hq * S * (s.head_dim + 2) * sizeof(float);
}

static MixCodec mix_codec_of(const kvq_packed& p) {
  const DevCodec d = dev_codec(p);
  MixCodec m{};
  m.codes = d.codes;
  m.scales = d.scales;
  m.mins = d.mins;
  m.chan = d.chan;
  m.row_bytes = (int)d.row_bytes;
  m.ng = d.ng;
  m.g = d.g;
  m.W = d.W;
  m.kappa = d.kappa;
  m.cb = d.cb;
  m.bits = d.bits;
  return m;
}

hipError_t launch_decode_mixed(const kvq_segment* segs, int n, int layers, int heads, int tokens, int Hq, int n_q,
                               const uint16_t* q, const int32_t* kv_len, float sm, float* out, float* lse,
                               void* part, bool mean_shift, hipStream_t st) {
  const kvq_shape s = mixed_shape(segs, layers, heads, tokens);
  MArgs a{};
  a.q = q;
  a.kv_len = kv_len;
  a.ws = static_cast<float*>(part);
  a.sm_scale = sm;
  a.B = s.batch; a.L = layers; a.H = heads; a.T = tokens; a.D = s.head_dim;
  a.Hq = Hq; a.G = Hq / heads; a.n_q = n_q;
  a.S = decode_wave_splits(s, Hq, n_q);
  const int rpw = wave_rows_per_step(a.D);
  a.chunk = ((tokens + a.S - 1) / a.S + rpw - 1) / rpw * rpw;
  a.lpt_log2 = lpt_log2_of(a.D);
  a.qp = wave_qp(a.G, n_q);
  a.nqg = wave_nqg(a.G, n_q);
  a.ntiles = n;
  a.tab = host_tables();
  CArgs c{};
  c.ws = a.ws;
  c.S = a.S / 4;                                     // one partial per block of 4 splits
  c.D = a.D; c.Hq = Hq; c.G = a.G; c.H = heads; c.L = layers; c.n_q = n_q;
  c.ntiles = n;
  c.q = q;
  c.sm = sm;
  for (int i = 0; i < n; ++i) {
    const kvq_segment& g = segs[i];
    MixTile& t = a.tile[i];
    t.k = mix_codec_of(*g.k);
    t.v = mix_codec_of(*g.v);
    t.l0 = g.layer0; t.ls = g.k->shape.layers; t.h0 = g.head0; t.hs = g.k->shape.heads;
    t.pair = mix_pair(*g.k, *g.v);
    MixV& m = c.tile[i];
    m.l0 = t.l0; m.ls = t.ls; m.h0 = t.h0; m.hs = t.hs;
    m.vW = g.v->codec.rot_width > 1 ? g.v->codec.rot_width : 0;
    m.vkappa = kappa_of(m.vW);
    m.vchan = g.v->chan_scale;
    m.kmean = mean_shift ? g.k->mean : nullptr;
  }
  const long long R = (long long)a.B * a.L * a.n_q;  // query rows per head
  const int HG = (a.G + kWaveHeads - 1) / kWaveHeads;
  const size_t smem = wave_smem_bytes(a.D);
  k_decode_wave_mix<<<dim3(a.S / 4, a.H * HG, (unsigned)((long long)a.B * a.L * a.nqg)), kBlock, smem, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_attn_combine<false><<<(unsigned)(R * Hq), kBlock, 0, st>>>(c, out, lse, nullptr, nullptr, ErrOut{});
  return hipGetLastError();
}

hipError_t launch_lse_mean(const AttnProblem& pr, hipStream_t st) {
  const kvq_shape& sh = pr.k->shape;
  const long long rows = (long long)sh.batch * sh.layers * pr.n_q * pr.Hq;
  if (rows == 0) return hipSuccess;
  const long long blocks = (rows + kBlock / 64 - 1) / (kBlock / 64);
  k_lse_mean<<<(unsigned)blocks, kBlock, 0, st>>>(pr.q, pr.k->mean, pr.lse, rows, sh.layers, pr.n_q, pr.Hq, sh.heads,
                                                  sh.head_dim, pr.sm_scale);
  return hipGetLastError();
}

}  // namespace kvq

namespace kvq {

// ------------------------------------------------------------------ segments of a logical cache
// A segment holds layers [l0, l0 + Ls) and tokens [t0, t0 + Ts) of a logical cache; it is
// decoded on its own and its (out, lse) merged into the logical result.

// Query rows of the segment's layers and query heads [j0, j0 + hq), copied out of
// q [B][L][n_q][Hq][D] into [B][Ls][n_q][hq][D] (16-byte units; D8 = D / 8).
__global__ void k_seg_gather_q(const uint4* __restrict__ src, uint4* __restrict__ dst, int L, int Ls, int l0,
                               int n_q, int Hq, int j0, int hq, int D8, long long total) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const long long per = (long long)hq * D8;
  const long long row = i / per, e = i - row * per;         // row = (b * Ls + l) * n_q + qi
  const long long qi = row % n_q, bl = row / n_q;
  const long long b = bl / Ls, l = bl - b * Ls;
  dst[i] = src[(((b * L + l0 + l) * n_q + qi) * Hq + j0) * D8 + e];
}

// Keys attended inside the segment: clamp(kv_len - t0, 0, Ts) for its layers.
__global__ void k_seg_kvlen(const int32_t* __restrict__ kvl, int32_t* __restrict__ out, int L, int Ls, int l0,
                            int n_q, int t0, int Ts, long long total) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const long long bl = i / n_q, j = i - bl * n_q;
  const long long b = bl / Ls, l = bl - b * Ls;
  const int v = kvl[(b * L + l0 + l) * n_q + j] - t0;
  out[i] = v < 0 ? 0 : (v > Ts ? Ts : v);
}

// Logical result before any segment: out = 0, lse = -inf.
__global__ void k_seg_init(float* __restrict__ out, float* __restrict__ lse, long long rows, int D) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < rows * D) out[i] = 0.0f;
  if (i < rows) lse[i] = -INFINITY;
}

// (out, lse) of every logical row <- the log-sum-exp merge with each listed segment
// covering the row's layer, in list order: weights e^(lse - m), m the larger lse.  One
// wavefront per logical row.
struct SegMergeArgs {
  int n;
  int l0[kMaxSegments], ls[kMaxSegments], j0[kMaxSegments], hq[kMaxSegments];
  const float* os[kMaxSegments];
  const float* lsp[kMaxSegments];
};

__global__ __launch_bounds__(kBlock) void k_seg_merge(SegMergeArgs sa, float* __restrict__ out, float* __restrict__ lse,
                                                      int L, int n_q, int Hq, int D, long long rows) {
  const long long g = (long long)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= rows) return;                                   // uniform per wavefront
  const int j = (int)(g % Hq);                             // g = ((b * L + l) * n_q + qi) * Hq + j
  const long long t = g / Hq;
  const long long qi = t % n_q, bl = t / n_q;
  const long long b = bl / L;
  const int l = (int)(bl - b * L);
  float la = lse[g];
  for (int i = 0; i < sa.n; ++i) {
    if (l < sa.l0[i] || l >= sa.l0[i] + sa.ls[i] || j < sa.j0[i] || j >= sa.j0[i] + sa.hq[i]) continue;
    const long long r = ((b * sa.ls[i] + (l - sa.l0[i])) * n_q + qi) * sa.hq[i] + (j - sa.j0[i]);   // its row
    const float lb = sa.lsp[i][r];
    const float m = __builtin_fmaxf(la, lb);
    if (m == -INFINITY) continue;                          // no keys on either side
    const float wa = la == -INFINITY ? 0.0f : expf(la - m);
    const float wb = lb == -INFINITY ? 0.0f : expf(lb - m);
    const float inv = 1.0f / (wa + wb);
    const float* os = sa.os[i] + r * D;
    for (int d = lane; d < D; d += 64) out[g * D + d] = (wa * out[g * D + d] + wb * os[d]) * inv;
    la = m + logf(wa + wb);
  }
  if (lane == 0) lse[g] = la;
}

hipError_t launch_seg_init(float* out, float* lse, long long rows, int D, hipStream_t st) {
  const long long n = rows * D;
  if (n == 0) return hipSuccess;
  k_seg_init<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, st>>>(out, lse, rows, D);
  return hipGetLastError();
}

hipError_t launch_seg_prepare(const uint16_t* q, const int32_t* kvl, uint16_t* qs, int32_t* kvls, int B, int L,
                              int Ls, int l0, int n_q, int Hq, int j0, int hq, int D, int t0, int Ts, hipStream_t st) {
  if (qs) {
    const long long tq = (long long)B * Ls * n_q * hq * (D / 8);
    k_seg_gather_q<<<(unsigned)((tq + kBlock - 1) / kBlock), kBlock, 0, st>>>(
        reinterpret_cast<const uint4*>(q), reinterpret_cast<uint4*>(qs), L, Ls, l0, n_q, Hq, j0, hq, D / 8, tq);
  }
  if (kvls) {
    const long long tk = (long long)B * Ls * n_q;
    k_seg_kvlen<<<(unsigned)((tk + kBlock - 1) / kBlock), kBlock, 0, st>>>(kvl, kvls, L, Ls, l0, n_q, t0, Ts, tk);
  }
  return hipGetLastError();
}

hipError_t launch_seg_merge(int n, const int* l0, const int* ls, const int* j0, const int* hq, float* const* os,
                            float* const* lsp, float* out, float* lse, int B, int L, int n_q, int Hq, int D,
                            hipStream_t st) {
  if (n == 0) return hipSuccess;
  SegMergeArgs sa{};
  sa.n = n;
  for (int i = 0; i < n; ++i) {
    sa.l0[i] = l0[i];
    sa.ls[i] = ls[i];
    sa.j0[i] = j0[i];
    sa.hq[i] = hq[i];
    sa.os[i] = os[i];
    sa.lsp[i] = lsp[i];
  }
  const long long rows = (long long)B * L * n_q * Hq;
  if (rows == 0) return hipSuccess;
  k_seg_merge<<<(unsigned)((rows + kBlock / 64 - 1) / (kBlock / 64)), kBlock, 0, st>>>(sa, out, lse, L, n_q, Hq, D,
                                                                                       rows);
  return hipGetLastError();
}

}  // namespace kvq

// MFMA decode attention over a packed cache with 4-bit signed-absmax keys
// (group 128 or 256, any Walsh-Hadamard rotation) and 2-bit signed-absmax
// values (group >= 16), head_dim 256, up to 4 query heads per KV head: the
// 64K-token decode workload of [E22L] ("Can 4-bit keys and 2-bit values hit a
// 1M-token memory budget?", What I tested: arm A, rotated 4-bit keys and 2-bit
// values at group 128).
//
// Why MFMA: at 0.39 bytes per cached value, HBM speed leaves about two VALU
// lane-ops per value, while unpacking plus four grouped-head multiply-adds per
// key and per value costs four to five.  Both contractions go to the matrix
// cores; the VALU only unpacks codes (one AND per pair of codes) and runs the
// softmax.
//
// Per wavefront, 32 tokens per step:
//  * Q.K^T: v_mfma_f32_16x16x32_f16, A = 16 tokens x 32 dims of key codes as
//    fp16 subnormals (code c -> c*2^-24, exact), B = the rotated query in fp16
//    with the 4 heads replicated over the 16 columns, so lane (kg, n) ends with
//    the logits of head n%4 for tokens 8kg..8kg+7.  Logit = sum over the two
//    scale groups of s_g * (2^24 C_g - 8 sum_g q), times the softmax scale.
//  * online softmax per head with a running maximum; the accumulators are
//    rescaled only when the maximum grows.
//  * P.V: v_mfma_f32_4x4x4_16b_f16, 16 blocks of (4 heads x 4 tokens) x
//    (4 tokens x 4 dims): lane l owns value word l%16 (16 dims, one scale
//    group) for tokens 8(l/16)..+7; B = 2-bit codes of 4 tokens at one dim as
//    fp16 subnormals c*4^i*2^-24 (pairs built with v_perm + AND), A = p*s/4^i.
//    Output: 2^24 * acc - 2 * sum p*s per group.
// Each wavefront writes (o, m, l) partials; the general combine kernel merges
// them and rotates rotated values back.
#include <cmath>

#include "kvq_internal.hpp"

namespace kvq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kFastD = 256;
constexpr int kStep = 32;          // tokens per wavefront step

struct FArgs {
  const uint8_t* kc;               // key codes, 128 B per row
  const uint16_t* ks;              // key scales, nks per row
  const uint8_t* vc;               // value codes, 64 B per row
  const uint16_t* vs;              // value scales, nvs per row
  const uint16_t* q;
  const int32_t* kv_len;
  const float* kchan;
  float* ws;
  int B, L, H, T, Hq, G, n_q;
  int nks, nvs, gv;                // scales per row, value group
  int kW;                          // key rotation width (0 = none)
  float kkappa;
  float sm_scale;
  int blocks_per_unit;             // partials per (query row, head)
  int wave_tokens;                 // tokens per wavefront (multiple of kStep)
};

__device__ __forceinline__ uint32_t h2bits(_Float16 h) { return (uint32_t)__builtin_bit_cast(uint16_t, h); }

struct StepData {
  u32x4_t kw[2][2];    // key codes: QK tile u, row half (words 4kg.. and 16+4kg..)
  u32x4_t ks[2];       // key scales of tokens 8kg..8kg+7
  uint32_t vw[8];      // value word of tokens 8kg + j
  u32x4_t vs[4];       // value scales of tokens 8kg..8kg+7
};

template <int NKS, int NVS>
__device__ __forceinline__ void load_step(const FArgs& a, size_t row0, int t0, int kg, int n16, StepData& d) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int tok = t0 + 8 * (n16 >> 2) + 4 * u + (n16 & 3);
    const uint8_t* kr = a.kc + (row0 + tok) * 128;
    d.kw[u][0] = *reinterpret_cast<const u32x4_t*>(kr + 16 * kg);
    d.kw[u][1] = *reinterpret_cast<const u32x4_t*>(kr + 64 + 16 * kg);
  }
  const size_t r8 = row0 + t0 + 8 * kg;
  d.ks[0] = *reinterpret_cast<const u32x4_t*>(a.ks + r8 * NKS);
  if (NKS == 2) d.ks[1] = *reinterpret_cast<const u32x4_t*>(a.ks + r8 * NKS + 8);
#pragma unroll
  for (int j = 0; j < 8; ++j) d.vw[j] = *reinterpret_cast<const uint32_t*>(a.vc + (r8 + j) * 64 + 4 * n16);
#pragma unroll
  for (int k = 0; k < NVS; ++k) d.vs[k] = *reinterpret_cast<const u32x4_t*>(a.vs + r8 * NVS + 8 * k);
}

// Half number `idx` (compile-time after unrolling) of a run of u32x4 words.
__device__ __forceinline__ uint16_t half_at(const u32x4_t* v, int idx) {
  const uint32_t w = v[idx >> 3][(idx >> 1) & 3];
  return (uint16_t)((idx & 1) ? (w >> 16) : (w & 0xffffu));
}

// Scale of token k (compile-time) in group grp (lane-varying) with NVS scales per row.
template <int NVS>
__device__ __forceinline__ uint16_t vscale_at(const u32x4_t* v, int k, int grp) {
  if constexpr (NVS == 1) {
    return half_at(v, k);
  } else if constexpr (NVS == 2) {
    const uint32_t w = v[k >> 2][k & 3];
    return (uint16_t)(grp ? (w >> 16) : (w & 0xffffu));
  } else {
    const uint32_t wa = v[k >> 1][(2 * k) & 3], wb = v[k >> 1][(2 * k + 1) & 3];
    const uint32_t w = (grp & 2) ? wb : wa;
    return (uint16_t)((grp & 1) ? (w >> 16) : (w & 0xffffu));
  }
}

template <int NKS, int NVS>
__global__ __launch_bounds__(kBlock, 2) void k_decode_mfma(FArgs a) {
  __shared__ float qs[4][kFastD + 16];
  __shared__ float qsum_s[4][2];
  __shared__ float so[4][4][kFastD];       // per-wave outputs [wave][head][dim]
  __shared__ float sm[4][4], sl[4][4];      // per-wave max (log2 units) and sum
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 4, n16 = lane & 15;
  const long long unit = blockIdx.y;                 // (b*L + l)*H + h
  const int h = (int)(unit % a.H);
  const long long bl = unit / a.H;                   // b*L + l
  const int l = (int)(bl % a.L);
  const int i = blockIdx.z;                          // query index
  const long long rq = bl * a.n_q + i;
  const int G = a.G;
  int n = a.T;
  if (a.kv_len) n = min(max(a.kv_len[rq], 0), a.T);

  // ---- query prologue: q in the key coordinates (divide channel scale, rotate), fp32 in LDS
  const uint16_t* qsrc = a.q + (size_t)rq * a.Hq * kFastD + (size_t)h * G * kFastD;
  for (int p = tid; p < 4 * kFastD; p += kBlock) {
    const int g = p >> 8, d = p & 255;
    float x = 0.0f;
    if (g < G) {
      x = h2f(qsrc[(size_t)g * kFastD + d]);
      if (a.kchan) x = x / a.kchan[((size_t)l * a.H + h) * kFastD + d];
    }
    qs[g][d] = x;
  }
  __syncthreads();
  if (a.kW > 1) {
    for (int s = 1; s < a.kW; s <<= 1) {
      for (int p = tid; p < 4 * (kFastD / 2); p += kBlock) {
        const int g = p >> 7, pp = p & 127;
        const int ii = (pp / s) * 2 * s + (pp % s);
        const float x = qs[g][ii], y = qs[g][ii + s];
        qs[g][ii] = x + y;
        qs[g][ii + s] = x - y;
      }
      __syncthreads();
    }
    for (int p = tid; p < 4 * kFastD; p += kBlock) qs[p >> 8][p & 255] *= a.kkappa;
    __syncthreads();
  }
  {  // per-group sums of the fp16 query (wave w: head w): sum_g q for the (c - 8) offset folding
    float s0 = (float)(_Float16)qs[wave][2 * lane] + (float)(_Float16)qs[wave][2 * lane + 1];
    float s1 = (float)(_Float16)qs[wave][128 + 2 * lane] + (float)(_Float16)qs[wave][128 + 2 * lane + 1];
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      s0 += __shfl_xor(s0, m);
      s1 += __shfl_xor(s1, m);
    }
    if (lane == 0) { qsum_s[wave][0] = s0; qsum_s[wave][1] = s1; }
  }
  // B operands: chunk c < 4 -> key word 4kg + c (dims 8w..8w+7, group 0), c >= 4 -> word 16 + 4kg + (c-4).
  // Register order of the 8 k-slots: dims (0,4), (1,5)/16, (2,6), (3,7)/16 of the word.
  half8_t qb[8];
  const int hq = n16 & 3;                            // query head of this column
  const bool hvalid = hq < G;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = (c < 4) ? (4 * kg + c) : (16 + 4 * kg + (c - 4));
    const int d0 = 8 * w;
    half8_t v;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const _Float16 lo = hvalid ? (_Float16)qs[hq][d0 + r] : (_Float16)0.0f;
      const _Float16 hi = hvalid ? (_Float16)qs[hq][d0 + r + 4] : (_Float16)0.0f;
      if (r & 1) {
        v[2 * r] = lo * (_Float16)0.0625f;
        v[2 * r + 1] = hi * (_Float16)0.0625f;
      } else {
        v[2 * r] = lo;
        v[2 * r + 1] = hi;
      }
    }
    qb[c] = v;
  }
  __syncthreads();
  constexpr float kLog2e = 1.4426950408889634f;
  const float lsc = a.sm_scale * kLog2e;             // logits kept in log2 units
  const float cK = lsc * 16777216.0f;                // 2^24
  const float off0 = hvalid ? lsc * 8.0f * qsum_s[hq][0] : 0.0f;
  const float off1 = hvalid ? lsc * 8.0f * qsum_s[hq][1] : 0.0f;
  constexpr bool kone = (NKS == 1);                  // key group 256: one scale per row

  // ---- token range of this wavefront
  const int t_begin = (blockIdx.x * 4 + wave) * a.wave_tokens;
  const int t_end = min(t_begin + a.wave_tokens, n);
  const size_t row0 = (size_t)unit * a.T;
  const int vgrp = (16 * n16) / a.gv;                // scale group of this lane's value word

  float4_t acc[16];
#pragma unroll
  for (int f = 0; f < 16; ++f) acc[f] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_ref = -INFINITY;       // running max (log2 units) of head hq
  float l_part = 0.0f;           // sum of p over this lane's tokens (head hq)
  float w_part = 0.0f;           // sum of fp16(p * s_v) over this lane's tokens (head hq, group vgrp)

  StepData nxt;
  if (t_begin < t_end) load_step<NKS, NVS>(a, row0, t_begin, kg, n16, nxt);
  for (int t0 = t_begin; t0 < t_end; t0 += kStep) {
    const StepData cur = nxt;
    if (t0 + kStep < t_end) load_step<NKS, NVS>(a, row0, t0 + kStep, kg, n16, nxt);   // prefetch the next step

    // ---- Q.K^T
    float4_t cq[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      cq[u][0] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      cq[u][1] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t w = cur.kw[u][c >> 2][c & 3];
        const uint32_t w2 = w >> 8;
        const u32x4_t pr = u32x4_t{w & 0x000F000Fu, w & 0x00F000F0u, w2 & 0x000F000Fu, w2 & 0x00F000F0u};
        const half8_t av = __builtin_bit_cast(half8_t, pr);
        cq[u][c >> 2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qb[c], cq[u][c >> 2], 0, 0, 0);
      }
    }
    // logits (log2 units) of tokens 8kg + 4u + r, head hq
    float lg[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * u + r;                      // token 8kg + j
        float s0, s1;
        if constexpr (kone) {
          s0 = s1 = h2f(half_at(cur.ks, j));
        } else {
          s0 = h2f(half_at(cur.ks, 2 * j));
          s1 = h2f(half_at(cur.ks, 2 * j + 1));
        }
        const float x = s0 * (cq[u][0][r] * cK - off0) + s1 * (cq[u][1][r] * cK - off1);
        lg[j] = (t0 + 8 * kg + j < t_end) ? x : -INFINITY;
      }
    }
    // ---- online softmax (per head; lanes with equal n16%4 hold identical values)
    float mt = lg[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mt = fmaxf(mt, lg[k]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool grow = mt > m_ref;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float al = (m_ref == -INFINITY) ? 0.0f : exp2f(m_ref - fmaxf(mt, m_ref));
      const float alpha = grow ? al : 1.0f;
      m_ref = fmaxf(mt, m_ref);
      l_part *= alpha;
      w_part *= alpha;
      // accumulator component c belongs to head c: take head c's factor from lane c
      const float a0 = __shfl(alpha, 0), a1 = __shfl(alpha, 1), a2 = __shfl(alpha, 2), a3 = __shfl(alpha, 3);
#pragma unroll
      for (int f = 0; f < 16; ++f) {
        acc[f][0] *= a0;
        acc[f][1] *= a1;
        acc[f][2] *= a2;
        acc[f][3] *= a3;
      }
    }
    // ---- P.V weights w = p * s_v(token, group of this lane's value word); A = w / 4^i for field shift i
    float wv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float p = (lg[k] == -INFINITY) ? 0.0f : exp2f(lg[k] - m_ref);
      l_part += p;
      wv[k] = p * h2f(vscale_at<NVS>(cur.vs, k, vgrp));
    }
    half4_t aw[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      half4_t base;
#pragma unroll
      for (int j = 0; j < 4; ++j) base[j] = hvalid ? (_Float16)wv[4 * s + j] : (_Float16)0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) w_part += (float)base[j];      // offset uses the MFMA's fp16 weights
      aw[s][0] = base;
      aw[s][1] = base * (_Float16)0.25f;
      aw[s][2] = base * (_Float16)0.0625f;
      aw[s][3] = base * (_Float16)0.015625f;
    }
    // ---- P.V: field f of byte k = f/4, shift i = f%4; B pairs (tokens 4s+0, 4s+1), (4s+2, 4s+3)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t sel = (uint32_t)k | (0x0Cu << 8) | ((uint32_t)(4 + k) << 16) | (0x0Cu << 24);
        const uint32_t r01 = __builtin_amdgcn_perm(cur.vw[4 * s + 1], cur.vw[4 * s + 0], sel);
        const uint32_t r23 = __builtin_amdgcn_perm(cur.vw[4 * s + 3], cur.vw[4 * s + 2], sel);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const uint32_t mask = 0x00030003u << (2 * ii);
          const u32x2_t bp = u32x2_t{r01 & mask, r23 & mask};
          const half4_t bv = __builtin_bit_cast(half4_t, bp);
          acc[4 * k + ii] = __builtin_amdgcn_mfma_f32_4x4x4f16(aw[s][ii], bv, acc[4 * k + ii], 0, 0, 0);
        }
      }
    }
  }

  // ---- reduce the token subsets of the four lane groups (same word, kg = 0..3)
#pragma unroll
  for (int f = 0; f < 16; ++f) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float x = acc[f][c];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[f][c] = x;
    }
  }
  l_part += __shfl_xor(l_part, 16);
  l_part += __shfl_xor(l_part, 32);
  w_part += __shfl_xor(w_part, 16);
  w_part += __shfl_xor(w_part, 32);
  // sum fp16(p*s_v) of head c in this lane's value group: the lane of the same 4-lane block with lane%4 == c
  const int base_l = lane & ~3;
  const float ws0 = __shfl(w_part, base_l | 0), ws1 = __shfl(w_part, base_l | 1);
  const float ws2 = __shfl(w_part, base_l | 2), ws3 = __shfl(w_part, base_l | 3);
  if (lane < 16) {
    const float wsum[4] = {ws0, ws1, ws2, ws3};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int f = 0; f < 16; ++f) so[wave][c][16 * n16 + f] = acc[f][c] * 16777216.0f - 2.0f * wsum[c];
    }
  }
  if (lane < 4) {
    sm[wave][lane] = m_ref;
    sl[wave][lane] = l_part;
  }
  __syncthreads();
  // ---- merge the four wavefronts of the block; one partial per (query row, head, block)
  constexpr float kLn2 = 0.6931471805599453f;
  const int P = kFastD + 2;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (c >= G) break;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][c]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = (sm[w][c] == -INFINITY) ? 0.0f : exp2f(sm[w][c] - M);
      L += wt * sl[w][c];
      O += wt * so[w][c][tid];
    }
    float* dst = a.ws + ((rq * a.Hq + (size_t)h * G + c) * a.blocks_per_unit + blockIdx.x) * P;
    dst[tid] = O;
    if (tid == 0) {
      dst[kFastD] = (M == -INFINITY) ? -INFINITY : M * kLn2;
      dst[kFastD + 1] = L;
    }
  }
}

// ------------------------------------------------------------------ host side

bool fast_decode_supported(const kvq_packed& k, const kvq_packed& v, int Hq) {
  const kvq_shape& s = k.shape;
  if (s.head_dim != kFastD) return false;
  if (s.tokens % kStep != 0 || s.tokens == 0) return false;
  if (Hq / s.heads > 4) return false;
  if (k.codec.codebook != KVQ_INT_ABSMAX || k.codec.bits != 4) return false;
  if (k.codec.group != 128 && k.codec.group != 256) return false;
  if (v.codec.codebook != KVQ_INT_ABSMAX || v.codec.bits != 2) return false;
  if (v.codec.group < 64) return false;   // a P.V block's 4 value words share one scale group
  if (v.chan_scale) return false;
  return true;
}

static void fast_split(const kvq_shape& s, int n_q, int* blocks_per_unit, int* wave_tokens) {
  const long long pairs = (long long)s.batch * s.layers * n_q * s.heads;
  // about two blocks of four wavefronts per CU (the kernel runs two wavefronts per SIMD)
  long long bpu = (512 + pairs - 1) / pairs;
  const long long max_bpu = std::max(1, s.tokens / (4 * kStep));
  if (bpu > max_bpu) bpu = max_bpu;
  if (bpu < 1) bpu = 1;
  const long long per_wave = (s.tokens + 4 * bpu - 1) / (4 * bpu);
  const int wt = (int)((per_wave + kStep - 1) / kStep * kStep);
  *wave_tokens = wt;
  *blocks_per_unit = (int)((s.tokens + 4LL * wt - 1) / (4LL * wt));
}

size_t fast_ws_bytes(const kvq_shape& s, int Hq, int n_q) {
  if (s.head_dim != kFastD || s.tokens % kStep != 0 || s.tokens == 0) return 0;
  int bpu, wt;
  fast_split(s, n_q, &bpu, &wt);
  return (size_t)s.batch * s.layers * n_q * Hq * bpu * (kFastD + 2) * sizeof(float);
}

hipError_t launch_decode_fast(const AttnProblem& pr, hipStream_t st) {
  const kvq_packed& k = *pr.k;
  const kvq_packed& v = *pr.v;
  const kvq_shape& s = k.shape;
  FArgs a{};
  a.kc = reinterpret_cast<const uint8_t*>(k.codes);
  a.ks = k.scales;
  a.vc = reinterpret_cast<const uint8_t*>(v.codes);
  a.vs = v.scales;
  a.q = pr.q;
  a.kv_len = pr.kv_len;
  a.kchan = k.chan_scale;
  a.ws = static_cast<float*>(pr.ws);
  a.B = s.batch; a.L = s.layers; a.H = s.heads; a.T = s.tokens; a.Hq = pr.Hq; a.G = pr.Hq / s.heads;
  a.n_q = pr.n_q;
  a.nks = kFastD / k.codec.group;
  a.nvs = kFastD / v.codec.group;
  a.gv = v.codec.group;
  a.kW = k.codec.rot_width > 1 ? k.codec.rot_width : 0;
  {
    int e = 0;
    while ((1 << e) < a.kW) ++e;
    a.kkappa = (a.kW > 1) ? ((e % 2 == 0) ? ldexpf(1.0f, -e / 2) : (float)(1.0 / std::sqrt((double)a.kW))) : 1.0f;
  }
  a.sm_scale = pr.sm_scale;
  fast_split(s, pr.n_q, &a.blocks_per_unit, &a.wave_tokens);
  const long long units = (long long)s.batch * s.layers * s.heads;
  const dim3 grid(a.blocks_per_unit, (unsigned)units, (unsigned)pr.n_q);
  if (a.nks == 2) {
    if (a.nvs == 1) k_decode_mfma<2, 1><<<grid, kBlock, 0, st>>>(a);
    else if (a.nvs == 2) k_decode_mfma<2, 2><<<grid, kBlock, 0, st>>>(a);
    else k_decode_mfma<2, 4><<<grid, kBlock, 0, st>>>(a);
  } else {
    if (a.nvs == 1) k_decode_mfma<1, 1><<<grid, kBlock, 0, st>>>(a);
    else if (a.nvs == 2) k_decode_mfma<1, 2><<<grid, kBlock, 0, st>>>(a);
    else k_decode_mfma<1, 4><<<grid, kBlock, 0, st>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine_partials(pr, a.blocks_per_unit, st);
}

}  // namespace kvq

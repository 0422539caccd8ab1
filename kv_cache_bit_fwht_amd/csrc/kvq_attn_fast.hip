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
//  * online softmax per head against a reference maximum that moves only when a
//    logit exceeds it by more than 1 (log2 units), so rescaling is rare.
//  * P.V: v_mfma_f32_4x4x4_16b_f16, 16 blocks of (4 heads x 4 tokens) x
//    (4 tokens x 4 dims): lane l owns value word l%16 (16 dims, one scale
//    group) for tokens 8(l/16)..+7; A = fp16(p) * s_v, B = one byte of each of
//    4 tokens' words masked to its low 2, 4, 6 or 8 bits as fp16 subnormals, so
//    four accumulators per byte hold prefix sums of its fields weighted 1, 4,
//    16, 64 and the fields come out as differences after the loop.
//    Output: 2^24 * field - 2 * sum of the weights per group.
// A block of 8 wavefronts (two per SIMD) covers one token range of one (query,
// KV head) and hands its steps out from an LDS counter; it merges its
// wavefronts and writes one (o, m, l) partial, and the general combine kernel
// merges the blocks and rotates rotated values back.
#include <cmath>

#include "kvq_internal.hpp"

namespace kvq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr int kFastD = 256;
constexpr int kStep = 32;          // tokens per wavefront step
constexpr int kFastBlock = 512;    // threads per block: two wavefronts per SIMD

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
  int blocks_per_unit;             // blocks (and partials) per (query row, KV head)
};

__device__ __forceinline__ uint32_t h2bits(_Float16 h) { return (uint32_t)__builtin_bit_cast(uint16_t, h); }

// Lane (kg, n16) of a wavefront step: key code words of its two QK tiles, value
// word n16 of tokens 8kg..8kg+7, and the scale words of one token, 8kg + n16%8;
// the other lanes of its 16-lane row fetch those of the other seven tokens and a
// DPP row broadcast hands them round when they are used.
template <int NVS>
struct StepData {
  u32x4_t kw[2][2];    // key codes: QK tile u, row half (words 4kg.. and 16+4kg..)
  uint32_t ks;         // key scale(s) of token 8kg + n16%8 (fp16; both groups when there are two)
  uint32_t vw[8];      // value word n16 of tokens 8kg + j
  uint32_t vs[NVS == 4 ? 2 : 1];   // value scales of token 8kg + n16%8
};

// Per-lane byte offsets of a step's loads, relative to the step's first row in each array.
struct LaneOffsets {
  uint32_t k[2];       // key code bytes of QK tile u (row half 0; half 1 is +64)
  uint32_t ks;         // key scale row of token 8kg + n16%8
  uint32_t v;          // value code bytes of token 8kg, word n16
  uint32_t vs;         // value scale row of token 8kg + n16%8
};

template <int NKS, int NVS>
__device__ __forceinline__ LaneOffsets lane_offsets(int kg, int n16) {
  LaneOffsets o;
#pragma unroll
  for (int u = 0; u < 2; ++u) o.k[u] = (uint32_t)(8 * (n16 >> 2) + 4 * u + (n16 & 3)) * 128u + 16u * kg;
  const uint32_t sc = (uint32_t)(8 * kg + (n16 & 7));
  o.ks = sc * 2u * NKS;
  o.v = (uint32_t)(8 * kg) * 64u + 4u * n16;
  o.vs = sc * 2u * NVS;
  return o;
}

// Loads of the step whose first row is `rb`.  `rb` is wavefront-uniform, so each
// address is a scalar base plus the lane's 32-bit byte offset; the offsets pass
// through an empty asm so that the compiler cannot fold them into loop-invariant
// 64-bit per-lane pointers (two registers per stream).
template <int NKS, int NVS>
__device__ __forceinline__ void load_step(const FArgs& a, size_t rb, LaneOffsets o, StepData<NVS>& d) {
  asm volatile("" : "+v"(o.k[0]), "+v"(o.k[1]), "+v"(o.ks), "+v"(o.v), "+v"(o.vs));
  const char* kb = reinterpret_cast<const char*>(a.kc) + rb * 128;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    d.kw[u][0] = *reinterpret_cast<const u32x4_t*>(kb + o.k[u]);
    d.kw[u][1] = *reinterpret_cast<const u32x4_t*>(kb + o.k[u] + 64);
  }
  const char* ksb = reinterpret_cast<const char*>(a.ks) + rb * (2 * NKS);
  if constexpr (NKS == 2) d.ks = *reinterpret_cast<const uint32_t*>(ksb + o.ks);
  else d.ks = *reinterpret_cast<const uint16_t*>(ksb + o.ks);
  const char* vb = reinterpret_cast<const char*>(a.vc) + rb * 64;
#pragma unroll
  for (int j = 0; j < 8; ++j) d.vw[j] = *reinterpret_cast<const uint32_t*>(vb + o.v + 64 * j);
  const char* vsb = reinterpret_cast<const char*>(a.vs) + rb * (2 * NVS);
  if constexpr (NVS == 4) {
    const u32x2_t v2 = *reinterpret_cast<const u32x2_t*>(vsb + o.vs);
    d.vs[0] = v2[0];
    d.vs[1] = v2[1];
  } else if constexpr (NVS == 2) {
    d.vs[0] = *reinterpret_cast<const uint32_t*>(vsb + o.vs);
  } else {
    d.vs[0] = *reinterpret_cast<const uint16_t*>(vsb + o.vs);
  }
}

// Value of lane j of this lane's 16-lane row (DPP row broadcast); j is a constant after unrolling.
template <int J>
__device__ __forceinline__ uint32_t row_bcast_c(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x150 + J, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t row_bcast(uint32_t x, int j) {
  switch (j) {
    case 0: return row_bcast_c<0>(x);
    case 1: return row_bcast_c<1>(x);
    case 2: return row_bcast_c<2>(x);
    case 3: return row_bcast_c<3>(x);
    case 4: return row_bcast_c<4>(x);
    case 5: return row_bcast_c<5>(x);
    case 6: return row_bcast_c<6>(x);
    default: return row_bcast_c<7>(x);
  }
}

// fp16 value scales of tokens 8kg + k and 8kg + k + 1 (k constant) in this lane's
// value group, packed low/high.  vsel picks the group's half of a scale word and the
// all-ones mask vhi the second word of a pair (four groups per row).
// The broadcasts run with every lane active (a DPP read from a lane that a branch has
// switched off returns 0), so the word of a pair is picked with a bit mask, not a branch.
template <int NVS>
__device__ __forceinline__ uint32_t vscale_pair(const uint32_t* vs, int k, uint32_t vsel, uint32_t vhi) {
  uint32_t w0, w1;
  if constexpr (NVS == 4) {
    const uint32_t a0 = row_bcast(vs[0], k), b0 = row_bcast(vs[1], k);
    const uint32_t a1 = row_bcast(vs[0], k + 1), b1 = row_bcast(vs[1], k + 1);
    w0 = a0 ^ ((a0 ^ b0) & vhi);
    w1 = a1 ^ ((a1 ^ b1) & vhi);
  } else {
    w0 = row_bcast(vs[0], k);
    w1 = row_bcast(vs[0], k + 1);
  }
  return __builtin_amdgcn_perm(w1, w0, vsel);
}

// One block per (unit, token range, query): 8 wavefronts, two per SIMD.  The two
// wavefronts that share a SIMD do not run at the same speed (the older one is
// issued first), so the block's 32-token steps are handed out dynamically from an
// LDS counter instead of being split evenly in advance.
template <int NKS, int NVS>
__global__ __launch_bounds__(kFastBlock, 1) void k_decode_mfma(FArgs a) {
  constexpr int NW = kFastBlock / 64;                // wavefronts per block
  __shared__ float qs[4][kFastD + 16];
  __shared__ float qsum_s[4][2];
  __shared__ float so[NW][4][kFastD];               // per-wave outputs [wave][head][dim]
  __shared__ float sm[NW][4], sl[NW][4];            // per-wave reference max (log2 units) and sum
  __shared__ half8_t qbs[8][16];                     // MFMA B operands [chunk][4 kg + head]
  __shared__ int next_step;                          // next step of the block not yet handed out
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wavefront-uniform
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

  // ---- token range of this block and its steps
  const int bpu = a.blocks_per_unit;
  const int per_block = ((a.T + bpu - 1) / bpu + kStep - 1) / kStep * kStep;   // tokens per block
  const int t_begin = blockIdx.x * per_block;
  const int t_end = min(t_begin + per_block, n);
  const int nsteps = (t_end > t_begin) ? (t_end - t_begin + kStep - 1) / kStep : 0;
  const size_t row0 = (size_t)unit * a.T;
  const int vgrp = (16 * n16) / a.gv;                // scale group of this lane's value word
  const uint32_t vsel = (NVS > 1 && (vgrp & 1)) ? 0x07060302u : 0x05040100u;
  const uint32_t vhi = (NVS == 4 && (vgrp & 2)) ? 0xFFFFFFFFu : 0u;
  auto step_tok = [&](int j) { return t_begin + j * kStep; };   // first token of local step j
  // first row of local step j, clamped into the block's steps: a step past the end stands
  // for the last one (loads of it are discarded), and a block without steps reads the
  // unit's first rows, which always exist
  auto step_row = [&](int j) -> size_t {
    return row0 + (nsteps > 0 ? step_tok(max(min(j, nsteps - 1), 0)) : 0);
  };

  // The query is read first so that the prologue waits for it alone; each wavefront's
  // first two steps (w and w + NW, handed out statically) are loaded right after it and
  // land while the prologue runs.  Loads are never issued under a branch, so that every
  // wait names exactly the data it needs.
  const uint16_t* qsrc = a.q + (size_t)rq * a.Hq * kFastD + (size_t)h * G * kFastD;
  uint32_t qraw = 0u;                                // elements 2 tid, 2 tid + 1 of [4 heads][256]
  if (2 * tid < G * kFastD) qraw = *reinterpret_cast<const uint32_t*>(qsrc + 2 * tid);
  float2_t kch = float2_t{1.0f, 1.0f};               // key channel scales of those dims
  if (a.kchan) kch = *reinterpret_cast<const float2_t*>(a.kchan + ((size_t)l * a.H + h) * kFastD + 2 * (tid & 127));
  const LaneOffsets lofs = lane_offsets<NKS, NVS>(kg, n16);
  int i0 = wave, i1 = wave + NW;                     // steps held by the two buffers
  StepData<NVS> b0, b1;
  load_step<NKS, NVS>(a, step_row(i0), lofs, b0);
  load_step<NKS, NVS>(a, step_row(i1), lofs, b1);

  // ---- query prologue: q in the key coordinates (divide channel scale, rotate), fp32 in LDS
  {
    const int g = tid >> 7, d0 = 2 * (tid & 127);
    float x0 = h2f((uint16_t)(qraw & 0xffffu)), x1 = h2f((uint16_t)(qraw >> 16));
    if (a.kchan) {
      x0 = x0 / kch[0];
      x1 = x1 / kch[1];
    }
    qs[g][d0] = x0;
    qs[g][d0 + 1] = x1;
  }
  if (tid == 0) next_step = 2 * NW;
  __syncthreads();
  if (a.kW > 1) {
    for (int ls = 0; (1 << ls) < a.kW; ++ls) {
      const int s = 1 << ls;
      const int g = tid >> 7, pp = tid & 127;        // one butterfly per thread and stage
      const int ii = ((pp >> ls) << (ls + 1)) | (pp & (s - 1));
      const float x = qs[g][ii], y = qs[g][ii + s];
      qs[g][ii] = x + y;
      qs[g][ii + s] = x - y;
      __syncthreads();
    }
    for (int p = tid; p < 4 * kFastD; p += kFastBlock) qs[p >> 8][p & 255] *= a.kkappa;
    __syncthreads();
  }
  if (wave < 4) {  // per-group sums of the fp16 query (wave w: head w): sum_g q for the (c - 8) offset folding
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
  // Columns of heads >= G see an all-zero query row; their logits and output rows
  // are computed but never written.  They stay in LDS (read once per step) to keep
  // registers for the second buffer of loads in flight.
  const int hq = n16 & 3;                            // query head of this column
  if (wave == 0 && n16 < 4) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int w = (c < 4) ? (4 * kg + c) : (16 + 4 * kg + (c - 4));
      const int d0 = 8 * w;
      half8_t v;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const _Float16 lo = (_Float16)qs[hq][d0 + r];
        const _Float16 hi = (_Float16)qs[hq][d0 + r + 4];
        if (r & 1) {
          v[2 * r] = lo * (_Float16)0.0625f;
          v[2 * r + 1] = hi * (_Float16)0.0625f;
        } else {
          v[2 * r] = lo;
          v[2 * r + 1] = hi;
        }
      }
      qbs[c][4 * kg + hq] = v;
    }
  }
  __syncthreads();
  constexpr float kLog2e = 1.4426950408889634f;
  const float lsc = a.sm_scale * kLog2e;             // logits kept in log2 units
  const float cK = lsc * 16777216.0f;                // 2^24
  const float off0 = lsc * 8.0f * qsum_s[hq][0];
  const float off1 = lsc * 8.0f * qsum_s[hq][1];
  constexpr bool kone = (NKS == 1);                  // key group 256: one scale per row

  float4_t acc[16];
#pragma unroll
  for (int f = 0; f < 16; ++f) acc[f] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_ref = -INFINITY;       // reference max (log2 units) of head hq
  float l_part = 0.0f;           // sum of p over this lane's tokens (head hq)
  float w_part = 0.0f;           // sum of the fp16 weights fp16(p) * s_v over this lane's tokens (head hq, group vgrp)

  // One 32-token step on the loaded data `cur` (consumed in place: no register copies,
  // so the other buffer's loads stay in flight while this one computes).
  auto process = [&](const StepData<NVS>& cur, const int t0) {
    // ---- Q.K^T
    float4_t cq[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      cq[u][0] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      cq[u][1] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // The LDS index is made opaque per step so the operands are re-read here rather
    // than hoisted out of the loop into 32 loop-carried registers.
    int qi = 4 * kg + hq;
    asm volatile("" : "+v"(qi));
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const half8_t bq = qbs[c][qi];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t w = cur.kw[u][c >> 2][c & 3];
        const uint32_t w2 = w >> 8;
        const u32x4_t pr = u32x4_t{w & 0x000F000Fu, w & 0x00F000F0u, w2 & 0x000F000Fu, w2 & 0x00F000F0u};
        const half8_t av = __builtin_bit_cast(half8_t, pr);
        cq[u][c >> 2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bq, cq[u][c >> 2], 0, 0, 0);
      }
    }
    // logits (log2 units) of tokens 8kg + 4u + r, head hq
    float lg[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * u + r;                      // token 8kg + j
        const uint32_t kw2 = row_bcast(cur.ks, j);
        float s0, s1;
        if constexpr (kone) {
          s0 = s1 = h2f((uint16_t)kw2);
        } else {
          s0 = h2f((uint16_t)kw2);
          s1 = h2f((uint16_t)(kw2 >> 16));
        }
        lg[j] = s0 * (cq[u][0][r] * cK - off0) + s1 * (cq[u][1][r] * cK - off1);
      }
    }
    if (t0 + kStep > t_end) {                        // partial step: mask tokens >= t_end
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (t0 + 8 * kg + j >= t_end) lg[j] = -INFINITY;
    }
    // ---- online softmax (per head; lanes with equal n16%4 hold identical values).
    // The reference maximum moves only when a logit exceeds it by more than 1 (log2
    // units), so weights stay below 2 and p * s_v stays inside fp16 range; the
    // result does not depend on where the reference sits.
    float mt = lg[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mt = fmaxf(mt, lg[k]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool grow = mt > m_ref + 1.0f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mt : m_ref;
      const float alpha = grow ? ((m_ref == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_ref - m_new)) : 1.0f;
      m_ref = m_new;
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
    // ---- P.V weights: fp16(p) * s_v(token, group of this lane's value word), in fp16 pairs
    half4_t aw[2];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {                   // tokens 2 s2, 2 s2 + 1
      const float p0 = __builtin_amdgcn_exp2f(lg[2 * s2] - m_ref);   // masked tokens: exp2(-inf) = 0
      const float p1 = __builtin_amdgcn_exp2f(lg[2 * s2 + 1] - m_ref);
      l_part += p0 + p1;
      const uint32_t sv = vscale_pair<NVS>(cur.vs, 2 * s2, vsel, vhi);
      const half2_t w2 = half2_t{(_Float16)p0, (_Float16)p1} * __builtin_bit_cast(half2_t, sv);
      w_part = __builtin_amdgcn_fdot2(w2, half2_t{(_Float16)1.0f, (_Float16)1.0f}, w_part, false);
      aw[s2 >> 1][2 * (s2 & 1)] = w2[0];
      aw[s2 >> 1][2 * (s2 & 1) + 1] = w2[1];
    }
    // ---- P.V: byte k of the value words of tokens (4s..4s+3) holds dims 4k..4k+3 of this
    // lane's word.  B = the byte masked to its low 2, 4, 6 and 8 bits (fp16 subnormals),
    // so the four accumulators of byte k hold prefix sums of the fields weighted 1, 4,
    // 16, 64; the fields are separated after the loop.
#pragma unroll
    for (int s4 = 0; s4 < 2; ++s4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t sel = (uint32_t)k | (0x0Cu << 8) | ((uint32_t)(4 + k) << 16) | (0x0Cu << 24);
        const uint32_t r01 = __builtin_amdgcn_perm(cur.vw[4 * s4 + 1], cur.vw[4 * s4 + 0], sel);
        const uint32_t r23 = __builtin_amdgcn_perm(cur.vw[4 * s4 + 3], cur.vw[4 * s4 + 2], sel);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const uint32_t mask = (0x00040004u << (2 * ii)) - 0x00010001u;   // low 2(ii+1) bits of each half
          const u32x2_t bp = (ii == 3) ? u32x2_t{r01, r23} : u32x2_t{r01 & mask, r23 & mask};
          const half4_t bv = __builtin_bit_cast(half4_t, bp);
          acc[4 * k + ii] = __builtin_amdgcn_mfma_f32_4x4x4f16(aw[s4], bv, acc[4 * k + ii], 0, 0, 0);
        }
      }
    }
  };

  // next unclaimed step of the block (wavefront-uniform).  Every lane takes part in
  // the atomic, lane 0 adding 1 and the others 0, so lane 0 receives the old count
  // whatever order the lanes are served in, and no single-lane branch (which would cost
  // registers in this loop) is needed.
  auto claim = [&]() -> int {
    const int v = atomicAdd(&next_step, lane == 0 ? 1 : 0);
    return __builtin_amdgcn_readfirstlane(v);
  };
  // Each buffer is refilled right after it is consumed, with the next step claimed
  // then.  Steps a wavefront holds only grow (i0 < i1 < next i0 ...), so the first one
  // past the range ends the loop.
  while (i0 < nsteps) {
    process(b0, step_tok(i0));
    i0 = claim();
    load_step<NKS, NVS>(a, step_row(i0), lofs, b0);
    if (i1 >= nsteps) break;
    process(b1, step_tok(i1));
    i1 = claim();
    load_step<NKS, NVS>(a, step_row(i1), lofs, b1);
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
  // sum of the fp16 weights of head c in this lane's value group: the lane of the same 4-lane block with lane%4 == c
  const int base_l = lane & ~3;
  const float ws0 = __shfl(w_part, base_l | 0), ws1 = __shfl(w_part, base_l | 1);
  const float ws2 = __shfl(w_part, base_l | 2), ws3 = __shfl(w_part, base_l | 3);
  if (lane < 16) {
    const float wsum[4] = {ws0, ws1, ws2, ws3};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // prefix sums M1..M4 of byte k -> fields f0 = M1, f1 = (M2-M1)/4, f2 = (M3-M2)/16, f3 = (M4-M3)/64
        const float m1 = acc[4 * k][c], m2 = acc[4 * k + 1][c], m3 = acc[4 * k + 2][c], m4 = acc[4 * k + 3][c];
        const float f[4] = {m1, (m2 - m1) * 0.25f, (m3 - m2) * 0.0625f, (m4 - m3) * 0.015625f};
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) so[wave][c][16 * n16 + 4 * k + ii] = f[ii] * 16777216.0f - 2.0f * wsum[c];
      }
    }
  }
  if (lane < 4) {
    sm[wave][lane] = m_ref;
    sl[wave][lane] = l_part;
  }
  __syncthreads();
  // ---- merge the wavefronts of the block; one partial per (query row, head, block)
  constexpr float kLn2 = 0.6931471805599453f;
  const int P = kFastD + 2;
  const int d = tid & (kFastD - 1);
#pragma unroll
  for (int c0 = 0; c0 < 4; c0 += kFastBlock / kFastD) {
    const int c = c0 + tid / kFastD;                 // head of this thread
    if (c < G) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[w][c]);
      float L = 0.0f, O = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float wt = (sm[w][c] == -INFINITY) ? 0.0f : exp2f(sm[w][c] - M);
        L += wt * sl[w][c];
        O += wt * so[w][c][d];
      }
      float* dst = a.ws + ((rq * a.Hq + (size_t)h * G + c) * a.blocks_per_unit + blockIdx.x) * P;
      dst[d] = O;
      if (d == 0) {
        dst[kFastD] = (M == -INFINITY) ? -INFINITY : M * kLn2;
        dst[kFastD + 1] = L;
      }
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

static int fast_blocks_per_unit(const kvq_shape& s, int n_q) {
  const long long pairs = (long long)s.batch * s.layers * n_q * s.heads;
  // about one block (eight wavefronts, two per SIMD) per CU, and at least one step per wavefront
  long long bpu = (256 + pairs - 1) / pairs;
  const long long max_bpu = std::max(1, s.tokens / (8 * kStep));
  if (bpu > max_bpu) bpu = max_bpu;
  if (bpu < 1) bpu = 1;
  return (int)bpu;
}

size_t fast_part_bytes(const kvq_shape& s, int Hq, int n_q) {
  if (s.head_dim != kFastD || s.tokens % kStep != 0 || s.tokens == 0) return 0;
  const int bpu = fast_blocks_per_unit(s, n_q);
  const size_t b = (size_t)s.batch * s.layers * n_q * Hq * bpu * (kFastD + 2) * sizeof(float);
  return (b + 255) / 256 * 256;
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
  a.blocks_per_unit = fast_blocks_per_unit(s, pr.n_q);
  const long long units = (long long)s.batch * s.layers * s.heads;
  const dim3 grid(a.blocks_per_unit, (unsigned)units, (unsigned)pr.n_q);
  if (a.nks == 2) {
    if (a.nvs == 1) k_decode_mfma<2, 1><<<grid, kFastBlock, 0, st>>>(a);
    else if (a.nvs == 2) k_decode_mfma<2, 2><<<grid, kFastBlock, 0, st>>>(a);
    else k_decode_mfma<2, 4><<<grid, kFastBlock, 0, st>>>(a);
  } else {
    if (a.nvs == 1) k_decode_mfma<1, 1><<<grid, kFastBlock, 0, st>>>(a);
    else if (a.nvs == 2) k_decode_mfma<1, 2><<<grid, kFastBlock, 0, st>>>(a);
    else k_decode_mfma<1, 4><<<grid, kFastBlock, 0, st>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine_partials(pr, a.blocks_per_unit, st);
}

}  // namespace kvq

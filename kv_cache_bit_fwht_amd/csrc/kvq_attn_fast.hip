// MFMA decode attention over a packed cache with 3-, 4- or 5-bit signed-absmax keys
// (group 128 or 256, any Walsh-Hadamard rotation) and
// 2- or 4-bit values on an
// affine grid (signed absmax or the symmetric grid, group >= 64), head_dim 256,
// up to 4 query heads per KV head: the 64K-token decode workload of [E22L] ("Can
// 4-bit keys and 2-bit values hit a 1M-token memory budget?", What I tested: arm
// A, rotated 4-bit keys and 2-bit values at group 128), and the same cache with
// 4-bit values (the q4_0-style pair of [LCPP] Finding 1).
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
//    scale groups of s_g * (2^24 C_g - 2^(b-1) sum_g q), times the softmax
//    scale.  At 4 bits one AND places two codes 16 bits apart (dims e and e+4 of
//    a word) in their fp16 halves; at other widths each code is cut out with a
//    bit-field extract and pairs are packed with a shift-or.
//  * online softmax per head against a reference maximum that moves only when a
//    logit exceeds it by more than 1 (log2 units), so rescaling is rare.
//  * P.V: v_mfma_f32_4x4x4_16b_f16, 16 blocks of (4 heads x 4 tokens) x
//    (4 tokens x 4 dims): lane l owns value dims 16(l%16)..+15 (one scale
//    group; one code word at 2 bits, two at 4 bits) for tokens 8(l/16)..+7;
//    A = fp16(p) * s_v, B = one byte of each of 4 tokens' codes masked to its
//    low 2, 4, 6 and 8 bits (2-bit codes) or its low 4 and 8 bits (4-bit codes)
//    as fp16 subnormals, so the accumulators of a byte hold prefix sums of its
//    fields weighted 1, 4, 16, 64 (or 1, 16) and the fields come out as
//    differences after the loop: 16 accumulators either way.
//    Output: 2^24 * field - o * sum of the weights per group, o = 2^(b-1) for
//    signed absmax codes (levels c - 2^(b-1)) and (2^b - 1)/2 for the symmetric
//    grid.
// Several blocks of 8 wavefronts (two per SIMD) share the tokens of one (query,
// KV head): each block claims chunks of steps from a device-wide counter of the
// unit and hands their steps to its wavefronts from an LDS counter, then merges
// its wavefronts into one (o, m, l) partial.  The unit's last block to finish
// merges the partials into the output; with rotated values, or with more units
// than the workspace has counters for, a separate kernel does that merge.
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
constexpr int kMaxChunks = 256;    // chunks per (query row, KV head) at most
constexpr int kMaxSlots = kMaxChunks + 4;

struct FArgs {
  const uint8_t* kc;               // key codes, 32 b bytes per row
  const uint16_t* ks;              // key scales, nks per row
  const uint8_t* vc;               // value codes, 64 B (2-bit) or 128 B (4-bit) per row
  const uint16_t* vs;              // value scales, nvs per row
  const uint16_t* q;
  const int32_t* kv_len;
  const float* kchan;
  float* ws;
  int B, L, H, T, Hq, G, n_q;
  int nks, nvs, gv;                // scales per row, value group
  int kW;                          // key rotation width (0 = none)
  float kkappa;
  int vW;                          // value rotation width (0 = none): the merge rotates the output back
  float vkappa;
  float sm_scale;
  float voff;                      // value code offset: 2 (signed absmax, c - 2) or 1.5 (symmetric grid, c - 1.5)
  int blocks_per_unit;             // blocks (and partials) per (query row, KV head)
  int chunk_log2;                  // log2 of the 32-token steps per chunk (>= 4)
  int* ctr;                        // per (query row, KV head) chunk counters, or null (static chunks)
  int* done;                       // per (query row, KV head) finished-block counters, or null (separate merge)
  float* out;                      // merged output and log-sum-exp, written when done is set
  float* lse;
};

__device__ __forceinline__ uint32_t h2bits(_Float16 h) { return (uint32_t)__builtin_bit_cast(uint16_t, h); }

// Lane (kg, n16) of a wavefront step: key code words of its two QK tiles, the value
// codes of dims 16 n16..16 n16+15 of tokens 8kg..8kg+7, and the scale words of one
// token, 8kg + n16%8; the other lanes of its 16-lane row fetch those of the other
// seven tokens and a DPP row broadcast hands them round when they are used.
// The KB code words of 32 key dims, held in the vector types they are loaded as (so
// each load lands in place: copying a register that a load in flight will write would
// make the copy wait for it).  w(i) reads word i (i a constant after unrolling).
template <int KB> struct KeyRun {
  uint32_t v[KB];                                   // 3 or 5 words: 4-byte loads
  __device__ __forceinline__ uint32_t w(int i) const { return v[i]; }
};
template <> struct KeyRun<4> {
  u32x4_t v;
  __device__ __forceinline__ uint32_t w(int i) const { return v[i]; }
};

// The 4 KB bytes at p (4-byte aligned; 16-byte at KB = 4).
template <int KB>
__device__ __forceinline__ void load_run(const char* p, KeyRun<KB>& r) {
  if constexpr (KB == 4) {
    r.v = *reinterpret_cast<const u32x4_t*>(p);
  } else {
#pragma unroll
    for (int i = 0; i < KB; ++i) r.v[i] = *reinterpret_cast<const uint32_t*>(p + 4 * i);
  }
}

template <int NVS, int VB, int KB>
struct StepData {
  KeyRun<KB> kw[2][2];     // key codes of QK tile u, row half h: dims 128h + 32kg .. +31
  uint32_t ks;         // key scale(s) of token 8kg + n16%8 (fp16; both groups when there are two)
  typename std::conditional<VB == 2, uint32_t, u32x2_t>::type vw[8];   // value words of token 8kg + j:
                                                  // 2-bit word n16; 4-bit words 2 n16, 2 n16 + 1
  uint32_t vs[NVS == 4 ? 2 : 1];   // value scales of token 8kg + n16%8
};

// Per-lane byte offsets of a step's loads, relative to the step's first row in each array.
struct LaneOffsets {
  uint32_t k[2];       // key code bytes of QK tile u (row half 0; half 1 is +16 b)
  uint32_t ks;         // key scale row of token 8kg + n16%8
  uint32_t v;          // value code bytes of token 8kg, dims 16 n16..
  uint32_t vs;         // value scale row of token 8kg + n16%8
};

template <int NKS, int NVS, int VB, int KB>
__device__ __forceinline__ LaneOffsets lane_offsets(int kg, int n16) {
  LaneOffsets o;
#pragma unroll
  for (int u = 0; u < 2; ++u)
    o.k[u] = (uint32_t)(8 * (n16 >> 2) + 4 * u + (n16 & 3)) * (32u * KB) + (uint32_t)(4 * KB) * kg;
  const uint32_t sc = (uint32_t)(8 * kg + (n16 & 7));
  o.ks = sc * 2u * NKS;
  o.v = (uint32_t)(8 * kg) * (32u * VB) + (uint32_t)(2 * VB) * n16;
  o.vs = sc * 2u * NVS;
  return o;
}

// Loads of the step whose first row is `rb`.  `rb` is wavefront-uniform, so each
// address is a scalar base plus the lane's 32-bit byte offset; the offsets pass
// through an empty asm so that the compiler cannot fold them into loop-invariant
// 64-bit per-lane pointers (two registers per stream).
template <int NKS, int NVS, int VB, int KB>
__device__ __forceinline__ void load_step(const FArgs& a, size_t rb, LaneOffsets o, StepData<NVS, VB, KB>& d) {
  asm volatile("" : "+v"(o.k[0]), "+v"(o.k[1]), "+v"(o.ks), "+v"(o.v), "+v"(o.vs));
  const char* kb = reinterpret_cast<const char*>(a.kc) + rb * (32 * KB);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) load_run<KB>(kb + o.k[u] + hh * (16 * KB), d.kw[u][hh]);
  }
  const char* ksb = reinterpret_cast<const char*>(a.ks) + rb * (2 * NKS);
  if constexpr (NKS == 2) d.ks = *reinterpret_cast<const uint32_t*>(ksb + o.ks);
  else d.ks = *reinterpret_cast<const uint16_t*>(ksb + o.ks);
  const char* vb = reinterpret_cast<const char*>(a.vc) + rb * (32 * VB);
  if constexpr (VB == 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) d.vw[j] = *reinterpret_cast<const uint32_t*>(vb + o.v + 64 * j);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) d.vw[j] = *reinterpret_cast<const u32x2_t*>(vb + o.v + 128 * j);
  }
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

// The KB-bit field at bit `pos` (a constant after unrolling) of the word run w.
template <int KB>
__device__ __forceinline__ uint32_t key_field(const KeyRun<KB>& r, int pos) {
  const int wi = pos >> 5, sh = pos & 31;
  const uint32_t x = (sh + KB <= 32) ? (r.w(wi) >> sh) : __builtin_amdgcn_alignbit(r.w(wi + 1), r.w(wi), sh);
  return x & ((1u << KB) - 1u);
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

// x + (x of the lane 4 places along in the same row of 16, cyclically): joins the
// high- and low-part logits of a query head, which sit in columns n and n ^ 4.
__device__ __forceinline__ float add_row_ror4(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124, 0xF, 0xF, true));
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

// Adds 1 to a device-wide counter from lane 0 alone and returns the old value to
// the whole wavefront.  Same-address atomics from several lanes are serialised at
// the memory side, so the other lanes are masked off for the one instruction;
// the result is waited for inside the block, as its register is written late.
// Needs every lane of the wavefront active.
__device__ __forceinline__ int claim_global(int* ctr) {
  int old = 0;
  unsigned long long saved;
  asm volatile(
      "s_mov_b64 %1, exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "global_atomic_add %0, %2, %3, off sc0\n\t"
      "s_waitcnt vmcnt(0)\n\t"
      "s_mov_b64 exec, %1\n\t"
      "s_nop 4"
      : "+v"(old), "=&s"(saved)
      : "v"(ctr), "v"(1)
      : "memory");
  return __builtin_amdgcn_readfirstlane(old);
}

// One block per (unit, token range, query): 8 wavefronts, two per SIMD.  The two
// wavefronts that share a SIMD do not run at the same speed (the older one is
// issued first), so the block's 32-token steps are handed out dynamically from an
// LDS counter instead of being split evenly in advance.
template <int NKS, int NVS, int VB, int KB>
__global__ __launch_bounds__(kFastBlock, 1) void k_decode_mfma(FArgs a) {
  constexpr int NW = kFastBlock / 64;                // wavefronts per block
  __shared__ __align__(16) float qs[4][kFastD + 16];
  __shared__ float qsum_s[2][4][2];                 // [part][head][key group] sums of the MFMA query operand
  __shared__ float so[NW][4][kFastD];               // per-wave outputs [wave][head][dim]
  __shared__ float sm[NW][4], sl[NW][4];            // per-wave reference max (log2 units) and sum
  __shared__ half8_t qbs[8][32];                     // MFMA B operands [chunk][16 part + 4 kg + head]
  __shared__ int next_local;                         // next step index of the block not yet handed out
  __shared__ int slot_chunk[kMaxSlots];              // chunk of each slot of C local indices (-1 = not yet known)
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

  // ---- steps.  The unit's 32-token steps are grouped in chunks of C = 2^chunk_log2.
  // Slot s < S0 of block x holds chunk x + s * bpu (about three quarters of the unit's
  // chunks, taken without any atomic); every later chunk comes from a counter shared by
  // the unit's blocks, which sit on different XCDs whose speeds differ from run to run,
  // so the fast ones take more of the tail.  Without counters every slot is static.
  // Inside the block, wavefronts take local step indices from an LDS counter: index k
  // is step (k mod C) of the chunk of slot k / C.  Chunks are claimed one slot ahead by
  // the wavefront that takes a slot's first index, and only after that slot's own chunk
  // is known, so a block's chunks increase with the slot (static ones lie below
  // S0 * bpu, counted ones above): once a slot holds the end marker every later one
  // does too.
  const int bpu = a.blocks_per_unit;
  const int x = blockIdx.x;
  const int cl2 = a.chunk_log2;
  const int t_end = n;                               // tokens >= t_end are masked
  const int total_steps = (n + kStep - 1) / kStep;
  const int total_chunks = (total_steps + (1 << cl2) - 1) >> cl2;
  int* const ctr = a.ctr ? a.ctr + (rq * a.H + h) : nullptr;
  // static slots per block: at least 2 (slots 0 and 1 are known at the start)
  const int S0 = ctr ? max(2, (3 * total_chunks) / (4 * bpu)) : 0x7fffffff;
  const size_t row0 = (size_t)unit * a.T;
  const int vgrp = (16 * n16) / a.gv;                // scale group of this lane's value word
  const uint32_t vsel = (NVS > 1 && (vgrp & 1)) ? 0x07060302u : 0x05040100u;
  const uint32_t vhi = (NVS == 4 && (vgrp & 2)) ? 0xFFFFFFFFu : 0u;
  // first row of step s; a refill past the end re-reads the wavefront's last valid step
  // (an L2 hit), and a wavefront that never had a step reads the unit's first rows
  auto step_row = [&](int s, int last) -> size_t {
    return row0 + (size_t)(s >= 0 ? s : (last >= 0 ? last : 0)) * kStep;
  };

  // The query is read first so that the prologue waits for it alone; each wavefront's
  // first two steps (w and w + NW, handed out statically) are loaded right after it and
  // land while the prologue runs.  Loads are never issued under a branch, so that every
  // wait names exactly the data it needs.
  const uint16_t* qsrc = a.q + (size_t)rq * a.Hq * kFastD + (size_t)h * G * kFastD;
  // wavefront w < 4 holds query head w, dims 4 lane .. 4 lane + 3 (zero for heads >= G)
  u32x2_t qraw = u32x2_t{0u, 0u};
  float4_t kch = float4_t{1.0f, 1.0f, 1.0f, 1.0f};   // key channel scales of those dims
  if (wave < G) {
    qraw = *reinterpret_cast<const u32x2_t*>(qsrc + (size_t)wave * kFastD + 4 * lane);
    if (a.kchan) kch = *reinterpret_cast<const float4_t*>(a.kchan + ((size_t)l * a.H + h) * kFastD + 4 * lane);
  }
  const LaneOffsets lofs = lane_offsets<NKS, NVS, VB, KB>(kg, n16);
  // local indices wave and wave + NW of slot 0 (chunk x, C >= 16) are handed out statically
  auto first_step = [&](int k) { return (x < total_chunks && (x << cl2) + k < total_steps) ? (x << cl2) + k : -1; };
  int i0 = first_step(wave), i1 = first_step(wave + NW);   // steps held by the two buffers (-1: none)
  int last = i1 >= 0 ? i1 : i0;                       // the wavefront's latest valid step
  StepData<NVS, VB, KB> b0, b1;
  load_step<NKS, NVS, VB, KB>(a, step_row(i0, last), lofs, b0);
  load_step<NKS, NVS, VB, KB>(a, step_row(i1, last), lofs, b1);

  // ---- query prologue, one wavefront per query head (no block barrier until the end):
  // q in the key coordinates (divide by the channel scale, rotate: strides 1 and 2 in the
  // lane, 4 to 128 across lanes), then the MFMA B operands and per-group offset sums.
  for (int k = tid; k < kMaxSlots; k += kFastBlock)
    slot_chunk[k] = (k == 0) ? min(x, total_chunks)
                  : (k == 1) ? (x < total_chunks ? min(x + bpu, total_chunks) : total_chunks) : -1;
  if (tid == 0) next_local = 2 * NW;
  // B operands: chunk c < 4 -> dims 32kg + 8c .. +7 (group 0), c >= 4 -> dims 128 + 32kg + 8(c-4) .. +7.
  // Register order of the 8 k-slots: at 4 bits dims (0,4), (1,5)/16, (2,6), (3,7)/16 of
  // the 8 (the order one AND per pair leaves the codes in); at other widths dims 0..7.
  // Column n holds query head n % 4: its fp16 rounding (high part) where n / 4 is
  // even, the fp16 rounding of what that leaves (low part) where it is odd, so the
  // two columns' logits add up to those of the query with 22 bits or so instead of
  // 11.  Each part folds the (c - 8) code offset with its own per-group sum.
  // Columns of heads >= G see an all-zero query row; their logits and output rows
  // are computed but never written.  They stay in LDS (read once per step) to keep
  // registers for the second buffer of loads in flight.
  if (wave < 4) {
    float v[4] = {h2f((uint16_t)(qraw[0] & 0xffffu)), h2f((uint16_t)(qraw[0] >> 16)),
                  h2f((uint16_t)(qraw[1] & 0xffffu)), h2f((uint16_t)(qraw[1] >> 16))};
    if (a.kchan) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = v[e] / kch[e];
    }
    if (a.kW > 1) {
      if (a.kW >= 2) {                               // stride 1
        const float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
        v[0] = x0 + x1; v[1] = x0 - x1; v[2] = x2 + x3; v[3] = x2 - x3;
      }
      if (a.kW >= 4) {                               // stride 2
        const float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
        v[0] = x0 + x2; v[2] = x0 - x2; v[1] = x1 + x3; v[3] = x1 - x3;
      }
      for (int m = 1; 4 * m < a.kW; m <<= 1) {       // stride 4m: lane ^ m
        const bool hi = (lane & m) != 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y = __shfl_xor(v[e], m);
          v[e] = hi ? (y - v[e]) : (v[e] + y);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] *= a.kkappa;
    }
    *reinterpret_cast<float4_t*>(&qs[wave][4 * lane]) = float4_t{v[0], v[1], v[2], v[3]};
    // lane -> B entry (chunk c, lane group kg, part); its 8 dims are d0 .. d0 + 7
    const int c = lane & 7, ekg = (lane >> 3) & 3, epart = lane >> 5;
    const int d0 = 8 * ((c < 4) ? (4 * ekg + c) : (16 + 4 * ekg + (c - 4)));
    const float4_t f0 = *reinterpret_cast<const float4_t*>(&qs[wave][d0]);
    const float4_t f1 = *reinterpret_cast<const float4_t*>(&qs[wave][d0 + 4]);
    const float f[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
    half8_t hv;
    float gsum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = e >> 1;                          // 4 bits: slot e is dim d0 + r (+4 when e is odd)
      const float sc = (KB == 4 && (r & 1)) ? 0.0625f : 1.0f;   // the shifted nibble reads as 16 c
      const float t = (KB == 4 ? f[r + 4 * (e & 1)] : f[e]) * sc;
      const _Float16 th = (_Float16)t;
      // the low part is held times 2^11, so it and its products with the subnormal codes
      // stay in the range of the high part's (where they lose no bits in the dot product)
      const _Float16 tv = epart ? (_Float16)((t - (float)th) * 2048.0f) : th;
      hv[e] = tv;
      gsum += (float)tv / sc;
    }
    qbs[c][16 * epart + 4 * ekg + wave] = hv;
    // sum over the lanes of the same (part, key group): lane bits 0, 1 (c % 4) and 3, 4 (kg)
    gsum += __shfl_xor(gsum, 1);
    gsum += __shfl_xor(gsum, 2);
    gsum += __shfl_xor(gsum, 8);
    gsum += __shfl_xor(gsum, 16);
    if ((lane & 0x1B) == 0) qsum_s[epart][wave][c >> 2] = gsum;
  }
  const int hq = n16 & 3;                            // query head of this lane's column
  const int part = (n16 >> 2) & 1;                   // 0: high part, 1: low part
  __syncthreads();
  constexpr float kLog2e = 1.4426950408889634f;
  const float lsc = a.sm_scale * kLog2e;             // logits kept in log2 units
  const float pscale = part ? (1.0f / 2048.0f) : 1.0f;   // undoes the low part's 2^11
  const float cK = lsc * 16777216.0f * pscale;       // 2^24
  constexpr float kKeyOff = (float)(1 << (KB - 1));  // key levels c - 2^(b-1)
  const float off0 = lsc * kKeyOff * qsum_s[part][hq][0] * pscale;
  const float off1 = lsc * kKeyOff * qsum_s[part][hq][1] * pscale;
  constexpr bool kone = (NKS == 1);                  // key group 256: one scale per row

  float4_t acc[16];
#pragma unroll
  for (int f = 0; f < 16; ++f) acc[f] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_ref = -INFINITY;       // reference max (log2 units) of head hq
  float l_part = 0.0f;           // sum of p over this lane's tokens (head hq)
  float w_part = 0.0f;           // sum of the fp16 weights fp16(p) * s_v over this lane's tokens (head hq, group vgrp)

  // One 32-token step on the loaded data `cur` (consumed in place: no register copies,
  // so the other buffer's loads stay in flight while this one computes).
  auto process = [&](const StepData<NVS, VB, KB>& cur, const int t0) {
    // ---- Q.K^T
    float4_t cq[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      cq[u][0] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      cq[u][1] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // The LDS index is made opaque per step so the operands are re-read here rather
    // than hoisted out of the loop into 32 loop-carried registers.
    int qi = 16 * part + 4 * kg + hq;
    asm volatile("" : "+v"(qi));
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const half8_t bq = qbs[c][qi];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4_t pr;
        if constexpr (KB == 4) {
          const uint32_t w = cur.kw[u][c >> 2].w(c & 3);
          const uint32_t w2 = w >> 8;
          pr = u32x4_t{w & 0x000F000Fu, w & 0x00F000F0u, w2 & 0x000F000Fu, w2 & 0x00F000F0u};
        } else {
          const KeyRun<KB>& wv = cur.kw[u][c >> 2];
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {           // dims 8(c%4) + 2pp, + 1 of the half's 32
            const int pos = (8 * (c & 3) + 2 * pp) * KB;
            pr[pp] = key_field<KB>(wv, pos) | (key_field<KB>(wv, pos + KB) << 16);
          }
        }
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
#pragma unroll
    for (int j = 0; j < 8; ++j) lg[j] = add_row_ror4(lg[j]);   // high + low part
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
    // ---- P.V: byte k of the lane's value codes of tokens (4s..4s+3) holds dims 4k..4k+3
    // (2-bit) or 2k, 2k+1 (4-bit) of its 16.  B = the byte masked to its low 2, 4, 6 and 8
    // bits, or its low 4 and 8 bits (fp16 subnormals), so the accumulators of byte k hold
    // prefix sums of the fields weighted 1, 4, 16, 64 (or 1, 16); the fields are
    // separated after the loop.
    constexpr int NB = (VB == 2) ? 4 : 8;            // code bytes per lane and token
    constexpr int NM = (VB == 2) ? 4 : 2;            // masks per byte
#pragma unroll
    for (int s4 = 0; s4 < 2; ++s4) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int kb = k & 3, wi = k >> 2;           // byte of the word, word of the lane (4-bit)
        const uint32_t sel = (uint32_t)kb | (0x0Cu << 8) | ((uint32_t)(4 + kb) << 16) | (0x0Cu << 24);
        auto word = [&](int t) -> uint32_t {         // the lane's code word wi of token t
          if constexpr (VB == 2) return cur.vw[t];
          else return cur.vw[t][wi];
        };
        const uint32_t r01 = __builtin_amdgcn_perm(word(4 * s4 + 1), word(4 * s4 + 0), sel);
        const uint32_t r23 = __builtin_amdgcn_perm(word(4 * s4 + 3), word(4 * s4 + 2), sel);
#pragma unroll
        for (int ii = 0; ii < NM; ++ii) {
          // low VB(ii+1) bits of each half
          const uint32_t mask = ((0x00010001u << (VB * (ii + 1))) - 0x00010001u);
          const u32x2_t bp = (ii == NM - 1) ? u32x2_t{r01, r23} : u32x2_t{r01 & mask, r23 & mask};
          const half4_t bv = __builtin_bit_cast(half4_t, bp);
          acc[NM * k + ii] = __builtin_amdgcn_mfma_f32_4x4x4f16(aw[s4], bv, acc[NM * k + ii], 0, 0, 0);
        }
      }
    }
  };

  // Next step for this wavefront (wavefront-uniform), or -1 when the block is done.
  // Every lane takes part in the LDS atomic (lane 0 adds 1, the others 0), so lane 0
  // receives the old count whatever order the lanes are served in, with no single-lane
  // branch (which would cost registers in this loop); the counter atomic likewise.
  auto claim = [&]() -> int {
    const int k = __builtin_amdgcn_readfirstlane(atomicAdd(&next_local, lane == 0 ? 1 : 0));
    const int sl = min(k >> cl2, kMaxSlots - 2), pos = k & ((1 << cl2) - 1);
    int c;
    do {                                             // the slot's chunk, once its claimer has written it
      c = __builtin_amdgcn_readfirstlane(
          __hip_atomic_load(&slot_chunk[sl], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    } while (c < 0);
    if (pos == 0) {                                  // first index of the slot: claim the next slot's chunk
      int nc = total_chunks;
      if (c < total_chunks) {
        nc = (sl + 1 < S0) ? c + bpu : S0 * bpu + claim_global(ctr);
        nc = min(nc, total_chunks);
      }
      __hip_atomic_store(&slot_chunk[sl + 1], nc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    const int step = (c << cl2) + pos;
    return (c < total_chunks && step < total_steps) ? step : -1;
  };
  // Each buffer is refilled right after it is consumed.  A wavefront's claims follow
  // its local indices, so once one returns -1 so do all later ones: the first -1 ends
  // the loop with no claimed step left unprocessed.
  while (i0 >= 0) {
    process(b0, i0 * kStep);
    i0 = claim();
    if (i0 >= 0) last = i0;
    load_step<NKS, NVS, VB, KB>(a, step_row(i0, last), lofs, b0);
    if (i1 < 0) break;
    process(b1, i1 * kStep);
    i1 = claim();
    if (i1 >= 0) last = i1;
    load_step<NKS, NVS, VB, KB>(a, step_row(i1, last), lofs, b1);
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
      if constexpr (VB == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // prefix sums M1..M4 of byte k -> fields f0 = M1, f1 = (M2-M1)/4, f2 = (M3-M2)/16, f3 = (M4-M3)/64
          const float m1 = acc[4 * k][c], m2 = acc[4 * k + 1][c], m3 = acc[4 * k + 2][c], m4 = acc[4 * k + 3][c];
          const float f[4] = {m1, (m2 - m1) * 0.25f, (m3 - m2) * 0.0625f, (m4 - m3) * 0.015625f};
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) so[wave][c][16 * n16 + 4 * k + ii] = f[ii] * 16777216.0f - a.voff * wsum[c];
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          // prefix sums M1, M2 of byte k -> fields f0 = M1, f1 = (M2-M1)/16
          const float m1 = acc[2 * k][c], m2 = acc[2 * k + 1][c];
          so[wave][c][16 * n16 + 2 * k] = m1 * 16777216.0f - a.voff * wsum[c];
          so[wave][c][16 * n16 + 2 * k + 1] = ((m2 - m1) * 0.0625f) * 16777216.0f - a.voff * wsum[c];
        }
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
      // merged in this kernel: device-coherent stores (written through to memory), so
      // that another XCD's block can read them without any cache being flushed
      auto put = [&](float* ptr, float val) {
        if (a.done) __hip_atomic_store(ptr, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else *ptr = val;
      };
      put(dst + d, O);
      if (d == 0) {
        put(dst + kFastD, (M == -INFINITY) ? -INFINITY : M * kLn2);
        put(dst + kFastD + 1, L);
      }
    }
  }
  if (!a.done) return;
  // ---- the unit's last block to finish merges the bpu partials:
  // out = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s, lse = M + ln(that sum).
  // Every thread waits until its coherent partial stores have completed before the
  // block is counted, and the last block reads the partials with coherent loads.
  __shared__ int is_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(a.done + (rq * a.H + h), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == bpu - 1);
  }
  __syncthreads();
  if (!is_last) return;
  auto get = [](const float* ptr) { return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  // (m, l) of every partial into LDS (the per-wave output buffer is free by now), all
  // loads in flight at once; then each thread's output loads go out 8 at a time.
  static_assert(8 * kMaxChunks + 4 * kFastD <= NW * 4 * kFastD, "merge tables exceed the per-wave output buffer");
  float* const pm = &so[0][0][0];                    // [head][block], stride kMaxChunks (blocks <= chunks)
  float* const pl = pm + 4 * kMaxChunks;
  float* const rot = pl + 4 * kMaxChunks;             // [head][dim] merged output before rotating back
  const float* const ubase = a.ws + (rq * a.Hq + (size_t)h * G) * bpu * P;
  for (int t = tid; t < G * bpu; t += kFastBlock) {
    const int c = t / bpu, sb = t - c * bpu;
    const float* p = ubase + (size_t)t * P;
    const float mv = get(p + kFastD), lv = get(p + kFastD + 1);
    pm[c * kMaxChunks + sb] = mv;
    pl[c * kMaxChunks + sb] = lv;
  }
  __syncthreads();
#pragma unroll
  for (int c0 = 0; c0 < 4; c0 += kFastBlock / kFastD) {
    const int c = c0 + tid / kFastD;
    if (c < G) {
      const size_t rh = rq * a.Hq + (size_t)h * G + c;
      const float* src = a.ws + rh * bpu * P;
      const float* cm = pm + c * kMaxChunks;
      const float* cl = pl + c * kMaxChunks;
      float M = -INFINITY;
      for (int sb = 0; sb < bpu; ++sb) M = fmaxf(M, cm[sb]);
      float L = 0.0f, O = 0.0f;
      for (int s0 = 0; s0 < bpu; s0 += 8) {
        float ov[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ov[j] = get(src + (size_t)min(s0 + j, bpu - 1) * P + d);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (s0 + j < bpu) {
            const float ms = cm[s0 + j];
            const float wt = (ms == -INFINITY) ? 0.0f : expf(ms - M);
            L += wt * cl[s0 + j];
            O += wt * ov[j];
          }
        }
      }
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      if (a.vW > 1) rot[c * kFastD + d] = O * inv;
      else a.out[rh * kFastD + d] = O * inv;
      if (d == 0 && a.lse) a.lse[rh] = L > 0.0f ? M + logf(L) : -INFINITY;
    }
  }
  if (a.vW > 1) {   // rotated values: the normalised transform is its own inverse
    __syncthreads();
    const int c = tid >> 7, pp = tid & 127;          // one butterfly per thread and stage (4 heads x 128)
    for (int ls = 0; (1 << ls) < a.vW; ++ls) {
      const int st = 1 << ls;
      const int ii = ((pp >> ls) << (ls + 1)) | (pp & (st - 1));
      if (c < G) {
        const float x = rot[c * kFastD + ii], y = rot[c * kFastD + ii + st];
        rot[c * kFastD + ii] = x + y;
        rot[c * kFastD + ii + st] = x - y;
      }
      __syncthreads();
    }
    for (int p = tid; p < G * kFastD; p += kFastBlock)
      a.out[(rq * a.Hq + (size_t)h * G) * kFastD + p] = rot[p] * a.vkappa;
  }
  if (tid == 0) {   // ready for the next call: every block of the unit has made its last claim
    ctr[0] = 0;
    a.done[rq * a.H + h] = 0;
  }
}

// Merge of the blocks' partials for one (query row, query head) per wavefront, when
// the values are not rotated and the blocks took fixed chunks (no counters):
// out = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s, lse = M + ln(that sum).
// Each lane owns 4 of the 256 dimensions.
__global__ __launch_bounds__(256) void k_fast_combine(const float* __restrict__ ws, int S, int Hq, int G, int H,
                                                      long long rows_hq, float* out, float* lse, int* ctr) {
  const long long rh = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rh >= rows_hq) return;
  const int lane = threadIdx.x & 63;
  constexpr int P = kFastD + 2;
  const float* src = ws + (size_t)rh * S * P;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, src[(size_t)s * P + kFastD]);
  float L = 0.0f;
  float4_t o = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < S; ++s) {
    const float* p = src + (size_t)s * P;
    const float ms = p[kFastD];
    const float w = (ms == -INFINITY) ? 0.0f : expf(ms - M);
    L += w * p[kFastD + 1];
    const float4_t v = *reinterpret_cast<const float4_t*>(p + 4 * lane);
    o += w * v;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  *reinterpret_cast<float4_t*>(out + (size_t)rh * kFastD + 4 * lane) = o * inv;
  const int j = (int)(rh % Hq);
  if (lane == 0) {
    if (lse) lse[rh] = L > 0.0f ? M + logf(L) : -INFINITY;
    if (ctr && j % G == 0) ctr[(rh / Hq) * H + j / G] = 0;   // ready for the next call
  }
}

// ------------------------------------------------------------------ host side

bool fast_decode_supported(const kvq_packed& k, const kvq_packed& v, int Hq) {
  const kvq_shape& s = k.shape;
  if (s.head_dim != kFastD) return false;
  if (s.tokens % kStep != 0 || s.tokens == 0) return false;
  if (Hq / s.heads > 4) return false;
  if (k.codec.codebook != KVQ_INT_ABSMAX) return false;
  const int kb = k.codec.bits;
  // 6- and 8-bit keys need more registers than two wavefronts per SIMD leave (scratch
  // spills); 2-bit keys came out with logit errors of ~1e-4 here (4x those of 4-bit keys,
  // over the 1e-4 lse bar), so they stay on the general kernel
  if (kb < 3 || kb > 5) return false;
  if (k.codec.group != 128 && k.codec.group != 256) return false;
  // 2- or 4-bit values: signed absmax (levels c - 2^(b-1)) or the symmetric grid (levels c - (2^b - 1)/2)
  if (v.codec.codebook != KVQ_INT_ABSMAX && v.codec.codebook != KVQ_INT_SYM) return false;
  if (v.codec.bits != 2 && v.codec.bits != 4) return false;
  if (v.codec.group < 64) return false;   // a P.V block's 4 value words share one scale group
  if (v.chan_scale) return false;
  return true;
}

// Chunk size: at least 16 steps (one step per wavefront of a block to start with), and
// at most kMaxChunks chunks per (query row, KV head).
static int fast_chunk_log2(const kvq_shape& s) {
  const long long steps = s.tokens / kStep;
  int cl2 = 4;
  while (((steps + (1LL << cl2) - 1) >> cl2) > kMaxChunks) ++cl2;
  return cl2;
}

static int fast_blocks_per_unit(const kvq_shape& s, int n_q) {
  const long long pairs = (long long)s.batch * s.layers * n_q * s.heads;
  // about one block (eight wavefronts, two per SIMD) per CU, and no more blocks than chunks
  long long bpu = (256 + pairs - 1) / pairs;
  const long long chunks = ((long long)(s.tokens / kStep) + (1LL << fast_chunk_log2(s)) - 1) >> fast_chunk_log2(s);
  if (bpu > chunks) bpu = chunks;
  if (bpu < 1) bpu = 1;
  return (int)bpu;
}

size_t fast_part_bytes(const kvq_shape& s, int Hq, int n_q) {
  if (s.head_dim != kFastD || s.tokens % kStep != 0 || s.tokens == 0) return 0;
  const int bpu = fast_blocks_per_unit(s, n_q);
  const size_t b = (size_t)s.batch * s.layers * n_q * Hq * bpu * (kFastD + 2) * sizeof(float);
  return (b + 255) / 256 * 256;
}

template <int VB, int KB>
static void launch_mfma(const FArgs& a, dim3 grid, hipStream_t st) {
  if (a.nks == 2) {
    if (a.nvs == 1) k_decode_mfma<2, 1, VB, KB><<<grid, kFastBlock, 0, st>>>(a);
    else if (a.nvs == 2) k_decode_mfma<2, 2, VB, KB><<<grid, kFastBlock, 0, st>>>(a);
    else k_decode_mfma<2, 4, VB, KB><<<grid, kFastBlock, 0, st>>>(a);
  } else {
    if (a.nvs == 1) k_decode_mfma<1, 1, VB, KB><<<grid, kFastBlock, 0, st>>>(a);
    else if (a.nvs == 2) k_decode_mfma<1, 2, VB, KB><<<grid, kFastBlock, 0, st>>>(a);
    else k_decode_mfma<1, 4, VB, KB><<<grid, kFastBlock, 0, st>>>(a);
  }
}

template <int KB>
static void launch_mfma_k(const FArgs& a, int vb, dim3 grid, hipStream_t st) {
  if (vb == 2) launch_mfma<2, KB>(a, grid, st);
  else launch_mfma<4, KB>(a, grid, st);
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
  a.vW = v.codec.rot_width > 1 ? v.codec.rot_width : 0;
  {
    int e = 0;
    while ((1 << e) < a.vW) ++e;
    a.vkappa = (a.vW > 1) ? ((e % 2 == 0) ? ldexpf(1.0f, -e / 2) : (float)(1.0 / std::sqrt((double)a.vW))) : 1.0f;
  }
  a.sm_scale = pr.sm_scale;
  const int vb = v.codec.bits;
  a.voff = (v.codec.codebook == KVQ_INT_SYM) ? 0.5f * (float)((1 << vb) - 1) : (float)(1 << (vb - 1));
  a.blocks_per_unit = fast_blocks_per_unit(s, pr.n_q);
  a.chunk_log2 = fast_chunk_log2(s);
  // shared chunk counters when the rows fit the workspace's counter region
  const long long rows_kv = (long long)s.batch * s.layers * pr.n_q * s.heads;
  a.ctr = (pr.ctr && rows_kv <= kWsCounterRows) ? pr.ctr : nullptr;
  // unrotated values without channel scales: the last block of a unit merges its partials
  const bool fused = a.ctr && !v.chan_scale;
  a.done = fused ? pr.ctr + kWsCounterRows : nullptr;
  a.out = pr.out;
  a.lse = pr.lse;
  const long long units = (long long)s.batch * s.layers * s.heads;
  const dim3 grid(a.blocks_per_unit, (unsigned)units, (unsigned)pr.n_q);
  switch (k.codec.bits) {
    case 3: launch_mfma_k<3>(a, vb, grid, st); break;
    case 4: launch_mfma_k<4>(a, vb, grid, st); break;
    default: launch_mfma_k<5>(a, vb, grid, st); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fused) return e;
  if (v.codec.rot_width > 1 || v.chan_scale) return launch_combine_partials(pr, a.blocks_per_unit, a.ctr, st);
  const long long rows_hq = (long long)s.batch * s.layers * pr.n_q * pr.Hq;
  k_fast_combine<<<(unsigned)((rows_hq + 3) / 4), 256, 0, st>>>(a.ws, a.blocks_per_unit, pr.Hq, a.G, s.heads, rows_hq,
                                                             pr.out, pr.lse, a.ctr);
  return hipGetLastError();
}

}  // namespace kvq

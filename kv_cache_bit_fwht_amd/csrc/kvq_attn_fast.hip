// MFMA decode attention over a packed cache with 2-, 3-, 4- or 5-bit signed-absmax keys
// (group 128 or 256, any Walsh-Hadamard rotation) and
// 2-, 3- or 4-bit values on an
// affine grid (signed absmax or the symmetric grid, group >= 64) or 2-bit Gaussian
// Lloyd-Max values ([E22L] Result: the next test, on rotated values), head_dim 256,
// up to 4 query heads per KV head: the 64K-token decode workload of [E22L] ("Can
// 4-bit keys and 2-bit values hit a 1M-token memory budget?", What I tested: arm
// A, rotated 4-bit keys and 2-bit values at group 128), and the same cache with
// 4-bit values (the q4_0-style pair of [LCPP] Finding 1).
//
// Why MFMA: at 0.39 bytes per cached value, HBM speed leaves about two VALU
// lane-ops per value, while unpacking plus four grouped-head multiply-adds per
// key and per value costs four to five.  Both contractions go to the matrix
// cores; the VALU only unpacks codes and runs the softmax.
//
// Per wavefront, 32 tokens per step:
//  * Q.K^T: v_mfma_i32_16x16x64_i8, A = 16 tokens x 64 dims of key codes as
//    bytes, B = the rotated query as an integer in four 7-bit digits, 4 digits x
//    4 heads over the 16 columns, so lane (kg, n) ends with digit n/4's exact
//    integer logits of head n%4 for tokens 8kg..8kg+7.  Logit = sum over the two
//    scale groups of s_g * (sum of digit * (c - 2^(b-1))), weighted 2^(7 digit)
//    over the query scale and added over the digit columns, times the softmax
//    scale.
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
#include "kvq_quant256.hpp"

namespace kvq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kFastD = 256;

// Timeline build (-DKVQ_TIMELINE, libkvq_timeline.so): lane 0 of every wavefront of the
// first kTimelineBlocks blocks records s_memrealtime (a 100 MHz clock) at fixed points of
// the MFMA decode, read back with kvq_timeline_read.  The default build compiles the
// stamps out.
constexpr int kTimelineBlocks = 4096;
constexpr int kTimelineSlots = 16;
#ifdef KVQ_TIMELINE
__device__ unsigned long long g_kvq_timeline[kTimelineBlocks * 8 * kTimelineSlots];
#define KVQ_STAMP(slot)                                                                                    \
  do {                                                                                                     \
    const unsigned long long t_ = __builtin_amdgcn_s_memrealtime();                                        \
    const long long b_ = blockIdx.x + (long long)gridDim.x * (blockIdx.y + (long long)gridDim.y * blockIdx.z); \
    if (lane == 0 && b_ < kTimelineBlocks) g_kvq_timeline[(b_ * 8 + wave) * kTimelineSlots + (slot)] = t_; \
  } while (0)
#else
#define KVQ_STAMP(slot) \
  do {                  \
  } while (0)
#endif
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
  const float* kmean;              // key mean [L][H][256] shifted into the lse by the in-kernel merge, or null
  float* ws;
  int B, L, H, T, Hq, G, n_q;
  int nks, nvs, gv;                // scales per row, value group
  int kW;                          // key rotation width (0 = none)
  float kkappa;
  int vW;                          // value rotation width (0 = none): the merge rotates the output back
  float vkappa;
  float sm_scale;
  float voff;                      // value code offset: 2 (signed absmax, c - 2) or 1.5 (symmetric grid, c - 1.5)
  uint32_t vlut_lo, vlut_hi;       // Lloyd-Max values: low and high bytes of levels 0-3 in fp16
  uint32_t vlut_lo2, vlut_hi2;     // 3-bit Lloyd-Max values: the same of levels 4-7
  int vll;                         // 1: Lloyd-Max values (levels from vlut, no offset)
  int blocks_per_unit;             // blocks (and partials) per (query row, KV head)
  int chunk_log2;                  // log2 of the 32-token steps per chunk (>= 3)
  int* ctr;                        // per (query row, KV head) chunk counters, or null (static chunks)
  int* done;                       // per (query row, KV head) finished-block counters, or null (separate merge)
  float* out;                      // merged output and log-sum-exp, written when done is set
  float* lse;
  // fused append: fp16 rows [B][L][H][app_n][256] coded into tokens [app_t0, app_t0 + app_n)
  // through the writable views below (app_n = 0: none)
  const uint16_t* app_k;
  const uint16_t* app_v;
  int app_t0, app_n;
  uint32_t* kcw;
  uint16_t* ksw;
  uint32_t* vcw;
  uint16_t* vsw;
  int app_kg, app_vg;              // key and value groups
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
  // 3-bit values: the lane's 6 bytes start at byte 6 n16, 2-byte aligned only; the lane
  // loads the 4-byte aligned 8 bytes around them (and drops 16 bits when n16 is odd)
  o.v = (uint32_t)(8 * kg) * (32u * VB) + (VB == 3 ? (uint32_t)((6 * n16) & ~3) : (uint32_t)(2 * VB) * n16);
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
    for (int j = 0; j < 8; ++j) d.vw[j] = *reinterpret_cast<const u32x2_t*>(vb + o.v + 32 * VB * j);
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

// The QK product runs on the int8 matrix cores: key codes as bytes (0 .. 2^KB - 1),
// the query as 7-bit digits of an integer, so every dot product is an
// exact integer sum.  Four digits (the B operand's 16 columns are 4 digits x 4 heads)
// carry the rotated fp32 query exactly.  (The fp16 matrix cores align their products by exponent field,
// so fp16 subnormal codes, the other cheap operand form, lose low bits of the smaller
// products: up to 1e-4 of the largest, biased, in measurement.)
// A operand of QK chunk c (0..3) of one tile: 16 bytes per lane, the codes of 16 of
// the lane's 64 key dims; key_dim gives which, for byte J of the lane's k group kg
// (the query operand is laid out by the same map).  Chunk c lies in the dims
// 128 (c >> 1) .. +127 (one key group of 128); run = the lane's 32 dims there.
template <int KB>
__device__ __forceinline__ int key_dim(int c, int kg, int J) {
  const int base = 128 * (c >> 1) + 32 * kg, p = c & 1;
  if constexpr (KB == 4) return base + 2 * J + p;                  // nibble p of byte J
  else if constexpr (KB == 2) return base + 16 * ((J >> 2) >> 1) + 4 * (J & 3) + 2 * p + ((J >> 2) & 1);
  else return base + 16 * p + J;                                   // half p of the run
}
template <int KB>
__device__ __forceinline__ i32x4_t key_bytes(const KeyRun<KB>& r, int p) {
  u32x4_t b;
  if constexpr (KB == 4) {                           // byte J = 4j + b of word j: nibble p of its byte b
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = (r.w(j) >> (4 * p)) & 0x0F0F0F0Fu;
  } else if constexpr (KB == 2) {                    // word 2m + t: fields 2p + t of the bytes of word m
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = (r.w(i >> 1) >> (2 * (2 * p + (i & 1)))) & 0x03030303u;
  } else {                                           // one field per byte, dims 16p .. 16p + 15
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 16 * p + 4 * i;
      const uint32_t lo = key_field<KB>(r, KB * d0) | (key_field<KB>(r, KB * (d0 + 1)) << 8);
      const uint32_t hi = key_field<KB>(r, KB * (d0 + 2)) | (key_field<KB>(r, KB * (d0 + 3)) << 8);
      b[i] = lo | (hi << 16);
    }
  }
  return __builtin_bit_cast(i32x4_t, b);
}

// x + (x of the lanes 4, 8 and 12 places along in the same row of 16): sums the
// four digit columns of one query head.
__device__ __forceinline__ float add_digit_cols(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true));
  return x + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124, 0xF, 0xF, true));
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
template <int NKS, int NVS, int VB, int KB, bool APP = false, bool LL = false>
__global__ __launch_bounds__(kFastBlock, 1) void k_decode_mfma(FArgs a) {
  constexpr int NW = kFastBlock / 64;                // wavefronts per block
  __shared__ __align__(16) float qs[4][kFastD + 16];
  __shared__ int qoff_s[4][4][2];                   // [head][digit][key group] sums of the query digits
  __shared__ float qinv_s[4];                        // [head] 1 / (the head's query scale)
  __shared__ float so[NW][4][kFastD];               // per-wave outputs [wave][head][dim]
  __shared__ float sm[NW][4], sl[NW][4];            // per-wave reference max (log2 units) and sum
  __shared__ i32x4_t qbs[4][4][16];                  // MFMA B operands [chunk][lane group][4 digit + head]
  __shared__ int next_local;                         // next step index of the block not yet handed out
  __shared__ int slot_chunk[kMaxSlots];              // chunk of each slot of C local indices (-1 = not yet known)
  const long long unit = blockIdx.y;                 // (b*L + l)*H + h
  const int h = (int)(unit % a.H);
  const long long bl = unit / a.H;                   // b*L + l
  const int l = (int)(bl % a.L);
  const long long rq = bl * a.n_q + blockIdx.z;      // blockIdx.z: query index
  const size_t urow0 = (size_t)unit * a.T;
  const float* const kchu = a.kchan ? a.kchan + ((size_t)l * a.H + h) * kFastD : nullptr;
  const float* const kmeanu = a.kmean ? a.kmean + ((size_t)l * a.H + h) * kFastD : nullptr;
#include "kvq_mfma_body.inc"
}

// ------------------------------------------------------------------ codec maps in one launch
//
// A cache tiled into (layer range x KV-head range) tiles over every token, each with its
// own key and value bit widths at group 128 (per-head key bits, [LCPP] Finding 2; a
// per-layer allocation, [E21W] Result): one launch decodes all of it.  Each block finds
// the tile of its (layer, KV head), takes that tile's arrays, rotations and value grid,
// and runs the decode compiled for the tile's (key bits, value bits).  Counters, partials,
// queries, lengths and outputs are indexed over the whole map, so the in-kernel merge
// writes the final rows.  The pairs compiled in (id, key bits, value bits):
#define KVQ_MFMA_MIX_PAIRS(X) \
  X(0, 3, 2) X(1, 4, 2) X(2, 5, 2) X(3, 3, 4) X(4, 4, 4) X(5, 5, 4) X(6, 2, 2) X(7, 2, 4)

struct MfmaTile {
  const uint8_t* kc;
  const uint16_t* ks;
  const uint8_t* vc;
  const uint16_t* vs;
  const float* kchan;              // [ls][hs][256] or null
  const float* kmean;              // [ls][hs][256] or null
  int l0, ls, h0, hs;              // layers [l0, l0 + ls) x KV heads [h0, h0 + hs)
  int kW, vW;
  float kkappa, vkappa, voff;
  int pair;                        // index into KVQ_MFMA_MIX_PAIRS
};

struct FMixArgs {
  FArgs base;                      // the whole map's geometry, counters, partials and outputs
  int ntiles;
  MfmaTile tile[kMaxSegments];
};

struct MfmaLds {                   // the LDS of one block (as k_decode_mfma declares it)
  alignas(16) float qs[4][kFastD + 16];
  int qoff_s[4][4][2];
  float qinv_s[4];
  float so[kFastBlock / 64][4][kFastD];
  float sm[kFastBlock / 64][4], sl[kFastBlock / 64][4];
  i32x4_t qbs[4][4][16];
  int next_local;
  int slot_chunk[kMaxSlots];
};

template <int VB, int KB>
__device__ __forceinline__ void mfma_tile_unit(const FArgs& a, MfmaLds& S, int h, long long rq, size_t urow0,
                                               const float* kchu, const float* kmeanu) {
  constexpr int NKS = 2, NVS = 2;                    // key and value group 128
  constexpr int NW = kFastBlock / 64;
  auto& qs = S.qs;
  auto& qoff_s = S.qoff_s;
  auto& qinv_s = S.qinv_s;
  auto& so = S.so;
  auto& sm = S.sm;
  auto& sl = S.sl;
  auto& qbs = S.qbs;
  int& next_local = S.next_local;
  auto& slot_chunk = S.slot_chunk;
  constexpr bool APP = false;
  constexpr bool LL = false;
#include "kvq_mfma_body.inc"
}

__global__ __launch_bounds__(kFastBlock, 1) void k_decode_mfma_mix(FMixArgs m) {
  __shared__ MfmaLds S;
  const FArgs& g = m.base;
  const long long unit = blockIdx.y;                 // (b*L + l)*H + h over the whole map
  const int h = (int)(unit % g.H);
  const long long bl = unit / g.H;
  const int l = (int)(bl % g.L);
  const long long b = bl / g.L;
  const long long rq = bl * g.n_q + blockIdx.z;
  int ti = 0;                                        // the tiles cover every (layer, head) once
  while (ti + 1 < m.ntiles) {
    const MfmaTile& t = m.tile[ti];
    if (l >= t.l0 && l < t.l0 + t.ls && h >= t.h0 && h < t.h0 + t.hs) break;
    ++ti;
  }
  const MfmaTile& t = m.tile[ti];
  const int ll = l - t.l0, hl = h - t.h0;
  FArgs a = g;
  a.kc = t.kc;
  a.ks = t.ks;
  a.vc = t.vc;
  a.vs = t.vs;
  a.kchan = t.kchan;
  a.kW = t.kW;
  a.kkappa = t.kkappa;
  a.vW = t.vW;
  a.vkappa = t.vkappa;
  a.voff = t.voff;
  const size_t urow0 = (((size_t)b * t.ls + ll) * t.hs + hl) * g.T;
  const float* const kchu = t.kchan ? t.kchan + ((size_t)ll * t.hs + hl) * kFastD : nullptr;
  const float* const kmeanu = t.kmean ? t.kmean + ((size_t)ll * t.hs + hl) * kFastD : nullptr;
  switch (t.pair) {
#define KVQ_MFMA_MIX_CASE(id, KB, VB) \
  case id: mfma_tile_unit<VB, KB>(a, S, h, rq, urow0, kchu, kmeanu); break;
    KVQ_MFMA_MIX_PAIRS(KVQ_MFMA_MIX_CASE)
#undef KVQ_MFMA_MIX_CASE
    default: break;
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
  if (s.tokens < kStep) return false;              // a last step short of 32 rows reads the unit's last 32
  if (Hq / s.heads > 4) return false;
  if (k.codec.codebook != KVQ_INT_ABSMAX) return false;
  const int kb = k.codec.bits;
  // 6- and 8-bit keys need more registers than two wavefronts per SIMD leave (scratch spills)
  if (kb < 2 || kb > 5) return false;
  if (k.codec.group != 128 && k.codec.group != 256) return false;
  // 2- or 4-bit values: signed absmax (levels c - 2^(b-1)) or the symmetric grid (levels c - (2^b - 1)/2)
  // affine 2- to 4-bit value grids, and 2- or 3-bit Lloyd-Max levels (four- or eight-entry tables)
  if (v.codec.codebook == KVQ_LLOYD) {
    if (v.codec.bits != 2 && v.codec.bits != 3) return false;
  } else if (v.codec.codebook != KVQ_INT_ABSMAX && v.codec.codebook != KVQ_INT_SYM) {
    return false;
  }
  if (v.codec.bits < 2 || v.codec.bits > 4) return false;
  if (v.codec.group < 64) return false;   // a P.V block's 4 value words share one scale group
  if (v.chan_scale) return false;
  return true;
}

// Chunk size: at least 8 steps, and at most kMaxChunks chunks per (query row, KV head).
// The unit's blocks finish within about one chunk of each other (a 16-step chunk is ~4 us
// of one block's share of the bandwidth at the 64K workload; 8 steps halve that).
static int fast_chunk_log2(const kvq_shape& s) {
  const long long steps = (s.tokens + kStep - 1) / kStep;
  int cl2 = 3;
  while (((steps + (1LL << cl2) - 1) >> cl2) > kMaxChunks) ++cl2;
  return cl2;
}

static int fast_blocks_per_unit(const kvq_shape& s, int n_q) {
  const long long pairs = (long long)s.batch * s.layers * n_q * s.heads;
  // about one block (eight wavefronts, two per SIMD) per CU, and no more blocks than chunks
  long long bpu = (256 + pairs - 1) / pairs;
  const long long chunks = ((long long)((s.tokens + kStep - 1) / kStep) + (1LL << fast_chunk_log2(s)) - 1) >>
                           fast_chunk_log2(s);
  if (bpu > chunks) bpu = chunks;
  if (bpu < 1) bpu = 1;
  return (int)bpu;
}

size_t fast_part_bytes(const kvq_shape& s, int Hq, int n_q) {
  if (s.head_dim != kFastD || s.tokens < kStep) return 0;
  const int bpu = fast_blocks_per_unit(s, n_q);
  const size_t b = (size_t)s.batch * s.layers * n_q * Hq * bpu * (kFastD + 2) * sizeof(float);
  return (b + 255) / 256 * 256;
}

template <int VB, int KB>
static void launch_mfma(const FArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (VB == 2 || VB == 3) {
    if (a.vll) {                                     // 2- and 3-bit Lloyd-Max values
      if (a.nks == 2) {
        if (a.nvs == 1) k_decode_mfma<2, 1, VB, KB, false, true><<<grid, kFastBlock, 0, st>>>(a);
        else if (a.nvs == 2) k_decode_mfma<2, 2, VB, KB, false, true><<<grid, kFastBlock, 0, st>>>(a);
        else k_decode_mfma<2, 4, VB, KB, false, true><<<grid, kFastBlock, 0, st>>>(a);
      } else {
        if (a.nvs == 1) k_decode_mfma<1, 1, VB, KB, false, true><<<grid, kFastBlock, 0, st>>>(a);
        else if (a.nvs == 2) k_decode_mfma<1, 2, VB, KB, false, true><<<grid, kFastBlock, 0, st>>>(a);
        else k_decode_mfma<1, 4, VB, KB, false, true><<<grid, kFastBlock, 0, st>>>(a);
      }
      return;
    }
  }
  if constexpr (KB == 4 && VB != 3) {
    if (a.app_n > 0) {                               // the fused-append instances
      if (a.nks == 2) {
        if (a.nvs == 1) k_decode_mfma<2, 1, VB, 4, true><<<grid, kFastBlock, 0, st>>>(a);
        else if (a.nvs == 2) k_decode_mfma<2, 2, VB, 4, true><<<grid, kFastBlock, 0, st>>>(a);
        else k_decode_mfma<2, 4, VB, 4, true><<<grid, kFastBlock, 0, st>>>(a);
      } else {
        if (a.nvs == 1) k_decode_mfma<1, 1, VB, 4, true><<<grid, kFastBlock, 0, st>>>(a);
        else if (a.nvs == 2) k_decode_mfma<1, 2, VB, 4, true><<<grid, kFastBlock, 0, st>>>(a);
        else k_decode_mfma<1, 4, VB, 4, true><<<grid, kFastBlock, 0, st>>>(a);
      }
      return;
    }
  }
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
  else if (vb == 3) launch_mfma<3, KB>(a, grid, st);
  else launch_mfma<4, KB>(a, grid, st);
}

bool fused_append_supported(const kvq_packed& k, const kvq_packed& v, int Hq, int n_new) {
  if (!fast_decode_supported(k, v, Hq)) return false;
  if (n_new < 1 || n_new > kFusedAppendRows) return false;
  if (k.codec.codebook != KVQ_INT_ABSMAX || k.codec.bits != 4 || k.chan_scale || k.mean) return false;
  if (v.codec.codebook != KVQ_INT_ABSMAX || v.chan_scale || v.mean) return false;
  if (v.codec.bits != 2 && v.codec.bits != 4) return false;   // the row coder packs 2- and 4-bit codes
  auto rot_ok = [](int w) { return w <= 1 || w == 256; };
  return rot_ok(k.codec.rot_width) && rot_ok(v.codec.rot_width);
}

static float kappa_w(int W) {
  if (W <= 1) return 1.0f;
  int e = 0;
  while ((1 << e) < W) ++e;
  return (e % 2 == 0) ? ldexpf(1.0f, -e / 2) : (float)(1.0 / std::sqrt((double)W));
}

static int mfma_mix_pair(int kb, int vb) {
#define KVQ_MFMA_MIX_ID(id, KB, VB) \
  if (kb == KB && vb == VB) return id;
  KVQ_MFMA_MIX_PAIRS(KVQ_MFMA_MIX_ID)
#undef KVQ_MFMA_MIX_ID
  return -1;
}

bool mixed_fast_supported(const kvq_segment* segs, int n, int layers, int heads, int tokens, int Hq, int n_q) {
  if (n < 1 || n > kMaxSegments || Hq % heads != 0) return false;
  const int G = Hq / heads;
  const kvq_shape& s0 = segs[0].k->shape;
  if ((long long)s0.batch * layers * n_q * heads > kWsCounterRows) return false;   // the merge needs counters
  if ((long long)s0.batch * layers * heads > 65535 || n_q > 65535) return false;    // launch grid (y, z)
  for (int i = 0; i < n; ++i) {
    const kvq_packed& k = *segs[i].k;
    const kvq_packed& v = *segs[i].v;
    if (segs[i].token0 != 0 || k.shape.tokens != tokens) return false;
    if (!fast_decode_supported(k, v, k.shape.heads * G)) return false;
    if (k.codec.group != 128 || v.codec.group != 128) return false;
    if (v.codec.codebook == KVQ_LLOYD) return false;    // affine value grids only
    if (mfma_mix_pair(k.codec.bits, v.codec.bits) < 0) return false;
  }
  return true;
}

size_t mixed_fast_ws_bytes(const kvq_segment* segs, int layers, int heads, int tokens, int Hq, int n_q) {
  kvq_shape s = segs[0].k->shape;
  s.layers = layers;
  s.heads = heads;
  s.tokens = tokens;
  return fast_part_bytes(s, Hq, n_q);
}

hipError_t launch_decode_fast_mixed(const kvq_segment* segs, int n, int layers, int heads, int tokens, int Hq,
                                    int n_q, const uint16_t* q, const int32_t* kv_len, float sm, float* out,
                                    float* lse, int* ctr, void* part, hipStream_t st) {
  kvq_shape s = segs[0].k->shape;
  s.layers = layers;
  s.heads = heads;
  s.tokens = tokens;
  FMixArgs m{};
  FArgs& a = m.base;
  a.q = q;
  a.kv_len = kv_len;
  a.ws = static_cast<float*>(part);
  a.B = s.batch; a.L = layers; a.H = heads; a.T = tokens; a.Hq = Hq; a.G = Hq / heads;
  a.n_q = n_q;
  a.nks = 2;
  a.nvs = 2;
  a.gv = 128;
  a.sm_scale = sm;
  a.blocks_per_unit = fast_blocks_per_unit(s, n_q);
  a.chunk_log2 = fast_chunk_log2(s);
  a.ctr = ctr;
  a.done = ctr + kWsCounterRows;
  a.out = out;
  a.lse = lse;
  m.ntiles = n;
  for (int i = 0; i < n; ++i) {
    const kvq_packed& k = *segs[i].k;
    const kvq_packed& v = *segs[i].v;
    MfmaTile& t = m.tile[i];
    t.kc = reinterpret_cast<const uint8_t*>(k.codes);
    t.ks = k.scales;
    t.vc = reinterpret_cast<const uint8_t*>(v.codes);
    t.vs = v.scales;
    t.kchan = k.chan_scale;
    t.kmean = k.mean;
    t.l0 = segs[i].layer0; t.ls = k.shape.layers; t.h0 = segs[i].head0; t.hs = k.shape.heads;
    t.kW = k.codec.rot_width > 1 ? k.codec.rot_width : 0;
    t.kkappa = kappa_w(t.kW);
    t.vW = v.codec.rot_width > 1 ? v.codec.rot_width : 0;
    t.vkappa = kappa_w(t.vW);
    const int vb = v.codec.bits;
    t.voff = (v.codec.codebook == KVQ_INT_SYM) ? 0.5f * (float)((1 << vb) - 1) : (float)(1 << (vb - 1));
    t.pair = mfma_mix_pair(k.codec.bits, vb);
  }
  const long long units = (long long)s.batch * layers * heads;
  k_decode_mfma_mix<<<dim3(a.blocks_per_unit, (unsigned)units, (unsigned)n_q), kFastBlock, 0, st>>>(m);
  return hipGetLastError();
}

hipError_t launch_decode_fast(const AttnProblem& pr, hipStream_t st, bool* mean_done) {
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
  if (v.codec.codebook == KVQ_LLOYD) {               // levels rounded to fp16, as the matrix cores take them
    a.vll = 1;
    a.voff = 0.0f;
    a.vlut_lo = a.vlut_hi = a.vlut_lo2 = a.vlut_hi2 = 0;
    for (int c = 0; c < (1 << vb); ++c) {
      const uint16_t hb = __builtin_bit_cast(uint16_t, (_Float16)host_tables().lloyd_lv[vb - 2][c]);
      uint32_t& lo = c < 4 ? a.vlut_lo : a.vlut_lo2;
      uint32_t& hi = c < 4 ? a.vlut_hi : a.vlut_hi2;
      lo |= (uint32_t)(hb & 0xFFu) << (8 * (c & 3));
      hi |= (uint32_t)(hb >> 8) << (8 * (c & 3));
    }
  }
  a.blocks_per_unit = fast_blocks_per_unit(s, pr.n_q);
  a.chunk_log2 = fast_chunk_log2(s);
  // shared chunk counters when the rows fit the workspace's counter region
  const long long rows_kv = (long long)s.batch * s.layers * pr.n_q * s.heads;
  a.ctr = (pr.ctr && rows_kv <= kWsCounterRows) ? pr.ctr : nullptr;
  // unrotated values without channel scales: the last block of a unit merges its partials
  const bool fused = a.ctr && !v.chan_scale;
  a.done = fused ? pr.ctr + kWsCounterRows : nullptr;
  a.kmean = fused ? k.mean : nullptr;              // the in-kernel merge applies a key mean's lse shift
  if (mean_done) *mean_done = fused && k.mean;
  a.out = pr.out;
  a.lse = pr.lse;
  if (pr.app_n > 0) {
    a.app_k = pr.app_k;
    a.app_v = pr.app_v;
    a.app_t0 = pr.app_t0;
    a.app_n = pr.app_n;
    a.kcw = k.codes;
    a.ksw = k.scales;
    a.vcw = v.codes;
    a.vsw = v.scales;
    a.app_kg = k.codec.group;
    a.app_vg = v.codec.group;
  }
  const long long units = (long long)s.batch * s.layers * s.heads;
  const dim3 grid(a.blocks_per_unit, (unsigned)units, (unsigned)pr.n_q);
  switch (k.codec.bits) {
    case 2: launch_mfma_k<2>(a, vb, grid, st); break;
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

#ifdef KVQ_TIMELINE
#include "kvq_timeline.h"
extern "C" kvq_status kvq_timeline_read(unsigned long long* dst, size_t count) {
  const size_t n = (size_t)kvq::kTimelineBlocks * 8 * kvq::kTimelineSlots;
  if (!dst || count > n) return KVQ_ERR_ARG;
  if (hipMemcpyFromSymbol(dst, HIP_SYMBOL(kvq::g_kvq_timeline), count * sizeof(unsigned long long)) != hipSuccess)
    return KVQ_ERR_HIP;
  static unsigned long long zeros[kvq::kTimelineBlocks * 8 * kvq::kTimelineSlots];
  if (hipMemcpyToSymbol(HIP_SYMBOL(kvq::g_kvq_timeline), zeros, sizeof(zeros)) != hipSuccess) return KVQ_ERR_HIP;
  return KVQ_OK;
}
#endif

// MFMA decode attention at head_dim 128 over the extreme low-bit caches of [FMAG-6]
// ("Milestone" and "Best results": ternary {-s, 0, +s} and sign {-s, +s} codes at
// group 8, the int8 per-token row as reference, and the fp16 anchor layer), up to 4
// query heads per KV head.  The general kernel decodes these codecs on the VALU at
// about nine lane-operations per cached value; here both contractions run on the
// matrix cores and the VALU only turns codes into MFMA operands.
//
// One wavefront per (query row, KV head, token split), 32 tokens per step:
//  * Q.K^T on v_mfma_f32_16x16x32_f16, two 16-token tiles per step.  A = the keys
//    of 16 tokens x 32 dims as fp16: ternary and sign levels times their fp16 scale
//    are exact fp16 values (+-s or 0), so the keys are formed exactly; int8 codes
//    are fp16 subnormals (code c -> c * 2^-24, exact) and the row's single scale and
//    its offset 127 are applied to the logit (offset folded as 127 * sum q); fp16
//    keys are used as they are.  B = the fp16 query, 4 heads in columns n % 4 (the
//    query is fp16 already, so one part is exact).
//  * 6-bit signed absmax keys at group 32 (the Hadamard arm of the matched-rate
//    transform control, [FMAG-R] Colab-probe reply): MFMA g takes group g's 32 dims,
//    A = the codes as exact fp16 integers c - 32, and the group's scale multiplies
//    that MFMA's logits.  The query is rotated in the prologue when the keys are
//    (kappa * H q, an orthonormal identity), scaled per head by a power of two, and
//    split into an fp16 high part and remainder, which fill alternate groups of four
//    B columns; a row rotation by four lanes adds the two.
//  * rFFT keys with 6-bit real and imaginary parts at group 32 (the real/imaginary
//    arm): the logit is the weighted sum over bins of Re Q Re Z + Im Q Im Z (Parseval),
//    so the keys enter as for 6-bit keys, MFMA g taking real groups 0, 1 then
//    imaginary groups 0, 1; bin 64 (its own scale group) is added on the VALU.  The
//    weighted query spectrum comes from k_m128_qspec, run just before on the stream.
//  * rFFT polar keys (5-bit magnitude at group 32, 7-bit phase): each bin's code pair
//    indexes a 4096-entry LDS table of the fp16 high part and remainder of A cos and
//    A sin of its sector; per bin four k-slots (query real weight twice, imaginary
//    twice), so two MFMAs per 16 dims' worth of bins, and the group scale after.
//  * online softmax per head in log2 units, against a reference maximum that moves
//    only when a logit exceeds it by more than 1, so weights stay at most 2.
//  * P.V on v_mfma_f32_16x16x16_f16: A = fp16(p) for 4 heads (rows 0-3) x 16
//    tokens, B = 16 tokens x 16 value dims as fp16 (ternary and sign exact, fp16 as
//    stored); int8 values enter as subnormal codes with A = fp16(p) * s_v and the
//    offset folded as 127 * sum of A, as for keys.
// Each wavefront writes one (o, m, l) partial per query head (m in natural-log
// units); k_m128_combine merges a row's splits in order.
//
// Lane layouts (l = lane, i = l % 16, kq = l / 16):
//  * Q.K^T tile u: A row i is token 8(i / 4) + 4u + i % 4 of the step, so the
//    output rows 4kq + r of lane l are tokens 8kq + 4u + r: a lane's 8 logits are
//    the 8 consecutive tokens 8kq .. 8kq + 7.  A's 8 k-values of lane l are dims of
//    its k-block kq (dims 32kq .. 32kq + 31 over the four 32-wide chunks, ordered
//    per codec so that unpacking is cheap; the query B operand uses the same order).
//  * P.V: MFMA u takes tokens 8kq + 4u + r in k-slots 4kq + r, so lane l supplies
//    A = its own weights of tokens 8kq + 4u + r and B = the values of those tokens
//    for value dim 8i + c (chunk c = 0..7): each lane reads 8 consecutive dims of
//    its 8 tokens, one scale group of the group-8 codecs.
#include <algorithm>
#include <cmath>

#include "kvq_internal.hpp"

namespace kvq {

namespace {

typedef _Float16 mh8 __attribute__((ext_vector_type(8)));
typedef _Float16 mh4 __attribute__((ext_vector_type(4)));
typedef _Float16 mh2 __attribute__((ext_vector_type(2)));
typedef float mf4 __attribute__((ext_vector_type(4)));
typedef uint32_t mu4 __attribute__((ext_vector_type(4)));
typedef uint32_t mu2 __attribute__((ext_vector_type(2)));

constexpr int kMD = 128;              // head_dim
constexpr int kMStep = 32;            // tokens per wavefront step
constexpr int kMWaves = 4;            // independent wavefronts per block
constexpr int kMPart = kMD + 2;       // floats per partial: o[128], m, l

// MC_NF4: keys only (NF4 at group 64); MC_I4: values only (4-bit signed absmax at group 64);
// MC_I6: keys only (6-bit signed absmax at group 32, unrotated or Hadamard-128 rotated);
// MC_RC: keys only (rFFT along head_dim, real and imaginary parts 6-bit at group 32);
// MC_RP: keys only (rFFT along head_dim, 5-bit magnitude at group 32 + 7-bit phase)
enum M128Codec { MC_TER = 0, MC_SIGN = 1, MC_INT8 = 2, MC_F16 = 3, MC_NF4 = 4, MC_I4 = 5, MC_I6 = 6, MC_RC = 7,
                 MC_RP = 8 };
constexpr int kQSpec = 132;           // floats per (query row, head) of a prepared query spectrum

struct M128Args {
  const uint8_t* kc;
  const uint16_t* ks;
  const uint8_t* vc;
  const uint16_t* vs;
  const uint16_t* q;                  // [rows][Hq][128] fp16
  const int32_t* kv_len;              // [rows] or null
  float* part;                        // [rows * Hq][S][130]
  int H, T, Hq, G, n_q, S, cs;        // cs: steps per split
  long long items;                    // rows * H * S
  float lsc;                          // softmax scale * log2(e)
  int krot;                           // 6-bit keys: 1 if rotated by the normalised Hadamard-128
  const float* qspec;                 // rFFT keys: [rows][Hq][kQSpec] weighted query spectra
  float dirc[128], dirs[128];         // polar rFFT keys: cos, sin of the 128 phase sectors (binary32)
  float nf4[16];                      // NF4 levels (binary32)
};

template <int C> struct Row {          // bytes of one row's codes, scales per row
  static constexpr int code = C == MC_TER ? 32 : C == MC_SIGN ? 16 : C == MC_INT8 ? 128 : C == MC_F16 ? 256
                              : C == MC_I6 ? 96 : (C == MC_RC || C == MC_RP) ? 100 : 64;
  static constexpr int scales = C == MC_TER || C == MC_SIGN ? 16 : C == MC_INT8 ? 1 : C == MC_F16 ? 0
                                : C == MC_I6 ? 4 : C == MC_RC ? 6 : C == MC_RP ? 3 : 2;
};

// ---- key data of one 16-token tile for lane (i, kq): token tok(i, u), dims 32kq .. 32kq + 31
template <int C> struct KTile;
template <> struct KTile<MC_TER> { mu2 c; mu2 s; };              // 64 code bits, groups 4kq .. 4kq + 3
template <> struct KTile<MC_SIGN> { uint32_t c; mu2 s; };        // 32 code bits, the same groups
template <> struct KTile<MC_INT8> { mu4 c0, c1; uint32_t s; };  // 32 code bytes; s: the scale of token 8kq + i % 8
template <> struct KTile<MC_F16> { mu4 c[4]; };                  // 32 fp16 values
template <> struct KTile<MC_NF4> { mu2 c[2]; uint32_t s; };  // 16 codes of each group (dims 64g + 16kq ..); s:
                                                             // the two scales of token 8kq + i % 8 (tile 0 only)
// 6-bit keys: c[g] = the dword-aligned 8 bytes holding the 48 code bits of dims
// 32g + 8kq .. + 7 (group g); s: the four group scales of token 8kq + i % 8 (tile 0 only)
template <> struct KTile<MC_I6> { mu2 c[4]; mu2 s; };
// rFFT Cartesian keys: c[0..1] = the windows of real bins 32g + 8kq .. + 7 (as for 6-bit
// keys), c[2..3] + x[0..1] = the dword-aligned 12 bytes holding imaginary bins
// 32g + 8kq .. + 7; for token 8kq + i % 8 (tile 0 only): s, s2 = its six scales (real
// groups 0-2, imaginary groups 0-2), n0, n1 = the words holding bin 64's real and
// imaginary codes
template <> struct KTile<MC_RC> { mu2 c[4]; uint32_t x[2]; mu2 s; uint32_t s2, n0, n1; };
// rFFT polar keys: m[g] = the dword-aligned 8 bytes holding the 40 magnitude bits of bins
// 32g + 8kq .. + 7, p[g] + px[g] = the 12 bytes holding their 56 phase bits; for token
// 8kq + i % 8 (tile 0 only): s01 = its scales of groups 0 and 1, s2 = group 2's (bin 64),
// n0, n1 = the words holding bin 64's magnitude and phase codes
template <> struct KTile<MC_RP> { mu2 m[2]; mu2 p[2]; uint32_t px[2]; uint32_t s01, s2, n0, n1; };

// ---- value data for lane (i, kq): dims 8i .. 8i + 7 of tokens 8kq .. 8kq + 7.  (Row
// scales of int8 tokens are loaded one per lane and shared by DPP broadcasts: eight
// adjacent 16-bit loads would be merged into one 16-byte load, which returned wrong data
// at the 2-byte alignment rows can have.)  Ternary
// and sign: one register per token pair for the codes (token 2j in the low half, 2j + 1
// in the high half) and one for the two scales, each filled by two 16-bit loads.
template <int C> struct VData;
template <> struct VData<MC_TER> { mh2 c[4], s[4]; };
template <> struct VData<MC_SIGN> { mh2 c[4], s[4]; };
template <> struct VData<MC_INT8> { mu2 c[8]; uint32_t s; };   // 8 code bytes per token; the scale of token 8kq + i % 8
template <> struct VData<MC_F16> { mu4 c[8]; };                  // 8 fp16 values per token
template <> struct VData<MC_I4> { uint32_t c[8]; uint32_t s; };  // 8 codes per token; the two scales of token 8kq + i % 8

template <int KC, int VC> struct MStep {
  KTile<KC> k[2];
  VData<VC> v;
};

__device__ __forceinline__ int tile_row(int i, int u) { return 8 * (i >> 2) + 4 * u + (i & 3); }

// Per-lane byte offsets of a step's loads relative to the step's first row in each array
// (a step's base address is wavefront-uniform: scalar base + 32-bit lane offset).
struct MOffsets {
  uint32_t kp[2];     // polar rFFT keys: phase codes of tile u
  uint32_t k[2];      // key codes of tile u
  uint32_t ks[2];     // key scales of tile u (ternary, sign); int8: first output token's scale
  uint32_t v;         // value codes of token 8kq, dims 8i ..
  uint32_t vs;        // value scale of token 8kq (group i, or the row's)
};

template <int KC, int VC>
__device__ __forceinline__ MOffsets m_offsets(int i, int kq) {
  MOffsets o;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t r = (uint32_t)tile_row(i, u);
    if constexpr (KC == MC_TER) { o.k[u] = r * 32 + 8 * kq; o.ks[u] = (r * 16 + 4 * kq) * 2; }
    else if constexpr (KC == MC_SIGN) { o.k[u] = r * 16 + 4 * kq; o.ks[u] = (r * 16 + 4 * kq) * 2; }
    else if constexpr (KC == MC_INT8) { o.k[u] = r * 128 + 32 * kq; o.ks[u] = (8 * kq + (i & 7)) * 2; }
    else if constexpr (KC == MC_F16) { o.k[u] = r * 256 + 64 * kq; o.ks[u] = 0; }
    else if constexpr (KC == MC_I6) { o.k[u] = r * 96 + ((6 * kq) & ~3u); o.ks[u] = (8 * kq + (i & 7)) * 8; }
    else if constexpr (KC == MC_RC) {              // ks[1]: code row of token 8kq + i % 8
      o.k[u] = r * 100 + ((6 * kq) & ~3u);
      o.ks[u] = u == 0 ? (8 * kq + (i & 7)) * 12 : (8 * kq + (i & 7)) * 100;
    } else if constexpr (KC == MC_RP) {
      // magnitudes of bins 8kq ..: bit 40kq, window at byte 4kq; phases: bit 325 + 56kq,
      // window at its dword
      o.k[u] = r * 100 + 4 * kq;
      o.kp[u] = r * 100 + ((325 + 56 * kq) >> 5) * 4;
      o.ks[u] = u == 0 ? (8 * kq + (i & 7)) * 6 : (8 * kq + (i & 7)) * 100;
    }
    else { o.k[u] = r * 64 + 8 * kq; o.ks[u] = (8 * kq + (i & 7)) * 4; }
  }
  const uint32_t t = 8 * kq;
  if constexpr (VC == MC_TER) { o.v = t * 32 + 2 * i; o.vs = (t * 16 + i) * 2; }
  else if constexpr (VC == MC_SIGN) { o.v = t * 16 + i; o.vs = (t * 16 + i) * 2; }
  else if constexpr (VC == MC_INT8) { o.v = t * 128 + 8 * i; o.vs = (t + (i & 7)) * 2; }
  else if constexpr (VC == MC_F16) { o.v = t * 256 + 16 * i; o.vs = 0; }
  else { o.v = t * 64 + 4 * i; o.vs = (t + (i & 7)) * 4; }
  asm volatile("" : "+v"(o.k[0]), "+v"(o.k[1]), "+v"(o.ks[0]), "+v"(o.ks[1]), "+v"(o.v), "+v"(o.vs));
  if constexpr (KC == MC_RP) asm volatile("" : "+v"(o.kp[0]), "+v"(o.kp[1]));
  return o;
}

// base: wavefront-uniform; off: the lane's offset; IMM: a constant the load instruction
// carries in its offset field (added in 64-bit, so it can be)
template <typename T, int IMM = 0>
__device__ __forceinline__ T ld(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const T*>(base + (size_t)off + IMM);
}

// Loads of the step whose first row (unit row base + first token) is rb: scalar bases
// plus the lane's 32-bit offsets (the offsets pass through an empty asm once, where they
// are made, so the compiler does not fold them into 64-bit per-lane pointers).
template <int J, int KC, int VC>
__device__ __forceinline__ void m_load_vpair(const uint8_t* vb, const uint8_t* vsb, const MOffsets& o, VData<VC>& v) {
  constexpr int R = Row<VC>::code;
  if constexpr (VC == MC_TER) {
    v.c[J][0] = ld<_Float16, R * (2 * J)>(vb, o.v);
    v.c[J][1] = ld<_Float16, R * (2 * J + 1)>(vb, o.v);
  } else if constexpr (VC == MC_SIGN) {                // a code byte, zero-extended into each half
    v.c[J] = __builtin_bit_cast(mh2, (uint32_t)ld<uint8_t, R * (2 * J)>(vb, o.v) |
                                         ((uint32_t)ld<uint8_t, R * (2 * J + 1)>(vb, o.v) << 16));
  } else if constexpr (VC == MC_INT8) {
    v.c[2 * J] = ld<mu2, R * (2 * J)>(vb, o.v);
    v.c[2 * J + 1] = ld<mu2, R * (2 * J + 1)>(vb, o.v);
    if constexpr (J == 0) v.s = ld<uint16_t>(vsb, o.vs);
  } else if constexpr (VC == MC_F16) {
    v.c[2 * J] = ld<mu4, R * (2 * J)>(vb, o.v);
    v.c[2 * J + 1] = ld<mu4, R * (2 * J + 1)>(vb, o.v);
  } else {
    v.c[2 * J] = ld<uint32_t, R * (2 * J)>(vb, o.v);
    v.c[2 * J + 1] = ld<uint32_t, R * (2 * J + 1)>(vb, o.v);
    if constexpr (J == 0) v.s = ld<uint32_t>(vsb, o.vs);
  }
  if constexpr (VC == MC_TER || VC == MC_SIGN) {
    v.s[J][0] = ld<_Float16, 32 * (2 * J)>(vsb, o.vs);
    v.s[J][1] = ld<_Float16, 32 * (2 * J + 1)>(vsb, o.vs);
  }
}

template <int KC, int VC>
__device__ __forceinline__ void m_load(const M128Args& a, size_t rb, const MOffsets& o, MStep<KC, VC>& d) {
  const uint8_t* kb = a.kc + rb * Row<KC>::code;
  const uint8_t* ksb = reinterpret_cast<const uint8_t*>(a.ks) + rb * 2 * Row<KC>::scales;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if constexpr (KC == MC_TER) {
      d.k[u].c = ld<mu2>(kb, o.k[u]);
      d.k[u].s = ld<mu2>(ksb, o.ks[u]);
    } else if constexpr (KC == MC_SIGN) {
      d.k[u].c = ld<uint32_t>(kb, o.k[u]);
      d.k[u].s = ld<mu2>(ksb, o.ks[u]);
    } else if constexpr (KC == MC_INT8) {
      d.k[u].c0 = ld<mu4>(kb, o.k[u]);
      d.k[u].c1 = ld<mu4, 16>(kb, o.k[u]);
      if (u == 0) d.k[0].s = ld<uint16_t>(ksb, o.ks[0]);
    } else if constexpr (KC == MC_RP) {
      // group 1 lies 32 bins on: 160 magnitude bits (20 bytes), 224 phase bits (28 bytes)
      d.k[u].m[0] = ld<mu2, 0>(kb, o.k[u]);
      d.k[u].m[1] = ld<mu2, 20>(kb, o.k[u]);
      d.k[u].p[0] = ld<mu2, 0>(kb, o.kp[u]);
      d.k[u].px[0] = ld<uint32_t, 8>(kb, o.kp[u]);
      d.k[u].p[1] = ld<mu2, 28>(kb, o.kp[u]);
      d.k[u].px[1] = ld<uint32_t, 36>(kb, o.kp[u]);
      if (u == 0) {                                   // scale rows are 6 bytes: 16-bit loads
        d.k[0].s01 = (uint32_t)ld<uint16_t>(ksb, o.ks[0]) | ((uint32_t)ld<uint16_t, 2>(ksb, o.ks[0]) << 16);
        d.k[0].s2 = ld<uint16_t, 4>(ksb, o.ks[0]);
        d.k[0].n0 = ld<uint32_t, 40>(kb, o.ks[1]);    // bits 320..351: bin 64 magnitude at 320
        d.k[0].n1 = ld<uint32_t, 96>(kb, o.ks[1]);    // bits 768..799: bin 64 phase at 773
      }
    } else if constexpr (KC == MC_RC) {
      // imaginary bin b starts at bit 390 + 6b: its window is the real one's plus 48 bytes
      d.k[u].c[0] = ld<mu2, 0>(kb, o.k[u]);
      d.k[u].c[1] = ld<mu2, 24>(kb, o.k[u]);
      d.k[u].c[2] = ld<mu2, 48>(kb, o.k[u]);
      d.k[u].x[0] = ld<uint32_t, 56>(kb, o.k[u]);
      d.k[u].c[3] = ld<mu2, 72>(kb, o.k[u]);
      d.k[u].x[1] = ld<uint32_t, 80>(kb, o.k[u]);
      if (u == 0) {
        d.k[0].s = ld<mu2>(ksb, o.ks[0]);
        d.k[0].s2 = ld<uint32_t, 8>(ksb, o.ks[0]);
        d.k[0].n0 = ld<uint32_t, 48>(kb, o.ks[1]);    // bits 384..415: bin 64 real at 384
        d.k[0].n1 = ld<uint32_t, 96>(kb, o.ks[1]);    // bits 768..799: bin 64 imaginary at 774
      }
    } else if constexpr (KC == MC_I6) {
      d.k[u].c[0] = ld<mu2, 0>(kb, o.k[u]);
      d.k[u].c[1] = ld<mu2, 24>(kb, o.k[u]);
      d.k[u].c[2] = ld<mu2, 48>(kb, o.k[u]);
      d.k[u].c[3] = ld<mu2, 72>(kb, o.k[u]);
      if (u == 0) d.k[0].s = ld<mu2>(ksb, o.ks[0]);
    } else if constexpr (KC == MC_F16) {
      d.k[u].c[0] = ld<mu4, 0>(kb, o.k[u]);
      d.k[u].c[1] = ld<mu4, 16>(kb, o.k[u]);
      d.k[u].c[2] = ld<mu4, 32>(kb, o.k[u]);
      d.k[u].c[3] = ld<mu4, 48>(kb, o.k[u]);
    } else {
      d.k[u].c[0] = ld<mu2, 0>(kb, o.k[u]);
      d.k[u].c[1] = ld<mu2, 32>(kb, o.k[u]);
      if (u == 0) d.k[0].s = ld<uint32_t>(ksb, o.ks[0]);
    }
  }
  const uint8_t* vb = a.vc + rb * Row<VC>::code;
  const uint8_t* vsb = reinterpret_cast<const uint8_t*>(a.vs) + rb * 2 * Row<VC>::scales;
  m_load_vpair<0, KC, VC>(vb, vsb, o, d.v);
  m_load_vpair<1, KC, VC>(vb, vsb, o, d.v);
  m_load_vpair<2, KC, VC>(vb, vsb, o, d.v);
  m_load_vpair<3, KC, VC>(vb, vsb, o, d.v);
}

// x of lane j of this lane's 16-lane row (DPP row broadcast; every lane of the row active)
template <int J>
__device__ __forceinline__ uint32_t m_bcast_c(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x150 + J, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t m_bcast(uint32_t x, int j) {   // j a constant after unrolling
  switch (j) {
    case 0: return m_bcast_c<0>(x);
    case 1: return m_bcast_c<1>(x);
    case 2: return m_bcast_c<2>(x);
    case 3: return m_bcast_c<3>(x);
    case 4: return m_bcast_c<4>(x);
    case 5: return m_bcast_c<5>(x);
    case 6: return m_bcast_c<6>(x);
    default: return m_bcast_c<7>(x);
  }
}

// (x & mask) | 0x64006400 as one v_and_or: the or-value is hidden from the compiler so
// that it stays in a register (a literal would split the pair into two instructions)
__device__ __forceinline__ uint32_t or6400(uint32_t x, uint32_t mask) {
  uint32_t m = 0x64006400u;
  asm("" : "+v"(m));
  return (x & mask) | m;
}

__device__ __forceinline__ uint32_t pk_unit_scale(uint32_t x, uint32_t s2) {
  // x: two ternary codes in the low bits of each half, or-ed with 0x6400 (the fp16
  // 1024 + c); (1024 + c) - 1025 = c - 1 exactly, times the scale pair: +-s or 0, exact
  const mh2 u = __builtin_bit_cast(mh2, x) - mh2{(_Float16)1025.0f, (_Float16)1025.0f};
  return __builtin_bit_cast(uint32_t, u * __builtin_bit_cast(mh2, s2));
}

// A operand of key chunk c (0..3) of a tile.  Ternary and sign: dword m of chunk c
// holds dims (p, p + 16) of the lane's 32, p = 4c + m; int8 and fp16: dims 8c .. 8c + 7
// in order.
template <int KC>
__device__ __forceinline__ mh8 key_operand(const KTile<KC>& t, int c) {
  mu4 r;
  if constexpr (KC == MC_TER) {
    // codes of dims p and p + 16 at bits 2p' and 16 + 2p' of z (p' = p mod 8)
    const uint32_t z = (c < 2) ? __builtin_amdgcn_perm(t.c.y, t.c.x, 0x05040100u)
                               : __builtin_amdgcn_perm(t.c.y, t.c.x, 0x07060302u);
    // scales of dims (p, p + 16): groups (p / 8, 2 + p / 8) of the lane's four
    const uint32_t s2 = (c < 2) ? __builtin_amdgcn_perm(t.s.y, t.s.x, 0x05040100u)
                                : __builtin_amdgcn_perm(t.s.y, t.s.x, 0x07060302u);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int sh = 2 * (4 * (c & 1) + m);
      r[m] = pk_unit_scale(or6400(z >> sh, 0x00030003u), s2);
    }
  } else if constexpr (KC == MC_SIGN) {
    const uint32_t s2 = (c < 2) ? __builtin_amdgcn_perm(t.s.y, t.s.x, 0x05040100u)
                                : __builtin_amdgcn_perm(t.s.y, t.s.x, 0x07060302u);
    const uint32_t neg = s2 ^ 0x80008000u;            // (-s_a, -s_b); code 1 flips the sign
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int p = 4 * c + m;                       // bits p and p + 16 -> 15 and 31
      r[m] = ((t.c << (15 - p)) & 0x80008000u) ^ neg;
    }
  } else if constexpr (KC == MC_INT8) {
    const uint32_t w0 = (c == 0) ? t.c0.x : (c == 1) ? t.c0.z : (c == 2) ? t.c1.x : t.c1.z;
    const uint32_t w1 = (c == 0) ? t.c0.y : (c == 1) ? t.c0.w : (c == 2) ? t.c1.y : t.c1.w;
    r[0] = __builtin_amdgcn_perm(0u, w0, 0x0C010C00u);   // bytes -> fp16 subnormals c * 2^-24
    r[1] = __builtin_amdgcn_perm(0u, w0, 0x0C030C02u);
    r[2] = __builtin_amdgcn_perm(0u, w1, 0x0C010C00u);
    r[3] = __builtin_amdgcn_perm(0u, w1, 0x0C030C02u);
  } else {
    r = t.c[c];
  }
  return __builtin_bit_cast(mh8, r);
}

// NF4 keys, MFMA c (0..7) of a tile: group c / 4, lane k-block kq, dims
// 64(c / 4) + 16kq + 4(c % 4) .. + 3; each dim fills two k-slots, its level's fp16 high
// part and fp16 remainder (22 significant bits together; the query operand repeats the
// dim's value in both), read per code byte (two dims) from a table in LDS.
__device__ __forceinline__ mh8 nf4_operand(const KTile<MC_NF4>& t, int c, const mu2* lut) {
  const uint32_t w = t.c[c >> 2][(c >> 1) & 1];      // the 8 codes of dims 64g + 16kq + 8((c / 2) % 2) ..
  const int sh = 16 * (c & 1);                       // its bytes for this MFMA's 4 dims
  const mu2 e0 = lut[(w >> sh) & 0xFFu], e1 = lut[(w >> (sh + 8)) & 0xFFu];
  return __builtin_bit_cast(mh8, mu4{e0.x, e0.y, e1.x, e1.y});
}

// 6-bit keys, MFMA g (group g): dims 32g + 8kq + e, e = 0..7 in order, as fp16 c - 32
// (exact).  The lane's 48 code bits start at bit sh (0 or 16) of its 8-byte window;
// dword m holds dims (2m, 2m + 1) in its halves: each half gets its code at bits 0-5
// (bit-field insert of two shifted copies), or-ed with 0x6400 (the fp16 1024 + c), and
// 1056 comes off both halves in one packed subtract.
__device__ __forceinline__ mh8 i6_codes(uint32_t lo, uint32_t hi) {
  const uint32_t hm = 0xFFFF0000u;
  uint32_t x[4];
  x[0] = ((lo << 10) & hm) | (lo & ~hm);                                                    // e0 (bit 0), e1 (6)
  x[1] = ((lo >> 2) & hm) | ((lo >> 12) & ~hm);                                             // e2 (12), e3 (18)
  x[2] = (__builtin_amdgcn_alignbit(hi, lo, 14) & hm) | (__builtin_amdgcn_alignbit(hi, lo, 24) & ~hm);   // e4 (24), e5 (30)
  x[3] = ((hi << 6) & hm) | ((hi >> 4) & ~hm);                                              // e6 (36), e7 (42)
  mu4 r;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const mh2 u = __builtin_bit_cast(mh2, or6400(x[m], 0x003F003Fu)) - mh2{(_Float16)1056.0f, (_Float16)1056.0f};
    r[m] = __builtin_bit_cast(uint32_t, u);
  }
  return __builtin_bit_cast(mh8, r);
}
__device__ __forceinline__ mh8 i6_operand(const KTile<MC_I6>& t, int g, int sh) {
  // code bits 0..31 and 32..47 of the lane's run
  return i6_codes(__builtin_amdgcn_alignbit(t.c[g].y, t.c[g].x, sh), t.c[g].y >> sh);
}
// rFFT Cartesian keys, MFMA g: real bins 32g + 8kq .. + 7 (g < 2), imaginary bins
// 32(g - 2) + 8kq .. + 7 (g >= 2), whose runs start at bit 6 or 22 of a 3-word window
__device__ __forceinline__ mh8 rc_operand(const KTile<MC_RC>& t, int g, int kq) {
  if (g < 2) {
    const int sh = (kq & 1) ? 16 : 0;
    return i6_codes(__builtin_amdgcn_alignbit(t.c[g].y, t.c[g].x, sh), t.c[g].y >> sh);
  }
  const int sh = (kq & 1) ? 22 : 6;
  return i6_codes(__builtin_amdgcn_alignbit(t.c[g].y, t.c[g].x, sh), __builtin_amdgcn_alignbit(t.x[g - 2], t.c[g].y, sh));
}

// nb bits at compile-time bit pos of the 64-bit (hi, lo)
template <int POS, int NB>
__device__ __forceinline__ uint32_t field64(uint32_t lo, uint32_t hi) {
  if constexpr (POS + NB <= 32) return __builtin_amdgcn_ubfe(lo, POS, NB);
  else if constexpr (POS >= 32) return __builtin_amdgcn_ubfe(hi, POS - 32, NB);
  else return __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(hi, lo, POS), 0, NB);
}
// rFFT polar keys, MFMA m: bins e0 = 2(m % 4), e0 + 1 of the lane's 8 in group m / 4; per
// bin four k-slots: fp16 high part and remainder of A cos(theta), then of A sin(theta),
// read from the block's table by (magnitude code | phase code << 5)
template <int M>
__device__ __forceinline__ mh8 rp_operand(const KTile<MC_RP>& t, int kq, const mu2* lut) {
  constexpr int g = M >> 2, e0 = 2 * (M & 3);
  const int shm = 8 * kq, shp = (325 + 56 * kq) & 31;
  const uint32_t ml = __builtin_amdgcn_alignbit(t.m[g].y, t.m[g].x, shm), mhw = t.m[g].y >> shm;
  const uint32_t pl = __builtin_amdgcn_alignbit(t.p[g].y, t.p[g].x, shp);
  const uint32_t ph = __builtin_amdgcn_alignbit(t.px[g], t.p[g].y, shp);
  const uint32_t i0 = field64<5 * e0, 5>(ml, mhw) | (field64<7 * e0, 7>(pl, ph) << 5);
  const uint32_t i1 = field64<5 * e0 + 5, 5>(ml, mhw) | (field64<7 * e0 + 7, 7>(pl, ph) << 5);
  const mu2 a0 = lut[i0], a1 = lut[i1];
  return __builtin_bit_cast(mh8, mu4{a0.x, a0.y, a1.x, a1.y});
}

// B operand of value chunk c (dim 8i + c) for tokens 4u .. 4u + 3 of the lane's 8.
// keep01 / keep23: all-ones halves for the tokens that count (partial steps).
template <int VC, bool MASK>
__device__ __forceinline__ mh4 value_operand(const VData<VC>& v, int u, int c, uint32_t keep01, uint32_t keep23) {
  mu2 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int pj = 2 * u + h;                        // token pair (4u + 2h, 4u + 2h + 1)
    uint32_t x;
    if constexpr (VC == MC_TER) {
      const uint32_t y = __builtin_bit_cast(uint32_t, v.c[pj]);
      x = pk_unit_scale(or6400(y >> (2 * c), 0x00030003u), __builtin_bit_cast(uint32_t, v.s[pj]));
    } else if constexpr (VC == MC_SIGN) {
      const uint32_t y = __builtin_bit_cast(uint32_t, v.c[pj]);
      x = ((y << (15 - c)) & 0x80008000u) ^ (__builtin_bit_cast(uint32_t, v.s[pj]) ^ 0x80008000u);
    } else if constexpr (VC == MC_INT8) {
      const uint32_t sel = (uint32_t)(c & 3) | (0x0Cu << 8) | ((uint32_t)(4 + (c & 3)) << 16) | (0x0Cu << 24);
      x = __builtin_amdgcn_perm(v.c[2 * pj + 1][c >> 2], v.c[2 * pj][c >> 2], sel);
    } else if constexpr (VC == MC_F16) {
      x = __builtin_amdgcn_perm(v.c[2 * pj + 1][c >> 1], v.c[2 * pj][c >> 1], (c & 1) ? 0x07060302u : 0x05040100u);
    } else {                                         // 4-bit codes as fp16 subnormals c * 2^-24
      const uint32_t y = __builtin_amdgcn_perm(v.c[2 * pj + 1], v.c[2 * pj], (c < 4) ? 0x05040100u : 0x07060302u);
      x = (y >> (4 * (c & 3))) & 0x000F000Fu;
    }
    if constexpr (MASK && VC != MC_INT8 && VC != MC_I4) x &= (h == 0) ? keep01 : keep23;
    r[h] = x;
  }
  return __builtin_bit_cast(mh4, r);
}

template <int KC, int VC>
__global__ __launch_bounds__(kMWaves * 64, ((KC <= MC_SIGN && VC <= MC_SIGN) || (KC == MC_NF4 && VC == MC_I4)) ? 3 : 2) void k_decode_m128(M128Args a) {
  const int lane = threadIdx.x & 63, i = lane & 15, kq = lane >> 4;
  // NF4 keys: the block's table of code bytes -> (high part, remainder) of two levels
  __shared__ mu2 nf4_lut[KC == MC_NF4 ? 256 : 1];
  // polar rFFT keys: the block's table of (magnitude A, phase sector k) -> fp16 high part
  // and remainder of RN32(A cos), then of RN32(A sin), at A | k << 5
  __shared__ mu2 rp_lut[KC == MC_RP ? 4096 : 1];
  if constexpr (KC == MC_RP) {
    for (int e = threadIdx.x; e < 4096; e += kMWaves * 64) {
      const float A = (float)(e & 31);
      const float vc = A * a.dirc[e >> 5], vs = A * a.dirs[e >> 5];
      const _Float16 hc = (_Float16)vc, hs = (_Float16)vs;
      const _Float16 lc = (_Float16)(vc - (float)hc), ls = (_Float16)(vs - (float)hs);
      rp_lut[e] = mu2{(uint32_t)__builtin_bit_cast(uint16_t, hc) | ((uint32_t)__builtin_bit_cast(uint16_t, lc) << 16),
                      (uint32_t)__builtin_bit_cast(uint16_t, hs) | ((uint32_t)__builtin_bit_cast(uint16_t, ls) << 16)};
    }
    __syncthreads();
  }
  if constexpr (KC == MC_NF4) {
    const int b = threadIdx.x;                       // 256 threads, one entry each
    const float l0 = a.nf4[b & 15], l1 = a.nf4[b >> 4];
    const _Float16 h0 = (_Float16)l0, h1 = (_Float16)l1;
    const _Float16 r0 = (_Float16)(l0 - (float)h0), r1 = (_Float16)(l1 - (float)h1);
    nf4_lut[b] = mu2{(uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, r0) << 16),
                     (uint32_t)__builtin_bit_cast(uint16_t, h1) | ((uint32_t)__builtin_bit_cast(uint16_t, r1) << 16)};
    __syncthreads();
  }
  // the wavefront index through readfirstlane: everything derived from it is known
  // to be wavefront-uniform (scalar registers, scalar address arithmetic)
  const long long item = (long long)blockIdx.x * kMWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (item >= a.items) return;                       // whole wavefront
  const int s = (int)(item % a.S);
  const long long x = item / a.S;
  const int h = (int)(x % a.H);
  const long long rq = x / a.H;                      // query row ((b * L + l) * n_q + query)
  const size_t urow = ((size_t)(rq / a.n_q) * a.H + h) * a.T;   // first row of the (b, l, h) unit
  const int hq = i & 3;                              // query head of this lane's column
  // ---- query operand (the fp16 query, exact) and, for int8 keys, the head's sum
  const bool head_ok = hq < a.G;
  const uint16_t* qrow = a.q + ((size_t)rq * a.Hq + (size_t)h * a.G + (head_ok ? hq : 0)) * kMD + 32 * kq;
  mu4 qw[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // NF4 keys: dims 64g + 16kq .. + 15 of group g = c / 2 (eight per load); otherwise the
    // lane's chunks are dims 32kq .. 32kq + 31
    // 6-bit keys: chunk c is dims 32c + 8kq .. + 7 (group c)
    const uint16_t* qp = (KC == MC_NF4) ? qrow - 32 * kq + 64 * (c >> 1) + 16 * kq + 8 * (c & 1)
                         : (KC == MC_I6) ? qrow - 32 * kq + 32 * c + 8 * kq : qrow + 8 * c;
    qw[c] = head_ok ? *reinterpret_cast<const mu4*>(qp) : mu4{0u, 0u, 0u, 0u};
  }
  mh8 bq[(KC == MC_NF4 || KC == MC_RP) ? 8 : 4];
  float qscale = 1.0f;                               // 6-bit / rFFT keys: the logit's factor of the head's query scaling
  float nyr = 0.0f, nyi = 0.0f;                      // rFFT keys: the scaled query weights of bin 64
  if constexpr (KC == MC_RP) {
    // the head's weighted query spectrum (k_m128_qspec): yr / yi = real / imaginary
    // weights of bins 32g + 8kq .. + 7; MFMA m's B column holds, for its bins e0 and
    // e0 + 1, (re, re, im, im) of each, matching the key operand's k-slots
    float yr[2][8], yi[2][8];
    const float* qsp = a.qspec + ((size_t)rq * a.Hq + (size_t)h * a.G + (head_ok ? hq : 0)) * kQSpec;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        const float4 v0 = *reinterpret_cast<const float4*>(qsp + 64 * part + 32 * g + 8 * kq);
        const float4 v1 = *reinterpret_cast<const float4*>(qsp + 64 * part + 32 * g + 8 * kq + 4);
        const float z[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) (part == 0 ? yr : yi)[g][e] = head_ok ? z[e] : 0.0f;
      }
    const float2 ny = *reinterpret_cast<const float2*>(qsp + 128);
    nyr = head_ok ? ny.x : 0.0f;
    nyi = head_ok ? ny.y : 0.0f;
    float amax = fmaxf(fabsf(nyr), fabsf(nyi));
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fmaxf(fabsf(yr[g][e]), fabsf(yi[g][e])));
    amax = max_rows(amax);
    int ex = 0;
    if (amax > 0.0f) (void)frexpf(amax, &ex);
    const int sc = min(max(14 - ex, -100), 100);
    qscale = ldexpf(1.0f, -sc);
    nyr = ldexpf(nyr, sc);
    nyi = ldexpf(nyi, sc);
    const int part = (i >> 2) & 1;                   // high part / remainder columns
    auto half = [&](float x) -> _Float16 {
      const float v = ldexpf(x, sc);
      const _Float16 hv = (_Float16)v;
      return part == 0 ? hv : (_Float16)(v - (float)hv);
    };
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int g = m >> 2, e0 = 2 * (m & 3);
      mh8 r;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const _Float16 re = half(yr[g][e0 + b]), im = half(yi[g][e0 + b]);
        r[4 * b] = re;
        r[4 * b + 1] = re;
        r[4 * b + 2] = im;
        r[4 * b + 3] = im;
      }
      bq[m] = r;
    }
  } else if constexpr (KC == MC_RC) {
    // the head's weighted query spectrum, prepared by k_m128_qspec: chunk c holds its
    // real (c < 2) or imaginary (c >= 2) weights of bins 32(c % 2) + 8kq .. + 7
    float y[4][8];
    const float* qsp = a.qspec + ((size_t)rq * a.Hq + (size_t)h * a.G + (head_ok ? hq : 0)) * kQSpec;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 v0 = *reinterpret_cast<const float4*>(qsp + 32 * c + 8 * kq);
      const float4 v1 = *reinterpret_cast<const float4*>(qsp + 32 * c + 8 * kq + 4);
      const float z[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) y[c][e] = head_ok ? z[e] : 0.0f;
    }
    const float2 ny = *reinterpret_cast<const float2*>(qsp + 128);
    nyr = head_ok ? ny.x : 0.0f;
    nyi = head_ok ? ny.y : 0.0f;
    float amax = fmaxf(fabsf(nyr), fabsf(nyi));
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[c][e]));
    amax = max_rows(amax);
    int ex = 0;
    if (amax > 0.0f) (void)frexpf(amax, &ex);
    const int sc = min(max(14 - ex, -100), 100);
    qscale = ldexpf(1.0f, -sc);
    nyr = ldexpf(nyr, sc);
    nyi = ldexpf(nyi, sc);
    const int part = (i >> 2) & 1;                   // as for 6-bit keys: high part / remainder columns
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      mh8 r;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = ldexpf(y[c][e], sc);
        const _Float16 hv = (_Float16)v;
        r[e] = part == 0 ? hv : (_Float16)(v - (float)hv);
      }
      bq[c] = r;
    }
  } else if constexpr (KC == MC_I6) {
    // q in the key coordinates: y = kappa * H q (Sylvester order, kappa = RN32(1/sqrt(128)))
    // when the keys are rotated.  Dim bits 0-2 and 5-6 are the lane's own (e and the
    // chunk), bits 3 and 4 are lane bits 4 and 5 (kq): those two stages pair lanes
    // through row swaps, the lane with the bit set taking (partner - own).
    float y[4][8];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) y[c][e] = h2f((uint16_t)(qw[c][e >> 1] >> (16 * (e & 1))));
    if (a.krot) {
#pragma unroll
      for (int st = 1; st < 8; st <<= 1)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (!(e & st)) {
              const float u = y[c][e], v = y[c][e + st];
              y[c][e] = u + v;
              y[c][e + st] = u - v;
            }
#pragma unroll
      for (int st = 1; st < 4; st <<= 1)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (!(c & st))
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float u = y[c][e], v = y[c + st][e];
              y[c][e] = u + v;
              y[c + st][e] = u - v;
            }
      const bool b16 = (lane & 16) != 0, b32 = (lane & 32) != 0;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t p0 = u_bits(y[c][e]), p1 = p0;
          swap_rows16(p0, p1);                       // p0: lane without bit 4, p1: lane with it
          float z = b16 ? f_bits(p0) - f_bits(p1) : f_bits(p0) + f_bits(p1);
          uint32_t r0 = u_bits(z), r1 = r0;
          swap_rows32(r0, r1);
          z = b32 ? f_bits(r0) - f_bits(r1) : f_bits(r0) + f_bits(r1);
          y[c][e] = z * 0x1.6a09e6p-4f;              // RN32(1/sqrt(128))
        }
    }
    // scale the head's query by a power of two so that its largest entry lies in
    // [2^13, 2^14): the fp16 operands cannot overflow, and the logit takes the factor back
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[c][e]));
    amax = max_rows(amax);
    int ex = 0;
    if (amax > 0.0f) (void)frexpf(amax, &ex);
    const int sc = min(max(14 - ex, -100), 100);
    qscale = ldexpf(1.0f, -sc);
    // columns i with (i / 4) even take the fp16 high part, odd the fp16 remainder: each
    // lane's partner four columns away (either way, mod 16) holds the other part
    const int part = (i >> 2) & 1;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      mh8 r;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = ldexpf(y[c][e], sc);
        const _Float16 hv = (_Float16)v;
        r[e] = part == 0 ? hv : (_Float16)(v - (float)hv);
      }
      bq[c] = r;
    }
  } else if constexpr (KC == MC_TER || KC == MC_SIGN) {
    // dword m of chunk c: dims (p, p + 16) of the lane's 32, p = 4c + m
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      mu4 r;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int p = 4 * c + m;
        const uint32_t lo = qw[p >> 3][(p & 7) >> 1], hi = qw[2 + (p >> 3)][(p & 7) >> 1];
        r[m] = __builtin_amdgcn_perm(hi, lo, (p & 1) ? 0x07060302u : 0x05040100u);
      }
      bq[c] = __builtin_bit_cast(mh8, r);
    }
  } else if constexpr (KC == MC_NF4) {
    // MFMA c: dims 64(c / 4) + 16kq + 4(c % 4) .. + 3, each twice (high part, remainder)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const mu4 src = qw[2 * (c >> 2) + ((c >> 1) & 1)];
      const uint32_t lo = src[2 * (c & 1)], hi = src[2 * (c & 1) + 1];
      bq[c] = __builtin_bit_cast(mh8, mu4{__builtin_amdgcn_perm(lo, lo, 0x01000100u), __builtin_amdgcn_perm(lo, lo, 0x03020302u),
                                          __builtin_amdgcn_perm(hi, hi, 0x01000100u), __builtin_amdgcn_perm(hi, hi, 0x03020302u)});
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) bq[c] = __builtin_bit_cast(mh8, qw[c]);
  }
  float koff = 0.0f;                                 // int8 keys: 127 * sum of the head's query
  if constexpr (KC == MC_INT8) {
    float qs = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const mh8 v = bq[c];
#pragma unroll
      for (int e = 0; e < 8; ++e) qs += (float)v[e];
    }
    koff = 127.0f * sum_rows(qs);
  }
  // ---- token range of this split: steps [k0, k1), tokens below t_hi
  int n = a.T;
  if (a.kv_len) n = min(max(a.kv_len[rq], 0), a.T);
  const int steps = (n + kMStep - 1) / kMStep;
  const int k0 = s * a.cs, k1 = min(k0 + a.cs, steps);
  const int t_hi = min(k1 * kMStep, n);
  // ---- state
  mf4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = mf4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_ref = -INFINITY;       // reference max (log2 units) of head hq
  float l_part = 0.0f;           // sum of p over this lane's tokens (head hq)
  float w_part = 0.0f;           // int8 values: sum of the fp16 weights fp16(p) * s_v (head hq)
  const float kscale = (KC == MC_INT8) ? a.lsc * 16777216.0f
                       : (KC == MC_I6 || KC == MC_RC || KC == MC_RP) ? a.lsc * qscale : a.lsc;

  // byte address for ds_bpermute of copy 0 of this lane's head in its row
  constexpr bool kDedup = KC != MC_RP;
  const int gsrc = 4 * ((lane & 0x30) | (i & 3));
  auto process = [&](const MStep<KC, VC>& d, int step) {
    const int t0 = step * kMStep;
    const int tb = min(t0, a.T - kMStep);            // first token of the rows loaded
    // ---- Q.K^T: tile u, output rows = tokens 8kq + 4u + r
    constexpr int NG = (KC == MC_I6 || KC == MC_RC) ? 4 : 2;
    mf4 cq[2][NG];                                   // [tile][key group] (group 1 for NF4, 1-3 for 6-bit keys)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int g = 0; g < NG; ++g) cq[u][g] = mf4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (KC == MC_RP) {
          // MFMAs 2c, 2c + 1: group c / 2
          const mh8 k0 = (c == 0) ? rp_operand<0>(d.k[u], kq, rp_lut) : (c == 1) ? rp_operand<2>(d.k[u], kq, rp_lut)
                         : (c == 2) ? rp_operand<4>(d.k[u], kq, rp_lut) : rp_operand<6>(d.k[u], kq, rp_lut);
          const mh8 k1 = (c == 0) ? rp_operand<1>(d.k[u], kq, rp_lut) : (c == 1) ? rp_operand<3>(d.k[u], kq, rp_lut)
                         : (c == 2) ? rp_operand<5>(d.k[u], kq, rp_lut) : rp_operand<7>(d.k[u], kq, rp_lut);
          cq[u][c >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, bq[2 * c], cq[u][c >> 1], 0, 0, 0);
          cq[u][c >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, bq[2 * c + 1], cq[u][c >> 1], 0, 0, 0);
        } else if constexpr (KC == MC_I6) {
          cq[u][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(i6_operand(d.k[u], c, (kq & 1) ? 16 : 0), bq[c], cq[u][c], 0, 0, 0);
        } else if constexpr (KC == MC_RC) {
          cq[u][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(rc_operand(d.k[u], c, kq), bq[c], cq[u][c], 0, 0, 0);
        } else if constexpr (KC == MC_NF4) {
#pragma unroll
          for (int cc = 2 * c; cc < 2 * c + 2; ++cc)
            cq[u][cc >> 2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(nf4_operand(d.k[u], cc, nf4_lut), bq[cc], cq[u][cc >> 2], 0, 0, 0);
        } else {
          cq[u][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(key_operand<KC>(d.k[u], c), bq[c], cq[u][0], 0, 0, 0);
        }
      }
    }
    float lg[8];
    float nre = 0.0f, nim = 0.0f;                    // rFFT keys: bin 64 of token 8kq + i % 8
    if constexpr (KC == MC_RP) {
      const mu2 e = rp_lut[(d.k[0].n0 & 31u) | (((d.k[0].n1 >> 5) & 127u) << 5)];
      const float s2 = h2f((uint16_t)d.k[0].s2);
      nre = s2 * ((float)__builtin_bit_cast(_Float16, (uint16_t)e.x) + (float)__builtin_bit_cast(_Float16, (uint16_t)(e.x >> 16)));
      nim = s2 * ((float)__builtin_bit_cast(_Float16, (uint16_t)e.y) + (float)__builtin_bit_cast(_Float16, (uint16_t)(e.y >> 16)));
    }
    if constexpr (KC == MC_RC) {
      const uint32_t s23 = d.k[0].s.y, s45 = d.k[0].s2;
      nre = (float)((int)(d.k[0].n0 & 63u) - 32) * h2f((uint16_t)s23);
      nim = (float)((int)((d.k[0].n1 >> 6) & 63u) - 32) * h2f((uint16_t)(s45 >> 16));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (KC == MC_INT8) {
          const float sk = h2f((uint16_t)m_bcast(d.k[0].s, 4 * u + r));   // token 8kq + 4u + r
          lg[4 * u + r] = sk * (cq[u][0][r] * kscale - koff * a.lsc);
        } else if constexpr (KC == MC_RP) {
          const int j = 4 * u + r;
          const uint32_t s01 = m_bcast(d.k[0].s01, j);
          float t = h2f((uint16_t)s01) * cq[u][0][r];
          t = __builtin_fmaf(h2f((uint16_t)(s01 >> 16)), cq[u][1][r], t);
          const float tr = f_bits((uint32_t)__builtin_amdgcn_mov_dpp((int)u_bits(t), 0x124, 0xF, 0xF, true));   // row_ror:4
          const float ny = __builtin_fmaf(nyr, f_bits(m_bcast(u_bits(nre), j)), nyi * f_bits(m_bcast(u_bits(nim), j)));
          lg[j] = (t + tr + ny) * kscale;
        } else if constexpr (KC == MC_RC) {
          // groups: real 0, 1 (s.x), imaginary 0 (s.y high), 1 (s2 low); bin 64 apart
          const int j = 4 * u + r;
          const uint32_t s01 = m_bcast(d.k[0].s.x, j), s23 = m_bcast(d.k[0].s.y, j), s45 = m_bcast(d.k[0].s2, j);
          float t = h2f((uint16_t)s01) * cq[u][0][r];
          t = __builtin_fmaf(h2f((uint16_t)(s01 >> 16)), cq[u][1][r], t);
          t = __builtin_fmaf(h2f((uint16_t)(s23 >> 16)), cq[u][2][r], t);
          t = __builtin_fmaf(h2f((uint16_t)s45), cq[u][3][r], t);
          const float tr = f_bits((uint32_t)__builtin_amdgcn_mov_dpp((int)u_bits(t), 0x124, 0xF, 0xF, true));   // row_ror:4
          const float ny = __builtin_fmaf(nyr, f_bits(m_bcast(u_bits(nre), j)), nyi * f_bits(m_bcast(u_bits(nim), j)));
          lg[j] = (t + tr + ny) * kscale;
        } else if constexpr (KC == MC_I6) {
          // its four group scales; then each column adds its partner's part (row
          // rotation by 4), so every lane holds the full logit of head i % 4
          const uint32_t s01 = m_bcast(d.k[0].s.x, 4 * u + r), s23 = m_bcast(d.k[0].s.y, 4 * u + r);
          float t = h2f((uint16_t)s01) * cq[u][0][r];
          t = __builtin_fmaf(h2f((uint16_t)(s01 >> 16)), cq[u][1][r], t);
          t = __builtin_fmaf(h2f((uint16_t)s23), cq[u][2][r], t);
          t = __builtin_fmaf(h2f((uint16_t)(s23 >> 16)), cq[u][3][r], t);
          const float tr = f_bits((uint32_t)__builtin_amdgcn_mov_dpp((int)u_bits(t), 0x124, 0xF, 0xF, true));   // row_ror:4
          lg[4 * u + r] = (t + tr) * kscale;
        } else if constexpr (KC == MC_NF4) {
          const uint32_t sw = m_bcast(d.k[0].s, 4 * u + r);                 // its two group scales
          lg[4 * u + r] = (h2f((uint16_t)sw) * cq[u][0][r] + h2f((uint16_t)(sw >> 16)) * cq[u][1][r]) * kscale;
        } else {
          lg[4 * u + r] = cq[u][0][r] * kscale;
        }
      }
    }
    const bool partial = (tb < t0) || (tb + kMStep > t_hi);   // wavefront-uniform
    uint32_t keep[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    if (partial) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = tb + 8 * kq + j;
        if (t < t0 || t >= t_hi) {
          lg[j] = -INFINITY;
          keep[j >> 1] &= (j & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
      }
    }
    // ---- online softmax.  Lanes with equal i % 4 hold the same head, and the four column
    // copies of a row (lanes i, i + 4, i + 8, i + 12) hold the same logits: each copy takes
    // one output row of each tile (row i / 4: token 8kq + 4u + i / 4), so the weights are
    // computed once.
    // (Polar rFFT keys keep the per-lane form: their registers have no room for the gather.)
    float lu[2];
    float mt;
    if constexpr (kDedup) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float x01 = (i & 4) ? lg[4 * u + 1] : lg[4 * u];
        const float x23 = (i & 4) ? lg[4 * u + 3] : lg[4 * u + 2];
        lu[u] = (i & 8) ? x23 : x01;
      }
      mt = fmaxf(lu[0], lu[1]);
      mt = fmaxf(mt, f_bits((uint32_t)__builtin_amdgcn_mov_dpp((int)u_bits(mt), 0x124, 0xF, 0xF, false)));   // row_ror:4
      mt = fmaxf(mt, f_bits((uint32_t)__builtin_amdgcn_mov_dpp((int)u_bits(mt), 0x128, 0xF, 0xF, false)));   // row_ror:8
    } else {
      mt = lg[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) mt = fmaxf(mt, lg[k]);
    }
    // (lane shuffles through the LDS crossbar here: this loop's VALU is the busy unit)
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool grow = mt > m_ref + 1.0f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mt : m_ref;
      const float alpha = grow ? ((m_ref == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_ref - m_new)) : 1.0f;
      m_ref = m_new;
      l_part *= alpha;
      w_part *= alpha;
      // accumulator component r belongs to head r (rows 0-3): take head r's factor from lane r
      const float a0 = __shfl(alpha, 0), a1 = __shfl(alpha, 1), a2 = __shfl(alpha, 2), a3 = __shfl(alpha, 3);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        acc[c][0] *= a0;
        acc[c][1] *= a1;
        acc[c][2] *= a2;
        acc[c][3] *= a3;
      }
    }
    // ---- P.V.  The lane's two weights (fp32 into l_part, its share of the head's sum),
    // then as fp16 to every lane of its head in this row: lane i gathers token r of each
    // tile from copy r (lane 4r + i % 4).
    mh2 pg[4];
    if constexpr (kDedup) {
      const float pu0 = __builtin_amdgcn_exp2f(lu[0] - m_ref), pu1 = __builtin_amdgcn_exp2f(lu[1] - m_ref);   // masked: 0
      l_part += pu0 + pu1;
      const int pp = (int)__builtin_bit_cast(uint32_t, mh2{(_Float16)pu0, (_Float16)pu1});
#pragma unroll
      for (int r = 0; r < 4; ++r) pg[r] = __builtin_bit_cast(mh2, __builtin_amdgcn_ds_bpermute(gsrc + 16 * r, pp));
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float q0 = __builtin_amdgcn_exp2f(lg[r] - m_ref), q1 = __builtin_amdgcn_exp2f(lg[4 + r] - m_ref);
        l_part += q0 + q1;
        pg[r] = mh2{(_Float16)q0, (_Float16)q1};
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      mh4 ap;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const _Float16 p = pg[r][u];                 // fp16 weight of token 8kq + 4u + r
        if constexpr (VC == MC_INT8 || VC == MC_I4) {
          // A = fp16(p) * the value scale; 4-bit values: rows 0-3 take group 0's scale (dims
          // 0-63), rows 4-7 group 1's.  A masked token may sit on a row nobody wrote yet: its
          // weight is 0, not 0 * scale.
          uint32_t sw = m_bcast(d.v.s, 4 * u + r);   // token 8kq + 4u + r
          if constexpr (VC == MC_I4) sw = (i & 4) ? (sw >> 16) : sw;
          _Float16 w = p * __builtin_bit_cast(_Float16, (uint16_t)sw);
          w = (p == (_Float16)0.0f) ? (_Float16)0.0f : w;
          w_part += (float)w;
          ap[r] = w;
        } else {
          ap[r] = p;
        }
      }
      // The B values of masked tokens must be 0, not NaN (their rows may hold anything):
      // ternary and sign take masked scales (a zero scale gives +-0 for any code), fp16
      // values are masked only in partial steps; int8 codes are always finite.
      if constexpr (VC == MC_TER || VC == MC_SIGN) {
        VData<VC> vm = d.v;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          vm.s[2 * u + h2] = __builtin_bit_cast(mh2, __builtin_bit_cast(uint32_t, d.v.s[2 * u + h2]) & keep[2 * u + h2]);
#pragma unroll
        for (int c = 0; c < 8; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(ap, value_operand<VC, false>(vm, u, c, 0u, 0u), acc[c], 0, 0, 0);
      } else if (VC == MC_F16 && partial) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(
              ap, value_operand<VC, true>(d.v, u, c, keep[2 * u], keep[2 * u + 1]), acc[c], 0, 0, 0);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(ap, value_operand<VC, false>(d.v, u, c, 0u, 0u), acc[c], 0, 0, 0);
      }
    }
  };

  // ---- steps k0 .. k1 - 1 with two steps of loads in flight (buffers refilled in place;
  // a third buffer measured no faster: the low-bit steps are bound by their VALU work)
  constexpr int NB = 2;
  MStep<KC, VC> b0, b1;
  const MOffsets mo = m_offsets<KC, VC>(i, kq);
  auto row_of = [&](int step) -> size_t {
    const int st = min(step, max(k1 - 1, 0));
    return urow + (size_t)min(st * kMStep, a.T - kMStep);
  };
  if (k0 < k1) {
    m_load<KC, VC>(a, row_of(k0), mo, b0);
    m_load<KC, VC>(a, row_of(k0 + 1), mo, b1);
    for (int k = k0; k < k1; k += NB) {
      process(b0, k);
      m_load<KC, VC>(a, row_of(k + NB), mo, b0);
      if (k + 1 >= k1) break;
      process(b1, k + 1);
      m_load<KC, VC>(a, row_of(k + NB + 1), mo, b1);
    }
  }
  // ---- the wavefront's partial per query head (l_part: over the rows, then the copies)
  l_part = sum_rows(l_part);
  if constexpr (kDedup) {
    l_part += f_bits((uint32_t)__builtin_amdgcn_mov_dpp((int)u_bits(l_part), 0x124, 0xF, 0xF, false));   // row_ror:4
    l_part += f_bits((uint32_t)__builtin_amdgcn_mov_dpp((int)u_bits(l_part), 0x128, 0xF, 0xF, false));   // row_ror:8
  }
  if constexpr (VC == MC_INT8 || VC == MC_I4) w_part = sum_rows(w_part);
  // lane r (< 4) holds head r's m and l; lanes 0-15 hold rows 0-3 (heads) of the outputs
  // the weight sum of output row 4kq + r (int8: rows 0-3; 4-bit values: rows 0-7)
  const float wp0 = __shfl(w_part, 4 * kq), wp1 = __shfl(w_part, 4 * kq + 1);
  const float wp2 = __shfl(w_part, 4 * kq + 2), wp3 = __shfl(w_part, 4 * kq + 3);
  // lanes holding outputs: rows 0-3 (heads) for every column; 4-bit values: rows 0-3 for
  // value dims 0-63 (columns 0-7), rows 4-7 for dims 64-127 (columns 8-15)
  const bool writer = (VC == MC_I4) ? (kq == (i >> 3)) : (kq == 0);
  if (writer) {
    const float wp[4] = {wp0, wp1, wp2, wp3};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r >= a.G) break;
      float* dst = a.part + (((size_t)rq * a.Hq + (size_t)h * a.G + r) * a.S + s) * kMPart;
      float o[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if constexpr (VC == MC_INT8) o[c] = acc[c][r] * 16777216.0f - 127.0f * wp[r];
        else if constexpr (VC == MC_I4) o[c] = acc[c][r] * 16777216.0f - 8.0f * wp[r];
        else o[c] = acc[c][r];
      }
      // a partial is 130 floats, so rows are 8-byte aligned: float2 stores
#pragma unroll
      for (int c = 0; c < 8; c += 2) *reinterpret_cast<float2*>(dst + 8 * i + c) = make_float2(o[c], o[c + 1]);
      if (kq == 0 && i == r) {
        dst[kMD] = (m_ref == -INFINITY) ? -INFINITY : m_ref * 0.69314718055994531f;
        dst[kMD + 1] = l_part;
      }
    }
  }
}

}  // namespace

}  // namespace kvq

namespace kvq {

namespace {

// Weighted query spectra for rFFT keys, one wavefront per (query row, query head):
// Q = DFT(q) (forward sign, Q_f = sum_n q_n e^{-2 pi i f n / 128}), and the logit of a
// key with spectrum Z is sum_f w_f (Re Q_f Re Z_f + Im Q_f Im Z_f) (Parseval for real
// rows), w = 1/128 at bins 0 and 64, 2/128 elsewhere.  Written as w Re Q of bins 0-63,
// w Im Q of bins 0-63, then bin 64's two, two zeros.
__global__ __launch_bounds__(64) void k_m128_qspec(const uint16_t* q, float* qs, FftTables tw) {
  __shared__ float x[kMD];
  __shared__ float2 w[kMD];                          // (cos, sin) of 2 pi m / 128
  const size_t p = blockIdx.x;
  const int t = threadIdx.x;
  x[t] = h2f(q[p * kMD + t]);
  x[t + 64] = h2f(q[p * kMD + 64 + t]);
  w[t] = make_float2(tw.tw_c[t], -tw.tw_s[t]);
  w[t + 64] = make_float2(-tw.tw_c[t], tw.tw_s[t]);
  __syncthreads();
  float* o = qs + p * kQSpec;
  for (int f = t; f <= 64; f += 64) {
    float sr = 0.0f, si = 0.0f;
#pragma unroll 8
    for (int n = 0; n < kMD; ++n) {
      const float2 cs = w[(f * n) & (kMD - 1)];
      sr = __builtin_fmaf(x[n], cs.x, sr);
      si = __builtin_fmaf(-x[n], cs.y, si);
    }
    const float wf = (f == 0 || f == 64) ? 1.0f / 128.0f : 2.0f / 128.0f;
    if (f < 64) {
      o[f] = sr * wf;
      o[64 + f] = si * wf;
    } else {
      o[128] = sr * wf;
      o[129] = si * wf;
      o[130] = 0.0f;
      o[131] = 0.0f;
    }
  }
}

// Merge of the splits' partials, one wavefront per (query row, query head): M = the
// largest split maximum, split weights e^(m_s - M), L = sum of l_s times them, out = the
// weighted sum of the splits' o over L (fp64, in split order), lse = M + ln L.  The
// values this kernel decodes are never rotated or channel-scaled and the keys carry no
// mean, so nothing else is applied.
constexpr int kMMaxSplits = 512;
__global__ __launch_bounds__(256) void k_m128_combine(const float* __restrict__ part, int S, long long rows_hq,
                                                      float* __restrict__ out, float* __restrict__ lse) {
  __shared__ double wsh[4][kMMaxSplits];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long rh = (long long)blockIdx.x * 4 + wave;
  if (rh >= rows_hq) return;                         // whole wavefront
  const float* src = part + (size_t)rh * S * kMPart;
  double* w = wsh[wave];
  double mx = -INFINITY;
  for (int s = lane; s < S; s += 64) mx = fmax(mx, (double)src[(size_t)s * kMPart + kMD]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
  double ls = 0.0;
  for (int s = lane; s < S; s += 64) {
    const double ms = (double)src[(size_t)s * kMPart + kMD];
    const double ww = (mx == -INFINITY || ms == -INFINITY) ? 0.0 : exp(ms - mx);
    w[s] = ww;
    ls += (double)src[(size_t)s * kMPart + kMD + 1] * ww;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
  wave_lds_sync();                                   // the weights in LDS, read by every lane
#pragma unroll
  for (int d0 = 0; d0 < kMD; d0 += 64) {
    const int d = d0 + lane;
    double acc = 0.0;
    int s = 0;
    for (; s + 8 <= S; s += 8) {                     // eight splits' loads in flight
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[(size_t)(s + u) * kMPart + d];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += (double)v[u] * w[s + u];
    }
    for (; s < S; ++s) acc += (double)src[(size_t)s * kMPart + d] * w[s];
    out[(size_t)rh * kMD + d] = ls > 0.0 ? (float)(acc / ls) : 0.0f;
  }
  if (lane == 0 && lse) lse[rh] = ls > 0.0 ? (float)(mx + log(ls)) : -INFINITY;
}

// The kernel's codec of a key (K) or value (V) codec, or -1.
int m128_codec(const kvq_codec& c, bool key) {
  // 6-bit signed absmax keys at group 32, unrotated or rotated over the whole row
  if (key && c.codebook == KVQ_INT_ABSMAX && c.bits == 6 && c.group == 32 && (c.rot_width <= 1 || c.rot_width == kMD))
    return MC_I6;
  // rFFT Cartesian keys with 6-bit parts at group 32
  if (key && c.codebook == KVQ_RFFT_CART && c.bits == 6 && c.group == 32) return MC_RC;
  // rFFT polar keys: 5-bit magnitudes at group 32, 7-bit phases (128 sectors)
  if (key && c.codebook == KVQ_RFFT_POLAR && c.bits == 5 && c.aux_bits == 7 && c.group == 32) return MC_RP;
  if (c.rot_width > 1) return -1;
  switch (c.codebook) {
    case KVQ_TERNARY: return c.group == 8 ? MC_TER : -1;
    case KVQ_SIGN: return c.group == 8 ? MC_SIGN : -1;
    case KVQ_INT8_SYM: return c.group == 128 ? MC_INT8 : -1;
    case KVQ_FP16: return MC_F16;
    case KVQ_NF4: return (key && c.group == 64) ? MC_NF4 : -1;
    case KVQ_INT_ABSMAX: return (!key && c.bits == 4 && c.group == 64) ? MC_I4 : -1;
    default: return -1;
  }
}

template <int KC>
hipError_t launch_m128_v(int vc, const M128Args& a, unsigned grid, hipStream_t st) {
  switch (vc) {
    case MC_TER: k_decode_m128<KC, MC_TER><<<grid, kMWaves * 64, 0, st>>>(a); break;
    case MC_SIGN: k_decode_m128<KC, MC_SIGN><<<grid, kMWaves * 64, 0, st>>>(a); break;
    case MC_INT8: k_decode_m128<KC, MC_INT8><<<grid, kMWaves * 64, 0, st>>>(a); break;
    case MC_I4: k_decode_m128<KC, MC_I4><<<grid, kMWaves * 64, 0, st>>>(a); break;
    default: k_decode_m128<KC, MC_F16><<<grid, kMWaves * 64, 0, st>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace

bool m128_decode_supported(const kvq_packed& k, const kvq_packed& v, int Hq) {
  const kvq_shape& s = k.shape;
  if (s.head_dim != kMD || s.tokens < kMStep || s.heads < 1 || Hq % s.heads != 0) return false;
  const int G = Hq / s.heads;
  if (G < 1 || G > 4) return false;
  if (k.chan_scale || k.mean || v.chan_scale || v.mean) return false;
  return m128_codec(k.codec, true) >= 0 && m128_codec(v.codec, false) >= 0;
}

hipError_t launch_decode_m128(const AttnProblem& pr, hipStream_t st) {
  const kvq_shape& s = pr.k->shape;
  M128Args a{};
  a.kc = reinterpret_cast<const uint8_t*>(pr.k->codes);
  a.ks = pr.k->scales;
  a.vc = reinterpret_cast<const uint8_t*>(pr.v->codes);
  a.vs = pr.v->scales;
  a.q = pr.q;
  a.kv_len = pr.kv_len;
  a.part = static_cast<float*>(pr.ws);
  a.H = s.heads;
  a.T = s.tokens;
  a.Hq = pr.Hq;
  a.G = pr.Hq / s.heads;
  a.n_q = pr.n_q;
  // splits as the workspace holds them, but at least 8 steps each (a wavefront's query
  // set-up and first loads are a fixed cost)
  const int nsteps = (s.tokens + kMStep - 1) / kMStep;
  a.S = std::max(1, std::min(decode_wave_split_count(s, pr.Hq, pr.n_q), nsteps / 8));
  const long long rows = (long long)s.batch * s.layers * pr.n_q;
  const int kcod = m128_codec(pr.k->codec, true);
  if ((kcod == MC_RC || kcod == MC_RP) && rows > 0) {
    // the query spectra follow the partials (16-byte aligned): at most as many splits
    // as leave room for them in the workspace
    const size_t per = pr.ws_bytes / ((size_t)rows * pr.Hq * sizeof(float));   // floats per (row, head)
    const long long fit = per >= (size_t)kQSpec + 4 ? (long long)(per - kQSpec - 4) / kMPart : 0;
    if (fit < 1) return hipErrorInvalidValue;
    a.S = (int)std::min<long long>(a.S, fit);
  }
  a.cs = (nsteps + a.S - 1) / a.S;
  a.items = rows * s.heads * a.S;
  a.lsc = pr.sm_scale * 1.4426950408889634f;
  a.krot = pr.k->codec.rot_width == kMD ? 1 : 0;
  if (a.items == 0) return hipSuccess;
  const size_t part_bytes = (size_t)rows * pr.Hq * a.S * kMPart * sizeof(float);
  if (part_bytes > pr.ws_bytes) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((a.items + kMWaves - 1) / kMWaves);
  hipError_t e;
  if (kcod == MC_RP) {
    PhaseTables pt;
    host_phase_tables(128, &pt);
    std::copy(pt.dir_c, pt.dir_c + 128, a.dirc);
    std::copy(pt.dir_s, pt.dir_s + 128, a.dirs);
  }
  if (kcod == MC_RC || kcod == MC_RP) {
    const size_t off = (part_bytes + 15) / 16 * 16;
    if (off + (size_t)rows * pr.Hq * kQSpec * sizeof(float) > pr.ws_bytes) return hipErrorInvalidValue;
    float* qs = reinterpret_cast<float*>(static_cast<char*>(pr.ws) + off);
    a.qspec = qs;
    FftTables tw;
    host_fft_tables(kMD, &tw);
    k_m128_qspec<<<(unsigned)(rows * pr.Hq), 64, 0, st>>>(pr.q, qs, tw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int vc = m128_codec(pr.v->codec, false);
  std::copy(host_tables().nf4_lv, host_tables().nf4_lv + 16, a.nf4);
  switch (kcod) {
    case MC_TER: e = launch_m128_v<MC_TER>(vc, a, grid, st); break;
    case MC_SIGN: e = launch_m128_v<MC_SIGN>(vc, a, grid, st); break;
    case MC_INT8: e = launch_m128_v<MC_INT8>(vc, a, grid, st); break;
    case MC_NF4: e = launch_m128_v<MC_NF4>(vc, a, grid, st); break;
    case MC_I6: e = launch_m128_v<MC_I6>(vc, a, grid, st); break;
    case MC_RC: e = launch_m128_v<MC_RC>(vc, a, grid, st); break;
    case MC_RP: e = launch_m128_v<MC_RP>(vc, a, grid, st); break;
    default: e = launch_m128_v<MC_F16>(vc, a, grid, st); break;
  }
  if (e != hipSuccess) return e;
  if (a.S > kMMaxSplits) return launch_combine_partials(pr, a.S, nullptr, st);
  const long long rows_hq = rows * pr.Hq;
  k_m128_combine<<<(unsigned)((rows_hq + 3) / 4), 256, 0, st>>>(a.part, a.S, rows_hq, pr.out, pr.lse);
  return hipGetLastError();
}

}  // namespace kvq

// Internal declarations shared by the libkvq translation units (not part of the ABI).
//
// Thread layout used by the row kernels ("layout 1"): a row of D values is
// owned by LPT = D/16 consecutive lanes of one wavefront, lane j holding the 16
// consecutive values [16j, 16j+16).  A 256-thread block therefore holds
// 256/LPT rows at a time.  "Layout 2" (used only inside the Walsh-Hadamard
// transform) has lane j holding values j + LPT*r, r = 0..15, so the transform
// stages with strides >= 16 run in registers; the two layouts are exchanged
// through a padded LDS tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kBlock = 256;      // threads per block for every kernel
constexpr int kMaxSegments = 16; // segments of one logical cache (kvq_decode_attn_segments)
constexpr int kVals = 16;        // values per lane in layout 1

// Constant tables passed by value in kernel arguments (no device globals).
struct Tables {
  float nf4_lv[16];
  float nf4_mid[16];             // 15 midpoints, [15] = +inf
  float lloyd_lv[3][16];         // Gaussian Lloyd-Max levels for 2, 3, 4 bits (ascending)
};

struct FftTables {               // for head_dim N <= 256 and up to 256 phase sectors
  float tw_c[128], tw_s[128];    // cos(2 pi k/N), -sin(2 pi k/N), k < N/2
};
struct PhaseTables {
  float dir_c[256], dir_s[256];  // cos/sin(2 pi k/P), k < P
  float bnd_c[32], bnd_s[32];    // first-octant boundaries (2j+1) pi / P, j < P/8
};

const Tables& host_tables();
void host_fft_tables(int N, FftTables* t);
void host_phase_tables(int P, PhaseTables* t);

// ------------------------------------------------------------------ device helpers
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// fp32 -> stored fp16 scale: saturate to +-65504, round to nearest even, -0 -> +0.
__device__ __forceinline__ uint16_t rn16(float x) {
  x = __builtin_fminf(__builtin_fmaxf(x, -65504.0f), 65504.0f);
  uint16_t b = __builtin_bit_cast(uint16_t, (_Float16)x);
  return (b & 0x7fffu) ? b : (uint16_t)0;
}

// Orders one wavefront's LDS accesses: every earlier LDS access of the wavefront has
// completed before any later one is issued, and the compiler moves no memory access
// across it.  Enough between lanes of one wavefront working on its own LDS region.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Correctly rounded binary32 square root.  (The hardware instruction alone is
// accurate to about one ulp; the builtin adds the exact residual checks.)
__device__ __forceinline__ float sqrt_rn(float x) { return __builtin_sqrtf(x); }

// Correctly rounded reciprocal of a stored scale; zero scale -> zero.  The hardware
// reciprocal is within one ulp; one Newton step with fused multiply-adds,
// y + y(1 - s y), then gives the correctly rounded binary32 1/s for every s with at
// most 11 significant bits (every fp16 value), from any start within two ulps: checked
// with exact rational arithmetic over all 1024 such significands (1/s stays a normal
// binary32 for every fp16 s, so the exponent plays no part).
__device__ __forceinline__ float inv_scale(uint16_t sb) {
  const float s = h2f(sb);
  const float y = __builtin_amdgcn_rcpf(s);
  const float r = __builtin_fmaf(y, __builtin_fmaf(-s, y, 1.0f), y);
  return s == 0.0f ? 0.0f : r;
}

// Maximum and minimum over aligned runs of `lpg` lanes (lpg a power of two, at most 16):
// pairs, pairs of pairs, then the two quads of each 8 lanes and the two halves of each
// 16 lanes exchange values through DPP lane permutations, one v_max/v_min per step
// (the compiler's own fmaxf would quiet the permuted operand first, two instructions
// more).  Each step reads only lanes of the same run, so a run whose lanes are all
// inactive disturbs no other.  The s_nop covers the wait states a DPP read needs after
// a VALU write of its operand or of EXEC.
#define KVQ_DPP_MAXMIN(CTRL)                                                     \
  asm("s_nop 4\n\tv_max_f32_dpp %0, %0, %0 " CTRL " row_mask:0xf bank_mask:0xf\n\t" \
      "v_min_f32_dpp %1, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf"             \
      : "+v"(mx), "+v"(mn))
#define KVQ_DPP_MAX(CTRL) \
  asm("s_nop 4\n\tv_max_f32_dpp %0, %0, %0 " CTRL " row_mask:0xf bank_mask:0xf" : "+v"(a))

__device__ __forceinline__ void run_maxmin(float& mx, float& mn, int lpg) {
  if (lpg >= 2) KVQ_DPP_MAXMIN("quad_perm:[1,0,3,2]");
  if (lpg >= 4) KVQ_DPP_MAXMIN("quad_perm:[2,3,0,1]");
  if (lpg >= 8) KVQ_DPP_MAXMIN("row_half_mirror");
  if (lpg >= 16) KVQ_DPP_MAXMIN("row_mirror");
}
__device__ __forceinline__ float run_max(float a, int lpg) {
  if (lpg >= 2) KVQ_DPP_MAX("quad_perm:[1,0,3,2]");
  if (lpg >= 4) KVQ_DPP_MAX("quad_perm:[2,3,0,1]");
  if (lpg >= 8) KVQ_DPP_MAX("row_half_mirror");
  if (lpg >= 16) KVQ_DPP_MAX("row_mirror");
  return a;
}
#undef KVQ_DPP_MAXMIN
#undef KVQ_DPP_MAX

__device__ __forceinline__ float xor_max(float v, int m) { return __builtin_fmaxf(v, __shfl_xor(v, m)); }
__device__ __forceinline__ float xor_min(float v, int m) { return __builtin_fminf(v, __shfl_xor(v, m)); }
__device__ __forceinline__ float xor_add(float v, int m) { return v + __shfl_xor(v, m); }

// Padded LDS index of value i of a row (one pad float per 16 values).
__device__ __forceinline__ int pidx(int i) { return i + (i >> 4); }

// Pack 16 codes of BITS bits into a little-endian bit string (2*BITS bytes).
template <int BITS>
__device__ __forceinline__ void pack16(const uint32_t c[16], uint32_t w[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k] = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int pos = i * BITS;
    const int wi = pos >> 5, sh = pos & 31;
    w[wi] |= c[i] << sh;
    if (sh + BITS > 32) w[wi + 1] |= c[i] >> (32 - sh);
  }
}

template <int BITS>
__device__ __forceinline__ void unpack16(const uint32_t w[8], uint32_t c[16]) {
  constexpr uint32_t mask = (BITS >= 32) ? 0xffffffffu : ((1u << BITS) - 1u);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int pos = i * BITS;
    const int wi = pos >> 5, sh = pos & 31;
    uint32_t v = w[wi] >> sh;
    if (sh + BITS > 32) v |= w[wi + 1] << (32 - sh);
    c[i] = v & mask;
  }
}

// Store / load a lane's 2*BITS-byte chunk at byte offset `off` of `base`.
// Offsets are multiples of 2*BITS bytes, so even BITS give 4-byte alignment.
template <int BITS>
__device__ __forceinline__ void store_chunk(uint8_t* base, size_t off, const uint32_t w[8]) {
  if constexpr (BITS == 8) {
    *reinterpret_cast<uint4*>(base + off) = make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (BITS == 16) {
    *reinterpret_cast<uint4*>(base + off) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(base + off + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  } else if constexpr (BITS == 4) {
    *reinterpret_cast<uint2*>(base + off) = make_uint2(w[0], w[1]);
  } else if constexpr ((BITS & 1) == 0) {
#pragma unroll
    for (int k = 0; k < BITS / 2; ++k) reinterpret_cast<uint32_t*>(base + off)[k] = w[k];
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(base + off);
#pragma unroll
    for (int k = 0; k < BITS; ++k) p[k] = (uint16_t)(w[k >> 1] >> ((k & 1) * 16));
  }
}

template <int BITS>
__device__ __forceinline__ void load_chunk(const uint8_t* base, size_t off, uint32_t w[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k] = 0u;
  if constexpr (BITS == 8) {
    uint4 t = *reinterpret_cast<const uint4*>(base + off);
    w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
  } else if constexpr (BITS == 16) {
    uint4 t = *reinterpret_cast<const uint4*>(base + off);
    uint4 u = *reinterpret_cast<const uint4*>(base + off + 16);
    w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    w[4] = u.x; w[5] = u.y; w[6] = u.z; w[7] = u.w;
  } else if constexpr (BITS == 4) {
    uint2 t = *reinterpret_cast<const uint2*>(base + off);
    w[0] = t.x; w[1] = t.y;
  } else if constexpr ((BITS & 1) == 0) {
#pragma unroll
    for (int k = 0; k < BITS / 2; ++k) w[k] = reinterpret_cast<const uint32_t*>(base + off)[k];
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base + off);
#pragma unroll
    for (int k = 0; k < BITS; ++k) w[k >> 1] |= (uint32_t)p[k] << ((k & 1) * 16);
  }
}

#endif  // device helpers

// ------------------------------------------------------------------ launchers
struct RowGeom {        // a [B][L][H][T][D] tensor seen as rows
  long long rows;
  int D, T, H, L;
};

hipError_t launch_quantize(const uint16_t* x, const kvq_packed& p, hipStream_t st);
hipError_t launch_quantize_tokens(const uint16_t* x, const kvq_packed& p, int t0, int n, hipStream_t st);
hipError_t launch_quantize_kv(const uint16_t* kx, const uint16_t* vx, const kvq_packed& kp, const kvq_packed& vp,
                              int t0, int n, hipStream_t st);
hipError_t launch_rfft_quantize_tokens(const uint16_t* x, const kvq_packed& p, int t0, int n, hipStream_t st);
hipError_t launch_dequant(const kvq_packed& p, float* xhat, hipStream_t st);
hipError_t launch_calibrate(const uint16_t* k, const kvq_shape& s, float* c, hipStream_t st);
hipError_t launch_key_mean(const uint16_t* k, const kvq_shape& s, float* mean, long long* ws, hipStream_t st);
hipError_t launch_rfft_quantize(const uint16_t* x, const kvq_packed& p, hipStream_t st);
hipError_t launch_rfft_dequant(const kvq_packed& p, float* xhat, hipStream_t st);
hipError_t launch_rfft_kverr(const uint16_t* x, const kvq_packed& p, double* part, int chunks, hipStream_t st);

struct AttnProblem {
  const kvq_packed* k;
  const kvq_packed* v;
  int Hq, n_q;
  const uint16_t* q;
  const int32_t* kv_len;
  float sm_scale;
  // decode outputs
  float* out;
  float* lse;
  // error outputs (attn_error only)
  const uint16_t* k16;
  const uint16_t* v16;
  float* kl;
  float* relerr;
  double* kv_err;
  float* renyi2;     // the further error outputs (attn_error_ex), each nullable
  float* js;
  float* logit_relerr;
  float* top1;
  void* ws;          // partials (the workspace past its counter region)
  size_t ws_bytes;
  int* ctr;          // the workspace's counter region (kWsCounterBytes, zero between calls)
  // fused append (MFMA decode only): fp16 K and V rows [B][L][H][app_n][D] coded into tokens
  // [app_t0, app_t0 + app_n) of k and v by the decode launch itself; app_n = 0: none
  const uint16_t* app_k;
  const uint16_t* app_v;
  int app_t0, app_n;
};

// The first bytes of every decode workspace hold two arrays of per-(query row,
// KV head) counters of the MFMA decode kernel, kWsCounterRows ints each: chunk
// claims, then finished blocks.  They are zero before the first call, and each
// call sets the ones it used back to zero.  Partials follow.
constexpr size_t kWsCounterBytes = 65536;
constexpr long long kWsCounterRows = (long long)(kWsCounterBytes / (2 * sizeof(int)));

size_t decode_ws_bytes(const kvq_shape& s, int Hq, int n_q);
size_t error_ws_bytes(const kvq_shape& s, int Hq, int n_q);
int decode_splits(const kvq_shape& s, int Hq, int n_q);
hipError_t launch_decode_generic(const AttnProblem& pr, hipStream_t st);
hipError_t launch_attn_error(const AttnProblem& pr, hipStream_t st);
hipError_t launch_lse_mean(const AttnProblem& pr, hipStream_t st);
// A codec map in one launch: segments that each cover every token of their (layer range
// x head range) tile, with codec pairs the mixed decode kernel compiles.  With
// mean_shift the combine adds each tile's key-mean shift to the lse (otherwise the
// caller does).
bool mixed_decode_supported(const kvq_segment* segs, int n, int layers, int heads, int tokens, int Hq, int n_q);
size_t mixed_ws_bytes(const kvq_segment* segs, int layers, int heads, int tokens, int Hq, int n_q);
hipError_t launch_decode_mixed(const kvq_segment* segs, int n, int layers, int heads, int tokens, int Hq, int n_q,
                               const uint16_t* q, const int32_t* kv_len, float sm, float* out, float* lse,
                               void* part, bool mean_shift, hipStream_t st);
// A codec map of MFMA tiles (3-5-bit keys, 2- or 4-bit values, groups of 128; a tile's
// key mean shifts its lse in the kernel's merge) in one launch of the MFMA kernel; ctr:
// the workspace's counter region.
bool mixed_fast_supported(const kvq_segment* segs, int n, int layers, int heads, int tokens, int Hq, int n_q);
size_t mixed_fast_ws_bytes(const kvq_segment* segs, int layers, int heads, int tokens, int Hq, int n_q);
hipError_t launch_decode_fast_mixed(const kvq_segment* segs, int n, int layers, int heads, int tokens, int Hq,
                                    int n_q, const uint16_t* q, const int32_t* kv_len, float sm, float* out,
                                    float* lse, int* ctr, void* part, hipStream_t st);
hipError_t launch_seg_init(float* out, float* lse, long long rows, int D, hipStream_t st);
hipError_t launch_seg_prepare(const uint16_t* q, const int32_t* kvl, uint16_t* qs, int32_t* kvls, int B, int L,
                              int Ls, int l0, int n_q, int Hq, int j0, int hq, int D, int t0, int Ts, hipStream_t st);
hipError_t launch_seg_merge(int n, const int* l0, const int* ls, const int* j0, const int* hq, float* const* os,
                            float* const* lsp, float* out, float* lse, int B, int L, int n_q, int Hq, int D,
                            hipStream_t st);
bool fast_decode_supported(const kvq_packed& k, const kvq_packed& v, int Hq);
// The MFMA decode can code appended rows itself: 4-bit signed-absmax keys at group 128
// or 256 and 2- or 4-bit signed-absmax values (rotation 0 or 256, no channel scales or
// mean), at most kFusedAppendRows rows per (sequence, layer, head).
constexpr int kFusedAppendRows = 8;
bool fused_append_supported(const kvq_packed& k, const kvq_packed& v, int Hq, int n_new);
// mean_done (optional): set when the kernel's own merge applied the key mean's lse shift.
hipError_t launch_decode_fast(const AttnProblem& pr, hipStream_t st, bool* mean_done = nullptr);
size_t fast_part_bytes(const kvq_shape& s, int Hq, int n_q);
hipError_t launch_combine_partials(const AttnProblem& pr, int S, int* ctr, hipStream_t st);
// Splits per (query row, query head) that the decode workspace holds partials for with the
// wavefront-per-split kernels.
int decode_wave_split_count(const kvq_shape& s, int Hq, int n_q);
// MFMA decode at head_dim 128: ternary and sign codes at group 8, int8 rows, fp16 (keys
// and values in any combination of these, no rotation, channel scales or mean), up to 4
// query heads per KV head, at least 32 tokens.  Partials go to pr.ws, then the combine.
bool m128_decode_supported(const kvq_packed& k, const kvq_packed& v, int Hq);
hipError_t launch_decode_m128(const AttnProblem& pr, hipStream_t st);

// Row swaps: v_permlane32_swap exchanges the upper 32 lanes of a with the lower 32 of b,
// v_permlane16_swap the odd 16-lane rows of a with the even rows of b, in the VALU (a
// lane shuffle would go through the LDS crossbar).  Written as inline asm with both
// registers read-write: this compiler's builtins for them have returned the first
// result in place of the second (a standalone kernel added a result to itself).  The
// s_nop covers the wait states a VALU write needs before a permute reads it.
__device__ __forceinline__ float f_bits(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t u_bits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ void swap_rows32(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_rows16(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
// Sum / maximum of x over the four 16-lane rows (lanes l, l^16, l^32, l^48), in every lane.
__device__ __forceinline__ float sum_rows(float x) {
  uint32_t a = u_bits(x), b = a;
  swap_rows32(a, b);
  const float y = f_bits(a) + f_bits(b);             // x + x of lane l^32
  uint32_t c = u_bits(y), d = c;
  swap_rows16(c, d);
  return f_bits(c) + f_bits(d);                      // y + y of lane l^16
}
__device__ __forceinline__ float max_rows(float x) {
  uint32_t a = u_bits(x), b = a;
  swap_rows32(a, b);
  const float y = __builtin_fmaxf(f_bits(a), f_bits(b));
  uint32_t c = u_bits(y), d = c;
  swap_rows16(c, d);
  return __builtin_fmaxf(f_bits(c), f_bits(d));
}


}  // namespace kvq

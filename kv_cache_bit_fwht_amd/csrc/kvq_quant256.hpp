// The 256-wide signed-absmax row coder shared by the quantise kernels and the fused
// append + decode kernel: one row per 16 lanes, the same binary32 steps as the CPU
// oracle (codes and scales bit-identical to it).
#pragma once

#include "kvq_internal.hpp"

namespace kvq {

constexpr int kRowLds = 256 + 16;                    // LDS floats per row (padding spreads banks)

// ---- one row quad per wavefront (no mean, no channel scales)
// The same codes as absmax256_rows with fewer instructions and a launch shape that
// streams better: every wavefront codes one quad of rows and exits, so the rows in
// flight at any moment are a contiguous window of the tensor (measured 10-15% faster
// than a grid-stride loop over a resident grid), and the fp16 input is read with
// non-temporal loads (it is read once).  Arithmetic changes, all exact rewrites:
//  * the first butterfly stage (strides 1: the two halves of one input word) is one
//    v_fma_mix per output, a*1 + b and a*1 - b on the fp16 halves with a single
//    rounding, which is RN32(a + b) of the converted values;
//  * without a rotation the group extremes are taken on the fp16 values (packed
//    fp16 max/min; conversion to fp32 is exact and monotone), and each code's
//    product RN32(x * inv) is one v_fma_mix on the fp16 operand (x*inv + 0 rounds
//    once; only the sign of a zero product can differ, and the bias added next
//    removes it).
typedef _Float16 kvq_h2 __attribute__((ext_vector_type(2)));
typedef unsigned int kvq_u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load_row256_nt(const uint16_t* x, long long rows, long long row, int j, uint4& p0,
                                               uint4& p1) {
  if (row >= rows) row = rows - 1;                   // the tail quad re-reads the last row
  const kvq_u4* src = reinterpret_cast<const kvq_u4*>(x + (size_t)row * 256 + 16 * j);
  const kvq_u4 a0 = __builtin_nontemporal_load(src), a1 = __builtin_nontemporal_load(src + 1);
  p0 = make_uint4(a0.x, a0.y, a0.z, a0.w);
  p1 = make_uint4(a1.x, a1.y, a1.z, a1.w);
}

__device__ __forceinline__ float max16(const float v[16]) {
  const float a = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), v[2]);
  const float b = __builtin_fmaxf(__builtin_fmaxf(v[3], v[4]), v[5]);
  const float c = __builtin_fmaxf(__builtin_fmaxf(v[6], v[7]), v[8]);
  const float d = __builtin_fmaxf(__builtin_fmaxf(v[9], v[10]), v[11]);
  const float e = __builtin_fmaxf(__builtin_fmaxf(v[12], v[13]), v[14]);
  return __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(a, b), c), __builtin_fmaxf(__builtin_fmaxf(d, e), v[15]));
}

__device__ __forceinline__ float min16(const float v[16]) {
  const float a = __builtin_fminf(__builtin_fminf(v[0], v[1]), v[2]);
  const float b = __builtin_fminf(__builtin_fminf(v[3], v[4]), v[5]);
  const float c = __builtin_fminf(__builtin_fminf(v[6], v[7]), v[8]);
  const float d = __builtin_fminf(__builtin_fminf(v[9], v[10]), v[11]);
  const float e = __builtin_fminf(__builtin_fminf(v[12], v[13]), v[14]);
  return __builtin_fminf(__builtin_fminf(__builtin_fminf(a, b), c), __builtin_fminf(__builtin_fminf(d, e), v[15]));
}

// Codes and scales of one row (16 lanes, lane j holding values 16j..16j+15 as the
// raw fp16 words p0, p1) of a 256-wide tensor with `g` values per scale, stored at row
// `orow` of codes / scales when `store` (else computed only).  CB: the signed absmax
// grid, the symmetric grid (s = RN16(absmax / h), k = rne(RN32(t + h)), h = (2^b - 1)/2)
// or Gaussian Lloyd-Max levels (s = RN16(sqrt(RN32(S / g))) with S the adjacent-pairs
// tree sum of the squares; k = midpoints below t), with the same binary32 steps as the
// codec's general kernel and the CPU oracle.  rl: this row's LDS region (kRowLds
// floats; used with ROT).  COH: the stores are device-coherent (written through to
// memory), for rows another block may read in the same launch.  tab: the Lloyd-Max
// levels (LLOYD only).
template <int BITS, bool ROT, bool COH, int CB = KVQ_INT_ABSMAX>
__device__ __forceinline__ void code_row256(uint32_t* codes, uint16_t* scales, int g, long long orow, bool store,
                                            const uint4 p0, const uint4 p1, float* rl, int j,
                                            const Tables* tab = nullptr) {
#pragma clang fp contract(off)
  constexpr int D = 256;
  constexpr float kFold = ROT ? 0.0625f : 1.0f;      // the 256-point transform's 1/sqrt(256)
  constexpr float neg_step = -kFold / (float)(1 << (BITS - 1));
  constexpr uint32_t kMagic = 0x4B400000u;           // bit pattern of 1.5 * 2^23
  constexpr float kBias = 12582912.0f + (float)(1 << (BITS - 1));
  const int lpg = g >> 4;                            // lanes per group
  const uint32_t raw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
  float v[16];
  float mx, mn;
  if constexpr (!ROT) {
    kvq_h2 hx = __builtin_bit_cast(kvq_h2, raw[0]), hn = hx;
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      hx = __builtin_elementwise_max(hx, __builtin_bit_cast(kvq_h2, raw[k]));
      hn = __builtin_elementwise_min(hn, __builtin_bit_cast(kvq_h2, raw[k]));
    }
    mx = __builtin_fmaxf((float)hx.x, (float)hx.y);
    mn = __builtin_fminf((float)hn.x, (float)hn.y);
  } else {
    // stride 1 from the fp16 halves of each word, strides 2, 4, 8 in the lane
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(v[2 * k]) : "v"(raw[k]));
      asm("v_fma_mix_f32 %0, %1, 1.0, -%1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(v[2 * k + 1]) : "v"(raw[k]));
    }
#pragma unroll
    for (int s = 2; s < 16; s <<= 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!(i & s)) {
          const float x = v[i], y = v[i + s];
          v[i] = x + y;
          v[i + s] = x - y;
        }
    }
    // transpose (lane j takes values j + 16 r), strides 16..128, transpose back; quads of
    // a lane's values sit at quad index (q ^ (owner & 3)) of the owner's 16-float slot
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(rl + 16 * j + 4 * (q ^ (j & 3))) =
          make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = rl[16 * r + 4 * ((j >> 2) ^ (r & 3)) + (j & 3)];
#pragma unroll
    for (int rs = 1; rs < 16; rs <<= 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!(i & rs)) {
          const float x = v[i], y = v[i + rs];
          v[i] = x + y;
          v[i + rs] = x - y;
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) rl[16 * r + 4 * ((j >> 2) ^ (r & 3)) + (j & 3)] = v[r];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 t = *reinterpret_cast<const float4*>(rl + 16 * j + 4 * (q ^ (j & 3)));
      v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
    }
    mx = max16(v);
    mn = min16(v);
  }
  uint16_t s16;
  if constexpr (CB == KVQ_LLOYD) {
    // sum of squares: adjacent pairs of the lane's 16 values, then adjacent lanes
    float sq[16];
    if constexpr (!ROT) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float a = h2f((uint16_t)(raw[k] & 0xffffu)), b = h2f((uint16_t)(raw[k] >> 16));
        sq[2 * k] = __fmul_rn(a, a);
        sq[2 * k + 1] = __fmul_rn(b, b);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) sq[i] = __fmul_rn(v[i], v[i]);   // 256 times the rotated square, exactly
    }
#pragma unroll
    for (int w = 1; w < 16; w <<= 1) {
#pragma unroll
      for (int i = 0; i < 16; i += 2 * w) sq[i] = __fadd_rn(sq[i], sq[i + w]);
    }
    float S = sq[0];
    for (int m = 1; m < lpg; m <<= 1) S = __fadd_rn(S, __shfl_xor(S, m));
    if constexpr (ROT) S = S * (1.0f / 256.0f);      // exact: a power of two
    s16 = rn16(sqrt_rn(__fmul_rn(S, 1.0f / (float)g)));   // 1/g exact: g is a power of two
  } else {
    run_maxmin(mx, mn, lpg);
    if constexpr (CB == KVQ_INT_SYM) {
      constexpr float h = (float)((1 << BITS) - 1) * 0.5f;
      const float am = __builtin_fmaxf(mx, -mn) * kFold;   // exact: kFold is a power of two
      s16 = rn16(__fdiv_rn(am, h));
    } else {
      const float ext = (-mn >= mx) ? mn : mx;
      s16 = rn16(ext * neg_step);                    // exact product: neg_step is a power of two
    }
  }
  const float inv = inv_scale(s16) * kFold;          // exact: kFold is a power of two
  uint32_t c[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float t;
    if constexpr (!ROT) {
      if (i & 1) asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(t) : "v"(raw[i >> 1]), "v"(inv));
      else asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(t) : "v"(raw[i >> 1]), "v"(inv));
    } else {
      t = __fmul_rn(v[i], inv);
    }
    if constexpr (CB == KVQ_INT_SYM) {
      constexpr float h = (float)((1 << BITS) - 1) * 0.5f;
      c[i] = (uint32_t)(int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(__fadd_rn(t, h)), 0.0f),
                                           (float)((1 << BITS) - 1));
    } else if constexpr (CB == KVQ_LLOYD) {
      const float* L = tab->lloyd_lv[BITS - 2];
      uint32_t k = 0;
#pragma unroll
      for (int m = 0; m < (1 << BITS) - 1; ++m) k += (__fmul_rn(__fadd_rn(L[m], L[m + 1]), 0.5f) < t) ? 1u : 0u;
      c[i] = k;
    } else {
      const float f = __fadd_rn(t, kBias);
      const int b = (int)__builtin_bit_cast(uint32_t, f);
      c[i] = (uint32_t)min(max(b, (int)kMagic), (int)(kMagic + (1u << BITS) - 1u));
    }
  }
  if (!store) return;
  uint32_t w[4];
  if constexpr (BITS == 4) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t t0 = (c[8 * k + 1] << 4) | c[8 * k + 0], t1 = (c[8 * k + 3] << 4) | c[8 * k + 2];
      const uint32_t t2 = (c[8 * k + 5] << 4) | c[8 * k + 4], t3 = (c[8 * k + 7] << 4) | c[8 * k + 6];
      const uint32_t h0 = __builtin_amdgcn_perm(t1, t0, 0x0C0C0400u);
      const uint32_t h1 = __builtin_amdgcn_perm(t3, t2, 0x0C0C0400u);
      w[k] = (h1 << 16) | h0;
    }
  } else if constexpr (BITS == 2) {
    uint32_t by[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = (c[4 * k + 1] << 2) | c[4 * k + 0], hi = (c[4 * k + 3] << 2) | c[4 * k + 2];
      by[k] = (hi << 4) | lo;
    }
    const uint32_t h0 = __builtin_amdgcn_perm(by[1], by[0], 0x0C0C0400u);
    const uint32_t h1 = __builtin_amdgcn_perm(by[3], by[2], 0x0C0C0400u);
    w[0] = (h1 << 16) | h0;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t h0 = __builtin_amdgcn_perm(c[4 * k + 1], c[4 * k + 0], 0x0C0C0400u);
      const uint32_t h1 = __builtin_amdgcn_perm(c[4 * k + 3], c[4 * k + 2], 0x0C0C0400u);
      w[k] = (h1 << 16) | h0;
    }
  }
  constexpr int nw = BITS / 2;                       // code words of the lane's 16 values
  uint32_t* dst = codes + (size_t)orow * (D * BITS / 32) + (size_t)j * nw;
  const int lg = __builtin_ctz(g);                   // g is a power of two (it divides 256)
  uint16_t* sdst = scales + (size_t)orow * (D >> lg) + (j >> (lg - 4));
  const bool first = (j & (lpg - 1)) == 0;
  if constexpr (COH) {
#pragma unroll
    for (int k = 0; k < nw; ++k) __hip_atomic_store(dst + k, w[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (first) __hip_atomic_store(sdst, s16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    if constexpr (nw == 2) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    else if constexpr (nw == 1) *dst = w[0];
    else *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    if (first) *sdst = s16;
  }
}

}  // namespace kvq

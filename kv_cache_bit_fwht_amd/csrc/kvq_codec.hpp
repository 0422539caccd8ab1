// Codebook device functions shared by the quantise, dequantise and attention
// kernels: the Walsh-Hadamard transform over rows in layout 1, group
// statistics, and the per-lane encode/decode of 16 values.  Scalar rules follow
// the CPU oracle step for step (binary32, round-to-nearest-even, fp16 scales).
#pragma once

#include "kvq_internal.hpp"

namespace kvq {

// Value of lane (l ^ X) of this lane's 16-lane row, X = 1, 2, 4 or 8 (every lane of the
// row active): DPP moves for 1, 2 and 8 (folded into the add that uses them), a
// swizzle in xor mode for 4 (it runs on the LDS crossbar, not the VALU, where DPP would
// take two masked moves).
template <int X>
__device__ __forceinline__ float lane_xor(float v) {
  const int x = __builtin_bit_cast(int, v);
  int r;
  if constexpr (X == 1) r = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);         // quad_perm 1,0,3,2
  else if constexpr (X == 2) r = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);    // quad_perm 2,3,0,1
  else if constexpr (X == 8) r = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true);   // row_ror 8
  else r = __builtin_amdgcn_ds_swizzle(x, (4 << 10) | 0x1F);                           // and 31, xor 4
  return __builtin_bit_cast(float, r);
}

// One butterfly stage of stride 16 X across the LPT lanes of a row: the lane without bit
// X takes (own + partner), the one with it (partner - own), the same two binary32
// operations as a butterfly held in one lane.  partner - own is computed as
// partner + (-own), which is the same IEEE operation, so one add serves both lanes.
template <int X>
__device__ __forceinline__ void fwht_lane_stage(float v[16], int j) {
  const uint32_t sg = (j & X) ? 0x80000000u : 0u;
  if constexpr (X == 4) {                            // swizzles: all issued first, then the adds
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = lane_xor<X>(v[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = p[i] + __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v[i]) ^ sg);
  } else {                                           // DPP moves fold into the adds
#pragma unroll
    for (int i = 0; i < 16; ++i)
      v[i] = lane_xor<X>(v[i]) + __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v[i]) ^ sg);
  }
}

// Normalised Walsh-Hadamard transform of the rows held by this block (layout
// 1 in, layout 1 out).  Butterfly stages in ascending stride, each pair (i, i+s)
// -> (RN32(u_i + u_{i+s}), RN32(u_i - u_{i+s})), then RN32(u * kappa).  Strides
// below 16 are within a lane; strides 16 .. 128 pair lanes 1, 2, 4 and 8 apart within
// the row's lanes (j = the lane's index in its row; rows of D <= 256 fill at most one
// 16-lane row).  Every lane of the wavefront must call it.
__device__ __forceinline__ void fwht_rows(float v[16], int j, int W, float kappa) {
#pragma unroll
  for (int s = 1; s < 16; s <<= 1) {
    if (s < W) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (!(i & s)) {
          const float a = v[i], b = v[i + s];
          v[i] = a + b;
          v[i + s] = a - b;
        }
    }
  }
  if (W > 16) fwht_lane_stage<1>(v, j);
  if (W > 32) fwht_lane_stage<2>(v, j);
  if (W > 64) fwht_lane_stage<4>(v, j);
  if (W > 128) fwht_lane_stage<8>(v, j);
  if (W > 1) {
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = v[k] * kappa;
  }
}

// ------------------------------------------------------------------ group statistics
// Two groups per lane when g == 8 (halves of the 16 values), else one group
// spread over g/16 lanes (DPP reductions inside the row's lanes).

__device__ __forceinline__ void stat_maxmin(const float v[16], int g, float mx[2], float mn[2]) {
  float a0 = v[0], b0 = v[0], a1 = v[8], b1 = v[8];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    a0 = __builtin_fmaxf(a0, v[i]); b0 = __builtin_fminf(b0, v[i]);
    a1 = __builtin_fmaxf(a1, v[8 + i]); b1 = __builtin_fminf(b1, v[8 + i]);
  }
  if (g == 8) {
    mx[0] = a0; mn[0] = b0; mx[1] = a1; mn[1] = b1;
    return;
  }
  float a = __builtin_fmaxf(a0, a1), b = __builtin_fminf(b0, b1);
  run_maxmin(a, b, g / 16);
  mx[0] = mx[1] = a;
  mn[0] = mn[1] = b;
}

__device__ __forceinline__ void stat_absmax(const float v[16], int g, float am[2]) {
  float a0 = __builtin_fabsf(v[0]), a1 = __builtin_fabsf(v[8]);
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    a0 = __builtin_fmaxf(a0, __builtin_fabsf(v[i]));
    a1 = __builtin_fmaxf(a1, __builtin_fabsf(v[8 + i]));
  }
  if (g == 8) { am[0] = a0; am[1] = a1; return; }
  float a = __builtin_fmaxf(a0, a1);
  a = run_max(a, g / 16);
  am[0] = am[1] = a;
}

// Pairwise tree of |v| (adjacent pairs first), continued across lanes.
__device__ __forceinline__ void stat_abssum(const float v[16], int g, float sm[2]) {
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = __builtin_fabsf(v[i]);
#pragma unroll
  for (int w = 1; w < 8; w <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; i += 2 * w) t[i] = t[i] + t[i + w];
  }
  if (g == 8) { sm[0] = t[0]; sm[1] = t[8]; return; }
  float s = t[0] + t[8];
  for (int m = 1; m < g / 16; m <<= 1) s = xor_add(s, m);
  sm[0] = sm[1] = s;
}

// Group sums of squares RN32(y^2) with the same fixed pairwise tree as stat_abssum.
__device__ __forceinline__ void stat_sqsum(const float v[16], int g, float sm[2]) {
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = v[i] * v[i];
#pragma unroll
  for (int w = 1; w < 8; w <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; i += 2 * w) t[i] = t[i] + t[i + w];
  }
  if (g == 8) { sm[0] = t[0]; sm[1] = t[8]; return; }
  float s = t[0] + t[8];
  for (int m = 1; m < g / 16; m <<= 1) s = xor_add(s, m);
  sm[0] = sm[1] = s;
}

// ------------------------------------------------------------------ codebooks

// NF4 code lookup: cell i of [-1, 1) (width 1/128, index trunc((t + 1) * 128) clamped to
// 0..255) holds the number of midpoints below -1 + (i - 1)/128 and the one midpoint in
// [-1 + (i - 1)/128, -1 + (i + 2)/128), or +inf.  The index is off by at most one cell
// from t's (fp32 rounding near a cell edge), so t lies in that three-cell window, which
// holds at most one midpoint (they are 0.08 apart or more); outside [-1, 1) the clamped
// end cells are right as well (every midpoint lies in (-0.85, 0.87)).  The code is the
// count plus (midpoint < t): the number of midpoints strictly below t, as compared one
// by one.  One cell per thread of a 256-thread block.
__device__ __forceinline__ void nf4_cells_init(const Tables& tab, float2* cells, int i) {
  const float lo = -1.0f + (float)(i - 1) * (1.0f / 128.0f);   // exact: multiples of 2^-7
  const float hi = -1.0f + (float)(i + 2) * (1.0f / 128.0f);
  float cnt = 0.0f, cand = __builtin_inff();
#pragma unroll
  for (int m = 0; m < 15; ++m) {
    const float mid = tab.nf4_mid[m];
    if (mid < lo) cnt += 1.0f;
    else if (mid < hi) cand = mid;
  }
  cells[i] = make_float2(cnt, cand);
}

// rne(clamp(t, lo, hi)) + off as an unsigned code (lo, hi integers, |lo|, |hi| < 2^22,
// lo + off >= 0).  Clamping to integer bounds and then rounding is rounding and then
// clamping; the clamped value plus 1.5 * 2^23 is rounded to the nearest integer (ties to
// even: 1.5 * 2^23 is even), which then sits in the low mantissa bits of the sum, so
// one add and one integer subtract replace the round and the float-to-int conversion.
__device__ __forceinline__ uint32_t rne_code(float t, float lo, float hi, uint32_t off) {
  const float x = __builtin_fminf(__builtin_fmaxf(t, lo), hi) + 12582912.0f;
  return __builtin_bit_cast(uint32_t, x) - (0x4B400000u - off);
}

template <int CB, int BITS>
__device__ __forceinline__ void encode16(const float v[16], int g, const Tables& tab, uint32_t c[16],
                                         uint16_t s16[2], uint16_t z16[2], const float2* nf4_cells = nullptr) {
  if constexpr (CB == KVQ_INT_ABSMAX) {
    float mx[2], mn[2];
    stat_maxmin(v, g, mx, mn);
    constexpr float neg_step = -1.0f / (float)(1 << (BITS - 1));
    constexpr float lo = -(float)(1 << (BITS - 1)), hi = (float)((1 << (BITS - 1)) - 1);
    float inv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float m = (-mn[h] >= mx[h]) ? mn[h] : mx[h];
      s16[h] = rn16(m * neg_step);
      inv[h] = inv_scale(s16[h]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      c[i] = rne_code(v[i] * inv[i >> 3], lo, hi, 1u << (BITS - 1));
    }
  } else if constexpr (CB == KVQ_INT_MINMAX) {
    float mx[2], mn[2];
    stat_maxmin(v, g, mx, mn);
    constexpr float steps = (float)((1 << BITS) - 1);
    float inv[2], zf[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s16[h] = rn16(__fdiv_rn(mx[h] - mn[h], steps));
      z16[h] = rn16(mn[h]);
      inv[h] = inv_scale(s16[h]);
      zf[h] = h2f(z16[h]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float t = (v[i] - zf[i >> 3]) * inv[i >> 3];
      c[i] = rne_code(t, 0.0f, steps, 0u);
    }
  } else if constexpr (CB == KVQ_TERNARY || CB == KVQ_NF4 || CB == KVQ_INT8_SYM) {
    float am[2];
    stat_absmax(v, g, am);
    float inv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s16[h] = (CB == KVQ_INT8_SYM) ? rn16(__fdiv_rn(am[h], 127.0f)) : rn16(am[h]);
      inv[h] = inv_scale(s16[h]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float t = v[i] * inv[i >> 3];
      if constexpr (CB == KVQ_TERNARY) {
        c[i] = rne_code(t, -1.0f, 1.0f, 1u);
      } else if constexpr (CB == KVQ_INT8_SYM) {
        c[i] = rne_code(t, -127.0f, 127.0f, 127u);
      } else {
        // number of midpoints strictly below t, from the cell table in LDS
        const int ci = min(max((int)((t + 1.0f) * 128.0f), 0), 255);
        const float2 e = nf4_cells[ci];
        c[i] = (uint32_t)e.x + ((e.y < t) ? 1u : 0u);
      }
    }
  } else if constexpr (CB == KVQ_INT_SYM) {
    // symmetric grid: levels k - h, h = (2^b - 1)/2; s = absmax / h; k = rne(RN32(t + h))
    float am[2];
    stat_absmax(v, g, am);
    constexpr float h = (float)((1 << BITS) - 1) * 0.5f;
    constexpr float top = (float)((1 << BITS) - 1);
    float inv[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      s16[hh] = rn16(__fdiv_rn(am[hh], h));
      inv[hh] = inv_scale(s16[hh]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float t = v[i] * inv[i >> 3];
      c[i] = rne_code(t + h, 0.0f, top, 0u);
    }
  } else if constexpr (CB == KVQ_LLOYD) {
    // Gaussian Lloyd-Max levels L; s = RMS = sqrt(RN32(sum y^2 * 1/g)); code = number of
    // midpoints RN32(L_m + L_m+1) * 1/2 strictly below t (uniform table indices)
    float sq[2];
    stat_sqsum(v, g, sq);
    const float invg = 1.0f / (float)g;   // exact: g is a power of two
    float inv[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      s16[hh] = rn16(sqrt_rn(sq[hh] * invg));
      inv[hh] = inv_scale(s16[hh]);
    }
    const float* L = tab.lloyd_lv[BITS - 2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float t = v[i] * inv[i >> 3];
      uint32_t k = 0;
#pragma unroll
      for (int m = 0; m < (1 << BITS) - 1; ++m) k += (((L[m] + L[m + 1]) * 0.5f) < t) ? 1u : 0u;
      c[i] = k;
    }
  } else if constexpr (CB == KVQ_SIGN) {
    float sm[2];
    stat_abssum(v, g, sm);
    const float invg = 1.0f / (float)g;   // exact: g is a power of two
#pragma unroll
    for (int h = 0; h < 2; ++h) s16[h] = rn16(sm[h] * invg);
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = (v[i] >= 0.0f) ? 1u : 0u;
  }
}

template <int CB, int BITS>
__device__ __forceinline__ void decode16(const uint32_t c[16], const uint16_t s16[2], const uint16_t z16[2],
                                         const Tables& tab, float v[16]) {
  const float s0 = h2f(s16[0]), s1 = h2f(s16[1]);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float s = (i < 8) ? s0 : s1;
    if constexpr (CB == KVQ_INT_ABSMAX) {
      v[i] = (float)((int)c[i] - (1 << (BITS - 1))) * s;
    } else if constexpr (CB == KVQ_INT_MINMAX) {
      v[i] = (float)c[i] * s + h2f(z16[i >> 3]);
    } else if constexpr (CB == KVQ_TERNARY) {
      v[i] = (float)((int)c[i] - 1) * s;
    } else if constexpr (CB == KVQ_SIGN) {
      v[i] = c[i] ? s : -s;
    } else if constexpr (CB == KVQ_NF4) {
      v[i] = tab.nf4_lv[c[i] & 15u] * s;
    } else if constexpr (CB == KVQ_INT8_SYM) {
      v[i] = (float)((int)c[i] - 127) * s;
    } else if constexpr (CB == KVQ_INT_SYM) {
      v[i] = ((float)c[i] - (float)((1 << BITS) - 1) * 0.5f) * s;
    } else if constexpr (CB == KVQ_LLOYD) {
      v[i] = tab.lloyd_lv[BITS - 2][c[i] & 15u] * s;
    } else {
      v[i] = h2f((uint16_t)c[i]);
    }
  }
}

}  // namespace kvq

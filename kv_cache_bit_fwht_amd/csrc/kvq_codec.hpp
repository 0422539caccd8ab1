// Codebook device functions shared by the quantise, dequantise and attention
// kernels: the Walsh-Hadamard transform over rows in layout 1, group
// statistics, and the per-lane encode/decode of 16 values.  Scalar rules follow
// the CPU oracle step for step (binary32, round-to-nearest-even, fp16 scales).
#pragma once

#include "kvq_internal.hpp"

namespace kvq {

// Normalised Walsh-Hadamard transform of the rows held by this block (layout
// 1 in, layout 1 out).  Butterfly stages in ascending stride, each pair (i, i+s)
// -> (RN32(u_i + u_{i+s}), RN32(u_i - u_{i+s})), then RN32(u * kappa).
__device__ __forceinline__ void fwht_rows(float v[16], float* rowlds, int j, int LPT, int W,
                                          float kappa) {
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
  if (W > 16) {
#pragma unroll
    for (int k = 0; k < 16; ++k) rowlds[17 * j + k] = v[k];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = rowlds[pidx(j + LPT * r)];
#pragma unroll
    for (int rs = 1; rs < 16; rs <<= 1) {
      const int S = rs * LPT;             // stride in value index
      if (S >= 16 && S < W) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!(i & rs)) {
            const float a = v[i], b = v[i + rs];
            v[i] = a + b;
            v[i + rs] = a - b;
          }
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) rowlds[pidx(j + LPT * r)] = v[r];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = rowlds[17 * j + k];
    __syncthreads();
  }
  if (W > 1) {
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = v[k] * kappa;
  }
}

// ------------------------------------------------------------------ group statistics
// Two groups per lane when g == 8 (halves of the 16 values), else one group
// spread over g/16 lanes (xor-shuffle reductions inside the row's lanes).

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
  for (int m = 1; m < g / 16; m <<= 1) { a = xor_max(a, m); b = xor_min(b, m); }
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
  for (int m = 1; m < g / 16; m <<= 1) a = xor_max(a, m);
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

template <int CB, int BITS>
__device__ __forceinline__ void encode16(const float v[16], int g, const Tables& tab, uint32_t c[16],
                                         uint16_t s16[2], uint16_t z16[2]) {
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
      const float q = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(v[i] * inv[i >> 3]), lo), hi);
      c[i] = (uint32_t)((int)q + (1 << (BITS - 1)));
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
      const float q = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(t), 0.0f), steps);
      c[i] = (uint32_t)(int)q;
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
        c[i] = (uint32_t)((int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(t), -1.0f), 1.0f) + 1);
      } else if constexpr (CB == KVQ_INT8_SYM) {
        c[i] = (uint32_t)((int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(t), -127.0f), 127.0f) + 127);
      } else {
        // number of midpoints strictly below t (the 15 compares use uniform table
        // indices: a per-lane index into the argument table would be a memory read)
        uint32_t k = 0;
#pragma unroll
        for (int m = 0; m < 15; ++m) k += (tab.nf4_mid[m] < t) ? 1u : 0u;
        c[i] = k;
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
      c[i] = (uint32_t)(int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(t + h), 0.0f), top);
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

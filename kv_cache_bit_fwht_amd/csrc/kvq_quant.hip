// Fused quantise + pack, dequantise, and per-channel key calibration kernels.
//
// Operation ([E22L] "Can 4-bit keys and 2-bit values hit a 1M-token memory
// budget?", What I tested; [E21W] "PROVISIONAL: known 3-bit KV cache methods
// ...", What I tested): post-RoPE K/V rows -> optional per-channel multiply ->
// optional Walsh-Hadamard rotation -> per-group fp16 scale -> code -> bit pack.
// Every step is one binary32 operation in the same order as the CPU oracle, so
// codes and scales are bit-identical to it.
//
// Memory: each lane reads its 16 fp16 values with two 16-byte loads (a row of
// D = 256 values is 512 contiguous bytes read by 16 lanes), writes a 2*b-byte
// code chunk at the matching offset of the packed row, and the group's first
// lane writes the fp16 scale.  The transform's strides >= 16 go through one
// padded LDS tile per block (17 floats per 16 values).
#include "kvq_internal.hpp"

namespace kvq {

struct QArgs {
  const uint16_t* x;      // fp16 input rows (quantise)
  float* xhat;            // fp32 output rows (dequantise)
  uint32_t* codes;
  uint16_t* scales;
  uint16_t* mins;
  const float* chan;      // [L][H][D] or null
  long long rows;
  int D, T, H, L;
  int lpt_log2;           // log2(D/16)
  int g;                  // group
  int W;                  // rotation width, 0 = none
  float kappa;            // 1/sqrt(W) as applied after the butterflies
  int ng;                 // scales per row
  Tables tab;
};

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
        // number of midpoints strictly below t (binary search; mid[15] = +inf)
        int k = 0;
#pragma unroll
        for (int st = 8; st >= 1; st >>= 1)
          if (tab.nf4_mid[k + st - 1] < t) k += st;
        c[i] = (uint32_t)k;
      }
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
    } else {
      v[i] = h2f((uint16_t)c[i]);
    }
  }
}

__device__ __forceinline__ void row_unit(long long row, int T, int H, int L, int& l, int& h) {
  const long long unit = row / T;
  h = (int)(unit % H);
  l = (int)((unit / H) % L);
}

template <int CB, int BITS>
__global__ __launch_bounds__(kBlock) void k_quantize(QArgs a) {
  __shared__ float lds[kBlock * 17];
  const int tid = threadIdx.x;
  const int LPT = 1 << a.lpt_log2;
  const int j = tid & (LPT - 1);
  const int rloc = tid >> a.lpt_log2;
  const int RPB = kBlock >> a.lpt_log2;
  float* rowlds = lds + rloc * 17 * LPT;
  const size_t row_bytes = (size_t)a.D * BITS / 8;
  uint8_t* cbytes = reinterpret_cast<uint8_t*>(a.codes);
  for (long long base = (long long)blockIdx.x * RPB; base < a.rows; base += (long long)gridDim.x * RPB) {
    const long long row = base + rloc;
    const bool active = row < a.rows;
    float v[16];
    uint32_t raw[8];
    if (active) {
      const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)row * a.D + 16 * j);
      const uint4 p0 = src[0], p1 = src[1];
      raw[0] = p0.x; raw[1] = p0.y; raw[2] = p0.z; raw[3] = p0.w;
      raw[4] = p1.x; raw[5] = p1.y; raw[6] = p1.z; raw[7] = p1.w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) raw[k] = 0u;
    }
    if constexpr (CB == KVQ_FP16) {
      if (active) store_chunk<16>(cbytes, (size_t)row * row_bytes + (size_t)j * 32, raw);
      continue;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[2 * k] = h2f((uint16_t)(raw[k] & 0xffffu));
      v[2 * k + 1] = h2f((uint16_t)(raw[k] >> 16));
    }
    if (a.chan != nullptr && active) {
      int l, h;
      row_unit(row, a.T, a.H, a.L, l, h);
      const float4* cp = reinterpret_cast<const float4*>(a.chan + ((size_t)l * a.H + h) * a.D + 16 * j);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 cc = cp[k];
        v[4 * k] = v[4 * k] * cc.x;
        v[4 * k + 1] = v[4 * k + 1] * cc.y;
        v[4 * k + 2] = v[4 * k + 2] * cc.z;
        v[4 * k + 3] = v[4 * k + 3] * cc.w;
      }
    }
    if (a.W > 1) fwht_rows(v, rowlds, j, LPT, a.W, a.kappa);
    uint32_t c[16];
    uint16_t s16[2], z16[2];
    encode16<CB, BITS>(v, a.g, a.tab, c, s16, z16);
    if (!active) continue;
    uint32_t w[8];
    pack16<BITS>(c, w);
    store_chunk<BITS>(cbytes, (size_t)row * row_bytes + (size_t)j * 2 * BITS, w);
    const size_t sbase = (size_t)row * a.ng;
    if (a.g == 8) {
      const uint32_t pk = (uint32_t)s16[0] | ((uint32_t)s16[1] << 16);
      *reinterpret_cast<uint32_t*>(a.scales + sbase + 2 * j) = pk;
      if constexpr (CB == KVQ_INT_MINMAX)
        *reinterpret_cast<uint32_t*>(a.mins + sbase + 2 * j) = (uint32_t)z16[0] | ((uint32_t)z16[1] << 16);
    } else {
      const int lpg = a.g >> 4;        // lanes per group
      if ((j & (lpg - 1)) == 0) {
        a.scales[sbase + j / lpg] = s16[0];
        if constexpr (CB == KVQ_INT_MINMAX) a.mins[sbase + j / lpg] = z16[0];
      }
    }
  }
}

template <int CB, int BITS>
__global__ __launch_bounds__(kBlock) void k_dequant(QArgs a) {
  __shared__ float lds[kBlock * 17];
  const int tid = threadIdx.x;
  const int LPT = 1 << a.lpt_log2;
  const int j = tid & (LPT - 1);
  const int rloc = tid >> a.lpt_log2;
  const int RPB = kBlock >> a.lpt_log2;
  float* rowlds = lds + rloc * 17 * LPT;
  const size_t row_bytes = (size_t)a.D * BITS / 8;
  const uint8_t* cbytes = reinterpret_cast<const uint8_t*>(a.codes);
  for (long long base = (long long)blockIdx.x * RPB; base < a.rows; base += (long long)gridDim.x * RPB) {
    const long long row = base + rloc;
    const bool active = row < a.rows;
    uint32_t w[8], c[16];
    uint16_t s16[2] = {0, 0}, z16[2] = {0, 0};
    if (active) {
      load_chunk<BITS>(cbytes, (size_t)row * row_bytes + (size_t)j * 2 * BITS, w);
      if constexpr (CB != KVQ_FP16) {
        const size_t sbase = (size_t)row * a.ng;
        if (a.g == 8) {
          s16[0] = a.scales[sbase + 2 * j]; s16[1] = a.scales[sbase + 2 * j + 1];
          if constexpr (CB == KVQ_INT_MINMAX) { z16[0] = a.mins[sbase + 2 * j]; z16[1] = a.mins[sbase + 2 * j + 1]; }
        } else {
          const int gi = (16 * j) / a.g;
          s16[0] = s16[1] = a.scales[sbase + gi];
          if constexpr (CB == KVQ_INT_MINMAX) z16[0] = z16[1] = a.mins[sbase + gi];
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) w[k] = 0u;
    }
    unpack16<BITS>(w, c);
    float v[16];
    decode16<CB, BITS>(c, s16, z16, a.tab, v);
    if (a.W > 1) fwht_rows(v, rowlds, j, LPT, a.W, a.kappa);
    if (!active) continue;
    if (a.chan != nullptr) {
      int l, h;
      row_unit(row, a.T, a.H, a.L, l, h);
      const float* cp = a.chan + ((size_t)l * a.H + h) * a.D + 16 * j;
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = __fdiv_rn(v[k], cp[k]);
    }
    float4* dst = reinterpret_cast<float4*>(a.xhat + (size_t)row * a.D + 16 * j);
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
}

// Per-channel absmax over tokens of the one calibration sequence -> RN32(1/lambda).
__global__ __launch_bounds__(kBlock) void k_calibrate(const uint16_t* __restrict__ k, int L, int H, int T,
                                                      int D, float* __restrict__ c) {
  const long long idx = (long long)blockIdx.x * kBlock + threadIdx.x;
  if (idx >= (long long)L * H * D) return;
  const int d = (int)(idx % D);
  const long long unit = idx / D;
  const uint16_t* p = k + (size_t)unit * T * D + d;
  float m = 0.0f;
  for (int t = 0; t < T; ++t) m = __builtin_fmaxf(m, __builtin_fabsf(h2f(p[(size_t)t * D])));
  c[idx] = (m == 0.0f) ? 1.0f : __fdiv_rn(1.0f, m);
}

// ------------------------------------------------------------------ host launchers

static QArgs make_args(const kvq_packed& p) {
  QArgs a{};
  a.codes = p.codes;
  a.scales = p.scales;
  a.mins = p.mins;
  a.chan = p.chan_scale;
  a.D = p.shape.head_dim;
  a.T = p.shape.tokens;
  a.H = p.shape.heads;
  a.L = p.shape.layers;
  a.rows = (long long)p.shape.batch * p.shape.layers * p.shape.heads * p.shape.tokens;
  a.lpt_log2 = (a.D == 64) ? 2 : (a.D == 128) ? 3 : 4;
  a.g = p.codec.group;
  a.W = p.codec.rot_width > 1 ? p.codec.rot_width : 0;
  int e = 0;
  while ((1 << e) < a.W) ++e;
  a.kappa = (a.W > 1) ? ((e % 2 == 0) ? ldexpf(1.0f, -e / 2) : (float)(1.0 / sqrt((double)a.W))) : 1.0f;
  a.ng = (p.codec.codebook == KVQ_FP16) ? 0 : a.D / a.g;
  a.tab = host_tables();
  return a;
}

static int grid_for(long long rows, int lpt_log2) {
  const long long rpb = kBlock >> lpt_log2;
  long long blocks = (rows + rpb - 1) / rpb;
  const long long cap = 256 * 8;
  if (blocks > cap) blocks = cap;
  return (int)(blocks < 1 ? 1 : blocks);
}

#define KVQ_DISPATCH_CODEC(CB_, BITS_, KERNEL, ...)                                              \
  switch (CB_) {                                                                                 \
    case KVQ_FP16: KERNEL<KVQ_FP16, 16> __VA_ARGS__; break;                                       \
    case KVQ_TERNARY: KERNEL<KVQ_TERNARY, 2> __VA_ARGS__; break;                                  \
    case KVQ_SIGN: KERNEL<KVQ_SIGN, 1> __VA_ARGS__; break;                                        \
    case KVQ_NF4: KERNEL<KVQ_NF4, 4> __VA_ARGS__; break;                                          \
    case KVQ_INT8_SYM: KERNEL<KVQ_INT8_SYM, 8> __VA_ARGS__; break;                                \
    case KVQ_INT_ABSMAX:                                                                         \
      switch (BITS_) {                                                                           \
        case 2: KERNEL<KVQ_INT_ABSMAX, 2> __VA_ARGS__; break;                                     \
        case 3: KERNEL<KVQ_INT_ABSMAX, 3> __VA_ARGS__; break;                                     \
        case 4: KERNEL<KVQ_INT_ABSMAX, 4> __VA_ARGS__; break;                                     \
        case 5: KERNEL<KVQ_INT_ABSMAX, 5> __VA_ARGS__; break;                                     \
        case 6: KERNEL<KVQ_INT_ABSMAX, 6> __VA_ARGS__; break;                                     \
        case 7: KERNEL<KVQ_INT_ABSMAX, 7> __VA_ARGS__; break;                                     \
        default: KERNEL<KVQ_INT_ABSMAX, 8> __VA_ARGS__; break;                                    \
      }                                                                                          \
      break;                                                                                     \
    default:                                                                                     \
      switch (BITS_) {                                                                           \
        case 2: KERNEL<KVQ_INT_MINMAX, 2> __VA_ARGS__; break;                                     \
        case 3: KERNEL<KVQ_INT_MINMAX, 3> __VA_ARGS__; break;                                     \
        case 4: KERNEL<KVQ_INT_MINMAX, 4> __VA_ARGS__; break;                                     \
        case 5: KERNEL<KVQ_INT_MINMAX, 5> __VA_ARGS__; break;                                     \
        case 6: KERNEL<KVQ_INT_MINMAX, 6> __VA_ARGS__; break;                                     \
        case 7: KERNEL<KVQ_INT_MINMAX, 7> __VA_ARGS__; break;                                     \
        default: KERNEL<KVQ_INT_MINMAX, 8> __VA_ARGS__; break;                                    \
      }                                                                                          \
  }

hipError_t launch_quantize(const uint16_t* x, const kvq_packed& p, hipStream_t st) {
  QArgs a = make_args(p);
  a.x = x;
  if (a.rows == 0) return hipSuccess;
  const dim3 grid(grid_for(a.rows, a.lpt_log2)), block(kBlock);
  KVQ_DISPATCH_CODEC(p.codec.codebook, p.codec.bits, k_quantize, <<<grid, block, 0, st>>>(a))
  return hipGetLastError();
}

hipError_t launch_dequant(const kvq_packed& p, float* xhat, hipStream_t st) {
  QArgs a = make_args(p);
  a.xhat = xhat;
  if (a.rows == 0) return hipSuccess;
  const dim3 grid(grid_for(a.rows, a.lpt_log2)), block(kBlock);
  KVQ_DISPATCH_CODEC(p.codec.codebook, p.codec.bits, k_dequant, <<<grid, block, 0, st>>>(a))
  return hipGetLastError();
}

hipError_t launch_calibrate(const uint16_t* k, const kvq_shape& s, float* c, hipStream_t st) {
  const long long n = (long long)s.layers * s.heads * s.head_dim;
  if (n == 0) return hipSuccess;
  k_calibrate<<<(unsigned)((n + kBlock - 1) / kBlock), kBlock, 0, st>>>(k, s.layers, s.heads, s.tokens,
                                                                        s.head_dim, c);
  return hipGetLastError();
}

}  // namespace kvq

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
#include "kvq_codec.hpp"

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

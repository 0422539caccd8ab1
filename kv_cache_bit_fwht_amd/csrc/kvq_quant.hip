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
#include "kvq_quant256.hpp"

namespace kvq {

struct QArgs {
  const uint16_t* x;      // fp16 input rows (quantise)
  float* xhat;            // fp32 output rows (dequantise)
  uint32_t* codes;
  uint16_t* scales;
  uint16_t* mins;
  const float* chan;      // [L][H][D] or null
  const float* mean;      // [L][H][D] or null
  long long rows;          // input rows: B * L * H * T
  int D, T, H, L;          // T: tokens per unit in the input
  int Tout, t0;            // output tensor's tokens per unit; the input's first token there
  int lpt_log2;           // log2(D/16)
  int g;                  // group
  int W;                  // rotation width, 0 = none
  float kappa;            // 1/sqrt(W) as applied after the butterflies
  int ng;                 // scales per row
  Tables tab;
};

// Output row of input row `row`: the same (sequence, layer, head) unit, token t0 + t.
__device__ __forceinline__ long long out_row(const QArgs& a, long long row) {
  if (a.T == a.Tout) return row;
  const long long u = row / a.T;
  return u * a.Tout + a.t0 + (row - u * a.T);
}

// (layer, head) of a row of a [B][L][H][T] row tensor; 32-bit division where the row
// index fits (64-bit division is a long software sequence).
__device__ __forceinline__ void row_unit(long long row, int T, int H, int L, int& l, int& h) {
  if (row < (1ll << 32)) {
    const uint32_t unit = (uint32_t)row / (uint32_t)T;
    h = (int)(unit % (uint32_t)H);
    l = (int)((unit / (uint32_t)H) % (uint32_t)L);
    return;
  }
  const long long unit = row / T;
  h = (int)(unit % H);
  l = (int)((unit / H) % L);
}

// The lane's 16 values (dims 16j .. 16j+15 at `off` in the [L][H][D] vectors): subtract
// the shared mean, then multiply by the channel scale, each rounded to binary32.
__device__ __forceinline__ void pre_row(float (&v)[16], const float* mean, const float* chan, size_t off) {
  if (mean != nullptr) {
    const float4* mp = reinterpret_cast<const float4*>(mean + off);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 m = mp[k];
      v[4 * k] = v[4 * k] - m.x;
      v[4 * k + 1] = v[4 * k + 1] - m.y;
      v[4 * k + 2] = v[4 * k + 2] - m.z;
      v[4 * k + 3] = v[4 * k + 3] - m.w;
    }
  }
  if (chan != nullptr) {
    const float4* cp = reinterpret_cast<const float4*>(chan + off);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 cc = cp[k];
      v[4 * k] = v[4 * k] * cc.x;
      v[4 * k + 1] = v[4 * k + 1] * cc.y;
      v[4 * k + 2] = v[4 * k + 2] * cc.z;
      v[4 * k + 3] = v[4 * k + 3] * cc.w;
    }
  }
}

template <int CB, int BITS>
__global__ __launch_bounds__(kBlock) void k_quantize(QArgs a) {
  __shared__ float2 nf4_cells[CB == KVQ_NF4 ? 256 : 1];
  const int tid = threadIdx.x;
  if constexpr (CB == KVQ_NF4) {
    static_assert(kBlock == 256, "one NF4 cell per thread");
    nf4_cells_init(a.tab, nf4_cells, tid);
    __syncthreads();
  }
  const int LPT = 1 << a.lpt_log2;
  const int j = tid & (LPT - 1);
  const int rloc = tid >> a.lpt_log2;
  const int RPB = kBlock >> a.lpt_log2;
  const size_t row_bytes = (size_t)a.D * BITS / 8;
  uint8_t* cbytes = reinterpret_cast<uint8_t*>(a.codes);
  for (long long base = (long long)blockIdx.x * RPB; base < a.rows; base += (long long)gridDim.x * RPB) {
    const long long row = base + rloc;
    const bool active = row < a.rows;
    float v[16];
    uint32_t raw[8];
    if (active) {                                    // read once: non-temporal loads
      typedef unsigned int u4v __attribute__((ext_vector_type(4)));
      const u4v* src = reinterpret_cast<const u4v*>(a.x + (size_t)row * a.D + 16 * j);
      const u4v p0 = __builtin_nontemporal_load(src), p1 = __builtin_nontemporal_load(src + 1);
      raw[0] = p0.x; raw[1] = p0.y; raw[2] = p0.z; raw[3] = p0.w;
      raw[4] = p1.x; raw[5] = p1.y; raw[6] = p1.z; raw[7] = p1.w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) raw[k] = 0u;
    }
    if constexpr (CB == KVQ_FP16) {
      if (active) store_chunk<16>(cbytes, (size_t)out_row(a, row) * row_bytes + (size_t)j * 32, raw);
      continue;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[2 * k] = h2f((uint16_t)(raw[k] & 0xffffu));
      v[2 * k + 1] = h2f((uint16_t)(raw[k] >> 16));
    }
    if ((a.chan != nullptr || a.mean != nullptr) && active) {
      int l, h;
      row_unit(row, a.T, a.H, a.L, l, h);
      pre_row(v, a.mean, a.chan, ((size_t)l * a.H + h) * a.D + 16 * j);
    }
    if (a.W > 1) fwht_rows(v, j, a.W, a.kappa);
    uint32_t c[16];
    uint16_t s16[2], z16[2];
    encode16<CB, BITS>(v, a.g, a.tab, c, s16, z16, nf4_cells);
    if (!active) continue;
    uint32_t w[8];
    pack16<BITS>(c, w);
    const long long orow = out_row(a, row);
    store_chunk<BITS>(cbytes, (size_t)orow * row_bytes + (size_t)j * 2 * BITS, w);
    const size_t sbase = (size_t)orow * a.ng;
    if (a.g == 8) {
      const uint32_t pk = (uint32_t)s16[0] | ((uint32_t)s16[1] << 16);
      *reinterpret_cast<uint32_t*>(a.scales + sbase + 2 * j) = pk;
      if constexpr (CB == KVQ_INT_MINMAX)
        *reinterpret_cast<uint32_t*>(a.mins + sbase + 2 * j) = (uint32_t)z16[0] | ((uint32_t)z16[1] << 16);
    } else {
      const int lg = __builtin_ctz(a.g);   // groups are powers of two
      if ((j & ((a.g >> 4) - 1)) == 0) {
        a.scales[sbase + (j >> (lg - 4))] = s16[0];
        if constexpr (CB == KVQ_INT_MINMAX) a.mins[sbase + (j >> (lg - 4))] = z16[0];
      }
    }
  }
}

template <int CB, int BITS>
__global__ __launch_bounds__(kBlock) void k_dequant(QArgs a) {
  const int tid = threadIdx.x;
  const int LPT = 1 << a.lpt_log2;
  const int j = tid & (LPT - 1);
  const int rloc = tid >> a.lpt_log2;
  const int RPB = kBlock >> a.lpt_log2;
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
    if (a.W > 1) fwht_rows(v, j, a.W, a.kappa);
    if (!active) continue;
    if (a.chan != nullptr || a.mean != nullptr) {
      int l, h;
      row_unit(row, a.T, a.H, a.L, l, h);
      const size_t off = ((size_t)l * a.H + h) * a.D + 16 * j;
      if (a.chan != nullptr) {
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = __fdiv_rn(v[k], a.chan[off + k]);
      }
      if (a.mean != nullptr) {
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = v[k] + a.mean[off + k];
      }
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

// Shared key mean ([LCPP] llama.cpp issue "Per-head adaptive KV cache quantization",
// the later comment on a shared per-head key mean): exact integer sums of the fp16
// values in units of 2^-24 (every fp16 value is such a multiple, so v * 2^24 is an
// integer below 2^40 and the sums are exact in any order), then one fp64 quotient.
__global__ void k_zero_u64(unsigned long long* p, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// Block (chunk, unit): tokens [t0, t1) of every sequence.  A thread takes 8
// consecutive channels of a row (one 16-byte load), so kBlock * 8 / D rows per pass.
__global__ __launch_bounds__(kBlock) void k_key_sum(const uint16_t* __restrict__ k, int B, int L, int H, int T,
                                                    int D, int chunk, unsigned long long* __restrict__ acc) {
  __shared__ long long red[kBlock];
  const int u = blockIdx.y, l = u / H, h = u - l * H;
  const int tpr = D / 8, rpi = kBlock / tpr;            // threads per row, rows per pass
  const int c8 = threadIdx.x % tpr, r0 = threadIdx.x / tpr;
  const int t0 = blockIdx.x * chunk, t1 = min(T, t0 + chunk);
  long long s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int b = 0; b < B; ++b) {
    const uint16_t* base = k + (((size_t)b * L + l) * H + h) * (size_t)T * D + 8 * c8;
    for (int t = t0 + r0; t < t1; t += rpi) {
      const uint4 p = *reinterpret_cast<const uint4*>(base + (size_t)t * D);
      const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[2 * i] += (long long)(h2f((uint16_t)(w[i] & 0xffffu)) * 16777216.0f);
        s[2 * i + 1] += (long long)(h2f((uint16_t)(w[i] >> 16)) * 16777216.0f);
      }
    }
  }
  // channel 8*c8 + i: sum over the rpi row slots, then one atomic per channel
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    red[threadIdx.x] = s[i];
    __syncthreads();
    if (r0 == 0) {
      long long v = s[i];
      for (int r = 1; r < rpi; ++r) v += red[r * tpr + c8];
      atomicAdd(&acc[(size_t)u * D + 8 * c8 + i], (unsigned long long)v);
    }
    __syncthreads();
  }
}

__global__ void k_key_mean_final(const unsigned long long* __restrict__ acc, long long total, long long n,
                                 float* __restrict__ mean) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const long long S = (long long)acc[i];
  mean[i] = n ? (float)(((double)S / (double)n) * 0x1p-24) : 0.0f;
}

// ------------------------------------------------------------------ host launchers

static QArgs make_args(const kvq_packed& p) {
  QArgs a{};
  a.codes = p.codes;
  a.scales = p.scales;
  a.mins = p.mins;
  a.chan = p.chan_scale;
  a.mean = p.mean;
  a.D = p.shape.head_dim;
  a.T = p.shape.tokens;
  a.Tout = p.shape.tokens;
  a.t0 = 0;
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

// The general quantise kernel's grid, as measured on head_dim-128 tensors of 16.8M rows
// (HIP events, one box; the kernel holds no LDS tile, so occupancy is set by registers):
// one block per RPB rows that codes its rows once and exits is fastest for unrotated
// codes (ternary 1,103 -> 1,021 us, 4-bit 1,166 -> 994 us against the grid capped at
// 2,048 blocks; sign 924 us, int8 1,106 us); NF4, which builds a cell table per block,
// and rotated codes are fastest on a grid-stride grid of 65,536 blocks (NF4 1,158 ->
// 1,026 us against 2,048 blocks and 1,389 us one-pass; rotated 6-bit 1,454 -> 1,294 us
// against 2,048 blocks and 1,416 us one-pass).  Rows of 256 values (16 lanes each) are
// faster on the 65,536-block grid as well (2.1M rows, unrotated: 4-bit min-max at group
// 32 271 us against 286 one-pass, 3-bit absmax 251 against 259-266).
static unsigned quantize_grid(long long rows, int lpt_log2, int codebook, int rot_width) {
  const long long rpb = kBlock >> lpt_log2;
  long long blocks = (rows + rpb - 1) / rpb;
  if ((codebook == KVQ_NF4 || rot_width > 1 || lpt_log2 >= 4) && blocks > 65536) blocks = 65536;
  return (unsigned)(blocks < 1 ? 1 : blocks);
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
    case KVQ_INT_SYM:                                                                            \
      switch (BITS_) {                                                                           \
        case 2: KERNEL<KVQ_INT_SYM, 2> __VA_ARGS__; break;                                        \
        case 3: KERNEL<KVQ_INT_SYM, 3> __VA_ARGS__; break;                                        \
        case 4: KERNEL<KVQ_INT_SYM, 4> __VA_ARGS__; break;                                        \
        case 5: KERNEL<KVQ_INT_SYM, 5> __VA_ARGS__; break;                                        \
        case 6: KERNEL<KVQ_INT_SYM, 6> __VA_ARGS__; break;                                        \
        case 7: KERNEL<KVQ_INT_SYM, 7> __VA_ARGS__; break;                                        \
        default: KERNEL<KVQ_INT_SYM, 8> __VA_ARGS__; break;                                       \
      }                                                                                          \
      break;                                                                                     \
    case KVQ_LLOYD:                                                                              \
      switch (BITS_) {                                                                           \
        case 2: KERNEL<KVQ_LLOYD, 2> __VA_ARGS__; break;                                          \
        case 3: KERNEL<KVQ_LLOYD, 3> __VA_ARGS__; break;                                          \
        default: KERNEL<KVQ_LLOYD, 4> __VA_ARGS__; break;                                         \
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


// ------------------------------------------------------------------ signed absmax, head_dim 256
// A leaner path for the signed-absmax codebook at head_dim 256 with rotation 0 or
// 256, group >= 16 and 2, 4 or 8 bits (the keys and values of the 64K decode
// workload).  Same arithmetic, same results as k_quantize, fewer instructions:
//  * a row is held by 16 lanes of one wavefront, so the FWHT's transposes through
//    LDS are wavefront-local and need no barrier; the contiguous side moves 16 bytes
//    per access (quads XOR-swizzled by lane, so the strided side is conflict-free);
//  * the 2^-4 normalisation of the 256-point transform is a power of two: scaling by
//    it is exact, so it is folded into the scale and its inverse instead of being
//    applied to every value (u * 2^-4 never underflows for fp16-derived values);
//  * the code is RN32(RN32(u * inv) + (1.5 * 2^23 + 2^(b-1))): in [2^23, 2^24) the ulp
//    is 1, so that addition performs the round-to-nearest-even, and the integer sits
//    in the low bits of the result (bits b..21 zero after clamping), ready to pack.

// Quads of rows q_first, q_first + q_stride, ... of one tensor; each wavefront of the
// caller owns one quad per step (16 lanes per row).
// PRE: bit 0 a mean, bit 1 channel scales (loaded with the row, applied before the
// rotation); 0 for neither.
template <int BITS, bool ROT, int PRE>
__device__ __forceinline__ void absmax256_rows(const QArgs& a, long long q_first, long long q_stride,
                                               float* rl, int lane) {
  constexpr int D = 256;
  constexpr float kFold = ROT ? 0.0625f : 1.0f;      // the 256-point transform's 1/sqrt(256)
  constexpr float neg_step = -kFold / (float)(1 << (BITS - 1));
  constexpr uint32_t kMagic = 0x4B400000u;           // bit pattern of 1.5 * 2^23
  constexpr float kBias = 12582912.0f + (float)(1 << (BITS - 1));
  const int j = lane & 15;                           // lane within the row
  const int lpg = a.g >> 4;                          // lanes per group
  const long long nquads = (a.rows + 3) >> 2;
  // PRE (a mean or channel scales; tokens per unit a multiple of 4, so a quad never
  // spans two units): the (layer, head) of the wavefront's quad, kept as uniform state
  // and stepped to the next unit without a division (64-bit division is a long
  // software sequence)
  long long w_lo = 0, w_hi = 0;
  int w_l = 0, w_h = 0;
  for (long long qd = q_first; qd < nquads; qd += q_stride) {
    const long long row = qd * 4 + (lane >> 4);
    const bool active = row < a.rows;
    if constexpr (PRE != 0) {
      const long long row0 = qd * 4;                 // the quad's first row (uniform)
      if (row0 < w_lo || row0 >= w_hi) {
        if (w_hi > 0 && row0 >= w_hi && row0 < w_hi + a.T) {   // the next unit
          w_lo = w_hi;
          w_hi += a.T;
          if (++w_h == a.H) {
            w_h = 0;
            if (++w_l == a.L) w_l = 0;
          }
        } else {
          const long long unit = row0 / a.T;
          w_lo = unit * a.T;
          w_hi = w_lo + a.T;
          w_h = (int)(unit % a.H);
          w_l = (int)((unit / a.H) % a.L);
        }
      }
    }
    uint4 p0 = make_uint4(0, 0, 0, 0), p1 = p0;
    // PRE: the lane's mean and scale values, loaded together with the row (one round trip)
    float4 pm[4], pc[4];
    if (active) {
      const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)row * D + 16 * j);
      p0 = src[0];
      p1 = src[1];
      if constexpr (PRE != 0) {
        const size_t off = ((size_t)w_l * a.H + w_h) * D + 16 * j;
        if constexpr ((PRE & 1) != 0) {
#pragma unroll
          for (int k = 0; k < 4; ++k) pm[k] = reinterpret_cast<const float4*>(a.mean + off)[k];
        }
        if constexpr ((PRE & 2) != 0) {
#pragma unroll
          for (int k = 0; k < 4; ++k) pc[k] = reinterpret_cast<const float4*>(a.chan + off)[k];
        }
      }
    }
    const uint32_t raw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    float v[16];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[2 * k] = h2f((uint16_t)(raw[k] & 0xffffu));
      v[2 * k + 1] = h2f((uint16_t)(raw[k] >> 16));
    }
    if constexpr (PRE != 0) {
      if (active) {
        if constexpr ((PRE & 1) != 0) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[4 * k] = v[4 * k] - pm[k].x;
            v[4 * k + 1] = v[4 * k + 1] - pm[k].y;
            v[4 * k + 2] = v[4 * k + 2] - pm[k].z;
            v[4 * k + 3] = v[4 * k + 3] - pm[k].w;
          }
        }
        if constexpr ((PRE & 2) != 0) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[4 * k] = v[4 * k] * pc[k].x;
            v[4 * k + 1] = v[4 * k + 1] * pc[k].y;
            v[4 * k + 2] = v[4 * k + 2] * pc[k].z;
            v[4 * k + 3] = v[4 * k + 3] * pc[k].w;
          }
        }
      }
    }
    if constexpr (ROT) {
      // strides 1, 2, 4, 8: inside the lane's 16 consecutive values
#pragma unroll
      for (int s = 1; s < 16; s <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!(i & s)) {
            const float x = v[i], y = v[i + s];
            v[i] = x + y;
            v[i + s] = x - y;
          }
      }
      // transpose: lane j takes values j + 16 r (r = 0..15); quads of a lane's values sit
      // at quad index (q ^ (owner & 3)) of the owner's 16-float slot
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(rl + 16 * j + 4 * (q ^ (j & 3))) =
            make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = rl[16 * r + 4 * ((j >> 2) ^ (r & 3)) + (j & 3)];
      // strides 16, 32, 64, 128: pairs (r, r + rs) of the transposed values
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
    }
    // group statistic: the signed extreme of the group (lpg lanes)
    float mx = v[0], mn = v[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      mx = __builtin_fmaxf(mx, v[i]);
      mn = __builtin_fminf(mn, v[i]);
    }
    run_maxmin(mx, mn, lpg);
    const float ext = (-mn >= mx) ? mn : mx;
    const uint16_t s16 = rn16(ext * neg_step);       // exact product: neg_step is a power of two
    const float inv = inv_scale(s16) * kFold;        // exact: kFold is a power of two
    uint32_t c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float f = __fadd_rn(__fmul_rn(v[i], inv), kBias);
      const int b = (int)__builtin_bit_cast(uint32_t, f);
      c[i] = (uint32_t)min(max(b, (int)kMagic), (int)(kMagic + (1u << BITS) - 1u));
    }
    if (!active) continue;
    const long long orow = out_row(a, row);
    uint8_t* dst = reinterpret_cast<uint8_t*>(a.codes) + (size_t)orow * (D * BITS / 8) + (size_t)j * 2 * BITS;
    if constexpr (BITS == 4) {
      uint32_t w[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t t0 = (c[8 * k + 1] << 4) | c[8 * k + 0], t1 = (c[8 * k + 3] << 4) | c[8 * k + 2];
        const uint32_t t2 = (c[8 * k + 5] << 4) | c[8 * k + 4], t3 = (c[8 * k + 7] << 4) | c[8 * k + 6];
        const uint32_t h0 = __builtin_amdgcn_perm(t1, t0, 0x0C0C0400u);
        const uint32_t h1 = __builtin_amdgcn_perm(t3, t2, 0x0C0C0400u);
        w[k] = (h1 << 16) | h0;
      }
      *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    } else if constexpr (BITS == 2) {
      uint32_t by[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = (c[4 * k + 1] << 2) | c[4 * k + 0], hi = (c[4 * k + 3] << 2) | c[4 * k + 2];
        by[k] = (hi << 4) | lo;
      }
      const uint32_t h0 = __builtin_amdgcn_perm(by[1], by[0], 0x0C0C0400u);
      const uint32_t h1 = __builtin_amdgcn_perm(by[3], by[2], 0x0C0C0400u);
      *reinterpret_cast<uint32_t*>(dst) = (h1 << 16) | h0;
    } else {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t h0 = __builtin_amdgcn_perm(c[4 * k + 1], c[4 * k + 0], 0x0C0C0400u);
        const uint32_t h1 = __builtin_amdgcn_perm(c[4 * k + 3], c[4 * k + 2], 0x0C0C0400u);
        w[k] = (h1 << 16) | h0;
      }
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    const int lg = __builtin_ctz(a.g);               // groups are powers of two
    if ((j & (lpg - 1)) == 0) a.scales[(size_t)orow * (D >> lg) + (j >> (lg - 4))] = s16;
  }
}

template <int BITS, bool ROT, int PRE>
__global__ __launch_bounds__(kBlock) void k_quantize_absmax256(QArgs a) {
  __shared__ float lds[kBlock / 16][kRowLds];
  constexpr int waves = kBlock / 64;
  const int tid = threadIdx.x;
  absmax256_rows<BITS, ROT, PRE>(a, (long long)blockIdx.x * waves + (tid >> 6), (long long)gridDim.x * waves,
                                 lds[tid >> 4], tid & 63);
}

constexpr int kQuadWaves = 4;                        // wavefronts (row quads) per block

template <int BITS, bool ROT, int CB = KVQ_INT_ABSMAX>
__global__ __launch_bounds__(kQuadWaves * 64) void k_quantize_q256(QArgs a) {
  __shared__ float lds[kQuadWaves * 4][kRowLds];
  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15;
  const long long row = ((long long)blockIdx.x * kQuadWaves + (tid >> 6)) * 4 + (lane >> 4);
  if (((long long)blockIdx.x * kQuadWaves + (tid >> 6)) * 4 >= a.rows) return;   // whole wavefront past the end
  uint4 p0, p1;
  load_row256_nt(a.x, a.rows, row, j, p0, p1);
  code_row256<BITS, ROT, false, CB>(a.codes, a.scales, a.g, out_row(a, row), row < a.rows, p0, p1, lds[tid >> 4], j,
                                    &a.tab);
}

// K and V of one cache in one launch: wavefront 2q codes quad q of the key rows and
// wavefront 2q + 1 the same quad of the value rows.  One launch keeps both streams in
// flight together and pays one launch and one tail.  Alternating the tensors by
// wavefront measured 6% faster than one wavefront coding both quads (and 2% faster
// than one launch per tensor): a wavefront has half the bytes to wait for, and the
// rotated keys' arithmetic overlaps the values' loads on the same SIMD.
template <int KB, bool KROT, int VB, bool VROT>
__global__ __launch_bounds__(kQuadWaves * 64) void k_quantize_kv256(QArgs ak, QArgs av) {
  __shared__ float lds[kQuadWaves * 4][kRowLds];
  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15;
  const long long w = (long long)blockIdx.x * kQuadWaves + (tid >> 6);
  const long long q0 = (w >> 1) * 4;
  if (q0 >= ak.rows) return;
  const long long row = q0 + (lane >> 4);
  uint4 p0, p1;
  if (w & 1) {
    load_row256_nt(av.x, av.rows, row, j, p0, p1);
    code_row256<VB, VROT, false>(av.codes, av.scales, av.g, out_row(av, row), row < av.rows, p0, p1, lds[tid >> 4], j);
  } else {
    load_row256_nt(ak.x, ak.rows, row, j, p0, p1);
    code_row256<KB, KROT, false>(ak.codes, ak.scales, ak.g, out_row(ak, row), row < ak.rows, p0, p1, lds[tid >> 4], j);
  }
}

static unsigned quad_blocks(long long rows) {
  const long long quads = (rows + 3) / 4;
  return (unsigned)((quads + kQuadWaves - 1) / kQuadWaves);
}

static bool absmax256_supported(const kvq_packed& p, int tokens_in) {
  const kvq_codec& c = p.codec;
  if (p.shape.head_dim != 256) return false;
  if (c.codebook == KVQ_INT_SYM || c.codebook == KVQ_LLOYD) {
    // the one-quad-per-wavefront coder has these grids too (without a mean or channel scales)
    if (p.chan_scale || p.mean) return false;
    if (c.codebook == KVQ_LLOYD && c.bits == 8) return false;
  } else if (c.codebook != KVQ_INT_ABSMAX) {
    return false;
  }
  if ((p.chan_scale || p.mean) && tokens_in % 4 != 0) return false;   // a quad would span two units
  if (c.bits != 2 && c.bits != 4 && c.bits != 8) return false;
  if (c.group < 16 || c.group > 256) return false;
  return c.rot_width <= 1 || c.rot_width == 256;
}

// At most the blocks that are resident at once: 8 wavefronts per SIMD, 6 for the
// variants that hold a mean or scale vector (more registers).
static long long absmax256_blocks(long long rows, int pre) {
  const long long quads = (rows + 3) / 4;
  long long blocks = (quads + (kBlock / 64) - 1) / (kBlock / 64);
  const long long cap = 256 * (pre ? 6 : 8);
  if (blocks > cap) blocks = cap;
  return blocks < 1 ? 1 : blocks;
}

template <int PRE>
static void launch_absmax256_pre(const QArgs& a, const kvq_codec& c, hipStream_t st) {
  const dim3 grid((unsigned)absmax256_blocks(a.rows, PRE));
  const bool rot = c.rot_width == 256;
  if (c.bits == 2) rot ? k_quantize_absmax256<2, true, PRE><<<grid, kBlock, 0, st>>>(a)
                       : k_quantize_absmax256<2, false, PRE><<<grid, kBlock, 0, st>>>(a);
  else if (c.bits == 4) rot ? k_quantize_absmax256<4, true, PRE><<<grid, kBlock, 0, st>>>(a)
                            : k_quantize_absmax256<4, false, PRE><<<grid, kBlock, 0, st>>>(a);
  else rot ? k_quantize_absmax256<8, true, PRE><<<grid, kBlock, 0, st>>>(a)
           : k_quantize_absmax256<8, false, PRE><<<grid, kBlock, 0, st>>>(a);
}

static void launch_absmax256(const QArgs& a, const kvq_codec& c, hipStream_t st) {
  const int pre = (a.mean != nullptr ? 1 : 0) | (a.chan != nullptr ? 2 : 0);
  if (pre == 0) {
    const dim3 grid(quad_blocks(a.rows));
    const bool rot = c.rot_width == 256;
    const dim3 blk(kQuadWaves * 64);
    if (c.codebook == KVQ_INT_SYM) {
      if (c.bits == 2) rot ? k_quantize_q256<2, true, KVQ_INT_SYM><<<grid, blk, 0, st>>>(a)
                           : k_quantize_q256<2, false, KVQ_INT_SYM><<<grid, blk, 0, st>>>(a);
      else if (c.bits == 4) rot ? k_quantize_q256<4, true, KVQ_INT_SYM><<<grid, blk, 0, st>>>(a)
                                : k_quantize_q256<4, false, KVQ_INT_SYM><<<grid, blk, 0, st>>>(a);
      else rot ? k_quantize_q256<8, true, KVQ_INT_SYM><<<grid, blk, 0, st>>>(a)
               : k_quantize_q256<8, false, KVQ_INT_SYM><<<grid, blk, 0, st>>>(a);
    } else if (c.codebook == KVQ_LLOYD) {
      if (c.bits == 2) rot ? k_quantize_q256<2, true, KVQ_LLOYD><<<grid, blk, 0, st>>>(a)
                           : k_quantize_q256<2, false, KVQ_LLOYD><<<grid, blk, 0, st>>>(a);
      else rot ? k_quantize_q256<4, true, KVQ_LLOYD><<<grid, blk, 0, st>>>(a)
               : k_quantize_q256<4, false, KVQ_LLOYD><<<grid, blk, 0, st>>>(a);
    } else {
      if (c.bits == 2) rot ? k_quantize_q256<2, true><<<grid, blk, 0, st>>>(a)
                           : k_quantize_q256<2, false><<<grid, blk, 0, st>>>(a);
      else if (c.bits == 4) rot ? k_quantize_q256<4, true><<<grid, blk, 0, st>>>(a)
                                : k_quantize_q256<4, false><<<grid, blk, 0, st>>>(a);
      else rot ? k_quantize_q256<8, true><<<grid, blk, 0, st>>>(a)
               : k_quantize_q256<8, false><<<grid, blk, 0, st>>>(a);
    }
  }
  else if (pre == 1) launch_absmax256_pre<1>(a, c, st);
  else if (pre == 2) launch_absmax256_pre<2>(a, c, st);
  else launch_absmax256_pre<3>(a, c, st);
}

hipError_t launch_quantize(const uint16_t* x, const kvq_packed& p, hipStream_t st) {
  QArgs a = make_args(p);
  a.x = x;
  if (a.rows == 0) return hipSuccess;
  if (absmax256_supported(p, a.T)) {
    launch_absmax256(a, p.codec, st);
    return hipGetLastError();
  }
  const dim3 grid(quantize_grid(a.rows, a.lpt_log2, p.codec.codebook, a.W)), block(kBlock);
  KVQ_DISPATCH_CODEC(p.codec.codebook, p.codec.bits, k_quantize, <<<grid, block, 0, st>>>(a))
  return hipGetLastError();
}

hipError_t launch_quantize_tokens(const uint16_t* x, const kvq_packed& p, int t0, int n, hipStream_t st) {
  QArgs a = make_args(p);
  a.x = x;
  a.T = n;
  a.t0 = t0;
  a.rows = (long long)p.shape.batch * p.shape.layers * p.shape.heads * n;
  if (a.rows == 0) return hipSuccess;
  if (absmax256_supported(p, n)) {
    launch_absmax256(a, p.codec, st);
    return hipGetLastError();
  }
  const dim3 grid(quantize_grid(a.rows, a.lpt_log2, p.codec.codebook, a.W)), block(kBlock);
  KVQ_DISPATCH_CODEC(p.codec.codebook, p.codec.bits, k_quantize, <<<grid, block, 0, st>>>(a))
  return hipGetLastError();
}

// ---- K and V in one launch

template <int KB, bool KROT>
static void launch_kv256_v(const QArgs& ak, const QArgs& av, int vb, bool vrot, dim3 grid, hipStream_t st) {
  constexpr int nt = kQuadWaves * 64;
  if (vb == 2) vrot ? k_quantize_kv256<KB, KROT, 2, true><<<grid, nt, 0, st>>>(ak, av)
                    : k_quantize_kv256<KB, KROT, 2, false><<<grid, nt, 0, st>>>(ak, av);
  else if (vb == 4) vrot ? k_quantize_kv256<KB, KROT, 4, true><<<grid, nt, 0, st>>>(ak, av)
                         : k_quantize_kv256<KB, KROT, 4, false><<<grid, nt, 0, st>>>(ak, av);
  else vrot ? k_quantize_kv256<KB, KROT, 8, true><<<grid, nt, 0, st>>>(ak, av)
            : k_quantize_kv256<KB, KROT, 8, false><<<grid, nt, 0, st>>>(ak, av);
}

// Both tensors 256-wide signed absmax without a mean or channel scales, of one shape:
// one launch.  Otherwise the two single-tensor launches (same results either way).
hipError_t launch_quantize_kv(const uint16_t* kx, const uint16_t* vx, const kvq_packed& kp, const kvq_packed& vp,
                              int t0, int n, hipStream_t st) {
  const bool window = !(t0 == 0 && n == kp.shape.tokens);
  auto lean = [&](const kvq_packed& p) {
    return absmax256_supported(p, n) && p.codec.codebook == KVQ_INT_ABSMAX && p.mean == nullptr &&
           p.chan_scale == nullptr;
  };
  // (symmetric-grid or Lloyd-Max values take two launches of the quad coder: one launch
  // for both measured no faster with rotated values)
  if (!lean(kp) || !lean(vp)) {
    hipError_t e = window ? launch_quantize_tokens(kx, kp, t0, n, st) : launch_quantize(kx, kp, st);
    if (e != hipSuccess) return e;
    return window ? launch_quantize_tokens(vx, vp, t0, n, st) : launch_quantize(vx, vp, st);
  }
  QArgs ak = make_args(kp), av = make_args(vp);
  ak.x = kx;
  av.x = vx;
  ak.T = av.T = n;
  ak.t0 = av.t0 = t0;
  ak.rows = av.rows = (long long)kp.shape.batch * kp.shape.layers * kp.shape.heads * n;
  if (ak.rows == 0) return hipSuccess;
  const long long waves = 2 * ((ak.rows + 3) / 4);  // two wavefronts (K, V) per row quad
  const dim3 grid((unsigned)((waves + kQuadWaves - 1) / kQuadWaves));
  const bool krot = kp.codec.rot_width == 256, vrot = vp.codec.rot_width == 256;
  const int vb = vp.codec.bits;
  switch (kp.codec.bits) {
    case 2: krot ? launch_kv256_v<2, true>(ak, av, vb, vrot, grid, st) : launch_kv256_v<2, false>(ak, av, vb, vrot, grid, st); break;
    case 4: krot ? launch_kv256_v<4, true>(ak, av, vb, vrot, grid, st) : launch_kv256_v<4, false>(ak, av, vb, vrot, grid, st); break;
    default: krot ? launch_kv256_v<8, true>(ak, av, vb, vrot, grid, st) : launch_kv256_v<8, false>(ak, av, vb, vrot, grid, st); break;
  }
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

hipError_t launch_key_mean(const uint16_t* k, const kvq_shape& s, float* mean, long long* ws, hipStream_t st) {
  const long long units = (long long)s.layers * s.heads, total = units * s.head_dim;
  if (total == 0) return hipSuccess;
  unsigned long long* acc = reinterpret_cast<unsigned long long*>(ws);
  k_zero_u64<<<(unsigned)((total + kBlock - 1) / kBlock), kBlock, 0, st>>>(acc, total);
  if (s.tokens > 0 && s.batch > 0) {
    const int rpi = kBlock * 8 / s.head_dim;
    long long chunks = (2048 + units - 1) / units;
    const long long max_chunks = (s.tokens + rpi * 32 - 1) / (rpi * 32);
    if (chunks > max_chunks) chunks = max_chunks;
    if (chunks < 1) chunks = 1;
    const int chunk = (int)((s.tokens + chunks - 1) / chunks);
    chunks = (s.tokens + chunk - 1) / chunk;
    k_key_sum<<<dim3((unsigned)chunks, (unsigned)units), kBlock, 0, st>>>(k, s.batch, s.layers, s.heads, s.tokens,
                                                                         s.head_dim, chunk, acc);
  }
  k_key_mean_final<<<(unsigned)((total + kBlock - 1) / kBlock), kBlock, 0, st>>>(
      acc, total, (long long)s.batch * s.tokens, mean);
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

// rFFT physical codecs ([FMAG-R] HF forum thread "Fourier Magnitude KV Cache
// Quantization", Colab-probe reply: rFFT + packed magnitude index + packed
// phase-angle index, and the real/imaginary control): quantise+pack and
// dequantise kernels.  A row is held by N/16 lanes, so a wavefront codes 16, 8 or
// 4 rows at once: each lane gathers 16 bit-reversed inputs and runs the radix-2
// stages of span <= 16 in registers; one wavefront-local LDS transpose hands every
// lane the inputs of the longer spans, which also run in registers with twiddles
// from LDS.  Scales come from DPP reductions over half rows, phase sectors from two
// side tests around an arctangent estimate, and codes are packed through LDS into
// coalesced stores.  No block barrier follows the table load.
#include "kvq_rfft.hpp"

namespace kvq {

struct RArgs {
  const uint16_t* x;
  float* xhat;
  uint32_t* codes;
  uint16_t* scales;
  const float* chan;
  const float* mean;
  long long rows;          // input rows: B * L * H * T
  int T, H, L;             // T: tokens per unit in the input
  int Tout, t0;            // output tensor's tokens per unit; the input's first token there
  RfftCodec c;
  FftTables tw;
  PhaseTables pt;
};

constexpr int kWaves = kBlock / 64;
constexpr int kMaxN = 256;

// The constant tables in LDS, copied once per block: per-lane indexed reads of the
// kernel-argument copies would each be a memory round trip.
struct LdsTables {
  float twc[kMaxN / 2], tws[kMaxN / 2];    // twiddles of head_dim
  float dirc[256], dirs[256];              // phase-sector directions
  float bndc[32], bnds[32];                // first-octant sector boundaries
};
__device__ __forceinline__ void load_tables(const RArgs& a, LdsTables& t) {
  for (int i = threadIdx.x; i < kMaxN / 2; i += kBlock) {
    t.twc[i] = a.tw.tw_c[i];
    t.tws[i] = a.tw.tw_s[i];
  }
  for (int i = threadIdx.x; i < 256; i += kBlock) {
    t.dirc[i] = a.pt.dir_c[i];
    t.dirs[i] = a.pt.dir_s[i];
  }
  for (int i = threadIdx.x; i < 32; i += kBlock) {
    t.bndc[i] = a.pt.bnd_c[i];
    t.bnds[i] = a.pt.bnd_s[i];
  }
  __syncthreads();
}

// (layer, head) of a row; 32-bit division where the row index fits.
__device__ __forceinline__ void unit_of(long long row, int T, int H, int L, int& l, int& h) {
  if (row < (1ll << 32)) {
    const uint32_t u = (uint32_t)row / (uint32_t)T;
    h = (int)(u % (uint32_t)H);
    l = (int)((u / (uint32_t)H) % (uint32_t)L);
    return;
  }
  const long long u = row / T;
  h = (int)(u % H);
  l = (int)((u / H) % L);
}

// ---------------------------------------------------------------- quantise + pack
//
// N/16 lanes per row and 64/(N/16) rows per wavefront; every butterfly of the
// transform is the radix-2 butterfly described above, with the same binary32
// operations, so the spectrum is the same bit for bit.  Lane l of a row first owns
// the 16 bit-reversed positions 16l .. 16l+15 (gathered straight from the row) and
// runs the four stages of span <= 16 in registers, skipping only products whose
// operands are known to be exactly real (finite inputs: the skipped terms are zeros).
// One LDS transpose then gives lane l the positions b + 16k for its 256/N values of b
// and every k, and the remaining stages run in registers; the lane ends holding bins
// b + 16k below N/2 (and lane 0 the Nyquist bin).  Group extremes come from
// cross-lane reductions over 8-bin cells, one lane per group forms each scale, the
// codes go to LDS as bytes, and each lane packs the run of 8 consecutive bins 8l ..
// 8l+7 of each field into the row's words with LDS ORs.
template <int N>
struct RegGeom {
  static constexpr int NB = (N == 64) ? 6 : (N == 128) ? 7 : 8;   // log2 N
  static constexpr int LPR = N / 16;          // lanes per row
  static constexpr int RPW = 64 / LPR;        // rows per wavefront
  static constexpr int BPL = 256 / N;         // values of b per lane after the transpose
  static constexpr int KN = N / 16;           // values of k
  static constexpr int KH = KN / 2;           // k of the bins below N/2
  static constexpr int ROWF = 2 * N + N / 4;  // floats per row in the transpose buffer
  static constexpr int FA = N / 2 + 8;        // code bytes per row and field
};

constexpr int kRegWaveFloats = 2304;           // RPW * ROWF for every N
constexpr int kMaxSectors8 = 32;               // P/8 for P = 256

// Code-byte, word, cell, scale regions inside a wavefront's transpose buffer, used
// after the transpose has been read back (bytes; every offset 16-aligned).
constexpr int kOffBytes = 0;        // [2][RPW][FA] code bytes                 <= 1280
constexpr int kOffWords = 1280;     // [RPW * words + 4] packed words           <= 1104
constexpr int kOffCells = 2400;     // [RPW][N/16] cell extremes (float or float4) 1024
constexpr int kOffCellX = 3424;     // [RPW] Nyquist-bin values (float2)          128
constexpr int kOffInv = 3552;       // [RPW * nscales] reciprocal scales          <= 640
constexpr int kOffScale = 4192;     // [RPW * nscales] fp16 scales                <= 320
static_assert(kOffScale + 320 <= kRegWaveFloats * 4, "regions fit the transpose buffer");

__device__ __forceinline__ constexpr int rev4(int e) {
  return ((e & 1) << 3) | ((e & 2) << 1) | ((e & 4) >> 1) | ((e & 8) >> 3);
}

template <int CTRL>
__device__ __forceinline__ float rdpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// max / min over the LPR/2 lanes of a half row (aligned groups of 2, 4 or 8 lanes)
template <int LPR>
__device__ __forceinline__ float half_row_max(float x) {
  x = __builtin_fmaxf(x, rdpp<0xB1>(x));                              // quad_perm [1,0,3,2]
  if constexpr (LPR >= 8) x = __builtin_fmaxf(x, rdpp<0x4E>(x));      // quad_perm [2,3,0,1]
  if constexpr (LPR >= 16) x = __builtin_fmaxf(x, rdpp<0x141>(x));    // row_half_mirror
  return x;
}
template <int LPR>
__device__ __forceinline__ float half_row_min(float x) {
  x = __builtin_fminf(x, rdpp<0xB1>(x));
  if constexpr (LPR >= 8) x = __builtin_fminf(x, rdpp<0x4E>(x));
  if constexpr (LPR >= 16) x = __builtin_fminf(x, rdpp<0x141>(x));
  return x;
}

// In-register stage of span 2^S (S = 1..4) over positions 16l + e.  Before it, the
// values at e mod 2^(S-1) in {0, 2^(S-2)} are exactly real (the outputs of twiddle-1
// butterflies, starting from a real row), and so are both operands of the butterflies
// with jj = 0 (twiddle (1, -0): t = b) and jj = half/2 (t = (b wr, b wi)).
template <int N, int S>
__device__ __forceinline__ void reg_stage_low(float (&re)[16], float (&im)[16], const FftTables& tw) {
  constexpr int H = 1 << (S - 1), SP = 1 << S;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    if ((e & (SP - 1)) >= H) continue;
    const int jj = e & (H - 1), f = e + H;
    const float xr = re[e], xi = im[e];
    if (jj == 0) {
      const float br = re[f];
      re[e] = xr + br;
      re[f] = xr - br;
    } else if (2 * jj == H) {
      const float wr = tw.tw_c[jj * (N / SP)], wi = tw.tw_s[jj * (N / SP)];
      const float tr = re[f] * wr, ti = re[f] * wi;
      re[e] = xr + tr;
      im[e] = ti;
      re[f] = xr - tr;
      im[f] = -ti;
    } else {
      const float wr = tw.tw_c[jj * (N / SP)], wi = tw.tw_s[jj * (N / SP)];
      const float br = re[f], bi = im[f];
      const float tr = br * wr - bi * wi;
      const float ti = br * wi + bi * wr;
      re[e] = xr + tr;
      im[e] = xi + ti;
      re[f] = xr - tr;
      im[f] = xi - ti;
    }
  }
}

// Stage of span 2^S >= 32 over positions b + 16k (b = BPL*l + i), twiddles from LDS.
template <int N, int S>
__device__ __forceinline__ void reg_stage_high(float (&xr)[RegGeom<N>::BPL][RegGeom<N>::KN],
                                               float (&xi)[RegGeom<N>::BPL][RegGeom<N>::KN], const float2* tw2,
                                               int b0) {
  using G = RegGeom<N>;
  constexpr int HK = (1 << (S - 1)) / 16, SP = 1 << S;
#pragma unroll
  for (int i = 0; i < G::BPL; ++i) {
#pragma unroll
    for (int k = 0; k < G::KN; ++k) {
      if (k & HK) continue;
      const float2 w = tw2[(b0 + i + 16 * (k & (HK - 1))) * (N / SP)];
      const float br = xr[i][k + HK], bi = xi[i][k + HK];
      const float tr = br * w.x - bi * w.y;
      const float ti = br * w.y + bi * w.x;
      const float ar = xr[i][k], ai = xi[i][k];
      xr[i][k] = ar + tr;
      xi[i][k] = ai + ti;
      xr[i][k + HK] = ar - tr;
      xi[i][k + HK] = ai - ti;
    }
  }
}

// Last stage (span N): the bins b + 16k below N/2 (tops) and, for i = 0, the bottom
// b + N/2, which is the Nyquist bin on lane 0.
template <int N>
__device__ __forceinline__ void reg_stage_last(float (&xr)[RegGeom<N>::BPL][RegGeom<N>::KN],
                                               float (&xi)[RegGeom<N>::BPL][RegGeom<N>::KN], const float2* tw2, int b0,
                                               float& nyr, float& nyi) {
  using G = RegGeom<N>;
#pragma unroll
  for (int i = 0; i < G::BPL; ++i) {
#pragma unroll
    for (int k = 0; k < G::KH; ++k) {
      const float2 w = tw2[b0 + i + 16 * k];
      const float br = xr[i][k + G::KH], bi = xi[i][k + G::KH];
      const float tr = br * w.x - bi * w.y;
      const float ti = br * w.y + bi * w.x;
      const float ar = xr[i][k], ai = xi[i][k];
      if (i == 0 && k == 0) {
        nyr = ar - tr;
        nyi = ai - ti;
      }
      xr[i][k] = ar + tr;
      xi[i][k] = ai + ti;
    }
  }
}

// Phase sector of (re, im) among P = 2^p sectors, the count of first-octant
// boundaries on or clockwise of the folded point as in phase_sector() above.  The side
// tests are monotone in j (binary32 rounding is monotone and the tables are), so the
// count is located from an arctangent estimate within one boundary of it and settled
// by the two side tests around the estimate; E[j + 1] = boundary j, with E[0] a test
// that always passes and E[P/8 + 1] one that fails for x > 0.  Where x is outside
// [2^-96, 2^96] (products may under- or overflow) the caller counts all boundaries.
struct Sector {
  float x, y;
  int k0;
  bool swap, neg_re, neg_im, slow;
};
__device__ __forceinline__ Sector sector_estimate(float re, float im, const float2* E, int P8, float kP) {
  Sector s;
  const float ar = __builtin_fabsf(re), ai = __builtin_fabsf(im);
  s.neg_re = re < 0.0f;
  s.neg_im = im < 0.0f;
  s.swap = ai > ar;
  s.x = __builtin_fmaxf(ar, ai);
  s.y = __builtin_fminf(ar, ai);
  const float r = s.y * __builtin_amdgcn_rcpf(s.x);
  const float t = r * __builtin_fmaf(-0.273f, r, 1.0584f);   // atan(r), |error| < 0.004
  float cf = __builtin_fmaf(t, kP, 0.5f);
  cf = __builtin_fminf(__builtin_fmaxf(cf, 0.0f), (float)P8);
  const int c = (int)cf;
  const float2 e0 = E[c], e1 = E[c + 1];
  const float s0 = e0.x * s.y - e0.y * s.x;
  const float s1 = e1.x * s.y - e1.y * s.x;
  s.k0 = c - 1 + (s0 >= 0.0f ? 1 : 0) + (s1 >= 0.0f ? 1 : 0);
  s.slow = (s.x != 0.0f) && !(s.x >= 0x1p-96f && s.x <= 0x1p96f);
  return s;
}
__device__ __forceinline__ uint32_t sector_finish(const Sector& s, int P) {
  int k = (s.x == 0.0f) ? 0 : s.k0;
  k = s.swap ? P / 4 - k : k;
  k = s.neg_re ? P / 2 - k : k;
  k = s.neg_im ? P - k : k;
  return (uint32_t)(k & (P - 1));
}
__device__ __forceinline__ void sector_count_all(Sector& s, const float2* E, int P8) {
  int n = 0;
  for (int j = 0; j < P8; ++j) {
    const float2 e = E[j + 1];
    n += (e.x * s.y - e.y * s.x >= 0.0f) ? 1 : 0;
  }
  s.k0 = n;
}

// Packs the 8 codes (bytes) of bins 8l .. 8l+7 of one field, B bits each, into the
// words at bit `pos` with LDS ORs.
__device__ __forceinline__ void or_run(uint32_t* w, uint2 bytes, int B, int pos) {
  uint64_t seg = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t c = ((i < 4 ? bytes.x : bytes.y) >> (8 * (i & 3))) & 0xffu;
    seg |= (uint64_t)c << (i * B);
  }
  const int wi = pos >> 5, sh = pos & 31;
  const uint64_t lo = seg << sh;
  const uint32_t hi = (uint32_t)((uint64_t)(uint32_t)(seg >> 32) >> (32 - sh));
  atomicOr(&w[wi], (uint32_t)lo);
  atomicOr(&w[wi + 1], (uint32_t)(lo >> 32));
  if (hi) atomicOr(&w[wi + 2], hi);
}

template <int N, bool CART>
__global__ __launch_bounds__(kBlock) void k_rfft_quantize(RArgs a) {
  using G = RegGeom<N>;
  __shared__ __align__(16) float s_buf[kWaves][kRegWaveFloats];
  __shared__ float2 s_tw[N / 2];
  __shared__ float2 s_E[kMaxSectors8 + 2];
  const RfftCodec& c = a.c;
  const int P = CART ? 8 : (1 << c.pbits), P8 = P / 8;
  for (int i = threadIdx.x; i < N / 2; i += kBlock) s_tw[i] = make_float2(a.tw.tw_c[i], a.tw.tw_s[i]);
  for (int i = threadIdx.x; i < P8 + 2; i += kBlock) {
    float2 e = make_float2(0.0f, i == P8 + 1 ? 1.0f : 0.0f);
    if (i >= 1 && i <= P8) e = make_float2(a.pt.bnd_c[i - 1], a.pt.bnd_s[i - 1]);
    s_E[i] = e;
  }
  __syncthreads();

  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rr = lane / G::LPR, l = lane % G::LPR;
  const int h = l / (G::LPR / 2);                 // half row: bins 8h .. 8h+7 of each 16
  const int b0 = G::BPL * l;
  const int words = c.words, ns = c.nscales, ng = c.ngroups, F = c.F;
  const int lg = __builtin_ctz((unsigned)c.g);
  const float kP = (float)P * 0.15915494309189535f;
  float* buf = s_buf[wv];
  float* rowb = buf + rr * G::ROWF;
  unsigned char* bytes = reinterpret_cast<unsigned char*>(buf) + kOffBytes;
  uint32_t* wbuf = reinterpret_cast<uint32_t*>(reinterpret_cast<unsigned char*>(buf) + kOffWords);
  float* cells = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(buf) + kOffCells);
  float2* cellx = reinterpret_cast<float2*>(reinterpret_cast<unsigned char*>(buf) + kOffCellX);
  float* invb = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(buf) + kOffInv);
  uint16_t* scb = reinterpret_cast<uint16_t*>(reinterpret_cast<unsigned char*>(buf) + kOffScale);
  const int rl = (int)(__brev((unsigned)l) >> (32 - (G::NB - 4)));   // bit-reversed lane

  const long long stride = (long long)gridDim.x * kWaves * G::RPW;
  for (long long base = ((long long)blockIdx.x * kWaves + wv) * G::RPW; base < a.rows; base += stride) {
    const long long row = min(base + rr, a.rows - 1);   // loads stay in bounds; stores are bounded below
    // 1. gather the row's bit-reversed positions 16l .. 16l+15
    float re[16], im[16];
    {
      const uint16_t* xp = a.x + (size_t)row * N + rl;
#pragma unroll
      for (int e = 0; e < 16; ++e) re[e] = h2f(xp[(N / 16) * rev4(e)]);
      if (a.chan || a.mean) {
        int ul, uh;
        unit_of(row, a.T, a.H, a.L, ul, uh);
        const size_t off = ((size_t)ul * a.H + uh) * N + rl;
        if (a.mean) {
#pragma unroll
          for (int e = 0; e < 16; ++e) re[e] = re[e] - a.mean[off + (N / 16) * rev4(e)];
        }
        if (a.chan) {
#pragma unroll
          for (int e = 0; e < 16; ++e) re[e] = re[e] * a.chan[off + (N / 16) * rev4(e)];
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) im[e] = 0.0f;
    }
    // 2. spans 2 .. 16 in registers
    reg_stage_low<N, 1>(re, im, a.tw);
    reg_stage_low<N, 2>(re, im, a.tw);
    reg_stage_low<N, 3>(re, im, a.tw);
    reg_stage_low<N, 4>(re, im, a.tw);
    // 3. transpose: position p at float 2p + 4(p >> 4) of the row
    {
      float4* dst = reinterpret_cast<float4*>(rowb + 36 * l);
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = make_float4(re[2 * e], im[2 * e], re[2 * e + 1], im[2 * e + 1]);
    }
    wave_lds_sync();
    float xr[G::BPL][G::KN], xi[G::BPL][G::KN];
#pragma unroll
    for (int k = 0; k < G::KN; ++k) {
      const float* src = rowb + 2 * b0 + 36 * k;
      if constexpr (G::BPL == 1) {
        const float2 v = *reinterpret_cast<const float2*>(src);
        xr[0][k] = v.x;
        xi[0][k] = v.y;
      } else {
#pragma unroll
        for (int q = 0; q < G::BPL / 2; ++q) {
          const float4 v = *reinterpret_cast<const float4*>(src + 4 * q);
          xr[2 * q][k] = v.x;
          xi[2 * q][k] = v.y;
          xr[2 * q + 1][k] = v.z;
          xi[2 * q + 1][k] = v.w;
        }
      }
    }
    // 4. spans 32 .. N in registers
    float nyr, nyi;
    reg_stage_high<N, 5>(xr, xi, s_tw, b0);
    if constexpr (G::NB >= 7) reg_stage_high<N, 6>(xr, xi, s_tw, b0);
    if constexpr (G::NB >= 8) reg_stage_high<N, 7>(xr, xi, s_tw, b0);
    reg_stage_last<N>(xr, xi, s_tw, b0, nyr, nyi);
    wave_lds_sync();   // transpose reads done before the regions below are written
    // 5. cell extremes (8 bins) and the Nyquist bin
    float mag[G::BPL][G::KH], magn = 0.0f;
    if constexpr (!CART) {
#pragma unroll
      for (int i = 0; i < G::BPL; ++i)
#pragma unroll
        for (int k = 0; k < G::KH; ++k) mag[i][k] = sqrt_rn(xr[i][k] * xr[i][k] + xi[i][k] * xi[i][k]);
      magn = sqrt_rn(nyr * nyr + nyi * nyi);
    }
#pragma unroll
    for (int k = 0; k < G::KH; ++k) {
      if constexpr (!CART) {
        float m = mag[0][k];
#pragma unroll
        for (int i = 1; i < G::BPL; ++i) m = __builtin_fmaxf(m, mag[i][k]);
        m = half_row_max<G::LPR>(m);
        if ((l & (G::LPR / 2 - 1)) == 0) cells[rr * (N / 16) + 2 * k + h] = m;
      } else {
        float rx = xr[0][k], rn = xr[0][k], ix = xi[0][k], in_ = xi[0][k];
#pragma unroll
        for (int i = 1; i < G::BPL; ++i) {
          rx = __builtin_fmaxf(rx, xr[i][k]);
          rn = __builtin_fminf(rn, xr[i][k]);
          ix = __builtin_fmaxf(ix, xi[i][k]);
          in_ = __builtin_fminf(in_, xi[i][k]);
        }
        rx = half_row_max<G::LPR>(rx);
        rn = half_row_min<G::LPR>(rn);
        ix = half_row_max<G::LPR>(ix);
        in_ = half_row_min<G::LPR>(in_);
        if ((l & (G::LPR / 2 - 1)) == 0)
          reinterpret_cast<float4*>(cells)[rr * (N / 16) + 2 * k + h] = make_float4(rx, rn, ix, in_);
      }
    }
    if (l == 0) cellx[rr] = CART ? make_float2(nyr, nyi) : make_float2(magn, 0.0f);
    wave_lds_sync();
    // 6. one lane per scale
    for (int j = l; j < ns; j += G::LPR) {
      const int comp = CART ? (j >= ng ? 1 : 0) : 0, gi = j - comp * ng;
      const int c0 = gi << (lg - 3), c1 = min(c0 + (1 << (lg - 3)), N / 16);
      const bool last = gi == ng - 1;
      uint16_t s16;
      if constexpr (!CART) {
        float m = last ? cellx[rr].x : -INFINITY;
        for (int q = c0; q < c1; ++q) m = __builtin_fmaxf(m, cells[rr * (N / 16) + q]);
        s16 = rn16(__fdiv_rn(m, (float)((1 << c.bits) - 1)));
      } else {
        const float nv = comp ? cellx[rr].y : cellx[rr].x;
        float mx = last ? nv : -INFINITY, mn = last ? nv : INFINITY;
        for (int q = c0; q < c1; ++q) {
          const float2 v = reinterpret_cast<const float2*>(cells)[(rr * (N / 16) + q) * 2 + comp];
          mx = __builtin_fmaxf(mx, v.x);
          mn = __builtin_fminf(mn, v.y);
        }
        const float m = (-mn >= mx) ? mn : mx;
        s16 = rn16(m * (-1.0f / (float)(1 << (c.bits - 1))));
      }
      scb[rr * ns + j] = s16;
      invb[rr * ns + j] = inv_scale(s16);
    }
    wave_lds_sync();
    // 7. codes of the lane's bins, as bytes
    uint32_t cA[G::KH], cB[G::KH], nA, nB;
    if constexpr (!CART) {
      const uint32_t hi = (1u << c.bits) - 1u;
      Sector sec[G::BPL][G::KH], secn;
      bool anyslow = false;
#pragma unroll
      for (int k = 0; k < G::KH; ++k) {
        const float inv = invb[rr * ns + (((16 * k) + 8 * h) >> lg)];
        cA[k] = 0;
#pragma unroll
        for (int i = 0; i < G::BPL; ++i) {
          const float q = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(mag[i][k] * inv), 0.0f), (float)hi);
          cA[k] |= (uint32_t)(int)q << (8 * i);
          sec[i][k] = sector_estimate(xr[i][k], xi[i][k], s_E, P8, kP);
          anyslow |= sec[i][k].slow;
        }
      }
      {
        const float inv = invb[rr * ns + ng - 1];
        nA = (uint32_t)(int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(magn * inv), 0.0f), (float)hi);
        secn = sector_estimate(nyr, nyi, s_E, P8, kP);
        anyslow |= secn.slow;
      }
      if (__builtin_amdgcn_ballot_w64(anyslow) != 0) {
#pragma unroll
        for (int k = 0; k < G::KH; ++k)
#pragma unroll
          for (int i = 0; i < G::BPL; ++i)
            if (sec[i][k].slow) sector_count_all(sec[i][k], s_E, P8);
        if (secn.slow) sector_count_all(secn, s_E, P8);
      }
#pragma unroll
      for (int k = 0; k < G::KH; ++k) {
        cB[k] = 0;
#pragma unroll
        for (int i = 0; i < G::BPL; ++i) cB[k] |= sector_finish(sec[i][k], P) << (8 * i);
      }
      nB = sector_finish(secn, P);
    } else {
      const float lo = -(float)(1 << (c.bits - 1)), hi = (float)((1 << (c.bits - 1)) - 1);
      const int off = 1 << (c.bits - 1);
#pragma unroll
      for (int k = 0; k < G::KH; ++k) {
        const int gi = ((16 * k) + 8 * h) >> lg;
        const float ir = invb[rr * ns + gi], ii = invb[rr * ns + ng + gi];
        cA[k] = 0;
        cB[k] = 0;
#pragma unroll
        for (int i = 0; i < G::BPL; ++i) {
          const int qr = (int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(xr[i][k] * ir), lo), hi) + off;
          const int qi = (int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(xi[i][k] * ii), lo), hi) + off;
          cA[k] |= (uint32_t)qr << (8 * i);
          cB[k] |= (uint32_t)qi << (8 * i);
        }
      }
      const float ir = invb[rr * ns + ng - 1], ii = invb[rr * ns + 2 * ng - 1];
      nA = (uint32_t)((int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(nyr * ir), lo), hi) + off);
      nB = (uint32_t)((int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(nyi * ii), lo), hi) + off);
    }
    {
      unsigned char* rA = bytes + rr * G::FA;
      unsigned char* rB = bytes + (G::RPW + rr) * G::FA;
#pragma unroll
      for (int k = 0; k < G::KH; ++k) {
        if constexpr (G::BPL == 1) {
          rA[b0 + 16 * k] = (unsigned char)cA[k];
          rB[b0 + 16 * k] = (unsigned char)cB[k];
        } else if constexpr (G::BPL == 2) {
          *reinterpret_cast<uint16_t*>(rA + b0 + 16 * k) = (uint16_t)cA[k];
          *reinterpret_cast<uint16_t*>(rB + b0 + 16 * k) = (uint16_t)cB[k];
        } else {
          *reinterpret_cast<uint32_t*>(rA + b0 + 16 * k) = cA[k];
          *reinterpret_cast<uint32_t*>(rB + b0 + 16 * k) = cB[k];
        }
      }
      if (l == 0) {
        rA[N / 2] = (unsigned char)nA;
        rB[N / 2] = (unsigned char)nB;
      }
    }
    for (int i = lane; i < G::RPW * words + 4; i += 64) wbuf[i] = 0u;
    wave_lds_sync();
    // 8. pack: lane l takes bins 8l .. 8l+7 of both fields, the last lane also bin N/2
    {
      const int BA = c.bits, BB = CART ? c.bits : c.pbits, baseB = F * c.bits;
      uint32_t* wrow = wbuf + rr * words;
      const uint2 ba = *reinterpret_cast<const uint2*>(bytes + rr * G::FA + 8 * l);
      const uint2 bb = *reinterpret_cast<const uint2*>(bytes + (G::RPW + rr) * G::FA + 8 * l);
      or_run(wrow, ba, BA, 8 * l * BA);
      or_run(wrow, bb, BB, baseB + 8 * l * BB);
      if (l == G::LPR - 1) {
        const uint32_t na = bytes[rr * G::FA + N / 2], nb = bytes[(G::RPW + rr) * G::FA + N / 2];
        const int pa = (N / 2) * BA, pb = baseB + (N / 2) * BB;
        const uint64_t va = (uint64_t)na << (pa & 31), vb = (uint64_t)nb << (pb & 31);
        atomicOr(&wrow[pa >> 5], (uint32_t)va);
        if (va >> 32) atomicOr(&wrow[(pa >> 5) + 1], (uint32_t)(va >> 32));
        atomicOr(&wrow[pb >> 5], (uint32_t)vb);
        if (vb >> 32) atomicOr(&wrow[(pb >> 5) + 1], (uint32_t)(vb >> 32));
      }
    }
    wave_lds_sync();
    // 9. the wavefront's rows are contiguous in the outputs (a token window: row by row)
    {
      const int nv = (int)min((long long)G::RPW, a.rows - base);
      if (a.T == a.Tout) {
        uint32_t* cw = a.codes + (size_t)base * words;
        for (int i = lane; i < nv * words; i += 64) cw[i] = wbuf[i];
        uint16_t* sw = a.scales + (size_t)base * ns;
        for (int i = lane; i < nv * ns; i += 64) sw[i] = scb[i];
      } else {
        for (int r = 0; r < nv; ++r) {
          const long long u = (base + r) / a.T;
          const long long orow = u * a.Tout + a.t0 + (base + r - u * a.T);
          for (int i = lane; i < words; i += 64) a.codes[(size_t)orow * words + i] = wbuf[r * words + i];
          for (int i = lane; i < ns; i += 64) a.scales[(size_t)orow * ns + i] = scb[r * ns + i];
        }
      }
    }
    wave_lds_sync();
  }
}

// Inverse: spectrum of one row (from its codes) -> real values in re[] (times 1/N).
__device__ void rfft_decode_row(const RArgs& a, const LdsTables& ltab, long long row, bool active, float* re, float* im,
                                int lane) {
  const RfftCodec& c = a.c;
  const int N = c.N, F = c.F, nb = __builtin_ctz((unsigned)N);
  const uint32_t* w = a.codes + (size_t)row * c.words;
  const uint16_t* s = a.scales + (size_t)row * c.nscales;
  for (int f = lane; f < F; f += 64) {
    float zr = 0.0f, zi = 0.0f;
    if (active) rfft_bin_value(c, w, s, f, ltab.dirc, ltab.dirs, zr, zi);
    re[bitrev(f, nb)] = zr;
    im[bitrev(f, nb)] = zi;
    if (f >= 1 && f < N / 2) {
      re[bitrev(N - f, nb)] = zr;
      im[bitrev(N - f, nb)] = -zi;
    }
  }
  wave_lds_sync();
  fft_lds(re, im, N, ltab.twc, ltab.tws, true, lane, 64);
}

__global__ __launch_bounds__(kBlock) void k_rfft_dequant(RArgs a) {
  __shared__ float s_re[kWaves][kMaxN], s_im[kWaves][kMaxN];
  __shared__ LdsTables ltab;
  load_tables(a, ltab);
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int N = a.c.N;
  const float invN = 1.0f / (float)N;
  for (long long base = (long long)blockIdx.x * kWaves; base < a.rows; base += (long long)gridDim.x * kWaves) {
    const long long row = base + wv;
    const bool active = row < a.rows;
    rfft_decode_row(a, ltab, row, active, s_re[wv], s_im[wv], lane);
    if (active) {
      const float* cp = nullptr;
      const float* mp = nullptr;
      if (a.chan || a.mean) {
        int l, h;
        unit_of(row, a.T, a.H, a.L, l, h);
        if (a.chan) cp = a.chan + ((size_t)l * a.H + h) * N;
        if (a.mean) mp = a.mean + ((size_t)l * a.H + h) * N;
      }
      for (int n = lane; n < N; n += 64) {
        float v = s_re[wv][n] * invN;
        if (cp) v = __fdiv_rn(v, cp[n]);
        if (mp) v = v + mp[n];
        a.xhat[(size_t)row * N + n] = v;
      }
    }
    wave_lds_sync();
  }
}

// Per-unit squared error of rFFT-coded keys against fp16: partial sums per block.
__global__ __launch_bounds__(kBlock) void k_rfft_kverr(RArgs a, double* part, int chunks) {
  __shared__ float s_re[kWaves][kMaxN], s_im[kWaves][kMaxN];
  __shared__ LdsTables ltab;
  load_tables(a, ltab);
  __shared__ double s_red[2][kBlock];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int N = a.c.N;
  const float invN = 1.0f / (float)N;
  const long long unit = blockIdx.y;
  const int T = a.T;
  const int per = (T + chunks - 1) / chunks;
  const int t0 = blockIdx.x * per, t1 = min(T, t0 + per);
  double se = 0.0, sx = 0.0;
  const float* cp = nullptr;
  const float* mp = nullptr;
  {
    const int h = (int)(unit % a.H), l = (int)((unit / a.H) % a.L);
    if (a.chan) cp = a.chan + ((size_t)l * a.H + h) * N;
    if (a.mean) mp = a.mean + ((size_t)l * a.H + h) * N;
  }
  for (int tb = t0; tb < t1; tb += kWaves) {
    const int t = tb + wv;
    const bool active = t < t1;
    const long long row = unit * T + t;
    rfft_decode_row(a, ltab, row, active, s_re[wv], s_im[wv], lane);
    if (active) {
      for (int n = lane; n < N; n += 64) {
        float v = s_re[wv][n] * invN;
        if (cp) v = __fdiv_rn(v, cp[n]);
        if (mp) v = v + mp[n];
        const double x = (double)h2f(a.x[(size_t)row * N + n]);
        const double d = (double)v - x;
        se += d * d;
        sx += x * x;
      }
    }
    wave_lds_sync();
  }
  s_red[0][threadIdx.x] = se;
  s_red[1][threadIdx.x] = sx;
  __syncthreads();
  for (int st = kBlock / 2; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) {
      s_red[0][threadIdx.x] += s_red[0][threadIdx.x + st];
      s_red[1][threadIdx.x] += s_red[1][threadIdx.x + st];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    part[(unit * chunks + blockIdx.x) * 2 + 0] = s_red[0][0];
    part[(unit * chunks + blockIdx.x) * 2 + 1] = s_red[1][0];
  }
}

static RArgs make_rargs(const kvq_packed& p) {
  RArgs a{};
  a.codes = p.codes;
  a.scales = p.scales;
  a.chan = p.chan_scale;
  a.mean = p.mean;
  a.rows = (long long)p.shape.batch * p.shape.layers * p.shape.heads * p.shape.tokens;
  a.T = p.shape.tokens;
  a.Tout = p.shape.tokens;
  a.t0 = 0;
  a.H = p.shape.heads;
  a.L = p.shape.layers;
  RfftCodec& c = a.c;
  c.cb = p.codec.codebook;
  c.N = p.shape.head_dim;
  c.F = c.N / 2 + 1;
  c.bits = p.codec.bits;
  c.pbits = (c.cb == KVQ_RFFT_POLAR) ? p.codec.aux_bits : 0;
  c.g = p.codec.group;
  c.ngroups = (c.F + c.g - 1) / c.g;
  c.nscales = (c.cb == KVQ_RFFT_POLAR) ? c.ngroups : 2 * c.ngroups;
  const long bits = (c.cb == KVQ_RFFT_POLAR) ? (long)c.F * (c.bits + c.pbits) : 2L * c.F * c.bits;
  c.words = (int)((bits + 31) / 32);
  host_fft_tables(c.N, &a.tw);
  host_phase_tables(c.cb == KVQ_RFFT_POLAR ? (1 << c.pbits) : 8, &a.pt);
  return a;
}

static unsigned rgrid(long long rows) {
  long long b = (rows + kWaves - 1) / kWaves;
  if (b > 2048) b = 2048;
  return (unsigned)(b < 1 ? 1 : b);
}

static hipError_t launch_rfft_quantize_args(const RArgs& a, hipStream_t st) {
  const int N = a.c.N, rpw = 64 / (N / 16);
  long long blocks = (a.rows + (long long)kWaves * rpw - 1) / ((long long)kWaves * rpw);
  const unsigned grid = (unsigned)(blocks > 4096 ? 4096 : blocks);
  const bool cart = a.c.cb == KVQ_RFFT_CART;
  if (N == 64) {
    if (cart) k_rfft_quantize<64, true><<<grid, kBlock, 0, st>>>(a);
    else k_rfft_quantize<64, false><<<grid, kBlock, 0, st>>>(a);
  } else if (N == 128) {
    if (cart) k_rfft_quantize<128, true><<<grid, kBlock, 0, st>>>(a);
    else k_rfft_quantize<128, false><<<grid, kBlock, 0, st>>>(a);
  } else if (N == 256) {
    if (cart) k_rfft_quantize<256, true><<<grid, kBlock, 0, st>>>(a);
    else k_rfft_quantize<256, false><<<grid, kBlock, 0, st>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rfft_quantize(const uint16_t* x, const kvq_packed& p, hipStream_t st) {
  RArgs a = make_rargs(p);
  a.x = x;
  if (a.rows == 0) return hipSuccess;
  return launch_rfft_quantize_args(a, st);
}

hipError_t launch_rfft_quantize_tokens(const uint16_t* x, const kvq_packed& p, int t0, int n, hipStream_t st) {
  RArgs a = make_rargs(p);
  a.x = x;
  a.T = n;
  a.t0 = t0;
  a.rows = (long long)p.shape.batch * p.shape.layers * p.shape.heads * n;
  if (a.rows == 0) return hipSuccess;
  return launch_rfft_quantize_args(a, st);
}

hipError_t launch_rfft_dequant(const kvq_packed& p, float* xhat, hipStream_t st) {
  RArgs a = make_rargs(p);
  a.xhat = xhat;
  if (a.rows == 0) return hipSuccess;
  k_rfft_dequant<<<rgrid(a.rows), kBlock, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_rfft_kverr(const uint16_t* x, const kvq_packed& p, double* part, int chunks, hipStream_t st) {
  RArgs a = make_rargs(p);
  a.x = x;
  const long long units = (long long)p.shape.batch * p.shape.layers * p.shape.heads;
  if (units == 0 || a.T == 0) return hipSuccess;
  k_rfft_kverr<<<dim3(chunks, (unsigned)units), kBlock, 0, st>>>(a, part, chunks);
  return hipGetLastError();
}

}  // namespace kvq

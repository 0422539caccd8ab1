// rFFT physical codecs ([FMAG-R] HF forum thread "Fourier Magnitude KV Cache
// Quantization", Colab-probe reply: rFFT + packed magnitude index + packed
// phase-angle index, and the real/imaginary control): quantise+pack and
// dequantise kernels.  One wavefront per row, in an LDS region of its own, so the
// per-row steps need no block barrier; the transform runs in LDS.
#include "kvq_rfft.hpp"

namespace kvq {

struct RArgs {
  const uint16_t* x;
  float* xhat;
  uint32_t* codes;
  uint16_t* scales;
  const float* chan;
  long long rows;
  int T, H, L;
  RfftCodec c;
  FftTables tw;
  PhaseTables pt;
};

constexpr int kWaves = kBlock / 64;
constexpr int kMaxN = 256;
constexpr int kMaxWords = 72;

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

__device__ __forceinline__ void unit_of(long long row, int T, int H, int L, int& l, int& h) {
  const long long u = row / T;
  h = (int)(u % H);
  l = (int)((u / H) % L);
}

__global__ __launch_bounds__(kBlock) void k_rfft_quantize(RArgs a) {
  __shared__ float s_re[kWaves][kMaxN], s_im[kWaves][kMaxN];
  __shared__ float s_val[kWaves][2][kMaxN / 2 + 1];
  __shared__ float s_inv[kWaves][64];
  __shared__ uint16_t s_sc[kWaves][64];
  __shared__ uint32_t s_w[kWaves][kMaxWords];
  __shared__ LdsTables ltab;
  load_tables(a, ltab);
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const RfftCodec& c = a.c;
  const int N = c.N, F = c.F, nb = __builtin_ctz((unsigned)N);
  float* re = s_re[wv];
  float* im = s_im[wv];
  for (long long base = (long long)blockIdx.x * kWaves; base < a.rows; base += (long long)gridDim.x * kWaves) {
    const long long row = base + wv;
    const bool active = row < a.rows;
    const float* cp = nullptr;
    if (active && a.chan) {
      int l, h;
      unit_of(row, a.T, a.H, a.L, l, h);
      cp = a.chan + ((size_t)l * a.H + h) * N;
    }
    for (int n = lane; n < N; n += 64) {
      float v = active ? h2f(a.x[(size_t)row * N + n]) : 0.0f;
      if (cp) v = v * cp[n];
      re[bitrev(n, nb)] = v;
      im[bitrev(n, nb)] = 0.0f;
    }
    wave_lds_sync();
    fft_lds(re, im, N, ltab.twc, ltab.tws, false, lane, 64);
    // per-bin value(s) to code
    for (int f = lane; f < F; f += 64) {
      if (c.cb == KVQ_RFFT_POLAR) {
        s_val[wv][0][f] = __fsqrt_rn(re[f] * re[f] + im[f] * im[f]);
      } else {
        s_val[wv][0][f] = re[f];
        s_val[wv][1][f] = im[f];
      }
    }
    for (int k = lane; k < c.words; k += 64) s_w[wv][k] = 0u;
    wave_lds_sync();
    // group scales: one lane per (component, group), serial extreme over the bins
    if (lane < c.nscales) {
      const int comp = lane / c.ngroups, gi = lane - comp * c.ngroups;
      const int f0 = gi * c.g, f1 = min(f0 + c.g, F);
      const float* v = s_val[wv][comp];
      uint16_t s16;
      if (c.cb == KVQ_RFFT_POLAR) {
        float m = v[f0];
        for (int f = f0 + 1; f < f1; ++f) m = __builtin_fmaxf(m, v[f]);
        s16 = rn16(__fdiv_rn(m, (float)((1 << c.bits) - 1)));
      } else {
        float mx = v[f0], mn = v[f0];
        for (int f = f0 + 1; f < f1; ++f) { mx = __builtin_fmaxf(mx, v[f]); mn = __builtin_fminf(mn, v[f]); }
        const float m = (-mn >= mx) ? mn : mx;
        s16 = rn16(m * (-1.0f / (float)(1 << (c.bits - 1))));
      }
      s_sc[wv][lane] = s16;
      s_inv[wv][lane] = inv_scale(s16);
    }
    wave_lds_sync();
    for (int f = lane; f < F; f += 64) {
      const int gi = f / c.g;
      if (c.cb == KVQ_RFFT_POLAR) {
        const float hi = (float)((1 << c.bits) - 1);
        const float q = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(s_val[wv][0][f] * s_inv[wv][gi]), 0.0f), hi);
        const uint32_t qm = (uint32_t)(int)q;
        const uint32_t k = (uint32_t)phase_sector(re[f], im[f], 1 << c.pbits, ltab.bndc, ltab.bnds);
        const int p0 = f * c.bits, p1 = F * c.bits + f * c.pbits;
        atomicOr(&s_w[wv][p0 >> 5], qm << (p0 & 31));
        if ((p0 & 31) + c.bits > 32) atomicOr(&s_w[wv][(p0 >> 5) + 1], qm >> (32 - (p0 & 31)));
        atomicOr(&s_w[wv][p1 >> 5], k << (p1 & 31));
        if ((p1 & 31) + c.pbits > 32) atomicOr(&s_w[wv][(p1 >> 5) + 1], k >> (32 - (p1 & 31)));
      } else {
        const float lo = -(float)(1 << (c.bits - 1)), hi = (float)((1 << (c.bits - 1)) - 1);
        const int off = 1 << (c.bits - 1);
#pragma unroll
        for (int comp = 0; comp < 2; ++comp) {
          const float t = s_val[wv][comp][f] * s_inv[wv][comp * c.ngroups + gi];
          const uint32_t q = (uint32_t)((int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(t), lo), hi) + off);
          const int p = (comp * F + f) * c.bits;
          atomicOr(&s_w[wv][p >> 5], q << (p & 31));
          if ((p & 31) + c.bits > 32) atomicOr(&s_w[wv][(p >> 5) + 1], q >> (32 - (p & 31)));
        }
      }
    }
    wave_lds_sync();
    if (active) {
      for (int k = lane; k < c.words; k += 64) a.codes[(size_t)row * c.words + k] = s_w[wv][k];
      if (lane < c.nscales) a.scales[(size_t)row * c.nscales + lane] = s_sc[wv][lane];
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
      if (a.chan) {
        int l, h;
        unit_of(row, a.T, a.H, a.L, l, h);
        cp = a.chan + ((size_t)l * a.H + h) * N;
      }
      for (int n = lane; n < N; n += 64) {
        float v = s_re[wv][n] * invN;
        if (cp) v = __fdiv_rn(v, cp[n]);
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
  if (a.chan) {
    const int h = (int)(unit % a.H), l = (int)((unit / a.H) % a.L);
    cp = a.chan + ((size_t)l * a.H + h) * N;
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
  a.rows = (long long)p.shape.batch * p.shape.layers * p.shape.heads * p.shape.tokens;
  a.T = p.shape.tokens;
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

hipError_t launch_rfft_quantize(const uint16_t* x, const kvq_packed& p, hipStream_t st) {
  RArgs a = make_rargs(p);
  a.x = x;
  if (a.rows == 0) return hipSuccess;
  k_rfft_quantize<<<rgrid(a.rows), kBlock, 0, st>>>(a);
  return hipGetLastError();
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

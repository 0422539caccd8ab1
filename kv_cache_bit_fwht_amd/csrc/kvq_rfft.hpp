// rFFT physical codecs along head_dim: device helpers.
//
// [FMAG-R] (HF forum thread "Fourier Magnitude KV Cache Quantization", the
// Colab-probe reply, physical-codec paragraph): real K -> rFFT (D/2 + 1 bins) ->
// packed magnitude index + packed phase-angle index -> irFFT; and the
// real/imaginary control at the same payload.  Readings (the page fixes none):
// radix-2 decimation-in-time FFT on bit-reversed input with binary32 twiddles
// rounded from fp64, complex product (RN(RN(ac)-RN(bd)), RN(RN(ad)+RN(bc))),
// magnitude RN(sqrt(RN(RN(re^2)+RN(im^2)))) on an unsigned grid with one fp16
// scale per `group` bins (last group ragged), phase = nearest of 2^p sectors
// decided by sign flips into the first octant and binary32 side tests (no
// atan2); Cartesian: real and imaginary rows on the signed absmax grid.
#pragma once

#include "kvq_internal.hpp"

namespace kvq {

struct RfftCodec {
  int cb;        // KVQ_RFFT_POLAR or KVQ_RFFT_CART
  int N;         // head_dim
  int F;         // N/2 + 1 bins
  int bits;      // magnitude bits (polar) or component bits (Cartesian)
  int pbits;     // phase bits (polar)
  int g;         // bins per scale
  int ngroups;   // ceil(F / g)
  int words;     // uint32 words per row
  int nscales;   // scales per row
};

__device__ __forceinline__ int bitrev(int i, int nb) { return (int)(__brev((unsigned)i) >> (32 - nb)); }

__device__ __forceinline__ int phase_sector(float re, float im, int P, const float* bc, const float* bs) {
  const bool neg_im = im < 0.0f;
  const float ai = neg_im ? -im : im;
  const bool neg_re = re < 0.0f;
  const float ar = neg_re ? -re : re;
  const bool swap = ai > ar;
  const float x = swap ? ai : ar;
  const float y = swap ? ar : ai;
  int k0 = 0;
  for (int j = 0; j < P / 8; ++j) {
    const float side = bc[j] * y - bs[j] * x;
    k0 += (side >= 0.0f) ? 1 : 0;
  }
  if (x == 0.0f) k0 = 0;
  int k = swap ? P / 4 - k0 : k0;
  k = neg_re ? P / 2 - k : k;
  k = neg_im ? P - k : k;
  return k & (P - 1);
}

// Extract `nb` bits starting at bit `pos` of a row's uint32 words.
__device__ __forceinline__ uint32_t get_bits(const uint32_t* w, int pos, int nb) {
  const int wi = pos >> 5, sh = pos & 31;
  uint32_t v = w[wi] >> sh;
  if (sh + nb > 32) v |= w[wi + 1] << (32 - sh);
  return v & ((1u << nb) - 1u);
}

// Dequantised spectrum value of bin f of one row (codes `w`, fp16 scales `s`).
__device__ __forceinline__ void rfft_bin_value(const RfftCodec& c, const uint32_t* w, const uint16_t* s, int f,
                                               const float* dir_c, const float* dir_s, float& re, float& im) {
  const int gi = f / c.g;
  if (c.cb == KVQ_RFFT_POLAR) {
    const uint32_t qm = get_bits(w, f * c.bits, c.bits);
    const uint32_t k = get_bits(w, c.F * c.bits + f * c.pbits, c.pbits);
    const float mu = (float)qm * h2f(s[gi]);
    re = mu * dir_c[k];
    im = mu * dir_s[k];
  } else {
    const int off = 1 << (c.bits - 1);
    const uint32_t qr = get_bits(w, f * c.bits, c.bits);
    const uint32_t qi = get_bits(w, (c.F + f) * c.bits, c.bits);
    re = (float)((int)qr - off) * h2f(s[gi]);
    im = (float)((int)qi - off) * h2f(s[c.ngroups + gi]);
  }
}

// In-place radix-2 DIT FFT of N complex values in LDS (already in bit-reversed
// order).  Butterflies are spread over the `nl` lanes [0, nl) of one wavefront,
// which owns the arrays; each stage ends with a wavefront-local LDS sync.  conj
// selects conjugate twiddles (the inverse transform, without the 1/N).
__device__ __forceinline__ void fft_lds(float* re, float* im, int N, const float* twc, const float* tws, bool conj,
                                        int lane,
                                        int nl) {
  for (int span = 2; span <= N; span <<= 1) {
    const int half = span >> 1, step = N / span;
    {
      for (int b = lane; b < N / 2; b += nl) {
        const int blk = b / half, jj = b - blk * half;
        const int top = blk * span + jj, bot = top + half;
        const float wr = twc[jj * step];
        const float wi = conj ? -tws[jj * step] : tws[jj * step];
        const float br = re[bot], bi = im[bot];
        const float tr = br * wr - bi * wi;
        const float ti = br * wi + bi * wr;
        const float xr = re[top], xi = im[top];
        re[bot] = xr - tr;
        im[bot] = xi - ti;
        re[top] = xr + tr;
        im[top] = xi + ti;
      }
    }
    wave_lds_sync();
  }
}

}  // namespace kvq

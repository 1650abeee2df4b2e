// dit_ln.hpp -- LayerNorm + AdaLN modulate helpers shared by the LN kernel
// (dit_ln.hip) and the gated residual + LayerNorm/AdaLN producer
// (dit_gate_ln.hip): two-pass statistics and the modulated output, with an
// optional E4M3 copy; and the statistics of a row published in LDS by the
// split-row layout (dit_split.hpp).
#pragma once

#include "dit_rows.hpp"
#include "dit_split.hpp"

namespace dit {

// ---------------------------------------------------------------------------
// LayerNorm + AdaLN modulate, as helpers on a row held by the wave.
// ---------------------------------------------------------------------------
// Two-pass statistics in order R: returns rho = 1 / sqrt(var + eps) and
// leaves the deviations x - mean (binary32) in d.
template <int NC, int MODE>
__device__ __forceinline__ float ln_stats(const V8 (&xv)[NC], float (&d)[NC][8], int lane,
                                          int dim, float eps) {
  float p = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (valid<NC>(c, lane, dim))
#pragma unroll
      for (int j = 0; j < 8; ++j) p = p + elem(xv[c], j);
  const float mean = wave_sum(p) / (float)dim;

  float q = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (valid<NC>(c, lane, dim))
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        d[c][j] = elem(xv[c], j) - mean;
        if (MODE == kLossless)
          q = q + d[c][j] * d[c][j];
        else
          q = fmaf(d[c][j], d[c][j], q);
      }
  const float var = wave_sum(q) / (float)dim;
  return rsqrt_mode<MODE>(var + eps);
}

// bf(1 + scale) of each of the 8 values.
__device__ __forceinline__ void one_plus8(const V8 &s, float (&f)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = 1.0f + lo(s.w[k]);
    f[2 * k + 1] = 1.0f + hi(s.w[k]);
    round2(f[2 * k], f[2 * k + 1]);
  }
}

// One output vector: bf(bf(bf(d * rho) * s1) + shift) of the deviations d,
// with bf(1 + scale) and shift as binary32 values.
__device__ __forceinline__ V8 ln_modulate_vec(const float (&d)[8], float rho, const float (&s1)[8],
                                              const float (&sh)[8]) {
  V8 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float n0 = d[2 * k] * rho, n1 = d[2 * k + 1] * rho;
    round2(n0, n1);                                             // LayerNorm output
    float p0 = n0 * s1[2 * k], p1 = n1 * s1[2 * k + 1];
    round2(p0, p1);                                             // product
    o.w[k] = pack(p0 + sh[2 * k], p1 + sh[2 * k + 1]);          // + shift
  }
  return o;
}

// Stores output vector o at element offset col of the row; F8: also its E4M3
// copy, qr = 1 / (double)s (dit_device.hpp, div_by_scale).
template <bool F8>
__device__ __forceinline__ void ln_store(uint16_t *orow, uint8_t *qrow, double qr, int col,
                                         const V8 &o) {
  store8(orow + col, o);
  if (F8) {
    uint32_t q0, q1;
    quant8(o.w, qr, q0, q1);
    store8b(qrow + col, q0, q1);
  }
}

// The modulated row; mod(c, s1, sh) gives chunk c's bf(1 + scale) and shift
// as binary32 values.
template <int NC, bool F8, class Mod>
__device__ __forceinline__ void ln_modulate_out(uint16_t *orow, uint8_t *qrow, double qr,
                                                const float (&d)[NC][8], float rho, int lane,
                                                int dim, Mod mod) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (!valid<NC>(c, lane, dim)) continue;
    float s1[8], sh[8];
    mod(c, s1, sh);
    ln_store<F8>(orow, qrow, qr, 512 * c + 8 * lane, ln_modulate_vec(d[c], rho, s1, sh));
  }
}

// Split-row layout, wave 0: the two passes of ln_stats, with the same
// operations in the same order, over the row published in LDS (xs);
// leaves st[0] = mean, st[1] = rho.  The deviations are formed again by the
// waves that write the output, bit for bit the same binary32 differences.
template <int NC, int MODE>
__device__ __forceinline__ void split_ln_stats(const uint4 *xs, float *st, int lane, int dim,
                                               float eps) {
  float p = 0.0f;
  split_walk<NC>(xs, lane, [&](int c, const V8 &v) {
    if (valid<NC>(c, lane, dim))
#pragma unroll
      for (int j = 0; j < 8; ++j) p = p + elem(v, j);
  });
  const float mean = wave_sum(p) / (float)dim;

  float q = 0.0f;
  split_walk<NC>(xs, lane, [&](int c, const V8 &v) {
    if (valid<NC>(c, lane, dim))
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float d = elem(v, j) - mean;
        if (MODE == kLossless)
          q = q + d * d;
        else
          q = fmaf(d, d, q);
      }
  });
  const float var = wave_sum(q) / (float)dim;
  if (lane == 0) {
    st[0] = mean;
    st[1] = rsqrt_mode<MODE>(var + eps);
  }
}

// Deviations x - mean of one vector.
__device__ __forceinline__ void deviations8(const V8 &x, float mean, float (&d)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) d[j] = elem(x, j) - mean;
}

}  // namespace dit

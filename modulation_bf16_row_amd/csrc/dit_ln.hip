// dit_ln.hip -- gfx950 LayerNorm + AdaLN modulate, with or without its E4M3 copy.
// Geometry, staging and launch shapes: dit_rows.hpp (per-batch modulation)
// and dit_split.hpp (otherwise); LN helpers: dit_ln.hpp.
#include "dit_ln.hpp"

namespace dit {

// ---------------------------------------------------------------------------
// LayerNorm + AdaLN modulate, per-batch modulation (the staged row layout,
// dit_rows.hpp); F8: also the E4M3 copy out8 = E4M3(out / s).
// LDS: [0] = bf(1 + scale), [1] = shift, binary32.
// ---------------------------------------------------------------------------
template <int NC, int MODE, bool F8>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_ln_modulate(LnModArgs a) {
  extern __shared__ float4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  constexpr int kRow = stage_vecs<NC>();
  const Span sp = mod_spans(a.per_mod, a.rows_per_wave, a.blocks_per_mod);
  const double qr = F8 ? 1.0 / (double)*a.fp8_scale : 1.0;   // E4M3 copy: 1 / scale
  V8 gs[stage_iters<NC>()], gf[stage_iters<NC>()], xv[NC];
  stage_fetch<NC>(gs, a.scale + sp.m * a.mod_rs, dim);
  stage_fetch<NC>(gf, a.shift + sp.m * a.mod_rs, dim);
  if (sp.begin < sp.end) load_row<NC, kNtLn>(xv, a.x + sp.begin * a.x_rs, lane, dim);
  stage_each<NC>(dim, [&](int i, int v) {
    float s1[8], sh[8];
    one_plus8(gs[i], s1);
    unpack8(gf[i], sh);
    stage_put(lds, v, s1);
    stage_put(lds + kRow, v, sh);
  });
  __syncthreads();

  for (int64_t r = sp.begin; r < sp.end; ++r) {
    if (r != sp.begin) load_row<NC, kNtLn>(xv, a.x + r * a.x_rs, lane, dim);
    float d[NC][8];
    const float rho = ln_stats<NC, MODE>(xv, d, lane, dim, a.eps);
    uint16_t *orow = a.out + r * a.out_rs;
    uint8_t *qrow = F8 ? a.out8 + r * a.out8_rs : nullptr;
    phase_barrier();
    ln_modulate_out<NC, F8>(orow, qrow, qr, d, rho, lane, dim,
                            [&](int c, float (&s1)[8], float (&sh)[8]) {
                              stage_get(lds, c, lane, s1);
                              stage_get(lds + kRow, c, lane, sh);
                            });
  }
}

// ---------------------------------------------------------------------------
// The same operation in the split-row layout (dit_split.hpp): one row per
// workgroup, two chunks per wave; wave 0 takes the statistics of the row
// published in LDS.  Modulation rows read by one row only (per-token) are
// streamed.
// ---------------------------------------------------------------------------
template <int NC, int MODE, bool F8>
__global__ DIT_SPLIT_KERNEL void k_ln_modulate_split(LnModArgs a) {
  __shared__ uint4 xs[NC * 64];
  __shared__ float st[2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, dim = (int)a.dim;
  const double qr = F8 ? 1.0 / (double)*a.fp8_scale : 1.0;   // E4M3 copy: 1 / scale
  const bool per_token = a.per_mod == 1;
  for (int64_t r = blockIdx.x; r < a.rows; r += gridDim.x) {
    const int64_t m = r / a.per_mod;
    V8 xv[kSplitChunks], sc[kSplitChunks], sf[kSplitChunks];
    split_load<NC, kNtLn>(xv, a.x + r * a.x_rs, w, lane, dim);
    if (per_token) {
      split_load<NC, true>(sc, a.scale + m * a.mod_rs, w, lane, dim);
      split_load<NC, true>(sf, a.shift + m * a.mod_rs, w, lane, dim);
    } else {
      split_load<NC, false>(sc, a.scale + m * a.mod_rs, w, lane, dim);
      split_load<NC, false>(sf, a.shift + m * a.mod_rs, w, lane, dim);
    }
    split_publish<NC>(xs, xv, w, lane);
    __syncthreads();
    if (w == 0) split_ln_stats<NC, MODE>(xs, st, lane, dim, a.eps);
    __syncthreads();
    const float mean = st[0], rho = st[1];
    uint16_t *orow = a.out + r * a.out_rs;
    uint8_t *qrow = F8 ? a.out8 + r * a.out8_rs : nullptr;
#pragma unroll
    for (int k = 0; k < kSplitChunks; ++k) {
      const int c = split_chunk(w, k);
      if (!split_has<NC>(c, lane, dim)) continue;
      float d[8], s1[8], sh[8];
      deviations8(xv[k], mean, d);
      one_plus8(sc[k], s1);
      unpack8(sf[k], sh);
      ln_store<F8>(orow, qrow, qr, 512 * c + 8 * lane, ln_modulate_vec(d, rho, s1, sh));
    }
    __syncthreads();                                   // xs and st serve the next row
  }
}

template <int MODE, bool F8>
static hipError_t ln_dispatch(LnModArgs a, hipStream_t s) {
  const Shape sh = row_shape(a.rows, a.per_mod, a.dim, 2);
  a.rows_per_wave = sh.rows_per_wave;
  a.blocks_per_mod = sh.blocks_per_mod;
#define X(N)                                                                               \
  case N:                                                                                  \
    if (sh.staged)                                                                         \
      DIT_LAUNCH((k_ln_modulate<N, MODE, F8>), sh.grid, dim3(kThreads),              \
                 stage_bytes(a.dim, 2), s, a);                                             \
    else                                                                                   \
      DIT_LAUNCH((k_ln_modulate_split<N, MODE, F8>), split_grid(a.rows),                   \
                 dim3(64 * split_waves<N>()), 0, s, a);                                    \
    break;
  DIT_ROW_DISPATCH();
#undef X
}

hipError_t launch_ln_modulate(const LnModArgs &a, int mode, hipStream_t s) {
  if (a.out8)
    return mode == kFast ? ln_dispatch<kFast, true>(a, s) : ln_dispatch<kLossless, true>(a, s);
  return mode == kFast ? ln_dispatch<kFast, false>(a, s) : ln_dispatch<kLossless, false>(a, s);
}

}  // namespace dit

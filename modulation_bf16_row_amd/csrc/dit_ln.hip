// dit_ln.hip -- gfx950 LayerNorm + AdaLN modulate, with or without its E4M3 copy.
// Geometry, staging and launch shapes: dit_rows.hpp; LN helpers: dit_ln.hpp.
#include "dit_ln.hpp"

namespace dit {

// ---------------------------------------------------------------------------
// LayerNorm + AdaLN modulate; F8: also the E4M3 copy out8 = E4M3(out / s).
// LDS (staged): [0] = bf(1 + scale), [1] = shift, binary32.
// ---------------------------------------------------------------------------
template <int NC, int MODE, bool STAGED, bool F8>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_ln_modulate(LnModArgs a) {
  extern __shared__ float4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  constexpr int kRow = stage_vecs<NC>();
  const Span sp = STAGED ? mod_spans(a.per_mod, a.rows_per_wave, a.blocks_per_mod)
                         : spans(a.rows, a.rows_per_wave);
  const double qr = F8 ? 1.0 / (double)*a.fp8_scale : 1.0;   // E4M3 copy: 1 / scale
  V8 gs[stage_iters<NC>()], gf[stage_iters<NC>()], xv[NC];
  if (STAGED) {
    stage_fetch<NC>(gs, a.scale + sp.m * a.mod_rs, dim);
    stage_fetch<NC>(gf, a.shift + sp.m * a.mod_rs, dim);
  }
  if (STAGED && sp.begin < sp.end) load_row<NC, kNtLn>(xv, a.x + sp.begin * a.x_rs, lane, dim);
  if (STAGED) {
    stage_each<NC>(dim, [&](int i, int v) {
      float s1[8], sh[8];
      one_plus8(gs[i], s1);
      unpack8(gf[i], sh);
      stage_put(lds, v, s1);
      stage_put(lds + kRow, v, sh);
    });
    __syncthreads();
  }

  for (int64_t r = sp.begin; r < sp.end; ++r) {
    V8 sc[NC], sf[NC];
    if (!STAGED || r != sp.begin) load_row<NC, kNtLn>(xv, a.x + r * a.x_rs, lane, dim);
    if (!STAGED) {
      const int64_t m = r / a.per_mod;
      load_mod_row<NC>(sc, a.scale + m * a.mod_rs, lane, dim, a.per_mod == 1);
      load_mod_row<NC>(sf, a.shift + m * a.mod_rs, lane, dim, a.per_mod == 1);
    }
    float d[NC][8];
    const float rho = ln_stats<NC, MODE>(xv, d, lane, dim, a.eps);
    uint16_t *orow = a.out + r * a.out_rs;
    uint8_t *qrow = F8 ? a.out8 + r * a.out8_rs : nullptr;
    if (STAGED) {
      phase_barrier();
      ln_modulate_out<NC, F8>(orow, qrow, qr, d, rho, lane, dim,
                              [&](int c, float (&s1)[8], float (&sh)[8]) {
                                stage_get(lds, c, lane, s1);
                                stage_get(lds + kRow, c, lane, sh);
                              });
    } else {
      ln_modulate_out<NC, F8>(orow, qrow, qr, d, rho, lane, dim,
                              [&](int c, float (&s1)[8], float (&sh)[8]) {
                                one_plus8(sc[c], s1);
                                unpack8(sf[c], sh);
                              });
    }
  }
}

template <int MODE, bool F8>
static hipError_t ln_dispatch(LnModArgs a, hipStream_t s) {
  const Shape sh = row_shape(a.rows, a.per_mod, a.dim, 2);
  a.rows_per_wave = sh.rows_per_wave;
  a.blocks_per_mod = sh.blocks_per_mod;
#define X(N)                                                                              \
  case N:                                                                                 \
    DIT_ROW_LAUNCH((k_ln_modulate<N, MODE, true, F8>), (k_ln_modulate<N, MODE, false, F8>), \
                   stage_bytes(a.dim, 2), 0);                                             \
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

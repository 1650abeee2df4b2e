// dit_gate_ln.hip -- gfx950 gated residual + LayerNorm/AdaLN producer, with or
// without its E4M3 copy.
// Geometry, staging and launch shapes: dit_rows.hpp; LN helpers: dit_ln.hpp.
#include "dit_ln.hpp"

namespace dit {

// ---------------------------------------------------------------------------
// Gated residual + LayerNorm + AdaLN modulate: r' = bf(residual + bf(gate * y))
// is written to out_res, and LN + modulate of r' to out.  The row is read
// once; r' never goes back through HBM before the LayerNorm.
// F8: also the E4M3 copy out8 = E4M3(out / s).
// LDS (staged): [0] = gate, [1] = bf(1 + scale), [2] = shift, binary32.
// ---------------------------------------------------------------------------
// Register budget: the per-token form holds five row-sized operands (residual,
// y, gate, scale and shift rows), so it asks for one wave per SIMD fewer than
// the staged form; with the staged form's budget it spilled at NC = 7, 11, 12.
template <int NC, int MODE, bool STAGED, bool F8>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, STAGED ? 3 : 2) void k_gate_add_ln_modulate(
    GateLnArgs a) {
  extern __shared__ float4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  constexpr int kRow = stage_vecs<NC>();
  const Span sp = STAGED ? mod_spans(a.per_mod, a.rows_per_wave, a.blocks_per_mod)
                         : spans(a.rows, a.rows_per_wave);
  const double qr = F8 ? 1.0 / (double)*a.fp8_scale : 1.0;   // E4M3 copy: 1 / scale
  V8 rv[NC], yv[NC];
  {
    V8 gg[stage_iters<NC>()], gs[stage_iters<NC>()], gf[stage_iters<NC>()];
    if (STAGED) {
      // The staging loads, then the first row's, with no branch among them,
      // so the row arrives while the workgroup stages (dit_rows.hpp,
      // load_row_nb).
      const int64_t off = sp.m * a.mod_rs;
      stage_fetch_nb<NC>(gg, a.gate + off, dim);
      stage_fetch_nb<NC>(gs, a.scale + off, dim);
      stage_fetch_nb<NC>(gf, a.shift + off, dim);
      phase_barrier();
      const int64_t r0 = sp.begin < a.rows ? sp.begin : a.rows - 1;   // (in the tensor)
      load_row_nb<NC, kNtGate>(rv, a.residual + r0 * a.res_rs, lane, dim);
      load_row_nb<NC, kNtGateLnY>(yv, a.y + r0 * a.y_rs, lane, dim);
      phase_barrier();
    }
    if (STAGED) {
      stage_each<NC>(dim, [&](int i, int v) {
        float g[8], s1[8], sh[8];
        unpack8(gg[i], g);
        one_plus8(gs[i], s1);
        unpack8(gf[i], sh);
        stage_put(lds, v, g);
        stage_put(lds + kRow, v, s1);
        stage_put(lds + 2 * kRow, v, sh);
      });
      __syncthreads();
    }
  }

  // One row whose residual and y are in rv and yv.
  auto row = [&](int64_t r) {
    const int64_t m = STAGED ? sp.m : r / a.per_mod;
    V8 xv[NC], sc[NC], sf[NC];
    {
      V8 gv[NC];
      if (!STAGED) {
        load_mod_row<NC>(gv, a.gate + m * a.mod_rs, lane, dim, a.per_mod == 1);
        load_mod_row<NC>(sc, a.scale + m * a.mod_rs, lane, dim, a.per_mod == 1);
        load_mod_row<NC>(sf, a.shift + m * a.mod_rs, lane, dim, a.per_mod == 1);
      }
      uint16_t *rrow = a.out_res + r * a.out_res_rs;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (!valid<NC>(c, lane, dim)) {
          xv[c] = V8{{0u, 0u, 0u, 0u}};                         // outside the row
          continue;
        }
        float g[8];
        if (STAGED)
          stage_get(lds, c, lane, g);
        else
          unpack8(gv[c], g);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float q0 = g[2 * k] * lo(yv[c].w[k]), q1 = g[2 * k + 1] * hi(yv[c].w[k]);
          round2(q0, q1);                                       // bf(gate * y)
          xv[c].w[k] = pack(lo(rv[c].w[k]) + q0, hi(rv[c].w[k]) + q1);
        }
        store8(rrow + 512 * c + 8 * lane, xv[c]);
      }
    }
    if (STAGED) phase_barrier();
    float d[NC][8];
    const float rho = ln_stats<NC, MODE>(xv, d, lane, dim, a.eps);
    uint16_t *orow = a.out + r * a.out_rs;
    uint8_t *qrow = F8 ? a.out8 + r * a.out8_rs : nullptr;
    if (STAGED) {
      phase_barrier();
      ln_modulate_out<NC, F8>(orow, qrow, qr, d, rho, lane, dim,
                              [&](int c, float (&s1)[8], float (&sh)[8]) {
                                stage_get(lds + kRow, c, lane, s1);
                                stage_get(lds + 2 * kRow, c, lane, sh);
                              });
    } else {
      ln_modulate_out<NC, F8>(orow, qrow, qr, d, rho, lane, dim,
                              [&](int c, float (&s1)[8], float (&sh)[8]) {
                                one_plus8(sc[c], s1);
                                unpack8(sf[c], sh);
                              });
    }
  };
  // The staged layout's first row was loaded before the staging; it is
  // handled apart from the loop so that rv and yv are not carried around it.
  int64_t r = sp.begin;
  if (STAGED && r < sp.end) row(r++);
  for (; r < sp.end; ++r) {
    load_row<NC, kNtGate>(rv, a.residual + r * a.res_rs, lane, dim);
    load_row<NC, kNtGateLnY>(yv, a.y + r * a.y_rs, lane, dim);
    row(r);
  }
}

template <int MODE, bool F8>
static hipError_t gate_ln_dispatch(GateLnArgs a, hipStream_t s) {
  const Shape sh = row_shape(a.rows, a.per_mod, a.dim, 3);
  a.rows_per_wave = sh.rows_per_wave;
  a.blocks_per_mod = sh.blocks_per_mod;
#define X(N)                                                                     \
  case N:                                                                        \
    DIT_ROW_LAUNCH((k_gate_add_ln_modulate<N, MODE, true, F8>),                  \
                   (k_gate_add_ln_modulate<N, MODE, false, F8>), stage_bytes(a.dim, 3), 0); \
    break;
  DIT_ROW_DISPATCH();
#undef X
}

hipError_t launch_gate_add_ln_modulate(const GateLnArgs &a, int mode, hipStream_t s) {
  if (a.out8)
    return mode == kFast ? gate_ln_dispatch<kFast, true>(a, s)
                         : gate_ln_dispatch<kLossless, true>(a, s);
  return mode == kFast ? gate_ln_dispatch<kFast, false>(a, s)
                       : gate_ln_dispatch<kLossless, false>(a, s);
}

}  // namespace dit

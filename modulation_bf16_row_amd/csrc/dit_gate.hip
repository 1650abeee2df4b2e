// dit_gate.hip -- gfx950 residual gate-add.
// Geometry, staging and launch shapes: dit_rows.hpp.
#include "dit_rows.hpp"

namespace dit {

// ---------------------------------------------------------------------------
// Residual gate-add: out = bf(residual + bf(gate * y)).
// LDS (staged): [0] = gate, binary32.
// ---------------------------------------------------------------------------
template <int NC, bool STAGED>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_residual_gate_add(
    GateAddArgs a) {
  extern __shared__ float4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  const Span sp = STAGED ? mod_spans(a.per_mod, a.rows_per_wave, a.blocks_per_mod)
                         : spans(a.rows, a.rows_per_wave);
  if (STAGED) {
    for (int v = threadIdx.x; v < dim / 8; v += kThreads) {
      float g[8];
      unpack8(load8(a.gate + sp.m * a.mod_rs + 8 * v), g);
      stage_put(lds, v, g);
    }
    __syncthreads();
  }

  for (int64_t r = sp.begin; r < sp.end; ++r) {
    V8 rv[NC], yv[NC], gv[NC];
    load_row<NC, kNtGate>(rv, a.residual + r * a.res_rs, lane, dim);
    load_row<NC, kNtGate>(yv, a.y + r * a.y_rs, lane, dim);
    const int64_t m = STAGED ? sp.m : r / a.per_mod;
    if (!STAGED) load_mod_row<NC>(gv, a.gate + m * a.mod_rs, lane, dim, a.per_mod == 1);
    uint16_t *orow = a.out + r * a.out_rs;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (!valid<NC>(c, lane, dim)) continue;
      float g[8];
      if (STAGED)
        stage_get(lds, c, lane, g);
      else
        unpack8(gv[c], g);
      V8 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float q0 = g[2 * k] * lo(yv[c].w[k]), q1 = g[2 * k + 1] * hi(yv[c].w[k]);
        round2(q0, q1);                                         // bf(gate * y)
        o.w[k] = pack(lo(rv[c].w[k]) + q0, hi(rv[c].w[k]) + q1);
      }
      store8(orow + 512 * c + 8 * lane, o);
    }
  }
}

static hipError_t gate_add_dispatch(GateAddArgs a, hipStream_t s) {
  const Shape sh = row_shape(a.rows, a.per_mod, a.dim, 1);
  a.rows_per_wave = sh.rows_per_wave;
  a.blocks_per_mod = sh.blocks_per_mod;
#define X(N)                                                                              \
  case N:                                                                                 \
    DIT_ROW_LAUNCH((k_residual_gate_add<N, true>), (k_residual_gate_add<N, false>),       \
                   stage_bytes(a.dim, 1), 0);                                             \
    break;
  DIT_ROW_DISPATCH();
#undef X
}

hipError_t launch_residual_gate_add(const GateAddArgs &a, hipStream_t s) {
  return gate_add_dispatch(a, s);
}

}  // namespace dit

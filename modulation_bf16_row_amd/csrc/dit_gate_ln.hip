// dit_gate_ln.hip -- gfx950 gated residual + LayerNorm/AdaLN producer, with or
// without its E4M3 copy.
// Geometry, staging and launch shapes: dit_rows.hpp (per-batch modulation)
// and dit_split.hpp (otherwise); LN helpers: dit_ln.hpp.
#include "dit_ln.hpp"

namespace dit {

// r' = bf(residual + bf(gate * y)) of one vector (gate as binary32 values).
__device__ __forceinline__ V8 gate_add_vec(const V8 &res, const V8 &y, const float (&g)[8]) {
  V8 x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float q0 = g[2 * k] * lo(y.w[k]), q1 = g[2 * k + 1] * hi(y.w[k]);
    round2(q0, q1);                                             // bf(gate * y)
    x.w[k] = pack(lo(res.w[k]) + q0, hi(res.w[k]) + q1);
  }
  return x;
}

// ---------------------------------------------------------------------------
// Gated residual + LayerNorm + AdaLN modulate: r' = bf(residual + bf(gate * y))
// is written to out_res, and LN + modulate of r' to out.  The row is read
// once; r' never goes back through HBM before the LayerNorm.
// F8: also the E4M3 copy out8 = E4M3(out / s).
// Per-batch modulation (the staged row layout, dit_rows.hpp).
// LDS: [0] = gate, [1] = bf(1 + scale), [2] = shift, binary32.
// ---------------------------------------------------------------------------
template <int NC, int MODE, bool F8>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_gate_add_ln_modulate(
    GateLnArgs a) {
  extern __shared__ float4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  constexpr int kRow = stage_vecs<NC>();
  const Span sp = mod_spans(a.per_mod, a.rows_per_wave, a.blocks_per_mod);
  const double qr = F8 ? 1.0 / (double)*a.fp8_scale : 1.0;   // E4M3 copy: 1 / scale
  V8 rv[NC], yv[NC];
  {
    // The staging loads, then the first row's, with no branch among them, so
    // the row arrives while the workgroup stages (dit_rows.hpp, load_row_nb).
    V8 gg[stage_iters<NC>()], gs[stage_iters<NC>()], gf[stage_iters<NC>()];
    const int64_t off = sp.m * a.mod_rs;
    stage_fetch_nb<NC>(gg, a.gate + off, dim);
    stage_fetch_nb<NC>(gs, a.scale + off, dim);
    stage_fetch_nb<NC>(gf, a.shift + off, dim);
    phase_barrier();
    const int64_t r0 = sp.begin < a.rows ? sp.begin : a.rows - 1;   // (in the tensor)
    load_row_nb<NC, kNtGate>(rv, a.residual + r0 * a.res_rs, lane, dim);
    load_row_nb<NC, kNtGateLnY>(yv, a.y + r0 * a.y_rs, lane, dim);
    phase_barrier();
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

  // One row whose residual and y are in rv and yv.
  auto row = [&](int64_t r) {
    V8 xv[NC];
    uint16_t *rrow = a.out_res + r * a.out_res_rs;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (!valid<NC>(c, lane, dim)) {
        xv[c] = V8{{0u, 0u, 0u, 0u}};                           // outside the row
        continue;
      }
      float g[8];
      stage_get(lds, c, lane, g);
      xv[c] = gate_add_vec(rv[c], yv[c], g);
      store8(rrow + 512 * c + 8 * lane, xv[c]);
    }
    phase_barrier();
    float d[NC][8];
    const float rho = ln_stats<NC, MODE>(xv, d, lane, dim, a.eps);
    uint16_t *orow = a.out + r * a.out_rs;
    uint8_t *qrow = F8 ? a.out8 + r * a.out8_rs : nullptr;
    phase_barrier();
    ln_modulate_out<NC, F8>(orow, qrow, qr, d, rho, lane, dim,
                            [&](int c, float (&s1)[8], float (&sh)[8]) {
                              stage_get(lds + kRow, c, lane, s1);
                              stage_get(lds + 2 * kRow, c, lane, sh);
                            });
  };
  // The first row was loaded before the staging; it is handled apart from the
  // loop so that rv and yv are not carried around it.
  int64_t r = sp.begin;
  if (r < sp.end) row(r++);
  for (; r < sp.end; ++r) {
    load_row<NC, kNtGate>(rv, a.residual + r * a.res_rs, lane, dim);
    load_row<NC, kNtGateLnY>(yv, a.y + r * a.y_rs, lane, dim);
    row(r);
  }
}

// ---------------------------------------------------------------------------
// The same operation in the split-row layout (dit_split.hpp): one row per
// workgroup, two chunks per wave.  Each wave forms and writes r' for its
// chunks and publishes them; wave 0 takes the LayerNorm statistics of the
// published r'.  Modulation rows read by one row only (per-token) are streamed.
// ---------------------------------------------------------------------------
// Register budget: the E4M3 copy's binary64 quotients do not fit beside the
// five operands in 64 VGPRs, so that form runs at 7 waves per SIMD.
template <int NC, int MODE, bool F8>
__global__ DIT_SPLIT_KERNEL_W(F8 ? 7 : 8) void k_gate_add_ln_modulate_split(GateLnArgs a) {
  __shared__ uint4 xs[NC * 64];
  __shared__ float st[2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, dim = (int)a.dim;
  const double qr = F8 ? 1.0 / (double)*a.fp8_scale : 1.0;   // E4M3 copy: 1 / scale
  const bool per_token = a.per_mod == 1;
  for (int64_t r = blockIdx.x; r < a.rows; r += gridDim.x) {
    const int64_t off = (r / a.per_mod) * a.mod_rs;
    V8 xv[kSplitChunks], sc[kSplitChunks], sf[kSplitChunks];
    {
      V8 rv[kSplitChunks], yv[kSplitChunks], gv[kSplitChunks];
      split_load<NC, kNtGate>(rv, a.residual + r * a.res_rs, w, lane, dim);
      split_load<NC, kNtGateLnY>(yv, a.y + r * a.y_rs, w, lane, dim);
      if (per_token) {
        split_load<NC, true>(gv, a.gate + off, w, lane, dim);
        split_load<NC, true>(sc, a.scale + off, w, lane, dim);
        split_load<NC, true>(sf, a.shift + off, w, lane, dim);
      } else {
        split_load<NC, false>(gv, a.gate + off, w, lane, dim);
        split_load<NC, false>(sc, a.scale + off, w, lane, dim);
        split_load<NC, false>(sf, a.shift + off, w, lane, dim);
      }
      uint16_t *rrow = a.out_res + r * a.out_res_rs;
#pragma unroll
      for (int k = 0; k < kSplitChunks; ++k) {
        const int c = split_chunk(w, k);
        float g[8];
        unpack8(gv[k], g);
        xv[k] = gate_add_vec(rv[k], yv[k], g);
        if (split_has<NC>(c, lane, dim)) store8(rrow + 512 * c + 8 * lane, xv[k]);
      }
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
static hipError_t gate_ln_dispatch(GateLnArgs a, hipStream_t s) {
  const Shape sh = row_shape(a.rows, a.per_mod, a.dim, 3);
  a.rows_per_wave = sh.rows_per_wave;
  a.blocks_per_mod = sh.blocks_per_mod;
#define X(N)                                                                     \
  case N:                                                                        \
    if (sh.staged)                                                               \
      DIT_LAUNCH((k_gate_add_ln_modulate<N, MODE, F8>), sh.grid, dim3(kThreads),  \
                 stage_bytes(a.dim, 3), s, a);                                   \
    else                                                                         \
      DIT_LAUNCH((k_gate_add_ln_modulate_split<N, MODE, F8>), split_grid(a.rows), \
                 dim3(64 * split_waves<N>()), 0, s, a);                          \
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

// dit_rms.hip -- gfx950 native-bf16 RMSNorm-scale and RMSNorm-tanh-residual.
// Geometry, staging and launch shapes: dit_rows.hpp.
#include "dit_rows.hpp"

namespace dit {

// ---------------------------------------------------------------------------
// Native-bf16 RMSNorm: the chain's bf16 rstd of one row.
// ---------------------------------------------------------------------------
template <int NC, int MODE>
__device__ __forceinline__ float rms_rstd(const V8 (&xv)[NC], int lane, int dim, float eps) {
  float p = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (valid<NC>(c, lane, dim))
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float t0 = lo(xv[c].w[k]), t1 = hi(xv[c].w[k]);
        t0 = t0 * t0;
        t1 = t1 * t1;
        round2(t0, t1);                                  // bf16 squares
        p = p + t0;
        p = p + t1;
      }
  const float ms = round1(wave_sum(p) / (float)dim);     // bf16 mean square
  const float v = round1(ms + eps);                      // bf16 (ms + eps)
  return rstd_bf16<MODE>(v);                              // bf16 rstd
}

// y2 = bf(bf(x * rstd) * w) for the pair in word xw (weights w0, w1).
__device__ __forceinline__ void rms_y2(float &y0, float &y1, uint32_t xw, float w0, float w1,
                                       float rstd) {
  y0 = lo(xw) * rstd;
  y1 = hi(xw) * rstd;
  round2(y0, y1);
  y0 = y0 * w0;
  y1 = y1 * w1;
  round2(y0, y1);
}


// out = bf(y2 * scale) for the row in xv; chunk c's weight and scale come from
// the staged rows (binary32) and, unstaged, the scale from sc.
template <int NC, int MODE, bool STAGED>
__device__ __forceinline__ void rms_scale_out(const RmsScaleArgs &a, const float4 *lds,
                                              const V8 (&xv)[NC], const V8 (&sc)[NC],
                                              int64_t r, int lane, int dim) {
  constexpr int kRow = stage_vecs<NC>();
  const float rstd = rms_rstd<NC, MODE>(xv, lane, dim, a.eps);
  phase_barrier();
  uint16_t *orow = a.out + r * a.out_rs;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (!valid<NC>(c, lane, dim)) continue;
    float w[8], s[8];
    stage_get(lds, c, lane, w);
    if (STAGED)
      stage_get(lds + kRow, c, lane, s);
    else
      unpack8(sc[c], s);
    V8 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float y0, y1;
      rms_y2(y0, y1, xv[c].w[k], w[2 * k], w[2 * k + 1], rstd);
      o.w[k] = pack(y0 * s[2 * k], y1 * s[2 * k + 1]);
    }
    store8(orow + 512 * c + 8 * lane, o);
  }
}

// LDS: [0] = weight (always), [1] = scale (staged), binary32.  The staged
// layout takes one row per wave (four per workgroup): the row's loads are
// issued, with no branch among them, after the staging loads and before the
// staging, so the row arrives while the workgroup stages.
template <int NC, int MODE, bool STAGED>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_rmsnorm_scale(RmsScaleArgs a) {
  extern __shared__ float4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  constexpr int kRow = stage_vecs<NC>();
  const Span sp = STAGED ? mod_spans(a.per_mod, 1, a.blocks_per_mod)
                         : spans(a.rows, a.rows_per_wave);
  if (sp.wg_empty) return;                                 // whole workgroup idle
  V8 gw[stage_iters<NC>()], gs[stage_iters<NC>()], xv[NC];
  stage_fetch_nb<NC>(gw, a.weight, dim);                   // weight: every launch
  if (STAGED) {
    stage_fetch_nb<NC>(gs, a.scale + sp.m * a.mod_rs, dim);
    phase_barrier();                                       // the staging loads first,
    const int64_t r0 = sp.begin < a.rows ? sp.begin : a.rows - 1;  // (in the tensor)
    load_row_nb<NC, kNtRms>(xv, a.x + r0 * a.x_rs, lane, dim);
    phase_barrier();                                       // then the row's
  }
  stage_each<NC>(dim, [&](int i, int v) {
    float w[8];
    unpack8(gw[i], w);
    stage_put(lds, v, w);
    if (STAGED) {
      unpack8(gs[i], w);
      stage_put(lds + kRow, v, w);
    }
  });
  __syncthreads();
  if (STAGED) {
    if (sp.begin < sp.end) rms_scale_out<NC, MODE, true>(a, lds, xv, xv, sp.begin, lane, dim);
    return;
  }
  for (int64_t r = sp.begin; r < sp.end; ++r) {
    V8 sc[NC];
    load_row<NC, kNtRms>(xv, a.x + r * a.x_rs, lane, dim);
    load_mod_row<NC>(sc, a.scale + (r / a.per_mod) * a.mod_rs, lane, dim, a.per_mod == 1);
    rms_scale_out<NC, MODE, false>(a, lds, xv, sc, r, lane, dim);
  }
}

// RMSNorm-tanh-residual output of the row in xv with residual rv; tanh(gate)
// comes from the staged row (binary32) or, unstaged, from the table lookup
// of the gate vectors tau.
template <int NC, int MODE, bool STAGED>
__device__ __forceinline__ void tanh_out(const RmsTanhArgs &a, const float4 *lds,
                                         const uint16_t *tab, const V8 (&xv)[NC],
                                         const V8 (&rv)[NC], const V8 (&tau)[NC], int64_t r,
                                         int lane, int dim) {
  constexpr int kRow = stage_vecs<NC>();
  const float rstd = rms_rstd<NC, MODE>(xv, lane, dim, a.eps);
  phase_barrier();
  uint16_t *orow = a.out + r * a.out_rs;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (!valid<NC>(c, lane, dim)) continue;
    float w[8], tg[8];
    stage_get(lds, c, lane, w);
    if (STAGED) {
      stage_get(lds + kRow, c, lane, tg);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) tg[j] = tanh_lookup(elem(tau[c], j), tab);
    }
    V8 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float y0, y1;
      rms_y2(y0, y1, xv[c].w[k], w[2 * k], w[2 * k + 1], rstd);
      float q0 = tg[2 * k] * y0, q1 = tg[2 * k + 1] * y1;
      round2(q0, q1);                                   // bf(tanh(gate) * y2)
      o.w[k] = pack(lo(rv[c].w[k]) + q0, hi(rv[c].w[k]) + q1);
    }
    store8(orow + 512 * c + 8 * lane, o);
  }
}

// LDS: [0] = weight (always), [1] = tanh(gate) (staged), binary32; then the
// tanh table.  tanh comes from the table in both modes.  The staged layout
// takes one row per wave, loaded as in k_rmsnorm_scale.
template <int NC, int MODE, bool STAGED>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_rmsnorm_tanh_residual(
    RmsTanhArgs a) {
  extern __shared__ float4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  constexpr int kRow = stage_vecs<NC>();
  uint16_t *tab = reinterpret_cast<uint16_t *>(lds + (STAGED ? 2 : 1) * kRow);
  const Span sp = STAGED ? mod_spans(a.per_mod, 1, a.blocks_per_mod)
                         : spans(a.rows, a.rows_per_wave);
  if (sp.wg_empty) return;                                 // whole workgroup idle
  V8 gw[stage_iters<NC>()], gg[stage_iters<NC>()], xv[NC], rv[NC];
  const uint4 tv = tanh_table_fetch(threadIdx.x);
  stage_fetch_nb<NC>(gw, a.weight, dim);                   // weight: every launch
  if (STAGED) {
    stage_fetch_nb<NC>(gg, a.gate + sp.m * a.mod_rs, dim);
    phase_barrier();                                       // the staging loads first,
    const int64_t r0 = sp.begin < a.rows ? sp.begin : a.rows - 1;  // (in the tensor)
    load_row_nb<NC, kNtTanh>(xv, a.x + r0 * a.x_rs, lane, dim);
    load_row_nb<NC, kNtTanh>(rv, a.residual + r0 * a.res_rs, lane, dim);
    phase_barrier();                                       // then the row's
  }
  tanh_table_put(tab, threadIdx.x, tv);
  stage_each<NC>(dim, [&](int i, int v) {
    float w[8];
    unpack8(gw[i], w);
    stage_put(lds, v, w);
  });
  __syncthreads();
  if (STAGED) {
    stage_each<NC>(dim, [&](int i, int v) {
      float t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = tanh_lookup(elem(gg[i], j), tab);
      stage_put(lds + kRow, v, t);
    });
    __syncthreads();
    if (sp.begin < sp.end) tanh_out<NC, MODE, true>(a, lds, tab, xv, rv, xv, sp.begin, lane, dim);
    return;
  }
  for (int64_t r = sp.begin; r < sp.end; ++r) {
    V8 tau[NC];
    load_row<NC, kNtTanh>(xv, a.x + r * a.x_rs, lane, dim);
    load_row<NC, kNtTanh>(rv, a.residual + r * a.res_rs, lane, dim);
    load_mod_row<NC>(tau, a.gate + (r / a.per_mod) * a.mod_rs, lane, dim, a.per_mod == 1);
    tanh_out<NC, MODE, false>(a, lds, tab, xv, rv, tau, r, lane, dim);
  }
}

template <int MODE>
static hipError_t rms_scale_dispatch(RmsScaleArgs a, hipStream_t s) {
  const Shape sh = row_shape(a.rows, a.per_mod, a.dim, 2);
  a.rows_per_wave = sh.rows_per_wave;
  a.blocks_per_mod = sh.blocks_per_mod;
#define X(N)                                                                              \
  case N:                                                                                 \
    DIT_ROW_LAUNCH((k_rmsnorm_scale<N, MODE, true>), (k_rmsnorm_scale<N, MODE, false>),   \
                   stage_bytes(a.dim, 2), stage_bytes(a.dim, 1));                         \
    break;
  DIT_ROW_DISPATCH();
#undef X
}

template <int MODE>
static hipError_t rms_tanh_dispatch(RmsTanhArgs a, hipStream_t s) {
  const Shape sh = row_shape(a.rows, a.per_mod, a.dim, 2);
  a.rows_per_wave = sh.rows_per_wave;
  a.blocks_per_mod = sh.blocks_per_mod;
  const size_t tab = kTanhTabVecs * sizeof(uint4);
#define X(N)                                                                          \
  case N:                                                                             \
    DIT_ROW_LAUNCH((k_rmsnorm_tanh_residual<N, MODE, true>),                          \
                   (k_rmsnorm_tanh_residual<N, MODE, false>),                         \
                   stage_bytes(a.dim, 2) + tab, stage_bytes(a.dim, 1) + tab);         \
    break;
  DIT_ROW_DISPATCH();
#undef X
}

hipError_t launch_rmsnorm_scale(const RmsScaleArgs &a, int mode, hipStream_t s) {
  return mode == kFast ? rms_scale_dispatch<kFast>(a, s) : rms_scale_dispatch<kLossless>(a, s);
}

hipError_t launch_rmsnorm_tanh_residual(const RmsTanhArgs &a, int mode, hipStream_t s) {
  return mode == kFast ? rms_tanh_dispatch<kFast>(a, s) : rms_tanh_dispatch<kLossless>(a, s);
}

}  // namespace dit

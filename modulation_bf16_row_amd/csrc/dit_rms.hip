// dit_rms.hip -- gfx950 native-bf16 RMSNorm-scale and RMSNorm-tanh-residual.
// Geometry, staging and launch shapes: dit_rows.hpp; RMSNorm-scale takes the
// split-row layout (dit_split.hpp) where the staged one does not apply.
// RMSNorm-tanh-residual keeps the row layout there too: in the split layout
// (the tanh table copied per workgroup, the weight read per row) it ran no
// faster at the Wan 720p shape with per-token gates, and back to back with
// itself it slowed to 564 us against 530 us in the row layout.
#include "dit_rows.hpp"
#include "dit_split.hpp"

namespace dit {

// ---------------------------------------------------------------------------
// Native-bf16 RMSNorm: the chain's bf16 rstd of one row.
// ---------------------------------------------------------------------------
// Adds the bf16 squares of one vector to this lane's partial, in element order.
__device__ __forceinline__ void rms_accumulate(float &p, const V8 &x) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float t0 = lo(x.w[k]), t1 = hi(x.w[k]);
    t0 = t0 * t0;
    t1 = t1 * t1;
    round2(t0, t1);                                      // bf16 squares
    p = p + t0;
    p = p + t1;
  }
}

// bf16 rstd from this lane's partial sum of squares.
template <int MODE>
__device__ __forceinline__ float rms_finish(float p, int dim, float eps) {
  const float ms = round1(wave_sum(p) / (float)dim);     // bf16 mean square
  const float v = round1(ms + eps);                      // bf16 (ms + eps)
  return rstd_bf16<MODE>(v);                              // bf16 rstd
}

template <int NC, int MODE>
__device__ __forceinline__ float rms_rstd(const V8 (&xv)[NC], int lane, int dim, float eps) {
  float p = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (valid<NC>(c, lane, dim)) rms_accumulate(p, xv[c]);
  return rms_finish<MODE>(p, dim, eps);
}

// Split-row layout, wave 0: the same sum over the row published in LDS;
// leaves the bf16 rstd in st[0].
template <int NC, int MODE>
__device__ __forceinline__ void split_rms_rstd(const uint4 *xs, float *st, int lane, int dim,
                                               float eps) {
  float p = 0.0f;
  split_walk<NC>(xs, lane, [&](int c, const V8 &v) {
    if (valid<NC>(c, lane, dim)) rms_accumulate(p, v);
  });
  const float rstd = rms_finish<MODE>(p, dim, eps);
  if (lane == 0) st[0] = rstd;
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


// out = bf(y2 * scale) for the row in xv; chunk c's weight and scale come
// from the staged rows (binary32).
template <int NC, int MODE>
__device__ __forceinline__ void rms_scale_out(const RmsScaleArgs &a, const float4 *lds,
                                              const V8 (&xv)[NC], int64_t r, int lane, int dim) {
  constexpr int kRow = stage_vecs<NC>();
  const float rstd = rms_rstd<NC, MODE>(xv, lane, dim, a.eps);
  phase_barrier();
  uint16_t *orow = a.out + r * a.out_rs;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (!valid<NC>(c, lane, dim)) continue;
    float w[8], s[8];
    stage_get(lds, c, lane, w);
    stage_get(lds + kRow, c, lane, s);
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

// RMSNorm-scale, per-batch modulation (the staged row layout, dit_rows.hpp).
// LDS: [0] = weight, [1] = scale, binary32.  One row per wave: the row's
// loads are issued, with no branch among them, after the staging loads and
// before the staging, so the row arrives while the workgroup stages.
template <int NC, int MODE>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_rmsnorm_scale(RmsScaleArgs a) {
  extern __shared__ float4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  constexpr int kRow = stage_vecs<NC>();
  const Span sp = mod_spans(a.per_mod, 1, a.blocks_per_mod);
  V8 gw[stage_iters<NC>()], gs[stage_iters<NC>()], xv[NC];
  stage_fetch_nb<NC>(gw, a.weight, dim);
  stage_fetch_nb<NC>(gs, a.scale + sp.m * a.mod_rs, dim);
  phase_barrier();                                         // the staging loads first,
  const int64_t r0 = sp.begin < a.rows ? sp.begin : a.rows - 1;   // (in the tensor)
  load_row_nb<NC, kNtRms>(xv, a.x + r0 * a.x_rs, lane, dim);
  phase_barrier();                                         // then the row's
  stage_each<NC>(dim, [&](int i, int v) {
    float w[8];
    unpack8(gw[i], w);
    stage_put(lds, v, w);
    unpack8(gs[i], w);
    stage_put(lds + kRow, v, w);
  });
  __syncthreads();
  if (sp.begin < sp.end) rms_scale_out<NC, MODE>(a, lds, xv, sp.begin, lane, dim);
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

// ---------------------------------------------------------------------------
// The split-row layout (dit_split.hpp): one row per workgroup, two chunks per
// wave; wave 0 takes the row's rstd from the row published in LDS.  The
// weight (shared by every row) keeps the default load policy; modulation rows
// read by one row only (per-token) are streamed.
// ---------------------------------------------------------------------------
template <int NC, int MODE>
__global__ DIT_SPLIT_KERNEL void k_rmsnorm_scale_split(RmsScaleArgs a) {
  __shared__ uint4 xs[NC * 64];
  __shared__ float st[1];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, dim = (int)a.dim;
  const bool per_token = a.per_mod == 1;
  for (int64_t r = blockIdx.x; r < a.rows; r += gridDim.x) {
    const uint16_t *srow = a.scale + (r / a.per_mod) * a.mod_rs;
    V8 xv[kSplitChunks], sc[kSplitChunks], wv[kSplitChunks];
    split_load<NC, kNtRms>(xv, a.x + r * a.x_rs, w, lane, dim);
    if (per_token)
      split_load<NC, true>(sc, srow, w, lane, dim);
    else
      split_load<NC, false>(sc, srow, w, lane, dim);
    split_load<NC, false>(wv, a.weight, w, lane, dim);
    split_publish<NC>(xs, xv, w, lane);
    __syncthreads();
    if (w == 0) split_rms_rstd<NC, MODE>(xs, st, lane, dim, a.eps);
    __syncthreads();
    const float rstd = st[0];
    uint16_t *orow = a.out + r * a.out_rs;
#pragma unroll
    for (int k = 0; k < kSplitChunks; ++k) {
      const int c = split_chunk(w, k);
      if (!split_has<NC>(c, lane, dim)) continue;
      V8 o;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        float y0, y1;
        rms_y2(y0, y1, xv[k].w[h], lo(wv[k].w[h]), hi(wv[k].w[h]), rstd);
        o.w[h] = pack(y0 * lo(sc[k].w[h]), y1 * hi(sc[k].w[h]));
      }
      store8(orow + 512 * c + 8 * lane, o);
    }
    __syncthreads();                                   // xs and st serve the next row
  }
}

template <int MODE>
static hipError_t rms_scale_dispatch(RmsScaleArgs a, hipStream_t s) {
  const Shape sh = row_shape(a.rows, a.per_mod, a.dim, 2);
  a.rows_per_wave = sh.rows_per_wave;
  a.blocks_per_mod = sh.blocks_per_mod;
#define X(N)                                                                              \
  case N:                                                                                 \
    if (sh.staged)                                                                        \
      DIT_LAUNCH((k_rmsnorm_scale<N, MODE>), sh.grid, dim3(kThreads),                     \
                 stage_bytes(a.dim, 2), s, a);                                            \
    else                                                                                  \
      DIT_LAUNCH((k_rmsnorm_scale_split<N, MODE>), split_grid(a.rows),                    \
                 dim3(64 * split_waves<N>()), 0, s, a);                                   \
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

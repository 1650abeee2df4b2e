// dit_rows.hip -- gfx950 kernels for the four row epilogues.
//
// Geometry: one 64-lane wave per row, four waves (rows) per 256-thread
// workgroup.  Lane l owns the 8-element vectors at 512c + 8l of chunk c
// (c < NC = ceil(dim / 512)), loaded with one 128-bit access each, so a
// wave-wide load is 1 KiB contiguous.  The row stays in VGPRs between the
// two LayerNorm passes (at most 16 vectors = 64 VGPRs for dim 8192), so x
// is read from HBM exactly once.  Row sums follow R(dim): each lane adds
// its own terms in (chunk, element) order, then a fixed xor butterfly.
//
// Sources: AdaLN rounding points -- page "基于Agent的SGLang扩散模型Kernel优化实践"
// (tahou.com), section "数学等价不代表结果完全一致"; native bf16 RMSNorm chain --
// page "#34085 [diffusion] Clean up kernels and shared fast paths", section
// "关键源码片段"; rmsnorm+tanh(gate)*x+residual and residual+gate*update --
// page "AI Agent 驱动的 SGLang Kernel 一等公民", section 0x3 / 3.2.
#include "dit_device.hpp"
#include "dit_launch.hpp"

namespace dit {

constexpr int kWavesPerBlock = 4;

struct RowCtx {
  int lane;
  int64_t row;
};

__device__ __forceinline__ RowCtx row_ctx() {
  RowCtx c;
  c.lane = threadIdx.x & 63;
  c.row = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  return c;
}

// Is chunk c of this lane inside the row?  Chunks before the last are full.
template <int NC>
__device__ __forceinline__ bool valid(int c, int lane, int dim) {
  return c < NC - 1 || 512 * c + 8 * lane < dim;
}

template <int NC>
__device__ __forceinline__ void load_row(V8 (&v)[NC], const uint16_t *base, int lane, int dim) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (valid<NC>(c, lane, dim))
      v[c] = load8(base + 512 * c + 8 * lane);
    else
      v[c] = V8{{0u, 0u, 0u, 0u}};
  }
}

// ---------------------------------------------------------------------------
// LayerNorm + AdaLN modulate
// ---------------------------------------------------------------------------
template <int NC, int MODE>
__global__ __launch_bounds__(256) void k_ln_modulate(LnModArgs a) {
  const RowCtx ctx = row_ctx();
  if (ctx.row >= a.rows) return;
  const int lane = ctx.lane, dim = (int)a.dim;
  const int64_t m = ctx.row / a.per_mod;

  V8 xv[NC], sc[NC], sh[NC];
  load_row<NC>(xv, a.x + ctx.row * a.x_rs, lane, dim);
  load_row<NC>(sc, a.scale + m * a.mod_rs, lane, dim);
  load_row<NC>(sh, a.shift + m * a.mod_rs, lane, dim);

  // pass 1: mean
  float p = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (valid<NC>(c, lane, dim))
#pragma unroll
      for (int j = 0; j < 8; ++j) p = p + elem(xv[c], j);
  const float mean = wave_sum(p) / (float)dim;

  // pass 2: variance of the deviations (recomputed identically below)
  float q = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (valid<NC>(c, lane, dim))
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float d = elem(xv[c], j) - mean;
        if (MODE == kLossless)
          q = q + d * d;
        else
          q = fmaf(d, d, q);
      }
  const float var = wave_sum(q) / (float)dim;
  const float rho = rsqrt_mode<MODE>(var + a.eps);

  uint16_t *orow = a.out + ctx.row * a.out_rs;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (!valid<NC>(c, lane, dim)) continue;
    V8 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float n0 = (lo(xv[c].w[k]) - mean) * rho;
      float n1 = (hi(xv[c].w[k]) - mean) * rho;
      round2(n0, n1);                                   // LayerNorm output
      float s0 = 1.0f + lo(sc[c].w[k]);
      float s1 = 1.0f + hi(sc[c].w[k]);
      round2(s0, s1);                                   // 1 + scale
      float p0 = n0 * s0, p1 = n1 * s1;
      round2(p0, p1);                                   // product
      o.w[k] = pack(p0 + lo(sh[c].w[k]), p1 + hi(sh[c].w[k]));  // + shift
    }
    store8(orow + 512 * c + 8 * lane, o);
  }
}

// ---------------------------------------------------------------------------
// Native-bf16 RMSNorm: y2 = bf(bf(x * rstd) * w), rstd from the bf16 chain.
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
        round2(t0, t1);                                 // bf16 squares
        p = p + t0;
        p = p + t1;
      }
  const float ms = round1(wave_sum(p) / (float)dim);    // bf16 mean square
  const float v = round1(ms + eps);                     // bf16 (ms + eps)
  return round1(rsqrt_mode<MODE>(v));                   // bf16 rstd
}

__device__ __forceinline__ void rms_y2(float &y0, float &y1, uint32_t xw, uint32_t ww,
                                       float rstd) {
  y0 = lo(xw) * rstd;
  y1 = hi(xw) * rstd;
  round2(y0, y1);
  y0 = y0 * lo(ww);
  y1 = y1 * hi(ww);
  round2(y0, y1);
}

template <int NC, int MODE>
__global__ __launch_bounds__(256) void k_rmsnorm_scale(RmsScaleArgs a) {
  const RowCtx ctx = row_ctx();
  if (ctx.row >= a.rows) return;
  const int lane = ctx.lane, dim = (int)a.dim;
  const int64_t m = ctx.row / a.per_mod;

  V8 xv[NC], wv[NC], sc[NC];
  load_row<NC>(xv, a.x + ctx.row * a.x_rs, lane, dim);
  load_row<NC>(wv, a.weight, lane, dim);
  load_row<NC>(sc, a.scale + m * a.mod_rs, lane, dim);

  const float rstd = rms_rstd<NC, MODE>(xv, lane, dim, a.eps);

  uint16_t *orow = a.out + ctx.row * a.out_rs;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (!valid<NC>(c, lane, dim)) continue;
    V8 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float y0, y1;
      rms_y2(y0, y1, xv[c].w[k], wv[c].w[k], rstd);
      o.w[k] = pack(y0 * lo(sc[c].w[k]), y1 * hi(sc[c].w[k]));
    }
    store8(orow + 512 * c + 8 * lane, o);
  }
}

template <int NC, int MODE>
__global__ __launch_bounds__(256) void k_rmsnorm_tanh_residual(RmsTanhArgs a) {
  const RowCtx ctx = row_ctx();
  if (ctx.row >= a.rows) return;
  const int lane = ctx.lane, dim = (int)a.dim;
  const int64_t m = ctx.row / a.per_mod;

  V8 xv[NC], wv[NC], gv[NC], rv[NC];
  load_row<NC>(xv, a.x + ctx.row * a.x_rs, lane, dim);
  load_row<NC>(rv, a.residual + ctx.row * a.res_rs, lane, dim);
  load_row<NC>(wv, a.weight, lane, dim);
  load_row<NC>(gv, a.gate + m * a.mod_rs, lane, dim);

  const float rstd = rms_rstd<NC, MODE>(xv, lane, dim, a.eps);

  uint16_t *orow = a.out + ctx.row * a.out_rs;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (!valid<NC>(c, lane, dim)) continue;
    V8 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float y0, y1;
      rms_y2(y0, y1, xv[c].w[k], wv[c].w[k], rstd);
      float q0 = tanh_bf16<MODE>(lo(gv[c].w[k])) * y0;
      float q1 = tanh_bf16<MODE>(hi(gv[c].w[k])) * y1;
      round2(q0, q1);
      o.w[k] = pack(lo(rv[c].w[k]) + q0, hi(rv[c].w[k]) + q1);
    }
    store8(orow + 512 * c + 8 * lane, o);
  }
}

// ---------------------------------------------------------------------------
// Residual gate-add: out = bf(residual + bf(gate * y)).
// ---------------------------------------------------------------------------
template <int NC>
__global__ __launch_bounds__(256) void k_residual_gate_add(GateAddArgs a) {
  const RowCtx ctx = row_ctx();
  if (ctx.row >= a.rows) return;
  const int lane = ctx.lane, dim = (int)a.dim;
  const int64_t m = ctx.row / a.per_mod;

  V8 rv[NC], yv[NC], gv[NC];
  load_row<NC>(rv, a.residual + ctx.row * a.res_rs, lane, dim);
  load_row<NC>(yv, a.y + ctx.row * a.y_rs, lane, dim);
  load_row<NC>(gv, a.gate + m * a.mod_rs, lane, dim);

  uint16_t *orow = a.out + ctx.row * a.out_rs;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (!valid<NC>(c, lane, dim)) continue;
    V8 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float g0 = lo(gv[c].w[k]) * lo(yv[c].w[k]);
      float g1 = hi(gv[c].w[k]) * hi(yv[c].w[k]);
      round2(g0, g1);
      o.w[k] = pack(lo(rv[c].w[k]) + g0, hi(rv[c].w[k]) + g1);
    }
    store8(orow + 512 * c + 8 * lane, o);
  }
}

// ---------------------------------------------------------------------------
// Launchers: NC = ceil(dim / 512) selects the instantiation.
// ---------------------------------------------------------------------------
static dim3 row_grid(int64_t rows) {
  return dim3((unsigned)((rows + kWavesPerBlock - 1) / kWavesPerBlock));
}

#define DIT_NC_CASES(X) \
  X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)

template <int MODE>
static hipError_t ln_dispatch(const LnModArgs &a, hipStream_t s) {
  const int nc = (int)((a.dim + 511) / 512);
  switch (nc) {
#define X(N) \
  case N:    \
    hipLaunchKernelGGL((k_ln_modulate<N, MODE>), row_grid(a.rows), dim3(256), 0, s, a); break;
    DIT_NC_CASES(X)
#undef X
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_ln_modulate(const LnModArgs &a, int mode, hipStream_t s) {
  return mode == kFast ? ln_dispatch<kFast>(a, s) : ln_dispatch<kLossless>(a, s);
}

template <int MODE>
static hipError_t rms_scale_dispatch(const RmsScaleArgs &a, hipStream_t s) {
  const int nc = (int)((a.dim + 511) / 512);
  switch (nc) {
#define X(N) \
  case N:    \
    hipLaunchKernelGGL((k_rmsnorm_scale<N, MODE>), row_grid(a.rows), dim3(256), 0, s, a); break;
    DIT_NC_CASES(X)
#undef X
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_scale(const RmsScaleArgs &a, int mode, hipStream_t s) {
  return mode == kFast ? rms_scale_dispatch<kFast>(a, s) : rms_scale_dispatch<kLossless>(a, s);
}

template <int MODE>
static hipError_t rms_tanh_dispatch(const RmsTanhArgs &a, hipStream_t s) {
  const int nc = (int)((a.dim + 511) / 512);
  switch (nc) {
#define X(N)                                                                             \
  case N:                                                                                \
    hipLaunchKernelGGL((k_rmsnorm_tanh_residual<N, MODE>), row_grid(a.rows), dim3(256), 0, \
                       s, a);                                                            \
    break;
    DIT_NC_CASES(X)
#undef X
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_tanh_residual(const RmsTanhArgs &a, int mode, hipStream_t s) {
  return mode == kFast ? rms_tanh_dispatch<kFast>(a, s) : rms_tanh_dispatch<kLossless>(a, s);
}

hipError_t launch_residual_gate_add(const GateAddArgs &a, hipStream_t s) {
  const int nc = (int)((a.dim + 511) / 512);
  switch (nc) {
#define X(N) \
  case N:    \
    hipLaunchKernelGGL((k_residual_gate_add<N>), row_grid(a.rows), dim3(256), 0, s, a); break;
    DIT_NC_CASES(X)
#undef X
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dit

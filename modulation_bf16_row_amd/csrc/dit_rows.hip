// dit_rows.hip -- gfx950 kernels for the row epilogues and the gated
// residual + LayerNorm/AdaLN producer.
//
// Geometry.  One 64-lane wave per row at a time; lane l owns the 8-element
// vectors at 512c + 8l of chunk c (c < NC = ceil(dim / 512)), each moved
// with one 128-bit access, so a wave-wide access is 1 KiB contiguous.  A
// wave walks a contiguous run of `rows_per_wave` rows of its workgroup
// (four waves).  The row stays in VGPRs between the LayerNorm passes, so x
// is read from HBM once; latency is hidden by the other waves resident on
// the SIMD.  Outputs move with the nontemporal cache policy, row inputs
// with the per-kernel policy below, shared operands with the default one.
//
// Modulation operands.  With per-batch modulation the grid is laid out per
// modulation row: blocks_per_mod workgroups cover the rows of one
// modulation row, so all rows of a workgroup share it.  The workgroup
// converts its per-element operands once into LDS as binary32 values --
// bf(1 + scale) and shift, the RMSNorm weight and scale, tanh(gate), or
// gate -- and the waves read them with two 128-bit LDS accesses per
// 8-element vector, with no bf16 unpacking in the row loop (the kernels
// are close to their vector-ALU budget, so every instruction per element
// counts).  With per-token modulation rows are laid out consecutively and
// each row's operands are loaded (and transformed) by the wave using them.
//
// Sums follow R(dim): each lane adds its own terms in (chunk, element)
// order, then a fixed xor butterfly across the 64 lanes.
//
// Sources: AdaLN rounding points -- page "基于Agent的SGLang扩散模型Kernel优化实践"
// (tahou.com), section "数学等价不代表结果完全一致"; gated residual +
// LayerNorm/AdaLN producer -- same page, sections "将FP8量化融合到前序算子" and
// "NVFP4的三组优化"; native bf16 RMSNorm chain -- page "#34085 [diffusion] Clean
// up kernels and shared fast paths", section "关键源码片段";
// rmsnorm+tanh(gate)*x+residual and residual+gate*update -- page "AI Agent
// 驱动的 SGLang Kernel 一等公民", section 0x3 / 3.2.
#include <stdlib.h>

#include "dit_device.hpp"
#include "dit_launch.hpp"

namespace dit {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = 64 * kWavesPerBlock;

// Load policy of the streamed row inputs, per kernel, as measured on MI355X
// (Qwen-Image and Wan shapes): the nontemporal policy helps the kernels that
// read two or more row streams and slows the single-stream norms.
#ifdef DIT_NO_NT_LOAD
constexpr bool kNtLn = false, kNtRms = false, kNtTanh = false, kNtGate = false;
#else
constexpr bool kNtLn = false, kNtRms = false, kNtTanh = true, kNtGate = true;
#endif

// Register budget: at least W6 waves per SIMD at dim <= 3072 (NC <= 6),
// scaled down in proportion (rounded) for longer rows.
constexpr int waves_per_simd(int nc, int w6) {
  return nc <= 6 ? w6 : ((w6 * 6 + nc / 2) / nc > 1 ? (w6 * 6 + nc / 2) / nc : 1);
}
#define DIT_OCCUPANCY(NC, W6) __attribute__((amdgpu_waves_per_eu(waves_per_simd(NC, W6), 8)))

// Chunk c of this lane lies inside the row?  Chunks before the last are full.
template <int NC>
__device__ __forceinline__ bool valid(int c, int lane, int dim) {
  return c < NC - 1 || 512 * c + 8 * lane < dim;
}

// One row of NC vectors; STREAM selects the nontemporal policy.
template <int NC, bool STREAM>
__device__ __forceinline__ void load_row(V8 (&v)[NC], const uint16_t *base, int lane, int dim) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (valid<NC>(c, lane, dim))
      v[c] = STREAM ? load8_stream(base + 512 * c + 8 * lane) : load8(base + 512 * c + 8 * lane);
    else
      v[c] = V8{{0u, 0u, 0u, 0u}};
  }
}

// Modulation rows read by one row only (per-token) are streamed; rows shared
// by a few consecutive rows keep the default policy.
template <int NC>
__device__ __forceinline__ void load_mod_row(V8 (&v)[NC], const uint16_t *base, int lane, int dim,
                                             bool per_token) {
  if (per_token)
    load_row<NC, true>(v, base, lane, dim);
  else
    load_row<NC, false>(v, base, lane, dim);
}

// Keeps the compiler from moving instructions across this point.  Placed
// between a row's statistics and its output loop, it stops the output's
// LDS reads from being hoisted above the reductions, where they would all
// be live at once (more VGPRs, fewer waves per SIMD).
__device__ __forceinline__ void phase_barrier() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ void unpack8(const V8 &v, float (&f)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = elem(v, j);
}

// ---------------------------------------------------------------------------
// binary32 staging rows in LDS.  Element 512c + 8l + j of a row is component
// j % 4 of float4 (2c + j / 4) * 64 + l: a lane reads the 8 values of its
// chunk c with two ds_read_b128, each covering 64 consecutive float4s across
// the wave (no bank conflicts).  A staged row takes NC * 128 float4s.
// ---------------------------------------------------------------------------
template <int NC>
constexpr int stage_vecs() {
  return NC * 128;
}

// Stores the 8 values of vector v (elements 8v .. 8v + 7).
__device__ __forceinline__ void stage_put(float4 *row, int v, const float (&f)[8]) {
  const int c = v >> 6, l = v & 63;
  row[(2 * c) * 64 + l] = make_float4(f[0], f[1], f[2], f[3]);
  row[(2 * c + 1) * 64 + l] = make_float4(f[4], f[5], f[6], f[7]);
}

__device__ __forceinline__ void stage_get(const float4 *row, int c, int lane, float (&f)[8]) {
  const float4 a = row[(2 * c) * 64 + lane], b = row[(2 * c + 1) * 64 + lane];
  f[0] = a.x;
  f[1] = a.y;
  f[2] = a.z;
  f[3] = a.w;
  f[4] = b.x;
  f[5] = b.y;
  f[6] = b.z;
  f[7] = b.w;
}

// ---------------------------------------------------------------------------
// Row runs of this wave.
// ---------------------------------------------------------------------------
struct Span {
  int64_t begin, end;   // the wave's rows [begin, end) (may be empty)
  int64_t m;            // modulation row of the workgroup (staged layout only)
  bool wg_empty;        // the whole workgroup has no rows
};

// Consecutive rows: workgroup b covers rows [4 b rpw, 4 (b + 1) rpw).
__device__ __forceinline__ Span spans(int64_t rows, int64_t rpw) {
  Span s;
  const int64_t wg_first = (int64_t)blockIdx.x * kWavesPerBlock * rpw;
  s.wg_empty = wg_first >= rows;
  s.begin = wg_first + (int64_t)(threadIdx.x >> 6) * rpw;
  s.end = s.begin + rpw < rows ? s.begin + rpw : rows;
  s.m = 0;
  return s;
}

// Per modulation row: workgroup b covers block b % blocks_per_mod of the
// rows of modulation row b / blocks_per_mod; the last block of a modulation
// row may be short (its trailing waves then have no rows).
__device__ __forceinline__ Span mod_spans(int64_t per_mod, int64_t rpw, int64_t blocks_per_mod) {
  Span s;
  s.m = (int64_t)blockIdx.x / blocks_per_mod;
  const int64_t i = (int64_t)blockIdx.x - s.m * blocks_per_mod;
  const int64_t mod_end = (s.m + 1) * per_mod;
  const int64_t wg_first = s.m * per_mod + i * kWavesPerBlock * rpw;
  s.wg_empty = false;                                       // i < blocks_per_mod
  s.begin = wg_first + (int64_t)(threadIdx.x >> 6) * rpw;
  s.end = s.begin + rpw < mod_end ? s.begin + rpw : mod_end;
  return s;
}

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

// out = bf(bf(bf(d * rho) * s1) + shift); mod(c, s1, sh) gives chunk c's
// bf(1 + scale) and shift as binary32 values.  F8: also qrow = E4M3(out / qs).
template <int NC, bool F8, class Mod>
__device__ __forceinline__ void ln_modulate_out(uint16_t *orow, uint8_t *qrow, float qs,
                                                const float (&d)[NC][8], float rho, int lane,
                                                int dim, Mod mod) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (!valid<NC>(c, lane, dim)) continue;
    float s1[8], sh[8];
    mod(c, s1, sh);
    V8 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float n0 = d[c][2 * k] * rho, n1 = d[c][2 * k + 1] * rho;
      round2(n0, n1);                                           // LayerNorm output
      float p0 = n0 * s1[2 * k], p1 = n1 * s1[2 * k + 1];
      round2(p0, p1);                                           // product
      o.w[k] = pack(p0 + sh[2 * k], p1 + sh[2 * k + 1]);        // + shift
    }
    store8(orow + 512 * c + 8 * lane, o);
    if (F8) {
      uint32_t q0, q1;
      quant8(o.w, qs, q0, q1);
      store8b(qrow + 512 * c + 8 * lane, q0, q1);
    }
  }
}


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
  const float qs = F8 ? *a.fp8_scale : 1.0f;
  if (STAGED) {
    for (int v = threadIdx.x; v < dim / 8; v += kThreads) {
      float s1[8], sh[8];
      one_plus8(load8(a.scale + sp.m * a.mod_rs + 8 * v), s1);
      unpack8(load8(a.shift + sp.m * a.mod_rs + 8 * v), sh);
      stage_put(lds, v, s1);
      stage_put(lds + kRow, v, sh);
    }
    __syncthreads();
  }

  for (int64_t r = sp.begin; r < sp.end; ++r) {
    V8 xv[NC], sc[NC], sf[NC];
    load_row<NC, kNtLn>(xv, a.x + r * a.x_rs, lane, dim);
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
      ln_modulate_out<NC, F8>(orow, qrow, qs, d, rho, lane, dim,
                              [&](int c, float (&s1)[8], float (&sh)[8]) {
                                stage_get(lds, c, lane, s1);
                                stage_get(lds + kRow, c, lane, sh);
                              });
    } else {
      ln_modulate_out<NC, F8>(orow, qrow, qs, d, rho, lane, dim,
                              [&](int c, float (&s1)[8], float (&sh)[8]) {
                                one_plus8(sc[c], s1);
                                unpack8(sf[c], sh);
                              });
    }
  }
}

// ---------------------------------------------------------------------------
// Gated residual + LayerNorm + AdaLN modulate: r' = bf(residual + bf(gate * y))
// is written to out_res, and LN + modulate of r' to out.  The row is read
// once; r' never goes back through HBM before the LayerNorm.
// F8: also the E4M3 copy out8 = E4M3(out / s).
// LDS (staged): [0] = gate, [1] = bf(1 + scale), [2] = shift, binary32.
// ---------------------------------------------------------------------------
template <int NC, int MODE, bool STAGED, bool F8>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_gate_add_ln_modulate(
    GateLnArgs a) {
  extern __shared__ float4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  constexpr int kRow = stage_vecs<NC>();
  const Span sp = STAGED ? mod_spans(a.per_mod, a.rows_per_wave, a.blocks_per_mod)
                         : spans(a.rows, a.rows_per_wave);
  const float qs = F8 ? *a.fp8_scale : 1.0f;
  if (STAGED) {
    for (int v = threadIdx.x; v < dim / 8; v += kThreads) {
      const int64_t off = sp.m * a.mod_rs + 8 * v;
      float g[8], s1[8], sh[8];
      unpack8(load8(a.gate + off), g);
      one_plus8(load8(a.scale + off), s1);
      unpack8(load8(a.shift + off), sh);
      stage_put(lds, v, g);
      stage_put(lds + kRow, v, s1);
      stage_put(lds + 2 * kRow, v, sh);
    }
    __syncthreads();
  }

  for (int64_t r = sp.begin; r < sp.end; ++r) {
    const int64_t m = STAGED ? sp.m : r / a.per_mod;
    V8 xv[NC], sc[NC], sf[NC];
    {
      V8 rv[NC], yv[NC], gv[NC];
      load_row<NC, kNtGate>(rv, a.residual + r * a.res_rs, lane, dim);
      load_row<NC, kNtGate>(yv, a.y + r * a.y_rs, lane, dim);
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
      ln_modulate_out<NC, F8>(orow, qrow, qs, d, rho, lane, dim,
                              [&](int c, float (&s1)[8], float (&sh)[8]) {
                                stage_get(lds + kRow, c, lane, s1);
                                stage_get(lds + 2 * kRow, c, lane, sh);
                              });
    } else {
      ln_modulate_out<NC, F8>(orow, qrow, qs, d, rho, lane, dim,
                              [&](int c, float (&s1)[8], float (&sh)[8]) {
                                one_plus8(sc[c], s1);
                                unpack8(sf[c], sh);
                              });
    }
  }
}

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
  return round1(rsqrt_mode<MODE>(v));                    // bf16 rstd
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

// The RMSNorm weight as a staged row (every launch, both layouts).
__device__ __forceinline__ void stage_weight(float4 *row, const uint16_t *weight, int dim) {
  for (int v = threadIdx.x; v < dim / 8; v += kThreads) {
    float w[8];
    unpack8(load8(weight + 8 * v), w);
    stage_put(row, v, w);
  }
}

// LDS: [0] = weight (always), [1] = scale (staged), binary32.
template <int NC, int MODE, bool STAGED>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_rmsnorm_scale(RmsScaleArgs a) {
  extern __shared__ float4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  constexpr int kRow = stage_vecs<NC>();
  const Span sp = STAGED ? mod_spans(a.per_mod, a.rows_per_wave, a.blocks_per_mod)
                         : spans(a.rows, a.rows_per_wave);
  if (sp.wg_empty) return;                                 // whole workgroup idle
  stage_weight(lds, a.weight, dim);
  if (STAGED) {
    for (int v = threadIdx.x; v < dim / 8; v += kThreads) {
      float s[8];
      unpack8(load8(a.scale + sp.m * a.mod_rs + 8 * v), s);
      stage_put(lds + kRow, v, s);
    }
  }
  __syncthreads();

  for (int64_t r = sp.begin; r < sp.end; ++r) {
    V8 xv[NC], sc[NC];
    load_row<NC, kNtRms>(xv, a.x + r * a.x_rs, lane, dim);
    const int64_t m = STAGED ? sp.m : r / a.per_mod;
    if (!STAGED) load_mod_row<NC>(sc, a.scale + m * a.mod_rs, lane, dim, a.per_mod == 1);
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
}

// LDS: [0] = weight (always), [1] = tanh(gate) (staged), binary32; then the
// tanh table.  tanh comes from the table in both modes.
template <int NC, int MODE, bool STAGED>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_rmsnorm_tanh_residual(
    RmsTanhArgs a) {
  extern __shared__ float4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  constexpr int kRow = stage_vecs<NC>();
  uint16_t *tab = reinterpret_cast<uint16_t *>(lds + (STAGED ? 2 : 1) * kRow);
  const Span sp = STAGED ? mod_spans(a.per_mod, a.rows_per_wave, a.blocks_per_mod)
                         : spans(a.rows, a.rows_per_wave);
  if (sp.wg_empty) return;                                 // whole workgroup idle
  tanh_table_fill(tab, threadIdx.x, kThreads);
  stage_weight(lds, a.weight, dim);
  __syncthreads();
  if (STAGED) {
    for (int v = threadIdx.x; v < dim / 8; v += kThreads) {
      const V8 g = load8(a.gate + sp.m * a.mod_rs + 8 * v);
      float t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = tanh_lookup(elem(g, j), tab);
      stage_put(lds + kRow, v, t);
    }
    __syncthreads();
  }

  for (int64_t r = sp.begin; r < sp.end; ++r) {
    V8 xv[NC], rv[NC], tau[NC];
    load_row<NC, kNtTanh>(xv, a.x + r * a.x_rs, lane, dim);
    load_row<NC, kNtTanh>(rv, a.residual + r * a.res_rs, lane, dim);
    const int64_t m = STAGED ? sp.m : r / a.per_mod;
    if (!STAGED) load_mod_row<NC>(tau, a.gate + m * a.mod_rs, lane, dim, a.per_mod == 1);
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
}

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

// ---------------------------------------------------------------------------
// Launch shapes.
//   One row per wave (four per workgroup) measured fastest for every kernel:
//   at the Wan 720p shape RMSNorm-tanh-residual takes 503 us with one row
//   per wave against 574 us with four, and the Qwen-Image shapes are within
//   noise.  Per-batch modulation (at least one workgroup's worth of rows per
//   modulation row) takes the staged layout: blocks_per_mod workgroups per
//   modulation row, each converting its modulation operands into LDS once.
//   Otherwise (per-token modulation) rows are laid out consecutively and
//   each wave loads them.
// ---------------------------------------------------------------------------

// Staging several binary32 rows stops paying once it limits the workgroups
// per CU; above this LDS size the waves load the operands themselves.
constexpr size_t kMaxStagedLds = 64 * 1024;

struct Shape {
  int64_t rows_per_wave, blocks_per_mod;
  bool staged;
  dim3 grid;
};

// LDS bytes of `rows` binary32 staged rows.
static size_t stage_bytes(int64_t dim, int rows) {
  return (size_t)rows * (size_t)((dim + 511) / 512) * 128 * sizeof(float4);
}

// staged_rows: binary32 rows the staged layout keeps in LDS.
static Shape row_shape(int64_t rows, int64_t per_mod, int64_t dim, int staged_rows) {
  Shape s;
  s.rows_per_wave = 1;
#ifdef DIT_TUNING
  if (const char *e = getenv("DIT_ROWS_PER_WAVE")) s.rows_per_wave = atoll(e);
#endif
  if (s.rows_per_wave < 1) s.rows_per_wave = 1;
  const int64_t wg_rows = kWavesPerBlock * s.rows_per_wave;
  s.staged = per_mod >= wg_rows && stage_bytes(dim, staged_rows) <= kMaxStagedLds;
#ifdef DIT_TUNING
  if (getenv("DIT_NO_STAGING")) s.staged = false;
#endif
  const int64_t blocks_per_mod = (per_mod + wg_rows - 1) / wg_rows;
  if (s.staged && rows / per_mod * blocks_per_mod > 0x7FFFFFFF) s.staged = false;
  if (s.staged) {
    s.blocks_per_mod = blocks_per_mod;
    s.grid = dim3((unsigned)(rows / per_mod * blocks_per_mod));
  } else {
    s.blocks_per_mod = 0;
    s.grid = dim3((unsigned)((rows + wg_rows - 1) / wg_rows));
  }
  return s;
}

#define DIT_NC_CASES(X) \
  X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)

// Selects the instantiation NC = ceil(dim / 512) through the X macro in scope.
#define DIT_ROW_DISPATCH()                      \
  do {                                          \
    switch ((int)((a.dim + 511) / 512)) {       \
      DIT_NC_CASES(X)                           \
      default: return hipErrorInvalidValue;     \
    }                                           \
    return hipGetLastError();                   \
  } while (0)

// The staged (KT) or unstaged (KF) instantiation, with its LDS bytes.
#define DIT_ROW_LAUNCH(KT, KF, shm_t, shm_f)                        \
  if (sh.staged)                                                    \
    DIT_LAUNCH(KT, sh.grid, dim3(kThreads), shm_t, s, a);           \
  else                                                              \
    DIT_LAUNCH(KF, sh.grid, dim3(kThreads), shm_f, s, a);

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

hipError_t launch_ln_modulate(const LnModArgs &a, int mode, hipStream_t s) {
  if (a.out8)
    return mode == kFast ? ln_dispatch<kFast, true>(a, s) : ln_dispatch<kLossless, true>(a, s);
  return mode == kFast ? ln_dispatch<kFast, false>(a, s) : ln_dispatch<kLossless, false>(a, s);
}

hipError_t launch_gate_add_ln_modulate(const GateLnArgs &a, int mode, hipStream_t s) {
  if (a.out8)
    return mode == kFast ? gate_ln_dispatch<kFast, true>(a, s)
                         : gate_ln_dispatch<kLossless, true>(a, s);
  return mode == kFast ? gate_ln_dispatch<kFast, false>(a, s)
                       : gate_ln_dispatch<kLossless, false>(a, s);
}

hipError_t launch_rmsnorm_scale(const RmsScaleArgs &a, int mode, hipStream_t s) {
  return mode == kFast ? rms_scale_dispatch<kFast>(a, s) : rms_scale_dispatch<kLossless>(a, s);
}

hipError_t launch_rmsnorm_tanh_residual(const RmsTanhArgs &a, int mode, hipStream_t s) {
  return mode == kFast ? rms_tanh_dispatch<kFast>(a, s) : rms_tanh_dispatch<kLossless>(a, s);
}

hipError_t launch_residual_gate_add(const GateAddArgs &a, hipStream_t s) {
  return gate_add_dispatch(a, s);
}

}  // namespace dit

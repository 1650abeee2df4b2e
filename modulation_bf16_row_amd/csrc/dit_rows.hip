// dit_rows.hip -- gfx950 kernels for the four row epilogues.
//
// Geometry.  One 64-lane wave per row at a time; lane l owns the 8-element
// vectors at 512c + 8l of chunk c (c < NC = ceil(dim / 512)), each moved
// with one 128-bit access, so a wave-wide access is 1 KiB contiguous.  A
// wave walks a contiguous run of `rows_per_wave` rows; a 256-thread
// workgroup (four waves) covers 4 * rows_per_wave consecutive rows.  The
// row stays in VGPRs between the LayerNorm passes, so x is read from HBM
// once; latency is hidden by the other waves resident on the SIMD.  Rows
// and outputs move with the nontemporal cache policy; shared operands with
// the default one.
//
// Modulation operands.  With per-batch modulation (a workgroup's rows meet
// at most two modulation rows), the workgroup computes the per-element
// operands once into LDS -- bf(1 + scale) and shift, the RMSNorm weight and
// scale, tanh(gate), or gate -- and every wave reads them with one 128-bit
// LDS access per vector.  With per-token modulation each row's operands are
// loaded (and transformed) by the wave that uses them.
//
// Sums follow R(dim): each lane adds its own terms in (chunk, element)
// order, then a fixed xor butterfly across the 64 lanes.
//
// Sources: AdaLN rounding points -- page "基于Agent的SGLang扩散模型Kernel优化实践"
// (tahou.com), section "数学等价不代表结果完全一致"; native bf16 RMSNorm chain --
// page "#34085 [diffusion] Clean up kernels and shared fast paths", section
// "关键源码片段"; rmsnorm+tanh(gate)*x+residual and residual+gate*update --
// page "AI Agent 驱动的 SGLang Kernel 一等公民", section 0x3 / 3.2.
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

// One LDS "row" holds NC * 64 vectors of 8 bf16 (vector index = element / 8).
template <int NC>
__device__ __forceinline__ void lds_row(V8 (&v)[NC], const uint4 *row, int lane, int dim) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (valid<NC>(c, lane, dim)) {
      const uint4 u = row[64 * c + lane];
      v[c] = V8{{u.x, u.y, u.z, u.w}};
    } else {
      v[c] = V8{{0u, 0u, 0u, 0u}};
    }
  }
}

// Chunk c of this lane from one LDS row.
__device__ __forceinline__ V8 lds_vec(const uint4 *row, int c, int lane) {
  const uint4 u = row[64 * c + lane];
  return V8{{u.x, u.y, u.z, u.w}};
}

__device__ __forceinline__ void lds_put(uint4 *row, int v, const V8 &x) {
  row[v] = make_uint4(x.w[0], x.w[1], x.w[2], x.w[3]);
}

// Rows of this workgroup and of this wave.
struct Span {
  int64_t wg_first, wg_last;    // inclusive range of the workgroup (may be empty)
  int64_t begin, end;           // the wave's run [begin, end)
};

__device__ __forceinline__ Span spans(int64_t rows, int64_t rpw) {
  Span s;
  s.wg_first = (int64_t)blockIdx.x * kWavesPerBlock * rpw;
  const int64_t wg_end = s.wg_first + kWavesPerBlock * rpw;
  s.wg_last = (wg_end < rows ? wg_end : rows) - 1;
  s.begin = s.wg_first + (int64_t)(threadIdx.x >> 6) * rpw;
  s.end = s.begin + rpw < rows ? s.begin + rpw : rows;
  return s;
}

// Modulation rows of the workgroup: m0 = first, count = 1 or 2.
struct ModSlots {
  int64_t m0;
  int count;
};

__device__ __forceinline__ ModSlots mod_slots(const Span &s, int64_t per_mod) {
  ModSlots ms;
  ms.m0 = s.wg_first / per_mod;
  ms.count = (int)(s.wg_last / per_mod - ms.m0) + 1;
  return ms;
}

// ---------------------------------------------------------------------------
// LayerNorm + AdaLN modulate, as two helpers on a row held by the wave.
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

// bf(1 + scale) of each element, in place.
template <int NC>
__device__ __forceinline__ void one_plus_row(V8 (&s)[NC]) {
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int k = 0; k < 4; ++k) s[c].w[k] = pack(1.0f + lo(s[c].w[k]), 1.0f + hi(s[c].w[k]));
}

// out = bf(bf(bf(d * rho) * s1) + shift); mod(c, s1, sh) fetches chunk c's
// bf(1 + scale) and shift.
template <int NC, class Mod>
__device__ __forceinline__ void ln_modulate_out(uint16_t *orow, const float (&d)[NC][8],
                                                float rho, int lane, int dim, Mod mod) {
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (!valid<NC>(c, lane, dim)) continue;
    V8 s1, sh;
    mod(c, s1, sh);
    V8 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float n0 = d[c][2 * k] * rho, n1 = d[c][2 * k + 1] * rho;
      round2(n0, n1);                                           // LayerNorm output
      float p0 = n0 * lo(s1.w[k]), p1 = n1 * hi(s1.w[k]);
      round2(p0, p1);                                           // product
      o.w[k] = pack(p0 + lo(sh.w[k]), p1 + hi(sh.w[k]));        // + shift
    }
    store8(orow + 512 * c + 8 * lane, o);
  }
}

// ---------------------------------------------------------------------------
// LayerNorm + AdaLN modulate
// LDS (staged): [2 slot] = bf(1 + scale), [2 slot + 1] = shift.
// ---------------------------------------------------------------------------
template <int NC, int MODE, bool STAGED>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_ln_modulate(LnModArgs a) {
  extern __shared__ uint4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  const Span sp = spans(a.rows, a.rows_per_wave);
  constexpr int kRow = NC * 64;
  ModSlots ms{0, 0};
  if (STAGED) {
    if (sp.wg_first > sp.wg_last) return;                  // whole workgroup idle
    ms = mod_slots(sp, a.per_mod);
    const int nv = dim / 8;
    for (int i = threadIdx.x; i < ms.count * nv; i += kThreads) {
      const int slot = i / nv, v = i - slot * nv;
      const int64_t m = ms.m0 + slot;
      V8 s = load8(a.scale + m * a.mod_rs + 8 * v);
#pragma unroll
      for (int k = 0; k < 4; ++k) s.w[k] = pack(1.0f + lo(s.w[k]), 1.0f + hi(s.w[k]));
      lds_put(lds + (2 * slot + 0) * kRow, v, s);
      lds_put(lds + (2 * slot + 1) * kRow, v, load8(a.shift + m * a.mod_rs + 8 * v));
    }
    __syncthreads();
  }

  for (int64_t r = sp.begin; r < sp.end; ++r) {
    V8 xv[NC];
    load_row<NC, kNtLn>(xv, a.x + r * a.x_rs, lane, dim);
    const int64_t m = r / a.per_mod;
    V8 s1[NC], sh[NC];
    if (!STAGED) {
      load_mod_row<NC>(s1, a.scale + m * a.mod_rs, lane, dim, a.per_mod == 1);
      load_mod_row<NC>(sh, a.shift + m * a.mod_rs, lane, dim, a.per_mod == 1);
    }
    float d[NC][8];
    const float rho = ln_stats<NC, MODE>(xv, d, lane, dim, a.eps);
    if (STAGED) {
      const int slot = (int)(m - ms.m0);
      lds_row<NC>(s1, lds + (2 * slot + 0) * kRow, lane, dim);
      lds_row<NC>(sh, lds + (2 * slot + 1) * kRow, lane, dim);
    } else {
      one_plus_row<NC>(s1);
    }
    ln_modulate_out<NC>(a.out + r * a.out_rs, d, rho, lane, dim,
                        [&](int c, V8 &u, V8 &v) { u = s1[c]; v = sh[c]; });
  }
}

// ---------------------------------------------------------------------------
// Gated residual + LayerNorm + AdaLN modulate: r' = bf(residual + bf(gate * y))
// is written to out_res, and LN + modulate of r' to out.  The row is read
// once; r' never goes back through HBM before the LayerNorm.
// LDS (staged): [3 slot] = gate, [3 slot + 1] = bf(1 + scale), [3 slot + 2] = shift.
// ---------------------------------------------------------------------------
template <int NC, int MODE, bool STAGED>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_gate_add_ln_modulate(
    GateLnArgs a) {
  extern __shared__ uint4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  const Span sp = spans(a.rows, a.rows_per_wave);
  constexpr int kRow = NC * 64;
  ModSlots ms{0, 0};
  if (STAGED) {
    if (sp.wg_first > sp.wg_last) return;                  // whole workgroup idle
    ms = mod_slots(sp, a.per_mod);
    const int nv = dim / 8;
    for (int i = threadIdx.x; i < ms.count * nv; i += kThreads) {
      const int slot = i / nv, v = i - slot * nv;
      const int64_t off = (ms.m0 + slot) * a.mod_rs + 8 * v;
      V8 s = load8(a.scale + off);
#pragma unroll
      for (int k = 0; k < 4; ++k) s.w[k] = pack(1.0f + lo(s.w[k]), 1.0f + hi(s.w[k]));
      lds_put(lds + (3 * slot + 0) * kRow, v, load8(a.gate + off));
      lds_put(lds + (3 * slot + 1) * kRow, v, s);
      lds_put(lds + (3 * slot + 2) * kRow, v, load8(a.shift + off));
    }
    __syncthreads();
  }

  for (int64_t r = sp.begin; r < sp.end; ++r) {
    const int64_t m = r / a.per_mod;
    const int slot = STAGED ? (int)(m - ms.m0) : 0;
    V8 xv[NC];
    {
      V8 rv[NC], yv[NC], gv[NC];
      load_row<NC, kNtGate>(rv, a.residual + r * a.res_rs, lane, dim);
      load_row<NC, kNtGate>(yv, a.y + r * a.y_rs, lane, dim);
      if (STAGED)
        lds_row<NC>(gv, lds + (3 * slot) * kRow, lane, dim);
      else
        load_mod_row<NC>(gv, a.gate + m * a.mod_rs, lane, dim, a.per_mod == 1);
      uint16_t *rrow = a.out_res + r * a.out_res_rs;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float q0 = lo(gv[c].w[k]) * lo(yv[c].w[k]), q1 = hi(gv[c].w[k]) * hi(yv[c].w[k]);
          round2(q0, q1);                                       // bf(gate * y)
          xv[c].w[k] = pack(lo(rv[c].w[k]) + q0, hi(rv[c].w[k]) + q1);
        }
        if (valid<NC>(c, lane, dim)) store8(rrow + 512 * c + 8 * lane, xv[c]);
      }
    }
    float d[NC][8];
    const float rho = ln_stats<NC, MODE>(xv, d, lane, dim, a.eps);
    uint16_t *orow = a.out + r * a.out_rs;
    if (STAGED) {
      const uint4 *s1row = lds + (3 * slot + 1) * kRow, *shrow = lds + (3 * slot + 2) * kRow;
      ln_modulate_out<NC>(orow, d, rho, lane, dim, [&](int c, V8 &u, V8 &v) {
        u = lds_vec(s1row, c, lane);
        v = lds_vec(shrow, c, lane);
      });
    } else {
      const uint16_t *sc = a.scale + m * a.mod_rs + 8 * lane;
      const uint16_t *sf = a.shift + m * a.mod_rs + 8 * lane;
      const bool tok = a.per_mod == 1;
      ln_modulate_out<NC>(orow, d, rho, lane, dim, [&](int c, V8 &u, V8 &v) {
        u = tok ? load8_stream(sc + 512 * c) : load8(sc + 512 * c);
        v = tok ? load8_stream(sf + 512 * c) : load8(sf + 512 * c);
#pragma unroll
        for (int k = 0; k < 4; ++k) u.w[k] = pack(1.0f + lo(u.w[k]), 1.0f + hi(u.w[k]));
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

// y2 = bf(bf(x * rstd) * w) for the pair in word xw.
__device__ __forceinline__ void rms_y2(float &y0, float &y1, uint32_t xw, uint32_t ww,
                                       float rstd) {
  y0 = lo(xw) * rstd;
  y1 = hi(xw) * rstd;
  round2(y0, y1);
  y0 = y0 * lo(ww);
  y1 = y1 * hi(ww);
  round2(y0, y1);
}

// LDS: [0] = weight (always), [1 + slot] = scale (staged).
template <int NC, int MODE, bool STAGED>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_rmsnorm_scale(RmsScaleArgs a) {
  extern __shared__ uint4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  const Span sp = spans(a.rows, a.rows_per_wave);
  constexpr int kRow = NC * 64;
  if (sp.wg_first > sp.wg_last) return;                    // whole workgroup idle
  const ModSlots ms = STAGED ? mod_slots(sp, a.per_mod) : ModSlots{0, 0};
  {
    const int nv = dim / 8;
    for (int i = threadIdx.x; i < (1 + ms.count) * nv; i += kThreads) {
      const int t = i / nv, v = i - t * nv;
      const uint16_t *src = t == 0 ? a.weight : a.scale + (ms.m0 + t - 1) * a.mod_rs;
      lds_put(lds + t * kRow, v, load8(src + 8 * v));
    }
    __syncthreads();
  }

  for (int64_t r = sp.begin; r < sp.end; ++r) {
    V8 xv[NC], wv[NC], sc[NC];
    load_row<NC, kNtRms>(xv, a.x + r * a.x_rs, lane, dim);
    const int64_t m = r / a.per_mod;
    if (!STAGED) load_mod_row<NC>(sc, a.scale + m * a.mod_rs, lane, dim, a.per_mod == 1);
    const float rstd = rms_rstd<NC, MODE>(xv, lane, dim, a.eps);
    lds_row<NC>(wv, lds, lane, dim);
    if (STAGED) lds_row<NC>(sc, lds + (1 + (int)(m - ms.m0)) * kRow, lane, dim);
    uint16_t *orow = a.out + r * a.out_rs;
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
}

// LDS: [0] = weight (always), [1 + slot] = tanh(gate) (staged), then the
// tanh table.  tanh comes from the table in both modes.
template <int NC, int MODE, bool STAGED>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_rmsnorm_tanh_residual(
    RmsTanhArgs a) {
  extern __shared__ uint4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  const Span sp = spans(a.rows, a.rows_per_wave);
  constexpr int kRow = NC * 64;
  uint16_t *tab = reinterpret_cast<uint16_t *>(lds + (STAGED ? 3 : 1) * kRow);
  if (sp.wg_first > sp.wg_last) return;                    // whole workgroup idle
  const ModSlots ms = STAGED ? mod_slots(sp, a.per_mod) : ModSlots{0, 0};
  {
    const int nv = dim / 8;
    tanh_table_fill(tab, threadIdx.x, kThreads);
    for (int v = threadIdx.x; v < nv; v += kThreads) lds_put(lds, v, load8(a.weight + 8 * v));
    __syncthreads();
    if (STAGED) {
      for (int i = threadIdx.x; i < ms.count * nv; i += kThreads) {
        const int t = i / nv, v = i - t * nv;
        V8 g = load8(a.gate + (ms.m0 + t) * a.mod_rs + 8 * v);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          g.w[k] = pack(tanh_lookup(lo(g.w[k]), tab), tanh_lookup(hi(g.w[k]), tab));
        lds_put(lds + (1 + t) * kRow, v, g);
      }
      __syncthreads();
    }
  }

  for (int64_t r = sp.begin; r < sp.end; ++r) {
    V8 xv[NC], rv[NC], tau[NC];
    load_row<NC, kNtTanh>(xv, a.x + r * a.x_rs, lane, dim);
    load_row<NC, kNtTanh>(rv, a.residual + r * a.res_rs, lane, dim);
    const int64_t m = r / a.per_mod;
    if (!STAGED) load_mod_row<NC>(tau, a.gate + m * a.mod_rs, lane, dim, a.per_mod == 1);
    const float rstd = rms_rstd<NC, MODE>(xv, lane, dim, a.eps);
    const uint4 *trow = STAGED ? lds + (1 + (int)(m - ms.m0)) * kRow : lds;
    uint16_t *orow = a.out + r * a.out_rs;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (!valid<NC>(c, lane, dim)) continue;
      const V8 wc = lds_vec(lds, c, lane);
      float tg[8];
      if (STAGED) {
        const V8 tc = lds_vec(trow, c, lane);
#pragma unroll
        for (int j = 0; j < 8; ++j) tg[j] = elem(tc, j);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) tg[j] = tanh_lookup(elem(tau[c], j), tab);
      }
      V8 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float y0, y1;
        rms_y2(y0, y1, xv[c].w[k], wc.w[k], rstd);
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
// LDS (staged): [slot] = gate.
// ---------------------------------------------------------------------------
template <int NC, bool STAGED>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_residual_gate_add(
    GateAddArgs a) {
  extern __shared__ uint4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  const Span sp = spans(a.rows, a.rows_per_wave);
  constexpr int kRow = NC * 64;
  ModSlots ms{0, 0};
  if (STAGED) {
    if (sp.wg_first > sp.wg_last) return;
    ms = mod_slots(sp, a.per_mod);
    const int nv = dim / 8;
    for (int i = threadIdx.x; i < ms.count * nv; i += kThreads) {
      const int t = i / nv, v = i - t * nv;
      lds_put(lds + t * kRow, v, load8(a.gate + (ms.m0 + t) * a.mod_rs + 8 * v));
    }
    __syncthreads();
  }

  for (int64_t r = sp.begin; r < sp.end; ++r) {
    V8 rv[NC], yv[NC], gv[NC];
    load_row<NC, kNtGate>(rv, a.residual + r * a.res_rs, lane, dim);
    load_row<NC, kNtGate>(yv, a.y + r * a.y_rs, lane, dim);
    const int64_t m = r / a.per_mod;
    if (STAGED)
      lds_row<NC>(gv, lds + (int)(m - ms.m0) * kRow, lane, dim);
    else
      load_mod_row<NC>(gv, a.gate + m * a.mod_rs, lane, dim, a.per_mod == 1);
    uint16_t *orow = a.out + r * a.out_rs;
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
}

// ---------------------------------------------------------------------------
// Launch shape.
//   Each wave gets a run of up to max_run rows, aiming at about kTargetWaves
//   waves (MI355X: 256 CUs x 4 SIMDs x 4).  Modulation is staged in LDS when
//   every workgroup's 4 * rows_per_wave rows meet at most two modulation
//   rows (per-batch modulation); otherwise each wave loads it (per-token).
// ---------------------------------------------------------------------------
constexpr int64_t kTargetWaves = 4096;
constexpr int64_t kMaxRun = 4;

struct Shape {
  int64_t rows_per_wave;
  bool staged;
  dim3 grid;
};

// max_run: 1 for the kernels whose per-row work is cheap (measured fastest
// with one row per wave); kMaxRun where staged per-batch work (tanh) is
// worth sharing across more rows.
static Shape row_shape(int64_t rows, int64_t per_mod, int64_t max_run) {
  Shape s;
  s.rows_per_wave = (rows + kTargetWaves - 1) / kTargetWaves;
  if (s.rows_per_wave > max_run) s.rows_per_wave = max_run;
#ifdef DIT_TUNING
  if (const char *e = getenv("DIT_ROWS_PER_WAVE")) s.rows_per_wave = atoll(e);
#endif
  if (s.rows_per_wave < 1) s.rows_per_wave = 1;
  s.staged = per_mod >= kWavesPerBlock * s.rows_per_wave;
#ifdef DIT_TUNING
  if (getenv("DIT_NO_STAGING")) s.staged = false;
#endif
  const int64_t wg_rows = kWavesPerBlock * s.rows_per_wave;
  s.grid = dim3((unsigned)((rows + wg_rows - 1) / wg_rows));
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

// LDS bytes of `rows` staged rows of NC vectors each.
static size_t lds_bytes(int64_t dim, int rows) {
  return (size_t)rows * (size_t)((dim + 511) / 512) * 64 * sizeof(uint4);
}

template <int MODE>
static hipError_t ln_dispatch(LnModArgs a, hipStream_t s) {
  const Shape sh = row_shape(a.rows, a.per_mod, 1);
  a.rows_per_wave = sh.rows_per_wave;
  const size_t shm = sh.staged ? lds_bytes(a.dim, 4) : 0;
#define X(N)                                                                          \
  case N:                                                                             \
    if (sh.staged)                                                                    \
      DIT_LAUNCH((k_ln_modulate<N, MODE, true>), sh.grid, dim3(kThreads), shm, s, a); \
    else                                                                              \
      DIT_LAUNCH((k_ln_modulate<N, MODE, false>), sh.grid, dim3(kThreads), 0, s, a);  \
    break;
  DIT_ROW_DISPATCH();
#undef X
}

// Staging three modulation rows per slot stops paying once it limits the
// workgroups per CU; above this LDS size the wave loads them itself.
constexpr size_t kMaxStagedLds = 64 * 1024;

template <int MODE>
static hipError_t gate_ln_dispatch(GateLnArgs a, hipStream_t s) {
  Shape sh = row_shape(a.rows, a.per_mod, 1);
  a.rows_per_wave = sh.rows_per_wave;
  if (lds_bytes(a.dim, 6) > kMaxStagedLds) sh.staged = false;
  const size_t shm = sh.staged ? lds_bytes(a.dim, 6) : 0;
#define X(N)                                                                                 \
  case N:                                                                                    \
    if (sh.staged)                                                                           \
      DIT_LAUNCH((k_gate_add_ln_modulate<N, MODE, true>), sh.grid, dim3(kThreads), shm, s, a); \
    else                                                                                     \
      DIT_LAUNCH((k_gate_add_ln_modulate<N, MODE, false>), sh.grid, dim3(kThreads), 0, s, a); \
    break;
  DIT_ROW_DISPATCH();
#undef X
}

template <int MODE>
static hipError_t rms_scale_dispatch(RmsScaleArgs a, hipStream_t s) {
  const Shape sh = row_shape(a.rows, a.per_mod, 1);
  a.rows_per_wave = sh.rows_per_wave;
  const size_t shm = lds_bytes(a.dim, sh.staged ? 3 : 1);
#define X(N)                                                                            \
  case N:                                                                               \
    if (sh.staged)                                                                      \
      DIT_LAUNCH((k_rmsnorm_scale<N, MODE, true>), sh.grid, dim3(kThreads), shm, s, a); \
    else                                                                                \
      DIT_LAUNCH((k_rmsnorm_scale<N, MODE, false>), sh.grid, dim3(kThreads), shm, s, a); \
    break;
  DIT_ROW_DISPATCH();
#undef X
}

template <int MODE>
static hipError_t rms_tanh_dispatch(RmsTanhArgs a, hipStream_t s) {
  const Shape sh = row_shape(a.rows, a.per_mod, kMaxRun);
  a.rows_per_wave = sh.rows_per_wave;
  const size_t shm = lds_bytes(a.dim, sh.staged ? 3 : 1) + kTanhTabVecs * sizeof(uint4);
#define X(N)                                                                                  \
  case N:                                                                                     \
    if (sh.staged)                                                                            \
      DIT_LAUNCH((k_rmsnorm_tanh_residual<N, MODE, true>), sh.grid, dim3(kThreads), shm, s, \
                 a);                                                                          \
    else                                                                                      \
      DIT_LAUNCH((k_rmsnorm_tanh_residual<N, MODE, false>), sh.grid, dim3(kThreads), shm, s, \
                 a);                                                                          \
    break;
  DIT_ROW_DISPATCH();
#undef X
}

static hipError_t gate_add_dispatch(GateAddArgs a, hipStream_t s) {
  const Shape sh = row_shape(a.rows, a.per_mod, 1);
  a.rows_per_wave = sh.rows_per_wave;
  const size_t shm = sh.staged ? lds_bytes(a.dim, 2) : 0;
#define X(N)                                                                              \
  case N:                                                                                 \
    if (sh.staged)                                                                        \
      DIT_LAUNCH((k_residual_gate_add<N, true>), sh.grid, dim3(kThreads), shm, s, a);    \
    else                                                                                  \
      DIT_LAUNCH((k_residual_gate_add<N, false>), sh.grid, dim3(kThreads), 0, s, a);     \
    break;
  DIT_ROW_DISPATCH();
#undef X
}

hipError_t launch_ln_modulate(const LnModArgs &a, int mode, hipStream_t s) {
  return mode == kFast ? ln_dispatch<kFast>(a, s) : ln_dispatch<kLossless>(a, s);
}

hipError_t launch_gate_add_ln_modulate(const GateLnArgs &a, int mode, hipStream_t s) {
  return mode == kFast ? gate_ln_dispatch<kFast>(a, s) : gate_ln_dispatch<kLossless>(a, s);
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

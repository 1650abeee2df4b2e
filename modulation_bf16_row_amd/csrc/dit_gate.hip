// dit_gate.hip -- gfx950 residual gate-add, out = bf(residual + bf(gate * y))
// (page "AI Agent 驱动的 SGLang Kernel 一等公民", section 0x3 / 3.2,
// residual+gate*update; page "#34085 [diffusion] Clean up kernels and shared
// fast paths", section "实现拆解", residual_gate_add).
//
// Geometry: nothing couples the elements of a row, so the rows are not held
// by waves; the [rows, D] problem is covered as groups of 8 elements (one
// 16-byte vector each of residual, y and the gate row, one 16-byte
// nontemporal store) in row-major order, one group per lane, by one-shot
// 64-thread workgroups -- the layout that streams best on MI355X.  Per-batch
// gate rows are read with the default policy (they stay cached); per-token
// ones stream with residual and y.  Group g splits into row r = g / (D/8)
// and gate row r / (rows / mod_rows) by multiply-high division
// (dit_divide.hpp) while g fits 32 bits; larger problems take a grid-stride
// loop with 64-bit division.  Row helpers: dit_rows.hpp.
#include "dit_divide.hpp"
#include "dit_rows.hpp"

namespace dit {

constexpr int kGateThreads = 64;

// Group i of row r with gate row m.
__device__ __forceinline__ void gate_group(const GateAddArgs &a, uint64_t r, uint64_t m,
                                           uint64_t i) {
  const uint16_t *rp = a.residual + r * a.res_rs + 8 * i, *yp = a.y + r * a.y_rs + 8 * i;
  const V8 rv = kNtGate ? load8_stream(rp) : load8(rp);
  const V8 yv = kNtGate ? load8_stream(yp) : load8(yp);
  const uint16_t *gp = a.gate + m * a.mod_rs + 8 * i;
  const V8 gv = a.per_mod == 1 ? load8_stream(gp) : load8(gp);
  V8 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float q0 = lo(gv.w[k]) * lo(yv.w[k]), q1 = hi(gv.w[k]) * hi(yv.w[k]);
    round2(q0, q1);                                             // bf(gate * y)
    o.w[k] = pack(lo(rv.w[k]) + q0, hi(rv.w[k]) + q1);
  }
  store8(a.out + r * a.out_rs + 8 * i, o);
}

// 32-bit group indices: one group per lane.
__global__ __launch_bounds__(kGateThreads) void k_residual_gate_add(GateAddArgs a, uint32_t groups,
                                                                    uint64_t m_row,
                                                                    uint64_t m_mod) {
  const uint32_t g = blockIdx.x * kGateThreads + threadIdx.x;
  if (g >= groups) return;
  const uint32_t gpr = (uint32_t)(a.dim / 8);
  const uint32_t r = div_by(g, m_row), i = g - r * gpr;
  gate_group(a, r, div_by(r, m_mod), i);
}

// 64-bit group indices, grid-stride.
__global__ __launch_bounds__(kGateThreads) void k_residual_gate_add_wide(GateAddArgs a) {
  const uint64_t gpr = (uint64_t)a.dim / 8, groups = (uint64_t)a.rows * gpr;
  const uint64_t step = (uint64_t)gridDim.x * kGateThreads;
  for (uint64_t g = (uint64_t)blockIdx.x * kGateThreads + threadIdx.x; g < groups; g += step) {
    const uint64_t r = g / gpr, i = g - r * gpr;
    gate_group(a, r, r / (uint64_t)a.per_mod, i);
  }
}

hipError_t launch_residual_gate_add(const GateAddArgs &a, hipStream_t s) {
  const uint64_t groups = (uint64_t)a.rows * (uint64_t)(a.dim / 8);
  if (groups < (1ull << 32)) {
    const dim3 grid((unsigned)((groups + kGateThreads - 1) / kGateThreads));
    DIT_LAUNCH(k_residual_gate_add, grid, dim3(kGateThreads), 0, s, a, (uint32_t)groups,
               reciprocal((uint64_t)(a.dim / 8)), reciprocal((uint64_t)a.per_mod));
  } else {
    const uint64_t blocks = (groups + kGateThreads - 1) / kGateThreads;
    const dim3 grid((unsigned)(blocks < 0x7FFFFFFF ? blocks : 0x7FFFFFFF));
    DIT_LAUNCH(k_residual_gate_add_wide, grid, dim3(kGateThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dit

// dit_mod.hip -- gfx950 standalone AdaLN modulate x * (1 + scale) + shift,
// the elementwise step that follows a norm computed elsewhere (page
// "#34085 [diffusion] Clean up kernels and shared fast paths", section
// "实现拆解", the modulate_scale_shift fast path), with the eager bf16
// chain's three roundings: bf(1 + scale), the product, the sum.
//
// Geometry: nothing couples the elements of a row, so the rows are not held
// by waves; the [rows, D] problem is covered as groups of 8 elements (one
// 16-byte vector of x, of the scale row and of the shift row, one 16-byte
// nontemporal store) in row-major order, one group per lane, by one-shot
// 64-thread workgroups -- the layout that streams best on MI355X.  Per-batch
// modulation rows are read with the default policy (they stay cached);
// per-token ones, like x, stream.  Group g splits into row r = g / (D/8) and
// modulation row r / (rows / mod_rows) by multiply-high division
// (dit_divide.hpp) while g fits 32 bits; larger problems take a grid-stride
// loop with 64-bit division.  one_plus8 and the row helpers: dit_ln.hpp,
// dit_rows.hpp.
#include "dit_divide.hpp"
#include "dit_ln.hpp"

namespace dit {

constexpr int kModThreads = 64;

// out = bf(bf(x * bf(1 + scale)) + shift) for the 8 elements of group i of
// row r, modulation row m.
__device__ __forceinline__ void modulate_group(const ModArgs &a, uint64_t r, uint64_t m,
                                               uint64_t i) {
  const V8 xv = kNtMod ? load8_stream(a.x + r * a.x_rs + 8 * i) : load8(a.x + r * a.x_rs + 8 * i);
  const uint16_t *sp = a.scale + m * a.mod_rs + 8 * i, *hp = a.shift + m * a.mod_rs + 8 * i;
  const bool per_token = a.per_mod == 1;
  const V8 sc = per_token ? load8_stream(sp) : load8(sp);
  const V8 sf = per_token ? load8_stream(hp) : load8(hp);
  float s1[8], sh[8];
  one_plus8(sc, s1);
  unpack8(sf, sh);
  V8 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float p0 = lo(xv.w[k]) * s1[2 * k], p1 = hi(xv.w[k]) * s1[2 * k + 1];
    round2(p0, p1);                                             // bf(x * (1 + scale))
    o.w[k] = pack(p0 + sh[2 * k], p1 + sh[2 * k + 1]);          // + shift
  }
  store8(a.out + r * a.out_rs + 8 * i, o);
}

// 32-bit group indices: one group per lane.
__global__ __launch_bounds__(kModThreads) void k_modulate_scale_shift(ModArgs a, uint32_t groups,
                                                                      uint64_t m_row,
                                                                      uint64_t m_mod) {
  const uint32_t g = blockIdx.x * kModThreads + threadIdx.x;
  if (g >= groups) return;
  const uint32_t gpr = (uint32_t)(a.dim / 8);
  const uint32_t r = div_by(g, m_row), i = g - r * gpr;
  modulate_group(a, r, div_by(r, m_mod), i);
}

// 64-bit group indices, grid-stride.
__global__ __launch_bounds__(kModThreads) void k_modulate_scale_shift_wide(ModArgs a) {
  const uint64_t gpr = (uint64_t)a.dim / 8, groups = (uint64_t)a.rows * gpr;
  const uint64_t step = (uint64_t)gridDim.x * kModThreads;
  for (uint64_t g = (uint64_t)blockIdx.x * kModThreads + threadIdx.x; g < groups; g += step) {
    const uint64_t r = g / gpr, i = g - r * gpr;
    modulate_group(a, r, r / (uint64_t)a.per_mod, i);
  }
}

hipError_t launch_modulate_scale_shift(const ModArgs &a, hipStream_t s) {
  const uint64_t groups = (uint64_t)a.rows * (uint64_t)(a.dim / 8);
  if (groups < (1ull << 32)) {
    const dim3 grid((unsigned)((groups + kModThreads - 1) / kModThreads));
    DIT_LAUNCH(k_modulate_scale_shift, grid, dim3(kModThreads), 0, s, a, (uint32_t)groups,
               reciprocal((uint64_t)(a.dim / 8)), reciprocal((uint64_t)a.per_mod));
  } else {
    const uint64_t blocks = (groups + kModThreads - 1) / kModThreads;
    const dim3 grid((unsigned)(blocks < 0x7FFFFFFF ? blocks : 0x7FFFFFFF));
    DIT_LAUNCH(k_modulate_scale_shift_wide, grid, dim3(kModThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dit

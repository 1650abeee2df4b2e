// dit_mod.hip -- gfx950 standalone AdaLN modulate x * (1 + scale) + shift,
// the elementwise step that follows a norm computed elsewhere (page
// "基于Agent的SGLang扩散模型Kernel优化实践", section "实现拆解", the
// modulate_scale_shift fast path), with the eager bf16 chain's three
// roundings: bf(1 + scale), the product, the sum.
// Geometry, staging and launch shapes: dit_rows.hpp; one_plus8: dit_ln.hpp.
#include "dit_ln.hpp"

namespace dit {

// ---------------------------------------------------------------------------
// out = bf(bf(x * bf(1 + scale)) + shift).
// LDS (staged): [0] = bf(1 + scale), [1] = shift, binary32.
// ---------------------------------------------------------------------------
template <int NC, bool STAGED>
__global__ __launch_bounds__(kThreads) DIT_OCCUPANCY(NC, 3) void k_modulate_scale_shift(
    ModArgs a) {
  extern __shared__ float4 lds[];
  const int lane = threadIdx.x & 63, dim = (int)a.dim;
  constexpr int kRow = stage_vecs<NC>();
  const Span sp = STAGED ? mod_spans(a.per_mod, a.rows_per_wave, a.blocks_per_mod)
                         : spans(a.rows, a.rows_per_wave);
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
    load_row<NC, kNtMod>(xv, a.x + r * a.x_rs, lane, dim);
    if (!STAGED) {
      const int64_t m = r / a.per_mod;
      load_mod_row<NC>(sc, a.scale + m * a.mod_rs, lane, dim, a.per_mod == 1);
      load_mod_row<NC>(sf, a.shift + m * a.mod_rs, lane, dim, a.per_mod == 1);
    }
    uint16_t *orow = a.out + r * a.out_rs;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (!valid<NC>(c, lane, dim)) continue;
      float s1[8], sh[8];
      if (STAGED) {
        stage_get(lds, c, lane, s1);
        stage_get(lds + kRow, c, lane, sh);
      } else {
        one_plus8(sc[c], s1);
        unpack8(sf[c], sh);
      }
      V8 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float p0 = lo(xv[c].w[k]) * s1[2 * k], p1 = hi(xv[c].w[k]) * s1[2 * k + 1];
        round2(p0, p1);                                         // bf(x * (1 + scale))
        o.w[k] = pack(p0 + sh[2 * k], p1 + sh[2 * k + 1]);      // + shift
      }
      store8(orow + 512 * c + 8 * lane, o);
    }
  }
}

static hipError_t mod_dispatch(ModArgs a, hipStream_t s) {
  const Shape sh = row_shape(a.rows, a.per_mod, a.dim, 2);
  a.rows_per_wave = sh.rows_per_wave;
  a.blocks_per_mod = sh.blocks_per_mod;
#define X(N)                                                                              \
  case N:                                                                                 \
    DIT_ROW_LAUNCH((k_modulate_scale_shift<N, true>), (k_modulate_scale_shift<N, false>), \
                   stage_bytes(a.dim, 2), 0);                                             \
    break;
  DIT_ROW_DISPATCH();
#undef X
}

hipError_t launch_modulate_scale_shift(const ModArgs &a, hipStream_t s) {
  return mod_dispatch(a, s);
}

}  // namespace dit

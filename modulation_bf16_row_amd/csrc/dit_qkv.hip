// dit_qkv.hip -- gfx950 kernel for the QKV epilogue after the merged QKV
// projection: Q/K RMSNorm per head, interleaved RoPE, V copy, and placement
// of text and image tokens into joint Q/K/V buffers (page
// "基于Agent的SGLang扩散模型Kernel优化实践", section "合并QKV投影时的数值问题").
//
// Geometry: the heads of one (batch, joint token) are split into `parts`
// runs of HG head groups, one wave each; a wave walks a contiguous run of
// `tokens_per_wave` tokens (one, unless the problem is huge).  Lanes
// 16g..16g+15 hold head 4(p HG + i) + g of part p, each lane 8 elements
// (128-bit access), so a wave-wide access is 1 KiB of the token's row.
// Each lane's four RoPE pairs (4r .. 4r+3 for r = lane % 16) have their
// cos/sin loaded once per token and part and reused for every head.
// Splitting a token over several waves trades a few repeated cos/sin and
// weight reads (cache hits) for fewer VGPRs per wave and more waves.
//
// Output placement: head h lands at (h / hpd) * dest_stride + (h % hpd) * 128
// of its token's output row.  hpd = heads gives the joint [B, S, H, 128]
// layout; hpd = H / P with dest_stride = the size of one destination's block
// writes the destination-major buffer whose P contiguous chunks an
// all-to-all hands one to each rank under Ulysses sequence parallelism (page
// "基于Agent的SGLang扩散模型Kernel优化实践", section "Ulysses QKV仅执行一次All-to-All").
#include "dit_device.hpp"
#include "dit_launch.hpp"

namespace dit {

constexpr int kQkvWaves = 4;
constexpr int kHeadDim = 128;

template <int MODE>
__device__ __forceinline__ V8 norm_rope(const V8 &x, const V8 &w, const float (&c)[4],
                                        const float (&z)[4], float eps) {
  // head sum of x*x over 16 lanes (binary32, not rounded)
  float xf[8];
  float p = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    xf[j] = elem(x, j);
    if (MODE == kLossless)
      p = p + xf[j] * xf[j];
    else
      p = fmaf(xf[j], xf[j], p);
  }
  const float ms = group16_sum(p) / (float)kHeadDim;
  const float rho = rsqrt_mode<MODE>(ms + eps);
  V8 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float a = xf[2 * k] * rho, b = xf[2 * k + 1] * rho;
    round2(a, b);                                        // bf(x * rho)
    a = a * lo(w.w[k]);
    b = b * hi(w.w[k]);
    round2(a, b);                                        // bf(. * w)
    float o0, o1;
    if (MODE == kLossless) {
      o0 = a * c[k] - b * z[k];
      o1 = a * z[k] + b * c[k];
    } else {
      o0 = fmaf(a, c[k], -(b * z[k]));
      o1 = fmaf(a, z[k], b * c[k]);
    }
    o.w[k] = pack(o0, o1);
  }
  return o;
}

// Everything one token needs, as held by one lane.
template <int HG>
struct Token {
  V8 q[HG], k[HG], v[HG];
  V8 wq, wk;
  float c[4], z[4];
  int64_t dst;
};

template <int HG>
__device__ __forceinline__ void load_token(Token<HG> &t, const QkvArgs &a, int64_t tok, int g0,
                                           int g, int r) {
  const int64_t b = tok / a.s_total;
  const int64_t jt = tok - b * a.s_total;
  const bool is_txt = jt < a.txt.tokens;
  const QkvStreamArgs &st = is_txt ? a.txt : a.img;
  const int64_t s = is_txt ? jt : jt - a.txt.tokens;
  const int64_t src = b * st.batch_stride + s * st.tok_stride + 8 * r;
#pragma unroll
  for (int i = 0; i < HG; ++i) {
    const int h = 4 * (g0 + i) + g;
    if (h < a.heads) {
      t.q[i] = load8_stream(st.q + src + h * kHeadDim);
      t.k[i] = load8_stream(st.k + src + h * kHeadDim);
      t.v[i] = load8_stream(st.v + src + h * kHeadDim);
    }
  }
  t.wq = load8(st.q_weight + 8 * r);
  t.wk = load8(st.k_weight + 8 * r);
  const float4 c4 = *reinterpret_cast<const float4 *>(a.cos + jt * (kHeadDim / 2) + 4 * r);
  const float4 z4 = *reinterpret_cast<const float4 *>(a.sin + jt * (kHeadDim / 2) + 4 * r);
  t.c[0] = c4.x; t.c[1] = c4.y; t.c[2] = c4.z; t.c[3] = c4.w;
  t.z[0] = z4.x; t.z[1] = z4.y; t.z[2] = z4.z; t.z[3] = z4.w;
  t.dst = b * a.out_bs + jt * a.out_ts + 8 * r;
}

template <int HG, int MODE>
__global__ __launch_bounds__(64 * kQkvWaves) __attribute__((amdgpu_waves_per_eu(3, 8))) void k_qk_norm_rope(
    QkvArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t total = a.batch * a.s_total;
  const int64_t w = (int64_t)blockIdx.x * kQkvWaves + (threadIdx.x >> 6);
  const int64_t run = w / a.parts;
  const int part = (int)(w - run * a.parts);
  const int64_t t0 = run * a.tokens_per_wave;
  if (t0 >= total) return;
  const int64_t t1 = t0 + a.tokens_per_wave < total ? t0 + a.tokens_per_wave : total;
  const int g0 = part * HG;          // first head group of this part
  const int g = lane >> 4;           // head within the group of four
  const int r = lane & 15;           // 8-element slice of the head

  // Output offset of each of the wave's heads within a token's row: its
  // destination's block, then its position there.
  int64_t ho[HG];
#pragma unroll
  for (int i = 0; i < HG; ++i) {
    const int h = 4 * (g0 + i) + g;
    const int hpd = (int)a.heads_per_dest;
    ho[i] = (int64_t)(h / hpd) * a.dest_stride + (int64_t)(h % hpd) * kHeadDim;
  }

  for (int64_t t = t0; t < t1; ++t) {
    Token<HG> cur;
    load_token<HG>(cur, a, t, g0, g, r);
#pragma unroll
    for (int i = 0; i < HG; ++i) {
      const int h = 4 * (g0 + i) + g;
      // Lanes of absent heads (h >= heads) fill whole 16-lane groups of
      // their own, so the group sums of present heads never read them.
      if (h < a.heads) {
        store8(a.v_out + cur.dst + ho[i], cur.v[i]);
        store8(a.q_out + cur.dst + ho[i], norm_rope<MODE>(cur.q[i], cur.wq, cur.c, cur.z, a.eps));
        store8(a.k_out + cur.dst + ho[i], norm_rope<MODE>(cur.k[i], cur.wk, cur.c, cur.z, a.eps));
      }
    }
  }
}

// One token per wave run; runs only start above ~1M tokens, to bound the
// grid.  Head groups per wave: at most kQkvGroups (HG), the token's
// ceil(heads / 4) groups split into as few equal parts as that allows.  At
// the Qwen-Image shape (24 heads) one group per wave (70 VGPRs, 7 waves per
// SIMD) measured 57.3 us against 58.4, 59.8 and 64.4 us for 2, 3 and 6.
constexpr int64_t kQkvTargetWaves = int64_t(1) << 20;
constexpr int kQkvGroups = 1;

template <int MODE>
static hipError_t qkv_dispatch(QkvArgs a, hipStream_t s) {
  const int64_t total = a.batch * a.s_total;
  a.tokens_per_wave = (total + kQkvTargetWaves - 1) / kQkvTargetWaves;
  const int groups = (int)((a.heads + 3) / 4);
  const int max_hg = kQkvGroups;
  a.parts = (groups + max_hg - 1) / max_hg;
  const int hg = (groups + (int)a.parts - 1) / (int)a.parts;
  const int64_t waves = (total + a.tokens_per_wave - 1) / a.tokens_per_wave * a.parts;
  const dim3 grid((unsigned)((waves + kQkvWaves - 1) / kQkvWaves));
  switch (hg) {
#define X(N) \
  case N: DIT_LAUNCH((k_qk_norm_rope<N, MODE>), grid, dim3(64 * kQkvWaves), 0, s, a); break;
    X(1)
#undef X
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const QkvArgs &a, int mode, hipStream_t s) {
  return mode == kFast ? qkv_dispatch<kFast>(a, s) : qkv_dispatch<kLossless>(a, s);
}

}  // namespace dit

// dit_qkv.hip -- gfx950 kernel for the QKV epilogue after the merged QKV
// projection: Q/K RMSNorm per head, interleaved RoPE, V copy, and placement
// of text and image tokens into joint Q/K/V buffers (page
// "基于Agent的SGLang扩散模型Kernel优化实践", section "合并QKV投影时的数值问题").
//
// Geometry: one 64-lane wave per (batch, joint token).  The wave covers four
// heads at a time: lanes 16g..16g+15 hold head 4i+g, each lane 8 elements
// (128-bit access), so a wave-wide access is 1 KiB of one token's row.  All
// of the token's Q, K and V vectors are issued before any arithmetic (up to
// 18 vectors per lane for 24 heads) to keep many bytes in flight.  Each
// lane's four RoPE pairs (4r .. 4r+3 for r = lane % 16) have their cos/sin
// loaded once per token and reused for every head.
#include "dit_device.hpp"
#include "dit_launch.hpp"

namespace dit {

constexpr int kQkvWaves = 4;
constexpr int kHeadDim = 128;

template <int MODE>
__device__ __forceinline__ V8 norm_rope(const V8 &x, const V8 &w, const float (&c)[4],
                                        const float (&z)[4], float eps) {
  // head sum of x*x over 16 lanes (binary32, not rounded)
  float p = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float v = elem(x, j);
    if (MODE == kLossless)
      p = p + v * v;
    else
      p = fmaf(v, v, p);
  }
  const float ms = group16_sum(p) / (float)kHeadDim;
  const float rho = rsqrt_mode<MODE>(ms + eps);
  V8 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float a = lo(x.w[k]) * rho, b = hi(x.w[k]) * rho;
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

template <int HG, int MODE>
__global__ __launch_bounds__(256) void k_qk_norm_rope(QkvArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * kQkvWaves + (threadIdx.x >> 6);
  if (tok >= a.batch * a.s_total) return;
  const int64_t b = tok / a.s_total;
  const int64_t jt = tok - b * a.s_total;
  const bool is_txt = jt < a.txt.tokens;
  const QkvStreamArgs &st = is_txt ? a.txt : a.img;
  const int64_t s = is_txt ? jt : jt - a.txt.tokens;

  const int g = lane >> 4;           // head within the group of four
  const int r = lane & 15;           // 8-element slice of the head
  const int64_t src = b * st.batch_stride + s * st.tok_stride + 8 * r;
  const int64_t dst = b * a.out_bs + jt * a.out_ts + 8 * r;

  V8 qv[HG], kv[HG], vv[HG];
#pragma unroll
  for (int i = 0; i < HG; ++i) {
    const int h = 4 * i + g;
    if (h < a.heads) {
      qv[i] = load8(st.q + src + h * kHeadDim);
      kv[i] = load8(st.k + src + h * kHeadDim);
      vv[i] = load8(st.v + src + h * kHeadDim);
    }
  }
  const V8 wq = load8(st.q_weight + 8 * r);
  const V8 wk = load8(st.k_weight + 8 * r);
  const float4 c4 = *reinterpret_cast<const float4 *>(a.cos + jt * (kHeadDim / 2) + 4 * r);
  const float4 z4 = *reinterpret_cast<const float4 *>(a.sin + jt * (kHeadDim / 2) + 4 * r);
  const float c[4] = {c4.x, c4.y, c4.z, c4.w};
  const float z[4] = {z4.x, z4.y, z4.z, z4.w};

#pragma unroll
  for (int i = 0; i < HG; ++i) {
    const int h = 4 * i + g;
    // Lanes of absent heads (h >= heads) sit in whole 16-lane groups of
    // their own, so the group sums of present heads never read them.
    if (h < a.heads) {
      store8(a.v_out + dst + h * kHeadDim, vv[i]);
      store8(a.q_out + dst + h * kHeadDim, norm_rope<MODE>(qv[i], wq, c, z, a.eps));
      store8(a.k_out + dst + h * kHeadDim, norm_rope<MODE>(kv[i], wk, c, z, a.eps));
    }
  }
}

template <int MODE>
static hipError_t qkv_dispatch(const QkvArgs &a, hipStream_t s) {
  const int hg = (int)((a.heads + 3) / 4);
  const dim3 grid((unsigned)((a.batch * a.s_total + kQkvWaves - 1) / kQkvWaves));
  switch (hg) {
#define X(N) \
  case N: hipLaunchKernelGGL((k_qk_norm_rope<N, MODE>), grid, dim3(256), 0, s, a); break;
    X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)
#undef X
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const QkvArgs &a, int mode, hipStream_t s) {
  return mode == kFast ? qkv_dispatch<kFast>(a, s) : qkv_dispatch<kLossless>(a, s);
}

}  // namespace dit

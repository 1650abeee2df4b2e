// dit_device.hpp -- device primitives shared by the gfx950 epilogue kernels.
//
// Numerics: every floating-point expression here is a single binary32
// operation.  The library is built with -ffp-contract=off (no fused
// multiply-add unless written as fmaf), denormals preserved
// (.amdhsa_float_denorm_mode_32 = 3) and clang's correctly rounded fp32
// division and square root; LOSSLESS code uses only those.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dit_tanh_table.hpp"

namespace dit {

enum { kLossless = 0, kFast = 1 };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// bf16 <-> binary32.  A 32-bit word holds two bf16 values: element 2k in the
// low half, element 2k+1 in the high half (little-endian memory order).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two binary32 values -> packed bf16 pair, round to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// bf(a), bf(b) returned as their exact binary32 values.
__device__ __forceinline__ void round2(float &a, float &b) {
  uint32_t w = pack(a, b);
  a = lo(w);
  b = hi(w);
}

__device__ __forceinline__ float round1(float a) { return lo(pack(a, a)); }

// ---------------------------------------------------------------------------
// Fixed reduction trees.  Lane l adds the partial of lane l^m for each m;
// fp32 addition is commutative, so both partners hold identical bits.
// ---------------------------------------------------------------------------
// The partner value of lane l ^ m, fetched with the cheapest exact exchange:
//   m = 1, 2: DPP quad_perm [1,0,3,2] / [2,3,0,1];
//   m = 4:    DPP row_shl:4 into banks 0 and 2 (lanes 0-3, 8-11 of each row
//             of 16 read lane + 4), then row_shr:4 into banks 1 and 3;
//   m = 8:    DPP row_ror:8 (lane i of a row reads lane (i + 8) mod 16);
//   m = 16:   ds_swizzle, bit mode: and 0x1F, or 0, xor 0x10;
//   m = 32:   ds_bpermute.
// (wave_sum takes its last two stages from row_pair_add / half_pair_add.)
__device__ __forceinline__ float partner(float p, int m) {
  const int v = __float_as_int(p);
  int r;
  switch (m) {
    case 1: r = __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false); break;
    case 4:
      r = __builtin_amdgcn_update_dpp(v, v, 0x104, 0xF, 0x5, false);
      r = __builtin_amdgcn_update_dpp(r, v, 0x114, 0xF, 0xA, false);
      break;
    case 8: r = __builtin_amdgcn_update_dpp(v, v, 0x128, 0xF, 0xF, false); break;
    case 16: r = __builtin_amdgcn_ds_swizzle(v, 0x401F); break;
    default: r = __shfl_xor(v, m); break;
  }
  return __int_as_float(r);
}

__device__ __forceinline__ float xor_add(float p, int m) { return p + partner(p, m); }

// Stages m = 16 and m = 32 of the tree once every row of 16 lanes (for 16),
// or every half of 32 lanes (for 32), holds a single value: the gfx950 swaps
// v_permlane16_swap (rows 0 <-> 1 and 2 <-> 3) and v_permlane32_swap
// (lanes 0-31 <-> 32-63) hand each lane its partner row's (half's) value
// through the VALU, without the LDS round trip of ds_swizzle/ds_bpermute.
// The swapped pair sums to p_a + p_b, the same bits as the xor partner.
__device__ __forceinline__ float row_pair_add(float p) {
  const uint32_t u = __float_as_uint(p);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float half_pair_add(float p) {
  const uint32_t u = __float_as_uint(p);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// All 64 lanes: m = 1, 2, 4, 8, 16, 32.
__device__ __forceinline__ float wave_sum(float p) {
  p = xor_add(p, 1);
  p = xor_add(p, 2);
  p = xor_add(p, 4);
  p = xor_add(p, 8);
  p = row_pair_add(p);     // m = 16
  p = half_pair_add(p);    // m = 32
  return p;
}

// Groups of 16 lanes: m = 1, 2, 4, 8.
__device__ __forceinline__ float group16_sum(float p) {
  p = xor_add(p, 1);
  p = xor_add(p, 2);
  p = xor_add(p, 4);
  p = xor_add(p, 8);
  return p;
}

// ---------------------------------------------------------------------------
// tanh of a bf16 gate by table, as the row kernels use it (both modes).
//   |g| < 2^-4:   bf(tanh g) = g, since the relative change of tanh, about
//                 g^2 / 3 < 2^-9.5, is below half a bf16 spacing (>= 2^-9
//                 relative, also just below a power of two for |g| < 0.076);
//                 this covers zero and subnormals;
//   |g| >= 3.5:   +-1, since tanh(3.5) > 1 - 2^-9, the midpoint below 1;
//                 infinities give +-1, NaN stays NaN (quiet);
//   otherwise:    one of the 736 magnitudes with bf16 codes 0x3D80..0x405F,
//                 looked up in a table of their correctly rounded tanh
//                 (dit_tanh_table.hpp, written by gen_tanh_table.py from
//                 80-digit decimal arithmetic); the sign is restored.
// Each workgroup copies the 1472-byte table from global memory (an L2 hit
// after the first workgroups) into LDS.  The exhaustive device test checks
// every one of the 65536 inputs.
// ---------------------------------------------------------------------------
// Four 32-bit words as one 128-bit vector value (loads, stores, asm operands).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kTanhTabLo = 0x3D80u, kTanhTabHi = 0x4060u;
constexpr int kTanhTabN = (int)(kTanhTabHi - kTanhTabLo);             // 736
constexpr int kTanhTabVecs = (kTanhTabN * 2 + 15) / 16;               // uint4s
static_assert(kTanhTabN == kTanhTabEntries && kTanhTabN % 8 == 0, "tanh table size");

// The copy in two halves, so that a kernel can issue other loads between
// them: tanh_table_fetch loads 16 bytes of the table for thread tid (threads
// past the table reload its first vector, so every thread loads, with no
// branch), tanh_table_put stores them into LDS for tid < kTanhTabVecs (tab:
// 16-byte aligned, kTanhTabVecs uint4s; the workgroup needs at least
// kTanhTabVecs threads).  An empty asm statement that passes the address
// through keeps the load where it is written: the optimizer would otherwise
// sink it to its use, past the row loads a kernel issues in between, and as
// a wave's loads return in order the staging would then wait for the rows.
__device__ __forceinline__ uint4 tanh_table_fetch(int tid) {
  typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
  global_u32x4 *p = (global_u32x4 *)(reinterpret_cast<const u32x4 *>(kTanhTabGlobal)) +
                    (tid < kTanhTabVecs ? tid : 0);
  asm volatile("" : "+v"(p));
  const u32x4 t = *p;
  return make_uint4(t[0], t[1], t[2], t[3]);
}

__device__ __forceinline__ void tanh_table_put(uint16_t *tab, int tid, uint4 v) {
  if (tid < kTanhTabVecs) reinterpret_cast<uint4 *>(tab)[tid] = v;
}

// g is a bf16 value (low 16 bits zero).  The table index is clamped, so the
// LDS access stays inside the table for every input.
__device__ __forceinline__ float tanh_lookup(float g, const uint16_t *tab) {
  const uint32_t u = __float_as_uint(g);
  const uint32_t ab = (u >> 16) & 0x7FFFu, sign = u & 0x80000000u;
  const uint32_t i = min(ab - kTanhTabLo, (uint32_t)kTanhTabN - 1u);  // wraps when ab < lo
  const float t = __uint_as_float(((uint32_t)tab[i] << 16) | sign);
  const float big = ab > 0x7F80u ? g + g : __uint_as_float(0x3F800000u | sign);
  return ab < kTanhTabLo ? g : (ab >= kTanhTabHi ? big : t);
}

// 1 / sqrt(v): IEEE square root and division (LOSSLESS) or the hardware
// reciprocal square root (FAST).
template <int MODE>
__device__ __forceinline__ float rsqrt_mode(float v) {
  if (MODE == kLossless) return 1.0f / __builtin_sqrtf(v);
  return __builtin_amdgcn_rsqf(v);
}

// bf16 rstd of the native-bf16 RMSNorm: bf(1 / sqrt(v)) for a bf16 v.
// FAST takes the hardware reciprocal square root and keeps it unless its
// binary32 result lies within 4 steps of a bf16 rounding midpoint (low half
// 0x8000), or v is not a positive normal number; there the IEEE square root
// and division decide (a rounding test in the manner of Ziv).  The hardware
// result and the IEEE two-step one each lie within a step of the exact
// value, so away from the midpoints they round to the same bf16, and the
// bf16 rstd is the same in both modes -- checked on all 65536 bf16 inputs.
// One evaluation per row, so the test costs nothing measurable.
template <int MODE>
__device__ __forceinline__ float rstd_bf16(float v) {
  if (MODE == kLossless) return round1(1.0f / __builtin_sqrtf(v));
  float r = __builtin_amdgcn_rsqf(v);
  const uint32_t low = __float_as_uint(r) & 0xFFFFu;
  if (low - 0x7FFCu <= 8u || !(v >= 1.17549435e-38f)) r = 1.0f / __builtin_sqrtf(v);
  return round1(r);
}

// ---------------------------------------------------------------------------
// 128-bit vectors of eight bf16 values.
// ---------------------------------------------------------------------------
struct V8 {
  uint32_t w[4];
};

// Cache policy.  Streamed operands (row inputs, per-token modulation,
// outputs) are touched once per call, so they are moved with nontemporal
// loads and stores, which measured 9% faster on a pure copy than the default
// policy.  Operands shared by many rows (weights, per-batch modulation rows,
// cos/sin) use the default policy so they stay cached.

__device__ __forceinline__ V8 load8(const uint16_t *p) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  return V8{{u.x, u.y, u.z, u.w}};
}

__device__ __forceinline__ V8 load8_stream(const uint16_t *p) {
  const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return V8{{u[0], u[1], u[2], u[3]}};
}

__device__ __forceinline__ void store8(uint16_t *p, const V8 &v) {
  const u32x4 u = {v.w[0], v.w[1], v.w[2], v.w[3]};
  __builtin_nontemporal_store(u, reinterpret_cast<u32x4 *>(p));
}

// Eight bytes (two words) with a nontemporal store.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store8b(uint8_t *p, uint32_t w0, uint32_t w1) {
  const u32x2 u = {w0, w1};
  __builtin_nontemporal_store(u, reinterpret_cast<u32x2 *>(p));
}

// ---------------------------------------------------------------------------
// OCP E4M3 codes of two binary32 values: saturated to +-448 (the largest
// finite E4M3 value), then converted by v_cvt_pk_fp8_f32 (round to nearest
// even, OCP format on gfx950); NaN passes the clamp unchanged and stays NaN.
// Returns the codes of a and b in bits 0-7 and 8-15.  The device test checks
// it against the oracle's encoder on every binary32 input between 2^-11 and
// 2^10 in magnitude and on the edges outside.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sat448(float v) {
  return v == v ? fminf(fmaxf(v, -448.0f), 448.0f) : v;
}

__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false) & 0xFFFFu;
}

// The binary32 quotient v / s of a bf16 value v by a binary32 scale s, for the
// E4M3 copy, as one binary64 product with r = 1 / (double)s (computed once
// per wave with the correctly rounded binary64 division):
// (float)((double)v * r).  Wherever the IEEE binary32 quotient is a normal
// number the two are equal bit for bit: v = X 2^b with X < 2^8, s = S 2^a
// with S < 2^24, and a midpoint between normal binary32 numbers has an odd
// significand M >= 2^24 + 1, so X 2^d = M S has no solution -- v / s is never
// a midpoint -- and |v / s - m| >= |m| 2^-49 for every midpoint m; the
// binary64 product is within 2^-51.9 |v / s| of v / s (two roundings at
// 2^-53, no underflow or overflow for any binary32 operands), so it rounds
// to the same binary32 value.  Where the quotient is subnormal (below
// 2^-126) the two may differ in the last places, but every such value -- and
// the exact one -- has the E4M3 code +0 or -0 of its sign.  Zero, infinite
// and NaN operands give the IEEE results (x * 0 for s = inf, x * inf for
// s = 0, NaN for 0 / 0 and inf / inf).
__device__ __forceinline__ float div_by_scale(float v, double r) {
  return (float)((double)v * r);
}

// E4M3 codes of the eight bf16 values of v divided by the scale (r = 1 /
// (double)s, see div_by_scale), as two words (codes of elements 0-3, 4-7).
__device__ __forceinline__ void quant8(const uint32_t (&w)[4], double r, uint32_t &q0,
                                       uint32_t &q1) {
  q0 = e4m3x2(div_by_scale(__uint_as_float(w[0] << 16), r),
              div_by_scale(__uint_as_float(w[0] & 0xFFFF0000u), r)) |
       (e4m3x2(div_by_scale(__uint_as_float(w[1] << 16), r),
               div_by_scale(__uint_as_float(w[1] & 0xFFFF0000u), r)) << 16);
  q1 = e4m3x2(div_by_scale(__uint_as_float(w[2] << 16), r),
              div_by_scale(__uint_as_float(w[2] & 0xFFFF0000u), r)) |
       (e4m3x2(div_by_scale(__uint_as_float(w[3] << 16), r),
               div_by_scale(__uint_as_float(w[3] & 0xFFFF0000u), r)) << 16);
}

__device__ __forceinline__ float elem(const V8 &v, int j) {
  return (j & 1) ? hi(v.w[j >> 1]) : lo(v.w[j >> 1]);
}

}  // namespace dit

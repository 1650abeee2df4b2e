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

// Correctly rounded bf16 of a binary64 value, via a binary32 value rounded to
// odd (truncate toward zero and set the last bit if anything was dropped):
// rounding to odd with 24 bits then to nearest with 8 bits equals one
// rounding to nearest with 8 bits, since 24 >= 8 + 2.
__device__ __forceinline__ float round_f64(double v) {
  float f = (float)v;                           // nearest
  if ((double)f != v && f == f) {
    uint32_t u = __float_as_uint(f);
    if (fabs((double)f) > fabs(v)) u -= 1;      // step back toward zero
    f = __uint_as_float(u | 1u);                // sticky bit: odd
  }
  return round1(f);
}

// ---------------------------------------------------------------------------
// Fixed reduction trees.  Lane l adds the partial of lane l^m for each m;
// fp32 addition is commutative, so both partners hold identical bits.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float xor_add(float p, int m) { return p + __shfl_xor(p, m); }

// All 64 lanes: m = 1, 2, 4, 8, 16, 32.
__device__ __forceinline__ float wave_sum(float p) {
  p = xor_add(p, 1);
  p = xor_add(p, 2);
  p = xor_add(p, 4);
  p = xor_add(p, 8);
  p = xor_add(p, 16);
  p = xor_add(p, 32);
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
// tanh of a bf16 gate, rounded to bf16.
//
// binary32 evaluation: tanh(a) = e / (e + 2) with e = expm1(2a), a = |g| < 4
// (for |g| >= 4 the bf16 result is +-1).  Its error is a few binary32 ulps.
// LOSSLESS adds Ziv's rounding test: when the binary32 value lies within
// kZivUlps ulps of a bf16 rounding boundary (its low 16 bits near 0x8000),
// tanh is re-evaluated in binary64 and rounded once.  The result is then the
// correctly rounded bf16 of tanh(g) for every one of the 65536 inputs, which
// the exhaustive device test checks.
// ---------------------------------------------------------------------------
constexpr int kZivUlps = 8;

// The rare binary64 path stays out of line: one copy per kernel instead of
// one per unrolled element.
static __device__ __noinline__ float tanh_f64_bf16(float a) { return round_f64(tanh((double)a)); }

template <int MODE>
__device__ __forceinline__ float tanh_bf16(float g) {
  float a = fabsf(g);
  float r;
  if (!(a < 4.0f)) {
    r = (a == a) ? 1.0f : a + a;                // saturate; NaN stays NaN (quiet)
  } else {
    float e = expm1f(a + a);
    float t = e / (e + 2.0f);
    if (MODE == kLossless) {
      int low = (int)(__float_as_uint(t) & 0xFFFFu);
      if (abs(low - 0x8000) <= kZivUlps)
        r = tanh_f64_bf16(a);
      else
        r = round1(t);
    } else {
      r = round1(t);
    }
  }
  return copysignf(r, g);
}

// 1 / sqrt(v): IEEE square root and division (LOSSLESS) or the hardware
// reciprocal square root (FAST).
template <int MODE>
__device__ __forceinline__ float rsqrt_mode(float v) {
  if (MODE == kLossless) return 1.0f / __builtin_sqrtf(v);
  return __builtin_amdgcn_rsqf(v);
}

// ---------------------------------------------------------------------------
// 128-bit vectors of eight bf16 values.
// ---------------------------------------------------------------------------
struct V8 {
  uint32_t w[4];
};

__device__ __forceinline__ V8 load8(const uint16_t *p) {
  uint4 u = *reinterpret_cast<const uint4 *>(p);
  return V8{{u.x, u.y, u.z, u.w}};
}

__device__ __forceinline__ void store8(uint16_t *p, const V8 &v) {
  *reinterpret_cast<uint4 *>(p) = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
}

__device__ __forceinline__ float elem(const V8 &v, int j) {
  return (j & 1) ? hi(v.w[j >> 1]) : lo(v.w[j >> 1]);
}

}  // namespace dit

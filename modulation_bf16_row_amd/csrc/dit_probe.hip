// dit_probe.hip -- kernels that run the epilogue kernels' own device
// primitives (bf16 rounding, 1 + scale, tanh, the RMSNorm rstd chain, fp32
// division / square root, the two reduction trees) over caller arrays, so
// the tests can check each primitive exhaustively against the oracle.
#include "dit_device.hpp"
#include "dit_launch.hpp"

namespace dit {

__global__ void k_probe_bf16_round(uint16_t *out, const float *in, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint16_t)(pack(in[i], 0.0f) & 0xFFFFu);
}

// op 0: bf(1 + s); op 2: bf(1 / sqrt(v)) as in RMSNorm; op 3: tanh through
// the row kernels' LDS table (copied by each workgroup).  (op 1, a binary32
// evaluation of tanh, is no longer part of the library; the host rejects it.)
template <int MODE>
__global__ __launch_bounds__(256) void k_probe_unary(int op, uint16_t *out, const uint16_t *in,
                                                     int64_t n) {
  __shared__ __attribute__((aligned(16))) uint16_t tab[kTanhTabN];
  static_assert(256 >= kTanhTabVecs, "one workgroup copies the tanh table in one pass");
  if (op == 3) {                                 // op is uniform: every thread reaches the barrier
    tanh_table_put(tab, threadIdx.x, tanh_table_fetch(threadIdx.x));
    __syncthreads();
  }
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = __uint_as_float((uint32_t)in[i] << 16);
  float r;
  if (op == 0)
    r = round1(1.0f + v);
  else if (op == 2)
    r = rstd_bf16<MODE>(v);
  else
    r = tanh_lookup(v, tab);
  out[i] = (uint16_t)(__float_as_uint(r) >> 16);
}

// op 0: a / b; op 1: sqrt(a); op 2: 1 / sqrt(a) (rsqrt_mode).
template <int MODE>
__global__ void k_probe_f32(int op, float *out, const float *a, const float *b, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float r;
  if (op == 0)
    r = a[i] / b[i];
  else if (op == 1)
    r = __builtin_sqrtf(a[i]);
  else
    r = rsqrt_mode<MODE>(a[i]);
  out[i] = r;
}

// head == 0: one wave per row of `dim` terms, R(dim) order.
// head == 1: 16 lanes per 128-term group (dim must be 128).
__global__ __launch_bounds__(64) void k_probe_row_sum(float *out, const float *t, int64_t rows,
                                                      int64_t dim, int head) {
  const int lane = threadIdx.x;
  if (head == 0) {
    const int64_t row = blockIdx.x;
    if (row >= rows) return;
    const float *tr = t + row * dim;
    float p = 0.0f;
    for (int c = 0; 512 * c < dim; ++c)
      for (int j = 0; j < 8; ++j) {
        const int64_t e = 512 * c + 8 * lane + j;
        if (e < dim) p = p + tr[e];
      }
    p = wave_sum(p);
    if (lane == 0) out[row] = p;
  } else {
    const int64_t grp = (int64_t)blockIdx.x * 4 + (lane >> 4);
    if (grp >= rows) return;                     // whole 16-lane groups exit together
    const float *tr = t + grp * 128 + 8 * (lane & 15);
    float p = 0.0f;
    for (int j = 0; j < 8; ++j) p = p + tr[j];
    p = group16_sum(p);
    if ((lane & 15) == 0) out[grp] = p;
  }
}

// Streaming copy of n 16-byte vectors with the epilogues' access pattern (each
// wave moves 1 KiB contiguous per instruction): the practical HBM ceiling.
// FLAGS bit 0: nontemporal loads; bit 1: nontemporal stores.
template <int FLAGS>
__global__ __launch_bounds__(256) void k_probe_copy(u32x4 *out, const u32x4 *in, int64_t n) {
  const int64_t step = (int64_t)gridDim.x * 1024;
  for (int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x; base < n; base += step) {
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t i = base + 256 * k;
      if (i < n) v[k] = (FLAGS & 1) ? __builtin_nontemporal_load(in + i) : in[i];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t i = base + 256 * k;
      if (i < n) {
        if (FLAGS & 2)
          __builtin_nontemporal_store(v[k], out + i);
        else
          out[i] = v[k];
      }
    }
  }
}

// The flat kernels' layout: one 16-byte vector per lane, one-shot 64-thread
// workgroups.
template <int FLAGS>
__global__ __launch_bounds__(64) void k_probe_stream(u32x4 *out, const u32x4 *in, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (i >= n) return;
  const u32x4 v = (FLAGS & 1) ? __builtin_nontemporal_load(in + i) : in[i];
  if (FLAGS & 2)
    __builtin_nontemporal_store(v, out + i);
  else
    out[i] = v;
}

static dim3 flat_grid(int64_t n, int block) { return dim3((unsigned)((n + block - 1) / block)); }

hipError_t launch_probe_copy(void *out, const void *in, int64_t n16, int flags, hipStream_t s) {
  u32x4 *o = static_cast<u32x4 *>(out);
  const u32x4 *i = static_cast<const u32x4 *>(in);
  if (flags & 4) {
    const dim3 grid = flat_grid(n16, 64);
    switch (flags & 3) {
      case 0: DIT_LAUNCH(k_probe_stream<0>, grid, dim3(64), 0, s, o, i, n16); break;
      case 1: DIT_LAUNCH(k_probe_stream<1>, grid, dim3(64), 0, s, o, i, n16); break;
      case 2: DIT_LAUNCH(k_probe_stream<2>, grid, dim3(64), 0, s, o, i, n16); break;
      default: DIT_LAUNCH(k_probe_stream<3>, grid, dim3(64), 0, s, o, i, n16); break;
    }
    return hipGetLastError();
  }
  int64_t blocks = (n16 + 1023) / 1024;
  if (blocks > 256 * 16) blocks = 256 * 16;
  const dim3 grid((unsigned)blocks);
  switch (flags & 3) {
    case 0: DIT_LAUNCH(k_probe_copy<0>, grid, dim3(256), 0, s, o, i, n16); break;
    case 1: DIT_LAUNCH(k_probe_copy<1>, grid, dim3(256), 0, s, o, i, n16); break;
    case 2: DIT_LAUNCH(k_probe_copy<2>, grid, dim3(256), 0, s, o, i, n16); break;
    default: DIT_LAUNCH(k_probe_copy<3>, grid, dim3(256), 0, s, o, i, n16); break;
  }
  return hipGetLastError();
}

// op 0: E4M3 code of the binary32 in[i]; op 1: E4M3 code of the bf16 in[i]
// divided by *scale -- the quantization of the dual-output producers.
__global__ void k_probe_fp8(int op, uint8_t *out, const void *in, int64_t n, const float *scale) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v;
  if (op == 0) {
    v = static_cast<const float *>(in)[i];
  } else {
    v = div_by_scale(__uint_as_float((uint32_t) static_cast<const uint16_t *>(in)[i] << 16),
                     1.0 / (double)*scale);
  }
  out[i] = (uint8_t)(e4m3x2(v, 0.0f) & 0xFFu);
}

hipError_t launch_probe_fp8(int op, uint8_t *out, const void *in, int64_t n, const float *scale,
                            hipStream_t s) {
  DIT_LAUNCH(k_probe_fp8, flat_grid(n, 256), dim3(256), 0, s, op, out, in, n, scale);
  return hipGetLastError();
}

hipError_t launch_probe_bf16_round(uint16_t *out, const float *in, int64_t n, hipStream_t s) {
  DIT_LAUNCH(k_probe_bf16_round, flat_grid(n, 256), dim3(256), 0, s, out, in, n);
  return hipGetLastError();
}

hipError_t launch_probe_unary(int op, uint16_t *out, const uint16_t *in, int64_t n, int mode,
                              hipStream_t s) {
  if (mode == kFast)
    DIT_LAUNCH(k_probe_unary<kFast>, flat_grid(n, 256), dim3(256), 0, s, op, out, in, n);
  else
    DIT_LAUNCH(k_probe_unary<kLossless>, flat_grid(n, 256), dim3(256), 0, s, op, out, in,
                       n);
  return hipGetLastError();
}

hipError_t launch_probe_f32(int op, float *out, const float *a, const float *b, int64_t n,
                            int mode, hipStream_t s) {
  if (mode == kFast)
    DIT_LAUNCH(k_probe_f32<kFast>, flat_grid(n, 256), dim3(256), 0, s, op, out, a, b, n);
  else
    DIT_LAUNCH(k_probe_f32<kLossless>, flat_grid(n, 256), dim3(256), 0, s, op, out, a, b,
                       n);
  return hipGetLastError();
}

hipError_t launch_probe_row_sum(float *out, const float *t, int64_t rows, int64_t dim, int head,
                                hipStream_t s) {
  const dim3 grid = head ? flat_grid(rows, 4) : dim3((unsigned)rows);
  DIT_LAUNCH(k_probe_row_sum, grid, dim3(64), 0, s, out, t, rows, dim, head);
  return hipGetLastError();
}

}  // namespace dit

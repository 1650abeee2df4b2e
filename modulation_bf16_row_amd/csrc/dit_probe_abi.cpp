// dit_probe_abi.cpp -- entry points of the instrumented build
// (libdit_probe.so): the probes of the kernels' device primitives
// (dit_probe.h) and the dispatch-timing hook (dit_timing.h).  That library
// links the same kernel and guard objects as libdit.so and adds these; the
// product library carries neither the probes nor any timing state.
#include <stdint.h>

#include "dit_guard.hpp"
#include "dit_launch.hpp"
#include "dit_probe.h"
#include "dit_timing.h"

namespace {

using dit::guard::aligned16;
using dit::guard::fail;
using dit::guard::hip_status;
using dit::guard::Span;
using dit::guard::spans_overlap;

// Event pair armed by dit_time_next_launch() on this thread.
thread_local hipEvent_t g_time_start = nullptr;
thread_local hipEvent_t g_time_stop = nullptr;

bool array_ok(const void *p, int64_t n, int64_t esz) {
  return dit::guard::extent_ok(p, 0, 1, n, esz);
}

}  // namespace

bool dit::take_timing_events(hipEvent_t *start, hipEvent_t *stop) {
  if (!g_time_start && !g_time_stop) return false;
  *start = g_time_start;
  *stop = g_time_stop;
  g_time_start = g_time_stop = nullptr;
  return true;
}

extern "C" dit_status_t dit_time_next_launch(hipEvent_t start, hipEvent_t stop) {
  g_time_start = start;
  g_time_stop = stop;
  return DIT_OK;
}

extern "C" {

dit_status_t dit_probe_bf16_round(uint16_t *out, const float *in, int64_t n, hipStream_t stream) {
  if (n < 0) return fail(DIT_ERR_INVALID, "negative size");
  if (n == 0) return DIT_OK;
  if (!out || !in) return fail(DIT_ERR_INVALID, "NULL pointer");
  if (n / 256 > 0x7FFFFFFF) return fail(DIT_ERR_UNSUPPORTED, "too many elements");
  if (!array_ok(out, n, 2) || !array_ok(in, n, 4)) return fail(DIT_ERR_INVALID, "array extent");
  return hip_status(dit::launch_probe_bf16_round(out, in, n, stream));
}

dit_status_t dit_probe_unary(int op, uint16_t *out, const uint16_t *in, int64_t n, int mode,
                             hipStream_t stream) {
  if (op != DIT_PROBE_ONE_PLUS && op != DIT_PROBE_RMS_RSTD && op != DIT_PROBE_TANH_TABLE)
    return fail(DIT_ERR_INVALID, "bad op");
  if (mode != DIT_MODE_LOSSLESS && mode != DIT_MODE_FAST)
    return fail(DIT_ERR_INVALID, "unknown mode");
  if (n < 0) return fail(DIT_ERR_INVALID, "negative size");
  if (n == 0) return DIT_OK;
  if (!out || !in) return fail(DIT_ERR_INVALID, "NULL pointer");
  if (n / 256 > 0x7FFFFFFF) return fail(DIT_ERR_UNSUPPORTED, "too many elements");
  if (!array_ok(out, n, 2) || !array_ok(in, n, 2)) return fail(DIT_ERR_INVALID, "array extent");
  return hip_status(dit::launch_probe_unary(op, out, in, n, mode, stream));
}

dit_status_t dit_probe_f32(int op, float *out, const float *a, const float *b, int64_t n, int mode,
                           hipStream_t stream) {
  if (op < DIT_PROBE_DIV || op > DIT_PROBE_RSQRT) return fail(DIT_ERR_INVALID, "bad op");
  if (mode != DIT_MODE_LOSSLESS && mode != DIT_MODE_FAST)
    return fail(DIT_ERR_INVALID, "unknown mode");
  if (n < 0) return fail(DIT_ERR_INVALID, "negative size");
  if (n == 0) return DIT_OK;
  if (!out || !a || (op == DIT_PROBE_DIV && !b)) return fail(DIT_ERR_INVALID, "NULL pointer");
  if (n / 256 > 0x7FFFFFFF) return fail(DIT_ERR_UNSUPPORTED, "too many elements");
  if (!array_ok(out, n, 4) || !array_ok(a, n, 4) || (b && !array_ok(b, n, 4)))
    return fail(DIT_ERR_INVALID, "array extent");
  return hip_status(dit::launch_probe_f32(op, out, a, b, n, mode, stream));
}

dit_status_t dit_probe_fp8(int op, uint8_t *out, const void *in, int64_t n, const float *scale,
                           hipStream_t stream) {
  if (op != DIT_PROBE_E4M3 && op != DIT_PROBE_FP8_QUANT) return fail(DIT_ERR_INVALID, "bad op");
  if (n < 0) return fail(DIT_ERR_INVALID, "negative size");
  if (n == 0) return DIT_OK;
  if (!out || !in || (op == DIT_PROBE_FP8_QUANT && !scale))
    return fail(DIT_ERR_INVALID, "NULL pointer");
  if (n / 256 > 0x7FFFFFFF) return fail(DIT_ERR_UNSUPPORTED, "too many elements");
  if (!array_ok(out, n, 1) || !array_ok(in, n, op == DIT_PROBE_E4M3 ? 4 : 2))
    return fail(DIT_ERR_INVALID, "array extent");
  return hip_status(dit::launch_probe_fp8(op, out, in, n, scale, stream));
}

dit_status_t dit_probe_copy(void *out, const void *in, int64_t bytes, int flags,
                            hipStream_t stream) {
  if (bytes < 0) return fail(DIT_ERR_INVALID, "negative size");
  if (flags < 0 || flags > 7) return fail(DIT_ERR_INVALID, "flags must be in [0, 7]");
  if (bytes == 0) return DIT_OK;
  if (!out || !in) return fail(DIT_ERR_INVALID, "NULL pointer");
  if (bytes % 16 != 0 || !aligned16(out) || !aligned16(in))
    return fail(DIT_ERR_UNSUPPORTED, "bytes and pointers must be multiples of 16");
  if (!array_ok(out, bytes, 1) || !array_ok(in, bytes, 1))
    return fail(DIT_ERR_INVALID, "array extent");
  if ((flags & 4) && bytes / 16 / 64 >= 0x7FFFFFFF)
    return fail(DIT_ERR_UNSUPPORTED, "too many vectors for the one-shot layout");
  if (spans_overlap(Span{reinterpret_cast<uintptr_t>(out), 0, 1, bytes},
                    Span{reinterpret_cast<uintptr_t>(in), 0, 1, bytes}))
    return fail(DIT_ERR_INVALID, "buffers overlap");
  return hip_status(dit::launch_probe_copy(out, in, bytes / 16, flags, stream));
}

dit_status_t dit_probe_row_sum(float *out, const float *t, int64_t rows, int64_t dim, int head,
                               hipStream_t stream) {
  if (rows < 0 || dim < 0) return fail(DIT_ERR_INVALID, "negative size");
  if (head != 0 && head != 1) return fail(DIT_ERR_INVALID, "head must be 0 or 1");
  if (rows == 0) return DIT_OK;
  if (!out || !t) return fail(DIT_ERR_INVALID, "NULL pointer");
  if (head == 0 && (dim == 0 || dim > DIT_MAX_DIM || dim % 8 != 0))
    return fail(DIT_ERR_UNSUPPORTED, "dim must be a multiple of 8 in [8, 8192]");
  if (head == 1 && dim != DIT_QK_HEAD_DIM) return fail(DIT_ERR_UNSUPPORTED, "dim must be 128");
  if (rows > 0x7FFFFFFF) return fail(DIT_ERR_UNSUPPORTED, "too many rows");
  if (!array_ok(out, rows, 4) || !array_ok(t, rows * dim, 4))
    return fail(DIT_ERR_INVALID, "array extent");
  return hip_status(dit::launch_probe_row_sum(out, t, rows, dim, head, stream));
}

}  // extern "C"

// dit_abi.cpp -- extern "C" entry points of the epilogue library: argument
// guards (pure host code, run before any HIP call) and dispatch to the
// kernel launchers.
//
// The guard rules follow the eligibility checks the pages describe for the
// shared native-bf16 kernels (page "#34085 [diffusion] Clean up kernels and
// shared fast paths", sections "实现拆解" and "关键源码片段": same device, all
// bf16, hidden size at most 8192, non-empty, weight shape and contiguity,
// flat row stride, rows divisible by modulation rows).  Where those return
// "no fast path" to the caller, this library returns DIT_ERR_UNSUPPORTED
// with a reason -- never a silent fallback.
#include <stdint.h>

#include <algorithm>

#include "dit.h"
#include "dit_guard.hpp"
#include "dit_launch.hpp"
#include "dit_producers.h"

namespace dit {
namespace guard {

namespace {
thread_local const char *g_reason = "";

using i128 = __int128;

i128 floor_div(i128 a, i128 b) {  // b > 0
  i128 q = a / b;
  return (a % b != 0 && a < 0) ? q - 1 : q;
}
}  // namespace

dit_status_t fail(dit_status_t s, const char *why) {
  g_reason = why;
  return s;
}

const char *reason() { return g_reason; }

dit_status_t hip_status(hipError_t e) {
  if (e != hipSuccess) return fail(DIT_ERR_HIP, hipGetErrorString(e));
  return DIT_OK;
}

bool extent_ok(const void *p, int64_t step, int64_t count, int64_t len, int64_t esz) {
  if (count <= 0 || len <= 0) return true;
  const i128 bytes = ((i128)(count - 1) * step + len) * esz;
  if (bytes > kMaxExtentBytes) return false;
  const unsigned __int128 end = (unsigned __int128)reinterpret_cast<uintptr_t>(p) + bytes;
  return end <= ((unsigned __int128)1 << 64);
}

bool spans_overlap(Span a, Span b) {
  if (a.count <= 0 || b.count <= 0 || a.len <= 0 || b.len <= 0) return false;
  if (a.count == 1 || a.step <= 0) { a.count = 1; a.step = b.step; }
  if (b.count == 1 || b.step <= 0) { b.count = 1; b.step = a.step; }
  const i128 a0 = (i128)a.base, b0 = (i128)b.base;
  const i128 a_end = a0 + (i128)(a.count - 1) * a.step + a.len;
  const i128 b_end = b0 + (i128)(b.count - 1) * b.step + b.len;
  if (a_end <= b0 || b_end <= a0) return false;
  if (a.step != b.step || a.step <= 0) return true;
  // overlap iff -a.len < delta + m*step < b.len for some m in
  // [-(a.count-1), b.count-1], delta = b.base - a.base
  const i128 delta = b0 - a0;
  i128 m = floor_div(-(i128)a.len - delta, a.step) + 1;
  m = std::max(m, -(i128)(a.count - 1));
  if (m > (i128)(b.count - 1)) return false;
  return delta + m * a.step < b.len;
}

}  // namespace guard
}  // namespace dit

namespace {

using dit::guard::aligned16;
using dit::guard::fail;
using dit::guard::hip_status;
using dit::guard::Span;
using dit::guard::spans_overlap;

// Byte segments of a flat row tensor (element stride 1, bf16).  The row
// stride only matters when there is more than one row.
Span rows_span(const void *p, int64_t rs, int64_t rows, int64_t dim) {
  return Span{reinterpret_cast<uintptr_t>(p), rows > 1 ? rs * 2 : 0, rows, dim * 2};
}

// Common checks of a row tensor argument; returns DIT_OK or the failure.
// The extent check comes before any other arithmetic on the stride.
dit_status_t check_rows(const void *p, int64_t rs, int64_t rows, int64_t dim, const char *null_msg,
                        const char *stride_msg) {
  if (!p) return fail(DIT_ERR_INVALID, null_msg);
  if (rs < 0) return fail(DIT_ERR_INVALID, stride_msg);
  if (!dit::guard::extent_ok(p, rs, rows, dim, 2))
    return fail(DIT_ERR_INVALID, "tensor extent exceeds 2^56 bytes or the address space");
  if (rows > 1 && (rs < dim || rs % 8 != 0)) return fail(DIT_ERR_UNSUPPORTED, stride_msg);
  if (!aligned16(p)) return fail(DIT_ERR_UNSUPPORTED, "tensor pointer is not 16-byte aligned");
  return DIT_OK;
}

// Shared checks of the four row ops.  `ins` are row inputs that `out` may
// equal exactly; `consts` are inputs it must not touch at all.
struct RowProblem {
  int64_t rows, dim, mod_rows;
  int mode;
};

// Row counts up to 4 (2^31 - 1): the row kernels' grids hold at most 2^31 - 1
// workgroups of four rows.
constexpr int64_t kMaxRows = int64_t(4) * 0x7FFFFFFF;

dit_status_t check_shape(const RowProblem &p, bool has_mode) {
  if (has_mode && p.mode != DIT_MODE_LOSSLESS && p.mode != DIT_MODE_FAST)
    return fail(DIT_ERR_INVALID, "unknown mode");
  if (p.rows < 0 || p.dim < 0 || p.mod_rows < 0)
    return fail(DIT_ERR_INVALID, "negative size");
  if (p.rows == 0) return DIT_OK;
  if (p.dim == 0) return fail(DIT_ERR_UNSUPPORTED, "dim == 0");
  if (p.dim > DIT_MAX_DIM) return fail(DIT_ERR_UNSUPPORTED, "dim > 8192");
  if (p.dim % 8 != 0) return fail(DIT_ERR_UNSUPPORTED, "dim % 8 != 0");
  if (p.mod_rows == 0) return fail(DIT_ERR_INVALID, "mod_rows == 0 with rows > 0");
  if (p.rows % p.mod_rows != 0) return fail(DIT_ERR_UNSUPPORTED, "rows % mod_rows != 0");
  if (p.rows > kMaxRows) return fail(DIT_ERR_UNSUPPORTED, "too many rows");
  return DIT_OK;
}

dit_status_t check_out_alias(const Span &out, const Span *ins, int n_ins, const Span *consts,
                             int n_consts) {
  for (int i = 0; i < n_ins; ++i) {
    const bool same = ins[i].base == out.base && (ins[i].step == out.step || out.count == 1);
    if (!same && spans_overlap(out, ins[i]))
      return fail(DIT_ERR_INVALID, "output partially overlaps a row input");
  }
  for (int i = 0; i < n_consts; ++i)
    if (spans_overlap(out, consts[i]))
      return fail(DIT_ERR_INVALID, "output overlaps a modulation or weight tensor");
  return DIT_OK;
}

#define DIT_TRY(expr)                    \
  do {                                   \
    dit_status_t _s = (expr);            \
    if (_s != DIT_OK) return _s;         \
  } while (0)

const uint16_t *u16(const void *p) { return static_cast<const uint16_t *>(p); }

}  // namespace

extern "C" {

int dit_abi_version(void) { return DIT_ABI_VERSION; }

const char *dit_status_string(dit_status_t s) {
  switch (s) {
    case DIT_OK: return "DIT_OK";
    case DIT_ERR_UNSUPPORTED: return "DIT_ERR_UNSUPPORTED";
    case DIT_ERR_INVALID: return "DIT_ERR_INVALID";
    case DIT_ERR_HIP: return "DIT_ERR_HIP";
  }
  return "DIT_STATUS_UNKNOWN";
}

const char *dit_status_reason(void) { return dit::guard::reason(); }

dit_status_t dit_ln_modulate(void *out, int64_t out_rs, const void *x, int64_t x_rs,
                             const void *scale, const void *shift, int64_t mod_rs,
                             int64_t mod_rows, int64_t rows, int64_t dim, float eps, int mode,
                             hipStream_t stream) {
  const RowProblem p{rows, dim, mod_rows, mode};
  DIT_TRY(check_shape(p, true));
  if (rows == 0) return DIT_OK;
  DIT_TRY(check_rows(out, out_rs, rows, dim, "out is NULL", "bad out row stride"));
  DIT_TRY(check_rows(x, x_rs, rows, dim, "x is NULL", "bad x row stride"));
  DIT_TRY(check_rows(scale, mod_rs, mod_rows, dim, "scale is NULL", "bad modulation row stride"));
  DIT_TRY(check_rows(shift, mod_rs, mod_rows, dim, "shift is NULL", "bad modulation row stride"));
  const Span so = rows_span(out, out_rs, rows, dim);
  const Span ins[] = {rows_span(x, x_rs, rows, dim)};
  const Span cs[] = {rows_span(scale, mod_rs, mod_rows, dim),
                     rows_span(shift, mod_rs, mod_rows, dim)};
  DIT_TRY(check_out_alias(so, ins, 1, cs, 2));
  dit::LnModArgs a{static_cast<uint16_t *>(out), u16(x), u16(scale), u16(shift), out_rs, x_rs,
                   mod_rs, rows, dim, rows / mod_rows, eps};
  return hip_status(dit::launch_ln_modulate(a, mode, stream));
}

dit_status_t dit_rmsnorm_scale(void *out, int64_t out_rs, const void *x, int64_t x_rs,
                               const void *weight, const void *scale, int64_t mod_rs,
                               int64_t mod_rows, int64_t rows, int64_t dim, float eps, int mode,
                               hipStream_t stream) {
  const RowProblem p{rows, dim, mod_rows, mode};
  DIT_TRY(check_shape(p, true));
  if (rows == 0) return DIT_OK;
  DIT_TRY(check_rows(out, out_rs, rows, dim, "out is NULL", "bad out row stride"));
  DIT_TRY(check_rows(x, x_rs, rows, dim, "x is NULL", "bad x row stride"));
  DIT_TRY(check_rows(weight, dim, 1, dim, "weight is NULL", "bad weight"));
  DIT_TRY(check_rows(scale, mod_rs, mod_rows, dim, "scale is NULL", "bad modulation row stride"));
  const Span so = rows_span(out, out_rs, rows, dim);
  const Span ins[] = {rows_span(x, x_rs, rows, dim)};
  const Span cs[] = {rows_span(weight, dim, 1, dim), rows_span(scale, mod_rs, mod_rows, dim)};
  DIT_TRY(check_out_alias(so, ins, 1, cs, 2));
  dit::RmsScaleArgs a{static_cast<uint16_t *>(out), u16(x), u16(weight), u16(scale), out_rs,
                      x_rs, mod_rs, rows, dim, rows / mod_rows, eps};
  return hip_status(dit::launch_rmsnorm_scale(a, mode, stream));
}

dit_status_t dit_rmsnorm_tanh_residual(void *out, int64_t out_rs, const void *x, int64_t x_rs,
                                       const void *residual, int64_t res_rs, const void *weight,
                                       const void *gate, int64_t mod_rs, int64_t mod_rows,
                                       int64_t rows, int64_t dim, float eps, int mode,
                                       hipStream_t stream) {
  const RowProblem p{rows, dim, mod_rows, mode};
  DIT_TRY(check_shape(p, true));
  if (rows == 0) return DIT_OK;
  DIT_TRY(check_rows(out, out_rs, rows, dim, "out is NULL", "bad out row stride"));
  DIT_TRY(check_rows(x, x_rs, rows, dim, "x is NULL", "bad x row stride"));
  DIT_TRY(check_rows(residual, res_rs, rows, dim, "residual is NULL", "bad residual row stride"));
  DIT_TRY(check_rows(weight, dim, 1, dim, "weight is NULL", "bad weight"));
  DIT_TRY(check_rows(gate, mod_rs, mod_rows, dim, "gate is NULL", "bad modulation row stride"));
  const Span so = rows_span(out, out_rs, rows, dim);
  const Span ins[] = {rows_span(x, x_rs, rows, dim), rows_span(residual, res_rs, rows, dim)};
  const Span cs[] = {rows_span(weight, dim, 1, dim), rows_span(gate, mod_rs, mod_rows, dim)};
  DIT_TRY(check_out_alias(so, ins, 2, cs, 2));
  dit::RmsTanhArgs a{static_cast<uint16_t *>(out), u16(x), u16(residual), u16(weight),
                     u16(gate), out_rs, x_rs, res_rs, mod_rs, rows, dim, rows / mod_rows, eps};
  return hip_status(dit::launch_rmsnorm_tanh_residual(a, mode, stream));
}

dit_status_t dit_residual_gate_add(void *out, int64_t out_rs, const void *residual,
                                   int64_t res_rs, const void *y, int64_t y_rs, const void *gate,
                                   int64_t mod_rs, int64_t mod_rows, int64_t rows, int64_t dim,
                                   int mode, hipStream_t stream) {
  const RowProblem p{rows, dim, mod_rows, mode};
  DIT_TRY(check_shape(p, true));
  if (rows == 0) return DIT_OK;
  DIT_TRY(check_rows(out, out_rs, rows, dim, "out is NULL", "bad out row stride"));
  DIT_TRY(check_rows(residual, res_rs, rows, dim, "residual is NULL", "bad residual row stride"));
  DIT_TRY(check_rows(y, y_rs, rows, dim, "y is NULL", "bad y row stride"));
  DIT_TRY(check_rows(gate, mod_rs, mod_rows, dim, "gate is NULL", "bad modulation row stride"));
  const Span so = rows_span(out, out_rs, rows, dim);
  const Span ins[] = {rows_span(residual, res_rs, rows, dim), rows_span(y, y_rs, rows, dim)};
  const Span cs[] = {rows_span(gate, mod_rs, mod_rows, dim)};
  DIT_TRY(check_out_alias(so, ins, 2, cs, 1));
  dit::GateAddArgs a{static_cast<uint16_t *>(out), u16(residual), u16(y), u16(gate), out_rs,
                     res_rs, y_rs, mod_rs, rows, dim, rows / mod_rows};
  return hip_status(dit::launch_residual_gate_add(a, stream));
}

dit_status_t dit_modulate_scale_shift(void *out, int64_t out_rs, const void *x, int64_t x_rs,
                                      const void *scale, const void *shift, int64_t mod_rs,
                                      int64_t mod_rows, int64_t rows, int64_t dim, int mode,
                                      hipStream_t stream) {
  const RowProblem p{rows, dim, mod_rows, mode};
  DIT_TRY(check_shape(p, true));
  if (rows == 0) return DIT_OK;
  DIT_TRY(check_rows(out, out_rs, rows, dim, "out is NULL", "bad out row stride"));
  DIT_TRY(check_rows(x, x_rs, rows, dim, "x is NULL", "bad x row stride"));
  DIT_TRY(check_rows(scale, mod_rs, mod_rows, dim, "scale is NULL", "bad modulation row stride"));
  DIT_TRY(check_rows(shift, mod_rs, mod_rows, dim, "shift is NULL", "bad modulation row stride"));
  const Span so = rows_span(out, out_rs, rows, dim);
  const Span ins[] = {rows_span(x, x_rs, rows, dim)};
  const Span cs[] = {rows_span(scale, mod_rs, mod_rows, dim),
                     rows_span(shift, mod_rs, mod_rows, dim)};
  DIT_TRY(check_out_alias(so, ins, 1, cs, 2));
  dit::ModArgs a{static_cast<uint16_t *>(out), u16(x), u16(scale), u16(shift), out_rs, x_rs,
                 mod_rs, rows, dim, rows / mod_rows};
  return hip_status(dit::launch_modulate_scale_shift(a, stream));
}

dit_status_t dit_gate_add_ln_modulate(void *out_residual, int64_t out_res_rs, void *out,
                                      int64_t out_rs, const void *residual, int64_t res_rs,
                                      const void *y, int64_t y_rs, const void *gate,
                                      const void *scale, const void *shift, int64_t mod_rs,
                                      int64_t mod_rows, int64_t rows, int64_t dim, float eps,
                                      int mode, hipStream_t stream) {
  const RowProblem p{rows, dim, mod_rows, mode};
  DIT_TRY(check_shape(p, true));
  if (rows == 0) return DIT_OK;
  DIT_TRY(check_rows(out_residual, out_res_rs, rows, dim, "out_residual is NULL",
                     "bad out_residual row stride"));
  DIT_TRY(check_rows(out, out_rs, rows, dim, "out is NULL", "bad out row stride"));
  DIT_TRY(check_rows(residual, res_rs, rows, dim, "residual is NULL", "bad residual row stride"));
  DIT_TRY(check_rows(y, y_rs, rows, dim, "y is NULL", "bad y row stride"));
  DIT_TRY(check_rows(gate, mod_rs, mod_rows, dim, "gate is NULL", "bad modulation row stride"));
  DIT_TRY(check_rows(scale, mod_rs, mod_rows, dim, "scale is NULL", "bad modulation row stride"));
  DIT_TRY(check_rows(shift, mod_rs, mod_rows, dim, "shift is NULL", "bad modulation row stride"));
  const Span sr = rows_span(out_residual, out_res_rs, rows, dim);
  const Span so = rows_span(out, out_rs, rows, dim);
  const Span ins[] = {rows_span(residual, res_rs, rows, dim), rows_span(y, y_rs, rows, dim)};
  const Span cs[] = {rows_span(gate, mod_rs, mod_rows, dim),
                     rows_span(scale, mod_rs, mod_rows, dim),
                     rows_span(shift, mod_rs, mod_rows, dim)};
  DIT_TRY(check_out_alias(sr, ins, 2, cs, 3));
  DIT_TRY(check_out_alias(so, ins, 2, cs, 3));
  if (spans_overlap(sr, so)) return fail(DIT_ERR_INVALID, "the two outputs overlap");
  dit::GateLnArgs a{static_cast<uint16_t *>(out_residual), static_cast<uint16_t *>(out),
                    u16(residual), u16(y), u16(gate), u16(scale), u16(shift), out_res_rs, out_rs,
                    res_rs, y_rs, mod_rs, rows, dim, rows / mod_rows, eps};
  return hip_status(dit::launch_gate_add_ln_modulate(a, mode, stream));
}

}  // extern "C"

namespace {

// Checks of the E4M3 output of the dual-output producers: a byte row tensor
// (8-byte aligned, row stride a multiple of 8 bytes) that overlaps no other
// argument, and a 4-byte aligned scale that no output touches.
dit_status_t check_fp8(void *out8, int64_t out8_rs, const float *fp8_scale, int64_t rows,
                       int64_t dim, const Span *others, int n_others) {
  if (!out8) return fail(DIT_ERR_INVALID, "out_fp8 is NULL");
  if (!fp8_scale) return fail(DIT_ERR_INVALID, "fp8_scale is NULL");
  if (out8_rs < 0) return fail(DIT_ERR_INVALID, "bad out_fp8 row stride");
  if (!dit::guard::extent_ok(out8, out8_rs, rows, dim, 1))
    return fail(DIT_ERR_INVALID, "out_fp8 extent exceeds 2^56 bytes or the address space");
  if (rows > 1 && (out8_rs < dim || out8_rs % 8 != 0))
    return fail(DIT_ERR_UNSUPPORTED, "bad out_fp8 row stride");
  if ((reinterpret_cast<uintptr_t>(out8) & 7u) != 0)
    return fail(DIT_ERR_UNSUPPORTED, "out_fp8 is not 8-byte aligned");
  if ((reinterpret_cast<uintptr_t>(fp8_scale) & 3u) != 0)
    return fail(DIT_ERR_UNSUPPORTED, "fp8_scale is not 4-byte aligned");
  const Span s8{reinterpret_cast<uintptr_t>(out8), rows > 1 ? out8_rs : 0, rows, dim};
  const Span sc{reinterpret_cast<uintptr_t>(fp8_scale), 0, 1, 4};
  if (spans_overlap(s8, sc)) return fail(DIT_ERR_INVALID, "out_fp8 overlaps fp8_scale");
  for (int i = 0; i < n_others; ++i) {
    if (spans_overlap(s8, others[i])) return fail(DIT_ERR_INVALID, "out_fp8 overlaps a tensor");
  }
  return DIT_OK;
}

}  // namespace

extern "C" {

dit_status_t dit_wan_modulation_table(float *out, const float *table, const void *temb,
                                      int64_t batch, int64_t tokens, int64_t n_mod, int64_t dim,
                                      hipStream_t stream) {
  if (batch < 0 || tokens < 0 || n_mod < 0 || dim < 0)
    return fail(DIT_ERR_INVALID, "negative size");
  if (batch == 0 || tokens == 0 || n_mod == 0) return DIT_OK;
  if (dim == 0 || dim % 8 != 0)
    return fail(DIT_ERR_UNSUPPORTED, "dim must be a positive multiple of 8");
  if (!out || !table || !temb) return fail(DIT_ERR_INVALID, "NULL pointer");
  if (!aligned16(out) || !aligned16(table) || !aligned16(temb))
    return fail(DIT_ERR_UNSUPPORTED, "tensor pointer is not 16-byte aligned");
  if (n_mod > 64) return fail(DIT_ERR_UNSUPPORTED, "n_mod > 64");
  if (batch > (int64_t(1) << 32) / tokens || dim > 65536)
    return fail(DIT_ERR_UNSUPPORTED, "problem too large");
  const int64_t n = n_mod * batch * tokens * dim;   // <= 2^54: bounded above
  if (!dit::guard::extent_ok(out, 0, 1, n, 4) || !dit::guard::extent_ok(temb, 0, 1, n, 2) ||
      !dit::guard::extent_ok(table, 0, 1, n_mod * dim, 4))
    return fail(DIT_ERR_INVALID, "tensor extent exceeds 2^56 bytes or the address space");
  const Span so{reinterpret_cast<uintptr_t>(out), 0, 1, n * 4};
  const Span st{reinterpret_cast<uintptr_t>(table), 0, 1, n_mod * dim * 4};
  const Span se{reinterpret_cast<uintptr_t>(temb), 0, 1, n * 2};
  if (spans_overlap(so, st) || spans_overlap(so, se))
    return fail(DIT_ERR_INVALID, "out overlaps an input");
  dit::ModTableArgs a{out, table, u16(temb), batch, tokens, n_mod, dim};
  return hip_status(dit::launch_wan_mod_table(a, stream));
}

dit_status_t dit_ln_modulate_fp8(void *out, int64_t out_rs, void *out_fp8, int64_t out_fp8_rs,
                                 const void *x, int64_t x_rs, const void *scale,
                                 const void *shift, int64_t mod_rs, int64_t mod_rows,
                                 int64_t rows, int64_t dim, float eps, const float *fp8_scale,
                                 int mode, hipStream_t stream) {
  const RowProblem p{rows, dim, mod_rows, mode};
  DIT_TRY(check_shape(p, true));
  if (rows == 0) return DIT_OK;
  DIT_TRY(check_rows(out, out_rs, rows, dim, "out is NULL", "bad out row stride"));
  DIT_TRY(check_rows(x, x_rs, rows, dim, "x is NULL", "bad x row stride"));
  DIT_TRY(check_rows(scale, mod_rs, mod_rows, dim, "scale is NULL", "bad modulation row stride"));
  DIT_TRY(check_rows(shift, mod_rs, mod_rows, dim, "shift is NULL", "bad modulation row stride"));
  const Span so = rows_span(out, out_rs, rows, dim);
  const Span ins[] = {rows_span(x, x_rs, rows, dim)};
  const Span cs[] = {rows_span(scale, mod_rs, mod_rows, dim),
                     rows_span(shift, mod_rs, mod_rows, dim)};
  DIT_TRY(check_out_alias(so, ins, 1, cs, 2));
  const Span sc{reinterpret_cast<uintptr_t>(fp8_scale), 0, 1, 4};
  if (fp8_scale && spans_overlap(so, sc)) return fail(DIT_ERR_INVALID, "out overlaps fp8_scale");
  const Span others[] = {so, ins[0], cs[0], cs[1]};
  DIT_TRY(check_fp8(out_fp8, out_fp8_rs, fp8_scale, rows, dim, others, 4));
  dit::LnModArgs a{static_cast<uint16_t *>(out), u16(x), u16(scale), u16(shift), out_rs, x_rs,
                   mod_rs, rows, dim, rows / mod_rows, eps};
  a.out8 = static_cast<uint8_t *>(out_fp8);
  a.out8_rs = out_fp8_rs;
  a.fp8_scale = fp8_scale;
  return hip_status(dit::launch_ln_modulate(a, mode, stream));
}

dit_status_t dit_gate_add_ln_modulate_fp8(
    void *out_residual, int64_t out_res_rs, void *out, int64_t out_rs, void *out_fp8,
    int64_t out_fp8_rs, const void *residual, int64_t res_rs, const void *y, int64_t y_rs,
    const void *gate, const void *scale, const void *shift, int64_t mod_rs, int64_t mod_rows,
    int64_t rows, int64_t dim, float eps, const float *fp8_scale, int mode, hipStream_t stream) {
  const RowProblem p{rows, dim, mod_rows, mode};
  DIT_TRY(check_shape(p, true));
  if (rows == 0) return DIT_OK;
  DIT_TRY(check_rows(out_residual, out_res_rs, rows, dim, "out_residual is NULL",
                     "bad out_residual row stride"));
  DIT_TRY(check_rows(out, out_rs, rows, dim, "out is NULL", "bad out row stride"));
  DIT_TRY(check_rows(residual, res_rs, rows, dim, "residual is NULL", "bad residual row stride"));
  DIT_TRY(check_rows(y, y_rs, rows, dim, "y is NULL", "bad y row stride"));
  DIT_TRY(check_rows(gate, mod_rs, mod_rows, dim, "gate is NULL", "bad modulation row stride"));
  DIT_TRY(check_rows(scale, mod_rs, mod_rows, dim, "scale is NULL", "bad modulation row stride"));
  DIT_TRY(check_rows(shift, mod_rs, mod_rows, dim, "shift is NULL", "bad modulation row stride"));
  const Span sr = rows_span(out_residual, out_res_rs, rows, dim);
  const Span so = rows_span(out, out_rs, rows, dim);
  const Span ins[] = {rows_span(residual, res_rs, rows, dim), rows_span(y, y_rs, rows, dim)};
  const Span cs[] = {rows_span(gate, mod_rs, mod_rows, dim),
                     rows_span(scale, mod_rs, mod_rows, dim),
                     rows_span(shift, mod_rs, mod_rows, dim)};
  DIT_TRY(check_out_alias(sr, ins, 2, cs, 3));
  DIT_TRY(check_out_alias(so, ins, 2, cs, 3));
  if (spans_overlap(sr, so)) return fail(DIT_ERR_INVALID, "the two outputs overlap");
  const Span sc{reinterpret_cast<uintptr_t>(fp8_scale), 0, 1, 4};
  if (fp8_scale && (spans_overlap(so, sc) || spans_overlap(sr, sc)))
    return fail(DIT_ERR_INVALID, "an output overlaps fp8_scale");
  const Span others[] = {sr, so, ins[0], ins[1], cs[0], cs[1], cs[2]};
  DIT_TRY(check_fp8(out_fp8, out_fp8_rs, fp8_scale, rows, dim, others, 7));
  dit::GateLnArgs a{static_cast<uint16_t *>(out_residual), static_cast<uint16_t *>(out),
                    u16(residual), u16(y), u16(gate), u16(scale), u16(shift), out_res_rs, out_rs,
                    res_rs, y_rs, mod_rs, rows, dim, rows / mod_rows, eps};
  a.out8 = static_cast<uint8_t *>(out_fp8);
  a.out8_rs = out_fp8_rs;
  a.fp8_scale = fp8_scale;
  return hip_status(dit::launch_gate_add_ln_modulate(a, mode, stream));
}

}  // extern "C"

namespace {

// Up to three (stride, count) levels of a strided view whose innermost
// runs are `width` elements: segment offsets sum_i k_i * stride_i, k_i <
// count_i.  Levels with one entry or stride 0 add no segments.
struct Lattice {
  int64_t stride[3], count[3];
};

// The view's segments as one Span: exact-or-wider (step = the smallest
// stride, every multiple of it up to the last offset) when each stride is a
// multiple of the smallest, else one segment covering the hull.
Span lattice_span(const void *p, const Lattice &l, int64_t width) {
  const uintptr_t base = reinterpret_cast<uintptr_t>(p);
  int64_t inner = 0, last = 0;
  for (int i = 0; i < 3; ++i)
    if (l.count[i] > 1 && l.stride[i] > 0) {
      last += (l.count[i] - 1) * l.stride[i];
      if (inner == 0 || l.stride[i] < inner) inner = l.stride[i];
    }
  if (inner == 0) return Span{base, 0, 1, width * 2};
  for (int i = 0; i < 3; ++i)
    if (l.count[i] > 1 && l.stride[i] > 0 && l.stride[i] % inner != 0)
      return Span{base, 0, 1, (last + width) * 2};
  return Span{base, inner * 2, last / inner + 1, width * 2};
}

// True when the view (elements of `esz` bytes) spans at most
// kMaxExtentBytes and stays inside the address space.  Checked before any
// other arithmetic on its strides.
bool lattice_extent_ok(const void *p, const Lattice &l, int64_t width, int64_t esz) {
  __int128 last = 0;
  for (int i = 0; i < 3; ++i)
    if (l.count[i] > 1) last += (__int128)(l.count[i] - 1) * l.stride[i];
  if (last > dit::guard::kMaxExtentBytes) return false;
  return dit::guard::extent_ok(p, (int64_t)last, 2, width, esz);
}

// True when the view's segments are pairwise disjoint because its levels
// nest: in increasing stride order each stride is at least the extent of
// everything inside it.  (A sufficient test; layouts whose levels
// interleave are rejected.)
bool lattice_disjoint(const Lattice &l, int64_t width) {
  int idx[3] = {0, 1, 2};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (l.stride[idx[j]] < l.stride[idx[i]]) std::swap(idx[i], idx[j]);
  int64_t extent = width;
  for (int i : idx) {
    if (l.count[i] <= 1) continue;
    if (l.stride[i] < extent) return false;
    extent += (l.count[i] - 1) * l.stride[i];
  }
  return true;
}

// Segments of a [batch, tokens, w] view with token stride ts and batch stride bs.
Span token_span(const void *p, int64_t ts, int64_t bs, int64_t batch, int64_t tokens,
                int64_t width) {
  return lattice_span(p, Lattice{{ts, bs, 0}, {tokens, batch, 1}}, width);
}

dit_status_t check_stream(const dit_qkv_stream_t *st, int64_t batch, int64_t width) {
  if (st->tokens < 0) return fail(DIT_ERR_INVALID, "negative token count");
  if (st->tokens == 0) return DIT_OK;
  if (!st->q || !st->k || !st->v || !st->q_weight || !st->k_weight)
    return fail(DIT_ERR_INVALID, "stream pointer is NULL");
  if (st->tok_stride < 0 || st->batch_stride < 0)
    return fail(DIT_ERR_INVALID, "negative stream stride");
  if (batch > 0x7FFFFFFF || st->tokens > (int64_t(1) << 40))
    return fail(DIT_ERR_UNSUPPORTED, "too many tokens");
  if ((st->tokens > 1 && st->tok_stride < width) || st->tok_stride % 8 != 0)
    return fail(DIT_ERR_UNSUPPORTED, "stream token stride");
  if (batch > 1 && (st->batch_stride % 8 != 0 || st->batch_stride < width))
    return fail(DIT_ERR_UNSUPPORTED, "stream batch stride");
  const void *ps[] = {st->q, st->k, st->v, st->q_weight, st->k_weight};
  for (const void *p : ps)
    if (!aligned16(p)) return fail(DIT_ERR_UNSUPPORTED, "stream pointer is not 16-byte aligned");
  const Lattice l{{st->tok_stride, st->batch_stride, 0}, {st->tokens, batch, 1}};
  for (const void *p : {st->q, st->k, st->v})
    if (!lattice_extent_ok(p, l, width, 2))
      return fail(DIT_ERR_INVALID, "stream extent exceeds 2^56 bytes or the address space");
  return DIT_OK;
}

dit_status_t qkv_impl(void *q_out, void *k_out, void *v_out, int64_t out_tok_stride,
                      int64_t out_batch_stride, int64_t heads_per_dest, int64_t dest_stride,
                      const dit_qkv_stream_t *txt, const dit_qkv_stream_t *img, const float *cos,
                      const float *sin, int64_t batch, int64_t heads, int64_t head_dim, float eps,
                      int mode, hipStream_t stream) {
  if (mode != DIT_MODE_LOSSLESS && mode != DIT_MODE_FAST)
    return fail(DIT_ERR_INVALID, "unknown mode");
  if (batch < 0 || heads < 0 || head_dim < 0) return fail(DIT_ERR_INVALID, "negative size");
  const dit_qkv_stream_t empty{};
  const dit_qkv_stream_t *st_txt = txt ? txt : &empty;
  const dit_qkv_stream_t *st_img = img ? img : &empty;
  if (st_txt->tokens < 0 || st_img->tokens < 0)
    return fail(DIT_ERR_INVALID, "negative token count");
  int64_t s_total;
  if (__builtin_add_overflow(st_txt->tokens, st_img->tokens, &s_total))
    return fail(DIT_ERR_UNSUPPORTED, "too many tokens");
  if (batch == 0 || heads == 0 || s_total == 0) return DIT_OK;
  if (head_dim != DIT_QK_HEAD_DIM) return fail(DIT_ERR_UNSUPPORTED, "head_dim != 128");
  if (heads > 64) return fail(DIT_ERR_UNSUPPORTED, "heads > 64");
  if (heads_per_dest <= 0 || heads % heads_per_dest != 0)
    return fail(DIT_ERR_INVALID, "heads_per_dest must divide heads");
  const int64_t dests = heads / heads_per_dest;
  if (dest_stride < 0) return fail(DIT_ERR_INVALID, "negative destination stride");
  if (dests > 1 && dest_stride % 8 != 0)
    return fail(DIT_ERR_UNSUPPORTED, "destination stride % 8 != 0");
  const int64_t width = heads * head_dim;         // one token of an input stream
  const int64_t dwidth = heads_per_dest * head_dim;  // one token of one destination
  DIT_TRY(check_stream(st_txt, batch, width));
  DIT_TRY(check_stream(st_img, batch, width));
  if (!q_out || !k_out || !v_out || !cos || !sin)
    return fail(DIT_ERR_INVALID, "output or table pointer is NULL");
  if (out_tok_stride < 0 || out_batch_stride < 0)
    return fail(DIT_ERR_INVALID, "negative output stride");
  if (out_tok_stride % 8 != 0 || out_batch_stride % 8 != 0)
    return fail(DIT_ERR_UNSUPPORTED, "output strides");
  const Lattice lo{{out_tok_stride, out_batch_stride, dest_stride}, {s_total, batch, dests}};
  for (const void *p : {q_out, k_out, v_out})
    if (!lattice_extent_ok(p, lo, dwidth, 2))
      return fail(DIT_ERR_INVALID, "output extent exceeds 2^56 bytes or the address space");
  if (!lattice_disjoint(lo, dwidth))
    return fail(DIT_ERR_UNSUPPORTED, "output strides make an output overlap itself");
  const void *ps[] = {q_out, k_out, v_out, cos, sin};
  for (const void *p : ps)
    if (!aligned16(p)) return fail(DIT_ERR_UNSUPPORTED, "pointer is not 16-byte aligned");
  if ((__int128)batch * s_total > kMaxRows) return fail(DIT_ERR_UNSUPPORTED, "too many tokens");
  if (!dit::guard::extent_ok(cos, 0, 1, s_total * (head_dim / 2), 4) ||
      !dit::guard::extent_ok(sin, 0, 1, s_total * (head_dim / 2), 4))
    return fail(DIT_ERR_INVALID, "table extent exceeds the address space");

  const Span outs[3] = {lattice_span(q_out, lo, dwidth), lattice_span(k_out, lo, dwidth),
                        lattice_span(v_out, lo, dwidth)};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (spans_overlap(outs[i], outs[j]))
        return fail(DIT_ERR_INVALID, "joint outputs overlap each other");
  Span ins[12];
  int n = 0;
  const dit_qkv_stream_t *sts[2] = {st_txt, st_img};
  for (const dit_qkv_stream_t *st : sts) {
    if (st->tokens == 0) continue;
    for (const void *p : {st->q, st->k, st->v})
      ins[n++] = token_span(p, st->tok_stride, st->batch_stride, batch, st->tokens, width);
    ins[n++] = Span{reinterpret_cast<uintptr_t>(st->q_weight), 0, 1, head_dim * 2};
    ins[n++] = Span{reinterpret_cast<uintptr_t>(st->k_weight), 0, 1, head_dim * 2};
  }
  ins[n++] = Span{reinterpret_cast<uintptr_t>(cos), 0, 1, s_total * (head_dim / 2) * 4};
  ins[n++] = Span{reinterpret_cast<uintptr_t>(sin), 0, 1, s_total * (head_dim / 2) * 4};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < n; ++j)
      if (spans_overlap(outs[i], ins[j])) return fail(DIT_ERR_INVALID, "output overlaps an input");

  dit::QkvArgs a;
  a.q_out = static_cast<uint16_t *>(q_out);
  a.k_out = static_cast<uint16_t *>(k_out);
  a.v_out = static_cast<uint16_t *>(v_out);
  a.out_ts = out_tok_stride;
  a.out_bs = out_batch_stride;
  const dit_qkv_stream_t *src[2] = {st_txt, st_img};
  dit::QkvStreamArgs *dst[2] = {&a.txt, &a.img};
  for (int i = 0; i < 2; ++i) {
    dst[i]->q = u16(src[i]->q);
    dst[i]->k = u16(src[i]->k);
    dst[i]->v = u16(src[i]->v);
    dst[i]->q_weight = u16(src[i]->q_weight);
    dst[i]->k_weight = u16(src[i]->k_weight);
    dst[i]->tok_stride = src[i]->tok_stride;
    dst[i]->batch_stride = src[i]->batch_stride;
    dst[i]->tokens = src[i]->tokens;
  }
  a.cos = cos;
  a.sin = sin;
  a.batch = batch;
  a.heads = heads;
  a.s_total = s_total;
  a.heads_per_dest = heads_per_dest;
  a.dest_stride = dests > 1 ? dest_stride : 0;
  a.eps = eps;
  return hip_status(dit::launch_qk_norm_rope(a, mode, stream));
}

}  // namespace

extern "C" dit_status_t dit_qk_norm_rope(void *q_out, void *k_out, void *v_out,
                                         int64_t out_tok_stride, int64_t out_batch_stride,
                                         const dit_qkv_stream_t *txt, const dit_qkv_stream_t *img,
                                         const float *cos, const float *sin, int64_t batch,
                                         int64_t heads, int64_t head_dim, float eps, int mode,
                                         hipStream_t stream) {
  return qkv_impl(q_out, k_out, v_out, out_tok_stride, out_batch_stride, heads > 0 ? heads : 1, 0,
                  txt, img, cos, sin, batch, heads, head_dim, eps, mode, stream);
}

extern "C" dit_status_t dit_qk_norm_rope_dest(void *q_out, void *k_out, void *v_out,
                                              int64_t out_tok_stride, int64_t out_batch_stride,
                                              int64_t heads_per_dest, int64_t dest_stride,
                                              const dit_qkv_stream_t *txt,
                                              const dit_qkv_stream_t *img, const float *cos,
                                              const float *sin, int64_t batch, int64_t heads,
                                              int64_t head_dim, float eps, int mode,
                                              hipStream_t stream) {
  return qkv_impl(q_out, k_out, v_out, out_tok_stride, out_batch_stride, heads_per_dest,
                  dest_stride, txt, img, cos, sin, batch, heads, head_dim, eps, mode, stream);
}

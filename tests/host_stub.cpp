// host_stub.cpp -- stand-ins for the kernel launchers, linked with the real
// C-ABI layer (dit_abi.cpp) into a CPU-only test library.  Each launcher
// records what it was asked to launch instead of touching a GPU, so the
// tests can check the host guards' accept paths and the arguments they pass
// on, without a device.
#include <string.h>

#include "dit_launch.hpp"

extern "C" {
int stub_calls = 0;
char stub_name[32] = "";
int64_t stub_vals[16];
int stub_mode = -1;
}

static void rec(const char *name, int mode, const int64_t *v, int n) {
  ++stub_calls;
  strncpy(stub_name, name, sizeof stub_name - 1);
  stub_mode = mode;
  for (int i = 0; i < 16; ++i) stub_vals[i] = i < n ? v[i] : 0;
}

namespace dit {

hipError_t launch_ln_modulate(const LnModArgs &a, int mode, hipStream_t) {
  const int64_t v[] = {a.rows, a.dim, a.per_mod, a.out_rs, a.x_rs, a.mod_rs, a.out8 != nullptr,
                       a.out8_rs};
  rec(a.out8 ? "ln_modulate_fp8" : "ln_modulate", mode, v, 8);
  return hipSuccess;
}

hipError_t launch_gate_add_ln_modulate(const GateLnArgs &a, int mode, hipStream_t) {
  const int64_t v[] = {a.rows,   a.dim,  a.per_mod, a.out_res_rs,        a.out_rs,
                       a.res_rs, a.y_rs, a.mod_rs,  a.out8 != nullptr, a.out8_rs};
  rec(a.out8 ? "gate_add_ln_modulate_fp8" : "gate_add_ln_modulate", mode, v, 10);
  return hipSuccess;
}

hipError_t launch_rmsnorm_scale(const RmsScaleArgs &a, int mode, hipStream_t) {
  const int64_t v[] = {a.rows, a.dim, a.per_mod, a.out_rs, a.x_rs, a.mod_rs};
  rec("rmsnorm_scale", mode, v, 6);
  return hipSuccess;
}

hipError_t launch_rmsnorm_tanh_residual(const RmsTanhArgs &a, int mode, hipStream_t) {
  const int64_t v[] = {a.rows, a.dim, a.per_mod, a.out_rs, a.x_rs, a.mod_rs, a.res_rs};
  rec("rmsnorm_tanh_residual", mode, v, 7);
  return hipSuccess;
}

hipError_t launch_residual_gate_add(const GateAddArgs &a, hipStream_t) {
  const int64_t v[] = {a.rows, a.dim, a.per_mod, a.out_rs, a.res_rs, a.mod_rs, a.y_rs};
  rec("residual_gate_add", 0, v, 7);
  return hipSuccess;
}

hipError_t launch_qk_norm_rope(const QkvArgs &a, int mode, hipStream_t) {
  const int64_t v[] = {a.batch,       a.heads,          a.s_total,         a.out_ts,
                       a.out_bs,      a.txt.tokens,     a.img.tokens,      a.txt.tok_stride,
                       a.img.tok_stride, a.heads_per_dest, a.dest_stride};
  rec("qk_norm_rope", mode, v, 11);
  return hipSuccess;
}

hipError_t launch_modulate_scale_shift(const ModArgs &a, hipStream_t) {
  const int64_t v[] = {a.rows, a.dim, a.per_mod, a.out_rs, a.x_rs, a.mod_rs};
  rec("modulate_scale_shift", 0, v, 6);
  return hipSuccess;
}

hipError_t launch_wan_mod_table(const ModTableArgs &a, hipStream_t) {
  const int64_t v[] = {a.batch, a.tokens, a.n_mod, a.dim};
  rec("wan_mod_table", 0, v, 4);
  return hipSuccess;
}

hipError_t launch_probe_fp8(int op, uint8_t *, const void *, int64_t n, const float *,
                            hipStream_t) {
  rec("probe_fp8", op, &n, 1);
  return hipSuccess;
}

hipError_t launch_probe_bf16_round(uint16_t *, const float *, int64_t n, hipStream_t) {
  rec("probe_bf16_round", 0, &n, 1);
  return hipSuccess;
}

hipError_t launch_probe_unary(int op, uint16_t *, const uint16_t *, int64_t n, int mode,
                              hipStream_t) {
  const int64_t v[] = {op, n};
  rec("probe_unary", mode, v, 2);
  return hipSuccess;
}

hipError_t launch_probe_f32(int op, float *, const float *, const float *, int64_t n, int mode,
                            hipStream_t) {
  const int64_t v[] = {op, n};
  rec("probe_f32", mode, v, 2);
  return hipSuccess;
}

hipError_t launch_probe_row_sum(float *, const float *, int64_t rows, int64_t dim, int head,
                                hipStream_t) {
  const int64_t v[] = {rows, dim, head};
  rec("probe_row_sum", 0, v, 3);
  return hipSuccess;
}

hipError_t launch_probe_copy(void *, const void *, int64_t n16, int flags, hipStream_t) {
  const int64_t v[] = {n16, flags};
  rec("probe_copy", 0, v, 2);
  return hipSuccess;
}

}  // namespace dit

// dit_launch.hpp -- internal kernel argument blocks and launchers.  The
// C-ABI layer validates every argument before it fills these.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

// Event pair registered by dit_time_next_launch() on the calling thread;
// returns false when none is pending.  Taking the pair clears it.
bool take_timing_events(hipEvent_t *start, hipEvent_t *stop);

// Kernel launch that, when a timing pair is pending, lets the dispatch
// itself record the start and stop events (hipExtLaunchKernelGGL).
#define DIT_LAUNCH(kernel, grid, block, shmem, stream, ...)                              \
  do {                                                                                   \
    hipEvent_t dit_ev_start_, dit_ev_stop_;                                              \
    if (::dit::take_timing_events(&dit_ev_start_, &dit_ev_stop_))                        \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, dit_ev_start_, dit_ev_stop_, \
                            0, __VA_ARGS__);                                             \
    else                                                                                 \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);               \
  } while (0)

struct LnModArgs {
  uint16_t *out;
  const uint16_t *x, *scale, *shift;
  int64_t out_rs, x_rs, mod_rs;
  int64_t rows, dim, per_mod;  // per_mod = rows / mod_rows
  float eps;
  int64_t rows_per_wave;       // set by the launcher
  int64_t blocks_per_mod;      // set by the launcher (staged layout)
  // BF16 + E4M3 dual output (null out8: BF16 only)
  uint8_t *out8;
  int64_t out8_rs;
  const float *fp8_scale;
};

struct GateLnArgs {
  uint16_t *out_res, *out;
  const uint16_t *residual, *y, *gate, *scale, *shift;
  int64_t out_res_rs, out_rs, res_rs, y_rs, mod_rs;
  int64_t rows, dim, per_mod;  // per_mod = rows / mod_rows
  float eps;
  int64_t rows_per_wave;       // set by the launcher
  int64_t blocks_per_mod;      // set by the launcher (staged layout)
  // BF16 + E4M3 dual output (null out8: BF16 only)
  uint8_t *out8;
  int64_t out8_rs;
  const float *fp8_scale;
};

struct RmsScaleArgs {
  uint16_t *out;
  const uint16_t *x, *weight, *scale;
  int64_t out_rs, x_rs, mod_rs;
  int64_t rows, dim, per_mod;
  float eps;
  int64_t rows_per_wave;       // set by the launcher
  int64_t blocks_per_mod;      // set by the launcher (staged layout)
};

struct RmsTanhArgs {
  uint16_t *out;
  const uint16_t *x, *residual, *weight, *gate;
  int64_t out_rs, x_rs, res_rs, mod_rs;
  int64_t rows, dim, per_mod;
  float eps;
  int64_t rows_per_wave;       // set by the launcher
  int64_t blocks_per_mod;      // set by the launcher (staged layout)
};

struct GateAddArgs {
  uint16_t *out;
  const uint16_t *residual, *y, *gate;
  int64_t out_rs, res_rs, y_rs, mod_rs;
  int64_t rows, dim, per_mod;
};

struct ModArgs {
  uint16_t *out;
  const uint16_t *x, *scale, *shift;
  int64_t out_rs, x_rs, mod_rs;
  int64_t rows, dim, per_mod;
};

struct QkvStreamArgs {
  const uint16_t *q, *k, *v;
  const uint16_t *q_weight, *k_weight;
  int64_t tok_stride, batch_stride;
  int64_t tokens;
};

struct QkvArgs {
  uint16_t *q_out, *k_out, *v_out;
  int64_t out_ts, out_bs;
  QkvStreamArgs txt, img;
  const float *cos, *sin;
  int64_t batch, heads, s_total;
  // Head h is written at (h / heads_per_dest) * dest_stride + (h % heads_per_dest) * 128
  // within its token's output row (heads_per_dest = heads: plain joint layout).
  int64_t heads_per_dest, dest_stride;
  float eps;
  int64_t tokens_per_wave;     // set by the launcher
  int64_t parts;               // set by the launcher: waves sharing one token's heads
};

struct ModTableArgs {
  float *out;                  // [n_mod, batch, tokens, dim]
  const float *table;          // [n_mod, dim]
  const uint16_t *temb;        // [batch, tokens, n_mod, dim] bf16
  int64_t batch, tokens, n_mod, dim;
};

hipError_t launch_wan_mod_table(const ModTableArgs &a, hipStream_t s);
hipError_t launch_ln_modulate(const LnModArgs &a, int mode, hipStream_t s);
hipError_t launch_gate_add_ln_modulate(const GateLnArgs &a, int mode, hipStream_t s);
hipError_t launch_rmsnorm_scale(const RmsScaleArgs &a, int mode, hipStream_t s);
hipError_t launch_rmsnorm_tanh_residual(const RmsTanhArgs &a, int mode, hipStream_t s);
hipError_t launch_residual_gate_add(const GateAddArgs &a, hipStream_t s);
hipError_t launch_modulate_scale_shift(const ModArgs &a, hipStream_t s);
hipError_t launch_qk_norm_rope(const QkvArgs &a, int mode, hipStream_t s);

// Device-primitive probes (exhaustive tests of the kernels' own helpers).
hipError_t launch_probe_bf16_round(uint16_t *out, const float *in, int64_t n, hipStream_t s);
hipError_t launch_probe_unary(int op, uint16_t *out, const uint16_t *in, int64_t n, int mode,
                              hipStream_t s);
hipError_t launch_probe_f32(int op, float *out, const float *a, const float *b, int64_t n,
                            int mode, hipStream_t s);
hipError_t launch_probe_row_sum(float *out, const float *t, int64_t rows, int64_t dim, int head,
                                hipStream_t s);
hipError_t launch_probe_copy(void *out, const void *in, int64_t n16, int flags, hipStream_t s);
hipError_t launch_probe_fp8(int op, uint8_t *out, const void *in, int64_t n, const float *scale,
                            hipStream_t s);

}  // namespace dit

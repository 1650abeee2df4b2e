/*
 * dit.h -- C ABI of the BF16 DiT row-epilogue library for MI355X (gfx950).
 *
 * Five fused, memory-bound epilogues of a diffusion-transformer (DiT) block,
 * each one hand-written HIP kernel:
 *
 *   dit_ln_modulate            LayerNorm then AdaLN modulate
 *   dit_rmsnorm_scale          native-bf16 RMSNorm, weight, then scale
 *   dit_rmsnorm_tanh_residual  native-bf16 RMSNorm, weight, tanh(gate) product,
 *                              residual add
 *   dit_residual_gate_add      residual + gate * y
 *   dit_qk_norm_rope           Q/K RMSNorm per head, interleaved RoPE, V copy,
 *                              text and image tokens written to joint Q/K/V
 *
 * and two companions: dit_modulate_scale_shift (the AdaLN modulate alone,
 * after a norm computed elsewhere) and dit_qk_norm_rope_dest (the QKV
 * epilogue writing a destination-major buffer for Ulysses all-to-all).
 *
 * Sources (web pages on SGLang's diffusion kernels):
 *   [P1] "基于Agent的SGLang扩散模型Kernel优化实践：Qwen-Image、FLUX.2和视频模型"
 *        (tahou.com): section "数学等价不代表结果完全一致" (AdaLN and the bf16
 *        rounding points of the eager chain), "合并QKV投影时的数值问题" (the
 *        four steps of the QKV epilogue), "质量分级机制" (lossless vs validated
 *        non-bit-exact levels), "Wan视频模型的数据搬运优化" (per-token
 *        modulation).
 *   [P3] "#34085 [diffusion] Clean up kernels and shared fast paths"
 *        (prhub.com.cn): section "实现拆解" (rmsnorm_scale,
 *        rmsnorm_tanh_residual, residual_gate_add and their guards) and
 *        "关键源码片段" (the native bf16 RMSNorm chain, the flat-row-stride
 *        rule, the row -> modulation-row mapping, hidden size <= 8192).
 *   [P4] "AI Agent 驱动的 SGLang Kernel 一等公民" (163.com): section 0x3, 3.2
 *        (the DiT fusion operators rmsnorm+tanh(gate)*x+residual,
 *        QK-norm+RoPE, residual+gate*update).
 *
 * ------------------------------------------------------------------------
 * Common conventions
 * ------------------------------------------------------------------------
 * Data.  Every tensor is bfloat16 (16-bit patterns) unless stated otherwise,
 *   in device memory owned by the caller.  Row tensors are "flat rows":
 *   element (r, i) lives at base + r * row_stride + i (strides in elements),
 *   which is how any [..., rows, dim] tensor whose outer dimensions fold into
 *   one uniform row stride is passed.
 * Modulation rows.  scale / shift / gate are [mod_rows, dim] with row stride
 *   mod_rs; row r of the input uses modulation row r / (rows / mod_rows).
 *   mod_rows = batch gives per-batch ([B, 1, D]) modulation, mod_rows = rows
 *   gives per-token ([B, S, D]) modulation.  rows % mod_rows must be 0.
 * Numerics (mode).  DIT_MODE_LOSSLESS: every step is one IEEE-754 binary32
 *   operation rounded to nearest even (correctly rounded division and square
 *   root, no fused multiply-add, subnormals kept); results are rounded to
 *   bf16 (nearest even) exactly where the eager PyTorch chain rounds; row
 *   sums use the order R(D) below.  The output is bit-for-bit deterministic.
 *   DIT_MODE_FAST: hardware reciprocal square root, fused multiply-add inside
 *   the sums and the RoPE products; every bf16 rounding point of the
 *   lossless chain is kept, and tanh(gate) is the same exact table value.
 *   The native-bf16 RMSNorm rounds its rstd to bf16 and takes the hardware
 *   value only where it is not within 4 binary32 steps of a bf16 rounding
 *   midpoint (else the IEEE quotient), so its bf16 rstd -- and with it
 *   dit_rmsnorm_scale and dit_rmsnorm_tanh_residual -- is the same in both
 *   modes.  Elsewhere the hardware rsqrt reads a subnormal argument as zero
 *   (result +inf); LayerNorm and the Q/K norm only reach that with
 *   eps < 2^-126.
 * Reduction order R(D) (D <= 8192, D % 8 == 0), defined on 64 lanes (the
 *   kernels may spread a row over several waves; the order is the same):
 *   lane l owns elements 512c + 8l + j (j = 0..7) of chunk c.  Each lane
 *   adds its own terms to +0 in (c, j) order; then, for m = 1, 2, 4, 8, 16,
 *   32, every lane adds the partial of lane l XOR m.  Q/K head sums use the
 *   same rule with 16 lanes (8 elements each, Dh = 128) and m = 1, 2, 4, 8.
 * Asynchrony and ownership.  Calls enqueue work on `stream` and return; the
 *   library never allocates, frees, copies between host and device, or
 *   synchronizes, and keeps no state between calls (thread-safe, re-entrant).
 * In place.  For the row ops `out` may be exactly one of the row inputs
 *   (same pointer and row stride); each row is fully read before it is
 *   written.  Any other overlap of the output with an input is rejected.
 * Alignment.  Tensor pointers must be 16-byte aligned and row strides
 *   multiples of 8 elements (one 128-bit vector), else DIT_ERR_UNSUPPORTED.
 * Errors.  Arguments are checked on the host before any HIP call; a
 *   rejected call touches neither the GPU nor its arguments.
 *   DIT_ERR_UNSUPPORTED: a legal problem outside this fast path (dim > 8192,
 *     dim % 8 != 0, rows % mod_rows != 0, stride < dim, misalignment,
 *     head_dim != 128); the caller should use another implementation.
 *   DIT_ERR_INVALID: null pointer, negative size, unknown mode, or an
 *     output that partially overlaps an input.
 *   DIT_ERR_HIP: the kernel launch failed (hipGetLastError after launch).
 *   rows == 0 (or zero tokens) is a valid empty problem and returns DIT_OK
 *   without launching anything.
 *   dit_status_reason() returns a short text for the calling thread's most
 *   recent non-OK status.
 */
#ifndef DIT_H
#define DIT_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIT_ABI_VERSION 3
#define DIT_MAX_DIM 8192
#define DIT_QK_HEAD_DIM 128

typedef enum {
  DIT_OK = 0,
  DIT_ERR_UNSUPPORTED = 1,
  DIT_ERR_INVALID = 2,
  DIT_ERR_HIP = 3
} dit_status_t;

typedef enum { DIT_MODE_LOSSLESS = 0, DIT_MODE_FAST = 1 } dit_mode_t;

/* DIT_ABI_VERSION of the built library. */
int dit_abi_version(void);

/* Static name of a status code. */
const char *dit_status_string(dit_status_t s);

/* Reason for the calling thread's most recent non-OK status ("" if none). */
const char *dit_status_reason(void);

/*
 * LayerNorm + AdaLN modulate  [P1 数学等价不代表结果完全一致]
 *   mu  = (sum_R x) / D
 *   d_i = x_i - mu
 *   var = (sum_R d*d) / D                          (biased, two passes)
 *   rho = 1 / sqrt(var + eps)
 *   n_i = bf(d_i * rho)                            LayerNorm output, no affine
 *   out = bf( bf( n * bf(1 + scale[m]) ) + shift[m] )
 * out, x: [rows, dim] with row strides out_rs, x_rs.
 * scale, shift: [mod_rows, dim], shared row stride mod_rs.
 * FAST mode: sum of d*d with fused multiply-add, rho from the hardware rsqrt.
 */
dit_status_t dit_ln_modulate(void *out, int64_t out_rs, const void *x, int64_t x_rs,
                             const void *scale, const void *shift, int64_t mod_rs,
                             int64_t mod_rows, int64_t rows, int64_t dim, float eps, int mode,
                             hipStream_t stream);

/*
 * Native-bf16 RMSNorm + scale  [P3 关键源码片段, rmsnorm_scale]
 *   t_i  = bf(x_i * x_i)
 *   ms   = bf((sum_R t) / D)
 *   v    = bf(ms + eps)
 *   rstd = bf(1 / sqrt(v))                         (same bf16 value in FAST)
 *   y2_i = bf( bf(x_i * rstd) * w_i )
 *   out  = bf(y2 * scale[m])
 * weight: [dim], contiguous.  scale: [mod_rows, dim], row stride mod_rs.
 */
dit_status_t dit_rmsnorm_scale(void *out, int64_t out_rs, const void *x, int64_t x_rs,
                               const void *weight, const void *scale, int64_t mod_rs,
                               int64_t mod_rows, int64_t rows, int64_t dim, float eps, int mode,
                               hipStream_t stream);

/*
 * Native-bf16 RMSNorm + tanh(gate) + residual
 *   [P4 0x3 3.2 rmsnorm+tanh(gate)*x+residual; P3 实现拆解 rmsnorm_tanh_residual]
 *   y2 as in dit_rmsnorm_scale
 *   tau = T(gate[m])  -- the correctly rounded bf16 of tanh of the bf16 gate
 *   out = bf( residual + bf(tau * y2) )
 * residual: [rows, dim], row stride res_rs.  gate: [mod_rows, dim].
 * tau is taken from a 736-entry table of correctly rounded values (built per
 * workgroup in LDS) for 2^-4 <= |gate| < 3.5; tau = gate below that range and
 * +-1 above it, both exact.  Both modes give the same result (the bf16 rstd
 * is the same, above).
 */
dit_status_t dit_rmsnorm_tanh_residual(void *out, int64_t out_rs, const void *x, int64_t x_rs,
                                       const void *residual, int64_t res_rs, const void *weight,
                                       const void *gate, int64_t mod_rs, int64_t mod_rows,
                                       int64_t rows, int64_t dim, float eps, int mode,
                                       hipStream_t stream);

/*
 * Residual gate-add  [P4 0x3 3.2 residual+gate*update; P3 实现拆解 residual_gate_add]
 *   out = bf( residual + bf(gate[m] * y) )
 * Both modes compute the same two roundings (there is nothing to relax).
 */
dit_status_t dit_residual_gate_add(void *out, int64_t out_rs, const void *residual,
                                   int64_t res_rs, const void *y, int64_t y_rs, const void *gate,
                                   int64_t mod_rs, int64_t mod_rows, int64_t rows, int64_t dim,
                                   int mode, hipStream_t stream);

/*
 * Standalone AdaLN modulate  [P3 实现拆解 modulate_scale_shift; P1 数学等价不代表结果完全一致]
 *   out = bf( bf(x * bf(1 + scale[m])) + shift[m] )
 * x, out: [rows, dim] flat rows; scale, shift: [mod_rows, dim], row stride
 * mod_rs; row r uses modulation row m = r / (rows / mod_rows).  The three
 * roundings are those of the eager bf16 chain x * (1 + scale) + shift;
 * both modes compute them identically.  out may be exactly x (in place).
 */
dit_status_t dit_modulate_scale_shift(void *out, int64_t out_rs, const void *x, int64_t x_rs,
                                      const void *scale, const void *shift, int64_t mod_rs,
                                      int64_t mod_rows, int64_t rows, int64_t dim, int mode,
                                      hipStream_t stream);

/*
 * One token stream (text or image) of the merged QKV projection output.
 * q, k, v: [batch, tokens, heads, head_dim] views (head stride head_dim,
 * element stride 1) sharing tok_stride and batch_stride (elements); for a
 * merged [B, S, 3*H*Dh] GEMM output they are its three column blocks with
 * tok_stride = 3*H*Dh and batch_stride = S*3*H*Dh.
 * q_weight, k_weight: [head_dim] RMSNorm weights of this stream.
 */
typedef struct {
  const void *q;
  const void *k;
  const void *v;
  int64_t tok_stride;
  int64_t batch_stride;
  const void *q_weight;
  const void *k_weight;
  int64_t tokens;
} dit_qkv_stream_t;

/*
 * Q/K RMSNorm + interleaved RoPE + joint QKV write  [P1 合并QKV投影时的数值问题]
 * For every batch b, joint token t and head h (head_dim = 128):
 *   Q/K:  rho = 1 / sqrt((sum_R16 x*x) / 128 + eps)       (binary32)
 *         u_i = bf( bf(x_i * rho) * w_i )                 (stream's q/k weight)
 *         for each pair (a, b) = (u_2i, u_2i+1), c = cos[t][i], z = sin[t][i]:
 *           o_2i   = bf(a*c - b*z)
 *           o_2i+1 = bf(a*z + b*c)
 *   V:    copied bit for bit.
 * Joint token order: text tokens [0, txt->tokens), then image tokens.
 * q_out, k_out, v_out: [batch, txt->tokens + img->tokens, heads, 128] with
 *   token stride out_tok_stride and batch stride out_batch_stride (elements,
 *   shared by the three; they may interleave inside one buffer).
 * cos, sin: float32 [txt->tokens + img->tokens, 64], contiguous, indexed by
 *   joint token.  Either stream may have zero tokens (or be NULL).
 * Outputs must not overlap any input or each other (DIT_ERR_INVALID).  The
 *   output strides must nest (the larger one at least spans every row of the
 *   smaller, the smaller at least a token's heads*128 elements), so no output
 *   overlaps itself (DIT_ERR_UNSUPPORTED).
 * FAST mode: fused multiply-add in the head sum and the rotation, rsqrt.
 */
dit_status_t dit_qk_norm_rope(void *q_out, void *k_out, void *v_out, int64_t out_tok_stride,
                              int64_t out_batch_stride, const dit_qkv_stream_t *txt,
                              const dit_qkv_stream_t *img, const float *cos, const float *sin,
                              int64_t batch, int64_t heads, int64_t head_dim, float eps, int mode,
                              hipStream_t stream);

/*
 * The same epilogue written destination-major  [P1 Ulysses QKV仅执行一次All-to-All]
 * The heads are dealt in contiguous groups of heads_per_dest to P = heads /
 * heads_per_dest destinations (ranks of a Ulysses group): head h goes to
 * destination p = h / heads_per_dest, at head position h % heads_per_dest,
 * i.e. element offset
 *   p * dest_stride + b * out_batch_stride + t * out_tok_stride
 *     + (h % heads_per_dest) * 128
 * from q_out (k_out, v_out).  Values are exactly those of dit_qk_norm_rope.
 * The packed buffer [P][B, S, 3, H/P, 128] that one all-to-all can send,
 * chunk p to rank p, is q_out = buf, k_out = buf + (H/P)*128, v_out = buf +
 * 2*(H/P)*128, out_tok_stride = 3*(H/P)*128, out_batch_stride = S *
 * out_tok_stride, dest_stride = B * out_batch_stride.
 * heads_per_dest must divide heads (DIT_ERR_INVALID); dest_stride >= 0, a
 * multiple of 8 when P > 1 (ignored when P = 1).  The three strides must
 * nest as above with (heads_per_dest * 128) as a token's width, so that no
 * output overlaps itself (DIT_ERR_UNSUPPORTED).  Other rules as for
 * dit_qk_norm_rope; heads_per_dest = heads with dest_stride 0 is exactly
 * dit_qk_norm_rope.
 */
dit_status_t dit_qk_norm_rope_dest(void *q_out, void *k_out, void *v_out, int64_t out_tok_stride,
                                   int64_t out_batch_stride, int64_t heads_per_dest,
                                   int64_t dest_stride, const dit_qkv_stream_t *txt,
                                   const dit_qkv_stream_t *img, const float *cos,
                                   const float *sin, int64_t batch, int64_t heads,
                                   int64_t head_dim, float eps, int mode, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DIT_H */

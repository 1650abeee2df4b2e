/*
 * dit_producers.h -- fused producers around the DiT row epilogues: each one
 * merges an epilogue of dit.h with the step that feeds it or that follows
 * it, so an intermediate tensor never makes a round trip through HBM.
 * Conventions (bf16 bit patterns, flat rows, modulation row mapping,
 * numerics modes and order R(D), ownership, asynchrony, status codes and
 * the thread-local reason, alignment) are those of dit.h.
 *
 * Source: [P1] "基于Agent的SGLang扩散模型Kernel优化实践：Qwen-Image、FLUX.2和视频模型"
 * (tahou.com), sections "将FP8量化融合到前序算子" (gated residual +
 * LayerNorm/AdaLN producers) and "NVFP4的三组优化" (the block's deferred
 * residual update merged into the next normalization/modulation).
 */
#ifndef DIT_PRODUCERS_H
#define DIT_PRODUCERS_H

#include "dit.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Gated residual + LayerNorm + AdaLN modulate  [P1 将FP8量化融合到前序算子]
 *   r'  = bf( residual + bf(gate[m] * y) )           -> out_residual
 *   out = bf( bf( bf(LN(r')) * bf(1 + scale[m]) ) + shift[m] )
 * with LN(r') exactly as dit_ln_modulate computes it on the bf16 row r'
 * (two-pass statistics in order R(D); FAST mode as there).  The result is
 * bit-identical to dit_residual_gate_add followed by dit_ln_modulate, with
 * one read of residual and y and no re-read of r'.
 * residual, y, out_residual, out: [rows, dim] flat rows with their own row
 * strides.  gate, scale, shift: [mod_rows, dim], one row stride mod_rs; row
 * r uses modulation row m = r / (rows / mod_rows).
 * In place: each output may be exactly one of residual or y (same pointer
 * and stride); the two outputs must not overlap each other
 * (DIT_ERR_INVALID), nor partially overlap an input or touch a modulation
 * tensor.
 */
dit_status_t dit_gate_add_ln_modulate(void *out_residual, int64_t out_res_rs, void *out,
                                      int64_t out_rs, const void *residual, int64_t res_rs,
                                      const void *y, int64_t y_rs, const void *gate,
                                      const void *scale, const void *shift, int64_t mod_rs,
                                      int64_t mod_rows, int64_t rows, int64_t dim, float eps,
                                      int mode, hipStream_t stream);

/*
 * BF16 + static E4M3 dual output  [P1 将FP8量化融合到前序算子]
 * The producers above also write an OCP E4M3 copy of their BF16 output for
 * an FP8 GEMM that follows:
 *   out_fp8 = E4M3( bf16_value(out) / *fp8_scale )
 * with a correctly rounded binary32 division (in both modes: the pages note
 * that a reciprocal one binary32 ulp off moves codes across E4M3 rounding
 * midpoints), E4M3 round to nearest even, values beyond +-448 saturated to
 * +-448, NaN kept.  The BF16 outputs are exactly those of the BF16-only
 * calls.
 * out_fp8: [rows, dim] bytes, row stride out_fp8_rs bytes (a multiple of 8,
 * >= dim), 8-byte aligned; it may overlap nothing else.
 * fp8_scale: device pointer to one float (static per-tensor scale), read by
 * the kernel, so a graph replay picks up a new value; 4-byte aligned.
 */
dit_status_t dit_ln_modulate_fp8(void *out, int64_t out_rs, void *out_fp8, int64_t out_fp8_rs,
                                 const void *x, int64_t x_rs, const void *scale,
                                 const void *shift, int64_t mod_rs, int64_t mod_rows,
                                 int64_t rows, int64_t dim, float eps, const float *fp8_scale,
                                 int mode, hipStream_t stream);

dit_status_t dit_gate_add_ln_modulate_fp8(
    void *out_residual, int64_t out_res_rs, void *out, int64_t out_rs, void *out_fp8,
    int64_t out_fp8_rs, const void *residual, int64_t res_rs, const void *y, int64_t y_rs,
    const void *gate, const void *scale, const void *shift, int64_t mod_rs, int64_t mod_rows,
    int64_t rows, int64_t dim, float eps, const float *fp8_scale, int mode, hipStream_t stream);

/*
 * Wan per-token modulation table  [P1 Wan视频模型的数据搬运优化]
 *   out[k][b][s][i] = table[k][i] + temb[b][s][k][i]     (one binary32 add)
 * The block's modulation table plus the per-token time embedding, written
 * as n_mod (6 in Wan) contiguous [batch, tokens, dim] tensors: the layout
 * the per-token modulated norms read, with no temporary and no chunked,
 * strided views to make contiguous later.  The addition is the one the
 * unfused expression performs, so the result is bit-identical to it.
 * table: [n_mod, dim] float32; temb: [batch, tokens, n_mod, dim] bf16;
 * out: [n_mod, batch, tokens, dim] float32; all contiguous, 16-byte
 * aligned, dim % 8 == 0 (else DIT_ERR_UNSUPPORTED); out must not overlap an
 * input (DIT_ERR_INVALID).  Empty problems return DIT_OK.  Independent of
 * the numerics mode (a single IEEE addition).
 */
dit_status_t dit_wan_modulation_table(float *out, const float *table, const void *temb,
                                      int64_t batch, int64_t tokens, int64_t n_mod, int64_t dim,
                                      hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DIT_PRODUCERS_H */

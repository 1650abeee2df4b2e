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

#ifdef __cplusplus
}
#endif
#endif /* DIT_PRODUCERS_H */

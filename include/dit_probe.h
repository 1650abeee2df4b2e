/*
 * dit_probe.h -- entry points that run the epilogue kernels' own device
 * primitives over caller arrays.  They exist so that each primitive can be
 * checked exhaustively (all 65536 bf16 inputs, all 2^32 binary32 inputs)
 * against an independent CPU reference; they are not needed to use the
 * epilogues, and only the instrumented build, libdit_probe.so (the same
 * kernel objects as libdit.so plus these and dit_timing.h), exports them.
 * Conventions (ownership, asynchrony, status codes, thread-local reason) are
 * those of dit.h; every array's extent is checked as there (DIT_ERR_INVALID
 * beyond 2^56 bytes or the end of the address space).  n == 0 is a valid
 * empty call.
 */
#ifndef DIT_PROBE_H
#define DIT_PROBE_H

#include "dit.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out[i] = bf16 bits of in[i] rounded to nearest even (the kernels' packer). */
dit_status_t dit_probe_bf16_round(uint16_t *out, const float *in, int64_t n, hipStream_t stream);

typedef enum {
  DIT_PROBE_ONE_PLUS = 0,   /* bf(1 + s)                                    */
  /* 1 is reserved (rejected with DIT_ERR_INVALID)                           */
  DIT_PROBE_RMS_RSTD = 2,   /* bf(1 / sqrt(v)) of the RMSNorm chain (mode)   */
  DIT_PROBE_TANH_TABLE = 3  /* bf16 tanh of a bf16 gate as
                               dit_rmsnorm_tanh_residual takes it: the
                               identity below 2^-4, +-1 from 3.5, else the
                               library's table of correctly rounded values
                               (mode-independent)                           */
} dit_probe_unary_t;

/* out[i] = op(in[i]) on bf16 bit patterns. */
dit_status_t dit_probe_unary(int op, uint16_t *out, const uint16_t *in, int64_t n, int mode,
                             hipStream_t stream);

typedef enum {
  DIT_PROBE_DIV = 0,    /* a / b                         */
  DIT_PROBE_SQRT = 1,   /* sqrt(a)                       */
  DIT_PROBE_RSQRT = 2   /* 1 / sqrt(a) as the norms use it (mode) */
} dit_probe_f32_t;

/* out[i] = op(a[i], b[i]) in binary32; b is ignored (may be NULL) unless op
 * is DIT_PROBE_DIV. */
dit_status_t dit_probe_f32(int op, float *out, const float *a, const float *b, int64_t n,
                           int mode, hipStream_t stream);

/* head == 0: out[r] = R(dim) sum of t[r*dim .. r*dim+dim) (dim <= 8192,
 *            dim % 8 == 0), one wave per row.
 * head == 1: out[g] = 16-lane head sum of t[g*128 .. g*128+128); dim must be
 *            128. */
dit_status_t dit_probe_row_sum(float *out, const float *t, int64_t rows, int64_t dim, int head,
                               hipStream_t stream);

/* Streaming copy of `bytes` (a multiple of 16; 16-byte aligned, non-overlapping
 * buffers) with the epilogues' access pattern: 128-bit accesses, 1 KiB
 * contiguous per wave instruction.  Used as the practical HBM ceiling and to
 * calibrate memory counters.  flags bit 0: nontemporal loads; bit 1:
 * nontemporal stores; bit 2: the flat kernels' layout instead (one 16-byte
 * vector per lane, one-shot 64-thread workgroups; bytes / 1024 < 2^31). */
dit_status_t dit_probe_copy(void *out, const void *in, int64_t bytes, int flags,
                            hipStream_t stream);

typedef enum {
  DIT_PROBE_E4M3 = 0,       /* out[i] = E4M3 code of the binary32 in[i]              */
  DIT_PROBE_FP8_QUANT = 1   /* out[i] = E4M3 code of (bf16 in[i]) / *scale, as the
                               dual-output producers quantize                      */
} dit_probe_fp8_t;

/* The E4M3 conversion of the dual-output producers (dit_producers.h) over an
 * array: saturation to +-448, round to nearest even, NaN kept.  in: float
 * (op 0) or bf16 (op 1) device array of n elements; scale: device pointer to
 * one float (op 1 only; may be NULL for op 0). */
dit_status_t dit_probe_fp8(int op, uint8_t *out, const void *in, int64_t n, const float *scale,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DIT_PROBE_H */

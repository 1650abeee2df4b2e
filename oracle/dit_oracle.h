/*
 * dit_oracle.h -- declarations of the CPU oracle (test infrastructure only).
 *
 * All bf16 tensors are uint16_t bit patterns.  Rows are flat: element (r, i)
 * of a row tensor lives at base + r * row_stride + i.  Row ops return 0, or 1
 * when rows / dim / mod_rows do not describe a valid problem.
 */
#ifndef DIT_ORACLE_H
#define DIT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

uint16_t orc_bf16_round(float v);
float orc_bf16_value(uint16_t h);
uint16_t orc_bf16_round_f64(double v);

float orc_sum_wave(const float *t, int64_t D);
float orc_sum_head(const float *t, int64_t Dh);

uint16_t orc_one_plus(uint16_t scale);
uint16_t orc_tanh(uint16_t g);
uint16_t orc_rms_rstd(uint16_t v);

void orc_ln_row(const uint16_t *x, int64_t D, float eps, uint16_t *n, float *stats);
void orc_rms_row(const uint16_t *x, const uint16_t *w, int64_t D, float eps, uint16_t *y2,
                 float *stats);
void orc_qk_head(const uint16_t *x, const uint16_t *w, const float *c, const float *z,
                 int64_t Dh, float eps, uint16_t *o);

int orc_ln_modulate(uint16_t *out, int64_t out_rs, const uint16_t *x, int64_t x_rs,
                    const uint16_t *scale, const uint16_t *shift, int64_t mod_rs,
                    int64_t mod_rows, int64_t rows, int64_t dim, float eps);
int orc_rmsnorm_scale(uint16_t *out, int64_t out_rs, const uint16_t *x, int64_t x_rs,
                      const uint16_t *w, const uint16_t *scale, int64_t mod_rs, int64_t mod_rows,
                      int64_t rows, int64_t dim, float eps);
int orc_rmsnorm_tanh_residual(uint16_t *out, int64_t out_rs, const uint16_t *x, int64_t x_rs,
                              const uint16_t *residual, int64_t res_rs, const uint16_t *w,
                              const uint16_t *gate, int64_t mod_rs, int64_t mod_rows,
                              int64_t rows, int64_t dim, float eps);
int orc_residual_gate_add(uint16_t *out, int64_t out_rs, const uint16_t *residual,
                          int64_t res_rs, const uint16_t *y, int64_t y_rs, const uint16_t *gate,
                          int64_t mod_rs, int64_t mod_rows, int64_t rows, int64_t dim);
int orc_gate_add_ln_modulate(uint16_t *out_res, int64_t out_res_rs, uint16_t *out,
                             int64_t out_rs, const uint16_t *residual, int64_t res_rs,
                             const uint16_t *y, int64_t y_rs, const uint16_t *gate,
                             const uint16_t *scale, const uint16_t *shift, int64_t mod_rs,
                             int64_t mod_rows, int64_t rows, int64_t dim, float eps);

int orc_modulate_scale_shift(uint16_t *out, int64_t out_rs, const uint16_t *x, int64_t x_rs,
                             const uint16_t *scale, const uint16_t *shift, int64_t mod_rs,
                             int64_t mod_rows, int64_t rows, int64_t dim);
double orc_e4m3_value(uint8_t c);
uint8_t orc_e4m3(float v);
int orc_ln_modulate_fp8(uint16_t *out, int64_t out_rs, uint8_t *out8, int64_t out8_rs,
                        const uint16_t *x, int64_t x_rs, const uint16_t *scale,
                        const uint16_t *shift, int64_t mod_rs, int64_t mod_rows, int64_t rows,
                        int64_t dim, float eps, float fp8_scale);
int orc_gate_add_ln_modulate_fp8(uint16_t *out_res, int64_t out_res_rs, uint16_t *out,
                                 int64_t out_rs, uint8_t *out8, int64_t out8_rs,
                                 const uint16_t *residual, int64_t res_rs, const uint16_t *y,
                                 int64_t y_rs, const uint16_t *gate, const uint16_t *scale,
                                 const uint16_t *shift, int64_t mod_rs, int64_t mod_rows,
                                 int64_t rows, int64_t dim, float eps, float fp8_scale);
int orc_wan_mod_table(float *out, const float *table, const uint16_t *temb, int64_t batch,
                      int64_t tokens, int64_t n_mod, int64_t dim);
void orc_e4m3_array(const float *in, uint8_t *out, int64_t n);
void orc_e4m3_bits_range(uint32_t first, int64_t n, uint8_t *out);

typedef struct {
  const uint16_t *q, *k, *v;      /* [B, S, H, Dh] views, head stride Dh */
  int64_t tok_stride, batch_stride;
  const uint16_t *q_weight, *k_weight;
  int64_t tokens;
} orc_qkv_stream;

int orc_qk_norm_rope(uint16_t *q_out, uint16_t *k_out, uint16_t *v_out, int64_t out_tok_stride,
                     int64_t out_batch_stride, const orc_qkv_stream *txt,
                     const orc_qkv_stream *img, const float *cos_t, const float *sin_t,
                     int64_t batch, int64_t heads, int64_t head_dim, float eps);
int orc_qk_norm_rope_dest(uint16_t *q_out, uint16_t *k_out, uint16_t *v_out,
                          int64_t out_tok_stride, int64_t out_batch_stride, int64_t hpd,
                          int64_t dest_stride, const orc_qkv_stream *txt,
                          const orc_qkv_stream *img, const float *cos_t, const float *sin_t,
                          int64_t batch, int64_t heads, int64_t head_dim, float eps);

void orc_bf16_round_array(const float *in, uint16_t *out, int64_t n);
void orc_bf16_round_bits_range(uint32_t first, int64_t n, uint16_t *out);
void orc_tanh_array(const uint16_t *in, uint16_t *out, int64_t n);
void orc_one_plus_array(const uint16_t *in, uint16_t *out, int64_t n);
void orc_rms_rstd_array(const uint16_t *in, uint16_t *out, int64_t n);
void orc_tanh_check_ld(const uint16_t *in, uint16_t *out, double *tie_margin, int64_t n);

#ifdef __cplusplus
}
#endif
#endif

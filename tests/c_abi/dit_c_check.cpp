// dit_c_check.cpp -- the epilogue library driven through its C ABI alone (no
// Python, no torch): device buffers from hipMalloc, calls on a HIP stream,
// every entry point of dit.h and dit_producers.h, results compared bit for
// bit with the CPU oracle (test infrastructure, linked beside the library;
// the two share no code).  Also checks that the guards' statuses reach a C
// caller.  Exit status 0 when every case passes.
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "dit.h"
#include "dit_oracle.h"
#include "dit_producers.h"

namespace {

int g_cases = 0, g_fail = 0;

// xorshift32 input generator (inputs only; none of the method's arithmetic).
uint32_t g_rng = 0x9E3779B9u;
uint32_t next_u32() {
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 17;
  g_rng ^= g_rng << 5;
  return g_rng;
}

// A bf16 pattern with a random sign and mantissa and a biased exponent in
// [e_lo, e_hi] (127 is 1.0).
uint16_t rnd_bf16(int e_lo, int e_hi) {
  const uint32_t u = next_u32();
  const uint32_t e = (uint32_t)e_lo + (u >> 8) % (uint32_t)(e_hi - e_lo + 1);
  return (uint16_t)(((u & 1u) << 15) | (e << 7) | ((u >> 1) & 0x7Fu));
}

std::vector<uint16_t> rnd_vec(size_t n, int e_lo, int e_hi) {
  std::vector<uint16_t> v(n);
  for (auto &x : v) x = rnd_bf16(e_lo, e_hi);
  return v;
}

#define HIP_CHECK(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(2);                                                              \
    }                                                                       \
  } while (0)

template <class T>
T *to_dev(const std::vector<T> &h) {
  T *d = nullptr;
  HIP_CHECK(hipMalloc(&d, h.size() * sizeof(T) + 16));
  HIP_CHECK(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
  return d;
}

template <class T>
std::vector<T> to_host(const T *d, size_t n) {
  std::vector<T> h(n);
  HIP_CHECK(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
  return h;
}

bool is_nan16(uint16_t h) { return (h & 0x7F80u) == 0x7F80u && (h & 0x7Fu) != 0; }

void expect_equal(const char *what, const std::vector<uint16_t> &got,
                  const std::vector<uint16_t> &ref) {
  ++g_cases;
  size_t bad = 0, first = 0;
  for (size_t i = 0; i < ref.size(); ++i) {
    const bool same = is_nan16(got[i]) ? is_nan16(ref[i]) : got[i] == ref[i];
    if (!same && bad++ == 0) first = i;
  }
  if (bad) {
    ++g_fail;
    printf("FAIL %s: %zu of %zu differ (first at %zu: got 0x%04x, oracle 0x%04x)\n", what, bad,
           ref.size(), first, got[first], ref[first]);
  } else {
    printf("ok   %s (%zu elements)\n", what, ref.size());
  }
}

template <class T>
void expect_same_bits(const char *what, const std::vector<T> &got, const std::vector<T> &ref) {
  ++g_cases;
  size_t bad = 0, first = 0;
  for (size_t i = 0; i < ref.size(); ++i)
    if (got[i] != ref[i] && bad++ == 0) first = i;
  if (bad) {
    ++g_fail;
    printf("FAIL %s: %zu of %zu differ (first at %zu)\n", what, bad, ref.size(), first);
  } else {
    printf("ok   %s (%zu elements)\n", what, ref.size());
  }
}

void expect_status(const char *what, dit_status_t got, dit_status_t want) {
  ++g_cases;
  if (got != want) {
    ++g_fail;
    printf("FAIL %s: status %s, expected %s (%s)\n", what, dit_status_string(got),
           dit_status_string(want), dit_status_reason());
  } else {
    printf("ok   %s: %s%s%s\n", what, dit_status_string(got), got ? " -- " : "",
           got ? dit_status_reason() : "");
  }
}

// Row ops on [rows, dim] with row stride rs (> dim: strided rows), per batch
// (one modulation row) or per token.
void row_ops(hipStream_t s, int64_t rows, int64_t dim, int64_t rs, bool per_token) {
  const int64_t mrows = per_token ? rows : 1;
  const float eps = 1e-6f;
  auto x = rnd_vec(rows * rs, 118, 129), res = rnd_vec(rows * rs, 118, 129);
  auto sc = rnd_vec(mrows * dim, 115, 124), sh = rnd_vec(mrows * dim, 115, 124);
  auto g = rnd_vec(mrows * dim, 120, 128), w = rnd_vec(dim, 125, 127);
  uint16_t *dx = to_dev(x), *dres = to_dev(res), *dsc = to_dev(sc), *dsh = to_dev(sh);
  uint16_t *dg = to_dev(g), *dw = to_dev(w), *dout = nullptr, *dout2 = nullptr;
  HIP_CHECK(hipMalloc(&dout, rows * rs * 2));
  HIP_CHECK(hipMalloc(&dout2, rows * rs * 2));
  std::vector<uint16_t> ref(rows * rs, 0), ref2(rows * rs, 0);
  char tag[96];
  snprintf(tag, sizeof tag, "[%lld x %lld, stride %lld, %s]", (long long)rows, (long long)dim,
           (long long)rs, per_token ? "per token" : "per batch");
  auto compare = [&](const char *op, uint16_t *d, std::vector<uint16_t> &r) {
    auto got = to_host(d, rows * rs);
    std::vector<uint16_t> gv, rv;
    for (int64_t i = 0; i < rows; ++i)
      for (int64_t j = 0; j < dim; ++j) {
        gv.push_back(got[i * rs + j]);
        rv.push_back(r[i * rs + j]);
      }
    char what[160];
    snprintf(what, sizeof what, "%s %s", op, tag);
    expect_equal(what, gv, rv);
  };

  expect_status("dit_ln_modulate call",
                dit_ln_modulate(dout, rs, dx, rs, dsc, dsh, dim, mrows, rows, dim, eps,
                                DIT_MODE_LOSSLESS, s), DIT_OK);
  HIP_CHECK(hipStreamSynchronize(s));
  orc_ln_modulate(ref.data(), rs, x.data(), rs, sc.data(), sh.data(), dim, mrows, rows, dim, eps);
  compare("ln_modulate", dout, ref);

  expect_status("dit_rmsnorm_tanh_residual call",
                dit_rmsnorm_tanh_residual(dout, rs, dx, rs, dres, rs, dw, dg, dim, mrows, rows,
                                          dim, eps, DIT_MODE_LOSSLESS, s), DIT_OK);
  HIP_CHECK(hipStreamSynchronize(s));
  orc_rmsnorm_tanh_residual(ref.data(), rs, x.data(), rs, res.data(), rs, w.data(), g.data(),
                            dim, mrows, rows, dim, eps);
  compare("rmsnorm_tanh_residual", dout, ref);

  expect_status("dit_rmsnorm_scale call",
                dit_rmsnorm_scale(dout, rs, dx, rs, dw, dsc, dim, mrows, rows, dim, eps,
                                  DIT_MODE_LOSSLESS, s), DIT_OK);
  HIP_CHECK(hipStreamSynchronize(s));
  orc_rmsnorm_scale(ref.data(), rs, x.data(), rs, w.data(), sc.data(), dim, mrows, rows, dim,
                    eps);
  compare("rmsnorm_scale", dout, ref);

  expect_status("dit_residual_gate_add call",
                dit_residual_gate_add(dout, rs, dres, rs, dx, rs, dg, dim, mrows, rows, dim,
                                      DIT_MODE_LOSSLESS, s), DIT_OK);
  HIP_CHECK(hipStreamSynchronize(s));
  orc_residual_gate_add(ref.data(), rs, res.data(), rs, x.data(), rs, g.data(), dim, mrows,
                        rows, dim);
  compare("residual_gate_add", dout, ref);

  expect_status("dit_gate_add_ln_modulate call",
                dit_gate_add_ln_modulate(dout2, rs, dout, rs, dres, rs, dx, rs, dg, dsc, dsh,
                                         dim, mrows, rows, dim, eps, DIT_MODE_LOSSLESS, s),
                DIT_OK);
  HIP_CHECK(hipStreamSynchronize(s));
  orc_gate_add_ln_modulate(ref2.data(), rs, ref.data(), rs, res.data(), rs, x.data(), rs,
                           g.data(), sc.data(), sh.data(), dim, mrows, rows, dim, eps);
  compare("gate_add_ln_modulate r'", dout2, ref2);
  compare("gate_add_ln_modulate out", dout, ref);

  expect_status("dit_modulate_scale_shift call",
                dit_modulate_scale_shift(dout, rs, dx, rs, dsc, dsh, dim, mrows, rows, dim,
                                         DIT_MODE_LOSSLESS, s), DIT_OK);
  HIP_CHECK(hipStreamSynchronize(s));
  orc_modulate_scale_shift(ref.data(), rs, x.data(), rs, sc.data(), sh.data(), dim, mrows, rows,
                           dim);
  compare("modulate_scale_shift", dout, ref);

  // E4M3 copies: byte rows, row stride rounded up to a multiple of 8
  const int64_t rs8 = (dim + 15) / 8 * 8;
  const float fs = 0.05f;
  float *dfs = to_dev(std::vector<float>{fs});
  uint8_t *d8 = nullptr;
  HIP_CHECK(hipMalloc(&d8, rows * rs8));
  std::vector<uint8_t> ref8(rows * rs8, 0);
  auto compare8 = [&](const char *op) {
    auto got = to_host(d8, rows * rs8);
    std::vector<uint8_t> gv, rv;
    for (int64_t i = 0; i < rows; ++i)
      for (int64_t j = 0; j < dim; ++j) {
        gv.push_back(got[i * rs8 + j]);
        rv.push_back(ref8[i * rs8 + j]);
      }
    char what[160];
    snprintf(what, sizeof what, "%s E4M3 %s", op, tag);
    expect_same_bits(what, gv, rv);
  };
  expect_status("dit_ln_modulate_fp8 call",
                dit_ln_modulate_fp8(dout, rs, d8, rs8, dx, rs, dsc, dsh, dim, mrows, rows, dim,
                                    eps, dfs, DIT_MODE_LOSSLESS, s), DIT_OK);
  HIP_CHECK(hipStreamSynchronize(s));
  orc_ln_modulate_fp8(ref.data(), rs, ref8.data(), rs8, x.data(), rs, sc.data(), sh.data(), dim,
                      mrows, rows, dim, eps, fs);
  compare("ln_modulate_fp8", dout, ref);
  compare8("ln_modulate_fp8");
  expect_status("dit_gate_add_ln_modulate_fp8 call",
                dit_gate_add_ln_modulate_fp8(dout2, rs, dout, rs, d8, rs8, dres, rs, dx, rs, dg,
                                             dsc, dsh, dim, mrows, rows, dim, eps, dfs,
                                             DIT_MODE_LOSSLESS, s), DIT_OK);
  HIP_CHECK(hipStreamSynchronize(s));
  orc_gate_add_ln_modulate_fp8(ref2.data(), rs, ref.data(), rs, ref8.data(), rs8, res.data(), rs,
                               x.data(), rs, g.data(), sc.data(), sh.data(), dim, mrows, rows,
                               dim, eps, fs);
  compare("gate_add_ln_modulate_fp8 r'", dout2, ref2);
  compare("gate_add_ln_modulate_fp8 out", dout, ref);
  compare8("gate_add_ln_modulate_fp8");
  HIP_CHECK(hipFree(d8));
  HIP_CHECK(hipFree(dfs));

  for (uint16_t *p : {dx, dres, dsc, dsh, dg, dw, dout, dout2}) HIP_CHECK(hipFree(p));
}

// The Wan modulation table on [1, 37 tokens, 6, 1040].
void mod_table(hipStream_t s) {
  const int64_t B = 1, T = 37, K = 6, D = 1040;
  std::vector<float> table(K * D);
  for (auto &v : table) v = (float)((int)(next_u32() % 2001) - 1000) / 4096.0f;
  auto temb = rnd_vec(B * T * K * D, 118, 129);
  float *dt = to_dev(table);
  uint16_t *de = to_dev(temb);
  float *dout = nullptr;
  HIP_CHECK(hipMalloc(&dout, K * B * T * D * sizeof(float)));
  expect_status("dit_wan_modulation_table call",
                dit_wan_modulation_table(dout, dt, de, B, T, K, D, s), DIT_OK);
  HIP_CHECK(hipStreamSynchronize(s));
  std::vector<float> ref(K * B * T * D);
  orc_wan_mod_table(ref.data(), table.data(), temb.data(), B, T, K, D);
  auto got = to_host(dout, ref.size());
  std::vector<uint32_t> gb(ref.size()), rb(ref.size());
  memcpy(gb.data(), got.data(), gb.size() * 4);
  memcpy(rb.data(), ref.data(), rb.size() * 4);
  expect_same_bits("wan_modulation_table [6, 1, 37, 1040]", gb, rb);
  HIP_CHECK(hipFree(dt));
  HIP_CHECK(hipFree(de));
  HIP_CHECK(hipFree(dout));
}

void qkv(hipStream_t s) {
  const int64_t B = 2, H = 3, Dh = 128, st = 3, si = 5, S = st + si, W = 3 * H * Dh;
  auto txt = rnd_vec(B * st * W, 118, 129), img = rnd_vec(B * si * W, 118, 129);
  auto w = rnd_vec(4 * Dh, 125, 127);
  std::vector<float> cs(S * Dh / 2), sn(S * Dh / 2);
  for (size_t i = 0; i < cs.size(); ++i) {       // any binary32 table values
    cs[i] = (float)((int)(next_u32() % 2001) - 1000) / 1000.0f;
    sn[i] = (float)((int)(next_u32() % 2001) - 1000) / 1000.0f;
  }
  uint16_t *dt = to_dev(txt), *di = to_dev(img), *dw = to_dev(w);
  float *dc = to_dev(cs), *dz = to_dev(sn);
  const int64_t n = B * S * H * Dh;
  uint16_t *q = nullptr, *k = nullptr, *v = nullptr;
  HIP_CHECK(hipMalloc(&q, n * 2));
  HIP_CHECK(hipMalloc(&k, n * 2));
  HIP_CHECK(hipMalloc(&v, n * 2));
  dit_qkv_stream_t ts_{dt, dt + H * Dh, dt + 2 * H * Dh, W, st * W, dw, dw + Dh, st};
  dit_qkv_stream_t is_{di, di + H * Dh, di + 2 * H * Dh, W, si * W, dw + 2 * Dh, dw + 3 * Dh, si};
  expect_status("dit_qk_norm_rope call",
                dit_qk_norm_rope(q, k, v, H * Dh, S * H * Dh, &ts_, &is_, dc, dz, B, H, Dh, 1e-6f,
                                 DIT_MODE_LOSSLESS, s), DIT_OK);
  HIP_CHECK(hipStreamSynchronize(s));
  std::vector<uint16_t> rq(n), rk(n), rv(n);
  orc_qkv_stream ot{txt.data(), txt.data() + H * Dh, txt.data() + 2 * H * Dh, W, st * W,
                    w.data(), w.data() + Dh, st};
  orc_qkv_stream oi{img.data(), img.data() + H * Dh, img.data() + 2 * H * Dh, W, si * W,
                    w.data() + 2 * Dh, w.data() + 3 * Dh, si};
  orc_qk_norm_rope(rq.data(), rk.data(), rv.data(), H * Dh, S * H * Dh, &ot, &oi, cs.data(),
                   sn.data(), B, H, Dh, 1e-6f);
  expect_equal("qk_norm_rope q [2, 3+5, 3, 128]", to_host(q, n), rq);
  expect_equal("qk_norm_rope k [2, 3+5, 3, 128]", to_host(k, n), rk);
  expect_equal("qk_norm_rope v [2, 3+5, 3, 128]", to_host(v, n), rv);

  // destination-major: P = 3 destinations of one head each, packed
  // [P][B, S, 3, 1, 128]
  const int64_t hpd = 1, ts = 3 * hpd * Dh, bs = S * ts, ds = B * bs, np = (H / hpd) * ds;
  uint16_t *buf = nullptr;
  HIP_CHECK(hipMalloc(&buf, np * 2));
  expect_status("dit_qk_norm_rope_dest call",
                dit_qk_norm_rope_dest(buf, buf + hpd * Dh, buf + 2 * hpd * Dh, ts, bs, hpd, ds,
                                      &ts_, &is_, dc, dz, B, H, Dh, 1e-6f, DIT_MODE_LOSSLESS, s),
                DIT_OK);
  HIP_CHECK(hipStreamSynchronize(s));
  std::vector<uint16_t> rp(np, 0);
  orc_qk_norm_rope_dest(rp.data(), rp.data() + hpd * Dh, rp.data() + 2 * hpd * Dh, ts, bs, hpd,
                        ds, &ot, &oi, cs.data(), sn.data(), B, H, Dh, 1e-6f);
  expect_equal("qk_norm_rope_dest packed [3][2, 8, 3, 1, 128]", to_host(buf, np), rp);
  HIP_CHECK(hipFree(buf));
  for (void *p : {(void *)dt, (void *)di, (void *)dw, (void *)dc, (void *)dz, (void *)q,
                  (void *)k, (void *)v})
    HIP_CHECK(hipFree(p));
}

void statuses(hipStream_t s) {
  uint16_t *a = nullptr, *b = nullptr, *c = nullptr;
  HIP_CHECK(hipMalloc(&a, 1 << 20));
  HIP_CHECK(hipMalloc(&b, 1 << 20));
  HIP_CHECK(hipMalloc(&c, 1 << 20));
  expect_status("dim 8200 (above 8192)",
                dit_ln_modulate(a, 8200, b, 8200, c, c, 8200, 1, 4, 8200, 1e-6f, 0, s),
                DIT_ERR_UNSUPPORTED);
  expect_status("NULL x", dit_ln_modulate(a, 512, nullptr, 512, c, c, 512, 1, 4, 512, 1e-6f, 0, s),
                DIT_ERR_INVALID);
  expect_status("rows 2^32 at stride 2^40",
                dit_ln_modulate(a, int64_t(1) << 40, b, int64_t(1) << 40, c, c, 512, 1,
                                int64_t(1) << 32, 512, 1e-6f, 0, s), DIT_ERR_INVALID);
  expect_status("empty problem", dit_ln_modulate(nullptr, 0, nullptr, 0, nullptr, nullptr, 0, 0,
                                                 0, 512, 1e-6f, 0, s), DIT_OK);
  expect_status("unknown mode", dit_ln_modulate(a, 512, b, 512, c, c, 512, 1, 4, 512, 1e-6f, 7, s),
                DIT_ERR_INVALID);
  HIP_CHECK(hipFree(a));
  HIP_CHECK(hipFree(b));
  HIP_CHECK(hipFree(c));
}

}  // namespace

int main() {
  printf("libdit ABI version %d\n", dit_abi_version());
  hipStream_t s;
  HIP_CHECK(hipStreamCreate(&s));
  row_ops(s, 37, 1032, 1040, false);
  row_ops(s, 37, 1032, 1032, true);
  row_ops(s, 9, 8192, 8192, true);
  row_ops(s, 64, 3072, 3072, false);
  qkv(s);
  mod_table(s);
  statuses(s);
  HIP_CHECK(hipStreamDestroy(s));
  printf("c-abi check: %d cases, %d failed\n", g_cases, g_fail);
  return g_fail ? 1 : 0;
}

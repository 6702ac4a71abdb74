/* Exercises every oracle entry point on small ragged inputs, for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts).
 * Exit status 0 and the line "sanitize: ok" mean no report was raised.  The
 * oracle is test infrastructure; so is this driver. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "coat_oracle.h"

static uint64_t rng_state = 0x243F6A8885A308D3ull;

static double urand(void) {  /* splitmix64 -> [0, 1) */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * 0x1p-53;
}

static float gauss_like(double scale) {  /* sum of uniforms, signed, scaled */
  double s = 0.0;
  for (int i = 0; i < 4; ++i) s += urand() - 0.5;
  return (float)(s * scale);
}

static uint16_t to_bf16(float f) {  /* truncation is enough for a driver */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

#define CHECK(call)                                              \
  do {                                                           \
    int rc_ = (call);                                            \
    if (rc_ != COAT_ORACLE_OK) {                                 \
      fprintf(stderr, "%s failed: %d\n", #call, rc_);            \
      return 1;                                                  \
    }                                                            \
  } while (0)

static int run_size(int64_t n, int32_t G) {
  const int64_t ng = (n + G - 1) / G;
  float* w = malloc(sizeof(float) * (size_t)n);
  uint16_t* g = malloc(sizeof(uint16_t) * (size_t)n);
  uint8_t* mc = calloc((size_t)n, 1);
  uint8_t* vc = calloc((size_t)n, 1);
  float* ms = calloc((size_t)ng, sizeof(float));
  float* mk = calloc((size_t)ng, sizeof(float));
  float* vs = calloc((size_t)ng, sizeof(float));
  float* vk = calloc((size_t)ng, sizeof(float));
  float* mo = malloc(sizeof(float) * (size_t)n);
  float* vo = malloc(sizeof(float) * (size_t)n);
  double* qm = malloc(sizeof(double) * (size_t)n);
  double* qv = malloc(sizeof(double) * (size_t)n);
  float* x = malloc(sizeof(float) * (size_t)n);
  if (!w || !g || !mc || !vc || !ms || !mk || !vs || !vk || !mo || !vo || !qm || !qv || !x) return 1;
  for (int64_t i = 0; i < n; ++i) w[i] = gauss_like(0.05);
  for (int t = 1; t <= 4; ++t) {
    for (int64_t i = 0; i < n; ++i) g[i] = (i % 17 == 3) ? 0 : to_bf16(gauss_like(1e-3));
    CHECK(coat_oracle_adamw_fp8_step(w, g, mc, ms, mk, vc, vs, vk, n, G, 1, 1e-3f, 0.9f,
                                     0.95f, 1e-8f, 0.1f, t, mo, vo, qm, qv));
  }
  CHECK(coat_oracle_dequantize_expand(mc, ms, mk, n, G, x));
  CHECK(coat_oracle_expand_quantize(x, n, G, 1, mc, ms, mk, qm));
  CHECK(coat_oracle_expand_quantize(x, n, G, 0, mc, ms, mk, NULL));
  CHECK(coat_oracle_adamw_step_fp32(w, g, mo, vo, n, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 5));
  free(w); free(g); free(mc); free(vc); free(ms); free(mk); free(vs); free(vk);
  free(mo); free(vo); free(qm); free(qv); free(x);
  return 0;
}

static int run_act(int64_t rows, int64_t cols, int32_t G) {
  uint16_t* x = malloc(sizeof(uint16_t) * (size_t)(rows * cols + 1));
  uint8_t* c = malloc((size_t)(rows * cols + 1));
  uint8_t* ct = malloc((size_t)(rows * cols + 1));
  float* s = malloc(sizeof(float) * (size_t)(rows * (cols / G) + 1));
  if (!x || !c || !ct || !s) return 1;
  for (int64_t i = 0; i < rows * cols; ++i) {
    float v = gauss_like(1.0);
    if (i % 29 == 0) v *= 1e-38f;  /* subnormal-range groups */
    x[i] = to_bf16(v);
  }
  CHECK(coat_oracle_quantize_act(x, rows, cols, G, c, s, ct));
  CHECK(coat_oracle_quantize_act(x, rows, cols, G, c, s, NULL));
  free(x); free(c); free(ct); free(s);
  return 0;
}

static int run_gemm(int64_t M, int64_t N, int64_t K, int32_t G) {
  uint8_t* a = malloc((size_t)(M * K + 1));
  uint8_t* b = malloc((size_t)(N * K + 1));
  uint8_t* c = malloc((size_t)(M * N + 1));
  float* s = malloc(sizeof(float) * (size_t)(M * (N / G) + 1));
  double* c64 = malloc(sizeof(double) * (size_t)(M * N + 1));
  float* c32 = malloc(sizeof(float) * (size_t)(M * N + 1));
  if (!a || !b || !c || !s || !c64 || !c32) return 1;
  for (int64_t i = 0; i < M * K; ++i) a[i] = (uint8_t)(urand() * 126.0) | (urand() < 0.5 ? 0x80 : 0);
  for (int64_t i = 0; i < N * K; ++i) b[i] = (uint8_t)(urand() * 126.0) | (urand() < 0.5 ? 0x80 : 0);
  CHECK(coat_oracle_gemm_fp8_group_quant(a, b, 0.5f, 3.0f, M, N, K, G, c, s, c64, c32));
  CHECK(coat_oracle_gemm_fp8_group_quant(a, b, 0.5f, 3.0f, M, N, K, G, c, s, NULL, NULL));
  free(a); free(b); free(c); free(s); free(c64); free(c32);
  return 0;
}

int main(void) {
  static const int64_t sizes[] = {1, 17, 127, 128, 129, 1000, 4096 + 5};
  static const int32_t groups[] = {16, 32, 64, 128};
  for (size_t gi = 0; gi < sizeof groups / sizeof groups[0]; ++gi) {
    for (size_t si = 0; si < sizeof sizes / sizeof sizes[0]; ++si)
      if (run_size(sizes[si], groups[gi])) return 1;
    if (run_act(3, 2 * groups[gi], groups[gi]) || run_act(37, groups[gi], groups[gi])) return 1;
    if (run_gemm(5, 2 * groups[gi], 17, groups[gi]) || run_gemm(1, groups[gi], 1, groups[gi])) return 1;
  }
  double xs[300];
  uint8_t cs[300];
  for (int i = 0; i < 300; ++i) xs[i] = (urand() - 0.5) * 1000.0;
  coat_oracle_e4m3_encode_array(xs, 300, cs);
  coat_oracle_e4m3_decode_array(cs, 300, xs);
  /* rejected arguments must not touch memory */
  if (coat_oracle_quantize_act(NULL, 2, 30, 16, NULL, NULL, NULL) != COAT_ORACLE_EINVAL) return 1;
  if (coat_oracle_expand_quantize(NULL, 10, 0, 1, NULL, NULL, NULL, NULL) != COAT_ORACLE_EINVAL)
    return 1;
  puts("sanitize: ok");
  return 0;
}

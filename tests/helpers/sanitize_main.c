/* Driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of the CPU
 * oracle and the brute-force encoder check (test infrastructure): one
 * translation unit with both sources, exercising tables, thresholds, encode,
 * quantize and dequantize at ragged sizes, the linear forward / input gradient
 * / LoRA gradients with and without an adapter, and a strided brute-force pass
 * of the threshold encoder. Exit status 0 when every check holds; the
 * sanitizers abort on the first memory or undefined-behaviour error. */
#include <stdio.h>

#include "../../oracle/nf4_oracle.c"
#include "encoder_bruteforce.c"

static uint32_t rng_state = 12345u;
static float frand(void) { /* xorshift32, uniform in [-1, 1) */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 17;
  rng_state ^= rng_state << 5;
  return (float)((double)rng_state / 2147483648.0 - 1.0);
}

static int check_quant(int64_t n, int dq) {
  int64_t lay[8];
  orc_layout(n, dq, lay);
  const int64_t nb = (n + 63) / 64, nn = (nb + 255) / 256;
  float* w = malloc(sizeof(float) * (size_t)n);
  uint8_t* codes = malloc((size_t)((n + 1) / 2));
  float* absmax = malloc(sizeof(float) * (size_t)nb);
  uint8_t* qabs = malloc((size_t)nb);
  float* nested = malloc(sizeof(float) * (size_t)nn);
  float offset = 0.0f;
  float* out = malloc(sizeof(float) * (size_t)n);
  uint16_t* outh = malloc(sizeof(uint16_t) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) w[i] = 0.02f * frand() * ((i % 97) == 0 ? 10.0f : 1.0f);
  if (n > 70) for (int64_t i = 64; i < 128 && i < n; ++i) w[i] = 0.0f; /* one all-zero block */
  int bad = 0;
  if (orc_quantize(w, n, dq, codes, absmax, dq ? qabs : NULL, dq ? nested : NULL, dq ? &offset : NULL) != 0) bad = 1;
  orc_dequantize(codes, n, dq, dq ? NULL : absmax, dq ? qabs : NULL, dq ? nested : NULL, offset, out, outh);
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(out[i]) || fabsf(out[i]) > 0.25f) bad = 1;
  if ((n & 1) && (codes[n / 2] & 0x0F) != 0) bad = 1; /* odd tail: zero low nibble */
  free(w); free(codes); free(absmax); free(qabs); free(nested); free(out); free(outh);
  return bad;
}

static int check_linear(int64_t M, int64_t K, int64_t N, int r) {
  float* x = malloc(sizeof(float) * (size_t)(M * K));
  float* dy = malloc(sizeof(float) * (size_t)(M * N));
  float* W = malloc(sizeof(float) * (size_t)(N * K));
  float* A = malloc(sizeof(float) * (size_t)(r > 0 ? r * K : 1));
  float* B = malloc(sizeof(float) * (size_t)(r > 0 ? N * r : 1));
  double* y = malloc(sizeof(double) * (size_t)(M * N));
  double* dx = malloc(sizeof(double) * (size_t)(M * K));
  double* T = malloc(sizeof(double) * (size_t)(r > 0 ? M * r : 1));
  double* U = malloc(sizeof(double) * (size_t)(r > 0 ? M * r : 1));
  double* dA = malloc(sizeof(double) * (size_t)(r > 0 ? r * K : 1));
  double* dB = malloc(sizeof(double) * (size_t)(r > 0 ? N * r : 1));
  for (int64_t i = 0; i < M * K; ++i) x[i] = frand();
  for (int64_t i = 0; i < M * N; ++i) dy[i] = frand();
  for (int64_t i = 0; i < N * K; ++i) W[i] = 0.02f * frand();
  for (int64_t i = 0; i < (r > 0 ? r * K : 1); ++i) A[i] = 0.1f * frand();
  for (int64_t i = 0; i < (r > 0 ? N * r : 1); ++i) B[i] = 0.01f * frand();
  orc_linear_fwd(x, M, K, W, N, r > 0 ? A : NULL, r > 0 ? B : NULL, r, 2.0f, y, r > 0 ? T : NULL);
  orc_linear_bwd_input(dy, M, N, W, K, r > 0 ? A : NULL, r > 0 ? B : NULL, r, 2.0f, dx, r > 0 ? U : NULL);
  if (r > 0) {
    orc_lora_grad(x, dy, M, K, N, T, U, r, 2.0f, dA, dB);
    orc_lora_grad(x, dy, M, K, N, T, NULL, r, 2.0f, NULL, dB); /* LoRA-FA */
  }
  int bad = 0;
  for (int64_t i = 0; i < M * N; ++i) if (!isfinite(y[i])) bad = 1;
  for (int64_t i = 0; i < M * K; ++i) if (!isfinite(dx[i])) bad = 1;
  free(x); free(dy); free(W); free(A); free(B); free(y); free(dx); free(T); free(U); free(dA); free(dB);
  return bad;
}

int main(void) {
  int bad = 0;
  double t64[256];
  float c4[16], d8[256], th4[15], th8[255];
  orc_nf4_table(t64, c4);
  orc_dyn8_table(t64, d8);
  orc_thresholds(c4, 16, th4);
  orc_thresholds(d8, 256, th8);
  const int64_t sizes[] = {1, 2, 3, 63, 64, 65, 127, 257, 16383, 16384, 16385, 70001};
  for (size_t i = 0; i < sizeof(sizes) / sizeof(sizes[0]); ++i)
    for (int dq = 0; dq < 2; ++dq) bad |= check_quant(sizes[i], dq) << 1;
  bad |= check_linear(5, 7, 3, 0) << 2;
  bad |= check_linear(9, 70, 33, 3) << 2;
  int64_t visited = 0;
  uint32_t first_bad = 0;
  if (brute_check(orc_encode_array, th4, c4, 16, 0, 4099, 4, &visited, &first_bad) != 0) bad |= 8;
  if (brute_check(orc_encode_array, th8, d8, 256, 1, 65537, 2, &visited, &first_bad) != 0) bad |= 16;
  printf("sanitized oracle checks: %s (flags %d)\n", bad ? "FAILED" : "ok", bad);
  return bad;
}

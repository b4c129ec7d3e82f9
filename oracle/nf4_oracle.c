/*
 * CPU oracle for NF4 double-quantized weight storage and the NF4 + LoRA linear
 * layer (forward, input gradient, LoRA factor gradients).
 *
 * TEST INFRASTRUCTURE ONLY. This library is loaded by the test suite, by the
 * package's smoke check and by the benchmark's CPU-baseline leg, and by nothing
 * else. The GPU product path never calls it and shares no code with it.
 *
 * It is written to be read against the pages, not to be fast:
 *  - Aner docs, "Native model adaptation and NF4", section "Packed NF4 and the
 *    portable QLoRA profile": every matrix uses the 16-value NF4 codebook and
 *    64-element absolute-maximum blocks, two indices per byte; with double
 *    quantization the block maxima are centred by their global FP32 mean and
 *    coded with the signed dynamic8 codebook in 256-element blocks.
 *  - Soup, "NF4 Layer Streaming - Gate results", section "P3 is solved": the
 *    stored bytes per weight are N/2 + N/64 + N/4096 + 4 and both code tables
 *    (16 and 256 fp32 entries) are the same for every weight.
 *  - Aner native training accelerated qualification (31 Oct 2026), key
 *    jit.kernel_identity: "fmad-off" and "decode-separate-rn", i.e. decoding is
 *    a sequence of separately rounded fp32 operations with no fused multiply-add.
 *  - Aner docs, sections "Adapter API" and "LoRA FA includes gradient
 *    preconditioning" (LoRA scale s = alpha / rank), and "Mixed precision keeps
 *    stable state in FP32" (decoded weights are rounded to the half type before
 *    the multiply; adapter contractions stay FP32).
 *
 * Where the pages leave a step open, the plainest reading is taken (each one is
 * marked READING below). Every dot product is accumulated in fp64 in the index
 * order of its definition.
 *
 * Parity status of the code tables: the construction is pinned to independent
 * library routines and to exact rational arithmetic by the tests; bit equality
 * with any third-party NF4 table is not claimed (parity unpinned on that point).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BLOCK 64    /* elements per absmax block */
#define ORC_NESTED 256  /* absmax values per nested (dynamic8) block */

int orc_abi_version(void) { return 1; }

void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Code tables                                                                */
/* ------------------------------------------------------------------------ */

/* Standard normal CDF from the C library's complementary error function. */
static double normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Inverse standard normal CDF by bisection on normal_cdf until the bracket is
 * two adjacent doubles; returns the endpoint whose CDF is closer to p. */
double orc_norm_ppf(double p) {
  double lo = -40.0, hi = 40.0;
  for (;;) {
    double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (normal_cdf(mid) < p)
      lo = mid;
    else
      hi = mid;
  }
  return (fabs(normal_cdf(lo) - p) <= fabs(normal_cdf(hi) - p)) ? lo : hi;
}

static int cmp_double(const void* a, const void* b) {
  double x = *(const double*)a, y = *(const double*)b;
  return (x > y) - (x < y);
}

/* NF4 codebook (QLoRA's normal-float construction, the codebook the pages
 * name). READING: offset delta = ((1 - 1/30) + (1 - 1/32)) / 2 taken as the
 * exact fraction; 8 positive quantiles at p = delta + (0.5 - delta) k / 8,
 * k = 0..7, and 7 negative ones at p = delta + (0.5 - delta) k / 7, k = 0..6;
 * add 0; divide by the largest (Phi^-1(delta)); sort; everything in fp64 and
 * rounded once to fp32. Result: 7 negative codes, 0 at index 7, 8 positive,
 * endpoints exactly -1 and +1. */
void orc_nf4_table(double out64[16], float out32[16]) {
  const double delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
  double v[16];
  int n = 0;
  double top = orc_norm_ppf(delta);
  for (int k = 0; k < 8; ++k) v[n++] = orc_norm_ppf(delta + (0.5 - delta) * k / 8.0) / top;
  v[n++] = 0.0;
  for (int k = 0; k < 7; ++k) v[n++] = -orc_norm_ppf(delta + (0.5 - delta) * k / 7.0) / top;
  qsort(v, 16, sizeof(double), cmp_double);
  for (int i = 0; i < 16; ++i) {
    if (out64) out64[i] = v[i];
    if (out32) out32[i] = (float)v[i];
  }
}

/* Signed dynamic8 codebook (the "bitsandbytes dynamic8" nested codebook the
 * pages name): for each decade E = 0..6 the 2^(6-E) bucket midpoints of the
 * linear fraction range [0.1, 1] scaled by 10^-E, with both signs, plus 0 and
 * +1 (READING: the 256th entry is +1, making the table asymmetric). Each value
 * is the exact rational (2^(n+1) + 18k + 9) / (20 * 2^n * 10^E), n = 6 - E,
 * computed in fp64 and rounded once to fp32. Index 127 holds 0. */
void orc_dyn8_table(double out64[256], float out32[256]) {
  double v[256];
  int n = 0;
  for (int E = 0; E <= 6; ++E) {
    int nb = 6 - E;
    double den = 20.0 * (double)(1 << nb);
    for (int e = 0; e < E; ++e) den *= 10.0;
    for (int k = 0; k < (1 << nb); ++k) {
      double num = (double)((2 << nb) + 18 * k + 9);
      double val = num / den;
      v[n++] = val;
      v[n++] = -val;
    }
  }
  v[n++] = 0.0;
  v[n++] = 1.0;
  qsort(v, 256, sizeof(double), cmp_double);
  for (int i = 0; i < 256; ++i) {
    if (out64) out64[i] = v[i];
    if (out32) out32[i] = (float)v[i];
  }
}

/* Decision thresholds between adjacent codes: T[k] is the exact midpoint of
 * table[k] and table[k+1] (computed in fp64, where it is exact) rounded toward
 * -infinity to fp32. For an fp32 input x, "x > T[k]" holds exactly when x lies
 * strictly above the exact midpoint, so counting the thresholds below x gives
 * the nearest code with ties going to the lower index (READING: ties -> lower). */
void orc_thresholds(const float* table, int count, float* thr) {
  for (int k = 0; k + 1 < count; ++k) {
    double mid = 0.5 * ((double)table[k] + (double)table[k + 1]);
    float f = (float)mid;                  /* round to nearest */
    if ((double)f > mid) f = nextafterf(f, -INFINITY); /* then step down if above */
    thr[k] = f;
  }
}

/* code(x) = number of thresholds strictly below x. */
static uint8_t encode_one(const float* thr, int nthr, float x) {
  int c = 0;
  for (int k = 0; k < nthr; ++k) c += (x > thr[k]) ? 1 : 0;
  return (uint8_t)c;
}

void orc_encode_array(const float* thr, int nthr, const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = encode_one(thr, nthr, x[i]);
}

/* ------------------------------------------------------------------------ */
/* Layout                                                                     */
/* ------------------------------------------------------------------------ */

/* Byte counts of one packed matrix of n elements (blocks run over the
 * flattened row-major matrix; the last block and nested block may be partial):
 * out[0] codes = ceil(n/2); out[1] scales = 4*nb (single) or nb (double);
 * out[2] nested = 4*ceil(nb/256) (double) or 0; out[3] offset = 4 (double) or 0;
 * out[4] = out[0]+out[1]+out[2] (device copy, which the pages store without the
 * offset); out[5] = out[4]+out[3]; out[6] = nb; out[7] = ceil(nb/256). */
void orc_layout(int64_t n, int double_quant, int64_t out[8]) {
  int64_t nb = (n + ORC_BLOCK - 1) / ORC_BLOCK;
  int64_t nn = (nb + ORC_NESTED - 1) / ORC_NESTED;
  out[0] = (n + 1) / 2;
  out[1] = double_quant ? nb : 4 * nb;
  out[2] = double_quant ? 4 * nn : 0;
  out[3] = double_quant ? 4 : 0;
  out[4] = out[0] + out[1] + out[2];
  out[5] = out[4] + out[3];
  out[6] = nb;
  out[7] = double_quant ? nn : 0;
}

/* ------------------------------------------------------------------------ */
/* Quantize                                                                   */
/* ------------------------------------------------------------------------ */

/* Pairwise fp64 sum of a[lo .. lo+len) with len a power of two and entries at
 * or beyond n read as zero: sum(lo, len) = sum(lo, len/2) + sum(lo+len/2, len/2).
 * READING: the pages fix only "global FP32 mean"; this fixed order makes the
 * mean reproducible. */
static double pairwise_sum(const float* a, int64_t n, int64_t lo, int64_t len) {
  if (lo >= n) return 0.0;
  if (len == 1) return (double)a[lo];
  int64_t h = len / 2;
  return pairwise_sum(a, n, lo, h) + pairwise_sum(a, n, lo + h, h);
}

/* Quantize n fp32 weights.
 *   codes [ceil(n/2)]: element 2p in the high nibble of byte p, element 2p+1 in
 *                      the low nibble; a trailing odd element leaves 0 in the
 *                      low nibble (READING: first element high, pad 0).
 *   absmax[nb]       : per-block max |w| (the stored scales when !double_quant).
 *   double_quant     : also qabs[nb] (dynamic8 codes), nested[nn] (per nested
 *                      block max |absmax - mean|) and offset[1] (the mean).
 * Returns 0, or -1 if any weight is not finite (outputs then unspecified). */
int orc_quantize(const float* w, int64_t n, int double_quant, uint8_t* codes, float* absmax,
                 uint8_t* qabs, float* nested, float* offset) {
  float c4[16], t4[15], d8[256], t8[255];
  orc_nf4_table(NULL, c4);
  orc_thresholds(c4, 16, t4);
  orc_dyn8_table(NULL, d8);
  orc_thresholds(d8, 256, t8);
  int64_t nb = (n + ORC_BLOCK - 1) / ORC_BLOCK;
  int bad = 0;
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(w[i])) bad = 1;
  if (bad) return -1;

  memset(codes, 0, (size_t)((n + 1) / 2));
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    int64_t lo = b * ORC_BLOCK, hi = lo + ORC_BLOCK < n ? lo + ORC_BLOCK : n;
    float a = 0.0f;
    for (int64_t i = lo; i < hi; ++i) {
      float m = fabsf(w[i]);
      if (m > a) a = m;
    }
    absmax[b] = a;
    for (int64_t i = lo; i < hi; ++i) {
      /* READING: an all-zero block stores code 7 (the 0.0 entry) everywhere. */
      uint8_t c = 7;
      if (a > 0.0f) {
        float x = w[i] / a; /* IEEE fp32 division, round to nearest */
        c = encode_one(t4, 15, x);
      }
      /* 64-element blocks start at even indices, so every byte lies inside
       * one block and each iteration owns its bytes. */
      if ((i & 1) == 0)
        codes[i >> 1] = (uint8_t)(codes[i >> 1] | (c << 4));
      else
        codes[i >> 1] = (uint8_t)(codes[i >> 1] | c);
    }
  }
  if (!double_quant) return 0;

  /* Double quantization (QLoRA): centre the block maxima by their mean, then
   * code each centred value relative to its nested block's max magnitude. The
   * NF4 codes above keep using the original absmax. */
  int64_t len = 1;
  while (len < nb) len *= 2;
  double S = pairwise_sum(absmax, nb, 0, len);
  float mu = (float)(S / (double)nb);
  *offset = mu;
  int64_t nn = (nb + ORC_NESTED - 1) / ORC_NESTED;
  for (int64_t j = 0; j < nn; ++j) {
    int64_t lo = j * ORC_NESTED, hi = lo + ORC_NESTED < nb ? lo + ORC_NESTED : nb;
    float m = 0.0f;
    for (int64_t b = lo; b < hi; ++b) {
      float c = absmax[b] - mu;
      float mag = fabsf(c);
      if (mag > m) m = mag;
    }
    nested[j] = m;
    for (int64_t b = lo; b < hi; ++b) {
      float c = absmax[b] - mu;
      /* READING: a nested block whose centred values are all zero stores the
       * dynamic8 code of 0.0 (index 127). */
      qabs[b] = (m > 0.0f) ? encode_one(t8, 255, c / m) : (uint8_t)127;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantize                                                                 */
/* ------------------------------------------------------------------------ */

/* Round-to-nearest-even of an fp32 value to bfloat16 (finite inputs). */
static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* Reconstruct n weights. Scale of block b:
 *   single quant: a'_b = absmax[b];
 *   double quant: a'_b = fl32(fl32(D8[qabs[b]] * nested[b/256]) + offset).
 * Weight: w_i = fl32(C4[code_i] * a'_b), each step rounded on its own.
 * Writes fp32 values to out_f32 and/or their bf16 RNE bits to out_bf16. */
void orc_dequantize(const uint8_t* codes, int64_t n, int double_quant, const float* absmax,
                    const uint8_t* qabs, const float* nested, float offset, float* out_f32,
                    uint16_t* out_bf16) {
  float c4[16], d8[256];
  orc_nf4_table(NULL, c4);
  orc_dyn8_table(NULL, d8);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t b = i / ORC_BLOCK;
    float scale;
    if (double_quant) {
      float t = d8[qabs[b]] * nested[b / ORC_NESTED];
      scale = t + offset;
    } else {
      scale = absmax[b];
    }
    uint8_t byte = codes[i >> 1];
    int code = (i & 1) ? (byte & 0x0f) : (byte >> 4);
    float v = c4[code] * scale;
    if (out_f32) out_f32[i] = v;
    if (out_bf16) out_bf16[i] = f32_to_bf16_rne(v);
  }
}

/* ------------------------------------------------------------------------ */
/* Linear layer, input gradient, LoRA gradients (fp64 accumulation)           */
/* ------------------------------------------------------------------------ */
/* Shapes follow nn.Linear: x [M,K], W [N,K] (the decoded weight the kernel
 * multiplies: fp32 values, or bf16 values held in fp32), y [M,N], A [r,K],
 * B [N,r]. All operand values are exactly representable in fp32; they are read
 * as given and every product and sum is formed in fp64. s is the resolved
 * adapter scale (alpha/r, or alpha/sqrt(r) for rsLoRA) as an fp32 number. */

/* Forward: T = x A^T (if r > 0); y = x W^T + s * T B^T. T may be NULL. */
void orc_linear_fwd(const float* x, int64_t M, int64_t K, const float* W, int64_t N, const float* A,
                    const float* B, int r, float s, double* y, double* T) {
  double* t = T;
  double* tbuf = NULL;
  if (r > 0 && !t) t = tbuf = (double*)malloc(sizeof(double) * (size_t)(M * r));
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    const float* xm = x + m * K;
    for (int rho = 0; rho < r; ++rho) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += (double)xm[k] * (double)A[rho * K + k];
      t[m * r + rho] = acc;
    }
    for (int64_t n = 0; n < N; ++n) {
      const float* wn = W + n * K;
      double base = 0.0;
      for (int64_t k = 0; k < K; ++k) base += (double)xm[k] * (double)wn[k];
      double lora = 0.0;
      for (int rho = 0; rho < r; ++rho) lora += t[m * r + rho] * (double)B[n * r + rho];
      y[m * N + n] = base + (double)s * lora;
    }
  }
  free(tbuf);
}

/* Input gradient: U = dY B (if r > 0); dX = dY W + s * U A. U may be NULL. */
void orc_linear_bwd_input(const float* dy, int64_t M, int64_t N, const float* W, int64_t K,
                          const float* A, const float* B, int r, float s, double* dx, double* U) {
  double* u = U;
  double* ubuf = NULL;
  if (r > 0 && !u) u = ubuf = (double*)malloc(sizeof(double) * (size_t)(M * r));
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    const float* dym = dy + m * N;
    for (int rho = 0; rho < r; ++rho) {
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) acc += (double)dym[n] * (double)B[n * r + rho];
      u[m * r + rho] = acc;
    }
    /* dx[m,k] = sum over n in order 0..N-1 of dy[m,n] W[n,k]; the loop over n
     * is outermost so that W is read row by row. */
    double* acc = dx + m * K;
    for (int64_t k = 0; k < K; ++k) acc[k] = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double g = (double)dym[n];
      const float* wn = W + n * K;
      for (int64_t k = 0; k < K; ++k) acc[k] += g * (double)wn[k];
    }
    for (int64_t k = 0; k < K; ++k) {
      double lora = 0.0;
      for (int rho = 0; rho < r; ++rho) lora += u[m * r + rho] * (double)A[rho * K + k];
      acc[k] = acc[k] + (double)s * lora;
    }
  }
  free(ubuf);
}

/* LoRA factor gradients of L with dL/dy = dY, given T = x A^T and U = dY B:
 *   dA[rho,k] = s * sum_m U[m,rho] x[m,k]     (skipped when dA is NULL: LoRA-FA)
 *   dB[n,rho] = s * sum_m dY[m,n] T[m,rho]
 * The sums over m run in order 0..M-1. */
void orc_lora_grad(const float* x, const float* dy, int64_t M, int64_t K, int64_t N, const double* T,
                   const double* U, int r, float s, double* dA, double* dB) {
  if (dA) {
#pragma omp parallel for schedule(static)
    for (int rho = 0; rho < r; ++rho) {
      double* row = dA + (int64_t)rho * K;
      for (int64_t k = 0; k < K; ++k) row[k] = 0.0;
      for (int64_t m = 0; m < M; ++m) {
        double u = U[m * r + rho];
        const float* xm = x + m * K;
        for (int64_t k = 0; k < K; ++k) row[k] += u * (double)xm[k];
      }
      for (int64_t k = 0; k < K; ++k) row[k] = (double)s * row[k];
    }
  }
  /* Each thread owns a range of output rows n; m stays the outer loop so that
   * dY is read row by row, and every dB element still sums m = 0..M-1 in order. */
  const int64_t chunk = 64;
#pragma omp parallel for schedule(dynamic)
  for (int64_t n0 = 0; n0 < N; n0 += chunk) {
    int64_t n1 = n0 + chunk < N ? n0 + chunk : N;
    for (int64_t n = n0; n < n1; ++n)
      for (int rho = 0; rho < r; ++rho) dB[n * r + rho] = 0.0;
    for (int64_t m = 0; m < M; ++m) {
      const double* tm = T + m * r;
      for (int64_t n = n0; n < n1; ++n) {
        double g = (double)dy[m * N + n];
        for (int rho = 0; rho < r; ++rho) dB[n * r + rho] += g * tm[rho];
      }
    }
    for (int64_t n = n0; n < n1; ++n)
      for (int rho = 0; rho < r; ++rho) dB[n * r + rho] = (double)s * dB[n * r + rho];
  }
}

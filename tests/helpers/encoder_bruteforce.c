/* Exhaustive check of a nearest-code encoder over fp32 inputs in [-1, 1].
 *
 * Test helper: for every fp32 bit pattern x in [-1, 1] (both signs, denormals
 * included) it calls the encoder under test (passed in as a function pointer)
 * and compares the code with its own answer, found without thresholds:
 *   mode 0: argmin over all table entries of |x - t|, ties to the lower index;
 *           distances formed in fp64, and any fp64 tie re-decided exactly by
 *           comparing 2x with t_i + t_j (both exact in fp64);
 *   mode 1: bracket [t_i, t_{i+1}] by binary search on the table values, then
 *           pick t_{i+1} iff 2x > t_i + t_{i+1} (exact in fp64).
 * `stride` > 1 visits every stride-th bit pattern plus every pattern within
 * `window` ulps of each midpoint between adjacent table entries. */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef void (*enc_fn)(const float* thr, int nthr, const float* x, int64_t n, uint8_t* out);

static float bits_to_f(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

static int nearest_argmin(const float* t, int nt, float x) {
  int best = 0;
  double bd = fabs((double)x - (double)t[0]);
  for (int i = 1; i < nt; ++i) {
    double d = fabs((double)x - (double)t[i]);
    if (d < bd) { bd = d; best = i; }
    else if (d == bd) {
      /* exact re-decision: is x strictly closer to t[i] than to t[best]? */
      double twox = 2.0 * (double)x, sum = (double)t[i] + (double)t[best];
      int closer_to_i = (t[i] > t[best]) ? (twox > sum) : (twox < sum);
      if (closer_to_i) { best = i; }
    }
  }
  return best;
}

static int nearest_bracket(const float* t, int nt, float x) {
  if (!(x > t[0])) return 0;               /* at or below the smallest entry */
  if (x >= t[nt - 1]) return nt - 1;
  int lo = 0, hi = nt - 1;                  /* invariant: t[lo] <= x < t[hi] */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (t[mid] <= x) lo = mid; else hi = mid;
  }
  return (2.0 * (double)x > (double)t[lo] + (double)t[hi]) ? hi : lo;
}

static int64_t check_range(enc_fn enc, const float* thr, const float* t, int nt, int mode,
                           uint32_t b0, uint32_t b1, uint32_t stride, uint32_t* first_bad) {
  int64_t bad = 0;
  const int64_t chunk = 1 << 16;
  int64_t count = ((int64_t)b1 - (int64_t)b0) / stride + 1;
#pragma omp parallel for schedule(dynamic) reduction(+ : bad)
  for (int64_t c0 = 0; c0 < count; c0 += chunk) {
    float xs[1 << 16];
    uint8_t codes[1 << 16];
    int64_t m = count - c0 < chunk ? count - c0 : chunk;
    for (int64_t i = 0; i < m; ++i) xs[i] = bits_to_f(b0 + (uint32_t)((c0 + i) * stride));
    enc(thr, nt - 1, xs, m, codes);
    for (int64_t i = 0; i < m; ++i) {
      int want = mode == 0 ? nearest_argmin(t, nt, xs[i]) : nearest_bracket(t, nt, xs[i]);
      if (codes[i] != want) {
        ++bad;
        uint32_t b; memcpy(&b, &xs[i], 4);
#pragma omp critical
        { if (*first_bad == 0xffffffffu) *first_bad = b; }
      }
    }
  }
  return bad;
}

/* Returns the number of mismatching inputs; visited receives the input count. */
int64_t brute_check(enc_fn enc, const float* thr, const float* table, int ntable, int mode,
                    uint32_t stride, uint32_t window, int64_t* visited, uint32_t* first_bad) {
  *first_bad = 0xffffffffu;
  int64_t bad = 0, seen = 0;
  const uint32_t one = 0x3f800000u;  /* bits of 1.0f */
  /* positive half [+0, 1] and negative half [-0, -1] */
  bad += check_range(enc, thr, table, ntable, mode, 0u, one, stride, first_bad);
  bad += check_range(enc, thr, table, ntable, mode, 0x80000000u, 0x80000000u | one, stride, first_bad);
  seen += 2 * ((int64_t)one / stride + 1);
  if (stride > 1) {
    for (int k = 0; k + 1 < ntable; ++k) {
      double mid = 0.5 * ((double)table[k] + (double)table[k + 1]);
      float f = (float)mid;
      uint32_t b; memcpy(&b, &f, 4);
      uint32_t mag = b & 0x7fffffffu, sign = b & 0x80000000u;
      uint32_t lo = mag > window ? mag - window : 0, hi = mag + window < one ? mag + window : one;
      bad += check_range(enc, thr, table, ntable, mode, sign | lo, sign | hi, 1, first_bad);
      seen += (int64_t)(hi - lo) + 1;
    }
  }
  *visited = seen;
  return bad;
}

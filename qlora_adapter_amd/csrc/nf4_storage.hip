// NF4 blockwise quantization with double quantization, and dequantization, for
// gfx950. Format and rounding rules: include/nf4lora.h (Aner docs "Packed NF4 and
// the portable QLoRA profile"; jit.kernel_identity "decode-separate-rn").
//
// Both directions are HBM-bound streams. Quantize reads 4 B/weight and writes
// 0.5 B (+ scales); dequantize reads 0.5 B (+ 1/64 B of scales) and writes 2 B
// (bf16) or 4 B (fp32). Every wave moves contiguous runs of 256 B to 1 KB per
// instruction; block maxima are reduced across the 8 lanes that hold one block,
// and the fp64 sum behind the double-quantization mean is formed as a fixed
// pairwise tree so that it is identical on every run.
#include <atomic>
#include <mutex>

#include "nf4_device.hpp"

namespace nf4 {

const uint32_t kHostNF4[NF4_CODES_COUNT] = {NF4_CODES_LIST};
const uint32_t kHostDyn8[DYN8_CODES_COUNT] = {DYN8_CODES_LIST};

namespace {

constexpr uint32_t kNF4Thr[NF4_THRESHOLDS_COUNT] = {NF4_THRESHOLDS_LIST};
constexpr uint32_t kDyn8Thr[DYN8_THRESHOLDS_COUNT] = {DYN8_THRESHOLDS_LIST};

// ---------------------------------------------------------------------------
// NF4 code lookup. The code of x = fl32(v / m) is the number of NF4
// thresholds strictly below x. The quantizer works on X = 128 x (an exact
// power-of-two scaling, so X > 128 t <=> x > t) and truncates X toward zero to
// a bin b in [-128, 128]; each of the 257 bins stores the scaled threshold
// nearest its centre and that threshold's index k, and code = k + (X > 128 t_k).
// Thresholds lie more than 0.07 (9 in X) apart and a bin is at most 2 wide,
// so a bin never reaches past its neighbouring thresholds and the count is
// exact for every X of the bin.
struct NF4Bins {
  float t[257];     // 128 t_k
  uint32_t k[257];  // k
};
constexpr NF4Bins make_nf4_bins() {
  NF4Bins r{};
  for (int i = 0; i < 257; ++i) {
    const int b = i - 128;
    const float c = b > 0 ? (float)b + 0.5f : (b < 0 ? (float)b - 0.5f : 0.0f);  // centre of the bin
    int best = 0;
    float bd = 1e30f;
    for (int k = 0; k < NF4_THRESHOLDS_COUNT; ++k) {
      float d = 128.0f * __builtin_bit_cast(float, kNF4Thr[k]) - c;
      if (d < 0) d = -d;
      if (d < bd) {
        bd = d;
        best = k;
      }
    }
    r.t[i] = 128.0f * __builtin_bit_cast(float, kNF4Thr[best]);
    r.k[i] = (uint32_t)best;
  }
  return r;
}
static __constant__ NF4Bins c_nf4_bins = make_nf4_bins();

// v_cvt_i32_f32: truncation toward zero, NaN -> 0, saturating (the defined
// hardware result also for the arguments C++ leaves undefined).
__device__ __forceinline__ int cvt_i32_rz(float x) {
  int r;
  asm volatile("v_cvt_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// Maximum of u over the 8 lanes of an aligned 8-lane group (DPP: quad lanes
// [1,0,3,2], then [2,3,0,1], then the mirror inside each half row).
__device__ __forceinline__ uint32_t max8_lanes(uint32_t u) {
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, true));
  return u;
}

constexpr float kSlowBand = 0.0001220703125f;  // 2^-13 in X = 2^-20 in x

// Codes of 8 weights of a lane; the block (64 weights) is held by 8 aligned
// lanes. Returns the packed code word (element 2p in the high nibble of byte
// p) and the block maximum m in m_out. bad is set if some weight of the block
// is not finite.
//
// m is the maximum of |v| by v_maximum3 (NaN-propagating), then over the 8
// lanes on the bit patterns (non-negative floats order like their bits, NaN
// and inf above every finite value). X is first taken as v * (128 rcp(m)):
// for 2^-120 <= m <= 2^126 (so that 1/m is normal and 128/m finite) this
// differs from 128 fl32(v/m) by at most 2^-22 |X| <= 2^-15, well inside the
// band |X - 128 t_k| < 2^-13; inside the band, and for every other m (0, below
// 2^-120, above 2^126, inf, NaN), the correctly rounded quotient decides.
// m = 0 gives the code of zero (7).
__device__ __forceinline__ uint32_t quantize8(const float (&v)[8], const float2* s_bin, float& m_out, bool& bad) {
  float mf = __builtin_elementwise_maximum(__builtin_elementwise_maximum(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
  mf = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mf, fabsf(v[3])), fabsf(v[4]));
  mf = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mf, fabsf(v[5])), fabsf(v[6]));
  mf = __builtin_elementwise_maximum(mf, fabsf(v[7]));
  const uint32_t mb = max8_lanes(__float_as_uint(mf) & 0x7fffffffu);
  bad |= mb >= 0x7f800000u;
  const bool exact = (mb - 0x03800000u) > (0x7e800000u - 0x03800000u);  // m outside [2^-120, 2^126]
  const float m = __uint_as_float(mb);
  m_out = m;
  // with exact, X = v * 0 is 0 or NaN, whose bin (128) is in range; otherwise
  // 128 rcp(m) <= 2^127 is finite and |v| <= m bounds |X| below 129
  const float rm = exact ? 0.0f : __builtin_amdgcn_rcpf(m) * 128.0f;
  float X[8];
  float2 e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    X[j] = v[j] * rm;
    e[j] = s_bin[cvt_i32_rz(X[j]) + 128];
  }
  uint32_t c[8];
  bool slow = exact;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float d = X[j] - e[j].x;
    c[j] = __float_as_uint(e[j].y) + ((d > 0.0f) ? 1u : 0u);
    slow |= fabsf(d) < kSlowBand;
  }
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(slow) != 0, 0)) {
    for (int j = 0; j < 8; ++j) {
      if (!(exact || fabsf(X[j] - e[j].x) < kSlowBand)) continue;
      if (!(m > 0.0f)) {
        c[j] = 7u;
        continue;
      }
      const float Xe = (v[j] / m) * 128.0f;  // correctly rounded quotient, scaled exactly
      int b = cvt_i32_rz(Xe);
      b = b < -128 ? -128 : (b > 128 ? 128 : b);
      const float2 ee = s_bin[b + 128];
      c[j] = __float_as_uint(ee.y) + ((Xe > ee.x) ? 1u : 0u);
    }
  }
  uint32_t packed = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) packed |= c[j] << (8 * (j >> 1) + ((j & 1) ? 0 : 4));
  return packed;
}

__global__ void k_set_status(int32_t* status) {
  if (threadIdx.x == 0) *status = 0;
}

// One workgroup (256 threads) = 64 blocks of 64 weights (4096 weights). Wave w
// (0..3) codes weights [1024 w, 1024 w + 1024) of the group in two passes of
// 512: in pass `it` lane l holds the 8 weights at 512 it + 8 l, so 8 lanes hold
// one block. Both passes' loads are issued before any coding; with 48 VGPRs
// eight waves share a SIMD, and small workgroups keep the CUs refilled (a
// 1024-thread form of the same waves streamed 8% slower from cold HBM). Writes
// the group's codes and block maxima (to `absmax`). The group's summary goes to
// *partial: with SUM the pairwise fp64 sum of its 64 maxima (zero beyond nb),
// NaN if the group holds a non-finite weight; without SUM and with partial !=
// NULL, 0 or NaN alike; with neither, *status = NF4_ENONFINITE on a non-finite
// weight.
constexpr int kQuantThreads = 256;
constexpr int64_t kQuantGroup = 4096;

template <bool SUM>
__device__ __forceinline__ void quantize_group(const float* __restrict__ w, int64_t n, int64_t group,
                                               uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                               double* __restrict__ partial, int32_t* __restrict__ status,
                                               float* s_max, float2* s_bin) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  s_bin[threadIdx.x] = make_float2(c_nf4_bins.t[threadIdx.x], __uint_as_float(c_nf4_bins.k[threadIdx.x]));
  if (threadIdx.x == 0) s_bin[256] = make_float2(c_nf4_bins.t[256], __uint_as_float(c_nf4_bins.k[256]));
  const int64_t g0 = group * kQuantGroup;
  const int64_t base = g0 + (int64_t)wave * 1024 + 8 * lane;
  const int blk0 = wave * 16 + (lane >> 3);  // block of pass 0 within the group
  bool bad = false;
  if (g0 + kQuantGroup <= n) {
    float v[2][8];
    const f32x4* p = reinterpret_cast<const f32x4*>(w + base);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const f32x4 a = p[128 * it], b = p[128 * it + 1];
      v[it][0] = a.x; v[it][1] = a.y; v[it][2] = a.z; v[it][3] = a.w;
      v[it][4] = b.x; v[it][5] = b.y; v[it][6] = b.z; v[it][7] = b.w;
    }
    uint32_t* cw = reinterpret_cast<uint32_t*>(codes) + base / 8;
    float* am = absmax + base / 64;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      float m;
      cw[64 * it] = quantize8(v[it], s_bin, m, bad);
      if ((lane & 7) == 0) {
        s_max[blk0 + 8 * it] = m;
        am[8 * it] = m;
      }
    }
  } else {
    // the matrix's last, partial group: zeros past the end, whole 8-weight
    // units with vector loads
    __syncthreads();
    const int64_t nbytes = (n + 1) / 2;
    for (int it = 0; it < 2; ++it) {
      const int64_t e0 = base + 512 * it;
      float u[8];
      if (e0 + 8 <= n) {
        const f32x4* p = reinterpret_cast<const f32x4*>(w + e0);
        const f32x4 a = p[0], b = p[1];
        u[0] = a.x; u[1] = a.y; u[2] = a.z; u[3] = a.w; u[4] = b.x; u[5] = b.y; u[6] = b.z; u[7] = b.w;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) u[j] = e0 + j < n ? w[e0 + j] : 0.0f;
      }
      float m;
      uint32_t packed = quantize8(u, s_bin, m, bad);
      if (e0 + 8 <= n) {
        *reinterpret_cast<uint32_t*>(codes + e0 / 2) = packed;
      } else if (e0 < n) {
#pragma unroll
        for (int j = 0; j < 8; ++j)  // padding nibbles past the end are zero
          if (e0 + j >= n) packed &= ~(0xfu << (8 * (j >> 1) + ((j & 1) ? 0 : 4)));
        for (int q = 0; q < 4; ++q)
          if (e0 / 2 + q < nbytes) codes[e0 / 2 + q] = (uint8_t)(packed >> (8 * q));
      }
      if ((lane & 7) == 0) {
        s_max[blk0 + 8 * it] = (e0 < n) ? m : 0.0f;
        if (e0 < n) absmax[e0 / 64] = m;
      }
    }
  }
  if (!SUM) {
    if (partial) {
      const bool group_bad = __syncthreads_or(bad);
      if (threadIdx.x == 0) *partial = group_bad ? __builtin_nan("") : 0.0;
    } else if (bad && status) {
      *status = NF4_ENONFINITE;
    }
    return;
  }
  // With double quantization the status word is written after the mean: a
  // group with a non-finite weight reports a NaN partial sum instead.
  const bool group_bad = __syncthreads_or(bad);
  if (wave == 0) {
    // Leaves 4l..4l+3 in tree order (lanes 16..63 hold zero), then a butterfly
    // that pairs lane l with l^1, l^2, ...: every step adds two adjacent,
    // equally sized subtrees, and the last two add zero subtrees.
    double t = 0.0;
    if (lane < 16)
      t = ((double)s_max[4 * lane] + (double)s_max[4 * lane + 1]) +
          ((double)s_max[4 * lane + 2] + (double)s_max[4 * lane + 3]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) t = t + __shfl_xor(t, off);
    if (lane == 0) *partial = group_bad ? __builtin_nan("") : t;
  }
}

// One matrix: workgroup g codes group g. DQ: maxima into `absmax` (workspace)
// and group sums into partials[g]; otherwise maxima into the fp32 scales and
// the status word on a non-finite weight.
template <bool DQ>
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ w, int64_t n,
                                                  uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                                  double* __restrict__ partials, int32_t* __restrict__ status) {
  __shared__ float s_max[64];
  __shared__ float2 s_bin[257];
  quantize_group<DQ>(w, n, blockIdx.x, codes, absmax, DQ ? partials + blockIdx.x : nullptr, status, s_max, s_bin);
}

// Several matrices in one launch (nf4_quantize_many): item k owns workgroups
// [group0, group0 + its groups) of the quantizer and [ngroup0, ...) of the
// nested coding (none for single quantization). Every item keeps one partial
// per group in the workspace: group sums with double quantization, 0 or NaN
// without; the per-item mean kernel turns them into the item's offset and a
// non-finite flag, and the nested-coding kernel writes the status word.
struct QuantItem {
  const float* w;
  uint8_t* codes;
  float* absmax;      // double quantization: workspace; single: the fp32 scales
  double* partials;   // workspace, one per group
  uint8_t* qabs;      // double quantization: the coded maxima (the tensor's scales)
  float* nested;
  float* offset;
  int64_t n;
  int64_t group0;
  int64_t ngroup0;
  int32_t dq;
};
struct QuantTable {
  QuantItem item[NF4_MAX_TENSORS_PER_CALL];
  int32_t count;
  int32_t* flags;   // workspace: 1 when the item holds a non-finite weight
  int32_t* status;  // may be null
};

__device__ __forceinline__ int find_item(const QuantTable& tab, int64_t b, bool nested) {
  int k = 0;
  while (k + 1 < tab.count && b >= (nested ? tab.item[k + 1].ngroup0 : tab.item[k + 1].group0)) ++k;
  return k;
}

__global__ __launch_bounds__(256) void k_quantize_many(QuantTable tab) {
  __shared__ float s_max[64];
  __shared__ float2 s_bin[257];
  const int k = find_item(tab, blockIdx.x, false);
  const QuantItem& it = tab.item[k];
  const int64_t g = (int64_t)blockIdx.x - it.group0;
  if (it.dq)
    quantize_group<true>(it.w, it.n, g, it.codes, it.absmax, it.partials + g, nullptr, s_max, s_bin);
  else
    quantize_group<false>(it.w, it.n, g, it.codes, it.absmax, it.partials + g, nullptr, s_max, s_bin);
}

// Pairwise fp64 sum of x[0..C) zero-padded to P = 2^k >= C, by the whole
// workgroup (WAVES waves), with coalesced loads. A 256-leaf subtree is loaded
// by one wave, 4 adjacent leaves per lane: levels 1-2 in the lane, levels 3-8
// by a butterfly across lanes (a + b == b + a, so every lane ends with the
// subtree's value). A round covers WAVES x J consecutive subtrees; the J
// subtree values of a wave form the next levels in registers, and the wave
// values a tree of their own through LDS. Rounds (aligned subtrees of
// 256 WAVES J leaves) are combined by a binary counter. Where P is smaller than
// a round the extra leaves are zero, and x + 0 == x leaves the P-leaf tree's
// value unchanged. Every thread returns the same value. s_wave holds WAVES
// doubles.
constexpr int kSumJ = 4;

template <int WAVES>
__device__ double pairwise_sum_wg(const double* __restrict__ x, int64_t C, double* s_wave) {
  constexpr int J = kSumJ;
  constexpr int64_t R = 256 * WAVES * J;
  int64_t P = 1;
  while (P < C) P <<= 1;
  const int64_t rounds = P > R ? P / R : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int MAXLV = 24;  // rounds < 2^24
  double stk[MAXLV];         // binary-counter stack, indexed by constants only
  double total = 0.0;
  for (int64_t r = 0; r < rounds; ++r) {
    double v[J][4];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int64_t f = r * R + ((int64_t)wave * J + j) * 256 + 4 * lane;
      if (f + 4 <= C) {
        const double2 a = *reinterpret_cast<const double2*>(x + f);
        const double2 b = *reinterpret_cast<const double2*>(x + f + 2);
        v[j][0] = a.x; v[j][1] = a.y; v[j][2] = b.x; v[j][3] = b.y;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[j][q] = f + q < C ? x[f + q] : 0.0;
      }
    }
    double s[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      double t = (v[j][0] + v[j][1]) + (v[j][2] + v[j][3]);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) t = t + __shfl_xor(t, off);
      s[j] = t;
    }
#pragma unroll
    for (int h = 1; h < J; h *= 2)
#pragma unroll
      for (int j = 0; j < J; j += 2 * h) s[j] = s[j] + s[j + h];
    if (lane == 0) s_wave[wave] = s[0];
    __syncthreads();
    double wv[WAVES];
#pragma unroll
    for (int i = 0; i < WAVES; ++i) wv[i] = s_wave[i];
#pragma unroll
    for (int h = 1; h < WAVES; h *= 2)
#pragma unroll
      for (int i = 0; i < WAVES; i += 2 * h) wv[i] = wv[i] + wv[i + h];
    double xr = wv[0];
    __syncthreads();
    if (rounds == 1) {
      total = xr;
      break;
    }
    bool carry = true;
#pragma unroll
    for (int lv = 0; lv < MAXLV; ++lv) {
      if (carry) {
        if ((r >> lv) & 1) {
          xr = stk[lv] + xr;
        } else {
          stk[lv] = xr;
          carry = false;
        }
      }
    }
  }
  if (rounds > 1) {
    const int top = 63 - __builtin_clzll((unsigned long long)rounds);
#pragma unroll
    for (int lv = 0; lv < MAXLV; ++lv)
      if (lv == top) total = stk[lv];
  }
  return total;
}

// The matrix mean alone, for large matrices (one workgroup of 1024 threads:
// 16384 partials per round): mu = fp32(S / nb) from the group partial sums;
// writes the offset and the status word (NF4_ENONFINITE when S is not finite,
// i.e. some weight was not finite).
__global__ __launch_bounds__(1024) void k_dq_mean(const double* __restrict__ partials, int64_t C, int64_t nb,
                                                  float* __restrict__ offset, int32_t* __restrict__ status) {
  __shared__ double s_wave[16];
  const double S = pairwise_sum_wg<16>(partials, C, s_wave);
  if (threadIdx.x == 0) {
    offset[0] = (float)(S / (double)nb);
    if (status) *status = isfinite(S) ? 0 : NF4_ENONFINITE;
  }
}

// ---------------------------------------------------------------------------
// dynamic8 code lookup for x = c / m in [-1, 1]: the number of dynamic8
// thresholds strictly below x, from two table reads. |x| is binned by its
// exponent and top 6 mantissa bits (bits 17..30 of the pattern; everything
// below 2^-22 falls in sub-bin 0, which holds no threshold); per sign and
// sub-bin, cb = the number of thresholds below the sub-bin. Every sub-bin
// holds at most one threshold (checked when the table is built), so the code
// is cb + (x > t_cb) (t_255 = +inf).
constexpr int kD8Sub = 1409;       // sub-bins per sign: (bits >> 17) - kD8Base in [0, 1408]
constexpr int kD8Base = 105 * 64;  // (bits >> 17) of 2^-22
struct D8Bins {
  uint8_t cb[2 * kD8Sub];  // [sign][sub-bin]
  bool ok;
};
// number of thresholds below x (strictly, or not above x when !strict)
constexpr int d8_count(float x, bool strict) {
  int lo = 0, hi = DYN8_THRESHOLDS_COUNT;
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    const float t = __builtin_bit_cast(float, kDyn8Thr[mid]);
    if (strict ? (t < x) : (t <= x))
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}
constexpr D8Bins make_d8_bins() {
  D8Bins r{};
  r.ok = true;
  for (int s = 0; s < 2; ++s)
    for (int i = 0; i < kD8Sub; ++i) {
      const float lo = i == 0 ? 0.0f : __builtin_bit_cast(float, (uint32_t)(kD8Base + i) << 17);
      const float hi = __builtin_bit_cast(float, (uint32_t)(kD8Base + i + 1) << 17);
      int cb, inside;
      if (s == 0) {  // x in [lo, hi)
        cb = d8_count(lo, true);
        inside = d8_count(hi, true) - cb;
      } else {  // x in (-hi, -lo]
        cb = d8_count(-hi, false);
        inside = d8_count(-lo, false) - cb;
      }
      if (inside > 1) r.ok = false;
      r.cb[s * kD8Sub + i] = (uint8_t)cb;
    }
  return r;
}
constexpr D8Bins kD8Bins = make_d8_bins();
static_assert(kD8Bins.ok, "a dynamic8 sub-bin holds more than one threshold");
constexpr int kD8Words = (2 * kD8Sub + 3) / 4;
struct D8Words {
  uint32_t w[kD8Words];
};
constexpr D8Words make_d8_words() {
  D8Words t{};
  for (int i = 0; i < 2 * kD8Sub; ++i) t.w[i / 4] |= (uint32_t)kD8Bins.cb[i] << (8 * (i % 4));
  return t;
}
static __constant__ D8Words c_d8_cb = make_d8_words();

__device__ __forceinline__ uint32_t dyn8_code(float x, const uint8_t* s_cb, const float* s_thr) {
  const uint32_t b = __float_as_uint(x);
  int i = (int)((b >> 17) & 0x3fffu) - kD8Base;
  i = i < 0 ? 0 : (i > kD8Sub - 1 ? kD8Sub - 1 : i);
  const uint32_t cb = s_cb[(b >> 31) * kD8Sub + i];
  return cb + ((x > s_thr[cb]) ? 1u : 0u);
}

// Double quantization after the quantizer: nested blocks j = 4 g + w, one per
// wave; lane l holds maxima 4l..4l+3 of the block, c = fl32(absmax - mu),
// nested[j] = max |c|, qabs = dynamic8 code of fl32(c / nested[j]) (127, the
// code of zero, when the block's maxima all equal mu).
struct D8Lds {
  uint32_t cbw[kD8Words];
  float thr[256];
};

// the two lookup tables into LDS (256 threads); t_255 = +inf, so x > t_255
// never holds
__device__ __forceinline__ void load_d8_tables(D8Lds& t) {
  for (int i = threadIdx.x; i < kD8Words; i += 256) t.cbw[i] = c_d8_cb.w[i];
  t.thr[threadIdx.x] = threadIdx.x < DYN8_THRESHOLDS_COUNT ? __uint_as_float(c_dyn8_thr[threadIdx.x]) : __builtin_inff();
}

__device__ __forceinline__ f32x4 load_maxima(const float* __restrict__ absmax, int64_t nb, int64_t b0) {
  f32x4 am;
  if (b0 + 4 <= nb) {
    am = *reinterpret_cast<const f32x4*>(absmax + b0);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) am[q] = (b0 + q < nb) ? absmax[b0 + q] : 0.0f;
  }
  return am;
}

// nested block j of one matrix (one wave; the tables already in LDS)
__device__ __forceinline__ void code_nested_block(f32x4 am, int64_t nb, float mu, int64_t j,
                                                  uint8_t* __restrict__ qabs, float* __restrict__ nested,
                                                  const D8Lds& t) {
  const int lane = threadIdx.x & 63;
  const int64_t b0 = j * 256 + 4 * lane;
  float c[4];
  float m = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c[q] = (b0 + q < nb) ? __fsub_rn(am[q], mu) : 0.0f;
    m = fmaxf(m, fabsf(c[q]));
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  const uint8_t* s_cb = reinterpret_cast<const uint8_t*>(t.cbw);
  uint32_t packed = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) packed |= ((m > 0.0f) ? dyn8_code(c[q] / m, s_cb, t.thr) : 127u) << (8 * q);
  if (b0 + 4 <= nb) {
    *reinterpret_cast<uint32_t*>(qabs + b0) = packed;
  } else {
    for (int q = 0; q < 4; ++q)
      if (b0 + q < nb) qabs[b0 + q] = (uint8_t)(packed >> (8 * q));
  }
  if (lane == 0) nested[j] = m;
}

// One matrix. With MEAN_IN (matrices of at most kFusedMeanPartials quantizer
// groups, one round of the sum) every workgroup forms the mean from the group
// partial sums itself, the same tree as k_dq_mean, and workgroup 0 writes the
// offset and the status word; otherwise the mean comes from k_dq_mean
// through `offset`.
constexpr int64_t kFusedMeanPartials = 4096;

template <bool MEAN_IN>
__global__ __launch_bounds__(256) void k_dq_nested(const double* __restrict__ partials, int64_t C,
                                                   const float* __restrict__ absmax, int64_t nb,
                                                   float* __restrict__ offset, uint8_t* __restrict__ qabs,
                                                   float* __restrict__ nested, int32_t* __restrict__ status) {
  __shared__ double s_wave[4];
  __shared__ D8Lds tables;
  load_d8_tables(tables);
  const int64_t nn = (nb + 255) / 256;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  // the maxima do not depend on the mean: their loads go out before it
  const f32x4 am = load_maxima(absmax, nb, j * 256 + 4 * (threadIdx.x & 63));
  float mu;
  if constexpr (MEAN_IN) {
    const double S = pairwise_sum_wg<4>(partials, C, s_wave);  // its barriers also publish the tables
    mu = (float)(S / (double)nb);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      offset[0] = mu;
      if (status) *status = isfinite(S) ? 0 : NF4_ENONFINITE;
    }
  } else {
    mu = offset[0];
    __syncthreads();
  }
  if (j < nn) code_nested_block(am, nb, mu, j, qabs, nested, tables);
}

// nf4_quantize_many, second launch: workgroup k (1024 threads) forms item k's
// pairwise group sum S; with double quantization offset = fp32(S / nb);
// flags[k] = S is not finite (for single quantization the partials are 0 or
// NaN).
__global__ __launch_bounds__(1024) void k_dq_mean_many(QuantTable tab) {
  __shared__ double s_wave[16];
  const QuantItem& it = tab.item[blockIdx.x];
  const int64_t nb = (it.n + 63) / 64, groups = (nb + kQuantGroupBlocks - 1) / kQuantGroupBlocks;
  const double S = pairwise_sum_wg<16>(it.partials, groups, s_wave);
  if (threadIdx.x == 0) {
    if (it.dq) it.offset[0] = (float)(S / (double)nb);
    tab.flags[blockIdx.x] = isfinite(S) ? 0 : 1;
  }
}

// nf4_quantize_many, third launch: the nested blocks of every double-quantized
// item (at least one workgroup); workgroup 0 writes the status word.
__global__ __launch_bounds__(256) void k_dq_nested_many(QuantTable tab) {
  __shared__ D8Lds tables;
  load_d8_tables(tables);
  if (blockIdx.x == 0 && threadIdx.x == 0 && tab.status) {
    int32_t any = 0;
    for (int k = 0; k < tab.count; ++k) any |= tab.flags[k];
    *tab.status = any ? NF4_ENONFINITE : 0;
  }
  const QuantItem& it = tab.item[find_item(tab, blockIdx.x, true)];
  __syncthreads();
  if (!it.dq) return;
  const int64_t nb = (it.n + 63) / 64, nn = (nb + 255) / 256;
  const int64_t j = ((int64_t)blockIdx.x - it.ngroup0) * 4 + (threadIdx.x >> 6);
  if (j < 0 || j >= nn) return;
  code_nested_block(load_maxima(it.absmax, nb, j * 256 + 4 * (threadIdx.x & 63)), nb, it.offset[0], j, it.qabs,
                    it.nested, tables);
}

// A unit is the 8 weights of one 32-bit code word (bytes 4u..4u+3). Wave w of
// group g handles units 64*DQ_UNITS*(4g+w) + l + 64q, q < DQ_UNITS: each code
// load is 256 contiguous bytes per wave and each bf16 store 1 KB. The group's
// blocks get their scales computed once, one thread per block, into LDS. Units past the
// last full one (n not a multiple of 8) are decoded element by element by
// group 0.
constexpr int DQ_UNITS = 8;

// Workgroup `group` of one matrix's decode (the grid of k_dequantize, or a
// range of k_dequantize_many's). The LDS arrays are the caller's.
template <bool DQ, bool BF16>
__device__ __forceinline__ void dequant_group(const uint8_t* __restrict__ codes, const void* __restrict__ scales,
                                              const float* __restrict__ nested, const float* __restrict__ offset,
                                              int64_t n, void* __restrict__ out, int64_t group, float* lut, float* sc) {
  constexpr int BLOCKS = 4 * 64 * DQ_UNITS / 8;  // blocks covered by one workgroup
  if (threadIdx.x < 16) lut[threadIdx.x] = nf4_value(threadIdx.x);
  const float mu = DQ ? offset[0] : 0.0f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t units = n / 8, nb = (n + 63) / 64;
  const int64_t ubase = (group * 4 + wave) * (64 * DQ_UNITS) + lane;
  const uint32_t* words = reinterpret_cast<const uint32_t*>(codes);
  uint32_t word[DQ_UNITS];
#pragma unroll
  for (int q = 0; q < DQ_UNITS; ++q) {
    const int64_t u = ubase + 64 * q;
    word[q] = (u < units) ? __builtin_nontemporal_load(&words[u]) : 0u;  // codes are read once
  }
  for (int t = threadIdx.x; t < BLOCKS; t += 256) {
    const int64_t b = group * BLOCKS + t;  // block of the group's range
    float a = 0.0f;
    if (b < nb) {
      if (DQ) {
        const uint8_t qv = static_cast<const uint8_t*>(scales)[b];
        a = __fadd_rn(__fmul_rn(dyn8_value(qv), nested[b >> 8]), mu);
      } else {
        a = static_cast<const float*>(scales)[b];
      }
    }
    sc[t] = a;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < DQ_UNITS; ++q) {
    const int64_t u = ubase + 64 * q;
    if (u >= units) break;
    const float a = sc[wave * 8 * DQ_UNITS + 8 * q + (lane >> 3)];
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t nib = (word[q] >> (8 * (j >> 1) + ((j & 1) ? 0 : 4))) & 15u;
      v[j] = __fmul_rn(lut[nib], a);
    }
    // streaming stores: the decoded matrix is not read back by this kernel
    if (BF16) {
      typedef float f2 __attribute__((ext_vector_type(2)));
      typedef __bf16 b2 __attribute__((ext_vector_type(2)));
      typedef uint32_t u4v __attribute__((ext_vector_type(4)));
      u4v o;
#pragma unroll
      for (int p = 0; p < 4; ++p)  // round to nearest even, one v_cvt_pk_bf16_f32 per pair
        o[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{v[2 * p], v[2 * p + 1]}), b2));
      __builtin_nontemporal_store(o, reinterpret_cast<u4v*>(out) + u);
    } else {
      typedef float f4v __attribute__((ext_vector_type(4)));
      f4v* o = reinterpret_cast<f4v*>(out) + 2 * u;
      __builtin_nontemporal_store((f4v{v[0], v[1], v[2], v[3]}), o);
      __builtin_nontemporal_store((f4v{v[4], v[5], v[6], v[7]}), o + 1);
    }
  }
  if (group == 0) {
    for (int64_t e = units * 8 + threadIdx.x; e < n; e += blockDim.x) {
      const int64_t b = e >> 6;
      const float a = DQ ? __fadd_rn(__fmul_rn(dyn8_value(static_cast<const uint8_t*>(scales)[b]), nested[b >> 8]), mu)
                         : static_cast<const float*>(scales)[b];
      const uint8_t byte = codes[e >> 1];
      const float v = __fmul_rn(lut[(e & 1) ? (byte & 15) : (byte >> 4)], a);
      if (BF16)
        static_cast<__bf16*>(out)[e] = (__bf16)v;
      else
        static_cast<float*>(out)[e] = v;
    }
  }
}

template <bool DQ, bool BF16>
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t* __restrict__ codes, const void* __restrict__ scales,
                                                    const float* __restrict__ nested, const float* __restrict__ offset,
                                                    int64_t n, void* __restrict__ out) {
  __shared__ float lut[16];
  __shared__ float sc[4 * 64 * DQ_UNITS / 8];
  dequant_group<DQ, BF16>(codes, scales, nested, offset, n, out, blockIdx.x, lut, sc);
}

// Up to NF4_MAX_TENSORS_PER_CALL matrices in one grid; the table travels in the
// kernel arguments and matrix k owns workgroups [group0, next group0).
struct DequantItem {
  const uint8_t* codes;
  const void* scales;
  const float* nested;
  const float* offset;
  void* out;
  int64_t n;
  int64_t group0;
  int32_t dq;
};
struct DequantTable {
  DequantItem item[NF4_MAX_TENSORS_PER_CALL];
  int32_t count;
};

template <bool BF16>
__global__ __launch_bounds__(256) void k_dequantize_many(DequantTable tab) {
  __shared__ float lut[16];
  __shared__ float sc[4 * 64 * DQ_UNITS / 8];
  const int64_t b = blockIdx.x;
  int k = 0;
  while (k + 1 < tab.count && b >= tab.item[k + 1].group0) ++k;
  const DequantItem& it = tab.item[k];
  if (it.dq)
    dequant_group<true, BF16>(it.codes, it.scales, it.nested, it.offset, it.n, it.out, b - it.group0, lut, sc);
  else
    dequant_group<false, BF16>(it.codes, it.scales, it.nested, it.offset, it.n, it.out, b - it.group0, lut, sc);
}

// Selected rows of a packed [V, D] table: out[t, :] = decoded row ids[t], the
// same values nf4_dequantize gives for those rows. VEC (D % 8 == 0): 8-element
// units, i.e. one 4-byte code word inside one block and one 16-byte bf16 (or
// two 16-byte fp32) stores; each thread takes EMB_UPT units 256 apart so that
// their dependent loads (id, then code word and scale) overlap. Otherwise one
// thread per element. An id outside [0, V) yields a zero row and NF4_EINVAL in
// the status word; no packed byte outside the table is read.
constexpr int EMB_UPT = 4;

template <bool DQ, bool BF16>
__device__ __forceinline__ void store_unit(void* out, int64_t o, const float (&v)[8]) {
  if (BF16) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    u4v q;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      q[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{v[2 * p], v[2 * p + 1]}), b2));
    *reinterpret_cast<u4v*>(static_cast<__bf16*>(out) + o) = q;
  } else {
    typedef float f4v __attribute__((ext_vector_type(4)));
    f4v* dst = reinterpret_cast<f4v*>(static_cast<float*>(out) + o);
    dst[0] = f4v{v[0], v[1], v[2], v[3]};
    dst[1] = f4v{v[4], v[5], v[6], v[7]};
  }
}

template <bool DQ, bool BF16, bool VEC>
__global__ __launch_bounds__(256) void k_embed_rows(NF4View w, int64_t V, int64_t D, const int64_t* __restrict__ ids,
                                                   int64_t units, void* __restrict__ out,
                                                   int32_t* __restrict__ status) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = nf4_value(threadIdx.x);
  __syncthreads();
  const float mu = DQ ? w.offset[0] : 0.0f;
  if constexpr (VEC) {
    const int64_t per_row = D / 8;
    const int64_t base = (int64_t)blockIdx.x * (256 * EMB_UPT) + threadIdx.x;
    int64_t t[EMB_UPT], c[EMB_UPT], id[EMB_UPT];
    bool live[EMB_UPT], ok[EMB_UPT];
#pragma unroll
    for (int q = 0; q < EMB_UPT; ++q) {
      const int64_t u = base + 256 * q;
      live[q] = u < units;
      t[q] = live[q] ? u / per_row : 0;
      c[q] = u - t[q] * per_row;
      id[q] = live[q] ? ids[t[q]] : 0;
    }
    uint32_t word[EMB_UPT];
    float a[EMB_UPT];
#pragma unroll
    for (int q = 0; q < EMB_UPT; ++q) {
      ok[q] = live[q] && id[q] >= 0 && id[q] < V;
      const int64_t f = ok[q] ? id[q] * D + 8 * c[q] : 0;
      word[q] = ok[q] ? reinterpret_cast<const uint32_t*>(w.codes)[f >> 3] : 0u;
      a[q] = ok[q] ? block_scale_of<DQ>(w, mu, f >> 6) : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < EMB_UPT; ++q) {
      if (!live[q]) continue;
      if (!ok[q] && status && c[q] == 0) *status = NF4_EINVAL;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = __fmul_rn(lut[(word[q] >> (8 * (j >> 1) + ((j & 1) ? 0 : 4))) & 15u], a[q]);
      store_unit<DQ, BF16>(out, t[q] * D + 8 * c[q], v);
    }
  } else {
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= units) return;
    const int64_t t = u / D, c = u - t * D;
    const int64_t id = ids[t];
    const bool ok = id >= 0 && id < V;
    if (!ok && status && c == 0) *status = NF4_EINVAL;
    const float v = ok ? decode_one<DQ>(w, mu, lut, id * D + c) : 0.0f;
    if (BF16)
      static_cast<__bf16*>(out)[u] = (__bf16)v;
    else
      static_cast<float*>(out)[u] = v;
  }
}

}  // namespace

int launch_embedding_rows(const nf4_tensor* E, int64_t V, int64_t D, const int64_t* ids, int64_t T, nf4_dtype dt,
                          void* out, int32_t* status, hipStream_t s) {
  if (status) hipLaunchKernelGGL(k_set_status, dim3(1), dim3(64), 0, s, status);
  if (T == 0) return launch_status();
  const bool vec = (D % 8) == 0, dq = E->double_quant != 0, bf = dt == NF4_BF16;
  const int64_t units = T * (vec ? D / 8 : D);
  const dim3 grid((unsigned)ceil_div(units, vec ? 256 * EMB_UPT : 256));
  const NF4View w = make_view(E);
#define NF4_EMBED(DQ_, BF_, VEC_) \
  hipLaunchKernelGGL((k_embed_rows<DQ_, BF_, VEC_>), grid, dim3(256), 0, s, w, V, D, ids, units, out, status)
  if (dq) {
    if (bf) {
      if (vec) NF4_EMBED(true, true, true); else NF4_EMBED(true, true, false);
    } else {
      if (vec) NF4_EMBED(true, false, true); else NF4_EMBED(true, false, false);
    }
  } else {
    if (bf) {
      if (vec) NF4_EMBED(false, true, true); else NF4_EMBED(false, true, false);
    } else {
      if (vec) NF4_EMBED(false, false, true); else NF4_EMBED(false, false, false);
    }
  }
#undef NF4_EMBED
  return launch_status();
}

int launch_quantize(const float* w, int64_t n, const nf4_tensor* t, void* ws, int32_t* status, hipStream_t s) {
  const int64_t nb = ceil_div(n, kBlock), nn = ceil_div(nb, kNested), groups = quant_groups(n);
  const dim3 grid((unsigned)groups);  // one workgroup per 4096 weights
  const dim3 block(kQuantThreads);
  int32_t* st = status;
  if (!t->double_quant) {
    // reset first; k_quantize writes the status word only on a non-finite weight
    if (st) hipLaunchKernelGGL(k_set_status, dim3(1), dim3(64), 0, s, st);
    hipLaunchKernelGGL(k_quantize<false>, grid, block, 0, s, w, n, t->codes, static_cast<float*>(t->scales),
                       nullptr, st);
    return launch_status();
  }
  float* absmax = static_cast<float*>(ws);
  double* partials = reinterpret_cast<double*>(static_cast<char*>(ws) + round_up(sizeof(float) * (size_t)nb, 256));
  hipLaunchKernelGGL(k_quantize<true>, grid, block, 0, s, w, n, t->codes, absmax, partials, nullptr);
  const dim3 ng((unsigned)ceil_div(nn, 4));  // one nested block per wave
  if (groups <= kFusedMeanPartials) {
    hipLaunchKernelGGL(k_dq_nested<true>, ng, dim3(256), 0, s, partials, groups, absmax, nb, t->offset,
                       static_cast<uint8_t*>(t->scales), t->nested, st);
  } else {
    hipLaunchKernelGGL(k_dq_mean, dim3(1), dim3(1024), 0, s, partials, groups, nb, t->offset, st);
    hipLaunchKernelGGL(k_dq_nested<false>, ng, dim3(256), 0, s, partials, groups, absmax, nb, t->offset,
                       static_cast<uint8_t*>(t->scales), t->nested, st);
  }
  return launch_status();
}

size_t quantize_many_ws_bytes(const nf4_tensor* t, int32_t count) {
  size_t bytes = 0;
  for (int32_t i = 0; i < count; ++i) {
    const int64_t nb = ceil_div(t[i].n, kBlock), groups = quant_groups(t[i].n);
    if (t[i].double_quant) bytes += round_up(sizeof(float) * (size_t)nb, 256);
    bytes += round_up(sizeof(double) * (size_t)groups, 256);
  }
  return bytes + round_up(sizeof(int32_t) * NF4_MAX_TENSORS_PER_CALL, 256);
}

int launch_quantize_many(const float* const* w, const nf4_tensor* t, int32_t count, void* ws, int32_t* status,
                         hipStream_t s) {
  QuantTable tab{};
  char* p = static_cast<char*>(ws);
  int64_t groups = 0, ngroups = 0;
  for (int32_t i = 0; i < count; ++i) {
    const int64_t nb = ceil_div(t[i].n, kBlock), g = quant_groups(t[i].n), nn = ceil_div(nb, kNested);
    QuantItem& it = tab.item[i];
    it.w = w[i];
    it.codes = t[i].codes;
    it.dq = t[i].double_quant;
    if (it.dq) {
      it.absmax = reinterpret_cast<float*>(p);
      p += round_up(sizeof(float) * (size_t)nb, 256);
      it.qabs = static_cast<uint8_t*>(t[i].scales);
      it.nested = t[i].nested;
      it.offset = t[i].offset;
    } else {
      it.absmax = static_cast<float*>(t[i].scales);
    }
    it.partials = reinterpret_cast<double*>(p);
    p += round_up(sizeof(double) * (size_t)g, 256);
    it.n = t[i].n;
    it.group0 = groups;
    it.ngroup0 = ngroups;
    groups += g;
    if (it.dq) ngroups += ceil_div(nn, 4);
  }
  tab.count = count;
  tab.flags = reinterpret_cast<int32_t*>(p);
  tab.status = status;
  hipLaunchKernelGGL(k_quantize_many, dim3((unsigned)groups), dim3(kQuantThreads), 0, s, tab);
  hipLaunchKernelGGL(k_dq_mean_many, dim3((unsigned)count), dim3(1024), 0, s, tab);
  hipLaunchKernelGGL(k_dq_nested_many, dim3((unsigned)(ngroups > 0 ? ngroups : 1)), dim3(256), 0, s, tab);
  return launch_status();
}

// Fixed device scratch of nf4_quantize_noalloc (the block maxima and the
// per-group partial sums that nf4_quantize keeps in its workspace): callers
// that cannot allocate pass no workspace, and every call on a device shares
// this array, which stays allocated on each device the library runs on until
// the process ends. k_quantize writes every entry a call reads before any
// kernel reads it, so nothing needs clearing between calls; calls that overlap
// on one device race on it.
static __device__ __align__(256) unsigned char scratch[kQuantizeScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

int quantize_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return NF4_EDEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      // the device address of this device's copy of the array (the host-side
      // name is only a stand-in and must not reach a kernel)
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return NF4_EDEVICE;
      }
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return NF4_OK;
}

static int64_t dequant_groups(int64_t n) {
  const int64_t units = n / 8;
  return units > 0 ? ceil_div(units, 4 * 64 * DQ_UNITS) : 1;
}

int launch_dequantize_many(const nf4_tensor* t, void* const* outs, int32_t count, nf4_dtype dt, hipStream_t s) {
  DequantTable tab{};
  int64_t groups = 0;
  for (int32_t i = 0; i < count; ++i) {
    tab.item[i] = DequantItem{t[i].codes, t[i].scales, t[i].nested, t[i].offset, outs[i], t[i].n, groups,
                              t[i].double_quant};
    groups += dequant_groups(t[i].n);
  }
  tab.count = count;
  if (dt == NF4_BF16)
    hipLaunchKernelGGL(k_dequantize_many<true>, dim3((unsigned)groups), dim3(256), 0, s, tab);
  else
    hipLaunchKernelGGL(k_dequantize_many<false>, dim3((unsigned)groups), dim3(256), 0, s, tab);
  return launch_status();
}

int launch_dequantize(const nf4_tensor* t, nf4_dtype dt, void* out, hipStream_t s) {
  const unsigned groups = (unsigned)dequant_groups(t->n);
  const bool dq = t->double_quant != 0;
  if (dq && dt == NF4_BF16)
    hipLaunchKernelGGL((k_dequantize<true, true>), dim3(groups), dim3(256), 0, s, t->codes, t->scales, t->nested,
                       t->offset, t->n, out);
  else if (dq)
    hipLaunchKernelGGL((k_dequantize<true, false>), dim3(groups), dim3(256), 0, s, t->codes, t->scales, t->nested,
                       t->offset, t->n, out);
  else if (dt == NF4_BF16)
    hipLaunchKernelGGL((k_dequantize<false, true>), dim3(groups), dim3(256), 0, s, t->codes, t->scales, t->nested,
                       t->offset, t->n, out);
  else
    hipLaunchKernelGGL((k_dequantize<false, false>), dim3(groups), dim3(256), 0, s, t->codes, t->scales,
                       t->nested, t->offset, t->n, out);
  return launch_status();
}

}  // namespace nf4

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

// NF4 code of x in [-1, 1]: the number of thresholds strictly below x (the
// thresholds are compile-time constants, so this is 15 compares with literals).
__device__ __forceinline__ uint32_t nf4_code(float x) {
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < NF4_THRESHOLDS_COUNT; ++k) c += (x > __uint_as_float(kNF4Thr[k])) ? 1u : 0u;
  return c;
}

// dynamic8 code of x in [-1, 1]: binary search for the number of the 255
// thresholds strictly below x.
__device__ __forceinline__ uint32_t dyn8_code(float x) {
  uint32_t c = 0;
#pragma unroll
  for (uint32_t step = 128; step >= 1; step >>= 1)
    if (x > __uint_as_float(c_dyn8_thr[c + step - 1])) c += step;
  return c;
}

__global__ void k_set_status(int32_t* status) {
  if (threadIdx.x == 0) *status = 0;
}

// One workgroup = 256 blocks of 64 weights = one nested block (16384 weights).
// Wave w owns blocks [64w, 64w+64) of the group; in pass `it` lane l holds the
// 8 weights starting at 512*it + 8*l of the wave's range, so 8 lanes hold one
// block. Writes codes, absmax (to `absmax`), and with DQ the group's pairwise
// fp64 sum of its 256 maxima (zero beyond nb) to partials[blockIdx.x], NaN if
// the group holds a non-finite weight.
//
// The code of x = fl32(v / m) is found through a 256-bin table over [-1, 1]:
// bin b = floor((x + 1) * 128) holds the threshold t_k nearest to its centre
// and k, and code = k + (x > t_k). Thresholds are more than 0.07 apart and a bin
// is 1/128 wide, so every x of the bin lies between t_(k-1) and t_(k+1) and the
// count is exact. x is first taken as v * rcp(m) (within 3e-7 of v / m for
// |v| <= m, m normal); only when it falls within 2^-14 |t_k| of t_k, or m is not
// a normal number, is the correctly rounded quotient computed, so the decision
// always matches fl32(v / m) > t_k.
template <bool DQ>
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ w, int64_t n,
                                                  uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                                  double* __restrict__ partials, int32_t* __restrict__ status) {
  __shared__ float s_max[256];
  __shared__ float2 s_bin[256];  // (t_k, k as bits) per bin
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  {
    const float centre = ((float)threadIdx.x + 0.5f) / 128.0f - 1.0f;
    int best = 0;
    float bd = fabsf(__uint_as_float(kNF4Thr[0]) - centre);
#pragma unroll
    for (int k = 1; k < NF4_THRESHOLDS_COUNT; ++k) {
      const float d = fabsf(__uint_as_float(kNF4Thr[k]) - centre);
      if (d < bd) {
        bd = d;
        best = k;
      }
    }
    s_bin[threadIdx.x] = make_float2(__uint_as_float(kNF4Thr[best]), __uint_as_float((uint32_t)best));
  }
  __syncthreads();
  const int64_t nbytes = (n + 1) / 2;
  const int64_t base = (int64_t)blockIdx.x * 16384 + (int64_t)wave * 4096 + 8 * lane;
  bool bad = false;
#pragma unroll 2
  for (int it = 0; it < 8; ++it) {
    const int64_t e0 = base + 512 * it;
    float v[8];
    if (e0 + 8 <= n) {
      const float4 p = *reinterpret_cast<const float4*>(w + e0);
      const float4 q = *reinterpret_cast<const float4*>(w + e0 + 4);
      v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w; v[4] = q.x; v[5] = q.y; v[6] = q.z; v[7] = q.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (e0 + j < n) ? w[e0 + j] : 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bad |= !isfinite(v[j]);
      m = fmaxf(m, fabsf(v[j]));
    }
    // maximum over the 8 lanes of the block with DPP moves (no LDS round trip):
    // quad lanes [1,0,3,2], then [2,3,0,1], then the mirror inside each 8-lane
    // half-row pairs the two quads
    m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, m), 0xB1, 0xF, 0xF, false)));
    m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, m), 0x4E, 0xF, 0xF, false)));
    m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, m), 0x141, 0xF, 0xF, false)));
    const bool exact = !(m >= 1.17549435e-38f && m <= 3.40282347e38f);  // m zero, denormal or not finite
    const float rm = __builtin_amdgcn_rcpf(m);
    // all eight table reads first, then the decisions
    float x[8];
    float2 e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = v[j] * rm;
      int b = (int)((x[j] + 1.0f) * 128.0f);
      b = b < 0 ? 0 : (b > 255 ? 255 : b);
      e[j] = s_bin[b];
    }
    uint32_t cj[8];
    uint32_t slow = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      cj[j] = __float_as_uint(e[j].y) + ((x[j] > e[j].x) ? 1u : 0u);
      slow |= (exact || fabsf(x[j] - e[j].x) < 6.103515625e-05f * fabsf(e[j].x)) ? (1u << j) : 0u;
    }
    // Rare: the correctly rounded quotient decides (kept behind a branch so the
    // division is not evaluated on the common path).
    if (__builtin_expect(slow != 0, 0)) {
      for (int j = 0; j < 8; ++j) {
        if (!((slow >> j) & 1u)) continue;
        const float xe = v[j] / m;  // IEEE division
        int be = (int)((xe + 1.0f) * 128.0f);
        be = be < 0 ? 0 : (be > 255 ? 255 : be);
        const float2 ee = s_bin[be];
        cj[j] = __float_as_uint(ee.y) + ((xe > ee.x) ? 1u : 0u);
      }
    }
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t c = cj[j];
      if (!(m > 0.0f)) c = 7u;
      if (e0 + j >= n) c = 0;  // padding nibble past the end
      // element 2p -> high nibble of byte p, element 2p+1 -> low nibble
      packed |= c << (8 * (j >> 1) + ((j & 1) ? 0 : 4));
    }
    if (e0 + 8 <= n) {
      *reinterpret_cast<uint32_t*>(codes + e0 / 2) = packed;
    } else if (e0 < n) {
      for (int p = 0; p < 4; ++p)
        if (e0 / 2 + p < nbytes) codes[e0 / 2 + p] = (uint8_t)(packed >> (8 * p));
    }
    if ((lane & 7) == 0) {
      const int local = wave * 64 + it * 8 + (lane >> 3);
      s_max[local] = (e0 < n) ? m : 0.0f;
      if (e0 < n) absmax[e0 / 64] = m;
    }
  }
  if (!DQ) {
    if (bad && status) *status = NF4_ENONFINITE;
    return;
  }
  // With double quantization the status word is written after the mean: a
  // group with a non-finite weight reports a NaN partial sum instead.
  const bool group_bad = __syncthreads_or(bad);
  if (wave == 0) {
    // Leaves 4l..4l+3 in tree order, then a butterfly that pairs lane l with
    // l^1, l^2, ...: every step adds two adjacent, equally sized subtrees.
    double t = ((double)s_max[4 * lane] + (double)s_max[4 * lane + 1]) +
               ((double)s_max[4 * lane + 2] + (double)s_max[4 * lane + 3]);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) t = t + __shfl_xor(t, off);
    if (lane == 0) partials[blockIdx.x] = group_bad ? __builtin_nan("") : t;
  }
}

// Pairwise fp64 sum of partials[0..C) zero-padded to a power of two, by the
// whole workgroup (256 threads): thread t sums an aligned run of L leaves with
// a binary-counter stack (left + right at every level); the 256 thread sums are
// then combined by a butterfly inside each wave and by (w0 + w1) + (w2 + w3)
// across the four waves. Every thread returns the same value.
__device__ double pairwise_sum_wg(const double* __restrict__ partials, int64_t C, double* s_wave) {
  int64_t P = 1;
  while (P < C) P <<= 1;
  const int64_t L = P >= 256 ? P / 256 : 1;
  const int64_t first = (int64_t)threadIdx.x * L;
  double t;
  if (L <= 16) {
    // the run's tree in registers: 16 slots, the L leaves first and zeros after
    // (x + 0 is exact, so the padded tree gives the L-leaf tree's value)
    double v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = (i < L && first + i < C) ? partials[first + i] : 0.0;
#pragma unroll
    for (int w = 1; w < 16; w *= 2)
#pragma unroll
      for (int i = 0; i < 16; i += 2 * w) v[i] = v[i] + v[i + w];
    t = v[0];
  } else {
    double stack[48];
    int top = 0;
    for (int64_t i = 0; i < L; ++i) {
      double v = (first + i < C) ? partials[first + i] : 0.0;
      int lv = 0;
      for (int64_t idx = i; idx & 1; idx >>= 1, ++lv) v = stack[lv] + v;
      stack[lv] = v;
      top = lv;
    }
    t = stack[top];
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) t = t + __shfl_xor(t, off);
  if (lane == 0) s_wave[wave] = t;
  __syncthreads();
  return (s_wave[0] + s_wave[1]) + (s_wave[2] + s_wave[3]);
}

// The matrix mean for large matrices: one workgroup forms mu = fp32(S / nb)
// from the group partial sums and writes the offset and the status word
// (NF4_ENONFINITE when S is not finite, i.e. some weight was not finite).
__global__ __launch_bounds__(256) void k_dq_mean(const double* __restrict__ partials, int64_t C, int64_t nb,
                                                 float* __restrict__ offset, int32_t* __restrict__ status) {
  __shared__ double s_wave[4];
  const double S = pairwise_sum_wg(partials, C, s_wave);
  if (threadIdx.x == 0) {
    offset[0] = (float)(S / (double)nb);
    if (status) *status = isfinite(S) ? 0 : NF4_ENONFINITE;
  }
}

// Double quantization after k_quantize. With FUSED_MEAN (matrices of at most
// kFusedMeanGroups groups) every workgroup forms the matrix mean from the group
// partial sums itself (the same code and order as k_dq_mean, so the same
// value) and workgroup 0 writes the offset and the status word; otherwise the
// mean comes from k_dq_mean through `offset`. Each wave handles nested blocks
// j = 16 g + 4 i + w, i < DQN_PER_WG / 4: lane l holds maxima 4l..4l+3 of the
// block, c = fl32(absmax - mu), nested[j] = max |c|, qabs = dynamic8 code of
// c / m.
constexpr int DQN_PER_WG = 4;
constexpr int64_t kFusedMeanGroups = 1024;

template <bool FUSED_MEAN>
__global__ __launch_bounds__(256) void k_dq_nested(const double* __restrict__ partials, int64_t C,
                                                   const float* __restrict__ absmax, int64_t nb,
                                                   float* __restrict__ offset, uint8_t* __restrict__ qabs,
                                                   float* __restrict__ nested, int32_t* __restrict__ status) {
  __shared__ double s_wave[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nn = (nb + 255) / 256;
  constexpr int IT = DQN_PER_WG / 4;
  // the maxima do not depend on the mean: their loads go out before it
  float am[IT][4];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int64_t b0 = ((int64_t)blockIdx.x * DQN_PER_WG + 4 * i + wave) * 256 + 4 * lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) am[i][q] = (b0 + q < nb) ? absmax[b0 + q] : 0.0f;
  }
  float mu;
  if constexpr (FUSED_MEAN) {
    const double S = pairwise_sum_wg(partials, C, s_wave);
    mu = (float)(S / (double)nb);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      offset[0] = mu;
      if (status) *status = isfinite(S) ? 0 : NF4_ENONFINITE;
    }
  } else {
    mu = offset[0];
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int64_t j = (int64_t)blockIdx.x * DQN_PER_WG + 4 * i + wave;
    if (j >= nn) break;
    const int64_t b0 = j * 256 + 4 * lane;
    float c[4];
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = (b0 + q < nb) ? __fsub_rn(am[i][q], mu) : 0.0f;
      m = fmaxf(m, fabsf(c[q]));
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    uint32_t packed = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) packed |= ((m > 0.0f) ? dyn8_code(c[q] / m) : 127u) << (8 * q);
    if (b0 + 4 <= nb) {
      *reinterpret_cast<uint32_t*>(qabs + b0) = packed;
    } else {
      for (int q = 0; q < 4; ++q)
        if (b0 + q < nb) qabs[b0 + q] = (uint8_t)(packed >> (8 * q));
    }
    if (lane == 0) nested[j] = m;
  }
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
  const int64_t nb = ceil_div(n, kBlock), nn = ceil_div(nb, kNested);
  const int64_t groups = nn;  // one workgroup per 16384 weights
  int32_t* st = status;
  if (!t->double_quant) {
    // reset first; k_quantize writes the status word only on a non-finite weight
    if (st) hipLaunchKernelGGL(k_set_status, dim3(1), dim3(64), 0, s, st);
    hipLaunchKernelGGL(k_quantize<false>, dim3((unsigned)groups), dim3(256), 0, s, w, n, t->codes,
                       static_cast<float*>(t->scales), nullptr, st);
    return launch_status();
  }
  float* absmax = static_cast<float*>(ws);
  double* partials = reinterpret_cast<double*>(static_cast<char*>(ws) + round_up(sizeof(float) * (size_t)nb, 256));
  hipLaunchKernelGGL(k_quantize<true>, dim3((unsigned)groups), dim3(256), 0, s, w, n, t->codes, absmax, partials,
                     nullptr);
  const dim3 ng((unsigned)ceil_div(nn, DQN_PER_WG));
  if (nn <= kFusedMeanGroups) {
    hipLaunchKernelGGL(k_dq_nested<true>, ng, dim3(256), 0, s, partials, nn, absmax, nb, t->offset,
                       static_cast<uint8_t*>(t->scales), t->nested, st);
  } else {
    hipLaunchKernelGGL(k_dq_mean, dim3(1), dim3(256), 0, s, partials, nn, nb, t->offset, st);
    hipLaunchKernelGGL(k_dq_nested<false>, ng, dim3(256), 0, s, partials, nn, absmax, nb, t->offset,
                       static_cast<uint8_t*>(t->scales), t->nested, st);
  }
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

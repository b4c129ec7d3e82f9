// Device-side helpers shared by the kernel translation units: the constant code
// tables (one copy per translation unit, no relocatable device code needed), a
// by-value view of a packed matrix, the per-element decode used by the general
// kernels, and MFMA operand types for gfx950.
#pragma once

#include "nf4_internal.hpp"

namespace nf4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMaxRank = 256;  // adapter rank limit (Aner docs "Adapter API": 1 to 256)

static __constant__ uint32_t c_nf4[NF4_CODES_COUNT] = {NF4_CODES_LIST};
static __constant__ uint32_t c_dyn8[DYN8_CODES_COUNT] = {DYN8_CODES_LIST};
static __constant__ uint32_t c_dyn8_thr[DYN8_THRESHOLDS_COUNT] = {DYN8_THRESHOLDS_LIST};

__device__ __forceinline__ float nf4_value(uint32_t code) { return __uint_as_float(c_nf4[code]); }
__device__ __forceinline__ float dyn8_value(uint32_t q) { return __uint_as_float(c_dyn8[q]); }

// Packed matrix passed by value to kernels.
struct NF4View {
  const uint8_t* codes;
  const void* scales;  // float absmax[nb] or uint8 qabs[nb]
  const float* nested;
  const float* offset;
  int64_t n;
};

inline NF4View make_view(const nf4_tensor* t) {
  return NF4View{t->codes, t->scales, t->nested, t->offset, t->n};
}

// Scale of block b: absmax (single) or fl32(fl32(D8[q] * nested) + mu) (double).
template <bool DQ>
__device__ __forceinline__ float block_scale_of(const NF4View& w, float mu, int64_t b) {
  if constexpr (DQ) {
    const uint8_t q = static_cast<const uint8_t*>(w.scales)[b];
    return __fadd_rn(__fmul_rn(dyn8_value(q), w.nested[b >> 8]), mu);
  } else {
    return static_cast<const float*>(w.scales)[b];
  }
}

// Decoded fp32 value of flat weight f (element 2p: high nibble of byte p).
template <bool DQ>
__device__ __forceinline__ float decode_one(const NF4View& w, float mu, const float* lut, int64_t f) {
  const uint8_t byte = w.codes[f >> 1];
  const uint32_t code = (f & 1) ? (byte & 15u) : (byte >> 4);
  return __fmul_rn(lut[code], block_scale_of<DQ>(w, mu, f >> 6));
}

// Tokens per partial sum of lora_grad for J output columns: enough chunks that
// (J / 512 column tiles) x chunks is about 512 workgroups, at least 32 tokens
// per chunk, a multiple of 8.
inline int64_t lora_chunk(int64_t M, int64_t J) {
  const int64_t col_tiles = (J + 511) / 512;
  int64_t chunks = (512 + col_tiles - 1) / col_tiles;
  int64_t chunk = (M + chunks - 1) / chunks;
  chunk = (chunk + 7) / 8 * 8;
  return chunk < 32 ? 32 : chunk;
}

// Large-tile bf16 kernels (nf4_gemm_fast.hip).
bool fast_linear_applies(const LinearArgs& g);
int launch_linear_fast(const LinearArgs& g, hipStream_t st);
bool group_gemm_applies(const LinearArgs* g, int n);
int launch_linear_fast_group(const LinearArgs* g, int n, hipStream_t st);
bool group_sum_applies(const LinearArgs* g, int n);
int launch_linear_fast_sum(const LinearArgs* g, int n, hipStream_t st);

}  // namespace nf4

// Causal grouped-query attention on the gfx950 matrix cores: bf16 q, k, v
// (and dO), fp32 accumulation, head dims 32, 64, 96 and 128. Same definition
// and layouts as the general kernels: softmax(q k^T / sqrt(d), causal) v per
// query head, head h reading key/value head h / (Hq / Hkv); rows are tokens,
// head h in columns h d .. h d + d - 1; the log-sum-exp of every query row
// is saved for the backward.
//
// Blocks of 32 queries and 32 keys. With the 32x32x16 bf16 MFMA, lane l
// (l32 = l % 32, group g = l / 32) of an accumulator holds column l32 and rows
// 8 i + 4 g + j in element 4 i + j. Scores are formed transposed or not so that
// the softmax runs along a lane's own elements:
//  - forward and dQ: S^T = K Q^T, so a lane owns one query and 16 of the
//    block's keys (the other 16 are in lane l ^ 32: one shuffle per row
//    reduction);
//  - dK/dV: S = Q K^T, a lane owns one key and 16 queries.
// The second product of each kernel (P V, dS K, P^T dO, dS^T Q) takes the
// lane's 16 probabilities (or dS values) as its B operand in element order:
// slot s of step t is element 8 t + s, i.e. row 16 t + 8 (s / 4) + 4 g + s % 4
// of the block; the A operand, the block transposed (d index by row), is
// gathered in that order from a row-major LDS tile with two transposing reads
// (ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i % 4 of the 4-element pieces addressed by lanes 4 e + i / 4, e = 0..3).
// P and dS are rounded to bf16 for these products; row sums, scores, dP and
// every accumulator stay fp32. Exponentials run in base 2 on log2(e)-scaled
// scores.
//
// Kernels (workgroups of 4 waves; the next block's tiles are prefetched into
// registers while the current one is multiplied):
//  k_attn_fwd_mfma  32 queries of one head; wave w takes key blocks w, w + 4,
//                   ... up to the diagonal with its own online softmax and V
//                   tile in LDS; the four (max, sum, O) are merged in LDS.
//                   Query blocks are numbered longest-first.
//  k_attn_dq_mfma   32 queries of one head: delta = rowsum(dO * O) (written
//                   for the dK/dV kernel), then dQ = scale sum_j dS_ij k_j with
//                   the key blocks split over the waves as in the forward.
//  k_attn_dkv_mfma  32 keys of one key/value head: the (query head of the
//                   group, query block at or after the keys) items are split
//                   over the waves, each staging its own Q and dO tiles.
// Partial results of the waves are added in LDS in the fixed order 3, 2, 1, 0,
// so every output is deterministic; no atomics.
#include <cmath>

#include "nf4_device.hpp"

namespace nf4 {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int AB = 32;  // rows per query or key block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 ld16(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ bf16x4 tr_read(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 __attribute__((address_space(3)))*)(p));
}

__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// Elements 8t .. 8t + 7 of a 16-element fp32 row, rounded to bf16 (nearest even).
__device__ __forceinline__ bf16x8 pack_half(const float (&x)[16], int t) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 r;
  r[0] = pk2(x[8 * t + 0], x[8 * t + 1]);
  r[1] = pk2(x[8 * t + 2], x[8 * t + 3]);
  r[2] = pk2(x[8 * t + 4], x[8 * t + 5]);
  r[3] = pk2(x[8 * t + 6], x[8 * t + 7]);
  return __builtin_bit_cast(bf16x8, r);
}

// Four consecutive accumulator elements 4i .. 4i + 3, scaled, stored as 4 bf16.
__device__ __forceinline__ void store4(__bf16* dst, const f32x16& a, int i, float sc) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x2 r;
  r[0] = pk2(a[4 * i + 0] * sc, a[4 * i + 1] * sc);
  r[1] = pk2(a[4 * i + 2] * sc, a[4 * i + 3] * sc);
  *reinterpret_cast<u32x2*>(dst) = r;
}

// A 32-row tile of columns col0 .. col0 + D - 1 of a [S, ld] bf16 matrix held
// in registers on its way to LDS: chunk c = lane + 64 i (i < D / 16) is row
// c / (D / 8), 16-byte column chunk c % (D / 8); rows past S - 1 are clamped.
template <int D>
struct TileRegs {
  bf16x8 c[D / 16];
};

template <int D>
__device__ __forceinline__ void tile_load(TileRegs<D>& t, const __bf16* src, int64_t ld, int64_t r0, int64_t S,
                                          int64_t col0, int lane) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int c = lane + 64 * i, row = c / CPR, ch = c - row * CPR;
    const int64_t gr = (r0 + row < S) ? r0 + row : S - 1;
    t.c[i] = ld16(src + gr * ld + col0 + 8 * ch);
  }
}

template <int D, int TP>
__device__ __forceinline__ void tile_store(const TileRegs<D>& t, __bf16* dst, int lane) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int c = lane + 64 * i, row = c / CPR, ch = c - row * CPR;
    *reinterpret_cast<bf16x8*>(dst + row * TP + 8 * ch) = t.c[i];
  }
}

// A operand of step t for accumulator tile tt: the transposed tile (row = d
// index 32 tt + l32) at the block rows slot order 16 t + 8 (s / 4) + 4 g + s % 4.
template <int TP>
__device__ __forceinline__ bf16x8 tr_operand(const __bf16* tile, int lane, int tt, int t) {
  const int mm = lane & 15, g = lane >> 5;
  const int c0 = 32 * tt + 16 * ((lane >> 4) & 1);
  const __bf16* base = tile + (16 * t + 4 * g + (mm >> 2)) * TP + c0 + 4 * (mm & 3);
  const bf16x4 a0 = tr_read(base), a1 = tr_read(base + 8 * TP);
  return bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
}

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int ND>
constexpr int tiles_bytes(int per_wave) {
  return 4 * per_wave * AB * (32 * ND + 16) * 2;
}

// ---------------------------------------------------------------- forward

// Workgroup = 4 waves on 32 queries of one head; wave w takes key blocks
// w, w + 4, ... up to the diagonal (next block's K fragments and V tile
// prefetched into registers), and the four (max, sum, O) triples are merged in
// LDS in the order 3, 2, 1, 0.
template <int ND>
__global__ __launch_bounds__(256) void k_attn_fwd_mfma(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                       const __bf16* __restrict__ v, int64_t S, int hq, int hkv,
                                                       int64_t lq, int64_t lk, float sl2, __bf16* __restrict__ o,
                                                       float* __restrict__ lse) {
  constexpr int D = 32 * ND, TP = D + 16, NE = ND * 16 + 2;
  constexpr int SMEM = tiles_bytes<ND>(1) > NE * 64 * 4 ? tiles_bytes<ND>(1) : NE * 64 * 4;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int h = blockIdx.y, kh = h / (hq / hkv);
  const int64_t nqb = (S + AB - 1) / AB;
  const int64_t q0 = (nqb - 1 - (int64_t)blockIdx.x) * AB;
  const int64_t ldq = lq, ldk = lk, ldo = (int64_t)hq * D;  // q rows, k and v rows, o rows
  const int64_t qi = q0 + l32, qr = qi < S ? qi : S - 1;
  bf16x8 qf[2 * ND];
#pragma unroll
  for (int st = 0; st < 2 * ND; ++st) qf[st] = ld16(q + qr * ldq + (int64_t)h * D + 16 * st + 8 * g);
  float m = -INFINITY, lsum = 0.0f;
  f32x16 acc[ND];
#pragma unroll
  for (int tt = 0; tt < ND; ++tt) acc[tt] = f32x16{};
  const int64_t kend = (q0 + AB < S) ? q0 + AB : S;
  const int64_t nkb = (kend + AB - 1) / AB;
  __bf16* vt = reinterpret_cast<__bf16*>(smem) + wave * AB * TP;
  const __bf16* kcol = k + (int64_t)kh * D + 8 * g;
  bf16x8 kc[2 * ND];
  TileRegs<D> vr;
  if (wave < nkb) {
    const int64_t kr = (wave * AB + l32 < S) ? wave * AB + l32 : S - 1;
#pragma unroll
    for (int st = 0; st < 2 * ND; ++st) kc[st] = ld16(kcol + kr * ldk + 16 * st);
    tile_load<D>(vr, v, ldk, wave * AB, S, (int64_t)kh * D, lane);
  }
  for (int64_t b = wave; b < nkb; b += 4) {
    const int64_t k0 = b * AB;
    tile_store<D, TP>(vr, vt, lane);
    const bool more = b + 4 < nkb;
    bf16x8 kn[2 * ND];
    if (more) {
      const int64_t k1 = k0 + 4 * AB;
      const int64_t kr = (k1 + l32 < S) ? k1 + l32 : S - 1;
#pragma unroll
      for (int st = 0; st < 2 * ND; ++st) kn[st] = ld16(kcol + kr * ldk + 16 * st);
      tile_load<D>(vr, v, ldk, k1, S, (int64_t)kh * D, lane);
    }
    f32x16 s = f32x16{};
#pragma unroll
    for (int st = 0; st < 2 * ND; ++st) s = mfma(kc[st], qf[st], s);
    float x[16];
    float bm = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t key = k0 + 8 * (e >> 2) + 4 * g + (e & 3);
      x[e] = key <= qi ? s[e] * sl2 : -INFINITY;
      bm = fmaxf(bm, x[e]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    // every query row sees a key of the block (keys k0 <= q0), so mn is finite
    const float mn = fmaxf(m, bm);
    const float alpha = exp2f(m - mn);
    float rs = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      x[e] = exp2f(x[e] - mn);
      rs += x[e];
    }
    rs += __shfl_xor(rs, 32);
    lsum = lsum * alpha + rs;
    m = mn;
    const bf16x8 pb0 = pack_half(x, 0), pb1 = pack_half(x, 1);
#pragma unroll
    for (int tt = 0; tt < ND; ++tt) {
      acc[tt] *= alpha;
      acc[tt] = mfma(tr_operand<TP>(vt, lane, tt, 0), pb0, acc[tt]);
      acc[tt] = mfma(tr_operand<TP>(vt, lane, tt, 1), pb1, acc[tt]);
    }
    if (more) {
#pragma unroll
      for (int st = 0; st < 2 * ND; ++st) kc[st] = kn[st];
    }
  }
  // merge: cb[e][lane] holds acc elements (e < 16 ND), then max and sum
  float* cb = reinterpret_cast<float*>(smem);
  __syncthreads();
  if (wave == 3) {
#pragma unroll
    for (int tt = 0; tt < ND; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) cb[(16 * tt + e) * 64 + lane] = acc[tt][e];
    cb[(NE - 2) * 64 + lane] = m;
    cb[(NE - 1) * 64 + lane] = lsum;
  }
#pragma unroll
  for (int w = 2; w >= 0; --w) {
    __syncthreads();
    if (wave == w) {
      const float mb = cb[(NE - 2) * 64 + lane], lb = cb[(NE - 1) * 64 + lane];
      const float M = fmaxf(mb, m);
      const float fb = (mb == -INFINITY) ? 0.0f : exp2f(mb - M);
      const float fw = (m == -INFINITY) ? 0.0f : exp2f(m - M);
      if (w > 0) {
#pragma unroll
        for (int tt = 0; tt < ND; ++tt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float* c = &cb[(16 * tt + e) * 64 + lane];
            *c = *c * fb + acc[tt][e] * fw;
          }
        cb[(NE - 2) * 64 + lane] = M;
        cb[(NE - 1) * 64 + lane] = lb * fb + lsum * fw;
      } else {
#pragma unroll
        for (int tt = 0; tt < ND; ++tt)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[tt][e] = cb[(16 * tt + e) * 64 + lane] * fb + acc[tt][e] * fw;
        lsum = lb * fb + lsum * fw;
        m = M;
      }
    }
  }
  if (wave == 0 && qi < S) {
    const float inv = 1.0f / lsum;
    __bf16* orow = o + qi * ldo + (int64_t)h * D;
#pragma unroll
    for (int tt = 0; tt < ND; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) store4(orow + 32 * tt + 8 * i + 4 * g, acc[tt], i, inv);
    if (g == 0) lse[(int64_t)h * S + qi] = (m + log2f(lsum)) * kLn2;
  }
}

// Adds the ND accumulator tiles of the four waves in the order 3, 2, 1, 0 through
// LDS (`buf`: 16 ND floats x 64 lanes); wave 0 ends with the sum. `wave` must
// be wave-uniform.
template <int ND>
__device__ __forceinline__ void wave_sum(f32x16 (&acc)[ND], float* buf, int wave, int lane) {
  __syncthreads();
  if (wave == 3) {
#pragma unroll
    for (int tt = 0; tt < ND; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) buf[(16 * tt + e) * 64 + lane] = acc[tt][e];
  }
#pragma unroll
  for (int w = 2; w >= 1; --w) {
    __syncthreads();
    if (wave == w) {
#pragma unroll
      for (int tt = 0; tt < ND; ++tt)
#pragma unroll
        for (int e = 0; e < 16; ++e) buf[(16 * tt + e) * 64 + lane] += acc[tt][e];
    }
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int tt = 0; tt < ND; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[tt][e] += buf[(16 * tt + e) * 64 + lane];
  }
}

// ---------------------------------------------------------------- dQ

// Workgroup = 4 waves on 32 queries of one head; wave w takes key blocks
// w, w + 4, ... up to the diagonal with the next K and V tiles prefetched into
// registers; the four partial dQ are added in LDS.
template <int ND>
__global__ __launch_bounds__(256) void k_attn_dq_mfma(const __bf16* __restrict__ dout, const __bf16* __restrict__ q,
                                                      const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                                                      const __bf16* __restrict__ o, const float* __restrict__ lse,
                                                      int64_t S, int hq, int hkv, int64_t lq, int64_t lk, float sl2,
                                                      float scale, float* __restrict__ delta,
                                                      __bf16* __restrict__ dq) {
  constexpr int D = 32 * ND, TP = D + 16;
  constexpr int SMEM = tiles_bytes<ND>(2) > ND * 16 * 64 * 4 ? tiles_bytes<ND>(2) : ND * 16 * 64 * 4;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int h = blockIdx.y, kh = h / (hq / hkv);
  const int64_t nqb = (S + AB - 1) / AB;
  const int64_t q0 = (nqb - 1 - (int64_t)blockIdx.x) * AB;
  const int64_t ldq = lq, ldk = lk, ldo = (int64_t)hq * D;  // q and dq rows, k and v rows, o and dO rows
  const int64_t qi = q0 + l32, qr = qi < S ? qi : S - 1;
  const __bf16* qrow = q + qr * ldq + (int64_t)h * D;
  const __bf16* drow = dout + qr * ldo + (int64_t)h * D;
  const __bf16* orow = o + qr * ldo + (int64_t)h * D;
  bf16x8 qf[2 * ND], df[2 * ND];
  float dl = 0.0f;
#pragma unroll
  for (int st = 0; st < 2 * ND; ++st) {
    qf[st] = ld16(qrow + 16 * st + 8 * g);
    df[st] = ld16(drow + 16 * st + 8 * g);
    const bf16x8 ov = ld16(orow + 16 * st + 8 * g);
#pragma unroll
    for (int u = 0; u < 8; ++u) dl += (float)df[st][u] * (float)ov[u];
  }
  dl += __shfl_xor(dl, 32);
  if (wave == 0 && qi < S && g == 0) delta[(int64_t)h * S + qi] = dl;
  const float L2 = lse[(int64_t)h * S + qr] * kLog2e;
  f32x16 acc[ND];
#pragma unroll
  for (int tt = 0; tt < ND; ++tt) acc[tt] = f32x16{};
  const int64_t kend = (q0 + AB < S) ? q0 + AB : S;
  const int64_t nkb = (kend + AB - 1) / AB;
  __bf16* kt = reinterpret_cast<__bf16*>(smem) + (2 * wave) * AB * TP;
  __bf16* vt = kt + AB * TP;
  TileRegs<D> kr, vr;
  if (wave < nkb) {
    tile_load<D>(kr, k, ldk, wave * AB, S, (int64_t)kh * D, lane);
    tile_load<D>(vr, v, ldk, wave * AB, S, (int64_t)kh * D, lane);
  }
  for (int64_t b = wave; b < nkb; b += 4) {
    const int64_t k0 = b * AB;
    tile_store<D, TP>(kr, kt, lane);
    tile_store<D, TP>(vr, vt, lane);
    if (b + 4 < nkb) {
      tile_load<D>(kr, k, ldk, k0 + 4 * AB, S, (int64_t)kh * D, lane);
      tile_load<D>(vr, v, ldk, k0 + 4 * AB, S, (int64_t)kh * D, lane);
    }
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int st = 0; st < 2 * ND; ++st) {
      s = mfma(ld16(kt + l32 * TP + 16 * st + 8 * g), qf[st], s);
      dp = mfma(ld16(vt + l32 * TP + 16 * st + 8 * g), df[st], dp);
    }
    float x[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t key = k0 + 8 * (e >> 2) + 4 * g + (e & 3);
      x[e] = key <= qi ? exp2f(s[e] * sl2 - L2) * (dp[e] - dl) : 0.0f;
    }
    const bf16x8 b0 = pack_half(x, 0), b1 = pack_half(x, 1);
#pragma unroll
    for (int tt = 0; tt < ND; ++tt) {
      acc[tt] = mfma(tr_operand<TP>(kt, lane, tt, 0), b0, acc[tt]);
      acc[tt] = mfma(tr_operand<TP>(kt, lane, tt, 1), b1, acc[tt]);
    }
  }
  wave_sum<ND>(acc, reinterpret_cast<float*>(smem), wave, lane);
  if (wave == 0 && qi < S) {
    __bf16* out = dq + qi * ldq + (int64_t)h * D;
#pragma unroll
    for (int tt = 0; tt < ND; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) store4(out + 32 * tt + 8 * i + 4 * g, acc[tt], i, scale);
  }
}

// ---------------------------------------------------------------- dK, dV

// Workgroup = 4 waves on 32 keys of one key/value head. The work items are
// the (query head of the group, query block at or after the keys) pairs,
// numbered head-major; wave w takes items w, w + 4, ... with the next item's
// Q and dO tiles, log-sum-exp and delta prefetched into registers. The four
// partial dK, dV are added in LDS.
template <int ND>
__global__ __launch_bounds__(256) void k_attn_dkv_mfma(const __bf16* __restrict__ dout, const __bf16* __restrict__ q,
                                                       const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                                                       const float* __restrict__ lse,
                                                       const float* __restrict__ delta, int64_t S, int hq, int hkv,
                                                       int64_t lq, int64_t lk, float sl2, float scale,
                                                       __bf16* __restrict__ dk, __bf16* __restrict__ dv) {
  constexpr int D = 32 * ND, TP = D + 16;
  constexpr int SMEM = tiles_bytes<ND>(2) > 2 * ND * 16 * 64 * 4 ? tiles_bytes<ND>(2) : 2 * ND * 16 * 64 * 4;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ float ls[4][AB], dls[4][AB];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int kh = blockIdx.y, grp = hq / hkv;
  const int64_t k0 = (int64_t)blockIdx.x * AB;
  const int64_t ldq = lq, ldk = lk, ldo = (int64_t)hq * D;  // q rows, k v dk dv rows, dO rows
  const int64_t kj = k0 + l32, kr = kj < S ? kj : S - 1;
  bf16x8 kf[2 * ND], vf[2 * ND];
#pragma unroll
  for (int st = 0; st < 2 * ND; ++st) {
    kf[st] = ld16(k + kr * ldk + (int64_t)kh * D + 16 * st + 8 * g);
    vf[st] = ld16(v + kr * ldk + (int64_t)kh * D + 16 * st + 8 * g);
  }
  f32x16 ak[ND], av[ND];
#pragma unroll
  for (int tt = 0; tt < ND; ++tt) ak[tt] = av[tt] = f32x16{};
  const int64_t nqb = (S + AB - 1) / AB, qb0 = k0 / AB, nq = nqb - qb0;
  const int64_t items = nq * grp;
  __bf16* qt = reinterpret_cast<__bf16*>(smem) + (2 * wave) * AB * TP;
  __bf16* dt = qt + AB * TP;
  TileRegs<D> qr_, dr_;
  float lr_ = 0.0f, dlr_ = 0.0f;
  auto fetch = [&](int64_t it) {
    const int h = kh * grp + (int)(it / nq);
    const int64_t q0 = (qb0 + it % nq) * AB;
    tile_load<D>(qr_, q, ldq, q0, S, (int64_t)h * D, lane);
    tile_load<D>(dr_, dout, ldo, q0, S, (int64_t)h * D, lane);
    const int64_t qq = (q0 + l32 < S) ? q0 + l32 : S - 1;
    lr_ = lse[(int64_t)h * S + qq] * kLog2e;
    dlr_ = delta[(int64_t)h * S + qq];
  };
  if (wave < items) fetch(wave);
  for (int64_t it = wave; it < items; it += 4) {
    const int64_t q0 = (qb0 + it % nq) * AB;
    tile_store<D, TP>(qr_, qt, lane);
    tile_store<D, TP>(dr_, dt, lane);
    if (lane < AB) {
      ls[wave][lane] = lr_;
      dls[wave][lane] = dlr_;
    }
    if (it + 4 < items) fetch(it + 4);
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int st = 0; st < 2 * ND; ++st) {
      s = mfma(ld16(qt + l32 * TP + 16 * st + 8 * g), kf[st], s);
      dp = mfma(ld16(dt + l32 * TP + 16 * st + 8 * g), vf[st], dp);
    }
    float p[16], ds[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int qrel = 8 * (e >> 2) + 4 * g + (e & 3);
      const int64_t qidx = q0 + qrel;
      const bool ok = qidx < S && kj <= qidx;
      p[e] = ok ? exp2f(s[e] * sl2 - ls[wave][qrel]) : 0.0f;
      ds[e] = p[e] * (dp[e] - dls[wave][qrel]);
    }
    const bf16x8 p0 = pack_half(p, 0), p1 = pack_half(p, 1);
    const bf16x8 d0 = pack_half(ds, 0), d1 = pack_half(ds, 1);
#pragma unroll
    for (int tt = 0; tt < ND; ++tt) {
      av[tt] = mfma(tr_operand<TP>(dt, lane, tt, 0), p0, av[tt]);
      av[tt] = mfma(tr_operand<TP>(dt, lane, tt, 1), p1, av[tt]);
      ak[tt] = mfma(tr_operand<TP>(qt, lane, tt, 0), d0, ak[tt]);
      ak[tt] = mfma(tr_operand<TP>(qt, lane, tt, 1), d1, ak[tt]);
    }
  }
  float* red = reinterpret_cast<float*>(smem);
  wave_sum<ND>(ak, red, wave, lane);
  wave_sum<ND>(av, red + ND * 16 * 64, wave, lane);
  if (wave == 0 && kj < S) {
    __bf16* krow = dk + kj * ldk + (int64_t)kh * D;
    __bf16* vrow = dv + kj * ldk + (int64_t)kh * D;
#pragma unroll
    for (int tt = 0; tt < ND; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        store4(krow + 32 * tt + 8 * i + 4 * g, ak[tt], i, scale);
        store4(vrow + 32 * tt + 8 * i + 4 * g, av[tt], i, 1.0f);
      }
  }
}

template <int ND>
void fwd_nd(const void* q, const void* k, const void* v, int64_t S, int hq, int hkv, int64_t lq, int64_t lk, float sl2,
            void* o, float* lse, hipStream_t st) {
  const dim3 grid((unsigned)ceil_div(S, AB), (unsigned)hq);
  hipLaunchKernelGGL(k_attn_fwd_mfma<ND>, grid, dim3(256), 0, st, static_cast<const __bf16*>(q),
                     static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), S, hq, hkv, lq, lk, sl2,
                     static_cast<__bf16*>(o), lse);
}

template <int ND>
void bwd_nd(const void* dout, const void* q, const void* k, const void* v, const void* o, const float* lse, int64_t S,
            int hq, int hkv, int64_t lq, int64_t lk, float sl2, float scale, float* delta, void* dq, void* dk, void* dv,
            hipStream_t st) {
  hipLaunchKernelGGL(k_attn_dq_mfma<ND>, dim3((unsigned)ceil_div(S, AB), (unsigned)hq), dim3(256), 0, st,
                     static_cast<const __bf16*>(dout), static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), static_cast<const __bf16*>(o), lse, S, hq, hkv, lq, lk, sl2, scale,
                     delta, static_cast<__bf16*>(dq));
  hipLaunchKernelGGL(k_attn_dkv_mfma<ND>, dim3((unsigned)ceil_div(S, AB), (unsigned)hkv), dim3(256), 0, st,
                     static_cast<const __bf16*>(dout), static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), lse, delta, S, hq, hkv, lq, lk, sl2, scale, static_cast<__bf16*>(dk),
                     static_cast<__bf16*>(dv));
}

}  // namespace

bool attention_mfma_supported(nf4_dtype dt, int32_t d) { return dt == NF4_BF16 && d % 32 == 0 && d <= 128; }

int launch_attention_fwd_mfma(const void* q, const void* k, const void* v, int64_t S, int32_t hq, int32_t hkv,
                              int32_t d, int64_t lq, int64_t lk, void* o, float* lse, hipStream_t st) {
  const float sl2 = (float)(kLog2e / std::sqrt((double)d));
  switch (d / 32) {
    case 1: fwd_nd<1>(q, k, v, S, hq, hkv, lq, lk, sl2, o, lse, st); break;
    case 2: fwd_nd<2>(q, k, v, S, hq, hkv, lq, lk, sl2, o, lse, st); break;
    case 3: fwd_nd<3>(q, k, v, S, hq, hkv, lq, lk, sl2, o, lse, st); break;
    case 4: fwd_nd<4>(q, k, v, S, hq, hkv, lq, lk, sl2, o, lse, st); break;
    default: return NF4_EUNSUPPORTED;
  }
  return launch_status();
}

int launch_attention_bwd_mfma(const void* dout, const void* q, const void* k, const void* v, const void* o,
                              const float* lse, int64_t S, int32_t hq, int32_t hkv, int32_t d, int64_t lq, int64_t lk,
                              float* delta, void* dq, void* dk, void* dv, hipStream_t st) {
  const double sc = 1.0 / std::sqrt((double)d);
  const float sl2 = (float)(kLog2e * sc), scale = (float)sc;
  switch (d / 32) {
    case 1: bwd_nd<1>(dout, q, k, v, o, lse, S, hq, hkv, lq, lk, sl2, scale, delta, dq, dk, dv, st); break;
    case 2: bwd_nd<2>(dout, q, k, v, o, lse, S, hq, hkv, lq, lk, sl2, scale, delta, dq, dk, dv, st); break;
    case 3: bwd_nd<3>(dout, q, k, v, o, lse, S, hq, hkv, lq, lk, sl2, scale, delta, dq, dk, dv, st); break;
    case 4: bwd_nd<4>(dout, q, k, v, o, lse, S, hq, hkv, lq, lk, sl2, scale, delta, dq, dk, dv, st); break;
    default: return NF4_EUNSUPPORTED;
  }
  return launch_status();
}

}  // namespace nf4

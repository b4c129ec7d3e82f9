// Fused NF4 + LoRA linear layer for gfx950: forward y = x W^T + s (x A^T) B^T,
// input gradient dX = dY W + s (dY B) A, and the LoRA gradients dA = s U^T x,
// dB = s dY^T T (Aner docs "Adapter API", "LoRA FA includes gradient
// preconditioning", "Mixed precision keeps stable state in FP32"; decoding as in
// include/nf4lora.h). Weights are decoded inside the matrix kernels (no decoded
// copy of W is written to memory) with the same separately rounded fp32
// operations as nf4_dequantize, then rounded to bf16 on the bf16 path.
//
// This file holds the shape-general kernels: any M, N, K, either dtype, any
// alignment of the row pitch. The large-tile bf16 kernels for 64-multiple
// shapes live in nf4_gemm_fast.hip and are chosen by launch_linear when they
// apply.
#include "nf4_internal.hpp"
#include "nf4_device.hpp"

namespace nf4 {
namespace {

// ---------------------------------------------------------------------------
// General fused linear: C[m][j] = sum_i A[m][i] * Wop[i][j] (+ LoRA epilogue)
//   forward : A = x  [M, K], i = k, j = n, Wop[k][n] = W_hat[n][k]
//   backward: A = dY [M, N], i = n, j = k, Wop[n][k] = W_hat[n][k]
// Tile 64 (m) x 64 (j), reduction step 32; 4 waves in 2 x 2, each owning one
// 32 x 32 MFMA accumulator. Operands are staged in LDS as [row][i] so that each
// lane reads its 8 (bf16) or 1 (fp32) consecutive reduction elements.
// ---------------------------------------------------------------------------
constexpr int GT = 64, GR = 32, GPAD = 8;

template <typename T, bool BWD, bool DQ>
__global__ __launch_bounds__(256) void k_linear_general(const T* __restrict__ a, int64_t M, int64_t K, int64_t N,
                                                        NF4View w, const float* __restrict__ Afac,
                                                        const float* __restrict__ Bfac, int r, float s,
                                                        const float* __restrict__ side, T* __restrict__ out) {
  __shared__ T As[GT][GR + GPAD];
  __shared__ T Bs[GT][GR + GPAD];
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = nf4_value(threadIdx.x);
  const int64_t I = BWD ? N : K;  // reduction length
  const int64_t J = BWD ? K : N;  // output columns
  const int64_t m0 = (int64_t)blockIdx.y * GT, j0 = (int64_t)blockIdx.x * GT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 32, wj = (wave & 1) * 32;
  const int lrow = tid >> 2, lcol = (tid & 3) * 8;  // loader: row, first of 8 reduction slots
  const float mu = DQ ? w.offset[0] : 0.0f;
  f32x16 acc = {};
  __syncthreads();
  for (int64_t i0 = 0; i0 < I; i0 += GR) {
    // stage A rows m0..m0+63 and decoded weights for columns j0..j0+63
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int64_t m = m0 + lrow, i = i0 + lcol + q;
      As[lrow][lcol + q] = (m < M && i < I) ? a[m * I + i] : (T)0.0f;
      const int64_t j = j0 + lrow;
      float v = 0.0f;
      if (j < J && i < I) {
        const int64_t f = BWD ? i * K + j : j * K + i;  // flat weight index n*K + k
        v = decode_one<DQ>(w, mu, lut, f);
      }
      Bs[lrow][lcol + q] = (T)v;
    }
    __syncthreads();
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int ks = 0; ks < GR; ks += 16) {
        bf16x8 av, bv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          av[e] = As[wm + (lane & 31)][ks + (lane >> 5) * 8 + e];
          bv[e] = Bs[wj + (lane & 31)][ks + (lane >> 5) * 8 + e];
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < GR; ks += 2) {
        const float av = As[wm + (lane & 31)][ks + (lane >> 5)];
        const float bv = Bs[wj + (lane & 31)][ks + (lane >> 5)];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // LoRA epilogue: forward adds s * T[m][rho] * B[n][rho]; backward adds
  // s * U[m][rho] * A[rho][k]; fp32 products and sums (32x32x2 fp32 MFMA).
  const int64_t mrow = m0 + wm + (lane & 31), jcol = j0 + wj + (lane & 31);
  for (int rho0 = 0; rho0 < r; rho0 += 2) {
    const int rho = rho0 + (lane >> 5);
    float av = 0.0f, bv = 0.0f;
    if (rho < r) {
      if (mrow < M) av = s * side[mrow * r + rho];
      if (jcol < J) bv = BWD ? Afac[(int64_t)rho * K + jcol] : Bfac[jcol * r + rho];
    }
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int64_t m = m0 + wm + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
    if (m < M && jcol < J) out[m * J + jcol] = (T)acc[e];
  }
}

// ---------------------------------------------------------------------------
// Adapter side product S[m][rho] = sum_i L[m][i] * R[i][rho] in fp32:
//   forward : L = x  [M, K], R[k][rho] = Afac[rho][k]   (T = x A^T)
//   backward: L = dY [M, N], R[n][rho] = Bfac[n][rho]   (U = dY B)
// A workgroup of 16 waves owns 16 rows; the waves split the reduction into 16
// contiguous slices, each accumulated with the 16x16x4 fp32 MFMA (lane l: row
// l % 16, reduction group G = l / 16 holding 8 consecutive i; MFMA step q uses
// element q, so step q covers i = 8G + q), with four 32-wide steps of loads in
// flight. The 16 slice sums are added in wave order.
// ---------------------------------------------------------------------------
constexpr int SR = 16;

template <typename T>
__device__ __forceinline__ void load8_row(const T* __restrict__ p, int64_t row_off, int64_t i, int64_t I, bool ok,
                                          float v[8]) {
  if (ok && i + 8 <= I && ((row_off + i) % 8) == 0) {
    if constexpr (sizeof(T) == 2) {
      const bf16x8 q = *reinterpret_cast<const bf16x8*>(p + row_off + i);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (float)q[e];
    } else {
      const float4 a = *reinterpret_cast<const float4*>(p + row_off + i);
      const float4 b = *reinterpret_cast<const float4*>(p + row_off + i + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (ok && i + e < I) ? (float)p[row_off + i + e] : 0.0f;
  }
}

template <typename T, bool BWD>
__global__ __launch_bounds__(1024) void k_side(const T* __restrict__ L, int64_t M, int64_t I,
                                               const float* __restrict__ fac, int r, float* __restrict__ outS) {
  constexpr int SW = 16;  // waves per workgroup, each reducing one slice of I
  __shared__ float red[SW][16 * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, G = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * SR;
  const int64_t m = m0 + row;
  const bool mok = m < M;
  // reduction slice of this wave, a multiple of 32 long
  const int64_t slice = ((I + SW - 1) / SW + 31) / 32 * 32;
  const int64_t ib = wave * slice, ie = (ib + slice < I) ? ib + slice : I;
  const int RT = (r + 15) / 16;
  f32x4 acc[kMaxRank / 16];
#pragma unroll
  for (int t = 0; t < kMaxRank / 16; ++t) acc[t] = f32x4{};
  for (int64_t i0 = ib; i0 < ie; i0 += 128) {
    // four 32-wide steps of L in flight at once
    float lv[4][8];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) load8_row<T>(L, m * I, i0 + 32 * q4 + 8 * G, ie, mok, lv[q4]);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int64_t i = i0 + 32 * q4 + 8 * G;
#pragma unroll
      for (int t = 0; t < kMaxRank / 16; ++t) {
        if (t >= RT) break;
        const int rho = 16 * t + row;
        float rv[8];
        if (BWD) {
#pragma unroll
          for (int e = 0; e < 8; ++e) rv[e] = (rho < r && i + e < ie) ? fac[(i + e) * r + rho] : 0.0f;
        } else {
          load8_row<float>(fac, (int64_t)rho * I, i, ie, rho < r, rv);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(lv[q4][q], rv[q], acc[t], 0, 0, 0);
      }
    }
  }
  // accumulator element j of lane l: row 4 * (l / 16) + j, column l % 16; the
  // 16 slice sums are added in wave order
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wave][(4 * G + j) * 16 + row] = acc[t][j];
    __syncthreads();
    if (tid < 256) {
      float v = 0.0f;
#pragma unroll
      for (int w2 = 0; w2 < SW; ++w2) v += red[w2][tid];
      const int rr = tid >> 4, cc = tid & 15;
      const int64_t mm = m0 + rr;
      const int rho = 16 * t + cc;
      if (mm < M && rho < r) outS[mm * r + rho] = v;
    }
    __syncthreads();
  }
}

// Transposing 8-byte LDS read (ds_read_b64_tr_b16): within a 16-lane group,
// lane i receives element i % 4 of the 4-element pieces addressed by lanes
// 4 e + i / 4, e = 0..3.
typedef __bf16 bf16x4l __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x4l lds_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4l __attribute__((address_space(3)))*)(p));
}

// Side product for bf16 activations and r <= 32: ranks rho0 .. rho0 + 16 RT - 1
// (ranks beyond 32 take k_side_wide, which shares each factor block between
// 128 rows). Same
// work split as k_side (16 rows per workgroup, 16 waves each reducing one
// slice of I, slice sums added in wave order), but on the bf16 16x16x32 MFMA:
// the fp32 factor is split into three bf16 parts whose sum is exact, so every
// product L * R_p is exact in fp32 and the sum keeps fp32 accuracy. Lane l
// handles row l % 16 of L, rank 16 t + l % 16 of the factor and reduction
// indices 8 (l / 16) .. + 8 of each 32-wide chunk; PD chunks of loads are in
// flight before any arithmetic (fewer for many rank tiles, to bound registers).
// The slice sums are reduced through LDS four rank tiles at a time.
// GRP (forward only, one rank tile): grid row y is projection y of a grouped
// call, its adapter (rank <= 16) grp.fac[y] and output grp.out[y], so one
// launch covers the side products of all the projections of a group.
struct SideGroup {
  const float* fac[4];
  float* out[4];
  int r[4];
};

template <bool BWD, int RT, bool GRP = false>
__global__ __launch_bounds__(1024) void k_side_bf16(const __bf16* __restrict__ L, int64_t M, int64_t I,
                                                    const float* __restrict__ fac, int r, int rho0,
                                                    float* __restrict__ outS, SideGroup grp = {}) {
  static_assert(!GRP || (!BWD && RT == 1), "grouped side products are forward ones, one rank tile each");
  if constexpr (GRP) {  // this workgroup's projection (workgroup-uniform)
    fac = grp.fac[blockIdx.y];
    outS = grp.out[blockIdx.y];
    r = grp.r[blockIdx.y];
  }
  static_assert(RT <= 4, "rank tiles per launch");
  constexpr int SW = 16, PD = RT <= 2 ? 4 : 2;
  constexpr int RR = RT < 4 ? RT : 4;  // rank tiles per reduction round
  __shared__ float red[SW][RR][16 * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * SR;
  const int64_t m = m0 + row;
  const bool mok = m < M;
  const int64_t mrow = mok ? m : M - 1;
  const int64_t NC = (I + 31) / 32;
  const int64_t cpw = (NC + SW - 1) / SW;
  const int64_t cb = wave * cpw, ce = (cb + cpw < NC) ? cb + cpw : NC;
  const bool vec_l = (I % 8) == 0;
  const bool vec_f = !BWD && (I % 4) == 0 && (reinterpret_cast<uintptr_t>(fac) % 16) == 0;
  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{};
  for (int64_t c0 = cb; c0 < ce; c0 += PD) {
    bf16x8 lv[PD];
    float rv[PD][RT][8];
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const bool cok = c0 + u < ce;
      const int64_t i = 32 * (cok ? c0 + u : ce - 1) + 8 * kg;
      // L[m][i .. i + 7], zero past I, past M or for a chunk past the slice
      if (vec_l && i + 8 <= I) {
        lv[u] = *reinterpret_cast<const bf16x8*>(L + mrow * I + i);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) lv[u][e] = (i + e < I) ? L[mrow * I + i + e] : (__bf16)0.0f;
      }
      if (!(cok && mok)) lv[u] = bf16x8{};
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int rho = rho0 + 16 * t + row;
        if (BWD) {
#pragma unroll
          for (int e = 0; e < 8; ++e) rv[u][t][e] = (rho < r && i + e < I) ? fac[(i + e) * r + rho] : 0.0f;
        } else if (vec_f && i + 8 <= I && rho < r) {
          const float4 a = *reinterpret_cast<const float4*>(fac + (int64_t)rho * I + i);
          const float4 b = *reinterpret_cast<const float4*>(fac + (int64_t)rho * I + i + 4);
          rv[u][t][0] = a.x; rv[u][t][1] = a.y; rv[u][t][2] = a.z; rv[u][t][3] = a.w;
          rv[u][t][4] = b.x; rv[u][t][5] = b.y; rv[u][t][6] = b.z; rv[u][t][7] = b.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) rv[u][t][e] = (rho < r && i + e < I) ? fac[(int64_t)rho * I + i + e] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < PD; ++u) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        bf16x8 p1, p2, p3;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = rv[u][t][e];
          const __bf16 h1 = (__bf16)v;
          const float r1 = v - (float)h1;
          const __bf16 h2 = (__bf16)r1;
          p1[e] = h1;
          p2[e] = h2;
          p3[e] = (__bf16)(r1 - (float)h2);
        }
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lv[u], p3, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lv[u], p2, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lv[u], p1, acc[t], 0, 0, 0);
      }
    }
  }
  // accumulator element j of lane l: row 4 (l / 16) + j, column l % 16; the
  // slice sums are added in wave order, RR rank tiles per round
#pragma unroll
  for (int t0 = 0; t0 < RT; t0 += RR) {
    if (t0 > 0) __syncthreads();  // the previous round's sums are read
#pragma unroll
    for (int q = 0; q < RR; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[wave][q][(4 * kg + j) * 16 + row] = acc[t0 + q][j];
    __syncthreads();
    if (tid < 256 * RR) {
      const int q = tid >> 8, e = tid & 255;
      float v = 0.0f;
#pragma unroll
      for (int w2 = 0; w2 < SW; ++w2) v += red[w2][q][e];
      const int64_t mm = m0 + (e >> 4);
      const int rho = rho0 + 16 * (t0 + q) + (e & 15);
      if (mm < M && rho < r) outS[mm * r + rho] = v;
    }
  }
}

// Side product for bf16 activations and ranks beyond 32, as a skinny GEMM
// with the reduction split: workgroup (b, ks, z) covers rows 128 b .. + 127,
// reduction indices [ks kc, ks kc + kc) and ranks 64 z .. 64 z + 63. Per
// 32-wide reduction step the whole workgroup stages the factor block (64 ranks
// x 32 indices, fp32) once: each thread loads 8 values with 16-byte loads,
// splits each into three bf16 parts whose sum is exact and stores the parts in
// LDS, where all four waves read them (so the split and the factor traffic are
// paid once per 128 rows). Forward (A [r][I]) the parts are stored [rank][i]
// and read with 16-byte loads; backward (B [I][r]) they are stored [i][rank]
// and gathered with transposing reads. Wave w multiplies rows 32 w .. + 31 (two
// 16-row tiles, its activations loaded directly as 8 consecutive indices per
// lane) on the 16x16x32 bf16 MFMA. The loads of steps s + 1 and s + 2 are in
// flight while step s multiplies. Each split writes its sums to out + ks *
// part_stride; with more than one split k_side_sum adds them in split order.
constexpr int SW_FP = 40;  // bf16 pitch of a staged forward factor row (32 indices + 8)
constexpr int SW_BP = 72;  // bf16 pitch of a staged backward factor row (64 ranks + 8)

template <bool BWD, bool FAST>
__global__ __launch_bounds__(256) void k_side_wide(const __bf16* __restrict__ L, int64_t M, int64_t I,
                                                   const float* __restrict__ fac, int r, int64_t kc,
                                                   float* __restrict__ out, int64_t part_stride) {
  constexpr int FSZ = BWD ? 32 * SW_BP : 64 * SW_FP;  // bf16 per part and stage
  __shared__ __attribute__((aligned(16))) __bf16 fp[2][3][FSZ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int64_t mw = (int64_t)blockIdx.x * 128 + 32 * wave;  // first row of this wave
  const int64_t kb = (int64_t)blockIdx.y * kc, ke = (kb + kc < I) ? kb + kc : I;
  const int rho0 = 64 * (int)blockIdx.z;
  const int64_t steps = (ke - kb + 31) / 32;
  // staging role: forward, rank sr = tid / 4 and indices 8 (tid % 4) .. + 7;
  // backward, index sr = tid / 8 and ranks 8 (tid % 8) .. + 7
  const int sr = BWD ? (tid >> 3) : (tid >> 2), sq = BWD ? (tid & 7) : (tid & 3);
  // one step's loads: the activations of the wave's two row tiles and the
  // thread's 8 factor values, with their in-range flags
  struct Set {
    bf16x8 lv[2];
    float fv[8];
    bool lok[2], fok;
  };
  // FAST (I % 8 == 0, r % 8 == 0, 16-byte aligned arrays): every 8-element
  // piece is wholly in range or wholly out, so each is one unconditional
  // 16-byte load from a clamped address, zeroed at its use when out of range
  // (a step past the last loads in-range data that is never used); no load
  // sits behind a branch and none waits on another. Otherwise element-wise
  // guards.
  auto load = [&](int64_t k0, Set& S) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int64_t m = mw + 16 * rt + row, i = k0 + 8 * kg;
      if constexpr (FAST) {
        S.lok[rt] = m < M && i < ke;
        S.lv[rt] = *reinterpret_cast<const bf16x8*>(L + (m < M ? m : M - 1) * I + (i < ke ? i : kb));
      } else {
        S.lok[rt] = true;
#pragma unroll
        for (int e = 0; e < 8; ++e) S.lv[rt][e] = (m < M && i + e < ke) ? L[m * I + i + e] : (__bf16)0.0f;
      }
    }
    // BWD: B[i][rho], i = k0 + sr, rho = rho0 + 8 sq + e
    // FWD: A[rho][i], rho = rho0 + sr, i = k0 + 8 sq + e
    const int64_t i = BWD ? k0 + sr : k0 + 8 * sq;
    const int rho = BWD ? rho0 + 8 * sq : rho0 + sr;
    if constexpr (FAST) {
      S.fok = i < ke && rho < r;
      const float* q = BWD ? fac + (i < ke ? i : kb) * r + (rho < r ? rho : 0)
                           : fac + (int64_t)(rho < r ? rho : 0) * I + (i < ke ? i : kb);
      const float4 a = *reinterpret_cast<const float4*>(q), b = *reinterpret_cast<const float4*>(q + 4);
      S.fv[0] = a.x; S.fv[1] = a.y; S.fv[2] = a.z; S.fv[3] = a.w;
      S.fv[4] = b.x; S.fv[5] = b.y; S.fv[6] = b.z; S.fv[7] = b.w;
    } else {
      S.fok = true;
      if (BWD) {
#pragma unroll
        for (int e = 0; e < 8; ++e) S.fv[e] = (i < ke && rho + e < r) ? fac[i * r + rho + e] : 0.0f;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) S.fv[e] = (rho < r && i + e < ke) ? fac[(int64_t)rho * I + i + e] : 0.0f;
      }
    }
  };
  f32x4 acc[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[rt][t] = f32x4{};
  // one step from register set S into LDS stage buf: stage the factor's three
  // exact bf16 parts, then (after the barrier) load step `next` into S and
  // multiply
  auto step = [&](int buf, Set& S, int64_t next) __attribute__((always_inline)) {
    {
      bf16x8 h[3];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = S.fok ? S.fv[e] : 0.0f;
        const __bf16 a1 = (__bf16)v;
        const float r1 = v - (float)a1;
        const __bf16 a2 = (__bf16)r1;
        h[0][e] = a1;
        h[1][e] = a2;
        h[2][e] = (__bf16)(r1 - (float)a2);
      }
      const int off = BWD ? sr * SW_BP + 8 * sq : sr * SW_FP + 8 * sq;
#pragma unroll
      for (int pp = 0; pp < 3; ++pp) *reinterpret_cast<bf16x8*>(&fp[buf][pp][off]) = h[pp];
    }
    const bf16x8 l0 = S.lok[0] ? S.lv[0] : bf16x8{}, l1 = S.lok[1] ? S.lv[1] : bf16x8{};
    __syncthreads();
    load(next, S);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int pp = 2; pp >= 0; --pp) {
        bf16x8 f;
        if (BWD) {
          bf16x4l v[2];
#pragma unroll
          for (int h = 0; h < 2; ++h)
            v[h] = lds_tr16(&fp[buf][pp][(8 * kg + 4 * h + (row >> 2)) * SW_BP + 16 * t + 4 * (row & 3)]);
          f = bf16x8{v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
        } else {
          f = *reinterpret_cast<const bf16x8*>(&fp[buf][pp][(16 * t + row) * SW_FP + 8 * kg]);
        }
        acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(l0, f, acc[0][t], 0, 0, 0);
        acc[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(l1, f, acc[1][t], 0, 0, 0);
      }
    }
  };
  // two register sets in turn: steps s + 1 and s + 2 are loading while step s
  // multiplies. The loop body has no branch (so the load waits stay exact):
  // an odd step count gets one more step past the end, all of whose values
  // are zeroed, and adding zero products leaves the sums unchanged.
  Set A, B;
  load(kb, A);
  load(kb + 32, B);
  for (int64_t s = 0; s < steps; s += 2) {
    step(0, A, kb + 32 * (s + 2));
    step(1, B, kb + 32 * (s + 3));
  }
  // accumulator element j of lane l: row 4 (l / 16) + j of the tile, rank 16 t + l % 16
  float* o = out + (int64_t)blockIdx.y * part_stride;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rho = rho0 + 16 * t + row;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t m = mw + 16 * rt + 4 * kg + j;
        if (m < M && rho < r) o[m * r + rho] = acc[rt][t][j];
      }
    }
}

// Side product for bf16 activations as a split skinny GEMM, streamed: workgroup
// (b, ks, z) covers rows 128 b .. + 127, reduction indices [ks kc, ks kc + kc)
// and the R = 16 RT ranks from R z. Per 64-wide reduction step the workgroup
// stages the factor block (R ranks x 64 indices, fp32) once, as three bf16
// parts whose sum is exact, in LDS where all four waves read them (so the split
// and the factor traffic are paid once per 128 rows); wave w multiplies rows
// 32 w .. + 31 (two 16-row tiles, activations loaded directly as 8 consecutive
// indices per lane) on the 16x16x32 bf16 MFMA. Forward (A [r][I]) the parts are
// stored [rank][index] and read with 16-byte loads; backward (B [I][r]) they
// are stored [index][rank] and gathered with transposing reads. The loads of
// the next D steps are in flight while a step multiplies (a ring of register
// sets, each refilled right after its step's barrier). Each split writes its
// sums to out + ks * part_stride; with more than one split k_side_sum adds them
// in split order.
template <bool BWD, int RT>
__global__ __launch_bounds__(256, 2) void k_side_tile(const __bf16* __restrict__ L, int64_t M, int64_t I,
                                                      const float* __restrict__ fac, int r, int64_t kc,
                                                      float* __restrict__ out, int64_t part_stride) {
  constexpr int R = 16 * RT;                  // ranks per workgroup
  constexpr int D = 3;                        // steps whose loads are in flight
  constexpr int FP = BWD ? R + 8 : 64 + 8;    // bf16 pitch of a staged factor row
  constexpr int FSZ = BWD ? 64 * FP : R * FP;  // bf16 per part and stage
  __shared__ __attribute__((aligned(16))) __bf16 fp[2][3][FSZ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, kg = lane >> 4;
  const int64_t mw = (int64_t)blockIdx.x * 128 + 32 * wave;  // first row of this wave
  const int64_t kb = (int64_t)blockIdx.y * kc, ke = (kb + kc < I) ? kb + kc : I;
  const int rho0 = R * (int)blockIdx.z;
  // factor staging: float4 q = tid + 256 u (u < RT) of the block; forward rank
  // q / 16, indices 4 (q % 16) ..; backward index q / (R / 4), ranks 4 (q % (R / 4)) ..
  auto fidx = [&](int u, int& i, int& rho) __attribute__((always_inline)) {
    const int q = tid + 256 * u;
    if (BWD) {
      i = q / (R / 4);
      rho = 4 * (q % (R / 4));
    } else {
      rho = q / 16;
      i = 4 * (q % 16);
    }
  };
  struct Set {
    uint4 lv[2][2];  // [row tile][32-wide half of the step]
    float4 fv[RT];
  };
  // Every 16-byte piece (I % 8 == 0, r % 4 == 0, 16-byte aligned arrays: the
  // caller checks) is wholly in range or wholly out, so each is one
  // unconditional load from a clamped address, masked at its use.
  auto load = [&](int64_t k0, Set& S) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int64_t m = mw + 16 * rt + row, mc = m < M ? m : M - 1;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t i = k0 + 32 * h + 8 * kg;
        S.lv[rt][h] = *reinterpret_cast<const uint4*>(L + mc * I + (i < ke ? i : kb));
      }
    }
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      int il, rl;
      fidx(u, il, rl);
      const int64_t i = k0 + il;
      const int rho = rho0 + rl;
      const float* q = BWD ? fac + (i < ke ? i : kb) * r + (rho < r ? rho : 0)
                           : fac + (int64_t)(rho < r ? rho : 0) * I + (i < ke ? i : kb);
      S.fv[u] = *reinterpret_cast<const float4*>(q);
    }
  };
  f32x4 acc[2][RT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[rt][t] = f32x4{};
  auto step = [&](int64_t k0, Set& S, int buf) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    // the factor block's three exact bf16 parts into LDS stage buf
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      int il, rl;
      fidx(u, il, rl);
      const bool ok = k0 + il < ke && rho0 + rl < r;
      const float v[4] = {S.fv[u].x, S.fv[u].y, S.fv[u].z, S.fv[u].w};
      uint16_t h[3][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = ok ? v[e] : 0.0f;
        const __bf16 a1 = (__bf16)x;
        const float r1 = x - (float)a1;
        const __bf16 a2 = (__bf16)r1;
        const __bf16 a3 = (__bf16)(r1 - (float)a2);
        h[0][e] = __builtin_bit_cast(uint16_t, a1);
        h[1][e] = __builtin_bit_cast(uint16_t, a2);
        h[2][e] = __builtin_bit_cast(uint16_t, a3);
      }
      const int off = BWD ? il * FP + rl : rl * FP + il;
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
        *reinterpret_cast<uint2*>(&fp[buf][pp][off]) =
            make_uint2(h[pp][0] | ((uint32_t)h[pp][1] << 16), h[pp][2] | ((uint32_t)h[pp][3] << 16));
    }
    // this step's activations, zeroed out of range (integer masks, so that no
    // branch waits for a load), copied out before the set is refilled
    bf16x8 l[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool ok = mw + 16 * rt + row < M && k0 + 32 * h + 8 * kg < ke;
        const uint32_t mk = ok ? 0xffffffffu : 0u;
        const uint4 v = S.lv[rt][h];
        l[rt][h] = __builtin_bit_cast(bf16x8, make_uint4(v.x & mk, v.y & mk, v.z & mk, v.w & mk));
      }
    __syncthreads();
    load(k0 + 64 * D, S);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int pp = 2; pp >= 0; --pp) {
          bf16x8 f;
          if (BWD) {
            bf16x4l v[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
              v[hh] = lds_tr16(&fp[buf][pp][(32 * h + 8 * kg + 4 * hh + (row >> 2)) * FP + 16 * t + 4 * (row & 3)]);
            f = bf16x8{v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
          } else {
            f = *reinterpret_cast<const bf16x8*>(&fp[buf][pp][(16 * t + row) * FP + 32 * h + 8 * kg]);
          }
          acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(l[0][h], f, acc[0][t], 0, 0, 0);
          acc[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(l[1][h], f, acc[1][t], 0, 0, 0);
        }
  };
  // whole rounds of D steps (no early exit, so the load waits are exact on
  // the back edge), then the last steps % D; the loads of the first D steps
  // are issued in order
  const int64_t steps = (ke - kb + 63) / 64, rounds = steps / D;
  Set S[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load(kb + 64 * d, S[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
  int64_t k0 = kb;
  int par = 0;
  for (int64_t i = 0; i < rounds; ++i) {
#pragma unroll
    for (int d = 0; d < D; ++d, k0 += 64, par ^= 1) step(k0, S[d], par);
  }
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    if (d >= steps - rounds * D) break;
    step(k0, S[d], par);
    k0 += 64;
    par ^= 1;
  }
  // accumulator element j of lane l: row 4 (l / 16) + j of the tile, rank 16 t + l % 16
  float* o = out + (int64_t)blockIdx.y * part_stride;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int rho = rho0 + 16 * t + row;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t m = mw + 16 * rt + 4 * kg + j;
        if (m < M && rho < r) o[m * r + rho] = acc[rt][t][j];
      }
    }
}

// out[e] = sum over splits ks = 0, 1, ... in order of part[ks * n + e]; four
// consecutive elements per thread (n % 4 == 0 and 16-byte aligned arrays: the
// caller checks) or one.
template <bool VEC4>
__global__ __launch_bounds__(256) void k_side_sum(const float* __restrict__ part, int64_t n, int splits,
                                                  float* __restrict__ out) {
  typedef float vec __attribute__((ext_vector_type(VEC4 ? 4 : 1)));
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * (VEC4 ? 4 : 1);
  if (e >= n) return;
  const vec* p = reinterpret_cast<const vec*>(part + e);
  const int64_t nv = n / (VEC4 ? 4 : 1);  // parts apart, in vectors
  vec v = p[0];
  // sixteen parts' loads in flight per group (a shorter last group is
  // predicated, not a chain of dependent loads), added in split order
  for (int ks = 1; ks < splits; ks += 16) {
    vec w[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) w[u] = ks + u < splits ? p[(int64_t)(ks + u) * nv] : vec{};
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (ks + u < splits) v += w[u];
  }
  *reinterpret_cast<vec*>(out + e) = v;
}

// ---------------------------------------------------------------------------
// LoRA gradients, stage 1: partial[c][rho][j] = sum over tokens m of chunk c, in
// order, of P[m][rho] * Q[m][j]; P fp32 [M, r], Q of type T [M, J]. Workgroup
// (512-column tile, chunk c); thread t owns columns j0 + 2t, j0 + 2t + 1 and a
// group of 16 ranks (groups run one after another). Each element of Q is read
// once per rank group and feeds 16 fp32 FMAs; the factor row P[m][16 g .. +16]
// is the same for the whole workgroup. The token loop is unrolled by 8 so that
// 8 rows of Q are in flight per thread.
// Stage 2 (k_lora_combine) adds the chunks in order c = 0, 1, ..., scales by s
// and writes dA ([r][J]) or dB ([J][r]).
// ---------------------------------------------------------------------------
constexpr int LCOLS = 512, LRG = 16;

// Two consecutive columns j, j + 1 of a row of Q as fp32. EVEN: J is even and
// j has been clamped to at most J - 2, so the pair is in range and aligned.
template <typename T, bool EVEN>
__device__ __forceinline__ void load_pair(const T* __restrict__ q, int64_t j, int64_t J, float& a, float& b) {
  if constexpr (EVEN) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(q + j);
      a = __uint_as_float(v << 16);
      b = __uint_as_float(v & 0xFFFF0000u);
    } else {
      const float2 v = *reinterpret_cast<const float2*>(q + j);
      a = v.x;
      b = v.y;
    }
  } else {
    a = (j < J) ? (float)q[j] : 0.0f;
    b = (j + 1 < J) ? (float)q[j + 1] : 0.0f;
  }
}

template <typename T, bool EVEN>
__global__ __launch_bounds__(256) void k_lora_partial(const float* __restrict__ P, const T* __restrict__ Q, int64_t M,
                                                      int64_t J, int r, int64_t chunk, float* __restrict__ partial) {
  constexpr int SLAB = 64;  // tokens of P staged in LDS at a time
  __shared__ __attribute__((aligned(16))) float ps[SLAB][LRG];
  const int tid = threadIdx.x;
  const int64_t j = (int64_t)blockIdx.x * LCOLS + 2 * tid;
  const int64_t jl = (EVEN && j > J - 2) ? J - 2 : j;  // load column (stores use j)
  const int64_t c = blockIdx.y;
  const int64_t mb = c * chunk, me = (mb + chunk < M) ? mb + chunk : M;
  for (int rg = 0; rg < r; rg += LRG) {
    float acc0[LRG], acc1[LRG];
#pragma unroll
    for (int q = 0; q < LRG; ++q) acc0[q] = acc1[q] = 0.0f;
    for (int64_t m0 = mb; m0 < me; m0 += SLAB) {
      // stage P[m0 .. m0 + 64][rg .. rg + 16], zero past the chunk and past rank r
#pragma unroll
      for (int e = tid; e < SLAB * LRG; e += 256) {
        const int mm = e / LRG, q = e % LRG;
        const int64_t m = m0 + mm;
        ps[mm][q] = (m < me && rg + q < r) ? P[m * r + rg + q] : 0.0f;
      }
      __syncthreads();
      const int nrow = (me - m0 < SLAB) ? (int)(me - m0) : SLAB;
      int u = 0;
      for (; u + 8 <= nrow; u += 8) {
        float qa[8], qb[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) load_pair<T, EVEN>(Q + (m0 + u + v) * J, jl, J, qa[v], qb[v]);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float4* pr = reinterpret_cast<const float4*>(ps[u + v]);
#pragma unroll
          for (int h = 0; h < LRG / 4; ++h) {
            const float4 p4 = pr[h];
            acc0[4 * h + 0] = fmaf(p4.x, qa[v], acc0[4 * h + 0]);
            acc0[4 * h + 1] = fmaf(p4.y, qa[v], acc0[4 * h + 1]);
            acc0[4 * h + 2] = fmaf(p4.z, qa[v], acc0[4 * h + 2]);
            acc0[4 * h + 3] = fmaf(p4.w, qa[v], acc0[4 * h + 3]);
            acc1[4 * h + 0] = fmaf(p4.x, qb[v], acc1[4 * h + 0]);
            acc1[4 * h + 1] = fmaf(p4.y, qb[v], acc1[4 * h + 1]);
            acc1[4 * h + 2] = fmaf(p4.z, qb[v], acc1[4 * h + 2]);
            acc1[4 * h + 3] = fmaf(p4.w, qb[v], acc1[4 * h + 3]);
          }
        }
      }
      for (; u < nrow; ++u) {
        float qa, qb;
        load_pair<T, EVEN>(Q + (m0 + u) * J, jl, J, qa, qb);
#pragma unroll
        for (int q = 0; q < LRG; ++q) {
          acc0[q] = fmaf(ps[u][q], qa, acc0[q]);
          acc1[q] = fmaf(ps[u][q], qb, acc1[q]);
        }
      }
      __syncthreads();
    }
    const int nr = (r - rg < LRG) ? r - rg : LRG;
#pragma unroll
    for (int q = 0; q < LRG; ++q) {
      if (q >= nr) break;
      float* out = partial + (c * r + rg + q) * J + j;
      if (j + 1 < J) {
        out[0] = acc0[q];
        out[1] = acc1[q];
      } else if (j < J) {
        out[0] = acc0[q];
      }
    }
  }
}

// Stage 1 on the bf16 MFMA for bf16 Q, same partial layout as k_lora_partial.
// The fp32 factor P is split into three bf16 parts whose sum is exact, so every
// product P_p[m][rho] * Q[m][j] is exact in fp32. Workgroup (256-column tile,
// chunk c) of 4 waves; wave w owns columns 64 w .. + 64 as 2 RB accumulators
// D[rho][j] of the 32x32x16 MFMA for the RB blocks of 32 ranks rho0 + 32 b ..
// (rank rows past r are zero); ranks beyond 32 RB take further launches over
// the same Q (RB = 4 covers 128 ranks). The chunk is walked in steps of 32 tokens: the workgroup stages
// Q[m .. m + 31][j0 .. j0 + 255] (rows padded to 576 bytes, so four consecutive
// rows fall in four different quarters of the banks) and the three parts of
// P[m .. m + 31][0 .. 31] (64-byte rows) in LDS; both MFMA operands need 8
// consecutive tokens per lane and are gathered with ds_read_b64_tr_b16 (within
// a 16-lane group, lane i receives element i % 4 of the 4-element pieces
// addressed by lanes 4 e + i / 4). The loads of the next two or three steps
// are in flight while the current one multiplies.
constexpr int LQP = 288;  // bf16 per staged Q row
constexpr int LPP = 32;   // bf16 per staged P row


// One token reduction of lora_grad: partial[c][rho][j] = sum over the tokens
// of chunk c of P[m][rho] Q[m][j].
struct LoraProb {
  const float* P;
  const __bf16* Q;
  int64_t J;
  int64_t chunk;
  int64_t col_tiles;  // ceil(J / 256)
  float* partial;
};

// Both reductions of one lora_grad call (dB's and dA's) share the grid:
// workgroups [0, blocks0) take problem 0, the rest problem 1; inside a problem
// workgroup b covers column tile b % col_tiles of chunk b / col_tiles.
template <int RB, bool FAST>
__global__ __launch_bounds__(256, RB <= 2 ? 2 : 1) void k_lora_mfma(LoraProb p0, LoraProb p1, int64_t blocks0,
                                                                    int64_t M, int r, int rho0) {
  // D token steps are loaded ahead into a ring of register sets, so that D
  // steps' loads are in flight while one step multiplies (two for 128 ranks
  // and for the element-wise loads, within the registers of two waves per
  // SIMD up to 64 ranks; four measured slower than three).
  constexpr int D = (RB == 4 || !FAST) ? 2 : 3;
  __shared__ __attribute__((aligned(16))) __bf16 qs[2][32 * LQP];
  __shared__ __attribute__((aligned(16))) __bf16 pls[2][RB][3][32 * LPP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = lane >> 4, i16 = lane & 15, kg = G >> 1, hs = G & 1;
  const bool second = (int64_t)blockIdx.x >= blocks0;
  const LoraProb& pr = second ? p1 : p0;
  const float* __restrict__ P = pr.P;
  const __bf16* __restrict__ Q = pr.Q;
  const int64_t J = pr.J, chunk = pr.chunk;
  float* __restrict__ partial = pr.partial;
  const int64_t b = (int64_t)blockIdx.x - (second ? blocks0 : 0);
  const int64_t j0 = (b % pr.col_tiles) * 256;
  const int64_t c = b / pr.col_tiles;
  const int64_t mb = c * chunk, me = (mb + chunk < M) ? mb + chunk : M;
  // staging roles: Q row 8 u + tid / 32 (u = 0..3), 16-byte chunk tid % 32;
  // P row tid / 8, ranks 4 (tid % 8) .. + 3
  const int qrow = tid >> 5, qch = tid & 31, prow = tid >> 3, prho = 4 * (tid & 7);
  const int64_t jq = j0 + 8 * qch;
  struct Set {
    uint4 q[4];
    float p[RB][4];
  };
  // FAST (J % 8 == 0, r % 4 == 0, 16-byte aligned Q and P): every 16-byte
  // piece is wholly in range or wholly out, so each is one unconditional load
  // from a clamped address, zeroed when it is staged if out of range (no load
  // sits behind a branch, so the waits for one set leave the later sets in
  // flight). Otherwise element-wise guards.
  auto load = [&](int64_t m, Set& S) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t mm = m + 8 * u + qrow;
      if constexpr (FAST) {
        S.q[u] = *reinterpret_cast<const uint4*>(Q + (mm < me ? mm : me - 1) * J + (jq < J ? jq : 0));
      } else {
        uint16_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          h[e] = (mm < me && jq + e < J) ? __builtin_bit_cast(uint16_t, Q[mm * J + jq + e]) : (uint16_t)0;
        S.q[u] = make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                            h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16));
      }
    }
    const int64_t mm = m + prow;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rho = rho0 + 32 * rb + prho;
      if constexpr (FAST) {
        const float4 v = *reinterpret_cast<const float4*>(P + (mm < me ? mm : me - 1) * r + (rho < r ? rho : 0));
        S.p[rb][0] = v.x; S.p[rb][1] = v.y; S.p[rb][2] = v.z; S.p[rb][3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) S.p[rb][e] = (mm < me && rho + e < r) ? P[mm * r + rho + e] : 0.0f;
      }
    }
  };
  // the register set of step m into LDS stage buf: Q as loaded, P as the
  // three bf16 parts of each value
  auto stage = [&](int64_t m, const Set& S, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // (an integer mask, not a select, so that no branch waits for the load)
      const uint32_t mk = (!FAST || (m + 8 * u + qrow < me && jq < J)) ? 0xffffffffu : 0u;
      *reinterpret_cast<uint4*>(&qs[buf][(8 * u + qrow) * LQP + 8 * qch]) =
          make_uint4(S.q[u].x & mk, S.q[u].y & mk, S.q[u].z & mk, S.q[u].w & mk);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bool ok = !FAST || (m + prow < me && rho0 + 32 * rb + prho < r);
      uint16_t h[3][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = ok ? S.p[rb][e] : 0.0f;
        const __bf16 a1 = (__bf16)v;
        const float r1 = v - (float)a1;
        const __bf16 a2 = (__bf16)r1;
        const __bf16 a3 = (__bf16)(r1 - (float)a2);
        h[0][e] = __builtin_bit_cast(uint16_t, a1);
        h[1][e] = __builtin_bit_cast(uint16_t, a2);
        h[2][e] = __builtin_bit_cast(uint16_t, a3);
      }
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
        *reinterpret_cast<uint2*>(&pls[buf][rb][pp][prow * LPP + prho]) =
            make_uint2(h[pp][0] | ((uint32_t)h[pp][1] << 16), h[pp][2] | ((uint32_t)h[pp][3] << 16));
    }
  };
  f32x16 acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) acc[rb][0] = acc[rb][1] = f32x16{};
  auto multiply = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x4l v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          v[h] = lds_tr16(&qs[buf][(16 * s2 + 8 * kg + 4 * h + (i16 >> 2)) * LQP + 64 * wave + 32 * t + 16 * hs +
                                   4 * (i16 & 3)]);
        b[t] = bf16x8{v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        bf16x8 a[3];
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) {
          bf16x4l v[2];
#pragma unroll
          for (int h = 0; h < 2; ++h)
            v[h] = lds_tr16(
                &pls[buf][rb][pp][(16 * s2 + 8 * kg + 4 * h + (i16 >> 2)) * LPP + 16 * hs + 4 * (i16 & 3)]);
          a[pp] = bf16x8{v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          acc[rb][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[t], acc[rb][t], 0, 0, 0);
          acc[rb][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[t], acc[rb][t], 0, 0, 0);
          acc[rb][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[t], acc[rb][t], 0, 0, 0);
        }
      }
    }
  };
  // Step i of the chunk (tokens mb + 32 i ..) stages set i % D into LDS stage
  // i % 2, then refills that set with step i + D while it multiplies. Every
  // load is unconditional (loads of steps past the chunk read clamped rows
  // that are never staged, or zeros), so the wait before each stage counts
  // exactly the later sets' loads.
  // (scheduling barriers keep the sets' loads in step order: the wait before
  // set d's stage counts the loads issued after it)
  Set S[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load(mb + 32 * d, S[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
  auto step = [&](int64_t mm, Set& St) __attribute__((always_inline)) {
    // (nothing is scheduled across step boundaries: staging a later set's
    // registers early would wait for its loads)
    __builtin_amdgcn_sched_barrier(0);
    const int buf = (int)(((mm - mb) >> 5) & 1);
    stage(mm, St, buf);
    __syncthreads();
    load(mm + 32 * D, St);
    multiply(buf);
  };
  // whole rounds of D steps (a loop without early exits, so that the wait
  // counts hold on its back edge), then the last nsteps % D steps
  const int64_t nsteps = mb < me ? (me - mb + 31) / 32 : 0, rounds = nsteps / D;
  int64_t m = mb;
  for (int64_t i = 0; i < rounds; ++i, m += 32 * D) {
#pragma unroll
    for (int d = 0; d < D; ++d) step(m + 32 * d, S[d]);
  }
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    if (d >= nsteps - rounds * D) break;
    step(m + 32 * d, S[d]);
  }
  // element e of accumulator (rb, t): rank rho0 + 32 rb + 8 (e / 4) + 4 (lane / 32) + e % 4, column
  // 64 wave + 32 t + lane % 32
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t j = j0 + 64 * wave + 32 * t + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rho = rho0 + 32 * rb + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (rho < r && j < J) partial[(c * r + rho) * J + j] = acc[rb][t][e];
      }
    }
}

// Stage 2 of one or two reductions: out = s * (sum of the chunks in order), in
// [J][r] (transpose_out) or [r][J] layout. Threads [0, r J0) take problem 0,
// the next r J1 problem 1.
struct LoraSum {
  const float* partial;
  int64_t chunks;
  int64_t J;
  bool transpose_out;
  float* out;
};

__global__ __launch_bounds__(256) void k_lora_combine(LoraSum q0, LoraSum q1, int r, float s) {
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool second = idx >= (int64_t)r * q0.J;
  if (second) idx -= (int64_t)r * q0.J;
  const LoraSum& q = second ? q1 : q0;
  const float* __restrict__ partial = q.partial;
  const int64_t chunks = q.chunks, J = q.J;
  const bool transpose_out = q.transpose_out;
  float* __restrict__ out = q.out;
  if (idx >= (int64_t)r * J) return;
  const int64_t rho = idx / J, j = idx % J;
  const float* p = partial + rho * J + j;
  const int64_t cs = (int64_t)r * J;  // stride between chunks
  float sum = 0.0f;
  // sixteen chunks' loads in flight (a shorter last group is predicated, not
  // a chain of dependent loads); the sum stays in chunk order
  for (int64_t c = 0; c < chunks; c += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = c + u < chunks ? p[(c + u) * cs] : 0.0f;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (c + u < chunks) sum += v[u];
  }
  const float v = s * sum;
  if (transpose_out)
    out[j * r + rho] = v;
  else
    out[rho * J + j] = v;
}

// The side product takes the split skinny GEMM (k_side_wide, then k_side_sum
// over the parts) for ranks beyond 32; for ranks up to 32 when k_side_bf16
// (16 rows per workgroup) would leave most of the chip idle, fewer than 256
// workgroups over a reduction of at least 2048 (a 512-token step through a
// 4096-wide layer: 32 workgroups of k_side_bf16); and for reductions of 8192
// or more, where k_side_bf16's workgroups would each read the whole fp32
// factor (twice the activation bytes for a 14336-long reduction at r = 16)
// while k_side_wide reads it once per 128 rows.
bool side_split_path(int64_t M, int64_t I, int32_t r) {
  return r > 32 || I >= 8192 || (ceil_div(M, SR) < 256 && I >= 2048);
}

// Split of the wide side product's reduction: about 512 workgroups of 128
// rows x 64 ranks, at least 4 steps of 32 per split.
struct SideSplit {
  int64_t splits;
  int64_t kc;  // reduction indices per split, a multiple of 32
};
SideSplit side_split_plan(int64_t M, int64_t I, int32_t r) {
  const int64_t tiles = ceil_div(M, 128) * ceil_div((int64_t)r, 64), steps = ceil_div(I, 32);
  int64_t ks = ceil_div(512, tiles);
  const int64_t maxks = steps / 4 > 1 ? steps / 4 : 1;
  if (ks > maxks) ks = maxks;
  const int64_t kc = ceil_div(steps, ks) * 32;
  return {ceil_div(I, kc), kc};
}

// Split of the streamed side product (k_side_tile): about 512 workgroups of 128
// rows x 16 ranks, at least 4 steps of 64 per split. It takes reductions of
// 8192 or more at ranks up to 16 (23 us against 30 us for k_side_wide, which
// always multiplies 64 ranks, on a 4096 x 14336 input); shorter reductions
// stay on k_side_bf16 (one launch, no partial sums: 14 us against 10 us + the
// 4.6 us sum at 4096 x 4096), larger ranks on k_side_wide.
bool side_tile_shape(int64_t I, int32_t r) { return I % 8 == 0 && r % 4 == 0 && r <= 16 && I >= 8192; }
SideSplit side_tile_plan(int64_t M, int64_t I, int32_t r) {
  (void)r;
  const int64_t tiles = ceil_div(M, 128), steps = ceil_div(I, 64);
  int64_t ks = ceil_div(512, tiles);
  const int64_t maxks = steps / 4 > 1 ? steps / 4 : 1;
  if (ks > maxks) ks = maxks;
  const int64_t kc = ceil_div(steps, ks) * 64;
  return {ceil_div(I, kc), kc};
}

// sum of the parts of a split side product, in split order
void launch_side_sum(const float* part, int64_t splits, int64_t n, float* out, hipStream_t st) {
  if (n % 4 == 0 && aligned(out, 16) && aligned(part, 16))
    hipLaunchKernelGGL(k_side_sum<true>, dim3((unsigned)ceil_div(n / 4, 256)), dim3(256), 0, st, part, n, (int)splits,
                       out);
  else
    hipLaunchKernelGGL(k_side_sum<false>, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, part, n, (int)splits,
                       out);
}

// Adapter side product (T = x A^T or U = dY B), needed by the main kernel's epilogue.
template <typename T>
void launch_side(const LinearArgs& g, hipStream_t st) {
  if (g.r <= 0) return;
  const int64_t I = g.backward ? g.N : g.K;
  const T* a = static_cast<const T*>(g.a);
  const dim3 sg((unsigned)ceil_div(g.M, SR));
  if constexpr (sizeof(T) == 2) {
    const float* fac = g.backward ? g.B : g.A;
    if (side_tile_shape(I, g.r) && aligned(a, 16) && aligned(fac, 16)) {
      const SideSplit sp = side_tile_plan(g.M, I, g.r);
      const dim3 grid((unsigned)ceil_div(g.M, 128), (unsigned)sp.splits, 1);
      float* dst = sp.splits > 1 ? g.side_part : g.side;
      const int64_t stride = g.M * (int64_t)g.r;
      if (g.backward)
        hipLaunchKernelGGL((k_side_tile<true, 1>), grid, dim3(256), 0, st, a, g.M, I, fac, g.r, sp.kc, dst, stride);
      else
        hipLaunchKernelGGL((k_side_tile<false, 1>), grid, dim3(256), 0, st, a, g.M, I, fac, g.r, sp.kc, dst, stride);
      if (sp.splits > 1) launch_side_sum(g.side_part, sp.splits, stride, g.side, st);
      return;
    }
    if (side_split_path(g.M, I, g.r)) {
      const SideSplit sp = side_split_plan(g.M, I, g.r);
      const dim3 grid((unsigned)ceil_div(g.M, 128), (unsigned)sp.splits, (unsigned)ceil_div((int64_t)g.r, 64));
      float* dst = sp.splits > 1 ? g.side_part : g.side;
      const int64_t stride = g.M * (int64_t)g.r;
      const bool fast = I % 8 == 0 && g.r % 8 == 0 && aligned(a, 16) && aligned(fac, 16);
#define NF4_WIDE(BWD, FAST) \
  hipLaunchKernelGGL((k_side_wide<BWD, FAST>), grid, dim3(256), 0, st, a, g.M, I, fac, g.r, sp.kc, dst, stride)
      if (g.backward && fast) NF4_WIDE(true, true);
      else if (g.backward) NF4_WIDE(true, false);
      else if (fast) NF4_WIDE(false, true);
      else NF4_WIDE(false, false);
#undef NF4_WIDE
      if (sp.splits > 1) launch_side_sum(g.side_part, sp.splits, stride, g.side, st);
      return;
    }
#define NF4_SIDE(BWD, RT) \
  hipLaunchKernelGGL((k_side_bf16<BWD, RT>), sg, dim3(1024), 0, st, a, g.M, I, fac, g.r, 0, g.side)
    if (g.backward) {
      if (g.r <= 16) NF4_SIDE(true, 1);
      else NF4_SIDE(true, 2);
    } else {
      if (g.r <= 16) NF4_SIDE(false, 1);
      else NF4_SIDE(false, 2);
    }
#undef NF4_SIDE
    return;
  }
  if (g.backward)
    hipLaunchKernelGGL((k_side<T, true>), sg, dim3(1024), 0, st, a, g.M, I, g.B, g.r, g.side);
  else
    hipLaunchKernelGGL((k_side<T, false>), sg, dim3(1024), 0, st, a, g.M, I, g.A, g.r, g.side);
}

template <typename T>
int run_linear_general(const LinearArgs& g, hipStream_t st) {
  const NF4View w = make_view(g.W);
  const int64_t J = g.backward ? g.K : g.N;
  const T* a = static_cast<const T*>(g.a);
  launch_side<T>(g, st);
  const dim3 grid((unsigned)ceil_div(J, GT), (unsigned)ceil_div(g.M, GT));
  T* out = static_cast<T*>(g.out);
#define NF4_GEN(BWD, DQ)                                                                                            \
  hipLaunchKernelGGL((k_linear_general<T, BWD, DQ>), grid, dim3(256), 0, st, a, g.M, g.K, g.N, w, g.A, g.B, g.r, \
                     g.s, g.side, out)
  const bool dq = g.W->double_quant != 0;
  if (g.backward && dq) NF4_GEN(true, true);
  else if (g.backward) NF4_GEN(true, false);
  else if (dq) NF4_GEN(false, true);
  else NF4_GEN(false, false);
#undef NF4_GEN
  return launch_status();
}

}  // namespace

int64_t side_split_ws_bytes(int64_t M, int64_t I, int32_t r) {
  if (r <= 0) return 0;
  // the larger of the two plans (which one runs also depends on the arrays' alignment)
  int64_t splits = 1;
  if (side_tile_shape(I, r)) splits = side_tile_plan(M, I, r).splits;
  if (side_split_path(M, I, r)) {
    const int64_t s2 = side_split_plan(M, I, r).splits;
    if (s2 > splits) splits = s2;
  }
  return splits > 1 ? (int64_t)round_up(sizeof(float) * (size_t)(splits * M * r), 256) : 0;
}

int launch_side_product(const void* L, nf4_dtype dt, int64_t M, int64_t I, const float* fac, int32_t r, bool backward,
                        float* out, float* part, hipStream_t st) {
  // A LinearArgs that carries only what launch_side reads.
  LinearArgs g{};
  g.a = L;
  g.dtype = dt;
  g.M = M;
  g.K = backward ? 1 : I;
  g.N = backward ? I : 1;
  g.A = backward ? nullptr : fac;
  g.B = backward ? fac : nullptr;
  g.r = r;
  g.side = out;
  g.side_part = part;
  g.backward = backward;
  if (dt == NF4_BF16)
    launch_side<__bf16>(g, st);
  else
    launch_side<float>(g, st);
  return launch_status();
}

int launch_linear(const LinearArgs& g, hipStream_t st) {
  if (g.dtype == NF4_BF16) {
    if (fast_linear_applies(g)) {
      launch_side<__bf16>(g, st);
      return launch_linear_fast(g, st);
    }
    return run_linear_general<__bf16>(g, st);
  }
  return run_linear_general<float>(g, st);
}

// Forward of n projections that read the same activations: their side
// products, then one launch set of the matrix kernel over all their output
// tiles when group_gemm_applies, else each projection as its own call.
int launch_linear_group(const LinearArgs* g, int n, hipStream_t st) {
  if (!group_gemm_applies(g, n)) {
    for (int i = 0; i < n; ++i)
      if (int rc = launch_linear(g[i], st)) return rc;
    return NF4_OK;
  }
  // The side products: one launch over the activation for all of them when
  // each adapter (rank 1 to 16) would take k_side_bf16 alone; else one each.
  bool one = n <= 4;
  for (int i = 0; i < n && one; ++i)
    one = g[i].r >= 1 && g[i].r <= 16 && !side_tile_shape(g[i].K, g[i].r) && !side_split_path(g[i].M, g[i].K, g[i].r);
  if (one) {
    SideGroup sgp{};
    for (int i = 0; i < n; ++i) {
      sgp.fac[i] = g[i].A;
      sgp.out[i] = g[i].side;
      sgp.r[i] = g[i].r;
    }
    const __bf16* x = static_cast<const __bf16*>(g[0].a);
    const dim3 grid((unsigned)ceil_div(g[0].M, SR), (unsigned)n);
    hipLaunchKernelGGL((k_side_bf16<false, 1, true>), grid, dim3(1024), 0, st, x, g[0].M, g[0].K, g[0].A, g[0].r, 0,
                       g[0].side, sgp);
  } else {
    for (int i = 0; i < n; ++i) launch_side<__bf16>(g[i], st);
  }
  return launch_linear_fast_group(g, n, st);
}

bool linear_bwd_sum_one_launch(const LinearArgs* g, int n) { return group_sum_applies(g, n); }

// Summed input gradient dX = sum_i (dY_i W_i + s_i U_i A_i) of n projections
// of one activation: their side products U_i, then one launch set of the
// matrix kernel whose reduction runs over every projection in turn; otherwise
// projection 0's call into dX and each other's into tmp, added in projection
// order (each part rounded to the output type first).
int launch_linear_bwd_sum(const LinearArgs* g, int n, void* tmp, hipStream_t st) {
  if (group_sum_applies(g, n)) {
    for (int i = 0; i < n; ++i) launch_side<__bf16>(g[i], st);
    return launch_linear_fast_sum(g, n, st);
  }
  const size_t esz = g[0].dtype == NF4_BF16 ? 2 : 4;
  const int64_t MK = g[0].M * g[0].K;
  if (int rc = launch_linear(g[0], st)) return rc;
  for (int i = 1; i < n; ++i) {
    LinearArgs q = g[i];
    q.out = static_cast<char*>(tmp) + (size_t)(i - 1) * esz * (size_t)MK;
    if (int rc = launch_linear(q, st)) return rc;
  }
  char* t = static_cast<char*>(tmp);
  for (int i = 1; i < n; i += 2) {
    const void* c = i + 1 < n ? t + (size_t)i * esz * (size_t)MK : nullptr;
    if (int rc = launch_add3(g[0].out, t + (size_t)(i - 1) * esz * (size_t)MK, c, g[0].dtype, MK, g[0].out, st))
      return rc;
  }
  return launch_status();
}

// Tokens per chunk of the bf16 MFMA reduction (a multiple of the 32-token
// step), for about 512 workgroups of 256 columns (two per CU):
//  - with dA, both reductions take 512 / (tiles(K) + tiles(N)) chunks, so every
//    workgroup walks the same number of steps and the fp32 partial sums (written
//    and read again by the combine) are as few as that parallelism allows;
//  - LoRA-FA (dB alone) takes 512 / tiles(N) chunks.
// Fewer, longer chunks than the general path keep the partial sums small next
// to the input.
int64_t lora_chunk_steps(int64_t M, int64_t tiles) {
  int64_t chunks = 512 / tiles;
  const int64_t steps = ceil_div(M, 32);
  if (chunks > steps) chunks = steps;
  if (chunks < 1) chunks = 1;
  return ceil_div(ceil_div(M, chunks), 32) * 32;
}
int64_t lora_chunk_mfma_b(int64_t M, int64_t N) { return lora_chunk_steps(M, ceil_div(N, 256)); }
int64_t lora_chunk_mfma_a(int64_t M, int64_t K, int64_t N) {
  return lora_chunk_steps(M, ceil_div(K, 256) + ceil_div(N, 256));
}

// Chunks of either path (the query does not know the dtype, so the workspace
// covers the larger).
int64_t lora_chunks_max(int64_t M, int64_t J, int64_t mfma_chunk) {
  const int64_t a = ceil_div(M, lora_chunk(M, J)), b = ceil_div(M, mfma_chunk);
  return a > b ? a : b;
}

size_t lora_grad_ws(int64_t M, int64_t K, int64_t N, int32_t r, int fa) {
  const int64_t chB = lora_chunks_max(M, N, lora_chunk_mfma_b(M, N));
  const int64_t chA = lora_chunks_max(M, K, lora_chunk_mfma_a(M, K, N));
  size_t bytes = round_up(sizeof(float) * (size_t)(chB * r * N), 256);
  if (!fa) bytes += round_up(sizeof(float) * (size_t)(chA * r * K), 256);
  return bytes;
}

namespace {
// partial[c][rho][j] for P [M, r] and Q [M, J], then the ordered chunk sum.
template <typename T>
void lora_side(const float* P, const T* Q, int64_t M, int64_t J, int32_t r, float s, bool transpose_out, float* part,
               float* out, hipStream_t st) {
  const int64_t chunk = lora_chunk(M, J), chunks = ceil_div(M, chunk);
  const dim3 grid((unsigned)ceil_div(J, LCOLS), (unsigned)chunks);
  if (J % 2 == 0 && J >= 2)
    hipLaunchKernelGGL((k_lora_partial<T, true>), grid, dim3(256), 0, st, P, Q, M, J, r, chunk, part);
  else
    hipLaunchKernelGGL((k_lora_partial<T, false>), grid, dim3(256), 0, st, P, Q, M, J, r, chunk, part);
  const LoraSum q{part, chunks, J, transpose_out, out};
  hipLaunchKernelGGL(k_lora_combine, dim3((unsigned)ceil_div((int64_t)r * J, 256)), dim3(256), 0, st, q, q, r, s);
}

// bf16 activations: dB's reduction (P = T, Q = dY) and, unless LoRA-FA, dA's
// (P = U, Q = x) in one MFMA launch per 128 ranks and one combine launch.
void lora_grad_mfma(const __bf16* x, const __bf16* dy, int64_t M, int64_t K, int64_t N, const float* t,
                    const float* u, int32_t r, float s, float* dA, float* dB, float* partA, float* partB,
                    hipStream_t st) {
  const int64_t chA = lora_chunk_mfma_a(M, K, N), chB = dA ? chA : lora_chunk_mfma_b(M, N);
  const LoraProb pb{t, dy, N, chB, ceil_div(N, 256), partB};
  const LoraProb pa{u, x, K, chA, ceil_div(K, 256), partA};
  const int64_t blocksB = pb.col_tiles * ceil_div(M, chB);
  const int64_t blocksA = dA ? pa.col_tiles * ceil_div(M, chA) : 0;
  // dA's (longer) workgroups first; 32, 64 or 128 ranks per launch (further
  // launches for the ranks past 128)
  const LoraProb& p0 = dA ? pa : pb;
  const int64_t blocks0 = dA ? blocksA : blocksB;
  const bool fast = N % 8 == 0 && r % 4 == 0 && aligned(dy, 16) && aligned(t, 16) &&
                    (!dA || (K % 8 == 0 && aligned(x, 16) && aligned(u, 16)));
  for (int r0 = 0; r0 < r; r0 += 128) {
    const int left = r - r0;
    const dim3 grid((unsigned)(blocksB + blocksA));
#define NF4_LORA(RB, FAST) hipLaunchKernelGGL((k_lora_mfma<RB, FAST>), grid, dim3(256), 0, st, p0, pb, blocks0, M, r, r0)
    if (left <= 32) {
      if (fast) NF4_LORA(1, true); else NF4_LORA(1, false);
    } else if (left <= 64) {
      if (fast) NF4_LORA(2, true); else NF4_LORA(2, false);
    } else {
      if (fast) NF4_LORA(4, true); else NF4_LORA(4, false);
    }
#undef NF4_LORA
  }
  const LoraSum qb{partB, ceil_div(M, chB), N, true, dB};
  const LoraSum qa{partA, ceil_div(M, chA), K, false, dA};
  const int64_t outs = (int64_t)r * N + (dA ? (int64_t)r * K : 0);
  hipLaunchKernelGGL(k_lora_combine, dim3((unsigned)ceil_div(outs, 256)), dim3(256), 0, st, qb, dA ? qa : qb, r, s);
}
}  // namespace

int launch_lora_grad(const void* x, const void* dy, nf4_dtype dt, int64_t M, int64_t K, int64_t N, const float* t,
                     const float* u, int32_t r, float s, float* dA, float* dB, void* ws, hipStream_t st) {
  const int64_t chunksB = lora_chunks_max(M, N, lora_chunk_mfma_b(M, N));
  float* partB = static_cast<float*>(ws);
  float* partA =
      reinterpret_cast<float*>(static_cast<char*>(ws) + round_up(sizeof(float) * (size_t)(chunksB * r * N), 256));
  if (dt == NF4_BF16) {
    lora_grad_mfma(static_cast<const __bf16*>(x), static_cast<const __bf16*>(dy), M, K, N, t, u, r, s, dA, dB, partA,
                   partB, st);
    return launch_status();
  }
  // dB[n][rho] = s * sum_m dY[m][n] T[m][rho]  ([N][r] layout)
  if (dt == NF4_BF16)
    lora_side<__bf16>(t, static_cast<const __bf16*>(dy), M, N, r, s, true, partB, dB, st);
  else
    lora_side<float>(t, static_cast<const float*>(dy), M, N, r, s, true, partB, dB, st);
  // dA[rho][k] = s * sum_m U[m][rho] x[m][k]  ([r][K] layout); skipped for LoRA-FA
  if (dA) {
    if (dt == NF4_BF16)
      lora_side<__bf16>(u, static_cast<const __bf16*>(x), M, K, r, s, false, partA, dA, st);
    else
      lora_side<float>(u, static_cast<const float*>(x), M, K, r, s, false, partA, dA, st);
  }
  return launch_status();
}

}  // namespace nf4

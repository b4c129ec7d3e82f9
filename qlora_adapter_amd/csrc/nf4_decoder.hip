// The operations around the NF4 linears in a Llama-shaped decoder layer, on
// gfx950: residual add + RMSNorm, rotary embedding, causal grouped-query
// attention, the SwiGLU gate and the token cross-entropy, each with its input
// gradient. Activations are bf16 (or fp32) rows, tokens first; all arithmetic
// is fp32.
//
// Definitions (the standard Llama ones; the pages name the model and its
// checkpointed training step without printing the layer's equations):
//  - RMSNorm: y = x / sqrt(mean(x^2) + eps) * gamma, gamma frozen.
//  - Rotary embedding, half-split pairs: for i < d/2 the pair
//    (x_i, x_{i+d/2}) is rotated by pos * theta^(-2 i / d).
//  - Attention: softmax(q k^T / sqrt(d), causal) v; query head h reads
//    key/value head h / (Hq / Hkv).
//  - SwiGLU: a = silu(g) * u.
//  - Cross-entropy: mean over tokens of logsumexp(z) - z[target].
//
// Kernels
//  k_add_rmsnorm   one workgroup per token row: optional residual add, the
//                  sum of squares in fp32 (wave shuffles, then LDS), the scaled
//                  row; saves rstd.
//  k_rmsnorm_bwd   one workgroup per row: dx = rstd (g - n mean(g n)) with
//                  g = dy gamma, n = x rstd, plus an optional residual
//                  gradient.
//  k_rope          one workgroup per token: the row's d/2 angles in fp64,
//                  cos/sin rounded to fp32, applied to every head in place,
//                  16 bytes of each half head per access where aligned.
//  Attention in bf16 with a head dim that is a multiple of 32 (up to 128)
//  runs on the matrix cores (nf4_attention.hip); the kernels below serve fp32
//  and the other head dims.
//  k_attn_fwd      workgroup = (head, 16 query rows); 16 threads per row.
//                  Keys and values pass through LDS in blocks of 64 with an
//                  online softmax; writes O and the row log-sum-exp.
//  k_attn_dq       same tiling: recomputes P from the log-sum-exp, writes
//                  delta = rowsum(dO * O) and dQ = scale * sum_j dS_ij k_j.
//  k_attn_dkv      workgroup = (key/value head, 16 key rows): loops over the
//                  query heads of the group and the query blocks at or after
//                  the keys; dV = sum_i P_ij dO_i, dK = scale sum_i dS_ij q_i.
//                  No atomics: every output row has one owner.
//  k_swiglu / k_swiglu_bwd / k_add3   elementwise.
//  bf16 rows with a width that is a multiple of 8 use vectorized forms
//  (k_add_rmsnorm_v, k_rmsnorm_bwd_v: the row in registers between the two
//  phases; k_xent_v: one pass for max and sum).
//  k_xent          one workgroup per token: max, sum of exponentials, the
//                  token loss, and the logit gradient (softmax - onehot) / T;
//                  k_xent_mean adds the token losses in index order.
#include <cmath>

#include "nf4_internal.hpp"

namespace nf4 {
namespace {

template <typename T>
__device__ __forceinline__ float ldf(const T* p, int64_t i) {
  return (float)p[i];
}
template <typename T>
__device__ __forceinline__ void stf(T* p, int64_t i, float v) {
  p[i] = (T)v;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Sum over the 256 threads of a workgroup, the same value returned to all.
__device__ __forceinline__ float block_sum256(float v, float* sh) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[wave] = v;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

__device__ __forceinline__ float block_max256(float v, float* sh) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

// ---------------------------------------------------------------- RMSNorm

template <typename T>
__global__ __launch_bounds__(256) void k_add_rmsnorm(const T* __restrict__ x, const T* __restrict__ res, int64_t D,
                                                     const float* __restrict__ gamma, float eps, T* __restrict__ sum,
                                                     T* __restrict__ y, float* __restrict__ rstd) {
  __shared__ float sh[4];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * D;
  float ss = 0.0f;
  for (int64_t i = threadIdx.x; i < D; i += 256) {
    float v = ldf(xr, i);
    if (res) {
      // the sum is stored in the activation type and normalized as stored
      v = (float)(T)(v + ldf(res + row * D, i));
      stf(sum + row * D, i, v);
    }
    ss += v * v;
  }
  const float r = 1.0f / sqrtf(block_sum256(ss, sh) / (float)D + eps);
  const T* src = res ? sum + row * D : xr;
  for (int64_t i = threadIdx.x; i < D; i += 256) stf(y + row * D, i, ldf(src, i) * r * gamma[i]);
  if (threadIdx.x == 0) rstd[row] = r;
}

template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const T* __restrict__ dy, const T* __restrict__ x,
                                                     const float* __restrict__ rstd, int64_t D,
                                                     const float* __restrict__ gamma, const T* __restrict__ dres,
                                                     T* __restrict__ dx) {
  __shared__ float sh[4];
  const int64_t row = blockIdx.x;
  const float r = rstd[row];
  float acc = 0.0f;
  for (int64_t i = threadIdx.x; i < D; i += 256) acc += ldf(dy + row * D, i) * gamma[i] * (ldf(x + row * D, i) * r);
  const float mgn = block_sum256(acc, sh) / (float)D;
  for (int64_t i = threadIdx.x; i < D; i += 256) {
    const float g = ldf(dy + row * D, i) * gamma[i];
    float v = r * (g - ldf(x + row * D, i) * r * mgn);
    if (dres) v += ldf(dres + row * D, i);
    stf(dx + row * D, i, v);
  }
}

// bf16 rows of width D % 8 == 0, D <= 2048 CPT: each thread keeps its CPT
// 8-element chunks (chunk c = thread + 256 j) in registers between the sum of
// squares and the scaling, with 16-byte loads and stores. Same arithmetic as
// the general kernels; only the order of the per-thread partial sums differs.
typedef __bf16 bf16x8d __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void load_gamma8(const float* __restrict__ gamma, int64_t i, float g[8]) {
  const float4 a = *reinterpret_cast<const float4*>(gamma + i);
  const float4 b = *reinterpret_cast<const float4*>(gamma + i + 4);
  g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w; g[4] = b.x; g[5] = b.y; g[6] = b.z; g[7] = b.w;
}

template <int CPT>
__global__ __launch_bounds__(256) void k_add_rmsnorm_v(const __bf16* __restrict__ x, const __bf16* __restrict__ res,
                                                       int64_t D, const float* __restrict__ gamma, float eps,
                                                       __bf16* __restrict__ sum, __bf16* __restrict__ y,
                                                       float* __restrict__ rstd) {
  __shared__ float sh[4];
  const int64_t row = blockIdx.x, nch = D / 8;
  float v[CPT][8];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t c = threadIdx.x + 256 * j;
    if (c >= nch) break;
    const bf16x8d xv = *reinterpret_cast<const bf16x8d*>(x + row * D + 8 * c);
    if (res) {
      const bf16x8d rv = *reinterpret_cast<const bf16x8d*>(res + row * D + 8 * c);
      bf16x8d sv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sv[e] = (__bf16)((float)xv[e] + (float)rv[e]);  // stored in bf16, normalized as stored
        v[j][e] = (float)sv[e];
      }
      *reinterpret_cast<bf16x8d*>(sum + row * D + 8 * c) = sv;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = (float)xv[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[j][e] * v[j][e];
  }
  const float r = 1.0f / sqrtf(block_sum256(ss, sh) / (float)D + eps);
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t c = threadIdx.x + 256 * j;
    if (c >= nch) break;
    float g[8];
    load_gamma8(gamma, 8 * c, g);
    bf16x8d o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)(v[j][e] * r * g[e]);
    *reinterpret_cast<bf16x8d*>(y + row * D + 8 * c) = o;
  }
  if (threadIdx.x == 0) rstd[row] = r;
}

template <int CPT>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd_v(const __bf16* __restrict__ dy, const __bf16* __restrict__ x,
                                                       const float* __restrict__ rstd, int64_t D,
                                                       const float* __restrict__ gamma,
                                                       const __bf16* __restrict__ dres, __bf16* __restrict__ dx) {
  __shared__ float sh[4];
  const int64_t row = blockIdx.x, nch = D / 8;
  const float r = rstd[row];
  float gv[CPT][8], xv[CPT][8];
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t c = threadIdx.x + 256 * j;
    if (c >= nch) break;
    const bf16x8d a = *reinterpret_cast<const bf16x8d*>(dy + row * D + 8 * c);
    const bf16x8d b = *reinterpret_cast<const bf16x8d*>(x + row * D + 8 * c);
    float g[8];
    load_gamma8(gamma, 8 * c, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gv[j][e] = (float)a[e] * g[e];
      xv[j][e] = (float)b[e];
      acc += gv[j][e] * (xv[j][e] * r);
    }
  }
  const float mgn = block_sum256(acc, sh) / (float)D;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t c = threadIdx.x + 256 * j;
    if (c >= nch) break;
    bf16x8d o;
    if (dres) {
      const bf16x8d d = *reinterpret_cast<const bf16x8d*>(dres + row * D + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)(r * (gv[j][e] - xv[j][e] * r * mgn) + (float)d[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (__bf16)(r * (gv[j][e] - xv[j][e] * r * mgn));
    }
    *reinterpret_cast<bf16x8d*>(dx + row * D + 8 * c) = o;
  }
}

// ---------------------------------------------------------------- rotary embedding


// ---------------------------------------------------------------- attention

constexpr int AQ = 16;    // query (or key) rows per workgroup
constexpr int AKB = 64;   // key (or query) rows per LDS block
constexpr int ADMAX = 128;

// Loads rows [r0, r0 + n) of head hd of a [S, ld] activation into s[n][d] (fp32), zero past S.
template <typename T>
__device__ __forceinline__ void load_rows(float* s, const T* src, int64_t ld, int64_t r0, int n, int64_t S, int hd,
                                          int d) {
  for (int e = threadIdx.x; e < n * d; e += 256) {
    const int rr = e / d, c = e - rr * d;
    const int64_t row = r0 + rr;
    s[rr * d + c] = row < S ? ldf(src, row * ld + (int64_t)hd * d + c) : 0.0f;
  }
}

// O and the row log-sum-exp for 16 query rows of one head. Thread t: row
// t / 16, lane c = t % 16 of the row; scores for keys c, c+16, c+32, c+48 of a
// block, outputs for dims c, c+16, ... (d / 16 of them).
template <typename T>
__global__ __launch_bounds__(256) void k_attn_fwd(const T* __restrict__ q, const T* __restrict__ k,
                                                  const T* __restrict__ v, int64_t S, int hq, int hkv, int d,
                                                  int64_t lq, int64_t lk, float scale, T* __restrict__ o,
                                                  float* __restrict__ lse) {
  __shared__ float qs[AQ * ADMAX];
  __shared__ float ks[AKB * ADMAX];
  __shared__ float vs[AKB * ADMAX];
  __shared__ float ps[AQ][AKB];
  const int h = blockIdx.y, kh = h / (hq / hkv);
  const int64_t q0 = (int64_t)blockIdx.x * AQ;
  const int t = threadIdx.x, r = t >> 4, c = t & 15;
  const int64_t qi = q0 + r;
  const int64_t ldq = lq, ldk = lk, ldo = (int64_t)hq * d;
  load_rows(qs, q, ldq, q0, AQ, S, h, d);
  float m = -INFINITY, l = 0.0f;
  float acc[ADMAX / 16];
#pragma unroll
  for (int j = 0; j < ADMAX / 16; ++j) acc[j] = 0.0f;
  const int nd = d / 16;
  const int64_t kend = (q0 + AQ < S ? q0 + AQ : S);  // keys past the last query row are masked everywhere
  for (int64_t k0 = 0; k0 < kend; k0 += AKB) {
    __syncthreads();
    load_rows(ks, k, ldk, k0, AKB, S, kh, d);
    load_rows(vs, v, ldk, k0, AKB, S, kh, d);
    __syncthreads();
    float s[4];
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kj = c + 16 * u;
      float dot = 0.0f;
      for (int e = 0; e < d; ++e) dot += qs[r * d + e] * ks[kj * d + e];
      s[u] = (k0 + kj <= qi && qi < S) ? dot * scale : -INFINITY;
      bm = fmaxf(bm, s[u]);
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) bm = fmaxf(bm, __shfl_xor(bm, off));
    const float mn = fmaxf(m, bm);
    const float alpha = (mn == -INFINITY) ? 1.0f : expf(m - mn);
    float bs = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float p = (s[u] == -INFINITY) ? 0.0f : expf(s[u] - mn);
      ps[r][c + 16 * u] = p;
      bs += p;
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) bs += __shfl_xor(bs, off);
    l = l * alpha + bs;
    m = mn;
    __syncthreads();
    for (int j = 0; j < nd; ++j) {
      float a = acc[j] * alpha;
      for (int kj = 0; kj < AKB; ++kj) a += ps[r][kj] * vs[kj * d + c + 16 * j];
      acc[j] = a;
    }
  }
  if (qi < S) {
    const float inv = 1.0f / l;
    for (int j = 0; j < nd; ++j) stf(o, qi * ldo + (int64_t)h * d + c + 16 * j, acc[j] * inv);
    if (c == 0) lse[(int64_t)h * S + qi] = m + logf(l);
  }
}

// dQ for 16 query rows of one head, and delta = rowsum(dO * O) for them.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_dq(const T* __restrict__ dout, const T* __restrict__ q,
                                                 const T* __restrict__ k, const T* __restrict__ v,
                                                 const T* __restrict__ o, const float* __restrict__ lse, int64_t S,
                                                 int hq, int hkv, int d, int64_t lq, int64_t lk, float scale,
                                                 float* __restrict__ delta, T* __restrict__ dq) {
  __shared__ float qs[AQ * ADMAX];
  __shared__ float dos[AQ * ADMAX];
  __shared__ float ks[AKB * ADMAX];
  __shared__ float vs[AKB * ADMAX];
  __shared__ float dss[AQ][AKB];
  const int h = blockIdx.y, kh = h / (hq / hkv);
  const int64_t q0 = (int64_t)blockIdx.x * AQ;
  const int t = threadIdx.x, r = t >> 4, c = t & 15;
  const int64_t qi = q0 + r;
  const int64_t ldq = lq, ldk = lk, ldo = (int64_t)hq * d;
  load_rows(qs, q, ldq, q0, AQ, S, h, d);
  load_rows(dos, dout, ldo, q0, AQ, S, h, d);
  const int nd = d / 16;
  // delta of this row (16 threads, d / 16 products each)
  float dl = 0.0f;
  for (int j = 0; j < nd; ++j) {
    const int e = c + 16 * j;
    dl += (qi < S) ? ldf(dout, qi * ldo + (int64_t)h * d + e) * ldf(o, qi * ldo + (int64_t)h * d + e) : 0.0f;
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) dl += __shfl_xor(dl, off);
  if (qi < S && c == 0) delta[(int64_t)h * S + qi] = dl;
  const float L = (qi < S) ? lse[(int64_t)h * S + qi] : 0.0f;
  float acc[ADMAX / 16];
#pragma unroll
  for (int j = 0; j < ADMAX / 16; ++j) acc[j] = 0.0f;
  const int64_t kend = (q0 + AQ < S ? q0 + AQ : S);
  for (int64_t k0 = 0; k0 < kend; k0 += AKB) {
    __syncthreads();
    load_rows(ks, k, ldk, k0, AKB, S, kh, d);
    load_rows(vs, v, ldk, k0, AKB, S, kh, d);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kj = c + 16 * u;
      float sd = 0.0f, pd = 0.0f;
      for (int e = 0; e < d; ++e) {
        sd += qs[r * d + e] * ks[kj * d + e];
        pd += dos[r * d + e] * vs[kj * d + e];
      }
      const bool ok = (k0 + kj <= qi) && qi < S;
      const float p = ok ? expf(sd * scale - L) : 0.0f;
      dss[r][kj] = p * (pd - dl);
    }
    __syncthreads();
    for (int j = 0; j < nd; ++j) {
      float a = acc[j];
      for (int kj = 0; kj < AKB; ++kj) a += dss[r][kj] * ks[kj * d + c + 16 * j];
      acc[j] = a;
    }
  }
  if (qi < S)
    for (int j = 0; j < nd; ++j) stf(dq, qi * ldq + (int64_t)h * d + c + 16 * j, acc[j] * scale);
}

// dK and dV for 16 key rows of one key/value head. Thread t: key row t / 16,
// lane c: queries c, c+16, c+32, c+48 of a block, output dims c, c+16, ...
template <typename T>
__global__ __launch_bounds__(256) void k_attn_dkv(const T* __restrict__ dout, const T* __restrict__ q,
                                                  const T* __restrict__ k, const T* __restrict__ v,
                                                  const float* __restrict__ lse, const float* __restrict__ delta,
                                                  int64_t S, int hq, int hkv, int d, int64_t lq, int64_t lk,
                                                  float scale, T* __restrict__ dk, T* __restrict__ dv) {
  __shared__ float ks[AQ * ADMAX];
  __shared__ float vs[AQ * ADMAX];
  __shared__ float qs[AKB * ADMAX];
  __shared__ float dos[AKB * ADMAX];
  __shared__ float pss[AQ][AKB];
  __shared__ float dss[AQ][AKB];
  __shared__ float ls[AKB], dls[AKB];
  const int kh = blockIdx.y, grp = hq / hkv;
  const int64_t k0 = (int64_t)blockIdx.x * AQ;
  const int t = threadIdx.x, r = t >> 4, c = t & 15;
  const int64_t kj = k0 + r;
  const int64_t ldq = lq, ldk = lk, ldo = (int64_t)hq * d;
  load_rows(ks, k, ldk, k0, AQ, S, kh, d);
  load_rows(vs, v, ldk, k0, AQ, S, kh, d);
  const int nd = d / 16;
  float adk[ADMAX / 16], adv[ADMAX / 16];
#pragma unroll
  for (int j = 0; j < ADMAX / 16; ++j) adk[j] = adv[j] = 0.0f;
  const int64_t qstart = k0 / AKB * AKB;  // first query block that can see these keys
  for (int hh = 0; hh < grp; ++hh) {
    const int h = kh * grp + hh;
    for (int64_t q0 = qstart; q0 < S; q0 += AKB) {
      __syncthreads();
      load_rows(qs, q, ldq, q0, AKB, S, h, d);
      load_rows(dos, dout, ldo, q0, AKB, S, h, d);
      for (int e = threadIdx.x; e < AKB; e += 256) {
        const int64_t qi = q0 + e;
        ls[e] = qi < S ? lse[(int64_t)h * S + qi] : 0.0f;
        dls[e] = qi < S ? delta[(int64_t)h * S + qi] : 0.0f;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int qq = c + 16 * u;
        const int64_t qi = q0 + qq;
        float sd = 0.0f, pd = 0.0f;
        for (int e = 0; e < d; ++e) {
          sd += qs[qq * d + e] * ks[r * d + e];
          pd += dos[qq * d + e] * vs[r * d + e];
        }
        const bool ok = (kj <= qi) && qi < S && kj < S;
        const float p = ok ? expf(sd * scale - ls[qq]) : 0.0f;
        pss[r][qq] = p;
        dss[r][qq] = p * (pd - dls[qq]);
      }
      __syncthreads();
      for (int j = 0; j < nd; ++j) {
        float a = adv[j], b = adk[j];
        for (int qq = 0; qq < AKB; ++qq) {
          a += pss[r][qq] * dos[qq * d + c + 16 * j];
          b += dss[r][qq] * qs[qq * d + c + 16 * j];
        }
        adv[j] = a;
        adk[j] = b;
      }
    }
  }
  if (kj < S)
    for (int j = 0; j < nd; ++j) {
      stf(dv, kj * ldk + (int64_t)kh * d + c + 16 * j, adv[j]);
      stf(dk, kj * ldk + (int64_t)kh * d + c + 16 * j, adk[j] * scale);
    }
}

// ---------------------------------------------------------------- sums

// out = a + b (+ c), fp32 sum rounded once to the activation type. No
// restrict qualifiers: out may alias an input (each entry is read, then
// written, by the same lane).
template <typename T>
__global__ __launch_bounds__(256) void k_add3(const T* a, const T* b, const T* c, int64_t n, T* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = ldf(a, i) + ldf(b, i);
  if (c) v += ldf(c, i);
  stf(out, i, v);
}

// ---------------------------------------------------------------- SwiGLU

// Rows of `width` entries; g, u (and dg, du) are rows ld apart, a and da dense.
// Thread t of workgroup (x, y) takes entries V (256 x + t) .. + V - 1 of rows
// y, y + gridDim.y, ...: V = 16 / sizeof(T) (one 16-byte access per array)
// when width, ld and the pointers allow it, else 1. The arithmetic per entry
// is the same either way.
template <typename T, int V>
struct Vec {
  T v[V];
};

template <typename T, int V>
__device__ __forceinline__ Vec<T, V> ldv(const T* p) {
  return *reinterpret_cast<const Vec<T, V>*>(p);
}

// Rotary embedding of one token per workgroup: its d/2 angles pos theta^(-2i/d)
// in fp64 (one sincos each), cos and sin rounded to fp32 in LDS, then every
// head rotated in place, V consecutive pairs per thread (one 16-byte access to
// each half of the head when d/2, ld and the row allow it, else V = 1).
template <typename T, int V>
__global__ __launch_bounds__(256) void k_rope(T* __restrict__ x, int64_t ld, int heads, int d, double theta,
                                              int inverse) {
  __shared__ float cs[2][256];
  const int64_t pos = blockIdx.x;
  const int h = d / 2;
  for (int i = threadIdx.x; i < h; i += 256) {
    const double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)d);
    double sn, cn;
    sincos(ang, &sn, &cn);
    cs[0][i] = (float)cn;
    cs[1][i] = (float)(inverse ? -sn : sn);
  }
  __syncthreads();
  T* row = x + pos * ld;
  const int hv = h / V;  // accesses per half head
  for (int e = threadIdx.x; e < heads * hv; e += 256) {
    const int hd = e / hv, i = (e - hd * hv) * V;
    T* p = row + (int64_t)hd * d + i;
    const Vec<T, V> a = ldv<T, V>(p), b = ldv<T, V>(p + h);
    Vec<T, V> ra, rb;
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const float af = (float)a.v[k], bf = (float)b.v[k], c = cs[0][i + k], sv = cs[1][i + k];
      ra.v[k] = (T)(af * c - bf * sv);
      rb.v[k] = (T)(bf * c + af * sv);
    }
    *reinterpret_cast<Vec<T, V>*>(p) = ra;
    *reinterpret_cast<Vec<T, V>*>(p + h) = rb;
  }
}

template <typename T, int V>
__global__ __launch_bounds__(256) void k_swiglu(const T* __restrict__ g, const T* __restrict__ u, int64_t rows,
                                                int64_t width, int64_t ld, T* __restrict__ a) {
  const int64_t j = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
  if (j >= width) return;
  for (int64_t m = blockIdx.y; m < rows; m += gridDim.y) {
    const Vec<T, V> gv = ldv<T, V>(g + m * ld + j), uv = ldv<T, V>(u + m * ld + j);
    Vec<T, V> av;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float z = (float)gv.v[e];
      av.v[e] = (T)(z / (1.0f + expf(-z)) * (float)uv.v[e]);
    }
    *reinterpret_cast<Vec<T, V>*>(a + m * width + j) = av;
  }
}

template <typename T, int V>
__global__ __launch_bounds__(256) void k_swiglu_bwd(const T* __restrict__ da, const T* __restrict__ g,
                                                    const T* __restrict__ u, int64_t rows, int64_t width, int64_t ld,
                                                    T* __restrict__ dg, T* __restrict__ du) {
  const int64_t j = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
  if (j >= width) return;
  for (int64_t m = blockIdx.y; m < rows; m += gridDim.y) {
    const int64_t e0 = m * ld + j;
    const Vec<T, V> gv = ldv<T, V>(g + e0), uv = ldv<T, V>(u + e0), dav = ldv<T, V>(da + m * width + j);
    Vec<T, V> dgv, duv;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float z = (float)gv.v[e], s = 1.0f / (1.0f + expf(-z)), d = (float)dav.v[e];
      dgv.v[e] = (T)(d * (float)uv.v[e] * s * (1.0f + z * (1.0f - s)));
      duv.v[e] = (T)(d * z * s);
    }
    *reinterpret_cast<Vec<T, V>*>(dg + e0) = dgv;
    *reinterpret_cast<Vec<T, V>*>(du + e0) = duv;
  }
}

// ---------------------------------------------------------------- cross-entropy

template <typename T>
__global__ __launch_bounds__(256) void k_xent(const T* __restrict__ z, const int64_t* __restrict__ target, int64_t V,
                                              float inv_tokens, float* __restrict__ tok_loss, T* __restrict__ dz,
                                              int32_t* __restrict__ status) {
  __shared__ float sh[4];
  const int64_t row = blockIdx.x;
  const T* zr = z + row * V;
  float mx = -INFINITY;
  for (int64_t i = threadIdx.x; i < V; i += 256) mx = fmaxf(mx, ldf(zr, i));
  mx = block_max256(mx, sh);
  float se = 0.0f;
  for (int64_t i = threadIdx.x; i < V; i += 256) se += expf(ldf(zr, i) - mx);
  se = block_sum256(se, sh);
  const float lse = mx + logf(se);
  const int64_t tg = target[row];
  const bool ok = tg >= 0 && tg < V;
  if (threadIdx.x == 0) {
    const float zt = ldf(zr, ok ? tg : 0);  // never indexes outside the row
    tok_loss[row] = ok ? lse - zt : 0.0f;
    if (!ok && status) *status = NF4_EINVAL;
  }
  if (dz)
    for (int64_t i = threadIdx.x; i < V; i += 256)
      stf(dz + row * V, i, (expf(ldf(zr, i) - lse) - (i == tg ? 1.0f : 0.0f)) * inv_tokens);
}

// bf16 logits with V % 8 == 0: one pass for the maximum and the sum of
// exponentials (each thread keeps a running (max, sum) pair, rescaled when its
// maximum grows; the pairs are merged across the workgroup), then one pass for
// the gradient; 16-byte loads and stores.
__global__ __launch_bounds__(256) void k_xent_v(const __bf16* __restrict__ z, const int64_t* __restrict__ target,
                                                int64_t V, float inv_tokens, float* __restrict__ tok_loss,
                                                __bf16* __restrict__ dz, int32_t* __restrict__ status) {
  __shared__ float shm[4], shs[4];
  const int64_t row = blockIdx.x, nch = V / 8;
  const __bf16* zr = z + row * V;
  float m = -INFINITY, se = 0.0f;
  for (int64_t c = threadIdx.x; c < nch; c += 256) {
    const bf16x8d v = *reinterpret_cast<const bf16x8d*>(zr + 8 * c);
    float cm = (float)v[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, (float)v[e]);
    if (cm > m) {
      se *= expf(m - cm);  // 0 while m is -inf
      m = cm;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) se += expf((float)v[e] - m);
  }
  // merge the (max, sum) pairs: wave shuffles, then the four waves
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float om = __shfl_xor(m, off), os = __shfl_xor(se, off);
    const float nm = fmaxf(m, om);
    se = (m == -INFINITY ? 0.0f : se * expf(m - nm)) + (om == -INFINITY ? 0.0f : os * expf(om - nm));
    m = nm;
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    shm[wave] = m;
    shs[wave] = se;
  }
  __syncthreads();
  const float mx = fmaxf(fmaxf(shm[0], shm[1]), fmaxf(shm[2], shm[3]));
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) tot += shm[w] == -INFINITY ? 0.0f : shs[w] * expf(shm[w] - mx);
  const float lse = mx + logf(tot);
  const int64_t tg = target[row];
  const bool ok = tg >= 0 && tg < V;
  if (threadIdx.x == 0) {
    const float zt = (float)zr[ok ? tg : 0];  // never indexes outside the row
    tok_loss[row] = ok ? lse - zt : 0.0f;
    if (!ok && status) *status = NF4_EINVAL;
  }
  if (!dz) return;
  for (int64_t c = threadIdx.x; c < nch; c += 256) {
    const bf16x8d v = *reinterpret_cast<const bf16x8d*>(zr + 8 * c);
    bf16x8d o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t i = 8 * c + e;
      o[e] = (__bf16)((expf((float)v[e] - lse) - (i == tg ? 1.0f : 0.0f)) * inv_tokens);
    }
    *reinterpret_cast<bf16x8d*>(dz + row * V + 8 * c) = o;
  }
}

__global__ __launch_bounds__(64) void k_xent_mean(const float* __restrict__ tok_loss, int64_t T,
                                                  float* __restrict__ loss) {
  if (threadIdx.x != 0) return;
  double s = 0.0;
  for (int64_t i = 0; i < T; ++i) s += (double)tok_loss[i];
  loss[0] = (float)(s / (double)T);
}

__global__ void k_status_zero(int32_t* status) {
  if (threadIdx.x == 0) *status = 0;
}

}  // namespace

#define NF4_DISPATCH(dt, BODY)        \
  do {                                \
    if ((dt) == NF4_BF16) {           \
      using T = __bf16;               \
      BODY;                           \
    } else {                          \
      using T = float;                \
      BODY;                           \
    }                                 \
  } while (0)

int launch_add_rmsnorm(const void* x, const void* res, nf4_dtype dt, int64_t rows, int64_t D, const float* gamma,
                       float eps, void* sum, void* y, float* rstd, hipStream_t st) {
  const bool vec = dt == NF4_BF16 && D % 8 == 0 && D <= 8192 && aligned16(gamma);
  if (vec) {
    const __bf16* xb = static_cast<const __bf16*>(x);
    const __bf16* rb = static_cast<const __bf16*>(res);
#define NF4_ARN(CPT)                                                                                          \
  hipLaunchKernelGGL(k_add_rmsnorm_v<CPT>, dim3((unsigned)rows), dim3(256), 0, st, xb, rb, D, gamma, eps,   \
                     static_cast<__bf16*>(sum), static_cast<__bf16*>(y), rstd)
    if (D <= 2048) NF4_ARN(1);
    else if (D <= 4096) NF4_ARN(2);
    else NF4_ARN(4);
#undef NF4_ARN
    return launch_status();
  }
  NF4_DISPATCH(dt, hipLaunchKernelGGL(k_add_rmsnorm<T>, dim3((unsigned)rows), dim3(256), 0, st,
                                      static_cast<const T*>(x), static_cast<const T*>(res), D, gamma, eps,
                                      static_cast<T*>(sum), static_cast<T*>(y), rstd));
  return launch_status();
}

int launch_rmsnorm_bwd(const void* dy, const void* x, const float* rstd, nf4_dtype dt, int64_t rows, int64_t D,
                       const float* gamma, const void* dres, void* dx, hipStream_t st) {
  const bool vec = dt == NF4_BF16 && D % 8 == 0 && D <= 8192 && aligned16(gamma);
  if (vec) {
#define NF4_RNB(CPT)                                                                                               \
  hipLaunchKernelGGL(k_rmsnorm_bwd_v<CPT>, dim3((unsigned)rows), dim3(256), 0, st, static_cast<const __bf16*>(dy), \
                     static_cast<const __bf16*>(x), rstd, D, gamma, static_cast<const __bf16*>(dres),             \
                     static_cast<__bf16*>(dx))
    if (D <= 2048) NF4_RNB(1);
    else if (D <= 4096) NF4_RNB(2);
    else NF4_RNB(4);
#undef NF4_RNB
    return launch_status();
  }
  NF4_DISPATCH(dt, hipLaunchKernelGGL(k_rmsnorm_bwd<T>, dim3((unsigned)rows), dim3(256), 0, st,
                                      static_cast<const T*>(dy), static_cast<const T*>(x), rstd, D, gamma,
                                      static_cast<const T*>(dres), static_cast<T*>(dx)));
  return launch_status();
}

int launch_rope(void* x, nf4_dtype dt, int64_t S, int32_t heads, int32_t d, int64_t ld, double theta, int inverse,
                hipStream_t st) {
  constexpr int kVB = 8, kVF = 4;  // 16-byte accesses
  const int64_t vw = dt == NF4_BF16 ? kVB : kVF;
  const bool vec = (d / 2) % vw == 0 && ld % vw == 0 && aligned16(x);
#define NF4_ROPE(T, V) \
  hipLaunchKernelGGL((k_rope<T, V>), dim3((unsigned)S), dim3(256), 0, st, static_cast<T*>(x), ld, heads, d, theta, inverse)
  if (dt == NF4_BF16) {
    if (vec) NF4_ROPE(__bf16, kVB);
    else NF4_ROPE(__bf16, 1);
  } else {
    if (vec) NF4_ROPE(float, kVF);
    else NF4_ROPE(float, 1);
  }
#undef NF4_ROPE
  return launch_status();
}

int launch_attention_fwd(const void* q, const void* k, const void* v, nf4_dtype dt, int64_t S, int32_t hq,
                         int32_t hkv, int32_t d, int64_t lq, int64_t lk, void* o, float* lse, hipStream_t st) {
  if (attention_mfma_supported(dt, d)) return launch_attention_fwd_mfma(q, k, v, S, hq, hkv, d, lq, lk, o, lse, st);
  const float scale = (float)(1.0 / std::sqrt((double)d));
  const dim3 grid((unsigned)ceil_div(S, AQ), (unsigned)hq);
  NF4_DISPATCH(dt, hipLaunchKernelGGL(k_attn_fwd<T>, grid, dim3(256), 0, st, static_cast<const T*>(q),
                                      static_cast<const T*>(k), static_cast<const T*>(v), S, hq, hkv, d, lq, lk,
                                      scale, static_cast<T*>(o), lse));
  return launch_status();
}

int launch_attention_bwd(const void* dout, const void* q, const void* k, const void* v, const void* o,
                         const float* lse, nf4_dtype dt, int64_t S, int32_t hq, int32_t hkv, int32_t d, int64_t lq,
                         int64_t lk, float* delta, void* dq, void* dk, void* dv, hipStream_t st) {
  if (attention_mfma_supported(dt, d))
    return launch_attention_bwd_mfma(dout, q, k, v, o, lse, S, hq, hkv, d, lq, lk, delta, dq, dk, dv, st);
  const float scale = (float)(1.0 / std::sqrt((double)d));
  NF4_DISPATCH(dt, {
    hipLaunchKernelGGL(k_attn_dq<T>, dim3((unsigned)ceil_div(S, AQ), (unsigned)hq), dim3(256), 0, st,
                       static_cast<const T*>(dout), static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), static_cast<const T*>(o), lse, S, hq, hkv, d, lq, lk, scale, delta,
                       static_cast<T*>(dq));
    hipLaunchKernelGGL(k_attn_dkv<T>, dim3((unsigned)ceil_div(S, AQ), (unsigned)hkv), dim3(256), 0, st,
                       static_cast<const T*>(dout), static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), lse, delta, S, hq, hkv, d, lq, lk, scale, static_cast<T*>(dk),
                       static_cast<T*>(dv));
  });
  return launch_status();
}

int launch_add3(const void* a, const void* b, const void* c, nf4_dtype dt, int64_t n, void* out, hipStream_t st) {
  NF4_DISPATCH(dt, hipLaunchKernelGGL(k_add3<T>, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st,
                                      static_cast<const T*>(a), static_cast<const T*>(b), static_cast<const T*>(c), n,
                                      static_cast<T*>(out)));
  return launch_status();
}

// Grid of the row-wise SwiGLU kernels for V entries per thread: column blocks
// of 256 V times up to 65535 row groups (rows beyond loop).
dim3 swiglu_grid(int64_t rows, int64_t width, int v) {
  return dim3((unsigned)ceil_div(width, 256 * (int64_t)v), (unsigned)(rows < 65535 ? rows : 65535));
}

// 16-byte vectors apply when every row start of every array is 16-byte aligned.
template <typename T>
bool swiglu_vec(int64_t width, int64_t ld, std::initializer_list<const void*> ptrs) {
  constexpr int V = 16 / sizeof(T);
  if (width % V != 0 || ld % V != 0) return false;
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return false;
  return true;
}

int launch_swiglu(const void* g, const void* u, nf4_dtype dt, int64_t rows, int64_t width, int64_t ld, void* a,
                  hipStream_t st) {
  NF4_DISPATCH(dt, {
    constexpr int V = 16 / sizeof(T);
    if (swiglu_vec<T>(width, ld, {g, u, a}))
      hipLaunchKernelGGL((k_swiglu<T, V>), swiglu_grid(rows, width, V), dim3(256), 0, st, static_cast<const T*>(g),
                         static_cast<const T*>(u), rows, width, ld, static_cast<T*>(a));
    else
      hipLaunchKernelGGL((k_swiglu<T, 1>), swiglu_grid(rows, width, 1), dim3(256), 0, st, static_cast<const T*>(g),
                         static_cast<const T*>(u), rows, width, ld, static_cast<T*>(a));
  });
  return launch_status();
}

int launch_swiglu_bwd(const void* da, const void* g, const void* u, nf4_dtype dt, int64_t rows, int64_t width,
                      int64_t ld, void* dg, void* du, hipStream_t st) {
  NF4_DISPATCH(dt, {
    constexpr int V = 16 / sizeof(T);
    if (swiglu_vec<T>(width, ld, {da, g, u, dg, du}))
      hipLaunchKernelGGL((k_swiglu_bwd<T, V>), swiglu_grid(rows, width, V), dim3(256), 0, st,
                         static_cast<const T*>(da), static_cast<const T*>(g), static_cast<const T*>(u), rows, width,
                         ld, static_cast<T*>(dg), static_cast<T*>(du));
    else
      hipLaunchKernelGGL((k_swiglu_bwd<T, 1>), swiglu_grid(rows, width, 1), dim3(256), 0, st,
                         static_cast<const T*>(da), static_cast<const T*>(g), static_cast<const T*>(u), rows, width,
                         ld, static_cast<T*>(dg), static_cast<T*>(du));
  });
  return launch_status();
}

int launch_cross_entropy(const void* z, nf4_dtype dt, int64_t tokens, int64_t V, const int64_t* target,
                         float* tok_loss, float* loss, void* dz, int32_t* status, hipStream_t st) {
  if (status) hipLaunchKernelGGL(k_status_zero, dim3(1), dim3(64), 0, st, status);
  if (dt == NF4_BF16 && V % 8 == 0) {
    hipLaunchKernelGGL(k_xent_v, dim3((unsigned)tokens), dim3(256), 0, st, static_cast<const __bf16*>(z), target, V,
                       (float)(1.0 / (double)tokens), tok_loss, static_cast<__bf16*>(dz), status);
    hipLaunchKernelGGL(k_xent_mean, dim3(1), dim3(64), 0, st, tok_loss, tokens, loss);
    return launch_status();
  }
  NF4_DISPATCH(dt, hipLaunchKernelGGL(k_xent<T>, dim3((unsigned)tokens), dim3(256), 0, st, static_cast<const T*>(z),
                                      target, V, (float)(1.0 / (double)tokens), tok_loss, static_cast<T*>(dz),
                                      status));
  hipLaunchKernelGGL(k_xent_mean, dim3(1), dim3(64), 0, st, tok_loss, tokens, loss);
  return launch_status();
}

#undef NF4_DISPATCH

}  // namespace nf4

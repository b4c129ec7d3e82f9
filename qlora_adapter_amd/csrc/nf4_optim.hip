// The optimizer step of a LoRA adapter on gfx950: the LoRA-FA preconditioner
// and one fused AdamW pass over both factors.
//
// Aner docs "Native model adaptation and NF4", section "LoRA FA includes
// gradient preconditioning": with A frozen (no gradient, no moments) the
// gradient of B is replaced by s^-2 g_B pinv(A A^T + 1e-8 I) before the Adam
// moments see it; the r x r matrix is computed once and kept with the adapter.
// Sections "Explicit accelerated training profiles" and "Mixed precision keeps
// stable state in FP32": the optimizer is AdamW over FP32 parameters and FP32
// moments. AdamW is the decoupled-decay form: p <- p (1 - lr wd), moments
// m <- b1 m + (1 - b1) g and v <- b2 v + (1 - b2) g^2, then
// p <- p - lr m_hat / (sqrt(v_hat) + eps) with m_hat = m / (1 - b1^t) and
// v_hat = v / (1 - b2^t).
//
// Kernels
//  k_gram_partial  fp64 partial Gram matrices A[:, slice] A[:, slice]^T. A
//                  workgroup owns one 16 x 16 tile of the upper triangle and
//                  one K slice; the fp32 products are exact in fp64. Tiles off
//                  the diagonal are mirrored, so every slice is a full r x r.
//  k_spd_invert    one workgroup of 1024 threads: sums the slices in slice
//                  order, adds the 1e-8 damping to the diagonal and inverts by
//                  Gauss-Jordan elimination without row exchanges (the damped
//                  Gram matrix is symmetric positive definite, so every pivot
//                  is positive). Each thread owns fixed entries, in registers
//                  up to r = 128 and in the workspace beyond; the pivot row and
//                  column of each step pass through LDS (double-buffered, one
//                  barrier per pivot). P is written in fp32.
//  k_lora_adamw    one pass that reads p, g, m, v and writes p, m, v for every
//                  entry of A and B of up to 16 adapters (28 bytes per
//                  parameter, 16-byte accesses); the tensors are described in
//                  the kernel arguments and dealt out in workgroup ranges.
//                  Under LoRA-FA each thread forms its four entries of the
//                  preconditioned B gradient row from g_B and P on the fly.
#include <cmath>

#include "nf4_internal.hpp"

namespace nf4 {
namespace {

constexpr int kGramTile = 16;        // Gram tile edge
constexpr int kGramChunk = 64;       // K columns staged per LDS pass
constexpr int64_t kGramTargetWG = 512;
constexpr double kDamping = 1e-8;

// Number of K slices of the Gram reduction (a pure function of r and K, so
// the workspace query and the launch agree).
int64_t gram_slices(int32_t r, int64_t K) {
  const int64_t nt = ceil_div(r, kGramTile);
  const int64_t tiles = nt * (nt + 1) / 2;
  const int64_t chunks = ceil_div(K, kGramChunk);
  int64_t s = kGramTargetWG / tiles;
  if (s < 1) s = 1;
  if (s > chunks) s = chunks;
  const int64_t per = ceil_div(chunks, s);  // chunks per slice
  return ceil_div(chunks, per);
}

int64_t gram_chunks_per_slice(int32_t r, int64_t K) {
  return ceil_div(ceil_div(K, kGramChunk), gram_slices(r, K));
}

__global__ __launch_bounds__(256) void k_gram_partial(const float* __restrict__ A, int32_t r, int64_t K,
                                                      int64_t chunks_per_slice, double* __restrict__ out) {
  __shared__ float sa[kGramTile][kGramChunk + 1];
  __shared__ float sb[kGramTile][kGramChunk + 1];
  const int t = threadIdx.x;
  // blockIdx.x enumerates the upper-triangle tiles (bi <= bj) row by row.
  const int nt = (r + kGramTile - 1) / kGramTile;
  int rem = blockIdx.x, bi = 0;
  while (rem >= nt - bi) {
    rem -= nt - bi;
    ++bi;
  }
  const int bj = bi + rem;
  const int64_t slice = blockIdx.y;
  const int64_t k_begin = slice * chunks_per_slice * kGramChunk;
  int64_t k_end = k_begin + chunks_per_slice * kGramChunk;
  if (k_end > K) k_end = K;

  const int ti = t / kGramTile, tj = t % kGramTile;
  double acc = 0.0;
  for (int64_t k0 = k_begin; k0 < k_end; k0 += kGramChunk) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = t + 256 * q;  // 0..1023 covers 16 rows x 64 columns
      const int row = e / kGramChunk, col = e % kGramChunk;
      const int64_t k = k0 + col;
      const int ra = bi * kGramTile + row, rb = bj * kGramTile + row;
      sa[row][col] = (ra < r && k < k_end) ? A[(int64_t)ra * K + k] : 0.0f;
      sb[row][col] = (rb < r && k < k_end) ? A[(int64_t)rb * K + k] : 0.0f;
    }
    __syncthreads();
#pragma unroll 16
    for (int c = 0; c < kGramChunk; ++c) acc += (double)sa[ti][c] * (double)sb[tj][c];
    __syncthreads();
  }
  const int i = bi * kGramTile + ti, j = bj * kGramTile + tj;
  if (i < r && j < r) {
    double* g = out + slice * (int64_t)r * r;
    g[(int64_t)i * r + j] = acc;
    if (bi != bj) g[(int64_t)j * r + i] = acc;
  }
}

// Inverse of the damped Gram matrix. Entry q of thread t is e = t + 1024 q of
// the row-major r x r matrix (r * r <= 1024 * EPT <= 65536). GLOBAL keeps the
// entries in slice 0 of the workspace instead of registers.
template <int EPT, bool GLOBAL>
__global__ __launch_bounds__(1024) void k_spd_invert(double* __restrict__ ws, int32_t r, int64_t slices,
                                                    float* __restrict__ P) {
  __shared__ double rowk[2][256];
  __shared__ double colk[2][256];
  const int t = threadIdx.x;
  const int rr = r * r;
  constexpr int NR = GLOBAL ? 1 : EPT;
  constexpr int UNR = GLOBAL ? 1 : EPT;  // the workspace-resident form is not unrolled
  double a[NR];
  int ei[NR], ej[NR];
  auto ld = [&](int q, int e) -> double {
    if constexpr (GLOBAL) return ws[e];
    else return a[q];
  };
  auto st = [&](int q, int e, double v) {
    if constexpr (GLOBAL) ws[e] = v;
    else a[q] = v;
  };
  // Sum of the slices in slice order, plus the damping on the diagonal.
#pragma unroll UNR
  for (int q = 0; q < EPT; ++q) {
    const int e = t + 1024 * q;
    if (e < rr) {
      // slice order; eight loads in flight at a time
      double v = 0.0;
      int64_t s = 0;
      for (; s + 8 <= slices; s += 8) {
        double x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = ws[(s + u) * rr + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) v += x[u];
      }
      for (; s < slices; ++s) v += ws[s * rr + e];
      const int i = e / r, j = e - (e / r) * r;
      if (i == j) v += kDamping;
      st(q, e, v);
      if constexpr (!GLOBAL) {
        ei[q] = i;
        ej[q] = j;
      }
    }
  }
  for (int k = 0; k < r; ++k) {
    const int buf = k & 1;
#pragma unroll UNR
    for (int q = 0; q < EPT; ++q) {
      const int e = t + 1024 * q;
      if (e < rr) {
        const int i = GLOBAL ? e / r : ei[GLOBAL ? 0 : q];
        const int j = GLOBAL ? e - i * r : ej[GLOBAL ? 0 : q];
        const double v = ld(q, e);
        if (i == k) rowk[buf][j] = v;
        if (j == k) colk[buf][i] = v;
      }
    }
    __syncthreads();
    const double inv = 1.0 / rowk[buf][k];
#pragma unroll UNR
    for (int q = 0; q < EPT; ++q) {
      const int e = t + 1024 * q;
      if (e < rr) {
        const int i = GLOBAL ? e / r : ei[GLOBAL ? 0 : q];
        const int j = GLOBAL ? e - i * r : ej[GLOBAL ? 0 : q];
        const double rp = (j == k) ? inv : rowk[buf][j] * inv;
        double v;
        if (i == k) {
          v = rp;
        } else {
          const double old = (j == k) ? 0.0 : ld(q, e);
          v = old - colk[buf][i] * rp;
        }
        st(q, e, v);
      }
    }
  }
#pragma unroll UNR
  for (int q = 0; q < EPT; ++q) {
    const int e = t + 1024 * q;
    if (e < rr) P[e] = (float)ld(q, e);
  }
}

// ---------------------------------------------------------------- AdamW

struct AdamwConst {
  float b1, b2;      // moment decay rates
  float omb1, omb2;  // 1 - b1, 1 - b2
  float dec;         // 1 - lr * wd
  float stepsz;      // lr / (1 - b1^t)
  float rbc2;        // 1 / sqrt(1 - b2^t)
  float eps;
};

// One tensor of one update: A or B of an adapter. mode 0: plain AdamW over n
// entries; 1: B with the preconditioned gradient, r % 4 == 0 (four entries of
// one row per thread); 2: the same for any r (one entry per thread).
struct AdamwSeg {
  float* p;
  const float* g;
  float* m;
  float* v;
  const float* P;  // r x r preconditioner (modes 1, 2)
  int64_t n;       // entries
  int64_t block0;  // first workgroup of this tensor
  int32_t r;
  int32_t mode;
  float pscale;    // s^-2 (modes 1, 2)
};

constexpr int kMaxSegs = 2 * NF4_MAX_ADAPTERS_PER_CALL;

// All tensors of one launch, passed by value in the kernel arguments.
struct AdamwTable {
  AdamwSeg seg[kMaxSegs];
  int32_t count;
};

__device__ __forceinline__ void adamw_one(float& p, float g, float& m, float& v, const AdamwConst& c) {
  m = c.b1 * m + c.omb1 * g;
  v = c.b2 * v + c.omb2 * (g * g);
  const float den = __builtin_sqrtf(v) * c.rbc2 + c.eps;
  p = p * c.dec - c.stepsz * (m / den);
}

using f4 = float __attribute__((ext_vector_type(4)));

// Four consecutive entries starting at e (e % 4 == 0, e + 3 < n) with gradient gv.
__device__ __forceinline__ void adamw_four(const AdamwSeg& s, int64_t e, f4 gv, const AdamwConst& c) {
  f4 p = *reinterpret_cast<const f4*>(s.p + e);
  f4 m = *reinterpret_cast<const f4*>(s.m + e);
  f4 v = *reinterpret_cast<const f4*>(s.v + e);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float pk = p[k], mk = m[k], vk = v[k];
    adamw_one(pk, gv[k], mk, vk, c);
    p[k] = pk;
    m[k] = mk;
    v[k] = vk;
  }
  *reinterpret_cast<f4*>(s.p + e) = p;
  *reinterpret_cast<f4*>(s.m + e) = m;
  *reinterpret_cast<f4*>(s.v + e) = v;
}

__global__ __launch_bounds__(256) void k_lora_adamw(AdamwTable tab, const float* __restrict__ gscale, AdamwConst c) {
  const float gs = gscale ? *gscale : 1.0f;
  const int64_t b = blockIdx.x;
  int k = 0;  // tensor of this workgroup (uniform)
  while (k + 1 < tab.count && b >= tab.seg[k + 1].block0) ++k;
  const AdamwSeg& s = tab.seg[k];
  const int64_t u = (b - s.block0) * 256 + threadIdx.x;
  if (s.mode == 0) {
    const int64_t e = 4 * u;
    if (e + 3 < s.n) {
      const f4 g = *reinterpret_cast<const f4*>(s.g + e);
      adamw_four(s, e, g * gs, c);
    } else {
      for (int64_t x = e; x < s.n; ++x) {
        float p = s.p[x], m = s.m[x], v = s.v[x];
        adamw_one(p, s.g[x] * gs, m, v, c);
        s.p[x] = p;
        s.m[x] = m;
        s.v[x] = v;
      }
    }
  } else if (s.mode == 1) {
    const int64_t e = 4 * u;
    if (e >= s.n) return;
    const int r = s.r;
    const int64_t o = e / r;
    const int i0 = (int)(e - o * r);
    const float* grow = s.g + o * r;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int j = 0; j < r; ++j) {
      const float gj = grow[j];
      const f4 pj = *reinterpret_cast<const f4*>(s.P + (int64_t)j * r + i0);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(gj, pj[q], acc[q]);
    }
    adamw_four(s, e, acc * (gs * s.pscale), c);
  } else {
    const int64_t e = u;
    if (e >= s.n) return;
    const int r = s.r;
    const int64_t o = e / r;
    const int i = (int)(e - o * r);
    const float* grow = s.g + o * r;
    float acc = 0.f;
    for (int j = 0; j < r; ++j) acc = __builtin_fmaf(grow[j], s.P[(int64_t)j * r + i], acc);
    float p = s.p[e], m = s.m[e], v = s.v[e];
    adamw_one(p, acc * (gs * s.pscale), m, v, c);
    s.p[e] = p;
    s.m[e] = m;
    s.v[e] = v;
  }
}

}  // namespace

size_t lorafa_ws_bytes(int32_t r, int64_t K) {
  return (size_t)gram_slices(r, K) * (size_t)r * (size_t)r * sizeof(double);
}

int launch_lorafa_preconditioner(const float* A, int32_t r, int64_t K, float* P, void* ws, hipStream_t st) {
  const int64_t nt = ceil_div(r, kGramTile);
  const int64_t slices = gram_slices(r, K);
  double* g = static_cast<double*>(ws);
  hipLaunchKernelGGL(k_gram_partial, dim3((unsigned)(nt * (nt + 1) / 2), (unsigned)slices), dim3(256), 0, st, A, r,
                     K, gram_chunks_per_slice(r, K), g);
  if (int rc = launch_status()) return rc;
  const int64_t rr = (int64_t)r * r;
  if (rr <= 1024)
    hipLaunchKernelGGL((k_spd_invert<1, false>), dim3(1), dim3(1024), 0, st, g, r, slices, P);
  else if (rr <= 4096)
    hipLaunchKernelGGL((k_spd_invert<4, false>), dim3(1), dim3(1024), 0, st, g, r, slices, P);
  else if (rr <= 16384)
    hipLaunchKernelGGL((k_spd_invert<16, false>), dim3(1), dim3(1024), 0, st, g, r, slices, P);
  else
    hipLaunchKernelGGL((k_spd_invert<64, true>), dim3(1), dim3(1024), 0, st, g, r, slices, P);
  return launch_status();
}

namespace {

// Per-update constants, formed in fp64 and rounded once to fp32.
AdamwConst make_adamw_const(const nf4_adamw& opt) {
  const double lr = opt.lr, b1 = opt.beta1, b2 = opt.beta2, wd = opt.weight_decay;
  const double t = (double)opt.step;
  const double bc1 = 1.0 - std::pow(b1, t), bc2 = 1.0 - std::pow(b2, t);
  AdamwConst c;
  c.b1 = opt.beta1;
  c.b2 = opt.beta2;
  c.omb1 = (float)(1.0 - b1);
  c.omb2 = (float)(1.0 - b2);
  c.dec = (float)(1.0 - lr * wd);
  c.stepsz = (float)(lr / bc1);
  c.rbc2 = (float)(1.0 / std::sqrt(bc2));
  c.eps = opt.eps;
  return c;
}

// Mode of a tensor (see AdamwSeg) and the s^-2 factor.
int seg_mode(const float* P, int32_t r) { return P ? ((r % 4 == 0) ? 1 : 2) : 0; }
float seg_pscale(const float* P, float s) { return P ? (float)(1.0 / ((double)s * (double)s)) : 1.0f; }
int64_t seg_blocks(int mode, int64_t n) { return ceil_div(mode == 2 ? n : ceil_div(n, 4), 256); }

}  // namespace

int launch_lora_adamw(const nf4_adamw& opt, const nf4_lora_state* ad, int32_t count, const float* grad_scale,
                      hipStream_t st) {
  const AdamwConst c = make_adamw_const(opt);
  AdamwTable tab{};
  int64_t blocks = 0;
  auto add = [&](float* p, const float* g, float* m, float* v, int64_t n, const float* P, int32_t r, float s) {
    const int mode = seg_mode(P, r);
    tab.seg[tab.count++] = AdamwSeg{p, g, m, v, P, n, blocks, r, mode, seg_pscale(P, s)};
    blocks += seg_blocks(mode, n);
  };
  for (int32_t i = 0; i < count; ++i) {
    const nf4_lora_state& a = ad[i];
    if (a.A) add(a.A, a.dA, a.mA, a.vA, (int64_t)a.r * a.K, nullptr, a.r, a.s);
    add(a.B, a.dB, a.mB, a.vB, a.N * a.r, a.precond, a.r, a.s);
  }
  hipLaunchKernelGGL(k_lora_adamw, dim3((unsigned)blocks), dim3(256), 0, st, tab, grad_scale, c);
  return launch_status();
}

}  // namespace nf4

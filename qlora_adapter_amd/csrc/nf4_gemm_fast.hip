// Large-tile fused NF4 GEMM kernels for gfx950 (bf16 operands, fp32 accumulate).
//
// Forward: y = x W_hat^T + s T B^T for K a multiple of 64. A workgroup owns a
// 256 (tokens) x 128 (outputs) tile and walks K in steps of 64, which is exactly
// one 64-element quantization block of every weight row. Four waves in a 2 x 2
// arrangement each own 128 x 64 outputs as 4 x 2 accumulators of the 32x32x16
// bf16 MFMA.
//  - x is staged through LDS (double-buffered, rows padded to 144 bytes so that
//    the 16-byte operand reads of 8 consecutive rows fall in distinct banks).
//  - The packed weights never touch LDS: each lane loads the 16 bytes (32
//    nibbles) of its weight row that its MFMA operands need, builds the 16-entry
//    bf16 table {bf16(fl32(C4[c] * a'))} of that row's block once, and turns
//    nibbles into bf16 with byte-select (v_perm_b32) lookups. The values are
//    bit-identical to nf4_dequantize's bf16 output.
//  - Lane group g = lane / 32 takes k in [32g, 32g + 32) of the block: MFMA step j
//    uses k = 32g + 8j .. +8 for both operands, a fixed permutation of the
//    reduction order.
//  - The LoRA term s T B^T is added to the fp32 accumulators with the 32x32x2
//    fp32 MFMA before the single bf16 rounding of the output.
//  - Workgroups are numbered so that each XCD gets a contiguous run of tiles,
//    and tiles are visited in groups of 4 token-tiles so that concurrently
//    running workgroups share x and weight tiles in L2.
//
// Input gradient: dX = dY W_hat + s U A for K and N multiples of 64. A
// workgroup owns 256 (tokens) x 128 (weight inputs k) of dX and walks the
// reduction over the weight outputs n in steps of 64. Here the weight operand
// needs consecutive n per lane while the packed rows run along k, so each step
// the workgroup decodes its 64 x 128 weight slice once, cooperatively, into an
// LDS tile stored transposed ([k][n], rows padded to 144 bytes): thread t
// decodes rows 2p, 2p+1 (p = t % 32) over 16 columns and pairs the two rows
// into one 32-bit LDS word per column with a byte select.
#include "nf4_device.hpp"

namespace nf4 {
namespace {

constexpr uint32_t kC4Bits[NF4_CODES_COUNT] = {NF4_CODES_LIST};

// 16-entry bf16 table of one block, split into low-byte and high-byte planes:
// lo[j] holds the low bytes of entries 4j..4j+3, hi[j] the high bytes.
struct Bf16Table {
  uint32_t lo[4], hi[4];
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ __forceinline__ Bf16Table build_table(float a) {
  uint32_t P[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    P[i] = pack_bf16x2(__fmul_rn(__uint_as_float(kC4Bits[2 * i]), a), __fmul_rn(__uint_as_float(kC4Bits[2 * i + 1]), a));
  Bf16Table t;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    t.lo[j] = __builtin_amdgcn_perm(P[2 * j + 1], P[2 * j], 0x06040200u);
    t.hi[j] = __builtin_amdgcn_perm(P[2 * j + 1], P[2 * j], 0x07050301u);
  }
  return t;
}

// Table lookup of four 4-bit indices held one per byte: sel = index & 7 per byte,
// hi8 = 0xFF in the bytes whose index is >= 8.
__device__ __forceinline__ void lookup4(const Bf16Table& t, uint32_t sel, uint32_t hi8, uint32_t& lo, uint32_t& hi) {
  const uint32_t lo_a = __builtin_amdgcn_perm(t.lo[1], t.lo[0], sel);
  const uint32_t lo_b = __builtin_amdgcn_perm(t.lo[3], t.lo[2], sel);
  const uint32_t hi_a = __builtin_amdgcn_perm(t.hi[1], t.hi[0], sel);
  const uint32_t hi_b = __builtin_amdgcn_perm(t.hi[3], t.hi[2], sel);
  lo = (hi8 & lo_b) | (~hi8 & lo_a);
  hi = (hi8 & hi_b) | (~hi8 & hi_a);
}

// Decode one 32-bit code word (8 weights; weight 2p in the high nibble of byte
// p) into 8 bf16 values in weight order.
__device__ __forceinline__ bf16x8 decode_word(uint32_t w, const Bf16Table& t) {
  // selector bytes 0x0C -> 0x00 and 0x0D -> 0xFF turn bit 3 of each index into a byte mask
  const uint32_t sel_e = (w >> 4) & 0x07070707u;
  const uint32_t msk_e = __builtin_amdgcn_perm(0u, 0u, ((w >> 7) & 0x01010101u) | 0x0C0C0C0Cu);
  const uint32_t sel_o = w & 0x07070707u;
  const uint32_t msk_o = __builtin_amdgcn_perm(0u, 0u, ((w >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
  uint32_t el, eh, ol, oh;
  lookup4(t, sel_e, msk_e, el, eh);  // weights 0, 2, 4, 6
  lookup4(t, sel_o, msk_o, ol, oh);  // weights 1, 3, 5, 7
  const uint32_t e01 = __builtin_amdgcn_perm(eh, el, 0x05010400u);  // bf16(w0) | bf16(w2) << 16
  const uint32_t e23 = __builtin_amdgcn_perm(eh, el, 0x07030602u);  // bf16(w4) | bf16(w6) << 16
  const uint32_t o01 = __builtin_amdgcn_perm(oh, ol, 0x05010400u);  // bf16(w1) | bf16(w3) << 16
  const uint32_t o23 = __builtin_amdgcn_perm(oh, ol, 0x07030602u);  // bf16(w5) | bf16(w7) << 16
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 d;
  d[0] = __builtin_amdgcn_perm(o01, e01, 0x05040100u);
  d[1] = __builtin_amdgcn_perm(o01, e01, 0x07060302u);
  d[2] = __builtin_amdgcn_perm(o23, e23, 0x05040100u);
  d[3] = __builtin_amdgcn_perm(o23, e23, 0x07060302u);
  return __builtin_bit_cast(bf16x8, d);
}

// Tile coordinates of workgroup b: a contiguous run of tiles per XCD (workgroups
// are dealt to the 8 XCDs round-robin), then groups of GM token-tiles walked
// token-tile-fastest.
__device__ __forceinline__ void tile_coords(int64_t b, int64_t MT, int64_t NT, int64_t& mt, int64_t& nt) {
  const int64_t nwg = MT * NT;
  int64_t t = b;
  if (nwg % 8 == 0) t = (b % 8) * (nwg / 8) + b / 8;
  constexpr int64_t GM = 4;
  const int64_t group = t / (GM * NT);
  const int64_t first_m = group * GM;
  const int64_t gm = (MT - first_m) < GM ? (MT - first_m) : GM;
  const int64_t within = t - group * GM * NT;
  mt = first_m + within % gm;
  nt = within / gm;
}

constexpr int FBM = 256, FBN = 128, FBK = 64;
constexpr int XPITCH = 72;  // bf16 per LDS row of the x tile (64 + 8 pad)

template <bool DQ>
__global__ __launch_bounds__(256) void k_fwd_fast(const __bf16* __restrict__ x, int64_t M, int64_t K, int64_t N,
                                                  NF4View w, const float* __restrict__ Bfac, int r, float s,
                                                  const float* __restrict__ T, __bf16* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) __bf16 xs[2][FBM * XPITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, g = lane >> 5, l32 = lane & 31;
  const int64_t MT = (M + FBM - 1) / FBM, NT = (N + FBN - 1) / FBN;
  int64_t mt, nt;
  tile_coords(blockIdx.x, MT, NT, mt, nt);
  const int64_t m0 = mt * FBM, n0 = nt * FBN;
  const int64_t KT = K / FBK;
  const float mu = DQ ? w.offset[0] : 0.0f;

  // x loader: thread t copies 16-byte chunk (t & 7) of rows (t >> 3) + 32 i.
  const int xc = tid & 7, xr = tid >> 3;
  uint4 xreg[8];
  // weight rows of this lane (one per 32-wide output subtile)
  int64_t nrow[2];
  bool nok[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    nrow[ni] = n0 + wn * 64 + ni * 32 + l32;
    nok[ni] = nrow[ni] < N;
  }
  uint4 wreg[2];
  float wsc[2];

  auto load_x = [&](int64_t kt) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m0 + xr + 32 * i;
      xreg[i] = (m < M) ? *reinterpret_cast<const uint4*>(x + m * K + kt * FBK + 8 * xc) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(&xs[buf][(xr + 32 * i) * XPITCH + 8 * xc]) = xreg[i];
  };
  auto load_w = [&](int64_t kt) {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      if (nok[ni]) {
        wreg[ni] = *reinterpret_cast<const uint4*>(w.codes + (nrow[ni] * K + kt * FBK) / 2 + 16 * g);
        wsc[ni] = block_scale_of<DQ>(w, mu, nrow[ni] * (K / FBK) + kt);
      } else {
        wreg[ni] = make_uint4(0, 0, 0, 0);
        wsc[ni] = 0.0f;
      }
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

  load_x(0);
  load_w(0);
  store_x(0);
  __syncthreads();
  for (int64_t kt = 0; kt < KT; ++kt) {
    const int cur = (int)(kt & 1);
    const uint4 wc0 = wreg[0], wc1 = wreg[1];
    const float sc0 = wsc[0], sc1 = wsc[1];
    if (kt + 1 < KT) {
      load_x(kt + 1);
      load_w(kt + 1);
    }
    bf16x8 bop[2][4];
    {
      const Bf16Table t0 = build_table(sc0);
      bop[0][0] = decode_word(wc0.x, t0);
      bop[0][1] = decode_word(wc0.y, t0);
      bop[0][2] = decode_word(wc0.z, t0);
      bop[0][3] = decode_word(wc0.w, t0);
      const Bf16Table t1 = build_table(sc1);
      bop[1][0] = decode_word(wc1.x, t1);
      bop[1][1] = decode_word(wc1.y, t1);
      bop[1][2] = decode_word(wc1.z, t1);
      bop[1][3] = decode_word(wc1.w, t1);
    }
    const __bf16* xb = xs[cur];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 aop[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        aop[mi] = *reinterpret_cast<const bf16x8*>(&xb[(wm * 128 + mi * 32 + l32) * XPITCH + 32 * g + 8 * j]);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[mi], bop[ni][j], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < KT) store_x(cur ^ 1);
    __syncthreads();
  }

  // LoRA: acc += (s T[m][rho]) * B[n][rho], two ranks per fp32 MFMA step.
  if (r > 0) {
    for (int rho0 = 0; rho0 < r; rho0 += 2) {
      const int rho = rho0 + g;
      float av[4], bv[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int64_t m = m0 + wm * 128 + mi * 32 + l32;
        av[mi] = (rho < r && m < M) ? s * T[m * r + rho] : 0.0f;
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) bv[ni] = (rho < r && nok[ni]) ? Bfac[nrow[ni] * r + rho] : 0.0f;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mi], bv[ni], acc[mi][ni], 0, 0, 0);
    }
  }

  // Store: accumulator element e of subtile (mi, ni) is row (e/4)*8 + 4g + e%4, column l32.
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      if (!nok[ni]) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * 128 + mi * 32 + (e >> 2) * 8 + g * 4 + (e & 3);
        if (m < M) y[m * N + nrow[ni]] = (__bf16)acc[mi][ni][e];
      }
    }
}

template <bool DQ>
__global__ __launch_bounds__(256) void k_bwd_fast(const __bf16* __restrict__ dy, int64_t M, int64_t K, int64_t N,
                                                  NF4View w, const float* __restrict__ Afac, int r, float s,
                                                  const float* __restrict__ U, __bf16* __restrict__ dx) {
  constexpr int BKO = 128, BNR = 64, WPITCH = 72;
  __shared__ __attribute__((aligned(16))) __bf16 ys[2][FBM * XPITCH];
  __shared__ __attribute__((aligned(16))) __bf16 wt[2][BKO * WPITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, g = lane >> 5, l32 = lane & 31;
  const int64_t MT = (M + FBM - 1) / FBM, KTL = (K + BKO - 1) / BKO;
  int64_t mt, kt_tile;
  tile_coords(blockIdx.x, MT, KTL, mt, kt_tile);
  const int64_t m0 = mt * FBM, k0 = kt_tile * BKO;
  const int64_t NS = N / BNR;  // reduction steps
  const int64_t KB = K / 64;   // blocks per weight row
  const float mu = DQ ? w.offset[0] : 0.0f;

  // dY loader (same pattern as x in the forward kernel)
  const int yc = tid & 7, yr = tid >> 3;
  uint4 yreg[8];
  // weight decoder: rows 2p, 2p+1 of the step, columns [16c, 16c + 16) of the tile
  const int p = tid & 31, c = tid >> 5;
  const bool cok = k0 + 16 * c < K;
  uint2 wreg[2];
  float wsc[2];

  auto load_y = [&](int64_t ns) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t m = m0 + yr + 32 * i;
      yreg[i] = (m < M) ? *reinterpret_cast<const uint4*>(dy + m * N + ns * BNR + 8 * yc) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_y = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(&ys[buf][(yr + 32 * i) * XPITCH + 8 * yc]) = yreg[i];
  };
  auto load_w = [&](int64_t ns) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t n = ns * BNR + 2 * p + e;
      if (cok) {
        wreg[e] = *reinterpret_cast<const uint2*>(w.codes + (n * K + k0 + 16 * c) / 2);
        wsc[e] = block_scale_of<DQ>(w, mu, n * KB + (k0 + 16 * c) / 64);
      } else {
        wreg[e] = make_uint2(0, 0);
        wsc[e] = 0.0f;
      }
    }
  };
  auto decode_store_w = [&](int buf) {
    const Bf16Table t0 = build_table(wsc[0]);
    const Bf16Table t1 = build_table(wsc[1]);
    bf16x8 r0[2], r1[2];
    r0[0] = decode_word(wreg[0].x, t0);
    r0[1] = decode_word(wreg[0].y, t0);
    r1[0] = decode_word(wreg[1].x, t1);
    r1[1] = decode_word(wreg[1].y, t1);
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 a = __builtin_bit_cast(u32x4, r0[h]);
      const u32x4 b = __builtin_bit_cast(u32x4, r1[h]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = 16 * c + 8 * h + 2 * q;  // columns kk, kk + 1
        uint32_t* base = reinterpret_cast<uint32_t*>(&wt[buf][0]);
        base[(kk * WPITCH + 2 * p) / 2] = __builtin_amdgcn_perm(b[q], a[q], 0x05040100u);
        base[((kk + 1) * WPITCH + 2 * p) / 2] = __builtin_amdgcn_perm(b[q], a[q], 0x07060302u);
      }
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

  load_y(0);
  load_w(0);
  store_y(0);
  decode_store_w(0);
  __syncthreads();
  for (int64_t ns = 0; ns < NS; ++ns) {
    const int cur = (int)(ns & 1);
    if (ns + 1 < NS) {
      load_y(ns + 1);
      load_w(ns + 1);
    }
    const __bf16* yb = ys[cur];
    const __bf16* wb = wt[cur];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 aop[4], bop[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        aop[mi] = *reinterpret_cast<const bf16x8*>(&yb[(wm * 128 + mi * 32 + l32) * XPITCH + 32 * g + 8 * j]);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bop[ni] = *reinterpret_cast<const bf16x8*>(&wb[(wn * 64 + ni * 32 + l32) * WPITCH + 32 * g + 8 * j]);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[mi], bop[ni], acc[mi][ni], 0, 0, 0);
    }
    if (ns + 1 < NS) {
      store_y(cur ^ 1);
      decode_store_w(cur ^ 1);
    }
    __syncthreads();
  }

  int64_t kcol[2];
  bool kok[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    kcol[ni] = k0 + wn * 64 + ni * 32 + l32;
    kok[ni] = kcol[ni] < K;
  }
  // LoRA: acc += (s U[m][rho]) * A[rho][k], two ranks per fp32 MFMA step.
  if (r > 0) {
    for (int rho0 = 0; rho0 < r; rho0 += 2) {
      const int rho = rho0 + g;
      float av[4], bv[2];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int64_t m = m0 + wm * 128 + mi * 32 + l32;
        av[mi] = (rho < r && m < M) ? s * U[m * r + rho] : 0.0f;
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) bv[ni] = (rho < r && kok[ni]) ? Afac[(int64_t)rho * K + kcol[ni]] : 0.0f;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mi], bv[ni], acc[mi][ni], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      if (!kok[ni]) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * 128 + mi * 32 + (e >> 2) * 8 + g * 4 + (e & 3);
        if (m < M) dx[m * K + kcol[ni]] = (__bf16)acc[mi][ni][e];
      }
    }
}

}  // namespace

bool fast_linear_applies(const LinearArgs& g) {
  if (g.dtype != NF4_BF16) return false;
  if (g.backward) return g.K % 64 == 0 && g.N % 64 == 0;
  return g.K % FBK == 0;
}

int launch_linear_fast(const LinearArgs& g, hipStream_t st) {
  const NF4View w = make_view(g.W);
  const bool dq = g.W->double_quant != 0;
  if (g.backward) {
    const int64_t MT = ceil_div(g.M, FBM), KTL = ceil_div(g.K, 128);
    const dim3 grid((unsigned)(MT * KTL));
    const __bf16* dy = static_cast<const __bf16*>(g.a);
    __bf16* dx = static_cast<__bf16*>(g.out);
    if (dq)
      hipLaunchKernelGGL(k_bwd_fast<true>, grid, dim3(256), 0, st, dy, g.M, g.K, g.N, w, g.A, g.r, g.s, g.side, dx);
    else
      hipLaunchKernelGGL(k_bwd_fast<false>, grid, dim3(256), 0, st, dy, g.M, g.K, g.N, w, g.A, g.r, g.s, g.side, dx);
    return launch_status();
  }
  const int64_t MT = ceil_div(g.M, FBM), NT = ceil_div(g.N, FBN);
  const dim3 grid((unsigned)(MT * NT));
  const __bf16* x = static_cast<const __bf16*>(g.a);
  __bf16* y = static_cast<__bf16*>(g.out);
  if (dq)
    hipLaunchKernelGGL(k_fwd_fast<true>, grid, dim3(256), 0, st, x, g.M, g.K, g.N, w, g.B, g.r, g.s, g.side, y);
  else
    hipLaunchKernelGGL(k_fwd_fast<false>, grid, dim3(256), 0, st, x, g.M, g.K, g.N, w, g.B, g.r, g.s, g.side, y);
  return launch_status();
}

}  // namespace nf4

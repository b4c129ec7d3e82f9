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
constexpr int XPITCH = 72;  // bf16 per padded LDS row (64 + 8) of the input-gradient kernel

// 16-byte chunk swizzle of the dense [rows][128 B] LDS tiles: chunk c of row r
// is stored at chunk c ^ swz(r). Eight consecutive rows hit eight different
// chunks, and sixteen consecutive rows cover all 64 four-byte banks, so the
// 16-byte MFMA operand reads are free of bank conflicts.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// Split an fp32 value into three bf16 parts whose sum is the value exactly.
__device__ __forceinline__ void split3(float v, __bf16& a, __bf16& b, __bf16& c) {
  a = (__bf16)v;
  const float r1 = v - (float)a;
  b = (__bf16)r1;
  const float r2 = r1 - (float)b;
  c = (__bf16)r2;
}

// Eight consecutive fp32 values p[0..7] with entries at or past `limit` read
// as zero, split into three bf16x8 vectors.
__device__ __forceinline__ void load_split8(const float* __restrict__ p, int avail, float scale, bf16x8& h,
                                            bf16x8& m, bf16x8& l) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = (e < avail) ? scale * p[e] : 0.0f;
    __bf16 a, b, c;
    split3(v, a, b, c);
    h[e] = a;
    m[e] = b;
    l[e] = c;
  }
}

// One weight-operand step: 16 bytes of codes per subtile and its block scale inputs.
template <int NS>
struct WStep {
  uint4 q[NS];
  uint32_t qa[NS];  // dynamic8 code (double quant) of the block
  float nv[NS];     // nested max (double quant) or absmax (single quant)
};

// 16-byte direct global -> LDS load: lane l writes dst + 16 l (dst wave-uniform).
__device__ __forceinline__ void lds_dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

template <int XI>
__device__ __forceinline__ void fwd_issue_x(const __bf16* __restrict__ x, const int32_t (&xoff)[XI], int64_t kt,
                                            __bf16* buf, int wave) {
#pragma unroll
  for (int i = 0; i < XI; ++i)
    lds_dma16(x + xoff[i] + kt * 64, buf + (4 * i + wave) * 512);
}

template <bool DQ, int NS>
__device__ __forceinline__ void fwd_load_w(const NF4View& w, const uint8_t* const (&wp)[NS],
                                           const int64_t (&nrow)[NS], int64_t KT, int64_t kt, WStep<NS>& st) {
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    st.q[t] = *reinterpret_cast<const uint4*>(wp[t] + 32 * kt);
    const int64_t blk = nrow[t] * KT + kt;
    if (DQ) {
      st.qa[t] = static_cast<const uint8_t*>(w.scales)[blk];
      st.nv[t] = w.nested[blk >> 8];
    } else {
      st.nv[t] = static_cast<const float*>(w.scales)[blk];
    }
  }
}

template <bool DQ, int NS>
__device__ __forceinline__ void fwd_decode(const WStep<NS>& st, const float* d8s, float mu, bf16x8 (&bop)[NS][4]) {
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const float a = DQ ? __fadd_rn(__fmul_rn(d8s[st.qa[t]], st.nv[t]), mu) : st.nv[t];
    const Bf16Table tb = build_table(a);
    bop[t][0] = decode_word(st.q[t].x, tb);
    bop[t][1] = decode_word(st.q[t].y, tb);
    bop[t][2] = decode_word(st.q[t].z, tb);
    bop[t][3] = decode_word(st.q[t].w, tb);
  }
}

template <int MS, int NS>
__device__ __forceinline__ void fwd_mfma(const __bf16* xb, const bf16x8 (&bop)[NS][4], f32x16 (&acc)[MS][NS], int g,
                                         int l32) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int row = 32 * i + l32;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&xb[row * 64 + 8 * ((4 * g + j) ^ swz(row))]);
#pragma unroll
      for (int t = 0; t < NS; ++t)
        acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop[t][j], acc[i][t], 0, 0, 0);
    }
  }
}

// Forward y = x W_hat^T + s T B^T, K % 64 == 0. Tile (32 MS) x (128 NS): each of
// the 4 waves owns all 32 MS rows and 32 NS weight rows, so every weight row is
// decoded by exactly one wave and the decode cost is spread over MS 32x32 MFMA
// tiles. x arrives by direct global->LDS loads into two swizzled stages; weight
// codes for step k+2 are loaded and step k+1 is decoded while step k multiplies.
template <bool DQ, int MS, int NS>
__global__ __launch_bounds__(256, NS == 1 ? 2 : 1)
void k_fwd(const __bf16* __restrict__ x, int64_t M, int64_t K, int64_t N, NF4View w, const float* __restrict__ Bfac,
           int r, float s, const float* __restrict__ T, __bf16* __restrict__ y) {
  constexpr int BM = 32 * MS, WN = 32 * NS, BN = 4 * WN;
  constexpr int STAGE = BM * 64;   // bf16 per x stage
  constexpr int XI = BM / 32;      // 1 KB direct loads per wave per stage
  __shared__ __attribute__((aligned(16))) __bf16 xs0[STAGE];
  __shared__ __attribute__((aligned(16))) __bf16 xs1[STAGE];
  __shared__ float d8s[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t MT = (M + BM - 1) / BM, NT = (N + BN - 1) / BN;
  int64_t mt, nt;
  tile_coords(blockIdx.x, MT, NT, mt, nt);
  const int64_t m0 = mt * BM, n0 = nt * BN;
  const int64_t KT = K / 64;
  if (DQ) d8s[tid] = dyn8_value((uint32_t)tid);
  const float mu = DQ ? w.offset[0] : 0.0f;

  // Direct x loads: instruction i of this wave fills rows 8G..8G+7, G = 4i + wave;
  // lane l writes physical chunk l % 8 of row 8G + l / 8, i.e. logical chunk
  // (l % 8) ^ swz(row). Rows past M are clamped (their outputs are not stored).
  // (offsets relative to row m0, so they fit in 32 bits: rows < 256, K < 2^22)
  const __bf16* xt = x + m0 * K;
  int32_t xoff[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int row = 8 * (4 * i + wave) + (lane >> 3);
    const int64_t m = (m0 + row < M) ? row : M - 1 - m0;
    xoff[i] = (int32_t)(m * K) + 8 * ((lane & 7) ^ swz(row));
  }
  // weight rows of this lane (clamped past N)
  int64_t nrow[NS];
  const uint8_t* wp[NS];
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const int64_t n = n0 + wave * WN + 32 * t + l32;
    nrow[t] = n < N ? n : N - 1;
    wp[t] = w.codes + nrow[t] * (K / 2) + 16 * g;
  }

  f32x16 acc[MS][NS];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int t = 0; t < NS; ++t) acc[i][t] = f32x16{};

  WStep<NS> wa, wb;
  bf16x8 bopa[NS][4], bopb[NS][4];
  fwd_issue_x<XI>(xt, xoff, 0, xs0, wave);
  fwd_load_w<DQ, NS>(w, wp, nrow, KT, 0, wb);
  if (KT > 1) fwd_load_w<DQ, NS>(w, wp, nrow, KT, 1, wa);
  __syncthreads();
  fwd_decode<DQ, NS>(wb, d8s, mu, bopa);

  // Step kt multiplies one x stage with the decoded weights of step kt while the
  // next x stage lands in the other buffer, the codes of step kt + 2 are loaded
  // and the codes of step kt + 1 are decoded. Unrolled by two so that the two x
  // buffers and register sets keep fixed roles.
  int64_t kt = 0;
  // Steady state: every load and decode of both half-steps is in range, so the
  // body has no branches (keeps the accumulators in place across iterations).
  for (; kt + 3 < KT; kt += 2) {
    fwd_issue_x<XI>(xt, xoff, kt + 1, xs1, wave);
    fwd_load_w<DQ, NS>(w, wp, nrow, KT, kt + 2, wb);
    fwd_decode<DQ, NS>(wa, d8s, mu, bopb);
    fwd_mfma<MS, NS>(xs0, bopa, acc, g, l32);
    __syncthreads();
    fwd_issue_x<XI>(xt, xoff, kt + 2, xs0, wave);
    fwd_load_w<DQ, NS>(w, wp, nrow, KT, kt + 3, wa);
    fwd_decode<DQ, NS>(wb, d8s, mu, bopa);
    fwd_mfma<MS, NS>(xs1, bopb, acc, g, l32);
    __syncthreads();
  }
  // Last one to three steps.
  for (; kt < KT; kt += 2) {
    if (kt + 1 < KT) fwd_issue_x<XI>(xt, xoff, kt + 1, xs1, wave);
    if (kt + 2 < KT) fwd_load_w<DQ, NS>(w, wp, nrow, KT, kt + 2, wb);
    if (kt + 1 < KT) fwd_decode<DQ, NS>(wa, d8s, mu, bopb);
    fwd_mfma<MS, NS>(xs0, bopa, acc, g, l32);
    __syncthreads();
    if (kt + 1 >= KT) break;
    if (kt + 2 < KT) fwd_issue_x<XI>(xt, xoff, kt + 2, xs0, wave);
    if (kt + 3 < KT) fwd_load_w<DQ, NS>(w, wp, nrow, KT, kt + 3, wa);
    if (kt + 2 < KT) fwd_decode<DQ, NS>(wb, d8s, mu, bopa);
    fwd_mfma<MS, NS>(xs1, bopb, acc, g, l32);
    __syncthreads();
  }

  // LoRA: acc += (s T[m][:]) . B[n][:], as six bf16 MFMA products of three-part
  // splits of both factors (the products that reach fp32 precision).
  if (r > 0) {
    for (int rho0 = 0; rho0 < r; rho0 += 16) {
      const int avail = r - (rho0 + 8 * g);
      bf16x8 b1[NS], b2[NS], b3[NS];
#pragma unroll
      for (int t = 0; t < NS; ++t) load_split8(Bfac + nrow[t] * r + rho0 + 8 * g, avail, 1.0f, b1[t], b2[t], b3[t]);
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const int64_t m = (m0 + 32 * i + l32 < M) ? m0 + 32 * i + l32 : M - 1;
        bf16x8 a1, a2, a3;
        load_split8(T + m * r + rho0 + 8 * g, avail, s, a1, a2, a3);
#pragma unroll
        for (int t = 0; t < NS; ++t) {
          f32x16 c = acc[i][t];
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, b1[t], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b2[t], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b3[t], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b1[t], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b2[t], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1[t], c, 0, 0, 0);
          acc[i][t] = c;
        }
      }
    }
  }

  // Store: element e of accumulator (i, t) is row 32 i + 8 (e / 4) + 4 g + e % 4, column l32.
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const int64_t n = n0 + wave * WN + 32 * t + l32;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + 32 * i + (e >> 2) * 8 + g * 4 + (e & 3);
        if (m < M) y[m * N + n] = (__bf16)acc[i][t][e];
      }
  }
}

// Input gradient dX = dY W_hat + s U A, K % 64 == 0 and N % 64 == 0. Tile
// (32 MS tokens) x 128 weight inputs k; reduction over the weight outputs n in
// steps of 64. dY arrives by direct loads into two swizzled LDS stages. Wave w
// owns outputs k in [32 w, 32 w + 32) of the tile: each step its lane l decodes
// weight row n0 + l over those 32 columns (one 64-element block, one table) and
// stores the bf16 values transposed into the wave's own [k][n] LDS tile, from
// which the MFMA B operand (8 consecutive n per lane) is read. Only the wave
// itself reads its tile, and a wave's LDS operations complete in order, so the
// tile needs no barrier and a single buffer.
template <bool DQ, int MS>
__global__ __launch_bounds__(256, 2) void k_bwd(const __bf16* __restrict__ dy, int64_t M, int64_t K, int64_t N,
                                                NF4View w, const float* __restrict__ Afac, int r, float s,
                                                const float* __restrict__ U, __bf16* __restrict__ dx) {
  constexpr int BM = 32 * MS, BKO = 128;
  constexpr int STAGE = BM * 64;  // bf16 per dY stage
  constexpr int YI = BM / 32;     // 1 KB direct loads per wave per stage
  constexpr int WTP = 64;         // bf16 per row of a wave's [k][n] tile (16-byte chunks swizzled)
  __shared__ __attribute__((aligned(16))) __bf16 ys0[STAGE];
  __shared__ __attribute__((aligned(16))) __bf16 ys1[STAGE];
  __shared__ __attribute__((aligned(16))) __bf16 wts[4][32 * WTP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t MT = (M + BM - 1) / BM, KTL = (K + BKO - 1) / BKO;
  int64_t mt, kt_tile;
  tile_coords(blockIdx.x, MT, KTL, mt, kt_tile);
  const int64_t m0 = mt * BM, k0 = kt_tile * BKO;
  const int64_t NSTEP = N / 64, KB = K / 64;
  const float mu = DQ ? w.offset[0] : 0.0f;

  const __bf16* yt = dy + m0 * N;
  int32_t yoff[YI];
#pragma unroll
  for (int i = 0; i < YI; ++i) {
    const int row = 8 * (4 * i + wave) + (lane >> 3);
    const int64_t m = (m0 + row < M) ? row : M - 1 - m0;
    yoff[i] = (int32_t)(m * N) + 8 * ((lane & 7) ^ swz(row));
  }
  auto issue_y = [&](int64_t ns, __bf16* buf) __device__ {
#pragma unroll
    for (int i = 0; i < YI; ++i) lds_dma16(yt + yoff[i] + ns * 64, buf + (4 * i + wave) * 512);
  };
  // This lane's weight slice: row n = 64 ns + lane, columns kc .. kc + 31 (clamped past K).
  const int64_t kc = (k0 + 32 * wave < K) ? k0 + 32 * wave : K - 32;
  const uint8_t* wbase = w.codes + kc / 2;
  __bf16* wt = wts[wave];
  // 32 columns = 16 bytes of codes per lane
  auto load_w = [&](int64_t ns, uint4& q, uint32_t& qa, float& nv) __device__ {
    const int64_t n = 64 * ns + lane;
    q = *reinterpret_cast<const uint4*>(wbase + n * (K / 2));
    const int64_t blk = n * KB + kc / 64;
    if (DQ) {
      qa = static_cast<const uint8_t*>(w.scales)[blk];
      nv = w.nested[blk >> 8];
    } else {
      nv = static_cast<const float*>(w.scales)[blk];
    }
  };
  auto decode_store = [&](const uint4& q, uint32_t qa, float nv) __device__ {
    const float a = DQ ? __fadd_rn(__fmul_rn(dyn8_value(qa), nv), mu) : nv;
    const Bf16Table tb = build_table(a);
    const uint32_t words[4] = {q.x, q.y, q.z, q.w};
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // word j = columns 8j .. 8j + 7 -> tile rows k = 8j .. 8j + 7
      const u32x4 d = __builtin_bit_cast(u32x4, decode_word(words[j], tb));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k_a = 8 * j + 2 * e, k_b = k_a + 1;
        uint16_t* row0 = reinterpret_cast<uint16_t*>(wt + k_a * WTP + 8 * ((lane >> 3) ^ swz(k_a)) + (lane & 7));
        uint16_t* row1 = reinterpret_cast<uint16_t*>(wt + k_b * WTP + 8 * ((lane >> 3) ^ swz(k_b)) + (lane & 7));
        *row0 = (uint16_t)(d[e] & 0xFFFFu);
        *row1 = (uint16_t)(d[e] >> 16);
      }
    }
  };

  f32x16 acc[MS];
#pragma unroll
  for (int i = 0; i < MS; ++i) acc[i] = f32x16{};

  auto mfma_step = [&](const __bf16* yb) __device__ {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(&wt[l32 * WTP + 8 * ((4 * g + j) ^ swz(l32))]);
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const int row = 32 * i + l32;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&yb[row * 64 + 8 * ((4 * g + j) ^ swz(row))]);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
      }
    }
  };

  uint4 qa_, qb_;
  uint32_t sa = 0, sb = 0;
  float va = 0.0f, vb = 0.0f;
  issue_y(0, ys0);
  load_w(0, qa_, sa, va);
  if (NSTEP > 1) load_w(1, qb_, sb, vb);
  __syncthreads();
  decode_store(qa_, sa, va);

  int64_t ns = 0;
  for (; ns + 3 < NSTEP; ns += 2) {
    issue_y(ns + 1, ys1);
    load_w(ns + 2, qa_, sa, va);
    mfma_step(ys0);
    decode_store(qb_, sb, vb);
    __syncthreads();
    issue_y(ns + 2, ys0);
    load_w(ns + 3, qb_, sb, vb);
    mfma_step(ys1);
    decode_store(qa_, sa, va);
    __syncthreads();
  }
  for (; ns < NSTEP; ns += 2) {
    if (ns + 1 < NSTEP) issue_y(ns + 1, ys1);
    if (ns + 2 < NSTEP) load_w(ns + 2, qa_, sa, va);
    mfma_step(ys0);
    if (ns + 1 < NSTEP) decode_store(qb_, sb, vb);
    __syncthreads();
    if (ns + 1 >= NSTEP) break;
    if (ns + 2 < NSTEP) issue_y(ns + 2, ys0);
    if (ns + 3 < NSTEP) load_w(ns + 3, qb_, sb, vb);
    mfma_step(ys1);
    if (ns + 2 < NSTEP) decode_store(qa_, sa, va);
    __syncthreads();
  }

  // LoRA: acc += (s U[m][:]) . A[:][k] as six bf16 products of exact splits.
  const int64_t kcol = k0 + 32 * wave + l32;
  const bool kok = kcol < K;
  if (r > 0) {
    for (int rho0 = 0; rho0 < r; rho0 += 16) {
      const int avail = r - (rho0 + 8 * g);
      float bv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[e] = (e < avail && kok) ? Afac[(int64_t)(rho0 + 8 * g + e) * K + kcol] : 0.0f;
      bf16x8 b1, b2, b3;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 h, m_, l;
        split3(bv[e], h, m_, l);
        b1[e] = h;
        b2[e] = m_;
        b3[e] = l;
      }
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const int64_t m = (m0 + 32 * i + l32 < M) ? m0 + 32 * i + l32 : M - 1;
        bf16x8 a1, a2, a3;
        load_split8(U + m * r + rho0 + 8 * g, avail, s, a1, a2, a3);
        f32x16 c = acc[i];
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, b1, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b2, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b3, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b1, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b2, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c, 0, 0, 0);
        acc[i] = c;
      }
    }
  }
  if (!kok) return;
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t m = m0 + 32 * i + (e >> 2) * 8 + g * 4 + (e & 3);
      if (m < M) dx[m * K + kcol] = (__bf16)acc[i][e];
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
    const __bf16* dy = static_cast<const __bf16*>(g.a);
    __bf16* dx = static_cast<__bf16*>(g.out);
    const bool big = ceil_div(g.M, 256) * ceil_div(g.K, 128) >= 224;
#define NF4_BWD(MS)                                                                                             \
  do {                                                                                                          \
    const dim3 grid((unsigned)(ceil_div(g.M, 32 * MS) * ceil_div(g.K, 128)));                                 \
    if (dq)                                                                                                     \
      hipLaunchKernelGGL((k_bwd<true, MS>), grid, dim3(256), 0, st, dy, g.M, g.K, g.N, w, g.A, g.r, g.s, g.side, \
                         dx);                                                                                   \
    else                                                                                                        \
      hipLaunchKernelGGL((k_bwd<false, MS>), grid, dim3(256), 0, st, dy, g.M, g.K, g.N, w, g.A, g.r, g.s,       \
                         g.side, dx);                                                                           \
  } while (0)
    if (big)
      NF4_BWD(8);
    else
      NF4_BWD(4);
#undef NF4_BWD
    return launch_status();
  }
  const __bf16* x = static_cast<const __bf16*>(g.a);
  __bf16* y = static_cast<__bf16*>(g.out);
  // Tile choice: 256 x 256 unless that leaves most of the 256 CUs idle.
  const int64_t wg22 = ceil_div(g.M, 256) * ceil_div(g.N, 256);
  const int64_t wg21 = ceil_div(g.M, 256) * ceil_div(g.N, 128);
#define NF4_FWD(MS, NS)                                                                                         \
  do {                                                                                                          \
    const dim3 grid((unsigned)(ceil_div(g.M, 32 * MS) * ceil_div(g.N, 128 * NS)));                            \
    if (dq)                                                                                                     \
      hipLaunchKernelGGL((k_fwd<true, MS, NS>), grid, dim3(256), 0, st, x, g.M, g.K, g.N, w, g.B, g.r, g.s,     \
                         g.side, y);                                                                            \
    else                                                                                                        \
      hipLaunchKernelGGL((k_fwd<false, MS, NS>), grid, dim3(256), 0, st, x, g.M, g.K, g.N, w, g.B, g.r, g.s,    \
                         g.side, y);                                                                            \
  } while (0)
  if (wg22 < 0)
    NF4_FWD(8, 2);
  else if (wg21 >= 224)
    NF4_FWD(8, 1);
  else
    NF4_FWD(4, 1);
#undef NF4_FWD
  return launch_status();
}

}  // namespace nf4

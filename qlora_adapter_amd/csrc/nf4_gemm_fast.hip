// Fused NF4 GEMM kernels for gfx950 (bf16 operands, fp32 accumulate): the
// forward y = x W_hat^T + s T B^T and the input gradient dX = dY W_hat + s U A
// with W_hat decoded from the packed NF4 weights on the fly, never stored as a
// dense matrix (Aner docs "Native model adaptation and NF4", sections "Packed
// NF4 and the portable QLoRA profile" and "Adapter API").
//
// Common to all kernels here:
//  - A step of the reduction covers 64 weight inputs, exactly one quantization
//    block of every weight row. Each decoding lane builds the 16-entry bf16
//    table {bf16(fl32(C4[c] * a))} of its block once and turns nibbles into
//    bf16 with byte-select (v_perm_b32) lookups; the values are bit-identical
//    to nf4_dequantize's bf16 output.
//  - Activations (x or dY) arrive by direct global->LDS loads into two
//    double-buffered, XOR-swizzled stages.
//  - MFMA step j of lane group g = lane / 32 uses reduction indices
//    32 g + 8 j .. + 8 of the step for both operands (a fixed permutation of
//    the reduction order).
//  - The LoRA term is added to the fp32 accumulators with six bf16 MFMA
//    products of exact three-part splits of both factors before the single
//    bf16 rounding of the output.
//  - Workgroups are numbered so that each XCD gets a contiguous run of tiles,
//    visited in groups of 4 token tiles so that concurrently running
//    workgroups share activation and weight tiles in L2.
//
// k_gemm (problems with at least 128 tiles of 256 x 256): each step the
// workgroup decodes its weight slice once into LDS, and every wave multiplies
// 128 tokens x 64 outputs from the two stages (see the comment above k_gemm).
//
// k_fwd / k_bwd (smaller problems): 32 MS tokens per workgroup; in k_fwd each
// lane decodes the 32 weights its own B operand needs straight into registers,
// in k_bwd each wave decodes its 64 x 32 weight slice into a private
// transposed LDS tile. A long reduction over few output tiles (short
// sequences through a wide layer) is split in parts: each workgroup writes the
// fp32 partial sum of its part to a caller-provided workspace and k_split_sum
// adds the parts in order, adds the LoRA term and rounds once.
#include "nf4_device.hpp"

namespace nf4 {
namespace {

constexpr uint32_t kC4Bits[NF4_CODES_COUNT] = {NF4_CODES_LIST};

// 16-entry bf16 table of one block, split into low-byte and high-byte planes:
// lo[j] holds the low bytes of entries 4j..4j+3, hi[j] the high bytes.
struct Bf16Table {
  uint32_t lo[4], hi[4];
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16(a) | bf16(b) << 16, both rounded to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
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

// The same table built by two adjacent lanes that decode the same block: the
// lane of parity p multiplies the scale by its own eight code values cs =
// entries 8p .. 8p + 7 (per-lane constants), splits them into byte planes and
// takes the whole table from the pair through DPP quad permutations (the even
// lane's planes give entries 0..7, the odd lane's 8..15). Identical entries to
// build_table (each is the same rounded product). Every lane of the wave must
// be active.
__device__ __forceinline__ Bf16Table build_table_pair(float a, const float (&cs)[8]) {
  uint32_t P[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) P[i] = pack_bf16x2(__fmul_rn(cs[2 * i], a), __fmul_rn(cs[2 * i + 1], a));
  Bf16Table t;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int lo = (int)__builtin_amdgcn_perm(P[2 * j + 1], P[2 * j], 0x06040200u);
    const int hi = (int)__builtin_amdgcn_perm(P[2 * j + 1], P[2 * j], 0x07050301u);
    // quad_perm [0,0,2,2]: the even lane of each pair; [1,1,3,3]: the odd lane
    t.lo[j] = (uint32_t)__builtin_amdgcn_mov_dpp(lo, 0xA0, 0xF, 0xF, false);
    t.lo[2 + j] = (uint32_t)__builtin_amdgcn_mov_dpp(lo, 0xF5, 0xF, 0xF, false);
    t.hi[j] = (uint32_t)__builtin_amdgcn_mov_dpp(hi, 0xA0, 0xF, 0xF, false);
    t.hi[2 + j] = (uint32_t)__builtin_amdgcn_mov_dpp(hi, 0xF5, 0xF, 0xF, false);
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Decode one 32-bit code word (8 weights; weight 2p in the high nibble of byte
// p) into 8 bf16 values in the order w0 w2 w4 w6 w1 w3 w5 w7.
__device__ __forceinline__ u32x4 decode_word_eo(uint32_t w, const Bf16Table& t) {
  // Bit 3 of each index becomes a byte mask through the sign-replicating
  // selectors 8..11 of v_perm_b32 (bits 15, 31, 47, 63 of the 64-bit source
  // {S0, S1}): for the even weights the index top bits are bits 7, 15, 23, 31
  // of w, for the odd weights bits 3, 11, 19, 27.
  const uint32_t sel_e = (w >> 4) & 0x07070707u;
  const uint32_t msk_e = __builtin_amdgcn_perm(w << 8, w, 0x090B080Au);
  const uint32_t sel_o = w & 0x07070707u;
  const uint32_t w4 = w << 4;
  const uint32_t msk_o = __builtin_amdgcn_perm(w4 << 8, w4, 0x090B080Au);
  uint32_t el, eh, ol, oh;
  lookup4(t, sel_e, msk_e, el, eh);  // weights 0, 2, 4, 6
  lookup4(t, sel_o, msk_o, ol, oh);  // weights 1, 3, 5, 7
  u32x4 d;
  d[0] = __builtin_amdgcn_perm(eh, el, 0x05010400u);  // bf16(w0) | bf16(w2) << 16
  d[1] = __builtin_amdgcn_perm(eh, el, 0x07030602u);  // bf16(w4) | bf16(w6) << 16
  d[2] = __builtin_amdgcn_perm(oh, ol, 0x05010400u);  // bf16(w1) | bf16(w3) << 16
  d[3] = __builtin_amdgcn_perm(oh, ol, 0x07030602u);  // bf16(w5) | bf16(w7) << 16
  return d;
}

// Decode one 32-bit code word into 8 bf16 values in weight order. The lookups
// take weights 0 1 4 5 and 2 3 6 7 together (index bytes from w and w >> 4,
// bit-3 masks from w, w << 4, w << 8 and w << 12 through the sign-replicating
// selectors), so that one interleave of each pair's low and high bytes gives
// the weight order directly.
__device__ __forceinline__ bf16x8 decode_word(uint32_t w, const Bf16Table& t) {
  const uint32_t sh = w >> 4;
  const uint32_t sel_a = __builtin_amdgcn_perm(sh, w, 0x02060004u) & 0x07070707u;  // weights 0 1 4 5
  const uint32_t sel_b = __builtin_amdgcn_perm(sh, w, 0x03070105u) & 0x07070707u;  // weights 2 3 6 7
  const uint32_t msk_a = __builtin_amdgcn_perm(w << 12, w << 8, 0x0B090A08u);     // bits 7 3 23 19
  const uint32_t msk_b = __builtin_amdgcn_perm(w << 4, w, 0x0B090A08u);           // bits 15 11 31 27
  uint32_t al, ah, bl, bh;
  lookup4(t, sel_a, msk_a, al, ah);
  lookup4(t, sel_b, msk_b, bl, bh);
  u32x4 d;
  d[0] = __builtin_amdgcn_perm(ah, al, 0x05010400u);  // bf16(w0) | bf16(w1) << 16
  d[1] = __builtin_amdgcn_perm(bh, bl, 0x05010400u);  // w2 w3
  d[2] = __builtin_amdgcn_perm(ah, al, 0x07030602u);  // w4 w5
  d[3] = __builtin_amdgcn_perm(bh, bl, 0x07030602u);  // w6 w7
  return __builtin_bit_cast(bf16x8, d);
}

// A workgroup-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Tile coordinates of workgroup b: a contiguous run of tiles per XCD (workgroups
// are dealt to the 8 XCDs round-robin), then groups of GM token-tiles walked
// token-tile-fastest.
__device__ __forceinline__ int64_t xcd_order(int64_t b, int64_t nwg) {
  return (nwg % 8 == 0) ? (b % 8) * (nwg / 8) + b / 8 : b;
}

__device__ __forceinline__ void group_map(int64_t t, int64_t MT, int64_t NT, int64_t& mt, int64_t& nt) {
  constexpr int64_t GM = 4;
  const int64_t group = t / (GM * NT);
  const int64_t first_m = group * GM;
  const int64_t gm = (MT - first_m) < GM ? (MT - first_m) : GM;
  const int64_t within = t - group * GM * NT;
  mt = first_m + within % gm;
  nt = within / gm;
}

__device__ __forceinline__ void tile_coords(int64_t b, int64_t MT, int64_t NT, int64_t& mt, int64_t& nt) {
  group_map(xcd_order(b, MT * NT), MT, NT, mt, nt);
}

// Tile and reduction range of workgroup b when the reduction of S steps is
// split in `nsplit` parts: split index b % nsplit (the slice of the partial
// sums it writes), output tile from b / nsplit as in tile_coords, steps
// [kbeg, kbeg + nk) of ceil(S / nsplit) each.
__device__ __forceinline__ void split_coords(int64_t b, int64_t MT, int64_t NT, int nsplit, int64_t S, int64_t& mt,
                                             int64_t& nt, int64_t& sp, int64_t& kbeg, int64_t& nk) {
  const int64_t per = (S + nsplit - 1) / nsplit;
  const int64_t bb = xcd_order(b, MT * NT * nsplit);
  sp = bb % nsplit;
  group_map(bb / nsplit, MT, NT, mt, nt);
  kbeg = sp * per;
  nk = (S - kbeg) < per ? (S - kbeg) : per;
  if (nk < 1) {  // an empty part (the launcher never makes one): a zero partial sum
    kbeg = 0;
    nk = 0;
  }
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

// The small kernels' operand loads go through buffer resources: a wave-uniform
// base (the tile's first activation row, the codes, the block scales), the
// lanes' 32-bit byte offsets and a scalar step offset, so no per-lane 64-bit
// address arithmetic runs per step.
// (The record count is an unsigned 32-bit field: up to 4 GiB - 1 bytes, the
// codes' limit on this path; larger activation ranges are clamped, their
// offsets stay below 2^31.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = (uint32_t)(bytes < 0xffffffffll ? (bytes > 0 ? bytes : 0) : 0xffffffffll);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, 0x00020000);
}

template <int XI>
__device__ __forceinline__ void fwd_issue_x(const __amdgpu_buffer_rsrc_t rx, const uint32_t (&xb)[XI], int kt,
                                            __bf16* buf, int wave) {
#pragma unroll
  for (int i = 0; i < XI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(buf + (4 * i + wave) * 512),
                                             16, (int)xb[i], __builtin_amdgcn_readfirstlane(128 * kt), 0, 0);
}

template <bool DQ, int NS>
__device__ __forceinline__ void fwd_load_w(const __amdgpu_buffer_rsrc_t rc, const __amdgpu_buffer_rsrc_t rs,
                                           const float* __restrict__ nested, const uint32_t (&cb)[NS],
                                           const uint32_t (&bb)[NS], int kt, WStep<NS>& st) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  kt = __builtin_amdgcn_readfirstlane(kt);  // (the step is wave-uniform: scalar offsets)
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)cb[t], 32 * kt, 0);
    st.q[t] = make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
    if (DQ) {
      st.qa[t] = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)bb[t], kt, 0);
      st.nv[t] = nested[(bb[t] + (uint32_t)kt) >> 8];
    } else {
      st.nv[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(4 * bb[t]), 4 * kt, 0));
    }
  }
}

template <bool DQ, int NS>
__device__ __forceinline__ void fwd_scales(const WStep<NS>& st, const float* d8s, float mu, float (&a)[NS]) {
#pragma unroll
  for (int t = 0; t < NS; ++t) a[t] = DQ ? __fadd_rn(__fmul_rn(d8s[st.qa[t]], st.nv[t]), mu) : st.nv[t];
}

template <int NS>
__device__ __forceinline__ void fwd_decode_scaled(const WStep<NS>& st, const float (&sa)[NS], bf16x8 (&bop)[NS][4]) {
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const Bf16Table tb = build_table(sa[t]);
    bop[t][0] = decode_word(st.q[t].x, tb);
    bop[t][1] = decode_word(st.q[t].y, tb);
    bop[t][2] = decode_word(st.q[t].z, tb);
    bop[t][3] = decode_word(st.q[t].w, tb);
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

// Half-step barrier of k_fwd / k_bwd. Each wave issues the next activation
// stage's direct loads first and its NCL code/scale loads for a later step
// after them (scheduling barriers keep that order), so vmcnt(NCL) means the
// activation stage has landed in LDS while the code loads may still be in
// flight; lgkmcnt(0) completes the wave's LDS reads and writes before the
// other waves go on. (A plain __syncthreads would wait for every load.)
template <int NCL>
__device__ __forceinline__ void small_step_barrier() {
  static_assert(NCL < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(NCL | (7 << 4));  // vmcnt(NCL) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// Forward y = x W_hat^T + s T B^T, K % 64 == 0. Tile (32 MS) x (128 NS): each of
// the 4 waves owns all 32 MS rows and 32 NS weight rows, so every weight row is
// decoded by exactly one wave and the decode cost is spread over MS 32x32 MFMA
// tiles. x arrives by direct global->LDS loads into two swizzled stages; weight
// codes for step k+2 are loaded and step k+1 is decoded while step k multiplies.
template <bool DQ, int MS, int NS>
__global__ __launch_bounds__(256, NS == 1 ? 2 : 1)
void k_fwd(const __bf16* __restrict__ x, int64_t M, int64_t K, int64_t N, NF4View w, const float* __restrict__ Bfac,
           int r, float s, const float* __restrict__ T, __bf16* __restrict__ y, int nsplit, float* __restrict__ part) {
  constexpr int BM = 32 * MS, WN = 32 * NS, BN = 4 * WN;
  constexpr int STAGE = BM * 64;   // bf16 per x stage
  constexpr int XI = BM / 32;      // 1 KB direct loads per wave per stage
  __shared__ __attribute__((aligned(16))) __bf16 xs0[STAGE];
  __shared__ __attribute__((aligned(16))) __bf16 xs1[STAGE];
  __shared__ float d8s[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t MT = (M + BM - 1) / BM, NT = (N + BN - 1) / BN;
  int64_t mt, nt, sp, kbeg, KT;
  split_coords(blockIdx.x, MT, NT, nsplit, K / 64, mt, nt, sp, kbeg, KT);
  // (tile coordinates in scalar registers, so that the buffer resources built
  // from them are scalar: otherwise each buffer load runs in a lane loop)
  sp = uniform64(sp);
  kbeg = uniform64(kbeg);
  KT = uniform64(KT);
  const int64_t m0 = uniform64(mt * BM), n0 = uniform64(nt * BN);
  if (DQ) d8s[tid] = dyn8_value((uint32_t)tid);
  const float mu = DQ ? w.offset[0] : 0.0f;

  // Direct x loads: instruction i of this wave fills rows 8G..8G+7, G = 4i + wave;
  // lane l writes physical chunk l % 8 of row 8G + l / 8, i.e. logical chunk
  // (l % 8) ^ swz(row). Rows past M are clamped (their outputs are not stored).
  // (offsets relative to row m0, so they fit in 32 bits: rows < 256, K < 2^22)
  const int64_t xfirst = m0 * K + kbeg * 64;
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x + xfirst, 2 * (M * K - xfirst));
  uint32_t xb[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int row = 8 * (4 * i + wave) + (lane >> 3);
    const int64_t m = (m0 + row < M) ? row : M - 1 - m0;
    xb[i] = (uint32_t)(2 * (m * K) + 16 * ((lane & 7) ^ swz(row)));
  }
  // weight rows of this lane (clamped past N): byte offset of its code words
  // and index of its first block at step 0 (the codes are under 4 GiB)
  int64_t nrow[NS];
  uint32_t cb[NS], bb[NS];
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const int64_t n = n0 + wave * WN + 32 * t + l32;
    nrow[t] = n < N ? n : N - 1;
    cb[t] = (uint32_t)(nrow[t] * (K / 2) + 32 * kbeg + 16 * g);
    bb[t] = (uint32_t)(nrow[t] * (K / 64) + kbeg);
  }
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(w.codes, N * (K / 2));
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(w.scales, (DQ ? 1 : 4) * N * (K / 64));

  f32x16 acc[MS][NS];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int t = 0; t < NS; ++t) acc[i][t] = f32x16{};

  WStep<NS> wa, wb;
  bf16x8 bopa[NS][4], bopb[NS][4];
  fwd_issue_x<XI>(rx, xb, 0, xs0, wave);
  fwd_load_w<DQ, NS>(rc, rs, w.nested, cb, bb, 0, wb);
  if (KT > 1) fwd_load_w<DQ, NS>(rc, rs, w.nested, cb, bb, 1, wa);
  __syncthreads();
  fwd_decode<DQ, NS>(wb, d8s, mu, bopa);

  // Step kt multiplies one x stage with the decoded weights of step kt while the
  // next x stage lands in the other buffer, the codes of step kt + 2 are loaded
  // and the codes of step kt + 1 are decoded. Unrolled by two so that the two x
  // buffers and register sets keep fixed roles.
  int kt = 0;
  // Steady state: every load and decode of both half-steps is in range, so the
  // body has no branches (keeps the accumulators in place across iterations).
  // (The barriers wait only for the activation loads: the code loads issued
  // after them stay in flight into the next half-step, see small_step_barrier.)
  constexpr int NCL = NS * (DQ ? 3 : 2);
  for (; kt + 3 < KT; kt += 2) {
    float sc[NS];
    fwd_scales<DQ, NS>(wa, d8s, mu, sc);
    __builtin_amdgcn_sched_barrier(0);
    fwd_issue_x<XI>(rx, xb, kt + 1, xs1, wave);
    __builtin_amdgcn_sched_barrier(0);
    fwd_load_w<DQ, NS>(rc, rs, w.nested, cb, bb, kt + 2, wb);
    fwd_decode_scaled<NS>(wa, sc, bopb);
    fwd_mfma<MS, NS>(xs0, bopa, acc, g, l32);
    small_step_barrier<NCL>();
    fwd_scales<DQ, NS>(wb, d8s, mu, sc);
    __builtin_amdgcn_sched_barrier(0);
    fwd_issue_x<XI>(rx, xb, kt + 2, xs0, wave);
    __builtin_amdgcn_sched_barrier(0);
    fwd_load_w<DQ, NS>(rc, rs, w.nested, cb, bb, kt + 3, wa);
    fwd_decode_scaled<NS>(wb, sc, bopa);
    fwd_mfma<MS, NS>(xs1, bopb, acc, g, l32);
    small_step_barrier<NCL>();
  }
  __syncthreads();
  // Last one to three steps.
  for (; kt < KT; kt += 2) {
    if (kt + 1 < KT) fwd_issue_x<XI>(rx, xb, kt + 1, xs1, wave);
    if (kt + 2 < KT) fwd_load_w<DQ, NS>(rc, rs, w.nested, cb, bb, kt + 2, wb);
    if (kt + 1 < KT) fwd_decode<DQ, NS>(wa, d8s, mu, bopb);
    fwd_mfma<MS, NS>(xs0, bopa, acc, g, l32);
    __syncthreads();
    if (kt + 1 >= KT) break;
    if (kt + 2 < KT) fwd_issue_x<XI>(rx, xb, kt + 2, xs0, wave);
    if (kt + 3 < KT) fwd_load_w<DQ, NS>(rc, rs, w.nested, cb, bb, kt + 3, wa);
    if (kt + 2 < KT) fwd_decode<DQ, NS>(wb, d8s, mu, bopa);
    fwd_mfma<MS, NS>(xs1, bopb, acc, g, l32);
    __syncthreads();
  }

  // LoRA: acc += (s T[m][:]) . B[n][:], as six bf16 MFMA products of three-part
  // splits of both factors (the products that reach fp32 precision). In a
  // split reduction only part 0 adds it.
  if (r > 0 && sp == 0) {
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

  // Split reduction: this workgroup's fp32 partial sum goes to its slice of
  // `part`; k_split_sum adds the slices in order and rounds once.
  if (part) {
    float* pz = part + (sp * M) * N;
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const int64_t n = n0 + wave * WN + 32 * t + l32;
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t m = m0 + 32 * i + (e >> 2) * 8 + g * 4 + (e & 3);
          if (m < M) pz[m * N + n] = acc[i][t][e];
        }
    }
    return;
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

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Transposing 8-byte LDS read (ds_read_b64_tr_b16): within each 16-lane group,
// lane i receives element i % 4 of the 4-element pieces addressed by lanes
// 4 e + i / 4, e = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 __attribute__((address_space(3)))*)(p));
}

// Chunk swizzle of the small input-gradient kernel's [64 n][32 k] weight tile
// (four 16-byte chunks per 64-byte row, chunk c of row n at c ^ wsw(n)): the 8
// rows of one 128-byte store phase hit 8 different bank groups, and so do the
// two-chunk pieces of rows 4a .. 4a + 3 that one transposing read phase covers.
__device__ __forceinline__ int wsw(int n) { return (n & 2) | ((n >> 2) & 1); }

// Input gradient dX = dY W_hat + s U A, K % 64 == 0 and N % 64 == 0. Tile
// (32 MS tokens) x 128 weight inputs k; reduction over the weight outputs n in
// steps of 64. dY arrives by direct loads into two swizzled LDS stages. Wave w
// owns outputs k in [32 w, 32 w + 32) of the tile: each step its lane l decodes
// weight row n0 + l over those 32 columns (half a 64-element block, one table)
// into the wave's own [n][k] LDS tile as four 16-byte chunks, and the MFMA B
// operand (8 consecutive n for one k) is gathered with two transposing reads.
// Only the wave itself reads its tile, and a wave's LDS operations complete in
// order, so the tile needs no barrier and a single buffer.
template <bool DQ, int MS>
__global__ __launch_bounds__(256, 2) void k_bwd(const __bf16* __restrict__ dy, int64_t M, int64_t K, int64_t N,
                                                NF4View w, const float* __restrict__ Afac, int r, float s,
                                                const float* __restrict__ U, __bf16* __restrict__ dx, int nsplit,
                                                float* __restrict__ part) {
  constexpr int BM = 32 * MS, BKO = 128;
  constexpr int STAGE = BM * 64;  // bf16 per dY stage
  constexpr int YI = BM / 32;     // 1 KB direct loads per wave per stage
  constexpr int WTP = 32;         // bf16 per row n of a wave's [n][k] tile
  __shared__ __attribute__((aligned(16))) __bf16 ys0[STAGE];
  __shared__ __attribute__((aligned(16))) __bf16 ys1[STAGE];
  __shared__ __attribute__((aligned(16))) __bf16 wts[4][64 * WTP];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t MT = (M + BM - 1) / BM, KTL = (K + BKO - 1) / BKO;
  int64_t mt, kt_tile, sp, nbeg, NSTEP;
  split_coords(blockIdx.x, MT, KTL, nsplit, N / 64, mt, kt_tile, sp, nbeg, NSTEP);
  // (scalar tile coordinates, as in k_fwd)
  sp = uniform64(sp);
  nbeg = uniform64(nbeg);
  NSTEP = uniform64(NSTEP);
  const int64_t m0 = uniform64(mt * BM), k0 = uniform64(kt_tile * BKO);
  const int64_t KB = K / 64;
  const float mu = DQ ? w.offset[0] : 0.0f;

  // (operand loads through buffer resources: wave-uniform bases, 32-bit lane
  // offsets, scalar step offsets; dY offsets stay below 2^31, the codes under
  // 4 GiB)
  const int64_t yfirst = m0 * N + nbeg * 64;
  const __amdgpu_buffer_rsrc_t ry = buffer_rsrc(dy + yfirst, 2 * (M * N - yfirst));
  uint32_t yb[YI];
#pragma unroll
  for (int i = 0; i < YI; ++i) {
    const int row = 8 * (4 * i + wave) + (lane >> 3);
    const int64_t m = (m0 + row < M) ? row : M - 1 - m0;
    yb[i] = (uint32_t)(2 * (m * N) + 16 * ((lane & 7) ^ swz(row)));
  }
  auto issue_y = [&](int ns, __bf16* buf) __device__ {
    const int so = __builtin_amdgcn_readfirstlane(128 * ns);  // (wave-uniform: a scalar offset)
#pragma unroll
    for (int i = 0; i < YI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ry, (__attribute__((address_space(3))) void*)(buf + (4 * i + wave) * 512), 16, (int)yb[i], so, 0, 0);
  };
  // This lane's weight slice: row n = 64 ns + lane, columns kc .. kc + 31 (clamped past K).
  const int64_t kc = (k0 + 32 * wave < K) ? k0 + 32 * wave : K - 32;
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(w.codes, N * (K / 2));
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(w.scales, (DQ ? 1 : 4) * N * KB);
  // step 0's byte offset of the lane's codes and index of its block; a step
  // adds 64 rows
  const uint32_t cl = (uint32_t)((64 * nbeg + lane) * (K / 2) + kc / 2);
  const uint32_t bl = (uint32_t)((64 * nbeg + lane) * KB + kc / 64);
  const uint32_t cstep = (uint32_t)(64 * (K / 2)), bstep = (uint32_t)(64 * KB);
  __bf16* wt = wts[wave];
  // 32 columns = 16 bytes of codes per lane
  auto load_w = [&](int ns, uint4& q, uint32_t& qa, float& nv) __device__ {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    ns = __builtin_amdgcn_readfirstlane(ns);  // (the step is wave-uniform: scalar offsets)
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)cl, (int)(ns * cstep), 0);
    q = make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
    if (DQ) {
      qa = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)bl, (int)(ns * bstep), 0);
      nv = w.nested[(bl + ns * bstep) >> 8];
    } else {
      nv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(4 * bl), (int)(4 * ns * bstep), 0));
    }
  };
  // Block scale a' = fl32(fl32(D8[qa] nv) + mu). The D8 value is a gather from
  // the constant table (a memory load), issued at the start of the half-step
  // that decodes the block, ahead of that half-step's other loads, so its
  // latency overlaps the MFMAs. (An LDS copy of the table would take the
  // 256-token tile's LDS past two workgroups per CU.)
  auto d8_of = [&](uint32_t qa) __device__ { return DQ ? dyn8_value(qa) : 0.0f; };
  auto scale_of = [&](float d8, float nv) __device__ { return DQ ? __fadd_rn(__fmul_rn(d8, nv), mu) : nv; };
  const int wsl = wsw(lane);
  auto decode_store = [&](const uint4& q, float a) __device__ {
    const Bf16Table tb = build_table(a);
    const uint32_t words[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)  // word j = columns 8 j .. 8 j + 7 of row n = lane
      *reinterpret_cast<bf16x8*>(wt + lane * WTP + 8 * (j ^ wsl)) = decode_word(words[j], tb);
  };
  // B operand of MFMA step j: lane (g, k = l32) takes n = 32 g + 8 j + 4 h + e,
  // e = 0..3, from transposing read h; the lane's own piece is row
  // 32 g + 8 j + 4 h + (lane % 16) / 4, columns kq .. kq + 3.
  const int kq = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  f32x16 acc[MS];
#pragma unroll
  for (int i = 0; i < MS; ++i) acc[i] = f32x16{};

  // operand reads are issued in groups of up to four before their MFMAs (more
  // would cost the 256-token tile its second wave per SIMD)
  constexpr int RG = MS < 4 ? MS : 4;
  auto mfma_step = [&](const __bf16* yb) __device__ {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = 32 * g + 8 * j + 4 * h + ((lane & 15) >> 2);
        v[h] = lds_read_tr16(&wt[n * WTP + 8 * ((kq >> 3) ^ wsw(n)) + (kq & 7)]);
      }
      const bf16x8 b = bf16x8{v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
#pragma unroll
      for (int i0 = 0; i0 < MS; i0 += RG) {
        bf16x8 a[RG];
#pragma unroll
        for (int i = 0; i < RG; ++i) {
          const int row = 32 * (i0 + i) + l32;
          a[i] = *reinterpret_cast<const bf16x8*>(&yb[row * 64 + 8 * ((4 * g + j) ^ swz(row))]);
        }
#pragma unroll
        for (int i = 0; i < RG; ++i)
          acc[i0 + i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, acc[i0 + i], 0, 0, 0);
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
  decode_store(qa_, scale_of(d8_of(sa), va));

  int ns = 0;
  constexpr int NCL = DQ ? 3 : 2;
  for (; ns + 3 < NSTEP; ns += 2) {
    float d8 = d8_of(sb);
    __builtin_amdgcn_sched_barrier(0);
    issue_y(ns + 1, ys1);
    __builtin_amdgcn_sched_barrier(0);
    load_w(ns + 2, qa_, sa, va);
    mfma_step(ys0);
    decode_store(qb_, scale_of(d8, vb));
    small_step_barrier<NCL>();
    d8 = d8_of(sa);
    __builtin_amdgcn_sched_barrier(0);
    issue_y(ns + 2, ys0);
    __builtin_amdgcn_sched_barrier(0);
    load_w(ns + 3, qb_, sb, vb);
    mfma_step(ys1);
    decode_store(qa_, scale_of(d8, va));
    small_step_barrier<NCL>();
  }
  __syncthreads();
  for (; ns < NSTEP; ns += 2) {
    if (ns + 1 < NSTEP) issue_y(ns + 1, ys1);
    if (ns + 2 < NSTEP) load_w(ns + 2, qa_, sa, va);
    mfma_step(ys0);
    if (ns + 1 < NSTEP) decode_store(qb_, scale_of(d8_of(sb), vb));
    __syncthreads();
    if (ns + 1 >= NSTEP) break;
    if (ns + 2 < NSTEP) issue_y(ns + 2, ys0);
    if (ns + 3 < NSTEP) load_w(ns + 3, qb_, sb, vb);
    mfma_step(ys1);
    if (ns + 2 < NSTEP) decode_store(qa_, scale_of(d8_of(sa), va));
    __syncthreads();
  }

  const int64_t kcol = k0 + 32 * wave + l32;
  const bool kok = kcol < K;
  // LoRA: acc += (s U[m][:]) . A[:][k] as six bf16 products of exact splits (in
  // a split reduction, part 0 only).
  if (r > 0 && sp == 0) {
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
  // Split reduction: fp32 partial sums to this workgroup's slice of `part`.
  if (part) {
    float* pz = part + (sp * M) * K;
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + 32 * i + (e >> 2) * 8 + g * 4 + (e & 3);
        if (m < M) pz[m * K + kcol] = acc[i][e];
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t m = m0 + 32 * i + (e >> 2) * 8 + g * 4 + (e & 3);
      if (m < M) dx[m * K + kcol] = (__bf16)acc[i][e];
    }
}


// ---------------------------------------------------------------------------
// Shared-decode GEMM for large problems: 256 x 256 output tiles, 512 threads
// (8 waves, two per SIMD), reduction in steps of 64. Each step the workgroup
// decodes its weight slice once into LDS (two lanes per 64-weight block, each
// writing four 16-byte chunks) while the activation slice arrives by direct
// global->LDS loads; wave (wm, wn) = (w % 2, w / 2) owns 128 x 64 outputs as
// 4 x 2 accumulators of the 32x32x16 bf16 MFMA.
//  - Forward (BWD = false): activations x [M][K], output columns are weight rows
//    n, the decoded slice is [256 n][64 k] and the B operand (8 consecutive k of
//    one row n) is a plain 16-byte read.
//  - Input gradient (BWD = true): activations dY [M][N], output columns are
//    weight inputs k, the decoded slice is [64 n][256 k] in natural row order
//    with each 8-column chunk stored in the order 0 2 4 6 1 3 5 7 (the decoder's
//    natural output; only the output column of each accumulator lane changes),
//    and the B operand (8 consecutive n for one k) is gathered with two
//    transposing reads (ds_read_b64_tr_b16: within each 16-lane group, lane i
//    receives element i % 4 of the 4-element pieces addressed by lanes
//    4 e + i / 4, e = 0..3).
//  - Operand k order: MFMA step j of lane group g uses reduction indices
//    32 g + 8 j .. + 8 of the step for both operands.
//  - The weight fragment is the MFMA's first operand, so each accumulator holds
//    a transposed 32 x 32 tile: lane l (l % 32 = token row) holds output columns
//    8 (e / 4) + 4 (l / 32) + e % 4 in element e, four consecutive columns per
//    group of four elements, stored as one 8-byte write.
//  - The decode of the next slice is spread over the first two MFMA steps (two
//    code words after each group of eight MFMAs), so that it overlaps the
//    matrix core and its LDS stores complete before the step barrier.
constexpr int GT = 256;          // output tile edge
constexpr int GSTAGE = GT * 64;  // bf16 per activation stage (and per forward weight stage)

// The [64][256] input-gradient weight slice has a row pitch of WPB = 288 bf16
// (576 bytes) and keeps chunk c of row r at c ^ (r % 4), which only permutes
// chunks within aligned groups of 4, so the column tile enters the read address
// as a constant offset; the 8 lanes of a decoder store phase (4 rows x the two
// halves of a block) and the 16 lanes of a transposing read phase then hit
// different bank groups. (Counters still show LDS bank conflicts on this
// kernel, about a fifth of its LDS cycles; a 544-byte pitch and plain reads at
// the same addresses measured the same.)
constexpr int WPB = 288;
__device__ __forceinline__ int xbr(int r) { return r & 3; }

// Codes of the DW code words (8 DW weights of one block) a lane decodes per
// step, with the block's scale inputs.
template <int DW>
struct WCodes {
  uint32_t q[DW];
  uint32_t qa;  // dynamic8 code of the block (double quant)
  float nv;     // nested max (double quant) or absmax
};

// The step-dependent parts of the code address and block index are uniform
// across the wave (scalar offsets cso bytes and bso blocks), the lane parts
// 32-bit offsets (cofs bytes, blane blocks); codes and block scales are read
// through buffer resources (rc, rs), so no per-lane 64-bit address arithmetic
// runs per step. (Codes are under 4 GiB; every offset fits 32 bits.)
template <bool DQ, int DW>
__device__ __forceinline__ void gemm_load_codes(const __amdgpu_buffer_rsrc_t rc, const __amdgpu_buffer_rsrc_t rs,
                                                const float* __restrict__ nested, uint32_t cso, uint32_t cofs,
                                                uint32_t bso, uint32_t blane, WCodes<DW>& c) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int u = 0; u < DW / 4; ++u) {
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(cofs + 16 * u), (int)cso, 0);
    c.q[4 * u] = (uint32_t)v[0];
    c.q[4 * u + 1] = (uint32_t)v[1];
    c.q[4 * u + 2] = (uint32_t)v[2];
    c.q[4 * u + 3] = (uint32_t)v[3];
  }
  if (DQ) {
    c.qa = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)blane, (int)bso, 0);
    c.nv = nested[(bso + blane) >> 8];
  } else {
    c.nv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(4 * blane), (int)(4 * bso), 0));
  }
}

template <bool DQ, int DW>
__device__ __forceinline__ float gemm_block_scale(const WCodes<DW>& c, const float* d8s, float mu) {
  return DQ ? __fadd_rn(__fmul_rn(d8s[c.qa], c.nv), mu) : c.nv;
}

// Decode one code word and store its 8 weights as one 16-byte chunk, in weight
// order (EO = false) or in the order 0 2 4 6 1 3 5 7 (EO = true).
template <bool EO>
__device__ __forceinline__ void gemm_decode_word(uint32_t word, const Bf16Table& tb, __bf16* dst) {
  if (EO)
    *reinterpret_cast<u32x4*>(dst) = decode_word_eo(word, tb);
  else
    *reinterpret_cast<bf16x8*>(dst) = decode_word(word, tb);
}

// Weight column held at position p of an even/odd-ordered 8-column chunk.
__device__ __forceinline__ int eo_col(int p) { return 2 * (p & 3) + (p >> 2); }

// Activation loads of one step (NA per wave) through a buffer resource based at
// the tile's first row: aoff holds the lanes' byte offsets, soff the step's
// column offset (wave-uniform, so no per-lane address arithmetic); instruction i
// of wave v fills stage rows 8 (NW i + v) .. + 7.
__device__ __forceinline__ void lds_buffer_load16(const __bf16* base, int nbytes, uint32_t voff, uint32_t soff,
                                                  __bf16* dst) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(base), 0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

template <int NA, int NW>
__device__ __forceinline__ void gemm_issue_act(const __bf16* base, int nbytes, uint32_t soff,
                                               const uint32_t (&aoff)[NA], __bf16* buf, int wave) {
#pragma unroll
  for (int i = 0; i < NA; ++i) lds_buffer_load16(base, nbytes, aoff[i], soff, buf + (NW * i + wave) * 512);
}

// Operand fragments of MFMA step j: A for the wave's MS 32-row tiles, B for
// its NT 32-column tiles (the wave's columns start at stage column cw).
template <bool BWD, int MS, int NT>
__device__ __forceinline__ void gemm_frags(const __bf16* as, const __bf16* ws, int j, int lane, int wm, int cw,
                                           bf16x8 (&a)[MS], bf16x8 (&b)[NT]) {
  const int g = lane >> 5, l32 = lane & 31;
  const int q = 4 * g + j;  // reduction chunk of this lane at step j
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!BWD) {
      const int row = cw + 32 * t + l32;
      b[t] = *reinterpret_cast<const bf16x8*>(&ws[row * 64 + 8 * (q ^ swz(row))]);
    } else {
      const int col = cw + 32 * t + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      bf16x4 v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * q + 4 * h + ((lane & 15) >> 2);
        v[h] = lds_read_tr16(&ws[row * WPB + 8 * ((col >> 3) ^ xbr(row)) + (col & 7)]);
      }
      b[t] = bf16x8{v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
    }
  }
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int row = 32 * MS * wm + 32 * i + l32;
    a[i] = *reinterpret_cast<const bf16x8*>(&as[row * 64 + 8 * (q ^ swz(row))]);
  }
}

// One 64-deep step of the wave's 32 MS x 32 NT tile from the activation stage
// `as` and the decoded weight stage `ws`. With DEC, the lane's DW code words of
// the next step (codes c, block scale sc) are decoded into `wdst` along the
// way, DW / 2 words after each of the first two MFMA steps: word u goes to
// element wbase + 8 (u ^ wsx).
template <bool BWD, bool DEC, int MS, int NT, int DW>
__device__ __forceinline__ void gemm_step(const __bf16* as, const __bf16* ws, f32x16 (&acc)[MS][NT], int lane, int wm,
                                          int cw, const WCodes<DW>& c, float sc, __bf16* wdst, int wbase, int wsx,
                                          const float (&cs)[8]) {
  Bf16Table tb;
  // The operands of MFMA step j + 1 are read while step j multiplies.
  bf16x8 a[2][MS], b[2][NT];
  gemm_frags<BWD, MS, NT>(as, ws, 0, lane, wm, cw, a[0], b[0]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j < 3) gemm_frags<BWD, MS, NT>(as, ws, j + 1, lane, wm, cw, a[(j + 1) & 1], b[(j + 1) & 1]);
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j & 1][t], a[j & 1][i], acc[i][t], 0, 0, 0);
    // The decode runs in the first two MFMA steps, so that its LDS stores are
    // issued early and complete well before the step barrier waits for them
    // (measured faster than one word after each of the four steps).
    if (DEC && j < 2) {
      if (j == 0) tb = build_table_pair(sc, cs);
#pragma unroll
      for (int u = j * DW / 2; u < (j + 1) * DW / 2; ++u)
        gemm_decode_word<BWD>(c.q[u], tb, wdst + wbase + 8 * (u ^ wsx));
    }
  }
}

// Step barrier of k_gemm. Every wave issues its activation loads for the next
// stage first and its NCL code/scale loads for a later step after them (a
// scheduling barrier keeps that order), so vmcnt(NCL) means the activation
// loads have landed in LDS while the code loads may still be in flight; they
// are first used one step later. lgkmcnt(0) completes this wave's decoder
// stores and operand reads before the other waves go on.
template <int NCL>
__device__ __forceinline__ void gemm_step_barrier() {
  static_assert(NCL < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(NCL | (7 << 4));  // vmcnt(NCL) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// LoRA part of the output tile: acc += (s S[m][:]) . F(:, c) as six bf16
// products of exact three-part splits of both factors (the F split is the first
// operand, like the weights). The column of lane l32 in the F fragment is a
// stage column, mapped to its weight column for the input gradient.
template <bool BWD, int MS, int NT>
__device__ __forceinline__ void gemm_lora(f32x16 (&acc)[MS][NT], int64_t M, int64_t K, int64_t N,
                                          const float* __restrict__ F, int r, float s, const float* __restrict__ S,
                                          int64_t m0, int64_t cc, int lane, int wm) {
  const int g = lane >> 5, l32 = lane & 31;
  for (int rho0 = 0; rho0 < r; rho0 += 16) {
    const int avail = r - (rho0 + 8 * g);
    bf16x8 f1[NT], f2[NT], f3[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t c = cc + 32 * t + (BWD ? (l32 & ~7) + eo_col(l32 & 7) : l32);
      if (!BWD) {
        const int64_t n = c < N ? c : N - 1;
        load_split8(F + n * r + rho0 + 8 * g, avail, 1.0f, f1[t], f2[t], f3[t]);
      } else {
        const bool cok = c < K;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = (e < avail && cok) ? F[(int64_t)(rho0 + 8 * g + e) * K + c] : 0.0f;
          __bf16 x1, x2, x3;
          split3(v, x1, x2, x3);
          f1[t][e] = x1;
          f2[t][e] = x2;
          f3[t][e] = x3;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const int64_t mr = m0 + 32 * MS * wm + 32 * i + l32;
      const int64_t m = mr < M ? mr : M - 1;
      bf16x8 a1, a2, a3;
      load_split8(S + m * r + rho0 + 8 * g, avail, s, a1, a2, a3);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x16 c = acc[i][t];
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1[t], a3, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f2[t], a2, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f3[t], a1, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1[t], a2, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f2[t], a1, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1[t], a1, c, 0, 0, 0);
        acc[i][t] = c;
      }
    }
  }
}

// Four bf16 output values of accumulator elements 4k .. 4k + 3 (token row
// m0 + 32 MS wm + 32 i + l32, stage columns cc + 32 t + 8 k + 4 g + 0..3): in
// the forward pass four consecutive output columns. In the input gradient the
// even/odd chunk order puts weight columns 8 k + g + {0, 2, 4, 6} in lane group
// g; the two lane groups swap half of their values so that each again holds
// four consecutive columns (g = 0: 8 k .. 8 k + 3, g = 1: 8 k + 4 .. 8 k + 7).
template <bool BWD>
__device__ __forceinline__ void gemm_pack4(const f32x16& a, int k, int g, uint32_t& lo, uint32_t& hi) {
  if (!BWD) {
    lo = pack_bf16x2(a[4 * k], a[4 * k + 1]);
    hi = pack_bf16x2(a[4 * k + 2], a[4 * k + 3]);
  } else {
    const uint32_t p01 = pack_bf16x2(a[4 * k], a[4 * k + 1]);      // g0: c0 c2  g1: c1 c3
    const uint32_t p23 = pack_bf16x2(a[4 * k + 2], a[4 * k + 3]);  // g0: c4 c6  g1: c5 c7
    const uint32_t recv = (uint32_t)__shfl_xor((int)(g ? p01 : p23), 32);
    // g0: own c0 c2, received c1 c3; g1: own c5 c7, received c4 c6
    const uint32_t ev = g ? recv : p01, od = g ? p23 : recv;
    lo = __builtin_amdgcn_perm(od, ev, 0x05040100u);
    hi = __builtin_amdgcn_perm(od, ev, 0x07060302u);
  }
}

// Output tile store for C % 4 == 4 (8 bytes per lane): each group of four
// columns is one 8-byte buffer store; stores outside the output get an offset
// past the buffer's end, which the hardware drops, so the epilogue has no
// branches.
template <bool BWD, int MS, int NT>
__device__ __forceinline__ void gemm_store(const f32x16 (&acc)[MS][NT], __bf16* __restrict__ out, int64_t M, int64_t C,
                                           int64_t m0, int64_t cc, int lane, int wm) {
  const int g = lane >> 5, l32 = lane & 31;
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(out, 0, (int)(2 * M * C), 0x00020000);
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int64_t m = m0 + 32 * MS * wm + 32 * i + l32;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t lo, hi;
        gemm_pack4<BWD>(acc[i][t], k, g, lo, hi);
        const int64_t c = cc + 32 * t + 8 * k + 4 * g;
        const uint32_t off = (m < M && c < C) ? (uint32_t)(2 * (m * C + c)) : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b64(i32x2{(int)lo, (int)hi}, orsrc, (int)off, 0, 0);
      }
    }
  }
}

// Output tile store for C % 8 == 0, through LDS: the tile's 64 MS rows x 256
// columns of bf16 are written into the (no longer needed) stage buffers, rows
// 64 q .. + 63 into region q (ws0, ws1, as0, as1), 16-byte chunk c of row r at
// chunk position c ^ (r % 32); then every thread stores whole 16-byte chunks,
// 32 lanes per 512-byte row, so each store instruction writes full cache lines
// (the accumulator layout itself would scatter 8 bytes over 32 rows per
// instruction). Chunks outside the output are dropped as in gemm_store.
template <bool BWD, int MS, int NT>
__device__ __forceinline__ void gemm_store_tile(const f32x16 (&acc)[MS][NT], __bf16* __restrict__ out, int64_t M,
                                                int64_t C, int64_t m0, int64_t c0, int cw, int tid, int wm,
                                                __bf16* q0, __bf16* q1, __bf16* q2, __bf16* q3) {
  constexpr int NW = 16 / NT, BM = 64 * MS;
  const int lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  // every wave's LDS reads and every activation load into the stages are done
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int q = (32 * MS * wm + 32 * i) >> 6;  // wave-uniform region
    __bf16* reg = q == 0 ? q0 : q == 1 ? q1 : q == 2 ? q2 : q3;
    const int lr = (32 * i + l32) & 63;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t lo, hi;
        gemm_pack4<BWD>(acc[i][t], k, g, lo, hi);
        const int c = cw + 32 * t + 8 * k + 4 * g;
        *reinterpret_cast<uint2*>(&reg[lr * 256 + 8 * ((c >> 3) ^ (lr & 31)) + (c & 7)]) = make_uint2(lo, hi);
      }
  }
  __syncthreads();
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(out, 0, (int)(2 * M * C), 0x00020000);
  const int ch = tid & 31;
  const int64_t col = c0 + 8 * ch;
#pragma unroll
  for (int it = 0; it < BM / (2 * NW); ++it) {
    const int row = 2 * NW * it + (tid >> 5);
    const int q = (2 * NW * it) >> 6;  // the iteration's rows lie in one region
    const __bf16* reg = q == 0 ? q0 : q == 1 ? q1 : q == 2 ? q2 : q3;
    const int lr = row & 63;
    const uint4 v = *reinterpret_cast<const uint4*>(&reg[lr * 256 + 8 * (ch ^ (lr & 31))]);
    const int64_t m = m0 + row;
    const uint32_t off = (m < M && col < C) ? (uint32_t)(2 * (m * C + col)) : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b128(i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, orsrc, (int)off, 0, 0);
  }
}

// out = act W_hat^T + s S F^T (forward: act = x [M][K], F = B [N][r], S = T [M][r])
// or out = act W_hat + s S F (input gradient: act = dY [M][N], F = A [r][K],
// S = U [M][r]) for a 64 MS x 256 output tile per workgroup of NW = 16 / NT
// waves; wave w owns rows 32 MS (w % 2) .. + 32 MS and 32 NT columns from
// 32 NT (w / 2). The 256 x 256 tiles of the problem are numbered as in
// group_map; a workgroup of the MS = 4 kernel computes tile tbase +
// xcd_order(b), one of the MS = 2 kernel the upper or lower half of tile
// tbase + xcd_order(b) / 2 (so that a grid that does not fill its last round
// of the chip with whole tiles can finish with half-height ones). The
// reduction length (K or N) is a multiple of 64 and below 2^22, the packed
// codes are under 4 GiB, the output has a multiple of 4 columns and is under
// 2 GiB.
// Further projections of a grouped forward call, all reading the same
// activations (such as q, k and v, or gate and up): the column tiles of the
// call are those of the projections side by side, projection 0 (the kernel's
// own arguments) first; part i owns the column tiles from ct0 on and brings its
// weight, factor B, side product T, output, width and adapter rank and scale.
// Each output tile is computed exactly as in a call of its projection alone.
// With GS (input gradient), the call instead sums the input gradients of the
// projections: dX = sum_i (dY_i W_i + s_i U_i A_i), the reduction run as one
// segment per projection (its dY, weight and width) into the same
// accumulators, then every projection's adapter term, in projection order.
struct GemmPart {
  NF4View w;
  const float* F;
  const float* S;
  __bf16* out;
  const __bf16* act;  // (input-gradient sum: this projection's dY)
  int64_t N, ct0;
  int r;
  float s;
};
constexpr int kGroupMax = 4;
struct GemmGroup {
  GemmPart p[kGroupMax - 1];
  int n;       // projections in the call (1: projection 0 alone)
  int64_t ct;  // column tiles of all of them
};

template <bool BWD, bool DQ, int NT, int MS, bool GS = false>
__global__ __launch_bounds__(64 * (16 / NT), 1) void k_gemm(const __bf16* __restrict__ act, int64_t M, int64_t K,
                                                            int64_t N, NF4View w, const float* __restrict__ F, int r,
                                                            float s, const float* __restrict__ S,
                                                            __bf16* __restrict__ out, int64_t tbase,
                                                            GemmGroup grp) {
  constexpr int NW = 16 / NT;         // waves
  constexpr int BM = 64 * MS;         // tile rows
  constexpr int NA = BM / (8 * NW);   // activation loads per wave per step
  constexpr int DW = 2 * NT;          // code words decoded per lane per step
  constexpr int LPR = 8 / DW;         // lanes per weight block
  constexpr int NCL = DW / 4 + (DQ ? 2 : 1);  // code and scale loads per lane per step
  constexpr int WSTAGE = BWD ? 64 * WPB : GSTAGE;  // bf16 per decoded weight stage
  __shared__ __attribute__((aligned(16))) __bf16 as0[BM * 64];
  __shared__ __attribute__((aligned(16))) __bf16 as1[BM * 64];
  __shared__ __attribute__((aligned(16))) __bf16 ws0[WSTAGE];
  __shared__ __attribute__((aligned(16))) __bf16 ws1[WSTAGE];
  __shared__ float d8s[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, cw = 32 * NT * (wave >> 1);
  const int64_t MT = (M + GT - 1) / GT;
  const int64_t CT = (!BWD && grp.n > 1) ? grp.ct : ((BWD ? K : N) + GT - 1) / GT;
  int64_t mt, ct;
  const int64_t xb = xcd_order(blockIdx.x, gridDim.x);
  group_map(tbase + (MS == 4 ? xb : xb >> 1), MT, CT, mt, ct);
  if constexpr (!BWD) {  // the projection that owns column tile ct (workgroup-uniform)
    const int64_t cg = ct;
#pragma unroll
    for (int i = 0; i < kGroupMax - 1; ++i)
      if (i + 1 < grp.n && cg >= grp.p[i].ct0) {  // (ct0 ascending: the last match owns it)
        const GemmPart& q = grp.p[i];
        w = q.w;
        F = q.F;
        S = q.S;
        out = q.out;
        N = q.N;
        r = q.r;
        s = q.s;
        ct = cg - q.ct0;
      }
  }
  static_assert(!GS || BWD, "summed groups are input gradients");
  int64_t R = BWD ? N : K;
  const int64_t C = BWD ? K : N;
  // The tile origin is workgroup-uniform; stated explicitly (scalar registers),
  // so that the activation loads' buffer resource is scalar too (otherwise the
  // compiler may wrap each of those loads in a loop over distinct lane values).
  const int64_t m0 = uniform64(mt * GT + (MS == 4 ? 0 : BM * (xb & 1))), c0 = uniform64(ct * GT);
  const int64_t KB = K / 64;
  if (DQ && tid < 256) d8s[tid] = dyn8_value((uint32_t)tid);
  f32x16 acc[MS][NT];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f32x16{};

  // One reduction segment (GS: one per projection of the group, each with its
  // own dY, weight and width; the stages are reused once every wave is done
  // with the previous segment's).
  const int nseg = GS ? grp.n : 1;
  for (int seg = 0; seg < nseg; ++seg) {
    if constexpr (GS) {
      if (seg > 0) {
#pragma unroll
        for (int i = 0; i < kGroupMax - 1; ++i)
          if (seg == i + 1) {
            act = grp.p[i].act;
            w = grp.p[i].w;
            N = grp.p[i].N;
          }
        R = N;
        __syncthreads();
      }
    }
    const int64_t KT = R / 64;
    const float mu = DQ ? w.offset[0] : 0.0f;

    // Activation loads: lane l of instruction i writes physical chunk l % 8 of
    // stage row 8 (NW i + wave) + l / 8, i.e. logical chunk (l % 8) ^ swz(row).
    // Rows past M are clamped (not stored).
    // (every offset used stays below 256 rows x 2^23 bytes = 2^31)
    const int64_t abytes = 2 * (M - m0) * R;
    const __bf16* at = act + m0 * R;
    const int an = (int)(abytes < 0x7fffffff ? abytes : 0x7fffffff);
    uint32_t aoff[NA];
  #pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int row = 8 * (NW * i + wave) + (lane >> 3);
      const int64_t m = (m0 + row < M) ? row : M - 1 - m0;
      aoff[i] = (uint32_t)(2 * m * R) + 16 * ((lane & 7) ^ swz(row));
    }

    // This lane's code words per step (at w.codes + kt * cstep + cofs, block
    // kt * bstep + blane) and where its decoded chunks go: word u to element
    // wbase + 8 (u ^ wsx) of the weight stage.
    uint32_t cofs, blane;
    int64_t cstep, bstep;
    int wbase, wsx;
    if (!BWD) {  // weight row c0 + rl (clamped past N), words h DW .. of block kt, h = tid % LPR
      // Within each group of 8 rows, lane pairs take rows 0 2 4 6 1 3 5 7: the 8
      // lanes of one 128-byte store phase then write 8 different bank groups.
      const int t = tid / LPR, h = tid % LPR;
      const int rl = (t & ~7) | ((t & 3) << 1) | ((t >> 2) & 1);
      const int64_t n = (c0 + rl < N) ? c0 + rl : N - 1;
      cofs = (uint32_t)(n * (K / 2) + 4 * DW * h);
      blane = (uint32_t)(n * KB);
      cstep = 32;
      bstep = 1;
      wbase = rl * 64;
      wsx = swz(rl) ^ (DW * h);  // chunk (DW h + u) ^ swz(rl) = u ^ wsx for u < DW
    } else {  // weight row 64 kt + rr, columns kc .. kc + 8 DW - 1 (clamped past K): block wave / 2 of the
              // tile, half lane % 2, so that the two halves of a block are adjacent lanes (LPR = 2)
      const int rr = (lane >> 1) + 32 * (wave & 1), half = lane & 1;
      const int64_t kcol = c0 + 64 * (wave >> 1) + 8 * DW * half;
      const int64_t kc = kcol < K ? kcol : K - 8 * DW;
      cofs = (uint32_t)(rr * (K / 2) + kc / 2);
      blane = (uint32_t)(rr * KB + kc / 64);
      cstep = 64 * (K / 2);
      bstep = 64 * KB;
      wbase = rr * WPB + 64 * (wave >> 1) + 8 * DW * half;  // chunks 8 (wave / 2) + 4 half .. + 3, permuted by rr % 4
      wsx = xbr(rr);
    }


    // Step indices past the end are clamped to the last step: the surplus loads
    // and decodes land in buffers that are not read again, and the loop body has
    // a single path.
    // (KT < 2^16 and the codes under 4 GiB: step indices and offsets fit 32 bits)
    const int last = (int)KT - 1;
    const int second = last < 1 ? last : 1;
    const uint32_t csu = (uint32_t)cstep, bsu = (uint32_t)bstep;
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(w.codes), 0, (int)(uint32_t)(N * (K / 2)), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(w.scales), 0, (int)(uint32_t)((DQ ? 1 : 4) * N * KB), 0x00020000);
    WCodes<DW> ca, cb;
    gemm_issue_act<NA, NW>(at, an, 0, aoff, as0, wave);
    gemm_load_codes<DQ, DW>(rc, rs, w.nested, 0, cofs, 0, blane, ca);
    gemm_load_codes<DQ, DW>(rc, rs, w.nested, second * csu, cofs, second * bsu, blane, cb);
    // The two lanes of a weight block (adjacent, LPR = 2) share its table; this
    // lane's code values are entries 8 (lane % 2) ..
    static_assert(LPR == 2 && DW == 4, "pair tables need two lanes per block");
    float cs[8];
  #pragma unroll
    for (int k = 0; k < 8; ++k) cs[k] = __uint_as_float(kC4Bits[(lane & 1) ? 8 + k : k]);
    __syncthreads();  // d8s
    {
      const float sc0 = gemm_block_scale<DQ, DW>(ca, d8s, mu);
      const Bf16Table tb = build_table_pair(sc0, cs);
  #pragma unroll
      for (int u = 0; u < DW; ++u) gemm_decode_word<BWD>(ca.q[u], tb, ws0 + wbase + 8 * (u ^ wsx));
    }
    __syncthreads();  // stage 0 complete

    // Step kt multiplies stage kt % 2 while the activations of step kt + 1 land
    // in the other stage, the codes of step kt + 2 are loaded and the codes of
    // step kt + 1 are decoded into the other weight stage.
    for (int kt = 0; kt < (int)KT; kt += 2) {
      const int k1 = kt + 1 < last ? kt + 1 : last, k2 = kt + 2 < last ? kt + 2 : last,
                k3 = kt + 3 < last ? kt + 3 : last;
      // (The scale's table read precedes the activation loads: an LDS read
      // issued after them would wait for them.)
      float sc = gemm_block_scale<DQ, DW>(cb, d8s, mu);
      __builtin_amdgcn_sched_barrier(0);
      gemm_issue_act<NA, NW>(at, an, (uint32_t)(128 * k1), aoff, as1, wave);
      __builtin_amdgcn_sched_barrier(0);
      gemm_load_codes<DQ, DW>(rc, rs, w.nested, k2 * csu, cofs, k2 * bsu, blane, ca);
      gemm_step<BWD, true, MS, NT, DW>(as0, ws0, acc, lane, wm, cw, cb, sc, ws1, wbase, wsx, cs);
      gemm_step_barrier<NCL>();
      if (kt + 1 >= (int)KT) break;
      sc = gemm_block_scale<DQ, DW>(ca, d8s, mu);
      __builtin_amdgcn_sched_barrier(0);
      gemm_issue_act<NA, NW>(at, an, (uint32_t)(128 * k2), aoff, as0, wave);
      __builtin_amdgcn_sched_barrier(0);
      gemm_load_codes<DQ, DW>(rc, rs, w.nested, k3 * csu, cofs, k3 * bsu, blane, cb);
      gemm_step<BWD, true, MS, NT, DW>(as1, ws1, acc, lane, wm, cw, ca, sc, ws0, wbase, wsx, cs);
      gemm_step_barrier<NCL>();
    }
  }  // segments

  // (The two paths store separately, so that no join merges the accumulators.)
  const int64_t cc = c0 + cw;
  const bool whole = C % 8 == 0;
  if constexpr (GS) {  // every projection's adapter term, in projection order, then the store
    if (r > 0) gemm_lora<BWD, MS, NT>(acc, M, K, N, F, r, s, S, m0, cc, lane, wm);
#pragma unroll
    for (int i = 0; i < kGroupMax - 1; ++i)
      if (i + 1 < grp.n && grp.p[i].r > 0)
        gemm_lora<BWD, MS, NT>(acc, M, K, N, grp.p[i].F, grp.p[i].r, grp.p[i].s, grp.p[i].S, m0, cc, lane, wm);
    if (whole)
      gemm_store_tile<BWD, MS, NT>(acc, out, M, C, m0, c0, cw, tid, wm, ws0, ws1, as0, as1);
    else
      gemm_store<BWD, MS, NT>(acc, out, M, C, m0, cc, lane, wm);
    return;
  }
  if (r > 0) {
    gemm_lora<BWD, MS, NT>(acc, M, K, N, F, r, s, S, m0, cc, lane, wm);
    if (whole)
      gemm_store_tile<BWD, MS, NT>(acc, out, M, C, m0, c0, cw, tid, wm, ws0, ws1, as0, as1);
    else
      gemm_store<BWD, MS, NT>(acc, out, M, C, m0, cc, lane, wm);
  } else {
    if (whole)
      gemm_store_tile<BWD, MS, NT>(acc, out, M, C, m0, c0, cw, tid, wm, ws0, ws1, as0, as1);
    else
      gemm_store<BWD, MS, NT>(acc, out, M, C, m0, cc, lane, wm);
  }
}


}  // namespace

// Shapes the bf16 kernels of this file take: the reduction (K forward, N input
// gradient) and, in the input gradient, the output width in whole 64-wide
// blocks; k_fwd and k_bwd keep per-lane activation offsets (rows < 256 of the
// tile times the reduction length) in 32 bits, so the reduction stays below
// 2^22, and read the codes (under 4 GiB) through 32-bit buffer offsets. Other
// shapes go to the general kernel.
bool fast_shape_ok(int64_t K, int64_t N, bool backward) {
  if (N * (K / 2) >= (int64_t(1) << 32)) return false;  // codes read through 32-bit buffer offsets
  if (backward) return K % 64 == 0 && N % 64 == 0 && N < (int64_t(1) << 22);
  return K % FBK == 0 && K < (int64_t(1) << 22);
}

bool fast_linear_applies(const LinearArgs& g) { return g.dtype == NF4_BF16 && fast_shape_ok(g.K, g.N, g.backward); }

// Problems of more than half a round of 256 x 256 tiles (on 256 CUs) take the
// shared-decode kernel; up to 128 tiles the small-tile kernels measured faster
// (a 128-tile problem by 5-13% against the kernel's half-height tiles).
constexpr int64_t kGemmMinTiles = 129;

namespace {

// Output width C (y columns or dX columns) and reduction length R of a call.
inline void out_red(int64_t K, int64_t N, bool backward, int64_t& C, int64_t& R) {
  C = backward ? K : N;
  R = backward ? N : K;
}

bool use_gemm256(int64_t M, int64_t K, int64_t N, bool backward) {
  int64_t C, R;
  out_red(K, N, backward, C, R);
  const int64_t tiles = ceil_div(M, GT) * ceil_div(C, GT);
  // (lane offsets into the activations and codes are 32-bit, the output is
  // written with 8-byte buffer stores at 31-bit offsets)
  return tiles >= kGemmMinTiles && R < (int64_t(1) << 22) && N * (K / 2) < (int64_t(1) << 32) && C % 4 == 0 &&
         2 * M * C < (int64_t(1) << 31);
}

// Token tile (32 MS rows) and reduction split of the k_fwd / k_bwd path, from a
// sweep at 512 tokens over the Llama-8B shapes. The per-lane weight decode
// costs about as many VALU cycles per step as a 128-token tile's MFMAs, so
// small tiles are VALU-bound: a reduction of >= 32 steps of 64 whose 128-token
// tiles give fewer than 256 workgroups is split in parts over 128-token tiles
// (256-token tiles when the reduction is long, >= 128 steps, or when they
// alone give >= 200 workgroups in an input gradient), for about 512
// workgroups (about 256 in the forward pass, where fewer parts' partial sums
// to add outweigh the lost parallelism: -0.75 ms on the 512-token training
// step). Otherwise: 256-token tiles when they give >= 448 workgroups,
// else 128 or 64 when those give >= 200, else 32. Parts are a power of two, at
// most 8, of at least 8 steps; their fp32 partial sums are added by
// k_split_sum (part 0 carries the LoRA term).
struct SmallPlan {
  int ms;
  int nsplit;
};

SmallPlan small_plan(int64_t M, int64_t K, int64_t N, bool backward) {
  int64_t C, R;
  out_red(K, N, backward, C, R);
  const int64_t ct = ceil_div(C, 128), steps = R / 64;
  auto wg = [&](int ms) { return ceil_div(M, 32 * ms) * ct; };
  auto parts = [&](int64_t target, int ms) {
    int64_t ns = 1;
    while (2 * ns <= 8 && 2 * ns * wg(ms) <= target && steps / (2 * ns) >= 8) ns *= 2;
    return ns;
  };
  SmallPlan p{1, 1};
  if (wg(8) >= 448)
    p.ms = 8;
  else if (wg(4) >= 200)
    p.ms = 4;
  else if (wg(2) >= 200)
    p.ms = 2;
  if (C % 4 != 0 || steps < 32) return p;
  int64_t ns = 1;
  if (steps >= 128 || (backward && wg(8) >= 200)) {
    p.ms = 8;
    ns = parts(backward ? 512 : 256, 8);
  } else if (wg(4) < 256) {
    p.ms = 4;
    ns = parts(backward ? 512 : 256, 4);
  }
  if (ns >= 2) p.nsplit = (int)ceil_div(steps, ceil_div(steps, ns));  // every part non-empty
  return p;
}

// out[m][c] = bf16(sum_p part[p][m][c]), parts added in index order (part 0
// already holds the LoRA term). Four consecutive columns per thread (C % 4 == 0).
__global__ __launch_bounds__(256) void k_split_sum(const float* __restrict__ part, int nsplit, int64_t M, int64_t C,
                                                   __bf16* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q * 4 >= M * C) return;
  f32x4 v = *reinterpret_cast<const f32x4*>(part + q * 4);
  // the other parts' loads are all in flight (at most 8 parts: predicated,
  // not a chain of dependent loads), then added in part order
  f32x4 u[7];
#pragma unroll
  for (int p = 1; p < 8; ++p)
    u[p - 1] = p < nsplit ? *reinterpret_cast<const f32x4*>(part + (int64_t)p * M * C + q * 4) : f32x4{};
#pragma unroll
  for (int p = 1; p < 8; ++p)
    if (p < nsplit) {
      v[0] += u[p - 1][0];
      v[1] += u[p - 1][1];
      v[2] += u[p - 1][2];
      v[3] += u[p - 1][3];
    }
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x2 o;
  o[0] = pack_bf16x2(v[0], v[1]);
  o[1] = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2*>(out + q * 4) = o;
}

}  // namespace

int64_t linear_fast_workspace_bytes(int64_t M, int64_t K, int64_t N, bool backward) {
  if (!fast_shape_ok(K, N, backward)) return 0;
  if (use_gemm256(M, K, N, backward)) return 0;
  const SmallPlan p = small_plan(M, K, N, backward);
  if (p.nsplit < 2) return 0;
  int64_t C, R;
  out_red(K, N, backward, C, R);
  if (C % 4 != 0) return 0;
  return (int64_t)p.nsplit * M * C * (int64_t)sizeof(float);
}

namespace {

// The 256 x 256 shared-decode kernel over `tiles` output tiles (of projection 0
// and the further parts in grp): whole tiles fill complete rounds of the chip
// (one workgroup per CU); a last round of at most half the CUs is run as twice
// as many half tiles.
template <bool BWD, bool DQ, bool GS = false>
void launch_gemm256(const LinearArgs& g, const NF4View& w, const GemmGroup& grp, int64_t tiles, hipStream_t st) {
  const __bf16* a = static_cast<const __bf16*>(g.a);
  __bf16* o = static_cast<__bf16*>(g.out);
  const float* F = g.backward ? g.A : g.B;
  constexpr int NT = 2;  // 32x32 column tiles per wave (two waves per SIMD)
  const dim3 block(64 * (16 / NT));
  const int64_t cus = device_cu_count();
  const int64_t tail = tiles > cus ? tiles % cus : 0;
  const int64_t whole = (tail > 0 && 2 * tail <= cus) ? tiles - tail : tiles;
  hipLaunchKernelGGL((k_gemm<BWD, DQ, NT, 4, GS>), dim3((unsigned)whole), block, 0, st, a, g.M, g.K, g.N, w, F, g.r,
                     g.s, g.side, o, (int64_t)0, grp);
  if (whole < tiles)
    hipLaunchKernelGGL((k_gemm<BWD, DQ, NT, 2, GS>), dim3((unsigned)(2 * (tiles - whole))), block, 0, st, a, g.M,
                       g.K, g.N, w, F, g.r, g.s, g.side, o, whole, grp);
}

}  // namespace

// A grouped forward call takes the 256 x 256 kernel as one launch set when its
// 2 to 4 projections read the same bf16 activations, are all single or all
// double quantized, each meets the kernel's own bounds and together give more
// than half a round of tiles.
bool group_gemm_applies(const LinearArgs* g, int n) {
  if (n < 2 || n > kGroupMax) return false;
  int64_t ct = 0;
  for (int i = 0; i < n; ++i) {
    const LinearArgs& q = g[i];
    if (q.dtype != NF4_BF16 || q.backward || q.a != g[0].a || q.M != g[0].M || q.K != g[0].K) return false;
    if (q.W->double_quant != g[0].W->double_quant || !fast_shape_ok(q.K, q.N, false)) return false;
    if (q.N % 4 != 0 || 2 * q.M * q.N >= (int64_t(1) << 31)) return false;
    ct += ceil_div(q.N, GT);
  }
  return ceil_div(g[0].M, GT) * ct >= kGemmMinTiles;
}

// The grouped forward's matrix products (the side products T already written):
// projection 0 through the kernel's arguments, the others through GemmGroup.
int launch_linear_fast_group(const LinearArgs* g, int n, hipStream_t st) {
  GemmGroup grp{};
  grp.n = n;
  int64_t ct = ceil_div(g[0].N, GT);
  for (int i = 1; i < n; ++i) {
    GemmPart& q = grp.p[i - 1];
    q.w = make_view(g[i].W);
    q.F = g[i].B;
    q.S = g[i].side;
    q.out = static_cast<__bf16*>(g[i].out);
    q.N = g[i].N;
    q.ct0 = ct;
    q.r = g[i].r;
    q.s = g[i].s;
    ct += ceil_div(g[i].N, GT);
  }
  grp.ct = ct;
  const int64_t tiles = ceil_div(g[0].M, GT) * ct;
  const NF4View w = make_view(g[0].W);
  if (g[0].W->double_quant)
    launch_gemm256<false, true>(g[0], w, grp, tiles, st);
  else
    launch_gemm256<false, false>(g[0], w, grp, tiles, st);
  return launch_status();
}

// A summed input gradient takes the 256 x 256 kernel as one launch set when its
// 2 to 4 projections share M and K (the output), are all single or all double
// quantized, each meets the input-gradient bounds, and the output has more than
// half a round of tiles.
bool group_sum_applies(const LinearArgs* g, int n) {
  if (n < 2 || n > kGroupMax) return false;
  for (int i = 0; i < n; ++i) {
    const LinearArgs& q = g[i];
    if (q.dtype != NF4_BF16 || !q.backward || q.M != g[0].M || q.K != g[0].K) return false;
    if (q.W->double_quant != g[0].W->double_quant || !fast_shape_ok(q.K, q.N, true)) return false;
  }
  const int64_t M = g[0].M, K = g[0].K;
  return K % 4 == 0 && 2 * M * K < (int64_t(1) << 31) && ceil_div(M, GT) * ceil_div(K, GT) >= kGemmMinTiles;
}

// The summed input gradient's matrix products (the side products U already
// written), into g[0].out: projection 0 through the kernel's arguments, the
// others through GemmGroup.
int launch_linear_fast_sum(const LinearArgs* g, int n, hipStream_t st) {
  GemmGroup grp{};
  grp.n = n;
  for (int i = 1; i < n; ++i) {
    GemmPart& q = grp.p[i - 1];
    q.w = make_view(g[i].W);
    q.F = g[i].A;
    q.S = g[i].side;
    q.act = static_cast<const __bf16*>(g[i].a);
    q.N = g[i].N;
    q.r = g[i].r;
    q.s = g[i].s;
  }
  const int64_t tiles = ceil_div(g[0].M, GT) * ceil_div(g[0].K, GT);
  const NF4View w = make_view(g[0].W);
  if (g[0].W->double_quant)
    launch_gemm256<true, true, true>(g[0], w, grp, tiles, st);
  else
    launch_gemm256<true, false, true>(g[0], w, grp, tiles, st);
  return launch_status();
}

int launch_linear_fast(const LinearArgs& g, hipStream_t st) {
  const NF4View w = make_view(g.W);
  const bool dq = g.W->double_quant != 0;
  if (use_gemm256(g.M, g.K, g.N, g.backward)) {
    int64_t C, R;
    out_red(g.K, g.N, g.backward, C, R);
    const int64_t tiles = ceil_div(g.M, GT) * ceil_div(C, GT);
    GemmGroup one{};
    one.n = 1;
    if (g.backward) {
      if (dq) launch_gemm256<true, true>(g, w, one, tiles, st);
      else launch_gemm256<true, false>(g, w, one, tiles, st);
    } else {
      if (dq) launch_gemm256<false, true>(g, w, one, tiles, st);
      else launch_gemm256<false, false>(g, w, one, tiles, st);
    }
    return launch_status();
  }
  SmallPlan p = small_plan(g.M, g.K, g.N, g.backward);
  float* part = nullptr;
  if (p.nsplit > 1) {
    const int64_t need = linear_fast_workspace_bytes(g.M, g.K, g.N, g.backward);
    if (need <= 0 || !g.ws || g.ws_bytes < (size_t)need) return NF4_EWORKSPACE;
    part = static_cast<float*>(g.ws);
  }
  if (g.backward) {
    const __bf16* dy = static_cast<const __bf16*>(g.a);
    __bf16* dx = static_cast<__bf16*>(g.out);
#define NF4_BWD(MS)                                                                                               \
  do {                                                                                                            \
    const dim3 grid((unsigned)(ceil_div(g.M, 32 * MS) * ceil_div(g.K, 128) * p.nsplit));                        \
    if (dq)                                                                                                       \
      hipLaunchKernelGGL((k_bwd<true, MS>), grid, dim3(256), 0, st, dy, g.M, g.K, g.N, w, g.A, g.r, g.s, g.side,  \
                         dx, p.nsplit, part);                                                                     \
    else                                                                                                          \
      hipLaunchKernelGGL((k_bwd<false, MS>), grid, dim3(256), 0, st, dy, g.M, g.K, g.N, w, g.A, g.r, g.s, g.side, \
                         dx, p.nsplit, part);                                                                     \
  } while (0)
    switch (p.ms) {
      case 8: NF4_BWD(8); break;
      case 4: NF4_BWD(4); break;
      case 2: NF4_BWD(2); break;
      default: NF4_BWD(1); break;
    }
#undef NF4_BWD
    if (part)
      hipLaunchKernelGGL(k_split_sum, dim3((unsigned)ceil_div(g.M * g.K / 4, 256)), dim3(256), 0, st, part,
                         p.nsplit, g.M, g.K, dx);
    return launch_status();
  }
  const __bf16* x = static_cast<const __bf16*>(g.a);
  __bf16* y = static_cast<__bf16*>(g.out);
#define NF4_FWD(MS, NS)                                                                                           \
  do {                                                                                                            \
    const dim3 grid((unsigned)(ceil_div(g.M, 32 * MS) * ceil_div(g.N, 128 * NS) * p.nsplit));                   \
    if (dq)                                                                                                       \
      hipLaunchKernelGGL((k_fwd<true, MS, NS>), grid, dim3(256), 0, st, x, g.M, g.K, g.N, w, g.B, g.r, g.s,       \
                         g.side, y, p.nsplit, part);                                                              \
    else                                                                                                          \
      hipLaunchKernelGGL((k_fwd<false, MS, NS>), grid, dim3(256), 0, st, x, g.M, g.K, g.N, w, g.B, g.r, g.s,      \
                         g.side, y, p.nsplit, part);                                                              \
  } while (0)
  switch (p.ms) {
    case 8: NF4_FWD(8, 1); break;
    case 4: NF4_FWD(4, 1); break;
    case 2: NF4_FWD(2, 1); break;
    default: NF4_FWD(1, 1); break;
  }
#undef NF4_FWD
  if (part)
    hipLaunchKernelGGL(k_split_sum, dim3((unsigned)ceil_div(g.M * g.N / 4, 256)), dim3(256), 0, st, part,
                       p.nsplit, g.M, g.N, y);
  return launch_status();
}

}  // namespace nf4

// Internal declarations shared by the library's translation units (host side
// launchers and small device helpers). Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "../../include/nf4lora.h"
#include "nf4_tables.inc"

namespace nf4 {

constexpr int64_t kBlock = 64;    // elements per absmax block
constexpr int64_t kNested = 256;  // absmax values per nested block

// Host copies of the constant tables (bit patterns), used by nf4_code_tables.
extern const uint32_t kHostNF4[NF4_CODES_COUNT];
extern const uint32_t kHostDyn8[DYN8_CODES_COUNT];

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// The quantizer's workgroups each code 64 blocks (4096 weights) and leave one
// fp64 partial sum of their block maxima.
constexpr int64_t kQuantGroupBlocks = 64;
inline int64_t quant_groups(int64_t n) { return ceil_div(ceil_div(n, kBlock), kQuantGroupBlocks); }

// Scratch layout of nf4_quantize with double quantization: fp32 absmax[nb]
// (256-byte aligned) followed by the fp64 partial sums, one per 4096 weights.
inline size_t quantize_ws_bytes(int64_t n, int dq) {
  if (!dq) return 0;
  const int64_t nb = ceil_div(n, kBlock);
  return round_up(sizeof(float) * (size_t)nb, 256) + sizeof(double) * (size_t)quant_groups(n);
}

// Size of the fixed device scratch behind nf4_quantize_noalloc, and its device
// address on the current device (looked up once per device).
constexpr size_t kQuantizeScratchBytes = size_t(16) << 20;
int quantize_scratch(void** ptr);

// Launchers (return NF4_OK or NF4_EDEVICE). Arguments are already validated.
int launch_quantize(const float* w, int64_t n, const nf4_tensor* t, void* ws, int32_t* status, hipStream_t s);
// Workspace of nf4_quantize_many: per tensor the fp32 block maxima (double
// quantization only) and one fp64 partial per 4096 weights, each 256-byte
// aligned, then the per-tensor non-finite flags.
size_t quantize_many_ws_bytes(const nf4_tensor* t, int32_t count);
int launch_quantize_many(const float* const* w, const nf4_tensor* t, int32_t count, void* ws, int32_t* status,
                         hipStream_t s);
int launch_dequantize(const nf4_tensor* t, nf4_dtype dt, void* out, hipStream_t s);
int launch_dequantize_many(const nf4_tensor* t, void* const* outs, int32_t count, nf4_dtype dt, hipStream_t s);
int launch_embedding_rows(const nf4_tensor* E, int64_t V, int64_t D, const int64_t* ids, int64_t T, nf4_dtype dt,
                          void* out, int32_t* status, hipStream_t s);

struct LinearArgs {
  const void* a;        // x (forward) or dY (input gradient): [M, Kred]
  nf4_dtype dtype;
  int64_t M;
  int64_t K;            // weight inputs (columns of W)
  int64_t N;            // weight outputs (rows of W)
  const nf4_tensor* W;
  const float* A;       // [r, K]
  const float* B;       // [N, r]
  int32_t r;
  float s;
  void* out;            // y [M, N] or dX [M, K]
  float* side;          // T = x A^T or U = dY B, [M, r]
  bool backward;        // false: y = x W^T + s T B^T; true: dX = dY W + s U A
  void* ws;             // split-reduction partial sums (linear_fast_workspace_bytes), may be null
  size_t ws_bytes;
  float* side_part;     // partial sums of a split side product (side_split_ws_bytes), may be null
};
// Workspace the bf16 fused path needs for these sizes (0 for most shapes).
int64_t linear_fast_workspace_bytes(int64_t M, int64_t K, int64_t N, bool backward);
int launch_linear(const LinearArgs& a, hipStream_t s);
int launch_linear_group(const LinearArgs* a, int n, hipStream_t s);
// Summed input gradient of n projections into a[0].out; `tmp` holds n - 1
// outputs of M x K (dtype) when the one-launch path does not apply.
bool linear_bwd_sum_one_launch(const LinearArgs* a, int n);
int launch_linear_bwd_sum(const LinearArgs* a, int n, void* tmp, hipStream_t s);
// Side product alone: out[m][rho] = sum_i L[m][i] R[i][rho] (fp32 [M, r]), with
// R[i][rho] = fac[rho][i] (backward = false: T = x A^T, I = K) or fac[i][rho]
// (backward = true: U = dY B, I = N). `part` holds side_split_ws_bytes(M, I, r)
// (bf16, r > 32). Arguments are already validated.
int launch_side_product(const void* L, nf4_dtype dt, int64_t M, int64_t I, const float* fac, int32_t r, bool backward,
                        float* out, float* part, hipStream_t s);
// Workspace of the split bf16 side product for ranks beyond 32 (0 when the
// reduction over I is not split).
int64_t side_split_ws_bytes(int64_t M, int64_t I, int32_t r);

size_t lora_grad_ws(int64_t M, int64_t K, int64_t N, int32_t r, int fa);
int launch_lora_grad(const void* x, const void* dy, nf4_dtype dt, int64_t M, int64_t K, int64_t N, const float* t,
                     const float* u, int32_t r, float s, float* dA, float* dB, void* ws, hipStream_t st);

// LoRA-FA preconditioner P = pinv(A A^T + 1e-8 I): fp64 workspace of the
// K-sliced Gram matrices, then one inversion.
size_t lorafa_ws_bytes(int32_t r, int64_t K);
int launch_lorafa_preconditioner(const float* A, int32_t r, int64_t K, float* P, void* ws, hipStream_t st);

// One AdamW update of `count` adapters (validated) in one launch.
int launch_lora_adamw(const nf4_adamw& opt, const nf4_lora_state* ad, int32_t count, const float* grad_scale,
                      hipStream_t st);

// Decoder-layer operations (nf4_decoder.hip).
int launch_add_rmsnorm(const void* x, const void* res, nf4_dtype dt, int64_t rows, int64_t D, const float* gamma,
                       float eps, void* sum, void* y, float* rstd, hipStream_t st);
int launch_rmsnorm_bwd(const void* dy, const void* x, const float* rstd, nf4_dtype dt, int64_t rows, int64_t D,
                       const float* gamma, const void* dres, void* dx, hipStream_t st);
// Row strides (elements): rope's ld for x; attention's lq for q and dq, lk for
// k, v, dk and dv (o and dO are dense, hq d per row).
int launch_rope(void* x, nf4_dtype dt, int64_t S, int32_t heads, int32_t d, int64_t ld, double theta, int inverse,
                hipStream_t st);
int launch_attention_fwd(const void* q, const void* k, const void* v, nf4_dtype dt, int64_t S, int32_t hq,
                         int32_t hkv, int32_t d, int64_t lq, int64_t lk, void* o, float* lse, hipStream_t st);
int launch_attention_bwd(const void* dout, const void* q, const void* k, const void* v, const void* o,
                         const float* lse, nf4_dtype dt, int64_t S, int32_t hq, int32_t hkv, int32_t d, int64_t lq,
                         int64_t lk, float* delta, void* dq, void* dk, void* dv, hipStream_t st);
// Matrix-core attention (nf4_attention.hip): bf16 with head dim 32, 64, 96 or 128.
bool attention_mfma_supported(nf4_dtype dt, int32_t d);
int launch_attention_fwd_mfma(const void* q, const void* k, const void* v, int64_t S, int32_t hq, int32_t hkv,
                              int32_t d, int64_t lq, int64_t lk, void* o, float* lse, hipStream_t st);
int launch_attention_bwd_mfma(const void* dout, const void* q, const void* k, const void* v, const void* o,
                              const float* lse, int64_t S, int32_t hq, int32_t hkv, int32_t d, int64_t lq, int64_t lk,
                              float* delta, void* dq, void* dk, void* dv, hipStream_t st);
int launch_add3(const void* a, const void* b, const void* c, nf4_dtype dt, int64_t n, void* out, hipStream_t st);
// SwiGLU over rows of `width`: g, u, dg, du rows ld apart; a and da dense.
int launch_swiglu(const void* g, const void* u, nf4_dtype dt, int64_t rows, int64_t width, int64_t ld, void* a,
                  hipStream_t st);
int launch_swiglu_bwd(const void* da, const void* g, const void* u, nf4_dtype dt, int64_t rows, int64_t width,
                      int64_t ld, void* dg, void* du, hipStream_t st);
int launch_cross_entropy(const void* z, nf4_dtype dt, int64_t T, int64_t V, const int64_t* target, float* tok_loss,
                         float* loss, void* dz, int32_t* status, hipStream_t st);

inline int launch_status() { return hipGetLastError() == hipSuccess ? NF4_OK : NF4_EDEVICE; }

// Compute units of the current device (256 on MI355X).
int64_t device_cu_count();

}  // namespace nf4

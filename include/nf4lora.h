/*
 * nf4lora.h - C ABI of the MI355X (gfx950) NF4 double-quantized weight store
 * and the fused NF4 + LoRA linear layer.
 *
 * What the operations compute (the pages' definitions):
 *  - Storage. Aner docs "Native model adaptation and NF4", section "Packed NF4
 *    and the portable QLoRA profile": each matrix is split into 64-element
 *    blocks of its flattened row-major elements; each block stores its
 *    absolute maximum and one 4-bit index into the 16-value NF4 codebook per
 *    element, two indices per byte. With double quantization the block maxima
 *    are centred by their FP32 mean and coded with the signed dynamic8
 *    codebook in blocks of 256 maxima. Soup "NF4 Layer Streaming - Gate
 *    results", section "P3 is solved": N/2 + N/64 + N/4096 + 4 bytes per
 *    N-element weight; the two code tables are the same for every weight.
 *  - Decoding. Aner native training accelerated qualification (31 Oct 2026),
 *    key jit.kernel_identity: decoding is separately rounded fp32 operations
 *    (no fused multiply-add) and uses no global decoded scratch; Aner docs
 *    section "Mixed precision keeps stable state in FP32": decoded weights are
 *    rounded to the half type before the multiply, accumulation is FP32, and
 *    adapter contractions stay FP32.
 *  - Linear layer. Aner docs sections "Adapter API" and "LoRA FA includes
 *    gradient preconditioning": y = x W^T + s (x A^T) B^T with s = alpha/rank
 *    (rsLoRA: alpha/sqrt(rank)); the input gradient runs through the frozen
 *    base and no base-weight gradient exists; LoRA-FA freezes A.
 *
 * Exact format (readings where the pages are silent are marked READING):
 *  - n elements, nb = ceil(n/64) blocks, nn = ceil(nb/256) nested blocks, all
 *    over the flattened row-major matrix (blocks may straddle rows).
 *  - codes: ceil(n/2) bytes; element 2p is the HIGH nibble of byte p, element
 *    2p+1 the low nibble; an odd n leaves a zero low nibble (READING).
 *  - code of w in block b: a = max|w| over b; if a == 0 the code is 7 (the 0.0
 *    entry, READING); else x = w / a (IEEE fp32 division, round to nearest)
 *    and the code is the nearest NF4 entry, ties to the lower index (READING).
 *  - single quant: scales = fp32 absmax[nb].
 *  - double quant: offset mu = fp32( fp64 pairwise sum of absmax[0..nb), in
 *    index order, zero-padded to a power of two / nb ) (READING: the pages fix
 *    only "global FP32 mean"); c_b = fl32(absmax_b - mu); nested[j] =
 *    max |c_b| over nested block j; scales = u8 qabs[nb], qabs_b = nearest
 *    dynamic8 entry to fl32(c_b / nested[j]) (ties lower), or 127 (the 0.0
 *    entry) when nested[j] == 0.
 *  - decode: a'_b = absmax_b (single) or fl32(fl32(D8[qabs_b] * nested[j]) + mu)
 *    (double); w_hat = fl32(C4[code] * a'_b); bf16 output = round-to-nearest-
 *    even of w_hat.
 *
 * Conventions for every entry point:
 *  - Memory: every array argument is a DEVICE pointer owned by the caller,
 *    row-major and contiguous; the library allocates nothing, keeps no pointer
 *    after returning, and has no mutable global state except a once-per-device
 *    capability check. Calls are thread-safe.
 *  - Streams: work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream) and the call returns without synchronizing. Buffers must stay
 *    valid until the stream has run the work.
 *  - Shapes follow nn.Linear: x [M,K], weight [N,K] (N outputs, K inputs),
 *    y [M,N], A [r,K], B [N,r], T = x A^T [M,r], U = dY B [M,r]. A, B, T, U,
 *    dA, dB are fp32; x, y, dY, dX are of the call's dtype.
 *  - Alignment: packed `codes`, and x / y / dY / dX / out pointers, must be
 *    16-byte aligned (NF4_EALIGN otherwise). Any M, N, K >= 1 is accepted.
 *  - Errors: 0 (NF4_OK) or a negative NF4_E* code. Every argument error is
 *    detected on the host before anything is enqueued. Data-dependent errors
 *    (non-finite weights) are written to an optional device status word. No
 *    C++ exception crosses this interface.
 *  - Device: the current HIP device must be gfx950 (NF4_EUNSUPPORTED otherwise).
 */
#ifndef NF4LORA_H
#define NF4LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NF4LORA_ABI_VERSION 8

enum nf4_status {
  NF4_OK = 0,
  NF4_EINVAL = -1,       /* null pointer, non-positive size, bad rank or flag */
  NF4_EALIGN = -2,       /* a pointer that must be 16-byte aligned is not */
  NF4_EUNSUPPORTED = -3, /* dtype not F32/BF16, or the device is not gfx950 */
  NF4_EDEVICE = -4,      /* HIP runtime or launch failure */
  NF4_ENONFINITE = -5,   /* written to the status word: a weight was NaN/Inf */
  NF4_EWORKSPACE = -6    /* workspace pointer NULL or smaller than required */
};

typedef enum nf4_dtype { NF4_F32 = 0, NF4_BF16 = 1 } nf4_dtype;

/* Opaque stream handle: pass a hipStream_t (or NULL). */
typedef void* nf4_stream_t;

/* Byte counts of one packed matrix (see nf4_layout). */
typedef struct nf4_sizes {
  int64_t codes_bytes;     /* ceil(n/2) */
  int64_t scales_bytes;    /* 4*nb (single) or nb (double) */
  int64_t nested_bytes;    /* 4*nn (double) or 0 */
  int64_t offset_bytes;    /* 4 (double) or 0 */
  int64_t nb;              /* ceil(n/64) */
  int64_t nn;              /* ceil(nb/256) (double) or 0 */
  int64_t quantize_workspace_bytes; /* scratch nf4_quantize needs */
} nf4_sizes;

/* One packed matrix. All pointers are device pointers owned by the caller.
 * double_quant == 0: scales is float[nb]; nested and offset are unused.
 * double_quant == 1: scales is uint8_t[nb]; nested is float[nn]; offset
 *                    points to one float. */
typedef struct nf4_tensor {
  uint8_t* codes;
  void* scales;
  float* nested;
  float* offset;
  int64_t n;
  int32_t double_quant;
} nf4_tensor;

/* Sizes of the packed buffers for n elements (Aner docs "Packed NF4 and the
 * portable QLoRA profile"; Soup gate results "P3 is solved"). Host-only; no
 * device needed. Returns NF4_EINVAL for n < 1, a bad flag or out == NULL. */
int nf4_layout(int64_t n, int double_quant, nf4_sizes* out);

/* Host copies of the library's constant code tables (Aner native adaptation
 * qualification, key nf4: the exact 16-value NF4 codebook and the signed
 * dynamic8 nested codebook; Soup gate results "P3 is solved": the two tables
 * are the same for every weight): nf4[16] (QLoRA normal float, ascending,
 * nf4[7] == 0) and dyn8[256] (signed dynamic tree, ascending, dyn8[127] == 0,
 * dyn8[255] == +1). Both are host arrays the caller owns. Host-only; NF4_EINVAL
 * for a NULL argument. */
int nf4_code_tables(float nf4[16], float dyn8[256]);

/* Quantize n fp32 weights (Aner docs "Native model adaptation and NF4",
 * section "Packed NF4 and the portable QLoRA profile": 64-element blocks with
 * an absolute maximum each, nearest NF4 index per element, and with double
 * quantization the block maxima centred by their FP32 mean and coded with
 * dynamic8 in blocks of 256). `w` is a device fp32 array of n elements, the
 * flattened row-major matrix; `out` is a host struct whose device buffers are
 * sized by nf4_layout (out->n and out->double_quant must equal n and
 * double_quant). `workspace` (device, 256-byte aligned) must hold
 * quantize_workspace_bytes (may be NULL when that is 0). `status` (optional
 * device int32) is set to 0 and then to NF4_ENONFINITE if any weight is NaN or
 * infinite; the outputs are then unspecified. Argument errors (NULL, n < 1,
 * sizes that disagree, misalignment, small workspace) return before any
 * launch. Deterministic: repeated calls give identical bytes. */
int nf4_quantize(const float* w, int64_t n, int double_quant, const nf4_tensor* out, void* workspace,
                 size_t workspace_bytes, int32_t* status, nf4_stream_t stream);

/* nf4_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same operation, arguments and results as nf4_quantize (bit for bit),
 * without the workspace argument. Double quantization uses a fixed scratch
 * array in device memory that the library holds on each device it runs on
 * until the process ends (16 MiB); an n whose scratch would not fit
 * (n > nf4_quantize_noalloc_max_elements(), about 2.66e8 weights with double
 * quantization; single quantization needs none) returns NF4_EWORKSPACE before
 * any launch. The call allocates nothing. Every call on one device shares the
 * scratch: calls that overlap on a device (concurrent streams or threads) race
 * and must be serialized by the caller. */
int nf4_quantize_noalloc(const float* w, int64_t n, int double_quant, const nf4_tensor* out, int32_t* status,
                         nf4_stream_t stream);

/* Largest n that nf4_quantize_noalloc accepts with double quantization.
 * Host-only. */
int64_t nf4_quantize_noalloc_max_elements(void);

/* Decode all n weights of `w` into `out` (Aner native training accelerated
 * qualification, key jit.kernel_identity: separately rounded fp32 decode
 * steps, no fused multiply-add): w_hat = fl32(C4[code] * a'_b), bf16 output
 * by round-to-nearest-even of w_hat. `w` is a host struct of device buffers;
 * `out` a device array of n elements of out_dtype (F32 or BF16, else
 * NF4_EUNSUPPORTED), 16-byte aligned. Argument errors return before any
 * launch. */
int nf4_dequantize(const nf4_tensor* w, nf4_dtype out_dtype, void* out, nf4_stream_t stream);

#define NF4_MAX_TENSORS_PER_CALL 16

/* nf4_dequantize for `count` (1 to NF4_MAX_TENSORS_PER_CALL) packed matrices
 * in one kernel launch, all to out_dtype: outs[i] (device, 16-byte aligned)
 * receives the tensors[i].n decoded weights of tensors[i]. `tensors` and `outs`
 * are host arrays read during the call; each tensor is validated as
 * nf4_dequantize validates its argument, single and double quantization may
 * be mixed, and the outputs must not overlap. The results equal `count`
 * separate nf4_dequantize calls bit for bit; one launch decodes a layer's
 * matrices without a launch tail per matrix. */
int nf4_dequantize_many(const nf4_tensor* tensors, void* const* outs, int32_t count, nf4_dtype out_dtype,
                        nf4_stream_t stream);

/* nf4_quantize for `count` (1 to NF4_MAX_TENSORS_PER_CALL) matrices in three
 * kernel launches (Aner docs "Native model adaptation and NF4", section
 * "Packed NF4 and the portable QLoRA profile", as for nf4_quantize): w[i]
 * (device fp32, 16-byte aligned) holds the out[i].n weights of matrix i and
 * out[i] (host struct of device buffers sized by nf4_layout) receives them
 * with out[i].double_quant; single and double quantization may be mixed.
 * `w` and `out` are host arrays read during the call; the outputs must not
 * overlap each other or the inputs. `workspace` (device, 256-byte aligned)
 * must hold nf4_quantize_many_workspace_bytes(out, count). `status` (optional
 * device int32) is set to 0, or to NF4_ENONFINITE if any weight of any matrix
 * is NaN or infinite (that matrix's outputs are then unspecified). Each
 * matrix's bytes equal those of a separate nf4_quantize call; the launches
 * cover all matrices at once, so a layer's weights are packed without a
 * launch tail per matrix. Argument errors return before any launch. */
int nf4_quantize_many(const float* const* w, const nf4_tensor* out, int32_t count, void* workspace,
                      size_t workspace_bytes, int32_t* status, nf4_stream_t stream);

/* Workspace bytes nf4_quantize_many needs for these outputs (their n and
 * double_quant): per matrix the fp32 block maxima (double quantization only)
 * and one fp64 partial sum per 4096 weights, each rounded up to 256 bytes,
 * plus 256. Host-only; NF4_EINVAL (negative) for a NULL array, a count
 * outside 1..NF4_MAX_TENSORS_PER_CALL or an n < 1. */
int64_t nf4_quantize_many_workspace_bytes(const nf4_tensor* out, int32_t count);

/* Selected rows of a packed embedding table (Aner docs "Native model
 * adaptation and NF4": section "Packed NF4 and the portable QLoRA profile",
 * embeddings decode only the selected rows; section "Fused GPU NF4 decodes
 * inside the matrix kernel", the selected-row kernel decodes codes and nested
 * scales on the device with no decoded copy of the table). E holds a [V, D]
 * table (E->n == V*D, flattened row-major, so blocks may straddle rows); ids
 * is a device int64 array of T token ids (8-byte aligned); out [T, D] of
 * out_dtype receives out[t, :] = decoded row ids[t], bit-identical to those
 * rows of nf4_dequantize. `status` (optional device int32) is set to 0 and then
 * to NF4_EINVAL if an id is outside [0, V); that output row is written as
 * zeros and nothing outside the table is read. T == 0 launches only the
 * status reset. */
int nf4_embedding_rows(const nf4_tensor* E, int64_t V, int64_t D, const int64_t* ids, int64_t T, nf4_dtype out_dtype,
                       void* out, int32_t* status, nf4_stream_t stream);

/* Fused forward (Aner docs "Native model adaptation and NF4", sections
 * "Adapter API" and "Fused GPU NF4 decodes inside the matrix kernel"):
 * y = x W_hat^T + s (x A^T) B^T, W_hat decoded inside the matrix kernel (no
 * decoded copy of W is written to memory). x [M,K] and y [M,N] are `dtype`
 * (F32: fp32 weights; BF16: weights rounded to bf16 before the multiply,
 * section "Mixed precision keeps stable state in FP32"); accumulation is fp32.
 * W->n must equal N*K. r == 0 disables the adapter (A, B, t_out may be NULL);
 * r in [1, min(256, K, N)] requires A [r,K] and B [N,r] (fp32). t_out [M,r]
 * (fp32) is optional: when given it receives T = x A^T, kept for lora_grad;
 * when NULL, T lives in the workspace for the duration of the call.
 * `workspace` (device; a non-NULL workspace must be 256-byte aligned, else
 * NF4_EALIGN) holds nf4_linear_workspace_bytes(M, K, N, r, t_out ? 0 :
 * NF4_WS_NO_SIDE_OUT) bytes (NULL when that is 0), else NF4_EWORKSPACE. Every
 * argument error is returned before any launch. */
int nf4_linear_fwd(const void* x, nf4_dtype dtype, int64_t M, int64_t K, const nf4_tensor* W, int64_t N,
                   const float* A, const float* B, int32_t r, float s, void* y, float* t_out, void* workspace,
                   size_t workspace_bytes, nf4_stream_t stream);

/* Fused input gradient through the frozen base (same page, sections "Adapter
 * API" and "LoRA FA includes gradient preconditioning": the base weight gets
 * no gradient): dX = dY W_hat + s (dY B) A. dY [M,N] and dX [M,K] are `dtype`.
 * r == 0 disables the adapter; r >= 1 requires A [r,K] and B [N,r]. u_out
 * [M,r] (fp32) is optional: when given it receives U = dY B; when NULL, U
 * lives in the workspace. `workspace` holds nf4_linear_workspace_bytes(M, K,
 * N, r, NF4_WS_BACKWARD | (u_out ? 0 : NF4_WS_NO_SIDE_OUT)) bytes (NULL when
 * that is 0). */
int nf4_linear_bwd_input(const void* dy, nf4_dtype dtype, int64_t M, int64_t N, const nf4_tensor* W,
                         int64_t K, const float* A, const float* B, int32_t r, float s, void* dx,
                         float* u_out, void* workspace, size_t workspace_bytes, nf4_stream_t stream);

/* Flags of nf4_linear_workspace_bytes. */
#define NF4_WS_BACKWARD 1     /* the call is nf4_linear_bwd_input (else nf4_linear_fwd) */
#define NF4_WS_NO_SIDE_OUT 2  /* the call passes no t_out / u_out */

/* Device workspace (bytes; pass it 256-byte aligned) that nf4_linear_fwd or
 * nf4_linear_bwd_input (NF4_WS_BACKWARD) needs for these sizes and adapter
 * rank r (0: no adapter). Three parts, each rounded up to 256 bytes: (1) bf16
 * only: a long reduction over few output tiles (short sequences through a
 * wide layer, e.g. 512 tokens through a 4096 x 14336 projection) is split in
 * parts whose fp32 partial sums the workspace holds; (2) r > 32, a reduction
 * of at least 8192, or fewer than 4096 token rows with a reduction of at least
 * 2048: the side product's
 * reduction (over K forward, N backward) is split in parts whose fp32 partial
 * sums of the M x r product the workspace holds; (3) with
 * NF4_WS_NO_SIDE_OUT, M * r fp32 for the side product itself. Partial sums are
 * added in a fixed order, so results stay run-to-run identical. A call with a
 * NULL or smaller workspace than it needs fails with NF4_EWORKSPACE.
 * Host-only; a negative NF4_E* code for invalid sizes or flags. */
int64_t nf4_linear_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t r, int flags);

#define NF4_MAX_PROJECTIONS_PER_GROUP 4

/* nf4_linear_fwd for `count` (1 to NF4_MAX_PROJECTIONS_PER_GROUP) projections
 * of the same activations x [M,K] (a block's q, k and v, or gate and up; Aner
 * docs "Native model adaptation and NF4", section "Fused GPU NF4 decodes inside
 * the matrix kernel", applied to every adapted projection): for each i,
 * y[i] = x W[i]_hat^T + s[i] (x A[i]^T) B[i]^T with W[i]->n == N[i]*K, A[i],
 * B[i], r[i], s[i], t_out[i] as in nf4_linear_fwd (A, B and t_out may be NULL
 * arrays: all entries NULL). The host arrays are read during the call only.
 * The outputs y[i] must not overlap one another or x. For bf16, when the
 * projections are all single or all double quantized and together give more
 * than half a round of 256 x 256 output tiles, their matrix products run as
 * one launch set over all their tiles (each tile computed exactly as in a
 * call of its projection alone; the side products T run first, one per
 * projection); otherwise each projection runs as its own nf4_linear_fwd.
 * `workspace` (256-byte aligned) holds at most
 * nf4_linear_fwd_group_workspace_bytes(M, K, count, N, r) bytes (the sum of
 * each projection's nf4_linear_workspace_bytes with NF4_WS_NO_SIDE_OUT, each
 * rounded up to 256; projections that pass t_out need less), else
 * NF4_EWORKSPACE. Every argument error is returned before any launch. */
int nf4_linear_fwd_group(const void* x, nf4_dtype dtype, int64_t M, int64_t K, int32_t count,
                         const nf4_tensor* const* W, const int64_t* N, const float* const* A, const float* const* B,
                         const int32_t* r, const float* s, void* const* y, float* const* t_out, void* workspace,
                         size_t workspace_bytes, nf4_stream_t stream);

/* Workspace bytes of nf4_linear_fwd_group with no t_out (an upper bound for
 * every call with these sizes). Host-only; NF4_EINVAL (negative) for NULL
 * arrays, a count outside 1..NF4_MAX_PROJECTIONS_PER_GROUP or invalid sizes. */
int64_t nf4_linear_fwd_group_workspace_bytes(int64_t M, int64_t K, int32_t count, const int64_t* N, const int32_t* r);

/* Summed input gradient of `count` (1 to NF4_MAX_PROJECTIONS_PER_GROUP)
 * projections of one activation (the gradient a block's x receives from q, k
 * and v, or from gate and up; same page, sections "Adapter API" and "Fused GPU
 * NF4 decodes inside the matrix kernel"): dX = sum_i (dY[i] W[i]_hat +
 * s[i] (dY[i] B[i]) A[i]), dY[i] [M,N[i]] and dX [M,K] `dtype`, W[i]->n ==
 * N[i]*K, A[i], B[i], r[i], s[i], u_out[i] as in nf4_linear_bwd_input (A, B
 * and u_out may be NULL arrays: all entries NULL). The host arrays are read
 * during the call only; dX must not overlap any dY[i]. For bf16, when the
 * projections are all single or all double quantized, each N[i] is a multiple
 * of 64 and dX has more than half a round of 256 x 256 tiles, the products
 * run as one launch set whose fp32 accumulators take every projection's
 * reduction in turn and then every adapter term in projection order (one
 * rounding to bf16); otherwise each projection runs as its own
 * nf4_linear_bwd_input (projection 0 into dX, the others into the workspace)
 * and the parts are added in projection order, each rounded to `dtype` first.
 * `workspace` (256-byte aligned) holds at most
 * nf4_linear_bwd_input_sum_workspace_bytes(M, K, count, N, r, dtype) bytes,
 * else NF4_EWORKSPACE. Every argument error is returned before any launch. */
int nf4_linear_bwd_input_sum(const void* const* dy, nf4_dtype dtype, int64_t M, int64_t K, int32_t count,
                             const nf4_tensor* const* W, const int64_t* N, const float* const* A,
                             const float* const* B, const int32_t* r, const float* s, void* dx,
                             float* const* u_out, void* workspace, size_t workspace_bytes, nf4_stream_t stream);

/* Workspace bytes of nf4_linear_bwd_input_sum with no u_out, on either path
 * (an upper bound for every call with these sizes): each projection's
 * nf4_linear_workspace_bytes with NF4_WS_BACKWARD | NF4_WS_NO_SIDE_OUT and
 * count - 1 outputs of M x K `dtype`, each rounded up to 256. Host-only;
 * NF4_EINVAL (negative) for NULL arrays, a count outside
 * 1..NF4_MAX_PROJECTIONS_PER_GROUP or invalid sizes; NF4_EUNSUPPORTED for an
 * unknown dtype. */
int64_t nf4_linear_bwd_input_sum_workspace_bytes(int64_t M, int64_t K, int32_t count, const int64_t* N,
                                                 const int32_t* r, nf4_dtype dtype);

/* LoRA factor gradients (Aner docs "Native model adaptation and NF4", sections
 * "Adapter API" and "LoRA FA includes gradient preconditioning"):
 * dA = s U^T x [r,K] and dB = s dY^T T [N,r] (fp32), with T = x A^T and
 * U = dY B, sums over the M tokens in a fixed order (no atomics, run-to-run
 * identical). x [M,K] and dY [M,N] are `dtype`; A [r,K], B [N,r], t and u
 * [M,r] are fp32.
 *  - LoRA-FA (A frozen): dA == NULL; only dB is computed and u, B are unused.
 *  - t (from nf4_linear_fwd) may be NULL: T is then recomputed from x and A.
 *  - u (from nf4_linear_bwd_input) may be NULL when dA is wanted: U is then
 *    recomputed from dY and B.
 *  - x is required unless LoRA-FA with t given; A is required when t is NULL;
 *    B when u is NULL and dA is wanted (NF4_EINVAL otherwise).
 * `workspace` (device, 256-byte aligned) must hold
 * lora_grad_workspace_bytes(M, K, N, r, dA == NULL, recompute) bytes, where
 * recompute has NF4_RECOMPUTE_T set when t is NULL and NF4_RECOMPUTE_U when u
 * is NULL and dA is wanted. Every argument error is returned before any
 * launch. */
#define NF4_RECOMPUTE_T 1
#define NF4_RECOMPUTE_U 2
int lora_grad(const void* x, const void* dy, nf4_dtype dtype, int64_t M, int64_t K, int64_t N, const float* A,
              const float* B, const float* t, const float* u, int32_t r, float s, float* dA, float* dB,
              void* workspace, size_t workspace_bytes, nf4_stream_t stream);

/* Workspace bytes lora_grad needs for these sizes (fa != 0: LoRA-FA;
 * recompute: NF4_RECOMPUTE_T | NF4_RECOMPUTE_U as above). Returns a negative
 * NF4_E* code for invalid sizes. Host-only. */
int64_t lora_grad_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t r, int fa, int recompute);

/* Hyperparameters of one AdamW update (host struct, read during the call).
 * The update is the decoupled-decay form with bias-corrected moments:
 *   p <- p (1 - lr wd); m <- b1 m + (1 - b1) g; v <- b2 v + (1 - b2) g^2;
 *   p <- p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
 * The bias corrections and 1 - lr wd are formed in fp64 on the host and
 * rounded once to fp32; the per-entry arithmetic is fp32. */
typedef struct nf4_adamw {
  float lr;           /* learning rate, finite, >= 0 */
  float beta1;        /* first-moment decay, in [0, 1) */
  float beta2;        /* second-moment decay, in [0, 1) */
  float eps;          /* added to the root of the corrected second moment, finite, > 0 */
  float weight_decay; /* decoupled decay coefficient, finite, >= 0 */
  int64_t step;       /* 1-based index t of this update */
} nf4_adamw;

/* Workspace bytes lorafa_preconditioner needs for A [r,K] (r in [1, 256],
 * K >= 1); a negative NF4_E* code for invalid sizes. Host-only. */
int64_t lorafa_preconditioner_workspace_bytes(int32_t r, int64_t K);

/* LoRA-FA preconditioner (Aner docs "Native model adaptation and NF4", section
 * "LoRA FA includes gradient preconditioning"): with A frozen, the gradient of
 * B is multiplied by s^-2 pinv(A A^T + 1e-8 I) before the Adam moments, and
 * that r x r matrix is computed once and stored with the adapter. This call
 * computes P = (A A^T + 1e-8 I)^-1 (the damped Gram matrix is positive
 * definite, so its pseudo-inverse is its inverse; no singular value is cut):
 * A [r,K] fp32, P [r,r] fp32 (written), the Gram matrix accumulated and
 * inverted in fp64. `workspace` (256-byte aligned) must hold
 * lorafa_preconditioner_workspace_bytes(r, K) bytes. Deterministic. */
int lorafa_preconditioner(const float* A, int32_t r, int64_t K, float* P, void* workspace, size_t workspace_bytes,
                          nf4_stream_t stream);

/* One fused AdamW update of a LoRA adapter, in place (same page, sections
 * "Adapter API", "LoRA FA includes gradient preconditioning" and "Mixed
 * precision keeps stable state in FP32": FP32 parameters and moments).
 *  - LoRA: A [r,K], dA, mA, vA and B [N,r], dB, mB, vB all given; both factors
 *    take an AdamW update with their own gradients.
 *  - LoRA-FA: A, dA, mA and vA all NULL (A is frozen and has no moments); only
 *    B is updated. With `precond` (P [r,r] from lorafa_preconditioner) the
 *    gradient of B is first replaced by s^-2 dB P, s the adapter scale
 *    (finite, non-zero) used in the forward pass. `precond` requires LoRA-FA.
 *  - grad_scale: optional device fp32 scalar that multiplies every gradient
 *    first (a clipping or loss-scale factor); NULL means 1.
 * Moments must hold zeros before step 1. Every array is a 16-byte aligned
 * fp32 device array; gradients and P are read only. One kernel launch; entries
 * are independent, so the result does not depend on the launch shape. */
int lora_adamw_step(const nf4_adamw* opt, int32_t r, int64_t K, int64_t N, float* A, const float* dA, float* mA,
                    float* vA, float* B, const float* dB, float* mB, float* vB, const float* precond, float s,
                    const float* grad_scale, nf4_stream_t stream);

/* One adapter's tensors for lora_adamw_step_many; each field means what the
 * argument of the same name means for lora_adamw_step. */
typedef struct nf4_lora_state {
  int32_t r;
  int64_t K;
  int64_t N;
  float* A;
  const float* dA;
  float* mA;
  float* vA;
  float* B;
  const float* dB;
  float* mB;
  float* vB;
  const float* precond;
  float s;
} nf4_lora_state;

#define NF4_MAX_ADAPTERS_PER_CALL 16

/* lora_adamw_step for `count` adapters (1 to NF4_MAX_ADAPTERS_PER_CALL) with
 * the same hyperparameters and grad_scale, in one kernel launch: the update of
 * a layer's adapters at the cost of one launch. `adapters` is a host array read
 * during the call; each entry is validated as lora_adamw_step validates its
 * arguments, and no tensor may overlap another. Entries are independent, so the
 * result equals `count` separate lora_adamw_step calls bit for bit. */
int lora_adamw_step_many(const nf4_adamw* opt, const nf4_lora_state* adapters, int32_t count,
                         const float* grad_scale, nf4_stream_t stream);

/* Paged moments (Aner docs "Native model adaptation and NF4", section "Paged
 * AdamW uses real CUDA managed memory"): the pages keep both FP32 moment
 * tensors in managed memory that prefers the CPU and let the update reach them
 * chunk by chunk. The MI355X devices this library targets report no
 * managed-memory support, so the moments stay in PINNED HOST memory instead:
 * every mA/vA/mB/vB of `adapters` is pinned host memory (hipHostMalloc, or a
 * pinned tensor; pageable or device memory is NF4_EINVAL), and the same
 * kernel as lora_adamw_step_many, in one launch for all adapters, reads and
 * writes them in place through their device-visible addresses (the host link
 * carries each moment once in each direction, with no staging copies). The
 * host must synchronize the stream before it reads the moments. `staging` and
 * `staging_bytes` are accepted and unused (NULL is fine); page_bytes, the
 * pages' chunk size, is still checked: a multiple of 4096 in [4096, 64 MiB].
 * Parameters, gradients and preconditioners are device memory. Results equal
 * lora_adamw_step_many's bit for bit. */
int lora_adamw_step_paged(const nf4_adamw* opt, const nf4_lora_state* adapters, int32_t count,
                          const float* grad_scale, void* staging, size_t staging_bytes, size_t page_bytes,
                          nf4_stream_t stream);

/* ---- Decoder-layer operations around the NF4 linears (a Llama-shaped layer).
 * Soup, "NF4 Layer Streaming - Gate results": the pages measure a full
 * training step of a checkpointed Llama-3.1-8B-shaped model on a frozen NF4
 * base; they name the model but print no layer equations, so these are the
 * standard Llama definitions. Activations are [rows, width] row-major arrays
 * of `dtype` (bf16 or fp32); all arithmetic is fp32; gamma, rstd, lse and
 * delta are fp32. Device pointers, caller-owned, 16-byte aligned
 * (NF4_EALIGN), enqueued on `stream`; argument errors are returned first. */

/* y = s / sqrt(mean(s^2) + eps) * gamma per row, s = x + res (res may be NULL:
 * s = x). With res, s is stored to `sum` in `dtype` and normalized as stored.
 * rstd [rows] receives 1 / sqrt(mean(s^2) + eps). */
int nf4_add_rmsnorm(const void* x, const void* res, nf4_dtype dtype, int64_t rows, int64_t width, const float* gamma,
                    float eps, void* sum, void* y, float* rstd, nf4_stream_t stream);

/* Input gradient of RMSNorm with gamma frozen: dx = rstd (g - n mean(g n)),
 * g = dy gamma, n = x rstd (x is the normalized input, rstd from the forward),
 * plus dres when it is not NULL (the residual path's gradient). */
int nf4_rmsnorm_bwd(const void* dy, const void* x, const float* rstd, nf4_dtype dtype, int64_t rows, int64_t width,
                    const float* gamma, const void* dres, void* dx, nf4_stream_t stream);

/* Row strides: an `ld` argument of 0 (or the row's width) means rows are
 * dense; otherwise it is the distance between rows in elements, larger than
 * the row's width and a multiple of 16 bytes (NF4_EALIGN), so a caller can
 * keep several activations side by side in one wider array (for example q, k
 * and v as column blocks of one [S, (hq + 2 hkv) d] projection output). */

/* Rotary embedding in place on x [S, heads*d] (rows ld apart): for every head
 * and i < d/2 the pair (x_i, x_{i+d/2}) of the row at position pos is rotated
 * by pos * theta^(-2 i / d) (inverse != 0: by the negative angle, which is the
 * input gradient of the forward rotation). Angles in fp64, cos/sin in fp32.
 * d even, d <= 256. */
int nf4_rope(void* x, nf4_dtype dtype, int64_t S, int32_t heads, int32_t d, int64_t ld, double theta, int inverse,
             nf4_stream_t stream);

/* Causal grouped-query attention: o = softmax(q k^T / sqrt(d), causal) v per
 * query head h, which reads key/value head h / (hq / hkv). q [S, hq*d], k and
 * v [S, hkv*d], with rows ld_qkv apart (0: each dense); o [S, hq*d] dense;
 * lse [hq, S] receives each row's log-sum-exp (scaled scores). d a multiple of
 * 16 up to 128; hq a multiple of hkv. */
int nf4_attention_fwd(const void* q, const void* k, const void* v, nf4_dtype dtype, int64_t S, int32_t hq,
                      int32_t hkv, int32_t d, int64_t ld_qkv, void* o, float* lse, nf4_stream_t stream);

/* Input gradients of nf4_attention_fwd from dout, the forward's q, k, v, o and
 * lse: dq [S, hq*d], dk and dv [S, hkv*d] (key/value gradients summed over the
 * query heads of their group). q, k, v, dq, dk and dv have rows ld_qkv apart
 * (0: each dense); dout and o are dense. delta [hq, S] is scratch that
 * receives rowsum(dout * o). No atomics; repeated calls are bitwise
 * identical. */
int nf4_attention_bwd(const void* dout, const void* q, const void* k, const void* v, const void* o, const float* lse,
                      nf4_dtype dtype, int64_t S, int32_t hq, int32_t hkv, int32_t d, int64_t ld_qkv, float* delta,
                      void* dq, void* dk, void* dv, nf4_stream_t stream);

/* out = a + b (+ c when c is not NULL) over n entries, summed in fp32 and
 * rounded once: the input gradient of a layer input that feeds several
 * projections. out may alias a. */
int nf4_add(const void* a, const void* b, const void* c, nf4_dtype dtype, int64_t n, void* out, nf4_stream_t stream);

/* a = silu(g) * u elementwise over rows x width entries, silu(z) =
 * z / (1 + exp(-z)); g and u have rows ld apart (0: dense), a is dense. */
int nf4_swiglu(const void* g, const void* u, nf4_dtype dtype, int64_t rows, int64_t width, int64_t ld, void* a,
               nf4_stream_t stream);

/* Input gradients of nf4_swiglu: dg = da u s (1 + g (1 - s)), du = da g s with
 * s = 1 / (1 + exp(-g)); g, u, dg and du have rows ld apart (0: dense), da is
 * dense. */
int nf4_swiglu_bwd(const void* da, const void* g, const void* u, nf4_dtype dtype, int64_t rows, int64_t width,
                   int64_t ld, void* dg, void* du, nf4_stream_t stream);

/* Token cross-entropy of logits z [T, V] against int64 targets [T]:
 * tok_loss[t] = logsumexp(z_t) - z_t[target_t] (fp32, [T]), loss[0] = their
 * mean, and, unless dz is NULL, dz = (softmax(z_t) - onehot) / T in `dtype`.
 * `status` (optional device int32) is set to 0, then to NF4_EINVAL if a
 * target is outside [0, V) (that token's loss is 0). */
int nf4_cross_entropy(const void* z, nf4_dtype dtype, int64_t T, int64_t V, const int64_t* target, float* tok_loss,
                      float* loss, void* dz, int32_t* status, nf4_stream_t stream);

/* Static text for a status code. */
const char* nf4_status_string(int status);

/* NF4LORA_ABI_VERSION of the built library. */
int nf4lora_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NF4LORA_H */

// C ABI entry points (include/nf4lora.h): argument validation on the host,
// then launches on the caller's stream. Every argument error is returned before
// anything is enqueued; no exception leaves this file.
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "nf4_internal.hpp"

using namespace nf4;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
std::atomic<int> g_device_cus[kMaxDevices];  // compute units, once known
std::mutex g_device_mu;

// The current device must be gfx950 (checked once per device).
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return NF4_EDEVICE;
  if (dev >= kMaxDevices) return NF4_EUNSUPPORTED;
  int state = g_device_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    std::lock_guard<std::mutex> lock(g_device_mu);
    state = g_device_ok[dev].load(std::memory_order_relaxed);
    if (state == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NF4_EDEVICE;
      state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
      g_device_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
      g_device_ok[dev].store(state, std::memory_order_release);
    }
  }
  return state == 1 ? NF4_OK : NF4_EUNSUPPORTED;
}

bool valid_dtype(nf4_dtype d) { return d == NF4_F32 || d == NF4_BF16; }

}  // namespace

// Compute units of the current device (known once check_device has run on it).
int64_t nf4::device_cu_count() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  const int n = g_device_cus[dev].load(std::memory_order_acquire);
  return n > 0 ? n : 256;
}

namespace {

// Structural checks of a packed tensor that holds n elements.
int check_tensor(const nf4_tensor* t, int64_t n) {
  if (!t || !t->codes || !t->scales) return NF4_EINVAL;
  if (t->n != n || n < 1) return NF4_EINVAL;
  if (t->double_quant != 0 && t->double_quant != 1) return NF4_EINVAL;
  if (t->double_quant && (!t->nested || !t->offset)) return NF4_EINVAL;
  if (!aligned(t->codes, 16) || !aligned(t->scales, 16)) return NF4_EALIGN;
  if (t->double_quant && (!aligned(t->nested, 4) || !aligned(t->offset, 4))) return NF4_EALIGN;
  return NF4_OK;
}

hipStream_t as_stream(nf4_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// Bytes of an M x r fp32 side product carved from a workspace (0 when r == 0).
int64_t side_ws_bytes(int64_t M, int32_t r) { return r > 0 ? (int64_t)round_up(sizeof(float) * (size_t)(M * r), 256) : 0; }

// Workspace of lora_grad: the reduction partial sums, the recomputed side
// products, and the partial sums of a split recomputation (the larger of the
// two, as they run one after the other).
size_t lora_grad_need(int64_t M, int64_t K, int64_t N, int32_t r, bool fa, bool need_t, bool need_u) {
  const size_t side = (size_t)side_ws_bytes(M, r);
  const int64_t pt = need_t ? side_split_ws_bytes(M, K, r) : 0, pu = need_u ? side_split_ws_bytes(M, N, r) : 0;
  return lora_grad_ws(M, K, N, r, fa) + (need_t ? side : 0) + (need_u ? side : 0) + (size_t)(pt > pu ? pt : pu);
}

// Sizes every linear call accepts: positive, and small enough that M * max(K, N)
// and N * K (elements) stay below 2^62.
bool linear_sizes_ok(int64_t M, int64_t K, int64_t N) {
  if (M < 1 || K < 1 || N < 1) return false;
  constexpr int64_t kLim = int64_t(1) << 62;
  const int64_t W = K > N ? K : N;
  return K <= kLim / N && M <= kLim / W;
}

// Workspace of a linear call: [split-reduction partial sums (bf16)][split side
// product partial sums (bf16, r > 32)][side product when the caller takes none].
struct LinearWs {
  int64_t split, side_part, side;
  int64_t total() const { return split + side_part + side; }
};
LinearWs linear_ws(nf4_dtype dt, int64_t M, int64_t K, int64_t N, int32_t r, bool own_side, bool backward) {
  const int64_t split = dt == NF4_BF16 ? linear_fast_workspace_bytes(M, K, N, backward) : 0;
  LinearWs w;
  w.split = split > 0 ? (int64_t)round_up((size_t)split, 256) : 0;
  w.side_part = (dt == NF4_BF16 && r > 0) ? side_split_ws_bytes(M, backward ? N : K, r) : 0;
  w.side = own_side ? side_ws_bytes(M, r) : 0;
  return w;
}

int linear_common(const void* a, nf4_dtype dt, int64_t M, int64_t K, int64_t N, const nf4_tensor* W, const float* A,
                  const float* B, int32_t r, float s, void* out, float* side, void* ws, size_t ws_bytes, bool backward,
                  nf4_stream_t stream) {
  if (!valid_dtype(dt)) return NF4_EUNSUPPORTED;
  if (!a || !out || !linear_sizes_ok(M, K, N)) return NF4_EINVAL;
  if (int rc = check_tensor(W, N * K)) return rc;
  if (r < 0 || r > 256) return NF4_EINVAL;
  if (r > 0 && (!A || !B || r > (K < N ? K : N))) return NF4_EINVAL;
  if (r > 0 && !std::isfinite(s)) return NF4_EINVAL;
  if (!aligned(a, 16) || !aligned(out, 16)) return NF4_EALIGN;
  if (r > 0 && (!aligned(A, 4) || !aligned(B, 4) || (side && !aligned(side, 4)))) return NF4_EALIGN;
  const LinearWs w = linear_ws(dt, M, K, N, r, r > 0 && !side, backward);
  const int64_t need = w.total();
  if (ws && !aligned(ws, 256)) return NF4_EALIGN;
  if (need > 0 && (!ws || ws_bytes < (size_t)need)) return NF4_EWORKSPACE;
  if (int rc = check_device()) return rc;
  char* base = static_cast<char*>(ws);
  float* side_part = w.side_part > 0 ? reinterpret_cast<float*>(base + w.split) : nullptr;
  if (w.side > 0) side = reinterpret_cast<float*>(base + w.split + w.side_part);
  LinearArgs g{a, dt, M, K, N, W, A, B, r, s, out, side, backward, ws, (size_t)w.split, side_part};
  return launch_linear(g, as_stream(stream));
}

}  // namespace

extern "C" {

int nf4lora_abi_version(void) { return NF4LORA_ABI_VERSION; }

const char* nf4_status_string(int status) {
  switch (status) {
    case NF4_OK: return "ok";
    case NF4_EINVAL: return "invalid argument";
    case NF4_EALIGN: return "pointer not 16-byte aligned";
    case NF4_EUNSUPPORTED: return "unsupported dtype or device (gfx950 required)";
    case NF4_EDEVICE: return "HIP runtime or launch failure";
    case NF4_ENONFINITE: return "non-finite weight";
    case NF4_EWORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int nf4_layout(int64_t n, int double_quant, nf4_sizes* out) {
  if (!out || n < 1 || (double_quant != 0 && double_quant != 1)) return NF4_EINVAL;
  const int64_t nb = ceil_div(n, kBlock), nn = ceil_div(nb, kNested);
  out->codes_bytes = (n + 1) / 2;
  out->scales_bytes = double_quant ? nb : 4 * nb;
  out->nested_bytes = double_quant ? 4 * nn : 0;
  out->offset_bytes = double_quant ? 4 : 0;
  out->nb = nb;
  out->nn = double_quant ? nn : 0;
  out->quantize_workspace_bytes = (int64_t)quantize_ws_bytes(n, double_quant);
  return NF4_OK;
}

int nf4_code_tables(float nf4_out[16], float dyn8_out[256]) {
  if (!nf4_out || !dyn8_out) return NF4_EINVAL;
  std::memcpy(nf4_out, kHostNF4, sizeof(kHostNF4));
  std::memcpy(dyn8_out, kHostDyn8, sizeof(kHostDyn8));
  return NF4_OK;
}

int nf4_quantize(const float* w, int64_t n, int double_quant, const nf4_tensor* out, void* workspace,
                 size_t workspace_bytes, int32_t* status, nf4_stream_t stream) {
  if (!w || n < 1 || (double_quant != 0 && double_quant != 1)) return NF4_EINVAL;
  if (int rc = check_tensor(out, n)) return rc;
  if (out->double_quant != double_quant) return NF4_EINVAL;
  if (!aligned(w, 16)) return NF4_EALIGN;
  if (status && !aligned(status, 4)) return NF4_EALIGN;
  const size_t need = quantize_ws_bytes(n, double_quant);
  if (need > 0 && (!workspace || workspace_bytes < need)) return NF4_EWORKSPACE;
  if (need > 0 && !aligned(workspace, 256)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_quantize(w, n, out, workspace, status, as_stream(stream));
}

int nf4_quantize_noalloc(const float* w, int64_t n, int double_quant, const nf4_tensor* out, int32_t* status,
                         nf4_stream_t stream) {
  if (!w || n < 1 || (double_quant != 0 && double_quant != 1)) return NF4_EINVAL;
  if (int rc = check_tensor(out, n)) return rc;
  if (out->double_quant != double_quant) return NF4_EINVAL;
  if (!aligned(w, 16)) return NF4_EALIGN;
  if (status && !aligned(status, 4)) return NF4_EALIGN;
  const size_t need = quantize_ws_bytes(n, double_quant);
  if (need > kQuantizeScratchBytes) return NF4_EWORKSPACE;
  if (int rc = check_device()) return rc;
  void* ws = nullptr;
  if (need > 0) {
    if (int rc = quantize_scratch(&ws)) return rc;
  }
  return launch_quantize(w, n, out, ws, status, as_stream(stream));
}

int64_t nf4_quantize_noalloc_max_elements(void) {
  // the largest n whose double-quantization scratch fits (the need grows with n)
  int64_t lo = 1, hi = int64_t(1) << 40;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (quantize_ws_bytes(mid, 1) <= kQuantizeScratchBytes)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

int nf4_dequantize(const nf4_tensor* w, nf4_dtype out_dtype, void* out, nf4_stream_t stream) {
  if (!valid_dtype(out_dtype)) return NF4_EUNSUPPORTED;
  if (!w || !out) return NF4_EINVAL;
  if (int rc = check_tensor(w, w->n)) return rc;
  if (!aligned(out, 16)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_dequantize(w, out_dtype, out, as_stream(stream));
}

int nf4_add_rmsnorm(const void* x, const void* res, nf4_dtype dtype, int64_t rows, int64_t width, const float* gamma,
                    float eps, void* sum, void* y, float* rstd, nf4_stream_t stream) {
  if (!valid_dtype(dtype)) return NF4_EUNSUPPORTED;
  if (!x || !gamma || !y || !rstd || rows < 1 || width < 1 || (res && !sum)) return NF4_EINVAL;
  if (!std::isfinite(eps) || eps < 0.0f || rows >= (int64_t(1) << 31)) return NF4_EINVAL;
  const void* arrays[] = {x, res, sum, y, gamma, rstd};
  for (const void* p : arrays)
    if (p && !aligned(p, 16)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_add_rmsnorm(x, res, dtype, rows, width, gamma, eps, sum, y, rstd, as_stream(stream));
}

int nf4_rmsnorm_bwd(const void* dy, const void* x, const float* rstd, nf4_dtype dtype, int64_t rows, int64_t width,
                    const float* gamma, const void* dres, void* dx, nf4_stream_t stream) {
  if (!valid_dtype(dtype)) return NF4_EUNSUPPORTED;
  if (!dy || !x || !rstd || !gamma || !dx || rows < 1 || width < 1 || rows >= (int64_t(1) << 31)) return NF4_EINVAL;
  const void* arrays[] = {dy, x, rstd, gamma, dres, dx};
  for (const void* p : arrays)
    if (p && !aligned(p, 16)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_rmsnorm_bwd(dy, x, rstd, dtype, rows, width, gamma, dres, dx, as_stream(stream));
}

namespace {
// Row stride of a strided activation: 0 (or `width`) means dense; a larger
// stride must be a whole number of 16-byte units (NF4_EALIGN).
int row_stride(nf4_dtype dtype, int64_t width, int64_t ld, int64_t* out) {
  if (ld == 0) ld = width;
  if (ld < width || ld > (int64_t(1) << 40)) return NF4_EINVAL;
  if (ld > width && (ld * (dtype == NF4_BF16 ? 2 : 4)) % 16 != 0) return NF4_EALIGN;
  *out = ld;
  return NF4_OK;
}
}  // namespace

int nf4_rope(void* x, nf4_dtype dtype, int64_t S, int32_t heads, int32_t d, int64_t ld, double theta, int inverse,
             nf4_stream_t stream) {
  if (!valid_dtype(dtype)) return NF4_EUNSUPPORTED;
  if (!x || S < 1 || S >= (int64_t(1) << 31) || heads < 1 || d < 2 || d > 256 || d % 2 != 0) return NF4_EINVAL;
  if (!std::isfinite(theta) || theta <= 1.0 || (inverse != 0 && inverse != 1)) return NF4_EINVAL;
  int64_t lx = 0;
  if (int rc = row_stride(dtype, (int64_t)heads * d, ld, &lx)) return rc;
  if (!aligned(x, 16)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_rope(x, dtype, S, heads, d, lx, theta, inverse, as_stream(stream));
}

namespace {
int check_attention(nf4_dtype dtype, int64_t S, int32_t hq, int32_t hkv, int32_t d) {
  if (!valid_dtype(dtype)) return NF4_EUNSUPPORTED;
  if (S < 1 || S >= (int64_t(1) << 31) || hq < 1 || hkv < 1 || hq % hkv != 0 || hq > 65535) return NF4_EINVAL;
  if (d < 16 || d > 128 || d % 16 != 0) return NF4_EINVAL;
  return NF4_OK;
}
}  // namespace

int nf4_attention_fwd(const void* q, const void* k, const void* v, nf4_dtype dtype, int64_t S, int32_t hq,
                      int32_t hkv, int32_t d, int64_t ld_qkv, void* o, float* lse, nf4_stream_t stream) {
  if (int rc = check_attention(dtype, S, hq, hkv, d)) return rc;
  if (!q || !k || !v || !o || !lse) return NF4_EINVAL;
  int64_t lq = 0, lk = 0;
  if (int rc = row_stride(dtype, (int64_t)hq * d, ld_qkv, &lq)) return rc;
  if (int rc = row_stride(dtype, (int64_t)hkv * d, ld_qkv, &lk)) return rc;
  const void* arrays[] = {q, k, v, o, lse};
  for (const void* p : arrays)
    if (!aligned(p, 16)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_attention_fwd(q, k, v, dtype, S, hq, hkv, d, lq, lk, o, lse, as_stream(stream));
}

int nf4_attention_bwd(const void* dout, const void* q, const void* k, const void* v, const void* o, const float* lse,
                      nf4_dtype dtype, int64_t S, int32_t hq, int32_t hkv, int32_t d, int64_t ld_qkv, float* delta,
                      void* dq, void* dk, void* dv, nf4_stream_t stream) {
  if (int rc = check_attention(dtype, S, hq, hkv, d)) return rc;
  if (!dout || !q || !k || !v || !o || !lse || !delta || !dq || !dk || !dv) return NF4_EINVAL;
  int64_t lq = 0, lk = 0;
  if (int rc = row_stride(dtype, (int64_t)hq * d, ld_qkv, &lq)) return rc;
  if (int rc = row_stride(dtype, (int64_t)hkv * d, ld_qkv, &lk)) return rc;
  const void* arrays[] = {dout, q, k, v, o, lse, delta, dq, dk, dv};
  for (const void* p : arrays)
    if (!aligned(p, 16)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_attention_bwd(dout, q, k, v, o, lse, dtype, S, hq, hkv, d, lq, lk, delta, dq, dk, dv,
                              as_stream(stream));
}

int nf4_add(const void* a, const void* b, const void* c, nf4_dtype dtype, int64_t n, void* out, nf4_stream_t stream) {
  if (!valid_dtype(dtype)) return NF4_EUNSUPPORTED;
  if (!a || !b || !out || n < 1 || n > (int64_t(1) << 40)) return NF4_EINVAL;
  const void* arrays[] = {a, b, c, out};
  for (const void* p : arrays)
    if (p && !aligned(p, 16)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_add3(a, b, c, dtype, n, out, as_stream(stream));
}

int nf4_swiglu(const void* g, const void* u, nf4_dtype dtype, int64_t rows, int64_t width, int64_t ld, void* a,
               nf4_stream_t stream) {
  if (!valid_dtype(dtype)) return NF4_EUNSUPPORTED;
  if (!g || !u || !a || rows < 1 || width < 1 || rows > (int64_t(1) << 40) / width) return NF4_EINVAL;
  int64_t lg = 0;
  if (int rc = row_stride(dtype, width, ld, &lg)) return rc;
  if (!aligned(g, 16) || !aligned(u, 16) || !aligned(a, 16)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_swiglu(g, u, dtype, rows, width, lg, a, as_stream(stream));
}

int nf4_swiglu_bwd(const void* da, const void* g, const void* u, nf4_dtype dtype, int64_t rows, int64_t width,
                   int64_t ld, void* dg, void* du, nf4_stream_t stream) {
  if (!valid_dtype(dtype)) return NF4_EUNSUPPORTED;
  if (!da || !g || !u || !dg || !du || rows < 1 || width < 1 || rows > (int64_t(1) << 40) / width) return NF4_EINVAL;
  int64_t lg = 0;
  if (int rc = row_stride(dtype, width, ld, &lg)) return rc;
  const void* arrays[] = {da, g, u, dg, du};
  for (const void* p : arrays)
    if (!aligned(p, 16)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_swiglu_bwd(da, g, u, dtype, rows, width, lg, dg, du, as_stream(stream));
}

int nf4_cross_entropy(const void* z, nf4_dtype dtype, int64_t T, int64_t V, const int64_t* target, float* tok_loss,
                      float* loss, void* dz, int32_t* status, nf4_stream_t stream) {
  if (!valid_dtype(dtype)) return NF4_EUNSUPPORTED;
  if (!z || !target || !tok_loss || !loss || T < 1 || V < 1 || T >= (int64_t(1) << 31)) return NF4_EINVAL;
  const void* arrays[] = {z, target, tok_loss, loss, dz};
  for (const void* p : arrays)
    if (p && !aligned(p, 16)) return NF4_EALIGN;
  if (status && !aligned(status, 4)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_cross_entropy(z, dtype, T, V, target, tok_loss, loss, dz, status, as_stream(stream));
}

int nf4_dequantize_many(const nf4_tensor* tensors, void* const* outs, int32_t count, nf4_dtype out_dtype,
                        nf4_stream_t stream) {
  if (!valid_dtype(out_dtype)) return NF4_EUNSUPPORTED;
  if (!tensors || !outs || count < 1 || count > NF4_MAX_TENSORS_PER_CALL) return NF4_EINVAL;
  int64_t groups = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (!outs[i]) return NF4_EINVAL;
    if (int rc = check_tensor(&tensors[i], tensors[i].n)) return rc;
    if (!aligned(outs[i], 16)) return NF4_EALIGN;
    groups += ceil_div(tensors[i].n / 8 > 0 ? tensors[i].n / 8 : 1, 2048);
  }
  if (groups >= (int64_t(1) << 31)) return NF4_EINVAL;
  if (int rc = check_device()) return rc;
  return launch_dequantize_many(tensors, outs, count, out_dtype, as_stream(stream));
}

int64_t nf4_quantize_many_workspace_bytes(const nf4_tensor* out, int32_t count) {
  if (!out || count < 1 || count > NF4_MAX_TENSORS_PER_CALL) return NF4_EINVAL;
  for (int32_t i = 0; i < count; ++i)
    if (out[i].n < 1 || (out[i].double_quant != 0 && out[i].double_quant != 1)) return NF4_EINVAL;
  return (int64_t)quantize_many_ws_bytes(out, count);
}

int nf4_quantize_many(const float* const* w, const nf4_tensor* out, int32_t count, void* workspace,
                      size_t workspace_bytes, int32_t* status, nf4_stream_t stream) {
  if (!w || !out || count < 1 || count > NF4_MAX_TENSORS_PER_CALL) return NF4_EINVAL;
  int64_t groups = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (!w[i]) return NF4_EINVAL;
    if (int rc = check_tensor(&out[i], out[i].n)) return rc;
    if (!aligned(w[i], 16)) return NF4_EALIGN;
    groups += quant_groups(out[i].n);
  }
  if (groups >= (int64_t(1) << 31)) return NF4_EINVAL;
  if (status && !aligned(status, 4)) return NF4_EALIGN;
  if (!workspace || workspace_bytes < quantize_many_ws_bytes(out, count)) return NF4_EWORKSPACE;
  if (!aligned(workspace, 256)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_quantize_many(w, out, count, workspace, status, as_stream(stream));
}

int nf4_embedding_rows(const nf4_tensor* E, int64_t V, int64_t D, const int64_t* ids, int64_t T, nf4_dtype out_dtype,
                       void* out, int32_t* status, nf4_stream_t stream) {
  if (!valid_dtype(out_dtype)) return NF4_EUNSUPPORTED;
  if (V < 1 || D < 1 || T < 0 || V > INT64_MAX / D) return NF4_EINVAL;
  if (T > 0 && (T > (int64_t(1) << 40) / D || !ids || !out)) return NF4_EINVAL;
  if (int rc = check_tensor(E, V * D)) return rc;
  if (T > 0 && (!aligned(ids, 8) || !aligned(out, 16))) return NF4_EALIGN;
  if (status && !aligned(status, 4)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_embedding_rows(E, V, D, ids, T, out_dtype, out, status, as_stream(stream));
}

int nf4_linear_fwd(const void* x, nf4_dtype dtype, int64_t M, int64_t K, const nf4_tensor* W, int64_t N,
                   const float* A, const float* B, int32_t r, float s, void* y, float* t_out, void* workspace,
                   size_t workspace_bytes, nf4_stream_t stream) {
  return linear_common(x, dtype, M, K, N, W, A, B, r, s, y, t_out, workspace, workspace_bytes, false, stream);
}

int nf4_linear_bwd_input(const void* dy, nf4_dtype dtype, int64_t M, int64_t N, const nf4_tensor* W, int64_t K,
                         const float* A, const float* B, int32_t r, float s, void* dx, float* u_out, void* workspace,
                         size_t workspace_bytes, nf4_stream_t stream) {
  return linear_common(dy, dtype, M, K, N, W, A, B, r, s, dx, u_out, workspace, workspace_bytes, true, stream);
}

int nf4_linear_fwd_group(const void* x, nf4_dtype dtype, int64_t M, int64_t K, int32_t count,
                         const nf4_tensor* const* W, const int64_t* N, const float* const* A, const float* const* B,
                         const int32_t* r, const float* s, void* const* y, float* const* t_out, void* workspace,
                         size_t workspace_bytes, nf4_stream_t stream) {
  if (!valid_dtype(dtype)) return NF4_EUNSUPPORTED;
  if (count < 1 || count > NF4_MAX_PROJECTIONS_PER_GROUP || !W || !N || !r || !s || !y || !x) return NF4_EINVAL;
  if (workspace && !aligned(workspace, 256)) return NF4_EALIGN;
  LinearArgs g[NF4_MAX_PROJECTIONS_PER_GROUP];
  int64_t need = 0;
  char* base = static_cast<char*>(workspace);
  for (int i = 0; i < count; ++i) {
    const float* Ai = A ? A[i] : nullptr;
    const float* Bi = B ? B[i] : nullptr;
    float* side = t_out ? t_out[i] : nullptr;
    const int32_t ri = r[i];
    if (!y[i] || !linear_sizes_ok(M, K, N[i])) return NF4_EINVAL;
    if (int rc = check_tensor(W[i], N[i] * K)) return rc;
    if (ri < 0 || ri > 256) return NF4_EINVAL;
    if (ri > 0 && (!Ai || !Bi || ri > (K < N[i] ? K : N[i]) || !std::isfinite(s[i]))) return NF4_EINVAL;
    if (!aligned(x, 16) || !aligned(y[i], 16)) return NF4_EALIGN;
    if (ri > 0 && (!aligned(Ai, 4) || !aligned(Bi, 4) || (side && !aligned(side, 4)))) return NF4_EALIGN;
    const LinearWs w = linear_ws(dtype, M, K, N[i], ri, ri > 0 && !side, false);
    char* part = base ? base + need : nullptr;
    float* side_part = w.side_part > 0 ? reinterpret_cast<float*>(part + w.split) : nullptr;
    if (w.side > 0) side = reinterpret_cast<float*>(part + w.split + w.side_part);
    g[i] = LinearArgs{x, dtype, M, K, N[i], W[i], Ai, Bi, ri, s[i], y[i], side, false, part, (size_t)w.split,
                      side_part};
    need += (int64_t)round_up((size_t)w.total(), 256);
  }
  if (need > 0 && (!workspace || workspace_bytes < (size_t)need)) return NF4_EWORKSPACE;
  if (int rc = check_device()) return rc;
  return launch_linear_group(g, count, as_stream(stream));
}

int64_t nf4_linear_fwd_group_workspace_bytes(int64_t M, int64_t K, int32_t count, const int64_t* N, const int32_t* r) {
  if (count < 1 || count > NF4_MAX_PROJECTIONS_PER_GROUP || !N || !r) return NF4_EINVAL;
  int64_t need = 0;
  for (int i = 0; i < count; ++i) {
    if (!linear_sizes_ok(M, K, N[i]) || r[i] < 0 || r[i] > 256) return NF4_EINVAL;
    need += (int64_t)round_up((size_t)linear_ws(NF4_BF16, M, K, N[i], r[i], r[i] > 0, false).total(), 256);
  }
  return need;
}

int nf4_linear_bwd_input_sum(const void* const* dy, nf4_dtype dtype, int64_t M, int64_t K, int32_t count,
                             const nf4_tensor* const* W, const int64_t* N, const float* const* A,
                             const float* const* B, const int32_t* r, const float* s, void* dx,
                             float* const* u_out, void* workspace, size_t workspace_bytes, nf4_stream_t stream) {
  if (!valid_dtype(dtype)) return NF4_EUNSUPPORTED;
  if (count < 1 || count > NF4_MAX_PROJECTIONS_PER_GROUP || !dy || !W || !N || !r || !s || !dx) return NF4_EINVAL;
  if (workspace && !aligned(workspace, 256)) return NF4_EALIGN;
  if (!aligned(dx, 16)) return NF4_EALIGN;
  LinearArgs g[NF4_MAX_PROJECTIONS_PER_GROUP];
  int64_t need = 0;
  char* base = static_cast<char*>(workspace);
  for (int i = 0; i < count; ++i) {
    const float* Ai = A ? A[i] : nullptr;
    const float* Bi = B ? B[i] : nullptr;
    float* side = u_out ? u_out[i] : nullptr;
    const int32_t ri = r[i];
    if (!dy[i] || !linear_sizes_ok(M, K, N[i])) return NF4_EINVAL;
    if (int rc = check_tensor(W[i], N[i] * K)) return rc;
    if (ri < 0 || ri > 256) return NF4_EINVAL;
    if (ri > 0 && (!Ai || !Bi || ri > (K < N[i] ? K : N[i]) || !std::isfinite(s[i]))) return NF4_EINVAL;
    if (!aligned(dy[i], 16)) return NF4_EALIGN;
    if (ri > 0 && (!aligned(Ai, 4) || !aligned(Bi, 4) || (side && !aligned(side, 4)))) return NF4_EALIGN;
    const LinearWs w = linear_ws(dtype, M, K, N[i], ri, ri > 0 && !side, true);
    char* part = base ? base + need : nullptr;
    float* side_part = w.side_part > 0 ? reinterpret_cast<float*>(part + w.split) : nullptr;
    if (w.side > 0) side = reinterpret_cast<float*>(part + w.split + w.side_part);
    g[i] = LinearArgs{dy[i], dtype, M, K, N[i], W[i], Ai, Bi, ri, s[i], dx, side, true, part, (size_t)w.split,
                      side_part};
    need += (int64_t)round_up((size_t)w.total(), 256);
  }
  void* tmp = nullptr;
  if (!linear_bwd_sum_one_launch(g, count) && count > 1) {
    tmp = base ? base + need : nullptr;
    need += (int64_t)round_up((size_t)(count - 1) * (dtype == NF4_BF16 ? 2 : 4) * (size_t)(M * K), 256);
  }
  if (need > 0 && (!workspace || workspace_bytes < (size_t)need)) return NF4_EWORKSPACE;
  if (int rc = check_device()) return rc;
  return launch_linear_bwd_sum(g, count, tmp, as_stream(stream));
}

int64_t nf4_linear_bwd_input_sum_workspace_bytes(int64_t M, int64_t K, int32_t count, const int64_t* N,
                                                 const int32_t* r, nf4_dtype dtype) {
  if (!valid_dtype(dtype)) return NF4_EUNSUPPORTED;
  if (count < 1 || count > NF4_MAX_PROJECTIONS_PER_GROUP || !N || !r) return NF4_EINVAL;
  int64_t need = 0;
  for (int i = 0; i < count; ++i) {
    if (!linear_sizes_ok(M, K, N[i]) || r[i] < 0 || r[i] > 256) return NF4_EINVAL;
    need += (int64_t)round_up((size_t)linear_ws(dtype, M, K, N[i], r[i], r[i] > 0, true).total(), 256);
  }
  if (count > 1) need += (int64_t)round_up((size_t)(count - 1) * (dtype == NF4_BF16 ? 2 : 4) * (size_t)(M * K), 256);
  return need;
}

int64_t nf4_linear_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t r, int flags) {
  if (!linear_sizes_ok(M, K, N) || r < 0 || r > 256) return NF4_EINVAL;
  if (flags & ~(NF4_WS_BACKWARD | NF4_WS_NO_SIDE_OUT)) return NF4_EINVAL;
  return linear_ws(NF4_BF16, M, K, N, r, r > 0 && (flags & NF4_WS_NO_SIDE_OUT), (flags & NF4_WS_BACKWARD) != 0)
      .total();
}

int64_t lora_grad_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t r, int fa, int recompute) {
  if (!linear_sizes_ok(M, K, N) || r < 1 || r > 256 || (fa != 0 && fa != 1)) return NF4_EINVAL;
  if (recompute < 0 || recompute > (NF4_RECOMPUTE_T | NF4_RECOMPUTE_U)) return NF4_EINVAL;
  return (int64_t)lora_grad_need(M, K, N, r, fa != 0, recompute & NF4_RECOMPUTE_T, !fa && (recompute & NF4_RECOMPUTE_U));
}

int lora_grad(const void* x, const void* dy, nf4_dtype dtype, int64_t M, int64_t K, int64_t N, const float* A,
              const float* B, const float* t, const float* u, int32_t r, float s, float* dA, float* dB,
              void* workspace, size_t workspace_bytes, nf4_stream_t stream) {
  if (!valid_dtype(dtype)) return NF4_EUNSUPPORTED;
  if (!linear_sizes_ok(M, K, N) || r < 1 || r > 256) return NF4_EINVAL;
  const bool fa = (dA == nullptr);
  const bool need_t = (t == nullptr), need_u = !fa && (u == nullptr);
  if (!dy || !dB || !std::isfinite(s)) return NF4_EINVAL;
  if ((!fa || need_t) && !x) return NF4_EINVAL;  // dA and a recomputed T read x
  if ((need_t && !A) || (need_u && !B)) return NF4_EINVAL;
  if (need_t && r > K) return NF4_EINVAL;
  if (!aligned(dy, 16) || !aligned(dB, 4) || (t && !aligned(t, 4))) return NF4_EALIGN;
  if (x && !aligned(x, 16)) return NF4_EALIGN;
  if (!fa && (!aligned(dA, 4) || (u && !aligned(u, 4)))) return NF4_EALIGN;
  if ((need_t && !aligned(A, 4)) || (need_u && !aligned(B, 4))) return NF4_EALIGN;
  const size_t base = lora_grad_ws(M, K, N, r, fa);
  const size_t side = (size_t)side_ws_bytes(M, r);
  const size_t need = lora_grad_need(M, K, N, r, fa, need_t, need_u);
  if (!workspace || workspace_bytes < need) return NF4_EWORKSPACE;
  if (!aligned(workspace, 256)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  // Recomputed side products follow the reduction partial sums in the
  // workspace, then the partial sums of a split side product (shared: the two
  // recomputations run one after the other on the stream).
  char* extra = static_cast<char*>(workspace) + base;
  float* part = reinterpret_cast<float*>(extra + (need_t ? side : 0) + (need_u ? side : 0));
  if (need_t) {  // T = x A^T
    float* tt = reinterpret_cast<float*>(extra);
    extra += side;
    if (int rc = launch_side_product(x, dtype, M, K, A, r, false, tt, part, as_stream(stream))) return rc;
    t = tt;
  }
  if (need_u) {  // U = dY B
    float* uu = reinterpret_cast<float*>(extra);
    if (int rc = launch_side_product(dy, dtype, M, N, B, r, true, uu, part, as_stream(stream))) return rc;
    u = uu;
  }
  return launch_lora_grad(fa ? nullptr : x, dy, dtype, M, K, N, t, fa ? nullptr : u, r, s, dA, dB, workspace,
                          as_stream(stream));
}

int64_t lorafa_preconditioner_workspace_bytes(int32_t r, int64_t K) {
  if (r < 1 || r > 256 || K < 1 || K > (INT64_MAX >> 8)) return NF4_EINVAL;
  return (int64_t)lorafa_ws_bytes(r, K);
}

int lorafa_preconditioner(const float* A, int32_t r, int64_t K, float* P, void* workspace, size_t workspace_bytes,
                          nf4_stream_t stream) {
  if (!A || !P || r < 1 || r > 256 || K < 1 || K > (INT64_MAX >> 8)) return NF4_EINVAL;
  if (!aligned(A, 4) || !aligned(P, 4)) return NF4_EALIGN;
  const size_t need = lorafa_ws_bytes(r, K);
  if (!workspace || workspace_bytes < need) return NF4_EWORKSPACE;
  if (!aligned(workspace, 256)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_lorafa_preconditioner(A, r, K, P, workspace, as_stream(stream));
}

}  // extern "C"

namespace {

int check_adamw(const nf4_adamw* opt) {
  if (!opt) return NF4_EINVAL;
  const float lr = opt->lr, b1 = opt->beta1, b2 = opt->beta2, eps = opt->eps, wd = opt->weight_decay;
  if (!std::isfinite(lr) || lr < 0.0f || !(b1 >= 0.0f && b1 < 1.0f) || !(b2 >= 0.0f && b2 < 1.0f)) return NF4_EINVAL;
  if (!std::isfinite(eps) || !(eps > 0.0f) || !std::isfinite(wd) || wd < 0.0f || opt->step < 1) return NF4_EINVAL;
  return NF4_OK;
}

// The device-visible address of pinned host memory p (NULL for pageable or
// device memory).
void* pinned_host_device_ptr(const void* p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the error an unknown (pageable) pointer leaves
    return nullptr;
  }
  return at.type == hipMemoryTypeHost ? at.devicePointer : nullptr;
}

int check_lora_state(const nf4_lora_state& a) {
  constexpr int64_t kMaxEntries = int64_t(1) << 40;
  const int32_t r = a.r;
  if (r < 1 || r > 256 || a.K < 1 || a.N < 1) return NF4_EINVAL;
  if (a.K > kMaxEntries / r || a.N > kMaxEntries / r) return NF4_EINVAL;
  if (!a.B || !a.dB || !a.mB || !a.vB) return NF4_EINVAL;
  const int a_given = (a.A != nullptr) + (a.dA != nullptr) + (a.mA != nullptr) + (a.vA != nullptr);
  if (a_given != 0 && a_given != 4) return NF4_EINVAL;
  if (a.precond && (a_given != 0 || !std::isfinite(a.s) || a.s == 0.0f)) return NF4_EINVAL;
  const void* arrays[] = {a.A, a.dA, a.mA, a.vA, a.B, a.dB, a.mB, a.vB, a.precond};
  for (const void* p : arrays)
    if (p && !aligned(p, 16)) return NF4_EALIGN;
  return NF4_OK;
}

}  // namespace

extern "C" {

int lora_adamw_step(const nf4_adamw* opt, int32_t r, int64_t K, int64_t N, float* A, const float* dA, float* mA,
                    float* vA, float* B, const float* dB, float* mB, float* vB, const float* precond, float s,
                    const float* grad_scale, nf4_stream_t stream) {
  if (int rc = check_adamw(opt)) return rc;
  const nf4_lora_state a{r, K, N, A, dA, mA, vA, B, dB, mB, vB, precond, s};
  if (int rc = check_lora_state(a)) return rc;
  if (grad_scale && !aligned(grad_scale, 4)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_lora_adamw(*opt, &a, 1, grad_scale, as_stream(stream));
}

int lora_adamw_step_paged(const nf4_adamw* opt, const nf4_lora_state* adapters, int32_t count,
                          const float* grad_scale, void* staging, size_t staging_bytes, size_t page_bytes,
                          nf4_stream_t stream) {
  if (int rc = check_adamw(opt)) return rc;
  if (!adapters || count < 1 || count > NF4_MAX_ADAPTERS_PER_CALL) return NF4_EINVAL;
  if (page_bytes < 4096 || page_bytes > (size_t(64) << 20) || page_bytes % 4096 != 0) return NF4_EINVAL;
  (void)staging;  // accepted for callers written against the staged schedule; not used
  (void)staging_bytes;
  for (int32_t i = 0; i < count; ++i)
    if (int rc = check_lora_state(adapters[i])) return rc;
  if (grad_scale && !aligned(grad_scale, 4)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  // the same update kernel, reading and writing every moment in place through
  // its device-visible address
  nf4_lora_state dev[NF4_MAX_ADAPTERS_PER_CALL];
  for (int32_t i = 0; i < count; ++i) {
    dev[i] = adapters[i];
    float** mom[] = {&dev[i].mA, &dev[i].vA, &dev[i].mB, &dev[i].vB};
    for (float** m : mom) {
      if (!*m) continue;
      void* d = pinned_host_device_ptr(*m);
      if (!d) return NF4_EINVAL;
      *m = static_cast<float*>(d);
    }
  }
  return launch_lora_adamw(*opt, dev, count, grad_scale, as_stream(stream));
}

int lora_adamw_step_many(const nf4_adamw* opt, const nf4_lora_state* adapters, int32_t count,
                         const float* grad_scale, nf4_stream_t stream) {
  if (int rc = check_adamw(opt)) return rc;
  if (!adapters || count < 1 || count > NF4_MAX_ADAPTERS_PER_CALL) return NF4_EINVAL;
  for (int32_t i = 0; i < count; ++i)
    if (int rc = check_lora_state(adapters[i])) return rc;
  if (grad_scale && !aligned(grad_scale, 4)) return NF4_EALIGN;
  if (int rc = check_device()) return rc;
  return launch_lora_adamw(*opt, adapters, count, grad_scale, as_stream(stream));
}

}  // extern "C"

// capi.hip -- the extern "C" entry points declared in include/qlora.h:
// host-side argument checks, workspace carving, and kernel enqueueing.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "qlora_internal.h"

namespace qlora {

namespace {
// T_j = smallest float32 strictly above the exact midpoint of levels j and
// j+1 (the midpoint of two float32 values is exact in double).  Then x >= T_j
// <=> x is nearer to a level above j, with an exact tie at the midpoint going
// to the lower level.  (Float4's repeated top level gives T_14 just above 1,
// which no normalized weight reaches: code 15 is never produced.)
Thresholds thresholds_of(const uint32_t *bits) {
  Thresholds t;
  for (int j = 0; j < 15; ++j) {
    float a, b;
    std::memcpy(&a, &bits[j], 4);
    std::memcpy(&b, &bits[j + 1], 4);
    const double mid = ((double)a + (double)b) * 0.5;
    float v = (float)mid;
    if ((double)v <= mid) v = std::nextafter(v, INFINITY);
    t.t[j] = v;
  }
  return t;
}
}  // namespace

const Thresholds &codebook_thresholds(int codebook) {
  static const Thresholds nf4 = thresholds_of(kNF4Bits), fp4 = thresholds_of(kFP4Bits),
                          e3m0 = thresholds_of(kE3M0Bits);
  return codebook == kCodebookE3M0 ? e3m0 : codebook == kCodebookFP4 ? fp4 : nf4;
}

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char *where) {
  return fail(QLORA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxElems = int64_t(1) << 40;  // sanity bound on n*k and M*k, M*n
constexpr int64_t kMaxK = int64_t(1) << 22;      // k < 2^22: a 256-row activation tile stays below 2^31 bytes

int check_shape(int64_t n, int64_t k) {
  if (n < 1 || k < kBlock || k % kBlock != 0)
    return fail(QLORA_ERR_BAD_SHAPE, "weight shape [%lld, %lld]: need n >= 1, k >= 64, k %% 64 == 0",
                (long long)n, (long long)k);
  if (n > kMaxElems / k || k >= kMaxK) return fail(QLORA_ERR_BAD_SHAPE, "weight too large");
  return QLORA_OK;
}

// A weight descriptor of either ABI form, flattened.
struct WeightIn {
  int64_t n = 0, k = 0;
  uint8_t *packed = nullptr, *scale_code = nullptr;
  float *group_amax = nullptr, *offset = nullptr;
  int codebook = QLORA_CODEBOOK_NF4, scales = QLORA_SCALES_DQ;
  float *absmax = nullptr;
};

int take(const qlora_nf4_weight *w, WeightIn *o) {
  if (!w) return fail(QLORA_ERR_NULL_ARG, "weight descriptor is NULL");
  o->n = w->n;
  o->k = w->k;
  o->packed = w->packed;
  o->scale_code = w->scale_code;
  o->group_amax = w->group_amax;
  o->offset = w->offset;
  return QLORA_OK;
}

int take_ex(const qlora_weight_ex *w, WeightIn *o) {
  if (!w) return fail(QLORA_ERR_NULL_ARG, "weight descriptor is NULL");
  if (w->size < sizeof(qlora_weight_ex))
    return fail(QLORA_ERR_BAD_CODEBOOK, "qlora_weight_ex.size = %zu < %zu", w->size, sizeof(qlora_weight_ex));
  if (int e = take(&w->base, o)) return e;
  o->codebook = w->codebook;
  o->scales = w->scales;
  o->absmax = w->absmax;
  return QLORA_OK;
}

bool known_codebook(int cb) {
  return cb == QLORA_CODEBOOK_NF4 || cb == QLORA_CODEBOOK_FP4_E2M1 || cb == QLORA_CODEBOOK_FP4_E3M0;
}

int check_weight(const WeightIn &w) {
  if (int e = check_shape(w.n, w.k)) return e;
  if (!known_codebook(w.codebook))
    return fail(QLORA_ERR_BAD_CODEBOOK, "codebook %d is none of NF4 (0), Float4 E2M1 (1), Float4 E3M0 (2)",
                (int)w.codebook);
  if (w.scales != QLORA_SCALES_DQ && w.scales != QLORA_SCALES_FP32)
    return fail(QLORA_ERR_BAD_CODEBOOK, "scales %d is neither DQ (0) nor FP32 (1)", (int)w.scales);
  if (w.scales == QLORA_SCALES_DQ) {
    if (!w.packed || !w.scale_code || !w.group_amax || !w.offset)
      return fail(QLORA_ERR_NULL_ARG, "a weight buffer is NULL");
    if (!aligned16(w.packed) || !aligned16(w.scale_code) || !aligned16(w.group_amax) || !aligned16(w.offset))
      return fail(QLORA_ERR_MISALIGNED, "weight buffers must be 16-byte aligned");
  } else {
    if (!w.packed || !w.absmax) return fail(QLORA_ERR_NULL_ARG, "a weight buffer is NULL");
    if (!aligned16(w.packed) || !aligned16(w.absmax))
      return fail(QLORA_ERR_MISALIGNED, "weight buffers must be 16-byte aligned");
  }
  return QLORA_OK;
}

Nf4View view_of(const WeightIn &w) {
  Nf4View v;
  v.n = w.n;
  v.k = w.k;
  v.nb = w.n * w.k / kBlock;
  v.ng = ceil_div(v.nb, kGroup);
  v.packed = w.packed;
  v.scale_code = w.scale_code;
  v.group_amax = w.group_amax;
  v.offset = w.offset;
  v.codebook = w.codebook;
  v.absmax = w.scales == QLORA_SCALES_FP32 ? w.absmax : nullptr;
  return v;
}

int check_linear_shape(int64_t n, int64_t k, int64_t M, int r) {
  if (int e = check_shape(n, k)) return e;
  if (M < 0) return fail(QLORA_ERR_BAD_SHAPE, "M = %lld < 0", (long long)M);
  if (M > kMaxElems / std::max<int64_t>(k, n)) return fail(QLORA_ERR_BAD_SHAPE, "M too large");
  if (r < 1 || r > 128) return fail(QLORA_ERR_BAD_RANK, "rank r = %d outside [1, 128]", r);
  return QLORA_OK;
}

int check_linear(const WeightIn &w, int64_t M, int r, float alpha) {
  if (int e = check_weight(w)) return e;
  if (int e = check_linear_shape(w.n, w.k, M, r)) return e;
  if (!std::isfinite(alpha)) return fail(QLORA_ERR_BAD_ALPHA, "alpha is not finite");
  return QLORA_OK;
}

int check_tensor(const void *p, const char *name) {
  if (!p) return fail(QLORA_ERR_NULL_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(QLORA_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
  return QLORA_OK;
}

int check_ws(void *ws, size_t have, size_t need) {
  if (need == 0) return QLORA_OK;
  if (!ws) return fail(QLORA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (have < need) return fail(QLORA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", have, need);
  if (!aligned16(ws)) return fail(QLORA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  return QLORA_OK;
}

// Workspace of qlora_linear_fwd_noalloc: a fixed array in device memory
// (every GPU the library runs on holds its own copy until the process ends).
// In host code `scratch` names a host-side stand-in; kernels get the device
// address hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kNoallocScratchBytes = size_t(128) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace
}  // namespace qlora

static __device__ __align__(256) unsigned char scratch[qlora::kNoallocScratchBytes];

namespace qlora {
namespace {

// The current device's copy of `scratch` (looked up on its first use, with
// that device current).
int device_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "qlora_linear_fwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QLORA_ERR_HIP, "qlora_linear_fwd_noalloc: device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "qlora_linear_fwd_noalloc: hipGetSymbolAddress(scratch)");
    if (!p) return fail(QLORA_ERR_HIP, "qlora_linear_fwd_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}

size_t quantize_ws(int64_t n, int64_t k) {
  const int64_t nb = n * k / kBlock, ng = ceil_div(nb, kGroup);
  return align_up((size_t)nb * sizeof(float), 256) + align_up((size_t)ng * sizeof(double), 256);
}

}  // namespace
}  // namespace qlora

using namespace qlora;

extern "C" {

int qlora_nf4_sizes(int64_t n, int64_t k, size_t *packed_bytes, size_t *scale_code_bytes, size_t *group_count) {
  if (int e = check_shape(n, k)) return e;
  const int64_t nb = n * k / kBlock;
  if (packed_bytes) *packed_bytes = (size_t)(n * k / 2);
  if (scale_code_bytes) *scale_code_bytes = (size_t)nb;
  if (group_count) *group_count = (size_t)ceil_div(nb, kGroup);
  return QLORA_OK;
}

size_t qlora_quantize_workspace_bytes(int64_t n, int64_t k) {
  if (n < 1 || k < kBlock || k % kBlock != 0 || n > kMaxElems / k || k >= kMaxK) return 0;
  return quantize_ws(n, k);
}

namespace {
int quantize_impl(const char *fn, const float *W, const WeightIn &out, void *ws, size_t ws_bytes, hipStream_t s) {
  if (int e = check_weight(out)) return e;
  if (int e = check_tensor(W, "W")) return e;
  const size_t need = quantize_ws(out.n, out.k);
  if (int e = check_ws(ws, ws_bytes, need)) return e;
  const int64_t nb = out.n * out.k / kBlock;
  const bool single = out.scales == QLORA_SCALES_FP32;
  float *ws_absmax = single ? out.absmax : static_cast<float *>(ws);
  double *ws_sum = reinterpret_cast<double *>(static_cast<char *>(ws) + align_up((size_t)nb * sizeof(float), 256));
  hipError_t e = launch_quantize(W, out.n, out.k, out.codebook, single, out.packed, out.scale_code, out.group_amax,
                                 out.offset, ws_absmax, ws_sum, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  return QLORA_OK;
}

int dequant_impl(const char *fn, const WeightIn &w, uint16_t *W_bf16, hipStream_t s) {
  if (int e = check_weight(w)) return e;
  if (int e = check_tensor(W_bf16, "W_bf16")) return e;
  hipError_t e = launch_dequant(view_of(w), W_bf16, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  return QLORA_OK;
}
}  // namespace

int qlora_quantize_nf4_dq(const float *W, const qlora_nf4_weight *out, void *ws, size_t ws_bytes, hipStream_t stream) {
  WeightIn o;
  if (int e = take(out, &o)) return e;
  return quantize_impl("qlora_quantize_nf4_dq", W, o, ws, ws_bytes, stream);
}

int qlora_quantize_ex(const float *W, const qlora_weight_ex *out, void *ws, size_t ws_bytes, hipStream_t stream) {
  WeightIn o;
  if (int e = take_ex(out, &o)) return e;
  return quantize_impl("qlora_quantize_ex", W, o, ws, ws_bytes, stream);
}

int qlora_dequant_bf16(const qlora_nf4_weight *w, uint16_t *W_bf16, hipStream_t stream) {
  WeightIn v;
  if (int e = take(w, &v)) return e;
  return dequant_impl("qlora_dequant_bf16", v, W_bf16, stream);
}

int qlora_dequant_bf16_ex(const qlora_weight_ex *w, uint16_t *W_bf16, hipStream_t stream) {
  WeightIn v;
  if (int e = take_ex(w, &v)) return e;
  return dequant_impl("qlora_dequant_bf16_ex", v, W_bf16, stream);
}

namespace {
int elementwise(int op, const char *fn, const uint16_t *x0, const uint16_t *x1, const uint16_t *x2, uint16_t *y0,
                uint16_t *y1, int64_t count, hipStream_t stream) {
  if (count < 0 || count > kMaxElems) return fail(QLORA_ERR_BAD_SHAPE, "count = %lld", (long long)count);
  if (count == 0) return QLORA_OK;
  if (int e = check_tensor(x0, "input")) return e;
  if (int e = check_tensor(x1, "input")) return e;
  if (op == 1)
    if (int e = check_tensor(x2, "dh")) return e;
  if (int e = check_tensor(y0, "output")) return e;
  if (op == 1)
    if (int e = check_tensor(y1, "du")) return e;
  hipError_t e = launch_swiglu(op, x0, x1, x2, y0, y1, count, stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return QLORA_OK;
}
}  // namespace

int qlora_swiglu_fwd(const uint16_t *gate, const uint16_t *up, uint16_t *h, int64_t count, hipStream_t stream) {
  return elementwise(0, "qlora_swiglu_fwd", gate, up, nullptr, h, nullptr, count, stream);
}

int qlora_swiglu_bwd(const uint16_t *gate, const uint16_t *up, const uint16_t *dh, uint16_t *d_gate, uint16_t *d_up,
                     int64_t count, hipStream_t stream) {
  return elementwise(1, "qlora_swiglu_bwd", gate, up, dh, d_gate, d_up, count, stream);
}

int qlora_add_bf16(const uint16_t *a, const uint16_t *b, uint16_t *out, int64_t count, hipStream_t stream) {
  return elementwise(2, "qlora_add_bf16", a, b, nullptr, out, nullptr, count, stream);
}

int qlora_add_bf16_n(const uint16_t *const *xs, int n, uint16_t *out, int64_t count, hipStream_t stream) {
  if (n < 2 || n > 4) return fail(QLORA_ERR_BAD_SHAPE, "n = %d (2..4 summands)", n);
  if (count < 0 || count > kMaxElems) return fail(QLORA_ERR_BAD_SHAPE, "count = %lld", (long long)count);
  if (count == 0) return QLORA_OK;
  if (!xs) return fail(QLORA_ERR_NULL_ARG, "xs is NULL");
  for (int i = 0; i < n; ++i)
    if (int e = check_tensor(xs[i], "summand")) return e;
  if (int e = check_tensor(out, "output")) return e;
  hipError_t e = launch_add_chain(xs, n, out, count, stream);
  if (e != hipSuccess) return hip_fail(e, "qlora_add_bf16_n");
  return QLORA_OK;
}

namespace {
// Shapes the attention calls accept; 0 = valid.
int check_attention(int64_t batch, int64_t seq, int64_t heads, int64_t d) {
  if (batch < 0 || seq < 0 || batch > 65535 || seq > 65536)
    return fail(QLORA_ERR_BAD_SHAPE, "batch = %lld, seq = %lld", (long long)batch, (long long)seq);
  if (heads < 1 || heads > 65535) return fail(QLORA_ERR_BAD_SHAPE, "heads = %lld", (long long)heads);
  if (d < 8 || d > 1024 || d % 8 != 0) return fail(QLORA_ERR_BAD_SHAPE, "head_dim = %lld (8..1024, a multiple of 8)", (long long)d);
  if (batch * seq > kMaxElems / (heads * d)) return fail(QLORA_ERR_BAD_SHAPE, "attention tensors too large");
  if (batch * heads > kMaxElems / (seq * seq + 1)) return fail(QLORA_ERR_BAD_SHAPE, "attention scores too large");
  return QLORA_OK;
}
}  // namespace

size_t qlora_attention_workspace_bytes(int64_t batch, int64_t seq, int64_t heads, int64_t head_dim) {
  if (batch < 0 || seq < 0 || batch > 65535 || seq > 65536 || heads < 1 || heads > 65535 || head_dim < 8 ||
      head_dim > 1024 || head_dim % 8 != 0 || batch * seq > kMaxElems / (heads * head_dim) ||
      batch * heads > kMaxElems / (seq * seq + 1))
    return 0;
  return attention_workspace_bytes(batch, seq, heads, head_dim);
}

int qlora_attention_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *o, float *lse,
                        int64_t batch, int64_t seq, int64_t heads, int64_t head_dim, void *ws, size_t ws_bytes,
                        hipStream_t stream) {
  if (int e = check_attention(batch, seq, heads, head_dim)) return e;
  if (batch == 0 || seq == 0) return QLORA_OK;
  if (int e = check_tensor(q, "q")) return e;
  if (int e = check_tensor(k, "k")) return e;
  if (int e = check_tensor(v, "v")) return e;
  if (int e = check_tensor(o, "o")) return e;
  if (int e = check_tensor(lse, "lse")) return e;
  if (int e = check_ws(ws, ws_bytes, attention_workspace_bytes(batch, seq, heads, head_dim))) return e;
  hipError_t e = launch_attention_fwd(q, k, v, o, lse, batch, seq, heads, head_dim, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "qlora_attention_fwd");
  return QLORA_OK;
}

int qlora_attention_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *d_o, const float *lse,
                        uint16_t *dq, uint16_t *dk, uint16_t *dv,
                        int64_t batch, int64_t seq, int64_t heads, int64_t head_dim, void *ws, size_t ws_bytes,
                        hipStream_t stream) {
  if (int e = check_attention(batch, seq, heads, head_dim)) return e;
  if (batch == 0 || seq == 0) return QLORA_OK;
  const void *ptrs[] = {q, k, v, d_o, lse, dq, dk, dv};
  const char *names[] = {"q", "k", "v", "d_o", "lse", "dq", "dk", "dv"};
  for (int i = 0; i < 8; ++i)
    if (int e = check_tensor(ptrs[i], names[i])) return e;
  if (int e = check_ws(ws, ws_bytes, attention_workspace_bytes(batch, seq, heads, head_dim))) return e;
  hipError_t e = launch_attention_bwd(q, k, v, d_o, lse, dq, dk, dv, batch, seq, heads, head_dim, ws,
                                      stream);
  if (e != hipSuccess) return hip_fail(e, "qlora_attention_bwd");
  return QLORA_OK;
}

int qlora_adamw_step(float *param, uint16_t *param_bf16, const uint16_t *grad, float *m, float *v, int64_t count,
                     float lr, float beta1, float beta2, float eps, float weight_decay, int64_t step, hipStream_t stream) {
  if (count < 0 || count > kMaxElems) return fail(QLORA_ERR_BAD_SHAPE, "count = %lld", (long long)count);
  if (step < 1) return fail(QLORA_ERR_BAD_SHAPE, "step = %lld (counts from 1)", (long long)step);
  if (!std::isfinite(lr) || !std::isfinite(eps) || !std::isfinite(weight_decay) || !(beta1 >= 0.f && beta1 < 1.f) ||
      !(beta2 >= 0.f && beta2 < 1.f) || !(eps > 0.f))
    return fail(QLORA_ERR_BAD_ALPHA, "AdamW hyperparameters out of range");
  if (count == 0) return QLORA_OK;
  if (int e = check_tensor(param, "param")) return e;
  if (int e = check_tensor(grad, "grad")) return e;
  if (int e = check_tensor(m, "m")) return e;
  if (int e = check_tensor(v, "v")) return e;
  if (param_bf16)
    if (int e = check_tensor(param_bf16, "param_bf16")) return e;
  hipError_t e = launch_adamw(param, param_bf16, grad, m, v, count, lr, beta1, beta2, eps, weight_decay, step,
                              stream);
  if (e != hipSuccess) return hip_fail(e, "qlora_adamw_step");
  return QLORA_OK;
}

size_t qlora_merge_workspace_bytes(int64_t n, int64_t k) {
  if (n < 1 || k < kBlock || k % kBlock != 0 || n > kMaxElems / k || k >= kMaxK) return 0;
  return align_up((size_t)(n * k) * sizeof(float), 256) + quantize_ws(n, k);
}

int qlora_merge_adapters(const qlora_weight_ex *wx, const uint16_t *A, const uint16_t *B, int r, float alpha,
                         uint16_t *W_merged, const qlora_weight_ex *outx, void *ws, size_t ws_bytes,
                         hipStream_t s) {
  WeightIn w, out;
  if (int e = take_ex(wx, &w)) return e;
  if (int e = check_weight(w)) return e;
  if (r < 1 || r > 128) return fail(QLORA_ERR_BAD_RANK, "rank r = %d outside [1, 128]", r);
  if (!std::isfinite(alpha)) return fail(QLORA_ERR_BAD_ALPHA, "alpha is not finite");
  if (int e = check_tensor(A, "A")) return e;
  if (int e = check_tensor(B, "B")) return e;
  if (W_merged)
    if (int e = check_tensor(W_merged, "W_merged")) return e;
  if (outx) {
    if (int e = take_ex(outx, &out)) return e;
    if (int e = check_weight(out)) return e;
    if (out.n != w.n || out.k != w.k) return fail(QLORA_ERR_BAD_SHAPE, "out is not [n, k] of w");
  }
  const size_t need = qlora_merge_workspace_bytes(w.n, w.k);
  if (int e = check_ws(ws, ws_bytes, need)) return e;
  float *Wm = static_cast<float *>(ws);
  hipError_t e = launch_merge(view_of(w), A, B, r, (float)alpha / (float)r, Wm, W_merged, s);
  if (e != hipSuccess) return hip_fail(e, "qlora_merge_adapters");
  if (outx) {
    char *qws = static_cast<char *>(ws) + align_up((size_t)(w.n * w.k) * sizeof(float), 256);
    const int64_t nb = out.n * out.k / kBlock;
    const bool single = out.scales == QLORA_SCALES_FP32;
    float *ws_absmax = single ? out.absmax : reinterpret_cast<float *>(qws);
    double *ws_sum = reinterpret_cast<double *>(qws + align_up((size_t)nb * sizeof(float), 256));
    e = launch_quantize(Wm, out.n, out.k, out.codebook, single, out.packed, out.scale_code, out.group_amax,
                        out.offset, ws_absmax, ws_sum, s);
    if (e != hipSuccess) return hip_fail(e, "qlora_merge_adapters (re-encode)");
  }
  return QLORA_OK;
}

size_t qlora_linear_workspace_bytes(int64_t M, int64_t n, int64_t k, int r) {
  if (n < 1 || k < kBlock || k % kBlock != 0 || M < 0 || r < 1 || r > 128) return 0;
  if (n > kMaxElems / k || k >= kMaxK || M > kMaxElems / std::max<int64_t>(k, n)) return 0;
  if (M == 0) return 0;
  return std::max(fwd_workspace_bytes(M, n, k, r), bwd_workspace_bytes(M, n, k, r));
}

namespace {
int fwd_impl(const char *fn, const WeightIn &w, const uint16_t *X, int64_t M, const uint16_t *A, const uint16_t *B,
             int r, float alpha, uint16_t *Y, float *H_out, void *ws, size_t ws_bytes, hipStream_t s) {
  if (int e = check_linear(w, M, r, alpha)) return e;
  if (M == 0) return QLORA_OK;
  if (int e = check_tensor(X, "X")) return e;
  if (int e = check_tensor(A, "A")) return e;
  if (int e = check_tensor(B, "B")) return e;
  if (int e = check_tensor(Y, "Y")) return e;
  if (H_out && !aligned16(H_out)) return fail(QLORA_ERR_MISALIGNED, "H_out is not 16-byte aligned");
  if (int e = check_ws(ws, ws_bytes, fwd_workspace_bytes_for(M, w.n, w.k, r, w.scales == QLORA_SCALES_FP32)))
    return e;
  LinearArgs a{view_of(w), M, r, (float)alpha / (float)r};
  hipError_t e = launch_linear_fwd(a, X, A, B, Y, H_out, ws, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  return QLORA_OK;
}

int bwd_impl(const char *fn, const WeightIn &w, const uint16_t *X, const uint16_t *dY, int64_t M, const uint16_t *A,
             const uint16_t *B, int r, float alpha, const float *H, uint16_t *dX, uint16_t *dA, uint16_t *dB,
             void *ws, size_t ws_bytes, hipStream_t s) {
  if (int e = check_linear(w, M, r, alpha)) return e;
  if (int e = check_tensor(dA, "dA")) return e;
  if (int e = check_tensor(dB, "dB")) return e;
  if (M > 0) {
    if (int e = check_tensor(X, "X")) return e;
    if (int e = check_tensor(dY, "dY")) return e;
    if (int e = check_tensor(A, "A")) return e;
    if (int e = check_tensor(B, "B")) return e;
    if (dX && !aligned16(dX)) return fail(QLORA_ERR_MISALIGNED, "dX is not 16-byte aligned");
    if (H && !aligned16(H)) return fail(QLORA_ERR_MISALIGNED, "H is not 16-byte aligned");
    if (int e = check_ws(ws, ws_bytes, bwd_workspace_bytes(M, w.n, w.k, r))) return e;
  }
  LinearArgs a{view_of(w), M, r, (float)alpha / (float)r};
  hipError_t e = launch_linear_bwd(a, X, dY, A, B, H, dX, dA, dB, ws, s);
  if (e != hipSuccess) return hip_fail(e, fn);
  return QLORA_OK;
}
}  // namespace

int qlora_linear_fwd(const qlora_nf4_weight *w, const uint16_t *X, int64_t M, const uint16_t *A, const uint16_t *B,
                     int r, float alpha, uint16_t *Y, float *H_out, void *ws, size_t ws_bytes, hipStream_t stream) {
  WeightIn v;
  if (int e = take(w, &v)) return e;
  return fwd_impl("qlora_linear_fwd", v, X, M, A, B, r, alpha, Y, H_out, ws, ws_bytes, stream);
}

int qlora_linear_fwd_ex(const qlora_weight_ex *w, const uint16_t *X, int64_t M, const uint16_t *A, const uint16_t *B,
                        int r, float alpha, uint16_t *Y, float *H_out, void *ws, size_t ws_bytes, hipStream_t stream) {
  WeightIn v;
  if (int e = take_ex(w, &v)) return e;
  return fwd_impl("qlora_linear_fwd_ex", v, X, M, A, B, r, alpha, Y, H_out, ws, ws_bytes, stream);
}

int qlora_linear_bwd(const qlora_nf4_weight *w, const uint16_t *X, const uint16_t *dY, int64_t M, const uint16_t *A,
                     const uint16_t *B, int r, float alpha, const float *H, uint16_t *dX, uint16_t *dA,
                     uint16_t *dB, void *ws, size_t ws_bytes, hipStream_t stream) {
  WeightIn v;
  if (int e = take(w, &v)) return e;
  return bwd_impl("qlora_linear_bwd", v, X, dY, M, A, B, r, alpha, H, dX, dA, dB, ws, ws_bytes, stream);
}

int qlora_linear_bwd_ex(const qlora_weight_ex *w, const uint16_t *X, const uint16_t *dY, int64_t M, const uint16_t *A,
                        const uint16_t *B, int r, float alpha, const float *H, uint16_t *dX, uint16_t *dA,
                        uint16_t *dB, void *ws, size_t ws_bytes, hipStream_t stream) {
  WeightIn v;
  if (int e = take_ex(w, &v)) return e;
  return bwd_impl("qlora_linear_bwd_ex", v, X, dY, M, A, B, r, alpha, H, dX, dA, dB, ws, ws_bytes, stream);
}

int qlora_linear_fwd_noalloc(const qlora_nf4_weight *w, const uint16_t *X, int64_t M, const uint16_t *A,
                             const uint16_t *B, int r, float alpha, uint16_t *Y, float *H_out, hipStream_t stream) {
  WeightIn v;
  if (int e = take(w, &v)) return e;
  if (int e = check_linear(v, M, r, alpha)) return e;
  if (M == 0) return QLORA_OK;
  const size_t need = fwd_workspace_bytes_for(M, v.n, v.k, r, false);
  if (need > kNoallocScratchBytes)
    return fail(QLORA_ERR_WORKSPACE,
                "qlora_linear_fwd_noalloc: M = %lld, [%lld, %lld], r = %d needs %zu bytes of scratch, above the "
                "library's fixed %zu",
                (long long)M, (long long)v.n, (long long)v.k, r, need, kNoallocScratchBytes);
  void *ptr = nullptr;
  if (int e = device_scratch(&ptr)) return e;
  return fwd_impl("qlora_linear_fwd_noalloc", v, X, M, A, B, r, alpha, Y, H_out, ptr, kNoallocScratchBytes, stream);
}

int qlora_linear_plan(int64_t M, int64_t n, int64_t k, int r, int32_t scales, qlora_linear_plan_info *out) {
  if (!out) return fail(QLORA_ERR_NULL_ARG, "out is NULL");
  if (scales != QLORA_SCALES_DQ && scales != QLORA_SCALES_FP32)
    return fail(QLORA_ERR_BAD_CODEBOOK, "scales %d is neither DQ (0) nor FP32 (1)", (int)scales);
  if (int e = check_linear_shape(n, k, M, r)) return e;
  const LinearPlan p = plan_linear(M, n, k, r, scales == QLORA_SCALES_FP32);
  out->fwd_path = p.fwd_path;
  out->fwd_splits = p.fwd_splits;
  out->dx_path = p.dx_path;
  out->dx_splits = p.dx_splits;
  return QLORA_OK;
}

void qlora_nf4_codebook(float out[16]) { qlora_codebook(QLORA_CODEBOOK_NF4, out); }

void qlora_nf4_thresholds(float out[15]) { qlora_thresholds(QLORA_CODEBOOK_NF4, out); }

int qlora_codebook(int codebook, float out[16]) {
  if (!known_codebook(codebook)) return fail(QLORA_ERR_BAD_CODEBOOK, "unknown codebook %d", codebook);
  if (!out) return fail(QLORA_ERR_NULL_ARG, "out is NULL");
  for (int j = 0; j < 16; ++j) std::memcpy(&out[j], &codebook_bits(codebook)[j], 4);
  return QLORA_OK;
}

int qlora_thresholds(int codebook, float out[15]) {
  if (!known_codebook(codebook)) return fail(QLORA_ERR_BAD_CODEBOOK, "unknown codebook %d", codebook);
  if (!out) return fail(QLORA_ERR_NULL_ARG, "out is NULL");
  const Thresholds &t = codebook_thresholds(codebook);
  for (int j = 0; j < 15; ++j) out[j] = t.t[j];
  return QLORA_OK;
}

const char *qlora_strerror(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL_ARG: return "null argument";
    case QLORA_ERR_BAD_SHAPE: return "bad shape";
    case QLORA_ERR_BAD_RANK: return "bad LoRA rank";
    case QLORA_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case QLORA_ERR_WORKSPACE: return "workspace missing or too small";
    case QLORA_ERR_HIP: return "HIP runtime error";
    case QLORA_ERR_BAD_ALPHA: return "alpha is not finite";
    case QLORA_ERR_BAD_CODEBOOK: return "unknown codebook";
    default: return "unknown status";
  }
}

const char *qlora_last_error(void) { return g_last_error; }

}  // extern "C"

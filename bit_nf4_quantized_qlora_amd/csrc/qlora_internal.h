// qlora_internal.h -- host-side launch interface between the C ABI (capi.hip)
// and the kernel translation units.  Not part of the public API.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlora_device.h"

namespace qlora {

// Read-only view of a quantized weight as the kernels take it.
struct Nf4View {
  int64_t n, k;
  int64_t nb;  // n*k/64 blocks
  int64_t ng;  // ceil(nb/256) groups
  const uint8_t *packed;
  const uint8_t *scale_code;
  const float *group_amax;
  const float *offset;
  int codebook;         // kCodebookNF4, kCodebookFP4 or kCodebookE3M0
  const float *absmax;  // single-level block constants (s_b = absmax_b); NULL: double quantization
};

// Decision thresholds of a codebook (kCodebookNF4 / kCodebookFP4 / kCodebookE3M0).
const Thresholds &codebook_thresholds(int codebook);

// quantize.hip
// single_level: write the block absmax to ws_absmax (the caller's absmax
// buffer) and skip the second level.
hipError_t launch_quantize(const float *W, int64_t n, int64_t k, int codebook, bool single_level, uint8_t *packed,
                           uint8_t *scale_code, float *group_amax, float *offset, float *ws_absmax,
                           double *ws_group_sum, hipStream_t s);

// dequant.hip
hipError_t launch_dequant(const Nf4View &w, uint16_t *out, hipStream_t s);

// swiglu.hip: op 0 y0 = bf16(silu(x0) x1); op 1 (y0, y1) = (dg, du) for
// g = x0, u = x1, dh = x2; op 2 y0 = bf16(x0 + x1).
// Causal attention core (attention.hip).
size_t attention_workspace_bytes(int64_t batch, int64_t seq, int64_t heads, int64_t d);
hipError_t launch_attention_fwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V, uint16_t *O, float *lse,
                                int64_t batch, int64_t seq, int64_t heads, int64_t d, void *ws, hipStream_t s);
hipError_t launch_attention_bwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const uint16_t *dO, const float *lse, uint16_t *dQ, uint16_t *dK, uint16_t *dV,
                                int64_t batch, int64_t seq, int64_t heads, int64_t d, void *ws, hipStream_t s);
hipError_t launch_swiglu(int op, const uint16_t *x0, const uint16_t *x1, const uint16_t *x2, uint16_t *y0,
                         uint16_t *y1, int64_t count, hipStream_t s);
// y = the left-to-right bf16-rounded sum of xs[0 .. n-1], 2 <= n <= 4.
hipError_t launch_add_chain(const uint16_t *const *xs, int n, uint16_t *y, int64_t count, hipStream_t s);

// adamw.hip: one AdamW step over count parameters (m, v may be host memory
// the device addresses).
hipError_t launch_adamw(float *P, uint16_t *P16, const uint16_t *G, float *M, float *V, int64_t count, float lr,
                        float b1, float b2, float eps, float wd, int64_t step, hipStream_t s);

// merge.hip: Wm [n, k] float32 = W_hat + s B A (fixed float64 order), and
// its bf16 rounding into Wb when Wb != NULL.
hipError_t launch_merge(const Nf4View &w, const uint16_t *A, const uint16_t *B, int r, float s, float *Wm,
                        uint16_t *Wb, hipStream_t st);

// linear_fwd.hip / linear_bwd.hip
struct LinearArgs {
  Nf4View w;
  int64_t M;
  int r;
  float s;  // fp32(alpha / r)
};

size_t fwd_workspace_bytes(int64_t M, int64_t n, int64_t k, int r);
// The forward workspace of the path one storage type's call takes.
size_t fwd_workspace_bytes_for(int64_t M, int64_t n, int64_t k, int r, bool single_level);

// The kernels a call of this shape runs (QLORA_PATH_*; splits of the tile
// launches' contraction): the one decision the launches and
// qlora_linear_plan share.
struct LinearPlan {
  int fwd_path = QLORA_PATH_NONE, fwd_splits = 1;
  int dx_path = QLORA_PATH_NONE, dx_splits = 1;
};
LinearPlan plan_linear(int64_t M, int64_t n, int64_t k, int r, bool single_level);
size_t bwd_workspace_bytes(int64_t M, int64_t n, int64_t k, int r);

hipError_t launch_linear_fwd(const LinearArgs &a, const uint16_t *X, const uint16_t *A, const uint16_t *B,
                             uint16_t *Y, float *H_out, void *ws, hipStream_t s);
#ifdef QLORA_PROFILE
hipError_t launch_linear_fwd_bf16w(const uint16_t *Wb, int64_t N, int64_t K, int64_t M, int r, float s_lora,
                                   const uint16_t *X, const uint16_t *A, const uint16_t *B, uint16_t *Y, float *H_out,
                                   void *ws, hipStream_t s);
#endif
hipError_t launch_linear_bwd(const LinearArgs &a, const uint16_t *X, const uint16_t *dY, const uint16_t *A,
                             const uint16_t *B, const float *H, uint16_t *dX, uint16_t *dA, uint16_t *dB,
                             void *ws, hipStream_t s);

#ifdef QLORA_PROFILE
// Per-kernel event timing, compiled into the separate tracing build
// libqlora_prof.so only (profile.hip): a scope around each launch.  The
// product library has no timer and no state behind it.
class ProfScope {
 public:
  ProfScope(const char *name, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope &) = delete;
  ProfScope &operator=(const ProfScope &) = delete;

 private:
  const char *name_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
};

#define QLORA_LAUNCH(name, kernel, grid, block, shmem, stream, ...)            \
  do {                                                                         \
    ::qlora::ProfScope qlora_prof_scope_(name, stream);                        \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);       \
  } while (0)
#else
#define QLORA_LAUNCH(name, kernel, grid, block, shmem, stream, ...) \
  hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__)
#endif

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace qlora

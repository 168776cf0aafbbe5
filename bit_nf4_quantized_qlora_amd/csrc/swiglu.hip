// swiglu.hip -- the elementwise pieces of the MLP block around the linears:
// the SwiGLU gate between the gate/up and down projections, its backward,
// and the bf16 sum of the two input gradients.
//
// The reading note places adapters on every linear layer, so the block's
// backward runs each projection's frozen-base backward in turn; the pages
// give no activation, and the LLaMA MLP whose shapes the workloads use
// gates with SwiGLU: h = silu(g) u, silu(x) = x sigma(x).  float32 inside,
// one bf16 rounding per output; expf is the device library's.
//
// HBM-bound: 4 B in + 2 B out per element forward, 6 B in + 4 B out
// backward, 4 + 2 for the sum.  Eight elements (16-byte accesses) per
// thread; the ragged tail element by element.
#include "lora_gemm.h"

namespace qlora {
namespace {

__device__ __forceinline__ float bf(uint32_t word, int hi) { return __uint_as_float(hi ? word & 0xFFFF0000u : word << 16); }
// e^-|x| never overflows: far below zero sigma keeps its (subnormal-range)
// value instead of 1/inf = 0
__device__ __forceinline__ float sigmoid(float x) {
  const float e = expf(-fabsf(x));
  return x >= 0.f ? 1.0f / (1.0f + e) : e / (1.0f + e);
}

template <int kOp>  // 0: h = silu(g) u;  1: (dg, du);  2: a + b
__global__ __launch_bounds__(256) void k_elementwise(const uint16_t *__restrict__ x0, const uint16_t *__restrict__ x1,
                                                     const uint16_t *__restrict__ x2, uint16_t *__restrict__ y0,
                                                     uint16_t *__restrict__ y1, int64_t count) {
  const int64_t i0 = 8 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (i0 >= count) return;
  auto one = [&](float a, float b, float c, float &o0, float &o1) {
    if constexpr (kOp == 0) {
      o0 = a * sigmoid(a) * b;
    } else if constexpr (kOp == 1) {
      const float s = sigmoid(a);
      o1 = c * (a * s);                          // du = dh silu(g)
      o0 = c * b * (s * (1.0f + a * (1.0f - s)));  // dg = dh u silu'(g)
    } else {
      o0 = a + b;
    }
  };
  if (i0 + 8 <= count) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(x0 + i0);
    const u32x4_t b = *reinterpret_cast<const u32x4_t *>(x1 + i0);
    u32x4_t c = {0u, 0u, 0u, 0u};
    if constexpr (kOp == 1) c = *reinterpret_cast<const u32x4_t *>(x2 + i0);
    u32x4_t r0, r1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float lo0, lo1 = 0.f, hi0, hi1 = 0.f;
      one(bf(a[q], 0), bf(b[q], 0), bf(c[q], 0), lo0, lo1);
      one(bf(a[q], 1), bf(b[q], 1), bf(c[q], 1), hi0, hi1);
      r0[q] = bf16x2_rne(lo0, hi0);
      r1[q] = bf16x2_rne(lo1, hi1);
    }
    *reinterpret_cast<u32x4_t *>(y0 + i0) = r0;
    if constexpr (kOp == 1) *reinterpret_cast<u32x4_t *>(y1 + i0) = r1;
  } else {
    for (int64_t i = i0; i < count; ++i) {
      float o0, o1 = 0.f;
      one(bf(x0[i], 0), bf(x1[i], 0), kOp == 1 ? bf(x2[i], 0) : 0.f, o0, o1);
      y0[i] = f32_to_bf16_bits(o0);
      if constexpr (kOp == 1) y1[i] = f32_to_bf16_bits(o1);
    }
  }
}

// out = bf16(...bf16(bf16(x0 + x1) + x2)... + x[n-1]), n = 2..4: each
// addition in float32 and rounded to bf16 before the next, left to right --
// the same operations, in the same order, as n - 1 chained k_add_bf16
// launches, in one pass (no intermediate written or read back).
__global__ __launch_bounds__(256) void k_add_chain(const uint16_t *__restrict__ x0, const uint16_t *__restrict__ x1,
                                                   const uint16_t *__restrict__ x2, const uint16_t *__restrict__ x3,
                                                   int n, uint16_t *__restrict__ y, int64_t count) {
  const int64_t i0 = 8 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (i0 >= count) return;
  auto rnd = [](float v) { return __uint_as_float((uint32_t)f32_to_bf16_bits(v) << 16); };
  if (i0 + 8 <= count) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(x0 + i0);
    const u32x4_t b = *reinterpret_cast<const u32x4_t *>(x1 + i0);
    u32x4_t c = {0u, 0u, 0u, 0u}, d = {0u, 0u, 0u, 0u};
    if (n > 2) c = *reinterpret_cast<const u32x4_t *>(x2 + i0);
    if (n > 3) d = *reinterpret_cast<const u32x4_t *>(x3 + i0);
    u32x4_t r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float lo = bf(a[q], 0) + bf(b[q], 0), hi = bf(a[q], 1) + bf(b[q], 1);
      if (n > 2) {
        lo = rnd(lo) + bf(c[q], 0);
        hi = rnd(hi) + bf(c[q], 1);
      }
      if (n > 3) {
        lo = rnd(lo) + bf(d[q], 0);
        hi = rnd(hi) + bf(d[q], 1);
      }
      r[q] = bf16x2_rne(lo, hi);
    }
    *reinterpret_cast<u32x4_t *>(y + i0) = r;
  } else {
    for (int64_t i = i0; i < count; ++i) {
      float v = bf(x0[i], 0) + bf(x1[i], 0);
      if (n > 2) v = rnd(v) + bf(x2[i], 0);
      if (n > 3) v = rnd(v) + bf(x3[i], 0);
      y[i] = f32_to_bf16_bits(v);
    }
  }
}

}  // namespace

hipError_t launch_add_chain(const uint16_t *const *xs, int n, uint16_t *y, int64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(ceil_div(count, 8), 256));
  QLORA_LAUNCH("k_add_chain", k_add_chain, grid, dim3(256), 0, s, xs[0], xs[1], n > 2 ? xs[2] : nullptr,
               n > 3 ? xs[3] : nullptr, n, y, count);
  return hipGetLastError();
}

hipError_t launch_swiglu(int op, const uint16_t *x0, const uint16_t *x1, const uint16_t *x2, uint16_t *y0,
                         uint16_t *y1, int64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(ceil_div(count, 8), 256));
  if (op == 0) QLORA_LAUNCH("k_swiglu_fwd", k_elementwise<0>, grid, dim3(256), 0, s, x0, x1, x2, y0, y1, count);
  else if (op == 1) QLORA_LAUNCH("k_swiglu_bwd", k_elementwise<1>, grid, dim3(256), 0, s, x0, x1, x2, y0, y1, count);
  else QLORA_LAUNCH("k_add_bf16", k_elementwise<2>, grid, dim3(256), 0, s, x0, x1, x2, y0, y1, count);
  return hipGetLastError();
}

}  // namespace qlora

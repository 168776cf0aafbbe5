// adamw.hip -- one AdamW step on an adapter tensor.
//
// "QLoRA Paper Breakdown" section 5: the adapters' Adam moments are the
// paged state, read back on demand by the optimizer step; "QLoRA,
// explained." step 6.  The pages print no update rule; the published AdamW
// (decoupled weight decay, bias-corrected moments) in float32, each
// operation rounded on its own, in this order:
//   g = float(grad);  m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) (g g)
//   p = p decay - step_size (m / (sqrt(v) / sqrt_bc2 + eps))
// decay, step_size and sqrt_bc2 come from the host (float64, rounded once).
//
// Memory-bound: 14 B read and 14 B written per parameter (p, m, v float32,
// grad and the bf16 copy 2 B).  m and v may be host memory the device
// addresses directly (the paged layout): the same loads then cross the
// host link.  Four parameters per thread, 16-byte accesses.
#include "lora_gemm.h"

namespace qlora {
namespace {

struct AdamCoef {
  float b1, omb1, b2, omb2, eps, decay, step_size, sqrt_bc2;
};

__device__ __forceinline__ void adam_one(float &p, float &m, float &v, float g, const AdamCoef &c) {
  m = __fadd_rn(__fmul_rn(c.b1, m), __fmul_rn(c.omb1, g));
  v = __fadd_rn(__fmul_rn(c.b2, v), __fmul_rn(c.omb2, __fmul_rn(g, g)));
  const float denom = __fadd_rn(__fdiv_rn(__fsqrt_rn(v), c.sqrt_bc2), c.eps);
  p = __fsub_rn(__fmul_rn(p, c.decay), __fmul_rn(c.step_size, __fdiv_rn(m, denom)));
}

__global__ __launch_bounds__(256) void k_adamw(float *__restrict__ P, uint16_t *__restrict__ P16,
                                               const uint16_t *__restrict__ G, float *__restrict__ Mo,
                                               float *__restrict__ Vo, int64_t count, AdamCoef c) {
  const int64_t i0 = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (i0 >= count) return;
  if (i0 + 4 <= count) {
    f32x4_t p = *reinterpret_cast<const f32x4_t *>(P + i0);
    f32x4_t m = *reinterpret_cast<const f32x4_t *>(Mo + i0);
    f32x4_t v = *reinterpret_cast<const f32x4_t *>(Vo + i0);
    const u32x2_t gb = *reinterpret_cast<const u32x2_t *>(G + i0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t word = gb[e >> 1];
      const float g = __uint_as_float(e & 1 ? word & 0xFFFF0000u : word << 16);
      float pe = p[e], me = m[e], ve = v[e];
      adam_one(pe, me, ve, g, c);
      p[e] = pe;
      m[e] = me;
      v[e] = ve;
    }
    *reinterpret_cast<f32x4_t *>(P + i0) = p;
    *reinterpret_cast<f32x4_t *>(Mo + i0) = m;
    *reinterpret_cast<f32x4_t *>(Vo + i0) = v;
    if (P16) *reinterpret_cast<u32x2_t *>(P16 + i0) = u32x2_t{bf16x2_rne(p[0], p[1]), bf16x2_rne(p[2], p[3])};
  } else {
    for (int64_t i = i0; i < count; ++i) {
      float pe = P[i], me = Mo[i], ve = Vo[i];
      adam_one(pe, me, ve, __uint_as_float((uint32_t)G[i] << 16), c);
      P[i] = pe;
      Mo[i] = me;
      Vo[i] = ve;
      if (P16) P16[i] = f32_to_bf16_bits(pe);
    }
  }
}

}  // namespace

hipError_t launch_adamw(float *P, uint16_t *P16, const uint16_t *G, float *M, float *V, int64_t count, float lr,
                        float b1, float b2, float eps, float wd, int64_t step, hipStream_t s) {
  if (count == 0) return hipSuccess;
  AdamCoef c;
  c.b1 = b1;
  c.omb1 = (float)(1.0 - (double)b1);
  c.b2 = b2;
  c.omb2 = (float)(1.0 - (double)b2);
  c.eps = eps;
  c.decay = (float)(1.0 - (double)lr * (double)wd);
  c.step_size = (float)((double)lr / (1.0 - std::pow((double)b1, (double)step)));
  c.sqrt_bc2 = (float)std::sqrt(1.0 - std::pow((double)b2, (double)step));
  QLORA_LAUNCH("k_adamw", k_adamw, dim3((unsigned)ceil_div(ceil_div(count, 4), 256)), dim3(256), 0, s, P, P16, G, M,
               V, count, c);
  return hipGetLastError();
}

}  // namespace qlora

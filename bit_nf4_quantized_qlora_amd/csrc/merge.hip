// merge.hip -- folding trained LoRA adapters into the frozen base.
//
// "QLoRA Paper Breakdown" section 'Limitations': full-rank updates need the
// adapters merged into 16-bit weights; section 4's forward pass fixes what
// the merged weight is, W_hat + s B A (n x k).  The pages fix no arithmetic;
// the library's definition, one float32 tensor:
//   t = sum over j = 0 .. r-1, in that order, of B[n][j] * A[j][k] (float64;
//       each bf16 x bf16 product is exact),
//   W' = float32( float64(w_hat) + float64(s) * t ),  s = float32(alpha / r),
// every float64 operation separately rounded.  W' feeds the encoder
// (re-quantization) and, rounded to bf16, the merged 16-bit weight.
//
// One thread per packed dword (8 weights of one row): the dword's BF16
// weights through the same dequant_word as every other consumer, the row's
// B values and the 8 columns of A per rank index.  A deployment-time pass:
// r float64 multiply-adds per weight.
#include "lora_gemm.h"

namespace qlora {
namespace {

__global__ __launch_bounds__(256) void k_merge(Nf4View w, const uint16_t *__restrict__ A,
                                               const uint16_t *__restrict__ B, int r, float s,
                                               float *__restrict__ Wm, uint16_t *__restrict__ Wb) {
  __shared__ float2 s_pair[256];
  fill_pair_table(s_pair, threadIdx.x, 256, w.codebook);
  __syncthreads();
  const int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x;  // packed dword: weights 8d .. 8d+7
  const int64_t ndw = w.n * w.k / 8;
  if (d >= ndw) return;
  const int64_t e0 = 8 * d, n = e0 / w.k, k0 = e0 - n * w.k;
  const int64_t b = e0 / kBlock;
  const float sb = w.absmax ? w.absmax[b] : block_scale(w.scale_code[b], w.group_amax[b / kGroup], *w.offset);
  uint32_t wb[4];
  dequant_word(reinterpret_cast<const uint32_t *>(w.packed)[d], sb, s_pair, wb);
  double t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = 0.0;
  const uint16_t *brow = B + n * r;
  for (int j = 0; j < r; ++j) {
    const double bj = (double)__uint_as_float((uint32_t)brow[j] << 16);
    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(A + (int64_t)j * w.k + k0);  // k0 % 8 == 0
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double aj = (double)__uint_as_float(e & 1 ? a[e >> 1] & 0xFFFF0000u : a[e >> 1] << 16);
      t[e] = __dadd_rn(t[e], __dmul_rn(bj, aj));
    }
  }
  const double sd = (double)s;
  float out[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double wh = (double)__uint_as_float(e & 1 ? wb[e >> 1] & 0xFFFF0000u : wb[e >> 1] << 16);
    out[e] = __double2float_rn(__dadd_rn(wh, __dmul_rn(sd, t[e])));
  }
  f32x4_t *dst = reinterpret_cast<f32x4_t *>(Wm + e0);
  dst[0] = f32x4_t{out[0], out[1], out[2], out[3]};
  dst[1] = f32x4_t{out[4], out[5], out[6], out[7]};
  if (Wb)
    *reinterpret_cast<u32x4_t *>(Wb + e0) = u32x4_t{bf16x2_rne(out[0], out[1]), bf16x2_rne(out[2], out[3]),
                                                     bf16x2_rne(out[4], out[5]), bf16x2_rne(out[6], out[7])};
}

}  // namespace

hipError_t launch_merge(const Nf4View &w, const uint16_t *A, const uint16_t *B, int r, float s, float *Wm,
                        uint16_t *Wb, hipStream_t st) {
  const int64_t ndw = w.n * w.k / 8;
  QLORA_LAUNCH("k_merge", k_merge, dim3((unsigned)ceil_div(ndw, 256)), dim3(256), 0, st, w, A, B, r, s, Wm, Wb);
  return hipGetLastError();
}

}  // namespace qlora

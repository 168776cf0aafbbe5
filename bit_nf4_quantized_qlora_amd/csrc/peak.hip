// peak.hip -- the attainable BF16 matrix-core rate of the GPU it runs on
// (tracing build only: a measurement denominator, not part of the layer).
//
// Each wave issues v_mfma_f32_16x16x32_bf16 -- the instruction the tile
// kernels use -- back to back on eight independent accumulator tiles held in
// AGPRs, with constant operands and no memory traffic inside the loop, so
// the only limit is the matrix pipes (and the clock the chip holds while
// they are all busy).  Two 4-wave workgroups per CU keep two waves on every
// SIMD.  The accumulators are written out at the end so nothing is dead code.
#include "../../include/qlora_profile.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int kPeakAcc = 8;  // independent accumulator tiles per wave

__global__ __launch_bounds__(256) void k_mfma_peak(int64_t iters, float *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  // operands: any finite bf16 values (1.0 and 2^-8 patterns), distinct per lane
  const uint32_t va = 0x3f803f80u ^ (uint32_t)(lane & 1), vb = 0x3b803b80u;
  const u32x4_t a = {va, va, va, va}, b = {vb, vb, vb, vb};
  f32x4_t acc[kPeakAcc];
#pragma unroll
  for (int j = 0; j < kPeakAcc; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kPeakAcc; ++j) mfma16_acc(acc[j], a, b);
  }
  mfma_acc_fence();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kPeakAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace
}  // namespace qlora

using namespace qlora;

extern "C" {

int qlora_profile_mfma_peak(int64_t iters, int32_t workgroups, float *out, double *flops, hipStream_t stream) {
  if (iters < 1 || workgroups < 1 || !out) return QLORA_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(k_mfma_peak, dim3((unsigned)workgroups), dim3(256), 0, stream, iters, out);
  if (hipGetLastError() != hipSuccess) return QLORA_ERR_HIP;
  if (flops) *flops = 2.0 * 16 * 16 * 32 * (double)kPeakAcc * (double)iters * 4.0 * (double)workgroups;
  return QLORA_OK;
}

}  // extern "C"

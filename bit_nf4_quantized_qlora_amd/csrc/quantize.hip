// quantize.hip -- NF4 + double-quantization encoder for gfx950.
//
// "QLoRA, explained." steps 1-3 and "QLoRA Paper Breakdown" sec. 3 (Level 1:
// blockwise absmax and nearest NF4 code; Level 2: mean-subtracted block
// constants coded to 8-bit floats with one fp32 constant per 256).
//
// Three launches, all HBM-streaming:
//   k_quantize_blocks  one workgroup per group of 256 blocks (64 KiB of W):
//                      absmax, codes, packed nibbles, and the group's fp64
//                      in-order absmax sum;
//   k_mean             one workgroup: group sums staged in LDS, each lane of
//                      a wave folds one run of 256 of them in order, then
//                      one lane the run sums -> offset;
//   k_encode_scales    one wave per group: dev = absmax - offset, group amax,
//                      E4M3 codes.
#include "qlora_internal.h"

namespace qlora {
namespace {

// a if b else c, as a bit blend: the operands are wave-uniform thresholds
// in scalar registers, so this stays a register select (a conditional
// element choice would be turned into an indexed load from a stack copy of
// the threshold array).
__device__ __forceinline__ float pick(bool b, float a, float c) {
  const uint32_t m = 0u - (uint32_t)b;
  return __uint_as_float((__float_as_uint(a) & m) | (__float_as_uint(c) & ~m));
}

// Index of the nearest NF4 level from the 15 thresholds: a 4-step binary
// search (each step a compare and selects between uniform thresholds).
__device__ __forceinline__ uint32_t nf4_code(float x, const float (&t)[15]) {
  const bool b3 = x >= t[7];
  const bool b2 = x >= pick(b3, t[11], t[3]);
  const bool b1 = x >= pick(b3, pick(b2, t[13], t[9]), pick(b2, t[5], t[1]));
  const float t0 = pick(b3, pick(b2, pick(b1, t[14], t[12]), pick(b1, t[10], t[8])),
                        pick(b2, pick(b1, t[6], t[4]), pick(b1, t[2], t[0])));
  const bool b0 = x >= t0;
  return (uint32_t(b3) << 3) | (uint32_t(b2) << 2) | (uint32_t(b1) << 1) | uint32_t(b0);
}

// Eight consecutive weights per lane, eight lanes per 64-weight block, so a
// wave covers 8 blocks (2 KiB) per step and a workgroup of 4 waves covers one
// group of 256 blocks in 8 steps.
__global__ __launch_bounds__(256) void k_quantize_blocks(const float *__restrict__ W, int64_t nb,
                                                         Thresholds T, uint8_t *__restrict__ packed,
                                                         float *__restrict__ absmax_out,
                                                         double *__restrict__ group_sum) {
  __shared__ float s_absmax[kGroup];
  float t[15];  // the thresholds in (scalar) registers
#pragma unroll
  for (int j = 0; j < 15; ++j) t[j] = T.t[j];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t first = (int64_t)blockIdx.x * kGroup;
  const int nblk = (int)min<int64_t>(kGroup, nb - first);

#pragma unroll 2
  for (int step = 0; step < 8; ++step) {
    const int lb = wave * 64 + step * 8 + (lane >> 3);  // block within the group
    const bool valid = lb < nblk;
    const int64_t e0 = (first + lb) * kBlock + (lane & 7) * 8;
    f32x4_t v0 = {0.f, 0.f, 0.f, 0.f}, v1 = v0;
    if (valid) {
      v0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(W + e0));
      v1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(W + e0) + 1);
    }
    float m = fmaxf(fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))),
                    fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)), fmaxf(fabsf(v1.z), fabsf(v1.w))));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    m = fmaxf(m, __shfl_xor(m, 4, 64));
    if (valid) {
      const float w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // IEEE round-to-nearest division; an all-zero block normalizes to 0.
        const float x = m > 0.f ? __fdiv_rn(w[i], m) : 0.f;
        word |= nf4_code(x, t) << (4 * i);
      }
      *reinterpret_cast<uint32_t *>(packed + e0 / 2) = word;
      if ((lane & 7) == 0) {
        absmax_out[first + lb] = m;
        s_absmax[lb] = m;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // block order; eight LDS reads in flight per batch
    double acc = 0.0;
    int i = 0;
    for (; i + 8 <= nblk; i += 8) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = s_absmax[i + q];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc += (double)v[q];
    }
    for (; i < nblk; ++i) acc += (double)s_absmax[i];
    group_sum[blockIdx.x] = acc;
  }
}

// offset = fp32( total / nb ) with the mean's fixed float64 order: each
// run of kMeanRun consecutive group sums folded left to right, then the run
// sums folded left to right.  One 1024-lane workgroup takes kMeanRuns runs
// per pass: every lane stages its share of their group sums in LDS (all
// loads issued before any store, one memory round trip), lane t of the
// first wave folds run t from LDS (reads a batch ahead of the adds; rows
// kMeanLd apart, so the lanes' reads spread over the banks), and lane 0
// folds the pass's run sums into the total.  Sums are non-negative, so the
// zeros that pad a short last run leave it unchanged.
constexpr int kMeanRun = 256;               // group sums per run
constexpr int kMeanRuns = 64;               // runs per pass (one wave)
constexpr int kMeanLd = kMeanRun + 1;       // LDS stride of a staged run (doubles)
constexpr int kMeanLanes = 1024;
constexpr int kMeanPer = kMeanRuns * kMeanRun / kMeanLanes;  // staged sums per lane and pass
__global__ __launch_bounds__(kMeanLanes) void k_mean(const double *__restrict__ group_sum, int64_t ng, int64_t nb,
                                                     float *__restrict__ offset) {
  constexpr int B = 16;  // LDS reads ahead of the adds
  __shared__ double s_sum[kMeanRuns * kMeanLd];
  __shared__ double s_run[kMeanRuns];
  const int64_t nruns = (ng + kMeanRun - 1) / kMeanRun;
  double total = 0.0;  // lane 0's fold of the run sums
  for (int64_t r0 = 0; r0 < nruns; r0 += kMeanRuns) {
    const int64_t g0 = r0 * kMeanRun;
    const int64_t n = min<int64_t>(kMeanRuns * kMeanRun, ng - g0);  // group sums of this pass
    double v[kMeanPer];
#pragma unroll
    for (int u = 0; u < kMeanPer; ++u) {
      const int e = (int)threadIdx.x + kMeanLanes * u;
      v[u] = e < n ? group_sum[g0 + e] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < kMeanPer; ++u) {
      const int e = (int)threadIdx.x + kMeanLanes * u;
      s_sum[(e / kMeanRun) * kMeanLd + e % kMeanRun] = v[u];
    }
    __syncthreads();
    if (threadIdx.x < kMeanRuns) {
      const double *p = s_sum + threadIdx.x * kMeanLd;
      double acc = 0.0, cur[B];
#pragma unroll
      for (int q = 0; q < B; ++q) cur[q] = p[q];
      for (int i = 0; i < kMeanRun; i += B) {
        double nx[B];
#pragma unroll
        for (int q = 0; q < B; ++q) nx[q] = i + B < kMeanRun ? p[i + B + q] : 0.0;
#pragma unroll
        for (int q = 0; q < B; ++q) acc += cur[q];
#pragma unroll
        for (int q = 0; q < B; ++q) cur[q] = nx[q];
      }
      s_run[threadIdx.x] = acc;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      const int m = (int)min<int64_t>(kMeanRuns, nruns - r0);
      for (int i = 0; i < m; ++i) total += s_run[i];
    }
    __syncthreads();  // the next pass overwrites s_sum and s_run
  }
  if (threadIdx.x == 0) *offset = (float)(total / (double)nb);
}

// One wave per group, four block constants per lane.
__global__ __launch_bounds__(256) void k_encode_scales(const float *__restrict__ absmax, int64_t nb,
                                                       int64_t ng, const float *__restrict__ offset_p,
                                                       uint8_t *__restrict__ scale_code,
                                                       float *__restrict__ group_amax) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= ng) return;
  const float offset = *offset_p;
  const int64_t b0 = g * kGroup + lane * 4;
  float dev[4];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dev[i] = 0.f;
    if (b0 + i < nb) {
      dev[i] = __fsub_rn(absmax[b0 + i], offset);
      m = fmaxf(m, fabsf(dev[i]));
    }
  }
  m = wave_max(m);
  uint32_t codes = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t c = m > 0.f ? e4m3_encode_rne(__fdiv_rn(dev[i], m)) : 0u;
    codes |= c << (8 * i);
  }
  if (b0 + 4 <= nb) {
    *reinterpret_cast<uint32_t *>(scale_code + b0) = codes;
  } else {
    for (int i = 0; i < 4; ++i)
      if (b0 + i < nb) scale_code[b0 + i] = (uint8_t)(codes >> (8 * i));
  }
  if (lane == 0) group_amax[g] = m;
}

}  // namespace

hipError_t launch_quantize(const float *W, int64_t n, int64_t k, int codebook, bool single_level, uint8_t *packed,
                           uint8_t *scale_code,
                           float *group_amax, float *offset, float *ws_absmax, double *ws_group_sum,
                           hipStream_t s) {
  const int64_t nb = n * k / kBlock;
  const int64_t ng = ceil_div(nb, kGroup);
  QLORA_LAUNCH("k_quantize_blocks", k_quantize_blocks, dim3((unsigned)ng), dim3(256), 0, s, W, nb, codebook_thresholds(codebook), packed,
                     ws_absmax, ws_group_sum);
  if (single_level) return hipGetLastError();
  QLORA_LAUNCH("k_mean", k_mean, dim3(1), dim3(kMeanLanes), 0, s, ws_group_sum, ng, nb, offset);
  QLORA_LAUNCH("k_encode_scales", k_encode_scales, dim3((unsigned)ceil_div(ng, 4)), dim3(256), 0, s, ws_absmax, nb, ng,
                     offset, scale_code, group_amax);
  return hipGetLastError();
}

}  // namespace qlora

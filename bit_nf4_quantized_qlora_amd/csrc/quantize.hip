// quantize.hip -- NF4 + double-quantization encoder for gfx950.
//
// "QLoRA, explained." steps 1-3 and "QLoRA Paper Breakdown" sec. 3 (Level 1:
// blockwise absmax and nearest NF4 code; Level 2: mean-subtracted block
// constants coded to 8-bit floats with one fp32 constant per 256).
//
// Two or three launches:
//   k_quantize_blocks  one workgroup per group of 256 blocks (64 KiB of W):
//                      absmax, codes, packed nibbles, and the group's fp64
//                      in-order absmax sum (HBM-streaming);
//   k_mean             one workgroup: group sums staged in LDS, each lane of
//                      a wave folds one run of 256 of them in order, then
//                      one lane the run sums -> offset;
//   k_encode_scales    one wave per group: dev = absmax - offset, group amax,
//                      E4M3 codes;
//   k_mean_encode      the last two in one launch for tensors of at most
//                      16384 groups (each workgroup folds the mean itself).
#include "qlora_internal.h"

namespace qlora {
namespace {

// Nearest-level code from a 129-entry table: code(x) = #{ j : x >= t[j] }
// for x = w / absmax in [-1, 1].  Bucket i = floor(64 x) + 64 covers
// [(i - 64)/64, (i - 63)/64) (x = 1 alone in bucket 128); 64 x is exact, so
// the bucket is too.  Entry i holds the count of thresholds at or below the
// bucket's lower edge and the one threshold strictly inside it (+inf if
// none), so code = count + (x >= inside).  No bucket of any of the three
// codebooks holds two thresholds (NF4's and E2M1's are more than 1/64
// apart; E3M0's sit just above +-1/128, +-3/128 and +-3/64 .. +-3/4, one to
// a bucket).
struct CodeEntry {
  float inside;
  uint32_t count;
};
constexpr int kCodeBuckets = 129;

__device__ __forceinline__ void fill_code_table(CodeEntry *tab, const float (&t)[15], int tid) {
  if (tid < kCodeBuckets) {
    const float lo = (float)(tid - 64) * (1.f / 64.f), hi = lo + 1.f / 64.f;  // exact
    uint32_t count = 0;
    float inside = __builtin_inff();
#pragma unroll
    for (int j = 0; j < 15; ++j) {
      count += t[j] <= lo ? 1u : 0u;
      if (t[j] > lo && t[j] < hi) inside = t[j];
    }
    tab[tid] = CodeEntry{inside, count};
  }
}

__device__ __forceinline__ uint32_t code_of(float x, const CodeEntry *tab) {
  const int b = min(max((int)floorf(x * 64.f) + 64, 0), kCodeBuckets - 1);  // the clamp only guards the read
  const CodeEntry e = tab[b];
  return e.count + (x >= e.inside ? 1u : 0u);
}

// x = RN(w / m) for |w| <= m.  For 2^-60 <= m <= 2^60 with y = RN(1 / m):
// q0 = RN(w y), the remainder w - q0 m is exact as one FMA, and
// RN(q0 + r y) is the correctly rounded quotient (Markstein's correction
// step for round-to-nearest); quotients that would be subnormal may differ
// by an ulp there, which no code decision sees (every threshold is more than
// 2^-8 from zero).  Other m: the IEEE division.
__device__ __forceinline__ float quotient(float w, float m, float y, bool fast) {
  if (fast) {
    const float q0 = __fmul_rn(w, y);
    const float r = __fmaf_rn(-q0, m, w);
    return __fmaf_rn(r, y, q0);
  }
  return m > 0.f ? __fdiv_rn(w, m) : 0.f;  // an all-zero block normalizes to 0
}

// Eight consecutive weights per lane, eight lanes per 64-weight block, so a
// wave covers 8 blocks (2 KiB) per step and a workgroup of 4 waves covers one
// group of 256 blocks in 8 steps.
__global__ __launch_bounds__(256) void k_quantize_blocks(const float *__restrict__ W, int64_t nb,
                                                         Thresholds T, uint8_t *__restrict__ packed,
                                                         float *__restrict__ absmax_out,
                                                         double *__restrict__ group_sum) {
  __shared__ float s_absmax[kGroup];
  __shared__ CodeEntry s_code[kCodeBuckets];
  float t[15];  // the thresholds in (scalar) registers
#pragma unroll
  for (int j = 0; j < 15; ++j) t[j] = T.t[j];
  fill_code_table(s_code, t, threadIdx.x);
  __syncthreads();
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
      const bool fast = m >= 0x1p-60f && m <= 0x1p60f;
      const float y = fast ? __fdiv_rn(1.f, m) : 0.f;
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= code_of(quotient(w[i], m, y, fast), s_code) << (4 * i);
      *reinterpret_cast<uint32_t *>(packed + e0 / 2) = word;
      if ((lane & 7) == 0) {
        absmax_out[first + lb] = m;
        s_absmax[lb] = m;
      }
    }
  }
  __syncthreads();
  // The group's float64 sum in block order.  Every absmax is a multiple of
  // 2^lo (the smallest ulp among them) and every partial sum is below
  // 2^(hi + 9) (256 values under 2^(hi+1)); when that span fits float64's 53
  // bits no addition rounds, so a tree over the waves gives the in-order
  // fold's bits exactly.  Otherwise one lane folds in block order.
  const float v = threadIdx.x < nblk ? s_absmax[threadIdx.x] : 0.f;
  const int ex = (int)((__float_as_uint(v) >> 23) & 0xFFu);
  int hi = v > 0.f ? (ex ? ex - 127 : -126) : -1000;  // v < 2^(hi+1)
  int lo = v > 0.f ? (ex ? ex - 150 : -149) : 1000;   // v is a multiple of 2^lo
  double sum = (double)v;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    hi = max(hi, __shfl_xor(hi, o, 64));
    lo = min(lo, __shfl_xor(lo, o, 64));
    sum += __shfl_xor(sum, o, 64);
  }
  __shared__ double s_wsum[4];
  __shared__ int s_span[4][2];
  if (lane == 0) {
    s_wsum[wave] = sum;
    s_span[wave][0] = hi;
    s_span[wave][1] = lo;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int ghi = max(max(s_span[0][0], s_span[1][0]), max(s_span[2][0], s_span[3][0]));
    const int glo = min(min(s_span[0][1], s_span[1][1]), min(s_span[2][1], s_span[3][1]));
    double acc = 0.0;
    if (ghi + 9 - glo <= 53) {
      acc = ((s_wsum[0] + s_wsum[1]) + s_wsum[2]) + s_wsum[3];
    } else {  // block order; eight LDS reads in flight per batch
      int i = 0;
      for (; i + 8 <= nblk; i += 8) {
        float u[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) u[q] = s_absmax[i + q];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc += (double)u[q];
      }
      for (; i < nblk; ++i) acc += (double)s_absmax[i];
    }
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
// The fold by the workgroup's kMeanLanes lanes; every lane gets the total.
__device__ __forceinline__ double mean_fold(const double *__restrict__ group_sum, int64_t ng, double *s_sum,
                                            double *s_run) {
  constexpr int B = 16;  // LDS reads ahead of the adds
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
  if (threadIdx.x == 0) s_run[0] = total;
  __syncthreads();
  return s_run[0];
}

__global__ __launch_bounds__(kMeanLanes) void k_mean(const double *__restrict__ group_sum, int64_t ng, int64_t nb,
                                                     float *__restrict__ offset) {
  __shared__ double s_sum[kMeanRuns * kMeanLd];
  __shared__ double s_run[kMeanRuns];
  const double total = mean_fold(group_sum, ng, s_sum, s_run);
  if (threadIdx.x == 0) *offset = (float)(total / (double)nb);
}

// Group g's 8-bit constants, by one wave: four block constants per lane.
__device__ __forceinline__ void encode_group(const float *__restrict__ absmax, int64_t nb, int64_t g, float offset,
                                             int lane, uint8_t *__restrict__ scale_code,
                                             float *__restrict__ group_amax) {
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

// One wave per group.
__global__ __launch_bounds__(256) void k_encode_scales(const float *__restrict__ absmax, int64_t nb,
                                                       int64_t ng, const float *__restrict__ offset_p,
                                                       uint8_t *__restrict__ scale_code,
                                                       float *__restrict__ group_amax) {
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= ng) return;
  encode_group(absmax, nb, g, *offset_p, (int)threadIdx.x & 63, scale_code, group_amax);
}

// Both in one launch when the group sums fit one staging pass (ng <=
// kMeanRuns * kMeanRun): every workgroup folds the mean itself, in the same
// order (so all hold the same offset, and workgroup 0 stores it), then its
// 16 waves encode groups blockIdx.x * 16 + wave, strided by the grid.
constexpr int64_t kFusedMeanMaxGroups = (int64_t)kMeanRuns * kMeanRun;
__global__ __launch_bounds__(kMeanLanes) void k_mean_encode(const double *__restrict__ group_sum,
                                                            const float *__restrict__ absmax, int64_t nb,
                                                            int64_t ng, float *__restrict__ offset_out,
                                                            uint8_t *__restrict__ scale_code,
                                                            float *__restrict__ group_amax) {
  __shared__ double s_sum[kMeanRuns * kMeanLd];
  __shared__ double s_run[kMeanRuns];
  const double total = mean_fold(group_sum, ng, s_sum, s_run);
  const float offset = (float)(total / (double)nb);
  if (blockIdx.x == 0 && threadIdx.x == 0) *offset_out = offset;
  const int wave = (int)threadIdx.x >> 6;
  for (int64_t g = (int64_t)blockIdx.x * (kMeanLanes / 64) + wave; g < ng; g += (int64_t)gridDim.x * (kMeanLanes / 64))
    encode_group(absmax, nb, g, offset, (int)threadIdx.x & 63, scale_code, group_amax);
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
  if (ng <= kFusedMeanMaxGroups) {  // one staging pass: mean and encoding in one launch
    const int64_t grid = std::min<int64_t>(256, ceil_div(ng, (int64_t)(kMeanLanes / 64)));
    QLORA_LAUNCH("k_mean_encode", k_mean_encode, dim3((unsigned)grid), dim3(kMeanLanes), 0, s, ws_group_sum,
                 ws_absmax, nb, ng, offset, scale_code, group_amax);
    return hipGetLastError();
  }
  QLORA_LAUNCH("k_mean", k_mean, dim3(1), dim3(kMeanLanes), 0, s, ws_group_sum, ng, nb, offset);
  QLORA_LAUNCH("k_encode_scales", k_encode_scales, dim3((unsigned)ceil_div(ng, 4)), dim3(256), 0, s, ws_absmax, nb, ng,
                     offset, scale_code, group_amax);
  return hipGetLastError();
}

}  // namespace qlora

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
// Each thread owns a register tile of kMergeRows weight rows x one packed
// dword (8 columns): per rank index j it widens its 8 values of A[j] to
// float64 once for all its rows and each row's B value once for all 8
// columns, then does the rows x 8 multiply-adds of that j.  The sum over j
// is the definition's, in the same order for every element; only the
// conversions are shared.  Consecutive threads take consecutive dwords of
// the same rows, so the A, code and output accesses are contiguous and the
// B reads of a wave are one address.  Then each row's dword of BF16
// weights through the same dequant_word as every other consumer.  A
// deployment-time pass: r float64 multiply-adds per weight.
#include "lora_gemm.h"

namespace qlora {
namespace {

constexpr int kMergeRows = 4;

__device__ __forceinline__ double bf16_lo(uint32_t v) { return (double)__uint_as_float(v << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t v) { return (double)__uint_as_float(v & 0xFFFF0000u); }

// t[i][e] += B[n0 + i][j] * A[j][k0 + e] for one rank index j, every
// operation separately rounded (the products of two bf16 are exact).
__device__ __forceinline__ void merge_rank_step(double (&t)[kMergeRows][8], const double (&bj)[kMergeRows],
                                                const u32x4_t &a) {
  double aj[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    aj[2 * e] = bf16_lo(a[e]);
    aj[2 * e + 1] = bf16_hi(a[e]);
  }
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) t[i][e] = __dadd_rn(t[i][e], __dmul_rn(bj[i], aj[e]));
}

// kVecB: r % 8 == 0, so each row's B values are read 8 at a time.
template <bool kVecB>
__global__ __launch_bounds__(256) void k_merge(Nf4View w, const uint16_t *__restrict__ A,
                                               const uint16_t *__restrict__ B, int r, float s,
                                               float *__restrict__ Wm, uint16_t *__restrict__ Wb) {
  __shared__ float2 s_pair[256];
  fill_pair_table(s_pair, threadIdx.x, 256, w.codebook);
  __syncthreads();
  const int64_t kd = w.k / 8;  // packed dwords per row
  const int64_t th = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rb = th / kd, cd = th - rb * kd;
  const int64_t n0 = rb * kMergeRows, k0 = 8 * cd;
  if (n0 >= w.n) return;
  const int nr = (int)min<int64_t>(kMergeRows, w.n - n0);
  // rows past n repeat the last real row (their sums are not stored)
  const uint16_t *brow[kMergeRows];
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i) brow[i] = B + (n0 + min(i, nr - 1)) * r;
  const uint16_t *acol = A + k0;  // k0 % 8 == 0: 16-byte pieces of A's rows
  double t[kMergeRows][8];
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) t[i][e] = 0.0;
  if constexpr (kVecB) {
    for (int j0 = 0; j0 < r; j0 += 8) {
      u32x4_t bq[kMergeRows];
#pragma unroll
      for (int i = 0; i < kMergeRows; ++i) bq[i] = *reinterpret_cast<const u32x4_t *>(brow[i] + j0);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t *>(acol + (int64_t)(j0 + jj) * w.k);
        double bj[kMergeRows];
#pragma unroll
        for (int i = 0; i < kMergeRows; ++i) bj[i] = jj & 1 ? bf16_hi(bq[i][jj >> 1]) : bf16_lo(bq[i][jj >> 1]);
        merge_rank_step(t, bj, a);
      }
    }
  } else {
    for (int j = 0; j < r; ++j) {
      const u32x4_t a = *reinterpret_cast<const u32x4_t *>(acol + (int64_t)j * w.k);
      double bj[kMergeRows];
#pragma unroll
      for (int i = 0; i < kMergeRows; ++i) bj[i] = bf16_lo(brow[i][j]);
      merge_rank_step(t, bj, a);
    }
  }
  const double sd = (double)s;
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i) {
    if (i >= nr) break;
    const int64_t e0 = (n0 + i) * w.k + k0;
    const int64_t b = e0 / kBlock;
    const float sb = w.absmax ? w.absmax[b] : block_scale(w.scale_code[b], w.group_amax[b / kGroup], *w.offset);
    uint32_t wb[4];
    dequant_word(reinterpret_cast<const uint32_t *>(w.packed)[e0 / 8], sb, s_pair, wb);
    float out[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double wh = e & 1 ? bf16_hi(wb[e >> 1]) : bf16_lo(wb[e >> 1]);
      out[e] = __double2float_rn(__dadd_rn(wh, __dmul_rn(sd, t[i][e])));
    }
    f32x4_t *dst = reinterpret_cast<f32x4_t *>(Wm + e0);
    dst[0] = f32x4_t{out[0], out[1], out[2], out[3]};
    dst[1] = f32x4_t{out[4], out[5], out[6], out[7]};
    if (Wb)
      *reinterpret_cast<u32x4_t *>(Wb + e0) = u32x4_t{bf16x2_rne(out[0], out[1]), bf16x2_rne(out[2], out[3]),
                                                       bf16x2_rne(out[4], out[5]), bf16x2_rne(out[6], out[7])};
  }
}

}  // namespace

hipError_t launch_merge(const Nf4View &w, const uint16_t *A, const uint16_t *B, int r, float s, float *Wm,
                        uint16_t *Wb, hipStream_t st) {
  const int64_t threads = ceil_div(w.n, (int64_t)kMergeRows) * (w.k / 8);
  const dim3 grid((unsigned)ceil_div(threads, 256));
  if (r % 8 == 0)
    QLORA_LAUNCH("k_merge", k_merge<true>, grid, dim3(256), 0, st, w, A, B, r, s, Wm, Wb);
  else
    QLORA_LAUNCH("k_merge", k_merge<false>, grid, dim3(256), 0, st, w, A, B, r, s, Wm, Wb);
  return hipGetLastError();
}

}  // namespace qlora

// lora_gemm.h -- skinny LoRA products and small layout kernels (lora_gemm.hip),
// plus the guarded 8-element loader shared by the tiled kernels.
#pragma once

#include <algorithm>
#include <type_traits>

#include "qlora_internal.h"

namespace qlora {

__device__ __forceinline__ int64_t ceil_div_d(int64_t a, int64_t b) { return (a + b - 1) / b; }

// 8 consecutive bf16 of a row-major matrix (row stride ld) at (row, col..col+7);
// elements outside [0, nrows) x [0, ncols) read as zero.  vec_ok: ld % 8 == 0
// (then an in-range chunk is one 16-byte load).
__device__ __forceinline__ u32x4_t load8(const uint16_t *m, int64_t ld, int64_t nrows, int64_t ncols, int64_t row,
                                         int64_t col, bool vec_ok) {
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (row < nrows && col < ncols) {
    const uint16_t *p = m + row * ld + col;
    if (vec_ok && col + 8 <= ncols) {
      v = *reinterpret_cast<const u32x4_t *>(p);
    } else {
      uint32_t e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = (col + i < ncols) ? p[i] : 0u;
      v = u32x4_t{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
    }
  }
  return v;
}

// A [rows][64] bf16 tile in LDS, 128 B per row; 16-byte chunk c of row r
// lives at chunk c ^ (r & 7), so the 16 rows one MFMA fragment read touches,
// and the 8 chunks of a row, fall in different banks.
__device__ __forceinline__ int xsw(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous run of tiles so tiles that share an operand panel meet in the
// same L2.  A bijection on [0, nblocks).
__device__ __forceinline__ int xcd_tile(int bid, int nblocks) {
  const int q = nblocks >> 3, rem = nblocks & 7, x = bid & 7, p = bid >> 3;
  return (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + p;
}

// Raw buffer resource over [base, base + bytes): loads past the end read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

struct SplitPlan {
  int splits = 1;
  int steps_per_split = 1;
};

int lora_rank_pad(int r);  // r rounded up to a multiple of 32
SplitPlan plan_split(int64_t tiles, int64_t steps);

hipError_t launch_nt_splitk(const uint16_t *P, int64_t rowsP, const uint16_t *Q, int rowsQ, int RP, int64_t lenC,
                            int64_t ld, const SplitPlan &sp, float *part, hipStream_t s);
// The same partials with Q given as its transpose Qr [lenC][r] (row stride
// r): Q[j][c] = Qr[c][j] for j < r, zero for r <= j < RP.  Needs
// nt_rows_supported (r % 8 == 0, r <= 64, ld % 8 == 0).
bool nt_rows_supported(int r, int64_t ld);
hipError_t launch_nt_rows(const uint16_t *P, int64_t rowsP, const uint16_t *Qr, int r, int RP, int64_t lenC,
                          int64_t ld, const SplitPlan &sp, float *part, hipStream_t s);
// rows_out: partials as [S][D][RP] (reduced with rows_out into [D][r]);
// otherwise [S][RP][D].
hipError_t launch_tn_splitk(const uint16_t *P, int64_t M, int64_t D, const uint16_t *Qt, int64_t ldq, int RP,
                            const SplitPlan &sp, bool rows_out, float *part, hipStream_t s);
hipError_t launch_reduce_rows(const float *part, int S, int64_t R, int RP, int r, float scale, float *out_f32,
                              uint16_t *out_b, uint16_t *out_bt, int64_t ldt, hipStream_t s);
hipError_t launch_reduce_cols(const float *part, int S, int64_t D, int RP, int r, bool rows_out, uint16_t *out,
                              hipStream_t s);
hipError_t launch_fill_zero_u16(uint16_t *p, int64_t n, hipStream_t s);

// Both transposed products of the backward in one launch (consecutive block
// ranges): problem q computes partials of Qt_q^T-weighted sums of P_q over M,
// exactly as launch_tn_splitk does for it alone.  Falls back to two launches
// when a problem cannot take the DMA kernel.
struct TnProblem {
  const uint16_t *P;  // [M][D]
  int64_t D;
  const uint16_t *Qt;  // [RP][ldq]
  int64_t ldq;
  SplitPlan sp;
  bool rows_out;
  float *part;
};
hipError_t launch_tn_pair(const TnProblem &p0, const TnProblem &p1, int64_t M, int RP, hipStream_t s);

// ---------------------------------------------------------------------------
// Small elementwise jobs (jobs.hip): layout copies, split-partial reductions
// and the tile kernels' block-scale tables.  Up to kMaxJobs independent jobs
// run as one launch over consecutive block ranges, which saves a launch ramp
// per job.  The reductions are those of the launch_reduce_* functions above.
// ---------------------------------------------------------------------------
enum JobKind : int {
  kJobTranspose,    // 64 x 64 tiles through LDS
  kJobReduceRows,   // elementwise
  kJobReduceCols,
  kJobScalesFwd,
  kJobScalesBwd,
  kJobSplitReduce,  // a split tile launch's partials, summed in split order (nf4_tile.h)
};
struct SmallJob {
  int kind = 0;
  int64_t count = 0;  // elements (one thread each)
  const void *in = nullptr;
  void *out = nullptr, *out2 = nullptr, *out3 = nullptr;
  int64_t a = 0, b = 0, c = 0, d = 0;
  int i = 0, j = 0;
  float f = 0.f;
  Nf4View w{};
};
constexpr int kMaxJobs = 4;
hipError_t launch_jobs(const char *name, const SmallJob *jobs, int n, hipStream_t s);
// out [out_rows][ldo] = in^T for a row-major bf16 in [rows][cols], zero-padded
SmallJob job_transpose_pad(const uint16_t *in, int64_t rows, int64_t cols, uint16_t *out, int64_t out_rows,
                           int64_t ldo);
// out [RP][ldo] = bf16(scale * H^T) for fp32 H [M][r], zero-padded
SmallJob job_scale_transpose(const float *H, int64_t M, int r, float scale, uint16_t *out, int RP, int64_t ldo);
SmallJob job_reduce_rows(const float *part, int S, int64_t R, int RP, int r, float scale, float *out_f32,
                         uint16_t *out_b, uint16_t *out_bt, int64_t ldt);
SmallJob job_reduce_cols(const float *part, int S, int64_t D, int RP, int r, bool rows_out, uint16_t *out);

}  // namespace qlora

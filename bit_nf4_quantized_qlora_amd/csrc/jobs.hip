// jobs.hip -- small elementwise jobs of the linear layer, several per launch.
//
// The layout copies the LoRA products need (B^T and A^T rank-padded,
// bf16(s H)^T), the fixed-order reductions of split partials, and the tile
// kernels' block-scale tables are each a few MB at most, so one launch per
// job is mostly launch ramp.  k_small_jobs takes up to kMaxJobs independent
// jobs and runs them on consecutive block ranges of one grid.
#include "nf4_tile.h"

namespace qlora {
namespace {

struct SmallJobs {
  SmallJob j[kMaxJobs];
  int64_t start[kMaxJobs + 1];  // first block of each job
  int n;
};

// out [out_rows][ldo] = in^T for a row-major in [rows][cols] (bf16), zero outside.
__device__ __forceinline__ void run_transpose_pad(const SmallJob &j, int64_t idx) {
  const uint16_t *in = static_cast<const uint16_t *>(j.in);
  const int64_t rows = j.a, cols = j.b, ldo = j.d;
  const int64_t c = idx / ldo, rr = idx - c * ldo;  // out[c][rr] = in[rr][c]
  static_cast<uint16_t *>(j.out)[idx] = (c < cols && rr < rows) ? in[rr * cols + c] : (uint16_t)0;
}

// out [RP][ldo] = bf16(scale * H^T) for H [M][r] fp32, zero outside.
__device__ __forceinline__ void run_scale_transpose(const SmallJob &j, int64_t idx) {
  const float *H = static_cast<const float *>(j.in);
  const int64_t M = j.a, ldo = j.d;
  const int r = j.i;
  const int64_t jj = idx / ldo, m = idx - jj * ldo;
  static_cast<uint16_t *>(j.out)[idx] = (jj < r && m < M) ? f32_to_bf16_bits(j.f * H[m * r + jj]) : (uint16_t)0;
}

// Rows form: part [S][R][RP] -> v = sum_s part[s][i][jj] (s in order):
//   out  (fp32) [R][r]    = v              (jj < r)
//   out2 (bf16) [R][RP]   = bf16(scale*v)  (all jj; columns >= r are zero)
//   out3 (bf16) [RP][ldt] = bf16(scale*v) transposed; columns i >= R zero
__device__ __forceinline__ void run_reduce_rows(const SmallJob &j, int64_t idx) {
  const float *part = static_cast<const float *>(j.in);
  const int64_t R = j.a, ldt = j.d;
  const int S = j.i, RP = (int)j.b, r = j.j;
  const int64_t i = idx / RP;
  const int jj = (int)(idx - i * RP);
  float v = 0.f;
  if (i < R) {
    for (int s = 0; s < S; ++s) v += part[(size_t)s * R * RP + idx];
    if (j.out && jj < r) static_cast<float *>(j.out)[i * r + jj] = v;
    if (j.out2) static_cast<uint16_t *>(j.out2)[idx] = f32_to_bf16_bits(j.f * v);
  }
  if (j.out3) static_cast<uint16_t *>(j.out3)[(int64_t)jj * ldt + i] = i < R ? f32_to_bf16_bits(j.f * v) : (uint16_t)0;
}

// Transposed-product partials -> bf16, summed over splits in order:
//   c == 0: part [S][RP][D] -> out [r][D]  (dA)
//   c == 1: part [S][D][RP] -> out [D][r]  (dB)
__device__ __forceinline__ void run_reduce_cols(const SmallJob &j, int64_t idx) {
  const float *part = static_cast<const float *>(j.in);
  const int64_t D = j.a;
  const int S = j.i, RP = (int)j.b, r = j.j;
  const int64_t src = j.c ? (idx / r) * RP + idx % r : idx;
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[(size_t)s * RP * D + src];
  static_cast<uint16_t *>(j.out)[idx] = f32_to_bf16_bits(v);
}

// Forward scale table: for weight tile to (rows 256to ..) and super-step sp
// (blocks 4sp .. 4sp+3 of each row) one contiguous 4 KB run,
// Sp[((to*nsup + sp)*256 + row)*4 + q]; rows past n and blocks past k/64 hold
// 0.  block_scale is the dequantization's own (bit-identical).
__device__ __forceinline__ void run_scales_fwd(const SmallJob &j, int64_t t) {
  const Nf4View &w = j.w;
  const int64_t nsup = j.a;
  const int64_t q = t >> 8, to = q / nsup, sp = q - to * nsup;
  const int64_t n = to * kTileRows + (t & 255), nkb = w.k / kBlock;
  f32x4_t v = {0.f, 0.f, 0.f, 0.f};
  if (n < w.n) {
    const float off = *w.offset;
#pragma unroll
    for (int u = 0; u < kTileSup; ++u) {
      const int64_t kb = kTileSup * sp + u, b = n * nkb + kb;
      if (kb < nkb) v[u] = block_scale(w.scale_code[b], w.group_amax[b / kGroup], off);
    }
  }
  *reinterpret_cast<f32x4_t *>(static_cast<float *>(j.out) + 4 * t) = v;
}

// Backward scale table: for column tile tk (k-blocks 4tk .. 4tk+3) and
// super-step sp (weight rows 256sp .. 256sp+255) one contiguous 4 KB run,
// Sp[((tk*nsup + sp)*4 + blk)*256 + row]; rows past n and blocks past k/64
// hold 0.
__device__ __forceinline__ void run_scales_bwd(const SmallJob &j, int64_t t) {
  const Nf4View &w = j.w;
  const int64_t nsup = j.a;
  const int64_t q = t >> 10, tk = q / nsup, sp = q - tk * nsup;
  const int64_t n = sp * kTileRows + (t & 255), kb = tk * kTileSup + ((t >> 8) & 3), nkb = w.k / kBlock;
  float v = 0.f;
  if (n < w.n && kb < nkb) {
    const int64_t b = n * nkb + kb;
    v = block_scale(w.scale_code[b], w.group_amax[b / kGroup], *w.offset);
  }
  static_cast<float *>(j.out)[t] = v;
}

__global__ __launch_bounds__(256) void k_small_jobs(SmallJobs js) {
  const int64_t blk = blockIdx.x;
  int q = 0;
  while (q + 1 < js.n && blk >= js.start[q + 1]) ++q;
  const SmallJob &j = js.j[q];
  const int64_t idx = (blk - js.start[q]) * 256 + threadIdx.x;
  if (idx >= j.count) return;
  switch (j.kind) {
    case kJobTransposePad: run_transpose_pad(j, idx); break;
    case kJobScaleTranspose: run_scale_transpose(j, idx); break;
    case kJobReduceRows: run_reduce_rows(j, idx); break;
    case kJobReduceCols: run_reduce_cols(j, idx); break;
    case kJobScalesFwd: run_scales_fwd(j, idx); break;
    case kJobScalesBwd: run_scales_bwd(j, idx); break;
    default: break;
  }
}

}  // namespace

hipError_t launch_jobs(const char *name, const SmallJob *jobs, int n, hipStream_t s) {
  if (n < 1 || n > kMaxJobs) return hipErrorInvalidValue;
  SmallJobs js{};
  js.n = 0;
  int64_t blocks = 0;
  for (int q = 0; q < n; ++q) {
    if (jobs[q].count <= 0) continue;
    js.j[js.n] = jobs[q];
    js.start[js.n] = blocks;
    blocks += ceil_div(jobs[q].count, 256);
    ++js.n;
  }
  if (js.n == 0) return hipSuccess;
  js.start[js.n] = blocks;
  QLORA_LAUNCH(name, k_small_jobs, dim3((unsigned)blocks), dim3(256), 0, s, js);
  return hipGetLastError();
}

SmallJob job_transpose_pad(const uint16_t *in, int64_t rows, int64_t cols, uint16_t *out, int64_t out_rows,
                           int64_t ldo) {
  SmallJob j;
  j.kind = kJobTransposePad;
  j.count = out_rows * ldo;
  j.in = in;
  j.out = out;
  j.a = rows;
  j.b = cols;
  j.d = ldo;
  return j;
}

SmallJob job_scale_transpose(const float *H, int64_t M, int r, float scale, uint16_t *out, int RP, int64_t ldo) {
  SmallJob j;
  j.kind = kJobScaleTranspose;
  j.count = (int64_t)RP * ldo;
  j.in = H;
  j.out = out;
  j.a = M;
  j.d = ldo;
  j.i = r;
  j.f = scale;
  return j;
}

SmallJob job_reduce_rows(const float *part, int S, int64_t R, int RP, int r, float scale, float *out_f32,
                         uint16_t *out_b, uint16_t *out_bt, int64_t ldt) {
  SmallJob j;
  j.kind = kJobReduceRows;
  j.count = (out_bt ? ldt : R) * RP;
  j.in = part;
  j.out = out_f32;
  j.out2 = out_b;
  j.out3 = out_bt;
  j.a = R;
  j.b = RP;
  j.d = ldt;
  j.i = S;
  j.j = r;
  j.f = scale;
  return j;
}

SmallJob job_reduce_cols(const float *part, int S, int64_t D, int RP, int r, bool rows_out, uint16_t *out) {
  SmallJob j;
  j.kind = kJobReduceCols;
  j.count = (int64_t)r * D;
  j.in = part;
  j.out = out;
  j.a = D;
  j.b = RP;
  j.c = rows_out ? 1 : 0;
  j.i = S;
  j.j = r;
  return j;
}

SmallJob job_scales_fwd(const Nf4View &w, float *scales) {
  SmallJob j;
  j.kind = kJobScalesFwd;
  j.a = tile_fwd_nsup(w.k);
  j.count = ceil_div(w.n, kTileRows) * j.a * 256;
  j.out = scales;
  j.w = w;
  return j;
}

SmallJob job_scales_bwd(const Nf4View &w, float *scales) {
  SmallJob j;
  j.kind = kJobScalesBwd;
  j.a = tile_bwd_nsup(w.n);
  j.count = ceil_div(w.k, kTileRows) * j.a * 1024;
  j.out = scales;
  j.w = w;
  return j;
}

}  // namespace qlora

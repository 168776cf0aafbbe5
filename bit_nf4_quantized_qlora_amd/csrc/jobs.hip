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

// Index arithmetic is 32-bit (every job's element count is below 2^31, which
// launch_jobs checks): a 64-bit division per element costs more than the
// element's memory traffic.

// Tiled transpose, one 256-thread block per 64 x 64 tile of the output:
// out[c][rr] = conv(in[rr][c]) for rr < rows, c < cols, zero elsewhere in
// out [out_rows][ldo]; conv copies bf16, or rounds scale * x for fp32 input
// (j.i == 1).  Each wave instruction reads 64 consecutive elements of one
// input row and writes 64 consecutive elements of one output row; the tile
// turns in LDS (row stride 65, so the column reads hit distinct banks).
__device__ __forceinline__ void run_transpose(const SmallJob &j, uint32_t idx, uint16_t (*t)[65]) {
  const uint32_t tile = idx >> 8, tid = idx & 255;
  const uint32_t rows = (uint32_t)j.a, cols = (uint32_t)j.b, out_rows = (uint32_t)j.c, ldo = (uint32_t)j.d;
  const uint32_t tiles_rr = (ldo + 63) / 64;
  const uint32_t tc = tile / tiles_rr, tr = tile - tc * tiles_rr;
  const uint32_t c0 = tc * 64, rr0 = tr * 64;
  const uint32_t col = tid & 63, c = c0 + col;
  // all 16 loads go out before any is used (out-of-range elements load
  // element 0 and are replaced by zero), so the tile waits for memory once
  uint32_t v[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t rr = rr0 + (tid >> 6) + 4 * e;
    const bool ok = rr < rows && c < cols;
    const uint32_t src = ok ? rr * cols + c : 0u;
    v[e] = j.i ? __float_as_uint(static_cast<const float *>(j.in)[src]) : static_cast<const uint16_t *>(j.in)[src];
    v[e] = ok ? v[e] : 0u;
  }
#pragma unroll
  for (int e = 0; e < 16; ++e)
    t[(tid >> 6) + 4 * e][col] = j.i ? f32_to_bf16_bits(j.f * __uint_as_float(v[e])) : (uint16_t)v[e];
  __syncthreads();
  uint16_t *out = static_cast<uint16_t *>(j.out);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t oc = (tid >> 6) + 4 * e;
    const uint32_t cc = c0 + oc, rr = rr0 + col;
    if (cc < out_rows && rr < ldo) out[cc * ldo + rr] = t[col][oc];
  }
}

// Sum over s < S of part[s * stride + src], in order of s: the first kSumBatch
// loads are issued together, so the sum waits for memory once.
constexpr int kSumBatch = 8;
__device__ __forceinline__ float sum_splits(const float *part, int S, size_t stride, size_t src) {
  float v[kSumBatch];
#pragma unroll
  for (int s = 0; s < kSumBatch; ++s) v[s] = s < S ? part[s * stride + src] : 0.f;
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < kSumBatch; ++s) acc += v[s];
  for (int s = kSumBatch; s < S; ++s) acc += part[s * stride + src];
  return acc;
}

// Rows form: part [S][R][RP] -> v = sum_s part[s][i][jj] (s in order):
//   out  (fp32) [R][r]    = v              (jj < r)
//   out2 (bf16) [R][RP]   = bf16(scale*v)  (all jj; columns >= r are zero)
//   out3 (bf16) [RP][ldt] = bf16(scale*v) transposed; columns i >= R zero
__device__ __forceinline__ void run_reduce_rows(const SmallJob &j, uint32_t idx) {
  const float *part = static_cast<const float *>(j.in);
  const int64_t R = j.a, ldt = j.d;
  const int S = j.i, r = j.j;
  const uint32_t RP = (uint32_t)j.b;
  const uint32_t i = idx / RP;
  const int jj = (int)(idx - i * RP);
  float v = 0.f;
  if (i < R) {
    v = sum_splits(part, S, (size_t)R * RP, idx);
    if (j.out && jj < r) static_cast<float *>(j.out)[(int64_t)i * r + jj] = v;
    if (j.out2) static_cast<uint16_t *>(j.out2)[idx] = f32_to_bf16_bits(j.f * v);
  }
  if (j.out3) static_cast<uint16_t *>(j.out3)[(int64_t)jj * ldt + i] = i < R ? f32_to_bf16_bits(j.f * v) : (uint16_t)0;
}

// Transposed-product partials -> bf16, summed over splits in order:
//   c == 0: part [S][RP][D] -> out [r][D]  (dA)
//   c == 1: part [S][D][RP] -> out [D][r]  (dB)
__device__ __forceinline__ void run_reduce_cols(const SmallJob &j, uint32_t idx) {
  const float *part = static_cast<const float *>(j.in);
  const int64_t D = j.a;
  const int S = j.i;
  const uint32_t RP = (uint32_t)j.b, r = (uint32_t)j.j;
  const uint32_t q = idx / r;
  const size_t src = j.c ? (size_t)q * RP + (idx - q * r) : idx;
  static_cast<uint16_t *>(j.out)[idx] = f32_to_bf16_bits(sum_splits(part, S, (size_t)RP * D, src));
}

// The four block scales of row n, blocks 4 kq .. 4 kq + 3 (0 past k/64 or n):
// with double-quantized constants and k/64 % 4 == 0 the four scale codes are
// one aligned 32-bit word and share one group constant (groups are 256
// blocks, so an aligned run of four never straddles two); otherwise one load
// per block.  Every load is issued before any use.  block_scale is the
// dequantization's own (bit-identical).
__device__ __forceinline__ void row_quad_scales(const Nf4View &w, int64_t n, int64_t kq, float (&v)[kTileSup]) {
  const int64_t nkb = w.k / kBlock;
#pragma unroll
  for (int u = 0; u < kTileSup; ++u) v[u] = 0.f;
  if (n >= w.n) return;
  const int64_t b0 = n * nkb + kTileSup * kq;
  if (!w.absmax && nkb % kTileSup == 0) {
    if (kTileSup * kq >= nkb) return;
    const uint32_t word = *reinterpret_cast<const uint32_t *>(w.scale_code + b0);
    const float ga = w.group_amax[b0 / kGroup], off = *w.offset;
#pragma unroll
    for (int u = 0; u < kTileSup; ++u) v[u] = block_scale((word >> (8 * u)) & 0xFFu, ga, off);
    return;
  }
  const float off = w.absmax ? 0.f : *w.offset;
  uint32_t c8[kTileSup];
  float ga[kTileSup];
#pragma unroll
  for (int u = 0; u < kTileSup; ++u) {
    const int64_t kb = kTileSup * kq + u, b = kb < nkb ? n * nkb + kb : 0;  // past k/64: block 0, then 0
    if (w.absmax) {
      c8[u] = __float_as_uint(w.absmax[b]);
      ga[u] = 0.f;
    } else {
      c8[u] = w.scale_code[b];
      ga[u] = w.group_amax[b / kGroup];
    }
  }
#pragma unroll
  for (int u = 0; u < kTileSup; ++u)
    if (kTileSup * kq + u < nkb) v[u] = w.absmax ? __uint_as_float(c8[u]) : block_scale(c8[u], ga[u], off);
}

// Forward scale table: for weight tile to (rows 256to ..) and super-step sp
// (blocks 4sp .. 4sp+3 of each row) one contiguous 4 KB run,
// Sp[((to*nsup + sp)*256 + row)*4 + q]; rows past n and blocks past k/64 hold
// 0.
__device__ __forceinline__ void run_scales_fwd(const SmallJob &j, uint32_t t) {
  const uint32_t nsup = (uint32_t)j.a;
  const uint32_t q = t >> 8, to = q / nsup, sp = q - to * nsup;
  float v[kTileSup];
  row_quad_scales(j.w, (int64_t)to * kTileRows + (t & 255), sp, v);
  *reinterpret_cast<f32x4_t *>(static_cast<float *>(j.out) + 4 * t) = f32x4_t{v[0], v[1], v[2], v[3]};
}

// Backward scale table: for column tile tk (k-blocks 4tk .. 4tk+3) and
// super-step sp (weight rows 256sp .. 256sp+255) one contiguous 4 KB run,
// Sp[((tk*nsup + sp)*4 + blk)*256 + row]; rows past n and blocks past k/64
// hold 0.  One thread per (tk, sp, row): the row's four scales, four
// coalesced stores.
__device__ __forceinline__ void run_scales_bwd(const SmallJob &j, uint32_t t) {
  const uint32_t nsup = (uint32_t)j.a;
  const uint32_t q = t >> 8, tk = q / nsup, sp = q - tk * nsup;
  float v[kTileSup];
  row_quad_scales(j.w, (int64_t)sp * kTileRows + (t & 255), tk, v);
  float *out = static_cast<float *>(j.out) + (size_t)q * 4 * 256 + (t & 255);
#pragma unroll
  for (int blk = 0; blk < kTileSup; ++blk) out[blk * 256] = v[blk];
}

__global__ __launch_bounds__(256) void k_small_jobs(SmallJobs js) {
  __shared__ uint16_t t[64][65];  // the tiled jobs' transpose buffer
  const int64_t blk = blockIdx.x;
  int q = 0;
  while (q + 1 < js.n && blk >= js.start[q + 1]) ++q;
  const SmallJob &j = js.j[q];
  const uint32_t idx = (uint32_t)(blk - js.start[q]) * 256u + threadIdx.x;
  if (idx >= j.count) return;
  switch (j.kind) {
    case kJobTranspose: run_transpose(j, idx, t); break;
    case kJobReduceRows: run_reduce_rows(j, idx); break;
    case kJobReduceCols: run_reduce_cols(j, idx); break;
    case kJobScalesFwd: run_scales_fwd(j, idx); break;
    case kJobScalesBwd: run_scales_bwd(j, idx); break;
    case kJobSplitReduce:
      split_reduce_slot(static_cast<const f32x4_t *>(j.in), j.i, (int)j.c, j.j, j.a, j.b,
                        static_cast<uint16_t *>(j.out), idx);
      break;
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
    if (jobs[q].count >= (int64_t(1) << 31) - 256) return hipErrorInvalidValue;  // 32-bit element indices
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

namespace {
int64_t tiles64(int64_t a, int64_t b) { return ((a + 63) / 64) * ((b + 63) / 64); }
}  // namespace

SmallJob job_transpose_pad(const uint16_t *in, int64_t rows, int64_t cols, uint16_t *out, int64_t out_rows,
                           int64_t ldo) {
  SmallJob j;
  j.kind = kJobTranspose;
  j.count = tiles64(out_rows, ldo) * 256;
  j.in = in;
  j.out = out;
  j.a = rows;
  j.b = cols;
  j.c = out_rows;
  j.d = ldo;
  return j;
}

SmallJob job_scale_transpose(const float *H, int64_t M, int r, float scale, uint16_t *out, int RP, int64_t ldo) {
  SmallJob j;
  j.kind = kJobTranspose;
  j.count = tiles64(RP, ldo) * 256;
  j.in = H;
  j.out = out;
  j.a = M;
  j.b = r;
  j.c = RP;
  j.d = ldo;
  j.i = 1;
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
  j.count = ceil_div(w.k, kTileRows) * j.a * 256;
  j.out = scales;
  j.w = w;
  return j;
}

}  // namespace qlora

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

// Sum over s < S of part[s * stride + src], in order of s.  The loads go out
// a batch at a time, all before any is used: up to 8 splits (the adapter
// gradients' products) in one short batch; the H and G products at M = 512
// split their contraction 16-29 ways, which take batches of 32, so the sum
// waits for memory once per batch rather than once per split.
template <int kBatch>
__device__ __forceinline__ float sum_batch(const float *part, int s0, int S, size_t stride, size_t src, float acc) {
  float v[kBatch];
#pragma unroll
  for (int s = 0; s < kBatch; ++s) v[s] = s0 + s < S ? part[(size_t)(s0 + s) * stride + src] : 0.f;
#pragma unroll
  for (int s = 0; s < kBatch; ++s) acc += v[s];  // the zeros past S leave acc unchanged (acc is never -0)
  return acc;
}
__device__ __forceinline__ float sum_splits(const float *part, int S, size_t stride, size_t src) {
  if (S <= 8) return sum_batch<8>(part, 0, S, stride, src, 0.f);
  float acc = 0.f;
  for (int s0 = 0; s0 < S; s0 += 32) acc = sum_batch<32>(part, s0, S, stride, src, acc);
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

// The scale tables are built one thread per (row, run of kRun consecutive
// quads of its blocks), so each thread reads kRun consecutive scale-code
// words of its row and the row's other quads -- the rest of the same 128-byte
// lines -- are read by the neighbouring workgroups, which k_small_jobs keeps
// on one XCD (one fetch of each line into that XCD's L2).  Thread t: row t %
// 256 of a 256-row tile, run (t / 256) % runs, tile (t / 256) / runs.
constexpr int kRun = 4;

// The block scales of row n, quads q0 .. q0 + kRun - 1 (blocks 4 q0 ..);
// zero past k/64 or n.  Bit for bit row_quad_scales, with every load of the
// run issued before any use.
__device__ __forceinline__ void row_run_scales(const Nf4View &w, int64_t n, int64_t q0,
                                               float (&v)[kRun][kTileSup]) {
  const int64_t nkb = w.k / kBlock;
  if (nkb % kTileSup != 0) {  // quads straddle rows: block by block
#pragma unroll
    for (int u = 0; u < kRun; ++u) row_quad_scales(w, n, q0 + u, v[u]);
    return;
  }
  const int64_t nq = nkb / kTileSup;
#pragma unroll
  for (int u = 0; u < kRun; ++u)
#pragma unroll
    for (int b = 0; b < kTileSup; ++b) v[u][b] = 0.f;
  if (n >= w.n) return;
  const int64_t b0 = n * nkb + kTileSup * q0;
  if (w.absmax) {  // single-level: the absmax values themselves, four per 16-byte load (the C ABI
                   // requires the buffer 16-byte aligned, and b0 is a multiple of 4)
    f32x4_t a[kRun];
#pragma unroll
    for (int u = 0; u < kRun; ++u)
      a[u] = q0 + u < nq ? *reinterpret_cast<const f32x4_t *>(w.absmax + b0 + kTileSup * u)
                         : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kRun; ++u)
#pragma unroll
      for (int b = 0; b < kTileSup; ++b) v[u][b] = a[u][b];
    return;
  }
  uint32_t word[kRun];
  float ga[kRun];
#pragma unroll
  for (int u = 0; u < kRun; ++u) {
    const bool in = q0 + u < nq;
    word[u] = in ? *reinterpret_cast<const uint32_t *>(w.scale_code + b0 + kTileSup * u) : 0u;
    ga[u] = in ? w.group_amax[(b0 + kTileSup * u) / kGroup] : 0.f;
  }
  const float off = *w.offset;
#pragma unroll
  for (int u = 0; u < kRun; ++u)
    if (q0 + u < nq)
#pragma unroll
      for (int b = 0; b < kTileSup; ++b) v[u][b] = block_scale((word[u] >> (8 * b)) & 0xFFu, ga[u], off);
}

// Forward scale table: for weight tile to (rows 256to ..) and super-step sp
// (blocks 4sp .. 4sp+3 of each row) one contiguous 4 KB run,
// Sp[((to*nsup + sp)*256 + row)*4 + q]; rows past n and blocks past k/64 hold
// 0.  A wave's store covers 64 consecutive rows (1 KB).
__device__ __forceinline__ void run_scales_fwd(const SmallJob &j, uint32_t t) {
  const uint32_t nsup = (uint32_t)j.a, runs = (nsup + kRun - 1) / kRun;
  const uint32_t q = t >> 8, to = q / runs, sp0 = (q - to * runs) * kRun, row = t & 255;
  float v[kRun][kTileSup];
  row_run_scales(j.w, (int64_t)to * kTileRows + row, sp0, v);
  f32x4_t *out = reinterpret_cast<f32x4_t *>(j.out) + ((size_t)to * nsup + sp0) * 256 + row;
#pragma unroll
  for (int u = 0; u < kRun; ++u)
    if (sp0 + u < nsup) out[u * 256] = f32x4_t{v[u][0], v[u][1], v[u][2], v[u][3]};
}

// Backward scale table: for column tile tk (k-blocks 4tk .. 4tk+3) and
// super-step sp (weight rows 256sp .. 256sp+255) one contiguous 4 KB run,
// Sp[((tk*nsup + sp)*4 + blk)*256 + row]; rows past n and blocks past k/64
// hold 0.  A wave's store covers 64 consecutive rows of one block (256 B).
__device__ __forceinline__ void run_scales_bwd(const SmallJob &j, uint32_t t) {
  const uint32_t nsup = (uint32_t)j.a, ntk = (uint32_t)j.b, runs = (ntk + kRun - 1) / kRun;
  const uint32_t q = t >> 8, sp = q / runs, tk0 = (q - sp * runs) * kRun, row = t & 255;
  float v[kRun][kTileSup];
  row_run_scales(j.w, (int64_t)sp * kTileRows + row, tk0, v);
  float *out = static_cast<float *>(j.out) + ((size_t)tk0 * nsup + sp) * 4 * 256 + row;
#pragma unroll
  for (int u = 0; u < kRun; ++u)
    if (tk0 + u < ntk)
#pragma unroll
      for (int blk = 0; blk < kTileSup; ++blk) out[((size_t)u * nsup * 4 + blk) * 256] = v[u][blk];
}

__global__ __launch_bounds__(256) void k_small_jobs(SmallJobs js) {
  __shared__ uint16_t t[64][65];  // the tiled jobs' transpose buffer
  const int64_t blk = blockIdx.x;
  int q = 0;
  while (q + 1 < js.n && blk >= js.start[q + 1]) ++q;
  const SmallJob &j = js.j[q];
  uint32_t lb = (uint32_t)(blk - js.start[q]);
  // scale tables: consecutive runs of one row tile share code lines, so a
  // contiguous range of them goes to each XCD (blocks are dealt to the XCDs
  // round-robin)
  if (j.kind == kJobScalesFwd || j.kind == kJobScalesBwd)
    lb = (uint32_t)xcd_tile((int)lb, (int)(js.start[q + 1] - js.start[q]));
  const uint32_t idx = lb * 256u + threadIdx.x;
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
  j.count = ceil_div(w.n, kTileRows) * ceil_div(j.a, kRun) * 256;
  j.out = scales;
  j.w = w;
  return j;
}

SmallJob job_scales_bwd(const Nf4View &w, float *scales) {
  SmallJob j;
  j.kind = kJobScalesBwd;
  j.a = tile_bwd_nsup(w.n);
  j.b = ceil_div(w.k, kTileRows);  // column tiles of four blocks
  j.count = j.a * ceil_div(j.b, kRun) * 256;
  j.out = scales;
  j.w = w;
  return j;
}

}  // namespace qlora

// nf4_tile.h -- launch interface of the NF4 x BF16 tile kernels (nf4_tile.hip).
#pragma once

#include "lora_gemm.h"

namespace qlora {

// Tile kernels: 256-row output tiles; codes and scales staged 4 steps (of 64
// contraction positions) at a time.
constexpr int kTileRows = 256;
constexpr int kTileSup = 4;
__host__ __device__ inline int64_t tile_fwd_nsup(int64_t k) { return (k / kBlock + kTileSup - 1) / kTileSup; }
__host__ __device__ inline int64_t tile_bwd_nsup(int64_t n) { return (n + kTileRows - 1) / kTileRows; }

// Device bytes of the block-scale table either pass stages for an [n, k]
// weight (the larger of the two layouts).
size_t tile_scales_bytes(int64_t n, int64_t k);

// Whether launch_bwd_dx_tiles handles this weight shape: n % 64 == 0, and
// the packed weight and a 256-row dY tile below 2^31 bytes (32-bit offsets).
bool bwd_tiles_supported(int64_t n, int64_t k);

// Contraction splits of one tile launch: `splits` workgroups per output
// tile, each over `lsteps` 64-wide steps (a multiple of 8), whose float32
// partial tiles a reduction kernel sums in split order.
struct TileSplit {
  int splits = 1;
  int lsteps = 8;
};
TileSplit plan_tile_split(int64_t tiles, int64_t nk, int64_t M, int64_t NO);
TileSplit plan_fwd_tiles(int64_t M, int64_t n, int64_t k);
TileSplit plan_dx_tiles(int64_t M, int64_t n, int64_t k);
// Device bytes of the partial tiles the forward / the dX tile launch writes
// (0 when unsplit).
size_t tile_fwd_partial_bytes(int64_t M, int64_t n, int64_t k);
size_t tile_dx_partial_bytes(int64_t M, int64_t n, int64_t k);

// One float4 slot of a split launch's partial tiles (slot = (tile * 64 + j)
// * 256 + t, the tile kernel's register order): out[m][o..o+3] = bf16( sum
// over s = 0 .. splits-1, in that order, of the slot's partials ), for the
// tile kernel's C[o][m] with o = 256 (tile % tiles_o) + 64 (t / 64) + 16 (j /
// 16) + 4 ((t % 64) / 16) and m = 256 (tile / tiles_o) + 16 (j % 16) + t % 16.
__device__ __forceinline__ void split_reduce_slot(const f32x4_t *__restrict__ part, int splits, int ntiles,
                                                  int tiles_o, int64_t M, int64_t NO, uint16_t *__restrict__ out,
                                                  int64_t slot) {
  const int t = (int)(slot & 255), lane = t & 63, wave = t >> 6;
  const int64_t tj = slot >> 8;  // tile * 64 + j
  const int j = (int)(tj & 63);
  const int64_t tile = tj >> 6;
  const int64_t to = tile % tiles_o, mt = tile / tiles_o;
  const int64_t o = to * kTileRows + 64 * wave + 16 * (j >> 4) + 4 * (lane >> 4);
  const int64_t m = mt * kTileRows + 16 * (j & 15) + (lane & 15);
  if (m >= M || o >= NO) return;
  const int64_t stride = (int64_t)ntiles * 64 * 256;
  f32x4_t a = part[slot];
  for (int s = 1; s < splits; ++s) {
    const f32x4_t b = part[s * stride + slot];
    a = f32x4_t{a[0] + b[0], a[1] + b[1], a[2] + b[2], a[3] + b[3]};
  }
  uint16_t *dst = out + m * NO + o;
  if ((NO & 3) == 0) {
    *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{bf16x2_rne(a[0], a[1]), bf16x2_rne(a[2], a[3])};
  } else {
    const uint32_t lo = bf16x2_rne(a[0], a[1]), hi = bf16x2_rne(a[2], a[3]);
    const uint16_t e[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (o + v < NO) dst[v] = e[v];
  }
}

// The same reduction as a small job (jobs.hip), to share a launch.
SmallJob job_split_reduce(const TileSplit &sp, int tiles_o, int tiles_m, int64_t M, int64_t NO, const float *tpart,
                          uint16_t *out);

// The block-scale tables the two tile kernels stream (jobs.hip, run by
// launch_jobs before the tile launch): `scales` is device scratch of
// tile_scales_bytes(n, k).
SmallJob job_scales_fwd(const Nf4View &w, float *scales);
SmallJob job_scales_bwd(const Nf4View &w, float *scales);

// Y[M, n] = bf16( X W_hat^T + sH B_lora^T ):  X [M, k], sH [M, RP] = bf16(s H)
// with the rank padded to RP by zeros, B_lora [n, r] (row stride r).
// `scales`: the table job_scales_fwd wrote.
// `tpart`: device scratch of tile_fwd_partial_bytes (may be NULL when it is 0).
hipError_t launch_fwd_tiles(const Nf4View &w, float *scales, const uint16_t *X, int64_t M, const uint16_t *Bl, int r,
                            int RP, const uint16_t *sH, uint16_t *Y, float *tpart, hipStream_t s);

#ifdef QLORA_PROFILE
// The same forward tile kernel on BF16 weights Wb [n, k] (no expansion):
// the 16-bit baseline of the tracing build.  One split, every shape the
// forward takes.
hipError_t launch_fwd_tiles_bf16w(const uint16_t *Wb, int64_t n, int64_t k, const uint16_t *X, int64_t M,
                                  const uint16_t *Bl, int r, int RP, const uint16_t *sH, uint16_t *Y, hipStream_t s);
#endif

// dX[M, k] = bf16( dY W_hat + G At^T ):  dY [M, n], At [k, RP] (A_lora
// transposed, rank padded), G [M, RP].  Requires bwd_tiles_supported;
// `scales`: the table job_scales_bwd wrote.
// With split_job != NULL a split launch's reduction is not launched but
// returned there (count 0 when the launch is unsplit), for a later jobs launch.
hipError_t launch_bwd_dx_tiles(const Nf4View &w, float *scales, const uint16_t *dY, int64_t M, const uint16_t *At,
                               int RP, const uint16_t *Gb, uint16_t *dX, float *tpart, hipStream_t s,
                               SmallJob *split_job = nullptr);

// Small-M forward (nf4_gemv.hip): the whole forward -- H, and
// Y = X W_hat^T + bf16(s H) B^T -- for 1 <= M <= kGemvMaxM in one pass over
// the packed weight.  Needs small_m_supported (k % 256 == 0, packed weight
// below 2^31 bytes, rank at most 128) and small_m_workspace_bytes of device
// scratch.
constexpr int64_t kGemvMaxM = 16;
bool small_m_supported(int64_t M, int64_t n, int64_t k, int r);
size_t small_m_workspace_bytes(int64_t M, int64_t n, int64_t k, int r);
hipError_t launch_fwd_small(const Nf4View &w, const uint16_t *X, int64_t M, const uint16_t *A, const uint16_t *B,
                            int r, float s, uint16_t *Y, float *H_out, void *ws, hipStream_t st);

}  // namespace qlora

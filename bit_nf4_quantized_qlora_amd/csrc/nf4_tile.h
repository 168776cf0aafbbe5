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

// Whether launch_bwd_dx_tiles handles this weight shape: n % 64 == 0 and the
// packed weight below 2^31 bytes (32-bit offsets into it).
bool bwd_tiles_supported(int64_t n, int64_t k);

// The block-scale tables the two tile kernels stream (jobs.hip, run by
// launch_jobs before the tile launch): `scales` is device scratch of
// tile_scales_bytes(n, k).
SmallJob job_scales_fwd(const Nf4View &w, float *scales);
SmallJob job_scales_bwd(const Nf4View &w, float *scales);

// Y[M, n] = bf16( X W_hat^T + sH B_lora^T ):  X [M, k], sH [M, RP] = bf16(s H)
// with the rank padded to RP by zeros, B_lora [n, r] (row stride r).
// `scales`: the table job_scales_fwd wrote.
hipError_t launch_fwd_tiles(const Nf4View &w, float *scales, const uint16_t *X, int64_t M, const uint16_t *Bl, int r,
                            int RP, const uint16_t *sH, uint16_t *Y, hipStream_t s);

// dX[M, k] = bf16( dY W_hat + G At^T ):  dY [M, n], At [k, RP] (A_lora
// transposed, rank padded), G [M, RP].  Requires bwd_tiles_supported;
// `scales`: the table job_scales_bwd wrote.
hipError_t launch_bwd_dx_tiles(const Nf4View &w, float *scales, const uint16_t *dY, int64_t M, const uint16_t *At,
                               int RP, const uint16_t *Gb, uint16_t *dX, hipStream_t s);

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

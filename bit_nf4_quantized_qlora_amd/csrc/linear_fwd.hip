// linear_fwd.hip -- forward pass of the frozen NF4 linear layer with LoRA.
//
// "QLoRA Paper Breakdown" sec. 4 Forward Pass: Y = X dequant(W)^T +
// (alpha/r) X L_1 L_2, with the weights expanded from NF4 to BF16 on every
// use ("QLoRA, explained." step 4).
//
//   1. H = X A^T (k_nt_dma, then its reduction in one launch with the
//      tile kernel's block-scale table): fp32 H (optional output) and
//      bf16(s*H) for the LoRA term.
//   2. k_fwd_nf4 (nf4_tile.hip): Y = X W_hat^T + sH B^T on
//      256x256 tiles, the NF4 codes expanded in registers straight into MFMA
//      operands and the LoRA up-projection added on the same accumulators;
//      Y is rounded to bf16 once.  When the tiles cannot fill the GPU (M =
//      512 on 4096- and 8192-wide layers) the contraction is split and
//      k_split_reduce sums the float32 partial tiles in split order.
// For 1 <= M <= 16 the whole forward is nf4_gemv.hip's instead (k_gemv_nf4,
// k_gemv_finish): one bandwidth-bound pass over the packed weight.
#include "nf4_tile.h"

namespace qlora {
namespace {

struct FwdWs {
  SplitPlan sp;
  int RP;
  size_t part_off, sh_off, scale_off, tpart_off, total;
};

// Tile-path layout (the small-M GEMV path lays out its own workspace).
FwdWs fwd_ws_layout(int64_t M, int64_t n, int64_t k, int r) {
  FwdWs l;
  l.RP = lora_rank_pad(r);
  l.sp = plan_split(ceil_div(M, 64), ceil_div(k, 64));
  l.part_off = 0;
  l.sh_off = align_up((size_t)l.sp.splits * M * l.RP * sizeof(float), 256);
  l.scale_off = l.sh_off + align_up((size_t)M * l.RP * sizeof(uint16_t), 256);
  l.tpart_off = l.scale_off + align_up(tile_scales_bytes(n, k), 256);
  l.total = l.tpart_off + align_up(tile_fwd_partial_bytes(M, n, k), 256);
  return l;
}

}  // namespace

size_t fwd_workspace_bytes_for(int64_t M, int64_t n, int64_t k, int r, bool single_level) {
  if (plan_linear(M, n, k, r, single_level).fwd_path == QLORA_PATH_GEMV) return small_m_workspace_bytes(M, n, k, r);
  return fwd_ws_layout(M, n, k, r).total;
}

// Either storage type's need (the public query does not know the type).
size_t fwd_workspace_bytes(int64_t M, int64_t n, int64_t k, int r) {
  return std::max(fwd_workspace_bytes_for(M, n, k, r, false), fwd_workspace_bytes_for(M, n, k, r, true));
}

LinearPlan plan_linear(int64_t M, int64_t n, int64_t k, int r, bool single_level) {
  LinearPlan p;
  if (M == 0) return p;
  (void)single_level;  // the GEMV takes either kind of block constants
  if (small_m_supported(M, n, k, r)) {
    p.fwd_path = QLORA_PATH_GEMV;
  } else {
    p.fwd_path = QLORA_PATH_TILE;
    p.fwd_splits = plan_fwd_tiles(M, n, k).splits;
  }
  if (bwd_tiles_supported(n, k)) {
    p.dx_path = QLORA_PATH_TILE;
    p.dx_splits = plan_dx_tiles(M, n, k).splits;
  } else {
    p.dx_path = QLORA_PATH_GENERAL;
  }
  return p;
}

hipError_t launch_linear_fwd(const LinearArgs &a, const uint16_t *X, const uint16_t *A, const uint16_t *B,
                             uint16_t *Y, float *H_out, void *ws, hipStream_t s) {
  const int64_t M = a.M, N = a.w.n, K = a.w.k;
  if (M == 0) return hipSuccess;
  if (plan_linear(M, N, K, a.r, a.w.absmax != nullptr).fwd_path == QLORA_PATH_GEMV)
    return launch_fwd_small(a.w, X, M, A, B, a.r, a.s, Y, H_out, ws, s);
  const FwdWs l = fwd_ws_layout(M, N, K, a.r);
  char *base = static_cast<char *>(ws);
  float *part = reinterpret_cast<float *>(base + l.part_off);
  uint16_t *sH = reinterpret_cast<uint16_t *>(base + l.sh_off);
  float *scales = reinterpret_cast<float *>(base + l.scale_off);
  float *tpart = reinterpret_cast<float *>(base + l.tpart_off);
  hipError_t e = launch_nt_splitk(X, M, A, a.r, l.RP, K, K, l.sp, part, s);
  if (e != hipSuccess) return e;
  // H's reduction and the tile kernel's scale table in one launch
  const SmallJob jobs[2] = {job_reduce_rows(part, l.sp.splits, M, l.RP, a.r, a.s, H_out, sH, nullptr, 0),
                            job_scales_fwd(a.w, scales)};
  e = launch_jobs("k_prep_fwd", jobs, 2, s);
  if (e != hipSuccess) return e;
  return launch_fwd_tiles(a.w, scales, X, M, B, a.r, l.RP, sH, Y, tpart, s);
}

#ifdef QLORA_PROFILE
// The forward with BF16 weights on the same kernels (tracing build): H and
// its reduction exactly as above, then the tile kernel reading Wb instead of
// expanding codes.  No block-scale table is needed.
hipError_t launch_linear_fwd_bf16w(const uint16_t *Wb, int64_t N, int64_t K, int64_t M, int r, float s_lora,
                                   const uint16_t *X, const uint16_t *A, const uint16_t *B, uint16_t *Y, float *H_out,
                                   void *ws, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const FwdWs l = fwd_ws_layout(M, N, K, r);
  char *base = static_cast<char *>(ws);
  float *part = reinterpret_cast<float *>(base + l.part_off);
  uint16_t *sH = reinterpret_cast<uint16_t *>(base + l.sh_off);
  hipError_t e = launch_nt_splitk(X, M, A, r, l.RP, K, K, l.sp, part, s);
  if (e != hipSuccess) return e;
  const SmallJob jobs[1] = {job_reduce_rows(part, l.sp.splits, M, l.RP, r, s_lora, H_out, sH, nullptr, 0)};
  e = launch_jobs("k_prep_fwd", jobs, 1, s);
  if (e != hipSuccess) return e;
  return launch_fwd_tiles_bf16w(Wb, N, K, X, M, B, r, l.RP, sH, Y, s);
}
#endif

}  // namespace qlora

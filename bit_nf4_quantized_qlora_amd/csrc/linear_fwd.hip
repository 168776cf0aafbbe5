// linear_fwd.hip -- forward pass of the frozen NF4 linear layer with LoRA.
//
// "QLoRA Paper Breakdown" sec. 4 Forward Pass: Y = X dequant(W)^T +
// (alpha/r) X L_1 L_2, with the weights expanded from NF4 to BF16 on every
// use ("QLoRA, explained." step 4).
//
//   1. H = X A^T (k_nt_splitk, then its reduction in one launch with the
//      tile kernel's block-scale table): fp32 H (optional output) and
//      bf16(s*H) for the LoRA term.
//   2. k_fwd_nf4 (nf4_tile.hip): Y = X W_hat^T + sH B^T on
//      256x256 tiles, the NF4 codes expanded in registers straight into MFMA
//      operands and the LoRA up-projection added on the same accumulators;
//      Y is rounded to bf16 once.
// For 1 <= M <= 16 the whole forward is nf4_gemv.hip's instead (k_gemv_nf4,
// k_gemv_finish): one bandwidth-bound pass over the packed weight.
#include "nf4_tile.h"

namespace qlora {
namespace {

struct FwdWs {
  SplitPlan sp;
  int RP;
  size_t part_off, sh_off, scale_off, total;
};

FwdWs fwd_ws_layout(int64_t M, int64_t n, int64_t k, int r) {
  FwdWs l;
  l.RP = lora_rank_pad(r);
  l.sp = plan_split(ceil_div(M, 64), ceil_div(k, 64));
  l.part_off = 0;
  l.sh_off = align_up((size_t)l.sp.splits * M * l.RP * sizeof(float), 256);
  l.scale_off = l.sh_off + align_up((size_t)M * l.RP * sizeof(uint16_t), 256);
  l.total = l.scale_off + align_up(tile_scales_bytes(n, k), 256);
  if (small_m_supported(M, n, k, r)) l.total = std::max(l.total, small_m_workspace_bytes(M, n, k, r));
  return l;
}

}  // namespace

size_t fwd_workspace_bytes(int64_t M, int64_t n, int64_t k, int r) { return fwd_ws_layout(M, n, k, r).total; }

hipError_t launch_linear_fwd(const LinearArgs &a, const uint16_t *X, const uint16_t *A, const uint16_t *B,
                             uint16_t *Y, float *H_out, void *ws, hipStream_t s) {
  const int64_t M = a.M, N = a.w.n, K = a.w.k;
  if (M == 0) return hipSuccess;
  // the GEMV decodes double-quantized constants only; single-level weights
  // take the tile kernels at every M
  if (!a.w.absmax && small_m_supported(M, N, K, a.r)) return launch_fwd_small(a.w, X, M, A, B, a.r, a.s, Y, H_out, ws, s);
  const FwdWs l = fwd_ws_layout(M, N, K, a.r);
  char *base = static_cast<char *>(ws);
  float *part = reinterpret_cast<float *>(base + l.part_off);
  uint16_t *sH = reinterpret_cast<uint16_t *>(base + l.sh_off);
  float *scales = reinterpret_cast<float *>(base + l.scale_off);
  hipError_t e = launch_nt_splitk(X, M, A, a.r, l.RP, K, K, l.sp, part, s);
  if (e != hipSuccess) return e;
  // H's reduction and the tile kernel's scale table in one launch
  const SmallJob jobs[2] = {job_reduce_rows(part, l.sp.splits, M, l.RP, a.r, a.s, H_out, sH, nullptr, 0),
                            job_scales_fwd(a.w, scales)};
  e = launch_jobs("k_prep_fwd", jobs, 2, s);
  if (e != hipSuccess) return e;
  return launch_fwd_tiles(a.w, scales, X, M, B, a.r, l.RP, sH, Y, s);
}

}  // namespace qlora

// linear_fwd.hip -- forward pass of the frozen NF4 linear layer with LoRA.
//
// "QLoRA Paper Breakdown" sec. 4 Forward Pass: Y = X dequant(W)^T +
// (alpha/r) X L_1 L_2, with the weights expanded from NF4 to BF16 on every
// use ("QLoRA, explained." step 4; "reading note": the multiply runs in 16
// bits).
//
//   1. H = X A^T (k_nt_splitk + reduction): fp32 H (optional output) and
//      bf16(s*H) for the epilogue.
//   2. k_fwd_main: C[n][m] = sum_k W_hat[n][k] X[m][k] + sum_j B[n][j] sH[m][j]
//      on 128x128 tiles.  Each K step (64 = one NF4 block per weight row)
//      streams 32 packed bytes per row, expands them in registers through the
//      shared dequant_word (so the tile equals the standalone dequant bit for
//      bit), and stages the BF16 tile to LDS next to the X tile; four waves
//      run 16x16x32 BF16 MFMAs on 64x64 sub-tiles.  The LoRA up-projection is
//      a few more MFMA steps on the same accumulators; Y is rounded to bf16
//      once at the end.
#include "lora_gemm.h"

namespace qlora {
namespace {

constexpr int FBN = 128, FBM = 128, FLD = 72;

__global__ __launch_bounds__(256, 2) void k_fwd_main(Nf4View w, const uint16_t *__restrict__ X, int64_t M,
                                                     const uint16_t *__restrict__ Bl, int r, int RP,
                                                     const uint16_t *__restrict__ sH, uint16_t *__restrict__ Y) {
  __shared__ __align__(16) uint16_t Ps[2 * FBN * FLD];  // W_hat tile [n][k]
  __shared__ __align__(16) uint16_t Qs[2 * FBM * FLD];  // X tile [m][k]
  __shared__ float2 s_pair[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t N = w.n, K = w.k, nk = K / kBlock;
  const int64_t n0 = (int64_t)blockIdx.x * FBN, m0 = (int64_t)blockIdx.y * FBM;
  fill_pair_table(s_pair, tid, 256);
  const float offset = *w.offset;

  // Weight staging: thread -> (row tid/2, half tid%2): 16 packed bytes = 32 codes.
  const int wr = tid >> 1, wh = tid & 1;
  const bool wvalid = n0 + wr < N;
  const int64_t wrow = wvalid ? n0 + wr : 0;
  const uint8_t *wsrc = w.packed + wrow * (K / 2) + wh * 16;
  const int64_t bbase = wrow * nk;

  u32x4_t wreg = {0u, 0u, 0u, 0u};
  uint32_t sc = 0;
  float ga = 0.f;
  u32x4_t xreg[4];
  auto gload = [&](int64_t kt) {
    wreg = *reinterpret_cast<const u32x4_t *>(wsrc + kt * 32);
    sc = w.scale_code[bbase + kt];
    ga = w.group_amax[(bbase + kt) >> 8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      xreg[i] = load8(X, K, M, K, m0 + row, kt * 64 + col, true);
    }
  };
  auto lstore = [&](int buf) {
    uint16_t *P = Ps + buf * FBN * FLD + wr * FLD + wh * 32;
    const float s = block_scale(sc, ga, offset);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t o[4];
      dequant_word(wreg[q], s, s_pair, o);
      *reinterpret_cast<u32x4_t *>(P + 8 * q) = wvalid ? u32x4_t{o[0], o[1], o[2], o[3]} : u32x4_t{0u, 0u, 0u, 0u};
    }
    uint16_t *Qb = Qs + buf * FBM * FLD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4_t *>(Qb + row * FLD + col) = xreg[i];
    }
  };

  __syncthreads();  // pair table ready
  gload(0);
  lstore(0);
  __syncthreads();

  const int wi = wave >> 1, wj = wave & 1;
  f32x4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < nk) gload(kt + 1);
    const uint16_t *Pb = Ps + buf * FBN * FLD, *Qb = Qs + buf * FBM * FLD;
    mma_step<4, 4>(acc, Pb, Qb, FLD, 64 * wi, 64 * wj, 0, lane);
    mma_step<4, 4>(acc, Pb, Qb, FLD, 64 * wi, 64 * wj, 32, lane);
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // LoRA up-projection: acc += B[n][:] . sH[m][:] over the padded rank.
  const int LE = RP + 8;
  const int cpr = RP / 8;  // 16-byte chunks per row
  const bool bvec = (r % 8) == 0;
  for (int c = tid; c < FBN * cpr; c += 256) {
    const int row = c / cpr, col = (c % cpr) * 8;
    *reinterpret_cast<u32x4_t *>(Ps + row * LE + col) = load8(Bl, r, N, r, n0 + row, col, bvec);
  }
  for (int c = tid; c < FBM * cpr; c += 256) {
    const int row = c / cpr, col = (c % cpr) * 8;
    *reinterpret_cast<u32x4_t *>(Qs + row * LE + col) = load8(sH, RP, M, RP, m0 + row, col, true);
  }
  __syncthreads();
  for (int kk = 0; kk < RP; kk += 32) mma_step<4, 4>(acc, Ps, Qs, LE, 64 * wi, 64 * wj, kk, lane);

  // acc[ti][tj][v] = C[n][m], n = .. + 4*(lane>>4) + v, m = .. + (lane & 15): four consecutive n of one Y row.
  const bool nvec = (N & 3) == 0;
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const int64_t n = n0 + 64 * wi + 16 * ti + 4 * (lane >> 4);
      const int64_t m = m0 + 64 * wj + 16 * tj + (lane & 15);
      if (m >= M) continue;
      const f32x4_t a = acc[ti][tj];
      uint16_t *dst = Y + m * N + n;
      if (nvec && n + 4 <= N) {
        *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{bf16x2_rne(a[0], a[1]), bf16x2_rne(a[2], a[3])};
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (n + v < N) dst[v] = f32_to_bf16_bits(a[v]);
      }
    }
}

struct FwdWs {
  SplitPlan sp;
  int RP;
  size_t part_off, sh_off, total;
};

FwdWs fwd_ws_layout(int64_t M, int64_t n, int64_t k, int r) {
  FwdWs l;
  l.RP = lora_rank_pad(r);
  l.sp = plan_split(ceil_div(M, 64), ceil_div(k, 64));
  l.part_off = 0;
  l.sh_off = align_up((size_t)l.sp.splits * M * l.RP * sizeof(float), 256);
  l.total = l.sh_off + align_up((size_t)M * l.RP * sizeof(uint16_t), 256);
  (void)n;
  return l;
}

}  // namespace

size_t fwd_workspace_bytes(int64_t M, int64_t n, int64_t k, int r) { return fwd_ws_layout(M, n, k, r).total; }

hipError_t launch_linear_fwd(const LinearArgs &a, const uint16_t *X, const uint16_t *A, const uint16_t *B,
                             uint16_t *Y, float *H_out, void *ws, hipStream_t s) {
  const int64_t M = a.M, N = a.w.n, K = a.w.k;
  if (M == 0) return hipSuccess;
  const FwdWs l = fwd_ws_layout(M, N, K, a.r);
  float *part = reinterpret_cast<float *>(static_cast<char *>(ws) + l.part_off);
  uint16_t *sH = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + l.sh_off);
  hipError_t e = launch_nt_splitk(X, M, A, a.r, l.RP, K, K, l.sp, part, s);
  if (e != hipSuccess) return e;
  e = launch_reduce_rows(part, l.sp.splits, M, l.RP, a.r, a.s, H_out, sH, nullptr, 0, s);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)ceil_div(N, FBN), (unsigned)ceil_div(M, FBM));
  QLORA_LAUNCH("k_fwd_main", k_fwd_main, grid, dim3(256), 0, s, a.w, X, M, B, a.r, l.RP, sH, Y);
  return hipGetLastError();
}

}  // namespace qlora

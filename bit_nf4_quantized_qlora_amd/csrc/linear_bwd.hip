// linear_bwd.hip -- backward pass of the frozen NF4 linear layer with LoRA.
//
// "QLoRA Paper Breakdown" sec. 4: the input gradient needs the NF4 weights
// dequantized again on the fly, and dL/dW is never materialized; "QLoRA,
// explained." step 5: gradients reach the adapters only.  With
// Y = X W_hat^T + s (X A^T) B^T:
//   G  = s dY B            (k_nt_dma on dY and B as it lies for r % 8 == 0,
//                           r <= 64; otherwise on dY and a copy of B^T)
//   dX = dY W_hat + G A    (k_bwd_dx_nf4 in nf4_tile.hip, its contraction
//                           split when the tiles cannot fill the GPU;
//                           k_bwd_dx below when n % 64 != 0)
//   dB = s dY^T H          (k_tn_splitk on dY and (sH)^T)
//   dA = G^T X             (k_tn_splitk on X and G^T; one launch with dB's,
//                           before the dX launch)
// The small layout copies (A^T, (sH)^T, and B^T where needed), the tile
// kernel's block-scale table and the partial reductions run as jobs.hip
// launches, several jobs per launch.
//
// k_bwd_dx, the general fallback, contracts over n, the row index of W, by
// laying the dequantized tile into LDS transposed: each thread expands one
// packed dword (8 codes along k) from each of 4 consecutive rows n,
// transposes the 4x8 block in registers with byte permutes and writes eight
// 8-byte runs of [k][n].  The output tile is computed as C[k][m] so a lane's
// four accumulators are four consecutive k of one dX row.
#include "nf4_tile.h"

namespace qlora {
namespace {

constexpr int DBK = 128, DBM = 128, DLD = 72;

__global__ __launch_bounds__(256, 2) void k_bwd_dx(Nf4View w, const uint16_t *__restrict__ dY, int64_t M,
                                                   const uint16_t *__restrict__ At, const uint16_t *__restrict__ Gb,
                                                   int RP, uint16_t *__restrict__ dX) {
  __shared__ __align__(16) uint16_t Ps[2 * DBK * DLD];  // W_hat^T tile [k][n]
  __shared__ __align__(16) uint16_t Qs[2 * DBM * DLD];  // dY tile [m][n]
  __shared__ float2 s_pair[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t N = w.n, K = w.k, nkb = K / kBlock;
  const int64_t k0 = (int64_t)blockIdx.x * DBK, m0 = (int64_t)blockIdx.y * DBM;
  const int64_t nsteps = ceil_div_d(N, 64);
  fill_pair_table(s_pair, tid, 256, w.codebook);
  const bool single = w.absmax != nullptr;  // s_b = absmax_b
  const float offset = single ? 0.f : *w.offset;
  const bool dyvec = (N % 8) == 0;

  // Weight staging: rows n0 + 4*ng + rho (rho = 0..3), codes k0 + 8*kg .. +7.
  const int ng = tid >> 4, kg = tid & 15;
  const int64_t kcol = k0 + 8 * kg;
  const bool kvalid = kcol < K;
  uint32_t wd[4], sc[4];
  float ga[4];
  bool wok[4];
  u32x4_t yreg[4];
  auto gload = [&](int64_t st) {
    const int64_t n0 = st * 64;
#pragma unroll
    for (int rho = 0; rho < 4; ++rho) {
      const int64_t n = n0 + 4 * ng + rho;
      const bool ok = kvalid && n < N;
      const int64_t nn = ok ? n : 0, kk = ok ? kcol : 0;  // out-of-range rows read row 0
      wd[rho] = *reinterpret_cast<const uint32_t *>(w.packed + (nn * K + kk) / 2);
      const int64_t b = nn * nkb + kk / kBlock;
      if (single) {
        sc[rho] = __float_as_uint(w.absmax[b]);
        ga[rho] = 0.f;
      } else {
        sc[rho] = w.scale_code[b];
        ga[rho] = w.group_amax[b >> 8];
      }
      wok[rho] = ok;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      yreg[i] = load8(dY, N, M, N, m0 + row, n0 + col, dyvec);
    }
  };
  auto lstore = [&](int buf) {
    uint32_t o[4][4];
#pragma unroll
    for (int rho = 0; rho < 4; ++rho) {
      dequant_word(wd[rho], single ? __uint_as_float(sc[rho]) : block_scale(sc[rho], ga[rho], offset), s_pair, o[rho]);
      if (!wok[rho]) o[rho][0] = o[rho][1] = o[rho][2] = o[rho][3] = 0u;
    }
    uint16_t *P = Ps + buf * DBK * DLD + 4 * ng;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      *reinterpret_cast<u32x2_t *>(P + (8 * kg + 2 * d) * DLD) =
          u32x2_t{pack_lo(o[0][d], o[1][d]), pack_lo(o[2][d], o[3][d])};
      *reinterpret_cast<u32x2_t *>(P + (8 * kg + 2 * d + 1) * DLD) =
          u32x2_t{pack_hi(o[0][d], o[1][d]), pack_hi(o[2][d], o[3][d])};
    }
    uint16_t *Qb = Qs + buf * DBM * DLD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4_t *>(Qb + row * DLD + col) = yreg[i];
    }
  };

  __syncthreads();
  gload(0);
  lstore(0);
  __syncthreads();

  const int wi = wave >> 1, wj = wave & 1;
  f32x4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t st = 0; st < nsteps; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < nsteps) gload(st + 1);
    const uint16_t *Pb = Ps + buf * DBK * DLD, *Qb = Qs + buf * DBM * DLD;
    mma_step<4, 4>(acc, Pb, Qb, DLD, 64 * wi, 64 * wj, 0, lane);
    mma_step<4, 4>(acc, Pb, Qb, DLD, 64 * wi, 64 * wj, 32, lane);
    if (st + 1 < nsteps) lstore(buf ^ 1);
    __syncthreads();
  }

  // LoRA term: acc += A^T[k][:] . G[m][:] over the padded rank.
  const int LE = RP + 8, cpr = RP / 8;
  for (int c = tid; c < DBK * cpr; c += 256) {
    const int row = c / cpr, col = (c % cpr) * 8;
    *reinterpret_cast<u32x4_t *>(Ps + row * LE + col) = load8(At, RP, K, RP, k0 + row, col, true);
  }
  for (int c = tid; c < DBM * cpr; c += 256) {
    const int row = c / cpr, col = (c % cpr) * 8;
    *reinterpret_cast<u32x4_t *>(Qs + row * LE + col) = load8(Gb, RP, M, RP, m0 + row, col, true);
  }
  __syncthreads();
  for (int kk = 0; kk < RP; kk += 32) mma_step<4, 4>(acc, Ps, Qs, LE, 64 * wi, 64 * wj, kk, lane);

#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      const int64_t k = k0 + 64 * wi + 16 * ti + 4 * (lane >> 4);
      const int64_t m = m0 + 64 * wj + 16 * tj + (lane & 15);
      if (m >= M || k >= K) continue;
      const f32x4_t a = acc[ti][tj];
      *reinterpret_cast<u32x2_t *>(dX + m * K + k) = u32x2_t{bf16x2_rne(a[0], a[1]), bf16x2_rne(a[2], a[3])};
    }
}

struct BwdWs {
  int RP;
  int64_t Mp;
  SplitPlan sp_h, sp_g, sp_b, sp_a;
  size_t part_off, parta_off, h_off, sht_off, bt_off, at_off, gb_off, gt_off, scale_off, tpart_off, total;
};

BwdWs bwd_ws_layout(int64_t M, int64_t N, int64_t K, int r) {
  BwdWs l;
  l.RP = lora_rank_pad(r);
  l.Mp = ceil_div(M, 64) * 64;
  l.sp_h = plan_split(ceil_div(M, 64), ceil_div(K, 64));
  l.sp_g = plan_split(ceil_div(M, 64), ceil_div(N, 64));
  l.sp_b = plan_split(ceil_div(N, 64), ceil_div(M, 64));
  l.sp_a = plan_split(ceil_div(K, 64), ceil_div(M, 64));
  // one partials region: H's or G's split partials, later dB's and dA's side by side
  l.parta_off = align_up((size_t)l.sp_b.splits * l.RP * N * sizeof(float), 256);
  size_t part = std::max({(size_t)l.sp_h.splits * M * l.RP * sizeof(float),
                          (size_t)l.sp_g.splits * M * l.RP * sizeof(float),
                          l.parta_off + (size_t)l.sp_a.splits * l.RP * K * sizeof(float)});
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes, 256);
    return at;
  };
  l.part_off = take(part);
  l.h_off = take((size_t)M * r * sizeof(float));
  l.sht_off = take((size_t)l.RP * l.Mp * 2);
  l.bt_off = take((size_t)l.RP * N * 2);
  l.at_off = take((size_t)K * l.RP * 2);
  l.gb_off = take((size_t)M * l.RP * 2);
  l.gt_off = take((size_t)l.RP * l.Mp * 2);
  l.scale_off = take(tile_scales_bytes(N, K));
  l.tpart_off = take(tile_dx_partial_bytes(M, N, K));
  l.total = off;
  return l;
}

}  // namespace

size_t bwd_workspace_bytes(int64_t M, int64_t n, int64_t k, int r) { return bwd_ws_layout(M, n, k, r).total; }

hipError_t launch_linear_bwd(const LinearArgs &a, const uint16_t *X, const uint16_t *dY, const uint16_t *A,
                             const uint16_t *B, const float *H, uint16_t *dX, uint16_t *dA, uint16_t *dB,
                             void *ws, hipStream_t s) {
  const int64_t M = a.M, N = a.w.n, K = a.w.k;
  const int r = a.r;
  hipError_t e;
#define QLORA_TRY(x)              \
  do {                            \
    e = (x);                      \
    if (e != hipSuccess) return e; \
  } while (0)
  if (M == 0) {  // empty batch: the adapter gradients are sums over nothing
    QLORA_TRY(launch_fill_zero_u16(dA, (int64_t)r * K, s));
    QLORA_TRY(launch_fill_zero_u16(dB, N * r, s));
    return hipSuccess;
  }
  const BwdWs l = bwd_ws_layout(M, N, K, r);
  char *base = static_cast<char *>(ws);
  float *part = reinterpret_cast<float *>(base + l.part_off);
  uint16_t *sHt = reinterpret_cast<uint16_t *>(base + l.sht_off);
  uint16_t *Bt = reinterpret_cast<uint16_t *>(base + l.bt_off);
  uint16_t *At = reinterpret_cast<uint16_t *>(base + l.at_off);
  uint16_t *Gb = reinterpret_cast<uint16_t *>(base + l.gb_off);
  uint16_t *Gt = reinterpret_cast<uint16_t *>(base + l.gt_off);
  const int RP = l.RP;

  if (H == nullptr) {  // recompute H = X A^T
    float *Hw = reinterpret_cast<float *>(base + l.h_off);
    QLORA_TRY(launch_nt_splitk(X, M, A, r, RP, K, K, l.sp_h, part, s));
    QLORA_TRY(launch_reduce_rows(part, l.sp_h.splits, M, RP, r, 1.f, Hw, nullptr, nullptr, 0, s));
    H = Hw;
  }
  // layouts: sHt = bf16(s H)^T [RP][Mp], At [K][RP]; and the dX tile
  // kernel's block-scale table.  G = s dY B -> Gb [M][RP], Gt [RP][Mp].
  // When the product can read B [N][r] as it lies (r % 8 == 0, r <= 64), G's
  // split partials come first and their reduction joins the layout jobs in
  // one launch; otherwise B is transposed to Bt [RP][N] first.
  const bool tiles = dX != nullptr && plan_linear(M, N, K, r, a.w.absmax != nullptr).dx_path == QLORA_PATH_TILE;
  float *scales = reinterpret_cast<float *>(base + l.scale_off);
  const bool b_rows = nt_rows_supported(r, N);
  SmallJob prep[kMaxJobs];
  int np = 0;
  prep[np++] = job_scale_transpose(H, M, r, a.s, sHt, RP, l.Mp);
  prep[np++] = job_transpose_pad(A, r, K, At, K, RP);
  if (tiles) prep[np++] = job_scales_bwd(a.w, scales);
  if (b_rows) {
    QLORA_TRY(launch_nt_rows(dY, M, B, r, RP, N, N, l.sp_g, part, s));
    prep[np++] = job_reduce_rows(part, l.sp_g.splits, M, RP, r, a.s, nullptr, Gb, Gt, l.Mp);
    QLORA_TRY(launch_jobs("k_prep_bwd", prep, np, s));
  } else {
    prep[np++] = job_transpose_pad(B, N, r, Bt, RP, N);
    QLORA_TRY(launch_jobs("k_prep_bwd", prep, np, s));
    QLORA_TRY(launch_nt_splitk(dY, M, Bt, RP, RP, N, N, l.sp_g, part, s));
    QLORA_TRY(launch_reduce_rows(part, l.sp_g.splits, M, RP, r, a.s, nullptr, Gb, Gt, l.Mp, s));
  }
  // dB = dY^T sH and dA = G^T X: one launch of split partials (before the
  // dX launch, so a split dX launch's reduction can share the launch of
  // their fixed-order reductions)
  float *part_b = part, *part_a = reinterpret_cast<float *>(base + l.part_off + l.parta_off);
  QLORA_TRY(launch_tn_pair(TnProblem{dY, N, sHt, l.Mp, l.sp_b, true, part_b},
                           TnProblem{X, K, Gt, l.Mp, l.sp_a, false, part_a}, M, RP, s));
  SmallJob red[3] = {job_reduce_cols(part_b, l.sp_b.splits, N, RP, r, true, dB),
                     job_reduce_cols(part_a, l.sp_a.splits, K, RP, r, false, dA), SmallJob{}};
  if (dX != nullptr) {
    if (tiles) {
      QLORA_TRY(launch_bwd_dx_tiles(a.w, scales, dY, M, At, RP, Gb, dX,
                                    reinterpret_cast<float *>(base + l.tpart_off), s, &red[2]));
    } else {  // ragged n: the general 128 x 128 kernel
      const dim3 grid((unsigned)ceil_div(K, DBK), (unsigned)ceil_div(M, DBM));
      QLORA_LAUNCH("k_bwd_dx", k_bwd_dx, grid, dim3(256), 0, s, a.w, dY, M, At, Gb, RP, dX);
    }
    QLORA_TRY(hipGetLastError());
  }
  QLORA_TRY(launch_jobs("k_reduce_grads", red, 3, s));
#undef QLORA_TRY
  return hipSuccess;
}

}  // namespace qlora

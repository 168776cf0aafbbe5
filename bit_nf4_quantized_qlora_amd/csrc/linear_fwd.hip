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

constexpr int FBN = 256, FBM = 256;  // block tile: weight rows (n) x X rows (m)

// C[n][m] = sum_k W_hat[n][k] X[m][k] + sum_j B[n][j] sH[m][j]  ->  Y[m][n]
// Wave w owns weight rows n0 + 64w .. +63 (four 16-row MFMA tiles) and all
// 256 X rows (sixteen 16-column tiles): 256 fp32 accumulators per lane.
// Its NF4 rows are expanded straight into MFMA A-operand registers: lane
// (li = lane & 15, g = lane >> 4) of row tile rt holds row n0+64w+16rt+li and
// codes 16g .. 16g+15 of the current 64-weight block (one 8-byte load), used
// as contraction slots 8t .. 8t+7 of sub-step t; the X fragment reads the
// same k positions, so the contraction is unchanged.
//
// Per 64-wide K step: the X tile of step kt+1 streams global -> LDS with
// buffer loads (no registers) into the other of two separate LDS arrays
// (separate objects, so the compiler knows the in-flight copy does not alias
// the tile being read), the packed codes of step kt+2 are loaded, and the
// codes of step kt+1 are expanded in eight pieces interleaved with the eight
// groups of 16 MFMAs of step kt.  Rows past N or M are clamped to a valid
// row: they only feed accumulators that are never stored.
// All per-lane addresses are one 32-bit VGPR offset into a buffer resource
// plus uniform (scalar) offsets; rows past N or M fall outside the resource's
// range and read as zero, and only feed accumulators that are never stored.
//
// Pipeline (per 64-wide K step kt, the loop unrolled by 4 so every buffer
// index is a compile-time constant):
//   X tile of step kt+2  -> LDS buffer (kt+2) % 4 by buffer_load ... lds
//   codes of step kt+3   -> registers (three code sets rotate)
//   codes of step kt+1   -> expanded into next-step operands, in 8 pieces;
//                           a piece's LDS table reads are issued one MFMA
//                           group before the arithmetic that uses them
//   MFMAs of step kt     on LDS buffer kt % 4 and the current operands
// The step ends waiting only for the loads issued one step earlier.
template <int kTail>  // (k/64) % 4: steps after the unrolled loop
__global__ __launch_bounds__(256, 1) void k_fwd_nf4(Nf4View w, const uint16_t *__restrict__ X, int64_t M,
                                                    const uint16_t *__restrict__ Bl, int r, int RP,
                                                    const uint16_t *__restrict__ sH, uint16_t *__restrict__ Y,
                                                    int tiles_n) {
  __shared__ __align__(16) uint16_t Xs0[FBM * 64];
  __shared__ __align__(16) uint16_t Xs1[FBM * 64];
  __shared__ __align__(16) uint16_t Xs2[FBM * 64];
  __shared__ __align__(16) uint16_t Xs3[FBM * 64];
  __shared__ float2 s_pair[256];
  // wave is uniform across the wave; say so, or wave-dependent scalar
  // offsets would be made uniform with a per-lane loop
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t n0 = (int64_t)(tile % tiles_n) * FBN, m0 = (int64_t)(tile / tiles_n) * FBM;
  const int64_t N = w.n, K = w.k, nk = K / kBlock;
  fill_pair_table(s_pair, tid, 256);
  const float offset = *w.offset;
  auto xbuf = [&](auto B) -> uint16_t * {
    constexpr int b = decltype(B)::value & 3;
    return b == 0 ? Xs0 : b == 1 ? Xs1 : b == 2 ? Xs2 : Xs3;
  };

  // Weight rows n0 .. n0+255: lane's row in row tile rt is n0 + 64w + 16rt + li.
  const int64_t nrows = min<int64_t>(FBN, N - n0);
  const __amdgpu_buffer_rsrc_t wrs = rsrc(w.packed + n0 * (K / 2), nrows * (K / 2));
  const __amdgpu_buffer_rsrc_t srs = rsrc(w.scale_code + n0 * nk, nrows * nk);
  const __amdgpu_buffer_rsrc_t grs = rsrc(w.group_amax, ceil_div_d(w.nb, kGroup) * 4);
  const uint32_t wv = (uint32_t)(li * (K / 2) + 8 * g), sv = (uint32_t)(li * nk);
  const int64_t wrow_w = 64 * wave;  // wave's first row within the tile
  // X rows m0 .. m0+255, staged global -> LDS: wave-instruction i fills LDS
  // chunks [512w + 64i, +64): row 64w + 8i + lane/8, logical chunk
  // (lane & 7) ^ ((lane/8) & 7) (the swizzle of xsw), so only the row term
  // varies with i and it is uniform.
  const int64_t xrows = min<int64_t>(FBM, M - m0);
  const __amdgpu_buffer_rsrc_t xrs = rsrc(X + m0 * K, xrows * K * 2);
  const uint32_t xv = (uint32_t)(((lane >> 3) * K + 8 * ((lane & 7) ^ ((lane >> 3) & 7))) * 2);
  auto xload = [&](int64_t kt, auto B) {
    uint16_t *dst = xbuf(B);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_ptr)(dst + (512 * wave + 64 * i) * 8), 16, xv,
                                               (int)((64 * wave + 8 * i) * K * 2 + kt * 128), 0, 0);
  };
  constexpr int kVmemPerStep = 8 + 12;  // X copy + codes, scale codes, group constants

  // Code sets, indexed by step mod 4 (compile-time in the unrolled loop, so
  // nothing is copied while its load is in flight): during step kt the set of
  // step kt+1 is expanded and the set of step kt+3 is loaded.
  struct Codes {
    u32x2_t wc[4];
    uint32_t sc[4];
    float ga[4];
  };
  Codes c[4];
  auto wload = [&](int64_t kt, Codes &d) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int64_t row = wrow_w + 16 * rt;  // uniform part of the lane's row
      d.wc[rt] = __builtin_amdgcn_raw_buffer_load_b64(wrs, wv, (int)(row * (K / 2) + kt * 32), 0);
      d.sc[rt] = __builtin_amdgcn_raw_buffer_load_b8(srs, sv, (int)(row * nk + kt), 0);
      const uint32_t gidx = (uint32_t)(((n0 + row) * nk + kt + sv) >> 8);
      d.ga[rt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(grs, gidx * 4, 0, 0));
    }
  };
  // a[rt][t]: operands of the current step.  Piece p of the next step's
  // expansion: p < 4 -> row tile p, sub-step 1 into an[p] (a[][1] is still
  // in use); p >= 4 -> row tile p-4, sub-step 0 straight into a[p-4][0]
  // (written in MFMA groups 9..15, after its last read in group 7).
  u32x4_t a[4][2], an[4];
  float sn[4];
  float2 pq[4];  // table reads of the piece in flight
  auto piece_read = [&](const Codes &cs, int p) {
    const int rt = p & 3, t = p < 4 ? 1 : 0;
    const uint32_t word = cs.wc[rt][t];
#pragma unroll
    for (int i = 0; i < 4; ++i) pq[i] = s_pair[(word >> (8 * i)) & 0xFFu];
  };
  auto piece_math = [&](const Codes &cs, int p) {
    const int rt = p & 3;
    if (p < 4) sn[rt] = block_scale(cs.sc[rt], cs.ga[rt], offset);
    const float s = sn[rt];
    const u32x4_t v = {bf16x2_rne(__fmul_rn(pq[0].x, s), __fmul_rn(pq[0].y, s)),
                       bf16x2_rne(__fmul_rn(pq[1].x, s), __fmul_rn(pq[1].y, s)),
                       bf16x2_rne(__fmul_rn(pq[2].x, s), __fmul_rn(pq[2].y, s)),
                       bf16x2_rne(__fmul_rn(pq[3].x, s), __fmul_rn(pq[3].y, s))};
    if (p < 4) an[rt] = v;
    else a[rt][0] = v;
  };

  f32x4_t acc[4][16];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Prologue: X of steps 0 and 1 in flight, step 0 expanded, codes of 1..3.
  __syncthreads();  // pair table
  xload(0, std::integral_constant<int, 0>());
  xload(min<int64_t>(1, nk - 1), std::integral_constant<int, 1>());
  wload(0, c[0]);
  wload(min<int64_t>(1, nk - 1), c[1]);
  wload(min<int64_t>(2, nk - 1), c[2]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    piece_read(c[0], p);
    piece_math(c[0], p);
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) a[rt][1] = an[rt];
  __syncthreads();

  auto step = [&](int64_t kt, auto B) {
    constexpr int buf = decltype(B)::value & 3;
    // Prefetches past the last step re-read the last step (in bounds, unused).
    xload(min<int64_t>(kt + 2, nk - 1), std::integral_constant<int, (buf + 2) & 3>());
    wload(min<int64_t>(kt + 3, nk - 1), c[(buf + 3) & 3]);
    const Codes &cn = c[(buf + 1) & 3];  // step kt+1
    // Fragment (column tile ct, sub-step t) sits at xrow[t] + 1024*ct: the
    // swizzle term depends on (row & 7) == (li & 7) only.
    const uint16_t *xs = xbuf(B);
    const uint16_t *xrow0 = xs + xsw(li, 2 * g), *xrow1 = xs + xsw(li, 2 * g + 1);
    u32x4_t bq[2][2];
    bq[0][0] = *reinterpret_cast<const u32x4_t *>(xrow0);
    bq[0][1] = *reinterpret_cast<const u32x4_t *>(xrow0 + 1024);
#pragma unroll
    for (int q = 0; q < 16; ++q) {  // group q: sub-step t = q/8, column tiles 2(q%8), +1
      const int t = q >> 3, ct0 = 2 * (q & 7);
      if (q < 15) {
        const int t1 = (q + 1) >> 3, c1 = 2 * ((q + 1) & 7);
        const uint16_t *xr = t1 ? xrow1 : xrow0;
        bq[(q + 1) & 1][0] = *reinterpret_cast<const u32x4_t *>(xr + 1024 * c1);
        bq[(q + 1) & 1][1] = *reinterpret_cast<const u32x4_t *>(xr + 1024 * (c1 + 1));
      }
      if ((q & 1) == 0) piece_read(cn, q >> 1);  // consumed by the next group
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) mfma16_acc(acc[rt][ct0 + cc], a[rt][t], bq[q & 1][cc]);
      if ((q & 1) == 1) piece_math(cn, q >> 1);  // (on the last step: codes that are never used)
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) a[rt][1] = an[rt];
    // Everything but this step's own loads has landed (X of step kt+1, codes
    // of kt+2), then a bare barrier: the only LDS writes in the loop are
    // those copies, so __syncthreads()'s release fence would merely wait for
    // the copies still in flight for step kt+2.  A buffer is refilled two
    // barriers after its last read.
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kVmemPerStep) : "memory");
  };
  const int64_t nquads = nk >> 2;
  for (int64_t p = 0; p < nquads; ++p) {
    step(4 * p, std::integral_constant<int, 0>());
    step(4 * p + 1, std::integral_constant<int, 1>());
    step(4 * p + 2, std::integral_constant<int, 2>());
    step(4 * p + 3, std::integral_constant<int, 3>());
  }
  if constexpr (kTail >= 1) step(nk - kTail, std::integral_constant<int, 0>());
  if constexpr (kTail >= 2) step(nk - kTail + 1, std::integral_constant<int, 1>());
  if constexpr (kTail >= 3) step(nk - kTail + 2, std::integral_constant<int, 2>());
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // LoRA up-projection in 64-wide chunks of the padded rank: the same
  // fragment layout with A = B_lora rows (direct loads) and the sH tile in LDS.
  const bool bvec = (r % 8) == 0;
  for (int jc = 0; jc < RP; jc += 64) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<u32x4_t *>(&Xs0[xsw(c >> 3, c & 7)]) =
          load8(sH, RP, M, RP, m0 + (c >> 3), jc + 8 * (c & 7), true);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        a[rt][t] = load8(Bl, r, N, r, n0 + 64 * wave + 16 * rt + li, jc + 16 * g + 8 * t, bvec);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ct = 0; ct < 16; ++ct) {
        const u32x4_t b = *reinterpret_cast<const u32x4_t *>(&Xs0[xsw(16 * ct + li, 2 * g + t)]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) mfma16_acc(acc[rt][ct], a[rt][t], b);
      }
    __syncthreads();
  }
  mfma_acc_fence();

  // acc[rt][ct][v] = C[n][m]: n = n0+64w+16rt+4g+v, m = m0+16ct+li (four consecutive n of one Y row).
  const bool nvec = (N & 3) == 0;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) {
      const int64_t n = n0 + 64 * wave + 16 * rt + 4 * g;
      const int64_t m = m0 + 16 * ct + li;
      if (m < M) {
        const f32x4_t v = acc[rt][ct];
        uint16_t *dst = Y + m * N + n;
        if (nvec && n + 4 <= N) {
          *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3])};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) dst[e] = f32_to_bf16_bits(v[e]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
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
  const int tiles_n = (int)ceil_div(N, FBN), tiles_m = (int)ceil_div(M, FBM);
  const dim3 grid((unsigned)(tiles_n * tiles_m));
  switch ((K / kBlock) & 3) {
    case 0: QLORA_LAUNCH("k_fwd_nf4", k_fwd_nf4<0>, grid, dim3(256), 0, s, a.w, X, M, B, a.r, l.RP, sH, Y, tiles_n); break;
    case 1: QLORA_LAUNCH("k_fwd_nf4", k_fwd_nf4<1>, grid, dim3(256), 0, s, a.w, X, M, B, a.r, l.RP, sH, Y, tiles_n); break;
    case 2: QLORA_LAUNCH("k_fwd_nf4", k_fwd_nf4<2>, grid, dim3(256), 0, s, a.w, X, M, B, a.r, l.RP, sH, Y, tiles_n); break;
    default: QLORA_LAUNCH("k_fwd_nf4", k_fwd_nf4<3>, grid, dim3(256), 0, s, a.w, X, M, B, a.r, l.RP, sH, Y, tiles_n); break;
  }
  return hipGetLastError();
}

}  // namespace qlora

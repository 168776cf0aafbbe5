// linear_bwd.hip -- backward pass of the frozen NF4 linear layer with LoRA.
//
// "QLoRA Paper Breakdown" sec. 4: the input gradient needs the NF4 weights
// dequantized again on the fly, and dL/dW is never materialized; "QLoRA,
// explained." step 5: gradients reach the adapters only.  With
// Y = X W_hat^T + s (X A^T) B^T:
//   G  = s dY B            (k_nt_splitk on dY and B^T)
//   dX = dY W_hat + G A    (k_bwd_dx, below)
//   dB = s dY^T H          (k_tn_splitk on dY and (sH)^T)
//   dA = G^T X             (k_tn_splitk on X and G^T)
//
// k_bwd_dx contracts over n, the row index of W, so the dequantized tile is
// laid into LDS transposed: each thread expands one packed dword (8 codes
// along k) from each of 4 consecutive rows n, transposes the 4x8 block in
// registers with byte permutes and writes eight 8-byte runs of [k][n].  The
// output tile is computed as C[k][m] so a lane's four accumulators are four
// consecutive k of one dX row.
#include "lora_gemm.h"

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
  fill_pair_table(s_pair, tid, 256);
  const float offset = *w.offset;
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
      sc[rho] = w.scale_code[b];
      ga[rho] = w.group_amax[b >> 8];
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
      dequant_word(wd[rho], block_scale(sc[rho], ga[rho], offset), s_pair, o[rho]);
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

// ---------------------------------------------------------------------------
// k_bwd_dx_nf4: the same product on 256 (k) x 256 (m) tiles, for n % 64 == 0.
// Wave w owns dX columns k0 + 64w .. +63 (four 16-row MFMA tiles of C[k][m])
// and all 256 m: 256 fp32 accumulators per lane, pinned to AGPRs.  Per
// 64-wide step over n:
//   * the dY tile [256 m][64 n] streams global -> LDS by buffer loads into
//     the other of two LDS arrays (the B operand, as X is in the forward);
//   * each thread expands an 8-row x 8-column block of codes (rows n, one
//     packed dword per row), transposes it with byte permutes and writes
//     eight 16-byte runs of W_hat^T [256 k][64 n] (the A operand) into the
//     other of two LDS arrays; the 256 block scales of a step are computed
//     once (one per thread) and shared through a small LDS table.
// Expansion of step s+1 is interleaved with the MFMA groups of step s.
// Lane (li, g) reads contraction slots 16g .. 16g+15 of the step (sub-step t:
// 16g + 8t .. +7) from both operands.
template <bool kOddSteps>
__global__ __launch_bounds__(256, 1) void k_bwd_dx_nf4(Nf4View w, const uint16_t *__restrict__ dY, int64_t M,
                                                       const uint16_t *__restrict__ At,
                                                       const uint16_t *__restrict__ Gb, int RP,
                                                       uint16_t *__restrict__ dX, int tiles_k) {
  __shared__ __align__(16) uint16_t Ds0[256 * 64];
  __shared__ __align__(16) uint16_t Ds1[256 * 64];
  __shared__ __align__(16) uint16_t Ws0[256 * 64];
  __shared__ __align__(16) uint16_t Ws1[256 * 64];
  __shared__ __align__(16) float Ss0[4 * 64];  // block scales of a step, [k-block][n]
  __shared__ __align__(16) float Ss1[4 * 64];
  __shared__ float2 s_pair[256];
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t k0 = (int64_t)(tile % tiles_k) * 256, m0 = (int64_t)(tile / tiles_k) * 256;
  const int64_t N = w.n, K = w.k, nkb = K / kBlock, nsteps = N / 64;
  fill_pair_table(s_pair, tid, 256);
  const float offset = *w.offset;

  // dY rows m0 .. m0+255 (buffer range ends at row M; the row offset is in
  // the range-checked per-lane offset, so rows past M read 0).
  const int64_t yrows = min<int64_t>(256, M - m0);
  const __amdgpu_buffer_rsrc_t yrs = rsrc(dY + m0 * N, yrows * N * 2);
  const uint32_t yv = (uint32_t)(((64 * wave + (lane >> 3)) * N + 8 * ((lane & 7) ^ ((lane >> 3) & 7))) * 2);
  auto yload = [&](int64_t st, auto BUF) {
    uint16_t *dst = decltype(BUF)::value ? Ds1 : Ds0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(yrs, (lds_ptr)(dst + (512 * wave + 64 * i) * 8), 16,
                                               yv + (uint32_t)(i * 16 * N), (int)(st * 128), 0, 0);
  };
  // Codes: thread (ng = tid >> 5, kg = tid & 31) covers rows 8ng .. 8ng+7 of
  // the step and columns k0 + 8kg .. +7 (one dword per row; columns past K
  // only feed rows of C that are never stored, and past the last row they
  // fall outside the range-checked offset and read 0).
  const int ng = tid >> 5, kg = tid & 31;
  const __amdgpu_buffer_rsrc_t wrs = rsrc(w.packed, w.n * (K / 2));
  const uint32_t wv = (uint32_t)(8 * ng * (K / 2) + (k0 + 8 * kg) / 2);
  // Scales: thread t computes the scale of step-row t >> 2, k-block t & 3.
  const int srow = tid >> 2, sblk = tid & 3;
  const int64_t sb_kb = min<int64_t>(k0 / kBlock + sblk, nkb - 1);
  const __amdgpu_buffer_rsrc_t srs = rsrc(w.scale_code, w.nb);
  const __amdgpu_buffer_rsrc_t grs = rsrc(w.group_amax, ceil_div_d(w.nb, kGroup) * 4);

  uint32_t wa[8], wb[8];
  uint32_t scb = 0;
  float gab = 0.f;
  auto wload = [&](int64_t st, uint32_t(&wc)[8]) {
#pragma unroll
    for (int rho = 0; rho < 8; ++rho)
      wc[rho] = __builtin_amdgcn_raw_buffer_load_b32(wrs, wv + (uint32_t)((st * 64 + rho) * (K / 2)), 0, 0);
  };
  auto sload = [&](int64_t st) {
    const int64_t b = (st * 64 + srow) * nkb + sb_kb;
    scb = __builtin_amdgcn_raw_buffer_load_b8(srs, (uint32_t)b, 0, 0);
    gab = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(grs, (uint32_t)((b >> 8) * 4), 0, 0));
  };
  auto sstore = [&](float *S) { S[sblk * 64 + srow] = block_scale(scb, gab, offset); };

  // Expansion of one step's codes (wa) into W_hat^T, in 8 pieces: pieces
  // 0-3 expand rows 2p, 2p+1; pieces 4-7 transpose and write columns
  // 2(p-4), 2(p-4)+1.
  uint32_t ex[8][4];
  float sx[8];
  auto expand_piece = [&](int p, const float *S, uint16_t *Wd) {
    if (p == 0) {
      const f32x4_t s0 = *reinterpret_cast<const f32x4_t *>(&S[(kg >> 3) * 64 + 8 * ng]);
      const f32x4_t s1 = *reinterpret_cast<const f32x4_t *>(&S[(kg >> 3) * 64 + 8 * ng + 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sx[i] = s0[i], sx[4 + i] = s1[i];
    }
    if (p < 4) {
      dequant_word(wa[2 * p], sx[2 * p], s_pair, ex[2 * p]);
      dequant_word(wa[2 * p + 1], sx[2 * p + 1], s_pair, ex[2 * p + 1]);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kc = 2 * (p - 4) + h, d = kc >> 1;
        u32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = (kc & 1) ? pack_hi(ex[2 * e][d], ex[2 * e + 1][d]) : pack_lo(ex[2 * e][d], ex[2 * e + 1][d]);
        *reinterpret_cast<u32x4_t *>(&Wd[xsw(8 * kg + kc, ng)]) = v;
      }
    }
  };

  f32x4_t acc[4][16];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Prologue: scales of steps 0 and 1, expanded step 0, codes of step 1.
  __syncthreads();  // pair table
  sload(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  sstore(Ss0);
  sload(min<int64_t>(1, nsteps - 1));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  sstore(Ss1);
  wload(0, wa);
  yload(0, std::integral_constant<int, 0>());
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 8; ++p) expand_piece(p, Ss0, Ws0);
  wload(min<int64_t>(1, nsteps - 1), wa);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  auto step = [&](int64_t st, auto BUF) {
    constexpr int buf = decltype(BUF)::value;
    const uint16_t *Ws = buf ? Ws1 : Ws0;
    const uint16_t *Ds = buf ? Ds1 : Ds0;
    uint16_t *Wn = buf ? Ws0 : Ws1;
    const float *Sn = buf ? Ss0 : Ss1;  // scales of step st+1
    float *Sf = buf ? Ss1 : Ss0;        // slot for step st+2's scales
    yload(min<int64_t>(st + 1, nsteps - 1), std::integral_constant<int, buf ^ 1>());
    wload(min<int64_t>(st + 2, nsteps - 1), wb);
    sload(min<int64_t>(st + 2, nsteps - 1));
    const uint16_t *d0 = Ds + xsw(li, 2 * g), *d1 = Ds + xsw(li, 2 * g + 1);
    u32x4_t a[4], bq[2][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) a[rt] = *reinterpret_cast<const u32x4_t *>(&Ws[xsw(64 * wave + 16 * rt + li, 2 * g)]);
    bq[0][0] = *reinterpret_cast<const u32x4_t *>(d0);
    bq[0][1] = *reinterpret_cast<const u32x4_t *>(d0 + 1024);
#pragma unroll
    for (int q = 0; q < 16; ++q) {  // group q: sub-step t = q/8, column tiles 2(q%8), +1
      const int ct0 = 2 * (q & 7);
      if (q == 8) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          a[rt] = *reinterpret_cast<const u32x4_t *>(&Ws[xsw(64 * wave + 16 * rt + li, 2 * g + 1)]);
      }
      if (q < 15) {
        const int t1 = (q + 1) >> 3, c1 = 2 * ((q + 1) & 7);
        const uint16_t *dr = t1 ? d1 : d0;
        bq[(q + 1) & 1][0] = *reinterpret_cast<const u32x4_t *>(dr + 1024 * c1);
        bq[(q + 1) & 1][1] = *reinterpret_cast<const u32x4_t *>(dr + 1024 * (c1 + 1));
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) mfma16_acc(acc[rt][ct0 + c], a[rt], bq[q & 1][c]);
      if ((q & 1) == 1) expand_piece(q >> 1, Sn, Wn);  // step st+1 (stale codes on the last step)
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    sstore(Sf);
#pragma unroll
    for (int rho = 0; rho < 8; ++rho) wa[rho] = wb[rho];
    __syncthreads();
  };
  const int64_t npairs = nsteps >> 1;
  for (int64_t p = 0; p < npairs; ++p) {
    step(2 * p, std::integral_constant<int, 0>());
    step(2 * p + 1, std::integral_constant<int, 1>());
  }
  if constexpr (kOddSteps) step(nsteps - 1, std::integral_constant<int, 0>());

  // LoRA term: acc += A^T[k][:] . G[m][:] over the padded rank, in 64-wide
  // chunks (A operand: rows of A^T straight from global; G tile in LDS).
  for (int jc = 0; jc < RP; jc += 64) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<u32x4_t *>(&Ds0[xsw(c >> 3, c & 7)]) =
          load8(Gb, RP, M, RP, m0 + (c >> 3), jc + 8 * (c & 7), true);
    }
    u32x4_t a[4][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int t = 0; t < 2; ++t) a[rt][t] = load8(At, RP, K, RP, k0 + 64 * wave + 16 * rt + li, jc + 16 * g + 8 * t, true);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ct = 0; ct < 16; ++ct) {
        const u32x4_t b = *reinterpret_cast<const u32x4_t *>(&Ds0[xsw(16 * ct + li, 2 * g + t)]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) mfma16_acc(acc[rt][ct], a[rt][t], b);
      }
    __syncthreads();
  }
  mfma_acc_fence();

  // acc[rt][ct][v] = C[k][m]: k = k0+64w+16rt+4g+v, m = m0+16ct+li -> dX[m][k..k+3].
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) {
      const int64_t k = k0 + 64 * wave + 16 * rt + 4 * g;
      const int64_t m = m0 + 16 * ct + li;
      if (m < M && k < K) {
        const f32x4_t v = acc[rt][ct];
        *reinterpret_cast<u32x2_t *>(dX + m * K + k) = u32x2_t{bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3])};
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

struct BwdWs {
  int RP;
  int64_t Mp;
  SplitPlan sp_h, sp_g, sp_b, sp_a;
  size_t part_off, h_off, sht_off, bt_off, at_off, gb_off, gt_off, total;
};

BwdWs bwd_ws_layout(int64_t M, int64_t N, int64_t K, int r) {
  BwdWs l;
  l.RP = lora_rank_pad(r);
  l.Mp = ceil_div(M, 64) * 64;
  l.sp_h = plan_split(ceil_div(M, 64), ceil_div(K, 64));
  l.sp_g = plan_split(ceil_div(M, 64), ceil_div(N, 64));
  l.sp_b = plan_split(ceil_div(N, 64), ceil_div(M, 64));
  l.sp_a = plan_split(ceil_div(K, 64), ceil_div(M, 64));
  size_t part = std::max({(size_t)l.sp_h.splits * M * l.RP, (size_t)l.sp_g.splits * M * l.RP,
                          (size_t)l.sp_b.splits * l.RP * N, (size_t)l.sp_a.splits * l.RP * K}) *
                sizeof(float);
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
  QLORA_TRY(launch_scale_transpose_f32(H, M, r, a.s, sHt, RP, l.Mp, s));
  QLORA_TRY(launch_transpose_pad(B, N, r, Bt, RP, N, s));  // Bt [RP][N]
  QLORA_TRY(launch_transpose_pad(A, r, K, At, K, RP, s));  // At [K][RP]
  // G = s dY B -> Gb [M][RP], Gt [RP][Mp]
  QLORA_TRY(launch_nt_splitk(dY, M, Bt, RP, RP, N, N, l.sp_g, part, s));
  QLORA_TRY(launch_reduce_rows(part, l.sp_g.splits, M, RP, r, a.s, nullptr, Gb, Gt, l.Mp, s));
  if (dX != nullptr) {
    // whole-tensor code offsets stay 32-bit below 2^31 bytes
    if (N % 64 == 0 && N * (K / 2) < (int64_t(1) << 31)) {
      const int tiles_k = (int)ceil_div(K, 256), tiles_m = (int)ceil_div(M, 256);
      const dim3 grid((unsigned)(tiles_k * tiles_m));
      if ((N / 64) & 1)
        QLORA_LAUNCH("k_bwd_dx_nf4", k_bwd_dx_nf4<true>, grid, dim3(256), 0, s, a.w, dY, M, At, Gb, RP, dX, tiles_k);
      else
        QLORA_LAUNCH("k_bwd_dx_nf4", k_bwd_dx_nf4<false>, grid, dim3(256), 0, s, a.w, dY, M, At, Gb, RP, dX, tiles_k);
    } else {  // ragged n: the general 128 x 128 kernel
      const dim3 grid((unsigned)ceil_div(K, DBK), (unsigned)ceil_div(M, DBM));
      QLORA_LAUNCH("k_bwd_dx", k_bwd_dx, grid, dim3(256), 0, s, a.w, dY, M, At, Gb, RP, dX);
    }
    QLORA_TRY(hipGetLastError());
  }
  QLORA_TRY(launch_tn_splitk(dY, M, N, sHt, l.Mp, RP, l.sp_b, part, s));
  QLORA_TRY(launch_reduce_cols(part, l.sp_b.splits, N, RP, r, true, dB, s));
  QLORA_TRY(launch_tn_splitk(X, M, K, Gt, l.Mp, RP, l.sp_a, part, s));
  QLORA_TRY(launch_reduce_cols(part, l.sp_a.splits, K, RP, r, false, dA, s));
#undef QLORA_TRY
  return hipSuccess;
}

}  // namespace qlora

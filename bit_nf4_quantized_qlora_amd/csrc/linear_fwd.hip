// linear_fwd.hip -- forward pass of the frozen NF4 linear layer with LoRA.
//
// "QLoRA Paper Breakdown" sec. 4 Forward Pass: Y = X dequant(W)^T +
// (alpha/r) X L_1 L_2, with the weights expanded from NF4 to BF16 on every
// use ("QLoRA, explained." step 4; "reading note": the multiply runs in 16
// bits).
//
//   1. H = X A^T (k_nt_splitk + reduction): fp32 H (optional output) and
//      bf16(s*H) for the epilogue.
//   2. k_tile_scales: s_b of every block, once per call, in the order the
//      main kernel streams them (k % 256 == 0).
//   3. k_fwd_nf4 (k % 256 == 0) or k_fwd_nf4_any (any k % 64 == 0):
//      C[n][m] = sum_k W_hat[n][k] X[m][k] + sum_j B[n][j] sH[m][j] on
//      256x256 tiles.  NF4 codes are expanded in registers straight into MFMA
//      operands through a 256-entry table of level pairs, bit-identical to
//      the standalone dequantization; the LoRA up-projection is a few more
//      MFMA steps on the same accumulators; Y is rounded to bf16 once.
#include "lora_gemm.h"

namespace qlora {
namespace {

constexpr int FBN = 256, FBM = 256;  // block tile: weight rows (n) x X rows (m)

// Shared tail of both forward kernels, after the main loop has drained
// (every copy landed, all waves past a barrier): the LoRA up-projection in
// 64-wide chunks of the padded rank -- the same fragment layout with
// A = B_lora rows (direct loads) and the sH tile staged in LDS (stage: 32 KB)
// -- then Y.  acc[rt][ct][v] = C[n][m] with n = nw + 16rt + 4g + v and
// m = m0 + 16ct + li (four consecutive n of one Y row).
__device__ __forceinline__ void fwd_epilogue(f32x4_t (&acc)[4][16], uint16_t *stage, const uint16_t *__restrict__ Bl,
                                             int r, int RP, const uint16_t *__restrict__ sH,
                                             uint16_t *__restrict__ Y, int64_t N, int64_t M, int64_t nw,
                                             int64_t m0) {
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const bool bvec = (r % 8) == 0;
  for (int jc = 0; jc < RP; jc += 64) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<u32x4_t *>(&stage[xsw(c >> 3, c & 7)]) =
          load8(sH, RP, M, RP, m0 + (c >> 3), jc + 8 * (c & 7), true);
    }
    u32x4_t a[4][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int t = 0; t < 2; ++t) a[rt][t] = load8(Bl, r, N, r, nw + 16 * rt + li, jc + 16 * g + 8 * t, bvec);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ct = 0; ct < 16; ++ct) {
        const u32x4_t b = *reinterpret_cast<const u32x4_t *>(&stage[xsw(16 * ct + li, 2 * g + t)]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) mfma16_acc(acc[rt][ct], a[rt][t], b);
      }
    __syncthreads();
  }
  mfma_acc_fence();

  const bool nvec = (N & 3) == 0;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) {
      const int64_t n = nw + 16 * rt + 4 * g;
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
__global__ __launch_bounds__(256, 1) void k_fwd_nf4_any(Nf4View w, const uint16_t *__restrict__ X, int64_t M,
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

  fwd_epilogue(acc, Xs0, Bl, r, RP, sH, Y, N, M, n0 + 64 * wave, m0);
}

constexpr int kSup = 4;  // K steps per staged weight chunk: 128 packed bytes per row

// s_b of every block, in the order k_fwd_nf4 streams them: for weight tile tn
// (rows 256tn .. 256tn+255) and super-step sp (blocks 4sp .. 4sp+3 of each
// row) one contiguous 4 KB run, Sp[((tn*nsup + sp)*256 + row)*4 + j]; rows
// past n hold 0.  block_scale is the dequantization's own (bit-identical).
__global__ __launch_bounds__(256) void k_tile_scales(Nf4View w, int64_t nsup, int64_t total,
                                                     float *__restrict__ Sp) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t q = t >> 8, tn = q / nsup, sp = q - tn * nsup;
  const int64_t n = tn * FBN + (t & 255);
  f32x4_t v = {0.f, 0.f, 0.f, 0.f};
  if (n < w.n) {
    const int64_t b = n * (nsup * kSup) + kSup * sp;  // 4 blocks in one group (256 % 4 == 0)
    const uint32_t c4 = *reinterpret_cast<const uint32_t *>(w.scale_code + b);
    const float ga = w.group_amax[b / kGroup], off = *w.offset;
#pragma unroll
    for (int j = 0; j < kSup; ++j) v[j] = block_scale((c4 >> (8 * j)) & 0xFFu, ga, off);
  }
  *reinterpret_cast<f32x4_t *>(Sp + 4 * t) = v;
}

// The forward for k % 256 == 0, with every operand streamed by LDS DMA.
// Same tiles, wave roles, fragment layout and expansion as k_fwd_nf4_any;
// the weight side differs: packed codes arrive 4 K steps (128 B = one cache
// line per row) at a time, with their precomputed block scales (k_tile_scales),
// straight into LDS, and each lane reads its 8-byte code chunks and scales
// from there.  (Per-step scattered loads of codes, scale codes and group
// constants from every lane were the kernel's main stall.)
//
// LDS: X tiles Xs0/Xs1 (2 x 32 KB), code tiles Wc0/Wc1 (2 x 32 KB: 256 rows x
// 128 B, 16-byte chunk c of row R at chunk c ^ (R & 7)), scale tiles Sc0/Sc1
// (2 x 4 KB: 256 rows x 4 fp32), pair table 2 KB.  Wave w copies and reads
// only its own 64 weight rows.
//
// Per K step kt (u = kt % 8, j = kt % 4, super-step sp = kt / 4; the loop is
// unrolled by 8 so every buffer choice is a compile-time constant):
//   X tile of step kt+1        -> Xs[(kt+1) % 2]         (DMA)
//   if j == 0: codes + scales of super-step sp+1 -> Wc/Sc[(sp+1) % 2] (DMA)
//   16 MFMA groups of step kt on Xs[kt % 2], interleaved with the expansion
//   of step kt+1 from the code/scale registers
//   LDS -> registers: codes and scales of step kt+2
//   wait for this step's X copy (and, from j == 1, the weight copy), barrier
// A weight buffer is refilled one step after its last register read; its
// copy has until the end of step 4sp+1, and is first read at the end of
// step 4sp+2.
template <int kOddSup>  // (k/256) odd: one 4-step super-step after the 8-step loop
__global__ __launch_bounds__(256, 1) void k_fwd_nf4(Nf4View w, const float *__restrict__ Sp,
                                                    const uint16_t *__restrict__ X, int64_t M,
                                                    const uint16_t *__restrict__ Bl, int r, int RP,
                                                    const uint16_t *__restrict__ sH, uint16_t *__restrict__ Y,
                                                    int tiles_n) {
  __shared__ __align__(16) uint16_t Xs0[FBM * 64];
  __shared__ __align__(16) uint16_t Xs1[FBM * 64];
  __shared__ __align__(16) uint8_t Wc0[FBN * 128];
  __shared__ __align__(16) uint8_t Wc1[FBN * 128];
  __shared__ __align__(16) float Sc0[FBN * kSup];
  __shared__ __align__(16) float Sc1[FBN * kSup];
  __shared__ float2 s_pair[256];
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int tn = tile % tiles_n;
  const int64_t n0 = (int64_t)tn * FBN, m0 = (int64_t)(tile / tiles_n) * FBM;
  const int64_t N = w.n, K = w.k, nk = K / kBlock, nsup = nk / kSup;
  fill_pair_table(s_pair, tid, 256);

  // X rows m0 .. m0+255: wave-instruction i fills LDS chunks [512w + 64i,
  // +64): row 64w + 8i + lane/8, logical chunk (lane & 7) ^ ((lane/8) & 7)
  // (the swizzle of xsw); rows past M read as zero.
  const int64_t xrows = min<int64_t>(FBM, M - m0);
  const __amdgpu_buffer_rsrc_t xrs = rsrc(X + m0 * K, xrows * K * 2);
  const uint32_t xv = (uint32_t)(((lane >> 3) * K + 8 * ((lane & 7) ^ ((lane >> 3) & 7))) * 2);
  auto xload = [&](int64_t kt, auto B) {
    uint16_t *dst = decltype(B)::value ? Xs1 : Xs0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_ptr)(dst + (512 * wave + 64 * i) * 8), 16, xv,
                                               (int)((64 * wave + 8 * i) * K * 2 + kt * 128), 0, 0);
  };
  // Weight rows n0 .. n0+255, 128 B of codes per row per super-step, in the
  // same swizzled order; rows past N read as zero.  Scales: 16 B per row,
  // lane = row within the wave's 64.
  const int64_t nrows = min<int64_t>(FBN, N - n0);
  const __amdgpu_buffer_rsrc_t wrs = rsrc(w.packed + n0 * (K / 2), nrows * (K / 2));
  const uint32_t wv = (uint32_t)((lane >> 3) * (K / 2) + 16 * ((lane & 7) ^ ((lane >> 3) & 7)));
  const __amdgpu_buffer_rsrc_t srs = rsrc(Sp + (int64_t)tn * nsup * FBN * kSup, nsup * FBN * kSup * 4);
  auto wload = [&](int64_t sp, auto B) {
    uint8_t *dst = decltype(B)::value ? Wc1 : Wc0;
    float *sdst = decltype(B)::value ? Sc1 : Sc0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_ptr)(dst + (512 * wave + 64 * i) * 16), 16, wv,
                                               (int)((64 * wave + 8 * i) * (K / 2) + sp * 128), 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_ptr)(sdst + 64 * wave * kSup), 16, (uint32_t)(lane * 16),
                                             (int)(sp * FBN * kSup * 4 + wave * 1024), 0, 0);
  };
  constexpr int kVmemW = 9;  // weight copy instructions per wave and super-step

  // Lane (li, g) of row tile rt expands row 64w + 16rt + li, codes 16g ..
  // 16g+15 of the step's block: bytes 8g .. 8g+7 = chunk 2j + g/2, half g%2.
  u32x2_t wcr[4];
  float sreg[4];
  const int wbase = wave * 8192 + li * 128 + 8 * (g & 1);
  const int sbase = (64 * wave + li) * kSup;
  auto cread = [&](auto S) {  // codes and scales of a step with (step % 8) == S
    constexpr int s8 = decltype(S)::value, j = s8 & 3;
    const uint8_t *wc = ((s8 >> 2) & 1) ? Wc1 : Wc0;
    const float *sc = ((s8 >> 2) & 1) ? Sc1 : Sc0;
    const int off = wbase + (((2 * j + (g >> 1)) ^ (li & 7)) << 4);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      wcr[rt] = *reinterpret_cast<const u32x2_t *>(wc + off + rt * 2048);
      sreg[rt] = sc[sbase + 16 * kSup * rt + j];
    }
  };
  // Piece p of the next step's expansion: p < 4 -> row tile p, sub-step 1
  // into an[p] (a[][1] is still in use); p >= 4 -> row tile p-4, sub-step 0
  // straight into a[p-4][0] (written in MFMA groups 9..15, after its last
  // read in group 7).
  u32x4_t a[4][2], an[4];
  float2 pq[4];  // table reads of the piece in flight
  auto piece_read = [&](int p) {
    const uint32_t word = wcr[p & 3][p < 4 ? 1 : 0];
#pragma unroll
    for (int i = 0; i < 4; ++i) pq[i] = s_pair[(word >> (8 * i)) & 0xFFu];
  };
  auto piece_math = [&](int p) {
    const int rt = p & 3;
    const float s = sreg[rt];
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

  // Prologue: X of step 0 and super-step 0's weights landed, step 0
  // expanded, codes of step 1 in registers.
  __syncthreads();  // pair table
  xload(0, std::integral_constant<int, 0>());
  wload(0, std::integral_constant<int, 0>());
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  cread(std::integral_constant<int, 0>());
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    piece_read(p);
    piece_math(p);
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) a[rt][1] = an[rt];
  cread(std::integral_constant<int, 1>());

  auto step = [&](int64_t kt, auto U) {
    constexpr int u = decltype(U)::value, j = u & 3;
    // Copies past the last step re-read the last one (in bounds, unused).
    xload(min<int64_t>(kt + 1, nk - 1), std::integral_constant<int, (u + 1) & 1>());
    if constexpr (j == 0)
      wload(min<int64_t>((kt >> 2) + 1, nsup - 1), std::integral_constant<int, ((u >> 2) + 1) & 1>());
    // Fragment (column tile ct, sub-step t) sits at xrow[t] + 1024*ct: the
    // swizzle term depends on (row & 7) == (li & 7) only.
    const uint16_t *xs = (u & 1) ? Xs1 : Xs0;
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
      if ((q & 1) == 0) piece_read(q >> 1);  // consumed by the next group
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) mfma16_acc(acc[rt][ct0 + cc], a[rt][t], bq[q & 1][cc]);
      if ((q & 1) == 1) piece_math(q >> 1);  // (on the last step: codes that are never used)
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) a[rt][1] = an[rt];
    cread(std::integral_constant<int, (u + 2) & 7>());  // (past the end: stale, unused)
    // Bare barrier: the loop's only LDS writes are the copies, so
    // __syncthreads()'s release fence would merely wait for the weight copy
    // that may stay in flight after a j == 0 step.
    if constexpr (j == 0)
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kVmemW) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  };
  const int64_t n8 = nk >> 3;
  for (int64_t p = 0; p < n8; ++p) {
    step(8 * p, std::integral_constant<int, 0>());
    step(8 * p + 1, std::integral_constant<int, 1>());
    step(8 * p + 2, std::integral_constant<int, 2>());
    step(8 * p + 3, std::integral_constant<int, 3>());
    step(8 * p + 4, std::integral_constant<int, 4>());
    step(8 * p + 5, std::integral_constant<int, 5>());
    step(8 * p + 6, std::integral_constant<int, 6>());
    step(8 * p + 7, std::integral_constant<int, 7>());
  }
  if constexpr (kOddSup) {
    step(nk - 4, std::integral_constant<int, 0>());
    step(nk - 3, std::integral_constant<int, 1>());
    step(nk - 2, std::integral_constant<int, 2>());
    step(nk - 1, std::integral_constant<int, 3>());
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  fwd_epilogue(acc, Xs0, Bl, r, RP, sH, Y, N, M, n0 + 64 * wave, m0);
}

struct FwdWs {
  SplitPlan sp;
  int RP;
  bool staged;  // k % 256 == 0: k_fwd_nf4 with precomputed tile scales
  size_t part_off, sh_off, scale_off, total;
};

FwdWs fwd_ws_layout(int64_t M, int64_t n, int64_t k, int r) {
  FwdWs l;
  l.RP = lora_rank_pad(r);
  l.sp = plan_split(ceil_div(M, 64), ceil_div(k, 64));
  l.staged = (k % (kBlock * kSup)) == 0;
  l.part_off = 0;
  l.sh_off = align_up((size_t)l.sp.splits * M * l.RP * sizeof(float), 256);
  l.scale_off = l.sh_off + align_up((size_t)M * l.RP * sizeof(uint16_t), 256);
  l.total = l.scale_off + (l.staged ? align_up((size_t)ceil_div(n, FBN) * FBN * (k / kBlock) * sizeof(float), 256) : 0);
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
  if (l.staged) {
    float *Sp = reinterpret_cast<float *>(static_cast<char *>(ws) + l.scale_off);
    const int64_t nsup = K / (kBlock * kSup), total = (int64_t)tiles_n * nsup * FBN;
    QLORA_LAUNCH("k_tile_scales", k_tile_scales, dim3((unsigned)(total / 256)), dim3(256), 0, s, a.w, nsup, total, Sp);
    if (nsup & 1)
      QLORA_LAUNCH("k_fwd_nf4", k_fwd_nf4<1>, grid, dim3(256), 0, s, a.w, Sp, X, M, B, a.r, l.RP, sH, Y, tiles_n);
    else
      QLORA_LAUNCH("k_fwd_nf4", k_fwd_nf4<0>, grid, dim3(256), 0, s, a.w, Sp, X, M, B, a.r, l.RP, sH, Y, tiles_n);
    return hipGetLastError();
  }
  switch ((K / kBlock) & 3) {
    case 0: QLORA_LAUNCH("k_fwd_nf4_any", k_fwd_nf4_any<0>, grid, dim3(256), 0, s, a.w, X, M, B, a.r, l.RP, sH, Y, tiles_n); break;
    case 1: QLORA_LAUNCH("k_fwd_nf4_any", k_fwd_nf4_any<1>, grid, dim3(256), 0, s, a.w, X, M, B, a.r, l.RP, sH, Y, tiles_n); break;
    case 2: QLORA_LAUNCH("k_fwd_nf4_any", k_fwd_nf4_any<2>, grid, dim3(256), 0, s, a.w, X, M, B, a.r, l.RP, sH, Y, tiles_n); break;
    default: QLORA_LAUNCH("k_fwd_nf4_any", k_fwd_nf4_any<3>, grid, dim3(256), 0, s, a.w, X, M, B, a.r, l.RP, sH, Y, tiles_n); break;
  }
  return hipGetLastError();
}

}  // namespace qlora

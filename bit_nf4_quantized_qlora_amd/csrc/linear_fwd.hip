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
//      main kernel streams them.
//   3. k_fwd_nf4: C[n][m] = sum_k W_hat[n][k] X[m][k] + sum_j B[n][j] sH[m][j]
//      on 256x256 tiles.  NF4 codes are expanded in registers straight into
//      MFMA operands through a 256-entry table of level pairs, bit-identical
//      to the standalone dequantization; the LoRA up-projection is a few more
//      MFMA steps on the same accumulators; Y is rounded to bf16 once.

#include "lora_gemm.h"

namespace qlora {
namespace {

constexpr int FBN = 256, FBM = 256;  // block tile: weight rows (n) x X rows (m)

// Tail of the forward kernel, after the main loop has drained
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

constexpr int kSup = 4;  // K steps per staged weight chunk: 128 packed bytes per row

// s_b of every block, in the order k_fwd_nf4 streams them: for weight tile tn
// (rows 256tn .. 256tn+255) and super-step sp (blocks 4sp .. 4sp+3 of each
// row) one contiguous 4 KB run, Sp[((tn*nsup + sp)*256 + row)*4 + j]; rows
// past n and blocks past k/64 hold 0.  block_scale is the dequantization's
// own (bit-identical).
__global__ __launch_bounds__(256) void k_tile_scales(Nf4View w, int64_t nsup, int64_t total,
                                                     float *__restrict__ Sp) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t q = t >> 8, tn = q / nsup, sp = q - tn * nsup;
  const int64_t n = tn * FBN + (t & 255), nk = w.k / kBlock;
  f32x4_t v = {0.f, 0.f, 0.f, 0.f};
  if (n < w.n) {
    const float off = *w.offset;
#pragma unroll
    for (int j = 0; j < kSup; ++j) {
      const int64_t kb = kSup * sp + j, b = n * nk + kb;
      if (kb < nk) v[j] = block_scale(w.scale_code[b], w.group_amax[b / kGroup], off);
    }
  }
  *reinterpret_cast<f32x4_t *>(Sp + 4 * t) = v;
}

// C[n][m] = sum_k W_hat[n][k] X[m][k] + sum_j B[n][j] sH[m][j]  ->  Y[m][n]
// Wave w owns weight rows n0 + 64w .. +63 (four 16-row MFMA tiles) and all
// 256 X rows (sixteen 16-column tiles): 256 fp32 accumulators per lane (all
// in AGPRs).  Its NF4 rows are expanded straight into MFMA A-operand
// registers: lane (li = lane & 15, g = lane >> 4) of row tile rt holds row
// n0+64w+16rt+li and codes 16g .. 16g+15 of the current 64-weight block,
// used as contraction slots 8t .. 8t+7 of sub-step t; the X fragment reads
// the same k positions, so the contraction is unchanged.  Every operand is
// streamed global -> LDS by buffer loads that write LDS directly: the X tile
// one 64-wide K step at a time, packed codes 4 K steps (128 B = one cache
// line per row) at a time with their precomputed block scales
// (k_tile_scales); lanes read their 8-byte code chunks and scales from LDS.
//
// LDS: X tiles Xs0/Xs1 (2 x 32 KB), code tiles Wc0/Wc1 (2 x 32 KB: 256 rows x
// 128 B, 16-byte chunk c of row R at chunk c ^ (R & 7)), scale tiles Sc0/Sc1
// (2 x 4 KB: 256 rows x 4 fp32), pair table 2 KB.  Wave w copies and reads
// only its own 64 weight rows.
//
// One wave per SIMD, so the wave's own instruction stream has to hide every
// latency: a K step is eight "pairs" of 16 MFMAs (pair P: sub-step P/4,
// column tiles 4(P%4) .. +3), and after each MFMA the wave issues one small
// piece of other work, all of it for later pairs:
//   the four X fragments of pair P+1            (LDS reads)
//   the four table reads of expansion piece P+1  (LDS reads)
//   the arithmetic of expansion piece P          (8 multiplies, 4 roundings)
//   in pair 6: codes and scales of step kt+2     (LDS reads)
// Expansion piece p covers row tile p % 4 and sub-step 1 (p < 4) or 0
// (p >= 4) of step kt+1; sub-step-1 operands alternate between two register
// sets by step parity, sub-step-0 operands are rewritten after their last
// use in pair 3.
//
// Barrier B(kt) sits between pairs 6 and 7 of step kt: it waits for the X
// tile of step kt+1 (so pair 7 can already read the next step's first
// fragments) and for this wave's reads of Xs[kt % 2]; right after it the X
// tile of step kt+2 is copied into Xs[kt % 2], and when kt % 4 == 3 the
// codes and scales of super-step kt/4 + 2 into the weight buffers of the
// current super-step, whose last register read was two steps earlier.  A
// weight copy lands by B(kt+2) and is first read in pair 6 of step kt+3.
// The loop is unrolled by 8 steps so every buffer choice is a compile-time
// constant.  k/64 is rounded up to a multiple of 8 steps: steps past the end
// copy zeros for X (zero-length buffer resource) and their blocks have zero
// scales, so they add nothing; this keeps a single loop with no tail (a tail
// would make the compiler move accumulators between register files right
// behind MFMAs it does not track).
//
// Every row-dependent offset goes in the per-lane VGPR offset, which the
// buffer range check covers: rows past M or N read zero and never touch
// memory past the tensors.
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
  const int64_t N = w.n, K = w.k, nk = K / kBlock, nsup = ceil_div_d(nk, kSup);
  const int64_t nk8 = ceil_div_d(nk, 8) * 8;  // steps run: whole 8-step rounds
  fill_pair_table(s_pair, tid, 256);

  // X rows m0 .. m0+255: wave-instruction i fills LDS chunks [512w + 64i,
  // +64): row 64w + 8i + lane/8, logical chunk (lane & 7) ^ ((lane/8) & 7)
  // (the swizzle of xsw).
  const int xbytes = (int)(min<int64_t>(FBM, M - m0) * K * 2);
  const uint32_t xv = (uint32_t)(((64 * wave + (lane >> 3)) * K + 8 * ((lane & 7) ^ ((lane >> 3) & 7))) * 2);
  auto xload = [&](int64_t kt, auto B) {
    uint16_t *dst = decltype(B)::value ? Xs1 : Xs0;
    const __amdgpu_buffer_rsrc_t rs = rsrc(X + m0 * K, kt < nk ? xbytes : 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(dst + (512 * wave + 64 * i) * 8), 16,
                                               xv + (uint32_t)(i * 16 * K), (int)(kt * 128), 0, 0);
  };
  // Weight rows n0 .. n0+255, 128 B of codes per row per super-step, in the
  // same swizzled order (the column offset is in the range-checked offset
  // too: a partial last super-step of the last row reads zeros, not past the
  // tensor).  Scales: 16 B per row, lane = row within the wave's 64 (the
  // table is padded to whole tiles and super-steps).
  const int wbytes = (int)(min<int64_t>(FBN, N - n0) * (K / 2));
  const uint32_t wv = (uint32_t)((64 * wave + (lane >> 3)) * (K / 2) + 16 * ((lane & 7) ^ ((lane >> 3) & 7)));
  const float *Spt = Sp + (int64_t)tn * nsup * FBN * kSup;
  auto wload = [&](int64_t sp, auto B) {
    uint8_t *dst = decltype(B)::value ? Wc1 : Wc0;
    float *sdst = decltype(B)::value ? Sc1 : Sc0;
    const bool real = sp < nsup;
    const __amdgpu_buffer_rsrc_t rs = rsrc(w.packed + n0 * (K / 2), real ? wbytes : 0);
    const __amdgpu_buffer_rsrc_t ss = rsrc(Spt, real ? (int)(nsup * FBN * kSup * 4) : 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(dst + (512 * wave + 64 * i) * 16), 16,
                                               wv + (uint32_t)(i * 4 * K + sp * 128), 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ss, (lds_ptr)(sdst + 64 * wave * kSup), 16,
                                             (uint32_t)(wave * 1024 + lane * 16), (int)(sp * FBN * kSup * 4), 0, 0);
  };
  constexpr int kVmemW = 9;  // weight copy instructions per wave and super-step

  // Codes and scales of step s live in set s % 2.  Lane (li, g) of row tile
  // rt expands row 64w + 16rt + li, codes 16g .. 16g+15 of the step's block:
  // bytes 8g .. 8g+7 = chunk 2j + g/2, half g%2.
  u32x2_t wcr[2][4];
  float sreg[2][4];
  const int wbase = wave * 8192 + li * 128 + 8 * (g & 1);
  const int sbase = (64 * wave + li) * kSup;
  auto cread = [&](auto S, int half) {  // step with (step % 8) == S; row tiles 2half, 2half+1
    constexpr int s8 = decltype(S)::value, j = s8 & 3, d = s8 & 1;
    const uint8_t *wc = ((s8 >> 2) & 1) ? Wc1 : Wc0;
    const int off = wbase + (((2 * j + (g >> 1)) ^ (li & 7)) << 4);
#pragma unroll
    for (int rt = 2 * half; rt < 2 * half + 2; ++rt) wcr[d][rt] = *reinterpret_cast<const u32x2_t *>(wc + off + rt * 2048);
  };
  auto sread = [&](auto S, int half) {
    constexpr int s8 = decltype(S)::value, j = s8 & 3, d = s8 & 1;
    const float *sc = ((s8 >> 2) & 1) ? Sc1 : Sc0;
#pragma unroll
    for (int rt = 2 * half; rt < 2 * half + 2; ++rt) sreg[d][rt] = sc[sbase + 16 * kSup * rt + j];
  };

  u32x4_t a0[4], a1[2][4];  // A operands: sub-step 0; sub-step 1 by step parity
  u32x4_t bq[2][4];         // X fragments of a pair, by pair parity
  float2 pq[2][4];          // table reads of an expansion piece, by piece parity
  // Table read i of piece p from code set d into pq[p % 2][i].
  auto tread = [&](int d, int p, int i) {
    const uint32_t word = wcr[d][p & 3][p < 4 ? 1 : 0];
    pq[p & 1][i] = s_pair[(word >> (8 * i)) & 0xFFu];
  };
  // Quarter i of piece p's arithmetic (scales of set d); operands for a
  // step of parity e.
  auto tmath = [&](int d, int e, int p, int i) {
    const float s = sreg[d][p & 3];
    const float2 v = pq[p & 1][i];
    const uint32_t x = bf16x2_rne(__fmul_rn(v.x, s), __fmul_rn(v.y, s));
    if (p < 4) a1[e][p & 3][i] = x;
    else a0[p & 3][i] = x;
  };
  auto xfrag = [&](const uint16_t *xs, int P, int cc) -> u32x4_t {
    const int t = P >> 2, ct = 4 * (P & 3) + cc;
    return *reinterpret_cast<const u32x4_t *>(xs + xsw(16 * ct + li, 2 * g + t));
  };

  f32x4_t acc[4][16];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Prologue: X of step 0 and super-step 0's weights landed; X of step 1
  // and super-step 1's weights in flight (the copy slot before B(0)); step 0
  // expanded; codes of step 1 in set 1; pair 0's fragments and piece 0's
  // table reads issued.
  __syncthreads();  // pair table
  xload(0, std::integral_constant<int, 0>());
  wload(0, std::integral_constant<int, 0>());
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  xload(1, std::integral_constant<int, 1>());
  wload(1, std::integral_constant<int, 1>());
  cread(std::integral_constant<int, 0>(), 0);
  cread(std::integral_constant<int, 0>(), 1);
  sread(std::integral_constant<int, 0>(), 0);
  sread(std::integral_constant<int, 0>(), 1);
#pragma unroll
  for (int p = 0; p < 8; ++p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) tread(0, p, i);
#pragma unroll
    for (int i = 0; i < 4; ++i) tmath(0, 0, p, i);
  }
  cread(std::integral_constant<int, 1>(), 0);
  cread(std::integral_constant<int, 1>(), 1);
  sread(std::integral_constant<int, 1>(), 0);
  sread(std::integral_constant<int, 1>(), 1);
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) bq[0][cc] = xfrag(Xs0, 0, cc);
#pragma unroll
  for (int i = 0; i < 4; ++i) tread(1, 0, i);

  auto step = [&](int64_t kt, auto U) {
    constexpr int u = decltype(U)::value, j = u & 3, e = u & 1;
    const uint16_t *xs = e ? Xs1 : Xs0, *xn = e ? Xs0 : Xs1;
    constexpr int dc = (u + 1) & 1;  // code set of step kt+1 (expanded now)
#pragma unroll
    for (int P = 0; P < 8; ++P) {
      const int t = P >> 2, ct0 = 4 * (P & 3);
      if (P == 7) {
        // B(kt): the X tile of step kt+1 landed everywhere, every wave done
        // reading Xs[kt % 2]; then refill it with step kt+2.
        if constexpr (j == 0)
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kVmemW) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // (copies past the end read zeros; their data is never used)
        xload(kt + 2, std::integral_constant<int, e>());
        if constexpr (j == 3) wload((kt >> 2) + 2, std::integral_constant<int, (u >> 2) & 1>());
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int cc = s >> 2, rt = s & 3;
        mfma16_acc(acc[rt][ct0 + cc], t ? a1[e][rt] : a0[rt], bq[P & 1][cc]);
        if (s < 12) {
          const int q = s / 3, kind = s % 3;
          if (kind == 0) {  // X fragment q of the next pair
            if (P < 7) bq[(P + 1) & 1][q] = xfrag(xs, P + 1, q);
            else bq[0][q] = xfrag(xn, 0, q);
          } else if (kind == 1) {  // table read q of the next piece
            if (P < 7) tread(dc, P + 1, q);
            else tread(e, 0, q);  // piece 0 of step kt+1's expansion: codes of kt+2
          } else {
            tmath(dc, e ^ 1, P, q);
          }
        } else if (P == 6) {  // codes and scales of step kt+2
          if (s == 12) cread(std::integral_constant<int, (u + 2) & 7>(), 0);
          if (s == 13) cread(std::integral_constant<int, (u + 2) & 7>(), 1);
          if (s == 14) sread(std::integral_constant<int, (u + 2) & 7>(), 0);
          if (s == 15) sread(std::integral_constant<int, (u + 2) & 7>(), 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int64_t p = 0; p < nk8 / 8; ++p) {
    step(8 * p, std::integral_constant<int, 0>());
    step(8 * p + 1, std::integral_constant<int, 1>());
    step(8 * p + 2, std::integral_constant<int, 2>());
    step(8 * p + 3, std::integral_constant<int, 3>());
    step(8 * p + 4, std::integral_constant<int, 4>());
    step(8 * p + 5, std::integral_constant<int, 5>());
    step(8 * p + 6, std::integral_constant<int, 6>());
    step(8 * p + 7, std::integral_constant<int, 7>());
  }
  mfma_acc_fence();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  fwd_epilogue(acc, Xs0, Bl, r, RP, sH, Y, N, M, n0 + 64 * wave, m0);
}

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
  l.total = l.scale_off +
            align_up((size_t)ceil_div(n, FBN) * ceil_div(k / kBlock, kSup) * FBN * kSup * sizeof(float), 256);
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
  float *Sp = reinterpret_cast<float *>(static_cast<char *>(ws) + l.scale_off);
  const int64_t nsup = ceil_div(K / kBlock, kSup), total = (int64_t)tiles_n * nsup * FBN;
  QLORA_LAUNCH("k_tile_scales", k_tile_scales, dim3((unsigned)(total / 256)), dim3(256), 0, s, a.w, nsup, total, Sp);
  QLORA_LAUNCH("k_fwd_nf4", k_fwd_nf4, dim3((unsigned)(tiles_n * tiles_m)), dim3(256), 0, s, a.w, Sp, X, M, B, a.r,
               l.RP, sH, Y, tiles_n);
  return hipGetLastError();
}

}  // namespace qlora

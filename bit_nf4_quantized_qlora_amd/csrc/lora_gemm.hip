// lora_gemm.hip -- the rank-r products of the LoRA path on BF16 MFMA.
//
// "QLoRA Paper Breakdown" sec. 4: the forward adds (alpha/r) X L_1 L_2
// (L_1 = A^T, L_2 = B^T), and the backward produces gradients for the
// adapters only ("QLoRA, explained." step 5).  The products here are skinny:
// one side has r <= 128 rows, the contraction runs over k, n or M.
//
//   k_nt_dma       part[s][i][j] = sum_{c in split s} P[i][c] * Q[j][c]
//                  (both operands contraction-contiguous): H = X A^T; and,
//                  with Q given as it lies ([c][j], read down its columns),
//                  G = dY B without a transposed copy of B.
//   k_tn_dma       part[s][j][i] = sum_{m in split s} P[m][i] * Qt[j][m]
//                  (P is a big row-major [M][D] operand, read transposed out
//                  of LDS): dB = dY^T (sH) and dA = G^T X, one launch.
//   k_nt_splitk,   the same products for row strides that are not a
//   k_tn_splitk    multiple of 8 elements (no 16-byte DMA copies).
//   Reductions     the split partials summed in a fixed order (deterministic)
//                  into the fp32 / bf16 / transposed forms needed next, as
//                  jobs of jobs.hip.
#include "lora_gemm.h"

namespace qlora {
namespace {

constexpr int LD = 72;  // LDS row stride (64 + 8 bf16 of padding)

template <int TJ>
__global__ __launch_bounds__(256) void k_nt_splitk(const uint16_t *__restrict__ P, int64_t rowsP,
                                                   const uint16_t *__restrict__ Q, int rowsQ, int64_t lenC,
                                                   int64_t ld, bool vec_ok, int steps_per_split,
                                                   float *__restrict__ part) {
  constexpr int RP = 16 * TJ;
  __shared__ __align__(16) uint16_t Ps[64 * LD];
  __shared__ __align__(16) uint16_t Qs[RP * LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  const int64_t nsteps = ceil_div_d(lenC, 64);
  const int64_t s0 = (int64_t)blockIdx.y * steps_per_split;
  const int64_t s1 = min<int64_t>(nsteps, s0 + steps_per_split);
  f32x4_t acc[1][TJ];
#pragma unroll
  for (int t = 0; t < TJ; ++t) acc[0][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t st = s0; st < s1; ++st) {
    const int64_t c0 = st * 64;
#pragma unroll
    for (int c = tid; c < 64 * 8; c += 256) {
      const int row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4_t *>(Ps + row * LD + col) = load8(P, ld, rowsP, lenC, i0 + row, c0 + col, vec_ok);
    }
#pragma unroll
    for (int c = tid; c < RP * 8; c += 256) {
      const int row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4_t *>(Qs + row * LD + col) = load8(Q, ld, rowsQ, lenC, row, c0 + col, vec_ok);
    }
    __syncthreads();
    mma_step<1, TJ>(acc, Ps, Qs, LD, wave * 16, 0, 0, lane);
    mma_step<1, TJ>(acc, Ps, Qs, LD, wave * 16, 0, 32, lane);
    __syncthreads();
  }
  float *out = part + (size_t)blockIdx.y * rowsP * RP;
#pragma unroll
  for (int t = 0; t < TJ; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t i = i0 + wave * 16 + 4 * (lane >> 4) + v;
      if (i < rowsP) out[i * RP + 16 * t + (lane & 15)] = acc[0][t][v];
    }
}

template <int TJ>
__global__ __launch_bounds__(256) void k_tn_splitk(const uint16_t *__restrict__ P, int64_t M, int64_t D,
                                                   bool vec_ok, const uint16_t *__restrict__ Qt, int64_t ldq,
                                                   int steps_per_split, bool rows_out, float *__restrict__ part) {
  constexpr int RP = 16 * TJ;
  __shared__ __align__(16) uint16_t Ps[64 * LD];  // [i][m]
  __shared__ __align__(16) uint16_t Qs[RP * LD];  // [j][m]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  const int64_t nsteps = ceil_div_d(M, 64);
  const int64_t s0 = (int64_t)blockIdx.y * steps_per_split;
  const int64_t s1 = min<int64_t>(nsteps, s0 + steps_per_split);
  f32x4_t acc[1][TJ];
#pragma unroll
  for (int t = 0; t < TJ; ++t) acc[0][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int mg = tid >> 3, ig = tid & 7;  // rows 2mg, 2mg+1; columns 8ig..8ig+7

  for (int64_t st = s0; st < s1; ++st) {
    const int64_t m0 = st * 64;
    {
      const u32x4_t r0 = load8(P, D, M, D, m0 + 2 * mg, i0 + 8 * ig, vec_ok);
      const u32x4_t r1 = load8(P, D, M, D, m0 + 2 * mg + 1, i0 + 8 * ig, vec_ok);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        *reinterpret_cast<uint32_t *>(Ps + (8 * ig + 2 * d) * LD + 2 * mg) = pack_lo(r0[d], r1[d]);
        *reinterpret_cast<uint32_t *>(Ps + (8 * ig + 2 * d + 1) * LD + 2 * mg) = pack_hi(r0[d], r1[d]);
      }
    }
#pragma unroll
    for (int c = tid; c < RP * 8; c += 256) {
      const int row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<u32x4_t *>(Qs + row * LD + col) = load8(Qt, ldq, RP, M, row, m0 + col, true);
    }
    __syncthreads();
    mma_step<1, TJ>(acc, Ps, Qs, LD, wave * 16, 0, 0, lane);
    mma_step<1, TJ>(acc, Ps, Qs, LD, wave * 16, 0, 32, lane);
    __syncthreads();
  }
  float *out = part + (size_t)blockIdx.y * RP * D;
#pragma unroll
  for (int t = 0; t < TJ; ++t) {
    const int j = 16 * t + (lane & 15);
    const int64_t i = i0 + wave * 16 + 4 * (lane >> 4);
    if (rows_out) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (i + v < D) out[(i + v) * RP + j] = acc[0][t][v];
    } else if (i + 4 <= D && (D & 3) == 0) {
      *reinterpret_cast<f32x4_t *>(out + j * D + i) = acc[0][t];
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (i + v < D) out[j * D + i + v] = acc[0][t][v];
    }
  }
}

// ---------------------------------------------------------------------------
// DMA-pipelined forms (row strides % 8 == 0).  Operand tiles stream global ->
// LDS by buffer loads that write LDS directly, four steps in flight (buffers
// b0..b3, one per step mod 4; separate arrays so the compiler sees that an
// in-flight copy never aliases the tile being read).  A 64-wide tile row is
// 128 B with its 16-byte chunk c at chunk c ^ ((row >> 1) & 7) (conflict-free
// MFMA fragment reads with 64 LDS banks); wave-instruction i of a copy fills
// rows 8i .. 8i+7, lane l taking row 8i + l/8 and physical chunk l & 7, so
// the logical chunk it copies depends on the parity of i.  Columns past the
// contraction length and rows past the operand are steered out of the buffer
// range (per-lane offset), so they read zero; steps past a split's end use
// zero-length resources.  The step count per split is a multiple of 4.

constexpr uint32_t kOOB = 0x80000000u;  // a per-lane offset past every buffer range

__device__ __forceinline__ int swz_chunk(int row, int c) { return c ^ ((row >> 1) & 7); }

// One copy of a [rows][64] bf16 tile (rows = 8 * ninstr per wave... see caller).
// base: operand origin; nrows/ncols: its extent; ld: row stride (elements);
// row0/col0: tile origin; dst: LDS tile; first: first tile row this wave copies.
template <int NI>
__device__ __forceinline__ void dma_tile(const uint16_t *base, int64_t nrows, int64_t ncols, int64_t ld, int64_t row0,
                                         int64_t col0, bool live, uint16_t *dst, int first, int lane) {
  const __amdgpu_buffer_rsrc_t rs = rsrc(base, live ? nrows * ld * 2 : 0);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = first + 8 * i + (lane >> 3);
    const int lc = swz_chunk(row, lane & 7);  // logical chunk this lane copies
    const int64_t gr = row0 + row, gc = col0 + 8 * lc;
    const uint32_t off = (gr < nrows && gc < ncols) ? (uint32_t)((gr * ld + gc) * 2) : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(dst + (first + 8 * i) * 64), 16, off, 0, 0, 0);
  }
}

// part[s][i][j] = sum over split s of P[i][c] Q[j][c]: 64 rows of P per
// workgroup (16 per wave), all RP rows of Q.
// kQRows: Q is given as its transpose, Qr [lenC][ldqr] (row c holds Q[.][c],
// its first rowsQ entries real; RP <= 64): each step stages the [64 c][64 j]
// tile of Qr as it lies and reads the MFMA operands down its columns with
// ds_read_b64_tr_b16 (as k_tn_dma reads its P tile), so no transposed copy
// of Q is needed.
template <int TJ, bool kQRows = false>
__global__ __launch_bounds__(256) void k_nt_dma(const uint16_t *__restrict__ P, int64_t rowsP,
                                                const uint16_t *__restrict__ Q, int rowsQ, int64_t lenC, int64_t ld,
                                                int steps_per_split, float *__restrict__ part, int64_t ldqr = 0) {
  static_assert(!kQRows || TJ <= 4, "the transposed Q form stages one 64-column tile");
  constexpr int RP = 16 * TJ, NQ = kQRows ? 2 : RP / 32, NV = 2 + NQ;  // copy instructions per wave and step
  constexpr int QT = kQRows ? 64 * 64 : RP * 64;  // elements of one staged Q tile
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  __shared__ __align__(16) uint16_t P0[64 * 64], P1[64 * 64], P2[64 * 64], P3[64 * 64];
  __shared__ __align__(16) uint16_t Q0[QT], Q1[QT], Q2[QT], Q3[QT];
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  const int64_t nsteps = ceil_div_d(lenC, 64);
  const int64_t s0 = (int64_t)blockIdx.y * steps_per_split;
  const int64_t s1 = min<int64_t>(nsteps, s0 + steps_per_split);
  auto pbuf = [&](auto B) -> uint16_t * {
    constexpr int b = decltype(B)::value & 3;
    return b == 0 ? P0 : b == 1 ? P1 : b == 2 ? P2 : P3;
  };
  auto qbuf = [&](auto B) -> uint16_t * {
    constexpr int b = decltype(B)::value & 3;
    return b == 0 ? Q0 : b == 1 ? Q1 : b == 2 ? Q2 : Q3;
  };
  auto copy = [&](int64_t st, auto B) {
    const bool live = st < s1;
    dma_tile<2>(P, rowsP, lenC, ld, i0, st * 64, live, pbuf(B), 16 * wave, lane);
    if constexpr (kQRows)
      dma_tile<2>(Q, lenC, rowsQ, ldqr, st * 64, 0, live, qbuf(B), 16 * wave, lane);
    else
      dma_tile<NQ>(Q, rowsQ, lenC, ld, 0, st * 64, live, qbuf(B), 8 * NQ * wave, lane);
  };
  f32x4_t acc[TJ];
#pragma unroll
  for (int t = 0; t < TJ; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // kQRows: transposed-read address of lane (li, g) for sub-step t, half h
  // and column tile jt: row 32t + 8g + 4h + li/4, columns 16jt + 4(li & 3) ..
  auto tr_off = [&](int t, int h, int jt) -> int {
    const int row = 32 * t + 8 * g + 4 * h + (li >> 2), col = 16 * jt + 4 * (li & 3);
    return row * 64 + swz_chunk(row, col >> 3) * 8 + (col & 7);
  };

  copy(s0, std::integral_constant<int, 0>());
  copy(s0 + 1, std::integral_constant<int, 1>());
  copy(s0 + 2, std::integral_constant<int, 2>());
  auto step = [&](int64_t st, auto B) {
    // this step's copies (three steps old) landed everywhere; every wave is
    // done reading the buffer the next copy refills
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * NV) : "memory");
    copy(st + 3, std::integral_constant<int, (decltype(B)::value + 3) & 3>());
    const uint16_t *ps = pbuf(B), *qs = qbuf(B);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = 16 * wave + li, c = 4 * t + g;
      const u32x4_t a = *reinterpret_cast<const u32x4_t *>(ps + row * 64 + swz_chunk(row, c) * 8);
#pragma unroll
      for (int jt = 0; jt < TJ; ++jt) {
        u32x4_t b;
        if constexpr (kQRows) {
          const s16x4_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t *)(qs + tr_off(t, 0, jt)));
          const s16x4_t h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t *)(qs + tr_off(t, 1, jt)));
          b = __builtin_bit_cast(u32x4_t, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          const int qr = 16 * jt + li;
          b = *reinterpret_cast<const u32x4_t *>(qs + qr * 64 + swz_chunk(qr, c) * 8);
        }
        acc[jt] = mfma16(a, b, acc[jt]);
      }
    }
  };
  for (int64_t st = s0; st < s1; st += 4) {
    step(st, std::integral_constant<int, 0>());
    step(st + 1, std::integral_constant<int, 1>());
    step(st + 2, std::integral_constant<int, 2>());
    step(st + 3, std::integral_constant<int, 3>());
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  float *out = part + (size_t)blockIdx.y * rowsP * RP;
#pragma unroll
  for (int jt = 0; jt < TJ; ++jt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t i = i0 + 16 * wave + 4 * g + v;
      if (i < rowsP) out[i * RP + 16 * jt + li] = acc[jt][v];
    }
}

// part = sum over split s of Qt[j][m] P[m][d]: 64 columns d per workgroup
// (16 per wave), all RP rows j.  The P tile [64 m][64 d] is read into MFMA B
// operands (contraction along m, down a column) by ds_read_b64_tr_b16: in a
// 16-lane group, lane i receives element i & 3 of the 8 bytes addressed by
// lanes 4q + i/4 (q = 0..3), so lanes addressing rows m + q, columns 4(j & 3)
// hand lane i four consecutive m of column i; two reads give the fragment.
// rows_out == true: part[s][d][j] (reduced into [D][r]); else part[s][j][d].
// One transposed product of a launch: see TnProblem.
struct TnArgs {
  const uint16_t *P;
  int64_t D;
  const uint16_t *Qt;
  int64_t ldq;
  int steps_per_split, tiles;
  bool rows_out;
  float *part;
};

// Blocks [0, nb0) take problem a0 (tile b % tiles, split b / tiles), the
// rest problem a1.
template <int TJ>
__global__ __launch_bounds__(256) void k_tn_dma(TnArgs a0, TnArgs a1, int nb0, int64_t M) {
  constexpr int RP = 16 * TJ, NQ = RP / 32, NV = 2 + NQ;
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  __shared__ __align__(16) uint16_t P0[64 * 64], P1[64 * 64], P2[64 * 64], P3[64 * 64];
  __shared__ __align__(16) uint16_t Q0[RP * 64], Q1[RP * 64], Q2[RP * 64], Q3[RP * 64];
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool second = (int)blockIdx.x >= nb0;
  const TnArgs &ta = second ? a1 : a0;
  const int bl = second ? (int)blockIdx.x - nb0 : (int)blockIdx.x;
  const uint16_t *__restrict__ P = ta.P;
  const uint16_t *__restrict__ Qt = ta.Qt;
  const int64_t D = ta.D, ldq = ta.ldq;
  const int steps_per_split = ta.steps_per_split;
  const bool rows_out = ta.rows_out;
  float *__restrict__ part = ta.part;
  const int split = bl / ta.tiles;
  const int64_t d0 = (int64_t)(bl - split * ta.tiles) * 64;
  const int64_t nsteps = ceil_div_d(M, 64);
  const int64_t s0 = (int64_t)split * steps_per_split;
  const int64_t s1 = min<int64_t>(nsteps, s0 + steps_per_split);
  auto pbuf = [&](auto B) -> uint16_t * {
    constexpr int b = decltype(B)::value & 3;
    return b == 0 ? P0 : b == 1 ? P1 : b == 2 ? P2 : P3;
  };
  auto qbuf = [&](auto B) -> uint16_t * {
    constexpr int b = decltype(B)::value & 3;
    return b == 0 ? Q0 : b == 1 ? Q1 : b == 2 ? Q2 : Q3;
  };
  auto copy = [&](int64_t st, auto B) {
    const bool live = st < s1;
    dma_tile<2>(P, M, D, D, st * 64, d0, live, pbuf(B), 16 * wave, lane);
    dma_tile<NQ>(Qt, RP, ldq, ldq, 0, st * 64, live, qbuf(B), 8 * NQ * wave, lane);
  };
  f32x4_t acc[TJ];
#pragma unroll
  for (int t = 0; t < TJ; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // transposed-read address of lane (j = li, g) for sub-step t, half h:
  // row 32t + 8g + 4h + j/4, columns 16*wave + 4(j & 3) .. +3
  auto tr_off = [&](int t, int h) -> int {
    const int row = 32 * t + 8 * g + 4 * h + (li >> 2), col = 16 * wave + 4 * (li & 3);
    return row * 64 + swz_chunk(row, col >> 3) * 8 + (col & 7);
  };

  copy(s0, std::integral_constant<int, 0>());
  copy(s0 + 1, std::integral_constant<int, 1>());
  copy(s0 + 2, std::integral_constant<int, 2>());
  auto step = [&](int64_t st, auto B) {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * NV) : "memory");
    copy(st + 3, std::integral_constant<int, (decltype(B)::value + 3) & 3>());
    const uint16_t *ps = pbuf(B), *qs = qbuf(B);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const s16x4_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t *)(ps + tr_off(t, 0)));
      const s16x4_t h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t *)(ps + tr_off(t, 1)));
      const u32x4_t b = __builtin_bit_cast(u32x4_t, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int jt = 0; jt < TJ; ++jt) {
        const int qr = 16 * jt + li, c = 4 * t + g;
        const u32x4_t a = *reinterpret_cast<const u32x4_t *>(qs + qr * 64 + swz_chunk(qr, c) * 8);
        acc[jt] = mfma16(a, b, acc[jt]);
      }
    }
  };
  for (int64_t st = s0; st < s1; st += 4) {
    step(st, std::integral_constant<int, 0>());
    step(st + 1, std::integral_constant<int, 1>());
    step(st + 2, std::integral_constant<int, 2>());
    step(st + 3, std::integral_constant<int, 3>());
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // acc[jt][v] = C[j = 16jt + 4g + v][d = d0 + 16*wave + li]
  const int64_t d = d0 + 16 * wave + li;
  if (d < D) {
    if (rows_out) {
      float *out = part + ((size_t)split * D + d) * RP;
#pragma unroll
      for (int jt = 0; jt < TJ; ++jt) *reinterpret_cast<f32x4_t *>(out + 16 * jt + 4 * g) = acc[jt];
    } else {
      float *out = part + (size_t)split * RP * D;
#pragma unroll
      for (int jt = 0; jt < TJ; ++jt)
#pragma unroll
        for (int v = 0; v < 4; ++v) out[(int64_t)(16 * jt + 4 * g + v) * D + d] = acc[jt][v];
    }
  }
}

__global__ __launch_bounds__(256) void k_fill_zero_u16(uint16_t *__restrict__ p, int64_t n) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < n) p[idx] = 0;
}

template <typename F>
hipError_t dispatch_tj(int RP, F &&f) {
  switch (RP) {
    case 32: return f(std::integral_constant<int, 2>());
    case 64: return f(std::integral_constant<int, 4>());
    case 96: return f(std::integral_constant<int, 6>());
    case 128: return f(std::integral_constant<int, 8>());
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int lora_rank_pad(int r) { return (r + 31) / 32 * 32; }

SplitPlan plan_split(int64_t tiles, int64_t steps) {
  // Aim for ~256 workgroups (one per CU; each keeps three steps of copies
  // in flight) with >= 8 contraction steps each, a multiple of 4.  Measured
  // on the 7B MLP shapes, 256 beat 512, 768 and 1024 (fewer splits write and
  // re-read fewer fp32 partials), and a deeper 8-step copy queue did not help.
  SplitPlan p;
  int64_t want = tiles >= 256 ? 1 : ceil_div(256, tiles);
  want = std::max<int64_t>(1, std::min<int64_t>(want, steps / 8 > 0 ? steps / 8 : 1));
  p.steps_per_split = (int)(ceil_div(ceil_div(steps, want), 4) * 4);
  p.splits = (int)ceil_div(steps, p.steps_per_split);
  return p;
}

hipError_t launch_nt_splitk(const uint16_t *P, int64_t rowsP, const uint16_t *Q, int rowsQ, int RP, int64_t lenC,
                            int64_t ld, const SplitPlan &sp, float *part, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(rowsP, 64), (unsigned)sp.splits);
  const bool vec_ok = (ld % 8) == 0;
  return dispatch_tj(RP, [&](auto tj) {
    if (vec_ok)
      QLORA_LAUNCH("k_nt_dma", k_nt_dma<decltype(tj)::value>, grid, dim3(256), 0, s, P, rowsP, Q, rowsQ, lenC, ld,
                   sp.steps_per_split, part);
    else
      QLORA_LAUNCH("k_nt_splitk", k_nt_splitk<decltype(tj)::value>, grid, dim3(256), 0, s, P, rowsP, Q, rowsQ, lenC,
                   ld, vec_ok, sp.steps_per_split, part);
    return hipGetLastError();
  });
}

bool nt_rows_supported(int r, int64_t ld) { return r % 8 == 0 && r <= 64 && ld % 8 == 0; }

hipError_t launch_nt_rows(const uint16_t *P, int64_t rowsP, const uint16_t *Qr, int r, int RP, int64_t lenC,
                          int64_t ld, const SplitPlan &sp, float *part, hipStream_t s) {
  if (!nt_rows_supported(r, ld) || RP > 64) return hipErrorInvalidValue;
  const dim3 grid((unsigned)ceil_div(rowsP, 64), (unsigned)sp.splits);
  if (RP == 32)
    QLORA_LAUNCH("k_nt_dma", (k_nt_dma<2, true>), grid, dim3(256), 0, s, P, rowsP, Qr, r, lenC, ld,
                 sp.steps_per_split, part, (int64_t)r);
  else
    QLORA_LAUNCH("k_nt_dma", (k_nt_dma<4, true>), grid, dim3(256), 0, s, P, rowsP, Qr, r, lenC, ld,
                 sp.steps_per_split, part, (int64_t)r);
  return hipGetLastError();
}

hipError_t launch_tn_splitk(const uint16_t *P, int64_t M, int64_t D, const uint16_t *Qt, int64_t ldq, int RP,
                            const SplitPlan &sp, bool rows_out, float *part, hipStream_t s) {
  const bool vec_ok = (D % 8) == 0;
  return dispatch_tj(RP, [&](auto tj) {
    if (vec_ok && ldq % 8 == 0) {
      const TnArgs a{P, D, Qt, ldq, sp.steps_per_split, (int)ceil_div(D, 64), rows_out, part};
      const int nb = a.tiles * sp.splits;
      QLORA_LAUNCH("k_tn_dma", k_tn_dma<decltype(tj)::value>, dim3((unsigned)nb), dim3(256), 0, s, a, a, nb, M);
    } else {
      const dim3 grid((unsigned)ceil_div(D, 64), (unsigned)sp.splits);
      QLORA_LAUNCH("k_tn_splitk", k_tn_splitk<decltype(tj)::value>, grid, dim3(256), 0, s, P, M, D, vec_ok, Qt, ldq,
                   sp.steps_per_split, rows_out, part);
    }
    return hipGetLastError();
  });
}

hipError_t launch_tn_pair(const TnProblem &p0, const TnProblem &p1, int64_t M, int RP, hipStream_t s) {
  auto dma_ok = [](const TnProblem &p) { return p.D % 8 == 0 && p.ldq % 8 == 0; };
  if (!dma_ok(p0) || !dma_ok(p1)) {
    hipError_t e = launch_tn_splitk(p0.P, M, p0.D, p0.Qt, p0.ldq, RP, p0.sp, p0.rows_out, p0.part, s);
    if (e != hipSuccess) return e;
    return launch_tn_splitk(p1.P, M, p1.D, p1.Qt, p1.ldq, RP, p1.sp, p1.rows_out, p1.part, s);
  }
  return dispatch_tj(RP, [&](auto tj) {
    const TnArgs a0{p0.P, p0.D, p0.Qt, p0.ldq, p0.sp.steps_per_split, (int)ceil_div(p0.D, 64), p0.rows_out, p0.part};
    const TnArgs a1{p1.P, p1.D, p1.Qt, p1.ldq, p1.sp.steps_per_split, (int)ceil_div(p1.D, 64), p1.rows_out, p1.part};
    const int nb0 = a0.tiles * p0.sp.splits, nb1 = a1.tiles * p1.sp.splits;
    QLORA_LAUNCH("k_tn_dma", k_tn_dma<decltype(tj)::value>, dim3((unsigned)(nb0 + nb1)), dim3(256), 0, s, a0, a1, nb0,
                 M);
    return hipGetLastError();
  });
}

hipError_t launch_reduce_rows(const float *part, int S, int64_t R, int RP, int r, float scale, float *out_f32,
                              uint16_t *out_b, uint16_t *out_bt, int64_t ldt, hipStream_t s) {
  const SmallJob j = job_reduce_rows(part, S, R, RP, r, scale, out_f32, out_b, out_bt, ldt);
  return launch_jobs("k_reduce_rows", &j, 1, s);
}

hipError_t launch_reduce_cols(const float *part, int S, int64_t D, int RP, int r, bool rows_out, uint16_t *out,
                              hipStream_t s) {
  const SmallJob j = job_reduce_cols(part, S, D, RP, r, rows_out, out);
  return launch_jobs("k_reduce_cols", &j, 1, s);
}

hipError_t launch_fill_zero_u16(uint16_t *p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  QLORA_LAUNCH("k_fill_zero_u16", k_fill_zero_u16, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace qlora

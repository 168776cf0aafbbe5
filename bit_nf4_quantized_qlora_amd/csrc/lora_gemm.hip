// lora_gemm.hip -- the rank-r products of the LoRA path on BF16 MFMA.
//
// "QLoRA Paper Breakdown" sec. 4: the forward adds (alpha/r) X L_1 L_2
// (L_1 = A^T, L_2 = B^T), and the backward produces gradients for the
// adapters only ("QLoRA, explained." step 5).  The products here are skinny:
// one side has r <= 128 rows, the contraction runs over k, n or M.
//
//   k_nt_splitk    part[s][i][j] = sum_{c in split s} P[i][c] * Q[j][c]
//                  (both operands contraction-contiguous): H = X A^T and
//                  G = dY B (with B pre-transposed).
//   k_tn_splitk    part[s][j][i] = sum_{m in split s} P[m][i] * Qt[j][m]
//                  (P is a big row-major [M][D] operand, transposed while it
//                  is staged to LDS): dB = dY^T (sH) and dA = G^T X.
//   k_reduce_*     sum the split partials in a fixed order (deterministic)
//                  and write the fp32 / bf16 / transposed forms needed next.
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
                                                   int steps_per_split, float *__restrict__ part) {
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
    if (i + 4 <= D && (D & 3) == 0) {
      *reinterpret_cast<f32x4_t *>(out + j * D + i) = acc[0][t];
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (i + v < D) out[j * D + i + v] = acc[0][t][v];
    }
  }
}

// Rows form: part [S][R][RP] -> v = sum_s part[s][i][j].
//   out_f32 [R][r]   = v            (j < r)
//   out_b   [R][RP]  = bf16(scale*v)  (all j; columns >= r are zero)
//   out_bt  [RP][ldt] = bf16(scale*v) transposed; columns i >= R zero-filled
__global__ __launch_bounds__(256) void k_reduce_rows(const float *__restrict__ part, int S, int64_t R, int RP,
                                                     int r, float scale, float *__restrict__ out_f32,
                                                     uint16_t *__restrict__ out_b, uint16_t *__restrict__ out_bt,
                                                     int64_t ldt) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t Rt = out_bt ? ldt : R;
  if (idx >= Rt * RP) return;
  const int64_t i = idx / RP;
  const int j = (int)(idx % RP);
  float v = 0.f;
  if (i < R) {
    for (int s = 0; s < S; ++s) v += part[(size_t)s * R * RP + idx];
    if (out_f32 && j < r) out_f32[i * r + j] = v;
    if (out_b) out_b[idx] = f32_to_bf16_bits(scale * v);
  }
  if (out_bt) out_bt[(int64_t)j * ldt + i] = i < R ? f32_to_bf16_bits(scale * v) : (uint16_t)0;
}

// Columns form: part [S][RP][D] -> v = sum_s part[s][j][i];
//   transpose == false: out [r][D] = bf16(v)   (dA)
//   transpose == true:  out [D][r] = bf16(v)   (dB)
__global__ __launch_bounds__(256) void k_reduce_cols(const float *__restrict__ part, int S, int64_t D, int RP,
                                                     int r, bool transpose, uint16_t *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)r * D) return;
  int64_t i;
  int j;
  if (transpose) {
    i = idx / r;
    j = (int)(idx % r);
  } else {
    j = (int)(idx / D);
    i = idx % D;
  }
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[(size_t)s * RP * D + (int64_t)j * D + i];
  out[idx] = f32_to_bf16_bits(v);
}

// out [RP][ldo] = in^T for a row-major in [rows][cols] (bf16), zero outside.
__global__ __launch_bounds__(256) void k_transpose_pad(const uint16_t *__restrict__ in, int64_t rows, int64_t cols,
                                                       uint16_t *__restrict__ out, int64_t out_rows,
                                                       int64_t ldo) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= out_rows * ldo) return;
  const int64_t c = idx / ldo, rr = idx % ldo;  // out[c][rr] = in[rr][c]
  out[idx] = (c < cols && rr < rows) ? in[rr * cols + c] : (uint16_t)0;
}

// out [RP][ldo] = bf16(scale * H^T) for H [M][r] fp32, zero outside.
__global__ __launch_bounds__(256) void k_scale_transpose_f32(const float *__restrict__ H, int64_t M, int r,
                                                             float scale, uint16_t *__restrict__ out, int RP,
                                                             int64_t ldo) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)RP * ldo) return;
  const int64_t j = idx / ldo, m = idx % ldo;
  out[idx] = (j < r && m < M) ? f32_to_bf16_bits(scale * H[m * r + j]) : (uint16_t)0;
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
  // Aim for >= ~1024 workgroups (4 per CU) with >= 4 contraction steps each.
  SplitPlan p;
  int64_t want = tiles >= 1024 ? 1 : ceil_div(1024, tiles);
  want = std::max<int64_t>(1, std::min<int64_t>(want, steps / 4 > 0 ? steps / 4 : 1));
  p.steps_per_split = (int)ceil_div(steps, want);
  p.splits = (int)ceil_div(steps, p.steps_per_split);
  return p;
}

hipError_t launch_nt_splitk(const uint16_t *P, int64_t rowsP, const uint16_t *Q, int rowsQ, int RP, int64_t lenC,
                            int64_t ld, const SplitPlan &sp, float *part, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(rowsP, 64), (unsigned)sp.splits);
  const bool vec_ok = (ld % 8) == 0;
  return dispatch_tj(RP, [&](auto tj) {
    QLORA_LAUNCH("k_nt_splitk", k_nt_splitk<decltype(tj)::value>, grid, dim3(256), 0, s, P, rowsP, Q, rowsQ, lenC, ld,
                       vec_ok, sp.steps_per_split, part);
    return hipGetLastError();
  });
}

hipError_t launch_tn_splitk(const uint16_t *P, int64_t M, int64_t D, const uint16_t *Qt, int64_t ldq, int RP,
                            const SplitPlan &sp, float *part, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(D, 64), (unsigned)sp.splits);
  const bool vec_ok = (D % 8) == 0;
  return dispatch_tj(RP, [&](auto tj) {
    QLORA_LAUNCH("k_tn_splitk", k_tn_splitk<decltype(tj)::value>, grid, dim3(256), 0, s, P, M, D, vec_ok, Qt, ldq,
                       sp.steps_per_split, part);
    return hipGetLastError();
  });
}

hipError_t launch_reduce_rows(const float *part, int S, int64_t R, int RP, int r, float scale, float *out_f32,
                              uint16_t *out_b, uint16_t *out_bt, int64_t ldt, hipStream_t s) {
  const int64_t total = (out_bt ? ldt : R) * RP;
  QLORA_LAUNCH("k_reduce_rows", k_reduce_rows, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, s, part, S, R, RP, r,
                     scale, out_f32, out_b, out_bt, ldt);
  return hipGetLastError();
}

hipError_t launch_reduce_cols(const float *part, int S, int64_t D, int RP, int r, bool transpose, uint16_t *out,
                              hipStream_t s) {
  QLORA_LAUNCH("k_reduce_cols", k_reduce_cols, dim3((unsigned)ceil_div((int64_t)r * D, 256)), dim3(256), 0, s, part, S, D,
                     RP, r, transpose, out);
  return hipGetLastError();
}

hipError_t launch_transpose_pad(const uint16_t *in, int64_t rows, int64_t cols, uint16_t *out, int64_t out_rows,
                                int64_t ldo, hipStream_t s) {
  QLORA_LAUNCH("k_transpose_pad", k_transpose_pad, dim3((unsigned)ceil_div(out_rows * ldo, 256)), dim3(256), 0, s, in, rows,
                     cols, out, out_rows, ldo);
  return hipGetLastError();
}

hipError_t launch_scale_transpose_f32(const float *H, int64_t M, int r, float scale, uint16_t *out, int RP,
                                      int64_t ldo, hipStream_t s) {
  QLORA_LAUNCH("k_scale_transpose_f32", k_scale_transpose_f32, dim3((unsigned)ceil_div((int64_t)RP * ldo, 256)), dim3(256), 0, s, H,
                     M, r, scale, out, RP, ldo);
  return hipGetLastError();
}

hipError_t launch_fill_zero_u16(uint16_t *p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  QLORA_LAUNCH("k_fill_zero_u16", k_fill_zero_u16, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace qlora

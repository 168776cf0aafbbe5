// nf4_gemv.hip -- the forward pass at small M (M <= 16): bound by reading the
// packed weight once from HBM.
//
// "QLoRA Paper Breakdown" sec. 4 Forward Pass, with the weights dequantized
// on the fly ("QLoRA, explained." step 4); at decode-sized M the multiply is
// a matrix-vector product, so the cost is streaming the packed codes and the
// two-level block constants (0.516 B per weight).
//
// k_gemv_nf4: one workgroup of eight waves per 64 weight rows; wave q takes
// the q-th eighth of the 256-wide K chunks (4 blocks per row).  Lane (li, g)
// of row tile rt (rows n0 + 16rt + li) owns block g of each chunk: it loads
// the block's 32 bytes of codes (two 16-byte loads), its scale code and group
// constant, and expands the 64 codes into eight BF16 MFMA A operands (256-entry
// table of level pairs, exactly as the standalone dequantization does).  X
// (M rows padded to 16 by out-of-range reads) is the B operand, read straight
// from global/L2: lane (li, g) takes X[li][256c + 64g + 8t .. +7] for
// sub-step t, the same k as its codes, and applies it to all four row tiles.
// No register prefetch: at ~120 VGPRs two workgroups (16 waves) fit per CU
// and every workgroup of a 65B-sized layer is resident at once.  The
// level-pair table has 32 copies, copy c in bank pair c (entry e at
// e*256 + 8c), so the 32 lanes of a half-wave never conflict on their random
// lookups; the table reads of a sub-step are issued before the arithmetic of
// the previous one.  The eight per-wave partial tiles are summed in LDS in
// wave order (deterministic; the table's space is reused), the LoRA term
// sum_j sH[m][j] B[n][j] is added in fp32, and Y is rounded to bf16 once.
#include "nf4_tile.h"

namespace qlora {
namespace {

constexpr int GW = 8;  // waves per workgroup: K split eight ways

__global__ __launch_bounds__(GW * 64) void k_gemv_nf4(Nf4View w, const uint16_t *__restrict__ X, int M,
                                                      const uint16_t *__restrict__ Bl, int r, int RP,
                                                      const uint16_t *__restrict__ sH, uint16_t *__restrict__ Y) {
  __shared__ __align__(16) float2 s_tab[256 * 32];  // 64 KB; later the reduction buffer
  f32x4_t(*red)[4][64] = reinterpret_cast<f32x4_t(*)[4][64]>(s_tab);  // [GW][4][64] = 32 KB
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t N = w.n, K = w.k, nkb = K / kBlock, nch = ceil_div_d(nkb, 4);
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int64_t cpw = ceil_div_d(nch, GW), c0 = min<int64_t>(nch, wave * cpw), c1 = min<int64_t>(nch, c0 + cpw);
  for (int i = tid; i < 256 * 32; i += GW * 64) {
    const int e = i >> 5;
    s_tab[i] = make_float2(__uint_as_float(kNF4Bits[e & 15]), __uint_as_float(kNF4Bits[e >> 4]));
  }
  const uint32_t tab_lane = (uint32_t)(lane & 31) * 8;  // byte offset of this lane's copy
  const char *tab = reinterpret_cast<const char *>(s_tab);
  const float offset = *w.offset;

  // Buffer resources: rows past N and blocks past k/64 fall outside the
  // ranges (per-lane offsets) and read zero; X rows past M likewise.
  const int64_t nrows = min<int64_t>(64, N - n0);
  const __amdgpu_buffer_rsrc_t crs = rsrc(w.packed + n0 * (K / 2), nrows * (K / 2));
  const __amdgpu_buffer_rsrc_t srs = rsrc(w.scale_code + n0 * nkb, nrows * nkb);
  const __amdgpu_buffer_rsrc_t grs = rsrc(w.group_amax, w.ng * 4);
  const __amdgpu_buffer_rsrc_t xrs = rsrc(X, (int64_t)M * K * 2);
  constexpr uint32_t kOut = 0x80000000u;

  f32x4_t acc[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // pair table

  for (int64_t c = c0; c < c1; ++c) {
    const int64_t kb = 4 * c + g;
    const bool bok = kb < nkb;
    u32x4_t code[4][2];  // [rt][half]: codes 64g + 32h .. +31 of row 16rt + li
    uint32_t sc[4];
    float ga[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int row = 16 * rt + li;
      const uint32_t co = bok ? (uint32_t)(row * (K / 2) + 128 * c + 32 * g) : kOut;
      code[rt][0] = __builtin_amdgcn_raw_buffer_load_b128(crs, co, 0, 0);
      code[rt][1] = __builtin_amdgcn_raw_buffer_load_b128(crs, co + 16, 0, 0);
      sc[rt] = __builtin_amdgcn_raw_buffer_load_b8(srs, bok ? (uint32_t)(row * nkb + kb) : kOut, 0, 0);
      ga[rt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             grs, (uint32_t)(((n0 + row) * nkb + kb) >> 8) * 4, 0, 0));
    }
    const uint32_t xo = (bok && li < M) ? (uint32_t)((li * K + 256 * c + 64 * g) * 2) : kOut;
    u32x4_t xf[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) xf[t] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xo + 16 * t, 0, 0);
    float s[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) s[rt] = block_scale(sc[rt], ga[rt], offset);
    // Piece (t, rt): codes 64g + 8t .. +7 of row tile rt.  Its table reads
    // are issued one piece ahead.
    float2 pq[2][4];
    auto look = [&](int p) {
      const int t = p >> 2, rt = p & 3;
      const uint32_t word = code[rt][t >> 2][t & 3];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pq[p & 1][i] = *reinterpret_cast<const float2 *>(tab + ((__builtin_amdgcn_ubfe(word, 8 * i, 8) << 8) | tab_lane));
    };
    look(0);
#pragma unroll
    for (int p = 0; p < 32; ++p) {
      const int t = p >> 2, rt = p & 3;
      if (p + 1 < 32) look(p + 1);
      __builtin_amdgcn_sched_barrier(0);
      u32x4_t a;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = bf16x2_rne(__fmul_rn(pq[p & 1][i].x, s[rt]), __fmul_rn(pq[p & 1][i].y, s[rt]));
      acc[rt] = mfma16(a, xf[t], acc[rt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // acc[rt][v] = partial C[n = n0 + 16rt + 4g + v][m = li]
  __syncthreads();  // every wave done with the table
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) red[wave][rt][lane] = acc[rt];
  __syncthreads();
  for (int e = tid; e < 4 * 64 * 4; e += GW * 64) {
    const int rt = e >> 8, l = (e >> 2) & 63, v = e & 3;
    const int64_t n = n0 + 16 * rt + 4 * (l >> 4) + v;
    const int m = l & 15;
    if (m >= M || n >= N) continue;
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < GW; ++q) sum += red[q][rt][l][v];
    float lo = 0.f;  // LoRA term: bf16 operands, exact products, fp32 sum
    for (int j = 0; j < r; ++j) {
      const float a = __uint_as_float((uint32_t)sH[(int64_t)m * RP + j] << 16);
      const float b = __uint_as_float((uint32_t)Bl[n * r + j] << 16);
      lo = __fmaf_rn(a, b, lo);
    }
    Y[(int64_t)m * N + n] = f32_to_bf16_bits(sum + lo);
  }
}

}  // namespace

hipError_t launch_fwd_gemv(const Nf4View &w, const uint16_t *X, int64_t M, const uint16_t *Bl, int r, int RP,
                           const uint16_t *sH, uint16_t *Y, hipStream_t s) {
  QLORA_LAUNCH("k_gemv_nf4", k_gemv_nf4, dim3((unsigned)ceil_div(w.n, 64)), dim3(GW * 64), 0, s, w, X, (int)M, Bl, r, RP,
               sH, Y);
  return hipGetLastError();
}

}  // namespace qlora

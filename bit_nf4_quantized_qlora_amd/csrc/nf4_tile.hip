// nf4_tile.hip -- the dense NF4 x BF16 tile kernel of the forward pass and of
// the input-gradient pass, and the block-scale pre-passes that feed it.
//
// "QLoRA Paper Breakdown" sec. 4: the forward multiplies X by the weights
// dequantized on the fly, and the backward pass needs dY W_hat through the
// same on-the-fly dequantization, never forming dL/dW ("QLoRA, explained."
// steps 4-5; "reading note": the multiply runs in 16 bits).  Both passes are
//   C[o][m] = sum_c A[o][c] B[m][c] + sum_j L[o][j] R[m][j],  out[m][o] = bf16(C[o][m])
//   forward:  o = n, c = k, A = W_hat,   B = X,  L = B_lora,    R = bf16(s H), out = Y
//   backward: o = k, c = n, A = W_hat^T, B = dY, L = A_lora^T, R = G,          out = dX
// on 256 (o) x 256 (m) tiles, one workgroup of four waves per tile.
//
// Wave w owns o-rows o0 + 64w .. +63 (four 16-row MFMA tiles rt) and all 256
// m (sixteen 16-column tiles ct): 256 fp32 accumulators per lane, pinned to
// AGPRs.  The A operand never exists as a BF16 tile: lane (li = lane & 15,
// g = lane >> 4) of row tile rt holds 16 NF4 codes of row o = o0+64w+16rt+li
// at contraction positions 16g .. 16g+15 of the current 64-wide step, and
// expands them in registers (256-entry table of level pairs, times the block
// scale, rounded to BF16 -- bit-identical to the standalone dequantization)
// straight into MFMA operands; sub-step t uses positions 16g+8t .. +7.  The B
// fragment of the same lane reads the same contraction positions, so the sum
// is unchanged.
//   forward:  the 16 codes are 8 consecutive bytes of weight row o (one
//             block, one scale), read from the staged code tile by ds_read_b64;
//   backward: they are one column k of 16 consecutive weight rows n, which
//             ds_read_b64_tr_b4 (a 16x16 nibble transpose across the 16 lanes
//             of a group) gathers from the staged code tile; each row has its
//             own block scale.
//
// Every operand streams global -> LDS by buffer loads that write LDS
// directly (no registers): the B tile one 64-wide step at a time, the packed
// codes 4 steps at a time (a "super-step": 256 rows x 128 B) together with
// their precomputed block scales (the scale-table jobs of jobs.hip).
//
// LDS: B tiles Bs0/Bs1 (2 x 32 KB), code tiles Wc0/Wc1 (2 x 32 KB), scale
// tiles Sc0/Sc1 (2 x 4 KB), pair table 2 KB.  Swizzles for 64 banks (256 B
// per bank row): in a B tile, row R (128 B) holds its 16-byte chunk c at
// chunk c ^ ((R >> 1) & 7), and each fragment is read as two 8-byte halves,
// the first being half g % 2, so every 32-lane half-wave read covers 32
// distinct bank pairs; code tiles use the same chunk swizzle.
//
// One wave per SIMD, so the wave's own instruction stream hides every
// latency: a step is eight "pairs" of 16 MFMAs (pair P: sub-step P/4, column
// tiles 4(P%4) .. +3), and after each MFMA the wave issues one small piece of
// other work for later pairs: a B fragment of pair P+1, a table read of
// expansion piece P+1, a quarter of the arithmetic of piece P, or (pair 6)
// the codes and scales of step kt+2.  Piece p covers row tile p % 4 and
// sub-step 1 (p < 4) or 0 (p >= 4) of step kt+1; sub-step-1 operands
// alternate between two register sets by step parity, sub-step-0 operands
// are rewritten after their last use in pair 3.
//
// Barrier B(kt) sits between pairs 6 and 7 of step kt: it waits for the B
// tile of step kt+1 (so pair 7 can already read the next step's first
// fragments) and for this wave's reads of Bs[kt % 2]; in pair 7, right after
// it, the B tile of step kt+2 is copied into Bs[kt % 2].  When kt % 4 == 0,
// pairs 0-2 copy the codes and scales of super-step kt/4 + 1 into the set of
// super-step kt/4 - 1, whose last register read was in step kt-3; that copy
// lands by B(kt+1) and is first read in pair 6 of step kt+2.  Copies go one
// per MFMA slot: issued back to back, the four waves' copies queue in the
// address unit and stall every wave's instruction stream.  The loop is
// unrolled by 8 steps so every buffer choice is a compile-time constant; the
// step count is rounded up to a multiple of 8, and steps past the end copy
// zeros for B (zero-length buffer resource) and have zero scales, so they add
// nothing.  A single loop with no tail also keeps the compiler from moving
// accumulators between register files right behind MFMAs it does not track.
//
// Every row-dependent offset goes in the per-lane VGPR offset, which the
// buffer range check covers: rows past M, N or the end of the weight read
// zero and never touch memory past the tensors.
#include "nf4_tile.h"

namespace qlora {
namespace {

constexpr int TO = kTileRows, TM = 256;  // tile: o rows x m rows
constexpr int kSup = kTileSup;           // steps per staged code chunk

// Output through LDS, once the main loop has drained (every copy landed,
// all waves past a barrier).  acc[rt][ct][v] = C[o][m] with o = ow + 16rt +
// 4g + v and m = m0 + 16ct + li.  Each wave writes its 64 o x 256 m block as
// bf16 into the four free 32 KB buffers (buffer q: tile rows m 64q .. +63, 512
// B per row, 16-byte chunk c of row r at c ^ (r & 15), so the 16 rows of one
// write land in distinct banks); then wave w stores tile rows 64w .. +63, two
// full 512-byte rows per instruction.
__device__ __forceinline__ void store_tile(const f32x4_t (&acc)[4][16], uint8_t *const (&buf)[4],
                                           uint16_t *__restrict__ out, int64_t NO, int64_t M, int64_t o0,
                                           int64_t m0, int wave) {
  const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ct = 0; ct < 16; ++ct)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const f32x4_t v = acc[rt][ct];
      const int c = 8 * wave + 2 * rt + (g >> 1);
      *reinterpret_cast<u32x2_t *>(buf[ct >> 2] + (16 * (ct & 3) + li) * 512 + ((c ^ li) << 4) + 8 * (g & 1)) =
          u32x2_t{bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3])};
    }
  __syncthreads();
  const uint8_t *src = buf[0];
#pragma unroll
  for (int q = 1; q < 4; ++q)
    if (wave == q) src = buf[q];
  const bool ovec = (NO & 7) == 0;
  const int c = lane & 31;
  const int64_t o = o0 + 8 * c;
#pragma unroll 4
  for (int i = 0; i < 32; ++i) {
    const int r = 2 * i + (lane >> 5);
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(src + r * 512 + ((c ^ (r & 15)) << 4));
    const int64_t m = m0 + 64 * wave + r;
    if (m < M && o < NO) {
      uint16_t *dst = out + m * NO + o;
      if (ovec) {
        *reinterpret_cast<u32x4_t *>(dst) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (o + e < NO) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

// Split-contraction output: the float32 partial tile of split `sidx`, in the
// tile's own register order (slot j = 16rt + ct of thread t at
// ((split * ntiles + tile) * 64 + j) * 256 + t), so each wave writes 1 KB
// contiguous per store; k_split_reduce sums the splits in order.
__device__ __forceinline__ void store_partial(const f32x4_t (&acc)[4][16], f32x4_t *__restrict__ part,
                                              int64_t slot) {
  f32x4_t *p = part + slot * 64 * 256 + threadIdx.x;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) p[(rt * 16 + ct) * 256] = acc[rt][ct];
}

// out = bf16 of the partial tiles summed in split order, one thread per
// float4 slot of the partial layout above.
__global__ __launch_bounds__(256) void k_split_reduce(const f32x4_t *__restrict__ part, int splits, int ntiles,
                                                      int tiles_o, int64_t M, int64_t NO,
                                                      uint16_t *__restrict__ out) {
  split_reduce_slot(part, splits, ntiles, tiles_o, M, NO, out, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// Grid: tiles x splits workgroups.  With splits > 1, workgroup (tile, s)
// runs contraction steps s*lsteps .. min(nk, (s+1)*lsteps) - 1 (lsteps a
// multiple of 8; split 0 also adds the LoRA term) and writes its float32
// partial tile to `part`; otherwise lsteps covers the whole contraction and
// the tile is rounded to bf16 into `out`.
//
// kW16 (forward only): the same kernel on weights already in BF16 (`Wb`
// [n][k] row-major, e.g. qlora_dequant_bf16's output) -- the 16-bit
// baseline the dequantization overhead is measured against.  The code
// buffers then hold one step of the BF16 weight tile each (256 rows x 128 B,
// the B tile's layout and swizzle), copied three steps ahead; an expansion
// piece becomes two 8-byte fragment reads (in the table-read slots) and four
// register moves (in the arithmetic slots), so the operands, their order and
// the result are bit for bit those of the NF4 kernel on the same W_hat.
template <bool kBwd, bool kW16 = false>
__global__ __launch_bounds__(256, 1) void k_nf4_tile(Nf4View w, const float *__restrict__ Sp,
                                                     const uint16_t *__restrict__ Bact, int64_t M,
                                                     const uint16_t *__restrict__ L, int lda, int RP,
                                                     const uint16_t *__restrict__ R, uint16_t *__restrict__ out,
                                                     int tiles_o, int splits, int lsteps,
                                                     f32x4_t *__restrict__ part, const uint16_t *__restrict__ Wb) {
  static_assert(!(kBwd && kW16), "the BF16-weight variant is forward only");
  __shared__ __align__(16) uint16_t Bs0[TM * 64];
  __shared__ __align__(16) uint16_t Bs1[TM * 64];
  __shared__ __align__(16) uint8_t Wc0[256 * 128];
  __shared__ __align__(16) uint8_t Wc1[256 * 128];
  __shared__ __align__(16) float Sc0[256 * kSup];
  __shared__ __align__(16) float Sc1[256 * kSup];
  __shared__ float2 s_pair[256];
  // wave is uniform across the wave; say so, or wave-dependent scalar
  // offsets would be made uniform with a per-lane loop
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Tiles in bands of ob o-tiles, m-major inside a band; each XCD takes a
  // contiguous run of that order (xcd_tile), so the tiles it holds form an
  // m x ob block and share both operand panels in its L2.
  const int ntiles = (int)gridDim.x / splits;
  const int lin = xcd_tile(blockIdx.x, gridDim.x);
  const int sidx = lin / ntiles;  // contraction split (split-major order)
  const int tile = lin - sidx * ntiles;
  const int tiles_m = ntiles / tiles_o;
  const int ob = (tiles_o + 1) / 2;
  const int band = tile / (ob * tiles_m), within = tile - band * ob * tiles_m;
  const int obw = min(ob, tiles_o - band * ob);  // the last band may be narrower
  const int to = band * ob + within % obw;
  const int64_t o0 = (int64_t)to * TO, m0 = (int64_t)(within / obw) * TM;
  const int64_t N = w.n, K = w.k;
  const int64_t NO = kBwd ? K : N, NC = kBwd ? N : K;  // output width, contraction length
  const int64_t ks0 = (int64_t)sidx * lsteps;                // first step of this split
  const int64_t nk = min<int64_t>(NC / kBlock - ks0, lsteps);  // 64-wide steps of this split
  const int64_t nsup_all = kBwd ? tile_bwd_nsup(N) : tile_fwd_nsup(K);
  const int64_t nsup = ceil_div_d(nk, kSup);  // super-steps of this split (ks0 % 8 == 0)
  const int64_t nk8 = ceil_div_d(nk, 8) * 8;  // steps run: whole 8-step rounds
  const int RPe = sidx == 0 ? RP : 0;         // the LoRA term goes into split 0 only
  if constexpr (!kW16) fill_pair_table(s_pair, tid, 256, w.codebook);

  // B rows m0 .. m0+255 (row stride NC): wave-instruction i fills LDS chunks
  // [512w + 64i, +64): row 64w + 8i + lane/8, physical chunk lane & 7, so the
  // logical chunk it copies depends on the parity of i.
  // (this split's contraction columns start ks0 * 64 elements into each row)
  const int bbytes = (int)(min<int64_t>(TM, M - m0) * NC * 2 - ks0 * 128);
  uint32_t bv[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    bv[par] = (uint32_t)(((64 * wave + (lane >> 3)) * NC + 8 * ((lane & 7) ^ (4 * par + (lane >> 4)))) * 2);
  // Instruction i (0..7) of the B-tile copy of step kt.
  auto bload = [&](int64_t kt, auto D, int i) {
    uint16_t *dst = decltype(D)::value ? Bs1 : Bs0;
    const __amdgpu_buffer_rsrc_t rs = rsrc(Bact + m0 * NC + ks0 * 64, kt < nk ? bbytes : 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(dst + (512 * wave + 64 * i) * 8), 16,
                                             bv[i & 1] + (uint32_t)(i * 16 * NC), (int)(kt * 128), 0, 0);
  };
  // kW16: instruction i (0..7) of the BF16 weight tile of step kt (rows o0
  // .. o0+255, row stride K), into code buffer D, the B tile's pattern.
  const int abytes = (int)(min<int64_t>(TO, N - o0) * NC * 2 - ks0 * 128);
  auto aload = [&](int64_t kt, auto D, int i) {
    uint16_t *dst = reinterpret_cast<uint16_t *>(decltype(D)::value ? Wc1 : Wc0);
    const __amdgpu_buffer_rsrc_t rs = rsrc(Wb + o0 * NC + ks0 * 64, kt < nk ? abytes : 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(dst + (512 * wave + 64 * i) * 8), 16,
                                             bv[i & 1] + (uint32_t)(i * 16 * NC), (int)(kt * 128), 0, 0);
  };
  // Code tile of a super-step: 256 rows x 128 B, same copy pattern and
  // swizzle.  Forward: row r = weight row o0 + r, bytes 128sp .. (4 steps of
  // k).  Backward: row r = weight row 256sp + r, bytes o0/2 .. (the tile's
  // 256 columns k).  Scales: 4 KB per super-step, 1 KB per wave.
  const int64_t kb2 = K / 2;  // packed bytes per weight row
  const uint8_t *wbase_g = kBwd ? w.packed + ks0 * 64 * kb2 : w.packed + o0 * kb2 + ks0 * 32;
  const int wbytes = (int)(kBwd ? (N - ks0 * 64) * kb2 : min<int64_t>(TO, N - o0) * kb2 - ks0 * 32);
  uint32_t wv[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    wv[par] = (uint32_t)((64 * wave + (lane >> 3)) * kb2 + (kBwd ? o0 / 2 : 0) +
                         16 * ((lane & 7) ^ (4 * par + (lane >> 4))));
  const float *Spt = Sp + ((int64_t)to * nsup_all + ks0 / kSup) * 256 * kSup;
  // Instruction i (0..8) of the code and scale copy of super-step sp: eight
  // for the codes, the last for the scales.
  auto wload = [&](int64_t sp, auto D, int i) {
    const bool real = sp < nsup;
    if (i < 8) {
      uint8_t *dst = decltype(D)::value ? Wc1 : Wc0;
      const __amdgpu_buffer_rsrc_t rs = rsrc(wbase_g, real ? wbytes : 0);
      const uint32_t spo = (uint32_t)(kBwd ? sp * 256 * kb2 : sp * 128);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(dst + (512 * wave + 64 * i) * 16), 16,
                                               wv[i & 1] + (uint32_t)(i * 8 * kb2) + spo, 0, 0, 0);
    } else {
      float *sdst = decltype(D)::value ? Sc1 : Sc0;
      const __amdgpu_buffer_rsrc_t ss = rsrc(Spt, real ? (int)(nsup * 256 * kSup * 4) : 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ss, (lds_ptr)(sdst + 64 * wave * kSup), 16,
                                               (uint32_t)(wave * 1024 + lane * 16), (int)(sp * 256 * kSup * 4), 0, 0);
    }
  };
  constexpr int kVmemW = kW16 ? 8 : 9;  // copy instructions per wave: code super-step / W16 step

  // Codes and scales of step s live in set s % 2 (q4 = s % 4 within its
  // super-step).  Forward: lane reads bytes 8g .. 8g+7 of its row's 32 bytes
  // of the step (chunk 2q4 + g/2, half g%2) and one scale per row tile.
  // Backward: lane (li, g) points at row 64q4 + 16g + li; the transposed read
  // returns for lane (li, g) column o0+64w+16rt+li of rows 64q4+16g .. +15
  // (chunk 2w + rt/2, half rt%2); the 16 row scales of block w are shared by
  // the four row tiles.
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  u32x2_t wcr[2][4];
  float sreg[2][kBwd ? 16 : 4];
  const int crow = kBwd ? 16 * g + li : 64 * wave + li;  // + 64q4 (bwd) / + 16rt (fwd)
  auto cread = [&](auto S, int half) {  // step with (step % 8) == S; row tiles 2half, 2half+1
    if constexpr (kW16) return;
    constexpr int s8 = decltype(S)::value, q4 = s8 & 3, d = s8 & 1;
    const uint8_t *wc = ((s8 >> 2) & 1) ? Wc1 : Wc0;
#pragma unroll
    for (int rt = 2 * half; rt < 2 * half + 2; ++rt) {
      if constexpr (kBwd) {
        const int off = (64 * q4 + crow) * 128 + (((2 * wave + (rt >> 1)) ^ (li >> 1)) << 4) + 8 * (rt & 1);
        const auto v = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t *)(wc + off));
        wcr[d][rt] = u32x2_t{(uint32_t)v[0], (uint32_t)v[1]};
      } else {
        const int off = (crow + 16 * rt) * 128 + (((2 * q4 + (g >> 1)) ^ (li >> 1)) << 4) + 8 * (g & 1);
        wcr[d][rt] = *reinterpret_cast<const u32x2_t *>(wc + off);
      }
    }
  };
  // Backward scales: register chunk a (4 floats) of lane (li, g) holds rows
  // 16g + 4(a ^ (g%2)) .. +3 -- the same half swap as the code bytes (tread).
  auto sread = [&](auto S, int half) {
    if constexpr (kW16) return;
    constexpr int s8 = decltype(S)::value, q4 = s8 & 3, d = s8 & 1;
    const float *sc = ((s8 >> 2) & 1) ? Sc1 : Sc0;
    if constexpr (kBwd) {
#pragma unroll
      for (int a = 2 * half; a < 2 * half + 2; ++a) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t *>(sc + wave * 256 + 64 * q4 + 16 * g + 4 * (a ^ (g & 1)));
#pragma unroll
        for (int e = 0; e < 4; ++e) sreg[d][4 * a + e] = v[e];
      }
    } else {
#pragma unroll
      for (int rt = 2 * half; rt < 2 * half + 2; ++rt) sreg[d][rt] = sc[(crow + 16 * rt) * kSup + q4];
    }
  };

  u32x4_t a0[4], a1[2][4];  // A operands: sub-step 0; sub-step 1 by step parity
  u32x4_t bq[2][4];         // B fragments of a pair, by pair parity
  float2 pq[2][4];          // table reads of an expansion piece, by piece parity
  u32x2_t aq[2][2];         // kW16: the two halves of a piece's fragment, by piece parity
  // Lanes of odd g hold their B fragment halves swapped (see bfrag), so
  // operand dword i takes code byte i ^ 2 there.
  uint32_t bsh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) bsh[i] = (uint32_t)(8 * (i ^ (2 * (g & 1))));
  // B fragment offsets (elements within a tile) of lane (li, g), sub-step t,
  // read i: row li, logical chunk 2g + t, 8-byte half i ^ (g % 2).
  uint32_t xb[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 2; ++i) xb[t][i] = (uint32_t)(li * 64 + (((2 * g + t) ^ (li >> 1)) << 3) + 4 * (i ^ (g & 1)));
  // Table read i of piece p from code set d into pq[p % 2][i].  kW16: reads
  // 0 and 1 are the two halves of the piece's fragment (row tile p % 4,
  // sub-step p < 4) from the weight tile in buffer d, at the B fragment's
  // offsets (same swizzle, same half order), so each lane holds exactly the
  // contraction positions its B fragment holds.
  auto tread = [&](int d, int p, int i) {
    if constexpr (kW16) {
      if (i < 2) {
        const uint16_t *ab = reinterpret_cast<const uint16_t *>(d ? Wc1 : Wc0);
        aq[p & 1][i] = *reinterpret_cast<const u32x2_t *>(ab + 4096 * wave + 1024 * (p & 3) + xb[p < 4 ? 1 : 0][i]);
      }
    } else {
      const uint32_t word = wcr[d][p & 3][p < 4 ? 1 : 0];
      pq[p & 1][i] = s_pair[__builtin_amdgcn_ubfe(word, bsh[i], 8)];
    }
  };
  // Quarter i of piece p's arithmetic (scales of set d); operands for a step
  // of parity e.
  auto tmath = [&](int d, int e, int p, int i) {
    if constexpr (kW16) {  // dword i of the fragment into its operand slot
      const uint32_t x = aq[p & 1][i >> 1][i & 1];
      if (p < 4) a1[e][p & 3][i] = x;
      else a0[p & 3][i] = x;
      return;
    }
    const float2 v = pq[p & 1][i];
    float sa, sb;
    if constexpr (kBwd) {
      const int t = p < 4 ? 1 : 0, base = 4 * (2 * t + (i >> 1)) + 2 * (i & 1);
      sa = sreg[d][base];
      sb = sreg[d][base + 1];
    } else {
      sa = sb = sreg[d][p & 3];
    }
    const uint32_t x = bf16x2_rne(__fmul_rn(v.x, sa), __fmul_rn(v.y, sb));
    if (p < 4) a1[e][p & 3][i] = x;
    else a0[p & 3][i] = x;
  };
  // B fragment (column tile ct, sub-step t) of lane (li, g): row 16ct + li,
  // logical chunk 2g + t, read as two 8-byte halves, the first being half
  // g % 2.  The row term 16ct*64 elements is an immediate.
  auto bfrag = [&](const uint16_t *bs, int P, int cc) -> u32x4_t {
    const int t = P >> 2, ct = 4 * (P & 3) + cc;
    const u32x2_t h0 = *reinterpret_cast<const u32x2_t *>(bs + xb[t][0] + 1024 * ct);
    const u32x2_t h1 = *reinterpret_cast<const u32x2_t *>(bs + xb[t][1] + 1024 * ct);
    return u32x4_t{h0[0], h0[1], h1[0], h1[1]};
  };

  f32x4_t acc[4][16];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Prologue: B of step 0 and super-step 0's codes landed; B of step 1 in
  // flight (super-step 1's codes follow in step 0's pairs 0-2); step 0
  // expanded; codes of step 1 in set 1; pair 0's fragments and piece 0's
  // table reads issued.
  //
  // The LoRA term comes first: C += L R^T over the padded rank in 64-wide
  // chunks, each chunk of R (rows m0 .. +255, row stride RP; columns past RP
  // and rows past M read zero) copied into Wc1 -- idle until step 0 copies
  // super-step 1 -- with the B-tile layout, and the matching L operands
  // (rows o, row stride lda) loaded straight into registers.  The first
  // chunk's loads go out before the copies of steps 0 and 1, so its MFMAs
  // wait only for them and run while the copies are in flight.
  const __amdgpu_buffer_rsrc_t rr = rsrc(R + m0 * RP, min<int64_t>(TM, M - m0) * RP * 2);
  uint16_t *rtile = reinterpret_cast<uint16_t *>(Wc1);
  const bool lvec = (lda % 8) == 0;
  u32x4_t la[4][2];
  auto lora_loads = [&](int jc) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 64 * wave + 8 * i + (lane >> 3);
      const int col = jc + 8 * ((lane & 7) ^ (4 * (i & 1) + (lane >> 4)));
      const uint32_t off = col < RP ? (uint32_t)((row * RP + col) * 2) : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_ptr)(rtile + (512 * wave + 64 * i) * 8), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        la[rt][t] = load8(L, lda, NO, lda, o0 + 64 * wave + 16 * rt + li, jc + 16 * g + 8 * t, lvec);
  };
  // bfrag hands odd-g lanes their two 8-byte halves swapped; swap the L
  // operand the same way so products pair up (after the loads have landed:
  // using a loaded value makes the compiler wait for it right there)
  auto lora_swap = [&]() {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        if (g & 1) la[rt][t] = u32x4_t{la[rt][t][2], la[rt][t][3], la[rt][t][0], la[rt][t][1]};
  };
  __syncthreads();  // pair table; Wc1 free
  if (RPe > 0) lora_loads(0);
#pragma unroll
  for (int i = 0; i < 8; ++i) bload(0, std::integral_constant<int, 0>(), i);
#pragma unroll
  for (int i = 0; i < kVmemW; ++i) {
    if constexpr (kW16) aload(0, std::integral_constant<int, 0>(), i);  // weight tile of step 0
    else wload(0, std::integral_constant<int, 0>(), i);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) bload(1, std::integral_constant<int, 1>(), i);
  {
    for (int jc = 0; jc < RPe; jc += 64) {
      if (jc == 0) {
        // the 8 + kVmemW + 8 copies issued after chunk 0's loads may stay in flight
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(8 + kVmemW + 8) : "memory");
      } else {
        lora_loads(jc);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      lora_swap();
      __syncthreads();
      // The MFMAs are inline asm, so the compiler does not pad the gap after
      // the VALU writes of the swap: keep those writes above this point and
      // add the wait states a VALU-written MFMA source needs.
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 4" ::: "memory");
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ct = 0; ct < 16; ++ct) {
          const u32x4_t b = bfrag(rtile, 4 * t + (ct >> 2), ct & 3);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) mfma16_acc(acc[rt][ct], la[rt][t], b);
        }
      __syncthreads();
    }
  }
  if constexpr (kW16) {
    // the LoRA chunks are done with Wc1: the weight tile of step 1 goes there
#pragma unroll
    for (int i = 0; i < 8; ++i) aload(1, std::integral_constant<int, 1>(), i);
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // step 0's copies landed (B and W of step 1 in flight)
  } else {
    // steps 0's copies landed everywhere (step 1's B may still be in flight)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  }
  __syncthreads();
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
  for (int cc = 0; cc < 4; ++cc) bq[0][cc] = bfrag(Bs0, 0, cc);
  if constexpr (kW16) {
    // step 1's tile landed and every wave is done reading step 0's: step 2's
    // tile goes into Wc0 (it lands by the first barrier of the loop)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) aload(2, std::integral_constant<int, 0>(), i);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) tread(1, 0, i);

  auto step = [&](int64_t kt, auto U) {
    constexpr int u = decltype(U)::value, j = u & 3, e = u & 1;
    const uint16_t *bs = e ? Bs1 : Bs0, *bn = e ? Bs0 : Bs1;
    constexpr int dc = (u + 1) & 1;  // code set of step kt+1 (expanded now)
#pragma unroll
    for (int P = 0; P < 8; ++P) {
      const int t = P >> 2, ct0 = 4 * (P & 3);
      if (P == 7) {
        // B(kt): the B tile of step kt+1 landed everywhere, every wave done
        // reading Bs[kt % 2]; then refill it with step kt+2.
        if constexpr (j == 0 && !kW16)
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kVmemW) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int cc = s >> 2, rt = s & 3;
        mfma16_acc(acc[rt][ct0 + cc], t ? a1[e][rt] : a0[rt], bq[P & 1][cc]);
        // Copies, one per slot, never in a burst (copies past the end read
        // zeros; their data is never used): in pair 7, after B(kt), the B
        // tile of step kt+2 into Bs[kt % 2]; when kt % 4 == 0, in pairs 0-2,
        // the codes and scales of super-step kt/4 + 1 into set (kt/4 + 1) % 2.
        if (P == 7 && (s & 1) == 0) bload(kt + 2, std::integral_constant<int, e>(), s >> 1);
        // kW16: the weight tile of step kt+3 into the buffer step kt+1's
        // pieces have finished reading (before B(kt))
        if constexpr (kW16)
          if (P == 7 && (s & 1) == 1) aload(kt + 3, std::integral_constant<int, (u + 3) & 1>(), s >> 1);
        if constexpr (j == 0 && !kW16) {
          if (P < 3 && s % 5 == 0 && 4 * P + s / 5 < kVmemW)
            wload((kt >> 2) + 1, std::integral_constant<int, ((u >> 2) + 1) & 1>(), 4 * P + s / 5);
        }
        if (s < 12) {
          const int q = s / 3, kind = s % 3;
          if (kind == 0) {  // B fragment q of the next pair
            if (P < 7) bq[(P + 1) & 1][q] = bfrag(bs, P + 1, q);
            else bq[0][q] = bfrag(bn, 0, q);
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
  // (inside the loop every MFMA source is written at least a pair ahead)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 4" ::: "memory");
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
  if (splits > 1) {
    store_partial(acc, part, (int64_t)sidx * ntiles + (m0 / TM) * tiles_o + to);
    return;
  }
  uint8_t *const bufs[4] = {reinterpret_cast<uint8_t *>(Bs0), reinterpret_cast<uint8_t *>(Bs1), Wc0, Wc1};
  store_tile(acc, bufs, out, NO, M, o0, m0, wave);
}

}  // namespace

size_t tile_scales_bytes(int64_t n, int64_t k) {
  const size_t f = (size_t)ceil_div(n, TO) * tile_fwd_nsup(k) * 256 * kSup;
  const size_t b = (size_t)ceil_div(k, TO) * tile_bwd_nsup(n) * 256 * kSup;
  return std::max(f, b) * sizeof(float);
}

// n % 64 == 0 (whole 64-row steps), the packed weight below 2^31 bytes and a
// 256-row dY tile (512 n bytes) below 2^31 bytes: 32-bit buffer offsets.
bool bwd_tiles_supported(int64_t n, int64_t k) {
  return n % 64 == 0 && n * (k / 2) < (int64_t(1) << 31) && 512 * n < (int64_t(1) << 31);
}

// Contraction splits of a tile launch.  Cost in units of one 64-wide step of
// a tile (~1.6 us): rounds of 256 workgroups x (steps per split + ~4 for the
// prologue and epilogue), plus, when split, the float32 partials written
// and read back once (~16 MB per unit: the writes overlap other workgroups'
// steps and the reads mostly hit the last-level cache; measured on the 4096
// and 8192 square layers at M = 512) and the reduction launch (~2 units).
// Only launches with too few tiles to fill the 256 CUs gain; the others
// stay at one split.
TileSplit plan_tile_split(int64_t tiles, int64_t nk, int64_t M, int64_t NO) {
  (void)M;
  (void)NO;
  TileSplit best;
  best.splits = 1;
  best.lsteps = (int)std::max<int64_t>(8, ceil_div(nk, 8) * 8);
  if (nk <= 8 || tiles < 1) return best;  // nothing to split
  auto cost = [&](int64_t S, int64_t L) {
    const double rounds = (double)ceil_div(tiles * S, 256);
    const double red = S > 1 ? 2.0 * S * tiles * 65536.0 * 4.0 / 16e6 + 2.0 : 0.0;
    return rounds * (double)(L + 4) + red;
  };
  double bc = cost(1, best.lsteps);
  for (int64_t want = 2; want <= 16; ++want) {
    const int64_t L = ceil_div(ceil_div(nk, want), 8) * 8;
    const int64_t S = ceil_div(nk, L);
    if (S < 2) continue;
    const double c = cost(S, L);
    if (c < 0.97 * bc) {
      bc = c;
      best.splits = (int)S;
      best.lsteps = (int)L;
    }
  }
  return best;
}

TileSplit plan_fwd_tiles(int64_t M, int64_t n, int64_t k) {
  return plan_tile_split(ceil_div(n, TO) * ceil_div(M, TM), k / kBlock, M, n);
}

TileSplit plan_dx_tiles(int64_t M, int64_t n, int64_t k) {
  return plan_tile_split(ceil_div(k, TO) * ceil_div(M, TM), n / kBlock, M, k);
}

size_t tile_fwd_partial_bytes(int64_t M, int64_t n, int64_t k) {
  const TileSplit f = plan_fwd_tiles(M, n, k);
  return f.splits > 1 ? (size_t)f.splits * ceil_div(n, TO) * ceil_div(M, TM) * 65536 * 4 : 0;
}

size_t tile_dx_partial_bytes(int64_t M, int64_t n, int64_t k) {
  if (!bwd_tiles_supported(n, k)) return 0;
  const TileSplit b = plan_dx_tiles(M, n, k);
  return b.splits > 1 ? (size_t)b.splits * ceil_div(k, TO) * ceil_div(M, TM) * 65536 * 4 : 0;
}

namespace {
hipError_t reduce_splits(const char *name, const TileSplit &sp, int tiles_o, int tiles_m, int64_t M, int64_t NO,
                         const float *tpart, uint16_t *out, hipStream_t s) {
  const int ntiles = tiles_o * tiles_m;
  QLORA_LAUNCH(name, k_split_reduce, dim3((unsigned)(ntiles * 64)), dim3(256), 0, s,
               reinterpret_cast<const f32x4_t *>(tpart), sp.splits, ntiles, tiles_o, M, NO, out);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fwd_tiles(const Nf4View &w, float *scales, const uint16_t *X, int64_t M, const uint16_t *Bl, int r,
                            int RP, const uint16_t *sH, uint16_t *Y, float *tpart, hipStream_t s) {
  const int tiles_o = (int)ceil_div(w.n, TO), tiles_m = (int)ceil_div(M, TM);
  const TileSplit sp = plan_fwd_tiles(M, w.n, w.k);
  QLORA_LAUNCH("k_fwd_nf4", k_nf4_tile<false>, dim3((unsigned)(tiles_o * tiles_m * sp.splits)), dim3(256), 0, s, w,
               scales, X, M, Bl, r, RP, sH, Y, tiles_o, sp.splits, sp.lsteps, reinterpret_cast<f32x4_t *>(tpart),
               nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp.splits == 1) return e;
  return reduce_splits("k_split_reduce", sp, tiles_o, tiles_m, M, w.n, tpart, Y, s);
}

#ifdef QLORA_PROFILE
hipError_t launch_fwd_tiles_bf16w(const uint16_t *Wb, int64_t n, int64_t k, const uint16_t *X, int64_t M,
                                  const uint16_t *Bl, int r, int RP, const uint16_t *sH, uint16_t *Y, hipStream_t s) {
  Nf4View w{};
  w.n = n;
  w.k = k;
  const int tiles_o = (int)ceil_div(n, TO), tiles_m = (int)ceil_div(M, TM);
  const int lsteps = (int)(ceil_div(k / kBlock, 8) * 8);  // one split
  QLORA_LAUNCH("k_fwd_bf16w", (k_nf4_tile<false, true>), dim3((unsigned)(tiles_o * tiles_m)), dim3(256), 0, s, w,
               nullptr, X, M, Bl, r, RP, sH, Y, tiles_o, 1, lsteps, nullptr, Wb);
  return hipGetLastError();
}
#endif

SmallJob job_split_reduce(const TileSplit &sp, int tiles_o, int tiles_m, int64_t M, int64_t NO, const float *tpart,
                          uint16_t *out) {
  SmallJob j;
  j.kind = kJobSplitReduce;
  j.count = sp.splits > 1 ? (int64_t)tiles_o * tiles_m * 64 * 256 : 0;
  j.in = tpart;
  j.out = out;
  j.a = M;
  j.b = NO;
  j.c = (int64_t)tiles_o * tiles_m;
  j.i = sp.splits;
  j.j = tiles_o;
  return j;
}

hipError_t launch_bwd_dx_tiles(const Nf4View &w, float *scales, const uint16_t *dY, int64_t M, const uint16_t *At,
                               int RP, const uint16_t *Gb, uint16_t *dX, float *tpart, hipStream_t s,
                               SmallJob *split_job) {
  const int tiles_o = (int)ceil_div(w.k, TO), tiles_m = (int)ceil_div(M, TM);
  const TileSplit sp = plan_dx_tiles(M, w.n, w.k);
  QLORA_LAUNCH("k_bwd_dx_nf4", k_nf4_tile<true>, dim3((unsigned)(tiles_o * tiles_m * sp.splits)), dim3(256), 0, s,
               w, scales, dY, M, At, RP, RP, Gb, dX, tiles_o, sp.splits, sp.lsteps,
               reinterpret_cast<f32x4_t *>(tpart), nullptr);
  hipError_t e = hipGetLastError();
  if (split_job) {
    *split_job = job_split_reduce(sp, tiles_o, tiles_m, M, w.k, tpart, dX);
    return e;
  }
  if (e != hipSuccess || sp.splits == 1) return e;
  return reduce_splits("k_split_reduce", sp, tiles_o, tiles_m, M, w.k, tpart, dX, s);
}

}  // namespace qlora

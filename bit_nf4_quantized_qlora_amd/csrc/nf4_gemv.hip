// nf4_gemv.hip -- the forward pass at small M (M <= 16): bound by reading the
// packed weight once from HBM.
//
// "QLoRA Paper Breakdown" sec. 4 Forward Pass, with the weights dequantized
// on the fly ("QLoRA, explained." step 4); at decode-sized M the multiply is
// a matrix-vector product, so the cost is streaming the packed codes and the
// two-level block constants (0.516 B per weight).
//
// Two launches:
//   k_gemv_nf4    partial sums of Y = X W_hat^T per workgroup and row group,
//                 and partial sums of H = X A^T over 512-wide K slices;
//   k_gemv_finish Y = bf16(sum of the partials + bf16(s H) B^T), H (fp32,
//                 the optional output).
//
// k_gemv_nf4 runs one 1024-thread workgroup per CU.  The weight rows are cut
// into groups of 256 (16 row tiles of 16) and each row into 64-wide blocks;
// the (group, block) pairs, taken group-major, are split into G equal
// contiguous ranges, one per workgroup (stream-K), so every CU streams the
// same number of bytes whatever the shape.  All 16 waves walk the
// workgroup's range together, wave w on row tile w of the current group, and
// write one partial per row group they touch.
//
// Per block the MFMA takes X as its A operand (rows m < M, the rest zero) and
// the weights as its B operand (columns = the 16 rows of the tile); a lane's
// four accumulators then belong to one weight row, whose block scale it
// computes exactly as the standalone dequantization does (E4M3 decode from
// a 256-entry LDS table, then the two separately rounded operations).  The
// weights are bf16(fp32(q * s)), bit for bit the dequantized BF16 weights:
// one LDS read of a level pair per packed byte from a 256-entry table with
// 32 copies (entry e of copy c at byte 256e + 8c, copy = lane % 32, so no
// half-wave read ever conflicts), addressed by a single byte permute of the
// code byte and the lane's offset.  Blocks go in pairs: lane (li, g) holds
// the 16 code bytes at byte 16g of row li's 64 bytes of the pair (block g/2,
// positions 32(g % 2) .. +31 of it; MFMA t takes bytes 4t .. 4t+3), so one
// load instruction reads 64 contiguous bytes of each of 16 rows and a lane
// needs one block scale per pair; codes are fetched 4 pairs ahead.  X is
// staged in LDS for the whole range, one 272-byte row per (pair, m), so X
// and the weights meet in the same order.
//
// Single-level weights (a float32 absmax per block, no double quantization)
// take the same kernel with s_b = absmax_b read four blocks per 16-byte load
// in place of the scale-code word, E4M3 table and group constants.
//
// H: workgroup t < nh takes rank tile t % (RP/16) and K slice t / (RP/16)
// (512 wide, 32 per wave); its operands are loaded before anything else so
// their latency hides under the table fill, one MFMA per wave, and the 16
// wave results are summed in LDS after the main loop.  k_gemv_finish sums
// the slices in order, adds the partial sums of each row group in workgroup
// order and the LoRA term (bf16 operands, exact products, fp32 sum), and
// rounds Y to bf16 once.
#include "nf4_tile.h"

namespace qlora {
namespace {

constexpr int kGvWaves = 16;               // waves per workgroup = row tiles per group
constexpr int kGvRows = 16 * kGvWaves;     // weight rows per row group
constexpr int kLdsAll = 160 * 1024;        // LDS of one workgroup
constexpr int kGvP = 4;                    // pairs of blocks of codes in flight per lane
constexpr int kLdsTab = 256 * 256;         // level-pair table, 32 copies
constexpr int kLdsDec = 256 * 4;           // E4M3 decode table
constexpr int kLdsVar = kLdsAll - kLdsTab - kLdsDec - 128 - 16;  // group constants + staged X
constexpr int kHSlice = 32 * kGvWaves;     // K per H slice: one 32-deep MFMA per wave
constexpr int kMaxG = 4096;                // most workgroups
constexpr int kXRow = 272;                 // staged X row: one pair of blocks (128 bf16) + 16 B of padding
constexpr int kXPer = 6;                   // staged 16-byte X chunks per thread (covers kLdsVar / kXRow rows)
constexpr int kGaPer = 2;                  // group constants per thread loaded ahead of the table fill

struct GemvPlan {
  int64_t nkb = 0, ngroups = 0, T = 0;  // blocks per row, row groups, (group, block) pairs
  int G = 0;                            // workgroups
  int seg = 1;                          // most row groups one workgroup touches
  int maxcov = 1;                       // most workgroups covering one row group
  bool sparse = false;                  // some workgroups have empty ranges
  int nht = 0, nh = 0;                  // rank tiles of 16; H slices x rank tiles
  int xoff = 0;                         // byte offset of the staged X in the variable area
  int q4 = 1;                           // ranges start on multiples of q4 blocks (4 if nkb % 4 == 0)
};

GemvPlan gemv_plan(int64_t M, int64_t n, int64_t k, int RP) {
  GemvPlan p;
  p.nkb = k / kBlock;
  p.ngroups = ceil_div(n, kGvRows);
  p.T = p.ngroups * p.nkb;
  p.nht = RP / 16;
  p.nh = (int)(ceil_div(k, kHSlice) * p.nht);
  // A row group's 256 x nkb blocks use exactly nkb group constants (one per
  // 256 consecutive blocks, rows laid end to end); a workgroup stages those
  // of the row groups its range touches, then its X columns.
  p.q4 = 4;  // needs nkb % 4 == 0 (small_m_supported)
  auto fit = [&](int64_t G) {
    int64_t seg = 1, nbmax = 0;
    for (int64_t i = 0; i < G; ++i) {
      const int64_t b0 = p.q4 * (i * (p.T / p.q4) / G), b1 = p.q4 * ((i + 1) * (p.T / p.q4) / G);
      if (b1 > b0) seg = std::max<int64_t>(seg, (b1 - 1) / p.nkb - b0 / p.nkb + 1);
      nbmax = std::max<int64_t>(nbmax, b1 - b0);
    }
    p.seg = (int)seg;
    p.xoff = (int)align_up((size_t)seg * p.nkb * 4, 16);
    return p.xoff + nbmax / 2 * M * kXRow <= kLdsVar;
  };
  // one workgroup per CU (more only if the staged X or the H slices need
  // them), never more than there are blocks or H slices to take
  int64_t G = std::max<int64_t>(std::min<int64_t>(256, p.T / p.q4), p.nh);
  while (G < kMaxG && !fit(G)) G = std::min<int64_t>(G + 256, kMaxG);
  p.G = fit(G) ? (int)G : kMaxG + 1;  // no fit: small_m_supported says no
  // partial sums are kept per (row group, covering workgroup): workgroup
  // q's range starts at block 4 floor(q (T/4) / G), so block b lies in
  // workgroup ((b/4 + 1) G - 1) / (T/4)
  const int64_t T4 = p.T / 4;
  p.sparse = p.G > T4;
  for (int64_t gr = 0; gr < p.ngroups && p.G <= kMaxG; ++gr) {
    const int64_t wlo = ((gr * p.nkb / 4 + 1) * p.G - 1) / T4, whi = ((((gr + 1) * p.nkb - 1) / 4 + 1) * p.G - 1) / T4;
    p.maxcov = (int)std::max<int64_t>(p.maxcov, whi - wlo + 1);
  }
  return p;
}

struct SmallWs {
  GemvPlan p;
  size_t h_off, part_off, total;
};

SmallWs small_ws_layout(int64_t M, int64_t n, int64_t k, int RP) {
  SmallWs l;
  l.p = gemv_plan(M, n, k, RP);
  l.h_off = 0;
  l.part_off = align_up((size_t)(l.p.nh / l.p.nht) * M * RP * sizeof(float), 256);
  l.total = l.part_off + (size_t)l.p.ngroups * l.p.maxcov * M * kGvRows * sizeof(float);
  return l;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// kSingle: single-level block constants (s_b = absmax_b, a float32 per
// block) instead of the double-quantized E4M3 codes, group constants and
// offset; four blocks' constants (two pairs) per 16-byte load.
template <bool kSingle>
__global__ __launch_bounds__(1024, 1) void k_gemv_nf4(Nf4View w, const uint16_t *__restrict__ X, int M,
                                                      const uint16_t *__restrict__ A, int r, int RP,
                                                      float *__restrict__ hpart, float *__restrict__ part,
                                                      int T4, int G, int gq, int grem, int seg, int maxcov, int nh,
                                                      int nht, int xoff_b) {
  // LDS: level-pair table (64 KB, first so its reads need no base add),
  // E4M3 decode table (1 KB), a zero row, then the group constants of the
  // row groups the range touches and the staged X.
  __shared__ __align__(16) uint8_t lds[kLdsAll];
  float2 *s_tab = reinterpret_cast<float2 *>(lds);
  float *s_dec = reinterpret_cast<float *>(lds + kLdsTab);
  constexpr int kZeroOff = kLdsTab + kLdsDec, kMiscOff = kZeroOff + 128, kGaOff = kMiscOff + 16;
  float *s_ga = reinterpret_cast<float *>(lds + kGaOff);
  const int xbase = kGaOff + xoff_b;
  uint8_t *s_x = lds + xbase;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t N = w.n, K = w.k, kb2 = K / 2;
  const int nkb = (int)(K / kBlock);
  const int wg = blockIdx.x;
  // range [b0, b1) = 4 floor(wg (T/4) / G) .. with T/4 = gq G + grem, in
  // 32-bit arithmetic (wg grem < 2^24); every wave of the 16 computes these
  // scalars, so they are kept cheap
  const int b0 = 4 * (wg * gq + (int)(((uint32_t)wg * (uint32_t)grem) / (uint32_t)G));
  const int b1 = 4 * ((wg + 1) * gq + (int)(((uint32_t)(wg + 1) * (uint32_t)grem) / (uint32_t)G));
  const int nb = b1 - b0;
  const int gfirst = b0 / nkb;
  const int lkb0 = b0 - gfirst * nkb;

  // Global loads go out first: the X columns and group constants the range
  // stages into LDS (small, so they return quickly), the H slice operands
  // and the scalar offset, then the first pairs of codes and scale words.
  // The table fill runs while they are in flight, and waiting for the staged
  // values leaves the code loads in flight.
  constexpr uint32_t kOut = 0x80000000u;
  // X columns of the range: staged row P = ip*M + m holds X[m][64 kb(2ip) ..
  // +127] (the pair's two blocks) at P * 272 (16 B of padding per row): the
  // 16 lanes of one read (consecutive rows, one chunk) then hit 16 distinct
  // bank groups, and a lane's four chunks of a pair are fixed offsets from
  // one address.
  // The LDS plan keeps nb * M * 8 <= kXPer * 1024.
  const int nxc = nb * M * 8;
  const __amdgpu_buffer_rsrc_t xrs = rsrc(X, (int64_t)M * K * 2);
  const uint32_t inv_m = (65536u + (uint32_t)M - 1) / (uint32_t)M;  // R / M = (R inv_m) >> 16 for R < 768, M <= 16
  // (a wave whose chunks all lie past the end issues no load: the address
  // unit is the prologue's bottleneck when 16 waves start at once)
  u32x4_t xv[kXPer];
#pragma unroll
  for (int u = 0; u < kXPer; ++u) {
    const int c = tid + 1024 * u;
    xv[u] = u32x4_t{0u, 0u, 0u, 0u};
    if (64 * wave + 1024 * u < nxc) {
      const int ch = c & 15, R = c >> 4, ip = (int)(((uint32_t)R * inv_m) >> 16), m = R - ip * M;
      int kb = lkb0 + 2 * ip;
      while (kb >= nkb) kb -= nkb;
      xv[u] = __builtin_amdgcn_raw_buffer_load_b128(
          xrs, c < nxc ? (uint32_t)((m * K + kb * kBlock + 8 * ch) * 2) : kOut, 0, 0);
    }
  }
  // group constants of the touched row groups: s_ga[t] = group_amax[gfirst*nkb + t]
  // (past the last group: zero, from the buffer range)
  const int64_t gi0 = (int64_t)gfirst * nkb;
  const int nga = kSingle ? 0 : seg * nkb;
  float gv[kGaPer];
#pragma unroll
  for (int u = 0; u < kGaPer; ++u) gv[u] = 0.f;
  if constexpr (!kSingle) {
    const __amdgpu_buffer_rsrc_t grs = rsrc(w.group_amax + gi0, (w.ng - gi0) * 4);
#pragma unroll
    for (int u = 0; u < kGaPer; ++u) {
      const int t = tid + 1024 * u;
      if (64 * wave + 1024 * u < nga)
        gv[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(grs, t < nga ? (uint32_t)t * 4 : kOut, 0, 0));
    }
  }

  // H slice operands: X rows li < M and A rows 16 jt + li < r at
  // k = 512 ks + 32 wave + 8g .. +7 (zero outside).
  const bool hwork = wg < nh;
  const int jt = wg % nht, ks = wg / nht;
  u32x4_t hx = {0u, 0u, 0u, 0u}, ha = {0u, 0u, 0u, 0u};
  if (hwork) {
    const int64_t kh = (int64_t)ks * kHSlice + 32 * wave + 8 * g;
    const int j = 16 * jt + li;
    const bool kin = hwork && kh < K;
    const __amdgpu_buffer_rsrc_t ar = rsrc(A, (int64_t)r * K * 2);
    hx = __builtin_amdgcn_raw_buffer_load_b128(xrs, kin && li < M ? (uint32_t)((li * K + kh) * 2) : kOut, 0, 0);
    ha = __builtin_amdgcn_raw_buffer_load_b128(ar, kin && j < r ? (uint32_t)((j * K + kh) * 2) : kOut, 0, 0);
  }
  float offset = 0.f;
  if constexpr (!kSingle) offset = *w.offset;

  // Per-lane streams (32-bit offsets): the codes of a pair of blocks of row
  // n, a word of four scale codes per two pairs, and the blocks' group
  // constants.  Rows past N read zero and give partial sums that are never
  // used; loads past the workgroup's last block take an out-of-range offset
  // (no memory traffic).
  const __amdgpu_buffer_rsrc_t crs = rsrc(w.packed, N * kb2);
  const __amdgpu_buffer_rsrc_t srs = kSingle ? rsrc(w.absmax, w.nb * 4) : rsrc(w.scale_code, w.nb);
  const int nrow = 16 * wave + li;  // row within the group
  const int nkb32 = nkb;
  const int hb = g >> 1;  // which block of a pair this lane's codes come from
  int lkb = lkb0;
  uint32_t lco = (uint32_t)((gfirst * kGvRows + nrow) * kb2 + lkb * 32 + 16 * g);
  uint32_t lbi = (uint32_t)((gfirst * kGvRows + nrow) * nkb + lkb);
  const uint32_t gstep_c = (uint32_t)(kGvRows * kb2 - nkb * 32), gstep_b = (uint32_t)(kGvRows * nkb - nkb);
  // codes of a pair of blocks: lane (li, g) takes the 16 bytes at 16g of the
  // row's 64 bytes (block hb, contraction positions 32(g & 1) .. +31), so a
  // wave instruction reads 64 contiguous bytes of each of its 16 rows
  u32x4_t cq[kGvP];
  auto load = [&](int slot, bool real) {
    cq[slot] = __builtin_amdgcn_raw_buffer_load_b128(crs, real ? lco : kOut, 0, 0);
    lco += 64;
    if ((lkb += 2) == nkb32) {
      lkb = 0;
      lco += gstep_c;
    }
  };
  // Scale codes four blocks (two pairs) per load (ranges and row groups
  // start on multiples of 4 blocks, and nkb % 4 == 0): word w of the row's
  // codes, all four lanes of a row reading the same word; two in flight.
  // (kSingle: the four blocks' float32 constants, 16 bytes, in scw4.)
  uint32_t scw[2];
  u32x4_t scw4[2];
  int skb = lkb;
  auto sload = [&](int slot, bool real) {
    if constexpr (kSingle)
      scw4[slot] = __builtin_amdgcn_raw_buffer_load_b128(srs, real ? lbi * 4u : kOut, 0, 0);
    else
      scw[slot] = __builtin_amdgcn_raw_buffer_load_b32(srs, real ? lbi : kOut, 0, 0);
    lbi += 4;
    if ((skb += 4) == nkb32) {
      skb = 0;
      lbi += gstep_b;
    }
  };
  sload(0, 0 < nb);
  sload(1, 4 < nb);
#pragma unroll
  for (int j = 0; j < kGvP; ++j) load(j, 2 * j < nb);

  // Level-pair table: entry e = {q[e & 15], q[e >> 4]} (low nibble = first
  // weight), copy c at byte 256e + 8c.  Wave w writes entries 16w .. 16w+15,
  // so q[e >> 4] is wave-uniform and q[e & 15] one of two constants: no
  // per-lane loads of the codebook (they would wait behind the loads above).
  {
    const int cb = w.codebook;
    const float qhi = __uint_as_float(codebook_level_bits(cb, wave));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = 16 * wave + 2 * i + (lane >> 5), c = lane & 31;
      const uint32_t hi_half = 0u - (uint32_t)(lane >> 5);  // all ones for lanes 32..63
      const uint32_t q0 = codebook_level_bits(cb, 2 * i), q1 = codebook_level_bits(cb, 2 * i + 1);
      const float qlo = __uint_as_float((q0 & ~hi_half) | (q1 & hi_half));
      s_tab[e * 32 + c] = make_float2(qlo, qhi);
    }
  }
  if (!kSingle && tid < 256) s_dec[tid] = e4m3_decode((uint32_t)tid);
  if (tid < 8) *reinterpret_cast<u32x4_t *>(lds + kZeroOff + 16 * tid) = u32x4_t{0u, 0u, 0u, 0u};
  // this workgroup's partial slot in its first row group: block b lies in
  // workgroup ((b/4 + 1) G - 1) / (T/4), so the group's first covering
  // workgroup is that of its block 0 (in later row groups of the range this
  // workgroup is the first); one 64-bit division, by one thread
  if (tid == 0)
    *reinterpret_cast<int *>(lds + kMiscOff) =
        wg - (int)((((int64_t)gfirst * nkb / 4 + 1) * G - 1) / T4);
#pragma unroll
  for (int u = 0; u < kXPer; ++u) {
    const int c = tid + 1024 * u;
    const int ch = c & 15, R = c >> 4;
    if (c < nxc) *reinterpret_cast<u32x4_t *>(s_x + R * kXRow + (ch << 4)) = xv[u];
  }
#pragma unroll
  for (int u = 0; u < kGaPer; ++u)
    if (tid + 1024 * u < nga) s_ga[tid + 1024 * u] = gv[u];
  for (int t = tid + 1024 * kGaPer; t < nga; t += 1024)  // very long rows only
    s_ga[t] = gi0 + t < w.ng ? w.group_amax[gi0 + t] : 0.f;
  __syncthreads();  // table and X staged

  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  const f32x4_t hacc = mfma16(hx, ha, zero);  // C[m = 4g+v][j = 16 jt + li]

  const char *tab = reinterpret_cast<const char *>(s_tab);
  const uint32_t lane_off = (uint32_t)(lane & 31) * 8;
  // X fragment of a pair for MFMA t: staged row ip*M + li, chunk 4g + t, at
  // xo + 16t (lanes li >= M read the zero row, which takes no step).
  const bool xreal = li < M;
  const uint32_t xo = xreal ? (uint32_t)(xbase + li * kXRow + 64 * g) : (uint32_t)kZeroOff;
  const uint32_t xstep = xreal ? (uint32_t)M * kXRow : 0u;
  uint32_t xoff = 0;
  // scale code byte of this lane's block in the word: 2(ip & 1) + hb
  const uint32_t ssh0 = 8u * hb, ssh1 = 16u + 8u * hb;
  // block index n*nkb + kb of this lane's block of the current pair; its
  // group constant is s_ga[(cbi >> 8) - gfirst*nkb]
  uint32_t cbi = (uint32_t)((gfirst * kGvRows + nrow) * nkb + (b0 - gfirst * nkb) + hb);
  const uint32_t ga_base = (uint32_t)kGaOff - (uint32_t)(gfirst * nkb) * 4;

  // partial slot of (row group gr, covering workgroup k = wg - first
  // covering workgroup): [(gr * maxcov + k) * M + m] * 256 + row
  int kslot = *reinterpret_cast<const int *>(lds + kMiscOff);
  int64_t cgr = gfirst;
  int ckb = lkb0;
  const int np = nb >> 1;
  f32x4_t acc = zero;
  // The loop leaves after the range's last pair (a uniform branch), so no
  // wave computes pairs it would not store; the codes and scale words loaded
  // ahead past the end take out-of-range offsets and are never used.
  for (int p0 = 0; p0 < np; p0 += kGvP) {
#pragma unroll
    for (int q = 0; q < kGvP; ++q) {
      const int ip = p0 + q;
      float sd = 0.f, ga = 0.f, s1 = 0.f;
      if constexpr (kSingle) {  // this lane's block: 2(ip & 1) + hb of the four
        const u32x4_t v = scw4[(q >> 1) & 1];
        s1 = __uint_as_float(hb ? v[2 * (q & 1) + 1] : v[2 * (q & 1)]);
      } else {
        const uint32_t sc = (scw[(q >> 1) & 1] >> ((q & 1) ? ssh1 : ssh0)) & 0xFFu;
        sd = s_dec[sc];
      }
      if (q & 1) sload((q >> 1) & 1, 2 * ip + 6 < nb);  // blocks 2ip+6 .. 2ip+9
      if constexpr (!kSingle) ga = *reinterpret_cast<const float *>(lds + ga_base + ((cbi >> 8) << 2));
      u32x4_t xa[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) xa[t] = *reinterpret_cast<const u32x4_t *>(lds + xo + xoff + 16 * t);
      if (2 * ip + 2 < nb) xoff += xstep;
      const u32x4_t cw = cq[q];
      float2 lv[16];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          lv[4 * t + e] = *reinterpret_cast<const float2 *>(
              tab + __builtin_amdgcn_perm(cw[t], lane_off, 0x0C0C0000u | ((4u + e) << 8)));
      load(q, 2 * ip + 2 * kGvP < nb);
      // the block scale, bit for bit the dequantization's block_scale
      const float s = kSingle ? s1 : __fadd_rn(__fmul_rn(sd, ga), offset);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x4_t wb;
#pragma unroll
        for (int e = 0; e < 4; ++e) wb[e] = bf16x2_rne(__fmul_rn(lv[4 * t + e].x, s), __fmul_rn(lv[4 * t + e].y, s));
        acc = mfma16(xa[t], wb, acc);
      }
      cbi += 2;
      if (ip < np && ((ckb += 2) == nkb32 || ip == np - 1)) {  // leaving a row group: partial out
        float *pp = part + ((cgr * maxcov + kslot) * M) * kGvRows + nrow;
        kslot = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (4 * g + v < M) pp[(4 * g + v) * kGvRows] = acc[v];
        acc = zero;
        if (ckb == nkb32) {
          ckb = 0;
          cbi += gstep_b;
          ++cgr;
        }
      }
      if (ip + 1 >= np) break;  // the last real pair (uniform)
    }
  }

  if (hwork) {  // sum the 16 wave results of the H slice in wave order
    __syncthreads();
    f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);
    red[wave * 64 + lane] = hacc;
    __syncthreads();
    if (wave == 0) {
      f32x4_t t = zero;
      for (int q = 0; q < kGvWaves; ++q) {
        const f32x4_t v = red[q * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] += v[e];
      }
      const int j = 16 * jt + li;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (4 * g + v < M && j < r) hpart[((int64_t)ks * M + 4 * g + v) * RP + j] = t[v];
    }
  }
}

// One workgroup per (row group, m), one thread per row n:
// y[m][n] = bf16(sum of the group's partials (workgroup order) +
// sum_j bf16(s H[m][j]) B[n][j]), H[m][j] summed over its slices in order.
// Every global load (partials, H slices, the group's B rows) is issued
// before any of them is used, so the kernel waits for memory once; B rows
// (contiguous, 256 r bf16) then go through LDS.
template <bool kVecB>  // r % 8 == 0: B staged by 16-byte loads
__global__ __launch_bounds__(256) void k_gemv_finish(int64_t N, int M, int fm, const float *__restrict__ hpart,
                                                     int nslices, const float *__restrict__ part,
                                                     const uint16_t *__restrict__ Bl, int r, int RP, float s,
                                                     int64_t T, int G, int maxcov, bool sparse, int64_t nkb,
                                                     uint16_t *__restrict__ Y, float *__restrict__ H_out) {
  // fm rows m0 .. m0+fm-1 of Y per workgroup (fm <= kFm, fm * r <= 256): the
  // group's B rows are staged once for all of them
  constexpr int kFm = 4, kPv = 8, kHv = 16, kBv = kGvRows * 128 / 8 / 256;  // loads in flight per thread
  __shared__ float s_h[kFm][128];                   // bf16(s H[m][j]) as floats
  extern __shared__ __align__(16) uint16_t s_b[];   // B rows of the group, row stride r (256 r bf16)
  const int tid = threadIdx.x, m0 = blockIdx.y * fm, nm = min(fm, M - m0);
  const int64_t gr = blockIdx.x;
  const int64_t n = gr * kGvRows + tid;
  const int64_t rows = std::min<int64_t>(kGvRows, N - gr * kGvRows);
  const uint16_t *bsrc = Bl + gr * kGvRows * r;
  // covering workgroups of the group: workgroup q's range starts at block
  // 4 floor(q (T/4) / G), so block b lies in workgroup ((b/4 + 1) G - 1) / (T/4)
  const int64_t T4 = T / 4;
  const int64_t wlo = ((gr * nkb / 4 + 1) * G - 1) / T4, whi = ((((gr + 1) * nkb - 1) / 4 + 1) * G - 1) / T4;
  const int nc = (int)(whi - wlo + 1);
  const bool live = n < N && !sparse;
  // every load first: partials of each row m, this thread's H slices (thread
  // (hm, hj) = (tid / r, tid % r) sums H[m0 + hm][hj]), the group's B rows
  float pv[kFm][kPv];
#pragma unroll
  for (int mm = 0; mm < kFm; ++mm) {
    const float *p = part + ((gr * maxcov) * M + m0 + mm) * kGvRows + tid;
#pragma unroll
    for (int k = 0; k < kPv; ++k) pv[mm][k] = live && mm < nm && k < nc ? p[(int64_t)k * M * kGvRows] : 0.f;
  }
  const int hm = tid / r, hj = tid - hm * r;
  const bool hlive = hm < nm;
  float hv[kHv];
#pragma unroll
  for (int q = 0; q < kHv; ++q) hv[q] = hlive && q < nslices ? hpart[((int64_t)q * M + m0 + hm) * RP + hj] : 0.f;
  u32x4_t bv[kBv];
  const int nch = kVecB ? (int)(rows * r / 8) : 0;
  if constexpr (kVecB) {
#pragma unroll
    for (int u = 0; u < kBv; ++u) {
      const int c = tid + 256 * u;
      bv[u] = c < nch ? *reinterpret_cast<const u32x4_t *>(bsrc + 8 * c) : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  if (hlive) {  // H[m0 + hm][hj], slice order
    float h = 0.f;
#pragma unroll
    for (int q = 0; q < kHv; ++q) h += hv[q];
    for (int q = kHv; q < nslices; ++q) h += hpart[((int64_t)q * M + m0 + hm) * RP + hj];
    if (gr == 0 && H_out) H_out[(int64_t)(m0 + hm) * r + hj] = h;
    s_h[hm][hj] = bf16_to_f32(f32_to_bf16_bits(__fmul_rn(s, h)));
  }
  if constexpr (kVecB) {
#pragma unroll
    for (int u = 0; u < kBv; ++u) {
      const int c = tid + 256 * u;
      if (c < nch) *reinterpret_cast<u32x4_t *>(s_b + 8 * c) = bv[u];
    }
  } else {
    for (int c = tid; c < rows * r; c += 256) s_b[c] = bsrc[c];
  }
  float y[kFm];
#pragma unroll
  for (int mm = 0; mm < kFm; ++mm) {
    y[mm] = 0.f;
    if (n < N && mm < nm) {
      const float *p = part + ((gr * maxcov) * M + m0 + mm) * kGvRows + tid;
      if (!sparse) {
#pragma unroll
        for (int k = 0; k < kPv; ++k) y[mm] += pv[mm][k];
        for (int k = kPv; k < nc; ++k) y[mm] += p[(int64_t)k * M * kGvRows];
      } else {
        for (int64_t q = wlo; q <= whi; ++q) {
          // an empty range (more workgroups than 4-block units) wrote nothing
          if (4 * ((q + 1) * T4 / G) == 4 * (q * T4 / G)) continue;
          y[mm] += p[(q - wlo) * M * kGvRows];
        }
      }
    }
  }
  __syncthreads();  // s_h, s_b
  if (n >= N) return;
  float lo[kFm] = {0.f, 0.f, 0.f, 0.f};
  const uint16_t *brow = s_b + tid * r;
  for (int j = 0; j < r; ++j) {
    const float b = bf16_to_f32(brow[j]);
#pragma unroll
    for (int mm = 0; mm < kFm; ++mm) lo[mm] = __fmaf_rn(s_h[mm][j], b, lo[mm]);
  }
#pragma unroll
  for (int mm = 0; mm < kFm; ++mm)
    if (mm < nm) Y[(int64_t)(m0 + mm) * N + n] = f32_to_bf16_bits(y[mm] + lo[mm]);
}

}  // namespace

bool small_m_supported(int64_t M, int64_t n, int64_t k, int r) {
  if (M < 1 || M > kGemvMaxM || r > 128 || k % (4 * kBlock) != 0 || n * (k / 2) >= (int64_t(1) << 31)) return false;
  return gemv_plan(M, n, k, lora_rank_pad(r)).G <= kMaxG;
}

size_t small_m_workspace_bytes(int64_t M, int64_t n, int64_t k, int r) {
  return small_ws_layout(M, n, k, lora_rank_pad(r)).total;
}

hipError_t launch_fwd_small(const Nf4View &w, const uint16_t *X, int64_t M, const uint16_t *A, const uint16_t *B,
                            int r, float s, uint16_t *Y, float *H_out, void *ws, hipStream_t st) {
  const int RP = lora_rank_pad(r);
  const SmallWs l = small_ws_layout(M, w.n, w.k, RP);
  const GemvPlan &p = l.p;
  char *base = static_cast<char *>(ws);
  float *hpart = reinterpret_cast<float *>(base + l.h_off);
  float *part = reinterpret_cast<float *>(base + l.part_off);
  const int T4 = (int)(p.T / 4);
  if (w.absmax)
    QLORA_LAUNCH("k_gemv_nf4", k_gemv_nf4<true>, dim3((unsigned)p.G), dim3(1024), 0, st, w, X, (int)M, A, r, RP,
                 hpart, part, T4, p.G, T4 / p.G, T4 % p.G, p.seg, p.maxcov, p.nh, p.nht, p.xoff);
  else
    QLORA_LAUNCH("k_gemv_nf4", k_gemv_nf4<false>, dim3((unsigned)p.G), dim3(1024), 0, st, w, X, (int)M, A, r, RP,
                 hpart, part, T4, p.G, T4 / p.G, T4 % p.G, p.seg, p.maxcov, p.nh, p.nht, p.xoff);
  // the group's B rows in LDS, sized by the rank (more workgroups per CU at small r)
  const size_t bshm = (size_t)kGvRows * r * sizeof(uint16_t);
  // rows of Y per workgroup: up to 4 (one H-summing thread per (row, rank)),
  // while the grid keeps at least one workgroup per CU
  int fm = 1;
  while (2 * fm <= std::min({4, 256 / r, (int)M}) && p.ngroups * ceil_div(M, (int64_t)(2 * fm)) >= 256) fm *= 2;
  const dim3 fgrid((unsigned)p.ngroups, (unsigned)ceil_div(M, (int64_t)fm));
  if (r % 8 == 0)
    QLORA_LAUNCH("k_gemv_finish", k_gemv_finish<true>, fgrid, dim3(256), bshm, st, w.n, (int)M, fm,
                 hpart, p.nh / p.nht, part, B, r, RP, s, p.T, p.G, p.maxcov, p.sparse, p.nkb, Y, H_out);
  else
    QLORA_LAUNCH("k_gemv_finish", k_gemv_finish<false>, fgrid, dim3(256), bshm, st, w.n, (int)M, fm,
                 hpart, p.nh / p.nht, part, B, r, RP, s, p.T, p.G, p.maxcov, p.sparse, p.nkb, Y, H_out);
  return hipGetLastError();
}

}  // namespace qlora

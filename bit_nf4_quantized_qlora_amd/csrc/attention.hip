// attention.hip -- the causal attention core between the q/k/v projections
// and the o projection of the decoder layer whose seven linears all carry
// adapters ("QLoRA, explained.", all-linear placement; the layer of
// "QLoRA Explained ... Part 2/6", App. G).
//
// The pages do not write attention out; this is the plain causal scaled
// dot-product attention of a LLaMA decoder layer, per sequence and head:
//   S = Q K^T / sqrt(d) for key j <= query i, P = softmax_j(S), O = P V,
//   lse_i = log sum_j exp S_ij;
//   dV = P^T dO, dP = dO V^T, dS = P (dP - D) with D_i = sum_j P_ij dP_ij,
//   dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d).
//
// Q, K, V, O (and their gradients) are [batch * seq, heads * d] row-major
// bf16, the projections' outputs as they come.
//
// Head dims 32, 64, 96 and 128 (the LLaMA layers' among them) take fused kernels that keep
// no score matrix in memory: a forward with an online softmax, and a
// backward in two launches, a query side (D_i = sum_j P_ij dP_ij from the
// row's own float32 P and dP, then dQ) and a key side (dK, dV).  Each
// recomputes S and dP per 64-row block on MFMA; P and dS are rounded to
// bf16 in the lane that computes them, the same rounding points as the
// materialised path below.
//
// Other head dims materialise the scores per (sequence, head) in the
// workspace: float32 S and dP, bf16 P and dS, each [batch][heads][seq][ldp]
// with ldp = seq rounded up to 8.
//
// Products of the materialised path: one batched MFMA kernel, 64 x 64
// output tiles, 4 waves of 2 x 2 16x16x32 bf16 MFMAs, a 64-deep contraction
// step staged through LDS with the next step's operands loaded into
// registers meanwhile.  Each operand is read along whichever axis is
// contiguous in memory (template flags) and staged as it lies; fragments of
// row-contiguous operands come from transposing LDS reads.  Causality
// prunes work: score tiles wholly above the diagonal are skipped, and the
// products with P or dS stop (or start) their contraction at the tile's
// diagonal.
//
// Row kernels of the materialised path: one wave per query row.  The
// forward softmax takes the row maximum and the sum of exponentials in
// float32 and writes P and lse; the backward row pass recomputes
// P = exp(S - lse), sums D from P and dP, and writes P and dS.  Both write
// zeros for the masked entries up to the end of the diagonal tile, the only
// masked entries a product reads.
#include <cmath>

#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int kT = 64;          // output tile edge

// Exponentials in base 2 on the hardware's v_exp_f32 / v_log_f32 (about one
// ulp; exp2(-inf) = 0): the kernels carry scores in base-2 exponent units,
// s * scale * log2(e), and lse in natural units.
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }
constexpr int kKs = 64;         // contraction per step (two 32-deep MFMA sub-steps)
constexpr int kLd = kKs + 8;    // LDS row stride in elements (144 B: a 16-lane fragment read is conflict-free)

struct Opnd {
  const uint16_t *p;
  int64_t ld, sb, sh;  // row stride, then the sequence and head offsets (elements)
};

struct GemmArgs {
  Opnd a, b;
  void *c;
  float alpha;
  int64_t ldc, csb, csh;
  int M, N, K, tiles_n;
  int mask;    // 1: skip tiles whose every column index exceeds every row index
  int krange;  // 0: whole contraction; 1: k < m0 + 64 (k <= row); 2: k >= m0 (k >= row)
};

// Eight elements of an operand X(i, k) as one 16-byte word, zero where out
// of range.  KC: X(i, k..k+7) at base[i*ld + k + j] (contraction contiguous);
// otherwise X(i..i+7, k) at base[k*ld + i + j].
template <bool KC>
__device__ __forceinline__ u32x4_t load8(const uint16_t *base, int64_t ld, int i, int k, int I, int K) {
  u32x4_t v = {0u, 0u, 0u, 0u};
  const bool row_ok = KC ? i < I : k < K;
  const int c = KC ? k : i, C = KC ? K : I;  // the contiguous index and its bound
  if (!row_ok) return v;
  const uint16_t *p = KC ? base + (int64_t)i * ld + k : base + (int64_t)k * ld + i;
  if (c + 8 <= C) return *reinterpret_cast<const u32x4_t *>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (c + j < C) v[j >> 1] |= (uint32_t)p[j] << (16 * (j & 1));
  return v;
}

// LDS tiles of one contraction step.  An operand with its contraction
// contiguous in memory (KC) is staged [row][contraction] (64 x kLd) and a
// fragment is one 16-byte read.  An operand with its rows contiguous is
// staged as it lies, [contraction][row] (64 x kLdT), by 16-byte copies, and
// a fragment is two ds_read_b64_tr_b16: in a 16-lane group, lane i receives
// element i & 3 of the 8 bytes addressed by lanes 4q + i/4 (q = 0..3), so
// lanes addressing contraction rows kk0 + 8g + 4h + q, columns
// row0 + 4(j & 3) hand lane i four consecutive contraction elements of row
// row0 + i.
// (Writing such operands transposed into LDS took eight 2-byte stores per
// thread and step.)  kLdT = 72: a 144-byte row stride, at most two lanes of
// a half-wave per bank for these reads.
constexpr int kLdT = kT + 8;
static_assert(kKs * kLdT <= kT * kLd, "both staging layouts fit one buffer");

template <bool KC>
__device__ __forceinline__ void store8(uint16_t *tile, int i, int k, const u32x4_t &v) {
  *reinterpret_cast<u32x4_t *>(tile + (KC ? i * kLd + k : k * kLdT + i)) = v;
}

template <bool KC>
__device__ __forceinline__ u32x4_t frag(const uint16_t *tile, int row0, int kk0, int lane) {
  if (KC) return lds_frag(tile, kLd, row0, kk0, lane);
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  const int j = lane & 15, g = lane >> 4;
  const uint16_t *p = tile + (kk0 + 8 * g + (j >> 2)) * kLdT + row0 + 4 * (j & 3);
  const s16x4_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t *)p);
  const s16x4_t h1 =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t *)(p + 4 * kLdT));
  return __builtin_bit_cast(u32x4_t, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Staging coordinates of 16-byte piece e (0..511) of a 64 x 64 tile: 8
// pieces of 8 contraction elements per row (KC), or 8 pieces of 8 rows per
// contraction index.
template <bool KC>
__device__ __forceinline__ void stage_coords(int e, int &i, int &k) {
  i = KC ? e >> 3 : (e & 7) * 8;
  k = KC ? (e & 7) * 8 : e >> 3;
}

// C[m][n] = alpha * sum_k A(m, k) B(n, k), one 64 x 64 tile per workgroup;
// blockIdx.y = head, blockIdx.z = sequence.
template <bool AKC, bool BKC, bool OUT_BF16>
__global__ __launch_bounds__(256) void k_attn_gemm(GemmArgs g) {
  __shared__ __align__(16) uint16_t sA[kT * kLd];
  __shared__ __align__(16) uint16_t sB[kT * kLd];
  const int tm = blockIdx.x / g.tiles_n, tn = blockIdx.x - tm * g.tiles_n;
  const int m0 = tm * kT, n0 = tn * kT;
  if (g.mask == 1 && n0 > m0 + kT - 1) return;  // the whole workgroup leaves together
  const int64_t z = blockIdx.z, y = blockIdx.y;
  const uint16_t *A = g.a.p + z * g.a.sb + y * g.a.sh;
  const uint16_t *B = g.b.p + z * g.b.sb + y * g.b.sh;
  const int kb = g.krange == 2 ? m0 : 0;
  const int ke = g.krange == 1 ? min(g.K, m0 + kT) : g.K;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = (w >> 1) * 32, wn = (w & 1) * 32;
  int ia[2], ka[2], ib[2], kbb[2];  // two pieces per thread and operand
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    stage_coords<AKC>(t + 256 * u, ia[u], ka[u]);
    stage_coords<BKC>(t + 256 * u, ib[u], kbb[u]);
  }

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t va[2], vb[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    va[u] = vb[u] = u32x4_t{0u, 0u, 0u, 0u};
    if (kb < ke) {
      va[u] = load8<AKC>(A, g.a.ld, m0 + ia[u], kb + ka[u], g.M, ke);
      vb[u] = load8<BKC>(B, g.b.ld, n0 + ib[u], kb + kbb[u], g.N, ke);
    }
  }
  for (int k0 = kb; k0 < ke; k0 += kKs) {
    __syncthreads();  // the previous step's fragment reads are done
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      store8<AKC>(sA, ia[u], ka[u], va[u]);
      store8<BKC>(sB, ib[u], kbb[u], vb[u]);
    }
    __syncthreads();
    if (k0 + kKs < ke) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        va[u] = load8<AKC>(A, g.a.ld, m0 + ia[u], k0 + kKs + ka[u], g.M, ke);
        vb[u] = load8<BKC>(B, g.b.ld, n0 + ib[u], k0 + kKs + kbb[u], g.N, ke);
      }
    }
#pragma unroll
    for (int kk0 = 0; kk0 < kKs; kk0 += 32) {
      u32x4_t fa[2], fb[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        fa[u] = frag<AKC>(sA, wm + 16 * u, kk0, lane);
        fb[u] = frag<BKC>(sB, wn + 16 * u, kk0, lane);
      }
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int tj = 0; tj < 2; ++tj) acc[ti][tj] = mfma16(fa[ti], fb[tj], acc[ti][tj]);
    }
  }

  const int64_t coff = z * g.csb + y * g.csh;
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int tj = 0; tj < 2; ++tj)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm + 16 * ti + 4 * (lane >> 4) + v;
        const int n = n0 + wn + 16 * tj + (lane & 15);
        if (m < g.M && n < g.N) {
          const float x = g.alpha * acc[ti][tj][v];
          if (OUT_BF16)
            static_cast<uint16_t *>(g.c)[coff + (int64_t)m * g.ldc + n] = f32_to_bf16_bits(x);
          else
            static_cast<float *>(g.c)[coff + (int64_t)m * g.ldc + n] = x;
        }
      }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Columns a row's products read: up to the end of its diagonal tile.
__device__ __forceinline__ int row_span(int q, int seq) { return min(seq, (q / kT + 1) * kT); }

// Row chunks: lane l holds columns c0 + 4l .. +3 and c0 + 256 + 4l .. +3, so
// a wave covers 512 columns with two 16-byte loads per lane, both issued
// before either is used.  A group starting at or past `lim` reads nothing;
// elements at or past `lim` inside a group are replaced by `fill` (a select:
// the memory there may hold anything).  Row starts are 32-byte aligned
// (ldp is a multiple of 8) and a group starting below lim <= ldp ends inside
// the row, so every load stays in the workspace.
constexpr int kChunk = 512;
__device__ __forceinline__ void load_chunk(const float *row, int c0, int lane, int lim, float fill, float (&x)[8]) {
  f32x4_t v[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = c0 + 256 * h + 4 * lane;
    v[h] = c < lim ? *reinterpret_cast<const f32x4_t *>(row + c) : f32x4_t{fill, fill, fill, fill};
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * h + e] = c0 + 256 * h + 4 * lane + e < lim ? v[h][e] : fill;
}

// Four bf16 of a chunk group to row[c..c+3], cut at `span`.
__device__ __forceinline__ void store4(uint16_t *row, int c, int span, const float (&y)[8], int h) {
  if (c >= span) return;
  if (c + 4 <= span) {
    u32x2_t w = {bf16x2_rne(y[4 * h], y[4 * h + 1]), bf16x2_rne(y[4 * h + 2], y[4 * h + 3])};
    *reinterpret_cast<u32x2_t *>(row + c) = w;
  } else {
    for (int e = 0; c + e < span; ++e) row[c + e] = f32_to_bf16_bits(y[4 * h + e]);
  }
}

// Forward softmax of the (already scaled) scores, one wave per row
// r = (sequence * heads + head) * seq + query: a running maximum and sum
// over 512-column chunks, then P = exp(S - max) / sum.
__global__ __launch_bounds__(256) void k_attn_softmax(const float *__restrict__ S, uint16_t *__restrict__ P,
                                                      float *__restrict__ lse, int64_t rows, int seq, int64_t ldp) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const int q = (int)(r % seq), n = q + 1;
  const float *s = S + r * ldp;
  uint16_t *p = P + r * ldp;
  float m = -INFINITY, zsum = 0.f;
  for (int c0 = 0; c0 < n; c0 += kChunk) {
    float x[8];
    load_chunk(s, c0, lane, n, -INFINITY, x);
    float cm = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, x[e]);
    const float mn = fmaxf(m, wave_max(cm));  // finite: every chunk holds a column < n
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) part += expf(x[e] - mn);
    zsum = zsum * expf(m - mn) + part;
    m = mn;
  }
  zsum = wave_sum(zsum);
  const int span = row_span(q, seq);
  for (int c0 = 0; c0 < span; c0 += kChunk) {
    float x[8], y[8];
    load_chunk(s, c0, lane, n, -INFINITY, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = expf(x[e] - m) / zsum;  // exp(-inf) = 0 past the diagonal
#pragma unroll
    for (int h = 0; h < 2; ++h) store4(p, c0 + 256 * h + 4 * lane, span, y, h);
  }
  if (lane == 0) lse[r] = m + logf(zsum);
}

// Backward row pass: P = exp(S - lse), D = sum_j P_j dP_j, dS = P (dP - D).
// D is summed from the float32 P and dP of the row itself (a first pass
// over the row), so each row of dS sums to zero up to float32 rounding;
// taking D = dO . O from the bf16 output instead would carry O's rounding
// into dP - D, which cancels where the attention is sharply peaked.
__global__ __launch_bounds__(256) void k_attn_bwd_rows(const float *__restrict__ S, const float *__restrict__ dP,
                                                       const float *__restrict__ lse, uint16_t *__restrict__ P,
                                                       uint16_t *__restrict__ dS, int64_t rows, int seq,
                                                       int64_t ldp) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const int q = (int)(r % seq), n = q + 1;
  const float L = lse[r];
  const float *s = S + r * ldp, *dp = dP + r * ldp;
  // the first chunk stays in registers for the second pass (rows up to 512
  // columns are read once)
  float x0[8], g0[8];
  load_chunk(s, 0, lane, n, -INFINITY, x0);
  load_chunk(dp, 0, lane, n, 0.f, g0);
  float D = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) D += expf(x0[e] - L) * g0[e];
  for (int c0 = kChunk; c0 < n; c0 += kChunk) {
    float x[8], g[8];
    load_chunk(s, c0, lane, n, -INFINITY, x);
    load_chunk(dp, c0, lane, n, 0.f, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) D += expf(x[e] - L) * g[e];
  }
  D = wave_sum(D);
  uint16_t *p = P + r * ldp, *ds = dS + r * ldp;
  const int span = row_span(q, seq);
  for (int c0 = 0; c0 < span; c0 += kChunk) {
    float x[8], g[8], pe[8], de[8];
    if (c0 == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = x0[e];
        g[e] = g0[e];
      }
    } else {
      load_chunk(s, c0, lane, n, -INFINITY, x);
      load_chunk(dp, c0, lane, n, 0.f, g);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pe[e] = expf(x[e] - L);  // 0 past the diagonal
      de[e] = pe[e] * (g[e] - D);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      store4(p, c0 + 256 * h + 4 * lane, span, pe, h);
      store4(ds, c0 + 256 * h + 4 * lane, span, de, h);
    }
  }
}

// Fused kernels (head dims 32, 64, 96, 128).  Each workgroup streams 64-row
// blocks of the other side's operands (K and V for a query tile, Q and dO
// for a key tile) through LDS, rows staged as they lie with row stride
// D + kRowPad, in two stages: block i is read while block i+1 is stored and
// block i+2 is loaded into registers, one barrier per block.  Fragments of
// a staged operand are 16-byte row reads (rows as MFMA rows, dims as the
// contraction) or transposing reads (dims as MFMA rows, rows as the
// contraction, at the rows whose scores the lane holds).  A row stride of
// D + 16 puts the four rows of a transposing read's 16-lane group on four
// disjoint bank octets (D + 8 doubled those reads: 105 against 117 us key
// side, 132 against 150 us query side at 8 x 512 x 32 x 128).
constexpr int kRowPad = 16;
constexpr int kQT = 128;                    // queries per fused-forward workgroup (8 waves)
constexpr int kBwdWaves = 8;                // waves per backward workgroup, 16 queries or keys each
constexpr int kBwdRows = 16 * kBwdWaves;    // queries (keys) per query-side (key-side) backward workgroup

// Two transposing LDS reads (ds_read_b64_tr_b16): lane (g = l >> 4,
// i = l & 15) receives X[r0 + 4g + e][c0 + i] for e = 0..3, then
// X[r1 + 4g + e][c0 + i], from a row-major LDS array X (row stride ld
// elements, a multiple of 8).  As an MFMA operand that is row c0 + i of X^T
// with contraction slots 8g .. 8g+3 on rows r0 + 4g .. +3 and 8g+4 .. 8g+7
// on rows r1 + 4g .. +3: the rows whose scores accumulator lanes of group g
// hold in the 16-row output tiles at r0 and r1.
__device__ __forceinline__ u32x4_t lds_frag_t2(const uint16_t *X, int ld, int r0, int r1, int c0, int lane) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  const int j = lane & 15, g = lane >> 4;
  const int off = (4 * g + (j >> 2)) * ld + c0 + 4 * (j & 3);
  const s16x4_t h0 =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t *)(X + r0 * ld + off));
  const s16x4_t h1 =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t *)(X + r1 * ld + off));
  return __builtin_bit_cast(u32x4_t, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 64 rows of an operand [row][D] in kPL 16-byte pieces per thread of an
// NT-thread workgroup: piece e is row e / (D/8), columns 8 (e % (D/8)) .. +7.
// Rows past the sequence repeat its last row (row0 < seq): every load is
// in bounds and unconditional, and the kernels make such rows contribute
// exactly nothing (their P is selected to 0, so their dS is 0 too), so they
// need only hold finite values.
template <int D, int NT>
struct Rows64 {
  static constexpr int kPieces = 8 * D;
  static constexpr int kPL = (kPieces + NT - 1) / NT;
  static constexpr int kLd = D + kRowPad;  // LDS row stride (elements)
  u32x4_t r[kPL];
  __device__ __forceinline__ void load(const uint16_t *g, int64_t ld, int row0, int seq, int t) {
#pragma unroll
    for (int i = 0; i < kPL; ++i) {
      const int e = t + NT * i;
      if (e < kPieces) {
        const int row = min(row0 + e / (D / 8), seq - 1);
        r[i] = *reinterpret_cast<const u32x4_t *>(g + (int64_t)row * ld + 8 * (e % (D / 8)));
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t *lds, int t) const {
#pragma unroll
    for (int i = 0; i < kPL; ++i) {
      const int e = t + NT * i;
      if (e < kPieces) *reinterpret_cast<u32x4_t *>(lds + (e / (D / 8)) * kLd + 8 * (e % (D / 8))) = r[i];
    }
  }
};

// Which (tile, head, sequence) a workgroup of a fused kernel takes.  The
// grid is (tiles, heads, batch) with tile 0 the longest (the most key or
// query blocks under the causal mask); workgroups are renumbered tile-major,
// every (sequence, head)'s tile 0 first, then every tile 1, and so on.
// Workgroups go to the eight XCDs in turn by linear id and each XCD hands
// them to its CUs as they free up, so this is list scheduling, longest
// first: at 8 x 512 x 32 x 128 the causal tiles (8, 6, 4 and 2 blocks) end
// in 20 block-times per CU instead of 24 with a (sequence, head)'s tiles back
// to back (backward 211 -> 161 us, forward 49 -> 44 us).  When heads x batch
// is a multiple of 8, the tiles of one (sequence, head) also land on one XCD
// and can share its L2.  A bijection on the grid, in 64-bit arithmetic.
struct AttnTile {
  int tile;
  int64_t h, b;
};
__device__ __forceinline__ AttnTile attn_tile() {
  const int64_t T = gridDim.x, H = gridDim.y, HB = H * (int64_t)gridDim.z;
  const int64_t L = blockIdx.x + T * (blockIdx.y + H * (int64_t)blockIdx.z);
  const int64_t bh = L % HB;
  return AttnTile{(int)(L / HB), bh % H, bh / H};
}

// Output of a wave's 16 x D tile held in the accumulator layout (lane
// (g, c) holds row c, columns 16 dt + 4g .. +3 of tile dt): the lane's
// 8-byte pieces, scaled and rounded to bf16, meet in LDS (stg: this wave's
// 16 rows of kOutLd elements), and after a barrier each row leaves in
// 16-byte pieces, whole lines at a time.  Stored straight from the
// accumulators the pieces of one line came from four lanes and, with two
// outputs interleaved, lines were written back half filled.
template <int D>
constexpr int kOutLd = D + 8;
template <int D>
__device__ __forceinline__ void stage_rows16(const f32x4_t (&acc)[D / 16], float mul, uint16_t *stg, int lane) {
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const u32x2_t v = {bf16x2_rne(acc[dt][0] * mul, acc[dt][1] * mul), bf16x2_rne(acc[dt][2] * mul, acc[dt][3] * mul)};
    *reinterpret_cast<u32x2_t *>(stg + c * kOutLd<D> + 16 * dt + 4 * g) = v;
  }
}
// rows row0 .. row0+15 below nrows of a row-major bf16 array (stride ld)
template <int D>
__device__ __forceinline__ void flush_rows16(const uint16_t *stg, uint16_t *out, int64_t ld, int row0, int nrows,
                                             int lane) {
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {  // 16 rows x D/8 pieces per wave: D/32 per lane
    const int e = lane + 64 * j, row = e / (D / 8), col = 8 * (e % (D / 8));
    if (row0 + row < nrows)
      *reinterpret_cast<u32x4_t *>(out + (int64_t)(row0 + row) * ld + col) =
          *reinterpret_cast<const u32x4_t *>(stg + row * kOutLd<D> + col);
  }
}

// Fused forward: one workgroup of 8 waves per (sequence, head, 128-query
// tile), wave w on queries q0 + 16w .. +15, so a staged key block serves 128
// queries; no score matrix in memory.  Per 64-key block (causal: blocks up
// to the diagonal one; a wave skips blocks wholly past its queries):
//   S^T = K Q^T on MFMA (A = K rows from LDS, B = Q from registers), so each
//   lane's accumulators all belong to one query (its column l & 15): the
//   online softmax (running max m in base-2 units, lane-partial sum l,
//   rescale of the output when some lane's maximum grew) needs only a max
//   over the lane's 16 values and lanes l ^ 16, 32;
//   O^T += V^T P^T on MFMA with P rounded to bf16: the MFMA contraction
//   slots 8g .. 8g+7 of lane group g = l >> 4 are assigned to the keys that
//   lane already holds (4g .. 4g+3 of two 16-key tiles), so P goes from
//   accumulator to operand without moving between lanes, and V^T comes from
//   transposing reads of the staged V rows at the same keys.
// Only the diagonal block masks (keys past the query, which covers keys past
// the sequence for every query in it).
template <int D>
__global__ __launch_bounds__(512) void k_attn_fwd_fused(const uint16_t *__restrict__ Qg, const uint16_t *__restrict__ Kg,
                                                        const uint16_t *__restrict__ Vg, uint16_t *__restrict__ Og,
                                                        float *__restrict__ lse, int seq, int heads, float scale) {
  using R = Rows64<D, 512>;
  constexpr int kLd = R::kLd;
  __shared__ __align__(16) uint16_t sK[2][kT * kLd];
  __shared__ __align__(16) uint16_t sV[2][kT * kLd];
  const AttnTile at = attn_tile();
  const int q0 = ((int)gridDim.x - 1 - at.tile) * kQT;  // the longest query tiles start first
  const int64_t h = at.h, b = at.b;
  const int64_t ld = (int64_t)heads * D;
  const int64_t base = b * seq * ld + h * D;
  const int t = threadIdx.x, lane = t & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int qw = q0 + 16 * w, qi = qw + c;  // this wave's first query, this lane's query

  u32x4_t qf[D / 32];  // B operand of K Q^T: Q[qi][32 ks + 8 g ..]
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    qf[ks] = u32x4_t{0u, 0u, 0u, 0u};
    if (qi < seq) qf[ks] = *reinterpret_cast<const u32x4_t *>(Qg + base + qi * ld + 32 * ks + 8 * g);
  }
  f32x4_t acc_o[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc_o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const float c2 = scale * kLog2e;  // scores in base-2 exponent units

  const int nblk = min((seq + kT - 1) / kT, (q0 + kQT) / kT);  // key blocks up to the diagonal
  R rk, rv;
  rk.load(Kg + base, ld, 0, seq, t);
  rv.load(Vg + base, ld, 0, seq, t);
  rk.store(sK[0], t);
  rv.store(sV[0], t);
  if (nblk > 1) {
    rk.load(Kg + base, ld, kT, seq, t);
    rv.load(Vg + base, ld, kT, seq, t);
  }
  for (int kb = 0; kb < nblk; ++kb) {
    const int k0 = kb * kT;
    const uint16_t *cK = sK[kb & 1], *cV = sV[kb & 1];
    __syncthreads();  // stage kb & 1 is stored; every read of the other stage (block kb - 1) is done
    if (kb + 1 < nblk) {
      rk.store(sK[(kb + 1) & 1], t);
      rv.store(sV[(kb + 1) & 1], t);
      if (kb + 2 < nblk) {
        rk.load(Kg + base, ld, k0 + 2 * kT, seq, t);
        rv.load(Vg + base, ld, k0 + 2 * kT, seq, t);
      }
    }
    if (k0 > qw + 15) continue;  // every key of the block follows every query of this wave

    // S^T for 4 key tiles of 16
    f32x4_t st[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) st[kt] = mfma16(lds_frag(cK, kLd, 16 * kt, 32 * ks, lane), qf[ks], st[kt]);
    }
    if (k0 + kT - 1 > qw) {  // the diagonal block
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (k0 + 16 * kt + 4 * g + v > qi) st[kt][v] = -INFINITY;
    }
    float bm = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) bm = fmaxf(bm, fmaxf(fmaxf(st[kt][0], st[kt][1]), fmaxf(st[kt][2], st[kt][3])));
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    // finite for a lane whose query is in the sequence: block 0 holds key 0
    // <= qi, and a later diagonal block holds keys up to qi or leaves
    // bm = -inf (m unchanged)
    const float mn = fmaxf(m, bm * c2);
    if (__any(mn > m)) {  // rescale only when some running maximum grew
      const float corr = exp2_fast(m - mn);
      l *= corr;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) acc_o[i] *= corr;
    }
    m = mn;
    uint32_t pw[4][2];  // P as bf16 pairs: tile kt, keys 4g + (0,1) and (2,3)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float e[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        e[v] = exp2_fast(fmaf(st[kt][v], c2, -mn));
        l += e[v];
      }
      pw[kt][0] = bf16x2_rne(e[0], e[1]);
      pw[kt][1] = bf16x2_rne(e[2], e[3]);
    }
    // O^T += V^T P^T, two 32-key contraction steps
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4_t pb = {pw[2 * ks][0], pw[2 * ks][1], pw[2 * ks + 1][0], pw[2 * ks + 1][1]};
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        acc_o[dt] = mfma16(lds_frag_t2(cV, kLd, 32 * ks, 32 * ks + 16, 16 * dt, lane), pb, acc_o[dt]);
    }
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (qi < seq && g == 0) lse[(b * heads + h) * seq + qi] = (m + log2_fast(l)) * kLn2;
  // O through LDS (the staged-block buffers, free once every wave is past
  // its last read); a lane whose query lies past the sequence stages
  // whatever it holds, and its row is not written
  static_assert(8 * 16 * kOutLd<D> <= 2 * kT * kLd, "a wave's output rows fit the block buffer");
  uint16_t *stg = &sK[0][0] + w * 16 * kOutLd<D>;
  __syncthreads();
  stage_rows16<D>(acc_o, 1.0f / l, stg, lane);
  __syncthreads();
  flush_rows16<D>(stg, Og + base, ld, qw, seq, lane);
}

// Backward, query side, for head dims 32, 64, 96, 128: one workgroup of 8 waves
// per (sequence, head, 128-query tile), wave w on queries q0 + 16w .. +15,
// key blocks of 64 (K and V rows staged in LDS as they lie, the next block
// loaded into registers meanwhile) up to the diagonal, twice:
//   pass 1: S^T = K Q^T and dP^T = V dO^T on MFMA (A from LDS, B = the
//     lane's query row of Q or dO in registers), P = exp(S - lse), and each
//     lane sums P dP over its keys; the sums of the four lane groups give
//     D = sum_j P_j dP_j for the lane's query (float32, from the row's own
//     P and dP, as the materialised path sums it), written for the key side;
//   pass 2: the same S^T and dP^T, dS^T = P^T (dP^T - D) rounded to bf16 in
//     the lane that computed it, dQ^T += K^T dS^T on MFMA with K^T read from
//     the staged K rows by transposing LDS reads at the keys the lane holds
//     (contraction slots as in the forward's O^T = V^T P^T).
// Blocks wholly past a wave's queries are skipped; only diagonal blocks
// mask.  A lane whose query lies past the sequence takes lse = +inf, so its
// P is 0, and writes nothing.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_attn_bwd_q(const uint16_t *__restrict__ Qg, const uint16_t *__restrict__ Kg,
                                                    const uint16_t *__restrict__ Vg, const uint16_t *__restrict__ dOg,
                                                    const float *__restrict__ lse, float *__restrict__ Dg,
                                                    uint16_t *__restrict__ dQg, int seq, int heads, float scale) {
  constexpr int NT = 64 * NW, QT = 16 * NW;
  using R = Rows64<D, NT>;
  constexpr int kLd = R::kLd;
  __shared__ __align__(16) uint16_t sK[2][kT * kLd];  // two stages: block i computes while block i+1 is stored
  __shared__ __align__(16) uint16_t sV[2][kT * kLd];
  const AttnTile at = attn_tile();
  const int q0 = ((int)gridDim.x - 1 - at.tile) * QT;  // the longest query tiles start first
  const int64_t h = at.h, b = at.b;
  const int64_t ld = (int64_t)heads * D;
  const int64_t base = b * seq * ld + h * D;
  const int64_t row = (b * heads + h) * seq;
  const int t = threadIdx.x, lane = t & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int qw = q0 + 16 * w, qi = qw + c;
  const bool qok = qi < seq;

  u32x4_t qf[D / 32], of[D / 32];  // B operands: Q and dO of the lane's query, dims 32 ks + 8 g ..
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    qf[ks] = of[ks] = u32x4_t{0u, 0u, 0u, 0u};
    if (qok) {
      qf[ks] = *reinterpret_cast<const u32x4_t *>(Qg + base + qi * ld + 32 * ks + 8 * g);
      of[ks] = *reinterpret_cast<const u32x4_t *>(dOg + base + qi * ld + 32 * ks + 8 * g);
    }
  }
  const float c2 = scale * kLog2e;
  const float l2 = qok ? lse[row + qi] * kLog2e : INFINITY;
  f32x4_t acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float dsum = 0.f, Dq = 0.f;

  const int nblk = min((seq + kT - 1) / kT, (q0 + QT + kT - 1) / kT);  // key blocks up to the diagonal
  // iteration it < nblk is pass 1 on key block it, it >= nblk pass 2 on
  // block it - nblk; block(it) is staged in LDS stage it & 1
  auto block = [&](int it) { return (it < nblk ? it : it - nblk) * kT; };
  R rk, rv;
  rk.load(Kg + base, ld, 0, seq, t);
  rv.load(Vg + base, ld, 0, seq, t);
  rk.store(sK[0], t);
  rv.store(sV[0], t);
  rk.load(Kg + base, ld, block(1), seq, t);  // 2 * nblk >= 2 iterations
  rv.load(Vg + base, ld, block(1), seq, t);
  for (int it = 0; it < 2 * nblk; ++it) {
    const bool second = it >= nblk;
    const int k0 = block(it);
    const uint16_t *cK = sK[it & 1], *cV = sV[it & 1];
    if (it == nblk) {
      Dq = dsum + __shfl_xor(dsum, 16, 64);
      Dq += __shfl_xor(Dq, 32, 64);
      if (qok && g == 0) Dg[row + qi] = Dq;
    }
    __syncthreads();  // stage it & 1 is stored; every read of the other stage (iteration it - 1) is done
    if (it + 1 < 2 * nblk) {
      rk.store(sK[(it + 1) & 1], t);
      rv.store(sV[(it + 1) & 1], t);
      if (it + 2 < 2 * nblk) {
        rk.load(Kg + base, ld, block(it + 2), seq, t);
        rv.load(Vg + base, ld, block(it + 2), seq, t);
      }
    }
    if (k0 > qw + 15) continue;  // every key of the block follows every query of this wave

    // the MFMA groups run at raised wave priority, so the other wave of a
    // SIMD, in its exponential or dS arithmetic, yields the issue slot to
    // them (120 against 128 us at 8 x 512 x 32 x 128; no gain on the key side)
    __builtin_amdgcn_s_setprio(1);
    f32x4_t st[4], dp[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      st[kt] = dp[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        st[kt] = mfma16(lds_frag(cK, kLd, 16 * kt, 32 * ks, lane), qf[ks], st[kt]);
        dp[kt] = mfma16(lds_frag(cV, kLd, 16 * kt, 32 * ks, lane), of[ks], dp[kt]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    float p[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) p[kt][v] = exp2_fast(fmaf(st[kt][v], c2, -l2));
    if (k0 + kT - 1 > qw) {  // the diagonal block: keys past the query drop out
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (k0 + 16 * kt + 4 * g + v > qi) p[kt][v] = 0.f;
    }
    if (!second) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) dsum = fmaf(p[kt][v], dp[kt][v], dsum);
      continue;
    }
    uint32_t sw[4][2];  // dS^T as bf16 pairs: tile kt, keys 4g + (0,1) and (2,3)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sw[kt][0] = bf16x2_rne(p[kt][0] * (dp[kt][0] - Dq), p[kt][1] * (dp[kt][1] - Dq));
      sw[kt][1] = bf16x2_rne(p[kt][2] * (dp[kt][2] - Dq), p[kt][3] * (dp[kt][3] - Dq));
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4_t sb = {sw[2 * ks][0], sw[2 * ks][1], sw[2 * ks + 1][0], sw[2 * ks + 1][1]};
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        acc[dt] = mfma16(lds_frag_t2(cK, kLd, 32 * ks, 32 * ks + 16, 16 * dt, lane), sb, acc[dt]);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  // dQ through LDS, as the forward's O
  static_assert(NW * 16 * kOutLd<D> <= 2 * kT * kLd, "a wave's output rows fit the block buffer");
  uint16_t *stg = &sK[0][0] + w * 16 * kOutLd<D>;
  __syncthreads();
  stage_rows16<D>(acc, scale, stg, lane);
  __syncthreads();
  flush_rows16<D>(stg, dQg + base, ld, qw, seq, lane);
}

// Backward, key side, for head dims 32, 64, 96, 128: one workgroup of 8 waves
// per (sequence, head, 128-key tile), wave w on keys k0 + 16w .. +15 (the
// lane's key row of K and V in registers), query blocks of 64 from the
// diagonal to the end of the sequence (Q and dO rows staged in LDS as they
// lie, with lse and the query side's D):
//   S = Q K^T and dP = dO V^T on MFMA (A = Q or dO rows from LDS, B = the
//   lane's key), so each lane holds 16 queries of its key; P = exp(S - lse),
//   dS = P (dP - D), both rounded to bf16 in that lane;
//   dV^T += dO^T P and dK^T += Q^T dS on MFMA, dO^T and Q^T read from the
//   staged rows by transposing LDS reads at the queries the lane holds.
// Queries past the sequence are staged with lse = +inf and D = 0 (P = dS
// = 0).  dK is scaled by 1/sqrt(d) once, at the store.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_attn_bwd_kv(const uint16_t *__restrict__ Qg, const uint16_t *__restrict__ Kg,
                                                     const uint16_t *__restrict__ Vg,
                                                     const uint16_t *__restrict__ dOg, const float *__restrict__ lse,
                                                     const float *__restrict__ Dg, uint16_t *__restrict__ dKg,
                                                     uint16_t *__restrict__ dVg, int seq, int heads, float scale) {
  constexpr int NT = 64 * NW, KT = 16 * NW;
  using R = Rows64<D, NT>;
  constexpr int kLd = R::kLd;
  __shared__ __align__(16) uint16_t sQ[2][kT * kLd];  // two stages, as on the query side
  __shared__ __align__(16) uint16_t sO[2][kT * kLd];
  __shared__ __align__(16) float sL[2][kT];
  __shared__ __align__(16) float sD[2][kT];
  const AttnTile at = attn_tile();
  const int k0 = at.tile * KT;  // the longest key tiles (most queries) start first
  const int64_t h = at.h, b = at.b;
  const int64_t ld = (int64_t)heads * D;
  const int64_t base = b * seq * ld + h * D;
  const int64_t row = (b * heads + h) * seq;
  const int t = threadIdx.x, lane = t & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int kw = k0 + 16 * w, kj = kw + c;
  const bool kok = kj < seq;

  u32x4_t kf[D / 32], vf[D / 32];  // B operands: K and V of the lane's key
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    kf[ks] = vf[ks] = u32x4_t{0u, 0u, 0u, 0u};
    if (kok) {
      kf[ks] = *reinterpret_cast<const u32x4_t *>(Kg + base + kj * ld + 32 * ks + 8 * g);
      vf[ks] = *reinterpret_cast<const u32x4_t *>(Vg + base + kj * ld + 32 * ks + 8 * g);
    }
  }
  const float c2 = scale * kLog2e;
  f32x4_t ak[D / 16], av[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) ak[i] = av[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int qb0 = k0 / kT, nqb = (seq + kT - 1) / kT;
  R rq, ro;
  // threads 0..63: lse and D of query q0 + t, used only after the next
  // loop-top wait (scaling lse here would wait for every load in flight)
  float rl = INFINITY, rd = 0.f;
  auto load_block = [&](int q0) {
    rq.load(Qg + base, ld, q0, seq, t);
    ro.load(dOg + base, ld, q0, seq, t);
    if (t < kT) {
      rl = INFINITY;
      rd = 0.f;
      if (q0 + t < seq) {
        rl = lse[row + q0 + t];
        rd = Dg[row + q0 + t];
      }
    }
  };
  auto store_block = [&](int stage) {
    rq.store(sQ[stage], t);
    ro.store(sO[stage], t);
    if (t < kT) {
      sL[stage][t] = rl * kLog2e;  // base-2 units (+inf past the sequence)
      sD[stage][t] = rd;
    }
  };
  load_block(qb0 * kT);
  store_block(0);
  if (qb0 + 1 < nqb) load_block((qb0 + 1) * kT);
  for (int qb = qb0; qb < nqb; ++qb) {
    const int q0 = qb * kT, cur = (qb - qb0) & 1;
    const uint16_t *cQ = sQ[cur], *cO = sO[cur];
    const float *cL = sL[cur], *cD = sD[cur];
    __syncthreads();  // stage cur is stored; every read of the other stage (block qb - 1) is done
    if (qb + 1 < nqb) {
      store_block(cur ^ 1);
      if (qb + 2 < nqb) load_block(q0 + 2 * kT);
    }
    if (kw > q0 + kT - 1) continue;  // every query of the block precedes every key of this wave

    f32x4_t st[4], dp[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      st[qt] = dp[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        st[qt] = mfma16(lds_frag(cQ, kLd, 16 * qt, 32 * ks, lane), kf[ks], st[qt]);
        dp[qt] = mfma16(lds_frag(cO, kLd, 16 * qt, 32 * ks, lane), vf[ks], dp[qt]);
      }
    }
    float p[4][4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const f32x4_t l4 = *reinterpret_cast<const f32x4_t *>(cL + 16 * qt + 4 * g);
#pragma unroll
      for (int v = 0; v < 4; ++v) p[qt][v] = exp2_fast(fmaf(st[qt][v], c2, -l4[v]));
    }
    if (kw + 15 > q0) {  // the diagonal block: queries before the key drop out
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (kj > q0 + 16 * qt + 4 * g + v) p[qt][v] = 0.f;
    }
    uint32_t pw[4][2], sw[4][2];  // P and dS as bf16 pairs: tile qt, queries 4g + (0,1) and (2,3)
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const f32x4_t d4 = *reinterpret_cast<const f32x4_t *>(cD + 16 * qt + 4 * g);
      float ds[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) ds[v] = p[qt][v] * (dp[qt][v] - d4[v]);
      pw[qt][0] = bf16x2_rne(p[qt][0], p[qt][1]);
      pw[qt][1] = bf16x2_rne(p[qt][2], p[qt][3]);
      sw[qt][0] = bf16x2_rne(ds[0], ds[1]);
      sw[qt][1] = bf16x2_rne(ds[2], ds[3]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4_t pb = {pw[2 * ks][0], pw[2 * ks][1], pw[2 * ks + 1][0], pw[2 * ks + 1][1]};
      const u32x4_t sb = {sw[2 * ks][0], sw[2 * ks][1], sw[2 * ks + 1][0], sw[2 * ks + 1][1]};
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        av[dt] = mfma16(lds_frag_t2(cO, kLd, 32 * ks, 32 * ks + 16, 16 * dt, lane), pb, av[dt]);
        ak[dt] = mfma16(lds_frag_t2(cQ, kLd, 32 * ks, 32 * ks + 16, 16 * dt, lane), sb, ak[dt]);
      }
    }
  }
  // dK and dV through LDS, as the forward's O (stored straight from the
  // accumulators, the two outputs interleaved, they took 126 MB of writes
  // for 67 MB of output at 8 x 512 x 32 x 128: 76 against 70 us)
  static_assert(NW * 16 * kOutLd<D> <= 2 * kT * kLd, "a wave's output rows fit a block buffer");
  uint16_t *stk = &sQ[0][0] + w * 16 * kOutLd<D>, *stv = &sO[0][0] + w * 16 * kOutLd<D>;
  __syncthreads();
  stage_rows16<D>(ak, scale, stk, lane);
  stage_rows16<D>(av, 1.0f, stv, lane);
  __syncthreads();
  flush_rows16<D>(stk, dKg + base, ld, kw, seq, lane);
  flush_rows16<D>(stv, dVg + base, ld, kw, seq, lane);
}

struct Dims {
  int64_t batch, seq, heads, d, ldp;
};

Opnd qkv(const uint16_t *p, const Dims &x) {  // [batch*seq, heads*d], per (sequence, head)
  return Opnd{p, x.heads * x.d, x.seq * x.heads * x.d, x.d};
}
Opnd scores(const uint16_t *p, const Dims &x) {  // [batch][heads][seq][ldp]
  return Opnd{p, x.ldp, x.heads * x.seq * x.ldp, x.seq * x.ldp};
}

template <bool AKC, bool BKC, bool OUT_BF16>
void gemm(const char *name, const Dims &x, Opnd a, Opnd b, void *c, bool c_scores, int M, int N, int K, float alpha,
          int mask, int krange, hipStream_t s) {
  GemmArgs g;
  g.a = a;
  g.b = b;
  g.c = c;
  g.alpha = alpha;
  g.ldc = c_scores ? x.ldp : x.heads * x.d;
  g.csb = c_scores ? x.heads * x.seq * x.ldp : x.seq * x.heads * x.d;
  g.csh = c_scores ? x.seq * x.ldp : x.d;
  g.M = M;
  g.N = N;
  g.K = K;
  g.tiles_n = (int)ceil_div(N, kT);
  g.mask = mask;
  g.krange = krange;
  const dim3 grid((unsigned)(ceil_div(M, kT) * g.tiles_n), (unsigned)x.heads, (unsigned)x.batch);
  QLORA_LAUNCH(name, (k_attn_gemm<AKC, BKC, OUT_BF16>), grid, dim3(256), 0, s, g);
}

bool fused(int64_t d) { return d == 32 || d == 64 || d == 96 || d == 128; }

// Materialised path (other head dims): float32 S and dP, bf16 P and dS,
// each [batch][heads][seq][ldp].  Fused path: the backward's D
// [batch][heads][seq] (the fused forward needs no workspace).
struct Ws {
  float *S, *dP, *D;
  uint16_t *P, *dS;
};

Ws carve(void *ws, const Dims &x) {
  char *p = static_cast<char *>(ws);
  Ws w{};
  if (fused(x.d)) {
    w.D = reinterpret_cast<float *>(p);
    return w;
  }
  const size_t e = (size_t)(x.batch * x.heads * x.seq * x.ldp);
  w.S = reinterpret_cast<float *>(p);
  p += align_up(e * 4, 256);
  w.dP = reinterpret_cast<float *>(p);
  p += align_up(e * 4, 256);
  w.P = reinterpret_cast<uint16_t *>(p);
  p += align_up(e * 2, 256);
  w.dS = reinterpret_cast<uint16_t *>(p);
  return w;
}

}  // namespace

size_t attention_workspace_bytes(int64_t batch, int64_t seq, int64_t heads, int64_t d) {
  const size_t ldp = align_up((size_t)seq, 8);
  if (fused(d)) return align_up((size_t)(batch * heads * seq) * 4, 256);
  const size_t e = (size_t)(batch * heads * seq) * ldp;
  return 2 * align_up(e * 4, 256) + 2 * align_up(e * 2, 256);
}

hipError_t launch_attention_fwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V, uint16_t *O, float *lse,
                                int64_t batch, int64_t seq, int64_t heads, int64_t d, void *ws, hipStream_t s) {
  const Dims x{batch, seq, heads, d, (int64_t)align_up((size_t)seq, 8)};
  const Ws w = carve(ws, x);
  const float scale = (float)(1.0 / std::sqrt((double)d));
  const int L = (int)seq, D = (int)d;
  if (fused(d)) {
    const int H = (int)heads;
    const dim3 gq((unsigned)ceil_div(seq, kQT), (unsigned)heads, (unsigned)batch);
    if (d == 32)
      QLORA_LAUNCH("k_attn_fwd_fused", k_attn_fwd_fused<32>, gq, dim3(512), 0, s, Q, K, V, O, lse, L, H, scale);
    else if (d == 64)
      QLORA_LAUNCH("k_attn_fwd_fused", k_attn_fwd_fused<64>, gq, dim3(512), 0, s, Q, K, V, O, lse, L, H, scale);
    else if (d == 96)
      QLORA_LAUNCH("k_attn_fwd_fused", k_attn_fwd_fused<96>, gq, dim3(512), 0, s, Q, K, V, O, lse, L, H, scale);
    else
      QLORA_LAUNCH("k_attn_fwd_fused", k_attn_fwd_fused<128>, gq, dim3(512), 0, s, Q, K, V, O, lse, L, H, scale);
    return hipGetLastError();
  }
  gemm<true, true, false>("k_attn_scores", x, qkv(Q, x), qkv(K, x), w.S, true, L, L, D, scale, 1, 0, s);
  const int64_t rows = batch * heads * seq;
  QLORA_LAUNCH("k_attn_softmax", k_attn_softmax, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, s, w.S, w.P, lse,
               rows, L, x.ldp);
  gemm<true, false, true>("k_attn_pv", x, scores(w.P, x), qkv(V, x), O, false, L, D, L, 1.0f, 0, 1, s);
  return hipGetLastError();
}

hipError_t launch_attention_bwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const uint16_t *dO, const float *lse, uint16_t *dQ, uint16_t *dK, uint16_t *dV,
                                int64_t batch, int64_t seq, int64_t heads, int64_t d, void *ws, hipStream_t s) {
  const Dims x{batch, seq, heads, d, (int64_t)align_up((size_t)seq, 8)};
  const Ws w = carve(ws, x);
  const float scale = (float)(1.0 / std::sqrt((double)d));
  const int L = (int)seq, D = (int)d;
  if (fused(d)) {
    const int H = (int)heads;
    const dim3 gq((unsigned)ceil_div(seq, kBwdRows), (unsigned)heads, (unsigned)batch);
    const dim3 gk((unsigned)ceil_div(seq, kBwdRows), (unsigned)heads, (unsigned)batch);
    const dim3 blk(64 * kBwdWaves);
#define QLORA_ATTN_BWD(DD)                                                                                     \
  QLORA_LAUNCH("k_attn_bwd_q", (k_attn_bwd_q<DD, kBwdWaves>), gq, blk, 0, s, Q, K, V, dO, lse, w.D, dQ, L, H,   \
               scale);                                                                                         \
  QLORA_LAUNCH("k_attn_bwd_kv", (k_attn_bwd_kv<DD, kBwdWaves>), gk, blk, 0, s, Q, K, V, dO, lse, w.D, dK, dV, L, \
               H, scale)
    if (d == 32) {
      QLORA_ATTN_BWD(32);
    } else if (d == 64) {
      QLORA_ATTN_BWD(64);
    } else if (d == 96) {
      QLORA_ATTN_BWD(96);
    } else {
      QLORA_ATTN_BWD(128);
    }
#undef QLORA_ATTN_BWD
    return hipGetLastError();
  }
  // (one launch computing both products over the same tiles was slower: 189 against 81 + 98 us)
  gemm<true, true, false>("k_attn_scores", x, qkv(Q, x), qkv(K, x), w.S, true, L, L, D, scale, 1, 0, s);
  gemm<true, true, false>("k_attn_dp", x, qkv(dO, x), qkv(V, x), w.dP, true, L, L, D, 1.0f, 1, 0, s);
  const int64_t rows = batch * heads * seq;
  QLORA_LAUNCH("k_attn_bwd_rows", k_attn_bwd_rows, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, s, w.S, w.dP,
               lse, w.P, w.dS, rows, L, x.ldp);
  // dV = P^T dO; dK = dS^T Q / sqrt(d): rows are keys, the contraction runs over queries >= key
  gemm<false, false, true>("k_attn_dv", x, scores(w.P, x), qkv(dO, x), dV, false, L, D, L, 1.0f, 0, 2, s);
  gemm<false, false, true>("k_attn_dk", x, scores(w.dS, x), qkv(Q, x), dK, false, L, D, L, scale, 0, 2, s);
  // dQ = dS K / sqrt(d): rows are queries, the contraction runs over keys <= query
  gemm<true, false, true>("k_attn_dq", x, scores(w.dS, x), qkv(K, x), dQ, false, L, D, L, scale, 0, 1, s);
  return hipGetLastError();
}

}  // namespace qlora

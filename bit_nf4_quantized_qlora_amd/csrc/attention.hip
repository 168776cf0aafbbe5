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
// bf16, the projections' outputs as they come.  The scores are materialised
// per (sequence, head) in the workspace: float32 S and dP, bf16 P and dS,
// each [batch][heads][seq][ldp] with ldp = seq rounded up to 8.  At the
// LLaMA-7B layer (32 heads of 128, sequence 512) that is 6 MB per sequence,
// and the six products are small next to the seven projections.
//
// Products: one batched MFMA kernel, 64 x 64 output tiles, 4 waves of 2 x 2
// 16x16x32 bf16 MFMAs, a 64-deep contraction step staged through LDS with
// the next step's operands loaded into registers meanwhile.  Each operand is
// read along whichever axis is contiguous in memory (template flags) and
// staged as it lies; fragments of row-contiguous operands come from
// transposing LDS reads.  Causality prunes work: score tiles wholly above
// the diagonal are skipped, and the products with P or dS stop (or start)
// their contraction at the tile's diagonal.
//
// Row kernels: one wave per query row.  The forward softmax takes the row
// maximum and the sum of exponentials in float32 and writes P and lse; the
// backward row pass recomputes P = exp(S - lse), sums D from P and dP, and
// writes P and dS.  Both
// write zeros for the masked entries up to the end of the diagonal tile,
// the only masked entries a product reads.
#include <cmath>

#include "qlora_internal.h"

namespace qlora {
namespace {

constexpr int kT = 64;          // output tile edge
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

// V^T for the fused forward: Vt[sequence][head][dim][key] (rows of ldp keys,
// zeros past the sequence), so the fused kernel stages V^T tiles with
// 16-byte row copies; transposing inside it took 2-byte LDS stores that
// fell on two banks.  One workgroup per (64 keys, head, sequence): coalesced
// 16-byte row loads into LDS, 16-byte stores of 8 keys of one dim.
template <int D>
__global__ __launch_bounds__(256) void k_attn_vt(const uint16_t *__restrict__ Vg, uint16_t *__restrict__ Vt, int seq,
                                                 int heads, int64_t ldp) {
  constexpr int kLd = D + 8;
  __shared__ __align__(16) uint16_t sv[kT * kLd];
  const int k0 = blockIdx.x * kT;
  const int64_t h = blockIdx.y, b = blockIdx.z;
  const int64_t ld = (int64_t)heads * D;
  const int t = threadIdx.x;
  for (int i = t; i < kT * (D / 8); i += 256) {
    const int key = k0 + i / (D / 8), col = 8 * (i % (D / 8));
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (key < seq) v = *reinterpret_cast<const u32x4_t *>(Vg + (b * seq + key) * ld + h * D + col);
    *reinterpret_cast<u32x4_t *>(sv + (i / (D / 8)) * kLd + col) = v;
  }
  __syncthreads();
  uint16_t *out = Vt + (b * heads + h) * D * ldp;
  for (int i = t; i < D * (kT / 8); i += 256) {
    const int dim = i / (kT / 8), kk = 8 * (i % (kT / 8));
    if (k0 + kk >= ldp) continue;
    u32x4_t v;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = (uint32_t)sv[(kk + 2 * j) * kLd + dim] | ((uint32_t)sv[(kk + 2 * j + 1) * kLd + dim] << 16);
    *reinterpret_cast<u32x4_t *>(out + dim * ldp + k0 + kk) = v;
  }
}

// Fused forward for head dims 32, 64, 128: one workgroup of 8 waves per
// (sequence, head, 128-query tile), wave w on queries q0 + 16w .. +15, so a
// staged key block serves 128 queries; no score matrix in memory.  Per 64-key block (causal: blocks up to the diagonal one):
//   S^T = K Q^T on MFMA (A = K rows from LDS, B = Q from registers), so each
//   lane's accumulators all belong to one query (its column l & 15): the
//   online softmax (running max m, lane-partial sum l, rescale of the
//   output) needs only a max over the lane's 16 values and lanes l ^ 16, 32;
//   O^T += V^T P^T on MFMA with P rounded to bf16: the MFMA contraction
//   slots 8g .. 8g+7 of lane group g = l >> 4 are assigned to the keys that
//   lane already holds (4g .. 4g+3 of two 16-key tiles), so P goes from
//   accumulator to operand without moving between lanes, and V^T is read
//   from a transposed LDS copy at the same keys.
// V^T comes from the copy k_attn_vt writes.  The next block's K and V^T
// are loaded into registers while this block computes.  Keys past the
// sequence are zero in LDS and masked to -inf.
constexpr int kQT = 128;  // queries per fused-forward workgroup
template <int D>
__global__ __launch_bounds__(512) void k_attn_fwd_fused(const uint16_t *__restrict__ Qg, const uint16_t *__restrict__ Kg,
                                                        const uint16_t *__restrict__ Vt, uint16_t *__restrict__ Og,
                                                        float *__restrict__ lse, int seq, int heads, int64_t ldp,
                                                        float scale) {
  constexpr int kLdK = D + 8, kLdV = kT + 8;   // LDS row strides (elements)
  constexpr int kPieces = 8 * D;               // 16-byte pieces per staged block and operand (64 x D / 8)
  constexpr int kKL = (kPieces + 511) / 512;   // per thread
  __shared__ __align__(16) uint16_t sK[kT * kLdK];
  __shared__ __align__(16) uint16_t sVt[D * kLdV];
  const int ntq = (seq + kQT - 1) / kQT;
  const int tq = ntq - 1 - (int)blockIdx.x;   // the longest query tiles start first
  const int q0 = tq * kQT;
  const int64_t h = blockIdx.y, b = blockIdx.z;
  const int64_t ld = (int64_t)heads * D;
  const int64_t base = b * seq * ld + h * D;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4, c = lane & 15;
  const int qi = q0 + 16 * w + c;             // this lane's query

  u32x4_t qf[D / 32];                          // B operand of K Q^T: Q[qi][32 ks + 8 g ..]
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    qf[ks] = u32x4_t{0u, 0u, 0u, 0u};
    if (qi < seq) qf[ks] = *reinterpret_cast<const u32x4_t *>(Qg + base + qi * ld + 32 * ks + 8 * g);
  }
  f32x4_t acc_o[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc_o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  // staging, kKL 16-byte pieces per thread and operand: piece e is K row
  // e / (D/8), dims 8 (e % (D/8)) .. +7, and V^T row (dim) e / 8, keys
  // 8 (e % 8) .. +7 of the transposed copy
  const uint16_t *vt = Vt + (b * heads + h) * D * ldp;
  u32x4_t rk[kKL], rv[kKL];
  auto load_block = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kKL; ++i) {
      const int e = t + 512 * i;
      rk[i] = rv[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (e < kPieces) {
        const int key = k0 + e / (D / 8), col = 8 * (e % (D / 8));
        if (key < seq) rk[i] = *reinterpret_cast<const u32x4_t *>(Kg + base + key * ld + col);
        const int dim = e / 8, kk = k0 + 8 * (e % 8);
        if (kk < ldp) rv[i] = *reinterpret_cast<const u32x4_t *>(vt + dim * ldp + kk);
      }
    }
  };
  const int nblk = min((seq + kT - 1) / kT, (q0 + kQT) / kT);  // key blocks up to the diagonal
  load_block(0);
  for (int kb = 0; kb < nblk; ++kb) {
    const int k0 = kb * kT;
    __syncthreads();  // the previous block's LDS reads are done
#pragma unroll
    for (int i = 0; i < kKL; ++i) {
      const int e = t + 512 * i;
      if (e < kPieces) {
        *reinterpret_cast<u32x4_t *>(sK + (e / (D / 8)) * kLdK + 8 * (e % (D / 8))) = rk[i];
        *reinterpret_cast<u32x4_t *>(sVt + (e / 8) * kLdV + 8 * (e % 8)) = rv[i];
      }
    }
    __syncthreads();
    if (kb + 1 < nblk) load_block(k0 + kT);

    // S^T for 4 key tiles of 16
    f32x4_t st[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      st[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) st[kt] = mfma16(lds_frag(sK, kLdK, 16 * kt, 32 * ks, lane), qf[ks], st[kt]);
    }
    float bm = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key = k0 + 16 * kt + 4 * g + v;
        const float x = (key <= qi && key < seq) ? st[kt][v] * scale : -INFINITY;
        st[kt][v] = x;
        bm = fmaxf(bm, x);
      }
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    // finite: block 0 holds key 0 <= qi; a later block whose keys all lie
    // past this wave's queries leaves m unchanged (corr = 1, e = 0)
    const float mn = fmaxf(m, bm);
    const float corr = expf(m - mn);
    m = mn;
    l *= corr;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc_o[i] *= corr;
    uint32_t pw[4][2];  // P as bf16 pairs: tile kt, keys 4g + (0,1) and (2,3)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float e[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        e[v] = expf(st[kt][v] - mn);
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
      for (int dt = 0; dt < D / 16; ++dt) {
        const uint16_t *vr = sVt + (16 * dt + c) * kLdV + 32 * ks + 4 * g;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(vr);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(vr + 16);
        const u32x4_t va = {lo[0], lo[1], hi[0], hi[1]};
        acc_o[dt] = mfma16(va, pb, acc_o[dt]);
      }
    }
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (qi < seq) {
    const float inv = 1.0f / l;
    uint16_t *orow = Og + base + qi * ld;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const u32x2_t o = {bf16x2_rne(acc_o[dt][0] * inv, acc_o[dt][1] * inv),
                         bf16x2_rne(acc_o[dt][2] * inv, acc_o[dt][3] * inv)};
      *reinterpret_cast<u32x2_t *>(orow + 16 * dt + 4 * g) = o;
    }
    if (g == 0) lse[(b * heads + h) * seq + qi] = m + logf(l);
  }
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

struct Ws {
  float *S, *dP;
  uint16_t *P, *dS, *Vt;  // Vt: [batch][heads][d][ldp], the fused forward's V^T
};

Ws carve(void *ws, const Dims &x) {
  const size_t e = (size_t)(x.batch * x.heads * x.seq * x.ldp);
  char *p = static_cast<char *>(ws);
  Ws w;
  w.S = reinterpret_cast<float *>(p);
  p += align_up(e * 4, 256);
  w.dP = reinterpret_cast<float *>(p);
  p += align_up(e * 4, 256);
  w.P = reinterpret_cast<uint16_t *>(p);
  p += align_up(e * 2, 256);
  w.dS = reinterpret_cast<uint16_t *>(p);
  p += align_up(e * 2, 256);
  w.Vt = reinterpret_cast<uint16_t *>(p);
  return w;
}

}  // namespace

size_t attention_workspace_bytes(int64_t batch, int64_t seq, int64_t heads, int64_t d) {
  const size_t ldp = align_up((size_t)seq, 8);
  const size_t e = (size_t)(batch * heads * seq) * ldp;
  return 2 * align_up(e * 4, 256) + 2 * align_up(e * 2, 256) + align_up((size_t)(batch * heads * d) * ldp * 2, 256);
}

hipError_t launch_attention_fwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V, uint16_t *O, float *lse,
                                int64_t batch, int64_t seq, int64_t heads, int64_t d, void *ws, hipStream_t s) {
  const Dims x{batch, seq, heads, d, (int64_t)align_up((size_t)seq, 8)};
  const Ws w = carve(ws, x);
  const float scale = (float)(1.0 / std::sqrt((double)d));
  const int L = (int)seq, D = (int)d;
  if (d == 32 || d == 64 || d == 128) {
    const dim3 grid((unsigned)ceil_div(seq, kT), (unsigned)heads, (unsigned)batch);
    const int H = (int)heads;
    const dim3 gq((unsigned)ceil_div(seq, kQT), (unsigned)heads, (unsigned)batch);
    if (d == 32) {
      QLORA_LAUNCH("k_attn_vt", k_attn_vt<32>, grid, dim3(256), 0, s, V, w.Vt, L, H, x.ldp);
      QLORA_LAUNCH("k_attn_fwd_fused", k_attn_fwd_fused<32>, gq, dim3(512), 0, s, Q, K, w.Vt, O, lse, L, H, x.ldp, scale);
    } else if (d == 64) {
      QLORA_LAUNCH("k_attn_vt", k_attn_vt<64>, grid, dim3(256), 0, s, V, w.Vt, L, H, x.ldp);
      QLORA_LAUNCH("k_attn_fwd_fused", k_attn_fwd_fused<64>, gq, dim3(512), 0, s, Q, K, w.Vt, O, lse, L, H, x.ldp, scale);
    } else {
      QLORA_LAUNCH("k_attn_vt", k_attn_vt<128>, grid, dim3(256), 0, s, V, w.Vt, L, H, x.ldp);
      QLORA_LAUNCH("k_attn_fwd_fused", k_attn_fwd_fused<128>, gq, dim3(512), 0, s, Q, K, w.Vt, O, lse, L, H, x.ldp, scale);
    }
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

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
// 16x16x32 bf16 MFMAs, a 32-deep contraction step staged through LDS with
// the next step's operands loaded into registers meanwhile.  Each operand is
// read along whichever axis is contiguous in memory (template flags); LDS
// always holds [row][contraction], so one fragment read is 16 contiguous
// bytes.  Causality prunes work: score tiles wholly above the diagonal are
// skipped, and the products with P or dS stop (or start) their contraction
// at the tile's diagonal.
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
constexpr int kKs = 32;         // contraction per step
constexpr int kLd = kKs + 8;    // LDS row stride in elements (80 B: rows start on staggered banks)

struct Opnd {
  const uint16_t *p;
  int64_t ld, sb, sh;  // row stride, then the sequence and head offsets (elements)
};

struct GemmArgs {
  Opnd a, b;
  void *c;
  int64_t ldc, csb, csh;
  int M, N, K, tiles_n;
  float alpha;
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

// The staged word into the [row][contraction] LDS tile.
template <bool KC>
__device__ __forceinline__ void store8(uint16_t *tile, int i, int k, const u32x4_t &v) {
  if (KC) {
    *reinterpret_cast<u32x4_t *>(tile + i * kLd + k) = v;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[(i + j) * kLd + k] = (uint16_t)(v[j >> 1] >> (16 * (j & 1)));
  }
}

// Thread t's staging coordinates in a 64 x 32 tile: 4 threads x 8 contraction
// elements per row (KC), or 8 threads x 8 rows per contraction index.
template <bool KC>
__device__ __forceinline__ void stage_coords(int t, int &i, int &k) {
  i = KC ? t >> 2 : (t & 7) * 8;
  k = KC ? (t & 3) * 8 : t >> 3;
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
  int ia, ka, ib, kbb;
  stage_coords<AKC>(t, ia, ka);
  stage_coords<BKC>(t, ib, kbb);

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t va = {0u, 0u, 0u, 0u}, vb = va;
  if (kb < ke) {
    va = load8<AKC>(A, g.a.ld, m0 + ia, kb + ka, g.M, ke);
    vb = load8<BKC>(B, g.b.ld, n0 + ib, kb + kbb, g.N, ke);
  }
  for (int k0 = kb; k0 < ke; k0 += kKs) {
    __syncthreads();  // the previous step's fragment reads are done
    store8<AKC>(sA, ia, ka, va);
    store8<BKC>(sB, ib, kbb, vb);
    __syncthreads();
    if (k0 + kKs < ke) {
      va = load8<AKC>(A, g.a.ld, m0 + ia, k0 + kKs + ka, g.M, ke);
      vb = load8<BKC>(B, g.b.ld, n0 + ib, k0 + kKs + kbb, g.N, ke);
    }
    mma_step<2, 2>(acc, sA, sB, kLd, wm, wn, 0, lane);
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

// Forward softmax of the (already scaled) scores, one wave per row
// r = (sequence * heads + head) * seq + query.
__global__ __launch_bounds__(256) void k_attn_softmax(const float *__restrict__ S, uint16_t *__restrict__ P,
                                                      float *__restrict__ lse, int64_t rows, int seq, int64_t ldp) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const int q = (int)(r % seq), n = q + 1;
  const float *s = S + r * ldp;
  uint16_t *p = P + r * ldp;
  float m = -INFINITY;
  for (int j = lane; j < n; j += 64) m = fmaxf(m, s[j]);
  m = wave_max(m);
  float zsum = 0.f;
  for (int j = lane; j < n; j += 64) zsum += expf(s[j] - m);
  zsum = wave_sum(zsum);
  const int span = row_span(q, seq);
  for (int j = lane; j < span; j += 64) p[j] = j < n ? f32_to_bf16_bits(expf(s[j] - m) / zsum) : uint16_t(0);
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
  float D = 0.f;
  for (int j = lane; j < n; j += 64) D += expf(s[j] - L) * dp[j];
  D = wave_sum(D);
  uint16_t *p = P + r * ldp, *ds = dS + r * ldp;
  const int span = row_span(q, seq);
  for (int j = lane; j < span; j += 64) {
    uint16_t pj = 0, dsj = 0;
    if (j < n) {
      const float e = expf(s[j] - L);
      pj = f32_to_bf16_bits(e);
      dsj = f32_to_bf16_bits(e * (dp[j] - D));
    }
    p[j] = pj;
    ds[j] = dsj;
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
  g.ldc = c_scores ? x.ldp : x.heads * x.d;
  g.csb = c_scores ? x.heads * x.seq * x.ldp : x.seq * x.heads * x.d;
  g.csh = c_scores ? x.seq * x.ldp : x.d;
  g.M = M;
  g.N = N;
  g.K = K;
  g.tiles_n = (int)ceil_div(N, kT);
  g.alpha = alpha;
  g.mask = mask;
  g.krange = krange;
  const dim3 grid((unsigned)(ceil_div(M, kT) * g.tiles_n), (unsigned)x.heads, (unsigned)x.batch);
  QLORA_LAUNCH(name, (k_attn_gemm<AKC, BKC, OUT_BF16>), grid, dim3(256), 0, s, g);
}

struct Ws {
  float *S, *dP;
  uint16_t *P, *dS;
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
  return w;
}

}  // namespace

size_t attention_workspace_bytes(int64_t batch, int64_t seq, int64_t heads) {
  const size_t e = (size_t)(batch * heads * seq * align_up((size_t)seq, 8));
  return 2 * align_up(e * 4, 256) + 2 * align_up(e * 2, 256);
}

hipError_t launch_attention_fwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V, uint16_t *O, float *lse,
                                int64_t batch, int64_t seq, int64_t heads, int64_t d, void *ws, hipStream_t s) {
  const Dims x{batch, seq, heads, d, (int64_t)align_up((size_t)seq, 8)};
  const Ws w = carve(ws, x);
  const float scale = (float)(1.0 / std::sqrt((double)d));
  const int L = (int)seq, D = (int)d;
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

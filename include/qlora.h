/*
 * qlora.h -- C ABI of libqlora.so: the frozen-base linear layer of QLoRA with
 * NF4 weights and double-quantized block constants, on AMD MI355X (gfx950).
 *
 * Method sources (web pages about QLoRA, Dettmers et al. 2023):
 *   "QLoRA, explained."  method steps 1-5 and the symbol list;
 *   "QLoRA Paper Breakdown: 4-Bit NormalFloat (NF4), Double Quantization, and
 *    Paged Optimizers"  sections 2 (codebook), 3 (blockwise quantization and
 *    double quantization), 4 (dequantization helper, forward pass, backward);
 *   "QLoRA Explained: What Actually Trains in 4 Bits? | Part 2/6"  (worked
 *    lookup and bits-per-weight arithmetic).
 *
 * Conventions shared by every call
 *   - Shapes follow PyTorch nn.Linear: W is [n, k] row-major (out, in); the
 *     activations X are [M, k]; Y and dY are [M, n]; LoRA A is [r, k] and
 *     B is [n, r] (the breakdown's L_1 = A^T, L_2 = B^T).  All row-major,
 *     densely packed (row stride == row length).
 *   - bfloat16 tensors travel as uint16_t bit patterns.
 *   - Every pointer argument to a tensor is DEVICE memory owned by the
 *     caller; the library never allocates, frees or keeps a pointer after the
 *     call returns.  Pointers must be 16-byte aligned.  Outputs must not
 *     overlap inputs or each other.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Each call checks
 *     its arguments on the host, enqueues its kernels on `stream` and returns
 *     without synchronizing; faults inside a kernel surface at the caller's
 *     next synchronization.
 *   - Return value: QLORA_OK (0) or a negative QLORA_ERR_* code; nothing is
 *     enqueued when an argument check fails.  qlora_last_error() gives a
 *     per-thread message for the last failure.
 *   - Weights must be finite; the encoding of NaN / Inf is not defined.
 */
#ifndef QLORA_H_
#define QLORA_H_

#include <stddef.h>
#include <stdint.h>

/* HIP's stream handle, declared exactly as the HIP runtime header declares it
 * (an identical typedef may be repeated), so this header needs no HIP include. */
typedef struct ihipStream_t *hipStream_t;

#ifdef __cplusplus
extern "C" {
#endif

enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL_ARG = -1,    /* a required pointer is NULL                         */
  QLORA_ERR_BAD_SHAPE = -2,   /* n < 1, k < 64, k % 64 != 0, k > 2^22, M < 0, too large */
  QLORA_ERR_BAD_RANK = -3,    /* r outside [1, 128]                                  */
  QLORA_ERR_MISALIGNED = -4,  /* a tensor pointer is not 16-byte aligned              */
  QLORA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than the *_workspace_bytes */
  QLORA_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed           */
  QLORA_ERR_BAD_ALPHA = -7,   /* alpha is not finite                                  */
  QLORA_ERR_BAD_CODEBOOK = -8 /* codebook / scales field not one of QLORA_CODEBOOK_* / _SCALES_* */
};

/*
 * 4-bit storage types (the `codebook` field of a weight).  NF4 is the
 * method's own ("QLoRA Paper Breakdown" sec. 2).  Float4 (E2M1) is the
 * 4-bit float the reading note's data-type comparison ranks below it
 * ("Why NF4 rather than any 4-bit type"): the 15 distinct OCP E2M1 values
 * +-{0, 0.5, 1, 1.5, 2, 3, 4, 6} divided by 6, ascending, code 15 repeating
 * 1.0 (never produced).  Float4 (E3M0), the table's other 4-bit float: a
 * sign and 3 exponent bits with no mantissa (field 0 is zero, no infinity
 * or NaN), so its 15 distinct values divided by the largest are 0 and
 * +-2^-j, j = 0..6; ascending, code 15 repeating 1.0 (never produced).
 * Everything else -- blocks, the nearest-level rule, double quantization,
 * dequantization -- is the same for all three.
 */
enum {
  QLORA_CODEBOOK_NF4 = 0,
  QLORA_CODEBOOK_FP4_E2M1 = 1,
  QLORA_CODEBOOK_FP4_E3M0 = 2
};

/*
 * Block constants (the `scales` field of a weight).  QLORA_SCALES_DQ is the
 * method's double quantization (scale_code, group_amax, offset).
 * QLORA_SCALES_FP32 is the single-level layout double quantization improves
 * on ("QLoRA Paper Breakdown" sec. 3, the hidden overhead of block scales:
 * one float32 per 64 weights, 4.5 bits per weight): absmax [nb] holds each
 * block's absmax and s_b = absmax_b.  Each layout needs only its own
 * buffers; the others may be NULL.
 */
enum {
  QLORA_SCALES_DQ = 0,
  QLORA_SCALES_FP32 = 1
};

/*
 * A quantized frozen weight W [n, k] in the method's own storage type: NF4
 * codes with double-quantized block constants ("QLoRA, explained.", symbol
 * list: W^NF4 plus the per-block and per-group constants; "QLoRA Paper
 * Breakdown" sec. 3).  Block b = 64 consecutive elements of row-major W (so
 * k % 64 == 0 keeps a block inside one row); group g = 256 consecutive
 * blocks; nb = n*k/64, ng = ceil(nb/256).  All buffers are device memory
 * owned by the caller.  The four calls of the layer (quantize, dequantize,
 * forward, backward) take this descriptor.
 */
typedef struct qlora_nf4_weight {
  int64_t n, k;
  uint8_t *packed;      /* [n*k/2] 4-bit codes, byte i = code[2i] | code[2i+1] << 4    */
  uint8_t *scale_code;  /* [nb] OCP E4M3FN code of (absmax_b - offset) / group_amax_g   */
  float *group_amax;    /* [ng] second-level constant: max |absmax_b - offset| in g     */
  float *offset;        /* [1] per-tensor mean of the fp32 block absmax values          */
} qlora_nf4_weight;

/*
 * Extended descriptor: the same weight in any storage type (codebook x
 * block constants above).  `size` must be set to sizeof(qlora_weight_ex) as
 * the caller compiled it; a smaller value is QLORA_ERR_BAD_CODEBOOK, so
 * fields appended later are never read from an older caller's struct.
 * codebook = QLORA_CODEBOOK_NF4 with scales = QLORA_SCALES_DQ is exactly
 * `base` passed to the plain calls.  With QLORA_SCALES_FP32 only base.n,
 * base.k, base.packed and `absmax` are read.
 */
typedef struct qlora_weight_ex {
  size_t size;            /* sizeof(qlora_weight_ex)                                   */
  qlora_nf4_weight base;  /* shape, codes and (QLORA_SCALES_DQ) the DQ constants       */
  int32_t codebook;       /* QLORA_CODEBOOK_NF4, _FP4_E2M1 or _FP4_E3M0                */
  int32_t scales;         /* QLORA_SCALES_DQ or QLORA_SCALES_FP32                      */
  float *absmax;          /* [nb] block absmax, QLORA_SCALES_FP32 only                 */
} qlora_weight_ex;

/* Sizes of the four buffers of an [n, k] weight.  Host only; no GPU use.
 * Returns QLORA_ERR_BAD_SHAPE unless n >= 1, k >= 64 and k % 64 == 0. */
int qlora_nf4_sizes(int64_t n, int64_t k, size_t *packed_bytes, size_t *scale_code_bytes,
                    size_t *group_count);

/* Workspace (device bytes) needed by qlora_quantize_nf4_dq: nb fp32 block
 * absmax values and ng fp64 group partial sums.  0 for an invalid shape. */
size_t qlora_quantize_workspace_bytes(int64_t n, int64_t k);

/*
 * Quantize a float32 weight W [n, k] (device) into `out` (its n, k must be
 * set and its four buffers allocated).
 * "QLoRA, explained." steps 1-3; "QLoRA Paper Breakdown" sec. 3 Level 1 and
 * Level 2:
 *   absmax_b = max |w| over block b;  x = fp32(w / absmax_b) (0 if absmax_b=0)
 *   code = index of the nearest NF4 level (ties to the lower index)
 *   offset = fp32( T / nb ), T in fp64, every sum a left-to-right fold: the
 *            absmax values of each group of 256 blocks, then the group sums
 *            of each run of 256 consecutive groups, then the run sums
 *   dev_b = fp32(absmax_b - offset); group_amax_g = max |dev_b| over g
 *   scale_code_b = E4M3FN round-to-nearest-even of fp32(dev_b / group_amax_g)
 *                  (0x00 when group_amax_g == 0)
 * The result is bit-for-bit deterministic.  `ws` >= qlora_quantize_workspace_bytes.
 */
int qlora_quantize_nf4_dq(const float *W, const qlora_nf4_weight *out, void *ws, size_t ws_bytes,
                          hipStream_t stream);
/* The same for any storage type: the nearest level of out->codebook, and with
 * out->scales == QLORA_SCALES_FP32 the second level skipped and absmax_b
 * stored in out->absmax. */
int qlora_quantize_ex(const float *W, const qlora_weight_ex *out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Dequantize to bfloat16: W_bf16 [n, k] (device).  "QLoRA Paper Breakdown"
 * sec. 4 Dequantization Helper; "QLoRA, explained." step 4:
 *   s_b = fp32( fp32(decode(scale_code_b) * group_amax_g) + offset )
 *   w_hat = bf16_round_nearest_even( fp32(q[code] * s_b) ), q = the NF4 levels
 * Bit-for-bit identical to the operand the fused linear kernels use.
 */
int qlora_dequant_bf16(const qlora_nf4_weight *w, uint16_t *W_bf16, hipStream_t stream);
/* The same for any storage type: q = w->codebook's levels; s_b = absmax_b
 * for QLORA_SCALES_FP32. */
int qlora_dequant_bf16_ex(const qlora_weight_ex *w, uint16_t *W_bf16, hipStream_t stream);

/* Workspace (device bytes) for qlora_linear_fwd / qlora_linear_bwd at these
 * sizes (the larger of the two).  0 for an invalid shape or rank. */
size_t qlora_linear_workspace_bytes(int64_t M, int64_t n, int64_t k, int r);

/*
 * Forward pass ("QLoRA Paper Breakdown" sec. 4 Forward Pass):
 *   H = X A^T                               [M, r], fp32 accumulation
 *   Y = bf16( X w_hat^T + s * H B^T ),      s = fp32(alpha / r)
 * w_hat is dequantized on the fly inside the kernels (never written to HBM).
 * X [M, k], A [r, k], B [n, r], Y [M, n] are bf16.  H_out [M, r] fp32 may be
 * NULL; when given it receives H for qlora_linear_bwd.  M == 0 is a no-op.
 * `ws` >= qlora_linear_workspace_bytes(M, n, k, r).
 */
int qlora_linear_fwd(const qlora_nf4_weight *w, const uint16_t *X, int64_t M, const uint16_t *A,
                     const uint16_t *B, int r, float alpha, uint16_t *Y, float *H_out, void *ws,
                     size_t ws_bytes, hipStream_t stream);
int qlora_linear_fwd_ex(const qlora_weight_ex *w, const uint16_t *X, int64_t M, const uint16_t *A,
                        const uint16_t *B, int r, float alpha, uint16_t *Y, float *H_out, void *ws,
                        size_t ws_bytes, hipStream_t stream);

/*
 * Backward pass ("QLoRA Paper Breakdown" sec. 4: dY/dX through the
 * dequantized W, dL/dW never materialized; "QLoRA, explained." step 5: only
 * the adapters receive gradients):
 *   G  = s * dY B                      [M, r]
 *   dX = bf16( dY w_hat + G A )        [M, k]   (skipped when dX == NULL)
 *   dB = bf16( s * dY^T H )            [n, r]
 *   dA = bf16( G^T X )                 [r, k]
 * H [M, r] fp32 from qlora_linear_fwd, or NULL to recompute it from X and A.
 * M == 0 writes zeros to dA and dB.  `ws` >= qlora_linear_workspace_bytes.
 */
int qlora_linear_bwd(const qlora_nf4_weight *w, const uint16_t *X, const uint16_t *dY, int64_t M,
                     const uint16_t *A, const uint16_t *B, int r, float alpha, const float *H,
                     uint16_t *dX, uint16_t *dA, uint16_t *dB, void *ws, size_t ws_bytes,
                     hipStream_t stream);
int qlora_linear_bwd_ex(const qlora_weight_ex *w, const uint16_t *X, const uint16_t *dY, int64_t M,
                        const uint16_t *A, const uint16_t *B, int r, float alpha, const float *H,
                        uint16_t *dX, uint16_t *dA, uint16_t *dB, void *ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * qlora_linear_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * qlora_linear_fwd (bit for bit); the workspace is instead a fixed 128 MiB
 * array of device memory inside the library, one per GPU it runs on, held
 * until the process ends.  Shapes whose forward workspace exceeds 128 MiB
 * return QLORA_ERR_WORKSPACE (every layer of the benchmark workloads fits:
 * the largest, a 65B down projection at M = 512, needs ~80 MB).  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (two
 * streams, two host threads) race and must be serialized by the caller.
 * Uses the current device's array; `stream` must belong to the current
 * device.  Nothing in the array needs to start at zero: every call writes
 * what it reads.
 */
int qlora_linear_fwd_noalloc(const qlora_nf4_weight *w, const uint16_t *X, int64_t M, const uint16_t *A,
                             const uint16_t *B, int r, float alpha, uint16_t *Y, float *H_out, hipStream_t stream);

/*
 * Which kernels a forward / backward call of this shape runs (host only, no
 * GPU use; the same decision the calls take).  Lets a caller or a test see
 * the path a shape takes:
 *   QLORA_PATH_TILE     256 x 256 output tiles with the weights expanded
 *                       into MFMA operands; `*_splits` > 1 when the
 *                       contraction is cut into that many equal ranges whose
 *                       float32 partial tiles are then summed in split order
 *                       (shapes with too few tiles to fill the GPU);
 *   QLORA_PATH_GEMV     forward only, 1 <= M <= 16 (either kind of block
 *                       constants): one bandwidth-bound pass over the weight;
 *   QLORA_PATH_GENERAL  input gradient only: the general kernel (n % 64 != 0,
 *                       or n * 512 at or above 2^31);
 *   QLORA_PATH_NONE     M == 0.
 * QLORA_OK, or the same argument errors as the calls.
 */
enum { QLORA_PATH_NONE = 0, QLORA_PATH_TILE = 1, QLORA_PATH_GEMV = 2, QLORA_PATH_GENERAL = 3 };
typedef struct qlora_linear_plan_info {
  int32_t fwd_path, fwd_splits;
  int32_t dx_path, dx_splits;
} qlora_linear_plan_info;
int qlora_linear_plan(int64_t M, int64_t n, int64_t k, int r, int32_t scales, qlora_linear_plan_info *out);

/*
 * Fold trained adapters into the base for deployment ("QLoRA Paper
 * Breakdown" section 'Limitations': full-rank updates merge the adapters
 * into 16-bit weights; the merged weight is section 4's W_hat + s B A).
 * The pages fix no arithmetic; this call's definition:
 *   t  = sum over j = 0 .. r-1, in that order, of B[n][j] * A[j][k]  (float64)
 *   W' = float32( float64(w_hat) + float64(s) * t ),   s = fp32(alpha / r)
 * with every float64 operation separately rounded.  Then
 *   W_merged [n, k] bf16 = bf16_round_nearest_even(W')   when W_merged != NULL;
 *   `out` (same n, k; its codebook and scales chosen by the caller) = the
 *   encoding of W' exactly as qlora_quantize_ex would give   when out != NULL.
 * Both descriptors are extended ones (any storage type on either side).
 * A [r, k] and B [n, r] bf16 as in the forward pass.  W' itself is left in
 * the first n*k*4 bytes of `ws`, which needs qlora_merge_workspace_bytes.
 */
size_t qlora_merge_workspace_bytes(int64_t n, int64_t k);
int qlora_merge_adapters(const qlora_weight_ex *w, const uint16_t *A, const uint16_t *B, int r, float alpha,
                         uint16_t *W_merged, const qlora_weight_ex *out, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * The elementwise pieces of the MLP block the adapted linears sit in (the
 * reading note's all-linear placement; the pages give no activation, and
 * the LLaMA MLP whose shapes the workloads use gates with SwiGLU):
 *   qlora_swiglu_fwd: h = bf16( silu(gate) * up ),  silu(x) = x / (1 + e^-x)
 *   qlora_swiglu_bwd: d_up = bf16( dh * silu(gate) ),
 *                     d_gate = bf16( dh * up * sigma(gate) (1 + gate (1 - sigma(gate))) )
 *   qlora_add_bf16:   out = bf16( a + b )  (the two input gradients of X)
 * count bf16 elements each, float32 inside, one rounding per output.
 * With qlora_linear_fwd / _bwd they make the block's step; its backward may
 * recompute the gate and up outputs from X (checkpointing) instead of
 * keeping them.
 */
int qlora_swiglu_fwd(const uint16_t *gate, const uint16_t *up, uint16_t *h, int64_t count, hipStream_t stream);
int qlora_swiglu_bwd(const uint16_t *gate, const uint16_t *up, const uint16_t *dh, uint16_t *d_gate, uint16_t *d_up,
                     int64_t count, hipStream_t stream);
int qlora_add_bf16(const uint16_t *a, const uint16_t *b, uint16_t *out, int64_t count, hipStream_t stream);
/* The sum of n = 2..4 bf16 tensors (host array xs of n device pointers, each
 * 16-byte aligned, count elements) in one pass: out = bf16(...bf16(bf16(
 * xs[0] + xs[1]) + xs[2]) ... + xs[n-1]), every addition in float32 and
 * rounded to bf16 before the next, so it equals n - 1 chained qlora_add_bf16
 * calls bit for bit (the layer backward's sums of input gradients).  out may
 * be the same pointer as any xs[i] (each element is read before it is
 * written); partly overlapping buffers are not allowed.  QLORA_ERR_BAD_SHAPE for n outside 2..4 or a bad count,
 * QLORA_ERR_NULL_ARG / _MISALIGNED for the pointers; nothing is launched
 * then. */
int qlora_add_bf16_n(const uint16_t *const *xs, int n, uint16_t *out, int64_t count, hipStream_t stream);

/*
 * The causal attention core between the q/k/v and o projections of the
 * decoder layer whose seven linears all hold adapters ("QLoRA, explained.",
 * all-linear placement; the LLaMA layer of "QLoRA Explained ... Part 2/6",
 * App. G).  The pages do not write attention out: this is the plain causal
 * scaled dot-product attention, per sequence and head, no positional
 * rotation (it holds no adapter):
 *   S = Q K^T / sqrt(head_dim) over keys j <= query i,  P = softmax_j(S),
 *   O = P V,  lse_i = log sum_j exp(S_ij);
 *   dV = P^T dO,  dP = dO V^T,  dS = P (dP - D), D_i = sum_j P_ij dP_ij,
 *   dQ = dS K / sqrt(head_dim),  dK = dS^T Q / sqrt(head_dim).
 * q, k, v, o, d_o, dq, dk, dv: device bf16 [batch*seq, heads*head_dim]
 * row-major (the projections' outputs; sequence b is rows b*seq ..
 * b*seq+seq-1, head h is columns h*head_dim ..), caller-owned, 16-byte
 * aligned.  lse: device float32 [batch][heads][seq], written by the forward
 * and read by the backward, which recomputes P from it (and does not read o:
 * D is summed from P and dP in float32).  P and dS are rounded to bf16 before the
 * products that take them; every product accumulates in float32 and rounds
 * its output once.
 * Shapes: head_dim a multiple of 8 in [8, 1024], heads in [1, 65535],
 * batch in [0, 65535], seq in [0, 65536]; otherwise QLORA_ERR_BAD_SHAPE.
 * batch == 0 or seq == 0 does nothing.  The workspace (device, 16-byte
 * aligned) holds, for head_dim 32, 64, 96 and 128 (fused kernels, no score
 * matrix in memory), the backward's D per query: 4 * seq * batch * heads
 * bytes (the forward uses none of it); for other head dims the float32
 * scores and their gradient and the bf16 P and dS: 12 * seq * roundup(seq,
 * 8) * batch * heads bytes; each part rounded up to 256 bytes:
 * qlora_attention_workspace_bytes (0 for shapes the calls reject).  The forward and the backward may share one workspace; the
 * backward reads nothing the forward left in it.
 */
size_t qlora_attention_workspace_bytes(int64_t batch, int64_t seq, int64_t heads, int64_t head_dim);
int qlora_attention_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *o, float *lse,
                        int64_t batch, int64_t seq, int64_t heads, int64_t head_dim, void *ws, size_t ws_bytes,
                        hipStream_t stream);
int qlora_attention_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *d_o, const float *lse,
                        uint16_t *dq, uint16_t *dk, uint16_t *dv,
                        int64_t batch, int64_t seq, int64_t heads, int64_t head_dim, void *ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * One AdamW step on an adapter tensor ("QLoRA Paper Breakdown" sec. 5, the
 * paged optimizer; "QLoRA, explained." step 6).  The pages print no update
 * rule; the published AdamW (decoupled weight decay, bias-corrected moments),
 * in float32 with every operation separately rounded, in this order:
 *   g = float(grad[i]);  m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*(g*g);
 *   p = p*decay - step_size * (m / (sqrt(v)/sqrt_bc2 + eps))
 *   decay = fp32(1 - lr*wd), step_size = fp32(lr / (1 - b1^t)),
 *   sqrt_bc2 = fp32(sqrt(1 - b2^t)),  (1-b1), (1-b2) rounded to float32,
 *   all computed on the host in float64.
 * param [count] float32 master values and m, v [count] float32 moments are
 * updated in place; param_bf16 [count] (may be NULL) receives bf16 of the
 * new values for the next forward pass; grad [count] bf16.  step = t >= 1.
 * m and v may be host memory mapped for the device (pinned / hipHostMalloc,
 * or hipMallocManaged): the paged layout, where the same accesses cross the
 * host link.  QLORA_ERR_BAD_ALPHA for hyperparameters out of range.
 */
int qlora_adamw_step(float *param, uint16_t *param_bf16, const uint16_t *grad, float *m, float *v, int64_t count,
                     float lr, float beta1, float beta2, float eps, float weight_decay, int64_t step, hipStream_t stream);

/* Host copies of the library's constants (host memory, no GPU use):
 * the 16 NF4 levels ("QLoRA Paper Breakdown" sec. 2) and the 15 float32
 * decision thresholds (T_j = smallest float32 above the exact midpoint of
 * levels j and j+1; code = number of thresholds <= x). */
void qlora_nf4_codebook(float out[16]);
void qlora_nf4_thresholds(float out[15]);
/* The same for any storage type (QLORA_CODEBOOK_*): QLORA_OK, or
 * QLORA_ERR_BAD_CODEBOOK / QLORA_ERR_NULL_ARG with `out` untouched. */
int qlora_codebook(int codebook, float out[16]);
int qlora_thresholds(int codebook, float out[15]);

/* Static text for a status code; per-thread detail of the last failure. */
const char *qlora_strerror(int status);
const char *qlora_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H_ */

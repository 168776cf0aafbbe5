// qlora_device.h -- device-side building blocks shared by the gfx950 kernels:
// the NF4 table, the 8-bit block-constant format, bf16 rounding, wave
// reductions and launch-side helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qlora.h"

// Every multiply and add below is rounded on its own: the block scale is
// defined with two roundings, and the library is also built with
// -ffp-contract=off, so no a*b+c is ever fused into one FMA.
#pragma clang fp contract(off)

namespace qlora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void *lds_ptr;        // for global_load_lds destinations
typedef __attribute__((address_space(1))) const void *glb_ptr;  // and sources

constexpr int kBlock = 64;   // weights per NF4 block ("QLoRA, explained." step 2)
constexpr int kGroup = 256;  // block constants per second-level group (step 3)

// The 16 NF4 levels ("QLoRA Paper Breakdown" sec. 2 prints them to 8
// decimals) as the float32 bit patterns of the normal-quantile construction.
// Level 6 is 0xbdba7871; parsing its printed decimals would give 0xbdba7872.
constexpr uint32_t kNF4Bits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b30u, 0xbeca32a0u, 0xbe91a24du, 0xbe3d353fu,
    0xbdba7871u, 0x00000000u, 0x3da2faffu, 0x3e24cae3u, 0x3e7c04ddu, 0x3ead033au,
    0x3ee1a4b8u, 0x3f1007abu, 0x3f3913b3u, 0x3f800000u};

// The Float4 (E2M1) storage type that "QLoRA Paper Breakdown"'s reading note
// compares NF4 with: the 15 distinct OCP E2M1 values (+-{0, 0.5, 1, 1.5, 2,
// 3, 4, 6}) divided by 6 in float32, ascending; code 15 repeats 1.0 and is
// never produced by the nearest-level rule.
constexpr uint32_t kFP4Bits[16] = {
    0xbf800000u, 0xbf2aaaabu, 0xbf000000u, 0xbeaaaaabu, 0xbe800000u, 0xbe2aaaabu,
    0xbdaaaaabu, 0x00000000u, 0x3daaaaabu, 0x3e2aaaabu, 0x3e800000u, 0x3eaaaaabu,
    0x3f000000u, 0x3f2aaaabu, 0x3f800000u, 0x3f800000u};

// The Float4 (E3M0) storage type of the same comparison: a sign and three
// exponent bits with no mantissa (field 0 is zero, no infinity or NaN), so
// the 15 distinct values are 0 and +-2^-j, j = 0..6, once divided by the
// largest magnitude; ascending, code 15 repeating 1.0 as for E2M1.
constexpr uint32_t kE3M0Bits[16] = {
    0xbf800000u, 0xbf000000u, 0xbe800000u, 0xbe000000u, 0xbd800000u, 0xbd000000u,
    0xbc800000u, 0x00000000u, 0x3c800000u, 0x3d000000u, 0x3d800000u, 0x3e000000u,
    0x3e800000u, 0x3f000000u, 0x3f800000u, 0x3f800000u};

// Storage types (the codebook field of a weight): 0 NF4, 1 Float4 (E2M1),
// 2 Float4 (E3M0).
constexpr int kCodebookNF4 = 0, kCodebookFP4 = 1, kCodebookE3M0 = 2;
__host__ __device__ constexpr const uint32_t *codebook_bits(int cb) {
  return cb == kCodebookE3M0 ? kE3M0Bits : cb == kCodebookFP4 ? kFP4Bits : kNF4Bits;
}
// Level j of codebook cb (cb uniform across the wave: scalar selects).
__host__ __device__ constexpr uint32_t codebook_level_bits(int cb, int j) {
  return cb == kCodebookE3M0 ? kE3M0Bits[j] : cb == kCodebookFP4 ? kFP4Bits[j] : kNF4Bits[j];
}

// Nearest-level decision thresholds, passed by value as a kernel argument
// (so they live in scalar registers): code = #{ j : x >= t[j] }.
struct Thresholds {
  float t[15];
};

// ---------------------------------------------------------------------------
// 8-bit block constants: OCP E4M3FN (1 sign, 4 exponent bits bias 7, 3
// mantissa bits, exponent 0 subnormal m*2^-9).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

// Round-to-nearest-even encode of |x| <= 1 (the only range the double
// quantization produces); the sign bit is kept, so -tiny encodes 0x80.
__device__ __forceinline__ uint32_t e4m3_encode_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (a < 0x1p-6f) {
    code = (uint32_t)rintf(a * 512.0f);  // subnormal grid m*2^-9; 8 is 2^-6 = code 0x08
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);    // round the mantissa to 3 bits, ties to even
    code = (u >> 20) - (120u << 3);       // rebias the exponent 127 -> 7
  }
  return code | sign;
}

// Block scale s_b = fp32(fp32(decode(c8) * group_amax) + offset): two
// separately rounded operations, never contracted into an FMA.
__device__ __forceinline__ float block_scale(uint32_t c8, float group_amax, float offset) {
  return __fadd_rn(__fmul_rn(e4m3_decode(c8), group_amax), offset);
}

// ---------------------------------------------------------------------------
// bfloat16 round-to-nearest-even of two floats into one packed dword (first
// argument in the low half): gfx950's v_cvt_pk_bf16_f32.  Checked on MI355X
// to equal integer round-to-nearest-even, u + 0x7FFF + ((u >> 16) & 1) >> 16,
// for every non-NaN float32 input, denormals included.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// NF4 expansion.  A 256-entry LDS table maps a packed byte (two codes, low
// nibble first) to its two levels, so one 8-byte LDS read serves two weights.
// w_hat = bf16_rne(fp32(q[code] * s)); every NF4 consumer goes through
// dequant_word, so the fused kernels see exactly the standalone dequant.
// ---------------------------------------------------------------------------
// Level c (0..15) selected in registers by the bits of c: a per-lane index
// into the constant array would become a memory load whose wait holds up
// the copies a kernel issues next.
__device__ __forceinline__ uint32_t nf4_level_bits(uint32_t c, int cb) {
  uint32_t v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = codebook_level_bits(cb, j);
#pragma unroll
  for (int b = 0, n = 8; b < 4; ++b, n >>= 1) {
    const uint32_t m = 0u - ((c >> b) & 1u);
#pragma unroll
    for (int j = 0; j < n; ++j) v[j] = (v[2 * j] & ~m) | (v[2 * j + 1] & m);
  }
  return v[0];
}

__device__ __forceinline__ void fill_pair_table(float2 *table, int tid, int nthreads, int cb) {
  for (int e = tid; e < 256; e += nthreads)
    table[e] = make_float2(__uint_as_float(nf4_level_bits(e & 15, cb)), __uint_as_float(nf4_level_bits(e >> 4, cb)));
}

// Eight codes (one packed dword) -> eight bf16 weights in four dwords.
__device__ __forceinline__ void dequant_word(uint32_t word, float s, const float2 *table, uint32_t out[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2 q = table[(word >> (8 * i)) & 0xFFu];
    out[i] = bf16x2_rne(__fmul_rn(q.x, s), __fmul_rn(q.y, s));
  }
}

// ---------------------------------------------------------------------------
// BF16 MFMA on 16x16 output tiles with a 32-deep contraction
// (v_mfma_f32_16x16x32_bf16).  Operand fragments: lane l holds 8 consecutive
// contraction elements kk = 8*(l>>4) .. +7 of row (l & 15), for both the A
// rows (output rows i) and the B rows (output columns j).  Accumulator: lane
// l holds C[4*(l>>4) + v][l & 15], v = 0..3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4_t mfma16(const u32x4_t &a, const u32x4_t &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// The same MFMA with the accumulator pinned to AGPRs ("+a"): the register
// allocator can then neither move accumulator tiles between register files
// nor copy them around a loop.  Only MFMAs touch these accumulators until
// mfma_acc_fence(), which waits out the MFMA result latency before ordinary
// code reads them.
__device__ __forceinline__ void mfma16_acc(f32x4_t &acc, const u32x4_t &a, const u32x4_t &b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_fence() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Fragment of a row-major LDS tile (row stride `ld` elements, contraction
// contiguous) for rows row0..row0+15 and contraction kk0..kk0+31.
__device__ __forceinline__ u32x4_t lds_frag(const uint16_t *tile, int ld, int row0, int kk0, int lane) {
  return *reinterpret_cast<const u32x4_t *>(tile + (row0 + (lane & 15)) * ld + kk0 + 8 * (lane >> 4));
}

// acc[ti][tj] += P[i0+16ti ..][kk0..kk0+31] * Q[j0+16tj ..][kk0..]^T
template <int TI, int TJ>
__device__ __forceinline__ void mma_step(f32x4_t (&acc)[TI][TJ], const uint16_t *P, const uint16_t *Q, int ld,
                                         int i0, int j0, int kk0, int lane) {
  u32x4_t a[TI], b[TJ];
#pragma unroll
  for (int t = 0; t < TI; ++t) a[t] = lds_frag(P, ld, i0 + 16 * t, kk0, lane);
#pragma unroll
  for (int t = 0; t < TJ; ++t) b[t] = lds_frag(Q, ld, j0 + 16 * t, kk0, lane);
#pragma unroll
  for (int ti = 0; ti < TI; ++ti)
#pragma unroll
    for (int tj = 0; tj < TJ; ++tj) acc[ti][tj] = mfma16(a[ti], b[tj], acc[ti][tj]);
}

// Transposes of bf16 pairs: low halves / high halves of (x, y) -> (x.h, y.h).
__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) { return (uint16_t)(bf16x2_rne(v, 0.f) & 0xFFFFu); }

// ---------------------------------------------------------------------------
// Wave (64-lane) reductions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace qlora

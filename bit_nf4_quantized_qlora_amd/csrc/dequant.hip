// dequant.hip -- standalone NF4 + double-quantization -> bfloat16 expansion.
//
// "QLoRA Paper Breakdown" sec. 4 Dequantization Helper: w_hat =
// NF4[code] * dequant(c8, c32), rounded to bf16 ("QLoRA, explained." step 4).
//
// HBM-streaming: 0.516 B read and 2 B written per weight.  A wave handles
// 256 packed dwords (2048 weights, 32 blocks): in each of 4 steps its 64
// lanes read 64 consecutive dwords (256 B) and write 64 consecutive 16 B
// chunks (1 KiB), so every load and store instruction is fully contiguous.
// Codes are looked up two at a time from a 256-entry LDS table of level
// pairs (entry = byte value, low nibble first).
#include "lora_gemm.h"

namespace qlora {
namespace {

__global__ __launch_bounds__(256) void k_dequant(const uint32_t *__restrict__ packed,
                                                 const uint8_t *__restrict__ scale_code,
                                                 const float *__restrict__ group_amax,
                                                 const float *__restrict__ offset_p,
                                                 const float *__restrict__ absmax, int64_t ndw, int codebook,
                                                 u32x4_t *__restrict__ out) {
  // packed/out start at this launch's first dword, scale_code/group_amax at
  // its first block and group (slices start on group boundaries); ndw < 2^29
  __shared__ float2 s_pair[256];
  fill_pair_table(s_pair, threadIdx.x, 256, codebook);
  const int lane = threadIdx.x & 63;
  const int64_t wave_base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 256;
  // All four steps' loads go out before any is used (past the end: zeros
  // from the buffer ranges, nothing stored).
  const int64_t nb = (ndw + 7) / 8;
  // single-level constants (absmax != NULL): s_b = absmax_b, read through
  // the scale-code slot's resource; otherwise the double-quantized decode
  const bool single = absmax != nullptr;
  const __amdgpu_buffer_rsrc_t prs = rsrc(packed, ndw * 4),
                               srs = single ? rsrc(absmax, nb * 4) : rsrc(scale_code, nb),
                               grs = rsrc(single ? absmax : group_amax, single ? 0 : ((nb + 255) / 256) * 4);
  uint32_t word[4], c8[4];
  float ga[4];
#pragma unroll
  for (int step = 0; step < 4; ++step) {
    const int64_t d = wave_base + step * 64 + lane;  // packed dword: 8 weights
    const int64_t b = d >> 3;                        // 8 dwords per 64-weight block
    const bool in = d < ndw;
    word[step] = __builtin_amdgcn_raw_buffer_load_b32(prs, in ? (uint32_t)(d * 4) : 0x80000000u, 0, 2);
    if (single) {
      c8[step] = __builtin_amdgcn_raw_buffer_load_b32(srs, in ? (uint32_t)(b * 4) : 0x80000000u, 0, 0);
      ga[step] = 0.f;
    } else {
      c8[step] = __builtin_amdgcn_raw_buffer_load_b8(srs, in ? (uint32_t)b : 0x80000000u, 0, 0);
      ga[step] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(grs, in ? (uint32_t)((b >> 8) * 4) : 0x80000000u, 0, 0));
    }
  }
  const float offset = single ? 0.f : *offset_p;
  __syncthreads();  // table
#pragma unroll
  for (int step = 0; step < 4; ++step) {
    const int64_t d = wave_base + step * 64 + lane;
    if (d >= ndw) break;
    const float s = single ? __uint_as_float(c8[step]) : block_scale(c8[step], ga[step], offset);
    uint32_t o[4];
    dequant_word(word[step], s, s_pair, o);
    const u32x4_t v = {o[0], o[1], o[2], o[3]};
    __builtin_nontemporal_store(v, out + d);
  }
}

}  // namespace

hipError_t launch_dequant(const Nf4View &w, uint16_t *out, hipStream_t s) {
  // slices of at most 2^28 dwords (1 GiB of codes), starting on group
  // boundaries (2048 dwords), keep every buffer offset 32-bit
  constexpr int64_t kSlice = int64_t(1) << 28;
  const int64_t ndw_all = w.n * w.k / 8;
  for (int64_t d0 = 0; d0 < ndw_all; d0 += kSlice) {
    const int64_t ndw = std::min(kSlice, ndw_all - d0);
    const int64_t grid = ceil_div(ndw, 4 * 256);
    QLORA_LAUNCH("k_dequant", k_dequant, dim3((unsigned)grid), dim3(256), 0, s,
                 reinterpret_cast<const uint32_t *>(w.packed) + d0, w.absmax ? nullptr : w.scale_code + d0 / 8,
                 w.absmax ? nullptr : w.group_amax + d0 / 8 / kGroup, w.offset, w.absmax ? w.absmax + d0 / 8 : nullptr,
                 ndw, w.codebook,
                 reinterpret_cast<u32x4_t *>(out) + d0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qlora

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
#include "qlora_internal.h"

namespace qlora {
namespace {

__global__ __launch_bounds__(256) void k_dequant(const uint32_t *__restrict__ packed,
                                                 const uint8_t *__restrict__ scale_code,
                                                 const float *__restrict__ group_amax,
                                                 const float *__restrict__ offset_p, int64_t ndw,
                                                 u32x4_t *__restrict__ out) {
  __shared__ float2 s_pair[256];
  fill_pair_table(s_pair, threadIdx.x, 256);
  __syncthreads();
  const float offset = *offset_p;
  const int lane = threadIdx.x & 63;
  const int64_t wave_base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 256;
#pragma unroll
  for (int step = 0; step < 4; ++step) {
    const int64_t d = wave_base + step * 64 + lane;  // packed dword: 8 weights
    if (d >= ndw) break;
    const uint32_t word = __builtin_nontemporal_load(packed + d);
    const int64_t b = d >> 3;  // 8 dwords per 64-weight block
    const float s = block_scale(scale_code[b], group_amax[b >> 8], offset);
    uint32_t o[4];
    dequant_word(word, s, s_pair, o);
    const u32x4_t v = {o[0], o[1], o[2], o[3]};
    __builtin_nontemporal_store(v, out + d);
  }
}

}  // namespace

hipError_t launch_dequant(const Nf4View &w, uint16_t *out, hipStream_t s) {
  const int64_t ndw = w.n * w.k / 8;
  const int64_t grid = ceil_div(ndw, 4 * 256);
  QLORA_LAUNCH("k_dequant", k_dequant, dim3((unsigned)grid), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t *>(w.packed), w.scale_code, w.group_amax, w.offset, ndw,
                     reinterpret_cast<u32x4_t *>(out));
  return hipGetLastError();
}

}  // namespace qlora

// Weighted combine back to token order.
//
// Method: a token's output is the sum over its k selected experts of the gate
// weight times that expert's output (ops-transformer MoE article, "原理" Step
// 4; MegaBlocks chapter 1, section 4.3, binned_scatter).  A dropped slot adds
// nothing and the remaining weights are not rescaled (same chapter, sections
// 3 and 4.5).
//
// gfx950 design: one thread per (token, 8 consecutive columns); it reads the
// k expert-output rows through slot_pos with 16-byte (bf16) or 32-byte (fp32)
// loads, all of them in flight together, and sums w_j * O in fp32, j ascending,
// in registers -- the [tokens, k, h] temporary of the page's scatter-then-sum is
// never formed.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

template <typename OT, typename YT, int KM>
__global__ __launch_bounds__(256) void combine_kernel(const OT* __restrict__ O, int parts, size_t part_stride,
                                                      const int* __restrict__ slot_pos,
                                                      const float* __restrict__ topk_w, int T, int h, int k,
                                                      YT* __restrict__ y) {
  const int groups = h >> 3;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)T * groups) return;
  const int t = (int)(gid / groups);
  const int c = (int)(gid % groups) * 8;
  // k <= KM slots: their rows and weights first, then the first part of every kept row, so
  // that all the row loads are in flight together; the sums then go in ascending j (and s)
  int pos[KM];
  float w[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    pos[j] = j < k ? slot_pos[(size_t)t * k + j] : -1;
    w[j] = j < k ? topk_w[(size_t)t * k + j] : 0.f;
  }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if constexpr (sizeof(OT) == 2) {
    u32x4 v[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (pos[j] >= 0) v[j] = *(const u32x4*)(O + (size_t)pos[j] * h + c);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (pos[j] < 0) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += w[j] * __uint_as_float(v[j][i] << 16);
        acc[2 * i + 1] += w[j] * __uint_as_float(v[j][i] & 0xFFFF0000u);
      }
    }
  } else {
    floatx4 v0[KM], v1[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (pos[j] >= 0) {
        const OT* src = O + (size_t)pos[j] * h + c;
        v0[j] = *(const floatx4*)src;
        v1[j] = *(const floatx4*)(src + 4);
      }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (pos[j] < 0) continue;
      const OT* src = O + (size_t)pos[j] * h + c;
      for (int s = 1; s < parts; ++s) {  // K parts of a split down projection, ascending
        v0[j] += *(const floatx4*)(src + s * part_stride);
        v1[j] += *(const floatx4*)(src + s * part_stride + 4);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += w[j] * v0[j][i];
        acc[4 + i] += w[j] * v1[j][i];
      }
    }
  }
  YT* dst = y + (size_t)t * h + c;
  if constexpr (sizeof(YT) == 2) {
    *(u32x4*)dst = u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                         pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  } else {
    *(floatx4*)dst = floatx4{acc[0], acc[1], acc[2], acc[3]};
    *(floatx4*)(dst + 4) = floatx4{acc[4], acc[5], acc[6], acc[7]};
  }
}

}  // namespace

hipError_t launch_combine(const void* O, bool o_f32, int o_parts, size_t o_part_stride, const int* slot_pos,
                          const float* topk_w, int T, int h, int k, bool bf16, void* y, hipStream_t st) {
  if (o_parts < 1 || (o_parts > 1 && !o_f32)) return hipErrorInvalidValue;
  const int64_t n = (int64_t)T * (h / 8);
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (grid == 0) return hipSuccess;
  if (k < 1 || k > 16) return hipErrorInvalidValue;
#define MOE_COMBINE(KM)                                                                                        \
  do {                                                                                                         \
    if (bf16 && o_f32)                                                                                         \
      hipLaunchKernelGGL((combine_kernel<float, bf16_t, KM>), dim3(grid), dim3(256), 0, st, (const float*)O,  \
                         o_parts, o_part_stride, slot_pos, topk_w, T, h, k, (bf16_t*)y);                      \
    else if (bf16)                                                                                             \
      hipLaunchKernelGGL((combine_kernel<bf16_t, bf16_t, KM>), dim3(grid), dim3(256), 0, st, (const bf16_t*)O, \
                         1, (size_t)0, slot_pos, topk_w, T, h, k, (bf16_t*)y);                                \
    else                                                                                                       \
      hipLaunchKernelGGL((combine_kernel<float, float, KM>), dim3(grid), dim3(256), 0, st, (const float*)O,   \
                         o_parts, o_part_stride, slot_pos, topk_w, T, h, k, (float*)y);                       \
  } while (0)
  if (k <= 2) MOE_COMBINE(2);
  else if (k <= 4) MOE_COMBINE(4);
  else if (k <= 8) MOE_COMBINE(8);
  else MOE_COMBINE(16);
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe

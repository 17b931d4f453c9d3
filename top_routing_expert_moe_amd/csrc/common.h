// Shared device helpers for the gfx950 MoE kernels: bf16 conversion, vector
// types, wave-level reductions.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bf16 bit pattern in memory

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Element type traits for the two storage dtypes.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(bf16_t* p, size_t i, float v) {
    p[i] = (bf16_t)f32_to_bf16_bits(v);
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
    uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
// SiLU for the bf16 GEMM epilogue: hardware exp2 and reciprocal (relative error ~1e-6,
// far below the bf16 rounding that follows).
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}
__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

// Height of an expert's m-tiles in the grouped GEMMs, given the launch's tile height fh, the
// launch's threshold `big` and the expert's row count: fh, except that in a launch of
// 128-row tiles an expert with at least `big` rows takes 256-row tiles.  Every builder of
// a tile list and every GEMM that walks one uses this same function with the same big.
__host__ __device__ __forceinline__ int m_tile_rows(int rows, int fh, int big) {
  return (fh == 128 && rows >= big) ? 256 : fh;
}
// an expert's m-tiles: ceil(rows / m_tile_rows(rows, fh, big)); the last may be partial
__host__ __device__ __forceinline__ int m_tile_count(int rows, int fh, int big) {
  const int fe = m_tile_rows(rows, fh, big);
  return (rows + fe - 1) / fe;
}

// Binary search: the expert e with tile_off[e] <= mt < tile_off[e+1] (E >= 1).
__device__ __forceinline__ int find_expert(const int* __restrict__ tile_off, int E, int mt) {
  int lo = 0, hi = E;  // invariant: tile_off[lo] <= mt < tile_off[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (tile_off[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace moe

// Shared definitions of libpkv's gfx950 device code.
//
// Cache layout (fixed by pkv.h), per cache:
//   K[num_blocks][H_kv][d / X][B][X]   with X = 16 / bytes_per_scalar
//   V[num_blocks][H_kv][d][B]
// A token's key row is cut into 16-byte pieces and piece p of all B tokens of
// a block lies together, so the 16 token rows of one matrix-core operand tile
// read 4 pieces as contiguous runs; a value tile is stored transposed, one
// row of B tokens per head dimension, which is the value operand's layout.
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

struct F32 {
  static constexpr int kItem = 4;
};
struct BF16 {
  static constexpr int kItem = 2;
};

// 16-byte load marked non-temporal: K/V tiles are read once per step, and the
// nt hint lets the memory system stream them (measured on MI355X: random
// 4 KiB tiles read at ~6.8 TB/s with it, ~6.0 TB/s without).
__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  const u32x4_t u = {v.x, v.y, v.z, v.w};
  return __builtin_bit_cast(bf16x8_t, u);
}

// Cross-row steps: lane l receives the partner value from lane l ^ 16 or
// l ^ 32 through the gfx950 permlane swaps (no LDS traffic).
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int item_size(int32_t kv_dtype) { return kv_dtype == PKV_F32 ? 4 : kv_dtype == PKV_BF16 ? 2 : 0; }
inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace pkv

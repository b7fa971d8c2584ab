// Shared definitions of libpkv's gfx950 device code.
//
// Cache layout (fixed by pkv.h), per cache:
//   V[num_blocks][H_kv][B][d]
//   K[num_blocks][H_kv][d / X][B][X]   with X = 128 / bytes_per_scalar
// A token's key row is cut into 128-byte pieces; piece p of all B tokens of a
// block lies together.  One wave-wide 16-byte load (1 KiB) then covers piece
// p of 8 consecutive tokens, giving each group of 8 lanes one token's piece;
// two such loads per piece cover a 16-token group, so every lane ends up with
// the same 16-byte columns of two tokens.  Values keep plain rows: a lane keeps
// the same output dimensions for every token it visits.
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kWave = 64;
constexpr int kKeyPiece = 128;  // bytes of one key piece

typedef short bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct F32 {
  static constexpr int kItem = 4;
  static constexpr uint32_t kSignMask = 0x80000000u;
};
struct BF16 {
  static constexpr int kItem = 2;
  static constexpr uint32_t kSignMask = 0x80008000u;
};

// 16-byte load marked non-temporal: K/V tiles are read once per step, and the
// nt hint lets the memory system stream them (measured on MI355X: random
// 4 KiB tiles read at ~6.8 TB/s with it, ~6.0 TB/s without).
__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }
__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  const u32x4_t u = {v.x, v.y, v.z, v.w};
  return __builtin_bit_cast(bf16x8_t, u);
}

// Partial dot product of 16 bytes of q with 16 bytes of k, accumulated in fp32.
__device__ __forceinline__ float dot16(BF16, const uint4& q, const uint4& k, float acc) {
  // v_dot2_f32_bf16: two exact bf16 products added to an fp32 accumulator.
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.x), as_bf16x2(k.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.y), as_bf16x2(k.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.z), as_bf16x2(k.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.w), as_bf16x2(k.w), acc, false);
  return acc;
}
__device__ __forceinline__ float dot16(F32, const uint4& q, const uint4& k, float acc) {
  acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

// Widen 16 bytes of stored values to fp32 (exact).
__device__ __forceinline__ void widen16(BF16, const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16);
  f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16);
  f[7] = __uint_as_float(v.w & 0xffff0000u);
}
__device__ __forceinline__ void widen16(F32, const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}

// DPP lane permutations inside a row of 16 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7-i within each half-row of 8

// Sum over the 8 lanes of a half-row (all lanes receive the total).
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowHalfMirror>(x);
  return x;
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

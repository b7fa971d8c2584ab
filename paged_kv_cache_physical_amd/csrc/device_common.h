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

// The same maxima with NaN propagation (no quieting of the operands).
__device__ __forceinline__ float nmax_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float nmax_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// Raw buffer resource over `bytes` bytes at p (32-bit data format); an access
// at an offset >= bytes is dropped (a store) or reads zeros (a load).
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kRsrcWord3);
}
constexpr int kNowhere = 0x40000000;  // a buffer offset past every resource: the access is dropped

// Cache-policy bits of a gfx950 buffer store: sc0 (bit 0), nt (bit 1), sc1
// (bit 4).  kStoreThrough (sc0 sc1 nt) writes through L2 as a streaming
// store.  One token's rows cover only a few bytes of each cache line they
// touch; left dirty in L2, such partly written lines made a later read of the
// same tile in the same kernel stall for several microseconds on MI355X.
constexpr int kStoreDefault = 0;
constexpr int kStoreThrough = 1 | 2 | 16;

// Stores one (token, head) pair of rows into its cache tiles: the K tile
// [d / X][B][X] (X = 16 bytes of scalars; lane c < d / X stores piece c) and
// the V tile [d][B] (lane l stores dims l and l + 64 in column `off`).  kv is
// the lane's key piece, v0 and v1 its values; kAux is the stores' cache policy.
template <class T, int kAux>
__device__ __forceinline__ void store_token_rows(char* k_cache, char* v_cache, int64_t tile, int off, int block_size,
                                                 int head_dim, int lane, uint4 kv, T v0, T v1) {
  constexpr int E = 16 / static_cast<int>(sizeof(T));
  const int pieces = head_dim / E;
  const int tile_bytes = head_dim * block_size * static_cast<int>(sizeof(T));
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k_cache + tile * tile_bytes, tile_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v_cache + tile * tile_bytes, tile_bytes);
  const u32x4_t k4 = {kv.x, kv.y, kv.z, kv.w};
  __builtin_amdgcn_raw_buffer_store_b128(k4, rk, lane < pieces ? (lane * block_size + off) * 16 : kNowhere, 0, kAux);
  const int v_off = (lane * block_size + off) * static_cast<int>(sizeof(T));
  const int v_off_hi = head_dim > 64 ? ((64 + lane) * block_size + off) * static_cast<int>(sizeof(T)) : kNowhere;
  if constexpr (sizeof(T) == 2) {
    __builtin_amdgcn_raw_buffer_store_b16(v0, rv, v_off, 0, kAux);
    __builtin_amdgcn_raw_buffer_store_b16(v1, rv, v_off_hi, 0, kAux);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(v0, rv, v_off, 0, kAux);
    __builtin_amdgcn_raw_buffer_store_b32(v1, rv, v_off_hi, 0, kAux);
  }
}

inline int item_size(int32_t kv_dtype) { return kv_dtype == PKV_F32 ? 4 : kv_dtype == PKV_BF16 ? 2 : 0; }
inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Launches the decode step's token write (cache_ops.hip): every sequence's
// token at position n - 1, through its block table.
hipError_t launch_write_last_token(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks, int32_t max_context_len, int32_t kv_dtype, hipStream_t stream);

// Runs of at most 16 / G queries per sequence on the decode kernel
// (attention.hip); PKV_ERR_UNSUPPORTED when the batch does not fit that path.
// skip_long: runs longer than max_query_len are left alone (another launch
// takes them) instead of being filled with NaN.
pkv_status runs_listed(float* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
                       int32_t num_query_rows, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t max_blocks, int32_t max_context_len,
                       int32_t max_query_len, bool skip_long, float scale, void* workspace, size_t workspace_bytes,
                       int32_t kv_dtype, hipStream_t stream);
size_t runs_listed_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_context_len, int32_t max_query_len);

}  // namespace pkv

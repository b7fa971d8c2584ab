// Cache writes and copies for gfx950: the slot scatter of new tokens'
// keys/values (reshape_and_cache), whole-block copies for copy-on-write and for
// swapping between device and host memory, and a plain streaming-read probe
// used to measure the HBM read ceiling.

#include <algorithm>
#include <cstdlib>
#include <vector>

#include "device_common.h"

namespace pkv {
namespace {

// One wave moves the key and value of one (token, head).  K tile
// [d / X][B][X] (X = 16 bytes): lane c < d / X stores piece c of the key row.
// V tile [d][B]: lane l stores the values of dims l, l + 64, ... into column
// `off` of the tile, so a store instruction covers consecutive rows.  The
// stores take the default write-back policy: when many tokens of one block
// are written, L2 merges their partial lines before they reach HBM (measured
// on MI355X: 1.2 TB/s for a 64K-token fill, 0.2 TB/s written through).
template <class T>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(const char* __restrict__ k_new,
                                                                const char* __restrict__ v_new,
                                                                char* __restrict__ k_cache, char* __restrict__ v_cache,
                                                                const int64_t* __restrict__ slots, int32_t num_tokens,
                                                                int32_t num_heads, int32_t block_size, int32_t head_dim,
                                                                int64_t num_slots) {
  constexpr int E = 16 / static_cast<int>(sizeof(T));  // scalars per key piece
  const int lane = threadIdx.x & 63;
  // token * H + head, wave-uniform
  const int64_t th = static_cast<int64_t>(blockIdx.x) * (blockDim.x / 64) +
                     __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / 64));
  if (th >= static_cast<int64_t>(num_tokens) * num_heads) return;
  const int64_t t = th / num_heads;
  const int h = static_cast<int>(th % num_heads);
  const int pieces = head_dim / E;  // <= 64
  // The row loads do not depend on the slot: issue them first.
  const T* krow = reinterpret_cast<const T*>(k_new) + th * head_dim;
  const T* vrow = reinterpret_cast<const T*>(v_new) + th * head_dim;
  const uint4 kv = *reinterpret_cast<const uint4*>(krow + (lane < pieces ? lane : 0) * E);
  const T v0 = vrow[lane];
  const T v1 = head_dim > 64 ? vrow[64 + lane] : T(0);
  // The slot list is never written here: a scalar load through the constant address space.
  const int64_t slot = ((const __attribute__((address_space(4))) int64_t*)slots)[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int off = static_cast<int>(slot % block_size);
  store_token_rows<T, kStoreDefault>(k_cache, v_cache, blk * num_heads + h, off, block_size, head_dim, lane, kv, v0, v1);
}

// The decode step's token write when the attention kernel cannot do it: one
// wave per (sequence, head) stores the token at position n - 1 into the slot
// its block table gives (block_tables[s][(n - 1) / B], offset (n - 1) % B).
// Sequences with n <= 0, n > max_context_len or n > max_blocks * B, and block
// ids outside the pool, are skipped.  One token per block leaves every line it
// touches partly written, so the stores go through L2 (kStoreThrough): the
// attention kernel that reads the tile next does not stall on them.
template <class T>
__global__ __launch_bounds__(256) void write_last_token_kernel(const char* __restrict__ k_new,
                                                               const char* __restrict__ v_new, char* k_cache,
                                                               char* v_cache, const int32_t* __restrict__ block_tables,
                                                               const int32_t* __restrict__ context_lens,
                                                               int32_t num_seqs, int32_t num_heads, int32_t block_size,
                                                               int32_t head_dim, int32_t num_blocks, int32_t max_blocks,
                                                               int32_t max_context_len) {
  constexpr int E = 16 / static_cast<int>(sizeof(T));
  const int lane = threadIdx.x & 63;
  const int64_t sh = static_cast<int64_t>(blockIdx.x) * (blockDim.x / 64) +
                     __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / 64));
  if (sh >= static_cast<int64_t>(num_seqs) * num_heads) return;
  const int64_t s = sh / num_heads;
  const int h = static_cast<int>(sh % num_heads);
  const int n = context_lens[s];
  if (n <= 0 || n > max_context_len || static_cast<int64_t>(n) > static_cast<int64_t>(max_blocks) * block_size) return;
  const int32_t blk = block_tables[s * max_blocks + (n - 1) / block_size];
  if (static_cast<unsigned>(blk) >= static_cast<unsigned>(num_blocks)) return;
  const int pieces = head_dim / E;
  const T* krow = reinterpret_cast<const T*>(k_new) + sh * head_dim;
  const T* vrow = reinterpret_cast<const T*>(v_new) + sh * head_dim;
  const uint4 kv = *reinterpret_cast<const uint4*>(krow + (lane < pieces ? lane : 0) * E);
  const T v0 = vrow[lane];
  const T v1 = head_dim > 64 ? vrow[64 + lane] : T(0);
  store_token_rows<T, kStoreThrough>(k_cache, v_cache, static_cast<int64_t>(blk) * num_heads + h, (n - 1) % block_size,
                                     block_size, head_dim, lane, kv, v0, v1);
}

// grid = (pairs, 2 caches, splits): each workgroup copies a slice of one block.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* k_cache, char* v_cache, const int32_t* __restrict__ pairs,
                                                          int32_t num_blocks, int64_t block_bytes) {
  const int pair = blockIdx.x;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (static_cast<unsigned>(src) >= static_cast<unsigned>(num_blocks) ||
      static_cast<unsigned>(dst) >= static_cast<unsigned>(num_blocks))
    return;
  char* base = blockIdx.y ? v_cache : k_cache;
  const uint4* s = reinterpret_cast<const uint4*>(base + src * block_bytes);
  uint4* d = reinterpret_cast<uint4*>(base + dst * block_bytes);
  const int64_t n16 = block_bytes / 16;
  for (int64_t i = static_cast<int64_t>(blockIdx.z) * blockDim.x + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.z) * blockDim.x)
    d[i] = s[i];
}

// grid = (pairs, 2 caches, splits): each workgroup copies a slice of one block
// from one cache pair to the other.  One side may be page-locked host memory,
// reached over the host link: each thread keeps kSwapUnroll 16-byte loads in
// flight before storing, so that reads across the link overlap.
constexpr int kSwapUnroll = 4;

__global__ __launch_bounds__(256) void swap_blocks_kernel(const char* src_k, const char* src_v, char* dst_k,
                                                          char* dst_v, const int32_t* pairs, int32_t src_blocks,
                                                          int32_t dst_blocks, int64_t block_bytes) {
  const int pair = blockIdx.x;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (static_cast<unsigned>(src) >= static_cast<unsigned>(src_blocks) ||
      static_cast<unsigned>(dst) >= static_cast<unsigned>(dst_blocks))
    return;
  const uint4* s = reinterpret_cast<const uint4*>((blockIdx.y ? src_v : src_k) + src * block_bytes);
  uint4* d = reinterpret_cast<uint4*>((blockIdx.y ? dst_v : dst_k) + dst * block_bytes);
  const int64_t n16 = block_bytes / 16;
  const int64_t step = static_cast<int64_t>(gridDim.z) * blockDim.x * kSwapUnroll;
  for (int64_t i = static_cast<int64_t>(blockIdx.z) * blockDim.x * kSwapUnroll + threadIdx.x; i < n16; i += step) {
    uint4 v[kSwapUnroll];
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
      const int64_t j = i + static_cast<int64_t>(u) * blockDim.x;
      if (j < n16) v[u] = s[j];
    }
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
      const int64_t j = i + static_cast<int64_t>(u) * blockDim.x;
      if (j < n16) d[j] = v[u];
    }
  }
}

// Plain streaming read: each workgroup owns consecutive 256 KiB chunks and
// its threads keep 16 non-temporal 16-byte loads in flight; the words are
// xor-folded and stored only for an impossible value, which keeps the loads
// live without writing anything.
constexpr int64_t kProbeChunk16 = 256 * 1024 / 16;
constexpr int kProbeUnroll = 16;

__global__ __launch_bounds__(256) void hbm_read_probe_kernel(const uint4* __restrict__ src, int64_t n16,
                                                             uint32_t* __restrict__ sink) {
  uint32_t x = 0;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kProbeChunk16; base < n16;
       base += static_cast<int64_t>(gridDim.x) * kProbeChunk16) {
    const int64_t end = base + kProbeChunk16 < n16 ? base + kProbeChunk16 : n16;
    int64_t i = base + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * 256 < end; i += kProbeUnroll * 256) {
      uint4 v[kProbeUnroll];
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) v[u] = load_nt(src + i + u * 256);
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += 256) {
      const uint4 v = load_nt(src + i);
      x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if (x == 0x9e3779b9u && threadIdx.x == 0x3ff) sink[0] = x;  // never taken for blockDim <= 1023
}

}  // namespace

hipError_t launch_write_last_token(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks, int32_t max_context_len, int32_t kv_dtype, hipStream_t stream) {
  const int64_t grid = ceil_div64(static_cast<int64_t>(num_seqs) * num_kv_heads, 4);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  auto kernel = item_size(kv_dtype) == 4 ? write_last_token_kernel<uint32_t> : write_last_token_kernel<uint16_t>;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, static_cast<const char*>(k_new),
                     static_cast<const char*>(v_new), static_cast<char*>(k_cache), static_cast<char*>(v_cache),
                     block_tables, context_lens, num_seqs, num_kv_heads, block_size, head_dim, num_blocks, max_blocks,
                     max_context_len);
  return hipGetLastError();
}

}  // namespace pkv

using namespace pkv;

namespace {
// Debug validation, on when the environment variable PKV_DEBUG is set to
// anything but "" or "0" (read once): the write targets of one call are copied
// to the host (the call then waits for its stream) and must be distinct, since
// two writers of one slot or one block would race.
bool debug_checks() {
  static const bool on = [] {
    const char* v = std::getenv("PKV_DEBUG");
    return v && v[0] && !(v[0] == '0' && v[1] == 0);
  }();
  return on;
}

template <class T>
bool fetch(std::vector<T>& host, const T* dev, size_t count, hipStream_t stream) {
  host.resize(count);
  return hipMemcpyAsync(host.data(), dev, count * sizeof(T), hipMemcpyDeviceToHost, stream) == hipSuccess &&
         hipStreamSynchronize(stream) == hipSuccess;
}

// Distinct values among those in [0, limit) (others are skipped by the kernels).
template <class T>
bool distinct_in_range(std::vector<T> v, int64_t limit) {
  v.erase(std::remove_if(v.begin(), v.end(), [&](T x) { return x < 0 || x >= limit; }), v.end());
  std::sort(v.begin(), v.end());
  return std::adjacent_find(v.begin(), v.end()) == v.end();
}
}  // namespace

extern "C" {

pkv_status pkv_reshape_and_cache(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                 const int64_t* slots, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, int32_t kv_dtype, hipStream_t stream) {
  const int item = item_size(kv_dtype);
  if (item == 0) return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PKV_ERR_INVALID_ARG;
  if ((head_dim != 64 && head_dim != 128) || (block_size != 16 && block_size != 32)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slots) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_INVALID_ARG;
  if (debug_checks()) {
    std::vector<int64_t> h;
    if (!fetch(h, slots, static_cast<size_t>(num_tokens), stream)) return PKV_ERR_HIP;
    if (!distinct_in_range(h, static_cast<int64_t>(num_blocks) * block_size)) return PKV_ERR_INVALID_ARG;
  }
  const int64_t waves = static_cast<int64_t>(num_tokens) * num_kv_heads;  // one per (token, head)
  const int64_t grid = ceil_div64(waves, 4);
  if (grid > 0x7fffffff) return PKV_ERR_INVALID_ARG;
  auto kernel = item == 4 ? reshape_and_cache_kernel<uint32_t> : reshape_and_cache_kernel<uint16_t>;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, static_cast<const char*>(k_new),
                     static_cast<const char*>(v_new), static_cast<char*>(k_cache), static_cast<char*>(v_cache), slots,
                     num_tokens, num_kv_heads, block_size, head_dim,
                     static_cast<int64_t>(num_blocks) * block_size);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t n_pairs, int32_t num_blocks,
                           int64_t block_bytes, hipStream_t stream) {
  if (n_pairs < 0 || num_blocks <= 0 || block_bytes <= 0 || block_bytes % 16) return PKV_ERR_INVALID_ARG;
  if (n_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID_ARG;
  if (debug_checks()) {
    std::vector<int32_t> h;
    if (!fetch(h, pairs, 2 * static_cast<size_t>(n_pairs), stream)) return PKV_ERR_HIP;
    std::vector<int32_t> dst;
    std::vector<char> is_src(static_cast<size_t>(num_blocks), 0);
    for (int32_t i = 0; i < n_pairs; ++i) {
      const int32_t src = h[2 * i], d = h[2 * i + 1];
      if (src < 0 || src >= num_blocks || d < 0 || d >= num_blocks) continue;  // pairs the kernel skips
      dst.push_back(d);
      is_src[static_cast<size_t>(src)] = 1;
    }
    if (!distinct_in_range(dst, num_blocks)) return PKV_ERR_INVALID_ARG;
    // all pairs run at once: a block that is read and written in one call races
    for (const int32_t d : dst)
      if (is_src[static_cast<size_t>(d)]) return PKV_ERR_INVALID_ARG;
  }
  const int64_t n16 = block_bytes / 16;
  const int64_t splits = ceil_div64(n16, 256);
  const unsigned z = static_cast<unsigned>(splits < 16 ? splits : 16);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n_pairs, 2, z), dim3(256), 0, stream, static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), pairs, num_blocks, block_bytes);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

namespace {
// The address the GPU uses for `bytes` bytes at p, or nullptr when p is not
// device memory or page-locked HIP host memory, or the range runs past the
// allocation.
const void* gpu_reachable(const void* p, int64_t bytes) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of a refused query
    return nullptr;
  }
  void* base = nullptr;
  size_t size = 0;
  const void* dp = nullptr;
  if (attr.type == hipMemoryTypeDevice) {
    dp = p;
  } else if (attr.type == hipMemoryTypeHost) {
    void* mapped = nullptr;
    if (hipHostGetDevicePointer(&mapped, const_cast<void*>(p), 0) != hipSuccess || !mapped) {
      (void)hipGetLastError();
      return nullptr;
    }
    dp = mapped;
  } else {
    return nullptr;
  }
  // the allocation holding p (looked up by the GPU address, else by p itself)
  const void* probe = dp;
  if (hipMemGetAddressRange(reinterpret_cast<hipDeviceptr_t*>(&base), &size, const_cast<void*>(dp)) != hipSuccess) {
    (void)hipGetLastError();
    probe = p;
    if (dp == p || hipMemGetAddressRange(reinterpret_cast<hipDeviceptr_t*>(&base), &size, const_cast<void*>(p)) !=
                       hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
  }
  const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(probe);
  if (q < b || q - b > size || static_cast<uint64_t>(bytes) > size - (q - b)) return nullptr;
  return dp;
}
}  // namespace

pkv_status pkv_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v, const int32_t* pairs,
                           int32_t n_pairs, int32_t src_blocks, int32_t dst_blocks, int64_t block_bytes,
                           hipStream_t stream) {
  if (n_pairs < 0 || src_blocks <= 0 || dst_blocks <= 0 || block_bytes <= 0 || block_bytes % 16)
    return PKV_ERR_INVALID_ARG;
  if (n_pairs == 0) return PKV_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return PKV_ERR_INVALID_ARG;
  if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v)) return PKV_ERR_INVALID_ARG;
  if (src_blocks > INT64_MAX / block_bytes || dst_blocks > INT64_MAX / block_bytes) return PKV_ERR_INVALID_ARG;
  const int64_t src_bytes = src_blocks * block_bytes, dst_bytes = dst_blocks * block_bytes;
  const void* sk = gpu_reachable(src_k, src_bytes);
  const void* sv = gpu_reachable(src_v, src_bytes);
  const void* dk = gpu_reachable(dst_k, dst_bytes);
  const void* dv = gpu_reachable(dst_v, dst_bytes);
  const void* pp = gpu_reachable(pairs, static_cast<int64_t>(n_pairs) * 8);
  if (!sk || !sv || !dk || !dv || !pp) return PKV_ERR_INVALID_ARG;
  const int64_t n16 = block_bytes / 16;
  const int64_t splits = ceil_div64(n16, 256 * kSwapUnroll);
  const unsigned z = static_cast<unsigned>(splits < 16 ? splits : 16);
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(n_pairs, 2, z), dim3(256), 0, stream, static_cast<const char*>(sk),
                     static_cast<const char*>(sv), static_cast<char*>(const_cast<void*>(dk)),
                     static_cast<char*>(const_cast<void*>(dv)), static_cast<const int32_t*>(pp), src_blocks,
                     dst_blocks, block_bytes);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes < 0 || bytes % 16 || (bytes > 0 && (!buf || !sink || !aligned16(buf)))) return PKV_ERR_INVALID_ARG;
  if (bytes == 0) return PKV_OK;
  const int64_t n16 = bytes / 16;
  const int64_t chunks = ceil_div64(n16, kProbeChunk16);
  const unsigned grid = static_cast<unsigned>(chunks < 8192 ? chunks : 8192);
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint4*>(buf), n16,
                     sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"

// Runs of causal queries over the paged cache: sequence s owns query rows
// query_start[s] .. query_start[s+1]-1, its last q_s positions, and the query
// at position p attends to the sequence's tokens 0 .. p read through its block
// table.  One call covers a prompt's own attention (q_s = n_s), the remaining
// tokens of a prompt whose leading blocks came from the prefix cache, and the
// verification of speculated tokens before a rollback ([P3] section 5:
// blockwise attention composes with paging, and speculative decoding stages
// and rolls back KV positions; [P4] "Preemption": a whole prompt's KV is
// computed in one parallel pass).
//
// Work unit: one wave per 16 rows of one (sequence, KV head), a row being a
// (query, query head of the group) pair, query-major.  The wave walks the
// sequence's tokens in 16-token chunks up to its last row's position:
//   S = K Q^T on the matrix cores (A = 16 tokens x 32 or 16 dims straight from
//       the 16-byte-piece key tile, B = the rows' queries held in registers),
//   causal mask per row, online softmax per row in the exp2 domain,
//   O += V P on the matrix cores (A = 16 dims x 4 tokens from the transposed
//       value tile, B = the probabilities as QK left them in the lanes;
//       for bf16 they enter as a high and a low bf16 term so the product keeps
//       fp32 accuracy).
// The next chunk's keys and values are loaded before the current chunk is
// used; past the last chunk the loads go through a size-0 buffer resource, so
// every path issues the same loads and the compiler's waits stay exact.

#include <type_traits>

#include "device_common.h"

namespace pkv {
namespace {

typedef const __attribute__((address_space(4))) int32_t* mq_const_i32_ptr;
__device__ __forceinline__ int32_t mq_ld(const int32_t* p, int64_t i) { return ((mq_const_i32_ptr)p)[i]; }

__device__ __forceinline__ uint4 mq_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 mq_load8(__amdgpu_buffer_rsrc_t r, int voff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
  return make_uint2(v[0], v[1]);
}

constexpr int kMqMaxWaves = 4;

struct MultiArgs {
  float* out;
  const void* q;
  const char* k_cache;
  const char* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;
  int num_query_rows;
  int num_q_heads;
  int num_kv_heads;
  int block_size;
  int num_blocks;
  int max_blocks;
  int max_context_len;
  int max_query_len;
  int wg_per_seq;  // workgroups per (sequence, KV head)
  float c;         // scale * log2(e)
};

template <class DT, int D>
struct Chunk {
  static constexpr bool kBF16 = std::is_same<DT, BF16>::value;
  static constexpr int KS = D * DT::kItem / 64;  // QK k-steps: four 16-byte pieces each
  static constexpr int NDT = D / 16;             // 16-dim tiles of the output
  uint4 k[KS];
  typename std::conditional<kBF16, uint2, uint4>::type v[NDT];  // 4 tokens of one dim
};

template <class DT, int D, int G>
__global__ __launch_bounds__(kWave* kMqMaxWaves) void paged_multi_query_kernel(const MultiArgs a) {
  using C = Chunk<DT, D>;
  constexpr bool kBF16 = C::kBF16;
  constexpr int kItem = DT::kItem;
  constexpr int KS = C::KS, NDT = C::NDT;
  constexpr int kTileBytes16 = D * kItem;  // bytes of one token row; a tile is B of them

  const int lane = threadIdx.x % kWave;
  const int m16 = lane % 16, kq = lane / 16;
  const int waves = blockDim.x / kWave;
  const int s = blockIdx.x / a.wg_per_seq;
  const int wg = a.wg_per_seq - 1 - blockIdx.x % a.wg_per_seq;  // rows with the most keys go first
  const int g = blockIdx.y;
  // The wave index is the same in every lane; saying so keeps the values
  // derived from it (row tile, chunk count, buffer resources) scalar.
  const int tile = wg * waves + __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));

  const int q0 = mq_ld(a.query_start, s);
  const int qs = mq_ld(a.query_start, s + 1) - q0;
  if (q0 < 0 || qs <= 0 || static_cast<int64_t>(q0) + qs > a.num_query_rows) return;  // nothing it may write
  const int n = mq_ld(a.context_lens, s);
  const bool bad = n > a.max_context_len || static_cast<int64_t>(n) > static_cast<int64_t>(a.max_blocks) * a.block_size ||
                   qs > n || qs > a.max_query_len;
  const int nrows = min(qs, a.max_query_len) * G;
  const int r0 = tile * 16;
  if (r0 >= nrows) return;  // wave-uniform

  const int rr = r0 + m16;
  const bool vrow = rr < nrows;
  const int qi = vrow ? rr / G : 0;
  const int h = g * G + (vrow ? rr % G : 0);
  const int64_t row_elem = (static_cast<int64_t>(q0 + qi) * a.num_q_heads + h) * D;

  f32x4_t res[NDT];
  if (bad) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) res[dt] = f32x4_t{NAN, NAN, NAN, NAN};
  } else {
    const int B = a.block_size;
    const int pos0 = n - qs;  // position of the run's first query
    const int p_row = pos0 + qi;
    const int p_max = pos0 + min(r0 + 15, nrows - 1) / G;
    const int nc = p_max / 16 + 1;
    const int tile_bytes = B * kTileBytes16;

    uint4 qv[KS];
    const char* qrow = static_cast<const char*>(a.q) + row_elem * kItem;
#pragma unroll
    for (int st = 0; st < KS; ++st)
      qv[st] = vrow ? *reinterpret_cast<const uint4*>(qrow + (st * 4 + kq) * 16) : make_uint4(0, 0, 0, 0);

    bool poison = false;
    const int64_t table_row = static_cast<int64_t>(s) * a.max_blocks;
    auto load = [&](int c, C& ch) __attribute__((always_inline)) {
      const int t0 = 16 * c;
      const bool in = c < nc;
      const int blk = in ? mq_ld(a.block_tables, table_row + t0 / B) : 0;
      const bool ok = blk >= 0 && blk < a.num_blocks;
      poison |= in && !ok;
      const int64_t off = ok ? (static_cast<int64_t>(blk) * a.num_kv_heads + g) * tile_bytes : 0;
      const int bytes = (in && ok) ? tile_bytes : 0;
      const auto rk = make_rsrc(a.k_cache + off, bytes);
      const auto rv = make_rsrc(a.v_cache + off, bytes);
      const int o = t0 % B;
#pragma unroll
      for (int st = 0; st < KS; ++st) ch.k[st] = mq_load16(rk, ((st * 4 + kq) * B + o + m16) * 16);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int voff = ((16 * dt + m16) * B + o + 4 * kq) * kItem;
        if constexpr (kBF16)
          ch.v[dt] = mq_load8(rv, voff);
        else
          ch.v[dt] = mq_load16(rv, voff);
      }
    };

    f32x4_t acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;

    C cur, nxt;
    load(0, cur);
    for (int c = 0; c < nc; ++c) {
      load(c + 1, nxt);
      const int t0 = 16 * c;

      // S[token 4 kq + r][row m16] on the matrix cores.
      f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const uint4 kv = cur.k[st], qq = qv[st];
        if constexpr (kBF16) {
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv), as_bf16x8(qq), sc, 0, 0, 0);
        } else {
          sc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.x), __uint_as_float(qq.x), sc, 0, 0, 0);
          sc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.y), __uint_as_float(qq.y), sc, 0, 0, 0);
          sc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.z), __uint_as_float(qq.z), sc, 0, 0, 0);
          sc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.w), __uint_as_float(qq.w), sc, 0, 0, 0);
        }
      }
      // Scaled logits; a token after the row's position (or past the
      // sequence, which is later still) gets -inf.
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = (t0 + 4 * kq + r <= p_row) ? sc[r] * a.c : -INFINITY;
      if (t0 + 16 > n) {
        // Values past the end may be anything (NaN poison included): zero them.
        const int rel = n - t0 - 4 * kq;  // valid tokens among this lane's four
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          if constexpr (kBF16) {
            cur.v[dt].x &= (rel > 0 ? 0x0000ffffu : 0u) | (rel > 1 ? 0xffff0000u : 0u);
            cur.v[dt].y &= (rel > 2 ? 0x0000ffffu : 0u) | (rel > 3 ? 0xffff0000u : 0u);
          } else {
            if (rel <= 0) cur.v[dt].x = 0u;
            if (rel <= 1) cur.v[dt].y = 0u;
            if (rel <= 2) cur.v[dt].z = 0u;
            if (rel <= 3) cur.v[dt].w = 0u;
          }
        }
      }
      // Online softmax per row (lane column m16; the four lane groups hold its tokens).
      float gm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      gm = max_xor32(max_xor16(gm));
      const float m_new = fmaxf(m_run, gm);  // finite from the first chunk on: token 0 is visible to every row
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
      l_run *= alpha;
      m_run = m_new;
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = __builtin_amdgcn_exp2f(sc[r] - m_run);
        l_run += p[r];
      }

      // O[dim][row] += V[dim][token] P[token][row].
      if constexpr (kBF16) {
        typedef short s4_t __attribute__((ext_vector_type(4)));
        typedef float f2_t __attribute__((ext_vector_type(2)));
        typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
        auto hi_bits = [](float x) __attribute__((always_inline)) { return __float_as_uint(x) & 0xffff0000u; };
        auto pack_hi = [&](float x, float y) __attribute__((always_inline)) { return (hi_bits(x) >> 16) | hi_bits(y); };
        auto pack_lo = [&](float x, float y) __attribute__((always_inline)) {
          const f2_t l = {x - __uint_as_float(hi_bits(x)), y - __uint_as_float(hi_bits(y))};
          return __builtin_bit_cast(uint32_t, __builtin_convertvector(l, b2_t));
        };
        const u32x2_t ph = {pack_hi(p[0], p[1]), pack_hi(p[2], p[3])};
        const u32x2_t pl = {pack_lo(p[0], p[1]), pack_lo(p[2], p[3])};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const u32x2_t av = {cur.v[dt].x, cur.v[dt].y};
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, av),
                                                              __builtin_bit_cast(s4_t, ph), acc[dt], 0, 0, 0);
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, av),
                                                              __builtin_bit_cast(s4_t, pl), acc[dt], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(cur.v[dt].x), p[0], acc[dt], 0, 0, 0);
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(cur.v[dt].y), p[1], acc[dt], 0, 0, 0);
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(cur.v[dt].z), p[2], acc[dt], 0, 0, 0);
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(cur.v[dt].w), p[3], acc[dt], 0, 0, 0);
        }
      }
      cur = nxt;
    }
    const float l_tot = sum_xor32(sum_xor16(l_run));
    const float inv = poison ? NAN : 1.0f / l_tot;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) res[dt] = acc[dt] * inv;
  }
  if (vrow) {
    float* orow = a.out + row_elem;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4_t*>(orow + 16 * dt + 4 * kq) = res[dt];
  }
}

template <class DT, int D>
hipError_t launch_multi_d(const MultiArgs& a, int G, dim3 grid, dim3 block, hipStream_t stream) {
  switch (G) {
    case 1: hipLaunchKernelGGL((paged_multi_query_kernel<DT, D, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((paged_multi_query_kernel<DT, D, 2>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((paged_multi_query_kernel<DT, D, 4>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((paged_multi_query_kernel<DT, D, 8>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class DT>
hipError_t launch_multi(const MultiArgs& a, int D, int G, dim3 grid, dim3 block, hipStream_t stream) {
  if (D == 64) return launch_multi_d<DT, 64>(a, G, grid, block, stream);
  if (D == 128) return launch_multi_d<DT, 128>(a, G, grid, block, stream);
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" pkv_status pkv_paged_attention_multi(float* out, const void* q, const void* k_cache, const void* v_cache,
                                                 const int32_t* block_tables, const int32_t* context_lens,
                                                 const int32_t* query_start, int32_t num_seqs,
                                                 int32_t num_query_rows, int32_t num_q_heads, int32_t num_kv_heads,
                                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                                 int32_t max_blocks, int32_t max_context_len, int32_t max_query_len,
                                                 float scale, int32_t kv_dtype, hipStream_t stream) {
  if (item_size(kv_dtype) == 0) return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_query_rows < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks <= 0 || max_context_len < 0 || max_query_len < 0 || num_kv_heads > 65535)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads) return PKV_ERR_INVALID_ARG;
  const int G = num_q_heads / num_kv_heads;
  if ((G != 1 && G != 2 && G != 4 && G != 8) || (head_dim != 64 && head_dim != 128) ||
      (block_size != 16 && block_size != 32))
    return PKV_ERR_UNSUPPORTED;
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return PKV_ERR_INVALID_ARG;
  // Every tile of one (block, KV head) must be addressable with 32-bit offsets.
  if (static_cast<int64_t>(block_size) * head_dim * item_size(kv_dtype) > INT32_MAX / 2) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0 || max_query_len == 0 || num_query_rows == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID_ARG;

  const int64_t tiles = (static_cast<int64_t>(max_query_len) * G + 15) / 16;  // 16-row wave tiles per (s, g)
  const int waves = static_cast<int>(tiles < kMqMaxWaves ? tiles : kMqMaxWaves);
  const int64_t wg_per_seq = (tiles + waves - 1) / waves;
  if (wg_per_seq * num_seqs > INT32_MAX) return PKV_ERR_INVALID_ARG;
  MultiArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = static_cast<const char*>(k_cache);
  a.v_cache = static_cast<const char*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_query_rows = num_query_rows;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks;
  a.max_context_len = max_context_len;
  a.max_query_len = max_query_len;
  a.wg_per_seq = static_cast<int>(wg_per_seq);
  a.c = scale * 1.4426950408889634f;
  const dim3 grid(static_cast<unsigned>(wg_per_seq * num_seqs), static_cast<unsigned>(num_kv_heads));
  const dim3 block(static_cast<unsigned>(waves * kWave));
  const hipError_t err = kv_dtype == PKV_BF16 ? launch_multi<BF16>(a, head_dim, G, grid, block, stream)
                                              : launch_multi<F32>(a, head_dim, G, grid, block, stream);
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

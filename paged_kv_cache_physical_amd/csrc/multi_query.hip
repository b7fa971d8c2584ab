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
// Work unit: a workgroup of four waves per 64 rows of one (sequence, KV
// head), a row being a (query, query head of the group) pair, query-major;
// each wave owns 16 of the rows.  The workgroup walks the sequence's tokens in
// chunks up to its last row's position.  Each chunk's keys and values
// are loaded once per workgroup (every thread loads 16-byte pieces of the
// tiles into registers, one chunk ahead) and parked in LDS, double-buffered
// with one barrier per chunk (a chunk is 32 tokens, 16 where 32 would not fit
// two buffers in 64 KiB); every wave then reads its operands from LDS:
//   S = K Q^T on the matrix cores (A = 16 tokens x 32 or 16 dims of the key
//       pieces, B = the wave's queries held in registers),
//   causal mask per row, online softmax per row in the exp2 domain,
//   O += V P on the matrix cores (A = 16 dims x 4 tokens of the transposed
//       values, B = the probabilities as QK left them in the lanes; bf16 takes
//       two sub-chunks per 16x16x32 step, and its probabilities enter as a
//       high and a low bf16 term so the product keeps fp32 accuracy).
// Past the last chunk the loads go through a size-0 buffer resource, so every
// path issues the same loads and the compiler's waits stay exact.
//
// Workgroups are renumbered so that each XCD (each with its own L2) takes one
// contiguous run of (sequence, KV head, row block) units.  When the batch has
// few (sequence, KV head) pairs whose rows fit one workgroup (verification of
// a few drafted tokens over long contexts), a caller-provided workspace lets
// each pair's context be cut into splits computed apart; multi_combine_kernel
// then merges the split partials with log-sum-exp weights.

#include <cstdlib>
#include <mutex>
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

constexpr int kMqWaves = 4;  // waves per workgroup
constexpr int kXcds = 8;     // accelerator complex dies of an MI355X

struct MultiArgs {
  float* out;
  const void* q;
  const char* k_cache;
  const char* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;
  const int32_t* seq_order;  // optional: the order in which to start the sequences
  int num_seqs;
  int num_query_rows;
  int num_q_heads;
  int num_kv_heads;
  int block_size;
  int num_blocks;
  int max_blocks;
  int max_context_len;
  int max_query_len;
  int wg_per_seq;  // row blocks per (sequence, KV head)
  int num_pairs;   // (sequence, KV head) pairs
  int pair_slots;  // with several row blocks per pair: ceil(num_pairs / 8), the pairs per XCD
  int nsplit;      // context splits per (sequence, KV head): 1, or several when its rows fit one block
  int split_len;   // tokens per split (a multiple of the chunk), when nsplit > 1
  float* ws_acc;   // split partials: [S][H_kv][nsplit][64 rows][d], un-normalised
  float* ws_m;     // [S][H_kv][nsplit][64 rows], running max (exp2 domain)
  float* ws_l;     // [S][H_kv][nsplit][64 rows], sum of weights
  float c;         // scale * log2(e)
};

constexpr int kMqRows = 16 * kMqWaves;  // rows per workgroup
constexpr int kMqChunk = 32;            // tokens per chunk (every supported shape)

// T: 16-row tiles per wave (1, or 2 for prompts: two independent chains per
// wave, each K/V operand read from LDS once for both).  One tile: three
// workgroups per CU, and at bf16/d = 128 the compiler then keeps the
// accumulators in VGPRs (146, no AGPR copies, no scratch).  Two tiles, and
// fp32 at d = 128 (32-token chunks of fp32 keys and values fill 64 KiB of LDS
// per workgroup, so no third fits the CU's 160 KiB), two per CU.
template <class DT, int D>
constexpr int mq_min_blocks(int T) { return (T == 1 && !(std::is_same<DT, F32>::value && D == 128)) ? 3 : 2; }
template <class DT, int D, int G, int T>
__global__ __launch_bounds__(kWave* kMqWaves, (mq_min_blocks<DT, D>(T))) void paged_multi_query_kernel(const MultiArgs a) {
  constexpr bool kBF16 = std::is_same<DT, BF16>::value;
  constexpr int kItem = DT::kItem;
  constexpr int KS = D * kItem / 64;  // QK k-steps: four 16-byte pieces each
  constexpr int NDT = D / 16;         // 16-dim tiles of the output
  constexpr int ITEMS = D * kItem;    // 16-byte pieces of 16 tokens' keys, and of their values
  constexpr int kSubBytes = 16 * ITEMS;
  // 16-token sub-chunks per chunk: 2, or 1 where two buffers of keys and values
  // would not fit in 64 KiB.  32-token chunks (32 KiB at bf16, d = 128) leave
  // room for three workgroups per CU; 64-token chunks measured slower.
  constexpr int NSUB = (65536 / (4 * kSubBytes)) < 2 ? (65536 / (4 * kSubBytes)) : 2;
  constexpr int CT = 16 * NSUB;  // tokens per chunk
  constexpr int kThreads = kWave * kMqWaves;
  constexpr int NIT = NSUB * ITEMS / kThreads;  // pieces per thread per cache per chunk
  static_assert(NSUB >= 1 && (NSUB * ITEMS) % kThreads == 0 && ITEMS % kWave == 0, "staging shape");
  // LDS per buffer and sub-chunk: keys [piece][16 tokens][16 B], then values
  // [dim][16 tokens] with the row's four 4-token slots XOR-swizzled by the dim
  // (slot t at t ^ ((dim >> 2) & 3) for bf16, t ^ ((dim >> 1) & 3) for fp32),
  // so that the sixteen rows a value read touches fall in distinct banks.
  __shared__ __attribute__((aligned(16))) char lds[2][NSUB][2 * kSubBytes];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int m16 = lane % 16, kq = lane / 16;
  // The wave index is the same in every lane; saying so keeps what derives from it scalar.
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  // Workgroup ids are dealt to the 8 XCDs in turn (id mod 8), each XCD with its
  // own L2.  With several row blocks per pair, renumber them so that each XCD
  // takes one contiguous run of units (below): the workgroups that read the
  // same keys and values then share an L2.
  // Only row blocks of one pair share keys and values; with one workgroup per
  // pair (verification, or context splits, which read disjoint ranges) the
  // hardware's round-robin is kept, so that a longest-first order is spread
  // over the XCDs instead of piling the longest pairs onto one.
  const int nwg = gridDim.x, xcd = blockIdx.x % kXcds, k = blockIdx.x / kXcds;
  const int per = nwg / kXcds, extra = nwg % kXcds;
  const int unit = a.wg_per_seq == 1 ? static_cast<int>(blockIdx.x)
                 : xcd < extra ? xcd * (per + 1) + k : extra * (per + 1) + (xcd - extra) * per + k;
  const int per_sg = a.wg_per_seq * a.nsplit;
  int sg = unit / per_sg;
  if (a.wg_per_seq > 1) {
    // XCD x holds pair slots [x m, (x + 1) m) (m = pair_slots); slot j is pair
    // 8 (j mod m) + j div m, so XCD x serves pairs x, x + 8, x + 16, ...: a pair's
    // row blocks share an L2 while the pairs, in their given order, are dealt
    // across the XCDs.  Slots past the last pair have nothing to do.
    sg = kXcds * (sg % a.pair_slots) + sg / a.pair_slots;
    if (sg >= a.num_pairs) return;
  }
  const int wg = a.wg_per_seq - 1 - (unit % per_sg) / a.nsplit;  // rows with the most keys go first
  const int split = unit % a.nsplit;
  const int g = sg % a.num_kv_heads;
  int s = sg / a.num_kv_heads;
  if (a.seq_order) {
    s = mq_ld(a.seq_order, s);
    if (s < 0 || s >= a.num_seqs) return;  // not a sequence: nothing to do
  }
  static_assert(CT == kMqChunk, "split lengths are counted in chunks");

  const int q0 = mq_ld(a.query_start, s);
  const int qs = mq_ld(a.query_start, s + 1) - q0;
  if (q0 < 0 || qs <= 0 || static_cast<int64_t>(q0) + qs > a.num_query_rows) return;  // nothing it may write
  const int n = mq_ld(a.context_lens, s);
  const bool bad = n > a.max_context_len || static_cast<int64_t>(n) > static_cast<int64_t>(a.max_blocks) * a.block_size ||
                   qs > n || qs > a.max_query_len;
  const int nrows = min(qs, a.max_query_len) * G;
  const int R0 = wg * 16 * kMqWaves * T;
  if (R0 >= nrows) return;  // the whole workgroup: no barrier is left waiting

  // Tile t of wave w holds rows R0 + 16 (w + kMqWaves t) + m16, so every wave has
  // rows from each part of the block.
  int r0[T], rr[T], qi[T];
  bool active[T], vrow[T];
  int64_t row_elem[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    r0[t] = R0 + 16 * (wave + kMqWaves * t);
    active[t] = r0[t] < nrows;  // wave-uniform
    rr[t] = r0[t] + m16;
    vrow[t] = rr[t] < nrows;
    qi[t] = vrow[t] ? rr[t] / G : 0;
    const int h = g * G + (vrow[t] ? rr[t] % G : 0);
    row_elem[t] = (static_cast<int64_t>(q0 + qi[t]) * a.num_q_heads + h) * D;
  }

  if (bad) {  // the same for every wave of the workgroup (the split combine skips such runs)
#pragma unroll
    for (int t = 0; t < T; ++t)
      if (vrow[t] && split == 0) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          *reinterpret_cast<f32x4_t*>(a.out + row_elem[t] + 16 * dt + 4 * kq) = f32x4_t{NAN, NAN, NAN, NAN};
      }
    return;
  }

  const int B = a.block_size;
  const int pos0 = n - qs;  // position of the run's first query
  int p_row[T];
  int p_wave = -1;  // the wave's last position (-1: no rows)
#pragma unroll
  for (int t = 0; t < T; ++t) {
    p_row[t] = pos0 + qi[t];
    if (active[t]) p_wave = max(p_wave, pos0 + min(r0[t] + 15, nrows - 1) / G);
  }
  const int p_last = pos0 + min(R0 + 16 * kMqWaves * T - 1, nrows - 1) / G;  // the workgroup's last position
  // Chunks [c_begin, nc): this split's tokens up to the last position.
  const int c_begin = a.nsplit > 1 ? split * (a.split_len / CT) : 0;
  const int nc = a.nsplit > 1 ? min((split + 1) * (a.split_len / CT), p_last / CT + 1) : p_last / CT + 1;
  const int tile_bytes = B * D * kItem;
  // Split partial row, indexed by the pair itself (not by its place in the order);
  // context splits are planned only for one tile per wave, rows < kMqRows.
  const int64_t part = ((static_cast<int64_t>(s) * a.num_kv_heads + g) * a.nsplit + split) * kMqRows + (rr[0] - R0);
  if (c_begin >= nc) {  // a split past every row's position: an empty partial
    if (vrow[0]) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4_t*>(a.ws_acc + part * D + 16 * dt + 4 * kq) = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      if (kq == 0) {
        a.ws_m[part] = -INFINITY;
        a.ws_l[part] = 0.0f;
      }
    }
    return;  // the same for the whole workgroup
  }

  uint4 qv[T][KS];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const char* qrow = static_cast<const char*>(a.q) + row_elem[t] * kItem;
#pragma unroll
    for (int st = 0; st < KS; ++st)
      qv[t][st] = vrow[t] ? *reinterpret_cast<const uint4*>(qrow + (st * 4 + kq) * 16) : make_uint4(0, 0, 0, 0);
  }

  // Staging: thread piece j of a chunk is i = tid + kThreads j, in sub-chunk
  // i / ITEMS (the same for a whole wave); within it, key piece ii is (key
  // piece ii / 16, token ii % 16) and value piece ii is (dim ii / kItem,
  // tokens (ii % kItem) * 16 / kItem + 0 ..).
  // A bad block id is seen only by the threads that stage its tile; the flag
  // is combined over the workgroup after the chunk loop, since every wave's
  // rows read the whole chunk from LDS.
  bool poison = false;
  __shared__ int poison_any;
  if (tid == 0) poison_any = 0;  // ordered before any write of 1 by the barriers below
  const int64_t table_row = static_cast<int64_t>(s) * a.max_blocks;
  uint4 kr[NIT], vr[NIT];
  auto stage = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int sub = (kWave * wave + kThreads * j) / ITEMS;  // wave-uniform
      const int ii = tid + kThreads * j - sub * ITEMS;
      const int t0 = CT * c + 16 * sub;
      const bool in = c < nc && t0 < n;
      const int blk = in ? mq_ld(a.block_tables, table_row + t0 / B) : 0;
      const bool ok = blk >= 0 && blk < a.num_blocks;
      poison |= in && !ok;
      const int64_t off = ok ? (static_cast<int64_t>(blk) * a.num_kv_heads + g) * tile_bytes : 0;
      const int bytes = (in && ok) ? tile_bytes : 0;
      const int o = t0 % B;
      kr[j] = mq_load16(make_rsrc(a.k_cache + off, bytes), ((ii >> 4) * B + o + (ii & 15)) * 16);
      vr[j] = mq_load16(make_rsrc(a.v_cache + off, bytes), ((ii / kItem) * B + o + (ii % kItem) * (16 / kItem)) * kItem);
    }
  };
  auto put = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int sub = (kWave * wave + kThreads * j) / ITEMS;
      const int ii = tid + kThreads * j - sub * ITEMS;
      *reinterpret_cast<uint4*>(&lds[buf][sub][16 * ii]) = kr[j];
      const int dim = ii / kItem, part = ii % kItem;
      if constexpr (kBF16) {
        // Piece = 4-token slots 2 part and 2 part + 1 of the row; slot t sits at t ^ sw.
        const int sw = (dim >> 2) & 3;
        const uint4 v = (sw & 1) ? make_uint4(vr[j].z, vr[j].w, vr[j].x, vr[j].y) : vr[j];
        *reinterpret_cast<uint4*>(&lds[buf][sub][kSubBytes + 32 * dim + 16 * (part ^ (sw >> 1))]) = v;
      } else {
        // Piece = 4-token slot `part` of the row; slot t sits at t ^ sw.
        const int sw = (dim >> 1) & 3;
        *reinterpret_cast<uint4*>(&lds[buf][sub][kSubBytes + 64 * dim + 16 * (part ^ sw)]) = vr[j];
      }
    }
  };

  f32x4_t acc[T][NDT];
  float m_run[T], l_run[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[t][dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m_run[t] = -INFINITY;
    l_run[t] = 0.0f;
  }

  stage(c_begin);
  put(c_begin & 1);
  stage(c_begin + 1);
  __syncthreads();
  for (int c = c_begin; c < nc; ++c) {
    if (CT * c <= p_wave) {  // some row of the wave sees this chunk (wave-uniform)
      // S[token 16 sub + 4 kq + r][row m16] on the matrix cores: NSUB tiles per
      // row tile, each summed in two halves (even and odd k-steps) so that more
      // independent chains overlap in the matrix pipeline; a key operand read
      // from LDS serves every row tile.
      f32x4_t sc[T][NSUB], sc2[T][NSUB];
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        const char* kl = lds[c & 1][u];
#pragma unroll
        for (int t = 0; t < T; ++t) {
          sc[t][u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
          sc2[t][u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          const uint4 kv = *reinterpret_cast<const uint4*>(kl + ((st * 4 + kq) * 16 + m16) * 16);
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const uint4 qq = qv[t][st];
            f32x4_t& acc_s = (st & 1) ? sc2[t][u] : sc[t][u];
            if constexpr (kBF16) {
              acc_s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv), as_bf16x8(qq), acc_s, 0, 0, 0);
            } else {
              acc_s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.x), __uint_as_float(qq.x), acc_s, 0, 0, 0);
              acc_s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.y), __uint_as_float(qq.y), acc_s, 0, 0, 0);
              acc_s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.z), __uint_as_float(qq.z), acc_s, 0, 0, 0);
              acc_s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.w), __uint_as_float(qq.w), acc_s, 0, 0, 0);
            }
          }
        }
#pragma unroll
        for (int t = 0; t < T; ++t) sc[t][u] += sc2[t][u];
      }
      float m_ref[T];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        // Scaled logits; a token after the row's position (or past the
        // sequence, which is later still) gets -inf.
        float gm = -INFINITY;
#pragma unroll
        for (int u = 0; u < NSUB; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sc[t][u][r] = (CT * c + 16 * u + 4 * kq + r <= p_row[t]) ? sc[t][u][r] * a.c : -INFINITY;
            gm = fmaxf(gm, sc[t][u][r]);
          }
        // Online softmax per row (lane column m16; the four lane groups hold its tokens).
        gm = max_xor32(max_xor16(gm));
        const float m_new = fmaxf(m_run[t], gm);
        // -inf only for a row that has seen no token yet (in a split that starts
        // after its position, or a tile past the run): then alpha and its weights
        // are 0, never inf - inf.
        m_ref[t] = m_new == -INFINITY ? 0.0f : m_new;
        if (__ballot(m_new > m_run[t])) {  // some row's maximum grew: rescale (wave-uniform branch)
          const float alpha = __builtin_amdgcn_exp2f(m_run[t] - m_ref[t]);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) acc[t][dt] *= alpha;
          l_run[t] *= alpha;
          m_run[t] = m_new;
        }
      }
      // The lane's value columns of sub-chunk u: dims 16 dt + m16, tokens 4 kq .. 4 kq + 3
      // (values past the end of the sequence may be anything, NaN poison included: zeroed).
      auto values = [&](int u, auto (&vv)[NDT]) __attribute__((always_inline)) {
        const int t0 = CT * c + 16 * u;
        const char* vl = lds[c & 1][u] + kSubBytes;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int dim = 16 * dt + m16;
          if constexpr (kBF16)
            vv[dt] = *reinterpret_cast<const uint2*>(vl + 32 * dim + 8 * (kq ^ ((dim >> 2) & 3)));
          else
            vv[dt] = *reinterpret_cast<const uint4*>(vl + 64 * dim + 16 * (kq ^ ((dim >> 1) & 3)));
        }
        if (t0 + 16 > n) {
          const int rel = n - t0 - 4 * kq;  // valid tokens among this lane's four
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            if constexpr (kBF16) {
              vv[dt].x &= (rel > 0 ? 0x0000ffffu : 0u) | (rel > 1 ? 0xffff0000u : 0u);
              vv[dt].y &= (rel > 2 ? 0x0000ffffu : 0u) | (rel > 3 ? 0xffff0000u : 0u);
            } else {
              if (rel <= 0) vv[dt].x = 0u;
              if (rel <= 1) vv[dt].y = 0u;
              if (rel <= 2) vv[dt].z = 0u;
              if (rel <= 3) vv[dt].w = 0u;
            }
          }
        }
      };
      float p[T][NSUB][4];
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int u = 0; u < NSUB; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[t][u][r] = __builtin_amdgcn_exp2f(sc[t][u][r] - m_ref[t]);
            l_run[t] += p[t][u][r];
          }
      // O[dim][row] += V[dim][token] P[token][row].
      if constexpr (kBF16) {
        // Sub-chunks in pairs on 16x16x32 steps: lane (kq, m16) supplies k-slots
        // 0-3 = tokens 4 kq + r of the first and 4-7 = the same of the second,
        // for P (its QK registers) and V alike.  P enters as a high and a low
        // bf16 term.
        static_assert(NSUB % 2 == 0, "bf16 chunks hold pairs of sub-chunks");
        typedef float f2_t __attribute__((ext_vector_type(2)));
        typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
        auto hi_bits = [](float x) __attribute__((always_inline)) { return __float_as_uint(x) & 0xffff0000u; };
        auto pack_hi = [&](float x, float y) __attribute__((always_inline)) { return (hi_bits(x) >> 16) | hi_bits(y); };
        auto pack_lo = [&](float x, float y) __attribute__((always_inline)) {
          const f2_t l = {x - __uint_as_float(hi_bits(x)), y - __uint_as_float(hi_bits(y))};
          return __builtin_bit_cast(uint32_t, __builtin_convertvector(l, b2_t));
        };
#pragma unroll
        for (int u = 0; u < NSUB; u += 2) {
          if (CT * c + 16 * u > p_wave) break;  // no row of the wave sees these tokens (wave-uniform)
          uint2 va[NDT], vb[NDT];
          values(u, va);
          values(u + 1, vb);
          u32x4_t ph[T], pl[T];
#pragma unroll
          for (int t = 0; t < T; ++t) {
            ph[t] = u32x4_t{pack_hi(p[t][u][0], p[t][u][1]), pack_hi(p[t][u][2], p[t][u][3]),
                            pack_hi(p[t][u + 1][0], p[t][u + 1][1]), pack_hi(p[t][u + 1][2], p[t][u + 1][3])};
            pl[t] = u32x4_t{pack_lo(p[t][u][0], p[t][u][1]), pack_lo(p[t][u][2], p[t][u][3]),
                            pack_lo(p[t][u + 1][0], p[t][u + 1][1]), pack_lo(p[t][u + 1][2], p[t][u + 1][3])};
          }
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const u32x4_t av = {va[dt].x, va[dt].y, vb[dt].x, vb[dt].y};
#pragma unroll
            for (int t = 0; t < T; ++t) {
              acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                                   __builtin_bit_cast(bf16x8_t, ph[t]), acc[t][dt], 0, 0, 0);
              acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                                   __builtin_bit_cast(bf16x8_t, pl[t]), acc[t][dt], 0, 0, 0);
            }
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < NSUB; ++u) {
          if (CT * c + 16 * u > p_wave) break;  // no row of the wave sees these tokens (wave-uniform)
          uint4 vv[NDT];
          values(u, vv);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int t = 0; t < T; ++t) {
              acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vv[dt].x), p[t][u][0], acc[t][dt], 0, 0, 0);
              acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vv[dt].y), p[t][u][1], acc[t][dt], 0, 0, 0);
              acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vv[dt].z), p[t][u][2], acc[t][dt], 0, 0, 0);
              acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vv[dt].w), p[t][u][3], acc[t][dt], 0, 0, 0);
            }
        }
      }
    }
    // Chunk c + 1 into the other buffer (its last readers passed the previous
    // barrier), then the loads of chunk c + 2.
    put((c + 1) & 1);
    stage(c + 2);
    __syncthreads();
  }
  if (__ballot(poison) != 0 && lane == 0) poison_any = 1;
  __syncthreads();
  poison = poison_any != 0;
  float l_tot[T];
#pragma unroll
  for (int t = 0; t < T; ++t) l_tot[t] = sum_xor32(sum_xor16(l_run[t]));  // every lane takes part in the swaps
  if (a.nsplit > 1) {
    // Split partial: un-normalised accumulator, max and sum (NaN if a block id was bad).
    const float f = poison ? NAN : 1.0f;
    if (vrow[0]) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4_t*>(a.ws_acc + part * D + 16 * dt + 4 * kq) = acc[0][dt] * f;
      if (kq == 0) {
        a.ws_m[part] = m_run[0];
        a.ws_l[part] = l_tot[0] * f;
      }
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const float inv = poison ? NAN : 1.0f / l_tot[t];
    if (vrow[t]) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4_t*>(a.out + row_elem[t] + 16 * dt + 4 * kq) = acc[t][dt] * inv;
    }
  }
}

// Log-sum-exp combination of the split partials of one row of one (sequence,
// KV head): out = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k with
// M = max_k m_k; a split that saw none of the row's tokens has m = -inf and
// weighs nothing.  One workgroup per (pair, row of the longest run): wave 0 turns the
// splits' maxima and sums into weights (one split per lane), then every
// thread sums a share of the splits for four dims and LDS adds the shares.
// Runs the attention kernel did not write, or wrote as NaN, are skipped.
constexpr int kMqMaxSplits = 64;  // one split per lane of the weighting wave
template <int D, int G>
__global__ __launch_bounds__(256) void multi_combine_kernel(const MultiArgs a) {
  constexpr int NQ = D / 4;       // four-dim quads of a row
  constexpr int KG = 256 / NQ;    // split groups: thread (kg, quad)
  __shared__ float wsh[kMqMaxSplits];
  __shared__ float inv_den;
  __shared__ f32x4_t red[KG][NQ];
  const int row_slots = a.max_query_len * G;  // rows a pair can have (at most kMqRows when split)
  const int sg = blockIdx.x / row_slots, rr = blockIdx.x % row_slots;
  const int s = sg / a.num_kv_heads, g = sg % a.num_kv_heads;
  const int q0 = mq_ld(a.query_start, s);
  const int qs = mq_ld(a.query_start, s + 1) - q0;
  if (q0 < 0 || qs <= 0 || static_cast<int64_t>(q0) + qs > a.num_query_rows) return;
  const int n = mq_ld(a.context_lens, s);
  if (n > a.max_context_len || static_cast<int64_t>(n) > static_cast<int64_t>(a.max_blocks) * a.block_size ||
      qs > n || qs > a.max_query_len || rr >= qs * G)  // the same for the whole workgroup
    return;
  const int64_t base = static_cast<int64_t>(sg) * a.nsplit * kMqRows + rr;  // split k's row: base + k * kMqRows
  const int tid = threadIdx.x;
  if (tid < kWave) {
    const bool in = tid < a.nsplit;
    const float m = in ? a.ws_m[base + tid * kMqRows] : -INFINITY;
    const float l = in ? a.ws_l[base + tid * kMqRows] : 0.0f;
    float M = m;
    for (int o = kWave / 2; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float w = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    float den = w * l;
    for (int o = kWave / 2; o > 0; o >>= 1) den += __shfl_xor(den, o);
    if (in) wsh[tid] = w;
    if (tid == 0) inv_den = 1.0f / den;
  }
  __syncthreads();
  const int kg = tid / NQ, quad = tid % NQ;
  f32x4_t sum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
  for (int k = kg; k < a.nsplit; k += KG)
    sum += wsh[k] * *reinterpret_cast<const f32x4_t*>(a.ws_acc + (base + k * kMqRows) * D + 4 * quad);
  red[kg][quad] = sum;
  __syncthreads();
  if (kg == 0) {
#pragma unroll
    for (int j = 1; j < KG; ++j) sum += red[j][quad];
    const int h = g * G + rr % G;
    float* o = a.out + (static_cast<int64_t>(q0 + rr / G) * a.num_q_heads + h) * D + 4 * quad;
    *reinterpret_cast<f32x4_t*>(o) = sum * inv_den;
  }
}

template <int D>
hipError_t launch_combine(const MultiArgs& a, int G, int units, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(units) * static_cast<unsigned>(a.max_query_len * G)), block(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((multi_combine_kernel<D, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((multi_combine_kernel<D, 2>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((multi_combine_kernel<D, 4>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((multi_combine_kernel<D, 8>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Split plan: a (sequence, KV head) whose rows fit one workgroup is cut into
// enough context splits for about kMqSplitTarget workgroups in all, each at
// least kMqMinSplit tokens and at most kMqMaxSplits of them, so that few long
// sequences still fill the chip.
constexpr int kMqSplitTarget = 2048;
constexpr int kMqMinSplit = 256;
struct MultiPlan {
  int nsplit = 1;
  int split_len = 0;
  size_t bytes = 0;
};

// Compute units of the current device, cached per device (256 if the query fails).
int device_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int cus = 0;
    cache[dev] = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0 ? cus : 256;
  }
  return cache[dev];
}

MultiPlan multi_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t G, int32_t head_dim, int32_t max_context_len,
                     int32_t max_query_len) {
  MultiPlan p;
  const int64_t units = static_cast<int64_t>(num_seqs) * num_kv_heads;
  if (units <= 0 || static_cast<int64_t>(max_query_len) * G > kMqRows || max_context_len < 2 * kMqMinSplit) return p;
  int64_t ns = (kMqSplitTarget + units - 1) / units;
  ns = ns < max_context_len / kMqMinSplit ? ns : max_context_len / kMqMinSplit;
  ns = ns < kMqMaxSplits ? ns : kMqMaxSplits;
  if (ns <= 1) return p;
  const int64_t len = ((max_context_len + ns - 1) / ns + kMqChunk - 1) / kMqChunk * kMqChunk;
  p.nsplit = static_cast<int>((max_context_len + len - 1) / len);
  if (p.nsplit <= 1) {
    p.nsplit = 1;
    return p;
  }
  p.split_len = static_cast<int>(len);
  const int64_t rows = units * p.nsplit * kMqRows;
  p.bytes = static_cast<size_t>(rows) * (head_dim + 2) * sizeof(float);
  return p;
}

template <class DT, int D, int T>
hipError_t launch_multi_t(const MultiArgs& a, int G, dim3 grid, dim3 block, hipStream_t stream) {
  switch (G) {
    case 1: hipLaunchKernelGGL((paged_multi_query_kernel<DT, D, 1, T>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((paged_multi_query_kernel<DT, D, 2, T>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((paged_multi_query_kernel<DT, D, 4, T>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((paged_multi_query_kernel<DT, D, 8, T>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class DT, int D>
hipError_t launch_multi_d(const MultiArgs& a, int G, int T, dim3 grid, dim3 block, hipStream_t stream) {
  return T == 2 ? launch_multi_t<DT, D, 2>(a, G, grid, block, stream) : launch_multi_t<DT, D, 1>(a, G, grid, block, stream);
}

template <class DT>
hipError_t launch_multi(const MultiArgs& a, int D, int G, int T, dim3 grid, dim3 block, hipStream_t stream) {
  if (D == 64) return launch_multi_d<DT, 64>(a, G, T, grid, block, stream);
  if (D == 128) return launch_multi_d<DT, 128>(a, G, T, grid, block, stream);
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" pkv_status pkv_paged_attention_multi(float* out, const void* q, const void* k_cache, const void* v_cache,
                                                 const int32_t* block_tables, const int32_t* context_lens,
                                                 const int32_t* query_start, const int32_t* seq_order,
                                                 int32_t num_seqs,
                                                 int32_t num_query_rows, int32_t num_q_heads, int32_t num_kv_heads,
                                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                                 int32_t max_blocks, int32_t max_context_len, int32_t max_query_len,
                                                 float scale, void* workspace, size_t workspace_bytes,
                                                 int32_t kv_dtype, hipStream_t stream) {
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

  // Two row tiles per wave when a pair has more rows than one workgroup of
  // one-tile waves holds, and the batch's rows (num_query_rows * G in all, the
  // host's only measure of the work) make at least one full round of
  // two-tile workgroups (two fit a CU); otherwise one tile per wave gives
  // twice the workgroups to spread a few long prompts over.
  // PKV_MULTI_TILES=1 or 2 (read at each call) forces the choice; both kernels
  // give the same rows.
  int T = 1;
  if (static_cast<int64_t>(max_query_len) * G > kMqRows) {
    const char* force = std::getenv("PKV_MULTI_TILES");
    if (force && (force[0] == '1' || force[0] == '2') && force[1] == 0) {
      T = force[0] - '0';
    } else {
      const int64_t blocks2 = (static_cast<int64_t>(num_query_rows) * G + 2 * kMqRows - 1) / (2 * kMqRows);
      if (blocks2 >= 2 * static_cast<int64_t>(device_cus())) T = 2;
    }
  }
  const int64_t rows_per_wg = static_cast<int64_t>(kMqRows) * T;
  const int64_t wg_per_seq = (static_cast<int64_t>(max_query_len) * G + rows_per_wg - 1) / rows_per_wg;
  // Split the context only when a workspace is given and the plan asks for it.
  MultiPlan plan = multi_plan(num_seqs, num_kv_heads, G, head_dim, max_context_len, max_query_len);
  if (!workspace) plan = MultiPlan{};
  if (plan.nsplit > 1 && (workspace_bytes < plan.bytes || !aligned16(workspace))) return PKV_ERR_WORKSPACE;
  const int64_t pairs = static_cast<int64_t>(num_seqs) * num_kv_heads;
  const int64_t pair_slots = (pairs + kXcds - 1) / kXcds;
  const int64_t grid_pairs = wg_per_seq > 1 ? kXcds * pair_slots : pairs;  // whole XCD runs when renumbering
  if (wg_per_seq * plan.nsplit * grid_pairs > INT32_MAX) return PKV_ERR_INVALID_ARG;
  MultiArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = static_cast<const char*>(k_cache);
  a.v_cache = static_cast<const char*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.seq_order = seq_order;
  a.num_seqs = num_seqs;
  a.num_query_rows = num_query_rows;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks;
  a.max_context_len = max_context_len;
  a.max_query_len = max_query_len;
  a.wg_per_seq = static_cast<int>(wg_per_seq);
  a.num_pairs = static_cast<int>(pairs);
  a.pair_slots = static_cast<int>(pair_slots);
  a.nsplit = plan.nsplit;
  a.split_len = plan.split_len;
  if (plan.nsplit > 1) {
    const int64_t rows = static_cast<int64_t>(num_seqs) * num_kv_heads * plan.nsplit * kMqRows;
    a.ws_acc = static_cast<float*>(workspace);
    a.ws_m = a.ws_acc + rows * head_dim;
    a.ws_l = a.ws_m + rows;
  }
  a.c = scale * 1.4426950408889634f;
  const dim3 grid(static_cast<unsigned>(wg_per_seq * plan.nsplit * grid_pairs));
  const dim3 block(static_cast<unsigned>(kMqWaves * kWave));
  hipError_t err = kv_dtype == PKV_BF16 ? launch_multi<BF16>(a, head_dim, G, T, grid, block, stream)
                                        : launch_multi<F32>(a, head_dim, G, T, grid, block, stream);
  if (err == hipSuccess && plan.nsplit > 1) {
    const int units = num_seqs * num_kv_heads;
    err = head_dim == 64 ? launch_combine<64>(a, G, units, stream) : launch_combine<128>(a, G, units, stream);
  }
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" size_t pkv_attention_multi_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                      int32_t head_dim, int32_t max_context_len, int32_t max_query_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || head_dim <= 0 ||
      max_context_len < 0 || max_query_len < 0)
    return 0;
  return multi_plan(num_seqs, num_kv_heads, num_q_heads / num_kv_heads, head_dim, max_context_len, max_query_len).bytes;
}

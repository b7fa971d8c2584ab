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
#include <cstring>
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

// 16-byte load of each lane straight into LDS: lane L's bytes land at
// dst + 16 L (dst: the wave's LDS block, the same for every lane).
__device__ __forceinline__ void load_to_lds16(__amdgpu_buffer_rsrc_t r, char* dst, int voff) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, 0, 0, 0);
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
  int skip_upto;   // runs of at most this many queries belong to another launch (0: none)
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
  // Chunks move straight from HBM into LDS: a wave's 16-byte load lands lane L's
  // bytes at its 1 KiB block's base + 16 L, so the layout is set by which source
  // unit each lane fetches.  Per buffer, NBLK blocks of keys then NBLK of values:
  //   keys: sub-chunk u at u kSubBytes, [piece][16 positions][16 B]; bf16 token
  //     t of the sub-chunk sits at position t ^ 4 (t >> 3) ^ 4 u, so that the
  //     sixteen rows of a score tile (below) fall in distinct banks.
  //   values, bf16: sub-chunk u at u kSubBytes, 1 KiB per 32 dims, the dim's
  //     two 8-token units at 2 (dim & 31) + (half ^ vflip(dim)); fp32: sub-chunk
  //     u at u kSubBytes, [dim][4-token slot ^ vswz(dim)][16 B].
  // bf16 score tiles take the chunk's tokens permuted: row r of tile u is token
  // 8 (r / 4) + 4 u + r % 4, so that lane (kq, m16) ends up holding the scores
  // of tokens 8 kq .. 8 kq + 7, the k-slots it feeds a 16x16x32 value step, and
  // its value operand is one 8-token unit.
  constexpr int NBLK = NSUB * kSubBytes / 1024;  // 1 KiB blocks of one cache per chunk
  constexpr int NB = NBLK / kMqWaves;           // blocks per wave per cache per chunk
  constexpr int BPS = kSubBytes / 1024;         // blocks per sub-chunk
  static_assert(NSUB >= 1 && NBLK % kMqWaves == 0 && kSubBytes % 1024 == 0, "staging shape");
  // Three buffers where they fit in 48 KiB (two chunks of loads in flight while
  // a third is computed), else two.
  // The buffers are separate LDS objects, indexed by compile-time constants
  // (the chunk loop below is unrolled over them), so that the compiler can
  // tell a read of one buffer from a load still landing in another and waits
  // only where a read needs its own wave's load.
  constexpr int NBUF = 3 * 2 * NSUB * kSubBytes <= 49152 ? 3 : 2;
  constexpr int kBufBytes = 2 * NSUB * kSubBytes;
  __shared__ __attribute__((aligned(1024))) char lds0[kBufBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[kBufBytes];
  __shared__ __attribute__((aligned(1024))) char lds2[NBUF == 3 ? kBufBytes : 16];
  auto lds_buf = [&](auto b) __attribute__((always_inline)) -> char* {
    constexpr int k = decltype(b)::value % NBUF;
    return k == 0 ? lds0 : k == 1 ? lds1 : lds2;
  };
  auto vswz = [](int dim) __attribute__((always_inline)) { return (dim >> 1) & 3; };
  auto vflip = [](int dim) __attribute__((always_inline)) { return ((dim >> 2) ^ (dim >> 3)) & 1; };
  auto kpos = [](int t, int u) __attribute__((always_inline)) { return kBF16 ? t ^ (4 * (t >> 3)) ^ (4 * u) : t; };

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
  if (q0 < 0 || qs <= a.skip_upto || static_cast<int64_t>(q0) + qs > a.num_query_rows) return;  // nothing to write
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

  // The softmax runs on logits c s (s = q . k) in the exp2 domain as
  // p = exp2(fma(s, c', -c' m)) with c' = |c| and m a per-row reference: with a
  // negative scale the queries enter with their sign bits flipped (exact), so
  // that c s = c' s' and the row maximum of the raw scores s' is the maximum
  // of the logits.  A zero scale is taken as the smallest normal float, which
  // leaves every exp2 argument within 2^-25 of 0 (weights exactly 1) and keeps
  // -inf * c' = -inf for masked tokens.
  const uint32_t qflip = a.c < 0.0f ? (kBF16 ? 0x80008000u : 0x80000000u) : 0u;
  const float cs = fmaxf(fabsf(a.c), FLT_MIN);
  uint4 qv[T][KS];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const char* qrow = static_cast<const char*>(a.q) + row_elem[t] * kItem;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const uint4 v = vrow[t] ? *reinterpret_cast<const uint4*>(qrow + (st * 4 + kq) * 16) : make_uint4(0, 0, 0, 0);
      qv[t][st] = make_uint4(v.x ^ qflip, v.y ^ qflip, v.z ^ qflip, v.w ^ qflip);
    }
  }

  // Wave w moves blocks w + 4 j (j < NB) of each cache per chunk.  A bad block
  // id is seen only by the waves that load its tiles; the flag is combined
  // over the workgroup after the chunk loop, since every wave's rows read the
  // whole chunk.
  bool poison = false;
  __shared__ int poison_any;
  if (tid == 0) poison_any = 0;  // ordered before any write of 1 by the barriers below
  const int64_t table_row = static_cast<int64_t>(s) * a.max_blocks;
  // Block sizes are 16 or 32 (checked by the host): shifts, not divisions.
  const int lgB = B == 16 ? 4 : 5;
  const int last_blk = (n - 1) >> lgB;  // n >= qs >= 1 here
  // Address parts fixed for the whole loop: a block's tile of this KV head
  // starts at cache + (head 0 of the KV head's tiles) + id * kstride
  // (kstride = H_kv tiles < 2^32 bytes, as H_kv <= 65535 and a tile <= 16 KiB),
  // and each lane's source units sit at fixed offsets in the tiles.
  const uint32_t kstride = static_cast<uint32_t>(a.num_kv_heads) * static_cast<uint32_t>(tile_bytes);
  const char* kbase = a.k_cache + static_cast<int64_t>(g) * tile_bytes;
  const char* vbase = a.v_cache + static_cast<int64_t>(g) * tile_bytes;
  // Lane parts of block j's source units, recomputed where used (cheaper than
  // holding them in registers): key offset, value offset, and the value
  // unit's first token in its sub-chunk.
  struct Src {
    int k, v, vtok;
  };
  auto unit_src = [&](int j) __attribute__((always_inline)) {
    const int blk = wave + kMqWaves * j, sub = blk / BPS, pg = blk % BPS;
    const int o = (16 * sub) & (B - 1);  // the sub-chunk's first row in its block (chunks start at block starts)
    const int piece = 4 * pg + (lane >> 4);
    Src r;
    r.k = (piece * B + o + kpos(lane & 15, sub & 1)) * 16;
    if constexpr (kBF16) {
      const int dim = 32 * pg + (lane >> 1), half = (lane & 1) ^ vflip(32 * pg + (lane >> 1));
      r.v = (dim * B + o + 8 * half) * 2;
      r.vtok = 8 * half;
    } else {
      const int dim = 16 * pg + (lane >> 2), slot = (lane & 3) ^ vswz(16 * pg + (lane >> 2));
      r.v = (dim * B + o + 4 * slot) * 4;
      r.vtok = 4 * slot;
    }
    return r;
  };
  // Block ids of chunk c's sub-chunks, read one iteration before they are
  // used (scalar loads; the index is clamped to the sequence's last block,
  // which matters only for sub-chunks past its end, which load nothing).
  auto chunk_ids = [&](int c, int (&ids)[NSUB]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NSUB; ++u) ids[u] = mq_ld(a.block_tables, table_row + min((CT * c + 16 * u) >> lgB, last_blk));
  };
  // Loads chunk c into buffer buf; sub-chunks past the sequence (and past the
  // last chunk) go through size-0 resources and land as zeros.
  auto issue = [&](int c, auto buf, const int (&ids)[NSUB]) __attribute__((always_inline)) {
    char* const lb = lds_buf(buf);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int blk_idx = wave + kMqWaves * j, sub = blk_idx / BPS;  // wave-uniform
      const bool in = c < nc && CT * c + 16 * sub < n;
      const int blk = ids[sub];
      const bool ok = static_cast<unsigned>(blk) < static_cast<unsigned>(a.num_blocks);
      poison |= in && !ok;
      const uint64_t off = ok ? static_cast<uint64_t>(static_cast<uint32_t>(blk)) * kstride : 0;
      const int bytes = (in && ok) ? tile_bytes : 0;
      const Src src = unit_src(j);
      load_to_lds16(make_rsrc(kbase + off, bytes), lb + 1024 * blk_idx, src.k);
      load_to_lds16(make_rsrc(vbase + off, bytes), lb + 1024 * (NBLK + blk_idx), src.v);
    }
  };
  // Values of tokens past the end of the sequence (the cache may hold anything
  // there, NaN poison included) become zeros once this wave's loads of chunk c
  // have landed, so that their zero weights give exact zeros; their keys'
  // scores are masked.  Each wave fixes the units it loaded.
  auto fix_tail = [&](int c, auto buf) __attribute__((always_inline)) {
    if (CT * c + CT <= n) return;  // wave-uniform
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int blk_idx = wave + kMqWaves * j, sub = blk_idx / BPS;
      const int rel = n - (CT * c + 16 * sub + unit_src(j).vtok);  // valid tokens of the unit (8 bf16 or 4 fp32)
      if (rel < (kBF16 ? 8 : 4)) {
        uint32_t* unit = reinterpret_cast<uint32_t*>(lds_buf(buf) + 1024 * (NBLK + blk_idx) + 16 * lane);
        u32x4_t w = *reinterpret_cast<u32x4_t*>(unit);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (kBF16)
            w[e] &= (2 * e < rel ? 0x0000ffffu : 0u) | (2 * e + 1 < rel ? 0xffff0000u : 0u);
          else if (e >= rel)
            w[e] = 0u;
        }
        *reinterpret_cast<u32x4_t*>(unit) = w;
      }
    }
  };

  // Row state: acc and l are relative to the reference m_ref (a raw score; -inf
  // until the row sees a token).  The reference moves lazily: only when some
  // row's maximum exceeds it by more than kLazy in the exp2 domain, so weights
  // stay below 2^kLazy and the accumulators are rarely rescaled.
  constexpr float kLazy = 8.0f;
  f32x4_t acc[T][NDT];
  float m_ref[T], l_run[T];
  int p_first[T];  // the tile's first row position: chunks past it need the causal mask
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[t][dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m_ref[t] = -INFINITY;
    l_run[t] = 0.0f;
    p_first[t] = pos0 + r0[t] / G;
  }

  // Scores of chunk c on the matrix cores, S[token][row m16] for the tokens of
  // score tile u (bf16: 8 (r / 4) + 4 u + r % 4 for tile row r; fp32: sub-chunk
  // u); lane (kq, m16) receives tile rows 4 kq .. 4 kq + 3.  T x NSUB
  // independent chains; a key operand read from LDS serves every row tile.
  auto qk = [&](auto buf, f32x4_t (&sc)[T][NSUB]) __attribute__((always_inline)) {
    const char* kl = lds_buf(buf);
#pragma unroll
    for (int st = 0; st < KS; ++st) {
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        // the key row this lane feeds: token tt of sub-chunk su
        const int tok = kBF16 ? 8 * (m16 >> 2) + 4 * u + (m16 & 3) : 16 * u + m16;
        const int su = tok >> 4, tt = tok & 15;
        const uint4 kv =
            *reinterpret_cast<const uint4*>(kl + su * kSubBytes + ((st * 4 + kq) * 16 + kpos(tt, su)) * 16);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint4 qq = qv[t][st];
          const f32x4_t prev = st == 0 ? f32x4_t{0.0f, 0.0f, 0.0f, 0.0f} : sc[t][u];
          if constexpr (kBF16) {
            sc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv), as_bf16x8(qq), prev, 0, 0, 0);
          } else {
            f32x4_t x = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.x), __uint_as_float(qq.x), prev, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.y), __uint_as_float(qq.y), x, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.z), __uint_as_float(qq.z), x, 0, 0, 0);
            sc[t][u] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.w), __uint_as_float(qq.w), x, 0, 0, 0);
          }
        }
      }
    }
  };

  // Causal mask of chunk c's scores (a token after the row's position, or past
  // the sequence, gets -inf), then the
  // row maxima gm[t] of the chunk (lane column m16; the four lane groups hold
  // its tokens), NaN-propagating: no quieting steps, and a NaN score (garbage
  // in the cache) makes its row NaN.  Chunks that end before the tile's first
  // row need no mask.
  auto mask_max = [&](int c, f32x4_t (&x)[T][NSUB], float (&gm)[T]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (CT * c + CT - 1 > p_first[t]) {
        // the lane's tokens: bf16 8 kq + 4 u + r, fp32 16 u + 4 kq + r
        const int lim = p_row[t] - CT * c - (kBF16 ? 8 : 4) * kq;
#pragma unroll
        for (int u = 0; u < NSUB; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) x[t][u][r] = (kBF16 ? 4 : 16) * u + r > lim ? -INFINITY : x[t][u][r];
      }
      float m = x[t][0][0];
#pragma unroll
      for (int i = 1; i < 4 * NSUB; i += 2) {
        const float y0 = x[t][i / 4][i % 4];
        const float y1 = i + 1 < 4 * NSUB ? x[t][(i + 1) / 4][(i + 1) % 4] : y0;
        m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, y0), y1);
      }
      gm[t] = nmax_xor32(nmax_xor16(m));
    }
  };
  // The lazy reference: when some row's maximum exceeds its reference by more
  // than kLazy (cs (m_new - m_ref) is +inf from an empty start and NaN for a
  // row still empty), every row whose maximum grew moves to it and its
  // accumulators are rescaled.
  auto update = [&](const float (&gm)[T]) __attribute__((always_inline)) {
    float m_new[T];
    bool far = false;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      m_new[t] = __builtin_elementwise_maximum(m_ref[t], gm[t]);
      far = far || cs * (m_new[t] - m_ref[t]) > kLazy;
    }
    if (__ballot(far)) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float alpha = m_new[t] == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(cs * (m_ref[t] - m_new[t]));
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[t][dt] *= alpha;
        l_run[t] *= alpha;
        m_ref[t] = m_new[t];
      }
    }
  };
  // Probabilities p[t][u][r] for the scores sc[t][u][r] of row m16 of tile t; a
  // row whose reference is still -inf (it has seen no token: a split that
  // starts after its position, or a tile past the run) gets weights 0.
  auto probs = [&](const f32x4_t (&x)[T][NSUB], float (&p)[T][NSUB][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float bias = m_ref[t] == -INFINITY ? 0.0f : cs * m_ref[t];
#pragma unroll
      for (int u = 0; u < NSUB; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[t][u][r] = __builtin_amdgcn_exp2f(fmaf(x[t][u][r], cs, -bias));
          l_run[t] += p[t][u][r];
        }
    }
  };
  // O[dim][row] += V[dim][token] P[token][row] for the chunk in buffer buf.
  auto pv = [&](auto buf, const float (&p)[T][NSUB][4], int c) __attribute__((always_inline)) {
    const char* vreg = lds_buf(buf) + 1024 * NBLK;
    if constexpr (kBF16) {
      // One 16x16x32 step per dim tile: lane (kq, m16) supplies k-slots
      // 8 kq .. 8 kq + 7 = tokens 8 kq .. 8 kq + 7 of the chunk, for P (its
      // score registers of tiles 0 and 1) and V (one 8-token unit) alike.  P
      // enters as hi + lo: hi = p truncated to bf16 (the upper halves of two
      // floats, one byte permutation), lo = bf16_rne(p - hi), so
      // |p - hi - lo| <= 2^-16 p.
      static_assert(NSUB == 2, "bf16 chunks are one pair of sub-chunks");
      typedef float f2_t __attribute__((ext_vector_type(2)));
      typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
      auto pack_hi = [](float x, float y) __attribute__((always_inline)) {
        return __builtin_amdgcn_perm(__float_as_uint(y), __float_as_uint(x), 0x07060302u);
      };
      auto pack_lo = [](float x, float y) __attribute__((always_inline)) {
        const f2_t l = {x - __uint_as_float(__float_as_uint(x) & 0xffff0000u),
                        y - __uint_as_float(__float_as_uint(y) & 0xffff0000u)};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(l, b2_t));
      };
      u32x4_t vv[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int dim = 16 * dt + m16;
        vv[dt] = *reinterpret_cast<const u32x4_t*>(vreg + (kq >> 1) * kSubBytes + 1024 * (dim >> 5) +
                                                   16 * (2 * (dim & 31) + ((kq & 1) ^ vflip(dim))));
      }
      u32x4_t ph[T], pl[T];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        ph[t] = u32x4_t{pack_hi(p[t][0][0], p[t][0][1]), pack_hi(p[t][0][2], p[t][0][3]),
                        pack_hi(p[t][1][0], p[t][1][1]), pack_hi(p[t][1][2], p[t][1][3])};
        pl[t] = u32x4_t{pack_lo(p[t][0][0], p[t][0][1]), pack_lo(p[t][0][2], p[t][0][3]),
                        pack_lo(p[t][1][0], p[t][1][1]), pack_lo(p[t][1][2], p[t][1][3])};
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int t = 0; t < T; ++t)
          acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vv[dt]),
                                                               __builtin_bit_cast(bf16x8_t, ph[t]), acc[t][dt], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < T; ++t)
          acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vv[dt]),
                                                               __builtin_bit_cast(bf16x8_t, pl[t]), acc[t][dt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        if (CT * c + 16 * u > p_wave) break;  // no row of the wave sees these tokens (wave-uniform)
        uint4 vv[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int dim = 16 * dt + m16;
          vv[dt] = *reinterpret_cast<const uint4*>(vreg + u * kSubBytes + 64 * dim + 16 * (kq ^ vswz(dim)));
        }
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
  };

  // Chunk c sits in LDS buffer (c - c_begin) mod NBUF.  Iteration c starts the
  // loads of chunk c + NBUF - 1 into the buffer chunk c - 1 left before the
  // previous barrier, computes chunk c (scores, softmax, value product), then
  // waits for this wave's loads of chunk c + 1 (issued at least one iteration
  // earlier), fixes its tail, and meets the other waves at the barrier.  The
  // barrier is a plain s_barrier after explicit waits: a workgroup fence there
  // would also wait for the loads still in flight.
  constexpr int NL = 2 * NB;  // loads per lane per chunk
  auto barrier_after_loads = [](auto keep) __attribute__((always_inline)) {
    // vmcnt(keep): at most `keep` of this wave's loads still outstanding; lgkmcnt(0): its LDS accesses done
    static_assert(decltype(keep)::value < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0070 | decltype(keep)::value);
    asm volatile("s_barrier" ::: "memory");
  };
  using Keep = std::integral_constant<int, (NBUF - 2) * NL>;
  int ids[NSUB];
  chunk_ids(c_begin, ids);
  issue(c_begin, std::integral_constant<int, 0>{}, ids);
  if constexpr (NBUF == 3) {
    chunk_ids(c_begin + 1, ids);
    issue(c_begin + 1, std::integral_constant<int, 1>{}, ids);
  }
  chunk_ids(c_begin + NBUF - 1, ids);  // for the first iteration
  __builtin_amdgcn_s_waitcnt(0x0070 | Keep::value);
  fix_tail(c_begin, std::integral_constant<int, 0>{});
  barrier_after_loads(Keep{});
  // One iteration, for chunk c in buffer `buf` (a compile-time constant).
  auto step = [&](int c, auto buf) __attribute__((always_inline)) {
    constexpr int b = decltype(buf)::value;
    issue(c + NBUF - 1, std::integral_constant<int, (b + NBUF - 1) % NBUF>{}, ids);
    chunk_ids(c + NBUF, ids);  // for the next iteration
    if (c < nc && CT * c <= p_wave) {  // a chunk of this split that some row of the wave sees (wave-uniform)
      f32x4_t sc[T][NSUB];
      float gm[T], p[T][NSUB][4];
      qk(buf, sc);
      mask_max(c, sc, gm);
      update(gm);
      probs(sc, p);
      pv(buf, p, c);
    }
    __builtin_amdgcn_s_waitcnt(0x0070 | Keep::value);
    fix_tail(c + 1, std::integral_constant<int, (b + 1) % NBUF>{});
    barrier_after_loads(Keep{});
  };
  // Whole rounds of NBUF steps: a step past the last chunk loads zeros and
  // computes nothing, and the steps need no branch between them (which keeps
  // the compiler's tracking of the loads in flight per buffer exact).
  for (int c = c_begin; c < nc; c += NBUF) {
    step(c, std::integral_constant<int, 0>{});
    step(c + 1, std::integral_constant<int, 1>{});
    if constexpr (NBUF == 3) step(c + 2, std::integral_constant<int, 2>{});
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
        a.ws_m[part] = m_ref[0] == -INFINITY ? -INFINITY : cs * m_ref[0];  // the reference, exp2 domain
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
// Runs the attention kernel did not write, or wrote as NaN, are skipped, and
// so are those it left to another launch.
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
  if (q0 < 0 || qs <= a.skip_upto || static_cast<int64_t>(q0) + qs > a.num_query_rows) return;
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

extern "C" size_t pkv_attention_multi_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                      int32_t head_dim, int32_t max_context_len, int32_t max_query_len);

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
  // A workspace, when given, has at least the advertised size for these sizes (whichever path the call takes).
  if (workspace) {
    const size_t need = pkv_attention_multi_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                            max_context_len, max_query_len);
    if (need > 0 && (workspace_bytes < need || !aligned16(workspace))) return PKV_ERR_WORKSPACE;
  }

  // Runs of at most 16 / G queries (verification of drafted tokens, decodes)
  // go to the decode kernel's listed path, where the queries of a run are
  // further matrix-core columns of one persistent, cost-balanced pass
  // (seq_order does not apply there).  A batch whose longest run is longer
  // and whose rows say that some runs are shorter (a mixed step: prompt chunks
  // beside decodes) takes two launches: the short runs there, then the
  // longer ones here.  PKV_MULTI_PATH=runs (read at each call) keeps every
  // run here.
  int skip_upto = 0;
  {
    const char* path = std::getenv("PKV_MULTI_PATH");
    if (!(path && std::strcmp(path, "runs") == 0)) {
      const int short_len = 16 / G;
      if (max_query_len <= short_len) {
        const pkv_status st = runs_listed(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                                          num_seqs, num_query_rows, num_q_heads, num_kv_heads, head_dim, block_size,
                                          num_blocks, max_blocks, max_context_len, max_query_len, false, scale,
                                          workspace, workspace_bytes, kv_dtype, stream);
        if (st != PKV_ERR_UNSUPPORTED) return st;
      } else if (static_cast<int64_t>(num_query_rows) < static_cast<int64_t>(num_seqs) * max_query_len) {
        const pkv_status st = runs_listed(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                                          num_seqs, num_query_rows, num_q_heads, num_kv_heads, head_dim, block_size,
                                          num_blocks, max_blocks, max_context_len, short_len, true, scale,
                                          workspace, workspace_bytes, kv_dtype, stream);
        if (st == PKV_OK) skip_upto = short_len;
        else if (st != PKV_ERR_UNSUPPORTED) return st;
      }
    }
  }

  // Two row tiles per wave when a pair has more rows than one workgroup of
  // one-tile waves holds and there is work enough for the coarser workgroups
  // (two fit a CU, against three of one tile; a two-tile workgroup reads each
  // chunk once for twice the rows).  The host's measures of the work are the
  // row counts: the batch's rows, num_query_rows * G, make at least one full
  // round of two-tile workgroups; or, with every run of this launch a long
  // one (the short runs taken by the decode kernel, or all runs of the longest
  // length) and contexts of at least twice the longest run (runs at the end of
  // longer contexts, as chunked prompts are, so that the row blocks of a pair
  // cost about the same), the rows of all pairs, num_query_rows * H_q, do.
  // Otherwise one tile per wave gives more, smaller workgroups to spread a
  // few causal prompts, or short runs, over.  PKV_MULTI_TILES=1 or 2 (read at
  // each call) forces the choice; both kernels give the same rows.
  int T = 1;
  if (static_cast<int64_t>(max_query_len) * G > kMqRows) {
    const char* force = std::getenv("PKV_MULTI_TILES");
    if (force && (force[0] == '1' || force[0] == '2') && force[1] == 0) {
      T = force[0] - '0';
    } else {
      const int64_t round2 = 2 * static_cast<int64_t>(device_cus()) * 2 * kMqRows;  // rows of one full round
      const bool long_only = skip_upto > 0 || static_cast<int64_t>(num_query_rows) ==
                                                  static_cast<int64_t>(num_seqs) * max_query_len;
      const bool tails = long_only && max_context_len >= 2 * static_cast<int64_t>(max_query_len);
      if (static_cast<int64_t>(num_query_rows) * G >= round2 ||
          (tails && static_cast<int64_t>(num_query_rows) * num_q_heads >= round2))
        T = 2;
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
  a.skip_upto = skip_upto;
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
  const size_t split = multi_plan(num_seqs, num_kv_heads, num_q_heads / num_kv_heads, head_dim, max_context_len,
                                  max_query_len).bytes;
  // the decode kernel takes the runs of at most 16 / G queries (all of them, or the short ones of a mixed step)
  const int32_t short_len = 16 / (num_q_heads / num_kv_heads);
  const size_t listed = runs_listed_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                                    max_query_len < short_len ? max_query_len : short_len);
  return split > listed ? split : listed;
}

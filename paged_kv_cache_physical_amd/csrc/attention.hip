// Paged decode attention for gfx950: one query token per sequence, keys and
// values read through block tables.  [P1] (lain42.top reading note), summary
// section 2, core method: one custom kernel fuses the table lookup, the fetch
// of scattered blocks and the attention; [P2] (aiplusplus.yigather.com
// explainer), key technical point 1: the kernel reads each sequence's blocks
// through its block table.  The pages do not describe cutting one context
// across workgroups: the split context and its log-sum-exp combination are
// this library's own, so that a few long sequences still fill the GPU.
//
// Unit of work: an item = the tokens of one sequence that a workgroup computes
// for one KV head: a segment of its run of the cost-ordered work (up to 4096
// sequences, see the kernel), or one context partition of at most P tokens.
// A workgroup of four waves walks its list of items (persistent grid).  Wave
// w takes the groups g = w, w + 4, ... of an item; a group is one cache block
// (bf16) or 16 tokens (fp32).  Per group a wave
//   - multiplies the group's keys with the G query heads of the KV head on the
//     matrix cores (QK^T: rows = tokens, columns = heads),
//   - folds the group into an online softmax per head (running maximum in the
//     exp2 domain, rescaling the accumulator when the maximum grows),
//   - multiplies the probabilities with the group's values on the matrix
//     cores (rows = head dimensions, columns = heads), accumulating in fp32.
// The groups' keys and values sit in a register ring of NBUF slots; after a
// slot is consumed it is refilled with the group NBUF positions ahead, which
// crosses into the next item of the workgroup, so loads stay in flight across
// item boundaries.  The four waves merge their (max, sum, acc) through LDS
// and write the item's output rows (one partition) or its partials.
//
// Precision.  QK: exact bf16 (or fp32) products, fp32 accumulation.  PV with
// bf16 caches: each probability p is split as p = hi + lo, hi its truncation
// to bf16 and lo = bf16_rne(p - hi), so |p - hi - lo| <= 2^-16 p; both halves
// multiply the exact bf16 values and PV keeps fp32-level accuracy.  fp32
// caches use the fp32 matrix instructions throughout.
//
// Loads.  Keys, values and the query go through buffer resources.  A ring
// slot with no group to hold uses a resource of size 0: the hardware returns
// zeros without touching memory.  Every load is issued on every path, which
// keeps the compiler's wait counters exact (a load behind a branch makes it
// wait for all earlier loads where the paths join).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "device_common.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;  // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxListedSeqs = 4096;    // sequences whose item list fits the LDS prefix sums
constexpr int kLoadNT = 2;              // buffer-load cache policy: nontemporal

struct AttnArgs {
  float* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const void* k_new;  // decode step: the new token of each sequence [S][H_kv][d], written to the caches
  const void* v_new;  // (nullptr: no write)
  // Workspace.  Item list (LIST): two records per workgroup b, record 2 b + j:
  //   j = 1: the run's last segment when the run ends inside a sequence (an
  //          empty segment for a run with no tokens that starts and ends there),
  //   j = 0: the run's first segment when it is the last one of a sequence that
  //          began in an earlier run (its "owner", which combines the sequence).
  // Partition items (not LIST): one slot per (sequence, KV head, partition).
  float* ws_acc;  // LIST [2 grid][G][d]; else [S][H_kv][max_parts][G][d]: un-normalised sums
  float* ws_m;    // LIST [2 grid][G];    else [S][H_kv][max_parts][G]: maximum logit, exp2 domain (scaled)
  float* ws_l;    // LIST [2 grid][G];    else [S][H_kv][max_parts][G]: sum of exp2(logit - max)
  int32_t* ws_seg;  // not LIST [S][H_kv][max_parts]: at a segment's slot, the slot of the sequence's next
                    // segment (num partitions after the last); at slot 0 of a sequence written whole: -1
  int32_t* ws_hdr;  // LIST [2 grid][4]: (sequence, first token, end token, 1 if record 0 of an owner)
  uint64_t* ws_tag; // LIST [2 grid][2]: (turn, flag) of each record, see tag_next
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t max_context_len;
  int32_t partition_size;  // tokens, multiple of block_size
  int32_t max_parts;
  int32_t total_items;     // max_parts * num_seqs * num_kv_heads
  float c;                 // scale * log2(e): the softmax runs on u = c * (q . k) in the exp2 domain
  // Runs of queries (kernels with QR > 1 queries per item): sequence s owns the
  // query rows query_start[s] .. query_start[s + 1] - 1 of q and out, which are
  // [num_query_rows][num_q_heads][d]; decode (QR = 1) has one row per sequence.
  const int32_t* query_start;
  int32_t num_q_heads;
  int32_t num_query_rows;
  int32_t max_query_len;
  int32_t skip_long;  // 1: a run longer than max_query_len belongs to another launch (nothing is written)
};

// Hand-over of a record between workgroups of one launch, with no contract on
// what the workspace holds beforehand.  Each record has a pair (turn, flag).
// The writer of a record stores its data, makes it visible to the device,
// then sets flag = tag_next(turn); the reader waits for exactly that value,
// reads the data, and sets turn = tag_next(turn), which leaves flag == turn.
// Visibility across the XCDs (each with its own L2) comes from the device
// scope of the accesses themselves, not from fences: every store of a record
// and of its pair has the device-scope bit (sc1), so it writes through the
// L2, and every load of them has it too, so it misses in any cache that is
// not coherent across the device; each writing wave waits for its stores to
// complete (vmcnt(0)) before the flag is stored.  (A device-scope release or
// acquire fence instead writes back or invalidates the XCD's whole L2 on
// gfx950; done at every hand-over it made the pass 60% slower.)
// tag_next is a bijection of 64-bit words (the output function of
// SplitMix64, Steele, Lea and Flood), so from any state that ended a hand-over
// (flag == turn) the next one needs a fresh write, and a pair that holds
// unrelated data matches tag_next by chance with probability 2^-64.  The
// pairs are indexed by record, whose position depends on the launch, so every
// hand-over reads its own turn instead of a value passed in: replays of a
// captured graph work the same way.
__device__ __forceinline__ uint64_t tag_next(uint64_t x) {
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}
constexpr int kMaxPolls = 1 << 20;  // about a second of polling: a record that never comes gives NaN rows
constexpr int kScopeDevice = 16;    // buffer-access cache policy: sc1, device scope (through L2)

__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
// Device-scope loads through a wave-uniform resource at a per-lane byte
// offset (an offset past the resource, such as kNowhere, reads zeros).
__device__ __forceinline__ f32x4_t load_dev4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kScopeDevice));
}
__device__ __forceinline__ float load_dev(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kScopeDevice));
}
__device__ __forceinline__ int4 load_dev_i4(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kScopeDevice);
  return make_int4(static_cast<int>(v[0]), static_cast<int>(v[1]), static_cast<int>(v[2]), static_cast<int>(v[3]));
}

// Number of partitions of a sequence of n_raw tokens (1 for an empty or
// invalid one); sets *bad for invalid lengths.
__device__ __forceinline__ int seq_parts(const AttnArgs& a, int n_raw, bool* bad) {
  *bad = n_raw < 0 || n_raw > a.max_context_len ||
         static_cast<int64_t>(n_raw) > static_cast<int64_t>(a.max_blocks) * a.block_size;
  if (*bad || n_raw == 0) return 1;
  return (n_raw + a.partition_size - 1) / a.partition_size;
}

// Marks a value wave-uniform (values read from LDS land in vector registers).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint64_t uni64(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(x)));
}

// Reads of the block tables and lengths go through the constant address space:
// the kernel never writes them, so the compiler may use scalar loads, which
// the vector loads' wait counter does not see.  (A vector load there makes
// every later wait for it also wait for all the ring loads issued before.)
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ int32_t ld_const(const int32_t* p, size_t i) {
  return ((const_i32_ptr)p)[i];
}

// A sequence's query rows (its run): rows q0 .. q0 + nq - 1 of q and out, at
// positions n - nq .. n - 1 of its context.  Decode (QR = 1): the
// sequence's own row.  A run can also be (as the runs kernel takes it):
// outside the rows (nothing is written), or impossible (longer than its
// context or than the batch's longest run: NaN rows, at most max_query_len of
// them).  With skip_long, a run longer than max_query_len is left to the runs
// kernel (nothing written).
struct RunRows {
  int q0, nq;
  bool bad;
};
template <int QR>
__device__ __forceinline__ RunRows run_rows(const AttnArgs& a, int s, int n) {
  if constexpr (QR == 1) return RunRows{s, 1, false};
  const int q0 = ld_const(a.query_start, s);
  const int qs = ld_const(a.query_start, s + 1) - q0;
  const bool rows = q0 >= 0 && qs > 0 && static_cast<int64_t>(q0) + qs <= a.num_query_rows &&
                    !(a.skip_long && qs > a.max_query_len);
  return RunRows{q0, rows ? min(qs, a.max_query_len) : 0, rows && (qs > n || qs > a.max_query_len)};
}
// Partitions of sequence s (1 when it has no tokens to read: *special), with
// *bad for NaN rows.
template <int QR>
__device__ __forceinline__ int seq_state(const AttnArgs& a, int s, int n, bool* special, bool* bad) {
  const int np = seq_parts(a, n, bad);
  if constexpr (QR == 1) {
    *special = *bad || n == 0;
    return np;
  }
  const RunRows r = run_rows<QR>(a, s, n);
  *bad = r.nq > 0 && (*bad || r.bad);
  *special = *bad || n == 0 || r.nq == 0;
  return *special ? 1 : np;
}

// voff: the lane's offset; soff: a wave-uniform offset added to it.  A load
// stays inside its tile, and a size-0 resource rejects every load, so the
// result does not depend on whether the range check includes soff.
template <int kAux>
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kAux);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
template <int kAux>
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kAux);
  return make_uint2(v[0], v[1]);
}

// Per-instantiation geometry.
//   K tile (one block, one KV head): [d / X][B][X], X = 16 bytes of scalars.
//   V tile: [d][B].
template <class DT, int D, int B>
struct Geo {
  static constexpr bool kBF16 = std::is_same<DT, BF16>::value;
  static constexpr int kItem = DT::kItem;
  static constexpr int R = D * kItem;                    // bytes of one token row
  static constexpr int TILE = B * R;                     // bytes of one (block, KV head) tile
  static constexpr int GT = kBF16 ? B : 16;              // tokens per group
  static constexpr int NT = GT / 16;                     // 16-token QK tiles per group
  static constexpr int KS = R / 64;                      // key registers (16 B) per lane per QK tile
  static constexpr int NDT = D / 16;                     // 16-row tiles of the head dimension
  static constexpr int VW = (kBF16 && B == 16) ? 2 : 4;  // value dwords per lane per d-tile
  static constexpr int NQ = KS;                          // query registers (16 B) per lane
  static constexpr int SLOT = NT * KS * 4 + NDT * VW;    // VGPRs of one ring slot
  static constexpr int NBUF = 128 / SLOT;                // ring slots: 128 VGPRs of loads in flight
  static_assert(NBUF >= 2 && (NBUF & (NBUF - 1)) == 0, "ring depth");
};

// One decoded item: a segment, i.e. tokens [tok_begin, tok_end) of one
// sequence for one KV head.  Every field is wave-uniform.
struct Item {
  int k;     // item index (>= the workgroup's end: none)
  int next;  // the item after it in this workgroup's list
  int seq, kvh;
  int part;       // workspace slot of the segment
  int part_next;  // slot of the sequence's next segment (num partitions after the last)
  int tok_begin, tok_end;
  int nk;     // groups of this wave
  int npad;   // ring positions of this wave: nk rounded up to NBUF, at least NBUF
  int flags;  // kDirect | kSplitSeq | kSpecial | kBad
  int n;      // the sequence's length
  int q0, nq; // its query rows (see run_rows)
  int new_id; // kNew: the block id of the slot of token n - 1
};
constexpr int kDirect = 1;    // the segment covers the whole sequence: write the output rows
constexpr int kSplitSeq = 2;  // the sequence has several partitions
constexpr int kSpecial = 4;   // empty or invalid sequence: no groups, fill the rows
constexpr int kBad = 8;       // invalid length: fill with NaN
constexpr int kNew = 16;      // decode step: the segment holds the new token (n - 1), taken from the inputs

// C: matrix-core columns in use, a (query, head) pair each (decode: the G
// heads).  Up to 8 columns the items alternate between two merge buffers (one
// barrier per item); 16 columns take one buffer and a second barrier.
template <int C, int D, bool LIST, int NEWW>
struct Shared {
  struct Merge {
    alignas(16) float region[kWaves][C][D + 4];  // per-wave partial output (padded rows)
    float wm[kWaves][C];                         // per-wave running maximum (exp2 domain, scaled)
    float wl[kWaves][C];                         // per-wave sum of probabilities
  } mb[C > 8 ? 1 : 2];
  uint32_t csum[LIST ? kMaxListedSeqs + 1 : 1];  // prefix sums of sequence costs
  int chain_first;  // combine: the first run holding a segment of the owner's sequence
  int chain_ok;     // combine: every segment arrived and belongs to the sequence
  // decode step (NEWW > 0): the new token's key and value rows (NEWW dwords
  // each) of the current item, in two entries that alternate between items
  alignas(16) uint32_t knew[NEWW > 0 ? 2 : 1][NEWW > 0 ? NEWW : 1];
  uint32_t vnew[NEWW > 0 ? 2 : 1][NEWW > 0 ? NEWW : 1];
};

// Cost of a partition in the work split: its groups plus a fixed charge for
// an item's start-up and merge, worth eight groups (a boundary drains and
// refills a wave's ring and meets the other waves twice; charges of 2 to 8
// were measured, 8 the fastest on the GQA and Llama-7B decode batches).
constexpr int kItemCharge = 8;

// Log-sum-exp combination of one sequence's segments for one KV head: the
// segments sit in record 1 of runs first .. last - 1 and record 0 of run last,
// in token order, and
//   out = sum_r 2^(m_r - M) acc_r / sum_r 2^(m_r - M) l_r,   M = max_r m_r,
// summed in that order (an empty segment has m = -inf and weighs nothing).
// Explicit fmaf keeps the rounding identical wherever this is inlined, so the
// fused and the two-stage paths give the same bits.  ok == false: NaN rows.
// Column h of a record is query h / G of the run, head h % G of the KV head.
template <int G, int QR, int D>
__device__ __forceinline__ void combine_runs(const AttnArgs& a, int seq, int kvh, int first, int last, bool ok,
                                             int tid) {
  constexpr int C = QR * G;
  constexpr int NC = D / 4;  // float4 chunks of one head's row
  constexpr int ITERS = (C * NC + kThreads - 1) / kThreads;
  const int Hkv = a.num_kv_heads;
  const RunRows run = run_rows<QR>(a, seq, 0);
  const int Hq = Hkv * G;
  float* out = a.out + (static_cast<size_t>(run.q0) * Hq + static_cast<size_t>(kvh) * G) * D;
  auto rec_of = [&](int L) __attribute__((always_inline)) { return 2 * (L * Hkv + kvh) + (L == last ? 0 : 1); };
  // the launch's records: 2 per workgroup (at most 2 * 2048 * 16 * 128 * 4 bytes of sums)
  const int recs = 2 * static_cast<int>(gridDim.x);
  const __amdgpu_buffer_rsrc_t r_acc = make_rsrc(a.ws_acc, recs * C * D * 4);
  const __amdgpu_buffer_rsrc_t r_m = make_rsrc(a.ws_m, recs * C * 4);
  const __amdgpu_buffer_rsrc_t r_l = make_rsrc(a.ws_l, recs * C * 4);
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int cidx = tid + it * kThreads;
    if (cidx >= C * NC) break;
    const int h = cidx / NC, d4 = (cidx % NC) * 4;
    if (h / G >= run.nq) break;  // columns past the run's queries (cidx grows with h)
    f32x4_t o = {__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    if (ok) {
      // Records in groups of kGroup whose loads are all in flight at once (a
      // record past the last one reads zeros, at an offset past the resource,
      // and weighs nothing).  Up to kGroup records take one round of loads;
      // more take a first round for the maximum.
      constexpr int kGroup = 8;
      float mv[kGroup], lv[kGroup];
      f32x4_t av[kGroup];
      auto load_group = [&](int L0, bool sums) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
          const int r = rec_of(L0 + j) * C + h;
          const bool in = L0 + j <= last;
          mv[j] = load_dev(r_m, in ? r * 4 : kNowhere);
          if (sums) {
            lv[j] = load_dev(r_l, in ? r * 4 : kNowhere);
            av[j] = load_dev4(r_acc, in ? (r * D + d4) * 4 : kNowhere);
          }
        }
      };
      float M = -INFINITY;
      f32x4_t sa = {0.0f, 0.0f, 0.0f, 0.0f};
      float sl = 0.0f;
      auto add_group = [&](int L0) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
          const float w = L0 + j <= last ? __builtin_amdgcn_exp2f(mv[j] - M) : 0.0f;
          sa.x = fmaf(w, av[j].x, sa.x);
          sa.y = fmaf(w, av[j].y, sa.y);
          sa.z = fmaf(w, av[j].z, sa.z);
          sa.w = fmaf(w, av[j].w, sa.w);
          sl = fmaf(w, lv[j], sl);
        }
      };
      if (last - first < kGroup) {
        load_group(first, true);
#pragma unroll
        for (int j = 0; j < kGroup; ++j) M = fmaxf(M, first + j <= last ? mv[j] : -INFINITY);
        add_group(first);
      } else {
        for (int L0 = first; L0 <= last; L0 += kGroup) {
          load_group(L0, false);
#pragma unroll
          for (int j = 0; j < kGroup; ++j) M = fmaxf(M, L0 + j <= last ? mv[j] : -INFINITY);
        }
        for (int L0 = first; L0 <= last; L0 += kGroup) {
          load_group(L0, true);
          add_group(L0);
        }
      }
      o = f32x4_t{sa.x / sl, sa.y / sl, sa.z / sl, sa.w / sl};
    }
    *reinterpret_cast<f32x4_t*>(out + (static_cast<size_t>(h / G) * Hq + h % G) * D + d4) = o;
  }
}

// Workgroup b serves KV head b % H_kv (the grid is a multiple of H_kv), so the
// H_kv workgroups of lane b / H_kv read the adjacent head tiles of the same
// blocks at about the same time.
// LIST (at most kMaxListedSeqs sequences): the sequences' work, laid out in
// order with LDS prefix sums of a cost per sequence (its groups plus a charge
// per partition), is cut into one contiguous run per lane, each starting
// where the cumulative cost reaches L C / lanes (C the total): the lanes get
// equal work to within one group.  A lane's run is walked one sequence at a
// time: an item is the run's tokens of one sequence, computed as one softmax,
// so only a sequence cut between lanes leaves partial results (one set per
// segment).  Otherwise every partition is an item: numbered part-major over
// max_parts, dealt round-robin to the lanes, the empty ones (partition past
// the sequence's end) skipped.  WRITE (LIST only): the decode step's variant,
// which also stores each sequence's new token (position n - 1): the segment
// that ends with it puts the token's key and value from the call's inputs
// into the ring registers in place of the cache slot's bytes (the same bits
// the cache holds once written, so the result equals the two-call path's),
// and the workgroups store the tokens into the caches at their start with no
// ordering against the reads; bf16 with 32-token blocks (no registers to
// spare) instead stores the tokens of its own run first and waits for them.
// FUSED (LIST only): the workgroup whose run starts with the last segment of a
// sequence cut between runs (its owner) combines that sequence's segments at
// the end of its run, once the earlier runs have handed their records over;
// without it, list_reduce_kernel does the same work as a second launch.  An
// owner waits only for runs of lower index, which never wait on it, and it
// waits after its own work is done, so every run's work proceeds.
// QR > 1 (runs of queries, LIST and FUSED only): each item carries up to QR
// queries of its sequence (its last positions), C = QR G columns of the
// matrix-core tiles, column h being query h / G and head h % G; query i of a
// run of nq sees the tokens up to position n - nq + i.
template <class DT, int D, int G, int B, bool LIST, bool WRITE, bool FUSED, int QR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void paged_decode_kernel(AttnArgs a) {
  using Gm = Geo<DT, D, B>;
  constexpr int GT = Gm::GT, NT = Gm::NT, KS = Gm::KS, NDT = Gm::NDT, VW = Gm::VW, NQ = Gm::NQ;
  constexpr int NBUF = Gm::NBUF, R = Gm::R, TILE = Gm::TILE;
  constexpr bool kBF16 = Gm::kBF16;
  constexpr int NCOL = QR * G;  // columns in use
  // WRITE: how the new token enters.  Late: the segment that ends with it
  // takes its key and value from the inputs and stores them at its end.
  // First: every run stores its sequences' tokens before reading (bf16 with
  // 32-token blocks, whose ring leaves no registers for the late form).
  constexpr bool kTokenFirst = WRITE && kBF16 && B == 32;
  constexpr bool kTokenLate = WRITE && !kTokenFirst;
  static_assert(NCOL <= 16 && (QR == 1 || (LIST && FUSED && !WRITE)), "runs: 16 columns, listed and fused");
  __shared__ Shared<NCOL, D, LIST, kTokenLate ? Gm::R / 4 : 0> sh;

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = uni(tid / kWave);
  const int m16 = lane & 15, kq = lane >> 4;
  const int S = a.num_seqs, Hkv = a.num_kv_heads;
  const int grid = static_cast<int>(gridDim.x);

  // ---- items ---------------------------------------------------------------
  const int P = a.partition_size;
  const int full_cost = P / GT + kItemCharge;  // cost of a full partition
  const int kvh_b = static_cast<int>(blockIdx.x) % Hkv;
  const int lanes = grid / Hkv;
  const int lane_b = static_cast<int>(blockIdx.x) / Hkv;
  if constexpr (LIST) {
    for (int s = tid; s < S; s += kThreads) {
      bool bad, special;
      const int n = ld_const(a.context_lens, s);
      const int np = seq_state<QR>(a, s, n, &special, &bad);
      const int last = special ? 0 : n - (np - 1) * P;  // tokens of the last partition
      sh.csum[s + 1] = static_cast<uint32_t>(np - 1) * full_cost + (last + GT - 1) / GT + kItemCharge;
    }
    if constexpr (kTokenLate) {
      // The new tokens into the caches, once the lengths are read: workgroup
      // (lane, KV head) stores the tokens of sequences lane, lane + lanes, ...
      // of its head, through L2, while it works out its run; it waits for the
      // stores before its first read.  No ordering with the reads of other workgroups is
      // needed, as the reading segment takes the token from the inputs.
      using TT = typename std::conditional<kBF16, uint16_t, uint32_t>::type;
      constexpr int E = 16 / static_cast<int>(sizeof(TT));
      for (int s = lane_b + lanes * wave; s < S; s += lanes * kWaves) {
        const int n = ld_const(a.context_lens, s);
        bool bad;
        seq_parts(a, n, &bad);
        if (bad || n == 0) continue;
        const int id = ld_const(a.block_tables, static_cast<size_t>(s) * a.max_blocks + (n - 1) / B);
        if (static_cast<unsigned>(id) >= static_cast<unsigned>(a.num_blocks)) continue;
        const size_t row = (static_cast<size_t>(s) * Hkv + kvh_b) * D;
        const TT* krow = static_cast<const TT*>(a.k_new) + row;
        const TT* vrow = static_cast<const TT*>(a.v_new) + row;
        const uint4 kv = *reinterpret_cast<const uint4*>(krow + (lane < D / E ? lane : 0) * E);
        const TT v0 = vrow[lane];
        const TT v1 = D > 64 ? vrow[64 + lane] : TT(0);
        store_token_rows<TT, kStoreThrough>(const_cast<char*>(static_cast<const char*>(a.k_cache)),
                                            const_cast<char*>(static_cast<const char*>(a.v_cache)),
                                            static_cast<int64_t>(id) * Hkv + kvh_b, (n - 1) % B, B, D, lane, kv, v0, v1);
      }
    }
    __syncthreads();
    if (wave == 0) {  // scan of the costs: a chunk per lane, then a wave-wide scan of the chunk sums
      uint32_t* arr = sh.csum;
      const int chunk = (S + kWave - 1) / kWave;
      const int lo = lane * chunk, hi = min(S, lo + chunk);
      uint32_t run = 0;
      for (int i = lo; i < hi; ++i) run += arr[i + 1];
      uint32_t incl = run;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      uint32_t base = incl - run;
      for (int i = lo; i < hi; ++i) {
        base += arr[i + 1];
        arr[i + 1] = base;
      }
      if (lane == 0) arr[0] = 0;
    }
    __syncthreads();
  }
  // LIST: the cut at cost position T, as (sequence, first token).  A sequence's
  // cost is laid out partition by partition: the charge, then one unit per
  // group.  T maps to the first group whose cost starts at or after it
  // ("fine" cuts), or, when lanes are short, to the first partition start at
  // or after it; a single-partition sequence is never cut (the nearer end
  // wins).  The result is monotone in T, so consecutive lanes tile the work.
  struct Cut {
    int seq, tok;
  };
  const uint64_t C = LIST ? uni64(sh.csum[S]) : 0;
  const bool fine = C >= static_cast<uint64_t>(4) * lanes * full_cost;
  // The cut inside sequence lo, where csum[lo] = base <= T < csum[lo + 1].
  auto cut_in = [&](int lo, uint64_t T, uint64_t base) __attribute__((always_inline)) {
    Cut c{S, 0};
    const int n = ld_const(a.context_lens, lo);
    bool bad, special;
    const int np = seq_state<QR>(a, lo, n, &special, &bad);
    const uint64_t rel = T - base;
    if (special) {  // no tokens: the sequence starts the run that holds its first cost unit
      c.seq = rel == 0 ? lo : lo + 1;
      return c;
    }
    const int p = rel >= static_cast<uint64_t>(np - 1) * full_cost ? np - 1 : static_cast<int>(rel / full_cost);
    const int u = static_cast<int>(rel - static_cast<uint64_t>(p) * full_cost);
    int tok;
    if (fine) {
      tok = p * P + max(0, u - kItemCharge) * GT;
      if (np == 1 && tok > 0 && tok < n) tok = tok < n / 2 ? 0 : n;
    } else {
      tok = (u == 0 ? p : p + 1) * P;
    }
    c.seq = tok >= n ? lo + 1 : lo;
    c.tok = tok >= n ? 0 : tok;
    return c;
  };
  auto cut_at = [&](uint64_t T) __attribute__((always_inline)) {
    if (T >= C) return Cut{S, 0};
    // csum[lo] <= T < csum[lo + 1]: csum rises strictly, so the lanes of a wave
    // test 64 evenly spaced candidates and narrow the range 64-fold per round
    // (two rounds for up to 4096 sequences).
    int lo = 0, span = S;
    while (span > 1) {
      const int step = (span + kWave - 1) / kWave, end = lo + span;
      const int idx = lo + lane * step;
      const uint64_t below = __ballot(idx < end && sh.csum[idx] <= T);
      lo += (__popcll(below) - 1) * step;
      span = min(step, end - lo);
    }
    return cut_in(lo, T, uni64(sh.csum[lo]));
  };
  // The same cut found by one lane alone (a binary search), for a different T per lane.
  auto cut_at_lane = [&](uint64_t T) __attribute__((always_inline)) {
    if (T >= C) return Cut{S, 0};
    int lo = 0, hi = S;  // csum[lo] <= T < csum[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sh.csum[mid] <= T)
        lo = mid;
      else
        hi = mid;
    }
    return cut_in(lo, T, sh.csum[lo]);
  };
  // Not LIST: first non-empty partition item at or after k in this workgroup's stride.
  const int total = a.total_items;
  auto seek = [&](int k) __attribute__((always_inline)) {
    for (; k < total; k += grid) {
      const int r = k / Hkv;
      bool bad;
      if (r / S < seq_parts(a, ld_const(a.context_lens, r % S), &bad)) break;
    }
    return uni(k);
  };

  // This workgroup's items: LIST, the sequences of its lane's run (first and
  // last possibly cut); otherwise partition items of its stride.
  int k_first, k_end;
  Cut run_begin{0, 0}, run_end{0, 0};
  if constexpr (LIST) {
    run_begin = cut_at((static_cast<uint64_t>(lane_b) * C + lanes - 1) / lanes);
    run_end = cut_at((static_cast<uint64_t>(lane_b + 1) * C + lanes - 1) / lanes);
    k_first = run_begin.seq;
    k_end = run_end.tok > 0 ? run_end.seq + 1 : run_end.seq;
    if (run_end.seq == run_begin.seq && run_end.tok <= run_begin.tok) k_end = k_first;  // empty run
  } else {
    k_first = seek(static_cast<int>(blockIdx.x));
    k_end = total;
  }
  // Workspace slot of a segment starting at token t of a sequence: its
  // partition, except that a start inside partition 0 (other than 0) uses
  // slot 1.  Lanes hold at least 4 partitions of cost when cuts are fine, so
  // no two segments of one sequence share a slot.
  auto slot_of = [&](int t) __attribute__((always_inline)) { return t == 0 ? 0 : max(1, t / P); };
  auto decode = [&](int k) __attribute__((always_inline)) {
    Item it;
    it.k = k;
    it.kvh = kvh_b;
    int n, nparts;
    bool bad;
    bool special;
    if constexpr (LIST) {
      it.seq = k;
      it.next = k - 1;  // a run is walked backwards, see below
      n = ld_const(a.context_lens, it.seq);
      nparts = seq_state<QR>(a, it.seq, n, &special, &bad);
      it.tok_begin = k == run_begin.seq ? run_begin.tok : 0;
      it.tok_end = k == run_end.seq ? run_end.tok : n;
    } else {
      const int r = k / Hkv;
      it.seq = r % S;
      const int part = r / S;
      it.next = seek(k + grid);
      n = ld_const(a.context_lens, it.seq);
      nparts = seq_parts(a, n, &bad);
      special = bad || n == 0;
      it.tok_begin = part * P;
      it.tok_end = min(n, it.tok_begin + P);
    }
    {
      const RunRows run = run_rows<QR>(a, it.seq, n);
      it.n = n;
      it.q0 = run.q0;
      it.nq = run.nq;
    }
    if (special) {
      it.tok_begin = 0;
      it.tok_end = 0;
    }
    const bool whole = special || (it.tok_begin == 0 && it.tok_end == n);
    it.part = slot_of(it.tok_begin);
    it.part_next = it.tok_end == n ? nparts : slot_of(it.tok_end);
    it.flags = (whole ? kDirect : 0) | (nparts > 1 ? kSplitSeq : 0) | (special ? kSpecial : 0) | (bad ? kBad : 0);
    it.new_id = 0;
    if constexpr (kTokenLate) {
      if (!special && it.tok_end == n) {
        it.flags |= kNew;
        it.new_id = ld_const(a.block_tables, static_cast<size_t>(it.seq) * a.max_blocks + (n - 1) / B);
      }
    }
    const int ngroups = (it.tok_end - it.tok_begin + GT - 1) / GT;
    it.nk = wave < ngroups ? (ngroups - wave + kWaves - 1) / kWaves : 0;
    it.npad = it.nk <= NBUF ? NBUF : (it.nk + NBUF - 1) & ~(NBUF - 1);
    return it;
  };

  // LIST: a run that starts inside a sequence and ends after it owns that
  // sequence's combination; a run that ends inside a sequence leaves record 1.
  bool owner = false;
  const bool split_ws = a.max_parts > 1;  // the workspace exists (otherwise no sequence is cut)
  // Hands record rec over once every wave's stores of it have completed (every thread calls it).
  auto publish = [&](int rec) __attribute__((always_inline)) {
    wait_stores();
    __syncthreads();
    if (tid == 0) {
      uint64_t* tg = a.ws_tag + 2 * static_cast<size_t>(rec);
      const uint64_t turn = __hip_atomic_load(tg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(tg + 1, tag_next(turn), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  if constexpr (LIST) {
    owner = split_ws && run_begin.tok > 0 && run_begin.seq < run_end.seq;
    if constexpr (!FUSED) {
      // the two-stage reduction finds the owners from these marks
      if (split_ws && tid == 0)
        *reinterpret_cast<int4*>(a.ws_hdr + 8 * static_cast<size_t>(blockIdx.x)) =
            make_int4(run_begin.seq, run_begin.tok, 0, owner ? 1 : 0);
    }
    if (k_first >= k_end && split_ws && run_end.tok > 0) {
      // No tokens, inside a sequence: an empty segment (m = -inf, l = 0, acc = 0) keeps the runs between the
      // sequence's first and its owner a contiguous chain of records.
      const int rec = 2 * static_cast<int>(blockIdx.x) + 1;
      const __amdgpu_buffer_rsrc_t r_acc = make_rsrc(a.ws_acc + static_cast<size_t>(rec) * NCOL * D, NCOL * D * 4);
      for (int i = tid; i < NCOL * D / 4; i += kThreads)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{0u, 0u, 0u, 0u}, r_acc, 16 * i, 0, kScopeDevice);
      const __amdgpu_buffer_rsrc_t r_m = make_rsrc(a.ws_m + static_cast<size_t>(rec) * NCOL, NCOL * 4);
      const __amdgpu_buffer_rsrc_t r_l = make_rsrc(a.ws_l + static_cast<size_t>(rec) * NCOL, NCOL * 4);
      const __amdgpu_buffer_rsrc_t r_hdr = make_rsrc(a.ws_hdr + 4 * static_cast<size_t>(rec), 16);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(-INFINITY), r_m, tid < NCOL ? 4 * tid : kNowhere, 0,
                                            kScopeDevice);
      __builtin_amdgcn_raw_buffer_store_b32(0u, r_l, tid < NCOL ? 4 * tid : kNowhere, 0, kScopeDevice);
      const u32x4_t hdr = {static_cast<uint32_t>(run_end.seq), static_cast<uint32_t>(run_end.tok),
                           static_cast<uint32_t>(run_end.tok), 0u};
      __builtin_amdgcn_raw_buffer_store_b128(hdr, r_hdr, tid == 0 ? 0 : kNowhere, 0, kScopeDevice);
      if constexpr (FUSED) publish(rec);
    }
  }
  if (k_first >= k_end) return;
  if constexpr (LIST && kTokenFirst) {
    // The decode step's new tokens.  The run holds the last token of every
    // sequence in [k_first, run_end.seq) (a sequence cut at run_end goes on in
    // the next run), and only this workgroup reads that token for its head, so
    // it writes it here, before its first load, through L2 (a partly written
    // line left dirty there stalls the read that follows); the waves wait for
    // the stores and meet at a barrier before the ring starts.
    using T = typename std::conditional<kBF16, uint16_t, uint32_t>::type;
    constexpr int E = 16 / static_cast<int>(sizeof(T));
    for (int s = k_first + wave; s < run_end.seq; s += kWaves) {
      const int n = ld_const(a.context_lens, s);
      bool bad;
      seq_parts(a, n, &bad);
      if (bad || n == 0) continue;
      const int id = ld_const(a.block_tables, static_cast<size_t>(s) * a.max_blocks + (n - 1) / B);
      if (static_cast<unsigned>(id) >= static_cast<unsigned>(a.num_blocks)) continue;
      const size_t row = (static_cast<size_t>(s) * Hkv + kvh_b) * D;
      const T* krow = static_cast<const T*>(a.k_new) + row;
      const T* vrow = static_cast<const T*>(a.v_new) + row;
      const uint4 kv = *reinterpret_cast<const uint4*>(krow + (lane < D / E ? lane : 0) * E);
      const T v0 = vrow[lane];
      const T v1 = D > 64 ? vrow[64 + lane] : T(0);
      store_token_rows<T, kStoreThrough>(const_cast<char*>(static_cast<const char*>(a.k_cache)),
                                         const_cast<char*>(static_cast<const char*>(a.v_cache)),
                                         static_cast<int64_t>(id) * Hkv + kvh_b, (n - 1) % B, B, D, lane, kv, v0, v1);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the stores have reached the cache hierarchy
    __syncthreads();
  }
  // LIST walks its run backwards, last sequence first: the run's last segment,
  // which a later run's owner combines, is computed and handed over first, and
  // an owner's own segment (the run's first) comes last, when the segments
  // before it have long been handed over.  Partition items go forwards.
  auto live = [&](int k) __attribute__((always_inline)) { return LIST ? k >= k_first : k < k_end; };
  Item cur = decode(LIST ? k_end - 1 : k_first);
  Item nxt = cur;
  if (live(cur.next)) nxt = decode(cur.next);
  nxt.k = cur.next;

  // ---- loads ---------------------------------------------------------------
  const char* kcache = static_cast<const char*>(a.k_cache);
  const char* vcache = static_cast<const char*>(a.v_cache);

  // Query rows of the item's KV head as the QK B operand: lane (m16, kq) holds
  // bytes [64 s + 16 kq, +16) of column m16, that is head m16 % G of query
  // m16 / G of the run (zeros for columns past the run's).
  auto load_query = [&](uint4 (&q)[NQ], const Item& it) __attribute__((always_inline)) {
    const char* base = static_cast<const char*>(a.q) +
                       (static_cast<size_t>(it.q0) * Hkv * G + static_cast<size_t>(it.kvh) * G) * R;
    // the run's rows from its first query's head 0 of this KV head on
    const int span = QR == 1 ? G * R : ((it.nq - 1) * Hkv * G + G) * R;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(base, it.nq > 0 ? span : 0);
    const int row = QR == 1 ? m16 : (m16 / G) * Hkv * G + m16 % G;
    const int off = m16 < it.nq * G ? row * R + 16 * kq : kNowhere;
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      q[s] = bload16<0>(rq, off, 64 * s);
    }
  };

  // Ring position p counted from the current item's start: positions past its
  // end belong to the next item (or to none after the last).  A position's
  // group gives the K and V resources of its tile (size 0 when the position
  // holds no group) and its first row in the tile (always 0 for bf16).
  struct Target {
    __amdgpu_buffer_rsrc_t kr, vr;
    int row0;
    bool poison;
  };
  struct Where {
    int seq, kvh, tok, valid;  // tok: the group's first token (or the item's first)
  };
  auto where = [&](int p, bool has_next) __attribute__((always_inline)) {
    const bool in_cur = p < cur.npad;
    const int i = in_cur ? p : p - cur.npad;
    const int nk = in_cur ? cur.nk : (has_next ? nxt.nk : 0);
    const int tb = in_cur ? cur.tok_begin : nxt.tok_begin;
    Where w;
    w.seq = in_cur ? cur.seq : nxt.seq;
    w.kvh = in_cur ? cur.kvh : nxt.kvh;
    w.valid = i < nk;
    w.tok = w.valid ? tb + GT * (wave + kWaves * i) : tb;
    return w;
  };
  auto table_entry = [&](const Where& w) __attribute__((always_inline)) {
    return ld_const(a.block_tables, static_cast<size_t>(w.seq) * a.max_blocks + w.tok / B);
  };
  auto make_target = [&](const Where& w, int id) __attribute__((always_inline)) {
    Target T;
    const bool oob = static_cast<unsigned>(id) >= static_cast<unsigned>(a.num_blocks);
    const size_t off = (static_cast<size_t>(oob ? 0 : id) * Hkv + w.kvh) * TILE;
    const int bytes = w.valid ? TILE : 0;
    T.kr = make_rsrc(kcache + off, bytes);
    T.vr = make_rsrc(vcache + off, bytes);
    T.row0 = kBF16 ? 0 : w.tok % B;
    T.poison = w.valid && oob;
    return T;
  };
  // K, QK A operand: lane (m16, kq) = token row m16 of QK tile t, key bytes
  // [64 s + 16 kq, +16), which is the 16-byte piece 4 s + kq.
  const int koff = (kq * B + m16) * 16;  // lane part of a key load
  auto load_keys = [&](uint4 (&kb)[NT][KS], const Target& T) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int s = 0; s < KS; ++s) kb[t][s] = bload16<kLoadNT>(T.kr, koff, (4 * s * B + T.row0 + 16 * t) * 16);
  };
  // V, PV A operand: lane (m16, kq) = head-dimension row 16 dt + m16 and the
  // tokens its PV form needs (bf16 B = 16: 4 kq .. 4 kq + 3; bf16 B = 32:
  // 8 kq .. 8 kq + 7; fp32: 4 kq .. 4 kq + 3 of the group).
  const int voff = (m16 * B + (kBF16 && B == 32 ? 8 : 4) * kq) * Gm::kItem;  // lane part of a value load
  auto load_values = [&](uint32_t (&vb)[NDT][VW], const Target& T) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int soff = (16 * dt * B + T.row0) * Gm::kItem;
      if constexpr (VW == 2) {
        const uint2 v = bload8<kLoadNT>(T.vr, voff, soff);
        vb[dt][0] = v.x;
        vb[dt][1] = v.y;
      } else {
        const uint4 v = bload16<kLoadNT>(T.vr, voff, soff);
        vb[dt][0] = v.x;
        vb[dt][1] = v.y;
        vb[dt][2] = v.z;
        vb[dt][3] = v.w;
      }
    }
  };

  // The next item's query is prefetched into registers when it is small (up
  // to 16 VGPRs); otherwise it is loaded when the item starts.
  constexpr bool kPrefetchQ = NQ <= 4;
  uint4 q_cur[NQ], q_nxt[kPrefetchQ ? NQ : 1];
  load_query(q_cur, cur);
  if constexpr (kPrefetchQ) load_query(q_nxt, live(nxt.k) ? nxt : cur);

  // Late token: the next item's key and value rows, dword j of a row in lane
  // j % 64 (register j / 64), loaded one item ahead like the query.  When an
  // item starts, every wave copies them into the item's entry of sh.knew and
  // sh.vnew (the same bytes from each wave, so a wave reads back its own
  // writes with no barrier; two entries alternate, and the merge barrier
  // between items keeps a wave from overwriting an entry another still
  // reads); the load is a whole item old by then, so the wait for it is exact.
  constexpr int NW = kTokenLate ? (R / 4 + kWave - 1) / kWave : 1;
  uint32_t kn_nxt[NW], vn_nxt[NW];
  int ord = 0;  // the current item's position in this workgroup's walk
  auto park_new = [&](int e) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      if (lane + kWave * j < R / 4) {
        sh.knew[e][lane + kWave * j] = kn_nxt[j];
        sh.vnew[e][lane + kWave * j] = vn_nxt[j];
      }
    }
  };
  auto load_new = [&](uint32_t (&kn)[NW], uint32_t (&vn)[NW], const Item& it, bool use)
                      __attribute__((always_inline)) {
    const bool has = use && (it.flags & kNew);
    const size_t row = (static_cast<size_t>(it.seq) * Hkv + it.kvh) * R;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const char*>(a.k_new) + row, has ? R : 0);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const char*>(a.v_new) + row, has ? R : 0);
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      kn[j] = __builtin_amdgcn_raw_buffer_load_b32(rk, 4 * (lane + kWave * j), 0, 0);
      vn[j] = __builtin_amdgcn_raw_buffer_load_b32(rv, 4 * (lane + kWave * j), 0, 0);
    }
  };
  if constexpr (kTokenLate) load_new(kn_nxt, vn_nxt, cur, true);  // parked once the ring's first loads are out
  // Token r of a group in the ring slot's operand registers: the key row in
  // the lanes of token row r % 16 of QK tile r / 16 (the 16 bytes at 64 st +
  // 16 kq of the row), the value of dim 16 dt + m16 in the lanes whose tokens
  // include r.  The rows go through the wave's own LDS copy (written and read
  // by the same wave, in order), so each lane reads its operand bytes at a
  // constant offset from one address.
  auto patch_keys = [&](uint4 (&kbs)[NT][KS], int r) __attribute__((always_inline)) {
    if (m16 == (r & 15)) {
      const char* row = reinterpret_cast<const char*>(sh.knew[ord & 1]) + 16 * kq;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (t == (r >> 4))
#pragma unroll
          for (int st = 0; st < KS; ++st) kbs[t][st] = *reinterpret_cast<const uint4*>(row + 64 * st);
    }
  };
  auto patch_values = [&](uint32_t (&vbs)[NDT][VW], int r) __attribute__((always_inline)) {
    constexpr int TPL = (kBF16 ? 2 : 1) * VW;  // tokens per lane and d-tile
    const int e = r % TPL;
    if (kq == r / TPL) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        if constexpr (kBF16) {
          const uint32_t v16 = reinterpret_cast<const uint16_t*>(sh.vnew[ord & 1])[16 * dt + m16];
#pragma unroll
          for (int w = 0; w < VW; ++w)
            if (w == (e >> 1))
              vbs[dt][w] = (e & 1) ? ((vbs[dt][w] & 0x0000ffffu) | (v16 << 16)) : ((vbs[dt][w] & 0xffff0000u) | v16);
        } else {
          const uint32_t x = sh.vnew[ord & 1][16 * dt + m16];
#pragma unroll
          for (int w = 0; w < VW; ++w)
            if (w == e) vbs[dt][w] = x;
        }
      }
    }
  };

  uint4 kb[NBUF][NT][KS];
  uint32_t vb[NBUF][NDT][VW];
  bool pois_cur = false, pois_nxt = false;
  if constexpr (kTokenLate) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this workgroup's token stores are done
  // The ring starts with positions 0 .. NBUF-1 of the first item.
#pragma unroll
  for (int s = 0; s < NBUF; ++s) {
    const Where w = where(s, false);
    const Target T = make_target(w, table_entry(w));
    pois_cur |= T.poison;
    load_keys(kb[s], T);
    load_values(vb[s], T);
  }
  // The block id of the next refill target is fetched one step ahead.
  int pend_id = table_entry(where(NBUF, live(nxt.k)));
  if constexpr (kTokenLate) {
    park_new(0);
    load_new(kn_nxt, vn_nxt, nxt, live(nxt.k));
  }

  const float c = a.c;
  int parity = 0;  // LDS merge buffer of the current item
  for (;;) {
    f32x4_t acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;
    const bool has_next = live(nxt.k);

    // npad >= NBUF: a loop that visibly runs at least once lets the compiler
    // count the ring's refills between the next query's prefetch and its use
    // at the item change (a zero-trip path would make it wait there for all
    // but the merge's stores, draining the ring at every item boundary).
    int i0 = 0;
    do {
#pragma unroll
      for (int s = 0; s < NBUF; ++s) {
        const int i = i0 + s;
        const bool valid = i < cur.nk;
        const int t_first = cur.tok_begin + GT * (wave + kWaves * i);
        // late token: the group holds it (then it is a valid group of the item)
        const int r_new = cur.n - 1 - t_first;
        const bool patch = kTokenLate && (cur.flags & kNew) && static_cast<unsigned>(r_new) < static_cast<unsigned>(GT);
        if constexpr (kTokenLate) {
          if (patch) patch_keys(kb[s], r_new);
        }

        // Refill target of this slot: ring position i + NBUF.
        const int ti = i + NBUF;
        const Target T = make_target(where(ti, has_next), pend_id);
        pend_id = table_entry(where(ti + 1, has_next));
        if (ti < cur.npad)
          pois_cur |= T.poison;
        else
          pois_nxt |= T.poison;

        // QK^T on the matrix cores: sc[t] rows = tokens 16 t + 4 kq + r, column = head m16.
        f32x4_t sc[NT];
        if (valid) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            sc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < KS; ++st) {
              const uint4 kv = kb[s][t][st], qv = q_cur[st];
              if constexpr (kBF16) {
                sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv), as_bf16x8(qv), sc[t], 0, 0, 0);
              } else {
                sc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.x), __uint_as_float(qv.x), sc[t], 0, 0, 0);
                sc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.y), __uint_as_float(qv.y), sc[t], 0, 0, 0);
                sc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.z), __uint_as_float(qv.z), sc[t], 0, 0, 0);
                sc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kv.w), __uint_as_float(qv.w), sc[t], 0, 0, 0);
              }
            }
          }
        }
        load_keys(kb[s], T);  // the slot's keys are consumed: refill
        __builtin_amdgcn_sched_barrier(0);

        if constexpr (kTokenLate) {
          if (patch) patch_values(vb[s], r_new);
        }
        if (valid) {
          // Scaled logits u = c (q . k).
#pragma unroll
          for (int t = 0; t < NT; ++t) sc[t] *= c;
          if (t_first + GT > cur.tok_end) {
            // Tokens past the end: logit -inf and value 0 (the cache may hold anything there).
            const int rel = cur.tok_end - t_first;  // valid tokens of the group
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (16 * t + 4 * kq + r >= rel) sc[t][r] = -INFINITY;
            if constexpr (kBF16) {
              const int first = (VW == 2 ? 4 : 8) * kq;
              uint32_t mask[VW];
#pragma unroll
              for (int w = 0; w < VW; ++w)
                mask[w] = (first + 2 * w < rel ? 0x0000ffffu : 0u) | (first + 2 * w + 1 < rel ? 0xffff0000u : 0u);
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int w = 0; w < VW; ++w) vb[s][dt][w] &= mask[w];
            } else {
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int w = 0; w < VW; ++w)
                  if (4 * kq + w >= rel) vb[s][dt][w] = 0u;
            }
          }
          if constexpr (QR > 1) {
            // Runs: query m16 / G, at position n - nq + m16 / G, sees the tokens up to
            // its position; only the run's last nq - 1 tokens are hidden from some.
            const int first_hidden = cur.n - cur.nq + 1;  // the first token hidden from query 0
            if (t_first + GT > first_hidden) {
              const int lim = first_hidden - 1 + m16 / G - t_first;  // the column's last visible token, in the group
#pragma unroll
              for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (16 * t + 4 * kq + r > lim) sc[t][r] = -INFINITY;
            }
          }
          // Online softmax, per column (lane column m16).
          float gm = -INFINITY;
#pragma unroll
          for (int t = 0; t < NT; ++t) gm = fmaxf(gm, fmaxf(fmaxf(sc[t][0], sc[t][1]), fmaxf(sc[t][2], sc[t][3])));
          gm = max_xor32(max_xor16(gm));
          const float m_new = fmaxf(m_run, gm);
          if (__ballot(m_new > m_run)) {
            const float alpha = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
            l_run *= alpha;
            m_run = m_new;
          }
          // (runs: a column that has seen no token yet, its tokens all after its
          // query, keeps m = -inf and gets weights exp2(-inf - 0) = 0)
          const float m_use = (QR > 1 && m_run == -INFINITY) ? 0.0f : m_run;
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              sc[t][r] = __builtin_amdgcn_exp2f(sc[t][r] - m_use);
              l_run += sc[t][r];
            }

          // PV on the matrix cores: acc[dt] rows = dims 16 dt + 4 kq + r, column = head m16.
          if constexpr (!kBF16) {
            // fp32: QK output register r of lane (kq, head) is the probability of token
            // 4 kq + r, exactly the B operand of k-step r.
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vb[s][dt][r]), sc[0][r], acc[dt], 0, 0, 0);
          } else {
            typedef float f2_t __attribute__((ext_vector_type(2)));
            typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
            auto hi_bits = [](float p) __attribute__((always_inline)) { return __float_as_uint(p) & 0xffff0000u; };
            auto pack_hi = [&](float x, float y) __attribute__((always_inline)) {
              return (hi_bits(x) >> 16) | hi_bits(y);
            };
            auto pack_lo = [&](float x, float y) __attribute__((always_inline)) {
              const f2_t l = {x - __uint_as_float(hi_bits(x)), y - __uint_as_float(hi_bits(y))};
              return __builtin_bit_cast(uint32_t, __builtin_convertvector(l, b2_t));
            };
            if constexpr (VW == 2) {
              // B = 16: 16x16x16 steps, k-slice kq = tokens 4 kq + r (r < 4): the QK
              // output registers of the lane, once as hi and once as lo.
              typedef short s4_t __attribute__((ext_vector_type(4)));
              const u32x2_t ph = {pack_hi(sc[0][0], sc[0][1]), pack_hi(sc[0][2], sc[0][3])};
              const u32x2_t pl = {pack_lo(sc[0][0], sc[0][1]), pack_lo(sc[0][2], sc[0][3])};
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt) {
                const u32x2_t av = {vb[s][dt][0], vb[s][dt][1]};
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, av),
                                                                    __builtin_bit_cast(s4_t, ph), acc[dt], 0, 0, 0);
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, av),
                                                                    __builtin_bit_cast(s4_t, pl), acc[dt], 0, 0, 0);
              }
            } else {
              // B = 32: k-slice kq = tokens 8 kq .. 8 kq + 7.  Two lane swaps move the QK
              // rows (tokens 4 kq' + r of tiles 0 and 1) into that order:
              // x[r] = token 8 kq + r, y[r] = token 8 kq + 4 + r.
              float x[4], y[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const auto s32 =
                    __builtin_amdgcn_permlane32_swap(__float_as_uint(sc[0][r]), __float_as_uint(sc[1][r]), false, false);
                const auto s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
                x[r] = __uint_as_float(s16[0]);
                y[r] = __uint_as_float(s16[1]);
              }
              const u32x4_t bh = {pack_hi(x[0], x[1]), pack_hi(x[2], x[3]), pack_hi(y[0], y[1]), pack_hi(y[2], y[3])};
              const u32x4_t bl = {pack_lo(x[0], x[1]), pack_lo(x[2], x[3]), pack_lo(y[0], y[1]), pack_lo(y[2], y[3])};
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt) {
                const u32x4_t av = {vb[s][dt][0], vb[s][dt][1], vb[s][dt][2], vb[s][dt][3]};
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                                  __builtin_bit_cast(bf16x8_t, bh), acc[dt], 0, 0, 0);
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                                  __builtin_bit_cast(bf16x8_t, bl), acc[dt], 0, 0, 0);
              }
            }
          }
        }
        load_values(vb[s], T);  // the slot's values are consumed: refill
        __builtin_amdgcn_sched_barrier(0);
      }
      i0 += NBUF;
    } while (i0 < cur.npad);

    // ---- merge the waves' partial results ------------------------------------
    // Each wave parks (acc, max, sum) in this item's LDS buffer; after one
    // barrier every thread combines four consecutive dims of one head.  The
    // buffers alternate between items, so the next item's barrier is what
    // orders the reuse of this one.
    const float l_tot = sum_xor32(sum_xor16(l_run));  // over the four token rows of each head
    auto& mb = sh.mb[NCOL > 8 ? 0 : parity];
    // columns in use: decode, the G heads; runs, those of the run's queries
    const int ncol = QR == 1 ? G : cur.nq * G;
    if (m16 < ncol) {
      float* reg = &mb.region[wave][m16][0];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        f32x4_t v = acc[dt];
        if (pois_cur) v = f32x4_t{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        *reinterpret_cast<f32x4_t*>(reg + 16 * dt + 4 * kq) = v;
      }
      if (kq == 0) {
        mb.wm[wave][m16] = m_run;
        mb.wl[wave][m16] = pois_cur ? __builtin_nanf("") : l_tot;
      }
    }
    __syncthreads();
    {
      // Every thread issues the same stores on every path (buffer stores; the
      // ones that must not land use a size-0 resource or an offset past the
      // resource and are dropped by the hardware): stores count in the same
      // wait counter as the ring's loads, and a store behind a branch would
      // make the compiler wait for all earlier loads after the merge.
      // A segment covering its whole sequence writes the output rows (and, for
      // a sequence of several partitions, marks partition 0 done for the
      // reduction); any other segment writes its partials at its first
      // partition, with its length.
      const bool direct = cur.flags & kDirect;
      // the item's output rows: decode, the G heads of its KV head; runs, those
      // of each query of the run, Hq rows apart
      const size_t head0 = static_cast<size_t>(cur.q0) * Hkv * G + static_cast<size_t>(cur.kvh) * G;
      const int out_rows = QR == 1 ? G : (cur.nq > 0 ? (cur.nq - 1) * Hkv * G + G : 0);
      // The partials' slot: LIST, record 0 of an owner's first item or record 1
      // of a run's last item; otherwise the segment's partition slot.
      const int rec = 2 * static_cast<int>(blockIdx.x) + ((owner && cur.k == k_first) ? 0 : 1);
      const size_t prow =
          LIST ? static_cast<size_t>(rec) : (static_cast<size_t>(cur.seq) * Hkv + cur.kvh) * a.max_parts + cur.part;
      const bool split = split_ws;
      const __amdgpu_buffer_rsrc_t r_out = make_rsrc(a.out + head0 * D, direct ? out_rows * D * 4 : 0);
      const __amdgpu_buffer_rsrc_t r_acc = make_rsrc(split ? a.ws_acc + prow * NCOL * D : a.out, direct ? 0 : NCOL * D * 4);
      const __amdgpu_buffer_rsrc_t r_m = make_rsrc(split ? a.ws_m + prow * NCOL : a.out, direct ? 0 : NCOL * 4);
      const __amdgpu_buffer_rsrc_t r_l = make_rsrc(split ? a.ws_l + prow * NCOL : a.out, direct ? 0 : NCOL * 4);
      if constexpr (LIST) {
        const __amdgpu_buffer_rsrc_t r_hdr =
            make_rsrc(split ? static_cast<const void*>(a.ws_hdr + 4 * prow) : static_cast<const void*>(a.out),
                      direct ? 0 : 16);
        const u32x4_t hdr = {static_cast<uint32_t>(cur.seq), static_cast<uint32_t>(cur.tok_begin),
                             static_cast<uint32_t>(cur.tok_end), (rec & 1) ? 0u : 1u};
        __builtin_amdgcn_raw_buffer_store_b128(hdr, r_hdr, tid == 0 ? 0 : kNowhere, 0, kScopeDevice);
      } else {
        const bool seg_store = split && (!direct || (cur.flags & kSplitSeq));
        const __amdgpu_buffer_rsrc_t r_seg = make_rsrc(
            split ? static_cast<const void*>(a.ws_seg + prow) : static_cast<const void*>(a.out), seg_store ? 4 : 0);
        __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(direct ? -1 : cur.part_next), r_seg,
                                              tid == 0 ? 0 : kNowhere, 0, 0);
      }
      constexpr int NC = D / 4;  // float4 chunks of one column's row
      constexpr int ITERS = (NCOL * NC + kThreads - 1) / kThreads;
      const float fill = (cur.flags & kBad) ? __builtin_nanf("") : 0.0f;
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int cidx = tid + it * kThreads;
        const bool live = cidx < ncol * NC;  // columns past those in use store nothing
        const int h = live ? cidx / NC : 0, d4 = live ? (cidx % NC) * 4 : 0;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mb.wm[w][h]);
        f32x4_t sa = {0.0f, 0.0f, 0.0f, 0.0f};
        float sl = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          // 0 for a wave that saw no token (runs: also when no wave saw one, M = -inf)
          const float wt = (QR > 1 && M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mb.wm[w][h] - M);
          sa += wt * *reinterpret_cast<const f32x4_t*>(&mb.region[w][h][d4]);
          sl = fmaf(wt, mb.wl[w][h], sl);
        }
        const f32x4_t o = (cur.flags & kSpecial) ? f32x4_t{fill, fill, fill, fill} : sa / sl;
        const int voff = live ? (h * D + d4) * 4 : kNowhere;
        const int soff = live && d4 == 0 ? h * 4 : kNowhere;
        const int ooff = QR == 1 ? voff : live && h / G < cur.nq ? (((h / G) * Hkv * G + h % G) * D + d4) * 4 : kNowhere;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o), r_out, ooff, 0, 0);
        // item-list records are read by another workgroup, maybe on another XCD: device scope
        constexpr int kRecAux = LIST ? kScopeDevice : 0;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, sa), r_acc, voff, 0, kRecAux | kLoadNT);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(M), r_m, soff, 0, kRecAux);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sl), r_l, soff, 0, kRecAux);
      }
      // FUSED: a run's last segment that a later run's owner combines is handed over.
      if constexpr (LIST && FUSED)
        if (!direct && (rec & 1)) publish(rec);
    }
    if constexpr (NCOL > 8) __syncthreads();  // one merge buffer: every thread has read it before the next item writes
    parity ^= 1;

    if (!has_next) break;
    // Advance: the ring already holds the next item's first NBUF positions.
    cur = nxt;
    pois_cur = pois_nxt;
    pois_nxt = false;
    if constexpr (kPrefetchQ) {
#pragma unroll
      for (int s = 0; s < NQ; ++s) q_cur[s] = q_nxt[s];
    } else {
      load_query(q_cur, cur);
    }
    {
      const int kn = cur.next;
      nxt = cur;
      if (live(kn)) nxt = decode(kn);
      nxt.k = kn;
    }
    if constexpr (kPrefetchQ) load_query(q_nxt, live(nxt.k) ? nxt : cur);
    if constexpr (kTokenLate) {
      ++ord;
      park_new(ord & 1);
      load_new(kn_nxt, vn_nxt, nxt, live(nxt.k));
    }
    // Ring position NBUF of the new item: when the item has only NBUF
    // positions it is the following item's first group, which the old item's
    // look-ahead could not know.
    pend_id = table_entry(where(NBUF, live(nxt.k)));
  }

  if constexpr (LIST && FUSED) {
    if (owner) {
      // Combine the owned sequence: its segments lie in record 1 of the runs
      // that start inside it, going down from this one, and of the run before
      // them (which holds its token 0), and in this run's record 0.
      const int seq = run_begin.seq;
      wait_stores();  // this run's record 0 is complete
      __syncthreads();
      if (wave == 0) {
        // first: the highest run below this one that does not start inside the
        // sequence (it holds token 0); 64 runs tested at once, one per lane.
        int first = -1;
        for (int top = lane_b - 1; first < 0; top -= kWave) {
          const int L = top - lane;
          bool inside = false;
          if (L >= 0) {
            const Cut c = cut_at_lane((static_cast<uint64_t>(L) * C + lanes - 1) / lanes);
            inside = c.seq == seq && c.tok > 0;
          }
          const uint64_t outside = __ballot(!inside);  // bit i: run top - i; run 0 never starts inside
          if (outside) first = top - (__ffsll(static_cast<unsigned long long>(outside)) - 1);
        }
        // Take the records of runs first .. lane_b - 1 over, 64 at a time, lane i
        // waiting for run first + i (also after a time-out, so that a late write
        // leaves flag == turn); their headers must tile the sequence's tokens
        // [0, this run's first token).
        bool ok = true;
        int carry = 0;  // where the next record must start
        for (int L0 = first; L0 < lane_b; L0 += kWave) {
          const int L = L0 + lane, count = min(kWave, lane_b - L0);
          int4 h = make_int4(seq, 0, 0, 0);
          bool good = true;
          if (L < lane_b) {
            const int rec = 2 * (L * Hkv + kvh_b) + 1;
            uint64_t* tg = a.ws_tag + 2 * static_cast<size_t>(rec);
            const uint64_t want = tag_next(__hip_atomic_load(tg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            int polls = 0;
            while (__hip_atomic_load(tg + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != want && polls < kMaxPolls) {
              __builtin_amdgcn_s_sleep(1);
              ++polls;
            }
            __hip_atomic_store(tg, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            h = load_dev_i4(make_rsrc(a.ws_hdr, 2 * static_cast<int>(gridDim.x) * 16), 16 * rec);
            good = polls < kMaxPolls && h.x == seq && h.z >= h.y;
          }
          const int before = __shfl(h.z, lane > 0 ? lane - 1 : 0);
          if (L < lane_b) good = good && h.y == (lane == 0 ? carry : before);
          ok = ok && __ballot(!good) == 0;
          carry = __shfl(h.z, count - 1);
        }
        if (lane == 0) {
          sh.chain_first = first;
          sh.chain_ok = ok && carry == run_begin.tok;
        }
      }
      __syncthreads();
      combine_runs<G, QR, D>(a, seq, kvh_b, sh.chain_first, lane_b, sh.chain_ok != 0, tid);
    }
  }
}

// ---------------------------------------------------------------------------
// The two-stage path's combination (item list): one workgroup per workgroup
// of the partition pass, same grid.  An owner (marked in its record 0) walks
// down the records 1 of the runs before it while they start inside its
// sequence, then combines them as the fused kernel does.
// ---------------------------------------------------------------------------
template <int G, int D>
__global__ __launch_bounds__(kThreads) void list_reduce_kernel(AttnArgs a) {
  const int b = blockIdx.x, Hkv = a.num_kv_heads, kvh = b % Hkv, lane_b = b / Hkv;
  const int4 mark = *reinterpret_cast<const int4*>(a.ws_hdr + 8 * static_cast<size_t>(b));
  if (mark.w != 1) return;
  __shared__ int first_sh, ok_sh;
  if (threadIdx.x == 0) {
    // The walk moves down and stops at run 0, so it ends whatever the workspace holds.
    int first = lane_b - 1, expect = mark.y;
    bool ok = true;
    for (; first >= 0; --first) {
      const int4 h = *reinterpret_cast<const int4*>(a.ws_hdr + 4 * (2 * static_cast<size_t>(first * Hkv + kvh) + 1));
      if (h.x != mark.x || h.z != expect || h.y > h.z) {
        ok = false;
        break;
      }
      if (h.y == 0) break;
      expect = h.y;
    }
    first_sh = first < 0 ? 0 : first;
    ok_sh = ok && first >= 0;
  }
  __syncthreads();
  combine_runs<G, 1, D>(a, mark.x, kvh, first_sh, lane_b, ok_sh != 0, threadIdx.x);
}

// ---------------------------------------------------------------------------
// Log-sum-exp combination of the partitions of one (sequence, query head):
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void lse_reduce_kernel(AttnArgs a, int num_q_heads) {
  // One workgroup per (sequence, KV head); wave w takes the query heads
  // g = w, w + 4, ... of the group.
  const int seq = blockIdx.x / a.num_kv_heads, kvh = blockIdx.x % a.num_kv_heads;
  bool bad;
  const int nparts = seq_parts(a, ld_const(a.context_lens, seq), &bad);
  if (nparts <= 1) return;  // written directly by the attention kernel
  // Partials of the segment in slot p: entry ((seq * H_kv + kvh) * max_parts + p) * G + g; ws_seg at
  // (seq * H_kv + kvh) * max_parts + p holds the slot of the sequence's next segment.
  const size_t srow = (static_cast<size_t>(seq) * a.num_kv_heads + kvh) * a.max_parts;
  const int32_t* seg = a.ws_seg + srow;
  if (seg[0] < 0) return;  // the sequence was written whole
  // The walk always moves forward, so it ends whatever the workspace holds.
  auto next = [&](int p) { return max(p + 1, seg[p]); };
  const int G = num_q_heads / a.num_kv_heads;
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int PER = D / kWave;
  for (int g = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); g < G; g += kWaves) {
    float M = -INFINITY;
    for (int p = 0; p < nparts; p = next(p)) M = fmaxf(M, a.ws_m[(srow + p) * G + g]);
    float o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.0f;
    float L = 0.0f;
    for (int p = 0; p < nparts; p = next(p)) {
      const size_t e_p = (srow + p) * G + g;
      const float w = __builtin_amdgcn_exp2f(a.ws_m[e_p] - M);
      L = fmaf(w, a.ws_l[e_p], L);
      const float* ap = a.ws_acc + e_p * D;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = fmaf(w, ap[lane + e * kWave], o[e]);
    }
    float* out = a.out + (static_cast<size_t>(seq) * num_q_heads + static_cast<size_t>(kvh) * G + g) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) out[lane + e * kWave] = o[e] / L;
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
// The item list needs its LDS prefix sums to fit, and the summed costs
// (groups of at least 16 tokens plus the per-partition charge) to fit 32 bits.
bool use_list(int32_t num_seqs, int32_t max_context_len, int32_t max_parts) {
  const uint64_t seq_cost_bound =
      static_cast<uint64_t>(max_context_len) / 16 + 1 + static_cast<uint64_t>(kItemCharge) * max_parts;
  return num_seqs <= kMaxListedSeqs && static_cast<uint64_t>(num_seqs) * seq_cost_bound < (1ull << 32);
}

// The persistent grid never exceeds this many workgroups (an MI355X holds 512
// to 768 of this kernel at once); it bounds the item list's records.
constexpr int kMaxGrid = 2048;

struct Plan {
  int32_t P;          // effective partition size
  int32_t max_parts;  // partitions of the longest sequence
  bool list;          // item list (records per workgroup), else a slot per partition
  int32_t grid_cap;   // the largest grid a launch uses (a multiple of H_kv)
  size_t off_m, off_l, off_seg, off_hdr, off_tag, bytes;
};

// cols: matrix-core columns per item (decode G; runs of queries 16).
Plan make_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
               int32_t max_context_len, int32_t partition_size, int32_t cols = 0) {
  Plan p{};
  const int64_t ctx = max_context_len > 0 ? max_context_len : 1;
  p.P = partition_size > 0 ? partition_size : static_cast<int32_t>(ceil_div64(ctx, block_size) * block_size);
  p.max_parts = static_cast<int32_t>(ceil_div64(ctx, p.P));
  p.list = use_list(num_seqs, max_context_len, p.max_parts);
  const int64_t items = static_cast<int64_t>(p.max_parts) * num_seqs * num_kv_heads;
  const int64_t want = items < kMaxGrid ? items : kMaxGrid;
  p.grid_cap = static_cast<int32_t>(want >= num_kv_heads ? want / num_kv_heads * num_kv_heads : num_kv_heads);
  if (p.max_parts <= 1 || num_seqs <= 0) return p;
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t G = static_cast<size_t>(cols > 0 ? cols : num_q_heads / num_kv_heads);
  if (p.list) {
    const size_t recs = 2 * static_cast<size_t>(p.grid_cap);
    p.off_m = up(recs * G * head_dim * sizeof(float));
    p.off_l = p.off_m + up(recs * G * sizeof(float));
    p.off_hdr = p.off_l + up(recs * G * sizeof(float));
    p.off_tag = p.off_hdr + up(recs * 4 * sizeof(int32_t));
    p.bytes = p.off_tag + up(recs * 2 * sizeof(uint64_t));
  } else {
    const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * p.max_parts;
    p.off_m = up(rows * head_dim * sizeof(float));
    p.off_l = p.off_m + up(rows * sizeof(float));
    p.off_seg = p.off_l + up(rows * sizeof(float));
    p.bytes = p.off_seg + up(rows * sizeof(int32_t));
  }
  return p;
}

// Workgroups of a kernel that fit the whole device at once, cached per device
// and per instantiation (each kernel type gets its own static cache).
template <class K, K kernel>
int resident_workgroups() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess) return 0;
    cache[dev] = cus * (per_cu > 0 ? per_cu : 1);
  }
  return cache[dev];
}

// The persistent grid: as many workgroups as fit at once, at most one per
// item and at most kMaxGrid, rounded to a multiple of H_kv: with the KV head
// varying fastest in the item order, workgroup b always serves head b % H_kv
// and the workgroups of all heads of one partition run side by side, reading
// adjacent tiles of the same blocks (and, for shared prefixes, the same
// blocks).
template <class DT, int D, int G, int B, bool LIST, bool WRITE, bool FUSED, int QR = 1>
int grid_for(const AttnArgs& a) {
  using K = void (*)(AttnArgs);
  constexpr K kernel = paged_decode_kernel<DT, D, G, B, LIST, WRITE, FUSED, QR>;
  const int fill = resident_workgroups<K, kernel>();
  if (fill <= 0) return 0;
  int want = a.total_items < fill ? a.total_items : fill;
  if (want > kMaxGrid) want = kMaxGrid;
  return want >= a.num_kv_heads ? want / a.num_kv_heads * a.num_kv_heads : a.num_kv_heads;
}

template <class DT, int D, int G, int B, bool LIST, bool WRITE, bool FUSED, int QR = 1>
hipError_t launch_kernel(const AttnArgs& a, hipStream_t stream) {
  const int grid = grid_for<DT, D, G, B, LIST, WRITE, FUSED, QR>(a);
  if (grid <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((paged_decode_kernel<DT, D, G, B, LIST, WRITE, FUSED, QR>), dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// What one launch does.  kPass: the partition pass alone (the two-stage path,
// or partition items); kFused: the item list with the combination inside;
// kWriteFused: the same, storing each sequence's new token first;
// kListReduce: the two-stage path's combination for the item list.
enum class Op { kPass, kFused, kWriteFused, kListReduce };

template <class DT, int D, int G, int B>
hipError_t launch_op_b(const AttnArgs& a, bool list, Op op, hipStream_t stream) {
  if (!list) return launch_kernel<DT, D, G, B, false, false, false>(a, stream);
  switch (op) {
    case Op::kPass: return launch_kernel<DT, D, G, B, true, false, false>(a, stream);
    case Op::kFused: return launch_kernel<DT, D, G, B, true, false, true>(a, stream);
    case Op::kWriteFused: return launch_kernel<DT, D, G, B, true, true, true>(a, stream);
    case Op::kListReduce: {
      // the same grid as the two-stage path's partition pass, whose records it reads
      const int grid = grid_for<DT, D, G, B, true, false, false>(a);
      if (grid <= 0) return hipErrorInvalidValue;
      hipLaunchKernelGGL((list_reduce_kernel<G, D>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream, a);
      return hipGetLastError();
    }
  }
  return hipErrorInvalidValue;
}

template <class DT, int D, int G>
hipError_t launch_op_g(const AttnArgs& a, bool list, Op op, hipStream_t stream) {
  return a.block_size == 16 ? launch_op_b<DT, D, G, 16>(a, list, op, stream)
                            : launch_op_b<DT, D, G, 32>(a, list, op, stream);
}

template <class DT, int D>
hipError_t launch_op_d(const AttnArgs& a, int G, bool list, Op op, hipStream_t stream) {
  switch (G) {
    case 1: return launch_op_g<DT, D, 1>(a, list, op, stream);
    case 2: return launch_op_g<DT, D, 2>(a, list, op, stream);
    case 4: return launch_op_g<DT, D, 4>(a, list, op, stream);
    case 8: return launch_op_g<DT, D, 8>(a, list, op, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class DT>
hipError_t launch_op(const AttnArgs& a, int D, int G, bool list, Op op, hipStream_t stream) {
  if (D == 64) return launch_op_d<DT, 64>(a, G, list, op, stream);
  if (D == 128) return launch_op_d<DT, 128>(a, G, list, op, stream);
  return hipErrorInvalidValue;
}

// Runs of queries: the listed, fused kernel with QR queries per item.
template <class DT, int D, int G, int QR>
hipError_t launch_runs_q(const AttnArgs& a, hipStream_t stream) {
  return a.block_size == 16 ? launch_kernel<DT, D, G, 16, true, false, true, QR>(a, stream)
                            : launch_kernel<DT, D, G, 32, true, false, true, QR>(a, stream);
}
// Queries per item: 16 / G (the whole column tile), or 4 for runs of at most
// 4 queries at G <= 2 (4 or 8 columns: smaller merge and partial records).
template <class DT, int D, int G>
hipError_t launch_runs_g(const AttnArgs& a, hipStream_t stream) {
  if constexpr (G <= 2) {
    if (a.max_query_len <= 4) return launch_runs_q<DT, D, G, 4>(a, stream);
  }
  return launch_runs_q<DT, D, G, 16 / G>(a, stream);
}
template <class DT, int D>
hipError_t launch_runs_d(const AttnArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_runs_g<DT, D, 1>(a, stream);
    case 2: return launch_runs_g<DT, D, 2>(a, stream);
    case 4: return launch_runs_g<DT, D, 4>(a, stream);
    case 8: return launch_runs_g<DT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}
template <class DT>
hipError_t launch_runs(const AttnArgs& a, int D, int G, hipStream_t stream) {
  if (D == 64) return launch_runs_d<DT, 64>(a, G, stream);
  if (D == 128) return launch_runs_d<DT, 128>(a, G, stream);
  return hipErrorInvalidValue;
}

enum : int { kStagePartitions = 1, kStageReduce = 2 };

pkv_status attention_stages(int stages, const void* k_new, const void* v_new, float* out, const void* q,
                            const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, int32_t max_blocks, int32_t max_context_len, float scale,
                            int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t kv_dtype,
                            hipStream_t stream) {
  if (item_size(kv_dtype) == 0) return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks <= 0 ||
      max_context_len < 0 || partition_size < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads) return PKV_ERR_INVALID_ARG;
  const int G = num_q_heads / num_kv_heads;
  if ((G != 1 && G != 2 && G != 4 && G != 8) || (head_dim != 64 && head_dim != 128) ||
      (block_size != 16 && block_size != 32))
    return PKV_ERR_UNSUPPORTED;
  if (partition_size % block_size) return PKV_ERR_INVALID_ARG;
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID_ARG;
  if ((k_new != nullptr) != (v_new != nullptr)) return PKV_ERR_INVALID_ARG;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return PKV_ERR_INVALID_ARG;

  const Plan plan =
      make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len, partition_size);
  const int64_t items = static_cast<int64_t>(plan.max_parts) * num_seqs * num_kv_heads;
  if (items > INT32_MAX / 2) return PKV_ERR_INVALID_ARG;
  AttnArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  if (plan.max_parts > 1) {
    if (!workspace || workspace_bytes < plan.bytes || !aligned16(workspace)) return PKV_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    a.ws_acc = reinterpret_cast<float*>(ws);
    a.ws_m = reinterpret_cast<float*>(ws + plan.off_m);
    a.ws_l = reinterpret_cast<float*>(ws + plan.off_l);
    if (plan.list) {
      a.ws_hdr = reinterpret_cast<int32_t*>(ws + plan.off_hdr);
      a.ws_tag = reinterpret_cast<uint64_t*>(ws + plan.off_tag);
    } else {
      a.ws_seg = reinterpret_cast<int32_t*>(ws + plan.off_seg);
    }
  }
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks;
  a.max_context_len = max_context_len;
  a.partition_size = plan.P;
  a.max_parts = plan.max_parts;
  a.total_items = static_cast<int32_t>(items);
  // Softmax of scale * (q . k), run in the exp2 domain (any sign of scale; a
  // zero scale gives equal weights).
  a.c = scale * 1.4426950408889634f;
  a.query_start = nullptr;  // decode: one query row per sequence
  a.num_q_heads = num_q_heads;
  a.num_query_rows = num_seqs;
  a.max_query_len = 1;

  auto run = [&](Op op) {
    return kv_dtype == PKV_BF16 ? launch_op<BF16>(a, head_dim, G, plan.list, op, stream)
                                : launch_op<F32>(a, head_dim, G, plan.list, op, stream);
  };
  const bool both = (stages & kStagePartitions) && (stages & kStageReduce);
  if (stages & kStagePartitions) {
    if (k_new) {
      // The item list writes the new tokens inside the attention kernel;
      // partition items take a separate write first.
      if (plan.list) {
        a.k_new = k_new;
        a.v_new = v_new;
      } else if (launch_write_last_token(k_new, v_new, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                                         block_tables, context_lens, num_seqs, num_kv_heads, head_dim, block_size,
                                         num_blocks, max_blocks, max_context_len, kv_dtype, stream) != hipSuccess) {
        return PKV_ERR_HIP;
      }
    }
    const Op op = !plan.list ? Op::kPass : k_new ? Op::kWriteFused : both ? Op::kFused : Op::kPass;
    if (run(op) != hipSuccess) return PKV_ERR_HIP;
  }
  if ((stages & kStageReduce) && plan.max_parts > 1) {
    if (!plan.list) {
      const dim3 rg(static_cast<unsigned>(num_seqs) * num_kv_heads);
      if (head_dim == 64)
        hipLaunchKernelGGL((lse_reduce_kernel<64>), rg, dim3(kThreads), 0, stream, a, num_q_heads);
      else
        hipLaunchKernelGGL((lse_reduce_kernel<128>), rg, dim3(kThreads), 0, stream, a, num_q_heads);
      if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
    } else if (!both) {
      if (run(Op::kListReduce) != hipSuccess) return PKV_ERR_HIP;
    }
  }
  return PKV_OK;
}

// The decode step's workspace for callers that cannot allocate: a
// file-scope device array, one per GPU the library runs on (the code object
// holds it until the process ends).  Its device address is looked up once per
// device, with that device current; the array's name is only a host-side
// stand-in and is never passed to a kernel.  Every call on one GPU shares it
// (the hand-over pairs need no clearing: see tag_next), so calls that overlap
// on one GPU race.
constexpr size_t kScratchBytes = size_t{18} << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

void* scratch_address() {
  static std::mutex mu;
  static void* cache[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    cache[dev] = p;
  }
  return cache[dev];
}

}  // namespace

// Runs of at most 16 / G queries per sequence (the verification of drafted
// tokens) on the decode kernel: its persistent, cost-balanced item list with
// the queries of a run as further matrix-core columns.  The partition size is
// 512 tokens, or 256 for a small batch (see runs_partition).  Arguments as
// pkv_paged_attention_multi takes them, already checked;
// PKV_ERR_UNSUPPORTED when the batch does not fit this path (too
// many sequences, runs too long, or no workspace where the split needs one),
// and the caller then uses the runs kernel; PKV_ERR_WORKSPACE for a workspace
// too small.  With skip_long, max_query_len is the longest run this launch
// takes, and the runs kernel takes the longer ones of the batch.
constexpr int32_t kRunsPartition = 512;
// The item list cuts its lanes' runs at single groups only when the batch's
// cost holds four partitions per lane, else at partition starts, which leaves
// lanes up to half a partition apart.  A batch whose cost, counted at its
// longest context, stays under six partitions of 512 per lane (about 512
// workgroups fill the GPU, H_kv per lane) takes 256-token partitions instead,
// whose cuts are then fine.  The count is an upper bound, hence the margin.
int32_t runs_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
  const int64_t lanes = std::max<int64_t>(1, 512 / std::max<int32_t>(num_kv_heads, 1));
  const int64_t groups = static_cast<int64_t>(num_seqs) * ((static_cast<int64_t>(max_context_len) + 15) / 16);
  return groups < 6 * lanes * (kRunsPartition / 16 + kItemCharge) ? kRunsPartition / 2 : kRunsPartition;
}

bool runs_listed_fits(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t max_context_len, int32_t max_query_len) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads) return false;
  const int G = num_q_heads / num_kv_heads;
  if (max_query_len < 1 || static_cast<int64_t>(max_query_len) * G > 16) return false;
  const Plan plan = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, 16, max_context_len,
                              runs_partition(num_seqs, num_kv_heads, max_context_len), 16);
  // the output offsets of one run stay within 32 bits
  return plan.list && static_cast<int64_t>(max_query_len) * num_q_heads * head_dim * 4 < (int64_t{1} << 31);
}

size_t runs_listed_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_context_len, int32_t max_query_len) {
  if (!runs_listed_fits(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, max_query_len)) return 0;
  return make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, 16, max_context_len,
                   runs_partition(num_seqs, num_kv_heads, max_context_len), 16)
      .bytes;
}

pkv_status runs_listed(float* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
                       int32_t num_query_rows, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t max_blocks, int32_t max_context_len,
                       int32_t max_query_len, bool skip_long, float scale, void* workspace, size_t workspace_bytes,
                       int32_t kv_dtype, hipStream_t stream) {
  if (!runs_listed_fits(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, max_query_len))
    return PKV_ERR_UNSUPPORTED;
  const int G = num_q_heads / num_kv_heads;
  const Plan plan =
      make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                runs_partition(num_seqs, num_kv_heads, max_context_len), 16);
  const int64_t items = static_cast<int64_t>(plan.max_parts) * num_seqs * num_kv_heads;
  if (items > INT32_MAX / 2) return PKV_ERR_UNSUPPORTED;
  AttnArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  if (plan.max_parts > 1) {
    // no workspace: the caller takes the runs kernel, which needs none; one too small is an error
    if (!workspace) return PKV_ERR_UNSUPPORTED;
    if (workspace_bytes < plan.bytes || !aligned16(workspace)) return PKV_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    a.ws_acc = reinterpret_cast<float*>(ws);
    a.ws_m = reinterpret_cast<float*>(ws + plan.off_m);
    a.ws_l = reinterpret_cast<float*>(ws + plan.off_l);
    a.ws_hdr = reinterpret_cast<int32_t*>(ws + plan.off_hdr);
    a.ws_tag = reinterpret_cast<uint64_t*>(ws + plan.off_tag);
  }
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks;
  a.max_context_len = max_context_len;
  a.partition_size = plan.P;
  a.max_parts = plan.max_parts;
  a.total_items = static_cast<int32_t>(items);
  a.c = scale * 1.4426950408889634f;
  a.query_start = query_start;
  a.num_q_heads = num_q_heads;
  a.num_query_rows = num_query_rows;
  a.max_query_len = max_query_len;
  a.skip_long = skip_long ? 1 : 0;
  const hipError_t err = kv_dtype == PKV_BF16 ? launch_runs<BF16>(a, head_dim, G, stream)
                                              : launch_runs<F32>(a, head_dim, G, stream);
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv

using namespace pkv;

extern "C" {

size_t pkv_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || head_dim <= 0 ||
      block_size <= 0 || max_context_len < 0 || partition_size < 0)
    return 0;
  return make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len, partition_size).bytes;
}

#define PKV_ATTN_PARAMS                                                                                          \
  float *out, const void *q, const void *k_cache, const void *v_cache, const int32_t *block_tables,             \
      const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, \
      int32_t block_size, int32_t num_blocks, int32_t max_blocks, int32_t max_context_len, float scale,           \
      int32_t partition_size, void *workspace, size_t workspace_bytes, int32_t kv_dtype, hipStream_t stream
#define PKV_ATTN_ARGS                                                                                      \
  out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,    \
      block_size, num_blocks, max_blocks, max_context_len, scale, partition_size, workspace, workspace_bytes, \
      kv_dtype, stream

pkv_status pkv_paged_attention_decode(PKV_ATTN_PARAMS) {
  return attention_stages(kStagePartitions | kStageReduce, nullptr, nullptr, PKV_ATTN_ARGS);
}

pkv_status pkv_paged_attention_partitions(PKV_ATTN_PARAMS) {
  return attention_stages(kStagePartitions, nullptr, nullptr, PKV_ATTN_ARGS);
}

pkv_status pkv_paged_attention_reduce(PKV_ATTN_PARAMS) {
  return attention_stages(kStageReduce, nullptr, nullptr, PKV_ATTN_ARGS);
}

pkv_status pkv_decode_step(const void* k_new, const void* v_new, PKV_ATTN_PARAMS) {
  if (!k_new || !v_new) return PKV_ERR_INVALID_ARG;
  return attention_stages(kStagePartitions | kStageReduce, k_new, v_new, PKV_ATTN_ARGS);
}

pkv_status pkv_decode_step_static(const void* k_new, const void* v_new, float* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t num_blocks, int32_t max_blocks, int32_t max_context_len,
                                  float scale, int32_t partition_size, int32_t kv_dtype, hipStream_t stream) {
  // Shapes the kernels take; anything else goes straight to pkv_decode_step,
  // which refuses it before any device work.
  const int G = num_kv_heads > 0 && num_q_heads > 0 && num_q_heads % num_kv_heads == 0 ? num_q_heads / num_kv_heads : 0;
  if (num_seqs > 0 && (G == 1 || G == 2 || G == 4 || G == 8) && (head_dim == 64 || head_dim == 128) &&
      (block_size == 16 || block_size == 32) && item_size(kv_dtype) != 0 && max_context_len >= 0 &&
      partition_size >= 0 && partition_size % block_size == 0) {
    const size_t need = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                                  partition_size).bytes;
    if (need > kScratchBytes) return PKV_ERR_WORKSPACE;
    if (need > 0) {
      void* ws = scratch_address();
      if (!ws) return PKV_ERR_HIP;
      return pkv_decode_step(k_new, v_new, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                             num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks,
                             max_context_len, scale, partition_size, ws, kScratchBytes, kv_dtype, stream);
    }
  }
  // no workspace needed, or arguments that pkv_decode_step refuses
  return pkv_decode_step(k_new, v_new, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                         num_kv_heads, head_dim, block_size, num_blocks, max_blocks, max_context_len, scale,
                         partition_size, nullptr, 0, kv_dtype, stream);
}

#undef PKV_ATTN_PARAMS
#undef PKV_ATTN_ARGS

}  // extern "C"

// Paged decode attention for gfx950: one query token per sequence, keys and
// values read through block tables, split-context partitions combined by a
// log-sum-exp reduction.
//
// Unit of work: an item = (sequence, KV head, context partition of at most P
// tokens).  A workgroup of 4 waves handles an item; wave w takes the 16-token
// groups g = w, w + 4, ... of the partition.  Per group a wave
//   - loads the group's 16 key rows (nontemporal 16-byte loads, one register
//     ring slot per group),
//   - computes the G logits of each token (raw q.k), writes them to its own LDS
//     region and tracks per-head maxima, then refills the slot with the group's
//     values, so the value loads overlap the rest of the QK work;
// then reduces the maxima across the wave, turns logits into probabilities in
// place (one fma + exp2 each), and accumulates p * V in fp32 from the ring.
// The G query heads of a KV head share every key and value load (GQA).  The
// four waves merge their (max, sum, acc) once, through LDS, and write the
// output rows (one partition) or the partition's partials.
//
// QK runs on the matrix cores (v_mfma_f32_16x16x32_bf16) for bf16 caches with
// G >= 4, where each 16-token group is a real [16 x d] x [d x G] contraction;
// on the vector ALUs (v_dot2_f32_bf16 or fp32 fma, 8-lane DPP sums) otherwise.
// PV always runs on the vector ALUs in fp32: probabilities are never rounded.
//
// Two kernels share these building blocks:
//   paged_decode_persistent  partitions of at most 512 tokens (one ring batch
//       per wave) and at most 4096 sequences: a grid sized to fill the chip
//       walks the item list (built per workgroup from an LDS prefix sum of the
//       partition counts); while a wave accumulates p * V of one item it
//       refills each consumed ring slot with the keys of its next item, so the
//       memory pipe stays busy across item boundaries.
//   paged_decode_items       any partition size: one workgroup per item, the
//       partition streamed in batches of ring slots with an online rescale.

#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "device_common.h"

namespace pkv {
namespace {

constexpr int kGroup = 16;                // tokens of one group
constexpr int kMaxPersistentSeqs = 4096;  // sequences the persistent kernel's LDS item list holds

struct AttnArgs {
  float* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_acc;  // [S][H_q][max_parts][d]
  float* ws_m;    // [S][H_q][max_parts]   maximum logit, exp2 domain (scaled)
  float* ws_l;    // [S][H_q][max_parts]   sum of exp2(logit - max)
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t max_context_len;
  int32_t partition_size;  // tokens, multiple of block_size
  int32_t max_parts;
  float c;          // |scale| * log2(e) (>= FLT_MIN): logits enter exp2 as fma(s, c, -m)
  uint32_t q_sign;  // xor mask applied to q's bits: flips its sign when scale < 0
};

// Number of partitions of a sequence of n_raw tokens (1 for an empty or
// invalid one); sets *bad for invalid lengths.
__device__ __forceinline__ int seq_parts(const AttnArgs& a, int n_raw, bool* bad) {
  *bad = n_raw < 0 || n_raw > a.max_context_len ||
         static_cast<int64_t>(n_raw) > static_cast<int64_t>(a.max_blocks) * a.block_size;
  if (*bad || n_raw == 0) return 1;
  return (n_raw + a.partition_size - 1) / a.partition_size;
}

// Per-instantiation geometry.
template <class DT, int D, int G>
struct Geo {
  static constexpr int kItem = DT::kItem;
  static constexpr int R = D * kItem;           // bytes of one token row
  static constexpr int NP = R / kKeyPiece;      // key pieces per row
  static constexpr int LR = R / 16;             // lanes covering one value row
  static constexpr int TPL = kWave / LR;        // value rows per wave load
  static constexpr int E = 16 / kItem;          // scalars per 16 bytes
  static constexpr int NB16 = R / 64;           // 16-byte registers per lane per group (K or V)
  // Waves per workgroup and ring slots (groups in flight) per wave: the ring
  // (NBUF * NB16 * 4 VGPRs), the accumulators (G * E) and two items' query
  // registers must fit 256 VGPRs for two waves per SIMD, so wide rows and
  // head groups trade ring depth for waves.  W * NBUF stays 32 groups.
  static constexpr int W = (G * NB16 >= 16) ? 8 : 4;
  static constexpr int NBUF = 32 / W;
  static constexpr int P1 = W * NBUF * kGroup;  // 512: longest partition one ring batch covers
  static constexpr int RF = (NBUF * kGroup * G > G * D) ? NBUF * kGroup * G : G * D;  // floats per wave region
  static constexpr int kThreads = W * kWave;
  static constexpr int kMinWaves = 2;  // occupancy the register budget targets (per SIMD)
  static_assert(R % kKeyPiece == 0 && kGroup % TPL == 0, "unsupported row size");
  static_assert(2 * NP == NB16 && kGroup / TPL == NB16, "K and V groups must fill the same registers");
};

template <class DT, int G>
constexpr bool kUseMfmaQK = std::is_same<DT, BF16>::value && G >= 4;

// Orders one wave's LDS writes before later LDS reads of other lanes of the
// same wave (a wave's LDS ops execute in order; this stops the compiler from
// moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Row rotations used for reductions over lanes with equal (lane mod n) inside a
// row of 16: x + ror_n(x) pairs lane i with lane (i + n) mod 16.
template <int N>
__device__ __forceinline__ float ror(float x) {
  return dpp<0x120 + N>(x);
}

// Sum over all lanes with the same (lane mod M), M a power of two <= 32.
template <int M>
__device__ __forceinline__ float sum_mod(float x) {
  if constexpr (M <= 1) x += ror<1>(x);
  if constexpr (M <= 2) x += ror<2>(x);
  if constexpr (M <= 4) x += ror<4>(x);
  if constexpr (M <= 8) x += ror<8>(x);
  if constexpr (M <= 16) x = sum_xor16(x);
  x = sum_xor32(x);
  return x;
}

template <bool V>
using Bool = std::integral_constant<bool, V>;

// ---------------------------------------------------------------------------
// Per-group building blocks.
// ---------------------------------------------------------------------------
template <class DT, int D, int G, bool QKM>
struct Ops {
  using Gm = Geo<DT, D, G>;
  static constexpr int NP = Gm::NP, E = Gm::E, R = Gm::R, TPL = Gm::TPL, LR = Gm::LR, NB16 = Gm::NB16;
  static constexpr int NQ = QKM ? NB16 : G * NP;  // 16-byte query registers per lane
  static constexpr int NM = QKM ? 1 : G;          // per-lane running maxima during QK

  // Matrix path: lane l feeds token row l % 16 and head column l % 16 with
  // bytes [64 st + 16 (l / 16), +16) of the row in step st, and receives the
  // logits of tokens 4 (l / 16) + r, r < 4, for head l % 16 (columns >= G are
  // zero).  Vector path: lane (l8, j8) holds the 16-byte column j8 of every
  // 128-byte key piece of tokens l8 and l8 + 8.
  __device__ __forceinline__ static void load_query(uint4 (&q)[NQ], const char* qrow, uint32_t sign, int lane) {
    if constexpr (QKM) {
      const int mi = lane & 15, mk = lane >> 4;
#pragma unroll
      for (int st = 0; st < NB16; ++st) {
        // Columns >= G read row 0 and are zeroed: no load sits behind a branch.
        const uint4 v = *reinterpret_cast<const uint4*>(qrow + (mi < G ? mi : 0) * R + st * 64 + mk * 16);
        const uint32_t s = mi < G ? sign : 0u, z = mi < G ? ~0u : 0u;
        q[st] = make_uint4((v.x ^ s) & z, (v.y ^ s) & z, (v.z ^ s) & z, (v.w ^ s) & z);
      }
    } else {
      const int j8 = lane & 7;
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const uint4 v = *reinterpret_cast<const uint4*>(qrow + h * R + i * kKeyPiece + j8 * 16);
          q[h * NP + i] = make_uint4(v.x ^ sign, v.y ^ sign, v.z ^ sign, v.w ^ sign);
        }
    }
  }

  // The 16 key rows starting at row0 of the key tile at ktile.
  __device__ __forceinline__ static void load_keys(uint4 (&kb)[NB16], const char* ktile, int row0, int B, int lane) {
    if constexpr (QKM) {
      const char* p = ktile + (row0 + (lane & 15)) * kKeyPiece + (lane >> 4) * 16;
#pragma unroll
      for (int st = 0; st < NB16; ++st)
        kb[st] = load_nt(p + static_cast<size_t>(st / 2) * B * kKeyPiece + (st % 2) * 64);
    } else {
      const char* p = ktile + (row0 + (lane >> 3)) * kKeyPiece + (lane & 7) * 16;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < NP; ++i)
          kb[hh * NP + i] = load_nt(p + static_cast<size_t>(i) * B * kKeyPiece + hh * 8 * kKeyPiece);
    }
  }

  // The 16 value rows starting at row0 of the value tile at vtile: lane holds
  // bytes [cv * 16, +16) of rows row0 + rv + TPL * jj.
  __device__ __forceinline__ static void load_values(uint4 (&vb)[NB16], const char* vtile, int row0, int lane) {
    const char* p = vtile + static_cast<size_t>(row0 + lane / LR) * R + (lane % LR) * 16;
#pragma unroll
    for (int jj = 0; jj < NB16; ++jj) vb[jj] = load_nt(p + static_cast<size_t>(jj) * TPL * R);
  }

  __device__ __forceinline__ static void max_init(float (&m)[NM]) {
#pragma unroll
    for (int h = 0; h < NM; ++h) m[h] = -INFINITY;
  }

  // Raw logits of one group into lg[t * G + h] (t < 16), -inf for tokens at
  // or past tok_end; folds them into the running maxima m.
  __device__ __forceinline__ static void qk_group(const uint4 (&q)[NQ], const uint4 (&kb)[NB16], float* lg, int t_first, int tok_end,
                                  float (&m)[NM], int lane) {
    if constexpr (QKM) {
      const int mi = lane & 15, mk = lane >> 4;
      f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int st = 0; st < NB16; ++st)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb[st]), as_bf16x8(q[st]), sc, 0, 0, 0);
      if (t_first + kGroup > tok_end) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t_first + 4 * mk + r >= tok_end) sc[r] = -INFINITY;
      }
      m[0] = fmaxf(m[0], fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
      if (mi < G) {
#pragma unroll
        for (int r = 0; r < 4; ++r) lg[(4 * mk + r) * G + mi] = sc[r];
      }
    } else {
      const int l8 = lane >> 3, j8 = lane & 7;
      float s[2][G];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float x = 0.0f;
#pragma unroll
          for (int i = 0; i < NP; ++i) x = dot16(DT{}, q[h * NP + i], kb[hh * NP + i], x);
          s[hh][h] = sum8(x);
        }
      if (t_first + kGroup > tok_end) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          if (t_first + hh * 8 + l8 >= tok_end) {
#pragma unroll
            for (int h = 0; h < G; ++h) s[hh][h] = -INFINITY;
          }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) m[h] = fmaxf(m[h], fmaxf(s[0][h], s[1][h]));
      if (j8 == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int h = 0; h < G; ++h) lg[(hh * 8 + l8) * G + h] = s[hh][h];
      }
    }
  }

  // Wave-uniform per-head maxima (raw logits) from the lane state.
  __device__ __forceinline__ static void max_finish(const float (&m)[NM], float (&lmax)[G]) {
    if constexpr (QKM) {
      const float x = max_xor32(max_xor16(m[0]));  // lane l: maximum of head l % 16
#pragma unroll
      for (int h = 0; h < G; ++h) lmax[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), h));
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) lmax[h] = max_xor32(max_xor16(fmaxf(m[h], ror<8>(m[h]))));
    }
  }

  // acc[h][e] += p[t][h] * V[t][e] over the group's tokens before tok_end.
  __device__ __forceinline__ static void pv_group(const uint4 (&vb)[NB16], const float* pg, int t_first, int tok_end,
                                  float (&acc)[G][E], int lane) {
    const int rv = lane / LR;
#pragma unroll
    for (int jj = 0; jj < NB16; ++jj) {
      const int tl = jj * TPL + rv;  // token within the group
      if (t_first + tl < tok_end) {
        float v[E];
        widen16(DT{}, vb[jj], v);
        const float* pp = pg + tl * G;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = pp[h];
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p, v[e], acc[h][e]);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Softmax of one batch and the workgroup merge, shared by both kernels.
// ---------------------------------------------------------------------------

// Folds a batch's maxima into the running state, rescales acc and l when an
// earlier batch exists, and turns the batch's nlog logits in reg into
// probabilities.  wm: this wave's slot of the per-wave maxima (LDS).
template <int G, int E>
__device__ __forceinline__ void softmax_batch(float* reg, int nlog, const float (&lmax)[G], float c, bool first,
                                              float (&m_run)[G], float& m_mine_run, float& l_mine,
                                              float (&acc)[G][E], float* wm, int lane) {
  float m_new[G];
#pragma unroll
  for (int h = 0; h < G; ++h) m_new[h] = fmaxf(m_run[h], lmax[h] * c);
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) wm[h] = m_new[h];
  }
  wave_lds_sync();
  const float m_mine = wm[lane % G];
  if (first) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float alpha = m_run[h] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[h] - m_new[h]);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
    }
    l_mine *= m_mine_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_mine_run - m_mine);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) m_run[h] = m_new[h];
  m_mine_run = m_mine;
  for (int e = lane; e < nlog; e += kWave) {
    const float p = __builtin_amdgcn_exp2f(fmaf(reg[e], c, -m_mine));
    reg[e] = p;
    l_mine += p;
  }
  wave_lds_sync();
}

template <int W, int RF, int G>
struct MergeShared {
  float region[W][RF];  // wave-private: logits, probabilities, then partial output
  float wm[W][G];       // per-wave maximum (scaled, exp2 domain)
  float wl[W][G];       // per-wave sum of probabilities
};

// Combine lanes, then waves; write the item's output rows (one partition) or
// its partials.  Ends with a barrier so the regions can be reused.  An item
// with fill set (an empty or invalid sequence) writes zeros, or NaN
// when bad, instead.
template <class DT, int D, int G, class SH>
__device__ __forceinline__ void merge_item(const AttnArgs& a, SH& sh, float (&acc)[G][Geo<DT, D, G>::E], float l_mine,
                                           bool poisoned, int seq, int kvh, int part, bool direct, bool fill = false,
                                           bool bad = false) {
  using Gm = Geo<DT, D, G>;
  constexpr int E = Gm::E, LR = Gm::LR, W = Gm::W, kThreads = Gm::kThreads;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: keeps per-wave math scalar
  l_mine = sum_mod<G>(l_mine);
  if (poisoned) l_mine = __builtin_nanf("");
  float* reg = sh.region[wave];
  // One head at a time keeps the cross-lane temporaries few: the next item's
  // keys already occupy the ring registers here.
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float x = sum_mod<LR>(acc[h][e]);
      if (lane < LR) reg[h * D + (lane % LR) * E + e] = poisoned ? __builtin_nanf("") : x;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (lane < G) sh.wl[wave][lane] = l_mine;  // sh.wm[wave] already holds the final maxima
  __syncthreads();
  const int Hq = a.num_kv_heads * G;
  float* out_rows = a.out + (static_cast<size_t>(seq) * Hq + static_cast<size_t>(kvh) * G) * D;
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sh.wm[w][h]);
    float sa = 0.0f, sl = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float wt = __builtin_amdgcn_exp2f(sh.wm[w][h] - M);  // 0 for a wave that saw no token
      sa = fmaf(wt, sh.region[w][i], sa);
      sl = fmaf(wt, sh.wl[w][h], sl);
    }
    if (fill) {
      out_rows[i] = bad ? __builtin_nanf("") : 0.0f;
    } else if (direct) {
      out_rows[i] = sa / sl;
    } else {
      const size_t row = (static_cast<size_t>(seq) * Hq + static_cast<size_t>(kvh) * G + h) * a.max_parts + part;
      a.ws_acc[row * D + i % D] = sa;
      if (i % D == 0) {
        a.ws_m[row] = M;
        a.ws_l[row] = sl;
      }
    }
  }
  __syncthreads();
}

// Rows of an empty (zeros) or invalid (NaN) sequence.
template <int D, int G, int kThreads>
__device__ __forceinline__ void fill_rows(const AttnArgs& a, int seq, int kvh, bool bad) {
  float* out_rows = a.out + (static_cast<size_t>(seq) * a.num_kv_heads * G + static_cast<size_t>(kvh) * G) * D;
  const float fill = bad ? __builtin_nanf("") : 0.0f;
  for (int i = threadIdx.x; i < G * D; i += kThreads) out_rows[i] = fill;
}

// Block ids of this wave's groups j < nk, counted from the table entry bt of
// the first group of the batch: lane j holds group j's id, lanes >= nk the id
// of the batch's first entry (a valid address for the unused ring slots).
// Out-of-range ids become 0; one read by a lane < nk sets *poisoned
// (wave-uniform).  The load is unconditional: a load behind a branch makes
// the compiler wait for every earlier load at the join.
template <int W>
__device__ __forceinline__ int load_ids(const AttnArgs& a, const int32_t* bt, int nk, int wave, int lane,
                                        bool* poisoned) {
  const int tok = lane < nk ? (wave + lane * W) * kGroup : 0;
  int id = bt[tok / a.block_size];
  const bool oob = static_cast<unsigned>(id) >= static_cast<unsigned>(a.num_blocks);
  *poisoned = __ballot(oob && lane < nk) != 0;
  return oob ? 0 : id;
}

// ---------------------------------------------------------------------------
// Kernel 1: one workgroup per item, any partition size.
// ---------------------------------------------------------------------------
template <class DT, int D, int G, bool QKM>
__global__ __launch_bounds__((Geo<DT, D, G>::kThreads)) __attribute__((amdgpu_waves_per_eu(Geo<DT, D, G>::kMinWaves)))
void paged_decode_items(AttnArgs a) {
  using Gm = Geo<DT, D, G>;
  using O = Ops<DT, D, G, QKM>;
  constexpr int E = Gm::E, R = Gm::R, NB16 = Gm::NB16, NBUF = Gm::NBUF, W = Gm::W;
  __shared__ MergeShared<W, Gm::RF, G> sh;

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: keeps per-wave math scalar
  const int Hkv = a.num_kv_heads;
  const int kvh = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int seq = rest % a.num_seqs;
  const int part = rest / a.num_seqs;
  const int B = a.block_size;

  const int n_raw = a.context_lens[seq];
  bool bad_len;
  const int nparts = seq_parts(a, n_raw, &bad_len);
  if (part >= nparts) return;
  if (bad_len || n_raw == 0) {
    fill_rows<D, G, Gm::kThreads>(a, seq, kvh, bad_len);
    return;
  }
  const int tok_begin = part * a.partition_size;
  const int tok_end = min(n_raw, tok_begin + a.partition_size);
  const int ngroups = (tok_end - tok_begin + kGroup - 1) / kGroup;
  const int nk = wave < ngroups ? (ngroups - wave + W - 1) / W : 0;  // this wave's groups

  const int32_t* bt = a.block_tables + static_cast<size_t>(seq) * a.max_blocks + tok_begin / B;
  const char* kbase = static_cast<const char*>(a.k_cache) + static_cast<size_t>(kvh) * B * R;
  const char* vbase = static_cast<const char*>(a.v_cache) + static_cast<size_t>(kvh) * B * R;
  const char* qrow =
      static_cast<const char*>(a.q) + (static_cast<size_t>(seq) * Hkv * G + static_cast<size_t>(kvh) * G) * R;
  const size_t block_stride = static_cast<size_t>(Hkv) * B * R;
  float* reg = sh.region[wave];

  float m_run[G];
  float acc[G][E];
  float l_mine = 0.0f;
  float m_mine_run = -INFINITY;
  bool poisoned = false;
#pragma unroll
  for (int h = 0; h < G; ++h) m_run[h] = -INFINITY;

  // Batches of NBUF groups; group b0 + j of this wave is partition group
  // wave + (b0 + j) * W.  A wave without groups still runs one empty batch so
  // that its state is defined.
  for (int b0 = 0; b0 < nk || b0 == 0; b0 += NBUF) {
    const int nb = min(NBUF, nk - b0);
    bool pois;
    const int idv = load_ids<W>(a, bt + (b0 * W * kGroup) / B, nb, wave, lane, &pois);
    poisoned |= pois;
    // Ring slot j >= nb repeats slot 0's addresses (the batch's first entry,
    // row 0, when the wave has no group), so every load is issued on every
    // path: a load behind a branch makes the compiler wait for all earlier
    // loads where the paths join.
    auto src = [&](int j) __attribute__((always_inline)) { return j < nb ? j : 0; };
    auto row = [&](int j) __attribute__((always_inline)) {
      return nb > 0 ? ((wave + (b0 + src(j)) * W) * kGroup) % B : 0;
    };
    auto t_first = [&](int j) __attribute__((always_inline)) { return tok_begin + (wave + (b0 + j) * W) * kGroup; };
    auto tile = [&](int j) __attribute__((always_inline)) {
      return static_cast<size_t>(__builtin_amdgcn_readlane(idv, src(j))) * block_stride;
    };

    // The query first: the load counter is in order, so the first group's
    // logits wait only for it and that group's keys.
    uint4 q[O::NQ];
    O::load_query(q, qrow, a.q_sign, lane);
    uint4 buf[NBUF][NB16];
#pragma unroll
    for (int j = 0; j < NBUF; ++j) O::load_keys(buf[j], kbase + tile(j), row(j), B, lane);
    float mstate[O::NM];
    O::max_init(mstate);
    {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        if (j < nb) O::qk_group(q, buf[j], reg + j * kGroup * G, t_first(j), tok_end, mstate, lane);
        O::load_values(buf[j], vbase + tile(j), row(j), lane);  // refill the consumed slot
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    float lmax[G];
    O::max_finish(mstate, lmax);
    softmax_batch<G, E>(reg, max(nb, 0) * kGroup * G, lmax, a.c, b0 == 0, m_run, m_mine_run, l_mine, acc,
                        sh.wm[wave], lane);
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      if (j < nb) O::pv_group(buf[j], reg + j * kGroup * G, t_first(j), tok_end, acc, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    wave_lds_sync();  // the next batch rewrites the region
  }
  merge_item<DT, D, G>(a, sh, acc, l_mine, poisoned, seq, kvh, part, nparts == 1);
}

// ---------------------------------------------------------------------------
// Kernel 2: persistent workgroups over the item list, one ring batch per item.
// ---------------------------------------------------------------------------
template <int W, int RF, int G>
struct PersistShared : MergeShared<W, RF, G> {
  int32_t psum[kMaxPersistentSeqs + 1];  // prefix sums of partition counts
};

struct Item {
  int seq, kvh, part, n, nparts, tok_begin, tok_end, nk;
  bool special, bad;
};

template <class DT, int D, int G, bool QKM>
__global__ __launch_bounds__((Geo<DT, D, G>::kThreads)) __attribute__((amdgpu_waves_per_eu(Geo<DT, D, G>::kMinWaves)))
void paged_decode_persistent(AttnArgs a) {
  using Gm = Geo<DT, D, G>;
  using O = Ops<DT, D, G, QKM>;
  constexpr int E = Gm::E, R = Gm::R, NB16 = Gm::NB16, NBUF = Gm::NBUF, W = Gm::W;
  __shared__ PersistShared<W, Gm::RF, G> sh;

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: keeps per-wave math scalar
  const int S = a.num_seqs;
  const int Hkv = a.num_kv_heads;
  const int B = a.block_size;
  const size_t block_stride = static_cast<size_t>(Hkv) * B * R;

  // Item list: prefix sums of the partition counts (wave 0 scans; S <= 4096).
  for (int s = tid; s < S; s += Gm::kThreads) {
    bool bad;
    sh.psum[s + 1] = seq_parts(a, a.context_lens[s], &bad);
  }
  __syncthreads();
  if (wave == 0) {
    const int chunk = (S + kWave - 1) / kWave;
    const int lo = lane * chunk, hi = min(S, lo + chunk);
    int run = 0;
    for (int i = lo; i < hi; ++i) run += sh.psum[i + 1];
    int incl = run;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    int base = incl - run;
    for (int i = lo; i < hi; ++i) {
      base += sh.psum[i + 1];
      sh.psum[i + 1] = base;
    }
    if (lane == 0) sh.psum[0] = 0;
  }
  __syncthreads();
  const int total = sh.psum[S] * Hkv;
  int k = blockIdx.x;
  if (k >= total) return;

  auto decode = [&](int kk) __attribute__((always_inline)) {
    Item it;
    it.kvh = kk % Hkv;
    const int pidx = kk / Hkv;
    // LDS reads land in vector registers; readfirstlane marks them
    // wave-uniform so that every branch on the item stays a scalar branch.
    int lo = 0, hi = S;  // psum[lo] <= pidx < psum[lo + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (__builtin_amdgcn_readfirstlane(sh.psum[mid]) <= pidx)
        lo = mid;
      else
        hi = mid;
    }
    it.seq = lo;
    it.part = pidx - __builtin_amdgcn_readfirstlane(sh.psum[lo]);
    it.n = a.context_lens[lo];
    it.nparts = seq_parts(a, it.n, &it.bad);
    it.special = it.bad || it.n == 0;
    it.tok_begin = it.part * a.partition_size;
    it.tok_end = min(it.n, it.tok_begin + a.partition_size);
    const int ngroups = it.special ? 0 : (it.tok_end - it.tok_begin + kGroup - 1) / kGroup;
    it.nk = wave < ngroups ? (ngroups - wave + W - 1) / W : 0;
    return it;
  };
  auto ktile = [&](const Item& it, int idv, int j) __attribute__((always_inline)) {
    return static_cast<const char*>(a.k_cache) + static_cast<size_t>(it.kvh) * B * R +
           static_cast<size_t>(__builtin_amdgcn_readlane(idv, j < it.nk ? j : 0)) * block_stride;
  };
  auto vtile = [&](const Item& it, int idv, int j) __attribute__((always_inline)) {
    return static_cast<const char*>(a.v_cache) + static_cast<size_t>(it.kvh) * B * R +
           static_cast<size_t>(__builtin_amdgcn_readlane(idv, j < it.nk ? j : 0)) * block_stride;
  };
  // Ring slot j >= nk repeats slot 0's addresses (the item's first entry,
  // row 0, when the wave has no group): every load is issued on every path.
  auto src = [&](const Item& it, int j) __attribute__((always_inline)) { return j < it.nk ? j : 0; };
  auto row = [&](const Item& it, int j) __attribute__((always_inline)) {
    return it.nk > 0 ? ((wave + src(it, j) * W) * kGroup) % B : 0;
  };
  auto t_first = [&](const Item& it, int j) __attribute__((always_inline)) { return it.tok_begin + (wave + j * W) * kGroup; };
  auto table = [&](const Item& it) __attribute__((always_inline)) {
    return a.block_tables + static_cast<size_t>(it.seq) * a.max_blocks + it.tok_begin / B;
  };
  auto qrow = [&](const Item& it) __attribute__((always_inline)) {
    return static_cast<const char*>(a.q) +
           (static_cast<size_t>(it.seq) * Hkv * G + static_cast<size_t>(it.kvh) * G) * R;
  };
  float* reg = sh.region[wave];

  Item cur = decode(k);
  bool pois_cur;
  int idv_cur = load_ids<W>(a, table(cur), cur.nk, wave, lane, &pois_cur);
  uint4 q_cur[O::NQ];
  O::load_query(q_cur, qrow(cur), a.q_sign, lane);
  uint4 buf[NBUF][NB16];
#pragma unroll
  for (int j = 0; j < NBUF; ++j) O::load_keys(buf[j], ktile(cur, idv_cur, j), row(cur, j), B, lane);

  for (;;) {
    // The next item: its ids and query are fetched now, its keys go into ring
    // slots as the current item's values are consumed.  After the last item
    // the current one stands in for it, so the loads stay unconditional.
    const int kn = k + static_cast<int>(gridDim.x);
    const bool has_next = kn < total;
    Item nxt = cur;
    if (has_next) nxt = decode(kn);
    bool pois_next;
    const int idv_next = load_ids<W>(a, table(nxt), nxt.nk, wave, lane, &pois_next);
    uint4 q_next[O::NQ];
    O::load_query(q_next, qrow(nxt), a.q_sign, lane);

    // An empty or invalid item has no groups; it runs the same path and its
    // merge writes zeros or NaN.
    float mstate[O::NM];
    O::max_init(mstate);
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      if (j < cur.nk) O::qk_group(q_cur, buf[j], reg + j * kGroup * G, t_first(cur, j), cur.tok_end, mstate, lane);
      O::load_values(buf[j], vtile(cur, idv_cur, j), row(cur, j), lane);  // refill the consumed slot
      __builtin_amdgcn_sched_barrier(0);
    }
    float lmax[G], m_run[G], acc[G][E];
    float l_mine = 0.0f, m_mine_run = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) m_run[h] = -INFINITY;
    O::max_finish(mstate, lmax);
    softmax_batch<G, E>(reg, cur.nk * kGroup * G, lmax, a.c, true, m_run, m_mine_run, l_mine, acc, sh.wm[wave], lane);
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      if (j < cur.nk) O::pv_group(buf[j], reg + j * kGroup * G, t_first(cur, j), cur.tok_end, acc, lane);
      O::load_keys(buf[j], ktile(nxt, idv_next, j), row(nxt, j), B, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    merge_item<DT, D, G>(a, sh, acc, l_mine, pois_cur, cur.seq, cur.kvh, cur.part, cur.nparts == 1, cur.special,
                         cur.bad);
    if (!has_next) break;
    cur = nxt;
    idv_cur = idv_next;
    pois_cur = pois_next;
#pragma unroll
    for (int i = 0; i < O::NQ; ++i) q_cur[i] = q_next[i];
    k = kn;
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp combination of the partitions of one (sequence, query head):
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kWave) void lse_reduce_kernel(AttnArgs a, int num_q_heads) {
  const int row = blockIdx.x;  // seq * H_q + h
  const int seq = row / num_q_heads;
  bool bad;
  const int nparts = seq_parts(a, a.context_lens[seq], &bad);
  if (nparts <= 1) return;  // written directly by the attention kernel
  const int lane = threadIdx.x;
  const size_t base = static_cast<size_t>(row) * a.max_parts;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, a.ws_m[base + p]);
  constexpr int PER = D / kWave;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.0f;
  float L = 0.0f;
  for (int p = 0; p < nparts; ++p) {
    const float w = __builtin_amdgcn_exp2f(a.ws_m[base + p] - M);
    L = fmaf(w, a.ws_l[base + p], L);
    const float* ap = a.ws_acc + (base + p) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = fmaf(w, ap[lane + e * kWave], o[e]);
  }
  float* out = a.out + static_cast<size_t>(row) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[lane + e * kWave] = o[e] / L;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
struct Plan {
  int32_t P;          // effective partition size
  int32_t max_parts;  // partitions of the longest sequence
  size_t off_m, off_l, bytes;
};

Plan make_plan(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t block_size, int32_t max_context_len,
               int32_t partition_size) {
  Plan p{};
  const int64_t ctx = max_context_len > 0 ? max_context_len : 1;
  p.P = partition_size > 0 ? partition_size : static_cast<int32_t>(ceil_div64(ctx, block_size) * block_size);
  p.max_parts = static_cast<int32_t>(ceil_div64(ctx, p.P));
  if (p.max_parts <= 1) return p;
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * p.max_parts;
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  p.off_m = up(rows * head_dim * sizeof(float));
  p.off_l = p.off_m + up(rows * sizeof(float));
  p.bytes = p.off_l + up(rows * sizeof(float));
  return p;
}

// Workgroups of a kernel that fit the whole device at once, cached per
// device and per instantiation (Tag makes each kernel its own cache).
template <class Tag, class K>
int resident_workgroups(K kernel, int threads) {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
    cache[dev] = cus * (per_cu > 0 ? per_cu : 1);
  }
  return cache[dev];
}

template <class DT, int D, int G>
hipError_t launch_attention_g(const AttnArgs& a, int64_t items, hipStream_t stream) {
  using Gm = Geo<DT, D, G>;
  constexpr bool QKM = kUseMfmaQK<DT, G>;
  if (a.partition_size <= Gm::P1 && a.num_seqs <= kMaxPersistentSeqs) {
    auto kernel = paged_decode_persistent<DT, D, G, QKM>;
    const int fill = resident_workgroups<Ops<DT, D, G, QKM>>(kernel, Gm::kThreads);
    if (fill <= 0) return hipErrorInvalidValue;
    const int64_t grid = items < fill ? items : fill;
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(Gm::kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((paged_decode_items<DT, D, G, QKM>), dim3(static_cast<unsigned>(items)), dim3(Gm::kThreads),
                       0, stream, a);
  }
  return hipGetLastError();
}

template <class DT, int D>
hipError_t launch_attention_d(const AttnArgs& a, int G, int64_t items, hipStream_t stream) {
  switch (G) {
    case 1: return launch_attention_g<DT, D, 1>(a, items, stream);
    case 2: return launch_attention_g<DT, D, 2>(a, items, stream);
    case 4: return launch_attention_g<DT, D, 4>(a, items, stream);
    case 8: return launch_attention_g<DT, D, 8>(a, items, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class DT>
hipError_t launch_attention(const AttnArgs& a, int D, int G, int64_t items, hipStream_t stream) {
  if (D == 64) return launch_attention_d<DT, 64>(a, G, items, stream);
  if (D == 128) return launch_attention_d<DT, 128>(a, G, items, stream);
  return hipErrorInvalidValue;
}

enum : int { kStagePartitions = 1, kStageReduce = 2 };

pkv_status attention_stages(int stages, float* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
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

  const Plan plan = make_plan(num_seqs, num_q_heads, head_dim, block_size, max_context_len, partition_size);
  const int64_t items = static_cast<int64_t>(plan.max_parts) * num_seqs * num_kv_heads;
  if (items > INT32_MAX) return PKV_ERR_INVALID_ARG;
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
  }
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks;
  a.max_context_len = max_context_len;
  a.partition_size = plan.P;
  a.max_parts = plan.max_parts;
  // Softmax of scale * (q . k) in the exp2 domain.  A negative scale is folded
  // into q's sign (exact in bf16 and fp32), so the kernel scales by |scale|;
  // a zero scale becomes the smallest normal float, which leaves every
  // weight equal to 1 up to a relative 1e-34.
  const float c = fabsf(scale) * 1.4426950408889634f;
  a.c = c > FLT_MIN ? c : FLT_MIN;
  a.q_sign = scale < 0.0f ? (kv_dtype == PKV_BF16 ? BF16::kSignMask : F32::kSignMask) : 0u;

  if (stages & kStagePartitions) {
    const hipError_t err = kv_dtype == PKV_BF16 ? launch_attention<BF16>(a, head_dim, G, items, stream)
                                                : launch_attention<F32>(a, head_dim, G, items, stream);
    if (err != hipSuccess) return PKV_ERR_HIP;
  }
  if ((stages & kStageReduce) && plan.max_parts > 1) {
    const dim3 rg(static_cast<unsigned>(num_seqs) * num_q_heads);
    if (head_dim == 64)
      hipLaunchKernelGGL((lse_reduce_kernel<64>), rg, dim3(kWave), 0, stream, a, num_q_heads);
    else
      hipLaunchKernelGGL((lse_reduce_kernel<128>), rg, dim3(kWave), 0, stream, a, num_q_heads);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" {

size_t pkv_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t block_size,
                                     int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_context_len < 0 ||
      partition_size < 0)
    return 0;
  return make_plan(num_seqs, num_q_heads, head_dim, block_size, max_context_len, partition_size).bytes;
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
  return attention_stages(kStagePartitions | kStageReduce, PKV_ATTN_ARGS);
}

pkv_status pkv_paged_attention_partitions(PKV_ATTN_PARAMS) {
  return attention_stages(kStagePartitions, PKV_ATTN_ARGS);
}

pkv_status pkv_paged_attention_reduce(PKV_ATTN_PARAMS) { return attention_stages(kStageReduce, PKV_ATTN_ARGS); }

#undef PKV_ATTN_PARAMS
#undef PKV_ATTN_ARGS

}  // extern "C"

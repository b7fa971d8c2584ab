// Paged decode attention for gfx950: one query token per sequence, keys and
// values read through block tables, split-context partitions combined by a
// log-sum-exp reduction.
//
// Work decomposition.  One workgroup (4 waves) per (sequence, KV head, context
// partition).  Each wave is an independent flash-decoding worker over the
// 16-token groups g = wave, wave + 4, ... of every chunk of its partition:
//   1. block ids of its groups: one vector load, lane k holding group k's id,
//      read back with readlane (the ids live in registers, not LDS);
//   2. keys streamed through a register ring (KPF groups in flight): the G
//      logits of each token (raw dot products) go to the wave's LDS region;
//      per-head maxima tracked in registers;
//   3. first value loads issued, maxima reduced across the wave, running state
//      rescaled (several chunks only), logits turned into probabilities in
//      place with one fma + exp2 each;
//   4. values streamed through a ring (VPF groups), p * V accumulated in fp32.
// The G query heads of a KV head share every key and value load (GQA).  Waves
// meet once, at the end, to merge their (max, sum, acc) through LDS, and then
// write the output rows (one partition) or the partition's partials.

#include "device_common.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = kWave * kWaves;  // 256
constexpr int kGroup = 16;                // tokens of one group
constexpr int kLogitFloats = 4096;        // LDS floats for logits, 1024 per wave

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
  float c;             // |scale| * log2(e) (>= FLT_MIN): logits enter exp2 as fma(s, c, -m)
  uint32_t q_sign;     // xor mask applied to q's bits: flips its sign when scale < 0
};

// Number of partitions of a sequence of n_raw tokens; sets *bad for invalid lengths.
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
  static constexpr int R = D * kItem;                // bytes of one token row
  static constexpr int NP = R / kKeyPiece;           // key pieces per row
  static constexpr int LR = R / 16;                  // lanes covering one value row
  static constexpr int TPL = kWave / LR;             // value rows per wave load
  static constexpr int NLV = kGroup / TPL;           // value loads per group
  static constexpr int E = 16 / kItem;               // scalars per 16 bytes
  static constexpr int WF = kLogitFloats / kWaves;   // floats of one wave's LDS region
  static constexpr int CW = WF / G;                  // tokens one wave holds per chunk
  static constexpr int C = CW * kWaves;              // tokens per chunk of the workgroup
  // Key groups in flight per wave: 3, or 2 where the query registers are many.
  static constexpr int KPF = (G * NP * 4 >= 64) ? 2 : 3;
  static constexpr int VPF = 2;                      // value groups in flight per wave
  static_assert(R % kKeyPiece == 0 && kGroup % TPL == 0, "unsupported row size");
  static_assert(G * D <= WF, "a wave's partial output must fit its LDS region");
  static_assert(CW / kGroup <= kWave, "a wave's block ids must fit one register");
};

template <int G>
struct AttnShared {
  float region[kWaves][kLogitFloats / kWaves];  // wave-private: logits, probabilities, then partial output
  float wm[kWaves][G];                          // per-wave maximum (scaled, exp2 domain)
  float wl[kWaves][G];                          // per-wave sum of probabilities
};

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

template <class DT, int D, int G, bool MULTI>
__global__ __launch_bounds__(kThreads) void paged_decode_kernel(AttnArgs a) {
  using Gm = Geo<DT, D, G>;
  constexpr int NP = Gm::NP, E = Gm::E, C = Gm::C, R = Gm::R, NLV = Gm::NLV, TPL = Gm::TPL, LR = Gm::LR;
  constexpr int KPF = Gm::KPF, VPF = Gm::VPF;
  __shared__ AttnShared<G> sh;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int Hkv = a.num_kv_heads;
  const int Hq = Hkv * G;
  const int kvh = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int seq = rest % a.num_seqs;
  const int part = rest / a.num_seqs;
  const int B = a.block_size;

  const int n_raw = a.context_lens[seq];
  bool bad_len;
  const int nparts = seq_parts(a, n_raw, &bad_len);
  if (part >= nparts) return;
  const bool direct = nparts == 1;
  float* out_rows = a.out + (static_cast<size_t>(seq) * Hq + static_cast<size_t>(kvh) * G) * D;
  if (bad_len || n_raw == 0) {
    const float fill = bad_len ? __builtin_nanf("") : 0.0f;
    for (int i = tid; i < G * D; i += kThreads) out_rows[i] = fill;
    return;
  }
  const int tok_begin = part * a.partition_size;
  const int tok_end = min(n_raw, tok_begin + a.partition_size);

  // Lane roles.  Keys: lane (l8, j8) holds the 16-byte column j8 of every
  // 128-byte piece of tokens l8 and l8 + 8 of a group.  Values: lane holds
  // bytes [cv*16, cv*16+16) of row rv of each wave load.
  const int l8 = lane >> 3;
  const int j8 = lane & 7;
  const int cv = lane % LR;
  const int rv = lane / LR;
  const int hm = lane % G;  // the head whose probabilities this lane sums
  const float c = a.c;

  const int32_t* bt = a.block_tables + static_cast<size_t>(seq) * a.max_blocks;
  const char* kbase = static_cast<const char*>(a.k_cache) + static_cast<size_t>(kvh) * B * R;
  const char* vbase = static_cast<const char*>(a.v_cache) + static_cast<size_t>(kvh) * B * R;
  const char* qrow = static_cast<const char*>(a.q) + (static_cast<size_t>(seq) * Hq + static_cast<size_t>(kvh) * G) * R;
  const size_t block_stride = static_cast<size_t>(Hkv) * B * R;  // bytes between consecutive blocks
  float* reg = sh.region[wave];

  float m_run[G];              // running maxima (scaled), uniform across the wave
  float acc[G][E];
  float l_mine = 0.0f;         // partial sum of probabilities of head hm
  float m_mine_run = -INFINITY;
  bool poisoned = false;
#pragma unroll
  for (int h = 0; h < G; ++h) m_run[h] = -INFINITY;

  for (int c0 = tok_begin; c0 < tok_end; c0 += C) {
    const bool first = c0 == tok_begin;
    const int cn = min(C, tok_end - c0);
    const int ngroups = (cn + kGroup - 1) / kGroup;
    const int nk = wave < ngroups ? (ngroups - wave + kWaves - 1) / kWaves : 0;  // this wave's groups

    // 1. block ids of this wave's groups, one per lane
    int idv = 0;
    bool bad_lane = false;
    if (lane < nk) {
      const int g = wave + lane * kWaves;
      idv = bt[c0 / B + (g * kGroup) / B];
      if (static_cast<unsigned>(idv) >= static_cast<unsigned>(a.num_blocks)) {
        bad_lane = true;
        idv = 0;
      }
    }
    poisoned |= __ballot(bad_lane) != 0;
    auto group_row = [&](int k) { return ((wave + k * kWaves) * kGroup) % B; };
    auto tile_off = [&](int k) { return static_cast<size_t>(__builtin_amdgcn_readlane(idv, k)) * block_stride; };
    auto load_k = [&](uint4 (&kr)[2][NP], int k) {
      const char* p = kbase + tile_off(k) + (group_row(k) + l8) * kKeyPiece + j8 * 16;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < NP; ++i)
          kr[hh][i] = load_nt(p + static_cast<size_t>(i) * B * kKeyPiece + hh * 8 * kKeyPiece);
    };
    auto load_v = [&](uint4 (&vr)[NLV], int k) {
      const char* p = vbase + tile_off(k) + static_cast<size_t>(group_row(k) + rv) * R + cv * 16;
#pragma unroll
      for (int j = 0; j < NLV; ++j) vr[j] = load_nt(p + static_cast<size_t>(j) * TPL * R);
    };

    // 2. logits (raw dot products)
    float lmax[G];
#pragma unroll
    for (int h = 0; h < G; ++h) lmax[h] = -INFINITY;
    {
      uint4 qr[G][NP];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          uint4 v = *reinterpret_cast<const uint4*>(qrow + h * R + i * kKeyPiece + j8 * 16);
          v.x ^= a.q_sign;
          v.y ^= a.q_sign;
          v.z ^= a.q_sign;
          v.w ^= a.q_sign;
          qr[h][i] = v;
        }
      uint4 kb[KPF][2][NP];
#pragma unroll
      for (int j = 0; j < KPF; ++j)
        if (j < nk) load_k(kb[j], j);
      for (int k0 = 0; k0 < nk; k0 += KPF) {
#pragma unroll
        for (int j = 0; j < KPF; ++j) {
          const int k = k0 + j;
          if (k < nk) {
            float s[2][G];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int h = 0; h < G; ++h) {
                float x = 0.0f;
#pragma unroll
                for (int i = 0; i < NP; ++i) x = dot16(DT{}, qr[h][i], kb[j][hh][i], x);
                s[hh][h] = x;
              }
            if (k + KPF < nk) load_k(kb[j], k + KPF);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int h = 0; h < G; ++h) s[hh][h] = sum8(s[hh][h]);
            const int t_first = c0 + (wave + k * kWaves) * kGroup;
            if (t_first + kGroup > tok_end) {  // the partition's last group: mask the tail
#pragma unroll
              for (int hh = 0; hh < 2; ++hh)
                if (t_first + hh * 8 + l8 >= tok_end) {
#pragma unroll
                  for (int h = 0; h < G; ++h) s[hh][h] = -INFINITY;
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) lmax[h] = fmaxf(lmax[h], fmaxf(s[0][h], s[1][h]));
            if (j8 == 0) {
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                float* dst = reg + (k * kGroup + hh * 8 + l8) * G;
#pragma unroll
                for (int h = 0; h < G; ++h) dst[h] = s[hh][h];
              }
            }
          }
        }
      }
    }

    // 3. first value loads, wave maxima, running-state rescale, probabilities
    uint4 vb[VPF][NLV];
#pragma unroll
    for (int j = 0; j < VPF; ++j)
      if (j < nk) load_v(vb[j], j);
    float m_new[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float m = fmaxf(lmax[h], ror<8>(lmax[h]));  // lanes of a half-row already agree
      m = max_xor16(m);
      m = max_xor32(m);
      m_new[h] = fmaxf(m_run[h], m * c);
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) sh.wm[wave][h] = m_new[h];
    }
    wave_lds_sync();
    const float m_mine = sh.wm[wave][hm];
    if (!MULTI || first) {
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
    const int nlog = nk * kGroup * G;
    for (int e = lane; e < nlog; e += kWave) {
      const float p = __builtin_amdgcn_exp2f(fmaf(reg[e], c, -m_mine));
      reg[e] = p;
      l_mine += p;
    }
    wave_lds_sync();

    // 4. p * V
    for (int k0 = 0; k0 < nk; k0 += VPF) {
#pragma unroll
      for (int j = 0; j < VPF; ++j) {
        const int k = k0 + j;
        if (k < nk) {
          const int t_first = c0 + (wave + k * kWaves) * kGroup;
#pragma unroll
          for (int jj = 0; jj < NLV; ++jj) {
            const int tl = jj * TPL + rv;  // token within the group
            if (t_first + tl < tok_end) {
              float v[E];
              widen16(DT{}, vb[j][jj], v);
              const float* pp = reg + (k * kGroup + tl) * G;
#pragma unroll
              for (int h = 0; h < G; ++h) {
                const float p = pp[h];
#pragma unroll
                for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p, v[e], acc[h][e]);
              }
            }
          }
          if (k + VPF < nk) load_v(vb[j], k + VPF);
        }
      }
    }
    wave_lds_sync();
  }

  // Merge: lanes first, then the four waves through LDS.
  l_mine = sum_mod<G>(l_mine);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = sum_mod<LR>(acc[h][e]);
  if (poisoned) {
    l_mine = __builtin_nanf("");
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = __builtin_nanf("");
  }
  if (lane < LR) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) reg[h * D + cv * E + e] = acc[h][e];
  }
  if (lane < G) sh.wl[wave][lane] = l_mine;  // sh.wm[wave] already holds the final maxima
  __syncthreads();
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sh.wm[w][h]);
    float sa = 0.0f, sl = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = __builtin_amdgcn_exp2f(sh.wm[w][h] - M);  // 0 for a wave that saw no token
      sa = fmaf(wt, sh.region[w][i], sa);
      sl = fmaf(wt, sh.wl[w][h], sl);
    }
    if (direct) {
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
}

// Log-sum-exp combination of the partitions of one (sequence, query head):
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
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

template <class DT, int D, int G>
void launch_attention_m(const AttnArgs& a, dim3 grid, hipStream_t stream) {
  if (a.partition_size <= Geo<DT, D, G>::C)
    hipLaunchKernelGGL((paged_decode_kernel<DT, D, G, false>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((paged_decode_kernel<DT, D, G, true>), grid, dim3(kThreads), 0, stream, a);
}

template <class DT, int D>
hipError_t launch_attention_g(const AttnArgs& a, int G, dim3 grid, hipStream_t stream) {
  switch (G) {
    case 1: launch_attention_m<DT, D, 1>(a, grid, stream); break;
    case 2: launch_attention_m<DT, D, 2>(a, grid, stream); break;
    case 4: launch_attention_m<DT, D, 4>(a, grid, stream); break;
    case 8: launch_attention_m<DT, D, 8>(a, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class DT>
hipError_t launch_attention_d(const AttnArgs& a, int D, int G, dim3 grid, hipStream_t stream) {
  if (D == 64) return launch_attention_g<DT, 64>(a, G, grid, stream);
  if (D == 128) return launch_attention_g<DT, 128>(a, G, grid, stream);
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
  const int64_t grid = static_cast<int64_t>(plan.max_parts) * num_seqs * num_kv_heads;
  if (grid > INT32_MAX) return PKV_ERR_INVALID_ARG;
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
    const dim3 g(static_cast<unsigned>(grid));
    const hipError_t err = kv_dtype == PKV_BF16 ? launch_attention_d<BF16>(a, head_dim, G, g, stream)
                                                : launch_attention_d<F32>(a, head_dim, G, g, stream);
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

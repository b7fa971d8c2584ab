// Device half of libpkv for gfx950 (CDNA4, wave64): the slot scatter of new
// K/V, whole-block copies for copy-on-write, and paged decode attention with a
// split-context log-sum-exp reduction.
//
// Cache layout (fixed by pkv.h):
//   V[num_blocks][H_kv][B][d]
//   K[num_blocks][H_kv][d / X][B][X]   with X = 64 / bytes_per_scalar
// A token's key row is cut into 64-byte pieces so that one wave-wide 16-byte
// load (1 KiB) covers piece i of 16 consecutive tokens, giving each group of 4
// lanes one whole token piece.  After all pieces are loaded every lane holds a
// quarter of one token's key; a QK dot product then needs only a 2-step
// in-quad DPP reduction.  Values keep plain rows: a lane keeps the same 16
// bytes of output dimensions for every token it visits, so the PV product
// accumulates in registers with no per-token cross-lane traffic.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = kWave * kWaves;  // 256
constexpr int kGroup = 16;                // tokens one wave handles per step
constexpr int kLogitFloats = 4096;        // LDS floats for one chunk's logits

typedef short bf16x2_t __attribute__((ext_vector_type(2)));

struct F32 {
  static constexpr int kItem = 4;
};
struct BF16 {
  static constexpr int kItem = 2;
};

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }

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

// Widen 16 bytes of stored values to fp32.
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

// In-quad butterfly steps (DPP quad_perm [1,0,3,2] and [2,3,0,1]).
__device__ __forceinline__ float quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}

struct AttnArgs {
  float* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_acc;  // [S][H_q][max_parts][d]
  float* ws_m;    // [S][H_q][max_parts]   running max, log2 domain
  float* ws_l;    // [S][H_q][max_parts]   sum of exp2(s - m)
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t max_context_len;
  int32_t partition_size;  // tokens, multiple of block_size
  int32_t max_parts;
  float scale_log2;  // scale * log2(e): logits are kept in the exp2 domain
};

// Number of partitions of sequence `seq`, 0 when its length is invalid.
__device__ __forceinline__ int seq_parts(const AttnArgs& a, int n_raw, bool* bad) {
  *bad = n_raw < 0 || n_raw > a.max_context_len ||
         static_cast<int64_t>(n_raw) > static_cast<int64_t>(a.max_blocks) * a.block_size;
  if (*bad || n_raw == 0) return 1;
  return (n_raw + a.partition_size - 1) / a.partition_size;
}

// Shared-memory state of one attention workgroup.
template <int G>
struct AttnShared {
  float logit[kLogitFloats];
  int32_t ids[kLogitFloats / G / kGroup];
  float wmax[kWaves][G];
  float wsum[kWaves][G];
  float mfin[G];
  int bad;
};

// Per-instantiation geometry.
template <class DT, int D, int G>
struct Geo {
  static constexpr int kItem = DT::kItem;
  static constexpr int R = D * kItem;        // bytes of one token row
  static constexpr int NP = R / 64;          // 64-byte key pieces per row
  static constexpr int LR = R / 16;          // lanes covering one value row
  static constexpr int TPL = kWave / LR;     // value rows per wave load
  static constexpr int NLV = kGroup / TPL;   // value loads per 16-token group
  static constexpr int E = 16 / kItem;       // scalars per 16 bytes
  static constexpr int C = kLogitFloats / G; // tokens per chunk
  static_assert(R % 64 == 0 && kGroup % TPL == 0, "unsupported row size");
  static_assert(kWaves * G * D <= kLogitFloats, "reduction buffer does not fit");
};

// Stage the chunk's block ids in LDS; returns false (after a barrier) if one
// is out of range.
template <int G>
__device__ __forceinline__ bool stage_ids(AttnShared<G>& sh, const int32_t* bt, int blk0, int nblk, int num_blocks) {
  if (threadIdx.x == 0) sh.bad = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < nblk; i += kThreads) {
    int id = bt[blk0 + i];
    if (static_cast<unsigned>(id) >= static_cast<unsigned>(num_blocks)) {
      sh.bad = 1;
      id = 0;
    }
    sh.ids[i] = id;
  }
  __syncthreads();
  return sh.bad == 0;
}

// Phase 1 over one chunk: logits of the wave's 16-token groups (exp2 domain,
// -inf past tok_end) into LDS, and this wave's per-head maxima into sh.wmax.
template <class DT, int D, int G>
__device__ __forceinline__ void qk_phase(const AttnArgs& a, AttnShared<G>& sh, const uint4 (&qr)[G][Geo<DT, D, G>::NP],
                                         const char* kbase, int kvh, int c0, int ngroups, int tok_end) {
  using Gm = Geo<DT, D, G>;
  constexpr int NP = Gm::NP;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int qd = lane >> 2;
  const int jq = lane & 3;
  const int B = a.block_size;
  const size_t tile = static_cast<size_t>(B) * Gm::R;
  auto load = [&](uint4 (&kr)[NP], int g) {
    const int t0 = g * kGroup;
    const char* kt = kbase + (static_cast<size_t>(sh.ids[t0 / B]) * a.num_kv_heads + kvh) * tile;
    const int row = t0 % B + qd;
#pragma unroll
    for (int i = 0; i < NP; ++i)
      kr[i] = *reinterpret_cast<const uint4*>(kt + static_cast<size_t>(i) * B * 64 + row * 64 + jq * 16);
  };
  float lmax[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lmax[h] = -INFINITY;
  uint4 kcur[NP];
  if (wave < ngroups) load(kcur, wave);
  for (int g = wave; g < ngroups; g += kWaves) {
    uint4 knext[NP];
    if (g + kWaves < ngroups) load(knext, g + kWaves);
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x = 0.0f;
#pragma unroll
      for (int i = 0; i < NP; ++i) x = dot16(DT{}, qr[h][i], kcur[i], x);
      s[h] = x;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] += quad_xor1(s[h]);
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] += quad_xor2(s[h]);
    const int t0 = g * kGroup;
    const bool valid = c0 + t0 + qd < tok_end;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s[h] = valid ? s[h] * a.scale_log2 : -INFINITY;
      lmax[h] = fmaxf(lmax[h], s[h]);
    }
    if (jq == 0) {
      float* dst = sh.logit + (t0 + qd) * G;
#pragma unroll
      for (int h = 0; h < G; ++h) dst[h] = s[h];
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) kcur[i] = knext[i];
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int off = 4; off < kWave; off <<= 1) lmax[h] = fmaxf(lmax[h], __shfl_xor(lmax[h], off));
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) sh.wmax[wave][h] = lmax[h];
  }
}

// Logits -> probabilities (in place) against the running maximum `m` of this
// thread's head; returns the thread's partial sum.
template <int G>
__device__ __forceinline__ float exp_pass(AttnShared<G>& sh, int nlog, float m) {
  float l = 0.0f;
  for (int e = threadIdx.x; e < nlog; e += kThreads) {
    const float p = __builtin_amdgcn_exp2f(sh.logit[e] - m);
    sh.logit[e] = p;
    l += p;
  }
  return l;
}

// Phase 2 over one chunk: acc[h][e] += p[t][h] * V[t][e] for the wave's groups.
template <class DT, int D, int G>
__device__ __forceinline__ void pv_phase(const AttnArgs& a, AttnShared<G>& sh,
                                         float (&acc)[G][Geo<DT, D, G>::E], const char* vbase, int kvh, int c0,
                                         int ngroups, int tok_end) {
  using Gm = Geo<DT, D, G>;
  constexpr int NLV = Gm::NLV, TPL = Gm::TPL, E = Gm::E, R = Gm::R;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int cv = lane % Gm::LR;
  const int rv = lane / Gm::LR;
  const int B = a.block_size;
  const size_t tile = static_cast<size_t>(B) * R;
  auto load = [&](uint4 (&vr)[NLV], int g) {
    const int t0 = g * kGroup;
    const char* vt = vbase + (static_cast<size_t>(sh.ids[t0 / B]) * a.num_kv_heads + kvh) * tile;
#pragma unroll
    for (int k = 0; k < NLV; ++k)
      vr[k] = *reinterpret_cast<const uint4*>(vt + static_cast<size_t>(t0 % B + k * TPL + rv) * R + cv * 16);
  };
  uint4 vcur[NLV];
  if (wave < ngroups) load(vcur, wave);
  for (int g = wave; g < ngroups; g += kWaves) {
    uint4 vnext[NLV];
    if (g + kWaves < ngroups) load(vnext, g + kWaves);
    const int t0 = g * kGroup;
#pragma unroll
    for (int k = 0; k < NLV; ++k) {
      const int tl = t0 + k * TPL + rv;  // chunk-relative token
      if (c0 + tl < tok_end) {
        float v[E];
        widen16(DT{}, vcur[k], v);
        const float* pp = sh.logit + tl * G;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = pp[h];
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p, v[e], acc[h][e]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NLV; ++k) vcur[k] = vnext[k];
  }
}

// Combine lanes and waves; write the output rows (single partition) or the
// partition's (acc, m, l) partials.
template <class DT, int D, int G>
__device__ __forceinline__ void finish(const AttnArgs& a, AttnShared<G>& sh, float (&acc)[G][Geo<DT, D, G>::E],
                                       float l_part, float m_mine, bool direct, float* out_rows, int seq, int kvh,
                                       int part) {
  using Gm = Geo<DT, D, G>;
  constexpr int E = Gm::E, LR = Gm::LR;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int cv = lane % LR;
  __syncthreads();  // every wave is done reading sh.logit
#pragma unroll
  for (int off = G; off < kWave; off <<= 1) l_part += __shfl_xor(l_part, off);
  if (lane < G) sh.wsum[wave][lane] = l_part;
  if (tid < G) sh.mfin[tid] = m_mine;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int off = LR; off < kWave; off <<= 1) acc[h][e] += __shfl_xor(acc[h][e], off);
  float* red = sh.logit;  // [kWaves][G][D]
  if (lane < LR) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) red[(wave * G + h) * D + cv * E + e] = acc[h][e];
  }
  __syncthreads();
  const int Hq = a.num_kv_heads * G;
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D;
    const int d = i % D;
    float sa = 0.0f, sl = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      sa += red[(w * G + h) * D + d];
      sl += sh.wsum[w][h];
    }
    if (direct) {
      out_rows[i] = sa / sl;
    } else {
      const size_t row = (static_cast<size_t>(seq) * Hq + static_cast<size_t>(kvh) * G + h) * a.max_parts + part;
      a.ws_acc[row * D + d] = sa;
      if (d == 0) {
        a.ws_m[row] = sh.mfin[h];
        a.ws_l[row] = sl;
      }
    }
  }
}

// Poison the outputs of a workgroup that met an out-of-range block id.
template <int D, int G>
__device__ __forceinline__ void write_nan(const AttnArgs& a, bool direct, float* out_rows, int seq, int kvh, int part) {
  const float nan = __builtin_nanf("");
  const int Hq = a.num_kv_heads * G;
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    if (direct) {
      out_rows[i] = nan;
    } else {
      const size_t row = (static_cast<size_t>(seq) * Hq + static_cast<size_t>(kvh) * G + i / D) * a.max_parts + part;
      a.ws_acc[row * D + i % D] = nan;
      if (i % D == 0) {
        a.ws_m[row] = nan;
        a.ws_l[row] = nan;
      }
    }
  }
}

// One workgroup = (sequence, KV head, context partition).  The partition is
// processed in chunks of C = kLogitFloats / G tokens:
//   phase 1: waves take 16-token groups round-robin, compute the G logits of
//            each token (scaled into the exp2 domain) into LDS and track maxima;
//   softmax: chunk maximum per head, logits -> probabilities in place, partial
//            sums; running state rescaled when a partition spans several chunks;
//   phase 2: the same groups again, accumulating p * V into registers.
// The G query heads of a KV head share every K/V load (GQA grouping).
// MULTI = false is the common case of a partition that fits one chunk: the
// query registers are dead before the accumulators are live, which keeps the
// register count (and so the occupancy) in check.
template <class DT, int D, int G, bool MULTI>
__global__ __launch_bounds__(kThreads) void paged_decode_kernel(AttnArgs a) {
  using Gm = Geo<DT, D, G>;
  constexpr int NP = Gm::NP, E = Gm::E, C = Gm::C, R = Gm::R;
  __shared__ AttnShared<G> sh;

  const int tid = threadIdx.x;
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
  const int hm = tid % G;  // the head whose probabilities this thread sums
  const int jq = tid & 3;

  const char* qrow = static_cast<const char*>(a.q) + (static_cast<size_t>(seq) * Hq + static_cast<size_t>(kvh) * G) * R;
  const int32_t* bt = a.block_tables + static_cast<size_t>(seq) * a.max_blocks;
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);

  if constexpr (!MULTI) {
    const int cn = tok_end - tok_begin;  // <= C
    const int ngroups = (cn + kGroup - 1) / kGroup;
    if (!stage_ids(sh, bt, tok_begin / B, (cn + B - 1) / B, a.num_blocks)) {
      write_nan<D, G>(a, direct, out_rows, seq, kvh, part);
      return;
    }
    {
      uint4 qr[G][NP];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < NP; ++i) qr[h][i] = *reinterpret_cast<const uint4*>(qrow + h * R + i * 64 + jq * 16);
      qk_phase<DT, D, G>(a, sh, qr, kbase, kvh, tok_begin, ngroups, tok_end);
    }
    __syncthreads();
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m = fmaxf(m, sh.wmax[w][hm]);
    const float l_part = exp_pass(sh, ngroups * kGroup * G, m);
    __syncthreads();
    float acc[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;
    pv_phase<DT, D, G>(a, sh, acc, vbase, kvh, tok_begin, ngroups, tok_end);
    finish<DT, D, G>(a, sh, acc, l_part, m, direct, out_rows, seq, kvh, part);
  } else {
    uint4 qr[G][NP];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < NP; ++i) qr[h][i] = *reinterpret_cast<const uint4*>(qrow + h * R + i * 64 + jq * 16);
    float m_run[G];
    float acc[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m_run[h] = -INFINITY;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = 0.0f;
    }
    float m_mine = -INFINITY;
    float l_part = 0.0f;
    for (int c0 = tok_begin; c0 < tok_end; c0 += C) {
      const int cn = min(C, tok_end - c0);
      const int ngroups = (cn + kGroup - 1) / kGroup;
      __syncthreads();  // the previous chunk is done with sh.logit and sh.ids
      if (!stage_ids(sh, bt, c0 / B, (cn + B - 1) / B, a.num_blocks)) {
        write_nan<D, G>(a, direct, out_rows, seq, kvh, part);
        return;
      }
      qk_phase<DT, D, G>(a, sh, qr, kbase, kvh, c0, ngroups, tok_end);
      __syncthreads();
      float m_new[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = m_run[h];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sh.wmax[w][h]);
        m_new[h] = mx;
      }
      float m_new_mine = m_mine;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) m_new_mine = fmaxf(m_new_mine, sh.wmax[w][hm]);
      if (c0 != tok_begin) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new[h]);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
        }
        l_part *= __builtin_amdgcn_exp2f(m_mine - m_new_mine);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) m_run[h] = m_new[h];
      m_mine = m_new_mine;
      l_part += exp_pass(sh, ngroups * kGroup * G, m_mine);
      __syncthreads();
      pv_phase<DT, D, G>(a, sh, acc, vbase, kvh, c0, ngroups, tok_end);
    }
    finish<DT, D, G>(a, sh, acc, l_part, m_mine, direct, out_rows, seq, kvh, part);
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

// One thread moves 16 bytes of K and 16 bytes of V for one (token, head).
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(const char* __restrict__ k_new,
                                                                const char* __restrict__ v_new,
                                                                char* __restrict__ k_cache, char* __restrict__ v_cache,
                                                                const int64_t* __restrict__ slots, int32_t num_tokens,
                                                                int32_t num_heads, int32_t block_size, int32_t row_bytes,
                                                                int64_t num_slots) {
  const int chunks = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(num_tokens) * num_heads * chunks;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int c = static_cast<int>(idx % chunks);
    const int64_t th = idx / chunks;  // token * H + head
    const int64_t t = th / num_heads;
    const int h = static_cast<int>(th % num_heads);
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot / block_size;
    const int off = static_cast<int>(slot % block_size);
    const uint4 kv = *reinterpret_cast<const uint4*>(k_new + th * row_bytes + c * 16);
    const uint4 vv = *reinterpret_cast<const uint4*>(v_new + th * row_bytes + c * 16);
    const int piece = (c * 16) / 64;
    const int within = (c * 16) % 64;
    const int64_t tile = blk * num_heads + h;
    *reinterpret_cast<uint4*>(k_cache + ((tile * (row_bytes / 64) + piece) * block_size + off) * 64 + within) = kv;
    *reinterpret_cast<uint4*>(v_cache + (tile * block_size + off) * row_bytes + c * 16) = vv;
  }
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

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int item_size(int32_t kv_dtype) { return kv_dtype == PKV_F32 ? 4 : kv_dtype == PKV_BF16 ? 2 : 0; }

struct Plan {
  int32_t P;          // effective partition size
  int32_t max_parts;  // partitions of the longest sequence
  size_t off_m, off_l, bytes;
};

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

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
  if (a.partition_size <= kLogitFloats / G)
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
  const int row_bytes = head_dim * item;
  const int64_t total = static_cast<int64_t>(num_tokens) * num_kv_heads * (row_bytes / 16);
  const int64_t want = ceil_div64(total, 256);
  const unsigned grid = static_cast<unsigned>(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const char*>(k_new),
                     static_cast<const char*>(v_new), static_cast<char*>(k_cache), static_cast<char*>(v_cache), slots,
                     num_tokens, num_kv_heads, block_size, row_bytes,
                     static_cast<int64_t>(num_blocks) * block_size);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t n_pairs, int32_t num_blocks,
                           int64_t block_bytes, hipStream_t stream) {
  if (n_pairs < 0 || num_blocks <= 0 || block_bytes <= 0 || block_bytes % 16) return PKV_ERR_INVALID_ARG;
  if (n_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_INVALID_ARG;
  const int64_t n16 = block_bytes / 16;
  const int64_t splits = ceil_div64(n16, 256);
  const unsigned z = static_cast<unsigned>(splits < 16 ? splits : 16);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n_pairs, 2, z), dim3(256), 0, stream, static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), pairs, num_blocks, block_bytes);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

size_t pkv_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t block_size,
                                     int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_context_len < 0 ||
      partition_size < 0)
    return 0;
  return make_plan(num_seqs, num_q_heads, head_dim, block_size, max_context_len, partition_size).bytes;
}

}  // extern "C"

namespace {

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
  a.scale_log2 = scale * 1.4426950408889634f;

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

extern "C" {

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

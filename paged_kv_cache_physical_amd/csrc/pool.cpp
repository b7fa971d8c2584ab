// Host block pool: fixed-size blocks, per-sequence block tables, on-demand
// allocation, refcounted sharing and copy-on-write.
//
// [P2] "core idea" items 1-4 and key technical points 1-3; [P3] section 3
// (sharing, refcounts tied to request lifetime, copy-on-write of a shared block
// that is not full, reclamation on finish/cancel); [P4] beam-search sharing.
//
// Free blocks sit in a FIFO ring: allocation takes the head, release appends
// to the tail.  An append batch is checked first (blocks needed, including the
// copies that refcounts will force) and only then applied, so a failure leaves
// the pool untouched.

#include <algorithm>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"

namespace {

struct Seq {
  std::vector<int32_t> table;
  int64_t length = 0;
  bool live = false;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

struct pkv_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ring;  // capacity num_blocks
  int64_t head = 0;
  int64_t count = 0;
  std::vector<int32_t> refcount;
  std::vector<Seq> seqs;  // index = sequence id
  int64_t live = 0;

  int32_t pop() {
    int32_t b = ring[head];
    head = (head + 1) % num_blocks;
    --count;
    refcount[b] = 1;
    return b;
  }
  void push(int32_t b) {
    ring[(head + count) % num_blocks] = b;
    ++count;
  }
  Seq* get(int32_t id) {
    if (id < 0 || static_cast<size_t>(id) >= seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
  const Seq* get(int32_t id) const {
    if (id < 0 || static_cast<size_t>(id) >= seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
};

extern "C" {

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_OUT_OF_BLOCKS: return "out of blocks";
    case PKV_ERR_NO_SUCH_SEQ: return "no such sequence";
    case PKV_ERR_REFCOUNT: return "pool invariant broken";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PKV_ERR_HIP: return "HIP launch error";
    case PKV_ERR_WORKSPACE: return "attention workspace missing or too small";
    default: return "unknown status";
  }
}

int32_t pkv_abi_version(void) { return 4; }

pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                           pkv_pool** out) {
  if (!out || num_blocks <= 0 || block_size <= 0) return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return PKV_ERR_INVALID_ARG;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->ring.resize(num_blocks);
  p->refcount.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        return PKV_ERR_INVALID_ARG;
      }
      seen[b] = 1;
      p->ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->ring[i] = i;
  }
  p->head = 0;
  p->count = num_blocks;
  *out = p;
  return PKV_OK;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

pkv_status pkv_seq_create(pkv_pool* pool, int32_t* out_seq) {
  if (!pool || !out_seq) return PKV_ERR_INVALID_ARG;
  if (pool->seqs.size() >= static_cast<size_t>(INT32_MAX)) return PKV_ERR_INVALID_ARG;
  pool->seqs.emplace_back();
  pool->seqs.back().live = true;
  ++pool->live;
  *out_seq = static_cast<int32_t>(pool->seqs.size() - 1);
  return PKV_OK;
}

pkv_status pkv_seq_fork(pkv_pool* pool, int32_t parent, int32_t* out_child) {
  if (!pool || !out_child) return PKV_ERR_INVALID_ARG;
  if (!pool->get(parent)) return PKV_ERR_NO_SUCH_SEQ;
  if (pool->seqs.size() >= static_cast<size_t>(INT32_MAX)) return PKV_ERR_INVALID_ARG;
  Seq child;
  child.table = pool->seqs[parent].table;  // copy before emplace may reallocate
  child.length = pool->seqs[parent].length;
  child.live = true;
  for (int32_t b : child.table) ++pool->refcount[b];
  pool->seqs.push_back(std::move(child));
  ++pool->live;
  *out_child = static_cast<int32_t>(pool->seqs.size() - 1);
  return PKV_OK;
}

pkv_status pkv_seq_free(pkv_pool* pool, int32_t seq) {
  if (!pool) return PKV_ERR_INVALID_ARG;
  Seq* s = pool->get(seq);
  if (!s) return PKV_ERR_NO_SUCH_SEQ;
  for (int32_t b : s->table) {
    if (--pool->refcount[b] == 0) pool->push(b);
  }
  s->table.clear();
  s->table.shrink_to_fit();
  s->length = 0;
  s->live = false;
  --pool->live;
  return PKV_OK;
}

pkv_status pkv_append_tokens(pkv_pool* pool, const int32_t* seqs, const int32_t* counts, int32_t n,
                             int64_t* out_slots, int64_t slots_cap, int32_t* out_cow_pairs,
                             int32_t cow_cap, int32_t* out_n_cow) {
  if (!pool || n < 0 || !out_n_cow) return PKV_ERR_INVALID_ARG;
  *out_n_cow = 0;
  if (n == 0) return PKV_OK;
  if (!seqs || !counts) return PKV_ERR_INVALID_ARG;
  const int64_t B = pool->block_size;

  // Pass 1: validate (argument errors first, then unknown ids), then count
  // what the batch needs.
  std::unordered_map<int32_t, int32_t> listed;
  for (int32_t i = 0; i < n; ++i) {
    if (counts[i] < 0 || !listed.emplace(seqs[i], i).second) return PKV_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (!pool->get(seqs[i])) return PKV_ERR_NO_SUCH_SEQ;
  }
  std::unordered_map<int32_t, int32_t> dropped;  // refcount drops from copies earlier in the batch
  int64_t total_slots = 0, need = 0;
  int32_t cows = 0;
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = pool->get(seqs[i]);
    const int64_t L = s->length, c = counts[i];
    total_slots += c;
    if (c == 0) continue;
    if (L % B != 0) {
      const int32_t last = s->table.back();
      auto it = dropped.find(last);
      const int32_t rc = pool->refcount[last] - (it == dropped.end() ? 0 : it->second);
      if (rc > 1) {
        ++need;
        ++cows;
        ++dropped[last];
      }
    }
    need += ceil_div(L + c, B) - ceil_div(L, B);
  }
  if (total_slots > 0 && (!out_slots || slots_cap < total_slots)) return PKV_ERR_INVALID_ARG;
  if (cows > 0 && (!out_cow_pairs || cow_cap < cows)) {
    *out_n_cow = cows;
    return PKV_ERR_INVALID_ARG;
  }
  if (need > pool->count) return PKV_ERR_OUT_OF_BLOCKS;

  // Pass 2: apply.
  int64_t k = 0;
  int32_t npairs = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = pool->seqs[seqs[i]];
    const int64_t L = s.length, c = counts[i];
    if (c == 0) continue;
    if (L % B != 0) {
      const int32_t last = s.table.back();
      if (pool->refcount[last] > 1) {
        const int32_t fresh = pool->pop();
        out_cow_pairs[2 * npairs] = last;
        out_cow_pairs[2 * npairs + 1] = fresh;
        ++npairs;
        --pool->refcount[last];
        s.table.back() = fresh;
      }
    }
    for (int64_t p = L; p < L + c; ++p) {
      if (p % B == 0) s.table.push_back(pool->pop());
      out_slots[k++] = static_cast<int64_t>(s.table[p / B]) * B + p % B;
    }
    s.length = L + c;
  }
  *out_n_cow = npairs;
  return PKV_OK;
}

pkv_status pkv_block_tables(const pkv_pool* pool, const int32_t* seqs, int32_t n, int32_t max_blocks,
                            int32_t* out_tables, int32_t* out_context_lens) {
  if (!pool || n < 0 || max_blocks < 0) return PKV_ERR_INVALID_ARG;
  if (n == 0) return PKV_OK;
  if (!seqs || !out_tables || !out_context_lens) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = pool->get(seqs[i]);
    if (!s) return PKV_ERR_NO_SUCH_SEQ;
    if (s->table.size() > static_cast<size_t>(max_blocks) || s->length > INT32_MAX) return PKV_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = pool->get(seqs[i]);
    int32_t* row = out_tables + static_cast<int64_t>(i) * max_blocks;
    const size_t nb = s->table.size();
    if (nb) std::memcpy(row, s->table.data(), nb * sizeof(int32_t));
    std::fill(row + nb, row + max_blocks, -1);
    out_context_lens[i] = static_cast<int32_t>(s->length);
  }
  return PKV_OK;
}

pkv_status pkv_seq_info(const pkv_pool* pool, int32_t seq, int32_t* out_len, int32_t* out_num_blocks) {
  if (!pool) return PKV_ERR_INVALID_ARG;
  const Seq* s = pool->get(seq);
  if (!s) return PKV_ERR_NO_SUCH_SEQ;
  if (out_len) *out_len = static_cast<int32_t>(s->length);
  if (out_num_blocks) *out_num_blocks = static_cast<int32_t>(s->table.size());
  return PKV_OK;
}

pkv_status pkv_pool_stats(const pkv_pool* pool, pkv_stats* out) {
  if (!pool || !out) return PKV_ERR_INVALID_ARG;
  pkv_stats st{};
  st.num_blocks = pool->num_blocks;
  st.free_blocks = pool->count;
  for (int32_t r : pool->refcount) {
    if (r > 0) ++st.used_blocks;
    st.sum_refcount += r;
  }
  st.num_seqs = pool->live;
  for (const Seq& s : pool->seqs) {
    if (!s.live) continue;
    st.logical_tokens += s.length;
    st.logical_blocks += static_cast<int64_t>(s.table.size());
  }
  st.allocated_slots = st.used_blocks * pool->block_size;
  st.table_bytes = 4 * st.logical_blocks;
  *out = st;
  return PKV_OK;
}

int32_t pkv_block_refcount(const pkv_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->num_blocks) return -1;
  return pool->refcount[block];
}

pkv_status pkv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* out_n) {
  if (!pool || !out_n) return PKV_ERR_INVALID_ARG;
  *out_n = static_cast<int32_t>(pool->count);
  if (cap < pool->count || (pool->count > 0 && !out)) return PKV_ERR_INVALID_ARG;
  for (int64_t i = 0; i < pool->count; ++i) out[i] = pool->ring[(pool->head + i) % pool->num_blocks];
  return PKV_OK;
}

pkv_status pkv_pool_validate(const pkv_pool* pool) {
  if (!pool) return PKV_ERR_INVALID_ARG;
  const int32_t NB = pool->num_blocks;
  std::vector<int64_t> held(NB, 0);
  for (const Seq& s : pool->seqs) {
    if (!s.live) continue;
    if (static_cast<int64_t>(s.table.size()) != ceil_div(s.length, pool->block_size)) return PKV_ERR_REFCOUNT;
    for (int32_t b : s.table) {
      if (b < 0 || b >= NB) return PKV_ERR_REFCOUNT;
      ++held[b];
    }
  }
  int64_t used = 0;
  for (int32_t b = 0; b < NB; ++b) {
    if (held[b] != pool->refcount[b]) return PKV_ERR_REFCOUNT;
    if (held[b] > 0) ++used;
  }
  std::vector<char> in_free(NB, 0);
  for (int64_t i = 0; i < pool->count; ++i) {
    const int32_t b = pool->ring[(pool->head + i) % NB];
    if (b < 0 || b >= NB || in_free[b] || pool->refcount[b] != 0) return PKV_ERR_REFCOUNT;
    in_free[b] = 1;
  }
  if (used + pool->count != NB) return PKV_ERR_REFCOUNT;
  return PKV_OK;
}

}  // extern "C"

// Host block pool: fixed-size blocks, per-sequence block tables, on-demand
// allocation, refcounted sharing and copy-on-write.
//
// [P2] "core idea" items 1-4 and key technical points 1-3; [P3] section 3
// (sharing, refcounts tied to request lifetime, copy-on-write of a shared block
// that is not full, reclamation on finish/cancel); [P4] beam-search sharing.
//
// Free blocks sit in a FIFO queue: allocation takes the head, release appends
// to the tail.  An append batch is checked first (blocks needed, including the
// copies that refcounts will force) and only then applied, so a failure leaves
// the pool untouched.
//
// Preemption by swapping ([P2] section 4, "first come first served plus
// preemption"; [P4] "Preemption"): an optional host tier with its own FIFO
// ring of host block ids.  A swap moves a whole sharing group between the
// tiers; a block keeps its refcount, and the sequences' tables are renamed.
//
// Automatic prefix caching ([P4] the note on identical KV blocks and the
// prefix-caching paragraph; [P2] section 3): a full block written with known
// token ids is registered under a key chained over every token before it and
// its own; a new prompt maps its longest run of registered leading blocks
// instead of computing them again.  Freed blocks stay findable until they are
// taken for new use (oldest freed first) or moved to the host tier.

#include <algorithm>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"

namespace {

struct Seq {
  std::vector<int32_t> table;  // block ids of the sequence's tier
  int64_t length = 0;
  bool live = false;
  bool on_host = false;  // swapped out
  bool tracked = true;    // every token so far came with its id
  uint64_t last_key = 0;  // key of the last full block (0 before the first)
  std::vector<int32_t> partial;  // ids of the tokens in the partly filled last block
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// One tier's blocks: refcounts and the FIFO queue of free ids, kept as a
// doubly linked list through the block ids so that a cached block found again
// can leave the queue from wherever it sits.
struct Tier {
  int32_t num_blocks = 0;
  std::vector<int32_t> next, prev;  // queue links; -1 past either end
  std::vector<char> queued;
  int32_t head = -1, tail = -1;
  int64_t count = 0;
  std::vector<int32_t> refcount;

  void reset(int32_t n) {
    num_blocks = n;
    next.assign(n, -1);
    prev.assign(n, -1);
    queued.assign(n, 0);
    head = tail = -1;
    count = 0;
    refcount.assign(n, 0);
  }
  void push(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    queued[b] = 1;
    ++count;
  }
  void remove(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    queued[b] = 0;
    --count;
  }
  int32_t pop() {
    const int32_t b = head;
    remove(b);
    refcount[b] = 1;
    return b;
  }
};

// FNV-1a, 64-bit (Fowler, Noll, Vo): xor in each byte, multiply by the prime.
constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

uint64_t fnv_bytes(uint64_t h, uint64_t v, int nbytes) {
  for (int i = 0; i < nbytes; ++i) {
    h ^= (v >> (8 * i)) & 0xFF;
    h *= kFnvPrime;
  }
  return h;
}

// Key of a full block: the parent block's key as 8 little-endian bytes, then
// the block's token ids as 4-byte little-endian integers.
uint64_t block_key(uint64_t parent, const int32_t* tokens, int64_t B) {
  uint64_t h = fnv_bytes(kFnvOffset, parent, 8);
  for (int64_t i = 0; i < B; ++i) h = fnv_bytes(h, static_cast<uint32_t>(tokens[i]), 4);
  return h;
}

}  // namespace

struct pkv_pool {
  int32_t block_size = 0;
  Tier dev;
  Tier host;
  std::vector<Seq> seqs;  // index = sequence id
  int64_t live = 0;
  // Prefix cache: key -> device block, and per device block its key, parent
  // key and token ids (tokens stored B per block, allocated on first use).
  std::unordered_map<uint64_t, int32_t> cached;
  std::vector<char> keyed;
  std::vector<uint64_t> bkey, bparent;
  std::vector<int32_t> btokens;
  // Scratch of pkv_append_tokens, kept between calls: a stamp per sequence id
  // (listed in this batch), and per device block the copies earlier in the
  // batch have taken from its refcount.
  std::vector<uint32_t> seq_stamp;
  uint32_t stamp = 0;
  std::vector<int32_t> blk_drop;
  std::vector<int32_t> blk_touched;

  Seq* get(int32_t id) {
    if (id < 0 || static_cast<size_t>(id) >= seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
  const Seq* get(int32_t id) const {
    if (id < 0 || static_cast<size_t>(id) >= seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
  // A block leaving the device tier's pool of findable blocks loses its key.
  void forget(int32_t b) {
    if (!keyed[b]) return;
    auto it = cached.find(bkey[b]);
    if (it != cached.end() && it->second == b) cached.erase(it);
    keyed[b] = 0;
  }
  // Taking a free device block for new use evicts its key.
  int32_t pop_dev() {
    const int32_t b = dev.pop();
    forget(b);
    return b;
  }
  bool matches(int32_t b, uint64_t key, uint64_t parent, const int32_t* tokens) const {
    return keyed[b] && bkey[b] == key && bparent[b] == parent &&
           std::equal(tokens, tokens + block_size, btokens.begin() + static_cast<int64_t>(b) * block_size);
  }
  // Extend s's key chain by the ids just appended (the last ids.size()
  // positions), registering each block they fill whose key is new.
  void track(Seq& s, const int32_t* ids, int64_t c) {
    if (!s.tracked) return;
    const int64_t B = block_size;
    int64_t pos = s.length - c;
    for (int64_t i = 0; i < c; ++i, ++pos) {
      s.partial.push_back(ids[i]);
      if (static_cast<int64_t>(s.partial.size()) < B) continue;
      const int32_t b = s.table[pos / B];
      const uint64_t key = block_key(s.last_key, s.partial.data(), B);
      if (cached.find(key) == cached.end()) {
        if (btokens.empty()) btokens.resize(static_cast<size_t>(dev.num_blocks) * B);
        cached.emplace(key, b);
        keyed[b] = 1;
        bkey[b] = key;
        bparent[b] = s.last_key;
        std::copy(s.partial.begin(), s.partial.end(), btokens.begin() + static_cast<int64_t>(b) * B);
      }
      s.last_key = key;
      s.partial.clear();
    }
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
    case PKV_ERR_SWAPPED: return "sequence is on the other tier (swapped out, or not)";
    default: return "unknown status";
  }
}

int32_t pkv_abi_version(void) { return 11; }

pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                           pkv_pool** out) {
  if (!out || num_blocks <= 0 || block_size <= 0) return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return PKV_ERR_INVALID_ARG;
  p->block_size = block_size;
  p->dev.reset(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        return PKV_ERR_INVALID_ARG;
      }
      seen[b] = 1;
    }
    for (int32_t i = 0; i < num_blocks; ++i) p->dev.push(free_order[i]);
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->dev.push(i);
  }
  p->keyed.assign(num_blocks, 0);
  p->bkey.assign(num_blocks, 0);
  p->bparent.assign(num_blocks, 0);
  *out = p;
  return PKV_OK;
}

pkv_status pkv_pool_set_host_blocks(pkv_pool* pool, int32_t num_host_blocks) {
  if (!pool || num_host_blocks < 0) return PKV_ERR_INVALID_ARG;
  for (const Seq& s : pool->seqs) {
    if (s.live && s.on_host) return PKV_ERR_INVALID_ARG;
  }
  pool->host.reset(num_host_blocks);
  for (int32_t i = 0; i < num_host_blocks; ++i) pool->host.push(i);
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
  if (pool->seqs[parent].on_host) return PKV_ERR_SWAPPED;
  if (pool->seqs.size() >= static_cast<size_t>(INT32_MAX)) return PKV_ERR_INVALID_ARG;
  Seq child;
  child.table = pool->seqs[parent].table;  // copy before emplace may reallocate
  child.length = pool->seqs[parent].length;
  child.tracked = pool->seqs[parent].tracked;
  child.last_key = pool->seqs[parent].last_key;
  child.partial = pool->seqs[parent].partial;
  child.live = true;
  for (int32_t b : child.table) ++pool->dev.refcount[b];
  pool->seqs.push_back(std::move(child));
  ++pool->live;
  *out_child = static_cast<int32_t>(pool->seqs.size() - 1);
  return PKV_OK;
}

pkv_status pkv_seq_free(pkv_pool* pool, int32_t seq) {
  if (!pool) return PKV_ERR_INVALID_ARG;
  Seq* s = pool->get(seq);
  if (!s) return PKV_ERR_NO_SUCH_SEQ;
  Tier& tier = s->on_host ? pool->host : pool->dev;
  for (int32_t b : s->table) {
    if (--tier.refcount[b] == 0) tier.push(b);
  }
  s->table.clear();
  s->table.shrink_to_fit();
  s->partial.clear();
  s->partial.shrink_to_fit();
  s->length = 0;
  s->live = false;
  s->on_host = false;
  --pool->live;
  return PKV_OK;
}

pkv_status pkv_append_tokens(pkv_pool* pool, const int32_t* seqs, const int32_t* counts, int32_t n,
                             const int32_t* token_ids, int64_t* out_slots, int64_t slots_cap,
                             int32_t* out_cow_pairs, int32_t cow_cap, int32_t* out_n_cow) {
  if (!pool || n < 0 || !out_n_cow) return PKV_ERR_INVALID_ARG;
  *out_n_cow = 0;
  if (n == 0) return PKV_OK;
  if (!seqs || !counts) return PKV_ERR_INVALID_ARG;
  const int64_t B = pool->block_size;

  // Pass 1: validate (argument errors first, then unknown ids), then count
  // what the batch needs.  Duplicates are found with the stamp of this call;
  // ids that are not sequence ids of the pool are compared among themselves.
  if (pool->seq_stamp.size() < pool->seqs.size()) pool->seq_stamp.resize(pool->seqs.size(), 0);
  if (++pool->stamp == 0) {
    std::fill(pool->seq_stamp.begin(), pool->seq_stamp.end(), 0);
    pool->stamp = 1;
  }
  std::vector<int32_t> strays;
  for (int32_t i = 0; i < n; ++i) {
    if (counts[i] < 0) return PKV_ERR_INVALID_ARG;
    const int32_t id = seqs[i];
    if (id >= 0 && static_cast<size_t>(id) < pool->seq_stamp.size()) {
      if (pool->seq_stamp[id] == pool->stamp) return PKV_ERR_INVALID_ARG;
      pool->seq_stamp[id] = pool->stamp;
    } else {
      strays.push_back(id);
    }
  }
  if (strays.size() > 1) {
    std::sort(strays.begin(), strays.end());
    if (std::adjacent_find(strays.begin(), strays.end()) != strays.end()) return PKV_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (!pool->get(seqs[i])) return PKV_ERR_NO_SUCH_SEQ;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (pool->seqs[seqs[i]].on_host) return PKV_ERR_SWAPPED;
  }
  if (pool->blk_drop.size() < static_cast<size_t>(pool->dev.num_blocks)) pool->blk_drop.assign(pool->dev.num_blocks, 0);
  int64_t total_slots = 0, need = 0;
  int32_t cows = 0;
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = pool->get(seqs[i]);
    const int64_t L = s->length, c = counts[i];
    total_slots += c;
    if (c == 0) continue;
    if (L % B != 0) {
      const int32_t last = s->table.back();
      if (pool->dev.refcount[last] - pool->blk_drop[last] > 1) {  // net of copies earlier in the batch
        ++need;
        ++cows;
        if (pool->blk_drop[last]++ == 0) pool->blk_touched.push_back(last);
      }
    }
    need += ceil_div(L + c, B) - ceil_div(L, B);
  }
  for (int32_t b : pool->blk_touched) pool->blk_drop[b] = 0;
  pool->blk_touched.clear();
  if (total_slots > 0 && (!out_slots || slots_cap < total_slots)) return PKV_ERR_INVALID_ARG;
  if (cows > 0 && (!out_cow_pairs || cow_cap < cows)) {
    *out_n_cow = cows;
    return PKV_ERR_INVALID_ARG;
  }
  if (need > pool->dev.count) return PKV_ERR_OUT_OF_BLOCKS;

  // Pass 2: apply.
  int64_t k = 0;
  int32_t npairs = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = pool->seqs[seqs[i]];
    const int64_t L = s.length, c = counts[i];
    if (c == 0) continue;
    if (L % B != 0) {
      const int32_t last = s.table.back();
      if (pool->dev.refcount[last] > 1) {
        const int32_t fresh = pool->pop_dev();
        out_cow_pairs[2 * npairs] = last;
        out_cow_pairs[2 * npairs + 1] = fresh;
        ++npairs;
        --pool->dev.refcount[last];
        s.table.back() = fresh;
      } else {
        pool->forget(last);  // written in place: a key kept from before a rollback no longer holds
      }
    }
    for (int64_t p = L; p < L + c; ++p) {
      if (p % B == 0) s.table.push_back(pool->pop_dev());
      out_slots[k++] = static_cast<int64_t>(s.table[p / B]) * B + p % B;
    }
    s.length = L + c;
  }
  // Pass 3: prefix keys, after every block of the batch has been taken (a
  // taken block's key is gone before any new key is registered).
  int64_t t = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = pool->seqs[seqs[i]];
    const int64_t c = counts[i];
    if (c == 0) continue;
    if (token_ids) {
      pool->track(s, token_ids + t, c);
    } else {
      s.tracked = false;
      s.partial.clear();
    }
    t += c;
  }
  *out_n_cow = npairs;
  return PKV_OK;
}

pkv_status pkv_seq_truncate(pkv_pool* pool, int32_t seq, int32_t new_len) {
  if (!pool) return PKV_ERR_INVALID_ARG;
  Seq* s = pool->get(seq);
  if (!s) return PKV_ERR_NO_SUCH_SEQ;
  if (s->on_host) return PKV_ERR_SWAPPED;
  if (new_len < 0 || new_len > s->length) return PKV_ERR_INVALID_ARG;
  if (new_len == s->length) return PKV_OK;
  const size_t keep = static_cast<size_t>(ceil_div(new_len, pool->block_size));
  for (size_t i = keep; i < s->table.size(); ++i) {
    const int32_t b = s->table[i];
    if (--pool->dev.refcount[b] == 0) pool->dev.push(b);
  }
  s->table.resize(keep);
  s->length = new_len;
  s->tracked = false;
  s->partial.clear();
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
    if (s->on_host) return PKV_ERR_SWAPPED;
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

pkv_status pkv_seq_table(const pkv_pool* pool, int32_t seq, int32_t* out, int32_t cap, int32_t* out_n,
                         int32_t* out_on_host) {
  if (!pool || !out_n) return PKV_ERR_INVALID_ARG;
  const Seq* s = pool->get(seq);
  if (!s) return PKV_ERR_NO_SUCH_SEQ;
  const int64_t nb = static_cast<int64_t>(s->table.size());
  *out_n = static_cast<int32_t>(nb);
  if (out_on_host) *out_on_host = s->on_host ? 1 : 0;
  if (cap < nb || (nb > 0 && !out)) return PKV_ERR_INVALID_ARG;
  if (nb) std::memcpy(out, s->table.data(), nb * sizeof(int32_t));
  return PKV_OK;
}

static pkv_status swap_tier(pkv_pool* pool, const int32_t* seqs, int32_t n, int32_t* out_pairs, int32_t pairs_cap,
                            int32_t* out_n_pairs, bool out) {
  if (!pool || n < 0 || !out_n_pairs) return PKV_ERR_INVALID_ARG;
  *out_n_pairs = 0;
  if (n == 0) return PKV_OK;
  if (!seqs) return PKV_ERR_INVALID_ARG;
  std::unordered_map<int32_t, int32_t> listed;
  for (int32_t i = 0; i < n; ++i) {
    if (!listed.emplace(seqs[i], i).second) return PKV_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (!pool->get(seqs[i])) return PKV_ERR_NO_SUCH_SEQ;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (pool->seqs[seqs[i]].on_host == out) return PKV_ERR_SWAPPED;
  }
  Tier& src = out ? pool->dev : pool->host;
  Tier& dst = out ? pool->host : pool->dev;
  // The listed tables' blocks in the order met, and how often the list holds each.
  std::vector<int32_t> met;
  std::unordered_map<int32_t, int32_t> held;
  for (int32_t i = 0; i < n; ++i) {
    for (int32_t b : pool->seqs[seqs[i]].table) {
      auto r = held.emplace(b, 0);
      if (r.second) met.push_back(b);
      ++r.first->second;
    }
  }
  for (int32_t b : met) {
    if (held[b] != src.refcount[b]) return PKV_ERR_INVALID_ARG;  // also held outside the list
  }
  const int64_t k = static_cast<int64_t>(met.size());
  if (k > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if (k > dst.count) return PKV_ERR_OUT_OF_BLOCKS;
  if (k > 0 && (!out_pairs || pairs_cap < k)) {
    *out_n_pairs = static_cast<int32_t>(k);
    return PKV_ERR_INVALID_ARG;
  }
  std::unordered_map<int32_t, int32_t> moved;
  for (int64_t j = 0; j < k; ++j) {
    const int32_t b = met[j];
    if (out) pool->forget(b);  // keys name device blocks only
    const int32_t nb = dst.pop();
    if (!out) pool->forget(nb);
    dst.refcount[nb] = src.refcount[b];
    src.refcount[b] = 0;
    src.push(b);
    moved[b] = nb;
    out_pairs[2 * j] = b;
    out_pairs[2 * j + 1] = nb;
  }
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = pool->seqs[seqs[i]];
    for (int32_t& b : s.table) b = moved[b];
    s.on_host = out;
  }
  *out_n_pairs = static_cast<int32_t>(k);
  return PKV_OK;
}

pkv_status pkv_swap_out(pkv_pool* pool, const int32_t* seqs, int32_t n, int32_t* out_pairs, int32_t pairs_cap,
                        int32_t* out_n_pairs) {
  return swap_tier(pool, seqs, n, out_pairs, pairs_cap, out_n_pairs, true);
}

pkv_status pkv_swap_in(pkv_pool* pool, const int32_t* seqs, int32_t n, int32_t* out_pairs, int32_t pairs_cap,
                       int32_t* out_n_pairs) {
  return swap_tier(pool, seqs, n, out_pairs, pairs_cap, out_n_pairs, false);
}

pkv_status pkv_pool_stats(const pkv_pool* pool, pkv_stats* out) {
  if (!pool || !out) return PKV_ERR_INVALID_ARG;
  pkv_stats st{};
  st.num_blocks = pool->dev.num_blocks;
  st.free_blocks = pool->dev.count;
  for (int32_t r : pool->dev.refcount) {
    if (r > 0) ++st.used_blocks;
    st.sum_refcount += r;
  }
  st.num_seqs = pool->live;
  for (const Seq& s : pool->seqs) {
    if (!s.live) continue;
    if (s.on_host) {
      ++st.swapped_seqs;
      st.swapped_tokens += s.length;
    } else {
      st.logical_tokens += s.length;
      st.logical_blocks += static_cast<int64_t>(s.table.size());
    }
  }
  st.allocated_slots = st.used_blocks * pool->block_size;
  st.table_bytes = 4 * st.logical_blocks;
  st.host_blocks = pool->host.num_blocks;
  st.host_free_blocks = pool->host.count;
  for (int32_t r : pool->host.refcount) {
    if (r > 0) ++st.host_used_blocks;
  }
  st.cached_blocks = static_cast<int64_t>(pool->cached.size());
  for (int32_t b = pool->dev.head; b >= 0; b = pool->dev.next[b]) {
    if (pool->keyed[b]) ++st.cached_free_blocks;
  }
  *out = st;
  return PKV_OK;
}

int32_t pkv_block_refcount(const pkv_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->dev.num_blocks) return -1;
  return pool->dev.refcount[block];
}

int32_t pkv_host_block_refcount(const pkv_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->host.num_blocks) return -1;
  return pool->host.refcount[block];
}

namespace {
pkv_status copy_free_list(const Tier& t, int32_t* out, int32_t cap, int32_t* out_n) {
  if (!out_n) return PKV_ERR_INVALID_ARG;
  *out_n = static_cast<int32_t>(t.count);
  if (cap < t.count || (t.count > 0 && !out)) return PKV_ERR_INVALID_ARG;
  int64_t i = 0;
  for (int32_t b = t.head; b >= 0; b = t.next[b]) out[i++] = b;
  return PKV_OK;
}

// Refcounts equal the holders among live tables of this tier; the free ring
// holds each zero-count block once; used plus free is the capacity.
bool tier_sound(const Tier& t, const std::vector<int64_t>& held) {
  int64_t used = 0;
  for (int32_t b = 0; b < t.num_blocks; ++b) {
    if (held[b] != t.refcount[b]) return false;
    if (held[b] > 0) ++used;
  }
  std::vector<char> in_free(t.num_blocks, 0);
  int64_t walked = 0;
  int32_t before = -1;
  for (int32_t b = t.head; b >= 0; b = t.next[b]) {
    if (b >= t.num_blocks || in_free[b] || !t.queued[b] || t.refcount[b] != 0 || t.prev[b] != before) return false;
    if (++walked > t.count) return false;
    in_free[b] = 1;
    before = b;
  }
  if (before != t.tail) return false;
  for (int32_t b = 0; b < t.num_blocks; ++b) {
    if (t.queued[b] != in_free[b]) return false;
  }
  return walked == t.count && used + t.count == t.num_blocks;
}
}  // namespace

pkv_status pkv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* out_n) {
  if (!pool) return PKV_ERR_INVALID_ARG;
  return copy_free_list(pool->dev, out, cap, out_n);
}

pkv_status pkv_pool_host_free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* out_n) {
  if (!pool) return PKV_ERR_INVALID_ARG;
  return copy_free_list(pool->host, out, cap, out_n);
}

pkv_status pkv_pool_validate(const pkv_pool* pool) {
  if (!pool) return PKV_ERR_INVALID_ARG;
  std::vector<int64_t> held_dev(pool->dev.num_blocks, 0), held_host(pool->host.num_blocks, 0);
  for (const Seq& s : pool->seqs) {
    if (!s.live) continue;
    if (static_cast<int64_t>(s.table.size()) != ceil_div(s.length, pool->block_size)) return PKV_ERR_REFCOUNT;
    std::vector<int64_t>& held = s.on_host ? held_host : held_dev;
    for (int32_t b : s.table) {
      if (b < 0 || static_cast<size_t>(b) >= held.size()) return PKV_ERR_REFCOUNT;
      ++held[b];
    }
  }
  if (!tier_sound(pool->dev, held_dev) || !tier_sound(pool->host, held_host)) return PKV_ERR_REFCOUNT;
  // Prefix cache: the key map and the keyed blocks name each other one to one.
  int64_t keyed = 0;
  for (int32_t b = 0; b < pool->dev.num_blocks; ++b) {
    if (!pool->keyed[b]) continue;
    ++keyed;
    auto it = pool->cached.find(pool->bkey[b]);
    if (it == pool->cached.end() || it->second != b) return PKV_ERR_REFCOUNT;
  }
  if (keyed != static_cast<int64_t>(pool->cached.size())) return PKV_ERR_REFCOUNT;
  return PKV_OK;
}

pkv_status pkv_seq_create_prefixed(pkv_pool* pool, const int32_t* token_ids, int32_t n_tokens, int32_t* out_seq,
                                   int32_t* out_cached_tokens) {
  if (!pool || !out_seq || !out_cached_tokens || n_tokens < 0 || (n_tokens > 0 && !token_ids)) {
    return PKV_ERR_INVALID_ARG;
  }
  const pkv_status st = pkv_seq_create(pool, out_seq);
  if (st != PKV_OK) return st;
  Seq& s = pool->seqs[*out_seq];
  const int64_t B = pool->block_size;
  const int64_t reusable = n_tokens > 0 ? (n_tokens - 1) / B : 0;  // one token is always left to compute
  for (int64_t i = 0; i < reusable; ++i) {
    const int32_t* toks = token_ids + i * B;
    const uint64_t key = block_key(s.last_key, toks, B);
    auto it = pool->cached.find(key);
    if (it == pool->cached.end() || !pool->matches(it->second, key, s.last_key, toks)) break;
    const int32_t b = it->second;
    if (pool->dev.refcount[b] == 0) pool->dev.remove(b);
    ++pool->dev.refcount[b];
    s.table.push_back(b);
    s.length += B;
    s.last_key = key;
  }
  *out_cached_tokens = static_cast<int32_t>(s.length);
  return PKV_OK;
}

pkv_status pkv_pool_cached_blocks(const pkv_pool* pool, uint64_t* out_keys, int32_t* out_blocks, int32_t cap,
                                  int32_t* out_n) {
  if (!pool || !out_n) return PKV_ERR_INVALID_ARG;
  const int64_t n = static_cast<int64_t>(pool->cached.size());
  *out_n = static_cast<int32_t>(n);
  if (cap < n || (n > 0 && (!out_keys || !out_blocks))) return PKV_ERR_INVALID_ARG;
  std::vector<std::pair<uint64_t, int32_t>> all(pool->cached.begin(), pool->cached.end());
  std::sort(all.begin(), all.end());
  for (int64_t i = 0; i < n; ++i) {
    out_keys[i] = all[i].first;
    out_blocks[i] = all[i].second;
  }
  return PKV_OK;
}

}  // extern "C"

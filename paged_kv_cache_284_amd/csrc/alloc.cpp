// Host block allocator behind the pa_alloc_* / pa_seq_* entry points.
//
// Fixed-size blocks handed out on demand, per-sequence block tables, reference counts and
// copy-on-write sharing ("How LLM Inference Serving Works": sections "PagedAttention: Virtual
// Memory for the KV Cache" and "Sharing comes for free"; "LLM serving ... Visual walkthrough":
// "Step 7", "Step 8").  Plain C++17, no HIP.
//
// Policy (the pages fix none; this one makes every table unique): FIFO free list seeded from the
// caller's order, allocations from the head, releases to the tail in table order, batch calls in
// the order given, ids never reused.  Multi-append calls are transactions: every change is
// logged, and running out of blocks rolls the log back so the state is exactly as before
// (released blocks go back to the *head* in reverse order, which restores the FIFO).
//
// Automatic prefix caching ("How LLM Inference Serving Works", "Prefix Caching and Chunked
// Prefill" / "Automatic prefix caching"; "Putting It Together: The Life of a Request").  A
// sequence created with its token ids publishes each full block under a hash of the block's
// tokens chained with the hash of everything before it (the first block's chain starts from a
// per-request salt), so a block matches only when the whole prefix up to it is identical.  A new
// request reuses the longest run of matching leading blocks.  A published block whose last
// reference goes is not freed: it waits, still matchable, on an LRU list and is evicted -- its
// hash dropped -- only when an allocation finds the free list empty.  The hash is 64-bit FNV-1a
// over little-endian bytes; a match also compares the stored tokens and parent hash, so a hash
// collision can never reuse the wrong block.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

namespace {

struct Sequence {
  bool live = false;
  int32_t len = 0;
  std::vector<int32_t> table;
  // prefix caching (sequences created with their token ids)
  bool hashed = false;
  uint64_t salt = 0;
  std::vector<int32_t> tokens;  // token ids known so far
  std::vector<uint64_t> chain;  // chained hash of each full block handled so far
  // swap preemption: while swapped out, the K/V sit in these host swap blocks, in table order
  bool swapped = false;
  std::vector<int32_t> cpu_table;
};

enum class Change : uint8_t { kInPlace, kNewBlock, kCopy };

struct LogEntry {
  int32_t seq;
  Change kind;
  int32_t logical;  // table index touched (kCopy)
  int32_t src;      // block replaced (kCopy)
  bool evicted;     // the new block was taken from the evictable cached blocks
};

constexpr uint64_t kFnvBasis = 14695981039346656037ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;

uint64_t fnv_u64(uint64_t h, uint64_t x) {
  for (int i = 0; i < 8; ++i) {
    h ^= (x >> (8 * i)) & 0xffu;
    h *= kFnvPrime;
  }
  return h;
}

uint64_t fnv_i32(uint64_t h, int32_t v) {
  const uint32_t x = static_cast<uint32_t>(v);
  for (int i = 0; i < 4; ++i) {
    h ^= (x >> (8 * i)) & 0xffu;
    h *= kFnvPrime;
  }
  return h;
}

// Chain start of a request: FNV-1a of the salt's 8 bytes.
uint64_t chain_root(uint64_t salt) { return fnv_u64(kFnvBasis, salt); }

// Hash of one full block: FNV-1a of the parent hash's 8 bytes, then the block's token ids.
uint64_t block_key(uint64_t parent, const int32_t* tokens, int32_t bs) {
  uint64_t h = fnv_u64(kFnvBasis, parent);
  for (int32_t i = 0; i < bs; ++i) h = fnv_i32(h, tokens[i]);
  return h;
}

struct AppendResult {
  int64_t slot;
  int32_t src, dst;     // copy-on-write pair, -1 if none
  int32_t logical;      // table index whose entry changed, -1 if none
};

}  // namespace

struct pa_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> refcount;
  std::vector<Sequence> seqs;
  // prefix cache: published blocks, and the unreferenced ones in LRU order (head = oldest)
  std::vector<uint8_t> cached;
  std::vector<uint64_t> block_hash, block_parent;
  std::vector<int32_t> block_tokens;  // [num_blocks][block_size], valid while cached
  std::unordered_map<uint64_t, int32_t> by_hash;
  std::vector<int32_t> lru_prev, lru_next;
  int32_t lru_head = -1, lru_tail = -1, lru_size = 0;

  // host swap space (preemption by swapping): FIFO free list of swap block ids
  int32_t num_cpu_blocks = 0;
  std::deque<int32_t> cpu_free;

  // a live sequence whose blocks are on the device
  bool valid_seq(int32_t s) const {
    return s >= 0 && s < static_cast<int32_t>(seqs.size()) && seqs[s].live && !seqs[s].swapped;
  }
  // a live sequence, resident or swapped out
  bool known_seq(int32_t s) const {
    return s >= 0 && s < static_cast<int32_t>(seqs.size()) && seqs[s].live;
  }

  // Drop one reference from each of a table's blocks: private blocks left without references
  // go to the free list in table order; cached ones join the LRU list last block first, so a
  // prefix outlives the blocks that extend it.
  void release_table(const std::vector<int32_t>& table) {
    for (int32_t b : table) {
      refcount[b] -= 1;
      if (refcount[b] == 0 && !cached[b]) free_list.push_back(b);
    }
    for (auto it = table.rbegin(); it != table.rend(); ++it)
      if (refcount[*it] == 0 && cached[*it]) lru_push_back(*it);
  }

  void lru_unlink(int32_t b) {
    (lru_prev[b] >= 0 ? lru_next[lru_prev[b]] : lru_head) = lru_next[b];
    (lru_next[b] >= 0 ? lru_prev[lru_next[b]] : lru_tail) = lru_prev[b];
    lru_prev[b] = lru_next[b] = -1;
    --lru_size;
  }
  void lru_push_back(int32_t b) {
    lru_prev[b] = lru_tail;
    lru_next[b] = -1;
    (lru_tail >= 0 ? lru_next[lru_tail] : lru_head) = b;
    lru_tail = b;
    ++lru_size;
  }
  void lru_push_front(int32_t b) {
    lru_next[b] = lru_head;
    lru_prev[b] = -1;
    (lru_head >= 0 ? lru_prev[lru_head] : lru_tail) = b;
    lru_head = b;
    ++lru_size;
  }

  // A block for a new allocation: the free list's head, else the least recently used
  // evictable cached block (its hash is dropped).  -1 when neither exists.
  int32_t take_block(bool* evicted) {
    int32_t b = -1;
    *evicted = false;
    if (!free_list.empty()) {
      b = free_list.front();
      free_list.pop_front();
    } else if (lru_head >= 0) {
      b = lru_head;
      lru_unlink(b);
      by_hash.erase(block_hash[b]);
      cached[b] = 0;
      *evicted = true;
    } else {
      return -1;
    }
    refcount[b] = 1;
    return b;
  }

  // Undo take_block (rollback, newest first).
  void give_back(int32_t b, bool evicted) {
    refcount[b] = 0;
    if (evicted) {
      cached[b] = 1;
      by_hash[block_hash[b]] = b;
      lru_push_front(b);
    } else {
      free_list.push_front(b);
    }
  }

  // The cached block holding exactly these tokens after this parent chain, or -1.
  int32_t lookup(uint64_t key, uint64_t parent, const int32_t* tokens) const {
    const auto it = by_hash.find(key);
    if (it == by_hash.end()) return -1;
    const int32_t b = it->second;
    if (block_parent[b] != parent) return -1;
    const int32_t* t = &block_tokens[static_cast<size_t>(b) * block_size];
    for (int32_t i = 0; i < block_size; ++i)
      if (t[i] != tokens[i]) return -1;
    return b;
  }

  // Publish every block of sequence s that is full and whose tokens are all known.  A block
  // whose content is already cached elsewhere stays private; the chain continues either way.
  void publish(int32_t s) {
    Sequence& q = seqs[s];
    if (!q.hashed) return;
    const int64_t known = std::min<int64_t>(q.len, static_cast<int64_t>(q.tokens.size()));
    const size_t full = static_cast<size_t>(known / block_size);
    while (q.chain.size() < full) {
      const size_t j = q.chain.size();
      const uint64_t parent = j == 0 ? chain_root(q.salt) : q.chain[j - 1];
      const int32_t* t = &q.tokens[j * block_size];
      const uint64_t key = block_key(parent, t, block_size);
      q.chain.push_back(key);
      const int32_t b = q.table[j];
      if (cached[b] || by_hash.count(key)) continue;
      cached[b] = 1;
      block_hash[b] = key;
      block_parent[b] = parent;
      std::copy_n(t, block_size, &block_tokens[static_cast<size_t>(b) * block_size]);
      by_hash[key] = b;
    }
  }

  // One append; false means no free block (nothing changed by this call).
  bool append_one(int32_t s, AppendResult* r, std::vector<LogEntry>* log) {
    Sequence& q = seqs[s];
    const int32_t j = q.len / block_size;
    const int32_t off = q.len % block_size;
    r->src = r->dst = -1;
    r->logical = -1;
    bool evicted = false;
    if (off == 0) {
      const int32_t blk = take_block(&evicted);
      if (blk < 0) return false;
      q.table.push_back(blk);
      r->logical = j;
      log->push_back({s, Change::kNewBlock, j, -1, evicted});
    } else if (refcount[q.table[j]] > 1) {
      const int32_t dst = take_block(&evicted);
      if (dst < 0) return false;
      const int32_t src = q.table[j];
      refcount[src] -= 1;
      q.table[j] = dst;
      r->src = src;
      r->dst = dst;
      r->logical = j;
      log->push_back({s, Change::kCopy, j, src, evicted});
    } else {
      log->push_back({s, Change::kInPlace, j, -1, false});
    }
    q.len += 1;
    r->slot = static_cast<int64_t>(q.table[j]) * block_size + off;
    return true;
  }

  void rollback(std::vector<LogEntry>* log) {
    for (auto it = log->rbegin(); it != log->rend(); ++it) {
      Sequence& q = seqs[it->seq];
      q.len -= 1;
      if (it->kind == Change::kNewBlock) {
        const int32_t blk = q.table.back();
        q.table.pop_back();
        give_back(blk, it->evicted);
      } else if (it->kind == Change::kCopy) {
        const int32_t dst = q.table[it->logical];
        q.table[it->logical] = it->src;
        refcount[it->src] += 1;
        give_back(dst, it->evicted);
      }
    }
    log->clear();
  }
};

extern "C" {

int pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                    pa_allocator** out) {
  if (!out || num_blocks < 1 || block_size < 1) return PA_ERR_INVALID;
  *out = nullptr;
  std::vector<int32_t> order(num_blocks);
  if (free_order) {
    std::vector<uint8_t> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) return PA_ERR_INVALID;
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
  }
  pa_allocator* a = new (std::nothrow) pa_allocator();
  if (!a) return PA_ERR_OOM;
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->free_list.assign(order.begin(), order.end());
  a->refcount.assign(num_blocks, 0);
  a->cached.assign(num_blocks, 0);
  a->block_hash.assign(num_blocks, 0);
  a->block_parent.assign(num_blocks, 0);
  a->block_tokens.assign(static_cast<size_t>(num_blocks) * block_size, 0);
  a->lru_prev.assign(num_blocks, -1);
  a->lru_next.assign(num_blocks, -1);
  *out = a;
  return PA_OK;
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

int pa_seq_create(pa_allocator* a, int32_t* seq) {
  if (!a || !seq) return PA_ERR_INVALID;
  if (a->seqs.size() >= static_cast<size_t>(INT32_MAX)) return PA_ERR_OOM;
  a->seqs.emplace_back();
  a->seqs.back().live = true;
  *seq = static_cast<int32_t>(a->seqs.size() - 1);
  return PA_OK;
}

int pa_seq_fork(pa_allocator* a, int32_t parent, int32_t n_tokens, int32_t* child) {
  if (!a || !child) return PA_ERR_INVALID;
  if (!a->valid_seq(parent)) return PA_ERR_STATE;
  if (n_tokens < 0 || n_tokens > a->seqs[parent].len) return PA_ERR_INVALID;
  const int32_t nblk = (n_tokens + a->block_size - 1) / a->block_size;
  const Sequence& p = a->seqs[parent];
  Sequence c;
  c.live = true;
  c.len = n_tokens;
  c.table.assign(p.table.begin(), p.table.begin() + nblk);
  for (int32_t b : c.table) a->refcount[b] += 1;
  if (p.hashed) {  // the child's first n_tokens are the parent's
    c.hashed = true;
    c.salt = p.salt;
    c.tokens.assign(p.tokens.begin(),
                    p.tokens.begin() + std::min<size_t>(p.tokens.size(), n_tokens));
    c.chain.assign(p.chain.begin(),
                   p.chain.begin() + std::min<size_t>(p.chain.size(), n_tokens / a->block_size));
  }
  a->seqs.push_back(std::move(c));
  *child = static_cast<int32_t>(a->seqs.size() - 1);
  return PA_OK;
}

int pa_seq_append_slot(pa_allocator* a, int32_t seq, int64_t* slot, int32_t* cow_src,
                       int32_t* cow_dst) {
  if (!a || !slot) return PA_ERR_INVALID;
  if (!a->valid_seq(seq)) return PA_ERR_STATE;
  std::vector<LogEntry> log;
  AppendResult r;
  if (!a->append_one(seq, &r, &log)) return PA_ERR_OOM;
  if (r.src >= 0 && (!cow_src || !cow_dst)) {
    a->rollback(&log);
    return PA_ERR_INVALID;
  }
  *slot = r.slot;
  if (cow_src) *cow_src = r.src;
  if (cow_dst) *cow_dst = r.dst;
  a->publish(seq);
  return PA_OK;
}

int pa_seq_reserve(pa_allocator* a, int32_t seq, int32_t n, int64_t* slots, int32_t* cow_pairs,
                   int32_t* n_cow) {
  if (!a || n < 0 || (n > 0 && (!slots || !cow_pairs)) || !n_cow) return PA_ERR_INVALID;
  if (!a->valid_seq(seq)) return PA_ERR_STATE;
  std::vector<LogEntry> log;
  log.reserve(n);
  int32_t k = 0;
  for (int32_t i = 0; i < n; ++i) {
    AppendResult r;
    if (!a->append_one(seq, &r, &log)) {
      a->rollback(&log);
      return PA_ERR_OOM;
    }
    slots[i] = r.slot;
    if (r.src >= 0) {
      cow_pairs[2 * k] = r.src;
      cow_pairs[2 * k + 1] = r.dst;
      ++k;
    }
  }
  *n_cow = k;
  a->publish(seq);
  return PA_OK;
}

int pa_step(pa_allocator* a, const int32_t* seqs, int32_t B, int64_t* slots, int32_t* seq_lens,
            int32_t* table_index, int32_t* cow_pairs, int32_t* n_cow) {
  if (!a || B < 0 || (B > 0 && (!seqs || !slots || !cow_pairs)) || !n_cow) return PA_ERR_INVALID;
  for (int32_t i = 0; i < B; ++i)
    if (!a->valid_seq(seqs[i])) return PA_ERR_STATE;
  std::vector<LogEntry> log;
  log.reserve(B);
  int32_t k = 0;
  for (int32_t i = 0; i < B; ++i) {
    AppendResult r;
    if (!a->append_one(seqs[i], &r, &log)) {
      a->rollback(&log);
      return PA_ERR_OOM;
    }
    slots[i] = r.slot;
    if (r.src >= 0) {
      cow_pairs[2 * k] = r.src;
      cow_pairs[2 * k + 1] = r.dst;
      ++k;
    }
    if (table_index) table_index[i] = r.logical;
    if (seq_lens) seq_lens[i] = a->seqs[seqs[i]].len;
  }
  *n_cow = k;
  for (int32_t i = 0; i < B; ++i) a->publish(seqs[i]);  // in batch order
  return PA_OK;
}

int pa_seq_free(pa_allocator* a, int32_t seq) {
  if (!a) return PA_ERR_INVALID;
  if (!a->known_seq(seq)) return PA_ERR_STATE;
  Sequence& q = a->seqs[seq];
  a->release_table(q.table);
  for (int32_t c : q.cpu_table) a->cpu_free.push_back(c);
  q.cpu_table.clear();
  q.swapped = false;
  q.table.clear();
  q.table.shrink_to_fit();
  q.tokens.clear();
  q.tokens.shrink_to_fit();
  q.chain.clear();
  q.chain.shrink_to_fit();
  q.len = 0;
  q.live = false;
  return PA_OK;
}

int pa_seq_create_prefix(pa_allocator* a, const int32_t* tokens, int32_t n, uint64_t salt,
                         int32_t* seq, int32_t* n_cached) {
  if (!a || !seq || !n_cached || n < 0 || (n > 0 && !tokens)) return PA_ERR_INVALID;
  if (a->seqs.size() >= static_cast<size_t>(INT32_MAX)) return PA_ERR_OOM;
  Sequence q;
  q.live = true;
  q.hashed = true;
  q.salt = salt;
  q.tokens.assign(tokens, tokens + n);
  // match full blocks among the first n - 1 tokens: at least one prompt token is always left
  // to compute, since generation needs its query
  const int32_t bs = a->block_size;
  const int32_t max_blocks = n > 0 ? (n - 1) / bs : 0;
  uint64_t parent = chain_root(salt);
  for (int32_t j = 0; j < max_blocks; ++j) {
    const int32_t* t = tokens + static_cast<int64_t>(j) * bs;
    const uint64_t key = block_key(parent, t, bs);
    const int32_t b = a->lookup(key, parent, t);
    if (b < 0) break;
    if (a->refcount[b] == 0) a->lru_unlink(b);
    a->refcount[b] += 1;
    q.table.push_back(b);
    q.chain.push_back(key);
    parent = key;
  }
  q.len = static_cast<int32_t>(q.table.size()) * bs;
  a->seqs.push_back(std::move(q));
  *seq = static_cast<int32_t>(a->seqs.size() - 1);
  *n_cached = a->seqs.back().len;
  return PA_OK;
}

int pa_seq_add_tokens(pa_allocator* a, int32_t seq, const int32_t* tokens, int32_t n) {
  if (!a || n < 0 || (n > 0 && !tokens)) return PA_ERR_INVALID;
  if (!a->valid_seq(seq)) return PA_ERR_STATE;
  Sequence& q = a->seqs[seq];
  if (!q.hashed) return PA_ERR_INVALID;
  q.tokens.insert(q.tokens.end(), tokens, tokens + n);
  a->publish(seq);
  return PA_OK;
}

int pa_alloc_set_swap(pa_allocator* a, int32_t num_cpu_blocks) {
  if (!a || num_cpu_blocks < 0) return PA_ERR_INVALID;
  if (a->num_cpu_blocks != 0) return PA_ERR_STATE;  // set once
  a->num_cpu_blocks = num_cpu_blocks;
  for (int32_t i = 0; i < num_cpu_blocks; ++i) a->cpu_free.push_back(i);
  return PA_OK;
}

int pa_seq_swap_out(pa_allocator* a, int32_t seq, int32_t* pairs, int32_t cap, int32_t* n) {
  if (!a || !n || cap < 0 || (cap > 0 && !pairs)) return PA_ERR_INVALID;
  if (!a->valid_seq(seq)) return PA_ERR_STATE;
  Sequence& q = a->seqs[seq];
  const int32_t m = static_cast<int32_t>(q.table.size());
  *n = m;
  if (cap < m) return PA_ERR_INVALID;
  if (static_cast<int32_t>(a->cpu_free.size()) < m) return PA_ERR_OOM;
  q.cpu_table.resize(m);
  for (int32_t j = 0; j < m; ++j) {
    q.cpu_table[j] = a->cpu_free.front();
    a->cpu_free.pop_front();
    pairs[2 * j] = q.table[j];
    pairs[2 * j + 1] = q.cpu_table[j];
  }
  a->release_table(q.table);
  q.table.clear();
  q.chain.clear();  // the blocks it published stay cached (or evictable) on their own
  q.swapped = true;
  return PA_OK;
}

int pa_seq_swap_in(pa_allocator* a, int32_t seq, int32_t* pairs, int32_t cap, int32_t* n) {
  if (!a || !n || cap < 0 || (cap > 0 && !pairs)) return PA_ERR_INVALID;
  if (!a->known_seq(seq) || !a->seqs[seq].swapped) return PA_ERR_STATE;
  Sequence& q = a->seqs[seq];
  const int32_t m = static_cast<int32_t>(q.cpu_table.size());
  *n = m;
  if (cap < m) return PA_ERR_INVALID;
  std::vector<int32_t> got;
  std::vector<uint8_t> evicted;
  got.reserve(m);
  for (int32_t j = 0; j < m; ++j) {
    bool ev = false;
    const int32_t b = a->take_block(&ev);
    if (b < 0) {  // undo, newest first
      for (int32_t k = static_cast<int32_t>(got.size()) - 1; k >= 0; --k)
        a->give_back(got[k], evicted[k]);
      return PA_ERR_OOM;
    }
    got.push_back(b);
    evicted.push_back(ev);
  }
  q.table = got;
  for (int32_t j = 0; j < m; ++j) {
    pairs[2 * j] = q.cpu_table[j];
    pairs[2 * j + 1] = got[j];
    a->cpu_free.push_back(q.cpu_table[j]);
  }
  q.cpu_table.clear();
  q.swapped = false;
  a->publish(seq);
  return PA_OK;
}

int pa_num_free_swap(const pa_allocator* a, int32_t* n) {
  if (!a || !n) return PA_ERR_INVALID;
  *n = static_cast<int32_t>(a->cpu_free.size());
  return PA_OK;
}

int pa_num_evictable(const pa_allocator* a, int32_t* n) {
  if (!a || !n) return PA_ERR_INVALID;
  *n = a->lru_size;
  return PA_OK;
}

int pa_evictable_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n) {
  if (!a || !n || cap < 0 || (cap > 0 && !out)) return PA_ERR_INVALID;
  *n = a->lru_size;
  int32_t k = 0;
  for (int32_t b = a->lru_head; b >= 0 && k < cap; b = a->lru_next[b]) out[k++] = b;
  return PA_OK;
}

int pa_block_hash(const pa_allocator* a, int32_t block, uint64_t* hash, int32_t* cached) {
  if (!a || !hash || !cached || block < 0 || block >= a->num_blocks) return PA_ERR_INVALID;
  *cached = a->cached[block];
  *hash = a->cached[block] ? a->block_hash[block] : 0;
  return PA_OK;
}

int pa_seq_len(const pa_allocator* a, int32_t seq, int32_t* len) {
  if (!a || !len) return PA_ERR_INVALID;
  if (!a->known_seq(seq)) return PA_ERR_STATE;
  *len = a->seqs[seq].len;
  return PA_OK;
}

int pa_seq_table(const pa_allocator* a, int32_t seq, int32_t* out, int32_t cap, int32_t* n) {
  if (!a || !n || cap < 0 || (cap > 0 && !out)) return PA_ERR_INVALID;
  if (!a->valid_seq(seq)) return PA_ERR_STATE;
  const auto& t = a->seqs[seq].table;
  *n = static_cast<int32_t>(t.size());
  std::copy_n(t.begin(), std::min<size_t>(t.size(), static_cast<size_t>(cap)), out);
  return PA_OK;
}

int pa_export_block_tables(const pa_allocator* a, const int32_t* seqs, int32_t B,
                           int32_t max_blocks, int32_t* tables, int32_t* seq_lens) {
  if (!a || B < 0 || max_blocks < 0 || (B > 0 && (!seqs || !seq_lens))) return PA_ERR_INVALID;
  if (B > 0 && max_blocks > 0 && !tables) return PA_ERR_INVALID;
  for (int32_t i = 0; i < B; ++i) {
    if (!a->valid_seq(seqs[i])) return PA_ERR_STATE;
    if (a->seqs[seqs[i]].table.size() > static_cast<size_t>(max_blocks)) return PA_ERR_INVALID;
  }
  for (int32_t i = 0; i < B; ++i) {
    const Sequence& q = a->seqs[seqs[i]];
    int32_t* row = tables + static_cast<int64_t>(i) * max_blocks;
    std::copy(q.table.begin(), q.table.end(), row);
    std::fill(row + q.table.size(), row + max_blocks, -1);
    seq_lens[i] = q.len;
  }
  return PA_OK;
}

int pa_block_refcount(const pa_allocator* a, int32_t block, int32_t* rc) {
  if (!a || !rc || block < 0 || block >= a->num_blocks) return PA_ERR_INVALID;
  *rc = a->refcount[block];
  return PA_OK;
}

int pa_num_free(const pa_allocator* a, int32_t* n) {
  if (!a || !n) return PA_ERR_INVALID;
  *n = static_cast<int32_t>(a->free_list.size());
  return PA_OK;
}

int pa_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n) {
  if (!a || !n || cap < 0 || (cap > 0 && !out)) return PA_ERR_INVALID;
  *n = static_cast<int32_t>(a->free_list.size());
  const size_t m = std::min<size_t>(a->free_list.size(), static_cast<size_t>(cap));
  std::copy_n(a->free_list.begin(), m, out);
  return PA_OK;
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_OOM: return "out of free blocks";
    case PA_ERR_DEVICE: return "device error";
    case PA_ERR_UNSUPPORTED: return "unsupported combination";
    case PA_ERR_STATE: return "unknown or released sequence";
    case PA_ERR_TOO_LARGE: return "needs more scratch than the library's fixed buffer holds";
    default: return "unknown status";
  }
}

int pa_abi_version(void) { return 6; }

}  // extern "C"

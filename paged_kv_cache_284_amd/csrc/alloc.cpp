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
#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <vector>

#include "pagedkv.h"

namespace {

struct Sequence {
  bool live = false;
  int32_t len = 0;
  std::vector<int32_t> table;
};

enum class Change : uint8_t { kInPlace, kNewBlock, kCopy };

struct LogEntry {
  int32_t seq;
  Change kind;
  int32_t logical;  // table index touched (kCopy)
  int32_t src;      // block replaced (kCopy)
};

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

  bool valid_seq(int32_t s) const {
    return s >= 0 && s < static_cast<int32_t>(seqs.size()) && seqs[s].live;
  }

  // One append; false means no free block (nothing changed by this call).
  bool append_one(int32_t s, AppendResult* r, std::vector<LogEntry>* log) {
    Sequence& q = seqs[s];
    const int32_t j = q.len / block_size;
    const int32_t off = q.len % block_size;
    r->src = r->dst = -1;
    r->logical = -1;
    if (off == 0) {
      if (free_list.empty()) return false;
      const int32_t blk = free_list.front();
      free_list.pop_front();
      refcount[blk] = 1;
      q.table.push_back(blk);
      r->logical = j;
      log->push_back({s, Change::kNewBlock, j, -1});
    } else if (refcount[q.table[j]] > 1) {
      if (free_list.empty()) return false;
      const int32_t src = q.table[j];
      const int32_t dst = free_list.front();
      free_list.pop_front();
      refcount[dst] = 1;
      refcount[src] -= 1;
      q.table[j] = dst;
      r->src = src;
      r->dst = dst;
      r->logical = j;
      log->push_back({s, Change::kCopy, j, src});
    } else {
      log->push_back({s, Change::kInPlace, j, -1});
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
        refcount[blk] = 0;
        free_list.push_front(blk);
      } else if (it->kind == Change::kCopy) {
        const int32_t dst = q.table[it->logical];
        q.table[it->logical] = it->src;
        refcount[it->src] += 1;
        refcount[dst] = 0;
        free_list.push_front(dst);
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
  Sequence c;
  c.live = true;
  c.len = n_tokens;
  c.table.assign(a->seqs[parent].table.begin(), a->seqs[parent].table.begin() + nblk);
  for (int32_t b : c.table) a->refcount[b] += 1;
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
  return PA_OK;
}

int pa_seq_free(pa_allocator* a, int32_t seq) {
  if (!a) return PA_ERR_INVALID;
  if (!a->valid_seq(seq)) return PA_ERR_STATE;
  Sequence& q = a->seqs[seq];
  for (int32_t b : q.table) {
    a->refcount[b] -= 1;
    if (a->refcount[b] == 0) a->free_list.push_back(b);
  }
  q.table.clear();
  q.table.shrink_to_fit();
  q.len = 0;
  q.live = false;
  return PA_OK;
}

int pa_seq_len(const pa_allocator* a, int32_t seq, int32_t* len) {
  if (!a || !len) return PA_ERR_INVALID;
  if (!a->valid_seq(seq)) return PA_ERR_STATE;
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
    default: return "unknown status";
  }
}

int pa_abi_version(void) { return 1; }

}  // extern "C"

// Host block allocator: a first-in-first-out queue of free blocks, per-block
// reference counts, fork and append with copy-on-write.
//
// Policy ("PagedAttention 源码解析：KV Cache 怎么管理" §二/§三; xdnf.cn
// PagedAttention article §3.1, §3.4, §4.2; "PagedAttention 实现细节" §3.3):
//  * allocation takes the head of the free queue; a block whose count drops to
//    zero is appended to the tail (the first page's worked example, requests of
//    32/16/48 tokens getting [0,1], [2], [3,4,5], fixes the queue order);
//  * n tokens occupy ceil(n / block_size) blocks;
//  * appending at position L opens a fresh block when L % bs == 0, otherwise it
//    writes into the last block, first replacing that block with a private copy
//    if its count is above one (the copy is done on the device by the caller);
//  * every call is all-or-nothing.
//
// Prefix caching ("PagedAttention 实现细节" §3.2): entries map a prompt
// prefix's tokens (compared in full) to the blocks holding its KV, count their
// users, and hold one reference per block.  A sequence built on an entry
// shares its blocks and puts its own tokens from the next block boundary on,
// leaving a hole [n_p, P * bs) that decode masks.
//
// Swap ("PagedAttention 实现细节" §3.4: the cache engine has a host-side pool used for swapping): a
// host pool with its own FIFO queue and counts; a group of sequences moves
// whole, one copy pair per distinct block.  Sliding window: blocks wholly
// before the last W positions are released and their entries become -1.
//
// The free queue is a ring buffer of num_blocks entries; a block is never in
// it twice, so it never overflows.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <string>
#include <mutex>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "status.hpp"

namespace {

// PA_LOG=1 (or any value but 0): pa_build_block_tables dumps the tables it
// builds.  Read on every call.
bool log_tables() {
  const char* v = std::getenv("PA_LOG");
  return v && v[0] != '\0' && std::strcmp(v, "0") != 0;
}

struct Seq {
  std::vector<int32_t> table;
  int32_t len = 0;
  int32_t hole_lo = 0, hole_hi = 0;  // positions [lo, hi) hold no token (lo == hi: none)
  int32_t window = 0;                // > 0: only the last `window` positions are live
  int32_t first_live = 0;            // table entries below it are -1 (released behind the window)
  bool swapped = false;              // the table holds host-pool ids
};

struct PrefixEntry {
  std::vector<int32_t> key;     // the prefix's tokens
  std::vector<int32_t> blocks;
  int32_t users = 0;
};

// FNV-1a over the token values, for bucketing; keys are compared in full.
struct TokensHash {
  size_t operator()(const std::vector<int32_t>& v) const {
    uint64_t h = 1469598103934665603ull;
    for (int32_t t : v) {
      uint32_t u = static_cast<uint32_t>(t);
      for (int i = 0; i < 4; ++i) {
        h ^= (u >> (8 * i)) & 0xffu;
        h *= 1099511628211ull;
      }
    }
    return static_cast<size_t>(h);
  }
};

}  // namespace

struct pa_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ring;  // free queue storage
  int32_t head = 0;           // index of the queue head in `ring`
  int32_t count = 0;          // number of free blocks
  std::vector<int32_t> refs;
  std::unordered_map<int64_t, Seq> seqs;
  std::unordered_map<int64_t, PrefixEntry> prefixes;                 // by entry id
  std::unordered_map<std::vector<int32_t>, int64_t, TokensHash> prefix_ids;  // by tokens
  int64_t next_prefix_id = 1;
  // host pool (swap): FIFO queue and counts, like the device pool
  int32_t num_host = 0;
  std::vector<int32_t> host_ring, host_refs;
  int32_t host_head = 0, host_count = 0;
  int32_t num_swapped = 0;
  pa_allocator_stats stats{0, 0, 0};
  mutable std::mutex mu;

  int32_t blocks_for(int64_t n) const {
    return static_cast<int32_t>((n + block_size - 1) / block_size);
  }
  int32_t pop_head() {
    int32_t b = ring[head];
    head = head + 1 == num_blocks ? 0 : head + 1;
    --count;
    refs[b] = 1;
    ++stats.blocks_allocated;
    return b;
  }
  void push_tail(int32_t b) {
    int64_t pos = static_cast<int64_t>(head) + count;
    ring[pos % num_blocks] = b;
    ++count;
    ++stats.blocks_freed;
  }
  void release(int32_t b) {
    if (--refs[b] == 0) push_tail(b);
  }
  int32_t host_pop() {
    int32_t h = host_ring[host_head];
    host_head = host_head + 1 == num_host ? 0 : host_head + 1;
    --host_count;
    host_refs[h] = 0;
    return h;
  }
  void host_release(int32_t h) {
    if (--host_refs[h] == 0) {
      host_ring[(static_cast<int64_t>(host_head) + host_count) % num_host] = h;
      ++host_count;
    }
  }
};

namespace {

using pa::fail;

// Undo log for a batch of appends, so a batch that runs out of blocks half way
// can be rolled back whole.
struct Journal {
  struct RefChange { int32_t block, old; };
  struct SeqChange { Seq* seq; int32_t old_len; int32_t index; int32_t old_block; bool appended; };
  std::vector<RefChange> refs;
  std::vector<SeqChange> seqs;
  int32_t head = 0, count = 0;
  pa_allocator_stats stats{0, 0, 0};
};

// Append one token to `s`.  Needs at most one free block, checked before any
// change.  With a journal, every change is logged for rollback.
pa_status append_one(pa_allocator* a, Seq& s, int32_t* slot, int32_t* src, int32_t* dst,
                     Journal* j) {
  const int32_t bs = a->block_size;
  const int32_t L = s.len;
  if (L == INT32_MAX) return fail(PA_ERR_INVALID_ARG, "sequence length overflow");
  const int32_t lb = L / bs;
  *src = -1;
  *dst = -1;
  if (L % bs == 0) {
    if (a->count == 0) return fail(PA_ERR_NO_FREE_BLOCKS, "no free block for a new token");
    if (j) j->seqs.push_back({&s, L, lb, -1, true});
    int32_t b = a->pop_head();
    if (j) j->refs.push_back({b, 0});
    s.table.push_back(b);
  } else {
    int32_t last = s.table[lb];
    if (a->refs[last] > 1) {
      if (a->count == 0) return fail(PA_ERR_NO_FREE_BLOCKS, "no free block for copy-on-write");
      if (j) j->seqs.push_back({&s, L, lb, last, false});
      int32_t b = a->pop_head();
      if (j) {
        j->refs.push_back({b, 0});
        j->refs.push_back({last, a->refs[last]});
      }
      --a->refs[last];
      s.table[lb] = b;
      ++a->stats.cow_copies;
      *src = last;
      *dst = b;
    } else if (j) {
      j->seqs.push_back({&s, L, lb, -1, false});
    }
  }
  *slot = s.table[lb] * bs + L % bs;
  s.len = L + 1;
  if (s.window > 0) {
    // release the blocks that fell wholly behind the window
    const int64_t start = static_cast<int64_t>(s.len) - s.window;
    while (s.first_live < static_cast<int32_t>(s.table.size()) &&
           static_cast<int64_t>(s.first_live + 1) * bs <= start) {
      const int32_t b = s.table[s.first_live];
      if (b >= 0) {
        if (j) {
          j->seqs.push_back({&s, L, s.first_live, b, false});
          j->refs.push_back({b, a->refs[b]});
        }
        a->release(b);
        s.table[s.first_live] = -1;
      }
      ++s.first_live;
    }
  }
  return PA_OK;
}

void rollback(pa_allocator* a, Journal& j) {
  for (auto it = j.refs.rbegin(); it != j.refs.rend(); ++it) a->refs[it->block] = it->old;
  for (auto it = j.seqs.rbegin(); it != j.seqs.rend(); ++it) {
    Seq& s = *it->seq;
    if (it->appended) s.table.pop_back();
    else if (it->old_block >= 0) s.table[it->index] = it->old_block;
    s.len = it->old_len;
    if (s.window > 0 && it->index < s.first_live && !it->appended && it->old_block >= 0 &&
        s.table[it->index] >= 0)
      s.first_live = it->index;  // a released entry is back: the live range starts there again
  }
  a->head = j.head;
  a->count = j.count;
  a->stats = j.stats;
}

// Release the blocks wholly behind the sequence's window (a fresh window or a
// fork; appends do the same inside append_one, under the journal).
void drop_behind_window(pa_allocator* a, Seq& s) {
  const int64_t start = static_cast<int64_t>(s.len) - s.window;
  while (s.first_live < static_cast<int32_t>(s.table.size()) &&
         static_cast<int64_t>(s.first_live + 1) * a->block_size <= start) {
    const int32_t b = s.table[s.first_live];
    if (b >= 0) {
      a->release(b);
      s.table[s.first_live] = -1;
    }
    ++s.first_live;
  }
}

// The sequences of a swap group (duplicates ignored, first appearance kept),
// checked, and their distinct non-negative table entries in order.
pa_status swap_group(pa_allocator* a, const int64_t* seq_ids, int32_t n, bool swapped, std::vector<Seq*>* group,
                     std::vector<int32_t>* distinct) {
  std::unordered_set<int64_t> seen_ids;
  for (int32_t i = 0; i < n; ++i) {
    if (!seen_ids.insert(seq_ids[i]).second) continue;
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence in the group");
    if (it->second.swapped != swapped)
      return fail(PA_ERR_INVALID_ARG, swapped ? "sequence is not swapped out" : "sequence already swapped out");
    group->push_back(&it->second);
  }
  std::unordered_set<int32_t> seen;
  for (Seq* s : *group)
    for (int32_t b : s->table)
      if (b >= 0 && seen.insert(b).second) distinct->push_back(b);
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_allocator_create(int32_t num_blocks, int32_t block_size,
                              const int32_t* initial_free_order, pa_allocator** out) {
  if (!out) return fail(PA_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  if (num_blocks < 0 || block_size <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_blocks must be >= 0 and block_size > 0");
  auto* a = new (std::nothrow) pa_allocator();
  if (!a) return fail(PA_ERR_INVALID_ARG, "out of host memory");
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->ring.resize(num_blocks);
  a->refs.assign(num_blocks, 0);
  if (initial_free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return fail(PA_ERR_INVALID_ARG, "initial free order is not a permutation of 0..num_blocks-1");
      }
      seen[b] = 1;
      a->ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->ring[i] = i;
  }
  a->head = 0;
  a->count = num_blocks;
  *out = a;
  return PA_OK;
}

void pa_allocator_destroy(pa_allocator* a) { delete a; }

pa_status pa_allocator_clone(const pa_allocator* a, pa_allocator** out) {
  if (!a || !out) return fail(PA_ERR_INVALID_ARG, "null argument");
  std::lock_guard<std::mutex> g(a->mu);
  auto* c = new (std::nothrow) pa_allocator();
  if (!c) return fail(PA_ERR_INVALID_ARG, "out of host memory");
  c->num_blocks = a->num_blocks;
  c->block_size = a->block_size;
  c->ring = a->ring;
  c->head = a->head;
  c->count = a->count;
  c->refs = a->refs;
  c->seqs = a->seqs;
  c->prefixes = a->prefixes;
  c->prefix_ids = a->prefix_ids;
  c->next_prefix_id = a->next_prefix_id;
  c->num_host = a->num_host;
  c->host_ring = a->host_ring;
  c->host_refs = a->host_refs;
  c->host_head = a->host_head;
  c->host_count = a->host_count;
  c->num_swapped = a->num_swapped;
  c->stats = a->stats;
  *out = c;
  return PA_OK;
}

pa_status pa_seq_create(pa_allocator* a, int64_t seq_id, int32_t num_tokens) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "null allocator");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens < 0");
  std::lock_guard<std::mutex> g(a->mu);
  if (a->seqs.count(seq_id)) return fail(PA_ERR_SEQ_EXISTS, "sequence id already in use");
  int32_t nb = a->blocks_for(num_tokens);
  if (nb > a->count) return fail(PA_ERR_NO_FREE_BLOCKS, "not enough free blocks for the sequence");
  Seq s;
  s.table.reserve(nb + 1);
  for (int32_t i = 0; i < nb; ++i) s.table.push_back(a->pop_head());
  s.len = num_tokens;
  a->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

pa_status pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child, int32_t num_tokens) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "null allocator");
  std::lock_guard<std::mutex> g(a->mu);
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown parent sequence");
  if (a->seqs.count(child)) return fail(PA_ERR_SEQ_EXISTS, "child id already in use");
  const Seq& p = it->second;
  if (p.swapped) return fail(PA_ERR_INVALID_ARG, "parent is swapped out");
  int32_t n = num_tokens < 0 ? p.len : num_tokens;
  if (n > p.len) return fail(PA_ERR_INVALID_ARG, "fork length beyond the parent's length");
  if (p.hole_lo < n && n < p.hole_hi) return fail(PA_ERR_INVALID_ARG, "fork length inside the prefix hole");
  int32_t nb = a->blocks_for(n);
  if (p.window > 0) {
    const int32_t first_live = std::max(0, n - p.window) / a->block_size;
    for (int32_t j = first_live; j < nb; ++j)
      if (p.table[j] < 0) return fail(PA_ERR_INVALID_ARG, "the child's window needs blocks the parent dropped");
  }
  Seq c;
  c.table.assign(p.table.begin(), p.table.begin() + nb);
  c.len = n;
  if (p.hole_lo < p.hole_hi && n >= p.hole_hi) {
    c.hole_lo = p.hole_lo;
    c.hole_hi = p.hole_hi;
  }
  for (int32_t b : c.table)
    if (b >= 0) ++a->refs[b];
  c.window = p.window;
  auto ins = a->seqs.emplace(child, std::move(c));
  if (p.window > 0) drop_behind_window(a, ins.first->second);
  return PA_OK;
}

pa_status pa_seq_append_slot(pa_allocator* a, int64_t seq_id, int32_t* slot, int32_t* cow_src,
                             int32_t* cow_dst) {
  if (!a || !slot || !cow_src || !cow_dst) return fail(PA_ERR_INVALID_ARG, "null argument");
  std::lock_guard<std::mutex> g(a->mu);
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence");
  if (it->second.swapped) return fail(PA_ERR_INVALID_ARG, "sequence is swapped out");
  return append_one(a, it->second, slot, cow_src, cow_dst, nullptr);
}

pa_status pa_seq_append_slots(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t* slots,
                              int32_t* cow_pairs, int32_t* num_pairs) {
  if (!a || !num_pairs || n < 0 || (n > 0 && (!seq_ids || !slots || !cow_pairs)))
    return fail(PA_ERR_INVALID_ARG, "null argument or negative count");
  std::lock_guard<std::mutex> g(a->mu);
  std::vector<Seq*> ptrs(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence in batch");
    ptrs[i] = &it->second;
  }
  for (int32_t i = 0; i < n; ++i)
    if (ptrs[i]->swapped) return fail(PA_ERR_INVALID_ARG, "a sequence in the batch is swapped out");
  // Each append needs at most one block: with n free blocks nothing can fail
  // for lack of blocks and the journal is skipped.
  Journal journal;
  Journal* j = nullptr;
  if (a->count < n) {
    journal.head = a->head;
    journal.count = a->count;
    journal.stats = a->stats;
    j = &journal;
  }
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    pa_status st = append_one(a, *ptrs[i], &slots[i], &src, &dst, j);
    if (st != PA_OK) {
      if (j) rollback(a, *j);
      return st;
    }
    if (src >= 0) {
      cow_pairs[2 * np] = src;
      cow_pairs[2 * np + 1] = dst;
      ++np;
    }
  }
  *num_pairs = np;
  return PA_OK;
}

pa_status pa_seq_free(pa_allocator* a, int64_t seq_id) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "null allocator");
  std::lock_guard<std::mutex> g(a->mu);
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence");
  const Seq& sq = it->second;
  for (int32_t b : sq.table) {
    if (b < 0) continue;  // released behind a window
    if (sq.swapped) a->host_release(b);
    else a->release(b);
  }
  if (sq.swapped) --a->num_swapped;
  a->seqs.erase(it);
  return PA_OK;
}

pa_status pa_can_allocate(const pa_allocator* a, int32_t num_blocks, int32_t* ok) {
  if (!a || !ok) return fail(PA_ERR_INVALID_ARG, "null argument");
  std::lock_guard<std::mutex> g(a->mu);
  *ok = num_blocks <= a->count ? 1 : 0;
  return PA_OK;
}

int32_t pa_num_free_blocks(const pa_allocator* a) {
  if (!a) return -1;
  std::lock_guard<std::mutex> g(a->mu);
  return a->count;
}

int32_t pa_ref_count(const pa_allocator* a, int32_t block) {
  if (!a) return -1;
  std::lock_guard<std::mutex> g(a->mu);
  if (block < 0 || block >= a->num_blocks) return -1;
  return a->refs[block];
}

pa_status pa_seq_len(const pa_allocator* a, int64_t seq_id, int32_t* len) {
  if (!a || !len) return fail(PA_ERR_INVALID_ARG, "null argument");
  std::lock_guard<std::mutex> g(a->mu);
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence");
  *len = it->second.len;
  return PA_OK;
}

pa_status pa_seq_block_table(const pa_allocator* a, int64_t seq_id, int32_t* out, int32_t capacity,
                             int32_t* num_blocks) {
  if (!a || !num_blocks || capacity < 0 || (capacity > 0 && !out))
    return fail(PA_ERR_INVALID_ARG, "null argument or negative capacity");
  std::lock_guard<std::mutex> g(a->mu);
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence");
  const auto& t = it->second.table;
  if (static_cast<int64_t>(t.size()) > capacity) return fail(PA_ERR_INVALID_ARG, "capacity too small");
  if (!t.empty()) std::memcpy(out, t.data(), t.size() * sizeof(int32_t));
  *num_blocks = static_cast<int32_t>(t.size());
  return PA_OK;
}

pa_status pa_free_list(const pa_allocator* a, int32_t* out, int32_t capacity, int32_t* n) {
  if (!a || !n || capacity < 0 || (capacity > 0 && !out))
    return fail(PA_ERR_INVALID_ARG, "null argument or negative capacity");
  std::lock_guard<std::mutex> g(a->mu);
  if (a->count > capacity) return fail(PA_ERR_INVALID_ARG, "capacity too small");
  for (int32_t i = 0; i < a->count; ++i)
    out[i] = a->ring[(static_cast<int64_t>(a->head) + i) % a->num_blocks];
  *n = a->count;
  return PA_OK;
}

pa_status pa_build_block_tables(const pa_allocator* a, const int64_t* seq_ids, int32_t n,
                                int32_t max_blocks, int32_t* tables, int32_t* context_lens) {
  if (!a || n < 0 || max_blocks < 0 ||
      (n > 0 && (!seq_ids || !context_lens || (max_blocks > 0 && !tables))))
    return fail(PA_ERR_INVALID_ARG, "null argument or negative size");
  std::lock_guard<std::mutex> g(a->mu);
  std::vector<const Seq*> ptrs(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence");
    if (it->second.swapped) return fail(PA_ERR_INVALID_ARG, "sequence is swapped out");
    if (static_cast<int64_t>(it->second.table.size()) > max_blocks)
      return fail(PA_ERR_INVALID_ARG, "a block table is longer than max_blocks");
    ptrs[i] = &it->second;
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& t = ptrs[i]->table;
    int32_t* row = tables + static_cast<int64_t>(i) * max_blocks;
    const int32_t k = static_cast<int32_t>(t.size());
    if (k) std::memcpy(row, t.data(), k * sizeof(int32_t));
    for (int32_t j = k; j < max_blocks; ++j) row[j] = -1;
    context_lens[i] = ptrs[i]->len;
  }
  if (log_tables()) {  // PA_LOG=1: one line per sequence on stderr, as "seq 0: [3, 7, 11] len 40"
    for (int32_t i = 0; i < n; ++i) {
      std::string line = "pa: seq " + std::to_string(seq_ids[i]) + ": [";
      const auto& t = ptrs[i]->table;
      for (size_t j = 0; j < t.size(); ++j) line += (j ? ", " : "") + std::to_string(t[j]);
      line += "] len " + std::to_string(ptrs[i]->len) + "\n";
      std::fputs(line.c_str(), stderr);
    }
  }
  return PA_OK;
}

pa_status pa_allocator_get_stats(const pa_allocator* a, pa_allocator_stats* out) {
  if (!a || !out) return fail(PA_ERR_INVALID_ARG, "null argument");
  std::lock_guard<std::mutex> g(a->mu);
  *out = a->stats;
  return PA_OK;
}

pa_status pa_prefix_get_or_create(pa_allocator* a, const int32_t* tokens, int32_t num_tokens,
                                  int64_t* prefix_id, int32_t* hit) {
  if (!a || !prefix_id || !hit || num_tokens < 0 || (num_tokens > 0 && !tokens))
    return fail(PA_ERR_INVALID_ARG, "null argument or negative count");
  std::lock_guard<std::mutex> g(a->mu);
  std::vector<int32_t> key(tokens, tokens + num_tokens);
  auto it = a->prefix_ids.find(key);
  if (it != a->prefix_ids.end()) {
    ++a->prefixes[it->second].users;
    *prefix_id = it->second;
    *hit = 1;
    return PA_OK;
  }
  const int32_t nb = a->blocks_for(num_tokens);
  if (nb > a->count) return fail(PA_ERR_NO_FREE_BLOCKS, "not enough free blocks for the prefix");
  PrefixEntry e;
  e.key = key;
  e.users = 1;
  e.blocks.reserve(nb);
  for (int32_t i = 0; i < nb; ++i) e.blocks.push_back(a->pop_head());
  const int64_t id = a->next_prefix_id++;
  a->prefixes.emplace(id, std::move(e));
  a->prefix_ids.emplace(std::move(key), id);
  *prefix_id = id;
  *hit = 0;
  return PA_OK;
}

pa_status pa_prefix_release(pa_allocator* a, int64_t prefix_id) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "null allocator");
  std::lock_guard<std::mutex> g(a->mu);
  auto it = a->prefixes.find(prefix_id);
  if (it == a->prefixes.end()) return fail(PA_ERR_UNKNOWN_PREFIX, "unknown prefix id");
  PrefixEntry& e = it->second;
  if (--e.users <= 0) {
    for (int32_t b : e.blocks) a->release(b);
    a->prefix_ids.erase(e.key);
    a->prefixes.erase(it);
  }
  return PA_OK;
}

pa_status pa_prefix_info(const pa_allocator* a, int64_t prefix_id, int32_t* blocks, int32_t capacity,
                         int32_t* num_blocks, int32_t* num_tokens, int32_t* users) {
  if (!a || !num_blocks || capacity < 0 || (capacity > 0 && !blocks))
    return fail(PA_ERR_INVALID_ARG, "null argument or negative capacity");
  std::lock_guard<std::mutex> g(a->mu);
  auto it = a->prefixes.find(prefix_id);
  if (it == a->prefixes.end()) return fail(PA_ERR_UNKNOWN_PREFIX, "unknown prefix id");
  const PrefixEntry& e = it->second;
  const int32_t nb = static_cast<int32_t>(e.blocks.size());
  if (blocks) {
    if (nb > capacity) return fail(PA_ERR_INVALID_ARG, "capacity too small");
    if (nb) std::memcpy(blocks, e.blocks.data(), nb * sizeof(int32_t));
  }
  *num_blocks = nb;
  if (num_tokens) *num_tokens = static_cast<int32_t>(e.key.size());
  if (users) *users = e.users;
  return PA_OK;
}

pa_status pa_seq_create_with_prefix(pa_allocator* a, int64_t seq_id, int64_t prefix_id, int32_t own_tokens) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "null allocator");
  std::lock_guard<std::mutex> g(a->mu);
  if (a->seqs.count(seq_id)) return fail(PA_ERR_SEQ_EXISTS, "sequence id already in use");
  if (own_tokens < 0) return fail(PA_ERR_INVALID_ARG, "own_tokens < 0");
  auto it = a->prefixes.find(prefix_id);
  if (it == a->prefixes.end()) return fail(PA_ERR_UNKNOWN_PREFIX, "unknown prefix id");
  const PrefixEntry& e = it->second;
  const int64_t start = static_cast<int64_t>(e.blocks.size()) * a->block_size;
  if (start + own_tokens > INT32_MAX) return fail(PA_ERR_INVALID_ARG, "sequence length overflow");
  const int32_t nb = a->blocks_for(own_tokens);
  if (nb > a->count) return fail(PA_ERR_NO_FREE_BLOCKS, "not enough free blocks for the sequence");
  Seq s;
  s.table.reserve(e.blocks.size() + nb + 1);
  for (int32_t b : e.blocks) {
    ++a->refs[b];
    s.table.push_back(b);
  }
  for (int32_t i = 0; i < nb; ++i) s.table.push_back(a->pop_head());
  s.len = static_cast<int32_t>(start) + own_tokens;
  if (static_cast<int64_t>(e.key.size()) < start) {
    s.hole_lo = static_cast<int32_t>(e.key.size());
    s.hole_hi = static_cast<int32_t>(start);
  }
  a->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

pa_status pa_build_masks(const pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t* mask_lo,
                         int32_t* mask_hi) {
  if (!a || n < 0 || (n > 0 && (!seq_ids || !mask_lo || !mask_hi)))
    return fail(PA_ERR_INVALID_ARG, "null argument or negative count");
  std::lock_guard<std::mutex> g(a->mu);
  std::vector<const Seq*> ptrs(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence");
    ptrs[i] = &it->second;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (ptrs[i]->window > 0) {
      mask_lo[i] = 0;
      mask_hi[i] = std::max(0, ptrs[i]->len - ptrs[i]->window);
    } else {
      mask_lo[i] = ptrs[i]->hole_lo;
      mask_hi[i] = ptrs[i]->hole_hi;
    }
  }
  return PA_OK;
}

pa_status pa_seq_set_window(pa_allocator* a, int64_t seq_id, int32_t window) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "null allocator");
  std::lock_guard<std::mutex> g(a->mu);
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence");
  if (window < 1) return fail(PA_ERR_INVALID_ARG, "window < 1");
  Seq& s = it->second;
  if (s.swapped || s.hole_lo < s.hole_hi)
    return fail(PA_ERR_INVALID_ARG, "window on a swapped sequence or one with a prefix hole");
  s.window = window;
  drop_behind_window(a, s);
  return PA_OK;
}

pa_status pa_allocator_set_host_pool(pa_allocator* a, int32_t num_host_blocks) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "null allocator");
  std::lock_guard<std::mutex> g(a->mu);
  if (num_host_blocks < 0) return fail(PA_ERR_INVALID_ARG, "num_host_blocks < 0");
  if (a->num_swapped > 0) return fail(PA_ERR_INVALID_ARG, "sequences are swapped out");
  a->num_host = num_host_blocks;
  a->host_ring.resize(num_host_blocks);
  for (int32_t i = 0; i < num_host_blocks; ++i) a->host_ring[i] = i;
  a->host_refs.assign(num_host_blocks, 0);
  a->host_head = 0;
  a->host_count = num_host_blocks;
  return PA_OK;
}

pa_status pa_seq_swap_out(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t* pairs, int32_t capacity,
                          int32_t* num_pairs) {
  if (!a || !num_pairs || n < 0 || capacity < 0 || (n > 0 && !seq_ids) || (capacity > 0 && !pairs))
    return fail(PA_ERR_INVALID_ARG, "null argument or negative count");
  std::lock_guard<std::mutex> g(a->mu);
  std::vector<Seq*> group;
  std::vector<int32_t> distinct;
  pa_status st = swap_group(a, seq_ids, n, false, &group, &distinct);
  if (st != PA_OK) return st;
  const int32_t k = static_cast<int32_t>(distinct.size());
  if (k > a->host_count) return fail(PA_ERR_NO_FREE_BLOCKS, "not enough free host blocks");
  if (k > capacity) return fail(PA_ERR_INVALID_ARG, "pairs capacity too small");
  std::unordered_map<int32_t, int32_t> where;
  for (int32_t i = 0; i < k; ++i) {
    const int32_t h = a->host_pop();
    where[distinct[i]] = h;
    pairs[2 * i] = distinct[i];
    pairs[2 * i + 1] = h;
  }
  for (Seq* s : group) {
    for (int32_t& b : s->table) {
      if (b < 0) continue;
      const int32_t h = where[b];
      ++a->host_refs[h];
      a->release(b);
      b = h;
    }
    s->swapped = true;
    ++a->num_swapped;
  }
  *num_pairs = k;
  return PA_OK;
}

pa_status pa_seq_swap_in(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t* pairs, int32_t capacity,
                         int32_t* num_pairs) {
  if (!a || !num_pairs || n < 0 || capacity < 0 || (n > 0 && !seq_ids) || (capacity > 0 && !pairs))
    return fail(PA_ERR_INVALID_ARG, "null argument or negative count");
  std::lock_guard<std::mutex> g(a->mu);
  std::vector<Seq*> group;
  std::vector<int32_t> distinct;
  pa_status st = swap_group(a, seq_ids, n, true, &group, &distinct);
  if (st != PA_OK) return st;
  const int32_t k = static_cast<int32_t>(distinct.size());
  if (k > a->count) return fail(PA_ERR_NO_FREE_BLOCKS, "not enough free device blocks");
  if (k > capacity) return fail(PA_ERR_INVALID_ARG, "pairs capacity too small");
  std::unordered_map<int32_t, int32_t> where;
  for (int32_t i = 0; i < k; ++i) {
    const int32_t d = a->pop_head();
    a->refs[d] = 0;
    where[distinct[i]] = d;
    pairs[2 * i] = distinct[i];
    pairs[2 * i + 1] = d;
  }
  for (Seq* s : group) {
    for (int32_t& h : s->table) {
      if (h < 0) continue;
      const int32_t d = where[h];
      ++a->refs[d];
      a->host_release(h);
      h = d;
    }
    s->swapped = false;
    --a->num_swapped;
  }
  *num_pairs = k;
  return PA_OK;
}

pa_status pa_host_free_list(const pa_allocator* a, int32_t* out, int32_t capacity, int32_t* n) {
  if (!a || !n || capacity < 0 || (capacity > 0 && !out))
    return fail(PA_ERR_INVALID_ARG, "null argument or negative capacity");
  std::lock_guard<std::mutex> g(a->mu);
  if (a->host_count > capacity) return fail(PA_ERR_INVALID_ARG, "capacity too small");
  for (int32_t i = 0; i < a->host_count; ++i)
    out[i] = a->host_ring[(static_cast<int64_t>(a->host_head) + i) % a->num_host];
  *n = a->host_count;
  return PA_OK;
}

int32_t pa_host_ref_count(const pa_allocator* a, int32_t block) {
  if (!a) return -1;
  std::lock_guard<std::mutex> g(a->mu);
  if (block < 0 || block >= a->num_host) return -1;
  return a->host_refs[block];
}

pa_status pa_order_longest_first(const int32_t* context_lens, int32_t n, int32_t* order) {
  if (n < 0 || (n > 0 && (!context_lens || !order))) return fail(PA_ERR_INVALID_ARG, "null argument");
  std::iota(order, order + n, 0);
  std::stable_sort(order, order + n,
                   [context_lens](int32_t x, int32_t y) { return context_lens[x] > context_lens[y]; });
  return PA_OK;
}

pa_status pa_shared_prefix_groups(const int32_t* tables, const int32_t* context_lens, int32_t n, int32_t max_blocks,
                                  int32_t block_size, int32_t* group_start, int32_t* prefix_len,
                                  int32_t* num_groups, int32_t* max_group_size) {
  if (n < 0 || max_blocks < 0 || block_size <= 0 || !group_start || !num_groups || !max_group_size ||
      (n > 0 && (!tables || !context_lens || !prefix_len)))
    return fail(PA_ERR_INVALID_ARG, "null argument or negative size");
  auto used = [&](int32_t i) -> int32_t {  // table entries holding the sequence's tokens
    const int64_t nb = (static_cast<int64_t>(std::max(context_lens[i], 0)) + block_size - 1) / block_size;
    return static_cast<int32_t>(std::min<int64_t>(nb, max_blocks));
  };
  auto row = [&](int32_t i) { return tables + static_cast<int64_t>(i) * max_blocks; };
  int32_t groups = 0, widest = n > 0 ? 1 : 0;
  int32_t i = 0;
  while (i < n) {
    // consecutive sequences whose first block is the leader's
    int32_t stop = i + 1;
    if (used(i) > 0)
      while (stop < n && used(stop) > 0 && row(stop)[0] == row(i)[0]) ++stop;
    if (stop - i > 1) {
      // the group's row: its longest member (the first of them); each member's prefix is
      // the leading blocks it shares with that row, capped at its context (the row's own
      // prefix is its whole context)
      int32_t r = i;
      for (int32_t m = i + 1; m < stop; ++m)
        if (context_lens[m] > context_lens[r]) r = m;
      group_start[groups++] = i;
      for (int32_t m = i; m < stop; ++m) {
        const int64_t n_m = std::max(context_lens[m], 0);
        int32_t j = 0;
        const int32_t lim = std::min(used(m), used(r));
        while (j < lim && row(m)[j] == row(r)[j]) ++j;
        prefix_len[m] = static_cast<int32_t>(m == r ? n_m : std::min<int64_t>(static_cast<int64_t>(j) * block_size, n_m));
      }
      widest = std::max(widest, stop - i);
    } else {  // nothing shared: a group of one
      group_start[groups++] = i;
      prefix_len[i] = 0;
    }
    i = stop;
  }
  group_start[groups] = n;
  *num_groups = groups;
  *max_group_size = widest;
  return PA_OK;
}

}  // extern "C"

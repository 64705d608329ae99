// block_manager.cpp -- host-side block manager and contiguous reservation
// allocator (include/pagedkv_blocks.h).
//
// The manager keeps, per physical block, a reference count and the number of
// token slots written in it, and per sequence its length and block table
// ("PagedAttention", shubhamtatvamasi.com, sections "The idea: page the KV
// cache" and "Sharing and copy-on-write").  Appending a token takes a new
// block only when the last one is full; a shared, partially filled last block
// is copied first (copy-on-write), and the copy pair is handed to the caller
// for copy_blocks.  All of it is ordinary host code: a decode step costs a
// few operations per sequence.

#include <algorithm>
#include <iterator>
#include <map>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"
#include "../../include/pagedkv_blocks.h"

struct pkv_block_manager {
  int32_t num_blocks, block_size, max_seqs, max_blocks_per_seq;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refcount;    // per physical block
  std::vector<int32_t> stored;      // token slots written, per physical block
  std::vector<char> live;           // per sequence id
  std::vector<int32_t> len;         // per sequence id
  std::vector<std::vector<int32_t>> table;

  // Prefix caching ("PagedAttention", shubhamtatvamasi.com, "Sharing and
  // copy-on-write": requests with the same system prompt share blocks).  A
  // full prompt block is registered under its content -- the key of the
  // prefix before it and its token ids -- and a later prompt whose leading
  // blocks have the same contents takes those blocks instead of new ones.
  // A registered block whose last reference goes stays registered, on the
  // evictable list (oldest release first), until an allocation finds the
  // free stack empty and reuses it.
  bool prefix_cache = false;
  std::vector<char> registered;          // per block
  std::vector<uint64_t> parent;          // key of the prefix before a block
  std::vector<int32_t> block_tokens;     // [num_blocks * block_size]
  std::vector<uint64_t> key;             // per registered block
  std::unordered_map<uint64_t, int32_t> index;  // key -> block
  std::map<int64_t, int32_t> evictable;  // release stamp -> block
  std::vector<int64_t> stamp;            // per block on the evictable list
  int64_t next_stamp = 0;
  int64_t hit_blocks = 0;

  int64_t available() const {
    return (int64_t)free_stack.size() + (int64_t)evictable.size();
  }
  int32_t take() {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
    } else {  // reuse the longest-released cached block
      b = evictable.begin()->second;
      evictable.erase(evictable.begin());
      unregister(b);
    }
    refcount[b] = 1;
    stored[b] = 0;
    return b;
  }
  void drop(int32_t b) {
    if (--refcount[b] != 0) return;
    if (prefix_cache && registered[b]) {
      stamp[b] = next_stamp++;
      evictable[stamp[b]] = b;
    } else {
      free_stack.push_back(b);
    }
  }
  void unregister(int32_t b) {
    const auto it = index.find(key[b]);
    if (it != index.end() && it->second == b) index.erase(it);
    registered[b] = 0;
  }
  bool seq_ok(int32_t s) const { return s >= 0 && s < max_seqs; }
};

namespace {

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

// Key of a full block: FNV-1a over the key of the prefix before it (0 for a
// sequence's first block) and its token ids, so a key stands for the whole
// prefix through that block.  A lookup also compares the stored parent key
// and tokens, so a collision of the final hash only costs a miss.
constexpr uint64_t kRootKey = 0;

uint64_t block_key(uint64_t parent, const int32_t* toks, int32_t n) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&](uint32_t v) {
    for (int i = 0; i < 4; ++i) {
      h ^= (v >> (8 * i)) & 0xFFu;
      h *= 1099511628211ull;
    }
  };
  mix((uint32_t)parent);
  mix((uint32_t)(parent >> 32));
  for (int32_t i = 0; i < n; ++i) mix((uint32_t)toks[i]);
  return h;
}

// The registered block with these contents, or -1.
int32_t lookup(const pkv_block_manager* bm, uint64_t parent,
               const int32_t* toks) {
  const int32_t bs = bm->block_size;
  const auto it = bm->index.find(block_key(parent, toks, bs));
  if (it == bm->index.end()) return -1;
  const int32_t b = it->second;
  if (bm->parent[b] != parent) return -1;
  if (!std::equal(toks, toks + bs, bm->block_tokens.begin() + (int64_t)b * bs))
    return -1;
  return b;
}

}  // namespace

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size,
                                 int32_t max_seqs, int32_t max_blocks_per_seq) {
  if (num_blocks < 1 || block_size < 1 || max_seqs < 1 || max_blocks_per_seq < 1)
    return nullptr;
  if ((int64_t)num_blocks * block_size > INT32_MAX) return nullptr;  // slots are int32
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager;
  if (!bm) return nullptr;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->max_seqs = max_seqs;
    bm->max_blocks_per_seq = max_blocks_per_seq;
    bm->free_stack.reserve(num_blocks);
    for (int32_t b = num_blocks - 1; b >= 0; --b) bm->free_stack.push_back(b);
    bm->refcount.assign(num_blocks, 0);
    bm->stored.assign(num_blocks, 0);
    bm->live.assign(max_seqs, 0);
    bm->len.assign(max_seqs, 0);
    bm->table.resize(max_seqs);
  } catch (...) {
    delete bm;
    return nullptr;
  }
  return bm;
}

pkv_block_manager* pkv_bm_create_prefix_cached(int32_t num_blocks,
                                               int32_t block_size,
                                               int32_t max_seqs,
                                               int32_t max_blocks_per_seq) {
  pkv_block_manager* bm =
      pkv_bm_create(num_blocks, block_size, max_seqs, max_blocks_per_seq);
  if (!bm) return nullptr;
  try {
    bm->prefix_cache = true;
    bm->registered.assign(num_blocks, 0);
    bm->parent.assign(num_blocks, 0);
    bm->block_tokens.assign((size_t)num_blocks * block_size, 0);
    bm->key.assign(num_blocks, 0);
    bm->stamp.assign(num_blocks, 0);
  } catch (...) {
    delete bm;
    return nullptr;
  }
  return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_add_sequence_tokens(pkv_block_manager* bm, int32_t seq,
                               const int32_t* tokens, int32_t num_tokens,
                               int32_t* slots_out, int32_t* cached_tokens_out) {
  if (!bm) return PKV_ERR_NULL;
  if (!bm->seq_ok(seq) || num_tokens < 0) return PKV_ERR_SHAPE;
  if (num_tokens > 0 && !tokens) return PKV_ERR_NULL;
  if (bm->live[seq]) return PKV_ERR_SEQ;
  const int32_t bs = bm->block_size;
  const int64_t nb = blocks_for(num_tokens, bs);
  if (nb > bm->max_blocks_per_seq) return PKV_ERR_SHAPE;
  // the leading full blocks whose contents are registered
  std::vector<int32_t> hits;
  if (bm->prefix_cache) {
    uint64_t prev = kRootKey;
    for (int64_t i = 0; i < num_tokens / bs; ++i) {
      const int32_t b = lookup(bm, prev, tokens + i * bs);
      if (b < 0) break;
      hits.push_back(b);
      prev = bm->key[b];
    }
  }
  int64_t hits_evictable = 0;
  for (int32_t b : hits)
    if (bm->refcount[b] == 0) ++hits_evictable;
  if (nb - (int64_t)hits.size() > bm->available() - hits_evictable)
    return PKV_ERR_NO_BLOCKS;
  std::vector<int32_t>& t = bm->table[seq];
  t.clear();
  for (int32_t b : hits) {  // taken off the evictable list first
    if (bm->refcount[b] == 0) bm->evictable.erase(bm->stamp[b]);
    ++bm->refcount[b];
    t.push_back(b);
  }
  bm->hit_blocks += (int64_t)hits.size();
  // the new full blocks are registered under the key chain of the prefix,
  // until a key turns out to be taken (a hash collision: stop registering)
  uint64_t prev = hits.empty() ? kRootKey : bm->key[hits.back()];
  bool chain = bm->prefix_cache;
  for (int64_t i = (int64_t)hits.size(); i < nb; ++i) {
    const int32_t b = bm->take();
    const int64_t left = num_tokens - i * bs;
    bm->stored[b] = (int32_t)std::min<int64_t>(left, bs);
    if (chain && left >= bs) {
      const uint64_t k = block_key(prev, tokens + i * bs, bs);
      if (!bm->index.count(k)) {
        bm->index[k] = b;
        bm->key[b] = k;
        bm->parent[b] = prev;
        std::copy(tokens + i * bs, tokens + (i + 1) * bs,
                  bm->block_tokens.begin() + (int64_t)b * bs);
        bm->registered[b] = 1;
        prev = k;
      } else {
        chain = false;
      }
    }
    t.push_back(b);
  }
  bm->live[seq] = 1;
  bm->len[seq] = num_tokens;
  if (slots_out)
    for (int32_t k = 0; k < num_tokens; ++k)
      slots_out[k] = t[k / bs] * bs + k % bs;
  if (cached_tokens_out) *cached_tokens_out = (int32_t)hits.size() * bs;
  return PKV_OK;
}

int pkv_bm_prefix_stats(const pkv_block_manager* bm, int64_t* registered,
                        int64_t* evictable, int64_t* hit_blocks) {
  if (!bm) return PKV_ERR_NULL;
  int64_t r = 0;
  if (bm->prefix_cache)
    for (int32_t b = 0; b < bm->num_blocks; ++b) r += bm->registered[b];
  if (registered) *registered = r;
  if (evictable) *evictable = (int64_t)bm->evictable.size();
  if (hit_blocks) *hit_blocks = bm->hit_blocks;
  return PKV_OK;
}

int pkv_bm_add_sequence(pkv_block_manager* bm, int32_t seq, int32_t num_tokens,
                        int32_t* slots_out) {
  if (!bm) return PKV_ERR_NULL;
  if (!bm->seq_ok(seq) || num_tokens < 0) return PKV_ERR_SHAPE;
  if (bm->live[seq]) return PKV_ERR_SEQ;
  const int64_t nb = blocks_for(num_tokens, bm->block_size);
  if (nb > bm->max_blocks_per_seq) return PKV_ERR_SHAPE;
  if (nb > bm->available()) return PKV_ERR_NO_BLOCKS;
  std::vector<int32_t>& t = bm->table[seq];
  t.clear();
  for (int64_t i = 0; i < nb; ++i) {
    const int32_t b = bm->take();
    const int64_t left = num_tokens - i * bm->block_size;
    bm->stored[b] = (int32_t)std::min<int64_t>(left, bm->block_size);
    t.push_back(b);
  }
  bm->live[seq] = 1;
  bm->len[seq] = num_tokens;
  if (slots_out)
    for (int32_t k = 0; k < num_tokens; ++k)
      slots_out[k] = t[k / bm->block_size] * bm->block_size + k % bm->block_size;
  return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* bm, int32_t parent, int32_t child) {
  if (!bm) return PKV_ERR_NULL;
  if (!bm->seq_ok(parent) || !bm->seq_ok(child)) return PKV_ERR_SHAPE;
  if (!bm->live[parent] || bm->live[child] || parent == child) return PKV_ERR_SEQ;
  bm->table[child] = bm->table[parent];
  for (int32_t b : bm->table[child]) ++bm->refcount[b];
  bm->len[child] = bm->len[parent];
  bm->live[child] = 1;
  return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* bm, const int32_t* seqs, int32_t n,
                  int32_t* slot_mapping, int32_t* pairs_out,
                  int32_t* num_pairs_out, int32_t* copy_tokens_out) {
  if (!bm) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  if (n > 0 && (!seqs || !slot_mapping || !pairs_out)) return PKV_ERR_NULL;
  if (!num_pairs_out) return PKV_ERR_NULL;
  const int32_t bs = bm->block_size;
  // dry run in batch order: which sequences take a block, with the reference
  // counts the copies earlier in the batch leave behind
  std::unordered_map<int32_t, int32_t> dropped;  // block -> references dropped
  std::unordered_map<int32_t, char> seen;
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = seqs[i];
    if (!bm->seq_ok(s)) return PKV_ERR_SHAPE;
    if (!bm->live[s] || seen.count(s)) return PKV_ERR_SEQ;
    seen[s] = 1;
    const int32_t L = bm->len[s];
    if (L % bs == 0) {  // no block yet, or the last one is full
      if (L / bs + 1 > bm->max_blocks_per_seq) return PKV_ERR_SHAPE;
      ++need;
    } else {
      const int32_t last = bm->table[s].back();
      const auto it = dropped.find(last);
      const int32_t rc = bm->refcount[last] - (it == dropped.end() ? 0 : it->second);
      if (rc > 1) {
        ++need;
        ++dropped[last];
      }
    }
  }
  if (need > bm->available()) return PKV_ERR_NO_BLOCKS;
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = seqs[i];
    std::vector<int32_t>& t = bm->table[s];
    const int32_t L = bm->len[s];
    if (L % bs == 0) {
      t.push_back(bm->take());
    } else if (bm->refcount[t.back()] > 1) {
      const int32_t old = t.back();
      const int32_t fresh = bm->take();
      bm->stored[fresh] = bm->stored[old];
      bm->drop(old);
      t.back() = fresh;
      pairs_out[2 * np] = old;
      pairs_out[2 * np + 1] = fresh;
      if (copy_tokens_out) copy_tokens_out[np] = bm->stored[old];
      ++np;
    }
    const int32_t b = t.back();
    ++bm->stored[b];
    slot_mapping[i] = b * bs + L % bs;
    bm->len[s] = L + 1;
  }
  *num_pairs_out = np;
  return PKV_OK;
}

int pkv_bm_free(pkv_block_manager* bm, int32_t seq) {
  if (!bm) return PKV_ERR_NULL;
  if (!bm->seq_ok(seq)) return PKV_ERR_SHAPE;
  if (!bm->live[seq]) return PKV_ERR_SEQ;
  for (int32_t b : bm->table[seq]) bm->drop(b);
  bm->table[seq].clear();
  bm->len[seq] = 0;
  bm->live[seq] = 0;
  return PKV_OK;
}

int pkv_bm_tables(const pkv_block_manager* bm, const int32_t* seqs, int32_t n,
                  int32_t* tables, int32_t row_stride, int32_t fill,
                  int32_t* lens) {
  if (!bm) return PKV_ERR_NULL;
  if (n < 0 || row_stride < bm->max_blocks_per_seq) return PKV_ERR_SHAPE;
  if (n > 0 && (!seqs || !tables)) return PKV_ERR_NULL;
  for (int32_t i = 0; i < n; ++i) {
    if (!bm->seq_ok(seqs[i])) return PKV_ERR_SHAPE;
    if (!bm->live[seqs[i]]) return PKV_ERR_SEQ;
  }
  for (int32_t i = 0; i < n; ++i) {
    const std::vector<int32_t>& t = bm->table[seqs[i]];
    int32_t* row = tables + (int64_t)i * row_stride;
    std::copy(t.begin(), t.end(), row);
    std::fill(row + t.size(), row + row_stride, fill);
    if (lens) lens[i] = bm->len[seqs[i]];
  }
  return PKV_OK;
}

int pkv_bm_blocks_unshared(const pkv_block_manager* bm, const int32_t* seqs,
                           int32_t n, int32_t* unshared) {
  if (!bm || !unshared) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  if (n > 0 && !seqs) return PKV_ERR_NULL;
  for (int32_t i = 0; i < n; ++i) {
    if (!bm->seq_ok(seqs[i])) return PKV_ERR_SHAPE;
    if (!bm->live[seqs[i]]) return PKV_ERR_SEQ;
  }
  std::vector<uint8_t> seen(bm->num_blocks, 0);
  *unshared = 1;
  for (int32_t i = 0; i < n && *unshared; ++i) {
    for (const int32_t b : bm->table[seqs[i]]) {
      if (seen[b]) {
        *unshared = 0;
        break;
      }
      seen[b] = 1;
    }
  }
  return PKV_OK;
}

int pkv_bm_get_stats(const pkv_block_manager* bm, pkv_bm_stats* out) {
  if (!bm || !out) return PKV_ERR_NULL;
  pkv_bm_stats st{};
  st.free_blocks = bm->available();
  for (int32_t b = 0; b < bm->num_blocks; ++b) {
    if (bm->refcount[b] == 0) continue;
    ++st.used_blocks;
    if (bm->refcount[b] > 1) ++st.shared_blocks;
    st.stored_tokens += bm->stored[b];
  }
  for (int32_t s = 0; s < bm->max_seqs; ++s)
    if (bm->live[s]) {
      ++st.live_sequences;
      st.logical_tokens += bm->len[s];
    }
  st.wasted_slots = st.used_blocks * bm->block_size - st.stored_tokens;
  *out = st;
  return PKV_OK;
}

int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->refcount[block];
}

int32_t pkv_bm_seq_len(const pkv_block_manager* bm, int32_t seq) {
  if (!bm || !bm->seq_ok(seq) || !bm->live[seq]) return -1;
  return bm->len[seq];
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Contiguous reservation: each request reserves its maximum length up front
// in one buffer of token slots; free space is a set of gaps (first fit).
// ---------------------------------------------------------------------------
struct pkv_contig_allocator {
  int64_t num_slots;
  int32_t max_requests;
  std::map<int64_t, int64_t> gaps;  // start -> length, disjoint, non-adjacent
  std::vector<int64_t> start, size;  // per request; size 0 = none
};

extern "C" {

pkv_contig_allocator* pkv_ca_create(int64_t num_slots, int32_t max_requests) {
  if (num_slots < 1 || max_requests < 1) return nullptr;
  pkv_contig_allocator* ca = new (std::nothrow) pkv_contig_allocator;
  if (!ca) return nullptr;
  try {
    ca->num_slots = num_slots;
    ca->max_requests = max_requests;
    ca->gaps[0] = num_slots;
    ca->start.assign(max_requests, 0);
    ca->size.assign(max_requests, 0);
  } catch (...) {
    delete ca;
    return nullptr;
  }
  return ca;
}

void pkv_ca_destroy(pkv_contig_allocator* ca) { delete ca; }

int pkv_ca_reserve(pkv_contig_allocator* ca, int32_t req, int64_t num_slots,
                   int64_t* start_out) {
  if (!ca || !start_out) return PKV_ERR_NULL;
  if (req < 0 || req >= ca->max_requests || num_slots < 1) return PKV_ERR_SHAPE;
  if (ca->size[req] != 0) return PKV_ERR_SEQ;
  for (auto it = ca->gaps.begin(); it != ca->gaps.end(); ++it) {
    if (it->second < num_slots) continue;
    const int64_t s = it->first, len = it->second;
    ca->gaps.erase(it);
    if (len > num_slots) ca->gaps[s + num_slots] = len - num_slots;
    ca->start[req] = s;
    ca->size[req] = num_slots;
    *start_out = s;
    return PKV_OK;
  }
  return PKV_ERR_NO_BLOCKS;
}

int pkv_ca_release(pkv_contig_allocator* ca, int32_t req) {
  if (!ca) return PKV_ERR_NULL;
  if (req < 0 || req >= ca->max_requests) return PKV_ERR_SHAPE;
  if (ca->size[req] == 0) return PKV_ERR_SEQ;
  int64_t s = ca->start[req], len = ca->size[req];
  ca->size[req] = 0;
  auto next = ca->gaps.lower_bound(s);
  if (next != ca->gaps.end() && next->first == s + len) {  // merge right
    len += next->second;
    next = ca->gaps.erase(next);
  }
  if (next != ca->gaps.begin()) {  // merge left
    auto prev = std::prev(next);
    if (prev->first + prev->second == s) {
      s = prev->first;
      len += prev->second;
      ca->gaps.erase(prev);
    }
  }
  ca->gaps[s] = len;
  return PKV_OK;
}

int pkv_ca_get_stats(const pkv_contig_allocator* ca, int64_t* free_slots,
                     int64_t* largest_gap, int64_t* reserved_slots) {
  if (!ca) return PKV_ERR_NULL;
  int64_t f = 0, g = 0;
  for (const auto& kv : ca->gaps) {
    f += kv.second;
    g = std::max(g, kv.second);
  }
  if (free_slots) *free_slots = f;
  if (largest_gap) *largest_gap = g;
  if (reserved_slots) *reserved_slots = ca->num_slots - f;
  return PKV_OK;
}

}  // extern "C"

// Block manager of the paged KV cache (host C++, C ABI in include/pa_blocks.h).
//
// Rules ("KV Cache Engineering for LLM Serving", sections 10 and 11;
// rajatmohan.com serving design, "Prefix sharing is where the real win
// lives"; "Taming the token torrent", "Implementing Radix Tree Prefix
// Caching"): a FIFO free list of block ids; every full block is kept under a
// key made of its whole token prefix and the model key, and reused with a
// reference count when another sequence has that exact prefix; a write into
// a block someone else holds goes to a private copy first.
//
// A local (sliding-window) layer's sequence can instead keep a ring table
// ("KV Cache Engineering for LLM Serving", section 3, sliding windows): a
// fixed number of entries, ceil(W / block_size) + 1 for a window of W
// tokens, logical block b at entry b % entries.  When a new block starts,
// the entry it lands on holds the block that has just left the window, and
// that block is written over in place: the sequence holds at most `entries`
// blocks however long it grows, and takes none from the pool once its ring
// is full.  Ring sequences keep no token ids and take part in no prefix
// sharing, since their blocks are rewritten as the window moves on.
//
// Prefix keys are interned: a full-block prefix is the pair (id of the prefix
// one block shorter, the block's tokens) under a model key, looked up in a
// hash map with exact key comparison, so equal prefixes always get the same
// id and different prefixes never do, whichever sequence built them.  An id
// lives while a sequence holds it or a longer interned prefix extends it
// (reference counted), so the table stays as large as the live prefixes.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pa_blocks.h"

namespace {

constexpr uint64_t kRoot = 0;  // id of the empty prefix

struct PrefixKey {
  uint64_t parent;   // id of the prefix one block shorter (kRoot for the first block)
  uint64_t model;
  std::vector<int32_t> tokens;  // this block's tokens
  bool operator==(const PrefixKey& o) const {
    return parent == o.parent && model == o.model && tokens == o.tokens;
  }
};

inline uint64_t mix(uint64_t h, uint64_t v) {
  // splitmix64 finaliser over h ^ v: a well-spread 64-bit hash step.
  uint64_t z = h ^ (v + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2));
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct PrefixKeyHash {
  size_t operator()(const PrefixKey& k) const {
    uint64_t h = mix(k.parent, k.model);
    for (int32_t t : k.tokens) h = mix(h, (uint32_t)t);
    return (size_t)h;
  }
};

struct Prefix {
  uint64_t id;
  int32_t holders;   // sequences holding this prefix + interned prefixes extending it
  int32_t block;     // block stored under this prefix, or -1
  PrefixKey key;     // kept to find the entry again by id
};

constexpr int32_t kReleased = -1;  // table entry released by a sliding-window trim
constexpr int32_t kSwapped = -2;   // table entry whose block was swapped out

struct Sequence {
  std::vector<int32_t> tokens;      // token ids (plain sequences only)
  std::vector<int32_t> table;       // physical block of each logical block (or kReleased / kSwapped);
                                    // ring sequences: of logical block b at entry b % ring
  std::vector<uint64_t> prefixes;   // prefix id of each full block (plain sequences only)
  uint64_t model = 0;
  int64_t len = 0;                  // tokens held
  int32_t ring = 0;                 // ring entries, 0 for a plain table
  bool swapped = false;

  // Table entry of the block holding position pos, or -1 when no entry
  // holds it any more (a ring whose entry has moved on).
  int64_t entry(int64_t pos, int32_t bs) const {
    const int64_t b = pos / bs;
    if (!ring) return b;
    const int64_t nb = (len + bs - 1) / bs;
    return b < nb - ring ? -1 : b % ring;
  }
};

}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0, block_size = 0;
  std::deque<int32_t> free_list;              // front = next to hand out
  std::vector<int32_t> ref;                   // references per block
  std::vector<uint64_t> stored;               // prefix id a block is stored under (0 = none)
  std::unordered_map<PrefixKey, uint64_t, PrefixKeyHash> ids;   // key -> prefix id
  std::unordered_map<uint64_t, Prefix> prefixes;                // id -> entry
  std::unordered_map<int64_t, Sequence> seqs;
  uint64_t next_id = 1;
  int64_t hits = 0, misses = 0;

  // Existing prefix id of (parent, model, tokens[b0, b0 + bs)), or 0.
  uint64_t find(uint64_t parent, uint64_t model, const int32_t* tokens) const {
    PrefixKey k{parent, model, std::vector<int32_t>(tokens, tokens + block_size)};
    auto it = ids.find(k);
    return it == ids.end() ? 0 : it->second;
  }

  // Prefix id of the block, interned if new; the caller's reference is added.
  uint64_t hold(uint64_t parent, uint64_t model, const int32_t* tokens) {
    PrefixKey k{parent, model, std::vector<int32_t>(tokens, tokens + block_size)};
    auto it = ids.find(k);
    uint64_t id;
    if (it != ids.end()) {
      id = it->second;
    } else {
      id = next_id++;
      ids.emplace(k, id);
      prefixes.emplace(id, Prefix{id, 0, -1, k});
      if (parent != kRoot) prefixes.at(parent).holders++;
    }
    prefixes.at(id).holders++;
    return id;
  }

  // Drops one reference to a prefix id; entries nobody holds are removed,
  // which releases the reference they held on the prefix they extend.
  void drop(uint64_t id) {
    while (id != kRoot) {
      Prefix& p = prefixes.at(id);
      if (--p.holders > 0) return;
      const uint64_t parent = p.key.parent;
      ids.erase(p.key);
      prefixes.erase(id);
      id = parent;
    }
  }

  int32_t take() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    ref[b] = 1;
    return b;
  }

  void release(int32_t b) {
    if (--ref[b] > 0) return;
    const uint64_t id = stored[b];
    if (id != 0) {
      auto it = prefixes.find(id);
      if (it != prefixes.end() && it->second.block == b) it->second.block = -1;
      stored[b] = 0;
    }
    free_list.push_back(b);
  }

  // Store a just-completed block under its prefix unless one is stored.
  void store(int32_t b, uint64_t id) {
    Prefix& p = prefixes.at(id);
    if (p.block < 0) {
      p.block = b;
      stored[b] = id;
    }
  }
};

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1) return PA_ERR_SHAPE;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager();
  if (!bm) return PA_ERR_SHAPE;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  bm->stored.assign(num_blocks, 0);
  for (int32_t b = 0; b < num_blocks; ++b) bm->free_list.push_back(b);
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status pa_bm_add_sequence(pa_block_manager* bm, int64_t seq, const int32_t* tokens,
                             int32_t n, uint64_t model_key, int32_t* reused) {
  if (!bm) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n > 0 && !tokens) return PA_ERR_NULL;
  if (bm->seqs.count(seq)) return PA_ERR_NOT_FOUND;
  const int32_t bs = bm->block_size;
  const int32_t full = n / bs;
  // Count the blocks to take before changing anything.  A prefix that is
  // not interned has no interned extension either, so every later full
  // block is new too.
  int32_t need = (n % bs) ? 1 : 0;
  {
    uint64_t parent = kRoot;
    bool interned = true;
    for (int32_t i = 0; i < full; ++i) {
      const uint64_t id = interned ? bm->find(parent, model_key, tokens + (int64_t)i * bs) : 0;
      if (id == 0) {
        interned = false;
        ++need;
        continue;
      }
      if (bm->prefixes.at(id).block < 0) ++need;
      parent = id;
    }
  }
  if (need > (int32_t)bm->free_list.size()) return PA_ERR_NO_BLOCKS;
  Sequence s;
  s.model = model_key;
  s.tokens.assign(tokens, tokens + n);
  s.len = n;
  int32_t hit_count = 0;
  uint64_t parent = kRoot;
  for (int32_t i = 0; i < full; ++i) {
    const uint64_t id = bm->hold(parent, model_key, tokens + (int64_t)i * bs);
    Prefix& p = bm->prefixes.at(id);
    int32_t b;
    if (p.block >= 0) {
      b = p.block;
      bm->ref[b]++;
      ++hit_count;
    } else {
      b = bm->take();
      bm->store(b, id);
    }
    s.table.push_back(b);
    s.prefixes.push_back(id);
    parent = id;
  }
  if (n % bs) s.table.push_back(bm->take());
  bm->hits += hit_count;
  bm->misses += (int64_t)s.table.size() - hit_count;
  bm->seqs.emplace(seq, std::move(s));
  if (reused) *reused = hit_count;
  return PA_OK;
}

pa_status pa_bm_add_ring_sequence(pa_block_manager* bm, int64_t seq, int32_t n, int32_t window,
                                  int32_t* ring_entries) {
  if (!bm) return PA_ERR_NULL;
  if (n < 0 || window < 1 || n >= INT32_MAX - 16) return PA_ERR_SHAPE;
  if (bm->seqs.count(seq)) return PA_ERR_NOT_FOUND;
  const int32_t bs = bm->block_size;
  const int64_t ring = ((int64_t)window + bs - 1) / bs + 1;
  if (ring > INT32_MAX / 2) return PA_ERR_SHAPE;
  const int64_t nb = ((int64_t)n + bs - 1) / bs;
  const int64_t held = std::min<int64_t>(nb, ring);
  if (held > (int64_t)bm->free_list.size()) return PA_ERR_NO_BLOCKS;
  Sequence s;
  s.len = n;
  s.ring = (int32_t)ring;
  s.table.assign((size_t)ring, kReleased);
  for (int64_t b = nb - held; b < nb; ++b) s.table[b % ring] = bm->take();
  bm->misses += held;
  bm->seqs.emplace(seq, std::move(s));
  if (ring_entries) *ring_entries = (int32_t)ring;
  return PA_OK;
}

pa_status pa_bm_slots(const pa_block_manager* bm, int64_t seq, int32_t first, int32_t count,
                      int64_t* slots) {
  if (!bm || (!slots && count > 0)) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  const Sequence& s = it->second;
  if (s.swapped) return PA_ERR_SWAPPED;
  if (first < 0 || count < 0 || (int64_t)first + count > s.len) return PA_ERR_SHAPE;
  const int32_t bs = bm->block_size;
  for (int32_t i = 0; i < count; ++i) {
    const int64_t pos = (int64_t)first + i;
    const int64_t e = s.entry(pos, bs);
    const int32_t b = e < 0 ? -1 : s.table[e];
    slots[i] = b < 0 ? -1 : (int64_t)b * bs + pos % bs;
  }
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end() || bm->seqs.count(child)) return PA_ERR_NOT_FOUND;
  if (it->second.swapped) return PA_ERR_SWAPPED;
  Sequence c = it->second;
  for (int32_t b : c.table)
    if (b >= 0) bm->ref[b]++;
  for (uint64_t id : c.prefixes) bm->prefixes.at(id).holders++;
  bm->seqs.emplace(child, std::move(c));
  return PA_OK;
}

pa_status pa_bm_append_token(pa_block_manager* bm, int64_t seq, int32_t token, int64_t* slot,
                             int32_t* copy_src, int32_t* copy_dst) {
  if (!bm || !slot || !copy_src || !copy_dst) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  Sequence& s = it->second;
  if (s.swapped) return PA_ERR_SWAPPED;
  const int32_t bs = bm->block_size;
  const int64_t pos = s.len;
  if (pos >= INT32_MAX - 16) return PA_ERR_SHAPE;
  if (s.ring) {
    // The entry of the new position's block.  A new block reuses the
    // entry's old block in place when only this sequence holds it; a shared
    // one (after a fork) is let go and a fresh block taken.  Inside a block,
    // a shared block is copied first, as for plain tables.
    const int64_t e = (pos / bs) % s.ring;
    const int32_t old = s.table[e];
    const bool fresh = old < 0 || (pos % bs == 0 && bm->ref[old] > 1);
    const bool copy = !fresh && pos % bs != 0 && bm->ref[old] > 1;
    if ((fresh || copy) && bm->free_list.empty()) return PA_ERR_NO_BLOCKS;
    int32_t src = -1, dst = -1;
    if (fresh) {
      if (old >= 0) bm->release(old);
      s.table[e] = bm->take();
    } else if (copy) {
      src = old;
      dst = bm->take();
      bm->ref[src]--;
      s.table[e] = dst;
    }
    s.len = pos + 1;
    *slot = (int64_t)s.table[e] * bs + pos % bs;
    *copy_src = src;
    *copy_dst = dst;
    return PA_OK;
  }
  const bool new_block = pos % bs == 0;
  if ((new_block || bm->ref[s.table.back()] > 1) && bm->free_list.empty()) return PA_ERR_NO_BLOCKS;
  int32_t src = -1, dst = -1;
  if (new_block) {
    s.table.push_back(bm->take());
  } else if (bm->ref[s.table.back()] > 1) {
    src = s.table.back();
    dst = bm->take();
    bm->ref[src]--;
    s.table.back() = dst;
  }
  s.tokens.push_back(token);
  s.len = pos + 1;
  const int32_t blk = s.table[pos / bs];
  if ((pos + 1) % bs == 0) {
    const uint64_t parent = s.prefixes.empty() ? kRoot : s.prefixes.back();
    const uint64_t id = bm->hold(parent, s.model, s.tokens.data() + (pos + 1 - bs));
    s.prefixes.push_back(id);
    bm->store(blk, id);
  }
  *slot = (int64_t)blk * bs + pos % bs;
  *copy_src = src;
  *copy_dst = dst;
  return PA_OK;
}

pa_status pa_bm_free_sequence(pa_block_manager* bm, int64_t seq) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  for (int32_t b : it->second.table)
    if (b >= 0) bm->release(b);
  for (uint64_t id : it->second.prefixes) bm->drop(id);
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_trim(pa_block_manager* bm, int64_t seq, int32_t keep_tokens, int32_t* released) {
  if (!bm) return PA_ERR_NULL;
  if (keep_tokens < 1) return PA_ERR_SHAPE;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  Sequence& s = it->second;
  if (s.swapped) return PA_ERR_SWAPPED;
  const int32_t bs = bm->block_size;
  const int64_t n = s.len;
  const int64_t first = (n > keep_tokens ? n - keep_tokens : 0) / bs;
  // Logical blocks before `first` that still have an entry.
  const int64_t start = s.ring ? std::max<int64_t>(0, (n + bs - 1) / bs - s.ring) : 0;
  int32_t count = 0;
  for (int64_t i = start; i < first; ++i) {
    const int64_t e = s.ring ? i % s.ring : i;
    if (s.table[e] >= 0) {
      bm->release(s.table[e]);
      s.table[e] = kReleased;
      ++count;
    }
  }
  if (released) *released = count;
  return PA_OK;
}

pa_status pa_bm_swap_out(pa_block_manager* bm, int64_t seq, int32_t* blocks, int32_t capacity,
                         int32_t* n) {
  if (!bm || !n || (!blocks && capacity > 0)) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  Sequence& s = it->second;
  if (s.swapped) return PA_ERR_SWAPPED;
  int32_t count = 0;
  for (int32_t b : s.table)
    if (b >= 0 && bm->ref[b] == 1) ++count;
  if (count > capacity) return PA_ERR_SHAPE;
  int32_t k = 0;
  for (int32_t& b : s.table) {
    if (b >= 0 && bm->ref[b] == 1) {
      blocks[k++] = b;
      bm->release(b);
      b = kSwapped;
    }
  }
  s.swapped = true;
  *n = count;
  return PA_OK;
}

pa_status pa_bm_swap_in(pa_block_manager* bm, int64_t seq, int32_t* blocks, int32_t capacity,
                        int32_t* n) {
  if (!bm || !n || (!blocks && capacity > 0)) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  Sequence& s = it->second;
  if (!s.swapped) return PA_ERR_SWAPPED;
  int32_t count = 0;
  for (int32_t b : s.table)
    if (b == kSwapped) ++count;
  if (count > capacity) return PA_ERR_SHAPE;
  if (count > (int32_t)bm->free_list.size()) return PA_ERR_NO_BLOCKS;
  int32_t k = 0;
  for (size_t i = 0; i < s.table.size(); ++i) {
    if (s.table[i] != kSwapped) continue;
    const int32_t b = bm->take();
    s.table[i] = b;
    blocks[k++] = b;
    if (i < s.prefixes.size()) bm->store(b, s.prefixes[i]);
  }
  s.swapped = false;
  *n = count;
  return PA_OK;
}

int32_t pa_bm_num_free(const pa_block_manager* bm) {
  return bm ? (int32_t)bm->free_list.size() : -1;
}

pa_status pa_bm_sequence_info(const pa_block_manager* bm, int64_t seq, int32_t* num_tokens,
                              int32_t* num_blocks) {
  if (!bm || !num_tokens || !num_blocks) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  *num_tokens = (int32_t)it->second.len;
  *num_blocks = (int32_t)it->second.table.size();
  return PA_OK;
}

pa_status pa_bm_block_table(const pa_block_manager* bm, int64_t seq, int32_t* out,
                            int32_t capacity) {
  if (!bm || (!out && capacity > 0)) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  const std::vector<int32_t>& t = it->second.table;
  if ((int64_t)t.size() > capacity) return PA_ERR_SHAPE;
  std::copy(t.begin(), t.end(), out);
  return PA_OK;
}

pa_status pa_bm_refcount(const pa_block_manager* bm, int32_t block, int32_t* ref) {
  if (!bm || !ref) return PA_ERR_NULL;
  if (block < 0 || block >= bm->num_blocks) return PA_ERR_SHAPE;
  *ref = bm->ref[block];
  return PA_OK;
}

pa_status pa_bm_stats(const pa_block_manager* bm, int64_t* hits, int64_t* misses) {
  if (!bm || !hits || !misses) return PA_ERR_NULL;
  *hits = bm->hits;
  *misses = bm->misses;
  return PA_OK;
}

pa_status pa_bm_batch(const pa_block_manager* bm, const int64_t* seqs, int32_t n,
                      int32_t max_blocks, int32_t* block_tables, int32_t* seq_lens) {
  if (!bm) return PA_ERR_NULL;
  if (n < 0 || max_blocks < 0) return PA_ERR_SHAPE;
  if (n == 0) return PA_OK;
  if (!seqs || !seq_lens || (!block_tables && max_blocks > 0)) return PA_ERR_NULL;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
    if (it->second.swapped) return PA_ERR_SWAPPED;
    if ((int64_t)it->second.table.size() > max_blocks) return PA_ERR_SHAPE;
    if (it->second.ring && it->second.ring != max_blocks) return PA_ERR_SHAPE;
  }
  for (int32_t i = 0; i < n; ++i) {
    const Sequence& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = block_tables + (int64_t)i * max_blocks;
    std::fill(row, row + max_blocks, -1);
    std::copy(s.table.begin(), s.table.end(), row);
    seq_lens[i] = (int32_t)s.len;
  }
  return PA_OK;
}

}  // extern "C"

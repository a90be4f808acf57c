// Host-side plan of the shared-prefix (cascade) decode: which runs of full
// blocks a batch's sequences share, and the work and storage of the decode
// that attends to each run once for all of its sequences.
//
// Sharing follows from the block tables alone: two sequences share logical
// block j when their tables agree on blocks 0..j and block j is full for
// both ("Taming the token torrent", "Implementing Radix Tree Prefix
// Caching": a sequence reusing a prefix points its table at the existing
// blocks).  A segment is a maximal run of positions shared by one and the
// same set of at least two sequences; the tables are walked as a tree of
// block-id paths, splitting the sequences at each position by their block
// there.  Each sequence's private part starts after its last shared block.
#include <algorithm>
#include <map>
#include <new>
#include <vector>

#include "../../include/pa.h"
#include "../../include/pa_cascade.h"

struct pa_cascade_plan {
  int32_t num_seqs = 0, max_blocks = 0, members_per_group = 0, chunk_blocks = 0;
  std::vector<int32_t> segments;        // [n][4]: first block, blocks, members offset, members
  std::vector<int32_t> seg_blocks;      // block ids, per segment chunk item (see items)
  std::vector<int32_t> members;         // member sequences of every segment, in order
  std::vector<int32_t> items;           // [n][8]
  std::vector<int32_t> parts_off, parts;
  std::vector<int32_t> private_tables, private_lens;
  int32_t num_slots = 0;
  int64_t shared_tokens = 0, segment_tokens = 0;
};

namespace {

struct Segment {
  int32_t first, blocks;
  std::vector<int32_t> members;
};

// Splits `group` (sequences agreeing on positions < j) by their block at j
// and records the maximal shared runs, depth first; an explicit stack keeps
// deep prefixes off the call stack.
void find_segments(const int32_t* bt, int32_t maxb, const std::vector<int32_t>& full,
                   std::vector<Segment>& out, std::vector<int32_t>& prefix_blocks) {
  struct Frame {
    std::vector<int32_t> group;
    int32_t j;
  };
  std::vector<Frame> stack;
  std::vector<int32_t> all(full.size());
  for (size_t s = 0; s < full.size(); ++s) all[s] = (int32_t)s;
  stack.push_back(Frame{all, 0});
  while (!stack.empty()) {
    Frame f = std::move(stack.back());
    stack.pop_back();
    std::map<int32_t, std::vector<int32_t>> by_block;
    for (int32_t s : f.group)
      if (f.j < full[s]) by_block[bt[(int64_t)s * maxb + f.j]].push_back(s);
    // Children in block-id order; pushed in reverse so they pop in order.
    std::vector<Frame> children;
    for (auto& kv : by_block) {
      std::vector<int32_t>& g = kv.second;
      if (g.size() < 2) continue;
      int32_t k = f.j + 1;
      for (;;) {
        bool same = true;
        for (int32_t s : g)
          if (k >= full[s] || bt[(int64_t)s * maxb + k] != bt[(int64_t)g[0] * maxb + k]) {
            same = false;
            break;
          }
        if (!same) break;
        ++k;
      }
      out.push_back(Segment{f.j, k - f.j, g});
      for (int32_t s : g) prefix_blocks[s] = k;
      children.push_back(Frame{g, k});
    }
    for (auto it = children.rbegin(); it != children.rend(); ++it) stack.push_back(std::move(*it));
  }
}

}  // namespace

extern "C" {

pa_status pa_cascade_plan_build(const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t block_size, int32_t num_kv_heads,
                                int32_t num_q_heads, int32_t chunk_tokens, pa_cascade_plan** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (num_seqs < 0 || max_blocks_per_seq < 0 || block_size < 16 || block_size % 16 != 0 ||
      num_kv_heads < 1 || num_q_heads < 1 || num_q_heads % num_kv_heads != 0 || chunk_tokens < 1)
    return PA_ERR_SHAPE;
  const int32_t G = num_q_heads / num_kv_heads;
  if (G > 16) return PA_ERR_UNSUPPORTED;
  if (num_seqs > 0 && (!block_tables || !seq_lens)) return PA_ERR_NULL;
  pa_cascade_plan* p = new (std::nothrow) pa_cascade_plan();
  if (!p) return PA_ERR_SHAPE;
  const int32_t S = num_seqs, maxb = max_blocks_per_seq, BS = block_size;
  p->num_seqs = S;
  p->max_blocks = maxb;
  p->members_per_group = PA_CASCADE_WAVES * (16 / G);
  p->chunk_blocks = std::min<int32_t>(PA_CASCADE_MAX_CHUNK_BLOCKS, std::max<int32_t>(1, chunk_tokens / BS));

  std::vector<int32_t> full(S), prefix_blocks(S, 0);
  for (int32_t s = 0; s < S; ++s) {
    const int64_t L = seq_lens[s];
    full[s] = (L >= 0 && L <= (int64_t)maxb * BS) ? (int32_t)(L / BS) : 0;
  }
  std::vector<Segment> segs;
  find_segments(block_tables, maxb, full, segs, prefix_blocks);

  const int32_t MG = p->members_per_group, CB = p->chunk_blocks;
  // Slots: per segment, chunk and member; slot_base[i] is the first slot of
  // segment i (chunk c, member k at slot_base + c * members + k).
  std::vector<int32_t> slot_base(segs.size());
  std::vector<std::vector<int32_t>> seq_parts(S);
  int32_t slots = 0;
  for (size_t i = 0; i < segs.size(); ++i) {
    const Segment& g = segs[i];
    const int32_t chunks = (g.blocks + CB - 1) / CB, n = (int32_t)g.members.size();
    slot_base[i] = slots;
    for (int32_t c = 0; c < chunks; ++c)
      for (int32_t k = 0; k < n; ++k) seq_parts[g.members[k]].push_back(slots + c * n + k);
    slots += chunks * n;
    p->segments.insert(p->segments.end(), {g.first, g.blocks, (int32_t)p->members.size(), n});
    p->members.insert(p->members.end(), g.members.begin(), g.members.end());
    p->shared_tokens += (int64_t)g.blocks * BS * n;
    p->segment_tokens += (int64_t)g.blocks * BS;
  }
  p->num_slots = slots;
  // Items: tuples (segment, chunk, KV head), 8 at a time, each tuple's
  // member groups 8 items apart, so that they run on the same XCD (work-
  // groups are dispatched round-robin over 8) and share the chunk's blocks
  // in its L2.  Rows are padded with empty items to keep that alignment.
  for (size_t i = 0; i < segs.size(); ++i) {
    const Segment& g = segs[i];
    const int32_t chunks = (g.blocks + CB - 1) / CB, n = (int32_t)g.members.size();
    const int32_t groups = (n + MG - 1) / MG;
    const int32_t mem_off = p->segments[4 * i + 2];
    std::vector<int32_t> chunk_off(chunks);
    for (int32_t c = 0; c < chunks; ++c) {
      chunk_off[c] = (int32_t)p->seg_blocks.size();
      const int32_t b0 = g.first + c * CB, nb = std::min(CB, g.blocks - c * CB);
      const int32_t s0 = g.members[0];
      for (int32_t b = 0; b < nb; ++b) p->seg_blocks.push_back(block_tables[(int64_t)s0 * maxb + b0 + b]);
    }
    const int32_t tuples = chunks * num_kv_heads;
    for (int32_t t0 = 0; t0 < tuples; t0 += 8) {
      for (int32_t mg = 0; mg < groups; ++mg) {
        for (int32_t t = t0; t < t0 + 8; ++t) {
          if (t >= tuples) {
            p->items.insert(p->items.end(), {0, 0, 0, 0, 0, 0, 0, 0});
            continue;
          }
          const int32_t c = t / num_kv_heads, h = t % num_kv_heads;
          const int32_t nb = std::min(CB, g.blocks - c * CB);
          const int32_t k0 = mg * MG, cnt = std::min(MG, n - k0);
          p->items.insert(p->items.end(),
                          {chunk_off[c], nb, mem_off + k0, cnt, h, slot_base[i] + c * n + k0, 0, 0});
        }
      }
    }
  }
  p->parts_off.assign(S + 1, 0);
  for (int32_t s = 0; s < S; ++s) {
    p->parts_off[s + 1] = p->parts_off[s] + (int32_t)seq_parts[s].size();
    p->parts.insert(p->parts.end(), seq_parts[s].begin(), seq_parts[s].end());
  }
  // Private parts: the blocks after the last shared one, as a table of their own.
  p->private_tables.assign((size_t)S * maxb, -1);
  p->private_lens.assign(S, 0);
  for (int32_t s = 0; s < S; ++s) {
    const int32_t pb = prefix_blocks[s];
    for (int32_t b = pb; b < maxb; ++b)
      p->private_tables[(size_t)s * maxb + (b - pb)] = block_tables[(int64_t)s * maxb + b];
    p->private_lens[s] = seq_lens[s] - pb * BS;   // invalid lengths stay invalid
    if (seq_lens[s] < 0 || (int64_t)seq_lens[s] > (int64_t)maxb * BS) p->private_lens[s] = seq_lens[s];
  }
  *out = p;
  return PA_OK;
}

void pa_cascade_plan_destroy(pa_cascade_plan* plan) { delete plan; }

pa_status pa_cascade_plan_get_info(const pa_cascade_plan* plan, pa_cascade_plan_info* info) {
  if (!plan || !info) return PA_ERR_NULL;
  info->num_segments = (int32_t)(plan->segments.size() / 4);
  info->num_items = (int32_t)(plan->items.size() / 8);
  info->num_slots = plan->num_slots;
  info->num_seg_blocks = (int32_t)plan->seg_blocks.size();
  info->num_members = (int32_t)plan->members.size();
  info->num_parts = (int32_t)plan->parts.size();
  info->members_per_workgroup = plan->members_per_group;
  info->chunk_blocks = plan->chunk_blocks;
  info->shared_tokens = plan->shared_tokens;
  info->segment_tokens = plan->segment_tokens;
  return PA_OK;
}

pa_status pa_cascade_plan_export(const pa_cascade_plan* plan, int32_t* items, int32_t* seg_blocks,
                                 int32_t* members, int32_t* parts_off, int32_t* parts,
                                 int32_t* private_tables, int32_t* private_lens, int32_t* segments) {
  if (!plan) return PA_ERR_NULL;
  auto put = [](const std::vector<int32_t>& v, int32_t* dst) {
    if (dst) std::copy(v.begin(), v.end(), dst);
    return dst != nullptr || v.empty();
  };
  bool ok = put(plan->items, items) & put(plan->seg_blocks, seg_blocks) & put(plan->members, members) &
            put(plan->parts_off, parts_off) & put(plan->parts, parts) &
            put(plan->private_tables, private_tables) & put(plan->private_lens, private_lens);
  if (segments) std::copy(plan->segments.begin(), plan->segments.end(), segments);
  return ok ? PA_OK : PA_ERR_NULL;
}

}  // extern "C"

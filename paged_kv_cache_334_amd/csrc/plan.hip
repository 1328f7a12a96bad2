// Host-side planner for cascade decode: finds groups of sequences whose block
// tables start with the same physical blocks (a prefix shared through the block
// tables, as copy-on-write forks and prefix caching leave it: "PagedAttention
// Explained", "Shared Prefix Caching"; "Master Paged Attention for LLM
// Inference", "How Paged Attention Works: The Mechanics", item 4) and writes
// the plan words the shared-prefix kernel and the suffix pass read.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/pkv.h"
#include "kernels.h"

namespace {

struct Group {
  int32_t prefix_blocks;  // shared run of block ids from the start of every member's table
  int32_t start_blocks;   // where the group's pass starts: its parent's covered end (0 for a root)
  int32_t parent;         // -1 for a root
  int32_t leader;
  std::vector<int32_t> members;
};

struct Planner {
  const int32_t* tables;
  int64_t mb;
  int32_t block_size, min_group_seqs, min_prefix_blocks;
  std::vector<int32_t> full;  // blocks fully inside each context
  std::vector<Group> groups;
  std::vector<int32_t> group_of;

  const int32_t* row(int32_t b) const { return tables + b * mb; }
  // blocks of one prefix-pass iteration (64 tokens), and how many of a run of
  // p shared blocks the pass covers (whole iterations)
  int32_t iter_blocks() const { return 64 % block_size == 0 ? 64 / block_size : 1; }
  int32_t covered(int32_t p) const { return p / iter_blocks() * iter_blocks(); }

  // Groups among `cands` (sorted) that share block ids beyond the parent's run
  // of `shared` blocks: candidates agreeing on the id at position `shared` form
  // a group when there are enough of them and their common run reaches far
  // enough; each group then looks for its own children, and a candidate whose
  // run falls short is searched again from the end of that run.
  void split(const std::vector<int32_t>& cands, int32_t shared, int32_t parent, int level) {
    std::vector<int32_t> order;
    for (int32_t b : cands)
      if (full[b] > shared && (parent >= 0 || full[b] >= min_prefix_blocks)) order.push_back(b);
    // candidates with the same id at `shared` become adjacent (ties keep index order)
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return row(x)[shared] < row(y)[shared]; });
    const int32_t start = parent >= 0 ? covered(groups[parent].prefix_blocks) : 0;
    for (size_t i = 0; i < order.size();) {
      size_t j = i + 1;
      while (j < order.size() && row(order[j])[shared] == row(order[i])[shared]) ++j;
      if ((int)(j - i) >= min_group_seqs) {
        Group g;
        g.members.assign(order.begin() + i, order.begin() + j);
        std::sort(g.members.begin(), g.members.end());
        g.leader = g.members[0];
        int32_t p = full[g.leader];
        for (int32_t b : g.members) p = std::min(p, full[b]);
        const int32_t* lead = row(g.leader);
        for (int32_t b : g.members) {
          const int32_t* r = row(b);
          int32_t k = 0;
          while (k < p && r[k] == lead[k]) ++k;
          p = k;
        }
        g.prefix_blocks = p;
        g.start_blocks = start;
        g.parent = parent;
        // a root needs min_prefix_blocks shared blocks; a child must add that
        // many (and at least one pass iteration) to its parent's coverage
        const bool keep = parent < 0 ? p >= min_prefix_blocks
                                     : covered(p) - start >= std::max(min_prefix_blocks, iter_blocks());
        if (keep) {
          const int32_t gi = (int32_t)groups.size();
          for (int32_t b : g.members) group_of[b] = gi;
          const std::vector<int32_t> members = g.members;
          groups.push_back(std::move(g));
          if (level + 1 < pkv::kMaxPrefixLevels) split(members, p, gi, level + 1);
        } else {
          // too short a common run: its members may still share long runs in
          // smaller sets past it (a short common start, then diverging
          // prompts); look for those at the same level, under the same parent.
          // Every member agrees on ids [0, p], so the position grows and the
          // search ends.
          split(g.members, p, parent, level);
        }
      }
      i = j;
    }
  }
};

}  // namespace

extern "C" size_t pkv_plan_shared_prefix(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                         int32_t max_blocks_per_seq, int32_t block_size, int32_t min_group_seqs,
                                         int32_t min_prefix_blocks, int32_t* plan, size_t plan_words) {
  if (!block_tables || !context_lens || num_seqs <= 0 || max_blocks_per_seq <= 0 || block_size <= 0) return 0;
  Planner pl;
  pl.tables = block_tables;
  pl.mb = max_blocks_per_seq;
  pl.block_size = block_size;
  pl.min_group_seqs = min_group_seqs < 2 ? 2 : min_group_seqs;
  pl.min_prefix_blocks = min_prefix_blocks < 1 ? 1 : min_prefix_blocks;
  pl.full.resize(num_seqs);
  pl.group_of.assign(num_seqs, -1);
  std::vector<int32_t> all(num_seqs);
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t c = context_lens[b] > 0 ? context_lens[b] : 0;
    pl.full[b] = (int32_t)std::min<int64_t>(c / block_size, pl.mb);
    all[b] = b;
  }
  pl.split(all, 0, -1, 0);
  const std::vector<Group>& groups = pl.groups;

  size_t members = 0;
  for (const Group& g : groups) members += g.members.size();
  const size_t need = pkv::kPlanHeader + 2 * (size_t)num_seqs + pkv::kGroupWords * groups.size() + members;
  if (!plan || plan_words < need) return need;

  std::memset(plan, 0, need * sizeof(int32_t));
  int32_t max_prefix = 0;
  for (const Group& g : groups) max_prefix = std::max(max_prefix, g.prefix_blocks);
  plan[0] = pkv::kPlanMagic;
  plan[pkv::kPlanSeqs] = num_seqs;
  plan[pkv::kPlanBlockSize] = block_size;
  plan[pkv::kPlanGroups] = (int32_t)groups.size();
  plan[pkv::kPlanMaxPrefix] = max_prefix;
  plan[pkv::kPlanMembers] = (int32_t)members;
  int32_t* prefix_of = plan + pkv::kPlanHeader;
  int32_t* group_of = prefix_of + num_seqs;
  int32_t* gw = group_of + num_seqs;
  int32_t* mw = gw + pkv::kGroupWords * groups.size();
  for (int b = 0; b < num_seqs; ++b) {
    group_of[b] = pl.group_of[b];
    prefix_of[b] = pl.group_of[b] >= 0 ? groups[pl.group_of[b]].prefix_blocks : 0;
  }
  int32_t begin = 0;
  for (size_t gi = 0; gi < groups.size(); ++gi) {
    const Group& g = groups[gi];
    int32_t* w = gw + pkv::kGroupWords * gi;
    w[pkv::kGroupPrefix] = g.prefix_blocks;
    w[pkv::kGroupBegin] = begin;
    w[pkv::kGroupCount] = (int32_t)g.members.size();
    w[pkv::kGroupLeader] = g.leader;
    w[pkv::kGroupStart] = g.start_blocks;
    w[pkv::kGroupParent] = g.parent;
    for (int32_t b : g.members) mw[begin++] = b;
  }
  return need;
}

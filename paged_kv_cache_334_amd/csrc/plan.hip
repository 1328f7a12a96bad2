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
  int32_t prefix_blocks;
  int32_t leader;
  std::vector<int32_t> members;
};

}  // namespace

extern "C" size_t pkv_plan_shared_prefix(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                         int32_t max_blocks_per_seq, int32_t block_size, int32_t min_group_seqs,
                                         int32_t min_prefix_blocks, int32_t* plan, size_t plan_words) {
  if (!block_tables || !context_lens || num_seqs <= 0 || max_blocks_per_seq <= 0 || block_size <= 0) return 0;
  if (min_group_seqs < 2) min_group_seqs = 2;
  if (min_prefix_blocks < 1) min_prefix_blocks = 1;
  const int64_t mb = max_blocks_per_seq;
  auto row = [&](int b) { return block_tables + b * mb; };

  // blocks fully inside each context: only those can be shared by every member
  std::vector<int32_t> full(num_seqs);
  std::vector<int32_t> order;
  order.reserve(num_seqs);
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t c = context_lens[b] > 0 ? context_lens[b] : 0;
    full[b] = (int32_t)std::min<int64_t>(c / block_size, mb);
    if (full[b] >= min_prefix_blocks) order.push_back(b);
  }
  // candidates with the same first physical block are adjacent after this sort
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return row(x)[0] < row(y)[0]; });

  std::vector<Group> groups;
  for (size_t i = 0; i < order.size();) {
    size_t j = i + 1;
    while (j < order.size() && row(order[j])[0] == row(order[i])[0]) ++j;
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
      if (p >= min_prefix_blocks) groups.push_back(std::move(g));
    }
    i = j;
  }

  size_t members = 0;
  for (const Group& g : groups) members += g.members.size();
  const size_t need = pkv::kPlanHeader + (size_t)num_seqs + pkv::kGroupWords * groups.size() + members;
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
  int32_t* gw = prefix_of + num_seqs;
  int32_t* mw = gw + pkv::kGroupWords * groups.size();
  int32_t begin = 0;
  for (size_t gi = 0; gi < groups.size(); ++gi) {
    const Group& g = groups[gi];
    gw[pkv::kGroupWords * gi + 0] = g.prefix_blocks;
    gw[pkv::kGroupWords * gi + 1] = begin;
    gw[pkv::kGroupWords * gi + 2] = (int32_t)g.members.size();
    gw[pkv::kGroupWords * gi + 3] = g.leader;
    for (int32_t b : g.members) {
      prefix_of[b] = g.prefix_blocks;
      mw[begin++] = b;
    }
  }
  return need;
}

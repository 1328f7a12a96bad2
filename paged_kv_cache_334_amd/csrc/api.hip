// C ABI of libpkv (declared in include/pkv.h): argument checks, kernel choice,
// split-K planning and launches.  Host code only; no host synchronization.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/pkv.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

pkv_status fail(pkv_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

pkv_status ok() {
  g_last_error.clear();
  return PKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elt_bytes(int32_t dtype) { return dtype == PKV_BF16 ? 2 : 4; }

pkv_status check_pool(const pkv_pool_desc* pool) {
  if (!pool) return fail(PKV_EINVAL, "pool descriptor is NULL");
  if (pool->num_blocks <= 0 || pool->num_kv_heads <= 0 || pool->block_size <= 0 || pool->head_dim <= 0)
    return fail(PKV_EINVAL, "pool sizes must be positive");
  if (pool->dtype != PKV_F32 && pool->dtype != PKV_BF16) return fail(PKV_EUNSUPPORTED, "dtype must be F32 or BF16");
  if (pool->block_size != 8 && pool->block_size != 16 && pool->block_size != 32)
    return fail(PKV_EUNSUPPORTED, "block_size must be 8, 16 or 32");
  if (pool->head_dim != 64 && pool->head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim must be 64 or 128");
  if ((int64_t)pool->num_blocks * pool->block_size >= (int64_t(1) << 31))
    return fail(PKV_EINVAL, "num_blocks * block_size must stay below 2^31");
  // one block of every kv head, in bytes: the kernels form block offsets as id * that in 32 x 32 -> 64 bits
  if ((int64_t)pool->num_kv_heads * pool->block_size * pool->head_dim * (pool->dtype == PKV_F32 ? 4 : 2) >= (int64_t(1) << 31))
    return fail(PKV_EINVAL, "num_kv_heads * block_size * head_dim * element size must stay below 2^31");
  return PKV_OK;
}

// Workgroups a decode launch should reach before it is worth splitting
// sequences: one per CU of the 256 on MI355X.  Measured on 8 x 32768-token
// sequences: 256 partitions of 8192 tokens stream faster than 512 of 4096.
constexpr int64_t kTargetWorkgroups = 256;

// Automatic split-K partition length in blocks.  One pass per work unit
// (sequence or row tile, kv head) when that already gives kTargetWorkgroups
// workgroups: a split costs a second kernel, the partials' traffic and a
// prologue/epilogue per workgroup, and measured slower than a single long walk
// whenever the GPU is already full.  Fewer units (long contexts, small
// batches) are split into equal partitions until about kTargetWorkgroups
// exist, each wave keeping at least two rounds of in-flight blocks.
int64_t auto_blocks_per_part(int64_t units, int64_t max_blocks, int64_t round, int64_t target = kTargetWorkgroups) {
  if (units >= target || max_blocks <= 2 * round || units == 0) return max_blocks > 0 ? max_blocks : 1;
  const int64_t parts = (target + units - 1) / units;
  int64_t bpp = (max_blocks + parts - 1) / parts;
  if (bpp < 2 * round) bpp = 2 * round;
  return (bpp + round - 1) / round * round;
}

// Partition plan of one decode call.
struct Plan {
  bool mfma = false;
  int group = 1;
  int blocks_per_part = 1;
  int num_parts = 1;
  int inflight = 1;
  int heads_per_wg = 1;
  // cascade over shared prefixes
  bool cascade = false;
  int prefix_tiles = 0;         // 128-row tiles over all groups
  int prefix_chunk_blocks = 0;  // prefix blocks per workgroup
  int prefix_chunks = 0;        // chunk slots per (sequence, query head)
  int prefix_grid_chunks = 0;   // chunks of the longest group
};

// Fewest effective tokens (sum w)^2 / sum w^2 a row's fp16 weights may sit on
// in the LDS-staged kernel, unless the caller says otherwise.  Rounding each
// weight to fp16 moves an output element by sum_t delta_t (v_t - out) / sum w
// with |delta_t| <= 2^-11 w_t: for unit-scale values a standard deviation of
// at most 2^-11 / sqrt(3 n_eff) (about 0.7 of that measured, rounding errors
// being mostly below the half-ulp bound).  At 128 effective tokens that is
// 1.8e-5, so 1e-4 (1% of an output of 1e-2) is more than five of them.
constexpr float kDefaultMinEffTokens = 128.f;
float min_eff_tokens(const pkv_decode_opts* opts) {
  const float v = opts ? opts->min_eff_tokens : 0.f;
  return v == 0.f ? kDefaultMinEffTokens : v;
}
pkv_status check_min_eff(const pkv_decode_opts* opts) {
  if (opts && !(opts->min_eff_tokens >= 0.f)) return fail(PKV_EINVAL, "min_eff_tokens must be >= 0 (or +inf)");
  return PKV_OK;
}

// Prefix-pass workgroups to aim for (two per CU).
constexpr int64_t kPrefixTargetWorkgroups = 512;

// Multi-token calls whose sequences bring at least this many rows (new tokens
// x query heads of one kv head) take the 128-row causal tiles when the caller
// leaves the kernel to the library: from there a tile's single read of each
// block serves enough rows to beat the 32-row tiles' repeated reads.
constexpr int64_t kTileMinRows = 64;
// Largest fp16 value copy the causal tiles make in the workspace (tile_value_copy).
constexpr int64_t kValueCopyMaxBytes = int64_t(1) << 30;

// Reads the host plan words: checks them against the call and sizes the
// prefix pass.  Sets plan->cascade when at least one group exists.
pkv_status plan_cascade(const pkv_pool_desc* pool, int32_t num_seqs, int32_t max_blocks_per_seq, int g,
                        const pkv_decode_opts* opts, Plan* plan) {
  const int32_t* w = opts->prefix_plan;
  const size_t nw = opts->prefix_plan_words;
  if (nw < (size_t)pkv::kPlanHeader || w[0] != pkv::kPlanMagic) return fail(PKV_EINVAL, "prefix plan: bad header");
  if (w[pkv::kPlanSeqs] != num_seqs) return fail(PKV_EINVAL, "prefix plan: made for another number of sequences");
  if (w[pkv::kPlanBlockSize] != pool->block_size) return fail(PKV_EINVAL, "prefix plan: made for another block size");
  const int64_t groups = w[pkv::kPlanGroups], members = w[pkv::kPlanMembers];
  if (groups < 0 || members < 0 ||
      nw < (size_t)(pkv::kPlanHeader + 2 * (int64_t)num_seqs + pkv::kGroupWords * groups + members))
    return fail(PKV_EINVAL, "prefix plan: truncated");
  if (!opts->prefix_plan_dev) return fail(PKV_EINVAL, "prefix plan: device copy missing");
  if (groups == 0) return PKV_OK;
  if (pool->dtype != PKV_BF16 || pool->head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "cascade decode needs bf16 pools with head_dim 128");
  // every index the kernels take from the plan is checked here, once, on the host
  const int bs = pool->block_size;
  const int32_t* start = w + pkv::kPlanHeader;
  const int32_t* group_of = pkv::plan_group_of(w);
  const int32_t* gw = pkv::plan_groups(w);
  const int32_t* mw = gw + pkv::kGroupWords * groups;
  int64_t tiles = 0, longest = 0;
  std::vector<std::pair<int64_t, int64_t>> work;  // (row tiles, blocks the pass covers) per group
  work.reserve(groups);
  std::vector<int32_t> listed(num_seqs, 0);  // groups whose member list holds the sequence
  for (int64_t gi = 0; gi < groups; ++gi) {
    const int32_t* gr = gw + pkv::kGroupWords * gi;
    const int32_t prefix = gr[pkv::kGroupPrefix], begin = gr[pkv::kGroupBegin];
    const int32_t count = gr[pkv::kGroupCount], leader = gr[pkv::kGroupLeader];
    const int32_t gstart = gr[pkv::kGroupStart], parent = gr[pkv::kGroupParent];
    if (prefix <= 0 || count <= 0 || begin < 0 || (int64_t)begin + count > members)
      return fail(PKV_EINVAL, "prefix plan: bad group");
    if (prefix > max_blocks_per_seq || leader < 0 || leader >= num_seqs)
      return fail(PKV_EINVAL, "prefix plan: group does not fit the block tables");
    // a child starts where its parent's pass ends; parents come first, depth is bounded
    if (parent < -1 || parent >= gi) return fail(PKV_EINVAL, "prefix plan: bad parent group");
    const int32_t want_start =
        parent < 0 ? 0 : pkv::prefix_covered_blocks(gw[pkv::kGroupWords * parent + pkv::kGroupPrefix], bs);
    if (gstart != want_start || (parent >= 0 && prefix <= gw[pkv::kGroupWords * parent + pkv::kGroupPrefix]))
      return fail(PKV_EINVAL, "prefix plan: group does not extend its parent");
    int depth = 0;
    for (int32_t a = parent; a >= 0; a = gw[pkv::kGroupWords * a + pkv::kGroupParent]) ++depth;
    if (depth >= pkv::kMaxPrefixLevels) return fail(PKV_EINVAL, "prefix plan: groups nested too deep");
    for (int32_t k = 0; k < count; ++k) {
      const int32_t b = mw[begin + k];
      if (b < 0 || b >= num_seqs || group_of[b] < 0 || group_of[b] >= groups)
        return fail(PKV_EINVAL, "prefix plan: member outside the batch or without a group");
      if (k > 0 && b <= mw[begin + k - 1]) return fail(PKV_EINVAL, "prefix plan: member list not increasing");
      ++listed[b];
      // gi must lie on the member's path from its deepest group to the root;
      // the walk reaches groups whose own words are checked later, so every
      // step must go to a smaller index
      int32_t a = group_of[b];
      while (a > gi) {
        const int32_t up = gw[pkv::kGroupWords * a + pkv::kGroupParent];
        if (up < -1 || up >= a) return fail(PKV_EINVAL, "prefix plan: bad parent group");
        a = up;
      }
      if (a != gi) return fail(PKV_EINVAL, "prefix plan: member not under its group");
    }
    const int64_t t = ((int64_t)count * g + 127) / 128;
    const int64_t n = std::max<int64_t>(pkv::prefix_covered_blocks(prefix, bs) - gstart, 0);
    tiles += t;
    longest = std::max<int64_t>(longest, n);
    work.emplace_back(t, n);
  }
  if (longest <= 0) return PKV_OK;  // every prefix shorter than one pass iteration: plain decode
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t gi = group_of[b];
    if (gi < -1 || gi >= groups || start[b] != (gi < 0 ? 0 : gw[pkv::kGroupWords * gi + pkv::kGroupPrefix]))
      return fail(PKV_EINVAL, "prefix plan: bad per-sequence prefix");
    // every group on the path from the deepest one to the root lists b (each
    // listing group was checked to be on the path): its chunk slots are written
    int32_t path = 0;
    for (int32_t a = gi; a >= 0; a = gw[pkv::kGroupWords * a + pkv::kGroupParent]) ++path;
    if (listed[b] != path) return fail(PKV_EINVAL, "prefix plan: sequence missing from a group on its path");
  }
  if (tiles > 0x7fffffff) return fail(PKV_EUNSUPPORTED, "prefix plan: too many rows");
  const int64_t per_iter = 64 / bs;  // blocks the prefix kernel moves per iteration
  // The shortest chunk (whole iterations) whose workgroups all fit at once: a
  // second, partial round of workgroups would double the pass's time.  Only
  // workgroups whose chunk lies inside their group's blocks count: a nested
  // group covers fewer blocks than the longest, and the rest of its grid
  // slots exit at once.
  auto workgroups = [&](int64_t cb) {
    int64_t n = 0;
    for (const auto& w : work) n += w.first * ((w.second + cb - 1) / cb);
    return n * pool->num_kv_heads;
  };
  int64_t lo = 1, hi = (longest + per_iter - 1) / per_iter;  // chunk length in iterations
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if (workgroups(mid * per_iter) <= kPrefixTargetWorkgroups) hi = mid;
    else lo = mid + 1;
  }
  const int64_t cb = lo * per_iter;
  // chunk slots of the deepest path (each sequence's partials run from the root down)
  int64_t slots = 0;
  for (int32_t b = 0; b < num_seqs; ++b)
    slots = std::max<int64_t>(slots, pkv::path_slots(gw, group_of[b], bs, (int)cb));
  plan->cascade = true;
  plan->prefix_tiles = (int)tiles;
  plan->prefix_chunk_blocks = (int)cb;
  plan->prefix_grid_chunks = (int)((longest + cb - 1) / cb);
  plan->prefix_chunks = (int)slots;
  if (plan->prefix_chunks > 65535) return fail(PKV_EUNSUPPORTED, "prefix plan: too many chunks");
  return PKV_OK;
}

// max_blocks_per_seq: the block tables' row length (INT32_MAX when only sizing the workspace).
pkv_status make_plan(const pkv_pool_desc* pool, int32_t num_seqs, int32_t num_heads, int32_t max_context_len,
                     int32_t max_blocks_per_seq,
                     const pkv_decode_opts* opts, Plan* plan) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_seqs < 0) return fail(PKV_EINVAL, "num_seqs must be >= 0");
  if (num_heads <= 0 || num_heads % pool->num_kv_heads != 0)
    return fail(PKV_EINVAL, "num_heads must be a positive multiple of num_kv_heads");
  if (max_context_len < 0) return fail(PKV_EINVAL, "max_context_len must be >= 0");
  if ((st = check_min_eff(opts)) != PKV_OK) return st;
  const int g = num_heads / pool->num_kv_heads;
  const int bf16 = pool->dtype == PKV_BF16;
  const int kernel = opts ? opts->kernel : PKV_KERNEL_AUTO;
  if (kernel != PKV_KERNEL_AUTO && kernel != PKV_KERNEL_VECTOR && kernel != PKV_KERNEL_MFMA)
    return fail(PKV_EINVAL, "unknown kernel selector");
  const bool mfma_ok = pkv::mfma_supported(bf16, pool->head_dim, pool->block_size, g);
  if (kernel == PKV_KERNEL_MFMA && !mfma_ok)
    return fail(PKV_EUNSUPPORTED, "MFMA kernel needs bf16, head_dim 128 and 4 or 8 query heads per kv head");
  // (blocks of 8, 16 or 32 tokens; 8-token blocks are walked in pairs)
  plan->mfma = (kernel == PKV_KERNEL_MFMA) || (kernel == PKV_KERNEL_AUTO && mfma_ok);
  if (!plan->mfma && !pkv::vector_supported(bf16, pool->head_dim, pool->block_size, g))
    return fail(PKV_EUNSUPPORTED, "query heads per kv head must be 1, 2, 4 or 8");
  plan->group = g;

  const int bs = pool->block_size;
  const int max_blocks = (max_context_len + bs - 1) / bs;
  if (opts && opts->prefix_plan) {
    st = plan_cascade(pool, num_seqs, max_blocks_per_seq, g, opts, plan);
    if (st != PKV_OK) return st;
  }
  const int inflight = opts ? opts->blocks_in_flight : 0;
  if (inflight < 0 || inflight > 2) return fail(PKV_EINVAL, "blocks_in_flight must be 0, 1 or 2");
  // matrix-core kernel: two 16-token sub-tiles in flight per wave (its registers
  // leave room; measured +3.5% on the 70B-shaped batch at 32-token blocks, equal
  // on 8 x 32k), one for the short suffixes after a shared prefix and for pairs
  // of 8-token blocks (their paired loads take the registers: -8% with two);
  // vector kernel: one (measured 1-2% faster than two at occupancy 4 vs 2)
  plan->inflight = inflight ? inflight : ((plan->mfma && bs >= 16 && !plan->cascade) ? 2 : 1);
  const int hpw = opts ? opts->heads_per_workgroup : 0;
  if (hpw < 0 || hpw > 2) return fail(PKV_EINVAL, "heads_per_workgroup must be 0, 1 or 2");
  const bool pairs_ok = !plan->mfma && g == 1 && pool->num_kv_heads % 2 == 0;
  if (hpw == 2 && !pairs_ok) return fail(PKV_EUNSUPPORTED, "two kv heads per workgroup need the vector kernel, one query head per kv head and an even kv-head count");
  if (hpw == 2) {
    if (inflight == 2) return fail(PKV_EUNSUPPORTED, "two kv heads per workgroup take one block in flight");
    plan->inflight = 1;
  }
  plan->heads_per_wg = hpw ? hpw : 1;
  int64_t part_tokens = opts ? opts->partition_tokens : 0;
  if (part_tokens < 0) return fail(PKV_EINVAL, "partition_tokens must be >= 0");
  int64_t bpp;
  if (plan->cascade) {
    // the suffix after a shared prefix is short: one pass, merged with the prefix partials in place
    bpp = max_blocks > 0 ? max_blocks : 1;
  } else if (part_tokens == 0) {
    bpp = auto_blocks_per_part((int64_t)num_seqs * pool->num_kv_heads, max_blocks,
                               (int64_t)pkv::kWaves * plan->inflight);
  } else {
    bpp = (part_tokens + bs - 1) / bs;
  }
  if (bpp < 1) bpp = 1;
  if (bpp >= max_blocks) bpp = max_blocks > 0 ? max_blocks : 1;
  plan->blocks_per_part = (int)bpp;
  plan->num_parts = max_blocks > 0 ? (int)((max_blocks + bpp - 1) / bpp) : 1;
  if (plan->num_parts > 65535) return fail(PKV_EUNSUPPORTED, "too many partitions; raise partition_tokens");
  return PKV_OK;
}

// Plan of one multi-token call (several new tokens per sequence).
struct MultiPlan {
  bool mfma = false;
  bool tile = false;      // 128-row causal tiles staged through LDS (the shared-prefix kernel's causal form)
  int group = 1;
  int col_tiles = 1;      // matrix-core kernel: 16-row column tiles per workgroup
  int rows_per_tile = 1;  // (token, head) rows per workgroup
  int row_tiles = 1;      // workgroup row tiles per (sequence, kv head)
  int inflight = 1;
  int blocks_per_part = 1;
  int num_parts = 1;
  // causal tiles: blocks per sequence in the fp16 value copy (0: no copy), and its bytes
  int copy_blocks = 0;
  size_t copy_bytes = 0;
};

pkv_status make_multi_plan(const pkv_pool_desc* pool, int32_t num_seqs, int32_t num_heads, int32_t num_query_tokens,
                           int32_t max_query_len, int32_t max_context_len, const pkv_decode_opts* opts,
                           MultiPlan* plan) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_query_tokens < 0 || max_query_len < 0 || max_context_len < 0)
    return fail(PKV_EINVAL, "num_seqs, num_query_tokens, max_query_len and max_context_len must be >= 0");
  if (num_heads <= 0 || num_heads % pool->num_kv_heads != 0)
    return fail(PKV_EINVAL, "num_heads must be a positive multiple of num_kv_heads");
  if (num_seqs > 65535 || max_query_len > 65535)
    return fail(PKV_EUNSUPPORTED, "num_seqs and max_query_len must stay below 65536");
  if (opts && opts->tile_value_copy != 0 && opts->tile_value_copy != -1)
    return fail(PKV_EINVAL, "tile_value_copy must be 0 or -1");
  const int g = num_heads / pool->num_kv_heads;
  const int bf16 = pool->dtype == PKV_BF16;
  if ((st = check_min_eff(opts)) != PKV_OK) return st;
  const int kernel = opts ? opts->kernel : PKV_KERNEL_AUTO;
  if (kernel != PKV_KERNEL_AUTO && kernel != PKV_KERNEL_VECTOR && kernel != PKV_KERNEL_MFMA &&
      kernel != PKV_KERNEL_TILE)
    return fail(PKV_EINVAL, "unknown kernel selector");
  if (opts && (opts->prefix_plan || opts->prefix_plan_dev))
    return fail(PKV_EUNSUPPORTED, "a shared-prefix plan is not taken with several new tokens per sequence");
  if (opts && opts->heads_per_workgroup > 1)
    return fail(PKV_EUNSUPPORTED, "several new tokens per sequence take one kv head per workgroup");
  if (opts && opts->heads_per_workgroup < 0) return fail(PKV_EINVAL, "heads_per_workgroup must be 0, 1 or 2");
  const int inflight = opts ? opts->blocks_in_flight : 0;
  if (inflight < 0 || inflight > 2) return fail(PKV_EINVAL, "blocks_in_flight must be 0, 1 or 2");
  const bool mfma_ok = pkv::multi_mfma_supported(bf16, pool->head_dim, pool->block_size, g);
  if ((kernel == PKV_KERNEL_MFMA || kernel == PKV_KERNEL_TILE) && !mfma_ok)
    return fail(PKV_EUNSUPPORTED, "the matrix-core kernels need bf16, head_dim 128 and 1, 2, 4 or 8 query heads per kv head");
  const int qmax = max_query_len > 0 ? max_query_len : 1;
  const int bs = pool->block_size;
  const int64_t max_blocks = (max_context_len + bs - 1) / bs;
  int64_t part_tokens = opts ? opts->partition_tokens : 0;
  if (part_tokens < 0) return fail(PKV_EINVAL, "partition_tokens must be >= 0");
  plan->group = g;
  plan->tile = kernel == PKV_KERNEL_TILE || (kernel == PKV_KERNEL_AUTO && mfma_ok && (int64_t)qmax * g >= kTileMinRows);
  if (plan->tile) {
    // whole 64-token stages per partition
    const int64_t stage = pkv::kPrefixIterTokens / bs;
    plan->rows_per_tile = 128;
    plan->row_tiles = (int)(((int64_t)qmax * g + 127) / 128);
    int64_t bpp = part_tokens == 0
                      ? auto_blocks_per_part((int64_t)num_seqs * pool->num_kv_heads * plan->row_tiles, max_blocks,
                                             stage, kPrefixTargetWorkgroups)
                      : (part_tokens + bs - 1) / bs;
    bpp = (bpp + stage - 1) / stage * stage;
    if (bpp >= max_blocks) bpp = max_blocks > 0 ? max_blocks : 1;
    plan->blocks_per_part = (int)bpp;
    plan->num_parts = max_blocks > 0 ? (int)((max_blocks + bpp - 1) / bpp) : 1;
    if (plan->num_parts > 65535) return fail(PKV_EUNSUPPORTED, "too many partitions; raise partition_tokens");
    // the fp16 value copy: whole stages of every sequence's blocks (a stage past
    // the last block reads zeros there)
    const int64_t copy_blocks = (max_blocks + stage - 1) / stage * stage;
    const int64_t copy_bytes =
        (int64_t)num_seqs * copy_blocks * pool->num_kv_heads * pool->block_size * pool->head_dim * 2;
    if ((!opts || opts->tile_value_copy == 0) && copy_blocks > 0 && copy_bytes <= kValueCopyMaxBytes) {
      plan->copy_blocks = (int)copy_blocks;
      plan->copy_bytes = (size_t)copy_bytes;
    }
    const int64_t units = (int64_t)plan->num_parts * pool->num_kv_heads * num_seqs;
    if ((units + pkv::kXcds - 1) / pkv::kXcds * pkv::kXcds * plan->row_tiles > 0x7fffffff)
      return fail(PKV_EUNSUPPORTED, "too many workgroups; raise partition_tokens");
    return PKV_OK;
  }
  plan->mfma = kernel == PKV_KERNEL_MFMA || (kernel == PKV_KERNEL_AUTO && mfma_ok);
  if (!plan->mfma && !pkv::vector_supported(bf16, pool->head_dim, pool->block_size, g))
    return fail(PKV_EUNSUPPORTED, "query heads per kv head must be 1, 2, 4 or 8");
  const int tile_bytes = pool->block_size * pool->head_dim * elt_bytes(pool->dtype);
  if (plan->mfma) {
    const int64_t rows = (int64_t)qmax * g;
    plan->col_tiles = rows <= 16 ? 1 : 2;
    plan->rows_per_tile = 16 * plan->col_tiles;
    plan->row_tiles = (int)((rows + plan->rows_per_tile - 1) / plan->rows_per_tile);
    if (plan->col_tiles == 2 && inflight == 2)
      return fail(PKV_EUNSUPPORTED, "row tiles of 32 take one block in flight");
    // two blocks in flight for 16-row tiles of 16-token blocks; one otherwise (the
    // 32-row accumulators, or the 8-token block pairs, take the registers)
    plan->inflight = inflight ? inflight : (plan->col_tiles == 1 && pool->block_size == 16 && tile_bytes <= 4096 ? 2 : 1);
  } else {
    plan->rows_per_tile = g;
    plan->row_tiles = qmax;
    plan->inflight = inflight ? inflight : 1;
    if ((int64_t)num_seqs * qmax > 65535)
      return fail(PKV_EUNSUPPORTED, "vector kernel: num_seqs * max_query_len must stay below 65536");
  }
  int64_t bpp = part_tokens == 0 ? auto_blocks_per_part((int64_t)num_seqs * pool->num_kv_heads * plan->row_tiles,
                                                        max_blocks, (int64_t)pkv::kWaves * plan->inflight)
                                 : (part_tokens + bs - 1) / bs;
  if (bpp < 1) bpp = 1;
  if (bpp >= max_blocks) bpp = max_blocks > 0 ? max_blocks : 1;
  plan->blocks_per_part = (int)bpp;
  plan->num_parts = max_blocks > 0 ? (int)((max_blocks + bpp - 1) / bpp) : 1;
  if (plan->num_parts > 65535) return fail(PKV_EUNSUPPORTED, "too many partitions; raise partition_tokens");
  if (plan->mfma) {
    const int64_t units = (int64_t)plan->num_parts * pool->num_kv_heads * num_seqs;
    if ((units + pkv::kXcds - 1) / pkv::kXcds * pkv::kXcds * plan->row_tiles > 0x7fffffff)
      return fail(PKV_EUNSUPPORTED, "too many workgroups; raise partition_tokens");
  }
  return PKV_OK;
}

// Workspace of a multi-token call: split-K partials (num_parts > 1), then the
// causal tiles' fp16 value copy at a 256-byte boundary.
size_t multi_partials(const MultiPlan& plan, int32_t num_query_tokens, int32_t num_heads, int32_t head_dim) {
  if (plan.num_parts <= 1) return 0;
  return (size_t)num_query_tokens * num_heads * plan.num_parts * (2 + (size_t)head_dim) * sizeof(float);
}
size_t multi_workspace(const MultiPlan& plan, int32_t num_query_tokens, int32_t num_heads, int32_t head_dim) {
  const size_t partials = multi_partials(plan, num_query_tokens, num_heads, head_dim);
  if (!plan.copy_bytes) return partials;
  return (partials + 255) / 256 * 256 + plan.copy_bytes;
}

// Workspace: split-K partials (num_parts > 1), then the prefix-pass partials.
size_t split_bytes(const Plan& plan, int32_t num_seqs, int32_t num_heads, int32_t head_dim) {
  if (plan.num_parts <= 1) return 0;
  const size_t rows = (size_t)num_seqs * num_heads * plan.num_parts;
  return rows * (2 + (size_t)head_dim) * sizeof(float);
}

size_t prefix_bytes(const Plan& plan, int32_t num_seqs, int32_t num_heads, int32_t head_dim) {
  if (!plan.cascade) return 0;
  const size_t rows = (size_t)num_seqs * num_heads * plan.prefix_chunks;
  return rows * (2 + (size_t)head_dim) * sizeof(float);
}

size_t workspace_for(const Plan& plan, int32_t num_seqs, int32_t num_heads, int32_t head_dim) {
  return split_bytes(plan, num_seqs, num_heads, head_dim) + prefix_bytes(plan, num_seqs, num_heads, head_dim);
}

// Pass blocks of a checked plan's groups (the fp16 prefix-value copy's blocks).
int64_t prefix_copy_blocks(const pkv_pool_desc* pool, const int32_t* w) {
  const int32_t* gw = pkv::plan_groups(w);
  int64_t n = 0;
  for (int32_t gi = 0; gi < w[pkv::kPlanGroups]; ++gi)
    n += pkv::group_pass_blocks(gw + pkv::kGroupWords * gi, pool->block_size);
  return n;
}

size_t prefix_copy_bytes(const pkv_pool_desc* pool, const int32_t* w) {
  return (size_t)prefix_copy_blocks(pool, w) * pool->num_kv_heads * pool->block_size * pool->head_dim * 2;
}

}  // namespace

extern "C" {

size_t pkv_paged_attn_workspace_bytes(const pkv_pool_desc* pool, int32_t num_seqs, int32_t num_heads,
                                      int32_t max_context_len, const pkv_decode_opts* opts) {
  Plan plan;
  if (make_plan(pool, num_seqs, num_heads, max_context_len, INT32_MAX, opts, &plan) != PKV_OK) return 0;
  return workspace_for(plan, num_seqs, num_heads, pool->head_dim);
}

size_t pkv_prefix_values_f16_bytes(const pkv_pool_desc* pool, const int32_t* plan, size_t plan_words) {
  if (check_pool(pool) != PKV_OK || pool->dtype != PKV_BF16 || pool->head_dim != 128) return 0;
  if (!plan || plan_words < (size_t)pkv::kPlanHeader || plan[0] != pkv::kPlanMagic) return 0;
  // checked as a decode call checks it (any device pointer will do for the size)
  pkv_decode_opts o{};
  o.prefix_plan = plan;
  o.prefix_plan_dev = plan;
  o.prefix_plan_words = plan_words;
  Plan p;
  if (plan_cascade(pool, plan[pkv::kPlanSeqs], INT32_MAX, 1, &o, &p) != PKV_OK || !p.cascade) return 0;
  return prefix_copy_bytes(pool, plan);
}

pkv_status pkv_prefix_values_f16(const void* v_pool, const int32_t* block_tables, int32_t num_seqs,
                                 int32_t max_blocks_per_seq, const pkv_pool_desc* pool, const int32_t* plan,
                                 const int32_t* plan_dev, size_t plan_words, void* out, size_t out_bytes,
                                 void* stream) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (pool->dtype != PKV_BF16 || pool->head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "the fp16 prefix-value copy needs a bf16 pool with head_dim 128");
  if (num_seqs < 0 || max_blocks_per_seq <= 0) return fail(PKV_EINVAL, "bad num_seqs or max_blocks_per_seq");
  if (!plan || !plan_dev) return fail(PKV_EINVAL, "prefix plan: host or device words missing");
  pkv_decode_opts o{};
  o.prefix_plan = plan;
  o.prefix_plan_dev = plan_dev;
  o.prefix_plan_words = plan_words;
  Plan p;
  if ((st = plan_cascade(pool, num_seqs, max_blocks_per_seq, 1, &o, &p)) != PKV_OK) return st;
  if (!p.cascade) return ok();  // no pass blocks: nothing to copy
  const int64_t blocks = prefix_copy_blocks(pool, plan);
  if (blocks > 0x7fffffff) return fail(PKV_EUNSUPPORTED, "prefix plan: too many pass blocks");
  if (!v_pool || !block_tables || !out) return fail(PKV_EINVAL, "a data pointer is NULL");
  if (!aligned16(v_pool) || !aligned16(out)) return fail(PKV_EINVAL, "v_pool and out must be 16-byte aligned");
  if (out_bytes < prefix_copy_bytes(pool, plan))
    return fail(PKV_EINVAL, "out is smaller than pkv_prefix_values_f16_bytes()");
  pkv::PrefixArgs a{};
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.plan = plan_dev;
  a.num_kv_heads = pool->num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = pool->num_blocks;
  a.v_copy = out;
  hipError_t e = pkv::launch_prefix_value_copy(a, pool->block_size, (int)blocks, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_EHIP, std::string("prefix value copy launch: ") + hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Decode with the plan already made (make_plan returned PKV_OK for these arguments).
pkv_status decode_planned(const Plan& plan, const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                          int32_t num_heads, int32_t max_blocks_per_seq, int32_t max_context_len,
                          const pkv_pool_desc* pool, float scale, int32_t out_dtype, void* out, void* workspace,
                          size_t workspace_bytes, const pkv_decode_opts* opts, void* stream) {
  if (num_seqs == 0) return ok();
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out)
    return fail(PKV_EINVAL, "a data pointer is NULL");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return fail(PKV_EINVAL, "q, pools and out must be 16-byte aligned");
  if (max_blocks_per_seq <= 0) return fail(PKV_EINVAL, "max_blocks_per_seq must be positive");
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * pool->block_size)
    return fail(PKV_EINVAL, "max_context_len exceeds max_blocks_per_seq * block_size");
  if (!std::isfinite(scale) || scale < 0.f) return fail(PKV_EINVAL, "scale must be finite and >= 0");
  if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) return fail(PKV_EINVAL, "out_dtype must be F32 or BF16");
  if (pool->dtype == PKV_F32 && out_dtype != PKV_F32) return fail(PKV_EUNSUPPORTED, "f32 inputs need an f32 output");
  const size_t need = workspace_for(plan, num_seqs, num_heads, pool->head_dim);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(PKV_EWORKSPACE, "workspace missing, misaligned or smaller than pkv_paged_attn_workspace_bytes()");
  const bool f16_copy = plan.cascade && opts->prefix_values_f16 != nullptr;
  if (f16_copy && (!aligned16(opts->prefix_values_f16) ||
                   opts->prefix_values_f16_bytes < prefix_copy_bytes(pool, opts->prefix_plan)))
    return fail(PKV_EINVAL, "prefix_values_f16 misaligned or smaller than pkv_prefix_values_f16_bytes()");

  pkv::DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = pool->num_blocks;
  a.max_context = max_context_len;
  a.blocks_per_part = plan.blocks_per_part;
  a.num_parts = plan.num_parts;
  // ordering pays for long walks; after a shared prefix the suffixes are short
  a.longest_first = !plan.cascade && num_seqs > 1 && num_seqs <= pkv::kMaxRankSeqs && max_context_len < (1 << 23);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.out_bf16 = out_dtype == PKV_BF16;
  if (plan.num_parts > 1) {
    const size_t rows = (size_t)num_seqs * num_heads * plan.num_parts;
    float* ws = static_cast<float*>(workspace);
    a.ws_m = ws;
    a.ws_l = ws + rows;
    a.ws_acc = ws + 2 * rows;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bf16 = pool->dtype == PKV_BF16;
  if (plan.cascade) {
    const size_t rows = (size_t)num_seqs * num_heads * plan.prefix_chunks;
    float* pre = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          split_bytes(plan, num_seqs, num_heads, pool->head_dim));
    pkv::PrefixArgs p{};
    p.q = q;
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.block_tables = block_tables;
    p.plan = opts->prefix_plan_dev;
    p.num_heads = num_heads;
    p.num_kv_heads = pool->num_kv_heads;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = pool->num_blocks;
    p.chunk_blocks = plan.prefix_chunk_blocks;
    p.num_chunks = plan.prefix_grid_chunks;
    p.num_slots = plan.prefix_chunks;
    p.num_tiles = plan.prefix_tiles;
    p.scale_log2 = a.scale_log2;
    p.min_eff = min_eff_tokens(opts);
    p.ws_m = pre;
    p.ws_l = pre + rows;
    p.ws_acc = pre + 2 * rows;
    p.v_copy = f16_copy ? const_cast<void*>(opts->prefix_values_f16) : nullptr;
    hipError_t pe = pkv::launch_prefix(p, pool->block_size, plan.group, false, s);
    if (pe != hipSuccess) return fail(PKV_EHIP, std::string("prefix launch: ") + hipGetErrorString(pe));
    a.start_blocks = opts->prefix_plan_dev + pkv::kPlanHeader;
    a.plan = opts->prefix_plan_dev;
    a.prefix_chunks = plan.prefix_chunks;
    a.prefix_chunk_blocks = plan.prefix_chunk_blocks;
    a.pre_m = p.ws_m;
    a.pre_l = p.ws_l;
    a.pre_acc = p.ws_acc;
  }
  hipError_t e = plan.mfma ? pkv::launch_decode_mfma(a, pool->head_dim, pool->block_size, plan.group, plan.inflight, s)
                           : pkv::launch_decode_vector(a, bf16, pool->head_dim, pool->block_size, plan.group,
                                                       plan.inflight, plan.heads_per_wg, s);
  if (e != hipSuccess) return fail(PKV_EHIP, std::string("decode launch: ") + hipGetErrorString(e));
  if (plan.num_parts > 1) {
    e = pkv::launch_splitk_reduce(a, pool->head_dim, pool->block_size, s);
    if (e != hipSuccess) return fail(PKV_EHIP, std::string("reduce launch: ") + hipGetErrorString(e));
  }
  return ok();
}

// Workspace of the allocation-free decode: one array in device memory per
// GPU, part of the library's code object (each device that loads the library
// holds its own copy until the process ends).  Its name is a host-side stand-in
// in host code: kernels get the device address that hipGetSymbolAddress
// returns, looked up once per device and kept.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

pkv_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_EUNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PKV_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attn_decode(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_heads, int32_t max_blocks_per_seq, int32_t max_context_len,
                                 const pkv_pool_desc* pool, float scale, int32_t out_dtype, void* out,
                                 void* workspace, size_t workspace_bytes, const pkv_decode_opts* opts,
                                 void* stream) {
  Plan plan;
  pkv_status st = make_plan(pool, num_seqs, num_heads, max_context_len, max_blocks_per_seq, opts, &plan);
  if (st != PKV_OK) return st;
  return decode_planned(plan, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads, max_blocks_per_seq,
                        max_context_len, pool, scale, out_dtype, out, workspace, workspace_bytes, opts, stream);
}

size_t pkv_paged_attn_decode_scratch_limit(void) { return kScratchBytes; }

pkv_status pkv_paged_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                         int32_t max_context_len, const pkv_pool_desc* pool, float scale,
                                         int32_t out_dtype, void* out, const pkv_decode_opts* opts, void* stream) {
  Plan plan;
  pkv_status st = make_plan(pool, num_seqs, num_heads, max_context_len, max_blocks_per_seq, opts, &plan);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return ok();
  const size_t need = workspace_for(plan, num_seqs, num_heads, pool->head_dim);
  if (need > kScratchBytes)
    return fail(PKV_EWORKSPACE, "the call needs " + std::to_string(need) + " bytes of workspace, above the " +
                                    std::to_string(kScratchBytes) +
                                    " of the library's scratch array; use pkv_paged_attn_decode with a workspace");
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_of_current_device(&ws);
    if (st != PKV_OK) return st;
  }
  return decode_planned(plan, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads, max_blocks_per_seq,
                        max_context_len, pool, scale, out_dtype, out, ws, need > 0 ? kScratchBytes : 0, opts, stream);
}

size_t pkv_paged_attn_multi_token_workspace_bytes(const pkv_pool_desc* pool, int32_t num_seqs, int32_t num_heads,
                                                  int32_t num_query_tokens, int32_t max_query_len,
                                                  int32_t max_context_len, const pkv_decode_opts* opts) {
  MultiPlan plan;
  if (make_multi_plan(pool, num_seqs, num_heads, num_query_tokens, max_query_len, max_context_len, opts, &plan) !=
      PKV_OK)
    return 0;
  return multi_workspace(plan, num_query_tokens, num_heads, pool->head_dim);
}

pkv_status pkv_paged_attn_multi_token(const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      const int32_t* query_start, int32_t num_seqs, int32_t num_heads,
                                      int32_t num_query_tokens, int32_t max_query_len, int32_t max_blocks_per_seq,
                                      int32_t max_context_len, const pkv_pool_desc* pool, float scale,
                                      int32_t out_dtype, void* out, void* workspace, size_t workspace_bytes,
                                      const pkv_decode_opts* opts, void* stream) {
  MultiPlan plan;
  pkv_status st =
      make_multi_plan(pool, num_seqs, num_heads, num_query_tokens, max_query_len, max_context_len, opts, &plan);
  if (st != PKV_OK) return st;
  if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0) return ok();
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start || !out)
    return fail(PKV_EINVAL, "a data pointer is NULL");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return fail(PKV_EINVAL, "q, pools and out must be 16-byte aligned");
  if (max_blocks_per_seq <= 0) return fail(PKV_EINVAL, "max_blocks_per_seq must be positive");
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * pool->block_size)
    return fail(PKV_EINVAL, "max_context_len exceeds max_blocks_per_seq * block_size");
  if (!std::isfinite(scale) || scale < 0.f) return fail(PKV_EINVAL, "scale must be finite and >= 0");
  if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) return fail(PKV_EINVAL, "out_dtype must be F32 or BF16");
  if (pool->dtype == PKV_F32 && out_dtype != PKV_F32) return fail(PKV_EUNSUPPORTED, "f32 inputs need an f32 output");
  const size_t need = multi_workspace(plan, num_query_tokens, num_heads, pool->head_dim);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(PKV_EWORKSPACE,
                "workspace missing, misaligned or smaller than pkv_paged_attn_multi_token_workspace_bytes()");

  pkv::DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = pool->num_blocks;
  a.max_context = max_context_len;
  a.blocks_per_part = plan.blocks_per_part;
  a.num_parts = plan.num_parts;
  // the matrix-core kernel orders sequences longest first (one ranking thread per sequence)
  a.longest_first = plan.mfma && !plan.tile && num_seqs > 1 && num_seqs <= pkv::kMaxRankSeqs && max_context_len < (1 << 23);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.out_bf16 = out_dtype == PKV_BF16;
  a.query_start = query_start;
  a.num_query_tokens = num_query_tokens;
  a.max_query_len = max_query_len;
  a.rows_per_tile = plan.rows_per_tile;
  a.row_tiles = plan.row_tiles;
  if (plan.num_parts > 1) {
    const size_t rows = (size_t)num_query_tokens * num_heads * plan.num_parts;
    float* ws = static_cast<float*>(workspace);
    a.ws_m = ws;
    a.ws_l = ws + rows;
    a.ws_acc = ws + 2 * rows;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bf16 = pool->dtype == PKV_BF16;
  hipError_t e;
  if (plan.tile) {
    pkv::PrefixArgs p{};
    p.q = q;
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.block_tables = block_tables;
    p.num_heads = num_heads;
    p.num_kv_heads = pool->num_kv_heads;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = pool->num_blocks;
    p.chunk_blocks = plan.blocks_per_part;
    p.num_chunks = plan.num_parts;
    p.num_tiles = plan.row_tiles;
    p.scale_log2 = a.scale_log2;
    p.min_eff = min_eff_tokens(opts);
    p.ws_m = a.ws_m;
    p.ws_l = a.ws_l;
    p.ws_acc = a.ws_acc;
    p.context_lens = context_lens;
    p.query_start = query_start;
    p.num_seqs = num_seqs;
    p.num_query_tokens = num_query_tokens;
    p.max_query_len = max_query_len;
    p.max_context = max_context_len;
    p.out = out;
    p.out_bf16 = a.out_bf16;
    p.longest_first = num_seqs > 1 && num_seqs <= pkv::kMaxRankSeqs && max_context_len < (1 << 23);
    if (plan.copy_bytes) {
      p.v_copy = static_cast<char*>(workspace) +
                 (multi_partials(plan, num_query_tokens, num_heads, pool->head_dim) + 255) / 256 * 256;
      p.copy_blocks = plan.copy_blocks;
      e = pkv::launch_value_copy(p, pool->block_size, s);
      if (e != hipSuccess) return fail(PKV_EHIP, std::string("value copy launch: ") + hipGetErrorString(e));
    }
    e = pkv::launch_prefix(p, pool->block_size, plan.group, true, s);
  } else if (plan.mfma) {
    e = pkv::launch_multi_mfma(a, pool->block_size, plan.group, plan.col_tiles, plan.inflight, s);
  } else {
    e = pkv::launch_decode_vector(a, bf16, pool->head_dim, pool->block_size, plan.group, plan.inflight, 1, s);
  }
  if (e != hipSuccess) return fail(PKV_EHIP, std::string("multi-token launch: ") + hipGetErrorString(e));
  if (plan.num_parts > 1) {
    e = pkv::launch_multi_reduce(a, pool->head_dim, pool->block_size, plan.group, s);
    if (e != hipSuccess) return fail(PKV_EHIP, std::string("multi-token reduce launch: ") + hipGetErrorString(e));
  }
  return ok();
}

pkv_status pkv_reshape_and_cache(const void* k, const void* v, int64_t k_token_stride, int64_t v_token_stride,
                                 const int32_t* slot_mapping, int32_t num_tokens, void* k_pool, void* v_pool,
                                 const pkv_pool_desc* pool, void* stream) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return fail(PKV_EINVAL, "num_tokens must be >= 0");
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) return fail(PKV_EINVAL, "a data pointer is NULL");
  const int elt = elt_bytes(pool->dtype);
  const int x = 16 / elt;
  const int64_t dense = (int64_t)pool->num_kv_heads * pool->head_dim;
  const int64_t ks = k_token_stride == 0 ? dense : k_token_stride;
  const int64_t vs = v_token_stride == 0 ? dense : v_token_stride;
  if (ks < dense || vs < dense || ks % x || vs % x)
    return fail(PKV_EINVAL, "token strides must be >= num_kv_heads*head_dim and a multiple of 16 bytes");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PKV_EINVAL, "k, v and pools must be 16-byte aligned");
  hipError_t e = pkv::launch_reshape_and_cache(k, v, ks, vs, slot_mapping, num_tokens, k_pool, v_pool,
                                               pool->num_blocks, pool->num_kv_heads, pool->block_size,
                                               pool->head_dim, elt, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_EHIP, std::string("reshape_and_cache launch: ") + hipGetErrorString(e));
  return ok();
}

pkv_status pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src_dst_pairs, int32_t num_pairs,
                           const pkv_pool_desc* pool, void* stream) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return fail(PKV_EINVAL, "num_pairs must be >= 0");
  if (num_pairs == 0) return ok();
  if (!k_pool || !v_pool || !src_dst_pairs) return fail(PKV_EINVAL, "a data pointer is NULL");
  if (!aligned16(k_pool) || !aligned16(v_pool)) return fail(PKV_EINVAL, "pools must be 16-byte aligned");
  const int64_t block_bytes =
      (int64_t)pool->num_kv_heads * pool->block_size * pool->head_dim * elt_bytes(pool->dtype);
  hipError_t e = pkv::launch_copy_blocks(k_pool, v_pool, src_dst_pairs, num_pairs, pool->num_blocks, block_bytes,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_EHIP, std::string("copy_blocks launch: ") + hipGetErrorString(e));
  return ok();
}

pkv_status pkv_swap_blocks(const void* src_k, const void* src_v, const pkv_pool_desc* src_pool, void* dst_k,
                           void* dst_v, const pkv_pool_desc* dst_pool, const int32_t* src_dst_pairs,
                           int32_t num_pairs, void* stream) {
  pkv_status st = check_pool(src_pool);
  if (st != PKV_OK) return st;
  st = check_pool(dst_pool);
  if (st != PKV_OK) return st;
  if (src_pool->num_kv_heads != dst_pool->num_kv_heads || src_pool->block_size != dst_pool->block_size ||
      src_pool->head_dim != dst_pool->head_dim || src_pool->dtype != dst_pool->dtype)
    return fail(PKV_EINVAL, "source and destination pools differ in shape or dtype");
  if (num_pairs < 0) return fail(PKV_EINVAL, "num_pairs must be >= 0");
  if (num_pairs == 0) return ok();
  if (!src_k || !src_v || !dst_k || !dst_v || !src_dst_pairs) return fail(PKV_EINVAL, "a data pointer is NULL");
  if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v))
    return fail(PKV_EINVAL, "pools must be 16-byte aligned");
  const int64_t block_bytes =
      (int64_t)src_pool->num_kv_heads * src_pool->block_size * src_pool->head_dim * elt_bytes(src_pool->dtype);
  hipError_t e = pkv::launch_swap_blocks(src_k, src_v, src_pool->num_blocks, dst_k, dst_v, dst_pool->num_blocks,
                                         src_dst_pairs, num_pairs, block_bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_EHIP, std::string("swap_blocks launch: ") + hipGetErrorString(e));
  return ok();
}

const char* pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported shape or type";
    case PKV_EWORKSPACE: return "workspace missing or too small";
    case PKV_EHIP: return "HIP runtime error";
    case PKV_ENOSPACE: return "no free block";
  }
  return "unknown status";
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

int32_t pkv_version(void) { return 300; }

}  // extern "C"

// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWaves = 4;          // waves per workgroup in the decode kernels
constexpr int kMaxRankSeqs = 256;  // most sequences the decode kernels order longest-first (one per thread)
constexpr int kXcds = 8;           // MI355X dies (XCDs); workgroup i is dispatched to XCD i % 8

// Everything a decode kernel reads, passed by value as the kernel argument.
struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;       // row stride of block_tables
  int32_t num_blocks;       // pool size, for the block id range check
  int32_t max_context;      // host bound of context_lens; a longer context makes its rows NaN
  int32_t blocks_per_part;  // split-K partition length in blocks
  int32_t num_parts;        // partitions allotted per sequence (grid x)
  int32_t longest_first;    // map sequence slots to sequences by decreasing context length
  float scale_log2;         // scale * log2(e): logits are kept in the base-2 domain
  void* out;
  int32_t out_bf16;
  // Partials when num_parts > 1, each indexed by (row*num_heads + h)*num_parts + part (row = b, or the
  // new token's query row with several per sequence):
  // ws_m (running max, base 2), ws_l (sum of exp2(s - m)), ws_acc (HD floats each).
  float* ws_m;
  float* ws_l;
  float* ws_acc;
  // Cascade (shared-prefix) mode: start_blocks[b] = raw prefix blocks of sequence
  // b's deepest group (NULL: none); the prefix pass covered
  // prefix_covered_blocks() of them.  Its partials, path_slots() of them for
  // the group plan_group_of(plan)[b], sit at (b*num_heads + h)*prefix_chunks + c
  // of pre_*.
  const int32_t* start_blocks;
  const int32_t* plan;
  int32_t prefix_chunks;
  int32_t prefix_chunk_blocks;
  const float* pre_m;
  const float* pre_l;
  const float* pre_acc;
  // Several new tokens per sequence (NULL: one each, the decode step).  New
  // token i of sequence b (n_b = query_start[b+1] - query_start[b] of them)
  // has query/output row query_start[b] + i, sits at position
  // context_lens[b] - n_b + i and sees the tokens up to and including it.
  // Partials are then indexed by that row instead of b.
  const int32_t* query_start;
  int32_t num_query_tokens;  // rows of q and out
  int32_t max_query_len;     // host bound of n_b; the grid covers that many tokens per sequence
  int32_t rows_per_tile;     // (token, head) rows of one kv head a workgroup takes (i-major: row = i*G + h)
  int32_t row_tiles;         // row tiles per (sequence, kv head)
};

// Shared-prefix plan words (built on the host by pkv_plan_shared_prefix):
//   [0] magic  [1] num_seqs  [2] block_size  [3] num_groups  [4] max prefix blocks
//   [5] total members, then prefix_blocks[num_seqs] (prefix of the sequence's
//   deepest group, 0 = none), then group_of[num_seqs] (that group, -1 = none),
//   then per group {prefix_blocks, member_begin, member_count, leader,
//   start_blocks, parent}, then the member lists.  Groups nest (a beam tree):
//   a child group's members are members of its parent, it starts where the
//   parent's pass coverage ends and extends the shared run; parents come first.
constexpr int32_t kPlanMagic = 0x32564b50;  // "PKV2"

// The shared-prefix pass moves 64 tokens per iteration and handles whole
// iterations only: it covers the largest multiple of 64/block_size blocks of
// a group's prefix, and the suffix pass starts there (reading the at most
// 64/block_size - 1 remaining prefix blocks per sequence, from cache).
constexpr int kPrefixIterTokens = 64;
__host__ __device__ constexpr int prefix_covered_blocks(int prefix_blocks, int block_size) {
  return prefix_blocks / (kPrefixIterTokens / block_size) * (kPrefixIterTokens / block_size);
}
constexpr int kPlanSeqs = 1;
constexpr int kPlanBlockSize = 2;
constexpr int kPlanGroups = 3;
constexpr int kPlanMaxPrefix = 4;
constexpr int kPlanMembers = 5;
constexpr int kPlanHeader = 6;
constexpr int kGroupWords = 6;
constexpr int kGroupPrefix = 0, kGroupBegin = 1, kGroupCount = 2, kGroupLeader = 3, kGroupStart = 4, kGroupParent = 5;
constexpr int kMaxPrefixLevels = 4;  // nesting depth of shared-prefix groups

// Plan sections.
__host__ __device__ inline const int32_t* plan_group_of(const int32_t* plan) {
  return plan + kPlanHeader + plan[kPlanSeqs];
}
__host__ __device__ inline const int32_t* plan_groups(const int32_t* plan) {
  return plan + kPlanHeader + 2 * plan[kPlanSeqs];
}
// Prefix chunks of one group (chunk_blocks blocks each, the last one shorter).
// Blocks of a group's own pass, [start, covered end): its part of the fp16
// copy of the prefix values (pkv_prefix_values_f16), in plan order.
__host__ __device__ inline int group_pass_blocks(const int32_t* gr, int block_size) {
  const int n = prefix_covered_blocks(gr[kGroupPrefix], block_size) - gr[kGroupStart];
  return n > 0 ? n : 0;
}

__host__ __device__ inline int group_chunks(const int32_t* gr, int block_size, int chunk_blocks) {
  const int n = prefix_covered_blocks(gr[kGroupPrefix], block_size) - gr[kGroupStart];
  return n > 0 ? (n + chunk_blocks - 1) / chunk_blocks : 0;
}
// Chunk partial slots of a sequence run through its groups from the root:
// group g's chunks sit after those of its ancestors.  Returns the slots of
// the groups from `gi` up to the root.
__host__ __device__ inline int path_slots(const int32_t* groups, int gi, int block_size, int chunk_blocks) {
  int n = 0;
  for (int depth = 0; gi >= 0 && depth < kMaxPrefixLevels; ++depth) {
    const int32_t* gr = groups + kGroupWords * gi;
    n += group_chunks(gr, block_size, chunk_blocks);
    gi = gr[kGroupParent];
  }
  return n;
}

// Everything the shared-prefix kernel reads.
struct PrefixArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* plan;  // device copy of the plan words
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t chunk_blocks;  // prefix blocks per workgroup (causal tiles: blocks per partition)
  int32_t num_chunks;    // chunks of the longest group (grid; causal tiles: partitions per sequence)
  int32_t num_slots;     // chunk slots per (sequence, query head)
  int32_t num_tiles;     // 128-row tiles over all groups (causal tiles: per sequence and kv head)
  float scale_log2;
  float min_eff;  // fewest effective tokens a row's fp16 weights may sit on (+inf: exact path only)
  float* ws_m;
  float* ws_l;
  float* ws_acc;
  // Causal tiles (several new tokens per sequence, the rows of one sequence and
  // kv head in 128-row tiles; plan unused): the multi-token call's arguments,
  // with the same meaning as in DecodeArgs.  One partition: the output rows
  // are written directly; several: partials at (row*num_heads + h)*num_chunks + part.
  const int32_t* context_lens;
  const int32_t* query_start;
  int32_t num_seqs;
  int32_t num_query_tokens;
  int32_t max_query_len;
  int32_t max_context;
  void* out;
  int32_t out_bf16;
  // An fp16 copy of the values the fast path stages (NULL: it converts them
  // in LDS), in the pool's tile layout.  Causal tiles: tile (sequence b,
  // logical block j, kv head h) at ((b * copy_blocks + j) * num_kv_heads + h),
  // tokens past the context zero (made by the call).  Shared-prefix pass: the
  // groups' pass blocks in plan order, tile (block j of group g, kv head h) at
  // ((first_g + j - start_g) * num_kv_heads + h), first_g = the pass blocks
  // of the groups before g (made by pkv_prefix_values_f16).
  void* v_copy;
  int32_t copy_blocks;
  // Causal tiles: sequences in order of decreasing context length (ties by
  // index), each one's row tiles from the last (longest walk) down.  The host
  // sets it for 2..kMaxRankSeqs sequences and max_context < 2^23.
  int32_t longest_first;
};

bool vector_supported(int dtype_bf16, int head_dim, int block_size, int group);
bool mfma_supported(int dtype_bf16, int head_dim, int block_size, int group);

// inflight = blocks whose tiles one wave loads before using the first (1 or 2);
// heads_per_wg = kv heads one workgroup walks together (2 only for group 1, inflight 1)
hipError_t launch_decode_vector(const DecodeArgs& a, int dtype_bf16, int head_dim, int block_size, int group,
                                int inflight, int heads_per_wg, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeArgs& a, int head_dim, int block_size, int group, int inflight,
                              hipStream_t stream);
// causal = false: the shared-prefix pass of cascade decode; true: 128-row
// causal tiles of several new tokens per sequence.
hipError_t launch_prefix(const PrefixArgs& p, int block_size, int group, bool causal, hipStream_t stream);
// Fills p.v_copy for the causal tiles (num_seqs x copy_blocks blocks of num_kv_heads tiles).
hipError_t launch_value_copy(const PrefixArgs& p, int block_size, hipStream_t stream);
// Fills p.v_copy with the fp16 values of the plan's pass blocks (total_blocks of them).
hipError_t launch_prefix_value_copy(const PrefixArgs& p, int block_size, int total_blocks, hipStream_t stream);
hipError_t launch_splitk_reduce(const DecodeArgs& a, int head_dim, int block_size, hipStream_t stream);

// Several new tokens per sequence (a.query_start set).  Matrix-core kernel:
// bf16, head_dim 128, group 1/2/4/8, row tiles of 16 * col_tiles rows
// (col_tiles 1 or 2).  The vector kernel runs one query token per workgroup
// through launch_decode_vector.  The merge handles both.
bool multi_mfma_supported(int dtype_bf16, int head_dim, int block_size, int group);
hipError_t launch_multi_mfma(const DecodeArgs& a, int block_size, int group, int col_tiles, int inflight,
                             hipStream_t stream);
hipError_t launch_multi_reduce(const DecodeArgs& a, int head_dim, int block_size, int group, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* k, const void* v, int64_t k_stride, int64_t v_stride,
                                    const int32_t* slots, int32_t num_tokens, void* k_pool, void* v_pool,
                                    int32_t num_blocks, int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                                    int32_t elt_bytes, hipStream_t stream);
hipError_t launch_swap_blocks(const void* src_k, const void* src_v, int32_t src_blocks, void* dst_k, void* dst_v,
                              int32_t dst_blocks, const int32_t* pairs, int32_t num_pairs, int64_t block_bytes,
                              hipStream_t stream);
hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int32_t num_pairs,
                              int32_t num_blocks, int64_t block_bytes, hipStream_t stream);

}  // namespace pkv

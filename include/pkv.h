/*
 * pkv.h -- C ABI of libpkv, paged KV-cache decode attention for AMD MI355X (gfx950).
 *
 * The operations follow the pages' statement of the problem:
 *
 *  - The KV cache is split into fixed-size blocks (8, 16 or 32 tokens) held in one
 *    preallocated pool; each sequence has a block table mapping its logical
 *    blocks to physical ones, which need not be contiguous ("Master Paged
 *    Attention for LLM Inference", section "How Paged Attention Works: The
 *    Mechanics", items 1-3; "PagedAttention Explained", section "Block Tables
 *    and Non-Contiguous Storage").
 *  - Decode attention follows each sequence's block table, reads its blocks and
 *    attends over their keys and values in logical order, with no gather into
 *    contiguous memory first ("PagedAttention Explained", sections "Block
 *    Tables and Non-Contiguous Storage" and the closing remark of
 *    "Implementing a Simplified Paged KV Cache").
 *  - A new token's key and value go to row `length % block_size` of the last
 *    block of its sequence (same page, "Implementing a Simplified Paged KV
 *    Cache", append_token); here the caller passes that position as a slot.
 *  - Blocks shared between sequences are copied before a sequence writes into
 *    them (copy-on-write; "Master Paged Attention for LLM Inference", item 4 of
 *    "How Paged Attention Works"; "PagedAttention Explained", "Shared Prefix
 *    Caching").
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers; the caller allocates and owns every
 *    buffer (the library allocates nothing).  Pointers to pkv_pool_desc /
 *    pkv_decode_opts are HOST pointers read during the call only.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *    work on it and never synchronize the host.  Calls on different streams may
 *    run concurrently when they write disjoint buffers.
 *  - Host-checkable argument errors return a status before anything is
 *    launched; the message of the last error on the calling thread is
 *    available from pkv_last_error().  Nothing aborts or throws across the ABI.
 *  - Values stored in device memory (block ids, context lengths, slots, copy
 *    pairs) are preconditions the host cannot check without a synchronization.
 *    The kernels still never touch memory outside the pools for a bad value:
 *    an out-of-range block id makes the affected sequence's output rows NaN,
 *    an out-of-range slot or copy pair is skipped.
 *
 * Pool layout (element = bfloat16 or float32; x = 16 / element bytes, i.e. one
 * 16-byte chunk; N blocks, Hkv kv heads, bs = block_size, D = head_dim):
 *  - key pool   [N][Hkv][D/x][bs][x]: key (block p, head h, row t, dim d) at
 *                element ((p*Hkv + h)*(D/x) + d/x)*(bs*x) + t*x + d%x
 *  - value pool [N][Hkv][D][bs]:      value (p, h, t, d) at element
 *                ((p*Hkv + h)*D + d)*bs + t
 *  Each (block, kv head) tile of either pool is one contiguous bs*D-element
 *  region.  Rows of a block at or past a sequence's length may hold any bits
 *  (blocks are reused without clearing); they never reach the output.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,         /* bad pointer, size, shape or combination */
  PKV_EUNSUPPORTED = 2,   /* valid but not built: block_size, head_dim, group size, dtype */
  PKV_EWORKSPACE = 3,     /* workspace missing or smaller than required */
  PKV_EHIP = 4,           /* the HIP runtime reported an error at launch */
  PKV_ENOSPACE = 5        /* block manager: no free block left for the request (nothing changed) */
} pkv_status;

/* Shapes shared by both pools. Supported: block_size 8, 16 or 32, head_dim 64
 * or 128, dtype PKV_F32 or PKV_BF16, num_blocks*block_size < 2^31.  Smaller
 * blocks leave less of a sequence's last block unused but mean more table
 * entries per token; larger ones the reverse ("PagedAttention Explained",
 * "Best Practices", "Choose the Right Block Size").  Every kernel takes all
 * three (the matrix-core decode kernels walk 8-token blocks in pairs; the
 * shared-prefix pass reads four 8-token blocks per 32-token run). */
typedef struct {
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t head_dim;
  int32_t dtype; /* pkv_dtype */
} pkv_pool_desc;

/* Decode kernel family. */
typedef enum {
  PKV_KERNEL_AUTO = 0,   /* MFMA for bf16, head_dim 128 and 4 or 8 query heads per kv head; vector otherwise */
  PKV_KERNEL_VECTOR = 1, /* per-lane dot products with cross-lane reductions (any supported group) */
  PKV_KERNEL_MFMA = 2,   /* grouped query tile on matrix cores (bf16, head_dim 128, group 4 or 8) */
  PKV_KERNEL_TILE = 3    /* multi-token calls only: 128-row causal tiles staged through LDS (bf16,
                            head_dim 128, group 1, 2, 4 or 8); partitions hold whole 64-token stages */
} pkv_kernel;

/* Optional decode settings (pass NULL for defaults). */
typedef struct {
  /* Tokens per split-K partition: 0 = chosen by the library from the shapes;
   * a positive value is rounded up to a whole number of blocks; a value at or
   * above max_context_len means one pass with no partials and no reduce. */
  int32_t partition_tokens;
  int32_t kernel; /* pkv_kernel */
  /* Blocks whose key/value tiles one wave loads before it uses the first:
   * 0 = chosen by the library, else 1 or 2. */
  int32_t blocks_in_flight;
  /* Kv heads one workgroup walks together, sharing the block-id lookups:
   * 0 = chosen by the library, 1, or 2 (one query head per kv head, an even
   * number of kv heads, one block in flight, vector kernel). */
  int32_t heads_per_workgroup;
  /* Cascade decode over shared prefixes (bf16, head_dim 128): the plan words
   * pkv_plan_shared_prefix() wrote for these block tables and context lengths,
   * in HOST memory (read during the call) and the same words copied to DEVICE
   * memory by the caller (read by the kernels).  NULL / 0 = no cascade. */
  const int32_t* prefix_plan;
  const int32_t* prefix_plan_dev;
  size_t prefix_plan_words;
  /* LDS-staged matrix-core kernel (the shared-prefix pass, PKV_KERNEL_TILE):
   * it forms the softmax weights in fp16 against values converted to fp16,
   * and walks a chunk again on its exact path (bf16 values, weights as bf16
   * hi + lo) when a value has no finite fp16 copy, or when some row's weights
   * sit on fewer than this many effective tokens, (sum w)^2 / sum w^2.  Each
   * fp16 weight is off by up to 2^-11 of itself: over many comparable weights
   * that averages out, over a few it can move a small output element by more
   * than 1% of itself.  A chunk whose rows see fewer tokens than this takes
   * the exact path from the start.  0 = the library's value, 128 (1e-4 on an
   * output of 1e-2 is then more than five standard deviations of the rounding
   * error for unit-scale values); +inf = always the exact path; 1 = the fp16
   * path wherever its values fit (error up to 2^-11 * (max |v| + |out|)).
   * Negative or NaN: PKV_EINVAL. */
  float min_eff_tokens;
  /* Multi-token calls on PKV_KERNEL_TILE: 0 = the library's choice, a one-pass
   * fp16 copy of the values the tiles walk, made at the start of the call in
   * the workspace (pkv_paged_attn_multi_token_workspace_bytes counts it) when
   * it takes at most 1 GiB, so that the tiles skip their own conversion;
   * -1 = never (each tile converts the values it stages, in LDS).  Other
   * values: PKV_EINVAL.  Ignored by the other calls and kernels. */
  int32_t tile_value_copy;
  /* Cascade decode: an fp16 copy of this plan's shared-prefix values, made by
   * pkv_prefix_values_f16 (DEVICE memory, 16-byte aligned), and its size in
   * bytes; NULL / 0 = none.  With it the shared-prefix pass stages those
   * values as they are instead of converting the bf16 values it reads to fp16
   * (the same bits; its exact path still reads the pool).  The copy holds as
   * long as the plan and the values of the prefix blocks do not change, which
   * copy-on-write guarantees for blocks that stay shared; the caller makes it
   * again otherwise.  A size below pkv_prefix_values_f16_bytes() for the plan,
   * or a misaligned pointer: PKV_EINVAL.  Ignored without a plan and by the
   * multi-token call. */
  const void* prefix_values_f16;
  size_t prefix_values_f16_bytes;
} pkv_decode_opts;

/*
 * Shared-prefix plan for cascade decode.  Sequences whose block tables start
 * with the same physical blocks share those tokens' keys and values (a common
 * system prompt, forked sequences sharing their history through copy-on-write:
 * "PagedAttention Explained", "Shared Prefix Caching"; "Paged Attention"
 * glossary, "Example").  Attention over such a prefix is computed once for all
 * query rows of the group on matrix cores, each prefix tile read once instead
 * of once per sequence; the rest of each sequence goes through the ordinary
 * paged walk, and the two are merged by their softmax (max, sum) states.  The
 * result equals the plain decode up to rounding.
 *
 * Groups: sequences with at least min_prefix_blocks full blocks whose first
 * block ids agree; the group's prefix is the longest run of identical block ids
 * at the start of every member's table, counting only blocks fully inside every
 * member's context.  Groups with fewer than min_group_seqs members (at least 2)
 * or a prefix shorter than min_prefix_blocks are dropped; the members of a
 * group dropped for a short run are searched again past it, so smaller sets
 * that share a long run behind a short common start still form groups.
 * Groups nest, as the forks of a beam search leave them under a shared system
 * prompt: members of a group that agree on the block id right after its prefix
 * form a child group by the same rule, kept when it extends the blocks the
 * parent's pass covers (whole 64-token iterations) by at least
 * min_prefix_blocks blocks and one iteration; the child's pass starts where the
 * parent's ends.  At most 4 levels.  Each sequence's prefix is that of its
 * deepest group.
 *
 *  block_tables  HOST [num_seqs][max_blocks_per_seq] int32
 *  context_lens  HOST [num_seqs] int32
 *  plan          HOST output of plan_words int32 words, or NULL to query the size
 * Returns the number of words the plan needs (written only when plan is not
 * NULL and plan_words is at least that), or 0 for invalid arguments.  The plan
 * stays valid while the tables' prefix entries and the context lengths do not
 * change; pass it (and a device copy) through pkv_decode_opts.
 */
size_t pkv_plan_shared_prefix(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_blocks_per_seq, int32_t block_size, int32_t min_group_seqs,
                              int32_t min_prefix_blocks, int32_t* plan, size_t plan_words);

/*
 * fp16 copy of a plan's shared-prefix values, for pkv_decode_opts.prefix_values_f16.
 * Shared blocks are read-only while they are shared (a write to one first
 * copies it: "PagedAttention Explained", "Shared Prefix Caching"), so the
 * fp16 form the shared-prefix pass feeds to the matrix cores can be made once
 * per plan and reused by every decode step that uses the plan, instead of once
 * per 128-row tile and step.  Bf16 pools with head_dim 128 only.
 *
 * Layout: the pass blocks of each group in plan order (group g's blocks
 * [start_g, covered end_g) of its leader's table, the blocks its pass walks),
 * each block's values for every kv head in the pool's tile layout, converted
 * to fp16 (round to nearest even; beyond fp16's range: +-inf, which the pass
 * then sends to its exact path).  A block id outside the pool gives zeros.
 *
 * pkv_prefix_values_f16_bytes: bytes of that copy for a HOST plan; 0 for an
 * invalid plan, a pool other than bf16 / head_dim 128, or a plan with no pass
 * blocks.
 *
 * pkv_prefix_values_f16: writes the copy to out (DEVICE, 16-byte aligned, at
 * least that many bytes) on stream, reading v_pool and the block tables
 * (DEVICE) through the plan (HOST words, checked as the decode call checks
 * them, and their DEVICE copy).  No copy needed (no pass blocks): PKV_OK with
 * nothing launched.  Errors, all before anything is launched: PKV_EUNSUPPORTED
 * for a pool other than bf16 / head_dim 128; PKV_EINVAL for a plan that does
 * not check against these tables, a NULL or misaligned pointer, or out_bytes
 * below the copy's size; PKV_EHIP when the launch fails.
 */
size_t pkv_prefix_values_f16_bytes(const pkv_pool_desc* pool, const int32_t* plan, size_t plan_words);
pkv_status pkv_prefix_values_f16(const void* v_pool, const int32_t* block_tables, int32_t num_seqs,
                                 int32_t max_blocks_per_seq, const pkv_pool_desc* pool, const int32_t* plan,
                                 const int32_t* plan_dev, size_t plan_words, void* out, size_t out_bytes,
                                 void* stream);

/* Bytes of workspace pkv_paged_attn_decode needs for these shapes and options
 * (0 when the call runs as a single pass).  Returns 0 for invalid shapes. */
size_t pkv_paged_attn_workspace_bytes(const pkv_pool_desc* pool, int32_t num_seqs, int32_t num_heads,
                                      int32_t max_context_len, const pkv_decode_opts* opts);

/*
 * Paged decode attention: for every sequence b < num_seqs and query head
 * h < num_heads,
 *     out[b][h][:] = sum_t softmax_t(scale * <q[b][h], k_t>) * v_t
 * over the sequence's tokens t < context_lens[b], where token t's key/value
 * are row t % block_size of physical block block_tables[b][t / block_size]
 * for kv head h / (num_heads / num_kv_heads).  context_lens[b] == 0 gives an
 * all-zero output row.  Arithmetic: products and sums in float32, softmax as a
 * running (max, sum) in float32 ("flash" form, exact up to rounding), output
 * rounded to nearest-even when out_dtype is PKV_BF16.
 *
 *  q             [num_seqs][num_heads][head_dim], pool->dtype
 *  k_pool/v_pool pools in the layout above
 *  block_tables  [num_seqs][max_blocks_per_seq] int32; entries past a
 *                sequence's last block may be read (they lie inside the row)
 *                but are never used as block ids, so they may hold anything
 *  context_lens  [num_seqs] int32, each in [0, max_context_len]
 *  max_context_len  host-side upper bound of context_lens (<= max_blocks_per_seq*block_size)
 *  out_dtype     PKV_BF16 or PKV_F32 for bf16 inputs; PKV_F32 for f32 inputs
 *  out           [num_seqs][num_heads][head_dim] out_dtype; must not alias inputs
 *  workspace     device scratch of at least pkv_paged_attn_workspace_bytes(); may be
 *                NULL when that is 0.  Not aliased by other in-flight calls.
 *  scale         finite and >= 0 (the kernels take the maximum of the unscaled
 *                logits); negative values return PKV_EINVAL.
 */
pkv_status pkv_paged_attn_decode(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_heads, int32_t max_blocks_per_seq, int32_t max_context_len,
                                 const pkv_pool_desc* pool, float scale, int32_t out_dtype, void* out,
                                 void* workspace, size_t workspace_bytes, const pkv_decode_opts* opts,
                                 void* stream);

/*
 * pkv_paged_attn_decode without a workspace argument and without any device
 * allocation, for callers that cannot allocate: code recorded into a HIP graph,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * results and errors as pkv_paged_attn_decode (same kernels, same plan), except
 * that the split-K and shared-prefix partials go to a scratch array the library
 * holds in device memory, one per GPU, for the life of the process
 * (pkv_paged_attn_decode_scratch_limit() bytes: 64 MiB).  A call whose
 * pkv_paged_attn_workspace_bytes() exceeds that returns PKV_EWORKSPACE before
 * anything is launched.  The first call on a device looks up that device's
 * array (no allocation).  Every call on one GPU shares its array: calls that
 * overlap in time on one GPU (on different streams, or from different
 * threads) race and must not be issued; calls in order on one stream are
 * fine.  Nothing in the array needs clearing: every partial a call reads, the
 * same call wrote first.
 */
pkv_status pkv_paged_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                         int32_t max_context_len, const pkv_pool_desc* pool, float scale,
                                         int32_t out_dtype, void* out, const pkv_decode_opts* opts, void* stream);
/* Bytes of the per-GPU scratch array pkv_paged_attn_decode_noalloc uses. */
size_t pkv_paged_attn_decode_scratch_limit(void);

/* Bytes of workspace pkv_paged_attn_multi_token needs (0 for a single pass). */
size_t pkv_paged_attn_multi_token_workspace_bytes(const pkv_pool_desc* pool, int32_t num_seqs, int32_t num_heads,
                                                  int32_t num_query_tokens, int32_t max_query_len,
                                                  int32_t max_context_len, const pkv_decode_opts* opts);
/*
 * Paged attention for several new tokens per sequence, causal among them: the
 * verify step of speculative decoding, or a chunk of a prompt, over the paged
 * cache (the pages name speculative decoding and forked sequences as users of
 * the shared blocks: "Master Paged Attention for LLM Inference", "How Paged
 * Attention Works: The Mechanics", item 4; "What is PagedAttention",
 * "PagedAttention vs Speculative Decoding"; and a prompt's prefill filling
 * the cache: "PagedAttention Explained", "Enabling Automatic Prefix
 * Caching").  The pages give no formula; the mask is the standard causal one.
 *
 * Sequence b has n_b = query_start[b+1] - query_start[b] new tokens, already
 * written to the cache (pkv_reshape_and_cache) as its last n_b of
 * context_lens[b] tokens.  New token i, at position context_lens[b] - n_b + i,
 * has query row r = query_start[b] + i and gets, for every query head h,
 *     out[r][h][:] = sum_t softmax_t(scale * <q[r][h], k_t>) * v_t
 * over the tokens t <= context_lens[b] - n_b + i (itself and everything
 * before it).  One new token per sequence is the decode step.  Arithmetic as
 * in pkv_paged_attn_decode.
 *
 *  q              [num_query_tokens][num_heads][head_dim], pool->dtype
 *  query_start    [num_seqs + 1] int32, device; non-decreasing, within [0, num_query_tokens]
 *  max_query_len  host bound of n_b (the grid covers that many tokens per sequence)
 *  out            [num_query_tokens][num_heads][head_dim] out_dtype
 *  opts           partition_tokens, kernel (the matrix-core kernels take bf16,
 *                 head_dim 128 and 1, 2, 4 or 8 query heads per kv head; AUTO
 *                 picks PKV_KERNEL_TILE for them once max_query_len * group >= 64,
 *                 where each block read serves up to 128 rows, the 32-row
 *                 MFMA tiles below that) and blocks_in_flight (MFMA kernel);
 *                 no shared-prefix plan, one kv head per workgroup.  The tile
 *                 kernel forms fp16 weights against fp16 values (from the
 *                 workspace copy or converted in LDS, tile_value_copy) and
 *                 takes the exact form (bf16 values, weights as bf16 hi + lo)
 *                 where min_eff_tokens says, as the shared-prefix pass does.
 * Other arguments as in pkv_paged_attn_decode.  Device-side preconditions:
 * n_b <= context_lens[b] <= max_context_len and n_b <= max_query_len; a
 * sequence breaking them gets NaN in the rows the grid covers.  A sequence
 * whose query_start entries are out of order or out of range gets nothing
 * written.
 */
pkv_status pkv_paged_attn_multi_token(const void* q, const void* k_pool, const void* v_pool,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      const int32_t* query_start, int32_t num_seqs, int32_t num_heads,
                                      int32_t num_query_tokens, int32_t max_query_len, int32_t max_blocks_per_seq,
                                      int32_t max_context_len, const pkv_pool_desc* pool, float scale,
                                      int32_t out_dtype, void* out, void* workspace, size_t workspace_bytes,
                                      const pkv_decode_opts* opts, void* stream);
/*
 * Cache write: for every token i < num_tokens with slot s = slot_mapping[i] >= 0,
 * copy the bits of k[i][h][:] / v[i][h][:] (all kv heads h) to row s % block_size
 * of block s / block_size of k_pool / v_pool.  Negative slots are skipped.
 *
 *  k, v          token i, head h starts at element i*token_stride + h*head_dim;
 *                token_stride = 0 means num_kv_heads*head_dim (dense [T][Hkv][D])
 *  slot_mapping  [num_tokens] int32; slots must be distinct (else the survivor is unspecified)
 */
pkv_status pkv_reshape_and_cache(const void* k, const void* v, int64_t k_token_stride, int64_t v_token_stride,
                                 const int32_t* slot_mapping, int32_t num_tokens, void* k_pool, void* v_pool,
                                 const pkv_pool_desc* pool, void* stream);

/*
 * Copy-on-write block copy: for every pair i < num_pairs, block
 * src_dst_pairs[2i+1] of both pools (all kv heads) becomes a bit copy of block
 * src_dst_pairs[2i].  Destinations must be distinct and no destination may be
 * a source of another pair (each copy then reads what its source held before
 * the call).  src_dst_pairs is a device array [num_pairs][2] int32.
 */
pkv_status pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src_dst_pairs, int32_t num_pairs,
                           const pkv_pool_desc* pool, void* stream);

/*
 * Block swap between two pools of the same shape: for every pair i, block
 * src_dst_pairs[2i+1] of (dst_k, dst_v) becomes a bit copy of block
 * src_dst_pairs[2i] of (src_k, src_v), all kv heads.  This moves blocks of
 * preempted sequences to a CPU-side pool and back (the swap space that
 * offloads KV-cache blocks to CPU memory: "PagedAttention Explained", section
 * "Programmatic Control Over KV Cache", engine argument swap_space).
 *
 * The two descriptors must agree in kv heads, block size, head dim and dtype
 * (their block counts may differ).  The four pool pointers and src_dst_pairs
 * ([num_pairs][2] int32) must be addressable by the device: device memory, or
 * host memory pinned with hipHostMalloc (torch pin_memory=True), which the
 * kernel reads or writes across the bus.  Destination blocks must be distinct
 * and, when both sides are the same pool, no destination may be a source.  A
 * pair with an id outside its pool is skipped.
 */
pkv_status pkv_swap_blocks(const void* src_k, const void* src_v, const pkv_pool_desc* src_pool, void* dst_k,
                           void* dst_v, const pkv_pool_desc* dst_pool, const int32_t* src_dst_pairs,
                           int32_t num_pairs, void* stream);

/*
 * Host-side block manager: the bookkeeping above the kernels.  It keeps the
 * free list of physical blocks, each sequence's block table and length, and a
 * reference count per block, and turns appends into slots
 * (pkv_reshape_and_cache) and copy-on-write pairs (pkv_copy_blocks).
 *
 * Rules ("PagedAttention Explained", "Implementing a Simplified Paged KV
 * Cache"): a sequence takes a new block from the front of the free list when
 * its length is a multiple of block_size; its next token goes to row
 * length % block_size of its last block (slot = block * block_size + row);
 * freeing a sequence drops one reference from each of its blocks and returns
 * blocks left with none to the back of the free list.  pkv_bm_fork makes a
 * child that shares all of the parent's blocks; the first write of either into
 * a shared, partly filled last block first moves the writer to a copy
 * ("Master Paged Attention for LLM Inference", "How Paged Attention Works: The
 * Mechanics", item 4), and the (source, destination) pair is queued for
 * pkv_bm_take_copies.
 *
 * Prefix caching ("Paged Attention" glossary, "Why it matters";
 * "PagedAttention Explained", "Enabling Automatic Prefix Caching"): when token
 * ids are passed to pkv_bm_append_tokens, every block that fills up is entered
 * in a cache under a hash of all token ids up to its end (64-bit, chained over
 * blocks; a hit also compares the block's own ids and its parent's hash).
 * pkv_bm_add_sequence_cached starts a sequence from a prompt and shares the
 * longest run of cached full blocks at its start (never the block holding the
 * prompt's last token).  A cached block whose last reference is dropped stays
 * in the cache, on the free list, until it is taken for other contents.
 *
 * Host memory only, no HIP calls; one manager must not be used from two
 * threads at once.  Sequence ids are any distinct int64 values.
 */
typedef struct pkv_block_manager pkv_block_manager;
/* free_order: NULL (blocks 0..num_blocks-1) or a permutation giving the initial
 * free-list order.  Returns NULL for bad arguments or no memory. */
pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order);
void pkv_bm_destroy(pkv_block_manager* bm);
/* Message of the manager's last error ("" before any). */
const char* pkv_bm_last_error(const pkv_block_manager* bm);
int32_t pkv_bm_num_free(const pkv_block_manager* bm);
/* References to a block (0 = free), -1 for an id outside the pool. */
int32_t pkv_bm_ref_count(const pkv_block_manager* bm, int32_t block);
/* Full blocks held in the prefix cache. */
int32_t pkv_bm_num_cached(const pkv_block_manager* bm);
pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq);
/* New sequence starting with the prompt tokens[0..num_tokens); shares cached
 * full blocks and writes how many leading tokens they cover to *cached_tokens
 * (a multiple of block_size, < num_tokens).  The caller appends the rest. */
pkv_status pkv_bm_add_sequence_cached(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                                      int32_t* cached_tokens);
pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);
/* Reserve slots for the next num_tokens tokens of seq: slots[0..num_tokens).
 * token_ids may be NULL (the sequence's later blocks then enter no cache).
 * PKV_ENOSPACE when the free list cannot cover the whole request; then nothing
 * changes. */
pkv_status pkv_bm_append_tokens(pkv_block_manager* bm, int64_t seq, int32_t num_tokens, const int32_t* token_ids,
                                int32_t* slots);
/* Copy-on-write pairs queued since the last call, as pairs[2i] = source,
 * pairs[2i+1] = destination.  pairs NULL: returns the count and keeps them;
 * else fills them (max_pairs must cover the count, else -1) and clears the queue. */
int32_t pkv_bm_take_copies(pkv_block_manager* bm, int32_t* pairs, int32_t max_pairs);
pkv_status pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq);
/* Tokens of a sequence, -1 if unknown. */
int32_t pkv_bm_sequence_length(const pkv_block_manager* bm, int64_t seq);
/* Its blocks in logical order (table NULL: count only); -1 if unknown or max_blocks too small. */
int32_t pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq, int32_t* table, int32_t max_blocks);
/* Block tables [num_seqs][max_blocks_per_seq] (entries past a sequence's
 * blocks set to pad) and context lengths [num_seqs] of the listed sequences,
 * in host memory, ready to copy to the device for the attention calls (and to
 * pass to pkv_plan_shared_prefix). */
pkv_status pkv_bm_export_batch(pkv_block_manager* bm, const int64_t* seqs, int32_t num_seqs, int32_t max_blocks_per_seq,
                               int32_t pad, int32_t* block_tables, int32_t* context_lens);
/* Static text for a status code. */
const char* pkv_status_string(pkv_status status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* pkv_last_error(void);

/* Library ABI version (major*10000 + minor*100 + patch). */
int32_t pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */

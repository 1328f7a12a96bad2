// Shared-prefix pass of cascade decode, and 128-row causal tiles of several
// new tokens per sequence (bf16, head_dim 128).
//
// Sequences that reference the same physical blocks for their first P blocks
// (a shared system prompt, a forked beam; "PagedAttention Explained", "Shared
// Prefix Caching"; "Paged Attention" glossary, "Example") would each read
// those blocks again in a per-sequence decode.  Here the prefix is read once
// per kv head for all query rows of the group: rows = (member sequence, query
// head of the kv head), so the per-tile work becomes a dense contraction
// [rows x tokens] = Q . K^T and [rows x D] += P . V, done on matrix cores,
// FlashAttention-style (tiles streamed through LDS, float32 online softmax;
// "Paged Attention" glossary, related term "FlashAttention").  Each workgroup
// covers 128 rows of one group and kv head and one chunk of the prefix, and
// writes a partial (max, sum, acc) per row; the suffix pass merges them.
//
// Causal tiles (a prompt chunk or a verify step appending n_b tokens to
// sequence b; "PagedAttention Explained", "Enabling Automatic Prefix
// Caching"): the same loop over the sequence's own blocks, rows = (new token,
// query head of the kv head), so one read of a block serves up to 128 rows.
// New token i sees the tokens up to its own position: each column has its
// own limit, logits past it become -inf, and the values past the last row's
// limit are zeroed in LDS (they may be another sequence's or NaN).  A
// sequence's walk is one partition (the tile writes its output rows) or
// several of whole 64-token stages (partials for the multi-token merge).
//
// Workgroup = 4 waves x 32 query rows (two 16-column MFMA tiles per wave).
// Per iteration (a stage of 64 tokens) the key and value tiles of the stage
// two ahead travel from memory straight into LDS (global_load_lds; keys in
// two buffers, values in three), each wave converts the values it loaded
// for the next stage to fp16, and one barrier publishes the stage.
// A stage is two runs of 32 tokens (four 8-token blocks, two 16-token
// blocks or one 32-token block).  Each run's logits come from two S tiles whose 16 rows interleave:
// tile X holds tokens 8j + 4X + r (j, r < 4), so after the product the lane of
// group kg owns tokens 8kg..8kg+7 of the run across the two tiles, exactly the
// 8 contraction indices it supplies to P.V, and the value operand is one
// 16-byte piece of a dim's row.
//  * S^T = K . Q^T, v_mfma_f32_16x16x32_bf16: A = keys (lane: the tile's row
//    n, lane group kg -> 16-byte chunk 4i+kg), B = queries (lane: column n,
//    dims 32i+8kg..+7); lane gets S^T[row 4kg+r][column n].
//  * O^T += V^T . P^T over the run, v_mfma_f32_16x16x32_f16: k = 8kg + j is
//    token 8kg + j, B = the lane's own 8 weights, A = values of dim 16nt+n at
//    those tokens.  Weights and values go in as fp16 (11 significant bits: a
//    weight's rounding is at most 2^-11 relative, against 2^-8 for bf16,
//    which left too little room to the 1% output bound in a float64
//    simulation of 30000-token rows).  The values
//    arrive as bf16 and are converted once per stage, in place in LDS, each
//    wave the pieces it loaded; a bf16 value is exact in fp16 within fp16's
//    range.  A chunk holding a value fp16 cannot hold (|v| > 65504, or NaN),
//    a logit far above the first stage's maximum (an infinite weight), or a
//    row whose weights sit on too few effective tokens (p.min_eff), is walked
//    again with bf16 values and weights split into bf16 hi + lo parts (two
//    instructions, ~16 significant bits), the exact form for any input.
// The LDS copy permutes 16-byte pieces so that both operand reads are free of
// bank conflicts (measured with the hardware counter): within a key chunk row
// the tokens of one S tile sit in 16 consecutive slots (key_slot_token), and a
// 32-token value row has its four pieces rotated by bits 1-2 of the dim.
#include <type_traits>

#include "decode_common.h"

namespace pkv {

namespace {

constexpr int HD = 128;
constexpr int TOK = kPrefixIterTokens;  // prefix tokens per iteration
constexpr int NW = kWaves;        // 4
constexpr int ROWS_PER_WAVE = 32; // two MFMA column tiles
constexpr int STAGE_HALF = TOK * HD * 2;  // bytes of keys (or values) per iteration: 16 KiB
constexpr int kPiecesPerWave = STAGE_HALF / 1024 / NW;  // 1 KiB loads per wave per stage, keys (and values): 4

// LDS byte address of a __shared__ location.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from gbase + voff (gbase wave-uniform) into LDS at
// lds + 16*lane.  Issued as inline assembly so that the compiler's own
// counter waits do not treat every LDS read as dependent on it; the caller
// waits with lds_dma_wait_all() before a barrier.
__device__ __forceinline__ void lds_dma16(uint32_t lds, const void* gbase, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds), "v"(voff), "s"(gbase)
      : "memory", "m0");
}
__device__ __forceinline__ void lds_dma_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of the wave's vector-memory loads are outstanding (the
// oldest complete first).
template <int N>
__device__ __forceinline__ void lds_dma_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Token (inside its block) whose key piece sits in slot s of an LDS key chunk
// row.  32-token blocks: slots 0-15 hold S tile 0's rows in order, 16-31 tile
// 1's.  16-token blocks (b = the block's place in its run): the first block
// keeps tile 0's tokens in slots 0-7 and tile 1's in 8-15, the second block the
// other way round, so one tile's read covers both halves of the row's banks.
template <int BS>
__device__ __forceinline__ int key_slot_token(int s, int b) {
  if constexpr (BS == 32) return 8 * ((s >> 2) & 3) + 4 * (s >> 4) + (s & 3);
  else return 8 * ((s >> 2) & 1) + 4 * (((s >> 3) & 1) ^ b) + (s & 3);
}
// Piece of a 32-token value row stored at slot s of dim d (and the inverse).
__device__ __forceinline__ int value_rot(int d) { return (d >> 1) & 3; }

// 8-token blocks: a 32-token run is four blocks, and one S tile's 16 lanes read
// four tokens of each (tokens 4X..4X+3 of block n / 4), whose tiles lie 2 KiB
// apart, i.e. on the same banks.  Block b of the run keeps key chunk c in chunk
// row c ^ (b & 1) and token t in slot t ^ 4(b >> 1) of that row, so the
// sixteen 16-byte reads cover sixteen different slots of a 256-byte bank row.
// Involutive: the same map takes a stored position to the pool's.
__device__ __forceinline__ int key8_row(int c, int b) { return c ^ (b & 1); }
__device__ __forceinline__ int key8_slot(int t, int b) { return t ^ (4 * ((b >> 1) & 1)); }

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two float32 -> packed fp16, round to nearest even (one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// The 16 bytes of values at v (bf16, eight of them) converted to fp16 in
// place.  Returns true when one of them has no finite fp16 copy (|v| > 65504,
// an infinity or a NaN): a packed fma(h, 0, acc) over the converted values
// turns NaN exactly then.
__device__ __forceinline__ bool values_to_f16(unsigned char* v) {
  uint4* piece = reinterpret_cast<uint4*>(v);
  const uint4 w = *piece;
  const uint32_t x[4] = {w.x, w.y, w.z, w.w};
  uint32_t h[4];
  f16x2 acc = {0, 0};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = pack_f16(bf16_lo(x[e]), bf16_hi(x[e]));
    acc = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, h[e]), f16x2{0, 0}, acc);
  }
  *piece = make_uint4(h[0], h[1], h[2], h[3]);
  return __builtin_isnan(acc[0]) || __builtin_isnan(acc[1]);
}

// Bits that keep the first `keep` (0..8) of a 16-byte piece's eight 16-bit
// elements, as four 32-bit masks (element 2e in the low half of word e).
__device__ __forceinline__ uint4 keep_mask(int keep) {
  uint32_t m[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) m[e] = (2 * e < keep ? 0x0000ffffu : 0u) | (2 * e + 1 < keep ? 0xffff0000u : 0u);
  return make_uint4(m[0], m[1], m[2], m[3]);
}
// values_to_f16 for a piece whose elements from `keep` on lie past the tokens
// a causal tile sees: those become zeros first (they may hold anything, NaN
// included, and enter the products with weight zero).
__device__ __forceinline__ void values_to_f16_head(unsigned char* v, int keep) {
  uint4* piece = reinterpret_cast<uint4*>(v);
  const uint4 mk = keep_mask(keep);
  const uint4 w = *piece;
  *piece = make_uint4(w.x & mk.x, w.y & mk.y, w.z & mk.z, w.w & mk.w);
  values_to_f16(v);
}
// Zeros in place of the elements from `keep` on of a 16-byte piece of bf16
// values (they lie past the tokens a causal tile sees and may hold anything,
// NaN included; they enter the products with weight zero).
__device__ __forceinline__ void values_zero_tail(unsigned char* v, int keep) {
  uint4* piece = reinterpret_cast<uint4*>(v);
  const uint4 mk = keep_mask(keep);
  const uint4 w = *piece;
  *piece = make_uint4(w.x & mk.x, w.y & mk.y, w.z & mk.z, w.w & mk.w);
}

static_assert(64 * NW >= kMaxRankSeqs, "longest-first ranking: one sequence per thread");
static_assert(2 * kMaxRankSeqs * sizeof(int) <= STAGE_HALF, "ranking scratch inside one value buffer");

template <int BS, int G, bool CAUSAL>
__global__ __launch_bounds__(64 * NW, 2) void prefix_kernel(PrefixArgs p) {
  constexpr int NB = TOK / BS;          // blocks per iteration
  constexpr int TILE = BS * HD * 2;     // bytes of one (block, kv head) tile
  constexpr int RUN_BYTES = 32 * HD * 2; // one 32-token run of keys (or values)
  static_assert(NB * TILE == STAGE_HALF, "stage size");

  // Keys in two buffers, values in three: a stage's keys are used one
  // iteration before its values (its logits are computed while the previous
  // stage's weights are formed), so values stay one iteration longer.  80 KiB:
  // two workgroups fill the CU's 160 KiB, with nothing else in LDS.
  __shared__ __attribute__((aligned(16))) unsigned char kbuf[2][STAGE_HALF];
  __shared__ __attribute__((aligned(16))) unsigned char vbuf[3][STAGE_HALF];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n = lane & 15;
  const int kg = lane >> 4;
  // XCD-aware order.  Workgroup i runs on XCD i % 8; a unit (kv head, chunk)
  // keeps all its row tiles on one XCD, dispatched back to back, so the tiles
  // after the first find the unit's keys and values in that XCD's L2.
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int unit = (slot / p.num_tiles) * kXcds + xcd;
  // Causal tiles in longest-first order: later row tiles walk more tokens, so
  // a unit's tiles run from the last down (the first one then also brings
  // every key and value the others read into the L2).
  int tile = CAUSAL && p.longest_first ? p.num_tiles - 1 - slot % p.num_tiles : slot % p.num_tiles;

  // What the two modes settle here: the kv head, the chunk's blocks
  // [blk_lo, blk_hi) of block-table row bt, the rows [0, rows) of the unit and
  // this wave's first row, and the query row of each (row_q).
  int kvh, blk_lo, blk_hi, rows;
  const int32_t* bt;
  // cascade: the group's members and the slot of the chunk's partials
  const int32_t* members = nullptr;
  int slot0 = 0;
  // shared-prefix pass: the group's first block in the fp16 value copy, and
  // the block of the group's pass that it holds
  int copy_first = 0, copy_start = 0;
  // causal tiles: the sequence's first query row, tokens new token 0 sees, the
  // sequence's partitions and this one, and the tokens of the chunk (from its
  // first) that the tile's last row sees
  int qs = 0, base = 0, nparts = 1, part = 0, walk_end = 0, seq = 0;
  int fewest = 0;  // fewest tokens of the chunk that a row of the tile sees
  if constexpr (CAUSAL) {
    if (unit >= p.num_chunks * p.num_kv_heads * p.num_seqs) return;
    part = unit % p.num_chunks;
    kvh = (unit / p.num_chunks) % p.num_kv_heads;
    int b = unit / (p.num_chunks * p.num_kv_heads);
    if (p.longest_first) {
      // b becomes the sequence of rank b by decreasing context length, every
      // workgroup ranking the lengths for itself (one sequence per thread):
      // key (length + 1) * 256 + 255 - index, distinct and larger for longer
      // sequences (and for smaller indices among equal lengths; a broken
      // length counts as -1), rank = how many keys are larger.  The scratch is
      // the third value buffer, which no load writes before the pipeline's
      // first barrier.
      int* sm_key = reinterpret_cast<int*>(&vbuf[2][0]);
      int* sm_pick = sm_key + kMaxRankSeqs;
      const int t = threadIdx.x;
      uint32_t key = 0;
      if (t < p.num_seqs) {
        const int raw = p.context_lens[t];
        const int len = raw < 0 || raw > p.max_context ? -1 : raw;
        key = (uint32_t)(len + 1) * 256u + (uint32_t)(255 - t);
        sm_key[t] = (int)key;
      }
      __syncthreads();
      if (t < p.num_seqs) {
        int rank = 0;
        for (int o = 0; o < p.num_seqs; ++o) rank += (uint32_t)sm_key[o] > key;
        if (rank == b) sm_pick[0] = t;
      }
      __syncthreads();
      b = sm_pick[0];
    }
    seq = b;
    qs = p.query_start[b];
    const int qe = p.query_start[b + 1];
    if (qs < 0 || qs > qe || qe > p.num_query_tokens) return;  // its rows are unknown: nothing is written
    const int qlen = qe - qs;
    const int nrows = min(qlen, p.max_query_len) * G;
    const int r0 = tile * 128;
    if (r0 >= nrows) return;
    rows = min(r0 + 128, nrows);
    const int ctx_raw = p.context_lens[b];
    const bool ctx_bad = ctx_raw < qlen || ctx_raw > p.max_context || qlen > p.max_query_len;
    base = ctx_raw - qlen + 1;
    const int walk = ctx_bad ? 0 : base + (rows - 1) / G;  // tokens the tile's last row sees
    const int nblocks = (walk + BS - 1) / BS;
    nparts = (nblocks + p.chunk_blocks - 1) / p.chunk_blocks;
    if (part >= nparts) {
      if (part == 0) {  // a broken length: NaN rows
        for (int idx = threadIdx.x; idx < (rows - r0) * HD; idx += blockDim.x) {
          const int row = r0 + idx / HD;
          const int64_t o = ((int64_t)(qs + row / G) * p.num_heads + kvh * G + row % G) * HD + idx % HD;
          if (p.out_bf16) reinterpret_cast<uint16_t*>(p.out)[o] = 0x7fc0;
          else reinterpret_cast<float*>(p.out)[o] = NAN;
        }
      }
      return;
    }
    blk_lo = part * p.chunk_blocks;
    blk_hi = min(nblocks, blk_lo + p.chunk_blocks);
    walk_end = min(walk, blk_hi * BS) - blk_lo * BS;
    fewest = min(base + r0 / G - blk_lo * BS, walk_end);
    bt = p.block_tables + (int64_t)b * p.max_blocks;
  } else {
    if (unit >= p.num_kv_heads * p.num_chunks) return;
    kvh = unit % p.num_kv_heads;
    const int chunk = unit / p.num_kv_heads;
    // which group and 128-row tile: groups hold their tiles in order
    const int32_t* plan = p.plan;
    const int num_groups = plan[kPlanGroups];
    const int32_t* groups = plan_groups(plan);
    int gi = 0;
    int gend = 0, gstart = 0, gbegin = 0, gcount = 0, leader = 0, parent = -1;
    for (; gi < num_groups; ++gi) {
      const int32_t* gr = groups + kGroupWords * gi;
      const int tiles = (gr[kGroupCount] * G + 127) / 128;
      if (tile >= tiles) copy_first += group_pass_blocks(gr, BS);
      if (tile < tiles) {
        gend = prefix_covered_blocks(gr[kGroupPrefix], BS);
        gstart = gr[kGroupStart];
        copy_start = gstart;
        gbegin = gr[kGroupBegin];
        gcount = gr[kGroupCount];
        leader = gr[kGroupLeader];
        parent = gr[kGroupParent];
        break;
      }
      tile -= tiles;
    }
    if (gi == num_groups) return;
    members = groups + kGroupWords * num_groups + gbegin;
    // chunk `chunk` of the group's blocks [gstart, gend); a nested group's slots
    // follow those of its ancestors
    blk_lo = gstart + chunk * p.chunk_blocks;
    blk_hi = min(gend, blk_lo + p.chunk_blocks);
    if (blk_lo >= blk_hi) return;  // the merge counts only the chunks the group's blocks reach
    slot0 = path_slots(groups, parent, BS, p.chunk_blocks) + chunk;
    rows = gcount * G;
    fewest = (blk_hi - blk_lo) * BS;
    bt = p.block_tables + (int64_t)leader * p.max_blocks;
  }
  const int row0 = tile * 128 + ROWS_PER_WAVE * wave;  // this wave's first row
  const bool wave_active = row0 < rows;
  // query row of unit row r (rows past the unit's end: any valid row)
  auto row_q = [&](int r) -> int64_t {
    if constexpr (CAUSAL) return (int64_t)(qs + r / G) * p.num_heads + kvh * G + r % G;
    else return (int64_t)members[r / G] * p.num_heads + kvh * G + r % G;
  };

  // queries: column tile ct, lane column n -> row row0 + 16ct + n
  bf16x8 qb[2][4];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int row = row0 + 16 * ct + n;
    const bool ok = row < rows;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + (ok ? row_q(row) : 0) * HD;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      qb[ct][i] = __builtin_bit_cast(bf16x8, ok ? load16(qrow + 32 * i + 8 * kg) : make_uint4(0, 0, 0, 0));
  }

  // Causal tiles: the tokens of the chunk (from its first) that the lane's
  // column sees, per column tile, and the fewest any row of the wave sees (its
  // first row's).  A stage reaching past that count has logits to mask.
  int lim[2] = {0, 0};
  int wave_lim = 0;
  if constexpr (CAUSAL) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) lim[ct] = min(base + (row0 + 16 * ct + n) / G - blk_lo * BS, walk_end);
    wave_lim = min(base + row0 / G - blk_lo * BS, walk_end);
  }

  // block ids of the chunk, 64 at a time (lane l: block c0 + l); ids outside the pool -> block 0 and NaN rows
  int bad = 0;
  int id_base = blk_lo;
  auto load_ids = [&](int first) {
    const int idx = first + lane;
    int id = idx < blk_hi ? bt[idx] : 0;
    const bool out = idx < blk_hi && (unsigned)id >= (unsigned)p.num_blocks;
    bad |= __ballot(out) != 0;
    return out ? 0 : id;
  };
  int ids = load_ids(id_base);

  const char* kpool = reinterpret_cast<const char*>(p.k_pool) + (int64_t)kvh * TILE;
  const char* vpool = reinterpret_cast<const char*>(p.v_pool) + (int64_t)kvh * TILE;
  // bytes of one block of every kv head: below 2^31 (the host checks the pool)
  const uint32_t block_bytes = (uint32_t)p.num_kv_heads * TILE;
  const int iters = (blk_hi - blk_lo + NB - 1) / NB;
  // With an fp16 copy of the values (causal tiles: the call's workspace copy,
  // zero past the context; shared-prefix pass: the caller's copy of the
  // groups' pass blocks) the fast path stages them from it and skips its own
  // conversion; the exact path still reads the pool.
  const bool from_copy = p.v_copy != nullptr;
  // block j of the walk at vcopy + j * block_bytes (the shared-prefix pass's
  // j starts at the group's start block: its copy begins at copy_first)
  const char* vcopy =
      !from_copy ? nullptr
      : CAUSAL   ? static_cast<const char*>(p.v_copy) + ((int64_t)seq * p.copy_blocks * p.num_kv_heads + kvh) * TILE
                 : reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(p.v_copy) +
                                                 ((int64_t)(copy_first - copy_start) * p.num_kv_heads + kvh) * TILE);

  // Staging: per iteration each wave moves four 1 KiB pieces of the keys and
  // four of the values straight from HBM/L2 into LDS (global_load_lds: lane l
  // lands at LDS base + 16*l, so a piece is a 1 KiB contiguous run of LDS and
  // each lane picks the global chunk that belongs at its spot).  The loads
  // take no registers; the wave waits for them with an explicit counter wait
  // before the barrier that publishes the buffer.
  auto stage_issue = [&](int it, int kb_i, int vb_i, bool copy = false) {
    const int first = blk_lo + it * NB;
    if (first - id_base >= 64) {  // next 64 ids
      id_base += 64;
      ids = load_ids(id_base);
    }
    // all of the stage's key loads first, then its value loads: the waits below
    // count on that order (keys are needed an iteration before the values)
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int k = 0; k < kPiecesPerWave; ++k) {
        const int piece = wave + NW * k;  // 1 KiB piece of the stage
        const int kb = piece * 1024 / TILE;
        const int in_tile = piece * 1024 % TILE;
        // ids are in [0, num_blocks) here (load_ids): 32 x 32 -> 64-bit product
        const uint64_t base = (uint64_t)(uint32_t)__builtin_amdgcn_readlane(ids, first + kb - id_base) * block_bytes;
        const int q = in_tile / 16 + lane;  // 16-byte piece of the tile that this lane's LDS spot holds
        if (half == 0) {
          // keys: chunk q / BS, slot q % BS <- that chunk's key_slot_token (16/32-token
          // blocks), or the swizzled row and slot of 8-token blocks
          const int kq = BS == 8 ? key8_row(q / 8, kb & 3) * 8 + key8_slot(q % 8, kb & 3)
                                 : (q / BS) * BS + key_slot_token<BS>(q % BS, kb & 1);
          lds_dma16(lds_addr(&kbuf[kb_i][piece * 1024]), kpool + base, kq * 16);
        } else {
          // values: 8- and 16-token rows keep the pool's order; 32-token rows are rotated
          const int d = q / (BS / 8);
          const int vpiece = BS == 32 ? ((q & 3) ^ value_rot(d)) : BS == 16 ? (q & 1) : 0;
          const char* vsrc = copy ? vcopy + (uint64_t)(uint32_t)(first + kb) * block_bytes : vpool + base;
          lds_dma16(lds_addr(&vbuf[vb_i][piece * 1024]), vsrc, d * (BS * 2) + vpiece * 16);
        }
      }
  };

  // Accumulators: O^T per column tile, and a ninth tile that multiplies the
  // weights by a row of ones, so each lane reads its column's weight sum there
  // (the fp16 path's softmax denominator, from the same rounded weights as the
  // numerator).  The exact path sums its weights in lsum (per lane, the
  // lane's own tokens) instead; the two are added at the end.
  f32x4 o[2][8], o1[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    o1[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[ct][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  // fast path: the Gram matrix W W^T of each column tile's (fp16) weights,
  // relative to the same m; its diagonal, each row's sum of squared weights,
  // with the weight sum gives the effective token count
  f32x4 g2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const f16x8 ones = {1, 1, 1, 1, 1, 1, 1, 1};

  // (A column that has seen nothing yet and sees nothing now keeps m = -inf:
  // its factor is 1, not 2^(-inf + inf).  The exact path rescales both column
  // tiles when any lane needs it; causal tiles mask whole columns.)
  auto rescale = [&](int ct, float mn) {
    const float alpha = CAUSAL && m[ct] == mn ? 1.f : fast_exp2(m[ct] - mn);
    lsum[ct] *= alpha;
    g2[ct] *= alpha * alpha;
    o1[ct] *= alpha;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[ct][nt] *= alpha;
    m[ct] = mn;
  };

  // key operands of S tile `sub` (run sub / 2, tile sub % 2) of the stage in kbuf[kb_i]
  auto load_keys = [&](int kb_i, int sub, bf16x8 (&ka)[4]) {
    const unsigned char* kt = &kbuf[kb_i][(sub >> 1) * RUN_BYTES];
    const int x = sub & 1;
    // the lane's row n of tile x: 32-token blocks slot 16x + n; 16-token blocks
    // block n / 8 of the run, slot n % 8 + 8 (x ^ block); 8-token blocks block
    // n / 4, token 4x + n % 4 (in its swizzled row and slot)
    if constexpr (BS == 8) {
      const int b = n >> 2;
      const int slot = key8_slot(4 * x + (n & 3), b);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ka[i] = *reinterpret_cast<const bf16x8*>(kt + b * TILE + (key8_row(4 * i + kg, b) * 8 + slot) * 16);
    } else {
      const int koff = BS == 32 ? 16 * x + n : (n >> 3) * (TILE / 16) + (n & 7) + 8 * (x ^ (n >> 3));
#pragma unroll
      for (int i = 0; i < 4; ++i) ka[i] = *reinterpret_cast<const bf16x8*>(kt + ((4 * i + kg) * BS + koff) * 16);
    }
  };
  // S^T of one iteration (64 tokens, always whole) from key buffer kb_i:
  // s[run * 2 + S tile][column tile].
  auto logits = [&](int kb_i, f32x4 (&s)[4][2]) {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      bf16x8 ka[4];
      load_keys(kb_i, sub, ka);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        s[sub][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[sub][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[i], qb[ct][i], s[sub][ct], 0, 0, 0);
      }
    }
  };
  // value operand of dim 16nt + n, tokens 8kg..8kg+7 of run `pair`
  auto value_piece = [&](int vb_i, int pair, int nt) {
    const int d = 16 * nt + n;
    const int off = BS == 32   ? d * 64 + 16 * (kg ^ value_rot(d))
                    : BS == 16 ? (kg >> 1) * TILE + d * 32 + 16 * (kg & 1)
                               : kg * TILE + d * 16;  // 8-token blocks: tokens 8kg.. are block kg
    return *reinterpret_cast<const uint4*>(&vbuf[vb_i][pair * RUN_BYTES] + off);
  };

  // First token (in its stage) of the eight values in the lane's 16 bytes of
  // the wave's own value piece k (pieces wave + NW*k: its loads landed exactly
  // those 16 bytes): the value staging map read backwards.
  auto own_value_token = [&](int k) {
    const int piece = wave + NW * k;
    const int q = piece * 1024 % TILE / 16 + lane;
    const int d = q / (BS / 8);
    const int vpiece = BS == 32 ? ((q & 3) ^ value_rot(d)) : BS == 16 ? (q & 1) : 0;
    return piece * 1024 / TILE * BS + 8 * vpiece;
  };
  // The wave's own pieces of a stage's values to fp16, in place.  The stage
  // must have landed (the barrier after the wave's counter wait).  A value
  // fp16 cannot hold becomes +-inf, or stays NaN.
  // With causal tiles, the stage reaching past the tokens the tile sees has
  // those values zeroed on the way.
  auto convert_own = [&](int vb_i, int stage) {
    if (from_copy) return;  // already fp16 in the copy (causal tiles: zero past the context)
    if (CAUSAL && (stage + 1) * TOK > walk_end) {
#pragma unroll
      for (int k = 0; k < kPiecesPerWave; ++k)
        values_to_f16_head(&vbuf[vb_i][(wave + NW * k) * 1024 + 16 * lane],
                           walk_end - stage * TOK - own_value_token(k));
    } else {
#pragma unroll
      for (int k = 0; k < kPiecesPerWave; ++k) values_to_f16(&vbuf[vb_i][(wave + NW * k) * 1024 + 16 * lane]);
    }
  };

  // Causal tiles: logits of tokens a column does not see -> -inf (weight 0),
  // s as computed for stage `stage` (token of s[sub][ct][r]: 32 (sub / 2) +
  // 8kg + 4 (sub % 2) + r of the stage).
  auto mask_logits = [&](f32x4 (&s)[4][2], int stage) {
    if constexpr (CAUSAL) {
      const int t0 = stage * TOK;
      if (t0 + TOK > wave_lim) {
#pragma unroll
        for (int sub = 0; sub < 4; ++sub)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (t0 + 32 * (sub >> 1) + 8 * kg + 4 * (sub & 1) + r >= lim[ct]) s[sub][ct][r] = -INFINITY;
      }
    }
  };
  // Weight 2^(s*scale - m) of logit s.  Causal tiles: a masked logit (-inf)
  // weighs 0 also where that formula would not give 0 (scale 0, or a column
  // with m = -inf that has seen nothing yet).
  auto weight = [&](float x, float neg_m) {
    const float w = fast_exp2(fmaf(x, p.scale_log2, neg_m));
    return CAUSAL && x == -INFINITY ? 0.f : w;
  };
  // column maximum of raw logits -> the scaled domain (scale >= 0; all masked: -inf)
  auto scaled_max = [&](float raw) {
    return CAUSAL && raw == -INFINITY ? -INFINITY : raw * p.scale_log2;
  };

  // Fast path (fp16 values in LDS), software-pipelined over iterations: stage
  // j's weights are formed while the matrix cores compute stage j + 1's
  // logits (logits_with_weights), then stage j's value products run beside
  // the conversion of stage j + 1's values (compute_fast).
  //
  // The reference m is the first stage's column maximum.  Weights
  // 2^(s*scale - m) then stay below 2^16, finite in fp16, unless a later logit
  // exceeds m by 16 or more; such a weight makes the accumulators infinite and
  // sends the chunk to the exact path at its end.  The last stage (and a walk
  // of one stage) forms its weights in compute_fast, which moves m instead: a
  // packed fma(w, 0, acc) turns NaN once a weight is infinite, and m then
  // moves to the stage's column maximum, the accumulators are rescaled and the
  // weights formed again.  fp16 keeps 11 bits of each weight down to 2^-14.
  //
  // Stage j + 1's logits (sn, keys in kbuf[kb_i]) on the matrix cores and
  // stage j's fp16 weights (from s, already masked) on the vector unit, one
  // logit instruction and one weight per step, in an order the scheduler must
  // keep: each step's vector work issues while the step's matrix instruction
  // runs.  No overflow check here: m was set from the first stage's column
  // maxima, and a weight that overflows fp16 later (a logit 16 or more above
  // them) makes the accumulators infinite, which sends the chunk to the exact
  // path at its end.
  auto logits_with_weights = [&](int kb_i, f32x4 (&sn)[4][2], const f32x4 (&s)[4][2], uint32_t (&w)[2][2][4]) {
    float neg_m[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) neg_m[ct] = CAUSAL ? fminf(-m[ct], __FLT_MAX__) : -m[ct];
    bf16x8 ka[2][4];
    load_keys(kb_i, 0, ka[0]);
    float prev = 0.f;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      if (sub < 3) load_keys(kb_i, sub + 1, ka[(sub + 1) & 1]);
      // shared-prefix pass: raised wave priority from the last quarter of the
      // step through the value products (compute_fast lowers it): see there
      if (!CAUSAL && sub == 3) __builtin_amdgcn_s_setprio(1);
      sn[sub][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      sn[sub][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = q >> 1, ct = q & 1;
        sn[sub][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[sub & 1][i], qb[ct][i], sn[sub][ct], 0, 0, 0);
        // weight k of this stage: run k / 16, column tile (k / 8) % 2, token 8kg + k % 8 of the run
        const int k = sub * 8 + q;
        const int pair = k >> 4, wct = (k >> 3) & 1, idx = k & 7;
        const float pr = fast_exp2(fmaf(s[2 * pair + (idx >> 2)][wct][idx & 3], p.scale_log2, neg_m[wct]));
        if (k & 1) {
          w[pair][wct][idx >> 1] = pack_f16(prev, pr);
        } else {
          prev = pr;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // w: the stage's weights, formed by the caller (fused_tag true:
  // logits_with_weights) or here, with the overflow check that moves m.
  auto compute_fast = [&](f32x4 (&s)[4][2], int stage, int vb_i, int convert_vb, auto convert_tag,
                          uint32_t (&w)[2][2][4], auto fused_tag) {
    if constexpr (!decltype(fused_tag)::value) mask_logits(s, stage);
    auto weights = [&]() {
      f16x2 ovf = {0, 0};
#pragma unroll
      for (int pair = 0; pair < 2; ++pair)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          // causal tiles: a column with m = -inf gets the largest float
          // instead, so a masked logit (-inf) still weighs 0 and any other
          // still overflows (and m moves); the scale is > 0 here
          const float neg_m = CAUSAL ? fminf(-m[ct], __FLT_MAX__) : -m[ct];
          float pr[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pr[r] = fast_exp2(fmaf(s[2 * pair][ct][r], p.scale_log2, neg_m));
            pr[4 + r] = fast_exp2(fmaf(s[2 * pair + 1][ct][r], p.scale_log2, neg_m));
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w[pair][ct][e] = pack_f16(pr[2 * e], pr[2 * e + 1]);
            ovf = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, w[pair][ct][e]), f16x2{0, 0}, ovf);
          }
        }
      return __ballot(__builtin_isnan(ovf[0]) || __builtin_isnan(ovf[1])) != 0;
    };
    if constexpr (!decltype(fused_tag)::value) {
      if (weights()) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          float a = s[0][ct][0];
#pragma unroll
          for (int sub = 0; sub < 4; ++sub)
#pragma unroll
            for (int r = 0; r < 4; ++r) a = maxp(a, s[sub][ct][r]);
          const float mx = maxp_xor32(maxp_xor16(a)) * p.scale_log2;  // the scale is >= 0
          if (!(mx <= m[ct])) rescale(ct, maxp(m[ct], mx));
        }
        weights();
      }
    }
    // The shared-prefix pass runs the value products and the conversion beside
    // them at raised wave priority (from the fused step's last quarter on):
    // when the SIMD's other wave, of the other workgroup on the CU, is in its
    // own fused step, its vector work then fills the cycles around this wave's
    // matrix instructions rather than the other way round.  Interleaved A/B
    // with the fp16 prefix copy: shared-prefix 6.9 us per call faster than
    // without; the causal tiles (prefill) 2.4 us slower, so they leave it.
    if constexpr (!CAUSAL) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int pair = 0; pair < 2; ++pair) {
      // all eight value pieces of the run read before its matrix instructions
      // (the scheduler otherwise keeps two in flight and waits on each pair):
      // shared-prefix -2.9 us, prefill -2.8 us per call, interleaved A/B
      uint4 vp[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) vp[nt] = value_piece(vb_i, pair, nt);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const f16x8 wp = __builtin_bit_cast(f16x8, make_uint4(w[pair][ct][0], w[pair][ct][1], w[pair][ct][2], w[pair][ct][3]));
        o1[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, wp, o1[ct], 0, 0, 0);
        // the same register as both operands: row i of A and column j of B are
        // both query row i (j) of the tile, over the run's 32 tokens
        g2[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wp, wp, g2[ct], 0, 0, 0);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const f16x8 va = __builtin_bit_cast(f16x8, vp[nt]);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          o[ct][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              va, __builtin_bit_cast(f16x8, make_uint4(w[pair][ct][0], w[pair][ct][1], w[pair][ct][2], w[pair][ct][3])),
              o[ct][nt], 0, 0, 0);
      }
    }
    // the next stage's values: after the value products in program order (the
    // buffer indices are not known at compile time, so these stores may not
    // pass their loads), in the same straight-line stretch so that the
    // conversion's vector work fills the matrix cores' cycles
    if constexpr (decltype(convert_tag)::value) {
      // this wave's values of that stage were loaded before the newest stage's
      // keys and values: those may still be in flight
      lds_dma_wait<2 * kPiecesPerWave>();
      convert_own(convert_vb, stage + 1);
    }
    if constexpr (!CAUSAL) __builtin_amdgcn_s_setprio(0);
  };

  // Exact path (bf16 values in LDS): per 32-token run, the reference moves
  // when a logit exceeds it by more than kRescaleSlack (weights below 2^8),
  // and the weights enter the matrix cores as bf16 hi + lo parts.
  auto compute_exact = [&](int kb_i, int vb_i, int stage) {
    f32x4 s[4][2];
    logits(kb_i, s);
    mask_logits(s, stage);
#pragma unroll
    for (int pair = 0; pair < 2; ++pair) {
      const f32x4* s0 = s[2 * pair];
      const f32x4* s1 = s[2 * pair + 1];
      // column maxima of the pair's raw logits (the scale, >= 0, is applied after)
      float mx[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const float a = maxp(maxp(maxp(s0[ct][0], s0[ct][1]), maxp(s0[ct][2], s0[ct][3])),
                             maxp(maxp(s1[ct][0], s1[ct][1]), maxp(s1[ct][2], s1[ct][3])));
        mx[ct] = scaled_max(maxp_xor32(maxp_xor16(a)));
      }
      if (__ballot(mx[0] > m[0] + kRescaleSlack || mx[1] > m[1] + kRescaleSlack) != 0) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) rescale(ct, maxp(m[ct], mx[ct]));
      }
      // weights: pr[j] is token 8kg + j of the run (tile 0's rows for j < 4, tile 1's for j >= 4)
      uint32_t hw[2][4], lw[2][4];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const float neg_m = -m[ct];
        float pr[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[r] = weight(s0[ct][r], neg_m);
          pr[4 + r] = weight(s1[ct][r], neg_m);
        }
        lsum[ct] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16(pr[2 * e], pr[2 * e + 1], &hw[ct][e], &lw[ct][e]);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const bf16x8 va = __builtin_bit_cast(bf16x8, value_piece(vb_i, pair, nt));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const bf16x8 ph = __builtin_bit_cast(bf16x8, make_uint4(hw[ct][0], hw[ct][1], hw[ct][2], hw[ct][3]));
          const bf16x8 pl = __builtin_bit_cast(bf16x8, make_uint4(lw[ct][0], lw[ct][1], lw[ct][2], lw[ct][3]));
          o[ct][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph, o[ct][nt], 0, 0, 0);
          o[ct][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl, o[ct][nt], 0, 0, 0);
        }
      }
    }
  };

  // Fast path.  Iteration j: the loads of stage j + 2 are issued; the logits
  // of stage j + 1 (keys published by the last barrier) are computed beside
  // stage j's weights, whose logits the previous iteration computed; stage j's
  // value products (values converted during the previous iteration) run beside
  // the conversion of stage j + 1's values; then the wave waits for its loads
  // and the barrier publishes all of it.  Buffers: keys of stage j in j % 2,
  // values in j % 3.
  // Waits: a stage's keys must have landed (all waves) by the barrier that ends
  // the iteration before they are used; its values only when this wave
  // converts its pieces, during that next iteration.  So the barrier waits
  // with the newest stage's value loads still outstanding, and the
  // conversion with the newest stage's keys and values outstanding.  Every
  // iteration issues a stage (the last two load the final stage again into
  // buffers that are free) so that those counts hold throughout.
  //
  // The exact path from the start when the caller asks for it, when some row
  // sees fewer tokens than p.min_eff (its effective count cannot reach it),
  // and for causal tiles with scale 0 (a masked logit times 0 is no longer
  // -inf).
  bool redo = !((float)fewest >= p.min_eff) || (CAUSAL && !(p.scale_log2 > 0.f));
  if (!redo) {
    if (iters > 0) {
      stage_issue(0, 0, 0, from_copy);
      stage_issue(min(1, iters - 1), 1, 1, from_copy);
      lds_dma_wait<kPiecesPerWave>();  // all but stage 1's values
      __syncthreads();
      convert_own(0, 0);
      // Waves with rows run the loop below; the others (past the group's rows)
      // only stage, convert and meet the same barriers.  Two loops, so that the
      // active one holds no branch between the value products and the
      // conversion.
      if (wave_active) {
        f32x4 s[4][2];
        logits(0, s);
        mask_logits(s, 0);
        // m from the first stage's column maxima (scale >= 0; a column that
        // sees nothing keeps -inf)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          float a = s[0][ct][0];
#pragma unroll
          for (int sub = 0; sub < 4; ++sub)
#pragma unroll
            for (int r = 0; r < 4; ++r) a = maxp(a, s[sub][ct][r]);
          const float raw = maxp_xor32(maxp_xor16(a));
          m[ct] = CAUSAL && raw == -INFINITY ? -INFINITY : raw * p.scale_log2;
        }
        __syncthreads();
        for (int it = 0; it + 1 < iters; ++it) {
          stage_issue(min(it + 2, iters - 1), it % 2, (it + 2) % 3, from_copy);  // those buffers' stages are used up
          f32x4 s_next[4][2];
          uint32_t w[2][2][4];
          mask_logits(s, it);
          logits_with_weights((it + 1) % 2, s_next, s, w);
          compute_fast(s, it, it % 3, (it + 1) % 3, std::true_type{}, w, std::true_type{});
#pragma unroll
          for (int sub = 0; sub < 4; ++sub)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) s[sub][ct] = s_next[sub][ct];
          lds_dma_wait<kPiecesPerWave>();
          __syncthreads();
        }
        uint32_t w[2][2][4];
        compute_fast(s, iters - 1, (iters - 1) % 3, 0, std::false_type{}, w, std::false_type{});
      } else {
        __syncthreads();
        for (int it = 0; it + 1 < iters; ++it) {
          stage_issue(min(it + 2, iters - 1), it % 2, (it + 2) % 3, from_copy);
          lds_dma_wait<2 * kPiecesPerWave>();
          convert_own((it + 1) % 3, it + 1);
          lds_dma_wait<kPiecesPerWave>();
          __syncthreads();
        }
      }
      lds_dma_wait_all();  // the last stage's repeated loads
    }

    // The workgroup computes its chunk again from scratch on the exact path
    // (bf16 values, weights as bf16 hi + lo) when some wave has
    //  * a non-finite accumulator: a value without a finite fp16 copy (|v| >
    //    65504, an infinity) or a NaN in the chunk; the exact path gives NaN
    //    or infinity only where the inputs do;
    //  * a row whose weights sit on too few tokens: effective count (sum w)^2 /
    //    sum w^2 below p.min_eff.  Each fp16 weight is off by up to 2^-11
    //    of itself; over many comparable weights those errors average out,
    //    over a handful (outlier keys) they can move a small output element
    //    by more than 1% of itself.
    // The flags go through the first key buffer, which nothing reads any more.
    bool nonfinite = false;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      nonfinite |= !__builtin_isfinite(o1[ct][0]);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) nonfinite |= !__builtin_isfinite(o[ct][nt][r]);
      const float l = o1[ct][0];
      // row n's sum of squares: the Gram diagonal element (n, n), which lane
      // 16 (n / 4) + n holds in register n % 4
      const f32x4 gg = g2[ct];
      const int r = n & 3;
      const float own = r == 0 ? gg[0] : r == 1 ? gg[1] : r == 2 ? gg[2] : gg[3];
      const float sq = __shfl(own, 16 * (n >> 2) + n);
      nonfinite |= row0 + 16 * ct + n < rows && l > 0.f && l * l < p.min_eff * sq;
    }
    const int wave_nonfinite = __ballot(nonfinite) != 0;
    int* flags = reinterpret_cast<int*>(&kbuf[0][0]);
    __syncthreads();
    flags[wave] = wave_nonfinite;  // every lane stores the same value
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) redo |= flags[w] != 0;
    __syncthreads();  // flags read before the exact path's loads overwrite them
  }
  if (redo) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      m[ct] = -INFINITY;
      lsum[ct] = 0.f;
      o1[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) o[ct][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (id_base != blk_lo) {  // back to the chunk's first 64 ids
      id_base = blk_lo;
      ids = load_ids(id_base);
    }
    stage_issue(0, 0, 0);
    lds_dma_wait_all();
    __syncthreads();
    for (int it = 0; it < iters; ++it) {
      const int buf = it & 1;
      if (it + 1 < iters) stage_issue(it + 1, buf ^ 1, buf ^ 1);  // buffers buf^1 were released by the last barrier
      if (CAUSAL && (it + 1) * TOK > walk_end) {  // the values past the tile's tokens -> zeros
#pragma unroll
        for (int k = 0; k < kPiecesPerWave; ++k)
          values_zero_tail(&vbuf[buf][(wave + NW * k) * 1024 + 16 * lane], walk_end - it * TOK - own_value_token(k));
        __syncthreads();
      }
      if (wave_active) compute_exact(buf, buf, it);
      lds_dma_wait_all();
      __syncthreads();
    }
  }

  if (!wave_active) return;
  // Cascade: partials, slot (b, h, chunk) of row -> (member sequence b, query
  // head h).  Causal tiles: the output row itself when the sequence's walk is
  // one partition, else partial `part` of the row (the multi-token merge
  // combines them).
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const float l = sum_xor32(sum_xor16(lsum[ct])) + o1[ct][0];
    const int row = row0 + 16 * ct + n;
    if (row >= rows) continue;
    const int64_t hrow = row_q(row);
    if (CAUSAL && nparts == 1) {
      const float inv = 1.f / l;
      if (p.out_bf16) {
        uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) + hrow * HD;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const f32x4 v = bad ? f32x4{NAN, NAN, NAN, NAN} : o[ct][nt] * inv;
          *reinterpret_cast<uint2*>(orow + 16 * nt + 4 * kg) =
              make_uint2(f32_to_bf16_rne(v[0]) | f32_to_bf16_rne(v[1]) << 16,
                         f32_to_bf16_rne(v[2]) | f32_to_bf16_rne(v[3]) << 16);
        }
      } else {
        float* orow = reinterpret_cast<float*>(p.out) + hrow * HD;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
          *reinterpret_cast<f32x4*>(orow + 16 * nt + 4 * kg) = bad ? f32x4{NAN, NAN, NAN, NAN} : o[ct][nt] * inv;
      }
      continue;
    }
    const int64_t pi = CAUSAL ? hrow * p.num_chunks + part : hrow * p.num_slots + slot0;
    float* acc = p.ws_acc + pi * HD;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      f32x4 v = o[ct][nt];
      if (bad) v = f32x4{NAN, NAN, NAN, NAN};
      *reinterpret_cast<f32x4*>(acc + 16 * nt + 4 * kg) = v;
    }
    if (kg == 0) {
      p.ws_m[pi] = bad ? NAN : m[ct];
      p.ws_l[pi] = bad ? NAN : l;
    }
  }
}


// The causal tiles' fp16 copy of the values: one workgroup per (sequence,
// logical block), all kv heads of the block.  Blocks the context reaches are
// read through the block table and converted as the tiles would convert them
// (bf16 -> fp16, round to nearest even; beyond fp16's range: +-inf); tokens
// past the context, blocks past it up to the end of its last 64-token stage,
// and blocks with an id outside the pool become zeros (such ids make the tile
// kernel's rows NaN anyway).  Blocks past that stage are never read and are
// left as they are.
template <int BS>
__global__ __launch_bounds__(256) void value_copy_kernel(PrefixArgs p) {
  constexpr int TILE = BS * HD * 2;
  constexpr int PIECES = TILE / 16;  // 16-byte pieces of a tile: dim q / (BS / 8), tokens 8 (q % (BS / 8)) ..
  constexpr int NB = TOK / BS;
  const int64_t bj = blockIdx.x;
  const int j = (int)(bj % p.copy_blocks);
  const int b = (int)(bj / p.copy_blocks);
  const int ctx = min(max(p.context_lens[b], 0), p.max_context);
  const int nblk = (ctx + BS - 1) / BS;
  if (j >= (nblk + NB - 1) / NB * NB) return;
  int id = -1;
  if (j < nblk && j < p.max_blocks) {
    id = p.block_tables[(int64_t)b * p.max_blocks + j];
    if ((unsigned)id >= (unsigned)p.num_blocks) id = -1;
  }
  const char* src = reinterpret_cast<const char*>(p.v_pool) + (int64_t)(id < 0 ? 0 : id) * p.num_kv_heads * TILE;
  uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(p.v_copy) + bj * p.num_kv_heads * TILE);
  const int total = p.num_kv_heads * PIECES;
  for (int x = threadIdx.x; x < total; x += 256) {
    const int q = x % PIECES;
    uint4 h = make_uint4(0, 0, 0, 0);
    if (id >= 0) {
      const int keep = min(max(ctx - (j * BS + 8 * (q % (BS / 8))), 0), 8);
      const uint4 mk = keep_mask(keep);
      const uint4 w = load16(src + 16 * (int64_t)x);
      const uint32_t v[4] = {w.x & mk.x, w.y & mk.y, w.z & mk.z, w.w & mk.w};
      h = make_uint4(pack_f16(bf16_lo(v[0]), bf16_hi(v[0])), pack_f16(bf16_lo(v[1]), bf16_hi(v[1])),
                     pack_f16(bf16_lo(v[2]), bf16_hi(v[2])), pack_f16(bf16_lo(v[3]), bf16_hi(v[3])));
    }
    dst[x] = h;
  }
}

// The fp16 copy of the plan's shared-prefix values (pkv_prefix_values_f16):
// workgroup x takes pass block x of all groups in plan order, group g's blocks
// [start_g, covered end_g) of its leader's table, every kv head of it.  A
// block id outside the pool gives zeros (the pass turns the group's rows into
// NaN on its own).  A value beyond fp16's range becomes +-inf, as in the
// pass's own conversion, and sends its chunk to the exact path.
template <int BS>
__global__ __launch_bounds__(256) void prefix_value_copy_kernel(PrefixArgs p) {
  constexpr int TILE = BS * HD * 2;
  const int32_t* groups = plan_groups(p.plan);
  const int num_groups = p.plan[kPlanGroups];
  int x = blockIdx.x, gi = 0;
  for (; gi < num_groups; ++gi) {
    const int n = group_pass_blocks(groups + kGroupWords * gi, BS);
    if (x < n) break;
    x -= n;
  }
  if (gi == num_groups) return;
  const int32_t* gr = groups + kGroupWords * gi;
  int id = p.block_tables[(int64_t)gr[kGroupLeader] * p.max_blocks + gr[kGroupStart] + x];
  if ((unsigned)id >= (unsigned)p.num_blocks) id = -1;
  const char* src = reinterpret_cast<const char*>(p.v_pool) + (int64_t)(id < 0 ? 0 : id) * p.num_kv_heads * TILE;
  uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(p.v_copy) + (int64_t)blockIdx.x * p.num_kv_heads * TILE);
  const int total = p.num_kv_heads * TILE / 16;
  for (int y = threadIdx.x; y < total; y += 256) {
    uint4 h = make_uint4(0, 0, 0, 0);
    if (id >= 0) {
      const uint4 w = load16(src + 16 * (int64_t)y);
      h = make_uint4(pack_f16(bf16_lo(w.x), bf16_hi(w.x)), pack_f16(bf16_lo(w.y), bf16_hi(w.y)),
                     pack_f16(bf16_lo(w.z), bf16_hi(w.z)), pack_f16(bf16_lo(w.w), bf16_hi(w.w)));
    }
    dst[y] = h;
  }
}

}  // namespace

hipError_t launch_prefix_value_copy(const PrefixArgs& p, int block_size, int total_blocks, hipStream_t s) {
  if (total_blocks <= 0 || !p.v_copy || !p.plan) return hipErrorInvalidValue;
  const dim3 grid((unsigned)total_blocks), block(256);
  if (block_size == 8) hipLaunchKernelGGL(prefix_value_copy_kernel<8>, grid, block, 0, s, p);
  else if (block_size == 16) hipLaunchKernelGGL(prefix_value_copy_kernel<16>, grid, block, 0, s, p);
  else if (block_size == 32) hipLaunchKernelGGL(prefix_value_copy_kernel<32>, grid, block, 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_value_copy(const PrefixArgs& p, int block_size, hipStream_t s) {
  const int64_t blocks = (int64_t)p.num_seqs * p.copy_blocks;
  if (blocks <= 0 || blocks > 0x7fffffff || !p.v_copy) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(256);
  if (block_size == 8) hipLaunchKernelGGL(value_copy_kernel<8>, grid, block, 0, s, p);
  else if (block_size == 16) hipLaunchKernelGGL(value_copy_kernel<16>, grid, block, 0, s, p);
  else if (block_size == 32) hipLaunchKernelGGL(value_copy_kernel<32>, grid, block, 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_prefix(const PrefixArgs& p, int block_size, int group, bool causal, hipStream_t s) {
  const int64_t units = (int64_t)p.num_kv_heads * p.num_chunks * (causal ? p.num_seqs : 1);
  const int64_t wgs = (units + kXcds - 1) / kXcds * kXcds * p.num_tiles;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  const dim3 block(64 * NW);
#define PKV_PREFIX(BS, G)                                                        \
  do {                                                                           \
    if (causal) hipLaunchKernelGGL((prefix_kernel<BS, G, true>), grid, block, 0, s, p);  \
    else hipLaunchKernelGGL((prefix_kernel<BS, G, false>), grid, block, 0, s, p);        \
  } while (0)
  if (block_size == 8) {
    switch (group) {
      case 1: PKV_PREFIX(8, 1); break;
      case 2: PKV_PREFIX(8, 2); break;
      case 4: PKV_PREFIX(8, 4); break;
      case 8: PKV_PREFIX(8, 8); break;
      default: return hipErrorInvalidValue;
    }
  } else if (block_size == 16) {
    switch (group) {
      case 1: PKV_PREFIX(16, 1); break;
      case 2: PKV_PREFIX(16, 2); break;
      case 4: PKV_PREFIX(16, 4); break;
      case 8: PKV_PREFIX(16, 8); break;
      default: return hipErrorInvalidValue;
    }
  } else if (block_size == 32) {
    switch (group) {
      case 1: PKV_PREFIX(32, 1); break;
      case 2: PKV_PREFIX(32, 2); break;
      case 4: PKV_PREFIX(32, 4); break;
      case 8: PKV_PREFIX(32, 8); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef PKV_PREFIX
  return hipGetLastError();
}

}  // namespace pkv

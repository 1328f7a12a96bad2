// Shared-prefix pass of cascade decode (bf16, head_dim 128).
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
// Workgroup = 4 waves x 32 query rows (two 16-column MFMA tiles per wave).
// Per iteration 64 prefix tokens: the next iteration's key and value tiles
// travel from memory straight into the other LDS buffer (global_load_lds)
// while the current one is computed (two buffers, one barrier per iteration).
// An iteration is two runs of 32 tokens (two 16-token blocks or one 32-token
// block).  Each run's logits come from two S tiles whose 16 rows interleave:
// tile X holds tokens 8j + 4X + r (j, r < 4), so after the product the lane of
// group kg owns tokens 8kg..8kg+7 of the run across the two tiles, exactly the
// 8 contraction indices it supplies to P.V, and the value operand is one
// 16-byte piece of a dim's row.
//  * S^T = K . Q^T, v_mfma_f32_16x16x32_bf16: A = keys (lane: the tile's row
//    n, lane group kg -> 16-byte chunk 4i+kg), B = queries (lane: column n,
//    dims 32i+8kg..+7); lane gets S^T[row 4kg+r][column n].
//  * O^T += V^T . P^T over the run, v_mfma_f32_16x16x32_bf16: k = 8kg + j is
//    token 8kg + j, B = the lane's own 8 weights, A = values of dim 16nt+n at
//    those tokens.  Weights go in as bf16 hi + lo parts (two instructions),
//    keeping ~16 significant bits.
// The LDS copy permutes 16-byte pieces so that both operand reads are free of
// bank conflicts (measured with the hardware counter): within a key chunk row
// the tokens of one S tile sit in 16 consecutive slots (key_slot_token), and a
// 32-token value row has its four pieces rotated by bits 1-2 of the dim.
#include "decode_common.h"

namespace pkv {

namespace {

constexpr int HD = 128;
constexpr int TOK = kPrefixIterTokens;  // prefix tokens per iteration
constexpr int NW = kWaves;        // 4
constexpr int ROWS_PER_WAVE = 32; // two MFMA column tiles
constexpr int STAGE_HALF = TOK * HD * 2;  // bytes of keys (or values) per iteration: 16 KiB

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

template <int BS, int G>
__global__ __launch_bounds__(64 * NW, 2) void prefix_kernel(PrefixArgs p) {
  constexpr int NB = TOK / BS;          // blocks per iteration
  constexpr int TILE = BS * HD * 2;     // bytes of one (block, kv head) tile
  constexpr int RUN_BYTES = 32 * HD * 2; // one 32-token run of keys (or values)
  static_assert(NB * TILE == STAGE_HALF, "stage size");

  __shared__ __attribute__((aligned(16))) unsigned char lds[2][2][STAGE_HALF];  // [buffer][K=0/V=1]

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
  if (unit >= p.num_kv_heads * p.num_chunks) return;
  const int kvh = unit % p.num_kv_heads;
  const int chunk = unit / p.num_kv_heads;

  // which group and 128-row tile: groups hold their tiles in order
  const int32_t* plan = p.plan;
  const int num_groups = plan[kPlanGroups];
  const int32_t* groups = plan_groups(plan);
  int tile = slot % p.num_tiles, gi = 0;
  int gend = 0, gstart = 0, gbegin = 0, gcount = 0, leader = 0, parent = -1;
  for (; gi < num_groups; ++gi) {
    const int32_t* gr = groups + kGroupWords * gi;
    const int tiles = (gr[kGroupCount] * G + 127) / 128;
    if (tile < tiles) {
      gend = prefix_covered_blocks(gr[kGroupPrefix], BS);
      gstart = gr[kGroupStart];
      gbegin = gr[kGroupBegin];
      gcount = gr[kGroupCount];
      leader = gr[kGroupLeader];
      parent = gr[kGroupParent];
      break;
    }
    tile -= tiles;
  }
  if (gi == num_groups) return;
  const int32_t* members = groups + kGroupWords * num_groups + gbegin;
  // chunk `chunk` of the group's blocks [gstart, gend); a nested group's slots
  // follow those of its ancestors
  const int blk_lo = gstart + chunk * p.chunk_blocks;
  const int blk_hi = min(gend, blk_lo + p.chunk_blocks);
  if (blk_lo >= blk_hi) return;  // the merge counts only the chunks the group's blocks reach
  const int slot0 = path_slots(groups, parent, BS, p.chunk_blocks) + chunk;
  const int rows = gcount * G;
  const int row0 = tile * 128 + ROWS_PER_WAVE * wave;  // this wave's first row
  const bool wave_active = row0 < rows;

  // queries: column tile ct, lane column n -> row row0 + 16ct + n
  bf16x8 qb[2][4];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int row = row0 + 16 * ct + n;
    const bool ok = row < rows;
    const int b = ok ? members[row / G] : 0;
    const int h = kvh * G + row % G;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)b * p.num_heads + h) * HD;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      qb[ct][i] = __builtin_bit_cast(bf16x8, ok ? load16(qrow + 32 * i + 8 * kg) : make_uint4(0, 0, 0, 0));
  }

  // block ids of the chunk, 64 at a time (lane l: block c0 + l); ids outside the pool -> block 0 and NaN rows
  const int32_t* bt = p.block_tables + (int64_t)leader * p.max_blocks;
  int bad = 0;
  int id_base = blk_lo;
  auto load_ids = [&](int base) {
    const int idx = base + lane;
    int id = idx < blk_hi ? bt[idx] : 0;
    const bool out = idx < blk_hi && (unsigned)id >= (unsigned)p.num_blocks;
    bad |= __ballot(out) != 0;
    return out ? 0 : id;
  };
  int ids = load_ids(id_base);

  const char* kpool = reinterpret_cast<const char*>(p.k_pool) + (int64_t)kvh * TILE;
  const char* vpool = reinterpret_cast<const char*>(p.v_pool) + (int64_t)kvh * TILE;
  const int64_t block_bytes = (int64_t)p.num_kv_heads * TILE;
  const int iters = (blk_hi - blk_lo + NB - 1) / NB;

  // Staging: per iteration each wave moves four 1 KiB pieces of the keys and
  // four of the values straight from HBM/L2 into LDS (global_load_lds: lane l
  // lands at LDS base + 16*l, so a piece is a 1 KiB contiguous run of LDS and
  // each lane picks the global chunk that belongs at its spot).  The loads
  // take no registers; the wave waits for them with an explicit counter wait
  // before the barrier that publishes the buffer.
  auto stage_issue = [&](int it, int buf) {
    const int first = blk_lo + it * NB;
    if (first - id_base >= 64) {  // next 64 ids
      id_base += 64;
      ids = load_ids(id_base);
    }
#pragma unroll
    for (int k = 0; k < STAGE_HALF / 1024 / NW; ++k) {
      const int piece = wave + NW * k;  // 1 KiB piece of the stage
      const int kb = piece * 1024 / TILE;
      const int in_tile = piece * 1024 % TILE;
      const int64_t base = (int64_t)__builtin_amdgcn_readlane(ids, first + kb - id_base) * block_bytes;
      const int q = in_tile / 16 + lane;  // 16-byte piece of the tile that this lane's LDS spot holds
      // keys: chunk q / BS, slot q % BS <- that chunk's key_slot_token
      lds_dma16(lds_addr(&lds[buf][0][piece * 1024]), kpool + base,
                ((q / BS) * BS + key_slot_token<BS>(q % BS, kb & 1)) * 16);
      // values: 16-token rows keep the pool's order; 32-token rows are rotated
      const int d = q / (BS / 8);
      const int vpiece = BS == 32 ? ((q & 3) ^ value_rot(d)) : (q & 1);
      lds_dma16(lds_addr(&lds[buf][1][piece * 1024]), vpool + base, d * (BS * 2) + vpiece * 16);
    }
  };

  f32x4 o[2][8];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[ct][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};

  // One iteration (64 tokens, always whole) of the wave's rows from LDS buffer
  // `buf`.  Program order: S^T of both 32-token pairs (matrix cores), then per
  // pair the online-softmax update and weights (vector unit) followed by its
  // P.V (matrix cores).  The second pair's S^T runs while the first pair's
  // weights are computed, and the first pair's P.V while the second's are.
  auto compute = [&](int buf) {
    f32x4 s[4][2];  // [run * 2 + S tile][column tile]
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const unsigned char* kt = &lds[buf][0][(sub >> 1) * RUN_BYTES];
      const int x = sub & 1;
      // the lane's row n of tile x: 32-token blocks slot 16x + n; 16-token blocks
      // block n / 8 of the run, slot n % 8 + 8 (x ^ block)
      const int koff = BS == 32 ? 16 * x + n : (n >> 3) * (TILE / 16) + (n & 7) + 8 * (x ^ (n >> 3));
      bf16x8 ka[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ka[i] = *reinterpret_cast<const bf16x8*>(kt + ((4 * i + kg) * BS + koff) * 16);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        s[sub][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[sub][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[i], qb[ct][i], s[sub][ct], 0, 0, 0);
      }
    }
#pragma unroll
    for (int pair = 0; pair < 2; ++pair) {
      const f32x4* s0 = s[2 * pair];
      const f32x4* s1 = s[2 * pair + 1];
      // column maxima of the pair's raw logits (the scale, > 0, is applied after)
      float mx[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const float a = maxp(maxp(maxp(s0[ct][0], s0[ct][1]), maxp(s0[ct][2], s0[ct][3])),
                             maxp(maxp(s1[ct][0], s1[ct][1]), maxp(s1[ct][2], s1[ct][3])));
        mx[ct] = maxp_xor32(maxp_xor16(a)) * p.scale_log2;
      }
      if (__ballot(mx[0] > m[0] + kRescaleSlack || mx[1] > m[1] + kRescaleSlack) != 0) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const float mn = maxp(m[ct], mx[ct]);
          const float alpha = fast_exp2(m[ct] - mn);
          lsum[ct] *= alpha;
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) o[ct][nt] *= alpha;
          m[ct] = mn;
        }
      }
      // weights as bf16 hi/lo operands: pr[j] is token 8kg + j of the run
      // (tile 0's rows for j < 4, tile 1's for j >= 4)
      bf16x8 pb_hi[2], pb_lo[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const float neg_m = -m[ct];
        float pr[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[r] = fast_exp2(fmaf(s0[ct][r], p.scale_log2, neg_m));
          pr[4 + r] = fast_exp2(fmaf(s1[ct][r], p.scale_log2, neg_m));
        }
        lsum[ct] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16(pr[2 * e], pr[2 * e + 1], &hw[e], &lw[e]);
        pb_hi[ct] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        pb_lo[ct] = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
      }
      const unsigned char* vr = &lds[buf][1][pair * RUN_BYTES];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        // dim 16nt + n, tokens 8kg..8kg+7 of the run
        const int d = 16 * nt + n;
        const int off = BS == 32 ? d * 64 + 16 * (kg ^ value_rot(d)) : (kg >> 1) * TILE + d * 32 + 16 * (kg & 1);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vr + off);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          o[ct][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb_hi[ct], o[ct][nt], 0, 0, 0);
          o[ct][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb_lo[ct], o[ct][nt], 0, 0, 0);
        }
      }
    }
  };

  stage_issue(0, 0);
  lds_dma_wait_all();
  __syncthreads();
  for (int it = 0; it < iters; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < iters;
    if (more) stage_issue(it + 1, buf ^ 1);  // buffer buf^1 was released by the last barrier
    if (wave_active) compute(buf);
    lds_dma_wait_all();
    __syncthreads();
  }

  if (!wave_active) return;
  // partials: row -> (member sequence, query head); slot (b, h, chunk)
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const float l = sum_xor32(sum_xor16(lsum[ct]));
    const int row = row0 + 16 * ct + n;
    if (row >= rows) continue;
    const int b = members[row / G];
    const int h = kvh * G + row % G;
    const int64_t pi = ((int64_t)b * p.num_heads + h) * p.num_slots + slot0;
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

}  // namespace

hipError_t launch_prefix(const PrefixArgs& p, int block_size, int group, hipStream_t s) {
  const int64_t units = (int64_t)p.num_kv_heads * p.num_chunks;
  const int64_t wgs = (units + kXcds - 1) / kXcds * kXcds * p.num_tiles;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  const dim3 block(64 * NW);
#define PKV_PREFIX(BS, G) hipLaunchKernelGGL((prefix_kernel<BS, G>), grid, block, 0, s, p)
  if (block_size == 16) {
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

// Pieces shared by the two decode kernel families (vector and matrix-core):
// the partition a workgroup owns, the block-id prefetch, and the merge of the
// per-wave softmax states into an output row or a split-K partial.
#pragma once

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace pkv {

// Longest sequences first.  Workgroups are dispatched in grid order, so when
// the sequence slot blockIdx.z names the slot-th longest sequence (ties by
// index), the long walks start first and the tail of the launch is short ones
// (largest-first scheduling).  Every workgroup ranks the context lengths itself
// (one candidate per thread, num_seqs <= kMaxRankSeqs), which costs one
// dependent load of the lengths; the host enables it for more than one sequence.

struct SeqPick {
  int b;
  int qrow;   // row of q and out (b, or the new token's row with several per sequence)
  int ctx_raw;
  int start;  // blocks covered by a shared-prefix pass (0 without one), not yet clipped to the context
  bool skip;  // the slot maps to no query row: the workgroup has nothing to do
};

// Blocks of sequence b that the shared-prefix pass covered (0 without one).
template <int BS>
__device__ __forceinline__ int covered_start(const DecodeArgs& a, int b) {
  return a.start_blocks ? prefix_covered_blocks(max(a.start_blocks[b], 0), BS) : 0;
}

// The sequence of rank `slot` when ordered by decreasing context length (ties
// by index), with its raw context length.  Every thread of the workgroup must
// call it (two barriers).  key = (length + 1) * 256 + 255 - index: distinct,
// larger for longer sequences and, among equal lengths, for smaller indices (a
// broken length counts as -1); rank = how many keys are larger.  The host
// enables it only for num_seqs <= kMaxRankSeqs and max_context < 2^23, so keys
// stay below 2^31.
__device__ __forceinline__ void sequence_of_rank(const DecodeArgs& a, int slot, int* sm_key, int* sm_pick, int* b,
                                                 int* ctx_raw) {
  const int t = threadIdx.x;
  const int nb = a.num_seqs;
  int raw = 0;
  uint32_t key = 0;
  if (t < nb) {
    raw = a.context_lens[t];
    const int len = (raw < 0 || raw > a.max_context) ? -1 : raw;
    key = (uint32_t)(len + 1) * 256u + (uint32_t)(255 - t);
    sm_key[t] = (int)key;
  }
  __syncthreads();
  if (t < nb) {
    int rank = 0;
    for (int o = 0; o < nb; ++o) rank += (uint32_t)sm_key[o] > key;
    if (rank == slot) {
      sm_pick[0] = t;
      sm_pick[1] = raw;
    }
  }
  __syncthreads();
  *b = sm_pick[0];
  *ctx_raw = sm_pick[1];
}

template <int BS>
__device__ __forceinline__ SeqPick pick_sequence(const DecodeArgs& a, int* sm_key, int* sm_pick) {
  if (a.query_start) {
    // several new tokens per sequence, one per slot: slot = b * max_query_len + i.
    // Token i sees context_lens[b] - n_b + i + 1 tokens, so it runs as a decode
    // over that many; a broken length (n_b > context, context > max_context,
    // n_b > max_query_len) turns the rows the grid covers into NaN.
    SeqPick p;
    p.b = blockIdx.z / a.max_query_len;
    const int i = blockIdx.z % a.max_query_len;
    const int qs = a.query_start[p.b], qe = a.query_start[p.b + 1];
    const int ctx = a.context_lens[p.b];
    const int qlen = qe - qs;
    p.skip = qs < 0 || qs > qe || qe > a.num_query_tokens || i >= qlen;
    p.qrow = qs + i;
    p.start = 0;
    const bool bad = ctx < qlen || ctx > a.max_context || qlen > a.max_query_len;
    p.ctx_raw = bad ? -1 : ctx - qlen + i + 1;
    return p;
  }
  if (!a.longest_first) {
    SeqPick p;
    p.b = blockIdx.z;
    p.qrow = p.b;
    p.ctx_raw = a.context_lens[p.b];
    p.start = covered_start<BS>(a, p.b);
    p.skip = false;
    return p;
  }
  SeqPick p;
  sequence_of_rank(a, blockIdx.z, sm_key, sm_pick, &p.b, &p.ctx_raw);
  p.qrow = p.b;
  p.start = covered_start<BS>(a, p.b);
  p.skip = false;
  return p;
}

// The (sequence, kv head, partition) a workgroup owns: grid = (partitions, kv
// heads, sequence slots), the slot mapped to a sequence by pick_sequence.
struct PartRange {
  int b, kvh, part;
  int qrow;     // row of q and out
  int start;    // first block of this pass (after a shared prefix)
  int ctx;      // context length (0 when context_lens[b] breaks its precondition)
  bool ctx_bad; // context_lens[b] < 0 or > max_context: the rows become NaN and nothing is read
  int nblocks;  // blocks of the sequence
  int nparts;   // partitions the sequence spans
  int blk_lo, blk_hi;
  int pre;      // shared-prefix partials merged at the end (0: none)
};

template <int BS>
__device__ __forceinline__ PartRange part_range(const DecodeArgs& a, const SeqPick& s) {
  PartRange r;
  r.part = blockIdx.x;
  r.kvh = blockIdx.y;
  r.b = s.b;
  r.qrow = s.qrow;
  const int ctx_raw = s.ctx_raw;
  r.ctx_bad = ctx_raw < 0 || ctx_raw > a.max_context;
  r.ctx = r.ctx_bad ? 0 : ctx_raw;
  r.nblocks = (r.ctx + BS - 1) / BS;
  r.start = min(s.start, r.nblocks);
  const int rest = r.nblocks - r.start;
  r.nparts = (rest + a.blocks_per_part - 1) / a.blocks_per_part;
  if (r.start > 0 && r.nparts == 0) r.nparts = 1;  // an empty suffix still merges the prefix partials
  r.blk_lo = r.start + r.part * a.blocks_per_part;
  r.blk_hi = min(r.nblocks, r.blk_lo + a.blocks_per_part);
  // The prefix partials of the sequence's group path, merged when this pass is
  // its only suffix partition.  Counted here, before the walk, so that the
  // dependent reads up the group tree overlap the first tile loads instead of
  // adding their round trips to the end of the workgroup.
  r.pre = (r.start > 0 && r.nparts == 1)
              ? path_slots(plan_groups(a.plan), plan_group_of(a.plan)[r.b], a.plan[kPlanBlockSize], a.prefix_chunk_blocks)
              : 0;
  return r;
}

// A workgroup past its sequence's last partition has nothing to read.  The one
// at partition 0 of an empty context writes the all-zero rows (NaN rows for a
// broken context length).  Returns true when the workgroup is done.
template <int G, int HD>
__device__ __forceinline__ bool finish_if_empty(const DecodeArgs& a, const PartRange& r) {
  if (r.part < r.nparts) return false;
  if (r.part == 0) {
    for (int idx = threadIdx.x; idx < G * HD; idx += blockDim.x) {
      const int64_t o = ((int64_t)r.qrow * a.num_heads + r.kvh * G + idx / HD) * HD + idx % HD;
      if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o] = r.ctx_bad ? 0x7fc0 : 0;
      else reinterpret_cast<float*>(a.out)[o] = r.ctx_bad ? NAN : 0.f;
    }
  }
  return true;
}

// Blocks of a partition are dealt to the waves round-robin: wave w takes
// partition blocks w, w + kWaves, w + 2*kWaves, ...; this is how many it gets.
__device__ __forceinline__ int wave_block_count(const PartRange& r, int wave) {
  const int n = max(r.blk_hi - r.blk_lo, 0);
  return n > wave ? (n - wave + kWaves - 1) / kWaves : 0;
}

// Block ids of one wave's blocks, 64 at a time: lane l holds the id of the
// wave's block 64*chunk + l.  One strided vector load per 64 blocks, then
// readlane; no tile load waits on a table lookup.
struct WaveIds {
  const int32_t* row;  // table entry of the wave's first block
  int limit;           // entries row[stride*i] with stride*i < limit lie inside the table row
  int stride;          // table entries between the wave's consecutive blocks
  int chunk;
  int ids;
};

// Ids of blocks first, first + stride, ... of sequence b's table row.  Entries
// past the sequence's last block may be read (they are inside the row of
// max_blocks entries) but never used.
__device__ __forceinline__ WaveIds wave_ids_from(const DecodeArgs& a, int b, int first, int lane,
                                                 int stride = kWaves) {
  WaveIds w;
  w.row = a.block_tables + (int64_t)b * a.max_blocks + first;
  w.limit = a.max_blocks - first;
  w.stride = stride;
  w.chunk = 0;
  w.ids = stride * lane < w.limit ? w.row[stride * lane] : 0;
  return w;
}

// Started before the context length is known, so the table load overlaps the
// context-length load.
__device__ __forceinline__ WaveIds wave_ids_begin(const DecodeArgs& a, const SeqPick& s, int wave, int lane) {
  return wave_ids_from(a, s.b, s.start + blockIdx.x * a.blocks_per_part + wave, lane);
}

// Checks the ids of the current chunk that the wave will use (its first cnt
// blocks): returns 1 when one lies outside the pool, and replaces it by block 0
// so that no load ever leaves the pool (the row turns NaN instead).
__device__ __forceinline__ int wave_ids_check(const DecodeArgs& a, WaveIds* w, int cnt, int lane) {
  const int used = cnt - 64 * w->chunk;
  const bool out = lane < used && (unsigned)w->ids >= (unsigned)a.num_blocks;
  if (out) w->ids = 0;
  return __ballot(out) != 0;
}

// Id of the wave's block i (i never decreases between calls).
__device__ __forceinline__ int wave_id_at(const DecodeArgs& a, WaveIds* w, int i, int cnt, int lane, int* bad) {
  const int c = i >> 6;
  if (c != w->chunk) {
    w->chunk = c;
    const int idx = w->stride * (64 * c + lane);
    w->ids = idx < w->limit ? w->row[idx] : 0;
    *bad |= wave_ids_check(a, w, cnt, lane);
  }
  return __builtin_amdgcn_readlane(w->ids, i & 63);
}

// Double-buffered walk over a wave's rounds of tiles: the loads of the next
// round are in flight while the current one is computed.  The steady-state
// loop always issues before it computes, and the last one or two rounds are
// peeled, so every path into a compute has the same number of younger loads
// outstanding and the wait before it covers only the round it uses.
template <typename Tile, typename Issue, typename Compute>
__device__ __forceinline__ void pipelined_rounds(int rounds, Tile* ta, Tile* tb, Issue&& issue, Compute&& compute) {
  if (rounds <= 0) return;
  issue(ta, 0);
  int rnd = 0;
  for (; rnd + 2 < rounds; rnd += 2) {
    issue(tb, rnd + 1);
    compute(ta, rnd);
    issue(ta, rnd + 2);
    compute(tb, rnd + 1);
  }
  if (rnd + 1 < rounds) {
    issue(tb, rnd + 1);
    compute(ta, rnd);
    compute(tb, rnd + 1);
  } else {
    compute(ta, rnd);
  }
}

// Per-wave softmax states in LDS, merged by the whole workgroup:
//   M = max_w m_w,  l = sum_w 2^(m_w - M) l_w,  acc = sum_w 2^(m_w - M) acc_w
// (logits in base 2).  A sequence inside one partition gets its output row
// acc / l (rounded to nearest even for bf16); otherwise the partial (M, l, acc)
// goes to the workspace for the split-K merge.  A bad block id anywhere in the
// partition turns the row into NaN.  After a shared-prefix pass the chunk
// partials of the prefix are folded in too, kPreBatch at a time: their loads
// are issued together (one memory round trip per batch, not one per partial)
// and the running maximum moves once per batch.  16 covers the 9 chunks of a
// 30000-token prefix in one trip (8 took two: shared-prefix call 188 -> 183
// us, one more register).
constexpr int kPreBatch = 16;

template <int G, int HD, int NW>
__device__ __forceinline__ void merge_waves_and_store(const DecodeArgs& a, const PartRange& r,
                                                      float (*sm_acc)[G][HD], float (*sm_m)[G], float (*sm_l)[G],
                                                      const int* sm_bad) {
  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) any_bad |= sm_bad[w];
  const int h0 = r.kvh * G;
  // E elements of row h, dims d0 + stride * e: one thread's share.  All its
  // prefix-partial loads of a batch are issued together, so a thread with
  // several elements of one row pays one round trip per batch, not one per
  // element, and loads the row's maxima and sums once.
  auto merge_row = [&](auto e_tag, int h, int d0, int stride) {
    constexpr int E = decltype(e_tag)::value;
    const int hq = h0 + h;
    // partials of the shared-prefix pass (counted in part_range)
    const int pre = r.pre;
    const int64_t pre_base = ((int64_t)r.b * a.num_heads + hq) * a.prefix_chunks;
    float big_m = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) big_m = fmaxf(big_m, sm_m[w][h]);
    float l = 0.f, acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = (sm_m[w][h] == -INFINITY) ? 0.f : fast_exp2(sm_m[w][h] - big_m);
      l = fmaf(f, sm_l[w][h], l);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(f, sm_acc[w][h][d0 + stride * e], acc[e]);
    }
    for (int c0 = 0; c0 < pre; c0 += kPreBatch) {
      // slots past the last partial are read in bounds (clamped) and dropped by a select
      float pm[kPreBatch], pl[kPreBatch], pa[kPreBatch][E];
#pragma unroll
      for (int k = 0; k < kPreBatch; ++k) {
        const int64_t s = pre_base + min(c0 + k, pre - 1);
        pm[k] = a.pre_m[s];
        pl[k] = a.pre_l[s];
#pragma unroll
        for (int e = 0; e < E; ++e) pa[k][e] = a.pre_acc[s * HD + d0 + stride * e];
      }
      float bm = -INFINITY;
#pragma unroll
      for (int k = 0; k < kPreBatch; ++k) bm = fmaxf(bm, c0 + k < pre ? pm[k] : -INFINITY);
      if (bm > big_m) {  // move the reference once for the batch
        const float f = big_m == -INFINITY ? 0.f : fast_exp2(big_m - bm);
        l *= f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] *= f;
        big_m = bm;
      }
#pragma unroll
      for (int k = 0; k < kPreBatch; ++k) {
        // a NaN partial (bad block id in the prefix) stays NaN through the exponent
        const float f = c0 + k < pre ? fast_exp2(pm[k] - big_m) : 0.f;
        l = fmaf(f, c0 + k < pre ? pl[k] : 0.f, l);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(f, c0 + k < pre ? pa[k][e] : 0.f, acc[e]);
      }
    }
    if (any_bad) {
      big_m = NAN;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = NAN;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = d0 + stride * e;
      if (r.nparts == 1) {
        const float o = acc[e] / l;
        const int64_t oi = ((int64_t)r.qrow * a.num_heads + hq) * HD + d;
        if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_rne(o);
        else reinterpret_cast<float*>(a.out)[oi] = o;
      } else {
        const int64_t pi = ((int64_t)r.qrow * a.num_heads + hq) * a.num_parts + r.part;
        a.ws_acc[pi * HD + d] = acc[e];
        if (d == 0) {
          a.ws_m[pi] = big_m;
          a.ws_l[pi] = l;
        }
      }
    }
  };
  constexpr int T = 64 * NW;
  if constexpr (G * HD >= T && T % G == 0 && HD % (T / G) == 0) {
    // T / G threads per row, HD * G / T consecutive-stride elements each
    constexpr int TPR = T / G;
    merge_row(std::integral_constant<int, HD / TPR>{}, (int)threadIdx.x / TPR, (int)threadIdx.x % TPR, TPR);
  } else {
    for (int idx = threadIdx.x; idx < G * HD; idx += T) merge_row(std::integral_constant<int, 1>{}, idx / HD, idx % HD, 1);
  }
}

}  // namespace pkv

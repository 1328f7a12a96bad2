// Paged attention for several new tokens per sequence, causal among them
// (bf16, head_dim 128), on matrix cores.
//
// A verify step of speculative decoding, or a chunk of a prompt, appends n_b
// tokens to sequence b and attends from each of them: new token i (position
// ctx - n_b + i) sees the cached tokens up to and including itself.  The pages
// name these uses of the paged cache (speculative decoding and forked
// sequences sharing it: "Master Paged Attention for LLM Inference", "How Paged
// Attention Works: The Mechanics", item 4; prompt prefill filling it:
// "PagedAttention Explained", "Enabling Automatic Prefix Caching") without a
// formula; the mask is the standard causal one of a decoder.
//
// All n_b * G query rows of one kv head read the same key/value tiles, so the
// per-tile work is dense: the rows (new token i, head h of the group), i-major
// (row = i*G + h), fill the columns of the matrix-core tile.  A workgroup takes
// 16 * CT rows (CT = 1 or 2 column tiles) of one (sequence, kv head,
// partition), and walks only the blocks its last row sees.
//
// One wave, per 16-token sub-tile:
//  * S^T = K . Q^T, v_mfma_f32_16x16x32_bf16, 4 instructions per 16-row column
//    tile; lane (column n, group kg) gets S^T[token 4kg+r][row 16ct + n].
//  * One 16-lane row swap per logit (v_permlane16_swap) regroups them so that
//    lane L holds tokens 8h..8h+7 (h = L / 32) of one column c = L % 32: with
//    two column tiles, rows 0..31 of the workgroup; with one, row c % 16, the
//    columns 16..31 repeating 0..15.  That is the B-operand layout of the
//    32x32x16 matrix instruction, so P.V runs on v_mfma_f32_32x32x16_bf16 (full
//    rate on gfx950, where the 16x16x16 form runs at half): O^T[32 dims x 32
//    columns] += V^T[32 dims x 16 tokens] . P^T, 4 instructions per 128 dims.
//    Weights go in as bf16 hi + lo parts: as two instructions with 32 rows,
//    as columns 0..15 (hi) and 16..31 (lo) of one with 16.
//  * Causal and context mask per lane: token < the row's limit (positions the
//    row sees).  Only sub-tiles reaching past the tile's smallest limit are
//    masked (a wave-uniform branch).
// Partition partials are merged by multi_reduce_kernel.
#include "decode_common.h"

namespace pkv {

// POLICY: cache policy of the tile loads; streaming with one row tile per unit,
// default when further row tiles read the same tiles again from L2.
template <int BS, int G, int CT, int U, int POLICY>
__global__ __launch_bounds__(64 * kWaves) void multi_mfma_kernel(DecodeArgs a) {
  constexpr int NW = kWaves;
  constexpr int HD = 128;
  constexpr bool PAIR = BS == 8;           // a 16-token unit spans two blocks, each lane loading from its own
  constexpr int SUB = PAIR ? 1 : BS / 16;  // 16-token sub-tiles per block
  constexpr int TILE_BYTES = HD * BS * 2;
  constexpr int R = 16 * CT;    // rows per workgroup
  // the two 16-token sub-tiles of a 32-token block share the value tile's
  // 128-byte lines: those loads keep the default policy
  constexpr int VPOLICY = BS <= 16 ? POLICY : kCacheDefault;
  static_assert(64 % ((U + SUB - 1) / SUB) == 0, "a round must not straddle two id loads");

  struct Tile {
    uint4 k[4];  // keys of the sub-tile's 16 tokens, MFMA A-operand order
    uint4 v[4];  // values: 32 dims x 16 tokens per instruction, 8 tokens of one dim per lane
  };

  __shared__ float sm_acc[NW][16][HD];
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  __shared__ int sm_bad[NW];
  __shared__ int sm_key[kMaxRankSeqs];
  __shared__ int sm_pick[2];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n = lane & 15;
  const int kg = lane >> 4;

  // Workgroup -> (unit, row tile), XCD-aware: workgroup i runs on XCD i % 8,
  // and the row tiles of one unit (partition, kv head, sequence) share an XCD
  // and are dispatched back to back, so all but the first find the unit's
  // tiles in that XCD's L2.
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int unit = (slot / a.row_tiles) * kXcds + xcd;
  const int rt = slot % a.row_tiles;
  if (unit >= a.num_parts * a.num_kv_heads * a.num_seqs) return;
  const int part = unit % a.num_parts;
  const int kvh = (unit / a.num_parts) % a.num_kv_heads;
  // sequence slot -> sequence: longest first when the host asks for it (the
  // long walks start first, the launch ends on short ones)
  int b = unit / (a.num_parts * a.num_kv_heads);
  int ctx_raw;
  if (a.longest_first) sequence_of_rank(a, b, sm_key, sm_pick, &b, &ctx_raw);
  else ctx_raw = a.context_lens[b];

  const int qs = a.query_start[b], qe = a.query_start[b + 1];
  if (qs < 0 || qs > qe || qe > a.num_query_tokens) return;  // its rows are unknown: nothing is written
  const int qlen = qe - qs;
  const int nrows = min(qlen, a.max_query_len) * G;  // rows the grid covers
  const int r0 = rt * R;
  if (r0 >= nrows) return;
  const int r_end = min(r0 + R, nrows);
  const bool ctx_bad = ctx_raw < qlen || ctx_raw > a.max_context || qlen > a.max_query_len;
  const int base = ctx_raw - qlen + 1;              // tokens new token 0 sees
  const int lim_min = base + r0 / G;                // tokens the tile's first row sees
  const int ctx = ctx_bad ? 0 : base + (r_end - 1) / G;  // ... and its last row: the tile's walk
  const int nblocks = (ctx + BS - 1) / BS;
  const int nparts = (nblocks + a.blocks_per_part - 1) / a.blocks_per_part;
  if (part >= nparts) {
    if (part == 0) {  // a broken length: NaN rows
      for (int idx = threadIdx.x; idx < (r_end - r0) * HD; idx += blockDim.x) {
        const int row = r0 + idx / HD;
        const int64_t o = ((int64_t)(qs + row / G) * a.num_heads + kvh * G + row % G) * HD + idx % HD;
        if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o] = 0x7fc0;
        else reinterpret_cast<float*>(a.out)[o] = NAN;
      }
    }
    return;
  }
  const int blk_lo = part * a.blocks_per_part;
  const int blk_hi = min(nblocks, blk_lo + a.blocks_per_part);

  // S^T columns: lane column n of column tile ct is row r0 + 16ct + n.
  bf16x8 qb[CT][4];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int row = r0 + 16 * ct + n;
    const bool used = row < r_end;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) +
                           ((int64_t)(qs + (used ? row / G : 0)) * a.num_heads + kvh * G + row % G) * HD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = used ? load16(qrow + 32 * i + 8 * kg) : make_uint4(0, 0, 0, 0);
      qb[ct][i] = __builtin_bit_cast(bf16x8, w);
    }
  }
  // After the regrouping: lane L has column c = L % 32, tokens 8h..8h+7 (h = L / 32);
  // its row is r0 + c with two column tiles, r0 + c % 16 with one.
  const int c = lane & 31;
  const int h = lane >> 5;
  const int my_row = r0 + (CT == 2 ? c : (c & 15));
  const int lim = my_row < r_end ? base + my_row / G : 0;  // tokens the lane's row sees
  const bool lo_col = CT == 1 && c >= 16;                   // one column tile: columns 16..31 take the lo parts

  // the wave's blocks w, w + NW, ...; with 8-token blocks its pairs p = w, w + NW, ...
  // (blocks 2p and 2p + 1, ids from two strided streams; cnt1 = pairs with a second block)
  const int nb_part = blk_hi - blk_lo;
  const int nunits = PAIR ? (nb_part + 1) / 2 : nb_part;
  const int nfull = nb_part / 2;
  const int cnt = nunits > wave ? (nunits - wave + NW - 1) / NW : 0;
  const int cnt1 = PAIR && nfull > wave ? (nfull - wave + NW - 1) / NW : 0;
  WaveIds wids = wave_ids_from(a, b, blk_lo + (PAIR ? 2 : 1) * wave, lane, (PAIR ? 2 : 1) * NW);
  WaveIds wids1{};
  if constexpr (PAIR) wids1 = wave_ids_from(a, b, blk_lo + 2 * wave + 1, lane, 2 * NW);
  int bad = wave_ids_check(a, &wids, cnt, lane);
  if constexpr (PAIR) bad |= wave_ids_check(a, &wids1, cnt1, lane);

  f32x16 o[4];  // O^T, 32 dims per instruction: lane holds column c, dims 32db + 8(i/4) + 4h + i%4
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (int64_t)kvh * TILE_BYTES;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (int64_t)kvh * TILE_BYTES;
  const int64_t block_bytes = (int64_t)a.num_kv_heads * TILE_BYTES;
  const int units = cnt * SUB;

  // loads of round rnd: sub-tiles rnd*U .. rnd*U+U-1 of the wave (a missing one
  // re-reads the wave's last sub-tile, a cache hit, and is not used)
  auto issue = [&](Tile* T, int rnd) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int x = min(rnd * U + u, units - 1);
      if constexpr (PAIR) {
        // a pair without a second block reads the first twice (those tokens lie past
        // the partition and are masked); ids are checked, so every address is in the pool
        const int id0 = wave_id_at(a, &wids, x, cnt, lane, &bad);
        const int id1 = x < cnt1 ? wave_id_at(a, &wids1, x, cnt1, lane, &bad) : id0;
        const char* kt = kbase + (int64_t)(n < 8 ? id0 : id1) * block_bytes;  // token n: row n % 8 of block n / 8
        const char* vt = vbase + (int64_t)(h == 0 ? id0 : id1) * block_bytes;  // tokens 8h..8h+7: all of block h
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const char* p = kt + ((4 * i + kg) * BS + (n & 7)) * 16;
          T[u].k[i] = POLICY == kCacheStream ? gload16_stream(p) : load16(p);
        }
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const char* p = vt + (32 * db + c) * BS * 2;
          T[u].v[db] = POLICY == kCacheStream ? gload16_stream(p) : load16(p);
        }
      } else {
        const int sub = x % SUB;
        const int64_t off = (int64_t)wave_id_at(a, &wids, x / SUB, cnt, lane, &bad) * block_bytes;
        const auto kt = tile_rsrc(kbase + off, TILE_BYTES);
        const auto vt = tile_rsrc(vbase + off, TILE_BYTES);
#pragma unroll
        for (int i = 0; i < 4; ++i) T[u].k[i] = bload16<POLICY>(kt, ((4 * i + kg) * BS + 16 * sub + n) * 16);
        // values: dim 32db + c, tokens 8h..8h+7 of the sub-tile (16 contiguous bytes of the dim-major tile)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          T[u].v[db] = bload16<VPOLICY>(vt, ((32 * db + c) * BS + 16 * sub + 8 * h) * 2);
      }
    }
  };

  auto compute = [&](Tile* T, int rnd) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int x = rnd * U + u;
      if (x >= units) break;
      // first token of the unit, and its rows inside the walk and the partition
      const int tok0 = PAIR ? (blk_lo + 2 * (wave + NW * x)) * BS : (blk_lo + wave + NW * (x / SUB)) * BS + 16 * (x % SUB);
      const int valid = min(ctx, blk_hi * BS) - tok0;
      if (valid <= 0) continue;  // second half of a block past the walk

      f32x4 s[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        s[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, T[u].k[i]), qb[ct][i], s[ct],
                                                          0, 0, 0);
      }
      // regroup: the swap exchanges odd 16-lane rows of its first operand with
      // even rows of its second, which leaves tokens 8h + r in the first result
      // and 8h + 4 + r in the second, for the lane's own column
      float t8[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(s[0][r]), __float_as_uint(s[CT - 1][r]),
                                                         false, false);
        t8[r] = __uint_as_float(sw[0]);
        t8[4 + r] = __uint_as_float(sw[1]);
      }
      // the row's visible tokens (every one when the sub-tile ends before the tile's
      // smallest limit and inside the partition).  A pair cut by the partition end
      // (valid == 8) holds a repeat of its first block in tokens 8..15: those lie
      // below the causal limit, so the partition bound must mask their logits too.
      const bool masked = tok0 + 16 > lim_min || valid < 16;
      bool keep[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) keep[e] = !masked || (8 * h + e < valid && tok0 + 8 * h + e < lim);

      // raw logits; the scale (>= 0) is applied to the maximum and inside the exponent
      float v8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v8[e] = keep[e] ? t8[e] : -INFINITY;
      const float raw = maxp_xor32(maxp(maxp(maxp(v8[0], v8[1]), maxp(v8[2], v8[3])),
                                        maxp(maxp(v8[4], v8[5]), maxp(v8[6], v8[7]))));
      const float mx = raw == -INFINITY ? -INFINITY : raw * a.scale_log2;  // nothing visible here
      if (__ballot(mx > m + kRescaleSlack) != 0) {
        const float mn = maxp(m, mx);
        const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m - mn);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;
        m = mn;
      }
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = keep[e] ? fast_exp2(fmaf(t8[e], a.scale_log2, -m)) : 0.f;
      lsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split_bf16(p[2 * e], p[2 * e + 1], &hw[e], &lw[e]);
      const bf16x8 pb_hi = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      const bf16x8 pb_lo = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));

      if (valid < 16) {  // value rows past the walk may hold NaN: zero them, a zero weight is not enough
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          uint32_t w[4] = {T[u].v[db].x, T[u].v[db].y, T[u].v[db].z, T[u].v[db].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (8 * h + 2 * e >= valid) w[e] &= 0xffff0000u;
            if (8 * h + 2 * e + 1 >= valid) w[e] &= 0x0000ffffu;
          }
          T[u].v[db] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 va = __builtin_bit_cast(bf16x8, T[u].v[db]);
        if constexpr (CT == 2) {
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb_hi, o[db], 0, 0, 0);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb_lo, o[db], 0, 0, 0);
        } else {
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, lo_col ? pb_lo : pb_hi, o[db], 0, 0, 0);
        }
      }
    }
  };

  Tile ta[U], tb[U];
  pipelined_rounds((units + U - 1) / U, ta, tb, issue, compute);

  // wave totals: the weight sum over both token halves; one column tile adds
  // each row's hi and lo columns (c and c + 16)
  const float l = sum_xor32(lsum);
  if constexpr (CT == 1) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] = sum_xor16(o[db][i]);
  }

  // Per group of 16 columns: the waves' states through LDS, merged by the
  // workgroup: M = max_w m_w, l = sum_w 2^(m_w - M) l_w, acc = sum_w 2^(m_w - M) acc_w.
  if (lane == 0) sm_bad[wave] = bad;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    if (ct) __syncthreads();  // the previous group's merge has read the buffers
    if ((c >> 4) == ct) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) sm_acc[wave][c & 15][32 * db + 8 * (i / 4) + 4 * h + i % 4] = o[db][i];
      if (h == 0) {
        sm_m[wave][c & 15] = m;
        sm_l[wave][c & 15] = l;
      }
    }
    __syncthreads();
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any_bad |= sm_bad[w];
    for (int idx = threadIdx.x; idx < 16 * HD; idx += 64 * NW) {
      const int col = idx / HD, d = idx % HD;
      const int row = r0 + 16 * ct + col;
      if (row >= r_end) continue;
      float big_m = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) big_m = fmaxf(big_m, sm_m[w][col]);
      float lt = 0.f, acc = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = sm_m[w][col] == -INFINITY ? 0.f : fast_exp2(sm_m[w][col] - big_m);
        lt = fmaf(f, sm_l[w][col], lt);
        acc = fmaf(f, sm_acc[w][col][d], acc);
      }
      if (any_bad) {
        big_m = NAN;
        acc = NAN;
      }
      const int64_t hrow = (int64_t)(qs + row / G) * a.num_heads + kvh * G + row % G;
      if (nparts == 1) {
        const float y = acc / lt;
        if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[hrow * HD + d] = (uint16_t)f32_to_bf16_rne(y);
        else reinterpret_cast<float*>(a.out)[hrow * HD + d] = y;
      } else {
        const int64_t pi = hrow * a.num_parts + part;
        a.ws_acc[pi * HD + d] = acc;
        if (d == 0) {
          a.ws_m[pi] = big_m;
          a.ws_l[pi] = lt;
        }
      }
    }
  }
}

bool multi_mfma_supported(int bf16, int hd, int bs, int g) {
  return bf16 && hd == 128 && (bs == 8 || bs == 16 || bs == 32) && (g == 1 || g == 2 || g == 4 || g == 8);
}

template <int CT, int U, int POLICY>
static hipError_t launch_ct(const DecodeArgs& a, int bs, int g, hipStream_t s) {
  const int64_t units = (int64_t)a.num_parts * a.num_kv_heads * a.num_seqs;
  const int64_t wgs = (units + kXcds - 1) / kXcds * kXcds * a.row_tiles;
  if (wgs <= 0 || wgs > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  const dim3 block(64 * kWaves);
#define PKV_MULTI(BS, G) hipLaunchKernelGGL((multi_mfma_kernel<BS, G, CT, U, POLICY>), grid, block, 0, s, a)
  if (bs == 8) {
    switch (g) {
      case 1: PKV_MULTI(8, 1); break;
      case 2: PKV_MULTI(8, 2); break;
      case 4: PKV_MULTI(8, 4); break;
      case 8: PKV_MULTI(8, 8); break;
      default: return hipErrorInvalidValue;
    }
  } else if (bs == 16) {
    switch (g) {
      case 1: PKV_MULTI(16, 1); break;
      case 2: PKV_MULTI(16, 2); break;
      case 4: PKV_MULTI(16, 4); break;
      case 8: PKV_MULTI(16, 8); break;
      default: return hipErrorInvalidValue;
    }
  } else if (bs == 32) {
    switch (g) {
      case 1: PKV_MULTI(32, 1); break;
      case 2: PKV_MULTI(32, 2); break;
      case 4: PKV_MULTI(32, 4); break;
      case 8: PKV_MULTI(32, 8); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef PKV_MULTI
  return hipGetLastError();
}

hipError_t launch_multi_mfma(const DecodeArgs& a, int bs, int g, int col_tiles, int inflight, hipStream_t s) {
  if (a.rows_per_tile != 16 * col_tiles) return hipErrorInvalidValue;
  const bool stream = a.row_tiles == 1;
  if (col_tiles == 1 && inflight == 2)
    return stream ? launch_ct<1, 2, kCacheStream>(a, bs, g, s) : launch_ct<1, 2, kCacheDefault>(a, bs, g, s);
  if (col_tiles == 1 && inflight == 1)
    return stream ? launch_ct<1, 1, kCacheStream>(a, bs, g, s) : launch_ct<1, 1, kCacheDefault>(a, bs, g, s);
  if (col_tiles == 2 && inflight == 1)
    return stream ? launch_ct<2, 1, kCacheStream>(a, bs, g, s) : launch_ct<2, 1, kCacheDefault>(a, bs, g, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv

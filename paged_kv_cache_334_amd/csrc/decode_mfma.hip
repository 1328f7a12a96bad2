// Paged decode attention for grouped query heads on matrix cores (bf16,
// head_dim 128, 4 or 8 query heads per kv head).
//
// When G query heads share one kv head, every key/value tile they read is the
// same, and the per-tile work is a small dense contraction: logits [G x 16
// tokens] = q [G x 128] . K^T, then acc [G x 128] += P [G x 16] . V.  This
// kernel puts both on MFMA instructions; HBM traffic is unchanged (each tile is
// read once per (sequence, kv head) as in the vector kernel).
//
// One wave, per 16-token sub-tile of a block:
//  * S^T = K . Q^T with v_mfma_f32_16x16x32_bf16 (4 instructions over the 128
//    dims).  A operand = keys: lane (row n = lane%16 = token, group kg =
//    lane/16) holds the 16-byte chunk 4i+kg of token n, which the key layout
//    stores contiguously for 16 consecutive tokens.  B operand = q^T: lane
//    (column n = head slot, group kg) holds dims 32i+8kg..+7 of that head.
//    Result: lane holds S^T[token 4kg+r][head slot n], r = 0..3.
//  * Online softmax per head slot: max over the lane's 4 tokens, then across
//    the 4 lane groups (xor 16, 32); weights p = exp2(s - m) in float32.
//  * O^T += V^T . P^T with v_mfma_f32_16x16x16_bf16 (8 instructions, one per
//    16 dims).  A operand = values: lane (row = dim 16nt + n, group kg) holds
//    tokens 4kg..4kg+3 of that dim -- 8 contiguous bytes of the dim-major value
//    tile.  B operand = P^T: exactly the 4 weights the lane already holds.
// Matrix cores take bfloat16 operands, so each weight is split as
// p = hi + lo (hi = bf16(p), lo = bf16(p - hi)); head slots 0..G-1 carry hi and
// G..2G-1 carry lo of the same heads (their q columns are duplicated), and the
// two output columns are added at the end.  The weight then keeps ~16
// significant bits instead of 8.
//
// Memory side as in the vector kernel (block ids per 64 blocks, broadcast with
// readlane; double-buffered rounds), with the 16-token sub-tile as the unit: a
// round is U sub-tiles, i.e. U blocks of 16 tokens, U/2 blocks of 32, or U
// pairs of consecutive 8-token blocks.  In a pair each lane's tokens lie in one
// of the two blocks: the lane picks its block's tile base and loads through a
// per-lane address (one streaming global load per operand).
#include "decode_common.h"

namespace pkv {

template <int BS, int G, int U>
__global__ __launch_bounds__(64 * kWaves) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NW = kWaves;
  constexpr int HD = 128;
  constexpr bool PAIR = BS == 8;           // a 16-token unit spans two blocks
  constexpr int SUB = PAIR ? 1 : BS / 16;  // 16-token sub-tiles per block
  constexpr int TILE_BYTES = HD * BS * 2;
  // With 32-token blocks a 128-byte line of the value tile holds 2 dims x 32
  // tokens, and the block's two 16-token sub-tiles each read half of it: the
  // second half must still be in cache, so those loads keep the default policy.
  constexpr int VPOLICY = BS <= 16 ? kCacheStream : kCacheDefault;
  static_assert(2 * G <= 16, "group too large for one 16-column tile");
  static_assert(64 % ((U + SUB - 1) / SUB) == 0, "a round must not straddle two id loads");

  struct Tile {
    uint4 k[4];  // keys of the sub-tile's 16 tokens, MFMA A-operand order
    uint2 v[8];  // values, 16 dims x 4 tokens per instruction
  };

  __shared__ float sm_acc[NW][G][HD];
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  __shared__ int sm_bad[NW];
  __shared__ int sm_key[kMaxRankSeqs];
  __shared__ int sm_pick[2];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n = lane & 15;   // MFMA column: head slot (S^T, O^T) / row: token (K) or dim (V)
  const int kg = lane >> 4;  // lane group
  const bool used = n < 2 * G;
  const bool lo_slot = n >= G;
  const int hslot = n % G;

  const SeqPick seq = pick_sequence<BS>(a, sm_key, sm_pick);
  // pairs of 8-token blocks: the wave's pairs p = wave, wave + NW, ... hold
  // blocks 2p and 2p + 1 of the partition, whose ids come from two strided streams
  WaveIds wids, wids1{};
  if constexpr (PAIR) {
    const int first = seq.start + blockIdx.x * a.blocks_per_part + 2 * wave;
    wids = wave_ids_from(a, seq.b, first, lane, 2 * NW);
    wids1 = wave_ids_from(a, seq.b, first + 1, lane, 2 * NW);
  } else {
    wids = wave_ids_begin(a, seq, wave, lane);
  }
  bf16x8 qb[4];
  {
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)seq.qrow * a.num_heads + blockIdx.y * G + hslot) * HD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 w = used ? load16(qrow + 32 * i + 8 * kg) : make_uint4(0, 0, 0, 0);
      qb[i] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const PartRange r = part_range<BS>(a, seq);
  if (finish_if_empty<G, HD>(a, r)) return;
  int cnt, cnt1 = 0;  // the wave's blocks (or pairs), and its pairs whose second block exists
  if constexpr (PAIR) {
    const int nb = max(r.blk_hi - r.blk_lo, 0);
    const int pairs = (nb + 1) / 2, full = nb / 2;
    cnt = pairs > wave ? (pairs - wave + NW - 1) / NW : 0;
    cnt1 = full > wave ? (full - wave + NW - 1) / NW : 0;
  } else {
    cnt = wave_block_count(r, wave);
  }
  int bad = wave_ids_check(a, &wids, cnt, lane);
  if constexpr (PAIR) bad |= wave_ids_check(a, &wids1, cnt1, lane);

  f32x4 o[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (int64_t)r.kvh * TILE_BYTES;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (int64_t)r.kvh * TILE_BYTES;
  const int64_t block_bytes = (int64_t)a.num_kv_heads * TILE_BYTES;
  const int units = cnt * SUB;

  // loads of round rnd: sub-tiles rnd*U .. rnd*U+U-1 of the wave (a missing one
  // re-reads the wave's last sub-tile, a cache hit, and is not used)
  auto issue = [&](Tile* T, int rnd) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int x = min(rnd * U + u, units - 1);
      if constexpr (PAIR) {
        // a pair without a second block (the partition's last, odd one) reads the
        // first block twice; those tokens lie past the partition and are masked
        // (ids are checked against the pool, so every address below lies inside it)
        const int id0 = wave_id_at(a, &wids, x, cnt, lane, &bad);
        const int id1 = x < cnt1 ? wave_id_at(a, &wids1, x, cnt1, lane, &bad) : id0;
        // keys: token n of the unit is row n % 8 of block n / 8
        const char* kt = kbase + (int64_t)(n < 8 ? id0 : id1) * block_bytes;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          T[u].k[i] = gload16_stream(kt + ((4 * i + kg) * BS + (n & 7)) * 16);
        // values: tokens 4kg..4kg+3 of the unit are rows 4(kg % 2).. of block kg / 2
        const char* vt = vbase + (int64_t)(kg < 2 ? id0 : id1) * block_bytes;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) T[u].v[nt] = gload8_stream(vt + ((16 * nt + n) * BS + 4 * (kg & 1)) * 2);
      } else {
        const int sub = x % SUB;
        const int64_t off = (int64_t)wave_id_at(a, &wids, x / SUB, cnt, lane, &bad) * block_bytes;
        const auto kt = tile_rsrc(kbase + off, TILE_BYTES);
        const auto vt = tile_rsrc(vbase + off, TILE_BYTES);
#pragma unroll
        for (int i = 0; i < 4; ++i) T[u].k[i] = bload16<kCacheStream>(kt, ((4 * i + kg) * BS + 16 * sub + n) * 16);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
          T[u].v[nt] = bload8<VPOLICY>(vt, ((16 * nt + n) * BS + 16 * sub + 4 * kg) * 2);
      }
    }
  };

  auto compute = [&](Tile* T, int rnd) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int x = rnd * U + u;
      if (x >= units) break;
      // first token of the unit, and its rows inside the context and the partition
      const int tok0 = PAIR ? (r.blk_lo + 2 * (wave + NW * x)) * BS
                            : (r.blk_lo + wave + NW * (x / SUB)) * BS + 16 * (x % SUB);
      const int valid = min(r.ctx, r.blk_hi * BS) - tok0;
      if (valid <= 0) continue;  // second half of a block past the context

      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, T[u].k[i]), qb[i], s, 0, 0, 0);

      // raw logits; the scale (> 0) is applied to the maximum and inside the exponent
      float sr[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sr[rr] = (4 * kg + rr < valid) ? s[rr] : -INFINITY;
      float mx = maxp(maxp(sr[0], sr[1]), maxp(sr[2], sr[3]));
      mx = maxp_xor32(maxp_xor16(mx)) * a.scale_log2;  // per column (head slot)
      if (__ballot(mx > m + kRescaleSlack) != 0) {
        const float mn = maxp(m, mx);
        const float alpha = fast_exp2(m - mn);
        lsum *= alpha;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) o[nt] *= alpha;
        m = mn;
      }
      // a select, not the -inf logit, zeroes the weight past the context (-inf times a zero scale is NaN)
      float p[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) p[rr] = (4 * kg + rr < valid) ? fast_exp2(fmaf(s[rr], a.scale_log2, -m)) : 0.f;
      lsum += (p[0] + p[1]) + (p[2] + p[3]);

      // columns 0..G-1 take the weights' bf16 hi parts, G..2G-1 their lo parts
      uint32_t pw[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        uint32_t hi, lo;
        split_bf16(p[2 * e], p[2 * e + 1], &hi, &lo);
        pw[e] = used ? (lo_slot ? lo : hi) : 0u;
      }
      const s16x4 pb = __builtin_bit_cast(s16x4, make_uint2(pw[0], pw[1]));

      if (valid < 16) {  // rows past the context may hold NaN: zero them, a zero weight is not enough
        const int first = 4 * kg;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          uint32_t w0 = T[u].v[nt].x, w1 = T[u].v[nt].y;
          if (first + 0 >= valid) w0 &= 0xffff0000u;
          if (first + 1 >= valid) w0 &= 0x0000ffffu;
          if (first + 2 >= valid) w1 &= 0xffff0000u;
          if (first + 3 >= valid) w1 &= 0x0000ffffu;
          T[u].v[nt] = make_uint2(w0, w1);
        }
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, T[u].v[nt]), pb, o[nt], 0, 0, 0);
    }
  };

  Tile ta[U], tb[U];
  pipelined_rounds((units + U - 1) / U, ta, tb, issue, compute);

  // wave totals: weight sum over the 4 lane groups; hi + lo columns of each head
  const float l = sum_xor32(sum_xor16(lsum));
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float other = shfl(o[nt][rr], (lane + G) & 63);
      if (n < G) sm_acc[wave][n][16 * nt + 4 * kg + rr] = o[nt][rr] + other;
    }
  }
  if (kg == 0 && n < G) {
    sm_m[wave][n] = m;
    sm_l[wave][n] = l;
  }
  if (lane == 0) sm_bad[wave] = bad;
  __syncthreads();
  merge_waves_and_store<G, HD, NW>(a, r, sm_acc, sm_m, sm_l, sm_bad);
}

bool mfma_supported(int bf16, int hd, int bs, int g) {
  return bf16 && hd == 128 && (bs == 8 || bs == 16 || bs == 32) && (g == 4 || g == 8);
}

template <int U>
static hipError_t launch_u(const DecodeArgs& a, int bs, int g, hipStream_t s) {
  const dim3 grid(a.num_parts, a.num_kv_heads, a.num_seqs);
  const dim3 block(64 * kWaves);
  if (bs == 8 && g == 4) hipLaunchKernelGGL((decode_mfma_kernel<8, 4, U>), grid, block, 0, s, a);
  else if (bs == 8 && g == 8) hipLaunchKernelGGL((decode_mfma_kernel<8, 8, U>), grid, block, 0, s, a);
  else if (bs == 16 && g == 4) hipLaunchKernelGGL((decode_mfma_kernel<16, 4, U>), grid, block, 0, s, a);
  else if (bs == 16 && g == 8) hipLaunchKernelGGL((decode_mfma_kernel<16, 8, U>), grid, block, 0, s, a);
  else if (bs == 32 && g == 4) hipLaunchKernelGGL((decode_mfma_kernel<32, 4, U>), grid, block, 0, s, a);
  else if (bs == 32 && g == 8) hipLaunchKernelGGL((decode_mfma_kernel<32, 8, U>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int hd, int bs, int g, int inflight, hipStream_t s) {
  if (hd != 128) return hipErrorInvalidValue;
  if (inflight == 1) return launch_u<1>(a, bs, g, s);
  if (inflight == 2) return launch_u<2>(a, bs, g, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv

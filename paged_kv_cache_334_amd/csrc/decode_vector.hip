// Paged decode attention, vector form: per-lane dot products and cross-lane
// reductions, float32 online softmax.  Used for float32 pools and for small
// query groups, where the grouped q x K tile is too thin for matrix cores.
//
// The kernel follows the block table of one (sequence, kv head, partition) and
// reads each block's tile straight from the pool, so attention covers the
// sequence's keys and values in logical order with no gather step ("PagedAttention
// Explained", "Block Tables and Non-Contiguous Storage").  The running
// max / sum form of softmax is the exact tiling of FlashAttention ("Paged
// Attention" glossary, related term "FlashAttention"; "Master Paged Attention
// for LLM Inference", "Optimizing Further").
//
// Work split.  Workgroup = kWaves waves = one (partition, kv head, sequence).
// Wave w takes the partition's blocks w, w + kWaves, ...  Their ids come in
// with one vector load per 64 of them (lane l holds the id of the wave's l-th
// block) and are broadcast with readlane, so no tile load waits on a table
// lookup.  The wave works in rounds of U blocks, double-buffered: the tile
// loads of round r+1 are issued before round r is computed, so the wave always
// has loads in flight.  Within a round:
//  * key pass: lane = (token t = lane % BS, lane group grp = lane / BS); the
//    lane loads 16-byte chunks grp, grp + 64/BS, ... of token t's key row
//    (the 8, 16 or 32 lanes of one chunk read BS*16 contiguous bytes of the key
//    tile), multiplies with q in float32 (bf16 pairs through the dot2
//    instruction, which returns a float32 sum), and the 64/BS lane groups are
//    summed with xor shuffles;
//  * value pass: the tile is dim-major [D][BS]; lane reads 16-byte chunks
//    lane, lane + 64, ... (fully contiguous per instruction), i.e. X tokens of
//    one dim, and needs the weights of those X tokens, fetched by shuffles
//    from the lanes that computed them.
// Each wave keeps (max, sum, acc) per query head; the waves merge through LDS
// and the workgroup writes the output row (one partition) or a partial.
#include "decode_common.h"

namespace pkv {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <bool BF16, int HD, int BS, int G, int HP, int U>
__global__ __launch_bounds__(64 * kWaves) void decode_vector_kernel(DecodeArgs a) {
  constexpr int R = HP * G;         // query heads of the workgroup: kv heads y*HP .. y*HP+HP-1
  constexpr int NW = kWaves;
  constexpr int ELT = BF16 ? 2 : 4;
  constexpr int X = 16 / ELT;       // elements per 16-byte chunk
  constexpr int NC = HD / X;        // chunks per key row
  constexpr int GK = 64 / BS;       // lane groups per token in the key pass
  constexpr int KC = NC / GK;       // key chunks per lane per block
  constexpr int RC = BS / X;        // chunks per value row
  constexpr int VC = HD * RC / 64;  // value chunks per lane per block
  constexpr int TILE_BYTES = HD * BS * ELT;
  static_assert(NC % GK == 0 && (HD * RC) % 64 == 0 && RC >= 1, "shape");
  static_assert(64 % U == 0, "a round must not straddle two id loads");

  struct Tile {
    uint4 k[HP][KC];
    uint4 v[HP][VC];
  };

  __shared__ float sm_acc[NW][R][HD];
  __shared__ float sm_m[NW][R];
  __shared__ float sm_l[NW][R];
  __shared__ int sm_bad[NW];
  __shared__ int sm_key[kMaxRankSeqs];
  __shared__ int sm_pick[2];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int t = lane % BS;
  const int grp = lane / BS;
  const int tk = (lane % RC) * X;  // first token of this lane's value chunks

  // Issued together before the context length is known: the wave's first
  // block ids (table entries past the sequence's end may be read, never used)
  // and q.
  const SeqPick seq = pick_sequence<BS>(a, sm_key, sm_pick);
  if (seq.skip) return;
  WaveIds wids = wave_ids_begin(a, seq, wave, lane);
  uint32_t qw[R][KC][4];  // the q chunks this lane meets in the key pass (bf16 pairs kept packed)
#pragma unroll
  for (int h = 0; h < R; ++h) {
    const char* qrow =
        reinterpret_cast<const char*>(a.q) + ((int64_t)seq.qrow * a.num_heads + blockIdx.y * R + h) * HD * ELT;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const uint4 w = load16(qrow + (grp + GK * i) * 16);
      qw[h][i][0] = w.x;
      qw[h][i][1] = w.y;
      qw[h][i][2] = w.z;
      qw[h][i][3] = w.w;
    }
  }

  const PartRange r = part_range<BS>(a, seq);
  if (finish_if_empty<R, HD>(a, r)) return;
  const int cnt = wave_block_count(r, wave);  // blocks of this wave
  int bad = wave_ids_check(a, &wids, cnt, lane);

  float m[R], lsum[R], acc[R][VC];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int j = 0; j < VC; ++j) acc[h][j] = 0.f;
  }

  // the HP kv heads of one block are adjacent tiles
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (int64_t)r.kvh * HP * TILE_BYTES;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (int64_t)r.kvh * HP * TILE_BYTES;
  const int64_t block_bytes = (int64_t)a.num_kv_heads * TILE_BYTES;

  // loads of round rnd: the wave's blocks rnd*U .. rnd*U+U-1 (a missing one
  // re-reads the wave's last block, a cache hit, and is not used)
  auto issue = [&](Tile* T, int rnd) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(rnd * U + u, cnt - 1);
      const int64_t off = (int64_t)wave_id_at(a, &wids, i, cnt, lane, &bad) * block_bytes;
      const auto kt = tile_rsrc(kbase + off, HP * TILE_BYTES);
      const auto vt = tile_rsrc(vbase + off, HP * TILE_BYTES);
#pragma unroll
      for (int hp = 0; hp < HP; ++hp) {
#pragma unroll
        for (int c = 0; c < KC; ++c) T[u].k[hp][c] = bload16<kCacheStream>(kt, hp * TILE_BYTES + ((grp + GK * c) * BS + t) * 16);
#pragma unroll
        for (int c = 0; c < VC; ++c) T[u].v[hp][c] = bload16<kCacheStream>(vt, hp * TILE_BYTES + (lane + 64 * c) * 16);
      }
    }
  };

  auto compute = [&](Tile* T, int rnd) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = rnd * U + u;
      if (i >= cnt) break;
      const int valid = r.ctx - (r.blk_lo + wave + NW * i) * BS;  // rows of this block inside the context, >= 1

      // value rows past the context may hold NaN: clear their bits (a zero weight is not enough)
      if (valid < BS) {
#pragma unroll
        for (int hp = 0; hp < HP; ++hp)
#pragma unroll
          for (int c = 0; c < VC; ++c) {
            uint32_t ws[4] = {T[u].v[hp][c].x, T[u].v[hp][c].y, T[u].v[hp][c].z, T[u].v[hp][c].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if constexpr (BF16) {
                if (tk + 2 * e >= valid) ws[e] &= 0xffff0000u;
                if (tk + 2 * e + 1 >= valid) ws[e] &= 0x0000ffffu;
              } else {
                if (tk + e >= valid) ws[e] = 0u;
              }
            }
            T[u].v[hp][c] = make_uint4(ws[0], ws[1], ws[2], ws[3]);
          }
      }

#pragma unroll
      for (int h = 0; h < R; ++h) {
        const int hp = h / G;  // kv head (tile) of query head h
        float s = 0.f, s2 = 0.f;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const uint32_t ws[4] = {T[u].k[hp][c].x, T[u].k[hp][c].y, T[u].k[hp][c].z, T[u].k[hp][c].w};
          if constexpr (BF16) {
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[h][c][e]),
                                                  __builtin_bit_cast(bf16x2, ws[e]), s, false);
              s2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[h][c][e + 1]),
                                                   __builtin_bit_cast(bf16x2, ws[e + 1]), s2, false);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              s = fmaf(__uint_as_float(qw[h][c][e]), __uint_as_float(ws[e]), s);
              s2 = fmaf(__uint_as_float(qw[h][c][e + 1]), __uint_as_float(ws[e + 1]), s2);
            }
          }
        }
        s += s2;
        // sum the lane groups of one token: lanes t, t+BS, ...
        if constexpr (BS == 8) s = sum_xor32(sum_xor16(sum_xor8(s)));
        else if constexpr (BS == 16) s = sum_xor32(sum_xor16(s));
        else s = sum_xor32(s);
        s = (t < valid) ? s * a.scale_log2 : -INFINITY;

        float mx = row_max16(s);  // with 8-token blocks lanes 8..15 repeat tokens 0..7
        if constexpr (BS == 32) mx = max_xor16(mx);
        mx = __builtin_amdgcn_readfirstlane(mx);  // the same in every lane
        if (mx > m[h] + kRescaleSlack) {
          const float alpha = fast_exp2(m[h] - mx);
          lsum[h] *= alpha;
#pragma unroll
          for (int c = 0; c < VC; ++c) acc[h][c] *= alpha;
          m[h] = mx;
        }
        const float p = fast_exp2(s - m[h]);
        lsum[h] += p;
        // weights of the lane's value tokens tk..tk+X-1; token k's weight sits in lane k
        // (and k + BS, ...).  With one or two chunks per value row, scalar broadcasts
        // and a per-lane select replace the LDS permutes.
        float pv[X];
        if constexpr (RC == 1) {
#pragma unroll
          for (int e = 0; e < X; ++e) pv[e] = readlane_f(p, e);
        } else if constexpr (RC == 2) {
          const bool second = lane & 1;  // tk == X
#pragma unroll
          for (int e = 0; e < X; ++e) {
            const float lo = readlane_f(p, e), hi = readlane_f(p, X + e);
            pv[e] = second ? hi : lo;
          }
        } else {
#pragma unroll
          for (int e = 0; e < X; ++e) pv[e] = shfl(p, tk + e);
        }
#pragma unroll
        for (int c = 0; c < VC; ++c) {
          const uint32_t ws[4] = {T[u].v[hp][c].x, T[u].v[hp][c].y, T[u].v[hp][c].z, T[u].v[hp][c].w};
          float racc = acc[h][c];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (BF16) {
              racc = fmaf(pv[2 * e], bf16_lo(ws[e]), racc);
              racc = fmaf(pv[2 * e + 1], bf16_hi(ws[e]), racc);
            } else {
              racc = fmaf(pv[e], __uint_as_float(ws[e]), racc);
            }
          }
          acc[h][c] = racc;
        }
      }
    }
  };

  Tile ta[U], tb[U];
  pipelined_rounds((cnt + U - 1) / U, ta, tb, issue, compute);

  // wave totals: the weight sum over the tokens of lane group 0 (every group
  // holds the same weights), and the RC lanes sharing a dim add their partial sums
#pragma unroll
  for (int h = 0; h < R; ++h) {
    float l = BS == 8 ? row_sum8(lsum[h]) : row_sum16(lsum[h]);
    if constexpr (BS == 32) l = sum_xor16(l);
#pragma unroll
    for (int c = 0; c < VC; ++c) {
      float racc = acc[h][c];
#pragma unroll
      for (int off = 1; off < RC; off <<= 1) racc += shfl_xor(racc, off);
      if (lane % RC == 0) sm_acc[wave][h][(lane + 64 * c) / RC] = racc;
    }
    if (lane == 0) {
      sm_m[wave][h] = m[h];
      sm_l[wave][h] = l;
    }
  }
  if (lane == 0) sm_bad[wave] = bad;
  __syncthreads();
  merge_waves_and_store<R, HD, NW>(a, r, sm_acc, sm_m, sm_l, sm_bad);
}

bool vector_supported(int bf16, int hd, int bs, int g) {
  (void)bf16;
  return (hd == 64 || hd == 128) && (bs == 8 || bs == 16 || bs == 32) && (g == 1 || g == 2 || g == 4 || g == 8);
}

// sequence slots: one per sequence, or one per (sequence, new token) with several
static unsigned seq_slots(const DecodeArgs& a) {
  return a.query_start ? (unsigned)a.num_seqs * a.max_query_len : (unsigned)a.num_seqs;
}

template <bool BF16, int HD, int BS, int HP, int U>
static hipError_t dispatch_g(const DecodeArgs& a, int g, hipStream_t s) {
  const dim3 grid(a.num_parts, a.num_kv_heads / HP, seq_slots(a));
  const dim3 block(64 * kWaves);
  switch (g) {
    case 1: hipLaunchKernelGGL((decode_vector_kernel<BF16, HD, BS, 1, HP, U>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_vector_kernel<BF16, HD, BS, 2, HP, U>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_vector_kernel<BF16, HD, BS, 4, HP, U>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_vector_kernel<BF16, HD, BS, 8, HP, U>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, int HP, int U>
static hipError_t dispatch_shape(const DecodeArgs& a, int hd, int bs, int g, hipStream_t s) {
  if (hd == 64 && bs == 8) return dispatch_g<BF16, 64, 8, HP, U>(a, g, s);
  if (hd == 128 && bs == 8) return dispatch_g<BF16, 128, 8, HP, U>(a, g, s);
  if (hd == 64 && bs == 16) return dispatch_g<BF16, 64, 16, HP, U>(a, g, s);
  if (hd == 64 && bs == 32) return dispatch_g<BF16, 64, 32, HP, U>(a, g, s);
  if (hd == 128 && bs == 16) return dispatch_g<BF16, 128, 16, HP, U>(a, g, s);
  if (hd == 128 && bs == 32) return dispatch_g<BF16, 128, 32, HP, U>(a, g, s);
  return hipErrorInvalidValue;
}

// two kv heads per workgroup (single-query groups only: their registers then
// match a group of two); grid y runs over kv-head pairs
template <bool BF16, int U>
static hipError_t dispatch_pairs(const DecodeArgs& a, int hd, int bs, hipStream_t s) {
  const dim3 grid(a.num_parts, a.num_kv_heads / 2, seq_slots(a));
  const dim3 block(64 * kWaves);
  if (hd == 64 && bs == 8) hipLaunchKernelGGL((decode_vector_kernel<BF16, 64, 8, 1, 2, U>), grid, block, 0, s, a);
  else if (hd == 128 && bs == 8) hipLaunchKernelGGL((decode_vector_kernel<BF16, 128, 8, 1, 2, U>), grid, block, 0, s, a);
  else if (hd == 64 && bs == 16) hipLaunchKernelGGL((decode_vector_kernel<BF16, 64, 16, 1, 2, U>), grid, block, 0, s, a);
  else if (hd == 64 && bs == 32) hipLaunchKernelGGL((decode_vector_kernel<BF16, 64, 32, 1, 2, U>), grid, block, 0, s, a);
  else if (hd == 128 && bs == 16) hipLaunchKernelGGL((decode_vector_kernel<BF16, 128, 16, 1, 2, U>), grid, block, 0, s, a);
  else if (hd == 128 && bs == 32) hipLaunchKernelGGL((decode_vector_kernel<BF16, 128, 32, 1, 2, U>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_vector(const DecodeArgs& a, int bf16, int hd, int bs, int g, int inflight,
                                int heads_per_wg, hipStream_t s) {
  if (heads_per_wg == 2) {
    if (g != 1 || a.num_kv_heads % 2 || inflight != 1) return hipErrorInvalidValue;
    return bf16 ? dispatch_pairs<true, 1>(a, hd, bs, s) : dispatch_pairs<false, 1>(a, hd, bs, s);
  }
  if (heads_per_wg != 1) return hipErrorInvalidValue;
  if (inflight == 1) return bf16 ? dispatch_shape<true, 1, 1>(a, hd, bs, g, s) : dispatch_shape<false, 1, 1>(a, hd, bs, g, s);
  if (inflight == 2) return bf16 ? dispatch_shape<true, 1, 2>(a, hd, bs, g, s) : dispatch_shape<false, 1, 2>(a, hd, bs, g, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv

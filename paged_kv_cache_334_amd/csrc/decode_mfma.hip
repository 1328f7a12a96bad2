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
#include "common.h"
#include "kernels.h"

namespace pkv {

template <int BS, int G>
__global__ __launch_bounds__(64 * kWaves) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NW = kWaves;
  constexpr int HD = 128;
  constexpr int TILE_ELEMS = HD * BS;
  static_assert(2 * G <= 16, "group too large for one 16-column tile");

  __shared__ float sm_acc[NW][G][HD];
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  __shared__ int sm_bad[NW];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int ctx_raw = a.context_lens[b];
  const bool ctx_bad = ctx_raw < 0 || ctx_raw > a.max_context;  // broken precondition: NaN rows, no reads
  const int ctx = ctx_bad ? 0 : ctx_raw;
  const int nblocks = (ctx + BS - 1) / BS;
  const int nparts = (nblocks + a.blocks_per_part - 1) / a.blocks_per_part;
  const int h0 = kvh * G;

  if (part >= nparts) {
    if (part == 0) {  // empty context: the output row is zero (NaN for a broken context length)
      for (int idx = threadIdx.x; idx < G * HD; idx += 64 * NW) {
        const int64_t o = ((int64_t)b * a.num_heads + h0 + idx / HD) * HD + idx % HD;
        if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o] = ctx_bad ? 0x7fc0 : 0;
        else reinterpret_cast<float*>(a.out)[o] = ctx_bad ? NAN : 0.f;
      }
    }
    return;
  }
  const int blk_lo = part * a.blocks_per_part;
  const int blk_hi = min(nblocks, blk_lo + a.blocks_per_part);

  const int n = lane & 15;   // MFMA column: head slot (S^T, O^T) / row: token (K) or dim (V)
  const int kg = lane >> 4;  // lane group
  const bool used = n < 2 * G;
  const bool lo_slot = n >= G;
  const int hslot = n % G;

  bf16x8 qb[4];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.num_heads + h0 + hslot) * HD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 w = used ? load16(qrow + 32 * i + 8 * kg) : make_uint4(0, 0, 0, 0);
      qb[i] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x4 o[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;
  int bad = 0;

  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;
  for (int j = blk_lo + wave; j < blk_hi; j += NW) {
    const int blk = uniform(bt[j]);
    if ((unsigned)blk >= (unsigned)a.num_blocks) {
      bad = 1;
      continue;
    }
    const int64_t tile = ((int64_t)blk * a.num_kv_heads + kvh) * TILE_ELEMS;
    const uint16_t* kt = reinterpret_cast<const uint16_t*>(a.k_pool) + tile;
    const uint16_t* vt = reinterpret_cast<const uint16_t*>(a.v_pool) + tile;
#pragma unroll
    for (int half = 0; half < BS / 16; ++half) {
      const int t0 = half * 16;
      const int valid = ctx - j * BS - t0;
      if (valid <= 0) break;
      uint4 kr[4];
      uint2 vr[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) kr[i] = load16(kt + ((4 * i + kg) * BS + t0 + n) * 8);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) vr[nt] = load8(vt + (16 * nt + n) * BS + t0 + 4 * kg);

      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[i]), qb[i], s, 0, 0, 0);

      float sr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sr[r] = (4 * kg + r < valid) ? s[r] * a.scale_log2 : -INFINITY;
      float mx = fmaxf(fmaxf(sr[0], sr[1]), fmaxf(sr[2], sr[3]));
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx);
      const float alpha = fast_exp2(m - mn);
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(sr[r] - mn);
      lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
      m = mn;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) o[nt] *= alpha;

      uint32_t pw[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        uint32_t half2[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float pr = p[2 * e + k];
          const uint32_t hi = f32_to_bf16_rne(pr);
          const uint32_t lo = f32_to_bf16_rne(pr - __uint_as_float(hi << 16));
          half2[k] = used ? (lo_slot ? lo : hi) : 0u;
        }
        pw[e] = half2[0] | (half2[1] << 16);
      }
      const s16x4 pb = __builtin_bit_cast(s16x4, make_uint2(pw[0], pw[1]));

      if (valid < 16) {  // rows past the context may hold NaN: zero them, a zero weight is not enough
        const int first = 4 * kg;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          uint32_t w0 = vr[nt].x, w1 = vr[nt].y;
          if (first + 0 >= valid) w0 &= 0xffff0000u;
          if (first + 1 >= valid) w0 &= 0x0000ffffu;
          if (first + 2 >= valid) w1 &= 0xffff0000u;
          if (first + 3 >= valid) w1 &= 0x0000ffffu;
          vr[nt] = make_uint2(w0, w1);
        }
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vr[nt]), pb, o[nt], 0, 0, 0);
    }
  }

  // wave totals: weight sum over the 4 lane groups; hi + lo columns of each head
  float l = lsum + shfl_xor(lsum, 16);
  l += shfl_xor(l, 32);
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float other = shfl(o[nt][r], (lane + G) & 63);
      if (n < G) sm_acc[wave][n][16 * nt + 4 * kg + r] = o[nt][r] + other;
    }
  }
  if (kg == 0 && n < G) {
    sm_m[wave][n] = m;
    sm_l[wave][n] = l;
  }
  if (lane == 0) sm_bad[wave] = bad;
  __syncthreads();

  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) any_bad |= sm_bad[w];
  for (int idx = threadIdx.x; idx < G * HD; idx += 64 * NW) {
    const int h = idx / HD, d = idx % HD;
    float big_m = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) big_m = fmaxf(big_m, sm_m[w][h]);
    float lt = 0.f, r = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = (sm_m[w][h] == -INFINITY) ? 0.f : fast_exp2(sm_m[w][h] - big_m);
      lt = fmaf(f, sm_l[w][h], lt);
      r = fmaf(f, sm_acc[w][h][d], r);
    }
    if (any_bad) {
      big_m = NAN;
      r = NAN;
    }
    const int hq = h0 + h;
    if (nparts == 1) {
      const float ov = r / lt;
      const int64_t oi = ((int64_t)b * a.num_heads + hq) * HD + d;
      if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_rne(ov);
      else reinterpret_cast<float*>(a.out)[oi] = ov;
    } else {
      const int64_t pi = ((int64_t)b * a.num_heads + hq) * a.num_parts + part;
      a.ws_acc[pi * HD + d] = r;
      if (d == 0) {
        a.ws_m[pi] = big_m;
        a.ws_l[pi] = lt;
      }
    }
  }
}

bool mfma_supported(int bf16, int hd, int bs, int g) {
  return bf16 && hd == 128 && (bs == 16 || bs == 32) && (g == 4 || g == 8);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int hd, int bs, int g, hipStream_t s) {
  if (hd != 128) return hipErrorInvalidValue;
  const dim3 grid(a.num_parts, a.num_kv_heads, a.num_seqs);
  const dim3 block(64 * kWaves);
  if (bs == 16 && g == 4) hipLaunchKernelGGL((decode_mfma_kernel<16, 4>), grid, block, 0, s, a);
  else if (bs == 16 && g == 8) hipLaunchKernelGGL((decode_mfma_kernel<16, 8>), grid, block, 0, s, a);
  else if (bs == 32 && g == 4) hipLaunchKernelGGL((decode_mfma_kernel<32, 4>), grid, block, 0, s, a);
  else if (bs == 32 && g == 8) hipLaunchKernelGGL((decode_mfma_kernel<32, 8>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv

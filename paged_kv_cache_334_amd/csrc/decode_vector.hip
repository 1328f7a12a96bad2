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
// Wave w takes blocks blk_lo + w, blk_lo + w + kWaves, ...  Within a wave:
//  * key pass: lane = (token t = lane % BS, lane group grp = lane / BS); the
//    lane loads 16-byte chunks grp, grp + 64/BS, ... of token t's key row
//    (each chunk is BS*16 bytes away from the next in the key tile, and the
//    16 or 32 lanes of one chunk read BS*16 contiguous bytes), multiplies with
//    q in float32, and the 64/BS lane groups are summed with xor shuffles;
//  * value pass: the tile is dim-major [D][BS]; lane reads 16-byte chunks
//    lane, lane + 64, ... (fully contiguous per instruction), i.e. X tokens of
//    one dim, and needs the weights of those X tokens, fetched by shuffles
//    from the lanes that computed them.
// Each wave keeps (max, sum, acc) per query head; the waves merge through LDS
// and the workgroup writes the output row (one partition) or a partial.
#include "common.h"
#include "kernels.h"

namespace pkv {

template <bool BF16, int HD, int BS, int G>
__global__ __launch_bounds__(64 * kWaves) void decode_vector_kernel(DecodeArgs a) {
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

  const int t = lane % BS;
  const int grp = lane / BS;
  const int tk = (lane % RC) * X;  // first token of this lane's value chunks

  // q in float32, the chunks this lane meets in the key pass
  float qf[G][KC][X];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const char* qrow = reinterpret_cast<const char*>(a.q) + ((int64_t)b * a.num_heads + h0 + h) * HD * ELT;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const uint4 w = load16(qrow + (grp + GK * i) * 16);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      if constexpr (BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qf[h][i][2 * e] = bf16_lo(ws[e]);
          qf[h][i][2 * e + 1] = bf16_hi(ws[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[h][i][e] = __uint_as_float(ws[e]);
      }
    }
  }

  float m[G], lsum[G], acc[G][VC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int j = 0; j < VC; ++j) acc[h][j] = 0.f;
  }
  int bad = 0;

  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;
  for (int j = blk_lo + wave; j < blk_hi; j += NW) {
    const int blk = uniform(bt[j]);
    if ((unsigned)blk >= (unsigned)a.num_blocks) {
      bad = 1;
      continue;
    }
    const int64_t tile = ((int64_t)blk * a.num_kv_heads + kvh) * TILE_BYTES;
    const char* kt = reinterpret_cast<const char*>(a.k_pool) + tile;
    const char* vt = reinterpret_cast<const char*>(a.v_pool) + tile;
    uint4 kr[KC], vr[VC];
#pragma unroll
    for (int i = 0; i < KC; ++i) kr[i] = load16(kt + ((grp + GK * i) * BS + t) * 16);
#pragma unroll
    for (int jv = 0; jv < VC; ++jv) vr[jv] = load16(vt + (lane + 64 * jv) * 16);
    const int valid = ctx - j * BS;  // rows of this block inside the context, >= 1

    // value elements as float32, with rows past the context set to 0 (they may hold NaN)
    float vf[VC][X];
#pragma unroll
    for (int jv = 0; jv < VC; ++jv) {
      const uint32_t ws[4] = {vr[jv].x, vr[jv].y, vr[jv].z, vr[jv].w};
      if constexpr (BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[jv][2 * e] = bf16_lo(ws[e]);
          vf[jv][2 * e + 1] = bf16_hi(ws[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) vf[jv][e] = __uint_as_float(ws[e]);
      }
    }
    if (valid < BS) {
#pragma unroll
      for (int jv = 0; jv < VC; ++jv)
#pragma unroll
        for (int e = 0; e < X; ++e) vf[jv][e] = (tk + e < valid) ? vf[jv][e] : 0.f;
    }

#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const uint32_t ws[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
        if constexpr (BF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s = fmaf(qf[h][i][2 * e], bf16_lo(ws[e]), s);
            s = fmaf(qf[h][i][2 * e + 1], bf16_hi(ws[e]), s);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) s = fmaf(qf[h][i][e], __uint_as_float(ws[e]), s);
        }
      }
#pragma unroll
      for (int off = BS; off < 64; off <<= 1) s += shfl_xor(s, off);
      s = (t < valid) ? s * a.scale_log2 : -INFINITY;

      float mx = s;
#pragma unroll
      for (int off = 1; off < BS; off <<= 1) mx = fmaxf(mx, shfl_xor(mx, off));
      const float mn = fmaxf(m[h], mx);
      const float alpha = fast_exp2(m[h] - mn);
      const float p = fast_exp2(s - mn);
      lsum[h] = lsum[h] * alpha + p;
      m[h] = mn;
      float pv[X];
#pragma unroll
      for (int e = 0; e < X; ++e) pv[e] = shfl(p, tk + e);
#pragma unroll
      for (int jv = 0; jv < VC; ++jv) {
        float r = acc[h][jv] * alpha;
#pragma unroll
        for (int e = 0; e < X; ++e) r = fmaf(pv[e], vf[jv][e], r);
        acc[h][jv] = r;
      }
    }
  }

  // wave totals: sum over the BS token lanes and over the RC lanes sharing a dim
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float l = lsum[h];
#pragma unroll
    for (int off = 1; off < BS; off <<= 1) l += shfl_xor(l, off);
#pragma unroll
    for (int jv = 0; jv < VC; ++jv) {
      float r = acc[h][jv];
#pragma unroll
      for (int off = 1; off < RC; off <<= 1) r += shfl_xor(r, off);
      if (lane % RC == 0) sm_acc[wave][h][(lane + 64 * jv) / RC] = r;
    }
    if (lane == 0) {
      sm_m[wave][h] = m[h];
      sm_l[wave][h] = l;
    }
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
    float l = 0.f, r = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = (sm_m[w][h] == -INFINITY) ? 0.f : fast_exp2(sm_m[w][h] - big_m);
      l = fmaf(f, sm_l[w][h], l);
      r = fmaf(f, sm_acc[w][h][d], r);
    }
    if (any_bad) {
      big_m = NAN;
      r = NAN;
    }
    const int hq = h0 + h;
    if (nparts == 1) {
      const float o = r / l;
      const int64_t oi = ((int64_t)b * a.num_heads + hq) * HD + d;
      if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_rne(o);
      else reinterpret_cast<float*>(a.out)[oi] = o;
    } else {
      const int64_t pi = ((int64_t)b * a.num_heads + hq) * a.num_parts + part;
      a.ws_acc[pi * HD + d] = r;
      if (d == 0) {
        a.ws_m[pi] = big_m;
        a.ws_l[pi] = l;
      }
    }
  }
}

bool vector_supported(int bf16, int hd, int bs, int g) {
  (void)bf16;
  return (hd == 64 || hd == 128) && (bs == 16 || bs == 32) && (g == 1 || g == 2 || g == 4 || g == 8);
}

template <bool BF16, int HD, int BS>
static hipError_t dispatch_g(const DecodeArgs& a, int g, hipStream_t s) {
  const dim3 grid(a.num_parts, a.num_kv_heads, a.num_seqs);
  const dim3 block(64 * kWaves);
  switch (g) {
    case 1: hipLaunchKernelGGL((decode_vector_kernel<BF16, HD, BS, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_vector_kernel<BF16, HD, BS, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_vector_kernel<BF16, HD, BS, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_vector_kernel<BF16, HD, BS, 8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16>
static hipError_t dispatch_shape(const DecodeArgs& a, int hd, int bs, int g, hipStream_t s) {
  if (hd == 64 && bs == 16) return dispatch_g<BF16, 64, 16>(a, g, s);
  if (hd == 64 && bs == 32) return dispatch_g<BF16, 64, 32>(a, g, s);
  if (hd == 128 && bs == 16) return dispatch_g<BF16, 128, 16>(a, g, s);
  if (hd == 128 && bs == 32) return dispatch_g<BF16, 128, 32>(a, g, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_vector(const DecodeArgs& a, int bf16, int hd, int bs, int g, hipStream_t s) {
  return bf16 ? dispatch_shape<true>(a, hd, bs, g, s) : dispatch_shape<false>(a, hd, bs, g, s);
}

}  // namespace pkv

// Split-K merge: combine the per-partition partials (m_p, l_p, acc_p) of one
// (sequence, query head) into the output row,
//     M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// (logits are kept in base 2).  The max rescaling keeps a partition whose
// logits are far larger than the others' (outlier keys) from overflowing and
// the others from being flushed before the comparison.  Sequences that fit in
// one partition were written directly by the partition kernel and are skipped.
#include "common.h"
#include "kernels.h"

namespace pkv {

template <int HD>
__global__ __launch_bounds__(HD) void splitk_reduce_kernel(DecodeArgs a, int block_size) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int ctx_raw = a.context_lens[b];
  const int ctx = (ctx_raw < 0 || ctx_raw > a.max_context) ? 0 : ctx_raw;  // the partition kernel wrote NaN
  const int nblocks = (ctx + block_size - 1) / block_size;
  const int nparts = (nblocks + a.blocks_per_part - 1) / a.blocks_per_part;
  if (nparts <= 1) return;
  const int64_t base = ((int64_t)b * a.num_heads + h) * a.num_parts;
  float big_m = -INFINITY;
  for (int p = 0; p < nparts; ++p) big_m = fmaxf(big_m, a.ws_m[base + p]);
  float l = 0.f, r = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float f = fast_exp2(a.ws_m[base + p] - big_m);
    l = fmaf(f, a.ws_l[base + p], l);
    r = fmaf(f, a.ws_acc[(base + p) * HD + d], r);
  }
  const float o = r / l;
  const int64_t oi = ((int64_t)b * a.num_heads + h) * HD + d;
  if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[oi] = (uint16_t)f32_to_bf16_rne(o);
  else reinterpret_cast<float*>(a.out)[oi] = o;
}

// The same merge with several new tokens per sequence: grid (query head, new
// token i, sequence b).  A row's partitions are those of its row tile, which
// walks the tokens the tile's last row sees; both kernels that write the
// partials (matrix-core tiles of rows_per_tile rows, vector workgroups of one
// token's G rows) use that rule.
template <int HD>
__global__ __launch_bounds__(HD) void multi_reduce_kernel(DecodeArgs a, int block_size, int group) {
  const int h = blockIdx.x;
  const int i = blockIdx.y;
  const int b = blockIdx.z;
  const int d = threadIdx.x;
  const int qs = a.query_start[b], qe = a.query_start[b + 1];
  if (qs < 0 || qs > qe || qe > a.num_query_tokens) return;
  const int qlen = qe - qs;
  const int covered = min(qlen, a.max_query_len);
  if (i >= covered) return;
  const int ctx_raw = a.context_lens[b];
  if (ctx_raw < qlen || ctx_raw > a.max_context || qlen > a.max_query_len) return;  // NaN rows already written
  const int row = i * group + h % group;
  const int r_end = min((row / a.rows_per_tile + 1) * a.rows_per_tile, covered * group);
  const int ctx = ctx_raw - qlen + 1 + (r_end - 1) / group;
  const int nblocks = (ctx + block_size - 1) / block_size;
  const int nparts = (nblocks + a.blocks_per_part - 1) / a.blocks_per_part;
  if (nparts <= 1) return;
  const int64_t hrow = (int64_t)(qs + i) * a.num_heads + h;
  const int64_t base = hrow * a.num_parts;
  float big_m = -INFINITY;
  for (int p = 0; p < nparts; ++p) big_m = fmaxf(big_m, a.ws_m[base + p]);
  float l = 0.f, r = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float mp = a.ws_m[base + p];
    const float f = mp == -INFINITY ? 0.f : fast_exp2(mp - big_m);  // a partition the row sees nothing of
    l = fmaf(f, a.ws_l[base + p], l);
    r = fmaf(f, a.ws_acc[(base + p) * HD + d], r);
  }
  const float o = r / l;
  if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[hrow * HD + d] = (uint16_t)f32_to_bf16_rne(o);
  else reinterpret_cast<float*>(a.out)[hrow * HD + d] = o;
}

hipError_t launch_multi_reduce(const DecodeArgs& a, int hd, int bs, int group, hipStream_t s) {
  const dim3 grid(a.num_heads, a.max_query_len, a.num_seqs);
  if (hd == 64) hipLaunchKernelGGL((multi_reduce_kernel<64>), grid, dim3(64), 0, s, a, bs, group);
  else if (hd == 128) hipLaunchKernelGGL((multi_reduce_kernel<128>), grid, dim3(128), 0, s, a, bs, group);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const DecodeArgs& a, int hd, int bs, hipStream_t s) {
  const dim3 grid(a.num_heads, a.num_seqs);
  if (hd == 64) hipLaunchKernelGGL((splitk_reduce_kernel<64>), grid, dim3(64), 0, s, a, bs);
  else if (hd == 128) hipLaunchKernelGGL((splitk_reduce_kernel<128>), grid, dim3(128), 0, s, a, bs);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv

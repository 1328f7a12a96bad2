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

hipError_t launch_splitk_reduce(const DecodeArgs& a, int hd, int bs, hipStream_t s) {
  const dim3 grid(a.num_heads, a.num_seqs);
  if (hd == 64) hipLaunchKernelGGL((splitk_reduce_kernel<64>), grid, dim3(64), 0, s, a, bs);
  else if (hd == 128) hipLaunchKernelGGL((splitk_reduce_kernel<128>), grid, dim3(128), 0, s, a, bs);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv

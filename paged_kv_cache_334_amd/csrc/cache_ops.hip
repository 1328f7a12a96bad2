// Cache write (reshape_and_cache) and copy-on-write block copy (copy_blocks).
//
// reshape_and_cache stores each new token's key and value at its slot
// s = block * block_size + row, the row being the sequence length modulo the
// block size ("PagedAttention Explained", "Implementing a Simplified Paged KV
// Cache", append_token).  copy_blocks duplicates a shared block before a
// sequence writes into it ("Master Paged Attention for LLM Inference", "How
// Paged Attention Works: The Mechanics", item 4).  Both move raw bits.
#include "common.h"
#include "kernels.h"

namespace pkv {

// One thread per (token, kv head, 16-byte chunk of the head's row).  The key
// chunk is stored whole (the key layout keeps 16-byte chunks intact); the value
// tile is dim-major, so the chunk's X elements go to X rows of the tile.
template <int ELT>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(const char* __restrict__ k, const char* __restrict__ v,
                                                                int64_t k_stride, int64_t v_stride,
                                                                const int32_t* __restrict__ slots, int32_t num_tokens,
                                                                char* __restrict__ k_pool, char* __restrict__ v_pool,
                                                                int32_t num_blocks, int32_t hkv, int32_t bs,
                                                                int32_t hd) {
  constexpr int X = 16 / ELT;
  const int nc = hd / X;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)num_tokens * hkv * nc;
  if (idx >= total) return;
  const int c = (int)(idx % nc);
  const int h = (int)((idx / nc) % hkv);
  const int64_t t = idx / ((int64_t)nc * hkv);
  const int32_t slot = slots[t];
  if (slot < 0 || slot >= num_blocks * bs) return;
  const int64_t blk = slot / bs;
  const int row = slot % bs;
  const int64_t tile = (blk * hkv + h) * (int64_t)hd * bs;  // elements
  const uint4 kw = load16(k + (t * k_stride + (int64_t)h * hd + (int64_t)c * X) * ELT);
  const uint4 vw = load16(v + (t * v_stride + (int64_t)h * hd + (int64_t)c * X) * ELT);
  *reinterpret_cast<uint4*>(k_pool + (tile + ((int64_t)c * bs + row) * X) * ELT) = kw;
  const uint32_t vs[4] = {vw.x, vw.y, vw.z, vw.w};
  if constexpr (ELT == 2) {
    uint16_t* vt = reinterpret_cast<uint16_t*>(v_pool) + tile + row;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vt[(int64_t)(c * X + 2 * e) * bs] = (uint16_t)(vs[e] & 0xffffu);
      vt[(int64_t)(c * X + 2 * e + 1) * bs] = (uint16_t)(vs[e] >> 16);
    }
  } else {
    uint32_t* vt = reinterpret_cast<uint32_t*>(v_pool) + tile + row;
#pragma unroll
    for (int e = 0; e < 4; ++e) vt[(int64_t)(c * X + e) * bs] = vs[e];
  }
}

// grid.x = pair, grid.y = slice of the block, grid.z = pool (0 keys, 1 values);
// each thread moves 16-byte chunks.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
                                                          const int32_t* __restrict__ pairs, int32_t num_blocks,
                                                          int64_t chunks_per_block) {
  const int32_t src = pairs[2 * (int64_t)blockIdx.x];
  const int32_t dst = pairs[2 * (int64_t)blockIdx.x + 1];
  if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) return;
  uint4* pool = blockIdx.z ? v_pool : k_pool;
  const uint4* from = pool + src * chunks_per_block;
  uint4* to = pool + dst * chunks_per_block;
  for (int64_t i = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; i < chunks_per_block;
       i += (int64_t)gridDim.y * blockDim.x)
    to[i] = from[i];
}

// Like copy_blocks_kernel between two pools (either may live in pinned host
// memory): grid.x = pair, grid.y = slice of the block, grid.z = keys/values.
__global__ __launch_bounds__(256) void swap_blocks_kernel(const uint4* __restrict__ src_k,
                                                          const uint4* __restrict__ src_v, int32_t src_blocks,
                                                          uint4* __restrict__ dst_k, uint4* __restrict__ dst_v,
                                                          int32_t dst_blocks, const int32_t* __restrict__ pairs,
                                                          int64_t chunks_per_block) {
  const int32_t src = pairs[2 * (int64_t)blockIdx.x];
  const int32_t dst = pairs[2 * (int64_t)blockIdx.x + 1];
  if ((unsigned)src >= (unsigned)src_blocks || (unsigned)dst >= (unsigned)dst_blocks) return;
  const uint4* from = (blockIdx.z ? src_v : src_k) + src * chunks_per_block;
  uint4* to = (blockIdx.z ? dst_v : dst_k) + dst * chunks_per_block;
  for (int64_t i = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; i < chunks_per_block;
       i += (int64_t)gridDim.y * blockDim.x)
    to[i] = from[i];
}

hipError_t launch_swap_blocks(const void* src_k, const void* src_v, int32_t src_blocks, void* dst_k, void* dst_v,
                              int32_t dst_blocks, const int32_t* pairs, int32_t num_pairs, int64_t block_bytes,
                              hipStream_t s) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t chunks = block_bytes / 16;
  const unsigned gy = (unsigned)((chunks + 255) / 256 < 8 ? (chunks + 255) / 256 : 8);
  hipLaunchKernelGGL(swap_blocks_kernel, dim3((unsigned)num_pairs, gy, 2), dim3(256), 0, s, (const uint4*)src_k,
                     (const uint4*)src_v, src_blocks, (uint4*)dst_k, (uint4*)dst_v, dst_blocks, pairs, chunks);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* k, const void* v, int64_t k_stride, int64_t v_stride,
                                    const int32_t* slots, int32_t num_tokens, void* k_pool, void* v_pool,
                                    int32_t num_blocks, int32_t hkv, int32_t bs, int32_t hd, int32_t elt,
                                    hipStream_t s) {
  const int x = 16 / elt;
  const int64_t total = (int64_t)num_tokens * hkv * (hd / x);
  const int64_t blocks = (total + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (elt == 2)
    hipLaunchKernelGGL(reshape_and_cache_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, (const char*)k,
                       (const char*)v, k_stride, v_stride, slots, num_tokens, (char*)k_pool, (char*)v_pool,
                       num_blocks, hkv, bs, hd);
  else
    hipLaunchKernelGGL(reshape_and_cache_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, (const char*)k,
                       (const char*)v, k_stride, v_stride, slots, num_tokens, (char*)k_pool, (char*)v_pool,
                       num_blocks, hkv, bs, hd);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int32_t num_pairs,
                              int32_t num_blocks, int64_t block_bytes, hipStream_t s) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t chunks = block_bytes / 16;
  const unsigned gy = (unsigned)((chunks + 255) / 256 < 8 ? (chunks + 255) / 256 : 8);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs, gy, 2), dim3(256), 0, s, (uint4*)k_pool,
                     (uint4*)v_pool, pairs, num_blocks, chunks);
  return hipGetLastError();
}

}  // namespace pkv

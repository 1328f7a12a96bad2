// Measurement kernels: a streaming read, a tile gather and a plain copy.  They
// are not part of paged attention; they give the bandwidth a kernel on this
// device can reach (the ceiling the decode kernels are compared with) and a
// copy of known size against which the hardware byte counters are scaled.
#include <hip/hip_runtime.h>

#include "../../include/pkv_probe.h"
#include "common.h"

namespace pkv {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per thread

// Every thread folds the words it read into one value; one word per workgroup
// is stored so the loads cannot be dropped.
__device__ __forceinline__ uint32_t fold(uint4 w) { return w.x ^ w.y ^ w.z ^ w.w; }

// Each wave streams whole 8 KiB pieces (kProbeUnroll loads of 1 KiB each in
// flight), pieces dealt to the waves of the grid round-robin.  Reads use the
// streaming cache policy (faster for data read once: 7.0 against 6.25 TB/s).
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* __restrict__ src, int64_t chunks,
                                                                   uint32_t* __restrict__ sink) {
  constexpr int PIECE = 64 * kProbeUnroll;  // 16-byte chunks per wave piece
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (kProbeThreads / 64);
  uint32_t acc = 0;
  for (int64_t piece = (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6); piece * PIECE < chunks;
       piece += waves) {
    const int64_t base = piece * PIECE + lane;
    if (base + (kProbeUnroll - 1) * 64 < chunks) {
      // buffer loads over the piece with the streaming policy, as the decode kernels read their tiles
      const auto r = tile_rsrc(src + piece * PIECE, PIECE * 16);
      uint4 w[kProbeUnroll];
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) w[u] = bload16<kCacheStream>(r, (u * 64 + lane) * 16);
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) acc ^= fold(w[u]);
    } else {
      for (int64_t i = base; i < chunks; i += 64) acc ^= fold(src[i]);
    }
  }
  __shared__ uint32_t red[kProbeThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < kProbeThreads; ++t) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}

// One wave per tile listed in ids: the wave reads tile_bytes at ids[i]*tile_bytes.
__global__ __launch_bounds__(kProbeThreads) void probe_gather_kernel(const char* __restrict__ pool,
                                                                     const int32_t* __restrict__ ids, int32_t n_ids,
                                                                     int32_t tile_bytes, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int waves = kProbeThreads / 64;
  const int chunks = tile_bytes / 16;
  uint32_t acc = 0;
  for (int64_t t = (int64_t)blockIdx.x * waves + (threadIdx.x >> 6); t < n_ids; t += (int64_t)gridDim.x * waves) {
    const auto r = tile_rsrc(pool + (int64_t)ids[t] * tile_bytes, tile_bytes);
    for (int c = lane; c < chunks; c += 64) acc ^= fold(bload16<kCacheStream>(r, c * 16));
  }
  __shared__ uint32_t red[kProbeThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < kProbeThreads; ++t) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const uint4* __restrict__ src,
                                                                   uint4* __restrict__ dst, int64_t chunks) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  for (int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < chunks; i += stride) dst[i] = src[i];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace pkv

extern "C" {

int32_t pkv_probe_read(const void* src, size_t bytes, uint32_t* sink, int32_t num_workgroups, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || !pkv::aligned16(src) || num_workgroups <= 0) return 1;
  hipLaunchKernelGGL(pkv::probe_read_kernel, dim3(num_workgroups), dim3(pkv::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int32_t pkv_probe_gather(const void* pool, const int32_t* tile_ids, int32_t num_ids, int32_t tile_bytes,
                         uint32_t* sink, int32_t num_workgroups, void* stream) {
  if (!pool || !tile_ids || !sink || num_ids <= 0 || tile_bytes <= 0 || tile_bytes % 16 || !pkv::aligned16(pool) ||
      num_workgroups <= 0)
    return 1;
  hipLaunchKernelGGL(pkv::probe_gather_kernel, dim3(num_workgroups), dim3(pkv::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(pool), tile_ids, num_ids, tile_bytes,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int32_t pkv_probe_copy(const void* src, void* dst, size_t bytes, int32_t num_workgroups, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 || !pkv::aligned16(src) || !pkv::aligned16(dst) ||
      num_workgroups <= 0)
    return 1;
  hipLaunchKernelGGL(pkv::probe_copy_kernel, dim3(num_workgroups), dim3(pkv::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), static_cast<uint4*>(dst),
                     (int64_t)(bytes / 16));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"

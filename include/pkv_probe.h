/*
 * pkv_probe.h -- measurement kernels shipped in libpkv beside the paged-attention
 * calls.  They compute nothing of the method: they measure what this device
 * gives a plain kernel, so that the decode kernels can be rated against it.
 *
 *  - pkv_probe_read: stream `bytes` from `src` once (plain 16-byte
 *    loads, several in flight per thread); the achievable HBM read rate.
 *  - pkv_probe_gather: read `num_ids` tiles of `tile_bytes` each at
 *    pool + tile_ids[i]*tile_bytes, one wave per tile; the rate of the same
 *    scattered-tile access a paged KV pool sees, without any arithmetic.
 *  - pkv_probe_copy: copy `bytes` from `src` to `dst`; a transfer of known
 *    size for scaling the hardware fetch/write byte counters.
 *
 * All pointers are DEVICE pointers owned by the caller, 16-byte aligned; sizes
 * are multiples of 16.  `sink` receives one 32-bit word per workgroup
 * (num_workgroups words) so the loads are not optimised away; its contents are
 * meaningless.  `stream` is a hipStream_t.  Return 0 on success, 1 for a bad
 * argument (nothing launched), 4 when the launch failed.  Tile ids are trusted:
 * each must lie inside the pool.
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t pkv_probe_read(const void* src, size_t bytes, uint32_t* sink, int32_t num_workgroups, void* stream);
int32_t pkv_probe_gather(const void* pool, const int32_t* tile_ids, int32_t num_ids, int32_t tile_bytes,
                         uint32_t* sink, int32_t num_workgroups, void* stream);
int32_t pkv_probe_copy(const void* src, void* dst, size_t bytes, int32_t num_workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */

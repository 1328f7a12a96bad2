// Device-side helpers shared by the gfx950 kernels of libpkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Online softmax with a lazily moved reference: the running reference m only
// moves when a new logit exceeds it by more than this many powers of two.
// Weights 2^(s - m) then stay below 2^8 (no overflow risk in float32), and
// the accumulators are rescaled a handful of times per sequence instead of
// once per tile.  The result is the same up to rounding: numerator and
// denominator are both taken relative to the same m.
constexpr float kRescaleSlack = 8.0f;

// Bits of a bfloat16 -> float32 (exact: a bfloat16 is the top half of a float32).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// float32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two float32 -> packed bfloat16 (a in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
// Weights for the bf16 matrix cores as hi + lo parts: hi = bf16(p), lo =
// bf16(p - hi); hi + lo keeps about 16 significant bits of p.
__device__ __forceinline__ void split_bf16(float a, float b, uint32_t* hi, uint32_t* lo) {
  const uint32_t h = pack_bf16(a, b);
  *hi = h;
  *lo = pack_bf16(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
}

// Wave-wide uniform value (the compiler keeps it in an SGPR).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ float shfl(float v, int src) { return __shfl(v, src, 64); }
// v of lane `src` (a constant) in every lane, through a scalar register
__device__ __forceinline__ float readlane_f(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// Cross-lane reductions without LDS.  Within a row of 16 lanes: DPP quad
// permutes (xor 1, xor 2), then the half-row and row mirrors, which pair each
// lane with one holding the other half once the smaller groups agree.  Across
// rows: the gfx950 row-swap instructions; swapping a value with itself and
// combining the two results combines rows r and r^1 (16-lane swap) or the two
// halves of the wave (32-lane swap).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_amdgcn_update_dpp(0.0f, v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within each 16
constexpr int kDppRor8 = 0x128;       // row_ror:8, lane i <-> i^8 within each 16

__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}
// sum over each group of 8 lanes
__device__ __forceinline__ float row_sum8(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  return v;
}
// v(lane) + v(lane ^ 8)
__device__ __forceinline__ float sum_xor8(float v) { return v + dpp<kDppRor8>(v); }
// v(lane) + v(lane ^ 16)
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// v(lane) + v(lane ^ 32)
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// NaN-propagating maximum (v_maximum3_f32 on gfx950).  fmaxf must quiet a
// signalling NaN input first, which costs one extra instruction per operand
// that the compiler cannot prove canonical (every matrix-core result).  Used
// where masked logits are already -inf, so a NaN can only come from the data
// itself, and then the output row is NaN either way.
__device__ __forceinline__ float maxp(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float maxp_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return maxp(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float maxp_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return maxp(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Buffer resource over one tile whose base is wave-uniform (kept in scalar
// registers): the per-lane offsets stay the same 32-bit values for every tile,
// and a load past `bytes` returns zeros instead of leaving the tile.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit dword access, no format conversion

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}
// Cache policy of a buffer load: kCacheDefault, or kCacheStream (the
// non-temporal hint) for data read once.  Measured on MI355X with plain read
// kernels: a streaming read of 2 GiB goes from 6.25 to 7.0 TB/s with the hint,
// a gather of random 4 KiB tiles from 5.98 to 6.75 TB/s.  Data that other
// workgroups read again from L2 keeps the default.
constexpr int kCacheDefault = 0;
constexpr int kCacheStream = 2;

template <int POLICY = kCacheDefault>
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
template <int POLICY = kCacheDefault>
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POLICY);
  return make_uint2(v[0], v[1]);
}

// Loads through a per-lane address with the streaming (non-temporal) hint.
__device__ __forceinline__ uint4 gload16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 gload8_stream(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v[0], v[1]);
}

// Load 16 bytes (one layout chunk).
__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// Load 8 bytes.
__device__ __forceinline__ uint2 load8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

}  // namespace pkv

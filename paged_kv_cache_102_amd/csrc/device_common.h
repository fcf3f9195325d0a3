// Helpers shared by libpagedkv's HIP sources (gfx950): element order inside
// a cache tile, wavefront reductions, operand conversions, buffer
// resources, scalar-cache loads, E4M3 expansion and a few host helpers.
// Everything is internal to each translation unit.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>

#include "pagedkv.h"

namespace {


constexpr int kBlock = PKV_BLOCK_SIZE;
constexpr int kDefaultPartition = 512;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ in-tile order
__host__ __device__ inline int k_elem(int t, int d) { return (d >> 3) * 128 + t * 8 + (d & 7); }
__host__ __device__ inline int v_elem(int t, int d) {
  return (d >> 5) * 512 + (t >> 2) * 128 + (d & 15) * 8 + ((d >> 4) & 1) * 4 + (t & 3);
}

// ------------------------------------------------------------------ wave helpers
// Reductions over the four lanes l, l^16, l^32, l^48 (one per 16-lane row)
// with the gfx950 row-swap permutes: permlane16_swap pairs rows (0,1) and
// (2,3), permlane32_swap pairs rows (0,2) and (1,3); both results of a swap
// hold the two partners, so combining them gives the pair's value in every lane.
// Maximum that propagates NaN (v_maximum3_f32 on gfx950): unlike fmaxf it
// needs no quieting of operands that come from the matrix cores or lane
// permutes, and two in a row fuse into one instruction.
__device__ inline float max_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ inline float group_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_nan(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nan(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float group_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ inline float wave_sum(float x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// Two weights as packed bf16 pairs: hi = the weights rounded to nearest even
// (gfx950's packed conversion), lo = the rounded remainders, so hi + lo
// carries each weight to about 16 significant bits.  Inputs are finite.
__device__ inline void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
  const f32x2 rest = {a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, bf16x2));
}

// Two bf16 -> two f16, exact for magnitudes below 65520 (8 significant bits
// fit in 11; under 2^-14 f16 is subnormal, within 2^-25 of the value);
// magnitudes of 65536 and up become infinities, and NaN stays NaN.
__device__ inline uint32_t bf16x2_to_f16x2(uint32_t w) {
  const f32x2 f = {__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

// Small index inputs of the cache-update kernels (slots, table deltas, block
// pairs) may sit in pinned host memory that the host refills between
// launches.  System-scope loads are never served from a cached copy, so a
// refilled buffer is seen as the host wrote it; within a wave, lanes reading
// the same word share one request.
__device__ inline int64_t ld_sys(const int64_t* p) {
  return __hip_atomic_load(const_cast<int64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ inline int32_t ld_sys(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Buffer resource over one cache tile: loads at byte offsets below `bytes`
// read memory; with bytes == 0 every load returns zeros without a memory
// request.  That lets the pipeline issue the same loads on every trip
// (so the load counter waits are static) while prefetches past the end of
// a partition cost nothing.
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Load of a wave-uniform element through the scalar data cache (read-only
// constant address space): it waits on the scalar counter, so it does not
// drain the vector loads in flight, as a vector load with a full wait would.
__device__ inline int load_uniform(const int* p, int64_t i) {
  using const_int_ptr = const __attribute__((address_space(4))) int*;
  return *((const_int_ptr)p + i);
}

// ------------------------------------------------------------------ FP8 E4M3 (OCP) codes
// Decode: every E4M3 value has at most 4 significant bits and an exponent
// inside bf16's range, so each code has an exact bf16.  gfx950's
// v_cvt_scalef32_pk_bf16_fp8 with scale 1 produces it for two codes in one
// instruction; it reads the OCP E4M3 encoding, and on MI355X its output
// equals the format's definition for all 256 codes (NaN codes give NaN).
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
template <bool HIGH>  // bytes 2, 3 of w when set, else bytes 0, 1
__device__ inline uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH));
}
// 8 codes (bytes of lo then hi) -> 8 bf16 in the same order
__device__ inline uint4 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  uint4 r;
  r.x = e4m3x2_to_bf16x2<false>(lo);
  r.y = e4m3x2_to_bf16x2<true>(lo);
  r.z = e4m3x2_to_bf16x2<false>(hi);
  r.w = e4m3x2_to_bf16x2<true>(hi);
  return r;
}
// The same 8 codes as f16 (v_cvt_scalef32_pk_f16_fp8, scale 1)
template <bool HIGH>
__device__ inline uint32_t e4m3x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HIGH));
}
__device__ inline uint4 e4m3x8_to_f16x8(uint32_t lo, uint32_t hi) {
  uint4 r;
  r.x = e4m3x2_to_f16x2<false>(lo);
  r.y = e4m3x2_to_f16x2<true>(lo);
  r.z = e4m3x2_to_f16x2<false>(hi);
  r.w = e4m3x2_to_f16x2<true>(hi);
  return r;
}

// ------------------------------------------------------------------ host helpers
pkv_status launch_status() {
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int env_int(const char* name, int dflt, int lo, int hi) {
  const char* v = std::getenv(name);
  if (!v) return dflt;
  const int x = std::atoi(v);
  return x < lo ? lo : (x > hi ? hi : x);
}

}  // namespace

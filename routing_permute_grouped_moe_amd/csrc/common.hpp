// Shared device helpers for the MoE kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

typedef uint16_t bf16_t;  // raw bf16 bits; arithmetic is always done in fp32

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

#define MOE_WAVE 64

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// IEEE round-to-nearest-even of fp32 to bf16 (NaN stays NaN): gfx950's
// hardware conversion, branch-free (a software version with a NaN test
// compiles to divergent branches per element).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)f);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int VEC = 4;  // elements per 16-byte chunk
  __device__ static float load(const float* p, long long i) { return p[i]; }
};
template <> struct Elem<bf16_t> {
  static constexpr int VEC = 8;
};

// Unpack a 16-byte chunk of T into fp32 (VEC values).
__device__ __forceinline__ void unpack16(const u32x4& v, float* out, float) {
  out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack16(const u32x4& v, float* out, bf16_t) {
  out[0] = __uint_as_float(v.x << 16); out[1] = __uint_as_float(v.x & 0xffff0000u);
  out[2] = __uint_as_float(v.y << 16); out[3] = __uint_as_float(v.y & 0xffff0000u);
  out[4] = __uint_as_float(v.z << 16); out[5] = __uint_as_float(v.z & 0xffff0000u);
  out[6] = __uint_as_float(v.w << 16); out[7] = __uint_as_float(v.w & 0xffff0000u);
}
__device__ __forceinline__ u32x4 pack16(const float* in, float) {
  u32x4 v;
  v.x = __float_as_uint(in[0]); v.y = __float_as_uint(in[1]);
  v.z = __float_as_uint(in[2]); v.w = __float_as_uint(in[3]);
  return v;
}
__device__ __forceinline__ u32x4 pack16(const float* in, bf16_t) {
  u32x4 v;
  v.x = f32_to_bf16(in[0]) | (f32_to_bf16(in[1]) << 16);
  v.y = f32_to_bf16(in[2]) | (f32_to_bf16(in[3]) << 16);
  v.z = f32_to_bf16(in[4]) | (f32_to_bf16(in[5]) << 16);
  v.w = f32_to_bf16(in[6]) | (f32_to_bf16(in[7]) << 16);
  return v;
}

// ---------------------------------------------------------------- buffer access
// Raw buffer loads/stores: an access at or beyond ``bytes`` from ``base``
// reads zero / is dropped by the hardware, so a wrong index can never fault.

#define MOE_RSRC_DW3 0x00020000

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           MOE_RSRC_DW3);
}

// Byte size of a range, clamped to the 32-bit limit of a buffer descriptor.
__host__ __device__ __forceinline__ uint32_t clamp_bytes(long long b) {
  return b <= 0 ? 0u : (b >= 0xffffffffLL ? 0xffffffffu : (uint32_t)b);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// Streaming read (cache policy nt): data read once, not worth keeping in the
// caches; measured about 12% more HBM read bandwidth than a plain load.
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
// Streaming write (cache policy nt) for rows written once and read by a
// later kernel: measured 3-6% faster for the gathers' row outputs (combine,
// its backward, the permute backward); for the permute's k-fold scatter it
// costs ~1% there but the grouped GEMM that follows runs ~3% faster (fewer
// dirty lines left to drain while it reads its operands).
__device__ __forceinline__ void buf_store16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 2);
}
// Streaming write at device scope (cache policy sc1 nt): the write goes
// through this XCD's L2, so once it has completed (vmcnt) a reader on any
// XCD sees it -- what the compiler emits for an agent-scope atomic store.
__device__ __forceinline__ void buf_store16_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 18);
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store2(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, off, 0, 0);
}

template <typename T>
__device__ __forceinline__ void buf_store_elem(__amdgpu_buffer_rsrc_t r, uint32_t elem, float v);
template <>
__device__ __forceinline__ void buf_store_elem<float>(__amdgpu_buffer_rsrc_t r, uint32_t elem,
                                                      float v) {
  buf_store4(r, elem * 4u, __float_as_uint(v));
}
template <>
__device__ __forceinline__ void buf_store_elem<bf16_t>(__amdgpu_buffer_rsrc_t r, uint32_t elem,
                                                       float v) {
  buf_store2(r, elem * 2u, f32_to_bf16(v));
}

template <typename T>
__device__ __forceinline__ float buf_load_elem(__amdgpu_buffer_rsrc_t r, uint32_t elem);
template <>
__device__ __forceinline__ float buf_load_elem<float>(__amdgpu_buffer_rsrc_t r, uint32_t elem) {
  return __uint_as_float(buf_load4(r, elem * 4u));
}
template <>
__device__ __forceinline__ float buf_load_elem<bf16_t>(__amdgpu_buffer_rsrc_t r, uint32_t elem) {
  uint32_t w = buf_load4(r, (elem * 2u) & ~3u);
  return __uint_as_float((elem & 1u) ? (w & 0xffff0000u) : (w << 16));
}

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MOE_WAVE));
  return v;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long long uniform(long long v) {
  const unsigned long long u = (unsigned long long)v;
  return (long long)(((unsigned long long)(uint32_t)uniform((int)(uint32_t)(u >> 32)) << 32) |
                     (uint32_t)uniform((int)(uint32_t)u));
}

// ---------------------------------------------------------------- host helpers
// (defined in api.cpp)
int moe_fail(int status, const char* fmt, ...);
int moe_check_launch(const char* what);
int moe_cu_count();
// router products on the bf16 MFMA path (gmm.hip)
int moe_gmm_router_fwd(const void* x, const void* wg3s, float* partials, int T, int H, int E, int S,
                       hipStream_t s);
int moe_gmm_router_dx(const void* dlb, const void* wgb, void* dx, int T, int H, int E,
                      hipStream_t s);
int moe_gmm_router_dwg(const void* x, const void* dl3s, float* partials, int T, int H, int E, int S,
                       hipStream_t s);

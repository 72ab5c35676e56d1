// Shared device/host helpers for the gfx950 kernels of libmi_moe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "mi_moe.h"

namespace mi {

// ---------------------------------------------------------------------------
// host-side error reporting
// ---------------------------------------------------------------------------
void set_error(const char* fmt, ...);
void clear_error();

#define MI_REQUIRE(cond, ...)            \
  do {                                   \
    if (!(cond)) {                       \
      ::mi::set_error(__VA_ARGS__);      \
      return MI_EINVAL;                  \
    }                                    \
  } while (0)

#define MI_REQUIRE_SUPPORTED(cond, ...)  \
  do {                                   \
    if (!(cond)) {                       \
      ::mi::set_error(__VA_ARGS__);      \
      return MI_EUNSUPPORTED;            \
    }                                    \
  } while (0)

mi_status launch_status(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// ---------------------------------------------------------------------------
// device types
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// IEEE round-to-nearest-even float -> bf16 bits; NaN -> canonical 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

template <typename T>
__device__ __forceinline__ T bitcast(const uint4& v) {
  return __builtin_bit_cast(T, v);
}

// raw buffer resource (gfx9 layout: dword 3 = 0x00020000) over `bytes` bytes
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2 buf_ld64(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf_ld32(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                             uint32_t soff) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Loads/stores through the global address space.  Pointers that reach a
// kernel through structs, LDS tables or the pointer tables are otherwise
// generic ("flat"); flat accesses share the LDS wait counter, so every LDS
// wait would also wait for them.
#define MI_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ T gld(const void* p) {
  return *(const MI_GLOBAL T*)(p);
}
template <typename T>
__device__ __forceinline__ void gst(void* p, const T& v) {
  *(MI_GLOBAL T*)(p) = v;
}
// a streaming (non-temporal) global load, for data read once
template <typename T>
__device__ __forceinline__ T gld_nt(const void* p) {
  return __builtin_nontemporal_load((const MI_GLOBAL T*)(p));
}

}  // namespace mi

// Shared device helpers and host-side validation for the gdnrt kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/gdnrt.h"

namespace gdnrt {

constexpr int kD = 128;      // d_k = d_v supported by this build
constexpr int kChunk = 64;   // chunk length of the prefill kernels
constexpr int kMaxWindow = 16;
constexpr int kMaxRank = 8;

// ------------------------------------------------------------------ host side

int set_error(int status, const char* fmt, ...);
int clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// true when [a, a+na) and [b, b+nb) share a byte
inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

inline int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(GDNRT_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return clear_error();
}

// ------------------------------------------------------------------ device side

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even: gfx950's packed convert (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two fp32 -> two bf16 in one dword (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// Cross-lane moves inside a 16-lane row (DPP). Controls: row_mirror 0x140,
// row_half_mirror 0x141, quad_perm(1,0,3,2) 0xB1, quad_perm(2,3,0,1) 0x4E.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane receives the total.
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0x140>(x);   // lane i + lane 15-i
  x += dpp<0x141>(x);   // fold the two half-rows
  x += dpp<0x4E>(x);    // lane i + lane i^2
  x += dpp<0xB1>(x);    // lane i + lane i^1
  return x;
}

// Sum over an aligned group of 8 lanes; every lane of the group receives it.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<0x141>(x);
  x += dpp<0x4E>(x);
  x += dpp<0xB1>(x);
  return x;
}

// Sum over an aligned group of 32 lanes.
__device__ __forceinline__ float sum32(float x) {
  x = sum16(x);
  // swizzle, bit-mask mode within 32 lanes: xor 16
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
  return x;
}

// Sum over the whole 64-lane wave.
__device__ __forceinline__ float sum64(float x) {
  x = sum32(x);
  x += __shfl_xor(x, 32);
  return x;
}

// Workgroup barrier that orders LDS only. __syncthreads() also fences global
// memory, which makes the compiler wait for every outstanding global load -- the
// register prefetches included -- at each barrier. The kernels here exchange data
// between threads only through LDS, so an LDS-scoped fence suffices.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename T> struct io_traits;
template <> struct io_traits<float> {
  __device__ static __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
  __device__ static __forceinline__ f32x4 ld4(const float* p, size_t i) {
    return *reinterpret_cast<const f32x4*>(p + i);
  }
  __device__ static __forceinline__ void st(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct io_traits<uint16_t> {
  __device__ static __forceinline__ float ld(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ static __forceinline__ f32x4 ld4(const uint16_t* p, size_t i) {
    uint2 w = *reinterpret_cast<const uint2*>(p + i);
    f32x4 r;
    r.x = __uint_as_float(w.x << 16);
    r.y = __uint_as_float(w.x & 0xffff0000u);
    r.z = __uint_as_float(w.y << 16);
    r.w = __uint_as_float(w.y & 0xffff0000u);
    return r;
  }
  __device__ static __forceinline__ void st(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16(x); }
};

}  // namespace gdnrt

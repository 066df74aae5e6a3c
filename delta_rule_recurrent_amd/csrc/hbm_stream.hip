// Streaming read + write of a large fp32 array: the HBM ceiling the decode rows are
// measured against. Not a step of the method; a measurement aid kept in the library
// so that the ceiling is taken with the same compiler, the same access pattern and the
// same cache hints as the decode kernel (one read and one write of every byte, 16-byte
// non-temporal accesses, 64-lane waves touching 1 KiB per instruction).
#include "common.hpp"

namespace gdnrt {

// Each thread moves VEC consecutive 16-byte pieces spaced one block-width apart, so
// every wave instruction covers 1 KiB of contiguous memory. dst may equal src (an
// in-place pass, as the decode updates its state); x -> x * scale.
template <int VEC>
__global__ __launch_bounds__(256) void hbm_stream_kernel(f32x4* dst, const f32x4* src, size_t n4,
                                                         float scale) {
  const size_t base = (size_t)blockIdx.x * (256 * VEC) + threadIdx.x;
  f32x4 r[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const size_t i = base + (size_t)j * 256;
    r[j] = i < n4 ? __builtin_nontemporal_load(src + i) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const size_t i = base + (size_t)j * 256;
    if (i < n4) __builtin_nontemporal_store(r[j] * scale, dst + i);
  }
}

}  // namespace gdnrt

using namespace gdnrt;

extern "C" int gdnrt_hbm_stream(float* dst, const float* src, size_t n, int vec, float scale,
                                void* stream) {
  const char* fn = "gdnrt_hbm_stream";
  if (n == 0) return clear_error();
  if (!dst || !src) return set_error(GDNRT_EINVAL, "%s: null pointer argument", fn);
  if (n % 4 != 0) return set_error(GDNRT_ESHAPE, "%s: n=%zu must be a multiple of 4", fn, n);
  if (vec != 1 && vec != 2 && vec != 4) return set_error(GDNRT_ESHAPE, "%s: vec=%d (1, 2 or 4)", fn, vec);
  if (!aligned16(dst) || !aligned16(src)) return set_error(GDNRT_EALIGN, "%s: dst, src must be 16-byte aligned", fn);
  if (dst != src && overlaps(dst, n * 4, src, n * 4))
    return set_error(GDNRT_EINVAL, "%s: dst and src overlap without being equal", fn);
  const size_t n4 = n / 4, per_block = (size_t)256 * vec;
  const size_t blocks = (n4 + per_block - 1) / per_block;
  if (blocks > 0x7fffffffu) return set_error(GDNRT_ESHAPE, "%s: n=%zu too large", fn, n);
  hipStream_t s = static_cast<hipStream_t>(stream);
  f32x4* d = reinterpret_cast<f32x4*>(dst);
  const f32x4* r = reinterpret_cast<const f32x4*>(src);
  switch (vec) {
    case 1: hipLaunchKernelGGL(hbm_stream_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, d, r, n4, scale); break;
    case 2: hipLaunchKernelGGL(hbm_stream_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, d, r, n4, scale); break;
    default: hipLaunchKernelGGL(hbm_stream_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, d, r, n4, scale); break;
  }
  return check_launch(fn);
}

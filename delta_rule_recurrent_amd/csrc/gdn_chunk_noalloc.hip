// Gated DeltaNet chunkwise forward without a caller workspace (gdn_chunk_fwd_noalloc).
#include "common.hpp"

#include <mutex>

namespace gdnrt {
int gdn_chunk_fwd_named(const char* fn, const void* q, const void* k, const void* v, const float* alpha,
                        const float* beta, const float* S0, float* ST, void* o, int N, int T, int dk,
                        int dv, int chunk, int io, void* workspace, size_t ws_bytes, void* stream);
}  // namespace gdnrt

using namespace gdnrt;

// ------------------------------------------------------------------ allocation-free variant
//
// gdn_chunk_fwd_noalloc: gdn_chunk_fwd for callers that cannot allocate device memory
// (code under graph capture, tight serving loops). Its per-chunk operands go to a
// fixed scratch array that the library holds on every GPU it runs on, instead of a
// caller's workspace. `scratch` below is a device symbol: in host code its name is not
// a device address, so host code only ever uses the address hipGetSymbolAddress gives
// for the current device, looked up once per device and kept.
namespace {

constexpr size_t kScratchBytes = (size_t)128 << 20;   // 1,637 chunks of 64 tokens
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(GDNRT_ELAUNCH, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(GDNRT_ELAUNCH, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(GDNRT_ELAUNCH, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                       hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDNRT_OK;
}

}  // namespace

extern "C" size_t gdn_chunk_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* alpha,
                                     const float* beta, const float* S0, float* ST, void* o, int N, int T,
                                     int dk, int dv, int chunk, int io, void* stream) {
  const char* fn = "gdn_chunk_fwd_noalloc";
  const size_t need = gdn_chunk_fwd_workspace_bytes(N, T, dk, dv, chunk);
  if (need > kScratchBytes)
    return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d needs %zu bytes of scratch, the maximum is %zu "
                     "(use gdn_chunk_fwd with a workspace)", fn, N, T, need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    int rc = scratch_for_current_device(fn, &ws);
    if (rc != GDNRT_OK) return rc;
  }
  return gdn_chunk_fwd_named(fn, q, k, v, alpha, beta, S0, ST, o, N, T, dk, dv, chunk, io, ws, need, stream);
}

// Per-chunk workspace layout of the GLA chunkwise forward, read after it by the
// sequence-parallel shard calls (cumulative decays, output correction):
//  Q^  Q o e^b, bf16, in 16 fragments f = 4 tb + ks of 1 KB: lane 16 lq + l16 of
//      fragment f holds token 16 tb + l16, keys 32 ks + 4 lq + e and 32 ks + 16 + 4 lq + e
//      (e < 4), in that order (16 bytes)
//  eC  e^{b_C} per key, fp32
// b is the inclusive cumulative log-gate in the chunk. The forward's own per-sequence
// buffers (segment end states and decays, start states) follow the chunks in the
// workspace.
#pragma once
#include <cstddef>

namespace gdnrt {
namespace gla {
constexpr size_t kWQ = 0, kWE = 16384, kWChunk = 16896;
}  // namespace gla
}  // namespace gdnrt

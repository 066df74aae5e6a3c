// Per-chunk workspace layout of the GLA chunkwise forward, read after it by the
// sequence-parallel shard calls (cumulative decays, output correction):
//  Q^  [64 tokens][128 keys] bf16, row-major
//  eC  e^{b_C} per key, fp32
// Q^ = Q o e^b, b the inclusive cumulative log-gate in the chunk. The forward's own
// per-sequence buffers (segment end states and decays, start states) follow the
// chunks in the workspace.
#pragma once
#include <cstddef>

namespace gdnrt {
namespace gla {
constexpr size_t kWQ = 0, kWE = 16384, kWChunk = 16896;
}  // namespace gla
}  // namespace gdnrt

// Per-chunk workspace layout of the GLA chunkwise forward, read by the forward's
// sequential pass and by the sequence-parallel shard calls (cumulative decays,
// output correction). With lane = 16 lq + l16 of a wave:
//  Q^  [64 tokens][128 keys]: 16 A-operand fragments (rb, ks) of 1 KB; the lane holds
//      token 16 rb + l16, keys 32 ks + 8 lq + {0..7}
//  K^  [64 tokens][128 keys]: 16 B-operand fragments (kb, js); the lane holds key
//      16 kb + l16, tokens 32 js + 8 lq + {0..7}
//  O~  [64 tokens][128 values]: 32 accumulator tiles (rb, vb) of 512 B; the lane holds
//      tokens 16 rb + 4 lq + {0..3} of value 16 vb + l16
//  eC  e^{b_C} per key, fp32
// Q^ = Q o e^b, K^ = K o e^{b_C - b}, b the inclusive cumulative log-gate in the chunk.
#pragma once
#include <cstddef>

namespace gdnrt {
namespace gla {
constexpr size_t kWQ = 0, kWK = 16384, kWO = 32768, kWE = 49152, kWChunk = 49664;
}  // namespace gla
}  // namespace gdnrt

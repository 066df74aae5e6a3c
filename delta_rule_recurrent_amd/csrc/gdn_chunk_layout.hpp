// Per-chunk workspace layout of the GDN / KDA chunk prep (state-independent operands
// of the UT form), shared by the chunkwise forward and backward. With
// lane = 16 lq + l16 of a wave:
//  W, Q' [64 tokens][128 keys]: 16 A-operand fragments (rb, ks) of 1 KB; lane holds
//        token rb*16 + l16, keys ks*32 + lq*4 + {0..3} then ks*32 + 16 + lq*4 + {0..3}
//  K^    [64 tokens][128 keys]: 16 B-operand fragments (kb, js) of 1 KB; lane holds
//        key kb*16 + l16, tokens js*32 + lq*8 + {0..7}
//  U~, O~ [64 tokens][128 values]: 32 accumulator tiles (rb, vb) of 512 B; lane holds
//        tokens rb*16 + lq*4 + {0..3} of value vb*16 + l16
//  g_C   16 copies (so that every lane loads it with a vector load)
// All bf16 except g_C (fp32).
#pragma once
#include <cstddef>

namespace gdnrt {
namespace gdc {
constexpr size_t kWsW = 0, kWsQ = 16384, kWsK = 32768, kWsU = 49152, kWsO = 65536;
constexpr size_t kWsG = 81920, kWsChunk = 81984;
}  // namespace gdc
}  // namespace gdnrt

// Gated linear attention, chunkwise forward from an incoming state (prefill shard).
//
// Method: "ZeCO: Zero Communication Overhead Sequence Parallelism for Linear
// Attention", section "Gated Linear Attention (GLA) Formulation" (per-token and
// chunk recurrences, inter/intra-chunk output) and section "The Complete Forward
// Algorithm" (the intra-chunk keys are divided by Lambda). In the [d_v][d_k] state
// layout, with b the inclusive cumulative log-gate inside a chunk of C = 64 tokens:
//
//   O   = (Q o e^b) S^T + [ ((Q o e^b)(K o e^-b)^T) o M ] V,     M lower incl. diag,
//   S  <- e^{b_C} (on key columns) o S + V^T (K o e^{b_C - b}).
//
// The value rows of S evolve independently, so a block owns one sequence and a
// 32-wide tile of value channels (4 blocks per sequence; the 4 are placed on one
// XCD so the shared q/k/g reads hit the same L2) and walks the chunks in order with
// its state tile resident in MFMA accumulators (fp32). Per chunk, bf16 MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation) forms the three contractions.
// The intra-chunk factors are taken relative to the chunk's middle token m,
// Q o e^{b - b_m} and K o e^{b_m - b}, which halves their dynamic range; the
// matching e^{b_m} is folded into the bf16 copy of the state used for Q S^T.
#include "common.hpp"

namespace gdnrt {

namespace gla {

constexpr int C = kChunk;   // 64 tokens
constexpr int VT = 32;      // value channels per block
constexpr int NW = 4;       // waves per block
constexpr int PQ = kD + 8;  // LDS pitch (bf16) of 128-wide rows: conflict-free 16-byte reads
constexpr int PC = C + 8;   // LDS pitch (bf16) of 64-wide rows

struct Smem {
  uint16_t Q[C * PQ];       // q, then q o e^{b - b_m}            [r][k]
  uint16_t K[C * PQ];       // k, then k o e^{b_m - b}            [j][k]
  uint16_t Kh[kD * PC];     // (k o e^{b_C - b})^T               [k][j]
  uint16_t Vt[VT * PC];     // v tile transposed                 [v][j]
  uint16_t A[C * PC];       // masked intra-chunk scores (bf16)  [r][j]
  uint16_t Sb[VT * PQ];     // bf16 state tile scaled by e^{b_m} [v][k]
  float G[C * kD];          // log-gates, then inclusive cumulative sums [r][k]
  float bm[kD], eC[kD];
};

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace gla

__global__ __launch_bounds__(256) void gla_chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ log_g, const float* __restrict__ S0, float* __restrict__ ST,
    uint16_t* __restrict__ o, int N, int T) {
  using namespace gla;
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;

  // block -> (sequence, value tile); tiles of one sequence share an XCD when N % 8 == 0
  int n, vt;
  const int bid = blockIdx.x;
  if ((N & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3;
    n = (slot >> 2) * 8 + xcd;
    vt = slot & 3;
  } else {
    n = bid >> 2;
    vt = bid & 3;
  }
  const int v0 = vt * VT;

  // state tiles of this wave: value blocks {0,1} x key blocks {2w, 2w+1}; lane holds
  // S[v0 + vb*16 + lq*4 + i][kb*16 + l16], i = 0..3
  f32x4 Sacc[2][2];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kcol = (2 * wave + kk) * 16 + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int vrow = v0 + vb * 16 + lq * 4 + i;
        Sacc[vb][kk][i] = S0 ? S0[((size_t)n * kD + vrow) * kD + kcol] : 0.f;
      }
    }

  const size_t seq = (size_t)n * T;
  for (int c0 = 0; c0 < T; c0 += C) {
    // ---- 1. stage q, k (16-byte pieces), the v tile (transposed) and the log-gates
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + 256 * i, row = p >> 4, seg = p & 15;
      const size_t off = (seq + c0 + row) * kD + seg * 8;
      *reinterpret_cast<uint4*>(sm.Q + row * PQ + seg * 8) = *reinterpret_cast<const uint4*>(q + off);
      *reinterpret_cast<uint4*>(sm.K + row * PQ + seg * 8) = *reinterpret_cast<const uint4*>(k + off);
    }
    {
      const int j = tid >> 2, seg = tid & 3;
      const uint4 w = *reinterpret_cast<const uint4*>(v + (seq + c0 + j) * kD + v0 + seg * 8);
      const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.Vt[(seg * 8 + 2 * e) * PC + j] = uint16_t(w4[e] & 0xffffu);
        sm.Vt[(seg * 8 + 2 * e + 1) * PC + j] = uint16_t(w4[e] >> 16);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = tid + 256 * i, row = p >> 5, seg = p & 31;
      *reinterpret_cast<f32x4*>(sm.G + row * kD + seg * 4) =
          *reinterpret_cast<const f32x4*>(log_g + (seq + c0 + row) * kD + seg * 4);
    }
    __syncthreads();

    // ---- 2. inclusive cumulative log-gates per key channel
    if (tid < kD) {
      float b = 0.f;
      for (int r = 0; r < C; ++r) {
        b += sm.G[r * kD + tid];
        sm.G[r * kD + tid] = b;
        if (r == C / 2 - 1) sm.bm[tid] = b;
      }
      sm.eC[tid] = __expf(b);
    }
    __syncthreads();

    // ---- 3. decay factors; bf16 state copy scaled by e^{b_m}
    {
      const int c = tid & (kD - 1), h = tid >> 7;
      const float bm = sm.bm[c];
      const float bC = sm.G[(C - 1) * kD + c];
      for (int r = h * 32; r < h * 32 + 32; ++r) {
        const float b = sm.G[r * kD + c];
        const float qv = bf16_to_f32(sm.Q[r * PQ + c]);
        const float kv = bf16_to_f32(sm.K[r * PQ + c]);
        sm.Q[r * PQ + c] = f32_to_bf16(qv * __expf(b - bm));
        sm.K[r * PQ + c] = f32_to_bf16(kv * __expf(bm - b));
        sm.Kh[c * PC + r] = f32_to_bf16(kv * __expf(bC - b));
      }
    }
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int kcol = (2 * wave + kk) * 16 + l16;
        const float em = __expf(sm.bm[kcol]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.Sb[(vb * 16 + lq * 4 + i) * PQ + kcol] = f32_to_bf16(Sacc[vb][kk][i] * em);
      }
    __syncthreads();

    // ---- 4. intra-chunk scores, row block = wave, causal mask, bf16
    {
      const int rb = wave;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (cb <= rb) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            acc = mfma(ld8(sm.Q + (rb * 16 + l16) * PQ + ks * 32 + lq * 8),
                       ld8(sm.K + (cb * 16 + l16) * PQ + ks * 32 + lq * 8), acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rb * 16 + lq * 4 + i, col = cb * 16 + l16;
          sm.A[row * PC + col] = f32_to_bf16(col <= row ? acc[i] : 0.f);
        }
      }
    }
    __syncthreads();

    // ---- 5. outputs of row block = wave: inter (Q S^T) + intra (A V)
    {
      const int rb = wave;
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc = mfma(ld8(sm.Q + (rb * 16 + l16) * PQ + ks * 32 + lq * 8),
                     ld8(sm.Sb + (vb * 16 + l16) * PQ + ks * 32 + lq * 8), acc);
#pragma unroll
        for (int js = 0; js < 2; ++js) {
          if (js * 32 <= rb * 16 + 15)
            acc = mfma(ld8(sm.A + (rb * 16 + l16) * PC + js * 32 + lq * 8),
                       ld8(sm.Vt + (vb * 16 + l16) * PC + js * 32 + lq * 8), acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rb * 16 + lq * 4 + i;
          o[(seq + c0 + row) * kD + v0 + vb * 16 + l16] = f32_to_bf16(acc[i]);
        }
      }
    }

    // ---- 6. state update: S <- e^{b_C} o S + V^T Kh^T
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int kb = 2 * wave + kk;
        f32x4 acc = Sacc[vb][kk] * sm.eC[kb * 16 + l16];
#pragma unroll
        for (int js = 0; js < 2; ++js)
          acc = mfma(ld8(sm.Vt + (vb * 16 + l16) * PC + js * 32 + lq * 8),
                     ld8(sm.Kh + (kb * 16 + l16) * PC + js * 32 + lq * 8), acc);
        Sacc[vb][kk] = acc;
      }
    __syncthreads();
  }

#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kcol = (2 * wave + kk) * 16 + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int vrow = v0 + vb * 16 + lq * 4 + i;
        ST[((size_t)n * kD + vrow) * kD + kcol] = Sacc[vb][kk][i];
      }
    }
}

}  // namespace gdnrt

using namespace gdnrt;

extern "C" int gla_chunk_fwd(const void* q, const void* k, const void* v, const float* log_g,
                             const float* S0, float* ST, void* o, int N, int T, int dk, int dv,
                             int chunk, int io, void* stream) {
  if (N < 0 || T < 0) return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: N=%d T=%d must be >= 0", N, T);
  if (dk != kD || dv != kD)
    return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: d_k=%d d_v=%d, only 128 is supported", dk, dv);
  if (chunk != kChunk) return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: chunk=%d, only 64 is supported", chunk);
  if (T % kChunk) return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: T=%d is not a multiple of 64", T);
  if (io != GDNRT_BF16) return set_error(GDNRT_EDTYPE, "gla_chunk_fwd: io must be GDNRT_BF16");
  if ((size_t)N * 4 > 0x7fffffffu) return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: N too large");
  if (N == 0) return clear_error();
  if (!ST || (T > 0 && (!q || !k || !v || !log_g || !o)))
    return set_error(GDNRT_EINVAL, "gla_chunk_fwd: null pointer argument");
  if ((T > 0 && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_g) || !aligned16(o))) ||
      !aligned4(ST) || (S0 && !aligned4(S0)))
    return set_error(GDNRT_EALIGN, "gla_chunk_fwd: q, k, v, log_g, o must be 16-byte aligned");
  const size_t ntok = (size_t)N * T, nIO = ntok * kD * 2, nG = ntok * kD * 4, nS = (size_t)N * kD * kD * 4;
  if (overlaps(o, nIO, q, nIO) || overlaps(o, nIO, k, nIO) || overlaps(o, nIO, v, nIO) ||
      overlaps(o, nIO, log_g, nG) || overlaps(o, nIO, ST, nS) || overlaps(o, nIO, S0, nS) ||
      overlaps(ST, nS, q, nIO) || overlaps(ST, nS, k, nIO) || overlaps(ST, nS, v, nIO) ||
      overlaps(ST, nS, log_g, nG) || (S0 && S0 != ST && overlaps(ST, nS, S0, nS)))
    return set_error(GDNRT_EINVAL, "gla_chunk_fwd: output buffers overlap inputs (ST may equal S0)");
  // T == 0 launches too: the kernel then copies the incoming state (or zeros) to ST
  hipLaunchKernelGGL(gla_chunk_kernel, dim3((unsigned)(N * 4)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), log_g, S0, ST,
                     static_cast<uint16_t*>(o), N, T);
  return check_launch("gla_chunk_fwd");
}

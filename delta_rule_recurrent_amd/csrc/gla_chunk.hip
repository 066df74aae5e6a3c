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
// Q o e^{b - b_m} and K o e^{b_m - b}, which halves their dynamic range; the inter
// term uses Q o e^{b} (never above |q|). 512 threads: for the elementwise work each
// thread owns two adjacent key channels of 8 tokens, whose log-gates, q and k are
// prefetched into registers one chunk ahead while the MFMA work runs; the
// cumulative sums are formed in registers with one exchange of per-eighth totals.
// The bf16 copy of the state is double-buffered so the update does not wait for
// the output products.
#include "common.hpp"

namespace gdnrt {

namespace gla {

constexpr int C = kChunk;   // 64 tokens
constexpr int VT = 32;      // value channels per block
constexpr int NT = 512;     // threads per block (8 waves)
constexpr int PQ = kD + 8;  // LDS pitch (bf16) of 128-wide rows: conflict-free 16-byte reads
constexpr int PC = C + 8;   // LDS pitch (bf16) of 64-wide rows

struct Smem {
  uint16_t Qr[C * PQ];      // q o e^{b - b_m}     [r][k]  (intra-chunk scores)
  uint16_t Qi[C * PQ];      // q o e^{b}           [r][k]  (inter-chunk output)
  uint16_t Kr[C * PQ];      // k o e^{b_m - b}     [j][k]
  uint16_t Kh[kD * PC];     // (k o e^{b_C - b})^T [k][j]
  uint16_t Vt[VT * PC];     // v tile transposed   [v][j]
  uint16_t A[C * PC];       // masked scores       [r][j]
  uint16_t Sb[2][VT * PQ];  // bf16 state tile     [v][k], double buffered
  float tot[8 * kD];        // per token-eighth log-gate sums
  float eC[kD];
};

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// One chunk's inputs for this thread: key channels (2cp, 2cp+1) of tokens
// [8e, 8e+8): log-gates, q and k pairs; and one 16-byte piece of the v tile.
struct Prefetch {
  f32x2 g[8];
  unsigned q[8], k[8];
  u32x4 v;
};

__device__ __forceinline__ void fetch(Prefetch& pf, const uint16_t* __restrict__ q,
                                      const uint16_t* __restrict__ k,
                                      const uint16_t* __restrict__ v,
                                      const float* __restrict__ log_g, size_t tok0, int v0) {
  const int t = threadIdx.x, cp = t & 63, e = t >> 6;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const size_t row = tok0 + 8 * e + i;
    pf.g[i] = *reinterpret_cast<const f32x2*>(log_g + row * kD + 2 * cp);
    pf.q[i] = *reinterpret_cast<const unsigned*>(q + row * kD + 2 * cp);
    pf.k[i] = *reinterpret_cast<const unsigned*>(k + row * kD + 2 * cp);
  }
  if (t < 256) {
    const int j = t >> 2, seg = t & 3;
    pf.v = *reinterpret_cast<const u32x4*>(v + (tok0 + j) * kD + v0 + seg * 8);
  }
}


}  // namespace gla

__global__ __launch_bounds__(512) void gla_chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ log_g, const float* __restrict__ S0, float* __restrict__ ST,
    uint16_t* __restrict__ o, int N, int T) {
  using namespace gla;
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int cp = tid & 63, e8 = tid >> 6;   // elementwise: key-channel pair, token eighth

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

  // state tiles of this wave: key block w, value blocks {0, 1}; lane holds
  // S[v0 + vb*16 + lq*4 + i][w*16 + l16], i = 0..3
  const int kcol = wave * 16 + l16;
  f32x4 Sacc[2];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vrow = v0 + vb * 16 + lq * 4 + i;
      Sacc[vb][i] = S0 ? S0[((size_t)n * kD + vrow) * kD + kcol] : 0.f;
      sm.Sb[0][(vb * 16 + lq * 4 + i) * PQ + kcol] = f32_to_bf16(Sacc[vb][i]);
    }

  const size_t seq = (size_t)n * T;
  Prefetch pf;
  if (T > 0) fetch(pf, q, k, v, log_g, seq, v0);
  int cur = 0;
  for (int c0 = 0; c0 < T; c0 += C) {
    // ---- E1: prefix sums of this thread's 8 tokens, eighth totals to LDS
    f32x2 b[8];
    b[0] = pf.g[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) b[i] = b[i - 1] + pf.g[i];
    *reinterpret_cast<f32x2*>(sm.tot + e8 * kD + 2 * cp) = b[7];
    __syncthreads();

    // ---- E2: decay factors; operands to LDS
    {
      f32x2 off = {0.f, 0.f}, bm = {0.f, 0.f}, bC = {0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const f32x2 te = *reinterpret_cast<const f32x2*>(sm.tot + e * kD + 2 * cp);
        if (e < e8) off += te;
        if (e < 4) bm += te;
        bC += te;
      }
      // one exponential and one reciprocal per element: p = e^{b - b_m};
      // e^{b} = p e^{b_m}, e^{b_m - b} = 1/p, e^{b_C - b} = e^{b_C - b_m} / p
      const f32x2 em = {__expf(bm.x), __expf(bm.y)};
      const f32x2 eCm = {__expf(bC.x - bm.x), __expf(bC.y - bm.y)};
      float kh0[8], kh1[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * e8 + i;
        const f32x2 bb = b[i] + off;
        const float q0 = __uint_as_float(pf.q[i] << 16), q1 = __uint_as_float(pf.q[i] & 0xffff0000u);
        const float k0 = __uint_as_float(pf.k[i] << 16), k1 = __uint_as_float(pf.k[i] & 0xffff0000u);
        const float p0 = __expf(bb.x - bm.x), p1 = __expf(bb.y - bm.y);
        const float r0 = __frcp_rn(p0), r1 = __frcp_rn(p1);
        *reinterpret_cast<unsigned*>(sm.Qi + r * PQ + 2 * cp) = pack_bf16(q0 * p0 * em.x, q1 * p1 * em.y);
        *reinterpret_cast<unsigned*>(sm.Qr + r * PQ + 2 * cp) = pack_bf16(q0 * p0, q1 * p1);
        *reinterpret_cast<unsigned*>(sm.Kr + r * PQ + 2 * cp) = pack_bf16(k0 * r0, k1 * r1);
        kh0[i] = k0 * r0 * eCm.x;
        kh1[i] = k1 * r1 * eCm.y;
      }
      u32x4 w0, w1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0[i] = pack_bf16(kh0[2 * i], kh0[2 * i + 1]);
        w1[i] = pack_bf16(kh1[2 * i], kh1[2 * i + 1]);
      }
      *reinterpret_cast<u32x4*>(sm.Kh + (2 * cp) * PC + 8 * e8) = w0;
      *reinterpret_cast<u32x4*>(sm.Kh + (2 * cp + 1) * PC + 8 * e8) = w1;
      if (e8 == 0) {
        sm.eC[2 * cp] = eCm.x * em.x;
        sm.eC[2 * cp + 1] = eCm.y * em.y;
      }
      if (tid < 256) {
        const int j = tid >> 2, seg = tid & 3;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.Vt[(seg * 8 + 2 * e) * PC + j] = uint16_t(pf.v[e] & 0xffffu);
          sm.Vt[(seg * 8 + 2 * e + 1) * PC + j] = uint16_t(pf.v[e] >> 16);
        }
      }
    }
    __syncthreads();
    if (c0 + C < T) fetch(pf, q, k, v, log_g, seq + c0 + C, v0);   // overlaps the MFMA work

    // ---- M1: masked intra-chunk scores; wave -> row block (w & 3), column blocks 2(w>>2)+{0,1}
    {
      const int rb = wave & 3;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int cb = 2 * (wave >> 2) + cc;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (cb <= rb) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            acc = mfma(ld8(sm.Qr + (rb * 16 + l16) * PQ + ks * 32 + lq * 8),
                       ld8(sm.Kr + (cb * 16 + l16) * PQ + ks * 32 + lq * 8), acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rb * 16 + lq * 4 + i, col = cb * 16 + l16;
          sm.A[row * PC + col] = f32_to_bf16(col <= row ? acc[i] : 0.f);
        }
      }
    }
    __syncthreads();

    // ---- M2: outputs (wave -> row block w & 3, value block w >> 2) and state update
    {
      const int rb = wave & 3, vb = wave >> 2;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma(ld8(sm.Qi + (rb * 16 + l16) * PQ + ks * 32 + lq * 8),
                   ld8(sm.Sb[cur] + (vb * 16 + l16) * PQ + ks * 32 + lq * 8), acc);
#pragma unroll
      for (int js = 0; js < 2; ++js)
        if (js * 32 <= rb * 16 + 15)
          acc = mfma(ld8(sm.A + (rb * 16 + l16) * PC + js * 32 + lq * 8),
                     ld8(sm.Vt + (vb * 16 + l16) * PC + js * 32 + lq * 8), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rb * 16 + lq * 4 + i;
        o[(seq + c0 + row) * kD + v0 + vb * 16 + l16] = f32_to_bf16(acc[i]);
      }
    }
    {
      const float dec = sm.eC[kcol];
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        f32x4 acc = Sacc[vb] * dec;
#pragma unroll
        for (int js = 0; js < 2; ++js)
          acc = mfma(ld8(sm.Vt + (vb * 16 + l16) * PC + js * 32 + lq * 8),
                     ld8(sm.Kh + (wave * 16 + l16) * PC + js * 32 + lq * 8), acc);
        Sacc[vb] = acc;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.Sb[cur ^ 1][(vb * 16 + lq * 4 + i) * PQ + kcol] = f32_to_bf16(acc[i]);
      }
    }
    cur ^= 1;
    __syncthreads();
  }

#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vrow = v0 + vb * 16 + lq * 4 + i;
      ST[((size_t)n * kD + vrow) * kD + kcol] = Sacc[vb][i];
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
  hipLaunchKernelGGL(gla_chunk_kernel, dim3((unsigned)(N * 4)), dim3(gla::NT), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), log_g, S0, ST,
                     static_cast<uint16_t*>(o), N, T);
  return check_launch("gla_chunk_fwd");
}

// Gated DeltaNet chunkwise forward (prefill) through the UT / WY form.
//
// The recurrence is the one of "LeapQuant: an 8-bit recurrent state that stops
// rounding every token", section "The state, from the update rule up" (eq. 3: decay,
// then one rank-one write of the correction u_t). The pages print no chunk form for
// the delta rule; unrolling eq. 3 inside a chunk of C = 64 tokens, with local
// positions r, j, g_r = prod_{i<=r} alpha_i and rows of K, V, Q, U being tokens,
// gives (state [d_v][d_k]):
//
//   (I + L) U = diag(beta) V - diag(beta g) K S_0^T,   L[r,j] = beta_r (g_r/g_j) k_r.k_j, j < r
//   U   = U~ - W S_0^T,   T = (I + L)^-1,  W = T diag(beta g) K,  U~ = T diag(beta) V,
//   O   = diag(g) Q S_0^T + A U,            A[r,j] = (g_r/g_j) q_r.k_j for j <= r, else 0,
//   S_C = g_C S_0 + U^T diag(g_C/g) K.
//
// W, U~ and A do not depend on the state. A first kernel forms them for every
// chunk in parallel (Gram and score products on bf16 MFMA, the triangular inverse in
// fp32 by 16 x 16 diagonal blocks and block rows) and writes them, bf16, to the
// caller's workspace. A second kernel walks the chunks of each sequence in order for
// a tile of value channels (the value rows of U and S are independent) with only
// MFMA work per chunk, its state tile in fp32 accumulators, and the next chunk's
// inputs prefetched into registers.
#include "common.hpp"

namespace gdnrt {

namespace gdc {

constexpr int C = kChunk;   // 64
constexpr int PQ = kD + 8;  // bf16 pitch of 128-wide rows
constexpr int PC = C + 8;   // bf16 pitch of 64-wide rows
constexpr int PF = C + 1;   // fp32 pitch of 64-wide rows

// workspace per chunk: W [64][128] bf16, U~ [64][128] bf16, A [64][64] bf16
constexpr size_t kWsW = 0, kWsU = (size_t)C * kD * 2, kWsA = 2 * (size_t)C * kD * 2;
constexpr size_t kWsChunk = kWsA + (size_t)C * C * 2;   // 40,960 bytes

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ float wave_scan(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

struct PrepSmem {
  uint16_t Q[C * PQ];     // [r][k]
  uint16_t K[C * PQ];     // [j][k]
  uint16_t Kt[kD * PC];   // [k][j]
  uint16_t Vt[kD * PC];   // [v][j]
  float L[C * PF];        // strict lower part of (I + L)
  float T[C * PF];        // (I + L)^-1
  float M[3 * 16 * 17];   // block-row partial products
  uint16_t Tw[C * PC];    // T diag(beta g), bf16
  uint16_t Tu[C * PC];    // T diag(beta), bf16
  float lg[C], bt[C];
};

}  // namespace gdc

// ============================================================== kernel 1: per-chunk prep
__global__ __launch_bounds__(256) void gdn_chunk_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, uint8_t* __restrict__ ws,
    int T) {
  using namespace gdc;
  __shared__ PrepSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int nc = T / C;
  const int n = blockIdx.x / nc, ci = blockIdx.x % nc;
  const size_t tok0 = (size_t)n * T + (size_t)ci * C;
  uint8_t* wsc = ws + (size_t)blockIdx.x * kWsChunk;

  // ---- stage q, k (and k^T), v^T; cumulative log-decays
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i, row = p >> 4, seg = p & 15;
    const size_t off = (tok0 + row) * kD + seg * 8;
    const uint4 qw = *reinterpret_cast<const uint4*>(q + off);
    const uint4 kw = *reinterpret_cast<const uint4*>(k + off);
    const uint4 vw = *reinterpret_cast<const uint4*>(v + off);
    *reinterpret_cast<uint4*>(sm.Q + row * PQ + seg * 8) = qw;
    *reinterpret_cast<uint4*>(sm.K + row * PQ + seg * 8) = kw;
    const uint32_t k4[4] = {kw.x, kw.y, kw.z, kw.w}, v4[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sm.Kt[(seg * 8 + 2 * e) * PC + row] = uint16_t(k4[e] & 0xffffu);
      sm.Kt[(seg * 8 + 2 * e + 1) * PC + row] = uint16_t(k4[e] >> 16);
      sm.Vt[(seg * 8 + 2 * e) * PC + row] = uint16_t(v4[e] & 0xffffu);
      sm.Vt[(seg * 8 + 2 * e + 1) * PC + row] = uint16_t(v4[e] >> 16);
    }
  }
  if (wave == 0) {
    const float lgv = wave_scan(__logf(alpha[tok0 + lane]));
    sm.lg[lane] = lgv;
    sm.bt[lane] = beta[tok0 + lane];
  }
  __syncthreads();

  // ---- Gram k.k and scores q.k, row block = wave, lower tiles; L and A
  {
    const int rb = wave;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      f32x4 g = {0.f, 0.f, 0.f, 0.f}, s = {0.f, 0.f, 0.f, 0.f};
      if (cb <= rb) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 kb = ld8(sm.K + (cb * 16 + l16) * PQ + ks * 32 + lq * 8);
          g = mfma(ld8(sm.K + (rb * 16 + l16) * PQ + ks * 32 + lq * 8), kb, g);
          s = mfma(ld8(sm.Q + (rb * 16 + l16) * PQ + ks * 32 + lq * 8), kb, s);
        }
      }
      uint16_t* Aw = reinterpret_cast<uint16_t*>(wsc + kWsA);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb * 16 + lq * 4 + i, j = cb * 16 + l16;
        const float dec = j <= r ? __expf(sm.lg[r] - sm.lg[j]) : 0.f;
        sm.L[r * PF + j] = j < r ? sm.bt[r] * dec * g[i] : 0.f;
        Aw[r * C + j] = f32_to_bf16(dec * s[i]);
      }
    }
  }
  __syncthreads();

  // ---- T = (I + L)^-1: diagonal 16 x 16 blocks by column forward substitution
  if (tid < 64) {
    const int b = tid >> 4, c = tid & 15, o = b * 16;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = i == c ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < i; ++j) s -= sm.L[(o + i) * PF + o + j] * x[j];
      x[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.T[(o + i) * PF + o + c] = x[i];
  }
  // zero the strictly upper blocks
  for (int e = tid; e < C * C; e += 256) {
    const int r = e >> 6, c = e & 63;
    if ((c >> 4) > (r >> 4)) sm.T[r * PF + c] = 0.f;
  }
  __syncthreads();
  // block rows I = 1..3: M_J = sum_{K=J}^{I-1} L_IK T_KJ, then T_IJ = -D_I M_J
  for (int I = 1; I < 4; ++I) {
    for (int e = tid; e < I * 256; e += 256) {
      const int J = e >> 8, i = (e >> 4) & 15, j = e & 15;
      float s = 0.f;
      for (int kk = J * 16; kk < I * 16; ++kk) s += sm.L[(I * 16 + i) * PF + kk] * sm.T[kk * PF + J * 16 + j];
      sm.M[J * 272 + i * 17 + j] = s;
    }
    __syncthreads();
    for (int e = tid; e < I * 256; e += 256) {
      const int J = e >> 8, i = (e >> 4) & 15, j = e & 15;
      float s = 0.f;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) s -= sm.T[(I * 16 + i) * PF + I * 16 + kk] * sm.M[J * 272 + kk * 17 + j];
      sm.T[(I * 16 + i) * PF + J * 16 + j] = s;
    }
    __syncthreads();
  }

  // ---- T diag(beta g) and T diag(beta) in bf16
  for (int e = tid; e < C * C; e += 256) {
    const int r = e >> 6, j = e & 63;
    const float t = sm.T[r * PF + j];
    const float bj = sm.bt[j];
    sm.Tw[r * PC + j] = f32_to_bf16(t * bj * __expf(sm.lg[j]));
    sm.Tu[r * PC + j] = f32_to_bf16(t * bj);
  }
  __syncthreads();

  // ---- W = Tw K, U~ = Tu V: row block = wave, 8 column blocks, K = 64
  {
    const int rb = wave;
    uint16_t* Ww = reinterpret_cast<uint16_t*>(wsc + kWsW);
    uint16_t* Uw = reinterpret_cast<uint16_t*>(wsc + kWsU);
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      f32x4 w = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        w = mfma(ld8(sm.Tw + (rb * 16 + l16) * PC + js * 32 + lq * 8),
                 ld8(sm.Kt + (cb * 16 + l16) * PC + js * 32 + lq * 8), w);
        u = mfma(ld8(sm.Tu + (rb * 16 + l16) * PC + js * 32 + lq * 8),
                 ld8(sm.Vt + (cb * 16 + l16) * PC + js * 32 + lq * 8), u);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb * 16 + lq * 4 + i, c = cb * 16 + l16;
        Ww[r * kD + c] = f32_to_bf16(w[i]);
        Uw[r * kD + c] = f32_to_bf16(u[i]);
      }
    }
  }
}

// ============================================================== kernel 2: sequential pass
namespace gdc {

template <int VT>
struct SeqSmem {
  uint16_t W[C * PQ];      // [r][k]
  uint16_t Qg[C * PQ];     // diag(g) Q   [r][k]
  uint16_t Kht[kD * PC];   // (diag(g_C/g) K)^T  [k][j]
  uint16_t A[C * PC];      // [r][j]
  uint16_t Sb[VT * PQ];    // bf16 state tile [v][k]
  uint16_t Ut[VT * PC];    // U^T tile [v][j]
  float g[C];              // cumulative log-decay of the chunk
};

}  // namespace gdc

// one chunk's inputs of the sequential pass, held in registers while the previous
// chunk computes: W, q, k (64 x 128 bf16, 4 x 16 bytes per thread), A (2 x 16 bytes),
// alpha (lanes of wave 0)
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // register-promotable across loops
struct Prefetch {
  u32x4 w[4], q[4], k[4], a[2];
  float al;
};

__device__ __forceinline__ void fetch_chunk(Prefetch& pf, const uint16_t* __restrict__ q,
                                            const uint16_t* __restrict__ k,
                                            const float* __restrict__ alpha,
                                            const uint8_t* __restrict__ ws, int n, int nc, int ci,
                                            int T) {
  using namespace gdc;
  const int tid = threadIdx.x;
  const size_t tok0 = (size_t)n * T + (size_t)ci * C;
  const uint8_t* wsc = ws + ((size_t)n * nc + ci) * kWsChunk;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i, row = p >> 4, seg = p & 15;
    pf.w[i] = *reinterpret_cast<const u32x4*>(wsc + kWsW + (size_t)(row * kD + seg * 8) * 2);
    pf.q[i] = *reinterpret_cast<const u32x4*>(q + (tok0 + row) * kD + seg * 8);
    pf.k[i] = *reinterpret_cast<const u32x4*>(k + (tok0 + row) * kD + seg * 8);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + 256 * i, row = p >> 3, seg = p & 7;
    pf.a[i] = *reinterpret_cast<const u32x4*>(wsc + kWsA + (size_t)(row * C + seg * 8) * 2);
  }
  pf.al = tid < C ? alpha[tok0 + tid] : 1.f;
}

template <int VT>
__global__ __launch_bounds__(256) void gdn_chunk_seq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ alpha,
    const uint8_t* __restrict__ ws, const float* __restrict__ S0, float* __restrict__ ST,
    uint16_t* __restrict__ o, int N, int T) {
  using namespace gdc;
  constexpr int NVB = VT / 16;           // value blocks in the tile
  constexpr int TPS = kD / VT;           // tiles per sequence
  __shared__ SeqSmem<VT> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n = blockIdx.x / TPS, vt = blockIdx.x % TPS, v0 = vt * VT;
  const int nc = T / C;

  // state tiles: value blocks vb < NVB x key blocks {2w, 2w+1}
  f32x4 Sacc[NVB][2];
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kc = (2 * wave + kk) * 16 + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Sacc[vb][kk][i] = S0 ? S0[((size_t)n * kD + v0 + vb * 16 + lq * 4 + i) * kD + kc] : 0.f;
    }

  // prefetch registers for one chunk
  Prefetch pf;
  if (nc > 0) fetch_chunk(pf, q, k, alpha, ws, n, nc, 0, T);

  for (int ci = 0; ci < nc; ++ci) {
    const size_t tok0 = (size_t)n * T + (size_t)ci * C;
    const uint8_t* wsc = ws + ((size_t)n * nc + ci) * kWsChunk;
    // ---- decays of this chunk
    if (wave == 0) sm.g[lane] = wave_scan(__logf(pf.al));   // cumulative log-decay
    // U~ tile straight into the accumulator layout (row block = wave)
    f32x4 Ut_acc[NVB];
    {
      const uint16_t* Uw = reinterpret_cast<const uint16_t*>(wsc + kWsU);
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Ut_acc[vb][i] = bf16_to_f32(Uw[(wave * 16 + lq * 4 + i) * kD + v0 + vb * 16 + l16]);
    }
    // bf16 copy of the state tile
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int kc = (2 * wave + kk) * 16 + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.Sb[(vb * 16 + lq * 4 + i) * PQ + kc] = f32_to_bf16(Sacc[vb][kk][i]);
      }
    // W and A to LDS as they are
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + 256 * i, row = p >> 4, seg = p & 15;
      *reinterpret_cast<u32x4*>(sm.W + row * PQ + seg * 8) = pf.w[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = tid + 256 * i, row = p >> 3, seg = p & 7;
      *reinterpret_cast<u32x4*>(sm.A + row * PC + seg * 8) = pf.a[i];
    }
    __syncthreads();   // g ready
    // diag(g) Q and (diag(g_C/g) K)^T, from cumulative log-decays
    {
      const float lC = sm.g[C - 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = tid + 256 * i, row = p >> 4, seg = p & 15;
        const float gr = __expf(sm.g[row]), kr = __expf(lC - sm.g[row]);
        const u32x4 q4 = pf.q[i], k4 = pf.k[i];
        uint32_t out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint16_t lo = f32_to_bf16(gr * __uint_as_float(q4[e] << 16));
          const uint16_t hi = f32_to_bf16(gr * __uint_as_float(q4[e] & 0xffff0000u));
          out[e] = uint32_t(lo) | (uint32_t(hi) << 16);
          sm.Kht[(seg * 8 + 2 * e) * PC + row] = f32_to_bf16(kr * __uint_as_float(k4[e] << 16));
          sm.Kht[(seg * 8 + 2 * e + 1) * PC + row] = f32_to_bf16(kr * __uint_as_float(k4[e] & 0xffff0000u));
        }
        *reinterpret_cast<u32x4*>(sm.Qg + row * PQ + seg * 8) = u32x4{out[0], out[1], out[2], out[3]};
      }
    }
    if (ci + 1 < nc) fetch_chunk(pf, q, k, alpha, ws, n, nc, ci + 1, T);   // overlaps the MFMA work below
    __syncthreads();

    // ---- U = U~ - W S^T (row block = wave), to LDS transposed
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma(ld8(sm.W + (wave * 16 + l16) * PQ + ks * 32 + lq * 8),
                   ld8(sm.Sb + (vb * 16 + l16) * PQ + ks * 32 + lq * 8), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sm.Ut[(vb * 16 + l16) * PC + wave * 16 + lq * 4 + i] = f32_to_bf16(Ut_acc[vb][i] - acc[i]);
    }
    __syncthreads();

    // ---- O = diag(g) Q S^T + A U (row block = wave)
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma(ld8(sm.Qg + (wave * 16 + l16) * PQ + ks * 32 + lq * 8),
                   ld8(sm.Sb + (vb * 16 + l16) * PQ + ks * 32 + lq * 8), acc);
#pragma unroll
      for (int js = 0; js < 2; ++js)
        if (js * 32 <= wave * 16 + 15)
          acc = mfma(ld8(sm.A + (wave * 16 + l16) * PC + js * 32 + lq * 8),
                     ld8(sm.Ut + (vb * 16 + l16) * PC + js * 32 + lq * 8), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[(tok0 + wave * 16 + lq * 4 + i) * kD + v0 + vb * 16 + l16] = f32_to_bf16(acc[i]);
    }

    // ---- S <- g_C S + U^T (diag(g_C/g) K)
    {
      const float gC = __expf(sm.g[C - 1]);
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int kb = 2 * wave + kk;
          f32x4 acc = Sacc[vb][kk] * gC;
#pragma unroll
          for (int js = 0; js < 2; ++js)
            acc = mfma(ld8(sm.Ut + (vb * 16 + l16) * PC + js * 32 + lq * 8),
                       ld8(sm.Kht + (kb * 16 + l16) * PC + js * 32 + lq * 8), acc);
          Sacc[vb][kk] = acc;
        }
    }
    __syncthreads();
  }

#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kc = (2 * wave + kk) * 16 + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ST[((size_t)n * kD + v0 + vb * 16 + lq * 4 + i) * kD + kc] = Sacc[vb][kk][i];
    }
}

}  // namespace gdnrt

using namespace gdnrt;

extern "C" size_t gdn_chunk_fwd_workspace_bytes(int N, int T, int dk, int dv, int chunk) {
  if (N <= 0 || T <= 0 || dk != kD || dv != kD || chunk != kChunk || T % kChunk) return 0;
  return (size_t)N * (T / kChunk) * gdc::kWsChunk;
}

extern "C" int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* S0, float* ST, void* o, int N, int T,
                             int dk, int dv, int chunk, int io, void* workspace, size_t ws_bytes,
                             void* stream) {
  if (N < 0 || T < 0) return set_error(GDNRT_ESHAPE, "gdn_chunk_fwd: N=%d T=%d must be >= 0", N, T);
  if (dk != kD || dv != kD)
    return set_error(GDNRT_ESHAPE, "gdn_chunk_fwd: d_k=%d d_v=%d, only 128 is supported", dk, dv);
  if (chunk != kChunk) return set_error(GDNRT_ESHAPE, "gdn_chunk_fwd: chunk=%d, only 64 is supported", chunk);
  if (T % kChunk) return set_error(GDNRT_ESHAPE, "gdn_chunk_fwd: T=%d is not a multiple of 64", T);
  if (io != GDNRT_BF16) return set_error(GDNRT_EDTYPE, "gdn_chunk_fwd: io must be GDNRT_BF16");
  if ((size_t)N * (T / kChunk) > 0x7fffffffu || (size_t)N * 8 > 0x7fffffffu)
    return set_error(GDNRT_ESHAPE, "gdn_chunk_fwd: N=%d T=%d too large", N, T);
  if (N == 0) return clear_error();
  if (!ST || (T > 0 && (!q || !k || !v || !alpha || !beta || !o)))
    return set_error(GDNRT_EINVAL, "gdn_chunk_fwd: null pointer argument");
  const size_t need = T > 0 ? (size_t)N * (T / kChunk) * gdc::kWsChunk : 0;
  if (ws_bytes < need || (need && !workspace))
    return set_error(GDNRT_EINVAL, "gdn_chunk_fwd: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if ((T > 0 && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace) ||
                 !aligned4(alpha) || !aligned4(beta))) ||
      !aligned4(ST) || (S0 && !aligned4(S0)))
    return set_error(GDNRT_EALIGN, "gdn_chunk_fwd: q, k, v, o, workspace must be 16-byte aligned");
  const size_t ntok = (size_t)N * T, nIO = ntok * kD * 2, nG = ntok * 4, nS = (size_t)N * kD * kD * 4;
  if (overlaps(o, nIO, q, nIO) || overlaps(o, nIO, k, nIO) || overlaps(o, nIO, v, nIO) ||
      overlaps(o, nIO, alpha, nG) || overlaps(o, nIO, beta, nG) || overlaps(o, nIO, ST, nS) ||
      overlaps(o, nIO, S0, nS) || overlaps(o, nIO, workspace, need) ||
      overlaps(ST, nS, q, nIO) || overlaps(ST, nS, k, nIO) || overlaps(ST, nS, v, nIO) ||
      overlaps(ST, nS, workspace, need) || (S0 && S0 != ST && overlaps(ST, nS, S0, nS)) ||
      overlaps(workspace, need, q, nIO) || overlaps(workspace, need, k, nIO) ||
      overlaps(workspace, need, v, nIO) || overlaps(workspace, need, S0, nS))
    return set_error(GDNRT_EINVAL, "gdn_chunk_fwd: buffers overlap (only ST may equal S0)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (T > 0) {
    hipLaunchKernelGGL(gdn_chunk_prep_kernel, dim3((unsigned)(N * (T / kChunk))), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), alpha, beta, ws, T);
    int rc = check_launch("gdn_chunk_fwd (prep)");
    if (rc != GDNRT_OK) return rc;
  }
  // value tiles of 16 when there are too few sequences to fill the chip with 32
  if (N * 4 < 256)
    hipLaunchKernelGGL((gdn_chunk_seq_kernel<16>), dim3((unsigned)(N * 8)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), alpha, ws,
                       S0, ST, static_cast<uint16_t*>(o), N, T);
  else
    hipLaunchKernelGGL((gdn_chunk_seq_kernel<32>), dim3((unsigned)(N * 4)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), alpha, ws,
                       S0, ST, static_cast<uint16_t*>(o), N, T);
  return check_launch("gdn_chunk_fwd");
}

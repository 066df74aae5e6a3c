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
// W, U~, A, diag(g) Q and diag(g_C/g) K do not depend on the state. A first kernel
// forms them for every chunk in parallel (Gram and score products on bf16 MFMA, the
// triangular inverse in fp32 by 16 x 16 diagonal blocks and block rows) and writes
// them, bf16, to the caller's workspace. A second kernel walks the chunks of each
// sequence in order for a tile of value channels (the value rows of U and S are
// independent): per chunk it only copies the prepared operands into LDS and runs
// MFMA, its state tile in fp32 accumulators, the next chunk's operands prefetched
// into registers.
#include "common.hpp"

namespace gdnrt {

namespace gdc {

constexpr int C = kChunk;   // 64
constexpr int NT = 512;     // threads per block, both kernels
constexpr int PQ = kD + 8;  // bf16 pitch of 128-wide rows (16-byte aligned, conflict-free reads)
constexpr int PC = C + 8;   // bf16 pitch of 64-wide rows
constexpr int PF = C + 4;   // fp32 pitch of 64-wide rows (16-byte aligned)

// workspace per chunk, all bf16: W [64][128], U~ [64][128], A [64][64],
// diag(g) Q [64][128] and (diag(g_C/g) K)^T [128][64]
constexpr size_t kWsW = 0, kWsU = (size_t)C * kD * 2, kWsA = 2 * (size_t)C * kD * 2;
constexpr size_t kWsQ = kWsA + (size_t)C * C * 2, kWsK = kWsQ + (size_t)C * kD * 2;
constexpr size_t kWsChunk = kWsK + (size_t)kD * C * 2;   // 73,728 bytes

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // register-promotable across loops

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
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

__device__ __forceinline__ float lo_bf(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

struct PrepSmem {
  union {
    struct {
      uint16_t Q[C * PQ];     // [r][k]
      uint16_t K[C * PQ];     // [j][k]
    } in;
    struct {
      uint16_t W[C * PQ];     // staged W   [r][k]
      uint16_t U[C * PQ];     // staged U~  [r][v]
    } out;
  } u;
  uint16_t Kt[kD * PC];   // [k][j]
  uint16_t Vt[kD * PC];   // [v][j]
  uint16_t A[C * PC];     // masked decayed scores [r][j]
  float L[C * PF];        // strict lower part of (I + L)
  float T[C * PF];        // (I + L)^-1
  float M[3 * 16 * 17];   // block-row partial products
  uint16_t Tw[C * PC];    // T diag(beta g), bf16
  uint16_t Tu[C * PC];    // T diag(beta), bf16
  float lg[C], bt[C];
};

}  // namespace gdc

// ============================================================== kernel 1: per-chunk prep
//
// Thread t stages key channels (2cp, 2cp+1) of tokens [8e, 8e+8) (cp = t % 64,
// e = t / 64): q, k row-major and k, v transposed with 16-byte writes.
__global__ __launch_bounds__(512) void gdn_chunk_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, uint8_t* __restrict__ ws,
    int T) {
  using namespace gdc;
  __shared__ PrepSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int cp = tid & 63, e8 = tid >> 6;
  const int nc = T / C;
  const int n = blockIdx.x / nc, ci = blockIdx.x % nc;
  const size_t tok0 = (size_t)n * T + (size_t)ci * C;
  uint8_t* wsc = ws + (size_t)blockIdx.x * kWsChunk;

  // ---- stage q, k (row-major), k^T and v^T; cumulative log-decays
  {
    unsigned qw[8], kw[8], vw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const size_t off = (tok0 + 8 * e8 + i) * kD + 2 * cp;
      qw[i] = *reinterpret_cast<const unsigned*>(q + off);
      kw[i] = *reinterpret_cast<const unsigned*>(k + off);
      vw[i] = *reinterpret_cast<const unsigned*>(v + off);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * e8 + i;
      *reinterpret_cast<unsigned*>(sm.u.in.Q + r * PQ + 2 * cp) = qw[i];
      *reinterpret_cast<unsigned*>(sm.u.in.K + r * PQ + 2 * cp) = kw[i];
    }
    u32x4 k0, k1, v0, v1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k0[i] = (kw[2 * i] & 0xffffu) | (kw[2 * i + 1] << 16);
      k1[i] = (kw[2 * i] >> 16) | (kw[2 * i + 1] & 0xffff0000u);
      v0[i] = (vw[2 * i] & 0xffffu) | (vw[2 * i + 1] << 16);
      v1[i] = (vw[2 * i] >> 16) | (vw[2 * i + 1] & 0xffff0000u);
    }
    *reinterpret_cast<u32x4*>(sm.Kt + (2 * cp) * PC + 8 * e8) = k0;
    *reinterpret_cast<u32x4*>(sm.Kt + (2 * cp + 1) * PC + 8 * e8) = k1;
    *reinterpret_cast<u32x4*>(sm.Vt + (2 * cp) * PC + 8 * e8) = v0;
    *reinterpret_cast<u32x4*>(sm.Vt + (2 * cp + 1) * PC + 8 * e8) = v1;
  }
  if (wave == 0) {
    sm.lg[lane] = wave_scan(__logf(alpha[tok0 + lane]));
    sm.bt[lane] = beta[tok0 + lane];
  }
  lds_barrier();

  // ---- the sequential pass's decayed operands: diag(g) Q and (diag(g_C/g) K)^T,
  // this thread's key channels (2cp, 2cp+1) of tokens [8e, 8e+8), from LDS
  {
    const float lC = sm.lg[C - 1];
    uint16_t* Qw = reinterpret_cast<uint16_t*>(wsc + kWsQ);
    uint16_t* Kw = reinterpret_cast<uint16_t*>(wsc + kWsK);
    float kh0[8], kh1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * e8 + i;
      const float lr = sm.lg[r];
      const float gr = __expf(lr), kr = __expf(lC - lr);
      const unsigned qw = *reinterpret_cast<const unsigned*>(sm.u.in.Q + r * PQ + 2 * cp);
      const unsigned kw = *reinterpret_cast<const unsigned*>(sm.u.in.K + r * PQ + 2 * cp);
      *reinterpret_cast<unsigned*>(Qw + r * kD + 2 * cp) = pack_bf16(gr * lo_bf(qw), gr * hi_bf(qw));
      kh0[i] = kr * lo_bf(kw);
      kh1[i] = kr * hi_bf(kw);
    }
    u32x4 w0, w1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0[i] = pack_bf16(kh0[2 * i], kh0[2 * i + 1]);
      w1[i] = pack_bf16(kh1[2 * i], kh1[2 * i + 1]);
    }
    *reinterpret_cast<u32x4*>(Kw + (2 * cp) * C + 8 * e8) = w0;
    *reinterpret_cast<u32x4*>(Kw + (2 * cp + 1) * C + 8 * e8) = w1;
  }

  // ---- Gram k.k and scores q.k: wave -> row block (w & 3), column blocks 2(w>>2)+{0,1}
  {
    const int rb = wave & 3;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int cb = 2 * (wave >> 2) + cc;
      f32x4 g = {0.f, 0.f, 0.f, 0.f}, s = {0.f, 0.f, 0.f, 0.f};
      if (cb <= rb) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 kb = ld8(sm.u.in.K + (cb * 16 + l16) * PQ + ks * 32 + lq * 8);
          g = mfma(ld8(sm.u.in.K + (rb * 16 + l16) * PQ + ks * 32 + lq * 8), kb, g);
          s = mfma(ld8(sm.u.in.Q + (rb * 16 + l16) * PQ + ks * 32 + lq * 8), kb, s);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb * 16 + lq * 4 + i, j = cb * 16 + l16;
        const float dec = j <= r ? __expf(sm.lg[r] - sm.lg[j]) : 0.f;
        sm.L[r * PF + j] = j < r ? sm.bt[r] * dec * g[i] : 0.f;
        sm.A[r * PC + j] = f32_to_bf16(dec * s[i]);
      }
    }
  }
  lds_barrier();

  // ---- T = (I + L)^-1: diagonal 16 x 16 blocks, one column per thread, in registers
  if (tid < 64) {
    const int b = tid >> 4, c = tid & 15, o = b * 16;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const f32x4* Lr = reinterpret_cast<const f32x4*>(sm.L + (o + i) * PF + o);
      const f32x4 l0 = Lr[0], l1 = Lr[1], l2 = Lr[2], l3 = Lr[3];
      const float li[16] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w,
                            l2.x, l2.y, l2.z, l2.w, l3.x, l3.y, l3.z, l3.w};
      float s = i == c ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < i; ++j) s -= li[j] * x[j];
      x[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.T[(o + i) * PF + o + c] = x[i];
  }
  for (int e = tid; e < C * C; e += NT) {   // strictly upper blocks are zero
    const int r = e >> 6, c = e & 63;
    if ((c >> 4) > (r >> 4)) sm.T[r * PF + c] = 0.f;
  }
  lds_barrier();
  // block rows I = 1..3: M_J = sum_{K=J}^{I-1} L_IK T_KJ, then T_IJ = -D_I M_J
  for (int I = 1; I < 4; ++I) {
    for (int e = tid; e < I * 256; e += NT) {
      const int J = e >> 8, i = (e >> 4) & 15, j = e & 15;
      float s = 0.f;
      for (int kk = J * 16; kk < I * 16; kk += 4) {
        const f32x4 lv = *reinterpret_cast<const f32x4*>(sm.L + (I * 16 + i) * PF + kk);
        s += lv.x * sm.T[kk * PF + J * 16 + j] + lv.y * sm.T[(kk + 1) * PF + J * 16 + j] +
             lv.z * sm.T[(kk + 2) * PF + J * 16 + j] + lv.w * sm.T[(kk + 3) * PF + J * 16 + j];
      }
      sm.M[J * 272 + i * 17 + j] = s;
    }
    lds_barrier();
    for (int e = tid; e < I * 256; e += NT) {
      const int J = e >> 8, i = (e >> 4) & 15, j = e & 15;
      float s = 0.f;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) s -= sm.T[(I * 16 + i) * PF + I * 16 + kk] * sm.M[J * 272 + kk * 17 + j];
      sm.T[(I * 16 + i) * PF + J * 16 + j] = s;
    }
    lds_barrier();
  }

  // ---- T diag(beta g) and T diag(beta) in bf16 (pairs of columns)
  for (int e = tid; e < C * C / 2; e += NT) {
    const int r = e >> 5, j = 2 * (e & 31);
    const f32x2 t = *reinterpret_cast<const f32x2*>(sm.T + r * PF + j);
    const float b0 = sm.bt[j], b1 = sm.bt[j + 1];
    *reinterpret_cast<unsigned*>(sm.Tw + r * PC + j) =
        pack_bf16(t.x * b0 * __expf(sm.lg[j]), t.y * b1 * __expf(sm.lg[j + 1]));
    *reinterpret_cast<unsigned*>(sm.Tu + r * PC + j) = pack_bf16(t.x * b0, t.y * b1);
  }
  lds_barrier();

  // ---- W = Tw K, U~ = Tu V: wave -> row block (w & 3), column blocks 4(w>>2)..+4; staged
  {
    const int rb = wave & 3;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int cb = 4 * (wave >> 2) + cc;
      f32x4 w = {0.f, 0.f, 0.f, 0.f}, uu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        w = mfma(ld8(sm.Tw + (rb * 16 + l16) * PC + js * 32 + lq * 8),
                 ld8(sm.Kt + (cb * 16 + l16) * PC + js * 32 + lq * 8), w);
        uu = mfma(ld8(sm.Tu + (rb * 16 + l16) * PC + js * 32 + lq * 8),
                  ld8(sm.Vt + (cb * 16 + l16) * PC + js * 32 + lq * 8), uu);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb * 16 + lq * 4 + i, c = cb * 16 + l16;
        sm.u.out.W[r * PQ + c] = f32_to_bf16(w[i]);
        sm.u.out.U[r * PQ + c] = f32_to_bf16(uu[i]);
      }
    }
  }
  lds_barrier();
  // ---- W, U~, A to the workspace with 16-byte stores
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + NT * i, row = p >> 4, seg = p & 15;
    *reinterpret_cast<u32x4*>(wsc + kWsW + (size_t)(row * kD + seg * 8) * 2) =
        *reinterpret_cast<const u32x4*>(sm.u.out.W + row * PQ + seg * 8);
    *reinterpret_cast<u32x4*>(wsc + kWsU + (size_t)(row * kD + seg * 8) * 2) =
        *reinterpret_cast<const u32x4*>(sm.u.out.U + row * PQ + seg * 8);
  }
  {
    const int row = tid >> 3, seg = tid & 7;
    *reinterpret_cast<u32x4*>(wsc + kWsA + (size_t)(row * C + seg * 8) * 2) =
        *reinterpret_cast<const u32x4*>(sm.A + row * PC + seg * 8);
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
  uint16_t Sb[2][VT * PQ]; // bf16 state tile [v][k], double buffered
  uint16_t Ut[VT * PC];    // U^T tile [v][j]
  uint16_t Ob[C * (VT + 8)]; // this chunk's outputs [r][v], stored at the next chunk
};

// Stores the staged outputs of the chunk starting at token tok0: VT / 8 per thread,
// the same single store in every thread.
template <int VT>
__device__ __forceinline__ void store_o(const SeqSmem<VT>& sm, uint16_t* __restrict__ o,
                                        size_t tok0, int v0) {
  constexpr int EPT = VT / 8, OBS = VT + 8;
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const int tid = threadIdx.x, row = tid >> 3, col = (tid & 7) * EPT;
  const uint16_t* src = sm.Ob + row * OBS + col;
  uint16_t* dst = o + (tok0 + row) * kD + v0 + col;
  if constexpr (EPT == 2)
    *reinterpret_cast<unsigned*>(dst) = *reinterpret_cast<const unsigned*>(src);
  else
    *reinterpret_cast<u32x2*>(dst) = *reinterpret_cast<const u32x2*>(src);
}

// One chunk's operands, held in registers while the previous chunk computes: 7
// sixteen-byte pieces per thread of W, A, diag(g) Q and (diag(g_C/g) K)^T (56 KB per
// chunk), alpha of token `lane`, and, for the waves that form U, the raw bf16 U~
// entries in accumulator layout (converting them here would make the compiler wait
// for the loads at once).
struct Prefetch {
  u32x4 w[2], a, qg[2], kh[2];
  float al;
  unsigned short ut[4];
};

template <int VT>
__device__ __forceinline__ void fetch_chunk(Prefetch& pf, const float* __restrict__ alpha,
                                            const uint8_t* __restrict__ ws, int n, int nc, int ci,
                                            int T, int v0) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const size_t tok0 = (size_t)n * T + (size_t)ci * C;
  const uint8_t* wsc = ws + ((size_t)n * nc + ci) * kWsChunk;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const size_t o16 = (size_t)(tid + NT * i) * 16;   // 16-byte piece of a 16 KB tile
    pf.w[i] = *reinterpret_cast<const u32x4*>(wsc + kWsW + o16);
    pf.qg[i] = *reinterpret_cast<const u32x4*>(wsc + kWsQ + o16);
    pf.kh[i] = *reinterpret_cast<const u32x4*>(wsc + kWsK + o16);
  }
  pf.a = *reinterpret_cast<const u32x4*>(wsc + kWsA + (size_t)tid * 16);
  pf.al = alpha[tok0 + lane];
  const int rb = wave & 3, vb = (wave >> 2) & (VT / 16 - 1);   // in bounds for every wave
  const uint16_t* Uw = reinterpret_cast<const uint16_t*>(wsc + kWsU);
#pragma unroll
  for (int i = 0; i < 4; ++i) pf.ut[i] = Uw[(rb * 16 + lq * 4 + i) * kD + v0 + vb * 16 + l16];
}

// One chunk of the sequential pass: starts the loads of the next chunk into `nx`,
// stores the previous chunk's staged outputs, then consumes `pf` (this chunk's
// operands). Every thread issues the same loads and the same store on every chunk
// (the last chunk loads itself again; the first chunk, FIRST, is a separate copy with
// nothing to store), so the wait for `pf` counts exactly the memory operations issued
// after it instead of waiting for them.
template <int VT, bool FIRST>
__device__ __forceinline__ void gdn_seq_chunk(SeqSmem<VT>& sm, Prefetch& pf, Prefetch& nx,
                                              f32x4 (&Sacc)[VT / 16], int& cur, int ci, int nc,
                                              int n, int T, int v0, const float* __restrict__ alpha,
                                              const uint8_t* __restrict__ ws,
                                              uint16_t* __restrict__ o) {
  constexpr int NVB = VT / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int kcol = wave * 16 + l16;
  const size_t tok0 = (size_t)n * T + (size_t)ci * C;
  fetch_chunk<VT>(nx, alpha, ws, n, nc, min(ci + 1, nc - 1), T, v0);
  if constexpr (!FIRST) store_o<VT>(sm, o, tok0 - C, v0);

  // ---- copy this chunk's operands into LDS; g_C from the decays (every wave)
  const float gC = __expf(__shfl(wave_scan(__logf(pf.al)), C - 1));
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + NT * i;
    *reinterpret_cast<u32x4*>(sm.W + (p >> 4) * PQ + (p & 15) * 8) = pf.w[i];
    *reinterpret_cast<u32x4*>(sm.Qg + (p >> 4) * PQ + (p & 15) * 8) = pf.qg[i];
    *reinterpret_cast<u32x4*>(sm.Kht + (p >> 3) * PC + (p & 7) * 8) = pf.kh[i];
  }
  *reinterpret_cast<u32x4*>(sm.A + (tid >> 3) * PC + (tid & 7) * 8) = pf.a;
  f32x4 ut;
#pragma unroll
  for (int i = 0; i < 4; ++i) ut[i] = bf16_to_f32(pf.ut[i]);
  lds_barrier();

  // ---- U = U~ - W S^T: wave -> (row block w & 3, value block w >> 2); to LDS transposed
  if (wave < 4 * NVB) {
    const int rb = wave & 3, vb = wave >> 2;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = mfma(ld8(sm.W + (rb * 16 + l16) * PQ + ks * 32 + lq * 8),
                 ld8(sm.Sb[cur] + (vb * 16 + l16) * PQ + ks * 32 + lq * 8), acc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sm.Ut[(vb * 16 + l16) * PC + rb * 16 + lq * 4 + i] = f32_to_bf16(ut[i] - acc[i]);
  }
  lds_barrier();

  // ---- O = diag(g) Q S^T + A U (same tile assignment)
  if (wave < 4 * NVB) {
    const int rb = wave & 3, vb = wave >> 2;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = mfma(ld8(sm.Qg + (rb * 16 + l16) * PQ + ks * 32 + lq * 8),
                 ld8(sm.Sb[cur] + (vb * 16 + l16) * PQ + ks * 32 + lq * 8), acc);
#pragma unroll
    for (int js = 0; js < 2; ++js)
      if (js * 32 <= rb * 16 + 15)
        acc = mfma(ld8(sm.A + (rb * 16 + l16) * PC + js * 32 + lq * 8),
                   ld8(sm.Ut + (vb * 16 + l16) * PC + js * 32 + lq * 8), acc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sm.Ob[(rb * 16 + lq * 4 + i) * (VT + 8) + vb * 16 + l16] = f32_to_bf16(acc[i]);
  }

  // ---- S <- g_C S + U^T (diag(g_C/g) K): key block = wave; next bf16 copy
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb) {
    f32x4 acc = Sacc[vb] * gC;
#pragma unroll
    for (int js = 0; js < 2; ++js)
      acc = mfma(ld8(sm.Ut + (vb * 16 + l16) * PC + js * 32 + lq * 8),
                 ld8(sm.Kht + (wave * 16 + l16) * PC + js * 32 + lq * 8), acc);
    Sacc[vb] = acc;
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.Sb[cur ^ 1][(vb * 16 + lq * 4 + i) * PQ + kcol] = f32_to_bf16(acc[i]);
  }
  cur ^= 1;
  lds_barrier();
}

}  // namespace gdc

template <int VT>
__global__ __launch_bounds__(512) void gdn_chunk_seq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ alpha,
    const uint8_t* __restrict__ ws, const float* __restrict__ S0, float* __restrict__ ST,
    uint16_t* __restrict__ o, int N, int T) {
  using namespace gdc;
  constexpr int NVB = VT / 16;           // value blocks in the tile
  constexpr int TPS = kD / VT;           // tiles per sequence
  __shared__ SeqSmem<VT> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  // block -> (sequence, value tile); the tiles of one sequence share an XCD (blocks
  // are dealt to the 8 XCDs round robin), so the chunk operands they all read are
  // fetched into that XCD's L2 once
  int n, vt;
  const int bid = blockIdx.x;
  if ((N & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3;
    n = (slot / TPS) * 8 + xcd;
    vt = slot % TPS;
  } else {
    n = bid / TPS;
    vt = bid % TPS;
  }
  const int v0 = vt * VT;
  const int nc = T / C;
  const int kcol = wave * 16 + l16;      // key column of this wave's state tiles

  // state tiles: key block = wave, value blocks vb < NVB; lane holds
  // S[v0 + vb*16 + lq*4 + i][kcol]
  f32x4 Sacc[NVB];
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Sacc[vb][i] = S0 ? S0[((size_t)n * kD + v0 + vb * 16 + lq * 4 + i) * kD + kcol] : 0.f;
      sm.Sb[0][(vb * 16 + lq * 4 + i) * PQ + kcol] = f32_to_bf16(Sacc[vb][i]);
    }

  if (nc > 0) {
    Prefetch pa, pb;
    int cur = 0;
    fetch_chunk<VT>(pa, alpha, ws, n, nc, 0, T, v0);
    gdn_seq_chunk<VT, true>(sm, pa, pb, Sacc, cur, 0, nc, n, T, v0, alpha, ws, o);
    int ci = 1;
    for (; ci + 1 < nc; ci += 2) {
      gdn_seq_chunk<VT, false>(sm, pb, pa, Sacc, cur, ci, nc, n, T, v0, alpha, ws, o);
      gdn_seq_chunk<VT, false>(sm, pa, pb, Sacc, cur, ci + 1, nc, n, T, v0, alpha, ws, o);
    }
    if (ci < nc) gdn_seq_chunk<VT, false>(sm, pb, pa, Sacc, cur, ci, nc, n, T, v0, alpha, ws, o);
    store_o<VT>(sm, o, (size_t)n * T + (size_t)(nc - 1) * C, v0);
  }

#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ST[((size_t)n * kD + v0 + vb * 16 + lq * 4 + i) * kD + kcol] = Sacc[vb][i];
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
    hipLaunchKernelGGL(gdn_chunk_prep_kernel, dim3((unsigned)(N * (T / kChunk))), dim3(gdc::NT), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), alpha, beta, ws, T);
    int rc = check_launch("gdn_chunk_fwd (prep)");
    if (rc != GDNRT_OK) return rc;
  }
  // value tiles of 16 when there are too few sequences to fill the chip with 32
  if (N * 4 < 256)
    hipLaunchKernelGGL((gdn_chunk_seq_kernel<16>), dim3((unsigned)(N * 8)), dim3(gdc::NT), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), alpha, ws,
                       S0, ST, static_cast<uint16_t*>(o), N, T);
  else
    hipLaunchKernelGGL((gdn_chunk_seq_kernel<32>), dim3((unsigned)(N * 4)), dim3(gdc::NT), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), alpha, ws,
                       S0, ST, static_cast<uint16_t*>(o), N, T);
  return check_launch("gdn_chunk_fwd");
}

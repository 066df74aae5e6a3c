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
// Substituting U into O gives O = Q' S_0^T + O~ with Q' = diag(g) Q - A W and
// O~ = A U~: the outputs of a chunk need only the state the chunk starts from, not
// this chunk's U. Everything but S_0 (W, U~, Q', O~, K^ = diag(g_C/g) K, g_C) is
// formed for every chunk in parallel by a first kernel and written, bf16, to the
// caller's workspace in the exact register order in which the second kernel feeds
// them to the matrix cores. The second kernel walks the chunks of each sequence in
// order for a tile of value channels (the value rows of U and S are independent):
// per chunk, four waves form U = U~ - W S_0^T while the other four form the outputs,
// then all eight update the state, S_C = g_C S_0 + U^T K^, which stays in fp32 MFMA
// accumulators; the operands of the next chunk are loaded straight into registers
// meanwhile. bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation throughout;
// the triangular inverse is fp32 (16 x 16 diagonal blocks by substitution, the
// blocks below by v_mfma_f32_16x16x4_f32).
#include "common.hpp"
#include "gdn_chunk_layout.hpp"
#include "chunk_device.hpp"

namespace gdnrt {

namespace gdc {

// Workspace per chunk: gdn_chunk_layout.hpp (kWsW .. kWsChunk).
// KDA: the chunk's state decay is a vector over key channels (128 fp32 at kWsG)
constexpr size_t kWsChunkKda = kWsG + kD * 4;
template <bool KDA>
constexpr size_t ws_chunk() { return KDA ? kWsChunkKda : kWsChunk; }

// LDS of the KDA prep (one block per CU)
struct alignas(16) PrepSmem {
  uint16_t Q[C * PQ];       // [r][k]
  uint16_t K[C * PQ];       // [j][k]
  uint16_t V[C * PQ];       // [j][v]
  uint16_t A[C * PC];       // masked decayed scores [r][j]
  union {
    float L[C * PF];        // strict lower part of (I + L), fp32
    uint16_t Wt[kD * PC];   // W^T [k][j]
  } rl;
  union {
    float T[C * PF];        // (I + L)^-1, lower blocks
    uint16_t Ut[kD * PC];   // U~^T [v][j]
  } rt;
  union {
    float scr[8][16 * 17];  // one 16 x 16 fp32 tile per wave (inverse)
    struct {
      uint16_t Tw[C * PC];  // T diag(beta) (the decays are inside the key operand K o Gamma)
      uint16_t Tu[C * PC];  // T diag(beta)
    } t;
  } rw;
  float bt[C], btg[C];      // beta, and beta again as the W factor
};

// one chunk's inputs for this thread: 16-byte pieces p = tid + 512 h (h = 0, 1) of
// q, k, v (token p >> 4, channels 8 (p & 15) ..), and alpha, beta of token tid % 64
// KDA: the per-channel decays of tokens 4 (tid >> 5) .. + 3, channels 4 (tid & 31) .. + 3
template <bool KDA>
struct PrepIn {
  u32x4 q[2], k[2], v[2];
  float al, be;
  f32x4 a4[KDA ? 4 : 1];
};

template <bool KDA>
__device__ __forceinline__ void prep_fetch(PrepIn<KDA>& in, const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ k,
                                           const uint16_t* __restrict__ v,
                                           const float* __restrict__ alpha,
                                           const float* __restrict__ beta, size_t tok0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = tid + NT * h;
    const size_t off = (tok0 + (p >> 4)) * kD + (p & 15) * 8;
    in.q[h] = *reinterpret_cast<const u32x4*>(q + off);
    in.k[h] = *reinterpret_cast<const u32x4*>(k + off);
    in.v[h] = *reinterpret_cast<const u32x4*>(v + off);
  }
  if constexpr (KDA) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      in.a4[i] = *reinterpret_cast<const f32x4*>(alpha + (tok0 + 4 * (tid >> 5) + i) * kD + 4 * (tid & 31));
  } else {
    in.al = alpha[tok0 + (tid & 63)];
  }
  in.be = beta[tok0 + (tid & 63)];
}

// A use of every input request of a block's last chunk at the end of the kernel. Those
// requests (the last chunk loads itself again) are otherwise dead on the way out, and
// the compiler then sinks the first chunk's requests below that chunk's stores into the
// loop's preheader; the loop's first wait, counting for both ways in, then also waits
// for most of the previous chunk's stores on every chunk.
template <bool KDA>
__device__ __forceinline__ void keep_inputs(const PrepIn<KDA>& in) {
  unsigned s = __float_as_uint(in.be);
#pragma unroll
  for (int h = 0; h < 2; ++h) s ^= in.q[h].x ^ in.k[h].x ^ in.v[h].x;
  if constexpr (KDA) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s ^= __float_as_uint(in.a4[i][0]);
  } else {
    s ^= __float_as_uint(in.al);
  }
  asm volatile("" ::"v"(s));
}

// KDA: the extra LDS of the prep. Km = K o exp(b_m - b) (bf16, the second operand of
// the Gram matrix and the scores), per-group totals of the cumulative log-decays and
// per-channel exp(b_m), exp(b_C - b_m), b_m the cumulative log-decay at token 31.
struct alignas(16) KdaPrepSmem {
  uint16_t Km[C * PQ];
  float tot[16][kD];
  float em[kD], ecm[kD];
};


}  // namespace gdc

namespace gdc {

// One chunk of the KDA prep (one block per CU): stages the inputs held in `in`, requests
// the next chunk's into `in`, and writes the chunk's operands to the workspace.
__device__ __forceinline__ void kda_prep_chunk(PrepSmem& sm, KdaPrepSmem& xs, PrepIn<true>& in, int cid,
                                               const uint16_t* __restrict__ q,
                                               const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                               const float* __restrict__ alpha, const float* __restrict__ beta,
                                               uint8_t* __restrict__ ws, int T, int nchunks) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int nc = T / C;
  uint8_t* wsc = ws + (size_t)cid * kWsChunkKda;

  // ---- stage q, k, v (row-major); decays
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = tid + NT * h, o = (p >> 4) * PQ + (p & 15) * 8;
    *reinterpret_cast<u32x4*>(sm.Q + o) = in.q[h];
    *reinterpret_cast<u32x4*>(sm.K + o) = in.k[h];
    *reinterpret_cast<u32x4*>(sm.V + o) = in.v[h];
  }
  // cumulative log-decays of this thread's 4 tokens x 4 channels, within its group
  f32x4 pre[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 a = in.a4[i];
    const f32x4 la = {__logf(a.x), __logf(a.y), __logf(a.z), __logf(a.w)};
    pre[i] = i == 0 ? la : pre[i - 1] + la;
  }
  *reinterpret_cast<f32x4*>(&xs.tot[tid >> 5][4 * (tid & 31)]) = pre[3];
  if (wave == 0) {
    sm.bt[lane] = in.be;
    sm.btg[lane] = in.be;   // the decays sit in the key operand of W
  }
  // next chunk's inputs (the last chunk of a block loads itself again)
  {
    const int nx = cid + (int)gridDim.x < nchunks ? cid + (int)gridDim.x : cid;
    prep_fetch<true>(in, q, k, v, alpha, beta, (size_t)(nx / nc) * T + (size_t)(nx % nc) * C);
  }
  // b = cumulative log-decay per channel; with b_m its value at token 31 (the middle),
  // Q <- Q o exp(b - b_m), K <- K o exp(b - b_m), Km = K o exp(b_m - b): the Gram
  // matrix and the scores then carry exp(b_r - b_j) inside their products, and no
  // factor exceeds exp(32 max|log alpha|)
  lds_barrier();
  const int tq = tid >> 5, c0 = 4 * (tid & 31);
  f32x4 base = {0.f, 0.f, 0.f, 0.f}, bm = {0.f, 0.f, 0.f, 0.f}, bC = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    const f32x4 t4 = *reinterpret_cast<const f32x4*>(&xs.tot[g][c0]);
    if (g < tq) base += t4;
    if (g < 8) bm += t4;
    bC += t4;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 4 * tq + i;
    const f32x4 b = base + pre[i];
    f32x4 fp, fm;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      fp[e] = __expf(b[e] - bm[e]);
      fm[e] = __expf(bm[e] - b[e]);
    }
    u32x2* qp = reinterpret_cast<u32x2*>(sm.Q + t * PQ + c0);
    u32x2* kp = reinterpret_cast<u32x2*>(sm.K + t * PQ + c0);
    const u32x2 qw = *qp, kw = *kp;
    *qp = u32x2{pack_bf16(lo_bf(qw.x) * fp[0], hi_bf(qw.x) * fp[1]), pack_bf16(lo_bf(qw.y) * fp[2], hi_bf(qw.y) * fp[3])};
    *kp = u32x2{pack_bf16(lo_bf(kw.x) * fp[0], hi_bf(kw.x) * fp[1]), pack_bf16(lo_bf(kw.y) * fp[2], hi_bf(kw.y) * fp[3])};
    *reinterpret_cast<u32x2*>(xs.Km + t * PQ + c0) =
        u32x2{pack_bf16(lo_bf(kw.x) * fm[0], hi_bf(kw.x) * fm[1]), pack_bf16(lo_bf(kw.y) * fm[2], hi_bf(kw.y) * fm[3])};
  }
  if (tq == 0) {
    f32x4 em, ecm, gc;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      em[e] = __expf(bm[e]);
      ecm[e] = __expf(bC[e] - bm[e]);
      gc[e] = __expf(bC[e]);
    }
    *reinterpret_cast<f32x4*>(&xs.em[c0]) = em;
    *reinterpret_cast<f32x4*>(&xs.ecm[c0]) = ecm;
    *reinterpret_cast<f32x4*>(wsc + kWsG + c0 * 4) = gc;
  }
  lds_barrier();

  // ---- K^ fragments (kb, js) = (f >> 1, f & 1), f = wave + 8 h, to the workspace:
  // K^ = Km o exp(b_C - b_m), one channel per lane
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int f = wave + 8 * h, j0 = (f & 1) * 32 + lq * 8;
    u32x4 w;
    const u32x4 raw = __builtin_bit_cast(u32x4, ld_tr8(xs.Km, PQ, (f & 1) * 32, (f >> 1) * 16));
    const float fc = xs.ecm[(f >> 1) * 16 + l16];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16(lo_bf(raw[e]) * fc, hi_bf(raw[e]) * fc);
    *reinterpret_cast<u32x4*>(wsc + kWsK + ((size_t)f * 64 + lane) * 16) = w;
  }
  // ---- Gram k.k -> L and scores q.k -> A: 20 tile products over the lower triangle,
  // up to three per wave, their products issued together (tile index uniform per wave)
  {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    f32x4 acc[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int u = wv + 8 * t;
      acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (u < 20) {
        int rb, cb;
        tri_pair(u >> 1, rb, cb);
        const uint16_t* X = (u & 1) ? sm.Q : sm.K;
        const uint16_t* Y = xs.Km;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc[t] = mfma(ld8(X + (rb * 16 + l16) * PQ + kk * 32 + lq * 8),
                        ld8(Y + (cb * 16 + l16) * PQ + kk * 32 + lq * 8), acc[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int u = wv + 8 * t;
      if (u < 20) {
        int rb, cb;
        tri_pair(u >> 1, rb, cb);
        const int j = cb * 16 + l16, r0 = rb * 16 + lq * 4;
        f32x4 val;
        // the decay is already inside the product; above the diagonal the product is
        // not a decayed one, so it is dropped by selection, never multiplied by 0
#pragma unroll
        for (int i = 0; i < 4; ++i) val[i] = j <= r0 + i ? acc[t][i] : 0.f;
        if (u & 1) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sm.A[(r0 + i) * PC + j] = f32_to_bf16(val[i]);
        } else {
          const f32x4 bt = *reinterpret_cast<const f32x4*>(sm.bt + r0);
#pragma unroll
          for (int i = 0; i < 4; ++i) sm.rl.L[(r0 + i) * PF + j] = j < r0 + i ? bt[i] * val[i] : 0.f;
        }
      }
    }
  }
  {   // the zero upper tiles that the 32-wide contraction slices of A reach: (0,1), (2,3)
    const int t = tid >> 8, e = tid & 255;
    sm.A[(t * 32 + (e >> 4)) * PC + t * 32 + 16 + (e & 15)] = 0;
  }
  lds_barrier();
  {   // K <- K o exp(b) (the key operand of W), this thread's 4 x 4 block
    const f32x4 em = *reinterpret_cast<const f32x4*>(&xs.em[c0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2* kp = reinterpret_cast<u32x2*>(sm.K + (4 * tq + i) * PQ + c0);
      const u32x2 kw = *kp;
      *kp = u32x2{pack_bf16(lo_bf(kw.x) * em[0], hi_bf(kw.x) * em[1]), pack_bf16(lo_bf(kw.y) * em[2], hi_bf(kw.y) * em[3])};
    }
  }

  // ---- T = (I + L)^-1. Diagonal blocks: wave w -> block w >> 1, columns
  // (w & 1) * 8 + 2 * (lane >> 4) + {0, 1}; lane & 15 is the row.
  {
    const int b = wave >> 1, i = l16;
    const int c0 = (wave & 1) * 8 + 2 * lq, c1 = c0 + 1;
    float lr[16];
    const f32x4* Lrow = reinterpret_cast<const f32x4*>(sm.rl.L + (b * 16 + i) * PF + b * 16);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f32x4 x = Lrow[s];
      lr[4 * s] = x.x; lr[4 * s + 1] = x.y; lr[4 * s + 2] = x.z; lr[4 * s + 3] = x.w;
    }
    float a0 = i == c0 ? 1.f : 0.f, a1 = i == c1 ? 1.f : 0.f;
    DiagSolve<0>::run(lr, a0, a1);
    sm.rt.T[(b * 16 + i) * PF + b * 16 + c0] = a0;
    sm.rt.T[(b * 16 + i) * PF + b * 16 + c1] = a1;
  }
  lds_barrier();
  // Blocks below the diagonal, by distance d = I - J:
  //   T_IJ = -D_I sum_{K=J}^{I-1} L_IK T_KJ   (D_I = T_II), wave J for J < 4 - d
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (wave < 4 - d) {
      const int J = wave, I = J + d;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      for (int K = J; K < I; ++K)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          x = mfma4(sm.rl.L[(I * 16 + l16) * PF + K * 16 + 4 * s + lq],
                    sm.rt.T[(K * 16 + 4 * s + lq) * PF + J * 16 + l16], x);
      float* scr = sm.rw.scr[wave];
#pragma unroll
      for (int i = 0; i < 4; ++i) scr[(4 * lq + i) * 17 + l16] = x[i];
      wave_lds_sync();
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        y = mfma4(sm.rt.T[(I * 16 + l16) * PF + I * 16 + 4 * s + lq], scr[(4 * s + lq) * 17 + l16], y);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.rt.T[(I * 16 + 4 * lq + i) * PF + J * 16 + l16] = -y[i];
    }
    lds_barrier();
  }

  // ---- T diag(beta g) and T diag(beta) in bf16 (zero above the diagonal blocks):
  // thread -> row tid / 8, columns 8 (tid % 8) .. + 7
  {
    const int r = tid >> 3, j0 = (tid & 7) * 8;
    f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = t0;
    if ((j0 >> 4) <= (r >> 4)) {
      t0 = *reinterpret_cast<const f32x4*>(sm.rt.T + r * PF + j0);
      t1 = *reinterpret_cast<const f32x4*>(sm.rt.T + r * PF + j0 + 4);
    }
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(sm.btg + j0), g1 = *reinterpret_cast<const f32x4*>(sm.btg + j0 + 4);
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(sm.bt + j0), b1 = *reinterpret_cast<const f32x4*>(sm.bt + j0 + 4);
    const f32x4 w0 = t0 * g0, w1 = t1 * g1, u0 = t0 * b0, u1 = t1 * b1;
    *reinterpret_cast<u32x4*>(sm.rw.t.Tw + r * PC + j0) =
        u32x4{pack_bf16(w0.x, w0.y), pack_bf16(w0.z, w0.w), pack_bf16(w1.x, w1.y), pack_bf16(w1.z, w1.w)};
    *reinterpret_cast<u32x4*>(sm.rw.t.Tu + r * PC + j0) =
        u32x4{pack_bf16(u0.x, u0.y), pack_bf16(u0.z, u0.w), pack_bf16(u1.x, u1.y), pack_bf16(u1.z, u1.w)};
  }
  lds_barrier();

  // ---- W = Tw K (to LDS as W^T), W^T fragments and U~ = Tu V (workspace, U~^T to LDS).
  // Row block rb only reaches tokens j <= 16 rb + 15: contraction slices js <= rb / 2.
  {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {   // W tile (rb, kb = wave) -> W^T [k][j]
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int js = 0; js <= rb / 2; ++js)
        acc = mfma(ld8(sm.rw.t.Tw + (rb * 16 + l16) * PC + js * 32 + lq * 8),
                   ld_tr8(sm.K, PQ, js * 32, wave * 16), acc);
      *reinterpret_cast<u32x2*>(sm.rl.Wt + (wave * 16 + l16) * PC + rb * 16 + lq * 4) =
          u32x2{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {      // W^T fragments (rb, ks): rb pairs {0,3}, {1,2}
      const int rb = h ? 3 - (wave & 3) : (wave & 3), ks = (wave >> 2) + 2 * h;
      f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
      for (int js = 0; js <= rb / 2; ++js) {
        const bf16x8 b = ld8(sm.rw.t.Tw + (rb * 16 + l16) * PC + js * 32 + lq * 8);
        t0 = mfma(ld_tr8(sm.K, PQ, js * 32, ks * 32), b, t0);
        t1 = mfma(ld_tr8(sm.K, PQ, js * 32, ks * 32 + 16), b, t1);
      }
      *reinterpret_cast<u32x4*>(wsc + kWsW + ((size_t)(rb * 4 + ks) * 64 + lane) * 16) =
          u32x4{pack_bf16(t0[0], t0[1]), pack_bf16(t0[2], t0[3]), pack_bf16(t1[0], t1[1]),
                pack_bf16(t1[2], t1[3])};
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {   // U~ tile (rb, vb = wave)
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int js = 0; js <= rb / 2; ++js)
        acc = mfma(ld8(sm.rw.t.Tu + (rb * 16 + l16) * PC + js * 32 + lq * 8),
                   ld_tr8(sm.V, PQ, js * 32, wave * 16), acc);
      const u32x2 p = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
      *reinterpret_cast<u32x2*>(wsc + kWsU + ((size_t)(rb * 8 + wave) * 64 + lane) * 8) = p;
      *reinterpret_cast<u32x2*>(sm.rt.Ut + (wave * 16 + l16) * PC + rb * 16 + lq * 4) = p;
    }
  }
  lds_barrier();

  // ---- Q'^T = (diag(g) Q)^T - W^T A^T as fragments; O~ = A U~ tiles
  {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rb = h ? 3 - (wave & 3) : (wave & 3), ks = (wave >> 2) + 2 * h;
      f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
      for (int js = 0; js <= rb / 2; ++js) {
        const bf16x8 b = ld8(sm.A + (rb * 16 + l16) * PC + js * 32 + lq * 8);
        t0 = mfma(ld8(sm.rl.Wt + (ks * 32 + l16) * PC + js * 32 + lq * 8), b, t0);
        t1 = mfma(ld8(sm.rl.Wt + (ks * 32 + 16 + l16) * PC + js * 32 + lq * 8), b, t1);
      }
      const int r = rb * 16 + l16;
      const u32x2 qa = *reinterpret_cast<const u32x2*>(sm.Q + r * PQ + ks * 32 + lq * 4);
      const u32x2 qb = *reinterpret_cast<const u32x2*>(sm.Q + r * PQ + ks * 32 + 16 + lq * 4);
      // exp(b_m) per channel (Q holds Q o exp(b - b_m))
      const f32x4 fa = *reinterpret_cast<const f32x4*>(&xs.em[ks * 32 + lq * 4]);
      const f32x4 fb = *reinterpret_cast<const f32x4*>(&xs.em[ks * 32 + 16 + lq * 4]);
      *reinterpret_cast<u32x4*>(wsc + kWsQ + ((size_t)(rb * 4 + ks) * 64 + lane) * 16) =
          u32x4{pack_bf16(fa[0] * lo_bf(qa.x) - t0[0], fa[1] * hi_bf(qa.x) - t0[1]),
                pack_bf16(fa[2] * lo_bf(qa.y) - t0[2], fa[3] * hi_bf(qa.y) - t0[3]),
                pack_bf16(fb[0] * lo_bf(qb.x) - t1[0], fb[1] * hi_bf(qb.x) - t1[1]),
                pack_bf16(fb[2] * lo_bf(qb.y) - t1[2], fb[3] * hi_bf(qb.y) - t1[3])};
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {   // O~ tile (rb, vb = wave)
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int js = 0; js <= rb / 2; ++js)
        acc = mfma(ld8(sm.A + (rb * 16 + l16) * PC + js * 32 + lq * 8),
                   ld8(sm.rt.Ut + (wave * 16 + l16) * PC + js * 32 + lq * 8), acc);
      *reinterpret_cast<u32x2*>(wsc + kWsO + ((size_t)(rb * 8 + wave) * 64 + lane) * 8) =
          u32x2{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
    }
  }
  lds_barrier();
}

}  // namespace gdc

// ------------------------------------------------------------------ per-chunk prep, GDN, two blocks per CU
// The GDN prep, laid out to fit two blocks in a CU's LDS (75,776 bytes): only the ten
// lower 16 x 16 blocks of L and T are kept; v waits in registers and is staged over k
// once W is formed; W and U~ stay in
// registers as accumulator tiles and enter the Q'^T and O~ products directly as the
// operands of v_mfma_f32_16x16x16_bf16, whose A and B lanes hold four consecutive
// rows of a 16 x 16 block, as an accumulator tile does.
namespace gdc {

struct alignas(16) Prep2Smem {
  uint16_t Q[C * PQ];    // q rows [t][k]
  uint16_t KV[C * PS];   // k rows [t][k]; once W is formed, v rows [t][v] (stored with swz)
  uint16_t A[C * PC];    // masked decayed scores [r][j]
  union {
    struct {
      float L[10][16 * PL];     // strict lower part of (I + L), lower blocks
      float scr[8][16 * PL];    // one 16 x 16 fp32 tile per wave (inverse)
    } inv;
    struct {
      uint16_t Tw[C * PC];      // T diag(beta g)
      uint16_t Tu[C * PC];      // T diag(beta)
    } t;
  } u;
  float T[10][16 * PL];         // (I + L)^-1, lower blocks
  float lg[C], g[C], kd[C], bt[C], btg[C];   // log g, g, g_C/g, beta, beta g
};

template <bool STORE_T>
__device__ __forceinline__ void prep2_chunk(Prep2Smem& sm, PrepIn<false>& in, int cid,
                                            const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                            const uint16_t* __restrict__ v, const float* __restrict__ alpha,
                                            const float* __restrict__ beta, uint8_t* __restrict__ ws,
                                            uint16_t* __restrict__ Tout, int T, int nchunks) {
  // the thread index passed through an opaque move, so that the many per-lane LDS
  // addresses are formed inside each chunk instead of being held across the loop
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int nc = T / C;
  uint8_t* wsc = ws + (size_t)cid * kWsChunk;

  // ---- stage q, k (row-major); v stays in registers until the keys are done; decays
  u32x4 vcur[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = tid + NT * h, o = (p >> 4) * PQ + (p & 15) * 8;
    *reinterpret_cast<u32x4*>(sm.Q + o) = in.q[h];
    *reinterpret_cast<u32x4*>(sm.KV + sw_off(p >> 4, (p & 15) * 8)) = in.k[h];
    vcur[h] = in.v[h];
  }
  {
    const float lgv = wave_scan(__logf(in.al));
    const float lC = __shfl(lgv, C - 1);
    if (wave == 0) {
      const float gv = __expf(lgv);
      sm.lg[lane] = lgv;
      sm.g[lane] = gv;
      sm.kd[lane] = __expf(lC - lgv);
      sm.bt[lane] = in.be;
      sm.btg[lane] = in.be * gv;
    }
    *reinterpret_cast<float*>(wsc + kWsG + (lane & 15) * 4) = __expf(lC);
  }
  lds_barrier();

  // ---- K^ fragments (kb, js) = (f >> 1, f & 1), f = wave + 8 h, to the workspace
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int f = wave + 8 * h, j0 = (f & 1) * 32 + lq * 8;
    const u32x4 raw = __builtin_bit_cast(u32x4, ld_tr8s(sm.KV, (f & 1) * 32, (f >> 1) * 16));
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = pack_bf16(lo_bf(raw[e]) * sm.kd[j0 + 2 * e], hi_bf(raw[e]) * sm.kd[j0 + 2 * e + 1]);
    *reinterpret_cast<u32x4*>(wsc + kWsK + ((size_t)f * 64 + lane) * 16) = w;
  }
  // ---- Gram k.k -> L (lower blocks) and scores q.k -> A: 20 tile products, up to
  // three per wave, one at a time (the other block on the CU hides their latency)
  {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll 1
    for (int u = wv; u < 20; u += 8) {
      int rb, cb;
      tri_pair(u >> 1, rb, cb);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 xa = (u & 1) ? ld8(sm.Q + (rb * 16 + l16) * PQ + kk * 32 + lq * 8)
                                  : ld8(sm.KV + sw_off(rb * 16 + l16, kk * 32 + lq * 8));
        acc = mfma(xa, ld8(sm.KV + sw_off(cb * 16 + l16, kk * 32 + lq * 8)), acc);
      }
      const int j = cb * 16 + l16, r0 = rb * 16 + lq * 4;
      const f32x4 lgr = *reinterpret_cast<const f32x4*>(sm.lg + r0);
      const float lgj = sm.lg[j];
      f32x4 val;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = __expf(lgr[i] - lgj) * acc[i];   // g_r / g_j for j <= r
        val[i] = j <= r0 + i ? x : 0.f;
      }
      if (u & 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.A[(r0 + i) * PC + j] = f32_to_bf16(val[i]);
      } else {
        const f32x4 bt = *reinterpret_cast<const f32x4*>(sm.bt + r0);
        float* Lb = sm.u.inv.L[u >> 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) Lb[(lq * 4 + i) * PL + l16] = j < r0 + i ? bt[i] * val[i] : 0.f;
      }
    }
  }
  lds_barrier();

  // ---- T = (I + L)^-1. Diagonal blocks: wave w -> block w >> 1, columns
  // (w & 1) * 8 + 2 * (lane >> 4) + {0, 1}; lane & 15 is the row.
  {
    const int b = wave >> 1, i = l16;
    const int c0 = (wave & 1) * 8 + 2 * lq, c1 = c0 + 1;
    float lr[16];
    const float* Lrow = sm.u.inv.L[tri(b, b)] + i * PL;
#pragma unroll
    for (int s = 0; s < 16; ++s) lr[s] = Lrow[s];
    float a0 = i == c0 ? 1.f : 0.f, a1 = i == c1 ? 1.f : 0.f;
    DiagSolve<0>::run(lr, a0, a1);
    sm.T[tri(b, b)][i * PL + c0] = a0;
    sm.T[tri(b, b)][i * PL + c1] = a1;
  }
  lds_barrier();
  // Blocks below the diagonal, by distance d = I - J:
  //   T_IJ = -D_I sum_{K=J}^{I-1} L_IK T_KJ   (D_I = T_II), wave J for J < 4 - d
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (wave < 4 - d) {
      const int J = wave, I = J + d;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      for (int K = J; K < I; ++K) {
        const float* Lb = sm.u.inv.L[tri(I, K)];
        const float* Tb = sm.T[tri(K, J)];
#pragma unroll
        for (int s = 0; s < 4; ++s) x = mfma4(Lb[l16 * PL + 4 * s + lq], Tb[(4 * s + lq) * PL + l16], x);
      }
      float* scr = sm.u.inv.scr[wave];
#pragma unroll
      for (int i = 0; i < 4; ++i) scr[(4 * lq + i) * PL + l16] = x[i];
      wave_lds_sync();
      const float* Dg = sm.T[tri(I, I)];
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) y = mfma4(Dg[l16 * PL + 4 * s + lq], scr[(4 * s + lq) * PL + l16], y);
      float* Tb = sm.T[tri(I, J)];
#pragma unroll
      for (int i = 0; i < 4; ++i) Tb[(4 * lq + i) * PL + l16] = -y[i];
    }
    lds_barrier();
  }

  // ---- T diag(beta g) and T diag(beta) in bf16 (zero above the diagonal blocks), over
  // the inverse's L and scratch: thread -> row tid / 8, columns 8 (tid % 8) .. + 7
  {
    const int r = tid >> 3, j0 = (tid & 7) * 8;
    const bool low = (j0 >> 4) <= (r >> 4);
    const float* tb = sm.T[tri(r >> 4, low ? (j0 >> 4) : (r >> 4))] + (r & 15) * PL + (j0 & 15);
    float tt[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) tt[e] = low ? tb[e] : 0.f;
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(sm.btg + j0), g1 = *reinterpret_cast<const f32x4*>(sm.btg + j0 + 4);
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(sm.bt + j0), b1 = *reinterpret_cast<const f32x4*>(sm.bt + j0 + 4);
    *reinterpret_cast<u32x4*>(sm.u.t.Tw + r * PC + j0) =
        u32x4{pack_bf16(tt[0] * g0.x, tt[1] * g0.y), pack_bf16(tt[2] * g0.z, tt[3] * g0.w),
              pack_bf16(tt[4] * g1.x, tt[5] * g1.y), pack_bf16(tt[6] * g1.z, tt[7] * g1.w)};
    *reinterpret_cast<u32x4*>(sm.u.t.Tu + r * PC + j0) =
        u32x4{pack_bf16(tt[0] * b0.x, tt[1] * b0.y), pack_bf16(tt[2] * b0.z, tt[3] * b0.w),
              pack_bf16(tt[4] * b1.x, tt[5] * b1.y), pack_bf16(tt[6] * b1.z, tt[7] * b1.w)};
    if constexpr (STORE_T) {   // T itself for the backward, bf16 [r][j], zero above the diagonal
#pragma unroll
      for (int e = 0; e < 8; ++e) tt[e] = j0 + e <= r ? tt[e] : 0.f;
      *reinterpret_cast<u32x4*>(Tout + (size_t)cid * C * C + r * C + j0) =
          u32x4{pack_bf16(tt[0], tt[1]), pack_bf16(tt[2], tt[3]), pack_bf16(tt[4], tt[5]), pack_bf16(tt[6], tt[7])};
    }
  }
  lds_barrier();

  // ---- W = Tw K: tiles (rb, kb = wave) kept in registers (bf16, as the A operands of
  // the Q'^T products); W^T fragments (rb, ks) to the workspace. Row block rb only
  // reaches tokens j <= 16 rb + 15.
  s16x4 wa[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int js = 0; js <= rb / 2; ++js)
      acc = mfma(ld8(sm.u.t.Tw + (rb * 16 + l16) * PC + js * 32 + lq * 8), ld_tr8s(sm.KV, js * 32, wave * 16), acc);
    wa[rb] = bf4(acc);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {      // W^T fragments (rb, ks): rb pairs {0,3}, {1,2}
    const int rb = h ? 3 - (wave & 3) : (wave & 3), ks = (wave >> 2) + 2 * h;
    f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
    for (int js = 0; js <= rb / 2; ++js) {
      const bf16x8 b = ld8(sm.u.t.Tw + (rb * 16 + l16) * PC + js * 32 + lq * 8);
      t0 = mfma(ld_tr8s(sm.KV, js * 32, ks * 32), b, t0);
      t1 = mfma(ld_tr8s(sm.KV, js * 32, ks * 32 + 16), b, t1);
    }
    *reinterpret_cast<u32x4*>(wsc + kWsW + ((size_t)(rb * 4 + ks) * 64 + lane) * 16) =
        u32x4{pack_bf16(t0[0], t0[1]), pack_bf16(t0[2], t0[3]), pack_bf16(t1[0], t1[1]), pack_bf16(t1[2], t1[3])};
  }
  lds_barrier();

  // ---- v over k, then the next chunk's inputs are requested (the last chunk of a block
  // loads itself again); U~ = Tu V: tiles (rb, vb = wave) to the workspace and kept
  // (bf16, as the B operands of the O~ products)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = tid + NT * h;
    *reinterpret_cast<u32x4*>(sm.KV + sw_off(p >> 4, (p & 15) * 8)) = vcur[h];
  }
  {
    const int nx = cid + (int)gridDim.x < nchunks ? cid + (int)gridDim.x : cid;
    prep_fetch<false>(in, q, k, v, alpha, beta, (size_t)(nx / nc) * T + (size_t)(nx % nc) * C);
  }
  lds_barrier();
  s16x4 ub[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int js = 0; js <= rb / 2; ++js)
      acc = mfma(ld8(sm.u.t.Tu + (rb * 16 + l16) * PC + js * 32 + lq * 8), ld_tr8s(sm.KV, js * 32, wave * 16), acc);
    const u32x2 pk = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
    *reinterpret_cast<u32x2*>(wsc + kWsU + ((size_t)(rb * 8 + wave) * 64 + lane) * 8) = pk;
    ub[rb] = __builtin_bit_cast(s16x4, pk);
  }

  // ---- Q'^T tiles (key block kb = wave, token block rb): g_r Q[r][key] minus
  // sum_{j <= r} W[j][key] A[r][j], with the W tiles as A operands (lane: key l16, four
  // tokens) and A read as B operands; each tile is one half of the Q' fragments
  // (rb, kb / 2), written as 8 of each lane's 16 bytes.
  {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jb = 0; jb <= rb; ++jb) acc = mfma16(wa[jb], ld4(sm.A + (rb * 16 + l16) * PC + jb * 16 + lq * 4), acc);
      const int r = rb * 16 + l16;
      const u32x2 qa = *reinterpret_cast<const u32x2*>(sm.Q + r * PQ + wave * 16 + lq * 4);
      const float gr = sm.g[r];
      *reinterpret_cast<u32x2*>(wsc + kWsQ + ((size_t)(rb * 4 + (wave >> 1)) * 64 + lane) * 16 + 8 * (wave & 1)) =
          u32x2{pack_bf16(gr * lo_bf(qa.x) - acc[0], gr * hi_bf(qa.x) - acc[1]),
                pack_bf16(gr * lo_bf(qa.y) - acc[2], gr * hi_bf(qa.y) - acc[3])};
    }
  }
  // ---- O~ = A U~ tiles (rb, vb = wave), with the U~ tiles as B operands (the forward's
  // outputs only: the backward, STORE_T, reads no O~)
  if constexpr (!STORE_T) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jb = 0; jb <= rb; ++jb) acc = mfma16(ld4(sm.A + (rb * 16 + l16) * PC + jb * 16 + lq * 4), ub[jb], acc);
      *reinterpret_cast<u32x2*>(wsc + kWsO + ((size_t)(rb * 8 + wave) * 64 + lane) * 8) =
          u32x2{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
    }
  }
  lds_barrier();
}

}  // namespace gdc

template <bool STORE_T>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void gdn_chunk_prep2_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, uint8_t* __restrict__ ws,
    uint16_t* __restrict__ Tout, int T, int nchunks) {
  using namespace gdc;
  __shared__ Prep2Smem sm;
  const int nc = T / C;
  PrepIn<false> in;
  int cid = blockIdx.x;   // the grid never exceeds nchunks
  prep_fetch<false>(in, q, k, v, alpha, beta, (size_t)(cid / nc) * T + (size_t)(cid % nc) * C);
  prep2_chunk<STORE_T>(sm, in, cid, q, k, v, alpha, beta, ws, Tout, T, nchunks);
  for (cid += gridDim.x; cid < nchunks; cid += gridDim.x)
    prep2_chunk<STORE_T>(sm, in, cid, q, k, v, alpha, beta, ws, Tout, T, nchunks);
  keep_inputs(in);
}

// KDA prep, persistent: block b handles chunks b, b + grid, ...; the next chunk's inputs
// are loaded into registers while this one is processed, and every thread issues the
// same loads and stores on every chunk so that those waits are exact (the first chunk
// is peeled, so that the loop's waits do not also serve the loads issued before it).
__global__ __launch_bounds__(512) void kda_chunk_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, uint8_t* __restrict__ ws, int T,
    int nchunks) {
  using namespace gdc;
  __shared__ PrepSmem sm;
  __shared__ KdaPrepSmem xs;
  const int nc = T / C;
  PrepIn<true> in;
  int cid = blockIdx.x;   // the grid never exceeds nchunks
  prep_fetch<true>(in, q, k, v, alpha, beta, (size_t)(cid / nc) * T + (size_t)(cid % nc) * C);
  kda_prep_chunk(sm, xs, in, cid, q, k, v, alpha, beta, ws, T, nchunks);
  for (cid += gridDim.x; cid < nchunks; cid += gridDim.x) kda_prep_chunk(sm, xs, in, cid, q, k, v, alpha, beta, ws, T, nchunks);
  keep_inputs(in);
}

// ------------------------------------------------------------------ sequential pass
namespace gdc {

constexpr int kAhead = 2;   // chunks of operands in flight ahead of the one in use (4 measured no faster)
constexpr int kWarm = 2;    // chunks between the L2 warm-up of a chunk and its loads

template <int VT>
struct alignas(16) SeqSmem {
  uint16_t Sb[2][VT * PQ];   // bf16 state tile [v][qcol(k)], double buffered
  uint16_t Ut[VT * PC];      // U^T tile [v][j]
  uint16_t Ot[2][VT * PC];   // outputs^T [v][r], by chunk parity
};

// One chunk's operands for this wave: waves 0-3 take W (role U), waves 4-7 take Q'
// (role O), both for token block rb = wave & 3, with U~ resp. O~ of the block's
// value tiles; every wave takes the K^ fragments of key block `wave` and g_C.
template <int NVB>
struct Prefetch {
  u32x4 m[4];
  u32x2 x[NVB];
  u32x4 kh[2];
  float gc;
  unsigned warm;   // one word of a line touched to bring it into L2 early (unused)
};

// The loads of a set are issued in two parts (PART 0: the W or Q' fragments; PART 1:
// the rest) at two points of a chunk, so that the address units work through them
// while the waves compute instead of holding the waves at a burst of loads.
template <int NVB, int PART, bool KDA>
__device__ __forceinline__ void fetch_chunk(Prefetch<NVB>& pf, const uint8_t* __restrict__ wsc,
                                            const uint8_t* __restrict__ warm, int vt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rb = wave & 3;
  const bool role_o = wave >= 4;
  if constexpr (PART == 0) {
    const uint8_t* mb = wsc + (role_o ? kWsQ : kWsW) + (size_t)rb * 4096 + lane * 16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pf.m[ks] = *reinterpret_cast<const u32x4*>(mb + ks * 1024);
    return;
  }
  const uint8_t* xb = wsc + (role_o ? kWsO : kWsU) + ((size_t)(rb * 8 + vt * NVB) * 64 + lane) * 8;
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb) pf.x[vb] = *reinterpret_cast<const u32x2*>(xb + vb * 512);
#pragma unroll
  for (int js = 0; js < 2; ++js)
    pf.kh[js] = *reinterpret_cast<const u32x4*>(wsc + kWsK + ((size_t)(wave * 2 + js) * 64 + lane) * 16);
  // the state decay of this lane's key column (GDN: one value, stored 16 times)
  pf.gc = *reinterpret_cast<const float*>(wsc + kWsG + (KDA ? wave * 16 + (lane & 15) : (lane & 15)) * 4);
  // L2 warm-up of a later chunk: the 8 / NVB value tiles of one sequence split its 384
  // lines of W, Q' and K^ (48 NVB each) and each touches the 32 NVB lines of its own
  // U~, O~; the remaining threads all touch one line
  {
    const int t = threadIdx.x;
    size_t off = 0;
    if (t < 48 * NVB) {
      off = (size_t)(vt * 48 * NVB + t) * 128;
    } else if (t < 80 * NVB) {
      const int j = t - 48 * NVB, reg = j / (16 * NVB), w = j % (16 * NVB);
      off = (reg ? kWsO : kWsU) + (size_t)(((w >> 2) / NVB) * 8 + vt * NVB + (w >> 2) % NVB) * 512 +
            (w & 3) * 128;
    }
    pf.warm = *reinterpret_cast<const unsigned*>(warm + off);
  }
}

// Stores the staged outputs of the chunk starting at token tok0: VT / 8 per thread,
// the same single store in every thread.
template <int VT>
__device__ __forceinline__ void store_o(const uint16_t* __restrict__ Ot, uint16_t* __restrict__ o,
                                        size_t tok0, int v0) {
  constexpr int EPT = VT / 8;
  const int tid = threadIdx.x, r = tid >> 3, c0 = (tid & 7) * EPT;
  uint16_t* dst = o + (tok0 + r) * kD + v0 + c0;
  if constexpr (EPT == 2) {
    *reinterpret_cast<unsigned*>(dst) = unsigned(Ot[c0 * PC + r]) | (unsigned(Ot[(c0 + 1) * PC + r]) << 16);
  } else {
    *reinterpret_cast<u32x2*>(dst) =
        u32x2{unsigned(Ot[c0 * PC + r]) | (unsigned(Ot[(c0 + 1) * PC + r]) << 16),
              unsigned(Ot[(c0 + 2) * PC + r]) | (unsigned(Ot[(c0 + 3) * PC + r]) << 16)};
  }
}

// One chunk: starts the loads of the operands of the chunk kAhead chunks later into
// `nx` and stores the previous chunk's outputs, then consumes `pf`. Every thread
// issues the same loads and the same store on every chunk (past the end the last
// chunk's operands are loaded again; the first chunk, FIRST, has nothing to store) so
// that the wait for `pf` counts exactly the memory operations issued after it instead
// of waiting for them.
template <int VT, bool FIRST, bool KDA>
__device__ __forceinline__ void gdn_seq_chunk(SeqSmem<VT>& sm, const Prefetch<VT / 16>& pf,
                                              Prefetch<VT / 16>& nx, f32x4 (&Sacc)[VT / 16],
                                              int& cur, unsigned& sink, int ci, int nc, size_t chunk0,
                                              size_t tok0, int vt, const uint8_t* __restrict__ ws,
                                              uint16_t* __restrict__ o) {
  constexpr int NVB = VT / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int rb = wave & 3, kcol = wave * 16 + l16, v0 = vt * VT;
  const bool role_o = wave >= 4;
  const uint8_t* nxc = ws + (chunk0 + min(ci + kAhead, nc - 1)) * ws_chunk<KDA>();
  const uint8_t* wmc = ws + (chunk0 + min(ci + kAhead + kWarm, nc - 1)) * ws_chunk<KDA>();
  fetch_chunk<NVB, 0, KDA>(nx, nxc, wmc, vt);
  sink ^= pf.warm;
  if constexpr (!FIRST) store_o<VT>(sm.Ot[(ci - 1) & 1], o, tok0 - C, v0);

  // keeps the unpacking of the operand sets still in flight from being moved up to
  // here, where it would have to wait for their loads
  __builtin_amdgcn_sched_barrier(0);

  // ---- role U: U = U~ - W S^T; role O: O = O~ + Q' S^T (to LDS, transposed)
  const float sgn = role_o ? 1.f : -1.f;
  uint16_t* dst = (role_o ? sm.Ot[ci & 1] : sm.Ut) + l16 * PC + rb * 16 + lq * 4;
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)   // keys 32 ks + 4 lq + {0..3}, 32 ks + 16 + 4 lq + {0..3}: one piece
      acc = mfma(as_bf8(pf.m[ks]), ld8(sm.Sb[cur] + (vb * 16 + l16) * PQ + ks * 32 + lq * 8), acc);
    const u32x2 xv = pf.x[vb];
    *reinterpret_cast<u32x2*>(dst + vb * 16 * PC) =
        u32x2{pack_bf16(lo_bf(xv.x) + sgn * acc[0], hi_bf(xv.x) + sgn * acc[1]),
              pack_bf16(lo_bf(xv.y) + sgn * acc[2], hi_bf(xv.y) + sgn * acc[3])};
  }
  fetch_chunk<NVB, 1, KDA>(nx, nxc, wmc, vt);
  lds_barrier();

  // ---- S <- g_C S + U^T K^: key block = wave; next bf16 copy
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb) {
    f32x4 acc = Sacc[vb] * pf.gc;
#pragma unroll
    for (int js = 0; js < 2; ++js)
      acc = mfma(ld8(sm.Ut + (vb * 16 + l16) * PC + js * 32 + lq * 8), as_bf8(pf.kh[js]), acc);
    Sacc[vb] = acc;
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.Sb[cur ^ 1][(vb * 16 + lq * 4 + i) * PQ + qcol(kcol)] = f32_to_bf16(acc[i]);
  }
  cur ^= 1;
  lds_barrier();
}

}  // namespace gdc

template <int VT, bool KDA>
__global__ __launch_bounds__(512) void gdn_chunk_seq_kernel(
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
      sm.Sb[0][(vb * 16 + lq * 4 + i) * PQ + qcol(kcol)] = f32_to_bf16(Sacc[vb][i]);
    }

  if (nc > 0) {
    const size_t chunk0 = (size_t)n * nc, tokn = (size_t)n * T;
    // kAhead + 1 operand sets in rotation: chunk ci uses set ci % NS and loads chunk
    // ci + kAhead into set (ci + kAhead) % NS (every index below is a constant after
    // unrolling, so the sets stay in registers)
    constexpr int NS = kAhead + 1;
    Prefetch<NVB> P[NS];
    int cur = 0;
    unsigned sink = 0;
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const uint8_t* ci_ = ws + (chunk0 + min(i, nc - 1)) * ws_chunk<KDA>();
      const uint8_t* wi_ = ws + (chunk0 + min(i + kWarm, nc - 1)) * ws_chunk<KDA>();
      fetch_chunk<NVB, 0, KDA>(P[i], ci_, wi_, vt);
      fetch_chunk<NVB, 1, KDA>(P[i], ci_, wi_, vt);
    }
    lds_barrier();
    gdn_seq_chunk<VT, true, KDA>(sm, P[0], P[kAhead], Sacc, cur, sink, 0, nc, chunk0, tokn, vt, ws, o);
    int ci = 1;
    for (; ci + NS - 1 < nc; ci += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u)
        gdn_seq_chunk<VT, false, KDA>(sm, P[(1 + u) % NS], P[(1 + u + kAhead) % NS], Sacc, cur, sink, ci + u, nc,
                                 chunk0, tokn + (size_t)(ci + u) * C, vt, ws, o);
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
      if (ci + u < nc)
        gdn_seq_chunk<VT, false, KDA>(sm, P[(1 + u) % NS], P[(1 + u + kAhead) % NS], Sacc, cur, sink, ci + u, nc,
                                 chunk0, tokn + (size_t)(ci + u) * C, vt, ws, o);
    store_o<VT>(sm.Ot[(nc - 1) & 1], o, tokn + (size_t)(nc - 1) * C, v0);
    asm volatile("" ::"v"(sink));   // keeps the warm-up loads
  }

#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ST[((size_t)n * kD + v0 + vb * 16 + lq * 4 + i) * kD + kcol] = Sacc[vb][i];
}

}  // namespace gdnrt

using namespace gdnrt;

namespace {

template <bool KDA>
size_t chunk_workspace_bytes(int N, int T, int dk, int dv, int chunk) {
  if (N <= 0 || T <= 0 || dk != kD || dv != kD || chunk != kChunk || T % kChunk) return 0;
  return (size_t)N * (T / kChunk) * gdc::ws_chunk<KDA>();
}

template <bool KDA>
int chunk_fwd(const char* fn, const void* q, const void* k, const void* v, const float* alpha,
              const float* beta, const float* S0, float* ST, void* o, int N, int T, int dk, int dv,
              int chunk, int io, void* workspace, size_t ws_bytes, void* stream) {
  if (N < 0 || T < 0) return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d must be >= 0", fn, N, T);
  if (dk != kD || dv != kD)
    return set_error(GDNRT_ESHAPE, "%s: d_k=%d d_v=%d, only 128 is supported", fn, dk, dv);
  if (chunk != kChunk) return set_error(GDNRT_ESHAPE, "%s: chunk=%d, only 64 is supported", fn, chunk);
  if (T % kChunk) return set_error(GDNRT_ESHAPE, "%s: T=%d is not a multiple of 64", fn, T);
  if (io != GDNRT_BF16) return set_error(GDNRT_EDTYPE, "%s: io must be GDNRT_BF16", fn);
  if ((size_t)N * (T / kChunk) > 0x7fffffffu || (size_t)N * 8 > 0x7fffffffu)
    return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d too large", fn, N, T);
  if (N == 0) return clear_error();
  if (!ST || (T > 0 && (!q || !k || !v || !alpha || !beta || !o)))
    return set_error(GDNRT_EINVAL, "%s: null pointer argument", fn);
  const size_t nchunks = (size_t)N * (T / kChunk);
  const size_t need = nchunks * gdc::ws_chunk<KDA>();
  if (ws_bytes < need || (need && !workspace))
    return set_error(GDNRT_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
  if ((T > 0 && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace) ||
                 (KDA ? !aligned16(alpha) : !aligned4(alpha)) || !aligned4(beta))) ||
      !aligned4(ST) || (S0 && !aligned4(S0)))
    return set_error(GDNRT_EALIGN, KDA ? "%s: q, k, v, o, alpha, workspace must be 16-byte aligned"
                                       : "%s: q, k, v, o, workspace must be 16-byte aligned", fn);
  const size_t ntok = (size_t)N * T, nIO = ntok * kD * 2, nG = ntok * 4 * (KDA ? kD : 1),
               nS = (size_t)N * kD * kD * 4;
  if (overlaps(o, nIO, q, nIO) || overlaps(o, nIO, k, nIO) || overlaps(o, nIO, v, nIO) ||
      overlaps(o, nIO, alpha, nG) || overlaps(o, nIO, beta, ntok * 4) || overlaps(o, nIO, ST, nS) ||
      overlaps(o, nIO, S0, nS) || overlaps(o, nIO, workspace, need) ||
      overlaps(ST, nS, q, nIO) || overlaps(ST, nS, k, nIO) || overlaps(ST, nS, v, nIO) ||
      overlaps(ST, nS, workspace, need) || (S0 && S0 != ST && overlaps(ST, nS, S0, nS)) ||
      overlaps(workspace, need, q, nIO) || overlaps(workspace, need, k, nIO) ||
      overlaps(workspace, need, v, nIO) || overlaps(workspace, need, S0, nS) ||
      overlaps(workspace, need, alpha, nG))
    return set_error(GDNRT_EINVAL, "%s: buffers overlap (only ST may equal S0)", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (T > 0) {
    // persistent blocks: GDN two per CU, KDA one (its LDS fills most of a CU)
    const size_t cap = KDA ? 256 : 512;
    const unsigned grid = (unsigned)(nchunks < cap ? nchunks : cap);
    if constexpr (KDA)
      hipLaunchKernelGGL(kda_chunk_prep_kernel, dim3(grid), dim3(gdc::NT), 0, s,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), alpha, beta, ws, T, (int)nchunks);
    else
      hipLaunchKernelGGL((gdn_chunk_prep2_kernel<false>), dim3(grid), dim3(gdc::NT), 0, s,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), alpha, beta, ws, nullptr, T, (int)nchunks);
    int rc = check_launch(fn);
    if (rc != GDNRT_OK) return rc;
  }
  // value tiles of 16 when there are too few sequences to fill the chip with 32
  if (N * 4 < 256)
    hipLaunchKernelGGL((gdn_chunk_seq_kernel<16, KDA>), dim3((unsigned)(N * 8)), dim3(gdc::NT), 0, s, ws, S0,
                       ST, static_cast<uint16_t*>(o), N, T);
  else
    hipLaunchKernelGGL((gdn_chunk_seq_kernel<32, KDA>), dim3((unsigned)(N * 4)), dim3(gdc::NT), 0, s, ws, S0,
                       ST, static_cast<uint16_t*>(o), N, T);
  return check_launch(fn);
}

}  // namespace

namespace gdnrt {
// The GDN chunk prep for the chunkwise backward: the forward's operands (at the
// forward's per-chunk stride) and each chunk's (I + L)^-1. T > 0, shapes checked by
// the caller.
void gdn_chunk_prep_with_inverse(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const float* alpha, const float* beta, uint8_t* ws, uint16_t* Tout,
                                 int T, int nchunks, hipStream_t s) {
  const unsigned grid = (unsigned)(nchunks < 512 ? nchunks : 512);
  hipLaunchKernelGGL((gdn_chunk_prep2_kernel<true>), dim3(grid), dim3(gdc::NT), 0, s, q, k, v, alpha,
                     beta, ws, Tout, T, nchunks);
}
}  // namespace gdnrt

namespace gdnrt {
// gdn_chunk_fwd under another entry point's name (its messages carry `fn`); the
// workspace argument as in gdn_chunk_fwd.
int gdn_chunk_fwd_named(const char* fn, const void* q, const void* k, const void* v, const float* alpha,
                        const float* beta, const float* S0, float* ST, void* o, int N, int T, int dk,
                        int dv, int chunk, int io, void* workspace, size_t ws_bytes, void* stream) {
  return chunk_fwd<false>(fn, q, k, v, alpha, beta, S0, ST, o, N, T, dk, dv, chunk, io, workspace,
                          ws_bytes, stream);
}
}  // namespace gdnrt

extern "C" size_t gdn_chunk_fwd_workspace_bytes(int N, int T, int dk, int dv, int chunk) {
  return chunk_workspace_bytes<false>(N, T, dk, dv, chunk);
}

extern "C" int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* S0, float* ST, void* o, int N, int T,
                             int dk, int dv, int chunk, int io, void* workspace, size_t ws_bytes,
                             void* stream) {
  return chunk_fwd<false>("gdn_chunk_fwd", q, k, v, alpha, beta, S0, ST, o, N, T, dk, dv, chunk, io,
                          workspace, ws_bytes, stream);
}

extern "C" size_t kda_chunk_fwd_workspace_bytes(int N, int T, int dk, int dv, int chunk) {
  return chunk_workspace_bytes<true>(N, T, dk, dv, chunk);
}

extern "C" int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* S0, float* ST, void* o, int N, int T,
                             int dk, int dv, int chunk, int io, void* workspace, size_t ws_bytes,
                             void* stream) {
  return chunk_fwd<true>("kda_chunk_fwd", q, k, v, alpha, beta, S0, ST, o, N, T, dk, dv, chunk, io,
                         workspace, ws_bytes, stream);
}

// Gated linear attention, chunkwise forward from an incoming state (prefill shard).
//
// Method: "ZeCO: Zero Communication Overhead Sequence Parallelism for Linear
// Attention", section "Gated Linear Attention (GLA) Formulation" (per-token and
// chunk recurrences, inter/intra-chunk output), section "The Complete Forward
// Algorithm" (the intra-chunk keys are divided by Lambda) and section "Global State
// Update Formula" (eq. 6: a shard's final state is its incoming state decayed by the
// shard's total gate plus its state from zero). In the [d_v][d_k] state layout, with
// b the inclusive cumulative log-gate inside a chunk of C = 64 tokens:
//
//   O   = (Q o e^b) S^T + [ ((Q o e^b)(K o e^-b)^T) o M ] V,   M lower incl. diag,
//   S  <- e^{b_C} (on key columns) o S + V^T (K o e^{b_C - b}).
//
// The chunks of each sequence are cut into P segments (eq. 6 applied inside the call):
//   pass 1   every segment but the last, in R pieces, from a zero state: each piece's
//            end state B_i and total decay gamma_i = exp(sum of its log-gates) per key;
//   combine  start states: S_0 the incoming state, then x <- gamma_i o x + B_i over the
//            pieces of segment s in order gives S_{s+1};
//   pass 2   every segment from its start state, with outputs.
// A 512-thread block runs one (sequence, segment or piece); the segments fill the GPU,
// pass 2 at one block per CU (the segment's state in registers), pass 1 at two. Per chunk the block forms, with m the chunk's middle token
// (which halves the range of the factors), Qr = Q o e^{b - b_m} and Kr = K o e^{b_m - b}
// once in LDS; every product goes through them:
//   scores      (Qr Kr^T) o M,
//   inter-chunk (Q o e^b) S^T = Qr (S o e^{b_m})^T, the state's key columns scaled in fp32,
//   state       V^T (K o e^{b_C - b}) = (V^T Kr) o e^{b_C - b_m}, scaled after the product.
// Thread (lane, wave w) loads channels 2 lane, 2 lane + 1 of tokens 8 w .. 8 w + 7 of q,
// k and the log-gates straight into registers, a chunk ahead and in three parts spread
// over the chunk, and forms their factors there (exponentials in base 2); v goes through
// LDS for the transposed operand reads. Wave w holds the state rows of value channels
// 16 w .. 16 w + 15 transposed (rows = keys) in fp32 MFMA accumulators, which are also
// the A operand of the inter-chunk product: their key order (four consecutive keys per
// lane from each of two 16-key blocks) is matched by storing Qr key-permuted in LDS, so
// that the B operand is one 16-byte read.
// bf16 MFMA (16x16x32) with fp32 accumulation throughout.
#include "chunk_device.hpp"
#include "gla_chunk_layout.hpp"

namespace gdnrt {

namespace gla {
using namespace gdc;   // C, PQ, PC, PS, swz, ld8, ld_tr8s, mfma, tri_pair, lo_bf, hi_bf

constexpr int NB = 512;       // threads per block: 8 waves
// Kr and v are read transposed (ds_read_b64_tr_b16) and Kr also by rows: both stored
// with swz (pitch PT = PS).
constexpr int PT = PS;
constexpr int kMaxSeg = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr size_t kStateBytes = (size_t)kD * kD * 4;

// Segments per sequence: one block per CU over the whole grid, at most kMaxSeg per
// sequence, every segment non-empty. Pass 1 cuts each of the first P - 1 segments into R
// pieces of L1 chunks (the combine folds them in order). Workspace after the chunks:
// B [N][P-1][R][128][128] fp32, gamma [N][P-1][R][128] fp32, start states
// [N][P][128][128] fp32.
struct Plan {
  int P, Lseg, R, L1;
  size_t b_off, g_off, s_off, total;
};

__host__ inline Plan plan(int N, int nc) {
  Plan p{};
  int P = N >= 256 ? 1 : (256 + N - 1) / N;
  P = P > kMaxSeg ? kMaxSeg : P;
  if (P > nc) P = nc;
  if (P < 1) P = 1;
  p.Lseg = nc > 0 ? (nc + P - 1) / P : 0;
  p.P = nc > 0 ? (nc + p.Lseg - 1) / p.Lseg : 1;
  p.R = p.Lseg % 2 == 0 ? 2 : 1;
  p.L1 = p.Lseg / p.R;
  const size_t pieces = p.P > 1 ? (size_t)N * (p.P - 1) * p.R : 0;
  p.b_off = (size_t)N * nc * kWChunk;
  p.g_off = p.b_off + pieces * kStateBytes;
  p.s_off = p.g_off + pieces * kD * 4;
  p.total = p.s_off + (p.P > 1 ? (size_t)N * p.P * kStateBytes : 0);
  return p;
}

struct alignas(16) Smem {
  uint16_t Qr[C * PQ];               // q o e^{b - b_m} [t][qcol(k)] (key-permuted, qcol)
  uint16_t Kr[C * PT];               // pass 2: k o e^{b_m - b}; pass 1: k o e^{b_C - b}
  uint16_t V[C * PT];                // v [t][v]
  uint16_t A[C * PC];                // masked scores [r][j]
  float tot[8 * kD];                 // log-gate sums of each group of 8 tokens
  float ec[kD], em[kD], ef[kD];      // e^{b_C}, e^{b_m}, e^{b_C - b_m} per key
};

// One chunk's inputs of a thread: q, k, log-gates of channels 2 cp, 2 cp + 1 of tokens
// 8 eg .. 8 eg + 7 (cp = lane, eg = wave), and the 16-byte pieces p = tid + 512 h of v.
struct In {
  unsigned q[8], k[8];
  f32x2 g[8];
  u32x4 v[2];
};

// Loads of one chunk's inputs, in parts (PART 1: q and k, 2: log-gates, 3: v, 0: all), so
// that a chunk's requests can be spread over the work on the previous one.
template <bool OUT, int PART>
__device__ __forceinline__ void fetch(In& in, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                      const uint16_t* __restrict__ v, const float* __restrict__ log_g, size_t tok0,
                                      int t) {
  const int cp = t & 63, eg = t >> 6;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const size_t off = (tok0 + 8 * eg + i) * kD + 2 * cp;
    if constexpr (PART == 0 || PART == 1) {
      if constexpr (OUT) in.q[i] = *reinterpret_cast<const unsigned*>(q + off);
      in.k[i] = *reinterpret_cast<const unsigned*>(k + off);
    }
    if constexpr (PART == 0 || PART == 2) in.g[i] = *reinterpret_cast<const f32x2*>(log_g + off);
  }
  if constexpr (PART == 0 || PART == 3) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int p = t + NB * h;
      in.v[h] = *reinterpret_cast<const u32x4*>(v + (tok0 + (p >> 4)) * kD + 8 * (p & 15));
    }
  }
}

// v to LDS; the thread's prefix sums of its log-gates in base 2 (in place) and their
// totals per group of 8 tokens to LDS.
__device__ __forceinline__ void stage(Smem& sm, In& in, int t) {
  const int cp = t & 63, eg = t >> 6;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = t + NB * h;
    *reinterpret_cast<u32x4*>(sm.V + (p >> 4) * PT + ((8 * (p & 15)) ^ swz(p >> 4))) = in.v[h];
  }
  in.g[0] *= kLog2e;
#pragma unroll
  for (int i = 1; i < 8; ++i) in.g[i] = in.g[i] * kLog2e + in.g[i - 1];
  *reinterpret_cast<f32x2*>(sm.tot + eg * kD + 2 * cp) = in.g[7];
}

__device__ __forceinline__ f32x2 bf2f(unsigned w) { return f32x2{lo_bf(w), hi_bf(w)}; }
__device__ __forceinline__ unsigned pk2(f32x2 x) { return pack_bf16(x[0], x[1]); }
__device__ __forceinline__ u32x2 pk4(f32x4 x) { return u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])}; }
// 2^x per component (v_exp_f32); the log-gates are carried in base 2 inside the kernel
__device__ __forceinline__ f32x2 exp2v(f32x2 x) {
  return f32x2{__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1])};
}

}  // namespace gla

// OUT: pass 2 (one block per (sequence, segment), outputs; KEEP: the shard calls' workspace);
// else pass 1 (one block per (sequence, piece of a segment < P - 1): end state from zero
// and the piece's decay). Wave w owns value channels 16 w .. 16 w + 15; in the
// elementwise work thread (lane, w) owns channels 2 lane, 2 lane + 1 of tokens 8 w .. 8 w + 7.
template <bool OUT, bool KEEP>
__global__ __launch_bounds__(512, OUT ? 2 : 4) void gla_fused_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ log_g, uint8_t* __restrict__ ws, const float* __restrict__ S0,
    const float* __restrict__ Sst, float* __restrict__ Bbuf, float* __restrict__ Gbuf,
    float* __restrict__ ST, uint16_t* __restrict__ o, int T, int P, int Lseg, int R) {
  using namespace gla;
  __shared__ Smem sm;
  __shared__ __attribute__((aligned(16))) uint16_t s_qh[KEEP ? C * PQ : 8];   // KEEP: Q^ [t][qcol(k)]
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave
  // MFMA lane roles (l16, lq) and the elementwise channel pair cp; the chunk loop forms
  // its own from an opaque copy of the thread index
  const int l16 = tid & 15, lq = (tid >> 4) & 3, cp = tid & 63;
  const int segs = OUT ? P : (P - 1) * R;   // blocks per sequence
  const int n = blockIdx.x / segs, s = blockIdx.x % segs;
  const int nc = T / C, len = OUT ? Lseg : Lseg / R;
  const int c0 = s * len, c1 = min(nc, c0 + len);
  const int vrow = 16 * w + l16;   // this lane's value channel in the MFMA layouts

  // St[kb][i] = S[vrow][16 kb + 4 lq + i]
  f32x4 St[8];
  {
    const float* src = nullptr;
    if constexpr (OUT) src = P > 1 ? Sst + ((size_t)n * P + s) * kD * kD : S0 ? S0 + (size_t)n * kD * kD : nullptr;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
      St[kb] = src ? *reinterpret_cast<const f32x4*>(src + (size_t)vrow * kD + 16 * kb + 4 * lq)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  f32x2 lsum = {0.f, 0.f};   // pass 1, wave 0: the piece's log-decay (base 2)

  if (c1 > c0) {
    const size_t tokn = (size_t)n * T;
    if constexpr (OUT) {   // the upper tiles (0,1), (2,3) that the 32-wide slices of A reach stay zero
      const int t2 = tid >> 8, x = tid & 255;
      sm.A[(32 * t2 + (x >> 4)) * PC + 32 * t2 + 16 + (x & 15)] = 0;
    }
    In in;
    fetch<OUT, 0>(in, q, k, v, log_g, tokn + (size_t)c0 * C, tid);
    stage(sm, in, tid);
    // all of the first chunk's loads complete here, so that inside the loop the waits for
    // the prefetched q and k count only what follows them (s_waitcnt vmcnt(0))
    __builtin_amdgcn_s_waitcnt(0xF70);
#pragma unroll 1
    for (int c = c0;;) {
      const size_t tok0 = tokn + (size_t)c * C;
      uint8_t* wsc = ws + ((size_t)n * nc + c) * kWChunk;
      // the thread index through an opaque move: the per-lane addresses are formed inside
      // each chunk instead of being held across the loop
      int t;
      asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(tid));
      const int lane = t & 63, l16 = lane & 15, lq = lane >> 4, cp = lane;
      lds_barrier();

      // ---- factors of the thread's elements (tokens 8 w .., channels 2 cp, 2 cp + 1)
      {
        f32x2 off = {0.f, 0.f}, bm = off, bC = off;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const f32x2 te = *reinterpret_cast<const f32x2*>(sm.tot + e * kD + 2 * cp);
          if (e < w) off += te;   // wave-uniform
          if (e < 4) bm += te;    // b at token 31, the middle of the chunk
          bC += te;
        }
        const f32x2 emv = exp2v(bm);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * w + i;
          const f32x2 b = in.g[i] + off;
          const f32x2 kf = bf2f(in.k[i]);
          if constexpr (OUT) {
            const f32x2 d = b - bm;
            const f32x2 qr = bf2f(in.q[i]) * exp2v(d);
            *reinterpret_cast<unsigned*>(sm.Qr + r * PQ + qcol(2 * cp)) = pk2(qr);
            *reinterpret_cast<unsigned*>(sm.Kr + r * PT + ((2 * cp) ^ swz(r))) = pk2(kf * exp2v(-d));
            if constexpr (KEEP) *reinterpret_cast<unsigned*>(s_qh + r * PQ + qcol(2 * cp)) = pk2(qr * emv);
          } else {
            *reinterpret_cast<unsigned*>(sm.Kr + r * PT + ((2 * cp) ^ swz(r))) = pk2(kf * exp2v(bC - b));
          }
        }
        // the next chunk's q and k go out before this chunk's workspace stores; its
        // log-gates and v follow later in the chunk
        if (c + 1 < c1) fetch<OUT, 1>(in, q, k, v, log_g, tok0 + C, t);
        if (w == 0) {
          const f32x2 ecv = exp2v(bC);
          *reinterpret_cast<f32x2*>(sm.ec + 2 * cp) = ecv;
          if constexpr (OUT) {
            *reinterpret_cast<f32x2*>(sm.em + 2 * cp) = emv;
            *reinterpret_cast<f32x2*>(sm.ef + 2 * cp) = exp2v(bC - bm);
            if constexpr (KEEP) *reinterpret_cast<f32x2*>(reinterpret_cast<float*>(wsc + kWE) + 2 * cp) = ecv;
          } else {
            lsum += bC;
          }
        }
      }
      lds_barrier();
      if constexpr (KEEP) {   // Q^ for the shard calls: fragment f = 4 tb + ks, 1 KB, in the
                              // order of the inter-chunk product's Qr pieces (16 bytes per lane)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int f = w + 8 * h;
          *reinterpret_cast<u32x4*>(wsc + kWQ + ((size_t)f * 64 + lane) * 16) =
              *reinterpret_cast<const u32x4*>(s_qh + (16 * (f >> 2) + l16) * PQ + 32 * (f & 3) + 8 * lq);
        }
      }

      // ---- wave w: the value operand of its tile (lane (l16, lq) holds v[32 js + 8 lq + e][16 w + l16])
      const bf16x8 vt0 = ld_tr8s(sm.V, 0, 16 * w), vt1 = ld_tr8s(sm.V, 32, 16 * w);
      f32x4 oacc[4];
      if constexpr (OUT) {
        // inter-chunk outputs, transposed: D[v][t] = sum_k (S o e^{b_m})[v][k] Qr[t][k],
        // contraction slot 8 lq + e <-> key 32 ks + 4 lq + e (e < 4), 32 ks + 16 + 4 lq + e - 4:
        // one 16-byte piece of Qr's row
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) oacc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const f32x4 e0 = *reinterpret_cast<const f32x4*>(sm.em + 32 * ks + 4 * lq);
          const f32x4 e1 = *reinterpret_cast<const f32x4*>(sm.em + 32 * ks + 16 + 4 * lq);
          const u32x2 a = pk4(St[2 * ks] * e0), b = pk4(St[2 * ks + 1] * e1);
          const bf16x8 sa = as_bf8(u32x4{a[0], a[1], b[0], b[1]});
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) oacc[tb] = mfma(sa, ld8(sm.Qr + (16 * tb + l16) * PQ + 32 * ks + 8 * lq), oacc[tb]);
        }
      }
      if (c + 1 < c1) fetch<OUT, 2>(in, q, k, v, log_g, tok0 + C, t);
      // state rows of the wave's tile: S^T <- e^{b_C} o S^T + K^T V through Kr
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const bf16x8 k0 = ld_tr8s(sm.Kr, 0, 16 * kb), k1 = ld_tr8s(sm.Kr, 32, 16 * kb);
        const f32x4 ecv = *reinterpret_cast<const f32x4*>(sm.ec + 16 * kb + 4 * lq);
        if constexpr (OUT) {
          const f32x4 efv = *reinterpret_cast<const f32x4*>(sm.ef + 16 * kb + 4 * lq);
          const f32x4 x = mfma(k1, vt1, mfma(k0, vt0, f32x4{0.f, 0.f, 0.f, 0.f}));
          St[kb] = St[kb] * ecv + x * efv;
        } else {
          St[kb] = mfma(k1, vt1, mfma(k0, vt0, St[kb] * ecv));
        }
      }
      if (c + 1 < c1) fetch<OUT, 3>(in, q, k, v, log_g, tok0 + C, t);
      if constexpr (OUT) {
        // masked scores over the lower triangle of 16 x 16 tiles; the keys of a 16-byte
        // piece of Qr come from two 8-byte pieces of Kr
        for (int u = w; u < 10; u += 8) {
          int rb, cb;
          tri_pair(u, rb, cb);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          const uint16_t* kp = sm.Kr + (cb * 16 + l16) * PT;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const u32x2 x0 = *reinterpret_cast<const u32x2*>(kp + ((32 * ks + 4 * lq) ^ swz(l16)));
            const u32x2 x1 = *reinterpret_cast<const u32x2*>(kp + ((32 * ks + 16 + 4 * lq) ^ swz(l16)));
            acc = mfma(ld8(sm.Qr + (rb * 16 + l16) * PQ + ks * 32 + lq * 8), as_bf8(u32x4{x0[0], x0[1], x1[0], x1[1]}),
                       acc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = rb * 16 + lq * 4 + i, jj = cb * 16 + l16;
            sm.A[r * PC + jj] = f32_to_bf16(jj <= r ? acc[i] : 0.f);
          }
        }
        lds_barrier();
        // intra-chunk outputs: D[v][t] += sum_j v[j][v] A[t][j]; the lane holds token
        // 16 tb + l16, value channels 16 w + 4 lq + i
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          oacc[tb] = mfma(vt0, ld8(sm.A + (16 * tb + l16) * PC + 8 * lq), oacc[tb]);
          if (tb >= 2) oacc[tb] = mfma(vt1, ld8(sm.A + (16 * tb + l16) * PC + 32 + 8 * lq), oacc[tb]);
          *reinterpret_cast<u32x2*>(o + (tok0 + 16 * tb + l16) * kD + 16 * w + 4 * lq) = pk4(oacc[tb]);
        }
      }
      if (++c == c1) break;
      // ---- the next chunk's inputs go to LDS once every wave is done with this one's; the
      // staging follows this chunk's stores on every path, so waiting for its loads never
      // waits for those stores
      if constexpr (!OUT) lds_barrier();
      stage(sm, in, t);
    }
  }

  float* dst;
  if constexpr (OUT) {
    if (s != P - 1) return;
    dst = ST + (size_t)n * kD * kD;
  } else {
    dst = Bbuf + ((size_t)n * segs + s) * kD * kD;
    if (w == 0) *reinterpret_cast<f32x2*>(Gbuf + ((size_t)n * segs + s) * kD + 2 * cp) = exp2v(lsum);
  }
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
    *reinterpret_cast<f32x4*>(dst + (size_t)vrow * kD + 16 * kb + 4 * lq) = St[kb];
}

// Start states of the segments, elementwise in fp32: Sst[n][0] = S0 (or 0), and each
// of the R pieces i of segment s in order, x <- gamma_i (per key) o x + B_i, gives
// Sst[n][s + 1]. One thread per four entries.
__global__ __launch_bounds__(256) void gla_seg_combine_kernel(const float* __restrict__ S0,
                                                              const float* __restrict__ Bbuf,
                                                              const float* __restrict__ Gbuf,
                                                              float* __restrict__ Sst, int P, int R) {
  const int n = blockIdx.x >> 4;
  const int e4 = ((blockIdx.x & 15) * 256 + threadIdx.x) * 4;   // entry of [128][128]
  const int key = e4 & (kD - 1);
  f32x4 x = S0 ? *reinterpret_cast<const f32x4*>(S0 + (size_t)n * kD * kD + e4) : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0;; ++s) {
    *reinterpret_cast<f32x4*>(Sst + ((size_t)n * P + s) * kD * kD + e4) = x;
    if (s == P - 1) break;
    for (int i = 0; i < R; ++i) {
      const size_t piece = ((size_t)n * (P - 1) + s) * R + i;
      const f32x4 g = *reinterpret_cast<const f32x4*>(Gbuf + piece * kD + key);
      const f32x4 bb = *reinterpret_cast<const f32x4*>(Bbuf + piece * kD * kD + e4);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = fmaf(g[j], x[j], bb[j]);
    }
  }
}

}  // namespace gdnrt

using namespace gdnrt;

extern "C" size_t gla_chunk_fwd_workspace_bytes(int N, int T, int dk, int dv, int chunk) {
  if (N <= 0 || T <= 0 || dk != kD || dv != kD || chunk != kChunk || T % kChunk) return 0;
  return gla::plan(N, T / kChunk).total;
}

extern "C" int gla_chunk_fwd(const void* q, const void* k, const void* v, const float* log_g,
                             const float* S0, float* ST, void* o, int N, int T, int dk, int dv,
                             int chunk, int io, void* workspace, size_t ws_bytes, void* stream) {
  if (N < 0 || T < 0) return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: N=%d T=%d must be >= 0", N, T);
  if (dk != kD || dv != kD)
    return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: d_k=%d d_v=%d, only 128 is supported", dk, dv);
  if (chunk != kChunk) return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: chunk=%d, only 64 is supported", chunk);
  if (T % kChunk) return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: T=%d is not a multiple of 64", T);
  const bool keep = (io & GDNRT_GLA_SHARD) != 0;
  if ((io & ~GDNRT_GLA_SHARD) != GDNRT_BF16)
    return set_error(GDNRT_EDTYPE, "gla_chunk_fwd: io must be GDNRT_BF16, optionally | GDNRT_GLA_SHARD");
  if ((size_t)N * (T / kChunk) > 0x7fffffffu || (size_t)N * 8 > 0x7fffffffu)
    return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: N=%d T=%d too large", N, T);
  if (N == 0) return clear_error();
  if (!ST || (T > 0 && (!q || !k || !v || !log_g || !o)))
    return set_error(GDNRT_EINVAL, "gla_chunk_fwd: null pointer argument");
  const gla::Plan pl = gla::plan(N, T / kChunk);
  const size_t need = T > 0 ? pl.total : 0;
  if (ws_bytes < need || (need && !workspace))
    return set_error(GDNRT_EINVAL, "gla_chunk_fwd: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if ((T > 0 && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_g) || !aligned16(o) ||
                 !aligned16(workspace))) ||
      !aligned4(ST) || (S0 && !aligned4(S0)))
    return set_error(GDNRT_EALIGN, "gla_chunk_fwd: q, k, v, log_g, o, workspace must be 16-byte aligned");
  const size_t ntok = (size_t)N * T, nIO = ntok * kD * 2, nG = ntok * kD * 4, nS = (size_t)N * kD * kD * 4;
  if (overlaps(o, nIO, q, nIO) || overlaps(o, nIO, k, nIO) || overlaps(o, nIO, v, nIO) ||
      overlaps(o, nIO, log_g, nG) || overlaps(o, nIO, ST, nS) || overlaps(o, nIO, S0, nS) ||
      overlaps(o, nIO, workspace, need) ||
      overlaps(ST, nS, q, nIO) || overlaps(ST, nS, k, nIO) || overlaps(ST, nS, v, nIO) ||
      overlaps(ST, nS, log_g, nG) || overlaps(ST, nS, workspace, need) ||
      (S0 && S0 != ST && overlaps(ST, nS, S0, nS)) ||
      overlaps(workspace, need, q, nIO) || overlaps(workspace, need, k, nIO) ||
      overlaps(workspace, need, v, nIO) || overlaps(workspace, need, log_g, nG) ||
      overlaps(workspace, need, S0, nS))
    return set_error(GDNRT_EINVAL, "gla_chunk_fwd: buffers overlap (only ST may equal S0)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  float* Bb = pl.P > 1 ? reinterpret_cast<float*>(ws + pl.b_off) : nullptr;
  float* Gb = pl.P > 1 ? reinterpret_cast<float*>(ws + pl.g_off) : nullptr;
  float* Sst = pl.P > 1 ? reinterpret_cast<float*>(ws + pl.s_off) : nullptr;
  if (pl.P > 1) {
    hipLaunchKernelGGL((gla_fused_kernel<false, false>), dim3((unsigned)(N * (pl.P - 1) * pl.R)), dim3(gla::NB), 0, s, q16,
                       k16, v16, log_g, ws, S0, (const float*)nullptr, Bb, Gb, (float*)nullptr, (uint16_t*)nullptr, T,
                       pl.P, pl.Lseg, pl.R);
    hipLaunchKernelGGL(gla_seg_combine_kernel, dim3((unsigned)(N * 16)), dim3(256), 0, s, S0, Bb, Gb, Sst, pl.P, pl.R);
  }
  // T == 0 launches too: the kernel then copies the incoming state (or zeros) to ST.
  if (keep)
    hipLaunchKernelGGL((gla_fused_kernel<true, true>), dim3((unsigned)(N * pl.P)), dim3(gla::NB), 0, s, q16, k16, v16,
                       log_g, ws, S0, Sst, Bb, Gb, ST, static_cast<uint16_t*>(o), T, pl.P, pl.Lseg, pl.R);
  else
    hipLaunchKernelGGL((gla_fused_kernel<true, false>), dim3((unsigned)(N * pl.P)), dim3(gla::NB), 0, s, q16, k16, v16,
                       log_g, ws, S0, Sst, Bb, Gb, ST, static_cast<uint16_t*>(o), T, pl.P, pl.Lseg, pl.R);
  return check_launch("gla_chunk_fwd");
}

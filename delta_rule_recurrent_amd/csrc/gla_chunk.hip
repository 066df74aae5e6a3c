// Gated linear attention, chunkwise forward from an incoming state (prefill shard).
//
// Method: "ZeCO: Zero Communication Overhead Sequence Parallelism for Linear
// Attention", section "Gated Linear Attention (GLA) Formulation" (per-token and
// chunk recurrences, inter/intra-chunk output) and section "The Complete Forward
// Algorithm" (the intra-chunk keys are divided by Lambda). In the [d_v][d_k] state
// layout, with b the inclusive cumulative log-gate inside a chunk of C = 64 tokens:
//
//   O   = (Q o e^b) S^T + O~,   O~ = [ ((Q o e^b)(K o e^-b)^T) o M ] V,   M lower incl. diag,
//   S  <- e^{b_C} (on key columns) o S + V^T (K o e^{b_C - b}).
//
// Everything but the state is per chunk. A first kernel forms, for every chunk in
// parallel, Q^ = Q o e^b, K^ = K o e^{b_C - b}, e^{b_C} and the intra-chunk output O~
// (its score factors taken relative to the chunk's middle token m, Q o e^{b - b_m} and
// K o e^{b_m - b}, which halves their range), and writes them to the caller's
// workspace, in bf16 and in the register order in which the second kernel feeds them
// to the matrix cores. The second kernel walks the chunks of each sequence in order
// for a tile of value channels (the value rows of S evolve independently; the tiles of
// a sequence share an XCD, so the operands they all read come from one L2): per chunk,
// O = O~ + Q^ S^T and S <- e^{b_C} o S + V^T K^, the state in fp32 MFMA accumulators,
// one barrier per chunk, the operands of the chunk two ahead in flight. bf16 MFMA
// (v_mfma_f32_16x16x32_bf16) with fp32 accumulation throughout.
#include "common.hpp"
#include "gla_chunk_layout.hpp"

namespace gdnrt {

namespace gla {

constexpr int C = kChunk;   // 64 tokens
constexpr int NT = 512;     // threads per block, both kernels
constexpr int PQ = kD + 8;   // bf16 pitch of 128-wide rows read by rows (conflict-free 16-byte reads)
constexpr int PT = kD + 16;  // bf16 pitch of 128-wide rows read transposed (conflict-free ds_read_b64_tr_b16)
constexpr int PC = C + 8;    // bf16 pitch of 64-wide rows

// The workspace layout per chunk (Q^, K^, O~ fragments, e^{b_C}) is in gla_chunk_layout.hpp.

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x8 as_bf8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float lo_bf(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// MFMA operand from a row-major [contraction][column] bf16 matrix in LDS through the
// transposing LDS read (ds_read_b64_tr_b16): lane (l16, lq) receives
// X[c0 + 8 lq + e][n0 + l16], e = 0..7.
__device__ __forceinline__ bf16x8 ld_tr8(const uint16_t* X, int pitch, int c0, int n0) {
  const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  const uint16_t* p = X + (c0 + 8 * g + (j >> 2)) * pitch + n0 + 4 * (j & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * pitch));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// lower-triangle 16 x 16 tile pairs (rb, cb), cb <= rb, numbered row by row
__device__ __forceinline__ void tri_pair(int p, int& rb, int& cb) {
  rb = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
  cb = p - (rb * (rb + 1)) / 2;
}

// ------------------------------------------------------------------ per-chunk prep

struct alignas(16) PrepSmem {
  uint16_t Q[C * PQ];       // raw q [t][k], then Q^ = q o e^b in place
  uint16_t K[C * PT];       // raw k, then K^ = k o e^{b_C - b} in place
  uint16_t V[C * PT];       // raw v [t][v]
  uint16_t Qr[C * PQ];      // q o e^{b - b_m}
  uint16_t Kr[C * PQ];      // k o e^{b_m - b}
  uint16_t A[C * PC];       // masked scores [r][j]
  float tot[8 * kD];        // log-gate sums of each group of 8 tokens
};

// One chunk's inputs: 16-byte pieces p = tid + 512 h of q, k, v (token p / 16, channels
// 8 (p % 16) ..), and the log-gates of the thread's elementwise share (channels 2 cp,
// 2 cp + 1 of tokens 8 eg .. 8 eg + 7, cp = tid % 64, eg = tid / 64).
struct PrepIn {
  u32x4 q[2], k[2], v[2];
  f32x2 g[8];
};

__device__ __forceinline__ void prep_fetch(PrepIn& in, const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ k,
                                           const uint16_t* __restrict__ v,
                                           const float* __restrict__ log_g, size_t tok0) {
  const int t = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = t + NT * h;
    const size_t off = (tok0 + (p >> 4)) * kD + (p & 15) * 8;
    in.q[h] = *reinterpret_cast<const u32x4*>(q + off);
    in.k[h] = *reinterpret_cast<const u32x4*>(k + off);
    in.v[h] = *reinterpret_cast<const u32x4*>(v + off);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    in.g[i] = *reinterpret_cast<const f32x2*>(log_g + (tok0 + 8 * (t >> 6) + i) * kD + 2 * (t & 63));
}

}  // namespace gla

namespace gla {

// One chunk of the prep: stages the inputs held in `in`, requests the next chunk's into
// `in`, and writes the chunk's operands to the workspace.
__device__ __forceinline__ void prep_chunk(PrepSmem& sm, PrepIn& in, int cid, const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                           const float* __restrict__ log_g, uint8_t* __restrict__ ws, int T,
                                           int nchunks) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int cp = tid & 63, eg = tid >> 6;   // elementwise: key-channel pair, token group of 8
  const int nc = T / C;
  uint8_t* wsc = ws + (size_t)cid * kWChunk;

  // ---- stage the raw inputs, prefix sums of the thread's log-gates (thread (cp, eg)
  // owns channels 2cp, 2cp+1 of tokens 8eg .. 8eg+7); request the next chunk's inputs
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int p = tid + NT * h, r = p >> 4, c = (p & 15) * 8;
    *reinterpret_cast<u32x4*>(sm.Q + r * PQ + c) = in.q[h];
    *reinterpret_cast<u32x4*>(sm.K + r * PT + c) = in.k[h];
    *reinterpret_cast<u32x4*>(sm.V + r * PT + c) = in.v[h];
  }
  f32x2 b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = i ? b[i - 1] + in.g[i] : in.g[i];
  *reinterpret_cast<f32x2*>(sm.tot + eg * kD + 2 * cp) = b[7];
  {
    const int nx = cid + (int)gridDim.x < nchunks ? cid + (int)gridDim.x : cid;
    prep_fetch(in, q, k, v, log_g, (size_t)(nx / nc) * T + (size_t)(nx % nc) * C);
  }
  lds_barrier();

  // ---- decayed factors of the thread's elements (each read and rewritten by its owner)
  {
    f32x2 off = {0.f, 0.f}, bm = {0.f, 0.f}, bC = {0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const f32x2 te = *reinterpret_cast<const f32x2*>(sm.tot + e * kD + 2 * cp);
      if (e < eg) off += te;
      if (e < 4) bm += te;   // b at token 31, the middle of the chunk
      bC += te;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int o = (8 * eg + i) * PQ + 2 * cp, ok = (8 * eg + i) * PT + 2 * cp;
      const f32x2 bb = b[i] + off;
      const unsigned qw = *reinterpret_cast<const unsigned*>(sm.Q + o);
      const unsigned kw = *reinterpret_cast<const unsigned*>(sm.K + ok);
      const float q0 = lo_bf(qw), q1 = hi_bf(qw), k0 = lo_bf(kw), k1 = hi_bf(kw);
      *reinterpret_cast<unsigned*>(sm.Qr + o) =
          pack_bf16(q0 * __expf(bb.x - bm.x), q1 * __expf(bb.y - bm.y));
      *reinterpret_cast<unsigned*>(sm.Kr + o) =
          pack_bf16(k0 * __expf(bm.x - bb.x), k1 * __expf(bm.y - bb.y));
      *reinterpret_cast<unsigned*>(sm.Q + o) = pack_bf16(q0 * __expf(bb.x), q1 * __expf(bb.y));
      *reinterpret_cast<unsigned*>(sm.K + ok) =
          pack_bf16(k0 * __expf(bC.x - bb.x), k1 * __expf(bC.y - bb.y));
    }
    if (eg == 0)
      *reinterpret_cast<f32x2*>(reinterpret_cast<float*>(wsc + kWE) + 2 * cp) =
          f32x2{__expf(bC.x), __expf(bC.y)};
  }
  lds_barrier();

  // ---- Q^ and K^ fragments to the workspace; masked scores A to LDS
#pragma unroll
  for (int h = 0; h < 2; ++h) {   // Q^ fragment (rb, ks) = (wave & 3, (wave >> 2) + 2h)
    const int rb = wave & 3, ks = (wave >> 2) + 2 * h;
    *reinterpret_cast<u32x4*>(wsc + kWQ + ((size_t)(rb * 4 + ks) * 64 + lane) * 16) =
        *reinterpret_cast<const u32x4*>(sm.Q + (rb * 16 + l16) * PQ + ks * 32 + lq * 8);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {   // K^ fragment f = 2 kb + js = wave + 8h
    const int f = wave + 8 * h;
    *reinterpret_cast<u32x4*>(wsc + kWK + ((size_t)f * 64 + lane) * 16) =
        __builtin_bit_cast(u32x4, ld_tr8(sm.K, PT, (f & 1) * 32, (f >> 1) * 16));
  }
  for (int u = wave; u < 10; u += 8) {   // score tiles over the lower triangle
    int rb, cb;
    tri_pair(u, rb, cb);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = mfma(ld8(sm.Qr + (rb * 16 + l16) * PQ + ks * 32 + lq * 8),
                 ld8(sm.Kr + (cb * 16 + l16) * PQ + ks * 32 + lq * 8), acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rb * 16 + lq * 4 + i, j = cb * 16 + l16;
      sm.A[r * PC + j] = f32_to_bf16(j <= r ? acc[i] : 0.f);
    }
  }
  {   // the zero upper tiles that the 32-wide contraction slices of A reach: (0,1), (2,3)
    const int t = tid >> 8, e = tid & 255;
    sm.A[(t * 32 + (e >> 4)) * PC + t * 32 + 16 + (e & 15)] = 0;
  }
  lds_barrier();

  // ---- O~ = A V: tiles (rb, vb = wave); row block rb reaches tokens <= 16 rb + 15
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int js = 0; js <= rb / 2; ++js)
      acc = mfma(ld8(sm.A + (rb * 16 + l16) * PC + js * 32 + lq * 8),
                 ld_tr8(sm.V, PT, js * 32, wave * 16), acc);
    *reinterpret_cast<u32x2*>(wsc + kWO + ((size_t)(rb * 8 + wave) * 64 + lane) * 8) =
        u32x2{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
  }
  lds_barrier();
}

}  // namespace gla

// Persistent: block b handles chunks b, b + grid, ...; the next chunk's inputs are
// loaded into registers while this one is processed, and every thread issues the
// same global loads and stores on every chunk so that the waits for them are exact
// (the first chunk is peeled, so that the loop's waits do not also serve the loads
// issued before it).
__global__ __launch_bounds__(512) void gla_chunk_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ log_g, uint8_t* __restrict__ ws, int T, int nchunks) {
  using namespace gla;
  __shared__ PrepSmem sm;
  const int nc = T / C;
  PrepIn in;
  int cid = blockIdx.x;   // the grid never exceeds nchunks
  prep_fetch(in, q, k, v, log_g, (size_t)(cid / nc) * T + (size_t)(cid % nc) * C);
  prep_chunk(sm, in, cid, q, k, v, log_g, ws, T, nchunks);
  for (cid += gridDim.x; cid < nchunks; cid += gridDim.x) prep_chunk(sm, in, cid, q, k, v, log_g, ws, T, nchunks);
}

// ------------------------------------------------------------------ sequential pass
namespace gla {

template <int VT>
struct alignas(16) SeqSmem {
  static constexpr int PV = VT == 16 ? 16 : 48;   // value-tile pitch (bf16)
  static constexpr int PO = VT + 4;               // output-tile pitch (bf16)
  uint16_t Sb[2][VT * PQ];       // bf16 copy of the state tile [v][k], by chunk parity
  uint16_t Vs[2][C * PV];        // the chunk's value tile [t][v], by chunk parity
  uint16_t Qs[2][16 * 64 * 8];   // the chunk's Q^ fragments, by chunk parity
  uint16_t Os[2][C * PO];        // the chunk's output tile [t][v], stored a chunk later
};

// VT / 8 bf16 of one token row: a thread's share of a [64][VT] tile (token tid / 8)
template <int VT>
using piece_t = typename std::conditional<VT == 32, u32x2, unsigned>::type;

// One chunk's operands for this wave, loaded two chunks ahead in three parts spread
// over the chunk's work (a burst of all of them would stall the waves' issue). Staged
// through LDS a chunk ahead (so loaded first): the thread's piece of the value tile and
// Q^ fragments `wave` and `wave + 8`, which the waves then read in the order of their
// output tiles. Kept in registers: the O~ tile (rb = wave & 3, value block
// (wave >> 2) % NVB) of the output tile, and the K^ fragments of key block `wave` with
// e^{b_C} of the lane's key for the state tiles.
template <int VT>
struct SeqIn {
  piece_t<VT> vp;
  u32x4 mq[2];
  u32x2 x;
  u32x4 kh[2];
  float ec;
};

template <int VT, int PART>
__device__ __forceinline__ void seq_fetch(SeqIn<VT>& in, const uint8_t* __restrict__ wsc,
                                          const uint16_t* __restrict__ v, size_t tok0, int vt) {
  constexpr int NVB = VT / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = wave & 3, vbl = (wave >> 2) % NVB;
  if constexpr (PART == 0) {
    in.vp = *reinterpret_cast<const piece_t<VT>*>(v + (tok0 + (tid >> 3)) * kD + vt * VT + (tid & 7) * (VT / 8));
#pragma unroll
    for (int h = 0; h < 2; ++h)
      in.mq[h] = *reinterpret_cast<const u32x4*>(wsc + kWQ + ((size_t)(wave + 8 * h) * 64 + lane) * 16);
  } else if constexpr (PART == 1) {
    in.x = *reinterpret_cast<const u32x2*>(wsc + kWO + ((size_t)(rb * 8 + vt * NVB + vbl) * 64 + lane) * 8);
    in.kh[0] = *reinterpret_cast<const u32x4*>(wsc + kWK + ((size_t)(wave * 2) * 64 + lane) * 16);
  } else {
    in.kh[1] = *reinterpret_cast<const u32x4*>(wsc + kWK + ((size_t)(wave * 2 + 1) * 64 + lane) * 16);
    in.ec = reinterpret_cast<const float*>(wsc + kWE)[wave * 16 + (lane & 15)];
  }
}

template <int VT>
__device__ __forceinline__ void seq_fetch_all(SeqIn<VT>& in, const uint8_t* __restrict__ wsc,
                                              const uint16_t* __restrict__ v, size_t tok0, int vt) {
  seq_fetch<VT, 0>(in, wsc, v, tok0, vt);
  seq_fetch<VT, 1>(in, wsc, v, tok0, vt);
  seq_fetch<VT, 2>(in, wsc, v, tok0, vt);
}

template <int VT>
__device__ __forceinline__ void stage(SeqSmem<VT>& sm, const SeqIn<VT>& in, int buf) {
  constexpr int PV = SeqSmem<VT>::PV;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  *reinterpret_cast<piece_t<VT>*>(sm.Vs[buf] + (tid >> 3) * PV + (tid & 7) * (VT / 8)) = in.vp;
#pragma unroll
  for (int h = 0; h < 2; ++h)
    *reinterpret_cast<u32x4*>(sm.Qs[buf] + ((wave + 8 * h) * 64 + lane) * 8) = in.mq[h];
}

// Stores the output tile staged in Os[buf] for the chunk starting at token tok0.
template <int VT>
__device__ __forceinline__ void store_o(const SeqSmem<VT>& sm, uint16_t* __restrict__ o, size_t tok0,
                                        int vt, int buf) {
  constexpr int PO = SeqSmem<VT>::PO;
  const int tid = threadIdx.x;
  *reinterpret_cast<piece_t<VT>*>(o + (tok0 + (tid >> 3)) * kD + vt * VT + (tid & 7) * (VT / 8)) =
      *reinterpret_cast<const piece_t<VT>*>(sm.Os[buf] + (tid >> 3) * PO + (tid & 7) * (VT / 8));
}

// One chunk: requests the operands of chunk ci + 2 into `nx` (in three parts), stores
// the previous chunk's output tile, forms this chunk's output tile into LDS, stages the
// next chunk's value tile and Q^ (from `nv`, loaded a chunk ago) and updates the state
// from `pf`. Every thread issues the same global loads and stores on every chunk (past
// the end the last chunk is loaded again; the first chunk is peeled), so the waits for
// `pf` and `nv` count exactly the memory operations issued after them.
template <int VT, bool FIRST>
__device__ __forceinline__ void gla_seq_chunk(SeqSmem<VT>& sm, const SeqIn<VT>& pf, const SeqIn<VT>& nv,
                                              SeqIn<VT>& nx, f32x4 (&Sacc)[VT / 16], int ci, int nc,
                                              size_t chunk0, size_t tokn, int vt,
                                              const uint8_t* __restrict__ ws,
                                              const uint16_t* __restrict__ v,
                                              uint16_t* __restrict__ o) {
  constexpr int NVB = VT / 16, PV = SeqSmem<VT>::PV, PO = SeqSmem<VT>::PO;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int rb = wave & 3, vbl = (wave >> 2) % NVB, kcol = wave * 16 + l16;
  const int cur = ci & 1;
  const int c2 = min(ci + 2, nc - 1);
  const uint8_t* wsc = ws + (chunk0 + c2) * kWChunk;
  const size_t tok2 = tokn + (size_t)c2 * C;
  seq_fetch<VT, 0>(nx, wsc, v, tok2, vt);
  if constexpr (!FIRST) store_o<VT>(sm, o, tokn + (size_t)(ci - 1) * C, vt, cur ^ 1);
  __builtin_amdgcn_sched_barrier(0);

  // ---- output tile (rb, vbl): O = O~ + Q^ S^T (waves w and w + 4 coincide when NVB = 1)
  {
    f32x4 acc = {lo_bf(pf.x.x), hi_bf(pf.x.x), lo_bf(pf.x.y), hi_bf(pf.x.y)};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      acc = mfma(ld8(sm.Qs[cur] + ((rb * 4 + ks) * 64 + lane) * 8),
                 ld8(sm.Sb[cur] + (vbl * 16 + l16) * PQ + ks * 32 + lq * 8), acc);
    }
    if (NVB == 2 || wave < 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.Os[cur][(rb * 16 + lq * 4 + i) * PO + vbl * 16 + l16] = f32_to_bf16(acc[i]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  seq_fetch<VT, 1>(nx, wsc, v, tok2, vt);
  __builtin_amdgcn_sched_barrier(0);
  stage<VT>(sm, nv, cur ^ 1);

  // ---- state tiles (vb, kb = wave): S <- e^{b_C} o S + V^T K^, and its next bf16 copy
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb) {
    f32x4 acc = Sacc[vb] * pf.ec;
#pragma unroll
    for (int js = 0; js < 2; ++js)
      acc = mfma(ld_tr8(sm.Vs[cur], PV, js * 32, vb * 16), as_bf8(pf.kh[js]), acc);
    Sacc[vb] = acc;
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.Sb[cur ^ 1][(vb * 16 + lq * 4 + i) * PQ + kcol] = f32_to_bf16(acc[i]);
  }
  __builtin_amdgcn_sched_barrier(0);
  seq_fetch<VT, 2>(nx, wsc, v, tok2, vt);
  lds_barrier();
}

}  // namespace gla

template <int VT>
__global__ __launch_bounds__(512) void gla_chunk_seq_kernel(
    const uint8_t* __restrict__ ws, const uint16_t* __restrict__ v, const float* __restrict__ S0,
    float* __restrict__ ST, uint16_t* __restrict__ o, int N, int T) {
  using namespace gla;
  constexpr int NVB = VT / 16;           // value blocks of 16 in the tile
  constexpr int TPS = kD / VT;           // tiles per sequence
  __shared__ SeqSmem<VT> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  // block -> (sequence, value tile); the tiles of one sequence share an XCD
  int n, vt;
  {
    const int bid = blockIdx.x;
    if ((N & 7) == 0) {
      const int xcd = bid & 7, slot = bid >> 3;
      n = (slot / TPS) * 8 + xcd;
      vt = slot % TPS;
    } else {
      n = bid / TPS;
      vt = bid % TPS;
    }
  }
  const int v0 = vt * VT;
  const int nc = T / C;
  const int kcol = wave * 16 + l16;

  // state tiles: key block = wave, value blocks vb < NVB; the lane holds
  // S[v0 + 16 vb + 4 lq + i][kcol]
  f32x4 Sacc[NVB];
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Sacc[vb][i] = S0 ? S0[((size_t)n * kD + v0 + vb * 16 + lq * 4 + i) * kD + kcol] : 0.f;
      sm.Sb[0][(vb * 16 + lq * 4 + i) * PQ + kcol] = f32_to_bf16(Sacc[vb][i]);
    }

  if (nc > 0) {
    const size_t chunk0 = (size_t)n * nc, tokn = (size_t)n * T;
    const uint8_t* wsn = ws + chunk0 * kWChunk;
    // three operand sets in rotation: chunk ci computes from set ci % 3, stages the
    // LDS operands of set (ci + 1) % 3 and loads chunk ci + 2 into set (ci + 2) % 3
    SeqIn<VT> p0, p1, p2;
    seq_fetch_all<VT>(p0, wsn, v, tokn, vt);
    {
      const int c1 = min(1, nc - 1);
      seq_fetch_all<VT>(p1, wsn + c1 * kWChunk, v, tokn + (size_t)c1 * C, vt);
    }
    stage<VT>(sm, p0, 0);
    lds_barrier();
    gla_seq_chunk<VT, true>(sm, p0, p1, p2, Sacc, 0, nc, chunk0, tokn, vt, ws, v, o);
    int ci = 1;
    for (; ci + 2 < nc; ci += 3) {
      gla_seq_chunk<VT, false>(sm, p1, p2, p0, Sacc, ci, nc, chunk0, tokn, vt, ws, v, o);
      gla_seq_chunk<VT, false>(sm, p2, p0, p1, Sacc, ci + 1, nc, chunk0, tokn, vt, ws, v, o);
      gla_seq_chunk<VT, false>(sm, p0, p1, p2, Sacc, ci + 2, nc, chunk0, tokn, vt, ws, v, o);
    }
    if (ci < nc) gla_seq_chunk<VT, false>(sm, p1, p2, p0, Sacc, ci, nc, chunk0, tokn, vt, ws, v, o);
    if (ci + 1 < nc) gla_seq_chunk<VT, false>(sm, p2, p0, p1, Sacc, ci + 1, nc, chunk0, tokn, vt, ws, v, o);
    store_o<VT>(sm, o, tokn + (size_t)(nc - 1) * C, vt, (nc - 1) & 1);
  }

#pragma unroll
  for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ST[((size_t)n * kD + v0 + vb * 16 + lq * 4 + i) * kD + kcol] = Sacc[vb][i];
}

}  // namespace gdnrt

using namespace gdnrt;

extern "C" size_t gla_chunk_fwd_workspace_bytes(int N, int T, int dk, int dv, int chunk) {
  if (N <= 0 || T <= 0 || dk != kD || dv != kD || chunk != kChunk || T % kChunk) return 0;
  return (size_t)N * (T / kChunk) * gla::kWChunk;
}

extern "C" int gla_chunk_fwd(const void* q, const void* k, const void* v, const float* log_g,
                             const float* S0, float* ST, void* o, int N, int T, int dk, int dv,
                             int chunk, int io, void* workspace, size_t ws_bytes, void* stream) {
  if (N < 0 || T < 0) return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: N=%d T=%d must be >= 0", N, T);
  if (dk != kD || dv != kD)
    return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: d_k=%d d_v=%d, only 128 is supported", dk, dv);
  if (chunk != kChunk) return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: chunk=%d, only 64 is supported", chunk);
  if (T % kChunk) return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: T=%d is not a multiple of 64", T);
  if (io != GDNRT_BF16) return set_error(GDNRT_EDTYPE, "gla_chunk_fwd: io must be GDNRT_BF16");
  if ((size_t)N * (T / kChunk) > 0x7fffffffu || (size_t)N * 8 > 0x7fffffffu)
    return set_error(GDNRT_ESHAPE, "gla_chunk_fwd: N=%d T=%d too large", N, T);
  if (N == 0) return clear_error();
  if (!ST || (T > 0 && (!q || !k || !v || !log_g || !o)))
    return set_error(GDNRT_EINVAL, "gla_chunk_fwd: null pointer argument");
  const size_t nchunks = (size_t)N * (T / kChunk);
  const size_t need = nchunks * gla::kWChunk;
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
  if (T > 0) {
    // one persistent block per CU (a block's LDS fills most of one)
    const unsigned grid = (unsigned)(nchunks < 256 ? nchunks : 256);
    hipLaunchKernelGGL(gla_chunk_prep_kernel, dim3(grid), dim3(gla::NT), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), log_g, ws, T, (int)nchunks);
    int rc = check_launch("gla_chunk_fwd (prep)");
    if (rc != GDNRT_OK) return rc;
  }
  // T == 0 launches too: the kernel then copies the incoming state (or zeros) to ST.
  // Value tiles of 16 when there are too few sequences to fill the chip with 32.
  if (N * 4 < 256)
    hipLaunchKernelGGL((gla_chunk_seq_kernel<16>), dim3((unsigned)(N * 8)), dim3(gla::NT), 0, s, ws,
                       static_cast<const uint16_t*>(v), S0, ST, static_cast<uint16_t*>(o), N, T);
  else
    hipLaunchKernelGGL((gla_chunk_seq_kernel<32>), dim3((unsigned)(N * 4)), dim3(gla::NT), 0, s, ws,
                       static_cast<const uint16_t*>(v), S0, ST, static_cast<uint16_t*>(o), N, T);
  return check_launch("gla_chunk_fwd");
}

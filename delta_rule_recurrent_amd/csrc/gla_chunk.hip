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
// The value rows of S evolve independently, so a block owns one sequence and a tile
// of value channels (the tiles of one sequence are placed on one XCD so their
// shared q/k/g reads hit the same L2) and walks the chunks in order with its state
// tile resident in MFMA accumulators (fp32). Per chunk, bf16 MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation) forms the three contractions.
// The intra-chunk factors are taken relative to the chunk's middle token m,
// Q o e^{b - b_m} and K o e^{b_m - b}, which halves their dynamic range; the
// matching e^{b_m} is folded into the bf16 copy of the state used for Q S^T.
// For the elementwise work each thread owns two adjacent key channels of a few
// consecutive tokens, whose log-gates, q, k and v are prefetched into registers
// while the previous chunk's MFMA work runs; the cumulative sums are formed in
// registers with one exchange of per-group totals.
#include "common.hpp"

namespace gdnrt {

namespace gla {

constexpr int C = kChunk;   // 64 tokens
constexpr int PQ = kD + 8;  // LDS pitch (bf16) of 128-wide rows: conflict-free 16-byte reads
constexpr int PC = C + 8;   // LDS pitch (bf16) of 64-wide rows

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// VT value channels per block, NW waves. Elementwise work: thread t owns key
// channels (2cp, 2cp+1), cp = t % 64, of TPT = 64 / NW consecutive tokens.
template <int VT, int NW>
struct Cfg {
  static constexpr int NT = 64 * NW;
  static constexpr int TPT = C / NW;           // tokens per thread
  static constexpr int NVB = VT / 16;          // value blocks
  static constexpr int SPW = 8 * NVB / NW;     // state tiles per wave
  static constexpr int OPW = 4 * NVB / NW;     // output tiles per wave
  static constexpr int APW = 16 / NW;          // score tiles per wave
  static_assert(SPW >= 1 && OPW >= 1 && APW >= 1, "tile split");
};

template <int VT, int NW>
struct Smem {
  uint16_t Qr[C * PQ];      // q o e^{b - b_m}     [r][k]
  uint16_t Kr[C * PQ];      // k o e^{b_m - b}     [j][k]
  uint16_t Kh[kD * PC];     // (k o e^{b_C - b})^T [k][j]
  uint16_t Vt[VT * PC];     // v tile transposed   [v][j]
  uint16_t A[C * PC];       // masked scores       [r][j]
  uint16_t Sb[VT * PQ];     // bf16 state tile times e^{b_m} (per key column) [v][k]
  float tot[NW * kD];       // per token-group log-gate sums
  float eC[kD];
};

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One chunk's inputs for this thread: log-gates, q, k pairs of its TPT tokens and,
// when 2cp < VT, the pair of value channels v0 + 2cp, +1.
template <int TPT>
struct Prefetch {
  f32x2 g[TPT];
  unsigned q[TPT], k[TPT], v[TPT];
};

template <int VT, int NW>
__device__ __forceinline__ void fetch(Prefetch<C / NW>& pf, const uint16_t* __restrict__ q,
                                      const uint16_t* __restrict__ k,
                                      const uint16_t* __restrict__ v,
                                      const float* __restrict__ log_g, size_t tok0, int v0) {
  constexpr int TPT = C / NW;
  const int t = threadIdx.x, cp = t & 63, e = t >> 6;
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const size_t row = tok0 + TPT * e + i;
    pf.g[i] = *reinterpret_cast<const f32x2*>(log_g + row * kD + 2 * cp);
    pf.q[i] = *reinterpret_cast<const unsigned*>(q + row * kD + 2 * cp);
    pf.k[i] = *reinterpret_cast<const unsigned*>(k + row * kD + 2 * cp);
    // every thread loads (an in-bounds pair when 2cp >= VT, unused): a select on a
    // loaded value would make the compiler wait for the load right here
    pf.v[i] = *reinterpret_cast<const unsigned*>(v + row * kD + v0 + ((2 * cp) & (VT - 1)));
  }
}

// One chunk: E1/E2 form the decayed operands from the prefetched inputs, then the
// next chunk's inputs are requested and M1/M2 run the contractions.
template <int VT, int NW>
__device__ __forceinline__ void gla_step(Smem<VT, NW>& sm, Prefetch<C / NW>& pf,
                                         f32x4 (&Sacc)[Cfg<VT, NW>::SPW],
                                         const uint16_t* __restrict__ q,
                                         const uint16_t* __restrict__ k,
                                         const uint16_t* __restrict__ v,
                                         const float* __restrict__ log_g,
                                         uint16_t* __restrict__ o, size_t seq, int c0, int T,
                                         int v0, int kcol, int vbase) {
  using CF = Cfg<VT, NW>;
  constexpr int TPT = CF::TPT, SPW = CF::SPW, OPW = CF::OPW, APW = CF::APW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int cp = tid & 63, eg = tid >> 6;
  // ---- E1: prefix sums of this thread's tokens, group totals to LDS
  f32x2 b[TPT];
  b[0] = pf.g[0];
#pragma unroll
  for (int i = 1; i < TPT; ++i) b[i] = b[i - 1] + pf.g[i];
  *reinterpret_cast<f32x2*>(sm.tot + eg * kD + 2 * cp) = b[TPT - 1];
  lds_barrier();

  // ---- E2: decay factors and operands; the bf16 state copy times e^{b_m}
  {
    f32x2 off = {0.f, 0.f}, bm = {0.f, 0.f}, bC = {0.f, 0.f};
#pragma unroll
    for (int e = 0; e < NW; ++e) {
      const f32x2 te = *reinterpret_cast<const f32x2*>(sm.tot + e * kD + 2 * cp);
      if (e < eg) off += te;
      if (e < NW / 2) bm += te;
      bC += te;
    }
    // one exponential and one reciprocal per element: p = e^{b - b_m};
    // e^{b_m - b} = 1/p, e^{b_C - b} = e^{b_C - b_m} / p
    const f32x2 eCm = {__expf(bC.x - bm.x), __expf(bC.y - bm.y)};
    float kh0[TPT], kh1[TPT], vv0[TPT], vv1[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int r = TPT * eg + i;
      const f32x2 bb = b[i] + off;
      const float p0 = __expf(bb.x - bm.x), p1 = __expf(bb.y - bm.y);
      const float r0 = __builtin_amdgcn_rcpf(p0), r1 = __builtin_amdgcn_rcpf(p1);
      const float k0 = __uint_as_float(pf.k[i] << 16), k1 = __uint_as_float(pf.k[i] & 0xffff0000u);
      *reinterpret_cast<unsigned*>(sm.Qr + r * PQ + 2 * cp) =
          pack_bf16(__uint_as_float(pf.q[i] << 16) * p0, __uint_as_float(pf.q[i] & 0xffff0000u) * p1);
      *reinterpret_cast<unsigned*>(sm.Kr + r * PQ + 2 * cp) = pack_bf16(k0 * r0, k1 * r1);
      kh0[i] = k0 * r0 * eCm.x;
      kh1[i] = k1 * r1 * eCm.y;
      vv0[i] = __uint_as_float(pf.v[i] << 16);
      vv1[i] = __uint_as_float(pf.v[i] & 0xffff0000u);
    }
    // transposed rows: TPT consecutive tokens of one key (value) channel
    if constexpr (TPT == 8) {
      u32x4 w0, w1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0[i] = pack_bf16(kh0[2 * i], kh0[2 * i + 1]);
        w1[i] = pack_bf16(kh1[2 * i], kh1[2 * i + 1]);
      }
      *reinterpret_cast<u32x4*>(sm.Kh + (2 * cp) * PC + TPT * eg) = w0;
      *reinterpret_cast<u32x4*>(sm.Kh + (2 * cp + 1) * PC + TPT * eg) = w1;
      {
        // every thread writes: threads whose channel pair repeats modulo VT hold
        // the same values (the load wraps the column), so their writes agree;
        // a branch here would make the compiler wait for every outstanding load
        const int vc = (2 * cp) & (VT - 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w0[i] = pack_bf16(vv0[2 * i], vv0[2 * i + 1]);
          w1[i] = pack_bf16(vv1[2 * i], vv1[2 * i + 1]);
        }
        *reinterpret_cast<u32x4*>(sm.Vt + vc * PC + TPT * eg) = w0;
        *reinterpret_cast<u32x4*>(sm.Vt + (vc + 1) * PC + TPT * eg) = w1;
      }
    } else {
      static_assert(TPT == 4, "4 or 8 tokens per thread");
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      u32x2 w0 = {pack_bf16(kh0[0], kh0[1]), pack_bf16(kh0[2], kh0[3])};
      u32x2 w1 = {pack_bf16(kh1[0], kh1[1]), pack_bf16(kh1[2], kh1[3])};
      *reinterpret_cast<u32x2*>(sm.Kh + (2 * cp) * PC + TPT * eg) = w0;
      *reinterpret_cast<u32x2*>(sm.Kh + (2 * cp + 1) * PC + TPT * eg) = w1;
      if (2 * cp < VT) {
        w0 = u32x2{pack_bf16(vv0[0], vv0[1]), pack_bf16(vv0[2], vv0[3])};
        w1 = u32x2{pack_bf16(vv1[0], vv1[1]), pack_bf16(vv1[2], vv1[3])};
        *reinterpret_cast<u32x2*>(sm.Vt + (2 * cp) * PC + TPT * eg) = w0;
        *reinterpret_cast<u32x2*>(sm.Vt + (2 * cp + 1) * PC + TPT * eg) = w1;
      }
    }
    if (eg == 0) {
      const f32x2 em = {__expf(bm.x), __expf(bm.y)};
      sm.eC[2 * cp] = eCm.x * em.x;
      sm.eC[2 * cp + 1] = eCm.y * em.y;
    }
    // this wave's state tiles, scaled by e^{b_m} of their key column
    float bmk = 0.f;
#pragma unroll
    for (int e = 0; e < NW / 2; ++e) bmk += sm.tot[e * kD + kcol];
    const float emk = __expf(bmk);
#pragma unroll
    for (int j = 0; j < SPW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sm.Sb[((vbase + j) * 16 + lq * 4 + i) * PQ + kcol] = f32_to_bf16(Sacc[j][i] * emk);
  }
  lds_barrier();
  // next chunk's inputs, overlapping the MFMA work; unconditional (the last chunk
  // loads itself again) so the waits for them count exactly the loads issued after
  fetch<VT, NW>(pf, q, k, v, log_g, seq + min(c0 + C, T - C), v0);

  // ---- M1: masked intra-chunk scores (APW tiles per wave)
#pragma unroll
  for (int j = 0; j < APW; ++j) {
    const int u = wave * APW + j, rb = u & 3, cb = u >> 2;
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
  lds_barrier();

  // ---- M2: outputs (OPW tiles per wave) and the state update
#pragma unroll
  for (int j = 0; j < OPW; ++j) {
    const int u = wave * OPW + j, rb = u & 3, vb = u >> 2;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = mfma(ld8(sm.Qr + (rb * 16 + l16) * PQ + ks * 32 + lq * 8),
                 ld8(sm.Sb + (vb * 16 + l16) * PQ + ks * 32 + lq * 8), acc);
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
    const int kb = wave & 7;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int vb = vbase + j;
      f32x4 acc = Sacc[j] * dec;
#pragma unroll
      for (int js = 0; js < 2; ++js)
        acc = mfma(ld8(sm.Vt + (vb * 16 + l16) * PC + js * 32 + lq * 8),
                   ld8(sm.Kh + (kb * 16 + l16) * PC + js * 32 + lq * 8), acc);
      Sacc[j] = acc;
    }
  }
  lds_barrier();
}

}  // namespace gla

template <int VT, int NW>
__global__ __launch_bounds__(64 * NW) void gla_chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ log_g, const float* __restrict__ S0, float* __restrict__ ST,
    uint16_t* __restrict__ o, int N, int T) {
  using namespace gla;
  using CF = Cfg<VT, NW>;
  constexpr int TPT = CF::TPT, NVB = CF::NVB, SPW = CF::SPW, OPW = CF::OPW, APW = CF::APW;
  constexpr int TPS = kD / VT;   // value tiles per sequence
  __shared__ Smem<VT, NW> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int cp = tid & 63, eg = tid >> 6;   // elementwise: key-channel pair, token group

  // block -> (sequence, value tile); the tiles of one sequence share an XCD
  int n, vt;
  const int bid = blockIdx.x;
  if (TPS > 1 && (N & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3;
    n = (slot / TPS) * 8 + xcd;
    vt = slot % TPS;
  } else {
    n = bid / TPS;
    vt = bid % TPS;
  }
  const int v0 = vt * VT;

  // state tiles: key block kb = wave % 8, value blocks (wave / 8) * SPW + j; lane holds
  // S[v0 + vb*16 + lq*4 + i][kb*16 + l16]
  const int kcol = (wave & 7) * 16 + l16;
  const int vbase = (wave >> 3) * SPW;
  f32x4 Sacc[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vrow = v0 + (vbase + j) * 16 + lq * 4 + i;
      Sacc[j][i] = S0 ? S0[((size_t)n * kD + vrow) * kD + kcol] : 0.f;
    }

  const size_t seq = (size_t)n * T;
  Prefetch<TPT> pf;
  if (T > 0) {
    fetch<VT, NW>(pf, q, k, v, log_g, seq, v0);
    // the first chunk is peeled so that the loop is entered, as on every later
    // iteration, with one chunk of loads and then that chunk's output stores in
    // flight: the waits for the loads then count the stores and do not wait for them
    gla_step<VT, NW>(sm, pf, Sacc, q, k, v, log_g, o, seq, 0, T, v0, kcol, vbase);
    for (int c0 = C; c0 < T; c0 += C)
      gla_step<VT, NW>(sm, pf, Sacc, q, k, v, log_g, o, seq, c0, T, v0, kcol, vbase);
  }

#pragma unroll
  for (int j = 0; j < SPW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int vrow = v0 + (vbase + j) * 16 + lq * 4 + i;
      ST[((size_t)n * kD + vrow) * kD + kcol] = Sacc[j][i];
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
  // four 32-channel value tiles per sequence, 8 waves each: measured on MI355X at
  // 64 sequences x 4096 tokens, this beats 64- and 128-channel tiles, whose MFMA
  // operands re-read from LDS saturate a single CU's LDS bandwidth
  hipLaunchKernelGGL((gla_chunk_kernel<32, 8>), dim3((unsigned)(N * 4)), dim3(512), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), log_g, S0,
                     ST, static_cast<uint16_t*>(o), N, T);
  return check_launch("gla_chunk_fwd");
}

// Gated linear attention, chunkwise backward of one sequence shard.
//
// Method: "ZeCO: Zero Communication Overhead Sequence Parallelism for Linear
// Attention", section "The Backward Algorithm and Gradient Flow": the state gradient
// runs backward over the chunks, dS <- gamma o dS + Q~^T dO, and each chunk's
// gradients combine an intra-chunk part (through its attention matrix) and an
// inter-chunk part (through the states). In the [d_v][d_k] layout, with b the
// inclusive cumulative log-gate inside a chunk of C = 64 tokens, b_m its value at
// token 31 and b_C at token 63, the forward of a chunk is
//
//   Q^ = Q o e^b, K^ = K o e^{b_C - b}, Q~ = Q o e^{b - b_m}, K~ = K o e^{b_m - b},
//   A = (Q~ K~^T) o M,  O = Q^ S_b^T + A V,  S_a = e^{b_C} o S_b + V^T K^
//
// (S_b the state before the chunk, S_a after), so with dS_a the gradient with respect
// to S_a and dO given:
//
//   dS_b = e^{b_C} o dS_a + dO^T Q^                         (the backward state scan)
//   dA = (dO V^T) o M,  dQ^ = dO S_b,  dQ~ = dA K~,  dK~ = dA^T Q~,  dK^ = V dS_a,
//   dq = (dQ^ e^{b_m} + dQ~) e^{b - b_m},   dk = (dK~ + dK^ e^{b_C - b_m}) e^{b_m - b},
//   dv = A^T dO + K^ dS_a^T.
//
// The gate gradient uses that b enters only through q o e^B and k o e^{-B} (B the
// cumulative log-gate over the whole sequence): dL/dB_t = q_t o dq_t - k_t o dk_t,
// and d log_g_t = sum_{s >= t} dL/dB_s. Shifting B on every token after a chunk (in one
// key channel) scales that key column of the state the next chunk starts from, so the
// part of the sum beyond the chunk is sum_v dS_a o S_a (dST o S_T after the last
// chunk): only sums over at most 64 tokens remain, and no rounding error accumulates
// along the sequence.
//
// Since S_a = e^{b_C} o S_b + V^T K^, that boundary sum is, per key channel,
// e^{b_C} sum_v dS_a o S_b + sum_t K^ o (V dS_a): both products are at hand where a
// chunk's gradients are formed, so the backward state scan needs no forward state.
//
// Three launches: a per-chunk prep (cumulative gates, the scaled operands); the forward
// state scan (the state before every chunk) and the backward state scan (the gradient
// after every chunk, and dS_0), independent of each other, side by side in one launch;
// and a per-chunk gradient kernel (bf16 MFMA, fp32 accumulation; also the boundary sums
// and the gate gradient).
#include "chunk_device.hpp"

namespace gdnrt {

namespace glab {

using namespace gdc;   // C, PS, sw_off, ld8, ld_tr8, ld_tr8s, mfma
constexpr int PT = PS;       // bf16 pitch of 128-wide rows, stored with swz (rows and transposed reads)
constexpr int PA = C + 8;    // bf16 pitch of 64-wide rows: a transposed read's groups of lanes,
                             // 8 rows apart, fall 32 banks apart; 16 rows read by rows on distinct banks
constexpr int PX = 16 + 16;  // bf16 pitch of 16-wide rows (one value tile), rows with bit 3 set
                             // in the upper half (columns 16..31): a transposed read's groups
                             // of lanes, 8 rows apart, on distinct banks
__device__ __forceinline__ int px_off(int row, int col) { return row * PX + col + ((row & 8) << 1); }

// Workspace per chunk (bytes): bf16 [64][128] Q^, K^; fp32 [64][128] E = e^{b - b_m};
// fp32 [128] e^{b_C}, e^{b_m}, e^{b_C - b_m}; bf16 [128][128] the state before the
// chunk and the state gradient after it.
constexpr size_t kQh = 0, kKh = 16384, kE = 32768, kEC = 65536, kEm = 66048, kECm = 66560,
                 kSb = 67072, kdS = 99840, kChunkB = 132608;

// ld_tr8 from a 16-wide tile stored with px_off
__device__ __forceinline__ bf16x8 ld_tr8x(const uint16_t* X, int c0) {
  const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  const uint16_t* p = X + px_off(c0 + 8 * g + (j >> 2), 4 * (j & 3));
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * PX));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace glab

// ------------------------------------------------------------------ prep
// One block of 256 threads per chunk: thread (cq = tid % 32, h = tid / 32) covers key
// channels 4 cq .. 4 cq + 3 over tokens 8 h .. 8 h + 7.
__global__ __launch_bounds__(256) void gla_bwd_prep_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           const float* __restrict__ log_g,
                                                           uint8_t* __restrict__ ws, int T) {
  using namespace glab;
  __shared__ f32x4 tot[8][32];
  const int tid = threadIdx.x, cq = tid & 31, h = tid >> 5, c0 = 4 * cq;
  const int nc = T / C, cid = blockIdx.x;
  const size_t tok0 = (size_t)(cid / nc) * T + (size_t)(cid % nc) * C + 8 * h;
  uint8_t* wsc = ws + (size_t)cid * kChunkB;
  f32x4 gv[8];
  u32x2 qv[8], kv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    gv[i] = *reinterpret_cast<const f32x4*>(log_g + (tok0 + i) * kD + c0);
    qv[i] = *reinterpret_cast<const u32x2*>(q + (tok0 + i) * kD + c0);
    kv[i] = *reinterpret_cast<const u32x2*>(k + (tok0 + i) * kD + c0);
  }
  f32x4 run = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    run += gv[i];
    gv[i] = run;   // prefix within the segment
  }
  tot[h][cq] = run;
  lds_barrier();
  f32x4 base = {0.f, 0.f, 0.f, 0.f}, bm = base, bC;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const f32x4 x = tot[j][cq];
    if (j < h) base += x;
    if (j < 4) bm += x;
  }
  bC = bm + tot[4][cq] + tot[5][cq] + tot[6][cq] + tot[7][cq];
  uint16_t* Qh = reinterpret_cast<uint16_t*>(wsc + kQh);
  uint16_t* Kh = reinterpret_cast<uint16_t*>(wsc + kKh);
  float* E = reinterpret_cast<float*>(wsc + kE);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = 8 * h + i;
    float qh[4], kh[4];
    f32x4 e;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float b = base[j] + gv[i][j];
      const float qf = bf16_to_f32(uint16_t(qv[i][j >> 1] >> (16 * (j & 1))));
      const float kf = bf16_to_f32(uint16_t(kv[i][j >> 1] >> (16 * (j & 1))));
      e[j] = __expf(b - bm[j]);
      qh[j] = qf * __expf(b);
      kh[j] = kf * __expf(bC[j] - b);
    }
    *reinterpret_cast<u32x2*>(Qh + t * kD + c0) = u32x2{pack_bf16(qh[0], qh[1]), pack_bf16(qh[2], qh[3])};
    *reinterpret_cast<u32x2*>(Kh + t * kD + c0) = u32x2{pack_bf16(kh[0], kh[1]), pack_bf16(kh[2], kh[3])};
    *reinterpret_cast<f32x4*>(E + t * kD + c0) = e;
  }
  if (h == 0) {
    f32x4 ec, em, ecm;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ec[j] = __expf(bC[j]);
      em[j] = __expf(bm[j]);
      ecm[j] = __expf(bC[j] - bm[j]);
    }
    *reinterpret_cast<f32x4*>(wsc + kEC + 4 * c0) = ec;
    *reinterpret_cast<f32x4*>(wsc + kEm + 4 * c0) = em;
    *reinterpret_cast<f32x4*>(wsc + kECm + 4 * c0) = ecm;
  }
}

// ------------------------------------------------------------------ state scans
// One block of 256 threads per (sequence, value tile of 16 rows); wave w owns key
// columns [32 w, 32 w + 32) as two 16 x 16 accumulator tiles (lane holds rows
// 4 lq + i, column 32 w + 16 j + l16). Per chunk (forward: first to last; reverse: last
// to first) the state is stored in bf16 to the workspace, then
//   forward:  S  <- e^{b_C} o S  + V^T K^     (X = V,  Y = K^)
//   reverse:  dS <- e^{b_C} o dS + dO^T Q^    (X = dO, Y = Q^).
// The next chunk's X and Y are loaded into registers while this one is computed.
// (bid, grid): this tile's block among the scan's blocks.
template <bool REV>
__device__ __forceinline__ void gla_scan_tile(const uint16_t* __restrict__ X, uint8_t* __restrict__ ws,
                                              const float* __restrict__ Sinit, float* __restrict__ Sout,
                                              int T, int bid, int grid) {
  using namespace glab;
  __shared__ __attribute__((aligned(16))) uint16_t sx[C * PX];
  __shared__ __attribute__((aligned(16))) uint16_t sy[C * PT];
  __shared__ __attribute__((aligned(16))) uint16_t sst[16 * PT];   // the tile in bf16
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, lq = lane >> 4;
  const int tr = tid >> 4, tc = 8 * (tid & 15);   // a thread's 8 entries of a [16][128] tile
  // block -> (sequence, value tile); the 8 tiles of one sequence share an XCD (blocks
  // are dealt to the 8 XCDs round robin), so the scaled keys or queries they all read
  // are fetched into that XCD's L2 once
  int n, vt;
  if ((grid & 63) == 0) {
    n = (bid >> 6) * 8 + (bid & 7);
    vt = (bid >> 3) & 7;
  } else {
    n = bid >> 3;
    vt = bid & 7;
  }
  const int v0 = vt * 16;
  const int nc = T / C;
  const size_t chunk0 = (size_t)n * nc;
  const size_t soff = REV ? kQh : kKh;   // Y: Q^ (reverse) or K^ (forward)
  f32x4 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[j][i] = Sinit ? Sinit[((size_t)n * kD + v0 + 4 * lq + i) * kD + 32 * w + 16 * j + l16] : 0.f;

  // thread's pieces: X row tid / 4, values 4 (tid % 4) ..; Y 16-byte pieces tid + 256 p
  struct Ops {
    u32x2 xr;
    u32x4 yr[4];
    float ec[2];
  };
  auto load = [&](int ci, Ops& o) {
    const size_t tok = (size_t)n * T + (size_t)ci * C;
    o.xr = *reinterpret_cast<const u32x2*>(X + (tok + (tid >> 2)) * kD + v0 + 4 * (tid & 3));
    const uint8_t* wsc = ws + (chunk0 + ci) * kChunkB;
#pragma unroll
    for (int p = 0; p < 4; ++p) o.yr[p] = *reinterpret_cast<const u32x4*>(wsc + soff + (size_t)(tid + 256 * p) * 16);
#pragma unroll
    for (int j = 0; j < 2; ++j) o.ec[j] = reinterpret_cast<const float*>(wsc + kEC)[32 * w + 16 * j + l16];
  };
  // chunk s from `cur`, requesting the next chunk's operands into `nxt` (past the end the
  // last chunk's again, so that every chunk issues the same loads and the waits count
  // exactly); the two sets alternate through a loop unrolled by two, so neither is
  // copied into the other (a copy would wait for the loads in the chunk that issued
  // them), and the first chunk is peeled, so that the loop is entered with the same
  // operations in flight on both paths (the next set's loads, then a store)
  auto body = [&](int s, const Ops& cur, Ops& nxt) {
    const int ci = REV ? nc - 1 - s : s;
    // this chunk's state (forward) or state gradient (reverse) in bf16, staged in LDS
    // and stored after the barrier one 16-byte piece per thread
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sst[sw_off(4 * lq + i, 32 * w + 16 * j + l16)] = f32_to_bf16(acc[j][i]);
    *reinterpret_cast<u32x2*>(sx + px_off(tid >> 2, 4 * (tid & 3))) = cur.xr;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int e = (tid + 256 * p) * 8;   // element index in [64][128]
      *reinterpret_cast<u32x4*>(sy + sw_off(e >> 7, e & 127)) = cur.yr[p];
    }
    load(REV ? (ci > 0 ? ci - 1 : 0) : (ci + 1 < nc ? ci + 1 : ci), nxt);
    lds_barrier();
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(ws + (chunk0 + ci) * kChunkB + (REV ? kdS : kSb)) +
                              (size_t)(v0 + tr) * kD + tc) = *reinterpret_cast<const u32x4*>(sst + sw_off(tr, tc));
    acc[0] *= cur.ec[0];
    acc[1] *= cur.ec[1];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 a = ld_tr8x(sx, 32 * ks);
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[j] = mfma(a, ld_tr8s(sy, 32 * ks, 32 * w + 16 * j), acc[j]);
    }
    lds_barrier();
  };
  if (nc > 0) {
    Ops A, B;
    load(REV ? nc - 1 : 0, A);
    body(0, A, B);
    int s = 1;
    for (; s + 2 <= nc; s += 2) {
      body(s, B, A);
      body(s + 1, A, B);
    }
    if (s < nc) body(s, B, A);
  }
  if (Sout)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) Sout[((size_t)n * kD + v0 + 4 * lq + i) * kD + 32 * w + 16 * j + l16] = acc[j][i];
}

// The two state scans in one launch: the first half of the blocks runs the forward
// scan's tiles (states before every chunk), the second half the backward scan's
// (gradients after every chunk, and dS_0), tile for tile, so that a tile's XCD is the
// same in both halves. Both are serial chains over the chunks at one block per tile.
__global__ __launch_bounds__(256) void gla_bwd_scans_kernel(const uint16_t* __restrict__ v,
                                                            const uint16_t* __restrict__ dO,
                                                            uint8_t* __restrict__ ws,
                                                            const float* __restrict__ S0,
                                                            const float* __restrict__ dST,
                                                            float* __restrict__ dS0, int T) {
  const int grid = (int)gridDim.x >> 1, b = blockIdx.x;
  if (b < grid)
    gla_scan_tile<false>(v, ws, S0, nullptr, T, b, grid);
  else
    gla_scan_tile<true>(dO, ws, dST, dS0, T, b - grid, grid);
}

// The backward state scan alone (a shard's dS_0 from a zero gradient, or T = 0).
__global__ __launch_bounds__(256) void gla_bwd_rscan_kernel(const uint16_t* __restrict__ dO,
                                                            uint8_t* __restrict__ ws,
                                                            const float* __restrict__ dST,
                                                            float* __restrict__ dS0, int T) {
  gla_scan_tile<true>(dO, ws, dST, dS0, T, blockIdx.x, gridDim.x);
}

// ------------------------------------------------------------------ gradients
// One block of 512 threads (8 waves) per chunk.
struct alignas(16) GradSmem {
  uint16_t Qt[kChunk * glab::PT], Kt[kChunk * glab::PT], dO[kChunk * glab::PT];   // [t][128]
  uint16_t Sb[kD * glab::PT], dS[kD * glab::PT];                                 // [v][c]
  uint16_t A[kChunk * glab::PA], dA[kChunk * glab::PA];                          // [r][j], upper tiles zero
  // per key channel: sum_v dS_a o S_b per wave, sum_t K~ o (V dS_a) per token block
  float b1[8][kD], b2[4][kD];
};

__global__ __launch_bounds__(512) void gla_bwd_grad_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const uint8_t* __restrict__ ws, uint16_t* __restrict__ dq, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    float* __restrict__ dg, int T) {
  using namespace glab;
  __shared__ GradSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, lq = lane >> 4;
  const int nc = T / C, cid = blockIdx.x;
  const size_t tok0 = (size_t)(cid / nc) * T + (size_t)(cid % nc) * C;
  const uint8_t* wsc = ws + (size_t)cid * kChunkB;

  // ---- stage: Q~ = Q o E, K~ = K / E and dO rows ([64][128]: 1024 pieces of 8
  // elements each), the state before the chunk and the gradient after it ([128][128]:
  // 2048 pieces each); zeros for A and dA
  const float* E = reinterpret_cast<const float*>(wsc + kE);
  // every global read of the staging is requested before the first one is used, so
  // that a block (one per CU) waits one memory round trip here instead of three
  u32x4 qin[2], kin[2], oin[2], sbin[4], dsin[4];
  f32x4 e0in[2], e1in[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int e = (tid + 512 * p) * 8, r = e >> 7, cc = e & 127;
    qin[p] = *reinterpret_cast<const u32x4*>(q + (tok0 + r) * kD + cc);
    kin[p] = *reinterpret_cast<const u32x4*>(k + (tok0 + r) * kD + cc);
    e0in[p] = *reinterpret_cast<const f32x4*>(E + e);
    e1in[p] = *reinterpret_cast<const f32x4*>(E + e + 4);
    oin[p] = *reinterpret_cast<const u32x4*>(dO + (tok0 + r) * kD + cc);
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int e = (tid + 512 * p) * 8;
    sbin[p] = *reinterpret_cast<const u32x4*>(wsc + kSb + (size_t)e * 2);
    dsin[p] = *reinterpret_cast<const u32x4*>(wsc + kdS + (size_t)e * 2);
  }
  // V fragments of the odd waves' dA tiles (below): tile u = w + 8 i, rows 16 cb + l16
  bf16x8 vin[3][4];
  if (w & 1) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int u = w + 8 * i;
      if (u >= 20) break;
      const int p = u >> 1;
      const int rb = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3, cb = p - (rb * (rb + 1)) / 2;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) vin[i][ks] = ld8(v + (tok0 + 16 * cb + l16) * kD + 32 * ks + 8 * lq);
    }
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int e = (tid + 512 * p) * 8, r = e >> 7, cc = e & 127;
    const u32x4 qq = qin[p], kk = kin[p];
    const f32x4 e0 = e0in[p], e1 = e1in[p];
    u32x4 qt, kt;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float ea = j < 2 ? e0[2 * j] : e1[2 * j - 4], eb = j < 2 ? e0[2 * j + 1] : e1[2 * j - 3];
      qt[j] = pack_bf16(bf16_to_f32(uint16_t(qq[j])) * ea, bf16_to_f32(uint16_t(qq[j] >> 16)) * eb);
      kt[j] = pack_bf16(bf16_to_f32(uint16_t(kk[j])) / ea, bf16_to_f32(uint16_t(kk[j] >> 16)) / eb);
    }
    *reinterpret_cast<u32x4*>(sm.Qt + sw_off(r, cc)) = qt;
    *reinterpret_cast<u32x4*>(sm.Kt + sw_off(r, cc)) = kt;
    *reinterpret_cast<u32x4*>(sm.dO + sw_off(r, cc)) = oin[p];
  }
  // and this thread's part of sum_v dS_a o S_b for its 8 key channels 8 (tid % 16) ..
  float b1[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int e = (tid + 512 * p) * 8, r = e >> 7, cc = e & 127;
    const u32x4 sb = sbin[p], ds = dsin[p];
    *reinterpret_cast<u32x4*>(sm.Sb + sw_off(r, cc)) = sb;
    *reinterpret_cast<u32x4*>(sm.dS + sw_off(r, cc)) = ds;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b1[2 * j] += lo_bf(sb[j]) * lo_bf(ds[j]);
      b1[2 * j + 1] += hi_bf(sb[j]) * hi_bf(ds[j]);
    }
  }
  // the four lanes of a wave with these channels, then one row of partials per wave
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    b1[j] += __shfl_xor(b1[j], 16);
    b1[j] += __shfl_xor(b1[j], 32);
  }
  if (lq == 0)
#pragma unroll
    for (int j = 0; j < 8; ++j) sm.b1[w][8 * l16 + j] = b1[j];
  for (int e = tid; e < C * PA / 2; e += 512) {
    reinterpret_cast<uint32_t*>(sm.A)[e] = 0u;
    reinterpret_cast<uint32_t*>(sm.dA)[e] = 0u;
  }
  lds_barrier();

  // ---- A = (Q~ K~^T) o M and dA = (dO V^T) o M: 10 lower tiles each; wave w takes
  // tiles u = w, w + 8, w + 16 (< 20), dA tiles on the odd waves, whose V fragments
  // were requested with the staging reads
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int u = w + 8 * i;
    if (u >= 20) break;
    const int p = u >> 1;
    const int rb = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3, cb = p - (rb * (rb + 1)) / 2;
    const bool grad = u & 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (grad) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma(ld8(sm.dO + sw_off(16 * rb + l16, 32 * ks + 8 * lq)), vin[i][ks], acc);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma(ld8(sm.Qt + sw_off(16 * rb + l16, 32 * ks + 8 * lq)),
                   ld8(sm.Kt + sw_off(16 * cb + l16, 32 * ks + 8 * lq)), acc);
    }
    uint16_t* dst = grad ? sm.dA : sm.A;
    const int j = 16 * cb + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rb + 4 * lq + i;
      dst[r * PA + j] = f32_to_bf16(j <= r ? acc[i] : 0.f);
    }
  }
  lds_barrier();

  // ---- output tiles (rb, cb): rows t = 16 rb + 4 lq + i, columns 16 cb + l16
  const float* em = reinterpret_cast<const float*>(wsc + kEm);
  const float* ecm = reinterpret_cast<const float*>(wsc + kECm);
  const uint16_t* Kh = reinterpret_cast<const uint16_t*>(wsc + kKh);
  const int rb = w & 3;
  float dB[4][4];   // dL/dB of this lane's tile elements
#pragma unroll 1
  for (int u = 0; u < 4; ++u) {
    const int cb = (w >> 2) * 4 + u;
    const int col = 16 * cb + l16;
    f32x4 dQh = {0.f, 0.f, 0.f, 0.f}, dQt = dQh, dKt = dQh, dKh = dQh, dV = dQh;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      dQh = mfma(ld8(sm.dO + sw_off(16 * rb + l16, 32 * ks + 8 * lq)), ld_tr8s(sm.Sb, 32 * ks, 16 * cb), dQh);
      dKh = mfma(ld8(v + (tok0 + 16 * rb + l16) * kD + 32 * ks + 8 * lq), ld_tr8s(sm.dS, 32 * ks, 16 * cb), dKh);
      dV = mfma(ld8(Kh + (16 * rb + l16) * kD + 32 * ks + 8 * lq), ld8(sm.dS + sw_off(16 * cb + l16, 32 * ks + 8 * lq)), dV);
    }
#pragma unroll
    for (int js = 0; js < 2; ++js) {
      if (js <= rb / 2)   // dA[t][j] is zero for j > t
        dQt = mfma(ld8(sm.dA + (16 * rb + l16) * PA + 32 * js + 8 * lq), ld_tr8s(sm.Kt, 32 * js, 16 * cb), dQt);
      if (32 * js + 31 >= 16 * rb) {   // dA[r][t], A[r][t] are zero for r < t
        dKt = mfma(ld_tr8(sm.dA, PA, 32 * js, 16 * rb), ld_tr8s(sm.Qt, 32 * js, 16 * cb), dKt);
        dV = mfma(ld_tr8(sm.A, PA, 32 * js, 16 * rb), ld_tr8s(sm.dO, 32 * js, 16 * cb), dV);
      }
    }
    const float emc = em[col], ecmc = ecm[col];
    float b2 = 0.f;   // sum over this lane's 4 tokens of K~ o (V dS_a); K^ = K~ e^{b_C - b_m}
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * rb + 4 * lq + i;
      const size_t g = (tok0 + t) * kD + col;
      const float e = E[t * kD + col];
      const float gq = (dQh[i] * emc + dQt[i]) * e;
      const float gk = (dKt[i] + dKh[i] * ecmc) / e;
      dq[g] = f32_to_bf16(gq);
      dk[g] = f32_to_bf16(gk);
      dv[g] = f32_to_bf16(dV[i]);
      const float x = bf16_to_f32(q[g]) * gq - bf16_to_f32(k[g]) * gk;
      b2 += bf16_to_f32(sm.Kt[sw_off(t, col)]) * dKh[i];
#pragma unroll
      for (int uu = 0; uu < 4; ++uu)   // constant register index under the rolled tile loop
        if (uu == u) dB[uu][i] = x;
    }
    b2 += __shfl_xor(b2, 16);
    b2 += __shfl_xor(b2, 32);
    if (lq == 0) sm.b2[rb][col] = b2 * ecmc;
  }

  // ---- d log_g: the reverse cumulative sum of dL/dB over the chunk's tokens (fp32
  // [64][132] over the state tiles, 16-token segment totals over A) plus the chunk's
  // sum_v dS_a o S_a = e^{b_C} sum_v dS_a o S_b + sum_t K^ o (V dS_a)
  constexpr int PG = kD + 4;
  float* G = reinterpret_cast<float*>(sm.Sb);
  float* seg = reinterpret_cast<float*>(sm.A);   // [4][128] segment totals
  lds_barrier();
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) G[(16 * rb + 4 * lq + i) * PG + 16 * ((w >> 2) * 4 + u) + l16] = dB[u][i];
  const int c = tid & (kD - 1), h = tid >> 7;
  float start;
  {
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s1 += sm.b1[i][c];
#pragma unroll
    for (int i = 0; i < 4; ++i) s2 += sm.b2[i][c];
    start = reinterpret_cast<const float*>(wsc + kEC)[c] * s1 + s2;
  }
  lds_barrier();
  float run = 0.f, x[16];
#pragma unroll
  for (int t = 15; t >= 0; --t) {
    run += G[(16 * h + t) * PG + c];
    x[t] = run;
  }
  seg[h * kD + c] = run;
  lds_barrier();
  float off = start;
  for (int j = 3; j > h; --j) off += seg[j * kD + c];
  float* p = dg + (tok0 + 16 * h) * kD + c;
#pragma unroll
  for (int t = 0; t < 16; ++t) p[(size_t)t * kD] = x[t] + off;
}

}  // namespace gdnrt

using namespace gdnrt;

extern "C" size_t gla_chunk_bwd_workspace_bytes(int N, int T, int dk, int dv, int chunk) {
  if (N <= 0 || T <= 0 || dk != kD || dv != kD || chunk != kChunk || T % kChunk) return 0;
  // per chunk the operands and states
  return (size_t)N * (T / kChunk) * glab::kChunkB;
}

// prepared: the per-chunk operands are already in the workspace (gla_shard_bwd_state
// ran on the same q, k, log_g), so the preparation kernel is not launched again
static int chunk_bwd(const char* fn, bool prepared, const void* q, const void* k, const void* v,
                     const float* log_g, const float* S0, const void* dO, const float* dST, void* dq,
                     void* dk, void* dv, float* dlog_g, float* dS0, int N, int T, int dk_, int dv_, int chunk,
                     int io, void* workspace, size_t ws_bytes, void* stream) {
  if (N < 0 || T < 0) return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d must be >= 0", fn, N, T);
  if (dk_ != kD || dv_ != kD) return set_error(GDNRT_ESHAPE, "%s: d_k=%d d_v=%d, only 128 is supported", fn, dk_, dv_);
  if (chunk != kChunk) return set_error(GDNRT_ESHAPE, "%s: chunk=%d, only 64 is supported", fn, chunk);
  if (T % kChunk) return set_error(GDNRT_ESHAPE, "%s: T=%d is not a multiple of 64", fn, T);
  if (io != GDNRT_BF16) return set_error(GDNRT_EDTYPE, "%s: io must be GDNRT_BF16", fn);
  if ((size_t)N * (T / kChunk) > 0x7fffffffu || (size_t)N * 16 > 0x7fffffffu)
    return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d too large", fn, N, T);
  if (N == 0) return clear_error();
  if (!dS0 || (T > 0 && (!q || !k || !v || !log_g || !dO || !dq || !dk || !dv || !dlog_g)))
    return set_error(GDNRT_EINVAL, "%s: null pointer argument", fn);
  const size_t nchunks = (size_t)N * (T / kChunk);
  const size_t need = nchunks * glab::kChunkB;
  if (ws_bytes < need || (need && !workspace))
    return set_error(GDNRT_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
  if ((T > 0 && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(log_g) ||
                 !aligned4(dq) || !aligned4(dk) || !aligned4(dv) || !aligned4(dlog_g))) ||
      !aligned16(workspace) || !aligned4(dS0) || (S0 && !aligned4(S0)) || (dST && !aligned4(dST)))
    return set_error(GDNRT_EALIGN, "%s: q, k, v, dO, log_g, workspace must be 16-byte aligned", fn);
  const size_t ntok = (size_t)N * T, nIO = ntok * kD * 2, nG = ntok * kD * 4, nS = (size_t)N * kD * kD * 4;
  const void* ins[] = {q, k, v, dO};
  const void* outs[] = {dq, dk, dv};
  for (const void* a : outs) {
    for (const void* b : ins)
      if (overlaps(a, nIO, b, nIO)) return set_error(GDNRT_EINVAL, "%s: a gradient overlaps an input", fn);
    for (const void* b : outs)
      if (a != b && overlaps(a, nIO, b, nIO)) return set_error(GDNRT_EINVAL, "%s: gradients overlap", fn);
    if (overlaps(a, nIO, dlog_g, nG) || overlaps(a, nIO, workspace, need) || overlaps(a, nIO, log_g, nG))
      return set_error(GDNRT_EINVAL, "%s: buffers overlap", fn);
  }
  for (const void* b : ins)
    if (overlaps(dlog_g, nG, b, nIO) || overlaps(workspace, need, b, nIO) || overlaps(dS0, nS, b, nIO))
      return set_error(GDNRT_EINVAL, "%s: buffers overlap", fn);
  if (overlaps(dlog_g, nG, log_g, nG) || overlaps(dlog_g, nG, workspace, need) ||
      overlaps(workspace, need, log_g, nG) || overlaps(dS0, nS, workspace, need) ||
      overlaps(dS0, nS, dlog_g, nG) || overlaps(workspace, need, S0, nS) || overlaps(workspace, need, dST, nS))
    return set_error(GDNRT_EINVAL, "%s: buffers overlap", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (T == 0) {   // no tokens: the state gradient passes through
    hipLaunchKernelGGL(gla_bwd_rscan_kernel, dim3((unsigned)(N * 8)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(dO), ws, dST, dS0, 0);
    return check_launch(fn);
  }
  if (!prepared) {
    hipLaunchKernelGGL(gla_bwd_prep_kernel, dim3((unsigned)nchunks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), log_g, ws, T);
    int rc = check_launch(fn);
    if (rc != GDNRT_OK) return rc;
  }
  hipLaunchKernelGGL(gla_bwd_scans_kernel, dim3((unsigned)(N * 16)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), ws, S0, dST, dS0, T);
  hipLaunchKernelGGL(gla_bwd_grad_kernel, dim3((unsigned)nchunks), dim3(512), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), ws,
                     static_cast<uint16_t*>(dq), static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv),
                     dlog_g, T);
  return check_launch(fn);
}

extern "C" int gla_chunk_bwd(const void* q, const void* k, const void* v, const float* log_g,
                             const float* S0, const void* dO, const float* dST, void* dq, void* dk,
                             void* dv, float* dlog_g, float* dS0, int N, int T, int dk_, int dv_,
                             int chunk, int io, void* workspace, size_t ws_bytes, void* stream) {
  return chunk_bwd("gla_chunk_bwd", false, q, k, v, log_g, S0, dO, dST, dq, dk, dv, dlog_g, dS0, N, T, dk_, dv_,
                   chunk, io, workspace, ws_bytes, stream);
}

extern "C" int gla_shard_bwd_grads(const void* q, const void* k, const void* v, const float* log_g,
                                   const float* S0, const void* dO, const float* dST, void* dq, void* dk,
                                   void* dv, float* dlog_g, float* dS0, int N, int T, int dk_, int dv_,
                                   int chunk, int io, void* workspace, size_t ws_bytes, void* stream) {
  return chunk_bwd("gla_shard_bwd_grads", true, q, k, v, log_g, S0, dO, dST, dq, dk, dv, dlog_g, dS0, N, T, dk_,
                   dv_, chunk, io, workspace, ws_bytes, stream);
}

extern "C" int gla_shard_bwd_state(const void* q, const void* k, const float* log_g, const void* dO, float* dS0,
                                   int N, int T, int dk_, int dv_, int chunk, int io, void* workspace,
                                   size_t ws_bytes, void* stream) {
  const char* fn = "gla_shard_bwd_state";
  if (N < 0 || T < 0) return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d must be >= 0", fn, N, T);
  if (dk_ != kD || dv_ != kD) return set_error(GDNRT_ESHAPE, "%s: d_k=%d d_v=%d, only 128 is supported", fn, dk_, dv_);
  if (chunk != kChunk) return set_error(GDNRT_ESHAPE, "%s: chunk=%d, only 64 is supported", fn, chunk);
  if (T % kChunk) return set_error(GDNRT_ESHAPE, "%s: T=%d is not a multiple of 64", fn, T);
  if (io != GDNRT_BF16) return set_error(GDNRT_EDTYPE, "%s: io must be GDNRT_BF16", fn);
  if ((size_t)N * (T / kChunk) > 0x7fffffffu) return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d too large", fn, N, T);
  if (N == 0) return clear_error();
  if (!dS0 || (T > 0 && (!q || !k || !log_g || !dO || !workspace)))
    return set_error(GDNRT_EINVAL, "%s: null pointer argument", fn);
  const size_t nchunks = (size_t)N * (T / kChunk);
  const size_t need = nchunks * glab::kChunkB;
  if (ws_bytes < need) return set_error(GDNRT_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
  if ((T > 0 && (!aligned16(q) || !aligned16(k) || !aligned16(dO) || !aligned16(log_g) || !aligned16(workspace))) ||
      !aligned4(dS0))
    return set_error(GDNRT_EALIGN, "%s: q, k, dO, log_g, workspace must be 16-byte aligned", fn);
  const size_t ntok = (size_t)N * T, nIO = ntok * kD * 2, nG = ntok * kD * 4, nS = (size_t)N * kD * kD * 4;
  const void* ins[] = {q, k, dO};
  for (const void* b : ins)
    if (overlaps(dS0, nS, b, nIO) || overlaps(workspace, need, b, nIO))
      return set_error(GDNRT_EINVAL, "%s: buffers overlap", fn);
  if (overlaps(dS0, nS, log_g, nG) || overlaps(dS0, nS, workspace, need) || overlaps(workspace, need, log_g, nG))
    return set_error(GDNRT_EINVAL, "%s: buffers overlap", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (T > 0) {
    hipLaunchKernelGGL(gla_bwd_prep_kernel, dim3((unsigned)nchunks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), log_g, ws, T);
    int rc = check_launch(fn);
    if (rc != GDNRT_OK) return rc;
  }
  // the reverse scan from a zero gradient
  hipLaunchKernelGGL(gla_bwd_rscan_kernel, dim3((unsigned)(N * 8)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(dO), ws, nullptr, dS0, T);
  return check_launch(fn);
}

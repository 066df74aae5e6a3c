// Gated DeltaNet chunkwise backward of one sequence shard.
//
// The recurrence is the one of "LeapQuant: an 8-bit recurrent state that stops
// rounding every token", section "The state, from the update rule up" (eq. 3); the
// pages print no chunk form and no backward for it. The forward's chunk form (UT /
// WY, state [d_v][d_k], C = 64 tokens, g_r = prod_{i<=r} alpha_i inside the chunk):
//
//   T = (I + L)^-1,  L[r,j] = beta_r (g_r/g_j) k_r.k_j (j < r),
//   W = T diag(beta g) K,  U~ = T diag(beta) V,  U = U~ - W S_b^T,
//   A = M o (g_r/g_j) o Q K^T,  O = diag(g) Q S_b^T + A U,
//   S_a = g_C S_b + U^T K^,  K^ = diag(g_C/g) K,   Q' = diag(g) Q - A W,
//
// (S_b the state before the chunk, S_a after). Differentiating it, with dS_a given:
//
//   dS_b = g_C dS_a + dO^T Q' - (K^ dS_a^T)^T W              (backward state scan)
//   dU   = A^T dO + K^ dS_a^T,   dA' = (dO U^T) o M o (g_r/g_j)
//   dq   = dA' K + diag(g) dO S_b
//   dk   = dA'^T Q + diag(g_C/g) U dS_a + (T diag(beta g))^T dW + dL' K + dL'^T K
//   dW   = -dU S_b,   dv = (T diag(beta))^T dU
//   dL   = -(T^T dW W^T + T^T dU U~^T) o strict_lower,  dL' = dL o (g_r/g_j) o beta_r
//   dbeta = g o rowdot(T^T dW, K) + rowdot(T^T dU, V) + rowsum(dL o (g_r/g_j) o K K^T)
//
// and the decay gradient from the fact that, with B_t the cumulative log-decay over
// the sequence, S_t e^{-B_t} follows the undecayed delta rule driven by v_t e^{-B_t}
// and read by q_t e^{B_t}: dL/dB_t = q_t.dq_t - v_t.dv_t and d log alpha_t =
// sum_{s >= t} dL/dB_s. Shifting B on every token after a chunk scales the state the
// next chunk starts from, so the part of that sum beyond the chunk is sum(dS_a o S_a)
// (dST o S_T after the last chunk); the rest is a sum over at most 64 tokens, and no
// rounding error accumulates along the sequence. dalpha = d log alpha / alpha.
//
// Since S_a = g_C S_b + U^T K^, that boundary sum is g_C sum(dS_a o S_b) +
// sum(diag(g_C/g) U dS_a o K), two products the chunk's gradients form anyway, so the
// backward state scan needs no forward state.
//
// Kernels: the forward's chunk prep (which also stores T); the forward state scan (the
// state before every chunk, bf16) and the backward state scan (the gradient after every
// chunk, bf16, and dS_0), independent of each other, side by side in one launch; and
// two gradient kernels over the chunks (persistent, one block per CU; bf16 MFMA, fp32
// accumulation), the first of which also forms each chunk's boundary sum.
#include "chunk_device.hpp"
#include "gdn_chunk_layout.hpp"

namespace gdnrt {

void gdn_chunk_prep_with_inverse(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const float* alpha, const float* beta, uint8_t* ws, uint16_t* Tout,
                                 int T, int nchunks, hipStream_t s);

namespace gdb {

using namespace gdc;   // C, PS, sw_off, ld8, ld_tr8, ld_tr8s, mfma, lo_bf, hi_bf, wave_scan, tri_pair
constexpr int PT = PS;       // bf16 pitch of 128-wide rows, stored with swz
constexpr int PA = C + 8;    // bf16 pitch of 64-wide rows (a transposed read's groups of
                             // lanes 8 rows apart fall 32 banks apart; rows read by 16
                             // lanes on distinct banks)
constexpr int PX = 16 + 16;  // bf16 pitch of 16-wide rows; rows with bit 3 set are stored in
                             // the upper half (columns 16..31), so that a transposed read's
                             // groups of lanes, 8 rows apart, fall on distinct banks
__device__ __forceinline__ int px_off(int row, int col) { return row * PX + col + ((row & 8) << 1); }
// ld_tr8 from a 16-wide tile stored with px_off
__device__ __forceinline__ bf16x8 ld_tr8x(const uint16_t* X, int c0) {
  const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  const uint16_t* p = X + px_off(c0 + 8 * g + (j >> 2), 4 * (j & 3));
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * PX));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
constexpr int PFK = kD + 4;  // fp32 pitch of 128-wide rows

__device__ __forceinline__ bf16x8 as_bf(u32x4 x) { return as_bf8(x); }
// 8 keys of row `row` of a tile stored with swz, in the prep fragments' order: 4 at
// column c, 4 at c + 16
__device__ __forceinline__ bf16x8 ld8_split_s(const uint16_t* X, int row, int c) {
  const u32x2 a = *reinterpret_cast<const u32x2*>(X + sw_off(row, c));
  const u32x2 b = *reinterpret_cast<const u32x2*>(X + sw_off(row, c + 16));
  return as_bf(u32x4{a.x, a.y, b.x, b.y});
}
// block -> (sequence, value tile of 16); the 8 tiles of one sequence share an XCD
// (blocks are dealt to the 8 XCDs round robin), so the chunk operands they all read
// are fetched into that XCD's L2 once
__device__ __forceinline__ void seq_tile(int& n, int& vt, int bid, int grid) {
  if ((grid & 63) == 0) {
    n = (bid >> 6) * 8 + (bid & 7);
    vt = (bid >> 3) & 7;
  } else {
    n = bid >> 3;
    vt = bid & 7;
  }
}

// Workspace regions of the backward, each an array over chunks (then sequences).
struct Ws {
  uint8_t* prep;   // the forward prep's operands, kWsChunk bytes per chunk
  uint16_t* T;     // (I + L)^-1, bf16 [64][64]
  uint16_t* Sb;    // state before the chunk, bf16 [128][128]
  uint16_t* dSa;   // state gradient after the chunk, bf16 [128][128]
  uint16_t* dU;    // dU, bf16 [64][128]
  u32x2* dK1;      // dA'^T Q + diag(g_C/g) U dS_a, bf16 in the gradient kernels' lane order:
                   // piece (wave, u, lane) holds the lane's 4 rows of tile (w % 4, 4 (w / 4) + u)
  float* qdq;      // q_t . dq_t, fp32 [64]
  float* bnd;      // sum(dS_a o S_a), fp32, one per chunk
};

}  // namespace gdb

// ------------------------------------------------------------------ forward state scan
// One block of 256 threads per (sequence, value tile of 16 rows); wave w owns key
// columns [32 w, 32 w + 32) of the state (lane holds rows 4 lq + i, columns
// 32 w + 16 j + l16) and token block w of U. Per chunk: store the state (bf16), then
// U = U~ - W S^T for this tile's values and S <- g_C S + U^T K^, with the prep's
// fragments as MFMA operands straight from registers (next chunk's loaded ahead).
// (bid, grid): this tile's block among the scan's blocks.
__device__ __forceinline__ void fscan_tile(const uint8_t* __restrict__ prep, const float* __restrict__ S0,
                                           uint16_t* __restrict__ Sb, int T, int bid, int grid) {
  using namespace gdb;
  __shared__ __attribute__((aligned(16))) uint16_t sS[16 * PT];
  __shared__ __attribute__((aligned(16))) uint16_t sU[16 * PA];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, lq = lane >> 4;
  int n, vt;
  seq_tile(n, vt, bid, grid);
  const int v0 = 16 * vt, nc = T / C;
  const size_t chunk0 = (size_t)n * nc;
  f32x4 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[j][i] = S0 ? S0[((size_t)n * kD + v0 + 4 * lq + i) * kD + 32 * w + 16 * j + l16] : 0.f;
  struct Ops {
    u32x4 w[4], kh[4];
    u32x2 u;
    float gc;
  };
  auto load = [&](size_t cid, Ops& o) {
    const uint8_t* pc = prep + cid * kWsChunk;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      o.w[ks] = *reinterpret_cast<const u32x4*>(pc + kWsW + ((size_t)(w * 4 + ks) * 64 + lane) * 16);
#pragma unroll
    for (int f = 0; f < 4; ++f)   // K^ fragments (kb, js) = (2 w + f / 2, f % 2)
      o.kh[f] = *reinterpret_cast<const u32x4*>(pc + kWsK + ((size_t)(4 * w + f) * 64 + lane) * 16);
    o.u = *reinterpret_cast<const u32x2*>(pc + kWsU + ((size_t)(w * 8 + vt) * 64 + lane) * 8);
    o.gc = *reinterpret_cast<const float*>(pc + kWsG + l16 * 4);
  };
  // chunk s: its operands were requested two chunks earlier; it requests those of
  // chunk s + 2 (past the end the last chunk's again, so that every chunk issues the same
  // loads and the waits count exactly) into the set chunk s - 1 used. The three sets
  // rotate through an unrolled loop, so each stays in registers.
  auto body = [&](int s, const Ops& cur, Ops& fut) {
    load(chunk0 + min(s + 2, nc - 1), fut);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sS[sw_off(4 * lq + i, 32 * w + 16 * j + l16)] = f32_to_bf16(acc[j][i]);
    lds_barrier();
    // the tile's bf16 copy to the workspace: row tid / 16, 8 columns per thread
    *reinterpret_cast<u32x4*>(Sb + (chunk0 + s) * kD * kD + (size_t)(v0 + (tid >> 4)) * kD + 8 * (tid & 15)) =
        *reinterpret_cast<const u32x4*>(sS + sw_off(tid >> 4, 8 * (tid & 15)));
    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) p = mfma(as_bf(cur.w[ks]), ld8_split_s(sS, l16, 32 * ks + 4 * lq), p);
    const float u0 = lo_bf(cur.u.x) - p[0], u1 = hi_bf(cur.u.x) - p[1];
    const float u2 = lo_bf(cur.u.y) - p[2], u3 = hi_bf(cur.u.y) - p[3];
    *reinterpret_cast<u32x2*>(sU + l16 * PA + 16 * w + 4 * lq) = u32x2{pack_bf16(u0, u1), pack_bf16(u2, u3)};
    lds_barrier();
    acc[0] *= cur.gc;
    acc[1] *= cur.gc;
#pragma unroll
    for (int js = 0; js < 2; ++js) {
      const bf16x8 a = ld8(sU + l16 * PA + 32 * js + 8 * lq);
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[j] = mfma(a, as_bf(cur.kh[2 * j + js]), acc[j]);
    }
  };
  if (nc > 0) {
    Ops P0, P1, P2;
    load(chunk0, P0);
    load(chunk0 + min(1, nc - 1), P1);
    int s = 0;
    for (; s + 3 <= nc; s += 3) {
      body(s, P0, P2);
      body(s + 1, P1, P0);
      body(s + 2, P2, P1);
    }
    if (s < nc) body(s, P0, P2);
    if (s + 1 < nc) body(s + 1, P1, P0);
  }
}

// ------------------------------------------------------------------ backward state scan
// One block of 256 threads per (sequence, value tile of 16 rows), chunks last to
// first; wave w owns key columns [32 w, 32 w + 32) of dS and token block w of
// K^ dS^T. Per chunk: store dS (bf16, the gradient after the chunk), stage K^ (as
// K^^T), Q', W and this tile's dO in LDS, then
//   dS <- g_C dS + dO^T Q' - (K^ dS^T)^T W.
// It reads no forward state, so it runs beside the forward scan (below).
__device__ __forceinline__ void rscan_tile(const uint8_t* __restrict__ prep, const uint16_t* __restrict__ dO,
                                           const float* __restrict__ dST, uint16_t* __restrict__ dSa,
                                           float* __restrict__ dS0, int T, int bid, int grid) {
  using namespace gdb;
  __shared__ __attribute__((aligned(16))) uint16_t sD[16 * PT];
  __shared__ __attribute__((aligned(16))) uint16_t sKt[kD * PA];
  __shared__ __attribute__((aligned(16))) uint16_t sQ[C * PT];
  __shared__ __attribute__((aligned(16))) uint16_t sW[C * PT];
  __shared__ __attribute__((aligned(16))) uint16_t sO[C * PX];
  __shared__ __attribute__((aligned(16))) uint16_t sdU[16 * PA];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, lq = lane >> 4;
  int n, vt;
  seq_tile(n, vt, bid, grid);
  const int v0 = 16 * vt, nc = T / C;
  const size_t chunk0 = (size_t)n * nc;
  const int tr = tid >> 4, tc = 8 * (tid & 15);   // a thread's 8 entries of a [16][128] tile
  f32x4 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[j][i] = dST ? dST[((size_t)n * kD + v0 + 4 * lq + i) * kD + 32 * w + 16 * j + l16] : 0.f;
  struct Ops {
    u32x4 kh[4], qp[4], w[4];
    u32x2 o;
    float gc;
  };
  // fragment f = w + 4 p of each 16-fragment operand, this lane's 16 bytes
  auto load = [&](int ci, Ops& o) {
    const uint8_t* pc = prep + (chunk0 + ci) * kWsChunk;
    o.gc = *reinterpret_cast<const float*>(pc + kWsG + l16 * 4);
    o.o = *reinterpret_cast<const u32x2*>(dO + ((size_t)n * T + (size_t)ci * C + (tid >> 2)) * kD + v0 + 4 * (tid & 3));
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const size_t off = ((size_t)(w + 4 * p) * 64 + lane) * 16;
      o.kh[p] = *reinterpret_cast<const u32x4*>(pc + kWsK + off);
      o.qp[p] = *reinterpret_cast<const u32x4*>(pc + kWsQ + off);
      o.w[p] = *reinterpret_cast<const u32x4*>(pc + kWsW + off);
    }
  };
  Ops cur, nxt;
  if (nc > 0) load(nc - 1, nxt);
  for (int s = 0; s < nc; ++s) {
    const int ci = nc - 1 - s;
    cur = nxt;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sD[sw_off(4 * lq + i, 32 * w + 16 * j + l16)] = f32_to_bf16(acc[j][i]);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int f = w + 4 * p;
      // K^ fragment (kb, js) = (f / 2, f % 2): key kb*16 + l16, tokens js*32 + lq*8 ..
      *reinterpret_cast<u32x4*>(sKt + ((f >> 1) * 16 + l16) * PA + (f & 1) * 32 + lq * 8) = cur.kh[p];
      // W, Q' fragments (rb, ks) = (f / 4, f % 4): token rb*16 + l16, keys split by 16
      const int rr = (f >> 2) * 16 + l16, c0 = (f & 3) * 32 + lq * 4;
      const int o0 = sw_off(rr, c0), o1 = sw_off(rr, c0 + 16);
      *reinterpret_cast<u32x2*>(sW + o0) = u32x2{cur.w[p].x, cur.w[p].y};
      *reinterpret_cast<u32x2*>(sW + o1) = u32x2{cur.w[p].z, cur.w[p].w};
      *reinterpret_cast<u32x2*>(sQ + o0) = u32x2{cur.qp[p].x, cur.qp[p].y};
      *reinterpret_cast<u32x2*>(sQ + o1) = u32x2{cur.qp[p].z, cur.qp[p].w};
    }
    *reinterpret_cast<u32x2*>(sO + px_off(tid >> 2, 4 * (tid & 3))) = cur.o;
    lds_barrier();
    // the tile's bf16 copy to the workspace, one 16-byte store per thread; then the
    // previous chunk's operands are requested (every chunk issues the same loads, the
    // last one chunk 0 again): the waits for them then never include this store
    *reinterpret_cast<u32x4*>(dSa + (chunk0 + ci) * kD * kD + (size_t)(v0 + tr) * kD + tc) =
        *reinterpret_cast<const u32x4*>(sD + sw_off(tr, tc));
    __builtin_amdgcn_sched_barrier(0);   // keeps the loads after the store
    load(ci > 0 ? ci - 1 : 0, nxt);
    // -(K^ dS^T)^T for tokens 16 w .. 16 w + 15: [v][t]
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) x = mfma(ld8(sD + sw_off(l16, 32 * ks + 8 * lq)), ld_tr8(sKt, PA, 32 * ks, 16 * w), x);
#pragma unroll
    for (int i = 0; i < 4; ++i) sdU[(4 * lq + i) * PA + 16 * w + l16] = f32_to_bf16(-x[i]);
    lds_barrier();
    acc[0] *= cur.gc;
    acc[1] *= cur.gc;
#pragma unroll
    for (int js = 0; js < 2; ++js) {
      const bf16x8 ao = ld_tr8x(sO, 32 * js);
      const bf16x8 au = ld8(sdU + l16 * PA + 32 * js + 8 * lq);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[j] = mfma(ao, ld_tr8s(sQ, 32 * js, 32 * w + 16 * j), acc[j]);
        acc[j] = mfma(au, ld_tr8s(sW, 32 * js, 32 * w + 16 * j), acc[j]);
      }
    }
    lds_barrier();
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) dS0[((size_t)n * kD + v0 + 4 * lq + i) * kD + 32 * w + 16 * j + l16] = acc[j][i];
}

// The two state scans in one launch: the first half of the blocks runs the forward
// scan's tiles, the second half the backward scan's, tile for tile, so that a tile's
// XCD (blocks are dealt to the XCDs round robin) is the same in both halves. Both are
// serial chains over the chunks at one block per tile. Measured on MI355X: with the
// halves interleaved every 8 blocks (so that a CU's two blocks took the same scan)
// the launch took 687 us at 32 x 16,384 tokens, with the halves 629 us, against
// 258 + 490 us as two launches; with the backward scan's waves at a higher issue
// priority (s_setprio) 531 us.
__global__ __launch_bounds__(256) void gdn_bwd_scans_kernel(const uint8_t* __restrict__ prep,
                                                            const float* __restrict__ S0,
                                                            uint16_t* __restrict__ Sb,
                                                            const uint16_t* __restrict__ dO,
                                                            const float* __restrict__ dST,
                                                            uint16_t* __restrict__ dSa,
                                                            float* __restrict__ dS0, int T) {
  const int grid = (int)gridDim.x >> 1, b = blockIdx.x, tile = b < grid ? b : b - grid;
  if (b < grid) {
    fscan_tile(prep, S0, Sb, T, tile, grid);
  } else {
    // the backward scan is the longer chain (about 490 against 258 us alone at 32 x
    // 16,384 tokens): its waves issue first, the forward scan's fill in around them
    __builtin_amdgcn_s_setprio(2);
    rscan_tile(prep, dO, dST, dSa, dS0, T, tile, grid);
  }
}

// T = 0: the state gradient passes through (dS0 = dST, or zero)
__global__ __launch_bounds__(256) void gdn_bwd_pass_kernel(const float* __restrict__ dST, float* __restrict__ dS0) {
  rscan_tile(nullptr, nullptr, dST, nullptr, dS0, 0, blockIdx.x, gridDim.x);
}

// ------------------------------------------------------------------ gradients, part 1
// Persistent blocks of 512 threads (8 waves), one per CU (LDS); block b takes chunks b,
// b + grid, ... and loads the next chunk's q, k, dO, S_b, dS_a and alpha into registers
// while it works on this one. Per chunk: U, A, dU (to the workspace), dA', dq (final,
// with q_t . dq_t) and dK1 = dA'^T Q + diag(g_C/g) U dS_a (to the workspace).
// Output tiles (rb, cb): wave w takes token block rb = w % 4 and column blocks
// cb = 4 (w / 4) .. + 3; lane holds rows 16 rb + 4 lq + i of column 16 cb + l16.
struct alignas(16) G1Smem {
  uint16_t Q[kChunk * gdb::PT], K[kChunk * gdb::PT], O[kChunk * gdb::PT];   // [t][128]
  uint16_t S[kD * gdb::PT], D[kD * gdb::PT];                                 // S_b, dS_a [v][c]
  uint16_t U[kChunk * gdb::PT];                                              // [t][v]
  uint16_t A[kChunk * gdb::PA];                                              // A, then dA' [r][j]
  float lg[kChunk], g[kChunk], kd[kChunk];
  float qdq[2][kChunk];   // q_t . dq_t over key blocks 0-3 and 4-7 (the two wave halves)
  float bs[8][2];         // per wave: sum(dS_a o S_b), sum(diag(g_C/g) U dS_a o K)
};

namespace gdb {
// one chunk's inputs of a grad1 thread: 16-byte pieces tid + 512 p of q, k, dO (rows of
// 128) and of S_b, dS_a; alpha of token lane
struct G1In {
  u32x4 q[2], k[2], o[2], s[4], d[4];
  float al;
};
__device__ __forceinline__ void g1_fetch(G1In& in, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                         const uint16_t* __restrict__ dO, const float* __restrict__ alpha,
                                         const Ws& ws, int cid, int T) {
  const int tid = threadIdx.x, nc = T / C;
  const size_t tok0 = (size_t)(cid / nc) * T + (size_t)(cid % nc) * C;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const size_t gi = tok0 * kD + (size_t)(tid + 512 * p) * 8;
    in.q[p] = *reinterpret_cast<const u32x4*>(q + gi);
    in.k[p] = *reinterpret_cast<const u32x4*>(k + gi);
    in.o[p] = *reinterpret_cast<const u32x4*>(dO + gi);
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const size_t e = (size_t)cid * kD * kD + (size_t)(tid + 512 * p) * 8;
    in.s[p] = *reinterpret_cast<const u32x4*>(ws.Sb + e);
    in.d[p] = *reinterpret_cast<const u32x4*>(ws.dSa + e);
  }
  in.al = alpha[tok0 + (tid & 63)];
}
}  // namespace gdb

__global__ __launch_bounds__(512) void gdn_bwd_grad1_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ dO,
    const float* __restrict__ alpha, gdb::Ws ws, uint16_t* __restrict__ dq, int T, int nchunks) {
  using namespace gdb;
  __shared__ G1Smem sm;
  const int nc = T / C;
  G1In in;
  g1_fetch(in, q, k, dO, alpha, ws, blockIdx.x, T);   // the grid never exceeds nchunks
  // the first chunk is peeled, so that the loop is entered with the same memory
  // operations in flight on both paths (the next chunk's loads, then this chunk's
  // stores) and the waits for the prefetched inputs never include the stores
  auto chunk = [&](const int cid) {
    // the thread index through an opaque move: the per-lane addresses are formed inside
    // each chunk instead of being held across the loop
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    const int lane = tid & 63, w = tid >> 6, l16 = lane & 15, lq = lane >> 4, rb = w & 3;
    const size_t tok0 = (size_t)(cid / nc) * T + (size_t)(cid % nc) * C;
    const uint8_t* pc = ws.prep + (size_t)cid * kWsChunk;

#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int e = (tid + 512 * p) * 8, r = e >> 7, cc = e & 127;
      *reinterpret_cast<u32x4*>(sm.Q + sw_off(r, cc)) = in.q[p];
      *reinterpret_cast<u32x4*>(sm.K + sw_off(r, cc)) = in.k[p];
      *reinterpret_cast<u32x4*>(sm.O + sw_off(r, cc)) = in.o[p];
    }
    float bs1 = 0.f;   // this thread's part of sum(dS_a o S_b)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int e = (tid + 512 * p) * 8, r = e >> 7, cc = e & 127;
      *reinterpret_cast<u32x4*>(sm.S + sw_off(r, cc)) = in.s[p];
      *reinterpret_cast<u32x4*>(sm.D + sw_off(r, cc)) = in.d[p];
      const uint32_t sv[4] = {in.s[p].x, in.s[p].y, in.s[p].z, in.s[p].w};
      const uint32_t dv[4] = {in.d[p].x, in.d[p].y, in.d[p].z, in.d[p].w};
#pragma unroll
      for (int i = 0; i < 4; ++i)   // two bf16 products per instruction, summed in fp32
        bs1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, sv[i]), __builtin_bit_cast(bf16x2, dv[i]), bs1, false);
    }
    for (int e = tid; e < C * PA / 2; e += 512) reinterpret_cast<uint32_t*>(sm.A)[e] = 0u;
    if (w == 0) {
      const float lgv = wave_scan(__logf(in.al));
      const float lC = __shfl(lgv, C - 1);
      sm.lg[lane] = lgv;
      sm.g[lane] = __expf(lgv);
      sm.kd[lane] = __expf(lC - lgv);
    }
    // this chunk's W and U~ fragments, then the next chunk's inputs (the last chunk of a
    // block loads itself again), so that waiting for the fragments leaves those in flight
    u32x4 wf[4];
    u32x2 ut[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      wf[ks] = *reinterpret_cast<const u32x4*>(pc + kWsW + ((size_t)(rb * 4 + ks) * 64 + lane) * 16);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      ut[u] = *reinterpret_cast<const u32x2*>(pc + kWsU + ((size_t)(rb * 8 + (w >> 2) * 4 + u) * 64 + lane) * 8);
    g1_fetch(in, q, k, dO, alpha, ws, cid + (int)gridDim.x < nchunks ? cid + (int)gridDim.x : cid, T);
    lds_barrier();

    // ---- A = M o (g_r/g_j) o Q K^T (lower tiles) and U = U~ - W S_b^T
    for (int t = w; t < 10; t += 8) {
      int ab, cb;
      tri_pair(t, ab, cb);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma(ld8(sm.Q + sw_off(16 * ab + l16, 32 * ks + 8 * lq)), ld8(sm.K + sw_off(16 * cb + l16, 32 * ks + 8 * lq)), acc);
      const int j = 16 * cb + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * ab + 4 * lq + i;
        sm.A[r * PA + j] = f32_to_bf16(j <= r ? __expf(sm.lg[r] - sm.lg[j]) * acc[i] : 0.f);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int vb = (w >> 2) * 4 + u;
      f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) p = mfma(as_bf(wf[ks]), ld8_split_s(sm.S, 16 * vb + l16, 32 * ks + 4 * lq), p);
      const float uu[4] = {lo_bf(ut[u].x) - p[0], hi_bf(ut[u].x) - p[1], lo_bf(ut[u].y) - p[2], hi_bf(ut[u].y) - p[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.U[sw_off(16 * rb + 4 * lq + i, 16 * vb + l16)] = f32_to_bf16(uu[i]);
    }
    lds_barrier();

    // ---- dU = A^T dO + diag(g_C/g) K dS_a^T (to the workspace); dO U^T on the lower tiles
    uint16_t* dUw = ws.dU + (size_t)cid * C * kD;
#pragma unroll 1
    for (int u = 0; u < 4; ++u) {
      const int vb = (w >> 2) * 4 + u;
      f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = a1;
#pragma unroll
      for (int js = 0; js < 2; ++js)
        if (32 * js + 31 >= 16 * rb)   // A[j][r] is zero for j < r
          a1 = mfma(ld_tr8(sm.A, PA, 32 * js, 16 * rb), ld_tr8s(sm.O, 32 * js, 16 * vb), a1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        a2 = mfma(ld8(sm.K + sw_off(16 * rb + l16, 32 * ks + 8 * lq)), ld8(sm.D + sw_off(16 * vb + l16, 32 * ks + 8 * lq)), a2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rb + 4 * lq + i;
        dUw[r * kD + 16 * vb + l16] = f32_to_bf16(a1[i] + sm.kd[r] * a2[i]);
      }
    }
    f32x4 da[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      da[h] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (w + 8 * h < 10) {
        int ab, cb;
        tri_pair(w + 8 * h, ab, cb);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          da[h] = mfma(ld8(sm.O + sw_off(16 * ab + l16, 32 * ks + 8 * lq)), ld8(sm.U + sw_off(16 * cb + l16, 32 * ks + 8 * lq)), da[h]);
      }
    }
    lds_barrier();
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (w + 8 * h < 10) {
        int ab, cb;
        tri_pair(w + 8 * h, ab, cb);
        const int j = 16 * cb + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * ab + 4 * lq + i;
          sm.A[r * PA + j] = f32_to_bf16(j <= r ? __expf(sm.lg[r] - sm.lg[j]) * da[h][i] : 0.f);
        }
      }
    lds_barrier();

    // ---- dq = dA' K + diag(g) dO S_b;  dK1 = dA'^T Q + diag(g_C/g) U dS_a
    u32x2* dK1 = ws.dK1 + (size_t)cid * (C * kD / 4);
    float qacc[4] = {0.f, 0.f, 0.f, 0.f};   // this lane's share of q.dq over its 4 key blocks
    float bs2 = 0.f;                         // this lane's part of sum(diag(g_C/g) U dS_a o K)
#pragma unroll 1
    for (int u = 0; u < 4; ++u) {
      const int kb = (w >> 2) * 4 + u;
      f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = a1, a3 = a1, a4 = a1;
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        if (js <= rb / 2)   // dA'[r][j] is zero for j > r
          a1 = mfma(ld8(sm.A + (16 * rb + l16) * PA + 32 * js + 8 * lq), ld_tr8s(sm.K, 32 * js, 16 * kb), a1);
        if (32 * js + 31 >= 16 * rb)   // dA'[i][r] is zero for i < r
          a3 = mfma(ld_tr8(sm.A, PA, 32 * js, 16 * rb), ld_tr8s(sm.Q, 32 * js, 16 * kb), a3);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        a2 = mfma(ld8(sm.O + sw_off(16 * rb + l16, 32 * ks + 8 * lq)), ld_tr8s(sm.S, 32 * ks, 16 * kb), a2);
        a4 = mfma(ld8(sm.U + sw_off(16 * rb + l16, 32 * ks + 8 * lq)), ld_tr8s(sm.D, 32 * ks, 16 * kb), a4);
      }
      const int col = 16 * kb + l16;
      float k1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rb + 4 * lq + i;
        const float gq = a1[i] + sm.g[r] * a2[i];
        dq[(tok0 + r) * kD + col] = f32_to_bf16(gq);
        const float ud = sm.kd[r] * a4[i];
        k1[i] = a3[i] + ud;
        qacc[i] += bf16_to_f32(sm.Q[sw_off(r, col)]) * gq;
        bs2 += ud * bf16_to_f32(sm.K[sw_off(r, col)]);
      }
      dK1[(w * 4 + u) * 64 + lane] = u32x2{pack_bf16(k1[0], k1[1]), pack_bf16(k1[2], k1[3])};
    }
    // fixed summation order (no atomics): the 16 lanes of a row, then each half of the
    // waves writes its own partial
#pragma unroll
    for (int i = 0; i < 4; ++i) qacc[i] = sum16(qacc[i]);
    if (l16 == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.qdq[w >> 2][16 * rb + 4 * lq + i] = qacc[i];
    bs1 = sum64(bs1);
    bs2 = sum64(bs2);
    if (lane == 0) {
      sm.bs[w][0] = bs1;
      sm.bs[w][1] = bs2;
    }
    lds_barrier();
    if (tid < C) ws.qdq[(size_t)cid * C + tid] = sm.qdq[0][tid] + sm.qdq[1][tid];
    // sum(dS_a o S_a) with S_a = g_C S_b + U^T K^ = g_C S_b + U^T diag(g_C/g) K
    if (tid == 0) {
      float b1 = 0.f, b2 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        b1 += sm.bs[i][0];
        b2 += sm.bs[i][1];
      }
      ws.bnd[cid] = sm.g[C - 1] * b1 + b2;
    }
  };
  chunk(blockIdx.x);
#pragma unroll 1
  for (int cid = blockIdx.x + gridDim.x; cid < nchunks; cid += gridDim.x) chunk(cid);
}

// ------------------------------------------------------------------ gradients, part 2
// Persistent blocks of 512 threads, one per CU (LDS), chunks strided by the grid. Per
// chunk: dW = -dU S_b, the WY gradients T^T dW and T^T dU, dv, dL, dk (with dK1), dbeta,
// and dalpha from dL/dB_t = q_t.dq_t - v_t.dv_t summed in reverse inside the chunk plus
// the chunk's sum(dS_a o S_a). The next chunk's k, v, dU, S_b, U~, T, alpha and beta are
// loaded into registers from the dL step on, after this chunk's own W fragments and dK1,
// so that no wait inside the chunk also waits for them.
struct alignas(16) G2Smem {
  uint16_t K[kChunk * gdb::PT], V[kChunk * gdb::PT], dU[kChunk * gdb::PT], dW[kChunk * gdb::PT];
  uint16_t Ut[kChunk * gdb::PT];   // U~ [t][v]
  uint16_t S[kD * gdb::PT];        // S_b [v][c], then T^T dW [t][c] and T^T dU [t][v]
  uint16_t T[kChunk * gdb::PA];    // (I + L)^-1 [r][j]
  uint16_t L[kChunk * gdb::PA];    // dL o (g_r/g_j) o beta_r and its transpose [r][j]
  float lg[kChunk], g[kChunk], bt[kChunk];
  // partial sums in a fixed order (no atomics): dbW, dbU per wave half, dbL per
  // column block of the strict lower part
  float dbW[2][kChunk], dbU[2][kChunk], dbL[4][kChunk];
};

namespace gdb {
// one chunk's inputs of a grad2 thread: 16-byte pieces tid + 512 p of k, v, dU and of
// S_b; the U~ fragments f = wave + 8 p (lane's 8 bytes); 16 bytes of T; alpha, beta of
// token lane
struct G2In {
  u32x4 k[2], v[2], du[2], s[4], t;
  u32x2 ut[4];
  float al, be;
};
__device__ __forceinline__ void g2_fetch(G2In& in, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                         const float* __restrict__ alpha, const float* __restrict__ beta,
                                         const Ws& ws, int cid, int T) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nc = T / C;
  const size_t tok0 = (size_t)(cid / nc) * T + (size_t)(cid % nc) * C;
  const uint8_t* pc = ws.prep + (size_t)cid * kWsChunk;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const size_t gi = tok0 * kD + (size_t)(tid + 512 * p) * 8;
    in.k[p] = *reinterpret_cast<const u32x4*>(k + gi);
    in.v[p] = *reinterpret_cast<const u32x4*>(v + gi);
    in.du[p] = *reinterpret_cast<const u32x4*>(ws.dU + (size_t)cid * C * kD + (size_t)(tid + 512 * p) * 8);
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    in.s[p] = *reinterpret_cast<const u32x4*>(ws.Sb + (size_t)cid * kD * kD + (size_t)(tid + 512 * p) * 8);
    in.ut[p] = *reinterpret_cast<const u32x2*>(pc + kWsU + ((size_t)(w + 8 * p) * 64 + lane) * 8);
  }
  in.t = *reinterpret_cast<const u32x4*>(ws.T + (size_t)cid * C * C + tid * 8);
  in.al = alpha[tok0 + lane];
  in.be = beta[tok0 + lane];
}
}  // namespace gdb

__global__ __launch_bounds__(512) void gdn_bwd_grad2_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, gdb::Ws ws, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    float* __restrict__ dbeta, float* __restrict__ dalpha, int T, int nchunks) {
  using namespace gdb;
  __shared__ G2Smem sm;
  const int nc = T / C;
  uint16_t* XW = sm.S;             // T^T dW, after dW is formed
  uint16_t* XU = sm.S + C * PT;    // T^T dU
  G2In in;
  g2_fetch(in, k, v, alpha, beta, ws, blockIdx.x, T);   // the grid never exceeds nchunks
  // the first chunk is peeled, so that the loop is entered with the same memory
  // operations in flight on both paths (the next chunk's loads, then this chunk's
  // stores) and the waits for the prefetched inputs never include the stores
  auto chunk = [&](const int cid) {
    // the thread index through an opaque move (per-lane addresses formed per chunk)
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    const int lane = tid & 63, w = tid >> 6, l16 = lane & 15, lq = lane >> 4, rb = w & 3;
    const size_t tok0 = (size_t)(cid / nc) * T + (size_t)(cid % nc) * C;
    const uint8_t* pc = ws.prep + (size_t)cid * kWsChunk;

#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int e = (tid + 512 * p) * 8, r = e >> 7, cc = e & 127;
      *reinterpret_cast<u32x4*>(sm.K + sw_off(r, cc)) = in.k[p];
      *reinterpret_cast<u32x4*>(sm.V + sw_off(r, cc)) = in.v[p];
      *reinterpret_cast<u32x4*>(sm.dU + sw_off(r, cc)) = in.du[p];
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int e = (tid + 512 * p) * 8, r = e >> 7, cc = e & 127;
      *reinterpret_cast<u32x4*>(sm.S + sw_off(r, cc)) = in.s[p];
      // U~ tile f = w + 8 p (rb, vb) = (f / 8, f % 8): tokens rb*16 + lq*4 + i of value vb*16 + l16
      const int f = w + 8 * p, ub = f >> 3, vb = f & 7;
      const float uv[4] = {lo_bf(in.ut[p].x), hi_bf(in.ut[p].x), lo_bf(in.ut[p].y), hi_bf(in.ut[p].y)};
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.Ut[sw_off(16 * ub + 4 * lq + i, 16 * vb + l16)] = f32_to_bf16(uv[i]);
    }
    {
      const int e = tid * 8, r = e >> 6, cc = e & 63;
      *reinterpret_cast<u32x4*>(sm.T + r * PA + cc) = in.t;
    }
    for (int e = tid; e < C * PA / 2; e += 512) reinterpret_cast<uint32_t*>(sm.L)[e] = 0u;
    if (w == 0) {
      const float lgv = wave_scan(__logf(in.al));
      sm.lg[lane] = lgv;
      sm.g[lane] = __expf(lgv);
      sm.bt[lane] = in.be;
#pragma unroll
      for (int c = 0; c < 4; ++c) sm.dbL[c][lane] = 0.f;
    }
    lds_barrier();

    // ---- dW = -dU S_b
#pragma unroll 1
    for (int u = 0; u < 4; ++u) {
      const int kb = (w >> 2) * 4 + u;
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        a = mfma(ld8(sm.dU + sw_off(16 * rb + l16, 32 * ks + 8 * lq)), ld_tr8s(sm.S, 32 * ks, 16 * kb), a);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.dW[sw_off(16 * rb + 4 * lq + i, 16 * kb + l16)] = f32_to_bf16(-a[i]);
    }
    lds_barrier();

    // ---- T^T dW and T^T dU; dv = beta o T^T dU; dK_W = beta g o T^T dW (kept)
    f32x4 kw[4];
    float su_acc[4] = {0.f, 0.f, 0.f, 0.f}, sw_acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cb = (w >> 2) * 4 + u;
      f32x4 xw = {0.f, 0.f, 0.f, 0.f}, xu = xw;
#pragma unroll
      for (int js = 0; js < 2; ++js)
        if (32 * js + 31 >= 16 * rb) {   // T[j][r] is zero for j < r
          const bf16x8 tt = ld_tr8(sm.T, PA, 32 * js, 16 * rb);
          xw = mfma(tt, ld_tr8s(sm.dW, 32 * js, 16 * cb), xw);
          xu = mfma(tt, ld_tr8s(sm.dU, 32 * js, 16 * cb), xu);
        }
      const int col = 16 * cb + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rb + 4 * lq + i;
        XW[sw_off(r, col)] = f32_to_bf16(xw[i]);
        XU[sw_off(r, col)] = f32_to_bf16(xu[i]);
        dv[(tok0 + r) * kD + col] = f32_to_bf16(sm.bt[r] * xu[i]);
        kw[u][i] = sm.bt[r] * sm.g[r] * xw[i];
        su_acc[i] += xu[i] * bf16_to_f32(sm.V[sw_off(r, col)]);
        sw_acc[i] += xw[i] * bf16_to_f32(sm.K[sw_off(r, col)]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // the lane's 4 column blocks, then the 16 lanes of a row
      su_acc[i] = sum16(su_acc[i]);
      sw_acc[i] = sum16(sw_acc[i]);
    }
    if (l16 == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sm.dbU[w >> 2][16 * rb + 4 * lq + i] = su_acc[i];
        sm.dbW[w >> 2][16 * rb + 4 * lq + i] = sw_acc[i];
      }
    // this chunk's W fragments (the wave's one or two lower tiles of dL) and dK1, then the
    // next chunk's inputs (the last chunk of a block loads itself again)
    u32x4 wfr[2][4];
    float k1[4][4];
    const u32x2* dK1 = ws.dK1 + (size_t)cid * (C * kD / 4);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int ab, cb;
      tri_pair(w + 8 * h < 10 ? w + 8 * h : w, ab, cb);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        wfr[h][ks] = *reinterpret_cast<const u32x4*>(pc + kWsW + ((size_t)(cb * 4 + ks) * 64 + lane) * 16);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x2 pk = dK1[(w * 4 + u) * 64 + lane];   // rows 16 rb + 4 lq + i of column block 4 (w / 4) + u
      k1[u][0] = lo_bf(pk.x);
      k1[u][1] = hi_bf(pk.x);
      k1[u][2] = lo_bf(pk.y);
      k1[u][3] = hi_bf(pk.y);
    }
    g2_fetch(in, k, v, alpha, beta, ws, cid + (int)gridDim.x < nchunks ? cid + (int)gridDim.x : cid, T);
    lds_barrier();

    // ---- dL = -(T^T dW W^T + T^T dU U~^T) on the strict lower part; with the Gram
    // matrix K K^T for dbeta; dL o (g_r/g_j) o beta_r and its transpose to LDS
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (w + 8 * h >= 10) continue;
      int ab, cb;
      tri_pair(w + 8 * h, ab, cb);
      f32x4 a = {0.f, 0.f, 0.f, 0.f}, gk = a;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        a = mfma(ld8_split_s(XW, 16 * ab + l16, 32 * ks + 4 * lq), as_bf(wfr[h][ks]), a);
        a = mfma(ld8(XU + sw_off(16 * ab + l16, 32 * ks + 8 * lq)), ld8(sm.Ut + sw_off(16 * cb + l16, 32 * ks + 8 * lq)), a);
        gk = mfma(ld8(sm.K + sw_off(16 * ab + l16, 32 * ks + 8 * lq)), ld8(sm.K + sw_off(16 * cb + l16, 32 * ks + 8 * lq)), gk);
      }
      const int j = 16 * cb + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * ab + 4 * lq + i;
        float x = 0.f, y = 0.f;
        if (j < r) {
          const float dl = -a[i] * __expf(sm.lg[r] - sm.lg[j]);
          x = dl * sm.bt[r];
          y = dl * gk[i];
          const uint16_t xb = f32_to_bf16(x);
          sm.L[r * PA + j] = xb;
          sm.L[j * PA + r] = xb;
        }
        const float sy = sum16(y);
        if (l16 == 0) sm.dbL[cb][r] = sy;   // one pair (ab, cb) per row block and column block
      }
    }
    lds_barrier();

    // ---- dk = dK1 + dK_W + (dL' + dL'^T) K
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kb = (w >> 2) * 4 + u;
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int js = 0; js < 2; ++js)
        a = mfma(ld8(sm.L + (16 * rb + l16) * PA + 32 * js + 8 * lq), ld_tr8s(sm.K, 32 * js, 16 * kb), a);
      const int col = 16 * kb + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rb + 4 * lq + i;
        dk[(tok0 + r) * kD + col] = f32_to_bf16(k1[u][i] + kw[u][i] + a[i]);
      }
    }
    lds_barrier();
    if (w == 0) {
      const int t = lane;
      const float dbU = sm.dbU[0][t] + sm.dbU[1][t], dbW = sm.dbW[0][t] + sm.dbW[1][t];
      const float dbL = (sm.dbL[0][t] + sm.dbL[1][t]) + (sm.dbL[2][t] + sm.dbL[3][t]);
      dbeta[tok0 + t] = sm.g[t] * dbW + dbU + dbL;
      const float dB = ws.qdq[(size_t)cid * C + t] - sm.bt[t] * dbU;
      const float off = ws.bnd[cid];
      // reverse inclusive sum inside the chunk: lane l scans token 63 - l
      const float rs = wave_scan(__shfl(dB, C - 1 - lane));
      dalpha[tok0 + t] = (__shfl(rs, C - 1 - t) + off) / alpha[tok0 + t];
    }
  };
  chunk(blockIdx.x);
#pragma unroll 1
  for (int cid = blockIdx.x + gridDim.x; cid < nchunks; cid += gridDim.x) chunk(cid);
}

}  // namespace gdnrt

using namespace gdnrt;

namespace {

struct BwdLayout {
  size_t prep, T, Sb, dSa, dU, dK1, qdq, bnd, total;
};

BwdLayout bwd_layout(size_t N, size_t nchunks) {
  BwdLayout L;
  L.prep = 0;
  L.T = L.prep + nchunks * gdc::kWsChunk;
  L.Sb = L.T + nchunks * kChunk * kChunk * 2;
  L.dSa = L.Sb + nchunks * kD * kD * 2;
  L.dU = L.dSa + nchunks * kD * kD * 2;
  L.dK1 = L.dU + nchunks * kChunk * kD * 2;
  L.qdq = L.dK1 + nchunks * kChunk * kD * 2;
  L.bnd = L.qdq + nchunks * kChunk * 4;
  L.total = L.bnd + nchunks * 4;
  return L;
}

}  // namespace

extern "C" size_t gdn_chunk_bwd_workspace_bytes(int N, int T, int dk, int dv, int chunk) {
  if (N <= 0 || T <= 0 || dk != kD || dv != kD || chunk != kChunk || T % kChunk) return 0;
  return bwd_layout((size_t)N, (size_t)N * (T / kChunk)).total;
}

extern "C" int gdn_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* S0, const void* dO, const float* dST,
                             void* dq, void* dk, void* dv, float* dalpha, float* dbeta, float* dS0, int N,
                             int T, int dk_, int dv_, int chunk, int io, void* workspace, size_t ws_bytes,
                             void* stream) {
  const char* fn = "gdn_chunk_bwd";
  if (N < 0 || T < 0) return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d must be >= 0", fn, N, T);
  if (dk_ != kD || dv_ != kD) return set_error(GDNRT_ESHAPE, "%s: d_k=%d d_v=%d, only 128 is supported", fn, dk_, dv_);
  if (chunk != kChunk) return set_error(GDNRT_ESHAPE, "%s: chunk=%d, only 64 is supported", fn, chunk);
  if (T % kChunk) return set_error(GDNRT_ESHAPE, "%s: T=%d is not a multiple of 64", fn, T);
  if (io != GDNRT_BF16) return set_error(GDNRT_EDTYPE, "%s: io must be GDNRT_BF16", fn);
  if ((size_t)N * (T / kChunk) > 0x7fffffffu || (size_t)N * 16 > 0x7fffffffu)
    return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d too large", fn, N, T);
  if (N == 0) return clear_error();
  if (!dS0 || (T > 0 && (!q || !k || !v || !alpha || !beta || !dO || !dq || !dk || !dv || !dalpha || !dbeta)))
    return set_error(GDNRT_EINVAL, "%s: null pointer argument", fn);
  const size_t nchunks = (size_t)N * (T / kChunk);
  const BwdLayout lay = bwd_layout((size_t)N, nchunks);
  const size_t need = T > 0 ? lay.total : 0;
  if (ws_bytes < need || (need && !workspace))
    return set_error(GDNRT_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need, ws_bytes);
  if ((T > 0 && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(workspace) ||
                 !aligned4(alpha) || !aligned4(beta) || !aligned4(dq) || !aligned4(dk) || !aligned4(dv) ||
                 !aligned4(dalpha) || !aligned4(dbeta))) ||
      !aligned4(dS0) || (S0 && !aligned4(S0)) || (dST && !aligned4(dST)))
    return set_error(GDNRT_EALIGN, "%s: q, k, v, dO, workspace must be 16-byte aligned", fn);
  const size_t ntok = (size_t)N * T, nIO = ntok * kD * 2, nG = ntok * 4, nS = (size_t)N * kD * kD * 4;
  struct Buf {
    const void* p;
    size_t n;
  };
  const Buf ins[] = {{q, nIO}, {k, nIO}, {v, nIO}, {dO, nIO}, {alpha, nG}, {beta, nG}, {S0, nS}, {dST, nS}};
  const Buf outs[] = {{dq, nIO}, {dk, nIO}, {dv, nIO}, {dalpha, nG}, {dbeta, nG}, {dS0, nS}, {workspace, need}};
  for (const Buf& a : outs) {
    for (const Buf& b : ins)
      if (overlaps(a.p, a.n, b.p, b.n)) return set_error(GDNRT_EINVAL, "%s: an output overlaps an input", fn);
    for (const Buf& b : outs)
      if (a.p != b.p && overlaps(a.p, a.n, b.p, b.n)) return set_error(GDNRT_EINVAL, "%s: outputs overlap", fn);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {   // no tokens: the state gradient passes through
    hipLaunchKernelGGL(gdn_bwd_pass_kernel, dim3((unsigned)(N * 8)), dim3(256), 0, s, dST, dS0);
    return check_launch(fn);
  }
  uint8_t* base = static_cast<uint8_t*>(workspace);
  gdb::Ws ws;
  ws.prep = base + lay.prep;
  ws.T = reinterpret_cast<uint16_t*>(base + lay.T);
  ws.Sb = reinterpret_cast<uint16_t*>(base + lay.Sb);
  ws.dSa = reinterpret_cast<uint16_t*>(base + lay.dSa);
  ws.dU = reinterpret_cast<uint16_t*>(base + lay.dU);
  ws.dK1 = reinterpret_cast<gdc::u32x2*>(base + lay.dK1);
  ws.qdq = reinterpret_cast<float*>(base + lay.qdq);
  ws.bnd = reinterpret_cast<float*>(base + lay.bnd);
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  const uint16_t* o16 = static_cast<const uint16_t*>(dO);
  gdn_chunk_prep_with_inverse(q16, k16, v16, alpha, beta, ws.prep, ws.T, T, (int)nchunks, s);
  int rc = check_launch(fn);
  if (rc != GDNRT_OK) return rc;
  hipLaunchKernelGGL(gdn_bwd_scans_kernel, dim3((unsigned)(N * 16)), dim3(256), 0, s, ws.prep, S0, ws.Sb, o16,
                     dST, ws.dSa, dS0, T);
  // persistent gradient blocks, one per CU (their LDS fills one)
  const unsigned ggrid = (unsigned)(nchunks < 256 ? nchunks : 256);
  hipLaunchKernelGGL(gdn_bwd_grad1_kernel, dim3(ggrid), dim3(512), 0, s, q16, k16, o16, alpha, ws,
                     static_cast<uint16_t*>(dq), T, (int)nchunks);
  hipLaunchKernelGGL(gdn_bwd_grad2_kernel, dim3(ggrid), dim3(512), 0, s, k16, v16, alpha, beta, ws,
                     static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), dbeta, dalpha, T, (int)nchunks);
  return check_launch(fn);
}

// LeapQuant windowed 8-bit Gated DeltaNet state: decode step and window flush.
//
// Method: "LeapQuant: an 8-bit recurrent state that stops rounding every token".
//  * section "Fix one: leap over a window", eq. 4 and eq. 10: inside a window the
//    state is the decayed stored state plus the decayed rank-one writes of the
//    buffered tokens, and S x is evaluated without forming S;
//  * section "Fix two: pull the outliers out as tokens", eq. 5: r compensator
//    tokens (fp16 rank-one pieces) subtracted before rounding, entering the next
//    window ahead of the real tokens with decay 1;
//  * section "Fix three: smooth what is left", eq. 7: one smoothing factor per key
//    channel, folded into the read vector;
//  * the quantiser: symmetric INT8, one scale per value channel (its largest
//    magnitude maps to 127).
// Layout [d_v][d_k] (rows = value channels); see include/gdnrt.h for the buffers.
#include "common.hpp"

namespace gdnrt {

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f2h(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

// sign-extend byte b of w to float
__device__ __forceinline__ float sb(uint32_t w, int b) { return (float)((int32_t)(w << (24 - 8 * b)) >> 24); }

// ============================================================== decode step
//
// Per head, with m = pos buffered records (k_j, u_j, a_j) and compensator pairs
// (kc_r, uc_r), the state after the m records applied to a vector x is
//   S_m x = G0 [ vscale * (Z (ksmooth o x)) / 127 + sum_r uc_r (kc_r . x) ]
//         + sum_j G_j u_j (k_j . x),   G0 = prod_{i<m} a_i,  G_j = prod_{j<i<m} a_i.
// The token then gives u = b (v - a S_m k), o = a S_m q + u (k . q), and its record
// is appended at slot m.
//
// The value rows of a head are independent given the per-head dot products, so a
// head is split over blocks of 128 threads, each taking 32 RPT rows (the blocks of
// one head on one XCD, so that the vectors they all read come from one L2). Thread
// (rq = tid / 4, quarter qt = tid % 4) owns 32 codes of each of its RPT rows
// part * 32 RPT + 32 i + rq, and their buffered and compensator values of slots
// = qt (mod 4). Each block forms the per-head dot products of q and k with the
// compensator keys, the buffered keys and k itself (16-lane groups, 8 entries per
// lane). Every global load that depends on no other is issued before the first
// barrier; more rows per thread keep more bytes in flight per block.

constexpr int kDecodeRPT = 2;   // value rows per thread of a decode block

template <typename IO, int RPT>
__global__ __launch_bounds__(128) void leapq_decode_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ vscale,
    const float* __restrict__ ksmooth, const uint16_t* __restrict__ ct_k,
    const uint16_t* __restrict__ ct_u, float* __restrict__ buf_k, float* __restrict__ buf_u,
    float* __restrict__ buf_a, int rank, int window, int m,
    const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, IO* __restrict__ o, int N) {
  constexpr int NT = 128;                                      // threads
  constexpr int RPB = 32 * RPT;                                // rows per block
  constexpr int PPH = kD / RPB;                                // blocks per head
  constexpr int NG = NT / 16;                                  // 16-lane groups
  constexpr int NP = (kMaxRank + kMaxWindow + NG - 1) / NG;    // dot vectors per group
  __shared__ f32x4 s_x4[2][kD / 4];            // ksmooth o k, ksmooth o q
  __shared__ float s_k[kD], s_q[kD];
  __shared__ float s_dk[kMaxRank + kMaxWindow], s_dq[kMaxRank + kMaxWindow];
  __shared__ float s_g[kMaxWindow + 1];        // s_g[j] = G_j for j < m, s_g[m] = G0

  const int tid = threadIdx.x;
  int head, part;
  {
    const int bid = blockIdx.x;
    if ((N & 7) == 0) {
      const int xcd = bid & 7, slot = bid >> 3;
      head = (slot / PPH) * 8 + xcd;
      part = slot % PPH;
    } else {
      head = bid / PPH;
      part = bid % PPH;
    }
  }
  const int rq = tid >> 2, qt = tid & 3;
  const size_t hk = (size_t)head * kD;
  float* bk = buf_k + (size_t)head * window * kD;
  float* bu = buf_u + (size_t)head * window * kD;
  const float* ba = buf_a + (size_t)head * window;
  const int nv = rank + m + 1;   // dot-product vectors: compensators, buffered keys, k

  // ---- independent loads
  uint4 z[RPT][2];
  float bur[RPT][kMaxWindow / 4], cur[RPT][kMaxRank / 4], vrow[RPT], vs[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = part * RPB + 32 * i + rq;
    const uint4* zp = reinterpret_cast<const uint4*>(codes + (hk + row) * kD + qt * 32);
    z[i][0] = zp[0];
    z[i][1] = zp[1];
#pragma unroll
    for (int jj = 0; jj < kMaxWindow / 4; ++jj) {
      const int j = 4 * jj + qt;
      bur[i][jj] = j < m ? bu[(size_t)j * kD + row] : 0.f;
    }
#pragma unroll
    for (int rr = 0; rr < kMaxRank / 4; ++rr) {
      const int r = 4 * rr + qt;
      cur[i][rr] = r < rank ? h2f(ct_u[((size_t)head * rank + r) * kD + row]) : 0.f;
    }
    vrow[i] = io_traits<IO>::ld(v, hk + row);
    vs[i] = vscale[hk + row];
  }
  const float a = alpha[head];
  const float b = beta[head];
  const int grp = tid >> 4, l16 = tid & 15, c0 = l16 * 8;
  float w[NP][8];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int vi = grp + NG * p;
    if (vi < rank) {
      const uint4 raw = *reinterpret_cast<const uint4*>(ct_k + ((size_t)head * rank + vi) * kD + c0);
      const uint32_t r4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[p][2 * e] = h2f(uint16_t(r4[e] & 0xffffu));
        w[p][2 * e + 1] = h2f(uint16_t(r4[e] >> 16));
      }
    } else if (vi < rank + m) {
      const f32x4* pp = reinterpret_cast<const f32x4*>(bk + (size_t)(vi - rank) * kD + c0);
      const f32x4 x0 = pp[0], x1 = pp[1];
      w[p][0] = x0.x; w[p][1] = x0.y; w[p][2] = x0.z; w[p][3] = x0.w;
      w[p][4] = x1.x; w[p][5] = x1.y; w[p][6] = x1.z; w[p][7] = x1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) w[p][e] = 0.f;
    }
  }
  {   // one thread per key channel
    const float kv = io_traits<IO>::ld(k, hk + tid);
    const float qv = io_traits<IO>::ld(q, hk + tid);
    const float c = ksmooth[hk + tid];
    s_k[tid] = kv;
    s_q[tid] = qv;
    reinterpret_cast<float*>(s_x4[0])[tid] = c * kv;
    reinterpret_cast<float*>(s_x4[1])[tid] = c * qv;
    if (part == 0) bk[(size_t)m * kD + tid] = kv;   // append this token's key
  }
  if (tid == 0) {
    float g = 1.f;
    for (int j = m - 1; j >= 0; --j) {      // suffix products of the buffered decays
      s_g[j] = g;
      g *= ba[j];
    }
    s_g[m] = g;
    if (part == 0) buf_a[(size_t)head * window + m] = a;
  }
  lds_barrier();

  // ---- per-head dot products
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int vi = grp + NG * p;
    if (vi < nv) {
      float pk = 0.f, pq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float we = vi == rank + m ? s_k[c0 + e] : w[p][e];
        pk += we * s_k[c0 + e];
        pq += we * s_q[c0 + e];
      }
      pk = sum16(pk);
      pq = sum16(pq);
      if (l16 == 0) {
        s_dk[vi] = pk;
        s_dq[vi] = pq;
      }
    }
  }
  lds_barrier();

  // ---- the rows: each quarter's share, then the four quarters summed
  const float g0 = s_g[m];
  const float kq = s_dq[rank + m];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const uint32_t zz[8] = {z[i][0].x, z[i][0].y, z[i][0].z, z[i][0].w,
                            z[i][1].x, z[i][1].y, z[i][1].z, z[i][1].w};
    float yk = 0.f, yq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const f32x4 xk = s_x4[0][qt * 8 + e];
      const f32x4 xq = s_x4[1][qt * 8 + e];
      const float z_0 = sb(zz[e], 0), z_1 = sb(zz[e], 1), z_2 = sb(zz[e], 2), z_3 = sb(zz[e], 3);
      yk += z_0 * xk.x + z_1 * xk.y + z_2 * xk.z + z_3 * xk.w;
      yq += z_0 * xq.x + z_1 * xq.y + z_2 * xq.z + z_3 * xq.w;
    }
    float ck = 0.f, cq = 0.f, tk = 0.f, tq = 0.f;
#pragma unroll
    for (int rr = 0; rr < kMaxRank / 4; ++rr) {
      const int r = 4 * rr + qt;
      if (r < rank) {
        ck += cur[i][rr] * s_dk[r];
        cq += cur[i][rr] * s_dq[r];
      }
    }
#pragma unroll
    for (int jj = 0; jj < kMaxWindow / 4; ++jj) {
      const int j = 4 * jj + qt;
      if (j < m) {
        const float wj = s_g[j] * bur[i][jj];
        tk += wj * s_dk[rank + j];
        tq += wj * s_dq[rank + j];
      }
    }
    const float sv = vs[i] * (1.0f / 127.0f);
    float Sk = g0 * (sv * yk + ck) + tk;   // this quarter's share; linear in the parts
    float Sq = g0 * (sv * yq + cq) + tq;
    Sk += dpp<0xB1>(Sk);                   // quarters 0+1, 2+3
    Sq += dpp<0xB1>(Sq);
    Sk += dpp<0x4E>(Sk);                   // all four
    Sq += dpp<0x4E>(Sq);
    const float u = b * (vrow[i] - a * Sk);
    const float oi = a * Sq + u * kq;
    if (qt == 0) {
      const int row = part * RPB + 32 * i + rq;
      bu[(size_t)m * kD + row] = u;
      io_traits<IO>::st(o, hk + row, oi);
    }
  }
}

// ============================================================== window flush
//
// One block of 128*NQ threads per head. Thread t owns value row v = t % 128 and
// key columns [c0, c0 + 128/NQ), c0 = (t / 128) * 128/NQ, of the dense state in
// registers; a copy in LDS ([128][129] fp32, conflict-free by rows and columns)
// serves the column operations. Steps: rebuild (eq. 4) or load `dense`;
// compensator fit by subspace iteration with CholeskyQR2; subtract the
// fp16-rounded pieces; smoothing factors; value-channel scales; codes.
// Per-head vectors in LDS are [r][128] (rank-major), so lane-indexed accesses are
// consecutive and column-indexed ones are broadcasts.

constexpr int kP = kD + 1;
constexpr int kFlushNQ = 8;   // 1024 threads per flush block, 16 key columns each

template <int NQ>
struct alignas(16) FlushSmem {
  float S[kD * kP];
  float K[(kMaxRank + kMaxWindow) * kD];   // keys of the rank-one terms: compensators, records
  float U[(kMaxRank + kMaxWindow) * kD];   // their value-side vectors
  float Qa[kMaxRank * kD];                 // [r][c]
  float Qb[kMaxRank * kD];
  float Y[kMaxRank * kD];                  // [r][v]
  float part[NQ * kMaxRank * kD];          // [p][r][x]
  double gram[2][2][kMaxRank * kMaxRank];  // [pass][wave 0, 1] partial Gram matrices
  float col[kD];
  float dec[kMaxWindow + 1];               // dec[j] = G_j for j < m, dec[m] = G0
  float red[NQ * kD];
};

// dst[r][x] = sum over the NQ partial sums, returned to threads t < 128 (row t)
template <int NQ, int RANK>
__device__ __forceinline__ void combine_parts(const FlushSmem<NQ>& sm, float (&x)[RANK]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int r = 0; r < RANK; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int p = 0; p < NQ; ++p) acc += sm.part[(p * kMaxRank + r) * kD + t];
    x[r] = acc;
  }
}

// DPP move of an fp64 value (both 32-bit halves)
template <int CTRL>
__device__ __forceinline__ double dpp64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// lane L's fp64 value, wave-uniform
__device__ __forceinline__ double lane64(double x, int L) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, L);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), L);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// sum over the 64 lanes of a wave, fp64: within rows of 16 by DPP, then the four
// row totals (wave-uniform)
__device__ __forceinline__ double wave_sum_f64(double x) {
  x += dpp64<0x140>(x);
  x += dpp64<0x141>(x);
  x += dpp64<0x4E>(x);
  x += dpp64<0xB1>(x);
  return (lane64(x, 0) + lane64(x, 16)) + (lane64(x, 32) + lane64(x, 48));
}

// Waves 0 and 1 (rows t < 128, x in registers): this wave's share of the Gram
// matrix x^T x (upper triangle) to g. The fit is ill-conditioned on states with
// outlier channels, so the Gram matrix, the Cholesky factor and the triangular
// solve are formed in fp64 (products of fp32 values are exact there).
template <int RANK>
__device__ __forceinline__ void partial_gram(const float (&x)[RANK], double* g) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < RANK; ++i)
#pragma unroll
    for (int j = i; j < RANK; ++j) {
      const double s = wave_sum_f64((double)x[i] * (double)x[j]);
      if (lane == 0) g[i * kMaxRank + j] = s;
    }
}

// One CholeskyQR step on row x (threads t < 128): x <- x L^{-T} with
// L L^T = G + (1e-6 tr G + 1e-30) I, G the sum of the two partial Gram matrices
// (read from LDS as needed). L is kept packed, row by row, and 1 / diag(L) apart.
template <int RANK>
__device__ __forceinline__ void chol_solve(float (&x)[RANK], const double* g0, const double* g1) {
  auto G = [&](int i, int j) { return g0[i * kMaxRank + j] + g1[i * kMaxRank + j]; };   // i <= j
  double tr = 0.0;
#pragma unroll
  for (int i = 0; i < RANK; ++i) tr += G(i, i);
  const double sh = 1e-6 * tr + 1e-30;
  double L[RANK * (RANK + 1) / 2], rd[RANK];   // L[i][j] at i (i + 1) / 2 + j
#pragma unroll
  for (int i = 0; i < RANK; ++i) {
#pragma unroll
    for (int j = 0; j <= i; ++j) {
      double s = G(j, i) + (i == j ? sh : 0.0);
#pragma unroll
      for (int p = 0; p < j; ++p) s -= L[i * (i + 1) / 2 + p] * L[j * (j + 1) / 2 + p];
      if (i == j) {
        const double d = sqrt(fmax(s, 0.0));
        L[i * (i + 1) / 2 + i] = d;
        rd[i] = 1.0 / d;
      } else {
        L[i * (i + 1) / 2 + j] = s * rd[j];
      }
    }
  }
  double y[RANK];
#pragma unroll
  for (int j = 0; j < RANK; ++j) {
    double s = x[j];
#pragma unroll
    for (int p = 0; p < j; ++p) s -= y[p] * L[j * (j + 1) / 2 + p];
    y[j] = s * rd[j];
  }
#pragma unroll
  for (int j = 0; j < RANK; ++j) x[j] = (float)y[j];
}

// four consecutive floats of LDS as a vector (16-byte aligned)
__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

template <int NQ, int RANK>
__global__ __launch_bounds__(128 * NQ) void leapq_flush_kernel(
    int8_t* __restrict__ codes, float* __restrict__ vscale, float* __restrict__ ksmooth,
    uint16_t* __restrict__ ct_k, uint16_t* __restrict__ ct_u, const float* __restrict__ buf_k,
    const float* __restrict__ buf_u, const float* __restrict__ buf_a, int window, int m,
    const float* __restrict__ dense, const float* __restrict__ q0, int iters, int smooth_mode,
    float* __restrict__ pre_round) {
  constexpr int NT = 128 * NQ, FC = kD / NQ;
  static_assert(FC == 16, "16 key columns per thread");
  constexpr int rank = RANK;
  __shared__ FlushSmem<NQ> sm;
  const int tid = threadIdx.x;
  const int head = blockIdx.x;
  const size_t hk = (size_t)head * kD;
  const int v = tid & (kD - 1), qd = tid >> 7, c0 = qd * FC;
  float S[FC];

  // ---------------------------------------------------------------- dense state
  if (dense) {
    const f32x4* Dp = reinterpret_cast<const f32x4*>(dense + (hk + v) * kD + c0);
#pragma unroll
    for (int i = 0; i < FC / 4; ++i) {
      const f32x4 x = Dp[i];
      S[4 * i] = x.x; S[4 * i + 1] = x.y; S[4 * i + 2] = x.z; S[4 * i + 3] = x.w;
    }
  } else {
    // every input of the rebuild is requested before the one wait: this row's codes
    // and scale, the rank-one terms (keys and value vectors) and decays to LDS
    const uint4 zw = *reinterpret_cast<const uint4*>(codes + (hk + v) * kD + c0);
    const float vsv = vscale[hk + v];
    const int nt = rank + m;
    {   // one piece of four entries of K and of U per thread (nt <= 24 rows of 32)
      const int j = tid >> 5, c = (tid & 31) * 4;
      if (j < rank) {
        const uint2 hk4 = *reinterpret_cast<const uint2*>(ct_k + ((size_t)head * rank + j) * kD + c);
        const uint2 hu4 = *reinterpret_cast<const uint2*>(ct_u + ((size_t)head * rank + j) * kD + c);
        *reinterpret_cast<f32x4*>(sm.K + j * kD + c) =
            f32x4{h2f(uint16_t(hk4.x)), h2f(uint16_t(hk4.x >> 16)), h2f(uint16_t(hk4.y)), h2f(uint16_t(hk4.y >> 16))};
        *reinterpret_cast<f32x4*>(sm.U + j * kD + c) =
            f32x4{h2f(uint16_t(hu4.x)), h2f(uint16_t(hu4.x >> 16)), h2f(uint16_t(hu4.y)), h2f(uint16_t(hu4.y >> 16))};
      } else if (j < nt) {
        const size_t off = ((size_t)head * window + (j - rank)) * kD + c;
        *reinterpret_cast<f32x4*>(sm.K + j * kD + c) = *reinterpret_cast<const f32x4*>(buf_k + off);
        *reinterpret_cast<f32x4*>(sm.U + j * kD + c) = *reinterpret_cast<const f32x4*>(buf_u + off);
      }
    }
    if (tid < kD) sm.col[tid] = ksmooth[hk + tid];
    if (tid == 0) {   // suffix products of the buffered decays, newest first
      const float* ba = buf_a + (size_t)head * window;
      float g = 1.f;
      for (int j = m - 1; j >= 0; --j) {
        sm.dec[j] = g;
        g *= ba[j];
      }
      sm.dec[m] = g;
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < FC; ++i) S[i] = 0.f;
    for (int j = 0; j < nt; ++j) {   // compensators (decay G0), then records (G_j)
      const float cj = (j < rank ? sm.dec[m] : sm.dec[j - rank]) * sm.U[j * kD + v];
      const float* Kj = sm.K + j * kD + c0;
#pragma unroll
      for (int i = 0; i < FC / 4; ++i) {
        const f32x4 kk = lds4(Kj + 4 * i);
        S[4 * i] += cj * kk.x; S[4 * i + 1] += cj * kk.y; S[4 * i + 2] += cj * kk.z; S[4 * i + 3] += cj * kk.w;
      }
    }
    const float sv = sm.dec[m] * vsv * (1.0f / 127.0f);
    const uint32_t z4[4] = {zw.x, zw.y, zw.z, zw.w};
#pragma unroll
    for (int i4 = 0; i4 < FC / 4; ++i4) {
      const f32x4 cc = lds4(sm.col + c0 + 4 * i4);
      S[4 * i4] += sv * sb(z4[i4], 0) * cc.x;
      S[4 * i4 + 1] += sv * sb(z4[i4], 1) * cc.y;
      S[4 * i4 + 2] += sv * sb(z4[i4], 2) * cc.z;
      S[4 * i4 + 3] += sv * sb(z4[i4], 3) * cc.w;
    }
  }
#pragma unroll
  for (int i = 0; i < FC; ++i) sm.S[v * kP + c0 + i] = S[i];

  // ---------------------------------------------------------------- compensators
  if constexpr (RANK > 0) {
    for (int i = tid; i < kD * rank; i += NT) sm.Qa[(i % rank) * kD + i / rank] = q0[i];
    lds_barrier();
    // the state is read back from its LDS copy below, so that its registers are free
    // during the fit
    for (int it = 0; it <= iters; ++it) {
      // Y = S Q (this thread's row segment)
      float acc[RANK];
#pragma unroll
      for (int r = 0; r < RANK; ++r) acc[r] = 0.f;
#pragma unroll
      for (int i4 = 0; i4 < FC / 4; ++i4) {
        const float* sr = sm.S + v * kP + c0 + 4 * i4;
        const float s0 = sr[0], s1 = sr[1], s2 = sr[2], s3 = sr[3];
#pragma unroll
        for (int r = 0; r < RANK; ++r) {
          const f32x4 qq = lds4(sm.Qa + r * kD + c0 + 4 * i4);
          acc[r] += s0 * qq.x + s1 * qq.y + s2 * qq.z + s3 * qq.w;
        }
      }
#pragma unroll
      for (int r = 0; r < RANK; ++r) sm.part[(qd * kMaxRank + r) * kD + v] = acc[r];
      lds_barrier();
      if (tid < kD) {
        float y[RANK];
        combine_parts<NQ, RANK>(sm, y);
#pragma unroll
        for (int r = 0; r < RANK; ++r) sm.Y[r * kD + tid] = y[r];
      }
      lds_barrier();
      if (it == iters) break;   // final Y = S Q: the compensator values
      // Q = S^T Y from the LDS copy: column c = v over rows [c0, c0 + FC)
#pragma unroll
      for (int r = 0; r < RANK; ++r) acc[r] = 0.f;
#pragma unroll
      for (int i4 = 0; i4 < FC / 4; ++i4) {
        const int vv = c0 + 4 * i4;
        const float s0 = sm.S[vv * kP + v], s1 = sm.S[(vv + 1) * kP + v];
        const float s2 = sm.S[(vv + 2) * kP + v], s3 = sm.S[(vv + 3) * kP + v];
#pragma unroll
        for (int r = 0; r < RANK; ++r) {
          const f32x4 yy = lds4(sm.Y + r * kD + vv);
          acc[r] += s0 * yy.x + s1 * yy.y + s2 * yy.z + s3 * yy.w;
        }
      }
#pragma unroll
      for (int r = 0; r < RANK; ++r) sm.part[(qd * kMaxRank + r) * kD + v] = acc[r];
      lds_barrier();
      // CholeskyQR2 on the rows of Q, carried by threads t < 128 in registers
      float x[RANK];
      if (tid < kD) {
        combine_parts<NQ, RANK>(sm, x);
        partial_gram<RANK>(x, sm.gram[0][tid >> 6]);
      }
      lds_barrier();
      if (tid < kD) {
        chol_solve<RANK>(x, sm.gram[0][0], sm.gram[0][1]);
        partial_gram<RANK>(x, sm.gram[1][tid >> 6]);
      }
      lds_barrier();
      if (tid < kD) {
        chol_solve<RANK>(x, sm.gram[1][0], sm.gram[1][1]);
#pragma unroll
        for (int r = 0; r < RANK; ++r) sm.Qa[r * kD + tid] = x[r];
      }
      lds_barrier();
    }
    // round to fp16, store, keep the rounded values for the residual
    if (tid < kD) {
#pragma unroll
      for (int r = 0; r < RANK; ++r) {
        const uint16_t hq = f2h(sm.Qa[r * kD + tid]);
        const uint16_t hy = f2h(sm.Y[r * kD + tid]);
        ct_k[((size_t)head * rank + r) * kD + tid] = hq;
        ct_u[((size_t)head * rank + r) * kD + tid] = hy;
        sm.Qb[r * kD + tid] = h2f(hq);
        sm.part[r * kD + tid] = h2f(hy);
      }
    }
    lds_barrier();
    // residual R = S - sum_r uh_r kh_r^T
#pragma unroll
    for (int i = 0; i < FC; ++i) S[i] = sm.S[v * kP + c0 + i];
    float yh[RANK];
#pragma unroll
    for (int r = 0; r < RANK; ++r) yh[r] = sm.part[r * kD + v];
#pragma unroll
    for (int r = 0; r < RANK; ++r)
#pragma unroll
      for (int i4 = 0; i4 < FC / 4; ++i4) {
        const f32x4 kh = lds4(sm.Qb + r * kD + c0 + 4 * i4);
        S[4 * i4] -= yh[r] * kh.x; S[4 * i4 + 1] -= yh[r] * kh.y;
        S[4 * i4 + 2] -= yh[r] * kh.z; S[4 * i4 + 3] -= yh[r] * kh.w;
      }
#pragma unroll
    for (int i = 0; i < FC; ++i) sm.S[v * kP + c0 + i] = S[i];
  }
  lds_barrier();

  // ---------------------------------------------------------------- smoothing
  {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < FC; ++i) {
      const float x = sm.S[(c0 + i) * kP + v];   // column v, rows [c0, c0 + FC)
      acc += smooth_mode == 1 ? x * x : fabsf(x);
    }
    sm.red[qd * kD + v] = acc;
    lds_barrier();
    if (tid < kD) {
      float tot = 0.f;
#pragma unroll
      for (int p = 0; p < NQ; ++p) tot += sm.red[p * kD + tid];
      const float cf = smooth_mode == 2 ? 1.f : fmaxf(sqrtf(tot * (1.0f / kD)), 1e-12f);
      ksmooth[hk + tid] = cf;
      sm.col[tid] = 1.0f / cf;
    }
    lds_barrier();
  }

  // ---------------------------------------------------------------- scales, codes
  {
    float mx = 0.f;
#pragma unroll
    for (int i4 = 0; i4 < FC / 4; ++i4) {
      const f32x4 cc = lds4(sm.col + c0 + 4 * i4);
      S[4 * i4] *= cc.x; S[4 * i4 + 1] *= cc.y; S[4 * i4 + 2] *= cc.z; S[4 * i4 + 3] *= cc.w;
    }
#pragma unroll
    for (int i = 0; i < FC; ++i) mx = fmaxf(mx, fabsf(S[i]));
    sm.red[qd * kD + v] = mx;
    lds_barrier();
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < NQ; ++p) s = fmaxf(s, sm.red[p * kD + v]);
    if (qd == 0) vscale[hk + v] = s;
    const float sc = s > 0.f ? 127.0f / s : 0.f;
    uint4* zr = reinterpret_cast<uint4*>(codes + (hk + v) * kD + c0);
    float* pr = pre_round ? pre_round + (hk + v) * kD + c0 : nullptr;
#pragma unroll
    for (int c16 = 0; c16 < FC / 16; ++c16) {
      uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float x = S[16 * c16 + e] * sc;
        if (pr) pr[16 * c16 + e] = x;
        const float qz = fminf(fmaxf(rintf(x), -127.f), 127.f);
        w[e >> 2] |= (uint32_t)((int32_t)qz & 0xff) << (8 * (e & 3));
      }
      zr[c16] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

static int check_state(const leapq_state* st, const char* fn) {
  if (!st) return set_error(GDNRT_EINVAL, "%s: null state", fn);
  if (st->dk != kD || st->dv != kD)
    return set_error(GDNRT_ESHAPE, "%s: d_k=%d d_v=%d, only 128 is supported", fn, st->dk, st->dv);
  if (st->N < 0) return set_error(GDNRT_ESHAPE, "%s: N=%d", fn, st->N);
  if (st->rank < 0 || st->rank > kMaxRank)
    return set_error(GDNRT_ESHAPE, "%s: rank=%d must be in [0, %d]", fn, st->rank, kMaxRank);
  if (st->window < 1 || st->window > kMaxWindow)
    return set_error(GDNRT_ESHAPE, "%s: window=%d must be in [1, %d]", fn, st->window, kMaxWindow);
  if ((size_t)st->N * 4 > 0x7fffffffu) return set_error(GDNRT_ESHAPE, "%s: N too large", fn);
  if (st->N == 0) return GDNRT_OK;
  if (!st->codes || !st->vscale || !st->ksmooth || !st->buf_k || !st->buf_u || !st->buf_a ||
      (st->rank > 0 && (!st->ct_k || !st->ct_u)))
    return set_error(GDNRT_EINVAL, "%s: null buffer in leapq_state", fn);
  if (!aligned16(st->codes) || !aligned16(st->buf_k) || !aligned16(st->buf_u) ||
      !aligned4(st->vscale) || !aligned4(st->ksmooth) || !aligned4(st->buf_a) ||
      (st->rank > 0 && (!aligned16(st->ct_k) || !aligned16(st->ct_u))))
    return set_error(GDNRT_EALIGN, "%s: codes, buf_k, buf_u, ct_k, ct_u must be 16-byte aligned", fn);
  return GDNRT_OK;
}

}  // namespace gdnrt

using namespace gdnrt;

extern "C" int leapq_decode_step(const leapq_state* st, int pos, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta, void* o,
                                 int io, void* stream) {
  int rc = check_state(st, "leapq_decode_step");
  if (rc != GDNRT_OK) return rc;
  if (io != GDNRT_F32 && io != GDNRT_BF16) return set_error(GDNRT_EDTYPE, "leapq_decode_step: io=%d", io);
  if (pos < 0 || pos >= st->window)
    return set_error(GDNRT_ESTATE, "leapq_decode_step: pos=%d outside [0, window=%d)", pos, st->window);
  if (st->N == 0) return clear_error();
  if (!q || !k || !v || !alpha || !beta || !o)
    return set_error(GDNRT_EINVAL, "leapq_decode_step: null pointer argument");
  if (!aligned4(q) || !aligned4(k) || !aligned4(v) || !aligned4(o) || !aligned4(alpha) || !aligned4(beta))
    return set_error(GDNRT_EALIGN, "leapq_decode_step: q, k, v, o, alpha, beta must be 4-byte aligned");
  const size_t es = io == GDNRT_F32 ? 4 : 2;
  const size_t N = st->N, nIO = N * kD * es, nB = N * st->window * kD * 4;
  if (overlaps(o, nIO, q, nIO) || overlaps(o, nIO, k, nIO) || overlaps(o, nIO, v, nIO) ||
      overlaps(o, nIO, st->buf_k, nB) || overlaps(o, nIO, st->buf_u, nB) ||
      overlaps(o, nIO, st->codes, N * kD * kD))
    return set_error(GDNRT_EINVAL, "leapq_decode_step: o overlaps another buffer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  constexpr int RPT = kDecodeRPT;
  const dim3 grid((unsigned)(N * (kD / (32 * RPT)))), block(128);
  if (io == GDNRT_F32)
    hipLaunchKernelGGL((leapq_decode_kernel<float, RPT>), grid, block, 0, s, st->codes, st->vscale,
                       st->ksmooth, st->ct_k, st->ct_u, st->buf_k, st->buf_u, st->buf_a, st->rank,
                       st->window, pos, static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), alpha, beta, static_cast<float*>(o), (int)N);
  else
    hipLaunchKernelGGL((leapq_decode_kernel<uint16_t, RPT>), grid, block, 0, s, st->codes, st->vscale,
                       st->ksmooth, st->ct_k, st->ct_u, st->buf_k, st->buf_u, st->buf_a, st->rank,
                       st->window, pos, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), alpha,
                       beta, static_cast<uint16_t*>(o), (int)N);
  return check_launch("leapq_decode_step");
}

extern "C" int leapq_window_flush(const leapq_state* st, int pos, const float* dense,
                                  const float* q0, int iters, int smooth_mode, float* pre_round,
                                  void* stream) {
  int rc = check_state(st, "leapq_window_flush");
  if (rc != GDNRT_OK) return rc;
  if (pos < 0 || pos > st->window)
    return set_error(GDNRT_ESTATE, "leapq_window_flush: pos=%d outside [0, window=%d]", pos, st->window);
  if (smooth_mode < 0 || smooth_mode > 2)
    return set_error(GDNRT_EINVAL, "leapq_window_flush: smooth_mode=%d", smooth_mode);
  if (iters < 0 || iters > 64) return set_error(GDNRT_EINVAL, "leapq_window_flush: iters=%d", iters);
  if (st->N == 0) return clear_error();
  if (st->rank > 0 && !q0) return set_error(GDNRT_EINVAL, "leapq_window_flush: q0 is null");
  if ((dense && !aligned16(dense)) || (pre_round && !aligned16(pre_round)) || (q0 && !aligned4(q0)))
    return set_error(GDNRT_EALIGN, "leapq_window_flush: dense, pre_round must be 16-byte aligned");
  const size_t N = st->N, nS = N * kD * kD * 4;
  if ((dense && (overlaps(dense, nS, st->codes, N * kD * kD) || overlaps(dense, nS, pre_round, nS))) ||
      (pre_round && overlaps(pre_round, nS, st->codes, N * kD * kD)))
    return set_error(GDNRT_EINVAL, "leapq_window_flush: dense / pre_round overlap the state");
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (st->rank) {
#define GDNRT_FLUSH(R)                                                                            \
  case R:                                                                                         \
    hipLaunchKernelGGL((leapq_flush_kernel<kFlushNQ, R>), dim3((unsigned)N), dim3(128 * kFlushNQ), \
                       0, s, st->codes, st->vscale, st->ksmooth, st->ct_k, st->ct_u, st->buf_k,   \
                       st->buf_u, st->buf_a, st->window, pos, dense, q0, iters, smooth_mode,      \
                       pre_round);                                                                \
    break;
    GDNRT_FLUSH(0) GDNRT_FLUSH(1) GDNRT_FLUSH(2) GDNRT_FLUSH(3) GDNRT_FLUSH(4)
    GDNRT_FLUSH(5) GDNRT_FLUSH(6) GDNRT_FLUSH(7) GDNRT_FLUSH(8)
#undef GDNRT_FLUSH
  }
  return check_launch("leapq_window_flush");
}

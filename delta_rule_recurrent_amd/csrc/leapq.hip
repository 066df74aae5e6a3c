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

constexpr int kP = kD + 1;
constexpr int kFlushNQ = 8;   // 1024 threads per flush block, 16 key columns each

template <int NQ>
struct FlushSmem {
  float S[kD * kP];
  float K[(kMaxRank + kMaxWindow) * kD];   // keys of the rank-one terms (rebuild)
  float Qa[kD * kMaxRank];                 // [c][r]
  float Qb[kD * kMaxRank];
  float Y[kD * kMaxRank];                  // [v][r]
  float part[NQ * kD * kMaxRank];
  float col[kD];
  float red[NQ * kD];
};

// Y[x][r] = sum over the NQ partial sums (threads t < 128 combine)
template <int NQ, int RANK>
__device__ __forceinline__ void combine_parts(FlushSmem<NQ>& sm, float* dst) {
  const int t = threadIdx.x;
  if (t < kD) {
#pragma unroll
    for (int r = 0; r < RANK; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int p = 0; p < NQ; ++p) acc += sm.part[(p * kD + t) * kMaxRank + r];
      dst[t * kMaxRank + r] = acc;
    }
  }
}

// One CholeskyQR pass: dst = src L^{-T}, L L^T = src^T src + (1e-6 tr + 1e-30) I.
// Every wave forms the Gram matrix itself (two rows per lane, wave sums), so the
// only barrier is the one after the rows are written.
template <int RANK>
__device__ void cholqr_pass(const float* src, float* dst) {
  const int lane = threadIdx.x & 63;
  float x0[RANK], x1[RANK];
#pragma unroll
  for (int i = 0; i < RANK; ++i) {
    x0[i] = src[(2 * lane) * kMaxRank + i];
    x1[i] = src[(2 * lane + 1) * kMaxRank + i];
  }
  float G[RANK][RANK];
#pragma unroll
  for (int i = 0; i < RANK; ++i)
#pragma unroll
    for (int j = i; j < RANK; ++j) G[i][j] = sum64(x0[i] * x0[j] + x1[i] * x1[j]);
  float tr = 0.f;
#pragma unroll
  for (int i = 0; i < RANK; ++i) tr += G[i][i];
  const float sh = 1e-6f * tr + 1e-30f;
  float L[RANK][RANK];
#pragma unroll
  for (int i = 0; i < RANK; ++i) {
#pragma unroll
    for (int j = 0; j <= i; ++j) {
      float s = G[j][i] + (i == j ? sh : 0.f);
#pragma unroll
      for (int p = 0; p < j; ++p) s -= L[i][p] * L[j][p];
      L[i][j] = i == j ? sqrtf(fmaxf(s, 0.f)) : s / L[j][j];
    }
  }
  const int t = threadIdx.x;
  if (t < kD) {   // row t: solve x L^T = src[t, :]
    float x[RANK];
#pragma unroll
    for (int j = 0; j < RANK; ++j) {
      float s = src[t * kMaxRank + j];
#pragma unroll
      for (int p = 0; p < j; ++p) s -= x[p] * L[j][p];
      x[j] = s / L[j][j];
      dst[t * kMaxRank + j] = x[j];
    }
  }
  lds_barrier();
}

template <int NQ, int RANK>
__global__ __launch_bounds__(128 * NQ) void leapq_flush_kernel(
    int8_t* __restrict__ codes, float* __restrict__ vscale, float* __restrict__ ksmooth,
    uint16_t* __restrict__ ct_k, uint16_t* __restrict__ ct_u, const float* __restrict__ buf_k,
    const float* __restrict__ buf_u, const float* __restrict__ buf_a, int window, int m,
    const float* __restrict__ dense, const float* __restrict__ q0, int iters, int smooth_mode,
    float* __restrict__ pre_round) {
  constexpr int NT = 128 * NQ, FC = kD / NQ;
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
    const int nt = rank + m;
    for (int i = tid; i < nt * kD; i += NT) {
      const int j = i / kD, c = i % kD;
      sm.K[i] = j < rank ? h2f(ct_k[((size_t)head * rank + j) * kD + c])
                         : buf_k[((size_t)head * window + (j - rank)) * kD + c];
    }
    if (tid < kD) sm.col[tid] = ksmooth[hk + tid];
    lds_barrier();
#pragma unroll
    for (int i = 0; i < FC; ++i) S[i] = 0.f;
    const float* ba = buf_a + (size_t)head * window;
    float g = 1.f;
    for (int j = m - 1; j >= 0; --j) {       // newest record first: suffix-product decays
      const float cj = g * buf_u[((size_t)head * window + j) * kD + v];
      const f32x4* Kj = reinterpret_cast<const f32x4*>(sm.K + (rank + j) * kD + c0);
#pragma unroll
      for (int i = 0; i < FC / 4; ++i) {
        const f32x4 kk = Kj[i];
        S[4 * i] += cj * kk.x; S[4 * i + 1] += cj * kk.y; S[4 * i + 2] += cj * kk.z; S[4 * i + 3] += cj * kk.w;
      }
      g *= ba[j];
    }
    const float g0 = g;
    for (int r = 0; r < rank; ++r) {
      const float cr = g0 * h2f(ct_u[((size_t)head * rank + r) * kD + v]);
      const f32x4* Kr = reinterpret_cast<const f32x4*>(sm.K + r * kD + c0);
#pragma unroll
      for (int i = 0; i < FC / 4; ++i) {
        const f32x4 kk = Kr[i];
        S[4 * i] += cr * kk.x; S[4 * i + 1] += cr * kk.y; S[4 * i + 2] += cr * kk.z; S[4 * i + 3] += cr * kk.w;
      }
    }
    const float sv = g0 * vscale[hk + v] * (1.0f / 127.0f);
    const uint4* zp = reinterpret_cast<const uint4*>(codes + (hk + v) * kD + c0);
#pragma unroll
    for (int c16 = 0; c16 < FC / 16; ++c16) {
      const uint4 zw = zp[c16];
      const uint32_t z4[4] = {zw.x, zw.y, zw.z, zw.w};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int i = 16 * c16 + e;
        S[i] += sv * sb(z4[e >> 2], e & 3) * sm.col[c0 + i];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < FC; ++i) sm.S[v * kP + c0 + i] = S[i];

  // ---------------------------------------------------------------- compensators
  if constexpr (RANK > 0) {
    for (int i = tid; i < kD * rank; i += NT) sm.Qa[(i / rank) * kMaxRank + (i % rank)] = q0[i];
    lds_barrier();
    for (int it = 0; it <= iters; ++it) {
      // Y = S Q from the registers
      float acc[RANK];
#pragma unroll
      for (int r = 0; r < RANK; ++r) acc[r] = 0.f;
#pragma unroll
      for (int i = 0; i < FC; ++i) {
        const float* qr = sm.Qa + (c0 + i) * kMaxRank;
#pragma unroll
        for (int r = 0; r < RANK; ++r) acc[r] += S[i] * qr[r];
      }
#pragma unroll
      for (int r = 0; r < RANK; ++r) sm.part[(qd * kD + v) * kMaxRank + r] = acc[r];
      lds_barrier();
      combine_parts<NQ, RANK>(sm, sm.Y);
      lds_barrier();
      if (it == iters) break;   // final Y = S Q: the compensator values
      // Q = S^T Y from the LDS copy: column c = v over rows [c0, c0 + FC)
#pragma unroll
      for (int r = 0; r < RANK; ++r) acc[r] = 0.f;
#pragma unroll
      for (int i = 0; i < FC; ++i) {
        const int vv = c0 + i;
        const float sc = sm.S[vv * kP + v];
        const float* yr = sm.Y + vv * kMaxRank;
#pragma unroll
        for (int r = 0; r < RANK; ++r) acc[r] += sc * yr[r];
      }
#pragma unroll
      for (int r = 0; r < RANK; ++r) sm.part[(qd * kD + v) * kMaxRank + r] = acc[r];
      lds_barrier();
      combine_parts<NQ, RANK>(sm, sm.Qa);
      lds_barrier();
      cholqr_pass<RANK>(sm.Qa, sm.Qb);
      cholqr_pass<RANK>(sm.Qb, sm.Qa);
    }
    // round to fp16, store, keep the rounded values for the residual
    if (tid < kD) {
      for (int r = 0; r < rank; ++r) {
        const uint16_t hq = f2h(sm.Qa[tid * kMaxRank + r]);
        const uint16_t hy = f2h(sm.Y[tid * kMaxRank + r]);
        ct_k[((size_t)head * rank + r) * kD + tid] = hq;
        ct_u[((size_t)head * rank + r) * kD + tid] = hy;
        sm.Qb[tid * kMaxRank + r] = h2f(hq);
        sm.part[tid * kMaxRank + r] = h2f(hy);
      }
    }
    lds_barrier();
    // residual R = S - sum_r uh_r kh_r^T
    float yh[RANK];
#pragma unroll
    for (int r = 0; r < RANK; ++r) yh[r] = sm.part[v * kMaxRank + r];
#pragma unroll
    for (int i = 0; i < FC; ++i) {
      const float* qr = sm.Qb + (c0 + i) * kMaxRank;
#pragma unroll
      for (int r = 0; r < RANK; ++r) S[i] -= yh[r] * qr[r];
      sm.S[v * kP + c0 + i] = S[i];
    }
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
    for (int i = 0; i < FC; ++i) {
      S[i] *= sm.col[c0 + i];
      mx = fmaxf(mx, fabsf(S[i]));
    }
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

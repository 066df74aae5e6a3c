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
// is appended at slot m. A block owns 32 value rows of one head (4 blocks per
// head): 8 lanes per 128-byte code row, one 16-byte load each; per-head dot
// products with the buffered and compensator keys are formed by 16-lane groups.

constexpr int kLqRows = 32;   // value rows per decode block
constexpr int kLqBPH = kD / kLqRows;

template <typename IO>
__global__ __launch_bounds__(256) void leapq_decode_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ vscale,
    const float* __restrict__ ksmooth, const uint16_t* __restrict__ ct_k,
    const uint16_t* __restrict__ ct_u, float* __restrict__ buf_k, float* __restrict__ buf_u,
    float* __restrict__ buf_a, int rank, int window, int m,
    const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, IO* __restrict__ o) {
  __shared__ float s_k[kD], s_q[kD], s_xk[kD], s_xq[kD];
  __shared__ float s_dk[kMaxRank + kMaxWindow + 1], s_dq[kMaxRank + kMaxWindow + 1];
  __shared__ float s_g[kMaxWindow + 1];   // s_g[j] = G_j for j < m, s_g[m] = G0

  const int tid = threadIdx.x;
  const int head = blockIdx.x / kLqBPH;
  const int rb = blockIdx.x % kLqBPH;
  const float a = alpha[head];
  const float b = beta[head];
  const size_t hk = (size_t)head * kD;
  float* bk = buf_k + (size_t)head * window * kD;
  float* bu = buf_u + (size_t)head * window * kD;
  const float* ba = buf_a + (size_t)head * window;

  if (tid < kD) {
    const float kv = io_traits<IO>::ld(k, hk + tid);
    const float qv = io_traits<IO>::ld(q, hk + tid);
    const float c = ksmooth[hk + tid];
    s_k[tid] = kv;
    s_q[tid] = qv;
    s_xk[tid] = c * kv;
    s_xq[tid] = c * qv;
    // append this token's key: each of the head's blocks writes its quarter
    if ((tid >> 5) == rb) bk[(size_t)m * kD + tid] = kv;
  } else if (tid == kD) {
    float g = 1.f;
    for (int j = m - 1; j >= 0; --j) {   // suffix products of the buffered decays
      s_g[j] = g;
      g *= ba[j];
    }
    s_g[m] = g;
    if (rb == 0) buf_a[(size_t)head * window + m] = a;
  }
  __syncthreads();

  // dot products of q and k with every compensator key, buffered key, and k itself
  const int nv = rank + m + 1;
  {
    const int grp = tid >> 4, l16 = tid & 15;
    const int c0 = l16 * 8;
    for (int vi = grp; vi < nv; vi += 16) {
      float w[8];
      if (vi < rank) {
        const uint4 raw = *reinterpret_cast<const uint4*>(ct_k + ((size_t)head * rank + vi) * kD + c0);
        const uint32_t r4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[2 * e] = h2f(uint16_t(r4[e] & 0xffffu));
          w[2 * e + 1] = h2f(uint16_t(r4[e] >> 16));
        }
      } else if (vi < rank + m) {
        const f32x4* p = reinterpret_cast<const f32x4*>(bk + (size_t)(vi - rank) * kD + c0);
        const f32x4 x0 = p[0], x1 = p[1];
        w[0] = x0.x; w[1] = x0.y; w[2] = x0.z; w[3] = x0.w;
        w[4] = x1.x; w[5] = x1.y; w[6] = x1.z; w[7] = x1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = s_k[c0 + e];
      }
      float pk = 0.f, pq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pk += w[e] * s_k[c0 + e];
        pq += w[e] * s_q[c0 + e];
      }
      pk = sum16(pk);
      pq = sum16(pq);
      if (l16 == 0) {
        s_dk[vi] = pk;
        s_dq[vi] = pq;
      }
    }
  }
  __syncthreads();

  // rows: 8 lanes per row, 16 codes per lane
  const int rl = tid >> 3, sub = tid & 7;
  const int row = rb * kLqRows + rl;
  const int c0 = sub * 16;
  const uint4 zw = *reinterpret_cast<const uint4*>(codes + ((size_t)head * kD + row) * kD + c0);
  const uint32_t z4[4] = {zw.x, zw.y, zw.z, zw.w};
  float yk = 0.f, yq = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const float z = sb(z4[e], bb);
      yk += z * s_xk[c0 + 4 * e + bb];
      yq += z * s_xq[c0 + 4 * e + bb];
    }
  }
  // compensator and buffered contributions of this row, split over the 8 lanes
  float ck = 0.f, cq = 0.f, tk = 0.f, tq = 0.f;
  for (int r = sub; r < rank; r += 8) {
    const float uc = h2f(ct_u[((size_t)head * rank + r) * kD + row]);
    ck += uc * s_dk[r];
    cq += uc * s_dq[r];
  }
  for (int j = sub; j < m; j += 8) {
    const float w = s_g[j] * bu[(size_t)j * kD + row];
    tk += w * s_dk[rank + j];
    tq += w * s_dq[rank + j];
  }
  yk = sum8(yk);
  yq = sum8(yq);
  ck = sum8(ck);
  cq = sum8(cq);
  tk = sum8(tk);
  tq = sum8(tq);
  const float g0 = s_g[m];
  const float sv = vscale[hk + row] * (1.0f / 127.0f);
  const float Sk = g0 * (sv * yk + ck) + tk;
  const float Sq = g0 * (sv * yq + cq) + tq;
  const float u = b * (io_traits<IO>::ld(v, hk + row) - a * Sk);
  const float oi = a * Sq + u * s_dq[rank + m];
  if (sub == 0) {
    bu[(size_t)m * kD + row] = u;
    io_traits<IO>::st(o, hk + row, oi);
  }
}

// ============================================================== window flush
//
// One 256-thread block per head; the dense state lives in LDS as [128][129] fp32.
// Thread t works on value row (t & 127) over key columns [64h, 64h+64), h = t >> 7,
// for row operations, and on key column (t & 127) over value rows [64h, 64h+64)
// for column operations; the two halves are combined through LDS. Steps:
//   rebuild (eq. 4) or load `dense`; compensator fit by subspace iteration with
//   CholeskyQR2; subtract the fp16-rounded pieces; smoothing factors; value-channel
//   scales; codes.

constexpr int kP = kD + 1;   // LDS pitch of the dense state (conflict-free rows and columns)

__device__ __forceinline__ void block_sync() { __syncthreads(); }

// LDS scratch of one flush block
struct FlushSmem {
  float S[kD * kP];                          // dense state, then residual
  float K[(kMaxRank + kMaxWindow) * kD];      // keys of the rank-one terms (rebuild), fp32
  float Q[kD * kMaxRank];                    // [c][r] current orthonormal block
  float Y[kD * kMaxRank];                    // [v][r] S Q
  float part[2 * kD * kMaxRank];             // half-sums
  float G[kMaxRank * kMaxRank];              // Gram / Cholesky factor
  float col[kD];                             // per key column: 1 / smoothing factor
  float red[2 * kD];
};

// Q <- Q L^{-T} where L L^T = Q^T Q + (1e-6 tr + 1e-30) I, twice (CholeskyQR2).
// Input and output in sm.Q ([c][r]); all threads participate.
__device__ void cholqr2(FlushSmem& sm, int rank) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int pass = 0; pass < 2; ++pass) {
    // Gram entries (i, j), i <= j, one wave per entry at a time: 2 rows per lane
    const int ne = rank * rank;
    for (int e = wave; e < ne; e += 4) {
      const int i = e / rank, j = e % rank;
      if (i > j) continue;
      float p = sm.Q[(2 * lane) * kMaxRank + i] * sm.Q[(2 * lane) * kMaxRank + j] +
                sm.Q[(2 * lane + 1) * kMaxRank + i] * sm.Q[(2 * lane + 1) * kMaxRank + j];
      p = sum64(p);
      if (lane == 0) sm.G[i * kMaxRank + j] = p;
    }
    block_sync();
    if (tid == 0) {
      float tr = 0.f;
      for (int i = 0; i < rank; ++i) tr += sm.G[i * kMaxRank + i];
      const float sh = 1e-6f * tr + 1e-30f;
      // Cholesky in place (lower factor in sm.G[i][j], j <= i), from the upper entries
      for (int i = 0; i < rank; ++i) {
        for (int j = 0; j <= i; ++j) {
          float s = sm.G[j * kMaxRank + i] + (i == j ? sh : 0.f);   // G[j][i] == G[i][j]
          for (int p = 0; p < j; ++p) s -= sm.G[i * kMaxRank + p] * sm.G[j * kMaxRank + p];
          if (i == j) sm.G[i * kMaxRank + i] = sqrtf(fmaxf(s, 0.f));
          else sm.G[i * kMaxRank + j] = s / sm.G[j * kMaxRank + j];
        }
      }
    }
    block_sync();
    if (tid < kD) {   // row c of Q: solve x L^T = Q[c, :]
      float x[kMaxRank];
#pragma unroll
      for (int j = 0; j < kMaxRank; ++j) {
        if (j < rank) {
          float s = sm.Q[tid * kMaxRank + j];
#pragma unroll
          for (int p = 0; p < j; ++p) s -= x[p] * sm.G[j * kMaxRank + p];
          x[j] = s / sm.G[j * kMaxRank + j];
        }
      }
#pragma unroll
      for (int j = 0; j < kMaxRank; ++j)
        if (j < rank) sm.Q[tid * kMaxRank + j] = x[j];
    }
    block_sync();
  }
}

// Y = S Q ([v][r]) from the dense state in LDS
__device__ void mul_SQ(FlushSmem& sm, int rank) {
  const int tid = threadIdx.x, v = tid & (kD - 1), h = tid >> 7;
  float acc[kMaxRank];
#pragma unroll
  for (int r = 0; r < kMaxRank; ++r) acc[r] = 0.f;
  for (int i = 0; i < 64; ++i) {
    const int c = h * 64 + i;
    const float s = sm.S[v * kP + c];
#pragma unroll
    for (int r = 0; r < kMaxRank; ++r)
      if (r < rank) acc[r] += s * sm.Q[c * kMaxRank + r];
  }
#pragma unroll
  for (int r = 0; r < kMaxRank; ++r)
    if (r < rank) sm.part[(h * kD + v) * kMaxRank + r] = acc[r];
  block_sync();
  if (tid < kD)
    for (int r = 0; r < rank; ++r)
      sm.Y[tid * kMaxRank + r] = sm.part[tid * kMaxRank + r] + sm.part[(kD + tid) * kMaxRank + r];
  block_sync();
}

// Q = S^T Y ([c][r])
__device__ void mul_StY(FlushSmem& sm, int rank) {
  const int tid = threadIdx.x, c = tid & (kD - 1), h = tid >> 7;
  float acc[kMaxRank];
#pragma unroll
  for (int r = 0; r < kMaxRank; ++r) acc[r] = 0.f;
  for (int i = 0; i < 64; ++i) {
    const int v = h * 64 + i;
    const float s = sm.S[v * kP + c];
#pragma unroll
    for (int r = 0; r < kMaxRank; ++r)
      if (r < rank) acc[r] += s * sm.Y[v * kMaxRank + r];
  }
#pragma unroll
  for (int r = 0; r < kMaxRank; ++r)
    if (r < rank) sm.part[(h * kD + c) * kMaxRank + r] = acc[r];
  block_sync();
  if (tid < kD)
    for (int r = 0; r < rank; ++r)
      sm.Q[tid * kMaxRank + r] = sm.part[tid * kMaxRank + r] + sm.part[(kD + tid) * kMaxRank + r];
  block_sync();
}

__global__ __launch_bounds__(256) void leapq_flush_kernel(
    int8_t* __restrict__ codes, float* __restrict__ vscale, float* __restrict__ ksmooth,
    uint16_t* __restrict__ ct_k, uint16_t* __restrict__ ct_u, const float* __restrict__ buf_k,
    const float* __restrict__ buf_u, const float* __restrict__ buf_a, int rank, int window, int m,
    const float* __restrict__ dense, const float* __restrict__ q0, int iters, int smooth_mode,
    float* __restrict__ pre_round) {
  __shared__ FlushSmem sm;
  const int tid = threadIdx.x;
  const int head = blockIdx.x;
  const size_t hk = (size_t)head * kD;
  const int v = tid & (kD - 1), h = tid >> 7;

  // ---------------------------------------------------------------- dense state
  if (dense) {
    const float* Dh = dense + hk * kD;
    for (int i = tid; i < kD * kD / 4; i += 256) {
      const f32x4 x = reinterpret_cast<const f32x4*>(Dh)[i];
      const int r = (4 * i) / kD, c = (4 * i) % kD;
      sm.S[r * kP + c] = x.x;
      sm.S[r * kP + c + 1] = x.y;
      sm.S[r * kP + c + 2] = x.z;
      sm.S[r * kP + c + 3] = x.w;
    }
    block_sync();
  } else {
    // keys of the rank-one terms: compensator keys first, then the buffered keys
    const int nt = rank + m;
    for (int i = tid; i < nt * kD; i += 256) {
      const int j = i / kD, c = i % kD;
      sm.K[i] = j < rank ? h2f(ct_k[((size_t)head * rank + j) * kD + c])
                         : buf_k[((size_t)head * window + (j - rank)) * kD + c];
    }
    if (tid < kD) sm.col[tid] = ksmooth[hk + tid];
    block_sync();
    // row v, columns [64h, 64h+64): buffered writes (newest first, suffix-product
    // decays), then the compensator pieces and the dequantised residual, both
    // decayed by G0
    const float* ba = buf_a + (size_t)head * window;
    float acc[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) acc[i] = 0.f;
    float g = 1.f;
    for (int j = m - 1; j >= 0; --j) {
      const float cj = g * buf_u[((size_t)head * window + j) * kD + v];
      const float* Kj = sm.K + (rank + j) * kD + h * 64;
#pragma unroll
      for (int i = 0; i < 64; ++i) acc[i] += cj * Kj[i];
      g *= ba[j];
    }
    const float g0 = g;
    for (int r = 0; r < rank; ++r) {
      const float cr = g0 * h2f(ct_u[((size_t)head * rank + r) * kD + v]);
      const float* Kr = sm.K + r * kD + h * 64;
#pragma unroll
      for (int i = 0; i < 64; ++i) acc[i] += cr * Kr[i];
    }
    const float sv = g0 * vscale[hk + v] * (1.0f / 127.0f);
    const int8_t* zr = codes + (hk + v) * kD + h * 64;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const uint4 zw = *reinterpret_cast<const uint4*>(zr + 16 * c4);
      const uint32_t z4[4] = {zw.x, zw.y, zw.z, zw.w};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int i = 16 * c4 + e;
        acc[i] += sv * sb(z4[e >> 2], e & 3) * sm.col[h * 64 + i];
      }
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) sm.S[v * kP + h * 64 + i] = acc[i];
    block_sync();
  }

  // ---------------------------------------------------------------- compensators
  if (rank > 0) {
    for (int i = tid; i < kD * rank; i += 256) sm.Q[(i / rank) * kMaxRank + (i % rank)] = q0[i];
    block_sync();
    for (int it = 0; it < iters; ++it) {
      mul_SQ(sm, rank);
      mul_StY(sm, rank);
      cholqr2(sm, rank);
    }
    mul_SQ(sm, rank);
    // round to fp16, store, keep the rounded values for the residual
    if (tid < kD) {
      for (int r = 0; r < rank; ++r) {
        const uint16_t hq = f2h(sm.Q[tid * kMaxRank + r]);
        const uint16_t hy = f2h(sm.Y[tid * kMaxRank + r]);
        ct_k[((size_t)head * rank + r) * kD + tid] = hq;
        ct_u[((size_t)head * rank + r) * kD + tid] = hy;
        sm.Q[tid * kMaxRank + r] = h2f(hq);
        sm.Y[tid * kMaxRank + r] = h2f(hy);
      }
    }
    block_sync();
    // residual R = S - sum_r uh_r kh_r^T, row-wise in place
    for (int i = 0; i < 64; ++i) {
      const int c = h * 64 + i;
      float s = sm.S[v * kP + c];
      for (int r = 0; r < rank; ++r) s -= sm.Y[v * kMaxRank + r] * sm.Q[c * kMaxRank + r];
      sm.S[v * kP + c] = s;
    }
    block_sync();
  }

  // ---------------------------------------------------------------- smoothing
  {
    const int c = v;
    float acc = 0.f;
    for (int i = 0; i < 64; ++i) {
      const float x = sm.S[(h * 64 + i) * kP + c];
      acc += smooth_mode == 1 ? x * x : fabsf(x);
    }
    sm.red[h * kD + c] = acc;
    block_sync();
    if (tid < kD) {
      float cf = 1.f;
      if (smooth_mode != 2) cf = fmaxf(sqrtf((sm.red[tid] + sm.red[kD + tid]) * (1.0f / kD)), 1e-12f);
      ksmooth[hk + tid] = cf;
      sm.col[tid] = 1.0f / cf;
    }
    block_sync();
  }

  // ---------------------------------------------------------------- scales, codes
  {
    float mx = 0.f;
    for (int i = 0; i < 64; ++i) {
      const int c = h * 64 + i;
      mx = fmaxf(mx, fabsf(sm.S[v * kP + c] * sm.col[c]));
    }
    sm.red[h * kD + v] = mx;
    block_sync();
    const float s = fmaxf(sm.red[v], sm.red[kD + v]);
    if (h == 0) vscale[hk + v] = s;
    const float sc = s > 0.f ? 127.0f / s : 0.f;
    int8_t* zr = codes + (hk + v) * kD + h * 64;
    float* pr = pre_round ? pre_round + (hk + v) * kD + h * 64 : nullptr;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = h * 64 + 16 * c4 + e;
        const float x = (sm.S[v * kP + c] * sm.col[c]) * sc;
        if (pr) pr[16 * c4 + e] = x;
        const float qz = fminf(fmaxf(rintf(x), -127.f), 127.f);
        w[e >> 2] |= (uint32_t)((int32_t)qz & 0xff) << (8 * (e & 3));
      }
      *reinterpret_cast<uint4*>(zr + 16 * c4) = make_uint4(w[0], w[1], w[2], w[3]);
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
  if ((size_t)st->N * kLqBPH > 0x7fffffffu) return set_error(GDNRT_ESHAPE, "%s: N too large", fn);
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
  const dim3 grid((unsigned)(N * kLqBPH)), block(256);
  if (io == GDNRT_F32)
    hipLaunchKernelGGL(leapq_decode_kernel<float>, grid, block, 0, s, st->codes, st->vscale,
                       st->ksmooth, st->ct_k, st->ct_u, st->buf_k, st->buf_u, st->buf_a, st->rank,
                       st->window, pos, static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), alpha, beta, static_cast<float*>(o));
  else
    hipLaunchKernelGGL(leapq_decode_kernel<uint16_t>, grid, block, 0, s, st->codes, st->vscale,
                       st->ksmooth, st->ct_k, st->ct_u, st->buf_k, st->buf_u, st->buf_a, st->rank,
                       st->window, pos, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), alpha,
                       beta, static_cast<uint16_t*>(o));
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
  hipLaunchKernelGGL(leapq_flush_kernel, dim3((unsigned)N), dim3(256), 0, s, st->codes,
                     st->vscale, st->ksmooth, st->ct_k, st->ct_u, st->buf_k, st->buf_u, st->buf_a,
                     st->rank, st->window, pos, dense, q0, iters, smooth_mode, pre_round);
  return check_launch("leapq_window_flush");
}

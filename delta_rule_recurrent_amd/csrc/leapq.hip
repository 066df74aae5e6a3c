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

// Packed code rows (bits = 4 or 6; one byte per code otherwise). A value row's 128 codes
// are 16 * bits bytes: at 4 bits byte j holds codes 2 j (low nibble) and 2 j + 1; at 6 bits
// each 3 bytes hold four codes, code 4 c + i in bits [6 i, 6 i + 6) of the little-endian
// 24-bit group c. Codes are two's complement in their width.
__host__ __device__ constexpr int row_bytes(int pk) { return pk == 8 ? 128 : 16 * pk; }

// four codes of width 4 or 6 in the low byte of each byte lane -> four int8 (sign extension)
template <int PK>
__device__ __forceinline__ uint32_t sext4(uint32_t x) {
  constexpr uint32_t sign = 0x01010101u << (PK - 1), high = 0xffu & ~((1u << PK) - 1u);
  return x | ((x & sign) >> (PK - 1)) * high;
}
// 8 codes at 4 bits (one word) -> 2 words of 4 int8, in order
__device__ __forceinline__ void unpack4(uint32_t w, uint32_t& a, uint32_t& b) {
  const uint32_t lo = sext4<4>(w & 0x0f0f0f0fu), hi = sext4<4>((w >> 4) & 0x0f0f0f0fu);
  a = __builtin_amdgcn_perm(hi, lo, 0x05010400u);   // codes 0..3: lo.b0, hi.b0, lo.b1, hi.b1
  b = __builtin_amdgcn_perm(hi, lo, 0x07030602u);   // codes 4..7
}
// 4 codes at 6 bits (one 24-bit group, low bits of g) -> 1 word of 4 int8
__device__ __forceinline__ uint32_t unpack6(uint32_t g) {
  const uint32_t x = (g & 0x3fu) | ((g << 2) & 0x3f00u) | ((g << 4) & 0x3f0000u) | ((g << 6) & 0x3f000000u);
  return sext4<6>(x);
}
// 16 codes at 6 bits (three words, 12 bytes) -> 4 words of 4 int8
__device__ __forceinline__ void unpack6x16(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t (&o)[4]) {
  o[0] = unpack6(w0);
  o[1] = unpack6(__builtin_amdgcn_alignbit(w1, w0, 24));
  o[2] = unpack6(__builtin_amdgcn_alignbit(w2, w1, 16));
  o[3] = unpack6(w2 >> 8);
}
// 8 int8 codes (two words) -> one word of 4-bit codes
__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b) {
  auto half = [](uint32_t x) {
    x &= 0x0f0f0f0fu;
    x = (x | (x >> 4)) & 0x00ff00ffu;
    return (x | (x >> 8)) & 0xffffu;
  };
  return half(a) | (half(b) << 16);
}
// 4 int8 codes (one word) -> one 24-bit group of 6-bit codes
__device__ __forceinline__ uint32_t pack6(uint32_t w) {
  const uint32_t x = w & 0x3f3f3f3fu;
  return (x & 0x3fu) | ((x >> 2) & 0xfc0u) | ((x >> 4) & 0x3f000u) | ((x >> 6) & 0xfc0000u);
}

// Suffix products of the m buffered decays a_0 .. a_{m-1} of one channel (stride
// floats apart): put(j, prod_{j<i<m} a_i) for j < m, then put(m, prod_{i<m} a_i),
// multiplied newest first. Every decay is requested before the first product, so
// the loads overlap instead of each waiting for the one before.
template <typename Put>
__device__ __forceinline__ void suffix_products(const float* __restrict__ a, size_t stride, int m, Put&& put) {
  float av[kMaxWindow];
#pragma unroll
  for (int j = 0; j < kMaxWindow; ++j) av[j] = j < m ? a[(size_t)j * stride] : 1.f;
  float gg = 1.f;
#pragma unroll
  for (int j = kMaxWindow - 1; j >= 0; --j) {
    if (j < m) {
      put(j, gg);
      gg *= av[j];
    }
  }
  put(m, gg);
}

// ============================================================== decode step
//
// Per head, with m = pos buffered records (k_j, u_j, a_j) and compensator pairs
// (kc_r, uc_r), the state after the m records applied to a vector x is
//   S_m x = G0 [ vscale * (Z (ksmooth o x)) / 127 + sum_r uc_r (kc_r . x) ]
//         + sum_j G_j u_j (k_j . x),   G0 = prod_{i<m} a_i,  G_j = prod_{j<i<m} a_i.
// The token then gives u = b (v - a S_m k), o = a S_m q + u (k . q), and its record
// is appended at slot m.
//
// One block of 256 threads (four waves) per head; wave w owns value rows
// [32 w, 32 w + 32) as two tiles of 16. The products Z x_k and Z x_q run on the
// int8 matrix cores with the stored codes as they are: each wave writes the two read
// vectors x = ksmooth o k, ksmooth o q as 22-bit fixed point relative to their
// largest entry (x ~= X 2^(e-22), |X| < 2^22), split into three signed int8 digits
// (X = 2^16 d0 + 2^8 d1 + d2, each in [-128, 127]), and v_mfma_i32_16x16x64_i8 forms
// the exact integer products of the digits with the code rows. The only rounding of
// the read-out is the fixed-point rounding of x (2^-23 of its largest entry) and the
// fp32 arithmetic after the integer sums. Everything else a row needs (compensator
// and buffered terms) comes from per-head dot products formed by 16-lane groups
// before the block's one barrier.

typedef int i32x4 __attribute__((ext_vector_type(4)));

// LDS written by some lanes of a wave and read by others of the same wave: the LDS
// executes a wave's instructions in order, so this only keeps the compiler from
// reordering the accesses
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// largest value over the 16 lanes of a DPP row (every lane receives it)
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp<0x140>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0xB1>(x));
  return x;
}

// Fixed-point digits of 8 values sharing the scale of `mx` (the largest magnitude
// of the vector): X = rint(x 2^(22 - e)), mx = f 2^e with f in [0.5, 1), so
// |X| < 2^22; balanced base-256 digits d0 (|d0| <= 64), d1, d2 in [-128, 127],
// packed 8 to a uint2 per digit. Returns e (0 for a zero vector).
__device__ __forceinline__ int fixed_digits(const float (&x)[8], float mx, uint2 (&d)[3]) {
  int e = 0;
  if (mx > 0.f) (void)frexpf(mx, &e);
  if (e < -100) e = 0, mx = 0.f;   // nothing measurable: a zero vector
  const float sc = mx > 0.f ? ldexpf(1.0f, 22 - e) : 0.f;
  uint32_t w[3][2] = {{0, 0}, {0, 0}, {0, 0}};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int X = (int)rintf(x[i] * sc);
    const int lo = ((X + 128) & 0xff) - 128;
    const int X1 = (X - lo) >> 8;
    const int mid = ((X1 + 128) & 0xff) - 128;
    const int hi = (X1 - mid) >> 8;
    w[0][i >> 2] |= (uint32_t)(hi & 0xff) << (8 * (i & 3));
    w[1][i >> 2] |= (uint32_t)(mid & 0xff) << (8 * (i & 3));
    w[2][i >> 2] |= (uint32_t)(lo & 0xff) << (8 * (i & 3));
  }
#pragma unroll
  for (int t = 0; t < 3; ++t) d[t] = make_uint2(w[t][0], w[t][1]);
  return e;
}

// PK: the code width in memory, 8 (one byte per code, read through LDS) or 4 / 6 (packed
// rows, read into registers and widened to int8 there).
template <typename IO, bool KDA, int PK>
__global__ __launch_bounds__(256) void leapq_decode_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ vscale,
    const float* __restrict__ ksmooth, const uint16_t* __restrict__ ct_k,
    const uint16_t* __restrict__ ct_u, float* __restrict__ buf_k, float* __restrict__ buf_u,
    float* __restrict__ buf_a, int rank, int window, int m, float qinv,
    const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, IO* __restrict__ o) {
  constexpr int NV = kMaxRank + kMaxWindow;   // dot-product vectors: compensators, records, k
  // this head's codes, straight from HBM (rows of eight 16-byte pieces; piece c of row r
  // at slot c ^ ((r >> 1) & 7), so that the 16 rows an MFMA operand read takes fall on
  // distinct banks)
  __shared__ __attribute__((aligned(16))) int8_t s_codes[PK == 8 ? kD * kD : 16];
  __shared__ __attribute__((aligned(16))) uint2 s_dig[4][8][kD / 8];   // per wave: digit rows
                                                                      // (x_k 0-2, x_q 3-5, 6-7 zero)
  __shared__ float s_dk[NV], s_dq[NV];
  __shared__ float s_g[kMaxWindow + 1];       // s_g[j] = G_j for j < m, s_g[m] = G0
  // KDA: the same products per key channel, s_gv[j][c] = prod_{j<i<m} a_i[c], s_gv[m] = G0
  __shared__ float s_gv[KDA ? kMaxWindow + 1 : 1][KDA ? kD : 1];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int head = blockIdx.x;
  const size_t hk = (size_t)head * kD;
  float* bk = buf_k + (size_t)head * window * kD;
  float* bu = buf_u + (size_t)head * window * kD;
  const float* ba = buf_a + (size_t)head * window;
  const int nv = rank + m;   // vectors before k itself
  const int row[2] = {32 * w + n, 32 * w + 16 + n};

  // ---- independent loads
  // the codes of this wave's rows go straight to LDS (LDS DMA: no registers, so more heads
  // fit on a CU): instruction i of wave w fills rows 32 w + 8 i .. + 7, lane L slot L & 7 of
  // row 32 w + 8 i + L / 8. Non-temporal: the codes of all heads do not fit the caches
  // between two steps, and keeping them out leaves room for the buffered records, which
  // every step re-reads.
  // Packed rows instead: the lane's codes (row 32 w + 16 T + n, codes 64 s + 16 g ..
  // + 15) as 8 or 12 bytes in registers.
  constexpr int RB = row_bytes(PK);
  uint32_t zp[2][2][PK == 6 ? 3 : 2];
  if constexpr (PK == 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * w + 8 * i + (lane >> 3), c = (lane & 7) ^ ((r >> 1) & 7);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(codes + (hk + r) * kD + 16 * c),
                                       (__attribute__((address_space(3))) void*)(s_codes + (32 * w + 8 * i) * kD),
                                       16, 0, 2 /* nt */);
    }
  } else {
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(codes + (hk + row[T]) * RB + (64 * s + 16 * g) * PK / 8);
#pragma unroll
        for (int e = 0; e < (PK == 6 ? 3 : 2); ++e) zp[T][s][e] = __builtin_nontemporal_load(src + e);
      }
  }
  // buffered corrections and compensator values of this lane's rows, slots = g (mod 4)
  float bur[2][kMaxWindow / 4], cur[2][kMaxRank / 4], vrow[2], vsr[2];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
#pragma unroll
    for (int jj = 0; jj < kMaxWindow / 4; ++jj) {
      const int j = 4 * jj + g;
      bur[T][jj] = j < m ? bu[(size_t)j * kD + row[T]] : 0.f;
    }
#pragma unroll
    for (int rr = 0; rr < kMaxRank / 4; ++rr) {
      const int r = 4 * rr + g;
      cur[T][rr] = r < rank ? h2f(ct_u[((size_t)head * rank + r) * kD + row[T]]) : 0.f;
    }
    vrow[T] = io_traits<IO>::ld(v, hk + row[T]);
    vsr[T] = vscale[hk + row[T]];
  }
  // this lane's key channels 8 n .. 8 n + 7 of k, q and the smoothing factors
  float kx[8], qx[8], cx[8];
  {
    const int c0 = 8 * n;
    const f32x4 k0 = io_traits<IO>::ld4(k, hk + c0), k1 = io_traits<IO>::ld4(k, hk + c0 + 4);
    const f32x4 q0 = io_traits<IO>::ld4(q, hk + c0), q1 = io_traits<IO>::ld4(q, hk + c0 + 4);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(ksmooth + hk + c0);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(ksmooth + hk + c0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kx[e] = k0[e]; kx[4 + e] = k1[e];
      qx[e] = q0[e]; qx[4 + e] = q1[e];
      cx[e] = s0[e]; cx[4 + e] = s1[e];
    }
  }
  // dot vectors of 16-lane group 4 w + g: indices 4 w + g and 4 w + g + 16
  float wv[2][8];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int vi = 4 * w + g + 16 * p;
    if (vi < rank) {
      const uint4 raw = *reinterpret_cast<const uint4*>(ct_k + ((size_t)head * rank + vi) * kD + 8 * n);
      const uint32_t r4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wv[p][2 * e] = h2f(uint16_t(r4[e] & 0xffffu));
        wv[p][2 * e + 1] = h2f(uint16_t(r4[e] >> 16));
      }
    } else if (vi < nv) {
      const f32x4* pp = reinterpret_cast<const f32x4*>(bk + (size_t)(vi - rank) * kD + 8 * n);
      const f32x4 x0 = pp[0], x1 = pp[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wv[p][e] = x0[e];
        wv[p][4 + e] = x1[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[p][e] = kx[e];   // k itself (vi == nv) or unused
    }
  }
  const float b = beta[head];
  // GDN: one decay per head; KDA: this lane's channels of the per-channel decay
  float a = 0.f, ax[8];
  if constexpr (KDA) {
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(alpha + hk + 8 * n);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(alpha + hk + 8 * n + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ax[e] = a0[e];
      ax[4 + e] = a1[e];
    }
  } else {
    a = alpha[head];
  }

  // ---- decays, appends
  if constexpr (KDA) {
    if (tid < kD)   // suffix products of channel tid's buffered decays
      suffix_products(buf_a + (size_t)head * window * kD + tid, kD, m,
                      [&](int j, float x) { s_gv[j][tid] = x; });
    lds_barrier();
  } else {
    if (tid == 0)   // suffix products of the buffered decays
      suffix_products(ba, 1, m, [&](int j, float x) { s_g[j] = x; });
  }
  // KDA: the vectors the state is applied to are yk = a o k, yq = a o q; the
  // compensators and the stored residual see them decayed by G0, record j by G_j
  float g0x[8], yk8[8], yq8[8];
  if constexpr (KDA) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      g0x[e] = s_gv[m][8 * n + e];
      yk8[e] = ax[e] * kx[e];
      yq8[e] = ax[e] * qx[e];
    }
  }

  // ---- per-head dot products
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int vi = 4 * w + g + 16 * p;
    if (vi <= nv) {
      float pk = 0.f, pq = 0.f;
      if (KDA && vi < nv) {   // (decayed a o k) . key of the compensator or record
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = vi < rank ? g0x[e] : s_gv[vi - rank][8 * n + e];
          pk += wv[p][e] * (d * yk8[e]);
          pq += wv[p][e] * (d * yq8[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pk += wv[p][e] * kx[e];
          pq += wv[p][e] * qx[e];
        }
      }
      pk = sum16(pk);
      pq = sum16(pq);
      if (n == 0) {
        s_dk[vi] = pk;
        s_dq[vi] = pq;
      }
    }
  }

  // ---- read vectors as fixed-point digits (every row of 16 lanes holds all 128
  // channels; row 0 of the wave writes the wave's copy)
  int ek, eq;
  {
    float xk[8], xq[8], mk = 0.f, mq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (KDA) {
        xk[e] = cx[e] * (g0x[e] * yk8[e]);
        xq[e] = cx[e] * (g0x[e] * yq8[e]);
      } else {
        xk[e] = cx[e] * kx[e];
        xq[e] = cx[e] * qx[e];
      }
      mk = fmaxf(mk, fabsf(xk[e]));
      mq = fmaxf(mq, fabsf(xq[e]));
    }
    mk = max16(mk);
    mq = max16(mq);
    uint2 dk3[3], dq3[3];
    ek = fixed_digits(xk, mk, dk3);
    eq = fixed_digits(xq, mq, dq3);
    if (g == 0) {
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        s_dig[w][t][n] = dk3[t];
        s_dig[w][3 + t][n] = dq3[t];
      }
      s_dig[w][6][n] = make_uint2(0, 0);
      s_dig[w][7][n] = make_uint2(0, 0);
    }
  }
  wave_lds_sync();

  // ---- Z x on the int8 matrix cores: A = digit rows (M), B = code rows (N): row
  // 32 w + 16 T + n, bytes 64 s + 16 g, from the wave's own LDS copy (complete once the
  // wave's vector memory operations are: the compiler does not order LDS reads after LDS
  // DMA, and before this point the wave has issued no stores)
  i32x4 zb[2][2];
  if constexpr (PK == 8) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int r = row[T], c = 4 * s + g;
        zb[T][s] = *reinterpret_cast<const i32x4*>(s_codes + r * kD + 16 * (c ^ ((r >> 1) & 7)));
      }
  } else {
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint32_t u[4];
        if constexpr (PK == 4) {
          unpack4(zp[T][s][0], u[0], u[1]);
          unpack4(zp[T][s][1], u[2], u[3]);
        } else {
          unpack6x16(zp[T][s][0], zp[T][s][1], zp[T][s][2], u);
        }
        zb[T][s] = i32x4{(int)u[0], (int)u[1], (int)u[2], (int)u[3]};
      }
  }
  i32x4 acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    i32x4 ad = {0, 0, 0, 0};
    if (n < 8) ad = *reinterpret_cast<const i32x4*>(&s_dig[w][n][8 * s + 2 * g]);
#pragma unroll
    for (int T = 0; T < 2; ++T) acc[T] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ad, zb[T][s], acc[T], 0, 0, 0);
  }
  // lane (n, 0) holds digits 0-3 of row 16 T + n, lane (n, 1) digits 4-7
  float yk[2], yq[2];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const int t4 = __shfl_xor(acc[T][0], 16), t5 = __shfl_xor(acc[T][1], 16);
    yk[T] = ldexpf(((float)acc[T][0] * 65536.0f + (float)acc[T][1] * 256.0f) + (float)acc[T][2], ek - 22);
    yq[T] = ldexpf(((float)acc[T][3] * 65536.0f + (float)t4 * 256.0f) + (float)t5, eq - 22);
  }
  lds_barrier();

  // ---- rows: compensator and buffered terms (slots = g mod 4), summed over the
  // four lanes of a row, then lane (n, 0) finishes rows 32 w + 16 T + n
  const float g0 = KDA ? 1.f : s_g[m];
  const float kq = s_dq[nv];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    float ck = 0.f, cq = 0.f, tk = 0.f, tq = 0.f;
#pragma unroll
    for (int rr = 0; rr < kMaxRank / 4; ++rr) {
      const int r = 4 * rr + g;
      if (r < rank) {
        ck += cur[T][rr] * s_dk[r];
        cq += cur[T][rr] * s_dq[r];
      }
    }
#pragma unroll
    for (int jj = 0; jj < kMaxWindow / 4; ++jj) {
      const int j = 4 * jj + g;
      if (j < m) {
        const float wj = KDA ? bur[T][jj] : s_g[j] * bur[T][jj];
        tk += wj * s_dk[rank + j];
        tq += wj * s_dq[rank + j];
      }
    }
    ck += __shfl_xor(ck, 16); cq += __shfl_xor(cq, 16); tk += __shfl_xor(tk, 16); tq += __shfl_xor(tq, 16);
    ck += __shfl_xor(ck, 32); cq += __shfl_xor(cq, 32); tk += __shfl_xor(tk, 32); tq += __shfl_xor(tq, 32);
    if (g == 0) {
      const float sv = vsr[T] * qinv;   // 1 / Q, Q = 127 at 8 bits
      const float Sk = g0 * (sv * yk[T] + ck) + tk;
      const float Sq = g0 * (sv * yq[T] + cq) + tq;
      const float u = KDA ? b * (vrow[T] - Sk) : b * (vrow[T] - a * Sk);
      const float oi = KDA ? Sq + u * kq : a * Sq + u * kq;
      bu[(size_t)m * kD + row[T]] = u;
      io_traits<IO>::st(o, hk + row[T], oi);
    }
  }
  // ---- this token's record m: its key, and its decay (GDN: one per head; KDA: per channel)
  if (w == 0 && g == 0) {
    f32x4* dst = reinterpret_cast<f32x4*>(bk + (size_t)m * kD + 8 * n);
    dst[0] = f32x4{kx[0], kx[1], kx[2], kx[3]};
    dst[1] = f32x4{kx[4], kx[5], kx[6], kx[7]};
    if constexpr (KDA) {
      f32x4* da = reinterpret_cast<f32x4*>(buf_a + ((size_t)head * window + m) * kD + 8 * n);
      da[0] = f32x4{ax[0], ax[1], ax[2], ax[3]};
      da[1] = f32x4{ax[4], ax[5], ax[6], ax[7]};
    } else if (n == 0) {
      buf_a[(size_t)head * window + m] = a;
    }
  }
}

// ============================================================== window flush
//
// One block of 256 threads (four waves) per head; the dense 128 x 128 state stays in
// fp32 MFMA accumulators from the rebuild to the codes. Wave w holds value rows
// [32 w, 32 w + 32) as two tiles t of 16 rows; lane (n = lane % 16, g = lane / 16)
// holds rows 32 w + 16 t + n and the 32 contiguous key channels [32 g, 32 g + 32):
// register e of accumulator tile (t, tc) is S[32 w + 16 t + n][32 g + 4 tc + e].
// For v_mfma_f32_16x16x4f32 the tile (t, tc) is the block D = S^T with its rows
// (key channels) permuted: D row i of tile tc is channel 32 (i / 4) + 4 tc + i % 4.
//
//  * rebuild (eq. 4): D starts as the decayed dequantised residual, then the
//    compensators and buffered records, four rank-one terms per MFMA:
//    A[i][k] = key of term k at channel i, B[k][j] = coefficient x value vector;
//  * compensator fit (eq. 5, subspace iteration with CholeskyQR2): Y = S Q is
//    summed within a lane over its 32 channels and across the four lanes of a
//    row; S^T Y within a lane over its two rows, across the 16 lanes of a DPP
//    row by a reduce-scatter, and across the four waves through LDS; one wave
//    orthonormalises in fp64;
//  * residual, smoothing factors (eq. 7), value-channel scales and codes, each
//    lane writing its 32 codes of a row as two 16-byte stores.

constexpr int kFlushNT = 256;
constexpr int kRP = kD + 16;   // fp32 pitch of staged rank-one rows: the rows read by the
                               // two half-waves of an MFMA operand load fall in other banks
constexpr int kMaxTerms = kMaxRank + kMaxWindow;

template <int RQ>
struct alignas(16) FlushSmem {
  union {
    struct {
      float K[kMaxTerms * kRP];   // term keys, channels permuted as the D rows of a tile
      float U[kMaxTerms * kRP];   // term value vectors
    } rb;
    float red[4 * kD * RQ];       // per-wave partial S^T Y, [wave][channel][r]
  } u;
  float Q[kD * RQ];               // subspace block, [channel][r] (r >= rank: zero)
  float Kh[kD * RQ];              // fp16-rounded compensator keys, [channel][r]
  float col[kD];                  // stored smoothing factors, then 1 / the new ones
  float cred[4 * kD];             // per-wave column statistics
  float dec[kMaxWindow + 1];      // dec[j] = G_j for j < m, dec[m] = G0
};

// KDA: the decays per key channel, gv[j][c] = prod_{j<i<m} a_i[c], gv[m] = G0
template <bool KDA>
struct alignas(16) FlushDecays {
  float gv[kMaxWindow + 1][kD];
};
template <>
struct alignas(16) FlushDecays<false> {   // Gated DeltaNet: scalar decays (FlushSmem::dec)
  float gv[1][4];
};

// fp32 16 x 16 x 4 MFMA: lane l holds A[l%16][l/16], B[l/16][l%16]; D[4(l/16)+e][l%16]
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One halving step of a reduce-scatter inside a 16-lane DPP row: x[0, M) becomes
// x[0, M/2), the half selected by `upper`, plus the partner lane's copy of that half.
// The partner (DPP control CTRL) differs from this lane in the bit that sets `upper`.
template <int M, int CTRL>
__device__ __forceinline__ void rs_step(float* x, bool upper) {
#pragma unroll
  for (int i = 0; i < M / 2; ++i) {
    const float keep = upper ? x[M / 2 + i] : x[i];
    const float give = upper ? x[i] : x[M / 2 + i];
    x[i] = keep + dpp<CTRL>(give);
  }
}

// Reduce-scatter over the 16 lanes of a DPP row: on entry each lane holds NV values;
// on return lane n holds, in x[0, NV/16), the row sums of values [n NV/16, (n+1) NV/16).
// Partners: row_ror:8 (n ^ 8), row_half_mirror (7 - n within 8: bit 2 differs),
// quad_perm(3,2,1,0) (bit 1 differs), quad_perm(1,0,3,2) (n ^ 1).
template <int NV>
__device__ __forceinline__ void reduce_scatter16(float (&x)[NV], int n) {
  static_assert(NV >= 16 && NV % 16 == 0, "16 lanes");
  rs_step<NV, 0x128>(x, n & 8);
  rs_step<NV / 2, 0x141>(x, n & 4);
  rs_step<NV / 4, 0x1B>(x, n & 2);
  rs_step<NV / 8, 0xB1>(x, n & 1);
}

// lane-to-lane move within a wave: value of lane (lane ^ M)
__device__ __forceinline__ float xor_lane(float x, int m) { return __shfl_xor(x, m); }

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
// DPP move of an fp64 value with a row mask: rows outside ROWS read zero
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp64_rows(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWS, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROWS, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// sum over the 64 lanes of a wave, fp64 (wave-uniform): within rows of 16 by DPP (every
// lane then holds its row's total), rows 1 and 3 add the totals of rows 0 and 2
// (row_bcast:15), rows 2 and 3 that of rows 0-1 (row_bcast:31); lane 63 holds the sum
__device__ __forceinline__ double wave_sum_f64(double x) {
  x += dpp64<0x140>(x);
  x += dpp64<0x141>(x);
  x += dpp64<0x4E>(x);
  x += dpp64<0xB1>(x);
  x += dpp64_rows<0x142, 0xA>(x);
  x += dpp64_rows<0x143, 0xC>(x);
  return lane64(x, 63);
}

// CholeskyQR2 of a 128 x RANK block held by one wave, rows lane and lane + 64:
// twice x <- x L^{-T} with L L^T = x^T x + (1e-6 tr + 1e-30) I. The fit is
// ill-conditioned on states with outlier channels, so the Gram matrix, the factor
// and the solve are fp64 (products of fp32 values are exact there).
template <int RANK>
__device__ __forceinline__ void cholqr2_wave(float (&x)[2][RANK]) {
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    double G[RANK][RANK];
#pragma unroll
    for (int i = 0; i < RANK; ++i)
#pragma unroll
      for (int j = i; j < RANK; ++j)
        G[i][j] = wave_sum_f64((double)x[0][i] * (double)x[0][j] + (double)x[1][i] * (double)x[1][j]);
    double tr = 0.0;
#pragma unroll
    for (int i = 0; i < RANK; ++i) tr += G[i][i];
    const double sh = 1e-6 * tr + 1e-30;
    double L[RANK * (RANK + 1) / 2], rd[RANK];   // L[i][j] at i (i + 1) / 2 + j
#pragma unroll
    for (int i = 0; i < RANK; ++i) {
#pragma unroll
      for (int j = 0; j <= i; ++j) {
        double s = G[j][i] + (i == j ? sh : 0.0);
#pragma unroll
        for (int p = 0; p < j; ++p) s -= L[i * (i + 1) / 2 + p] * L[j * (j + 1) / 2 + p];
        if (i == j) {
          // 1 / sqrt(s) from the hardware estimate and two Newton steps (each squares
          // the relative error), instead of a square root and a division
          double r = __builtin_amdgcn_rsq(s);
          r = r * (1.5 - 0.5 * s * r * r);
          r = r * (1.5 - 0.5 * s * r * r);
          const bool pos = s > 0.0;
          L[i * (i + 1) / 2 + i] = pos ? s * r : 0.0;
          rd[i] = pos ? r : __builtin_inf();
        } else {
          L[i * (i + 1) / 2 + j] = s * rd[j];
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      double y[RANK];
#pragma unroll
      for (int j = 0; j < RANK; ++j) {
        double s = x[h][j];
#pragma unroll
        for (int p = 0; p < j; ++p) s -= y[p] * L[j * (j + 1) / 2 + p];
        y[j] = s * rd[j];
      }
#pragma unroll
      for (int j = 0; j < RANK; ++j) x[h][j] = (float)y[j];
    }
  }
}

// four consecutive floats of LDS as a vector (16-byte aligned)
__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// The token of the window's last position, decoded inside the flush.
// io: GDNRT_F32 or GDNRT_BF16 for q, k, v, o.
struct FlushToken {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  void* o;
  int io;
};

__device__ __forceinline__ float ld_io(const void* p, size_t i, int io) {
  return io == GDNRT_F32 ? static_cast<const float*>(p)[i] : bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <int RANK, bool KDA, bool TOK>
__global__ __launch_bounds__(kFlushNT) __attribute__((amdgpu_waves_per_eu(RANK <= 4 && !TOK ? 4 : RANK <= 5 ? 3 : 2))) void leapq_flush_kernel(
    int8_t* __restrict__ codes, float* __restrict__ vscale, float* __restrict__ ksmooth,
    uint16_t* __restrict__ ct_k, uint16_t* __restrict__ ct_u, const float* __restrict__ buf_k,
    const float* __restrict__ buf_u, const float* __restrict__ buf_a, int window, int m,
    const float* __restrict__ dense, const float* __restrict__ q0, int iters, int smooth_mode,
    float qf, float qinv, float* __restrict__ pre_round, FlushToken tok, int pk) {
  constexpr int RQ = RANK <= 4 ? 4 : 8;   // padded rank of the LDS blocks
  __shared__ FlushSmem<RQ> sm;
  __shared__ FlushDecays<KDA> dk_[1];
  // TOK: the token's k, q, decays and v (kD each), then beta
  __shared__ __attribute__((aligned(16))) float s_tok[TOK ? 4 * kD + 4 : 4];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int head = blockIdx.x;
  const size_t hk = (size_t)head * kD;
  const int vrow[2] = {32 * w + n, 32 * w + 16 + n};
  f32x4 acc[2][8];

  // ---------------------------------------------------------------- inputs
  if constexpr (RANK > 0) {
    float qs[kD * RQ / kFlushNT];   // all requested before the first is stored
#pragma unroll
    for (int it = 0; it < kD * RQ / kFlushNT; ++it) {
      const int i = tid + kFlushNT * it, c = i / RQ, r = i % RQ;
      qs[it] = r < RANK ? q0[c * RANK + r] : 0.f;
    }
#pragma unroll
    for (int it = 0; it < kD * RQ / kFlushNT; ++it) sm.Q[tid + kFlushNT * it] = qs[it];
  }
  const int nt = dense ? 0 : RANK + m;   // rank-one terms of the rebuild
  const int ns = (nt + 3) >> 2;          // MFMA steps of four terms
  uint4 z[2][2];   // the lane's 32 codes of each row: 32, 16 or 24 bytes as stored (pk)
  float vs[2];
  const int RB = row_bytes(pk);
  if constexpr (TOK) {
    if (tid < kD) {
      s_tok[tid] = ld_io(tok.k, hk + tid, tok.io);
      s_tok[kD + tid] = ld_io(tok.q, hk + tid, tok.io);
      s_tok[2 * kD + tid] = KDA ? tok.alpha[hk + tid] : tok.alpha[head];
    } else {
      s_tok[3 * kD + tid - kD] = ld_io(tok.v, hk + tid - kD, tok.io);
      if (tid == kD) s_tok[4 * kD] = tok.beta[head];
    }
  }
  if (dense) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int tc = 0; tc < 8; ++tc)
        acc[t][tc] = *reinterpret_cast<const f32x4*>(dense + (hk + vrow[t]) * kD + 32 * g + 4 * tc);
  } else {
    // every input of the rebuild is requested before the one wait
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int8_t* zr = codes + (hk + vrow[t]) * RB + 4 * pk * g;
      if (pk == 8) {
        z[t][0] = reinterpret_cast<const uint4*>(zr)[0];
        z[t][1] = reinterpret_cast<const uint4*>(zr)[1];
      } else if (pk == 4) {
        z[t][0] = *reinterpret_cast<const uint4*>(zr);
      } else {   // 24 bytes, 8-byte aligned
        const uint2 a = reinterpret_cast<const uint2*>(zr)[0], b = reinterpret_cast<const uint2*>(zr)[1],
                    c = reinterpret_cast<const uint2*>(zr)[2];
        z[t][0] = make_uint4(a.x, a.y, b.x, b.y);
        z[t][1] = make_uint4(c.x, c.y, 0u, 0u);
      }
      vs[t] = vscale[hk + vrow[t]];
    }
    // term rows (compensators, then records; zero up to a multiple of four): piece q
    // of a row is channels [4 q, 4 q + 4); keys go to D-row order, values as they are.
    // At most three pieces per thread (24 rows of 32 pieces over 256 threads).
    f32x4 kk[3], uu[3];
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const int idx = tid + kFlushNT * it, j = idx >> 5, q = idx & 31;
      kk[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      uu[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j < RANK) {
        const uint2 hk4 = *reinterpret_cast<const uint2*>(ct_k + ((size_t)head * RANK + j) * kD + 4 * q);
        const uint2 hu4 = *reinterpret_cast<const uint2*>(ct_u + ((size_t)head * RANK + j) * kD + 4 * q);
        kk[it] = f32x4{h2f(uint16_t(hk4.x)), h2f(uint16_t(hk4.x >> 16)), h2f(uint16_t(hk4.y)), h2f(uint16_t(hk4.y >> 16))};
        uu[it] = f32x4{h2f(uint16_t(hu4.x)), h2f(uint16_t(hu4.x >> 16)), h2f(uint16_t(hu4.y)), h2f(uint16_t(hu4.y >> 16))};
      } else if (j < nt) {
        const size_t off = ((size_t)head * window + (j - RANK)) * kD + 4 * q;
        kk[it] = *reinterpret_cast<const f32x4*>(buf_k + off);
        uu[it] = *reinterpret_cast<const f32x4*>(buf_u + off);
      }
    }
    if constexpr (KDA) {
      // suffix products of channel tid's buffered decays, newest first; the stored
      // residual's smoothing factors carry G0, so the dequantised term decays with it
      if (tid < kD) {
        suffix_products(buf_a + (size_t)head * window * kD + tid, kD, m,
                        [&](int j, float x) { dk_[0].gv[j][tid] = x; });
        sm.col[tid] = ksmooth[hk + tid] * dk_[0].gv[m][tid];
      }
      if (tid == 0) {
#pragma unroll
        for (int j = 0; j <= kMaxWindow; ++j) sm.dec[j] = 1.f;
      }
      lds_barrier();
    } else {
      if (tid < kD) sm.col[tid] = ksmooth[hk + tid];
      if (tid == 0)   // suffix products of the buffered decays
        suffix_products(buf_a + (size_t)head * window, 1, m, [&](int j, float x) { sm.dec[j] = x; });
    }
#pragma unroll
    for (int it = 0; it < 3; ++it) {
      const int idx = tid + kFlushNT * it, j = idx >> 5, q = idx & 31;
      if (idx < ns * 4 * 32) {
        f32x4 kv = kk[it];
        if constexpr (KDA) {   // KDA: the key of a term carries its decay (G0 for compensators)
          if (j < nt) kv *= *reinterpret_cast<const f32x4*>(&dk_[0].gv[j < RANK ? m : j - RANK][4 * q]);
        }
        *reinterpret_cast<f32x4*>(sm.u.rb.K + j * kRP + 16 * (q & 7) + 4 * (q >> 3)) = kv;
        *reinterpret_cast<f32x4*>(sm.u.rb.U + j * kRP + 4 * q) = uu[it];
      }
    }
  }
  lds_barrier();

  // ---------------------------------------------------------------- rebuild
  if (!dense) {
    const float g0 = sm.dec[m];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float sv = g0 * vs[t] * qinv;
      uint32_t zw[8] = {z[t][0].x, z[t][0].y, z[t][0].z, z[t][0].w, z[t][1].x, z[t][1].y, z[t][1].z, z[t][1].w};
      if (pk == 4) {
        const uint4 p4 = z[t][0];
        unpack4(p4.x, zw[0], zw[1]);
        unpack4(p4.y, zw[2], zw[3]);
        unpack4(p4.z, zw[4], zw[5]);
        unpack4(p4.w, zw[6], zw[7]);
      } else if (pk == 6) {
        uint32_t u[4];
        const uint4 a = z[t][0], b = z[t][1];
        unpack6x16(a.x, a.y, a.z, u);
        zw[0] = u[0]; zw[1] = u[1]; zw[2] = u[2]; zw[3] = u[3];
        unpack6x16(a.w, b.x, b.y, u);
        zw[4] = u[0]; zw[5] = u[1]; zw[6] = u[2]; zw[7] = u[3];
      }
#pragma unroll
      for (int tc = 0; tc < 8; ++tc) {
        const f32x4 cc = lds4(sm.col + 32 * g + 4 * tc);
        acc[t][tc] = f32x4{sv * sb(zw[tc], 0) * cc.x, sv * sb(zw[tc], 1) * cc.y,
                           sv * sb(zw[tc], 2) * cc.z, sv * sb(zw[tc], 3) * cc.w};
      }
    }
    for (int s = 0; s < ns; ++s) {
      const int j = 4 * s + g;   // this lane's term (the k index of its A and B entries)
      const float cj = j < RANK ? g0 : (j < nt ? sm.dec[j - RANK] : 0.f);
      const float b0 = cj * sm.u.rb.U[j * kRP + 32 * w + n];
      const float b1 = cj * sm.u.rb.U[j * kRP + 32 * w + 16 + n];
#pragma unroll
      for (int tc = 0; tc < 8; ++tc) {
        const float a = sm.u.rb.K[j * kRP + 16 * tc + n];
        acc[0][tc] = mfma4(a, b0, acc[0][tc]);
        acc[1][tc] = mfma4(a, b1, acc[1][tc]);
      }
    }
  }

  // ---------------------------------------------------------------- the window's last token
  // With m = window - 1 records rebuilt, acc holds S_m. The token is decoded from it
  // (eq. 3 with the decay a = alpha on every key channel, or the KDA decay vector):
  //   u = beta (v - S_m (a o k)),  o = S_m (a o q) + u (k . q),  S <- S_m Diag(a) + u k^T,
  // the same step the decode kernel takes through eq. 10, and the flush goes on from S.
  if constexpr (TOK) {
    const float* s_tk = s_tok;
    const float* s_tq = s_tok + kD;
    const float* s_ta = s_tok + 2 * kD;
    const float tb = s_tok[4 * kD];
    float sk[2] = {0.f, 0.f}, sq[2] = {0.f, 0.f}, kq = 0.f;
#pragma unroll
    for (int tc = 0; tc < 8; ++tc) {
      const f32x4 k4 = lds4(s_tk + 32 * g + 4 * tc), q4 = lds4(s_tq + 32 * g + 4 * tc);
      const f32x4 a4 = lds4(s_ta + 32 * g + 4 * tc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ak = a4[e] * k4[e], aq = a4[e] * q4[e];
        kq += k4[e] * q4[e];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          sk[t] += acc[t][tc][e] * ak;
          sq[t] += acc[t][tc][e] * aq;
        }
      }
    }
    kq += xor_lane(kq, 16);
    kq += xor_lane(kq, 32);
    float u[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sk[t] += xor_lane(sk[t], 16);
      sk[t] += xor_lane(sk[t], 32);
      sq[t] += xor_lane(sq[t], 16);
      sq[t] += xor_lane(sq[t], 32);
      u[t] = tb * (s_tok[3 * kD + vrow[t]] - sk[t]);
      if (g == 0) {
        const float oi = sq[t] + u[t] * kq;
        if (tok.io == GDNRT_F32) static_cast<float*>(tok.o)[hk + vrow[t]] = oi;
        else static_cast<uint16_t*>(tok.o)[hk + vrow[t]] = f32_to_bf16(oi);
      }
    }
#pragma unroll
    for (int tc = 0; tc < 8; ++tc) {
      const f32x4 k4 = lds4(s_tk + 32 * g + 4 * tc), a4 = lds4(s_ta + 32 * g + 4 * tc);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][tc][e] = fmaf(acc[t][tc][e], a4[e], u[t] * k4[e]);
    }
  }

  // ---------------------------------------------------------------- compensators
  if constexpr (RANK > 0) {
    lds_barrier();   // the term rows share LDS with the S^T Y partials
    float y[2][RANK];
    for (int it = 0;; ++it) {
      // Y = S Q: this lane's 32 channels, then the four lanes of the row
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < RANK; ++r) y[t][r] = 0.f;
#pragma unroll
      for (int tc = 0; tc < 8; ++tc)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float qv[RQ];
#pragma unroll
          for (int r4 = 0; r4 < RQ / 4; ++r4) {
            const f32x4 q4 = lds4(sm.Q + (32 * g + 4 * tc + e) * RQ + 4 * r4);
            qv[4 * r4] = q4.x; qv[4 * r4 + 1] = q4.y; qv[4 * r4 + 2] = q4.z; qv[4 * r4 + 3] = q4.w;
          }
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < RANK; ++r) y[t][r] += acc[t][tc][e] * qv[r];
        }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < RANK; ++r) {
          y[t][r] += xor_lane(y[t][r], 16);
          y[t][r] += xor_lane(y[t][r], 32);
        }
      if (it == iters) break;   // final Y = S Q: the compensator values
      // S^T Y: this lane's two rows, then the 16 rows of the DPP row, then the waves
#pragma unroll
      for (int tc = 0; tc < 8; ++tc) {
        float p[4 * RQ];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int r = 0; r < RANK; ++r) p[e * RQ + r] = acc[0][tc][e] * y[0][r] + acc[1][tc][e] * y[1][r];
#pragma unroll
          for (int r = RANK; r < RQ; ++r) p[e * RQ + r] = 0.f;
        }
        reduce_scatter16<4 * RQ>(p, n);
        float* dst = sm.u.red + w * kD * RQ + (32 * g + 4 * tc) * RQ + n * (RQ / 4);
#pragma unroll
        for (int k2 = 0; k2 < RQ / 4; ++k2) dst[k2] = p[k2];
      }
      lds_barrier();
      if (w == 0) {
        float x[2][RANK];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < RANK; ++r) {
            const int o = (lane + 64 * h) * RQ + r;
            x[h][r] = (sm.u.red[o] + sm.u.red[kD * RQ + o]) + (sm.u.red[2 * kD * RQ + o] + sm.u.red[3 * kD * RQ + o]);
          }
        cholqr2_wave<RANK>(x);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < RANK; ++r) sm.Q[(lane + 64 * h) * RQ + r] = x[h][r];
      }
      lds_barrier();
    }
    // fp16 pieces: stored, and their rounded values kept for the residual
    float yh[2][RANK];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < RANK; ++r) {
        const uint16_t hy = f2h(y[t][r]);
        yh[t][r] = h2f(hy);
        if (g == 0) ct_u[((size_t)head * RANK + r) * kD + vrow[t]] = hy;
      }
    if (tid < kD) {
#pragma unroll
      for (int r = 0; r < RQ; ++r) {
        float kh = 0.f;
        if (r < RANK) {
          const uint16_t hq = f2h(sm.Q[tid * RQ + r]);
          ct_k[((size_t)head * RANK + r) * kD + tid] = hq;
          kh = h2f(hq);
        }
        sm.Kh[tid * RQ + r] = kh;
      }
    }
    lds_barrier();
    // residual R = S - sum_r uh_r kh_r^T
#pragma unroll
    for (int tc = 0; tc < 8; ++tc)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float kv[RQ];
#pragma unroll
        for (int r4 = 0; r4 < RQ / 4; ++r4) {
          const f32x4 k4 = lds4(sm.Kh + (32 * g + 4 * tc + e) * RQ + 4 * r4);
          kv[4 * r4] = k4.x; kv[4 * r4 + 1] = k4.y; kv[4 * r4 + 2] = k4.z; kv[4 * r4 + 3] = k4.w;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < RANK; ++r) acc[t][tc][e] -= yh[t][r] * kv[r];
      }
  }

  // ---------------------------------------------------------------- smoothing
  if (smooth_mode != 2) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {   // channels 32 g + 16 hf + [0, 16)
      float cs[16];
#pragma unroll
      for (int tc = 0; tc < 4; ++tc)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a0 = acc[0][4 * hf + tc][e], a1 = acc[1][4 * hf + tc][e];
          cs[4 * tc + e] = smooth_mode == 1 ? a0 * a0 + a1 * a1 : fabsf(a0) + fabsf(a1);
        }
      reduce_scatter16<16>(cs, n);   // lane n: channel 32 g + 16 hf + n
      sm.cred[w * kD + 32 * g + 16 * hf + n] = cs[0];
    }
  }
  lds_barrier();
  if (tid < kD) {
    float cf = 1.f;
    if (smooth_mode != 2) {
      const float tot = (sm.cred[tid] + sm.cred[kD + tid]) + (sm.cred[2 * kD + tid] + sm.cred[3 * kD + tid]);
      cf = fmaxf(sqrtf(tot * (1.0f / kD)), 1e-12f);
    }
    ksmooth[hk + tid] = cf;
    sm.col[tid] = 1.0f / cf;
  }
  lds_barrier();

  // ---------------------------------------------------------------- scales, codes
#pragma unroll
  for (int tc = 0; tc < 8; ++tc) {
    const f32x4 cc = lds4(sm.col + 32 * g + 4 * tc);
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[t][tc] *= cc;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float mx = 0.f;
#pragma unroll
    for (int tc = 0; tc < 8; ++tc)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(acc[t][tc][e]));
    mx = fmaxf(mx, xor_lane(mx, 16));
    mx = fmaxf(mx, xor_lane(mx, 32));
    if (g == 0) vscale[hk + vrow[t]] = mx;
    const float sc = mx > 0.f ? qf / mx : 0.f;   // Q / max, Q = 2^(bits-1) - 1
    uint32_t wd[8];
#pragma unroll
    for (int tc = 0; tc < 8; ++tc) {
      const f32x4 x = acc[t][tc] * sc;
      if (pre_round) *reinterpret_cast<f32x4*>(pre_round + (hk + vrow[t]) * kD + 32 * g + 4 * tc) = x;
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float qz = fminf(fmaxf(rintf(x[e]), -qf), qf);
        word |= (uint32_t)((int32_t)qz & 0xff) << (8 * e);
      }
      wd[tc] = word;
    }
    int8_t* zo = codes + (hk + vrow[t]) * RB + 4 * pk * g;
    if (pk == 8) {
      reinterpret_cast<uint4*>(zo)[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      reinterpret_cast<uint4*>(zo)[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
    } else if (pk == 4) {
      *reinterpret_cast<uint4*>(zo) =
          make_uint4(pack4(wd[0], wd[1]), pack4(wd[2], wd[3]), pack4(wd[4], wd[5]), pack4(wd[6], wd[7]));
    } else {   // eight 24-bit groups -> six words
      uint32_t gr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) gr[i] = pack6(wd[i]);
      uint2* zo2 = reinterpret_cast<uint2*>(zo);
      zo2[0] = make_uint2(gr[0] | (gr[1] << 24), (gr[1] >> 8) | (gr[2] << 16));
      zo2[1] = make_uint2((gr[2] >> 16) | (gr[3] << 8), gr[4] | (gr[5] << 24));
      zo2[2] = make_uint2((gr[5] >> 8) | (gr[6] << 16), (gr[6] >> 16) | (gr[7] << 8));
    }
  }
}

// largest code of the state's grid: 2^(bits-1) - 1, bits = 0 meaning 8
static int code_max(const leapq_state* st) { return (1 << ((st->bits ? st->bits : 8) - 1)) - 1; }
// code width in memory: 4 and 6 bits are packed, every other width takes a byte
static int packing(const leapq_state* st) { return st->bits == 4 || st->bits == 6 ? st->bits : 8; }
// bytes of the stored codes of all heads
static size_t code_bytes(const leapq_state* st) { return (size_t)st->N * kD * row_bytes(packing(st)); }

static int check_state(const leapq_state* st, const char* fn) {
  if (!st) return set_error(GDNRT_EINVAL, "%s: null state", fn);
  if (st->dk != kD || st->dv != kD)
    return set_error(GDNRT_ESHAPE, "%s: d_k=%d d_v=%d, only 128 is supported", fn, st->dk, st->dv);
  if (st->N < 0) return set_error(GDNRT_ESHAPE, "%s: N=%d", fn, st->N);
  if (st->rank < 0 || st->rank > kMaxRank)
    return set_error(GDNRT_ESHAPE, "%s: rank=%d must be in [0, %d]", fn, st->rank, kMaxRank);
  if (st->window < 1 || st->window > kMaxWindow)
    return set_error(GDNRT_ESHAPE, "%s: window=%d must be in [1, %d]", fn, st->window, kMaxWindow);
  if (st->bits != 0 && (st->bits < 2 || st->bits > 8))
    return set_error(GDNRT_ESHAPE, "%s: bits=%d must be 0 (8) or in [2, 8]", fn, st->bits);
  if ((size_t)st->N * 4 > 0x7fffffffu) return set_error(GDNRT_ESHAPE, "%s: N too large", fn);
  if (st->N == 0) return GDNRT_OK;
  if (!st->codes || !st->vscale || !st->ksmooth || !st->buf_k || !st->buf_u || !st->buf_a ||
      (st->rank > 0 && (!st->ct_k || !st->ct_u)))
    return set_error(GDNRT_EINVAL, "%s: null buffer in leapq_state", fn);
  if (!aligned16(st->codes) || !aligned16(st->buf_k) || !aligned16(st->buf_u) ||
      !aligned4(st->vscale) || !aligned16(st->ksmooth) || !aligned4(st->buf_a) ||
      (st->rank > 0 && (!aligned16(st->ct_k) || !aligned16(st->ct_u))))
    return set_error(GDNRT_EALIGN, "%s: codes, ksmooth, buf_k, buf_u, ct_k, ct_u must be 16-byte aligned", fn);
  return GDNRT_OK;
}

}  // namespace gdnrt

using namespace gdnrt;

namespace {

template <bool KDA>
int decode_step(const char* fn, const leapq_state* st, int pos, const void* q, const void* k,
                const void* v, const float* alpha, const float* beta, void* o, int io, void* stream) {
  int rc = check_state(st, fn);
  if (rc != GDNRT_OK) return rc;
  if (io != GDNRT_F32 && io != GDNRT_BF16) return set_error(GDNRT_EDTYPE, "%s: io=%d", fn, io);
  if (pos < 0 || pos >= st->window)
    return set_error(GDNRT_ESTATE, "%s: pos=%d outside [0, window=%d)", fn, pos, st->window);
  if (st->N == 0) return clear_error();
  if (!q || !k || !v || !alpha || !beta || !o) return set_error(GDNRT_EINVAL, "%s: null pointer argument", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned4(v) || !aligned4(o) || !aligned4(beta) ||
      (KDA ? !aligned16(alpha) : !aligned4(alpha)))
    return set_error(GDNRT_EALIGN, KDA ? "%s: q, k, alpha must be 16-byte aligned, v, o, beta 4-byte"
                                       : "%s: q, k must be 16-byte aligned, v, o, alpha, beta 4-byte", fn);
  const size_t es = io == GDNRT_F32 ? 4 : 2;
  const size_t N = st->N, nIO = N * kD * es, nB = N * st->window * kD * 4;
  if (overlaps(o, nIO, q, nIO) || overlaps(o, nIO, k, nIO) || overlaps(o, nIO, v, nIO) ||
      overlaps(o, nIO, st->buf_k, nB) || overlaps(o, nIO, st->buf_u, nB) ||
      overlaps(o, nIO, st->codes, code_bytes(st)))
    return set_error(GDNRT_EINVAL, "%s: o overlaps another buffer", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)N), block(256);
  const float qinv = 1.0f / (float)code_max(st);
#define GDNRT_DECODE(IOT, PKV)                                                                        \
  hipLaunchKernelGGL((leapq_decode_kernel<IOT, KDA, PKV>), grid, block, 0, s, st->codes, st->vscale,   \
                     st->ksmooth, st->ct_k, st->ct_u, st->buf_k, st->buf_u, st->buf_a, st->rank,       \
                     st->window, pos, qinv, static_cast<const IOT*>(q), static_cast<const IOT*>(k),   \
                     static_cast<const IOT*>(v), alpha, beta, static_cast<IOT*>(o))
  const int pk = packing(st);
  if (io == GDNRT_F32) {
    if (pk == 4) GDNRT_DECODE(float, 4);
    else if (pk == 6) GDNRT_DECODE(float, 6);
    else GDNRT_DECODE(float, 8);
  } else {
    if (pk == 4) GDNRT_DECODE(uint16_t, 4);
    else if (pk == 6) GDNRT_DECODE(uint16_t, 6);
    else GDNRT_DECODE(uint16_t, 8);
  }
#undef GDNRT_DECODE
  return check_launch(fn);
}

template <bool KDA>
int window_flush(const char* fn, const leapq_state* st, int pos, const float* dense, const float* q0,
                 int iters, int smooth_mode, float* pre_round, void* stream, FlushToken tok = FlushToken{}) {
  int rc = check_state(st, fn);
  if (rc != GDNRT_OK) return rc;
  if (pos < 0 || pos > st->window)
    return set_error(GDNRT_ESTATE, "%s: pos=%d outside [0, window=%d]", fn, pos, st->window);
  if (smooth_mode < 0 || smooth_mode > 2) return set_error(GDNRT_EINVAL, "%s: smooth_mode=%d", fn, smooth_mode);
  if (iters < 0 || iters > 64) return set_error(GDNRT_EINVAL, "%s: iters=%d", fn, iters);
  if (st->N == 0) return clear_error();
  if (st->rank > 0 && !q0) return set_error(GDNRT_EINVAL, "%s: q0 is null", fn);
  if ((dense && !aligned16(dense)) || (pre_round && !aligned16(pre_round)) || (q0 && !aligned4(q0)) ||
      (KDA && !aligned16(st->buf_a)))
    return set_error(GDNRT_EALIGN, "%s: dense, pre_round%s must be 16-byte aligned", fn, KDA ? ", buf_a" : "");
  const size_t N = st->N, nS = N * kD * kD * 4;
  if ((dense && (overlaps(dense, nS, st->codes, code_bytes(st)) || overlaps(dense, nS, pre_round, nS))) ||
      (pre_round && overlaps(pre_round, nS, st->codes, code_bytes(st))))
    return set_error(GDNRT_EINVAL, "%s: dense / pre_round overlap the state", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float qf = (float)code_max(st), qinv = 1.0f / qf;
  const int pk = packing(st);
  switch (st->rank) {
#define GDNRT_FLUSH(R)                                                                            \
  case R:                                                                                         \
    if (tok.q)                                                                                    \
      hipLaunchKernelGGL((leapq_flush_kernel<R, KDA, true>), dim3((unsigned)N), dim3(kFlushNT),  \
                         0, s, st->codes, st->vscale, st->ksmooth, st->ct_k, st->ct_u, st->buf_k, \
                         st->buf_u, st->buf_a, st->window, pos, dense, q0, iters, smooth_mode,    \
                         qf, qinv, pre_round, tok, pk);                                           \
    else                                                                                          \
      hipLaunchKernelGGL((leapq_flush_kernel<R, KDA, false>), dim3((unsigned)N), dim3(kFlushNT), \
                         0, s, st->codes, st->vscale, st->ksmooth, st->ct_k, st->ct_u, st->buf_k, \
                         st->buf_u, st->buf_a, st->window, pos, dense, q0, iters, smooth_mode,    \
                         qf, qinv, pre_round, tok, pk);                                           \
    break;
    GDNRT_FLUSH(0) GDNRT_FLUSH(1) GDNRT_FLUSH(2) GDNRT_FLUSH(3) GDNRT_FLUSH(4)
    GDNRT_FLUSH(5) GDNRT_FLUSH(6) GDNRT_FLUSH(7) GDNRT_FLUSH(8)
#undef GDNRT_FLUSH
  }
  return check_launch(fn);
}

// The last token of a window and the flush in one launch: the arguments of
// leapq_decode_step at pos = window - 1, then those of leapq_window_flush.
template <bool KDA>
int decode_flush(const char* fn, const leapq_state* st, const void* q, const void* k, const void* v,
                 const float* alpha, const float* beta, void* o, int io, const float* q0, int iters,
                 int smooth_mode, void* stream) {
  int rc = check_state(st, fn);
  if (rc != GDNRT_OK) return rc;
  if (io != GDNRT_F32 && io != GDNRT_BF16) return set_error(GDNRT_EDTYPE, "%s: io=%d", fn, io);
  if (st->N == 0) return clear_error();
  if (!q || !k || !v || !alpha || !beta || !o) return set_error(GDNRT_EINVAL, "%s: null pointer argument", fn);
  if (!aligned4(q) || !aligned4(k) || !aligned4(v) || !aligned4(o) || !aligned4(alpha) || !aligned4(beta))
    return set_error(GDNRT_EALIGN, "%s: q, k, v, o, alpha, beta must be 4-byte aligned", fn);
  const size_t es = io == GDNRT_F32 ? 4 : 2;
  const size_t N = st->N, nIO = N * kD * es, nB = N * st->window * kD * 4;
  const size_t nA = KDA ? N * kD * 4 : N * 4, nBA = KDA ? nB : N * st->window * 4;
  const size_t nCT = N * st->rank * kD * 2, nV = N * kD * 4;
  // o is written by every block; the stored state is rewritten by each head's block while
  // the other blocks still read their token inputs, so no input may share a byte with o or
  // with the state the launch writes (a cross-block race otherwise).
  struct Span { const void* p; size_t n; };
  const Span written[] = {{o, nIO}, {st->codes, code_bytes(st)}, {st->vscale, nV}, {st->ksmooth, nV},
                          {st->ct_k, nCT}, {st->ct_u, nCT}};
  const Span read[] = {{q, nIO}, {k, nIO}, {v, nIO}, {alpha, nA}, {beta, N * 4},
                       {st->buf_k, nB}, {st->buf_u, nB}, {st->buf_a, nBA}};
  for (const Span& r : read)
    if (overlaps(o, nIO, r.p, r.n)) return set_error(GDNRT_EINVAL, "%s: o overlaps an input", fn);
  for (int w = 1; w < 6; ++w)
    if (overlaps(o, nIO, written[w].p, written[w].n))
      return set_error(GDNRT_EINVAL, "%s: o overlaps the stored state", fn);
  for (int i = 0; i < 5; ++i)        // the token's inputs (the buffer is the state's own)
    for (int w = 1; w < 6; ++w)
      if (overlaps(read[i].p, read[i].n, written[w].p, written[w].n))
        return set_error(GDNRT_EINVAL, "%s: a token input overlaps the stored state", fn);
  return window_flush<KDA>(fn, st, st->window - 1, nullptr, q0, iters, smooth_mode, nullptr, stream,
                           FlushToken{q, k, v, alpha, beta, o, io});
}

}  // namespace

extern "C" int leapq_decode_flush(const leapq_state* st, const void* q, const void* k, const void* v,
                                  const float* alpha, const float* beta, void* o, int io, const float* q0,
                                  int iters, int smooth_mode, void* stream) {
  return decode_flush<false>("leapq_decode_flush", st, q, k, v, alpha, beta, o, io, q0, iters, smooth_mode,
                             stream);
}

extern "C" int kda_leapq_decode_flush(const leapq_state* st, const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta, void* o, int io,
                                      const float* q0, int iters, int smooth_mode, void* stream) {
  return decode_flush<true>("kda_leapq_decode_flush", st, q, k, v, alpha, beta, o, io, q0, iters, smooth_mode,
                            stream);
}

extern "C" int leapq_decode_step(const leapq_state* st, int pos, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta, void* o,
                                 int io, void* stream) {
  return decode_step<false>("leapq_decode_step", st, pos, q, k, v, alpha, beta, o, io, stream);
}

extern "C" int leapq_window_flush(const leapq_state* st, int pos, const float* dense,
                                  const float* q0, int iters, int smooth_mode, float* pre_round,
                                  void* stream) {
  return window_flush<false>("leapq_window_flush", st, pos, dense, q0, iters, smooth_mode, pre_round, stream);
}

extern "C" int kda_leapq_decode_step(const leapq_state* st, int pos, const void* q, const void* k,
                                     const void* v, const float* alpha, const float* beta, void* o,
                                     int io, void* stream) {
  return decode_step<true>("kda_leapq_decode_step", st, pos, q, k, v, alpha, beta, o, io, stream);
}

extern "C" int kda_leapq_window_flush(const leapq_state* st, int pos, const float* dense,
                                      const float* q0, int iters, int smooth_mode, float* pre_round,
                                      void* stream) {
  return window_flush<true>("kda_leapq_window_flush", st, pos, dense, q0, iters, smooth_mode, pre_round,
                            stream);
}

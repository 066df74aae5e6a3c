// Gated DeltaNet decode with the state re-rounded after every token: the per-step
// baselines of "LeapQuant: an 8-bit recurrent state that stops rounding every token",
// section "Rounding every token" (eq. 2: the next state is computed from the stored
// low-precision one and stored again).
//
//   BF16 state:  S is kept in bf16; each token computes u_i = b (v_i - a S_i.k),
//                o_i = a S_i.q + u_i (k.q) and S_i <- a S_i + u_i k in fp32 from the stored
//                row, then rounds the row to bf16 (nearest even).
//   b-bit state: S is kept as codes Z in [-Q, Q] (Q = 2^(b-1) - 1, int8 container) and
//                one fp32 scale per value row, m_i = max_k |S_i,k|, dequantised as
//                m_i Z_i,k / Q; after the same fp32 step the row is requantised:
//                m_i <- max |S_i|, Z_i <- clamp(rint(S_i (Q / m_i)), -Q, Q).
//                No smoothing and no compensator tokens: the page's eq. 2 scheme.
//
// Mapping: every lane holds 16 bytes of each of its rows (8 bf16 entries, or 16 codes),
// so a row is 16 (bf16) or 8 (codes) consecutive lanes and one wave instruction moves 1
// KiB of state, as in the fp32 decode kernel; each lane group carries 2 rows, 16 (bf16)
// or 32 (codes) apart, so that its q and k entries, loaded once, serve both, and a
// 256-thread block owns 32 (bf16) or 64 (codes) rows of one head. The state is streamed with non-temporal loads and stores
// (it is read and written once per step and does not fit the caches). Over T tokens in one launch the row stays in registers
// and is rounded after every token exactly as a launch per token would.
#include "common.hpp"

namespace gdnrt {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// reductions over an aligned group of L = 16 or 8 lanes (DPP inside 16-lane rows)
template <int L>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (L == 16) return sum16(x);
  else return sum8(x);
}
template <int L>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (L == 16) x = fmaxf(x, dpp<0x140>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0xB1>(x));
  return x;
}

__device__ __forceinline__ float bf16_round(float x) { return bf16_to_f32(f32_to_bf16(x)); }

// E entries of a q/k row at column c (fp32 or bf16 storage)
template <typename IO, int E>
__device__ __forceinline__ void load_vec(const IO* p, float (&x)[E]) {
#pragma unroll
  for (int e = 0; e < E; e += 4) {
    const f32x4 w = io_traits<IO>::ld4(p, e);
    x[e] = w.x;
    x[e + 1] = w.y;
    x[e + 2] = w.z;
    x[e + 3] = w.w;
  }
}

template <typename IO, bool BF16STATE>
__global__ __launch_bounds__(256) void gdn_decode_lowp_kernel(
    void* __restrict__ Sv, float* __restrict__ rowmax, float qf, float qinv, const IO* __restrict__ q,
    const IO* __restrict__ k, const IO* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, IO* __restrict__ o, int T) {
  constexpr int E = BF16STATE ? 8 : 16;   // entries per lane and row (16 bytes)
  constexpr int L = kD / E;               // lanes per row
  constexpr int R = 2;                    // rows per lane group: q and k are loaded once for R rows
  constexpr int RPB = 256 / L * R;        // rows per block
  constexpr int BPH = kD / RPB;           // blocks per head
  const int tid = threadIdx.x;
  const int head = blockIdx.x / BPH;
  const int row0 = (blockIdx.x % BPH) * RPB + tid / L;   // rows row0 + (256 / L) r
  const int col = (tid % L) * E;
  const bool lead = (tid % L) == 0;
  auto erow = [&](int r) { return (size_t)head * kD * kD + (size_t)(row0 + (256 / L) * r) * kD + col; };
  auto rrow = [&](int r) { return (size_t)head * kD + row0 + (256 / L) * r; };

  float s[R][E];
  float m[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = 0.f;
    if constexpr (BF16STATE) {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(Sv) + erow(r)));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[r][2 * j] = __uint_as_float(w[j] << 16);
        s[r][2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      }
    } else {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const int8_t*>(Sv) + erow(r)));
      m[r] = rowmax[rrow(r)];
      const float sv = m[r] * qinv;
#pragma unroll
      for (int e = 0; e < E; ++e) s[r][e] = sv * (float)(int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xff);
    }
  }
  uint32_t zw[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) zw[r][j] = 0u;

  for (int t = 0; t < T; ++t) {
    const size_t tok = (size_t)head * T + t;
    float k4[E], q4[E];
    load_vec<IO, E>(k + tok * kD + col, k4);
    load_vec<IO, E>(q + tok * kD + col, q4);
    const float a = alpha[tok], b = beta[tok];
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) kq += k4[e] * q4[e];
    kq = group_sum<L>(kq);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = row0 + (256 / L) * r;
      const float vi = io_traits<IO>::ld(v, tok * kD + row);
      float pk = 0.f, pq = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        pk += s[r][e] * k4[e];
        pq += s[r][e] * q4[e];
      }
      pk = group_sum<L>(pk);
      pq = group_sum<L>(pq);
      const float u = b * (vi - a * pk);
      const float oi = a * pq + u * kq;
      if (lead) io_traits<IO>::st(o, tok * kD + row, oi);
      float sn[E];
#pragma unroll
      for (int e = 0; e < E; ++e) sn[e] = a * s[r][e] + u * k4[e];
      if constexpr (BF16STATE) {
#pragma unroll
        for (int e = 0; e < E; ++e) s[r][e] = bf16_round(sn[e]);
      } else {
        float mx = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) mx = fmaxf(mx, fabsf(sn[e]));
        m[r] = group_max<L>(mx);
        const float sc = m[r] > 0.f ? qf / m[r] : 0.f, sv = m[r] * qinv;
#pragma unroll
        for (int j = 0; j < 4; ++j) zw[r][j] = 0u;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float z = fminf(fmaxf(rintf(sn[e] * sc), -qf), qf);
          s[r][e] = sv * z;
          zw[r][e >> 2] |= (uint32_t)((int32_t)z & 0xff) << (8 * (e & 3));
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if constexpr (BF16STATE) {
      __builtin_nontemporal_store(u32x4{pack_bf16(s[r][0], s[r][1]), pack_bf16(s[r][2], s[r][3]),
                                        pack_bf16(s[r][4], s[r][5]), pack_bf16(s[r][6], s[r][7])},
                                  reinterpret_cast<u32x4*>(static_cast<uint16_t*>(Sv) + erow(r)));
    } else if (T > 0) {
      __builtin_nontemporal_store(u32x4{zw[r][0], zw[r][1], zw[r][2], zw[r][3]},
                                  reinterpret_cast<u32x4*>(static_cast<int8_t*>(Sv) + erow(r)));
      if (lead) rowmax[rrow(r)] = m[r];
    }
  }
}

}  // namespace gdnrt

using namespace gdnrt;

static int lowp_decode(const char* fn, bool bf16state, void* S, float* rowmax, int bits, const void* q,
                       const void* k, const void* v, const float* alpha, const float* beta, void* o, int N,
                       int T, int dk, int dv, int io, void* stream) {
  if (N < 0 || T < 0) return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d must be >= 0", fn, N, T);
  if (dk != kD || dv != kD)
    return set_error(GDNRT_ESHAPE, "%s: d_k=%d d_v=%d, only 128 is supported", fn, dk, dv);
  if (!bf16state && (bits < 2 || bits > 8)) return set_error(GDNRT_ESHAPE, "%s: bits=%d must be in [2, 8]", fn, bits);
  if (io != GDNRT_F32 && io != GDNRT_BF16) return set_error(GDNRT_EDTYPE, "%s: io=%d", fn, io);
  if (N == 0 || T == 0) return clear_error();
  if (!S || (!bf16state && !rowmax) || !q || !k || !v || !alpha || !beta || !o)
    return set_error(GDNRT_EINVAL, "%s: null pointer argument", fn);
  if ((size_t)N * (kD / 8) > 0x7fffffffu || (size_t)N * (size_t)T > ((size_t)1 << 36))
    return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d too large", fn, N, T);
  if (!aligned16(S) || !aligned16(q) || !aligned16(k) || !aligned4(v) || !aligned4(o) || !aligned4(alpha) ||
      !aligned4(beta) || (!bf16state && !aligned4(rowmax)))
    return set_error(GDNRT_EALIGN, "%s: S, q, k must be 16-byte aligned, the rest 4-byte", fn);
  const size_t es = io == GDNRT_F32 ? 4 : 2, ntok = (size_t)N * T;
  const size_t nS = (size_t)N * kD * kD * (bf16state ? 2 : 1), nM = (size_t)N * kD * 4;
  const size_t nIO = ntok * kD * es, nG = ntok * 4;
  const void* ins[] = {q, k, v};
  for (const void* b : ins)
    if (overlaps(o, nIO, b, nIO) || overlaps(S, nS, b, nIO) || (rowmax && overlaps(rowmax, nM, b, nIO)))
      return set_error(GDNRT_EINVAL, "%s: buffers overlap", fn);
  if (overlaps(o, nIO, S, nS) || overlaps(o, nIO, alpha, nG) || overlaps(o, nIO, beta, nG) ||
      overlaps(S, nS, alpha, nG) || overlaps(S, nS, beta, nG) ||
      (rowmax && (overlaps(rowmax, nM, S, nS) || overlaps(rowmax, nM, o, nIO))))
    return set_error(GDNRT_EINVAL, "%s: buffers overlap", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // blocks per head: 4 (bf16 rows, 32 per block) or 2 (code rows, 64 per block)
  const dim3 grid((unsigned)(N * (bf16state ? 4 : 2))), block(256);
  const float qf = bf16state ? 0.f : (float)((1 << (bits - 1)) - 1), qinv = bf16state ? 0.f : 1.0f / qf;
#define GDNRT_LOWP(IOT, B)                                                                              \
  hipLaunchKernelGGL((gdn_decode_lowp_kernel<IOT, B>), grid, block, 0, s, S, rowmax, qf, qinv,         \
                     static_cast<const IOT*>(q), static_cast<const IOT*>(k), static_cast<const IOT*>(v), \
                     alpha, beta, static_cast<IOT*>(o), T)
  if (io == GDNRT_F32) {
    if (bf16state) GDNRT_LOWP(float, true); else GDNRT_LOWP(float, false);
  } else {
    if (bf16state) GDNRT_LOWP(uint16_t, true); else GDNRT_LOWP(uint16_t, false);
  }
#undef GDNRT_LOWP
  return check_launch(fn);
}

extern "C" int gdn_decode_step_bf16_state(uint16_t* S, const void* q, const void* k, const void* v,
                                          const float* alpha, const float* beta, void* o, int N, int T,
                                          int dk, int dv, int io, void* stream) {
  return lowp_decode("gdn_decode_step_bf16_state", true, S, nullptr, 0, q, k, v, alpha, beta, o, N, T, dk, dv,
                     io, stream);
}

extern "C" int gdn_decode_step_int_state(int8_t* codes, float* rowmax, int bits, const void* q, const void* k,
                                         const void* v, const float* alpha, const float* beta, void* o, int N,
                                         int T, int dk, int dv, int io, void* stream) {
  return lowp_decode("gdn_decode_step_int_state", false, codes, rowmax, bits, q, k, v, alpha, beta, o, N, T, dk,
                     dv, io, stream);
}

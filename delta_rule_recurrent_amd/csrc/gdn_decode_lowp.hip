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
// Mapping as the fp32 decode kernel: a 256-thread block owns 8 rows of one head, 32
// lanes per row, four key columns per lane; over T tokens in one launch the row stays
// in registers and is rounded after every token exactly as a launch per token would.
#include "common.hpp"

namespace gdnrt {

// max over the 32 lanes of a row group (DPP inside 16-lane rows, then xor 16)
__device__ __forceinline__ float max32(float x) {
  x = fmaxf(x, dpp<0x140>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F)));
  return x;
}

__device__ __forceinline__ float bf16_round(float x) { return bf16_to_f32(f32_to_bf16(x)); }

template <typename IO, bool BF16STATE>
__global__ __launch_bounds__(256) void gdn_decode_lowp_kernel(
    void* __restrict__ Sv, float* __restrict__ rowmax, float qf, float qinv, const IO* __restrict__ q,
    const IO* __restrict__ k, const IO* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, IO* __restrict__ o, int T) {
  constexpr int kRowsPerBlock = 8;
  constexpr int BPH = kD / kRowsPerBlock;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int head = blockIdx.x / BPH;
  const int row = (blockIdx.x % BPH) * kRowsPerBlock + wave * 2 + (lane >> 5);
  const int col = (lane & 31) * 4;
  const size_t e0 = (size_t)head * kD * kD + (size_t)row * kD + col;
  const size_t r0 = (size_t)head * kD + row;

  f32x4 s;
  uint32_t zw = 0;   // b-bit: this lane's 4 codes
  float m = 0.f;
  if constexpr (BF16STATE) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(Sv) + e0);
    s = f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
              __uint_as_float(w.y & 0xffff0000u)};
  } else {
    zw = *reinterpret_cast<const uint32_t*>(static_cast<const int8_t*>(Sv) + e0);
    m = rowmax[r0];
    const float sv = m * qinv;
    s = f32x4{sv * (float)(int8_t)(zw & 0xff), sv * (float)(int8_t)((zw >> 8) & 0xff),
              sv * (float)(int8_t)((zw >> 16) & 0xff), sv * (float)(int8_t)(zw >> 24)};
  }

  for (int t = 0; t < T; ++t) {
    const size_t tok = (size_t)head * T + t;
    const f32x4 k4 = io_traits<IO>::ld4(k, tok * kD + col);
    const f32x4 q4 = io_traits<IO>::ld4(q, tok * kD + col);
    const float a = alpha[tok], b = beta[tok];
    const float vi = io_traits<IO>::ld(v, tok * kD + row);
    const float kq = sum32(k4.x * q4.x + k4.y * q4.y + k4.z * q4.z + k4.w * q4.w);
    const float pk = sum32(s.x * k4.x + s.y * k4.y + s.z * k4.z + s.w * k4.w);
    const float pq = sum32(s.x * q4.x + s.y * q4.y + s.z * q4.z + s.w * q4.w);
    const float u = b * (vi - a * pk);
    const float oi = a * pq + u * kq;
    const f32x4 sn = a * s + u * k4;
    if ((lane & 31) == 0) io_traits<IO>::st(o, tok * kD + row, oi);
    if constexpr (BF16STATE) {
      s = f32x4{bf16_round(sn.x), bf16_round(sn.y), bf16_round(sn.z), bf16_round(sn.w)};
    } else {
      m = max32(fmaxf(fmaxf(fabsf(sn.x), fabsf(sn.y)), fmaxf(fabsf(sn.z), fabsf(sn.w))));
      const float sc = m > 0.f ? qf / m : 0.f, sv = m * qinv;
      zw = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float z = fminf(fmaxf(rintf(sn[e] * sc), -qf), qf);
        s[e] = sv * z;
        zw |= (uint32_t)((int32_t)z & 0xff) << (8 * e);
      }
    }
  }
  if constexpr (BF16STATE) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Sv) + e0) =
        make_uint2(pack_bf16(s.x, s.y), pack_bf16(s.z, s.w));
  } else {
    *reinterpret_cast<uint32_t*>(static_cast<int8_t*>(Sv) + e0) = zw;
    if ((lane & 31) == 0) rowmax[r0] = m;
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
  const dim3 grid((unsigned)(N * (kD / 8))), block(256);
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

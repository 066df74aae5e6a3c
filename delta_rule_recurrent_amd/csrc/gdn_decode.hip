// Gated DeltaNet recurrent step (decode), fp32 state streamed through HBM.
//
// Method: "LeapQuant: an 8-bit recurrent state that stops rounding every token",
// section "The state, from the update rule up" (delta rule with a scalar decay,
// eq. 3's correction form) and section "Why a decode step is a memory copy". In the
// [d_v][d_k] layout the update S_t = a S (I - b k k^T) + b v k^T splits by rows:
// row i needs only its own dot products with k and q,
//
//     u_i = b (v_i - a S_i.k),   o_i = a S_i.q + u_i (k.q),   S_i <- a S_i + u_i k,
//
// so one read and one write of each 512-byte row per token is the whole traffic;
// o uses the pre-update row and k.q instead of a second pass over the new row.
//
// Mapping: a 256-thread block (four 64-lane waves) owns 16 rows of one head, so a
// head is 8 blocks. Each row is held by 32 lanes, four consecutive floats per lane:
// one 16-byte load per lane covers two whole rows, a perfectly coalesced 1 KiB per
// wave instruction. Each 32-lane group holds two rows 8 apart, so the lane's q and
// k entries (and k.q) serve both. The state is touched once per step and does not
// fit in any cache, so it is read and written with non-temporal hints. Measured on
// MI355X, two rows per lane group beat one (KDA 2% faster, its decay vector loaded
// once for both rows; GDN up to 2%, on some boxes within noise) and four (4% slower,
// fewer blocks in flight); small blocks beat larger persistent tiles and a plain copy
// kernel. Row sums use DPP inside 16-lane rows plus one swizzle across the two halves
// of a 32-lane group.
//
// Kimi Delta Attention (same section: the decay becomes a vector alpha_t, one factor
// per key channel, eq. 1) runs through the same kernel: with the decay folded into
// the two read vectors,
//
//     u_i = b (v_i - S_i.(a o k)),   o_i = S_i.(a o q) + u_i (k.q),   S_i <- a o S_i + u_i k.
#include "common.hpp"

namespace gdnrt {

// VEC: alpha is [N][T][d_k] (one decay per key channel, KDA) instead of [N][T].
// R: rows per lane, 8 apart, so that the lane's q, k (and decay) entries serve R rows.
template <typename IO, bool VEC, int R>
__global__ __launch_bounds__(256) void gdn_decode_kernel(
    float* __restrict__ S, const IO* __restrict__ q, const IO* __restrict__ k,
    const IO* __restrict__ v, const float* __restrict__ alpha, const float* __restrict__ beta,
    IO* __restrict__ o, int T) {
  constexpr int kRowsPerBlock = 8 * R;
  constexpr int BPH = kD / kRowsPerBlock;   // blocks per head
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int head = blockIdx.x / BPH;
  const int row0 = (blockIdx.x % BPH) * kRowsPerBlock + wave * 2 + (lane >> 5);   // rows row0 + 8 r
  const int col = (lane & 31) * 4;      // first key column of this lane

  f32x4* Sp[R];
  f32x4 s[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    Sp[r] = reinterpret_cast<f32x4*>(S + (size_t)head * kD * kD + (size_t)(row0 + 8 * r) * kD + col);
    s[r] = __builtin_nontemporal_load(Sp[r]);
  }

  for (int t = 0; t < T; ++t) {
    const size_t tok = (size_t)head * T + t;
    const f32x4 k4 = io_traits<IO>::ld4(k, tok * kD + col);
    const f32x4 q4 = io_traits<IO>::ld4(q, tok * kD + col);
    const float b = beta[tok];
    const float kq = sum32(k4.x * q4.x + k4.y * q4.y + k4.z * q4.z + k4.w * q4.w);
    f32x4 a4, ak, aq;
    float a = 1.f;
    if constexpr (VEC) {
      a4 = *reinterpret_cast<const f32x4*>(alpha + tok * kD + col);
      ak = a4 * k4;
      aq = a4 * q4;
    } else {
      a = alpha[tok];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = row0 + 8 * r;
      const float vi = io_traits<IO>::ld(v, tok * kD + row);
      float u, oi;
      if constexpr (VEC) {
        const float pk = sum32(s[r].x * ak.x + s[r].y * ak.y + s[r].z * ak.z + s[r].w * ak.w);
        const float pq = sum32(s[r].x * aq.x + s[r].y * aq.y + s[r].z * aq.z + s[r].w * aq.w);
        u = b * (vi - pk);
        oi = pq + u * kq;
        s[r] = a4 * s[r] + u * k4;
      } else {
        const float pk = sum32(s[r].x * k4.x + s[r].y * k4.y + s[r].z * k4.z + s[r].w * k4.w);
        const float pq = sum32(s[r].x * q4.x + s[r].y * q4.y + s[r].z * q4.z + s[r].w * q4.w);
        u = b * (vi - a * pk);
        oi = a * pq + u * kq;
        s[r] = a * s[r] + u * k4;
      }
      if ((lane & 31) == 0) io_traits<IO>::st(o, tok * kD + row, oi);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) __builtin_nontemporal_store(s[r], Sp[r]);
}

template <typename IO, bool VEC>
static void launch_decode(float* S, const void* q, const void* k, const void* v,
                          const float* alpha, const float* beta, void* o, int N, int T,
                          hipStream_t stream) {
  constexpr int R = 2;
  hipLaunchKernelGGL((gdn_decode_kernel<IO, VEC, R>), dim3(N * (kD / (8 * R))), dim3(256), 0, stream, S,
                     static_cast<const IO*>(q), static_cast<const IO*>(k),
                     static_cast<const IO*>(v), alpha, beta, static_cast<IO*>(o), T);
}

}  // namespace gdnrt

using namespace gdnrt;

// Shared by the scalar-decay (GDN) and per-channel-decay (KDA) entry points; `vec`
// selects the decay layout ([N][T] or [N][T][d_k]).
static int decode_step(const char* fn, bool vec, float* S, const void* q, const void* k, const void* v,
                       const float* alpha, const float* beta, void* o, int N, int T, int dk, int dv,
                       int io, void* stream) {
  if (N < 0 || T < 0) return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d must be >= 0", fn, N, T);
  if (dk != kD || dv != kD)
    return set_error(GDNRT_ESHAPE, "%s: d_k=%d d_v=%d, only 128 is supported", fn, dk, dv);
  if (io != GDNRT_F32 && io != GDNRT_BF16) return set_error(GDNRT_EDTYPE, "%s: io=%d", fn, io);
  if (N == 0 || T == 0) return clear_error();
  if (!S || !q || !k || !v || !alpha || !beta || !o)
    return set_error(GDNRT_EINVAL, "%s: null pointer argument", fn);
  if ((size_t)N * (kD / 8) > 0x7fffffffu || (size_t)N * (size_t)T > ((size_t)1 << 36))
    return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d too large", fn, N, T);
  if (!aligned16(S) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (vec ? !aligned16(alpha) : !aligned4(alpha)) || !aligned4(beta))
    return set_error(GDNRT_EALIGN, vec ? "%s: S, q, k, v, o, alpha must be 16-byte aligned, beta 4-byte"
                                       : "%s: S, q, k, v, o must be 16-byte aligned, gates 4-byte", fn);
  const size_t es = io == GDNRT_F32 ? 4 : 2;
  const size_t ntok = (size_t)N * T;
  const size_t nS = (size_t)N * kD * kD * 4, nIO = ntok * kD * es, nG = ntok * 4, nA = vec ? ntok * kD * 4 : nG;
  if (overlaps(o, nIO, S, nS) || overlaps(o, nIO, q, nIO) || overlaps(o, nIO, k, nIO) ||
      overlaps(o, nIO, v, nIO) || overlaps(o, nIO, alpha, nA) || overlaps(o, nIO, beta, nG) ||
      overlaps(S, nS, q, nIO) || overlaps(S, nS, k, nIO) || overlaps(S, nS, v, nIO) ||
      overlaps(S, nS, alpha, nA) || overlaps(S, nS, beta, nG))
    return set_error(GDNRT_EINVAL, "%s: S or o overlaps another buffer", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (io == GDNRT_F32)
    vec ? launch_decode<float, true>(S, q, k, v, alpha, beta, o, N, T, s)
        : launch_decode<float, false>(S, q, k, v, alpha, beta, o, N, T, s);
  else
    vec ? launch_decode<uint16_t, true>(S, q, k, v, alpha, beta, o, N, T, s)
        : launch_decode<uint16_t, false>(S, q, k, v, alpha, beta, o, N, T, s);
  return check_launch(fn);
}

extern "C" int gdn_decode_step(float* S, const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta, void* o, int N, int T,
                               int dk, int dv, int io, void* stream) {
  return decode_step("gdn_decode_step", false, S, q, k, v, alpha, beta, o, N, T, dk, dv, io, stream);
}

extern "C" int kda_decode_step(float* S, const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta, void* o, int N, int T,
                               int dk, int dv, int io, void* stream) {
  return decode_step("kda_decode_step", true, S, q, k, v, alpha, beta, o, N, T, dk, dv, io, stream);
}

// The per-device pieces of ZeCO's sequence-parallel GLA forward ("ZeCO: Zero
// Communication Overhead Sequence Parallelism for Linear Attention", sections
// "Local State Computation", "Global State Update Formula", "All-Scan Collective
// Communication" and "The Complete Forward Algorithm").
//
// A device holding one shard of the sequence runs gla_chunk_fwd from a zero state:
// that gives its local outputs and its local final state S_[N], and leaves in the
// workspace, per chunk, Q^ = Q o e^b and the chunk decay gamma = e^{b_C}. Then:
//
//   gla_shard_decay           gamma~_[c] = prod_{i<c} gamma_[i] per key channel, for
//                             c = 0..nc (the decays the later phases need);
//   gla_all_scan_step         the device's All-Scan update of a block of key
//                             channels: S_send = gamma~_[N] o S_recv + S_[N];
//   gla_shard_output_correct  the received state's share of the outputs:
//                             o_t += S_recv (q_t o e^{b_t} o gamma~_[c(t)]),
//                             chunk by chunk, (Q^ o gamma~) S_recv^T.
//
// Because the read-out is linear in the state, the local outputs plus the
// correction are the outputs ZeCO's third phase forms from S_[n-1] + gamma~ o S_recv;
// the correction reads only Q^ (bf16) and the decays from the workspace and o, not
// the per-chunk local states.
#include "chunk_device.hpp"
#include "gla_chunk_layout.hpp"

namespace gdnrt {

namespace zeco {

constexpr int PQ = kD + 8;   // bf16 pitch of the staged state rows (conflict-free 16-byte reads)
constexpr int NT = 512;      // threads per block of the correction

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float lo_bf(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace zeco

// gamma[n][c][k] = prod_{i<c} e^{b_C}(n, i)[k] for c = 0..nc: one thread per
// (sequence, key channel), the chunk decays loaded 16 at a time.
__global__ __launch_bounds__(64) void gla_shard_decay_kernel(const uint8_t* __restrict__ ws,
                                                             float* __restrict__ gamma, int nc) {
  constexpr size_t kStride = gla::kWChunk / 4;   // floats between two chunks' decays
  constexpr int B = 16;
  const int n = blockIdx.x >> 1, key = (blockIdx.x & 1) * 64 + threadIdx.x;
  const float* ec = reinterpret_cast<const float*>(ws + (size_t)n * nc * gla::kWChunk + gla::kWE) + key;
  float* out = gamma + (size_t)n * (nc + 1) * kD + key;
  float g = 1.f;
  out[0] = g;
  int c = 0;
  for (; c + B <= nc; c += B) {
    float e[B];
#pragma unroll
    for (int j = 0; j < B; ++j) e[j] = ec[(size_t)(c + j) * kStride];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      g *= e[j];
      out[(size_t)(c + j + 1) * kD] = g;
    }
  }
  for (; c < nc; ++c) {
    g *= ec[(size_t)c * kStride];
    out[(size_t)(c + 1) * kD] = g;
  }
}

// S_send[n][v][k] = gamma[n][k] S_recv[n][v][k] + S_local[n][v][k] for k in [k0, k0 + kw);
// S_recv null: S_send = S_local. One thread per element.
__global__ __launch_bounds__(256) void gla_all_scan_step_kernel(const float* S_recv, const float* __restrict__ gamma,
                                                                size_t gstride, const float* S_local, float* S_send,
                                                                size_t rows, int k0, int kw) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * (size_t)kw) return;
  const size_t r = i / (size_t)kw;
  const int k = k0 + (int)(i - r * (size_t)kw);
  const size_t e = r * kD + k;
  float s = S_local[e];
  if (S_recv) s = fmaf(gamma[(r / kD) * gstride + k], S_recv[e], s);
  S_send[e] = s;
}

namespace zeco {

// One chunk's operands of a correction wave: its four Q^ operands of its token block
// and its 32 bytes of o (16 consecutive value channels of one token).
struct CorrIn {
  u32x4 qf[4];
  u32x4 ov[2];
};

__device__ __forceinline__ void corr_load(CorrIn& in, const uint8_t* __restrict__ ws,
                                          const uint16_t* __restrict__ o, int n, int nc, int c, int tb,
                                          int vb0) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, lq = lane >> 4;
  const uint8_t* wsc = ws + ((size_t)n * nc + c) * gla::kWChunk + gla::kWQ;
  const uint16_t* orow = o + (((size_t)n * nc + c) * kChunk + tb * 16 + l16) * kD + 16 * (vb0 + lq);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    in.qf[ks] = *reinterpret_cast<const u32x4*>(wsc + ((size_t)(tb * 4 + ks) * 64 + lane) * 16);
  in.ov[0] = *reinterpret_cast<const u32x4*>(orow);
  in.ov[1] = *reinterpret_cast<const u32x4*>(orow + 8);
}

// Element offset of S[v][k] in the staged state: rows of PQ bf16, the 16-byte groups of
// rows with bit 4 of v set moved by four groups, so that the eight rows
// b + {0..3, 16..19} that eight lanes read together fall on distinct bank groups.
__device__ __forceinline__ int s_off(int v, int k) {
  return v * PQ + ((k & ~7) ^ (((v >> 4) & 1) << 5)) + (k & 7);
}

}  // namespace zeco

// o[n][t] += S_in[n] (Q^ o gamma~_[c])_t over the chunks [part * cpb, part * cpb + cpb) of
// sequence n. The block stages S_in[n] in LDS as bf16; wave w forms four transposed
// output tiles of each chunk, D[v][t] = sum_k S[v][k] (Q^ o gamma~)[t][k], for the
// tokens of block tb = w & 3 and the 64 value channels from 16 vb0, vb0 = 4 (w >> 2):
// the workspace's 16-byte pieces of Q^ are the B operand of that product (lane l16 =
// token, keys 32 ks + 4 lq + e and 32 ks + 16 + 4 lq + e), scaled by the decay of those
// keys; the state is staged with its keys in the same order (gdc::qcol), so that the
// A operand is one 16-byte read. Row i = 4 lq + r of tile
// j stands for value channel 16 vb0 + 16 lq + 4 j + r, so that the 16 D values a lane
// holds over the four tiles are 16 consecutive channels of one token: o is read and
// written as 32 contiguous bytes per lane.
__global__ __launch_bounds__(512) void gla_shard_correct_kernel(const uint8_t* __restrict__ ws,
                                                                const float* __restrict__ gamma,
                                                                const float* __restrict__ S_in,
                                                                uint16_t* __restrict__ o, int N, int nc, int cpb,
                                                                int nblk) {
  using namespace zeco;
  __shared__ __attribute__((aligned(16))) uint16_t Ss[kD * PQ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  // block -> (sequence, chunk range); the blocks of one sequence share an XCD
  int n, part;
  {
    const int bid = blockIdx.x;
    if ((N & 7) == 0) {
      const int xcd = bid & 7, slot = bid >> 3;
      n = (slot / nblk) * 8 + xcd;
      part = slot % nblk;
    } else {
      n = bid / nblk;
      part = bid % nblk;
    }
  }
  const int tb = wave & 3, vb0 = (wave >> 2) * 4;
  const int c0 = part * cpb, c1 = min(nc, c0 + cpb);
  // the first chunk's operands are requested before the state is staged
  CorrIn in;
  corr_load(in, ws, o, n, nc, c0, tb, vb0);
  {
    const float* Sn = S_in + (size_t)n * kD * kD;
#pragma unroll
    for (int h = 0; h < kD * kD / 4 / NT; ++h) {
      const int i = tid + NT * h, r = i >> 5, c = (i & 31) * 4;
      const f32x4 x = *reinterpret_cast<const f32x4*>(Sn + 4 * (size_t)i);
      *reinterpret_cast<u32x2*>(Ss + s_off(r, gdc::qcol(c))) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
    }
  }
  lds_barrier();

  // the LDS row each lane reads as the A operand of tile j: value 16 vb0 + 16 (l16 >> 2) + 4 j + (l16 & 3)
  const int vrow = 16 * vb0 + 16 * (l16 >> 2) + (l16 & 3);
  for (int c = c0; c < c1; ++c) {
    // the state fragments are read from LDS for every chunk rather than held in 64
    // registers across the loop: fewer registers let more blocks share a CU
    asm volatile("" ::: "memory");
    if (c > c0) corr_load(in, ws, o, n, nc, c, tb, vb0);
    const float* gr = gamma + ((size_t)n * (nc + 1) + c) * kD;
    uint16_t* orow = o + (((size_t)n * nc + c) * kChunk + tb * 16 + l16) * kD + 16 * (vb0 + lq);
    bf16x8 bq[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(gr + 32 * ks + 4 * lq);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(gr + 32 * ks + 16 + 4 * lq);
      const u32x4 w = in.qf[ks];
      const u32x4 r = {pack_bf16(lo_bf(w[0]) * g0[0], hi_bf(w[0]) * g0[1]),
                       pack_bf16(lo_bf(w[1]) * g0[2], hi_bf(w[1]) * g0[3]),
                       pack_bf16(lo_bf(w[2]) * g1[0], hi_bf(w[2]) * g1[1]),
                       pack_bf16(lo_bf(w[3]) * g1[2], hi_bf(w[3]) * g1[3])};
      bq[ks] = __builtin_bit_cast(bf16x8, r);
    }
    u32x4 out[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                       Ss + s_off(vrow + 4 * j, 32 * ks + 8 * lq))),
                   bq[ks], acc);
      const unsigned w0 = in.ov[j >> 1][2 * (j & 1)], w1 = in.ov[j >> 1][2 * (j & 1) + 1];
      out[j >> 1][2 * (j & 1)] = pack_bf16(lo_bf(w0) + acc[0], hi_bf(w0) + acc[1]);
      out[j >> 1][2 * (j & 1) + 1] = pack_bf16(lo_bf(w1) + acc[2], hi_bf(w1) + acc[3]);
    }
    *reinterpret_cast<u32x4*>(orow) = out[0];
    *reinterpret_cast<u32x4*>(orow + 8) = out[1];
  }
}

}  // namespace gdnrt

using namespace gdnrt;

static int shard_shape(const char* fn, int N, int T, int dk, int dv, int chunk) {
  if (N < 0 || T < 0) return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d must be >= 0", fn, N, T);
  if (dk != kD || dv != kD) return set_error(GDNRT_ESHAPE, "%s: d_k=%d d_v=%d, only 128 is supported", fn, dk, dv);
  if (chunk != kChunk) return set_error(GDNRT_ESHAPE, "%s: chunk=%d, only 64 is supported", fn, chunk);
  if (T % kChunk) return set_error(GDNRT_ESHAPE, "%s: T=%d is not a multiple of 64", fn, T);
  if ((size_t)N * (T / kChunk + 1) > 0x7fffffffu || (size_t)N * 2 > 0x7fffffffu)
    return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d too large", fn, N, T);
  return GDNRT_OK;
}

extern "C" int gla_shard_decay(const void* workspace, size_t ws_bytes, float* gamma, int N, int T, int dk,
                               int chunk, void* stream) {
  const char* fn = "gla_shard_decay";
  int rc = shard_shape(fn, N, T, dk, dk, chunk);
  if (rc != GDNRT_OK) return rc;
  if (N == 0) return clear_error();
  const int nc = T / kChunk;
  const size_t need = (size_t)N * nc * gla::kWChunk, nG = (size_t)N * (nc + 1) * kD * 4;
  if (!gamma || (need && !workspace)) return set_error(GDNRT_EINVAL, "%s: null pointer argument", fn);
  if (ws_bytes < need)
    return set_error(GDNRT_EINVAL, "%s: workspace of %zu bytes expected, %zu given", fn, need, ws_bytes);
  if ((need && !aligned16(workspace)) || !aligned16(gamma))
    return set_error(GDNRT_EALIGN, "%s: workspace and gamma must be 16-byte aligned", fn);
  if (overlaps(gamma, nG, workspace, need)) return set_error(GDNRT_EINVAL, "%s: buffers overlap", fn);
  hipLaunchKernelGGL(gla_shard_decay_kernel, dim3((unsigned)(2 * N)), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(workspace), gamma, nc);
  return check_launch(fn);
}

extern "C" int gla_all_scan_step(const float* S_recv, const float* gamma, size_t gamma_stride, const float* S_local,
                                 float* S_send, int N, int dk, int dv, int k0, int k1, void* stream) {
  const char* fn = "gla_all_scan_step";
  if (N < 0) return set_error(GDNRT_ESHAPE, "%s: N=%d must be >= 0", fn, N);
  if (dk != kD || dv != kD) return set_error(GDNRT_ESHAPE, "%s: d_k=%d d_v=%d, only 128 is supported", fn, dk, dv);
  if (k0 < 0 || k1 < k0 || k1 > dk)
    return set_error(GDNRT_ESHAPE, "%s: key block [%d, %d) is not inside [0, %d)", fn, k0, k1, dk);
  if ((size_t)N * kD * kD > ((size_t)1 << 40)) return set_error(GDNRT_ESHAPE, "%s: N=%d too large", fn, N);
  if (N == 0 || k0 == k1) return clear_error();
  if (!S_local || !S_send || (S_recv && !gamma)) return set_error(GDNRT_EINVAL, "%s: null pointer argument", fn);
  if (S_recv && gamma_stride < (size_t)kD)
    return set_error(GDNRT_ESHAPE, "%s: gamma_stride=%zu must be >= %d", fn, gamma_stride, kD);
  if (!aligned4(S_local) || !aligned4(S_send) || (S_recv && (!aligned4(S_recv) || !aligned4(gamma))))
    return set_error(GDNRT_EALIGN, "%s: pointers must be 4-byte aligned", fn);
  const size_t nS = (size_t)N * kD * kD * 4, nG = S_recv ? ((size_t)(N - 1) * gamma_stride + kD) * 4 : 0;
  if ((S_send != S_local && overlaps(S_send, nS, S_local, nS)) ||
      (S_recv && S_send != S_recv && overlaps(S_send, nS, S_recv, nS)) || overlaps(S_send, nS, gamma, nG))
    return set_error(GDNRT_EINVAL, "%s: buffers overlap (S_send may only equal S_local or S_recv)", fn);
  const size_t rows = (size_t)N * kD, total = rows * (size_t)(k1 - k0);
  hipLaunchKernelGGL(gla_all_scan_step_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), S_recv, gamma, gamma_stride, S_local, S_send, rows, k0,
                     k1 - k0);
  return check_launch(fn);
}

extern "C" int gla_shard_output_correct(const void* workspace, size_t ws_bytes, const float* gamma,
                                        const float* S_in, void* o, int N, int T, int dk, int dv, int chunk,
                                        int io, void* stream) {
  const char* fn = "gla_shard_output_correct";
  int rc = shard_shape(fn, N, T, dk, dv, chunk);
  if (rc != GDNRT_OK) return rc;
  if (io != GDNRT_BF16) return set_error(GDNRT_EDTYPE, "%s: io must be GDNRT_BF16", fn);
  if (N == 0 || T == 0 || !S_in) return clear_error();
  if (!workspace || !gamma || !o) return set_error(GDNRT_EINVAL, "%s: null pointer argument", fn);
  const int nc = T / kChunk;
  const size_t need = (size_t)N * nc * gla::kWChunk;
  if (ws_bytes < need)
    return set_error(GDNRT_EINVAL, "%s: workspace of %zu bytes expected, %zu given", fn, need, ws_bytes);
  if (!aligned16(workspace) || !aligned16(gamma) || !aligned16(S_in) || !aligned16(o))
    return set_error(GDNRT_EALIGN, "%s: workspace, gamma, S_in and o must be 16-byte aligned", fn);
  const size_t nIO = (size_t)N * T * kD * 2, nG = (size_t)N * (nc + 1) * kD * 4, nS = (size_t)N * kD * kD * 4;
  if (overlaps(o, nIO, workspace, need) || overlaps(o, nIO, gamma, nG) || overlaps(o, nIO, S_in, nS))
    return set_error(GDNRT_EINVAL, "%s: o overlaps an input", fn);
  // about four blocks per CU over the whole call, each staging the state once
  const size_t chunks = (size_t)N * nc;
  int cpb = (int)((chunks + 1023) / 1024);
  cpb = cpb < 1 ? 1 : cpb > 16 ? 16 : cpb;
  const int nblk = (nc + cpb - 1) / cpb;
  if ((size_t)N * nblk > 0x7fffffffu) return set_error(GDNRT_ESHAPE, "%s: N=%d T=%d too large", fn, N, T);
  hipLaunchKernelGGL(gla_shard_correct_kernel, dim3((unsigned)(N * nblk)), dim3(zeco::NT), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(workspace), gamma, S_in,
                     static_cast<uint16_t*>(o), N, nc, cpb, nblk);
  return check_launch(fn);
}

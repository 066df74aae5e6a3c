// Device helpers shared by the chunkwise kernels of the delta rule (gfx950): tile
// pitches, bf16 MFMA wrappers, LDS fragment reads (plain and transposing), DPP row
// broadcasts, the 16 x 16 forward substitution and the lower-triangle tile order.
#pragma once

#include "common.hpp"

namespace gdnrt {
namespace gdc {

constexpr int C = kChunk;   // 64
constexpr int NT = 512;     // threads per block, both kernels
constexpr int PQ = kD + 8;  // bf16 pitch of 128-wide rows (16-byte aligned, conflict-free reads)
constexpr int PC = C + 8;   // bf16 pitch of 64-wide rows
constexpr int PF = C + 4;   // fp32 pitch of 64-wide rows (16-byte aligned)

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // register-promotable across loops
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x8 as_bf8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp32 16 x 16 x 4: lane l holds A[l%16][l/16], B[l/16][l%16]; D[4(l/16)+i][l%16]
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ float wave_scan(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ float lo_bf(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// LDS written by some lanes of a wave and read by others of the same wave: the LDS
// executes a wave's instructions in order, so this only keeps the compiler from
// reordering the accesses
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// value of lane J of this lane's row of 16 (DPP row_newbcast)
template <int J>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + J, 0xF, 0xF, false));
}

// Forward substitution for two columns of a unit lower triangular 16 x 16 block,
// lane i of a row of 16 holding row i: at step J the entry of row J is final and
// every row below subtracts its multiple (lr[J] is zero for rows i <= J).
template <int J>
struct DiagSolve {
  __device__ static __forceinline__ void run(const float (&lr)[16], float& a0, float& a1) {
    const float x0 = row_bcast<J>(a0), x1 = row_bcast<J>(a1);
    a0 = fmaf(-lr[J], x0, a0);
    a1 = fmaf(-lr[J], x1, a1);
    DiagSolve<J + 1>::run(lr, a0, a1);
  }
};
template <>
struct DiagSolve<16> {
  __device__ static __forceinline__ void run(const float (&)[16], float&, float&) {}
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// MFMA operand from a row-major [contraction][column] bf16 matrix in LDS, through
// the transposing LDS read (ds_read_b64_tr_b16): lane (l16, lq) receives
// X[c0 + 8 lq + e][n0 + l16], e = 0..7. Within a group of 16 lanes, lane 4a + b of
// the result takes element b of the rows addressed by lanes a, a + 4, a + 8, a + 12,
// so lane j of group g addresses row c0 + 8g + j/4 (+4 for the second half) at
// column n0 + 4 (j % 4).
__device__ __forceinline__ bf16x8 ld_tr8(const uint16_t* X, int pitch, int c0, int n0) {
  const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  const uint16_t* p = X + (c0 + 8 * g + (j >> 2)) * pitch + n0 + 4 * (j & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * pitch));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}


// Row-major bf16 [contraction][128] tiles that are read both transposed (ld_tr8) and by
// rows (ld8) are stored at a pitch of PS = 144 with column c of every row that has bit 3
// set at c ^ 72. In each group of 16 lanes a transposed read takes 4 rows at 8-bank steps
// and its groups are 8 rows apart: bit 6 of the swap moves those by 32 banks. A row read
// takes 16 consecutive rows, r and r + 8 on the same banks without the swap: bit 3 moves
// them by 4 banks. Both swaps move whole 8-column pieces, so every access stays one piece.
constexpr int PS = kD + 16;
__device__ __forceinline__ int swz(int row) { return (row & 8) * 9; }
__device__ __forceinline__ int sw_off(int row, int col) { return row * PS + (col ^ swz(row)); }

// ld_tr8 from a tile stored with swz: lane (l16, lq) receives X[c0 + 8 lq + e][n0 + l16]
__device__ __forceinline__ bf16x8 ld_tr8s(const uint16_t* X, int c0, int n0) {
  const int lane = threadIdx.x & 63, j = lane & 15, g = lane >> 4;
  const int row = c0 + 8 * g + (j >> 2);
  const uint16_t* p = X + sw_off(row, n0 + 4 * (j & 3));
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * PS));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Key order of a bf16 [..][128] tile whose rows meet, in one MFMA operand, four keys from
// each 16-key half of a 32-key block (the order of a state tile held in fp32 accumulators,
// rows = keys): key 32 ks + 16 h + 4 a + b at column 32 ks + 8 a + 4 h + b, so that the
// eight keys {32 ks + 4 a + e, 32 ks + 16 + 4 a + e} (e < 4) are one 16-byte piece
__device__ __forceinline__ int qcol(int key) {
  return (key & ~31) | ((key & 12) << 1) | ((key & 16) >> 2) | (key & 3);
}

// lower-triangle 16 x 16 tile pairs (rb, cb), cb <= rb
__device__ __forceinline__ void tri_pair(int p, int& rb, int& cb) {
  rb = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
  cb = p - (rb * (rb + 1)) / 2;
}

constexpr int PL = 17;   // fp32 pitch of the 16 x 16 blocks of the triangular inverse

typedef short s16x4 __attribute__((ext_vector_type(4)));
// bf16 16 x 16 x 16: lane l holds A[l%16][4(l/16) + e], B[4(l/16) + e][l%16]; D[4(l/16)+i][l%16]
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4 bf4(f32x4 x) {
  return __builtin_bit_cast(s16x4, u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])});
}
__device__ __forceinline__ s16x4 ld4(const uint16_t* p) {
  return __builtin_bit_cast(s16x4, *reinterpret_cast<const u32x2*>(p));
}
__device__ __forceinline__ int tri(int I, int J) { return I * (I + 1) / 2 + J; }   // lower block (I, J), J <= I


}  // namespace gdc
}  // namespace gdnrt

// Device helpers shared by the gfx950 kernels: bf16 conversion, MFMA tiles,
// wavefront reductions and the tiled layout of the compressed factors.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ap {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // raw bfloat16 payload

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // running-max start: finite so exp2 never sees inf - inf

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

// float -> bfloat16, round to nearest, ties to even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}
// Two floats -> two bfloat16 packed in one dword (lo = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const v2f x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, v2bf));
}

template <class T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) { return bf16_to_f32(x); }

template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// Order-preserving map of a float score to an unsigned key (larger score -> larger key).
// -0 is folded onto +0 so that equal scores give equal keys.
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  // negative: all bits flipped; otherwise only the sign bit set
  const uint32_t neg = static_cast<uint32_t>(static_cast<int32_t>(u) >> 31);
  return u ^ (neg | 0x80000000u);
}

// All ones when bit i of m is set, else zero (a select without a lane mask register).
__device__ __forceinline__ uint32_t bit_mask(uint32_t m, int i) {
  return static_cast<uint32_t>(-static_cast<int32_t>((m >> i) & 1u));
}

// 2^x with the hardware v_exp_f32 alone (exp2f adds a range check and rescale for
// results below 2^-126, which softmax weights can ignore): exp2(-inf) = 0.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- MFMA tiles
// 16x16 output tile D[i][j]: lane l holds D[4*(l/16) + t][l%16], t = 0..3.
// bf16 16x16x16: lane l supplies A[l%16][4*(l/16) + e] and B[4*(l/16) + e][l%16], e = 0..3.
__device__ __forceinline__ v4f mfma_bf16(v4s a, v4s b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// bf16 16x16x32 (gfx950): lane l supplies 8 k-values of row/column l%16 for its lane
// group l/16; A and B use the same k-slot assignment, so any token order works as long
// as the two operands agree.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v4f mfma_bf16_k32(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp32 16x16x4: lane l supplies A[l%16][l/16] and B[l/16][l%16].
__device__ __forceinline__ v4f mfma_f32(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, kWave));
}

// Maximum over the four lanes l%16 + 16k (the same column of a 16x16 tile), with the
// gfx950 lane swaps: permlane16 pairs rows 0/1 and 2/3, permlane32 pairs the two halves.
__device__ __forceinline__ float column_max4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// DPP lane moves inside a row of 16 lanes (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Sum over aligned groups of n lanes (n = 1, 2, 4, 8, 16, 32 or 64); every lane of a
// group gets the group's sum.  Within a 16-lane row: quad swaps, then half-row and
// row mirrors (sums are order-free, so mirrors serve as well as xor swaps).
__device__ __forceinline__ float group_sum(float v, int n) {
  if (n >= 2) v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]
  if (n >= 4) v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
  if (n >= 8) v += dpp_f32<0x141>(v);   // row_half_mirror
  if (n >= 16) v += dpp_f32<0x140>(v);  // row_mirror
  if (n >= 32) v += __shfl_xor(v, 16, kWave);
  if (n >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// ---------------------------------------------------------------- factor tiling
// A factor U (N x r) is stored per sequence as panels of 16 columns and blocks of
// 32 tokens.  Block (panel p, token block t) holds 512 elements laid out
// [lane 0..63][half 0..1][e 0..3]; lane l loads its 8 elements with one vector load.
//   K-layout (score operand A, rows = tokens):
//     token = 32t + 16*half + l%16,        column = 16p + 4*(l/16) + e
//   V-layout (value operand A^T, rows = columns of U):
//     token = 32t + 16*half + 4*(l/16) + e, column = 16p + l%16
// U_k and U_v share one buffer, block-major: for sequence b and token block t the NP
// K panels are followed by the NP V panels, so the 2*NP KB one 32-token step of the
// flash-decode kernel reads are contiguous.  With U_v = U_k + NP*512 elements,
// panel p of block t of sequence b starts at element ((b*nblk + t)*2*NP + p)*512 of
// either base.
constexpr int kBlockTok = 32;
constexpr int kBlockElems = 512;

__host__ __device__ __forceinline__ size_t tile_base(int b, int p, int t, int NP, int nblk) {
  return (((size_t)b * nblk + t) * 2 * NP + p) * kBlockElems;
}

// Element index inside a block of (lane, half, e).
__host__ __device__ __forceinline__ int tile_elem(int lane, int half, int e) {
  return (lane * 2 + half) * 4 + e;
}

}  // namespace ap

// 4-bit token factors: codes, block scales, their tiled layout, and the operand
// expansion the decode kernels use.
//
// The pages say the method composes with 4-bit quantization of the cache ([es §3
// "Integración Modular"], [fr §4 "Compatibilité"], [de §3 "Kombinierbarkeit"]) and
// warn that plain quantization suffers from outliers ([fr §1 "Limites des solutions
// existantes"]).  Format used here (no format is given on the pages):
//   * only U is quantized; B stays bf16;
//   * one scale per (32-token block, column): scale = bf16_rne(fp32(max|x|) *
//     fp32(1/7)); code = x / scale rounded to nearest, ties to even, in [-7, 7]
//     (scale 0 gives code 0); the stored value is code * scale;
//   * a lane's 8 elements of a tiled panel (the K or V layout of device_common.h) sit
//     in one 32-bit word as nibbles holding code + 8: element 2j at bits 4j..4j+3,
//     element 2j+1 at bits 16+4j..16+4j+3, so (word >> 4j) & 0x000F000F puts the pair
//     in the low bits of two bf16 halves;
//   * a panel is 256 bytes; U_k and U_v keep the block-major order of the bf16 layout
//     (byte offset = element offset / 2);
//   * scales: bf16 [B][nblk][2 (K, V)][r_pad], the column c = 16p + 4g + e stored at
//     g*4*NP + 4p + e, so a lane group g finds the scales of its columns (the same
//     columns in both layouts' MFMA operands) in one contiguous run.
#pragma once
#include <type_traits>

#include "device_common.h"

namespace ap {

struct i4_t {   // storage tag: pointers of this type count bytes of packed codes
  uint8_t raw;
};

constexpr int kQMax = 7;

// Element type of B (and of the dense tokens): the storage type, bf16 for 4-bit U.
template <class T>
using StoreB = typename std::conditional<std::is_same<T, i4_t>::value, bf16_t, T>::type;

__device__ __forceinline__ const i4_t* tile_ptr(const i4_t* base, size_t elem) { return base + elem / 2; }
__device__ __forceinline__ i4_t* tile_ptr(i4_t* base, size_t elem) { return base + elem / 2; }
template <class T>
__device__ __forceinline__ const T* tile_ptr(const T* base, size_t elem) { return base + elem; }

// Scale index of column c inside a block's K or V row of r_pad scales.
__host__ __device__ __forceinline__ int scale_slot(int c, int NP) {
  return ((c & 15) >> 2) * 4 * NP + 4 * (c >> 4) + (c & 3);
}

// Scale of a column whose largest magnitude is m.
__device__ __forceinline__ float q4_scale(float m) {
  return bf16_to_f32(f32_to_bf16(__fmul_rn(m, 1.0f / 7.0f)));
}

// Exact round-half-even of x / s in [-7, 7]: every midpoint (j + 1/2) s is exact in
// fp32 (s has 8 significant bits), so comparing against them decides exactly.
__device__ __forceinline__ int q4_code(float x, float s) {
  if (!(s > 0.f)) return 0;
  const float a = fabsf(x);
  int k = 0;
#pragma unroll
  for (int j = 0; j < kQMax; ++j) {
    const float mid = __fmul_rn(static_cast<float>(j) + 0.5f, s);
    k += (a > mid || (a == mid && (j & 1))) ? 1 : 0;
  }
  return x < 0.f ? -k : k;
}

// Nibble position of element i (0..7) of a lane's word.
__host__ __device__ __forceinline__ int q4_shift(int i) { return (i & 1) ? 16 + 2 * (i - 1) : 2 * i; }

// bf16 bits of 136 + code for a lane's 8 elements (an exact small integer: 128 + nibble).
__device__ __forceinline__ uint4 q4_expand(uint32_t w) {
  return make_uint4(0x43004300u | (w & 0x000F000Fu), 0x43004300u | ((w >> 4) & 0x000F000Fu),
                    0x43004300u | ((w >> 8) & 0x000F000Fu), 0x43004300u | ((w >> 12) & 0x000F000Fu));
}
// bf16 -136 in every element: the offset the expanded codes carry, cancelled by one more
// product with the same other operand.
constexpr uint32_t kQ4NegOffset2 = 0xC308C308u;
constexpr float kQ4Offset = 136.f;

// Quantize and store one 32-token block of one factor (K or V layout).  Ub: LDS
// [32][ld] fp32 values (rows >= ntok and columns >= r zero), written by the caller
// before a barrier; scl: LDS scratch of r_pad floats.  Every thread of the workgroup
// calls this.  tiles: the block's first panel (K or V); srow: the block's K or V
// scale row.
template <bool VL>
__device__ void q4_store_block(const float* Ub, int ld, int NP, i4_t* tiles, bf16_t* srow,
                               float* scl) {
  const int rp = 16 * NP;
  for (int c = threadIdx.x; c < rp; c += blockDim.x) {
    float m = 0.f;
    for (int t = 0; t < kBlockTok; ++t) m = fmaxf(m, fabsf(Ub[t * ld + c]));
    const float s = q4_scale(m);
    scl[c] = s;
    srow[scale_slot(c, NP)] = f32_to_bf16(s);
  }
  __syncthreads();
  uint32_t* wout = reinterpret_cast<uint32_t*>(tiles);
  for (int idx = threadIdx.x; idx < NP * 64; idx += blockDim.x) {
    const int p = idx >> 6, lane = idx & 63;
    uint32_t w = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int half = i >> 2, e = i & 3;
      int token, col;
      if (!VL) {
        token = 16 * half + (lane & 15);
        col = 16 * p + 4 * (lane >> 4) + e;
      } else {
        token = 16 * half + 4 * (lane >> 4) + e;
        col = 16 * p + (lane & 15);
      }
      const uint32_t nib = static_cast<uint32_t>(q4_code(Ub[token * ld + col], scl[col]) + 8);
      w |= nib << q4_shift(i);
    }
    wout[p * 64 + lane] = w;
  }
}

}  // namespace ap

// MFMA operand tiles shared by the decode kernels: one lane's slice of a tiled
// factor block, split latent-query operands, probability operands, and the two
// 16x16 tile products (scores and latent values).
#pragma once
#include <type_traits>

#include "device_common.h"
#include "quant4.h"

namespace ap {

// ---------------------------------------------------------------- operand loads
// The 8 elements of one lane in one tiled block: half 0 = elements 0..3, half 1 = 4..7.
template <class T> struct LaneTile;
template <> struct LaneTile<bf16_t> {
  uint4 raw;
  __device__ __forceinline__ void load(const bf16_t* base, int lane) {
    raw = *reinterpret_cast<const uint4*>(base + lane * 8);
  }
  __device__ __forceinline__ v4s half(int hf) const {
    uint2 w = hf == 0 ? make_uint2(raw.x, raw.y) : make_uint2(raw.z, raw.w);
    return __builtin_bit_cast(v4s, w);
  }
};
template <> struct LaneTile<float> {
  float4 h0, h1;
  __device__ __forceinline__ void load(const float* base, int lane) {
    const float4* p = reinterpret_cast<const float4*>(base + lane * 8);
    h0 = p[0];
    h1 = p[1];
  }
  __device__ __forceinline__ float4 half(int hf) const { return hf == 0 ? h0 : h1; }
};

// 4-bit codes: one 32-bit word per lane, expanded to bf16 (136 + code) for the MFMA.
template <> struct LaneTile<i4_t> {
  uint32_t w;
  __device__ __forceinline__ void load(const i4_t* base, int lane) {
    w = reinterpret_cast<const uint32_t*>(base)[lane];
  }
  __device__ __forceinline__ uint4 deq() const { return q4_expand(w); }
};

// Four bf16 block scales (one lane's columns of one panel) as floats.
__device__ __forceinline__ void q4_scales(uint2 x, float (&s)[4]) {
  s[0] = __uint_as_float(x.x << 16);
  s[1] = __uint_as_float(x.x & 0xFFFF0000u);
  s[2] = __uint_as_float(x.y << 16);
  s[3] = __uint_as_float(x.y & 0xFFFF0000u);
}

// A latent-query operand: 4 values (one lane's k-slice) split for the dtype's MFMA.
template <class T> struct QOp;
template <> struct QOp<bf16_t> {
  v4s hi, lo;  // q = hi + lo: keeps ~16 significant bits through bf16 MFMA
  __device__ __forceinline__ void set(const float v[4]) {
    for (int e = 0; e < 4; ++e) {
      bf16_t h = f32_to_bf16(v[e]);
      hi[e] = static_cast<short>(h);
      lo[e] = static_cast<short>(f32_to_bf16(v[e] - bf16_to_f32(h)));
    }
  }
  __device__ __forceinline__ QOp masked(int lane_cols_lo, int lim, bool keep_below) const {
    // zero the elements whose column (lane_cols_lo + e) is on the wrong side of lim
    QOp o = *this;
    for (int e = 0; e < 4; ++e) {
      bool below = lane_cols_lo + e < lim;
      if (below != keep_below) { o.hi[e] = 0; o.lo[e] = 0; }
    }
    return o;
  }
};
template <> struct QOp<float> {
  float v[4];
  __device__ __forceinline__ void set(const float x[4]) {
    for (int e = 0; e < 4; ++e) v[e] = x[e];
  }
  __device__ __forceinline__ QOp masked(int lane_cols_lo, int lim, bool keep_below) const {
    QOp o = *this;
    for (int e = 0; e < 4; ++e) {
      bool below = lane_cols_lo + e < lim;
      if (below != keep_below) o.v[e] = 0.f;
    }
    return o;
  }
};

// D += A(tokens x 16 cols of one panel, one half) * q(16 cols x 16 heads)
__device__ __forceinline__ v4f score_mma(const LaneTile<bf16_t>& a, int hf, const QOp<bf16_t>& q, v4f acc) {
  v4s x = a.half(hf);
  acc = mfma_bf16(x, q.hi, acc);
  return mfma_bf16(x, q.lo, acc);
}
__device__ __forceinline__ v4f score_mma(const LaneTile<float>& a, int hf, const QOp<float>& q, v4f acc) {
  float4 x = a.half(hf);
  acc = mfma_f32(x.x, q.v[0], acc);
  acc = mfma_f32(x.y, q.v[1], acc);
  acc = mfma_f32(x.z, q.v[2], acc);
  return mfma_f32(x.w, q.v[3], acc);
}

// Probability operand (16 tokens x 16 heads): lane holds tokens 4*(l/16)+t of head l%16.
template <class T> struct POp;
template <> struct POp<bf16_t> {
  v4s v;
  __device__ __forceinline__ void set(const float p[4]) {
    const uint2 w = make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
    v = __builtin_bit_cast(v4s, w);
  }
};
template <> struct POp<float> {
  float v[4];
  __device__ __forceinline__ void set(const float p[4]) {
    for (int t = 0; t < 4; ++t) v[t] = p[t];
  }
};

// Z^T(16 latent cols x 16 heads) += U_v^T(16 cols x 16 tokens of one half) * P(16 tokens x 16 heads)
__device__ __forceinline__ v4f value_mma(const LaneTile<bf16_t>& a, int hf, bool keep, const POp<bf16_t>& p, v4f acc) {
  v4s x = a.half(hf);
  if (!keep) x = v4s{0, 0, 0, 0};
  return mfma_bf16(x, p.v, acc);
}
__device__ __forceinline__ v4f value_mma(const LaneTile<float>& a, int hf, bool keep, const POp<float>& p, v4f acc) {
  float4 x = a.half(hf);
  if (!keep) x = make_float4(0.f, 0.f, 0.f, 0.f);
  acc = mfma_f32(x.x, p.v[0], acc);
  acc = mfma_f32(x.y, p.v[1], acc);
  acc = mfma_f32(x.z, p.v[2], acc);
  return mfma_f32(x.w, p.v[3], acc);
}

// 16 bytes of storage elements read with one vector load.
template <class T> struct Vec16;   // 16 bytes of storage elements
// load_nt: a non-temporal load, for rows a workgroup reads once, so that they do not
// push the token factors (which the head groups of a sequence re-read) out of L2.
template <> struct Vec16<bf16_t> {
  static constexpr int n = 8;
  uint4 raw;
  __device__ __forceinline__ void load(const bf16_t* p) { raw = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void load_nt(const bf16_t* p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    raw = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
  }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t w = e < 2 ? raw.x : (e < 4 ? raw.y : (e < 6 ? raw.z : raw.w));
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};
template <> struct Vec16<float> {
  static constexpr int n = 4;
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void load_nt(const float* p) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    v = __builtin_bit_cast(float4, __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)));
  }
  __device__ __forceinline__ float get(int e) const { return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w)); }
};

}  // namespace ap

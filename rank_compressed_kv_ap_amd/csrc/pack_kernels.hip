// Conversion between the plain factor layout U [B][N][r] (row-major, as in the
// page's K ~= K* D_k, [fr §2.A "Mécanisme"]) and the tiled layouts the decode
// kernels read with one vector load per lane (see device_common.h), including the
// 4-bit layout (quant4.h), whose codes are chosen here from fp32 rows.
#include "ap_internal.h"
#include "device_common.h"
#include "quant4.h"

namespace ap {

// (token, column) of element `within` of a tiled block.
template <bool VL>
__device__ __forceinline__ void tile_coord(int t, int p, int within, int& token, int& col) {
  const int e = within & 3, half = (within >> 2) & 1, lane = within >> 3;
  if (!VL) {
    token = kBlockTok * t + 16 * half + (lane & 15);
    col = 16 * p + 4 * (lane >> 4) + e;
  } else {
    token = kBlockTok * t + 16 * half + 4 * (lane >> 4) + e;
    col = 16 * p + (lane & 15);
  }
}

template <class T, bool VL>
__global__ __launch_bounds__(256) void k_pack_u(const T* __restrict__ src, T* __restrict__ dst,
                                                int B, int N, int r, int NP, int nblk) {
  const size_t total = (size_t)B * NP * nblk * kBlockElems;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int within = static_cast<int>(idx % kBlockElems);
    const size_t blk = idx / kBlockElems;
    const int t = static_cast<int>(blk % nblk);
    const size_t bp = blk / nblk;
    const int p = static_cast<int>(bp % NP);
    const int b = static_cast<int>(bp / NP);
    int token, col;
    tile_coord<VL>(t, p, within, token, col);
    T v = T(0);
    if (token < N && col < r) v = src[((size_t)b * N + token) * r + col];
    dst[tile_base(b, p, t, NP, nblk) + within] = v;
  }
}

template <class T, bool VL>
__global__ __launch_bounds__(256) void k_unpack_u(const T* __restrict__ src, T* __restrict__ dst,
                                                  int B, int N, int r, int NP, int nblk) {
  const size_t total = (size_t)B * N * r;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int c = static_cast<int>(idx % r);
    const size_t bn = idx / r;
    const int n = static_cast<int>(bn % N);
    const int b = static_cast<int>(bn / N);
    const int t = n / kBlockTok, nn = n % kBlockTok, half = nn >> 4;
    const int p = c >> 4, cc = c & 15;
    int lane, e;
    if (!VL) {
      lane = (cc >> 2) * 16 + (nn & 15);
      e = cc & 3;
    } else {
      const int rem = nn & 15;
      lane = (rem >> 2) * 16 + cc;
      e = rem & 3;
    }
    dst[idx] = src[tile_base(b, p, t, NP, nblk) + tile_elem(lane, half, e)];
  }
}

static dim3 grid_for(size_t total) {
  size_t g = (total + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return dim3(static_cast<unsigned>(g));
}

template <class T>
static hipError_t pack_t(const ap_cache* c, const void* src, void* dst, bool vl, bool unpack,
                         hipStream_t st) {
  const Dims& dm = c->dm;
  if (!unpack) {
    const size_t total = (size_t)dm.B * dm.NP * dm.nblk * kBlockElems;
    if (vl)
      hipLaunchKernelGGL((k_pack_u<T, true>), grid_for(total), dim3(256), 0, st,
                         static_cast<const T*>(src), static_cast<T*>(dst), dm.B, dm.N, dm.r, dm.NP, dm.nblk);
    else
      hipLaunchKernelGGL((k_pack_u<T, false>), grid_for(total), dim3(256), 0, st,
                         static_cast<const T*>(src), static_cast<T*>(dst), dm.B, dm.N, dm.r, dm.NP, dm.nblk);
  } else {
    const size_t total = (size_t)dm.B * dm.N * dm.r;
    if (vl)
      hipLaunchKernelGGL((k_unpack_u<T, true>), grid_for(total), dim3(256), 0, st,
                         static_cast<const T*>(src), static_cast<T*>(dst), dm.B, dm.N, dm.r, dm.NP, dm.nblk);
    else
      hipLaunchKernelGGL((k_unpack_u<T, false>), grid_for(total), dim3(256), 0, st,
                         static_cast<const T*>(src), static_cast<T*>(dst), dm.B, dm.N, dm.r, dm.NP, dm.nblk);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- 4-bit factors
// One workgroup per (sequence, token block): the fp32 rows of U [B][N][r] are staged in
// LDS, then quantized and stored in the tiled 4-bit layout with their block scales.
template <bool VL>
__global__ __launch_bounds__(256) void k_pack_u4(const float* __restrict__ src, i4_t* __restrict__ dst,
                                                 bf16_t* __restrict__ scales, int N, int r, int NP,
                                                 int nblk) {
  extern __shared__ __align__(16) float sh[];
  const int rp = 16 * NP, ld = rp + 1;
  float* Ub = sh;               // [32][ld]
  float* scl = Ub + 32 * ld;    // [rp]
  const int b = blockIdx.x / nblk, t = blockIdx.x % nblk;
  for (int idx = threadIdx.x; idx < 32 * rp; idx += blockDim.x) {
    const int rr = idx / rp, col = idx % rp, token = kBlockTok * t + rr;
    Ub[rr * ld + col] = (token < N && col < r) ? src[((size_t)b * N + token) * r + col] : 0.f;
  }
  __syncthreads();
  q4_store_block<VL>(Ub, ld, NP, tile_ptr(dst, tile_base(b, 0, t, NP, nblk)),
                     scales + (((size_t)b * nblk + t) * 2 + (VL ? 1 : 0)) * rp, scl);
}

// Dequantized values code * scale back to the plain fp32 layout.
template <bool VL>
__global__ __launch_bounds__(256) void k_unpack_u4(const i4_t* __restrict__ src,
                                                   const bf16_t* __restrict__ scales,
                                                   float* __restrict__ dst, int B, int N, int r,
                                                   int NP, int nblk) {
  const size_t total = (size_t)B * N * r;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int c = static_cast<int>(idx % r);
    const size_t bn = idx / r;
    const int n = static_cast<int>(bn % N);
    const int b = static_cast<int>(bn / N);
    const int t = n / kBlockTok, nn = n % kBlockTok, half = nn >> 4;
    const int p = c >> 4, cc = c & 15;
    int lane, e;
    if (!VL) {
      lane = (cc >> 2) * 16 + (nn & 15);
      e = cc & 3;
    } else {
      const int rem = nn & 15;
      lane = (rem >> 2) * 16 + cc;
      e = rem & 3;
    }
    const uint32_t w = reinterpret_cast<const uint32_t*>(tile_ptr(src, tile_base(b, p, t, NP, nblk)))[lane];
    const int code = static_cast<int>((w >> q4_shift(4 * half + e)) & 0xFu) - 8;
    const float s = bf16_to_f32(scales[(((size_t)b * nblk + t) * 2 + (VL ? 1 : 0)) * 16 * NP + scale_slot(c, NP)]);
    dst[idx] = static_cast<float>(code) * s;
  }
}

static hipError_t pack_u4(const ap_cache* c, const void* src, void* dst, bool vl, bool unpack,
                          hipStream_t st) {
  const Dims& dm = c->dm;
  if (!unpack) {
    const size_t lds = (32 * (dm.r_pad + 1) + dm.r_pad) * sizeof(float);
    if (vl)
      hipLaunchKernelGGL(k_pack_u4<true>, dim3(dm.B * dm.nblk), dim3(256), lds, st,
                         static_cast<const float*>(src), static_cast<i4_t*>(dst),
                         reinterpret_cast<bf16_t*>(c->Usc), dm.N, dm.r, dm.NP, dm.nblk);
    else
      hipLaunchKernelGGL(k_pack_u4<false>, dim3(dm.B * dm.nblk), dim3(256), lds, st,
                         static_cast<const float*>(src), static_cast<i4_t*>(dst),
                         reinterpret_cast<bf16_t*>(c->Usc), dm.N, dm.r, dm.NP, dm.nblk);
  } else {
    const size_t total = (size_t)dm.B * dm.N * dm.r;
    if (vl)
      hipLaunchKernelGGL(k_unpack_u4<true>, grid_for(total), dim3(256), 0, st,
                         static_cast<const i4_t*>(src), reinterpret_cast<const bf16_t*>(c->Usc), static_cast<float*>(dst), dm.B, dm.N,
                         dm.r, dm.NP, dm.nblk);
    else
      hipLaunchKernelGGL(k_unpack_u4<false>, grid_for(total), dim3(256), 0, st,
                         static_cast<const i4_t*>(src), reinterpret_cast<const bf16_t*>(c->Usc), static_cast<float*>(dst), dm.B, dm.N,
                         dm.r, dm.NP, dm.nblk);
  }
  return hipGetLastError();
}

hipError_t launch_pack_u(const ap_cache* c, const void* src, void* dst, bool v_layout, hipStream_t st) {
  if (c->dm.storage == AP_INT4) return pack_u4(c, src, dst, v_layout, false, st);
  if (c->dm.storage == AP_BF16) return pack_t<bf16_t>(c, src, dst, v_layout, false, st);
  return pack_t<float>(c, src, dst, v_layout, false, st);
}

hipError_t launch_unpack_u(const ap_cache* c, const void* src, void* dst, bool v_layout, hipStream_t st) {
  if (c->dm.storage == AP_INT4) return pack_u4(c, src, dst, v_layout, true, st);
  if (c->dm.storage == AP_BF16) return pack_t<bf16_t>(c, src, dst, v_layout, true, st);
  return pack_t<float>(c, src, dst, v_layout, true, st);
}

}  // namespace ap

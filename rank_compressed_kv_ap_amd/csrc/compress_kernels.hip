// Randomized low-rank factorisation of the heads-merged K and V caches (gfx950).
//
// [fr §2.A "Approche"/"Mécanisme"], [es §2.A], [de §2.A "Technik"]: per sequence the
// keys of all heads form one N x W matrix A (heads concatenated along the hidden
// axis), compressed by a singular value decomposition into U (N x r) and B (r x W);
// K and V separately.  The SVD is reached by randomized subspace iteration (Halko,
// Martinsson & Tropp 2011) with ell = min(r + p, N, W) probe columns and q power
// iterations:
//   Y = A Omega; Q = orth(Y); q times { Q~ = orth(A^T Q); Q = orth(A Q~) }
//   C^T = A^T Q = Qc R;  R^T = P Sigma S^T (one-sided Jacobi)
//   U = Q P[:, :r] Sigma_r,   B = (Qc S[:, :r])^T
// All 2B matrices of a batch are processed together, launch by launch.
//
// Kernels:
//   k_gemm_n / k_gemm_t   Y = A X, Y = A^T X (X given transposed, k contiguous); bf16 MFMA
//                         16x16x32 with A tiles staged in LDS (transposed for A^T); fp32 out
//   k_gram / k_chol       Gram Y^T Y (fp32 MFMA, split over rows), shifted Cholesky,
//                         inverse of the triangular factor
//   k_apply               Q = Y R^-1 in place (fp32 MFMA), plus Q^T in storage precision
//   k_jacobi              one-sided Jacobi SVD of R^T in LDS, components sorted by sigma
//   k_assemble_u / _b     factors in the decode layouts
//   k_omega_*             the test matrix: copied from the caller, or random signs from
//                         Philox4x32-10 (Salmon et al., SC'11) keyed by the seed
#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <type_traits>

#include "ap_internal.h"
#include "device_common.h"
#include "quant4.h"

namespace ap {

constexpr int kMaxEll = 144;          // largest ell: 9 column tiles of 16; the Cholesky and the
                                      // core SVD keep one ell x ell matrix per workgroup in LDS

// ---------------------------------------------------------------- workspace
struct CompressWs {
  int nmat, M, ellp;                  // matrices, max(N, W), ell padded to 16
  void* omT = nullptr;                // [nmat][ellp][W]   storage dtype
  float* Y = nullptr;                 // [nmat][M][ellp]   products, then orthonormal bases
  void* XT = nullptr;                 // [nmat][ellp][M]   basis transposed, storage dtype
  void* XTlo = nullptr;               // [nmat][ellp][M]   its rounding remainder (bf16 only)
  float* Qn = nullptr;                // [nmat][N][ellp]   final range basis of A
  float* Qc = nullptr;                // [nmat][W][ellp]   basis of C^T
  float* Gpart = nullptr;             // [nmat][nsplit][ellp][ellp] partial Grams
  float* Gsum = nullptr;              // [nmat][ellp][ellp] their sum
  float* Rinv = nullptr;              // [nmat][ellp][ellp]
  float* Racc = nullptr;              // [nmat][ellp][ellp] R of the last orthonormalisation
  float* PS = nullptr;                // [nmat][ellp][ellp] P Sigma (columns sorted)
  float* Sv = nullptr;                // [nmat][ellp][ellp] S (columns sorted)
  float* sig = nullptr;               // [nmat][ellp]
};

// ================================================================ test matrix
// Philox4x32-10 (Salmon, Moraes, Dror & Shaw, SC'11): counter-based, 10 rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint2 k) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = M0 * c.x, hi0 = __umulhi(M0, c.x);
    const uint32_t lo1 = M1 * c.z, hi1 = __umulhi(M1, c.z);
    c = make_uint4(hi1 ^ c.y ^ k.x, lo1, hi0 ^ c.w ^ k.y, lo0);
    k.x += W0;
    k.y += W1;
  }
  return c;
}

// Omega^T[mat][j][w]: element (w, j) of the W x ell random-sign test matrix of
// matrix mat (sub-Gaussian test matrices: Halko, Martinsson & Tropp 2011, §4.6).
// Linear index i = j*W + w; one Philox call with counter (i/128, mat, 0, 0) and key
// (seed lo, seed hi) yields 128 bits for elements 128*(i/128) ..; bit i%32 of word
// (i/32)%4 set means -1.  One thread per 8 consecutive elements (the 16 threads of
// a 128-element block each evaluate its Philox call).
template <class T>
__global__ __launch_bounds__(256) void k_omega_philox(T* __restrict__ omT, int nmat, int W, int ell,
                                                      int ellp, uint64_t seed) {
  // grid: x over the 8-element groups of one matrix, y over the matrices (32-bit
  // indices: ell * W is far below 2^31)
  const int per = ell * W;
  const int groups = (per + 7) / 8;
  const int mat = blockIdx.y;
  const uint2 key = make_uint2(static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
  for (int g = blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += gridDim.x * blockDim.x) {
    const int i0 = 8 * g;
    const uint4 x = philox4x32_10(make_uint4(static_cast<uint32_t>(i0 / 128), static_cast<uint32_t>(mat), 0u, 0u), key);
    const int t0 = i0 & 127;
    const uint32_t word = (t0 >> 5) == 0 ? x.x : ((t0 >> 5) == 1 ? x.y : ((t0 >> 5) == 2 ? x.z : x.w));
    const uint32_t bits = (word >> (t0 & 31)) & 0xffu;
    int j = i0 / W, w = i0 - (i0 / W) * W;
    const int cnt = per - i0 < 8 ? per - i0 : 8;
    T* dst = omT + ((size_t)mat * ellp + j) * W + w;
    if constexpr (std::is_same<T, bf16_t>::value) {
      if (cnt == 8 && w + 8 <= W && (W & 7) == 0) {   // 8 signs of one row: one 16-byte store
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          h[e] = (((bits >> (2 * e)) & 1u) ? 0xBF80u : 0x3F80u) | ((((bits >> (2 * e + 1)) & 1u) ? 0xBF80u : 0x3F80u) << 16);
        *reinterpret_cast<uint4*>(dst) = make_uint4(h[0], h[1], h[2], h[3]);
        continue;
      }
    }
    for (int t = 0; t < cnt; ++t) {
      omT[((size_t)mat * ellp + j) * W + w] = from_f32<T>(((bits >> t) & 1u) ? -1.f : 1.f);
      if (++w == W) { w = 0; ++j; }
    }
  }
}

// Caller's Omega [B][2][W][ell] float32 -> Omega^T[mat][j][w] in storage precision.
template <class T>
__global__ __launch_bounds__(256) void k_omega_copy(const float* __restrict__ om, T* __restrict__ omT,
                                                    int nmat, int W, int ell, int ellp) {
  const size_t total = (size_t)nmat * ell * W;
  for (size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (size_t)gridDim.x * blockDim.x) {
    const int mat = static_cast<int>(g / ((size_t)ell * W));
    const size_t rem = g % ((size_t)ell * W);
    const int j = static_cast<int>(rem / W), w = static_cast<int>(rem % W);
    omT[((size_t)mat * ellp + j) * W + w] = from_f32<T>(om[((size_t)mat * W + w) * ell + j]);
  }
}

// ================================================================ tall-skinny GEMMs
// Output Y[mat][m][j] (fp32, row stride ellp) for m in a BM-row tile (BM = 128 or 256,
// 32 rows per wavefront):
//   TRANS = false: Y = A X,   A [M][K] rows m, X^T [ellp][K]        (M = N, K = W)
//   TRANS = true : Y = A^T X, A [K][M] columns m, X^T [ellp][K]     (M = W, K = N)
// A 64-wide k slice of A is staged in LDS as [BM m][64 k] (transposed on the way in
// for TRANS), so both MFMA operands read 8 consecutive k values per lane.  The next
// slice of A and of X is loaded into registers while the current one is multiplied
// (software pipelining: the loads of slice s+1 are in flight during the MFMAs of s).
constexpr int kGemmBK = 64, kGemmLdsStride = kGemmBK + 8;  // padded bf16 row

// VEC (W and K multiples of 8, K >= 8): every load of a slice is issued unconditionally,
// clamped in bounds, so the compiler tracks the slice in flight exactly and waits only
// for the slice being staged.  Past the edge of K the X^T values are zeroed, which
// cancels the clamped (finite) A values they meet; A values past M only reach output
// rows that are not stored.  Otherwise per-element fallbacks for unaligned rows.
template <class T, bool TRANS, int NT, bool SPLIT, bool VEC, int BM>
__global__ __launch_bounds__(2 * BM) void k_gemm(const T* __restrict__ Kmat,
                                                        const T* __restrict__ Vmat,
                                                        const T* __restrict__ XT,
                                                        const T* __restrict__ XTlo, float* __restrict__ Y,
                                                        int N, int W, int ellp, size_t x_mat_stride,
                                                        int tiles_m) {
  static_assert(std::is_same<T, bf16_t>::value, "MFMA GEMM path is bf16");
  constexpr int GT = 2 * BM;                         // threads: 32 rows per wavefront
  constexpr int XR = NT * 16;                        // rows of X^T (= ellp)
  constexpr int CPR = kGemmBK / 8;                   // 16-byte chunks per k slice row
  constexpr int XU = (XR * CPR + GT - 1) / GT;   // 16-byte X loads per thread
  constexpr int AU = BM * CPR / GT;   // 16-byte A loads per thread
  constexpr int RPP = GT / CPR;            // A rows per pass (not TRANS)
  constexpr int MG = BM / 8;                    // 8-wide m groups of a k row (TRANS)
  static_assert(BM == 32 * (GT / 64) && AU * (GT / MG) == kGemmBK,
                "32 rows per wavefront; TRANS: AU k rows per thread cover the slice");
  __shared__ __align__(16) bf16_t As[BM * kGemmLdsStride];
  __shared__ __align__(16) bf16_t Xs[(SPLIT ? 2 : 1) * XR * kGemmLdsStride];
  // workgroups are dealt to the 8 XCDs in turn: when the matrices come in eights, the
  // row tiles of one matrix all land on one XCD, whose L2 then holds its X^T slices
  int mat, tile;
  if ((gridDim.x / tiles_m) % 8 == 0) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    mat = (slot / tiles_m) * 8 + xcd;
    tile = slot % tiles_m;
  } else {
    mat = blockIdx.x / tiles_m;
    tile = blockIdx.x % tiles_m;
  }
  const int m0 = tile * BM;
  const int b = mat >> 1;
  const T* A = ((mat & 1) ? Vmat : Kmat) + (size_t)b * N * W;
  const int M = TRANS ? W : N;
  const int K = TRANS ? N : W;
  const T* X = XT + (size_t)mat * x_mat_stride;
  const T* Xl = SPLIT ? XTlo + (size_t)mat * x_mat_stride : nullptr;
  const bool avec = (W & 7) == 0;   // 16-byte loads of A rows stay aligned
  const bool xvec = (K & 7) == 0;   // 16-byte loads of X^T rows stay aligned
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  // wave owns rows m0 + 32*wave .. +31 (two 16-row tiles) x NT column tiles
  v4f acc[2][NT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[i][c] = v4f{0, 0, 0, 0};

  // For TRANS the A tile is written as 8-byte pieces of rows 8 apart, which the padded
  // row stride maps onto the same LDS banks; the 16-byte chunk index of row r is then
  // XOR-ed with (r >> 3) & 7 on the write and on the read.
  auto achunk = [](int row, int chunk) { return TRANS ? (chunk ^ ((row >> 3) & 7)) : chunk; };
  auto pack8 = [](const uint16_t* t) {
    return make_uint4(t[0] | (uint32_t(t[1]) << 16), t[2] | (uint32_t(t[3]) << 16),
                      t[4] | (uint32_t(t[5]) << 16), t[6] | (uint32_t(t[7]) << 16));
  };
  // ---- one 64-wide k slice in registers: A (4 x 8 elements per thread) and X^T
  // (XU x 8 elements per thread), both staged in LDS before the MFMAs
  struct Slice {
    uint4 a[AU];
    uint4 x[XU];
    uint4 xl[SPLIT ? XU : 1];
  };
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
  auto load_slice = [&](int k0, Slice& sl) {
    if constexpr (VEC) {
      if (!TRANS) {
        // rows tid / CPR + RPP h, k = k0 + 8 (tid % CPR) .. +7 (a run lies wholly inside K or past it)
#pragma unroll
        for (int h = 0; h < AU; ++h) {
          const int row = tid / CPR + RPP * h, gk = k0 + (tid % CPR) * 8;
          const uint4 t = *reinterpret_cast<const uint4*>(A + (size_t)min(m0 + row, M - 1) * W + min(gk, K - 8));
          sl.a[h] = t;
        }
      } else {
        // k rows AU (tid / MG) + h, m = m0 + 8 (tid % MG) .. +7
#pragma unroll
        for (int h = 0; h < AU; ++h) {
          const int gk = k0 + AU * (tid / MG) + h, gm = m0 + (tid % MG) * 8;
          sl.a[h] = *reinterpret_cast<const uint4*>(A + (size_t)min(gk, K - 1) * W + min(gm, M - 8));
        }
      }
#pragma unroll
      for (int u = 0; u < XU; ++u) {
        const int idx = min(tid + u * GT, XR * CPR - 1);
        const int j = idx / CPR, gk = k0 + 8 * (idx % CPR);
        const size_t off = (size_t)j * K + min(gk, K - 8);
        const uint4 t = *reinterpret_cast<const uint4*>(X + off);
        sl.x[u] = gk < K ? t : z4;
        if constexpr (SPLIT) {
          const uint4 tl = *reinterpret_cast<const uint4*>(Xl + off);
          sl.xl[u] = gk < K ? tl : z4;
        }
      }
    } else {
    if (!TRANS) {
      // rows tid / CPR + RPP h, k = k0 + 8 (tid % CPR) .. +7
#pragma unroll
      for (int h = 0; h < AU; ++h) {
        const int row = tid / CPR + RPP * h, kk = (tid % CPR) * 8;
        const int gm = min(m0 + row, M - 1), gk = k0 + kk;
        if (avec && gk + 8 <= K) {
          sl.a[h] = *reinterpret_cast<const uint4*>(A + (size_t)gm * W + gk);
        } else {
          uint16_t t[8];
          for (int e = 0; e < 8; ++e) t[e] = gk + e < K ? A[(size_t)gm * W + gk + e] : bf16_t(0);
          sl.a[h] = pack8(t);
        }
      }
    } else {
      // k rows AU (tid / MG) + h, m = m0 + 8 (tid % MG) .. +7 (transposed into LDS later)
#pragma unroll
      for (int h = 0; h < AU; ++h) {
        const int kk = AU * (tid / MG) + h, mm = (tid % MG) * 8;
        const int gk = k0 + kk, gm = m0 + mm;
        if (avec && gk < K && gm + 8 <= M) {
          sl.a[h] = *reinterpret_cast<const uint4*>(A + (size_t)gk * W + gm);
        } else {
          uint16_t t[8];
          for (int e = 0; e < 8; ++e) t[e] = (gk < K && gm + e < M) ? A[(size_t)gk * W + gm + e] : bf16_t(0);
          sl.a[h] = pack8(t);
        }
      }
    }
    // X^T rows j = idx / 8, k = k0 + 8 (idx % 8) .. +7 (zero past K)
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int idx = min(tid + u * GT, XR * CPR - 1);
      const int j = idx / CPR, gk = k0 + 8 * (idx % CPR);
      const size_t off = (size_t)j * K + gk;
      if (xvec && gk + 8 <= K) {
        sl.x[u] = *reinterpret_cast<const uint4*>(X + off);
        if constexpr (SPLIT) sl.xl[u] = *reinterpret_cast<const uint4*>(Xl + off);
      } else {
        uint16_t t[8], tl[8];
        for (int e = 0; e < 8; ++e) {
          t[e] = gk + e < K ? X[off + e] : bf16_t(0);
          if constexpr (SPLIT) tl[e] = gk + e < K ? Xl[off + e] : bf16_t(0);
        }
        sl.x[u] = pack8(t);
        if constexpr (SPLIT) sl.xl[u] = pack8(tl);
      }
    }
    }
  };
  auto stage = [&](const Slice& sl) {
    if (!TRANS) {
#pragma unroll
      for (int h = 0; h < AU; ++h)
        *reinterpret_cast<uint4*>(&As[(tid / CPR + RPP * h) * kGemmLdsStride + (tid % CPR) * 8]) = sl.a[h];
    } else {
      // groups of 4 k rows x 8 m columns in registers -> 8 columns of 4 consecutive k (8 bytes)
#pragma unroll
      for (int q = 0; q < AU / 4; ++q) {
        const int kk = AU * (tid / MG) + 4 * q, mm = (tid % MG) * 8;
        const uint4 a0 = sl.a[4 * q], a1 = sl.a[4 * q + 1], a2 = sl.a[4 * q + 2], a3 = sl.a[4 * q + 3];
        const uint32_t r0[4] = {a0.x, a0.y, a0.z, a0.w};
        const uint32_t r1[4] = {a1.x, a1.y, a1.z, a1.w};
        const uint32_t r2[4] = {a2.x, a2.y, a2.z, a2.w};
        const uint32_t r3[4] = {a3.x, a3.y, a3.z, a3.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint2 ev = make_uint2((r0[c] & 0xffffu) | (r1[c] << 16), (r2[c] & 0xffffu) | (r3[c] << 16));
          const uint2 od = make_uint2((r0[c] >> 16) | (r1[c] & 0xffff0000u), (r2[c] >> 16) | (r3[c] & 0xffff0000u));
          const int re = mm + 2 * c, ro = re + 1;   // 16-byte chunk kk / 8, 8-byte half (kk / 4) & 1
          *reinterpret_cast<uint2*>(&As[re * kGemmLdsStride + 8 * achunk(re, kk >> 3) + (kk & 4)]) = ev;
          *reinterpret_cast<uint2*>(&As[ro * kGemmLdsStride + 8 * achunk(ro, kk >> 3) + (kk & 4)]) = od;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int idx = min(tid + u * GT, XR * CPR - 1);
      const int o = (idx / CPR) * kGemmLdsStride + 8 * (idx % CPR);
      *reinterpret_cast<uint4*>(&Xs[o]) = sl.x[u];
      if constexpr (SPLIT) *reinterpret_cast<uint4*>(&Xs[XR * kGemmLdsStride + o]) = sl.xl[u];
    }
  };

  auto multiply = [&]() {
#pragma unroll
    for (int s2 = 0; s2 < kGemmBK / 32; ++s2) {
      v8bf ab[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 32 * wave + 16 * i + l16;
        ab[i] = __builtin_bit_cast(
            v8bf, *reinterpret_cast<const uint4*>(&As[row * kGemmLdsStride + 8 * achunk(row, 4 * s2 + lg)]));
      }
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const int xo = (16 * c + l16) * kGemmLdsStride + 32 * s2 + 8 * lg;
        const v8bf xb = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(&Xs[xo]));
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][c] = mfma_bf16_k32(ab[i], xb, acc[i][c]);
        if constexpr (SPLIT) {
          const v8bf xlb = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(&Xs[XR * kGemmLdsStride + xo]));
#pragma unroll
          for (int i = 0; i < 2; ++i) acc[i][c] = mfma_bf16_k32(ab[i], xlb, acc[i][c]);
        }
      }
    }
  };
  Slice cur, nxt;
  load_slice(0, cur);
  for (int k0 = 0; k0 < K; k0 += kGemmBK) {
    const bool more = k0 + kGemmBK < K;
    if (more) load_slice(k0 + kGemmBK, nxt);   // in flight during this slice's MFMAs
    stage(cur);
    __syncthreads();
    multiply();
    __syncthreads();
    if (more) cur = nxt;
  }
  // D tile: lane holds rows 4*lg + t, column l16
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = m0 + 32 * wave + 16 * i + 4 * lg + t;
        if (m < M) Y[((size_t)mat * (TRANS ? W : N) + m) * ellp + 16 * c + l16] = acc[i][c][t];
      }
}

// fp32 storage: the same products on fp32 MFMA (16x16x4), operands read straight from
// global memory (L1/L2 serve the re-reads; fp32 factorisation is for small layers).
// Workgroup = (matrix, 128 rows of Y), four wavefronts of two 16-row tiles each, every
// 16-column tile of Y.  A 16-wide k step is four MFMA k steps; lane l supplies the k
// values 4 (l / 16) + s of sub-step s, so that its four A (and X^T) values of a step are
// consecutive in k.
//   TRANS = false: D = A X with A as the MFMA A operand (rows m, 4 consecutive k per
//                  lane: one float4 when W is a multiple of 4);
//   TRANS = true : D^T = X^T A with X^T as the A operand and A's rows (consecutive m
//                  across the 16 lanes of a row group) as the B operand, so each lane
//                  ends holding 4 consecutive columns of one row of Y.
// k past K reads as zero on both operands.
constexpr int kGemmF32Rows = 128;

template <bool TRANS, int NT>
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ Kmat,
                                                  const float* __restrict__ Vmat,
                                                  const float* __restrict__ XT, float* __restrict__ Y,
                                                  int N, int W, int ellp, size_t x_mat_stride, int tiles_m) {
  const int M = TRANS ? W : N, K = TRANS ? N : W;
  const int mat = blockIdx.x / tiles_m, tm = blockIdx.x - mat * tiles_m;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const float* A = ((mat & 1) ? Vmat : Kmat) + (size_t)(mat >> 1) * N * W;
  const float* X = XT + (size_t)mat * x_mat_stride;
  const int mb = tm * kGemmF32Rows + 32 * wave;   // this wavefront's two 16-row tiles
  v4f acc[2][NT];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[i][c] = v4f{0.f, 0.f, 0.f, 0.f};
  const bool kvec = K % 4 == 0;   // rows of X^T (and of A when not transposed) as float4
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int kk = k0 + 4 * lg;   // this lane's first k of the step
    float a[2][4], x[NT][4];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const float* xr = X + (size_t)(16 * c + l16) * K;
      if (kvec) {
        const float4 v = kk < K ? *reinterpret_cast<const float4*>(xr + kk) : make_float4(0.f, 0.f, 0.f, 0.f);
        x[c][0] = v.x; x[c][1] = v.y; x[c][2] = v.z; x[c][3] = v.w;
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) x[c][s] = kk + s < K ? xr[kk + s] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = mb + 16 * i + l16;
      const bool live = m < M;
      if (!TRANS) {
        const float* ar = A + (size_t)(live ? m : 0) * W;
        if (kvec) {
          const float4 v = live && kk < K ? *reinterpret_cast<const float4*>(ar + kk) : make_float4(0.f, 0.f, 0.f, 0.f);
          a[i][0] = v.x; a[i][1] = v.y; a[i][2] = v.z; a[i][3] = v.w;
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) a[i][s] = live && kk + s < K ? ar[kk + s] : 0.f;
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) a[i][s] = live && kk + s < K ? A[(size_t)(kk + s) * W + m] : 0.f;
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < NT; ++c)
          acc[i][c] = TRANS ? mfma_f32(x[c][s], a[i][s], acc[i][c]) : mfma_f32(a[i][s], x[c][s], acc[i][c]);
  }
  // D row 4 lg + t, column l16: (m, 16c + l16) untransposed, (m = l16 tile row,
  // 16c + 4 lg + t) transposed
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      if (!TRANS) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int m = mb + 16 * i + 4 * lg + t;
          if (m < M) Y[((size_t)mat * M + m) * ellp + 16 * c + l16] = acc[i][c][t];
        }
      } else {
        const int m = mb + 16 * i + l16;
        if (m < M)
          *reinterpret_cast<float4*>(Y + ((size_t)mat * M + m) * ellp + 16 * c + 4 * lg) =
              make_float4(acc[i][c][0], acc[i][c][1], acc[i][c][2], acc[i][c][3]);
      }
    }
}

// ================================================================ orthonormalisation
// Shifted Cholesky QR, two passes (CholeskyQR2 with a shift on the first Gram, in the
// spirit of Fukaya et al. 2020): G = Y^T Y, G + eps I = L L^T, Q = Y L^-T.
//
// k_gram: partial Grams.  Workgroup (mat, split) takes rows [split*rows, +rows) of
// Y [M][ellp]; each wavefront accumulates every upper 16x16 tile (fp32 MFMA 16x16x4,
// one 4-row slice per k-step) over its share of them, all loads of UR slices issued
// before their products.  The wavefronts' tiles are summed by halving (the upper half
// of the wavefronts hands its tiles to the lower half through LDS, one float4 per lane
// and tile), and wavefront 0 writes Gpart[mat][split] (full, symmetric) from its
// registers.  Deterministic: a fixed order throughout, and the partials are summed in
// a fixed order by k_chol.
constexpr int kGramThreads = 256;
constexpr int kGramChunk = 15;   // tiles handed over per LDS round

__host__ __device__ inline size_t gram_lds_floats() { return (size_t)(kGramThreads / 128) * kGramChunk * 256; }

template <int T>   // ellp / 16
__global__ __launch_bounds__(kGramThreads) void k_gram(const float* __restrict__ Y, int M, int ellp,
                                                       int rows, int nsplit, float* __restrict__ Gpart) {
  extern __shared__ __align__(16) float sh[];
  constexpr int NW = kGramThreads / 64, NTILE = T * (T + 1) / 2;
  constexpr int NCH = (NTILE + kGramChunk - 1) / kGramChunk;
  float4* red = reinterpret_cast<float4*>(sh);   // [NW / 2][kGramChunk][64 lanes]
  const int mat = blockIdx.x / nsplit, split = blockIdx.x % nsplit;
  const float* Ym = Y + (size_t)mat * M * ellp;
  const int r0 = split * rows, r1 = min(M, r0 + rows);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  v4f acc[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) acc[t] = v4f{0, 0, 0, 0};
  constexpr int UR = 4;   // 4-row k-steps whose loads are in flight together
  for (int n0 = r0 + 4 * UR * wave; n0 < r1; n0 += 4 * UR * NW) {
    float y[UR][T];
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int n = n0 + 4 * u + lg;
      const bool live = n < r1;
      const float* row = Ym + (size_t)(live ? n : r0) * ellp + l16;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float v = row[16 * t];
        y[u][t] = live ? v : 0.f;
      }
    }
    // every load of the slice is issued before the first product (left to itself the
    // scheduler moves each load down to its use, leaving a few in flight)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      int idx = 0;
#pragma unroll
      for (int ti = 0; ti < T; ++ti)
#pragma unroll
        for (int tj = ti; tj < T; ++tj, ++idx) acc[idx] = mfma_f32(y[u][ti], y[u][tj], acc[idx]);
    }
  }
  // ---- sum over the wavefronts by halving
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    for (int h = NW / 2; h >= 1; h >>= 1) {
      if (wave >= h && wave < 2 * h) {
#pragma unroll
        for (int idx = ch * kGramChunk; idx < NTILE && idx < (ch + 1) * kGramChunk; ++idx)
          red[((wave - h) * kGramChunk + idx - ch * kGramChunk) * 64 + lane] =
              make_float4(acc[idx][0], acc[idx][1], acc[idx][2], acc[idx][3]);
      }
      __syncthreads();
      if (wave < h) {
#pragma unroll
        for (int idx = ch * kGramChunk; idx < NTILE && idx < (ch + 1) * kGramChunk; ++idx) {
          const float4 o = red[(wave * kGramChunk + idx - ch * kGramChunk) * 64 + lane];
          acc[idx][0] += o.x; acc[idx][1] += o.y; acc[idx][2] += o.z; acc[idx][3] += o.w;
        }
      }
      __syncthreads();
    }
  }
  if (wave != 0) return;
  // lane holds G[16 ti + 4 lg + t][16 tj + l16], t = 0..3; the mirrored tile takes the
  // four as one 16-byte run of row 16 tj + l16
  float* out = Gpart + ((size_t)mat * nsplit + split) * ellp * ellp;
  int idx = 0;
#pragma unroll
  for (int ti = 0; ti < T; ++ti)
#pragma unroll
    for (int tj = ti; tj < T; ++tj, ++idx) {
      const int i = 16 * ti + 4 * lg, j = 16 * tj + l16;
#pragma unroll
      for (int t = 0; t < 4; ++t) out[(size_t)(i + t) * ellp + j] = acc[idx][t];
      if (ti != tj)
        *reinterpret_cast<float4*>(out + (size_t)j * ellp + i) = make_float4(acc[idx][0], acc[idx][1], acc[idx][2], acc[idx][3]);
    }
}

// Sum of the partial Grams in a fixed order (deterministic), four floats per thread.
__global__ __launch_bounds__(256) void k_gram_reduce(const float* __restrict__ Gpart, int nsplit, int nmat,
                                                     int e2, float* __restrict__ G) {
  const int e4 = e2 >> 2;   // e2 = ellp^2 is a multiple of 256
  const int total = nmat * e4;   // 32-bit: at most 2^31 / 4 matrices of 144^2
  for (int g = blockIdx.x * blockDim.x + threadIdx.x; g < total; g += gridDim.x * blockDim.x) {
    const int mat = g / e4, i = g - (g / e4) * e4;
    const float4* src = reinterpret_cast<const float4*>(Gpart + (size_t)mat * nsplit * e2) + i;
    float4 acc = src[0];
    for (int sp = 1; sp < nsplit; ++sp) {
      const float4 v = src[(size_t)sp * e4];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    reinterpret_cast<float4*>(G + (size_t)mat * e2)[i] = acc;
  }
}

// k_chol: one workgroup (4 wavefronts) per matrix, blocked over 16 x 16 tiles.
// Sums the partial Grams, adds the shift eps = 1e-6 * trace / ell (padded columns
// get a unit diagonal) and factors G + eps I = L L^T right-looking by block
// columns: the diagonal block is factored and inverted in registers by wavefront 0
// (lane i holds row i; values broadcast with readlane), the panel below it is
// L_IJ = A_IJ L_JJ^-T and the trailing update A_IK -= L_IJ L_KJ^T, both on fp32
// MFMA.  X = L^-1 follows by block forward substitution, one block column per
// wavefront at a time (X_IJ = -X_II sum_K L_IK X_KJ involves block column J only),
// each column written out as rows of Rinv = X^T; when Rout is given, R = L^T Rprev
// block column by block column (Rprev NULL: identity; Rprev may equal Rout: a
// wavefront stages the whole block column it reads before it writes that column).
// Only the Gram / L is ell x ell in LDS, so ell up to 144 fits.
constexpr int kCholThreads = 256;
constexpr int kTileF = 16 * 17;      // one padded 16 x 16 tile in LDS (floats)

__host__ __device__ inline size_t chol_lds_floats(int ellp) {
  // L [ellp][ellp + 1], diagonal inverses [T][16][17], one block column per wavefront
  // [4][ellp][17], one tile of scratch per wavefront [4][16][17]
  return (size_t)ellp * (ellp + 1) + (size_t)(ellp / 16) * kTileF + 4 * (size_t)ellp * 17 + 4 * kTileF;
}

__device__ __forceinline__ float lane_bcast(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// acc += op(A) op(B) for 16 x 16 tiles of LDS matrices with row strides SA, SB.
template <bool TA, bool TB, bool NEG>
__device__ __forceinline__ v4f tile_mma(const float* MA, int ar, int ac, int SA, const float* MB, int br,
                                        int bc, int SB, v4f acc, int l16, int lg) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float a = TA ? MA[(ar + 4 * ks + lg) * SA + ac + l16] : MA[(ar + l16) * SA + ac + 4 * ks + lg];
    const float b = TB ? MB[(br + l16) * SB + bc + 4 * ks + lg] : MB[(br + 4 * ks + lg) * SB + bc + l16];
    if (NEG) a = -a;
    acc = mfma_f32(a, b, acc);
  }
  return acc;
}
__device__ __forceinline__ v4f tile_load(const float* M, int r0, int c0, int S, int l16, int lg) {
  v4f d;
#pragma unroll
  for (int t = 0; t < 4; ++t) d[t] = M[(r0 + 4 * lg + t) * S + c0 + l16];
  return d;
}
__device__ __forceinline__ void tile_store(float* M, int r0, int c0, int S, int l16, int lg, v4f d) {
#pragma unroll
  for (int t = 0; t < 4; ++t) M[(r0 + 4 * lg + t) * S + c0 + l16] = d[t];
}

// TT = ellp / 16 is a template argument: the index arithmetic of the staging, shift
// and write-back loops then divides by constants.
template <int TT>
__global__ __launch_bounds__(kCholThreads) void k_chol(const float* __restrict__ Gpart, int nsplit, int ell,
                                                       float* __restrict__ Rinv,
                                                       const float* __restrict__ Rprev,
                                                       float* __restrict__ Rout) {
  extern __shared__ __align__(16) float sh[];
  constexpr int ellp = 16 * TT;
  constexpr int S = ellp + 1;
  constexpr int T = TT;
  float* G = sh;                 // [ellp][S] Gram, then L (lower; diagonal blocks exact)
  float* D = G + ellp * S;       // [T][16][17] inverses of the diagonal blocks of L
  float* Cb = D + T * kTileF;    // [4][ellp][17] per-wavefront block column
  float* Wk = Cb + 4 * ellp * 17;  // [4][16][17] per-wavefront scratch tile
  const int mat = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const size_t e2 = (size_t)ellp * ellp;
  // ---- sum of the partial Grams (fixed order).  16-byte loads, a batch of 8 per
  // thread issued before any is used (ellp^2 / 4 is a multiple of 64)
  const float4* gp = reinterpret_cast<const float4*>(Gpart + (size_t)mat * nsplit * e2);
  const int e4 = static_cast<int>(e2 / 4);
  for (int i0 = 0; i0 < e4; i0 += 8 * kCholThreads) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = gp[min(i0 + u * kCholThreads + tid, e4 - 1)];
    for (int sp = 1; sp < nsplit; ++sp)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float4 w = gp[(size_t)sp * e4 + min(i0 + u * kCholThreads + tid, e4 - 1)];
        v[u].x += w.x; v[u].y += w.y; v[u].z += w.z; v[u].w += w.w;
      }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kCholThreads + tid;
      if (i < e4) {
        const int r = (4 * i) / ellp, c = 4 * i - r * ellp;
        float* g = G + r * S + c;
        g[0] = v[u].x; g[1] = v[u].y; g[2] = v[u].z; g[3] = v[u].w;
      }
    }
  }
  __syncthreads();
  // ---- shift; padded rows and columns become the identity
  __shared__ float trace_sh;
  if (wave == 0) {
    float tr = 0.f;
    for (int i = lane; i < ell; i += 64) tr += G[i * S + i];
    tr = group_sum(tr, 64);
    if (lane == 0) trace_sh = tr;
  }
  __syncthreads();
  const float eps = 1e-6f * (trace_sh / static_cast<float>(ell > 0 ? ell : 1)) + 1e-30f;
  // the diagonal only, then the padded rows and columns (none when ell = ellp)
  for (int i = tid; i < ell; i += kCholThreads) G[i * S + i] += eps;
  for (int idx = tid; idx < (ellp - ell) * ellp; idx += kCholThreads) {
    const int i = ell + idx / ellp, j = idx % ellp;   // row i >= ell, and its mirror column
    G[i * S + j] = i == j ? 1.f : 0.f;
    G[j * S + i] = i == j ? 1.f : 0.f;
  }
  __syncthreads();
  // ---- blocked Cholesky
  for (int J = 0; J < T; ++J) {
    const int c0 = 16 * J;
    float* DJ = D + J * kTileF;
    if (wave == 0) {
      const int li = lane < 16 ? lane : 15;
      float row[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) row[c] = G[(c0 + li) * S + c0 + c];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        // hardware square root and reciprocal (about 1 ulp each): the second pass of the
        // orthonormalisation removes what the first leaves
        const float d = __builtin_amdgcn_sqrtf(fmaxf(lane_bcast(row[j], j), 1e-30f));
        const float inv = __builtin_amdgcn_rcpf(d);
        row[j] = lane == j ? d : (lane > j ? row[j] * inv : 0.f);
#pragma unroll
        for (int k = j + 1; k < 16; ++k) row[k] = fmaf(-row[j], lane_bcast(row[j], k), row[k]);
      }
      // inverse of the 16 x 16 block: lane c computes column c of X_JJ
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = lane == i ? 1.f : 0.f;
#pragma unroll
        for (int k = 0; k < i; ++k) v = fmaf(-lane_bcast(row[k], i), x[k], v);
        x[i] = v * __builtin_amdgcn_rcpf(lane_bcast(row[i], i));
      }
      if (lane < 16) {
#pragma unroll
        for (int c = 0; c < 16; ++c) G[(c0 + lane) * S + c0 + c] = row[c];
#pragma unroll
        for (int i = 0; i < 16; ++i) DJ[i * 17 + lane] = x[i];
      }
    }
    __syncthreads();
    // panel: L_IJ = A_IJ X_JJ^T
    for (int I = J + 1 + wave; I < T; I += 4) {
      const v4f p = tile_mma<false, true, false>(G, 16 * I, c0, S, DJ, 0, 0, 17, v4f{0, 0, 0, 0}, l16, lg);
      tile_store(G, 16 * I, c0, S, l16, lg, p);
    }
    __syncthreads();
    // trailing update of the lower block triangle: A_IK -= L_IJ L_KJ^T, J < K <= I
    const int m = T - J - 1;
    for (int t = wave; t < m * (m + 1) / 2; t += 4) {
      int I = 0, rem = t;
      while (rem > I) { rem -= I + 1; ++I; }   // t -> (I, K) with K <= I
      const int Ib = J + 1 + I, Kb = J + 1 + rem;
      v4f acc = tile_load(G, 16 * Ib, 16 * Kb, S, l16, lg);
      acc = tile_mma<false, true, true>(G, 16 * Ib, c0, S, G, 16 * Kb, c0, S, acc, l16, lg);
      tile_store(G, 16 * Ib, 16 * Kb, S, l16, lg, acc);
    }
    __syncthreads();
  }
  // ---- X = L^-1 by block columns (wavefront-private: no workgroup barrier inside)
  float* cb = Cb + wave * ellp * 17;   // rows 16 Jb .. ellp - 1 of this block column of X
  float* wk = Wk + wave * kTileF;
  auto wave_sync = []() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  float* Ri = Rinv + (size_t)mat * e2;
  for (int Jb = wave; Jb < T; Jb += 4) {
    const float* DJ = D + Jb * kTileF;
    for (int idx = lane; idx < 256; idx += 64) cb[(16 * Jb + (idx >> 4)) * 17 + (idx & 15)] = DJ[(idx >> 4) * 17 + (idx & 15)];
    wave_sync();
    for (int I = Jb + 1; I < T; ++I) {
      v4f acc = v4f{0, 0, 0, 0};
      for (int K = Jb; K < I; ++K)
        acc = tile_mma<false, false, false>(G, 16 * I, 16 * K, S, cb, 16 * K, 0, 17, acc, l16, lg);
      tile_store(wk, 0, 0, 17, l16, lg, acc);
      wave_sync();
      const v4f xr = tile_mma<false, false, true>(D + I * kTileF, 0, 0, 17, wk, 0, 0, 17, v4f{0, 0, 0, 0}, l16, lg);
      tile_store(cb, 16 * I, 0, 17, l16, lg, xr);
      wave_sync();
    }
    // rows 16 Jb .. 16 Jb + 15 of Rinv = X^T: Rinv[16 Jb + c][i] = X[i][16 Jb + c], zero for
    // i below the block column's first row
    for (int idx = lane; idx < 16 * ellp; idx += 64) {
      const int c = idx / ellp, i = idx - c * ellp;
      Ri[(size_t)(16 * Jb + c) * ellp + i] = i < 16 * Jb ? 0.f : cb[i * 17 + c];
    }
    wave_sync();
  }
  if (Rout == nullptr) return;
  // ---- R = L^T Rprev, block column by block column: R[:, Jb] = L^T Rprev[:, Jb]
  const float* Rp = Rprev ? Rprev + (size_t)mat * e2 : nullptr;
  float* Ro = Rout + (size_t)mat * e2;
  for (int Jb = wave; Jb < T; Jb += 4) {
    // stage Rprev[:, 16 Jb .. 16 Jb + 15] (4 consecutive columns per load)
    for (int i0 = 0; i0 < 4 * ellp; i0 += 4 * 64) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = min(i0 + u * 64 + lane, 4 * ellp - 1);
        const int r = idx >> 2, c = 4 * (idx & 3);
        v[u] = Rp ? *reinterpret_cast<const float4*>(Rp + (size_t)r * ellp + 16 * Jb + c)
                  : make_float4(r == 16 * Jb + c, r == 16 * Jb + c + 1, r == 16 * Jb + c + 2, r == 16 * Jb + c + 3);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = i0 + u * 64 + lane;
        if (idx < 4 * ellp) {
          const int r = idx >> 2, c = 4 * (idx & 3);
          float* x = cb + r * 17 + c;
          x[0] = v[u].x; x[1] = v[u].y; x[2] = v[u].z; x[3] = v[u].w;
        }
      }
    }
    wave_sync();
    for (int I = 0; I < T; ++I) {
      v4f acc = v4f{0, 0, 0, 0};
      for (int K = I; K < T; ++K)
        acc = tile_mma<true, false, false>(G, 16 * K, 16 * I, S, cb, 16 * K, 0, 17, acc, l16, lg);
#pragma unroll
      for (int u = 0; u < 4; ++u) Ro[(size_t)(16 * I + 4 * lg + u) * ellp + 16 * Jb + l16] = acc[u];
    }
    wave_sync();
  }
}

using CholFn = void (*)(const float*, int, int, float*, const float*, float*);
static CholFn chol_kernel(int t) {
  switch (t) {
    case 1: return &k_chol<1>;
    case 2: return &k_chol<2>;
    case 3: return &k_chol<3>;
    case 4: return &k_chol<4>;
    case 5: return &k_chol<5>;
    case 6: return &k_chol<6>;
    case 7: return &k_chol<7>;
    case 8: return &k_chol<8>;
    case 9: return &k_chol<9>;
    default: return nullptr;
  }
}

// Q = Y Rinv for 256 rows per workgroup (fp32 MFMA 16x16x4; wavefront w takes rows
// 64w .. 64w + 63 of the tile as four 16-row tiles), written to Qout (Y itself for a
// basis that is orthonormalised again, another buffer for a basis kept for the
// factors, or nowhere when only Q^T is used); optionally Q^T in storage precision for
// the next product (XT[mat][j][m]), and the rounding remainder Q^T - XT in XTlo for a
// two-term product.
// The rows of Y go straight from HBM into registers, all of a wavefront's loads issued
// before the first product: lane (i, g) of a row tile holds columns 16 kc + 4 g .. +3
// of row i, so the MFMA k index runs over (kc, g, e) -> 16 kc + 4 g + e and R^-1 (in
// LDS) is read with the same order.  R^-1 is upper triangular: column tile c of Q
// takes k < 16 (c + 1) only.  Each lane ends with four consecutive rows of one column
// of Q, written to Q^T as one 4-element run.
constexpr int kApplyRT = 4;                  // 16-row tiles per wavefront
constexpr int kApplyRows = 64 * kApplyRT;    // rows per workgroup

template <class T, int NT>   // NT = ellp / 16
__global__ __launch_bounds__(256) void k_apply(const float* Y, float* Qout, int M,
                                               const float* __restrict__ Rinv, T* __restrict__ XT,
                                               T* __restrict__ XTlo, size_t xt_mat_stride, int tiles_m) {
  extern __shared__ __align__(16) float sh[];
  constexpr int ellp = 16 * NT;
  constexpr int RS = ellp + 4;     // LDS row stride: the four 4-row groups of a read meet
                                   // different banks (4 RS = 16 mod 64 words)
  float* Rs = sh;                  // [ellp][RS]
  const int mat = blockIdx.x / tiles_m;
  const int m0 = (blockIdx.x - mat * tiles_m) * kApplyRows;
  const float* Ym = Y + (size_t)mat * M * ellp;
  float* Qm = Qout != nullptr ? Qout + (size_t)mat * M * ellp : nullptr;
  const float* Rm = Rinv + (size_t)mat * ellp * ellp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int base = m0 + 64 * wave;   // first row of this wavefront
  float4 y[kApplyRT][NT];
#pragma unroll
  for (int rt = 0; rt < kApplyRT; ++rt) {
    const int row = min(base + 16 * rt + l16, M - 1);   // rows past M: clamped, never stored
#pragma unroll
    for (int kc = 0; kc < NT; ++kc)
      y[rt][kc] = *reinterpret_cast<const float4*>(Ym + (size_t)row * ellp + 16 * kc + 4 * lg);
  }
  // R^-1 into LDS (16-byte loads, 8 in flight per thread)
  constexpr int nr4 = ellp * ellp / 4;
  for (int i0 = 0; i0 < nr4; i0 += 8 * 256) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = reinterpret_cast<const float4*>(Rm)[min(i0 + u * 256 + tid, nr4 - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 256 + tid;
      if (i < nr4) *reinterpret_cast<float4*>(Rs + (i / (ellp / 4)) * RS + 4 * (i % (ellp / 4))) = v[u];
    }
  }
  __syncthreads();
  T* xt = XT != nullptr ? XT + (size_t)mat * xt_mat_stride : nullptr;
  T* xl = XTlo != nullptr ? XTlo + (size_t)mat * xt_mat_stride : nullptr;
  const bool vec4 = (M & 3) == 0;
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    v4f acc[kApplyRT];
#pragma unroll
    for (int rt = 0; rt < kApplyRT; ++rt) acc[rt] = v4f{0, 0, 0, 0};
#pragma unroll
    for (int kc = 0; kc <= c; ++kc) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float b = Rs[(16 * kc + 4 * lg + e) * RS + 16 * c + l16];
#pragma unroll
        for (int rt = 0; rt < kApplyRT; ++rt) {
          const float a = e == 0 ? y[rt][kc].x : e == 1 ? y[rt][kc].y : e == 2 ? y[rt][kc].z : y[rt][kc].w;
          acc[rt] = mfma_f32(a, b, acc[rt]);
        }
      }
    }
    // lane holds Q[r + t][j], r = base + 16 rt + 4 lg, t = 0..3, j = 16 c + l16
    const int j = 16 * c + l16;
#pragma unroll
    for (int rt = 0; rt < kApplyRT; ++rt) {
      const int r = base + 16 * rt + 4 * lg;
      if (Qm != nullptr) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (r + t < M) Qm[(size_t)(r + t) * ellp + j] = acc[rt][t];
      }
      if (xt == nullptr) continue;
      T* dst = xt + (size_t)j * M + r;
      T* dlo = xl != nullptr ? xl + (size_t)j * M + r : nullptr;
      if constexpr (std::is_same<T, bf16_t>::value) {
        if (vec4 && r + 4 <= M) {
          const uint32_t h0 = pack_bf16x2(acc[rt][0], acc[rt][1]), h1 = pack_bf16x2(acc[rt][2], acc[rt][3]);
          *reinterpret_cast<uint2*>(dst) = make_uint2(h0, h1);
          if (dlo != nullptr)
            *reinterpret_cast<uint2*>(dlo) =
                make_uint2(pack_bf16x2(acc[rt][0] - __uint_as_float(h0 << 16), acc[rt][1] - __uint_as_float(h0 & 0xffff0000u)),
                           pack_bf16x2(acc[rt][2] - __uint_as_float(h1 << 16), acc[rt][3] - __uint_as_float(h1 & 0xffff0000u)));
          continue;
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (r + t >= M) break;
        const T hi = from_f32<T>(acc[rt][t]);
        dst[t] = hi;
        if (dlo != nullptr) dlo[t] = from_f32<T>(acc[rt][t] - to_f32<T>(hi));
      }
    }
  }
}

template <class T>
using ApplyFn = void (*)(const float*, float*, int, const float*, T*, T*, size_t, int);
template <class T>
static ApplyFn<T> apply_kernel(int nt) {
  switch (nt) {
    case 1: return &k_apply<T, 1>;
    case 2: return &k_apply<T, 2>;
    case 3: return &k_apply<T, 3>;
    case 4: return &k_apply<T, 4>;
    case 5: return &k_apply<T, 5>;
    case 6: return &k_apply<T, 6>;
    case 7: return &k_apply<T, 7>;
    case 8: return &k_apply<T, 8>;
    case 9: return &k_apply<T, 9>;
    default: return nullptr;
  }
}

// ================================================================ core SVD
// One-sided Jacobi on the columns of Mj = R^T (ell x ell, LDS): rotations make the
// columns mutually orthogonal, Mj J = P Sigma, J = S.  Round-robin (tournament) pair
// order; one 16-lane group per pair, each lane holding every 16th row, reductions
// by DPP inside the group; a step's E/2 disjoint pairs run at once, one barrier per
// step.  Stops when every pair is orthogonal to 3e-6 relative (fp32), or after 40
// sweeps.
// The rotations depend on Mj alone, and each row of J is rotated independently of
// the others.  When Mj and all of J do not fit one workgroup's LDS (ell > 128), or
// when the matrices are too few to occupy the CUs, the rows of J are split over
// `jsplit` workgroups per matrix (at most 4): each runs the same
// rotations on its own copy of Mj (the same arithmetic in the same order, so the
// copies stay identical) and accumulates its share of J's rows; the first writes
// P Sigma and the singular values.
__host__ __device__ inline int jacobi_rows(int ellp, int jsplit) {   // rows of J per workgroup
  return ((ellp / 16 + jsplit - 1) / jsplit) * 16;
}
__host__ __device__ inline size_t jacobi_lds_floats(int ellp, int jsplit) {
  return (size_t)(ellp + jacobi_rows(ellp, jsplit)) * (ellp + 1) + 2 * (size_t)ellp;
}

// NT = ellp / 16 and JT = jacobi_rows / 16 are compile-time, so that every LDS read
// of a step (both columns of Mj and of this workgroup's rows of J) is issued at once
// and the columns stay in registers from the dot products to the rotation: one LDS
// round trip per step instead of one per 16-row slice.
template <int NT, int JT>
__global__ __launch_bounds__(1024) void k_jacobi(const float* __restrict__ Rm, int ell, int ellp_arg,
                                                 int jsplit, float* __restrict__ PS,
                                                 float* __restrict__ Sv, float* __restrict__ sig) {
  extern __shared__ __align__(16) float sh[];
  (void)ellp_arg;
  constexpr int ellp = 16 * NT;            // index arithmetic divides by constants
  constexpr int S = ellp + 1;              // row offsets become immediates
  const int E = (ell + 1) & ~1;            // even number of columns for the tournament
  const int mat = blockIdx.x / jsplit, js = blockIdx.x - (blockIdx.x / jsplit) * jsplit;
  const int JR = 16 * JT;                  // rows of J per workgroup
  const int j0 = js * JR;                  // first row of J held here
  const int jn = min(JR, ellp - j0);       // rows held (a multiple of 16, >= 16)
  float* Mj = sh;                          // [ellp][S]  (row i, column j)
  float* J = Mj + ellp * S;                // [JR][S]    rows j0 .. j0 + JR - 1 of J
  float* nrm = J + JR * S;                 // [ellp]
  int* perm = reinterpret_cast<int*>(nrm + ellp);  // [ellp]
  __shared__ unsigned int rotated;
  const float* R = Rm + (size_t)mat * ellp * ellp;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int l16 = tid & 15, slot = tid >> 4, nslot = nthr >> 4;
  for (int idx = tid; idx < ellp * ellp; idx += nthr) {
    const int i = idx / ellp, j = idx % ellp;
    Mj[i * S + j] = (i < ell && j < ell) ? R[j * ellp + i] : 0.f;   // transpose
  }
  for (int idx = tid; idx < JR * ellp; idx += nthr) {   // rows past jn: zero, never stored
    const int i = idx / ellp, j = idx % ellp;
    J[i * S + j] = j0 + i == j ? 1.f : 0.f;
  }
  __syncthreads();
  for (int sweep = 0; sweep < 40; ++sweep) {
    if (tid == 0) rotated = 0u;
    __syncthreads();
    for (int step = 0; step < E - 1; ++step) {
      for (int pr = slot; pr < E / 2; pr += nslot) {
        // round-robin pairing: slot pr meets positions pr and E-1-pr; every position but
        // 0 moves one place per step (indices below 2(E-1): one conditional subtraction)
        int p = 0;
        if (pr != 0) { p = pr - 1 + step; p = 1 + (p >= E - 1 ? p - (E - 1) : p); }
        int qq = E - 2 - pr + step;
        qq = 1 + (qq >= E - 1 ? qq - (E - 1) : qq);
        if (p > qq) { const int t = p; p = qq; qq = t; }
        if (qq >= ell) continue;           // uniform over the 16-lane group
        // rows ell..ellp-1 of Mj are zero; all reads of the step are issued together
        float x[NT], y[NT], u[JT], v[JT];
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          x[k] = Mj[(l16 + 16 * k) * S + p];
          y[k] = Mj[(l16 + 16 * k) * S + qq];
        }
#pragma unroll
        for (int k = 0; k < JT; ++k) {
          u[k] = J[(l16 + 16 * k) * S + p];
          v[k] = J[(l16 + 16 * k) * S + qq];
        }
        float a = 0.f, bsum = 0.f, g = 0.f;
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          a = fmaf(x[k], x[k], a);
          bsum = fmaf(y[k], y[k], bsum);
          g = fmaf(x[k], y[k], g);
        }
        a = group_sum(a, 16);
        bsum = group_sum(bsum, 16);
        g = group_sum(g, 16);
        // J's rows stay requested with the columns (not sunk below the test)
#pragma unroll
        for (int k = 0; k < JT; ++k) asm volatile("" ::"v"(u[k]), "v"(v[k]));
        // |g| <= 3e-6 sqrt(a b), squared (column norms are far from the fp32 range ends)
        if (g * g <= 9e-12f * (a * bsum)) continue;
        if (l16 == 0) rotated = 1u;
        // rotation angle from the hardware reciprocal and reciprocal square root (about
        // 1 ulp each): any rotation close to the exact one is orthogonal to within
        // rounding (c^2 + s^2 = 1), and the next sweep measures what is left
        const float zeta = (bsum - a) * __builtin_amdgcn_rcpf(2.f * g);
        const float t = copysignf(__builtin_amdgcn_rcpf(fabsf(zeta) + __builtin_amdgcn_sqrtf(fmaf(zeta, zeta, 1.f))), zeta);
        const float c = __builtin_amdgcn_rsqf(fmaf(t, t, 1.f)), s = c * t;
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          Mj[(l16 + 16 * k) * S + p] = c * x[k] - s * y[k];
          Mj[(l16 + 16 * k) * S + qq] = s * x[k] + c * y[k];
        }
#pragma unroll
        for (int k = 0; k < JT; ++k) {
          J[(l16 + 16 * k) * S + p] = c * u[k] - s * v[k];
          J[(l16 + 16 * k) * S + qq] = s * u[k] + c * v[k];
        }
      }
      __syncthreads();
    }
    if (rotated == 0u) break;
    __syncthreads();
  }
  // singular values and their descending order (ties: lower column first)
  for (int j = tid; j < ellp; j += nthr) {
    float s2 = 0.f;
    for (int i = 0; i < ellp; ++i) s2 = fmaf(Mj[i * S + j], Mj[i * S + j], s2);
    nrm[j] = j < ell ? sqrtf(s2) : -1.f;
  }
  __syncthreads();
  for (int j = tid; j < ellp; j += nthr) {
    int rank = 0;
    for (int o = 0; o < ellp; ++o) rank += (nrm[o] > nrm[j] || (nrm[o] == nrm[j] && o < j)) ? 1 : 0;
    perm[rank] = j;
  }
  __syncthreads();
  float* PSm = PS + (size_t)mat * ellp * ellp;
  float* Sm = Sv + (size_t)mat * ellp * ellp;
  if (js == 0) {
    for (int idx = tid; idx < ellp * ellp; idx += nthr) {
      const int i = idx / ellp, c = idx % ellp;
      PSm[idx] = Mj[i * S + perm[c]];
    }
    for (int c = tid; c < ellp; c += nthr) sig[(size_t)mat * ellp + c] = fmaxf(nrm[perm[c]], 0.f);
  }
  for (int idx = tid; idx < jn * ellp; idx += nthr) {
    const int i = idx / ellp, c = idx % ellp;
    Sm[(size_t)(j0 + i) * ellp + c] = J[i * S + perm[c]];
  }
}

using JacobiFn = void (*)(const float*, int, int, int, float*, float*, float*);
// Instances: NT = ellp / 16 up to 9, JT = ceil(NT / jsplit) for jsplit = 1 .. 4.
template <int NT>
static JacobiFn jacobi_kernel_nt(int jt) {
  if (jt == NT) return &k_jacobi<NT, NT>;
  if (jt == (NT + 1) / 2) return &k_jacobi<NT, (NT + 1) / 2>;
  if (jt == (NT + 2) / 3) return &k_jacobi<NT, (NT + 2) / 3>;
  if (jt == (NT + 3) / 4) return &k_jacobi<NT, (NT + 3) / 4>;
  return nullptr;
}
static JacobiFn jacobi_kernel(int nt, int jt) {
  switch (nt) {
    case 1: return jacobi_kernel_nt<1>(jt);
    case 2: return jacobi_kernel_nt<2>(jt);
    case 3: return jacobi_kernel_nt<3>(jt);
    case 4: return jacobi_kernel_nt<4>(jt);
    case 5: return jacobi_kernel_nt<5>(jt);
    case 6: return jacobi_kernel_nt<6>(jt);
    case 7: return jacobi_kernel_nt<7>(jt);
    case 8: return jacobi_kernel_nt<8>(jt);
    case 9: return jacobi_kernel_nt<9>(jt);
    default: return nullptr;
  }
}

// ================================================================ assembly
// Stages a rows x cols block of fp32 (cols a multiple of 4; global rows 16-byte aligned
// with stride gs, cols <= gs) into LDS with row stride ls: 16-byte loads, 8 per thread
// issued before any is stored.  Rows >= vrows (vrows >= 1) and columns >= vcols read
// as zero; their loads are clamped into the block.
__device__ __forceinline__ void stage_f32(float* dst, int ls, const float* src, int gs, int rows, int cols,
                                          int vrows, int vcols) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int c4 = cols / 4, n4 = rows * c4;
  for (int i0 = 0; i0 < n4; i0 += 8 * nthr) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = min(i0 + u * nthr + tid, n4 - 1);
      const int r = i / c4, c = 4 * (i - r * c4);
      v[u] = *reinterpret_cast<const float4*>(src + (size_t)min(r, vrows - 1) * gs + c);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * nthr + tid;
      if (i < n4) {
        const int r = i / c4, c = 4 * (i - r * c4);
        const bool live = r < vrows;
        float* d = dst + r * ls + c;
        d[0] = live && c < vcols ? v[u].x : 0.f;
        d[1] = live && c + 1 < vcols ? v[u].y : 0.f;
        d[2] = live && c + 2 < vcols ? v[u].z : 0.f;
        d[3] = live && c + 3 < vcols ? v[u].w : 0.f;
      }
    }
  }
}

// U[n][i] = sum_j Qn[n][j] PS[j][i] (i < r) straight into the decode tiles, on fp32
// MFMA 16x16x4 in the layout of k_apply: 256 tokens per workgroup (wavefront wv takes
// tokens 64 wv .. 64 wv + 63, two 32-token blocks of two 16-row tiles), each lane holding
// four consecutive columns j of one token in registers, PS[:, :r_pad] in LDS.
// V tiles (element [lane][half][e] = token 16 half + 4 (lane / 16) + e, column lane % 16)
// are the MFMA output layout itself; K tiles (token 16 half + lane % 16, column
// 4 (lane / 16) + e) are its transpose, so for U_k the two operands swap places (PS
// columns as the A operand, tokens as the B operand).  Either way a lane ends with the
// 8 elements it owns in a tile, written in one 16-byte store (two for fp32).  Tokens
// past N read as zero.
template <class T, int NT, int NR>   // NT = ellp / 16, NR = r_pad / 16
__global__ __launch_bounds__(256) void k_assemble_u(const float* __restrict__ Qn, const float* __restrict__ PS,
                                                    T* __restrict__ Ukv, int N, int r, int nblk, int tiles_n) {
  extern __shared__ __align__(16) float sh[];
  constexpr int ellp = 16 * NT, rp = 16 * NR;
  constexpr int PSS = rp + 4;      // LDS row stride (4 PSS = 16 mod 64 words)
  float* Ps = sh;                  // [ellp][PSS]
  const int mat = blockIdx.x / tiles_n;
  const int n0 = (blockIdx.x - mat * tiles_n) * 256;
  const int b = mat >> 1;
  const bool vl = mat & 1;
  const float* Q = Qn + (size_t)mat * N * ellp;
  const float* P = PS + (size_t)mat * ellp * ellp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int base = n0 + 64 * wave;
  float4 y[4][NT];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int tok = base + 16 * rt + l16;
    const float* row = Q + (size_t)min(tok, N - 1) * ellp + 4 * lg;
#pragma unroll
    for (int kc = 0; kc < NT; ++kc) {
      const float4 v = *reinterpret_cast<const float4*>(row + 16 * kc);
      y[rt][kc] = tok < N ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  for (int idx = tid; idx < ellp * (rp / 4); idx += 256) {
    const int j = idx / (rp / 4), c = 4 * (idx - j * (rp / 4));
    float4 v = *reinterpret_cast<const float4*>(P + (size_t)j * ellp + c);
    if (c + 0 >= r) v.x = 0.f;
    if (c + 1 >= r) v.y = 0.f;
    if (c + 2 >= r) v.z = 0.f;
    if (c + 3 >= r) v.w = 0.f;
    *reinterpret_cast<float4*>(Ps + j * PSS + c) = v;
  }
  __syncthreads();
  T* tiles = Ukv + (vl ? (size_t)(rp / 16) * kBlockElems : 0);
#pragma unroll
  for (int p = 0; p < NR; ++p) {
    v4f acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0, 0, 0, 0};
#pragma unroll
    for (int kc = 0; kc < NT; ++kc) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = Ps[(16 * kc + 4 * lg + e) * PSS + 16 * p + l16];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const float tv = e == 0 ? y[rt][kc].x : e == 1 ? y[rt][kc].y : e == 2 ? y[rt][kc].z : y[rt][kc].w;
          acc[rt] = vl ? mfma_f32(tv, pv, acc[rt]) : mfma_f32(pv, tv, acc[rt]);
        }
      }
    }
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {        // the wavefront's two 32-token blocks
      const int blk = (base >> 5) + hb;
      if (blk >= nblk) continue;
      T* dst = tiles + tile_base(b, p, blk, rp / 16, nblk) + 8 * lane;
      const v4f h0 = acc[2 * hb], h1 = acc[2 * hb + 1];   // tile halves 0 and 1
      if constexpr (std::is_same<T, bf16_t>::value) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(h0[0], h0[1]), pack_bf16x2(h0[2], h0[3]),
                                                    pack_bf16x2(h1[0], h1[1]), pack_bf16x2(h1[2], h1[3]));
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(h0[0], h0[1], h0[2], h0[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(h1[0], h1[1], h1[2], h1[3]);
      }
    }
  }
}

template <class T>
using AssembleUFn = void (*)(const float*, const float*, T*, int, int, int, int);
template <class T, int NT, int NR>
static AssembleUFn<T> assemble_u_if() {
  if constexpr (NR <= NT) return &k_assemble_u<T, NT, NR>;
  else return nullptr;
}
template <class T, int NT>
static AssembleUFn<T> assemble_u_nt(int nr) {
  switch (nr) {
    case 1: return assemble_u_if<T, NT, 1>();
    case 2: return assemble_u_if<T, NT, 2>();
    case 3: return assemble_u_if<T, NT, 3>();
    case 4: return assemble_u_if<T, NT, 4>();
    case 5: return assemble_u_if<T, NT, 5>();
    case 6: return assemble_u_if<T, NT, 6>();
    case 7: return assemble_u_if<T, NT, 7>();
    case 8: return assemble_u_if<T, NT, 8>();
    default: return nullptr;
  }
}
template <class T>
static AssembleUFn<T> assemble_u_kernel(int nt, int nr) {
  if (nr > nt) return nullptr;
  switch (nt) {
    case 1: return assemble_u_nt<T, 1>(nr);
    case 2: return assemble_u_nt<T, 2>(nr);
    case 3: return assemble_u_nt<T, 3>(nr);
    case 4: return assemble_u_nt<T, 4>(nr);
    case 5: return assemble_u_nt<T, 5>(nr);
    case 6: return assemble_u_nt<T, 6>(nr);
    case 7: return assemble_u_nt<T, 7>(nr);
    case 8: return assemble_u_nt<T, 8>(nr);
    case 9: return assemble_u_nt<T, 9>(nr);
    default: return nullptr;
  }
}

// 4-bit factors: the same product for one block, kept in LDS in fp32, then quantized
// with the block's per-column scales (quant4.h).
__global__ __launch_bounds__(256) void k_assemble_u4(const float* __restrict__ Qn, const float* __restrict__ PS,
                                                     i4_t* __restrict__ Ukv, bf16_t* __restrict__ scales,
                                                     int N, int ellp, int r, int NP, int nblk) {
  extern __shared__ __align__(16) float sh[];
  const int rp = 16 * NP, ld = rp + 1;
  float* Qs = sh;                      // [32][ellp + 1]
  float* Ps = Qs + 32 * (ellp + 1);    // [ellp][rp]
  float* Ub = Ps + ellp * rp;          // [32][ld]
  float* scl = Ub + 32 * ld;           // [rp]
  const int mat = blockIdx.x / nblk, t = blockIdx.x % nblk;
  const int b = mat >> 1;
  const bool vl = mat & 1;
  const float* Q = Qn + (size_t)mat * N * ellp;
  const float* P = PS + (size_t)mat * ellp * ellp;
  stage_f32(Qs, ellp + 1, Q + (size_t)kBlockTok * t * ellp, ellp, 32, ellp, N - kBlockTok * t, ellp);
  stage_f32(Ps, rp, P, ellp, ellp, rp, ellp, r);
  __syncthreads();
  for (int idx = threadIdx.x; idx < 32 * rp; idx += blockDim.x) {
    const int rr = idx / rp, col = idx % rp;
    float v = 0.f;
    for (int j = 0; j < ellp; ++j) v = fmaf(Qs[rr * (ellp + 1) + j], Ps[j * rp + col], v);
    Ub[rr * ld + col] = v;
  }
  __syncthreads();
  i4_t* tiles = tile_ptr(Ukv, tile_base(b, 0, t, NP, nblk) + (vl ? (size_t)NP * kBlockElems : 0));
  bf16_t* srow = scales + (((size_t)b * nblk + t) * 2 + (vl ? 1 : 0)) * rp;
  if (vl) q4_store_block<true>(Ub, ld, NP, tiles, srow, scl);
  else q4_store_block<false>(Ub, ld, NP, tiles, srow, scl);
}

// B[i][w] = sum_j Qc[w][j] S[j][i] for i < r (rows r..r_pad-1 stay zero), on fp32 MFMA
// 16x16x4 in the layout of k_apply: 256 rows w per workgroup (wavefront wv takes rows
// 64 wv .. 64 wv + 63 as four 16-row tiles), each lane holding four consecutive columns
// j of one row in registers straight from HBM, S[:, :r_pad] in LDS read in the same k
// order.  A lane ends with B[i][w .. w+3] for one i: one 4-element run per store.
template <class T, int NT, int NR>   // NT = ellp / 16, NR = r_pad / 16
__global__ __launch_bounds__(256) void k_assemble_b(const float* __restrict__ Qc, const float* __restrict__ Sv,
                                                    T* __restrict__ Bk, T* __restrict__ Bv, int W, int r,
                                                    int tiles_w) {
  extern __shared__ __align__(16) float sh[];
  constexpr int ellp = 16 * NT, rp = 16 * NR;
  constexpr int SS = rp + 4;       // LDS row stride: the four 4-row groups of a read meet
                                   // different banks (4 SS = 16 mod 64 words)
  float* Ss = sh;                  // [ellp][SS]
  const int mat = blockIdx.x / tiles_w;
  const int w0 = (blockIdx.x - mat * tiles_w) * 256;
  const float* Q = Qc + (size_t)mat * W * ellp;
  const float* Sm = Sv + (size_t)mat * ellp * ellp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int base = w0 + 64 * wave;
  float4 y[4][NT];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int row = min(base + 16 * rt + l16, W - 1);   // rows past W: clamped, never stored
#pragma unroll
    for (int kc = 0; kc < NT; ++kc)
      y[rt][kc] = *reinterpret_cast<const float4*>(Q + (size_t)row * ellp + 16 * kc + 4 * lg);
  }
  // S[:, :rp] into LDS, columns >= r zeroed
  for (int idx = tid; idx < ellp * (rp / 4); idx += 256) {
    const int j = idx / (rp / 4), c = 4 * (idx - j * (rp / 4));
    float4 v = *reinterpret_cast<const float4*>(Sm + (size_t)j * ellp + c);
    if (c + 0 >= r) v.x = 0.f;
    if (c + 1 >= r) v.y = 0.f;
    if (c + 2 >= r) v.z = 0.f;
    if (c + 3 >= r) v.w = 0.f;
    *reinterpret_cast<float4*>(Ss + j * SS + c) = v;
  }
  __syncthreads();
  T* B = ((mat & 1) ? Bv : Bk) + (size_t)(mat >> 1) * rp * W;
  const bool vec4 = (W & 3) == 0;
#pragma unroll
  for (int c = 0; c < NR; ++c) {
    v4f acc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[rt] = v4f{0, 0, 0, 0};
#pragma unroll
    for (int kc = 0; kc < NT; ++kc) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float bv = Ss[(16 * kc + 4 * lg + e) * SS + 16 * c + l16];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const float av = e == 0 ? y[rt][kc].x : e == 1 ? y[rt][kc].y : e == 2 ? y[rt][kc].z : y[rt][kc].w;
          acc[rt] = mfma_f32(av, bv, acc[rt]);
        }
      }
    }
    // lane holds B[i][w + t], i = 16 c + l16, w = base + 16 rt + 4 lg, t = 0..3
    const int i = 16 * c + l16;
    if (i >= r) continue;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int w = base + 16 * rt + 4 * lg;
      T* dst = B + (size_t)i * W + w;
      if (vec4 && w + 4 <= W) {
        if constexpr (std::is_same<T, bf16_t>::value)
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[rt][0], acc[rt][1]), pack_bf16x2(acc[rt][2], acc[rt][3]));
        else
          *reinterpret_cast<float4*>(dst) = make_float4(acc[rt][0], acc[rt][1], acc[rt][2], acc[rt][3]);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (w + t < W) dst[t] = from_f32<T>(acc[rt][t]);
      }
    }
  }
}

template <class T>
using AssembleBFn = void (*)(const float*, const float*, T*, T*, int, int, int);
template <class T, int NT, int NR>
static AssembleBFn<T> assemble_b_if() {
  if constexpr (NR <= NT) return &k_assemble_b<T, NT, NR>;
  else return nullptr;
}
template <class T, int NT>
static AssembleBFn<T> assemble_b_nt(int nr) {
  switch (nr) {
    case 1: return assemble_b_if<T, NT, 1>();
    case 2: return assemble_b_if<T, NT, 2>();
    case 3: return assemble_b_if<T, NT, 3>();
    case 4: return assemble_b_if<T, NT, 4>();
    case 5: return assemble_b_if<T, NT, 5>();
    case 6: return assemble_b_if<T, NT, 6>();
    case 7: return assemble_b_if<T, NT, 7>();
    case 8: return assemble_b_if<T, NT, 8>();
    default: return nullptr;
  }
}
template <class T>
static AssembleBFn<T> assemble_b_kernel(int nt, int nr) {
  if (nr > nt) return nullptr;
  switch (nt) {
    case 1: return assemble_b_nt<T, 1>(nr);
    case 2: return assemble_b_nt<T, 2>(nr);
    case 3: return assemble_b_nt<T, 3>(nr);
    case 4: return assemble_b_nt<T, 4>(nr);
    case 5: return assemble_b_nt<T, 5>(nr);
    case 6: return assemble_b_nt<T, 6>(nr);
    case 7: return assemble_b_nt<T, 7>(nr);
    case 8: return assemble_b_nt<T, 8>(nr);
    case 9: return assemble_b_nt<T, 9>(nr);
    default: return nullptr;
  }
}

__global__ void k_copy_sigma(const float* __restrict__ sig, float* __restrict__ sk, float* __restrict__ sv,
                             int nmat, int ellp, int r) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= nmat * r) return;
  const int mat = g / r, i = g % r;
  ((mat & 1) ? sv : sk)[(size_t)(mat >> 1) * r + i] = sig[(size_t)mat * ellp + i];
}

// ================================================================ launch sequence
// Clears a buffer (16-byte words; a kernel rather than hipMemsetAsync, so that a caller
// may capture the whole factorisation in a graph).
__global__ __launch_bounds__(256) void k_zero(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

static dim3 grid_1d(size_t total, int threads = 256) {
  size_t g = (total + threads - 1) / threads;
  g = g < 1 ? 1 : (g > 65536 ? 65536 : g);
  return dim3(static_cast<unsigned>(g));
}

template <class T>
static hipError_t gemm(const ap_cache* c, const void* k, const void* v, const void* XT, const void* XTlo,
                       float* Y, bool trans, size_t x_stride, hipStream_t st) {
  const Dims& dm = c->dm;
  const int nmat = 2 * dm.B;
  const int ellp = (dm.ell + 15) / 16 * 16;
  const int M = trans ? dm.W : dm.N;
  if constexpr (std::is_same<T, bf16_t>::value) {
    const int K = trans ? dm.N : dm.W;
    const bool vec = dm.W % 8 == 0 && K % 8 == 0 && K >= 8;
    // 256-row tiles (8 wavefronts) halve the X^T re-reads per byte of A: the plain
    // transposed product (batch-32 layer 350 -> 283 us per pass, batch-256 layer 3.82 ->
    // 3.15 ms) and the untransposed one when M is a multiple of 256 (batch-256 layer
    // 3.55 -> 3.38 ms; at M = 2880 its last, mostly empty tile costs more than it saves).
    // The two-term product keeps 128-row tiles: it needs the registers.
#define AP_GEMM_LAUNCH_V(TR, NTV, SP, VC, BMV)                                                          \
  do {                                                                                                  \
    const int tiles_m = (M + (BMV) - 1) / (BMV);                                                        \
    hipLaunchKernelGGL((k_gemm<bf16_t, TR, NTV, SP, VC, BMV>), dim3(nmat * tiles_m), dim3(2 * (BMV)), 0, \
                       st, static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),                \
                       static_cast<const bf16_t*>(XT), static_cast<const bf16_t*>(XTlo), Y, dm.N, dm.W, \
                       ellp, x_stride, tiles_m);                                                        \
  } while (0)
#define AP_GEMM_LAUNCH_B(TR, NTV, SP, BMV)                                                              \
  do {                                                                                                  \
    if (vec) AP_GEMM_LAUNCH_V(TR, NTV, SP, true, BMV);                                                  \
    else AP_GEMM_LAUNCH_V(TR, NTV, SP, false, BMV);                                                     \
  } while (0)
#define AP_GEMM_LAUNCH(TR, NTV, SP)                                                                     \
  do {                                                                                                  \
    if constexpr (SP) AP_GEMM_LAUNCH_B(TR, NTV, SP, 128);                                               \
    else if ((TR) || M % 256 == 0) AP_GEMM_LAUNCH_B(TR, NTV, SP, 256);                                  \
    else AP_GEMM_LAUNCH_B(TR, NTV, SP, 128);                                                            \
  } while (0)
#define AP_GEMM_CASE(NTV)                                                                              \
  case NTV:                                                                                            \
    if (trans && XTlo != nullptr) AP_GEMM_LAUNCH(true, NTV, true);                                     \
    else if (trans) AP_GEMM_LAUNCH(true, NTV, false);                                                  \
    else AP_GEMM_LAUNCH(false, NTV, false);                                                            \
    break;
    switch (ellp / 16) {
      AP_GEMM_CASE(1) AP_GEMM_CASE(2) AP_GEMM_CASE(3) AP_GEMM_CASE(4)
      AP_GEMM_CASE(5) AP_GEMM_CASE(6) AP_GEMM_CASE(7) AP_GEMM_CASE(8) AP_GEMM_CASE(9)
      default: return hipErrorInvalidValue;
    }
#undef AP_GEMM_CASE
#undef AP_GEMM_LAUNCH
#undef AP_GEMM_LAUNCH_B
#undef AP_GEMM_LAUNCH_V
  } else {
    const int tiles_m = (M + kGemmF32Rows - 1) / kGemmF32Rows;
#define AP_GEMM_F32_CASE(NTV)                                                                         \
  case NTV:                                                                                           \
    if (trans)                                                                                        \
      hipLaunchKernelGGL((k_gemm_f32<true, NTV>), dim3(nmat * tiles_m), dim3(256), 0, st,             \
                         static_cast<const float*>(k), static_cast<const float*>(v),                  \
                         static_cast<const float*>(XT), Y, dm.N, dm.W, ellp, x_stride, tiles_m);      \
    else                                                                                              \
      hipLaunchKernelGGL((k_gemm_f32<false, NTV>), dim3(nmat * tiles_m), dim3(256), 0, st,            \
                         static_cast<const float*>(k), static_cast<const float*>(v),                  \
                         static_cast<const float*>(XT), Y, dm.N, dm.W, ellp, x_stride, tiles_m);      \
    break;
    switch (ellp / 16) {
      AP_GEMM_F32_CASE(1) AP_GEMM_F32_CASE(2) AP_GEMM_F32_CASE(3) AP_GEMM_F32_CASE(4)
      AP_GEMM_F32_CASE(5) AP_GEMM_F32_CASE(6) AP_GEMM_F32_CASE(7) AP_GEMM_F32_CASE(8) AP_GEMM_F32_CASE(9)
      default: return hipErrorInvalidValue;
    }
#undef AP_GEMM_F32_CASE
  }
  return hipGetLastError();
}

// Row split of the Gram of an M-row basis: about 512 workgroups over all matrices,
// at least 64 rows each.
static void gram_split(int M, int nmat, int& rows, int& nsplit) {
  int want = (512 + nmat - 1) / std::max(nmat, 1);
  want = std::max(1, std::min(want, (M + 63) / 64));
  rows = ((M + want - 1) / want + 63) / 64 * 64;
  nsplit = (M + rows - 1) / rows;
}

// Shifted Cholesky QR of Y [nmat][M][ellp], `passes` times (1 for bases that only feed
// the next power-iteration product, 2 where U or B are built from the basis): earlier
// passes write Q over Y, the last one to Qlast (if given; [nmat][M][ellp]); Q^T to XT
// after the last pass (if given); R to Racc (if given).
template <class T>
static hipError_t orth(const ap_cache* c, CompressWs& ws, int M, void* XT, void* XTlo, float* Racc,
                       int passes, float* Qlast, hipStream_t st) {
  const Dims& dm = c->dm;
  const int nmat = 2 * dm.B, ellp = ws.ellp;
  const size_t lds_gram = gram_lds_floats() * sizeof(float);
  const size_t lds_chol = chol_lds_floats(ellp) * sizeof(float);
  const size_t lds_apply = (size_t)ellp * (ellp + 4) * sizeof(float);
  const int tiles_m = (M + kApplyRows - 1) / kApplyRows;
  const ApplyFn<T> apply_fn = apply_kernel<T>(ellp / 16);
  if (apply_fn == nullptr) return hipErrorInvalidValue;
  const CholFn chol_fn = chol_kernel(ellp / 16);
  if (chol_fn == nullptr) return hipErrorInvalidValue;
  int rows, nsplit;
  gram_split(M, nmat, rows, nsplit);
  for (int pass = 0; pass < passes; ++pass) {
    const bool last = pass == passes - 1;
    switch (ellp / 16) {
#define AP_GRAM_CASE(TV)                                                                              \
  case TV:                                                                                            \
    hipLaunchKernelGGL(k_gram<TV>, dim3(nmat * nsplit), dim3(kGramThreads), lds_gram, st, ws.Y, M, ellp, \
                       rows, nsplit, ws.Gpart);                                                       \
    break;
      AP_GRAM_CASE(1) AP_GRAM_CASE(2) AP_GRAM_CASE(3) AP_GRAM_CASE(4)
      AP_GRAM_CASE(5) AP_GRAM_CASE(6) AP_GRAM_CASE(7) AP_GRAM_CASE(8) AP_GRAM_CASE(9)
#undef AP_GRAM_CASE
      default: return hipErrorInvalidValue;
    }
    const float* Gsum = ws.Gpart;
    if (nsplit > 1) {
      hipLaunchKernelGGL(k_gram_reduce, grid_1d((size_t)nmat * ellp * ellp / 4), dim3(256), 0, st, ws.Gpart,
                         nsplit, nmat, ellp * ellp, ws.Gsum);
      Gsum = ws.Gsum;
    }
    hipLaunchKernelGGL(chol_fn, dim3(nmat), dim3(kCholThreads), lds_chol, st, Gsum, 1, dm.ell,
                       ws.Rinv, pass == 0 ? nullptr : Racc, Racc);
    hipLaunchKernelGGL(apply_fn, dim3(nmat * tiles_m), dim3(256), lds_apply, st, ws.Y, last ? Qlast : ws.Y, M,
                       ws.Rinv, static_cast<T*>(last ? XT : nullptr), static_cast<T*>(last ? XTlo : nullptr),
                       (size_t)ellp * ws.M, tiles_m);
  }
  return hipGetLastError();
}

// The factorisation workspace comes from stream-ordered allocations (fixed == nullptr)
// or is carved out of the caller's fixed buffer of fixed_bytes (then nothing is
// allocated, and a workspace that does not fit is refused before anything is enqueued).
template <class T>
static hipError_t compress_t(ap_cache* c, const void* k, const void* v, hipStream_t st, void* fixed,
                             size_t fixed_bytes) {
  const Dims& dm = c->dm;
  CompressWs ws;
  ws.nmat = 2 * dm.B;
  ws.M = std::max(dm.N, dm.W);
  ws.ellp = (dm.ell + 15) / 16 * 16;
  if (ws.ellp > kMaxEll) {
    set_error("ap_compress: ell = min(rank + oversample, n_tokens, width) must be <= 144");
    return hipErrorNotSupported;
  }
  const int nmat = ws.nmat, ellp = ws.ellp;
  const size_t es = sizeof(T);
  int rows_n, split_n, rows_w, split_w;
  gram_split(dm.N, nmat, rows_n, split_n);
  gram_split(dm.W, nmat, rows_w, split_w);
  const size_t max_split = (size_t)std::max(split_n, split_w);
  struct Buf { void** p; size_t bytes; };
  Buf bufs[] = {
      {&ws.omT, (size_t)nmat * ellp * dm.W * es},
      {reinterpret_cast<void**>(&ws.Y), (size_t)nmat * ws.M * ellp * 4},
      {&ws.XT, (size_t)nmat * ellp * ws.M * es},
      {&ws.XTlo, std::is_same<T, bf16_t>::value ? (size_t)nmat * ellp * ws.M * es : 0},
      {reinterpret_cast<void**>(&ws.Qn), (size_t)nmat * dm.N * ellp * 4},
      {reinterpret_cast<void**>(&ws.Qc), (size_t)nmat * dm.W * ellp * 4},
      {reinterpret_cast<void**>(&ws.Gpart), (size_t)nmat * max_split * ellp * ellp * 4},
      {reinterpret_cast<void**>(&ws.Gsum), (size_t)nmat * ellp * ellp * 4},
      {reinterpret_cast<void**>(&ws.Rinv), (size_t)nmat * ellp * ellp * 4},
      {reinterpret_cast<void**>(&ws.Racc), (size_t)nmat * ellp * ellp * 4},
      {reinterpret_cast<void**>(&ws.PS), (size_t)nmat * ellp * ellp * 4},
      {reinterpret_cast<void**>(&ws.Sv), (size_t)nmat * ellp * ellp * 4},
      {reinterpret_cast<void**>(&ws.sig), (size_t)nmat * ellp * 4},
  };
  hipError_t e = hipSuccess;
  if (fixed != nullptr) {
    // 256-byte aligned pieces of the fixed buffer, in order
    size_t off = 0;
    for (Buf& bf : bufs) {
      if (bf.bytes == 0) continue;
      off = (off + 255) & ~(size_t)255;
      *bf.p = static_cast<unsigned char*>(fixed) + off;
      off += bf.bytes;
    }
    if (off > fixed_bytes) {
      for (Buf& bf : bufs) *bf.p = nullptr;
      set_error("ap_recompress_noalloc: this shape needs " + std::to_string(off) +
                " bytes of factorisation workspace, the fixed workspace holds " + std::to_string(fixed_bytes));
      return hipErrorNotSupported;
    }
  } else {
    for (Buf& bf : bufs) {
      if (bf.bytes == 0) continue;
      e = hipMallocAsync(bf.p, bf.bytes, st);
      if (e != hipSuccess) break;
    }
  }
  auto release = [&]() {
    if (fixed != nullptr) return;
    for (Buf& bf : bufs)
      if (*bf.p) (void)hipFreeAsync(*bf.p, st);
  };
  if (e != hipSuccess) {
    set_error("compress workspace allocation failed");
    release();
    return hipErrorOutOfMemory;
  }
  auto fail_stage = [&](hipError_t err, const char* stage) {
    set_error(std::string("ap_compress, ") + stage + ": " + hipGetErrorString(err));
    release();
    return err;
  };
  // padded rows of Omega^T and X^T must read as zero (each buffer's byte count is a
  // multiple of 16: ellp is a multiple of 16)
  for (void* z : {ws.omT, ws.XT, ws.XTlo}) {
    if (z == nullptr) continue;
    const size_t bytes = (size_t)nmat * ellp * (z == ws.omT ? dm.W : ws.M) * es;
    hipLaunchKernelGGL(k_zero, grid_1d(bytes / 16), dim3(256), 0, st, static_cast<uint4*>(z), bytes / 16);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return fail_stage(e, "workspace clear");
  if (c->params.omega != nullptr)
    hipLaunchKernelGGL(k_omega_copy<T>, grid_1d((size_t)nmat * dm.ell * dm.W), dim3(256), 0, st,
                       c->params.omega, static_cast<T*>(ws.omT), nmat, dm.W, dm.ell, ellp);
  else
    hipLaunchKernelGGL(k_omega_philox<T>,
                       dim3(static_cast<unsigned>(std::min<size_t>(((dm.ell * (size_t)dm.W + 7) / 8 + 255) / 256, 4096)),
                            static_cast<unsigned>(nmat)),
                       dim3(256), 0, st, static_cast<T*>(ws.omT), nmat, dm.W, dm.ell, ellp, c->params.seed);
  e = hipGetLastError();
  if (e != hipSuccess) return fail_stage(e, "test matrix");

  // dynamic LDS above the 64 KB default: request exactly what each launch uses
  const size_t lds_chol = chol_lds_floats(ellp) * sizeof(float);
  // the rows of the core SVD's rotation matrix are split over two workgroups per matrix
  // when they do not fit one workgroup's LDS beside the matrix itself
  int jsplit = jacobi_lds_floats(ellp, 1) * sizeof(float) <= 160 * 1024 ? 1 : 2;
  // while the matrices leave CUs idle, the rotation matrix's rows are spread over more
  // workgroups (up to 4 per matrix): each step then rotates fewer rows per workgroup
  while (jsplit < 4 && (size_t)nmat * (jsplit + 1) <= 256 &&
         jacobi_rows(ellp, jsplit + 1) < jacobi_rows(ellp, jsplit))
    ++jsplit;
  const size_t lds_jac = jacobi_lds_floats(ellp, jsplit) * sizeof(float);
  const JacobiFn jac_fn = jacobi_kernel(ellp / 16, jacobi_rows(ellp, jsplit) / 16);
  if (jac_fn == nullptr) return fail_stage(hipErrorInvalidValue, "core SVD shape");
  const size_t lds_apply = (size_t)ellp * (ellp + 4) * sizeof(float);
  const ApplyFn<T> apply_fn = apply_kernel<T>(ellp / 16);
  if (apply_fn == nullptr) return fail_stage(hipErrorInvalidValue, "orthonormalisation shape");
  const bool u4 = dm.storage == AP_INT4;
  const size_t lds_u = (size_t)(32 * (ellp + 1) + ellp * 16 * dm.NP + 32 * (16 * dm.NP + 1) +
                                (u4 ? 16 * dm.NP : 0)) * sizeof(float);
  const size_t lds_u2 = (size_t)ellp * (dm.r_pad + 4) * sizeof(float);
  const AssembleUFn<T> asm_u_fn = u4 ? nullptr : assemble_u_kernel<T>(ellp / 16, dm.r_pad / 16);
  if (!u4 && asm_u_fn == nullptr) return fail_stage(hipErrorInvalidValue, "factor assembly shape");
  const size_t lds_b = (size_t)ellp * (dm.r_pad + 4) * sizeof(float);
  const AssembleBFn<T> asm_b_fn = assemble_b_kernel<T>(ellp / 16, dm.r_pad / 16);
  if (asm_b_fn == nullptr) return fail_stage(hipErrorInvalidValue, "factor assembly shape");
  const struct { const void* fn; size_t bytes; const char* name; } lds_req[] = {
      {reinterpret_cast<const void*>(chol_kernel(ellp / 16)), lds_chol, "LDS size of k_chol"},
      {reinterpret_cast<const void*>(asm_b_fn), lds_b, "LDS size of k_assemble_b"},
      {reinterpret_cast<const void*>(jac_fn), lds_jac, "LDS size of k_jacobi"},
      {reinterpret_cast<const void*>(apply_fn), lds_apply, "LDS size of k_apply"},
      {u4 ? reinterpret_cast<const void*>(&k_assemble_u4) : reinterpret_cast<const void*>(asm_u_fn),
       u4 ? lds_u : lds_u2, "LDS size of k_assemble_u"},
  };
  for (const auto& rq : lds_req) {
    e = hipFuncSetAttribute(rq.fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(rq.bytes));
    if (e != hipSuccess) return fail_stage(e, rq.name);
  }
  // Y = A Omega ; Q = orth(Y)
  // The last basis of range(A) also keeps its bf16 rounding remainder, so that the
  // projection C^T = A^T Q is taken with Q to about 16 bits (U is built from the
  // fp32 Q; with Q rounded to 8 bits here the two would disagree at 2^-9).
  e = gemm<T>(c, k, v, ws.omT, nullptr, ws.Y, false, (size_t)ellp * dm.W, st);
  if (e != hipSuccess) return fail_stage(e, "A Omega");
  e = orth<T>(c, ws, dm.N, ws.XT, dm.q == 0 ? ws.XTlo : nullptr, nullptr, dm.q == 0 ? 2 : 1,
              dm.q == 0 ? ws.Qn : nullptr, st);
  if (e != hipSuccess) return fail_stage(e, "orthonormalisation of A Omega");
  for (int it = 0; it < dm.q; ++it) {
    const bool final_basis = it == dm.q - 1;
    e = gemm<T>(c, k, v, ws.XT, nullptr, ws.Y, true, (size_t)ellp * ws.M, st);     // A^T Q
    if (e == hipSuccess) e = orth<T>(c, ws, dm.W, ws.XT, nullptr, nullptr, 1, nullptr, st);
    if (e == hipSuccess) e = gemm<T>(c, k, v, ws.XT, nullptr, ws.Y, false, (size_t)ellp * ws.M, st);  // A Q~
    if (e == hipSuccess)
      e = orth<T>(c, ws, dm.N, ws.XT, final_basis ? ws.XTlo : nullptr, nullptr, final_basis ? 2 : 1,
                  final_basis ? ws.Qn : nullptr, st);
    if (e != hipSuccess) return fail_stage(e, "power iteration");
  }
  // Q (fp32, kept in Qn for U), then C^T = A^T Q and its QR (basis kept in Qc for B)
  e = gemm<T>(c, k, v, ws.XT, ws.XTlo, ws.Y, true, (size_t)ellp * ws.M, st);
  if (e == hipSuccess) e = orth<T>(c, ws, dm.W, nullptr, nullptr, ws.Racc, 2, ws.Qc, st);
  if (e != hipSuccess) return fail_stage(e, "projection C^T = A^T Q");
  const int jac_threads = std::min(1024, std::max(64, (16 * ((dm.ell + 1) / 2) + 63) / 64 * 64));
  hipLaunchKernelGGL(jac_fn, dim3(nmat * jsplit), dim3(jac_threads), lds_jac, st, ws.Racc, dm.ell, ellp,
                     jsplit, ws.PS, ws.Sv, ws.sig);
  e = hipGetLastError();
  if (e != hipSuccess) return fail_stage(e, "core SVD");
  if (u4)
    hipLaunchKernelGGL(k_assemble_u4, dim3(nmat * dm.nblk), dim3(256), lds_u, st, ws.Qn, ws.PS,
                       static_cast<i4_t*>(c->Uk), reinterpret_cast<bf16_t*>(c->Usc), dm.N, ellp, dm.r,
                       dm.NP, dm.nblk);
  else
    hipLaunchKernelGGL(asm_u_fn, dim3(nmat * ((dm.N + 255) / 256)), dim3(256), lds_u2, st, ws.Qn, ws.PS,
                       static_cast<T*>(c->Uk), dm.N, dm.r, dm.nblk, (dm.N + 255) / 256);
  const int tiles_w = (dm.W + 255) / 256;
  hipLaunchKernelGGL(asm_b_fn, dim3(nmat * tiles_w), dim3(256), lds_b, st, ws.Qc, ws.Sv,
                     static_cast<T*>(c->Bk), static_cast<T*>(c->Bv), dm.W, dm.r, tiles_w);
  hipLaunchKernelGGL(k_copy_sigma, grid_1d((size_t)nmat * dm.r), dim3(256), 0, st, ws.sig, c->sigma_k,
                     c->sigma_v, nmat, ellp, dm.r);
  e = hipGetLastError();
  if (e != hipSuccess) return fail_stage(e, "factor assembly");
  release();
  return e;
}

hipError_t run_compress(ap_cache* c, const void* k, const void* v, hipStream_t st) {
  // 4-bit caches take bf16 K and V and keep B in bf16; only U's assembly differs
  if (c->dm.storage != AP_F32) return compress_t<bf16_t>(c, k, v, st, nullptr, 0);
  return compress_t<float>(c, k, v, st, nullptr, 0);
}

// ---------------------------------------------------------------- fixed workspace
// The factorisation workspace of the allocation-free re-factorisation: one fixed
// device array, which every GPU the library runs on holds until the process ends.
// Host code never passes the array's name to a kernel: on the host it is only a
// stand-in for the symbol.  Its device address on each GPU is looked up once per
// device (hipGetSymbolAddress with that device current) and kept.
static __device__ __align__(256) unsigned char scratch[kNoAllocWorkspaceBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_dev[64];   // per device: the address of that device's copy

static hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

hipError_t run_compress_noalloc(ap_cache* c, const void* k, const void* v, hipStream_t st) {
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) {
    set_error(std::string("ap_recompress_noalloc: device address of the fixed workspace: ") +
              hipGetErrorString(e));
    return e;
  }
  if (c->dm.storage != AP_F32) return compress_t<bf16_t>(c, k, v, st, ws, kNoAllocWorkspaceBytes);
  return compress_t<float>(c, k, v, st, ws, kNoAllocWorkspaceBytes);
}

}  // namespace ap

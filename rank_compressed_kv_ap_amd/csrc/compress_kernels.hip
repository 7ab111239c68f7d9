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
#include <type_traits>

#include "ap_internal.h"
#include "device_common.h"
#include "quant4.h"

namespace ap {

constexpr int kGemmThreads = 256;
constexpr int kMaxEll = 128;          // largest ell the LDS-resident Cholesky/Jacobi handle

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
  const size_t per = (size_t)ell * W;
  const size_t groups = (per + 7) / 8;
  const uint2 key = make_uint2(static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
  for (size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups * nmat;
       g += (size_t)gridDim.x * blockDim.x) {
    const int mat = static_cast<int>(g / groups);
    const size_t i0 = 8 * (g % groups);
    const size_t blk = i0 / 128;
    const uint4 x = philox4x32_10(make_uint4(static_cast<uint32_t>(blk), static_cast<uint32_t>(mat), 0u, 0u), key);
    const int t0 = static_cast<int>(i0 % 128);
    const uint32_t word = (t0 >> 5) == 0 ? x.x : ((t0 >> 5) == 1 ? x.y : ((t0 >> 5) == 2 ? x.z : x.w));
    const uint32_t bits = (word >> (t0 & 31)) & 0xffu;
    int j = static_cast<int>(i0 / W), w = static_cast<int>(i0 % W);
    const int cnt = static_cast<int>(per - i0 < 8 ? per - i0 : 8);
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
// Output Y[mat][m][j] (fp32, row stride ellp) for m in a 128-row tile:
//   TRANS = false: Y = A X,   A [M][K] rows m, X^T [ellp][K]        (M = N, K = W)
//   TRANS = true : Y = A^T X, A [K][M] columns m, X^T [ellp][K]     (M = W, K = N)
// A 64-wide k slice of A is staged in LDS as [128 m][64 k] (transposed on the way in
// for TRANS), so both MFMA operands read 8 consecutive k values per lane.  The next
// slice of A and of X is loaded into registers while the current one is multiplied
// (software pipelining: the loads of slice s+1 are in flight during the MFMAs of s).
constexpr int kGemmBM = 128, kGemmBK = 64, kGemmLdsStride = kGemmBK + 8;  // padded bf16 row

// VEC (W and K multiples of 8, K >= 8): every load of a slice is issued unconditionally,
// clamped in bounds, so the compiler tracks the slice in flight exactly and waits only
// for the slice being staged.  Past the edge of K the X^T values are zeroed, which
// cancels the clamped (finite) A values they meet; A values past M only reach output
// rows that are not stored.  Otherwise per-element fallbacks for unaligned rows.
template <class T, bool TRANS, int NT, bool SPLIT, bool VEC>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(const T* __restrict__ Kmat,
                                                        const T* __restrict__ Vmat,
                                                        const T* __restrict__ XT,
                                                        const T* __restrict__ XTlo, float* __restrict__ Y,
                                                        int N, int W, int ellp, size_t x_mat_stride,
                                                        int tiles_m) {
  static_assert(std::is_same<T, bf16_t>::value, "MFMA GEMM path is bf16");
  constexpr int XR = NT * 16;                        // rows of X^T (= ellp)
  constexpr int XU = (XR * 8 + kGemmThreads - 1) / kGemmThreads;   // 16-byte X loads per thread
  __shared__ __align__(16) bf16_t As[kGemmBM * kGemmLdsStride];
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
  const int m0 = tile * kGemmBM;
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
    uint4 a[4];
    uint4 x[XU];
    uint4 xl[SPLIT ? XU : 1];
  };
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
  auto load_slice = [&](int k0, Slice& sl) {
    if constexpr (VEC) {
      if (!TRANS) {
        // rows (tid >> 3) + 32 h, k = k0 + 8 (tid & 7) .. +7 (a run lies wholly inside K or past it)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int row = (tid >> 3) + 32 * h, gk = k0 + (tid & 7) * 8;
          const uint4 t = *reinterpret_cast<const uint4*>(A + (size_t)min(m0 + row, M - 1) * W + min(gk, K - 8));
          sl.a[h] = t;
        }
      } else {
        // k rows 4 (tid >> 4) + h, m = m0 + 8 (tid & 15) .. +7
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int gk = k0 + 4 * (tid >> 4) + h, gm = m0 + (tid & 15) * 8;
          sl.a[h] = *reinterpret_cast<const uint4*>(A + (size_t)min(gk, K - 1) * W + min(gm, M - 8));
        }
      }
#pragma unroll
      for (int u = 0; u < XU; ++u) {
        const int idx = min(tid + u * kGemmThreads, XR * 8 - 1);
        const int j = idx >> 3, gk = k0 + 8 * (idx & 7);
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
      // rows (tid >> 3) + 32 h, k = k0 + 8 (tid & 7) .. +7
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int row = (tid >> 3) + 32 * h, kk = (tid & 7) * 8;
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
      // k rows 4 (tid >> 4) + h, m = m0 + 8 (tid & 15) .. +7 (transposed into LDS later)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int kk = 4 * (tid >> 4) + h, mm = (tid & 15) * 8;
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
      const int idx = min(tid + u * kGemmThreads, XR * 8 - 1);
      const int j = idx >> 3, gk = k0 + 8 * (idx & 7);
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
      for (int h = 0; h < 4; ++h)
        *reinterpret_cast<uint4*>(&As[((tid >> 3) + 32 * h) * kGemmLdsStride + (tid & 7) * 8]) = sl.a[h];
    } else {
      // 4 k rows x 8 m columns in registers -> 8 columns of 4 consecutive k (8 bytes)
      const int kk = 4 * (tid >> 4), mm = (tid & 15) * 8;
      const uint32_t r0[4] = {sl.a[0].x, sl.a[0].y, sl.a[0].z, sl.a[0].w};
      const uint32_t r1[4] = {sl.a[1].x, sl.a[1].y, sl.a[1].z, sl.a[1].w};
      const uint32_t r2[4] = {sl.a[2].x, sl.a[2].y, sl.a[2].z, sl.a[2].w};
      const uint32_t r3[4] = {sl.a[3].x, sl.a[3].y, sl.a[3].z, sl.a[3].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint2 ev = make_uint2((r0[c] & 0xffffu) | (r1[c] << 16), (r2[c] & 0xffffu) | (r3[c] << 16));
        const uint2 od = make_uint2((r0[c] >> 16) | (r1[c] & 0xffff0000u), (r2[c] >> 16) | (r3[c] & 0xffff0000u));
        const int re = mm + 2 * c, ro = re + 1;   // 16-byte chunk kk / 8, 8-byte half (kk / 4) & 1
        *reinterpret_cast<uint2*>(&As[re * kGemmLdsStride + 8 * achunk(re, kk >> 3) + (kk & 4)]) = ev;
        *reinterpret_cast<uint2*>(&As[ro * kGemmLdsStride + 8 * achunk(ro, kk >> 3) + (kk & 4)]) = od;
      }
    }
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int idx = min(tid + u * kGemmThreads, XR * 8 - 1);
      const int o = (idx >> 3) * kGemmLdsStride + 8 * (idx & 7);
      *reinterpret_cast<uint4*>(&Xs[o]) = sl.x[u];
      if constexpr (SPLIT) *reinterpret_cast<uint4*>(&Xs[XR * kGemmLdsStride + o]) = sl.xl[u];
    }
  };

  auto multiply = [&]() {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
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

// fp32 storage: plain VALU products (small shapes only).
template <bool TRANS>
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ Kmat,
                                                  const float* __restrict__ Vmat,
                                                  const float* __restrict__ XT, float* __restrict__ Y,
                                                  int N, int W, int ellp, size_t x_mat_stride, int nmat) {
  const int M = TRANS ? W : N, K = TRANS ? N : W;
  const size_t total = (size_t)nmat * M * ellp;
  for (size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (size_t)gridDim.x * blockDim.x) {
    const int j = static_cast<int>(g % ellp);
    const int m = static_cast<int>((g / ellp) % M);
    const int mat = static_cast<int>(g / ((size_t)ellp * M));
    const float* A = ((mat & 1) ? Vmat : Kmat) + (size_t)(mat >> 1) * N * W;
    const float* x = XT + (size_t)mat * x_mat_stride + (size_t)j * K;
    float acc = 0.f;
    if (!TRANS) {
      for (int k = 0; k < K; ++k) acc = fmaf(A[(size_t)m * W + k], x[k], acc);
    } else {
      for (int k = 0; k < K; ++k) acc = fmaf(A[(size_t)k * W + m], x[k], acc);
    }
    Y[((size_t)mat * M + m) * ellp + j] = acc;
  }
}

// ================================================================ orthonormalisation
// Shifted Cholesky QR, two passes (CholeskyQR2 with a shift on the first Gram, in the
// spirit of Fukaya et al. 2020): G = Y^T Y, G + eps I = L L^T, Q = Y L^-T.
//
// k_gram: partial Grams.  Workgroup (mat, split) takes rows [split*rows, +rows) of
// Y [M][ellp]; each wavefront accumulates every upper 16x16 tile (fp32 MFMA 16x16x4,
// one 4-row slice per k-step) over its quarter of them, the four are summed in LDS
// and the workgroup writes Gpart[mat][split] (full, symmetric).  Deterministic:
// the partials are summed in a fixed order by k_chol.
constexpr int kGramThreads = 256;

template <int T>   // ellp / 16
__global__ __launch_bounds__(kGramThreads) void k_gram(const float* __restrict__ Y, int M, int ellp,
                                                       int rows, int nsplit, float* __restrict__ Gpart) {
  extern __shared__ __align__(16) float sh[];
  const int S = ellp + 1;
  float* G = sh;   // [ellp][S]
  const int mat = blockIdx.x / nsplit, split = blockIdx.x % nsplit;
  const float* Ym = Y + (size_t)mat * M * ellp;
  const int r0 = split * rows, r1 = min(M, r0 + rows);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  v4f acc[T * (T + 1) / 2];
#pragma unroll
  for (int t = 0; t < T * (T + 1) / 2; ++t) acc[t] = v4f{0, 0, 0, 0};
  constexpr int UR = 4;   // 4-row k-steps whose loads are in flight together
  for (int n0 = r0 + 4 * UR * wave; n0 < r1; n0 += 4 * UR * 4) {
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
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      int idx = 0;
#pragma unroll
      for (int ti = 0; ti < T; ++ti)
#pragma unroll
        for (int tj = ti; tj < T; ++tj, ++idx) acc[idx] = mfma_f32(y[u][ti], y[u][tj], acc[idx]);
    }
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
      int idx = 0;
#pragma unroll
      for (int ti = 0; ti < T; ++ti)
#pragma unroll
        for (int tj = ti; tj < T; ++tj, ++idx) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int i = 16 * ti + 4 * lg + t, j = 16 * tj + l16;
            const float v = acc[idx][t] + (w == 0 ? 0.f : G[i * S + j]);
            G[i * S + j] = v;
            if (ti != tj) G[j * S + i] = v;
          }
        }
    }
    __syncthreads();
  }
  float* out = Gpart + ((size_t)mat * nsplit + split) * ellp * ellp;
  for (int idx = tid; idx < ellp * ellp; idx += kGramThreads) {
    const int i = idx / ellp, j = idx % ellp;
    out[idx] = G[i * S + j];
  }
}

// Sum of the partial Grams in a fixed order (deterministic), four floats per thread.
__global__ __launch_bounds__(256) void k_gram_reduce(const float* __restrict__ Gpart, int nsplit, int nmat,
                                                     int e2, float* __restrict__ G) {
  const int e4 = e2 >> 2;   // e2 = ellp^2 is a multiple of 256
  const size_t total = (size_t)nmat * e4;
  for (size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x; g < total; g += (size_t)gridDim.x * blockDim.x) {
    const size_t mat = g / e4, i = g % e4;
    const float4* src = reinterpret_cast<const float4*>(Gpart + mat * nsplit * (size_t)e2) + i;
    float4 acc = src[0];
    for (int sp = 1; sp < nsplit; ++sp) {
      const float4 v = src[(size_t)sp * e4];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    reinterpret_cast<float4*>(G + mat * (size_t)e2)[i] = acc;
  }
}

// k_chol: one workgroup (4 wavefronts) per matrix, blocked over 16 x 16 tiles.
// Sums the partial Grams, adds the shift eps = 1e-6 * trace / ell (padded columns
// get a unit diagonal) and factors G + eps I = L L^T right-looking by block
// columns: the diagonal block is factored and inverted in registers by wavefront 0
// (lane i holds row i; values broadcast with readlane), the panel below it is
// L_IJ = A_IJ L_JJ^-T and the trailing update A_IK -= L_IJ L_KJ^T, both on fp32
// MFMA.  L^-1 follows by block forward substitution (X_IJ = -X_II sum_K L_IK X_KJ),
// Rinv = L^-T is written, and when Rout is given R = L^T Rprev (Rprev NULL:
// identity; Rprev may equal Rout: it is staged in LDS before R is written).
constexpr int kCholThreads = 256;

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

__global__ __launch_bounds__(kCholThreads) void k_chol(const float* __restrict__ Gpart, int nsplit, int ell,
                                                       int ellp, float* __restrict__ Rinv,
                                                       const float* __restrict__ Rprev,
                                                       float* __restrict__ Rout) {
  extern __shared__ __align__(16) float sh[];
  const int S = ellp + 1;
  float* G = sh;                 // [ellp][S] Gram, then L (lower; diagonal blocks exact)
  float* X = G + ellp * S;       // [ellp][S] L^-1, later Rprev
  float* Wk = X + ellp * S;      // [4][16][17] per-wavefront scratch tile
  const int mat = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int T = ellp / 16;
  const size_t e2 = (size_t)ellp * ellp;
  // ---- sum of the partial Grams (fixed order), X = 0.  16-byte loads, a batch of 8 per
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
        float* x = X + r * S + c;
        x[0] = 0.f; x[1] = 0.f; x[2] = 0.f; x[3] = 0.f;
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
  for (int idx = tid; idx < ellp * ellp; idx += kCholThreads) {
    const int i = idx / ellp, j = idx % ellp;
    if (i >= ell || j >= ell) G[i * S + j] = i == j ? 1.f : 0.f;
    else if (i == j) G[i * S + j] += eps;
  }
  __syncthreads();
  // ---- blocked Cholesky
  for (int J = 0; J < T; ++J) {
    const int c0 = 16 * J;
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
        for (int i = 0; i < 16; ++i) X[(c0 + i) * S + c0 + lane] = x[i];
      }
    }
    __syncthreads();
    // panel: L_IJ = A_IJ X_JJ^T
    for (int I = J + 1 + wave; I < T; I += 4) {
      const v4f p = tile_mma<false, true, false>(G, 16 * I, c0, S, X, c0, c0, S, v4f{0, 0, 0, 0}, l16, lg);
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
  // ---- L^-1 below the diagonal blocks, block row by block row
  float* wk = Wk + wave * 16 * 17;
  for (int I = 1; I < T; ++I) {
    for (int Jb = wave; Jb < I; Jb += 4) {
      v4f acc = v4f{0, 0, 0, 0};
      for (int K = Jb; K < I; ++K)
        acc = tile_mma<false, false, false>(G, 16 * I, 16 * K, S, X, 16 * K, 16 * Jb, S, acc, l16, lg);
      tile_store(wk, 0, 0, 17, l16, lg, acc);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const v4f xr = tile_mma<false, false, true>(X, 16 * I, 16 * I, S, wk, 0, 0, 17, v4f{0, 0, 0, 0}, l16, lg);
      tile_store(X, 16 * I, 16 * Jb, S, l16, lg, xr);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __syncthreads();
  }
  // ---- Rinv = X^T
  float* Ri = Rinv + (size_t)mat * e2;
  for (int idx = tid; idx < ellp * ellp; idx += kCholThreads) {
    const int i = idx / ellp, j = idx % ellp;
    Ri[idx] = X[j * S + i];
  }
  if (Rout == nullptr) return;
  __syncthreads();
  // ---- R = L^T Rprev
  const float4* Rp = Rprev ? reinterpret_cast<const float4*>(Rprev + (size_t)mat * e2) : nullptr;
  for (int i0 = 0; i0 < e4; i0 += 8 * kCholThreads) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = min(i0 + u * kCholThreads + tid, e4 - 1);
      if (Rp) {
        v[u] = Rp[i];
      } else {
        const int r = (4 * i) / ellp, c = 4 * i - r * ellp;
        v[u] = make_float4(r == c, r == c + 1, r == c + 2, r == c + 3);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kCholThreads + tid;
      if (i < e4) {
        const int r = (4 * i) / ellp, c = 4 * i - r * ellp;
        float* x = X + r * S + c;
        x[0] = v[u].x; x[1] = v[u].y; x[2] = v[u].z; x[3] = v[u].w;
      }
    }
  }
  __syncthreads();
  float* Ro = Rout + (size_t)mat * e2;
  for (int t = wave; t < T * T; t += 4) {
    const int I = t / T, Jb = t % T;
    v4f acc = v4f{0, 0, 0, 0};
    for (int K = I; K < T; ++K)
      acc = tile_mma<true, false, false>(G, 16 * K, 16 * I, S, X, 16 * K, 16 * Jb, S, acc, l16, lg);
#pragma unroll
    for (int u = 0; u < 4; ++u) Ro[(size_t)(16 * I + 4 * lg + u) * ellp + 16 * Jb + l16] = acc[u];
  }
}

// Row tile of k_apply.
static int apply_rows(int) { return 64; }

// Q = Y Rinv for a tile of rows per workgroup (fp32 MFMA), written to Qout (Y itself for
// a basis that is orthonormalised again, another buffer for a basis kept for the
// factors, or nowhere when only Q^T is used); optionally Q^T in storage precision for
// the next product (XT[mat][j][m]), and the rounding remainder Q^T - XT in XTlo for a
// two-term product.  The Q tile is kept in LDS so that Q^T leaves in 16-byte runs along m.
template <class T>
__global__ __launch_bounds__(256) void k_apply(const float* Y, float* Qout, int M, int ellp,
                                               const float* __restrict__ Rinv, T* __restrict__ XT,
                                               T* __restrict__ XTlo, size_t xt_mat_stride, int tiles_m,
                                               int rows) {
  extern __shared__ __align__(16) float sh[];
  constexpr int kMaxRT = 2, kMaxCT = kMaxEll / 16;   // row tiles per wavefront (rows <= 128)
  const int nrt = rows / 64;                          // rows is 64 or 128
  const int S = ellp + 1;
  float* Ys = sh;                  // [rows][S]
  float* Rs = Ys + rows * S;       // [ellp][ellp]
  const int mat = blockIdx.x / tiles_m;
  const int m0 = (blockIdx.x % tiles_m) * rows;
  const float* Ym = Y + (size_t)mat * M * ellp;
  float* Qm = Qout != nullptr ? Qout + (size_t)mat * M * ellp : nullptr;
  const float* Rm = Rinv + (size_t)mat * ellp * ellp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  // stage the Y tile and R^-1: 16-byte loads, 8 independent ones in flight per thread
  // (indices clamped so every load is issued; rows past M are zeroed after the load)
  const int ell4 = ellp / 4;   // ellp is a multiple of 16
  const int ny = rows * ell4, nr = ellp * ell4;
  for (int i0 = 0; i0 < ny + nr; i0 += 8 * 256) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = min(i0 + u * 256 + tid, ny + nr - 1);
      if (idx < ny) {
        const int r = idx / ell4, j4 = idx - r * ell4;
        v[u] = *reinterpret_cast<const float4*>(Ym + (size_t)min(m0 + r, M - 1) * ellp + 4 * j4);
      } else {
        v[u] = *reinterpret_cast<const float4*>(Rm + (size_t)4 * (idx - ny));
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = i0 + u * 256 + tid;
      if (idx < ny) {
        const int r = idx / ell4, j4 = idx - r * ell4;
        const bool live = m0 + r < M;
        float* d = Ys + r * S + 4 * j4;
        d[0] = live ? v[u].x : 0.f;
        d[1] = live ? v[u].y : 0.f;
        d[2] = live ? v[u].z : 0.f;
        d[3] = live ? v[u].w : 0.f;
      } else if (idx < ny + nr) {
        *reinterpret_cast<float4*>(Rs + 4 * (idx - ny)) = v[u];
      }
    }
  }
  __syncthreads();
  const int T16 = ellp / 16;
  // wave owns row tiles wave and wave + 4 (16 rows each), all column tiles
  v4f acc[kMaxRT][kMaxCT];
#pragma unroll
  for (int i = 0; i < kMaxRT; ++i)
#pragma unroll
    for (int c = 0; c < kMaxCT; ++c) acc[i][c] = v4f{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < kMaxRT; ++i) {
    const int rt = wave + 4 * i;
    if (i >= nrt) break;
    for (int k0 = 0; k0 < ellp; k0 += 4) {
      const float a = Ys[(16 * rt + l16) * S + k0 + lg];
#pragma unroll
      for (int c = 0; c < kMaxCT; ++c)
        if (c < T16) acc[i][c] = mfma_f32(a, Rs[(k0 + lg) * ellp + 16 * c + l16], acc[i][c]);
    }
  }
  __syncthreads();   // every read of the Y tile is done: it now takes Q
#pragma unroll
  for (int i = 0; i < kMaxRT; ++i) {
    const int rt = wave + 4 * i;
    if (i >= nrt) break;
#pragma unroll
    for (int c = 0; c < kMaxCT; ++c) {
      if (c >= T16) continue;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 16 * rt + 4 * lg + t, j = 16 * c + l16;
        Ys[r * S + j] = acc[i][c][t];
        if (Qm != nullptr && m0 + r < M) Qm[(size_t)(m0 + r) * ellp + j] = acc[i][c][t];
      }
    }
  }
  if (XT == nullptr) return;
  __syncthreads();
  // Q^T[j][m0 .. m0 + rows): 8 consecutive m per thread
  const int R8 = rows / 8;
  T* xt = XT + (size_t)mat * xt_mat_stride;
  T* xl = XTlo != nullptr ? XTlo + (size_t)mat * xt_mat_stride : nullptr;
  const bool vec = std::is_same<T, bf16_t>::value && (M & 7) == 0;
  for (int idx = tid; idx < ellp * R8; idx += 256) {
    const int j = idx / R8, m8 = idx - (idx / R8) * R8;
    const int mb = m0 + 8 * m8;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = Ys[(8 * m8 + e) * S + j];
    if (vec && mb + 8 <= M) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hw[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        const float r0 = v[2 * e] - __uint_as_float(hw[e] << 16);
        const float r1 = v[2 * e + 1] - __uint_as_float(hw[e] & 0xffff0000u);
        lw[e] = pack_bf16x2(r0, r1);
      }
      *reinterpret_cast<uint4*>(xt + (size_t)j * M + mb) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      if (xl != nullptr) *reinterpret_cast<uint4*>(xl + (size_t)j * M + mb) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    } else {
      for (int e = 0; e < 8; ++e) {
        if (mb + e >= M) break;
        const T hi = from_f32<T>(v[e]);
        xt[(size_t)j * M + mb + e] = hi;
        if (xl != nullptr) xl[(size_t)j * M + mb + e] = from_f32<T>(v[e] - to_f32<T>(hi));
      }
    }
  }
}

// ================================================================ core SVD
// One-sided Jacobi on the columns of Mj = R^T (ell x ell, LDS): rotations make the
// columns mutually orthogonal, Mj J = P Sigma, J = S.  Round-robin (tournament) pair
// order; one 16-lane group per pair, each lane holding every 16th row, reductions
// by DPP inside the group; a step's E/2 disjoint pairs run at once, one barrier per
// step.  Stops when every pair is orthogonal to 3e-6 relative (fp32), or after 40
// sweeps.
__global__ __launch_bounds__(1024) void k_jacobi(const float* __restrict__ Rm, int ell, int ellp,
                                                 float* __restrict__ PS, float* __restrict__ Sv,
                                                 float* __restrict__ sig) {
  extern __shared__ __align__(16) float sh[];
  const int S = ellp + 1;
  const int E = (ell + 1) & ~1;            // even number of columns for the tournament
  float* Mj = sh;                          // [ellp][S]  (row i, column j)
  float* J = Mj + ellp * S;                // [ellp][S]
  float* nrm = J + ellp * S;               // [ellp]
  int* perm = reinterpret_cast<int*>(nrm + ellp);  // [ellp]
  __shared__ unsigned int rotated;
  const int mat = blockIdx.x;
  const float* R = Rm + (size_t)mat * ellp * ellp;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int l16 = tid & 15, slot = tid >> 4, nslot = nthr >> 4;
  for (int idx = tid; idx < ellp * ellp; idx += nthr) {
    const int i = idx / ellp, j = idx % ellp;
    Mj[i * S + j] = (i < ell && j < ell) ? R[j * ellp + i] : 0.f;   // transpose
    J[i * S + j] = i == j ? 1.f : 0.f;
  }
  __syncthreads();
  for (int sweep = 0; sweep < 40; ++sweep) {
    if (tid == 0) rotated = 0u;
    __syncthreads();
    for (int step = 0; step < E - 1; ++step) {
      for (int pr = slot; pr < E / 2; pr += nslot) {
        const int x0 = pr, x1 = E - 1 - pr;
        int p = x0 == 0 ? 0 : 1 + (x0 - 1 + step) % (E - 1);
        int qq = 1 + (x1 - 1 + step) % (E - 1);
        if (p > qq) { const int t = p; p = qq; qq = t; }
        if (qq >= ell) continue;           // uniform over the 16-lane group
        // rows ell..ellp-1 of Mj are zero: the loops run over ellp rows, unrolled with a
        // wavefront-uniform bound so that the LDS reads of a column issue together
        float a = 0.f, bsum = 0.f, g = 0.f;
#pragma unroll
        for (int k = 0; k < kMaxEll / 16; ++k) {
          if (16 * k >= ellp) break;
          const int i = l16 + 16 * k;
          const float x = Mj[i * S + p], y = Mj[i * S + qq];
          a = fmaf(x, x, a);
          bsum = fmaf(y, y, bsum);
          g = fmaf(x, y, g);
        }
        a = group_sum(a, 16);
        bsum = group_sum(bsum, 16);
        g = group_sum(g, 16);
        if (g == 0.f || fabsf(g) <= 3e-6f * sqrtf(a * bsum)) continue;
        if (l16 == 0) rotated = 1u;
        // rotation angle from the hardware reciprocal and reciprocal square root (about
        // 1 ulp each): any rotation close to the exact one is orthogonal to within
        // rounding (c^2 + s^2 = 1), and the next sweep measures what is left
        const float zeta = (bsum - a) * __builtin_amdgcn_rcpf(2.f * g);
        const float t = copysignf(__builtin_amdgcn_rcpf(fabsf(zeta) + __builtin_amdgcn_sqrtf(fmaf(zeta, zeta, 1.f))), zeta);
        const float c = __builtin_amdgcn_rsqf(fmaf(t, t, 1.f)), s = c * t;
#pragma unroll
        for (int k = 0; k < kMaxEll / 16; ++k) {
          if (16 * k >= ellp) break;
          const int i = l16 + 16 * k;
          const float x = Mj[i * S + p], y = Mj[i * S + qq];
          Mj[i * S + p] = c * x - s * y;
          Mj[i * S + qq] = s * x + c * y;
          const float u = J[i * S + p], v = J[i * S + qq];
          J[i * S + p] = c * u - s * v;
          J[i * S + qq] = s * u + c * v;
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
  for (int idx = tid; idx < ellp * ellp; idx += nthr) {
    const int i = idx / ellp, c = idx % ellp;
    const int j = perm[c];
    PSm[idx] = Mj[i * S + j];
    Sm[idx] = J[i * S + j];
  }
  for (int c = tid; c < ellp; c += nthr) sig[(size_t)mat * ellp + c] = fmaxf(nrm[perm[c]], 0.f);
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

// U[n][i] = sum_j Qn[n][j] PS[j][i] (i < r) into the decode tiles of one 32-token block;
// the block's 32 rows of Qn and the r_pad used columns of PS are staged in LDS, their
// product formed on fp32 MFMA (16 x 16 tiles, one or two per wavefront) into LDS.
template <class T>
__global__ __launch_bounds__(256) void k_assemble_u(const float* __restrict__ Qn, const float* __restrict__ PS,
                                                    T* __restrict__ Ukv, int N, int ellp, int r, int NP,
                                                    int nblk) {
  extern __shared__ __align__(16) float sh[];
  const int rp = 16 * NP, ld = rp + 1;
  float* Qs = sh;                      // [32][ellp + 1]
  float* Ps = Qs + 32 * (ellp + 1);    // [ellp][rp]
  float* Ub = Ps + ellp * rp;          // [32][ld]
  const int mat = blockIdx.x / nblk, t = blockIdx.x % nblk;
  const int b = mat >> 1;
  const bool vl = mat & 1;
  const float* Q = Qn + (size_t)mat * N * ellp;
  const float* P = PS + (size_t)mat * ellp * ellp;
  stage_f32(Qs, ellp + 1, Q + (size_t)kBlockTok * t * ellp, ellp, 32, ellp, N - kBlockTok * t, ellp);
  stage_f32(Ps, rp, P, ellp, ellp, rp, ellp, r);
  __syncthreads();
  {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, lg = lane >> 4;
    for (int tl = wave; tl < 2 * NP; tl += 4) {   // tile tl: rows 16 (tl & 1), columns 16 (tl >> 1)
      v4f acc = v4f{0, 0, 0, 0};
      for (int kb = 0; kb < ellp; kb += 16)
        acc = tile_mma<false, false, false>(Qs, 16 * (tl & 1), kb, ellp + 1, Ps, kb, 16 * (tl >> 1), rp, acc,
                                            l16, lg);
      tile_store(Ub, 16 * (tl & 1), 16 * (tl >> 1), ld, l16, lg, acc);
    }
  }
  __syncthreads();
  T* base = Ukv + (vl ? (size_t)NP * kBlockElems : 0);
  for (int idx = threadIdx.x; idx < NP * kBlockElems; idx += blockDim.x) {
    const int p = idx / kBlockElems, within = idx % kBlockElems;
    const int e = within & 3, half = (within >> 2) & 1, lane = within >> 3;
    int rr, col;
    if (!vl) {
      rr = 16 * half + (lane & 15);
      col = 16 * p + 4 * (lane >> 4) + e;
    } else {
      rr = 16 * half + 4 * (lane >> 4) + e;
      col = 16 * p + (lane & 15);
    }
    base[tile_base(b, p, t, NP, nblk) + within] = from_f32<T>(Ub[rr * ld + col]);
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

// B[i][w] = sum_j Qc[w][j] S[j][i] for i < r (rows r..r_pad-1 stay zero).  One
// workgroup per (matrix, 64 columns w): the 64 rows of Qc and S[:, :r_pad] are staged
// in LDS; each thread accumulates a 4 (i) x 4 (w) block and stores 4 consecutive w.
template <class T>
__global__ __launch_bounds__(256) void k_assemble_b(const float* __restrict__ Qc, const float* __restrict__ Sv,
                                                    T* __restrict__ Bk, T* __restrict__ Bv, int W, int ellp,
                                                    int r, int r_pad, int tiles_w) {
  extern __shared__ __align__(16) float sh[];
  const int QS = ellp + 1;
  float* Qs = sh;                 // [64][QS]
  float* Ss = Qs + 64 * QS;       // [ellp][r_pad]
  const int mat = blockIdx.x / tiles_w;
  const int w0 = (blockIdx.x % tiles_w) * 64;
  const float* Q = Qc + (size_t)mat * W * ellp;
  const float* Sm = Sv + (size_t)mat * ellp * ellp;
  stage_f32(Qs, QS, Q + (size_t)w0 * ellp, ellp, 64, ellp, W - w0, ellp);
  stage_f32(Ss, r_pad, Sm, ellp, ellp, r_pad, ellp, r);
  __syncthreads();
  T* B = ((mat & 1) ? Bv : Bk) + (size_t)(mat >> 1) * r_pad * W;
  const int wb = (threadIdx.x & 15) * 4;          // 4 consecutive columns
  for (int ib = (threadIdx.x >> 4) * 4; ib < r; ib += 64) {
    float acc[4][4] = {};
    for (int j = 0; j < ellp; ++j) {
      const float4 sv = *reinterpret_cast<const float4*>(&Ss[j * r_pad + ib]);
      const float sj[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float q = Qs[(wb + c) * QS + j];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u][c] = fmaf(q, sj[u], acc[u][c]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = ib + u;
      if (i >= r) break;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (w0 + wb + c < W) B[(size_t)i * W + w0 + wb + c] = from_f32<T>(acc[u][c]);
    }
  }
}

__global__ void k_copy_sigma(const float* __restrict__ sig, float* __restrict__ sk, float* __restrict__ sv,
                             int nmat, int ellp, int r) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= nmat * r) return;
  const int mat = g / r, i = g % r;
  ((mat & 1) ? sv : sk)[(size_t)(mat >> 1) * r + i] = sig[(size_t)mat * ellp + i];
}

// ================================================================ driver
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
    const int tiles_m = (M + kGemmBM - 1) / kGemmBM;
    const dim3 grid(nmat * tiles_m);
    const int K = trans ? dm.N : dm.W;
    const bool vec = dm.W % 8 == 0 && K % 8 == 0 && K >= 8;
#define AP_GEMM_LAUNCH_V(TR, NTV, SP, VC)                                                               \
  hipLaunchKernelGGL((k_gemm<bf16_t, TR, NTV, SP, VC>), grid, dim3(kGemmThreads), 0, st,               \
                     static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),                     \
                     static_cast<const bf16_t*>(XT), static_cast<const bf16_t*>(XTlo), Y, dm.N, dm.W, \
                     ellp, x_stride, tiles_m)
#define AP_GEMM_LAUNCH(TR, NTV, SP)                                                                     \
  do {                                                                                                  \
    if (vec) AP_GEMM_LAUNCH_V(TR, NTV, SP, true);                                                       \
    else AP_GEMM_LAUNCH_V(TR, NTV, SP, false);                                                          \
  } while (0)
#define AP_GEMM_CASE(NTV)                                                                              \
  case NTV:                                                                                            \
    if (trans && XTlo != nullptr) AP_GEMM_LAUNCH(true, NTV, true);                                     \
    else if (trans) AP_GEMM_LAUNCH(true, NTV, false);                                                  \
    else AP_GEMM_LAUNCH(false, NTV, false);                                                            \
    break;
    switch (ellp / 16) {
      AP_GEMM_CASE(1) AP_GEMM_CASE(2) AP_GEMM_CASE(3) AP_GEMM_CASE(4)
      AP_GEMM_CASE(5) AP_GEMM_CASE(6) AP_GEMM_CASE(7) AP_GEMM_CASE(8)
      default: return hipErrorInvalidValue;
    }
#undef AP_GEMM_CASE
#undef AP_GEMM_LAUNCH
#undef AP_GEMM_LAUNCH_V
  } else {
    if (trans)
      hipLaunchKernelGGL((k_gemm_f32<true>), grid_1d((size_t)nmat * M * ellp), dim3(256), 0, st,
                         static_cast<const float*>(k), static_cast<const float*>(v),
                         static_cast<const float*>(XT), Y, dm.N, dm.W, ellp, x_stride, nmat);
    else
      hipLaunchKernelGGL((k_gemm_f32<false>), grid_1d((size_t)nmat * M * ellp), dim3(256), 0, st,
                         static_cast<const float*>(k), static_cast<const float*>(v),
                         static_cast<const float*>(XT), Y, dm.N, dm.W, ellp, x_stride, nmat);
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
  const size_t lds_gram = (size_t)ellp * (ellp + 1) * sizeof(float);
  const size_t lds_chol = (size_t)(2 * ellp * (ellp + 1) + 4 * 16 * 17) * sizeof(float);
  const int arows = apply_rows(ellp);
  const size_t lds_apply = (size_t)(arows * (ellp + 1) + ellp * ellp) * sizeof(float);
  const int tiles_m = (M + arows - 1) / arows;
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
      AP_GRAM_CASE(5) AP_GRAM_CASE(6) AP_GRAM_CASE(7) AP_GRAM_CASE(8)
#undef AP_GRAM_CASE
      default: return hipErrorInvalidValue;
    }
    const float* Gsum = ws.Gpart;
    if (nsplit > 1) {
      hipLaunchKernelGGL(k_gram_reduce, grid_1d((size_t)nmat * ellp * ellp / 4), dim3(256), 0, st, ws.Gpart,
                         nsplit, nmat, ellp * ellp, ws.Gsum);
      Gsum = ws.Gsum;
    }
    hipLaunchKernelGGL(k_chol, dim3(nmat), dim3(kCholThreads), lds_chol, st, Gsum, 1, dm.ell, ellp,
                       ws.Rinv, pass == 0 ? nullptr : Racc, Racc);
    hipLaunchKernelGGL(k_apply<T>, dim3(nmat * tiles_m), dim3(256), lds_apply, st, ws.Y, last ? Qlast : ws.Y, M,
                       ellp, ws.Rinv,
                       static_cast<T*>(last ? XT : nullptr), static_cast<T*>(last ? XTlo : nullptr),
                       (size_t)ellp * ws.M, tiles_m, arows);
  }
  return hipGetLastError();
}

template <class T>
static hipError_t compress_t(ap_cache* c, const void* k, const void* v, hipStream_t st) {
  const Dims& dm = c->dm;
  CompressWs ws;
  ws.nmat = 2 * dm.B;
  ws.M = std::max(dm.N, dm.W);
  ws.ellp = (dm.ell + 15) / 16 * 16;
  if (ws.ellp > kMaxEll) {
    set_error("ap_compress: ell = min(rank + oversample, n_tokens, width) must be <= 128");
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
  for (Buf& bf : bufs) {
    if (bf.bytes == 0) continue;
    e = hipMallocAsync(bf.p, bf.bytes, st);
    if (e != hipSuccess) break;
  }
  auto release = [&]() {
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
  // padded rows of Omega^T and X^T must read as zero
  e = hipMemsetAsync(ws.omT, 0, (size_t)nmat * ellp * dm.W * es, st);
  if (e == hipSuccess) e = hipMemsetAsync(ws.XT, 0, (size_t)nmat * ellp * ws.M * es, st);
  if (e == hipSuccess && ws.XTlo) e = hipMemsetAsync(ws.XTlo, 0, (size_t)nmat * ellp * ws.M * es, st);
  if (e != hipSuccess) return fail_stage(e, "workspace clear");
  if (c->params.omega != nullptr)
    hipLaunchKernelGGL(k_omega_copy<T>, grid_1d((size_t)nmat * dm.ell * dm.W), dim3(256), 0, st,
                       c->params.omega, static_cast<T*>(ws.omT), nmat, dm.W, dm.ell, ellp);
  else
    hipLaunchKernelGGL(k_omega_philox<T>, grid_1d((size_t)nmat * ((dm.ell * (size_t)dm.W + 7) / 8)),
                       dim3(256), 0, st, static_cast<T*>(ws.omT), nmat, dm.W, dm.ell, ellp, c->params.seed);
  e = hipGetLastError();
  if (e != hipSuccess) return fail_stage(e, "test matrix");

  // dynamic LDS above the 64 KB default: request exactly what each launch uses
  const size_t lds_chol = (size_t)(2 * ellp * (ellp + 1) + 4 * 16 * 17) * sizeof(float);
  const size_t lds_jac = (size_t)(2 * ellp * (ellp + 1) + 2 * ellp) * sizeof(float);
  const size_t lds_apply = (size_t)(apply_rows(ellp) * (ellp + 1) + ellp * ellp) * sizeof(float);
  const bool u4 = dm.storage == AP_INT4;
  const size_t lds_u = (size_t)(32 * (ellp + 1) + ellp * 16 * dm.NP + 32 * (16 * dm.NP + 1) +
                                (u4 ? 16 * dm.NP : 0)) * sizeof(float);
  const size_t lds_b = (size_t)(64 * (ellp + 1) + ellp * dm.r_pad) * sizeof(float);
  const struct { const void* fn; size_t bytes; const char* name; } lds_req[] = {
      {reinterpret_cast<const void*>(&k_gram<8>), (size_t)ellp * (ellp + 1) * sizeof(float), "LDS size of k_gram"},
      {reinterpret_cast<const void*>(&k_chol), lds_chol, "LDS size of k_chol"},
      {reinterpret_cast<const void*>(&k_assemble_b<T>), lds_b, "LDS size of k_assemble_b"},
      {reinterpret_cast<const void*>(&k_jacobi), lds_jac, "LDS size of k_jacobi"},
      {reinterpret_cast<const void*>(&k_apply<T>), lds_apply, "LDS size of k_apply"},
      {u4 ? reinterpret_cast<const void*>(&k_assemble_u4) : reinterpret_cast<const void*>(&k_assemble_u<T>),
       lds_u, "LDS size of k_assemble_u"},
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
  hipLaunchKernelGGL(k_jacobi, dim3(nmat), dim3(jac_threads), lds_jac, st, ws.Racc, dm.ell, ellp, ws.PS,
                     ws.Sv, ws.sig);
  e = hipGetLastError();
  if (e != hipSuccess) return fail_stage(e, "core SVD");
  if (u4)
    hipLaunchKernelGGL(k_assemble_u4, dim3(nmat * dm.nblk), dim3(256), lds_u, st, ws.Qn, ws.PS,
                       static_cast<i4_t*>(c->Uk), reinterpret_cast<bf16_t*>(c->Usc), dm.N, ellp, dm.r,
                       dm.NP, dm.nblk);
  else
    hipLaunchKernelGGL(k_assemble_u<T>, dim3(nmat * dm.nblk), dim3(256), lds_u, st, ws.Qn, ws.PS,
                       static_cast<T*>(c->Uk), dm.N, ellp, dm.r, dm.NP, dm.nblk);
  const int tiles_w = (dm.W + 63) / 64;
  hipLaunchKernelGGL(k_assemble_b<T>, dim3(nmat * tiles_w), dim3(256), lds_b, st, ws.Qc, ws.Sv,
                     static_cast<T*>(c->Bk), static_cast<T*>(c->Bv), dm.W, ellp, dm.r, dm.r_pad, tiles_w);
  hipLaunchKernelGGL(k_copy_sigma, grid_1d((size_t)nmat * dm.r), dim3(256), 0, st, ws.sig, c->sigma_k,
                     c->sigma_v, nmat, ellp, dm.r);
  e = hipGetLastError();
  if (e != hipSuccess) return fail_stage(e, "factor assembly");
  release();
  return e;
}

hipError_t run_compress(ap_cache* c, const void* k, const void* v, hipStream_t st) {
  // 4-bit caches take bf16 K and V and keep B in bf16; only U's assembly differs
  if (c->dm.storage != AP_F32) return compress_t<bf16_t>(c, k, v, st);
  return compress_t<float>(c, k, v, st);
}

}  // namespace ap

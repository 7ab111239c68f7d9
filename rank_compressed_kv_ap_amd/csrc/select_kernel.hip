// Per-head top-k selection of the tokens decompressed at full rank (gfx950).
//
// [fr §2.B "Stratégie"]: the most important tokens get the full rank R, the others a
// reduced rank; [es §4 "Análisis de Sensibilidad"]: 25% at full rank.  Importance of
// token n for query head h is its low-rank logit s_lo = U_k[n, :r_lo] . q~_h[:r_lo];
// the k largest are chosen, ties to the lower token index.
//
// One workgroup per (sequence, group of query heads):
//  0. latent queries q~_h = B_k[:, head g's columns] q_h (written for the flash-decode
//     kernel as well);
//  1. low-rank scores of every token by MFMA; each score is mapped to a 16-bit bin by a
//     monotone linear map over [-M_h, M_h], where M_h = |q~_h[:r_lo]| * max_n |U_k[n,:r_lo]|
//     bounds |s_lo| (Cauchy-Schwarz).  Bins (2 bytes per token) stay in LDS;
//  2. two 8-bit histogram passes over the bins locate the bin b* holding the k-th
//     largest score and how many of its tokens are still needed;
//  3. if only part of b* is taken, its tokens' exact scores are recomputed (same MFMA
//     sequence, so bit-identical) and ranked exactly by (score desc, index asc); if b*
//     is very large (ties, a zero query) an exact radix select over recomputed 32-bit
//     keys decides instead;
//  4. one wavefront per head writes the selection bitmask per 32-token block (and, on
//     request, the ascending selected ids).
#include <hip/hip_ext.h>

#include "ap_internal.h"
#include "device_common.h"
#include "tiles.h"

namespace ap {

constexpr int kSelThreads = 512;     // 8 wavefronts
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kMaxHg = 8;             // heads per workgroup (one wavefront per head in per-head steps)
constexpr int kSelCap = 128;          // boundary-bin tokens resolved by exact ranking
constexpr int kSelList = 512;         // tokens of the coarse boundary digit remembered per head

enum SelMode : int { kNone = 0, kAll = 1, kWholeBin = 2, kRank = 3, kRadix = 4 };

struct SelState {
  int nlist;      // tokens of the coarse boundary digit (list holds the first kSelList)
  int bstar;      // boundary bin (coarse digit after the first pass)
  int need;       // tokens still to take inside the boundary bin
  int cnt;        // tokens in the boundary bin
  int mode;
  int ncand;      // candidates gathered (kRank)
  uint32_t tau;   // kRadix: key of the k-th token
  unsigned long long thr;  // kRank: composite (key << 32 | ~index) of the k-th token
};

struct SelLayout {
  size_t bins, hc, selb, qs, mm, st, bflag, list, total;
};

// hc holds the 256-bin histogram of each head, later its candidates (kSelCap x 8 bytes);
// selb holds the q vectors while the latent queries are formed, later the selected-token
// bits of the boundary bin.
__host__ __device__ inline SelLayout sel_layout(int Hg, int N_pad, int nblk, int r_pad, int d) {
  auto up = [](size_t x) { return (x + 15) & ~(size_t)15; };
  SelLayout L;
  size_t o = 0;
  L.bins = o;  o = up(o + (size_t)Hg * N_pad * 2);
  L.hc = o;    o = up(o + (size_t)Hg * 256 * 4);
  L.selb = o;  o = up(o + (size_t)Hg * (nblk > d ? nblk : d) * 4);
  L.qs = o;    o = up(o + (size_t)Hg * r_pad * 4);
  L.mm = o;    o = up(o + (size_t)Hg * 2 * 4);
  L.st = o;    o = up(o + (size_t)Hg * sizeof(SelState));
  L.bflag = o; o = up(o + (size_t)nblk * 4);
  L.list = o;  o = up(o + (size_t)Hg * kSelList * 2);
  L.total = o;
  return L;
}

// Monotone map of a score to a 16-bit bin: floor((s + M) * mul) clamped to [0, 65535],
// computed as one fused multiply-add (Mmul = M * mul) and a median-of-three clamp.
__device__ __forceinline__ uint32_t score_bin(float s, float Mmul, float mul) {
  const float x = __builtin_amdgcn_fmed3f(fmaf(s, mul, Mmul), 0.f, 65535.f);
  return static_cast<uint32_t>(x);
}

// Low-rank score operand of panel p for this lane (head l%16, columns 16p+4(l/16)+e < r_lo).
template <class T>
__device__ __forceinline__ QOp<T> low_qop(const float* qs, int r_pad, int nh, int r_lo, int p, int lane) {
  const int l16 = lane & 15, c0 = 16 * p + 4 * (lane >> 4);
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (l16 < nh && c0 + e < r_lo) ? qs[l16 * r_pad + c0 + e] : 0.f;
  QOp<T> qo;
  qo.set(v);
  return qo;
}

// Scores of the 32 tokens of block blk (lane head = l%16); the MFMA sequence is the same
// one every pass uses, so a recomputed score is bit-identical to the first.
template <class T>
__device__ __forceinline__ void score_block(const T* __restrict__ Uk, int b, int blk, int NP,
                                            int nblk, int r_lo, const float* qs, int r_pad,
                                            int nh, int lane, v4f& a0, v4f& a1) {
  const int nplo = (r_lo + 15) >> 4;
  a0 = v4f{0, 0, 0, 0};
  a1 = v4f{0, 0, 0, 0};
  for (int p = 0; p < nplo; ++p) {
    LaneTile<T> a;
    a.load(Uk + tile_base(b, p, blk, NP, nblk), lane);
    const QOp<T> qo = low_qop<T>(qs, r_pad, nh, r_lo, p, lane);
    a0 = score_mma(a, 0, qo, a0);
    a1 = score_mma(a, 1, qo, a1);
  }
}

// Wavefront search over a 256-bin histogram (descending digit order): the digit D whose
// bin holds the need-th largest element, and how many elements lie in bins above D.
__device__ __forceinline__ bool digit_search(const uint32_t* hist, uint32_t need, int lane,
                                             int* digit, uint32_t* above, uint32_t* in_bin) {
  const uint4 c4 = *reinterpret_cast<const uint4*>(hist + 252 - 4 * lane);  // bins 252-4l..255-4l
  const uint32_t c0 = c4.w, c1 = c4.z, c2 = c4.y, c3 = c4.x;               // descending digits
  const uint32_t tot = c0 + c1 + c2 + c3;
  uint32_t incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  const uint32_t excl = incl - tot;
  if (!(excl < need && incl >= need)) return false;
  uint32_t run = excl;
  int e = 0;
  uint32_t c = c0;
  if (run + c0 < need) { run += c0; e = 1; c = c1;
    if (run + c1 < need) { run += c1; e = 2; c = c2;
      if (run + c2 < need) { run += c2; e = 3; c = c3; } } }
  *digit = 255 - (4 * lane + e);
  *above = run;
  *in_bin = c;
  return true;
}

// UB: blocks per wavefront whose U_k loads are in flight at once (12 or 16 with one low
// panel, 8 with two); UB == 0 walks blocks one at a time (more than two low panels).
template <class T, int UB>
__global__ __launch_bounds__(kSelThreads) void k_select(
    const T* __restrict__ Uk, const T* __restrict__ Bk, const float* __restrict__ rn,
    const float* __restrict__ q, float* __restrict__ qt, uint32_t* __restrict__ mask,
    int32_t* __restrict__ sel_out, int B, int N, int N_pad, int nblk, int NP, int r_pad, int W,
    int d, int G, int Hq, int Hq_pad, int Hg, int HG, int r_lo, int top_k) {
  constexpr int NPL = UB >= 12 ? 1 : 2;   // low panels held per block
  constexpr int UBA = UB > 0 ? UB : 1;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  // All head groups of one sequence share blockIdx % 8 (one XCD), so its L2 serves
  // the repeated reads of U_k's low panels.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int b = (slot / HG) * 8 + xcd;
  const int hg = slot % HG;
  if (b >= B) return;
  const int h0 = hg * Hg;
  const int nh = min(Hg, Hq - h0);
  if (nh <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;

  const SelLayout Ly = sel_layout(Hg, N_pad, nblk, r_pad, d);
  uint16_t* bins = reinterpret_cast<uint16_t*>(smem_raw + Ly.bins);
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem_raw + Ly.hc);
  unsigned long long* cand = reinterpret_cast<unsigned long long*>(smem_raw + Ly.hc);
  uint32_t* selb = reinterpret_cast<uint32_t*>(smem_raw + Ly.selb);
  float* qh = reinterpret_cast<float*>(smem_raw + Ly.selb);
  float* qs = reinterpret_cast<float*>(smem_raw + Ly.qs);
  float* mm = reinterpret_cast<float*>(smem_raw + Ly.mm);
  SelState* st = reinterpret_cast<SelState*>(smem_raw + Ly.st);
  uint32_t* bflag = reinterpret_cast<uint32_t*>(smem_raw + Ly.bflag);
  uint16_t* list = reinterpret_cast<uint16_t*>(smem_raw + Ly.list);

  const bool none = top_k <= 0, all = top_k >= N;
  const bool select = !none && !all;
  const int nplo = (r_lo + 15) >> 4;

  // ---- A. loads in flight together: B_k rows first (the latent queries wait only for
  // them), then q, then the first batch of U_k low panels
  LaneTile<T> a[UBA][NPL];
  constexpr int V = Vec16<T>::n;
  constexpr int XB = 8;    // B_k row slices per lane in flight (256 rows of 16 lanes per pass)
  const int ginv_num = (65536 + G - 1) / G;   // (h * ginv_num) >> 16 == h / G for h, G <= 64
  const int LPR = d / V;
  const bool vec = d % V == 0 && LPR > 0 && LPR <= 64 && (LPR & (LPR - 1)) == 0 &&
                   ((size_t)W * sizeof(T)) % 16 == 0;
  const int nrows = nh * r_pad;
  const int RPW = vec ? 64 / LPR : 1, seg = vec ? lane % LPR : 0, rw = vec ? lane / LPR : 0;
  const int rstep = kSelWaves * RPW;
  const float inv_rpad = 1.0f / static_cast<float>(r_pad);
  // head of a flattened (head, latent row) index without an integer division:
  // (row + 0.5) / r_pad is never within float rounding of an integer here
  auto head_of = [&](int row) { return static_cast<int>((static_cast<float>(row) + 0.5f) * inv_rpad); };
  Vec16<T> x[XB];
  auto load_rows = [&](int r0) {
#pragma unroll
    for (int u = 0; u < XB; ++u) {
      const int row = min(r0 + u * rstep, nrows - 1);   // clamped: loads stay unconditional
      const int hl = head_of(row), i = row - hl * r_pad;
      x[u].load(Bk + ((size_t)b * r_pad + i) * W + (size_t)(((h0 + hl) * ginv_num) >> 16) * d + seg * V);
    }
  };
  if (vec) load_rows(wave * RPW + rw);
  constexpr int QPT = (kMaxHg * 256 + kSelThreads - 1) / kSelThreads;   // q values per thread
  float qv[QPT];
  const int nq = nh * d;
#pragma unroll
  for (int u = 0; u < QPT; ++u) qv[u] = q[((size_t)b * Hq + h0) * d + min(tid + u * kSelThreads, nq - 1)];
  if (UB > 0 && select) {
#pragma unroll
    for (int u = 0; u < UBA; ++u) {
      const int blk = min(wave + u * kSelWaves, nblk - 1);   // clamped: loads stay unconditional
      a[u][0].load(Uk + tile_base(b, 0, blk, NP, nblk), lane);
      if (NPL > 1) a[u][NPL - 1].load(Uk + tile_base(b, NPL - 1, blk, NP, nblk), lane);
    }
  }
#pragma unroll
  for (int u = 0; u < QPT; ++u)
    if (tid + u * kSelThreads < nq) qh[tid + u * kSelThreads] = qv[u];
  for (int i = tid; i < nh * 256; i += kSelThreads) hist[i] = 0;
  for (int i = tid; i < nblk; i += kSelThreads) bflag[i] = 0;
  if (tid < nh) {
    st[tid].mode = none ? kNone : (all ? kAll : kWholeBin);
    st[tid].ncand = 0;
    st[tid].nlist = 0;
  }
  __syncthreads();
  // latent queries q~[h][i] = B_k[i, g*d : g*d+d] . q_h
  if (vec) {
    for (int r0 = wave * RPW + rw; r0 - rw < nrows; r0 += XB * rstep) {
      if (r0 != wave * RPW + rw) load_rows(r0);
#pragma unroll
      for (int u = 0; u < XB; ++u) {
        const int row = r0 + u * rstep;
        float part = 0.f;
        if (row < nrows) {
          const float* qv = qh + head_of(row) * d + seg * V;
#pragma unroll
          for (int e = 0; e < V; ++e) part = fmaf(x[u].get(e), qv[e], part);
        }
        part = group_sum(part, LPR);
        if (seg == 0 && row < nrows) qs[row] = part;   // row = hl * r_pad + i
      }
    }
  } else {
    for (int idx = tid; idx < nrows; idx += kSelThreads) {
      const int hl = idx / r_pad, i = idx - hl * r_pad;
      const T* brow = Bk + ((size_t)b * r_pad + i) * W + (size_t)((h0 + hl) / G) * d;
      const float* qv = qh + hl * d;
      float acc = 0.f;
      for (int j = 0; j < d; ++j) acc = fmaf(to_f32(brow[j]), qv[j], acc);
      qs[hl * r_pad + i] = acc;
    }
  }
  __syncthreads();

  if (select) {
    // ---- B. score bounds; scores -> 16-bit bins; coarse histogram
    if (tid < nh) {
      float n2 = 0.f;
      for (int i = 0; i < r_lo; ++i) n2 = fmaf(qs[tid * r_pad + i], qs[tid * r_pad + i], n2);
      const float M = sqrtf(n2) * rn[(size_t)b * NP + nplo - 1] * 1.0001f + 1e-30f;
      const float mul = (M < 3.0e38f && M > 1e-30f) ? 32767.0f / M : 0.f;
      mm[2 * tid] = M * mul;
      mm[2 * tid + 1] = mul;
    }
    __syncthreads();
    const float Mmulh = l16 < nh ? mm[2 * l16] : 0.f, mulh = l16 < nh ? mm[2 * l16 + 1] : 0.f;
    auto put = [&](int blk, int t, float sv) {
      const int n = blk * kBlockTok + 16 * (t >> 2) + 4 * lg + (t & 3);
      if (n < N) {
        const uint32_t bn = score_bin(sv, Mmulh, mulh);
        bins[(size_t)l16 * N_pad + n] = static_cast<uint16_t>(bn);
        atomicAdd(&hist[l16 * 256 + (bn >> 8)], 1u);
      }
    };
    if constexpr (UB > 0) {
      const QOp<T> q0 = low_qop<T>(qs, r_pad, nh, r_lo, 0, lane);
      const QOp<T> q1 = low_qop<T>(qs, r_pad, nh, r_lo, NPL - 1, lane);
      for (int base = wave; base < nblk; base += kSelWaves * UB) {
        if (base != wave) {
#pragma unroll
          for (int u = 0; u < UB; ++u) {
            const int blk = min(base + u * kSelWaves, nblk - 1);
            a[u][0].load(Uk + tile_base(b, 0, blk, NP, nblk), lane);
            if (NPL > 1) a[u][NPL - 1].load(Uk + tile_base(b, NPL - 1, blk, NP, nblk), lane);
          }
        }
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          const int blk = base + u * kSelWaves;
          if (blk < nblk) {
            v4f s0 = v4f{0, 0, 0, 0}, s1 = v4f{0, 0, 0, 0};
            s0 = score_mma(a[u][0], 0, q0, s0);
            s1 = score_mma(a[u][0], 1, q0, s1);
            if (NPL > 1 && nplo > 1) {
              s0 = score_mma(a[u][NPL - 1], 0, q1, s0);
              s1 = score_mma(a[u][NPL - 1], 1, q1, s1);
            }
            if (l16 < nh) {
#pragma unroll
              for (int t = 0; t < 8; ++t) put(blk, t, t < 4 ? s0[t & 3] : s1[t & 3]);
            }
          }
        }
      }
    } else {
      for (int blk = wave; blk < nblk; blk += kSelWaves) {
        v4f s0, s1;
        score_block(Uk, b, blk, NP, nblk, r_lo, qs, r_pad, nh, lane, s0, s1);
        if (l16 < nh) {
#pragma unroll
          for (int t = 0; t < 8; ++t) put(blk, t, t < 4 ? s0[t & 3] : s1[t & 3]);
        }
      }
    }
    __syncthreads();

    // ---- C. coarse boundary digit, fine histogram inside it, fine boundary bin
    if (wave < nh) {
      int dg; uint32_t above, inb;
      if (digit_search(hist + wave * 256, static_cast<uint32_t>(top_k), lane, &dg, &above, &inb)) {
        st[wave].bstar = dg;
        st[wave].need = top_k - static_cast<int>(above);
      }
    }
    __syncthreads();
    for (int i = tid; i < nh * 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    {
      const int n8 = N_pad / 8;   // 8 bins per 16-byte read
      for (int idx = tid; idx < nh * n8; idx += kSelThreads) {
        const int hl = idx / n8, j = idx - hl * n8;
        const uint32_t c = static_cast<uint32_t>(st[hl].bstar);
        const uint4 x8 = *reinterpret_cast<const uint4*>(bins + (size_t)hl * N_pad + 8 * j);
        const uint32_t w8[4] = {x8.x, x8.y, x8.z, x8.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int n = 8 * j + e;
          const uint32_t bn = (e & 1) ? (w8[e >> 1] >> 16) : (w8[e >> 1] & 0xffffu);
          if (n < N && (bn >> 8) == c) {
            atomicAdd(&hist[hl * 256 + (bn & 255u)], 1u);
            const int pos = atomicAdd(&st[hl].nlist, 1);
            if (pos < kSelList) list[hl * kSelList + pos] = static_cast<uint16_t>(n);
          }
        }
      }
    }
    __syncthreads();
    if (wave < nh) {
      int dg; uint32_t above, inb;
      if (digit_search(hist + wave * 256, static_cast<uint32_t>(st[wave].need), lane, &dg, &above, &inb)) {
        const int need = st[wave].need - static_cast<int>(above);
        st[wave].bstar = (st[wave].bstar << 8) | dg;
        st[wave].need = need;
        st[wave].cnt = static_cast<int>(inb);
        st[wave].mode = need == static_cast<int>(inb) ? kWholeBin
                        : (inb <= static_cast<uint32_t>(kSelCap) ? kRank : kRadix);
      }
    }
    __syncthreads();

    // ---- D. exact resolution inside a boundary bin that is only partly taken
    bool any_rank = false, any_radix = false;
    for (int hl = 0; hl < nh; ++hl) {
      any_rank |= st[hl].mode == kRank;
      any_radix |= st[hl].mode == kRadix;
    }
    if (any_rank || any_radix) {
      for (int i = tid; i < nh * nblk; i += kSelThreads) selb[i] = 0;
      for (int hl = 0; hl < nh; ++hl) {
        if (st[hl].mode < kRank) continue;
        const uint16_t bs = static_cast<uint16_t>(st[hl].bstar);
        const uint16_t* bh = bins + (size_t)hl * N_pad;
        if (st[hl].nlist <= kSelList) {
          for (int i = tid; i < st[hl].nlist; i += kSelThreads) {
            const int n = list[hl * kSelList + i];
            if (bh[n] == bs) bflag[n / kBlockTok] = 1u;
          }
        } else {
          for (int n = tid; n < N; n += kSelThreads)
            if (bh[n] == bs) bflag[n / kBlockTok] = 1u;
        }
      }
      __syncthreads();
    }
    if (any_rank) {
      for (int blk = wave; blk < nblk; blk += kSelWaves) {
        if (!bflag[blk]) continue;
        v4f s0, s1;
        score_block(Uk, b, blk, NP, nblk, r_lo, qs, r_pad, nh, lane, s0, s1);
        if (l16 < nh && st[l16].mode == kRank) {
          const uint16_t bs = static_cast<uint16_t>(st[l16].bstar);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int n = blk * kBlockTok + 16 * (t >> 2) + 4 * lg + (t & 3);
            if (n < N && bins[(size_t)l16 * N_pad + n] == bs) {
              const unsigned long long comp =
                  (static_cast<unsigned long long>(score_key(t < 4 ? s0[t & 3] : s1[t & 3])) << 32) |
                  static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(n));
              const int pos = atomicAdd(&st[l16].ncand, 1);
              if (pos < kSelCap) cand[l16 * kSelCap + pos] = comp;
            }
          }
        }
      }
      __syncthreads();
      for (int hl = 0; hl < nh; ++hl) {
        if (st[hl].mode != kRank) continue;
        const int C = min(st[hl].ncand, kSelCap);
        const unsigned long long* ch = cand + hl * kSelCap;
        for (int c = tid; c < C; c += kSelThreads) {
          const unsigned long long me = ch[c];
          int rank = 0;
          for (int o = 0; o < C; ++o) rank += ch[o] > me ? 1 : 0;
          if (rank < st[hl].need) {
            const uint32_t n = 0xFFFFFFFFu - static_cast<uint32_t>(me & 0xFFFFFFFFull);
            atomicOr(&selb[hl * nblk + n / kBlockTok], 1u << (n % kBlockTok));
          }
        }
      }
      __syncthreads();
    }
    if (any_radix) {
      // Exact radix select over the 32-bit keys of the boundary-bin tokens, keys recomputed
      // per pass; then the boundary tokens are taken in index order (ties to lower index).
      for (int hl = 0; hl < nh; ++hl) {
        if (st[hl].mode != kRadix) continue;
        const uint16_t bs = static_cast<uint16_t>(st[hl].bstar);
        uint32_t prefix = 0;
        uint32_t need = static_cast<uint32_t>(st[hl].need);
        for (int pass = 0; pass < 4; ++pass) {
          const int shift = 24 - 8 * pass;
          const uint32_t pmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
          for (int i = tid; i < 256; i += kSelThreads) hist[hl * 256 + i] = 0;
          __syncthreads();
          for (int blk = wave; blk < nblk; blk += kSelWaves) {
            if (!bflag[blk]) continue;
            v4f s0, s1;
            score_block(Uk, b, blk, NP, nblk, r_lo, qs, r_pad, nh, lane, s0, s1);
            if (l16 == hl) {
#pragma unroll
              for (int t = 0; t < 8; ++t) {
                const int n = blk * kBlockTok + 16 * (t >> 2) + 4 * lg + (t & 3);
                if (n < N && bins[(size_t)hl * N_pad + n] == bs) {
                  const uint32_t key = score_key(t < 4 ? s0[t & 3] : s1[t & 3]);
                  if ((key & pmask) == prefix) atomicAdd(&hist[hl * 256 + ((key >> shift) & 255u)], 1u);
                }
              }
            }
          }
          __syncthreads();
          if (wave == 0) {
            int dg; uint32_t above, inb;
            if (digit_search(hist + hl * 256, need, lane, &dg, &above, &inb)) {
              st[hl].tau = prefix | (static_cast<uint32_t>(dg) << shift);
              st[hl].need = static_cast<int>(need - above);
            }
          }
          __syncthreads();
          prefix = st[hl].tau;
          need = static_cast<uint32_t>(st[hl].need);
        }
        if (wave == 0) {
          const uint32_t tau = prefix;
          uint32_t left = need;
          for (int blk = 0; blk < nblk; ++blk) {
            if (!bflag[blk]) continue;
            v4f s0, s1;
            score_block(Uk, b, blk, NP, nblk, r_lo, qs, r_pad, nh, lane, s0, s1);
            uint32_t gtm = 0, eqm = 0;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const int hf = t >> 2, tt = t & 3;
              const int n = blk * kBlockTok + 16 * hf + 4 * lg + tt;
              bool gt = false, eq = false;
              if (l16 == hl && n < N && bins[(size_t)hl * N_pad + n] == bs) {
                const uint32_t key = score_key(t < 4 ? s0[tt] : s1[tt]);
                gt = key > tau;
                eq = key == tau;
              }
              const uint64_t bg = __ballot(gt), be = __ballot(eq);
#pragma unroll
              for (int g4 = 0; g4 < 4; ++g4) {
                const int bit = 16 * hf + 4 * g4 + tt;
                if ((bg >> (g4 * 16 + hl)) & 1ull) gtm |= 1u << bit;
                if ((be >> (g4 * 16 + hl)) & 1ull) eqm |= 1u << bit;
              }
            }
            uint32_t take = gtm;
            while (eqm && left) {
              const uint32_t low = eqm & (~eqm + 1u);
              take |= low;
              eqm ^= low;
              --left;
            }
            if (lane == 0) selb[hl * nblk + blk] |= take;
          }
        }
        __syncthreads();
      }
    }
  }

  // ---- E. selection bits per (head, 32-token block)
  if (sel_out == nullptr) {
    for (int idx = tid; idx < nh * nblk; idx += kSelThreads) {
      const int hl = idx / nblk, blk = idx - hl * nblk;
      const int mode = st[hl].mode;
      uint32_t word = 0;
      const int nvalid = min(kBlockTok, N - blk * kBlockTok);
      const uint32_t valid = nvalid >= 32 ? 0xFFFFFFFFu : ((1u << nvalid) - 1u);
      if (mode == kAll) {
        word = valid;
      } else if (mode != kNone) {
        const uint32_t bs = static_cast<uint32_t>(st[hl].bstar);
        const uint4* bp = reinterpret_cast<const uint4*>(bins + (size_t)hl * N_pad + blk * kBlockTok);
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const uint4 x = bp[v4];
          const uint32_t w8[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = w8[e] & 0xffffu, hi = w8[e] >> 16;
            const int bit = 8 * v4 + 2 * e;
            gt |= (lo > bs ? 1u : 0u) << bit;
            gt |= (hi > bs ? 1u : 0u) << (bit + 1);
            eq |= (lo == bs ? 1u : 0u) << bit;
            eq |= (hi == bs ? 1u : 0u) << (bit + 1);
          }
        }
        word = (mode == kWholeBin) ? (gt | eq) : (gt | (eq & selb[hl * nblk + blk]));
        word &= valid;
      }
      mask[((size_t)b * nblk + blk) * Hq_pad + h0 + hl] = word;
    }
  } else {
    // ascending ids as well: one wavefront per head walks its tokens in order
    for (int hl = wave; hl < nh; hl += kSelWaves) {
      const int h = h0 + hl;
      const int mode = st[hl].mode;
      const uint32_t bs = mode >= kWholeBin ? static_cast<uint32_t>(st[hl].bstar) : 0u;
      uint32_t run_sel = 0;
      const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      for (int c0 = 0; c0 < N_pad; c0 += 64) {
        const int n = c0 + lane;
        const bool valid = n < N;
        bool sel;
        if (mode == kNone) {
          sel = false;
        } else if (mode == kAll) {
          sel = valid;
        } else {
          const uint32_t bn = valid ? bins[(size_t)hl * N_pad + n] : 0u;
          if (mode == kWholeBin)
            sel = valid && bn >= bs;
          else
            sel = valid && (bn > bs || (bn == bs && ((selb[hl * nblk + n / kBlockTok] >> (n % kBlockTok)) & 1u)));
        }
        const uint64_t sb = __ballot(sel);
        const int t0 = c0 / kBlockTok;
        if (lane == 0) {
          mask[((size_t)b * nblk + t0) * Hq_pad + h] = static_cast<uint32_t>(sb);
          if (t0 + 1 < nblk) mask[((size_t)b * nblk + t0 + 1) * Hq_pad + h] = static_cast<uint32_t>(sb >> 32);
        }
        const uint32_t pos = run_sel + static_cast<uint32_t>(__popcll(sb & lt_mask));
        if (sel) sel_out[((size_t)b * Hq + h) * top_k + pos] = n;
        run_sel += static_cast<uint32_t>(__popcll(sb));
      }
    }
  }
  // latent queries for the flash-decode kernel (stored last: stores share the load counter)
  for (int i = tid; i < nh * r_pad; i += kSelThreads)
    qt[((size_t)b * Hq_pad + h0) * r_pad + i] = qs[i];
}

// ---------------------------------------------------------------- row-norm bound
// rn[b][p] = max_n |U_k[n, :16(p+1)]|_2 (slightly rounded up): bounds the low-rank score.
template <class T>
__global__ __launch_bounds__(256) void k_rownorm(const T* __restrict__ Uk, float* __restrict__ rn,
                                                 int N, int NP, int nblk) {
  __shared__ uint32_t mx[16];
  const int b = blockIdx.x;
  if (threadIdx.x < 16) mx[threadIdx.x] = 0u;
  __syncthreads();
  float best[16];
  for (int p = 0; p < NP; ++p) best[p] = 0.f;
  for (int n = threadIdx.x; n < N; n += blockDim.x) {
    const int t = n / kBlockTok, nn = n % kBlockTok, half = nn >> 4;
    float cum = 0.f;
    for (int p = 0; p < NP; ++p) {
      const T* base = Uk + tile_base(b, p, t, NP, nblk);
      for (int cc = 0; cc < 16; ++cc) {
        const int lane = (cc >> 2) * 16 + (nn & 15);
        const float v = to_f32(base[tile_elem(lane, half, cc & 3)]);
        cum = fmaf(v, v, cum);
      }
      best[p] = fmaxf(best[p], cum);
    }
  }
  for (int p = 0; p < NP; ++p) atomicMax(&mx[p], __float_as_uint(best[p]));
  __syncthreads();
  if (threadIdx.x < NP) rn[(size_t)b * NP + threadIdx.x] = sqrtf(__uint_as_float(mx[threadIdx.x])) * 1.0001f;
}

// ---------------------------------------------------------------- launchers
int select_heads_per_group(const Dims& dm) {
  // LDS budget ~150 KB, and enough workgroups to cover the GPU's 256 CUs
  int hg_lds = kMaxHg;
  while (hg_lds > 1 && sel_layout(hg_lds, dm.N_pad, dm.nblk, dm.r_pad, dm.d).total > 150 * 1024) --hg_lds;
  int groups = (dm.Hq + hg_lds - 1) / hg_lds;
  const int want = dm.B > 0 ? (256 + dm.B - 1) / dm.B : 1;
  groups = std::max(groups, std::min(dm.Hq, want));
  return (dm.Hq + groups - 1) / groups;
}

size_t select_lds_bytes(const Dims& dm, int Hg) {
  return sel_layout(Hg, dm.N_pad, dm.nblk, dm.r_pad, dm.d).total;
}

template <class T>
static hipError_t launch_select_t(const ap_cache* c, const float* q, int r_lo, int top_k,
                                  int32_t* sel_out, hipStream_t st, const KernelEvents& ev) {
  const Dims& dm = c->dm;
  const int Hg = select_heads_per_group(dm);
  const int HG = (dm.Hq + Hg - 1) / Hg;
  const size_t lds = select_lds_bytes(dm, Hg);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const int nplo = (r_lo + 15) / 16;
  // one low panel: 12 blocks per wavefront in flight when that covers the sequence
  const int which = nplo == 1 ? (dm.nblk <= 12 * kSelWaves ? 0 : 1) : (nplo == 2 ? 2 : 3);
  const void* fns[4] = {reinterpret_cast<const void*>(&k_select<T, 12>),
                        reinterpret_cast<const void*>(&k_select<T, 16>),
                        reinterpret_cast<const void*>(&k_select<T, 8>),
                        reinterpret_cast<const void*>(&k_select<T, 0>)};
  static bool attr_set[4] = {false, false, false, false};
  if (!attr_set[which]) {
    hipError_t e = hipFuncSetAttribute(fns[which], hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set[which] = true;
  }
  const int grid = ((dm.B + 7) / 8) * 8 * HG;
#define AP_SELECT_ARGS static_cast<const T*>(c->Uk), static_cast<const T*>(c->Bk), c->rn, q, c->qt, \
      c->mask, sel_out, dm.B, dm.N, dm.N_pad, dm.nblk, dm.NP, dm.r_pad, dm.W, dm.d, dm.G, dm.Hq,  \
      dm.Hq_pad, Hg, HG, r_lo, top_k
#define AP_SELECT_LAUNCH(UBV) \
  hipExtLaunchKernelGGL((k_select<T, UBV>), dim3(grid), dim3(kSelThreads), lds, st, ev.start, ev.stop, 0, AP_SELECT_ARGS)
  switch (which) {
    case 0: AP_SELECT_LAUNCH(12); break;
    case 1: AP_SELECT_LAUNCH(16); break;
    case 2: AP_SELECT_LAUNCH(8); break;
    default: AP_SELECT_LAUNCH(0); break;
  }
#undef AP_SELECT_LAUNCH
#undef AP_SELECT_ARGS
  return hipGetLastError();
}

hipError_t launch_select(const ap_cache* c, const float* q, int r_lo, int top_k, int32_t* sel_out,
                         hipStream_t st, const KernelEvents& ev) {
  if (c->dm.storage == AP_BF16) return launch_select_t<bf16_t>(c, q, r_lo, top_k, sel_out, st, ev);
  return launch_select_t<float>(c, q, r_lo, top_k, sel_out, st, ev);
}

hipError_t launch_rownorm(const ap_cache* c, hipStream_t st) {
  const Dims& dm = c->dm;
  if (dm.storage == AP_BF16)
    hipLaunchKernelGGL(k_rownorm<bf16_t>, dim3(dm.B), dim3(256), 0, st,
                       static_cast<const bf16_t*>(c->Uk), c->rn, dm.N, dm.NP, dm.nblk);
  else
    hipLaunchKernelGGL(k_rownorm<float>, dim3(dm.B), dim3(256), 0, st,
                       static_cast<const float*>(c->Uk), c->rn, dm.N, dm.NP, dm.nblk);
  return hipGetLastError();
}

}  // namespace ap

// Decode step over the compressed visual cache (gfx950).
//
// Method: AttentionPack summaries (gist.science es/fr/de), [fr §2.B "Stratégie"]:
// per token and step, the most important tokens are decompressed at the full rank
// and the others at a reduced rank; [es §4 "Análisis de Sensibilidad"]: 25% at full
// rank.  Importance is the current-step low-rank logit per query head.  Nothing is
// ever decompressed explicitly: scores and values are accumulated in factor space,
//   s[n] = scale * U_k[n, :r(n)] . q~[:r(n)],   z = sum_n p[n] U_v[n, :r(n)],
//   out  = z B_v (per head slice) / l,
// which is the same number as decompress-then-attend.
//
// Three kernels per call:
//   k_select  (sequence, head group): latent queries q~ = B_k,g q_h, low-rank scores
//             for every token by MFMA, exact top-k by MSB-first radix select over
//             order-preserving keys held in LDS, selection bitmask per 32-token block.
//   k_attn    (sequence, N-split): mixed-rank rescoring, online softmax and latent V
//             accumulation on MFMA tiles, cross-wavefront merge in LDS, one partial
//             (m, l, z[Hq][r]) per split.
//   k_combine (sequence, query head): dense text tokens, log-sum-exp merge of the
//             splits, projection of z through B_v, output.
#include <type_traits>

#include "ap_internal.h"
#include "device_common.h"

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
    for (int t = 0; t < 4; ++t) v[t] = static_cast<short>(f32_to_bf16(p[t]));
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

// ================================================================ k_select
// LDS layout: keys[Hg][N_pad] u32 | hist[Hg][256] u32 | qs[Hg][r_pad] f32 | st[Hg][4] i32
// st: 0 prefix of the k-th key, 1 keys still to take at the prefix, 2 keys above prefix.
template <class T>
__global__ __launch_bounds__(256) void k_select(
    const T* __restrict__ Uk, const T* __restrict__ Bk, const float* __restrict__ q,
    float* __restrict__ qt, uint32_t* __restrict__ mask, int32_t* __restrict__ sel_out,
    int B, int N, int N_pad, int nblk, int NP, int r_pad, int W, int d, int G, int Hq,
    int Hq_pad, int Hg, int HG, int r_lo, int top_k) {
  extern __shared__ __align__(16) uint32_t smem_u[];
  // Sequences are spread so that all head groups of one sequence share blockIdx % 8,
  // i.e. the same XCD and L2, which then serves the repeated reads of U_k's low panels.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int b = (slot / HG) * 8 + xcd;
  const int hg = slot % HG;
  if (b >= B) return;
  const int h0 = hg * Hg;
  const int nh = min(Hg, Hq - h0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;

  uint32_t* keys = smem_u;
  uint32_t* hist = keys + (size_t)Hg * N_pad;
  float* qs = reinterpret_cast<float*>(hist + Hg * 256);
  int* st = reinterpret_cast<int*>(qs + Hg * r_pad);

  // 1. latent queries q~[h][i] = sum_j B_k[i][g*d + j] q_h[j]
  for (int idx = tid; idx < nh * r_pad; idx += 256) {
    const int hl = idx / r_pad, i = idx - hl * r_pad;
    const int h = h0 + hl, g = h / G;
    const T* brow = Bk + ((size_t)b * r_pad + i) * W + (size_t)g * d;
    const float* qh = q + ((size_t)b * Hq + h) * d;
    float acc = 0.f;
    for (int j = 0; j < d; ++j) acc = fmaf(to_f32(brow[j]), qh[j], acc);
    qs[hl * r_pad + i] = acc;
    qt[((size_t)b * Hq_pad + h) * r_pad + i] = acc;
  }
  __syncthreads();

  const bool none = top_k <= 0;
  const bool all = top_k >= N;

  if (!none && !all) {
    // 2. low-rank scores of every token for the nh heads (columns 0..r_lo-1)
    const int nplo = (r_lo + 15) >> 4;
    const int hq = l16 < nh ? l16 : -1;
    for (int blk = wave; blk < nblk; blk += 4) {
      v4f acc[2] = {v4f{0, 0, 0, 0}, v4f{0, 0, 0, 0}};
      for (int p = 0; p < nplo; ++p) {
        LaneTile<T> a;
        a.load(Uk + tile_base(b, p, blk, NP, nblk), lane);
        float v[4];
        const int c0 = 16 * p + 4 * lg;
        for (int e = 0; e < 4; ++e) v[e] = (hq >= 0 && c0 + e < r_lo) ? qs[hq * r_pad + c0 + e] : 0.f;
        QOp<T> qo;
        qo.set(v);
        acc[0] = score_mma(a, 0, qo, acc[0]);
        acc[1] = score_mma(a, 1, qo, acc[1]);
      }
      if (hq >= 0) {
        for (int hf = 0; hf < 2; ++hf)
          for (int t = 0; t < 4; ++t) {
            const int n = blk * kBlockTok + 16 * hf + 4 * lg + t;
            if (n < N) keys[(size_t)hq * N_pad + n] = score_key(acc[hf][t]);
          }
      }
    }
    if (tid < nh) {
      st[tid * 4 + 0] = 0;
      st[tid * 4 + 1] = top_k;
      st[tid * 4 + 2] = 0;
    }
    __syncthreads();

    // 3. MSB-first radix select, 8 bits per pass, all nh heads at once
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const uint32_t pmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
      for (int i = tid; i < nh * 256; i += 256) hist[i] = 0;
      __syncthreads();
      for (int hl = 0; hl < nh; ++hl) {
        const uint32_t pre = static_cast<uint32_t>(st[hl * 4 + 0]);
        const uint32_t* kh = keys + (size_t)hl * N_pad;
        for (int n = tid; n < N; n += 256) {
          const uint32_t key = kh[n];
          if ((key & pmask) == pre) atomicAdd(&hist[hl * 256 + ((key >> shift) & 255u)], 1u);
        }
      }
      __syncthreads();
      for (int hl = wave; hl < nh; hl += 4) {
        // lane covers digits 255-4*lane .. 252-4*lane (descending)
        uint32_t c[4];
        uint32_t tot = 0;
        for (int e = 0; e < 4; ++e) {
          c[e] = hist[hl * 256 + 255 - (4 * lane + e)];
          tot += c[e];
        }
        uint32_t incl = tot;
        for (int off = 1; off < 64; off <<= 1) {
          uint32_t y = __shfl_up(incl, off, 64);
          if (lane >= off) incl += y;
        }
        const uint32_t excl = incl - tot;
        const uint32_t need = static_cast<uint32_t>(st[hl * 4 + 1]);
        if (excl < need && incl >= need) {
          uint32_t run = excl;
          int dig = 0;
          for (int e = 0; e < 4; ++e) {
            if (run + c[e] >= need) {
              dig = 255 - (4 * lane + e);
              break;
            }
            run += c[e];
          }
          st[hl * 4 + 0] = static_cast<int>(static_cast<uint32_t>(st[hl * 4 + 0]) | (static_cast<uint32_t>(dig) << shift));
          st[hl * 4 + 1] = static_cast<int>(need - run);
          st[hl * 4 + 2] += static_cast<int>(run);
        }
      }
      __syncthreads();
    }
  }

  // 4. selection bits per 32-token block (and optional ascending ids), one wave per head.
  //    Keys equal to the k-th key are taken in token order until k are chosen.
  for (int hl = wave; hl < nh; hl += 4) {
    const int h = h0 + hl;
    uint32_t tau = 0, need = 0;
    if (!none && !all) {
      tau = static_cast<uint32_t>(st[hl * 4 + 0]);
      need = static_cast<uint32_t>(st[hl * 4 + 1]);
    }
    uint32_t run_eq = 0, run_sel = 0;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < N_pad; c0 += 64) {
      const int n = c0 + lane;
      const bool valid = n < N;
      bool sel;
      if (none) {
        sel = false;
      } else if (all) {
        sel = valid;
      } else {
        const uint32_t key = valid ? keys[(size_t)hl * N_pad + n] : 0u;
        const bool gt = valid && key > tau;
        const bool eq = valid && key == tau;
        const uint64_t eqb = __ballot(eq);
        const uint32_t before = run_eq + static_cast<uint32_t>(__popcll(eqb & lt_mask));
        sel = gt || (eq && before < need);
        run_eq += static_cast<uint32_t>(__popcll(eqb));
      }
      const uint64_t sb = __ballot(sel);
      const int t0 = c0 / kBlockTok;
      if (lane == 0) {
        mask[((size_t)b * nblk + t0) * Hq_pad + h] = static_cast<uint32_t>(sb);
        if (t0 + 1 < nblk) mask[((size_t)b * nblk + t0 + 1) * Hq_pad + h] = static_cast<uint32_t>(sb >> 32);
      }
      if (sel_out != nullptr) {
        const uint32_t pos = run_sel + static_cast<uint32_t>(__popcll(sb & lt_mask));
        if (sel) sel_out[((size_t)b * Hq + h) * top_k + pos] = n;
        run_sel += static_cast<uint32_t>(__popcll(sb));
      }
    }
  }
}

// ================================================================ k_attn
template <class T, int NP, int HT>
__global__ __launch_bounds__(256) void k_attn(
    const T* __restrict__ Uk, const T* __restrict__ Uv, const float* __restrict__ qt,
    const uint32_t* __restrict__ mask, float* __restrict__ part_z, float* __restrict__ part_ml,
    int N, int nblk, int CB, int S, int Hq, int r_lo, float sl2) {
  constexpr int RP = NP * 16, HP = HT * 16, ZS = RP + 1;
  extern __shared__ __align__(16) float smem_f[];
  const int b = blockIdx.x / S, s = blockIdx.x - (blockIdx.x / S) * S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int blk0 = s * CB, blk1 = min(nblk, blk0 + CB);

  // latent-query operands: panel p, head tile ht, this lane's 4 columns 16p+4lg+e
  QOp<T> qop[NP][HT];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = 16 * ht + l16;
      float v[4];
      for (int e = 0; e < 4; ++e)
        v[e] = h < Hq ? qt[((size_t)b * HP + h) * RP + 16 * p + 4 * lg + e] : 0.f;
      qop[p][ht].set(v);
    }

  v4f Z[NP][HT];
  float m[HT], lsum[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    m[ht] = kNegBig;
    lsum[ht] = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) Z[p][ht] = v4f{0, 0, 0, 0};
  }

  for (int blk = blk0 + wave; blk < blk1; blk += 4) {
    LaneTile<T> uk[NP], uv[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      uk[p].load(Uk + tile_base(b, p, blk, NP, nblk), lane);
      uv[p].load(Uv + tile_base(b, p, blk, NP, nblk), lane);
    }
    uint32_t mw[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int h = 16 * ht + l16;
      mw[ht] = h < Hq ? mask[((size_t)b * nblk + blk) * HP + h] : 0u;
    }

    float sc[2][HT][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        v4f slo = v4f{0, 0, 0, 0}, shi = v4f{0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          if (16 * p + 16 <= r_lo) {
            slo = score_mma(uk[p], hf, qop[p][ht], slo);
          } else if (16 * p >= r_lo) {
            shi = score_mma(uk[p], hf, qop[p][ht], shi);
          } else {
            const int cl = 16 * p + 4 * lg;
            slo = score_mma(uk[p], hf, qop[p][ht].masked(cl, r_lo, true), slo);
            shi = score_mma(uk[p], hf, qop[p][ht].masked(cl, r_lo, false), shi);
          }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int pos = 16 * hf + 4 * lg + t;
          const bool bit = (mw[ht] >> pos) & 1u;
          const float v = (slo[t] + (bit ? shi[t] : 0.f)) * sl2;
          sc[hf][ht][t] = (blk * kBlockTok + pos < N) ? v : -INFINITY;
        }
      }

    POp<T> pa[2][HT], ph[2][HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float bm = -INFINITY;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int t = 0; t < 4; ++t) bm = fmaxf(bm, sc[hf][ht][t]);
      bm = wave_max_xor(bm, 16);
      bm = wave_max_xor(bm, 32);
      const float mn = fmaxf(m[ht], bm);
      const float alpha = exp2f(m[ht] - mn);
      m[ht] = mn;
      lsum[ht] *= alpha;
#pragma unroll
      for (int p = 0; p < NP; ++p) Z[p][ht] *= alpha;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float pv[4], phv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float e = exp2f(sc[hf][ht][t] - mn);
          lsum[ht] += e;
          pv[t] = e;
          phv[t] = ((mw[ht] >> (16 * hf + 4 * lg + t)) & 1u) ? e : 0.f;
        }
        pa[hf][ht].set(pv);
        ph[hf][ht].set(phv);
      }
    }

#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          if (16 * p + 16 <= r_lo) {
            Z[p][ht] = value_mma(uv[p], hf, true, pa[hf][ht], Z[p][ht]);
          } else if (16 * p >= r_lo) {
            Z[p][ht] = value_mma(uv[p], hf, true, ph[hf][ht], Z[p][ht]);
          } else {
            const bool lo_row = 16 * p + l16 < r_lo;  // this lane's A row is latent column 16p+l16
            Z[p][ht] = value_mma(uv[p], hf, lo_row, pa[hf][ht], Z[p][ht]);
            Z[p][ht] = value_mma(uv[p], hf, !lo_row, ph[hf][ht], Z[p][ht]);
          }
        }
  }

  // per-head sums over the four lane groups
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    lsum[ht] += __shfl_xor(lsum[ht], 16, 64);
    lsum[ht] += __shfl_xor(lsum[ht], 32, 64);
  }

  // cross-wavefront merge
  float* zb = smem_f;                 // [4][HP][ZS]
  float* mb = zb + 4 * HP * ZS;       // [4][HP]
  float* lb = mb + 4 * HP;            // [4][HP]
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        zb[(wave * HP + 16 * ht + l16) * ZS + 16 * p + 4 * lg + t] = Z[p][ht][t];
  if (lg == 0) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      mb[wave * HP + 16 * ht + l16] = m[ht];
      lb[wave * HP + 16 * ht + l16] = lsum[ht];
    }
  }
  __syncthreads();
  const size_t pbase = ((size_t)b * S + s) * HP;
  for (int idx = tid; idx < HP * RP; idx += 256) {
    const int h = idx / RP, i = idx - h * RP;
    float M = mb[h];
    for (int w = 1; w < 4; ++w) M = fmaxf(M, mb[w * HP + h]);
    float z = 0.f;
    for (int w = 0; w < 4; ++w) z += exp2f(mb[w * HP + h] - M) * zb[(w * HP + h) * ZS + i];
    part_z[(pbase + h) * RP + i] = z;
  }
  for (int h = tid; h < HP; h += 256) {
    float M = mb[h];
    for (int w = 1; w < 4; ++w) M = fmaxf(M, mb[w * HP + h]);
    float L = 0.f;
    for (int w = 0; w < 4; ++w) L += exp2f(mb[w * HP + h] - M) * lb[w * HP + h];
    part_ml[(pbase + h) * 2 + 0] = M;
    part_ml[(pbase + h) * 2 + 1] = L;
  }
}

// ================================================================ k_combine
__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  // 128 threads = 2 wavefronts
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(v, off, 64);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return is_max ? fmaxf(red[0], red[1]) : red[0] + red[1];
}

template <class T>
__global__ __launch_bounds__(128) void k_combine(
    const float* __restrict__ part_z, const float* __restrict__ part_ml, const T* __restrict__ Bv,
    const float* __restrict__ q, float* __restrict__ out, const T* __restrict__ text_k,
    const T* __restrict__ text_v, int S, int Hq, int HP, int RP, int W, int d, int G, int Tn,
    float sl2) {
  extern __shared__ __align__(16) float smem_c[];
  float* qh = smem_c;          // [d]
  float* zz = qh + d;          // [RP]
  float* pt = zz + RP;         // [128]
  float* red = pt + 128;       // [2]
  const int b = blockIdx.x / Hq, h = blockIdx.x - (blockIdx.x / Hq) * Hq;
  const int g = h / G;
  const int tid = threadIdx.x;
  const size_t pb = (size_t)b * S * HP;

  for (int j = tid; j < d; j += 128) qh[j] = q[((size_t)b * Hq + h) * d + j];

  // visual splits: running maxima
  float mv = kNegBig;
  for (int s = tid; s < S; s += 128) mv = fmaxf(mv, part_ml[(pb + (size_t)s * HP + h) * 2]);
  mv = block_reduce(mv, red, true);

  // dense text tokens, online softmax over chunks of 128
  constexpr int kMaxJ = 2;  // d <= 256
  float acc[kMaxJ] = {0.f, 0.f};
  float mt = kNegBig, lt = 0.f;
  for (int t0 = 0; t0 < Tn; t0 += 128) {
    const int t = t0 + tid;
    float sv = -INFINITY;
    if (t < Tn) {
      const T* row = text_k + ((size_t)b * Tn + t) * W + (size_t)g * d;
      float dot = 0.f;
      for (int j = 0; j < d; ++j) dot = fmaf(to_f32(row[j]), qh[j], dot);
      sv = dot * sl2;
    }
    const float cm = block_reduce(sv, red, true);
    const float mn = fmaxf(mt, cm);
    const float alpha = exp2f(mt - mn);
    const float pv = t < Tn ? exp2f(sv - mn) : 0.f;
    pt[tid] = pv;
    const float ls = block_reduce(pv, red, false);  // also orders pt writes before reads
    lt = lt * alpha + ls;
    mt = mn;
    const int tc = min(128, Tn - t0);
    for (int jj = 0; jj < kMaxJ; ++jj) {
      const int j = tid + 128 * jj;
      if (j < d) {
        float a = acc[jj] * alpha;
        const T* col = text_v + ((size_t)b * Tn + t0) * W + (size_t)g * d + j;
        for (int tt = 0; tt < tc; ++tt) a = fmaf(pt[tt], to_f32(col[(size_t)tt * W]), a);
        acc[jj] = a;
      }
    }
    __syncthreads();
  }

  const float M = fmaxf(mv, mt);
  float L = 0.f;
  for (int s = tid; s < S; s += 128) {
    const float* ml = part_ml + (pb + (size_t)s * HP + h) * 2;
    L += exp2f(ml[0] - M) * ml[1];
  }
  L = block_reduce(L, red, false);
  const float wt = exp2f(mt - M);
  L += wt * lt;

  for (int i = tid; i < RP; i += 128) {
    float z = 0.f;
    for (int s = 0; s < S; ++s)
      z += exp2f(part_ml[(pb + (size_t)s * HP + h) * 2] - M) * part_z[(pb + (size_t)s * HP + h) * RP + i];
    zz[i] = z;
  }
  __syncthreads();
  const float invL = 1.f / L;
  for (int jj = 0; jj < kMaxJ; ++jj) {
    const int j = tid + 128 * jj;
    if (j < d) {
      float o = wt * acc[jj];
      const T* col = Bv + (size_t)b * RP * W + (size_t)g * d + j;
      for (int i = 0; i < RP; ++i) o = fmaf(zz[i], to_f32(col[(size_t)i * W]), o);
      out[((size_t)b * Hq + h) * d + j] = o * invL;
    }
  }
}

// ================================================================ launchers
int select_heads_per_group(const Dims& dm) {
  const size_t per_head = (size_t)dm.N_pad * 4 + 256 * 4 + (size_t)dm.r_pad * 4 + 16;
  int hg = static_cast<int>((64 * 1024) / per_head);
  hg = hg < 1 ? 1 : hg;
  hg = hg > 16 ? 16 : hg;
  hg = hg > dm.Hq ? dm.Hq : hg;
  return hg;
}

size_t select_lds_bytes(const Dims& dm, int Hg) {
  return (size_t)Hg * ((size_t)dm.N_pad * 4 + 256 * 4 + (size_t)dm.r_pad * 4 + 16);
}

template <class T>
static hipError_t launch_select_t(const ap_cache* c, const float* q, int r_lo, int top_k,
                                  int32_t* sel_out, hipStream_t st) {
  const Dims& dm = c->dm;
  const int Hg = select_heads_per_group(dm);
  const int HG = (dm.Hq + Hg - 1) / Hg;
  const size_t lds = select_lds_bytes(dm, Hg);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_select<T>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = ((dm.B + 7) / 8) * 8 * HG;
  hipLaunchKernelGGL(k_select<T>, dim3(grid), dim3(256), lds, st,
                     static_cast<const T*>(c->Uk), static_cast<const T*>(c->Bk), q, c->qt, c->mask,
                     sel_out, dm.B, dm.N, dm.N_pad, dm.nblk, dm.NP, dm.r_pad, dm.W, dm.d, dm.G,
                     dm.Hq, dm.Hq_pad, Hg, HG, r_lo, top_k);
  return hipGetLastError();
}

hipError_t launch_select(const ap_cache* c, const float* q, int r_lo, int top_k, int32_t* sel_out,
                         hipStream_t st) {
  if (c->dm.storage == AP_BF16) return launch_select_t<bf16_t>(c, q, r_lo, top_k, sel_out, st);
  return launch_select_t<float>(c, q, r_lo, top_k, sel_out, st);
}

template <class T, int NP, int HT>
static hipError_t launch_attn_t(const ap_cache* c, int r_lo, float sl2, int S, int CB, hipStream_t st) {
  const Dims& dm = c->dm;
  constexpr int RP = NP * 16, HP = HT * 16;
  const size_t lds = (size_t)(4 * HP * (RP + 1) + 8 * HP) * sizeof(float);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn<T, NP, HT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_attn<T, NP, HT>), dim3(dm.B * S), dim3(256), lds, st,
                     static_cast<const T*>(c->Uk), static_cast<const T*>(c->Uv), c->qt, c->mask,
                     c->part_z, c->part_ml, dm.N, dm.nblk, CB, S, dm.Hq, r_lo, sl2);
  return hipGetLastError();
}

template <class T, int HT>
static hipError_t dispatch_np(const ap_cache* c, int r_lo, float sl2, int S, int CB, hipStream_t st) {
  switch (c->dm.NP) {
    case 1: return launch_attn_t<T, 1, HT>(c, r_lo, sl2, S, CB, st);
    case 2: return launch_attn_t<T, 2, HT>(c, r_lo, sl2, S, CB, st);
    case 3: return launch_attn_t<T, 3, HT>(c, r_lo, sl2, S, CB, st);
    case 4: return launch_attn_t<T, 4, HT>(c, r_lo, sl2, S, CB, st);
    default: break;
  }
  if constexpr (HT <= 2) {
    switch (c->dm.NP) {
      case 5: return launch_attn_t<T, 5, HT>(c, r_lo, sl2, S, CB, st);
      case 6: return launch_attn_t<T, 6, HT>(c, r_lo, sl2, S, CB, st);
      case 7: return launch_attn_t<T, 7, HT>(c, r_lo, sl2, S, CB, st);
      case 8: return launch_attn_t<T, 8, HT>(c, r_lo, sl2, S, CB, st);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

template <class T>
static hipError_t dispatch_ht(const ap_cache* c, int r_lo, float sl2, int S, int CB, hipStream_t st) {
  switch (c->dm.HT) {
    case 1: return dispatch_np<T, 1>(c, r_lo, sl2, S, CB, st);
    case 2: return dispatch_np<T, 2>(c, r_lo, sl2, S, CB, st);
    case 4: return dispatch_np<T, 4>(c, r_lo, sl2, S, CB, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn(const ap_cache* c, int r_lo, float sl2, int S, int CB, hipStream_t st) {
  if (c->dm.storage == AP_BF16) return dispatch_ht<bf16_t>(c, r_lo, sl2, S, CB, st);
  return dispatch_ht<float>(c, r_lo, sl2, S, CB, st);
}

template <class T>
static hipError_t launch_combine_t(const ap_cache* c, const float* q, float* out, float sl2, int S,
                                   int Tn, const void* tk, const void* tv, hipStream_t st) {
  const Dims& dm = c->dm;
  const size_t lds = (size_t)(dm.d + dm.r_pad + 128 + 2) * sizeof(float);
  hipLaunchKernelGGL(k_combine<T>, dim3(dm.B * dm.Hq), dim3(128), lds, st, c->part_z, c->part_ml,
                     static_cast<const T*>(c->Bv), q, out, static_cast<const T*>(tk),
                     static_cast<const T*>(tv), S, dm.Hq, dm.Hq_pad, dm.r_pad, dm.W, dm.d, dm.G, Tn,
                     sl2);
  return hipGetLastError();
}

hipError_t launch_combine(const ap_cache* c, const float* q, float* out, float sl2, int S, int Tn,
                          const void* tk, const void* tv, hipStream_t st) {
  if (c->dm.storage == AP_BF16) return launch_combine_t<bf16_t>(c, q, out, sl2, S, Tn, tk, tv, st);
  return launch_combine_t<float>(c, q, out, sl2, S, Tn, tk, tv, st);
}

}  // namespace ap

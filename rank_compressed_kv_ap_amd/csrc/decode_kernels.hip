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
//             for every token by MFMA (kept in registers), exact top-k through a
//             linear-bin histogram and an exact resolution of the boundary bin,
//             selection bitmask per 32-token block.
//   k_attn    (sequence, N-split): mixed-rank rescoring, online softmax and latent V
//             accumulation on MFMA tiles, cross-wavefront merge in LDS, one partial
//             (m, l, z[Hq][r]) per split.
//   k_combine (sequence, query head): dense text tokens, log-sum-exp merge of the
//             splits, projection of z through B_v, output.
#include <type_traits>

#include <hip/hip_ext.h>

#include "ap_internal.h"
#include "device_common.h"
#include "tiles.h"

namespace ap {

// ================================================================ k_attn
// Each wavefront walks its 32-token blocks with the next blocks' U_k / U_v tiles and
// selection words already in flight (a ring of 2-4 stages, as deep as the registers
// allow), and updates the online softmax per 16-token half so few values stay live.  The
// latent query's columns below r_lo enter the low-rank logits as bf16 hi + lo (about 16
// bits, as in the selection kernel's scores); the columns at and above r_lo are rounded
// once to bf16, which moves a selected token's full-rank term by about 2^-9 of its size,
// far inside the output tolerance.
template <class T, int NP, int HT>
__device__ __forceinline__ void attn_load(const T* __restrict__ Uk, const T* __restrict__ Uv,
                                          const uint32_t* __restrict__ mask, int b, int blk,
                                          int nblk, int Hq, int lane, LaneTile<T> (&uk)[NP],
                                          LaneTile<T> (&uv)[NP], uint32_t (&mw)[HT]) {
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    uk[p].load(tile_ptr(Uk, tile_base(b, p, blk, NP, nblk)), lane);
    uv[p].load(tile_ptr(Uv, tile_base(b, p, blk, NP, nblk)), lane);
  }
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int h = 16 * ht + (lane & 15);
    const uint32_t w = mask[((size_t)b * nblk + blk) * (HT * 16) + h];   // padded heads: ignored
    mw[ht] = h < Hq ? w : 0u;
  }
}

// two workgroups per CU while the tiles fit the registers (4-bit codes hold as many
// expanded values as bf16)
template <class T>
constexpr int kAttnElemRegBytes = sizeof(T) == 1 ? 2 : static_cast<int>(sizeof(T));
// PLT > 0: r_lo = 16 * PLT, so which panels hold low-rank columns is known at compile
// time and the per-panel MFMAs need no branches; PLT = 0: any r_lo, tested at run time.
template <class T, int NP, int HT, int PLT>
__global__ __launch_bounds__(256, (NP * HT * kAttnElemRegBytes<T> <= 16) ? 2 : 1) void k_attn(
    const T* __restrict__ Uk, const T* __restrict__ Uv, const bf16_t* __restrict__ Usc,
    const float* __restrict__ qt, const uint32_t* __restrict__ mask, float* __restrict__ part_z,
    float* __restrict__ part_ml, float* __restrict__ ema_s, int N, int nblk, int CB, int S, int Hq,
    int r_lo, float sl2) {
  constexpr int RP = NP * 16, HP = HT * 16, ZS = RP + 1;
  // 4-bit codes run the bf16 MFMA path on codes expanded to 136 + code; each product
  // gets one more MFMA with -136 in every A element and the same other operand, which
  // cancels the offset, and the block scales are folded into the latent query (scores)
  // or applied to each block's product (values)
  constexpr bool U4 = std::is_same<T, i4_t>::value;
  constexpr bool BF = std::is_same<T, bf16_t>::value || U4;
  extern __shared__ __align__(16) float smem_f[];
  const int b = blockIdx.x / S, s = blockIdx.x - (blockIdx.x / S) * S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int blk0 = s * CB, blk1 = min(nblk, blk0 + CB);
  // panels wholly below r_lo, and wholly at or above it (one panel may straddle)
  auto lo_panel = [&](int p) { return PLT > 0 ? p < PLT : 16 * p + 16 <= r_lo; };
  auto hi_panel = [&](int p) { return PLT > 0 ? p >= PLT : 16 * p >= r_lo; };

  // latent-query operands: panel p, head tile ht, this lane's 4 columns 16p+4lg+e.
  // Rows of padded heads are loaded too (the buffer holds them) and zeroed after, so
  // every load is unconditional and all of them are in flight together.
  using QT = typename std::conditional<
      U4, float4, typename std::conditional<BF, v4s, QOp<float>>::type>::type;
  QT qop[NP][HT];
  // bf16 factors: the bf16 rounding remainder of the latent query's columns below r_lo
  // (zero above), a second operand for the low-rank logits, which then carry about 16
  // bits of q~ as the selector's do (4-bit codes form it per block, after the scales)
  [[maybe_unused]] v4s qrem[U4 || !BF ? 1 : NP][HT];
  {
    float4 qraw[NP][HT];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
        qraw[p][ht] = *reinterpret_cast<const float4*>(qt + ((size_t)b * HP + 16 * ht + l16) * RP + 16 * p + 4 * lg);
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        // the softmax scale (in log2 units) is folded into the latent query
        const float f = 16 * ht + l16 < Hq ? sl2 : 0.f;
        const float v[4] = {qraw[p][ht].x * f, qraw[p][ht].y * f, qraw[p][ht].z * f, qraw[p][ht].w * f};
        if constexpr (U4) {
          qop[p][ht] = make_float4(v[0], v[1], v[2], v[3]);
        } else if constexpr (BF) {
          const uint2 w = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          qop[p][ht] = __builtin_bit_cast(v4s, w);
          float rr[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            rr[e] = 16 * p + 4 * lg + e < r_lo ? v[e] - bf16_to_f32(f32_to_bf16(v[e])) : 0.f;
          qrem[p][ht] = __builtin_bit_cast(v4s, make_uint2(pack_bf16x2(rr[0], rr[1]), pack_bf16x2(rr[2], rr[3])));
        } else {
          qop[p][ht].set(v);
        }
      }
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

  // Prefetch ring: each wavefront walks its blocks (blk0 + wave + 4i) with the next
  // PD - 1 blocks' tiles and selection words in flight; loads past the wavefront's last
  // block repeat that block (an L2 hit) so that every load is unconditional and the
  // wait before each block counts exactly the PD - 1 younger stages.
  constexpr int PD = U4 ? 4 : (BF && NP * HT <= 8 && NP <= 5 ? 3 : 2);
  LaneTile<T> rk[PD][NP], rv[PD][NP];
  uint32_t rm[PD][HT];
  const int first = blk0 + wave;
  const int nmine = first < blk1 ? (blk1 - first + 3) / 4 : 0;
  auto bidx = [&](int i) { return min(first + 4 * i, blk1 - 1); };
  if (nmine > 0) {
#pragma unroll
    for (int j = 0; j + 1 < PD; ++j)
      attn_load<T, NP, HT>(Uk, Uv, mask, b, bidx(j), nblk, Hq, lane, rk[j], rv[j], rm[j]);
  }
  // 4-bit codes: this workgroup's block scales, [block][K row, V row] as bf16 pairs
  [[maybe_unused]] uint32_t* ssl = reinterpret_cast<uint32_t*>(smem_f + 4 * HP * ZS + 8 * HP);
  if constexpr (U4) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(Usc) + ((size_t)b * nblk + blk0) * RP;
    for (int i = tid; i < (blk1 - blk0) * RP; i += 256) ssl[i] = src[i];
    __syncthreads();
  }

  auto process = [&](const LaneTile<T> (&uk)[NP], const LaneTile<T> (&uv)[NP],
                     const uint32_t (&mw)[HT], int blk) {
    const bool tail = (blk + 1) * kBlockTok > N;
    [[maybe_unused]] uint2 ssc[2][NP];   // 4-bit codes: K and V scales of the lane's columns
    if constexpr (U4) {
      const uint32_t* row = ssl + (blk - blk0) * RP + lg * 2 * NP;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        ssc[0][p] = *reinterpret_cast<const uint2*>(row + 2 * p);
        ssc[1][p] = *reinterpret_cast<const uint2*>(row + RP / 2 + 2 * p);
      }
    }

    if constexpr (BF) {
      // bf16: one 32-token step per head tile.  Scores per 16-token half, one column
      // max for the block, and the value product of both halves in one 16x16x32 MFMA
      // (k-slot 8*(l/16) + 4*half + e <-> token 16*half + 4*(l/16) + e, which is how
      // the V-layout tile and the score tiles already place their elements).
      [[maybe_unused]] uint4 dk[NP];
      if constexpr (U4) {
#pragma unroll
        for (int p = 0; p < NP; ++p) dk[p] = uk[p].deq();
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        v4f slo[2] = {v4f{0, 0, 0, 0}, v4f{0, 0, 0, 0}}, shi[2] = {v4f{0, 0, 0, 0}, v4f{0, 0, 0, 0}};
        v4s qb[NP], qr[NP];   // this block's latent-query operands, and the remainders
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          if constexpr (U4) {
            float s[4];
            q4_scales(ssc[0][p], s);
            const float4 qv = qop[p][ht];
            const float f[4] = {qv.x * s[0], qv.y * s[1], qv.z * s[2], qv.w * s[3]};
            qb[p] = __builtin_bit_cast(v4s, make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])));
            if (!hi_panel(p)) {
              float rr[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                rr[e] = 16 * p + 4 * lg + e < r_lo ? f[e] - bf16_to_f32(f32_to_bf16(f[e])) : 0.f;
              qr[p] = __builtin_bit_cast(v4s, make_uint2(pack_bf16x2(rr[0], rr[1]), pack_bf16x2(rr[2], rr[3])));
            }
          } else {
            qb[p] = qop[p][ht];
            if (!hi_panel(p)) qr[p] = qrem[p][ht];
          }
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            v4s a;
            if constexpr (U4) {
              a = __builtin_bit_cast(v4s, hf == 0 ? make_uint2(dk[p].x, dk[p].y) : make_uint2(dk[p].z, dk[p].w));
            } else {
              a = uk[p].half(hf);
            }
            if (lo_panel(p)) {
              slo[hf] = mfma_bf16(a, qb[p], slo[hf]);
              slo[hf] = mfma_bf16(a, qr[p], slo[hf]);
            } else if (hi_panel(p)) {
              shi[hf] = mfma_bf16(a, qb[p], shi[hf]);
            } else {
              v4s ql = qb[p], qh = qb[p];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (16 * p + 4 * lg + e < r_lo) qh[e] = 0; else ql[e] = 0;
              }
              slo[hf] = mfma_bf16(a, ql, slo[hf]);
              slo[hf] = mfma_bf16(a, qr[p], slo[hf]);   // zero at the columns >= r_lo
              shi[hf] = mfma_bf16(a, qh, shi[hf]);
            }
          }
        if constexpr (U4) {
          // the offset 136 of every expanded code: -136 * (sum of the query operand), the
          // same for every token row, from the same bf16 operands
          const v4s an = __builtin_bit_cast(v4s, make_uint2(kQ4NegOffset2, kQ4NegOffset2));
          v4f clo = v4f{0, 0, 0, 0}, chi = v4f{0, 0, 0, 0};
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            if (lo_panel(p)) {
              clo = mfma_bf16(an, qb[p], clo);
              clo = mfma_bf16(an, qr[p], clo);
            } else if (hi_panel(p)) {
              chi = mfma_bf16(an, qb[p], chi);
            } else {
              v4s ql = qb[p], qh = qb[p];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (16 * p + 4 * lg + e < r_lo) qh[e] = 0; else ql[e] = 0;
              }
              clo = mfma_bf16(an, ql, clo);
              clo = mfma_bf16(an, qr[p], clo);
              chi = mfma_bf16(an, qh, chi);
            }
          }
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            slo[hf] += clo;
            shi[hf] += chi;
          }
        }
        uint32_t bit[8];
        float sc[8];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const uint32_t wb = mw[ht] >> (16 * hf + 4 * lg);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            bit[4 * hf + t] = __builtin_amdgcn_ubfe(wb, t, 1);
            sc[4 * hf + t] = bit[4 * hf + t] ? slo[hf][t] + shi[hf][t] : slo[hf][t];
          }
        }
        if (tail) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (blk * kBlockTok + 16 * (j >> 2) + 4 * lg + (j & 3) >= N) sc[j] = -INFINITY;
        }
        if (ema_s != nullptr) {   // moving-average selector: this step's logits (log2 units)
          const int h = 16 * ht + l16;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int n = blk * kBlockTok + 16 * (j >> 2) + 4 * lg + (j & 3);
            if (h < Hq && n < N) ema_s[((size_t)b * Hq + h) * N + n] = sc[j];
          }
        }
        float bm = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                         fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
        bm = column_max4(bm);
        const float mn = fmaxf(m[ht], bm);
        if (__ballot(mn > m[ht])) {   // rescale only when some running max grew
          const float alpha = hw_exp2(m[ht] - mn);
          lsum[ht] *= alpha;
#pragma unroll
          for (int p = 0; p < NP; ++p) Z[p][ht] *= alpha;
          m[ht] = mn;
        }
        float pv[8];
        uint32_t pa[4], ph[4];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = hw_exp2(sc[j] - mn);
          lsum[ht] += pv[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pa[j] = pack_bf16x2(pv[2 * j], pv[2 * j + 1]);
          ph[j] = pack_bf16x2(bit[2 * j] ? pv[2 * j] : 0.f, bit[2 * j + 1] ? pv[2 * j + 1] : 0.f);
        }
        const v8bf pa8 = __builtin_bit_cast(v8bf, make_uint4(pa[0], pa[1], pa[2], pa[3]));
        const v8bf ph8 = __builtin_bit_cast(v8bf, make_uint4(ph[0], ph[1], ph[2], ph[3]));
        if constexpr (U4) {
          // per block: D = sum over its 32 tokens of code * p (offset cancelled), then
          // Z += scale(column) * D; D row t of this lane is latent column 16p + 4(l/16) + t
          const v8bf an8 = __builtin_bit_cast(v8bf, make_uint4(kQ4NegOffset2, kQ4NegOffset2, kQ4NegOffset2, kQ4NegOffset2));
          const v4f z0 = v4f{0, 0, 0, 0};
          const v4f cpa = mfma_bf16_k32(an8, pa8, z0), cph = mfma_bf16_k32(an8, ph8, z0);
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const v8bf a8 = __builtin_bit_cast(v8bf, uv[p].deq());
            v4f D;
            if (lo_panel(p)) {
              D = mfma_bf16_k32(a8, pa8, cpa);
            } else if (hi_panel(p)) {
              D = mfma_bf16_k32(a8, ph8, cph);
            } else {
              const v4f D1 = mfma_bf16_k32(a8, pa8, cpa), D2 = mfma_bf16_k32(a8, ph8, cph);
#pragma unroll
              for (int t = 0; t < 4; ++t) D[t] = 16 * p + 4 * lg + t < r_lo ? D1[t] : D2[t];
            }
            float s[4];
            q4_scales(ssc[1][p], s);
#pragma unroll
            for (int t = 0; t < 4; ++t) Z[p][ht][t] = fmaf(s[t], D[t], Z[p][ht][t]);
          }
        } else {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const v8bf a8 = __builtin_bit_cast(v8bf, uv[p].raw);
          if (lo_panel(p)) {
            Z[p][ht] = mfma_bf16_k32(a8, pa8, Z[p][ht]);
          } else if (hi_panel(p)) {
            Z[p][ht] = mfma_bf16_k32(a8, ph8, Z[p][ht]);
          } else {
            const bool lo_row = 16 * p + l16 < r_lo;  // this lane's A row is latent column 16p+l16
            const v8bf zero8 = __builtin_bit_cast(v8bf, make_uint4(0u, 0u, 0u, 0u));
            Z[p][ht] = mfma_bf16_k32(lo_row ? a8 : zero8, pa8, Z[p][ht]);
            Z[p][ht] = mfma_bf16_k32(lo_row ? zero8 : a8, ph8, Z[p][ht]);
          }
        }
        }
      }
    } else {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
  #pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          v4f slo = v4f{0, 0, 0, 0}, shi = v4f{0, 0, 0, 0};
  #pragma unroll
          for (int p = 0; p < NP; ++p) {
            if constexpr (BF) {
              const v4s a = uk[p].half(hf);
              if (lo_panel(p)) {
                slo = mfma_bf16(a, qop[p][ht], slo);
              } else if (hi_panel(p)) {
                shi = mfma_bf16(a, qop[p][ht], shi);
              } else {
                v4s ql = qop[p][ht], qh = qop[p][ht];
  #pragma unroll
                for (int e = 0; e < 4; ++e) {
                  if (16 * p + 4 * lg + e < r_lo) qh[e] = 0; else ql[e] = 0;
                }
                slo = mfma_bf16(a, ql, slo);
                shi = mfma_bf16(a, qh, shi);
              }
            } else {
              if (lo_panel(p)) {
                slo = score_mma(uk[p], hf, qop[p][ht], slo);
              } else if (hi_panel(p)) {
                shi = score_mma(uk[p], hf, qop[p][ht], shi);
              } else {
                const int cl = 16 * p + 4 * lg;
                slo = score_mma(uk[p], hf, qop[p][ht].masked(cl, r_lo, true), slo);
                shi = score_mma(uk[p], hf, qop[p][ht].masked(cl, r_lo, false), shi);
              }
            }
          }
          // selection bits of this lane's 4 tokens, scores already scaled (log2 units)
          const uint32_t wb = mw[ht] >> (16 * hf + 4 * lg);
          uint32_t bit[4];
          float sc[4];
  #pragma unroll
          for (int t = 0; t < 4; ++t) {
            bit[t] = __builtin_amdgcn_ubfe(wb, t, 1);
            sc[t] = bit[t] ? slo[t] + shi[t] : slo[t];
          }
          if (tail) {
  #pragma unroll
            for (int t = 0; t < 4; ++t)
              if (blk * kBlockTok + 16 * hf + 4 * lg + t >= N) sc[t] = -INFINITY;
          }
          if (ema_s != nullptr) {   // moving-average selector: this step's logits (log2 units)
            const int h = 16 * ht + l16;
  #pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int n = blk * kBlockTok + 16 * hf + 4 * lg + t;
              if (h < Hq && n < N) ema_s[((size_t)b * Hq + h) * N + n] = sc[t];
            }
          }
          float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
          bm = wave_max_xor(bm, 16);
          bm = wave_max_xor(bm, 32);
          const float mn = fmaxf(m[ht], bm);
          if (__ballot(mn > m[ht])) {   // rescale only when some running max grew
            const float alpha = hw_exp2(m[ht] - mn);
            lsum[ht] *= alpha;
  #pragma unroll
            for (int p = 0; p < NP; ++p) Z[p][ht] *= alpha;
            m[ht] = mn;
          }
          float pv[4], phv[4];
  #pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float e = hw_exp2(sc[t] - mn);
            lsum[ht] += e;
            pv[t] = e;
            phv[t] = bit[t] ? e : 0.f;
          }
          POp<T> pa, ph;
          pa.set(pv);
          ph.set(phv);
  #pragma unroll
          for (int p = 0; p < NP; ++p) {
            if (lo_panel(p)) {
              Z[p][ht] = value_mma(uv[p], hf, true, pa, Z[p][ht]);
            } else if (hi_panel(p)) {
              Z[p][ht] = value_mma(uv[p], hf, true, ph, Z[p][ht]);
            } else {
              const bool lo_row = 16 * p + l16 < r_lo;  // this lane's A row is latent column 16p+l16
              Z[p][ht] = value_mma(uv[p], hf, lo_row, pa, Z[p][ht]);
              Z[p][ht] = value_mma(uv[p], hf, !lo_row, ph, Z[p][ht]);
            }
          }
        }
      }
    }
  };

  for (int i0 = 0; i0 < nmine; i0 += PD) {
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      const int i = i0 + j;
      if (i < nmine) {
        const int ld = (j + PD - 1) % PD;
        attn_load<T, NP, HT>(Uk, Uv, mask, b, bidx(i + PD - 1), nblk, Hq, lane, rk[ld], rv[ld], rm[ld]);
        process(rk[j], rv[j], rm[j], first + 4 * i);
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
// One workgroup of 128 threads per (sequence, query head).  Text rows, partials and
// B_v rows are read with 16-byte loads spread over a lane group (LPR lanes per row,
// RPP = 128/LPR rows at a time) so that many independent loads are in flight.
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

constexpr int kCombThreads = 128;
constexpr int kTextChunk = 256;

template <class T, bool TEXT>
__global__ __launch_bounds__(kCombThreads) void k_combine(
    const float* __restrict__ part_z, const float* __restrict__ part_ml, const T* __restrict__ Bv,
    const float* __restrict__ q, float* __restrict__ out, const T* __restrict__ text_k,
    const T* __restrict__ text_v, int S, int Hq, int HP, int RP, int W, int d, int G, int Tn,
    float sl2, float* __restrict__ ml_out, const float* __restrict__ xo,
    const float* __restrict__ xml) {
  constexpr int V = Vec16<T>::n;
  constexpr int U = 8;                   // rows per thread with loads in flight
  extern __shared__ __align__(16) float smem_c[];
  const int LPR = d / V;                 // lanes per row (a power of two dividing 64)
  const int RPP = kCombThreads / LPR;    // rows per pass
  float* qh = smem_c;                    // [d]
  float* zz = qh + d;                    // [RP]
  float* pt = zz + RP;                   // [kTextChunk]
  float* red = pt + kTextChunk;          // [4]
  float* accb = red + 4;                 // [RPP][d] partial sums across row groups
  float* ws = accb + RPP * d;            // [S] split weights (running maxima first)
  float* ls = ws + S;                    // [S] split sums
  const int b = blockIdx.x / Hq, h = blockIdx.x - (blockIdx.x / Hq) * Hq;
  const int g = h / G;
  const int tid = threadIdx.x;
  const int seg = tid % LPR, rg = tid / LPR;
  const size_t pb = (size_t)b * S * HP;

  // Every load that does not wait on another value is issued here, so that one memory
  // latency covers the partials, the split sums and (with no text tokens, whose row loads
  // would need the same registers) the first pass of B_v rows: the B_v rows of this
  // head's columns (the first U * RPP of them) and this thread's latent column's
  // partials of the first U splits.
  const T* bbase = Bv + (size_t)b * RP * W + (size_t)g * d + seg * V;
  Vec16<T> xb[U];
  // B_v rows are read once per step (non-temporal: they do not displace the token
  // factors in the caches; batch-256 layer combine 28.5 -> 26.3 us)
  if constexpr (!TEXT) {
#pragma unroll
    for (int u = 0; u < U; ++u) xb[u].load_nt(bbase + (size_t)min(u * RPP + rg, RP - 1) * W);
  }
  float zv0[U];
  {
    const float* zb = part_z + pb * RP + (size_t)h * RP + min(tid, RP - 1);
#pragma unroll
    for (int u = 0; u < U; ++u) zv0[u] = zb[(size_t)min(u, S - 1) * HP * RP];
  }
  for (int j = tid; j < d; j += kCombThreads) qh[j] = q[((size_t)b * Hq + h) * d + j];
  float mv = kNegBig;
  for (int s = tid; s < S; s += kCombThreads) {
    const float2 ml = *reinterpret_cast<const float2*>(part_ml + (pb + (size_t)s * HP + h) * 2);
    ws[s] = ml.x;
    ls[s] = ml.y;
    mv = fmaxf(mv, ml.x);
  }
  mv = block_reduce(mv, red, true);   // also publishes qh, ws, ls

  float acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.f;
  float mt = kNegBig, lt = 0.f;
  for (int t0 = 0; TEXT && t0 < Tn; t0 += kTextChunk) {
    const int tc = min(kTextChunk, Tn - t0);
    const T* kbase = text_k + ((size_t)b * Tn + t0) * W + (size_t)g * d + seg * V;
    const T* vbase = text_v + ((size_t)b * Tn + t0) * W + (size_t)g * d + seg * V;
    // scores of the chunk: LPR lanes per text row
    for (int r0 = 0; r0 < tc; r0 += U * RPP) {
      Vec16<T> x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u].load(kbase + (size_t)min(r0 + u * RPP + rg, tc - 1) * W);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < V; ++e) part = fmaf(x[u].get(e), qh[seg * V + e], part);
        part = group_sum(part, LPR);
        const int r = r0 + u * RPP + rg;
        if (seg == 0 && r < tc) pt[r] = part * sl2;
      }
    }
    __syncthreads();
    float cm = -INFINITY;
    for (int i = tid; i < tc; i += kCombThreads) cm = fmaxf(cm, pt[i]);
    cm = block_reduce(cm, red, true);
    const float mn = fmaxf(mt, cm);
    const float alpha = exp2f(mt - mn);
    float lsum = 0.f;
    for (int i = tid; i < tc; i += kCombThreads) {
      const float e = exp2f(pt[i] - mn);
      pt[i] = e;
      lsum += e;
    }
    lsum = block_reduce(lsum, red, false);  // also publishes pt
    lt = lt * alpha + lsum;
    mt = mn;
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] *= alpha;
    for (int r0 = 0; r0 < tc; r0 += U * RPP) {
      Vec16<T> x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u].load(vbase + (size_t)min(r0 + u * RPP + rg, tc - 1) * W);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * RPP + rg;
        const float pr = r < tc ? pt[min(r, tc - 1)] : 0.f;
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = fmaf(pr, x[u].get(e), acc[e]);
      }
    }
    __syncthreads();
  }

  // another segment's attention, already merged over its own tokens: its normalised
  // output xo with its softmax maximum and sum (xml), joined as one more partial
  const size_t bh = (size_t)b * Hq + h;
  const float xm = xml != nullptr ? xml[bh * 2] : kNegBig;
  const float xl = xml != nullptr ? xml[bh * 2 + 1] : 0.f;
  const float M = fmaxf(fmaxf(mv, mt), xm);
  float L = 0.f;
  for (int s = tid; s < S; s += kCombThreads) {
    const float w = exp2f(ws[s] - M);
    L += w * ls[s];
    ws[s] = w;
  }
  L = block_reduce(L, red, false);   // also publishes the weights
  const float wt = exp2f(mt - M);
  const float wx = exp2f(xm - M) * xl;
  L += wt * lt + wx;

  // merge the split partials: z[i] = sum_s w_s z_s[i]
  for (int i = tid; i < RP; i += kCombThreads) {
    const float* zb = part_z + pb * RP + (size_t)h * RP + i;
    float z = 0.f;
    for (int s0 = 0; s0 < S; s0 += U) {
      float zv[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        zv[u] = (i == tid && s0 == 0) ? zv0[u] : zb[(size_t)min(s0 + u, S - 1) * HP * RP];
#pragma unroll
      for (int u = 0; u < U; ++u) z = fmaf(s0 + u < S ? ws[min(s0 + u, S - 1)] : 0.f, zv[u], z);
    }
    zz[i] = z;
  }
  __syncthreads();
  // projection through B_v: row group rg takes latent rows rg, rg+RPP, ... (the first
  // pass's rows were loaded at the start when there is no text)
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] *= wt;
  for (int i0 = 0; i0 < RP; i0 += U * RPP) {
    if (TEXT || i0 > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) xb[u].load_nt(bbase + (size_t)min(i0 + u * RPP + rg, RP - 1) * W);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * RPP + rg;
      const float zi = i < RP ? zz[min(i, RP - 1)] : 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = fmaf(zi, xb[u].get(e), acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < V; ++e) accb[rg * d + seg * V + e] = acc[e];
  __syncthreads();
  const float invL = 1.f / L;
  if (ml_out != nullptr && tid == 0) {   // softmax max (log2 units) and sum, for the selector state
    ml_out[((size_t)b * Hq + h) * 2] = M;
    ml_out[((size_t)b * Hq + h) * 2 + 1] = L;
  }
  for (int j = tid; j < d; j += kCombThreads) {
    float o = xml != nullptr ? wx * xo[bh * d + j] : 0.f;
    for (int r = 0; r < RPP; ++r) o += accb[r * d + j];
    out[((size_t)b * Hq + h) * d + j] = o * invL;
  }
}

// ================================================================ k_combine_wide
// The combine of a batch with no text tokens and no second segment, for wide rows of
// B_v: one workgroup per (sequence, block of CW columns = whole KV heads), every query
// head of those KV heads.  Per head: the log-sum-exp merge of the splits (maximum,
// split weights, sum); per (head, latent row): the merged latent sum; then each thread
// takes one V-element column chunk and the latent rows rg, rg + RG, ... of its row
// group, the first UB of them requested before the merge, and the row groups' partial
// sums meet in LDS.
constexpr int kWideThreadsMax = 256;
constexpr int kWideMaxG = 4;       // query heads per KV head held in registers

template <class T, int G>
__global__ __launch_bounds__(kWideThreadsMax) void k_combine_wide(
    const float* __restrict__ part_z, const float* __restrict__ part_ml, const T* __restrict__ Bv,
    float* __restrict__ out, int S, int Hq, int HP, int RP, int W, int d, int CW, int RG,
    float* __restrict__ ml_out) {
  constexpr int V = Vec16<T>::n;
  constexpr int UB = G <= 1 ? 16 : 8;   // B_v rows per thread in flight (registers)
  extern __shared__ __align__(16) float smem_w[];
  const int CH = W / CW;
  const int b = blockIdx.x / CH, cb = blockIdx.x - (blockIdx.x / CH) * CH;
  const int c0 = cb * CW;
  const int kv0 = c0 / d;
  const int h0 = kv0 * G;                // first query head of this block
  const int nh = (CW / d) * G;           // query heads of this block
  const int nchunk = CW / V;
  const int tid = threadIdx.x;
  const int chunk = tid % nchunk, rg = tid / nchunk;   // blockDim = nchunk * RG
  float* zf = smem_w;                    // [nh][RP] merged latent sums
  float* linv = zf + nh * RP;            // [nh] 1 / softmax sum
  float* wgt = linv + nh;                // [nh][S] split weights
  float* red = wgt + nh * S;             // [RG][G][CW] row-group partial sums
  const size_t pb = (size_t)b * S * HP;
  const int col = c0 + chunk * V;        // first column of this thread's chunk
  const int hl0 = (col / d - kv0) * G;   // its first query head, local
  const T* bbase = Bv + (size_t)b * RP * W + col;
  const int nrow = (RP - rg + RG - 1) / RG;

  Vec16<T> xb[UB];
#pragma unroll
  for (int u = 0; u < UB; ++u) xb[u].load(bbase + (size_t)min(rg + u * RG, RP - 1) * W);

  for (int hl = tid; hl < nh; hl += blockDim.x) {
    const int h = h0 + hl;
    float M = kNegBig;
    for (int s = 0; s < S; ++s) M = fmaxf(M, part_ml[(pb + (size_t)s * HP + h) * 2]);
    float L = 0.f;
    for (int s = 0; s < S; ++s) {
      const float2 ml = *reinterpret_cast<const float2*>(part_ml + (pb + (size_t)s * HP + h) * 2);
      const float w = exp2f(ml.x - M);
      wgt[hl * S + s] = w;
      L += w * ml.y;
    }
    linv[hl] = 1.f / L;
    if (ml_out != nullptr) {   // softmax max (log2 units) and sum, for the selector state
      ml_out[((size_t)b * Hq + h) * 2] = M;
      ml_out[((size_t)b * Hq + h) * 2 + 1] = L;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < nh * RP; idx += blockDim.x) {
    const int hl = idx / RP, i = idx - hl * RP;
    const float* zb = part_z + (pb + h0 + hl) * RP + i;
    float z = 0.f;
#pragma unroll 4
    for (int s = 0; s < S; ++s) z = fmaf(wgt[hl * S + s], zb[(size_t)s * HP * RP], z);
    zf[idx] = z;
  }
  __syncthreads();

  float acc[G][V];
#pragma unroll
  for (int gh = 0; gh < G; ++gh)
#pragma unroll
    for (int e = 0; e < V; ++e) acc[gh][e] = 0.f;
  for (int u0 = 0; u0 < nrow; u0 += UB) {
    if (u0 > 0) {
#pragma unroll
      for (int u = 0; u < UB; ++u) xb[u].load(bbase + (size_t)min(rg + (u0 + u) * RG, RP - 1) * W);
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int row = rg + (u0 + u) * RG;
      if (u0 + u < nrow) {
#pragma unroll
        for (int gh = 0; gh < G; ++gh) {
          const float z = zf[(hl0 + gh) * RP + row];
#pragma unroll
          for (int e = 0; e < V; ++e) acc[gh][e] = fmaf(z, xb[u].get(e), acc[gh][e]);
        }
      }
    }
  }
#pragma unroll
  for (int gh = 0; gh < G; ++gh)
#pragma unroll
    for (int e = 0; e < V; ++e) red[((size_t)rg * G + gh) * CW + chunk * V + e] = acc[gh][e];
  __syncthreads();
  for (int idx = tid; idx < G * CW; idx += blockDim.x) {
    const int gh = idx / CW, cc = idx - gh * CW;
    const int kv = (c0 + cc) / d, j = (c0 + cc) - kv * d;
    const int hl = (kv - kv0) * G + gh;
    float o = 0.f;
    for (int r = 0; r < RG; ++r) o += red[((size_t)r * G + gh) * CW + cc];
    out[((size_t)b * Hq + h0 + hl) * d + j] = o * linv[hl];
  }
}

// Scalar variant for head sizes the 16-byte path does not tile.
template <class T>
__global__ __launch_bounds__(kCombThreads) void k_combine_scalar(
    const float* __restrict__ part_z, const float* __restrict__ part_ml, const T* __restrict__ Bv,
    const float* __restrict__ q, float* __restrict__ out, const T* __restrict__ text_k,
    const T* __restrict__ text_v, int S, int Hq, int HP, int RP, int W, int d, int G, int Tn,
    float sl2, float* __restrict__ ml_out, const float* __restrict__ xo,
    const float* __restrict__ xml) {
  extern __shared__ __align__(16) float smem_c[];
  float* qh = smem_c;
  float* zz = qh + d;
  float* pt = zz + RP;
  float* red = pt + kCombThreads;
  const int b = blockIdx.x / Hq, h = blockIdx.x - (blockIdx.x / Hq) * Hq;
  const int g = h / G;
  const int tid = threadIdx.x;
  const size_t pb = (size_t)b * S * HP;
  for (int j = tid; j < d; j += kCombThreads) qh[j] = q[((size_t)b * Hq + h) * d + j];
  float mv = kNegBig;
  for (int s = tid; s < S; s += kCombThreads) mv = fmaxf(mv, part_ml[(pb + (size_t)s * HP + h) * 2]);
  mv = block_reduce(mv, red, true);
  constexpr int kMaxJ = 2;  // d <= 256
  float acc[kMaxJ] = {0.f, 0.f};
  float mt = kNegBig, lt = 0.f;
  for (int t0 = 0; t0 < Tn; t0 += kCombThreads) {
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
    const float ls = block_reduce(pv, red, false);
    lt = lt * alpha + ls;
    mt = mn;
    const int tc = min(kCombThreads, Tn - t0);
    for (int jj = 0; jj < kMaxJ; ++jj) {
      const int j = tid + kCombThreads * jj;
      if (j < d) {
        float a = acc[jj] * alpha;
        const T* col = text_v + ((size_t)b * Tn + t0) * W + (size_t)g * d + j;
        for (int tt = 0; tt < tc; ++tt) a = fmaf(pt[tt], to_f32(col[(size_t)tt * W]), a);
        acc[jj] = a;
      }
    }
    __syncthreads();
  }
  const size_t bh = (size_t)b * Hq + h;
  const float xm = xml != nullptr ? xml[bh * 2] : kNegBig;
  const float xl = xml != nullptr ? xml[bh * 2 + 1] : 0.f;
  const float M = fmaxf(fmaxf(mv, mt), xm);
  float L = 0.f;
  for (int s = tid; s < S; s += kCombThreads) {
    const float* ml = part_ml + (pb + (size_t)s * HP + h) * 2;
    L += exp2f(ml[0] - M) * ml[1];
  }
  L = block_reduce(L, red, false);
  const float wt = exp2f(mt - M);
  const float wx = exp2f(xm - M) * xl;
  L += wt * lt + wx;
  for (int i = tid; i < RP; i += kCombThreads) {
    float z = 0.f;
    for (int s = 0; s < S; ++s)
      z += exp2f(part_ml[(pb + (size_t)s * HP + h) * 2] - M) * part_z[(pb + (size_t)s * HP + h) * RP + i];
    zz[i] = z;
  }
  __syncthreads();
  const float invL = 1.f / L;
  if (ml_out != nullptr && tid == 0) {
    ml_out[((size_t)b * Hq + h) * 2] = M;
    ml_out[((size_t)b * Hq + h) * 2 + 1] = L;
  }
  for (int jj = 0; jj < kMaxJ; ++jj) {
    const int j = tid + kCombThreads * jj;
    if (j < d) {
      float o = wt * acc[jj] + (xml != nullptr ? wx * xo[bh * d + j] : 0.f);
      const T* col = Bv + (size_t)b * RP * W + (size_t)g * d + j;
      for (int i = 0; i < RP; ++i) o = fmaf(zz[i], to_f32(col[(size_t)i * W]), o);
      out[((size_t)b * Hq + h) * d + j] = o * invL;
    }
  }
}

// ================================================================ launchers
template <class T, int NP, int HT, int PLT>
static hipError_t launch_attn_t(const ap_cache* c, int r_lo, float sl2, int S, int CB, float* ema_s, hipStream_t st,
                                const KernelEvents& ev) {
  const Dims& dm = c->dm;
  constexpr int RP = NP * 16, HP = HT * 16;
  // merge buffers, then (4-bit codes) the workgroup's block scales
  const size_t lds = (size_t)(4 * HP * (RP + 1) + 8 * HP) * sizeof(float) +
                     (std::is_same<T, i4_t>::value ? (size_t)CB * RP * 4 : 0);
  static std::atomic<uint32_t> lds_set{0};
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(&k_attn<T, NP, HT, PLT>), 160 * 1024, lds_set);
  if (e != hipSuccess) return e;
  hipExtLaunchKernelGGL((k_attn<T, NP, HT, PLT>), dim3(dm.B * S), dim3(256), lds, st, ev.start, ev.stop, 0,
                     static_cast<const T*>(c->Uk), static_cast<const T*>(c->Uv),
                     reinterpret_cast<const bf16_t*>(c->Usc), c->qt, c->mask,
                     c->part_z, c->part_ml, ema_s, dm.N, dm.nblk, CB, S, dm.Hq, r_lo, sl2);
  return hipGetLastError();
}

// bf16 / 4-bit factors with r <= 64 and r_lo a multiple of 16: the compile-time panel split
template <class T, int NP, int HT>
static hipError_t launch_attn_r(const ap_cache* c, int r_lo, float sl2, int S, int CB, float* ema_s,
                                hipStream_t st, const KernelEvents& ev) {
  if constexpr (!std::is_same<T, float>::value && NP <= 4) {
    if (r_lo % 16 == 0) {
      switch (r_lo / 16) {
        case 1: return launch_attn_t<T, NP, HT, 1>(c, r_lo, sl2, S, CB, ema_s, st, ev);
        case 2: if constexpr (NP >= 2) return launch_attn_t<T, NP, HT, 2>(c, r_lo, sl2, S, CB, ema_s, st, ev); break;
        case 3: if constexpr (NP >= 3) return launch_attn_t<T, NP, HT, 3>(c, r_lo, sl2, S, CB, ema_s, st, ev); break;
        case 4: if constexpr (NP >= 4) return launch_attn_t<T, NP, HT, 4>(c, r_lo, sl2, S, CB, ema_s, st, ev); break;
        default: break;
      }
    }
  }
  return launch_attn_t<T, NP, HT, 0>(c, r_lo, sl2, S, CB, ema_s, st, ev);
}

template <class T, int HT>
static hipError_t dispatch_np(const ap_cache* c, int r_lo, float sl2, int S, int CB, float* ema_s, hipStream_t st,
                              const KernelEvents& ev) {
  switch (c->dm.NP) {
    case 1: return launch_attn_r<T, 1, HT>(c, r_lo, sl2, S, CB, ema_s, st, ev);
    case 2: return launch_attn_r<T, 2, HT>(c, r_lo, sl2, S, CB, ema_s, st, ev);
    case 3: return launch_attn_r<T, 3, HT>(c, r_lo, sl2, S, CB, ema_s, st, ev);
    case 4: return launch_attn_r<T, 4, HT>(c, r_lo, sl2, S, CB, ema_s, st, ev);
    default: break;
  }
  if constexpr (HT <= 2) {
    switch (c->dm.NP) {
      case 5: return launch_attn_r<T, 5, HT>(c, r_lo, sl2, S, CB, ema_s, st, ev);
      case 6: return launch_attn_r<T, 6, HT>(c, r_lo, sl2, S, CB, ema_s, st, ev);
      case 7: return launch_attn_r<T, 7, HT>(c, r_lo, sl2, S, CB, ema_s, st, ev);
      case 8: return launch_attn_r<T, 8, HT>(c, r_lo, sl2, S, CB, ema_s, st, ev);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

template <class T>
static hipError_t dispatch_ht(const ap_cache* c, int r_lo, float sl2, int S, int CB, float* ema_s, hipStream_t st,
                              const KernelEvents& ev) {
  switch (c->dm.HT) {
    case 1: return dispatch_np<T, 1>(c, r_lo, sl2, S, CB, ema_s, st, ev);
    case 2: return dispatch_np<T, 2>(c, r_lo, sl2, S, CB, ema_s, st, ev);
    case 4: return dispatch_np<T, 4>(c, r_lo, sl2, S, CB, ema_s, st, ev);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn(const ap_cache* c, int r_lo, float sl2, int S, int CB, float* ema_s, hipStream_t st,
                       const KernelEvents& ev) {
  if (c->dm.storage == AP_INT4) return dispatch_ht<i4_t>(c, r_lo, sl2, S, CB, ema_s, st, ev);
  if (c->dm.storage == AP_BF16) return dispatch_ht<bf16_t>(c, r_lo, sl2, S, CB, ema_s, st, ev);
  return dispatch_ht<float>(c, r_lo, sl2, S, CB, ema_s, st, ev);
}

template <class T>
static hipError_t launch_combine_t(const ap_cache* c, const float* q, float* out, float sl2, int S,
                                   int Tn, const void* tk, const void* tv, float* ml_out,
                                   const float* xo, const float* xml, hipStream_t st,
                                   const KernelEvents& ev) {
  const Dims& dm = c->dm;
  constexpr int V = 16 / sizeof(T);
  const int lpr = dm.d / V;
  const bool pow2 = lpr > 0 && (lpr & (lpr - 1)) == 0 && lpr <= 64;
  const bool aligned = (reinterpret_cast<uintptr_t>(tk) % 16 == 0) && (reinterpret_cast<uintptr_t>(tv) % 16 == 0);
  const bool vec = dm.d % V == 0 && pow2 && ((size_t)dm.W * sizeof(T)) % 16 == 0 && aligned;
  if (vec) {
    const int rpp = kCombThreads / lpr;
    const size_t lds = (size_t)(dm.d + dm.r_pad + kTextChunk + 4 + rpp * dm.d + 2 * S) * sizeof(float);
    if (Tn > 0)
      hipExtLaunchKernelGGL((k_combine<T, true>), dim3(dm.B * dm.Hq), dim3(kCombThreads), lds, st, ev.start,
                            ev.stop, 0, c->part_z, c->part_ml, static_cast<const T*>(c->Bv), q, out,
                            static_cast<const T*>(tk), static_cast<const T*>(tv), S, dm.Hq, dm.Hq_pad,
                            dm.r_pad, dm.W, dm.d, dm.G, Tn, sl2, ml_out, xo, xml);
    else
      hipExtLaunchKernelGGL((k_combine<T, false>), dim3(dm.B * dm.Hq), dim3(kCombThreads), lds, st,
                            ev.start, ev.stop, 0, c->part_z, c->part_ml, static_cast<const T*>(c->Bv), q,
                            out, static_cast<const T*>(tk), static_cast<const T*>(tv), S, dm.Hq,
                            dm.Hq_pad, dm.r_pad, dm.W, dm.d, dm.G, Tn, sl2, ml_out, xo, xml);
  } else {
    const size_t lds = (size_t)(dm.d + dm.r_pad + kCombThreads + 4) * sizeof(float);
    hipExtLaunchKernelGGL(k_combine_scalar<T>, dim3(dm.B * dm.Hq), dim3(kCombThreads), lds, st,
                          ev.start, ev.stop, 0,
                       c->part_z, c->part_ml, static_cast<const T*>(c->Bv), q, out,
                       static_cast<const T*>(tk), static_cast<const T*>(tv), S, dm.Hq, dm.Hq_pad,
                       dm.r_pad, dm.W, dm.d, dm.G, Tn, sl2, ml_out, xo, xml);
  }
  return hipGetLastError();
}

// The wide combine's plan: the fewest column blocks (whole KV heads, a divisor of Hkv)
// that give about 2048 workgroups; row groups as many as the threads, the rows and a
// 32 KB partial-sum buffer allow.  Returns false where it does not apply.  It serves
// grouped-query layers (G >= 2: each B_v row chunk is read once for the G query heads
// that share it, instead of once per query head; batch-64 GQA layer combine 9.9 -> 8.3
// us) with few splits; with one query head per KV head the per-head kernel is as fast
// (batch-256 layer: 28 us both), and with many splits (64 on the batch-4 long-video
// layer) its per-head merge loops are the shorter chain (8.9 against 28 us).
static bool wide_plan(const Dims& dm, int S, int* CW, int* RG, int* threads, size_t* lds) {
  constexpr int V = 8;   // bf16 elements per 16-byte load
  if (dm.storage == AP_F32 || dm.G < 2 || dm.G > kWideMaxG || S > 16 || dm.d % V != 0 || dm.W % V != 0)
    return false;
  int CH = dm.Hkv;
  for (int c = 1; c <= dm.Hkv; ++c)
    if (dm.Hkv % c == 0 && (long long)dm.B * c >= 2048) { CH = c; break; }
  const int cw = dm.W / CH;
  const int nchunk = cw / V;
  if (nchunk > kWideThreadsMax) return false;
  int rg = 1;
  while (2 * rg <= dm.r_pad && nchunk * 2 * rg <= kWideThreadsMax && 2 * rg * dm.G * cw <= 8192) rg *= 2;
  const int nh = (cw / dm.d) * dm.G;
  const size_t bytes = ((size_t)nh * dm.r_pad + nh + (size_t)nh * S + (size_t)rg * dm.G * cw) * sizeof(float);
  if (bytes > 64 * 1024) return false;
  *CW = cw;
  *RG = rg;
  *threads = nchunk * rg;
  *lds = bytes;
  return true;
}

template <int G>
static hipError_t launch_wide_g(const ap_cache* c, float* out, int S, int CW, int RG, int threads, size_t lds,
                                float* ml_out, hipStream_t st, const KernelEvents& ev) {
  const Dims& dm = c->dm;
  hipExtLaunchKernelGGL((k_combine_wide<bf16_t, G>), dim3(dm.B * (dm.W / CW)), dim3(threads), lds, st,
                        ev.start, ev.stop, 0, c->part_z, c->part_ml, static_cast<const bf16_t*>(c->Bv), out,
                        S, dm.Hq, dm.Hq_pad, dm.r_pad, dm.W, dm.d, CW, RG, ml_out);
  return hipGetLastError();
}

hipError_t launch_combine(const ap_cache* c, const float* q, float* out, float sl2, int S, int Tn,
                          const void* tk, const void* tv, float* ml_out, const float* xo,
                          const float* xml, hipStream_t st, const KernelEvents& ev) {
  // grouped-query layers with no text tokens and no second segment: the wide combine
  int CW = 0, RG = 0, threads = 0;
  size_t lds = 0;
  if (Tn == 0 && xo == nullptr && xml == nullptr && wide_plan(c->dm, S, &CW, &RG, &threads, &lds)) {
    switch (c->dm.G) {
      case 2: return launch_wide_g<2>(c, out, S, CW, RG, threads, lds, ml_out, st, ev);
      case 3: return launch_wide_g<3>(c, out, S, CW, RG, threads, lds, ml_out, st, ev);
      case 4: return launch_wide_g<4>(c, out, S, CW, RG, threads, lds, ml_out, st, ev);
      default: break;
    }
  }
  // B and the text tokens are bf16 for 4-bit caches too
  if (c->dm.storage != AP_F32)
    return launch_combine_t<bf16_t>(c, q, out, sl2, S, Tn, tk, tv, ml_out, xo, xml, st, ev);
  return launch_combine_t<float>(c, q, out, sl2, S, Tn, tk, tv, ml_out, xo, xml, st, ev);
}

// ================================================================ k_text_seg
// A small factored segment (the text tokens factored apart) of one (sequence, query
// head), whole, in one workgroup: latent query q~ = B_k[:, g's columns] q_h, scores of
// every token at the low rank and the remainder up to the full rank, the segment's
// top_k tokens by low-rank score (ties to the lower id) at full rank, softmax, latent
// values z = sum_n p[n] U_v[n, :r(n)], projection through the segment's B_v.  Writes
// the normalised output and the softmax maximum and sum (log2 units), which the visual
// combine merges as one more partial.  The segment's U_k, U_v (through the tiled
// layouts, 4-bit codes with their block scales) and this KV head's rows of B_k, B_v are
// first staged in LDS in one round of independent loads.
constexpr int kSegThreads = 256;

// One lane's 8 elements of a tiled panel as floats (4-bit codes times their block scales).
template <class T>
__device__ __forceinline__ void seg_lane8(const T* __restrict__ U, const bf16_t* __restrict__ Usc,
                                          bool vl, int b, int p, int blk, int lane, int NP, int nblk,
                                          float (&v)[8]) {
  const size_t base = tile_base(b, p, blk, NP, nblk);
  if constexpr (std::is_same<T, i4_t>::value) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(tile_ptr(U, base))[lane];
    const bf16_t* srow = Usc + (((size_t)b * nblk + blk) * 2 + (vl ? 1 : 0)) * 16 * NP;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int col = vl ? 16 * p + (lane & 15) : 16 * p + 4 * (lane >> 4) + (i & 3);
      v[i] = static_cast<float>(static_cast<int>((w >> q4_shift(i)) & 0xFu) - 8) *
             bf16_to_f32(srow[scale_slot(col, NP)]);
    }
  } else if constexpr (std::is_same<T, bf16_t>::value) {
    const uint4 raw = *reinterpret_cast<const uint4*>(U + base + lane * 8);
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float((i & 1) ? (wd[i >> 1] & 0xFFFF0000u) : (wd[i >> 1] << 16));
  } else {
    const float4 a = *reinterpret_cast<const float4*>(U + base + lane * 8);
    const float4 c = *reinterpret_cast<const float4*>(U + base + lane * 8 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
  }
}

template <class T>
__global__ __launch_bounds__(kSegThreads) void k_text_seg(
    const T* __restrict__ Uk, const T* __restrict__ Uv, const bf16_t* __restrict__ Usc,
    const StoreB<T>* __restrict__ Bk, const StoreB<T>* __restrict__ Bv, const float* __restrict__ q,
    float* __restrict__ xo, float* __restrict__ xml, int32_t* __restrict__ sel_out, int N, int nblk,
    int NP, int r, int W, int d, int G, int Hq, int r_lo, int top_k, float sl2) {
  extern __shared__ __align__(16) float smem_s[];
  const int RP = 16 * NP, US = RP + 1;   // padded rows: no bank conflicts across tokens
  float* uk = smem_s;            // [N][US] U_k of the segment (columns >= r zero)
  float* uv = uk + N * US;       // [N][US] U_v
  float* bv = uv + N * US;       // [RP][d] this KV head's columns of B_v
  float* qt = bv + RP * d;       // [RP] latent query, scaled to log2 units
  float* slo = qt + RP;          // [N] low-rank scores
  float* sc = slo + N;           // [N] scores, then weights
  float* fl = sc + N;            // [N] 1 for the segment's top_k tokens
  float* zz = fl + N;            // [RP]
  float* red = zz + RP;          // [kSegThreads / 64]
  const int b = blockIdx.x / Hq, h = blockIdx.x - (blockIdx.x / Hq) * Hq;
  const int g = h / G, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto block_red = [&](float v, bool is_max) {   // also publishes earlier LDS writes
    for (int off = 32; off > 0; off >>= 1) {
      const float o = __shfl_xor(v, off, 64);
      v = is_max ? fmaxf(v, o) : v + o;
    }
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float x = red[0];
    for (int w = 1; w < kSegThreads / 64; ++w) x = is_max ? fmaxf(x, red[w]) : x + red[w];
    __syncthreads();
    return x;
  };
  // ---- stage everything the segment reads: batches of 4 independent 16-byte loads per
  // thread (indices clamped, so every load is issued), then the LDS stores
  // Latent query from the loaded chunks: a row of B_k is cpr consecutive lanes (cpr a
  // power of two dividing 64), each dotting its chunk with q, summed across the lanes.
  using TB = StoreB<T>;
  constexpr int V = Vec16<TB>::n;
  const float* qg = q + ((size_t)b * Hq + h) * d;
  const int cpr = d / V, nch = RP * cpr;
  for (int c0 = 0; c0 < nch; c0 += 4 * kSegThreads) {
    Vec16<TB> xk[4], xv[4];
    float qv[4][V];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cc = min(c0 + u * kSegThreads + tid, nch - 1), i = cc / cpr, jc = cc - (cc / cpr) * cpr;
      const size_t off = ((size_t)b * RP + i) * W + (size_t)g * d + jc * V;
      xk[u].load(Bk + off);
      xv[u].load(Bv + off);
#pragma unroll
      for (int e = 0; e < V; ++e) qv[u][e] = qg[jc * V + e];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cc = c0 + u * kSegThreads + tid;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) part = fmaf(xk[u].get(e), qv[u][e], part);
      part = group_sum(part, cpr);   // uniform trip count: every lane takes part
      if (cc < nch) {
        const int i = cc / cpr, jc = cc - (cc / cpr) * cpr;
        if (jc == 0) qt[i] = i < r ? part * sl2 : 0.f;
#pragma unroll
        for (int e = 0; e < V; ++e) bv[i * d + jc * V + e] = xv[u].get(e);
      }
    }
  }
  const int nlw = nblk * NP * 64;   // lane words of one factor
  for (int w0 = 0; w0 < nlw; w0 += 2 * kSegThreads) {
    float a[2][8], c[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = min(w0 + u * kSegThreads + tid, nlw - 1);
      const int ln = idx & 63, p = (idx >> 6) % NP, blk = (idx >> 6) / NP;
      seg_lane8<T>(Uk, Usc, false, b, p, blk, ln, NP, nblk, a[u]);
      seg_lane8<T>(Uv, Usc, true, b, p, blk, ln, NP, nblk, c[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = w0 + u * kSegThreads + tid;
      if (idx < nlw) {
        const int ln = idx & 63, p = (idx >> 6) % NP, blk = (idx >> 6) / NP;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int half = i >> 2, e = i & 3;
          const int tk = 32 * blk + 16 * half + (ln & 15), ck = 16 * p + 4 * (ln >> 4) + e;   // K layout
          const int tv = 32 * blk + 16 * half + 4 * (ln >> 4) + e, cv = 16 * p + (ln & 15);  // V layout
          if (tk < N) uk[tk * US + ck] = ck < r ? a[u][i] : 0.f;
          if (tv < N) uv[tv * US + cv] = cv < r ? c[u][i] : 0.f;
        }
      }
    }
  }
  __syncthreads();
  for (int n = tid; n < N; n += kSegThreads) {
    float lo = 0.f, hi = 0.f;
#pragma unroll 8
    for (int i = 0; i < RP; ++i) {
      const float v = uk[n * US + i] * qt[i];
      if (i < r_lo) lo += v; else hi += v;
    }
    slo[n] = lo;
    sc[n] = hi;
  }
  __syncthreads();
  // the segment's top_k by low-rank score, ties to the lower id: n is taken when fewer
  // than top_k tokens rank ahead of it.  Four lanes count for one token, a quarter of
  // the tokens each, and their counts are summed across the quad.
  float mloc = -INFINITY;
  const int quarter = (N + 3) / 4;
  for (int n0 = 0; n0 < N; n0 += kSegThreads / 4) {
    const int n = n0 + (tid >> 2), part = tid & 3;
    const float s = slo[min(n, N - 1)];
    int ahead = 0;
    const int m1 = min(N, (part + 1) * quarter);
#pragma unroll 4
    for (int m = part * quarter; m < m1; ++m) {
      const float t = slo[m];
      ahead += (t > s || (t == s && m < n)) ? 1 : 0;
    }
    ahead += __shfl_xor(ahead, 1, 64);
    ahead += __shfl_xor(ahead, 2, 64);
    if (n < N && part == 0) {
      const bool sel = ahead < top_k;
      const float v = sel ? s + sc[n] : s;
      sc[n] = v;
      fl[n] = sel ? 1.f : 0.f;
      mloc = fmaxf(mloc, v);
    }
  }
  const float M = block_red(mloc, true);   // its barriers also publish fl[]
  if (sel_out != nullptr && wave == 0) {
    // the selected ids in ascending order: ballots over 64 tokens at a time
    int32_t* so = sel_out + ((size_t)b * Hq + h) * top_k;
    int carry = 0;
    for (int n0 = 0; n0 < N; n0 += 64) {
      const int n = n0 + lane;
      const bool taken = n < N && fl[n] > 0.f;
      const unsigned long long m = __ballot(taken);
      const int pos = carry + __popcll(m & ((1ull << lane) - 1ull));
      if (taken && pos < top_k) so[pos] = n;
      carry += __popcll(m);
    }
  }
  float lsum = 0.f;
  for (int n = tid; n < N; n += kSegThreads) {
    const float e = hw_exp2(sc[n] - M);
    sc[n] = e;
    lsum += e;
  }
  const float L = block_red(lsum, false);
  // latent values: 16 lanes per latent column, each over every 16th token, then summed
  // across the 16 lanes (fixed order)
  for (int i0 = 0; i0 < RP; i0 += kSegThreads / 16) {
    const int i = i0 + (tid >> 4), part = tid & 15;
    float z = 0.f;
    if (i < RP) {
#pragma unroll 4
      for (int n = part; n < N; n += 16) z = fmaf((i < r_lo || fl[n] > 0.f) ? sc[n] : 0.f, uv[n * US + i], z);
    }
    z = group_sum(z, 16);
    if (i < RP && part == 0) zz[i] = z;
  }
  __syncthreads();
  const float invL = 1.f / L;
  for (int j = tid; j < d; j += kSegThreads) {
    float o = 0.f;
#pragma unroll 8
    for (int i = 0; i < RP; ++i) o = fmaf(zz[i], bv[i * d + j], o);
    xo[((size_t)b * Hq + h) * d + j] = o * invL;
  }
  if (tid == 0) {
    xml[((size_t)b * Hq + h) * 2] = M;
    xml[((size_t)b * Hq + h) * 2 + 1] = L;
  }
}

static size_t text_seg_lds(const Dims& dm) {
  return (size_t)(2 * dm.N * (dm.r_pad + 1) + dm.r_pad * dm.d + 2 * dm.r_pad + 3 * dm.N +
                  kSegThreads / 64) * sizeof(float);
}

bool text_seg_supported(const Dims& dm) {
  // B rows read as 16-byte chunks of this head's columns, a power of two of them per row
  const int V = dm.storage == AP_F32 ? 4 : 8;
  const int cpr = dm.d / V;
  return text_seg_lds(dm) <= 96 * 1024 && dm.d % V == 0 && dm.W % V == 0 && cpr <= 64 &&
         (cpr & (cpr - 1)) == 0;
}

hipError_t launch_text_seg(const ap_cache* c, const float* q, int r_lo, int top_k, int32_t* sel_out,
                           float sl2, hipStream_t st, const KernelEvents& ev) {
  const Dims& dm = c->dm;
  const size_t lds = text_seg_lds(dm);
  auto go = [&](auto tag) {
    using T = decltype(tag);
    static std::atomic<uint32_t> lds_set{0};
    hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(&k_text_seg<T>), 96 * 1024, lds_set);
    if (e != hipSuccess) return e;
    hipExtLaunchKernelGGL(k_text_seg<T>, dim3(dm.B * dm.Hq), dim3(kSegThreads), lds, st, ev.start,
                          ev.stop, 0, static_cast<const T*>(c->Uk), static_cast<const T*>(c->Uv),
                          reinterpret_cast<const bf16_t*>(c->Usc), static_cast<const StoreB<T>*>(c->Bk),
                          static_cast<const StoreB<T>*>(c->Bv), q, c->out_part, c->ml_final, sel_out, dm.N,
                          dm.nblk, dm.NP, dm.r, dm.W, dm.d, dm.G, dm.Hq, r_lo, top_k, sl2);
    return hipGetLastError();
  };
  if (dm.storage == AP_INT4) return go(i4_t{});
  if (dm.storage == AP_BF16) return go(bf16_t{});
  return go(float{});
}

// ================================================================ k_ema_update
// Moving-average importance after a step ([fr §2.B "Score d'importance"]): the weight
// of visual token n for head h is p = exp2(s - M_h) / L_h, with s the step's logit
// (log2 units, written by k_attn) and (M_h, L_h) the softmax maximum and sum over
// text and visual tokens (written by k_combine).  Per head: I[b][h][n] <- a I + (1-a) p;
// per token: I[b][n] <- a I + (1-a) mean_h p (heads summed in a fixed order).  first:
// no history yet, I <- p.
// One thread per token; blockIdx.y is the state row (b * Hq + h per head, b per token), so
// the softmax statistics are uniform per workgroup.  Per token, the heads' logits are
// independent loads issued together, then summed in head order.
__global__ __launch_bounds__(256) void k_ema_update(const float* __restrict__ s,
                                                    const float* __restrict__ ml,
                                                    float* __restrict__ imp, int Hq, int N,
                                                    int rows, int per_head, int first,
                                                    float alpha) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  for (size_t row = blockIdx.y; row < (size_t)rows; row += gridDim.y) {
    float p;
    if (per_head) {
      p = exp2f(s[row * N + n] - ml[row * 2]) / ml[row * 2 + 1];
    } else {
      const float* sb = s + row * Hq * N + n;
      const float* mb = ml + row * Hq * 2;
      float acc = 0.f;
      int h = 0;
      for (; h + 8 <= Hq; h += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = sb[(size_t)(h + j) * N];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += exp2f(v[j] - mb[2 * (h + j)]) / mb[2 * (h + j) + 1];
      }
      for (; h < Hq; ++h) acc += exp2f(sb[(size_t)h * N] - mb[2 * h]) / mb[2 * h + 1];
      p = acc / static_cast<float>(Hq);
    }
    const size_t idx = row * N + n;
    imp[idx] = first ? p : fmaf(alpha, imp[idx], (1.f - alpha) * p);
  }
}

// Per-token state after a single-kernel step: part [B][G4][N] holds, per group of four
// query heads, the sum of their weights p; I[b][n] <- alpha I + (1 - alpha) mean_h p with
// the groups summed in order (I <- mean_h p on the first step).  One thread per token.
__global__ __launch_bounds__(256) void k_ema_fold(const float* __restrict__ part,
                                                  float* __restrict__ imp, int G4, int Hq, int N,
                                                  int first, float alpha) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const size_t b = blockIdx.y;
  const float* pb = part + b * G4 * N + n;
  float acc = 0.f;
  for (int g = 0; g < G4; ++g) acc += pb[(size_t)g * N];
  const float p = acc / static_cast<float>(Hq);
  const size_t idx = b * N + n;
  imp[idx] = first ? p : fmaf(alpha, imp[idx], (1.f - alpha) * p);
}

hipError_t launch_ema_fold(const ap_cache* c, const float* part, float* imp, bool first, float alpha,
                           hipStream_t st, const KernelEvents& ev) {
  const Dims& dm = c->dm;
  if (dm.B > 65535) return hipErrorInvalidValue;
  hipExtLaunchKernelGGL(k_ema_fold, dim3((unsigned)((dm.N + 255) / 256), (unsigned)dm.B), dim3(256), 0, st,
                        ev.start, ev.stop, 0, part, imp, (dm.Hq + 3) / 4, dm.Hq, dm.N, first ? 1 : 0, alpha);
  return hipGetLastError();
}

hipError_t launch_ema_update(const ap_cache* c, const float* s, const float* ml, float* imp,
                             bool per_head, bool first, float alpha, hipStream_t st,
                             const KernelEvents& ev) {
  const Dims& dm = c->dm;
  const int rows = dm.B * (per_head ? dm.Hq : 1);
  hipExtLaunchKernelGGL(k_ema_update, dim3((unsigned)((dm.N + 255) / 256), (unsigned)std::min(rows, 65535)),
                        dim3(256), 0, st, ev.start, ev.stop, 0, s, ml, imp, dm.Hq, dm.N, rows,
                        per_head ? 1 : 0, first ? 1 : 0, alpha);
  return hipGetLastError();
}

}  // namespace ap

// Per-head top-k selection of the tokens decompressed at full rank (gfx950).
//
// [fr §2.B "Stratégie"]: the most important tokens get the full rank R, the others a
// reduced rank; [es §4 "Análisis de Sensibilidad"]: 25% at full rank.  Importance of
// token n for query head h is its low-rank logit s_lo = U_k[n, :r_lo] . q~_h[:r_lo];
// the k largest are chosen, ties to the lower token index.
//
// One workgroup per (sequence, group of HG query heads), 16 wavefronts:
//  A. latent queries q~_h = B_k[:, head g's columns] q_h (on MFMA for bf16 rows with d a
//     multiple of 32 up to 128; also written out for the flash-decode kernel), with the
//     first U_k low-panel tiles already in flight;
//  B. low-rank scores of every token on MFMA.  The 16 output columns of a 16x16x32 tile
//     are (token block, tile half, head) triples: the latent-query operand of a column
//     is non-zero only in the k-slots of its own half and only for its own block, so
//     one accumulation yields the scores of 8/HG blocks x 32 tokens x HG heads and
//     every lane holds four scores of one head.  Scores stay in registers;
//  C. each head's scores are mapped by a monotone linear map over [min, max] onto
//     1024 bins; one LDS histogram locates the bin b* holding the k-th largest score;
//  D. tokens above b* are taken; inside b*, either all of it is taken, or its few
//     tokens are ranked exactly by (score desc, index asc), or - when b* is crowded
//     (ties, a zero query, an outlier stretching the range) - an MSB-first radix
//     select over the exact 32-bit keys finds the cutoff key and ties at it are
//     taken in index order;
//  E. the selection bits per (head, 32-token block) are written (and, on request, the
//     ascending selected ids).
#include <type_traits>

#include <hip/hip_ext.h>

#include "ap_internal.h"
#include "device_common.h"
#include "tiles.h"

namespace ap {

constexpr int kSelMaxWaves = 16;
constexpr int kSelBins = 1024;   // linear bins of the histogram pass
constexpr int kSelCap = 128;     // boundary-bin tokens ranked exactly by comparison

enum SelMode : int { kNone = 0, kAll = 1, kWholeBin = 2, kRank = 3, kRadix = 4 };

struct SelState {
  int bstar;       // boundary bin
  int need;        // tokens still to take inside the boundary bin (radix: ties at tau)
  int cnt;         // tokens in the boundary bin
  int mode;
  int ncand;       // kRank: candidates gathered
  uint32_t tau;    // kRadix: key of the last token taken
};

struct SelLayout {
  size_t qh, qb, qs, st, rng, hist, selw, cand;
  size_t sts, zs, hmx, lpart, ltx, lfin, red;   // single-kernel decode only
  size_t pst;      // single-kernel moving-average selector: [stash][1024 threads] weights
  size_t total;
  int hs;          // words per head in hist
};

// hist holds each head's bin counts; in the radix fallback it is reused as
// [256 digit counts][nblk tie bits][nblk tie prefix] per head, and in the single-kernel
// decode as the per-wavefront latent sums and then the output partial sums.
// Tn > 0 (text tokens) or fused adds the single-kernel decode regions.
__host__ __device__ inline SelLayout sel_layout(int HG, int nblk, int r_pad, int d, bool fused = false,
                                                int Tn = 0, int stash = 0) {
  auto up = [](size_t x) { return (x + 15) & ~(size_t)15; };
  SelLayout L;
  L.hs = kSelBins > 256 + 2 * nblk ? kSelBins : 256 + 2 * nblk;
  size_t o = 0;
  L.qh = o;   o = up(o + (size_t)(HG * d > 1024 ? HG * d : 1024) * 4);   // >= one float per thread
  L.qb = o;   o = up(o + (size_t)2 * HG * d * 2);                          // q as bf16 hi, then lo
  L.qs = o;   o = up(o + (size_t)HG * r_pad * 4);
  L.st = o;   o = up(o + (size_t)HG * sizeof(SelState));
  L.rng = o;  o = up(o + (size_t)HG * 2 * 4);
  L.hist = o; o = up(o + (size_t)HG * L.hs * 4);
  L.selw = o; o = up(o + (size_t)HG * nblk * 4);
  L.cand = o; o = up(o + (size_t)HG * kSelCap * 8);
  L.sts = L.zs = L.hmx = L.lpart = L.ltx = L.lfin = L.red = o;
  if (fused) {
    L.sts = o;   o = up(o + (size_t)HG * Tn * 4);
    L.zs = o;    o = up(o + (size_t)HG * r_pad * 4);
    L.hmx = o;   o = up(o + (size_t)HG * 4);
    L.lpart = o; o = up(o + (size_t)kSelMaxWaves * HG * 4);
    L.ltx = o;   o = up(o + (size_t)HG * 4);
    L.lfin = o;  o = up(o + (size_t)HG * 4);
    // the output partial sums [1024 threads][8 floats]
    L.red = o;   o = up(o + (size_t)1024 * 8 * 4);
    L.pst = o;   o = up(o + (size_t)stash * 1024 * 4);
  }
  L.total = o;
  return L;
}

// Workgroup barrier that orders LDS only: the workgroup's waves exchange data through
// LDS alone, so global loads still in flight (prefetched tiles and rows) are not
// waited for here, as a full __syncthreads() would.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inverse of score_key.
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int N>
__device__ __forceinline__ float dpp_ror_max(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, true)));
}
template <int N>
__device__ __forceinline__ float dpp_ror_min(float v) {
  return fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, true)));
}
// Maximum and minimum of floats over the lanes of a wavefront that hold the same head
// (lane%16 congruent mod HG), as head_max below.
template <int HG>
__device__ __forceinline__ float head_fmax(float v) {
  if constexpr (HG <= 1) v = dpp_ror_max<1>(v);
  if constexpr (HG <= 2) v = dpp_ror_max<2>(v);
  if constexpr (HG <= 4) v = dpp_ror_max<4>(v);
  if constexpr (HG <= 8) v = dpp_ror_max<8>(v);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
template <int HG>
__device__ __forceinline__ float head_fmin(float v) {
  if constexpr (HG <= 1) v = dpp_ror_min<1>(v);
  if constexpr (HG <= 2) v = dpp_ror_min<2>(v);
  if constexpr (HG <= 4) v = dpp_ror_min<4>(v);
  if constexpr (HG <= 8) v = dpp_ror_min<8>(v);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fminf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

template <int N>
__device__ __forceinline__ uint32_t dpp_ror(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x120 + N, 0xF, 0xF, true));
}

// Maximum over the lanes of a wavefront that hold the same head (lane%16 congruent
// mod HG): rotations by HG, 2HG, .. inside each 16-lane row, then across the 4 rows.
template <int HG>
__device__ __forceinline__ uint32_t head_max(uint32_t v) {
  if constexpr (HG <= 1) v = max(v, dpp_ror<1>(v));
  if constexpr (HG <= 2) v = max(v, dpp_ror<2>(v));
  if constexpr (HG <= 4) v = max(v, dpp_ror<4>(v));
  if constexpr (HG <= 8) v = max(v, dpp_ror<8>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(a[0], a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(c[0], c[1]);
}

// Inclusive prefix sum over the 64 lanes with DPP only: shifts by 1, 2, 4, 8 inside
// each 16-lane row (lanes shifted in from outside the row read 0), then lane 15 of each
// row added to the next row and lane 31 to the upper half.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROWS, 0xF, true));
}
// Sum over the lanes of one 16-lane row that hold the same head (lane%16 congruent mod
// HG), by rotations; every such lane gets the sum.
template <int N>
__device__ __forceinline__ float dpp_ror_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, true));
}
template <int HG>
__device__ __forceinline__ float head_sum_row(float v) {
  if constexpr (HG <= 1) v += dpp_ror_f<1>(v);
  if constexpr (HG <= 2) v += dpp_ror_f<2>(v);
  if constexpr (HG <= 4) v += dpp_ror_f<4>(v);
  if constexpr (HG <= 8) v += dpp_ror_f<8>(v);
  return v;
}
// The same over the whole wavefront (then across the 4 rows).
template <int HG>
__device__ __forceinline__ float head_sum(float v) {
  v = head_sum_row<HG>(v);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int) {
  v += dpp_u32<0x111, 0xF>(v);   // row_shr:1
  v += dpp_u32<0x112, 0xF>(v);   // row_shr:2
  v += dpp_u32<0x114, 0xF>(v);   // row_shr:4
  v += dpp_u32<0x118, 0xF>(v);   // row_shr:8
  v += dpp_u32<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_u32<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// Wavefront search over a 256-bin histogram (descending digit order): the digit D whose
// bin holds the need-th largest element, and how many elements lie in bins above D.
__device__ __forceinline__ bool digit_search(const uint32_t* hist, uint32_t need, int lane,
                                             int* digit, uint32_t* above, uint32_t* in_bin) {
  const uint4 c4 = *reinterpret_cast<const uint4*>(hist + 252 - 4 * lane);  // bins 252-4l..255-4l
  const uint32_t c0 = c4.w, c1 = c4.z, c2 = c4.y, c3 = c4.x;               // descending digits
  const uint32_t tot = c0 + c1 + c2 + c3;
  const uint32_t incl = wave_incl_scan(tot, lane);
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

// The same search over kSelBins bins, by a whole wavefront: lane l first sums the SPL
// bins [kSelBins-SPL(l+1), kSelBins-SPL*l); then the SPL bins of the slice holding the
// need-th element are scanned one per lane.  Every lane returns the result.
__device__ __forceinline__ void bin_search(const uint32_t* hist, uint32_t need, int lane,
                                           int* bin, uint32_t* above, uint32_t* in_bin) {
  constexpr int SPL = kSelBins / 64;
  static_assert(SPL % 4 == 0 && SPL <= 64, "whole 16-byte reads, one scan");
  const uint4* sl = reinterpret_cast<const uint4*>(hist + kSelBins - SPL * (lane + 1));
  uint32_t tot = 0;
#pragma unroll
  for (int v = 0; v < SPL / 4; ++v) {
    const uint4 x = sl[v];
    tot += x.x + x.y + x.z + x.w;
  }
  const uint32_t incl = wave_incl_scan(tot, lane);
  const uint32_t excl = incl - tot;
  const uint64_t hit = __ballot(excl < need && incl >= need);
  const int L = hit ? static_cast<int>(__ffsll(static_cast<unsigned long long>(hit))) - 1 : 63;
  const uint32_t base = __shfl(excl, L, 64);
  // bins of slice L in descending order, one per lane 0..SPL-1
  const uint32_t c = lane < SPL ? hist[kSelBins - SPL * L - 1 - lane] : 0u;
  const uint32_t ci = base + wave_incl_scan(c, lane);
  const uint64_t hit2 = __ballot(lane < SPL && ci >= need);
  const int e = hit2 ? static_cast<int>(__ffsll(static_cast<unsigned long long>(hit2))) - 1 : SPL - 1;
  *bin = kSelBins - SPL * L - 1 - e;
  *in_bin = __shfl(c, e, 64);
  *above = __shfl(ci, e, 64) - *in_bin;
}

// Scores of one accumulation step (one panel): NSL tiles of 32 tokens.  Column
// c = l%16 of the tile is (block slot c / 2HG, half (c / HG) % 2, head c % HG); its
// latent-query operand is this lane's 4 values placed in the k-slots of its half,
// and zero for every other slot.
template <int NSL>
__device__ __forceinline__ v4f score_step(const LaneTile<bf16_t> (&t)[NSL], uint4 bh, uint4 bl,
                                          int my_slot, int my_j, v4f acc) {
  (void)my_j;
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
    const bool on = sl == my_slot;
    const uint4 h = on ? bh : make_uint4(0u, 0u, 0u, 0u);
    const uint4 l = on ? bl : make_uint4(0u, 0u, 0u, 0u);
    const v8bf a = __builtin_bit_cast(v8bf, t[sl].raw);
    acc = mfma_bf16_k32(a, __builtin_bit_cast(v8bf, h), acc);
    acc = mfma_bf16_k32(a, __builtin_bit_cast(v8bf, l), acc);
  }
  return acc;
}
template <int NSL>
__device__ __forceinline__ v4f score_step(const LaneTile<float> (&t)[NSL], const float (&qv)[4],
                                          int my_slot, int my_j, v4f acc) {
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const bool on = sl == my_slot && hf == my_j;
      const float4 x = t[sl].half(hf);
      acc = mfma_f32(x.x, on ? qv[0] : 0.f, acc);
      acc = mfma_f32(x.y, on ? qv[1] : 0.f, acc);
      acc = mfma_f32(x.z, on ? qv[2] : 0.f, acc);
      acc = mfma_f32(x.w, on ? qv[3] : 0.f, acc);
    }
  }
  return acc;
}

// Latent-query operand of one panel for this lane (head my_h, columns 16p+4lg+e < r_lo).
template <class T> struct SelQ;
template <> struct SelQ<bf16_t> {
  uint4 h, l;
  __device__ __forceinline__ void set(const float v[4], int my_j) {
    QOp<bf16_t> qo;
    qo.set(v);
    const uint2 hh = __builtin_bit_cast(uint2, qo.hi), ll = __builtin_bit_cast(uint2, qo.lo);
    h = my_j == 0 ? make_uint4(hh.x, hh.y, 0u, 0u) : make_uint4(0u, 0u, hh.x, hh.y);
    l = my_j == 0 ? make_uint4(ll.x, ll.y, 0u, 0u) : make_uint4(0u, 0u, ll.x, ll.y);
  }
  template <int NSL>
  __device__ __forceinline__ v4f step(const LaneTile<bf16_t> (&t)[NSL], uint2, int my_slot, int my_j, v4f acc) const {
    return score_step<NSL>(t, h, l, my_slot, my_j, acc);
  }
};
template <> struct SelQ<float> {
  float v[4];
  __device__ __forceinline__ void set(const float x[4], int) {
    for (int e = 0; e < 4; ++e) v[e] = x[e];
  }
  template <int NSL>
  __device__ __forceinline__ v4f step(const LaneTile<float> (&t)[NSL], uint2, int my_slot, int my_j, v4f acc) const {
    return score_step<NSL>(t, v, my_slot, my_j, acc);
  }
};
// 4-bit codes: the block scales of this lane's own slot (scw, its 4 columns) are folded
// into the latent query before the hi/lo split; the codes enter as 136 + code and one
// more pair of products with -136 in every A element removes the offset (the operands
// of the other slots are zero in this lane, so one pair serves all slots).
template <> struct SelQ<i4_t> {
  float v[4];
  __device__ __forceinline__ void set(const float x[4], int) {
    for (int e = 0; e < 4; ++e) v[e] = x[e];
  }
  template <int NSL>
  __device__ __forceinline__ v4f step(const LaneTile<i4_t> (&t)[NSL], uint2 scw, int my_slot, int my_j, v4f acc) const {
    float s[4];
    q4_scales(scw, s);
    const float f[4] = {v[0] * s[0], v[1] * s[1], v[2] * s[2], v[3] * s[3]};
    SelQ<bf16_t> qb;
    qb.set(f, my_j);
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const bool on = sl == my_slot;
      const uint4 h = on ? qb.h : make_uint4(0u, 0u, 0u, 0u);
      const uint4 l = on ? qb.l : make_uint4(0u, 0u, 0u, 0u);
      const v8bf a = __builtin_bit_cast(v8bf, t[sl].deq());
      acc = mfma_bf16_k32(a, __builtin_bit_cast(v8bf, h), acc);
      acc = mfma_bf16_k32(a, __builtin_bit_cast(v8bf, l), acc);
    }
    const v8bf an = __builtin_bit_cast(v8bf, make_uint4(kQ4NegOffset2, kQ4NegOffset2, kQ4NegOffset2, kQ4NegOffset2));
    acc = mfma_bf16_k32(an, __builtin_bit_cast(v8bf, qb.h), acc);
    return mfma_bf16_k32(an, __builtin_bit_cast(v8bf, qb.l), acc);
  }
};

// Operands of the single-kernel decode (unused by the selection-only kernel).
struct FusedArgs {
  const void* Uv;       // V-layout panels
  const void* Bv;       // [B][r_pad][W]
  const void* text_k;   // [B][Tn][W] or null
  const void* text_v;
  float* out;           // [B][Hq][d]
  int Tn;
  float sl2;            // softmax scale in log2 units
  // selection-only kernel: rank by these keys (the moving-average importance) instead
  // of the low-rank logits; [B][Hq][N] when keys_per_head, else [B][N] shared by heads
  const float* keys;
  int keys_per_head;
  // 4-bit codes: bf16 block scales [B][nblk][2][r_pad] (quant4.h)
  const bf16_t* Usc;
  // single-kernel decode with the moving-average selector: it ranks by keys (the state;
  // null on a sequence's first step: by the low-rank logits), then per head blends the
  // step's attention weights into imp ([B][Hq][N]), or per token writes the sum of its
  // heads' weights to ema_part ([B][head groups][N]) for the fold that follows
  float* imp;
  float* ema_part;
  float alpha;
  int ema_first;
};

// HG: query heads per workgroup (4 or 1); NPL: low panels (1 or 2 with the tiles of
// several steps in flight; 8 = any count up to 8, one panel's tiles at a time); NACC:
// accumulation steps per wavefront (2, 3, 4 or 8).  FUSED: the same workgroup goes on
// to the attention of its heads over all tokens, the text tokens and the output
// projection (bf16 factors, HG = 4, r <= 64), so one kernel makes the whole step.
template <class T, int HG, int NPL, int NACC, bool FUSED, int NPX = 0, bool MQ = false, bool EMA = false>
__device__ __forceinline__ void select_body(
    const T* __restrict__ Uk, const StoreB<T>* __restrict__ Bk, const float* __restrict__ q,
    float* __restrict__ qt, uint32_t* __restrict__ mask, int32_t* __restrict__ sel_out, int B,
    int N, int nblk, int NP, int r_pad, int W, int d, int G, int Hq, int Hq_pad, int HGN,
    int r_lo, int top_k, const FusedArgs& fa) {
  constexpr bool U4 = std::is_same<T, i4_t>::value;
  static_assert(!FUSED || (HG == 4 && NPL <= 2 && (std::is_same<T, bf16_t>::value || (U4 && NPX > 0))),
                "single-kernel decode: bf16, or 4-bit codes with the panel split known at compile "
                "time, four heads per workgroup");
  using TB = StoreB<T>;   // element type of B (and of the text tokens)
  // NPX > 0 (single-kernel decode): the factors have NPX panels and r_lo = 16 * NPL, so
  // the panel loops of the attention phases are resolved at compile time
  const int NPr = NPX > 0 ? NPX : NP;
  const int rlo = NPX > 0 ? 16 * NPL : r_lo;
  constexpr int NSL = 8 / HG;                                   // token blocks per step
  constexpr int KPL = 4 * NACC;                                 // scores per lane
  constexpr int NSTEP = NACC * NPL;
  constexpr int TREG = static_cast<int>(sizeof(LaneTile<T>) / 4);
  constexpr int PBUD = (NACC <= 4 ? 64 : 32) / TREG / NSL;      // steps in flight (register budget)
  constexpr int PREF = PBUD < 1 ? 1 : (PBUD > NSTEP ? NSTEP : PBUD);
  extern __shared__ __align__(16) unsigned char smem_raw[];
  // All head groups of one sequence share blockIdx % 8 (one XCD), so its L2 serves
  // the repeated reads of U_k's low panels.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int b = (slot / HGN) * 8 + xcd;
  const int hg = slot % HGN;
  if (b >= B) return;
  const int h0 = hg * HG;
  const int nh = min(HG, Hq - h0);
  if (nh <= 0) return;
  const int nthr = blockDim.x, nwv = nthr >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: tile offsets in SGPRs
  const int c16 = lane & 15, lg = lane >> 4;
  const int my_slot = c16 / (2 * HG), my_j = (c16 / HG) & 1, my_h = c16 % HG;
  const bool my_on = my_h < nh;

  const SelLayout Ly = sel_layout(HG, nblk, r_pad, d, FUSED, FUSED ? fa.Tn : 0, FUSED && EMA ? 4 * NACC : 0);
  float* qh = reinterpret_cast<float*>(smem_raw + Ly.qh);
  bf16_t* qb = reinterpret_cast<bf16_t*>(smem_raw + Ly.qb);
  float* qs = reinterpret_cast<float*>(smem_raw + Ly.qs);
  SelState* st = reinterpret_cast<SelState*>(smem_raw + Ly.st);
  uint32_t* rng = reinterpret_cast<uint32_t*>(smem_raw + Ly.rng);
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem_raw + Ly.hist);
  uint32_t* selw = reinterpret_cast<uint32_t*>(smem_raw + Ly.selw);
  unsigned long long* cand = reinterpret_cast<unsigned long long*>(smem_raw + Ly.cand);
  const int HS = Ly.hs;

  const bool none = top_k <= 0, all = top_k >= N;
  const bool select = !none && !all;
  const int nplo = (r_lo + 15) >> 4;

  // ---- A. loads in flight together: q first, then the B_k rows the low-rank scores
  // need and the first U_k low-panel tiles; (bf16 rows on MFMA) the B_k rows of the
  // latent columns >= r_lo are requested once the low rows are in and used at the end
  // of the selection.  Rows read once are loaded non-temporally, so that they do not
  // push the token factors, which the head groups of a sequence share, out of L2.
  constexpr int V = Vec16<TB>::n;
  constexpr int XB = 4;    // B_k row slices per lane in flight
  const int ginv_num = (65536 + G - 1) / G;   // (h * ginv_num) >> 16 == h / G for h, G <= 64
  const int LPR = d / V;
  const bool vec = d % V == 0 && LPR > 0 && LPR <= 64 && (LPR & (LPR - 1)) == 0 &&
                   ((size_t)W * sizeof(TB)) % 16 == 0;
  const int nrows = nh * r_pad;
  const int RPW = vec ? 64 / LPR : 1, seg = vec ? lane % LPR : 0, rw = vec ? lane / LPR : 0;
  const int rstep = nwv * RPW;
  const float inv_rpad = 1.0f / static_cast<float>(r_pad);
  // head of a flattened (head, latent row) index without an integer division:
  // (row + 0.5) / r_pad is never within float rounding of an integer here
  auto head_of = [&](int row) { return static_cast<int>((static_cast<float>(row) + 0.5f) * inv_rpad); };
  Vec16<TB> x[XB];
  auto load_rows = [&](int r0) {
#pragma unroll
    for (int u = 0; u < XB; ++u) {
      const int row = min(r0 + u * rstep, nrows - 1);   // clamped: loads stay unconditional
      const int hl = head_of(row), i = row - hl * r_pad;
      x[u].load_nt(Bk + ((size_t)b * r_pad + i) * W + (size_t)(((h0 + hl) * ginv_num) >> 16) * d + seg * V);
    }
  };
  // bf16 rows with d a multiple of 32 (up to 128): latent queries and text scores on
  // MFMA.  A wavefront takes (head, 16-row tile) pairs; lane l loads the 8 elements of
  // row l%16 at d-offset 32 ks + 8 (l/16) of each 32-wide k step (its A operand) into
  // the same registers the other path uses, and q_h, split into bf16 hi + lo, is the only
  // non-zero column (0) of the B operand, so lanes 0, 16, 32, 48 end up holding the
  // tile's 16 dot products.
  // MQ: chosen at launch for bf16 rows with d a multiple of 32 up to 128
  constexpr bool kBfRows = MQ && std::is_same<TB, bf16_t>::value;
  constexpr bool mq = kBfRows;
  const int nks = d >> 5;
  const int qtiles = r_pad >> 4;                      // latent-row tiles per head
  const int npair_q = nh * qtiles;
  auto load_tile_rows = [&](Vec16<TB>(&dst)[XB], const TB* base, int row, int hl) {
    if constexpr (kBfRows) {
      const TB* src = base + (size_t)row * W + (size_t)(((h0 + hl) * ginv_num) >> 16) * d + 8 * lg;
#pragma unroll
      for (int ks = 0; ks < XB; ++ks)
        if (ks < nks) dst[ks].load_nt(src + 32 * ks);
    }
  };
  // the tile's dot products with q_h (this lane's A operands in a); q_h's bf16 hi and lo
  // halves come from LDS (qb), non-zero only in column 0 of the B operand
  auto tile_dot = [&](const Vec16<TB>(&a)[XB], int hl) {
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (kBfRows) {
      const uint32_t on = c16 == 0 ? ~0u : 0u;
#pragma unroll
      for (int ks = 0; ks < XB; ++ks) {
        if (ks < nks) {
          const int o = hl * d + 32 * ks + 8 * lg;
          const uint4 hw = *reinterpret_cast<const uint4*>(qb + o);
          const uint4 lw = *reinterpret_cast<const uint4*>(qb + HG * d + o);
          const v8bf av = __builtin_bit_cast(v8bf, a[ks].raw);
          acc = mfma_bf16_k32(av, __builtin_bit_cast(v8bf, make_uint4(hw.x & on, hw.y & on, hw.z & on, hw.w & on)), acc);
          acc = mfma_bf16_k32(av, __builtin_bit_cast(v8bf, make_uint4(lw.x & on, lw.y & on, lw.z & on, lw.w & on)), acc);
        }
      }
    }
    return acc;
  };
  // (head, latent-row tile) pairs whose rows lie below r_lo: needed by the low-rank scores
  auto lo_pair = [&](int pair) { return 16 * (pair - (pair / qtiles) * qtiles) < rlo; };
  // More pairs than wavefronts (8 wavefronts, four heads): the pairs are dealt from a
  // list holding every pair below r_lo first, wavefront w taking items w, w + nwv, ...
  // Each wavefront's first item is requested at the start; its items below r_lo and its
  // first item are done before the scores, and only then is its next item requested,
  // so that those rows arrive during the selection.  No wavefront then waits for a
  // second load before the scores or at the end.
  const bool spread = !FUSED && mq && npair_q > nwv;   // (the single kernel runs 16 wavefronts)
  const int nlo_t = min((rlo + 15) >> 4, qtiles);
  const int nlo_p = nh * nlo_t, nhi_t = max(qtiles - nlo_t, 1);
  auto pair_at = [&](int idx) {
    if (idx < nlo_p) {
      const int hl = idx / nlo_t;
      return hl * qtiles + (idx - hl * nlo_t);
    }
    const int j = idx - nlo_p, hl = j / nhi_t;
    return hl * qtiles + nlo_t + (j - hl * nhi_t);
  };
  auto load_pair = [&](int pr) {
    const int hl = pr / qtiles, it = pr - hl * qtiles;
    load_tile_rows(x, Bk + (size_t)b * r_pad * W, 16 * it + c16, hl);
  };
  auto dot_pair = [&](int pr) {
    const int hl = pr / qtiles, it = pr - hl * qtiles;
    const v4f acc = tile_dot(x, hl);
    if (c16 == 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) qs[hl * r_pad + 16 * it + 4 * lg + t] = acc[t];
    }
  };
  // one q value per thread (HG * d <= threads, checked at launch); stored unconditionally so the
  // load is never sunk behind the tile loads
  const int nq = nh * d;
  const float qv = q[((size_t)b * Hq + h0) * d + min(tid, nq - 1)];
  if (mq) {
    if (spread) {
      load_pair(pair_at(wave));
    } else if (wave < npair_q && lo_pair(wave)) {
      const int hl = wave / qtiles, it = wave - hl * qtiles;
      load_tile_rows(x, Bk + (size_t)b * r_pad * W, 16 * it + c16, hl);
    }
  } else if (vec) {
    load_rows(wave * RPW + rw);
  }
  // single-kernel decode: the first text K rows ride along (text scores need only q)
  const int Tn = FUSED ? fa.Tn : 0;
  const int nrt = nh * Tn;                   // text rows (head, token)
  // with no text the loads read B_k instead (always valid), so they stay unconditional
  const TB* __restrict__ tk = Tn > 0 ? static_cast<const TB*>(fa.text_k) : Bk;
  Vec16<TB> xt[XB];
  auto load_text = [&](int r0) {
#pragma unroll
    for (int u = 0; u < XB; ++u) {
      const int row = max(min(r0 + u * rstep, nrt - 1), 0);
      const int hl = row / max(Tn, 1), t = row - hl * Tn;
      xt[u].load_nt(tk + ((size_t)b * Tn + t) * W + (size_t)(((h0 + hl) * ginv_num) >> 16) * d + seg * V);
    }
  };

  LaneTile<T> tb[PREF][NSL];
  [[maybe_unused]] uint2 tsc[PREF];   // 4-bit codes: K scales of this lane's slot and columns
  // 4-bit codes: K (or V) scale word of block blk, panel p, for this lane's columns
  // 16p + 4lg + e
  auto scale_word = [&](int blk, int p, bool vrow = false) {
    const bf16_t* row = fa.Usc + (((size_t)b * nblk + blk) * 2 + (vrow ? 1 : 0)) * r_pad + lg * 4 * NP + 4 * p;
    return *reinterpret_cast<const uint2*>(row);
  };
  auto load_step = [&](int s) {   // s is a compile-time constant after unrolling
    const int a = s / NPL, p = s % NPL;
    const int grp = wave + nwv * a;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const int blk = min(grp * NSL + sl, nblk - 1);   // clamped: loads stay unconditional
      tb[s % PREF][sl].load(tile_ptr(Uk, tile_base(b, min(p, nplo - 1), blk, NP, nblk)), lane);
    }
    if constexpr (U4) tsc[s % PREF] = scale_word(min(grp * NSL + my_slot, nblk - 1), min(p, nplo - 1));
  };
  if constexpr (NPL <= 2) {
#pragma unroll
    for (int s = 0; s < PREF; ++s) load_step(s);
  }
  qh[tid] = qv;
  if (tid < HG * d) {
    const bf16_t hi = f32_to_bf16(qv);
    qb[tid] = hi;
    qb[HG * d + tid] = f32_to_bf16(qv - bf16_to_f32(hi));
  }
  for (int i = tid; i < nh * HS; i += nthr) hist[i] = 0;
  for (int i = tid; i < nh * nblk; i += nthr) selw[i] = 0;
  if (tid < nh) {
    st[tid].mode = none ? kNone : (all ? kAll : kWholeBin);
    st[tid].ncand = 0;
    rng[2 * tid] = 0u;
    rng[2 * tid + 1] = 0u;
    if constexpr (FUSED) {
      reinterpret_cast<uint32_t*>(smem_raw + Ly.hmx)[tid] = 0u;
      reinterpret_cast<float*>(smem_raw + Ly.ltx)[tid] = 0.f;
    }
  }
  lds_barrier();
  // latent queries q~[h][i] = B_k[i, g*d : g*d+d] . q_h (on MFMA: the rows below r_lo
  // now, the others at the end of the selection)
  bool x_first = true;   // x still holds the rows of this wavefront's first pair
  auto latent_pairs = [&](bool low) {
    for (int pair = wave; pair < npair_q; pair += nwv) {
      if (lo_pair(pair) != low) continue;
      const int hl = pair / qtiles, it = pair - hl * qtiles;
      if (pair != wave || !x_first) {
        load_tile_rows(x, Bk + (size_t)b * r_pad * W, 16 * it + c16, hl);
        x_first = false;
      }
      const v4f acc = tile_dot(x, hl);
      if (c16 == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) qs[hl * r_pad + 16 * it + 4 * lg + t] = acc[t];
      }
    }
  };
  int next_item = npair_q;   // spread: this wavefront's first item not yet done
  if (spread) {
    int idx = wave;
    for (; idx < npair_q; idx += nwv) {
      const int pr = pair_at(idx);
      if (idx != wave && !lo_pair(pr)) break;
      if (idx != wave) load_pair(pr);
      dot_pair(pr);
    }
    next_item = idx;
    if (next_item < npair_q) load_pair(pair_at(next_item));
  } else if (mq) {
    latent_pairs(true);
    // the B_k rows of the latent columns >= r_lo: requested only now, so that they do not
    // hold up q and the low rows in the memory system at the start
    if (wave < npair_q && !lo_pair(wave)) {
      const int hl = wave / qtiles, it = wave - hl * qtiles;
      load_tile_rows(x, Bk + (size_t)b * r_pad * W, 16 * it + c16, hl);
      x_first = true;
    }
  } else if (vec) {
    for (int r0 = wave * RPW + rw; r0 - rw < nrows; r0 += XB * rstep) {
      if (r0 != wave * RPW + rw) load_rows(r0);
#pragma unroll
      for (int u = 0; u < XB; ++u) {
        const int row = r0 + u * rstep;
        float part = 0.f;
        if (row < nrows) {
          const float* qp = qh + head_of(row) * d + seg * V;
#pragma unroll
          for (int e = 0; e < V; ++e) part = fmaf(x[u].get(e), qp[e], part);
        }
        part = group_sum(part, LPR);
        if (seg == 0 && row < nrows) qs[row] = part;   // row = hl * r_pad + i
      }
    }
  } else {
    for (int idx = tid; idx < nrows; idx += nthr) {
      const int hl = idx / r_pad, i = idx - hl * r_pad;
      const TB* brow = Bk + ((size_t)b * r_pad + i) * W + (size_t)((h0 + hl) / G) * d;
      const float* qp = qh + hl * d;
      float acc = 0.f;
      for (int j = 0; j < d; ++j) acc = fmaf(to_f32(brow[j]), qp[j], acc);
      qs[hl * r_pad + i] = acc;
    }
  }
  lds_barrier();
  // single-kernel decode: the text K rows are requested now, behind B_k, and scored
  // after the selection
  const int ttiles = max((Tn + 15) >> 4, 1);          // 16-token tiles per head
  const int npair_t = Tn > 0 ? nh * ttiles : 0;
  auto load_text_tile = [&](int pair) {
    const int hl = pair / ttiles, it = pair - hl * ttiles;
    load_tile_rows(xt, tk + (size_t)b * Tn * W, min(16 * it + c16, Tn - 1), hl);
  };
  if constexpr (FUSED) {
    if (mq) {
      if (wave < npair_t) load_text_tile(wave);
    } else {
      load_text(wave * RPW + rw);
    }
  }

  // single-kernel decode: tiles of the full-rank score pass (U_k panels holding columns
  // >= r_lo) and then of the value pass (all U_v panels), 2 tiles per step, PD steps in
  // flight; the first ones are issued right after the low-rank scores
  constexpr int NPM = 4;                        // panels (r <= 64)
  constexpr int NSK = NACC * NPM;               // steps of each pass
  constexpr int PD = NACC <= 4 ? 4 : 2;
  const int p0 = rlo >> 4;                      // first panel with a column >= r_lo
  LaneTile<T> rb[FUSED ? PD : 1][NSL];
  // 4-bit codes: the K (full-rank pass) or V (value pass) scales of the block in this
  // lane's slot, for the lane's columns of the step's panel
  [[maybe_unused]] uint2 rsc[FUSED && U4 ? PD : 1];
  auto ld = [&](int s) {   // s is a compile-time constant after unrolling
    const bool isv = s >= NSK;
    const int ss = isv ? s - NSK : s;
    const int a = ss / NPM, j = ss % NPM;
    const int grp = wave + nwv * a;
    const int pan = isv ? min(j, NPr - 1) : min(p0 + j, NPr - 1);
    const T* base = isv ? static_cast<const T*>(fa.Uv) : Uk;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const int blk = min(grp * NSL + sl, nblk - 1);   // clamped: loads stay unconditional
      rb[s % PD][sl].load(tile_ptr(base, tile_base(b, pan, blk, NP, nblk)), lane);
    }
    if constexpr (FUSED && U4) rsc[s % PD] = scale_word(min(grp * NSL + my_slot, nblk - 1), pan, isv);
  };

  // ---- B. scores of this lane's tokens (head my_h), kept in registers
  float sc[KPL];
  // token of score 4a+t: 32 * (block of step a) + 16 * my_j + 4 * lg + t
  auto tok = [&](int a) { return 32 * ((wave + nwv * a) * NSL + my_slot) + 16 * my_j + 4 * lg; };

  if (!FUSED && fa.keys != nullptr) {
    // moving-average selector: the keys are the importance state, read from memory
    if (select) {
      const size_t kb = fa.keys_per_head ? ((size_t)b * Hq + h0 + (my_on ? my_h : 0)) * N : (size_t)b * N;
#pragma unroll
      for (int a = 0; a < NACC; ++a) {
        const int n0 = tok(a);
#pragma unroll
        for (int t = 0; t < 4; ++t) sc[4 * a + t] = (my_on && n0 + t < N) ? fa.keys[kb + n0 + t] : 0.f;
      }
    }
  } else if (select || FUSED) {
    constexpr int NQ = NPL <= 2 ? NPL : 1;
    SelQ<T> qop[NQ];
#pragma unroll
    for (int p = 0; p < NQ; ++p) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = 16 * p + 4 * lg + e;
        v[e] = (my_on && col < r_lo) ? qs[my_h * r_pad + col] : 0.f;
      }
      qop[p].set(v, my_j);
    }
    if constexpr (NPL <= 2) {
#pragma unroll
      for (int a = 0; a < NACC; ++a) {
        v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NPL; ++p) {
          const int s = a * NPL + p;
          acc = qop[p].template step<NSL>(tb[s % PREF], U4 ? tsc[s % PREF] : make_uint2(0u, 0u), my_slot, my_j, acc);
          if (s + PREF < NSTEP) load_step(s + PREF);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) sc[4 * a + t] = acc[t];
      }
    } else {
      // many low panels: one panel's tiles at a time, the latent-query operand rebuilt
      // from LDS per panel
#pragma unroll
      for (int a = 0; a < NACC; ++a) {
        v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
        const int grp = wave + nwv * a;
        for (int p = 0; p < nplo; ++p) {
          LaneTile<T> t1[NSL];
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl)
            t1[sl].load(tile_ptr(Uk, tile_base(b, p, min(grp * NSL + sl, nblk - 1), NP, nblk)), lane);
          const uint2 scw = U4 ? scale_word(min(grp * NSL + my_slot, nblk - 1), p) : make_uint2(0u, 0u);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int col = 16 * p + 4 * lg + e;
            v[e] = (my_on && col < r_lo) ? qs[my_h * r_pad + col] : 0.f;
          }
          SelQ<T> q1;
          q1.set(v, my_j);
          acc = q1.template step<NSL>(t1, scw, my_slot, my_j, acc);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) sc[4 * a + t] = acc[t];
      }
    }
  }

  // single-kernel decode with the moving-average selector: the selection ranks this
  // lane's tokens by the state, requested once the score tiles are consumed (earlier,
  // its registers would be live beside the tile prefetch); the logits wait in the
  // lane's own LDS slots
  if constexpr (FUSED && EMA) {
    if (fa.keys != nullptr) {
      const size_t kb = fa.keys_per_head ? ((size_t)b * Hq + h0 + (my_on ? my_h : 0)) * N : (size_t)b * N;
      float* pst = reinterpret_cast<float*>(smem_raw + Ly.pst);
#pragma unroll
      for (int i = 0; i < KPL; ++i) pst[i * nthr + tid] = sc[i];
#pragma unroll
      for (int a = 0; a < NACC; ++a) {
        const int n0 = tok(a);
#pragma unroll
        for (int t = 0; t < 4; ++t) sc[4 * a + t] = (my_on && n0 + t < N) ? fa.keys[kb + n0 + t] : 0.f;
      }
    }
  }
  // bit 4a+t: score of a real token of a present head
  uint32_t vm = 0u;
#pragma unroll
  for (int a = 0; a < NACC; ++a) {
    const int nv = min(max(N - tok(a), 0), 4);
    vm |= (my_on ? (1u << nv) - 1u : 0u) << (4 * a);
  }

  if (select) {
    // every score of this wavefront is a real token of a present head (wave-uniform):
    // the range, histogram and mark loops then run without per-score validity tests
    const uint32_t vfull = KPL >= 32 ? 0xFFFFFFFFu : ((1u << (KPL & 31)) - 1u);
    const bool all_ok = __ballot(vm != vfull) == 0ull;
    // ---- C. per-head range, linear bins, histogram, boundary bin
    {
      // range on the float scores (fmax / fmin ignore NaN), one conversion to keys per
      // lane; absent scores replaced by -inf / +inf
      float fmx = -INFINITY, fmn = INFINITY;
      if (all_ok) {
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          fmx = fmaxf(fmx, sc[i]);
          fmn = fminf(fmn, sc[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          const bool ok = (vm >> i) & 1u;
          fmx = fmaxf(fmx, ok ? sc[i] : -INFINITY);
          fmn = fminf(fmn, ok ? sc[i] : INFINITY);
        }
      }
      fmx = head_fmax<HG>(fmx);
      fmn = head_fmin<HG>(fmn);
      const uint32_t kmax = fmx == -INFINITY ? 0u : score_key(fmx);
      const uint32_t kmin = fmn == INFINITY ? 0u : ~score_key(fmn);   // kmin holds ~key
      if (lg == 0 && c16 < HG && my_on) {
        atomicMax(&rng[2 * my_h], kmax);
        atomicMax(&rng[2 * my_h + 1], kmin);
      }
    }
    lds_barrier();
    // bin(s) = min(kSelBins - 1, (s - lo) * mul): every lane derives its head's lo and
    // mul from the range words itself (the same arithmetic in every lane of a head)
    float lo_h = 0.f, mul_h = 0.f;
    if (my_on) {
      const float hi = key_score(rng[2 * my_h]);
      lo_h = key_score(~rng[2 * my_h + 1]);
      const float range = hi - lo_h;
      mul_h = (range > 1e-30f && range < 3.0e38f) ? static_cast<float>(kSelBins - 1) / range : 0.f;
    }
    // bin(s) = s * mul - lo * mul, clamped in float first (one fma and one med3): a
    // monotone map, and any input (NaN included: bin 0) gives a bin in [0, kSelBins)
    const float off_h = -lo_h * mul_h;
    auto bin_of = [&](float s) {
      return static_cast<uint32_t>(__builtin_amdgcn_fmed3f(fmaf(s, mul_h, off_h), 0.f, static_cast<float>(kSelBins - 1)));
    };
    {
      // branch-free: tokens past N (and absent heads) add 0, so the LDS atomics issue
      // back to back; any float maps to a bin inside the head's range
      uint32_t* hh = hist + my_h * HS;
      if (all_ok) {
#pragma unroll
        for (int i = 0; i < KPL; ++i) atomicAdd(&hh[bin_of(sc[i])], 1u);
      } else {
#pragma unroll
        for (int i = 0; i < KPL; ++i) atomicAdd(&hh[bin_of(sc[i])], (vm >> i) & 1u);
      }
    }
    lds_barrier();
    if (wave < nh) {
      int bn; uint32_t above, inb;
      bin_search(hist + wave * HS, static_cast<uint32_t>(top_k), lane, &bn, &above, &inb);
      if (lane == 0) {
        const int need = top_k - static_cast<int>(above);
        st[wave].bstar = bn;
        st[wave].need = need;
        st[wave].cnt = static_cast<int>(inb);
        st[wave].mode = need == static_cast<int>(inb) ? kWholeBin
                        : (inb <= static_cast<uint32_t>(kSelCap) ? kRank : kRadix);
      }
    }
    lds_barrier();

    // ---- D. tokens above the boundary bin (and all of it when it is taken whole);
    // candidates of a partly taken bin
    bool any_rank = false, any_radix = false;
    for (int hl = 0; hl < nh; ++hl) {
      any_rank |= st[hl].mode == kRank;
      any_radix |= st[hl].mode == kRadix;
    }
    const int bstar_h = my_on ? st[my_h].bstar : 0;
    const int mode_h = my_on ? st[my_h].mode : kNone;
    {
      // Bins compared through x = fma(s, mul, off), the value bin_of clamps and
      // truncates: for an integer B in [1, kSelBins - 1], bin_of(s) >= B exactly when
      // x >= B (NaN: bin 0, and x >= B is false).  B <= 0 takes every score; B >=
      // kSelBins none (a NaN threshold compares false).
      const int bwhole = mode_h == kWholeBin ? bstar_h : bstar_h + 1;   // lowest bin taken whole
      const bool take_all = bwhole <= 0;
      const float fwhole = bwhole >= kSelBins ? __builtin_nanf("") : static_cast<float>(bwhole);
      // a partly taken boundary bin (mode kRank, bwhole = bstar + 1): bin(s) == bstar
      // exactly when s is not taken and (bstar == 0 or x >= bstar)
      const bool rank_h = mode_h == kRank;
      const bool b0 = bstar_h == 0;
      const float fbstar = static_cast<float>(bstar_h);
      uint32_t cbits = 0;   // scores in a partly taken boundary bin (bit 4a+t)
      // Per step, the four scores' decisions are gathered as nibbles: tn (taken), cn (in
      // the boundary bin, for the exact ranking); the per-head cases (every score taken,
      // boundary bin 0) and the validity of each score are applied once per nibble, and
      // validity only where the wavefront holds absent scores (ALLOK: none).
      auto mark = [&](auto RANK, auto ALLOK) {
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
          const int n0 = tok(a);
          uint32_t tn = 0, cn = 0;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float x = fmaf(sc[4 * a + t], mul_h, off_h);
            tn |= x >= fwhole ? (1u << t) : 0u;
            if constexpr (decltype(RANK)::value) cn |= x >= fbstar ? (1u << t) : 0u;
          }
          tn = take_all ? 0xFu : tn;
          if constexpr (!decltype(ALLOK)::value) tn &= (vm >> (4 * a)) & 0xFu;
          if constexpr (decltype(RANK)::value) {
            cn = (b0 ? 0xFu : cn) & ~tn;
            if constexpr (!decltype(ALLOK)::value) cn &= (vm >> (4 * a)) & 0xFu;
            cbits |= cn << (4 * a);
          }
          const uint32_t nib = tn;
          // The eight lanes holding the tokens of one (head, block) word are the two tile
          // halves (lane%16 apart by HG) in each of the four 16-lane rows: OR them together
          // (a rotation by HG inside the row leaves the pair in the upper half's lane, then
          // the row swaps), and the upper half's lane of row 0 stores the word.
          uint32_t wv = nib << (n0 & 31);
          wv |= dpp_ror<HG>(wv);
          const auto r1 = __builtin_amdgcn_permlane16_swap(wv, wv, false, false);
          wv = r1[0] | r1[1];
          const auto r2 = __builtin_amdgcn_permlane32_swap(wv, wv, false, false);
          wv = r2[0] | r2[1];
          const int blk = n0 >> 5;
          if (my_j == 1 && lg == 0 && my_on && blk < nblk) selw[my_h * nblk + blk] = wv;
        }
      };
      if (all_ok) {
        if (any_rank) mark(std::true_type{}, std::true_type{});
        else mark(std::false_type{}, std::true_type{});
      } else {
        if (any_rank) mark(std::true_type{}, std::false_type{});
        else mark(std::false_type{}, std::false_type{});
      }
      if (!rank_h) cbits = 0u;
      if (cbits) {
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if ((cbits >> (4 * a + t)) & 1u) {
              const int n = tok(a) + t;
              const unsigned long long comp =
                  (static_cast<unsigned long long>(score_key(sc[4 * a + t])) << 32) |
                  static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(n));
              const int pos = atomicAdd(&st[my_h].ncand, 1);
              if (pos < kSelCap) cand[my_h * kSelCap + pos] = comp;
            }
          }
        }
      }
    }
    if (any_rank) {
      lds_barrier();
      if (wave < nh && st[wave].mode == kRank) {
        const int C = min(st[wave].ncand, kSelCap);
        const unsigned long long* ch = cand + wave * kSelCap;
        for (int c = lane; c < C; c += 64) {
          const unsigned long long me = ch[c];
          int rank = 0;
          for (int o = 0; o < C; ++o) rank += ch[o] > me ? 1 : 0;
          if (rank < st[wave].need) {
            const uint32_t n = 0xFFFFFFFFu - static_cast<uint32_t>(me & 0xFFFFFFFFull);
            atomicOr(&selw[wave * nblk + (n >> 5)], 1u << (n & 31));
          }
        }
      }
    }
    if (any_radix) {
      // Exact MSB-first radix select over the 32-bit keys of the boundary-bin tokens of
      // every head in this mode, then ties at the cutoff key taken in index order.
      uint32_t* rh = hist + my_h * HS;                 // this lane's head: digit counts
      const bool in_radix = mode_h == kRadix;
      lds_barrier();
      for (int i = tid; i < nh * HS; i += nthr) hist[i] = 0;
      if (tid < nh) st[tid].tau = 0u;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        const uint32_t pmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
        lds_barrier();
        if (pass > 0)
          for (int i = tid; i < nh * 256; i += nthr) hist[(i >> 8) * HS + (i & 255)] = 0;
        lds_barrier();
        if (in_radix) {
          const uint32_t prefix = st[my_h].tau;
#pragma unroll
          for (int a = 0; a < NACC; ++a) {
            const int n0 = tok(a);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              if (n0 + t < N && static_cast<int>(bin_of(sc[4 * a + t])) == bstar_h) {
                const uint32_t key = score_key(sc[4 * a + t]);
                if ((key & pmask) == prefix) atomicAdd(&rh[(key >> shift) & 255u], 1u);
              }
            }
          }
        }
        lds_barrier();
        if (wave < nh && st[wave].mode == kRadix) {
          int dg; uint32_t above, inb;
          if (digit_search(hist + wave * HS, static_cast<uint32_t>(st[wave].need), lane, &dg, &above, &inb)) {
            st[wave].tau |= static_cast<uint32_t>(dg) << shift;
            st[wave].need -= static_cast<int>(above);
          }
        }
      }
      lds_barrier();
      // tie bits per block, then their exclusive prefix counts in index order
      uint32_t* tie = hist + my_h * HS + 256;
      const uint32_t tau_h = in_radix ? st[my_h].tau : 0u;
      if (in_radix) {
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
          const int n0 = tok(a);
          uint32_t nib = 0;
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (n0 + t < N && static_cast<int>(bin_of(sc[4 * a + t])) == bstar_h &&
                score_key(sc[4 * a + t]) == tau_h)
              nib |= 1u << t;
          if (nib) atomicOr(&tie[n0 >> 5], nib << (n0 & 31));
        }
      }
      lds_barrier();
      if (wave < nh && st[wave].mode == kRadix) {
        const uint32_t* tw = hist + wave * HS + 256;
        uint32_t* tp = hist + wave * HS + 256 + nblk;
        uint32_t carry = 0;
        for (int c0 = 0; c0 < nblk; c0 += 64) {
          const int blk = c0 + lane;
          const uint32_t cnt = blk < nblk ? static_cast<uint32_t>(__popc(tw[blk])) : 0u;
          const uint32_t incl = wave_incl_scan(cnt, lane);
          if (blk < nblk) tp[blk] = carry + incl - cnt;
          carry += __shfl(incl, 63, 64);
        }
      }
      lds_barrier();
      if (in_radix) {
        const uint32_t* tp = hist + my_h * HS + 256 + nblk;
        const uint32_t need_t = static_cast<uint32_t>(st[my_h].need);
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
          const int n0 = tok(a);
          uint32_t nib = 0;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int n = n0 + t;
            if (n < N && static_cast<int>(bin_of(sc[4 * a + t])) == bstar_h) {
              const uint32_t key = score_key(sc[4 * a + t]);
              bool take = key > tau_h;
              if (key == tau_h) {
                const uint32_t w = tie[n >> 5];
                const uint32_t pos = tp[n >> 5] + static_cast<uint32_t>(__popc(w & ((1u << (n & 31)) - 1u)));
                take = pos < need_t;
              }
              if (take) nib |= 1u << t;
            }
          }
          if (nib) atomicOr(&selw[my_h * nblk + (n0 >> 5)], nib << (n0 & 31));
        }
      }
    }
  }
  // the remaining latent queries: their B_k rows arrived during the selection
  if (spread) {
    for (int idx = next_item; idx < npair_q; idx += nwv) {
      const int pr = pair_at(idx);
      if (idx != next_item) load_pair(pr);
      dot_pair(pr);
    }
  } else if (mq) {
    latent_pairs(false);
  }
  lds_barrier();

  // ---- E. selection bits per (head, 32-token block)
  auto word_of = [&](int hl, int blk) -> uint32_t {
    const int mode = st[hl].mode;
    if (mode == kNone) return 0u;
    if (mode == kAll) {
      const int nvalid = min(kBlockTok, N - blk * kBlockTok);
      return nvalid >= 32 ? 0xFFFFFFFFu : ((1u << nvalid) - 1u);
    }
    return selw[hl * nblk + blk];
  };
  if constexpr (!FUSED) {
    for (int idx = tid; idx < nh * nblk; idx += nthr) {
      const int blk = idx / nh, hl = idx - blk * nh;
      mask[((size_t)b * nblk + blk) * Hq_pad + h0 + hl] = word_of(hl, blk);
    }
  }
  if (sel_out != nullptr) {
    // ascending ids: one wavefront per head, block counts prefix-summed in order
    for (int hl = wave; hl < nh; hl += nwv) {
      int32_t* out = sel_out + ((size_t)b * Hq + h0 + hl) * top_k;
      uint32_t carry = 0;
      for (int c0 = 0; c0 < nblk; c0 += 64) {
        const int blk = c0 + lane;
        uint32_t w = blk < nblk ? word_of(hl, blk) : 0u;
        const uint32_t cnt = static_cast<uint32_t>(__popc(w));
        const uint32_t incl = wave_incl_scan(cnt, lane);
        uint32_t pos = carry + incl - cnt;
        while (w) {
          const int bit = __ffs(w) - 1;
          w &= w - 1u;
          if (pos < static_cast<uint32_t>(top_k)) out[pos] = blk * kBlockTok + bit;
          ++pos;
        }
        carry += __shfl(incl, 63, 64);
      }
    }
  }
  if constexpr (!FUSED) {
    // latent queries for the flash-decode kernel (stored last: stores share the load counter)
    for (int i = tid; i < nh * r_pad; i += nthr)
      qt[((size_t)b * Hq_pad + h0) * r_pad + i] = qs[i];
  } else {
    // ================= single-kernel decode of heads h0..h0+nh-1 over every token
    const T* __restrict__ Uv = static_cast<const T*>(fa.Uv);
    const TB* __restrict__ Bv = static_cast<const TB*>(fa.Bv);
    const TB* __restrict__ tv = static_cast<const TB*>(fa.text_v);
    const float sl2 = fa.sl2;
    (void)Uv;
    float* sts = reinterpret_cast<float*>(smem_raw + Ly.sts);      // [HG][Tn] text scores, then p
    float* zs = reinterpret_cast<float*>(smem_raw + Ly.zs);        // [HG][r_pad] latent sums
    uint32_t* hmx = reinterpret_cast<uint32_t*>(smem_raw + Ly.hmx);  // [HG] max score key
    float* lpart = reinterpret_cast<float*>(smem_raw + Ly.lpart);  // [waves][HG]
    float* ltx = reinterpret_cast<float*>(smem_raw + Ly.ltx);      // [HG] text sums
    float* lfin = reinterpret_cast<float*>(smem_raw + Ly.lfin);    // [HG] softmax denominators
    float* zpart = reinterpret_cast<float*>(hist);                 // [waves][HG][r_pad]
    float* red = reinterpret_cast<float*>(smem_raw + Ly.red);      // [row groups][HG * d]
    if constexpr (EMA) {
      if (fa.keys != nullptr) {   // the logits back in sc
        const float* pst = reinterpret_cast<const float*>(smem_raw + Ly.pst);
#pragma unroll
        for (int i = 0; i < KPL; ++i) sc[i] = pst[i * nthr + tid];
      }
    }

    // ---- F1. text scores in log2 units, running max per head: on MFMA, one (head,
    // 16-token tile) pair per wavefront, or LPR lanes per text row; the first pair or
    // XB * rstep rows come from the loads issued after the latent queries, any further
    // ones are loaded here
    auto text_scores = [&](int r0) {
#pragma unroll
      for (int u = 0; u < XB; ++u) {
        const int row = r0 + u * rstep;
        const int hl = max(min(row, nrt - 1), 0) / max(Tn, 1);
        const float* qp = qh + hl * d + seg * V;
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < V; ++e) part = fmaf(xt[u].get(e), qp[e], part);
        part = group_sum(part, LPR);
        if (seg == 0 && row < nrt) {
          const float sv = part * fa.sl2;
          sts[row] = sv;
          atomicMax(&hmx[hl], score_key(sv));
        }
      }
    };
    // at most one (head, tile) pair per wavefront (its rows already in xt): the first
    // tiles of the full-rank score pass are requested before the text scores, whose
    // products then overlap their latency; with more pairs (text rows loaded here) they
    // are requested after them
    const bool one_pair = mq && npair_t <= nwv;
    if (one_pair) {
#pragma unroll
      for (int s = 0; s < PD; ++s) ld(s);
    }
    auto text_pair = [&](int pair) {
      const int hl = pair / ttiles, it = pair - hl * ttiles;
      const v4f acc = tile_dot(xt, hl);
      if (c16 == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int tok = 16 * it + 4 * lg + t;
          if (tok < Tn) {
            const float sv = acc[t] * fa.sl2;
            sts[hl * Tn + tok] = sv;
            atomicMax(&hmx[hl], score_key(sv));
          }
        }
      }
    };
    if (one_pair) {
      // straight-line code: the wait before the product counts the tile loads above
      if (wave < npair_t) text_pair(wave);
    } else if (mq) {
      for (int pair = wave; pair < npair_t; pair += nwv) {
        if (pair != wave) load_text_tile(pair);
        text_pair(pair);
      }
    } else if (Tn > 0) {
      text_scores(wave * RPW + rw);
      for (int r0 = wave * RPW + rw + XB * rstep; r0 - rw < nrt; r0 += XB * rstep) {
        load_text(r0);
        text_scores(r0);
      }
    }

    // first tiles of the full-rank score pass (unless requested above): requested after
    // the text scores, whose rows then are the only loads ahead of them (requests in
    // flight during the selection's LDS-bound phases slow them more than they gain)
    if (!one_pair) {
#pragma unroll
      for (int s = 0; s < PD; ++s) ld(s);
    }
    // ---- F2. full-rank part of the selected tokens' scores (columns >= r_lo), on the
    // same block-diagonal tiles as the low-rank scores; final scores in log2 units
    const int nph = NPr - p0;
    uint2 qhi[NPM];
    [[maybe_unused]] float qhf[U4 ? NPM : 1][4];   // 4-bit codes: the values, scaled per block below
#pragma unroll
    for (int j = 0; j < NPM; ++j) {
      const int p = p0 + j;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = 16 * p + 4 * lg + e;
        v[e] = (my_on && p < NPr && col >= rlo) ? qs[my_h * r_pad + col] : 0.f;
      }
      if constexpr (U4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) qhf[j][e] = v[e];
      } else {
        qhi[j] = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
    // block-diagonal B operands: a lane feeds only the dwords of its own slot and tile half
    uint32_t om[NSL][2];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) om[sl][hf] = (sl == my_slot && hf == my_j) ? ~0u : 0u;
    auto diag = [&](uint32_t x, uint32_t y, int sl) {
      return __builtin_bit_cast(v8bf, make_uint4(x & om[sl][0], y & om[sl][0], x & om[sl][1], y & om[sl][1]));
    };
    // 4-bit codes: a lane's operand for every slot at once (non-zero in its own slot only),
    // against which one product with -136 in every A element cancels the offset 136 the
    // expanded codes of all the step's tiles carry
    [[maybe_unused]] const uint32_t mj0 = my_j == 0 ? ~0u : 0u, mj1 = ~mj0;
    [[maybe_unused]] auto own = [&](uint32_t x, uint32_t y) {
      return __builtin_bit_cast(v8bf, make_uint4(x & mj0, y & mj0, x & mj1, y & mj1));
    };
    [[maybe_unused]] const v8bf an8 = __builtin_bit_cast(
        v8bf, make_uint4(kQ4NegOffset2, kQ4NegOffset2, kQ4NegOffset2, kQ4NegOffset2));
    uint32_t selb = 0;   // bit 4a+t: token at full rank
#pragma unroll
    for (int a = 0; a < NACC; ++a) {
      const int n0 = tok(a);
      const uint32_t w = word_of(my_h, min(n0 >> 5, nblk - 1)) >> (n0 & 31);
      v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NPM; ++j) {
        const int s = a * NPM + j;
        if (j < nph) {
          if constexpr (U4) {
            // the K scales of the block in this lane's slot, folded into its latent-query values
            float sk[4];
            q4_scales(rsc[s % PD], sk);
            const uint32_t x = pack_bf16x2(qhf[j][0] * sk[0], qhf[j][1] * sk[1]);
            const uint32_t y = pack_bf16x2(qhf[j][2] * sk[2], qhf[j][3] * sk[3]);
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl)
              acc = mfma_bf16_k32(__builtin_bit_cast(v8bf, rb[s % PD][sl].deq()), diag(x, y, sl), acc);
            acc = mfma_bf16_k32(an8, own(x, y), acc);
          } else {
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl)
              acc = mfma_bf16_k32(__builtin_bit_cast(v8bf, rb[s % PD][sl].raw), diag(qhi[j].x, qhi[j].y, sl), acc);
          }
        }
        if (s + PD < 2 * NSK) ld(s + PD);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bool ok = (vm >> (4 * a + t)) & 1u;
        const bool full = ok && ((w >> t) & 1u);
        selb |= full ? (1u << (4 * a + t)) : 0u;
        sc[4 * a + t] = ok ? sl2 * (sc[4 * a + t] + (full ? acc[t] : 0.f)) : -INFINITY;
      }
    }
    // ---- F3. softmax over text and visual tokens: per-head maximum, probabilities, sums
    {
      // absent scores are -inf; a head's maximum of finite scores is finite
      float fm = -INFINITY;
#pragma unroll
      for (int i = 0; i < KPL; ++i) fm = fmaxf(fm, sc[i]);
      fm = head_fmax<HG>(fm);
      if (lg == 0 && c16 < HG && my_on) atomicMax(&hmx[my_h], fm == -INFINITY ? 0u : score_key(fm));
    }
    lds_barrier();
    {
      const float Mh = my_on ? key_score(hmx[my_h]) : 0.f;
      float lp = 0.f;
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const float pv = hw_exp2(sc[i] - Mh);   // -inf -> 0
        sc[i] = pv;
        lp += pv;
      }
      lp = head_sum<HG>(lp);
      if (lg == 0 && c16 < HG) lpart[wave * HG + c16] = lp;
      if (wave < nh && Tn > 0) {
        const float M = key_score(hmx[wave]);
        float lt = 0.f;
        for (int t = lane; t < Tn; t += 64) {
          const float pv = hw_exp2(sts[wave * Tn + t] - M);
          sts[wave * Tn + t] = pv;
          lt += pv;
        }
        lt = group_sum(lt, 64);
        if (lane == 0) ltx[wave] = lt;
      }
    }
    // output rows (F5): thread = (head, 16-byte column chunk, row group); rows 0..r_pad-1
    // of a head are B_v rows, then its text V rows.  The first UP rows of each thread are
    // requested as soon as the value pass has issued its last tile load.  Units cover all
    // HG heads (a power of two: LPR is one here); units of absent heads read the last
    // present head's rows and store nothing.
    const int lpr_sh = 31 - __builtin_clz(LPR);
    const int ounits = HG * LPR;
    const int RS = nthr >> (lpr_sh + 2);
    const int ounit = tid & (ounits - 1), rsub = tid >> (lpr_sh + 2);
    const int ohl = ounit >> lpr_sh, occ = ounit & (LPR - 1);
    const int og = ((h0 + min(ohl, nh - 1)) * ginv_num) >> 16;
    const int orows = r_pad + Tn;
    constexpr int UP = 8;
    Vec16<TB> xo[UP];
    auto load_out = [&](int r0) {
#pragma unroll
      for (int u = 0; u < UP; ++u) {
        const int row = min(r0 + u * RS, orows - 1);   // clamped: loads stay unconditional
        const TB* src = row < r_pad ? Bv + ((size_t)b * r_pad + row) * W
                                    : tv + ((size_t)b * Tn + (row - r_pad)) * W;
        xo[u].load_nt(src + (size_t)og * d + occ * V);
      }
    };

    // ---- F4. latent values z_h = sum_n p[n] U_v[n, :r(n)]: U_v tiles as the A operand
    // (rows = latent columns), probabilities as the block-diagonal B operand
    v4f Z[NPM];
#pragma unroll
    for (int p = 0; p < NPM; ++p) Z[p] = v4f{0.f, 0.f, 0.f, 0.f};
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int a = 0; a < NACC; ++a) {
      const float* pv = sc + 4 * a;
      const uint32_t pa0 = pack_bf16x2(pv[0], pv[1]), pa1 = pack_bf16x2(pv[2], pv[3]);
      // the same probabilities with those of tokens below full rank cleared
      auto sel_p = [&](int t) { return __uint_as_float(__float_as_uint(pv[t]) & bit_mask(selb, 4 * a + t)); };
      const uint32_t ps0 = pack_bf16x2(sel_p(0), sel_p(1)), ps1 = pack_bf16x2(sel_p(2), sel_p(3));
      // 4-bit codes: the offset products of this step (all tokens, and selected tokens only)
      [[maybe_unused]] v4f cpa, cps;
      if constexpr (U4) {
        const v4f z0 = v4f{0.f, 0.f, 0.f, 0.f};
        cpa = mfma_bf16_k32(an8, own(pa0, pa1), z0);
        cps = mfma_bf16_k32(an8, own(ps0, ps1), z0);
      }
#pragma unroll
      for (int p = 0; p < NPM; ++p) {
        const int s = NSK + a * NPM + p;
        if constexpr (U4) {
          // per step: D = sum over the step's tokens of code * p (offset cancelled), then
          // Z += scale * D, the V scale of the block in this lane's slot for D's row
          // (latent column 16p + 4lg + t); no panel straddles r_lo (r_lo = 16 NPL)
          if (p < NPr) {
            const bool lo = 16 * p + 16 <= rlo;
            v4f D = lo ? cpa : cps;
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl)
              D = mfma_bf16_k32(__builtin_bit_cast(v8bf, rb[s % PD][sl].deq()),
                                lo ? diag(pa0, pa1, sl) : diag(ps0, ps1, sl), D);
            float sv[4];
            q4_scales(rsc[s % PD], sv);
#pragma unroll
            for (int t = 0; t < 4; ++t) Z[p][t] = fmaf(sv[t], D[t], Z[p][t]);
          }
        } else if (p < NPr) {
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) {
            const v8bf ba = diag(pa0, pa1, sl);
            const v8bf bs = diag(ps0, ps1, sl);
            const v8bf av = __builtin_bit_cast(v8bf, rb[s % PD][sl].raw);
            if (16 * p + 16 <= rlo) {
              Z[p] = mfma_bf16_k32(av, ba, Z[p]);
            } else if (16 * p >= rlo) {
              Z[p] = mfma_bf16_k32(av, bs, Z[p]);
            } else {   // panel straddling r_lo: this lane's A row is latent column 16p + c16
              const bool lo_row = 16 * p + c16 < rlo;
              const v8bf zz = __builtin_bit_cast(v8bf, z4);
              Z[p] = mfma_bf16_k32(lo_row ? av : zz, ba, Z[p]);
              Z[p] = mfma_bf16_k32(lo_row ? zz : av, bs, Z[p]);
            }
          }
        }
        if (s + PD < 2 * NSK) ld(s + PD);
        if (s + PD == 2 * NSK - 1) {
          load_out(rsub);   // right after the last tile load
          // a compiler memory barrier: the loads stay here instead of being sunk to their
          // use after the value reduction (it waits for nothing)
          asm volatile("" ::: "memory");
        }
      }
    }
    // moving-average selector: this lane's exp2(s - M) wait in LDS (lane-private slots)
    // for the softmax sums, which the reductions below complete
    if constexpr (EMA) {
      float* pst = reinterpret_cast<float*>(smem_raw + Ly.pst);
#pragma unroll
      for (int i = 0; i < KPL; ++i) pst[i * nthr + tid] = sc[i];
    }
    // lane l holds Z for latent columns 16p + 4lg + t and tile column c16: sum the
    // columns of one head inside the row, one partial per wavefront (fixed-order sums)
#pragma unroll
    for (int p = 0; p < NPM; ++p)
#pragma unroll
      for (int t = 0; t < 4; ++t) Z[p][t] = head_sum_row<HG>(Z[p][t]);
    if (c16 < HG) {
#pragma unroll
      for (int p = 0; p < NPM; ++p)
        if (p < NPr) {
#pragma unroll
          for (int t = 0; t < 4; ++t) zpart[(wave * HG + c16) * r_pad + 16 * p + 4 * lg + t] = Z[p][t];
        }
    }
    lds_barrier();
    for (int idx = tid; idx < nh * r_pad; idx += nthr) {
      const int hl = idx / r_pad, i = idx - hl * r_pad;
      float z = 0.f;
      for (int w2 = 0; w2 < nwv; ++w2) z += zpart[(w2 * HG + hl) * r_pad + i];
      zs[idx] = z;
    }
    if (tid < nh) {
      float l = ltx[tid];
      for (int w2 = 0; w2 < nwv; ++w2) l += lpart[w2 * HG + tid];
      lfin[tid] = l;
    }
    lds_barrier();
    // moving-average selector per head (not the first step): the state this step blends
    // into, requested before the output pass, which hides the wait
    [[maybe_unused]] float old[EMA ? KPL : 1];
    if constexpr (EMA) {
      if (fa.imp != nullptr && fa.ema_first == 0 && fa.keys != nullptr) {
        const float* row = fa.imp + ((size_t)b * Hq + h0 + (my_on ? my_h : 0)) * N;
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
          const int n0 = tok(a);
#pragma unroll
          for (int t = 0; t < 4; ++t) old[4 * a + t] = row[min(n0 + t, N - 1)];
        }
      }
    }

    // ---- F5. out_h = (z_h B_v[:, g's columns] + sum_t p_t V_text[t, g's columns]) / l_h:
    // weighted sums of the r_pad + Tn output rows, partial sums per row group
    {
      float acc[V];
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = 0.f;
      auto accumulate = [&](int r0) {
#pragma unroll
        for (int u = 0; u < UP; ++u) {
          const int row = r0 + u * RS;
          const float wgt = row < orows ? (row < r_pad ? zs[ohl * r_pad + row] : sts[ohl * Tn + row - r_pad]) : 0.f;
#pragma unroll
          for (int e = 0; e < V; ++e) acc[e] = fmaf(wgt, xo[u].get(e), acc[e]);
        }
      };
      accumulate(rsub);
      for (int r0 = rsub + UP * RS; r0 < orows; r0 += UP * RS) {
        load_out(r0);
        accumulate(r0);
      }
      const int units = ounits, unit = ounit;
      if (rsub < RS) {
#pragma unroll
        for (int e = 0; e < V; ++e) red[(rsub * units + unit) * V + e] = acc[e];
      }
      lds_barrier();
      for (int idx = tid; idx < units * V; idx += nthr) {
        float o = 0.f;
        for (int r = 0; r < RS; ++r) o += red[(size_t)r * units * V + idx];
        const int h2 = idx >> (lpr_sh + 3), j = idx & (d - 1);   // d = 8 LPR
        if (h2 < nh) fa.out[((size_t)b * Hq + h0 + h2) * d + j] = o / lfin[h2];
      }
    }
    if constexpr (EMA) {
      // the step's attention weights of this lane's tokens, p = exp2(s - M) / l (0 for
      // absent tokens and heads)
      const float* pst = reinterpret_cast<const float*>(smem_raw + Ly.pst);
      const float linv = my_on ? 1.0f / lfin[my_h] : 0.f;
      if (fa.imp != nullptr) {
        // per head: I <- alpha I + (1 - alpha) p, or I <- p on the first step
        float* row = fa.imp + ((size_t)b * Hq + h0 + (my_on ? my_h : 0)) * N;
        const float al = fa.alpha, bl = 1.f - fa.alpha;
        const bool first = fa.ema_first != 0 || fa.keys == nullptr;
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
          const int n0 = tok(a);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float pw = pst[(4 * a + t) * nthr + tid] * linv;
            if (my_on && n0 + t < N) row[n0 + t] = first ? pw : fmaf(al, old[4 * a + t], bl * pw);
          }
        }
      } else {
        // per token: the sum over this workgroup's heads (the four lanes of a quad hold the
        // four heads of the same tokens), one store per token
        float* row = fa.ema_part + ((size_t)b * HGN + hg) * N;
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
          const int n0 = tok(a);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            float v = pst[(4 * a + t) * nthr + tid] * linv;
            v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
            v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
            if (my_h == 0 && n0 + t < N) row[n0 + t] = v;
          }
        }
      }
    }
  }
}

// Selection only: writes the selection words and the latent queries for the split-N
// flash-decode kernel.
template <class T, int HG, int NPL, int NACC, bool MQ>
__global__ __launch_bounds__(1024) void k_select(
    const T* __restrict__ Uk, const StoreB<T>* __restrict__ Bk, const float* __restrict__ q,
    float* __restrict__ qt, uint32_t* __restrict__ mask, int32_t* __restrict__ sel_out, int B,
    int N, int nblk, int NP, int r_pad, int W, int d, int G, int Hq, int Hq_pad, int HGN,
    int r_lo, int top_k, FusedArgs fa) {
  select_body<T, HG, NPL, NACC, false, 0, MQ>(Uk, Bk, q, qt, mask, sel_out, B, N, nblk, NP, r_pad, W, d,
                                              G, Hq, Hq_pad, HGN, r_lo, top_k, fa);
}

// The whole decode step of four query heads of one sequence (bf16 factors, or 4-bit U
// codes with bf16 B).
template <class T, int NPL, int NACC, int NPX, bool MQ, bool EMA>
__global__ __launch_bounds__(1024) void k_decode(
    const T* __restrict__ Uk, const StoreB<T>* __restrict__ Bk, const float* __restrict__ q,
    float* __restrict__ qt, uint32_t* __restrict__ mask, int32_t* __restrict__ sel_out, int B,
    int N, int nblk, int NP, int r_pad, int W, int d, int G, int Hq, int Hq_pad, int HGN,
    int r_lo, int top_k, FusedArgs fa) {
  select_body<T, 4, NPL, NACC, true, NPX, MQ, EMA>(Uk, Bk, q, qt, mask, sel_out, B, N, nblk, NP, r_pad,
                                                   W, d, G, Hq, Hq_pad, HGN, r_lo, top_k, fa);
}

// ---------------------------------------------------------------- launchers
struct SelPlan {
  int HG, NPL, NACC, waves;
};

static SelPlan select_plan(const Dims& dm, int r_lo, bool single_kernel) {
  const int nplo = (r_lo + 15) / 16;
  SelPlan pl;
  // 16 wavefronts; four heads per workgroup while 8 steps per wavefront cover the
  // tokens and the low rank fits two panels, else one head with the panels streamed one
  // at a time.  Steps per wavefront: the fewest of 2, 3, 4, 8 that cover the tokens.
  const int g4 = (dm.nblk + 1) / 2;
  pl.HG = (nplo <= 2 && g4 <= kSelMaxWaves * 8) ? 4 : 1;
  pl.NPL = pl.HG == 1 ? 8 : (nplo <= 1 ? 1 : 2);
  const int ngrp = (dm.nblk + 8 / pl.HG - 1) / (8 / pl.HG);
  pl.waves = kSelMaxWaves;
  // More workgroups than CUs (selection alone): 8 wavefronts, so two workgroups share a
  // CU and one's loads overlap the other's selection (the batch-256 layer: 108 -> 77 us).
  // Needs 8 steps per wavefront to cover the tokens and one q value per thread.
  const size_t wgs = (size_t)dm.B * ((dm.Hq + pl.HG - 1) / pl.HG);
  if (!single_kernel && pl.HG == 4 && wgs > 256 && ngrp <= 8 * 8 && 4 * dm.d <= 8 * 64)
    pl.waves = 8;
  const int per = (ngrp + pl.waves - 1) / pl.waves;
  pl.NACC = pl.HG == 1 ? 8 : (per <= 2 ? 2 : (per <= 3 ? 3 : (per <= 4 ? 4 : 8)));
  return pl;
}

template <class T, int HG, int NPL, int NACC, bool FUSED, int NPX = 0, bool MQ = false, bool EMA = false>
static hipError_t launch_select_v(const ap_cache* c, const float* q, int r_lo, int top_k,
                                  int32_t* sel_out, int waves, const FusedArgs& fa, hipStream_t st,
                                  const KernelEvents& ev) {
  const Dims& dm = c->dm;
  const int HGN = (dm.Hq + HG - 1) / HG;
  const size_t lds = sel_layout(HG, dm.nblk, dm.r_pad, dm.d, FUSED, FUSED ? fa.Tn : 0, FUSED && EMA ? 4 * NACC : 0).total;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  if ((dm.nblk + 8 / HG - 1) / (8 / HG) > waves * NACC) return hipErrorInvalidValue;
  if (HG * dm.d > 64 * waves) return hipErrorInvalidValue;
  const void* fn;
  if constexpr (FUSED) fn = reinterpret_cast<const void*>(&k_decode<T, NPL, NACC, NPX, MQ, EMA>);
  else fn = reinterpret_cast<const void*>(&k_select<T, HG, NPL, NACC, MQ>);
  static std::atomic<uint32_t> lds_set{0};
  hipError_t e = ensure_lds_limit(fn, 160 * 1024, lds_set);
  if (e != hipSuccess) return e;
  const int grid = ((dm.B + 7) / 8) * 8 * HGN;
  if constexpr (FUSED)
    hipExtLaunchKernelGGL((k_decode<T, NPL, NACC, NPX, MQ, EMA>), dim3(grid), dim3(64 * waves), lds, st, ev.start,
                          ev.stop, 0, static_cast<const T*>(c->Uk), static_cast<const StoreB<T>*>(c->Bk), q,
                          c->qt, c->mask, sel_out, dm.B, dm.N, dm.nblk, dm.NP, dm.r_pad, dm.W, dm.d,
                          dm.G, dm.Hq, dm.Hq_pad, HGN, r_lo, top_k, fa);
  else
    hipExtLaunchKernelGGL((k_select<T, HG, NPL, NACC, MQ>), dim3(grid), dim3(64 * waves), lds, st,
                          ev.start, ev.stop, 0, static_cast<const T*>(c->Uk),
                          static_cast<const StoreB<T>*>(c->Bk), q, c->qt, c->mask, sel_out, dm.B, dm.N,
                          dm.nblk, dm.NP, dm.r_pad, dm.W, dm.d, dm.G, dm.Hq, dm.Hq_pad, HGN, r_lo,
                          top_k, fa);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_select_t(const ap_cache* c, const float* q, int r_lo, int top_k,
                                  int32_t* sel_out, const float* keys, bool keys_per_head,
                                  hipStream_t st, const KernelEvents& ev) {
  const SelPlan pl = select_plan(c->dm, r_lo, false);
  FusedArgs fa{};
  fa.keys = keys;
  fa.keys_per_head = keys_per_head ? 1 : 0;
  fa.Usc = reinterpret_cast<const bf16_t*>(c->Usc);
  // latent queries on MFMA for bf16 B_k rows with d a multiple of 32 up to 128
  constexpr bool kMq = !std::is_same<T, float>::value;
  const bool mq = kMq && c->dm.d % 32 == 0 && c->dm.d <= 128;
#define AP_SEL(HGV, NPLV, NACCV)                                                        \
  if (pl.HG == HGV && pl.NPL == NPLV && pl.NACC == NACCV)                               \
    return mq ? launch_select_v<T, HGV, NPLV, NACCV, false, 0, kMq>(c, q, r_lo, top_k, sel_out, pl.waves, fa, st, ev) \
              : launch_select_v<T, HGV, NPLV, NACCV, false>(c, q, r_lo, top_k, sel_out, pl.waves, fa, st, ev);
  AP_SEL(4, 1, 2)
  AP_SEL(4, 1, 3)
  AP_SEL(4, 1, 4)
  AP_SEL(4, 1, 8)
  AP_SEL(4, 2, 2)
  AP_SEL(4, 2, 3)
  AP_SEL(4, 2, 4)
  AP_SEL(4, 2, 8)
  AP_SEL(1, 8, 8)
#undef AP_SEL
  return hipErrorInvalidValue;
}

hipError_t launch_select(const ap_cache* c, const float* q, int r_lo, int top_k, int32_t* sel_out,
                         const float* keys, bool keys_per_head, hipStream_t st, const KernelEvents& ev) {
  if (c->dm.storage == AP_INT4)
    return launch_select_t<i4_t>(c, q, r_lo, top_k, sel_out, keys, keys_per_head, st, ev);
  if (c->dm.storage == AP_BF16)
    return launch_select_t<bf16_t>(c, q, r_lo, top_k, sel_out, keys, keys_per_head, st, ev);
  return launch_select_t<float>(c, q, r_lo, top_k, sel_out, keys, keys_per_head, st, ev);
}

// The single kernel's compile-time panel split: r = 64 (4 panels) with r_lo = 16,
// latent queries on MFMA, 2 or 3 steps per wavefront.  4-bit codes and the
// moving-average selector take the single kernel only there.
static bool fused_exact_shape(const Dims& dm, int r_lo, const SelPlan& pl) {
  return dm.NP == 4 && pl.NPL == 1 && r_lo == 16 && (pl.NACC == 2 || pl.NACC == 3) &&
         dm.d % 32 == 0 && dm.d <= 128;
}

bool decode_fused_supported(const Dims& dm, int r_lo, int n_text) {
  if ((dm.storage != AP_BF16 && dm.storage != AP_INT4) || dm.NP > 4 || n_text > 1024) return false;
  const SelPlan pl = select_plan(dm, r_lo, true);
  if (pl.HG != 4) return false;
  if (dm.storage == AP_INT4 && !fused_exact_shape(dm, r_lo, pl)) return false;
  // each workgroup re-reads its sequence's U_k / U_v from L2 and runs one long chain:
  // worth it while the workgroups fit the GPU at one per CU (256 CUs); with more, the
  // split-N path spreads the same bytes better (measured on the batch-64 GQA and the
  // batch-256 layers)
  if ((size_t)dm.B * ((dm.Hq + 3) / 4) > 256) return false;
  const int LPR = dm.d / 8;
  if (dm.d % 8 != 0 || LPR > 64 || (LPR & (LPR - 1)) != 0 || dm.W % 8 != 0) return false;
  return sel_layout(4, dm.nblk, dm.r_pad, dm.d, true, n_text).total <= 160 * 1024;
}

// The moving-average selector in the single kernel: bf16 factors in the same
// compile-time panel split (the state's registers fit beside the scores there).
bool decode_fused_ema_supported(const Dims& dm, int r_lo, int n_text) {
  if (dm.storage != AP_BF16 || !decode_fused_supported(dm, r_lo, n_text)) return false;
  const SelPlan pl = select_plan(dm, r_lo, true);
  return fused_exact_shape(dm, r_lo, pl) &&
         sel_layout(4, dm.nblk, dm.r_pad, dm.d, true, n_text, 4 * pl.NACC).total <= 160 * 1024;
}

hipError_t launch_decode_fused(const ap_cache* c, const float* q, float* out, int r_lo, int top_k,
                               int32_t* sel_out, int n_text, const void* text_k, const void* text_v,
                               float sl2, const FusedEma* ema, hipStream_t st, const KernelEvents& ev) {
  const SelPlan pl = select_plan(c->dm, r_lo, true);
  FusedArgs fa;
  fa.Uv = c->Uv;
  fa.Bv = c->Bv;
  fa.text_k = n_text > 0 ? text_k : nullptr;
  fa.text_v = n_text > 0 ? text_v : nullptr;
  fa.out = out;
  fa.Tn = n_text;
  fa.sl2 = sl2;
  fa.keys = nullptr;
  fa.keys_per_head = 0;
  fa.Usc = reinterpret_cast<const bf16_t*>(c->Usc);
  fa.imp = nullptr;
  fa.ema_part = nullptr;
  fa.alpha = 0.f;
  fa.ema_first = 0;
  // r = 64 (4 panels) with r_lo = 16: the panel split known at compile time (variants
  // that fit the registers without spilling)
  const bool exact = c->dm.NP == 4 && r_lo == 16 * pl.NPL;
  // latent queries and text scores on MFMA: d a multiple of 32 up to 128
  const bool mq = c->dm.d % 32 == 0 && c->dm.d <= 128;
  if (ema != nullptr) {
    if (c->dm.storage != AP_BF16 || !fused_exact_shape(c->dm, r_lo, pl)) return hipErrorInvalidValue;
    fa.keys = ema->first ? nullptr : ema->keys;
    fa.keys_per_head = ema->per_head ? 1 : 0;
    fa.imp = ema->per_head ? ema->imp : nullptr;
    fa.ema_part = ema->per_head ? nullptr : ema->part;
    fa.alpha = ema->alpha;
    fa.ema_first = ema->first ? 1 : 0;
    if (pl.NACC == 2)
      return launch_select_v<bf16_t, 4, 1, 2, true, 4, true, true>(c, q, r_lo, top_k, sel_out, pl.waves, fa, st, ev);
    return launch_select_v<bf16_t, 4, 1, 3, true, 4, true, true>(c, q, r_lo, top_k, sel_out, pl.waves, fa, st, ev);
  }
  if (c->dm.storage == AP_INT4) {
    if (!fused_exact_shape(c->dm, r_lo, pl)) return hipErrorInvalidValue;
    if (pl.NACC == 2)
      return launch_select_v<i4_t, 4, 1, 2, true, 4, true>(c, q, r_lo, top_k, sel_out, pl.waves, fa, st, ev);
    return launch_select_v<i4_t, 4, 1, 3, true, 4, true>(c, q, r_lo, top_k, sel_out, pl.waves, fa, st, ev);
  }
#define AP_FUS(NPLV, NACCV)                                                             \
  if (pl.NPL == NPLV && pl.NACC == NACCV)                                               \
    return launch_select_v<bf16_t, 4, NPLV, NACCV, true, 0>(c, q, r_lo, top_k, sel_out, pl.waves, fa, st, ev);
#define AP_FUS_X(NPLV, NACCV)                                                           \
  if (pl.NPL == NPLV && pl.NACC == NACCV)                                               \
    return exact ? (mq ? launch_select_v<bf16_t, 4, NPLV, NACCV, true, 4, true>(c, q, r_lo, top_k, sel_out, pl.waves, fa, st, ev) \
                       : launch_select_v<bf16_t, 4, NPLV, NACCV, true, 4>(c, q, r_lo, top_k, sel_out, pl.waves, fa, st, ev)) \
                 : launch_select_v<bf16_t, 4, NPLV, NACCV, true, 0>(c, q, r_lo, top_k, sel_out, pl.waves, fa, st, ev);
  AP_FUS_X(1, 2)
  AP_FUS_X(1, 3)
  AP_FUS(1, 4)
  AP_FUS(1, 8)
  AP_FUS(2, 2)
  AP_FUS(2, 3)
  AP_FUS(2, 4)
  AP_FUS(2, 8)
#undef AP_FUS_X
#undef AP_FUS
  return hipErrorInvalidValue;
}

}  // namespace ap

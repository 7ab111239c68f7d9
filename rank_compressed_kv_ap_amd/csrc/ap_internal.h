// Host-side internals shared by the API implementation and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <string>
#include <vector>

#include "../../include/ap.h"

namespace ap {

constexpr int kBlockTokHost = 32;                  // tokens per tiled block
constexpr float kLog2eHost = 1.4426950408889634f;  // scores are kept in log2 units

// Derived sizes of one cache.
struct Dims {
  int B, N, Hkv, Hq, d, W, r, ell, p, q;
  int storage;          // ap_dtype
  int esize;            // bytes per stored element of B (and of K, V, text): 4 f32, 2 bf16 / int4
  int ubytes;           // bytes per tiled U panel of 512 elements: 256 with 4-bit codes
  int NP;               // panels of 16 columns: r_pad = 16 * NP
  int r_pad;
  int N_pad;            // tokens rounded up to a 32-token block
  int nblk;             // N_pad / 32
  int HT;               // query-head tiles of 16: Hq_pad = 16 * HT
  int Hq_pad;
  int G;                // Hq / Hkv
  int S_cap;            // most N-splits the decode workspace holds
};

struct TimingState {
  int max_calls = 0;
  int calls = 0;
  std::vector<hipEvent_t> ev;  // [max_calls][AP_N_KERNELS][2]
  std::vector<uint8_t> used;   // [max_calls][AP_N_KERNELS]: the kernel ran in that call
};

}  // namespace ap

struct ap_cache {
  ap::Dims dm;
  ap_compress_params params;
  // factors
  void* Uk = nullptr;   // [B][nblk][2][NP][512]: K-layout panels then V-layout panels
  void* Uv = nullptr;   // = Uk + NP*512 elements (same allocation)
  uint16_t* Usc = nullptr;  // 4-bit codes only: bf16 block scales [B][nblk][2][r_pad]
  void* Bk = nullptr;   // [B][r_pad][W] row-major (rows r..r_pad-1 zero)
  void* Bv = nullptr;
  float* sigma_k = nullptr;  // [B][r]
  float* sigma_v = nullptr;
  // decode workspace
  float* qt = nullptr;        // [B][Hq_pad][r_pad] latent queries
  uint32_t* mask = nullptr;   // [B][nblk][Hq_pad] selection bits per 32-token block
  float* part_z = nullptr;    // [B][S_cap][Hq_pad][r_pad]
  float* part_ml = nullptr;   // [B][S_cap][Hq_pad][2]  (running max in log2 units, sum)
  float* ml_final = nullptr;  // [B][Hq][2] softmax max (log2 units) and sum of the last step
  float* out_part = nullptr;  // [B][Hq][d] this cache's normalised attention output when it
                              // serves as another cache's second (text) segment
  size_t factor_bytes = 0;
  size_t device_bytes = 0;
  hipStream_t last_stream = nullptr;
  ap::TimingState timing;
};

namespace ap {

void set_error(const std::string& msg);

// Raise a kernel's dynamic LDS limit on the current device, once per device (devices
// 0..31 remembered in `done`, one flag set per kernel instantiation).
inline hipError_t ensure_lds_limit(const void* fn, int bytes, std::atomic<uint32_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint32_t bit = 1u << (dev & 31);
  if (dev < 32 && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && dev < 32) done.fetch_or(bit, std::memory_order_relaxed);
  return e;
}

// Events that a launch's own dispatch timestamps at the kernel's start and end
// (hipExtLaunchKernelGGL), or null for an untimed launch.
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// ---- launchers (decode_kernels.hip, select_kernel.hip)
hipError_t launch_select(const ap_cache* c, const float* q, int r_lo, int top_k,
                         int32_t* sel_out, const float* keys, bool keys_per_head, hipStream_t st,
                         const KernelEvents& ev);
hipError_t launch_attn(const ap_cache* c, int r_lo, float scale_log2e, int S, int CB, float* ema_s,
                       hipStream_t st, const KernelEvents& ev);
// Single-kernel decode (select_kernel.hip): shapes it takes, and its launch.
// The moving-average selector in the single kernel: keys = the state it ranks by (null
// on the first step: the low-rank logits); per head the kernel blends the step's
// weights into imp itself, per token it writes per-head-group sums to part, which
// launch_ema_fold then folds into imp.
struct FusedEma {
  const float* keys;
  float* imp;
  float* part;
  float alpha;
  bool per_head;
  bool first;
};
bool decode_fused_supported(const Dims& dm, int r_lo, int n_text);
bool decode_fused_ema_supported(const Dims& dm, int r_lo, int n_text);
hipError_t launch_decode_fused(const ap_cache* c, const float* q, float* out, int r_lo, int top_k,
                               int32_t* sel_out, int n_text, const void* text_k, const void* text_v,
                               float sl2, const FusedEma* ema, hipStream_t st, const KernelEvents& ev);
// xo, xml (optional): another segment's normalised output [B][Hq][d] and its softmax
// maximum and sum [B][Hq][2], merged as one more partial.
hipError_t launch_combine(const ap_cache* c, const float* q, float* out, float scale_log2e,
                          int S, int T, const void* text_k, const void* text_v, float* ml_out,
                          const float* xo, const float* xml, hipStream_t st,
                          const KernelEvents& ev);
// A small factored segment (its factors and one KV head's B rows fit 96 KB of LDS) of
// every (sequence, query head) in one kernel: writes c->out_part and c->ml_final, merged
// by another cache's combine; sel_out (optional) receives the selected ids [B][Hq][top_k].
bool text_seg_supported(const Dims& dm);
hipError_t launch_text_seg(const ap_cache* c, const float* q, int r_lo, int top_k, int32_t* sel_out,
                           float sl2, hipStream_t st, const KernelEvents& ev);
hipError_t launch_ema_update(const ap_cache* c, const float* s, const float* ml, float* imp,
                             bool per_head, bool first, float alpha, hipStream_t st,
                             const KernelEvents& ev);
// Per-token state after a single-kernel step: I[b][n] <- alpha I + (1 - alpha) mean_h p
// from the per-head-group sums part [B][ceil(Hq / 4)][N] (summed in group order).
hipError_t launch_ema_fold(const ap_cache* c, const float* part, float* imp, bool first, float alpha,
                           hipStream_t st, const KernelEvents& ev);

// ---- launchers (pack_kernels.hip)
hipError_t launch_pack_u(const ap_cache* c, const void* src, void* dst, bool v_layout,
                         hipStream_t st);
hipError_t launch_unpack_u(const ap_cache* c, const void* src, void* dst, bool v_layout,
                           hipStream_t st);

// ---- launchers (compress_kernels.hip)
hipError_t run_compress(ap_cache* c, const void* k, const void* v, hipStream_t st);
// The same factorisation with its workspace in the library's fixed device array of
// kNoAllocWorkspaceBytes (no allocation; hipErrorNotSupported when it does not fit).
constexpr size_t kNoAllocWorkspaceBytes = size_t(128) << 20;
hipError_t run_compress_noalloc(ap_cache* c, const void* k, const void* v, hipStream_t st);

}  // namespace ap

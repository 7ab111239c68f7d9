// C ABI of the compressed-KV decode-attention library: argument validation,
// ownership of device memory, and the stream-ordered launch sequence.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "ap_internal.h"

namespace ap {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

static ap_status fail(ap_status s, const std::string& msg) {
  set_error(msg);
  return s;
}

static ap_status hip_fail(hipError_t e, const char* what) {
  set_error(std::string(what) + ": " + hipGetErrorString(e));
  return AP_ERR_HIP;
}

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

// N-splits of the flash-decode kernel for one cache: about one workgroup per CU, >= 5
// token blocks each; splits > 0 is the caller's count.  Returns the split count and sets the blocks per split.
static int split_plan(const Dims& dm, int splits, int* CB) {
  int S = splits;
  if (S == 0) {
    // about one flash-decode workgroup per CU (256) for bf16 factors: measured best on
    // the batch-4 long-video (64 splits), batch-64 GQA (4), batch-32 LLaVA (8) and
    // batch-256 (1) layers, where twice as many workgroups cost 2-11% more per step; 4-bit
    // codes keep two per CU (the expansion makes that kernel issue-bound: batch-64 GQA
    // attention 26.9 us at 8 splits, 34.7 us at 4)
    S = ceil_div(dm.storage == AP_INT4 ? 512 : 256, dm.B);
    S = std::min(S, std::max(1, dm.nblk / 5));
  }
  // 4-bit codes: a workgroup stages the block scales of its tokens in LDS (<= 64 blocks)
  if (dm.storage == AP_INT4) S = std::max(S, ceil_div(dm.nblk, 64));
  S = std::max(1, std::min(S, dm.S_cap));
  *CB = ceil_div(dm.nblk, S);
  return ceil_div(dm.nblk, *CB);
}

static ap_status validate_shape(const ap_compress_params* p) {
  if (p->storage != AP_F32 && p->storage != AP_BF16 && p->storage != AP_INT4)
    return fail(AP_ERR_BAD_DTYPE, "storage must be AP_F32, AP_BF16 or AP_INT4");
  if (p->reserved != 0) return fail(AP_ERR_BAD_SHAPE, "reserved must be 0");
  if (p->batch < 0) return fail(AP_ERR_BAD_SHAPE, "batch < 0");
  if (p->n_tokens < 1) return fail(AP_ERR_BAD_SHAPE, "n_tokens < 1");
  if (p->n_kv_heads < 1 || p->n_q_heads < 1) return fail(AP_ERR_BAD_SHAPE, "head counts must be >= 1");
  if (p->n_q_heads % p->n_kv_heads != 0) return fail(AP_ERR_BAD_SHAPE, "n_q_heads must be a multiple of n_kv_heads");
  if (p->head_dim < 1) return fail(AP_ERR_BAD_SHAPE, "head_dim < 1");
  const long long W = (long long)p->n_kv_heads * p->head_dim;
  if (p->rank < 1 || p->rank > p->n_tokens || p->rank > W) return fail(AP_ERR_BAD_SHAPE, "need 1 <= rank <= min(n_tokens, n_kv_heads*head_dim)");
  if (p->oversample < 0) return fail(AP_ERR_BAD_SHAPE, "oversample < 0");
  if (p->power_iters < 0) return fail(AP_ERR_BAD_SHAPE, "power_iters < 0");
  // limits of the kernels' tiling
  if (p->n_tokens > 32768) return fail(AP_ERR_UNSUPPORTED, "n_tokens > 32768");
  if (p->batch > 32767) return fail(AP_ERR_UNSUPPORTED, "batch > 32767 (2 * batch matrices index one grid dimension)");
  if (p->head_dim > 256) return fail(AP_ERR_UNSUPPORTED, "head_dim > 256");
  if (p->n_q_heads > 64) return fail(AP_ERR_UNSUPPORTED, "n_q_heads > 64");
  if (p->rank > 128) return fail(AP_ERR_UNSUPPORTED, "rank > 128");
  if (p->power_iters > 8) return fail(AP_ERR_UNSUPPORTED, "power_iters > 8");
  if (W > (1 << 20)) return fail(AP_ERR_UNSUPPORTED, "n_kv_heads*head_dim > 2^20");
  const int NP = ceil_div(p->rank, 16);
  const int hq_pad = p->n_q_heads <= 16 ? 16 : (p->n_q_heads <= 32 ? 32 : 64);
  if (NP * (hq_pad / 16) > 16) return fail(AP_ERR_UNSUPPORTED, "rank x query heads too large for one tile set (need ceil(r/16)*ceil(Hq/16) <= 16)");
  return AP_OK;
}

static Dims make_dims(const ap_compress_params* p) {
  Dims d{};
  d.B = p->batch;
  d.N = p->n_tokens;
  d.Hkv = p->n_kv_heads;
  d.Hq = p->n_q_heads;
  d.d = p->head_dim;
  d.W = d.Hkv * d.d;
  d.r = p->rank;
  d.p = p->oversample;
  d.q = p->power_iters;
  d.ell = std::min(std::min(d.r + d.p, d.N), d.W);
  d.storage = p->storage;
  d.esize = p->storage == AP_F32 ? 4 : 2;
  d.ubytes = p->storage == AP_INT4 ? 256 : 512 * d.esize;
  d.NP = ceil_div(d.r, 16);
  d.r_pad = 16 * d.NP;
  d.N_pad = ceil_div(d.N, kBlockTokHost) * kBlockTokHost;
  d.nblk = d.N_pad / kBlockTokHost;
  d.Hq_pad = d.Hq <= 16 ? 16 : (d.Hq <= 32 ? 32 : 64);
  d.HT = d.Hq_pad / 16;
  d.G = d.Hq / d.Hkv;
  const int want = d.B > 0 ? ceil_div(4096, d.B) : 1;
  d.S_cap = std::min(d.nblk, std::max(16, want));
  return d;
}

static void free_all(ap_cache* c) {
  void* ptrs[] = {c->Uk, c->Usc, c->Bk, c->Bv, c->sigma_k, c->sigma_v, c->qt, c->mask, c->part_z, c->part_ml,
                  c->ml_final, c->out_part};
  for (void* q : ptrs)
    if (q) (void)hipFree(q);
  for (hipEvent_t e : c->timing.ev) (void)hipEventDestroy(e);
  c->timing.ev.clear();
}

static ap_status alloc_cache(ap_cache* c) {
  const Dims& dm = c->dm;
  struct Req { void** ptr; size_t bytes; };
  const size_t upan = (size_t)dm.B * dm.NP * dm.nblk;   // panels per factor
  const size_t usc = dm.storage == AP_INT4 ? (size_t)dm.B * dm.nblk * 2 * dm.r_pad * 2 : 0;
  Req reqs[] = {
      {&c->Uk, 2 * upan * dm.ubytes},
      {reinterpret_cast<void**>(&c->Usc), usc},
      {&c->Bk, (size_t)dm.B * dm.r_pad * dm.W * dm.esize},
      {&c->Bv, (size_t)dm.B * dm.r_pad * dm.W * dm.esize},
      {reinterpret_cast<void**>(&c->sigma_k), (size_t)dm.B * dm.r * 4},
      {reinterpret_cast<void**>(&c->sigma_v), (size_t)dm.B * dm.r * 4},
      {reinterpret_cast<void**>(&c->qt), (size_t)dm.B * dm.Hq_pad * dm.r_pad * 4},
      {reinterpret_cast<void**>(&c->mask), (size_t)dm.B * dm.nblk * dm.Hq_pad * 4},
      {reinterpret_cast<void**>(&c->part_z), (size_t)dm.B * dm.S_cap * dm.Hq_pad * dm.r_pad * 4},
      {reinterpret_cast<void**>(&c->part_ml), (size_t)dm.B * dm.S_cap * dm.Hq_pad * 2 * 4},
      {reinterpret_cast<void**>(&c->ml_final), (size_t)dm.B * dm.Hq * 2 * 4},
      {reinterpret_cast<void**>(&c->out_part), (size_t)dm.B * dm.Hq * dm.d * 4},
  };
  size_t total = 0;
  for (const Req& r : reqs) {
    if (r.bytes == 0) continue;
    hipError_t e = hipMalloc(r.ptr, r.bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      free_all(c);
      return fail(AP_ERR_OUT_OF_MEMORY, std::string("hipMalloc failed: ") + hipGetErrorString(e));
    }
    total += r.bytes;
  }
  c->Uv = c->Uk ? static_cast<char*>(c->Uk) + (size_t)dm.NP * dm.ubytes : nullptr;
  c->factor_bytes = 2 * upan * dm.ubytes + usc + 2 * (size_t)dm.B * dm.r_pad * dm.W * dm.esize;
  c->device_bytes = total;
  // padded rows of B and the singular values start at zero
  hipError_t e = hipSuccess;
  if (dm.B > 0) {
    e = hipMemset(c->Bk, 0, (size_t)dm.B * dm.r_pad * dm.W * dm.esize);
    if (e == hipSuccess) e = hipMemset(c->Bv, 0, (size_t)dm.B * dm.r_pad * dm.W * dm.esize);
    if (e == hipSuccess) e = hipMemset(c->sigma_k, 0, (size_t)dm.B * dm.r * 4);
    if (e == hipSuccess) e = hipMemset(c->sigma_v, 0, (size_t)dm.B * dm.r * 4);
  }
  if (e != hipSuccess) {
    free_all(c);
    return hip_fail(e, "hipMemset");
  }
  return AP_OK;
}

}  // namespace ap

using namespace ap;

extern "C" {

const char* ap_status_string(ap_status s) {
  switch (s) {
    case AP_OK: return "ok";
    case AP_ERR_NULL_ARG: return "null argument";
    case AP_ERR_BAD_SHAPE: return "bad shape";
    case AP_ERR_BAD_DTYPE: return "bad dtype";
    case AP_ERR_UNSUPPORTED: return "unsupported";
    case AP_ERR_OUT_OF_MEMORY: return "out of device memory";
    case AP_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* ap_last_error(void) { return g_last_error.c_str(); }

ap_status ap_compress(const void* k, const void* v, const ap_compress_params* p, void* stream,
                      ap_cache** out) {
  if (out) *out = nullptr;
  if (!p || !out) return fail(AP_ERR_NULL_ARG, "params and out must not be NULL");
  if ((k == nullptr) != (v == nullptr)) return fail(AP_ERR_NULL_ARG, "k and v must both be set or both be NULL");
  ap_status s = validate_shape(p);
  if (s != AP_OK) return s;
  if (k != nullptr) {
    const int W = p->n_kv_heads * p->head_dim;
    const int ell = std::min(std::min(p->rank + p->oversample, p->n_tokens), W);
    if (ell > 144) return fail(AP_ERR_UNSUPPORTED, "min(rank + oversample, n_tokens, width) must be <= 144");
  }
  ap_cache* c = new (std::nothrow) ap_cache();
  if (!c) return fail(AP_ERR_OUT_OF_MEMORY, "host allocation failed");
  c->params = *p;
  c->params.omega = nullptr;
  c->dm = make_dims(p);
  s = alloc_cache(c);
  if (s != AP_OK) {
    delete c;
    return s;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  c->last_stream = st;
  if (k != nullptr && c->dm.B > 0) {
    set_error("");
    c->params.omega = p->omega;
    hipError_t e = run_compress(c, k, v, st);
    c->params.omega = nullptr;
    if (e != hipSuccess) {
      std::string detail = g_last_error;
      free_all(c);
      delete c;
      if (e == hipErrorOutOfMemory) return fail(AP_ERR_OUT_OF_MEMORY, "compress workspace: " + detail);
      if (e == hipErrorNotSupported) return fail(AP_ERR_UNSUPPORTED, detail);
      return fail(AP_ERR_HIP, std::string("compress: ") + hipGetErrorString(e) +
                                  (detail.empty() ? std::string() : " (" + detail + ")"));
    }
  }
  *out = c;
  return AP_OK;
}

ap_status ap_recompress(ap_cache* c, const void* k, const void* v, const float* omega, uint64_t seed,
                        void* stream) {
  if (!c || !k || !v) return fail(AP_ERR_NULL_ARG, "cache, k and v must not be NULL");
  const Dims& dm = c->dm;
  const int ell = std::min(std::min(dm.r + dm.p, dm.N), dm.W);
  if (ell > 144) return fail(AP_ERR_UNSUPPORTED, "min(rank + oversample, n_tokens, width) must be <= 144");
  if (dm.B == 0) return AP_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  c->last_stream = st;
  set_error("");
  c->params.omega = omega;
  const uint64_t seed0 = c->params.seed;
  c->params.seed = seed;
  hipError_t e = run_compress(c, k, v, st);
  c->params.omega = nullptr;
  if (e != hipSuccess) {
    c->params.seed = seed0;
    std::string detail = g_last_error;
    if (e == hipErrorOutOfMemory) return fail(AP_ERR_OUT_OF_MEMORY, "compress workspace: " + detail);
    if (e == hipErrorNotSupported) return fail(AP_ERR_UNSUPPORTED, detail);
    return fail(AP_ERR_HIP, std::string("compress: ") + hipGetErrorString(e) +
                                (detail.empty() ? std::string() : " (" + detail + ")"));
  }
  return AP_OK;
}

ap_status ap_recompress_noalloc(ap_cache* c, const void* k, const void* v, const float* omega, uint64_t seed,
                                void* stream) {
  if (!c || !k || !v) return fail(AP_ERR_NULL_ARG, "cache, k and v must not be NULL");
  const Dims& dm = c->dm;
  const int ell = std::min(std::min(dm.r + dm.p, dm.N), dm.W);
  if (ell > 144) return fail(AP_ERR_UNSUPPORTED, "min(rank + oversample, n_tokens, width) must be <= 144");
  if (dm.B == 0) return AP_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  set_error("");
  const float* omega0 = c->params.omega;
  const uint64_t seed0 = c->params.seed;
  c->params.omega = omega;
  c->params.seed = seed;
  hipError_t e = run_compress_noalloc(c, k, v, st);
  c->params.omega = omega0;
  if (e != hipSuccess) {
    c->params.seed = seed0;
    std::string detail = g_last_error;
    if (e == hipErrorNotSupported) return fail(AP_ERR_UNSUPPORTED, detail);
    return fail(AP_ERR_HIP, std::string("ap_recompress_noalloc: ") + hipGetErrorString(e) +
                                (detail.empty() ? std::string() : " (" + detail + ")"));
  }
  c->last_stream = st;
  return AP_OK;
}

ap_status ap_cache_set_factors(ap_cache* c, const void* U_k, const void* B_k, const void* U_v,
                               const void* B_v, void* stream) {
  if (!c || !U_k || !B_k || !U_v || !B_v) return fail(AP_ERR_NULL_ARG, "cache and all factor pointers must be set");
  const Dims& dm = c->dm;
  if (dm.B == 0) return AP_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  c->last_stream = st;
  hipError_t e = launch_pack_u(c, U_k, c->Uk, false, st);
  if (e == hipSuccess) e = launch_pack_u(c, U_v, c->Uv, true, st);
  const size_t row = (size_t)dm.r * dm.W * dm.esize;
  const size_t dpitch = (size_t)dm.r_pad * dm.W * dm.esize;
  if (e == hipSuccess) e = hipMemcpy2DAsync(c->Bk, dpitch, B_k, row, row, dm.B, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess) e = hipMemcpy2DAsync(c->Bv, dpitch, B_v, row, row, dm.B, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "set_factors");
  return AP_OK;
}

ap_status ap_cache_get_factors(const ap_cache* c, void* U_k, void* B_k, void* U_v, void* B_v, void* stream) {
  if (!c) return fail(AP_ERR_NULL_ARG, "cache is NULL");
  const Dims& dm = c->dm;
  if (dm.B == 0) return AP_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (U_k) e = launch_unpack_u(c, c->Uk, U_k, false, st);
  if (e == hipSuccess && U_v) e = launch_unpack_u(c, c->Uv, U_v, true, st);
  const size_t row = (size_t)dm.r * dm.W * dm.esize;
  const size_t spitch = (size_t)dm.r_pad * dm.W * dm.esize;
  if (e == hipSuccess && B_k) e = hipMemcpy2DAsync(B_k, row, c->Bk, spitch, row, dm.B, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && B_v) e = hipMemcpy2DAsync(B_v, row, c->Bv, spitch, row, dm.B, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "get_factors");
  return AP_OK;
}

ap_status ap_cache_get_sigma(const ap_cache* c, float* sigma_k, float* sigma_v, void* stream) {
  if (!c) return fail(AP_ERR_NULL_ARG, "cache is NULL");
  const Dims& dm = c->dm;
  if (dm.B == 0) return AP_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t bytes = (size_t)dm.B * dm.r * 4;
  hipError_t e = hipSuccess;
  if (sigma_k) e = hipMemcpyAsync(sigma_k, c->sigma_k, bytes, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && sigma_v) e = hipMemcpyAsync(sigma_v, c->sigma_v, bytes, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "get_sigma");
  return AP_OK;
}

ap_status ap_cache_info(const ap_cache* c, ap_compress_params* p_out, size_t* factor_bytes, size_t* device_bytes) {
  if (!c) return fail(AP_ERR_NULL_ARG, "cache is NULL");
  if (p_out) *p_out = c->params;
  if (factor_bytes) *factor_bytes = c->factor_bytes;
  if (device_bytes) *device_bytes = c->device_bytes;
  return AP_OK;
}

ap_status ap_decode_attn(ap_cache* c, const float* q, float* out, const ap_decode_params* p, void* stream) {
  if (!p) return fail(AP_ERR_NULL_ARG, "params must not be NULL");
  // checks of the parameters alone come first, then those against the cache
  if (!(std::isfinite(p->scale) && p->scale > 0.f)) return fail(AP_ERR_BAD_SHAPE, "scale must be finite and > 0");
  if (p->n_text < 0) return fail(AP_ERR_BAD_SHAPE, "n_text < 0");
  if (p->n_text == 0 && (p->text_k || p->text_v))
    return fail(AP_ERR_BAD_SHAPE, "text_k/text_v must be NULL when n_text == 0");
  if (p->splits < 0) return fail(AP_ERR_BAD_SHAPE, "splits < 0");
  if (p->select_mode < AP_SELECT_LOGIT || p->select_mode > AP_SELECT_EMA_HEAD)
    return fail(AP_ERR_BAD_SHAPE, "select_mode must be AP_SELECT_LOGIT, AP_SELECT_EMA_TOKEN or AP_SELECT_EMA_HEAD");
  const bool ema = p->select_mode != AP_SELECT_LOGIT;
  if (ema && !(p->ema_alpha >= 0.f && p->ema_alpha < 1.f))
    return fail(AP_ERR_BAD_SHAPE, "ema_alpha must satisfy 0 <= alpha < 1");
  if (!c) return fail(AP_ERR_NULL_ARG, "cache must not be NULL");
  const Dims& dm = c->dm;
  if (p->r_lo < 1 || p->r_lo > dm.r) return fail(AP_ERR_BAD_SHAPE, "need 1 <= r_lo <= rank");
  if (p->top_k < 0 || p->top_k > dm.N) return fail(AP_ERR_BAD_SHAPE, "need 0 <= top_k <= n_tokens");
  ap_cache* tc = const_cast<ap_cache*>(p->text_cache);   // its workspace is written
  if (tc) {
    const Dims& dt = tc->dm;
    if (tc == c) return fail(AP_ERR_BAD_SHAPE, "text_cache must be another cache");
    if (dt.B != dm.B || dt.Hq != dm.Hq || dt.Hkv != dm.Hkv || dt.d != dm.d)
      return fail(AP_ERR_BAD_SHAPE, "text_cache must have the same batch, query/KV heads and head_dim");
    if (p->text_r_lo < 1 || p->text_r_lo > dt.r) return fail(AP_ERR_BAD_SHAPE, "need 1 <= text_r_lo <= text rank");
    if (p->text_top_k < 0 || p->text_top_k > dt.N)
      return fail(AP_ERR_BAD_SHAPE, "need 0 <= text_top_k <= text n_tokens");
  }
  if (dm.B == 0) return AP_OK;
  if (!q || !out) return fail(AP_ERR_NULL_ARG, "q and out must not be NULL");
  if (p->n_text > 0 && (!p->text_k || !p->text_v)) return fail(AP_ERR_NULL_ARG, "text_k/text_v must be set when n_text > 0");
  if (p->n_text > (1 << 20)) return fail(AP_ERR_UNSUPPORTED, "n_text > 2^20");
  if (ema && (!p->importance || !p->ema_scratch))
    return fail(AP_ERR_NULL_ARG, "importance and ema_scratch must be set for the moving-average selector");

  int CB = 0;
  const int S = split_plan(dm, p->splits, &CB);

  hipStream_t st = static_cast<hipStream_t>(stream);
  c->last_stream = st;
  const float sl2 = p->scale * kLog2eHost;
  TimingState& tm = c->timing;
  const bool timed = tm.max_calls > 0 && tm.calls < tm.max_calls;
  // timed calls: each kernel's own dispatch stamps its start and end events
  auto events = [&](int kernel) {
    KernelEvents ev;
    if (timed) {
      ev.start = tm.ev[((size_t)tm.calls * AP_N_KERNELS + kernel) * 2];
      ev.stop = tm.ev[((size_t)tm.calls * AP_N_KERNELS + kernel) * 2 + 1];
      tm.used[(size_t)tm.calls * AP_N_KERNELS + kernel] = 1;
    }
    return ev;
  };
  if (timed)
    for (int k = 0; k < AP_N_KERNELS; ++k) tm.used[(size_t)tm.calls * AP_N_KERNELS + k] = 0;
  hipError_t e = hipSuccess;
  const bool per_head = p->select_mode == AP_SELECT_EMA_HEAD;
  if (tc) {
    // the factored text segment first: its own selection, flash-decode and combine give
    // its normalised output and softmax statistics, merged by the visual combine below
    tc->last_stream = st;
    const KernelEvents evt = events(AP_KERNEL_TEXT);
    if (text_seg_supported(tc->dm)) {
      // small segment: the whole segment of a (sequence, head) in one workgroup
      e = launch_text_seg(tc, q, p->text_r_lo, p->text_top_k, p->text_sel_out, sl2, st, evt);
    } else {
      int CBt = 0;
      const int St = split_plan(tc->dm, 0, &CBt);
      e = launch_select(tc, q, p->text_r_lo, p->text_top_k, p->text_sel_out, nullptr, false, st,
                        KernelEvents{evt.start, nullptr});
      if (e == hipSuccess) e = launch_attn(tc, p->text_r_lo, sl2, St, CBt, nullptr, st, KernelEvents{});
      if (e == hipSuccess)
        e = launch_combine(tc, q, tc->out_part, sl2, St, 0, nullptr, nullptr, tc->ml_final, nullptr,
                           nullptr, st, KernelEvents{nullptr, evt.stop});
    }
    if (e != hipSuccess) return hip_fail(e, "text segment launch");
  }
  const float* xo = tc ? tc->out_part : nullptr;
  const float* xml = tc ? tc->ml_final : nullptr;
  if (!ema && !tc && p->splits == 0 && decode_fused_supported(dm, p->r_lo, p->n_text)) {
    // one kernel per step: each (sequence, 4 heads) workgroup selects, attends and projects
    e = launch_decode_fused(c, q, out, p->r_lo, p->top_k, p->sel_out, p->n_text, p->text_k,
                            p->text_v, sl2, nullptr, st, events(AP_KERNEL_DECODE));
  } else if (ema && !tc && p->splits == 0 && decode_fused_ema_supported(dm, p->r_lo, p->n_text)) {
    // the moving-average selector in the same kernel: it ranks by the state and blends
    // the step's weights into it (per head), or leaves per-head-group sums of the weights
    // in ema_scratch for a fold into the per-token state
    const FusedEma fe{p->importance, p->importance, p->ema_scratch, p->ema_alpha, per_head,
                      p->ema_first != 0};
    e = launch_decode_fused(c, q, out, p->r_lo, p->top_k, p->sel_out, p->n_text, p->text_k,
                            p->text_v, sl2, &fe, st, events(AP_KERNEL_DECODE));
    if (e == hipSuccess && !per_head)
      e = launch_ema_fold(c, p->ema_scratch, p->importance, p->ema_first != 0, p->ema_alpha, st,
                          events(AP_KERNEL_EMA));
  } else {
    // the moving-average selector ranks by the importance state, except on its first
    // step (no history yet), which ranks by the low-rank logits like the default
    const float* keys = (ema && !p->ema_first) ? p->importance : nullptr;
    e = launch_select(c, q, p->r_lo, p->top_k, p->sel_out, keys, per_head, st, events(AP_KERNEL_SELECT));
    if (e == hipSuccess)
      e = launch_attn(c, p->r_lo, sl2, S, CB, ema ? p->ema_scratch : nullptr, st, events(AP_KERNEL_ATTN));
    if (e == hipSuccess)
      e = launch_combine(c, q, out, sl2, S, p->n_text, p->text_k, p->text_v, ema ? c->ml_final : nullptr,
                         xo, xml, st, events(AP_KERNEL_COMBINE));
    if (e == hipSuccess && ema)
      e = launch_ema_update(c, p->ema_scratch, c->ml_final, p->importance, per_head, p->ema_first != 0,
                            p->ema_alpha, st, events(AP_KERNEL_EMA));
  }
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (timed) tm.calls++;
  return AP_OK;
}

void ap_free(ap_cache* c) {
  if (!c) return;
  (void)hipStreamSynchronize(c->last_stream);
  free_all(c);
  delete c;
}

ap_status ap_timing_enable(ap_cache* c, int32_t max_calls) {
  if (!c) return fail(AP_ERR_NULL_ARG, "cache is NULL");
  if (max_calls < 0) return fail(AP_ERR_BAD_SHAPE, "max_calls < 0");
  TimingState& tm = c->timing;
  for (hipEvent_t e : tm.ev) (void)hipEventDestroy(e);
  tm.ev.clear();
  tm.calls = 0;
  tm.max_calls = 0;
  const size_t n = (size_t)max_calls * AP_N_KERNELS * 2;
  tm.ev.resize(n, nullptr);
  tm.used.assign((size_t)max_calls * AP_N_KERNELS, 0);
  for (size_t i = 0; i < n; ++i) {
    hipError_t e = hipEventCreate(&tm.ev[i]);
    if (e != hipSuccess) {
      for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(tm.ev[j]);
      tm.ev.clear();
      return hip_fail(e, "hipEventCreate");
    }
  }
  tm.max_calls = max_calls;
  return AP_OK;
}

ap_status ap_timing_read(ap_cache* c, float* ms_per_kernel, int32_t* calls) {
  if (!c || !ms_per_kernel) return fail(AP_ERR_NULL_ARG, "cache and ms_per_kernel must not be NULL");
  TimingState& tm = c->timing;
  for (int k = 0; k < AP_N_KERNELS; ++k) ms_per_kernel[k] = 0.f;
  for (int i = 0; i < tm.calls; ++i)
    for (int k = 0; k < AP_N_KERNELS; ++k) {
      if (!tm.used[(size_t)i * AP_N_KERNELS + k]) continue;   // not launched in that call
      hipEvent_t a = tm.ev[((size_t)i * AP_N_KERNELS + k) * 2];
      hipEvent_t b = tm.ev[((size_t)i * AP_N_KERNELS + k) * 2 + 1];
      hipError_t e = hipEventSynchronize(b);
      float ms = 0.f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
      if (e != hipSuccess) return hip_fail(e, "timing read");
      ms_per_kernel[k] += ms;
    }
  if (calls) *calls = tm.calls;
  tm.calls = 0;
  return AP_OK;
}

}  // extern "C"

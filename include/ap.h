/*
 * ap.h — C ABI of the compressed-KV decode-attention library (libap.so, gfx950).
 *
 * The method is AttentionPack as summarised on the gist.science pages (es, fr, de)
 * for "Attention-aware Inference Optimizations for Large Vision-Language Models with
 * Memory-efficient Decoding"; sections are cited as [fr §2.A] etc.
 *
 * Conventions for every entry point:
 *   - Plain C types only.  Device buffers are passed as device pointers, the HIP
 *     stream as `void*` (a hipStream_t; NULL = the null stream).
 *   - Every call validates all of its arguments before it enqueues anything.  On a
 *     validation error nothing is enqueued, nothing is allocated and output
 *     handles are set to NULL.  ap_last_error() gives a message for the failure.
 *   - Work is enqueued asynchronously on `stream`; a kernel fault surfaces at the
 *     caller's next synchronisation, as with any stream API.  Inputs must stay
 *     valid, and outputs untouched, until the stream has passed the call.
 *   - A cache handle is used by one stream at a time; calls on one handle from
 *     several streams at once race.  Different handles are independent.
 *   - No C++ exception crosses this boundary.
 */
#ifndef RANK_COMPRESSED_KV_AP_H
#define RANK_COMPRESSED_KV_AP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AP_OK = 0,
  AP_ERR_NULL_ARG = 1,       /* a required pointer was NULL                          */
  AP_ERR_BAD_SHAPE = 2,      /* sizes out of range or inconsistent                   */
  AP_ERR_BAD_DTYPE = 3,      /* storage dtype not one of ap_dtype                    */
  AP_ERR_UNSUPPORTED = 4,    /* valid by the method, outside what the library handles */
  AP_ERR_OUT_OF_MEMORY = 5,  /* a device allocation failed                           */
  AP_ERR_HIP = 6             /* a HIP runtime call failed                            */
} ap_status;

/* Storage of a cache.  AP_F32, AP_BF16: K, V in and U, B stored in that type.
 * AP_INT4: 4-bit token factors.  [es §3 "Integración Modular"], [fr §4 "Compatibilité"],
 * [de §3 "Kombinierbarkeit"]: the method composes with 4-bit quantization of the cache;
 * [fr §1 "Limites des solutions existantes"]: plain quantization struggles with
 * outliers.  The pages fix no format; here K, V come in as bf16, B is stored bf16 and
 * U as symmetric codes in [-7, 7] with one bf16 scale per (32-token block, column):
 * scale = bf16_rne(fp32(max |x|) * fp32(1/7)) over the block's tokens of that column,
 * code = x / scale rounded to nearest with ties to even (0 when the scale is 0), and
 * the stored value is code * scale.  Decoding attends over exactly those values. */
typedef enum { AP_F32 = 0, AP_BF16 = 1, AP_INT4 = 2 } ap_dtype;

/* Shape of one attention layer's visual cache and how it is factored.
 *
 * [fr §2.A "Approche", de §2.A "Optimierung"]: the keys of all KV heads are
 * concatenated along the hidden axis, so one sequence's visual keys form one
 * N x W matrix, W = n_kv_heads * head_dim, columns head-major (head g owns
 * columns g*d .. g*d+d-1).  The same holds for the values.
 * [fr §2.A "Mécanisme"/"Gain"]: each matrix is stored as a compressed matrix
 * U (N x rank) and a decompression matrix B (rank x W).
 */
typedef struct {
  int32_t batch;        /* 0 <= B <= 32767 sequences (0: an empty cache, every call is  
                           a no-op; larger B: AP_ERR_UNSUPPORTED)                        */
  int32_t n_tokens;     /* N, 1 <= N <= 32768 visual tokens per sequence                */
  int32_t n_kv_heads;   /* Hkv >= 1                                                      */
  int32_t n_q_heads;    /* Hq, a multiple of Hkv, Hq <= 64 (decode workspace is sized here) */
  int32_t head_dim;     /* d, 1 <= d <= 256                                              */
  int32_t rank;         /* r, 1 <= r <= min(128, N, W)                                   */
  int32_t oversample;   /* p >= 0; the range finder keeps ell = min(r + p, N, W) columns */
  int32_t power_iters;  /* q, 0 <= q <= 8 power iterations                               */
  int32_t storage;      /* ap_dtype of K, V in and of U, B stored (AP_INT4: K, V and B
                           bf16, U 4-bit)                                                */
  int32_t reserved;     /* must be 0                                                     */
  uint64_t seed;        /* omega == NULL: the test matrix of matrix m (2b: K, 2b+1: V) has
                           entry (w, j) = -1 if bit i%32 of word (i/32)%4 of
                           Philox4x32-10(counter (i/128, m, 0, 0), key (seed lo, seed hi))
                           is set, else +1, with i = j*W + w (random signs)               */
  const float* omega;   /* optional device [B][2][W][ell] float32 test matrices
                           (index 0: for K, 1: for V), row-major, caller-owned and read
                           during ap_compress only; NULL: drawn on the device from seed. */
} ap_compress_params;

/* Opaque handle: the factored cache of a batch plus its decode workspace.  All of
 * its device memory is owned by the library and released by ap_free. */
typedef struct ap_cache ap_cache;

/* Factor each sequence's heads-merged visual K and V to rank r.
 *
 * Defines: [fr §2.A], [es §2.A], [de §2.A] — K ~= K* D_k and V ~= V* D_v by a
 * singular value decomposition of the heads-merged matrix, K and V separately, no
 * token removed.  This library computes it by randomized subspace iteration (Halko,
 * Martinsson & Tropp 2011): ell = min(r+p, N, W) probe columns, q power iterations,
 * then a one-sided Jacobi SVD of the ell x ell core; U = Q V_r diag(sigma_r) carries
 * the singular values, B has orthonormal rows, components in decreasing order.
 *
 * k, v:   device [B][N][W] row-major in p->storage dtype, caller-owned, read on
 *         `stream` during the call.  k == v == NULL allocates the cache without
 *         computing factors (load them with ap_cache_set_factors).  Exactly one of
 *         them NULL is AP_ERR_NULL_ARG.
 * p:      host struct, read during the call only.
 * out:    receives the new handle (NULL on any error).  The call allocates device
 *         memory synchronously (the cache, plus a workspace of about
 *         2B * ell * (3 max(N, W) + N + W) * 4 bytes held until the enqueued work is
 *         done), then enqueues the factorisation on `stream`.
 * Limit:  when factoring (k, v set) ell = min(r + p, N, W) must be <= 144 (r = 128 with
 *         the usual p = 16): the Cholesky and the core SVD keep an ell x ell matrix of
 *         each factorisation in one workgroup's LDS.  Larger ell is AP_ERR_UNSUPPORTED
 *         before anything is allocated.
 * Errors: AP_ERR_NULL_ARG, AP_ERR_BAD_SHAPE, AP_ERR_BAD_DTYPE, AP_ERR_UNSUPPORTED,
 *         AP_ERR_OUT_OF_MEMORY, AP_ERR_HIP.
 */
ap_status ap_compress(const void* k, const void* v, const ap_compress_params* p,
                      void* stream, ap_cache** out);

/* Factor new K and V of the cache's own shape into an existing cache, replacing its
 * factors and singular values (a serving slot reused for another batch).  Same
 * method, layout and limits as ap_compress ([fr §2.A], [es §2.A], [de §2.A]); the
 * cache's decode workspace is kept, only the factorisation workspace is taken
 * (stream-ordered) and released on `stream`.
 * k, v:   device [B][N][W] in the cache's storage dtype, caller-owned, read on `stream`.
 * omega:  optional device [B][2][W][ell] float32 test matrices (as in
 *         ap_compress_params); NULL: random signs from `seed`, as ap_compress draws them.
 * Errors: AP_ERR_NULL_ARG, AP_ERR_UNSUPPORTED (ell > 144), AP_ERR_OUT_OF_MEMORY,
 *         AP_ERR_HIP.  On an error the factors are unspecified. */
ap_status ap_recompress(ap_cache* c, const void* k, const void* v, const float* omega, uint64_t seed,
                        void* stream);

/* The same re-factorisation as ap_recompress, allocating nothing: for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops that
 * forbid hipMalloc).  Its factorisation workspace is a fixed device array inside the
 * library, 128 MiB (134217728 bytes) on each GPU the library runs on, held until the
 * process ends.  A shape whose workspace does not fit returns AP_ERR_UNSUPPORTED (the
 * message gives the bytes needed) before anything is enqueued.  The workspace needs
 * about 2B * ell_pad * (W s + max(N, W) (4 + 2 s) + N 4 + W 4) bytes, ell_pad = ell
 * rounded up to 16, s = 2 (bf16, 4-bit) or 4 (fp32).
 * Every call on a GPU uses that GPU's one array, which keeps the last call's contents:
 * calls that overlap on one GPU (several streams, or several host threads) race and
 * must be serialised by the caller.  Results equal ap_recompress's bit for bit.
 * Arguments, ownership and the other errors as for ap_recompress. */
ap_status ap_recompress_noalloc(ap_cache* c, const void* k, const void* v, const float* omega, uint64_t seed,
                                void* stream);

/* Load factors into a cache: U_k, U_v device [B][N][r], B_k, B_v device [B][r][W],
 * row-major, in the cache's storage dtype, caller-owned, read on `stream`.  The
 * layout is the plain one of [fr §2.A "Mécanisme"] (K ~= U_k B_k); the cache keeps
 * its own tiled copy.  AP_INT4 caches take U as float32 and quantize it on the device
 * (the codes and scales defined at ap_dtype), and B as bf16.
 * Errors: AP_ERR_NULL_ARG, AP_ERR_HIP. */
ap_status ap_cache_set_factors(ap_cache* c, const void* U_k, const void* B_k,
                               const void* U_v, const void* B_v, void* stream);

/* Copy the factors out in the same plain layout as ap_cache_set_factors (any of the
 * four pointers may be NULL to skip it).  AP_INT4 caches give U as float32, the stored
 * values code * scale.  sigma_k / sigma_v variants: see below. */
ap_status ap_cache_get_factors(const ap_cache* c, void* U_k, void* B_k, void* U_v,
                               void* B_v, void* stream);

/* Copy the r leading singular values found by ap_compress for each sequence,
 * device [B][r] float32 each (NULL to skip).  Zeros if the factors were loaded. */
ap_status ap_cache_get_sigma(const ap_cache* c, float* sigma_k, float* sigma_v, void* stream);

/* Shape of a cache and the device bytes it holds (factors + decode workspace). */
ap_status ap_cache_info(const ap_cache* c, ap_compress_params* p_out, size_t* factor_bytes,
                        size_t* device_bytes);

/* Per-step decode parameters.
 * [fr §2.B "Stratégie"]: the most important tokens are decompressed at the full rank
 * R_kv, the others at a reduced rank (R_kv/4 is the page's example).  [es §4 "Análisis
 * de Sensibilidad"]: 25% of the tokens at full rank.  Importance here is the
 * current-step low-rank logit of each token for each query head (see ap_decode_attn). */
typedef struct {
  int32_t r_lo;          /* reduced rank, 1 <= r_lo <= r                                  */
  int32_t top_k;         /* tokens at full rank per (sequence, query head), 0 <= k <= N   */
  float scale;           /* softmax scale, finite and > 0 (usually 1/sqrt(d))              */
  int32_t n_text;        /* T >= 0 dense text tokens joining the softmax                  */
  const void* text_k;    /* device [B][T][W] storage dtype (bf16 for AP_INT4), NULL iff T == 0
                            (set with T == 0, or NULL with T > 0: AP_ERR_BAD_SHAPE /
                            AP_ERR_NULL_ARG)                                             */
  const void* text_v;    /* device [B][T][W] storage dtype (bf16 for AP_INT4), NULL iff T == 0 */
  int32_t* sel_out;      /* optional device [B][Hq][top_k] int32: the selected token ids,
                            ascending per (sequence, head); NULL to skip                  */
  int32_t splits;        /* 0: library's choice (one kernel per step for the shapes it
                            covers, else split-N); >= 1: the split-N path with that many
                            N-splits per sequence (clamped to the workspace sized at
                            ap_compress)                                                 */
  /* Which tokens get full rank.  [es §2.B], [fr §2.B "Score d'importance"], [de §2.B
   * "Mechanismus"]: a moving average (parameter alpha) of the attention each token has
   * received.  AP_SELECT_LOGIT (0, the default when the struct is zeroed): the current
   * step's low-rank logit, no state.  AP_SELECT_EMA_TOKEN: one importance per token,
   * fed with the mean over query heads of the attention weights and shared by all
   * heads.  AP_SELECT_EMA_HEAD: one importance per (query head, token).  The moving-
   * average modes rank by the importance the earlier steps left (ema_first: no history
   * yet, rank by the low-rank logit), then blend in this step's attention weights p
   * (softmax over text and visual tokens): I <- alpha * I + (1 - alpha) * p, or I <- p
   * on the first step.  With splits == 0, bf16 factors of rank 64 and r_lo = 16 run
   * them in the single-kernel decode (per token, a second kernel then folds the
   * per-head-group sums of the weights into the state); otherwise the split-N path. */
  int32_t select_mode;
  float ema_alpha;       /* 0 <= alpha < 1: weight of the history                          */
  int32_t ema_first;     /* nonzero on the first step of a sequence's decode              */
  float* importance;     /* device float32 state, caller-owned, read then updated in place:
                            [B][N] (EMA_TOKEN) or [B][Hq][N] (EMA_HEAD)                    */
  float* ema_scratch;    /* device float32 workspace [B][Hq][N], caller-owned: the step's
                            logits (split-N path) or sums of the weights per group of four
                            query heads (single kernel, per token); contents undefined
                            between calls                                                 */
  /* A second factored segment.  [es §2.A], [fr §2.A "Traitement séparé"], [de §2.A
   * "Optimierung"]: text tokens are factored by their own SVD, apart from the visual
   * ones.  text_cache: a cache of the same batch, query/KV heads and head_dim holding
   * the text tokens' factors (its own rank, token count and storage), or NULL.  Its
   * tokens are selected and decompressed like the visual ones, within the segment: per
   * query head the text_top_k tokens of largest low-rank score (first text_r_lo
   * components) at the text cache's full rank, the rest at text_r_lo.  All segments
   * (visual, factored text, dense tokens) share one softmax.  The call writes the text
   * cache's decode workspace, so the text cache must not be in use on another stream.
   * The dense tokens above then serve as the tokens appended while decoding and not yet
   * factored; re-factoring them together with the text is the caller's (ap_compress). */
  const ap_cache* text_cache;
  int32_t text_r_lo;     /* 1 <= text_r_lo <= the text cache's rank (when text_cache set)   */
  int32_t text_top_k;    /* 0 <= text_top_k <= the text cache's n_tokens                    */
  int32_t* text_sel_out; /* optional device [B][Hq][text_top_k] int32: the text segment's
                            tokens taken at full rank, ascending per (sequence, head); NULL
                            to skip (ignored without text_cache)                          */
} ap_decode_params;

enum { AP_SELECT_LOGIT = 0, AP_SELECT_EMA_TOKEN = 1, AP_SELECT_EMA_HEAD = 2 };

/* One decode step of attention over the compressed cache, for every sequence.
 *
 * Defines: [es §2.B], [fr §2.B], [de §2.B] — per token and step, important tokens are
 * decompressed at full rank and the rest at reduced rank; attention follows.  For
 * sequence b and query head h (KV head g = h / (Hq/Hkv)), with q~ = B_k[:, g-th
 * head's columns] q_h:
 *   s_lo[n] = scale * U_k[n, :r_lo] . q~[:r_lo]                     (all n)
 *   Top_h   = the top_k tokens of largest s_lo (ties: lower index)
 *   s[n]    = s_lo[n] + [n in Top_h] * scale * U_k[n, r_lo:] . q~[r_lo:]
 *   p       = softmax over the N visual scores and the T text scores
 *             scale * K_text[t, g-th head's columns] . q_h
 *   out_h   = (sum_n p[n] U_v[n, :r(n)]) B_v[:r(n), g-th head's columns]
 *             + sum_t p[t] V_text[t, g-th head's columns],   r(n) = r if n in Top_h else r_lo
 * which equals explicit decompression K^[n] = U_k[n, :r(n)] B_k[:r(n)] followed by
 * dense attention, without forming K^ or V^.
 *
 * q:    device [B][Hq*d] float32, caller-owned.
 * out:  device [B][Hq*d] float32, caller-owned, fully overwritten.
 * With a factored text segment (text_cache) the visual sum above also runs over the
 * text segment's tokens, each scored and decompressed at its own rank in that segment.
 * The call allocates nothing.  It enqueues one kernel on `stream` when splits == 0 and
 * the shape allows (bf16 factors, r <= 64, r_lo <= 32, N <= 8192, head_dim a power of
 * two multiple of 8, T <= 1024, B * ceil(Hq/4) <= 256, no text_cache, the logit
 * selector): one workgroup per (sequence, 4 query heads) then selects, attends over all
 * tokens and projects.  Otherwise three kernels: selection, split-N flash-decode,
 * combine, and three more before them for a factored text segment.
 * Errors: AP_ERR_NULL_ARG, AP_ERR_BAD_SHAPE, AP_ERR_UNSUPPORTED (r_lo or r not
 * supported by the tiling), AP_ERR_HIP.
 */
ap_status ap_decode_attn(ap_cache* c, const float* q, float* out, const ap_decode_params* p,
                         void* stream);

/* Release a cache (NULL is a no-op).  Waits for the last stream used with the cache,
 * then frees all of its device memory. */
void ap_free(ap_cache* c);

/* Kernel timing for measurement.  While enabled, ap_decode_attn records HIP events
 * around each of its kernels on the caller's stream (at most max_calls calls are
 * recorded; later calls are not timed).  ap_timing_read waits for the recorded events,
 * writes the summed milliseconds per kernel (index: 0 select, 1 attention, 2 combine,
 * 3 the single-kernel decode, 4 the importance-state update, 5 the three kernels of the
 * factored text segment together) and the number of timed calls, and starts a new
 * recording.  max_calls == 0 disables. */
enum { AP_KERNEL_SELECT = 0, AP_KERNEL_ATTN = 1, AP_KERNEL_COMBINE = 2, AP_KERNEL_DECODE = 3,
       AP_KERNEL_EMA = 4, AP_KERNEL_TEXT = 5, AP_N_KERNELS = 6 };
ap_status ap_timing_enable(ap_cache* c, int32_t max_calls);
ap_status ap_timing_read(ap_cache* c, float* ms_per_kernel /* [AP_N_KERNELS] */, int32_t* calls);

/* Streaming-read ceiling of the device (a measurement aid, not part of the method): one
 * untimed and then `passes` timed runs of a plain grid-stride kernel that reads all of
 * `buf` (device memory, caller-owned, 16-byte aligned, `bytes` a multiple of 16) on
 * `stream`; writes the mean milliseconds per pass and returns after the passes finish.
 * Use a buffer well beyond the 256 MB last-level cache so that the reads come from HBM.
 * AP_ERR_NULL_ARG / AP_ERR_BAD_SHAPE before anything is enqueued; AP_ERR_HIP on a
 * runtime failure. */
ap_status ap_read_bandwidth(const void* buf, size_t bytes, int32_t passes, void* stream, float* ms_per_pass);

/* Text for a status code, and the detail of the calling thread's last failure. */
const char* ap_status_string(ap_status s);
const char* ap_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RANK_COMPRESSED_KV_AP_H */

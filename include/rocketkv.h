/*
 * rocketkv.h -- C ABI of librocketkv.so, the MI355X (gfx950) hot path of
 * RocketKV two-stage KV-cache compression: SnapKV-style permanent eviction
 * (stage 1) and Hybrid Sparse Attention decode (stage 2).
 *
 * Sources cited below:
 *   [RKV]   papercache.org deep notes "RocketKV: Accelerating Long-Context LLM
 *           Inference via Two-Stage KV Cache Compression" (arXiv 2502.14051).
 *   [GUIDE] aifetchly blog "RocketKV Guide: Two-Stage KV Cache Compression for
 *           LLMs", section "Stage 1: Coarse-Grain Permanent Eviction via SnapKV"
 *           (and, for the paged pool, its serving section).
 *
 * Conventions shared by every call:
 *   - Pointers named q*, k*, v*, kmax, kmin, out, *_idx, *_opt and ws are
 *     DEVICE pointers on the current HIP device; rk_shape and rk_split_out
 *     are HOST pointers.
 *   - Tensors are dense row-major.  B = batch, Hq = query heads, Hkv = KV
 *     heads, G = Hq / Hkv (query head j belongs to KV head j / G), d = head
 *     dim.  One (batch, KV head) pair is a "unit"; units are independent.
 *   - Element type of q, q_win, k, v, kmax, kmin is shape->dtype: RK_F32 or
 *     RK_BF16 (bf16 = the upper 16 bits of an IEEE float32).  Supported head
 *     dims: 64 and 128.  Scores, outputs and internal accumulation are float32.
 *   - Ownership: the caller owns every buffer.  The library allocates no
 *     device memory and keeps no pointer after a call returns; scratch space
 *     is the caller's workspace `ws` of at least *_workspace_bytes() bytes
 *     (256-byte aligned), except for rk_hsa_decode_noalloc, which uses a
 *     static device array of the library instead.
 *   - Calls that take a stream enqueue asynchronously on it (NULL = the null
 *     stream).  Outputs are valid after the stream reaches that point; inputs
 *     must stay alive until then.  Calls on one workspace must not overlap.
 *   - Errors: every argument is checked on the host before any launch; on an
 *     error nothing is enqueued and the code is returned.  A failed launch
 *     returns RK_EDEVICE.  rk_last_error() gives a thread-local message about
 *     the last failure.  Inputs must be finite; NaN/Inf give unspecified
 *     results (never out-of-bounds accesses).
 */
#ifndef ROCKETKV_H_
#define ROCKETKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RK_OK = 0,
  RK_EINVAL = 1,        /* bad argument: null pointer, size out of range   */
  RK_EUNSUPPORTED = 2,  /* valid but not built: dtype/head dim/group size  */
  RK_EWORKSPACE = 3,    /* workspace smaller than *_workspace_bytes()      */
  RK_EDEVICE = 4        /* a HIP launch or runtime call failed             */
} rk_status;

typedef enum { RK_F32 = 0, RK_BF16 = 1 } rk_dtype;

/* Sequence pooling of the stage-1 window scores: the windowed sum (the
 * reading built by default; it ranks as average pooling does) or the
 * windowed maximum (the notes say only "pooling"; max pooling is the other
 * plain reading). */
typedef enum { RK_POOL_SUM = 0, RK_POOL_MAX = 1 } rk_pool_op;

/* A hipStream_t, passed as an opaque pointer. */
typedef void* rk_stream;

typedef struct {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  rk_dtype dtype;
} rk_shape;

typedef struct {
  double r;          /* split factor, clamp(0.2 + 0.06 log2 c, 0.2, 0.8)      */
  double c1;         /* stage-1 compression c^r                               */
  double c2;         /* stage-2 compression c^(1-r)                           */
  double budget_t;   /* token budget t = S / c (KV pairs per attention op)    */
  int64_t n_keep;    /* stage-1 kept tokens: min(S, max(W, ceil(S / c^r)))    */
  int32_t k2_blocks; /* stage-2 pages: ceil(t / block)                        */
  int32_t paper_page;/* the notes' own page size ceil(c^((1-r)/2))            */
  double paper_k1;   /* the notes' own head-dim share: d / (c^(1-r)/page)     */
  int32_t paper_k1_channels; /* paper_k1 rounded to nearest, within [1, d]    */
  int32_t paper_k2_blocks;   /* the notes' step-3 half of the budget in their
                                own pages: ceil((t / 2) / paper_page)         */
} rk_split_out;

/*
 * rk_split -- the adaptive compression split.
 * [RKV] method details: adaptive split equation r = min(0.2 + 0.06 log2 c,
 * 0.8) with r restricted to [0.2, 0.8]; stage 1 takes c^r, stage 2 c^(1-r);
 * token budget paragraph: t = S / c per GQA group, shared evenly between
 * HSA steps 2 and 3; split inside HSA: page = ceil(c^((1-r)/2)), the head-dim
 * axis gets c^(1-r)/page.  k2_blocks gives step 3 the whole budget in pages
 * of `block` tokens (the workloads' sizing); the paper_* fields give the
 * notes' own decomposition (their page, k1 and the step-3 half of t).
 * c >= 1, 1 <= window <= seq_len, block >= 1, head_dim >= 1.  Pure host math
 * in double; touches no device.  RK_EINVAL on bad arguments or out == NULL.
 */
rk_status rk_split(double c, int64_t seq_len, int32_t window, int32_t block,
                   int32_t head_dim, rk_split_out* out);

/*
 * rk_snapkv_workspace_bytes -- workspace needed by rk_snapkv_evict for this
 * shape, prompt length and window (0 if the arguments are invalid).
 */
size_t rk_snapkv_workspace_bytes(const rk_shape* shape, int64_t seq_len, int32_t window);

/*
 * rk_snapkv_evict -- stage 1: SnapKV-style permanent eviction per unit.
 * [RKV] quick read (stage 1) and method details (SnapKV paragraph, GQA
 * group-level selection, pooling kernel 63); [GUIDE] stage 1 (observation
 * window, softmax(Q K^T / sqrt(D)) summed over the window).
 *
 * For each unit: the G*W window queries of its group attend causally (window
 * row r sits at position S-W+r) over the S prompt keys with scale 1/sqrt(d);
 * each row is softmax-normalised; score[j] = sum over the G heads and W rows
 * of the probability of key j, for the prefix j < S-W; pooled[j] = the sum of
 * score over [j-h, j+h] (h = (pool_kernel-1)/2, zero outside the prefix; for
 * kernel 63 the terms are grouped so neighbouring outputs share their common
 * middle, which moves a sum by a few ulp at most); the n_keep - W prefix
 * positions with the largest pooled score (ties to the lower position) are
 * kept, ascending, followed by the W window positions S-W .. S-1.
 *
 *   q_win    [B, Hq, W, d]          window queries (rows in position order)
 *   k, v     [B, Hkv, kv_cap, d]    prompt keys/values, first seq_len valid;
 *                                   v is read only when v_out != NULL
 *   kept_idx [B, Hkv, n_keep]       out: kept positions (int32, ascending)
 *   k_out, v_out [B, Hkv, out_cap, d]  out: compact cache rows 0..n_keep-1
 *                                   (row n = k[kept_idx[n]]).  Both NULL for
 *                                   the RocketKV-MT form (indices only).
 *   pooled_opt [B, Hkv, seq_len-W]  out (optional, float32): pooled scores
 *   kmax_opt, kmin_opt [B, Hkv, d, nblk_cap]  out (optional, with k_out): the
 *                                   HSA step-1 Kmax/Kmin of the compact cache
 *                                   in pages of `block` tokens, exactly what
 *                                   rk_hsa_build_aux(k_out, n_keep, 0, block,
 *                                   ...) writes; built while the rows are
 *                                   compacted, so the compact K is not read
 *                                   again.  Both NULL: no aux (block and
 *                                   nblk_cap are then ignored).
 * Requires 1 <= W <= seq_len <= kv_cap, W <= n_keep <= seq_len, odd
 * pool_kernel >= 1, out_cap >= n_keep when k_out is given, seq_len < 2^31;
 * with the aux outputs also k_out, block >= 1, ceil(n_keep/block) <=
 * nblk_cap, nblk_cap a multiple of 8.
 */
rk_status rk_snapkv_evict(const rk_shape* shape, const void* q_win, const void* k,
                          const void* v, int64_t kv_cap, int64_t seq_len, int32_t window,
                          int32_t pool_kernel, int64_t n_keep, int32_t* kept_idx,
                          void* k_out, void* v_out, int64_t out_cap, float* pooled_opt,
                          void* kmax_opt, void* kmin_opt, int64_t nblk_cap, int32_t block,
                          void* ws, size_t ws_bytes, rk_stream stream);

/*
 * rk_snapkv_evict_pool -- rk_snapkv_evict with the pooling operation given:
 * RK_POOL_SUM is rk_snapkv_evict; RK_POOL_MAX makes pooled[j] the largest
 * score over [j-h, j+h] within the prefix ([RKV] quick read and method
 * details, pooling paragraph: the kind of pooling is not stated).  A maximum
 * involves no rounding, so pooled is then exact for any grouping.  Other
 * arguments, requirements and errors as rk_snapkv_evict; RK_EINVAL for any
 * other pool_op.
 */
rk_status rk_snapkv_evict_pool(const rk_shape* shape, const void* q_win, const void* k,
                               const void* v, int64_t kv_cap, int64_t seq_len, int32_t window,
                               int32_t pool_kernel, int32_t pool_op, int64_t n_keep,
                               int32_t* kept_idx, void* k_out, void* v_out, int64_t out_cap,
                               float* pooled_opt, void* kmax_opt, void* kmin_opt, int64_t nblk_cap,
                               int32_t block, void* ws, size_t ws_bytes, rk_stream stream);

/*
 * rk_adakv_evict -- stage 1 with Ada-KV's shared budget.  [RKV] method
 * details, "the second stage and the framework's generality" (SnapKV or
 * Ada-KV as stage 1) and the GQA paragraph (group-level selection following
 * Ada-KV).  The notes name Ada-KV's adaptive budgets without their rule; the
 * rule built here: window scores and pooling per unit as rk_snapkv_evict,
 * then for each sequence the Hkv * (n_keep - W) prefix slots of its heads go
 * to the largest pooled scores over all its KV heads together (ties to the
 * lower head, then the lower position), so a head whose group attends to few
 * tokens keeps few; each head also keeps its W window positions.  Head h of
 * sequence b keeps kept_count[b, h] tokens: its chosen prefix positions
 * ascending, then S-W .. S-1.
 *
 *   kept_idx   [B, Hkv, out_cap] int32  out: rows 0 .. kept_count-1 valid
 *   kept_count [B, Hkv] int32           out
 *   k_out, v_out [B, Hkv, out_cap, d]   out (optional, both or neither):
 *                                       compact rows 0 .. kept_count-1
 *   kmax_opt, kmin_opt                  out (optional, with k_out): aux of
 *                                       each unit's kept_count tokens
 *   others as rk_snapkv_evict (same workspace size)
 * out_cap must be at least min(seq_len, Hkv * (n_keep - W) + W) (one head may
 * take the whole budget); Hkv <= 64.
 */
rk_status rk_adakv_evict(const rk_shape* shape, const void* q_win, const void* k, const void* v,
                         int64_t kv_cap, int64_t seq_len, int32_t window, int32_t pool_kernel,
                         int64_t n_keep, int32_t* kept_idx, int32_t* kept_count, void* k_out,
                         void* v_out, int64_t out_cap, float* pooled_opt, void* kmax_opt,
                         void* kmin_opt, int64_t nblk_cap, int32_t block, void* ws, size_t ws_bytes,
                         rk_stream stream);

/*
 * rk_adakv_evict_pool -- rk_adakv_evict with the pooling operation given
 * (RK_POOL_SUM or RK_POOL_MAX, as rk_snapkv_evict_pool); otherwise the same.
 */
rk_status rk_adakv_evict_pool(const rk_shape* shape, const void* q_win, const void* k, const void* v,
                              int64_t kv_cap, int64_t seq_len, int32_t window, int32_t pool_kernel,
                              int32_t pool_op, int64_t n_keep, int32_t* kept_idx,
                              int32_t* kept_count, void* k_out, void* v_out, int64_t out_cap,
                              float* pooled_opt, void* kmax_opt, void* kmin_opt, int64_t nblk_cap,
                              int32_t block, void* ws, size_t ws_bytes, rk_stream stream);

/*
 * rk_hsa_build_aux -- HSA step 1: per-page element-wise Kmax / Kmin.
 * [RKV] method details, HSA step 1: keys are grouped into consecutive pages
 * of `block` tokens; the element-wise max and min of each page are stored
 * aligned along the head dimension and refreshed whenever new keys arrive.
 *
 *   k        [B, Hkv, k_cap, d]     keys
 *   idx_opt  [B, Hkv, idx_stride]   optional candidate rows (RocketKV-MT): page
 *                                   token n is key row idx_opt[n]; NULL means
 *                                   token n is row n
 *   kmax, kmin [B, Hkv, d, nblk_cap]  out, channel-major (page index fastest);
 *                                   nblk_cap must be a multiple of 8 so every
 *                                   channel row starts 16-byte aligned.  kmin
 *                                   may be NULL: only Kmax is written (with
 *                                   pages of one token Kmax = Kmin = the keys
 *                                   themselves, channel-major: SparQ's second
 *                                   copy of K)
 * Pages first_token/block .. ceil(n_tokens/block)-1 are (re)computed from
 * tokens [page*block, min((page+1)*block, n_tokens)); other pages are left
 * untouched, so after appending tokens n_old..n_tokens-1 a call with
 * first_token = n_old equals a full rebuild bit for bit.  Exact: max/min only.
 * Requires 0 <= first_token < n_tokens, ceil(n_tokens/block) <= nblk_cap
 * (a multiple of 8),
 * n_tokens <= k_cap (identity map) or <= idx_stride (candidate map); every
 * idx_opt entry must lie in [0, k_cap).
 */
rk_status rk_hsa_build_aux(const rk_shape* shape, const void* k, int64_t k_cap,
                           const int32_t* idx_opt, int64_t idx_stride, int64_t n_tokens,
                           int64_t first_token, int32_t block, void* kmax, void* kmin,
                           int64_t nblk_cap, rk_stream stream);

/*
 * rk_append_kv -- append one decode token per unit and refresh its page.
 * [RKV] method details, HSA step 1: the auxiliary max/min data is updated
 * whenever a new key is generated.
 *
 *   k_new, v_new [B, Hkv, d]         the new key / value rows
 *   k, v     [B, Hkv, kv_cap, d]     compact cache; row `pos` is written
 *   kmax, kmin [B, Hkv, d, nblk_cap] page pos/block becomes the element-wise
 *                                    max / min of its old value and k_new, or
 *                                    k_new itself when pos starts the page
 * Pages before pos/block are untouched.  If the aux data was valid for tokens
 * [0, pos), it equals rk_hsa_build_aux over [0, pos] bit for bit afterwards.
 * Requires 0 <= pos < kv_cap, pos/block < nblk_cap (a multiple of 8).
 */
rk_status rk_append_kv(const rk_shape* shape, const void* k_new, const void* v_new, void* k,
                       void* v, int64_t kv_cap, int64_t pos, void* kmax, void* kmin,
                       int64_t nblk_cap, int32_t block, rk_stream stream);

/*
 * rk_hsa_workspace_bytes -- workspace needed by rk_hsa_decode / _mt for this
 * shape, token count, page size and k1/k2 (0 if the arguments are invalid).
 */
size_t rk_hsa_workspace_bytes(const rk_shape* shape, int64_t n_tokens, int32_t block,
                              int32_t k1, int32_t k2);

/*
 * rk_hsa_decode -- HSA steps 2 and 3 for one decode query per head.
 * [RKV] method details, HSA steps 2-3, and Algorithm 1:
 *   a_i   = sum_g |q_g,i|, q_bar_i = sum_g q_g,i     (float32, g ascending)
 *   i1    = the k1 channels of largest a_i (ties to the lower channel)
 *   P_i   = Kmax row i if q_bar_i >= 0, else Kmin row i
 *   s1[b] = sum over i in i1, ascending, of q_bar_i * P_i[b]  (float32,
 *           one rounded multiply and one rounded add per term)
 *   i2    = the min(k2, nblk) pages of largest s1 (ties to the lower page)
 *   out_g = softmax(q_g . K_T^T / sqrt(d)) V_T over the valid tokens T of
 *           the pages i2, for each head g of the group (float32 accumulation)
 *
 *   q        [B, Hq, d]             decode queries
 *   k, v     [B, Hkv, kv_cap, d]    compact cache, tokens 0..n_tokens-1 valid
 *   kmax, kmin [B, Hkv, d, nblk_cap]  from rk_hsa_build_aux
 *   out      [B, Hq, d] float32     out
 *   sel_blocks_opt   [B, Hkv, min(k2, nblk)] int32  out (optional): i2 ascending
 *   sel_channels_opt [B, Hkv, k1] int32             out (optional): i1 ascending
 *   block_scores_opt [B, Hkv, nblk] float32         out (optional): s1
 * nblk = ceil(n_tokens / block).  Requires 1 <= n_tokens <= kv_cap,
 * nblk <= nblk_cap (a multiple of 8), nblk <= 2^22, 1 <= k1 <= d, k2 >= 1,
 * G in {1, 2, 4, 8}.  Beyond 12288 pages per unit the page choice runs in a
 * launch of its own before the attention.
 */
rk_status rk_hsa_decode(const rk_shape* shape, const void* q, const void* k, const void* v,
                        int64_t kv_cap, const void* kmax, const void* kmin, int64_t nblk_cap,
                        int64_t n_tokens, int32_t block, int32_t k1, int32_t k2, float* out,
                        int32_t* sel_blocks_opt, int32_t* sel_channels_opt,
                        float* block_scores_opt, void* ws, size_t ws_bytes, rk_stream stream);

/*
 * rk_hsa_decode_ragged -- rk_hsa_decode where unit u has its own token count
 * unit_tokens[u] (device int32 [B, Hkv], each in [1, max_tokens]; values
 * outside are clamped into that range in-kernel), e.g. the kept_count of
 * rk_adakv_evict.  Each unit chooses min(k2, its pages) pages;
 * sel_blocks_opt [B, Hkv, min(k2, ceil(max_tokens / block))] holds -1 past a
 * unit's choice, block_scores_opt [B, Hkv, ceil(max_tokens / block)] is
 * valid for the unit's own pages.  max_tokens <= kv_cap and at most 12288
 * pages; workspace rk_hsa_workspace_bytes(shape, max_tokens, ...).
 */
rk_status rk_hsa_decode_ragged(const rk_shape* shape, const void* q, const void* k, const void* v,
                               int64_t kv_cap, const void* kmax, const void* kmin, int64_t nblk_cap,
                               const int32_t* unit_tokens, int64_t max_tokens, int32_t block,
                               int32_t k1, int32_t k2, float* out, int32_t* sel_blocks_opt,
                               int32_t* sel_channels_opt, float* block_scores_opt, void* ws,
                               size_t ws_bytes, rk_stream stream);

/*
 * rk_hsa_append_decode -- one decode step that appends its token first:
 * rk_append_kv(k_new, v_new at pos) followed by rk_hsa_decode over
 * n_tokens = pos + 1, in one call.  [RKV] method details, HSA step 1 (the
 * aux data follows every generated key) and steps 2-3.
 *
 *   q        [B, Hq, d]             decode queries
 *   k_new, v_new [B, Hkv, d]        the step's new key / value rows
 *   k, v     [B, Hkv, kv_cap, d]    compact cache, tokens 0..pos-1 valid;
 *                                   row pos is written
 *   kmax, kmin [B, Hkv, d, nblk_cap]  valid for tokens 0..pos-1; page
 *                                   pos/block is refreshed as rk_append_kv does
 *   out, sel_blocks_opt, sel_channels_opt, block_scores_opt, ws: as for
 *   rk_hsa_decode with n_tokens = pos + 1 (workspace from
 *   rk_hsa_workspace_bytes(shape, pos + 1, ...)).
 * Afterwards k, v, kmax, kmin equal the state rk_append_kv leaves, bit for
 * bit; the selections equal rk_hsa_decode's on that state, and out equals
 * it to float32 rounding.  Large batches run both in one launch (the new
 * token enters the attention from registers); small ones append with a
 * launch of its own first.  Requires 0 <= pos < kv_cap, k_new and v_new
 * 16-byte aligned, and everything rk_hsa_decode requires.
 */
rk_status rk_hsa_append_decode(const rk_shape* shape, const void* q, const void* k_new,
                               const void* v_new, void* k, void* v, int64_t kv_cap, int64_t pos,
                               void* kmax, void* kmin, int64_t nblk_cap, int32_t block, int32_t k1,
                               int32_t k2, float* out, int32_t* sel_blocks_opt,
                               int32_t* sel_channels_opt, float* block_scores_opt, void* ws,
                               size_t ws_bytes, rk_stream stream);

/*
 * rk_hsa_decode_noalloc -- rk_hsa_decode without a caller workspace and
 * without any allocation.  For callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as rk_hsa_decode (minus
 * ws / ws_bytes); the scratch space is a static device array of the library
 * (rk_hsa_decode_noalloc_max_bytes() bytes, 16 MiB, one copy per GPU, held
 * until the process ends).  A call whose workspace
 * (rk_hsa_workspace_bytes of the same arguments) exceeds that returns
 * RK_EWORKSPACE before touching the device.  Every call on one GPU shares
 * that GPU's scratch: calls that overlap on one GPU (two streams, two host
 * threads) race and give undefined results; serialise them.  Nothing in the
 * scratch needs to start at zero (every value a call reads it has written
 * earlier in the same call).  Calls no hipMalloc, hipFree or other
 * allocating routine.
 */
rk_status rk_hsa_decode_noalloc(const rk_shape* shape, const void* q, const void* k,
                                const void* v, int64_t kv_cap, const void* kmax, const void* kmin,
                                int64_t nblk_cap, int64_t n_tokens, int32_t block, int32_t k1,
                                int32_t k2, float* out, int32_t* sel_blocks_opt,
                                int32_t* sel_channels_opt, float* block_scores_opt,
                                rk_stream stream);

/* Size of rk_hsa_decode_noalloc's static scratch in bytes (16 MiB). */
size_t rk_hsa_decode_noalloc_max_bytes(void);

/*
 * Paged K/V pools.  The aifetchly guide's serving section ("Production
 * Deployment", Step 1: building the engine) serves RocketKV from a paged KV
 * cache of 64 tokens per block; here K and V of the whole batch live in one
 * pool of physical pages and a block table maps each sequence's logical
 * pages to them, so sequences grow a page at a time without reallocating or
 * copying.  The HSA aux data (Kmax/Kmin) stays dense per unit, as for the
 * contiguous cache (it is 2/block of the keys).
 *
 *   k_pool, v_pool [n_pages, Hkv, page_tokens, d]  bf16, one physical page
 *                  holds page_tokens consecutive tokens of one sequence for
 *                  every KV head
 *   block_table    [B, table_stride] int32 (device): logical page j of
 *                  sequence b is physical page block_table[b * table_stride
 *                  + j]; token n of sequence b, KV head h is pool row
 *                  (block_table[b, n / page_tokens] * Hkv + h) * page_tokens
 *                  + n % page_tokens.  Entries are clamped into [0, n_pages)
 *                  in-kernel (a bad entry gives wrong values, never an
 *                  out-of-bounds access).  The caller owns page allocation.
 * page_tokens is a power of two in [1, 32768]; n_pages * Hkv * page_tokens <
 * 2^31; every sequence of a call has the same n_tokens (at most table_stride
 * * page_tokens).  bf16 only (RK_EUNSUPPORTED otherwise).
 */
typedef struct {
  const int32_t* block_table;
  int64_t table_stride;
  int64_t n_pages;
  int32_t page_tokens;
} rk_paged_kv;

/*
 * rk_paged_write_kv -- copy rows [first_token, first_token + n_tokens) of a
 * contiguous cache k_src, v_src [B, Hkv, src_cap, d] (e.g. the compact cache
 * rk_snapkv_evict writes) to the same token positions of the paged pool.
 */
rk_status rk_paged_write_kv(const rk_shape* shape, const void* k_src, const void* v_src,
                           int64_t src_cap, int64_t first_token, int64_t n_tokens, void* k_pool,
                           void* v_pool, const rk_paged_kv* pages, rk_stream stream);

/*
 * rk_paged_build_aux -- rk_hsa_build_aux over the keys of a paged pool
 * (tokens 0..n_tokens-1 of every sequence; pages from first_token/block on
 * are (re)built).  [RKV] method details, HSA step 1.
 */
rk_status rk_paged_build_aux(const rk_shape* shape, const void* k_pool, const rk_paged_kv* pages,
                             int64_t n_tokens, int64_t first_token, int32_t block, void* kmax,
                             void* kmin, int64_t nblk_cap, rk_stream stream);

/*
 * rk_paged_append_kv -- rk_append_kv into a paged pool: token `pos` of every
 * sequence (its page must already be in the block table).
 */
rk_status rk_paged_append_kv(const rk_shape* shape, const void* k_new, const void* v_new,
                             void* k_pool, void* v_pool, const rk_paged_kv* pages, int64_t pos,
                             void* kmax, void* kmin, int64_t nblk_cap, int32_t block,
                             rk_stream stream);

/*
 * rk_paged_hsa_decode / rk_paged_hsa_append_decode -- rk_hsa_decode and
 * rk_hsa_append_decode over a paged pool: same selection and arithmetic (the
 * results equal the contiguous calls on the same tokens bit for bit), the
 * K/V rows addressed through the block table.  Workspace from
 * rk_hsa_workspace_bytes.
 */
rk_status rk_paged_hsa_decode(const rk_shape* shape, const void* q, const void* k_pool,
                              const void* v_pool, const rk_paged_kv* pages, const void* kmax,
                              const void* kmin, int64_t nblk_cap, int64_t n_tokens, int32_t block,
                              int32_t k1, int32_t k2, float* out, int32_t* sel_blocks_opt,
                              int32_t* sel_channels_opt, float* block_scores_opt, void* ws,
                              size_t ws_bytes, rk_stream stream);
rk_status rk_paged_hsa_append_decode(const rk_shape* shape, const void* q, const void* k_new,
                                     const void* v_new, void* k_pool, void* v_pool,
                                     const rk_paged_kv* pages, int64_t pos, void* kmax, void* kmin,
                                     int64_t nblk_cap, int32_t block, int32_t k1, int32_t k2,
                                     float* out, int32_t* sel_blocks_opt, int32_t* sel_channels_opt,
                                     float* block_scores_opt, void* ws, size_t ws_bytes,
                                     rk_stream stream);

/*
 * rk_hsa_decode_mt -- RocketKV-MT decode: HSA over a candidate subset of a
 * full, never-evicted cache.
 * [RKV] method details, RocketKV-MT: every token stays in memory, but stage 2
 * chooses only among the N tokens that stage 1 kept for this turn.  Pages are
 * formed over the ascending candidate list: page token n is key/value row
 * cand_idx[n] of the full cache, and kmax/kmin must have been built by
 * rk_hsa_build_aux with idx_opt = cand_idx.  Otherwise identical to
 * rk_hsa_decode with n_tokens = n_cand.
 *
 *   k, v     [B, Hkv, kv_cap, d]    full cache
 *   cand_idx [B, Hkv, cand_stride]  candidate rows, entries 0..n_cand-1 used,
 *                                   each in [0, kv_cap)
 */
rk_status rk_hsa_decode_mt(const rk_shape* shape, const void* q, const void* k, const void* v,
                           int64_t kv_cap, const int32_t* cand_idx, int64_t cand_stride,
                           int64_t n_cand, const void* kmax, const void* kmin, int64_t nblk_cap,
                           int32_t block, int32_t k1, int32_t k2, float* out,
                           int32_t* sel_blocks_opt, int32_t* sel_channels_opt,
                           float* block_scores_opt, void* ws, size_t ws_bytes,
                           rk_stream stream);

/*
 * Dynamic-selection methods compared with HSA on the same inputs.
 * [RKV] background (Exact-TopK, the ideal top-k attention), method details
 * (limits of existing dynamic selection: Quest's per-page element-wise
 * min/max along the sequence, SparQ's head-dimension sparsity; the token
 * budget t = S / c), appendix A.3 (for Quest and SparQ the budget is shared
 * evenly between the approximate scoring and the sparse attention; Quest
 * chooses per attention group on accumulated scores) and B.1.1 (standalone
 * HSA against Quest and SparQ).  Every method scores pages, keeps the
 * top-k2 (ties to the lower page, ascending) and attends exactly over their
 * tokens, as rk_hsa_decode does:
 *   RK_SEL_HSA   Algorithm 1 (k1 = channels, pages of `page` tokens)
 *   RK_SEL_QUEST page score sum over all d channels of max(q_bar_i Kmax_i,
 *                q_bar_i Kmin_i), the bound of every token's accumulated
 *                logit q_bar . k in the page (equals HSA with k1 = d)
 *   RK_SEL_SPARQ token score over the `channels` channels of largest
 *                sum_g |q_g|: sum_i q_bar_i k_n,i (pages of one token)
 *   RK_SEL_EXACT the exact accumulated logit q_bar . k_n of every token, over
 *                the key rows (pages of one token, every channel)
 * with q_bar = sum_g q_g over the group's heads (float32, g ascending) and
 * every score a float32 sum in ascending channel order, one rounded multiply
 * and one rounded add per term.
 */
typedef enum {
  RK_SEL_HSA = 0,
  RK_SEL_QUEST = 1,
  RK_SEL_SPARQ = 2,
  RK_SEL_EXACT = 3
} rk_select_method;

typedef struct {
  int32_t page;        /* tokens per page (1: token-level selection)          */
  int32_t channels;    /* channels read per page when scoring (k1)            */
  int32_t k2;          /* pages attended                                      */
  int64_t attn_tokens; /* min(S, k2 * page) tokens attended                   */
  double budget_t;     /* t = S / c                                           */
  double est_pairs;    /* scoring traffic in KV pairs: channels values per
                          page over ceil(S / page) pages, 2d values per pair  */
} rk_select_plan_out;

/*
 * rk_select_plan -- page size, channels and attended pages of a method at
 * total compression c with estimation and attention sharing t evenly
 * ([RKV] A.3; the split inside HSA with all of c in stage 2):
 *   HSA   page = ceil(sqrt(c)), channels = round(d * page / c) in [1, d]
 *   QUEST page = ceil(c), channels = d (d of its 2d aux values per page)
 *   SPARQ page = 1, channels = round(d / c) in [1, d]
 *   EXACT page = 1, channels = d, k2 = ceil(t) (the ideal: no estimation
 *         cost counted against the budget)
 * and k2 = ceil((t / 2) / page) pages for the first three.  Host math only.
 * RK_EINVAL on c < 1, seq_len < 1, head_dim < 1, an unknown method or NULL out.
 */
rk_status rk_select_plan(rk_select_method method, double c, int64_t seq_len, int32_t head_dim,
                         rk_select_plan_out* out);

/*
 * rk_select_decode -- one decode step of a selection method (see above).
 *   q, k, v, kv_cap, n_tokens, out: as for rk_hsa_decode (pages are `page`
 *                                   consecutive tokens of the cache)
 *   kmax, kmin [B, Hkv, d, nblk_cap]  HSA and QUEST: from rk_hsa_build_aux in
 *                                   pages of `page` tokens.  SPARQ: kmax from
 *                                   rk_hsa_build_aux with block 1 (the keys
 *                                   channel-major), kmin ignored.  EXACT:
 *                                   both ignored (may be NULL); the scores
 *                                   come from the key rows.
 *   channels                        HSA/SPARQ: channels scored (1..d);
 *                                   QUEST/EXACT: must be d
 *   sel_opt [B, Hkv, min(k2, pages)] out (optional): chosen pages ascending
 *   scores_opt [B, Hkv, pages] float32 out (optional): the page scores
 *   ws      workspace of rk_hsa_workspace_bytes(shape, n_tokens, page,
 *           channels, k2) bytes
 * SPARQ and EXACT require page = 1.  More than 12288 pages per unit take a
 * separate page-choice launch; at most 2^22 pages.  Errors as rk_hsa_decode.
 */
rk_status rk_select_decode(const rk_shape* shape, rk_select_method method, const void* q,
                           const void* k, const void* v, int64_t kv_cap, const void* kmax,
                           const void* kmin, int64_t nblk_cap, int64_t n_tokens, int32_t page,
                           int32_t channels, int32_t k2, float* out, int32_t* sel_opt,
                           float* scores_opt, void* ws, size_t ws_bytes, rk_stream stream);

/*
 * Kernel timing (measurement support, not part of the method).
 * Between rk_profile_begin() and rk_profile_end() every kernel the library
 * launches is bracketed by a pair of HIP events recorded on the stream it is
 * launched on.  rk_profile_end() waits for those events, stops recording and
 * writes, per kernel name in order of first launch, the launch count and the
 * summed event-to-event time into out[0 .. *n_out) (at most `cap` entries).
 * Process-wide; not meant to be used concurrently from several threads.
 * RK_EDEVICE if an event call fails, RK_EINVAL on NULL arguments.
 */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
} rk_kernel_time;

rk_status rk_profile_begin(void);
rk_status rk_profile_end(rk_kernel_time* out, int32_t cap, int32_t* n_out);

/* Static name of a status code. */
const char* rk_status_string(rk_status status);

/* Thread-local description of the last error on this thread ("" if none). */
const char* rk_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ROCKETKV_H_ */

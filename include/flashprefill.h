/*
 * flashprefill.h -- C ABI of the MI355X (gfx950) block-sparse causal prefill
 * attention library (FlashPrefill method).
 *
 * The method runs in two stages (FlashPrefill V2 paper reading, section 四):
 * an indexing stage that pools K/V per 128-token block, scores every query
 * block against the pooled keys and keeps the blocks whose score reaches
 * alpha times the row maximum plus forced sink and local blocks, emitting
 * compact per-row index lists; and an attention stage that walks only the
 * listed blocks of a paged KV cache and folds a block-mean correction for
 * every pruned block into the same softmax.
 *
 * Three calls implement the path, in order:
 *   fp_discover          pooling + pooled block scores    (indexing, part 1)
 *   fp_select            threshold + compaction to CSR     (indexing, part 2)
 *   fp_sparse_attn_paged sparse paged attention + correction (attention)
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer, except fp_problem itself and
 *     fp_problem.cu_seqlens_host, which live in host memory.
 *   - The caller owns and allocates every buffer, including the workspace
 *     (size from fp_workspace_bytes).  The library allocates nothing.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t passed as
 *     void*; NULL = the default stream).  They never synchronise the host.
 *   - Return value: FP_OK (0) on success, a negative fp_status otherwise.  On
 *     error nothing is launched and fp_last_error() returns a message
 *     (thread-local).  Faults inside kernels (e.g. an out-of-range page id)
 *     surface at the caller's next synchronisation.
 *   - Results are deterministic: identical inputs give bit-identical outputs.
 *   - Shapes: head_dim = 128 and block_size = 128.  Sequence s has
 *     q_s = cu_seqlens[s+1] - cu_seqlens[s] query tokens, the positions
 *     c_s .. c_s + q_s - 1 of the sequence, where c_s = ctx_lens[s] is the
 *     number of tokens already in the KV cache before them (0 when ctx_lens
 *     is NULL: a whole prompt; else a multiple of 128: chunked prefill, where
 *     each chunk redoes the block selection for its own query blocks against
 *     all cached keys; "長文本推理越來越長但你的顯卡等不起…FlashPrefill V2",
 *     chunked-prefill (分塊預填充) passage).  Its KV cache holds
 *     len_s = c_s + q_s tokens: nk_s = ceil(len_s / 128) key blocks and
 *     nq_s = nk_s - c_s / 128 query blocks (I = c_s/128 .. nk_s - 1).
 *     T = cu_seqlens[num_seqs] query tokens, N = sum_s nk_s key blocks,
 *     NQ = sum_s nq_s query blocks, n_max = max_s nk_s.  Without ctx_lens,
 *     NQ = N.
 *   - Layouts (row-major, innermost last):
 *       q          [T, Hq, 128]                      dtype qk_dtype
 *       k_cache    [num_pages, page_size, Hkv, 128]  dtype qk_dtype
 *       v_cache    [num_pages, page_size, Hkv, 128]  dtype v_dtype
 *       page_table [num_seqs, max_pages_per_seq] int32: token p of sequence
 *                  s lives at page page_table[s][p / page_size], slot
 *                  p % page_size (FlashPrefill V2 article, paged KV section:
 *                  page base from the table plus in-page offset).
 *       k_mean, v_mean [Hkv, N, 128] float64 (key block J of sequence s at
 *                  row kboff_s + J, kboff_s = sum of nk over earlier
 *                  sequences)
 *       block_scores   [Lo, NQ, n_max] float32 (query block I of sequence s
 *                  at row qboff_s + I - c_s/128, qboff_s = sum of nq over
 *                  earlier sequences; entry J for J <= I)
 *       row_ptr    [Lo * NQ + 1] int32, rows ordered (list owner, sequence,
 *                  query block); col_idx int32 block indices inside the
 *                  sequence, ascending per row.
 *     Lo, the list owners: Lo = Hkv (one index list per KV group, shared by
 *     its Hq / Hkv query heads: the default) or Lo = Hq with head_lists = 1
 *     (one list per query head, scored from that head's rows alone and used
 *     by that head alone; owner hq reads KV head hq / (Hq / Hkv)).  This is
 *     the reading of the V2 article's CSR index-memory figure, which fits
 *     per-query-head lists; PackGQA tiles suggest per-group lists.
 *       out        [T, Hq, 128] dtype out_dtype
 *       lse        [Hq, T] float32 (natural log), optional
 *   - Query head hq reads KV head hq / (Hq / Hkv).
 *   - fp32 Q/K/V are rounded to bf16 (nearest even) when the kernels load
 *     them; e4m3 values are the OCP E4M3FN codes times a per-head fp32 scale.
 */
#ifndef FLASHPREFILL_H
#define FLASHPREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP_F32 = 0,
  FP_BF16 = 1,
  FP_E4M3 = 2
} fp_dtype;

typedef enum {
  FP_OK = 0,
  FP_ERR_INVALID = -1,      /* a NULL pointer, a bad size or an inconsistent shape */
  FP_ERR_UNSUPPORTED = -2,  /* head_dim / block_size / dtype combination not built */
  FP_ERR_WORKSPACE = -3,    /* ws_bytes smaller than fp_workspace_bytes(...)        */
  FP_ERR_CAPACITY = -4,     /* col_capacity smaller than fp_csr_capacity(...)       */
  FP_ERR_HIP = -5           /* a HIP launch error                                   */
} fp_status;

typedef enum {
  FP_WS_DISCOVER = 0,
  FP_WS_SELECT = 1,
  FP_WS_ATTN = 2,
  FP_WS_DENSE = 3
} fp_workspace_kind;

typedef struct {
  int32_t num_seqs;                /* >= 1                                            */
  const int32_t* cu_seqlens_host;  /* HOST   [num_seqs + 1], cu[0] = 0, nondecreasing */
  const int32_t* cu_seqlens_dev;   /* DEVICE [num_seqs + 1], same values              */
  int32_t num_q_heads;             /* Hq, a multiple of Hkv, Hq / Hkv <= 16            */
  int32_t num_kv_heads;            /* Hkv >= 1                                        */
  int32_t head_dim;                /* must be 128                                     */
  int32_t block_size;              /* must be 128                                     */
  int32_t page_size;               /* divides 128, or is a multiple of 128            */
  int32_t max_pages_per_seq;       /* >= ceil(max_s len_s / page_size)                */
  int64_t num_pages;               /* pages in k_cache / v_cache; every page id in the
                                      table (for existing tokens) must be < num_pages */
  const int32_t* page_table_dev;   /* DEVICE [num_seqs, max_pages_per_seq]            */
  int32_t qk_dtype;                /* fp_dtype of q and k_cache                       */
  int32_t v_dtype;                 /* fp_dtype of v_cache                              */
  int32_t out_dtype;               /* FP_F32 or FP_BF16                               */
  const float* q_scale_dev;        /* DEVICE [Hq]  (qk_dtype == FP_E4M3), else NULL   */
  const float* k_scale_dev;        /* DEVICE [Hkv] (qk_dtype == FP_E4M3), else NULL   */
  float softmax_scale;             /* logit scale; <= 0 selects 1/sqrt(head_dim)      */
  const int32_t* ctx_lens_host;    /* HOST   [num_seqs] cached prefix per sequence, a
                                      multiple of 128, or NULL for none             */
  const int32_t* ctx_lens_dev;     /* DEVICE [num_seqs], same values (NULL iff host is) */
  int32_t attn_splits;             /* KV split of fp_sparse_attn_paged: 0 = automatic,
                                      1 = never split, n = split every row into n
                                      parts (at most 8)                              */
  int32_t head_lists;              /* 0: one index list per KV head (rows (kv head,
                                      seq, block)); 1: one per query head (rows
                                      (q head, seq, block)); every call of one
                                      pass must use the same value               */
} fp_problem;

/* Supported dtype combinations (qk, v): (F32, F32), (BF16, BF16), (E4M3, BF16);
 * out_dtype F32 or BF16 with any of them.  Longest sequence <= 8192 blocks.
 * row_ptr / col_idx offsets are int32, so Lo times the number of causal
 * blocks of the query blocks (fp_csr_capacity) must not exceed INT32_MAX;
 * larger batches are rejected with FP_ERR_UNSUPPORTED by every call. */

/* ---- size queries (host only, read cu_seqlens_host / ctx_lens_host) ---- */
int64_t fp_num_blocks(const fp_problem* p);       /* N = sum_s nk_s (pooled rows) */
int64_t fp_num_query_blocks(const fp_problem* p); /* NQ = sum_s nq_s              */
int32_t fp_max_blocks(const fp_problem* p);       /* n_max                        */
int64_t fp_num_rows(const fp_problem* p);         /* Lo * NQ (CSR rows)           */
int64_t fp_scores_elems(const fp_problem* p);     /* Lo * NQ * (n_max + 1): the
                                                     scores, then one error bound
                                                     per score row               */
int64_t fp_csr_capacity(const fp_problem* p);     /* Lo * sum over query blocks of
                                                     (I + 1): every causal block kept
                                                     (<= INT32_MAX)               */
/* Bytes of the workspace of kind `which` (fp_workspace_kind).  A workspace
 * holds intermediate data and counters of one call: calls that may run at the
 * same time (different streams) need workspaces of their own. */
size_t fp_workspace_bytes(const fp_problem* p, int32_t which);
const char* fp_status_string(int32_t status);
const char* fp_last_error(void);

/*
 * fp_discover -- block pooling and pooled block scores.
 *
 * Pooling (FlashPrefill summary "长上下文加速 28 倍", 3.1 key pooling; V2 paper
 * reading 4.1): k_mean[h][kboff_s + J] = mean of the keys of block J of
 * sequence s for KV head h (n_J = tokens actually in the block); v_mean the
 * same for values.  The means are summed and divided in float64, i.e. they
 * are the exact block means of the stored values up to float64 rounding.
 *
 * Scores (same summary, 3.1 query pooling + global re-weighting): for list
 * owner h (KV head h; with head_lists, query head h) and query block I, let
 * rows(I) be every (query head of h's group, or query head h alone with
 * head_lists; query token of block I) and x_rJ = softmax_scale * q_r . kbar_J
 * for J <= I, kbar of the owner's KV head (key blocks of the cached prefix
 * included).  Then
 *     block_scores[h][qboff_s + I - c_s/128][J] = M_IJ + ln S_IJ,
 *     M_IJ = max_r x_rJ,  S_IJ = sum_r exp(x_rJ - M_IJ),
 * the log of the max-normalised exp-sum.  Re-weighting a row against its top
 * block is a subtraction of max_J of this value (done by fp_select).
 * Entries with J > I are left unspecified.
 *
 * The dot products run on bf16 MFMA against s_J = bf16(c kbar_J), the exact
 * mean scaled by c = softmax_scale * log2(e) in float64 and rounded once,
 * with fp32 accumulation (log2-domain logits).  After the Lo * NQ * n_max
 * scores, block_scores holds one float per score row (same row order): a
 * bound E on how far the dot products can move any entry of the row from
 * exact arithmetic,
 *     E = ln(2) * max_r |q_r|_2 *
 *         max_{J<=I} (|c kbar_J - s_J|_2 + 2^-15 |s_J|_2)
 * (Cauchy-Schwarz on the rounding of c kbar_J, plus twice the worst case of
 * an fp32 sum of 128 exact products with any faithful rounding; |q_r|
 * includes q_scale for e4m3; a log-sum-exp over rows moves by at most its
 * largest shift), which fp_select uses.  The fp32 statistics (exp2 / log2 /
 * sums) add an absolute error below 1e-4 and a relative one below 2^-19 of
 * |L| on top of E.
 *
 * q, k_cache, v_cache: inputs (layouts above).  k_mean, v_mean, block_scores:
 * outputs.  ws: FP_WS_DISCOVER workspace.
 */
int fp_discover(const fp_problem* p, const void* q, const void* k_cache,
                const void* v_cache, double* k_mean, double* v_mean,
                float* block_scores, void* ws, size_t ws_bytes, void* stream);

/*
 * fp_select -- max-based dynamic threshold, forced blocks, compaction.
 *
 * Row (h, s, I) keeps block J <= I iff
 *     J < ceil(sink_tokens / 128)                 (attention sinks), or
 *     I - J < max(1, ceil(local_tokens / 128))    (local window; the diagonal
 *                                                  block is always kept), or
 *     exp(L_IJ - max_{J' <= I} L_IJ') >= alpha    (threshold alpha * max score,
 *                                                  FlashPrefill summary 3.2)
 * where L = block_scores.  alpha <= 0 keeps every causal block.
 * Kept indices are written ascending (compaction, same summary 3.3).
 *
 * Because block_scores comes from a bf16 fast path, every entry whose fast
 * value lies within 2 E + stat(l) + stat(lmax) of the threshold (E = the
 * row's bound stored after the scores, stat(x) = 1e-3 + 2^-17 |x| an
 * allowance of several times the fp32 statistics' error, l the entry and
 * lmax the row maximum, natural-log units), together with the row's
 * candidates for the maximum (within the same guard of it), is re-evaluated
 * in float64 from q and the float64 means k_mean before it is decided.
 * Every other decision follows from the bound.  So the lists equal those of
 * exact arithmetic on the stored q and the exact block means, except for
 * entries whose exact normalised score is within float64 rounding (about
 * 1e-12 relative) of alpha.
 *
 * q, k_mean, block_scores: inputs from the same problem.  row_ptr
 * [fp_num_rows + 1], col_idx [col_capacity]: outputs.  col_capacity must be
 * >= fp_csr_capacity(p).  ws: FP_WS_SELECT workspace.
 */
int fp_select(const fp_problem* p, const void* q, const double* k_mean,
              const float* block_scores, float alpha, int32_t sink_tokens,
              int32_t local_tokens, int32_t* row_ptr, int32_t* col_idx,
              int64_t col_capacity, void* ws, size_t ws_bytes, void* stream);

/*
 * fp_select_noalloc -- fp_select without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, decisions, outputs and errors as fp_select, bit-identical
 * results; the FP_WS_SELECT workspace is instead a static device array of
 * 8 MiB inside the library (one per device, held until the process ends;
 * its address is looked up on the first call on each device).  A batch whose
 * FP_WS_SELECT workspace exceeds 8 MiB is rejected with FP_ERR_WORKSPACE
 * before anything runs (the benchmark shapes need 0.5-2 MiB: 4 bytes per 32
 * key blocks per CSR row, plus the row counts).  Nothing is allocated or
 * freed, and no memset is issued: the kernels overwrite everything they read
 * from the array.  Every call on one device shares the array, so calls that
 * can overlap on a device (on different streams, or from several threads)
 * race and give unspecified lists; calls in one stream order are safe.
 */
int fp_select_noalloc(const fp_problem* p, const void* q, const double* k_mean,
                      const float* block_scores, float alpha, int32_t sink_tokens,
                      int32_t local_tokens, int32_t* row_ptr, int32_t* col_idx,
                      int64_t col_capacity, void* stream);

/*
 * fp_select_topk / fp_select_topp -- ranked block selection, the strategies
 * of the prior methods that the max-based threshold replaces (FlashPrefill
 * summary "长上下文加速 28 倍", section 二: top-k needs a sort, top-p a
 * running probability sum; its ablation 4.4 compares them with fp_select),
 * for comparisons on the same scores.
 *
 * Row (h, s, I) ranks its causal blocks J <= I by block_scores (descending,
 * ties toward the lower J) and keeps the forced blocks (sinks and local
 * window, as in fp_select) plus
 *   top-k: the first top_k ranked blocks that are not forced (all of them if
 *          fewer), or
 *   top-p: the shortest ranked prefix of all causal blocks whose share of
 *          sum_J e^{L_IJ} reaches top_p (top_p <= 0: forced blocks only).
 * Unlike fp_select, the decisions use the fp32 scores as given, without a
 * float64 re-check: blocks whose scores lie within the fast path's error of
 * the cut may rank differently from exact arithmetic.  Outputs, capacity and
 * workspace (FP_WS_SELECT) as for fp_select; q and k_mean are not needed.
 */
int fp_select_topk(const fp_problem* p, const float* block_scores, int32_t top_k,
                   int32_t sink_tokens, int32_t local_tokens, int32_t* row_ptr,
                   int32_t* col_idx, int64_t col_capacity, void* ws, size_t ws_bytes,
                   void* stream);
int fp_select_topp(const fp_problem* p, const float* block_scores, float top_p,
                   int32_t sink_tokens, int32_t local_tokens, int32_t* row_ptr,
                   int32_t* col_idx, int64_t col_capacity, void* ws, size_t ws_bytes,
                   void* stream);

/*
 * fp_sparse_attn_paged -- sparse causal attention over the listed blocks with
 * block-mean correction.
 *
 * For query head hq, query token at position p (counted from the start of
 * the sequence, cached prefix included) of block I of sequence s, and the
 * list K(h, s, I) = col_idx[row_ptr[r] .. row_ptr[r+1]) of row r = (h, s, I),
 * h = hq / (Hq / Hkv) its KV head, or h = hq with head_lists:
 *   E = { tokens j <= p of the listed blocks },  y_j = softmax_scale * q . k_j
 *   C = { J <= I not listed } if mean_correction, else empty,
 *       z_J = softmax_scale * q . kbar_J + ln n_J,  value vbar_J
 *   out = (sum_E e^{y_j} v_j + sum_C e^{z_J} vbar_J) / (sum_E e^{y_j} + sum_C e^{z_J})
 *   lse = ln(sum_E e^{y_j} + sum_C e^{z_J})
 * (V2 paper reading 4.1: each pruned block contributes n_J e^{q.kbar} vbar to
 * the numerator and n_J e^{q.kbar} to the denominator.)  Every list must
 * contain its diagonal block I; listed blocks must be <= I, ascending.
 *
 * The g = Hq / Hkv query heads of a KV head are packed into shared K/V tiles
 * (PackGQA, V2 paper reading 4.2(1)); K/V tiles are gathered through the page
 * table without a contiguous copy (4.3).  QK^T runs on bf16 MFMA (fp8 e4m3
 * MFMA when qk_dtype == FP_E4M3), PV on bf16 MFMA; softmax in fp32.  Rows
 * are launched last query block first (the work of a row grows with its
 * position: its pooled tiles and, on average, its list), KV heads
 * interleaved, the g/2 workgroups of a row together on one XCD.
 *
 * KV split ("長文本推理越來越長但你的顯卡等不起…FlashPrefill V2", KV-split
 * load-balancing passage: work is divided by the selected blocks, not by
 * position): when a launch has at most 128 (row, head pair) workgroups
 * (small chunks) and attn_splits == 0, each row's tile list (listed blocks,
 * then correction tiles) is cut into floor(256 / workgroups) contiguous parts
 * (at most 8) with equal tile counts, each part run by its own workgroup,
 * and a combine pass merges the parts by their log-sum-exp.  The split changes only the rounding of a
 * row, never which keys it sees; attn_splits = 1 makes a row's result
 * independent of the rest of the batch (no split ever).  The split count is
 * a function of the descriptor, so fp_workspace_bytes(FP_WS_ATTN) covers the
 * partial outputs.  A list entry
 * outside [0, I] or a list longer than I + 1 gives unspecified output for
 * that row but no out-of-bounds access.
 *
 * q, k_cache, v_cache, row_ptr, col_idx, k_mean, v_mean: inputs (k_mean /
 * v_mean may be NULL when mean_correction == 0).  out: output.  lse: output
 * or NULL.  ws: FP_WS_ATTN workspace.
 */
int fp_sparse_attn_paged(const fp_problem* p, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* row_ptr,
                         const int32_t* col_idx, const double* k_mean,
                         const double* v_mean, int32_t mean_correction, void* out,
                         float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * fp_dense_attn_paged -- dense causal attention over the same paged cache, on
 * the same kernel: every causal block 0..I of each query block, in order,
 * with no index lists and no mean correction.  It is the aligned dense
 * baseline of the sparse call (FlashPrefill V2 paper reading, section 五:
 * the sparse operator's speed-up is quoted against a dense kernel built on
 * the same stack; 5.3 and 5.6 state the ratios), and equals
 * fp_sparse_attn_paged with every causal block listed and mean_correction = 0.
 *
 * For query head hq and query token at position p (KV head hq / (Hq / Hkv)):
 *   out = sum_{j <= p} e^{y_j} v_j / sum_{j <= p} e^{y_j},
 *   lse = ln sum_{j <= p} e^{y_j},  y_j = softmax_scale * q . k_j
 * (keys of the cached prefix included).  The g query heads of a KV head are
 * packed into shared K/V tiles whatever head_lists says.  Small launches
 * split rows as fp_sparse_attn_paged does.  q, k_cache, v_cache: inputs;
 * out: output; lse: output or NULL; ws: FP_WS_DENSE workspace.
 */
int fp_dense_attn_paged(const fp_problem* p, const void* q, const void* k_cache,
                        const void* v_cache, void* out, float* lse, void* ws,
                        size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASHPREFILL_H */

/*
 * libfocus: the token-eviction hot path of FOCUS for block-diffusion LLM
 * decoding, as hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * Sources for what each call computes: the pith.science review page of
 * "FOCUS: DLLMs Know How to Tame Their Compute Bound" (arXiv 2601.23278),
 * cited as "Pith page", and the sciencestack.ai summary page of the same
 * paper, cited as "ScienceStack page".
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every array pointer is caller-owned DEVICE memory, contiguous,
 *    row-major and 16-byte aligned. The library keeps no pointer after a
 *    call returns and allocates no device memory; its only global state is
 *    the static scratch of focus_block_attn_importance_noalloc.
 *  - Outputs must not alias inputs.
 *  - Each call only enqueues kernels on `stream` (a hipStream_t; NULL is the
 *    default stream) and never synchronises. Device-side faults surface at
 *    the caller's next synchronisation. No call allocates, sets memory or
 *    synchronises, so a sequence of calls on a capturing stream can be
 *    recorded into a HIP graph (the workspace, when one is needed, must
 *    then outlive the graph); replays give the same bits as the calls.
 *  - Device arrays (cu_prefix, k_keep, cu_ret, idx, keep) are never read on
 *    the host. Host integers documented as promises (max_prefix, n_ret,
 *    max_ret) must be true upper bounds / counts; the kernels clamp where
 *    stated and otherwise trust them.
 *  - Host-visible arguments are checked before any launch; a failed check
 *    enqueues nothing and returns an error code. focus_last_error() then
 *    gives a thread-local description. No C++ exception crosses this ABI.
 *  - Element types: FOCUS_BF16 tensors hold bfloat16, FOCUS_F32 float32.
 *    Accumulation is float32 in both cases; O is rounded to the tensor type
 *    with round-to-nearest-even. Importances and lse are float32.
 *  - Supported shapes: 1 <= B <= 128, head_dim d in {64, 128}, Hq a
 *    multiple of Hkv. Query head h reads KV head h / (Hq / Hkv).
 *  - Calls are reentrant and thread-safe, except that calls of
 *    focus_block_attn_importance_noalloc that overlap in time on one GPU
 *    share its static scratch and race.
 */
#ifndef FOCUS_H_
#define FOCUS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FOCUS_OK = 0,
  FOCUS_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misaligned pointer */
  FOCUS_ERR_UNSUPPORTED = 2,  /* valid but not built: d, dtype, Hq % Hkv   */
  FOCUS_ERR_WORKSPACE = 3,    /* workspace smaller than the queried size    */
  FOCUS_ERR_HIP = 4           /* a HIP runtime call or launch failed        */
} focus_status;

typedef enum { FOCUS_F32 = 0, FOCUS_BF16 = 1 } focus_dtype;

/* Library version string, e.g. "libfocus 0.1.0 gfx950". Static storage. */
const char* focus_version(void);

/* Name of a status code. Static storage. */
const char* focus_status_string(focus_status s);

/* Thread-local description of the last non-OK status returned on this
 * thread ("" if none). Valid until the next libfocus call on the thread. */
const char* focus_last_error(void);

/*
 * Visiting order of the sequences for the attention calls of one step:
 * longest prefix first, equal lengths by lower index. The attention work of
 * a sequence grows with its prefix length, and visiting the long ones
 * first keeps every compute unit streaming until the end of the launch.
 * The pages' scheduler prepares per-sequence metadata for each step
 * before the kernels run (Pith page, scheduler appendix fragments); this
 * call is that step for the work order, done on the device from cu_prefix.
 *
 *  cu_prefix   device int32 [batch+1] as in focus_block_attn_importance.
 *              Only the differences cu_prefix[b+1] - cu_prefix[b] are
 *              used; they are compared as signed int32, so a non-monotone
 *              array (negative lengths) still yields a permutation, with
 *              those sequences last.
 *  order       device int32 [batch] output, a permutation of 0..batch-1;
 *              nothing past order[batch-1] is written.
 * Batches above 16384 keep their natural order.
 * Errors: INVALID_ARG (batch < 1, NULL pointer), HIP.
 */
focus_status focus_schedule(int batch, const int32_t* cu_prefix, int32_t* order,
                            void* stream);

/* Workspace bytes that focus_block_attn_importance needs for these sizes.
 * Writes *bytes; never fails for valid sizes. */
focus_status focus_block_attn_importance_workspace(
    int batch, int B, int Hq, int Hkv, int d, int max_prefix, size_t* bytes);

/*
 * Block attention with importance (one layer).
 *
 * Follows the Pith page, "What carries the argument": the importance I_j of
 * block token j is the sum, over all B block queries, of the softmax
 * attention weight that token j receives; the softmax runs along each query
 * row (Referee Report, minor comment on Eq. 2). Every block query attends
 * to its sequence's P_b prefix tokens and to all B block tokens, with no
 * mask. Layers 0 and 1 are each one call ("The pith": the first two layers
 * run on the whole block).
 *
 * Per sequence b (block rows b*B .. b*B+B-1, prefix tokens
 * cu_prefix[b] .. cu_prefix[b+1]-1) and query head h with KV head
 * g = h / (Hq/Hkv):
 *    s_ij  = scale * q_i . k_j   over the P_b prefix keys then the B block keys
 *    lse_i = log sum_j exp(s_ij)                       (natural log)
 *    out_i = sum_j exp(s_ij - lse_i) v_j
 *    imp[b,h,j] = sum_{i<B} exp(s_i,(P_b+j) - lse_i)   for block token j < B
 *
 *  dt          FOCUS_BF16 or FOCUS_F32 (type of q, k_*, v_*, out).
 *  scale       softmax scale; <= 0 means 1/sqrt(d).
 *  q           [batch*B, Hq, d]
 *  k_blk,v_blk [batch*B, Hkv, d]   the block tokens' keys / values
 *  k_cache,v_cache [cu_prefix[batch], Hkv, d]  packed prefix KV, sequence
 *              after sequence
 *  cu_prefix   device int32 [batch+1], cu_prefix[0] = 0, non-decreasing.
 *  order       device int32 [batch]: the order in which sequences are
 *              visited, a permutation of 0..batch-1 (focus_schedule writes
 *              the longest-prefix-first one). Results do not depend on it;
 *              only the run time does. Entries are clamped to [0, batch).
 *              NULL: the call writes that order into the workspace first
 *              (one extra kernel launch).
 *  max_prefix  host promise: max_b P_b (sizes the launch).
 *  out         [batch*B, Hq, d] attention output (type dt), or NULL for
 *              importance only: then v_blk and v_cache are not read (may
 *              be NULL) and no P V product is formed, while imp and lse
 *              are the same values, bit for bit, as with out given. This
 *              matches where the Pith page (Figures, Fig. 5 caption) puts
 *              the eviction: right after layer 1's Q/K projections, so
 *              layer 1 needs no attention output.
 *  imp         float32 [batch, Hq, B] importance of the block columns.
 *  lse         float32 [batch, Hq, B] natural-log row lse, or NULL.
 *  workspace   device scratch of at least the queried size, needed only
 *              when order is NULL; its contents on entry do not matter.
 * Errors: INVALID_ARG (null required pointer, batch < 1, B not in [1,128],
 * Hq or Hkv < 1, Hq > 4096, max_prefix < 0, misaligned pointer),
 * UNSUPPORTED (d not 64/128, bad dt, Hq % Hkv != 0), WORKSPACE, HIP.
 */
focus_status focus_block_attn_importance(
    focus_dtype dt, int batch, int B, int Hq, int Hkv, int d, float scale,
    const void* q, const void* k_blk, const void* v_blk,
    const void* k_cache, const void* v_cache, const int32_t* cu_prefix,
    const int32_t* order, int max_prefix, void* out, float* imp, float* lse,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * focus_block_attn_importance with order = NULL, for callers that cannot
 * allocate device memory or hand in a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). Same
 * computation and outputs, bit for bit; arguments as there, without order,
 * workspace and workspace_bytes.
 *
 * The longest-prefix-first visiting order this call computes goes to a
 * static device array inside the library instead of a workspace: at most
 * 65536 sequences (256 KiB of int32), held on every GPU the library runs
 * on until the process ends. The call allocates nothing (no hipMalloc, no
 * hipFree). The scratch of the stream's device is looked up once, on the
 * first call on that device. Every call on one GPU shares that GPU's
 * scratch and overwrites it: two calls that overlap in time on the same
 * GPU (different streams, or threads without ordering) race, so
 * concurrent callers must serialise, e.g. by using one stream.
 * Errors: as focus_block_attn_importance; WORKSPACE for batch > 65536;
 * HIP if the stream's device or the scratch address cannot be obtained.
 */
focus_status focus_block_attn_importance_noalloc(
    focus_dtype dt, int batch, int B, int Hq, int Hkv, int d, float scale,
    const void* q, const void* k_blk, const void* v_blk,
    const void* k_cache, const void* v_cache, const int32_t* cu_prefix,
    int max_prefix, void* out, float* imp, float* lse, void* stream);

/*
 * focus_block_attn_importance over a paged prefix KV cache: the same
 * computation and outputs (bit for bit), with the prefix keys/values held
 * in fixed-size pages, the cache form of the serving engine the pages'
 * system is built into (LMDeploy: Pith page, Referee Report; PagedAttention
 * is listed among the works it builds on on the mlsanity page, "Builds
 * on").
 *
 *  k_pages, v_pages  [n_pages, page_size, Hkv, d] page pools (type dt).
 *  page_table  device int32 [batch, pages_per_seq]: token t of sequence b
 *              is slot t % page_size of page page_table[b][t / page_size].
 *              Entries past a sequence's last page are not read.
 *  page_size   tokens per page, a positive multiple of 32.
 *  pages_per_seq  row stride of page_table; pages_per_seq * page_size
 *              must cover max_prefix. A sequence whose cu_prefix length
 *              exceeds pages_per_seq * page_size (a broken max_prefix
 *              promise) is cut at the end of its row: only the tokens its
 *              row holds are attended, and no other row is read.
 *  cu_prefix   as above; only the lengths cu_prefix[b+1] - cu_prefix[b]
 *              are used.
 * Other arguments as focus_block_attn_importance.
 * Errors: as focus_block_attn_importance, plus UNSUPPORTED for a page_size
 * that is not a positive multiple of 32 and INVALID_ARG for a NULL
 * page_table (max_prefix > 0) or pages that cannot hold max_prefix.
 */
focus_status focus_block_attn_importance_paged(
    focus_dtype dt, int batch, int B, int Hq, int Hkv, int d, float scale,
    const void* q, const void* k_blk, const void* v_blk,
    const void* k_pages, const void* v_pages, const int32_t* page_table,
    int page_size, int pages_per_seq, const int32_t* cu_prefix,
    const int32_t* order, int max_prefix, void* out, float* imp, float* lse,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Head mean, MaxPool1D smoothing, importance delta and per-sequence top-K.
 *
 * Follows the Pith page, "What carries the argument": the importance is
 * smoothed by MaxPool1D (kernel 3 in the Free-Parameter Ledger, Eq. 15),
 * the delta is layer-1 minus layer-0 importance (Eq. 3), and the top
 * candidates by delta are kept under the budget (also ScienceStack page,
 * Fig. 5). Per sequence b and block position j:
 *    Ibar_l[j]  = (1/Hq) sum_h imp_l[b,h,j]              (l = 0, 1)
 *    Itil_l[j]  = max{ Ibar_l[t] : |t - j| <= (pool_k-1)/2, 0 <= t < B }
 *                 (the window is cut at the block edges, i.e. padded with
 *                 -inf; pool_k may exceed B, and from pool_k >= 2B-1 on
 *                 every position takes the block's maximum)
 *    dI[b,j]    = Itil_1[j] - Itil_0[j]
 *    keep[b,j]  = 1 for the min(max(k_keep[b],0),B) largest dI[b,.],
 *                 equal values ordered by lower j first; else 0.
 *
 *  imp0, imp1  float32 [batch, Hq, B] from focus_block_attn_importance on
 *              layer 0 and layer 1.
 *  k_keep      device int32 [batch] budgets, clamped to [0, B].
 *  keep        uint8 [batch, B] output, 0/1.
 *  dI          float32 [batch, B] output, or NULL.
 * Errors: INVALID_ARG (null required pointer, batch < 1, B not in [1,128],
 * Hq < 1), UNSUPPORTED (pool_k even, < 1 or > 255), HIP.
 */
focus_status focus_delta_topk(
    int batch, int B, int Hq, int pool_k, const float* imp0,
    const float* imp1, const int32_t* k_keep, uint8_t* keep, float* dI,
    void* stream);

/*
 * Stream compaction of the retained tokens: the tokens kept by top-K go on
 * to the remaining layers (Pith page, "The pith").
 *    idx    = every b*B + j with keep[b,j] != 0, b ascending, then j
 *             ascending; int32, capacity batch*B (entries past the total are
 *             left untouched).
 *    cu_ret = int32 [batch+1]: cu_ret[0] = 0, cu_ret[b+1] - cu_ret[b] = the
 *             number kept in sequence b.
 * Errors: INVALID_ARG (null pointer, batch < 1, B not in [1,128]), HIP.
 */
focus_status focus_compact(int batch, int B, const uint8_t* keep,
                           int32_t* idx, int32_t* cu_ret, void* stream);

/*
 * focus_delta_topk followed by focus_compact, in one launch.
 *
 * Same definitions and outputs as those two calls (keep, dI, idx, cu_ret
 * are bit-identical to calling them in sequence): the importance delta and
 * top-K of the Pith page, "What carries the argument", then the retained
 * tokens' index list for the remaining layers ("The pith"). Each sequence's
 * offset in idx is the sum of min(max(K_b', 0), B) over the sequences
 * before it, which is what top-K keeps. One kernel instead of two on the
 * per-step path; the per-sequence offset sum costs O(batch) per sequence,
 * so batches above 4096 sequences run the two kernels instead.
 *
 *  idx     int32, capacity batch*B; cu_ret int32 [batch+1]; others as in
 *          focus_delta_topk. dI may be NULL.
 * Errors: as focus_delta_topk, plus INVALID_ARG for NULL idx / cu_ret.
 */
focus_status focus_select(int batch, int B, int Hq, int pool_k,
                          const float* imp0, const float* imp1,
                          const int32_t* k_keep, uint8_t* keep, float* dI,
                          int32_t* idx, int32_t* cu_ret, void* stream);

/* Structural constraints of focus_select_masked (bit flags). */
#define FOCUS_KEEP_PREDECESSOR 1   /* keep position j-1 of each candidate j */
#define FOCUS_KEEP_MASKED_PREFIX 2 /* keep every masked position left of the
                                      rightmost candidate */

/*
 * Top-K over the still-masked positions, then the two structural
 * constraints, then (optionally) compaction.
 *
 * Follows the Pith page, "What carries the argument": top-K candidates by
 * importance delta under the budget, then retain each candidate's
 * immediate predecessor and all masked tokens before the rightmost
 * candidate. Only tokens that are still masked can be candidates (the
 * method predicts which masked tokens will decode; Pith page, Referee
 * Report). Per sequence b, with M = { j : masked[b,j] != 0 } (all j if
 * masked is NULL) and dI as in focus_delta_topk:
 *    cand  = the min(max(k_keep[b],0), |M|) positions of M with the largest
 *            dI, equal values ordered by lower j first;
 *    keep  = cand
 *            + { j-1 : j in cand, j > 0 }           if FOCUS_KEEP_PREDECESSOR
 *            + { j in M : j < max(cand) }           if FOCUS_KEEP_MASKED_PREFIX
 *            (nothing when cand is empty).
 * With masked NULL and rules 0 this is focus_delta_topk (+ focus_compact).
 * The retained count per sequence is data-dependent here: size the
 * retained attention with n_ret = batch*B and max_ret = B (upper bounds)
 * or read cu_ret back.
 *
 *  masked  uint8 [batch, B], non-zero = still masked (a candidate), or NULL.
 *  rules   OR of FOCUS_KEEP_PREDECESSOR and FOCUS_KEEP_MASKED_PREFIX.
 *  keep    uint8 [batch, B] output: the retained set.
 *  cand    uint8 [batch, B] output: the top-K candidates, or NULL.
 *  dI      float32 [batch, B] output, or NULL.
 *  idx, cu_ret  as focus_compact over keep, or both NULL (no compaction).
 * Two kernels: the selection (one wavefront per sequence) and, when idx is
 * given, the one-workgroup compaction.
 * Errors: as focus_delta_topk; INVALID_ARG if exactly one of idx / cu_ret
 * is NULL; UNSUPPORTED for unknown rule bits.
 */
focus_status focus_select_masked(int batch, int B, int Hq, int pool_k,
                                 const float* imp0, const float* imp1,
                                 const uint8_t* masked, const int32_t* k_keep,
                                 int rules, uint8_t* keep, uint8_t* cand,
                                 float* dI, int32_t* idx, int32_t* cu_ret,
                                 void* stream);

/*
 * focus_select_masked with the budget set on the device from the block's
 * own deltas and the decoding history: a READING of the pages' dynamic
 * budgeting, whose formula the pages do not print (parity against the
 * pages is unpinned; the oracle implements the same reading). The pages
 * name its inputs: the historical decoding yield and within-block delta
 * statistics (Pith page, summary), the expansion factor alpha of Eq. 4
 * (default 1.5; Axiom & Free-Parameter Ledger) and a +Std threshold on
 * the delta (Fig. 14 caption). Read as, per sequence b over its masked
 * positions M (all positions if masked is NULL):
 *    mu, sigma = mean and population std of dI over M;
 *    n   = #{ j in M : dI[b,j] > mu + sigma };
 *    K_b = min(|M|, max(1, ceil(alpha * max(yield_hist[b], n)))),
 *          0 when M is empty;
 * computed in fp32 with fixed-order reductions; then candidates, rules
 * and compaction exactly as focus_select_masked with k_keep = K.
 *
 *  yield_hist  device float32 [batch]: the decoding yield history of each
 *              sequence (e.g. tokens decoded at its previous step).
 *  alpha       expansion factor, in (0, 1e6).
 *  k_used      device int32 [batch] output: K_b, or NULL.
 * Other arguments and errors as focus_select_masked, plus INVALID_ARG for
 * a NULL yield_hist or alpha out of range.
 */
focus_status focus_select_dynamic(int batch, int B, int Hq, int pool_k,
                                  const float* imp0, const float* imp1,
                                  const uint8_t* masked, const float* yield_hist,
                                  float alpha, int rules, int32_t* k_used,
                                  uint8_t* keep, uint8_t* cand, float* dI,
                                  int32_t* idx, int32_t* cu_ret, void* stream);

/* Workspace bytes that focus_retained_attn needs for these sizes. */
focus_status focus_retained_attn_workspace(
    int batch, int Hq, int Hkv, int d, int max_prefix, int n_ret,
    int max_ret, size_t* bytes);

/*
 * Retained-query attention for one further layer: the layers after the
 * first two run only on the retained tokens (Pith page, "The pith"). Every
 * retained query of sequence b attends to that layer's P_b prefix keys and
 * to the block keys of b's retained tokens only (no mask).
 *
 *  q_src       [batch*B, Hq, d]  the layer's block queries; rows read via idx.
 *  k_src,v_src [batch*B, Hkv, d] the layer's block keys/values; via idx.
 *  idx, cu_ret from focus_compact (device).
 *  n_ret       host promise: cu_ret[batch] <= n_ret (rows of out); an
 *              upper bound such as batch*B is allowed (rows past
 *              cu_ret[batch] are left untouched).
 *  max_ret     host promise: max_b (cu_ret[b+1] - cu_ret[b]) <= max_ret
 *              <= B. Sizes the launch; a sequence with more retained rows
 *              than max_ret only gets its first max_ret rows computed.
 *  k_cache,v_cache,cu_prefix,order,max_prefix  as in
 *              focus_block_attn_importance, for this layer.
 *  out         [n_ret, Hq, d] (type dt), row r is the query of idx[r].
 * n_ret == 0 enqueues nothing and returns FOCUS_OK.
 * Errors: as focus_block_attn_importance, plus INVALID_ARG for n_ret < 0 or
 * max_ret outside [0, B] or max_ret == 0 < n_ret.
 */
focus_status focus_retained_attn(
    focus_dtype dt, int batch, int B, int Hq, int Hkv, int d, float scale,
    const void* q_src, const void* k_src, const void* v_src,
    const int32_t* idx, const int32_t* cu_ret, int n_ret, int max_ret,
    const void* k_cache, const void* v_cache, const int32_t* cu_prefix,
    const int32_t* order, int max_prefix, void* out, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * focus_retained_attn over a paged prefix KV cache (layout and page
 * arguments as in focus_block_attn_importance_paged); same outputs, bit
 * for bit.
 */
focus_status focus_retained_attn_paged(
    focus_dtype dt, int batch, int B, int Hq, int Hkv, int d, float scale,
    const void* q_src, const void* k_src, const void* v_src,
    const int32_t* idx, const int32_t* cu_ret, int n_ret, int max_ret,
    const void* k_pages, const void* v_pages, const int32_t* page_table,
    int page_size, int pages_per_seq, const int32_t* cu_prefix,
    const int32_t* order, int max_prefix, void* out, void* workspace,
    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FOCUS_H_ */

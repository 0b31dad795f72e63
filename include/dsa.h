/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention (DSA) hot path on AMD
 * Instinct MI355X (gfx950).
 *
 * DSA (DeepSeek-V3.2-Exp deployment article, section 1; SGLang day-0
 * DeepSeek-V3.2 announcement, "DeepSeek Sparse Attention" section) runs in
 * three stages per query token:
 *   1. a light FP8 "Lightning Indexer" scores every causal predecessor token;
 *   2. top-k token selection keeps the k best (k = 2048 in the deployment
 *      configs of the article's section 3);
 *   3. attention (multi-head latent attention, MLA) runs over only the
 *      selected latent key/value rows, so its cost is O(L k) instead of
 *      O(L^2).
 * Storage follows the announcement's "DeepSeek Sparse Attention" section:
 * the indexer keeps a key & key_scale cache with page size 64, the sparse
 * attention operator reads a token-granular (page size 1) latent KV cache.
 *
 * Conventions for every entry point below:
 *  - All tensor pointers are DEVICE pointers (hipMalloc / torch CUDA
 *    tensors) into dense row-major arrays with the layouts stated; the
 *    caller owns every buffer.  The library allocates, frees and retains no
 *    device memory and keeps no state besides its loaded code and a
 *    thread-local error string.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls are asynchronous: they validate, enqueue and return.
 *  - Every argument is validated on the host before anything is enqueued.
 *    On any non-DSA_OK return nothing has been enqueued and no output has
 *    been touched; dsa_last_error() describes the problem.  A failed kernel
 *    launch returns DSA_ERR_HIP.  The library never prints, aborts or
 *    synchronizes.
 *  - Results are deterministic: no floating-point atomics, fixed reduction
 *    orders.
 *  - Device-resident index data (page tables, slot tables, positions, top-k
 *    indices) cannot be validated on the host.  Kernels bound-check every
 *    gathered address: an entry that points outside its table or cache is
 *    skipped as documented per function, never dereferenced.
 *  - Pointers must be 16-byte aligned (DSA_ERR_MISALIGNED otherwise).
 *  - A zero count (n = 0, n_q = 0) is valid: the shape, dtype and support
 *    checks still apply, the data pointers may be NULL, and nothing is
 *    enqueued.
 *
 * FP8 is OCP E4M3 ("e4m3fn": bias 7, max 448, no infinities, S.1111.111 =
 * NaN), the "fp8_e4m3" KV-cache dtype of the deployment article, section 3.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1
#define DSA_PAGE_SIZE 64      /* tokens per indexer key-cache page */
#define DSA_LATENT_DIM 576    /* latent key width: 512 value dims + 64 rope dims */
#define DSA_VALUE_DIM 512     /* leading dims of a latent row that form the value */
#define DSA_MAX_TOPK 2048
#define DSA_MAX_TOPK_ROW 262144   /* longest score row dsa_topk accepts (scores_ld) */

typedef enum dsa_status {
    DSA_OK = 0,
    DSA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
    DSA_ERR_BAD_SHAPE = 2,           /* a size / leading dimension is out of range */
    DSA_ERR_UNSUPPORTED = 3,         /* a valid but unsupported shape (see each call) */
    DSA_ERR_MISALIGNED = 4,          /* a pointer is not 16-byte aligned */
    DSA_ERR_WORKSPACE_TOO_SMALL = 5, /* ws_bytes below the matching *_workspace_size() */
    DSA_ERR_HIP = 6,                 /* the HIP runtime reported an error */
    DSA_ERR_NO_DEVICE = 7            /* no gfx950 device is visible */
} dsa_status;

typedef enum dsa_kv_dtype {
    DSA_KV_BF16 = 0,      /* latent cache rows: 576 bf16 (1152 bytes) */
    DSA_KV_FP8_E4M3 = 1   /* latent cache rows: 576 E4M3 codes + one fp32 scale per row */
} dsa_kv_dtype;

/* DSA_ABI_VERSION of the loaded library. */
int dsa_abi_version(void);

/* Static name of a status code ("DSA_OK", ...). */
const char *dsa_status_string(int status);

/* Detail of the last non-OK status returned on the calling thread (static
 * thread-local storage; valid until the next call on that thread). */
const char *dsa_last_error(void);

/* ------------------------------------------------------------------------
 * Cache stores
 * ------------------------------------------------------------------------ */

/* Indexer key-cache store (announcement, "DeepSeek Sparse Attention": a
 * dedicated key & key_scale cache, page size 64).
 *   k_fp8           [n, d_i] E4M3 codes of the new tokens' indexer keys
 *   k_scale         [n] fp32 per-token scale
 *   slot            [n] int64, slot of token i = physical_page * 64 + offset;
 *                   a slot outside [0, n_pages * 64) is skipped
 *   key_cache       n_pages pages of 64 * d_i E4M3 codes (written), each page
 *                   fragment-major: a run of 1 KB blocks where block
 *                   (kt * d_i / 64 + c) * 2 + h, 16-byte slot l (l < 64) holds
 *                   bytes g * d_i / 2 + 32 c + 16 h .. +16 of the page's key
 *                   32 kt + l % 32, g = l / 32 (kt < 2, c < d_i / 64, h < 2).
 *                   The scorers load each block as one contiguous 1 KB run that
 *                   is already their FP8 MFMA operand.
 *   key_scale_cache [n_pages, 64] fp32 (written)
 * A byte copy.  d_i in {64, 128}; n >= 0 (n == 0 enqueues nothing). */
dsa_status dsa_indexer_cache_store(const uint8_t *k_fp8, const float *k_scale, const int64_t *slot,
                                   int32_t n, int32_t d_i, uint8_t *key_cache, float *key_scale_cache,
                                   int64_t n_pages, void *stream);

/* Latent KV-cache store, token granular (page size 1).
 *   kv_bf16   [n, 576] bf16 latent rows of the new tokens
 *   slot      [n] int64 destination slot; outside [0, n_slots) is skipped
 *   dt == DSA_KV_BF16:     kv_cache [n_slots, 576] bf16 (uint16 bits); kv_scale unused (may be NULL)
 *   dt == DSA_KV_FP8_E4M3: kv_cache [n_slots, 576] E4M3 codes; kv_scale [n_slots] fp32.
 *     Per-token quantization (deployment article, section 3: "kv_cache_dtype
 *     fp8_e4m3"): scale = amax / 448 over the row in fp32 (1 if the row is all
 *     zero); code = E4M3(x / scale), IEEE fp32 division, round to nearest
 *     even, saturating at +-448. */
dsa_status dsa_kv_cache_store(const uint16_t *kv_bf16, const int64_t *slot, int32_t n, dsa_kv_dtype dt,
                              void *kv_cache, float *kv_scale, int64_t n_slots, void *stream);

/* Both stores above in one launch, writing new tokens into the two caches of
 * the announcement's "DeepSeek Sparse Attention" section: the indexer keys of
 * n_keys tokens (as dsa_indexer_cache_store) and the latent rows of n_kv
 * tokens (as dsa_kv_cache_store), with the same arguments, layouts and
 * skipped slots; the bytes written are the same as those of the two calls.
 * A decode step stores a handful of tokens, for which each store alone is a
 * short launch whose fixed cost exceeds its work.  n_keys == 0 or n_kv == 0
 * leaves that cache alone (its pointers may then be NULL); both zero
 * enqueues nothing.  Argument errors are those of the two calls, reported
 * before anything is enqueued. */
dsa_status dsa_cache_store(const uint8_t *k_fp8, const float *k_scale, const int64_t *key_slot, int32_t n_keys,
                           int32_t d_i, uint8_t *key_cache, float *key_scale_cache, int64_t n_pages,
                           const uint16_t *kv_bf16, const int64_t *kv_slot, int32_t n_kv, dsa_kv_dtype dt,
                           void *kv_cache, float *kv_scale, int64_t n_slots, void *stream);

/* ------------------------------------------------------------------------
 * Stage 1: Lightning Indexer scores
 * ------------------------------------------------------------------------ */

/* For every query t and predecessor position s in [0, q_pos[t]] of its
 * sequence b = q_seq[t] (deployment article, section 1: the indexer scores
 * the predecessor tokens; context-parallel article, section 1: its relevance
 * is a reduce-sum over the indexer heads):
 *
 *   score[t, s] = q_scale[t] * k_scale[s] * sum_j w[t, j] * ReLU( sum_i q[t, j, i] * k[s, i] )
 *
 *   q_fp8      [n_q, h_i, d_i] E4M3 codes, q_scale [n_q] fp32
 *   w          per-head weights, row t at w + t * w_ld (w_ld = h_i for [n_q, h_i];
 *              w_ld = 0: one [h_i] vector shared by every query)
 *   key_cache / key_scale_cache  as written by dsa_indexer_cache_store
 *   page_table [B, pt_ld] int32: logical page p of sequence b -> physical page
 *   q_seq, q_pos [n_q] int32
 *   scores     [n_q, scores_ld] fp32; columns 0..q_pos[t] of row t are written,
 *              the rest of the row is left untouched.
 * The q.k contraction runs on FP8 MFMA with fp32 accumulation; ReLU, weights
 * and the head sum run in fp32.  A logical page past pt_ld, or a physical
 * page outside [0, n_pages), yields NaN scores for its tokens.  Columns at or
 * beyond scores_ld are never written.
 * Supported: (h_i, d_i) in {(16, 64), (64, 128)}; n_q >= 0. */
dsa_status dsa_indexer_scores(const uint8_t *q_fp8, const float *q_scale, const float *w, int64_t w_ld,
                              const uint8_t *key_cache, const float *key_scale_cache, int64_t n_pages,
                              const int32_t *page_table, int64_t pt_ld,
                              const int32_t *q_seq, const int32_t *q_pos, int32_t n_q,
                              int32_t h_i, int32_t d_i, float *scores, int64_t scores_ld, void *stream);

/* ------------------------------------------------------------------------
 * Stage 2: top-k selection
 * ------------------------------------------------------------------------ */

/* Bytes of workspace with which dsa_topk splits each of few long rows over
 * several workgroups (each keeps the k best of its part of the row, a second
 * pass selects among the survivors; the result is identical).  0 when these
 * sizes are not split.  The workspace is optional: with ws = NULL or fewer
 * bytes every row is selected by one workgroup. */
size_t dsa_topk_workspace_size(int32_t n_q, int64_t max_len, int32_t k);

/* Per row t, over candidates s in [0, q_pos[t]] of scores[t, :]: keep the
 * min(k, q_pos[t] + 1) largest (announcement: "top-k token selection"),
 * ranking by score descending and, among equal scores, by lower index
 * (-0.0 and +0.0 are equal).  When a row has no more candidates than k,
 * all of them are kept (the dense degeneration of the deployment article,
 * section 5.1).  idx[t, :] receives the kept positions in ascending order,
 * then -1 in the remaining slots.  Integer selection: the result is
 * bit-exact for given scores.  NaN scores rank by their bit pattern (a
 * positive NaN above +inf); valid inputs produce none.
 *   scores [n_q, scores_ld] fp32 (q_pos[t] < scores_ld is the caller's contract;
 *          columns at or beyond scores_ld are never read)
 *   idx    [n_q, k] int32
 *   ws     optional device workspace (see dsa_topk_workspace_size), any
 *          alignment; owned by the caller and not read back by it
 * Supported: 1 <= k <= 2048, scores_ld <= DSA_MAX_TOPK_ROW (DSA_ERR_UNSUPPORTED
 * otherwise). */
dsa_status dsa_topk(const float *scores, int64_t scores_ld, const int32_t *q_pos, int32_t n_q, int32_t k,
                    int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Stages 1 + 2 fused (decode form)
 * ------------------------------------------------------------------------ */

/* Bytes of the workspace of dsa_indexer_topk for n_q queries: a block of
 * 106,560 bytes per query (query t's at byte t * 106560, so a call with fewer
 * queries uses a prefix of a larger workspace): 8256 bytes that must be zero
 * (the row's key histogram and the selection's counters), then 96 KiB of
 * scratch (the row's bitmap of kept indices and its candidate list). */
size_t dsa_indexer_topk_workspace_size(int32_t n_q);

/* dsa_indexer_scores followed by dsa_topk, with the selection's first pass
 * fused into the scorer (the fused indexer -> top-k mode the SGLang DeepSeek
 * V3.2 usage guide's MI350/MI355 recipe names): every scoring workgroup counts
 * the order-preserving keys of the scores it writes in a histogram of their
 * top 11 bits and adds it to its row's histogram in `ws` with integer atomics
 * (the sum is order-independent, so results stay deterministic).  The
 * selection then knows each row's threshold bin before reading a score: it
 * reads every row once, in parts of 32K scores on separate workgroups, and the
 * workgroup that finishes a row's last part completes that row.  Arguments,
 * layouts and results are those of the two calls (scores are written as by
 * dsa_indexer_scores, idx as by dsa_topk, bit-identical to them).
 *   ws  at least dsa_indexer_topk_workspace_size(n_q) bytes of device memory,
 *       16-byte aligned, ZERO before the first call; every successful call
 *       leaves it as the next call needs it (the selection clears the regions
 *       that must be zero), so one zeroed workspace serves every later call,
 *       also in a replayed HIP graph.  Calls that use one workspace must not
 *       overlap.  After a DSA_ERR_HIP return it must be zeroed again.
 * Supported: the decode form, n_q <= 256 (DSA_ERR_UNSUPPORTED above: use the
 * two calls); otherwise as dsa_indexer_scores and dsa_topk. */
dsa_status dsa_indexer_topk(const uint8_t *q_fp8, const float *q_scale, const float *w, int64_t w_ld,
                            const uint8_t *key_cache, const float *key_scale_cache, int64_t n_pages,
                            const int32_t *page_table, int64_t pt_ld,
                            const int32_t *q_seq, const int32_t *q_pos, int32_t n_q, int32_t h_i, int32_t d_i,
                            float *scores, int64_t scores_ld, int32_t k, int32_t *idx, void *ws, size_t ws_bytes,
                            void *stream);

/* dsa_topk for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same selection
 * and result, with the split rows' survivors in a static device array of the
 * library (8 MiB + 256 bytes per device, held until the process ends) instead
 * of a caller workspace.  Nothing is allocated or freed; the array's address
 * is looked up once per device, on the first call with that device current
 * (the stream must belong to the current device).  Calls that overlap on one
 * device share the array and race: serialise them (one stream, or events).
 * Sizes whose split would exceed the array return DSA_ERR_WORKSPACE_TOO_SMALL
 * (none does for k <= 2048); otherwise arguments and errors as dsa_topk. */
dsa_status dsa_topk_static(const float *scores, int64_t scores_ld, const int32_t *q_pos, int32_t n_q, int32_t k,
                           int32_t *idx, void *stream);

/* ------------------------------------------------------------------------
 * Stage 3: sparse MLA over the selected latent rows
 * ------------------------------------------------------------------------ */

/* For query t, head h and its selected set S_t = { idx[t, i] >= 0 }
 * (usage guide, "attention kernel selection": bf16 q; bf16 kv or bf16 q
 * with an fp8 k_cache):
 *
 *   l_s = sm_scale * q[t, h, :] . K[s, :]            (576-d latent keys)
 *   out[t, h, :] = sum_s softmax(l)_s * K[s, 0:512]   (values = first 512 dims)
 *   lse[t, h]    = log sum_s exp(l_s)                 (natural log)
 *
 *   q             [n_q, h, 576] bf16
 *   kv_cache      as written by dsa_kv_cache_store with dtype dt; kv_scale
 *                 [n_slots] fp32 for DSA_KV_FP8_E4M3 (NULL allowed for bf16)
 *   kv_slot_table [B, kv_pt_ld] int32: logical position -> slot for sequence b
 *   q_seq         [n_q] int32 sequence of each query
 *   idx           [n_q, k] int32 logical positions (as produced by dsa_topk);
 *                 -1, positions >= kv_pt_ld and slots outside [0, n_slots)
 *                 are skipped
 *   out           [n_q, h, 512] bf16;  lse [n_q, h] fp32 or NULL
 * A query with no valid index gets out = 0 and lse = -inf.
 * bf16 MFMA with fp32 accumulation and an online softmax; FP8 rows are
 * expanded to bf16 exactly and their per-row scale applied in fp32.
 * Supported: h a multiple of 8 in [8, 128]; 1 <= k <= 2048. */
dsa_status dsa_sparse_mla_prefill(const uint16_t *q, const void *kv_cache, const float *kv_scale,
                                  dsa_kv_dtype dt, int64_t n_slots,
                                  const int32_t *kv_slot_table, int64_t kv_pt_ld,
                                  const int32_t *q_seq, const int32_t *idx, int32_t n_q, int32_t h,
                                  int32_t k, float sm_scale, uint16_t *out, float *lse, void *stream);

/* Bytes of workspace dsa_sparse_mla_decode needs (n_splits = 0: the value
 * the library would pick automatically for these sizes); 0 when the index lists
 * are not split. */
size_t dsa_sparse_mla_decode_workspace_size(int32_t n_q, int32_t h, int32_t k, int32_t n_splits);

/* Decode form of dsa_sparse_mla_prefill for few queries (one or a few per
 * sequence): same arguments and result.
 *   n_splits = 1: one workgroup per (query, group of 32 heads) attends over the
 *     query's whole selection; no workspace (ws may be NULL).
 *   n_splits > 1 (at most 32): each query's index list is cut into n_splits
 *     chunks processed in parallel, each producing a partial output and
 *     log-sum-exp in `ws`, merged afterwards with LSE weights.
 *   n_splits = 0 picks: 1 when n_q * ceil(h / 32) >= 128, else a split count
 *     that gives about one workgroup per compute unit.
 * ws_bytes must be at least dsa_sparse_mla_decode_workspace_size(n_q, h, k,
 * n_splits) (DSA_ERR_WORKSPACE_TOO_SMALL otherwise). */
dsa_status dsa_sparse_mla_decode(const uint16_t *q, const void *kv_cache, const float *kv_scale,
                                 dsa_kv_dtype dt, int64_t n_slots,
                                 const int32_t *kv_slot_table, int64_t kv_pt_ld,
                                 const int32_t *q_seq, const int32_t *idx, int32_t n_q, int32_t h,
                                 int32_t k, float sm_scale, uint16_t *out, float *lse,
                                 int32_t n_splits, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */

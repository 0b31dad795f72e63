// dsa_api.cpp -- the C ABI declared in include/dsa.h: argument validation,
// error reporting and kernel launch.  Validation happens entirely on the host
// before anything touches the GPU, so every error path is reachable without
// a device.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/dsa.h"
#include "dsa_internal.h"

#define DSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

dsa_status fail(dsa_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

dsa_status hip_fail(hipError_t e, const char *what) {
    return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

#define REQUIRE_PTR(p)                                                                                  \
    do {                                                                                                \
        if ((p) == nullptr) return fail(DSA_ERR_NULL_POINTER, "%s: %s is NULL", __func__, #p);         \
        if (misaligned(p)) return fail(DSA_ERR_MISALIGNED, "%s: %s is not 16-byte aligned", __func__, #p); \
    } while (0)

#define REQUIRE(cond, status, ...)                                                                      \
    do {                                                                                                \
        if (!(cond)) return fail(status, __VA_ARGS__);                                                  \
    } while (0)

}  // namespace

DSA_EXPORT int dsa_abi_version(void) { return DSA_ABI_VERSION; }

DSA_EXPORT const char *dsa_status_string(int s) {
    switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL_POINTER: return "DSA_ERR_NULL_POINTER";
    case DSA_ERR_BAD_SHAPE: return "DSA_ERR_BAD_SHAPE";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_MISALIGNED: return "DSA_ERR_MISALIGNED";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "DSA_ERR_WORKSPACE_TOO_SMALL";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
    case DSA_ERR_NO_DEVICE: return "DSA_ERR_NO_DEVICE";
    default: return "DSA_ERR_UNKNOWN";
    }
}

DSA_EXPORT const char *dsa_last_error(void) { return g_err; }

DSA_EXPORT dsa_status dsa_indexer_cache_store(const uint8_t *k_fp8, const float *k_scale, const int64_t *slot,
                                              int32_t n, int32_t d_i, uint8_t *key_cache, float *key_scale_cache,
                                              int64_t n_pages, void *stream) {
    REQUIRE(n >= 0, DSA_ERR_BAD_SHAPE, "dsa_indexer_cache_store: n = %d < 0", n);
    REQUIRE(n_pages >= 0, DSA_ERR_BAD_SHAPE, "dsa_indexer_cache_store: n_pages = %lld < 0", (long long)n_pages);
    REQUIRE(d_i == 64 || d_i == 128, DSA_ERR_UNSUPPORTED, "dsa_indexer_cache_store: d_i = %d not in {64, 128}", d_i);
    if (n == 0) return DSA_OK;
    REQUIRE_PTR(k_fp8);
    REQUIRE_PTR(k_scale);
    REQUIRE_PTR(slot);
    REQUIRE_PTR(key_cache);
    REQUIRE_PTR(key_scale_cache);
    hipError_t e = dsa::launch_indexer_store(k_fp8, k_scale, slot, n, d_i, key_cache, key_scale_cache, n_pages,
                                             (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dsa_indexer_cache_store launch");
    return DSA_OK;
}

DSA_EXPORT dsa_status dsa_kv_cache_store(const uint16_t *kv_bf16, const int64_t *slot, int32_t n, dsa_kv_dtype dt,
                                         void *kv_cache, float *kv_scale, int64_t n_slots, void *stream) {
    REQUIRE(n >= 0, DSA_ERR_BAD_SHAPE, "dsa_kv_cache_store: n = %d < 0", n);
    REQUIRE(n_slots >= 0, DSA_ERR_BAD_SHAPE, "dsa_kv_cache_store: n_slots < 0");
    REQUIRE(dt == DSA_KV_BF16 || dt == DSA_KV_FP8_E4M3, DSA_ERR_UNSUPPORTED, "dsa_kv_cache_store: bad dtype %d",
            (int)dt);
    if (n == 0) return DSA_OK;
    REQUIRE_PTR(kv_bf16);
    REQUIRE_PTR(slot);
    REQUIRE_PTR(kv_cache);
    if (dt == DSA_KV_FP8_E4M3) REQUIRE_PTR(kv_scale);
    hipError_t e = dsa::launch_kv_store(kv_bf16, slot, n, (int)dt, kv_cache, kv_scale, n_slots, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dsa_kv_cache_store launch");
    return DSA_OK;
}

DSA_EXPORT dsa_status dsa_cache_store(const uint8_t *k_fp8, const float *k_scale, const int64_t *key_slot,
                                      int32_t n_keys, int32_t d_i, uint8_t *key_cache, float *key_scale_cache,
                                      int64_t n_pages, const uint16_t *kv_bf16, const int64_t *kv_slot, int32_t n_kv,
                                      dsa_kv_dtype dt, void *kv_cache, float *kv_scale, int64_t n_slots,
                                      void *stream) {
    REQUIRE(n_keys >= 0 && n_kv >= 0, DSA_ERR_BAD_SHAPE, "dsa_cache_store: n_keys = %d, n_kv = %d (need >= 0)", n_keys,
            n_kv);
    REQUIRE(n_pages >= 0, DSA_ERR_BAD_SHAPE, "dsa_cache_store: n_pages = %lld < 0", (long long)n_pages);
    REQUIRE(n_slots >= 0, DSA_ERR_BAD_SHAPE, "dsa_cache_store: n_slots < 0");
    REQUIRE(d_i == 64 || d_i == 128, DSA_ERR_UNSUPPORTED, "dsa_cache_store: d_i = %d not in {64, 128}", d_i);
    REQUIRE(dt == DSA_KV_BF16 || dt == DSA_KV_FP8_E4M3, DSA_ERR_UNSUPPORTED, "dsa_cache_store: bad dtype %d", (int)dt);
    if (n_keys == 0 && n_kv == 0) return DSA_OK;
    if (n_keys > 0) {
        REQUIRE_PTR(k_fp8);
        REQUIRE_PTR(k_scale);
        REQUIRE_PTR(key_slot);
        REQUIRE_PTR(key_cache);
        REQUIRE_PTR(key_scale_cache);
    }
    if (n_kv > 0) {
        REQUIRE_PTR(kv_bf16);
        REQUIRE_PTR(kv_slot);
        REQUIRE_PTR(kv_cache);
        if (dt == DSA_KV_FP8_E4M3) REQUIRE_PTR(kv_scale);
    }
    hipError_t e = dsa::launch_cache_store(k_fp8, k_scale, key_slot, n_keys, d_i, key_cache, key_scale_cache, n_pages,
                                           kv_bf16, kv_slot, n_kv, (int)dt, kv_cache, kv_scale, n_slots,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dsa_cache_store launch");
    return DSA_OK;
}

DSA_EXPORT dsa_status dsa_indexer_scores(const uint8_t *q_fp8, const float *q_scale, const float *w, int64_t w_ld,
                                         const uint8_t *key_cache, const float *key_scale_cache, int64_t n_pages,
                                         const int32_t *page_table, int64_t pt_ld, const int32_t *q_seq,
                                         const int32_t *q_pos, int32_t n_q, int32_t h_i, int32_t d_i, float *scores,
                                         int64_t scores_ld, void *stream) {
    REQUIRE(n_q >= 0, DSA_ERR_BAD_SHAPE, "dsa_indexer_scores: n_q = %d < 0", n_q);
    REQUIRE((h_i == 64 && d_i == 128) || (h_i == 16 && d_i == 64), DSA_ERR_UNSUPPORTED,
            "dsa_indexer_scores: (h_i, d_i) = (%d, %d) not in {(16, 64), (64, 128)}", h_i, d_i);
    REQUIRE(w_ld == 0 || w_ld >= h_i, DSA_ERR_BAD_SHAPE, "dsa_indexer_scores: w_ld = %lld (need 0 or >= h_i)",
            (long long)w_ld);
    REQUIRE(n_pages >= 0 && pt_ld >= 1, DSA_ERR_BAD_SHAPE, "dsa_indexer_scores: n_pages / pt_ld out of range");
    REQUIRE(scores_ld >= 1, DSA_ERR_BAD_SHAPE, "dsa_indexer_scores: scores_ld = %lld < 1", (long long)scores_ld);
    if (n_q == 0) return DSA_OK;
    REQUIRE_PTR(q_fp8);
    REQUIRE_PTR(q_scale);
    REQUIRE_PTR(w);
    REQUIRE_PTR(key_cache);
    REQUIRE_PTR(key_scale_cache);
    REQUIRE_PTR(page_table);
    REQUIRE_PTR(q_seq);
    REQUIRE_PTR(q_pos);
    REQUIRE_PTR(scores);
    dsa::IndexerArgs a{q_fp8, q_scale, w, w_ld, key_cache, key_scale_cache, n_pages, page_table, pt_ld,
                       q_seq, q_pos, n_q, h_i, d_i, scores, scores_ld};
    hipError_t e = dsa::launch_indexer(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dsa_indexer_scores launch");
    return DSA_OK;
}

DSA_EXPORT size_t dsa_indexer_topk_workspace_size(int32_t n_q) {
    return n_q > 0 ? dsa::fused_topk_ws_bytes(n_q) : 0;
}

DSA_EXPORT dsa_status dsa_indexer_topk(const uint8_t *q_fp8, const float *q_scale, const float *w, int64_t w_ld,
                                       const uint8_t *key_cache, const float *key_scale_cache, int64_t n_pages,
                                       const int32_t *page_table, int64_t pt_ld, const int32_t *q_seq,
                                       const int32_t *q_pos, int32_t n_q, int32_t h_i, int32_t d_i, float *scores,
                                       int64_t scores_ld, int32_t k, int32_t *idx, void *ws, size_t ws_bytes,
                                       void *stream) {
    REQUIRE(n_q >= 0, DSA_ERR_BAD_SHAPE, "dsa_indexer_topk: n_q = %d < 0", n_q);
    REQUIRE(n_q <= dsa::kIndexerDecodeMaxQ, DSA_ERR_UNSUPPORTED,
            "dsa_indexer_topk: n_q = %d > %d (the fused call is the decode form; use dsa_indexer_scores + dsa_topk)",
            n_q, dsa::kIndexerDecodeMaxQ);
    REQUIRE((h_i == 64 && d_i == 128) || (h_i == 16 && d_i == 64), DSA_ERR_UNSUPPORTED,
            "dsa_indexer_topk: (h_i, d_i) = (%d, %d) not in {(16, 64), (64, 128)}", h_i, d_i);
    REQUIRE(w_ld == 0 || w_ld >= h_i, DSA_ERR_BAD_SHAPE, "dsa_indexer_topk: w_ld = %lld (need 0 or >= h_i)",
            (long long)w_ld);
    REQUIRE(n_pages >= 0 && pt_ld >= 1, DSA_ERR_BAD_SHAPE, "dsa_indexer_topk: n_pages / pt_ld out of range");
    REQUIRE(scores_ld >= 1, DSA_ERR_BAD_SHAPE, "dsa_indexer_topk: scores_ld = %lld < 1", (long long)scores_ld);
    REQUIRE(scores_ld <= DSA_MAX_TOPK_ROW, DSA_ERR_UNSUPPORTED, "dsa_indexer_topk: scores_ld = %lld > %d",
            (long long)scores_ld, DSA_MAX_TOPK_ROW);
    REQUIRE(k >= 1 && k <= DSA_MAX_TOPK, DSA_ERR_UNSUPPORTED, "dsa_indexer_topk: k = %d not in [1, %d]", k,
            DSA_MAX_TOPK);
    if (n_q == 0) return DSA_OK;
    REQUIRE_PTR(q_fp8);
    REQUIRE_PTR(q_scale);
    REQUIRE_PTR(w);
    REQUIRE_PTR(key_cache);
    REQUIRE_PTR(key_scale_cache);
    REQUIRE_PTR(page_table);
    REQUIRE_PTR(q_seq);
    REQUIRE_PTR(q_pos);
    REQUIRE_PTR(scores);
    REQUIRE_PTR(idx);
    const size_t need = dsa::fused_topk_ws_bytes(n_q);
    REQUIRE(ws_bytes >= need, DSA_ERR_WORKSPACE_TOO_SMALL, "dsa_indexer_topk: ws_bytes = %zu < %zu needed", ws_bytes,
            need);
    REQUIRE_PTR(ws);
    dsa::IndexerArgs a{q_fp8, q_scale, w, w_ld, key_cache, key_scale_cache, n_pages, page_table, pt_ld,
                       q_seq, q_pos, n_q, h_i, d_i, scores, scores_ld, reinterpret_cast<uint32_t *>(ws)};
    hipError_t e = dsa::launch_indexer(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dsa_indexer_topk: scorer launch");
    e = dsa::launch_topk_fused(scores, scores_ld, q_pos, n_q, k, idx, reinterpret_cast<uint32_t *>(ws),
                               (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dsa_indexer_topk: selection launch");
    return DSA_OK;
}

DSA_EXPORT size_t dsa_topk_workspace_size(int32_t n_q, int64_t max_len, int32_t k) {
    if (n_q <= 0 || max_len <= 0 || k < 1 || k > DSA_MAX_TOPK || max_len > DSA_MAX_TOPK_ROW) return 0;
    return dsa::topk_ws_bytes(n_q, max_len, k);
}

DSA_EXPORT dsa_status dsa_topk(const float *scores, int64_t scores_ld, const int32_t *q_pos, int32_t n_q, int32_t k,
                               int32_t *idx, void *ws, size_t ws_bytes, void *stream) {
    REQUIRE(n_q >= 0, DSA_ERR_BAD_SHAPE, "dsa_topk: n_q = %d < 0", n_q);
    REQUIRE(k >= 1 && k <= DSA_MAX_TOPK, DSA_ERR_UNSUPPORTED, "dsa_topk: k = %d not in [1, %d]", k, DSA_MAX_TOPK);
    REQUIRE(scores_ld >= 1, DSA_ERR_BAD_SHAPE, "dsa_topk: scores_ld = %lld < 1", (long long)scores_ld);
    REQUIRE(scores_ld <= DSA_MAX_TOPK_ROW, DSA_ERR_UNSUPPORTED, "dsa_topk: scores_ld = %lld > %d",
            (long long)scores_ld, DSA_MAX_TOPK_ROW);
    if (n_q == 0) return DSA_OK;
    REQUIRE_PTR(scores);
    REQUIRE_PTR(q_pos);
    REQUIRE_PTR(idx);
    hipError_t e = dsa::launch_topk(scores, scores_ld, q_pos, n_q, k, idx, ws, ws ? ws_bytes : 0, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dsa_topk launch");
    return DSA_OK;
}

DSA_EXPORT dsa_status dsa_topk_static(const float *scores, int64_t scores_ld, const int32_t *q_pos, int32_t n_q,
                                      int32_t k, int32_t *idx, void *stream) {
    REQUIRE(n_q >= 0, DSA_ERR_BAD_SHAPE, "dsa_topk_static: n_q = %d < 0", n_q);
    REQUIRE(k >= 1 && k <= DSA_MAX_TOPK, DSA_ERR_UNSUPPORTED, "dsa_topk_static: k = %d not in [1, %d]", k,
            DSA_MAX_TOPK);
    REQUIRE(scores_ld >= 1, DSA_ERR_BAD_SHAPE, "dsa_topk_static: scores_ld = %lld < 1", (long long)scores_ld);
    REQUIRE(scores_ld <= DSA_MAX_TOPK_ROW, DSA_ERR_UNSUPPORTED, "dsa_topk_static: scores_ld = %lld > %d",
            (long long)scores_ld, DSA_MAX_TOPK_ROW);
    if (n_q == 0) return DSA_OK;
    REQUIRE_PTR(scores);
    REQUIRE_PTR(q_pos);
    REQUIRE_PTR(idx);
    const size_t need = dsa::topk_ws_bytes(n_q, scores_ld, k);
    void *ws = nullptr;
    size_t cap = 0;
    if (need > 0) {
        hipError_t e = dsa::topk_static_workspace(&ws, &cap);
        if (e != hipSuccess) return hip_fail(e, "dsa_topk_static: static workspace lookup");
        REQUIRE(need <= cap, DSA_ERR_WORKSPACE_TOO_SMALL,
                "dsa_topk_static: the split rows need %zu bytes, more than the static workspace's %zu", need, cap);
    }
    hipError_t e = dsa::launch_topk(scores, scores_ld, q_pos, n_q, k, idx, ws, need > 0 ? cap : 0,
                                    (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dsa_topk_static launch");
    return DSA_OK;
}

namespace {
dsa_status check_mla(const char *fn, const uint16_t *q, const void *kv_cache, const float *kv_scale, dsa_kv_dtype dt,
                     int64_t n_slots, const int32_t *kv_slot_table, int64_t kv_pt_ld, const int32_t *q_seq,
                     const int32_t *idx, int32_t n_q, int32_t h, int32_t k, float sm_scale, uint16_t *out,
                     float *lse) {
    REQUIRE(n_q >= 0, DSA_ERR_BAD_SHAPE, "%s: n_q = %d < 0", fn, n_q);
    REQUIRE(h >= 8 && h <= 128 && h % 8 == 0, DSA_ERR_UNSUPPORTED, "%s: h = %d (need a multiple of 8 in [8, 128])",
            fn, h);
    REQUIRE(k >= 1 && k <= DSA_MAX_TOPK, DSA_ERR_UNSUPPORTED, "%s: k = %d not in [1, %d]", fn, k, DSA_MAX_TOPK);
    REQUIRE(dt == DSA_KV_BF16 || dt == DSA_KV_FP8_E4M3, DSA_ERR_UNSUPPORTED, "%s: bad kv dtype %d", fn, (int)dt);
    REQUIRE(n_slots >= 1 && kv_pt_ld >= 1, DSA_ERR_BAD_SHAPE, "%s: n_slots / kv_pt_ld must be >= 1", fn);
    REQUIRE(sm_scale == sm_scale && sm_scale > 0.0f, DSA_ERR_BAD_SHAPE, "%s: sm_scale must be > 0", fn);
    if (n_q == 0) return DSA_OK;
    REQUIRE_PTR(q);
    REQUIRE_PTR(kv_cache);
    if (dt == DSA_KV_FP8_E4M3) REQUIRE_PTR(kv_scale);
    REQUIRE_PTR(kv_slot_table);
    REQUIRE_PTR(q_seq);
    REQUIRE_PTR(idx);
    REQUIRE_PTR(out);
    if (lse != nullptr && misaligned(lse)) return fail(DSA_ERR_MISALIGNED, "%s: lse is not 16-byte aligned", fn);
    return DSA_OK;
}
}  // namespace

DSA_EXPORT dsa_status dsa_sparse_mla_prefill(const uint16_t *q, const void *kv_cache, const float *kv_scale,
                                             dsa_kv_dtype dt, int64_t n_slots, const int32_t *kv_slot_table,
                                             int64_t kv_pt_ld, const int32_t *q_seq, const int32_t *idx, int32_t n_q,
                                             int32_t h, int32_t k, float sm_scale, uint16_t *out, float *lse,
                                             void *stream) {
    dsa_status s = check_mla("dsa_sparse_mla_prefill", q, kv_cache, kv_scale, dt, n_slots, kv_slot_table, kv_pt_ld,
                             q_seq, idx, n_q, h, k, sm_scale, out, lse);
    if (s != DSA_OK || n_q == 0) return s;
    dsa::MlaArgs a{q, kv_cache, kv_scale, dt == DSA_KV_FP8_E4M3, n_slots, kv_slot_table, kv_pt_ld, q_seq, idx,
                   n_q, h, k, sm_scale, out, lse};
    hipError_t e = dsa::launch_mla_prefill(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dsa_sparse_mla_prefill launch");
    return DSA_OK;
}

DSA_EXPORT size_t dsa_sparse_mla_decode_workspace_size(int32_t n_q, int32_t h, int32_t k, int32_t n_splits) {
    if (n_q <= 0 || h <= 0 || k <= 0) return 0;
    if (n_splits <= 0) n_splits = dsa::mla_decode_auto_splits(n_q, h, k);
    return dsa::mla_decode_ws_bytes(n_q, h, n_splits);
}

DSA_EXPORT dsa_status dsa_sparse_mla_decode(const uint16_t *q, const void *kv_cache, const float *kv_scale,
                                            dsa_kv_dtype dt, int64_t n_slots, const int32_t *kv_slot_table,
                                            int64_t kv_pt_ld, const int32_t *q_seq, const int32_t *idx, int32_t n_q,
                                            int32_t h, int32_t k, float sm_scale, uint16_t *out, float *lse,
                                            int32_t n_splits, void *ws, size_t ws_bytes, void *stream) {
    dsa_status s = check_mla("dsa_sparse_mla_decode", q, kv_cache, kv_scale, dt, n_slots, kv_slot_table, kv_pt_ld,
                             q_seq, idx, n_q, h, k, sm_scale, out, lse);
    if (s != DSA_OK) return s;
    REQUIRE(n_splits >= 0 && n_splits <= 32, DSA_ERR_UNSUPPORTED, "dsa_sparse_mla_decode: n_splits = %d not in [0, 32]",
            n_splits);
    if (n_q == 0) return DSA_OK;
    if (n_splits == 0) n_splits = dsa::mla_decode_auto_splits(n_q, h, k);
    const size_t need = dsa::mla_decode_ws_bytes(n_q, h, n_splits);
    REQUIRE(ws_bytes >= need, DSA_ERR_WORKSPACE_TOO_SMALL,
            "dsa_sparse_mla_decode: ws_bytes = %zu < %zu needed", ws_bytes, need);
    if (need > 0) REQUIRE_PTR(ws);
    dsa::MlaArgs a{q, kv_cache, kv_scale, dt == DSA_KV_FP8_E4M3, n_slots, kv_slot_table, kv_pt_ld, q_seq, idx,
                   n_q, h, k, sm_scale, out, lse};
    hipError_t e = dsa::launch_mla_decode(a, n_splits, ws, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "dsa_sparse_mla_decode launch");
    return DSA_OK;
}

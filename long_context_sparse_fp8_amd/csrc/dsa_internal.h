// dsa_internal.h -- launchers behind the C ABI (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Calls with at most this many queries use the split-key indexer (decode
// shape); larger calls use the query-blocked one (prefill shape).
constexpr int kIndexerDecodeMaxQ = 256;

// Indexer key pages (64 keys of d_i E4M3 bytes) are stored fragment-major: the
// page is a run of 1 KB blocks, block ((kt * d_i / 64) + c) * 2 + h holding in
// slot l (16 bytes) the bytes 32 c + 16 h .. +16 of the lane-group half
// g = l / 32 (bytes [g d_i / 2, (g + 1) d_i / 2)) of key 32 kt + l % 32.  That
// is exactly the B operand of the FP8 MFMA of the scorers (lane l: key l % 32,
// K bytes of group g), so a wave reads each block as one contiguous 1 KB load.
// Byte offset within the page of bytes 16 piece .. +16 of key `key`:
__host__ __device__ constexpr int idx_key_piece_offset(int key, int piece, int d_i) {
    const int half = d_i / 2, o = 16 * piece;
    const int g = o / half, c = (o % half) / 32, h = (o % 32) / 16;
    return (((key / 32) * (d_i / 64) + c) * 2 + h) * 1024 + (32 * g + key % 32) * 16;
}

// Top-k limits: k <= kTopkMaxK, score rows of at most kTopkMaxRow columns.
constexpr int kTopkMaxK = 2048;
constexpr int64_t kTopkMaxRow = 262144;
// Workspace of the fused indexer -> top-k call: one block of kFusedRowStride
// words per query row t (at t * kFusedRowStride, so calls with fewer rows use
// a prefix of it), holding
//   * kFusedRowWords words that must be zero before the call and are left zero
//     by it: the row's first-digit histogram (order-preserving key bits
//     31..21, built by the split-key scorer), then the selection's part
//     ticket, candidate count and overflow flag;
//   * scratch: the row's bitmap of kept indices and its candidate list.
constexpr int kTopkHistBins = 2048;
constexpr int kFusedRowWords = kTopkHistBins + 16;
constexpr int kFusedCand = 8192;                                   // candidate list capacity per row
constexpr int64_t kFusedScratchWords = kTopkMaxRow / 32 + 2 * kFusedCand;
constexpr int64_t kFusedRowStride = kFusedRowWords + kFusedScratchWords;
constexpr size_t fused_topk_ws_bytes(int32_t n_q) {
    return (size_t)n_q * (size_t)kFusedRowStride * sizeof(uint32_t);
}

struct IndexerArgs {
    const uint8_t *q_fp8;
    const float *q_scale;
    const float *w;
    int64_t w_ld;
    const uint8_t *key_cache;
    const float *key_scale;
    int64_t n_pages;
    const int32_t *page_table;
    int64_t pt_ld;
    const int32_t *q_seq;
    const int32_t *q_pos;
    int32_t n_q, h_i, d_i;
    float *scores;
    int64_t scores_ld;
    uint32_t *hist = nullptr;   // row t's histogram at hist + t * kFusedRowStride (zeroed): accumulated into
};

struct MlaArgs {
    const uint16_t *q;
    const void *kv_cache;
    const float *kv_scale;
    bool fp8;
    int64_t n_slots;
    const int32_t *kv_slot_table;
    int64_t kv_pt_ld;
    const int32_t *q_seq;
    const int32_t *idx;
    int32_t n_q, h, k;
    float sm_scale;
    uint16_t *out;
    float *lse;
};

hipError_t launch_indexer_store(const uint8_t *k, const float *ks, const int64_t *slot, int32_t n, int32_t d_i,
                                uint8_t *cache, float *scache, int64_t n_pages, hipStream_t stream);
hipError_t launch_kv_store(const uint16_t *kv, const int64_t *slot, int32_t n, int dt, void *cache, float *scale,
                           int64_t n_slots, hipStream_t stream);
// both stores in one launch (n_keys or n_kv may be 0)
hipError_t launch_cache_store(const uint8_t *k, const float *ks, const int64_t *key_slot, int32_t n_keys, int32_t d_i,
                              uint8_t *key_cache, float *key_scache, int64_t n_pages, const uint16_t *kv,
                              const int64_t *kv_slot, int32_t n_kv, int dt, void *kv_cache, float *kv_scale,
                              int64_t n_slots, hipStream_t stream);
hipError_t launch_indexer(const IndexerArgs &a, hipStream_t stream);
hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *q_pos, int32_t n_q, int32_t k, int32_t *idx,
                       void *ws, size_t ws_bytes, hipStream_t stream);
// Top-k of rows whose first-digit histograms the split-key scorer accumulated
// in the fused workspace `ws` (fused_topk_ws_bytes(n_q) bytes, laid out as
// above; the regions that must be zero are left zero).
hipError_t launch_topk_fused(const float *scores, int64_t ld, const int32_t *q_pos, int32_t n_q, int32_t k,
                             int32_t *idx, uint32_t *ws, hipStream_t stream);
// Workspace that lets dsa_topk split few long rows over several workgroups
// (0 when it does not split at these sizes).
size_t topk_ws_bytes(int32_t n_q, int64_t ld, int32_t k);
// The current device's static top-k workspace (looked up once per device) and its size.
hipError_t topk_static_workspace(void **ptr, size_t *bytes);
hipError_t launch_mla_prefill(const MlaArgs &a, hipStream_t stream);
hipError_t launch_mla_decode(const MlaArgs &a, int n_splits, void *ws, hipStream_t stream);
int mla_decode_auto_splits(int32_t n_q, int32_t h, int32_t k);
size_t mla_decode_ws_bytes(int32_t n_q, int32_t h, int32_t n_splits);

}  // namespace dsa

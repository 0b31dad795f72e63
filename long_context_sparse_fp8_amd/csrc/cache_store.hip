// cache_store.hip -- scatter new tokens into the two DSA caches.
//
//  * indexer key & key_scale cache, page size 64 (SGLang day-0 DeepSeek-V3.2
//    announcement, "DeepSeek Sparse Attention"): a byte copy of each token's
//    E4M3 key and its fp32 scale to slot = page * 64 + offset;
//  * token-granular latent KV cache (page size 1): a bf16 row copy, or
//    per-token FP8 quantization for the "kv_cache_dtype fp8_e4m3" cache of
//    the deployment article (section 3): scale = amax / 448, code =
//    E4M3(x / scale) with IEEE division, round to nearest even, saturating.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

// Thread `gid` of the key store: one 16-byte chunk of a key (d_i / 16 per key).
__device__ __forceinline__ void indexer_store_chunk(int64_t gid, const uint8_t *__restrict__ k,
                                                    const float *__restrict__ ks, const int64_t *__restrict__ slot,
                                                    int32_t n, int32_t d_i, uint8_t *__restrict__ cache,
                                                    float *__restrict__ scache, int64_t n_slots) {
    const int chunks = d_i / 16;
    const int64_t tok = gid / chunks;
    const int c = (int)(gid - tok * chunks);
    if (tok >= n) return;
    const int64_t sl = slot[tok];
    if (sl < 0 || sl >= n_slots) return;
    const uint4 v = reinterpret_cast<const uint4 *>(k + tok * d_i)[c];
    const int64_t page = sl / kPage;
    const int key = (int)(sl - page * kPage);
    *reinterpret_cast<uint4 *>(cache + page * (kPage * d_i) + idx_key_piece_offset(key, c, d_i)) = v;
    if (c == 0) scache[sl] = ks[tok];
}

// Thread `gid` of the bf16 latent store: one 16-byte chunk of a row (72 per row).
__device__ __forceinline__ void kv_store_bf16_chunk(int64_t gid, const uint16_t *__restrict__ kv,
                                                    const int64_t *__restrict__ slot, int32_t n,
                                                    uint16_t *__restrict__ cache, int64_t n_slots) {
    constexpr int kChunks = kDk * 2 / 16;
    const int64_t tok = gid / kChunks;
    const int c = (int)(gid - tok * kChunks);
    if (tok >= n) return;
    const int64_t sl = slot[tok];
    if (sl < 0 || sl >= n_slots) return;
    reinterpret_cast<uint4 *>(cache + sl * kDk)[c] = reinterpret_cast<const uint4 *>(kv + tok * kDk)[c];
}

// FP8 latent store of token `tok` by one whole wave (tok is wave-uniform): lane
// l owns elements l + 64 j, j < 9.
__device__ __forceinline__ void kv_store_fp8_row(int64_t tok, int lane, const uint16_t *__restrict__ kv,
                                                 const int64_t *__restrict__ slot, int32_t n,
                                                 uint8_t *__restrict__ cache, float *__restrict__ scale_out,
                                                 int64_t n_slots) {
    constexpr int kPer = kDk / kWave;  // 9
    if (tok >= n) return;
    const int64_t sl = slot[tok];
    if (sl < 0 || sl >= n_slots) return;
    float x[kPer];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        x[j] = bf16_bits_to_f32(kv[tok * kDk + lane + kWave * j]);
        amax = fmaxf(amax, __builtin_fabsf(x[j]));
    }
    amax = wave_max(amax);
    const float scale = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        cache[sl * kDk + lane + kWave * j] = (uint8_t)f32_to_e4m3(__fdiv_rn(x[j], scale));
    if (lane == 0) scale_out[sl] = scale;
}

__global__ __launch_bounds__(256) void indexer_store_kernel(const uint8_t *__restrict__ k, const float *__restrict__ ks,
                                                            const int64_t *__restrict__ slot, int32_t n, int32_t d_i,
                                                            uint8_t *__restrict__ cache, float *__restrict__ scache,
                                                            int64_t n_slots) {
    indexer_store_chunk((int64_t)blockIdx.x * blockDim.x + threadIdx.x, k, ks, slot, n, d_i, cache, scache, n_slots);
}

__global__ __launch_bounds__(256) void kv_store_bf16_kernel(const uint16_t *__restrict__ kv,
                                                            const int64_t *__restrict__ slot, int32_t n,
                                                            uint16_t *__restrict__ cache, int64_t n_slots) {
    kv_store_bf16_chunk((int64_t)blockIdx.x * blockDim.x + threadIdx.x, kv, slot, n, cache, n_slots);
}

// four tokens per 256-thread block
__global__ __launch_bounds__(256) void kv_store_fp8_kernel(const uint16_t *__restrict__ kv,
                                                            const int64_t *__restrict__ slot, int32_t n,
                                                            uint8_t *__restrict__ cache,
                                                            float *__restrict__ scale_out, int64_t n_slots) {
    kv_store_fp8_row((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6), threadIdx.x & 63, kv, slot, n, cache, scale_out,
                     n_slots);
}

// Both stores in one launch: blocks [0, key_blocks) store keys, the rest latent
// rows (the branch is uniform per block).  A step's new tokens are few, so each
// store alone is a short launch whose fixed cost exceeds its work.
template <bool FP8>
__global__ __launch_bounds__(256) void cache_store_kernel(const uint8_t *__restrict__ k, const float *__restrict__ ks,
                                                          const int64_t *__restrict__ key_slot, int32_t n_keys,
                                                          int32_t d_i, uint8_t *__restrict__ key_cache,
                                                          float *__restrict__ key_scache, int64_t n_key_slots,
                                                          int64_t key_blocks, const uint16_t *__restrict__ kv,
                                                          const int64_t *__restrict__ kv_slot, int32_t n_kv,
                                                          void *__restrict__ kv_cache, float *__restrict__ kv_scale,
                                                          int64_t n_slots) {
    const int64_t b = blockIdx.x;
    if (b < key_blocks) {
        indexer_store_chunk(b * 256 + threadIdx.x, k, ks, key_slot, n_keys, d_i, key_cache, key_scache, n_key_slots);
    } else if constexpr (FP8) {
        kv_store_fp8_row((b - key_blocks) * 4 + (threadIdx.x >> 6), threadIdx.x & 63, kv, kv_slot, n_kv,
                         (uint8_t *)kv_cache, kv_scale, n_slots);
    } else {
        kv_store_bf16_chunk((b - key_blocks) * 256 + threadIdx.x, kv, kv_slot, n_kv, (uint16_t *)kv_cache, n_slots);
    }
}

hipError_t launch_indexer_store(const uint8_t *k, const float *ks, const int64_t *slot, int32_t n, int32_t d_i,
                                uint8_t *cache, float *scache, int64_t n_pages, hipStream_t stream) {
    const int64_t threads = (int64_t)n * (d_i / 16);
    const int block = 256;
    const int64_t grid = (threads + block - 1) / block;
    hipLaunchKernelGGL(indexer_store_kernel, dim3((unsigned)grid), dim3(block), 0, stream, k, ks, slot, n, d_i,
                       cache, scache, n_pages * kPage);
    return hipGetLastError();
}

hipError_t launch_kv_store(const uint16_t *kv, const int64_t *slot, int32_t n, int dt, void *cache, float *scale,
                           int64_t n_slots, hipStream_t stream) {
    if (dt == 0) {
        const int64_t threads = (int64_t)n * (kDk * 2 / 16);
        const int64_t grid = (threads + 255) / 256;
        hipLaunchKernelGGL(kv_store_bf16_kernel, dim3((unsigned)grid), dim3(256), 0, stream, kv, slot, n,
                           (uint16_t *)cache, n_slots);
    } else {
        const int64_t grid = ((int64_t)n + 3) / 4;
        hipLaunchKernelGGL(kv_store_fp8_kernel, dim3((unsigned)grid), dim3(256), 0, stream, kv, slot, n,
                           (uint8_t *)cache, scale, n_slots);
    }
    return hipGetLastError();
}

hipError_t launch_cache_store(const uint8_t *k, const float *ks, const int64_t *key_slot, int32_t n_keys, int32_t d_i,
                              uint8_t *key_cache, float *key_scache, int64_t n_pages, const uint16_t *kv,
                              const int64_t *kv_slot, int32_t n_kv, int dt, void *kv_cache, float *kv_scale,
                              int64_t n_slots, hipStream_t stream) {
    const int64_t key_blocks = ((int64_t)n_keys * (d_i / 16) + 255) / 256;
    const int64_t kv_blocks = dt == 0 ? ((int64_t)n_kv * (kDk * 2 / 16) + 255) / 256 : ((int64_t)n_kv + 3) / 4;
    const dim3 grid((unsigned)(key_blocks + kv_blocks));
    if (dt == 0)
        hipLaunchKernelGGL(cache_store_kernel<false>, grid, dim3(256), 0, stream, k, ks, key_slot, n_keys, d_i,
                           key_cache, key_scache, n_pages * kPage, key_blocks, kv, kv_slot, n_kv, kv_cache, kv_scale,
                           n_slots);
    else
        hipLaunchKernelGGL(cache_store_kernel<true>, grid, dim3(256), 0, stream, k, ks, key_slot, n_keys, d_i,
                           key_cache, key_scache, n_pages * kPage, key_blocks, kv, kv_slot, n_kv, kv_cache, kv_scale,
                           n_slots);
    return hipGetLastError();
}

}  // namespace dsa

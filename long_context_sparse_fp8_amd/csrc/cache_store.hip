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

// one thread per 16-byte chunk of a key
__global__ void indexer_store_kernel(const uint8_t *__restrict__ k, const float *__restrict__ ks,
                                     const int64_t *__restrict__ slot, int32_t n, int32_t d_i,
                                     uint8_t *__restrict__ cache, float *__restrict__ scache,
                                     int64_t n_slots) {
    const int chunks = d_i / 16;
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t tok = gid / chunks;
    int c = (int)(gid - tok * chunks);
    if (tok >= n) return;
    int64_t sl = slot[tok];
    if (sl < 0 || sl >= n_slots) return;
    const uint4 v = reinterpret_cast<const uint4 *>(k + tok * d_i)[c];
    const int64_t page = sl / kPage;
    const int key = (int)(sl - page * kPage);
    *reinterpret_cast<uint4 *>(cache + page * (kPage * d_i) + idx_key_piece_offset(key, c, d_i)) = v;
    if (c == 0) scache[sl] = ks[tok];
}

// bf16 cache: one thread per 16-byte chunk (72 per row)
__global__ void kv_store_bf16_kernel(const uint16_t *__restrict__ kv, const int64_t *__restrict__ slot,
                                     int32_t n, uint16_t *__restrict__ cache, int64_t n_slots) {
    constexpr int kChunks = kDk * 2 / 16;
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t tok = gid / kChunks;
    int c = (int)(gid - tok * kChunks);
    if (tok >= n) return;
    int64_t sl = slot[tok];
    if (sl < 0 || sl >= n_slots) return;
    reinterpret_cast<uint4 *>(cache + sl * kDk)[c] = reinterpret_cast<const uint4 *>(kv + tok * kDk)[c];
}

// FP8 cache: one wave per token row; lane l owns elements l + 64 j, j < 9
__global__ __launch_bounds__(256) void kv_store_fp8_kernel(const uint16_t *__restrict__ kv,
                                                            const int64_t *__restrict__ slot, int32_t n,
                                                            uint8_t *__restrict__ cache,
                                                            float *__restrict__ scale_out, int64_t n_slots) {
    constexpr int kPer = kDk / kWave;  // 9
    const int lane = threadIdx.x & 63;
    int64_t tok = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6);
    if (tok >= n) return;
    int64_t sl = slot[tok];
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

}  // namespace dsa

// topk.hip -- per-row top-k selection by radix select (gfx950).
//
// Keeps the k best of scores[t, 0..q_pos[t]] under (score descending, index
// ascending) -- the "top-k token selection" of the SGLang DeepSeek-V3.2
// announcement -- and writes them in ascending index order, -1 padded.  A
// row with no more than k candidates keeps all of them (the dense
// degeneration of the deployment article, section 5.1).
//
// Scores become order-preserving uint32 keys.  Four MSB-first passes with
// 8-bit digits find the k-th largest key T and how many keys equal to T must
// be taken (`need`); the histograms live in LDS, one private copy per wave
// so the ~16 busiest bins of a normal-shaped row do not serialize the whole
// workgroup.  A final pass walks the row in index order and keeps keys > T
// plus the first `need` keys == T, placing each kept index with wavefront
// ballot / popcount prefix sums.  Everything is integer: the selection is
// exact for the given scores.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;

__device__ __forceinline__ uint32_t lane_prefix_count(uint64_t mask, int lane) {
    return __builtin_popcountll(mask & ((1ull << lane) - 1ull));
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float *__restrict__ scores, int64_t ld,
                                                             const int32_t *__restrict__ q_pos, int32_t k,
                                                             int32_t *__restrict__ idx) {
    __shared__ uint32_t hist[kTopkWaves][256];
    __shared__ uint32_t total[256];
    __shared__ uint32_t sel_bin, sel_rem;
    __shared__ uint32_t wcnt[2][kTopkWaves];

    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int64_t n = (int64_t)q_pos[t] + 1;
    if (n > ld) n = ld;
    if (n < 0) n = 0;
    const float *row = scores + (int64_t)t * ld;
    int32_t *out = idx + (int64_t)t * k;

    if (n <= k) {   // every candidate is kept
        for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
        return;
    }

    uint32_t prefix = 0, pmask = 0, rem = (uint32_t)k;   // rem: how many still to take at/below the prefix
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < kTopkWaves * 256; i += kTopkThreads) (&hist[0][0])[i] = 0;
        __syncthreads();
        for (int64_t i = tid; i < n; i += kTopkThreads) {
            const uint32_t key = f32_order_key(row[i]);
            if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 256) {
            uint32_t s = 0;
#pragma unroll
            for (int wv = 0; wv < kTopkWaves; ++wv) s += hist[wv][tid];
            total[tid] = s;
        }
        __syncthreads();
        // bins from the top: find the bin holding the rem-th largest key.
        // Threads 0..255 (4 waves) own bin 255 - tid: an inclusive scan within
        // each wave, then the preceding waves' totals are added.
        uint32_t v = 0, incl = 0;
        if (tid < 256) {
            v = total[255 - tid];
            incl = v;
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t u = __shfl_up(incl, o);
                if (lane >= o) incl += u;
            }
            if (lane == 63) wcnt[0][wave] = incl;
        }
        __syncthreads();
        if (tid < 256) {
            for (int wv = 0; wv < wave; ++wv) incl += wcnt[0][wv];
            const uint32_t excl = incl - v;
            if (excl < rem && incl >= rem) {
                sel_bin = 255u - (uint32_t)tid;
                sel_rem = rem - excl;
            }
        }
        __syncthreads();
        const uint32_t b = sel_bin;
        rem = sel_rem;
        prefix |= b << shift;
        pmask |= 255u << shift;
        __syncthreads();
    }
    const uint32_t T = prefix;
    const uint32_t need = rem;       // keys equal to T to take, lowest indices first

    // ordered compaction
    uint32_t eq_seen = 0, out_pos = 0;
    for (int64_t base = 0; base < n; base += kTopkThreads) {
        const int64_t i = base + tid;
        uint32_t key = 0;
        if (i < n) key = f32_order_key(row[i]);
        const bool gt = i < n && key > T;
        const bool eq = i < n && key == T;
        const uint64_t beq = __ballot(eq);
        if (lane == 0) wcnt[0][wave] = (uint32_t)__builtin_popcountll(beq);
        __syncthreads();
        uint32_t eq_before = eq_seen;
        uint32_t eq_chunk = 0;
        for (int wv = 0; wv < kTopkWaves; ++wv) {
            const uint32_t c = wcnt[0][wv];
            if (wv < wave) eq_before += c;
            eq_chunk += c;
        }
        eq_before += lane_prefix_count(beq, lane);
        const bool sel = gt || (eq && eq_before < need);
        const uint64_t bsel = __ballot(sel);
        if (lane == 0) wcnt[1][wave] = (uint32_t)__builtin_popcountll(bsel);
        __syncthreads();
        uint32_t pos = out_pos, sel_chunk = 0;
        for (int wv = 0; wv < kTopkWaves; ++wv) {
            const uint32_t c = wcnt[1][wv];
            if (wv < wave) pos += c;
            sel_chunk += c;
        }
        pos += lane_prefix_count(bsel, lane);
        if (sel && pos < (uint32_t)k) out[pos] = (int32_t)i;
        eq_seen += eq_chunk;
        out_pos += sel_chunk;
        __syncthreads();
        if (out_pos >= (uint32_t)k) break;
    }
}

hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *q_pos, int32_t n_q, int32_t k, int32_t *idx,
                       hipStream_t stream) {
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)n_q), dim3(kTopkThreads), 0, stream, scores, ld, q_pos, k, idx);
    return hipGetLastError();
}

}  // namespace dsa

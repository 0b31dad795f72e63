// sparse_mla.hip -- attention over the top-k selected latent rows (gfx950).
//
// For query t, head h and the selected set S_t (DeepSeek-V3.2-Exp deployment
// article, section 1: only the top-k key/value entries enter attention; SGLang
// usage guide, "attention kernel selection": bf16 q with bf16 or fp8 kv):
//   l_s = sm_scale * q[t,h,:] . K[s,:]   (576-d latent keys)
//   out[t,h,:] = softmax(l) @ K[S_t, :512],  lse[t,h] = log sum exp(l)
//
// One workgroup per query (decode: per query and index split).  Every wave
// owns 32 heads, so 128 heads are 4 waves, one per SIMD; Q^T (144 VGPRs) and
// the fp32 O^T accumulator (256) stay in registers for the whole query.  Each
// gathered row is read from memory once per query and shared by all heads
// through LDS.  Per 64-row tile:
//   * the selected rows are gathered straight into LDS with
//     global_load_lds_dwordx4 (no register staging), double-buffered, rows
//     padded to 1168 bytes and the MFMA rows mapped to tile rows so that both
//     the row reads and the transposed reads below are bank-conflict free;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = 32 gathered rows from LDS,
//     B = the wave's 32 query heads held in VGPRs): each 16-byte LDS fragment
//     feeds 32 heads, which halves LDS traffic per flop against 16-head tiles;
//   * softmax per head (= per lane column) in the exp2 domain against a fixed
//     reference: the head's maximum over its first tile.  Probabilities of later
//     tiles may exceed 1 by up to 2^64 before the reference must move; that
//     range is exact in fp32 sums and bf16 probabilities, and the final division
//     gives the same softmax as a running-max rescale.  A tile beyond it restarts
//     the query with a raised reference instead of rescaling the accumulators,
//     which keeps O^T in accumulation registers that VALU code never touches;
//   * O^T += V^T P^T: P^T is the S^T accumulator re-packed to bf16 in place
//     (its lane layout already is the B operand, with the k index permuted
//     consistently on both operands), V^T comes from the same LDS tile through
//     ds_read_b64_tr_b16 transposed reads.
// FP8 rows (E4M3 + per-row scale) are gathered as bytes, expanded to bf16 in
// LDS exactly, and their scale is applied to the logits and to P in fp32.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kTile = 64;                         // gathered rows per tile
constexpr int kRowB = kDk * 2 + 16;               // padded bf16 LDS row, bytes (1168)
constexpr int kRowC = kRowB / 16;                 // 16-byte chunks per padded row (73)
constexpr int kTileB = kTile * kRowB;             // 74752 bytes
constexpr int kF8RowC = kDk / 16;                 // 16-byte chunks per FP8 row (36)
constexpr int kF8TileB = kTile * kDk;             // 36864 bytes
constexpr int kMaxK = 2048;
constexpr int kKSteps = kDk / 16;                 // 36 k-steps of 16 latent dims
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kHeadroom = 64.0f;                // log2 range allowed above a head's reference max
constexpr int kLookK = 4;                         // K fragments in flight per wave
constexpr int kLookV = 4;                         // V^T fragments in flight per wave

typedef __attribute__((address_space(3))) void lds_void;

// 16-byte asynchronous global -> LDS copies: lane l of the wave writes
// lds_base + 16 * l.
__device__ __forceinline__ void g2lds16(const void *gsrc, lds_void *lds_base) {
    __builtin_amdgcn_global_load_lds(gsrc, lds_base, 16, 0, 0);
}

__device__ __forceinline__ lds_void *to_lds(void *p) { return (lds_void *)(p); }

__device__ __forceinline__ bf16x4 lds_tr16(const uint8_t *p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(const_cast<uint8_t *>(p)));
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ f32x16 mfma32_bf16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Tile rows are padded to 1168 bytes (73 16-byte chunks): 16 consecutive rows
// then start on 16 distinct chunk columns modulo 16, so the row reads (16 lanes =
// 16 rows x 16 bytes per cycle on gfx950's 64 banks) are conflict-free.  The
// transposed reads fetch 4 rows x 32 bytes per 16-lane group; they are
// conflict-free when those 4 rows are 4 apart.  So the MFMA row index rho (the
// S^T accumulator row, and the k index of the PV product) maps to the tile row
// tau(rho) that transposes the 4x4 blocks of every 16 rows:
//   tau(16 B + 4 a + b) = 16 B + 4 b + a,
// under which each transposed read's 4 consecutive k slots are tile rows 4
// apart, and every fragment address is one per-lane base plus a constant.
__device__ __forceinline__ int tau(int rho) { return (rho & ~15) | ((rho & 3) << 2) | ((rho >> 2) & 3); }

// Tile buffers live in separate __shared__ arrays, each named statically at every
// use, so that the compiler can tell the asynchronous gather into one buffer from
// the reads of the other and does not make the reads wait for the gather.
template <int NW, bool FP8, bool SPLIT>
struct MlaSmem {
    float f8scale[FP8 ? kTile : 1];
    int32_t slots[kMaxK];
    uint32_t wcount[NW];
    int32_t n_valid;
    uint32_t restart;
};

template <int NW, bool FP8, bool SPLIT>
__global__ __launch_bounds__(NW * 64, 1) void sparse_mla_kernel(
    const uint16_t *__restrict__ q, const void *__restrict__ kv_cache, const float *__restrict__ kv_scale,
    int64_t n_slots, const int32_t *__restrict__ kv_slot_table, int64_t kv_pt_ld, const int32_t *__restrict__ q_seq,
    const int32_t *__restrict__ idx, int32_t h, int32_t k, float sm_scale, uint16_t *__restrict__ out,
    float *__restrict__ lse, int32_t n_splits, float *__restrict__ ws_o, float *__restrict__ ws_lse) {
    constexpr int NT = NW * 64;
    constexpr int R = (kMaxK + NT - 1) / NT;      // index entries per thread
    __shared__ __attribute__((aligned(16))) MlaSmem<NW, FP8, SPLIT> sm;
    // bf16 cache: tile_a / tile_b double buffer.  FP8 cache: codes staged in
    // f8_a / f8_b (double buffer), expanded into tile_a.
    __shared__ __attribute__((aligned(16))) uint8_t tile_a[kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t tile_b[FP8 ? 16 : kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t f8_a[FP8 ? kF8TileB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t f8_b[FP8 ? kF8TileB : 16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;     // lane half, lane within the half
    const int i16 = lane & 15, hd = (lane >> 4) & 1;
    const int t = SPLIT ? (int)blockIdx.x / n_splits : (int)blockIdx.x;
    const int split = SPLIT ? (int)blockIdx.x % n_splits : 0;
    const int per_split = SPLIT ? (k + n_splits - 1) / n_splits : k;
    const int i_begin = split * per_split;
    const int i_end = min(k, i_begin + per_split);
    const int head = 32 * wave + l32;
    const bool head_ok = head < h;

    // ---- resolve the selected rows to cache slots, compacted in index order
    {
        const int32_t *idx_row = idx + (int64_t)t * k;
        const int32_t *st_row = kv_slot_table + (int64_t)q_seq[t] * kv_pt_ld;
        int32_t s[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = i_begin + tid + NT * r;
            s[r] = i < i_end ? idx_row[i] : -1;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int32_t sl = -1;
            if (s[r] >= 0 && s[r] < kv_pt_ld) {
                const int32_t v = st_row[s[r]];
                if (v >= 0 && v < n_slots) sl = v;
            }
            s[r] = sl;
        }
        int base = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (i_begin + NT * r >= i_end) break;     // uniform
            const bool ok = s[r] >= 0;
            const uint64_t bal = __ballot(ok);
            if (lane == 0) sm.wcount[wave] = (uint32_t)__builtin_popcountll(bal);
            __syncthreads();
            int before = base, tot = 0;
#pragma unroll
            for (int wv = 0; wv < NW; ++wv) {
                const int c = (int)sm.wcount[wv];
                if (wv < wave) before += c;
                tot += c;
            }
            if (ok) sm.slots[before + (int)__builtin_popcountll(bal & ((1ull << lane) - 1ull))] = s[r];
            base += tot;
            __syncthreads();
        }
        if (tid == 0) {
            sm.n_valid = base;
            sm.restart = 0;
        }
    }
    __syncthreads();
    const int n_valid = sm.n_valid;
    const int n_tiles = (n_valid + kTile - 1) / kTile;

    // ---- Q^T fragments of this wave's 32 heads (B operand): k-step ks holds
    // latent dims 16 ks + 8 g .. +8 of head `head`
    bf16x8 qf[kKSteps];
    {
        const uint16_t *qrow = q + ((int64_t)t * h + (head_ok ? head : 0)) * kDk + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (head_ok) v = *reinterpret_cast<const uint4 *>(qrow + 16 * ks);
            qf[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // ---- tile gather (asynchronous, straight to LDS, swizzled through the source addresses)
    auto gather = [&](int j, uint8_t *dst) {
        const int row0 = j * kTile;
        const uint8_t *kvb = reinterpret_cast<const uint8_t *>(kv_cache);
        if constexpr (!FP8) {
            for (int ins = wave; ins < kRowC; ins += NW) {   // 73 wave-wide 1 KB copies
                const int c = ins * 64 + lane;
                const int r = c / kRowC, col = c - r * kRowC;
                const int rr = row0 + r < n_valid ? row0 + r : 0;
                const int64_t sl = sm.slots[rr];
                // the pad chunk (col 72) takes a duplicate of chunk 71
                g2lds16(kvb + sl * (kDk * 2) + (col < kRowC - 1 ? col : kRowC - 2) * 16, to_lds(dst + ins * 1024));
            }
        } else {
            for (int ins = wave; ins < kF8RowC; ins += NW) {  // 36 wave-wide 1 KB copies
                const int c = ins * 64 + lane;
                const int r = c / kF8RowC, col = c - r * kF8RowC;
                const int rr = row0 + r < n_valid ? row0 + r : 0;
                const int64_t sl = sm.slots[rr];
                g2lds16(kvb + sl * kDk + col * 16, to_lds(dst + ins * 1024));
            }
        }
    };
    // FP8: expand the staged codes of tile j into the bf16 tile (exact), fetch row scales
    auto expand = [&](int j, const uint8_t *src, uint8_t *dst_tile) {
        if constexpr (FP8) {
            const int row0 = j * kTile;
            for (int c = tid; c < kTile * kF8RowC; c += NT) {
                const int r = c / kF8RowC, col = c - r * kF8RowC;
                const uint4 v = *reinterpret_cast<const uint4 *>(&src[r * kDk + col * 16]);
                const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
                uint32_t o8[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)wds[e], false);   // bytes 0, 1
                    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)wds[e], true);    // bytes 2, 3
                    bf16x2 b0 = {(__bf16)lo[0], (__bf16)lo[1]};
                    bf16x2 b1 = {(__bf16)hi[0], (__bf16)hi[1]};
                    o8[2 * e] = __builtin_bit_cast(uint32_t, b0);
                    o8[2 * e + 1] = __builtin_bit_cast(uint32_t, b1);
                }
                uint4 *d = reinterpret_cast<uint4 *>(&dst_tile[r * kRowB + col * 32]);
                d[0] = make_uint4(o8[0], o8[1], o8[2], o8[3]);
                d[1] = make_uint4(o8[4], o8[5], o8[6], o8[7]);
            }
            if (tid < kTile) {
                const int rr = row0 + tid < n_valid ? row0 + tid : 0;
                sm.f8scale[tid] = kv_scale[sm.slots[rr]];
            }
        }
    };

    // Per-lane LDS byte offsets within a tile.  K fragment (k-step ks, half hf): tile
    // row tau(l32) + 32 hf, dims 16 ks + 8 g  -> k_base + 32 hf rows + 32 ks bytes.
    // V^T fragment (k-step kk, dim tile dt): k slots 8 g + e (e < 4) are rho =
    // 16 kk + 4 g + e (lo) and rho + 8 (hi), i.e. tile rows 16 kk + 4 e + g and
    // 16 kk + 4 e + g + 2; lane i16 of a 16-lane group supplies row e = i16 / 4,
    // dims 32 dt + 16 hd + 4 (i16 % 4)  -> v_base + 16 kk rows + 64 dt bytes (+2 rows).
    const int k_base = tau(l32) * kRowB + 16 * g;
    const int v_base = (4 * (i16 >> 2) + g) * kRowB + 32 * hd + 8 * (i16 & 3);

    // O^T accumulators: o[dt][i] holds latent dim 32 dt + 8 (i / 4) + 4 g + i % 4 of head `head`
    f32x16 o[16];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
    // Softmax reference: each head's maximum over its first tile.  Later tiles are
    // exponentiated against it as long as their maximum stays within kHeadroom
    // (log2 units) of it, which fp32 sums and bf16 probabilities hold exactly as
    // the rescaled form would; a tile beyond that restarts the query with the
    // larger reference, so the accumulators are never rescaled.
    float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.0f;
    const float c2 = sm_scale * kLog2e;

    // Attempts: the second and later ones only run after a tile exceeded its head's
    // reference by more than kHeadroom (practically never); they restart from tile
    // 0 with every reference raised to the largest maximum seen so far.
    bool again = true;
    while (again) {
        // one tile: `cur` holds tile j (bf16 rows, or FP8 codes to expand), the gather
        // of tile j + 1 goes to `nxt`; returns true when the query must restart
        auto step = [&](const int j, uint8_t *cur, uint8_t *nxt) -> bool {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();                              // tile j landed; everyone is done with tile j-1
            if (sm.restart != 0) return true;             // workgroup-uniform; nothing is in flight
            if (j + 1 < n_tiles) gather(j + 1, nxt);
            const uint8_t *tile = cur;
            if constexpr (FP8) {
                expand(j, cur, tile_a);
                __syncthreads();
                tile = tile_a;
            }

            // S^T = K Q^T: s[hf] covers rho = 32 hf + 8 (i / 4) + 4 g + i % 4.  The 72
            // (k-step, half) fragment loads run kLookK steps ahead of their MFMA in a
            // register ring; the scheduling barriers keep that order.
            f32x16 s[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[hf][i] = 0.0f;
            {
                const uint8_t *kb = tile + k_base;
                auto kload = [&](int f) {
                    return *reinterpret_cast<const uint4 *>(kb + (f & 1) * 32 * kRowB + 32 * (f >> 1));
                };
                uint4 ring[kLookK];
#pragma unroll
                for (int f = 0; f < kLookK; ++f) ring[f] = kload(f);
#pragma unroll
                for (int f = 0; f < 2 * kKSteps; ++f) {
                    const uint4 cur = ring[f % kLookK];
                    if (f + kLookK < 2 * kKSteps) ring[f % kLookK] = kload(f + kLookK);
                    s[f & 1] = mfma32_bf16(__builtin_bit_cast(bf16x8, cur), qf[f >> 1], s[f & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            // softmax (exp2 domain) per head = per lane column; lanes l and l ^ 32 hold
            // disjoint rows of the same head
            const int row0 = j * kTile;
            float tmax = -INFINITY;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = tau(32 * hf + 8 * (i >> 2) + 4 * g + (i & 3));   // tile row
                    float x = s[hf][i] * c2;
                    if constexpr (FP8) x *= sm.f8scale[r];
                    x = (row0 + r < n_valid) ? x : -INFINITY;
                    s[hf][i] = x;
                    tmax = fmaxf(tmax, x);
                }
            }
            tmax = fmaxf(tmax, swap_halves(tmax));
            m_seen = fmaxf(m_seen, tmax);
            if (m_ref == -INFINITY) m_ref = tmax;             // first tile of this head: nothing accumulated yet
            if (__ballot(tmax > m_ref + kHeadroom) != 0) sm.restart = 1u;   // acted on after the next barrier
            const float m_use = m_ref == -INFINITY ? 0.0f : m_ref;
            float psum = 0.0f;
            bf16x8 pb[4];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float p = __builtin_amdgcn_exp2f(s[hf][i] - m_use);
                    psum += p;
                    if constexpr (FP8) p *= sm.f8scale[tau(32 * hf + 8 * (i >> 2) + 4 * g + (i & 3))];
                    pb[2 * hf + (i >> 3)][i & 7] = (__bf16)p;
                }
            }
            l_run += psum;

            // O^T += V^T P^T: k-step kk covers rho 16 kk + {4 g + e} u {16 kk + 8 + 4 g + e},
            // dim tile dt covers dims 32 dt .. +32.  Same bounded look-ahead as above.
            {
                const uint8_t *vb = tile + v_base;
                auto vload = [&](int f, bf16x4 &lo, bf16x4 &hi) {
                    const uint8_t *p = vb + (f >> 4) * 16 * kRowB + 64 * (f & 15);
                    lo = lds_tr16(p);
                    hi = lds_tr16(p + 2 * kRowB);
                };
                bf16x4 rlo[kLookV], rhi[kLookV];
#pragma unroll
                for (int f = 0; f < kLookV; ++f) vload(f, rlo[f], rhi[f]);
#pragma unroll
                for (int f = 0; f < 64; ++f) {
                    const bf16x4 lo = rlo[f % kLookV], hi = rhi[f % kLookV];
                    if (f + kLookV < 64) vload(f + kLookV, rlo[f % kLookV], rhi[f % kLookV]);
                    const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    o[f & 15] = mfma32_bf16(a, pb[f >> 4], o[f & 15]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            return false;
        };
        uint8_t *const buf_a = FP8 ? f8_a : tile_a;
        uint8_t *const buf_b = FP8 ? f8_b : tile_b;
        if (n_tiles > 0) gather(0, buf_a);
        for (int j = 0; j < n_tiles; j += 2) {
            if (step(j, buf_a, buf_b)) break;
            if (j + 1 < n_tiles && step(j + 1, buf_b, buf_a)) break;
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        again = sm.restart != 0;
        if (again) {
            __syncthreads();                              // everyone has read the flag
            if (tid == 0) sm.restart = 0;
#pragma unroll
            for (int dt = 0; dt < 16; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
            l_run = 0.0f;
            m_ref = m_seen;
        }
    }

    // ---- finish: lanes l and l ^ 32 hold disjoint row subsets of each head
    const float l_tot = l_run + swap_halves(l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float m_fin = m_ref == -INFINITY ? 0.0f : m_ref;
    const float lse_v = l_tot > 0.0f ? (m_fin + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    if (!head_ok) return;
    if constexpr (!SPLIT) {
        uint16_t *orow = out + ((int64_t)t * h + head) * kDv + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                bf16x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[dt][4 * q4 + e] * inv);
                *reinterpret_cast<bf16x4 *>(orow + 32 * dt + 8 * q4) = v;
            }
        }
        if (lse != nullptr && g == 0) lse[(int64_t)t * h + head] = lse_v;
    } else {
        float *orow = ws_o + (((int64_t)t * n_splits + split) * h + head) * kDv + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *reinterpret_cast<float4 *>(orow + 32 * dt + 8 * q4) =
                    make_float4(o[dt][4 * q4] * inv, o[dt][4 * q4 + 1] * inv, o[dt][4 * q4 + 2] * inv,
                                o[dt][4 * q4 + 3] * inv);
        if (g == 0) ws_lse[((int64_t)t * n_splits + split) * h + head] = lse_v;
    }
}

// LSE-weighted merge of the decode splits: one wave per (query, head).
__global__ __launch_bounds__(256) void mla_combine_kernel(const float *__restrict__ ws_o,
                                                          const float *__restrict__ ws_lse, int32_t n_q,
                                                          int32_t h, int32_t n_splits, uint16_t *__restrict__ out,
                                                          float *__restrict__ lse) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (int64_t)n_q * h) return;
    const int64_t t = item / h, hd = item % h;
    float mx = -INFINITY;
    for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, ws_lse[(t * n_splits + s) * h + hd]);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float wsum = 0.0f;
    for (int s = 0; s < n_splits; ++s) {
        const float ls = ws_lse[(t * n_splits + s) * h + hd];
        if (ls == -INFINITY) continue;
        const float wgt = __expf(ls - mx);
        wsum += wgt;
        const float4 *src = reinterpret_cast<const float4 *>(ws_o + ((t * n_splits + s) * h + hd) * kDv + 8 * lane);
        const float4 a = src[0], b = src[1];
        acc[0] += wgt * a.x; acc[1] += wgt * a.y; acc[2] += wgt * a.z; acc[3] += wgt * a.w;
        acc[4] += wgt * b.x; acc[5] += wgt * b.y; acc[6] += wgt * b.z; acc[7] += wgt * b.w;
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)(acc[e] * inv);
    *reinterpret_cast<bf16x8 *>(out + (t * h + hd) * kDv + 8 * lane) = v;
    if (lse != nullptr && lane == 0) lse[t * h + hd] = wsum > 0.0f ? mx + __logf(wsum) : -INFINITY;
}

template <int NW, bool FP8, bool SPLIT>
static void launch_mla_t(const MlaArgs &a, int n_splits, float *ws_o, float *ws_lse, hipStream_t stream) {
    const unsigned grid = (unsigned)((int64_t)a.n_q * (SPLIT ? n_splits : 1));
    hipLaunchKernelGGL((sparse_mla_kernel<NW, FP8, SPLIT>), dim3(grid), dim3(NW * 64), 0, stream, a.q, a.kv_cache,
                       a.kv_scale, a.n_slots, a.kv_slot_table, a.kv_pt_ld, a.q_seq, a.idx, a.h, a.k, a.sm_scale,
                       a.out, a.lse, n_splits, ws_o, ws_lse);
}

template <bool FP8, bool SPLIT>
static void launch_mla_nw(const MlaArgs &a, int n_splits, float *ws_o, float *ws_lse, hipStream_t stream) {
    const int nw = (a.h + 31) / 32;   // 32 heads per wave
    switch (nw) {
    case 1: launch_mla_t<1, FP8, SPLIT>(a, n_splits, ws_o, ws_lse, stream); break;
    case 2: launch_mla_t<2, FP8, SPLIT>(a, n_splits, ws_o, ws_lse, stream); break;
    case 3: launch_mla_t<3, FP8, SPLIT>(a, n_splits, ws_o, ws_lse, stream); break;
    default: launch_mla_t<4, FP8, SPLIT>(a, n_splits, ws_o, ws_lse, stream); break;
    }
}

hipError_t launch_mla_prefill(const MlaArgs &a, hipStream_t stream) {
    if (a.fp8) launch_mla_nw<true, false>(a, 1, nullptr, nullptr, stream);
    else launch_mla_nw<false, false>(a, 1, nullptr, nullptr, stream);
    return hipGetLastError();
}

int mla_decode_auto_splits(int32_t n_q, int32_t k) {
    // One workgroup fills a CU (LDS-bound), so aim for about one workgroup per CU
    // (256): every extra split re-reads the query's 128 x 576 q block and writes
    // and re-reads a 128 x 512 fp32 partial, which at 64 queries costs more than
    // the parallelism it adds (measured: 8 splits 120 us, 4 splits 85 us).
    int s = 1;
    while (s < 32 && (int64_t)n_q * s < 256 && k / (2 * s) >= 2 * kTile) s *= 2;
    return s;
}

size_t mla_decode_ws_bytes(int32_t n_q, int32_t h, int32_t n_splits) {
    const size_t o = (size_t)n_q * n_splits * h * kDv * sizeof(float);
    const size_t l = (size_t)n_q * n_splits * h * sizeof(float);
    return o + ((l + 255) / 256) * 256 + 256;
}

hipError_t launch_mla_decode(const MlaArgs &a, int n_splits, void *ws, hipStream_t stream) {
    float *ws_o = reinterpret_cast<float *>(ws);
    float *ws_lse = ws_o + (size_t)a.n_q * n_splits * a.h * kDv;
    if (a.fp8) launch_mla_nw<true, true>(a, n_splits, ws_o, ws_lse, stream);
    else launch_mla_nw<false, true>(a, n_splits, ws_o, ws_lse, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = (int64_t)a.n_q * a.h;
    hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, stream, ws_o, ws_lse,
                       a.n_q, a.h, n_splits, a.out, a.lse);
    return hipGetLastError();
}

}  // namespace dsa

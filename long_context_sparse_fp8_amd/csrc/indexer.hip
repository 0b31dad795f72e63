// indexer.hip -- Lightning Indexer scores on FP8 MFMA (gfx950).
//
// score[t, s] = q_scale[t] * k_scale[s] * sum_j w[t, j] * ReLU(sum_i q[t, j, i] k[s, i])
// for s in [0, q_pos[t]] (DeepSeek-V3.2-Exp deployment article, section 1:
// an FP8 scorer over predecessor tokens; context-parallel article, section
// 1: relevance is a reduce-sum over the indexer heads).  Keys come from the
// page-64 key & key_scale cache (SGLang DeepSeek-V3.2 announcement).
//
// MFMA mapping (v_mfma_f32_32x32x64_f8f6f4): A = 32 indexer heads of one
// query, B = 32 keys, K = 64 bytes of the head dim.  Lane group g = l / 32
// owns head-dim bytes [g * D_I/2, (g+1) * D_I/2) in both operands (the same
// K permutation on both sides leaves the dot product unchanged).  The fp32
// accumulator gives lane l one key (l % 32) and 16 heads, so ReLU, weight
// and most of the head sum stay in the lane; one half-wave swap finishes the
// head sum and leaves key l of the 64-key page in lane l for a coalesced
// store.
#include <algorithm>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

typedef int v4i32 __attribute__((ext_vector_type(4)));   // for the non-temporal load builtin

template <int H_I, int D_I>
struct IdxShape {
    static constexpr int HT = (H_I + 31) / 32;   // 32-head MFMA row tiles
    static constexpr int KC = D_I / 64;          // 32-byte K chunks per lane
    static constexpr int HALF = D_I / 2;         // head-dim bytes owned by a lane group
    static constexpr int ROW = D_I + 16;         // padded LDS row (bytes): conflict-free 16-byte reads
    static constexpr int CH = D_I / 16;          // 16-byte chunks per key
};

// Register-resident operands of one query.
template <int H_I, int D_I>
struct QueryFrag {
    using S = IdxShape<H_I, D_I>;
    i32x8 a[S::HT][S::KC];
    float w[S::HT][16];
};

template <int H_I, int D_I>
__device__ __forceinline__ void load_query(QueryFrag<H_I, D_I> &q, const uint8_t *__restrict__ q_fp8,
                                           const float *__restrict__ w, int64_t w_ld, int t, int lane) {
    using S = IdxShape<H_I, D_I>;
    const int g = lane >> 5;
#pragma unroll
    for (int ht = 0; ht < S::HT; ++ht) {
        const int head = 32 * ht + (lane & 31);
#pragma unroll
        for (int c = 0; c < S::KC; ++c) {
            i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
            if (head < H_I) {
                const uint4 *src = reinterpret_cast<const uint4 *>(q_fp8 + ((int64_t)t * H_I + head) * D_I +
                                                                   g * S::HALF + 32 * c);
                const uint4 lo = src[0], hi = src[1];
                v = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
            q.a[ht][c] = v;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int hh = 32 * ht + 8 * (i >> 2) + 4 * g + (i & 3);
            q.w[ht][i] = hh < H_I ? w[(int64_t)t * w_ld + hh] : 0.0f;
        }
    }
}

// max(x, 0) on the bit pattern: one integer max, where the float max of an
// MFMA result first has to quiet a possible signalling NaN.  Equal to the
// float max for every number.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// One query against one 64-key page whose B fragments are in `b`.
// Returns the (unscaled) score of key `lane` of the page.
template <int H_I, int D_I>
__device__ __forceinline__ float page_scores(const QueryFrag<H_I, D_I> &q,
                                             const i32x8 (&b)[2][IdxShape<H_I, D_I>::KC]) {
    using S = IdxShape<H_I, D_I>;
    float part[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        f32x16 acc[S::HT];
#pragma unroll
        for (int ht = 0; ht < S::HT; ++ht) {
            acc[ht] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < S::KC; ++c) acc[ht] = mfma_f8_32x32x64(q.a[ht][c], b[kt][c], acc[ht]);
        }
        float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
        for (int ht = 0; ht < S::HT; ++ht) {
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                s0 = fmaf(q.w[ht][i + 0], relu_bits(acc[ht][i + 0]), s0);
                s1 = fmaf(q.w[ht][i + 1], relu_bits(acc[ht][i + 1]), s1);
                s2 = fmaf(q.w[ht][i + 2], relu_bits(acc[ht][i + 2]), s2);
                s3 = fmaf(q.w[ht][i + 3], relu_bits(acc[ht][i + 3]), s3);
            }
        }
        part[kt] = (s0 + s1) + (s2 + s3);
    }
    // lane i < 32: key i (tile 0); lane 32 + i: key 32 + i (tile 1)
    return halves_reduce_scatter(part[0], part[1]);
}

// ------------------------------------------------------------------ prefill
// Workgroup = 4 waves = 4 * QPW consecutive queries.  Queries of the same
// sequence share every key page, staged once in LDS (double-buffered).
template <int H_I, int D_I, int QPW>
__global__ __launch_bounds__(256, 2) void indexer_prefill_kernel(
    const uint8_t *__restrict__ q_fp8, const float *__restrict__ q_scale, const float *__restrict__ w, int64_t w_ld,
    const uint8_t *__restrict__ key_cache, const float *__restrict__ key_scale, int64_t n_pages,
    const int32_t *__restrict__ page_table, int64_t pt_ld, const int32_t *__restrict__ q_seq,
    const int32_t *__restrict__ q_pos, int32_t n_q, float *__restrict__ scores, int64_t ld) {
    using S = IdxShape<H_I, D_I>;
    constexpr int QB = 4 * QPW;
    constexpr int kChunks = kPage * S::CH;             // 16-byte chunks per page
    constexpr int kPer = (kChunks + 255) / 256;        // per thread
    __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][kPage * D_I];   // pages as stored (fragment-major)
    __shared__ float sbuf[2][kPage];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nqb = (n_q + QB - 1) / QB;
    const int t0 = (nqb - 1 - (int)blockIdx.x) * QB;   // latest (longest) query blocks first

    QueryFrag<H_I, D_I> q[QPW];
    float qs[QPW];
    int qp[QPW];
#pragma unroll
    for (int qq = 0; qq < QPW; ++qq) {
        const int t = t0 + wave * QPW + qq;
        const int tc = t < n_q ? t : n_q - 1;
        load_query<H_I, D_I>(q[qq], q_fp8, w, w_ld, tc, lane);
        qs[qq] = q_scale[tc];
        qp[qq] = q_pos[tc];
    }
    const int64_t max_page = (ld + kPage - 1) / kPage;

    uint32_t done = 0;
#pragma unroll
    for (int r = 0; r < QB; ++r)
        if (t0 + r >= n_q) done |= 1u << r;

    while (done != (1u << QB) - 1) {
        // next sequence group among the not-yet-processed rows (uniform over the workgroup)
        const int first = __builtin_ctz(~done);
        const int seq = q_seq[t0 + first];
        uint32_t active = 0;
        int pmax = -1;
#pragma unroll
        for (int r = 0; r < QB; ++r) {
            if (!((done >> r) & 1u) && q_seq[t0 + r] == seq) {
                active |= 1u << r;
                pmax = max(pmax, q_pos[t0 + r]);
            }
        }
        done |= active;
        int64_t n_pg = pmax < 0 ? 0 : (int64_t)pmax / kPage + 1;
        if (n_pg > max_page) n_pg = max_page;
        const int32_t *pt_row = page_table + (int64_t)seq * pt_ld;

        uint4 stage[kPer];
        float sstage = 0.0f;
        auto fetch = [&](int64_t p) {
            const int64_t phys = p < pt_ld ? (int64_t)pt_row[p] : -1;
            const bool ok = phys >= 0 && phys < n_pages;
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int ch = threadIdx.x + 256 * j;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (ok && ch < kChunks)
                    v = reinterpret_cast<const uint4 *>(key_cache + phys * (kPage * D_I))[ch];
                stage[j] = v;
            }
            if (threadIdx.x < kPage) sstage = ok ? key_scale[phys * kPage + threadIdx.x] : __builtin_nanf("");
        };
        auto commit = [&](int buf) {
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int ch = threadIdx.x + 256 * j;
                if (ch < kChunks) *reinterpret_cast<uint4 *>(&kbuf[buf][16 * ch]) = stage[j];
            }
            if (threadIdx.x < kPage) sbuf[buf][threadIdx.x] = sstage;
        };

        if (n_pg > 0) {
            fetch(0);
            commit(0);
        }
        __syncthreads();
        for (int64_t p = 0; p < n_pg; ++p) {
            const int buf = (int)(p & 1);
            if (p + 1 < n_pg) fetch(p + 1);
            i32x8 b[2][S::KC];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int c = 0; c < S::KC; ++c) {
                    const uint8_t *blk = &kbuf[buf][(kt * S::KC + c) * 2048 + 16 * lane];
                    const uint4 lo = *reinterpret_cast<const uint4 *>(blk);
                    const uint4 hi = *reinterpret_cast<const uint4 *>(blk + 1024);
                    b[kt][c] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                }
            }
            const float ksc = sbuf[buf][lane];
            const int64_t key = p * kPage + lane;
            // Every query of the wave is scored, active or not (an inactive one's
            // scores are not stored): with no branch between them the compiler
            // can put one query's MFMAs under the other's epilogue.
            float sc[QPW];
#pragma unroll
            for (int qq = 0; qq < QPW; ++qq) sc[qq] = page_scores<H_I, D_I>(q[qq], b);
            // the next page goes to LDS before the score stores: loads and stores
            // share one counter, so a store issued first would be waited for too
            if (p + 1 < n_pg) commit(buf ^ 1);
#pragma unroll
            for (int qq = 0; qq < QPW; ++qq) {
                const int r = wave * QPW + qq;
                if (((active >> r) & 1u) && key <= qp[qq] && key < ld)
                    scores[(int64_t)(t0 + r) * ld + key] = sc[qq] * (qs[qq] * ksc);
            }
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------------ decode
constexpr int kWavePages = 16;                    // page slots per wave (4 waves: 64 pages per split)
constexpr int kDecDepth = 1;                      // pages per wave in flight while one is scored

// Workgroup = query t x a range of at most 64 key pages; the 4 waves take
// pages round-robin and load B fragments straight from the cache.  Queries
// 2i and 2i + 1 of one sequence (several query tokens per sequence, as
// multi-token prediction presents them) are scored together: each page is
// loaded once for both, the pair's two workgroups taking half the range each.  The queries' A fragments and head weights are staged in LDS
// (shared by the 4 waves) and read from there for every page; every wave keeps
// kDecDepth page(s) in flight while it scores one, and the split's page-table
// entries are read once up front (lane i holds page p_begin + i, broadcast
// with a lane read), so no key load waits on a table load.  A wave's scores
// stay in registers and are stored after its last page: stores and loads share
// one completion counter, so a store between the page loads would make every
// later wait also wait for it (measured: 20% of the scan).
//
// HIST (the fused indexer -> top-k call): every workgroup also counts the keys
// of the scores it writes in an LDS histogram of the top-k's first digit (key
// bits 31..21, two lane-interleaved copies) and adds its non-zero bins to the
// row's histogram in `hist` with integer atomics (order-independent), so the
// top-k starts from the finished histogram instead of a sweep over the row.
template <int H_I, int D_I, bool HIST>
__global__ __launch_bounds__(256, 2) void indexer_decode_kernel(
    const uint8_t *__restrict__ q_fp8, const float *__restrict__ q_scale, const float *__restrict__ w, int64_t w_ld,
    const uint8_t *__restrict__ key_cache, const float *__restrict__ key_scale, int64_t n_pages,
    const int32_t *__restrict__ page_table, int64_t pt_ld, const int32_t *__restrict__ q_seq,
    const int32_t *__restrict__ q_pos, int32_t n_q, float *__restrict__ scores, int64_t ld, int pages_per_split,
    uint32_t *__restrict__ hist) {
    using S = IdxShape<H_I, D_I>;
    constexpr int NH = 32 * S::HT;                   // heads rounded up to MFMA row tiles
    __shared__ __attribute__((aligned(16))) uint8_t q_lds[2][NH * S::ROW];   // padded rows: conflict-free reads
    __shared__ __attribute__((aligned(16))) float w_lds[2][NH];
    __shared__ __attribute__((aligned(16))) uint32_t h_lds[HIST ? 2 : 1][HIST ? 2 * kTopkHistBins : 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5;
    const int t = blockIdx.x;
    const int64_t max_page = (ld + kPage - 1) / kPage;

    // Score queries t1 .. t1 + NQ - 1 (one sequence) against pages p_begin ..
    // p_begin + 4 SLOTS - 1 (at most 64: one page-table entry per lane).
    auto run = [&](auto nq_c, auto slots_c, const int t1, const int64_t p_begin) {
        constexpr int NQ = decltype(nq_c)::value, SLOTS = decltype(slots_c)::value;
        static_assert(4 * SLOTS <= 64, "one page-table entry per lane");
        int pos[NQ], pmax = -1;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            pos[j] = q_pos[t1 + j];
            pmax = max(pmax, pos[j]);
        }
        int64_t n_pg = pmax < 0 ? 0 : (int64_t)pmax / kPage + 1;
        if (n_pg > max_page) n_pg = max_page;
        const int64_t p_end = min(n_pg, p_begin + 4 * SLOTS);
        if (p_begin >= p_end) return;                // uniform over the workgroup
        if (n_pages <= 0) {                          // no page can be read: every score is NaN
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const int64_t k0 = p_begin * kPage, k1 = min(p_end * kPage, min((int64_t)pos[j] + 1, ld));
                for (int64_t key = k0 + threadIdx.x; key < k1; key += 256)
                    scores[(int64_t)(t1 + j) * ld + key] = __builtin_nanf("");
                if (HIST && threadIdx.x == 0 && k1 > k0)
                    atomicAdd(&hist[(int64_t)(t1 + j) * kFusedRowStride + (f32_order_key(__builtin_nanf("")) >> 21)],
                              (uint32_t)(k1 - k0));
            }
            return;
        }
        // physical page of page p_begin + lane, -1 when absent or out of range
        int32_t my_phys = -1;
        {
            const int32_t *pt_row = page_table + (int64_t)q_seq[t1] * pt_ld;
            const int64_t pp = p_begin + lane;
            if (pp < p_end && pp < pt_ld) {
                const int32_t v = pt_row[pp];
                if (v >= 0 && v < n_pages) my_phys = v;
            }
        }
        // the queries' FP8 rows (heads past H_I zero) and weights
        __syncthreads();                             // a previous run's readers are done
        if constexpr (HIST) {
            for (int b = threadIdx.x; b < NQ * 2 * kTopkHistBins; b += 256) h_lds[b / (2 * kTopkHistBins)][b % (2 * kTopkHistBins)] = 0u;
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            for (int c = threadIdx.x; c < NH * S::CH; c += 256) {
                const int head = c / S::CH, col = c % S::CH;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (head < H_I) v = reinterpret_cast<const uint4 *>(q_fp8 + ((int64_t)(t1 + j) * H_I + head) * D_I)[col];
                *reinterpret_cast<uint4 *>(&q_lds[j][head * S::ROW + col * 16]) = v;
            }
            for (int hh = threadIdx.x; hh < NH; hh += 256) w_lds[j][hh] = hh < H_I ? w[(int64_t)(t1 + j) * w_ld + hh] : 0.0f;
        }
        float qs[NQ];
#pragma unroll
        for (int j = 0; j < NQ; ++j) qs[j] = q_scale[t1 + j];
        __syncthreads();

        // Score of key `lane` of a page whose B fragments are in `b` for query j
        // (same mapping as the prefill scorer, with A fragments and weights
        // read from LDS for every page).
        auto scores_of = [&](const i32x8 (&b)[2][S::KC], const int j) -> float {
            asm volatile("" ::: "memory");           // q and w come from LDS, not kept in registers
            float part[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                f32x16 acc[S::HT];
#pragma unroll
                for (int ht = 0; ht < S::HT; ++ht) {
                    acc[ht] = f32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
                    const uint8_t *qrow = &q_lds[j][(32 * ht + (lane & 31)) * S::ROW + g * S::HALF];
#pragma unroll
                    for (int c = 0; c < S::KC; ++c) {
                        const uint4 lo = *reinterpret_cast<const uint4 *>(qrow + 32 * c);
                        const uint4 hi = *reinterpret_cast<const uint4 *>(qrow + 32 * c + 16);
                        const i32x8 a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                        acc[ht] = mfma_f8_32x32x64(a, b[kt][c], acc[ht]);
                    }
                }
                float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
                for (int ht = 0; ht < S::HT; ++ht) {
#pragma unroll
                    for (int i = 0; i < 16; i += 4) {
                        // accumulator element i: head 32 ht + 8 (i / 4) + 4 g + i % 4
                        const float4 wv = *reinterpret_cast<const float4 *>(&w_lds[j][32 * ht + 2 * i + 4 * g]);
                        s0 = fmaf(wv.x, relu_bits(acc[ht][i + 0]), s0);
                        s1 = fmaf(wv.y, relu_bits(acc[ht][i + 1]), s1);
                        s2 = fmaf(wv.z, relu_bits(acc[ht][i + 2]), s2);
                        s3 = fmaf(wv.w, relu_bits(acc[ht][i + 3]), s3);
                    }
                }
                part[kt] = (s0 + s1) + (s2 + s3);
            }
            // lane i < 32: key i (tile 0); lane 32 + i: key 32 + i (tile 1)
            return halves_reduce_scatter(part[0], part[1]);
        };

        // Page slot m of this wave is page p_begin + wave + 4 m.  Every wave runs all
        // SLOTS slots, fully unrolled and branch-free: a slot past the split
        // loads a page of the split again and stores nothing.  With no loop back-edge
        // the compiler can wait for exactly the page being scored while the next ones
        // stay in flight.
        auto fetch = [&](int m, i32x8 (&b)[2][S::KC], float &ksc) {
            const int64_t p = min(p_begin + wave + 4 * m, p_end - 1);
            const int32_t phys0 = __builtin_amdgcn_readlane(my_phys, (int)(p - p_begin));
            const int32_t phys = phys0 < 0 ? 0 : phys0;      // absent page: scores become NaN below
            const uint8_t *base = key_cache + (int64_t)phys * (kPage * D_I);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int c = 0; c < S::KC; ++c) {
                    // blocks h = 0, 1: one contiguous 1 KB load each, marked non-temporal:
                    // every key is read once per step, so the scan should not evict what
                    // the caches hold (measured: 159 -> 146 us for 64 x U[32K, 128K])
                    const v4i32 *src = reinterpret_cast<const v4i32 *>(base + (kt * S::KC + c) * 2048 + 16 * lane);
                    const v4i32 lo = __builtin_nontemporal_load(src), hi = __builtin_nontemporal_load(src + 64);
                    b[kt][c] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                }
            }
            const float k = key_scale[(int64_t)phys * kPage + lane];
            ksc = phys0 < 0 ? __builtin_nanf("") : k;
        };
        float sreg[NQ][SLOTS];
        constexpr int D = kDecDepth + 1;             // ring slots: in flight + the one scored
        i32x8 bf[D][2][S::KC];
        float kf[D];
#pragma unroll
        for (int m = 0; m < kDecDepth; ++m) fetch(m, bf[m], kf[m]);
#pragma unroll
        for (int m = 0; m < SLOTS; ++m) {
            if (m + kDecDepth < SLOTS) fetch(m + kDecDepth, bf[(m + kDecDepth) % D], kf[(m + kDecDepth) % D]);
#pragma unroll
            for (int j = 0; j < NQ; ++j) sreg[j][m] = scores_of(bf[m % D], j) * (qs[j] * kf[m % D]);
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int64_t k_end = min(p_end * kPage, min((int64_t)pos[j] + 1, ld));
            float *srow = scores + (int64_t)(t1 + j) * ld;
#pragma unroll
            for (int m = 0; m < SLOTS; ++m) {
                const int64_t key = (p_begin + wave + 4 * m) * kPage + lane;
                if (key < k_end) {
                    srow[key] = sreg[j][m];
                    if constexpr (HIST) atomicAdd(&h_lds[j][(f32_order_key(sreg[j][m]) >> 21) * 2 + (lane & 1)], 1u);
                }
            }
        }
        if constexpr (HIST) {
            __syncthreads();
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                for (int b = threadIdx.x; b < kTopkHistBins; b += 256) {
                    const uint32_t c = h_lds[j][2 * b] + h_lds[j][2 * b + 1];
                    if (c != 0u) atomicAdd(&hist[(int64_t)(t1 + j) * kFusedRowStride + b], c);
                }
            }
        }
    };

    // Queries 2i, 2i + 1 of one sequence: the two workgroups of a split score
    // both queries, each over half of the split's pages.  The decision is
    // uniform over the workgroup.
    const int64_t p_split = (int64_t)blockIdx.y * pages_per_split;   // pages_per_split = 4 kWavePages
    const int partner = t ^ 1;
    if (partner < n_q && q_seq[partner] == q_seq[t])
        run(std::integral_constant<int, 2>{}, std::integral_constant<int, kWavePages / 2>{}, t & ~1,
            p_split + (t & 1) * (2 * kWavePages));
    else
        run(std::integral_constant<int, 1>{}, std::integral_constant<int, kWavePages>{}, t, p_split);
}

// ------------------------------------------------------------------ launch
template <int H_I, int D_I>
static hipError_t launch_indexer_t(const IndexerArgs &a, hipStream_t stream) {
    if (a.n_q <= kIndexerDecodeMaxQ) {
        // few queries: split each query's key range over workgroups
        // Splits cover every logical page a score row can reach: those of the page
        // table and those past it (up to the row length), which get NaN scores.
        const int pps = 4 * kWavePages;            // 64: one page-table entry per lane
        const int64_t row_pages = (a.scores_ld + kPage - 1) / kPage;
        const int64_t splits = (std::max(a.pt_ld, row_pages) + pps - 1) / pps;
        dim3 grid((unsigned)a.n_q, (unsigned)(splits > 0 ? splits : 1));
        if (a.hist != nullptr)
            hipLaunchKernelGGL((indexer_decode_kernel<H_I, D_I, true>), grid, dim3(256), 0, stream, a.q_fp8,
                               a.q_scale, a.w, a.w_ld, a.key_cache, a.key_scale, a.n_pages, a.page_table, a.pt_ld,
                               a.q_seq, a.q_pos, a.n_q, a.scores, a.scores_ld, pps, a.hist);
        else
            hipLaunchKernelGGL((indexer_decode_kernel<H_I, D_I, false>), grid, dim3(256), 0, stream, a.q_fp8,
                               a.q_scale, a.w, a.w_ld, a.key_cache, a.key_scale, a.n_pages, a.page_table, a.pt_ld,
                               a.q_seq, a.q_pos, a.n_q, a.scores, a.scores_ld, pps, nullptr);
    } else {
        constexpr int QPW = 2;
        const int nqb = (a.n_q + 4 * QPW - 1) / (4 * QPW);
        hipLaunchKernelGGL((indexer_prefill_kernel<H_I, D_I, QPW>), dim3((unsigned)nqb), dim3(256), 0, stream,
                           a.q_fp8, a.q_scale, a.w, a.w_ld, a.key_cache, a.key_scale, a.n_pages, a.page_table, a.pt_ld,
                           a.q_seq, a.q_pos, a.n_q, a.scores, a.scores_ld);
    }
    return hipGetLastError();
}

hipError_t launch_indexer(const IndexerArgs &a, hipStream_t stream) {
    if (a.h_i == 64 && a.d_i == 128) return launch_indexer_t<64, 128>(a, stream);
    if (a.h_i == 16 && a.d_i == 64) return launch_indexer_t<16, 64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace dsa

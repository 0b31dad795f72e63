// topk.hip -- per-row top-k selection by radix select (gfx950).
//
// Keeps the k best of scores[t, 0..q_pos[t]] under (score descending, index
// ascending) -- the "top-k token selection" of the SGLang DeepSeek-V3.2
// announcement -- and writes them in ascending index order, -1 padded.  A
// row with no more than k candidates keeps all of them (the dense
// degeneration of the deployment article, section 5.1).
//
// One workgroup per row: 512 threads when many rows of at most 32K scores are
// selected at once (three workgroups share a CU, so one row's barriers and
// loads overlap the others' work), else 1024.  Every score is touched by only two
// cheap sweeps:
//   1. an 11-bit histogram of the top key bits (sign, exponent, two mantissa
//      bits) in LDS, NT / 128 lane-interleaved copies; a block scan of the 2048
//      bins from the top finds the bin holding the k-th largest key;
//   2. every key above that bin sets its bit in an LDS bitmap of the kept
//      indices, and the bin's own keys (a few percent of the row) go to
//      per-wave LDS candidate lists (ballot and lane count, no atomics).  The
//      radix select finishes on the lists alone (8-, 8- and 5-bit digits; it
//      stops early once a bin is taken whole).  Ties at the threshold key T are
//      resolved by a second radix select over the candidates' indices: the
//      `need` lowest indices equal to T are kept, i.e. every index up to a cut.
//      The kept candidates (key > T, or key == T at an index up to the cut)
//      join the bitmap, and a block scan of the bitmap words' popcounts writes
//      the kept indices in ascending order.  If a wave's list overflows (a row
//      of mostly equal scores) the same passes run over the whole row instead.
// Scores become order-preserving uint32 keys.  The row is cut into chunks of
// 4 NT scores (NT threads); in chunk c thread i owns the four consecutive
// scores starting at c * 4 NT + 4 i, so every wave-wide load is one contiguous
// 1 KB run.  Rows of at most 4 NT C scores are read once and kept in registers
// (every row of a 32K prefill); longer rows are streamed for each sweep,
// kStreamAhead chunks in flight per thread.
// Everything is integer, so the selection is exact for the given scores.
//
// Few long rows (decode: one row of up to 128K scores per sequence) would leave
// most of the chip idle with one workgroup per row.  With a workspace, such a
// row is cut into P parts of at least 2k scores: each part keeps its own k best
// (PART launch, one workgroup per part), and a second selection over the P x k
// survivors, laid out in index order, picks the final k (MERGE launch).  Every
// element of the row's top-k is in its part's top-k under the same ranking, and
// ties between survivors still fall to the lower original index, so the result
// is the same as the one-workgroup selection.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kBins0 = 2048;                    // first digit: key bits 31..21
constexpr int kBins = 512;                      // later digits (<= 9 bits)
constexpr int kCopies = 4;                      // lane-interleaved copies of the later histograms
constexpr int kStreamAhead = 8;                 // chunks in flight per thread when a row is streamed

// Workgroup shape: NT threads (1024, or 512 for rows of at most 32K scores,
// three workgroups per CU), chunks of 4 NT scores; C > 0 chunks per row in
// registers, C == 0 streamed.
template <int NT, int C>
struct TopkShape {
    static constexpr int kWaves = NT / kWave;
    static constexpr int kChunk = 4 * NT;                            // scores per chunk
    static constexpr int kCopies0 = NT / 128;                        // copies of the first histogram
    static constexpr int kCandCap = 8 * NT;                          // candidate list capacity
    static constexpr int64_t kMaxRow = C > 0 ? (int64_t)C * 4 * NT : kTopkMaxRow;
    static constexpr int kWords = (int)(kMaxRow / 32);               // bitmap words
    static constexpr int kBinsPer = kBins0 / NT;                     // first-digit bins per thread in the scan
    static_assert(kCopies0 % 4 == 0, "the scan reads the first histogram's copies four at a time");
    static_assert(kBins0 % NT == 0, "whole first-digit bins per thread");
};

template <int NT, int C>
struct TopkSmem {
    using S = TopkShape<NT, C>;
    static constexpr int kThreads = NT;
    union {
        uint32_t hist0[kBins0 * S::kCopies0];   // hist0[bin * kCopies0 + lane % kCopies0]
        struct {
            uint32_t key[S::kCandCap];
            int32_t idx[S::kCandCap];
        } cand;
    };
    uint32_t hist[kBins * kCopies];             // hist[bin * 4 + lane % 4]
    uint32_t bitmap[S::kWords];
    int32_t stage[kTopkMaxK];
    uint32_t wsum[S::kWaves];
    uint32_t wcnt[S::kWaves];                   // per-wave candidate list lengths
    uint32_t sel_bin, sel_rem, sel_done;
};

// Block-wide exclusive scan (all NT threads call it); returns the sum over
// lower threads, `total` gets the block sum.
template <class SM>
__device__ __forceinline__ uint32_t block_excl_scan(SM &sm, uint32_t a, uint32_t &total) {
    constexpr int NT = SM::kThreads;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t ia = a;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_up(ia, o);
        if (lane >= o) ia += u;
    }
    if (lane == 63) sm.wsum[wave] = ia;
    __syncthreads();
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        const uint32_t x = sm.wsum[w];
        pre += w < wave ? x : 0u;
        tot += x;
    }
    total = tot;
    __syncthreads();   // wsum may be reused by the next scan
    return pre + ia - a;
}

// Keys of one chunk for the calling thread: scores 4 NT c + 4 tid + e, e = 0..3.
// Branch-free: the load address is clamped into the row and keys past n are
// zeroed afterwards, so every load of a row is issued before the first wait.
template <int NT, bool VEC>
__device__ __forceinline__ void load_chunk(const float *row, int n, int c, uint32_t (&key)[4]) {
    const int i = c * 4 * NT + 4 * (int)threadIdx.x;
    float x[4];
    if constexpr (VEC) {   // row 16-byte aligned; ceil4(n) <= ld
        const float4 v = *reinterpret_cast<const float4 *>(row + min(i, ((n + 3) & ~3) - 4));
        x[0] = v.x;
        x[1] = v.y;
        x[2] = v.z;
        x[3] = v.w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = row[min(i + e, n - 1)];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) key[e] = f32_order_key(x[e]) & (0u - (uint32_t)(i + e < n));
}

// Radix-select digit: counts are in sm.hist[bin * 4 + copy] for bins [0, nb).
// Scans from the top (desc = true) or from the bottom and picks the bin that
// holds the rem-th element.  Wave 0 only; the caller synchronises.  Kept out of
// line: inlined, its reads get scheduled into the callers' loops and pin
// registers for the whole kernel.
template <class SM>
__device__ __noinline__ void pick_digit(SM &sm, int nb, uint32_t rem, bool desc) {
    const int lane = threadIdx.x & 63;
    uint32_t c[8];   // lane owns 8 consecutive bins in scan order (nb <= 512)
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = 8 * lane + j;                  // rank in scan order
        const int b = desc ? nb - 1 - r : r;
        uint32_t s = 0;
        if (r < nb) {
            const uint4 v = *reinterpret_cast<const uint4 *>(&sm.hist[b * kCopies]);
            s = (v.x + v.y) + (v.z + v.w);
        }
        c[j] = s;
        tot += s;
    }
    uint32_t incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_up(incl, o);
        if (lane >= o) incl += u;
    }
    uint32_t excl = incl - tot;
    if (excl < rem && incl >= rem) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (excl < rem && excl + c[j] >= rem) {
                const int r = 8 * lane + j;
                sm.sel_bin = (uint32_t)(desc ? nb - 1 - r : r);
                sm.sel_rem = rem - excl;
                sm.sel_done = (excl + c[j] == rem) ? 1u : 0u;   // the whole bin is taken
            }
            excl += c[j];
        }
    }
}

enum TopkMode { kWholeRow = 0, kPart = 1, kMerge = 2 };

// Parts of a row of n scores when splitting into at most `parts`.  Every part
// must hold more than k scores, so that it runs the selection and leaves its k
// survivors in the workspace (a part of at most k scores would take the
// keep-everything exit instead).  Parts are whole 4-score groups: with
// q = ceil(n / 4) groups over P parts, the shortest part holds at least
// 4 floor(q / P) - 3 scores (the last one may end short), which exceeds k
// once floor(q / P) >= ceil((k + 4) / 4).  For k >= 4 the first bound (at
// least 2k scores per part on average) already implies it; it matters for
// k < 4, e.g. k = 1 on a row of 8 scores.
__device__ __forceinline__ int topk_row_parts(int n, int k, int parts) {
    const int groups_per_part = (k + 7) / 4;   // ceil((k + 4) / 4)
    return max(1, min(min(parts, n / (2 * k)), ((n + 3) / 4) / groups_per_part));
}

// C > 0: rows of at most C chunks, keys held in registers.  C == 0: chunks are
// streamed from memory in every sweep.  MODE kWholeRow: row t of scores.
// kPart: part blockIdx.y of row t; a row of one part writes the final result,
// otherwise the part's k survivors (original index and score) go to the
// workspace at [t, part].  kMerge: the survivors of row t (rows of one part are
// done already).
// Waves per SIMD (launch bound): 6 for the register forms of 512 threads, i.e.
// three workgroups per CU, which their LDS (at most 53 KB) allows; the rows of
// up to 32K scores then keep 80 registers and park two chunks of keys in
// scratch, and still run 19% faster than two workgroups per CU (0.95 against
// 1.19 ms for the 32K prefill): the selection waits on barriers and loads.
template <int NT, int C, bool VEC, int MODE>
__global__ __launch_bounds__(NT, NT == 512 && C > 0 ? 6 : 1024 / NT) void topk_kernel(const float *__restrict__ scores, int64_t ld,
                                                             const int32_t *__restrict__ q_pos, int32_t k,
                                                             int32_t *__restrict__ idx, int32_t parts,
                                                             float *__restrict__ ws_score,
                                                             int32_t *__restrict__ ws_idx) {
    using S = TopkShape<NT, C>;
    constexpr int kChunk = S::kChunk, kCopies0 = S::kCopies0;
    __shared__ __attribute__((aligned(16))) TopkSmem<NT, C> sm;
    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int64_t n64 = (int64_t)q_pos[t] + 1;
    if (n64 > ld) n64 = ld;
    if (n64 < 0) n64 = 0;
    int n = (int)n64;   // n <= ld <= kTopkMaxRow (checked by the API)
    int32_t *out = idx + (int64_t)t * k;
    const float *row = scores + (int64_t)t * ld;
    int base = 0, n_parts = 1;
    if constexpr (MODE == kPart) {
        n_parts = topk_row_parts(n, k, parts);
        const int p = blockIdx.y;
        if (p >= n_parts) return;
        // parts of whole 4-score groups (aligned loads), the last one ending at n:
        // at most 4 ceil(ceil(n / 4) / n_parts) scores each
        const int64_t quads = (n + 3) / 4;
        const int b0 = (int)(4 * ((int64_t)p * quads / n_parts));
        const int b1 = p + 1 == n_parts ? n : (int)(4 * ((int64_t)(p + 1) * quads / n_parts));
        base = b0;
        row += b0;
        n = b1 - b0;
    } else if constexpr (MODE == kMerge) {
        n_parts = topk_row_parts(n, k, parts);
        if (n_parts == 1) return;
        row = ws_score + (int64_t)t * parts * k;
        n = n_parts * k;
    }

    if (n <= k) {   // every candidate is kept (a whole row, or a row of one part)
        for (int i = tid; i < k; i += NT) out[i] = i < n ? i : -1;
        return;
    }
    const int nc = (n + kChunk - 1) / kChunk;   // chunks of this row (uniform)

    uint32_t reg[C > 0 ? C : 1][4];
    if constexpr (C > 0) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (c < nc) {
                load_chunk<NT, VEC>(row, n, c, reg[c]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) reg[c][e] = 0u;
            }
        }
    }
    // fn(key, index) for every score of the row owned by this thread.  Slots past
    // n hold key 0; with CHECK they are skipped, without it they are passed on
    // (register form only), which keeps the per-slot range test out of the hot
    // sweeps: key 0 falls below every threshold unless the threshold bin is bin 0,
    // and the callers switch to CHECK exactly then.
    auto each_key = [&](auto check, auto fn) {
        constexpr bool CHECK = decltype(check)::value;
        if constexpr (C > 0) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if (c < nc) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = c * kChunk + 4 * tid + e;
                        if (!CHECK || i < n) fn(reg[c][e], i);
                    }
                }
            }
        } else {
            // kStreamAhead chunks per step, all loads issued before the first is used
            // (the chunk index is clamped, so the loads need no branch)
            for (int c0 = 0; c0 < nc; c0 += kStreamAhead) {
                uint32_t key[kStreamAhead][4];
#pragma unroll
                for (int u = 0; u < kStreamAhead; ++u) load_chunk<NT, VEC>(row, n, min(c0 + u, nc - 1), key[u]);
#pragma unroll
                for (int u = 0; u < kStreamAhead; ++u) {
                    if (c0 + u < nc) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int i = (c0 + u) * kChunk + 4 * tid + e;
                            if (i < n) fn(key[u][e], i);
                        }
                    }
                }
            }
        }
    };
    using Checked = std::integral_constant<bool, true>;
    using Unchecked = std::integral_constant<bool, false>;
    auto clear = [&](uint32_t *p, int words) {
        for (int i = tid; i < words / 4; i += NT) reinterpret_cast<uint4 *>(p)[i] = make_uint4(0, 0, 0, 0);
    };

    // ---- sweep 1: 11-bit histogram of the top key bits
    clear(sm.hist0, kBins0 * kCopies0);
    __syncthreads();
    {
        uint32_t *h = sm.hist0 + (lane & (kCopies0 - 1));
        each_key(Unchecked{}, [&](uint32_t key, int) { atomicAdd(&h[(key >> 21) * kCopies0], 1u); });
    }
    __syncthreads();
    uint32_t rem;
    uint32_t b0;
    {
        // thread tid owns bins 2047 - B tid - j, j = 0 .. B-1 (scan order: descending), B = 2048 / NT
        constexpr int B = S::kBinsPer;
        uint32_t cnt[B], mine = 0;
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const uint32_t *hb = sm.hist0 + (kBins0 - 1 - B * tid - j) * kCopies0;
            uint32_t c = 0;
#pragma unroll
            for (int q = 0; q < kCopies0; q += 4) {
                const uint4 v = *reinterpret_cast<const uint4 *>(hb + q);
                c += (v.x + v.y) + (v.z + v.w);
            }
            cnt[j] = c;
        }
        if (C > 0 && tid == NT - 1) cnt[B - 1] -= (uint32_t)(nc * kChunk - n);   // padding keys in bin 0
#pragma unroll
        for (int j = 0; j < B; ++j) mine += cnt[j];
        uint32_t total;
        uint32_t excl = block_excl_scan(sm, mine, total);
        const uint32_t kk = (uint32_t)k;
        if (excl < kk && excl + mine >= kk) {
#pragma unroll
            for (int j = 0; j < B; ++j) {
                if (excl < kk && excl + cnt[j] >= kk) {
                    sm.sel_bin = (uint32_t)(kBins0 - 1 - B * tid - j);
                    sm.sel_rem = kk - excl;
                    sm.sel_done = (excl + cnt[j] == kk) ? 1u : 0u;
                }
                excl += cnt[j];
            }
        }
        __syncthreads();
        b0 = sm.sel_bin;
        rem = sm.sel_rem;
    }
    bool done = sm.sel_done != 0;
    uint32_t prefix = b0 << 21, pmask = 0xFFE00000u;
    // padding keys (0) can only tie with a threshold in bin 0
    auto each_row = [&](auto fn) {
        if (b0 == 0) each_key(Checked{}, fn);
        else each_key(Unchecked{}, fn);
    };

    // ---- sweep 2: every key above the threshold bin (and the bin itself when it
    // is taken whole) sets its bit in the bitmap of kept indices; the bin's keys
    // go to per-wave LDS lists (ballot and lane count, no atomics).  A wave list
    // that overflows (a row of mostly equal scores) makes the select finish over
    // the whole row instead.
    const bool whole_bin = done;
    constexpr int R = S::kCandCap / S::kWaves;     // per-wave list capacity
    const int nwords = (n + 31) >> 5;
    clear(sm.bitmap, (nwords + 3) & ~3);
    __syncthreads();                               // (the first-digit reads of hist0, which the lists alias, are done)
    {
        uint32_t wfill = 0;                        // this wave's list length (uniform)
        each_row([&](uint32_t key, int i) {
            const uint32_t bin = key >> 21;
            if (bin > b0 || (whole_bin && bin == b0)) atomicOr(&sm.bitmap[i >> 5], 1u << (i & 31));
            if (!whole_bin) {
                const bool me = bin == b0;
                const uint64_t m = __ballot(me);
                if (m != 0ull) {
                    const uint32_t slot = wfill + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                    if (me && slot < (uint32_t)R) {
                        sm.cand.key[wave * R + slot] = key;
                        sm.cand.idx[wave * R + slot] = i;
                    }
                    wfill += (uint32_t)__popcll(m);
                }
            }
        });
        if (lane == 0) sm.wcnt[wave] = wfill;
    }
    __syncthreads();
    bool use_list = !whole_bin;
#pragma unroll
    for (int w = 0; w < S::kWaves; ++w) use_list = use_list && sm.wcnt[w] <= (uint32_t)R;
    const uint32_t my_cnt = sm.wcnt[wave];
    // fn(key, index) over the elements still in play: each wave's own candidate
    // list, or (a list overflowed) the whole row, re-read from memory so that the
    // register copy stays out of the pass loops
    auto each_live = [&](auto fn) {
        if (use_list) {
            for (int j = lane; j < (int)my_cnt; j += kWave) fn(sm.cand.key[wave * R + j], sm.cand.idx[wave * R + j]);
        } else {
            for (int c = 0; c < nc; ++c) {
                uint32_t key[4];
                load_chunk<NT, VEC>(row, n, c, key);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = c * kChunk + 4 * tid + e;
                    if (i < n) fn(key[e], i);
                }
            }
        }
    };
    uint32_t *hc = sm.hist + (lane & (kCopies - 1));

    // ---- finish the key select on the live set: digits 8, 8, 5 below the first 11 bits
    if (!done) {
#pragma unroll 1
        for (int pass = 0; pass < 3 && !done; ++pass) {
            const int shift = pass == 0 ? 13 : (pass == 1 ? 5 : 0);
            const int width = pass == 2 ? 5 : 8;
            const uint32_t dmask = (1u << width) - 1u;
            clear(sm.hist, kBins * kCopies);
            __syncthreads();
            each_live([&](uint32_t key, int) {
                if ((key & pmask) == prefix) atomicAdd(&hc[((key >> shift) & dmask) * kCopies], 1u);
            });
            __syncthreads();
            if (wave == 0) pick_digit(sm, 1 << width, rem, true);
            __syncthreads();
            prefix |= sm.sel_bin << shift;
            pmask |= dmask << shift;
            rem = sm.sel_rem;
            done = sm.sel_done != 0;
            __syncthreads();
        }
    }
    // keys with (key & pmask) > prefix are kept; of those equal to it, the `rem`
    // lowest indices: every index <= cut
    int cut = 0x7FFFFFFF;
    if (!done) {
        // radix select of the rem-th smallest index among keys equal to prefix
        // (indices < 2^18: digits 9 + 9)
        uint32_t ipre = 0, imask = 0;
#pragma unroll 1
        for (int pass = 0; pass < 2; ++pass) {
            const int shift = pass == 0 ? 9 : 0;
            clear(sm.hist, kBins * kCopies);
            __syncthreads();
            each_live([&](uint32_t key, int i) {
                if ((key & pmask) == prefix && ((uint32_t)i & imask) == ipre)
                    atomicAdd(&hc[(((uint32_t)i >> shift) & 511u) * kCopies], 1u);
            });
            __syncthreads();
            if (wave == 0) pick_digit(sm, kBins, rem, false);
            __syncthreads();
            ipre |= sm.sel_bin << shift;
            imask |= 511u << shift;
            rem = sm.sel_rem;
            __syncthreads();
        }
        cut = (int)ipre;
    }

    // ---- the threshold bin's kept keys (key > T, or key == T at an index up to
    // the cut) join the bitmap (a bin taken whole is there already); then the
    // ordered output
    if (!whole_bin) {
        each_live([&](uint32_t key, int i) {
            const uint32_t km = key & pmask;
            if ((key >> 21) == b0 && (km > prefix || (km == prefix && i <= cut)))
                atomicOr(&sm.bitmap[i >> 5], 1u << (i & 31));
        });
    }
    __syncthreads();
    {
        const int W = (nwords + NT - 1) / NT;   // words per thread, in order
        const int w0 = min(nwords, tid * W), w1 = min(nwords, w0 + W);
        uint32_t cnt = 0;
        for (int w = w0; w < w1; ++w) cnt += (uint32_t)__builtin_popcount(sm.bitmap[w]);
        uint32_t total;
        uint32_t pos = block_excl_scan(sm, cnt, total);
        for (int w = w0; w < w1; ++w) {
            uint32_t bits = sm.bitmap[w];
            while (bits) {
                const int b = __builtin_ctz(bits);
                bits &= bits - 1;
                if (pos < (uint32_t)k) sm.stage[pos] = 32 * w + b;   // exactly k are kept
                ++pos;
            }
        }
    }
    __syncthreads();
    if (MODE == kWholeRow || (MODE == kPart && n_parts == 1)) {
        for (int i = tid; i < k; i += NT) out[i] = sm.stage[i];
    } else if (MODE == kPart) {
        const int64_t o = ((int64_t)t * parts + blockIdx.y) * k;
        for (int i = tid; i < k; i += NT) {
            const int pos = sm.stage[i];
            ws_idx[o + i] = base + pos;
            ws_score[o + i] = row[pos];
        }
    } else {
        const int32_t *map = ws_idx + (int64_t)t * parts * k;
        for (int i = tid; i < k; i += NT) out[i] = map[sm.stage[i]];
    }
}

// ---------------------------------------------------------------- fused selection
// The fused indexer -> top-k call.  The split-key scorer has accumulated each
// row's first-digit histogram (key bits 31..21) in the workspace, so the
// threshold bin b0 of a row, how many keys it holds and how many of them are
// still needed are known before a score is read.  Two launches, each row read
// once:
//   PART (one workgroup per kFusedPart scores of a row; every part scans the
//   same histogram and finds the same b0): the part's scores are loaded into
//   registers; every key above b0 (at or above it when the bin is taken whole)
//   sets its bit in the part's slice of the row's bitmap of kept indices, and
//   the keys of bin b0 are appended to per-wave LDS lists (ballot and lane
//   count: no atomics in the sweep), then copied to the row's candidate list
//   in the workspace (one global atomic per wave reserves the range);
//   MERGE (one workgroup per row): reads the bitmap and the candidates,
//   finishes the radix select on the candidates (8-, 8- and 5-bit digits, then
//   the index cut among keys equal to the threshold), adds the kept ones to the
//   bitmap, writes the kept indices in ascending order and clears the row's
//   histogram and counters for the next call.
// When the threshold bin holds more keys than the list (a row of mostly equal
// scores) or a wave's list overflows, MERGE finishes the select over the whole
// row instead, re-reading it.  Everything is integer: the result is that of
// topk_kernel.  (A single launch, whose last part workgroup merges, needs a
// device-scope release fence per workgroup -- an L2 write-back -- that costs
// more than the second launch.)
constexpr int kFusedPartNT = 512;
constexpr int kFusedC = 8;                                        // chunks of 4 NT scores per part
constexpr int kFusedPart = kFusedC * 4 * kFusedPartNT;            // 16384 scores per part workgroup
constexpr int kFusedWaveCand = 256;                               // per-wave LDS list of a part
constexpr int kFusedMergeNT = 1024;
// row header in the zero region, after the histogram
constexpr int kHdrCand = kTopkHistBins, kHdrOverflow = kTopkHistBins + 1, kHdrB0 = kTopkHistBins + 2,
              kHdrRem = kTopkHistBins + 3, kHdrFlags = kTopkHistBins + 4;
static_assert(kFusedPart % 32 == 0, "parts cover whole bitmap words");
static_assert(kHdrFlags < kFusedRowWords, "header inside the zero region");

struct FusedPartSmem {
    static constexpr int kThreads = kFusedPartNT;
    uint32_t bitmap[kFusedPart / 32];
    struct {
        uint32_t key[kFusedWaveCand];
        int32_t idx[kFusedWaveCand];
    } list[kFusedPartNT / kWave];
    uint32_t wsum[kFusedPartNT / kWave];
    uint32_t sel_bin, sel_rem, sel_done, sel_cnt;
};

struct FusedMergeSmem {
    static constexpr int kThreads = kFusedMergeNT;
    uint32_t bitmap[kTopkMaxRow / 32];
    struct {
        uint32_t key[kFusedCand];
        int32_t idx[kFusedCand];
    } cand;
    uint32_t hist[kBins * kCopies];
    int32_t stage[kTopkMaxK];
    uint32_t wsum[kFusedMergeNT / kWave];
    uint32_t sel_bin, sel_rem, sel_done;
};

__device__ __forceinline__ int fused_row_len(const int32_t *q_pos, int t, int64_t ld) {
    int64_t n = (int64_t)q_pos[t] + 1;
    if (n > ld) n = ld;
    if (n < 0) n = 0;
    return (int)n;   // n <= ld <= kTopkMaxRow (checked by the API)
}

template <bool VEC>
__global__ __launch_bounds__(kFusedPartNT, 2) void topk_fused_part_kernel(const float *__restrict__ scores,
                                                                         int64_t ld,
                                                                         const int32_t *__restrict__ q_pos,
                                                                         int32_t k, uint32_t *__restrict__ ws) {
    constexpr int NT = kFusedPartNT, C = kFusedC, kChunk = 4 * NT, R = kFusedWaveCand;
    __shared__ __attribute__((aligned(16))) FusedPartSmem sm;
    const int t = blockIdx.x, part = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = fused_row_len(q_pos, t, ld);
    if (n <= k) return;                           // MERGE keeps every candidate
    const int base = part * kFusedPart;
    if (base >= n) return;
    const int n_here = min(kFusedPart, n - base), nc = (n_here + kChunk - 1) / kChunk;
    uint32_t *zr = ws + (int64_t)t * kFusedRowStride;
    uint32_t *rbits = zr + kFusedRowWords;
    uint32_t *rkey = rbits + kTopkMaxRow / 32;
    int32_t *ridx = reinterpret_cast<int32_t *>(rkey + kFusedCand);
    const float *row = scores + (int64_t)t * ld + base;

    // the histogram first, then the part's raw scores: the scan below waits for
    // the histogram only, while the scores are still on their way
    constexpr int B = kTopkHistBins / NT;         // bins per thread (4), descending from the top
    static_assert(B == 4, "one 16-byte histogram load per thread");
    const uint4 hv = reinterpret_cast<const uint4 *>(zr)[kTopkHistBins / 4 - 1 - tid];
    float x[C][4];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int i = min(c, nc - 1) * kChunk + 4 * tid;
        if constexpr (VEC) {   // the row is 16-byte aligned; ceil4(n) <= ld
            const float4 v = *reinterpret_cast<const float4 *>(row + min(i, ((n_here + 3) & ~3) - 4));
            x[c][0] = v.x;
            x[c][1] = v.y;
            x[c][2] = v.z;
            x[c][3] = v.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[c][e] = row[min(i + e, n_here - 1)];
        }
    }
    // ---- the threshold bin b0 (bins scanned from the top)
    if (tid == 0) {   // defaults for a histogram that does not hold the row (never for a zeroed workspace)
        sm.sel_bin = 0u;
        sm.sel_rem = (uint32_t)k;
        sm.sel_done = 0u;
        sm.sel_cnt = 0xFFFFFFFFu;
    }
    for (int w = tid; w < kFusedPart / 32; w += NT) sm.bitmap[w] = 0u;
    {
        const uint32_t cnt[B] = {hv.w, hv.z, hv.y, hv.x};   // bins 2047 - 4 tid - j
        const uint32_t mine = (cnt[0] + cnt[1]) + (cnt[2] + cnt[3]);
        uint32_t total;
        uint32_t excl = block_excl_scan(sm, mine, total);   // (its barriers also order the clears above)
        const uint32_t kk = (uint32_t)k;
        if (excl < kk && excl + mine >= kk) {
#pragma unroll
            for (int j = 0; j < B; ++j) {
                if (excl < kk && excl + cnt[j] >= kk) {
                    sm.sel_bin = (uint32_t)(kTopkHistBins - 1 - B * tid - j);
                    sm.sel_rem = kk - excl;
                    sm.sel_done = (excl + cnt[j] == kk) ? 1u : 0u;
                    sm.sel_cnt = cnt[j];
                }
                excl += cnt[j];
            }
        }
        __syncthreads();
    }
    const uint32_t b0 = sm.sel_bin;
    const bool whole_bin = sm.sel_done != 0u;
    const bool collect = !whole_bin && sm.sel_cnt <= (uint32_t)kFusedCand;
    if (part == 0 && tid == 0) {                  // for MERGE (every part finds the same)
        zr[kHdrB0] = b0;
        zr[kHdrRem] = sm.sel_rem;
        zr[kHdrFlags] = (whole_bin ? 1u : 0u) | (collect ? 2u : 0u);
    }

    // ---- sweep: bitmap slice of the keys above b0, per-wave lists of bin b0
    uint32_t wfill = 0;                           // this wave's list length (uniform)
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if (c < nc) {
            const int i0 = c * kChunk + 4 * tid;  // index within the part; its 4 keys share a bitmap word
            uint32_t above = 0, mine = 0, key[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                key[e] = f32_order_key(x[c][e]);
                const uint32_t bin = key[e] >> 21;
                const bool v = i0 + e < n_here;
                above |= (uint32_t)(v && (bin > b0 || (whole_bin && bin == b0))) << e;
                mine |= (uint32_t)(v && collect && bin == b0) << e;
            }
            if (above != 0u) atomicOr(&sm.bitmap[i0 >> 5], above << (i0 & 31));
            if (collect) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool me = ((mine >> e) & 1u) != 0u;
                    const uint64_t m = __ballot(me);
                    if (m != 0ull) {
                        const uint32_t slot =
                            wfill + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                        if (me && slot < (uint32_t)R) {
                            sm.list[wave].key[slot] = key[e];
                            sm.list[wave].idx[slot] = base + i0 + e;
                        }
                        wfill += (uint32_t)__popcll(m);
                    }
                }
            }
        }
    }
    // this wave's list to the row's candidates (a wave reads back only its own list)
    if (collect && wfill > 0u) {
        uint32_t g0 = 0u;
        if (lane == 0) g0 = wfill > (uint32_t)R ? 0u : atomicAdd(&zr[kHdrCand], wfill);
        g0 = (uint32_t)__shfl((int)g0, 0);
        if (wfill <= (uint32_t)R && g0 + wfill <= (uint32_t)kFusedCand) {
            for (uint32_t j = lane; j < wfill; j += kWave) {
                rkey[g0 + j] = sm.list[wave].key[j];
                ridx[g0 + j] = sm.list[wave].idx[j];
            }
        } else if (lane == 0) {
            atomicOr(&zr[kHdrOverflow], 1u);      // MERGE re-reads the row
        }
    }
    __syncthreads();
    {
        const int w0 = base >> 5, nw = (n_here + 31) >> 5;
        for (int w = tid; w < nw; w += NT) rbits[w0 + w] = sm.bitmap[w];
    }
}

template <bool VEC>
__global__ __launch_bounds__(kFusedMergeNT, 1) void topk_fused_merge_kernel(const float *__restrict__ scores,
                                                                           int64_t ld,
                                                                           const int32_t *__restrict__ q_pos,
                                                                           int32_t k, int32_t *__restrict__ idx,
                                                                           uint32_t *__restrict__ ws) {
    constexpr int NT = kFusedMergeNT, kChunk = 4 * NT;
    __shared__ __attribute__((aligned(16))) FusedMergeSmem sm;
    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = fused_row_len(q_pos, t, ld);
    uint32_t *zr = ws + (int64_t)t * kFusedRowStride;
    int32_t *out = idx + (int64_t)t * k;
    if (n <= k) {   // every candidate is kept
        for (int i = tid; i < k; i += NT) out[i] = i < n ? i : -1;
        for (int b = tid; b < kFusedRowWords; b += NT) zr[b] = 0u;
        return;
    }
    const uint32_t *rbits = zr + kFusedRowWords;
    const uint32_t *rkey = rbits + kTopkMaxRow / 32;
    const int32_t *ridx = reinterpret_cast<const int32_t *>(rkey + kFusedCand);
    const float *row = scores + (int64_t)t * ld;
    const uint32_t b0 = zr[kHdrB0], flags = zr[kHdrFlags];
    uint32_t rem = zr[kHdrRem];
    const bool whole_bin = (flags & 1u) != 0u;
    const bool use_list = (flags & 2u) != 0u && zr[kHdrOverflow] == 0u;
    const uint32_t n_list = use_list ? min(zr[kHdrCand], (uint32_t)kFusedCand) : 0u;
    const int nwords = (n + 31) >> 5;
    for (int w = tid; w < nwords; w += NT) sm.bitmap[w] = rbits[w];
    for (int j = tid; j < (int)n_list; j += NT) {
        sm.cand.key[j] = rkey[j];
        sm.cand.idx[j] = ridx[j];
    }
    __syncthreads();
    // fn(key, index) over the keys still in play: the row's candidates, or the whole row re-read
    auto each_live = [&](auto fn) {
        if (use_list) {
            for (int j = tid; j < (int)n_list; j += NT) fn(sm.cand.key[j], sm.cand.idx[j]);
        } else {
            const int ncr = (n + kChunk - 1) / kChunk;
            for (int c = 0; c < ncr; ++c) {
                uint32_t key[4];
                load_chunk<NT, VEC>(row, n, c, key);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = c * kChunk + 4 * tid + e;
                    if (i < n) fn(key[e], i);
                }
            }
        }
    };
    uint32_t *hc = sm.hist + (lane & (kCopies - 1));
    auto clear_hist = [&]() {
        for (int i = tid; i < kBins * kCopies / 4; i += NT)
            reinterpret_cast<uint4 *>(sm.hist)[i] = make_uint4(0, 0, 0, 0);
    };
    bool done = whole_bin;
    uint32_t prefix = b0 << 21, pmask = 0xFFE00000u;
    if (!done) {   // digits 8, 8, 5 below the first 11 bits
#pragma unroll 1
        for (int pass = 0; pass < 3 && !done; ++pass) {
            const int shift = pass == 0 ? 13 : (pass == 1 ? 5 : 0);
            const int width = pass == 2 ? 5 : 8;
            const uint32_t dmask = (1u << width) - 1u;
            clear_hist();
            __syncthreads();
            each_live([&](uint32_t key, int) {
                if ((key & pmask) == prefix) atomicAdd(&hc[((key >> shift) & dmask) * kCopies], 1u);
            });
            __syncthreads();
            if (wave == 0) pick_digit(sm, 1 << width, rem, true);
            __syncthreads();
            prefix |= sm.sel_bin << shift;
            pmask |= dmask << shift;
            rem = sm.sel_rem;
            done = sm.sel_done != 0u;
            __syncthreads();
        }
    }
    // keys with (key & pmask) > prefix are kept; of those equal to it, the `rem`
    // lowest indices: every index <= cut
    int cut = 0x7FFFFFFF;
    if (!done) {   // radix select of the rem-th smallest index among keys equal to prefix (digits 9 + 9)
        uint32_t ipre = 0, imask = 0;
#pragma unroll 1
        for (int pass = 0; pass < 2; ++pass) {
            const int shift = pass == 0 ? 9 : 0;
            clear_hist();
            __syncthreads();
            each_live([&](uint32_t key, int i) {
                if ((key & pmask) == prefix && ((uint32_t)i & imask) == ipre)
                    atomicAdd(&hc[(((uint32_t)i >> shift) & 511u) * kCopies], 1u);
            });
            __syncthreads();
            if (wave == 0) pick_digit(sm, kBins, rem, false);
            __syncthreads();
            ipre |= sm.sel_bin << shift;
            imask |= 511u << shift;
            rem = sm.sel_rem;
            __syncthreads();
        }
        cut = (int)ipre;
    }
    if (!whole_bin) {   // the kept keys of bin b0 join the bitmap
        each_live([&](uint32_t key, int i) {
            const uint32_t km = key & pmask;
            if ((key >> 21) == b0 && (km > prefix || (km == prefix && i <= cut)))
                atomicOr(&sm.bitmap[i >> 5], 1u << (i & 31));
        });
    }
    __syncthreads();
    {
        const int W = (nwords + NT - 1) / NT;     // words per thread, in order
        const int w0 = min(nwords, tid * W), w1 = min(nwords, w0 + W);
        uint32_t cnt = 0;
        for (int w = w0; w < w1; ++w) cnt += (uint32_t)__builtin_popcount(sm.bitmap[w]);
        uint32_t total;
        uint32_t pos = block_excl_scan(sm, cnt, total);
        for (int w = w0; w < w1; ++w) {
            uint32_t bits = sm.bitmap[w];
            while (bits) {
                const int b = __builtin_ctz(bits);
                bits &= bits - 1;
                if (pos < (uint32_t)k) sm.stage[pos] = 32 * w + b;   // exactly k are kept
                ++pos;
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < k; i += NT) out[i] = sm.stage[i];
    for (int b = tid; b < kFusedRowWords; b += NT) zr[b] = 0u;   // histogram and header, for the next call
}

int topk_parts(int32_t n_q, int64_t ld, int32_t k) {
    // split only when the rows alone cannot fill the chip: about one part per
    // CU of a 256-CU device (one round of workgroups measured faster than two
    // rounds of smaller parts), parts of at least 4k scores on average ...
    if (n_q > 128) return 1;
    int p = 8;
    while (p > 1 && ((int64_t)n_q * p > 256 || ld / p < 4 * (int64_t)k)) p >>= 1;
    // ... unless a part would then be too long to stay in registers (over 32K
    // scores): two rounds of register-resident parts beat one round that reads
    // its part from memory several times (128 rows of 128K: 65 -> 58 us)
    if (p < 8 && (ld + p - 1) / p > 8 * 4096 && (int64_t)n_q * 2 * p <= 512) p *= 2;
    return p;
}

size_t topk_ws_bytes(int32_t n_q, int64_t ld, int32_t k) {
    const int p = topk_parts(n_q, ld, k);
    return p > 1 ? (size_t)n_q * p * k * (sizeof(float) + sizeof(int32_t)) + 256 : 0;
}

// Whole rows of up to `len` scores, VEC when row starts are 16-byte aligned.
template <int MODE>
static void launch_rows(dim3 grid, int64_t len, bool vec, const float *scores, int64_t ld, const int32_t *q_pos,
                        int32_t k, int32_t *idx, int parts, float *ws_score, int32_t *ws_idx, hipStream_t stream) {
#define DSA_TOPK_GO(NT, C, V)                                                                                    \
    hipLaunchKernelGGL((topk_kernel<NT, C, V, MODE>), grid, dim3(NT), 0, stream, scores, ld, q_pos, k, idx, parts,    \
                       ws_score, ws_idx)
    if constexpr (MODE != kMerge) {
        // more rows (or parts) than a 256-CU device has CUs: workgroups of 512,
        // three per CU, while a row fits their registers (128 decode rows in 4
        // parts, then two per CU: 58 -> 51 us); with fewer, one workgroup of 1024
        // per row
        if (len <= 16 * 2048 && (int64_t)grid.x * grid.y > 256) {
            if (vec) {
                if (len <= 8 * 2048) DSA_TOPK_GO(512, 8, true);
                else DSA_TOPK_GO(512, 16, true);
            } else {
                if (len <= 8 * 2048) DSA_TOPK_GO(512, 8, false);
                else DSA_TOPK_GO(512, 16, false);
            }
            return;
        }
    }
    if (vec) {
        if (len <= 4 * 4096) DSA_TOPK_GO(1024, 4, true);
        else if (len <= 8 * 4096) DSA_TOPK_GO(1024, 8, true);
        else DSA_TOPK_GO(1024, 0, true);
    } else {
        if (len <= 8 * 4096) DSA_TOPK_GO(1024, 8, false);
        else DSA_TOPK_GO(1024, 0, false);
    }
#undef DSA_TOPK_GO
}

// ---------------------------------------------------------------- static workspace
// The split rows' survivors of dsa_topk_static live in this file-scope device
// array instead of a caller workspace, for callers that cannot allocate (HIP
// graph capture, serving loops).  Every split made above fits: at most 512
// parts (rows x parts) of k <= 2048 survivors of 8 bytes, plus the 256-byte
// alignment slack, 8 MiB + 256 bytes per device, held until the process ends.
// Every call on a device shares that device's copy; nothing in it must start
// at zero (each part writes all of its survivors before the merge reads them).
constexpr size_t kTopkStaticBytes = (size_t)512 * kTopkMaxK * (sizeof(float) + sizeof(int32_t)) + 256;
static __device__ __align__(256) uint8_t scratch[kTopkStaticBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t topk_static_workspace(void **ptr, size_t *bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        // this device's copy of the array (host code must not use its name as an address)
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = kTopkStaticBytes;
    return hipSuccess;
}

hipError_t launch_topk_fused(const float *scores, int64_t ld, const int32_t *q_pos, int32_t n_q, int32_t k,
                             int32_t *idx, uint32_t *ws, hipStream_t stream) {
    const int64_t parts = (ld + kFusedPart - 1) / kFusedPart;
    dim3 grid((unsigned)n_q, (unsigned)(parts > 0 ? parts : 1));
    // scores is 16-byte aligned (checked by the API), so rows are when ld % 4 == 0
    if ((ld & 3) == 0) {
        hipLaunchKernelGGL(topk_fused_part_kernel<true>, grid, dim3(kFusedPartNT), 0, stream, scores, ld, q_pos, k,
                           ws);
        hipLaunchKernelGGL(topk_fused_merge_kernel<true>, dim3((unsigned)n_q), dim3(kFusedMergeNT), 0, stream,
                           scores, ld, q_pos, k, idx, ws);
    } else {
        hipLaunchKernelGGL(topk_fused_part_kernel<false>, grid, dim3(kFusedPartNT), 0, stream, scores, ld, q_pos, k,
                           ws);
        hipLaunchKernelGGL(topk_fused_merge_kernel<false>, dim3((unsigned)n_q), dim3(kFusedMergeNT), 0, stream,
                           scores, ld, q_pos, k, idx, ws);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *q_pos, int32_t n_q, int32_t k, int32_t *idx,
                       void *ws, size_t ws_bytes, hipStream_t stream) {
    // scores is 16-byte aligned (checked by the API), so rows are when ld % 4 == 0
    const bool vec = (ld & 3) == 0;
    const int parts = topk_parts(n_q, ld, k);
    if (parts == 1 || ws == nullptr || ws_bytes < topk_ws_bytes(n_q, ld, k)) {
        launch_rows<kWholeRow>(dim3((unsigned)n_q), ld, vec, scores, ld, q_pos, k, idx, 1, nullptr, nullptr, stream);
        return hipGetLastError();
    }
    float *ws_score = reinterpret_cast<float *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
    int32_t *ws_idx = reinterpret_cast<int32_t *>(ws_score + (size_t)n_q * parts * k);
    // longest part: 4 ceil(ceil(ld / 4) / parts) scores, or about 4k in a row of
    // fewer parts (a row of n scores has n / 2k of them)
    const int64_t part_len = std::max<int64_t>(4 * (((ld + 3) / 4 + parts - 1) / parts), 4 * (int64_t)k + 4);
    launch_rows<kPart>(dim3((unsigned)n_q, (unsigned)parts), part_len, vec, scores, ld, q_pos, k, idx, parts, ws_score,
                       ws_idx, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_rows<kMerge>(dim3((unsigned)n_q), (int64_t)parts * k, ((int64_t)parts * k) % 4 == 0, scores, ld, q_pos, k,
                        idx, parts, ws_score, ws_idx, stream);
    return hipGetLastError();
}

}  // namespace dsa

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
//     global_load_lds_dwordx4 (no register staging), double-buffered.  The tile
//     is stored as eighteen 64-byte column blocks of 64 rows with the 16-byte
//     chunks of every row XOR-swizzled, so that one copy instruction moves 16
//     rows x 64 contiguous bytes, each lane keeps one source row for the whole
//     tile (one slot lookup, then immediate offsets), and both MFMA operand
//     reads below are bank-conflict free;
//   * the copies of tile j + 1 are spread between the MFMAs of tile j, one
//     every few MFMAs, so their latency is hidden behind the tile's work;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = 32 gathered rows from LDS,
//     B = the wave's 32 query heads held in VGPRs), in two 32-row halves with
//     an accumulator each.  The softmax of half 0 is spread over the MFMAs of
//     half 1 and that of half 1 over the O^T MFMAs of rows 0..31, a few VALU
//     instructions per MFMA in a three-stage software pipeline (a wave issues
//     independent VALU work while its own MFMA executes, but in order, so no
//     instruction may wait on another of the same slot).  FP8 rows keep half
//     0's softmax between the MFMAs (one accumulator), half 1's runs under the
//     O^T MFMAs of rows 0..31 likewise;
//   * softmax per head (= per lane column) in the exp2 domain against a fixed
//     reference: the head's maximum over the first 32 rows.  Probabilities of
//     later rows may exceed 1 by up to 2^64 before the reference must move; that
//     range is exact in fp32 sums and bf16 probabilities, and the final division
//     gives the same softmax as a running-max rescale.  A tile beyond it restarts
//     the query with a raised reference instead of rescaling the accumulators,
//     which keeps O^T in accumulation registers that VALU code never touches;
//   * O^T += V^T P^T: P^T is the S^T accumulator re-packed to bf16 in place
//     (its lane layout already is the B operand), V^T comes from the same LDS
//     tile through ds_read_b64_tr_b16 transposed reads.
// FP8 rows (E4M3 + per-row scale) are gathered as bytes, expanded to bf16 in
// LDS exactly, and their scale is applied to the logits and to P in fp32.
#include <type_traits>
#include <utility>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kTile = 64;                         // gathered rows per tile
constexpr int kRowB = kDk * 2;                    // bf16 row bytes (1152)
constexpr int kTileB = kTile * kRowB;             // 73728 bytes
constexpr int kColB = kTile * 64;                 // one 64-byte column block of a tile (4096 bytes)
constexpr int kF8TileB = kTile * kDk;             // 36864 bytes of staged FP8 codes
constexpr int kMaxK = 2048;
constexpr int kKSteps = kDk / 16;                 // 36 k-steps of 16 latent dims
constexpr int kQK = 2 * kKSteps;                  // S^T MFMAs per tile per wave (two 32-row halves)
constexpr int kPV = 4 * (kDv / 32);               // O^T MFMAs per tile per wave (4 k-steps x 16 dim tiles)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kHeadroom = 64.0f;                // log2 range allowed above a head's reference max
// K / V^T fragments in flight per wave (register rings); the FP8 variant needs
// registers for its row scales and keeps shorter rings.
template <bool FP8> constexpr int kLookK = 4;
template <bool FP8> constexpr int kLookV = FP8 ? 2 : 4;
constexpr int kCopySpan = 136;                    // the next tile's copies are spread over this many MFMAs

typedef __attribute__((address_space(3))) void lds_void;

// 16-byte asynchronous global -> LDS copy: lane l of the wave reads gsrc + IMM
// and writes lds_base + IMM + 16 l (the immediate offset advances both
// addresses).  Written as inline assembly because the compiler models the
// builtin form as an LDS access that may complete out of order, and then waits
// for every outstanding LDS read (lgkmcnt(0)) after each copy, which drains the
// register-ring prefetch of the MFMA operands.  The copy is tracked by vmcnt
// only; its destination is read after an explicit s_waitcnt and a barrier.  It
// has no register results.  m0 is a reserved register on this target, so the
// compiler ignores the clobber (with a warning); nothing else in these kernels
// uses m0 (the generated code sets it only in these copies).
template <int IMM>
__device__ __forceinline__ void g2lds16(const void *gsrc, uint32_t lds_base) {
    static_assert(IMM >= 0 && IMM < 4096, "immediate offset");
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2"
                 :
                 : "v"(gsrc), "s"(lds_base), "i"(IMM)
                 : "memory", "m0");
}

__device__ __forceinline__ lds_void *to_lds(void *p) { return (lds_void *)(p); }
// LDS byte address of a __shared__ object (wave-uniform)
__device__ __forceinline__ uint32_t lds_addr(void *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)to_lds(p));
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1, so that
// the body can use I where a constant expression is required.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ bf16x4 lds_tr16(const uint8_t *p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(const_cast<uint8_t *>(p)));
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ f32x16 mfma32_bf16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// O^T += V^T P^T with the accumulator pinned to the AGPR file.  This file is
// compiled with the VGPR form of the compiler's own MFMAs, so S^T lands in
// VGPRs where the softmax reads it; the 256 O^T accumulators per lane stay in
// AGPRs through this asm form instead of being moved between the files.  The
// compiler does not see an MFMA here, so the required wait states are written
// out by the caller: after VALU writes of the operands before the first one,
// and before the accumulators are read or rewritten after the last one.
__device__ __forceinline__ void mfma32_bf16_acc(f32x16 &c, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Workgroup barrier after this wave's LDS accesses and all but the newest N
// vector-memory loads (in issue order) have completed.  The copies above are
// invisible to the compiler's counter tracking, so every wait for them is written
// out here; the empty asm statements keep memory accesses on their side.
template <int N>
__device__ __forceinline__ void barrier_after_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Tile layout: row r (0..63), 16-byte chunk c (0..71) of the bf16 row lives at
//   (c / 4) * 4096 + 64 r + 16 ((c % 4) ^ swz(r)),  swz(r) = (r / 4) % 4.
// The K fragment reads (16 lanes = 16 consecutive rows x one chunk per LDS cycle)
// and the transposed V^T reads (32 lanes = 4 consecutive rows x 4 chunks x two
// 8-byte halves) then touch 16 resp. 32 distinct bank groups.  A staged FP8
// tile uses the same column blocks without the swizzle (9 blocks of 64 codes).
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int tile_off(int r, int c) { return (c >> 2) * kColB + 64 * r + 16 * ((c & 3) ^ swz(r)); }

// Tile buffers live in separate __shared__ arrays, each named statically at every
// use, so that the compiler can tell the asynchronous gather into one buffer from
// the reads of the other and does not make the reads wait for the gather.
template <int NW, bool FP8, bool SPLIT>
struct MlaSmem {
    float f8scale[FP8 ? kTile : 1];               // FP8 row scale
    float f8logit[FP8 ? kTile : 1];               // FP8 row scale x sm_scale x log2(e)
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
    static_assert(NW == 1 || NW == 2 || NW == 4, "waves per workgroup");
    constexpr int NT = NW * 64;
    constexpr int R = (kMaxK + NT - 1) / NT;      // index entries per thread
    // Copies per tile: one instruction moves 16 rows x 64 bytes (a 1 KB block of a
    // column block); bf16 tiles have 18 column blocks, staged FP8 tiles 9, and 4
    // row blocks each.  Wave w takes the row blocks w, w + NW, ..., so that a
    // lane's source row is fixed for the tile.
    constexpr int kCols = FP8 ? 9 : 18;
    constexpr int kRBW = 4 / NW;                  // row blocks per wave
    constexpr int kCopies = kCols * kRBW;         // copy instructions per wave per tile
    constexpr int kCopyEvery = kCopySpan / kCopies > 0 ? kCopySpan / kCopies : 1;
    static_assert(kCopies * kCopyEvery <= kQK + kPV, "copies must fit the MFMA stream");
    __shared__ __attribute__((aligned(16))) MlaSmem<NW, FP8, SPLIT> sm;
    // bf16 cache: tile_a / tile_b double buffer.  FP8 cache: codes staged in
    // f8_a / f8_b (double buffer), expanded into tile_a.
    __shared__ __attribute__((aligned(16))) uint8_t tile_a[kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t tile_b[FP8 ? 16 : kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t f8_a[FP8 ? kF8TileB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t f8_b[FP8 ? kF8TileB : 16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;     // lane half, lane within the half
    const int i16 = lane & 15, hd = (lane >> 4) & 1;
    // decode: workgroup b takes query b % n_q, split b / n_q, so that the splits of
    // a query are n_q apart in launch order and (with workgroups dealt round-robin
    // to the 8 XCDs, n_q a multiple of 8) share one XCD's L2 for q and the indices.
    // prefill: the last query first.  Later rows of a causal prefill select from
    // longer prefixes, all but the first k rows the same number of entries, so
    // the workgroups that start together end together and the next ones again
    // start together; each walks its selection in ascending position, so the
    // queries an XCD runs at once gather from the same stretch of the cache at
    // the same time (more L2 hits than when the short first rows start the
    // launch and scatter the phases).
    const int n_q_split = SPLIT ? (int)gridDim.x / n_splits : 0;
    const int t = SPLIT ? (int)blockIdx.x % n_q_split : (int)(gridDim.x - 1 - blockIdx.x);
    const int split = SPLIT ? (int)blockIdx.x / n_q_split : 0;
    const int per_split = SPLIT ? (k + n_splits - 1) / n_splits : k;
    const int i_begin = split * per_split;
    const int i_end = min(k, i_begin + per_split);
    const int head = 32 * wave + l32;
    const bool head_ok = head < h;

    // ---- resolve the selected rows to cache slots, compacted in index order:
    // thread tid takes entries i_begin + R tid .. + R-1
    {
        const int32_t *idx_row = idx + (int64_t)t * k;
        const int32_t *st_row = kv_slot_table + (int64_t)q_seq[t] * kv_pt_ld;
        // loads are issued unconditionally (clamped addresses, results selected
        // afterwards), so that each round trip is waited for once
        int32_t s[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = i_begin + R * tid + r;
            const int32_t v = idx_row[min(max(i, 0), k - 1)];
            s[r] = i < i_end ? v : -1;
        }
        int c = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool in_table = s[r] >= 0 && s[r] < kv_pt_ld;
            const int32_t v = st_row[in_table ? s[r] : 0];
            const int32_t sl = in_table && v >= 0 && v < n_slots ? v : -1;
            s[r] = sl;
            c += sl >= 0;
        }
        int x = c;                                // inclusive scan of the counts over the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (lane == 63) sm.wcount[wave] = (uint32_t)x;
        __syncthreads();
        int pos = x - c, tot = 0;
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) {
            const int cw = (int)sm.wcount[wv];
            if (wv < wave) pos += cw;
            tot += cw;
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (s[r] >= 0) sm.slots[pos++] = s[r];
        if (tid == 0) {
            sm.n_valid = tot;
            sm.restart = 0;
        }
    }
    __syncthreads();
    const int n_valid = sm.n_valid;
    const int n_tiles = (n_valid + kTile - 1) / kTile;

    // ---- Q^T fragments of this wave's 32 heads (B operand): k-step ks holds
    // latent dims 16 ks + 8 g .. +8 of head `head` (a missing head reads the
    // last head's row; its results are never stored).  Loaded after the first
    // tile's copies are issued.
    bf16x8 qf[kKSteps];
    auto load_q = [&]() {
        const uint16_t *qrow = q + ((int64_t)t * h + (head_ok ? head : h - 1)) * kDk + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qrow + 16 * ks));
    };

    // ---- tile copies.  In row block b (16 rows) lane l takes row 16 b + l / 4 and
    // the 16-byte piece l % 4 of each 64-byte column block, which for a bf16 tile
    // holds chunk 4 col + ((l % 4) ^ swz(row)); swz(row) = (l / 16) % 4 for every
    // row block.  So a copy is the lane's row address plus an immediate offset;
    // the same immediate also advances the LDS address, which the LDS base
    // argument compensates.
    const float c2 = sm_scale * kLog2e;           // logits in log2 units: c2 * (q . k)
    const uint8_t *kvb = reinterpret_cast<const uint8_t *>(kv_cache);
    const int piece = FP8 ? (lane & 3) : ((lane & 3) ^ ((lane >> 4) & 3));
    auto copy_src = [&](int j, int b) -> const uint8_t * {
        const int r = 16 * (wave + NW * b) + (lane >> 2);
        const int rr = j * kTile + r < n_valid ? j * kTile + r : 0;
        const int64_t sl = sm.slots[rr];
        return kvb + sl * (FP8 ? kDk : kRowB) + 16 * piece;
    };
    // copy instruction n (0 .. kCopies-1) of this wave: row block n / kCols, column block n % kCols
    auto copy_one = [&](auto nc, const uint8_t *const *src, uint8_t *dst) {
        constexpr int n = decltype(nc)::value;
        constexpr int b = n / kCols, col = n % kCols;
        const int rb = wave + NW * b;
        g2lds16<64 * col>(src[b], lds_addr(dst) + col * (kColB - 64) + rb * 1024);
    };
    // FP8: expand the staged codes of tile j into the bf16 tile (exact) and fetch
    // the row scales.  Staged block blk (1 KB) holds rows 16 (blk % 4) + l / 4,
    // codes 64 (blk / 4) + 16 (l % 4) .. +16 in lane l's 16 bytes.
    auto expand = [&](int j, const uint8_t *src, uint8_t *dst_tile) {
        if constexpr (FP8) {
#pragma unroll 1
            for (int n = 0; n < 36 / NW; ++n) {
                const int blk = wave + NW * n;
                const int r = 16 * (blk & 3) + (lane >> 2), c8 = 4 * (blk >> 2) + (lane & 3);
                const uint4 v = *reinterpret_cast<const uint4 *>(&src[blk * 1024 + 16 * lane]);
                const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
                uint32_t o8[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // E4M3 -> bf16 is exact (scale 1): one instruction per two codes
                    const bf16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[e], 1.0f, false);  // bytes 0, 1
                    const bf16x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wds[e], 1.0f, true);   // bytes 2, 3
                    o8[2 * e] = __builtin_bit_cast(uint32_t, b0);
                    o8[2 * e + 1] = __builtin_bit_cast(uint32_t, b1);
                }
                *reinterpret_cast<uint4 *>(&dst_tile[tile_off(r, 2 * c8)]) = make_uint4(o8[0], o8[1], o8[2], o8[3]);
                *reinterpret_cast<uint4 *>(&dst_tile[tile_off(r, 2 * c8 + 1)]) = make_uint4(o8[4], o8[5], o8[6], o8[7]);
            }
            if (tid < kTile) {
                const int rr = j * kTile + tid < n_valid ? j * kTile + tid : 0;
                const float sc = kv_scale[sm.slots[rr]];
                sm.f8scale[tid] = sc;
                sm.f8logit[tid] = sc * c2;
            }
        }
    };

    // Per-lane LDS byte offsets within a tile.
    // K fragment (half hf, k-step ks): row 32 hf + l32, chunk 2 ks + g
    //   -> (ks / 2) * 4096 + 2048 hf + k_off[ks % 2].
    // V^T fragment (k-step kk, dim tile dt, lo / hi): lane i16 of a 16-lane group
    // supplies row 16 kk + 8 hi + 4 g + i16 / 4 at dims 32 dt + 16 hd + 4 (i16 % 4),
    // i.e. chunk 4 dt + 2 hd + (i16 / 2) % 2, half i16 % 2
    //   -> dt * 4096 + 1024 kk + v_off[hi].
    int k_off[2], v_off[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) k_off[qq] = 64 * l32 + 16 * ((2 * qq + g) ^ swz(l32));
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
        const int r = 8 * hi + 4 * g + (i16 >> 2), cq = 2 * hd + ((i16 >> 1) & 1);
        v_off[hi] = 64 * r + 16 * (cq ^ swz(r)) + 8 * (i16 & 1);
    }

    // O^T accumulators: o[dt][i] holds latent dim 32 dt + 8 (i / 4) + 4 g + i % 4 of head `head`
    f32x16 o[16];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
    // Softmax reference: each head's maximum over the first 32 rows.  Later rows
    // are exponentiated against it as long as their tile's maximum stays within
    // kHeadroom (log2 units) of it, which fp32 sums and bf16 probabilities hold
    // exactly as the rescaled form would; a tile beyond that restarts the query
    // with the larger reference, so the accumulators are never rescaled.
    float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.0f;

    // Attempts: the second and later ones only run after a tile exceeded its head's
    // reference by more than kHeadroom (practically never); they restart from tile
    // 0 with every reference raised to the largest maximum seen so far.
    bool again = true, first_attempt = true;
    while (again) {
        // one tile: `cur` holds tile j (bf16 rows, or FP8 codes to expand), the copies
        // of tile j + 1 go to `nxt`; returns true when the query must restart
        auto step = [&](const int j, uint8_t *cur, uint8_t *nxt) -> bool {
            barrier_after_loads<0>();                     // tile j landed; everyone is done with tile j - 1
            if (sm.restart != 0) return true;             // workgroup-uniform; nothing is in flight
            // copies of tile j + 1 (the last tile copies its own rows again, into the
            // idle buffer, so that the MFMA stream below has no branches)
            const int jn = j + 1 < n_tiles ? j + 1 : j;
            const uint8_t *src[kRBW];
#pragma unroll
            for (int b = 0; b < kRBW; ++b) src[b] = copy_src(jn, b);
            const uint8_t *tile = cur;
            if constexpr (FP8) {
                expand(j, cur, tile_a);
                barrier_after_loads<kKSteps>();
                tile = tile_a;
            }
            const int lim = n_valid - j * kTile - 4 * g;  // element (hf, i) is a valid row iff 32 hf + 8 (i/4) + i%4 < lim
            const bool partial = j * kTile + kTile > n_valid;

            // S^T = K Q^T in two halves of 32 rows (accumulator s covers rows
            // 32 hf + 8 (i / 4) + 4 g + i % 4), each followed by its softmax; then
            // O^T += V^T P^T.  K fragments run kLookK MFMAs ahead in a register
            // ring, V^T fragments kLookV; the copies of the next tile are spread
            // over all MFMAs.  Scheduling barriers keep that order.
            f32x16 s;
            float rmax = -INFINITY, psum = 0.0f;          // raw max of q.k (FP8: of the log2 logits), sum of p
            uint32_t pw[4][4];                            // P^T as bf16 pairs: k-step kk, pair e of 4
            auto kload = [&](int f) {
                const int hf = f / kKSteps, ks = f % kKSteps;
                return *reinterpret_cast<const uint4 *>(tile + (ks >> 1) * kColB + 2048 * hf + k_off[ks & 1]);
            };
            auto vload = [&](int f, bf16x4 &lo, bf16x4 &hi) {
                const int kk = f >> 4, dt = f & 15;
                const uint8_t *p = tile + dt * kColB + 1024 * kk;
                lo = lds_tr16(p + v_off[0]);
                hi = lds_tr16(p + v_off[1]);
            };
            // FP8 rows: softmax of the half just finished, p = 2^(logit - m_ref) with
            // the logit c2 q.k times the row scale, and p times the row scale again
            // (the scale of V), packed to bf16 pairs of the P^T operand
            auto softmax_half = [&](int hf) {
                if (first_attempt && j == 0 && hf == 0) {   // reference of every head: max over rows 0..31
                    float mx = -INFINITY;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float x = s[i] * sm.f8logit[8 * (i >> 2) + 4 * g + (i & 3)];
                        mx = fmaxf(mx, 8 * (i >> 2) + (i & 3) < lim ? x : -INFINITY);
                    }
                    m_ref = fmaxf(mx, swap_halves(mx));
                }
                // rows past the selection only occur in the last tile: a separate
                // (uniform) path keeps the masking out of every other tile
                auto body = [&](auto masked) {
#pragma unroll
                    for (int i = 0; i < 16; i += 2) {
                        float p[2];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int ii = i + e, rl = 32 * hf + 8 * (ii >> 2) + (ii & 3);
                            float v = s[ii] * sm.f8logit[rl + 4 * g];
                            float x = v - m_ref;
                            if constexpr (decltype(masked)::value) {
                                if (!(rl < lim)) { x = -INFINITY; v = -INFINITY; }
                            }
                            rmax = fmaxf(rmax, v);
                            p[e] = __builtin_amdgcn_exp2f(x);
                            psum += p[e];
                            p[e] *= sm.f8scale[rl + 4 * g];
                        }
                        const bf16x2 pk = {(__bf16)p[0], (__bf16)p[1]};
                        pw[2 * hf + (i >> 3)][(i & 7) >> 1] = __builtin_bit_cast(uint32_t, pk);
                    }
                };
                if (partial) body(std::true_type{});
                else body(std::false_type{});
            };
            // The MFMA stream of one tile.  SERIAL (FP8 rows): half 0's softmax runs
            // between the S^T MFMAs of the two halves (one accumulator), half 1's is
            // spread over the O^T MFMAs of rows 0..31.  bf16 rows: the softmax is spread
            // over the following MFMAs, about one element per MFMA (an exp2 and five
            // other VALU instructions, which the wave issues while its MFMA executes):
            // half 0's under the S^T MFMAs of half 1 (a second accumulator), half 1's
            // under the O^T MFMAs of rows 0..31, which only need half 0's
            // probabilities.  Rows past the selection (last tile only) hold copies of
            // the first selected row, so they change no maximum; their probabilities
            // are set to zero.
            auto run = [&](auto serial_c) {
                constexpr bool kSerial = decltype(serial_c)::value;
                uint4 kr[kLookK<FP8>];
                bf16x4 vlo[kLookV<FP8>], vhi[kLookV<FP8>];
                f32x16 s1;
                // Softmax of one half, software-pipelined over 18 MFMA slots so that no
                // instruction in a slot waits for another of the same slot: slot t forms
                // the logit of element t, exponentiates element t - 1 and masks, sums
                // and packs element t - 2 (element e: row rl of lanes 0..31, rl + 4 of
                // lanes 32..63; a row past the selection iff rl >= lim).
                float xs[3], pes[3], pprev = 0.0f;
                bool keep[3];
                auto sm_slot = [&](auto hfc, auto tc, const f32x16 &sv) {
                    constexpr int hf = decltype(hfc)::value, t = decltype(tc)::value;
                    if constexpr (t >= 2 && t < 18) {
                        constexpr int e = t - 2;
                        const float p = keep[e % 3] ? pes[e % 3] : 0.0f;
                        psum += p;
                        asm volatile("" : "+v"(psum));           // summed here, in row order
                        if constexpr (e & 1) {
                            const bf16x2 pk = {(__bf16)pprev, (__bf16)p};
                            pw[2 * hf + (e >> 3)][(e & 7) >> 1] = __builtin_bit_cast(uint32_t, pk);
                        } else {
                            pprev = p;
                        }
                    }
                    if constexpr (t >= 1 && t < 17) {
                        constexpr int e = t - 1;
                        pes[e % 3] = __builtin_amdgcn_exp2f(xs[e % 3]);
                        keep[e % 3] = 32 * hf + 8 * (e >> 2) + (e & 3) < lim;
                    }
                    if constexpr (t < 16) {
                        const float v = sv[t];
                        rmax = fmaxf(rmax, v);
                        xs[t % 3] = fmaf(v, c2, -m_ref);
                    }
                };
                float lg1[16], sc1[16];               // FP8: half 1's row scales of this lane
                auto f8_slot = [&](auto tc, const f32x16 &sv) {
                    constexpr int t = decltype(tc)::value;
                    if constexpr (t >= 2 && t < 18) {
                        constexpr int e = t - 2;
                        float p = keep[e % 3] ? pes[e % 3] : 0.0f;
                        psum += p;
                        asm volatile("" : "+v"(psum));
                        p *= sc1[e];
                        if constexpr (e & 1) {
                            const bf16x2 pk = {(__bf16)pprev, (__bf16)p};
                            pw[2 + (e >> 3)][(e & 7) >> 1] = __builtin_bit_cast(uint32_t, pk);
                        } else {
                            pprev = p;
                        }
                    }
                    if constexpr (t >= 1 && t < 17) {
                        constexpr int e = t - 1;
                        pes[e % 3] = __builtin_amdgcn_exp2f(xs[e % 3]);
                        keep[e % 3] = 32 + 8 * (e >> 2) + (e & 3) < lim;
                    }
                    if constexpr (t < 16) {
                        const float v = sv[t] * lg1[t];
                        rmax = fmaxf(rmax, v);
                        xs[t % 3] = v - m_ref;
                    }
                };
#pragma unroll
                for (int f = 0; f < kLookK<FP8>; ++f) kr[f] = kload(f);
                static_for<kQK>([&](auto fc) {
                    constexpr int f = decltype(fc)::value;
                    constexpr int ks = f % kKSteps;
                    if constexpr (f == kKSteps) {
                        if constexpr (kSerial) {
                            softmax_half(0);
                        } else if (first_attempt && j == 0) {   // reference of every head: max over rows 0..31
                            float mx = -INFINITY;
#pragma unroll
                            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i] * c2);
                            m_ref = fmaxf(mx, swap_halves(mx));
                        }
                    }
                    const uint4 kc = kr[f % kLookK<FP8>];
                    if constexpr (f + kLookK<FP8> < kQK) kr[f % kLookK<FP8>] = kload(f + kLookK<FP8>);
                    else if constexpr (f + kLookK<FP8> - kQK < kLookV<FP8>)
                        vload(f + kLookK<FP8> - kQK, vlo[f + kLookK<FP8> - kQK], vhi[f + kLookK<FP8> - kQK]);
                    if constexpr (kSerial || f < kKSteps)
                        s = mfma32_bf16(__builtin_bit_cast(bf16x8, kc), qf[ks], ks == 0 ? f32x16{} : s);
                    else
                        s1 = mfma32_bf16(__builtin_bit_cast(bf16x8, kc), qf[ks], ks == 0 ? f32x16{} : s1);
                    if constexpr (f % kCopyEvery == 0 && f / kCopyEvery < kCopies)
                        copy_one(std::integral_constant<int, f / kCopyEvery>{}, src, nxt);
                    if constexpr (!kSerial && f >= kKSteps + 2 && f < kKSteps + 20)
                        sm_slot(std::integral_constant<int, 0>{}, std::integral_constant<int, f - kKSteps - 2>{}, s);
                    __builtin_amdgcn_sched_barrier(0);
                });
                if constexpr (kSerial) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float4 a = *reinterpret_cast<const float4 *>(&sm.f8logit[32 + 8 * jj + 4 * g]);
                        const float4 b = *reinterpret_cast<const float4 *>(&sm.f8scale[32 + 8 * jj + 4 * g]);
                        lg1[4 * jj] = a.x; lg1[4 * jj + 1] = a.y; lg1[4 * jj + 2] = a.z; lg1[4 * jj + 3] = a.w;
                        sc1[4 * jj] = b.x; sc1[4 * jj + 1] = b.y; sc1[4 * jj + 2] = b.z; sc1[4 * jj + 3] = b.w;
                    }
                }
                static_for<kPV>([&](auto fc) {
                    constexpr int f = decltype(fc)::value;
                    if constexpr ((f + kQK) % kCopyEvery == 0 && (f + kQK) / kCopyEvery < kCopies)
                        copy_one(std::integral_constant<int, (f + kQK) / kCopyEvery>{}, src, nxt);
                    const bf16x4 lo = vlo[f % kLookV<FP8>], hi = vhi[f % kLookV<FP8>];
                    if constexpr (f + kLookV<FP8> < kPV) vload(f + kLookV<FP8>, vlo[f % kLookV<FP8>], vhi[f % kLookV<FP8>]);
                    const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    const uint4 bw = make_uint4(pw[f >> 4][0], pw[f >> 4][1], pw[f >> 4][2], pw[f >> 4][3]);
                    // wait states: P^T was just written by VALU code (serial: before the
                    // first O^T MFMA; overlapped: half 1's before the first MFMA of rows 32..63)
                    if constexpr (f == kPV / 2) asm volatile("s_nop 4");
                    mfma32_bf16_acc(o[f & 15], a, __builtin_bit_cast(bf16x8, bw));
                    if constexpr (!kSerial && f >= 2 && f < 20)
                        sm_slot(std::integral_constant<int, 1>{}, std::integral_constant<int, f - 2>{}, s1);
                    if constexpr (kSerial && f >= 2 && f < 20) f8_slot(std::integral_constant<int, f - 2>{}, s);
                    __builtin_amdgcn_sched_barrier(0);
                });
            };
            run(std::integral_constant<bool, FP8>{});
            float tmax = FP8 ? rmax : rmax * c2;          // c2 > 0: the max of the log2 logits
            tmax = fmaxf(tmax, swap_halves(tmax));
            m_seen = fmaxf(m_seen, tmax);
            if (__ballot(tmax > m_ref + kHeadroom) != 0) sm.restart = 1u;   // acted on after the next barrier
            l_run += psum;
            return false;
        };
        uint8_t *const buf_a = FP8 ? f8_a : tile_a;
        uint8_t *const buf_b = FP8 ? f8_b : tile_b;
        if (n_tiles > 0) {
            const uint8_t *src[kRBW];
#pragma unroll
            for (int b = 0; b < kRBW; ++b) src[b] = copy_src(0, b);
            static_for<kCopies>([&](auto nc) { copy_one(nc, src, buf_a); });
        }
        if (first_attempt) {
            load_q();
            // q is complete before the tile loop, so that the compiler's own counter
            // tracking does not wait for it (and for the copies behind it) inside
            __builtin_amdgcn_s_waitcnt(0);
        }
        for (int j = 0; j < n_tiles; j += 2) {
            if (step(j, buf_a, buf_b)) break;
            if (j + 1 < n_tiles && step(j + 1, buf_b, buf_a)) break;
        }
        barrier_after_loads<0>();
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");   // the last O^T MFMA has written back
        again = sm.restart != 0;
        first_attempt = false;
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

// ------------------------------------------------------------------ decode by head group
// One workgroup per (query, group of 32 heads) covers the query's whole
// selection, so no partial outputs leave the chip and no merge launch follows.
// The 4 waves share the group's 32 heads and take a quarter of the selected
// rows each, gathered into private 16-row sub-tiles (double-buffered; waves never
// wait for each other inside the row loop):
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: A = 16 gathered rows x 32 dims
//     from LDS, B = 16 heads of Q^T held in VGPRs; both head halves use each A
//     read.  The accumulator leaves lane l with head l % 16 of its half and rows
//     4 (l / 16) .. +3;
//   * softmax in the exp2 domain against a per-wave fixed reference (the
//     maximum over the wave's first sub-tile), restarting the wave's rows with a
//     raised reference when a logit exceeds it by more than kHeadroom, as above;
//   * O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with K = the sub-tile's 16
//     rows: one v_permlane16_swap per register pair turns the two halves' packed
//     probabilities into the B operand (lane l: head l % 32, rows 8 (l / 32) ..
//     +7), and the transposed V^T reads take the same rows;
//   * at the end the waves' partial outputs, each against its own reference,
//     are merged in LDS with log-sum-exp weights and normalised.
// The head groups of one query are n_q workgroups apart in launch order, so with
// workgroups dealt round-robin to the 8 XCDs (n_q a multiple of 8) they run on
// one XCD and each gathered row comes from HBM once, the other reads from L2.
// A wave keeps one sub-tile in flight while it computes the other (LDS holds
// no more), so the gather latency is what bounds it; loading one dword of every
// cache line three sub-tiles ahead to warm L2 doubled the line requests and
// measured slower (58.6 -> 75.5 us for 64 queries x 2048 rows x 128 heads).
constexpr int kSub = 16;                          // rows of a wave's sub-tile
constexpr int kSubB = kSub * kRowB;               // 18432 bytes of bf16 rows
constexpr int kSubColB = kSub * 64;               // one 64-byte column block of a sub-tile
constexpr int kF8SubB = kSub * kDk;               // 9216 bytes of staged FP8 codes
constexpr int kK32 = kDk / 32;                    // 18 k-steps of 32 latent dims
constexpr int kHgRowsPerWave = kMaxK / 4;         // selected entries per wave (at most)

// 4-byte asynchronous global -> LDS copy: lane l reads gsrc + IMM and writes
// lds_base + IMM + 4 l (same conventions as g2lds16).
template <int IMM>
__device__ __forceinline__ void g2lds4(const void *gsrc, uint32_t lds_base) {
    static_assert(IMM >= 0 && IMM < 4096, "immediate offset");
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off offset:%2"
                 :
                 : "v"(gsrc), "s"(lds_base), "i"(IMM)
                 : "memory", "m0");
}

// This wave's LDS accesses and all but its newest N vector-memory loads (in
// issue order) have completed; no workgroup barrier.
template <int N>
__device__ __forceinline__ void wave_wait_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ f32x4 mfma16_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max over the four lanes l % 16 + 16 m (the rows of one head in the 16x16 layout)
__device__ __forceinline__ float max_over_row_groups(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float sum_over_row_groups(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// Eight E4M3 codes -> eight bf16 values (exact), in order.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(const uint2 v) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Transposed 8-byte LDS read (measured lane layout): within each 16-lane group,
// lane 2 r + h supplies 8 bytes (row r, columns 8 h .. +7 of an 8 x 16 byte
// block) and lane i receives column i, rows 0..7 as bytes 0..7.
__device__ __forceinline__ uint2 lds_tr8(const uint8_t *p) {
    typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(const_cast<uint8_t *>(p)));
    return make_uint2((uint32_t)v.x, (uint32_t)v.y);
}

template <bool FP8>
__global__ __launch_bounds__(256, 1) void sparse_mla_hg_kernel(
    const uint16_t *__restrict__ q, const void *__restrict__ kv_cache, const float *__restrict__ kv_scale,
    int64_t n_slots, const int32_t *__restrict__ kv_slot_table, int64_t kv_pt_ld, const int32_t *__restrict__ q_seq,
    const int32_t *__restrict__ idx, int32_t n_q, int32_t h, int32_t k, float sm_scale, uint16_t *__restrict__ out,
    float *__restrict__ lse) {
    constexpr int kCols = FP8 ? 9 : 18;                 // 64-byte column blocks copied per sub-tile
    constexpr int kC = kCols + (FP8 ? 1 : 0);           // copy instructions per sub-tile (FP8: + the row scales)
    constexpr int kLookK = 4, kLookV = 4;               // operand fragments in flight (register rings)
    // Ring of sub-tile stages per wave: bf16 rows double-buffered (the next copies go
    // into the stage being computed, block by block after its last read), FP8 codes
    // in 4 stages with 3 sub-tiles in flight (copies go into the stage computed last).
    constexpr int kStages = FP8 ? 4 : 2;
    constexpr int kStageB = FP8 ? kF8SubB : kSubB;
    constexpr int kWaitN = FP8 ? 2 * kC : kC;           // copies issued after a sub-tile's, at its wait
    __shared__ __attribute__((aligned(16))) int32_t slots[4][kHgRowsPerWave];
    __shared__ __attribute__((aligned(16))) uint8_t stages[4][kStages][kStageB];   // also the merge buffer
    __shared__ __attribute__((aligned(16))) float fscale[FP8 ? 4 : 1][FP8 ? kStages : 1][64];   // FP8 row scales
    __shared__ float stat_m[4][32], stat_l[4][32];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = (int)blockIdx.x % n_q, grp = (int)blockIdx.x / n_q;
    const int l16 = lane & 15, q4 = lane >> 4, g = lane >> 5, hd = (lane >> 4) & 1;

    // ---- this wave's entries [e0, e1) of the index list, resolved to slots and
    // compacted in order
    int n_w;
    {
        const int per_wave = (k + 3) / 4;
        const int e0 = wave * per_wave, e1 = min(k, e0 + per_wave);
        const int32_t *idx_row = idx + (int64_t)t * k;
        const int32_t *st_row = kv_slot_table + (int64_t)q_seq[t] * kv_pt_ld;
        int32_t s[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int i = e0 + 8 * lane + r;
            const int32_t v = idx_row[min(i, k - 1)];
            s[r] = i < e1 ? v : -1;
        }
        int c = 0;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const bool in_table = s[r] >= 0 && s[r] < kv_pt_ld;
            const int32_t v = st_row[in_table ? s[r] : 0];
            const int32_t sl = in_table && v >= 0 && v < n_slots ? v : -1;
            s[r] = sl;
            c += sl >= 0;
        }
        int x = c;                                    // inclusive scan of the counts over the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        n_w = __builtin_amdgcn_readlane(x, 63);
        int pos = x - c;
#pragma unroll
        for (int r = 0; r < 8; ++r)
            if (s[r] >= 0) slots[wave][pos++] = s[r];
    }
    __builtin_amdgcn_s_waitcnt(0);                    // the slot list is in LDS before any lane reads it
    __builtin_amdgcn_wave_barrier();
    const int n_sub = (n_w + kSub - 1) / kSub;

    // ---- copies of sub-tile j (16 rows).  Copy instruction c moves column block c
    // (64 bytes of each row): lane l takes row l / 4 and the 16-byte piece
    // (l % 4) ^ swz(l / 4) of the block, so slot p of row r in LDS holds piece
    // p ^ swz(r) (swz(l / 4) = (l / 16) % 4).
    const uint8_t *kvb = reinterpret_cast<const uint8_t *>(kv_cache);
    constexpr int kRowBytes = FP8 ? kDk : kRowB;
    const int piece = (lane & 3) ^ ((lane >> 4) & 3);
    auto slot_of = [&](int r) -> int64_t { return slots[wave][r < n_w ? r : 0]; };
    auto copy_src = [&](int j) { return kvb + slot_of(16 * j + (lane >> 2)) * kRowBytes + 16 * piece; };
    auto copy_col = [&](auto cc, const uint8_t *src, uint8_t *dst) {   // column block c
        constexpr int c = decltype(cc)::value;
        g2lds16<64 * c>(src, lds_addr(dst) + c * (kSubColB - 64));
    };
    auto copies = [&](int j, uint8_t *dst, float *sdst) {
        const uint8_t *src = copy_src(j);
        static_for<kCols>([&](auto cc) { copy_col(cc, src, dst); });
        if constexpr (FP8) g2lds4<0>(kv_scale + slot_of(16 * j + (lane & 15)), lds_addr(sdst));
    };
    auto stage_of = [&](int s_) { return &stages[wave][s_][0]; };
    auto scale_of = [&](int s_) { return &fscale[FP8 ? wave : 0][FP8 ? s_ : 0][0]; };

    // ---- Q^T of the group's heads (B operands): head 32 grp + 16 hh + l % 16, dims
    // 32 ks + 8 (l / 16) .. +8 (a head past h reads the last head; never stored)
    bf16x8 qf[2][kK32];
    auto load_q = [&]() {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int hq = min(32 * grp + 16 * hh + l16, h - 1);
            const uint16_t *qrow = q + ((int64_t)t * h + hq) * kDk + 8 * q4;
#pragma unroll
            for (int ks = 0; ks < kK32; ++ks)
                qf[hh][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(qrow + 32 * ks));
        }
    };

    // Per-lane LDS offsets within a stage.
    // bf16 K fragment of k-step ks: row l % 16, chunk l / 16 of column block ks.
    // bf16 V^T fragment of dim tile dt (lo / hi): lane i16 of a 16-lane group
    // supplies row 8 g + 4 hi + i16 / 4 at dims 32 dt + 16 hd + 4 (i16 % 4), so the
    // transposed reads give lane l rows 8 (l / 32) .. +7 of dim 32 dt + l % 32.
    // FP8 K fragment of k-step ks: row l % 16, codes 32 ks + 8 (l / 16) .. +8, i.e.
    // column block ks / 2, piece 2 (ks % 2) + (l / 16) / 2, half (l / 16) % 2.
    // FP8 V^T fragment of dim tile dt: lane 2 r + h of group G = l / 16 supplies row
    // 8 (G / 2) + r, codes 32 dt + 16 (G % 2) + 8 h .. +8 (column block dt / 2,
    // piece 2 (dt % 2) + G % 2), so the transposed read gives lane l rows
    // 8 (l / 32) .. +7 of dim 32 dt + l % 32.
    int k_off[2], v_off[2];
    if constexpr (FP8) {
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            k_off[par] = 64 * l16 + 16 * ((2 * par + (q4 >> 1)) ^ swz(l16)) + 8 * (q4 & 1);
            const int r = 8 * (q4 >> 1) + (l16 >> 1), pc = 2 * par + (q4 & 1);
            v_off[par] = 64 * r + 16 * (pc ^ swz(r)) + 8 * (l16 & 1);
        }
    } else {
        k_off[0] = k_off[1] = 64 * l16 + 16 * (q4 ^ swz(l16));
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
            const int r = 8 * g + 4 * hi + (l16 >> 2), cq = 2 * hd + ((l16 >> 1) & 1);
            v_off[hi] = 64 * r + 16 * (cq ^ swz(r)) + 8 * (l16 & 1);
        }
    }

    const float c2 = sm_scale * kLog2e;               // logits in log2 units: c2 * (q . k)
    // O^T accumulators: o[dt][i] holds dim 32 dt + 8 (i / 4) + 4 g + i % 4 of head 32 grp + l % 32
    f32x16 o[16];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
    // softmax state per head half hh (head 32 grp + 16 hh + l % 16): reference, row
    // sum of this lane's rows, largest logit above the reference seen in this attempt
    float m_ref[2] = {-INFINITY, -INFINITY}, psum[2] = {0.0f, 0.0f}, xmax[2] = {-INFINITY, -INFINITY};
    bool first_attempt = true, again = n_sub > 0;

    while (again) {
        again = false;
        // one sub-tile in stage S: returns true when this wave must start over with a
        // raised reference
        auto step = [&](auto sc_, const int j) -> bool {
            constexpr int S = decltype(sc_)::value;
            uint8_t *cur = stage_of(S);
            wave_wait_loads<kWaitN>();                // sub-tile j landed
            float sc[4], sl[4];                        // FP8: row scale, and scale x c2, of rows 4 q4 + i
            const uint8_t *nsrc = nullptr;
            if constexpr (FP8) {
                const float4 f = *reinterpret_cast<const float4 *>(scale_of(S) + 4 * q4);
                sc[0] = f.x; sc[1] = f.y; sc[2] = f.z; sc[3] = f.w;
#pragma unroll
                for (int i = 0; i < 4; ++i) sl[i] = sc[i] * c2;
                // sub-tile j + 3 goes into the stage computed last (its reads are done)
                constexpr int SN = (S + 3) % 4;
                copies(j + 3 < n_sub ? j + 3 : n_sub - 1, stage_of(SN), scale_of(SN));
            } else {
                // sub-tile j + 2 goes into this stage column block by column block,
                // each right after the block's last read (the rope blocks 16, 17 after
                // the S^T MFMAs, block dt after the O^T MFMA of dim tile dt), spread
                // over the MFMAs instead of issued in one burst
                nsrc = copy_src(j + 2 < n_sub ? j + 2 : n_sub - 1);
            }
            const int lim = n_w - 16 * j - 4 * q4;    // element i is a selected row iff i < lim
            const bool partial = 16 * j + 16 > n_w;

            // S^T for both head halves over 18 k-steps; K fragments kLookK ahead
            using KFrag = std::conditional_t<FP8, uint2, uint4>;
            using VFrag = std::conditional_t<FP8, uint2, uint4>;
            auto kload = [&](int ks) -> KFrag {
                return *reinterpret_cast<const KFrag *>(cur + (FP8 ? (ks >> 1) : ks) * kSubColB + k_off[ks & 1]);
            };
            auto kfrag = [&](const KFrag &v) -> bf16x8 {
                if constexpr (FP8) return fp8x8_to_bf16(v);
                else return __builtin_bit_cast(bf16x8, v);
            };
            auto vload = [&](int dt) -> VFrag {
                if constexpr (FP8) {
                    return lds_tr8(cur + (dt >> 1) * kSubColB + v_off[dt & 1]);
                } else {
                    const uint8_t *p = cur + dt * kSubColB;
                    const bf16x4 lo = lds_tr16(p + v_off[0]), hi = lds_tr16(p + v_off[1]);
                    return __builtin_bit_cast(uint4, bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
                }
            };
            auto vfrag = [&](const VFrag &v) -> bf16x8 {
                if constexpr (FP8) return fp8x8_to_bf16(v);
                else return __builtin_bit_cast(bf16x8, v);
            };
            f32x4 s[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
            KFrag kr[kLookK];
            VFrag vr[kLookV];
#pragma unroll
            for (int f = 0; f < kLookK; ++f) kr[f] = kload(f);
            // FP8: each K fragment is expanded one k-step ahead, under the MFMAs of
            // the step before, so that no MFMA waits on its own conversion
            bf16x8 a_next;
            if constexpr (FP8) a_next = kfrag(kr[0]);
            static_for<kK32>([&](auto kc) {
                constexpr int ks = decltype(kc)::value;
                const bf16x8 a = FP8 ? a_next : kfrag(kr[ks % kLookK]);
                if constexpr (ks + kLookK < kK32) kr[ks % kLookK] = kload(ks + kLookK);
                else vr[ks + kLookK - kK32] = vload(ks + kLookK - kK32);
                s[0] = mfma16_bf16(a, qf[0][ks], s[0]);
                s[1] = mfma16_bf16(a, qf[1][ks], s[1]);
                if constexpr (FP8 && ks + 1 < kK32) a_next = kfrag(kr[(ks + 1) % kLookK]);
                if constexpr (!FP8 && ks == kK32 - 1) {
                    copy_col(std::integral_constant<int, 16>{}, nsrc, cur);
                    copy_col(std::integral_constant<int, 17>{}, nsrc, cur);
                }
                __builtin_amdgcn_sched_barrier(0);
            });

            // softmax: p = 2^(c2 q.k - m_ref) (FP8: the row scale in the logit and in p)
            if (first_attempt && j == 0) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, i < lim ? s[hh][i] * (FP8 ? sl[i] : c2) : -INFINITY);
                    m_ref[hh] = max_over_row_groups(mx);
                }
            }
            uint32_t pk[2][2];
            auto body = [&](auto masked) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    float p[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float x = FP8 ? s[hh][i] * sl[i] - m_ref[hh] : fmaf(s[hh][i], c2, -m_ref[hh]);
                        if constexpr (decltype(masked)::value) {
                            if (!(i < lim)) x = -INFINITY;
                        }
                        xmax[hh] = fmaxf(xmax[hh], x);
                        p[i] = __builtin_amdgcn_exp2f(x);
                        psum[hh] += p[i];
                        if constexpr (FP8) p[i] *= sc[i];
                    }
                    const bf16x2 p01 = {(__bf16)p[0], (__bf16)p[1]}, p23 = {(__bf16)p[2], (__bf16)p[3]};
                    pk[hh][0] = __builtin_bit_cast(uint32_t, p01);
                    pk[hh][1] = __builtin_bit_cast(uint32_t, p23);
                }
            };
            if (partial) body(std::true_type{});
            else body(std::false_type{});
            // lane l of row group G holds head 16 hh + l % 16, rows 4 G .. +3; after the
            // swaps, r0[0], r1[0] hold rows 8 (l / 32) + 0..3 and r0[1], r1[1] rows
            // 8 (l / 32) + 4..7 of head l % 32
            const auto r0 = __builtin_amdgcn_permlane16_swap(pk[0][0], pk[1][0], false, false);
            const auto r1 = __builtin_amdgcn_permlane16_swap(pk[0][1], pk[1][1], false, false);
            const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(r0[0], r1[0], r0[1], r1[1]));

            // O^T += V^T P^T over the 16 dim tiles; V^T fragments kLookV ahead (FP8:
            // expanded one MFMA ahead, as the K fragments above)
            bf16x8 v_next;
            if constexpr (FP8) v_next = vfrag(vr[0]);
            static_for<16>([&](auto dc) {
                constexpr int dt = decltype(dc)::value;
                const bf16x8 a = FP8 ? v_next : vfrag(vr[dt % kLookV]);
                if constexpr (dt + kLookV < 16) vr[dt % kLookV] = vload(dt + kLookV);
                // wait states: pb (and, FP8, the expanded V^T fragment) were written by VALU code
                if constexpr (dt == 0 || FP8) asm volatile("s_nop 4");
                mfma32_bf16_acc(o[dt], a, pb);                    // its operand reads of block dt are done
                if constexpr (FP8 && dt + 1 < 16) v_next = vfrag(vr[(dt + 1) % kLookV]);
                if constexpr (!FP8) copy_col(dc, nsrc, cur);
                __builtin_amdgcn_sched_barrier(0);
            });
            return __ballot(fmaxf(xmax[0], xmax[1]) > kHeadroom) != 0;
        };
        // prologue: the sub-tiles in flight when step 0 starts (bf16: 0, 1; FP8: 0, 1, 2)
        static_for<FP8 ? kStages - 1 : kStages>([&](auto sc_) {
            constexpr int S = decltype(sc_)::value;
            copies(S < n_sub ? S : n_sub - 1, stage_of(S), scale_of(S));
        });
        if (first_attempt) {
            load_q();
            __builtin_amdgcn_s_waitcnt(0);            // q complete before the row loop (see the kernel above)
        }
        for (int j = 0; j < n_sub; j += kStages) {
            if (step(std::integral_constant<int, 0>{}, j)) { again = true; break; }
            if (j + 1 < n_sub && step(std::integral_constant<int, 1>{}, j + 1)) { again = true; break; }
            if constexpr (kStages == 4) {
                if (j + 2 < n_sub && step(std::integral_constant<int, 2>{}, j + 2)) { again = true; break; }
                if (j + 3 < n_sub && step(std::integral_constant<int, 3>{}, j + 3)) { again = true; break; }
            }
        }
        wave_wait_loads<0>();                         // nothing of this attempt is in flight
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");   // the last O^T MFMA has written back
        first_attempt = false;
        if (again) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                m_ref[hh] += max_over_row_groups(xmax[hh]);
                xmax[hh] = -INFINITY;
                psum[hh] = 0.0f;
            }
#pragma unroll
            for (int dt = 0; dt < 16; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
        }
    }

    // ---- merge the 4 waves' partial outputs of each head with weights 2^(m_w - M)
    {
        const float l0 = sum_over_row_groups(psum[0]), l1 = sum_over_row_groups(psum[1]);
        if (lane < 16) {
            stat_m[wave][lane] = m_ref[0];
            stat_m[wave][16 + lane] = m_ref[1];
            stat_l[wave][lane] = l0;
            stat_l[wave][16 + lane] = l1;
        }
    }
    __syncthreads();
    const int hl = lane & 31;                         // head 32 grp + hl in the O^T layout
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, stat_m[w][hl]);
    float Lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float mw = stat_m[w][hl];
        Lsum += mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M) * stat_l[w][hl];
    }
    const float f_own = stat_m[wave][hl] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(stat_m[wave][hl] - M);
    const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
    const int head = 32 * grp + hl;
    // rounds of 4 dim tiles: every wave writes its scaled partials of the round's
    // tiles, wave w sums tile 4 round + w over the waves.  Float4 e of lane l sits at
    // float4 index 4 l + ((e + l / 4) % 4) of a tile block: conflict-free.
    float4 *mbuf = reinterpret_cast<float4 *>(&stages[0][0][0]);   // [wave][tile][64 lanes x 4]
    auto slot4 = [&](int w, int d, int e) { return (w * 4 + d) * 256 + 4 * lane + ((e + (lane >> 2)) & 3); };
#pragma unroll
    for (int round = 0; round < 4; ++round) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const f32x16 &ot = o[4 * round + d];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mbuf[slot4(wave, d, e)] = make_float4(ot[4 * e] * f_own, ot[4 * e + 1] * f_own, ot[4 * e + 2] * f_own,
                                                      ot[4 * e + 3] * f_own);
        }
        __syncthreads();
        const int dt = 4 * round + wave;
        float acc[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float4 v = mbuf[slot4(w, wave, e)];
                acc[4 * e] += v.x;
                acc[4 * e + 1] += v.y;
                acc[4 * e + 2] += v.z;
                acc[4 * e + 3] += v.w;
            }
        }
        if (head < h) {
            uint16_t *orow = out + ((int64_t)t * h + head) * kDv + 32 * dt + 4 * g;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bf16x4 v;
#pragma unroll
                for (int x = 0; x < 4; ++x) v[x] = (__bf16)(acc[4 * e + x] * inv);
                *reinterpret_cast<bf16x4 *>(orow + 8 * e) = v;
            }
        }
        __syncthreads();
    }
    if (lse != nullptr && wave == 0 && g == 0 && head < h)
        lse[(int64_t)t * h + head] = Lsum > 0.0f ? (M + __log2f(Lsum)) * 0.6931471805599453f : -INFINITY;
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
    default: launch_mla_t<4, FP8, SPLIT>(a, n_splits, ws_o, ws_lse, stream); break;   // 3 x 32 heads run as 4
    }
}

hipError_t launch_mla_prefill(const MlaArgs &a, hipStream_t stream) {
    if (a.fp8) launch_mla_nw<true, false>(a, 1, nullptr, nullptr, stream);
    else launch_mla_nw<false, false>(a, 1, nullptr, nullptr, stream);
    return hipGetLastError();
}

static int mla_head_groups(int32_t h) { return (h + 31) / 32; }

int mla_decode_auto_splits(int32_t n_q, int32_t h, int32_t k) {
    // One workgroup per (query, 32 heads) when that gives between half and all of a
    // 256-CU device one workgroup each (64 queries x 128 heads: 256 workgroups):
    // nothing leaves the chip but the output.  More workgroups would run in two
    // rounds (128 queries: 164 us against 120 us with 2 splits).  Otherwise the
    // index list is split, each split writing an fp32 partial output that a second
    // launch merges: about one workgroup per CU (every split re-reads the query's
    // q block and writes and re-reads a 128 x 512 fp32 partial).
    const int64_t wg = (int64_t)n_q * mla_head_groups(h);
    if (wg >= 128 && wg <= 256) return 1;
    int s = 1;
    while (s < 32 && (int64_t)n_q * s < 256 && k / (2 * s) >= 2 * kTile) s *= 2;
    return s > 1 ? s : 2;
}

size_t mla_decode_ws_bytes(int32_t n_q, int32_t h, int32_t n_splits) {
    if (n_splits <= 1) return 0;
    const size_t o = (size_t)n_q * n_splits * h * kDv * sizeof(float);
    const size_t l = (size_t)n_q * n_splits * h * sizeof(float);
    return o + ((l + 255) / 256) * 256 + 256;
}

template <bool FP8>
static void launch_mla_hg(const MlaArgs &a, hipStream_t stream) {
    const unsigned grid = (unsigned)((int64_t)a.n_q * mla_head_groups(a.h));
    hipLaunchKernelGGL((sparse_mla_hg_kernel<FP8>), dim3(grid), dim3(256), 0, stream, a.q,
                       a.kv_cache, a.kv_scale, a.n_slots, a.kv_slot_table, a.kv_pt_ld, a.q_seq, a.idx, a.n_q, a.h, a.k,
                       a.sm_scale, a.out, a.lse);
}

hipError_t launch_mla_decode(const MlaArgs &a, int n_splits, void *ws, hipStream_t stream) {
    if (n_splits <= 1) {
        if (a.fp8) launch_mla_hg<true>(a, stream);
        else launch_mla_hg<false>(a, stream);
        return hipGetLastError();
    }
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

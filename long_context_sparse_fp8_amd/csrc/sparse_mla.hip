// sparse_mla.hip -- attention over the top-k selected latent rows (gfx950).
//
// For query t, head h and the selected set S_t (DeepSeek-V3.2-Exp deployment
// article, section 1: only the top-k key/value entries enter attention; SGLang
// usage guide, "attention kernel selection": bf16 q with bf16 or fp8 kv):
//   l_s = sm_scale * q[t,h,:] . K[s,:]   (576-d latent keys)
//   out[t,h,:] = softmax(l) @ K[S_t, :512],  lse[t,h] = log sum exp(l)
//
// One workgroup per query (decode: per query and index split); every wave
// owns 16 heads, so 128 heads are 8 waves (2 per SIMD) and Q^T (72 VGPRs)
// plus the fp32 O^T accumulator (128) stay in registers for the whole query.
// Per 64-row tile:
//   * the selected rows are gathered straight into LDS with
//     global_load_lds_dwordx4 (no register staging), double-buffered, rows
//     padded to 1168 bytes so both the row reads and the transposed reads
//     below are bank-conflict free;
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A = 16 gathered rows from LDS,
//     B = the wave's 16 query heads held in VGPRs);
//   * online softmax per head (= per lane column), exp2 domain;
//   * O^T += V^T P^T: P^T is the S^T accumulator re-packed to bf16 in place
//     (its lane layout already is the B operand), V^T comes from the same LDS
//     tile through ds_read_b64_tr_b16 transposed reads.
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
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLook = 4;                          // LDS fragment loads in flight per wave

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

template <int NW, bool FP8, bool SPLIT>
struct MlaSmem {
    // bf16 tiles: two for the bf16 cache (double buffer), one for FP8 (filled by conversion)
    uint8_t tile[FP8 ? 1 : 2][kTileB];
    uint8_t f8[FP8 ? 2 : 1][FP8 ? kF8TileB : 16];
    float f8scale[FP8 ? kTile : 1];
    int32_t slots[kMaxK];
    uint32_t wcount[NW];
    int32_t n_valid;
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

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = lane >> 4, i16 = lane & 15;     // 16-lane group, lane within it
    const int t = SPLIT ? (int)blockIdx.x / n_splits : (int)blockIdx.x;
    const int split = SPLIT ? (int)blockIdx.x % n_splits : 0;
    const int per_split = SPLIT ? (k + n_splits - 1) / n_splits : k;
    const int i_begin = split * per_split;
    const int i_end = min(k, i_begin + per_split);
    const int head = 16 * wave + i16;
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
        if (tid == 0) sm.n_valid = base;
    }
    __syncthreads();
    const int n_valid = sm.n_valid;
    const int n_tiles = (n_valid + kTile - 1) / kTile;

    // ---- Q^T fragments of this wave's 16 heads (B operand, K = 576 in 18 steps of 32)
    bf16x8 qf[18];
    {
        const uint16_t *qrow = q + ((int64_t)t * h + (head_ok ? head : 0)) * kDk + 8 * G;
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (head_ok) v = *reinterpret_cast<const uint4 *>(qrow + 32 * ks);
            qf[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // ---- tile gather (asynchronous, straight to LDS)
    auto gather = [&](int j, int buf) {
        const int row0 = j * kTile;
        const uint8_t *kvb = reinterpret_cast<const uint8_t *>(kv_cache);
        if constexpr (!FP8) {
            uint8_t *dst = sm.tile[buf];
            for (int ins = wave; ins < kRowC; ins += NW) {   // 73 wave-wide 1 KB copies
                const int c = ins * 64 + lane;
                const int r = c / kRowC, col = c - r * kRowC;
                const int rr = row0 + r < n_valid ? row0 + r : 0;
                const int64_t sl = sm.slots[rr];
                g2lds16(kvb + sl * (kDk * 2) + (col < kRowC - 1 ? col : kRowC - 2) * 16, to_lds(dst + ins * 1024));
            }
        } else {
            uint8_t *dst = sm.f8[buf];
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
    auto expand = [&](int j, int buf) {
        if constexpr (FP8) {
            const int row0 = j * kTile;
            for (int c = tid; c < kTile * kF8RowC; c += NT) {
                const int r = c / kF8RowC, col = c - r * kF8RowC;
                const uint4 v = *reinterpret_cast<const uint4 *>(&sm.f8[buf][r * kDk + col * 16]);
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
                uint4 *d = reinterpret_cast<uint4 *>(&sm.tile[0][r * kRowB + col * 32]);
                d[0] = make_uint4(o8[0], o8[1], o8[2], o8[3]);
                d[1] = make_uint4(o8[4], o8[5], o8[6], o8[7]);
            }
            if (tid < kTile) {
                const int rr = row0 + tid < n_valid ? row0 + tid : 0;
                sm.f8scale[tid] = kv_scale[sm.slots[rr]];
            }
        }
    };

    // O^T accumulators: tile dt holds dims 16 dt + 4 G + i of head `head`
    f32x4 o[32];
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) o[dt] = f32x4{0, 0, 0, 0};
    float m_run = -INFINITY, l_run = 0.0f;
    const float c2 = sm_scale * kLog2e;

    if (n_tiles > 0) gather(0, 0);
    for (int j = 0; j < n_tiles; ++j) {
        const int buf = j & 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();                                  // tile j landed; everyone is done with tile j-1
        if (j + 1 < n_tiles) gather(j + 1, FP8 ? buf ^ 1 : buf ^ 1);
        if constexpr (FP8) {
            expand(j, buf);
            __syncthreads();
        }
        const uint8_t *tile = sm.tile[FP8 ? 0 : buf];

        // S^T = K Q^T : four 16-row subtiles; element i of subtile n is row 16 n + 4 G + i.
        // The 72 (subtile, k-step) fragment loads run kLook steps ahead of their MFMA
        // in a register ring; the scheduling barriers keep that order so the live
        // register set stays bounded (Q^T and O^T already hold 200 VGPRs).
        f32x4 s[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) s[n] = f32x4{0, 0, 0, 0};
        {
            const uint8_t *kbase = tile + i16 * kRowB + 16 * G;
            auto kload = [&](int f) {
                return *reinterpret_cast<const uint4 *>(kbase + (f / 18) * 16 * kRowB + 64 * (f % 18));
            };
            uint4 ring[kLook];
#pragma unroll
            for (int f = 0; f < kLook; ++f) ring[f] = kload(f);
#pragma unroll
            for (int f = 0; f < 72; ++f) {
                const uint4 cur = ring[f % kLook];
                if (f + kLook < 72) ring[f % kLook] = kload(f + kLook);
                s[f / 18] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur), qf[f % 18],
                                                                    s[f / 18], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // online softmax in the exp2 domain (per head = per lane column)
        const int row0 = j * kTile;
        float tmax = -INFINITY;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * n + 4 * G + i;
                float x = s[n][i] * c2;
                if constexpr (FP8) x *= sm.f8scale[r];
                x = (row0 + r < n_valid) ? x : -INFINITY;
                s[n][i] = x;
                tmax = fmaxf(tmax, x);
            }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        float psum = 0.0f;
        bf16x8 pb[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int n = 2 * m + hh;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float p = __builtin_amdgcn_exp2f(s[n][i] - m_use);
                    psum += p;
                    if constexpr (FP8) p *= sm.f8scale[16 * n + 4 * G + i];
                    pb[m][4 * hh + i] = (__bf16)p;
                }
            }
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) o[dt] *= alpha;

        // O^T += V^T P^T; k-step m covers rows {32 m + 4 G + i} u {32 m + 16 + 4 G + i}.
        // Same bounded look-ahead as above over the 64 (k-step, dim-tile) steps.
        {
            const uint8_t *vbase = tile + (4 * G + (i16 >> 2)) * kRowB + 4 * (i16 & 3) * 2;
            auto vload = [&](int f, bf16x4 &lo, bf16x4 &hi) {
                const uint8_t *p = vbase + (f / 32) * 32 * kRowB + 32 * (f % 32);
                lo = lds_tr16(p);
                hi = lds_tr16(p + 16 * kRowB);
            };
            bf16x4 rlo[kLook], rhi[kLook];
#pragma unroll
            for (int f = 0; f < kLook; ++f) vload(f, rlo[f], rhi[f]);
#pragma unroll
            for (int f = 0; f < 64; ++f) {
                const bf16x4 lo = rlo[f % kLook], hi = rhi[f % kLook];
                if (f + kLook < 64) vload(f + kLook, rlo[f % kLook], rhi[f % kLook]);
                const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                o[f % 32] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[f / 32], o[f % 32], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // ---- finish: the four 16-lane groups hold disjoint key subsets of each head
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse_v = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    if (!head_ok) return;
    if constexpr (!SPLIT) {
        uint16_t *orow = out + ((int64_t)t * h + head) * kDv + 4 * G;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[dt][e] * inv);
            *reinterpret_cast<bf16x4 *>(orow + 16 * dt) = v;
        }
        if (lse != nullptr && G == 0) lse[(int64_t)t * h + head] = lse_v;
    } else {
        float *orow = ws_o + (((int64_t)t * n_splits + split) * h + head) * kDv + 4 * G;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt)
            *reinterpret_cast<float4 *>(orow + 16 * dt) =
                make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
        if (G == 0) ws_lse[((int64_t)t * n_splits + split) * h + head] = lse_v;
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
    const int nw = (a.h + 15) / 16;
    switch (nw) {
    case 1: launch_mla_t<1, FP8, SPLIT>(a, n_splits, ws_o, ws_lse, stream); break;
    case 2: launch_mla_t<2, FP8, SPLIT>(a, n_splits, ws_o, ws_lse, stream); break;
    case 4: launch_mla_t<4, FP8, SPLIT>(a, n_splits, ws_o, ws_lse, stream); break;
    default: launch_mla_t<8, FP8, SPLIT>(a, n_splits, ws_o, ws_lse, stream); break;
    }
}

hipError_t launch_mla_prefill(const MlaArgs &a, hipStream_t stream) {
    if (a.fp8) launch_mla_nw<true, false>(a, 1, nullptr, nullptr, stream);
    else launch_mla_nw<false, false>(a, 1, nullptr, nullptr, stream);
    return hipGetLastError();
}

int mla_decode_auto_splits(int32_t n_q, int32_t k) {
    // aim for >= 2 workgroups per CU over 256 CUs, at least 2 tiles per split
    int s = 1;
    while (s < 32 && (int64_t)n_q * s < 512 && k / (2 * s) >= 2 * kTile) s *= 2;
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

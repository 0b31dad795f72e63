/*
 * dsa_oracle.c -- plain, slow, double-precision CPU reference of the
 * DeepSeek Sparse Attention (DSA) hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle the GPU library is
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may build, load or call it; the product path never does.
 * It shares no code, header, table or constant with the GPU library.
 *
 * Sources (cited by page title and section):
 *  - "DeepSeek-V3.2-Exp ... DSA" deployment article (m.nxbn.cn), section 1:
 *    a light FP8 "Lightning Indexer" scores the predecessor tokens of every
 *    query, only the top-k (k = 2048) key/value entries enter attention, and
 *    the main attention cost drops from O(L^2) to O(Lk).  Section 5.1: when
 *    top-k is at least the sequence length, DSA degenerates to dense attention.
 *  - SGLang day-0 DeepSeek-V3.2 announcement (winzheng.jp), "DeepSeek Sparse
 *    Attention" section: FP8 indexer, top-k token selection, a key & key_scale
 *    indexer cache with page size 64, token-level sparse operator with page
 *    size 1.
 *  - SGLang DeepSeek V3.2 usage guide, "attention kernel selection": the
 *    sparse MLA kernels take bf16 q and bf16 (or fp8) kv.
 *  - Context-parallel article (lpqz.cn), section 1: the indexer's relevance is
 *    a reduce-sum over its heads.
 *  Readings where the pages are silent (indexer epilogue = ReLU, per-head
 *  weight, head sum, scales; tie rule; index order; 576/512 latent split)
 *  are listed in the design notes and in each function's comment below.
 *
 * Number formats are decoded from their definitions:
 *  - FP8 E4M3 "fn" (OCP 8-bit floating point specification): 1 sign bit,
 *    4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
 *    subnormal (m/8 * 2^-6); S.1111.111 is NaN; there are no infinities;
 *    the largest finite magnitude is 1.75 * 2^8 = 448.
 *  - bfloat16: the upper 16 bits of an IEEE binary32.
 *
 * Everything is computed in double.  The indexer's head dot products are
 * exact in double (products of two E4M3 values carry at most 8 significant
 * bits and 128 of them sum within 53 bits), so their summation order does not
 * matter.  Rows are independent, so they are spread over OpenMP threads; this
 * changes no result.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_NAN 1      /* a NaN score reached the selection step */
#define ORC_ERR_ARG 2      /* an argument is out of range */

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* OCP E4M3 (fn variant) code -> exact double.  NaN codes return NaN. */
double orc_e4m3_decode(uint8_t code)
{
    int sign = code >> 7;
    int expo = (code >> 3) & 15;
    int mant = code & 7;
    double v;
    if (expo == 15 && mant == 7)
        return NAN;
    if (expo == 0)
        v = ldexp((double)mant / 8.0, -6);          /* subnormal */
    else
        v = ldexp(1.0 + (double)mant / 8.0, expo - 7);
    return sign ? -v : v;
}

/* bfloat16 bits -> exact double. */
double orc_bf16_decode(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* float -> OCP E4M3 code: round to nearest, ties to even mantissa, values
 * beyond the largest finite magnitude saturate to +-448 (the quantizer's
 * "sat" behaviour).  Written as "pick the nearest grid point": the grid
 * spacing in the binade [2^e, 2^(e+1)) is 2^(e-3); below 2^-6 the spacing is
 * the subnormal step 2^-9. */
uint8_t orc_e4m3_encode(float xf)
{
    double x = (double)xf;
    uint8_t sign = 0;
    if (isnan(x))
        return 0x7F;
    if (signbit(x)) {
        sign = 0x80;
        x = -x;
    }
    if (x >= 448.0)
        return sign | 0x7E;
    if (x == 0.0)
        return sign;
    int e;
    frexp(x, &e);               /* x = f * 2^e with f in [0.5, 1) -> binade 2^(e-1) */
    int binade = e - 1;
    if (binade < -6)
        binade = -6;            /* subnormal range shares the 2^-9 step */
    double step = ldexp(1.0, binade - 3);
    double q = x / step;        /* exact: division by a power of two */
    double fl = floor(q);
    double frac = q - fl;
    double n;
    if (frac > 0.5)
        n = fl + 1.0;
    else if (frac < 0.5)
        n = fl;
    else
        n = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;   /* tie: even multiple */
    double r = n * step;        /* nearest grid value, may be 2^(binade+1) */
    if (r >= 448.0)
        return sign | 0x7E;
    if (r == 0.0)
        return sign;
    /* encode r exactly */
    int re;
    frexp(r, &re);
    int rb = re - 1;            /* r in [2^rb, 2^(rb+1)) */
    if (rb < -6) {              /* subnormal: r = m * 2^-9 */
        int m = (int)(r / ldexp(1.0, -9));
        return sign | (uint8_t)m;
    }
    int m = (int)((r / ldexp(1.0, rb) - 1.0) * 8.0);
    return sign | (uint8_t)(((rb + 7) << 3) | m);
}

/* ------------------------------------------------------------------ */
/* Cache-store reference: FP8 latent row quantization                  */
/* ------------------------------------------------------------------ */

/* One latent row of n bf16 values -> n E4M3 codes and one fp32 scale.
 * Reading of the FP8 KV cache ("kv_cache_dtype fp8_e4m3" with a per-token
 * scale): scale = amax / 448 computed in fp32 (amax itself is exact),
 * scale = 1 for an all-zero row, and code_i = E4M3(x_i / scale) with the
 * division done in IEEE fp32. */
void orc_kv_quantize_row(const uint16_t *row_bf16, int n, uint8_t *codes, float *scale_out)
{
    float amax = 0.0f;
    for (int i = 0; i < n; i++) {
        float a = (float)fabs(orc_bf16_decode(row_bf16[i]));
        if (a > amax)
            amax = a;
    }
    volatile float scale = (amax > 0.0f) ? amax / 448.0f : 1.0f;
    for (int i = 0; i < n; i++) {
        volatile float xi = (float)orc_bf16_decode(row_bf16[i]);
        volatile float y = xi / scale;
        codes[i] = orc_e4m3_encode(y);
    }
    *scale_out = scale;
}

void orc_kv_quantize_rows(const uint16_t *rows, int64_t n_rows, int width, uint8_t *codes, float *scales)
{
    for (int64_t r = 0; r < n_rows; r++)
        orc_kv_quantize_row(rows + r * width, width, codes + r * width, scales + r);
}

/* ------------------------------------------------------------------ */
/* O1: Lightning Indexer scores                                        */
/* ------------------------------------------------------------------ */

/* For query t (sequence b = q_seq[t], position p = q_pos[t]) and every
 * predecessor s in [0, p] (inclusive: the token itself is its own
 * predecessor, which keeps the k >= L case equal to dense causal attention):
 *
 *   D_j   = sum_i q[t,j,i] * k[s,i]                 (per indexer head j)
 *   score = q_scale[t] * k_scale[s] * sum_j w[t,j] * max(D_j, 0)
 *
 * q and k are E4M3 codes with one fp32 scale per token (k is one vector per
 * token shared by all indexer heads).  w has one fp32 weight per (query,
 * head); w_ld = 0 means one weight vector shared by all queries.  The double
 * result is rounded once to fp32.  Keys are given in logical order: the row
 * of token s of sequence b is seq_start[b] + s.  Entries s > p of a score row
 * are left untouched. */
int orc_indexer_scores(int n_q, int h_i, int d_i,
                       const uint8_t *q, const float *q_scale,
                       const float *w, int64_t w_ld,
                       const uint8_t *k, const float *k_scale,
                       const int64_t *seq_start, const int32_t *q_seq, const int32_t *q_pos,
                       float *scores, int64_t ld, int n_threads)
{
    if (n_q < 0 || h_i <= 0 || d_i <= 0)
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int t = 0; t < n_q; t++) {
        double *qd = (double *)malloc(sizeof(double) * (size_t)h_i * d_i);
        double *kd = (double *)malloc(sizeof(double) * (size_t)d_i);
        const uint8_t *qt = q + (int64_t)t * h_i * d_i;
        for (int x = 0; x < h_i * d_i; x++)
            qd[x] = orc_e4m3_decode(qt[x]);
        const float *wt = w + (int64_t)t * w_ld;
        int64_t base = seq_start[q_seq[t]];
        for (int64_t s = 0; s <= q_pos[t]; s++) {
            const uint8_t *kr = k + (base + s) * d_i;
            for (int i = 0; i < d_i; i++)
                kd[i] = orc_e4m3_decode(kr[i]);
            double acc = 0.0;
            for (int j = 0; j < h_i; j++) {
                double dj = 0.0;
                for (int i = 0; i < d_i; i++)
                    dj += qd[j * d_i + i] * kd[i];
                if (dj > 0.0)
                    acc += (double)wt[j] * dj;
            }
            scores[(int64_t)t * ld + s] = (float)((double)q_scale[t] * (double)k_scale[base + s] * acc);
        }
        free(qd);
        free(kd);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* O2: top-k selection                                                 */
/* ------------------------------------------------------------------ */

typedef struct {
    float v;
    int32_t s;
} orc_cand;

/* larger score first; equal scores (with -0 == +0) -> lower index first */
static int orc_cand_cmp(const void *a, const void *b)
{
    const orc_cand *x = (const orc_cand *)a, *y = (const orc_cand *)b;
    if (x->v > y->v)
        return -1;
    if (x->v < y->v)
        return 1;
    return (x->s < y->s) ? -1 : (x->s > y->s);
}

static int orc_int_cmp(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* For each row t, the candidates are s in [0, q_pos[t]].  Keep the
 * min(k, q_pos[t] + 1) best under (score descending, index ascending); when a
 * row has no more than k candidates all of them are kept (the dense
 * degeneration).  The kept indices are written in ascending order and the
 * rest of the k slots are -1.  A NaN score is an error. */
int orc_topk(const float *scores, int64_t ld, const int32_t *q_pos, int n_q, int k,
             int32_t *idx, int n_threads)
{
    int err = ORC_OK;
    if (k <= 0)
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int t = 0; t < n_q; t++) {
        int64_t n = (int64_t)q_pos[t] + 1;
        orc_cand *c = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)n);
        int bad = 0;
        for (int64_t s = 0; s < n; s++) {
            float v = scores[(int64_t)t * ld + s];
            if (isnan(v))
                bad = 1;
            c[s].v = (v == 0.0f) ? 0.0f : v;     /* -0 and +0 are the same score */
            c[s].s = (int32_t)s;
        }
        qsort(c, (size_t)n, sizeof(orc_cand), orc_cand_cmp);
        int64_t m = n < k ? n : k;
        int32_t *row = idx + (int64_t)t * k;
        for (int64_t i = 0; i < m; i++)
            row[i] = c[i].s;
        qsort(row, (size_t)m, sizeof(int32_t), orc_int_cmp);
        for (int64_t i = m; i < k; i++)
            row[i] = -1;
        free(c);
        if (bad) {
#pragma omp atomic write
            err = ORC_ERR_NAN;
        }
    }
    return err;
}

/* ------------------------------------------------------------------ */
/* O3: sparse MLA attention over the selected latent rows              */
/* ------------------------------------------------------------------ */

/* Latent row s (after multi-head latent attention's weight absorption) has
 * dk = 576 dims; its first dv = 512 dims are the value.  For query t and
 * head h, over the selected set S_t = { idx[t, i] : idx[t, i] >= 0 }:
 *
 *   l_s  = sm_scale * sum_{d < dk} q[t,h,d] * K[s,d]
 *   m    = max_s l_s,   p_s = exp(l_s - m),   Z = sum_s p_s
 *   out[t,h,:] = sum_s p_s * K[s, :dv] / Z,      lse[t,h] = m + log Z
 *
 * K is bf16 (kv_fp8 == 0: kv holds uint16 bf16 bits) or E4M3 codes times a
 * per-row fp32 scale (kv_fp8 == 1: kv holds uint8 codes, kv_scale the
 * scales).  Rows are in logical order: row of token s of sequence b is
 * seq_start[b] + s.  An empty selection gives out = 0, lse = -inf. */
int orc_sparse_mla(int n_q, int h, int dk, int dv,
                   const uint16_t *q,
                   const void *kv, const float *kv_scale, int kv_fp8,
                   const int64_t *seq_start, const int32_t *q_seq,
                   const int32_t *idx, int k, float sm_scale,
                   double *out, double *lse, int n_threads)
{
    if (n_q < 0 || h <= 0 || dk <= 0 || dv <= 0 || dv > dk || k <= 0)
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int t = 0; t < n_q; t++) {
        const int32_t *sel = idx + (int64_t)t * k;
        int64_t base = seq_start[q_seq[t]];
        int ns = 0;
        for (int i = 0; i < k; i++)
            if (sel[i] >= 0)
                ns++;
        /* decode the selected rows once */
        double *kd = (double *)malloc(sizeof(double) * ((size_t)ns * dk + 1));
        int r = 0;
        for (int i = 0; i < k; i++) {
            if (sel[i] < 0)
                continue;
            int64_t row = base + sel[i];
            for (int d = 0; d < dk; d++) {
                if (kv_fp8)
                    kd[(int64_t)r * dk + d] = orc_e4m3_decode(((const uint8_t *)kv)[row * dk + d]) *
                                              (double)kv_scale[row];
                else
                    kd[(int64_t)r * dk + d] = orc_bf16_decode(((const uint16_t *)kv)[row * dk + d]);
            }
            r++;
        }
        double *qd = (double *)malloc(sizeof(double) * (size_t)dk);
        double *l = (double *)malloc(sizeof(double) * ((size_t)ns + 1));
        for (int hh = 0; hh < h; hh++) {
            double *o = out + ((int64_t)t * h + hh) * dv;
            const uint16_t *qh = q + ((int64_t)t * h + hh) * dk;
            for (int d = 0; d < dk; d++)
                qd[d] = orc_bf16_decode(qh[d]);
            for (int d = 0; d < dv; d++)
                o[d] = 0.0;
            if (ns == 0) {
                if (lse)
                    lse[(int64_t)t * h + hh] = -INFINITY;
                continue;
            }
            double m = -INFINITY;
            for (int i = 0; i < ns; i++) {
                double dot = 0.0;
                for (int d = 0; d < dk; d++)
                    dot += qd[d] * kd[(int64_t)i * dk + d];
                l[i] = (double)sm_scale * dot;
                if (l[i] > m)
                    m = l[i];
            }
            double z = 0.0;
            for (int i = 0; i < ns; i++) {
                double p = exp(l[i] - m);
                z += p;
                for (int d = 0; d < dv; d++)
                    o[d] += p * kd[(int64_t)i * dk + d];
            }
            for (int d = 0; d < dv; d++)
                o[d] /= z;
            if (lse)
                lse[(int64_t)t * h + hh] = m + log(z);
        }
        free(kd);
        free(qd);
        free(l);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* O4: dense causal MLA = O3 with every predecessor selected           */
/* ------------------------------------------------------------------ */

int orc_dense_mla(int n_q, int h, int dk, int dv,
                  const uint16_t *q,
                  const void *kv, const float *kv_scale, int kv_fp8,
                  const int64_t *seq_start, const int32_t *q_seq, const int32_t *q_pos,
                  float sm_scale, double *out, double *lse, int n_threads)
{
    int kmax = 1;
    for (int t = 0; t < n_q; t++)
        if (q_pos[t] + 1 > kmax)
            kmax = q_pos[t] + 1;
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_q * kmax);
    for (int t = 0; t < n_q; t++)
        for (int i = 0; i < kmax; i++)
            idx[(int64_t)t * kmax + i] = (i <= q_pos[t]) ? i : -1;
    int rc = orc_sparse_mla(n_q, h, dk, dv, q, kv, kv_scale, kv_fp8, seq_start, q_seq, idx, kmax,
                            sm_scale, out, lse, n_threads);
    free(idx);
    return rc;
}

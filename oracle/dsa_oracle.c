/*
 * dsa_oracle.c -- plain, slow, CPU reference of the DeepSeek Sparse Attention
 * (DSA) forward path.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the CPU-baseline leg of the benchmark call it; the library never does.
 * It shares no code, header, table or constant with the HIP path.
 *
 * Source: the DeepSeek-V3.2 model documentation page (Transformers),
 * section "DeepSeek Sparse Attention (DSA)":
 *   item 1 (lightning indexer): an index score between each query and all
 *     previous keys; the reference runs it in FP8 behind an orthogonal
 *     Hadamard rotation, which leaves q.k unchanged;
 *   item 2 (fine-grained token selection): each query keeps its top
 *     index_topk tokens and main MLA attention runs only over them (an
 *     additive mask in Transformers, a gather at O(index_topk) per query
 *     with a sparse kernel);
 *   indexer key cache: one head of width index_head_dim per token.
 * The ReLU / weighted head-sum form of the score and the absorbed-latent
 * form of MLA are not written on the page; the readings used here are the
 * plainest ones (score = sum_h w_h * relu(q_h . k); one shared latent row
 * [c_kv | k_rope] serves as key, its first v_dim columns as value).
 *
 * Everything accumulates in double.  Inputs arrive as float32 arrays that
 * hold the exact values the device receives (bf16 and fp32 values are exact
 * in float32; fp8 inputs arrive as codes plus float scales).
 *
 * Query t of sequence b sits at position p = L - T + t, L = min(kv_len[b], Lmax),
 * and may see keys s = 0..p (itself included).
 *
 * Parity pins live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

int orc_num_threads(void) { return omp_get_max_threads(); }

/* Threads of the following parallel loops (timing of the oracle only). */
void orc_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* ------------------------------------------------------------------ */
/* OCP FP8 E4M3FN codec (sign, 4 exponent bits with bias 7, 3 mantissa */
/* bits; no infinities; 0x7F / 0xFF are NaN; largest finite 448).       */
/* ------------------------------------------------------------------ */

double orc_e4m3_decode(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, 1 - 7);        /* subnormal: m/8 * 2^-6 */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Round-to-nearest-even onto the finite e4m3fn grid, saturating at +-448.
 * Done as a plain search of the 127 non-negative finite magnitudes, which
 * increase with the code: find the two neighbours and take the nearer one,
 * the one with the even code on an exact tie. */
uint8_t orc_e4m3_encode(float y)
{
    double a = fabs((double)y);
    uint8_t sign = (signbit(y) ? 0x80 : 0x00);
    if (isnan(y))
        return 0x7F;
    if (a >= 448.0)
        return sign | 0x7E;
    int lo = 0, hi = 0x7E;                        /* decode(lo) <= a < decode(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (orc_e4m3_decode((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - orc_e4m3_decode((uint8_t)lo);
    double dhi = orc_e4m3_decode((uint8_t)hi) - a;
    int c;
    if (dlo < dhi)
        c = lo;
    else if (dhi < dlo)
        c = hi;
    else
        c = (lo % 2 == 0) ? lo : hi;
    return sign | (uint8_t)c;
}

void orc_e4m3_encode_array(long n, const float* y, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (long i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode(y[i]);
}

/* ------------------------------------------------------------------ */
/* Hadamard rotation: H[i][j] = (-1)^popcount(i & j) / sqrt(D) (Sylvester */
/* order, orthonormal), applied as an explicit matrix-vector product.   */
/* ------------------------------------------------------------------ */

static int popcount_u32(uint32_t v)
{
    int n = 0;
    while (v) {
        n += (int)(v & 1u);
        v >>= 1;
    }
    return n;
}

void orc_hadamard_matrix(int D, double* H)
{
    double s = 1.0 / sqrt((double)D);
    for (int i = 0; i < D; ++i)
        for (int j = 0; j < D; ++j)
            H[(size_t)i * D + j] = (popcount_u32((uint32_t)(i & j)) & 1) ? -s : s;
}

/* out[r] = fp32(H x[r]) for each row of length D, with H = S / sqrt(D) and S
 * the +-1 Sylvester matrix: the +-1 product is summed in double, then scaled
 * once by 1/sqrt(D), so the irrational scale is not rounded into every term. */
void orc_rotate(long rows, int D, const float* x, float* out)
{
    const double scale = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        const float* xr = x + (size_t)r * D;
        for (int i = 0; i < D; ++i) {
            double acc = 0.0;
            for (int j = 0; j < D; ++j) {
                int neg = popcount_u32((uint32_t)(i & j)) & 1;
                acc += neg ? -(double)xr[j] : (double)xr[j];
            }
            out[(size_t)r * D + i] = (float)(acc * scale);
        }
    }
}

/* Rotate, then quantise each row to e4m3 with one float scale per row:
 *   x' = fp32(H x);  amax = max |x'_i|;
 *   amax == 0  -> all codes 0, scale 1;
 *   otherwise  r = fp32(448 / amax), y_i = fp32(x'_i * r),
 *              code_i = e4m3(y_i), scale = fp32(amax / 448).
 * A dequantised element is decode(code) * scale. */
void orc_rotate_quant(long rows, int D, const float* x, uint8_t* codes, float* scales)
{
    float* xr = (float*)malloc(sizeof(float) * (size_t)rows * D);
    orc_rotate(rows, D, x, xr);
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        const float* v = xr + (size_t)r * D;
        float amax = 0.0f;
        for (int i = 0; i < D; ++i) {
            float a = fabsf(v[i]);
            if (a > amax)
                amax = a;
        }
        if (amax == 0.0f) {
            for (int i = 0; i < D; ++i)
                codes[(size_t)r * D + i] = 0;
            scales[r] = 1.0f;
            continue;
        }
        float rcp = (float)(448.0 / (double)amax);   /* correctly rounded fp32 quotient */
        for (int i = 0; i < D; ++i) {
            float y = v[i] * rcp;                     /* fp32 product */
            codes[(size_t)r * D + i] = orc_e4m3_encode(y);
        }
        scales[r] = (float)((double)amax / 448.0);
    }
    free(xr);
}

/* The same per-row e4m3 quantisation without the rotation, for the MLA
 * latent cache and queries when the attention runs on fp8 codes.  The value
 * columns of a latent row must stay in the latent basis, so no rotation is
 * applied; every other step is the one of orc_rotate_quant. */
void orc_quant(long rows, int D, const float* x, uint8_t* codes, float* scales)
{
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        const float* v = x + (size_t)r * D;
        float amax = 0.0f;
        for (int i = 0; i < D; ++i) {
            float a = fabsf(v[i]);
            if (a > amax)
                amax = a;
        }
        if (amax == 0.0f) {
            for (int i = 0; i < D; ++i)
                codes[(size_t)r * D + i] = 0;
            scales[r] = 1.0f;
            continue;
        }
        float rcp = (float)(448.0 / (double)amax);
        for (int i = 0; i < D; ++i)
            codes[(size_t)r * D + i] = orc_e4m3_encode(v[i] * rcp);
        scales[r] = (float)((double)amax / 448.0);
    }
}

/* ------------------------------------------------------------------ */
/* Row lists.  A "row" is one query (b, t), numbered r = b * T + t; the  */
/* i-th listed row is rows[i] (rows == NULL lists every row in order).  */
/* With compact != 0 the per-query inputs (q, w, codes, scales) hold     */
/* only the listed rows, the i-th listed row at index i; keys, values and */
/* kv_len are always whole.                                             */
/* ------------------------------------------------------------------ */

static long row_at(long i, const long* rows) { return rows ? rows[i] : i; }

/* A sequence's length as the path reads it: kv_len[b] clamped to the cache
 * capacity Lmax (a length past the cache cannot have cached keys), so a query
 * never sees a position outside its sequence's cache rows. */
static long seq_len(int kv_len, int Lmax) { return kv_len < Lmax ? (long)kv_len : (long)Lmax; }

/* Lightning-indexer scores for the listed rows.
 *   q  [B, T, H, D]   w [B, T, H]   k [B, Lmax, D]   kv_len [B]
 *   out [n_rows, Lmax]: I[s] = sum_h w[h] * max(0, q[h] . k[s]) for s <= p,
 *   -inf for s > p.  Accumulated in double, stored as fp32. */
void orc_index_scores(int B, int T, int Lmax, int H, int D,
                      const float* q, const float* w, const float* k,
                      const int* kv_len, long n_rows, const long* rows, int compact, float* out)
{
    (void)B;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < n_rows; ++i) {
        long r = row_at(i, rows);
        long b = r / T, t = r % T;
        long p = seq_len(kv_len[b], Lmax) - T + t;
        long qi = compact ? i : r;
        const float* qr = q + (size_t)qi * H * D;
        const float* wr = w + (size_t)qi * H;
        const float* kb = k + (size_t)b * Lmax * D;
        float* o = out + (size_t)i * Lmax;
        for (long s = 0; s < Lmax; ++s) {
            if (s > p) {
                o[s] = -INFINITY;
                continue;
            }
            double I = 0.0;
            for (int h = 0; h < H; ++h) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += (double)qr[(size_t)h * D + d] * (double)kb[(size_t)s * D + d];
                if (dot > 0.0)
                    I += (double)wr[h] * dot;
            }
            o[s] = (float)I;
        }
    }
}

/* The same scores on fp8 operands: q and k are their dequantised values
 * decode(code) * scale (q: one scale per (token, head) row; k: one scale per
 * token row). */
void orc_index_scores_fp8(int B, int T, int Lmax, int H, int D,
                          const uint8_t* qc, const float* qs, const float* w,
                          const uint8_t* kc, const float* ks,
                          const int* kv_len, long n_rows, const long* rows, int compact, float* out)
{
    (void)B;
    double table[256];
    for (int c = 0; c < 256; ++c)
        table[c] = orc_e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < n_rows; ++i) {
        long r = row_at(i, rows);
        long b = r / T, t = r % T;
        long p = seq_len(kv_len[b], Lmax) - T + t;
        long qi = compact ? i : r;
        double* qd = (double*)malloc(sizeof(double) * (size_t)H * D);
        for (int h = 0; h < H; ++h)
            for (int d = 0; d < D; ++d)
                qd[(size_t)h * D + d] = table[qc[((size_t)qi * H + h) * D + d]] * (double)qs[(size_t)qi * H + h];
        const float* wr = w + (size_t)qi * H;
        float* o = out + (size_t)i * Lmax;
        for (long s = 0; s < Lmax; ++s) {
            if (s > p) {
                o[s] = -INFINITY;
                continue;
            }
            const uint8_t* kr = kc + ((size_t)b * Lmax + s) * D;
            double ksc = (double)ks[(size_t)b * Lmax + s];
            double I = 0.0;
            for (int h = 0; h < H; ++h) {
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += qd[(size_t)h * D + d] * (table[kr[d]] * ksc);
                if (dot > 0.0)
                    I += (double)wr[h] * dot;
            }
            o[s] = (float)I;
        }
        free(qd);
    }
}

/* ------------------------------------------------------------------ */
/* Top-k: keep k_eff = min(K, p + 1) of the candidates s = 0..p, ordered */
/* by (score descending, index ascending); pad with -1.                 */
/* ------------------------------------------------------------------ */

typedef struct {
    float v;
    int s;
} cand_t;

static int cand_cmp(const void* a, const void* b)
{
    const cand_t* x = (const cand_t*)a;
    const cand_t* y = (const cand_t*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->s < y->s) ? -1 : (x->s > y->s);
}

/* scores [n_rows, Lmax] (row i belongs to query rows[i]); idx [n_rows, K]. */
void orc_topk(int B, int T, int Lmax, int K, const int* kv_len,
              long n_rows, const long* rows, const float* scores, int* idx)
{
    (void)B;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < n_rows; ++i) {
        long r = row_at(i, rows);
        long b = r / T, t = r % T;
        long p = seq_len(kv_len[b], Lmax) - T + t;
        long n = p + 1 > 0 ? p + 1 : 0; /* p < 0: no candidates */
        long keff = n < K ? n : K;
        cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
        for (long s = 0; s < n; ++s) {
            c[s].v = scores[(size_t)i * Lmax + s];
            c[s].s = (int)s;
        }
        qsort(c, (size_t)n, sizeof(cand_t), cand_cmp);
        for (long j = 0; j < K; ++j)
            idx[(size_t)i * K + j] = (j < keff) ? c[j].s : -1;
        free(c);
    }
}

/* ------------------------------------------------------------------ */
/* Sparse absorbed MLA over a selected index set.                        */
/*   q [B, T, H, Dqk]; kv [B, Lmax, Dqk] (key = the whole row, value =   */
/*   its first Dv columns); idx [n_rows, K] with -1 entries skipped.     */
/*   z_j = sm_scale * q . kv[idx_j];  o = sum_j softmax(z)_j kv[idx_j,:Dv]; */
/*   lse = log sum_j exp z_j.  A row with no valid entry gives o = 0,     */
/*   lse = -inf.                                                          */
/* ------------------------------------------------------------------ */

void orc_sparse_mla(int B, int T, int Lmax, int H, int Dqk, int Dv, int K, double sm_scale,
                    const float* q, const float* kv, long n_rows, const long* rows, int compact,
                    const int* idx, double* out, double* lse)
{
    (void)B;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < n_rows; ++i) {
        long r = row_at(i, rows);
        long b = r / T;
        const int* ir = idx + (size_t)i * K;
        const float* kvb = kv + (size_t)b * Lmax * Dqk;
        double* z = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        for (int h = 0; h < H; ++h) {
            const float* qh = q + ((size_t)(compact ? i : r) * H + h) * Dqk;
            double* o = out + ((size_t)i * H + h) * Dv;
            double m = -INFINITY;
            for (int j = 0; j < K; ++j) {
                if (ir[j] < 0) continue;
                const float* row = kvb + (size_t)ir[j] * Dqk;
                double dot = 0.0;
                for (int d = 0; d < Dqk; ++d)
                    dot += (double)qh[d] * (double)row[d];
                z[j] = sm_scale * dot;
                if (z[j] > m) m = z[j];
            }
            for (int e = 0; e < Dv; ++e)
                o[e] = 0.0;
            if (m == -INFINITY) {
                lse[(size_t)i * H + h] = -INFINITY;
                continue;
            }
            double Z = 0.0;
            for (int j = 0; j < K; ++j) {
                if (ir[j] < 0) continue;
                double pj = exp(z[j] - m);
                Z += pj;
                const float* row = kvb + (size_t)ir[j] * Dqk;
                for (int e = 0; e < Dv; ++e)
                    o[e] += pj * (double)row[e];
            }
            for (int e = 0; e < Dv; ++e)
                o[e] /= Z;
            lse[(size_t)i * H + h] = m + log(Z);
        }
        free(z);
    }
}

/* Backward of the sparse MLA.  The page calls DSA trainable; for the loss
 * L = sum over the listed rows, heads and value dims of dO * O it returns the
 * gradients with respect to q and kv.  With z_j = sm q . k_j over the listed
 * entries j (k_j = row idx_j, v_j its first Dv columns), p = softmax(z) and
 * O = sum_j p_j v_j:
 *   dP_j = dO . v_j,   D = dO . O,   dz_j = p_j (dP_j - D),
 *   dq   = sm sum_j dz_j k_j,
 *   dkv[idx_j] += sm dz_j q  (all Dqk columns)  +  p_j dO  (first Dv columns);
 * an index listed twice contributes twice.  dq [n_rows, H, Dqk]; dkv
 * [B, Lmax, Dqk] is accumulated into (the caller zeroes it). */
void orc_sparse_mla_bwd(int B, int T, int Lmax, int H, int Dqk, int Dv, int K, double sm,
                        const float* q, const float* kv, const float* dout, long n_rows, const long* rows,
                        int compact, const int* idx, double* dq, double* dkv)
{
    (void)B;
#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double* pr = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double* o = (double*)malloc(sizeof(double) * (size_t)Dv);
        double* g = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * Dqk);
#pragma omp for schedule(dynamic, 1)
        for (long i = 0; i < n_rows; ++i) {
            long r = row_at(i, rows);
            long b = r / T;
            const int* ir = idx + (size_t)i * K;
            const float* kvb = kv + (size_t)b * Lmax * Dqk;
            for (size_t u = 0; u < (size_t)K * Dqk; ++u)
                g[u] = 0.0;
            for (int h = 0; h < H; ++h) {
                const size_t qi = (size_t)(compact ? i : r) * H + h;
                const float* qh = q + qi * Dqk;
                const float* doh = dout + qi * Dv;
                double* dqh = dq + ((size_t)i * H + h) * Dqk;
                for (int d = 0; d < Dqk; ++d)
                    dqh[d] = 0.0;
                double m = -INFINITY;
                for (int j = 0; j < K; ++j) {
                    if (ir[j] < 0) continue;
                    const float* row = kvb + (size_t)ir[j] * Dqk;
                    double dot = 0.0;
                    for (int d = 0; d < Dqk; ++d)
                        dot += (double)qh[d] * (double)row[d];
                    z[j] = sm * dot;
                    if (z[j] > m) m = z[j];
                }
                if (m == -INFINITY) continue;
                double Z = 0.0;
                for (int j = 0; j < K; ++j) {
                    if (ir[j] < 0) continue;
                    pr[j] = exp(z[j] - m);
                    Z += pr[j];
                }
                for (int e = 0; e < Dv; ++e)
                    o[e] = 0.0;
                for (int j = 0; j < K; ++j) {
                    if (ir[j] < 0) continue;
                    pr[j] /= Z;
                    const float* row = kvb + (size_t)ir[j] * Dqk;
                    for (int e = 0; e < Dv; ++e)
                        o[e] += pr[j] * (double)row[e];
                }
                double Dsum = 0.0;
                for (int e = 0; e < Dv; ++e)
                    Dsum += (double)doh[e] * o[e];
                for (int j = 0; j < K; ++j) {
                    if (ir[j] < 0) continue;
                    const float* row = kvb + (size_t)ir[j] * Dqk;
                    double dp = 0.0;
                    for (int e = 0; e < Dv; ++e)
                        dp += (double)doh[e] * (double)row[e];
                    const double dz = pr[j] * (dp - Dsum);
                    double* gj = g + (size_t)j * Dqk;
                    for (int d = 0; d < Dqk; ++d) {
                        dqh[d] += sm * dz * (double)row[d];
                        gj[d] += sm * dz * (double)qh[d];
                    }
                    for (int e = 0; e < Dv; ++e)
                        gj[e] += pr[j] * (double)doh[e];
                }
            }
#pragma omp critical
            for (int j = 0; j < K; ++j) {
                if (ir[j] < 0) continue;
                double* dst = dkv + ((size_t)b * Lmax + ir[j]) * Dqk;
                const double* gj = g + (size_t)j * Dqk;
                for (int d = 0; d < Dqk; ++d)
                    dst[d] += gj[d];
            }
        }
        free(z);
        free(pr);
        free(o);
        free(g);
    }
}

/* Second formulation (the additive-mask form): dense logits over every
 * s = 0..p, plus a mask that is 0 on the selected s and -inf elsewhere,
 * then a softmax over all of them.  Must agree with orc_sparse_mla. */
void orc_masked_dense_mla(int B, int T, int Lmax, int H, int Dqk, int Dv, int K, double sm_scale,
                          const float* q, const float* kv, const int* kv_len,
                          long n_rows, const long* rows, int compact, const int* idx,
                          double* out, double* lse)
{
    (void)B;
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < n_rows; ++i) {
        long r = row_at(i, rows);
        long b = r / T, t = r % T;
        long p = seq_len(kv_len[b], Lmax) - T + t;
        long n = p + 1 > 0 ? p + 1 : 0; /* p < 0: no candidates */
        const int* ir = idx + (size_t)i * K;
        const float* kvb = kv + (size_t)b * Lmax * Dqk;
        double* mask = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        double* z = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        for (long s = 0; s < n; ++s)
            mask[s] = -INFINITY;
        for (int j = 0; j < K; ++j)
            if (ir[j] >= 0 && ir[j] < n)
                mask[ir[j]] = 0.0;
        for (int h = 0; h < H; ++h) {
            const float* qh = q + ((size_t)(compact ? i : r) * H + h) * Dqk;
            double* o = out + ((size_t)i * H + h) * Dv;
            double m = -INFINITY;
            for (long s = 0; s < n; ++s) {
                const float* row = kvb + (size_t)s * Dqk;
                double dot = 0.0;
                for (int d = 0; d < Dqk; ++d)
                    dot += (double)qh[d] * (double)row[d];
                z[s] = sm_scale * dot + mask[s];
                if (z[s] > m) m = z[s];
            }
            for (int e = 0; e < Dv; ++e)
                o[e] = 0.0;
            if (m == -INFINITY) {
                lse[(size_t)i * H + h] = -INFINITY;
                continue;
            }
            double Z = 0.0;
            for (long s = 0; s < n; ++s) {
                double ps = exp(z[s] - m);
                Z += ps;
                const float* row = kvb + (size_t)s * Dqk;
                for (int e = 0; e < Dv; ++e)
                    o[e] += ps * (double)row[e];
            }
            for (int e = 0; e < Dv; ++e)
                o[e] /= Z;
            lse[(size_t)i * H + h] = m + log(Z);
        }
        free(mask);
        free(z);
    }
}

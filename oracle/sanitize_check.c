/*
 * sanitize_check.c -- drives every entry point of dsa_oracle.c through its edge
 * cases.  TEST INFRASTRUCTURE ONLY: tests/test_oracle_sanitize.py builds it
 * together with dsa_oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer and fails on any report or a non-zero exit.
 *
 * The cases are the shapes the DSA path meets at its edges (DeepSeek-V3.2 model
 * documentation, "DeepSeek Sparse Attention (DSA)", items 1 and 2): sequences
 * shorter than their query block (a query before the start of the cache),
 * empty sequences, lengths past the cache capacity, fewer candidates than
 * index_topk, index lists with skipped, repeated and all-skipped entries, zero
 * rows for the fp8 codec, and every codec special value.
 *
 * The prototypes are declared here (the oracle has no header); inputs come from
 * a fixed linear congruential generator.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_e4m3_decode(uint8_t c);
uint8_t orc_e4m3_encode(float y);
void orc_e4m3_encode_array(long n, const float* y, uint8_t* out);
void orc_hadamard_matrix(int D, double* H);
void orc_rotate(long rows, int D, const float* x, float* out);
void orc_rotate_quant(long rows, int D, const float* x, uint8_t* codes, float* scales);
void orc_quant(long rows, int D, const float* x, uint8_t* codes, float* scales);
void orc_index_scores(int B, int T, int Lmax, int H, int D, const float* q, const float* w, const float* k,
                      const int* kv_len, long n_rows, const long* rows, int compact, float* out);
void orc_index_scores_fp8(int B, int T, int Lmax, int H, int D, const uint8_t* qc, const float* qs, const float* w,
                          const uint8_t* kc, const float* ks, const int* kv_len, long n_rows, const long* rows,
                          int compact, float* out);
void orc_topk(int B, int T, int Lmax, int K, const int* kv_len, long n_rows, const long* rows, const float* scores,
              int* idx);
void orc_sparse_mla(int B, int T, int Lmax, int H, int Dqk, int Dv, int K, double sm_scale, const float* q,
                    const float* kv, long n_rows, const long* rows, int compact, const int* idx, double* out,
                    double* lse);
void orc_sparse_mla_bwd(int B, int T, int Lmax, int H, int Dqk, int Dv, int K, double sm, const float* q,
                        const float* kv, const float* dout, long n_rows, const long* rows, int compact,
                        const int* idx, double* dq, double* dkv);
void orc_masked_dense_mla(int B, int T, int Lmax, int H, int Dqk, int Dv, int K, double sm_scale, const float* q,
                          const float* kv, const int* kv_len, long n_rows, const long* rows, int compact,
                          const int* idx, double* out, double* lse);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static float next_unit(void)
{
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((double)(g_state >> 40) / (double)(1ull << 24)) * 2.0f - 1.0f;
}

static float* rand_f32(size_t n)
{
    float* p = (float*)malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i)
        p[i] = next_unit();
    return p;
}

static int g_fail = 0;

static void expect(int ok, const char* what)
{
    if (!ok) {
        fprintf(stderr, "check failed: %s\n", what);
        g_fail = 1;
    }
}

static void codec_cases(void)
{
    for (int c = 0; c < 256; ++c) {
        double v = orc_e4m3_decode((uint8_t)c);
        if (c != 0x7F && c != 0xFF)
            expect(orc_e4m3_encode((float)v) == (uint8_t)c || (c == 0x80 && orc_e4m3_encode((float)v) == 0x80),
                   "e4m3 round trip");
    }
    const float specials[] = {0.0f, -0.0f, NAN, INFINITY, -INFINITY, 1e30f, -1e30f, 448.0f, 449.0f,
                              1e-45f, -1e-45f, 1.0625f, 1.1875f};
    uint8_t out[sizeof(specials) / sizeof(specials[0])];
    orc_e4m3_encode_array((long)(sizeof(specials) / sizeof(specials[0])), specials, out);
    expect(out[3] == 0x7E && out[4] == 0xFE, "saturation of infinities");
}

static void rotation_cases(void)
{
    for (int D = 2; D <= 256; D *= 2) {
        double* Hm = (double*)malloc(sizeof(double) * (size_t)D * D);
        orc_hadamard_matrix(D, Hm);
        free(Hm);
    }
    for (int D = 16; D <= 256; D *= 2) {
        const long rows = 5;
        float* x = rand_f32((size_t)rows * D);
        memset(x + D, 0, sizeof(float) * (size_t)D); /* a zero row */
        float* xr = (float*)malloc(sizeof(float) * (size_t)rows * D);
        uint8_t* codes = (uint8_t*)malloc((size_t)rows * D);
        float* sc = (float*)malloc(sizeof(float) * (size_t)rows);
        orc_rotate(rows, D, x, xr);
        orc_rotate_quant(rows, D, x, codes, sc);
        expect(sc[1] == 1.0f, "zero row scale");
        free(x);
        free(xr);
        free(codes);
        free(sc);
    }
    for (int D = 16; D <= 1024; D += 16 * 7) {
        const long rows = 3;
        float* x = rand_f32((size_t)rows * D);
        memset(x, 0, sizeof(float) * (size_t)D);
        uint8_t* codes = (uint8_t*)malloc((size_t)rows * D);
        float* sc = (float*)malloc(sizeof(float) * (size_t)rows);
        orc_quant(rows, D, x, codes, sc);
        free(x);
        free(codes);
        free(sc);
    }
}

/* Sequences: full, shorter than T (queries before position 0), empty, longer than
 * the cache (clamped to it), and one exactly T long. */
enum { B = 5, T = 4, LMAX = 9, H = 3, D = 16, K1 = 16, K2 = 3 };
static const int kv_len[B] = {9, 2, 0, 14, 4};

static void indexer_topk_cases(void)
{
    const long n_all = (long)B * T;
    float* q = rand_f32((size_t)n_all * H * D);
    float* w = rand_f32((size_t)n_all * H);
    float* k = rand_f32((size_t)B * LMAX * D);
    float* sc = (float*)malloc(sizeof(float) * (size_t)n_all * LMAX);
    orc_index_scores(B, T, LMAX, H, D, q, w, k, kv_len, n_all, NULL, 0, sc);
    for (long r = 0; r < n_all; ++r) {
        long b = r / T, t = r % T;
        long L = kv_len[b] < LMAX ? kv_len[b] : LMAX;
        long p = L - T + t;
        for (long s = 0; s < LMAX; ++s)
            expect((s <= p) == isfinite(sc[(size_t)r * LMAX + s]), "causal -inf pattern");
    }
    /* a row subset in compact form */
    const long rows[3] = {19, 2, 8};
    float* qc = (float*)malloc(sizeof(float) * 3 * H * D);
    float* wc = (float*)malloc(sizeof(float) * 3 * H);
    for (int i = 0; i < 3; ++i) {
        memcpy(qc + (size_t)i * H * D, q + (size_t)rows[i] * H * D, sizeof(float) * H * D);
        memcpy(wc + (size_t)i * H, w + (size_t)rows[i] * H, sizeof(float) * H);
    }
    float* sc3 = (float*)malloc(sizeof(float) * 3 * LMAX);
    orc_index_scores(B, T, LMAX, H, D, qc, wc, k, kv_len, 3, rows, 1, sc3);
    for (int i = 0; i < 3; ++i)
        expect(memcmp(sc3 + (size_t)i * LMAX, sc + (size_t)rows[i] * LMAX, sizeof(float) * LMAX) == 0,
               "compact rows equal full rows");

    /* the fp8 variant on codes and scales of the same shapes */
    uint8_t* qcode = (uint8_t*)malloc((size_t)n_all * H * D);
    float* qs = (float*)malloc(sizeof(float) * (size_t)n_all * H);
    uint8_t* kcode = (uint8_t*)malloc((size_t)B * LMAX * D);
    float* ks = (float*)malloc(sizeof(float) * (size_t)B * LMAX);
    orc_rotate_quant(n_all * H, D, q, qcode, qs);
    orc_rotate_quant((long)B * LMAX, D, k, kcode, ks);
    float* sc8 = (float*)malloc(sizeof(float) * (size_t)n_all * LMAX);
    orc_index_scores_fp8(B, T, LMAX, H, D, qcode, qs, w, kcode, ks, kv_len, n_all, NULL, 0, sc8);

    /* top-k with more slots than candidates, and with fewer */
    for (int pass = 0; pass < 2; ++pass) {
        const int K = pass ? K2 : K1;
        int* idx = (int*)malloc(sizeof(int) * (size_t)n_all * K);
        orc_topk(B, T, LMAX, K, kv_len, n_all, NULL, pass ? sc8 : sc, idx);
        for (long r = 0; r < n_all; ++r) {
            long b = r / T, t = r % T;
            long L = kv_len[b] < LMAX ? kv_len[b] : LMAX;
            long p = L - T + t;
            long keff = p + 1 < 0 ? 0 : (p + 1 < K ? p + 1 : K);
            for (int j = 0; j < K; ++j) {
                int v = idx[(size_t)r * K + j];
                expect(j < keff ? (v >= 0 && v <= p) : v == -1, "top-k entries and padding");
            }
        }
        free(idx);
    }
    free(q);
    free(w);
    free(k);
    free(sc);
    free(qc);
    free(wc);
    free(sc3);
    free(qcode);
    free(qs);
    free(kcode);
    free(ks);
    free(sc8);
}

static void mla_cases(void)
{
    enum { HM = 2, DQK = 32, DV = 16, K = 5 };
    const long n_all = (long)B * T;
    float* q = rand_f32((size_t)n_all * HM * DQK);
    float* kv = rand_f32((size_t)B * LMAX * DQK);
    float* dout = rand_f32((size_t)n_all * HM * DV);
    int idx[B * T * K];
    for (long r = 0; r < n_all; ++r) {
        for (int j = 0; j < K; ++j)
            idx[r * K + j] = (int)((r * 7 + j * 3) % LMAX);
        idx[r * K + 1] = -1;               /* skipped */
        idx[r * K + 2] = idx[r * K + 0];   /* listed twice */
    }
    for (int j = 0; j < K; ++j)
        idx[3 * K + j] = -1;               /* a row with nothing to attend */
    double* out = (double*)malloc(sizeof(double) * (size_t)n_all * HM * DV);
    double* lse = (double*)malloc(sizeof(double) * (size_t)n_all * HM);
    orc_sparse_mla(B, T, LMAX, HM, DQK, DV, K, 0.25, q, kv, n_all, NULL, 0, idx, out, lse);
    expect(isinf(lse[3 * HM]) && lse[3 * HM] < 0, "empty row lse");
    double* out2 = (double*)malloc(sizeof(double) * (size_t)n_all * HM * DV);
    double* lse2 = (double*)malloc(sizeof(double) * (size_t)n_all * HM);
    orc_masked_dense_mla(B, T, LMAX, HM, DQK, DV, K, 0.25, q, kv, kv_len, n_all, NULL, 0, idx, out2, lse2);
    double* dq = (double*)malloc(sizeof(double) * (size_t)n_all * HM * DQK);
    double* dkv = (double*)calloc((size_t)B * LMAX * DQK, sizeof(double));
    orc_sparse_mla_bwd(B, T, LMAX, HM, DQK, DV, K, 0.25, q, kv, dout, n_all, NULL, 0, idx, dq, dkv);
    /* K = 1 and a compact subset */
    const long rows[2] = {5, 0};
    int idx1[2] = {3, -1};
    float qc[2 * HM * DQK];
    memcpy(qc, q + 5 * HM * DQK, sizeof(float) * HM * DQK);
    memcpy(qc + HM * DQK, q, sizeof(float) * HM * DQK);
    orc_sparse_mla(B, T, LMAX, HM, DQK, DV, 1, 0.5, qc, kv, 2, rows, 1, idx1, out, lse);
    free(q);
    free(kv);
    free(dout);
    free(out);
    free(lse);
    free(out2);
    free(lse2);
    free(dq);
    free(dkv);
}

int main(void)
{
    codec_cases();
    rotation_cases();
    indexer_topk_cases();
    mla_cases();
    if (g_fail)
        return 1;
    printf("sanitize_check: all oracle entry points ran\n");
    return 0;
}

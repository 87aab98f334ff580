/* Address / undefined-behaviour sanitizer driver of the CPU oracle
 * (oracle/flo_oracle.c): every function on small seeded inputs, including
 * the edge cases the tests pin (one row, a single column, all-equal keys,
 * signed zeros, zero groups, every code width, both quantisers, sparse and
 * dense attention, pruned-column caches, column statistics).  Built with
 * -fsanitize=address,undefined by tests/test_sanitize_cpu.py; any report
 * aborts the run.  Exit 0 = no finding. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int flo_active_count(double rho, int N, int n_prev);
void flo_delta_norm(const float*, const float*, int, const int*, int, float*);
void flo_delta_norm_rel(const float*, const float*, int, const int*, int, float*);
int flo_top_select(const float*, const int*, int, int, int*);
int flo_select_columns(const float*, const int*, int, int, int, int, int*);
void flo_quant_group(const float*, int, int, int8_t*, float*);
void flo_quantize_rows(const float*, const float*, long, int, int, int, int, int8_t*, float*,
                       float*, float*);
void flo_pack_codes(const int8_t*, long, int, uint8_t*);
void flo_quant_asym_group(const float*, int, long, int, uint8_t*, long, float*, float*);
void flo_quantize_rows_asym(const float*, const float*, long, int, int, int, int, int, uint8_t*,
                            float*, float*, float*);
void flo_attend(int, int, int, float, const float*, const float*, const float*, const int*, int,
                const int*, int, const float*, const float*, float*, float*);
void flo_unselected_cache(int, int, int, float, const float*, const float*, const float*,
                          const int*, int, const int*, int, const int*, int, const float*,
                          const float*, const float*, float*, float*);
void flo_column_stats(int, int, int, float, const float*, const float*, const int*, int,
                      const int*, int, const float*, const float*, const float*, float*);

static uint64_t rs = 88172645463325252ull;
static float rnd(void) { /* xorshift64, uniform in [-1, 1) */
    rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17;
    return (float)((rs >> 11) * (1.0 / 9007199254740992.0)) * 2.0f - 1.0f;
}
static float* vec(long n, float scale) {
    float* x = malloc((size_t)n * sizeof(float));
    for (long i = 0; i < n; ++i) x[i] = rnd() * scale;
    return x;
}
static int fails = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "FAILED %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

static void case_attention(int N, int H, int d, int k, int n_sink) {
    const float sm = 1.0f / sqrtf((float)d);
    float *q = vec((long)N * H * d, 1.0f), *kh = vec((long)N * H * d, 1.0f), *vh = vec((long)N * H * d, 1.0f);
    int* rows = malloc(sizeof(int) * N);
    int n = 0;
    for (int i = 0; i < N; i += 2) rows[n++] = i;                /* every other row */
    float *out = malloc(sizeof(float) * (size_t)N * H * d), *lse = malloc(sizeof(float) * (size_t)N * H);
    flo_attend(N, H, d, sm, q, kh, vh, NULL, N, NULL, N, NULL, NULL, out, lse);  /* dense */
    for (long t = 0; t < (long)N * H; ++t) EXPECT(isfinite(lse[t]));
    float* cs = malloc(sizeof(float) * (size_t)H * N);
    flo_column_stats(N, H, d, sm, q, kh, NULL, N, NULL, N, lse, NULL, vh, cs);
    /* column selection, the pruned-column caches and a sparse loop */
    int kk = k < N ? k : N;
    int* sel = malloc(sizeof(int) * (size_t)H * kk);
    EXPECT(flo_select_columns(cs, NULL, H, N, n_sink, kk, sel) == 0);
    for (int h = 0; h < H; ++h)
        for (int p = 1; p < kk; ++p) EXPECT(sel[h * kk + p] > sel[h * kk + p - 1]);
    float *lse_r = malloc(sizeof(float) * (size_t)n * H), *mu = malloc(sizeof(float) * (size_t)n * H);
    float* ou = malloc(sizeof(float) * (size_t)n * H * d);
    for (int t = 0; t < n; ++t)
        for (int h = 0; h < H; ++h) lse_r[t * H + h] = lse[(long)rows[t] * H + h];
    flo_unselected_cache(N, H, d, sm, q, kh, vh, rows, n, NULL, N, sel, kk, lse_r, NULL, NULL, mu, ou);
    float *o2 = malloc(sizeof(float) * (size_t)n * H * d), *l2 = malloc(sizeof(float) * (size_t)n * H);
    flo_attend(N, H, d, sm, q, kh, vh, rows, n, sel, kk, mu, ou, o2, l2);
    float* c2 = malloc(sizeof(float) * (size_t)H * kk);
    flo_column_stats(N, H, d, sm, q, kh, rows, n, sel, kk, l2, mu, NULL, c2);
    /* a further pruning from the sparse selection */
    int k3 = kk > n_sink + 1 ? kk - 1 : kk;
    int* sel3 = malloc(sizeof(int) * (size_t)H * k3);
    EXPECT(flo_select_columns(c2, sel, H, kk, n_sink, k3, sel3) == 0);
    float *mu3 = malloc(sizeof(float) * (size_t)n * H), *ou3 = malloc(sizeof(float) * (size_t)n * H * d);
    flo_unselected_cache(N, H, d, sm, q, kh, vh, rows, n, sel, kk, sel3, k3, l2, mu, ou, mu3, ou3);
    free(q); free(kh); free(vh); free(rows); free(out); free(lse); free(cs); free(sel); free(lse_r);
    free(mu); free(ou); free(o2); free(l2); free(c2); free(sel3); free(mu3); free(ou3);
}

int main(void) {
    /* counts */
    EXPECT(flo_active_count(0.4, 32768, 32768) == 13108);
    EXPECT(flo_active_count(0.0, 10, 10) == 1);
    /* statistics and selection, including ties, signed zeros and one row */
    int N = 37, D = 24;
    float *h0 = vec((long)N * D, 1.0f), *h1 = vec((long)N * D, 1.0f), st[64];
    int cand[40], act[40];
    for (int i = 0; i < N; ++i) cand[i] = i;
    flo_delta_norm(h1, h0, D, NULL, N, st);
    flo_delta_norm_rel(h1, h0, D, cand, N, st);
    memset(h0, 0, sizeof(float) * D);                              /* a zero previous state */
    flo_delta_norm_rel(h1, h0, D, cand, 1, st);
    EXPECT(isinf(st[0]));
    for (int i = 0; i < N; ++i) st[i] = (i % 3) ? 0.0f : -0.0f;    /* all equal */
    EXPECT(flo_top_select(st, cand, N, 5, act) == 0);
    for (int i = 0; i < 5; ++i) EXPECT(act[i] == i);
    EXPECT(flo_top_select(st, NULL, 1, 1, act) == 0 && act[0] == 0);
    st[3] = NAN;
    EXPECT(flo_top_select(st, NULL, N, 5, act) != 0);
    /* quantisers: every width, zero groups, both schemes */
    const int bits_list[4] = {2, 4, 8, 32};
    for (int bi = 0; bi < 4; ++bi) {
        int b = bits_list[bi], n = 9, H = 2, d = 64, g = 32;
        long m = (long)n * H * d;
        float *x = vec(m, 3.0f), *xp = vec(m, 3.0f), *xh = malloc(sizeof(float) * m);
        memset(x, 0, sizeof(float) * g);                           /* one zero group */
        int8_t* codes = malloc(m);
        float* sc = malloc(sizeof(float) * m / g);
        float* raw = malloc(sizeof(float) * m);
        if (b == 32) flo_quantize_rows(x, xp, n, H, d, g, 32, NULL, NULL, raw, xh);
        else {
            flo_quantize_rows(x, NULL, n, H, d, g, b, codes, sc, NULL, xh);
            flo_quantize_rows(x, xp, n, H, d, g, b, codes, sc, NULL, xh);
            uint8_t* packed = malloc((size_t)(m * b / 8));
            flo_pack_codes(codes, m, b, packed);
            free(packed);
            int8_t c1[32]; float s1;
            flo_quant_group(x + g, g, b, c1, &s1);
            uint8_t* uc = malloc(m);
            float *ks = malloc(sizeof(float) * m), *kz = malloc(sizeof(float) * m);
            flo_quantize_rows_asym(x, NULL, n, H, d, g, b, 1, uc, ks, kz, xh);   /* keys, ragged groups */
            flo_quantize_rows_asym(x, xp, n, H, d, g, b, 0, uc, ks, kz, xh);     /* values */
            uint8_t ucg[32]; float s2, z2;
            flo_quant_asym_group(x, g, 1, b, ucg, 1, &s2, &z2);
            free(uc); free(ks); free(kz);
        }
        free(x); free(xp); free(xh); free(codes); free(sc); free(raw);
    }
    /* attention family: tiny, ragged, and a single sink budget */
    case_attention(1, 1, 64, 5, 4);
    case_attention(29, 3, 64, 12, 4);
    case_attention(70, 2, 128, 20, 4);
    case_attention(9, 1, 64, 5, 4);
    free(h0); free(h1);
    if (fails) { fprintf(stderr, "%d expectation(s) failed\n", fails); return 1; }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}

/*
 * FlashLoop oracle: a plain, slow fp32 CPU implementation of one lazy-update
 * loop of attention in a looped (weight-shared, R-times repeated) Transformer.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU
 * baseline leg of the benchmark are the only callers.  Nothing here is shared
 * with the GPU library: no header, kernel, helper, table or constant.
 *
 * Source: "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
 * Updates" (arXiv 2609.29812), as cited per function below:
 *   Sec. 4.1  cross-loop token-sparse updates (top-k active tokens, nested sets)
 *   Sec. 4.2  loop-aware sparse attention (column ranking from the previous
 *             loop, cached global probability mass, progressive pruning)
 *   Sec. 3.3, Sec. 4.3, App. E "Quantization Setting"  quantised base plus
 *             low-bit cross-loop residuals, group size 64
 * The paper gives no equations (its Eq. 3 and App. D are not in the text), so
 * the formulation below is the one fixed for this implementation:
 *   o_r(i) = (1 - M_U(i)) * softmax_{S(i)}(s) . V + O_U(i)
 * where M_U / O_U are the probability mass / partial output, under the
 * previous loop's distribution, of the causal columns that are not selected.
 *
 * Every float operation is fp32, evaluated in program order.  Build with
 * -ffp-contract=off and without -ffast-math so that a*b+c is two roundings.
 * OpenMP only splits independent (row, head) or (head, column) work items; each
 * item is computed sequentially, so results do not depend on thread count.
 *
 * Layouts: per-token tensors are row-major [N][H][d] indexed by token position;
 * per-row loop state is [n_rows][H] / [n_rows][H][d] aligned with a row list;
 * column sets are [H][k], ascending positions per head.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int flo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Sec. 4.1: how many tokens stay active in a loop.  The paper keeps the
 * top-k tokens with a loop-dependent k; the workloads give k as a fraction rho
 * of the sequence length N.  Reading: n = ceil(rho*N) (a 1e-9 guard absorbs the
 * binary representation of rho), at least one token, never more than the
 * previous loop's active set (sets are nested). */
int flo_active_count(double rho, int N, int n_prev) {
    int n = (int)ceil(rho * (double)N - 1e-9);
    if (n < 1) n = 1;
    if (n > n_prev) n = n_prev;
    return n;
}

/* ------------------------------------------------------------------------ */
/* Sec. 4.1: token-change statistic ||h_r(i) - h_{r-1}(i)||_2 for each
 * candidate token (the tokens active in the previous loop).  h is [N][D]. */
void flo_delta_norm(const float* h_cur, const float* h_prev, int D,
                    const int* cand, int n_cand, float* stat) {
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < n_cand; ++t) {
        long i = cand ? cand[t] : t;
        const float* a = h_cur + i * (long)D;
        const float* b = h_prev + i * (long)D;
        float s = 0.0f;
        for (int c = 0; c < D; ++c) {
            float e = a[c] - b[c];
            float e2 = e * e;
            s = s + e2;
        }
        stat[t] = sqrtf(s);
    }
}

/* Sec. 4.1 ranks tokens by their *normalized* hidden-state change.  Read as
 * the change relative to the previous loop's state:
 *   stat(i) = ||h_r(i) - h_{r-1}(i)||_2 / ||h_{r-1}(i)||_2
 * (both norms fp32, then one division).  A token whose previous state is the
 * zero vector has no scale to normalise by: its statistic is 0 if it did not
 * change and +infinity otherwise (any change of a zero state is unbounded
 * relative to it). */
void flo_delta_norm_rel(const float* h_cur, const float* h_prev, int D,
                        const int* cand, int n_cand, float* stat) {
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < n_cand; ++t) {
        long i = cand ? cand[t] : t;
        const float* a = h_cur + i * (long)D;
        const float* b = h_prev + i * (long)D;
        float num = 0.0f, den = 0.0f;
        for (int c = 0; c < D; ++c) {
            float e = a[c] - b[c];
            float e2 = e * e;
            num = num + e2;
            float p2 = b[c] * b[c];
            den = den + p2;
        }
        float dn = sqrtf(num);
        float pn = sqrtf(den);
        if (pn > 0.0f) stat[t] = dn / pn;
        else stat[t] = dn > 0.0f ? INFINITY : 0.0f;
    }
}

/* ------------------------------------------------------------------------ */
/* Top-k selection used for both active tokens (Sec. 4.1) and columns
 * (Sec. 4.2): keep the n_sel candidates with the largest key; equal keys go to
 * the lower position; the result is listed in ascending position order.
 * -0.0 ranks as +0.0.  Returns -1 on a NaN key, else 0. */
typedef struct { float key; int pos; } flo_pair;

static int flo_cmp_rank(const void* pa, const void* pb) {
    const flo_pair* a = (const flo_pair*)pa;
    const flo_pair* b = (const flo_pair*)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    if (a->pos < b->pos) return -1;
    if (a->pos > b->pos) return 1;
    return 0;
}

static int flo_cmp_int(const void* pa, const void* pb) {
    int a = *(const int*)pa, b = *(const int*)pb;
    return (a > b) - (a < b);
}

int flo_top_select(const float* key, const int* pos, int n, int n_sel, int* out) {
    if (n_sel > n || n_sel < 0) return -1;
    flo_pair* p = (flo_pair*)malloc(sizeof(flo_pair) * (size_t)(n > 0 ? n : 1));
    for (int t = 0; t < n; ++t) {
        float k = key[t];
        if (isnan(k)) { free(p); return -1; }
        if (k == 0.0f) k = 0.0f; /* canonicalise -0 */
        p[t].key = k;
        p[t].pos = pos ? pos[t] : t;
    }
    qsort(p, (size_t)n, sizeof(flo_pair), flo_cmp_rank);
    for (int t = 0; t < n_sel; ++t) out[t] = p[t].pos;
    qsort(out, (size_t)n_sel, sizeof(int), flo_cmp_int);
    free(p);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Sec. 4.2: column selection for loop r from the statistics of loop r-1.
 * Per head: the n_sink first positions are always kept and counted inside the
 * budget k; the other k - n_sink columns are the top ones of the previous
 * selection by column statistic.  If the previous set already fits the budget
 * it is kept as is (selection only prunes, so sets are nested).
 * sel_prev == NULL means all positions 0..k_prev-1 (the dense first loop).
 * cstat is [H][k_prev] aligned with sel_prev.  Returns -1 on bad input. */
int flo_select_columns(const float* cstat, const int* sel_prev, int H, int k_prev,
                       int n_sink, int k, int* sel_out) {
    if (k_prev <= k) {
        for (int h = 0; h < H; ++h)
            for (int p = 0; p < k_prev; ++p)
                sel_out[(long)h * k_prev + p] = sel_prev ? sel_prev[(long)h * k_prev + p] : p;
        return 0;
    }
    if (n_sink > k) return -1;
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int h = 0; h < H; ++h) {
        const int* sp = sel_prev ? sel_prev + (long)h * k_prev : NULL;
        const float* cs = cstat + (long)h * k_prev;
        int* so = sel_out + (long)h * k;
        float* key = (float*)malloc(sizeof(float) * (size_t)k_prev);
        int* pos = (int*)malloc(sizeof(int) * (size_t)k_prev);
        int n_cand = 0, n_sink_found = 0;
        for (int p = 0; p < k_prev; ++p) {
            int j = sp ? sp[p] : p;
            if (j < n_sink) { n_sink_found++; continue; }
            key[n_cand] = cs[p];
            pos[n_cand] = j;
            n_cand++;
        }
        if (n_sink_found != n_sink || k - n_sink > n_cand) { bad = 1; }
        else {
            for (int s = 0; s < n_sink; ++s) so[s] = s;
            if (flo_top_select(key, pos, n_cand, k - n_sink, so + n_sink) != 0) bad = 1;
        }
        free(key); free(pos);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Sec. 3.3 / Sec. 4.3 / App. E: group quantiser.  Symmetric absmax scale per
 * group of g contiguous channels: s = max|x| / qmax with qmax = 2^(b-1)-1
 * (127 int8, 7 int4, 1 int2), code = round-half-even(x / s) clamped to
 * [-qmax, qmax]; an all-zero group (or a scale that underflows to 0) gets s and
 * codes of 0.  Division is IEEE fp32. */
void flo_quant_group(const float* x, int g, int bits, int8_t* code, float* scale) {
    int qmax = (1 << (bits - 1)) - 1;
    float a = 0.0f;
    for (int c = 0; c < g; ++c) {
        float ax = fabsf(x[c]);
        if (ax > a) a = ax;
    }
    float s = a / (float)qmax;
    for (int c = 0; c < g; ++c) {
        if (s == 0.0f) { code[c] = 0; continue; }
        float t = x[c] / s;
        float r = rintf(t); /* default rounding mode: nearest, ties to even */
        if (r > (float)qmax) r = (float)qmax;
        if (r < -(float)qmax) r = -(float)qmax;
        code[c] = (int8_t)r;
    }
    *scale = s;
}

/* One quantised level of the KV cache for n rows ([n][H][d] each).
 * xhat_prev == NULL: the base level (loop 1) quantises x_new itself.
 * Otherwise the residual x = x_new - xhat_prev against the previous loop's
 * dequantised value is quantised, and xhat = xhat_prev + code*s (the product
 * and the sum are rounded separately).  bits == 32 keeps the residual as raw
 * fp32 in resid_raw (the "unquantised" mode).  codes are unpacked int8
 * [n][H][d]; scales [n][H][d/g]. */
void flo_quantize_rows(const float* x_new, const float* xhat_prev, long n, int H, int d,
                       int g, int bits, int8_t* codes, float* scales, float* resid_raw,
                       float* xhat_out) {
    int G = d / g;
    #pragma omp parallel for schedule(static)
    for (long rh = 0; rh < n * H; ++rh) {
        const float* xn = x_new + rh * d;
        const float* xp = xhat_prev ? xhat_prev + rh * d : NULL;
        float* xo = xhat_out + rh * d;
        float buf[512];
        for (int c = 0; c < d; ++c) buf[c] = xp ? xn[c] - xp[c] : xn[c];
        if (bits == 32) {
            for (int c = 0; c < d; ++c) {
                if (resid_raw) resid_raw[rh * d + c] = buf[c];
                xo[c] = xp ? xp[c] + buf[c] : buf[c];
            }
            continue;
        }
        for (int q = 0; q < G; ++q) {
            int8_t* cq = codes + rh * d + (long)q * g;
            float s;
            flo_quant_group(buf + q * g, g, bits, cq, &s);
            scales[rh * G + q] = s;
            for (int c = 0; c < g; ++c) {
                float deq = (float)cq[c] * s;
                xo[q * g + c] = xp ? xp[q * g + c] + deq : deq;
            }
        }
    }
}

/* Storage packing of codes (two's complement): int8 one per byte; int4 two per
 * byte, even channel in the low nibble; int2 four per byte, channel c at bits
 * 2*(c mod 4). */
void flo_pack_codes(const int8_t* codes, long count, int bits, uint8_t* out) {
    if (bits == 8) {
        for (long i = 0; i < count; ++i) out[i] = (uint8_t)codes[i];
        return;
    }
    int per = 8 / bits;
    uint8_t mask = (uint8_t)((1u << bits) - 1u);
    memset(out, 0, (size_t)(count / per));
    for (long i = 0; i < count; ++i)
        out[i / per] |= (uint8_t)(((uint8_t)codes[i] & mask) << (bits * (int)(i % per)));
}

/* ------------------------------------------------------------------------ */
/* App. E ("Quantization Setting"): the paper's own quantiser, asymmetric
 * min/max group quantisation.  For the n values x[i*stride] of one group:
 *   z = min x,  s = (max x - min x) / qmax  (qmax = 2^b - 1: 15 for INT4),
 *   code = round-half-even((x - z) / s) clamped to [0, qmax],
 *   dequantised value = code*s + z  (product and sum rounded separately).
 * A constant group (or one whose range underflows to s = 0) gets codes 0 and
 * is reproduced exactly by z.  Codes are unsigned; a zero offset or scale is
 * stored as +0. */
void flo_quant_asym_group(const float* x, int n, long stride, int bits, uint8_t* code,
                          long code_stride, float* scale, float* zero) {
    int qmax = (1 << bits) - 1;
    float mn = x[0], mx = x[0];
    for (int i = 1; i < n; ++i) {
        float v = x[(long)i * stride];
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    /* a signed zero in the group could make min / max (hence z and s) -0 or
     * +0 depending on the order of comparison; both are stored as +0 (x + 0
     * leaves every other value unchanged), so the stored words are unique */
    mn = mn + 0.0f;
    float range = mx - mn;
    float s = range / (float)qmax + 0.0f;
    for (int i = 0; i < n; ++i) {
        uint8_t c = 0;
        if (s != 0.0f) {
            float t = x[(long)i * stride] - mn;
            float r = rintf(t / s);
            if (r > (float)qmax) r = (float)qmax;
            if (r < 0.0f) r = 0.0f;
            c = (uint8_t)r;
        }
        code[(long)i * code_stride] = c;
    }
    *scale = s;
    *zero = mn;
}

/* One level of the KV cache under the paper's quantiser, for n packed rows
 * ([n][H][d]).  The quantised quantity is x = x_new - xhat_prev (xhat_prev ==
 * NULL: the base level, x = x_new), and xhat = xhat_prev + (code*s + z).
 *   per_channel = 0 (values, per token): groups of g contiguous channels of a
 *     (row, head); scales / zeros [n][H][d/g].
 *   per_channel = 1 (post-RoPE keys, per channel): for each (head, channel),
 *     groups of g consecutive packed rows (the last group may be shorter);
 *     scales / zeros [ceil(n/g)][H][d].
 * codes: unpacked unsigned [n][H][d]. */
void flo_quantize_rows_asym(const float* x_new, const float* xhat_prev, long n, int H, int d,
                            int g, int bits, int per_channel, uint8_t* codes, float* scales,
                            float* zeros, float* xhat_out) {
    long HD = (long)H * d;
    float* x = (float*)malloc(sizeof(float) * (size_t)(n * HD > 0 ? n * HD : 1));
    for (long e = 0; e < n * HD; ++e) x[e] = xhat_prev ? x_new[e] - xhat_prev[e] : x_new[e];
    if (per_channel) {
        long ng = (n + g - 1) / g;
        #pragma omp parallel for schedule(static)
        for (long gc = 0; gc < ng * HD; ++gc) {
            long grp = gc / HD, ch = gc % HD;
            long r0 = grp * g;
            int len = (int)((n - r0) < g ? (n - r0) : g);
            flo_quant_asym_group(x + r0 * HD + ch, len, HD, bits, codes + r0 * HD + ch, HD,
                                 scales + gc, zeros + gc);
        }
    } else {
        int G = d / g;
        #pragma omp parallel for schedule(static)
        for (long q = 0; q < n * H * G; ++q)
            flo_quant_asym_group(x + q * g, g, 1, bits, codes + q * g, 1, scales + q, zeros + q);
    }
    #pragma omp parallel for schedule(static)
    for (long e = 0; e < n * HD; ++e) {
        long row = e / HD, ch = e % HD;
        long si = per_channel ? (row / g) * HD + ch : e / g;
        float deq = (float)codes[e] * scales[si];
        deq = deq + zeros[si];
        xhat_out[e] = xhat_prev ? xhat_prev[e] + deq : deq;
    }
    free(x);
}

/* ------------------------------------------------------------------------ */
/* Sec. 4.2: sparse attention of loop r for the active rows.  For row i (a
 * token position) and head h the causal selected columns are
 * S(i) = { j in sel[h] : j <= i }.  Logits s = sm * q(i).khat(j); lse = log of
 * the sum of exp(s) over S(i); P = (1 - M_U(i)) * exp(s - lse) (softmax over
 * the selected logits rescaled to the cached mass of the selected set);
 * o(i) = sum_{S(i)} P * vhat(j) + O_U(i).
 * sel == NULL means all columns (k == N): the dense first loop, with M_U and
 * O_U given as NULL (zero).  q, khat, vhat are [N][H][d] by position; mass_u,
 * lse are [n_rows][H]; out_u, out are [n_rows][H][d]. */
void flo_attend(int N, int H, int d, float sm, const float* q, const float* khat,
                const float* vhat, const int* rows, int n_rows, const int* sel, int k,
                const float* mass_u, const float* out_u, float* out, float* lse) {
    (void)N;
    #pragma omp parallel for schedule(dynamic, 4)
    for (long th = 0; th < (long)n_rows * H; ++th) {
        long t = th / H;
        int h = (int)(th % H);
        long i = rows ? rows[t] : t;
        const float* qi = q + (i * H + h) * d;
        const int* sh = sel ? sel + (long)h * k : NULL;
        /* pass 1: max logit over S(i) */
        float m = -INFINITY;
        int cnt = 0;
        for (int p = 0; p < k; ++p) {
            long j = sh ? sh[p] : p;
            if (j > i) break;
            const float* kj = khat + (j * H + h) * d;
            float s = 0.0f;
            for (int c = 0; c < d; ++c) { float pr = qi[c] * kj[c]; s = s + pr; }
            s = s * sm;
            if (s > m) m = s;
            cnt++;
        }
        float* oi = out + th * d;
        float u = mass_u ? mass_u[th] : 0.0f;
        if (cnt == 0) {
            /* no selected causal column (cannot happen with sinks) */
            for (int c = 0; c < d; ++c) oi[c] = out_u ? out_u[th * d + c] : 0.0f;
            lse[th] = -INFINITY;
            continue;
        }
        /* pass 2: normaliser */
        float z = 0.0f;
        for (int p = 0; p < cnt; ++p) {
            long j = sh ? sh[p] : p;
            const float* kj = khat + (j * H + h) * d;
            float s = 0.0f;
            for (int c = 0; c < d; ++c) { float pr = qi[c] * kj[c]; s = s + pr; }
            s = s * sm;
            z = z + expf(s - m);
        }
        float l = m + logf(z);
        lse[th] = l;
        /* pass 3: output */
        for (int c = 0; c < d; ++c) oi[c] = 0.0f;
        for (int p = 0; p < cnt; ++p) {
            long j = sh ? sh[p] : p;
            const float* kj = khat + (j * H + h) * d;
            const float* vj = vhat + (j * H + h) * d;
            float s = 0.0f;
            for (int c = 0; c < d; ++c) { float pr = qi[c] * kj[c]; s = s + pr; }
            s = s * sm;
            float P = (1.0f - u) * expf(s - l);
            for (int c = 0; c < d; ++c) { float pv = P * vj[c]; oi[c] = oi[c] + pv; }
        }
        for (int c = 0; c < d; ++c) oi[c] = oi[c] + (out_u ? out_u[th * d + c] : 0.0f);
    }
}

/* ------------------------------------------------------------------------ */
/* Sec. 4.2 ("indices and their probability mass are propagated"): caches of
 * the columns dropped when loop r prunes the selection.  For each active row i
 * and head h, over j in S_{r-1}(i) \ S_r(i), under loop r-1's distribution
 *   P_{r-1}(i,j) = (1 - M_U^{r-1}(i)) * exp(sm*q_{r-1}(i).khat_{r-1}(j) - lse_{r-1}(i))
 *   M_U^r(i) = M_U^{r-1}(i) + sum P_{r-1}(i,j)
 *   O_U^r(i) = O_U^{r-1}(i) + sum P_{r-1}(i,j) * vhat_{r-1}(j)
 * (additive form).  sel_prev == NULL: all columns (k_prev == N, after the dense
 * first loop) with mass_u_prev / out_u_prev NULL (zero).  lse_prev,
 * mass_u_prev, out_u_prev are aligned with rows. */
void flo_unselected_cache(int N, int H, int d, float sm, const float* q_prev,
                          const float* khat_prev, const float* vhat_prev, const int* rows,
                          int n_rows, const int* sel_prev, int k_prev, const int* sel_new,
                          int k_new, const float* lse_prev, const float* mass_u_prev,
                          const float* out_u_prev, float* mass_u, float* out_u) {
    (void)N;
    #pragma omp parallel for schedule(dynamic, 4)
    for (long th = 0; th < (long)n_rows * H; ++th) {
        long t = th / H;
        int h = (int)(th % H);
        long i = rows[t];
        const float* qi = q_prev + (i * H + h) * d;
        const int* sp = sel_prev ? sel_prev + (long)h * k_prev : NULL;
        const int* sn = sel_new + (long)h * k_new;
        float u_prev = mass_u_prev ? mass_u_prev[th] : 0.0f;
        float M = u_prev;
        float* O = out_u + th * d;
        for (int c = 0; c < d; ++c) O[c] = out_u_prev ? out_u_prev[th * d + c] : 0.0f;
        int pn = 0; /* merge walk over the ascending new selection */
        for (int p = 0; p < k_prev; ++p) {
            long j = sp ? sp[p] : p;
            if (j > i) break;
            while (pn < k_new && sn[pn] < j) pn++;
            if (pn < k_new && sn[pn] == j) continue; /* still selected */
            const float* kj = khat_prev + (j * H + h) * d;
            const float* vj = vhat_prev + (j * H + h) * d;
            float s = 0.0f;
            for (int c = 0; c < d; ++c) { float pr = qi[c] * kj[c]; s = s + pr; }
            s = s * sm;
            float P = (1.0f - u_prev) * expf(s - lse_prev[th]);
            M = M + P;
            for (int c = 0; c < d; ++c) { float pv = P * vj[c]; O[c] = O[c] + pv; }
        }
        mass_u[th] = M;
    }
}

/* ------------------------------------------------------------------------ */
/* Sec. 4.2 ("rank the attention columns using statistics from the previous
 * loop"): the attention-contribution statistic of each selected column, read
 * as its probability mass summed over the rows computed in this loop:
 *   c(j) = sum_{i in rows, i >= j} (1 - M_U(i)) * exp(sm*q(i).khat(j) - lse(i)).
 * sel == NULL means all columns (k == N).  cstat is [H][k].
 * With vhat != NULL ([N][H][d], the dequantised values the loop attended to)
 * each column's mass is weighted by the norm of its value vector, which reads
 * the statistic as the size of the column's contribution to the loop's
 * outputs: sum_i (1 - M_U(i)) P(i,j) ||vhat(j)||_2 = sum_i ||(1 - M_U(i)) P(i,j) vhat(j)||_2. */
void flo_column_stats(int N, int H, int d, float sm, const float* q, const float* khat,
                      const int* rows, int n_rows, const int* sel, int k, const float* lse,
                      const float* mass_u, const float* vhat, float* cstat) {
    (void)N;
    #pragma omp parallel for schedule(dynamic, 16)
    for (long hp = 0; hp < (long)H * k; ++hp) {
        int h = (int)(hp / k);
        int p = (int)(hp % k);
        long j = sel ? sel[hp] : p;
        const float* kj = khat + (j * H + h) * d;
        float c = 0.0f;
        for (int t = 0; t < n_rows; ++t) {
            long i = rows ? rows[t] : t;
            if (i < j) continue;
            const float* qi = q + (i * H + h) * d;
            float s = 0.0f;
            for (int e = 0; e < d; ++e) { float pr = qi[e] * kj[e]; s = s + pr; }
            s = s * sm;
            long th = (long)t * H + h;
            float u = mass_u ? mass_u[th] : 0.0f;
            float P = (1.0f - u) * expf(s - lse[th]);
            c = c + P;
        }
        if (vhat) {
            /* value-weighted variant: the column's mass times ||vhat(j)||_2 */
            const float* vj = vhat + (j * H + h) * d;
            float v2 = 0.0f;
            for (int e = 0; e < d; ++e) { float sq = vj[e] * vj[e]; v2 = v2 + sq; }
            c = c * sqrtf(v2);
        }
        cstat[hp] = c;
    }
}

// Host side of the C ABI declared in include/flashloop.h: argument
// validation (before anything is enqueued), workspace carving and kernel
// sequencing for one loop of FlashLoop's lazy-update attention step.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "fl_kernels.h"


namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(FL_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define FL_REQUIRE(cond, ...)                                        \
    do {                                                             \
        if (!(cond)) return fail(FL_ERR_INVALID_ARG, __VA_ARGS__);   \
    } while (0)
#define FL_HIP(expr, where)                                          \
    do {                                                             \
        hipError_t e_ = (expr);                                      \
        if (e_ != hipSuccess) return hip_fail(e_, where);            \
    } while (0)

constexpr long kAlign = 256;
long align_up(long x) { return (x + kAlign - 1) / kAlign * kAlign; }
long kpad(long k) { return (k + 63) / 64 * 64; }

// Workspace of fl_sparse_loop_attn (k selected columns, n active rows):
//  * compact bf16 copies of the selected columns, K and V^T, each with a "lo"
//    copy (the residual x - bf16(x)), for the current loop and, for a cache
//    rebuild, the previous one: 8 buffers of H x kp x d bf16, kp = the padded
//    column count plus room for the [normal | pad | outlier] slot order;
//  * per side: column positions and slot order [H][kp], the parts' sizes
//    [H][2], the row order [H][n] and normal-row count [H]; one [H][n] byte
//    plane of row flags; the value norms [H][kp]; the pruned-column list of
//    an additive rebuild [H][kp] (six [H][kp] int planes in all);
//  * the in-tile path adds per-level quantised planes (codes <= 8 bits, fp32
//    scales per group of >= 32 channels) for K and V.
long kslots(long k) { return kpad(k) + 128; }
long quant_plane_bytes(long H, long kp, long d) {
    return 2 * (align_up(H * kp * d) + align_up(H * kp * (d / 32) * 4));
}
long attn_ws_bytes_once(long H, long k, long d, long n) {
    const long kp = kslots(k);
    return 8 * align_up(H * kp * d * 2) + 6 * align_up(H * kp * 4) + align_up(H * kp) +
           2 * align_up(H * 2 * 4) + align_up(H * fl::class_row_stride(n)) + 2 * align_up(H * n * 4) +
           2 * align_up(H * 4) +
           kAlign;
}
long attn_ws_bytes(long H, long k, long d, long n, long levels) {
    if (levels <= 0 || levels > FL_MAX_LEVELS) levels = FL_MAX_LEVELS;
    return attn_ws_bytes_once(H, k, d, n) + levels * quant_plane_bytes(H, kslots(k), d);
}

// workspace of fl_block_step: compact bf16 activations of the active rows
// (normed input, qkv, q/k/v, attention output, SwiGLU output) followed by the
// attention workspace.
long block_ws_bytes(long N, long H, long d, long F) {
    const long D = H * d;
    return align_up(N * D * 2) * 5 + align_up(N * 3 * D * 2) + align_up(N * F * 2) +
           attn_ws_bytes_once(H, N, d, N) + kAlign;
}

// Operand precision of the attention products: residual levels hold the
// cross-loop updates, which sit below bf16's resolution of the summed value,
// so a cache with residual levels feeds K, V and P as hi + lo bf16 pairs;
// fp32 inputs split q as well.
int attn_prec(int dtype, int level) { return dtype == FL_F32 ? 2 : (level >= 1 ? 1 : 0); }

// ---- optional per-kernel HIP-event timing of the library's launches ----
struct TimedLaunch {
    std::string name;
    hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_timing = false;  // per-kernel event pairs
bool g_phases = false;  // per-phase event pairs of fl_loop_step
// prefix of kernel timing names inside a phase of fl_loop_step ("loop<r>.a5-a8/")
thread_local std::string g_prefix;
std::vector<TimedLaunch> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t ev_get() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// set while an allocation-free call runs on this thread: no events
thread_local bool g_no_events = false;

template <class F>
hipError_t timed(const char* name, hipStream_t st, F&& f) {
    if (!g_timing || g_no_events) return f();
    std::lock_guard<std::mutex> lk(g_tmu);
    hipEvent_t a = ev_get(), b = ev_get();
    if (a) (void)hipEventRecord(a, st);
    const hipError_t e = f();
    if (b) (void)hipEventRecord(b, st);
    if (a && b) g_recs.push_back({g_prefix + name, a, b});
    return e;
}

// An event recorded on the stream when phase timing is on (else NULL);
// phase_end records the closing event and keeps the pair under `name`.
hipEvent_t phase_begin(hipStream_t st) {
    if (!g_phases || g_no_events) return nullptr;
    std::lock_guard<std::mutex> lk(g_tmu);
    hipEvent_t a = ev_get();
    if (a && hipEventRecord(a, st) != hipSuccess) {
        g_pool.push_back(a);
        return nullptr;
    }
    return a;
}
void phase_end(hipEvent_t a, const std::string& name, hipStream_t st) {
    if (!a) return;
    std::lock_guard<std::mutex> lk(g_tmu);
    hipEvent_t b = ev_get();
    if (b && hipEventRecord(b, st) == hipSuccess) {
        g_recs.push_back({name, a, b});
    } else {
        g_pool.push_back(a);
        if (b) g_pool.push_back(b);
    }
}

// timing names of the block's projections, by output tile width (64 / 128)
const char* const kGemmQkv[2] = {"gemm_qkv.w64", "gemm_qkv.w128"};
const char* const kGemmO[2] = {"gemm_o.w64", "gemm_o.w128"};
const char* const kGemmGateUp[2] = {"gemm_gate_up.w64", "gemm_gate_up.w128"};
const char* const kGemmDown[2] = {"gemm_down.w64", "gemm_down.w128"};
const char* gemm_name(const char* const* names, const fl::GemmParams& G) {
    return names[fl::gemm_tile_n(G) == 128 ? 1 : 0];
}

// ---- input validation (fl_check_indices / fl_check_finite / fl_set_checks) ----
bool g_checks = false;

// idx[0..n) strictly ascending, each in [lo, hi); on failure names `what`,
// the row (for row-wise lists) and the first offending element
int check_idx_host(const int32_t* idx, long n, long lo, long hi, const char* what, long row = -1) {
    char rs[32] = "";
    if (row >= 0) snprintf(rs, sizeof rs, " row %ld", row);
    for (long i = 0; i < n; ++i) {
        if (idx[i] < lo || idx[i] >= hi)
            return fail(FL_ERR_INVALID_ARG, "%s%s: element %ld = %d outside [%ld, %ld)", what, rs, i,
                        idx[i], lo, hi);
        if (i > 0 && idx[i] <= idx[i - 1])
            return fail(FL_ERR_INVALID_ARG, "%s%s: element %ld = %d not above element %ld = %d "
                        "(ascending, unique)", what, rs, i, idx[i], i - 1, idx[i - 1]);
    }
    return FL_OK;
}
int check_finite_host(const float* x, long n, const char* what, bool allow_inf = false) {
    for (long i = 0; i < n; ++i)
        if (allow_inf ? std::isnan(x[i]) : !std::isfinite(x[i]))
            return fail(FL_ERR_INVALID_ARG, "%s: element %ld = %g is not %s", what, i, (double)x[i],
                        allow_inf ? "a number" : "finite");
    return FL_OK;
}
// Check mode: device arrays copied to the host (after the stream's pending
// work, which may produce them) and validated there before anything is
// enqueued.  rows x n row-wise lists, each row checked on its own.
int check_idx_dev(const int32_t* d_idx, long rows, long n, long lo, long hi, const char* what,
                  hipStream_t st) {
    if (!g_checks || !d_idx || rows * n == 0) return FL_OK;
    std::vector<int32_t> h((size_t)(rows * n));
    FL_HIP(hipStreamSynchronize(st), "check: sync");
    FL_HIP(hipMemcpy(h.data(), d_idx, h.size() * 4, hipMemcpyDeviceToHost), "check: copy");
    for (long r = 0; r < rows; ++r) {
        const int rc = check_idx_host(h.data() + r * n, n, lo, hi, what, rows > 1 ? r : -1);
        if (rc) return rc;
    }
    return FL_OK;
}
int check_finite_dev(const float* d_x, long n, const char* what, hipStream_t st,
                     bool allow_inf = false) {
    if (!g_checks || !d_x || n == 0) return FL_OK;
    std::vector<float> h((size_t)n);
    FL_HIP(hipStreamSynchronize(st), "check: sync");
    FL_HIP(hipMemcpy(h.data(), d_x, h.size() * 4, hipMemcpyDeviceToHost), "check: copy");
    return check_finite_host(h.data(), n, what, allow_inf);
}
// the row lists of residual levels 1..upto (ascending positions in [0, N))
int check_levels_dev(const fl_kv_cache& C, int upto, hipStream_t st) {
    if (!g_checks) return FL_OK;
    for (int l = 1; l <= upto; ++l) {
        char what[48];
        snprintf(what, sizeof what, "level %d rows", l);
        const int rc = check_idx_dev(C.level[l].rows, 1, C.level[l].n_rows, 0, C.N, what, st);
        if (rc) return rc;
    }
    return FL_OK;
}

bool dtype_ok(int dt) { return dt == FL_F32 || dt == FL_BF16; }
bool stat_kinds_ok(int token_stat, int col_stat) {
    return (token_stat == FL_TOKEN_STAT_ABS || token_stat == FL_TOKEN_STAT_REL) &&
           (col_stat == FL_COL_STAT_MASS || col_stat == FL_COL_STAT_VNORM);
}

int check_cache(const fl_kv_cache* c, int upto) {
    FL_REQUIRE(c != nullptr, "cache is NULL");
    FL_REQUIRE(c->N > 0 && c->H > 0, "cache: N=%d H=%d", c->N, c->H);
    if (!(c->d == 64 || c->d == 128)) return fail(FL_ERR_UNSUPPORTED, "head dim %d (64 or 128)", c->d);
    if (!(c->g == 32 || c->g == 64) || c->d % c->g)
        return fail(FL_ERR_UNSUPPORTED, "group size %d (32 or 64, dividing d)", c->g);
    FL_REQUIRE(c->H * c->d <= 8192, "H*d = %d > 8192", c->H * c->d);
    FL_REQUIRE(upto >= 0 && upto < FL_MAX_LEVELS, "level %d out of range", upto);
    FL_REQUIRE(c->scheme == FL_QUANT_ABSMAX || c->scheme == FL_QUANT_ASYM, "scheme %d", c->scheme);
    const bool asym = c->scheme == FL_QUANT_ASYM;
    for (int l = 0; l <= upto; ++l) {
        const fl_kv_level& L = c->level[l];
        if (asym) {
            if (!(L.bits == 2 || L.bits == 4 || L.bits == 8))
                return fail(FL_ERR_UNSUPPORTED, "level %d bits %d (2, 4 or 8 under FL_QUANT_ASYM)", l,
                            L.bits);
            FL_REQUIRE(L.k_zero && L.v_zero, "level %d: offset buffers NULL", l);
        }
        if (l == 0) {
            if (!asym && !(L.bits == 8 || L.bits == 32))
                return fail(FL_ERR_UNSUPPORTED, "base level bits %d (8 or 32)", L.bits);
        } else {
            if (!(L.bits == 2 || L.bits == 4 || L.bits == 8 || L.bits == 32))
                return fail(FL_ERR_UNSUPPORTED, "level %d bits %d", l, L.bits);
            FL_REQUIRE(L.rows && L.slot, "level %d: rows/slot NULL", l);
            FL_REQUIRE(L.n_rows >= 0 && L.n_rows <= c->N, "level %d: n_rows %d", l, L.n_rows);
        }
        FL_REQUIRE(L.k_codes && L.v_codes, "level %d: code buffers NULL", l);
        FL_REQUIRE(L.bits == 32 || (L.k_scale && L.v_scale), "level %d: scale buffers NULL", l);
    }
    return FL_OK;
}

// per-sequence capacities of the batched decode cache
int decode_caps(const fl_decode_cfg* cfg, const fl_kv_cache& C, int upto, fl::DecodeParams& P) {
    P.pos_cap = cfg->N_cap ? cfg->N_cap : cfg->N;
    FL_REQUIRE(cfg->N <= P.pos_cap, "N=%d exceeds N_cap=%d", cfg->N, P.pos_cap);
    for (int l = 1; l <= upto; ++l) {
        P.rows_cap[l] = cfg->rows_cap[l] ? cfg->rows_cap[l] : C.level[l].n_rows;
        FL_REQUIRE(C.level[l].n_rows <= P.rows_cap[l], "level %d: n_rows %d exceeds rows_cap %d", l,
                   C.level[l].n_rows, P.rows_cap[l]);
    }
    // asymmetric key groups: g rows from row 0 below the origin, g rows from
    // the origin on (the groups appended during generation)
    const int g = C.g;
    for (int l = 0; l <= upto; ++l) {
        const int o = C.scheme == FL_QUANT_ASYM ? cfg->key_group_origin[l] : 0;
        const int cap = l == 0 ? P.pos_cap : P.rows_cap[l];
        FL_REQUIRE(o >= 0 && o <= cap, "level %d: key_group_origin %d outside 0..%d", l, o, cap);
        const int below = (o + g - 1) / g;
        P.kg_origin[l] = o;
        P.kg_pad[l] = below * g - o;
        P.kg_count[l] = below + (cap - o + g - 1) / g;
    }
    return FL_OK;
}

} // namespace

extern "C" {

const char* fl_last_error(void) { return g_err; }

const char* fl_version(void) { return "flashloop-mi355x 0.1 (gfx950)"; }

int fl_check_indices(const int32_t* idx, long n, long lo, long hi) {
    FL_REQUIRE(n >= 0 && (n == 0 || idx), "idx NULL or n = %ld", n);
    return check_idx_host(idx, n, lo, hi, "indices");
}

int fl_check_finite(const float* x, long n) {
    FL_REQUIRE(n >= 0 && (n == 0 || x), "x NULL or n = %ld", n);
    return check_finite_host(x, n, "values");
}

int fl_set_checks(int on) {
    g_checks = on != 0;
    return FL_OK;
}

size_t fl_workspace_size(int op, long a, long b, long c, long e) {
    switch (op) {
    case FL_WS_SELECT_ACTIVE: return a > 0 ? (size_t)kAlign : 0;
    case FL_WS_SELECT_COLUMNS: return (a > 0 && b > 0) ? (size_t)kAlign : 0;
    case FL_WS_BLOCK_STEP:
        if (a <= 0 || b <= 0 || !(c == 64 || c == 128) || e <= 0) return 0;
        return (size_t)block_ws_bytes(a, b, c, e);
    case FL_WS_SQ_ERR:
        return a > 0 ? (size_t)(align_up(16L * fl::sq_err_blocks(a)) + kAlign) : 0;
    case FL_WS_SPARSE_ATTN:
        if (a <= 0 || b <= 0 || !(c == 64 || c == 128) || e <= 0) return 0;
        return (size_t)attn_ws_bytes_once(a, b, c, e);
    case FL_WS_LOOP_STEP:
        if (a <= 0 || b <= 0 || !(c == 64 || c == 128)) return 0;
        return (size_t)attn_ws_bytes(a, b, c, b, e);
    default: return 0;
    }
}

int fl_timing_enable(int level) {
    if (level < 0 || level > 2) return fail(FL_ERR_INVALID_ARG, "timing level %d (0, 1 or 2)", level);
    std::lock_guard<std::mutex> lk(g_tmu);
    g_timing = level == 1;
    g_phases = level != 0;
    return FL_OK;
}

int fl_timing_report(char* buf, size_t len) {
    std::lock_guard<std::mutex> lk(g_tmu);
    std::map<std::string, std::pair<long, double>> agg;
    int rc = FL_OK;
    for (auto& r : g_recs) {
        float ms = 0.0f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess) rc = hip_fail(e, "timing");
        auto& x = agg[r.name];
        x.first += 1;
        x.second += ms;
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_recs.clear();
    std::string out;
    char line[160];
    for (auto& kv : agg) {
        snprintf(line, sizeof line, "%s %ld %.6f\n", kv.first.c_str(), kv.second.first, kv.second.second);
        out += line;
    }
    if (buf && len) {
        snprintf(buf, len, "%s", out.c_str());
        if (out.size() + 1 > len) rc = fail(FL_ERR_INVALID_ARG, "timing report truncated");
    }
    return rc;
}

int fl_select_active(int dtype, int stat_kind, const void* h_cur, const void* h_prev, int N, int D,
                     const int32_t* cand, int n_cand, int n_select, const float* stat_in,
                     float* stat_out, int32_t* active_out, int32_t* slot_out, void* ws,
                     size_t ws_bytes, fl_stream_t stream) {
    (void)ws; (void)ws_bytes;
    FL_REQUIRE(N > 0, "N = %d", N);
    FL_REQUIRE(n_cand >= 1 && n_cand <= N, "n_cand %d not in [1, N=%d]", n_cand, N);
    FL_REQUIRE(n_select >= 1 && n_select <= n_cand, "n_select %d not in [1, n_cand=%d]", n_select, n_cand);
    FL_REQUIRE(active_out != nullptr, "active_out is NULL");
    FL_REQUIRE(stat_kind == FL_TOKEN_STAT_ABS || stat_kind == FL_TOKEN_STAT_REL, "stat_kind %d",
               stat_kind);
    if (!stat_in) {
        FL_REQUIRE(dtype_ok(dtype), "dtype %d", dtype);
        FL_REQUIRE(h_cur && h_prev && stat_out, "h_cur/h_prev/stat_out NULL");
        FL_REQUIRE(D >= 8 && D % 8 == 0, "D = %d (multiple of 8 required)", D);
    }
    hipStream_t st = (hipStream_t)stream;
    int rc = check_idx_dev(cand, 1, n_cand, 0, N, "cand", st);
    if (!rc) rc = check_finite_dev(stat_in, n_cand, "stat_in", st);
    if (rc) return rc;
    const float* keys = stat_in;
    if (!stat_in) {
        FL_HIP(timed("delta_norm", st, [&] {
                   return fl::launch_delta_norm(h_cur, h_prev, dtype, D, cand, n_cand,
                                                stat_kind == FL_TOKEN_STAT_REL, stat_out, st);
               }),
               "delta_norm");
        keys = stat_out;
        // the normalised statistic is +inf for a changed zero state; NaN (from
        // non-finite hidden states) cannot be ranked
        rc = check_finite_dev(stat_out, n_cand, "statistic (from h_cur / h_prev)", st, true);
        if (rc) return rc;
    }
    FL_HIP(timed("select_topk", st, [&] {
               return fl::launch_topk(keys, 0, cand, 0, n_cand, n_select, 0, active_out, 0, slot_out,
                                      slot_out ? N : 0, 1, st);
           }),
           "topk");
    return FL_OK;
}

int fl_sq_err(const float* x, const float* ref, long n, double* out, void* ws, size_t ws_bytes,
              fl_stream_t stream) {
    FL_REQUIRE(n >= 1, "n = %ld", n);
    FL_REQUIRE(x && ref && out, "x/ref/out NULL");
    FL_REQUIRE(((uintptr_t)x % 16) == 0 && ((uintptr_t)ref % 16) == 0, "x/ref not 16-byte aligned");
    const long need = align_up(16L * fl::sq_err_blocks(n)) + kAlign;
    if (!ws || (long)ws_bytes < need)
        return fail(FL_ERR_WORKSPACE, "workspace %zu < %ld bytes", ws_bytes, need);
    double* part = (double*)(((uintptr_t)ws + kAlign - 1) / kAlign * kAlign);
    hipStream_t st = (hipStream_t)stream;
    FL_HIP(timed("sq_err", st, [&] { return fl::launch_sq_err(x, ref, n, part, out, st); }), "sq_err");
    return FL_OK;
}

int fl_select_columns(const float* col_stat, const int32_t* cand_cols, int H, int n_cand,
                      int n_sink, int k, int32_t* sel_out, void* ws, size_t ws_bytes,
                      fl_stream_t stream) {
    (void)ws; (void)ws_bytes;
    FL_REQUIRE(H >= 1 && n_cand >= 1, "H=%d n_cand=%d", H, n_cand);
    FL_REQUIRE(sel_out != nullptr, "sel_out is NULL");
    FL_REQUIRE(n_sink >= 0, "n_sink %d", n_sink);
    FL_REQUIRE(k > n_sink, "k=%d must exceed n_sink=%d", k, n_sink);
    hipStream_t st = (hipStream_t)stream;
    int rc = check_idx_dev(cand_cols, H, n_cand, 0, 0x7fffffff, "cand_cols", st);
    if (rc) return rc;
    if (n_cand <= k) {
        FL_HIP(fl::launch_copy_or_iota(cand_cols, sel_out, (long)H * n_cand, n_cand, st), "copy");
        return FL_OK;
    }
    rc = check_finite_dev(col_stat, (long)H * n_cand, "col_stat", st);
    if (rc) return rc;
    FL_REQUIRE(col_stat != nullptr, "col_stat is NULL");
    FL_REQUIRE(n_sink <= n_cand, "n_sink %d > n_cand %d", n_sink, n_cand);
    FL_HIP(timed("select_columns", st, [&] {
               return fl::launch_topk(col_stat, n_cand, cand_cols, cand_cols ? n_cand : 0, n_cand,
                                      k - n_sink, n_sink, sel_out, k, nullptr, 0, H, st);
           }),
           "topk");
    return FL_OK;
}

int fl_kv_residual_quant(const fl_kv_cache* cache, int level, int dtype, const void* k_new,
                         const void* v_new, int new_gathered, fl_stream_t stream) {
    int rc = check_cache(cache, level);
    if (rc) return rc;
    FL_REQUIRE(dtype_ok(dtype), "dtype %d", dtype);
    FL_REQUIRE(k_new && v_new, "k_new/v_new NULL");
    hipStream_t st = (hipStream_t)stream;
    rc = check_levels_dev(*cache, level, st);
    if (rc) return rc;
    FL_HIP(timed("kv_quant", st, [&] {
               return fl::launch_quant(*cache, level, dtype, k_new, v_new, new_gathered, st);
           }),
           "quant");
    return FL_OK;
}

int fl_kv_dequant(const fl_kv_cache* cache, int level, int which, float* out, fl_stream_t stream) {
    int rc = check_cache(cache, level);
    if (rc) return rc;
    FL_REQUIRE(which == 0 || which == 1, "which %d (0 keys, 1 values)", which);
    FL_REQUIRE(out && ((uintptr_t)out % 16) == 0, "out NULL or not 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    FL_HIP(timed("kv_dequant", st, [&] { return fl::launch_dequant(*cache, level, which, out, st); }),
           "kv_dequant");
    return FL_OK;
}

// fl_sparse_loop_attn, optionally also writing the output as bf16 [n][H][d]
// by active index (out_bf; the block step's input of the output projection)
static int sparse_loop_attn(const fl_kv_cache* cache, const fl_attn_args* a, void* ws,
                            size_t ws_bytes, fl_stream_t stream, __bf16* out_bf) {
    FL_REQUIRE(a != nullptr, "args NULL");
    int rc = check_cache(cache, a->level);
    if (rc) return rc;
    const int H = cache->H, d = cache->d, N = cache->N;
    FL_REQUIRE(dtype_ok(a->dtype), "dtype %d", a->dtype);
    FL_REQUIRE(a->q && a->active && a->out && a->lse, "q/active/out/lse NULL");
    FL_REQUIRE(a->n >= 1 && a->n <= N, "n=%d", a->n);
    FL_REQUIRE(a->k >= 1 && a->k <= N, "k=%d", a->k);
    FL_REQUIRE(a->sel || a->k == N, "sel NULL requires k == N");
    FL_REQUIRE(a->cache_op >= FL_CACHE_CARRY && a->cache_op <= FL_CACHE_REBUILD, "cache_op %d", a->cache_op);
    FL_REQUIRE(a->cache_op == FL_CACHE_ZERO || (a->mass_u && a->out_u), "mass_u/out_u NULL");
    if (a->cache_op == FL_CACHE_REBUILD) {
        FL_REQUIRE(a->level >= 1, "cache rebuild needs a previous loop (level >= 1)");
        FL_REQUIRE(a->q_prev != nullptr, "q_prev NULL");
        if (a->sel_prev)
            FL_REQUIRE(a->k_prev >= a->k && a->k_prev <= N, "k_prev %d not in [k=%d, N=%d]", a->k_prev,
                       a->k, N);
    }
    FL_REQUIRE(a->mode >= FL_DEQ_AUTO && a->mode <= FL_DEQ_IN_TILE, "mode %d", a->mode);
    FL_REQUIRE(a->col_stat_kind == FL_COL_STAT_MASS || a->col_stat_kind == FL_COL_STAT_VNORM,
               "col_stat_kind %d", a->col_stat_kind);
    {
        hipStream_t st0 = (hipStream_t)stream;
        rc = check_idx_dev(a->active, 1, a->n, 0, N, "active", st0);
        if (!rc) rc = check_idx_dev(a->sel, H, a->k, 0, N, "sel", st0);
        if (!rc && a->cache_op == FL_CACHE_REBUILD)
            rc = check_idx_dev(a->sel_prev, H, a->k_prev, 0, N, "sel_prev", st0);
        if (!rc) rc = check_levels_dev(*cache, a->level, st0);
        if (rc) return rc;
    }
    const int prec = attn_prec(a->dtype, a->level);
    const int prec_old = attn_prec(a->dtype, a->level - 1);
    // FL_DEQ_AUTO resolves to FL_DEQ_ONCE: on the 32K, 4-loop workload the
    // in-tile placement repeats the dequantisation for every 128-row query
    // tile and, with both on the LDS-DMA pipeline, measured 1.9x slower on
    // the dense loop (7.67 vs 4.11 ms) and 3.1x on the sparse loops' steps
    // a5-a8 (2.54 vs 0.82 ms).
    const bool in_tile = a->mode == FL_DEQ_IN_TILE;
    if (in_tile && cache->scheme != FL_QUANT_ABSMAX)
        return fail(FL_ERR_UNSUPPORTED, "FL_DEQ_IN_TILE needs a FL_QUANT_ABSMAX cache");
    if (in_tile)
        for (int l = 0; l <= a->level; ++l)
            if (cache->level[l].bits == 32)
                return fail(FL_ERR_UNSUPPORTED, "FL_DEQ_IN_TILE needs quantised levels (level %d is raw)", l);
    // Precision-adaptive operands (bf16 queries over a cache with residual
    // levels): columns and rows are classed per head, and only outlier rows
    // or columns take hi + lo operand pairs.  A rebuild after a sparse loop
    // takes the additive form over the pruned columns (it does not inherit
    // the previous loop's output error).
    const bool adapt = !in_tile && a->dtype == FL_BF16 && a->level >= 1;
    const bool adapt_old = !in_tile && a->dtype == FL_BF16 && a->level - 1 >= 1;
    const bool rebuild_add = a->cache_op == FL_CACHE_REBUILD && adapt_old && a->sel_prev;
    const int kcols = rebuild_add ? a->k_prev : a->k;
    const long need = in_tile ? attn_ws_bytes(H, kcols, d, a->n, a->level + 1)
                              : attn_ws_bytes_once(H, kcols, d, a->n);
    if (!ws || (long)ws_bytes < need)
        return fail(FL_ERR_WORKSPACE, "workspace %zu < %ld bytes", ws_bytes, need);
    hipStream_t st = (hipStream_t)stream;
    const int kp = (int)kslots(kcols);
    char* p = (char*)(((uintptr_t)ws + kAlign - 1) / kAlign * kAlign);
    auto take = [&](long bytes) { char* q = p; p += align_up(bytes); return q; };
    __bf16* buf[8];
    for (int i = 0; i < 8; ++i) buf[i] = (__bf16*)take((long)H * kp * d * 2);
    int32_t* cpos = (int32_t*)take((long)H * kp * 4);
    int32_t* cpos_old = (int32_t*)take((long)H * kp * 4);
    float* vnorm_buf = (float*)take((long)H * kp * 4);
    int32_t* perm = (int32_t*)take((long)H * kp * 4);
    int32_t* perm_old = (int32_t*)take((long)H * kp * 4);
    uint8_t* colflags = (uint8_t*)take((long)H * kp);
    int32_t* pruned = (int32_t*)take((long)H * kp * 4);
    int32_t* colseg = (int32_t*)take((long)H * 2 * 4);
    int32_t* colseg_old = (int32_t*)take((long)H * 2 * 4);
    uint8_t* rowflags = (uint8_t*)take((long)H * fl::class_row_stride(a->n));
    int32_t* rowperm = (int32_t*)take((long)H * a->n * 4);
    int32_t* rowperm_old = (int32_t*)take((long)H * a->n * 4);
    int32_t* rowseg = (int32_t*)take((long)H * 4);
    int32_t* rowseg_old = (int32_t*)take((long)H * 4);
    char* qbase = p;
    // value norms of the current loop's columns, written by its gather
    float* vn = (a->col_stat && a->col_stat_kind == FL_COL_STAT_VNORM) ? vnorm_buf : nullptr;
    // new side: K, V^T (+ lo parts); previous-loop side for a rebuild
    __bf16 *Kc = buf[0], *Vt = buf[1], *Kc_old = buf[2], *Vt_old = buf[3];
    __bf16 *Kl = buf[4], *Vl = buf[5], *Kl_old = buf[6], *Vl_old = buf[7];
    const float c2 = a->sm * 1.4426950408889634f;

    fl::AttnParams P{};
    P.H = H; P.n = a->n; P.k = a->k; P.kp = kp; P.dtype = a->dtype; P.cache_op = a->cache_op;
    P.c2 = c2; P.active = a->active; P.cpos = cpos;
    P.out = a->out; P.lse = a->lse; P.mass_u = a->mass_u; P.out_u = a->out_u; P.out_bf = out_bf;
    // one side's compact columns (and, adaptive, its column and row orders)
    // the current side's operand classes come from the cache's per-token
    // classes when the caller says they are those of this level
    const uint8_t* cls_cur = a->cls_current && cache->cls && cache->scheme == FL_QUANT_ABSMAX ? cache->cls : nullptr;
    auto prepare = [&](const int32_t* sel, int k, int upto, bool ad, int pr, const void* q, int q_gathered,
                       int32_t* cp, int32_t* pm, int32_t* cs, int32_t* rp, int32_t* rs, __bf16* K_, __bf16* V_,
                       __bf16* Kl_, __bf16* Vl_, float* vnorm, const uint8_t* cls_side) -> int {
        if (ad)
            FL_HIP(timed("classify", st, [&] {
                       return fl::launch_classify(*cache, upto, sel, k, kp, q, a->dtype, q_gathered,
                                                  a->active, a->n, fl::kTauCol, fl::kTauRow, colflags, pm,
                                                  cs, rowflags, rp, rs, cls_side, st);
                   }),
                   "classify");
        FL_HIP(timed("gather", st, [&] {
                   return fl::launch_gather_bf16(*cache, upto, sel, k, kp, ad || pr >= 1, K_, V_, Kl_,
                                                 Vl_, cp, vnorm, ad ? pm : nullptr, ad ? cs : nullptr, st);
               }),
               "gather");
        return FL_OK;
    };
    if (in_tile) {
        fl::QTiles& qt = P.qt;
        qt.n_levels = a->level + 1;
        qt.g = cache->g;
        char* q = qbase;
        const int G = d / cache->g;
        for (int l = 0; l <= a->level; ++l) {
            const int b = cache->level[l].bits;
            qt.bits[l] = b;
            qt.kq[l] = (uint8_t*)q; q += align_up((long)H * kp * d * b / 8);
            qt.ks[l] = (float*)q;   q += align_up((long)H * kp * G * 4);
            qt.vq[l] = (uint8_t*)q; q += align_up((long)H * kp * d * b / 8);
            qt.vs[l] = (float*)q;   q += align_up((long)H * kp * G * 4);
        }
        FL_HIP(timed("gather_q", st, [&] {
                   return fl::launch_gather_q(*cache, a->level, a->sel, a->k, kp, qt, cpos, st);
               }),
               "gather_q");
    } else {
        rc = prepare(a->sel, a->k, a->level, adapt, prec, a->q, a->q_gathered, cpos, perm, colseg, rowperm,
                     rowseg, Kc, Vt, Kl, Vl, vn, cls_cur);
        if (rc) return rc;
    }
    // After the dense first loop (previous side plain bf16, subtract form)
    // the rebuild runs inside the attention's workgroups, before their
    // attention pass (MODE_ATTN_RB): one launch, one prologue per row tile.
    const bool fuse_rb = a->cache_op == FL_CACHE_REBUILD && adapt && !adapt_old && !rebuild_add && !in_tile &&
                         prec_old == 0;
    if (a->cache_op == FL_CACHE_REBUILD) {
        fl::AttnParams R = P;
        if (in_tile) {
            R.deq_levels = a->level; // the previous loop's cache: levels 0..level-1
        } else {
            // additive form: the previous loop's side over the pruned columns
            const int32_t* osel = a->sel;
            int ok = a->k;
            if (rebuild_add) {
                FL_HIP(timed("prune_list", st, [&] {
                           return fl::launch_set_diff(a->sel_prev, a->k_prev, a->sel, a->k, H, pruned, st);
                       }),
                       "set_diff");
                osel = pruned;
                ok = a->k_prev - a->k;
            }
            if (ok > 0) {
                rc = prepare(osel, ok, a->level - 1, adapt_old, prec_old, a->q_prev, a->q_prev_gathered, cpos_old,
                             perm_old, colseg_old, rowperm_old, rowseg_old, Kc_old, Vt_old, Kl_old, Vl_old,
                             nullptr, nullptr);
                if (rc) return rc;
            }
            R.k = ok;
            R.Kc = Kc_old; R.Vt = Vt_old; R.Kc_lo = Kl_old; R.Vt_lo = Vl_old; R.cpos = cpos_old;
        }
        R.q = a->q_prev; R.q_gathered = a->q_prev_gathered;
        if (fuse_rb) {
            P.Kc_old = R.Kc; P.Vt_old = R.Vt; P.cpos_old = R.cpos; P.k_old = R.k;
            P.q_old = a->q_prev; P.q_old_gathered = a->q_prev_gathered;
        } else if (adapt_old) {
            R.rowperm = rowperm_old; R.rowseg = rowseg_old; R.colseg = colseg_old;
            if (R.k > 0 || !rebuild_add)
                FL_HIP(timed(rebuild_add ? "attn_ad_rebuild_add" : "attn_ad_rebuild", st, [&] {
                           return fl::launch_attn_ad(d, rebuild_add ? fl::MODE_REBUILD_ADD : fl::MODE_REBUILD, R, st);
                       }),
                       "attn(rebuild)");
        } else {
            FL_HIP(timed(prec_old ? "attn_rebuild_split" : "attn_rebuild", st,
                         [&] { return fl::launch_attn(d, fl::MODE_REBUILD, prec_old, in_tile, R, st); }),
                   "attn(rebuild)");
        }
    }
    P.q = a->q; P.q_gathered = a->q_gathered; P.Kc = Kc; P.Vt = Vt; P.Kc_lo = Kl; P.Vt_lo = Vl;
    P.deq_levels = a->level + 1;
    // timing names follow the kernel: bf16 operands ("attn", the dense first
    // loop), precision-adaptive ("attn_ad"), hi/lo split ("attn_split")
    if (adapt) {
        P.rowperm = rowperm; P.rowseg = rowseg; P.colseg = colseg;
        if (fuse_rb)
            FL_HIP(timed("attn_ad_rb", st, [&] { return fl::launch_attn_ad(d, fl::MODE_ATTN_RB, P, st); }),
                   "attn");
        else
            FL_HIP(timed("attn_ad", st, [&] { return fl::launch_attn_ad(d, fl::MODE_ATTN, P, st); }), "attn");
    } else {
        FL_HIP(timed(prec ? "attn_split" : "attn", st,
                     [&] { return fl::launch_attn(d, fl::MODE_ATTN, prec, in_tile, P, st); }),
               "attn");
    }
    if (a->col_stat) {
        if (in_tile) // the statistics sweep reads the keys as compact bf16
            FL_HIP(timed("gather", st, [&] {
                       return fl::launch_gather_bf16(*cache, a->level, a->sel, a->k, kp, prec >= 1, Kc,
                                                     Vt, Kl, Vl, cpos, vn, nullptr, nullptr, st);
                   }),
                   "gather");
        fl::ColParams C{};
        C.H = H; C.n = a->n; C.k = a->k; C.kp = kp; C.dtype = a->dtype; C.q_gathered = a->q_gathered;
        C.cache_op = a->cache_op == FL_CACHE_ZERO ? FL_CACHE_ZERO : FL_CACHE_CARRY;
        C.c2 = c2; C.q = a->q; C.active = a->active; C.Kc = Kc; C.Kc_lo = Kl; C.cpos = cpos;
        C.lse = a->lse; C.mass_u = a->mass_u; C.col_stat = a->col_stat; C.vnorm = vn;
        C.perm = adapt ? perm : nullptr;
        const int cprec = adapt ? 1 : prec;
        FL_HIP(timed(cprec ? "colstat_split" : "colstat", st,
                     [&] { return fl::launch_colstat(d, cprec, C, st); }),
               "colstat");
    }
    return FL_OK;
}

int fl_sparse_loop_attn(const fl_kv_cache* cache, const fl_attn_args* a, void* ws,
                        size_t ws_bytes, fl_stream_t stream) {
    return sparse_loop_attn(cache, a, ws, ws_bytes, stream, nullptr);
}

} // extern "C"

// Scratch of fl_sparse_loop_attn_noalloc: one copy per GPU the library runs
// on, for the life of the process.  In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) char scratch[FL_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's scratch address (looked up once per device)
int scratch_of_current_device(void** out) {
    int dev = -1;
    FL_HIP(hipGetDevice(&dev), "hipGetDevice");
    FL_REQUIRE(dev >= 0 && dev < kMaxDevices, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        FL_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        FL_REQUIRE(p != nullptr, "scratch address of device %d is NULL", dev);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FL_OK;
}

struct NoEvents {
    NoEvents() { g_no_events = true; }
    ~NoEvents() { g_no_events = false; }
};
} // namespace

extern "C" {

int fl_sparse_loop_attn_noalloc(const fl_kv_cache* cache, const fl_attn_args* a, fl_stream_t stream) {
    void* ws = nullptr;
    const int rc = scratch_of_current_device(&ws);
    if (rc) return rc;
    NoEvents guard;
    return sparse_loop_attn(cache, a, ws, (size_t)FL_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

// Phase events of fl_loop_step: e0 opens steps a1-a4 at the call's start;
// at the split point (after the quantisation) it is closed and `mark` opens
// steps a5-a8, which the caller closes at the end of the loop.
struct LoopPhases {
    hipEvent_t e0 = nullptr, mark = nullptr;
    std::string tag;
    void split(hipStream_t st) {
        if (g_phases) g_prefix = tag + ".a5-a8/";
        if (!e0) return;
        phase_end(e0, tag + ".a1-a4", st);
        e0 = nullptr;
        mark = phase_begin(st);
    }
    void release() {
        g_prefix.clear();
        std::lock_guard<std::mutex> lk(g_tmu);
        if (e0) g_pool.push_back(e0);
        if (mark) g_pool.push_back(mark);
        e0 = mark = nullptr;
    }
};

static int loop_step(const fl_loop_cfg* cfg, fl_loop_state* S, const fl_loop_inputs* in, int r,
                     void* ws, size_t ws_bytes, fl_stream_t stream, LoopPhases& ph);

int fl_loop_step(const fl_loop_cfg* cfg, fl_loop_state* S, const fl_loop_inputs* in, int r,
                 void* ws, size_t ws_bytes, fl_stream_t stream) {
    hipStream_t st = (hipStream_t)stream;
    LoopPhases ph;
    ph.tag = "loop" + std::to_string(r);
    ph.e0 = phase_begin(st);
    if (g_phases) g_prefix = ph.tag + ".a1-a4/";
    const int rc = loop_step(cfg, S, in, r, ws, ws_bytes, stream, ph);
    if (rc == FL_OK && ph.mark) {
        phase_end(ph.mark, ph.tag + ".a5-a8", st);
        ph.mark = nullptr;
    }
    ph.release();
    return rc;
}

static int loop_step(const fl_loop_cfg* cfg, fl_loop_state* S, const fl_loop_inputs* in, int r,
                     void* ws, size_t ws_bytes, fl_stream_t stream, LoopPhases& ph) {
    FL_REQUIRE(cfg && S && in, "cfg/state/inputs NULL");
    FL_REQUIRE(r >= 1 && r <= cfg->R && cfg->R <= FL_MAX_LEVELS, "loop %d of R=%d", r, cfg->R);
    FL_REQUIRE(stat_kinds_ok(cfg->token_stat, cfg->col_stat), "token_stat %d / col_stat %d",
               cfg->token_stat, cfg->col_stat);
    const int N = cfg->N, H = cfg->H, d = cfg->d;
    fl_kv_cache& C = S->cache;
    FL_REQUIRE(C.N == N && C.H == H && C.d == d && C.g == cfg->g, "cache dims differ from cfg");
    FL_REQUIRE(in->q && in->k && in->v, "q/k/v NULL");
    FL_REQUIRE(S->out && S->lse && S->mass_u && S->out_u, "state arrays NULL");
    hipStream_t st = (hipStream_t)stream;
    const float sm = 1.0f / sqrtf((float)d);
    fl_attn_args A{};
    A.cls_current = 1;  // this loop's quantisation precedes its attention
    A.dtype = cfg->dtype; A.q = in->q; A.q_gathered = 0; A.sm = sm; A.mode = cfg->mode;
    A.col_stat_kind = cfg->col_stat;
    A.out = S->out; A.lse = S->lse; A.mass_u = S->mass_u; A.out_u = S->out_u;
    if (r == 1) {
        FL_REQUIRE(S->active[0] != nullptr, "active[0] (iota buffer) NULL");
        C.level[0].bits = cfg->bits[0];
        C.level[0].n_rows = N;
        C.level[0].rows = nullptr; C.level[0].slot = nullptr;
        C.n_levels = 1;
        int rc = fl_kv_residual_quant(&C, 0, cfg->dtype, in->k, in->v, 0, stream);
        if (rc) return rc;
        FL_HIP(fl::launch_copy_or_iota(nullptr, S->active[0], N, N, st), "iota");
        // M_U = 0 after the dense loop; O_U is zeroed only if a later loop
        // carries it over without a rebuild (see below)
        FL_HIP(fl::launch_fill_f32(S->mass_u, (long)N * H, 0.0f, st), "fill");
        ph.split(st);
        S->k_cur[0] = N;
        S->sel_used[0] = nullptr;
        A.active = S->active[0]; A.n = N; A.sel = nullptr; A.k = N; A.level = 0;
        A.cache_op = FL_CACHE_ZERO;
        A.col_stat = (cfg->R > 1 && cfg->k_cols[1] < N) ? S->col_stat[0] : nullptr;
        return fl_sparse_loop_attn(&C, &A, ws, ws_bytes, stream);
    }
    FL_REQUIRE(in->h_cur && in->h_prev && in->q_prev, "h_cur/h_prev/q_prev NULL");
    const int n_prev = r == 2 ? N : cfg->n_active[r - 2];
    const int n_r = cfg->n_active[r - 1];
    FL_REQUIRE(n_r >= 1 && n_r <= n_prev, "n_active[%d] = %d (prev %d)", r - 1, n_r, n_prev);
    FL_REQUIRE(S->active[r - 1] && S->slot[r - 1] && S->stat, "active/slot/stat buffers NULL");
    int rc = fl_select_active(cfg->dtype, cfg->token_stat, in->h_cur, in->h_prev, N, H * d,
                              S->active[r - 2], n_prev,
                              n_r, nullptr, S->stat, S->active[r - 1], S->slot[r - 1], ws, ws_bytes,
                              stream);
    if (rc) return rc;
    fl_kv_level& L = C.level[r - 1];
    L.bits = cfg->bits[r - 1];
    L.n_rows = n_r;
    L.rows = S->active[r - 1];
    L.slot = S->slot[r - 1];
    C.n_levels = r;
    rc = fl_kv_residual_quant(&C, r - 1, cfg->dtype, in->k, in->v, 0, stream);
    if (rc) return rc;
    ph.split(st);
    const int k_prev = S->k_cur[r - 2];
    const int k_r = cfg->k_cols[r - 1];
    bool changed = false;
    if (k_prev <= k_r) {
        S->k_cur[r - 1] = k_prev;
        S->sel_used[r - 1] = S->sel_used[r - 2];
        // every loop so far attended all columns: O_U = 0 is carried
        if (!S->sel_used[r - 1])
            FL_HIP(fl::launch_fill_f32(S->out_u, (long)N * H * d, 0.0f, st), "fill");
    } else {
        FL_REQUIRE(S->sel[r - 1] && S->col_stat[r - 2], "sel/col_stat buffers NULL");
        rc = fl_select_columns(S->col_stat[r - 2], S->sel_used[r - 2], H, k_prev, cfg->n_sink, k_r,
                               S->sel[r - 1], ws, ws_bytes, stream);
        if (rc) return rc;
        S->k_cur[r - 1] = k_r;
        S->sel_used[r - 1] = S->sel[r - 1];
        changed = true;
    }
    A.active = S->active[r - 1]; A.n = n_r;
    A.sel = S->sel_used[r - 1]; A.k = S->k_cur[r - 1]; A.level = r - 1;
    A.cache_op = changed ? FL_CACHE_REBUILD : FL_CACHE_CARRY;
    A.q_prev = in->q_prev; A.q_prev_gathered = 0;
    A.sel_prev = S->sel_used[r - 2]; A.k_prev = k_prev;
    const bool need_c = r < cfg->R && cfg->k_cols[r] < S->k_cur[r - 1];
    A.col_stat = need_c ? S->col_stat[r - 1] : nullptr;
    FL_REQUIRE(!need_c || A.col_stat, "col_stat[%d] buffer NULL", r - 1);
    return fl_sparse_loop_attn(&C, &A, ws, ws_bytes, stream);
}

int fl_block_step(const fl_block_cfg* cfg, const fl_layer_weights* W, fl_block_state* S, int r,
                  void* ws, size_t ws_bytes, fl_stream_t stream) {
    FL_REQUIRE(cfg && W && S && S->layers, "cfg/weights/state NULL");
    FL_REQUIRE(r >= 1 && r <= cfg->R && cfg->R <= FL_MAX_LEVELS, "loop %d of R=%d", r, cfg->R);
    const int N = cfg->N, H = cfg->H, d = cfg->d, D = H * d, F = cfg->ffn, L = cfg->n_layers;
    FL_REQUIRE(N > 0 && L >= 1, "N=%d layers=%d", N, L);
    FL_REQUIRE(stat_kinds_ok(cfg->token_stat, cfg->col_stat), "token_stat %d / col_stat %d",
               cfg->token_stat, cfg->col_stat);
    FL_REQUIRE(cfg->mode == FL_DEQ_AUTO || cfg->mode == FL_DEQ_ONCE || cfg->mode == FL_DEQ_IN_TILE,
               "mode %d", cfg->mode);
    if (cfg->mode == FL_DEQ_IN_TILE)
        return fail(FL_ERR_UNSUPPORTED, "fl_block_step uses the compact-gather path (FL_DEQ_ONCE)");
    if (!(d == 64 || d == 128)) return fail(FL_ERR_UNSUPPORTED, "head dim %d", d);
    if (D % 128 || F % 128) return fail(FL_ERR_UNSUPPORTED, "D=%d and ffn=%d must be multiples of 128", D, F);
    FL_REQUIRE(S->h && S->h_entry && S->stat, "h/h_entry/stat NULL");
    const long need = block_ws_bytes(N, H, d, F);
    if (!ws || (long)ws_bytes < need)
        return fail(FL_ERR_WORKSPACE, "workspace %zu < %ld bytes", ws_bytes, need);
    hipStream_t st = (hipStream_t)stream;
    char* p = (char*)(((uintptr_t)ws + kAlign - 1) / kAlign * kAlign);
    auto take = [&](long bytes) { char* q = p; p += align_up(bytes); return q; };
    __bf16* a_buf = (__bf16*)take((long)N * D * 2);
    __bf16* qc = (__bf16*)take((long)N * D * 2);
    __bf16* kc = (__bf16*)take((long)N * D * 2);
    __bf16* vc = (__bf16*)take((long)N * D * 2);
    __bf16* attn_in = (__bf16*)take((long)N * D * 2);
    __bf16* qkv = (__bf16*)take((long)N * 3 * D * 2);
    __bf16* act_buf = (__bf16*)take((long)N * F * 2);
    void* aws = p;
    const size_t aws_bytes = (size_t)attn_ws_bytes_once(H, N, d, N);

    // ---- the loop's active tokens (Sec. 4.1) ----
    int n;
    if (r == 1) {
        FL_REQUIRE(S->active[0] != nullptr, "active[0] (iota buffer) NULL");
        FL_HIP(fl::launch_copy_or_iota(nullptr, S->active[0], N, N, st), "iota");
        n = N;
    } else {
        const int n_prev = r == 2 ? N : cfg->n_active[r - 2];
        n = cfg->n_active[r - 1];
        FL_REQUIRE(n >= 1 && n <= n_prev, "n_active[%d] = %d (prev %d)", r - 1, n, n_prev);
        FL_REQUIRE(S->active[r - 1] && S->slot[r - 1], "active/slot buffers NULL");
        int rc = fl_select_active(FL_F32, cfg->token_stat, S->h, S->h_entry, N, D, S->active[r - 2],
                                  n_prev, n, nullptr,
                                  S->stat, S->active[r - 1], S->slot[r - 1], nullptr, 0, stream);
        if (rc) return rc;
    }
    const int32_t* act = S->active[r - 1];
    FL_HIP(hipMemcpyAsync(S->h_entry, S->h, (size_t)N * D * 4, hipMemcpyDeviceToDevice, st), "copy");

    const float sm = 1.0f / sqrtf((float)d);
    for (int l = 0; l < L; ++l) {
        const fl_layer_weights& w = W[l];
        fl_layer_state& Ls = S->layers[l];
        FL_REQUIRE(w.w_qkv && w.w_o && w.w_gu && w.w_down && w.norm1 && w.norm2, "layer %d weights NULL", l);
        FL_REQUIRE(Ls.q_state && Ls.out && Ls.lse && Ls.mass_u && Ls.out_u, "layer %d state NULL", l);
        fl_kv_cache& C = Ls.cache;
        FL_REQUIRE(C.N == N && C.H == H && C.d == d && C.g == cfg->g, "layer %d cache dims", l);
        // attention sub-block on the active rows
        FL_HIP(timed("rmsnorm", st, [&] {
                   return fl::launch_rmsnorm_gather(S->h, act, n, D, (const __bf16*)w.norm1,
                                                    cfg->norm_eps, a_buf, st);
               }), "rmsnorm");
        fl::GemmParams G{};
        G.M = n; G.N = 3 * D; G.K = D; G.A = a_buf; G.lda = D; G.B = (const __bf16*)w.w_qkv;
        G.Cb = qkv; G.ldc = 3 * D;
        FL_HIP(timed(gemm_name(kGemmQkv, G), st, [&] { return fl::launch_gemm(fl::EPI_STORE, G, st); }), "gemm");
        FL_HIP(timed("rope", st, [&] {
                   return fl::launch_rope_split(qkv, act, n, H, d, cfg->rope_theta, qc, kc, vc, st);
               }), "rope");
        // K/V cache level of this loop (keys after RoPE)
        if (r == 1) {
            C.level[0].bits = cfg->bits[0];
            C.level[0].n_rows = N;
            C.level[0].rows = nullptr;
            C.level[0].slot = nullptr;
            C.n_levels = 1;
            // M_U = 0 after the dense loop; O_U is zeroed only if a later
            // loop carries it over without a rebuild
            FL_HIP(fl::launch_fill_f32(Ls.mass_u, (long)N * H, 0.0f, st), "fill");
        } else {
            fl_kv_level& Lv = C.level[r - 1];
            Lv.bits = cfg->bits[r - 1];
            Lv.n_rows = n;
            Lv.rows = act;
            Lv.slot = S->slot[r - 1];
            C.n_levels = r;
        }
        if (Ls.k_in)
            FL_HIP(hipMemcpyAsync(Ls.k_in, kc, (size_t)n * D * 2, hipMemcpyDeviceToDevice, st), "copy");
        if (Ls.v_in)
            FL_HIP(hipMemcpyAsync(Ls.v_in, vc, (size_t)n * D * 2, hipMemcpyDeviceToDevice, st), "copy");
        int rc = fl_kv_residual_quant(&C, r - 1, FL_BF16, kc, vc, 1, stream);
        if (rc) return rc;
        fl_attn_args A{};
        A.cls_current = 1;  // this loop's quantisation precedes its attention
        A.dtype = FL_BF16; A.q = qc; A.q_gathered = 1; A.active = act; A.n = n; A.sm = sm;
        A.level = r - 1; A.mode = cfg->mode; A.col_stat_kind = cfg->col_stat;
        A.out = Ls.out; A.lse = Ls.lse; A.mass_u = Ls.mass_u; A.out_u = Ls.out_u;
        A.q_prev = Ls.q_state; A.q_prev_gathered = 0;
        if (r == 1) {
            Ls.k_cur[0] = N;
            Ls.sel_used[0] = nullptr;
            A.sel = nullptr; A.k = N; A.cache_op = FL_CACHE_ZERO;
            A.col_stat = (cfg->R > 1 && cfg->k_cols[1] < N) ? Ls.col_stat[0] : nullptr;
        } else {
            const int k_prev = Ls.k_cur[r - 2], k_r = cfg->k_cols[r - 1];
            bool changed = false;
            if (k_prev <= k_r) {
                Ls.k_cur[r - 1] = k_prev;
                Ls.sel_used[r - 1] = Ls.sel_used[r - 2];
                if (!Ls.sel_used[r - 1])
                    FL_HIP(fl::launch_fill_f32(Ls.out_u, (long)N * H * d, 0.0f, st), "fill");
            } else {
                FL_REQUIRE(Ls.sel[r - 1] && Ls.col_stat[r - 2], "layer %d sel/col_stat buffers NULL", l);
                rc = fl_select_columns(Ls.col_stat[r - 2], Ls.sel_used[r - 2], H, k_prev, cfg->n_sink,
                                       k_r, Ls.sel[r - 1], nullptr, 0, stream);
                if (rc) return rc;
                Ls.k_cur[r - 1] = k_r;
                Ls.sel_used[r - 1] = Ls.sel[r - 1];
                changed = true;
            }
            A.sel = Ls.sel_used[r - 1]; A.k = Ls.k_cur[r - 1];
            A.cache_op = changed ? FL_CACHE_REBUILD : FL_CACHE_CARRY;
            A.sel_prev = Ls.sel_used[r - 2]; A.k_prev = k_prev;
            const bool need_c = r < cfg->R && cfg->k_cols[r] < Ls.k_cur[r - 1];
            A.col_stat = need_c ? Ls.col_stat[r - 1] : nullptr;
            FL_REQUIRE(!need_c || A.col_stat, "layer %d col_stat[%d] NULL", l, r - 1);
        }
        // the attention output lands in the state (fp32, by position) and as the
        // bf16 compact input of the output projection
        rc = sparse_loop_attn(&C, &A, aws, aws_bytes, stream, attn_in);
        if (rc) return rc;
        FL_HIP(fl::launch_scatter_rows_bf16(qc, act, n, D, (__bf16*)Ls.q_state, st), "scatter");
        G = fl::GemmParams{};
        G.M = n; G.N = D; G.K = D; G.A = attn_in; G.lda = D; G.B = (const __bf16*)w.w_o;
        G.Cf = S->h; G.ldc = D; G.rows = act;
        FL_HIP(timed(gemm_name(kGemmO, G), st, [&] { return fl::launch_gemm(fl::EPI_RESID, G, st); }), "gemm");
        // MLP sub-block
        FL_HIP(timed("rmsnorm", st, [&] {
                   return fl::launch_rmsnorm_gather(S->h, act, n, D, (const __bf16*)w.norm2,
                                                    cfg->norm_eps, a_buf, st);
               }), "rmsnorm");
        G = fl::GemmParams{};
        G.M = n; G.N = 2 * F; G.K = D; G.A = a_buf; G.lda = D; G.B = (const __bf16*)w.w_gu;
        G.Cb = act_buf; G.ldc = F;
        FL_HIP(timed(gemm_name(kGemmGateUp, G), st, [&] { return fl::launch_gemm(fl::EPI_SWIGLU, G, st); }), "gemm");
        G = fl::GemmParams{};
        G.M = n; G.N = D; G.K = F; G.A = act_buf; G.lda = F; G.B = (const __bf16*)w.w_down;
        G.Cf = S->h; G.ldc = D; G.rows = act;
        FL_HIP(timed(gemm_name(kGemmDown, G), st, [&] { return fl::launch_gemm(fl::EPI_RESID, G, st); }), "gemm");
    }
    return FL_OK;
}

int fl_decode_step(const fl_decode_cfg* cfg, fl_decode_state* S, const fl_decode_inputs* in,
                   int r, fl_stream_t stream) {
    FL_REQUIRE(cfg && S && in, "cfg/state/inputs NULL");
    FL_REQUIRE(r >= 1 && r <= cfg->R && cfg->R <= FL_MAX_LEVELS, "loop %d of R=%d", r, cfg->R);
    const int B = cfg->B, N = cfg->N, H = cfg->H, d = cfg->d;
    FL_REQUIRE(B >= 1 && N >= 1 && H >= 1, "B=%d N=%d H=%d", B, N, H);
    const fl_decode_window* W = in->win;
    if (W) {
        FL_REQUIRE(W->cap >= 1 && W->count >= 1 && W->count <= W->cap, "window count %d / cap %d",
                   W->count, W->cap);
        FL_REQUIRE(W->start >= 0 && W->start < W->cap, "window start %d / cap %d", W->start, W->cap);
        for (int l = (r >= 2 ? r - 2 : 0); l < r; ++l)
            FL_REQUIRE(W->k[l] && W->v[l], "window buffers of loop %d NULL", l + 1);
    }
    const int T = W ? W->count : 1;
    FL_REQUIRE(N + T <= 12288, "N=%d + %d bf16 columns: decode keeps the probabilities in LDS (<= 12288)",
               N, T);
    fl_kv_cache& C = S->cache;
    FL_REQUIRE(C.N == N && C.H == H && C.d == d && C.g == cfg->g, "cache dims differ from cfg");
    int rc = check_cache(&C, r - 1);
    if (rc) return rc;
    if (C.scheme == FL_QUANT_ABSMAX && C.level[0].bits != 8)
        return fail(FL_ERR_UNSUPPORTED, "decode: base level bits %d (8)", C.level[0].bits);
    for (int l = 1; l < r; ++l)
        if (C.level[l].bits == 32)
            return fail(FL_ERR_UNSUPPORTED, "decode: level %d is raw (quantised levels only)", l);
    FL_REQUIRE(in->q && (W || (in->k_self && in->v_self)), "q/k_self/v_self NULL");
    FL_REQUIRE(S->out && S->lse && S->mass_u && S->out_u, "state arrays NULL");
    hipStream_t st = (hipStream_t)stream;
    fl::DecodeParams P{};
    rc = decode_caps(cfg, C, r - 1, P);
    if (rc) return rc;
    P.B = B; P.H = H; P.sm = 1.0f / sqrtf((float)d); P.cache = C;
    P.out = S->out; P.lse = S->lse; P.mass_u = S->mass_u; P.out_u = S->out_u;
    P.n_tail = T;
    P.tail_cap = W ? W->cap : 1;
    P.tail_start = W ? W->start : 0;
    // the bf16 columns of loop r (and r - 1, for a rebuild)
    auto tails = [&](fl::DecodeParams& Q, int loop, const void* ks, const void* vs) {
        Q.tail_k = W ? W->k[loop - 1] : ks;
        Q.tail_v = W ? W->v[loop - 1] : vs;
    };
    if (r == 1) {
        S->k_cur[0] = N;
        S->sel_used[0] = nullptr;
        P.k = N; P.sel = nullptr; P.level = 0; P.cache_op = FL_CACHE_ZERO;
        P.q = in->q;
        tails(P, 1, in->k_self, in->v_self);
        P.col_stat = (cfg->R > 1 && cfg->k_cols[1] < N) ? S->col_stat[0] : nullptr;
        FL_HIP(fl::launch_fill_f32(S->mass_u, (long)B * H, 0.0f, st), "fill");
        FL_HIP(fl::launch_fill_f32(S->out_u, (long)B * H * d, 0.0f, st), "fill");
        FL_HIP(timed("decode_dense", st, [&] { return fl::launch_decode(d, fl::MODE_ATTN, P, st); }),
               "decode");
        return FL_OK;
    }
    FL_REQUIRE(in->q_prev && (W || (in->k_self_prev && in->v_self_prev)), "previous-loop inputs NULL");
    const int k_prev = S->k_cur[r - 2], k_r = cfg->k_cols[r - 1];
    bool changed = false;
    if (k_prev <= k_r) {
        S->k_cur[r - 1] = k_prev;
        S->sel_used[r - 1] = S->sel_used[r - 2];
    } else {
        FL_REQUIRE(S->sel[r - 1] && S->col_stat[r - 2], "sel/col_stat buffers NULL");
        rc = fl_select_columns(S->col_stat[r - 2], S->sel_used[r - 2], B * H, k_prev, cfg->n_sink, k_r,
                               S->sel[r - 1], nullptr, 0, stream);
        if (rc) return rc;
        S->k_cur[r - 1] = k_r;
        S->sel_used[r - 1] = S->sel[r - 1];
        changed = true;
    }
    P.k = S->k_cur[r - 1];
    P.sel = S->sel_used[r - 1];
    rc = check_idx_dev(P.sel, (long)B * H, P.k, 0, N, "sel", st);
    if (!rc) rc = check_levels_dev(C, r - 1, st);
    if (rc) return rc;
    // a sparse loop keeps the probabilities and every level's row of each
    // selected column in LDS
    if (P.sel && (size_t)(P.k + T) * 4 + (size_t)r * P.k * 4 > 48 * 1024)
        return fail(FL_ERR_UNSUPPORTED, "decode: %d columns x %d levels exceed the LDS budget", P.k, r);
    if (changed) {
        fl::DecodeParams R = P;
        R.level = r - 2; R.cache_op = FL_CACHE_REBUILD;
        R.q = in->q_prev; R.col_stat = nullptr;
        tails(R, r - 1, in->k_self_prev, in->v_self_prev);
        FL_HIP(timed("decode_rebuild", st, [&] { return fl::launch_decode(d, fl::MODE_REBUILD, R, st); }),
               "decode(rebuild)");
    }
    P.level = r - 1; P.cache_op = FL_CACHE_CARRY;
    P.q = in->q;
    tails(P, r, in->k_self, in->v_self);
    const bool need_c = r < cfg->R && cfg->k_cols[r] < S->k_cur[r - 1];
    P.col_stat = need_c ? S->col_stat[r - 1] : nullptr;
    FL_REQUIRE(!need_c || P.col_stat, "col_stat[%d] NULL", r - 1);
    FL_HIP(timed(P.sel ? "decode" : "decode_dense", st,
                 [&] { return fl::launch_decode(d, fl::MODE_ATTN, P, st); }), "decode");
    return FL_OK;
}

int fl_decode_append(fl_decode_cfg* cfg, fl_decode_state* S, const fl_decode_window* W, int slot,
                     int n, fl_stream_t stream) {
    FL_REQUIRE(cfg && S && W, "cfg/state/window NULL");
    const int B = cfg->B, N = cfg->N, H = cfg->H, d = cfg->d, R = cfg->R;
    FL_REQUIRE(B >= 1 && R >= 1 && R <= FL_MAX_LEVELS, "B=%d R=%d", B, R);
    fl_kv_cache& C = S->cache;
    FL_REQUIRE(C.N == N && C.H == H && C.d == d && C.g == cfg->g, "cache dims differ from cfg");
    int rc = check_cache(&C, R - 1);
    if (rc) return rc;
    const bool asym = C.scheme == FL_QUANT_ASYM;
    if (!asym && C.level[0].bits != 8)
        return fail(FL_ERR_UNSUPPORTED, "append: FL_QUANT_ABSMAX caches with an int8 base only");
    for (int l = 1; l < R; ++l)
        if (C.level[l].bits == 32)
            return fail(FL_ERR_UNSUPPORTED, "append: level %d is raw (quantised levels only)", l);
    if (asym && n != C.g)
        return fail(FL_ERR_UNSUPPORTED, "append: FL_QUANT_ASYM appends one key group (n = g = %d, not %d)",
                    C.g, n);
    FL_REQUIRE(n >= 1 && n <= W->cap, "append: %d tokens from a window of %d", n, W->cap);
    FL_REQUIRE(slot >= 0 && slot < W->cap, "slot %d outside the window of %d", slot, W->cap);
    for (int l = 0; l < R; ++l) FL_REQUIRE(W->k[l] && W->v[l], "window buffers of loop %d NULL", l + 1);
    fl::DecodeParams caps{};
    rc = decode_caps(cfg, C, R - 1, caps);
    if (rc) return rc;
    FL_REQUIRE(N + n <= caps.pos_cap, "append: N_cap %d reached", caps.pos_cap);
    fl::AppendParams P{};
    P.B = B; P.H = H; P.g = C.g; P.R = R; P.pos = N; P.slot = slot; P.n = n; P.win_cap = W->cap;
    P.pos_cap = caps.pos_cap;
    for (int l = 0; l < R; ++l) {
        P.lev[l] = C.level[l];
        P.bits[l] = C.level[l].bits;
        P.wk[l] = W->k[l];
        P.wv[l] = W->v[l];
        P.kg_pad[l] = caps.kg_pad[l];
        P.kg_count[l] = caps.kg_count[l];
        const int row0 = l == 0 ? N : C.level[l].n_rows;
        if (l >= 1) {
            P.rows_cap[l] = caps.rows_cap[l];
            P.n_rows[l] = row0;
            FL_REQUIRE(row0 + n <= caps.rows_cap[l], "append: level %d rows_cap %d reached", l,
                       caps.rows_cap[l]);
        }
        if (asym)
            FL_REQUIRE(row0 >= caps.kg_origin[l] && (row0 - caps.kg_origin[l]) % C.g == 0,
                       "append: level %d row %d does not start a key group (key_group_origin %d, g %d)", l,
                       row0, caps.kg_origin[l], C.g);
    }
    hipStream_t st = (hipStream_t)stream;
    FL_HIP(timed("decode_append", st, [&] { return fl::launch_decode_append(d, C.scheme, P, st); }),
           "append");
    cfg->N = N + n;
    C.N = N + n;
    for (int l = 1; l < R; ++l) C.level[l].n_rows += n;
    return FL_OK;
}

} // extern "C"

namespace fl {
__global__ void k_fill_f32(float* p, long n, float v) {
    const long i = blockIdx.x * (long)blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}
hipError_t launch_fill_f32(float* p, long n, float v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}
} // namespace fl

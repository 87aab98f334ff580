/*
 * flashloop.h -- C ABI of the MI355X (gfx950) FlashLoop lazy-update loop
 * attention library (libflashloop.so).
 *
 * Method: "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
 * Updates" (arXiv 2609.29812).  One call sequence per loop r of a looped
 * (weight-shared, R-times repeated) Transformer layer:
 *   fl_select_active      Sec. 4.1  token-change statistic + nested top-k
 *   fl_kv_residual_quant  Sec. 3.3, 4.3, App. E  int8 base / int4,int2 residual
 *   fl_select_columns     Sec. 4.2  column ranking from the previous loop
 *   fl_sparse_loop_attn   Sec. 4.2  sparse attention with cached pruned mass
 *   fl_loop_step          Sec. 4.1-4.3  one whole loop (the four above)
 *
 * Conventions (all entry points):
 *  - Return FL_OK (0) or a negative FL_ERR_*; fl_last_error() gives a
 *    thread-local message for the last failure on the calling thread.
 *  - Arguments are validated on the host before anything is enqueued; a call
 *    that fails validation has no side effects.
 *  - Tensor pointers are DEVICE pointers owned by the caller; the library
 *    never frees them and keeps no reference after the call returns.  Work is
 *    enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *    stream); outputs are valid in stream order.  No call synchronises the
 *    device with the host.
 *  - Scratch memory comes from a caller workspace sized by fl_workspace_size.
 *  - Layouts are row-major.  Per-token tensors are [N][H][d] indexed by token
 *    position; per-row loop state (out, lse, mass_u, out_u) is also indexed by
 *    token position ([N][H][d] / [N][H]) so that rows that are inactive in a
 *    loop keep the values of the last loop that computed them.
 *  - Index lists are int32, ascending, unique.
 *  - Supported shapes: d in {64, 128}; g in {32, 64} dividing d; H*d <= 8192.
 */
#ifndef FLASHLOOP_H
#define FLASHLOOP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FL_VERSION_MAJOR 0
#define FL_VERSION_MINOR 1

typedef void* fl_stream_t; /* hipStream_t */

enum fl_status {
    FL_OK = 0,
    FL_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shapes */
    FL_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. d = 96)   */
    FL_ERR_WORKSPACE = -3,   /* workspace smaller than fl_workspace_size  */
    FL_ERR_HIP = -4          /* a HIP runtime call failed                 */
};

enum fl_dtype { FL_F32 = 0, FL_BF16 = 1 };

#define FL_MAX_LEVELS 32

/* One level of the loop-indexed KV cache (paper Sec. 3.3 / 4.3: a quantised
 * base state plus quantised cross-loop residuals; residuals exist only for
 * the tokens active in that loop).
 *   level 0 (loop 1): all N tokens, bits 8 (int8) or 32 (raw fp32).
 *   level l >= 1 (loop l+1): the n_rows tokens active in loop l+1 (ascending
 *   positions `rows`, and `slot` mapping position -> packed row or -1),
 *   bits 4, 2, 8 or 32.
 * Codes: two's complement, per (row, head) d*bits/8 bytes; int4 holds the
 * even channel in the low nibble, int2 holds channel c at bits 2*(c mod 4);
 * bits 32 stores the raw fp32 values (residuals) instead of codes.
 * Scales: fp32 [n_rows][H][d/g], one per group of g contiguous channels
 * (unused for bits 32).  The dequantised value of a token at loop r is
 *   xhat = code_0*s_0, then xhat = xhat + code_l*s_l for l = 1..r-1 while the
 * token is present in level l (sets are nested, so presence stops at the first
 * absent level).
 *
 * Scheme FL_QUANT_ASYM (the paper's own quantiser, App. E "Quantization
 * Setting": asymmetric min/max groups; post-RoPE keys per channel, values per
 * token) changes the format of every level:
 *   bits 2, 4 or 8 at every level (the paper uses 4), unsigned codes packed
 *   as above; per group z = min, s = (max - min)/(2^bits - 1), code =
 *   round-half-even((x - z)/s) clamped to [0, 2^bits - 1] (s = 0 -> 0), a zero
 *   z or s stored as +0; dequantised value code*s + z;
 *   values: groups of g contiguous channels of a (row, head):
 *     v_scale / v_zero [n_rows][H][d/g];
 *   keys: per (head, channel), groups of g consecutive rows of the level
 *     (packed order; the last group may be shorter):
 *     k_scale / k_zero [ceil(n_rows/g)][H][d];
 *   xhat = (code_0*s_0 + z_0), then xhat = xhat + (code_l*s_l + z_l). */
enum fl_quant_scheme {
    FL_QUANT_ABSMAX = 0, /* symmetric absmax, int8 base + 2/4/8-bit residuals   */
    FL_QUANT_ASYM = 1    /* asymmetric min/max, keys per channel, values per token */
};

typedef struct fl_kv_level {
    int bits;
    int n_rows;
    const int32_t* rows; /* [n_rows]; NULL for level 0 */
    const int32_t* slot; /* [N];      NULL for level 0 */
    void* k_codes;       /* [n_rows][H][d*bits/8] */
    void* v_codes;
    float* k_scale;      /* [n_rows][H][d/g]; FL_QUANT_ASYM: [ceil(n_rows/g)][H][d] */
    float* v_scale;      /* [n_rows][H][d/g] */
    float* k_zero;       /* FL_QUANT_ASYM only: offsets, laid out as k_scale */
    float* v_zero;       /* FL_QUANT_ASYM only: offsets, laid out as v_scale */
} fl_kv_level;

typedef struct fl_kv_cache {
    int N, H, d, g;
    int n_levels; /* levels 0..n_levels-1 hold data */
    int scheme;   /* fl_quant_scheme */
    fl_kv_level level[FL_MAX_LEVELS];
    /* Optional (NULL: not kept): [2][N][H] bytes, keys then values.  Under
     * FL_QUANT_ABSMAX, fl_kv_residual_quant(level) sets entry [w][i][h] of
     * every token i it quantises to 1 when some channel of that token's
     * dequantised value through `level` (head h, keys w = 0 / values w = 1)
     * has magnitude above 4 or is not finite, else 0.  Tokens not quantised
     * keep their entry, which is then their newest level's (the levels are
     * nested).  fl_sparse_loop_attn reads it when args->cls_current is set:
     * it is the operand class of a selected column (see fl_attn_args). */
    uint8_t* cls;
} fl_kv_cache;

/* ------------------------------------------------------------------------
 * Workspace sizing.  op is one of the fl_ws_op values; the remaining
 * arguments are the sizes the call will use (unused ones are ignored).
 * Returns the byte count, or 0 when the sizes are invalid. */
enum fl_ws_op {
    FL_WS_SELECT_ACTIVE = 1,  /* a = n_cand                                    */
    FL_WS_SELECT_COLUMNS = 2, /* a = H, b = n_cand                             */
    FL_WS_SPARSE_ATTN = 3,    /* a = H, b = k (k_prev for a rebuild with sel_prev),
                                 c = d, e = n (active rows of the call);
                                 FL_DEQ_IN_TILE calls need FL_WS_LOOP_STEP's size */
    FL_WS_LOOP_STEP = 4,      /* a = H, b = N (largest k and n), c = d, e = R  */
    FL_WS_BLOCK_STEP = 5,     /* a = N, b = H, c = d, e = ffn width            */
    FL_WS_SQ_ERR = 6          /* a = n                                         */
};
size_t fl_workspace_size(int op, long a, long b, long c, long e);

/* ------------------------------------------------------------------------
 * fl_select_active -- paper Sec. 4.1 (cross-loop token-sparse updates).
 * For each candidate token cand[t] (the tokens active in the previous loop;
 * NULL = all positions 0..n_cand-1) computes the statistic (stat_kind)
 *   FL_TOKEN_STAT_ABS: stat_out[t] = || h_cur[i] - h_prev[i] ||_2
 *   FL_TOKEN_STAT_REL: stat_out[t] = || h_cur[i] - h_prev[i] ||_2 / || h_prev[i] ||_2
 *                      (Sec. 4.1's normalised change; 0 when h_prev[i] = 0 and
 *                      h_cur[i] = h_prev[i], +inf when only h_prev[i] = 0)
 * with i = cand[t], in fp32 over D channels (h_* are [N][D], dtype FL_BF16 or
 * FL_F32), then selects the
 * n_select candidates with the largest statistic; equal statistics go to the
 * lower position; -0 ranks as +0; statistics must be finite.
 * If stat_in != NULL the statistic is not computed and stat_in[n_cand] is
 * ranked instead (h_cur / h_prev may then be NULL).
 * Outputs: active_out[n_select] ascending positions; slot_out (optional, [N])
 * gets slot_out[active_out[s]] = s and -1 for every other position.
 * Workspace: fl_workspace_size(FL_WS_SELECT_ACTIVE, n_cand, ...).
 * Errors: FL_ERR_INVALID_ARG for null required pointers, n_select outside
 * [1, n_cand], n_cand > N, D < 1, an unknown stat_kind. */
enum fl_token_stat { FL_TOKEN_STAT_ABS = 0, FL_TOKEN_STAT_REL = 1 };

int fl_select_active(int dtype, int stat_kind, const void* h_cur, const void* h_prev, int N, int D,
                     const int32_t* cand, int n_cand, int n_select, const float* stat_in,
                     float* stat_out, int32_t* active_out, int32_t* slot_out, void* ws,
                     size_t ws_bytes, fl_stream_t stream);

/* ------------------------------------------------------------------------
 * fl_select_columns -- paper Sec. 4.2 (loop-aware sparse attention: rank the
 * columns with the previous loop's statistics, keep the top-K under a
 * loop-specific budget, prune progressively).
 * Per head h: candidates cand_cols[h][0..n_cand-1] (ascending positions that
 * include the sinks 0..n_sink-1; NULL = positions 0..n_cand-1) with
 * statistics col_stat[h][n_cand].  Output sel_out[h][k]: the sinks plus the
 * k - n_sink non-sink candidates with the largest statistic (ties to the
 * lower position), ascending.  If n_cand <= k the candidates are copied
 * (sel_out is then [H][n_cand]).
 * Errors: FL_ERR_INVALID_ARG for null pointers, n_sink < 0, k <= n_sink,
 * k - n_sink > n_cand - n_sink. */
int fl_select_columns(const float* col_stat, const int32_t* cand_cols, int H, int n_cand,
                      int n_sink, int k, int32_t* sel_out, void* ws, size_t ws_bytes,
                      fl_stream_t stream);

/* ------------------------------------------------------------------------
 * fl_kv_residual_quant -- paper Sec. 3.3, Sec. 4.3, App. E (quantised base
 * plus low-bit cross-loop residuals; residuals only for the active tokens).
 * Writes codes and scales of cache->level[level] (descriptor filled by the
 * caller: bits, n_rows, rows, slot and the code/scale buffers).
 *   level 0: quantises k_new / v_new of all N tokens (int8, or raw fp32).
 *   level l >= 1: for each row t, token i = rows[t]:
 *     x = new(i) - xhat_{l-1}(i)   (fp32; xhat from levels 0..l-1 of token i)
 *     per group: s = max|x| / qmax (qmax = 2^(bits-1)-1), code =
 *     round-half-even(x/s) clamped to [-qmax, qmax] (s = 0 -> codes 0).
 * The arithmetic is IEEE fp32 with correctly rounded division and no fused
 * multiply-add, so codes and scales are reproducible bit for bit.
 * k_new / v_new: dtype FL_BF16 or FL_F32, [N][H][d] by position
 * (new_gathered = 0) or [n_rows][H][d] aligned with rows (new_gathered = 1).
 * Under FL_QUANT_ASYM the groups, codes and offsets follow that scheme's
 * definition above (keys per channel over g consecutive rows of the level,
 * values per token), with the same bit-for-bit arithmetic rules.
 * Errors: FL_ERR_INVALID_ARG (null buffers, level >= FL_MAX_LEVELS, levels
 * below `level` missing, n_rows > N, unknown scheme), FL_ERR_UNSUPPORTED (bits
 * not in {2,4,8,32}, or not in {2,4,8} under FL_QUANT_ASYM; d or g
 * unsupported). */
int fl_kv_residual_quant(const fl_kv_cache* cache, int level, int dtype, const void* k_new,
                         const void* v_new, int new_gathered, fl_stream_t stream);

/* ------------------------------------------------------------------------
 * fl_kv_dequant -- the reconstruction the cache stores (paper Sec. 3.3 / App.
 * E: base state plus cross-loop residuals): out[i][h][c] = xhat of every
 * token i = 0..N-1 at loop level+1, i.e. levels 0..level in order, each
 * token's chain stopping at the first level it is absent from, with the
 * arithmetic of fl_kv_residual_quant (so out equals the residual target that
 * the next level's quantisation uses, bit for bit).
 * which: 0 = keys, 1 = values.  out: fp32 [N][H][d] device buffer, 16-byte
 * aligned.  Errors: as fl_kv_residual_quant for the cache; FL_ERR_INVALID_ARG
 * for which outside {0, 1} or a NULL / misaligned out. */
int fl_kv_dequant(const fl_kv_cache* cache, int level, int which, float* out, fl_stream_t stream);

/* ------------------------------------------------------------------------
 * fl_sparse_loop_attn -- paper Sec. 4.2 (sparse attention over the selected
 * columns; the softmax over the selected logits is rescaled by the cached
 * probability mass of the selected set, and the pruned columns' cached
 * contribution is added back):
 *   S(i) = { j in sel[h] : j <= i }
 *   lse(i) = log sum_{j in S(i)} exp(sm * q(i).khat(j))
 *   o(i)   = (1 - M_U(i)) * sum_{j in S(i)} exp(sm*q(i).khat(j) - lse(i)) vhat(j)
 *            + O_U(i)
 * for each active row i and head h, with khat / vhat dequantised from cache
 * levels 0..level (dequantisation happens inside the kernel's column-tile loop
 * or once per head into a compact bf16 buffer, see `mode`).
 * Cache build (cache_op FL_CACHE_REBUILD; needed when the column set shrank):
 * before the
 * attention M_U and O_U of the active rows are rebuilt under the previous
 * loop's distribution (query q_prev, cache levels 0..level-1, the previous
 * selection, lse and M_U as stored in the state arrays):
 *   M_U(i) = 1 - sum_{j in S(i)} P_prev(i,j)
 *   O_U(i) = o_prev(i) - sum_{j in S(i)} P_prev(i,j) vhat_prev(j)
 *   P_prev(i,j) = (1 - M_U_prev(i)) exp(sm*q_prev(i).khat_prev(j) - lse_prev(i))
 * (the difference form of the pruned columns' mass and output).
 * Column statistics (col_stat != NULL): after the attention,
 *   col_stat[h][p] = sum_{active i >= sel[h][p]} (1 - M_U(i)) *
 *                    exp(sm*q(i).khat(sel[h][p]) - lse(i))
 * (the previous-loop statistic that ranks the next loop's columns).  With
 * col_stat_kind = FL_COL_STAT_VNORM each column's value is multiplied by
 * || vhat(sel[h][p]) ||_2 (fp32, of the dequantised value vector the loop
 * attended to): the size of the column's contribution to the loop's outputs.
 * With sel == NULL (all N columns, k == N) and M_U = O_U = 0 this is the
 * dense first loop.
 */
enum fl_col_stat {
    FL_COL_STAT_MASS = 0,  /* probability mass of the column (default)          */
    FL_COL_STAT_VNORM = 1  /* mass times the column's dequantised value norm     */
};
enum fl_attn_mode {
    FL_DEQ_AUTO = 0,    /* library choice (currently FL_DEQ_ONCE, the faster)  */
    FL_DEQ_ONCE = 1,    /* dequantise the selected columns once per head into a
                           compact bf16 buffer, then stream it per tile        */
    FL_DEQ_IN_TILE = 2  /* gather quantised codes compactly, dequantise inside
                           the attention kernel's column-tile loop (caches of
                           scheme FL_QUANT_ABSMAX only)                        */
};

enum fl_cache_op {
    FL_CACHE_CARRY = 0,   /* read M_U / O_U of the active rows as stored        */
    FL_CACHE_ZERO = 1,    /* treat M_U = O_U = 0 (dense first loop); not read   */
    FL_CACHE_REBUILD = 2  /* rebuild M_U / O_U from the previous loop first     */
};

typedef struct fl_attn_args {
    int dtype;                 /* of q and q_prev: FL_BF16 or FL_F32            */
    const void* q;             /* [N][H][d] by position, or [n][H][d] gathered  */
    int q_gathered;            /* 1: q rows aligned with `active`               */
    const int32_t* active;     /* [n] ascending positions                       */
    int n;
    const int32_t* sel;        /* [H][k] ascending, or NULL (all columns, k = N) */
    int k;
    float sm;                  /* softmax scale, normally 1/sqrt(d)             */
    int level;                 /* newest cache level used (loop level+1)        */
    int mode;                  /* fl_attn_mode                                  */
    int cache_op;              /* fl_cache_op                                   */
    /* loop state, fp32, indexed by token position: */
    float* out;                /* [N][H][d]: o_prev read (rebuild), o written   */
    float* lse;                /* [N][H]: lse_prev read (rebuild), lse written  */
    float* mass_u;             /* [N][H]: M_U (read; written on rebuild)        */
    float* out_u;              /* [N][H][d]: O_U (read; written on rebuild)     */
    float* col_stat;           /* NULL or [H][k]: written                       */
    /* rebuild input: the previous loop's queries (same layout rules as q) */
    const void* q_prev;
    int q_prev_gathered;
    int col_stat_kind;         /* fl_col_stat (used when col_stat != NULL)      */
    /* rebuild after a sparse loop: that loop's column set [H][k_prev]
     * (ascending, sel a subset of it per head).  Given, the rebuild adds the
     * pruned columns' share to the carried caches (additive form,
     * M_U += sum P_prev, O_U += sum P_prev V^_prev over S_prev \ sel) and
     * does not read o_prev; NULL, it subtracts the selected columns' share
     * from o_prev (after the dense first loop, where S_prev is every column). */
    const int32_t* sel_prev;
    int k_prev;
    /* 1: cache->cls holds the classes of this call's level (the newest
     * level quantised into the cache, as right after fl_kv_residual_quant
     * of `level`), so the operand classes of the selected columns are read
     * from it instead of being recomputed from the cache.  Ignored when
     * cache->cls is NULL or the scheme is not FL_QUANT_ABSMAX.  0: always
     * recomputed (calls at an older level must pass 0). */
    int cls_current;
} fl_attn_args;

int fl_sparse_loop_attn(const fl_kv_cache* cache, const fl_attn_args* args, void* ws,
                        size_t ws_bytes, fl_stream_t stream);

/* fl_sparse_loop_attn_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): fl_sparse_loop_attn with its workspace taken from a
 * scratch area the library keeps in every GPU's memory for the life of the
 * process (FL_NOALLOC_SCRATCH_BYTES per GPU), instead of a caller workspace.
 * The caller still passes the cache, inputs and outputs.  The call makes no
 * device allocation (no hipMalloc / hipFree; with the timing aid on, no
 * events are recorded for it) and needs no zeroed memory: every part of the
 * scratch it reads it has written in the same call.  Its first call on a
 * device looks up that device's scratch address (the device must be
 * current).  All calls on one GPU share its scratch, so calls that overlap
 * on one GPU (on different streams, or from several threads without stream
 * ordering between them) race; calls ordered on one stream do not.
 * Limit: the workspace the call needs (fl_workspace_size(FL_WS_SPARSE_ATTN,
 * H, k, d, n) in the default mode; more for FL_DEQ_IN_TILE) must fit
 * FL_NOALLOC_SCRATCH_BYTES -- e.g. 16 heads x 128 with up to 2048 selected
 * columns and 32768 active rows.  Errors: as fl_sparse_loop_attn;
 * FL_ERR_WORKSPACE (before anything is enqueued) when the call needs more,
 * FL_ERR_HIP when the scratch address cannot be looked up. */
#define FL_NOALLOC_SCRATCH_BYTES (80L << 20)
int fl_sparse_loop_attn_noalloc(const fl_kv_cache* cache, const fl_attn_args* args,
                                fl_stream_t stream);

/* ------------------------------------------------------------------------
 * fl_loop_step -- one whole loop r >= 1 of the lazy-update attention step
 * (paper Sec. 4.1-4.3) in attention-only form: the loop's hidden states and
 * q/k/v projections are given for all N tokens; the step uses the rows it
 * selects.
 *   r == 1: base level, dense attention, column statistics (if r < R needs them).
 *   r >= 2: fl_select_active over the previous active set, the residual level
 *           r-1, fl_select_columns when the budget shrinks, cache build when the
 *           column set changed, sparse attention, column statistics when the
 *           next loop prunes further.
 * All state lives in caller-owned device buffers listed in fl_loop_state.
 * Loop 1 sets mass_u to 0 and leaves out_u unwritten (O_U is never read
 * after a dense loop); a later loop that keeps all columns zeroes out_u,
 * and one that prunes rebuilds it.
 */
typedef struct fl_loop_cfg {
    int N, H, d, g, R, n_sink;
    int dtype;              /* of h / q / k / v                                */
    int n_active[FL_MAX_LEVELS]; /* active rows per loop (index r-1); [0] = N   */
    int k_cols[FL_MAX_LEVELS];   /* column budget per loop; [0] = N             */
    int bits[FL_MAX_LEVELS];     /* [0] base bits (8/32), [r-1] residual bits   */
    int mode;               /* fl_attn_mode                                    */
    int token_stat;         /* fl_token_stat: ranking of active tokens         */
    int col_stat;           /* fl_col_stat: ranking of columns                 */
} fl_loop_cfg;

typedef struct fl_loop_state {
    fl_kv_cache cache;      /* level buffers pre-allocated by the caller        */
    int32_t* active[FL_MAX_LEVELS]; /* [n_active[r-1]] per loop; active[0] unused */
    int32_t* slot[FL_MAX_LEVELS];   /* [N] per loop (r >= 2)                     */
    float* stat;            /* [N] scratch for the token statistic              */
    int32_t* sel[FL_MAX_LEVELS];    /* [H][k_cols[r-1]] per loop (r >= 2)        */
    const int32_t* sel_used[FL_MAX_LEVELS]; /* filled by the step: the column set
                                       used in each loop (NULL = all columns)   */
    int k_cur[FL_MAX_LEVELS];       /* filled by the step: columns used per loop  */
    float* col_stat[FL_MAX_LEVELS]; /* [H][k of loop r] when computed, per loop  */
    float* out; float* lse; float* mass_u; float* out_u; /* position-indexed    */
} fl_loop_state;

typedef struct fl_loop_inputs {
    const void* h_cur;      /* [N][H*d] hidden state entering loop r           */
    const void* h_prev;     /* [N][H*d] hidden state entering loop r-1 (r >= 2) */
    const void* q;          /* [N][H][d] loop r queries                        */
    const void* k;          /* [N][H][d] loop r keys                           */
    const void* v;          /* [N][H][d] loop r values                         */
    const void* q_prev;     /* [N][H][d] loop r-1 queries (r >= 2)              */
} fl_loop_inputs;

int fl_loop_step(const fl_loop_cfg* cfg, fl_loop_state* st, const fl_loop_inputs* in, int r,
                 void* ws, size_t ws_bytes, fl_stream_t stream);

/* ------------------------------------------------------------------------
 * fl_block_step -- one loop r of a whole looped block of n_layers
 * pre-norm Transformer layers (paper Sec. 4.1: the block computes only the
 * active tokens, inactive tokens keep their states and reuse their K/V;
 * Sec. 4.4: active tokens are gathered into compact buffers so the
 * projections stay regular GEMMs).  Per loop r: (r >= 2) the token statistic
 * ||h - h_entry|| over the previous active set and the nested top-n_active[r-1]
 * selection; then for every layer, on the active rows only:
 *   a = RMSNorm(h) * norm1;  [q k v] = a W_qkv^T;  RoPE(q, k) at the token
 *   positions (theta = rope_theta, rotate-half);  residual level r-1 of the
 *   layer's K/V cache (keys after RoPE);  column selection, cache rebuild and
 *   sparse attention exactly as fl_loop_step;  h += attn W_o^T;
 *   b = RMSNorm(h) * norm2;  h += (silu(b W_g^T) * (b W_u^T)) W_down^T.
 * RMSNorm(x) = x / sqrt(mean(x^2) + norm_eps).  GEMMs are bf16 MFMA with fp32
 * accumulation; the residual stream h is fp32.  Loop 1 runs every token and
 * dense attention.  h_entry receives a copy of h at the start of every loop.
 * Weights (bf16, output-major [out][in]): w_qkv [3D][D] (q rows, then k, then
 * v), w_o [D][D], w_gu [2F][D] with row 2j the gate and row 2j+1 the up
 * projection of hidden unit j, w_down [D][F]; norm1/norm2 [D].
 * Requirements: D = H*d a multiple of 128, F a multiple of 128 (and of 32).
 * Workspace: fl_workspace_size(FL_WS_BLOCK_STEP, N, H, d, F).
 */
typedef struct fl_block_cfg {
    int N, H, d, g, R, n_sink;
    int n_layers, ffn;
    float rope_theta, norm_eps;
    int n_active[FL_MAX_LEVELS];
    int k_cols[FL_MAX_LEVELS];
    int bits[FL_MAX_LEVELS];
    int mode;               /* fl_attn_mode: FL_DEQ_AUTO or FL_DEQ_ONCE        */
    int token_stat;         /* fl_token_stat */
    int col_stat;           /* fl_col_stat   */
} fl_block_cfg;

typedef struct fl_layer_weights {
    const void* w_qkv;
    const void* w_o;
    const void* w_gu;
    const void* w_down;
    const void* norm1;
    const void* norm2;
} fl_layer_weights;

typedef struct fl_layer_state {
    fl_kv_cache cache;      /* level buffers pre-allocated by the caller        */
    void* q_state;          /* bf16 [N][H][d]: latest queries per token         */
    float* out; float* lse; float* mass_u; float* out_u; /* as fl_loop_state   */
    int32_t* sel[FL_MAX_LEVELS];
    const int32_t* sel_used[FL_MAX_LEVELS];
    int k_cur[FL_MAX_LEVELS];
    float* col_stat[FL_MAX_LEVELS];
    /* optional (NULL: not written): bf16 [n_active[r-1]][H][d] each; receive
     * the loop's keys (after RoPE) and values of the active rows, in active
     * order, exactly as the layer's quantiser reads them.  A checker can then
     * re-quantise the same values independently (App. E: keys are quantised
     * after RoPE). */
    void* k_in;
    void* v_in;
} fl_layer_state;

typedef struct fl_block_state {
    float* h;               /* fp32 [N][D] residual stream                      */
    float* h_entry;         /* fp32 [N][D] h at the entry of the previous loop   */
    int32_t* active[FL_MAX_LEVELS]; /* [n_active[r-1]] per loop (active[0]: iota) */
    int32_t* slot[FL_MAX_LEVELS];   /* [N] per loop r >= 2                      */
    float* stat;            /* [N]                                              */
    fl_layer_state* layers; /* host array [n_layers]                            */
} fl_block_state;

int fl_block_step(const fl_block_cfg* cfg, const fl_layer_weights* w, fl_block_state* st, int r,
                  void* ws, size_t ws_bytes, fl_stream_t stream);

/* ------------------------------------------------------------------------
 * fl_decode_step -- one loop r of batched decode (paper Sec. 4.2; Sec. 5.3.1
 * reports decode as bound by KV traffic): B sequences, each with a cached
 * prefix of N tokens stored as the loop-indexed quantised cache (base level
 * plus residual levels for the prefix tokens active in each loop), and one
 * new query token per sequence.  For each sequence and head the key columns
 * are the selected prefix columns S_r (all N at r = 1) plus the token's own
 * fresh bf16 key/value (the self column, always included):
 *   P(j) = (1 - M_U) softmax over S_r and self of sm * q.khat_r(j)
 *   o = sum_j P(j) vhat_r(j) + O_U,  khat_r/vhat_r from cache levels 0..r-1.
 * r >= 2: columns are re-selected (sinks + top by the previous loop's P over
 * the prefix) when the budget shrinks, and M_U / O_U are rebuilt under the
 * previous loop's distribution (its query and self column) as in
 * fl_sparse_loop_attn.  The previous loop's P over the kept prefix columns
 * is the column statistic (col_stat).
 * Cache layout: cache.level[l] describes sequence 0 with the usual fields;
 * sequence b's rows/slot/codes/scales follow at b * (R_l, P, R_l*H*d*bits/8
 * bytes, R_l*H*d/g floats) -- B sequences of equal geometry -- with the
 * per-sequence capacities P = N_cap (or N) positions and R_l = rows_cap[l]
 * (or n_rows; level 0: P) rows.  Under FL_QUANT_ASYM the value offsets
 * follow the value scales' layout, and the key scales and offsets (one per
 * channel for every g rows) follow at b * G_l*H*d floats.  Key group i of a
 * level covers rows [i*g, (i+1)*g) below the level's origin
 * o_l = cfg->key_group_origin[l] (the last of them possibly partial) and,
 * from the origin on, rows [o_l + j*g, o_l + (j+1)*g) for i = ceil(o_l/g) + j
 * (the groups that generation appends); G_l = ceil(o_l/g) + ceil((R_l-o_l)/g)
 * (ceil(R_l/g) with the default origin 0).
 * Requirements: N + T <= 12288 (T bf16 columns: 1, or the window count; the
 * probabilities stay in LDS); quantised levels: FL_QUANT_ABSMAX with an
 * int8 base, or FL_QUANT_ASYM with 2-, 4- or 8-bit levels
 * (FL_ERR_UNSUPPORTED otherwise); a
 * sparse loop r keeps 4 * ((k + 1) + r * k) bytes in LDS, at most 48 KiB.
 */
typedef struct fl_decode_cfg {
    int B, N, H, d, g, R, n_sink;
    int k_cols[FL_MAX_LEVELS];  /* [0] = N */
    /* per-sequence capacities of a cache that grows during generation
     * (fl_decode_append); 0 = exactly N positions / n_rows rows: */
    int N_cap;                  /* positions (slot maps, level-0 rows)       */
    int rows_cap[FL_MAX_LEVELS]; /* rows of level l >= 1 (index l)           */
    /* FL_QUANT_ASYM: the row (index 0: position) of each level at which the
     * appended key groups begin -- the prompt's N and n_rows when the cache
     * grows during generation; 0 (the default) = groups of g rows from row 0
     * throughout.  Ignored under FL_QUANT_ABSMAX. */
    int key_group_origin[FL_MAX_LEVELS];
} fl_decode_cfg;

/* Generation-time bf16 window (App. E: the most recent 64 tokens stay in
 * BF16).  Per loop r a ring of `cap` slots per sequence holds the loop-r
 * keys / values of the most recent generated tokens and of the token being
 * decoded: k[r-1], v[r-1] bf16 [B][cap][H][d].  The `count` valid slots are
 * (start + i) mod cap, i = 0..count-1, 0 <= start < cap (which slot holds
 * which token does not matter to attention: all are earlier than or equal to
 * the new token).  Every valid slot is an extra key column of every loop,
 * always included like the self column. */
typedef struct fl_decode_window {
    int cap;
    int count;
    int start;
    const void* k[FL_MAX_LEVELS];
    const void* v[FL_MAX_LEVELS];
} fl_decode_window;

typedef struct fl_decode_state {
    fl_kv_cache cache;
    float* out; float* lse; float* mass_u; float* out_u; /* [B][H][d], [B][H] */
    int32_t* sel[FL_MAX_LEVELS];            /* [B][H][k_cols[r-1]] (r >= 2)     */
    const int32_t* sel_used[FL_MAX_LEVELS]; /* filled by the step                */
    int k_cur[FL_MAX_LEVELS];               /* filled by the step                */
    float* col_stat[FL_MAX_LEVELS];         /* [B][H][k of loop r]               */
} fl_decode_state;

typedef struct fl_decode_inputs {
    const void* q;       /* bf16 [B][H][d] loop r query of the new token        */
    const void* k_self;  /* bf16 [B][H][d] loop r key / value of the new token  */
    const void* v_self;
    const void* q_prev;  /* loop r-1 values (r >= 2)                            */
    const void* k_self_prev;
    const void* v_self_prev;
    /* generation: when win != NULL its `count` slots of loop r (and r-1 for a
     * rebuild) are the bf16 columns in place of k_self / v_self (the caller
     * has written the new token into one of them) */
    const fl_decode_window* win;
} fl_decode_inputs;

int fl_decode_step(const fl_decode_cfg* cfg, fl_decode_state* st, const fl_decode_inputs* in,
                   int r, fl_stream_t stream);

/* ------------------------------------------------------------------------
 * fl_decode_append -- generation-time growth of the quantised cache (Sec.
 * 4.3, App. E): the n tokens in ring slots (slot + j) mod cap, j = 0..n-1, of
 * every loop's window (generated tokens, computed in all R loops) are
 * appended, in that order, to every sequence's cache at positions
 * p_j = cfg->N + j: level 0 stores their loop-1 K/V quantised as the base,
 * level l >= 1 appends rows n_rows_l + j holding the residual of their
 * loop-(l+1) K/V against their dequantised loop-l values
 * (rows[n_rows_l + j] = p_j, slot[p_j] = n_rows_l + j), with the arithmetic
 * of fl_kv_residual_quant.  Under FL_QUANT_ABSMAX each token is quantised on
 * its own (any n >= 1).  Under FL_QUANT_ASYM the keys are quantised per
 * channel over g rows, so n must be g and the block becomes one new key
 * group of every level: cfg->N and each n_rows_l must lie a whole number of
 * groups past cfg->key_group_origin (set the origins to the prompt's sizes
 * before the first append); the value groups stay per token.  Then cfg->N,
 * st->cache.N and every st->cache.level[l].n_rows (l = 1..R-1) grow by n.
 * The cache must have been allocated with capacities cfg->N_cap and
 * cfg->rows_cap (and, FL_QUANT_ASYM, the key groups those and the origins
 * imply), quantised levels and, FL_QUANT_ABSMAX, an int8 base.
 * Errors: FL_ERR_INVALID_ARG (NULL pointers, slots outside the ring, a
 * capacity exceeded, a block not on a key-group boundary),
 * FL_ERR_UNSUPPORTED (cache format, n != g under FL_QUANT_ASYM). */
int fl_decode_append(fl_decode_cfg* cfg, fl_decode_state* st, const fl_decode_window* win,
                     int slot, int n, fl_stream_t stream);

/* ------------------------------------------------------------------------
 * Input validation.  The entry points take index lists and statistics as
 * device arrays and by default trust them (checking them would need a copy
 * to the host and a synchronisation).  The paper's selections (Sec. 4.1,
 * 4.2) assume ascending, unique positions and rankable statistics:
 *
 * fl_check_indices(idx, n, lo, hi): HOST array idx[0..n) strictly ascending
 *   (hence unique) with every element in [lo, hi).  Returns FL_OK, or
 *   FL_ERR_INVALID_ARG with fl_last_error() naming the first bad element.
 * fl_check_finite(x, n): HOST array x[0..n) all finite (no NaN / inf);
 *   FL_OK or FL_ERR_INVALID_ARG as above.
 * fl_set_checks(on): check mode for this process (default off).  When on,
 *   every entry point first waits for its stream, copies its device index
 *   lists and statistics to the host and validates them as above, returning
 *   FL_ERR_INVALID_ARG before anything of the call is enqueued:
 *     fl_select_active: cand (ascending in [0, N)), stat_in (finite); the
 *       computed statistic (no NaN; the normalised one may be +inf) before
 *       the selection;
 *     fl_select_columns: every head's cand_cols row (ascending, >= 0),
 *       col_stat (finite);
 *     fl_kv_residual_quant, fl_sparse_loop_attn, fl_loop_step,
 *       fl_block_step, fl_decode_step: residual levels' row lists (ascending
 *       in [0, N)), active (ascending in [0, N)), every head's sel row
 *       (ascending in [0, N)).
 *   Check mode synchronises the stream inside the calls; it is a debugging
 *   aid, not for timed runs. */
int fl_check_indices(const int32_t* idx, long n, long lo, long hi);
int fl_check_finite(const float* x, long n);
int fl_set_checks(int on);

/* ------------------------------------------------------------------------
 * Per-kernel and per-phase timing (profiling aid).  fl_timing_enable(level):
 *   0  off;
 *   1  every later launch of the library records a HIP event pair around
 *      each kernel on the launch stream, and fl_loop_step also records the
 *      phases below;
 *   2  phases only: fl_loop_step records an event pair around steps a1-a4
 *      (token statistic, selection, quantisation; for r = 1 the base level)
 *      named "loop<r>.a1-a4" and one around steps a5-a8 (column selection,
 *      pruned-column caches, sparse attention, column statistics) named
 *      "loop<r>.a5-a8" (paper Sec. 4.1-4.3), with no per-kernel events
 *      between them.
 * fl_timing_report waits for those events and writes one line per name,
 * "name launches total_ms\n", into buf (NUL-terminated, truncated to len),
 * then forgets the recorded launches.  Returns FL_OK, or FL_ERR_INVALID_ARG
 * when the report was truncated or the level is unknown, FL_ERR_HIP on an
 * event error. */
int fl_timing_enable(int on);
int fl_timing_report(char* buf, size_t len);

/* ------------------------------------------------------------------------ */
const char* fl_last_error(void);
const char* fl_version(void);

/* ------------------------------------------------------------------------
 * fl_sq_err -- the reconstruction error behind the retention calibration of
 * the paper's App. E ("Quantization Setting": each loop keeps the smallest
 * retention ratio whose hidden states or attention outputs stay below a
 * relative reconstruction error of 5% against the reference).  Computes, over
 * n fp32 values,
 *   out[0] = sum_i (x[i] - ref[i])^2,   out[1] = sum_i ref[i]^2
 * in fp64 (out: device pointer to 2 doubles); the relative error is
 * sqrt(out[0] / out[1]).  x and ref are device pointers aligned to 16 bytes.
 * The summation order depends only on n (deterministic).
 * Workspace: fl_workspace_size(FL_WS_SQ_ERR, n).
 * Errors: FL_ERR_INVALID_ARG for null or misaligned pointers or n < 1;
 * FL_ERR_WORKSPACE. */
int fl_sq_err(const float* x, const float* ref, long n, double* out, void* ws, size_t ws_bytes,
              fl_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FLASHLOOP_H */

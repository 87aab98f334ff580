/* Address / undefined-behaviour sanitizer driver of the C ABI's host code
 * (argument validation, error messages, workspace sizing, timing and check
 * switches): every entry point is called with arguments its validation must
 * reject before touching a device, plus the host-array validators.  No GPU
 * is needed and no device memory is touched: pointers that validation
 * accepts are never dereferenced on these paths.  Built by
 * tests/test_sanitize_cpu.py against a library whose host code carries the
 * sanitizers; any report aborts the run.  Exit 0 = no finding. */
#include <stdio.h>
#include <string.h>

#include "flashloop.h"

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "FAILED line %d: %s (%s)\n", __LINE__, #c, fl_last_error()); ++fails; } } while (0)

int main(void) {
    void* F = (void*)0x10000;  /* non-null, never dereferenced by validation */
    EXPECT(strstr(fl_version(), "gfx950") != NULL);
    EXPECT(fl_workspace_size(FL_WS_SPARSE_ATTN, 16, 2048, 128, 4) > 0);
    EXPECT(fl_workspace_size(FL_WS_SPARSE_ATTN, 16, 2048, 96, 4) == 0);
    EXPECT(fl_workspace_size(FL_WS_BLOCK_STEP, 8192, 16, 128, 5632) > 0);
    EXPECT(fl_workspace_size(99, 1, 1, 1, 1) == 0);
    /* selection */
    EXPECT(fl_select_active(FL_BF16, 0, F, F, 100, 64, NULL, 100, 0, NULL, F, F, NULL, NULL, 0, NULL) == FL_ERR_INVALID_ARG);
    EXPECT(fl_select_active(FL_BF16, 0, F, F, 100, 60, NULL, 100, 5, NULL, F, F, NULL, NULL, 0, NULL) == FL_ERR_INVALID_ARG);
    EXPECT(fl_select_active(FL_BF16, 9, F, F, 100, 64, NULL, 100, 5, NULL, F, F, NULL, NULL, 0, NULL) == FL_ERR_INVALID_ARG);
    EXPECT(fl_select_columns(F, NULL, 2, 100, 4, 4, F, NULL, 0, NULL) == FL_ERR_INVALID_ARG);
    EXPECT(fl_select_columns(F, NULL, 0, 100, 4, 10, F, NULL, 0, NULL) == FL_ERR_INVALID_ARG);
    /* cache formats */
    fl_kv_cache c;
    memset(&c, 0, sizeof c);
    c.N = 64; c.H = 2; c.d = 96; c.g = 32; c.n_levels = 1;
    c.level[0].bits = 8; c.level[0].n_rows = 64;
    c.level[0].k_codes = c.level[0].v_codes = F;
    c.level[0].k_scale = c.level[0].v_scale = F;
    EXPECT(fl_kv_residual_quant(&c, 0, FL_BF16, F, F, 0, NULL) == FL_ERR_UNSUPPORTED);
    c.d = 128; c.g = 48;
    EXPECT(fl_kv_residual_quant(&c, 0, FL_BF16, F, F, 0, NULL) == FL_ERR_UNSUPPORTED);
    c.g = 64; c.level[0].bits = 3;
    EXPECT(fl_kv_residual_quant(&c, 0, FL_BF16, F, F, 0, NULL) == FL_ERR_UNSUPPORTED);
    c.level[0].bits = 8;
    EXPECT(fl_kv_residual_quant(&c, 0, FL_BF16, NULL, F, 0, NULL) == FL_ERR_INVALID_ARG);
    EXPECT(fl_kv_residual_quant(&c, FL_MAX_LEVELS, FL_BF16, F, F, 0, NULL) == FL_ERR_INVALID_ARG);
    c.level[1].bits = 4; c.level[1].n_rows = 100; c.level[1].rows = F; c.level[1].slot = F;
    c.level[1].k_codes = c.level[1].v_codes = F; c.level[1].k_scale = c.level[1].v_scale = F;
    EXPECT(fl_kv_residual_quant(&c, 1, FL_BF16, F, F, 0, NULL) == FL_ERR_INVALID_ARG);  /* n_rows > N */
    c.scheme = 7;
    EXPECT(fl_kv_residual_quant(&c, 0, FL_BF16, F, F, 0, NULL) == FL_ERR_INVALID_ARG);
    c.scheme = FL_QUANT_ABSMAX;
    /* attention */
    fl_attn_args a;
    memset(&a, 0, sizeof a);
    a.dtype = FL_BF16; a.q = F; a.active = F; a.n = 10; a.k = 64; a.out = F; a.lse = F;
    a.cache_op = FL_CACHE_ZERO; a.sm = 0.1f;
    EXPECT(fl_sparse_loop_attn(&c, &a, NULL, 0, NULL) == FL_ERR_WORKSPACE);
    a.n = 0;
    EXPECT(fl_sparse_loop_attn(&c, &a, F, 1 << 30, NULL) == FL_ERR_INVALID_ARG);
    a.n = 10; a.k = 65;
    EXPECT(fl_sparse_loop_attn(&c, &a, F, 1 << 30, NULL) == FL_ERR_INVALID_ARG);
    a.k = 64; a.cache_op = FL_CACHE_REBUILD;
    EXPECT(fl_sparse_loop_attn(&c, &a, F, 1 << 30, NULL) == FL_ERR_INVALID_ARG);   /* level 0 rebuild */
    a.cache_op = FL_CACHE_ZERO; a.mode = 9;
    EXPECT(fl_sparse_loop_attn(&c, &a, F, 1 << 30, NULL) == FL_ERR_INVALID_ARG);
    EXPECT(fl_sparse_loop_attn(&c, NULL, F, 1 << 30, NULL) == FL_ERR_INVALID_ARG);
    /* loop, block and decode steps */
    fl_loop_cfg lc;
    memset(&lc, 0, sizeof lc);
    lc.N = 64; lc.H = 2; lc.d = 128; lc.g = 64; lc.R = 2; lc.n_sink = 4;
    fl_loop_state ls;
    memset(&ls, 0, sizeof ls);
    fl_loop_inputs li;
    memset(&li, 0, sizeof li);
    EXPECT(fl_loop_step(&lc, &ls, &li, 3, F, 1 << 30, NULL) == FL_ERR_INVALID_ARG);
    EXPECT(fl_loop_step(NULL, &ls, &li, 1, F, 1 << 30, NULL) == FL_ERR_INVALID_ARG);
    fl_block_cfg bc;
    memset(&bc, 0, sizeof bc);
    bc.N = 64; bc.H = 2; bc.d = 96; bc.R = 2; bc.n_layers = 1; bc.ffn = 256;
    fl_layer_weights lw;
    memset(&lw, 0, sizeof lw);
    fl_layer_state lst;
    memset(&lst, 0, sizeof lst);
    fl_block_state bs;
    memset(&bs, 0, sizeof bs);
    bs.layers = &lst;
    EXPECT(fl_block_step(&bc, &lw, &bs, 1, F, 1 << 30, NULL) < 0);
    fl_decode_cfg dc;
    memset(&dc, 0, sizeof dc);
    fl_decode_state ds;
    memset(&ds, 0, sizeof ds);
    fl_decode_inputs di;
    memset(&di, 0, sizeof di);
    EXPECT(fl_decode_step(&dc, &ds, &di, 1, NULL) == FL_ERR_INVALID_ARG);
    EXPECT(fl_decode_append(&dc, &ds, NULL, 0, 1, NULL) == FL_ERR_INVALID_ARG);
    /* host validators and switches */
    const int ok[4] = {0, 2, 5, 9}, bad[3] = {0, 5, 5};
    const float fin[3] = {0.0f, -1.0f, 2.0f};
    float nonfin[2] = {1.0f, 0.0f};
    nonfin[1] = nonfin[1] / nonfin[1] * 0.0f + 1.0f / 0.0f; /* +inf */
    EXPECT(fl_check_indices(ok, 4, 0, 10) == FL_OK);
    EXPECT(fl_check_indices(bad, 3, 0, 10) == FL_ERR_INVALID_ARG);
    EXPECT(fl_check_indices(ok, 4, 0, 9) == FL_ERR_INVALID_ARG);
    EXPECT(fl_check_finite(fin, 3) == FL_OK);
    EXPECT(fl_check_finite(nonfin, 2) == FL_ERR_INVALID_ARG);
    EXPECT(fl_set_checks(1) == FL_OK && fl_set_checks(0) == FL_OK);
    EXPECT(fl_timing_enable(3) == FL_ERR_INVALID_ARG);
    EXPECT(fl_timing_enable(2) == FL_OK && fl_timing_enable(0) == FL_OK);
    char buf[64];
    EXPECT(fl_timing_report(buf, sizeof buf) == FL_OK);
    if (fails) { fprintf(stderr, "%d expectation(s) failed\n", fails); return 1; }
    printf("ABI sanitizer driver: ok\n");
    return 0;
}

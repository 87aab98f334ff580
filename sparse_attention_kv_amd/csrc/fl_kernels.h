// Launch interface between the host ABI (abi.hip) and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flashloop.h"

namespace fl {

// Compact quantised copies of the selected columns, one plane per cache level
// (absent levels hold zero codes and scales):
//   kq[l] [H][kp][d*bits/8]  codes, column-major rows as stored
//   ks[l] [H][kp][d/g]       scales
//   vq[l] [H][kp/64][d][64*bits/8]  codes transposed per 64-column tile, keys
//                                    in the MFMA-operand order
//   vs[l] [H][kp/64][d/g][64]        scales, same key order
struct QTiles {
    int n_levels;
    int g;
    int bits[FL_MAX_LEVELS];
    uint8_t* kq[FL_MAX_LEVELS];
    float* ks[FL_MAX_LEVELS];
    uint8_t* vq[FL_MAX_LEVELS];
    float* vs[FL_MAX_LEVELS];
};

struct AttnParams {
    int H, n, k, kp, dtype, q_gathered, cache_op;
    float c2;        // softmax scale * log2(e)
    const void* q;
    const int32_t* active;
    const __bf16* Kc;      // [H][kp][d] compact bf16 keys
    const __bf16* Vt;      // [H][kp/64][d][64] compact bf16 values, transposed tiles
    const __bf16* Kc_lo;   // fp32 inputs: bf16 rounding of the residual x - bf16(x)
    const __bf16* Vt_lo;
    const int32_t* cpos;   // [H][kp] column positions (INT32_MAX for padding)
    float* out;
    float* lse;
    float* mass_u;
    float* out_u;
    __bf16* out_bf;        // optional: the output also as bf16 [n][H][d] by active index
    // precision-adaptive kernel (k_attn_ad): per head, the row order
    // [normal | outlier] (indices into `active`) and the normal row count,
    // and the column parts (normal count, outlier count) of the compact
    // buffers, laid out [normal | pad to 64 | outlier]
    const int32_t* rowperm;  // [H][n]
    const int32_t* rowseg;   // [H]
    const int32_t* colseg;   // [H][2]
    int xcd_remap;
    // MODE_ATTN_RB (k_attn_ad): the previous loop's side of a subtract-form
    // cache rebuild, run by the same workgroups before the attention: its
    // compact bf16 K / V^T (plain layout, k_old selected columns in
    // selection order, kp slots), positions, and queries
    const __bf16* Kc_old;
    const __bf16* Vt_old;
    const int32_t* cpos_old;
    int k_old;
    const void* q_old;
    int q_old_gathered;
    int deq_levels;        // in-tile dequantisation: levels 0..deq_levels-1 of q
    QTiles qt;
};

struct ColParams {
    int H, n, k, kp, dtype, q_gathered, cache_op;
    float c2;
    const void* q;
    const int32_t* active;
    const __bf16* Kc;
    const __bf16* Kc_lo;
    const int32_t* cpos;
    const float* lse;
    const float* mass_u;
    const float* vnorm;    // [H][kp] value norms (value-weighted statistic) or NULL
    const int32_t* perm;   // [H][kp] selection index of each compact slot (-1: pad), or NULL
    float* col_stat;
};

// MODE_REBUILD: pruned-column caches by subtraction from o_prev over the
// selected columns; MODE_REBUILD_ADD: added to the carried caches over the
// pruned columns (k_attn_ad only); MODE_ATTN_RB: the subtract-form rebuild
// over the previous loop's side, then the attention, in one launch
// (k_attn_ad only)
enum { MODE_ATTN = 0, MODE_REBUILD = 1, MODE_REBUILD_ADD = 2, MODE_ATTN_RB = 3 };

// Batched decode: B sequences x H heads, one new query token each.
struct DecodeParams {
    int B, H, k, level, cache_op;
    float sm;
    fl_kv_cache cache;      // one sequence's geometry; level buffers hold B sequences
    int pos_cap;            // per-sequence stride of slot maps and level-0 rows
    int rows_cap[FL_MAX_LEVELS]; // per-sequence row stride of level l >= 1
    const int32_t* sel;     // [B*H][k] selected prefix columns, or NULL (all N)
    const void* q;          // bf16 [B][H][d]
    const void* tail_k;     // bf16 [B][tail_cap][H][d]: the always-included columns
    const void* tail_v;     //   (the token's own, and the generation window)
    int n_tail, tail_cap;
    int tail_start;         // tail column t is ring slot (tail_start + t) mod tail_cap
    // asymmetric keys: group of row x of level l is (x + (x >= origin ? pad : 0)) / g,
    // and a sequence holds kg_count[l] groups of H*d scales / offsets
    int kg_origin[FL_MAX_LEVELS];
    int kg_pad[FL_MAX_LEVELS];
    int kg_count[FL_MAX_LEVELS];
    float* out; float* lse; float* mass_u; float* out_u; float* col_stat;
    int pairs;              // set by the launcher: sparse absmax passes over (column, level) pairs
};

struct AppendParams {
    int B, H, g, R, pos, slot, win_cap, pos_cap;
    int n;                       // tokens appended (ring slots slot .. slot + n - 1 mod win_cap)
    int kg_pad[FL_MAX_LEVELS];   // asymmetric keys: as in DecodeParams
    int kg_count[FL_MAX_LEVELS];
    int rows_cap[FL_MAX_LEVELS];
    int n_rows[FL_MAX_LEVELS];   // rows already stored per level (the new row's index)
    int bits[FL_MAX_LEVELS];
    fl_kv_level lev[FL_MAX_LEVELS];
    const void* wk[FL_MAX_LEVELS];
    const void* wv[FL_MAX_LEVELS];
};

// Kernels take the cache descriptor (and, on the in-tile path, the level
// code planes) by value.  A 3648-byte by-value argument was checked to arrive
// intact on gfx950; every kernel's arguments stay within that size.
constexpr size_t kKernargChecked = 3648;
static_assert(sizeof(fl_kv_cache) + sizeof(QTiles) + 48 <= kKernargChecked,
              "k_gather_q arguments exceed the checked kernel-argument size");
static_assert(sizeof(DecodeParams) + 16 <= kKernargChecked,
              "k_decode arguments exceed the checked kernel-argument size");
static_assert(sizeof(AppendParams) + 16 <= kKernargChecked,
              "k_decode_append arguments exceed the checked kernel-argument size");
static_assert(sizeof(fl_kv_cache) + 64 <= kKernargChecked,
              "cache-descriptor kernels exceed the checked kernel-argument size");

// C = A[M][K] . B[N][K]^T (bf16 in, fp32 accumulate); N % 128 == 0, K % 32 == 0
enum { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };
struct GemmParams {
    int M, N, K;
    const __bf16* A;       // [M][lda]
    long lda;
    const __bf16* B;       // [N][K] (weights, output-major)
    __bf16* Cb;            // EPI_STORE: [M][ldc]; EPI_SWIGLU: [M][ldc] with ldc >= N/2
    float* Cf;             // EPI_RESID: fp32 [*][ldc], rows selected by `rows`
    long ldc;
    const int32_t* rows;   // EPI_RESID: destination row of each of the M rows
};

// select.hip
hipError_t launch_delta_norm(const void* h_cur, const void* h_prev, int dtype, int D,
                             const int32_t* cand, int n_cand, bool relative, float* stat,
                             hipStream_t st);
hipError_t launch_topk(const float* keys, long key_stride, const int32_t* pos, long pos_stride,
                       int n, int n_sel, int n_prefix, int32_t* out, long out_stride,
                       int32_t* slot, int n_slot, int n_seg, hipStream_t st);
hipError_t launch_copy_or_iota(const int32_t* src, int32_t* dst, long n, long row, hipStream_t st);
// quant.hip
hipError_t launch_dequant(const fl_kv_cache& cache, int level, int which, float* out,
                          hipStream_t st);
hipError_t launch_decode_append(int d, int scheme, const AppendParams& P, hipStream_t st);
hipError_t launch_quant(const fl_kv_cache& cache, int level, int dtype, const void* k_new,
                        const void* v_new, int gathered, hipStream_t st);
// attn.hip
// perm (NULL: slot p holds selection index p): [H][kp] selection index of
// each compact slot, -1 for padding
hipError_t launch_gather_bf16(const fl_kv_cache& c, int upto, const int32_t* sel, int k, int kp,
                              bool split, __bf16* Kc, __bf16* Vt, __bf16* Kc_lo, __bf16* Vt_lo,
                              int32_t* cpos, float* vnorm, const int32_t* perm, const int32_t* colseg,
                              hipStream_t st);
// prec: 0 bf16 operands, 1 K/V/P as hi+lo bf16 pairs, 2 also q (fp32 inputs)
hipError_t launch_gather_q(const fl_kv_cache& c, int upto, const int32_t* sel, int k, int kp,
                           const QTiles& out, int32_t* cpos, hipStream_t st);
hipError_t launch_attn(int d, int mode, int prec, bool in_tile, const AttnParams& P, hipStream_t st);
hipError_t launch_colstat(int d, int prec, const ColParams& P, hipStream_t st);
// adaptive.hip: operand-precision classes of the selected columns and the
// active rows (per head), and the precision-adaptive attention
constexpr float kTauCol = 4.0f;  // |K^|, |V^| bound of a "normal" column
constexpr float kTauRow = 6.0f;  // |q| bound of a "normal" query row
// class flag planes: colflags [H][kp], rowflags [H][class_row_stride(n)] (rows 16-byte aligned);
// cls (or NULL): the cache's per-token classes [2][N][H], read instead of
// dequantising the selected columns
inline long class_row_stride(long n) { return (n + 15) / 16 * 16; }
hipError_t launch_classify(const fl_kv_cache& c, int upto, const int32_t* sel, int k, int kp,
                           const void* q, int dtype, int q_gathered, const int32_t* active, int n,
                           float tau_col, float tau_row, uint8_t* colflags, int32_t* perm, int32_t* colseg,
                           uint8_t* rowflags, int32_t* rowperm, int32_t* rowseg, const uint8_t* cls,
                           hipStream_t st);
hipError_t launch_attn_ad(int d, int mode, const AttnParams& P, hipStream_t st);
// per head, the columns of sel_prev [H][k_prev] absent from sel [H][k]
// (ascending; k_prev - k of them) -> pruned [H][k_prev - k]
hipError_t launch_set_diff(const int32_t* sel_prev, int k_prev, const int32_t* sel, int k, int H,
                           int32_t* pruned, hipStream_t st);
// calib.hip
int sq_err_blocks(long n);
hipError_t launch_sq_err(const float* x, const float* ref, long n, double* part, double* out,
                         hipStream_t st);
// block.hip
hipError_t launch_rmsnorm_gather(const float* x, const int32_t* rows, int n, int D,
                                 const __bf16* w, float eps, __bf16* out, hipStream_t st);
hipError_t launch_gemm(int epi, const GemmParams& G, hipStream_t st);
// output columns per workgroup launch_gemm uses for G (64 or 128)
int gemm_tile_n(const GemmParams& G);
hipError_t launch_rope_split(const __bf16* qkv, const int32_t* rows, int n, int H, int d,
                             float theta, __bf16* q, __bf16* k, __bf16* v, hipStream_t st);
hipError_t launch_scatter_rows_bf16(const __bf16* src, const int32_t* rows, long n, int D,
                                    __bf16* dst, hipStream_t st);
// decode.hip
hipError_t launch_decode(int d, int mode, const DecodeParams& P, hipStream_t st);
// abi.hip
hipError_t launch_fill_f32(float* p, long n, float v, hipStream_t st);

} // namespace fl

// Precision-adaptive operands of the sparse-loop attention (FlashLoop paper,
// Sec. 4.2 loop-aware sparse attention over the dequantised residual cache
// of Sec. 4.3).
//
// From the second loop on, a dequantised key or value is the int8 base plus
// residual levels.  For a column whose values stay small, and a query row
// whose values stay small, bf16 MFMA operands keep the products within the
// output tolerance, exactly as in the dense first loop; a large-magnitude
// column or query row needs more than bf16's 8 significant bits (the
// heavy-tailed cross-loop updates make some keys, values and queries tens of
// units large).  So each loop's selected columns and active rows are split
// per head into a "normal" and an "outlier" part:
//   k_class_flags    an outlier flag per selected column (some |K^| or |V^|
//                    of its dequantised row above the column bound) and per
//                    (active row, head) (some |q| above the row bound);
//   k_class_scan     one workgroup per head and kind: the columns' compact
//                    slot order [normal | pad to 64 | outlier] and the rows'
//                    order [normal | outlier], each part in selection order.
// k_attn_ad then runs every (normal row tile, normal column tile) with plain
// bf16 operands in 64-column tiles, outlier row tiles over normal columns
// with hi + lo keys (scores as hi.q + lo.q) and single P, V, and every tile
// of outlier columns with hi + lo pairs throughout (P.V as hi.hi + hi.lo +
// lo.hi), the last two kinds in 32-column tiles, in one online softmax.  All
// kinds occupy the same LDS: a 64-column bf16 K / V^T tile, or a 32-column
// hi and lo pair.
#include <type_traits>

#include "fl_device.h"
#include "fl_kernels.h"

namespace fl {

// ---------------------------------------------------------------------------
// exclusive block scan of one int per thread (1024 threads); returns the
// prefix and sets *total
__device__ __forceinline__ int block_scan_1024(int v, int* sh, int* total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[w] = x;
    __syncthreads();
    if (w == 0) {
        int s = lane < 16 ? sh[lane] : 0;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int y = __shfl_up(s, o);
            if (lane >= o) s += y;
        }
        if (lane < 16) sh[16 + lane] = s;  // inclusive over waves
    }
    __syncthreads();
    const int base = w > 0 ? sh[16 + w - 1] : 0;
    *total = sh[16 + 15];
    __syncthreads();
    return base + x - v;
}

// Class flags, one launch for both kinds:
//  * blocks [0, ncolblk): selected column p of head h is an outlier when
//    some |K^| or |V^| of its dequantised row (levels 0..upto, the values
//    the gather writes) exceeds tau_col or is not finite; D/8 threads per
//    column, 8 channels each; or, given the cache's per-token classes (kept
//    by the quantiser with the same bound), one lookup per column;
//  * the rest: active row t of head h is an outlier when max |q| exceeds
//    tau_row or is not finite; 16 lanes per (row, head), kRowItems of them
//    per lane group (the items of one pass are consecutive (row, head)
//    pairs, so the query reads coalesce).
// The flag planes have 16-byte aligned rows (strides cstride, rstride).
constexpr int kRowItems = 4;
template <int D, int NB>
__global__ __launch_bounds__(256) void k_class_flags(fl_kv_cache c, int upto, const int32_t* __restrict__ sel,
                                                     int k, int ncolblk, float tau_col,
                                                     const uint8_t* __restrict__ cls,
                                                     uint8_t* __restrict__ colflags, int cstride,
                                                     const void* __restrict__ q, int dtype, int q_gathered,
                                                     const int32_t* __restrict__ active, int n, float tau_row,
                                                     uint8_t* __restrict__ rowflags, int rstride) {
    const int tid = threadIdx.x;
    const int H = c.H;
    auto amax = [](float m, float a) { a = fabsf(a); return a <= m ? m : (a > m ? a : INFINITY); };
    if ((int)blockIdx.x < ncolblk && cls) {  // classes kept by the quantiser: one column per thread
        const int per_head = (k + 255) / 256;
        const int h = blockIdx.x / per_head;
        const int p = (blockIdx.x % per_head) * 256 + tid;
        if (p < k) {
            const long o = (sel ? (long)sel[(long)h * k + p] : (long)p) * H + h;
            colflags[(long)h * cstride + p] = (cls[o] | cls[(long)c.N * H + o]) ? 1 : 0;
        }
        return;
    }
    if ((int)blockIdx.x < ncolblk) {
        constexpr int TPC = D / 8, CPB = 256 / TPC;
        const int per_head = (k + CPB - 1) / CPB;
        const int h = blockIdx.x / per_head;
        const int p = (blockIdx.x % per_head) * CPB + tid / TPC;
        const int c0 = (tid % TPC) * 8;
        const bool live = p < k;
        float m = 0.0f;
        if (live) {
            const long j = sel ? sel[(long)h * k + p] : p;
            float x[2][8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[0][e] = x[1][e] = 0.0f;
            if constexpr (NB > 0)  // the gather's batched level walk (NB > kDeqBatch: chunks)
                deq_col8_kv<NB <= kDeqBatch ? NB : kDeqBatch, (NB > kDeqBatch)>(c, upto, j, H * D, h * D + c0,
                                                                                 x[0], x[1]);
            else
#pragma unroll
                for (int which = 0; which < 2; ++which) deq_col8(c, upto, which, j, H * D, h * D + c0, x[which]);
#pragma unroll
            for (int which = 0; which < 2; ++which)
#pragma unroll
                for (int e = 0; e < 8; ++e) m = amax(m, x[which][e]);
        }
#pragma unroll
        for (int o = 1; o < TPC; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        if (live && tid % TPC == 0) colflags[(long)h * cstride + p] = !(m <= tau_col);
        return;
    }
    constexpr int CPL = D / 16;  // channels per lane (8 or 4)
    const int nh = n * H;
    const int ngroups = (gridDim.x - ncolblk) * 16;
    const int g = (blockIdx.x - ncolblk) * 16 + (tid >> 4);
    const int sub = tid & 15;
    float x[kRowItems][8];
    int tt[kRowItems], hh[kRowItems];
#pragma unroll
    for (int u = 0; u < kRowItems; ++u) {
        const int item = g + u * ngroups;
        tt[u] = item / H;
        hh[u] = item - tt[u] * H;
#pragma unroll
        for (int i = 0; i < 8; ++i) x[u][i] = 0.0f;
        if (item < nh) {
            const long row = q_gathered ? (long)tt[u] : (long)active[tt[u]];
            const long e = (row * H + hh[u]) * D + sub * CPL;
            if (CPL == 8) {
                load8_f32(q, e, dtype, x[u]);
            } else if (dtype == FL_BF16) {
                const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(q) + e);
                x[u][0] = __uint_as_float(w.x << 16); x[u][1] = __uint_as_float(w.x & 0xffff0000u);
                x[u][2] = __uint_as_float(w.y << 16); x[u][3] = __uint_as_float(w.y & 0xffff0000u);
            } else {
                const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(q) + e);
                x[u][0] = f.x; x[u][1] = f.y; x[u][2] = f.z; x[u][3] = f.w;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kRowItems; ++u) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) m = amax(m, x[u][i]);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        if (g + u * ngroups < nh && sub == 0) rowflags[(long)hh[u] * rstride + tt[u]] = !(m <= tau_row);
    }
}

// Orders from the flags, one workgroup per (kind, head):
//  * blocks [0, H): the compact slot order of head h's columns,
//    [normal | pad to a multiple of 64 | outlier], each part in selection
//    order (perm[h][slot] = selection index, -1 for pads), colseg = sizes;
//  * blocks [H, 2H): head h's row order [normal | outlier] (indices into
//    the active list), rowseg = the normal count.
// Each thread reads a run of 16 flags with one 16-byte load (the planes' rows
// are 16-byte aligned), one pass per 16K flags.
__global__ __launch_bounds__(1024) void k_class_scan(const uint8_t* __restrict__ colflags, int k, int cstride,
                                                     int kp, int32_t* __restrict__ perm,
                                                     int32_t* __restrict__ colseg,
                                                     const uint8_t* __restrict__ rowflags, int n, int rstride,
                                                     int H, int32_t* __restrict__ rowperm,
                                                     int32_t* __restrict__ rowseg) {
    constexpr int E = 16, CH = 1024 * E;
    __shared__ int sh[32];
    const bool cols = (int)blockIdx.x < H;
    const int h = cols ? blockIdx.x : blockIdx.x - H;
    const int tid = threadIdx.x;
    const int len = cols ? k : n;
    const uint8_t* f = cols ? colflags + (long)h * cstride : rowflags + (long)h * rstride;
    int32_t* out = cols ? perm + (long)h * kp : rowperm + (long)h * n;
    if (cols)
        for (int p = tid; p < kp; p += 1024) out[p] = -1;
    // flags of run base + 16 tid .. +15 as bits (bit i: entry i is an outlier,
    // entries past len count as neither part)
    auto run = [&](int base, uint32_t& outl, uint32_t& live) {
        const int x0 = base + tid * E;
        outl = 0;
        live = 0;
        if (x0 < len) {
            const uint4 w = *reinterpret_cast<const uint4*>(f + x0);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < E; ++i)
                if (x0 + i < len) {
                    live |= 1u << i;
                    if ((ws[i >> 2] >> (8 * (i & 3))) & 255u) outl |= 1u << i;
                }
        }
    };
    if (len <= CH) {  // one pass: one read of the flags, one scan
        uint32_t outl, live;
        run(0, outl, live);
        int n_norm;
        int in_ = block_scan_1024(__popc(live & ~outl), sh, &n_norm);
        const int seg1 = cols ? (n_norm + 63) / 64 * 64 : n_norm;
        // (the scan's barriers order the -1 fill before these writes)
        int io = seg1 + (min(tid * E, len) - in_);
#pragma unroll
        for (int i = 0; i < E; ++i) {
            if (!((live >> i) & 1u)) continue;
            if ((outl >> i) & 1u) out[io++] = tid * E + i;
            else out[in_++] = tid * E + i;
        }
        if (tid == 0) {
            if (cols) {
                colseg[2 * h] = n_norm;
                colseg[2 * h + 1] = len - n_norm;
            } else {
                rowseg[h] = n_norm;
            }
        }
        return;
    }
    int cnt = 0;
    for (int base = 0; base < len; base += CH) {
        uint32_t outl, live;
        run(base, outl, live);
        cnt += __popc(live & ~outl);
    }
    int n_norm;
    block_scan_1024(cnt, sh, &n_norm);
    const int seg1 = cols ? (n_norm + 63) / 64 * 64 : n_norm;
    // (the scans' barriers order the -1 fill before these writes)
    int done = 0;  // normal entries of the earlier passes
    for (int base = 0; base < len; base += CH) {
        uint32_t outl, live;
        run(base, outl, live);
        int pass_norm;
        int in_ = done + block_scan_1024(__popc(live & ~outl), sh, &pass_norm);
        // outlier entries before this run: all entries before it minus the normal ones
        int io = seg1 + (min(base + tid * E, len) - in_);
#pragma unroll
        for (int i = 0; i < E; ++i) {
            if (!((live >> i) & 1u)) continue;
            const int x = base + tid * E + i;
            if ((outl >> i) & 1u) out[io++] = x;
            else out[in_++] = x;
        }
        done += pass_norm;
    }
    if (tid == 0) {
        if (cols) {
            colseg[2 * h] = n_norm;
            colseg[2 * h + 1] = len - n_norm;
        } else {
            rowseg[h] = n_norm;
        }
    }
}

// ---------------------------------------------------------------------------
constexpr int kAdBM = 128;  // query rows per workgroup (4 waves x 32)

// Attention of the loop's active rows over its selected columns with
// precision-adaptive operands (see the top of this file).  One workgroup =
// 128 rows of one head in the head's row order; tiles of the normal column
// part are plain 64-column tiles when all 128 rows are normal, else hi/lo
// 32-column tiles; the outlier part is always hi/lo.  The K / V^T tiles
// are copied by LDS-DMA into two buffers (the next tile lands while this one
// is computed), XOR-swizzled as in the other attention kernels.
template <int D, int MODE>
__global__ __launch_bounds__(256, 2) void k_attn_ad(AttnParams P) {
    constexpr int KB = 64 * D * 2;          // bytes of one K (or V^T) region
    constexpr int KCPR = D * 2 / 16;        // 16-byte chunks per K row
    constexpr int MPW = KB / 1024 / 4;      // LDS-DMA instructions per wave per region
    constexpr int HPW = MPW / 2;            //   ... per half region (a hi or lo part)
    __shared__ __attribute__((aligned(1024))) __bf16 sK0[KB / 2];
    __shared__ __attribute__((aligned(1024))) __bf16 sV0[KB / 2];
    __shared__ __attribute__((aligned(1024))) __bf16 sK1[KB / 2];
    __shared__ __attribute__((aligned(1024))) __bf16 sV1[KB / 2];
    __shared__ __attribute__((aligned(256))) int sC0[64];
    __shared__ __attribute__((aligned(256))) int sC1[64];
    __shared__ int s_mn[4], s_mx[4], s_bd[6];
    constexpr bool RB = MODE == MODE_ATTN_RB;  // rebuild pass first (see the pass below)
    const int n_tiles = (P.n + kAdBM - 1) / kAdBM;
    int tile, h;
    block_coords(P.xcd_remap, n_tiles, P.H, tile, h);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, half = lane >> 5;
    const int tt = tile * kAdBM + w * 32 + r;  // place in the head's row order
    const bool valid = tt < P.n;
    const int32_t* cpos_h = P.cpos + (long)h * P.kp;
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(cpos_h, (uint32_t)P.kp * 4);
    // Prologue: the head's column positions are copied into the second tile
    // buffer (idle until the first tile is computed) while the row indices
    // are looked up; the causal bounds are then searched in LDS, and the
    // query fragments are loaded together with the first tile.
    const bool cpos_lds = P.kp * 4 <= KB;
    const int32_t* cpos_old_h = RB ? P.cpos_old + (long)h * P.kp : nullptr;
    const __amdgpu_buffer_rsrc_t rC_old = make_rsrc(RB ? cpos_old_h : cpos_h, (uint32_t)P.kp * 4);
    if (cpos_lds)
        for (int m = w; m * 1024 < P.kp * 4; m += 4) {
            buf_dma16(rC, reinterpret_cast<char*>(sK1) + m * 1024, lane * 16, m * 1024);
            if (RB) buf_dma16(rC_old, reinterpret_cast<char*>(sV1) + m * 1024, lane * 16, m * 1024);
        }
    const int nn_l = P.colseg[2 * h], no_l = P.colseg[2 * h + 1];
    const int rseg_l = P.rowseg ? P.rowseg[h] : 0;
    const int t = valid ? (P.rowperm ? P.rowperm[(long)h * P.n + tt] : tt) : 0;
    const int rowpos = valid ? P.active[t] : -1;
    {
        int mn = valid ? rowpos : 0x7fffffff, mx = rowpos;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            mn = min(mn, __shfl_xor(mn, o));
            mx = max(mx, __shfl_xor(mx, o));
        }
        if (lane == 0) { s_mn[w] = mn; s_mx[w] = mx; }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this lane's position copies landed
    __syncthreads();
    const int minpos = __builtin_amdgcn_readfirstlane(min(min(s_mn[0], s_mn[1]), min(s_mn[2], s_mn[3])));
    const int maxpos = __builtin_amdgcn_readfirstlane(max(max(s_mx[0], s_mx[1]), max(s_mx[2], s_mx[3])));
    // the two column parts and their causal bounds for these rows: wave w
    // finds bound w (columns <= the last / first row position, in the normal /
    // outlier part)
    const int nn = __builtin_amdgcn_readfirstlane(nn_l);
    const int no = __builtin_amdgcn_readfirstlane(no_l);
    const int seg1 = (nn + 63) / 64 * 64;
    {
        const int v = w & 1 ? minpos : maxpos;
        const int off = w < 2 ? 0 : seg1, len = w < 2 ? nn : no;
        const int b = cpos_lds ? wave_ubound(reinterpret_cast<const int32_t*>(sK1) + off, len, v)
                               : wave_ubound(cpos_h + off, len, v);
        if (lane == 0) s_bd[w] = b;
        if (RB && w < 2) {  // the previous side's bounds (all its columns plain)
            const int b2 = cpos_lds ? wave_ubound(reinterpret_cast<const int32_t*>(sV1), P.k_old, v)
                                    : wave_ubound(cpos_old_h, P.k_old, v);
            if (lane == 0) s_bd[4 + w] = b2;
        }
    }
    __syncthreads();
    const int pe0 = __builtin_amdgcn_readfirstlane(s_bd[0]);
    const int pf0 = __builtin_amdgcn_readfirstlane(s_bd[1]);
    const int pe1 = __builtin_amdgcn_readfirstlane(s_bd[2]);
    const int pf1 = __builtin_amdgcn_readfirstlane(s_bd[3]);
    const int tile_end = min(tile * kAdBM + kAdBM, P.n);
    const bool rnorm = P.rowseg ? tile_end <= __builtin_amdgcn_readfirstlane(rseg_l) : false;
    const int W0 = rnorm ? 64 : 32;
    const int T0 = (pe0 + W0 - 1) / W0;
    const int T = T0 + (pe1 + 31) / 32;
    bf16x8 qf[D / 16];
    auto load_q = [&](const void* qsrc, int gathered) {
        const long qrow = gathered ? (long)t : (long)rowpos;
        const long qoff = (qrow * P.H + h) * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            if (valid) qf[kk] = load8_bf16(qsrc, qoff + 16 * kk, P.dtype);
            else {
#pragma unroll
                for (int i = 0; i < 8; ++i) qf[kk][i] = (__bf16)0.0f;
            }
        }
    };
    if (RB) load_q(P.q_old, P.q_old_gathered);
    else load_q(P.q, P.q_gathered);
    const long rh = valid ? (long)rowpos * P.H + h : 0;
    // reb: the pass in progress is a cache rebuild (fixed exponent reference
    // lse_prev, probabilities weighted by w = 1 - M_U_prev).  The weight
    // folds into the reference, p w = 2^(s c2 - (lse_prev2 - log2 w)); a
    // weight that rounding left at or below zero (M_U_prev >= 1) gives p = 0.
    bool reb = MODE != MODE_ATTN;
    float lse_prev2 = 0.0f, mu_prev = 0.0f;
    if (reb && valid) {
        mu_prev = P.mass_u[rh];
        const float wgt = 1.0f - mu_prev;
        lse_prev2 = P.lse[rh] * 1.4426950408889634f - (wgt > 0.0f ? __log2f(wgt) : -INFINITY);
    }

    const long koff = (long)h * P.kp * D;
    const long voff = (long)h * (P.kp / 64) * D * 64;
    const uint32_t kbytes = (uint32_t)P.kp * D * 2;
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(P.Kc + koff, kbytes), rV = make_rsrc(P.Vt + voff, kbytes);
    const __amdgpu_buffer_rsrc_t rKl = make_rsrc(P.Kc_lo + koff, kbytes), rVl = make_rsrc(P.Vt_lo + voff, kbytes);
    // per-lane byte offsets: plain tiles (64 keys: K rows of D, V^T rows of 64
    // keys) and hi/lo tiles (32 keys: each part half a region, V^T rows of 32
    // keys inside the stored 64-key rows)
    uint32_t kvo[MPW], vvo[MPW], kso[HPW], vso[HPW];
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
        const int off = (w * MPW + i) * 1024 + lane * 16;
        const int kr = off / (D * 2), kc = ((off % (D * 2)) >> 4) ^ swz<KCPR>(kr);
        kvo[i] = kr * (D * 2) + kc * 16;
        const int vr = off / 128, vc = ((off % 128) >> 4) ^ swz<8>(vr);
        vvo[i] = vr * 128 + vc * 16;
    }
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        const int off = (w * HPW + i) * 1024 + lane * 16;
        const int kr = off / (D * 2), kc = ((off % (D * 2)) >> 4) ^ swz<KCPR>(kr);
        kso[i] = kr * (D * 2) + kc * 16;
        const int vr = off / 64, vc = ((off % 64) >> 4) ^ swz<4>(vr);
        vso[i] = vr * 128 + vc * 16;
    }
    // tile i: its first column slot and kind: plain 64-column tiles (normal
    // rows, normal columns), 32-column tiles with hi/lo keys and single P, V
    // (outlier rows, normal columns: only the scores need the keys' lo part,
    // P.V over values within the column bound keeps bf16), and 32-column
    // hi/lo tiles (outlier columns)
    auto tile_p0 = [&](int i) { return i < T0 ? i * W0 : seg1 + (i - T0) * 32; };
    auto tile_split = [&](int i) { return i >= T0 || !rnorm; };
    auto tile_full = [&](int i) { return i >= T0; };
    auto issue = [&](int i, __bf16* sK, __bf16* sV, int* sC) {
        const int p0 = tile_p0(i);
        if (!tile_split(i)) {
            const uint32_t ks = (uint32_t)p0 * D * 2, vs = (uint32_t)(p0 / 64) * D * 64 * 2;
#pragma unroll
            for (int j = 0; j < MPW; ++j) {
                const int m = w * MPW + j;
                buf_dma16(rK, reinterpret_cast<char*>(sK) + m * 1024, kvo[j], ks);
                buf_dma16(rV, reinterpret_cast<char*>(sV) + m * 1024, vvo[j], vs);
            }
            if (w == 0) buf_dma4(rC, sC, lane * 4, p0 * 4);
        } else {
            const uint32_t ks = (uint32_t)p0 * D * 2;
            const uint32_t vs = ((uint32_t)(p0 / 64) * D * 64 + p0 % 64) * 2;
            const bool vlo = tile_full(i);
#pragma unroll
            for (int part = 0; part < 2; ++part) {
#pragma unroll
                for (int j = 0; j < HPW; ++j) {
                    const int m = part * (HPW * 4) + w * HPW + j;
                    buf_dma16(part ? rKl : rK, reinterpret_cast<char*>(sK) + m * 1024, kso[j], ks);
                    if (part == 0 || vlo)
                        buf_dma16(part ? rVl : rV, reinterpret_cast<char*>(sV) + m * 1024, vso[j], vs);
                }
            }
            if (w == 0 && lane < 32) buf_dma4(rC, sC, lane * 4, p0 * 4);
        }
    };

    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
    if constexpr (RB) {
        // the rebuild pass accumulates onto -o_prev (its exponent reference
        // is fixed, so the accumulators are never rescaled): it ends holding
        // -O_U, and the previous output's loads overlap the first tiles
        if (valid) {
            const float* orow_prev = P.out + rh * D;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int jq = 0; jq < 4; ++jq) {
                    const float4 op = *reinterpret_cast<const float4*>(orow_prev + 32 * dt + jq * 8 + half * 4);
                    o[dt][4 * jq + 0] = -op.x;
                    o[dt][4 * jq + 1] = -op.y;
                    o[dt][4 * jq + 2] = -op.z;
                    o[dt][4 * jq + 3] = -op.w;
                }
        }
    }
    float m_run = -INFINITY, l_run = 0.0f;

    // online softmax over one 32-column block's scores (shared by both kinds)
    auto softmax_ref = [&](f32x16* s, int KT) -> float {
        if (reb) return lse_prev2;
        float tmax = -INFINITY;
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int j = 0; j < 16; ++j) tmax = fmaxf(tmax, s[kt][j]);
        tmax = max_xor32(tmax);
        const float m_new = fmaxf(m_run, tmax * P.c2);
        // lazy exponent reference: rescale only when some row's max passes
        // it by more than 8 (log2 units); the result does not depend on it
        if (__ballot(m_new > m_run + 8.0f)) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.0f : m_new));
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
            m_run = m_new;
        }
        return m_run == -INFINITY ? 0.0f : m_run;
    };

    // a plain tile at column slot p0; columns from slot pf on may lie past the first row
    auto compute_plain = [&](int p0, int pf, const __bf16* sK, const __bf16* sV, const int* sC)
        {
        f32x16 s[2];
        __builtin_amdgcn_s_setprio(1);
        // the two 32-key blocks' chains alternate (each keeps its own order)
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int key = 32 * kt + r;
                const int e = key * D + (((2 * kk + half) ^ swz<KCPR>(key)) << 3);
                s[kt] = mfma32(*reinterpret_cast<const bf16x8*>(&sK[e]), qf[kk], s[kt]);
            }
        sched_reads_ahead16();
        __builtin_amdgcn_s_setprio(0);
        if (p0 + 64 > pf) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = 32 * kt + (j >> 2) * 8 + half * 4 + (j & 3);
                    if (sC[key] > rowpos) s[kt][j] = -INFINITY;
                }
        }
        const float m_use = softmax_ref(s, 2);
        bf16x8 pb[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float pj = __builtin_amdgcn_exp2f(fmaf(s[kt][j], P.c2, -m_use));
                pb[kt][j >> 3][j & 7] = (__bf16)pj;
                l_run += pj;
            }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const int row = 32 * dt + r;
#pragma unroll
                for (int jh = 0; jh < 2; ++jh) {
                    const int e = row * 64 + (((4 * kt + 2 * jh + half) ^ swz<8>(row)) << 3);
                    o[dt] = mfma32(*reinterpret_cast<const bf16x8*>(&sV[e]), pb[kt][jh], o[dt]);
                }
            }
    };

    auto compute_split = [&](auto full, int i, const __bf16* sK, const __bf16* sV, const int* sC) {
        constexpr bool FULL = decltype(full)::value;
        const int p0 = tile_p0(i);
        const bool seg = i >= T0;
        const __bf16* sKl = sK + 32 * D;       // lo part: second half of the region
        const __bf16* sVl = sV + 32 * D;
        f32x16 s[1];
        s[0] = f32x16{};
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const int e = r * D + (((2 * kk + half) ^ swz<KCPR>(r)) << 3);
            s[0] = mfma32(*reinterpret_cast<const bf16x8*>(&sK[e]), qf[kk], s[0]);
            s[0] = mfma32(*reinterpret_cast<const bf16x8*>(&sKl[e]), qf[kk], s[0]);
        }
        sched_reads_ahead16();
        __builtin_amdgcn_s_setprio(0);
        const bool mask = seg ? (p0 - seg1) + 32 > pf1 : p0 + 32 > pf0;
        if (mask) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = (j >> 2) * 8 + half * 4 + (j & 3);
                if (sC[key] > rowpos) s[0][j] = -INFINITY;
            }
        }
        const float m_use = softmax_ref(s, 1);
        bf16x8 pb[2], pl[2];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float pj = __builtin_amdgcn_exp2f(fmaf(s[0][j], P.c2, -m_use));
            const __bf16 hi = (__bf16)pj;
            pb[j >> 3][j & 7] = hi;
            if (FULL) pl[j >> 3][j & 7] = (__bf16)(pj - (float)hi);
            l_run += pj;
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const int row = 32 * dt + r;
#pragma unroll
            for (int jh = 0; jh < 2; ++jh) {
                const int e = row * 32 + (((2 * jh + half) ^ swz<4>(row)) << 3);
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sV[e]);
                o[dt] = mfma32(a, pb[jh], o[dt]);
                if (FULL) {
                    const bf16x8 al = *reinterpret_cast<const bf16x8*>(&sVl[e]);
                    o[dt] = mfma32(a, pl[jh], o[dt]);
                    o[dt] = mfma32(al, pb[jh], o[dt]);
                }
            }
        }
    };

    float mu_rb = 0.0f;  // RB: M_U of these rows after the rebuild pass
    if constexpr (RB) {
        // Rebuild pass (subtract form, as MODE_REBUILD): the previous loop's
        // probabilities over its columns S (all plain tiles), weighted by
        // 1 - M_U_prev; O_U = o_prev - sum_S P V^, M_U = 1 - sum_S P are
        // written for these rows, then the attention pass starts afresh.
        const int peA = __builtin_amdgcn_readfirstlane(s_bd[4]);
        const int pfA = __builtin_amdgcn_readfirstlane(s_bd[5]);
        const int TA = (peA + 63) / 64;
        const __amdgpu_buffer_rsrc_t rKo = make_rsrc(P.Kc_old + koff, kbytes), rVo = make_rsrc(P.Vt_old + voff, kbytes);
        auto issue_old = [&](int i, __bf16* sK, __bf16* sV, int* sC) {
            const uint32_t ks = (uint32_t)(64 * i) * D * 2, vs = (uint32_t)i * D * 64 * 2;
#pragma unroll
            for (int j = 0; j < MPW; ++j) {
                const int m = w * MPW + j;
                buf_dma16(rKo, reinterpret_cast<char*>(sK) + m * 1024, kvo[j], ks);
                buf_dma16(rVo, reinterpret_cast<char*>(sV) + m * 1024, vvo[j], vs);
            }
            if (w == 0) buf_dma4(rC_old, sC, lane * 4, 64 * i * 4);
        };
        if (TA > 0) issue_old(0, sK0, sV0, sC0);
        for (int i = 0; i < TA;) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (i + 1 < TA) issue_old(i + 1, sK1, sV1, sC1);
            compute_plain(64 * i, pfA, sK0, sV0, sC0);
            if (++i >= TA) break;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (i + 1 < TA) issue_old(i + 1, sK0, sV0, sC0);
            compute_plain(64 * i, pfA, sK1, sV1, sC1);
            ++i;
        }
        // the attention pass's queries: loads in flight during the stores
        load_q(P.q, P.q_gathered);
        const float l_a = l_run + __shfl_xor(l_run, 32);
        mu_rb = 1.0f - l_a;
        if (valid) {
            float* ourow = P.out_u + rh * D;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int jq = 0; jq < 4; ++jq)
                    *reinterpret_cast<float4*>(ourow + 32 * dt + jq * 8 + half * 4) =
                        make_float4(-o[dt][4 * jq + 0], -o[dt][4 * jq + 1], -o[dt][4 * jq + 2],
                                    -o[dt][4 * jq + 3]);
            if (half == 0) P.mass_u[rh] = mu_rb;
        }
        // the attention pass: its own queries, fresh accumulators
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
        l_run = 0.0f;
        m_run = -INFINITY;
        reb = false;
        __syncthreads();  // every wave is done with the tile buffers
    }

    // Tile i sits in buffer i & 1.  The tile kinds occupy consecutive ranges
    // ([0, T0) plain or hi/lo-key tiles, [T0, T) full hi/lo tiles), and each
    // range runs in a loop of its own: with one kind per loop body the
    // accumulators keep their registers from tile to tile (a loop that
    // branches between kinds gets them copied at every join).
    auto run = [&](auto kind, auto odd, int ib, int ie) {
        constexpr int KIND = decltype(kind)::value;
        constexpr bool ODD = decltype(odd)::value;
        __bf16* const kA = ODD ? sK1 : sK0;
        __bf16* const vA = ODD ? sV1 : sV0;
        int* const cA = ODD ? sC1 : sC0;
        __bf16* const kB = ODD ? sK0 : sK1;
        __bf16* const vB = ODD ? sV0 : sV1;
        int* const cB = ODD ? sC0 : sC1;
        auto step = [&](int i, const __bf16* sK, const __bf16* sV, const int* sC) {
            if constexpr (KIND == 0) compute_plain(tile_p0(i), pf0, sK, sV, sC);
            else compute_split(std::integral_constant<bool, KIND == 2>{}, i, sK, sV, sC);
        };
        for (int i = ib; i < ie;) {
            __builtin_amdgcn_s_waitcnt(0); // this lane's copies of the current tile landed
            __syncthreads();               // ... every lane's; the other buffer is free
            if (i + 1 < T) issue(i + 1, kB, vB, cB);
            step(i, kA, vA, cA);
            if (++i >= ie) break;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (i + 1 < T) issue(i + 1, kA, vA, cA);
            step(i, kB, vB, cB);
            ++i;
        }
    };
    using plain_k = std::integral_constant<int, 0>;
    using split_k = std::integral_constant<int, 1>;
    using full_k = std::integral_constant<int, 2>;
    if (T > 0) issue(0, sK0, sV0, sC0);
    if (rnorm) run(plain_k{}, std::false_type{}, 0, T0);
    else run(split_k{}, std::false_type{}, 0, T0);
    if (T0 & 1) run(full_k{}, std::true_type{}, T0, T);
    else run(full_k{}, std::false_type{}, T0, T);

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!valid) return;
    float* orow = P.out + rh * D;
    if (MODE == MODE_ATTN || RB) {
        // every load of the caches before the first store (the stores could
        // alias them for the compiler, which would then serialise each pair)
        const bool cached = RB || P.cache_op != FL_CACHE_ZERO;
        const float* ourow = P.out_u + rh * D;
        float4 uc[D / 32][4];
        float mu = 0.0f;
        if (cached) {
            mu = RB ? mu_rb : P.mass_u[rh];
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int jq = 0; jq < 4; ++jq)
                    uc[dt][jq] = *reinterpret_cast<const float4*>(ourow + 32 * dt + jq * 8 + half * 4);
        } else {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int jq = 0; jq < 4; ++jq) uc[dt][jq] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        const float scale = l_tot > 0.0f ? (1.0f - mu) / l_tot : 0.0f;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jq = 0; jq < 4; ++jq) {
                const int d0 = 32 * dt + jq * 8 + half * 4;
                const float4 u = uc[dt][jq];
                float4 v;
                v.x = o[dt][4 * jq + 0] * scale + u.x;
                v.y = o[dt][4 * jq + 1] * scale + u.y;
                v.z = o[dt][4 * jq + 2] * scale + u.z;
                v.w = o[dt][4 * jq + 3] * scale + u.w;
                *reinterpret_cast<float4*>(orow + d0) = v;
                if (P.out_bf) {
                    const __bf16 b4[4] = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
                    uint16_t u16[4];
                    __builtin_memcpy(u16, b4, sizeof(u16));
                    *reinterpret_cast<uint2*>(P.out_bf + ((long)t * P.H + h) * D + d0) =
                        make_uint2(u16[0] | ((uint32_t)u16[1] << 16), u16[2] | ((uint32_t)u16[3] << 16));
                }
            }
        if (half == 0)
            P.lse[rh] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    } else {
        // subtract form: O_U = o_prev - sum_S P V^, M_U = 1 - sum_S P;
        // additive form: O_U += sum_pruned P V^, M_U += sum_pruned P
        float* ourow = P.out_u + rh * D;
        const float* base = MODE == MODE_REBUILD ? orow : ourow;
        const float sg = MODE == MODE_REBUILD ? -1.0f : 1.0f;
        float4 bc[D / 32][4];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jq = 0; jq < 4; ++jq)
                bc[dt][jq] = *reinterpret_cast<const float4*>(base + 32 * dt + jq * 8 + half * 4);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jq = 0; jq < 4; ++jq) {
                const int d0 = 32 * dt + jq * 8 + half * 4;
                const float4 op = bc[dt][jq];
                float4 v;
                v.x = op.x + sg * o[dt][4 * jq + 0];
                v.y = op.y + sg * o[dt][4 * jq + 1];
                v.z = op.z + sg * o[dt][4 * jq + 2];
                v.w = op.w + sg * o[dt][4 * jq + 3];
                *reinterpret_cast<float4*>(ourow + d0) = v;
            }
        if (half == 0) P.mass_u[rh] = MODE == MODE_REBUILD ? 1.0f - l_tot : mu_prev + l_tot;
    }
}

// ---------------------------------------------------------------------------
// per head: the columns of S_prev absent from S (S a subset of S_prev, both
// ascending), in ascending order; one workgroup per head
__global__ __launch_bounds__(1024) void k_set_diff(const int32_t* __restrict__ sel_prev, int k_prev,
                                                   const int32_t* __restrict__ sel, int k,
                                                   int32_t* __restrict__ pruned) {
    __shared__ int sh[32];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int32_t* a = sel_prev + (long)h * k_prev;
    const int32_t* b = sel + (long)h * k;
    const int per = (k_prev + 1023) / 1024;
    const int t0 = tid * per, t1 = min(t0 + per, k_prev);
    auto kept = [&](int x) {
        int lo = 0, hi = k;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (b[mid] < x) lo = mid + 1; else hi = mid;
        }
        return lo < k && b[lo] == x;
    };
    int cnt = 0;
    for (int t = t0; t < t1; ++t) cnt += kept(a[t]) ? 0 : 1;
    int total;
    int o = block_scan_1024(cnt, sh, &total);
    int32_t* out = pruned + (long)h * (k_prev - k);
    for (int t = t0; t < t1; ++t)
        if (!kept(a[t]) && o < k_prev - k) out[o++] = a[t];
}

hipError_t launch_set_diff(const int32_t* sel_prev, int k_prev, const int32_t* sel, int k, int H,
                           int32_t* pruned, hipStream_t st) {
    hipLaunchKernelGGL(k_set_diff, dim3(H), dim3(1024), 0, st, sel_prev, k_prev, sel, k, pruned);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
hipError_t launch_classify(const fl_kv_cache& c, int upto, const int32_t* sel, int k, int kp,
                           const void* q, int dtype, int q_gathered, const int32_t* active, int n,
                           float tau_col, float tau_row, uint8_t* colflags, int32_t* perm, int32_t* colseg,
                           uint8_t* rowflags, int32_t* rowperm, int32_t* rowseg, const uint8_t* cls,
                           hipStream_t st) {
    const int H = c.H;
    const int cpb = cls ? 256 : 256 / (c.d / 8);
    const int ncolblk = H * ((k + cpb - 1) / cpb);
    const int nrowblk = (int)(((long)n * H + 16 * kRowItems - 1) / (16 * kRowItems));
    const unsigned nblk = (unsigned)(ncolblk + nrowblk);
    const int cstride = kp, rstride = (int)class_row_stride(n);
    // the columns' level walk: batched as in the gather where the cache allows
    const int nb = cls || !deq_batch_ok(c, upto) ? 0 : upto < kDeqBatch ? upto + 1 : kDeqBatch + 1;
#define FL_FLAGS(D_, NB_)                                                                             \
    hipLaunchKernelGGL((k_class_flags<D_, NB_>), dim3(nblk), dim3(256), 0, st, c, upto, sel, k, ncolblk, \
                       tau_col, cls, colflags, cstride, q, dtype, q_gathered, active, n, tau_row, rowflags, rstride)
#define FL_FLAGS_B(D_) {                                                       \
        switch (nb) {                                                          \
        case 1: FL_FLAGS(D_, 1); break;                                        \
        case 2: FL_FLAGS(D_, 2); break;                                        \
        case 3: FL_FLAGS(D_, 3); break;                                        \
        case 4: FL_FLAGS(D_, 4); break;                                        \
        case 5: FL_FLAGS(D_, 5); break;                                        \
        default: FL_FLAGS(D_, 0);                                              \
        } }
    if (c.d == 128) FL_FLAGS_B(128) else FL_FLAGS_B(64)
#undef FL_FLAGS_B
#undef FL_FLAGS
    hipLaunchKernelGGL(k_class_scan, dim3(2 * H), dim3(1024), 0, st, colflags, k, cstride, kp, perm, colseg,
                       rowflags, n, rstride, H, rowperm, rowseg);
    return hipGetLastError();
}

hipError_t launch_attn_ad(int d, int mode, const AttnParams& P, hipStream_t st) {
    const int n_tiles = (P.n + kAdBM - 1) / kAdBM;
    AttnParams Q = P;
    Q.xcd_remap = (P.H % 8) == 0;
    const dim3 grid(n_tiles * P.H);
#define FL_AD(D_)                                                                                        \
    if (mode == MODE_ATTN) hipLaunchKernelGGL((k_attn_ad<D_, MODE_ATTN>), grid, dim3(256), 0, st, Q);        \
    else if (mode == MODE_REBUILD) hipLaunchKernelGGL((k_attn_ad<D_, MODE_REBUILD>), grid, dim3(256), 0, st, Q); \
    else if (mode == MODE_ATTN_RB) hipLaunchKernelGGL((k_attn_ad<D_, MODE_ATTN_RB>), grid, dim3(256), 0, st, Q); \
    else hipLaunchKernelGGL((k_attn_ad<D_, MODE_REBUILD_ADD>), grid, dim3(256), 0, st, Q);
    if (d == 128) { FL_AD(128) } else { FL_AD(64) }
#undef FL_AD
    return hipGetLastError();
}

} // namespace fl

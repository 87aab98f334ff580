// Sparse loop attention (FlashLoop paper, Sec. 4.2 loop-aware sparse
// attention; Sec. 4.4 compact buffers of the selected keys).
//
// Kernels (bf16 MFMA 32x32x16 on gfx950, fp32 softmax and accumulation):
//   k_gather_bf16   dequantise the selected columns of every head once per
//                   loop (base + residual chain) into a compact bf16 buffer:
//                   K as [H][kp][d] and V transposed per 64-column tile as
//                   [H][kp/64][d][64] (key order permuted inside each 16-key
//                   group so one 16-byte LDS read feeds one MFMA operand).
//   k_attn<MODE>    one workgroup = 128 gathered active query rows (4 waves x
//                   32 rows) of one head; loops over 64-column tiles of the
//                   head's selected columns up to the tile's causal bound.
//                   Each wave computes S^T = K Q^T (the lane owns one query
//                   row), masks j > i, runs the softmax in registers and
//                   accumulates O^T = V^T P^T.
//                   MODE_ATTN: online softmax, o = (1-M_U) o~ / l + O_U, lse.
//                   MODE_REBUILD: the previous loop's probabilities with its
//                   known lse: M_U = 1 - sum P_prev, O_U = o_prev - sum P_prev V.
//   k_attn_lds      the same attention over compact bf16 tiles copied by
//                   LDS-DMA into two buffers (the dequantise-once placement);
//   k_attn_lds_dq   its in-tile variant: each tile's quantised planes are
//                   copied into a staging buffer and expanded by the
//                   workgroup into the operand tile (Sec. 4.4 fuses the cache
//                   into the attention kernel).
//   k_colstat       column statistics c(j) = sum_i (1-M_U(i)) exp(s - lse(i))
//                   for the next loop's column ranking: one workgroup = 128
//                   selected columns (a wave keeps its 32 columns' keys in
//                   registers) sweeping the active query rows from the first
//                   causal one; per-lane sequential sums (deterministic).
#include "fl_device.h"
#include "fl_kernels.h"

namespace fl {

// four fp32 values rounded to bf16 (nearest-even) and stored as 8 bytes
__device__ __forceinline__ void store_bf16x4(__bf16* dst, float4 v) {
    const __bf16 b[4] = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
    uint16_t u[4];
    __builtin_memcpy(u, b, sizeof(u));
    *reinterpret_cast<uint2*>(dst) = make_uint2(u[0] | ((uint32_t)u[1] << 16), u[2] | ((uint32_t)u[3] << 16));
}

constexpr int BM = 128; // query rows per workgroup (4 waves x 32)
constexpr int BN = 64;  // columns per tile

__host__ __device__ __forceinline__ long round_up(long x, long m) { return (x + m - 1) / m * m; }

// stored offset (0..15) inside a 16-key group -> key offset
__device__ __forceinline__ int vt_key_of_slot(int so) {
    return (so >> 3) * 4 + ((so >> 2) & 1) * 8 + (so & 3);
}

// ---------------------------------------------------------------------------
// Compact gather + dequantisation of the selected columns (levels 0..upto).
// With X3 (fp32 inputs) a second "lo" copy holds the bf16 rounding of
// x - bf16(x), so that products can be formed as hi*hi + hi*lo + lo*hi.
// One thread per 8 channels of a column (D/8 threads per column), so a
// workgroup covers GC = 2048/D columns -- one or two of the 16-key groups of
// the transposed V tile, which it writes on its own; a column's dequantisation
// chain walks the levels in order, stopping at the first one the token is
// absent from (the sets are nested).  NB > 0: the levels in chunks of NB,
// each chunk's slots, then its codes and scales, loaded together
// (deq_col8_kv); the kernel then stays at eight waves per SIMD, so a whole
// gather's workgroups are resident at once.
template <int D>
constexpr int gather_cols() { return 256 / (D / 8); }

template <int D, bool X3, int NB>
__global__ __launch_bounds__(256, 8) void k_gather_bf16(fl_kv_cache c, int upto,
                                                     const int32_t* __restrict__ sel, int k,
                                                     int kp, __bf16* __restrict__ Kc,
                                                     __bf16* __restrict__ Vt,
                                                     __bf16* __restrict__ Kc_lo,
                                                     __bf16* __restrict__ Vt_lo,
                                                     int32_t* __restrict__ cpos,
                                                     float* __restrict__ vnorm,
                                                     const int32_t* __restrict__ perm,
                                                     const int32_t* __restrict__ colseg) {
    constexpr int TPC = D / 8;            // threads per column
    constexpr int GC = gather_cols<D>();  // columns per workgroup (16 or 32)
    __shared__ __bf16 sV[X3 ? 2 : 1][GC][D + 8];
    const int h = blockIdx.y;
    const int p0 = blockIdx.x * GC;
    const int tid = threadIdx.x;
    const int col = tid / TPC;
    const int c0 = (tid % TPC) * 8;
    const int p = p0 + col;  // compact slot
    const int src = perm ? perm[(long)h * kp + p] : (p < k ? p : -1);  // selection index
    const bool live = src >= 0;
    const long j = live ? (sel ? (long)sel[(long)h * k + src] : (long)src) : 0;
    if (c0 == 0) cpos[(long)h * kp + p] = live ? (int32_t)j : 0x7fffffff;
    const int HD = c.H * D;
    const int ch = h * D + c0;
    float xkv[2][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        xkv[0][e] = 0.0f;
        xkv[1][e] = 0.0f;
    }
    if constexpr (NB > 0) {  // NB > kDeqBatch: chunks of kDeqBatch
        if (live) deq_col8_kv<NB <= kDeqBatch ? NB : kDeqBatch, (NB > kDeqBatch)>(c, upto, j, HD, ch, xkv[0], xkv[1]);
    }
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        float* x = xkv[which];
        if constexpr (NB == 0) {
            if (live) deq_col8(c, upto, which, j, HD, ch, x);
        }
        if (which == 0) {
            bf16x8 v, vl;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[i] = (__bf16)x[i];
                if (X3) vl[i] = (__bf16)(x[i] - (float)v[i]);
            }
            *reinterpret_cast<bf16x8*>(Kc + ((long)h * kp + p) * D + c0) = v;
            if (X3) *reinterpret_cast<bf16x8*>(Kc_lo + ((long)h * kp + p) * D + c0) = vl;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const __bf16 hi = (__bf16)x[e];
                sV[0][col][c0 + e] = hi;
                if (X3) sV[X3 ? 1 : 0][col][c0 + e] = (__bf16)(x[e] - (float)hi);
            }
            if (vnorm) { // ||vhat(j)||_2 in fp32 for the value-weighted column statistic
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = ss + x[e] * x[e];
#pragma unroll
                for (int o = 1; o < TPC; o <<= 1) ss = ss + __shfl_xor(ss, o);
                if (c0 == 0) vnorm[(long)h * kp + p] = sqrtf(ss);
            }
        }
    }
    __syncthreads();
    // transpose this workgroup's columns of the V tile: rows d, its GC keys
    // (whole 16-key groups, key order permuted inside each group), 16-byte stores
    const int tile = p0 / BN, kbase = p0 % BN;
    // with a slot order only the outlier part's tiles read the values' lo
    // parts (normal columns enter P.V as bf16 in every tile kind)
    const bool vlo = X3 && !(perm && colseg && p0 + GC <= (colseg[2 * h] + BN - 1) / BN * BN);
#pragma unroll
    for (int part = 0; part < (X3 ? 2 : 1); ++part) {
        if (part && !vlo) break;
        __bf16* vdst = (part ? Vt_lo : Vt) + ((long)h * (kp / BN) + tile) * D * BN + kbase;
        for (int idx = tid; idx < D * (GC / 8); idx += 256) {
            const int dd = idx / (GC / 8);
            const int oct = idx % (GC / 8);
            bf16x8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int so = oct * 8 + i;                      // stored position in the group(s)
                const int key = (so & ~15) + vt_key_of_slot(so & 15);
                v[i] = sV[part][key][dd];
            }
            *reinterpret_cast<bf16x8*>(vdst + (long)dd * BN + oct * 8) = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Compact gather of the quantised levels of the selected columns (for the
// in-tile dequantisation path): K code rows are copied as stored, V codes are
// transposed per 64-column tile into the key order of the MFMA operand, and
// scales follow their codes.  Absent levels are written as zeros.
template <int D>
__global__ __launch_bounds__(256) void k_gather_q(fl_kv_cache c, int upto,
                                                  const int32_t* __restrict__ sel, int k, int kp,
                                                  QTiles out, int32_t* __restrict__ cpos) {
    constexpr int G_MAX = D / 32;
    __shared__ int8_t sV[BN][D + 4];
    __shared__ float sVs[BN][G_MAX];
    const int h = blockIdx.y, tile = blockIdx.x, p0 = tile * BN;
    const int tid = threadIdx.x, col = tid >> 2;
    constexpr int CPT = D / 4;
    const int c0 = (tid & 3) * CPT;
    const int p = p0 + col;
    const bool live = p < k;
    const long j = live ? (sel ? (long)sel[(long)h * k + p] : (long)p) : 0;
    if ((tid & 3) == 0) cpos[(long)h * kp + p] = live ? (int32_t)j : 0x7fffffff;
    const int g = c.g, G = D / g, HD = c.H * D;
    const long prow = (long)h * kp + p;
    const int nt = kp / BN;
    for (int l = 0; l <= upto; ++l) {
        const fl_kv_level& L = c.level[l];
        const int b = L.bits;
        long row = -1;
        if (live) row = l == 0 ? j : (long)L.slot[j];
        const bool present = row >= 0;
        // K: copy this thread's CPT codes and (once per group) the scale
        {
            const uint32_t* src = reinterpret_cast<const uint32_t*>(
                reinterpret_cast<const uint8_t*>(L.k_codes) + ((row * HD + (long)h * D + c0) * b) / 8);
            uint32_t* dst = reinterpret_cast<uint32_t*>(out.kq[l] + ((prow * D + c0) * b) / 8);
            for (int wi = 0; wi < CPT * b / 32; ++wi) dst[wi] = present ? src[wi] : 0u;
            if (c0 % g == 0)
                out.ks[l][prow * G + c0 / g] = present ? L.k_scale[(row * HD + (long)h * D + c0) / g] : 0.0f;
        }
        // V: unpack this thread's codes into LDS
        {
            const long e0 = row * HD + (long)h * D + c0;
#pragma unroll
            for (int e8 = 0; e8 < CPT; e8 += 8) {
                const uint64_t w = present ? load_codes8(L.v_codes, e0 + e8, b) : 0ull;
#pragma unroll
                for (int i = 0; i < 8; ++i) sV[col][c0 + e8 + i] = (int8_t)code_at(w, b, i);
            }
            if (c0 % g == 0) sVs[col][c0 / g] = present ? L.v_scale[e0 / g] : 0.0f;
        }
        __syncthreads();
        // V codes: [d][64 keys in operand order], bits per code, 8 keys per step
        for (int idx = tid; idx < D * (BN / 8); idx += 256) {
            const int dd = idx / (BN / 8), oct = idx % (BN / 8);
            uint64_t w = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int so = oct * 8 + i;
                const int key = (so & ~15) + vt_key_of_slot(so & 15);
                w |= (uint64_t)((uint32_t)(int)sV[key][dd] & ((1u << b) - 1u)) << (b * i);
            }
            uint8_t* dst = out.vq[l] + ((((long)h * nt + tile) * D + dd) * BN + oct * 8) * b / 8;
            if (b == 8) *reinterpret_cast<uint64_t*>(dst) = w;
            else if (b == 4) *reinterpret_cast<uint32_t*>(dst) = (uint32_t)w;
            else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w;
        }
        for (int idx = tid; idx < G * BN; idx += 256) {
            const int gg = idx / BN, so = idx % BN;
            const int key = (so & ~15) + vt_key_of_slot(so & 15);
            out.vs[l][(((long)h * nt + tile) * G + gg) * BN + so] = sVs[key][gg];
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// PREC 0: bf16 operands (a cache without residual levels); 1: K, V and P as
// hi + lo bf16 pairs (residual levels carry information below bf16's
// resolution of the summed value); 2: q split as well (fp32 inputs).
// DEQ: the tiles are dequantised from compact quantised planes while staged.
// The running max is tracked on raw scores (the scale is folded into the
// exponent's fma) and the accumulators are rescaled only when some row's max
// passes the exponent reference by more than 8 (log2 units).  (A register-prefetch, two-buffer LDS variant of the tile loop
// measured slower on gfx950 -- 10.6 vs 8.6 ms for the 32K dense + sparse
// loop pair -- and is not used.)
template <int D, int MODE, int PREC, bool DEQ>
__global__ __launch_bounds__(256, 2) void k_attn(AttnParams P) {
    constexpr bool X3 = PREC >= 1;
    constexpr bool QS = PREC == 2;
    constexpr int NP = X3 ? 2 : 1;            // hi (+ lo) parts
    constexpr int CH = (BN * D / 8) / 256;    // 16-byte chunks per thread per tile
    __shared__ __bf16 Ks[1][NP][BN][D + 8];
    __shared__ __bf16 Vs[1][NP][D][BN + 8];
    __shared__ int cps[1][BN];
    __shared__ int s_bounds[2];
    const int n_tiles = (P.n + BM - 1) / BM;
    int tile, h;
    block_coords(P.xcd_remap, n_tiles, P.H, tile, h);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 31, half = lane >> 5;
    const int t0 = tile * BM;
    const int t = t0 + w * 32 + r;
    const bool valid = t < P.n;
    const int rowpos = valid ? P.active[t] : -1;
    const int32_t* cpos_h = P.cpos + (long)h * P.kp;
    if (w < 2) {  // wave 0: p_end (columns <= the last row's position), wave 1: p_full (first row's)
        const int b = wave_ubound(cpos_h, P.k, P.active[w == 0 ? min(t0 + BM, P.n) - 1 : t0]);
        if (lane == 0) s_bounds[w] = b;
    }
    // query fragment: B operand of S^T = K Q^T (lane: row r, d = 16kk + 8half)
    bf16x8 qf[D / 16], ql[QS ? D / 16 : 1];
    {
        const long qrow = P.q_gathered ? (long)t : (long)rowpos;
        const long qoff = (qrow * P.H + h) * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            if (QS) {
                float f[8];
                if (valid) load8_f32(P.q, qoff + 16 * kk, P.dtype, f);
                else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) f[i] = 0.0f;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    qf[kk][i] = (__bf16)f[i];
                    ql[QS ? kk : 0][i] = (__bf16)(f[i] - (float)qf[kk][i]);
                }
            } else if (valid) {
                qf[kk] = load8_bf16(P.q, qoff + 16 * kk, P.dtype);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) qf[kk][i] = (__bf16)0.0f;
            }
        }
    }
    const long rh = valid ? (long)rowpos * P.H + h : 0;
    float lse_prev2 = 0.0f, wgt = 1.0f;
    if (MODE == MODE_REBUILD && valid) {
        lse_prev2 = P.lse[rh] * 1.4426950408889634f;
        wgt = 1.0f - P.mass_u[rh];
    }
    __syncthreads();
    // wave-uniform loop bounds (scalar registers keep the tile loop uniform)
    const int p_end = __builtin_amdgcn_readfirstlane(s_bounds[0]);
    const int p_full = __builtin_amdgcn_readfirstlane(s_bounds[1]);

    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;

    const long koff = (long)h * P.kp * D;
    const long voff = (long)h * (P.kp / BN) * D * BN;

    for (int p0 = 0; p0 < p_end; p0 += BN) {
        constexpr int b = 0;
        {
            // ---- stage the K and V^T tiles in LDS ----
            if (DEQ) {
                // dequantise the tile's levels straight into the LDS operand tiles
                const int g = P.qt.g, G = D / g;
                {
                    const int col = tid >> 2, c0 = (tid & 3) * (D / 4);
                    const long prow = (long)h * P.kp + p0 + col;
                    float x[D / 4];
#pragma unroll
                    for (int e = 0; e < D / 4; ++e) x[e] = 0.0f;
                    for (int l = 0; l < P.deq_levels; ++l) {
                        const int bits = P.qt.bits[l];
                        const float sc = P.qt.ks[l][prow * G + c0 / g];
#pragma unroll
                        for (int e8 = 0; e8 < D / 4; e8 += 8) {
                            const uint64_t wd = load_codes8(P.qt.kq[l], prow * D + c0 + e8, bits);
#pragma unroll
                            for (int i = 0; i < 8; ++i) x[e8 + i] += (float)code_at(wd, bits, i) * sc;
                        }
                    }
#pragma unroll
                    for (int e8 = 0; e8 < D / 4; e8 += 8) {
                        bf16x8 v, vl;
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            v[i] = (__bf16)x[e8 + i];
                            if (X3) vl[i] = (__bf16)(x[e8 + i] - (float)v[i]);
                        }
                        *reinterpret_cast<bf16x8*>(&Ks[0][0][col][c0 + e8]) = v;
                        if (X3) *reinterpret_cast<bf16x8*>(&Ks[0][NP - 1][col][c0 + e8]) = vl;
                    }
                }
                const long tbase = (long)h * (P.kp / BN) + p0 / BN;
#pragma unroll
                for (int m = 0; m < (D * (BN / 8)) / 256; ++m) {
                    const int idx = tid + m * 256;
                    const int dd = idx / (BN / 8), oc = idx % (BN / 8);
                    float y[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) y[i] = 0.0f;
                    for (int l = 0; l < P.deq_levels; ++l) {
                        const int bits = P.qt.bits[l];
                        const uint64_t wd = load_codes8(P.qt.vq[l], (tbase * D + dd) * BN + oc * 8, bits);
                        const float4* sp = reinterpret_cast<const float4*>(
                            P.qt.vs[l] + (tbase * G + dd / g) * BN + oc * 8);
                        const float4 s0 = sp[0], s1 = sp[1];
                        const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
                        for (int i = 0; i < 8; ++i) y[i] += (float)code_at(wd, bits, i) * sc[i];
                    }
                    bf16x8 v, vl;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        v[i] = (__bf16)y[i];
                        if (X3) vl[i] = (__bf16)(y[i] - (float)v[i]);
                    }
                    *reinterpret_cast<bf16x8*>(&Vs[0][0][dd][oc * 8]) = v;
                    if (X3) *reinterpret_cast<bf16x8*>(&Vs[0][NP - 1][dd][oc * 8]) = vl;
                }
            } else {
#pragma unroll
                for (int part = 0; part < NP; ++part) {
                    const __bf16* Kh = (part ? P.Kc_lo : P.Kc) + koff;
                    const __bf16* Vh = (part ? P.Vt_lo : P.Vt) + voff;
#pragma unroll
                    for (int m = 0; m < CH; ++m) {
                        const int idx = tid + m * 256;
                        const int key = idx / (D / 8), c8 = idx % (D / 8);
                        *reinterpret_cast<uint4*>(&Ks[0][part][key][c8 * 8]) =
                            *reinterpret_cast<const uint4*>(Kh + (long)(p0 + key) * D + c8 * 8);
                        const int dd = idx / (BN / 8), oc = idx % (BN / 8);
                        *reinterpret_cast<uint4*>(&Vs[0][part][dd][oc * 8]) =
                            *reinterpret_cast<const uint4*>(Vh + ((long)(p0 / BN) * D + dd) * BN + oc * 8);
                    }
                }
            }
            if (tid < BN) cps[0][tid] = cpos_h[p0 + tid];
            __syncthreads();
        }

        // ---- S^T = K Q^T: two 32-key tiles ----
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            s[kt] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[b][0][32 * kt + r][16 * kk + 8 * half]);
                s[kt] = mfma32(a, qf[kk], s[kt]);
                if (X3) {
                    const bf16x8 al = *reinterpret_cast<const bf16x8*>(&Ks[b][NP - 1][32 * kt + r][16 * kk + 8 * half]);
                    s[kt] = mfma32(al, qf[kk], s[kt]);
                }
                if (QS) s[kt] = mfma32(a, ql[QS ? kk : 0], s[kt]);
            }
        }
        const bool need_mask = p0 + BN > p_full;
        if (need_mask) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = 32 * kt + (j >> 2) * 8 + half * 4 + (j & 3);
                    if (cps[b][key] > rowpos) s[kt][j] = -INFINITY;
                }
        }
        bf16x8 pb[2][2], pl[X3 ? 2 : 1][2];
        if (MODE == MODE_ATTN) {
            float tmax = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) tmax = fmaxf(tmax, s[kt][j]);
            tmax = max_xor32(tmax);
            const float m_new = fmaxf(m_run, tmax * P.c2);
            // The exponent reference m_run follows the running max lazily:
            // it moves (with a rescale of l and O) only when some row's max
            // exceeds it by more than 8, so probabilities stay <= 2^8 and
            // most tiles skip the rescale (the result does not depend on
            // the reference).
            if (__ballot(m_new > m_run + 8.0f)) {
                const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.0f : m_new));
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
                m_run = m_new;
            }
            const float m_use = m_run == -INFINITY ? 0.0f : m_run;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float pj = __builtin_amdgcn_exp2f(fmaf(s[kt][j], P.c2, -m_use));
                    pb[kt][j >> 3][j & 7] = (__bf16)pj;
                    l_run += pj; // fp32 row sum: lse feeds later loops' caches
                    if (X3) pl[X3 ? kt : 0][j >> 3][j & 7] = (__bf16)(pj - (float)pb[kt][j >> 3][j & 7]);
                }
        } else {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float pj = wgt * __builtin_amdgcn_exp2f(fmaf(s[kt][j], P.c2, -lse_prev2));
                    l_run += pj;
                    pb[kt][j >> 3][j & 7] = (__bf16)pj;
                    if (X3) pl[X3 ? kt : 0][j >> 3][j & 7] = (__bf16)(pj - (float)pb[kt][j >> 3][j & 7]);
                }
        }
        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int jh = 0; jh < 2; ++jh) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                        &Vs[b][0][32 * dt + r][32 * kt + 16 * jh + 8 * half]);
                    o[dt] = mfma32(a, pb[kt][jh], o[dt]);
                    if (X3) {
                        const bf16x8 al = *reinterpret_cast<const bf16x8*>(
                            &Vs[b][NP - 1][32 * dt + r][32 * kt + 16 * jh + 8 * half]);
                        o[dt] = mfma32(a, pl[X3 ? kt : 0][jh], o[dt]);
                        o[dt] = mfma32(al, pb[kt][jh], o[dt]);
                    }
                }
        __syncthreads();
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!valid) return;
    float* orow = P.out + rh * D;
    if (MODE == MODE_ATTN) {
        // every load of the caches before the first store (the stores could
        // alias them for the compiler, which would then serialise each pair)
        const bool cached = P.cache_op != FL_CACHE_ZERO;
        const float* ourow = P.out_u + rh * D;
        float4 uc[D / 32][4];
        float mu = 0.0f;
        if (cached) {
            mu = P.mass_u[rh];
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
                if (P.out_bf) store_bf16x4(P.out_bf + ((long)t * P.H + h) * D + d0, v);
            }
        if (half == 0)
            P.lse[rh] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    } else {
        float* ourow = P.out_u + rh * D;
        float4 bc[D / 32][4];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jq = 0; jq < 4; ++jq)
                bc[dt][jq] = *reinterpret_cast<const float4*>(orow + 32 * dt + jq * 8 + half * 4);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jq = 0; jq < 4; ++jq) {
                const int d0 = 32 * dt + jq * 8 + half * 4;
                const float4 op = bc[dt][jq];
                float4 v;
                v.x = op.x - o[dt][4 * jq + 0];
                v.y = op.y - o[dt][4 * jq + 1];
                v.z = op.z - o[dt][4 * jq + 2];
                v.w = op.w - o[dt][4 * jq + 3];
                *reinterpret_cast<float4*>(ourow + d0) = v;
            }
        if (half == 0) P.mass_u[rh] = 1.0f - l_tot;
    }
}

// ---------------------------------------------------------------------------
// Attention over compact bf16 tiles with an asynchronous two-buffer LDS
// pipeline: the next K / V^T tile is copied straight from global memory into
// the other LDS buffer (gfx950 LDS-DMA loads, 16 bytes per lane, no register
// staging) while the current tile is computed, so one barrier per tile and
// no exposed load latency.  (Running keys one tile ahead of values, to
// overlap the next tile's QK^T with this tile's softmax inside a wave, needs
// more than the 256 registers per lane of two waves per SIMD: it spilled.)
// A wave's LDS-DMA copy lands 64 consecutive
// 16-byte chunks, so the tiles are stored XOR-swizzled (chunk c of row x at
// c ^ swz(x)): the lanes' global addresses apply the swizzle, and the MFMA
// operand reads (sixteen rows at one logical chunk per LDS cycle) stay free
// of bank conflicts.  The two buffers are distinct LDS objects so the
// compiler's wait-count analysis sees that reads of one do not wait for
// copies into the other.  Arithmetic as k_attn (PREC 0/1, DEQ off).
constexpr int kAttnLdsSplit = 1;  // PREC value routed to the LDS-DMA kernel besides 0

// With DQ (the in-tile dequantisation placement) the tiles arrive as the
// compact quantised planes of every level (codes and fp32 scales, as written
// by k_gather_q): each tile's planes are copied by LDS-DMA into one staging
// buffer while the previous tile is computed, and the workgroup then
// dequantises them cooperatively (levels summed in order, rounded to bf16,
// plus the lo part with PREC 1) into a single operand tile in the layout
// the MFMA fragment reads expect; two barriers per tile.
constexpr int kDqCap = 40960;  // staging bytes of one tile's planes (all levels, K and V)

template <int D, int MODE, int PREC, int BT, bool DQ>
__device__ __forceinline__ void attn_lds_body(AttnParams P) {
    static_assert(PREC == 0 || PREC == 1, "bf16 queries only");
    constexpr bool X3 = PREC >= 1;
    constexpr int NP = X3 ? 2 : 1;
    static_assert(BT == 32 || BT == 64, "32- or 64-column tiles");
    constexpr int KT = BT / 32;             // 32-column MFMA blocks per tile
    constexpr int TB = BT * D * 2;          // bytes of one operand tile
    constexpr int MPW = TB / 1024 / 4;      // LDS-DMA instructions per wave per operand tile
    __shared__ __attribute__((aligned(1024))) __bf16 sK0[NP][BT * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sV0[NP][D * BT];
    // DQ: one operand tile; the second buffer is the planes' staging area
    __shared__ __attribute__((aligned(1024))) __bf16 sK1[DQ ? 1 : NP][DQ ? 8 : BT * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sV1[DQ ? 1 : NP][DQ ? 8 : D * BT];
    __shared__ __attribute__((aligned(1024))) char sQ[DQ ? kDqCap : 16];
    __shared__ __attribute__((aligned(256))) int sC0[64];
    __shared__ __attribute__((aligned(256))) int sC1[64];
    __shared__ int s_bounds[2];
    const int n_tiles = (P.n + BM - 1) / BM;
    int tile, h;
    block_coords(P.xcd_remap, n_tiles, P.H, tile, h);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, half = lane >> 5;
    const int t0 = tile * BM;
    const int t = t0 + w * 32 + r;
    const bool valid = t < P.n;
    const int rowpos = valid ? P.active[t] : -1;
    const int32_t* cpos_h = P.cpos + (long)h * P.kp;
    if (w < 2) {  // wave 0: p_end (columns <= the last row's position), wave 1: p_full (first row's)
        const int b = wave_ubound(cpos_h, P.k, P.active[w == 0 ? min(t0 + BM, P.n) - 1 : t0]);
        if (lane == 0) s_bounds[w] = b;
    }
    bf16x8 qf[D / 16];
    {
        const long qrow = P.q_gathered ? (long)t : (long)rowpos;
        const long qoff = (qrow * P.H + h) * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            if (valid) qf[kk] = load8_bf16(P.q, qoff + 16 * kk, P.dtype);
            else {
#pragma unroll
                for (int i = 0; i < 8; ++i) qf[kk][i] = (__bf16)0.0f;
            }
        }
    }
    const long rh = valid ? (long)rowpos * P.H + h : 0;
    float lse_prev2 = 0.0f, wgt = 1.0f;
    if (MODE == MODE_REBUILD && valid) {
        lse_prev2 = P.lse[rh] * 1.4426950408889634f;
        wgt = 1.0f - P.mass_u[rh];
    }
    __syncthreads();
    const int p_end = __builtin_amdgcn_readfirstlane(s_bounds[0]);
    const int p_full = __builtin_amdgcn_readfirstlane(s_bounds[1]);

    const long koff = (long)h * P.kp * D;
    const long voff = (long)h * (P.kp / BN) * D * BN;
    constexpr int KCPR = D * 2 / 16, VCPR = BT * 2 / 16;
    // copy the tile at column p0 into one LDS buffer (swizzled, see above);
    // a 32-column tile is one half of the stored 64-column V^T tile
    const uint32_t kbytes = (uint32_t)P.kp * D * 2, vbytes = kbytes;
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(P.Kc + koff, kbytes), rV = make_rsrc(P.Vt + voff, vbytes);
    const __amdgpu_buffer_rsrc_t rKl = make_rsrc(X3 ? P.Kc_lo + koff : P.Kc, kbytes);
    const __amdgpu_buffer_rsrc_t rVl = make_rsrc(X3 ? P.Vt_lo + voff : P.Vt, vbytes);
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(cpos_h, (uint32_t)P.kp * 4);
    // per-lane byte offsets of this wave's copies inside a tile
    uint32_t kvo[MPW], vvo[MPW];
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
        const int off = (w * MPW + i) * 1024 + lane * 16;
        const int kr = off / (D * 2), kc = ((off % (D * 2)) >> 4) ^ swz<KCPR>(kr);
        kvo[i] = kr * (D * 2) + kc * 16;
        const int vr = off / (BT * 2), vc = ((off % (BT * 2)) >> 4) ^ swz<VCPR>(vr);
        vvo[i] = vr * (BN * 2) + vc * 16;
    }
    auto issue = [&](int p0, __bf16 (*sK)[BT * D], __bf16 (*sV)[BT * D], int* sC) {
        const uint32_t ks = (uint32_t)p0 * D * 2;
        const uint32_t vs = ((uint32_t)(p0 / BN) * D * BN + p0 % BN) * 2;
#pragma unroll
        for (int part = 0; part < NP; ++part) {
#pragma unroll
            for (int i = 0; i < MPW; ++i) {
                const int m = w * MPW + i;
                buf_dma16(part ? rKl : rK, reinterpret_cast<char*>(sK[part]) + m * 1024, kvo[i], ks);
                buf_dma16(part ? rVl : rV, reinterpret_cast<char*>(sV[part]) + m * 1024, vvo[i], vs);
            }
        }
        if (w == 0 && lane < BT) buf_dma4(rC, sC, lane * 4, p0 * 4);
    };

    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;

    auto compute = [&](int p0, const __bf16 (*sK)[BT * D], const __bf16 (*sV)[BT * D], const int* sC) {
        f32x16 s[KT];
        // raised issue priority while this wave feeds its QK^T MFMAs: the
        // two waves sharing a SIMD then drift apart, one on the matrix
        // cores while the other runs its softmax (measured 4.15 -> 3.98 ms)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) s[kt] = f32x16{};
        // the key blocks' chains alternate (each chain keeps its own order)
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const int key = 32 * kt + r;
                const int e = key * D + (((2 * kk + half) ^ swz<KCPR>(key)) << 3);
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sK[0][e]);
                s[kt] = mfma32(a, qf[kk], s[kt]);
                if (X3) {
                    const bf16x8 al = *reinterpret_cast<const bf16x8*>(&sK[NP - 1][e]);
                    s[kt] = mfma32(al, qf[kk], s[kt]);
                }
            }
        if constexpr (KT == 2 && !X3) sched_reads_ahead16();
        __builtin_amdgcn_s_setprio(0);
        if (p0 + BT > p_full) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = 32 * kt + (j >> 2) * 8 + half * 4 + (j & 3);
                    if (sC[key] > rowpos) s[kt][j] = -INFINITY;
                }
        }
        bf16x8 pb[KT][2], pl[X3 ? KT : 1][2];
        float m_use = lse_prev2;
        if (MODE == MODE_ATTN) {
            float tmax = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int j = 0; j < 16; ++j) tmax = fmaxf(tmax, s[kt][j]);
            tmax = max_xor32(tmax);
            const float m_new = fmaxf(m_run, tmax * P.c2);
            // lazy exponent reference, as in k_attn
            if (__ballot(m_new > m_run + 8.0f)) {
                const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.0f : m_new));
                l_run *= alpha;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
                m_run = m_new;
            }
            m_use = m_run == -INFINITY ? 0.0f : m_run;
        }
        // probabilities of 32-column block kt, and O^T += V^T P^T over it
        auto expb = [&](int kt) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float pj = __builtin_amdgcn_exp2f(fmaf(s[kt][j], P.c2, -m_use));
                if (MODE == MODE_REBUILD) pj *= wgt;
                pb[kt][j >> 3][j & 7] = (__bf16)pj;
                l_run += pj;
                if (X3) pl[X3 ? kt : 0][j >> 3][j & 7] = (__bf16)(pj - (float)pb[kt][j >> 3][j & 7]);
            }
        };
        auto pvb = [&](int kt) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const int row = 32 * dt + r;
#pragma unroll
                for (int jh = 0; jh < 2; ++jh) {
                    const int e = row * BT + (((4 * kt + 2 * jh + half) ^ swz<VCPR>(row)) << 3);
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sV[0][e]);
                    o[dt] = mfma32(a, pb[kt][jh], o[dt]);
                    if (X3) {
                        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&sV[NP - 1][e]);
                        o[dt] = mfma32(a, pl[X3 ? kt : 0][jh], o[dt]);
                        o[dt] = mfma32(al, pb[kt][jh], o[dt]);
                    }
                }
            }
        };
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) expb(kt);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) pvb(kt);
    };

    if constexpr (DQ) {
        // the staging buffer holds, level by level: K codes [BT][D] (b bits
        // each), K scales [BT][G], V codes [D][BT] (key order of the V^T
        // operand), V scales [G][BT]
        const int nl = P.deq_levels, g = P.qt.g, G = D / g;
        const int nt = P.kp / BN;
        // copy `rows` rows of `rb` bytes (rb a power of two, a multiple of 4)
        // found `stride` bytes apart into consecutive staging bytes; 16-byte
        // copies where rows allow, else 4-byte ones; the waves take turns
        auto stage_rows = [&](__amdgpu_buffer_rsrc_t rs, uint32_t soff, int rows, int rb, uint32_t stride,
                              uint32_t dst) {
            const int gs = rb % 16 == 0 ? 16 : 4;
            const int lrg = __builtin_ctz(rb / gs);
            const int total = rows << lrg;
            for (int base = w * 64; base < total; base += 256) {
                const int i = base + lane;
                if (i < total) {
                    const uint32_t src = (uint32_t)(i >> lrg) * stride + (uint32_t)(i & ((1 << lrg) - 1)) * gs;
                    if (gs == 16) buf_dma16(rs, sQ + dst + base * 16, src, soff);
                    else buf_dma4(rs, sQ + dst + base * 4, src, soff);
                }
            }
        };
        auto issue_q = [&](int p0, int* sC) {
            uint32_t off = 0;
            for (int l = 0; l < nl; ++l) {
                const int b = P.qt.bits[l];
                const int cb = BT * D * b / 8, sb = BT * G * 4;
                const long hk = (long)h * P.kp;
                const __amdgpu_buffer_rsrc_t rkq = make_rsrc(P.qt.kq[l] + hk * D * b / 8, (uint32_t)P.kp * D * b / 8);
                const __amdgpu_buffer_rsrc_t rks = make_rsrc(P.qt.ks[l] + hk * G, (uint32_t)P.kp * G * 4);
                const __amdgpu_buffer_rsrc_t rvq =
                    make_rsrc(P.qt.vq[l] + (long)h * nt * D * BN * b / 8, (uint32_t)P.kp * D * b / 8);
                const __amdgpu_buffer_rsrc_t rvs = make_rsrc(P.qt.vs[l] + (long)h * nt * G * BN, (uint32_t)P.kp * G * 4);
                stage_rows(rkq, (uint32_t)p0 * D * b / 8, 1, cb, 0, off);
                off += cb;
                stage_rows(rks, (uint32_t)p0 * G * 4, 1, sb, 0, off);
                off += sb;
                stage_rows(rvq, ((uint32_t)(p0 / BN) * D * BN + p0 % BN) * b / 8, D, BT * b / 8, BN * b / 8, off);
                off += cb;
                stage_rows(rvs, ((uint32_t)(p0 / BN) * G * BN + p0 % BN) * 4, G, BT * 4, BN * 4, off);
                off += sb;
            }
            if (w == 0 && lane < BT) buf_dma4(rC, sC, lane * 4, p0 * 4);
        };
        // the staged levels summed in order into the operand tile (bf16 hi,
        // and the bf16 rounding of the remainder as lo with PREC 1)
        auto dequant = [&]() {
#pragma unroll
            for (int it = tid; it < BT * (D / 8); it += 256) {
                const int key = it / (D / 8), c8 = it % (D / 8);
                float x[8] = {};
                uint32_t off = 0;
                for (int l = 0; l < nl; ++l) {
                    const int b = P.qt.bits[l];
                    const int cb = BT * D * b / 8;
                    const float sc = *reinterpret_cast<const float*>(sQ + off + cb + (key * G + c8 * 8 / g) * 4);
                    const int e = key * D + c8 * 8;
                    const uint64_t wd = b == 8 ? *reinterpret_cast<const uint64_t*>(sQ + off + e)
                                      : b == 4 ? *reinterpret_cast<const uint32_t*>(sQ + off + e / 2)
                                               : *reinterpret_cast<const uint16_t*>(sQ + off + e / 4);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float t = (float)code_at(wd, b, i) * sc;
                        x[i] = l == 0 ? t : x[i] + t;
                    }
                    off += 2 * (cb + BT * G * 4);
                }
                bf16x8 hi, lo;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    hi[i] = (__bf16)x[i];
                    if (X3) lo[i] = (__bf16)(x[i] - (float)hi[i]);
                }
                const int ep = key * D + ((c8 ^ swz<KCPR>(key)) << 3);
                *reinterpret_cast<bf16x8*>(&sK0[0][ep]) = hi;
                if (X3) *reinterpret_cast<bf16x8*>(&sK0[NP - 1][ep]) = lo;
            }
#pragma unroll
            for (int it = tid; it < D * (BT / 8); it += 256) {
                const int dd = it / (BT / 8), oc = it % (BT / 8);
                float y[8] = {};
                uint32_t off = 0;
                for (int l = 0; l < nl; ++l) {
                    const int b = P.qt.bits[l];
                    const int cb = BT * D * b / 8, sb = BT * G * 4;
                    const int e = dd * BT + oc * 8;
                    const char* vc = sQ + off + cb + sb;
                    const uint64_t wd = b == 8 ? *reinterpret_cast<const uint64_t*>(vc + e)
                                      : b == 4 ? *reinterpret_cast<const uint32_t*>(vc + e / 2)
                                               : *reinterpret_cast<const uint16_t*>(vc + e / 4);
                    const float4* sp =
                        reinterpret_cast<const float4*>(sQ + off + 2 * cb + sb + ((dd / g) * BT + oc * 8) * 4);
                    const float4 s0 = sp[0], s1 = sp[1];
                    const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float t = (float)code_at(wd, b, i) * sc[i];
                        y[i] = l == 0 ? t : y[i] + t;
                    }
                    off += 2 * (cb + sb);
                }
                bf16x8 hi, lo;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    hi[i] = (__bf16)y[i];
                    if (X3) lo[i] = (__bf16)(y[i] - (float)hi[i]);
                }
                const int ep = dd * BT + ((oc ^ swz<VCPR>(dd)) << 3);
                *reinterpret_cast<bf16x8*>(&sV0[0][ep]) = hi;
                if (X3) *reinterpret_cast<bf16x8*>(&sV0[NP - 1][ep]) = lo;
            }
        };
        if (p_end > 0) issue_q(0, sC0);
        for (int p0 = 0; p0 < p_end; p0 += BT) {
            const bool odd = (p0 / BT) & 1;
            __builtin_amdgcn_s_waitcnt(0); // this lane's copies of the tile's planes landed
            __syncthreads();               // ... every lane's; the operand tile is free
            dequant();
            __syncthreads();               // operand tile complete; the staging buffer is free
            if (p0 + BT < p_end) issue_q(p0 + BT, odd ? sC0 : sC1);
            compute(p0, sK0, sV0, odd ? sC1 : sC0);
        }
    } else {
    if (p_end > 0) issue(0, sK0, sV0, sC0);
    for (int p0 = 0; p0 < p_end;) {
        __builtin_amdgcn_s_waitcnt(0); // this lane's copies of the current tile landed
        __syncthreads();               // ... every lane's; the other buffer is free
        if (p0 + BT < p_end) issue(p0 + BT, sK1, sV1, sC1);
        compute(p0, sK0, sV0, sC0);
        p0 += BT;
        if (p0 >= p_end) break;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (p0 + BT < p_end) issue(p0 + BT, sK0, sV0, sC0);
        compute(p0, sK1, sV1, sC1);
        p0 += BT;
    }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!valid) return;
    float* orow = P.out + rh * D;
    if (MODE == MODE_ATTN) {
        // every load of the caches before the first store (the stores could
        // alias them for the compiler, which would then serialise each pair)
        const bool cached = P.cache_op != FL_CACHE_ZERO;
        const float* ourow = P.out_u + rh * D;
        float4 uc[D / 32][4];
        float mu = 0.0f;
        if (cached) {
            mu = P.mass_u[rh];
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
                if (P.out_bf) store_bf16x4(P.out_bf + ((long)t * P.H + h) * D + d0, v);
            }
        if (half == 0)
            P.lse[rh] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    } else {
        float* ourow = P.out_u + rh * D;
        float4 bc[D / 32][4];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jq = 0; jq < 4; ++jq)
                bc[dt][jq] = *reinterpret_cast<const float4*>(orow + 32 * dt + jq * 8 + half * 4);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int jq = 0; jq < 4; ++jq) {
                const int d0 = 32 * dt + jq * 8 + half * 4;
                const float4 op = bc[dt][jq];
                float4 v;
                v.x = op.x - o[dt][4 * jq + 0];
                v.y = op.y - o[dt][4 * jq + 1];
                v.z = op.z - o[dt][4 * jq + 2];
                v.w = op.w - o[dt][4 * jq + 3];
                *reinterpret_cast<float4*>(ourow + d0) = v;
            }
        if (half == 0) P.mass_u[rh] = 1.0f - l_tot;
    }
}

template <int D, int MODE, int PREC, int BT>
__global__ __launch_bounds__(256, PREC == 0 ? (BT == 32 ? 3 : 2) : (BT == 32 ? 2 : 1)) void k_attn_lds(AttnParams P) {
    attn_lds_body<D, MODE, PREC, BT, false>(P);
}

// in-tile dequantisation over the same pipeline (see attn_lds_body)
template <int D, int MODE, int PREC, int BT>
__global__ __launch_bounds__(256, 2) void k_attn_lds_dq(AttnParams P) {
    attn_lds_body<D, MODE, PREC, BT, true>(P);
}

// ---------------------------------------------------------------------------

__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int n, int v) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < v) lo = mid + 1; else hi = mid;
    }
    return lo;
}

constexpr int CT = 128; // columns per workgroup (4 waves x 32)
constexpr int RT = 32;  // query rows per step

// Column block and head of this workgroup (one-dimensional grid of n_blk * H
// blocks).  The first columns of a head are seen by the most query rows, so
// blocks are started heaviest first with the heads interleaved; when H is a
// multiple of 8 each head's blocks stay on one XCD (workgroups are dealt to
// the 8 XCDs round-robin), so its query rows stream through one L2.
__device__ __forceinline__ void col_coords(int H, int& blk, int& h) {
    const int b = blockIdx.x;
    if ((H & 7) == 0) {
        const int x = b & 7, m = b >> 3, hp = H >> 3;
        h = x + 8 * (m % hp);
        blk = m / hp;
    } else {
        h = b % H;
        blk = b / H;
    }
}

template <int D, int PREC>
__global__ __launch_bounds__(256, 2) void k_colstat(ColParams P) {
    constexpr bool X3 = PREC >= 1;  // keys as hi + lo
    constexpr bool QS = PREC == 2;  // queries as hi + lo
    constexpr int NP = QS ? 2 : 1;
    __shared__ __bf16 Qs[NP][RT][D + 8];
    __shared__ int rpos[RT];
    __shared__ float rlse[RT], rw[RT];
    __shared__ int s_start;
    int blk, h;
    col_coords(P.H, blk, h);
    const int pc0 = blk * CT;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 31, half = lane >> 5;
    const int p = pc0 + w * 32 + r; // this lane's column (slot in the selection)
    const int32_t* cpos_h = P.cpos + (long)h * P.kp;
    const bool colv = p < P.k;
    const int cp = colv ? cpos_h[p] : 0x7fffffff;
    bf16x8 kf[D / 16], kl[X3 ? D / 16 : 1];
    {
        const long ko = ((long)h * P.kp + (colv ? p : 0)) * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            kf[kk] = *reinterpret_cast<const bf16x8*>(P.Kc + ko + 16 * kk);
            if (X3) kl[X3 ? kk : 0] = *reinterpret_cast<const bf16x8*>(P.Kc_lo + ko + 16 * kk);
        }
    }
    if (tid == 0) s_start = lower_bound_i32(P.active, P.n, cpos_h[pc0]);
    __syncthreads();
    const int t_start = __builtin_amdgcn_readfirstlane(s_start);
    float csum = 0.0f;
    for (int t0 = t_start; t0 < P.n; t0 += RT) {
        // stage 32 query rows (bf16) and their lse / weight
        for (int idx = tid; idx < RT * (D / 8); idx += 256) {
            const int rr = idx / (D / 8), c8 = idx % (D / 8);
            const int t = t0 + rr;
            float f[8];
            if (t < P.n) {
                const long qrow = P.q_gathered ? (long)t : (long)P.active[t];
                load8_f32(P.q, (qrow * P.H + h) * D + c8 * 8, P.dtype, f);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) f[i] = 0.0f;
            }
            bf16x8 v, vl;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[i] = (__bf16)f[i];
                if (QS) vl[i] = (__bf16)(f[i] - (float)v[i]);
            }
            *reinterpret_cast<bf16x8*>(&Qs[0][rr][c8 * 8]) = v;
            if (QS) *reinterpret_cast<bf16x8*>(&Qs[NP - 1][rr][c8 * 8]) = vl;
        }
        if (tid < RT) {
            const int t = t0 + tid;
            if (t < P.n) {
                const int pos = P.active[t];
                const long rh = (long)pos * P.H + h;
                rpos[tid] = pos;
                rlse[tid] = P.lse[rh] * 1.4426950408889634f;
                rw[tid] = P.cache_op == FL_CACHE_ZERO ? 1.0f : 1.0f - P.mass_u[rh];
            } else {
                rpos[tid] = -1; rlse[tid] = 0.0f; rw[tid] = 0.0f;
            }
        }
        __syncthreads();
        f32x16 s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Qs[0][r][16 * kk + 8 * half]);
            s = mfma32(a, kf[kk], s);
            if (X3) s = mfma32(a, kl[X3 ? kk : 0], s);
            if (QS) {
                const bf16x8 al = *reinterpret_cast<const bf16x8*>(&Qs[NP - 1][r][16 * kk + 8 * half]);
                s = mfma32(al, kf[kk], s);
            }
        }
        // s[j]: column r of this wave, row (j/4)*8 + half*4 + j%4
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int row = (j >> 2) * 8 + half * 4 + (j & 3);
            const float v = s[j] * P.c2 - rlse[row];
            const float pj = rw[row] * __builtin_amdgcn_exp2f(v);
            csum += (rpos[row] >= cp) ? pj : 0.0f;
        }
        __syncthreads();
    }
    csum += __shfl_xor(csum, 32);
    if (colv && half == 0)
        P.col_stat[(long)h * P.k + p] = P.vnorm ? csum * P.vnorm[(long)h * P.kp + p] : csum;
}

// Column statistics for bf16 queries (PREC 0/1): the query rows are swept
// in 64-row steps from the last row down to the block's diagonal, each wave
// covering its 32 columns for both 32-row halves of a step (steps from the
// bottom keep the column blocks of a head on the same query rows in L2).  The
// weight 1 - M_U is folded into a per-row exponent offset (off = lse*log2(e)
// - log2(1 - M_U)), so a pair costs one fma, one exp2 and one add; the causal
// mask is only applied on diagonal steps.
constexpr int RT2 = 64;

// Column statistics with the Q steps copied by LDS-DMA into two distinct LDS
// buffers (swizzled as in k_attn_lds): one barrier per 64-row step, the next
// step's rows land while the current one is computed.  The per-row exponent
// offsets and positions are prefetched through registers by one wave.
// NW waves per workgroup, 32 columns each: every query tile copied into LDS
// feeds 32 * NW columns, so the queries are streamed from memory
// k / (32 * NW) times per head.
// KB key blocks of 32 columns per wave: with KB = 2 every query fragment read
// from LDS feeds two MFMAs (half the LDS operand traffic per MFMA, which
// otherwise bounds the MFMA side of the sweep), at three workgroups per CU.
template <int KB>
constexpr int colstat_min_blocks() { return KB == 2 ? 3 : 1; }

template <int D, int PREC, int NW, int KB>
__global__ __launch_bounds__(64 * NW, colstat_min_blocks<KB>()) void k_colstat_lds(ColParams P) {
    constexpr bool X3 = PREC >= 1;
    static_assert(KB == 1 || (KB == 2 && !X3), "two key blocks per wave with plain bf16 keys");
    constexpr int CTW = 32 * NW * KB;        // columns per workgroup
    constexpr int QB = RT2 * D * 2;         // bytes of one step's query rows
    constexpr int MPW = QB / 1024 / NW;     // LDS-DMA instructions per wave per step
    static_assert(MPW >= 1 && QB % (1024 * NW) == 0, "step copy split over the waves");
    __shared__ __attribute__((aligned(1024))) __bf16 sQ0[RT2 * D];
    __shared__ __attribute__((aligned(1024))) __bf16 sQ1[RT2 * D];
    __shared__ int rp0[RT2], rp1[RT2];
    __shared__ float ro0[RT2], ro1[RT2];
    __shared__ int s_start, s_cmax;
    int blk, h;
    col_coords(P.H, blk, h);
    const int pc0 = blk * CTW;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, half = lane >> 5;
    const int32_t* cpos_h = P.cpos + (long)h * P.kp;
    // this lane's columns (compact slots) and their selection indices (a
    // slot order from k_classify_cols puts pads between and after its two
    // ascending parts)
    int p[KB], src[KB], cp[KB];
    bool colv[KB];
    bf16x8 kf[KB][D / 16], kl[X3 ? D / 16 : 1];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        p[kb] = pc0 + (w * KB + kb) * 32 + r;
        src[kb] = P.perm ? (p[kb] < P.kp ? P.perm[(long)h * P.kp + p[kb]] : -1) : (p[kb] < P.k ? p[kb] : -1);
        colv[kb] = src[kb] >= 0;
        cp[kb] = colv[kb] ? cpos_h[p[kb]] : 0x7fffffff;
        const long ko = ((long)h * P.kp + (colv[kb] ? p[kb] : 0)) * D + 8 * half;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            kf[kb][kk] = *reinterpret_cast<const bf16x8*>(P.Kc + ko + 16 * kk);
            if (X3) kl[X3 ? kk : 0] = *reinterpret_cast<const bf16x8*>(P.Kc_lo + ko + 16 * kk);
        }
    }
    // the block's first and last column positions
    if (tid == 0) { s_start = 0x7fffffff; s_cmax = -1; }
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
        if (colv[kb]) { atomicMin(&s_start, cp[kb]); atomicMax(&s_cmax, cp[kb]); }
    __syncthreads();
    if (tid == 0) s_start = lower_bound_i32(P.active, P.n, s_start);
    __syncthreads();
    const int t_start = __builtin_amdgcn_readfirstlane(s_start);
    const int cmax = __builtin_amdgcn_readfirstlane(s_cmax);
    const int nsteps = t_start < P.n ? (P.n - t_start + RT2 - 1) / RT2 : 0;
    const int t_last = t_start + (nsteps - 1) * RT2;
    // this thread's LDS-DMA rows inside a step and their logical chunk
    int drow[MPW], dchunk[MPW];
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
        const int off = (w * MPW + i) * 1024 + lane * 16;
        drow[i] = off / (D * 2);
        dchunk[i] = ((off % (D * 2)) >> 4) ^ swz<D * 2 / 16>(drow[i]);
    }
    // Query rows of a step are addressed through their positions, which are
    // loaded one step ahead of the copy (two ahead of the compute), so no
    // copy waits on a dependent load.  Rows past n repeat row n-1; their
    // offset is +inf and position -1, so they add nothing.
    // (kept as int until used: widening a just-loaded value would wait for it)
    int qr_next[MPW];
    auto load_rows = [&](int t0) {
#pragma unroll
        for (int i = 0; i < MPW; ++i) {
            const int tt = min(t0 + drow[i], P.n - 1);
            qr_next[i] = P.q_gathered ? tt : P.active[tt];
        }
    };
    // query rows of head h: row x at byte x * H * D * 2 from the head's base
    const uint32_t qstride = (uint32_t)P.H * D * 2;
    const __amdgpu_buffer_rsrc_t rQ =
        make_rsrc(reinterpret_cast<const uint16_t*>(P.q) + (long)h * D,
                  (uint32_t)(P.q_gathered ? P.n : P.active[P.n - 1] + 1) * qstride);
    auto issue = [&](__bf16* sQ) {
#pragma unroll
        for (int i = 0; i < MPW; ++i)
            buf_dma16(rQ, reinterpret_cast<char*>(sQ) + (w * MPW + i) * 1024,
                      (uint32_t)qr_next[i] * qstride + dchunk[i] * 16, 0);
    };
    // wave 0: lane l's row position (loaded a step ahead) and its exponent
    // offset lse*log2(e) - log2(1 - M_U)
    int mpos_next = -1, mpos = -1;
    float mlse = 0.0f, mmu = 0.0f;
    auto meta_pos = [&](int t0) {
        const int tt = t0 + lane;
        mpos_next = tt < P.n ? P.active[tt] : -1;
    };
    auto meta_vals = [&]() {
        mpos = mpos_next;
        if (mpos >= 0) {
            const long rh = (long)mpos * P.H + h;
            mlse = P.lse[rh];
            mmu = P.cache_op == FL_CACHE_ZERO ? 0.0f : P.mass_u[rh];
        }
    };
    auto meta_store = [&](int* rp, float* ro) {
        const float wgt = fmaxf(1.0f - mmu, 0.0f);
        rp[lane] = mpos;
        ro[lane] = mpos >= 0 ? mlse * 1.4426950408889634f - __log2f(wgt) : INFINITY;
    };
    float csum[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) csum[kb] = 0.0f;
    auto compute = [&](int t0, const __bf16* sQ, const int* rpos, const float* roff) {
        const bool full = rpos[0] >= cmax && t0 + RT2 <= P.n;
        // (computing both halves' S^T before their exponentials, with or
        // without raised issue priority, measured slower: 3.08 / 3.12 vs
        // 3.01 ms at 32K)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            f32x16 s[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
            const int row = 32 * sub + r;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                const int e = row * D + (((2 * kk + half) ^ swz<D * 2 / 16>(row)) << 3);
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sQ[e]);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) s[kb] = mfma32(a, kf[kb][kk], s[kb]);
                if (X3) s[0] = mfma32(a, kl[X3 ? kk : 0], s[0]);
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                if (full) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int rw = 32 * sub + (j >> 2) * 8 + half * 4 + (j & 3);
                        csum[kb] += __builtin_amdgcn_exp2f(fmaf(s[kb][j], P.c2, -roff[rw]));
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int rw = 32 * sub + (j >> 2) * 8 + half * 4 + (j & 3);
                        const float pj = __builtin_amdgcn_exp2f(fmaf(s[kb][j], P.c2, -roff[rw]));
                        csum[kb] += (rpos[rw] >= cp[kb]) ? pj : 0.0f;
                    }
                }
            }
        }
    };
    // prologue: step 0 copied and its metadata stored; positions of step 1
    if (nsteps > 0) {
        load_rows(t_last);
        issue(sQ0);
        if (w == 0) {
            meta_pos(t_last);
            meta_vals();
            meta_store(rp0, ro0);
        }
        if (nsteps > 1) {
            load_rows(t_last - RT2);
            if (w == 0) meta_pos(t_last - RT2);
        }
    }
    // steps from the last one down to the block's diagonal;
    // iteration it computes step it, copies step it+1, loads positions of it+2
    for (int it = 0; it < nsteps;) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int t0 = t_last - it * RT2;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            const bool more = it + 1 < nsteps;
            if (more) {
                issue(b ? sQ0 : sQ1);
                if (w == 0) meta_vals();
                if (it + 2 < nsteps) {
                    load_rows(t0 - 2 * RT2);
                    if (w == 0) meta_pos(t0 - 2 * RT2);
                }
            }
            compute(t0, b ? sQ1 : sQ0, b ? rp1 : rp0, b ? ro1 : ro0);
            if (more && w == 0) meta_store(b ? rp0 : rp1, b ? ro0 : ro1);
            if (++it >= nsteps) break;
        }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const float cs = csum[kb] + __shfl_xor(csum[kb], 32);
        if (colv[kb] && half == 0)
            P.col_stat[(long)h * P.k + src[kb]] = P.vnorm ? cs * P.vnorm[(long)h * P.kp + p[kb]] : cs;
    }
}

// ---------------------------------------------------------------------------
// launchers
hipError_t launch_gather_bf16(const fl_kv_cache& c, int upto, const int32_t* sel, int k, int kp,
                              bool x3, __bf16* Kc, __bf16* Vt, __bf16* Kc_lo, __bf16* Vt_lo,
                              int32_t* cpos, float* vnorm, const int32_t* perm, const int32_t* colseg,
                              hipStream_t st) {
    dim3 grid(kp / (c.d == 128 ? gather_cols<128>() : gather_cols<64>()), c.H);
    // the keys' and values' level rows loaded together where the cache allows
    // (kDeqBatch + 1: levels in several chunks)
    const int nb = !deq_batch_ok(c, upto) ? 0 : upto < kDeqBatch ? upto + 1 : kDeqBatch + 1;
#define FL_GATHER(D_, X_, B_)                                                                       \
    hipLaunchKernelGGL((k_gather_bf16<D_, X_, B_>), grid, dim3(256), 0, st, c, upto, sel, k, kp, Kc, \
                       Vt, Kc_lo, Vt_lo, cpos, vnorm, perm, colseg)
#define FL_GATHER_B(D_, X_) {                                                   \
        switch (nb) {                                                           \
        case 1: FL_GATHER(D_, X_, 1); break;                                    \
        case 2: FL_GATHER(D_, X_, 2); break;                                    \
        case 3: FL_GATHER(D_, X_, 3); break;                                    \
        case 4: FL_GATHER(D_, X_, 4); break;                                    \
        case 5: FL_GATHER(D_, X_, 5); break;                                    \
        default: FL_GATHER(D_, X_, 0);                                          \
        } }
    if (c.d == 128) { if (x3) FL_GATHER_B(128, true) else FL_GATHER_B(128, false) }
    else { if (x3) FL_GATHER_B(64, true) else FL_GATHER_B(64, false) }
#undef FL_GATHER_B
#undef FL_GATHER
    return hipGetLastError();
}

hipError_t launch_gather_q(const fl_kv_cache& c, int upto, const int32_t* sel, int k, int kp,
                           const QTiles& out, int32_t* cpos, hipStream_t st) {
    dim3 grid(kp / BN, c.H);
    if (c.d == 128)
        hipLaunchKernelGGL(k_gather_q<128>, grid, dim3(256), 0, st, c, upto, sel, k, kp, out, cpos);
    else
        hipLaunchKernelGGL(k_gather_q<64>, grid, dim3(256), 0, st, c, upto, sel, k, kp, out, cpos);
    return hipGetLastError();
}

// the LDS-DMA pipelined kernels for bf16 queries: 64-column tiles for plain
// bf16 operands; with hi/lo operand pairs (PREC 1) 32-column tiles, so the
// doubled tiles still leave two workgroups per CU (64-column hi/lo tiles
// allow one and measured slower than the register-staged kernel: 1.11 vs
// 0.87 ms for the 32K sparse loops)
static bool lds_path(int prec) { return prec == 0 || prec == kAttnLdsSplit; }

// in-tile placement: the LDS-DMA kernel takes bf16 queries (PREC 0 / 1) when
// one tile's planes of every level fit its staging buffer; deeper caches and
// fp32 queries use the register-staged kernel
static bool dq_lds_fits(int d, int prec, const AttnParams& P) {
    if (prec > 1) return false;
    const int bt = prec == 0 ? 64 : 32, G = d / P.qt.g;
    long bytes = 0;
    for (int l = 0; l < P.deq_levels; ++l) bytes += 2L * ((long)bt * d * P.qt.bits[l] / 8 + (long)bt * G * 4);
    return bytes <= kDqCap;
}

hipError_t launch_attn(int d, int mode, int prec, bool in_tile, const AttnParams& P, hipStream_t st) {
    const int n_tiles = (P.n + BM - 1) / BM;
    AttnParams Q = P;
    Q.xcd_remap = (P.H % 8) == 0;
    dim3 grid(n_tiles * P.H);
#define FL_ATTN(D_, M_, P_, Q_) hipLaunchKernelGGL((k_attn<D_, M_, P_, Q_>), grid, dim3(256), 0, st, Q)
#define FL_ATTN_LDS(D_, M_, P_) hipLaunchKernelGGL((k_attn_lds<D_, M_, P_, P_ == 0 ? 64 : 32>), grid, dim3(256), 0, st, Q)
    // bf16 queries over compact bf16 tiles: the LDS-DMA pipelined kernel
#define FL_ATTN_DQ(D_, M_, P_) hipLaunchKernelGGL((k_attn_lds_dq<D_, M_, P_, P_ == 0 ? 64 : 32>), grid, dim3(256), 0, st, Q)
#define FL_ATTN_Q(D_, M_, P_)                                   \
    if (in_tile && P_ <= 1 && dq_lds_fits(D_, P_, Q)) FL_ATTN_DQ(D_, M_, (P_ <= 1 ? P_ : 0)); \
    else if (in_tile) FL_ATTN(D_, M_, P_, true);               \
    else if (P_ <= 1 && lds_path(P_)) FL_ATTN_LDS(D_, M_, (P_ <= 1 ? P_ : 0)); \
    else FL_ATTN(D_, M_, P_, false);
#define FL_ATTN_M(D_, M_) \
    if (prec == 0) { FL_ATTN_Q(D_, M_, 0) } else if (prec == 1) { FL_ATTN_Q(D_, M_, 1) } else { FL_ATTN_Q(D_, M_, 2) }
#define FL_ATTN_D(D_) \
    if (mode == MODE_ATTN) { FL_ATTN_M(D_, MODE_ATTN) } else { FL_ATTN_M(D_, MODE_REBUILD) }
    if (d == 128) { FL_ATTN_D(128) } else { FL_ATTN_D(64) }
#undef FL_ATTN_D
#undef FL_ATTN_M
#undef FL_ATTN_Q
#undef FL_ATTN_LDS
#undef FL_ATTN_DQ
#undef FL_ATTN
    return hipGetLastError();
}

// waves per workgroup of the LDS-DMA column statistics: 8 (256 columns) with
// plain bf16 keys; hi/lo keys take more registers, so 4 keep 3 waves per SIMD
template <int PREC>
constexpr int colstat_waves() { return PREC == 0 ? 4 : 4; }
// key blocks per wave (two with plain bf16 keys, see k_colstat_lds)
template <int PREC>
constexpr int colstat_kb() { return PREC == 0 ? 2 : 1; }

hipError_t launch_colstat(int d, int prec, const ColParams& P, hipStream_t st) {
    // one-dimensional grids of column blocks x heads (see col_coords); with a
    // slot order every compact slot is covered
    const int ncol = P.perm ? P.kp : P.k;
    const dim3 grid(((ncol + CT - 1) / CT) * P.H);
#define FL_COL(D_, P_) hipLaunchKernelGGL((k_colstat<D_, P_>), grid, dim3(256), 0, st, P)
#define FL_COLL(D_, P_)                                                                        \
    hipLaunchKernelGGL((k_colstat_lds<D_, P_, colstat_waves<P_>(), colstat_kb<P_>()>),        \
                       dim3(((ncol + 32 * colstat_waves<P_>() * colstat_kb<P_>() - 1) /              \
                             (32 * colstat_waves<P_>() * colstat_kb<P_>())) * P.H),                  \
                       dim3(64 * colstat_waves<P_>()), 0, st, P)
#define FL_COL_D(D_) \
    if (prec == 0) FL_COLL(D_, 0); else if (prec == 1) FL_COLL(D_, 1); else FL_COL(D_, 2);
    if (d == 128) { FL_COL_D(128) } else { FL_COL_D(64) }
#undef FL_COL_D
#undef FL_COLL
#undef FL_COL
    return hipGetLastError();
}

} // namespace fl

// Batched decode of the lazy-update loop attention (FlashLoop paper,
// Sec. 4.2 sparse attention over the selected key columns with the cached
// probability mass; Sec. 5.3.1: decode is bound by KV traffic, which the
// column sparsity and the low-bit residuals cut).
//
// One workgroup per (sequence, head) and one new query token.  The key
// columns are the selected prefix columns (all of them in the dense first
// loop) plus T always-included bf16 columns: the token's own fresh key/value
// ("self" column) and, during generation, the window of recent tokens.
// A column's row of d codes is read by d/16 neighbouring lanes, 16 codes
// each, so every wave load covers whole 2^k-byte code rows (coalesced), and
// several column groups are in flight per wave.
//   rows     (sparse) every level's cache row of every selected column is
//            looked up once, all levels in parallel, into LDS;
//   phase 1  scores: per lane a 16-channel dot product with the dequantised
//            chain (codes x group scale, levels summed; a level absent from
//            the nested sets has row -1 and is predicated off), reduced
//            across the column's lanes;
//   phase 2  block max / sum -> lse, probabilities kept in LDS;
//   phase 3  P.V: per lane 16 channels accumulated over its columns with
//            p x scale folded into one factor per (column, level, group),
//            reduced across lanes and waves.
// MODE_ATTN writes o = sum P V + O_U (P carries 1 - M_U), lse and the column
// probabilities (the next loop's column statistic).  MODE_REBUILD recomputes
// the previous loop's probabilities on the kept columns and its self column
// and stores M_U = 1 - sum P, O_U = o_prev - sum P V.
#include "fl_device.h"
#include "fl_kernels.h"

namespace fl {

constexpr int DT = 256;      // threads per workgroup (512 measured slower)
constexpr size_t kDecodePairLds = 48 * 1024;  // dynamic LDS bound for the pair lists
constexpr int DNW = DT / 64; // waves

struct SeqLevel {
    const uint8_t* codes;
    const float* scales;
    const float* zeros;     // asymmetric scheme: the offsets beside the scales
    const int32_t* slot;
    int bits;
};

// level l of sequence b: the B sequences are stored back to back with the
// per-sequence capacities (positions pos_cap; rows rows_cap[l] for l >= 1).
// Absmax and value scales: one per (row, head, g channels); asymmetric key
// scales and offsets: one per (key group of g rows, head, channel), a
// sequence holding kg_count[l] groups of them.
template <int D, bool ASYM>
__device__ __forceinline__ SeqLevel seq_level(const DecodeParams& P, int l, int b, int which) {
    const fl_kv_cache& c = P.cache;
    const fl_kv_level& L = c.level[l];
    const long rows = l == 0 ? P.pos_cap : P.rows_cap[l];
    SeqLevel s;
    s.bits = L.bits;
    s.codes = reinterpret_cast<const uint8_t*>(which ? L.v_codes : L.k_codes) +
              b * (rows * c.H * D * L.bits / 8);
    const long sstride = (ASYM && which == 0) ? (long)P.kg_count[l] * c.H * D : rows * c.H * (D / c.g);
    s.scales = (which ? L.v_scale : L.k_scale) + b * sstride;
    s.zeros = ASYM ? (which ? L.v_zero : L.k_zero) + b * sstride : nullptr;
    s.slot = l == 0 ? nullptr : L.slot + (long)b * P.pos_cap;
    return s;
}

// Asymmetric key group of row x of level l: groups of g rows from row 0 up
// to the level's origin (the prompt's rows, the last group possibly
// partial), then groups of g rows from the origin (appended during
// generation).
__device__ __forceinline__ int key_group(const DecodeParams& P, int l, int x) {
    return (x >= P.kg_origin[l] ? x + P.kg_pad[l] : x) / P.cache.g;
}

// 16 consecutive unsigned codes (asymmetric scheme) starting at code index e
// (16-aligned)
__device__ __forceinline__ void load_ucodes16(const uint8_t* base, long e, int bits, float (&x)[16]) {
    if (bits == 8) {
        const uint4 u = *reinterpret_cast<const uint4*>(base + e);
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (float)((wd[i >> 2] >> (8 * (i & 3))) & 255u);
    } else if (bits == 4) {
        const uint2 u = *reinterpret_cast<const uint2*>(base + e / 2);
        const uint64_t wd = ((uint64_t)u.y << 32) | u.x;
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (float)((uint32_t)(wd >> (4 * i)) & 15u);
    } else { // bits == 2
        const uint32_t wd = *reinterpret_cast<const uint32_t*>(base + e / 4);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (float)((wd >> (2 * i)) & 3u);
    }
}

// The same 16 unsigned codes in two steps, for a width known at compile
// time: the raw words (so the loads of several columns can be issued before
// any is used), then the codes as floats.
template <int BITS>
__device__ __forceinline__ uint4 load_raw16(const uint8_t* base, long e) {
    if (BITS == 8) return *reinterpret_cast<const uint4*>(base + e);
    if (BITS == 4) {
        const uint2 u = *reinterpret_cast<const uint2*>(base + e / 2);
        return make_uint4(u.x, u.y, 0u, 0u);
    }
    return make_uint4(*reinterpret_cast<const uint32_t*>(base + e / 4), 0u, 0u, 0u);
}
template <int BITS>
__device__ __forceinline__ void decode_u16(const uint4 r, float (&x)[16]) {
    const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
    constexpr int PER = 32 / BITS;  // codes per word
#pragma unroll
    for (int i = 0; i < 16; ++i)
        x[i] = (float)((wd[i / PER] >> (BITS * (i % PER))) & ((1u << BITS) - 1u));
}

// 16 signed codes (absmax scheme) in two steps for a width known only at
// run time (uniform across a level): the raw words, then the codes as
// floats, so the loads of several columns are in flight before any is used.
__device__ __forceinline__ uint4 load_raw16_rt(const uint8_t* base, long e, int bits) {
    if (bits == 8) return *reinterpret_cast<const uint4*>(base + e);
    if (bits == 4) {
        const uint2 u = *reinterpret_cast<const uint2*>(base + e / 2);
        return make_uint4(u.x, u.y, 0u, 0u);
    }
    return make_uint4(*reinterpret_cast<const uint32_t*>(base + e / 4), 0u, 0u, 0u);
}
// load_raw16_rt through a global-address-space pointer: the pair passes
// take the level bases from LDS, where the compiler cannot tell them from
// flat addresses (a flat load also holds up every LDS wait of the wave)
#define FL_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ uint4 load_raw16_g(const uint8_t* base, long e, int bits) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const FL_GLOBAL uint8_t* g = (const FL_GLOBAL uint8_t*)base;
    if (bits == 8) {
        const u32x4 v = *(const FL_GLOBAL u32x4*)(g + e);
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    if (bits == 4) {
        const u32x2 v = *(const FL_GLOBAL u32x2*)(g + e / 2);
        return make_uint4(v.x, v.y, 0u, 0u);
    }
    return make_uint4(*(const FL_GLOBAL uint32_t*)(g + e / 4), 0u, 0u, 0u);
}
__device__ __forceinline__ float load_f32_global(const float* base, long i) {
    return ((const FL_GLOBAL float*)base)[i];
}
__device__ __forceinline__ void decode_s16_rt(const uint4 r, int bits, float (&x)[16]) {
    if (bits == 8) {
        const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (float)(int8_t)(wd[i >> 2] >> (8 * (i & 3)));
    } else if (bits == 4) {
        const uint64_t wd = ((uint64_t)r.y << 32) | r.x;
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (float)((int)((int64_t)(wd << (60 - 4 * i)) >> 60));
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (float)((int)((int32_t)(r.x << (30 - 2 * i)) >> 30));
    }
}

// 16 consecutive fp32 values
__device__ __forceinline__ void load_f32x16(const float* p, float (&x)[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 v = reinterpret_cast<const float4*>(p)[i];
        x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
    }
}

// 16 consecutive bf16 values as fp32
__device__ __forceinline__ void load_bf16x16(const void* base, long e, float (&x)[16]) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + e);
    const uint4 a = p[0], b = p[1];
    const uint32_t wd[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        x[2 * i] = __uint_as_float(wd[i] << 16);
        x[2 * i + 1] = __uint_as_float(wd[i] & 0xffff0000u);
    }
}

// 16 consecutive codes starting at code index e (16-aligned)
__device__ __forceinline__ void load_codes16(const uint8_t* base, long e, int bits, float (&x)[16]) {
    if (bits == 8) {
        const uint4 u = *reinterpret_cast<const uint4*>(base + e);
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (float)(int8_t)(wd[i >> 2] >> (8 * (i & 3)));
    } else if (bits == 4) {
        const uint2 u = *reinterpret_cast<const uint2*>(base + e / 2);
        const uint64_t wd = ((uint64_t)u.y << 32) | u.x;
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (float)((int)((int64_t)(wd << (60 - 4 * i)) >> 60));
    } else { // bits == 2
        const uint32_t wd = *reinterpret_cast<const uint32_t*>(base + e / 4);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (float)((int)((int32_t)(wd << (30 - 2 * i)) >> 30));
    }
}

// ASYM: the cache holds the asymmetric scheme (unsigned codes, code * s + z;
// keys with a scale and offset per channel for every g rows of a level,
// values per g channels of a row); L0 then only restricts the walk to level 0.
// B0: the base level's code width when fixed at compile time (0 = read it
// from the cache).  A width known here lets the compiler issue the U column
// loads of a pass together instead of one load-wait pair per column.
template <int D, int MODE, bool SPARSE, bool L0, bool ASYM, int B0>
__global__ __launch_bounds__(DT) void k_decode(DecodeParams P) {
    constexpr int LPC = D / 16;     // lanes per column
    constexpr int CPW = 64 / LPC;   // columns per wave per load
    constexpr int CPI = CPW * DNW;  // columns per workgroup pass
    // passes in flight: 4 for 16-byte code rows (8 measured no faster); a
    // narrower fixed base keeps the bytes in flight per lane the same
    constexpr int U = (ASYM && L0 && B0 == 4) ? 8 : (ASYM && L0 && B0 == 2) ? 16 : 4;
    // the selected columns' level-by-level passes (absmax): 8 columns per
    // lane, so that k = 256 takes one pass per level
    constexpr int US = 8;
    extern __shared__ float dyn[];  // sc[k + T], then (sparse) rows[level + 1][k]
    __shared__ float qs[D];
    __shared__ float red[DNW];
    __shared__ float ored[DNW][D];
    // (sparse absmax) per level and side: code and scale bases, code width
    __shared__ const uint8_t* lv_codes[2][FL_MAX_LEVELS];
    __shared__ const float* lv_scales[2][FL_MAX_LEVELS];
    __shared__ int lv_bits[FL_MAX_LEVELS];
    __shared__ int s_cnt[DNW];
    // blocks are dealt to the 8 XCDs round-robin; with B a multiple of 8 all
    // heads of a sequence run on one XCD, so a token's scale line (all heads'
    // group scales are adjacent) is fetched into one L2 only
    int b, h;
    if (P.B % 8 == 0) {
        const int x = blockIdx.x & 7, m = blockIdx.x >> 3;
        b = 8 * (m / P.H) + x;
        h = m % P.H;
    } else {
        b = blockIdx.x / P.H;
        h = blockIdx.x % P.H;
    }
    const int bh = b * P.H + h;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int cl = lane / LPC, cs = lane % LPC;
    const fl_kv_cache& C = P.cache;
    const int H = C.H, G = D / C.g;
    const int k = P.k;
    const int T = P.n_tail;
    const int kt = k + T;
    const int nlev = L0 ? 1 : P.level + 1;
    const long qo = (long)bh * D;
    float* sc = dyn;
    int* rowtab = reinterpret_cast<int*>(dyn + kt);
    // tail column t of this (sequence, head): element offset of its row
    auto tail_off = [&](int t) -> long {
        int sl = P.tail_start + t;
        if (sl >= P.tail_cap) sl -= P.tail_cap;
        return (((long)b * P.tail_cap + sl) * H + h) * D;
    };
    for (int c = tid; c < D; c += DT)
        qs[c] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(P.q)[qo + c]);
    // (sparse absmax, levels beyond the base) the selected columns' present
    // cache rows as (column, level) pairs, level-major with the columns in
    // selection order inside a level (a wave's loads then share one code
    // width, and a pass walks one level's rows in order; column-major pairs
    // measured 1.5x slower); ppart[l * k + c] receives pair (c, l)'s partial
    // score
    constexpr bool PAIRS_OK = SPARSE && !ASYM;
    const bool use_pairs = PAIRS_OK && P.pairs;
    int* pairs = rowtab + (P.level + 1) * k;
    float* ppart = reinterpret_cast<float*>(pairs + (P.level + 1) * k);
    if (use_pairs && tid < nlev) {
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const SeqLevel L = seq_level<D, ASYM>(P, tid, b, which);
            lv_codes[which][tid] = L.codes;
            lv_scales[which][tid] = L.scales;
        }
        lv_bits[tid] = L0 ? 8 : P.cache.level[tid].bits;
    }
    if (SPARSE) {
        const int32_t* sel = P.sel + (long)bh * k;
        for (int c = tid; c < k; c += DT) {
            const int j = sel[c];
            rowtab[c] = j;
            for (int l = 1; l < nlev; ++l) rowtab[l * k + c] = seq_level<D, ASYM>(P, l, b, 0).slot[j];
        }
    }
    __syncthreads();
    int npairs = 0;
    if (use_pairs) {
        for (int l = 0; l < nlev; ++l)
            for (int c0 = 0; c0 < k; c0 += DT) {
                const int c = c0 + tid;
                const bool f = c < k && rowtab[l * k + c] >= 0;
                const unsigned long long bal = __ballot(f);
                if (lane == 0) s_cnt[w] = __popcll(bal);
                __syncthreads();
                int base = npairs, tot = 0;
#pragma unroll
                for (int i = 0; i < DNW; ++i) {
                    if (i < w) base += s_cnt[i];
                    tot += s_cnt[i];
                }
                if (f) pairs[base + __popcll(bal & ((1ull << lane) - 1))] = (l << 26) | c;
                npairs += tot;
                __syncthreads();
            }
    }
    float qv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) qv[i] = qs[cs * 16 + i];
    const float c2 = P.sm * 1.4426950408889634f;
    const int grp = cs * 16 / C.g;  // this lane's scale group
    // code width of level l
    auto bits_of = [&](const SeqLevel& L, int l) -> int {
        if (!ASYM && L0) return 8;
        if (B0 && l == 0) return B0;
        return L.bits;
    };

    auto row_of = [&](int l, int c) -> int {
        if (SPARSE) return rowtab[l * k + c];
        if (l == 0) return c;
        return seq_level<D, ASYM>(P, l, b, 0).slot[c];
    };

    // ---- phase 1: scores (log2 units) ----
    if (ASYM && L0 && !SPARSE) {
        // the level-0 rows in order: a wave takes CPW * U consecutive columns
        // per pass, so a key group's per-channel scales and offsets (shared by
        // g rows) are loaded once per group for this lane's 16 channels and
        // folded into the query: q . (code * s + z) = (q s) . code + q . z
        // (the columns of one step share a group except across the origin of
        // the appended groups, where each lane follows its own column)
        const SeqLevel L = seq_level<D, ASYM>(P, 0, b, 0);
        constexpr int BB = B0 ? B0 : 8;  // launched with the base width fixed
        int gcur = -1;
        float qs[16], qz = 0.0f;
        for (int c0 = 0; c0 < k; c0 += CPI * U) {
            // the pass's code loads first (a column past k re-reads the last)
            uint4 raw[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + w * (CPW * U) + u * CPW + cl;
                raw[u] = load_raw16<BB>(L.codes, ((long)(c < k ? c : k - 1) * H + h) * D + cs * 16);
            }
            float part[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + w * (CPW * U) + u * CPW + cl;
                part[u] = 0.0f;
                const int cg = key_group(P, 0, c);
                if (c < k && cg != gcur) {
                    const long si = ((long)cg * H + h) * D + cs * 16;
                    float sv[16], zv[16];
                    load_f32x16(L.scales + si, sv);
                    load_f32x16(L.zeros + si, zv);
                    qz = 0.0f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        qs[i] = qv[i] * sv[i];
                        qz = fmaf(qv[i], zv[i], qz);
                    }
                    gcur = cg;
                }
                if (c < k) {
                    float x[16];
                    decode_u16<BB>(raw[u], x);
                    float dot = qz;
#pragma unroll
                    for (int i = 0; i < 16; ++i) dot = fmaf(qs[i], x[i], dot);
                    part[u] = dot;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float v = part[u];
#pragma unroll
                for (int o = 1; o < LPC; o <<= 1) v += __shfl_xor(v, o);
                const int c = c0 + w * (CPW * U) + u * CPW + cl;
                if (cs == 0 && c < k) sc[c] = v * c2;
            }
        }
    } else if (PAIRS_OK && use_pairs) {
        // selected columns' present rows as (column, level) pairs: each pass
        // issues its US pairs' code and scale loads before using any; a pair's
        // partial score goes to LDS, and a column sums its levels in level
        // order afterwards
        for (int p0 = 0; p0 < npairs; p0 += CPI * US) {
            uint4 raw[US];
            float sv[US];
            int pk[US];
#pragma unroll
            for (int u = 0; u < US; ++u) {
                const int pi = p0 + u * CPI + w * CPW + cl;
                pk[u] = pi < npairs ? pairs[pi] : -1;
                raw[u] = make_uint4(0u, 0u, 0u, 0u);
                sv[u] = 0.0f;
                if (pk[u] >= 0) {
                    const int l = pk[u] >> 26, c = pk[u] & 0x3ffffff;
                    const long rr = (long)rowtab[l * k + c] * H + h;
                    raw[u] = load_raw16_g(lv_codes[0][l], rr * D + cs * 16, lv_bits[l]);
                    sv[u] = load_f32_global(lv_scales[0][l], rr * G + grp);
                }
            }
#pragma unroll
            for (int u = 0; u < US; ++u) {
                float v = 0.0f;
                if (pk[u] >= 0) {
                    float x[16];
                    decode_s16_rt(raw[u], lv_bits[pk[u] >> 26], x);
                    float dot = 0.0f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) dot = fmaf(qv[i], x[i], dot);
                    v = dot * sv[u];
                }
#pragma unroll
                for (int o = 1; o < LPC; o <<= 1) v += __shfl_xor(v, o);
                if (cs == 0 && pk[u] >= 0) ppart[(pk[u] >> 26) * k + (pk[u] & 0x3ffffff)] = v;
            }
        }
        __syncthreads();
        for (int c = tid; c < k; c += DT) {
            float v = 0.0f;
            for (int l = 0; l < nlev; ++l)
                if (rowtab[l * k + c] >= 0) v += ppart[l * k + c];
            sc[c] = v * c2;
        }
    } else if (!ASYM && SPARSE) {
        // selected columns: level by level, each pass issues its US columns'
        // code and scale loads before using any (an absent level's row is
        // -1 and its column is skipped); a column still sums its levels in
        // level order
        for (int c0 = 0; c0 < k; c0 += CPI * US) {
            float part[US];
#pragma unroll
            for (int u = 0; u < US; ++u) part[u] = 0.0f;
            for (int l = 0; l < nlev; ++l) {
                const SeqLevel L = seq_level<D, ASYM>(P, l, b, 0);
                const int bits = bits_of(L, l);
                uint4 raw[US];
                float sv[US];
                int rowv[US];
#pragma unroll
                for (int u = 0; u < US; ++u) {
                    const int c = c0 + u * CPI + w * CPW + cl;
                    rowv[u] = c < k ? row_of(l, c) : -1;
                    raw[u] = make_uint4(0u, 0u, 0u, 0u);
                    sv[u] = 0.0f;
                    if (rowv[u] >= 0) {
                        const long rr = (long)rowv[u] * H + h;
                        raw[u] = load_raw16_rt(L.codes, rr * D + cs * 16, bits);
                        sv[u] = L.scales[rr * G + grp];
                    }
                }
#pragma unroll
                for (int u = 0; u < US; ++u) {
                    if (rowv[u] >= 0) {
                        float x[16];
                        decode_s16_rt(raw[u], bits, x);
                        float dot = 0.0f;
#pragma unroll
                        for (int i = 0; i < 16; ++i) dot = fmaf(qv[i], x[i], dot);
                        part[u] = fmaf(dot, sv[u], part[u]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < US; ++u) {
                float v = part[u];
#pragma unroll
                for (int o = 1; o < LPC; o <<= 1) v += __shfl_xor(v, o);
                const int c = c0 + u * CPI + w * CPW + cl;
                if (cs == 0 && c < k) sc[c] = v * c2;
            }
        }
    } else
    for (int c0 = 0; c0 < k; c0 += CPI * U) {
        float part[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            part[u] = 0.0f;
            const int c = c0 + u * CPI + w * CPW + cl;
            if (c < k) {
                // absent levels are predicated off (not a break), so the
                // loads of a column's levels are issued together
#pragma unroll 4
                for (int l = 0; l < nlev; ++l) {
                    const int row = row_of(l, c);
                    if (row >= 0) {
                        const SeqLevel L = seq_level<D, ASYM>(P, l, b, 0);
                        const long rr = (long)row * H + h;
                        float x[16];
                        if (ASYM) {
                            // x = code * s + z per channel (scale / offset of the row's group)
                            load_ucodes16(L.codes, rr * D + cs * 16, bits_of(L, l), x);
                            const long si = ((long)key_group(P, l, row) * H + h) * D + cs * 16;
                            float sv[16], zv[16];
                            load_f32x16(L.scales + si, sv);
                            load_f32x16(L.zeros + si, zv);
                            float dot = 0.0f;
#pragma unroll
                            for (int i = 0; i < 16; ++i) dot = fmaf(qv[i], x[i] * sv[i] + zv[i], dot);
                            part[u] += dot;
                        } else {
                            load_codes16(L.codes, rr * D + cs * 16, bits_of(L, l), x);
                            float dot = 0.0f;
#pragma unroll
                            for (int i = 0; i < 16; ++i) dot = fmaf(qv[i], x[i], dot);
                            part[u] = fmaf(dot, L.scales[rr * G + grp], part[u]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float v = part[u];
#pragma unroll
            for (int o = 1; o < LPC; o <<= 1) v += __shfl_xor(v, o);
            const int c = c0 + u * CPI + w * CPW + cl;
            if (cs == 0 && c < k) sc[c] = v * c2;
        }
    }
    // the T always-included bf16 columns (self, window), laid out like the cache
    for (int t0 = 0; t0 < T; t0 += CPI) {
        const int t = t0 + w * CPW + cl;
        float v = 0.0f;
        if (t < T) {
            float x[16];
            load_bf16x16(P.tail_k, tail_off(t) + cs * 16, x);
#pragma unroll
            for (int i = 0; i < 16; ++i) v = fmaf(qv[i], x[i], v);
        }
#pragma unroll
        for (int o = 1; o < LPC; o <<= 1) v += __shfl_xor(v, o);
        if (cs == 0 && t < T) sc[k + t] = v * c2;
    }
    __syncthreads();

    // ---- phase 2: softmax statistics ----
    float wgt, lse2;
    if (MODE == MODE_ATTN) {
        float m = -INFINITY;
        for (int c = tid; c < kt; c += DT) m = fmaxf(m, sc[c]);
        m = wave_max(m);
        if (lane == 0) red[w] = m;
        __syncthreads();
        m = red[0];
#pragma unroll
        for (int i = 1; i < DNW; ++i) m = fmaxf(m, red[i]);
        __syncthreads();
        float z = 0.0f;
        for (int c = tid; c < kt; c += DT) z += __builtin_amdgcn_exp2f(sc[c] - m);
        z = wave_sum(z);
        if (lane == 0) red[w] = z;
        __syncthreads();
        z = 0.0f;
#pragma unroll
        for (int i = 0; i < DNW; ++i) z += red[i];
        lse2 = m + __log2f(z);
        wgt = P.cache_op == FL_CACHE_ZERO ? 1.0f : 1.0f - P.mass_u[bh];
    } else {
        lse2 = P.lse[bh] * 1.4426950408889634f;
        wgt = 1.0f - P.mass_u[bh];
    }
    float psum = 0.0f;
    for (int c = tid; c < kt; c += DT) {
        const float p = wgt * __builtin_amdgcn_exp2f(sc[c] - lse2);
        sc[c] = p;
        psum += p;
    }
    __syncthreads();

    // ---- phase 3: P.V ----
    float acc[16];
    float accz = 0.0f;  // asymmetric offsets: sum of p z, common to the 16 channels
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    if (ASYM && L0 && !SPARSE) {
        // level 0 in column order: each pass issues its U columns' code,
        // scale and offset loads before using any of them
        const SeqLevel L = seq_level<D, ASYM>(P, 0, b, 1);
        constexpr int BB = B0 ? B0 : 8;
        for (int c0 = 0; c0 < k; c0 += CPI * U) {
            uint4 raw[U];
            float sv[U], zv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * CPI + w * CPW + cl;
                const long rr = (long)(c < k ? c : k - 1) * H + h;
                raw[u] = load_raw16<BB>(L.codes, rr * D + cs * 16);
                sv[u] = L.scales[rr * G + grp];
                zv[u] = L.zeros[rr * G + grp];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * CPI + w * CPW + cl;
                if (c < k) {
                    // p * (code * s + z) = code * (p s) + p z
                    const float p = sc[c];
                    const float ps = p * sv[u];
                    accz = fmaf(p, zv[u], accz);
                    float x[16];
                    decode_u16<BB>(raw[u], x);
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[i] = fmaf(x[i], ps, acc[i]);
                }
            }
        }
    } else if (PAIRS_OK && use_pairs) {
        // as in phase 1: (column, level) pairs, a pass's loads issued together
        for (int p0 = 0; p0 < npairs; p0 += CPI * US) {
            uint4 raw[US];
            float sv[US], pu[US];
            int pk[US];
#pragma unroll
            for (int u = 0; u < US; ++u) {
                const int pi = p0 + u * CPI + w * CPW + cl;
                pk[u] = pi < npairs ? pairs[pi] : -1;
                raw[u] = make_uint4(0u, 0u, 0u, 0u);
                sv[u] = 0.0f;
                pu[u] = 0.0f;
                if (pk[u] >= 0) {
                    const int l = pk[u] >> 26, c = pk[u] & 0x3ffffff;
                    const long rr = (long)rowtab[l * k + c] * H + h;
                    raw[u] = load_raw16_g(lv_codes[1][l], rr * D + cs * 16, lv_bits[l]);
                    sv[u] = load_f32_global(lv_scales[1][l], rr * G + grp);
                    pu[u] = sc[c];
                }
            }
#pragma unroll
            for (int u = 0; u < US; ++u) {
                if (pk[u] >= 0) {
                    const float ps = pu[u] * sv[u];
                    float x[16];
                    decode_s16_rt(raw[u], lv_bits[pk[u] >> 26], x);
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[i] = fmaf(x[i], ps, acc[i]);
                }
            }
        }
    } else if (!ASYM && SPARSE) {
        // as in phase 1: level by level, a pass's loads issued together
        for (int c0 = 0; c0 < k; c0 += CPI * US) {
            float pu[US];
#pragma unroll
            for (int u = 0; u < US; ++u) {
                const int c = c0 + u * CPI + w * CPW + cl;
                pu[u] = c < k ? sc[c] : 0.0f;
            }
            for (int l = 0; l < nlev; ++l) {
                const SeqLevel L = seq_level<D, ASYM>(P, l, b, 1);
                const int bits = bits_of(L, l);
                uint4 raw[US];
                float sv[US];
                int rowv[US];
#pragma unroll
                for (int u = 0; u < US; ++u) {
                    const int c = c0 + u * CPI + w * CPW + cl;
                    rowv[u] = c < k ? row_of(l, c) : -1;
                    raw[u] = make_uint4(0u, 0u, 0u, 0u);
                    sv[u] = 0.0f;
                    if (rowv[u] >= 0) {
                        const long rr = (long)rowv[u] * H + h;
                        raw[u] = load_raw16_rt(L.codes, rr * D + cs * 16, bits);
                        sv[u] = L.scales[rr * G + grp];
                    }
                }
#pragma unroll
                for (int u = 0; u < US; ++u) {
                    if (rowv[u] >= 0) {
                        const float ps = pu[u] * sv[u];
                        float x[16];
                        decode_s16_rt(raw[u], bits, x);
#pragma unroll
                        for (int i = 0; i < 16; ++i) acc[i] = fmaf(x[i], ps, acc[i]);
                    }
                }
            }
        }
    } else
    for (int c0 = 0; c0 < k; c0 += CPI * U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * CPI + w * CPW + cl;
            if (c < k) {
                const float p = sc[c];
#pragma unroll 4
                for (int l = 0; l < nlev; ++l) {
                    const int row = row_of(l, c);
                    if (row >= 0) {
                        const SeqLevel L = seq_level<D, ASYM>(P, l, b, 1);
                        const long rr = (long)row * H + h;
                        float x[16];
                        if (ASYM) {
                            // p * (code * s + z) = code * (p s) + p z
                            load_ucodes16(L.codes, rr * D + cs * 16, bits_of(L, l), x);
                            const float ps = p * L.scales[rr * G + grp];
                            accz = fmaf(p, L.zeros[rr * G + grp], accz);
#pragma unroll
                            for (int i = 0; i < 16; ++i) acc[i] = fmaf(x[i], ps, acc[i]);
                        } else {
                            load_codes16(L.codes, rr * D + cs * 16, bits_of(L, l), x);
                            const float ps = p * L.scales[rr * G + grp];
#pragma unroll
                            for (int i = 0; i < 16; ++i) acc[i] = fmaf(x[i], ps, acc[i]);
                        }
                    }
                }
            }
        }
    }
    for (int t0 = 0; t0 < T; t0 += CPI) {
        const int t = t0 + w * CPW + cl;
        if (t < T) {
            const float p = sc[k + t];
            float x[16];
            load_bf16x16(P.tail_v, tail_off(t) + cs * 16, x);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = fmaf(x[i], p, acc[i]);
        }
    }
    if (ASYM) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += accz;
    }
    // lanes with the same channel slice hold partial sums over different columns
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int o = LPC; o < 64; o <<= 1) acc[i] += __shfl_xor(acc[i], o);
    }
    if (cl == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) ored[w][cs * 16 + i] = acc[i];
    }
    psum = wave_sum(psum);
    if (lane == 0) red[w] = psum;
    __syncthreads();
    float ptot = 0.0f;
#pragma unroll
    for (int i = 0; i < DNW; ++i) ptot += red[i];
    for (int c = tid; c < D; c += DT) {
        float o = 0.0f;
#pragma unroll
        for (int i = 0; i < DNW; ++i) o += ored[i][c];
        if (MODE == MODE_ATTN) {
            const float u = P.cache_op == FL_CACHE_ZERO ? 0.0f : P.out_u[qo + c];
            P.out[qo + c] = o + u;
        } else {
            P.out_u[qo + c] = P.out[qo + c] - o;
        }
    }
    if (tid == 0) {
        if (MODE == MODE_ATTN) P.lse[bh] = lse2 * 0.6931471805599453f;
        else P.mass_u[bh] = 1.0f - ptot;
    }
    if (MODE == MODE_ATTN && P.col_stat)
        for (int c = tid; c < k; c += DT) P.col_stat[(long)bh * k + c] = sc[c];
}

// One (D, MODE, SPARSE, L0) kernel: absmax, or the asymmetric scheme with
// the base level's width fixed when only the base level is read.
template <int D, int M, bool S, bool L>
void launch_decode_one(bool asym, int b0, dim3 grid, size_t shm, const DecodeParams& P, hipStream_t st) {
    if (!asym) {
        hipLaunchKernelGGL((k_decode<D, M, S, L, false, 0>), grid, dim3(DT), shm, st, P);
    } else if constexpr (!L) {
        hipLaunchKernelGGL((k_decode<D, M, S, L, true, 0>), grid, dim3(DT), shm, st, P);
    } else {
        if (b0 == 8) hipLaunchKernelGGL((k_decode<D, M, S, L, true, 8>), grid, dim3(DT), shm, st, P);
        else if (b0 == 4) hipLaunchKernelGGL((k_decode<D, M, S, L, true, 4>), grid, dim3(DT), shm, st, P);
        else hipLaunchKernelGGL((k_decode<D, M, S, L, true, 2>), grid, dim3(DT), shm, st, P);
    }
}

template <int D>
void launch_decode_d(int mode, bool sp, bool l0, bool asym, int b0, dim3 grid, size_t shm,
                     const DecodeParams& P, hipStream_t st) {
    if (mode == MODE_REBUILD) {
        if (l0) launch_decode_one<D, MODE_REBUILD, true, true>(asym, b0, grid, shm, P, st);
        else launch_decode_one<D, MODE_REBUILD, true, false>(asym, b0, grid, shm, P, st);
    } else if (sp) {
        if (l0) launch_decode_one<D, MODE_ATTN, true, true>(asym, b0, grid, shm, P, st);
        else launch_decode_one<D, MODE_ATTN, true, false>(asym, b0, grid, shm, P, st);
    } else {
        if (l0) launch_decode_one<D, MODE_ATTN, false, true>(asym, b0, grid, shm, P, st);
        else launch_decode_one<D, MODE_ATTN, false, false>(asym, b0, grid, shm, P, st);
    }
}

hipError_t launch_decode(int d, int mode, const DecodeParams& P, hipStream_t st) {
    const bool sp = P.sel != nullptr;
    size_t shm = (size_t)(P.k + P.n_tail) * sizeof(float) + (sp ? (size_t)(P.level + 1) * P.k * 4 : 0);
    // the (column, level) pair list and partial scores of the sparse absmax
    // passes over more than the base level, when they fit the workgroup's LDS
    // share (else level by level; a base-level-only pass gains nothing)
    DecodeParams Q = P;
    const size_t pair_shm = (size_t)2 * (P.level + 1) * P.k * 4;
    Q.pairs = sp && P.level >= 1 && P.cache.scheme != FL_QUANT_ASYM && P.k < (1 << 26) &&
              shm + pair_shm <= kDecodePairLds;
    if (Q.pairs) shm += pair_shm;
    const dim3 grid(P.B * P.H);
    const bool l0 = P.level == 0;
    const bool asym = P.cache.scheme == FL_QUANT_ASYM;
    const int b0 = P.cache.level[0].bits;
    if (d == 128) launch_decode_d<128>(mode, sp, l0, asym, b0, grid, shm, Q, st);
    else launch_decode_d<64>(mode, sp, l0, asym, b0, grid, shm, Q, st);
    return hipGetLastError();
}

} // namespace fl

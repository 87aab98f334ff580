// Device-side helpers shared by the gfx950 kernels of libflashloop.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flashloop.h"

namespace fl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// 8 consecutive input values as fp32 (bf16 or fp32 storage).
__device__ __forceinline__ void load8_f32(const void* base, long elem_off, int dtype, float* o) {
    if (dtype == FL_BF16) {
        const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem_off);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem_off);
        const float4 a = p[0], b = p[1];
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
}

// 8 consecutive input values as a bf16x8 MFMA operand (fp32 inputs are rounded
// to nearest even).
__device__ __forceinline__ bf16x8 load8_bf16(const void* base, long elem_off, int dtype) {
    if (dtype == FL_BF16) {
        const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem_off);
        return __builtin_bit_cast(bf16x8, u);
    }
    float f[8];
    load8_f32(base, elem_off, FL_F32, f);
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)f[i];
    return r;
}

// Extract code c (0..7) of 8 consecutive codes stored with `bits` per code in
// little-endian order (two's complement), sign-extended.
__device__ __forceinline__ int code_at(uint64_t packed, int bits, int c) {
    const int sh = 64 - bits;
    return (int)((int64_t)(packed << (sh - bits * c)) >> sh);
}

// Load the 8*bits/8 bytes holding 8 consecutive codes.
__device__ __forceinline__ uint64_t load_codes8(const void* base, long code_off, int bits) {
    const uint8_t* p = reinterpret_cast<const uint8_t*>(base) + (code_off * bits) / 8;
    if (bits == 8) return *reinterpret_cast<const uint64_t*>(p);
    if (bits == 4) return *reinterpret_cast<const uint32_t*>(p);
    return *reinterpret_cast<const uint16_t*>(p); // bits == 2
}

// Unsigned code c (0..7) of 8 consecutive codes (asymmetric quantiser).
__device__ __forceinline__ uint32_t ucode_at(uint64_t packed, int bits, int c) {
    return (uint32_t)(packed >> (bits * c)) & ((1u << bits) - 1u);
}

// One level of the asymmetric (min/max) scheme: the dequantised terms
// code*s + z of 8 consecutive channels (offset ch, a multiple of 8, within a
// row of HD = H*d) of row `row` of the level.  Keys carry a scale and offset
// per channel for each group of g consecutive rows; values one per group of
// g channels.  The product and the sum are separate roundings unless the
// including file allows contraction.
__device__ __forceinline__ void deq8_asym(const fl_kv_level& L, int which, long row, int HD,
                                          int ch, int g, float* o) {
    const long e = row * HD + ch;
    const uint64_t w = load_codes8(which ? L.v_codes : L.k_codes, e, L.bits);
    if (which == 0) {
        const long si = (row / g) * HD + ch;
        const float4 s0 = *reinterpret_cast<const float4*>(L.k_scale + si);
        const float4 s1 = *reinterpret_cast<const float4*>(L.k_scale + si + 4);
        const float4 z0 = *reinterpret_cast<const float4*>(L.k_zero + si);
        const float4 z1 = *reinterpret_cast<const float4*>(L.k_zero + si + 4);
        const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const float z[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = (float)ucode_at(w, L.bits, i) * s[i];
            o[i] = p + z[i];
        }
    } else {
        const float s = L.v_scale[e / g], z = L.v_zero[e / g];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = (float)ucode_at(w, L.bits, i) * s;
            o[i] = p + z;
        }
    }
}

// 8 consecutive channels (offset ch, a multiple of 8, within a row of
// HD = H*d) of token j's dequantised keys (which = 0) or values (1) at cache
// levels 0..upto: the base row, then each residual level's row while the
// token is present (the sets are nested, so presence stops at the first
// absent level), summed in level order.  Raw (32-bit) levels hold fp32 values.
__device__ __forceinline__ void deq_col8(const fl_kv_cache& c, int upto, int which, long j, int HD,
                                         int ch, float* x) {
    if (c.scheme == FL_QUANT_ASYM) {
        deq8_asym(c.level[0], which, j, HD, ch, c.g, x);
        for (int l = 1; l <= upto; ++l) {
            const int sl = c.level[l].slot[j];
            if (sl < 0) break;
            float t[8];
            deq8_asym(c.level[l], which, sl, HD, ch, c.g, t);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] += t[i];
        }
        return;
    }
    const fl_kv_level& L0 = c.level[0];
    const long e0 = j * HD + ch;
    const void* codes = which ? L0.v_codes : L0.k_codes;
    if (L0.bits == 32) {
        const float* src = reinterpret_cast<const float*>(codes) + e0;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = src[e];
    } else {
        const float s = (which ? L0.v_scale : L0.k_scale)[e0 / c.g];
        const uint64_t w = load_codes8(codes, e0, 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (float)code_at(w, 8, i) * s;
    }
    for (int l = 1; l <= upto; ++l) {
        const fl_kv_level& L = c.level[l];
        const int sl = L.slot[j];
        if (sl < 0) break;
        const long el = (long)sl * HD + ch;
        const void* cl = which ? L.v_codes : L.k_codes;
        if (L.bits == 32) {
            const float* src = reinterpret_cast<const float*>(cl) + el;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] += src[e];
        } else {
            const float s = (which ? L.v_scale : L.k_scale)[el / c.g];
            const uint64_t w = load_codes8(cl, el, L.bits);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] += (float)code_at(w, L.bits, i) * s;
        }
    }
}

// deq_col8 for the key and the value of one column together, for absmax
// caches with an int8 base and no fp32 levels (deq_batch_ok): the levels go
// in chunks of NB, each chunk's slots in one round of loads and its present
// levels' K and V codes and scales in one more, instead of a slot-then-codes
// round trip per level and side.  The sums keep deq_col8's level order and
// its stop at the first absent level.
constexpr int kDeqBatch = 4;
inline bool deq_batch_ok(const fl_kv_cache& c, int upto) {
    if (c.scheme == FL_QUANT_ASYM) return false;
    for (int l = 0; l <= upto; ++l)
        if (c.level[l].bits == 32 || (l == 0 && c.level[l].bits != 8)) return false;
    return true;
}

// one chunk: levels l0..l0+NB-1 (those <= upto and present) added to x, or
// with l0 == 0 the base level written first; returns false once a level of
// the chunk is absent (all later ones are too)
template <int NB, bool BASE>
__device__ __forceinline__ bool deq_chunk_kv(const fl_kv_cache& c, int upto, int l0, long j, int HD, int ch,
                                             float* xk, float* xv) {
    long row[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u)
        row[u] = (BASE && u == 0) ? j : (l0 + u <= upto ? (long)c.level[l0 + u].slot[j] : -1);
#pragma unroll
    for (int u = 1; u < NB; ++u)
        if (row[u - 1] < 0) row[u] = -1;
    uint64_t wk[NB], wv[NB];
    float sk[NB], sv[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        wk[u] = 0;
        wv[u] = 0;
        sk[u] = 0.0f;
        sv[u] = 0.0f;
        if (row[u] >= 0) {
            const fl_kv_level& L = c.level[l0 + u];
            const int b = (BASE && u == 0) ? 8 : L.bits;
            const long e = row[u] * HD + ch;
            wk[u] = load_codes8(L.k_codes, e, b);
            wv[u] = load_codes8(L.v_codes, e, b);
            sk[u] = L.k_scale[e / c.g];
            sv[u] = L.v_scale[e / c.g];
        }
    }
    if constexpr (BASE) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            xk[i] = (float)code_at(wk[0], 8, i) * sk[0];
            xv[i] = (float)code_at(wv[0], 8, i) * sv[0];
        }
    }
#pragma unroll
    for (int u = BASE ? 1 : 0; u < NB; ++u) {
        if (row[u] >= 0) {
            const int b = c.level[l0 + u].bits;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xk[i] += (float)code_at(wk[u], b, i) * sk[u];
                xv[i] += (float)code_at(wv[u], b, i) * sv[u];
            }
        }
    }
    return row[NB - 1] >= 0;
}

// requires deq_batch_ok(c, upto); one chunk of NB = upto + 1 levels, or
// (CHUNKS) chunks of NB = kDeqBatch
template <int NB, bool CHUNKS>
__device__ __forceinline__ void deq_col8_kv(const fl_kv_cache& c, int upto, long j, int HD, int ch,
                                            float* xk, float* xv) {
    static_assert(NB >= 1 && NB <= kDeqBatch, "levels per chunk");
    bool more = deq_chunk_kv<NB, true>(c, upto, 0, j, HD, ch, xk, xv);
    if constexpr (CHUNKS)
        for (int l0 = NB; more && l0 <= upto; l0 += NB) more = deq_chunk_kv<NB, false>(c, upto, l0, j, HD, ch, xk, xv);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max of a value over lanes l and l ^ 32: gfx950's cross-half lane swap
// (no LDS round trip); the pair's two halves hold x_l and x_{l^32} as a set
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Instruction-order hint for a score block of 16 LDS fragment reads feeding
// 16 MFMAs (place it after the block, inside the same basic block): four
// reads first, then one read behind each MFMA, so every read has about three
// MFMAs' time to land instead of stalling the chain on its own latency.
__device__ __forceinline__ void sched_reads_ahead16() {
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS reads
#pragma unroll
    for (int g = 0; g < 12; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// ---- LDS-DMA tiles (gfx950) ----

// 16-byte-chunk swizzle of a tile row with CPR chunks: the 16 lanes that one
// 128-bit LDS read serves per cycle (16 consecutive rows at one logical
// chunk) land on 16 distinct chunk slots of a 256-byte bank window.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
    static_assert(CPR == 4 || CPR == 8 || CPR == 16, "rows of 64, 128 or 256 bytes");
    return CPR == 16 ? (row & 15) : CPR == 8 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

// Raw buffer resource over [base, base + bytes) (gfx9 data-format word); a
// copy through it takes a scalar base, a per-lane 32-bit offset and a
// scalar offset, so issuing it costs no vector instructions, and offsets
// past `bytes` read zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t r, void* l, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)l, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buf_dma4(__amdgpu_buffer_rsrc_t r, void* l, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)l, 4, voff, soff, 0, 0);
}

// ---- work mapping and position bounds ----

// (row tile, head) of this workgroup, the costliest (latest-position) tiles
// first.  With xcd_remap (H % 8 == 0) every head's workgroups stay on one
// XCD (blocks are dealt to the 8 XCDs round-robin), so the head's compact
// K / V stays in that L2, and the XCD's heads are interleaved so that each
// one's costliest tiles start in the first wave of workgroups.
__device__ __forceinline__ void block_coords(int xcd_remap, int n_tiles, int H, int& tile, int& h) {
    const int b = blockIdx.x;
    if (xcd_remap) {
        const int hpx = H / 8;
        const int x = b & 7, m = b >> 3;
        h = x + 8 * (m % hpx);
        tile = n_tiles - 1 - m / hpx;
    } else {
        h = b / n_tiles;
        tile = n_tiles - 1 - (b % n_tiles);
    }
}

// Number of elements <= v of the ascending a[0, n), found by one whole wave
// (every lane calls it with the same arguments): the last element of each
// of 64 equal blocks, then the block that holds the boundary -- two
// dependent rounds of loads for n <= 4096.
__device__ __forceinline__ int wave_ubound(const int32_t* a, int n, int v) {
    const int lane = threadIdx.x & 63;
    if (n <= 0) return 0;
    const int S = (n + 63) >> 6;
    const bool whole = lane * S < n && a[min((lane + 1) * S, n) - 1] <= v;
    const int lo = __popcll(__ballot(whole)) * S;
    if (lo >= n) return n;
    const int hi = min(lo + S, n);
    int cnt = lo;
    for (int j = lo; j < hi; j += 64) cnt += __popcll(__ballot(j + lane < hi && a[j + lane] <= v));
    return cnt;
}

} // namespace fl

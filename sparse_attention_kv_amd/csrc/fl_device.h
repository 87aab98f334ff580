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

} // namespace fl

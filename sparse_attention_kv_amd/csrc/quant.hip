// KV residual quantisation (FlashLoop paper, Sec. 3.3, Sec. 4.3, App. E
// "Quantization Setting"): the loop-1 K/V are stored as an int8 group-quantised
// base; every later loop stores, for its active tokens only, a low-bit
// quantised residual against the previous loop's dequantised K/V.
//
// One thread owns 8 consecutive channels of one (token, head); the g/8
// threads of a quantisation group are adjacent lanes of one wavefront, so the
// group absmax is a few lane exchanges.  Per token the kernel reads the new
// bf16/fp32 values and the token's previous levels (int8 base + residual
// codes and scales), and writes the new level's codes and scale.  It is
// HBM-bound; the arithmetic is kept bit-reproducible: IEEE fp32, correctly
// rounded division, round-half-even (v_rndne), and no multiply-add
// contraction, so xhat = xhat + code*s rounds the product and the sum
// separately in level order.
#include "fl_device.h"
#include "fl_kernels.h"

#pragma clang fp contract(off)

namespace fl {

struct QuantArgs {
    int N, H, d, g, level, bits, dtype, gathered;
    const void* k_new;
    const void* v_new;
    fl_kv_cache cache;
};

// Dequantise 8 consecutive channels (flat element offset within a token row
// of H*d) of one token from levels 0..upto (inclusive) in level order.
__device__ __forceinline__ void dequant8_chain(const fl_kv_cache& c, int which, long pos,
                                               int ch, int upto, float* x) {
    const int HD = c.H * c.d;
    {
        const fl_kv_level& L = c.level[0];
        const void* codes = which ? L.v_codes : L.k_codes;
        const long e = pos * HD + ch;
        if (L.bits == 32) {
            const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(codes) + e);
            const float4 a = p[0], b = p[1];
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
            x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        } else {
            const float s = (which ? L.v_scale : L.k_scale)[e / c.g];
            const uint64_t w = load_codes8(codes, e, L.bits);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = (float)code_at(w, L.bits, i) * s;
        }
    }
    for (int l = 1; l <= upto; ++l) {
        const fl_kv_level& L = c.level[l];
        const int sl = L.slot[pos];
        if (sl < 0) break; // nested sets: absent here means absent later
        const void* codes = which ? L.v_codes : L.k_codes;
        const long e = (long)sl * HD + ch;
        if (L.bits == 32) {
            const float* p = reinterpret_cast<const float*>(codes) + e;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = x[i] + p[i];
        } else {
            const float s = (which ? L.v_scale : L.k_scale)[e / c.g];
            const uint64_t w = load_codes8(codes, e, L.bits);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float dq = (float)code_at(w, L.bits, i) * s;
                x[i] = x[i] + dq;
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_quant(QuantArgs a, long n_threads) {
    const long gid = blockIdx.x * (long)blockDim.x + threadIdx.x;
    const int which = blockIdx.y; // 0 = K, 1 = V
    const int HD = a.H * a.d;
    const int per_row = HD / 8;
    const long t = gid / per_row;
    const int ch = (int)(gid % per_row) * 8;
    const bool live = gid < n_threads;
    const fl_kv_level& L = a.cache.level[a.level];
    const long pos = live ? (a.level == 0 ? t : (long)L.rows[t]) : 0;

    float x[8];
    if (live) {
        const void* src = which ? a.v_new : a.k_new;
        const long row = a.gathered ? t : pos;
        load8_f32(src, row * HD + ch, a.dtype, x);
        if (a.level > 0) {
            float xp[8];
            dequant8_chain(a.cache, which, pos, ch, a.level - 1, xp);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = x[i] - xp[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.0f;
    }
    void* codes = which ? L.v_codes : L.k_codes;
    const long e = t * HD + ch;
    if (a.bits == 32) {
        if (live) {
            float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(codes) + e);
            p[0] = make_float4(x[0], x[1], x[2], x[3]);
            p[1] = make_float4(x[4], x[5], x[6], x[7]);
        }
        return;
    }
    // group absmax across the g/8 adjacent lanes of this group
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    for (int o = 1; o < a.g / 8; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if (!live) return;
    const int qmax = (1 << (a.bits - 1)) - 1;
    const float s = amax / (float)qmax;
    uint64_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int q = 0;
        if (s != 0.0f) {
            float r = __builtin_rintf(x[i] / s);
            r = fminf(fmaxf(r, -(float)qmax), (float)qmax);
            q = (int)r;
        }
        packed |= (uint64_t)((uint32_t)q & ((1u << a.bits) - 1u)) << (a.bits * i);
    }
    uint8_t* dst = reinterpret_cast<uint8_t*>(codes) + (e * a.bits) / 8;
    if (a.bits == 8) *reinterpret_cast<uint64_t*>(dst) = packed;
    else if (a.bits == 4) *reinterpret_cast<uint32_t*>(dst) = (uint32_t)packed;
    else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
    if ((ch % a.g) == 0) (which ? L.v_scale : L.k_scale)[e / a.g] = s;
}

hipError_t launch_quant(const fl_kv_cache& cache, int level, int dtype, const void* k_new,
                        const void* v_new, int gathered, hipStream_t st) {
    QuantArgs a;
    a.N = cache.N; a.H = cache.H; a.d = cache.d; a.g = cache.g;
    a.level = level; a.bits = cache.level[level].bits; a.dtype = dtype; a.gathered = gathered;
    a.k_new = k_new; a.v_new = v_new; a.cache = cache;
    const long rows = level == 0 ? cache.N : cache.level[level].n_rows;
    const long n_threads = rows * (cache.H * cache.d / 8);
    if (n_threads == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n_threads + 255) / 256);
    hipLaunchKernelGGL(k_quant, dim3(blocks, 2), dim3(256), 0, st, a, n_threads);
    return hipGetLastError();
}

} // namespace fl

// KV residual quantisation (FlashLoop paper, Sec. 3.3, Sec. 4.3, App. E
// "Quantization Setting"): the loop-1 K/V are stored as an int8 group-quantised
// base; every later loop stores, for its active tokens only, a low-bit
// quantised residual against the previous loop's dequantised K/V.  Under the
// asymmetric scheme (the paper's own: min/max groups, keys per channel over g
// consecutive packed rows, values per token) values take the same per-thread
// path with a min/max group reduction and keys go through k_quant_kchan.
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
    if (c.scheme == FL_QUANT_ASYM) {
        deq8_asym(c.level[0], which, pos, HD, ch, c.g, x);
        for (int l = 1; l <= upto; ++l) {
            const int sl = c.level[l].slot[pos];
            if (sl < 0) break;
            float t[8];
            deq8_asym(c.level[l], which, sl, HD, ch, c.g, t);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = x[i] + t[i];
        }
        return;
    }
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

// The value to quantise for 8 channels of packed row t: the new value, minus
// the token's previous dequantised value for a residual level.
// xp: the previous dequantised value (zeros at level 0).
__device__ __forceinline__ void quant_input8(const QuantArgs& a, int which, long t, long pos,
                                             int ch, float* x, float* xp) {
    const int HD = a.H * a.d;
    const void* src = which ? a.v_new : a.k_new;
    const long row = a.gathered ? t : pos;
    load8_f32(src, row * HD + ch, a.dtype, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) xp[i] = 0.0f;
    if (a.level > 0) {
        dequant8_chain(a.cache, which, pos, ch, a.level - 1, xp);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = x[i] - xp[i];
    }
}

// The token's operand class for one head (cache.cls): 1 when some channel
// of its new dequantised value xh (8 per lane, d/8 adjacent lanes per head)
// exceeds kTauCol in magnitude or is not finite.  Every lane of the head
// group takes part; lane 0 of the group writes.
__device__ __forceinline__ void store_class8(const QuantArgs& a, int which, long pos, int ch,
                                             const float* xh) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float v = fabsf(xh[i]);
        m = v <= m ? m : (v > m ? v : INFINITY);
    }
    for (int o = 1; o < a.d / 8; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (ch % a.d == 0)
        a.cache.cls[((long)which * a.N + pos) * a.H + ch / a.d] = !(m <= kTauCol);
}

__device__ __forceinline__ void store_codes8(void* codes, long e, int bits, uint64_t packed) {
    uint8_t* dst = reinterpret_cast<uint8_t*>(codes) + (e * bits) / 8;
    if (bits == 8) *reinterpret_cast<uint64_t*>(dst) = packed;
    else if (bits == 4) *reinterpret_cast<uint32_t*>(dst) = (uint32_t)packed;
    else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
}

// Asymmetric code of x: round-half-even((x - z)/s) clamped to [0, qmax].
__device__ __forceinline__ uint32_t asym_code(float x, float s, float z, int qmax) {
    if (s == 0.0f) return 0u;
    const float t = x - z;
    float r = __builtin_rintf(t / s);
    r = fminf(fmaxf(r, 0.0f), (float)qmax);
    return (uint32_t)r;
}

// Keys of an asymmetric level: one workgroup per (group of G consecutive
// packed rows, 256 channels).  Lane l of wave w owns 8 channels (l mod 32)
// and the rows rl, rl + 8, ... of the group (rl = 2w + l/32), keeping their
// inputs in registers; the per-channel minimum and maximum are reduced over
// the 8 row lanes (exact, so independent of order; a signed zero is stored
// as +0), then each lane writes its rows' codes.
template <int G>
__global__ __launch_bounds__(256) void k_quant_kchan(QuantArgs a) {
    constexpr int RPT = G / 8; // rows per thread
    __shared__ float s_mn[4][32][8], s_mx[4][32][8];
    const int HD = a.H * a.d;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cl = lane & 31;
    const int rl = wave * 2 + (lane >> 5);
    const long grp = blockIdx.x;
    const int ch = blockIdx.y * 256 + cl * 8;
    const bool live_ch = ch < HD;
    const fl_kv_level& L = a.cache.level[a.level];
    const long n_rows = a.level == 0 ? a.N : L.n_rows;
    const long r0 = grp * G;
    float x[RPT][8];
    float mn[8], mx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { mn[i] = __builtin_inff(); mx[i] = -__builtin_inff(); }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const long t = r0 + rl + 8 * j;
        if (live_ch && t < n_rows) {
            const long pos = a.level == 0 ? t : (long)L.rows[t];
            float xp[8];
            quant_input8(a, 0, t, pos, ch, x[j], xp);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (x[j][i] < mn[i]) mn[i] = x[j][i];
                if (x[j][i] > mx[i]) mx[i] = x[j][i];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float omn = __shfl_xor(mn[i], 32), omx = __shfl_xor(mx[i], 32);
        if (omn < mn[i]) mn[i] = omn;
        if (omx > mx[i]) mx[i] = omx;
    }
    if (lane < 32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) { s_mn[wave][cl][i] = mn[i]; s_mx[wave][cl][i] = mx[i]; }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        mn[i] = s_mn[0][cl][i]; mx[i] = s_mx[0][cl][i];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            if (s_mn[w][cl][i] < mn[i]) mn[i] = s_mn[w][cl][i];
            if (s_mx[w][cl][i] > mx[i]) mx[i] = s_mx[w][cl][i];
        }
    }
    if (!live_ch) return;
    const int qmax = (1 << a.bits) - 1;
    float s[8], z[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        z[i] = mn[i] + 0.0f;
        const float range = mx[i] - z[i];
        s[i] = range / (float)qmax + 0.0f;
    }
    if (rl == 0) {
        const long si = grp * HD + ch;
        *reinterpret_cast<float4*>(L.k_scale + si) = make_float4(s[0], s[1], s[2], s[3]);
        *reinterpret_cast<float4*>(L.k_scale + si + 4) = make_float4(s[4], s[5], s[6], s[7]);
        *reinterpret_cast<float4*>(L.k_zero + si) = make_float4(z[0], z[1], z[2], z[3]);
        *reinterpret_cast<float4*>(L.k_zero + si + 4) = make_float4(z[4], z[5], z[6], z[7]);
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const long t = r0 + rl + 8 * j;
        if (t < n_rows) {
            uint64_t packed = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                packed |= (uint64_t)asym_code(x[j][i], s[i], z[i], qmax) << (a.bits * i);
            store_codes8(L.k_codes, t * HD + ch, a.bits, packed);
        }
    }
}

// which0 = 0: keys and values (grid.y = 2); which0 = 1: values only.
__global__ __launch_bounds__(256) void k_quant(QuantArgs a, long n_threads, int which0) {
    const long gid = blockIdx.x * (long)blockDim.x + threadIdx.x;
    const int which = which0 + blockIdx.y; // 0 = K, 1 = V
    const int HD = a.H * a.d;
    const int per_row = HD / 8;
    const long t = gid / per_row;
    const int ch = (int)(gid % per_row) * 8;
    const bool live = gid < n_threads;
    const fl_kv_level& L = a.cache.level[a.level];
    const long pos = live ? (a.level == 0 ? t : (long)L.rows[t]) : 0;

    float x[8], xp[8];
    if (live) {
        quant_input8(a, which, t, pos, ch, x, xp);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = xp[i] = 0.0f;
    }
    // per-token classes kept for the attention (symmetric scheme)
    const bool keep_cls = a.cache.cls != nullptr && a.cache.scheme == FL_QUANT_ABSMAX;
    void* codes = which ? L.v_codes : L.k_codes;
    const long e = t * HD + ch;
    if (a.bits == 32) {
        if (live) {
            float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(codes) + e);
            p[0] = make_float4(x[0], x[1], x[2], x[3]);
            p[1] = make_float4(x[4], x[5], x[6], x[7]);
            if (keep_cls) {  // (live is uniform over a head's lanes)
                float xh[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) xh[i] = a.level > 0 ? xp[i] + x[i] : x[i];
                store_class8(a, which, pos, ch, xh);
            }
        }
        return;
    }
    if (a.cache.scheme == FL_QUANT_ASYM) {
        // group min / max across the g/8 adjacent lanes of this group
        float mn = x[0], mx = x[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            if (x[i] < mn) mn = x[i];
            if (x[i] > mx) mx = x[i];
        }
        for (int o = 1; o < a.g / 8; o <<= 1) {
            const float omn = __shfl_xor(mn, o), omx = __shfl_xor(mx, o);
            if (omn < mn) mn = omn;
            if (omx > mx) mx = omx;
        }
        if (!live) return;
        const int qmax = (1 << a.bits) - 1;
        const float z = mn + 0.0f;
        const float range = mx - z;
        const float s = range / (float)qmax + 0.0f;
        uint64_t packed = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) packed |= (uint64_t)asym_code(x[i], s, z, qmax) << (a.bits * i);
        store_codes8(codes, e, a.bits, packed);
        if ((ch % a.g) == 0) {
            L.v_scale[e / a.g] = s;
            L.v_zero[e / a.g] = z;
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
    float xh[8];  // the new dequantised value, in the readers' order: previous + code * s
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int q = 0;
        if (s != 0.0f) {
            float r = __builtin_rintf(x[i] / s);
            r = fminf(fmaxf(r, -(float)qmax), (float)qmax);
            q = (int)r;
        }
        packed |= (uint64_t)((uint32_t)q & ((1u << a.bits) - 1u)) << (a.bits * i);
        const float dq = (float)q * s;
        xh[i] = a.level > 0 ? xp[i] + dq : dq;
    }
    store_codes8(codes, e, a.bits, packed);
    if ((ch % a.g) == 0) (which ? L.v_scale : L.k_scale)[e / a.g] = s;
    if (keep_cls) store_class8(a, which, pos, ch, xh);
}

// Reconstruction of every token's K or V at loop level+1 (levels 0..level in
// order, each token's chain stopping at its first absent level), fp32.
__global__ __launch_bounds__(256) void k_dequant(fl_kv_cache c, int level, int which,
                                                 float* __restrict__ out, long n_threads) {
    const long gid = blockIdx.x * (long)blockDim.x + threadIdx.x;
    if (gid >= n_threads) return;
    const int HD = c.H * c.d;
    const int per_row = HD / 8;
    const long pos = gid / per_row;
    const int ch = (int)(gid % per_row) * 8;
    float x[8];
    dequant8_chain(c, which, pos, ch, level, x);
    float4* o = reinterpret_cast<float4*>(out + pos * HD + ch);
    o[0] = make_float4(x[0], x[1], x[2], x[3]);
    o[1] = make_float4(x[4], x[5], x[6], x[7]);
}

hipError_t launch_dequant(const fl_kv_cache& cache, int level, int which, float* out,
                          hipStream_t st) {
    const long n_threads = (long)cache.N * (cache.H * cache.d / 8);
    hipLaunchKernelGGL(k_dequant, dim3((unsigned)((n_threads + 255) / 256)), dim3(256), 0, st,
                       cache, level, which, out, n_threads);
    return hipGetLastError();
}

// Generation-time append: the P.n tokens in window slots P.slot + z (mod the
// ring; computed in all R loops) become positions P.pos + z of every
// sequence's cache.  One workgroup per (sequence, K or V, token z); a thread
// owns 8 channels per pass.  Level 0 quantises the loop-1 value (row =
// position); level l >= 1 appends row n_rows[l] + z with the residual of the
// loop-(l+1) value against the running dequantised value, which is then
// updated with the level's own dequantised term -- the same roundings, in
// the same order, as k_quant and its dequantisation chain.
__global__ __launch_bounds__(256) void k_decode_append(AppendParams P, int D) {
    const int b = blockIdx.x, which = blockIdx.y, z = blockIdx.z;
    const int HD = P.H * D;
    const int g = P.g;
    int wslot = P.slot + z;
    if (wslot >= P.win_cap) wslot -= P.win_cap;
    for (int base = 0; base < HD; base += 256 * 8) {
        const int ch = base + threadIdx.x * 8;
        const bool live = ch < HD;
        float xh[8];
        for (int l = 0; l < P.R; ++l) {
            const void* src = which ? P.wv[l] : P.wk[l];
            float x[8];
            if (live) {
                load8_f32(src, ((long)b * P.win_cap + wslot) * HD + ch, FL_BF16, x);
                if (l > 0) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) x[i] = x[i] - xh[i];
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = 0.0f;
            }
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
            for (int o = 1; o < g / 8; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
            const int bits = P.bits[l];
            const int qmax = (1 << (bits - 1)) - 1;
            const float s = amax / (float)qmax;
            uint64_t packed = 0;
            int q[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                q[i] = 0;
                if (s != 0.0f) {
                    float r = __builtin_rintf(x[i] / s);
                    r = fminf(fmaxf(r, -(float)qmax), (float)qmax);
                    q[i] = (int)r;
                }
                packed |= (uint64_t)((uint32_t)q[i] & ((1u << bits) - 1u)) << (bits * i);
            }
            if (live) {
                const fl_kv_level& L = P.lev[l];
                const long rows = l == 0 ? P.pos_cap : P.rows_cap[l];
                const long row = (l == 0 ? P.pos : P.n_rows[l]) + z;
                uint8_t* codes = reinterpret_cast<uint8_t*>(which ? L.v_codes : L.k_codes) +
                                 (long)b * (rows * HD * bits / 8);
                float* scales = (which ? L.v_scale : L.k_scale) + (long)b * (rows * (HD / g));
                const long e = row * HD + ch;
                store_codes8(codes, e, bits, packed);
                if ((ch % g) == 0) scales[e / g] = s;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float dq = (float)q[i] * s;
                    xh[i] = l == 0 ? dq : xh[i] + dq;
                }
            }
        }
    }
    if (which == 0 && threadIdx.x == 0) {
        for (int l = 1; l < P.R; ++l) {
            int32_t* rows = const_cast<int32_t*>(P.lev[l].rows) + (long)b * P.rows_cap[l];
            int32_t* slot = const_cast<int32_t*>(P.lev[l].slot) + (long)b * P.pos_cap;
            rows[P.n_rows[l] + z] = P.pos + z;
            slot[P.pos + z] = P.n_rows[l] + z;
        }
    }
}

// Generation-time append under the asymmetric scheme: the G tokens in window
// slots P.slot + j (mod the ring) become positions P.pos + j and one new key
// group of every level (group (row0 + kg_pad) / G of the level's first new
// row row0).  One workgroup per (sequence, 256 channels, K or V) with the
// thread layout of k_quant_kchan: lane l of wave w owns 8 channels (l mod 32)
// and the tokens rl, rl + 8, ... (rl = 2w + l/32), keeping their inputs and
// running dequantised values in registers across the levels.  Keys: per
// channel minimum / maximum over the G tokens (lane pairs, then the 4 waves
// through LDS); values: per token over G channels (G/8 adjacent lanes).  The
// codes, scales and offsets, and the chain xhat += code * s + z, round as
// k_quant_kchan, k_quant and their dequantisation do.
template <int G>
__global__ __launch_bounds__(256) void k_decode_append_asym(AppendParams P, int D) {
    constexpr int RPT = G / 8; // tokens per thread
    __shared__ float s_mn[4][32][8], s_mx[4][32][8];
    const int b = blockIdx.x, which = blockIdx.z;
    const int HD = P.H * D;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cl = lane & 31;
    const int rl = wave * 2 + (lane >> 5);
    const int ch = blockIdx.y * 256 + cl * 8;
    const bool live = ch < HD;
    float xh[RPT][8];
    for (int l = 0; l < P.R; ++l) {
        const void* src = which ? P.wv[l] : P.wk[l];
        float x[RPT][8];
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            int ws = P.slot + rl + 8 * j;
            if (ws >= P.win_cap) ws -= P.win_cap;
            if (live) {
                load8_f32(src, ((long)b * P.win_cap + ws) * HD + ch, FL_BF16, x[j]);
                if (l > 0) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) x[j][i] = x[j][i] - xh[j][i];
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) x[j][i] = 0.0f;
            }
        }
        const int bits = P.bits[l];
        const int qmax = (1 << bits) - 1;
        const fl_kv_level& L = P.lev[l];
        const long rows = l == 0 ? P.pos_cap : P.rows_cap[l];
        const long row0 = l == 0 ? P.pos : P.n_rows[l];
        uint8_t* codes = reinterpret_cast<uint8_t*>(which ? L.v_codes : L.k_codes) +
                         (long)b * (rows * HD * bits / 8);
        if (which == 0) {
            float mn[8], mx[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) { mn[i] = x[0][i]; mx[i] = x[0][i]; }
#pragma unroll
            for (int j = 1; j < RPT; ++j)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (x[j][i] < mn[i]) mn[i] = x[j][i];
                    if (x[j][i] > mx[i]) mx[i] = x[j][i];
                }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float omn = __shfl_xor(mn[i], 32), omx = __shfl_xor(mx[i], 32);
                if (omn < mn[i]) mn[i] = omn;
                if (omx > mx[i]) mx[i] = omx;
            }
            __syncthreads(); // the previous level's reads of s_mn / s_mx are done
            if (lane < 32) {
#pragma unroll
                for (int i = 0; i < 8; ++i) { s_mn[wave][cl][i] = mn[i]; s_mx[wave][cl][i] = mx[i]; }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                mn[i] = s_mn[0][cl][i]; mx[i] = s_mx[0][cl][i];
#pragma unroll
                for (int w = 1; w < 4; ++w) {
                    if (s_mn[w][cl][i] < mn[i]) mn[i] = s_mn[w][cl][i];
                    if (s_mx[w][cl][i] > mx[i]) mx[i] = s_mx[w][cl][i];
                }
            }
            float s[8], zz[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                zz[i] = mn[i] + 0.0f;
                const float range = mx[i] - zz[i];
                s[i] = range / (float)qmax + 0.0f;
            }
            if (live) {
                if (rl == 0) {
                    const long si = ((long)b * P.kg_count[l] + (row0 + P.kg_pad[l]) / G) * HD + ch;
                    *reinterpret_cast<float4*>(L.k_scale + si) = make_float4(s[0], s[1], s[2], s[3]);
                    *reinterpret_cast<float4*>(L.k_scale + si + 4) = make_float4(s[4], s[5], s[6], s[7]);
                    *reinterpret_cast<float4*>(L.k_zero + si) = make_float4(zz[0], zz[1], zz[2], zz[3]);
                    *reinterpret_cast<float4*>(L.k_zero + si + 4) = make_float4(zz[4], zz[5], zz[6], zz[7]);
                }
#pragma unroll
                for (int j = 0; j < RPT; ++j) {
                    uint64_t packed = 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint32_t q = asym_code(x[j][i], s[i], zz[i], qmax);
                        packed |= (uint64_t)q << (bits * i);
                        const float p = (float)q * s[i];
                        const float t = p + zz[i];
                        xh[j][i] = l == 0 ? t : xh[j][i] + t;
                    }
                    store_codes8(codes, (row0 + rl + 8 * j) * HD + ch, bits, packed);
                }
            }
        } else {
            float* vs = L.v_scale + (long)b * (rows * (HD / G));
            float* vz = L.v_zero + (long)b * (rows * (HD / G));
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                float mn = x[j][0], mx = x[j][0];
#pragma unroll
                for (int i = 1; i < 8; ++i) {
                    if (x[j][i] < mn) mn = x[j][i];
                    if (x[j][i] > mx) mx = x[j][i];
                }
#pragma unroll
                for (int o = 1; o < G / 8; o <<= 1) {
                    const float omn = __shfl_xor(mn, o), omx = __shfl_xor(mx, o);
                    if (omn < mn) mn = omn;
                    if (omx > mx) mx = omx;
                }
                const float zz = mn + 0.0f;
                const float range = mx - zz;
                const float s = range / (float)qmax + 0.0f;
                if (live) {
                    const long e = (row0 + rl + 8 * j) * HD + ch;
                    uint64_t packed = 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint32_t q = asym_code(x[j][i], s, zz, qmax);
                        packed |= (uint64_t)q << (bits * i);
                        const float p = (float)q * s;
                        const float t = p + zz;
                        xh[j][i] = l == 0 ? t : xh[j][i] + t;
                    }
                    store_codes8(codes, e, bits, packed);
                    if ((ch % G) == 0) {
                        vs[e / G] = s;
                        vz[e / G] = zz;
                    }
                }
            }
        }
    }
    if (which == 0 && blockIdx.y == 0 && threadIdx.x < G) {
        const int j = threadIdx.x;
        for (int l = 1; l < P.R; ++l) {
            int32_t* rows = const_cast<int32_t*>(P.lev[l].rows) + (long)b * P.rows_cap[l];
            int32_t* slot = const_cast<int32_t*>(P.lev[l].slot) + (long)b * P.pos_cap;
            rows[P.n_rows[l] + j] = P.pos + j;
            slot[P.pos + j] = P.n_rows[l] + j;
        }
    }
}

hipError_t launch_decode_append(int d, int scheme, const AppendParams& P, hipStream_t st) {
    if (scheme == FL_QUANT_ASYM) {
        const dim3 grid(P.B, (unsigned)((P.H * d + 255) / 256), 2);
        if (P.g == 64) hipLaunchKernelGGL(k_decode_append_asym<64>, grid, dim3(256), 0, st, P, d);
        else hipLaunchKernelGGL(k_decode_append_asym<32>, grid, dim3(256), 0, st, P, d);
    } else {
        hipLaunchKernelGGL(k_decode_append, dim3(P.B, 2, P.n), dim3(256), 0, st, P, d);
    }
    return hipGetLastError();
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
    if (cache.scheme == FL_QUANT_ASYM) {
        hipLaunchKernelGGL(k_quant, dim3(blocks, 1), dim3(256), 0, st, a, n_threads, 1);
        const dim3 kgrid((unsigned)((rows + cache.g - 1) / cache.g),
                         (unsigned)((cache.H * cache.d + 255) / 256));
        if (cache.g == 64) hipLaunchKernelGGL(k_quant_kchan<64>, kgrid, dim3(256), 0, st, a);
        else hipLaunchKernelGGL(k_quant_kchan<32>, kgrid, dim3(256), 0, st, a);
    } else {
        hipLaunchKernelGGL(k_quant, dim3(blocks, 2), dim3(256), 0, st, a, n_threads, 0);
    }
    return hipGetLastError();
}

} // namespace fl

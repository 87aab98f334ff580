// Batched decode of the lazy-update loop attention (FlashLoop paper,
// Sec. 4.2 sparse attention over the selected key columns with the cached
// probability mass; Sec. 5.3.1: decode is bound by KV traffic, which the
// column sparsity and the low-bit residuals cut).
//
// One workgroup per (sequence, head) and one new query token.  The key
// columns are the selected prefix columns (all of them in the dense first
// loop) plus the token's own fresh bf16 key/value ("self" column).
//   phase 1  score of every column, one column per thread: the quantised
//            base + residual chain of the key is read straight from the cache
//            (int8 row of d bytes, then the present residual levels) and
//            dotted with q in fp32, scale applied per group;
//   phase 2  block max / sum -> lse, probabilities kept in LDS;
//   phase 3  P.V with d/8 channel groups x 2048/d column slices per
//            workgroup (a wavefront reads 64*8/d value rows of d bytes per
//            load), slices reduced through LDS.
// MODE_ATTN writes o = sum P V + O_U (P carries 1 - M_U), lse and the column
// probabilities (the next loop's column statistic).  MODE_REBUILD recomputes
// the previous loop's probabilities on the kept columns and its self column
// and stores M_U = 1 - sum P, O_U = o_prev - sum P V.
#include "fl_device.h"
#include "fl_kernels.h"

namespace fl {

constexpr int DT = 256; // threads per workgroup

template <int D>
__device__ __forceinline__ void seq_level_ptrs(const fl_kv_cache& c, int l, int b, int which,
                                               const uint8_t*& codes, const float*& scales,
                                               const int32_t*& slot, long& rows) {
    const fl_kv_level& L = c.level[l];
    rows = l == 0 ? c.N : L.n_rows;
    const long cb = (long)rows * c.H * D * L.bits / 8;
    const long sb = (long)rows * c.H * (D / c.g);
    codes = reinterpret_cast<const uint8_t*>(which ? L.v_codes : L.k_codes) + b * cb;
    scales = (which ? L.v_scale : L.k_scale) + b * sb;
    slot = l == 0 ? nullptr : L.slot + (long)b * c.N;
}

template <int D, int MODE, bool SPARSE>
__global__ __launch_bounds__(DT) void k_decode(DecodeParams P) {
    extern __shared__ float sc[]; // [k + 1] scores / probabilities
    __shared__ float qs[D];
    __shared__ float red[DT / 64];
    constexpr int CG = D / 8, CS = DT / CG; // channel groups of 8 x column slices
    __shared__ float ored[CS][D + 4];
    const int bh = blockIdx.x;
    const int b = bh / P.H, h = bh % P.H;
    const int tid = threadIdx.x;
    const fl_kv_cache& C = P.cache;
    const int G = D / C.g;
    const int k = P.k;
    const long qo = (long)bh * D;
    for (int c = tid; c < D; c += DT)
        qs[c] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(P.q)[qo + c]);
    __syncthreads();
    const int32_t* sel = SPARSE ? P.sel + (long)bh * k : nullptr;
    const float c2 = P.sm * 1.4426950408889634f;

    // ---- phase 1: scores (log2 units) ----
    for (int c = tid; c < k; c += DT) {
        const long j = SPARSE ? sel[c] : c;
        float s = 0.0f;
        for (int l = 0; l <= P.level; ++l) {
            const uint8_t* codes; const float* scales; const int32_t* slot; long rows;
            seq_level_ptrs<D>(C, l, b, 0, codes, scales, slot, rows);
            const long row = l == 0 ? j : (long)slot[j];
            if (row < 0) break; // nested sets: absent here means absent later
            const int bits = C.level[l].bits;
            const long e0 = (row * C.H + h) * D;
            for (int gi = 0; gi < G; ++gi) {
                float acc = 0.0f;
                for (int e8 = 0; e8 < C.g; e8 += 8) {
                    const uint64_t w = load_codes8(codes, e0 + gi * C.g + e8, bits);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc += qs[gi * C.g + e8 + i] * (float)code_at(w, bits, i);
                }
                s += acc * scales[(row * C.H + h) * G + gi];
            }
        }
        sc[c] = s * c2;
    }
    if (tid < 64) { // self column: the token's own bf16 key
        float s = 0.0f;
        for (int c = tid; c < D; c += 64)
            s += qs[c] * bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(P.kself)[qo + c]);
        s = wave_sum(s);
        if (tid == 0) sc[k] = s * c2;
    }
    __syncthreads();

    // ---- phase 2: softmax statistics ----
    float wgt, lse2;
    if (MODE == MODE_ATTN) {
        float m = -INFINITY;
        for (int c = tid; c <= k; c += DT) m = fmaxf(m, sc[c]);
        m = wave_max(m);
        if ((tid & 63) == 0) red[tid >> 6] = m;
        __syncthreads();
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
        float z = 0.0f;
        for (int c = tid; c <= k; c += DT) z += __builtin_amdgcn_exp2f(sc[c] - m);
        z = wave_sum(z);
        if ((tid & 63) == 0) red[tid >> 6] = z;
        __syncthreads();
        z = red[0] + red[1] + red[2] + red[3];
        lse2 = m + __log2f(z);
        wgt = P.cache_op == FL_CACHE_ZERO ? 1.0f : 1.0f - P.mass_u[bh];
    } else {
        lse2 = P.lse[bh] * 1.4426950408889634f;
        wgt = 1.0f - P.mass_u[bh];
    }
    float psum = 0.0f;
    for (int c = tid; c <= k; c += DT) {
        const float p = wgt * __builtin_amdgcn_exp2f(sc[c] - lse2);
        sc[c] = p;
        psum += p;
    }
    __syncthreads();

    // ---- phase 3: P.V ----
    const int cg = tid % CG, cs = tid / CG;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int c = cs; c < k; c += CS) {
        const long j = SPARSE ? sel[c] : c;
        const float p = sc[c];
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
        for (int l = 0; l <= P.level; ++l) {
            const uint8_t* codes; const float* scales; const int32_t* slot; long rows;
            seq_level_ptrs<D>(C, l, b, 1, codes, scales, slot, rows);
            const long row = l == 0 ? j : (long)slot[j];
            if (row < 0) break;
            const int bits = C.level[l].bits;
            const long e = (row * C.H + h) * D + cg * 8;
            const float s = scales[e / C.g];
            const uint64_t w = load_codes8(codes, e, bits);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] += (float)code_at(w, bits, i) * s;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += p * v[i];
    }
    if (cs == 0) {
        const float p = sc[k];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] += p * bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(P.vself)[qo + cg * 8 + i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) ored[cs][cg * 8 + i] = acc[i];
    psum = wave_sum(psum);
    if ((tid & 63) == 0) red[tid >> 6] = psum;
    __syncthreads();
    const float ptot = red[0] + red[1] + red[2] + red[3];
    for (int c = tid; c < D; c += DT) {
        float o = 0.0f;
#pragma unroll
        for (int s = 0; s < CS; ++s) o += ored[s][c];
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

hipError_t launch_decode(int d, int mode, const DecodeParams& P, hipStream_t st) {
    const size_t shm = (size_t)(P.k + 1) * sizeof(float);
    dim3 grid(P.B * P.H);
    const bool sp = P.sel != nullptr;
#define FL_DEC(D_, M_, S_) hipLaunchKernelGGL((k_decode<D_, M_, S_>), grid, dim3(DT), shm, st, P)
#define FL_DEC_D(D_)                                                                     \
    if (mode == MODE_REBUILD) FL_DEC(D_, MODE_REBUILD, true);                           \
    else if (sp) FL_DEC(D_, MODE_ATTN, true);                                           \
    else FL_DEC(D_, MODE_ATTN, false);
    if (d == 128) { FL_DEC_D(128) } else { FL_DEC_D(64) }
#undef FL_DEC_D
#undef FL_DEC
    return hipGetLastError();
}

} // namespace fl

// Token-sparse looped block (FlashLoop paper, Sec. 4.1 "the looped
// Transformer block performs computation only on the selected active
// tokens"; Sec. 4.4 "gathering selected tokens ... into compact,
// compute-friendly buffers to preserve regular GEMM execution").
//
//   k_rmsnorm_gather  active rows of the fp32 residual stream -> RMSNorm ->
//                     compact bf16 [n][D] (the gather is fused into the norm)
//   k_gemm_lds<EPI,TN> C = A[M][K] . W[N][K]^T, bf16 MFMA 32x32x16 with fp32
//                     accumulation; 128 x TN output tile per workgroup (4 waves
//                     of 64 x TN/2), 64-deep K tiles in a two-buffer LDS-DMA
//                     pipeline.  Epilogues: bf16 store; residual scatter-add
//                     into the fp32 stream at the active rows; SwiGLU on
//                     interleaved (gate, up) column pairs.
//   k_rope_split      [n][3D] bf16 -> q, k, v [n][H][d] bf16 with rotary
//                     position embedding (rotate-half) on q and k at the rows'
//                     token positions (keys are quantised after RoPE).
//   k_scatter_rows_bf16: row scatter helper.
#include "fl_device.h"
#include "fl_kernels.h"

namespace fl {

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rmsnorm_gather(const float* __restrict__ x,
                                                        const int32_t* __restrict__ rows, int D,
                                                        const __bf16* __restrict__ w, float eps,
                                                        __bf16* __restrict__ out) {
    __shared__ float red[4];
    const int m = blockIdx.x;
    const long row = rows ? rows[m] : m;
    const float* xr = x + row * D;
    float ss = 0.0f;
    for (int c = threadIdx.x * 4; c < D; c += 256 * 4) {
        const float4 v = *reinterpret_cast<const float4*>(xr + c);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = red[0] + red[1] + red[2] + red[3];
    const float inv = rsqrtf(tot / (float)D + eps);
    __bf16* o = out + (long)m * D;
    for (int c = threadIdx.x * 4; c < D; c += 256 * 4) {
        const float4 v = *reinterpret_cast<const float4*>(xr + c);
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) o[c + i] = (__bf16)(vv[i] * inv * (float)w[c + i]);
    }
}

// ---------------------------------------------------------------------------
constexpr int GBM = 128; // output rows per workgroup

// ---------------------------------------------------------------------------
// C = A[M][K] . W[N][K]^T, bf16 MFMA 32x32x16 with fp32 accumulation, with
// 64-deep K tiles copied by LDS-DMA (buffer loads with a
// scalar base and constant per-lane offsets; rows past M read zeros) into two
// distinct LDS buffers, XOR-swizzled as the attention tiles (16 rows at one
// logical chunk hit 16 distinct slots of a 256-byte bank window): one barrier
// per K tile, the next tile lands while the current one is multiplied.
constexpr int LBK = 64;

template <int EPI, int TN>
__global__ __launch_bounds__(256, 2) void k_gemm_lds(GemmParams G) {
    // TN: output columns per workgroup (128, or 64 for narrow outputs: twice
    // the workgroups); each of the 4 waves computes 64 x TN/2
    constexpr int NJ = TN / 64;              // 32-column MFMA blocks per wave
    constexpr int TBA = GBM * LBK * 2, TBB = TN * LBK * 2;
    constexpr int MPA = TBA / 1024 / 4, MPB = TBB / 1024 / 4; // LDS-DMA instructions per wave
    constexpr int CPR = LBK * 2 / 16;        // 16-byte chunks per tile row
    __shared__ __attribute__((aligned(1024))) __bf16 sA0[GBM * LBK];
    __shared__ __attribute__((aligned(1024))) __bf16 sB0[TN * LBK];
    __shared__ __attribute__((aligned(1024))) __bf16 sA1[GBM * LBK];
    __shared__ __attribute__((aligned(1024))) __bf16 sB1[TN * LBK];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, half = lane >> 5;
    const int wm = w >> 1, wn = w & 1;
    const int n0 = blockIdx.x * TN;
    const int m0 = blockIdx.y * GBM;
    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(G.A + (long)m0 * G.lda, (uint32_t)((long)(G.M - m0) * G.lda * 2));
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(G.B + (long)n0 * G.K, (uint32_t)((long)TN * G.K * 2));
    uint32_t ao[MPA], bo[MPB];
#pragma unroll
    for (int i = 0; i < MPA; ++i) {
        const int off = (w * MPA + i) * 1024 + lane * 16;
        const int row = off / (LBK * 2), ch = ((off % (LBK * 2)) >> 4) ^ swz<CPR>(row);
        ao[i] = (uint32_t)(row * G.lda * 2 + ch * 16);
    }
#pragma unroll
    for (int i = 0; i < MPB; ++i) {
        const int off = (w * MPB + i) * 1024 + lane * 16;
        const int row = off / (LBK * 2), ch = ((off % (LBK * 2)) >> 4) ^ swz<CPR>(row);
        bo[i] = (uint32_t)(row * G.K * 2 + ch * 16);
    }
    auto issue = [&](int kt, __bf16* sA, __bf16* sB) {
        const uint32_t so = (uint32_t)kt * LBK * 2;
#pragma unroll
        for (int i = 0; i < MPA; ++i)
            buf_dma16(rA, reinterpret_cast<char*>(sA) + (w * MPA + i) * 1024, ao[i], so);
#pragma unroll
        for (int i = 0; i < MPB; ++i)
            buf_dma16(rB, reinterpret_cast<char*>(sB) + (w * MPB + i) * 1024, bo[i], so);
    };
    f32x16 acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
    auto compute = [&](const __bf16* sA, const __bf16* sB) {
#pragma unroll
        for (int ks = 0; ks < LBK / 16; ++ks) {
            bf16x8 a[2], bb[NJ];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + 32 * i + r;
                a[i] = *reinterpret_cast<const bf16x8*>(&sA[row * LBK + (((2 * ks + half) ^ swz<CPR>(row)) << 3)]);
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int row = wn * (TN / 2) + 32 * j + r;
                bb[j] = *reinterpret_cast<const bf16x8*>(&sB[row * LBK + (((2 * ks + half) ^ swz<CPR>(row)) << 3)]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32(a[i], bb[j], acc[i][j]);
        }
    };
    const int nk = G.K / LBK;
    issue(0, sA0, sB0);
    for (int kt = 0; kt < nk;) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 < nk) issue(kt + 1, sA1, sB1);
        compute(sA0, sB0);
        if (++kt >= nk) break;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 < nk) issue(kt + 1, sA0, sB0);
        compute(sA1, sB1);
        ++kt;
    }
    // acc[i][j][e]: row m0 + wm*64 + 32i + (e/4)*8 + half*4 + e%4,
    // col n0 + wn*TN/2 + 32j + r
    if (EPI == EPI_RESID) {
        // residual stream += C at the active rows: a block's 16 values are
        // all loaded before any is stored (stores through the same pointer
        // would otherwise order every later load behind them)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            long dst[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + wm * 64 + 32 * i + (e >> 2) * 8 + half * 4 + (e & 3);
                dst[e] = m < G.M ? (G.rows ? (long)G.rows[m] : (long)m) * G.ldc : -1;
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int n = n0 + wn * (TN / 2) + 32 * j + r;
                float cur[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) cur[e] = dst[e] >= 0 ? G.Cf[dst[e] + n] : 0.0f;
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (dst[e] >= 0) G.Cf[dst[e] + n] = cur[e] + acc[i][j][e];
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int n = n0 + wn * (TN / 2) + 32 * j + r;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + wm * 64 + 32 * i + (e >> 2) * 8 + half * 4 + (e & 3);
                const float v = acc[i][j][e];
                if (EPI == EPI_SWIGLU) {
                    const float u = __shfl_xor(v, 1); // (gate, up) column pair
                    if (m < G.M && (r & 1) == 0) {
                        const float sg = v / (1.0f + __expf(-v));
                        G.Cb[(long)m * G.ldc + (n >> 1)] = (__bf16)(sg * u);
                    }
                } else if (m < G.M) {
                    G.Cb[(long)m * G.ldc + n] = (__bf16)v;
                }
            }
        }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rope_split(const __bf16* __restrict__ qkv,
                                                    const int32_t* __restrict__ rows, int n, int H,
                                                    int d, float log2_theta, __bf16* __restrict__ q,
                                                    __bf16* __restrict__ k, __bf16* __restrict__ v) {
    const long gid = blockIdx.x * (long)blockDim.x + threadIdx.x;
    const int halfd = d / 2;
    const long per_row = (long)H * halfd;
    if (gid >= (long)n * per_row) return;
    const int m = (int)(gid / per_row);
    const int rem = (int)(gid % per_row);
    const int h = rem / halfd, i = rem % halfd;
    const float pos = (float)(rows ? rows[m] : m);
    // inverse frequency theta^(-2i/d), angle = pos * inv_freq (fp32)
    const float inv_freq = exp2f(-(float)(2 * i) / (float)d * log2_theta);
    float sn, cs;
    sincosf(pos * inv_freq, &sn, &cs);
    const long D = (long)H * d;
    const __bf16* src = qkv + (long)m * 3 * D + (long)h * d;
    const long o = ((long)m * H + h) * d;
#pragma unroll
    for (int part = 0; part < 2; ++part) { // q, k
        const float x1 = (float)src[part * D + i], x2 = (float)src[part * D + i + halfd];
        __bf16* dst = part ? k : q;
        dst[o + i] = (__bf16)(x1 * cs - x2 * sn);
        dst[o + i + halfd] = (__bf16)(x2 * cs + x1 * sn);
    }
    v[o + i] = src[2 * D + i];
    v[o + i + halfd] = src[2 * D + i + halfd];
}

__global__ void k_scatter_rows_bf16(const __bf16* __restrict__ src, const int32_t* __restrict__ rows,
                                    long n, int D, __bf16* __restrict__ dst) {
    const long gid = blockIdx.x * (long)blockDim.x + threadIdx.x;
    if (gid >= n * D) return;
    const long m = gid / D;
    const int c = (int)(gid % D);
    const long row = rows ? rows[m] : m;
    dst[row * D + c] = src[gid];
}

// ---------------------------------------------------------------------------
hipError_t launch_rmsnorm_gather(const float* x, const int32_t* rows, int n, int D,
                                 const __bf16* w, float eps, __bf16* out, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_rmsnorm_gather, dim3(n), dim3(256), 0, st, x, rows, D, w, eps, out);
    return hipGetLastError();
}

constexpr long kNarrowTiles = 1024; // 128-wide tiles per two workgroup slots (512 and 2048 measured no better)

// Output columns per workgroup: narrow outputs with few tiles take 64-wide
// tiles, twice the workgroups (2048-wide o / down projections of the
// 24-layer step: 9.7 -> 6.4 ms and 13.6 -> 12.5 ms); the rest 128.
int gemm_tile_n(const GemmParams& G) {
    const bool narrow = G.N <= 2048 && (long)(G.N / 128) * ((G.M + GBM - 1) / GBM) < kNarrowTiles;
    return narrow ? 64 : 128;
}

hipError_t launch_gemm(int epi, const GemmParams& G, hipStream_t st) {
    if (G.M <= 0) return hipSuccess;
    if (G.K % LBK != 0 || G.N % 128 != 0) return hipErrorInvalidValue; // checked by the caller
    const int tn = gemm_tile_n(G);
    const dim3 grid(G.N / tn, (G.M + GBM - 1) / GBM);
    if (tn == 64) {
        if (epi == EPI_STORE) hipLaunchKernelGGL((k_gemm_lds<EPI_STORE, 64>), grid, dim3(256), 0, st, G);
        else if (epi == EPI_RESID) hipLaunchKernelGGL((k_gemm_lds<EPI_RESID, 64>), grid, dim3(256), 0, st, G);
        else hipLaunchKernelGGL((k_gemm_lds<EPI_SWIGLU, 64>), grid, dim3(256), 0, st, G);
    } else {
        if (epi == EPI_STORE) hipLaunchKernelGGL((k_gemm_lds<EPI_STORE, 128>), grid, dim3(256), 0, st, G);
        else if (epi == EPI_RESID) hipLaunchKernelGGL((k_gemm_lds<EPI_RESID, 128>), grid, dim3(256), 0, st, G);
        else hipLaunchKernelGGL((k_gemm_lds<EPI_SWIGLU, 128>), grid, dim3(256), 0, st, G);
    }
    return hipGetLastError();
}

hipError_t launch_rope_split(const __bf16* qkv, const int32_t* rows, int n, int H, int d,
                             float theta, __bf16* q, __bf16* k, __bf16* v, hipStream_t st) {
    const long total = (long)n * H * (d / 2);
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_rope_split, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, qkv,
                       rows, n, H, d, log2f(theta), q, k, v);
    return hipGetLastError();
}

hipError_t launch_scatter_rows_bf16(const __bf16* src, const int32_t* rows, long n, int D,
                                    __bf16* dst, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_scatter_rows_bf16, dim3((unsigned)((n * D + 255) / 256)), dim3(256), 0, st,
                       src, rows, n, D, dst);
    return hipGetLastError();
}

} // namespace fl

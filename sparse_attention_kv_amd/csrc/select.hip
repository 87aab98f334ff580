// Token and column selection (FlashLoop paper, Sec. 4.1 and Sec. 4.2).
//
//  k_delta_norm  stat[t] = ||h_cur[i] - h_prev[i]||_2 for candidate i = cand[t]
//                (REL: divided by ||h_prev[i]||_2, the normalised change)
//                one wavefront per row; HBM-streaming (two rows of D values in,
//                one float out).
//  k_topk        exact top-n selection of one segment (the token set, or one
//                head's column candidates) by (key desc, position asc), written
//                in ascending position order.  One 1024-thread workgroup per
//                segment: a four-pass 8-bit MSB radix select finds the n-th
//                largest key T and how many keys equal to T are taken, then an
//                ordered block-scan compaction walks the candidates in position
//                order.  The result is unique given the keys, so it matches any
//                correct selector bit for bit.
//  k_topk_res    the same for segments of up to 32K candidates, held in
//                registers (contiguous runs of a multiple of 4 per thread,
//                read with 16-byte loads); 256-thread workgroups when many
//                segments of up to 8K candidates fill the GPU (the decode's
//                per-(sequence, head) column selections), 1024 otherwise.
#include "fl_device.h"
#include "fl_kernels.h"

#pragma clang fp contract(off)

namespace fl {

template <int kChunk, bool REL>
__global__ __launch_bounds__(256) void k_delta_norm(const void* __restrict__ h_cur,
                                                    const void* __restrict__ h_prev, int dtype,
                                                    int D, const int32_t* __restrict__ cand,
                                                    int n_cand, float* __restrict__ stat) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= n_cand) return;
    const long i = cand ? cand[t] : t;
    const long base = i * (long)D;
    float acc = 0.0f, pacc = 0.0f;
    int c = lane * 8;
    for (; c + 8 <= D; c += 64 * 8) {
        float a[8], b[8];
        load8_f32(h_cur, base + c, dtype, a);
        load8_f32(h_prev, base + c, dtype, b);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float df = a[e] - b[e];
            acc = acc + df * df;
            if (REL) pacc = pacc + b[e] * b[e];
        }
    }
    // tail (D not a multiple of 8 * lanes handled above)
    for (int cc = (D / 8) * 8 + lane; cc < D; cc += 64) {
        float a, b;
        if (dtype == FL_BF16) {
            a = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(h_cur)[base + cc]);
            b = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(h_prev)[base + cc]);
        } else {
            a = reinterpret_cast<const float*>(h_cur)[base + cc];
            b = reinterpret_cast<const float*>(h_prev)[base + cc];
        }
        const float df = a - b;
        acc = acc + df * df;
        if (REL) pacc = pacc + b * b;
    }
    acc = wave_sum(acc);
    if (REL) {
        pacc = wave_sum(pacc);
        const float dn = sqrtf(acc), pn = sqrtf(pacc);
        if (lane == 0) stat[t] = pn > 0.0f ? dn / pn : (dn > 0.0f ? __builtin_inff() : 0.0f);
    } else if (lane == 0) {
        stat[t] = sqrtf(acc);
    }
}

// Ordered key: larger float -> larger unsigned; -0 ranks as +0.
__device__ __forceinline__ uint32_t order_key(float f) {
    if (f == 0.0f) f = 0.0f;
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Exclusive block scan of v (0/1 or small counts) over the NW waves of the
// workgroup; returns the exclusive prefix and stores the block total in *total.
template <int NW = kSelWaves>
__device__ __forceinline__ int block_excl_scan(int v, int* s_wave, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) s_wave[w] = incl;
    __syncthreads();
    if (w == 0) {
        int x = lane < NW ? s_wave[lane] : 0;
        int xi = x;
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) {
            const int y = __shfl_up(xi, o);
            if (lane >= o) xi += y;
        }
        if (lane < NW) s_wave[NW + lane] = xi - x;
        if (lane == NW - 1) s_wave[2 * NW] = xi;
    }
    __syncthreads();
    const int r = s_wave[NW + w] + incl - v;
    *total = s_wave[2 * NW];
    __syncthreads();
    return r;
}

// One segment per workgroup.  Candidates t = 0..n-1 with keys key[t] and
// positions pos[t] (NULL: pos = t).  Candidates with position < n_prefix are
// not ranked: positions 0..n_prefix-1 are written first (the always-kept
// sinks, which the candidates must contain).  Then the n_sel ranked winners.
// slot (optional, [n_slot]): -1 everywhere, then slot[out[s]] = s.
__global__ __launch_bounds__(kSelThreads) void k_topk(
    const float* __restrict__ keys, long key_stride, const int32_t* __restrict__ pos,
    long pos_stride, int n, int n_sel, int n_prefix, int32_t* __restrict__ out,
    long out_stride, int32_t* __restrict__ slot, int n_slot) {
    __shared__ int s_hist[256];
    __shared__ int s_wave[2 * kSelWaves + 1];
    __shared__ uint32_t s_prefix;
    __shared__ int s_need;
    const int seg = blockIdx.x;
    keys += seg * key_stride;
    if (pos) pos += seg * pos_stride;
    out += seg * out_stride;
    const int tid = threadIdx.x;

    if (slot) {
        for (int i = tid; i < n_slot; i += kSelThreads) slot[i] = -1;
    }
    for (int s = tid; s < n_prefix; s += kSelThreads) {
        out[s] = s;
        if (slot && s < n_slot) slot[s] = s;
    }

    // ---- radix select of the n_sel-th largest ranked key ----
    uint32_t prefix = 0, pmask = 0;
    int need = n_sel;
    if (n_sel > 0) {
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            for (int b = tid; b < 256; b += kSelThreads) s_hist[b] = 0;
            if (tid == 0) { s_prefix = prefix; s_need = need; }
            __syncthreads();
            for (int t = tid; t < n; t += kSelThreads) {
                const int p = pos ? pos[t] : t;
                if (p < n_prefix) continue;
                const uint32_t u = order_key(keys[t]);
                if ((u & pmask) == prefix) atomicAdd(&s_hist[(u >> shift) & 255], 1);
            }
            __syncthreads();
            if (tid < 64) {
                // buckets 255..0 in descending order: lane L owns buckets
                // 255-4L .. 252-4L; suffix sums from the top.
                int c[4], lsum = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) { c[e] = s_hist[255 - 4 * tid - e]; lsum += c[e]; }
                int incl = lsum;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(incl, o);
                    if (tid >= o) incl += y;
                }
                int above = incl - lsum; // count in higher buckets
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (above < need && need <= above + c[e]) {
                        s_prefix = prefix | ((uint32_t)(255 - 4 * tid - e) << shift);
                        s_need = need - above;
                    }
                    above += c[e];
                }
            }
            __syncthreads();
            prefix = s_prefix;
            need = s_need;
            pmask |= 255u << shift;
            __syncthreads();
        }
    }
    const uint32_t T = prefix;
    __syncthreads();

    // ---- ordered compaction ----
    int out_base = n_prefix, eq_base = 0;
    for (int t0 = 0; t0 < n && n_sel > 0; t0 += kSelThreads) {
        const int t = t0 + tid;
        int p = -1, gt = 0, eq = 0;
        if (t < n) {
            p = pos ? pos[t] : t;
            if (p >= n_prefix) {
                const uint32_t u = order_key(keys[t]);
                gt = u > T;
                eq = u == T;
            }
        }
        int eq_tot;
        const int eq_rank = block_excl_scan(eq, s_wave, &eq_tot);
        const int take = gt || (eq && eq_base + eq_rank < need);
        int take_tot;
        const int at = block_excl_scan(take, s_wave, &take_tot);
        const int o = out_base + at;
        if (take && o < n_prefix + n_sel) {
            out[o] = p;
            if (slot && p >= 0 && p < n_slot) slot[p] = o;
        }
        out_base += take_tot;
        eq_base += eq_tot;
    }
}

// The same selection with every thread holding a contiguous run of at most
// kRes candidates in registers (segments of up to kRes * 1024 candidates):
// the radix passes read no memory, and the ordered compaction takes two
// block scans in all (tied keys before each run, then output offsets)
// instead of two per 1024 candidates.
constexpr int kRes = 32;

template <int NT>
__global__ __launch_bounds__(NT) void k_topk_res(
    const float* __restrict__ keys, long key_stride, const int32_t* __restrict__ pos,
    long pos_stride, int n, int n_sel, int n_prefix, int32_t* __restrict__ out,
    long out_stride, int32_t* __restrict__ slot, int n_slot) {
    __shared__ int s_hist[256];
    constexpr int NW = NT / 64;
    __shared__ int s_wave[2 * NW + 1];
    __shared__ uint32_t s_prefix;
    __shared__ int s_need;
    const int seg = blockIdx.x;
    keys += seg * key_stride;
    if (pos) pos += seg * pos_stride;
    out += seg * out_stride;
    const int tid = threadIdx.x;
    // runs of a multiple of 4 candidates (at most kRes), so that with
    // 16-byte aligned key / position arrays every run is read in 16-byte loads
    const int C = (((n + NT - 1) / NT) + 3) & ~3;
    const int t0 = min(tid * C, n), t1 = min(t0 + C, n);

    if (slot) {
        for (int i = tid; i < n_slot; i += NT) slot[i] = -1;
    }
    for (int q = tid; q < n_prefix; q += NT) {
        out[q] = q;
        if (slot && q < n_slot) slot[q] = q;
    }
    // this thread's run: ordered keys and positions; unranked entries
    // (sinks, padding) get rank flag 0
    uint32_t u[kRes];
    int pp[kRes];
    uint32_t ranked = 0;   // bit e: entry e takes part in the ranking
    const bool vec = ((reinterpret_cast<uintptr_t>(keys) | reinterpret_cast<uintptr_t>(pos)) & 15) == 0;
#pragma unroll
    for (int e4 = 0; e4 < kRes / 4; ++e4) {
        const int t = t0 + 4 * e4;
        float kv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        int pv[4] = {-1, -1, -1, -1};
        if (vec && t + 3 < t1) {
            const float4 k4 = *reinterpret_cast<const float4*>(keys + t);
            kv[0] = k4.x; kv[1] = k4.y; kv[2] = k4.z; kv[3] = k4.w;
            if (pos) {
                const int4 p4 = *reinterpret_cast<const int4*>(pos + t);
                pv[0] = p4.x; pv[1] = p4.y; pv[2] = p4.z; pv[3] = p4.w;
            } else {
                pv[0] = t; pv[1] = t + 1; pv[2] = t + 2; pv[3] = t + 3;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (t + i < t1) {
                    kv[i] = keys[t + i];
                    pv[i] = pos ? pos[t + i] : t + i;
                }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * e4 + i;
            u[e] = 0;
            pp[e] = -1;
            if (t + i < t1) {
                pp[e] = pv[i];
                if (pv[i] >= n_prefix) {
                    u[e] = order_key(kv[i]);
                    ranked |= 1u << e;
                }
            }
        }
    }

    // ---- radix select of the n_sel-th largest ranked key ----
    uint32_t prefix = 0, pmask = 0;
    int need = n_sel;
    if (n_sel > 0) {
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            for (int b = tid; b < 256; b += NT) s_hist[b] = 0;
            __syncthreads();
            // a run's keys mostly share their leading bytes: count equal
            // consecutive bins in a register and add each count once (the
            // LDS atomics on one bin from a whole wave serialise)
            int cur = -1, cnt = 0;
#pragma unroll
            for (int e = 0; e < kRes; ++e)
                if (((ranked >> e) & 1u) && (u[e] & pmask) == prefix) {
                    const int b = (u[e] >> shift) & 255;
                    if (b != cur) {
                        if (cnt) atomicAdd(&s_hist[cur], cnt);
                        cur = b;
                        cnt = 0;
                    }
                    ++cnt;
                }
            if (cnt) atomicAdd(&s_hist[cur], cnt);
            __syncthreads();
            if (tid < 64) {
                int c[4], lsum = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) { c[e] = s_hist[255 - 4 * tid - e]; lsum += c[e]; }
                int incl = lsum;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(incl, o);
                    if (tid >= o) incl += y;
                }
                int above = incl - lsum;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (above < need && need <= above + c[e]) {
                        s_prefix = prefix | ((uint32_t)(255 - 4 * tid - e) << shift);
                        s_need = need - above;
                    }
                    above += c[e];
                }
            }
            __syncthreads();
            prefix = s_prefix;
            need = s_need;
            pmask |= 255u << shift;
            __syncthreads();
        }
    }
    if (n_sel <= 0) return;
    const uint32_t T = prefix;

    // ---- ordered compaction: runs are in position order ----
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int e = 0; e < kRes; ++e) {
        const bool r = (ranked >> e) & 1u;
        n_gt += r && u[e] > T;
        n_eq += r && u[e] == T;
    }
    int eq_tot;
    const int eq_before = block_excl_scan<NW>(n_eq, s_wave, &eq_tot);
    const int eq_take = min(max(need - eq_before, 0), n_eq);  // this run's first eq_take ties
    int take_tot;
    int o = n_prefix + block_excl_scan<NW>(n_gt + eq_take, s_wave, &take_tot);
    int eq_seen = 0;
#pragma unroll
    for (int e = 0; e < kRes; ++e) {
        const bool r = (ranked >> e) & 1u;
        const bool eq = r && u[e] == T;
        const bool take = r && (u[e] > T || (eq && eq_seen < eq_take));
        eq_seen += eq;
        if (take && o < n_prefix + n_sel) { // (the bound holds for finite keys)
            out[o] = pp[e];
            if (slot && pp[e] < n_slot) slot[pp[e]] = o;
        }
        o += take;
    }
}

__global__ void k_copy_or_iota(const int32_t* __restrict__ src, int32_t* __restrict__ dst, long n,
                               long row) {
    const long i = blockIdx.x * (long)blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : (int32_t)(i % row);
}

// ---- launchers ----
hipError_t launch_delta_norm(const void* h_cur, const void* h_prev, int dtype, int D,
                             const int32_t* cand, int n_cand, bool relative, float* stat,
                             hipStream_t st) {
    const int blocks = (n_cand + 3) / 4;
    if (relative)
        hipLaunchKernelGGL((k_delta_norm<8, true>), dim3(blocks), dim3(256), 0, st, h_cur, h_prev,
                           dtype, D, cand, n_cand, stat);
    else
        hipLaunchKernelGGL((k_delta_norm<8, false>), dim3(blocks), dim3(256), 0, st, h_cur, h_prev,
                           dtype, D, cand, n_cand, stat);
    return hipGetLastError();
}

hipError_t launch_topk(const float* keys, long key_stride, const int32_t* pos, long pos_stride,
                       int n, int n_sel, int n_prefix, int32_t* out, long out_stride,
                       int32_t* slot, int n_slot, int n_seg, hipStream_t st) {
    if (n <= kRes * 256 && n_seg >= 256)
        hipLaunchKernelGGL(k_topk_res<256>, dim3(n_seg), dim3(256), 0, st, keys, key_stride, pos,
                           pos_stride, n, n_sel, n_prefix, out, out_stride, slot, n_slot);
    else if (n <= kRes * kSelThreads)
        hipLaunchKernelGGL(k_topk_res<kSelThreads>, dim3(n_seg), dim3(kSelThreads), 0, st, keys, key_stride, pos,
                           pos_stride, n, n_sel, n_prefix, out, out_stride, slot, n_slot);
    else
        hipLaunchKernelGGL(k_topk, dim3(n_seg), dim3(kSelThreads), 0, st, keys, key_stride, pos,
                           pos_stride, n, n_sel, n_prefix, out, out_stride, slot, n_slot);
    return hipGetLastError();
}

hipError_t launch_copy_or_iota(const int32_t* src, int32_t* dst, long n, long row,
                               hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_copy_or_iota, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src,
                       dst, n, row);
    return hipGetLastError();
}

} // namespace fl

// Bandwidth- and latency-bound kernels of the AuraFlow forward on gfx950:
// timestep features, GEMV (timestep MLP and every block's adaLN modulation at
// once), patch embedding with the centre-cropped position table, register
// tokens, key-padding bias, fused fp32 LayerNorm + shift/scale modulation,
// pre-final modulation fused with the output projection and unpatchify, the
// Euler + CFG update, weight packing and fp32-path helpers.
//
// Page tags: [PIPE], [TRANS], [DEEP] as listed in include/auraflow.h.
#include <algorithm>

#include "af_internal.h"

namespace af {

// ============================================================================ timestep features
// [TRANS] 前向传播流程 (Timesteps, 256 channels): u = timestep_scale * tau;
// e = [cos(u f_k) (k < half), sin(u f_k)], f_k = 10000^(-k/half). Computed in
// double so the features carry no fp32 argument-rounding error (u reaches 1000 rad).
__global__ void k_timestep_features(const float* __restrict__ tau, int B, int half, double tscale,
                                    float* __restrict__ e) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= B * half) return;
    int b = i / half, k = i % half;
    double u = tscale * (double)tau[b];
    double f = exp(-log(10000.0) * (double)k / (double)half);
    double a = u * f;
    e[b * 2 * half + k] = (float)cos(a);
    e[b * 2 * half + half + k] = (float)sin(a);
}

hipError_t timestep_features(const float* tau, int B, int half, float tscale, float* e, hipStream_t s) {
    int n = B * half;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_timestep_features, dim3((n + 255) / 256), dim3(256), 0, s, tau, B, half,
                       (double)tscale, e);
    return hipGetLastError();
}

// ============================================================================ GEMV
// y[b, n] = sum_k W[n, k] act(x[b, k]) + bias[n]. One wave per output row
// (grid-stride), each lane owning fixed 16-byte chunks of k so the activation
// values stay in registers across rows. Batches go in passes of BC.
template <typename WT> struct WChunk;
template <> struct WChunk<bf16_t> {
    static constexpr int E = 8;
    __device__ static void load(const bf16_t* p, float* o) {
        uint4 v = *reinterpret_cast<const uint4*>(p);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
    __device__ static float one(const bf16_t* p) { return bf2f(*p); }
};
template <> struct WChunk<float> {
    static constexpr int E = 4;
    __device__ static void load(const float* p, float* o) {
        float4 v = *reinterpret_cast<const float4*>(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    __device__ static float one(const float* p) { return *p; }
};

template <typename WT, int BC, int MAXI>
__global__ __launch_bounds__(256) void k_gemv(const float* __restrict__ x, int B, int K,
                                              const WT* __restrict__ W, int N,
                                              const WT* __restrict__ bias, int silu_in,
                                              float* __restrict__ y, int b0) {
    constexpr int E = WChunk<WT>::E;
    const int lane = threadIdx.x & 63;
    const int nb = min(BC, B - b0);
    float xr[MAXI][BC][E];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        int k0 = (lane + 64 * i) * E;
#pragma unroll
        for (int b = 0; b < BC; ++b)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float v = 0.f;
                if (b < nb && k0 + e < K) {
                    v = x[(long)(b0 + b) * K + k0 + e];
                    if (silu_in) v = silu_f(v);
                }
                xr[i][b][e] = v;
            }
    }
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int nwaves = (gridDim.x * blockDim.x) >> 6;
    for (int n = wave; n < N; n += nwaves) {
        const WT* row = W + (long)n * K;
        float acc[BC];
#pragma unroll
        for (int b = 0; b < BC; ++b) acc[b] = 0.f;
#pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            int k0 = (lane + 64 * i) * E;
            if (k0 < K) {
                float w[E];
                WChunk<WT>::load(row + k0, w);
#pragma unroll
                for (int b = 0; b < BC; ++b)
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[b] += w[e] * xr[i][b][e];
            }
        }
#pragma unroll
        for (int b = 0; b < BC; ++b) acc[b] = wave_sum(acc[b]);
        if (lane == 0) {
            float bb = bias ? WChunk<WT>::one(bias + n) : 0.f;
            for (int b = 0; b < nb; ++b) y[(long)(b0 + b) * N + n] = acc[b] + bb;
        }
    }
}

// bf16 weights: each wave takes R rows at a time (all R x NI 16-byte weight
// chunks of a lane requested before any arithmetic), so a wave keeps R rows of
// weights in flight while the input vectors stay in registers.
template <int BC, int NI, int R>
__global__ __launch_bounds__(256) void k_gemv_bf16(const float* __restrict__ x, int B, int K,
                                                   const bf16_t* __restrict__ W, int N,
                                                   const bf16_t* __restrict__ bias, int silu_in,
                                                   float* __restrict__ y, int b0) {
    const int lane = threadIdx.x & 63;
    const int nb = min(BC, B - b0);
    float xr[NI][BC][8];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int k0 = (lane + 64 * i) * 8;
#pragma unroll
        for (int b = 0; b < BC; ++b)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = 0.f;
                if (b < nb && k0 + e < K) {
                    v = x[(long)(b0 + b) * K + k0 + e];
                    if (silu_in) v = silu_f(v);
                }
                xr[i][b][e] = v;
            }
    }
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int nwaves = (gridDim.x * blockDim.x) >> 6;
    for (int n0 = wave * R; n0 < N; n0 += nwaves * R) {
        uint4 w[R][NI];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int k0 = (lane + 64 * i) * 8;
                w[r][i] = (n0 + r < N && k0 < K) ? *reinterpret_cast<const uint4*>(W + (long)(n0 + r) * K + k0)
                                                 : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float acc[BC];
#pragma unroll
            for (int b = 0; b < BC; ++b) acc[b] = 0.f;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const uint32_t u[4] = {w[r][i].x, w[r][i].y, w[r][i].z, w[r][i].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float lo = __uint_as_float(u[q] << 16), hi = __uint_as_float(u[q] & 0xFFFF0000u);
#pragma unroll
                    for (int b = 0; b < BC; ++b) acc[b] += lo * xr[i][b][2 * q] + hi * xr[i][b][2 * q + 1];
                }
            }
#pragma unroll
            for (int b = 0; b < BC; ++b) acc[b] = wave_sum(acc[b]);
            const int n = n0 + r;
            if (lane == 0 && n < N) {
                const float bb = bias ? bf2f(bias[n]) : 0.f;
                for (int b = 0; b < nb; ++b) y[(long)(b0 + b) * N + n] = acc[b] + bb;
            }
        }
    }
}

// bf16 weights, K = 512 NI (the modulation GEMV streams 4.6 GB of them
// once per forward): the input vectors sit in LDS instead of registers, so a wave
// holds only its R x NI weight chunks and six waves fit a SIMD; the weights are
// read with non-temporal loads, as they are used once. Lane l's chunk i covers
// k = 512 i + 8 l .. + 7, stored as two float4 at 512 i + 256 h + 4 l (h the
// half), so each of a wave's 16-byte LDS reads is one contiguous 1 KB row.
// Same summation order as k_gemv_bf16: results are bit-identical.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int BC, int NI, int R, int NT = 256>
__global__ __launch_bounds__(NT) void k_gemv_bf16_lds(const float* __restrict__ x, int B, int K,
                                                       const bf16_t* __restrict__ W, int N,
                                                       const bf16_t* __restrict__ bias, int silu_in,
                                                       float* __restrict__ y, int b0) {
    __shared__ float4 sx[BC][NI * 128];
    const int lane = threadIdx.x & 63;
    const int nb = min(BC, B - b0);
    for (int idx = threadIdx.x; idx < BC * NI * 128; idx += blockDim.x) {
        const int b = idx / (NI * 128), q = idx % (NI * 128);
        const int k = 512 * (q / 128) + 8 * (q & 63) + 4 * ((q / 64) & 1);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (b < nb) {
            v = *reinterpret_cast<const float4*>(x + (long)(b0 + b) * K + k);
            if (silu_in) v = make_float4(silu_f(v.x), silu_f(v.y), silu_f(v.z), silu_f(v.w));
        }
        sx[b][q] = v;
    }
    __syncthreads();
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int nwaves = (gridDim.x * blockDim.x) >> 6;
    for (int n0 = wave * R; n0 < N; n0 += nwaves * R) {
        asm volatile("" ::: "memory");   // keeps the LDS reads of x in the loop (not hoisted into registers)
        uint4 w[R][NI];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bf16_t* row = W + (long)min(n0 + r, N - 1) * K + 8 * lane;   // rows past N: read, unused
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + 512 * i));
                w[r][i] = make_uint4(t.x, t.y, t.z, t.w);
            }
        }
        float acc[R][BC];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < BC; ++b) acc[r][b] = 0.f;
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int b = 0; b < BC; ++b) {
                const float4 x0 = sx[b][128 * i + lane], x1 = sx[b][128 * i + 64 + lane];
                const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t u[4] = {w[r][i].x, w[r][i].y, w[r][i].z, w[r][i].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[r][b] += __uint_as_float(u[q] << 16) * xv[2 * q] +
                                     __uint_as_float(u[q] & 0xFFFF0000u) * xv[2 * q + 1];
                }
            }
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int b = 0; b < BC; ++b) acc[r][b] = wave_sum(acc[r][b]);
            const int n = n0 + r;
            if (lane == 0 && n < N) {
                const float bb = bias ? bf2f(bias[n]) : 0.f;
                for (int b = 0; b < nb; ++b) y[(long)(b0 + b) * N + n] = acc[r][b] + bb;
            }
        }
    }
}

hipError_t gemv(const float* x, int B, int K, const void* W, af_dtype wdt, int N, const void* bias,
                int silu_in, float* y, hipStream_t s) {
    if (B == 0 || N == 0) return hipSuccess;
    constexpr int BC = 2;
    if (K > 4096) return hipErrorInvalidValue;
    // K = 3072 with more than two samples: eight samples per pass over the
    // weights (96 KB of inputs in LDS, one 512-thread workgroup per CU), so a
    // batch of 8 streams the weights once. Each (row, sample) dot product is
    // summed in the same order as in the two-sample instance: bit-identical.
    if (wdt == AF_BF16 && K == 3072 && B > 2) {
        constexpr int BC8 = 8, R = 4, NT = 512;
        for (int b0 = 0; b0 < B; b0 += BC8) {
            hipLaunchKernelGGL((k_gemv_bf16_lds<BC8, 6, R, NT>), dim3(min((N + 8 * R - 1) / (8 * R), 2048)), dim3(NT),
                               0, s, x, B, K, (const bf16_t*)W, N, (const bf16_t*)bias, silu_in, y, b0);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    for (int b0 = 0; b0 < B; b0 += BC) {
        if (wdt == AF_BF16) {
            const int ni = (K + 511) / 512;
            const bf16_t* Wb = (const bf16_t*)W;
            const bf16_t* bb = (const bf16_t*)bias;
#define AF_GEMV(NI, R)                                                                                       \
    hipLaunchKernelGGL((k_gemv_bf16<BC, NI, R>), dim3(min((N + 4 * R - 1) / (4 * R), 2048)), dim3(256), 0, s, x, \
                       B, K, Wb, N, bb, silu_in, y, b0)
#define AF_GEMV_LDS(NI, R)                                                                                        \
    hipLaunchKernelGGL((k_gemv_bf16_lds<BC, NI, R>), dim3(min((N + 4 * R - 1) / (4 * R), 4096)), dim3(256), 0, s, \
                       x, B, K, Wb, N, bb, silu_in, y, b0)
            if (K == 3072) AF_GEMV_LDS(6, 4);   // the pages' width (the instance the parity tests run)
            else if (ni <= 1) AF_GEMV(1, 4);
            else if (ni <= 2) AF_GEMV(2, 4);
            else if (ni <= 4) AF_GEMV(4, 4);
            else if (ni <= 6) AF_GEMV(6, 4);
            else AF_GEMV(8, 2);
#undef AF_GEMV
#undef AF_GEMV_LDS
        } else {
            int blocks = (N + 3) / 4;
            if (blocks > 4096) blocks = 4096;
            hipLaunchKernelGGL((k_gemv<float, BC, 16>), dim3(blocks), dim3(256), 0, s, x, B, K,
                               (const float*)W, N, (const float*)bias, silu_in, y, b0);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ============================================================================ patch embed
// [PIPE] 深入源码 (Patch Embed) / [TRANS] 核心子模块架构 (Patch Embedding): the
// latent is cut into p x p patches (feature order channel, row-in-patch,
// column-in-patch), projected by a Linear with bias, and the learned position
// row of the centre crop of the G x G table is added. Token t = i*w + j lands in
// residual row (b, Nt + t). One thread per output column; the patch vectors
// of a run of tokens are staged in LDS.
constexpr int PE_ROWS = 64;
constexpr int PE_MAXF = 64;

template <typename WT>
__global__ __launch_bounds__(256) void k_patch_embed(const float* __restrict__ lat, int C, int H, int W,
                                                     int p, const WT* __restrict__ pe_w,
                                                     const WT* __restrict__ pe_b,
                                                     const float* __restrict__ pos, int G,
                                                     float* __restrict__ resid, RowGeom g, int d) {
    __shared__ float sp[PE_ROWS][PE_MAXF];
    const int Pd = C * p * p;
    const int h = H / p, w = W / p;
    const int ntok = h * w;
    const int b = blockIdx.z;
    const int t0 = blockIdx.y * PE_ROWS;
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    // every one of the PE_MAXF columns is written (zero past Pd): the dot product
    // below runs over all of them, and 0 times a stale non-finite LDS word is NaN
    for (int i = threadIdx.x; i < PE_ROWS * PE_MAXF; i += blockDim.x) {
        int r = i / PE_MAXF, f = i % PE_MAXF;
        int t = t0 + r;
        float v = 0.f;
        if (t < ntok && f < Pd) {
            int ti = t / w, tj = t % w;
            int ch = f / (p * p), py = (f / p) % p, px = f % p;
            v = lat[(((long)b * C + ch) * H + ti * p + py) * W + tj * p + px];
        }
        sp[r][f] = v;
    }
    __syncthreads();
    if (c >= d) return;
    float wr[PE_MAXF];
#pragma unroll
    for (int f = 0; f < PE_MAXF; ++f) wr[f] = f < Pd ? WChunk<WT>::one(pe_w + (long)c * Pd + f) : 0.f;
    const float bc = WChunk<WT>::one(pe_b + c);
    const int r0 = (G - h) / 2, c0 = (G - w) / 2;
    for (int r = 0; r < PE_ROWS; ++r) {
        int t = t0 + r;
        if (t >= ntok) break;
        float acc = bc;
#pragma unroll
        for (int f = 0; f < PE_MAXF; ++f) acc += wr[f] * sp[r][f];
        int ti = t / w, tj = t % w;
        long pidx = (long)(r0 + ti) * G + (c0 + tj);
        acc += pos[pidx * d + c];
        resid[(long)g.row_of(b, g.Nt + t) * d + c] = acc;
    }
}

hipError_t patch_embed(const float* lat, int C, int H, int W, int p, const void* pe_w, const void* pe_b,
                       af_dtype wdt, const float* pos, int G, float* resid, RowGeom g, int d,
                       hipStream_t s) {
    int ntok = (H / p) * (W / p);
    if (g.B == 0 || ntok == 0) return hipSuccess;
    dim3 grid((d + 255) / 256, (ntok + PE_ROWS - 1) / PE_ROWS, g.B);
    if (wdt == AF_BF16)
        hipLaunchKernelGGL(k_patch_embed<bf16_t>, grid, dim3(256), 0, s, lat, C, H, W, p,
                           (const bf16_t*)pe_w, (const bf16_t*)pe_b, pos, G, resid, g, d);
    else
        hipLaunchKernelGGL(k_patch_embed<float>, grid, dim3(256), 0, s, lat, C, H, W, p,
                           (const float*)pe_w, (const float*)pe_b, pos, G, resid, g, d);
    return hipGetLastError();
}

// ============================================================================ register tokens
// [TRANS] 核心子模块架构 (Register Tokens): R learned tokens at the head of the text sequence.
template <typename WT>
__global__ void k_registers(const WT* __restrict__ reg, int R, float* __restrict__ resid, RowGeom g, int d) {
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    long n = (long)g.B * R * d;
    if (i >= n) return;
    int c = i % d;
    int r = (i / d) % R;
    int b = i / ((long)R * d);
    resid[(long)g.row_of(b, r) * d + c] = WChunk<WT>::one(reg + (long)r * d + c);
}

hipError_t copy_registers(const void* reg, af_dtype wdt, int R, float* resid, RowGeom g, int d,
                          hipStream_t s) {
    long n = (long)g.B * R * d;
    if (n == 0) return hipSuccess;
    dim3 grid((unsigned)((n + 255) / 256));
    if (wdt == AF_BF16)
        hipLaunchKernelGGL(k_registers<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)reg, R, resid, g, d);
    else
        hipLaunchKernelGGL(k_registers<float>, grid, dim3(256), 0, s, (const float*)reg, R, resid, g, d);
    return hipGetLastError();
}

// ============================================================================ fp32 -> bf16 (text)
__global__ void k_f32_to_bf16(const float* __restrict__ src, bf16_t* __restrict__ dst, long n) {
    long i = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i + 3 < n) {
        float4 v = *reinterpret_cast<const float4*>(src + i);
        uint2 o = {pack2bf(v.x, v.y), pack2bf(v.z, v.w)};
        *reinterpret_cast<uint2*>(dst + i) = o;
    } else {
        for (; i < n; ++i) dst[i] = f2bf(src[i]);
    }
}

hipError_t f32_to_bf16(const float* src, bf16_t* dst, long n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    long threads = (n + 3) / 4;
    hipLaunchKernelGGL(k_f32_to_bf16, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

// ============================================================================ key-padding bias
// Sequence position s of sample b: registers [0, R) always valid, text [R, Nt)
// valid where mask[b, s - R] != 0, image [Nt, S) always valid, padding
// [S, S_pad) never valid. Valid -> 0, excluded -> -inf.
__global__ void k_key_bias(const uint8_t* __restrict__ mask, int T, int R, RowGeom g, int S_pad, float keep,
                           float* __restrict__ bias) {
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)g.B * S_pad) return;
    int b = i / S_pad, s = i % S_pad;
    bool valid;
    if (s >= g.S()) valid = false;
    else if (s >= R && s < g.Nt) valid = mask == nullptr || mask[(long)b * T + (s - R)] != 0;
    else valid = true;
    bias[i] = valid ? keep : -INFINITY;
}

hipError_t key_bias(const uint8_t* mask, int T, int R, RowGeom g, int S_pad, float keep, float* bias,
                    hipStream_t s) {
    long n = (long)g.B * S_pad;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_key_bias, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, mask, T, R, g,
                       S_pad, keep, bias);
    return hipGetLastError();
}

// ============================================================================ LayerNorm + modulate
// [TRANS] 核心子模块架构 (调制与归一化): FP32 LayerNorm (no affine, biased
// variance, eps) followed by x (1 + scale) + shift with the block's adaLN
// vectors. One wave per row, the row held in registers (d <= 4096), two-pass
// mean / variance.
template <typename OT> __device__ __forceinline__ void store4(OT* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
    uint2 o = {pack2bf(a, b), pack2bf(c, d)};
    *reinterpret_cast<uint2*>(p) = o;
}
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// EXACT: d == 256 MAXV, every lane's MAXV chunks are in the row and the loops carry
// no per-chunk condition (with one, each chunk's shift/scale loads and store sat in
// a branch of its own behind a full wait: twelve serial L2 round trips per row).
template <typename OT, int MAXV, bool EXACT = false>   // MAXV float4 per lane: d <= 256 MAXV
__global__ __launch_bounds__(256) void k_ln_modulate(const float* __restrict__ x, int M, int d, RowGeom g,
                                                     int split, const float* __restrict__ mod,
                                                     long mod_stride, int sh_a, int sc_a, int sh_b,
                                                     int sc_b, OT* __restrict__ out, float eps) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const int nv = EXACT ? 64 * MAXV : d / 4;
    const float* xr = x + (long)row * d;
    float4 v[MAXV];
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int c4 = lane + 64 * i;
        v[i] = c4 < nv ? reinterpret_cast<const float4*>(xr)[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    const float mean = wave_sum(sum) / (float)d;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int c4 = lane + 64 * i;
        if (c4 < nv) {
            float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, e = v[i].w - mean;
            sq += (a * a + b * b) + (c * c + e * e);
        }
    }
    const float rstd = rsqrtf(wave_sum(sq) / (float)d + eps);
    const int bidx = g.batch_of(row);
    const bool first = row < split;
    const float* shp = mod + (long)bidx * mod_stride + (first ? sh_a : sh_b);
    const float* scp = mod + (long)bidx * mod_stride + (first ? sc_a : sc_b);
    OT* orow = out + (long)row * d;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int c4 = lane + 64 * i;
        if (c4 < nv) {
            const float4 sh = reinterpret_cast<const float4*>(shp)[c4];
            const float4 sc = reinterpret_cast<const float4*>(scp)[c4];
            store4<OT>(orow + 4 * c4, (v[i].x - mean) * rstd * (1.f + sc.x) + sh.x,
                       (v[i].y - mean) * rstd * (1.f + sc.y) + sh.y,
                       (v[i].z - mean) * rstd * (1.f + sc.z) + sh.z,
                       (v[i].w - mean) * rstd * (1.f + sc.w) + sh.w);
        }
    }
}

template <typename OT>
static void launch_ln_modulate(int per_lane, dim3 grid, hipStream_t s, const float* x, int M, int d, RowGeom g,
                               int split, const float* mod, long mod_stride, int sh_a, int sc_a, int sh_b, int sc_b,
                               OT* out, float eps) {
    if (d == 256 * 12) {   // the pages' width, 3072
        hipLaunchKernelGGL((k_ln_modulate<OT, 12, true>), grid, dim3(256), 0, s, x, M, d, g, split, mod, mod_stride,
                           sh_a, sc_a, sh_b, sc_b, out, eps);
        return;
    }
#define AF_LNM(V) hipLaunchKernelGGL((k_ln_modulate<OT, V>), grid, dim3(256), 0, s, x, M, d, g, split, mod, \
                                     mod_stride, sh_a, sc_a, sh_b, sc_b, out, eps)
    if (per_lane <= 1) AF_LNM(1);
    else if (per_lane <= 2) AF_LNM(2);
    else if (per_lane <= 4) AF_LNM(4);
    else if (per_lane <= 8) AF_LNM(8);
    else if (per_lane <= 12) AF_LNM(12);
    else AF_LNM(16);
#undef AF_LNM
}

hipError_t ln_modulate(const float* x, int M, int d, RowGeom g, int split, const float* mod, long mod_stride,
                       int sh_a, int sc_a, int sh_b, int sc_b, void* out, af_dtype odt, float eps,
                       hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (d % 4 != 0 || d > 4096) return hipErrorInvalidValue;
    const int per_lane = (d / 4 + 63) / 64;
    dim3 grid((M + 3) / 4);
    if (odt == AF_BF16)
        launch_ln_modulate<bf16_t>(per_lane, grid, s, x, M, d, g, split, mod, mod_stride, sh_a, sc_a, sh_b, sc_b,
                                   (bf16_t*)out, eps);
    else
        launch_ln_modulate<float>(per_lane, grid, s, x, M, d, g, split, mod, mod_stride, sh_a, sc_a, sh_b, sc_b,
                                  (float*)out, eps);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- MXFP8 output
// The same LayerNorm + modulate with an MXFP8 output for the MXFP8 GEMMs: each
// 32 consecutive values of a row share the scale 2^e, e = floor(log2(max |y|)) - 8
// (at least -127), and are stored as E4M3 bytes of y / 2^e (clamped to +-448,
// rounded to nearest even); scale bytes e + 127 in the [d/64][sc_rows][2] layout.
// Lane l holds columns 4 (l + 64 i) .. + 3, so one 32-value block is the 8 lanes
// 8q .. 8q + 7 of one i.
// EXACT: d == 256 MAXV, the per-chunk conditions vanish (as in k_ln_modulate).
template <int MAXV, bool EXACT = false>
__global__ __launch_bounds__(256) void k_ln_modulate_mx(const float* __restrict__ x, int M, int d, RowGeom g,
                                                        int split, const float* __restrict__ mod, long mod_stride,
                                                        int sh_a, int sc_a, int sh_b, int sc_b,
                                                        uint8_t* __restrict__ out, uint8_t* __restrict__ sc,
                                                        long sc_rows, float eps) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const int nv = EXACT ? 64 * MAXV : d / 4;
    const float* xr = x + (long)row * d;
    float4 v[MAXV];
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int c4 = lane + 64 * i;
        v[i] = c4 < nv ? reinterpret_cast<const float4*>(xr)[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    const float mean = wave_sum(sum) / (float)d;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int c4 = lane + 64 * i;
        if (c4 < nv) {
            float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, e = v[i].w - mean;
            sq += (a * a + b * b) + (c * c + e * e);
        }
    }
    const float rstd = rsqrtf(wave_sum(sq) / (float)d + eps);
    const int bidx = g.batch_of(row);
    const bool first = row < split;
    const float* shp = mod + (long)bidx * mod_stride + (first ? sh_a : sh_b);
    const float* scp = mod + (long)bidx * mod_stride + (first ? sc_a : sc_b);
    uint8_t* orow = out + (long)row * d;
    // every shift/scale load first, then y in place of v: the loads of all chunks
    // are in flight together (the scale-byte stores below are a divergent branch
    // per chunk, which loads inside the chunk loop could not be moved across)
    float4 shv[MAXV], scv[MAXV];
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int c4 = lane + 64 * i;
        if (i * 64 < nv) {                   // uniform: d is a multiple of 256
            shv[i] = reinterpret_cast<const float4*>(shp)[c4];
            scv[i] = reinterpret_cast<const float4*>(scp)[c4];
        }
    }
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        if (i * 64 < nv) {
            v[i].x = (v[i].x - mean) * rstd * (1.f + scv[i].x) + shv[i].x;
            v[i].y = (v[i].y - mean) * rstd * (1.f + scv[i].y) + shv[i].y;
            v[i].z = (v[i].z - mean) * rstd * (1.f + scv[i].z) + shv[i].z;
            v[i].w = (v[i].w - mean) * rstd * (1.f + scv[i].w) + shv[i].w;
        }
    }
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int c4 = lane + 64 * i;
        if (i * 64 < nv) {
            const float y0 = v[i].x, y1 = v[i].y, y2 = v[i].z, y3 = v[i].w;
            float amax = fmaxf(fmaxf(fabsf(y0), fabsf(y1)), fmaxf(fabsf(y2), fabsf(y3)));
            amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
            amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
            amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
            const int e = mx_scale_exp(amax);
            const float inv = pow2f(-e);
            *reinterpret_cast<uint32_t*>(orow + 4 * c4) = pack4_e4m3(y0 * inv, y1 * inv, y2 * inv, y3 * inv);
            if ((lane & 7) == 0) {
                const int blk = c4 >> 3;
                sc[((long)(blk >> 1) * sc_rows + row) * 2 + (blk & 1)] = (uint8_t)(e + 127);
            }
        }
    }
}

hipError_t ln_modulate_mx(const float* x, int M, int d, RowGeom g, int split, const float* mod, long mod_stride,
                          int sh_a, int sc_a, int sh_b, int sc_b, uint8_t* out, uint8_t* sc, long sc_rows, float eps,
                          hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (d % 256 != 0 || d > 4096) return hipErrorInvalidValue;
    dim3 grid((M + 3) / 4);
#define AF_LNMX(V) hipLaunchKernelGGL((k_ln_modulate_mx<V>), grid, dim3(256), 0, s, x, M, d, g, split, mod, mod_stride, \
                                      sh_a, sc_a, sh_b, sc_b, out, sc, sc_rows, eps)
    const int per_lane = d / 256;
    if (d == 256 * 12) {   // the pages' width, 3072
        hipLaunchKernelGGL((k_ln_modulate_mx<12, true>), grid, dim3(256), 0, s, x, M, d, g, split, mod, mod_stride,
                           sh_a, sc_a, sh_b, sc_b, out, sc, sc_rows, eps);
        return hipGetLastError();
    }
    if (per_lane <= 4) AF_LNMX(4);
    else if (per_lane <= 8) AF_LNMX(8);
    else if (per_lane <= 12) AF_LNMX(12);
    else AF_LNMX(16);
#undef AF_LNMX
    return hipGetLastError();
}

// ============================================================================ pre-final + proj_out + unpatchify
// [TRANS] 核心子模块架构 (调制与归一化) and 前向传播流程: y = x (1 + scale) + shift
// on the image rows (modulation only), z = y W_out^T (no bias), and z's
// features (row-in-patch, column-in-patch, channel) scattered back to
// [B, C_out, H, W]. fp32 arithmetic.
//
// bf16 weights: one workgroup of 8 waves per CU stages W_out (p^2 C_out <= 16 rows of
// d <= 4096; 96 KB at d = 3072) in LDS once; each wave then takes image tokens in turn, holds the
// modulated row in registers, accumulates all p^2 C_out dot products from 8-byte
// LDS reads of W_out and reduces them across the wave independently of each other.
constexpr int PF_MAXV = 16;
constexpr int PF_MAXO = 16;
constexpr int PF_LDS = 16 * 4096;   // bf16 elements of W_out the LDS stage holds (128 KB)

template <int NV4>   // d = 256 NV4: every lane holds NV4 float4 of a row, no partial chunks
__global__ __launch_bounds__(512) void k_prefinal_project_bf16(const float* __restrict__ resid, RowGeom g, int d,
                                                               const float* __restrict__ mod, long mod_stride,
                                                               int sc_off, int sh_off,
                                                               const bf16_t* __restrict__ Wout, int Cout, int p,
                                                               int h, int w, float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) bf16_t sW[PF_LDS];
    const int Pout = p * p * Cout;
    for (int e = threadIdx.x * 8; e < Pout * d; e += blockDim.x * 8)
        *reinterpret_cast<uint4*>(sW + e) = *reinterpret_cast<const uint4*>(Wout + e);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int nwaves = (gridDim.x * blockDim.x) >> 6;
    const int ntok = g.B * g.Ni;
    const int H = h * p, W = w * p;
    for (int t = wave; t < ntok; t += nwaves) {
        const int b = t / g.Ni, tok = t % g.Ni;
        const float4* xr = reinterpret_cast<const float4*>(resid + (long)(g.B * g.Nt + t) * d);
        const float4* sc = reinterpret_cast<const float4*>(mod + (long)b * mod_stride + sc_off);
        const float4* sh = reinterpret_cast<const float4*>(mod + (long)b * mod_stride + sh_off);
        float4 y[NV4];
#pragma unroll
        for (int i = 0; i < NV4; ++i) {
            const int c4 = lane + 64 * i;
            const float4 xv = xr[c4], s4 = sc[c4], h4 = sh[c4];
            y[i] = make_float4(xv.x * (1.f + s4.x) + h4.x, xv.y * (1.f + s4.y) + h4.y,
                               xv.z * (1.f + s4.z) + h4.z, xv.w * (1.f + s4.w) + h4.w);
        }
        float acc[PF_MAXO];
#pragma unroll
        for (int o = 0; o < PF_MAXO; ++o) {
            float a = 0.f;
            if (o < Pout) {   // wave-uniform
#pragma unroll
                for (int i = 0; i < NV4; ++i) {
                    const uint2 wv = *reinterpret_cast<const uint2*>(sW + o * d + 4 * (lane + 64 * i));
                    a += y[i].x * __uint_as_float(wv.x << 16) + y[i].y * __uint_as_float(wv.x & 0xffff0000u) +
                         y[i].z * __uint_as_float(wv.y << 16) + y[i].w * __uint_as_float(wv.y & 0xffff0000u);
                }
            }
            acc[o] = a;
        }
#pragma unroll
        for (int o = 0; o < PF_MAXO; ++o) acc[o] = wave_sum(acc[o]);
        const int ti = tok / w, tj = tok % w;
        if (lane < Pout) {
            float v = 0.f;
#pragma unroll
            for (int o = 0; o < PF_MAXO; ++o) v = lane == o ? acc[o] : v;
            const int o = lane, py = o / (p * Cout), px = (o / Cout) % p, ch = o % Cout;
            out[(((long)b * Cout + ch) * H + ti * p + py) * W + tj * p + px] = v;
        }
    }
}

// fp32 weights (the full-precision configuration, small widths): one wave per token.
__global__ __launch_bounds__(256) void k_prefinal_project_f32(const float* __restrict__ resid, RowGeom g, int d,
                                                              const float* __restrict__ mod, long mod_stride,
                                                              int sc_off, int sh_off, const float* __restrict__ Wout,
                                                              int Cout, int p, int h, int w,
                                                              float* __restrict__ out) {
    constexpr int MAXO = 64;
    const int lane = threadIdx.x & 63;
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int nwaves = (gridDim.x * blockDim.x) >> 6;
    const int ntok = g.B * g.Ni;
    const int nv = d / 4;
    const int Pout = p * p * Cout;
    for (int t = wave; t < ntok; t += nwaves) {
        const int b = t / g.Ni, tok = t % g.Ni;
        const float* xr = resid + (long)(g.B * g.Nt + t) * d;
        const float* sc = mod + (long)b * mod_stride + sc_off;
        const float* sh = mod + (long)b * mod_stride + sh_off;
        float4 y[PF_MAXV];
#pragma unroll
        for (int i = 0; i < PF_MAXV; ++i) {
            int c4 = lane + 64 * i;
            if (c4 < nv) {
                float4 xv = reinterpret_cast<const float4*>(xr)[c4];
                float4 s4 = reinterpret_cast<const float4*>(sc)[c4];
                float4 h4 = reinterpret_cast<const float4*>(sh)[c4];
                y[i] = make_float4(xv.x * (1.f + s4.x) + h4.x, xv.y * (1.f + s4.y) + h4.y,
                                   xv.z * (1.f + s4.z) + h4.z, xv.w * (1.f + s4.w) + h4.w);
            } else {
                y[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        const int ti = tok / w, tj = tok % w;
        const int H = h * p, W = w * p;
        for (int o = 0; o < Pout && o < MAXO; ++o) {
            const float* wr = Wout + (long)o * d;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < PF_MAXV; ++i) {
                int c4 = lane + 64 * i;
                if (c4 < nv) {
                    const float4 wv = reinterpret_cast<const float4*>(wr)[c4];
                    acc += y[i].x * wv.x + y[i].y * wv.y + y[i].z * wv.z + y[i].w * wv.w;
                }
            }
            acc = wave_sum(acc);
            if (lane == 0) {
                int py = o / (p * Cout), px = (o / Cout) % p, ch = o % Cout;
                out[(((long)b * Cout + ch) * H + ti * p + py) * W + tj * p + px] = acc;
            }
        }
    }
}

hipError_t prefinal_project(const float* resid, RowGeom g, int d, const float* mod, long mod_stride, int sc_off,
                            int sh_off, const void* Wout, af_dtype wdt, int Cout, int p, int h, int w,
                            float* out, hipStream_t s) {
    const int ntok = g.B * g.Ni;
    if (ntok == 0) return hipSuccess;
    const int Pout = p * p * Cout;
    if (wdt == AF_BF16) {
        if (Pout > PF_MAXO || (long)Pout * d > PF_LDS || d % 256 != 0) return hipErrorInvalidValue;
        int n_cu = 0, dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
            n_cu = 256;
        const int blocks = std::min(n_cu, (ntok + 7) / 8);   // one workgroup of 8 waves per CU
#define AF_PF(V) hipLaunchKernelGGL(k_prefinal_project_bf16<V>, dim3(blocks), dim3(512), 0, s, resid, g, d, mod, \
                                    mod_stride, sc_off, sh_off, (const bf16_t*)Wout, Cout, p, h, w, out)
        switch (d / 256) {   // the bf16 path has d a multiple of 256, at most 4096
            case 1: AF_PF(1); break;   case 2: AF_PF(2); break;   case 3: AF_PF(3); break;
            case 4: AF_PF(4); break;   case 5: AF_PF(5); break;   case 6: AF_PF(6); break;
            case 7: AF_PF(7); break;   case 8: AF_PF(8); break;   case 9: AF_PF(9); break;
            case 10: AF_PF(10); break; case 11: AF_PF(11); break; case 12: AF_PF(12); break;
            case 13: AF_PF(13); break; case 14: AF_PF(14); break; case 15: AF_PF(15); break;
            case 16: AF_PF(16); break;
            default: return hipErrorInvalidValue;
        }
#undef AF_PF
    } else {
        const int blocks = std::min(2048, (ntok + 3) / 4);
        hipLaunchKernelGGL(k_prefinal_project_f32, dim3(blocks), dim3(256), 0, s, resid, g, d, mod, mod_stride,
                           sc_off, sh_off, (const float*)Wout, Cout, p, h, w, out);
    }
    return hipGetLastError();
}

// ============================================================================ Euler + CFG
// [PIPE] AuraFlowPipeline 核心参数详解 / [TRANS] 在 AuraFlowPipeline 中的实际调用:
// v_hat = v_u + s (v_c - v_u) with v = [uncond; cond] when CFG is on, else v;
// x <- x + (sigma_next - sigma) v_hat.
__global__ void k_euler_cfg(float* __restrict__ x, const float* __restrict__ v, long n, float dt, float gs,
                            int cfg_on) {
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float vh;
    if (cfg_on) {
        float vu = v[i], vc = v[n + i];
        vh = vu + gs * (vc - vu);
    } else {
        vh = v[i];
    }
    x[i] = x[i] + dt * vh;
}

hipError_t euler_cfg(float* x, const float* v, long n, float dt, float guidance, int cfg_on, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_euler_cfg, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, v, n, dt, guidance,
                       cfg_on);
    return hipGetLastError();
}

// x_in = [x; x] (cfg_on) or [x], tau[:] = sigma. vec: n % 4 == 0 and both
// pointers 16-byte aligned, one float4 per thread; otherwise one element per
// thread. The grid covers max(copy work, nt) threads.
__global__ void k_cfg_inputs(const float* __restrict__ x, long n, int cfg_on, float sigma, float* __restrict__ xin,
                             float* __restrict__ tau, int nt, int vec) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nt) tau[i] = sigma;
    if (vec) {
        if (4 * i < n) {
            const float4 v = reinterpret_cast<const float4*>(x)[i];
            reinterpret_cast<float4*>(xin)[i] = v;
            if (cfg_on) reinterpret_cast<float4*>(xin + n)[i] = v;
        }
    } else if (i < n) {
        xin[i] = x[i];
        if (cfg_on) xin[n + i] = x[i];
    }
}

hipError_t cfg_inputs(const float* x, long n, int Bi, int cfg_on, float sigma, float* xin, float* tau,
                      hipStream_t s) {
    if (n == 0) return hipSuccess;
    const int nt = cfg_on ? 2 * Bi : Bi;
    const int vec = (n % 4 == 0) && (((uintptr_t)x | (uintptr_t)xin) % 16 == 0);
    const long work = std::max<long>(vec ? n / 4 : n, nt);
    hipLaunchKernelGGL(k_cfg_inputs, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, x, n, cfg_on, sigma, xin,
                       tau, nt, vec);
    return hipGetLastError();
}

// ============================================================================ weight packing
// Canonical fp32 tensors -> device layout. FFN gate/up rows are interleaved in
// 32-row groups ([F, d] gate rows f -> packed row (f/32)*64 + f%32, up rows ->
// (f/32)*64 + 32 + f%32) so that a 64-column GEMM tile holds matching gate and
// up columns in the same lane.
__global__ void k_pack(const float* __restrict__ src, long n, long first, void* __restrict__ dst, int to_bf16,
                       int layout, int cols) {
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    long e = first + i;
    long o = e;
    if (layout != PACK_PLAIN) {
        long f = e / cols, c = e % cols;
        long prow = (f / 32) * 64 + (layout == PACK_FFN_UP ? 32 : 0) + f % 32;
        o = prow * cols + c;
    }
    if (to_bf16) ((bf16_t*)dst)[o] = f2bf(src[i]);
    else ((float*)dst)[o] = src[i];
}

hipError_t pack_weights(const float* src, long n, long first, void* dst, af_dtype ddt, int layout, int cols,
                        hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_pack, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, n, first, dst,
                       ddt == AF_BF16 ? 1 : 0, layout, cols);
    return hipGetLastError();
}

// ============================================================================ MXFP8 weights
// bf16 weight [N, K] -> E4M3 [N, K] + block scales [K/64][N][2] (the MXFP8 rule
// of the activations: scale 2^(floor(log2 amax) - 8) per 32 values along K). One
// thread per (row, 32-value block).
__global__ void k_mx_quant_rows(const bf16_t* __restrict__ src, long N, int K, uint8_t* __restrict__ dst,
                                uint8_t* __restrict__ sc) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const int nb = K / 32;
    if (i >= N * nb) return;
    const long n = i / nb;
    const int b = (int)(i % nb);
    const bf16_t* p = src + n * K + b * 32;
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 u = *reinterpret_cast<const uint4*>(p + 8 * q);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            v[8 * q + 2 * r] = __uint_as_float(w[r] << 16);
            v[8 * q + 2 * r + 1] = __uint_as_float(w[r] & 0xFFFF0000u);
        }
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(v[k]));
    const int e = mx_scale_exp(amax);
    const float inv = pow2f(-e);
    uint32_t o[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = pack4_e4m3(v[4 * q] * inv, v[4 * q + 1] * inv, v[4 * q + 2] * inv, v[4 * q + 3] * inv);
    uint4* d4 = reinterpret_cast<uint4*>(dst + n * K + b * 32);
    d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
    sc[((long)(b >> 1) * N + n) * 2 + (b & 1)] = (uint8_t)(e + 127);
}

hipError_t mx_quantize_rows(const bf16_t* src, long N, int K, uint8_t* dst, uint8_t* sc, hipStream_t s) {
    if (N == 0) return hipSuccess;
    if (K % 64 != 0) return hipErrorInvalidValue;
    const long n = N * (K / 32);
    hipLaunchKernelGGL(k_mx_quant_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, N, K, dst, sc);
    return hipGetLastError();
}

// ============================================================================ residual -> [B, S, d]
__global__ void k_taps(const float* __restrict__ resid, RowGeom g, int d, float* __restrict__ out) {
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    long n = (long)g.B * g.S() * d;
    if (i >= n) return;
    int c = i % d;
    long bs = i / d;
    int s_ = bs % g.S(), b = bs / g.S();
    out[i] = resid[(long)g.row_of(b, s_) * d + c];
}

hipError_t taps_permute(const float* resid, RowGeom g, int d, float* out, hipStream_t s) {
    long n = (long)g.B * g.S() * d;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_taps, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, resid, g, d, out);
    return hipGetLastError();
}

// ============================================================================ fp32 path helpers
// raw [M, 3d] = [q | k | v]; q and k get a per-head LayerNorm over hd (QK-norm,
// [TRANS] 注意力处理器与 QKV 融合), all three are scattered to [B, H, S_pad, hd].
__global__ void k_qknorm_scatter_f32(const float* __restrict__ raw, int M, RowGeom g, int H, int hd, int S_pad,
                                     float eps, float* __restrict__ q, float* __restrict__ k,
                                     float* __restrict__ v, int row0) {
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)M * H * 3) return;
    int which = i % 3;
    int h = (i / 3) % H;
    int m = i / (3 * H);
    int d = H * hd;
    int r = row0 + m;
    int b = g.batch_of(r), s_ = g.seq_of(r);
    const float* src = raw + (long)m * 3 * d + which * d + h * hd;
    float* dst = (which == 0 ? q : which == 1 ? k : v) + (((long)b * H + h) * S_pad + s_) * hd;
    if (which == 2) {
        for (int t = 0; t < hd; ++t) dst[t] = src[t];
        return;
    }
    float mean = 0.f;
    for (int t = 0; t < hd; ++t) mean += src[t];
    mean /= (float)hd;
    float var = 0.f;
    for (int t = 0; t < hd; ++t) { float c = src[t] - mean; var += c * c; }
    float rstd = rsqrtf(var / (float)hd + eps);
    for (int t = 0; t < hd; ++t) dst[t] = (src[t] - mean) * rstd;
}

hipError_t qknorm_scatter_f32(const float* raw, int M, RowGeom g, int H, int hd, int S_pad, float eps, float* q,
                              float* k, float* v, int row0, hipStream_t s) {
    long n = (long)M * H * 3;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_qknorm_scatter_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, raw, M, g, H, hd,
                       S_pad, eps, q, k, v, row0);
    return hipGetLastError();
}

// raw [M, 2F] in the 32-column gate/up interleave -> h[m, f] = silu(gate) * up.
__global__ void k_swiglu_f32(const float* __restrict__ raw, int M, int F, float* __restrict__ h) {
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)M * F) return;
    int f = i % F;
    long m = i / F;
    long base = m * 2 * F + (f / 32) * 64 + f % 32;
    float a = raw[base], u = raw[base + 32];
    h[i] = silu_f(a) * u;
}

hipError_t swiglu_f32(const float* raw, int M, int F, float* h, hipStream_t s) {
    long n = (long)M * F;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_swiglu_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, raw, M, F, h);
    return hipGetLastError();
}

}  // namespace af

namespace af {

// ============================================================================ split-K sum
// resid[i] += part[0][i] + part[1][i] + ... + part[ks - 1][i], added in that order
// (deterministic); four consecutive values per thread.
__global__ void k_splitk_resid(const float* __restrict__ part, int ks, long n, float* __restrict__ resid) {
    const long i = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i >= n) return;
    float4 acc = *reinterpret_cast<const float4*>(part + i);
    for (int s = 1; s < ks; ++s) {
        const float4 p = *reinterpret_cast<const float4*>(part + (long)s * n + i);
        acc.x += p.x;
        acc.y += p.y;
        acc.z += p.z;
        acc.w += p.w;
    }
    float4 r = *reinterpret_cast<const float4*>(resid + i);
    r.x += acc.x;
    r.y += acc.y;
    r.z += acc.z;
    r.w += acc.w;
    *reinterpret_cast<float4*>(resid + i) = r;
}

hipError_t splitk_resid(const float* part, int ks, long M, int N, float* resid, hipStream_t s) {
    const long n = M * N;
    if (n == 0) return hipSuccess;
    if (N % 4 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_splitk_resid, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, part, ks, n, resid);
    return hipGetLastError();
}

}  // namespace af

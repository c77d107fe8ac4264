// Kernels of the VAE decode (the AutoencoderKL decoder the pipeline runs on the
// sampler's latents: [PIPE] AuraFlow 模型与管线概述, [TRANS] 在 AuraFlowPipeline
// 中的实际调用). The 3x3 and 1x1 convolutions and the attention's products run
// on the bf16 GEMM (EPI_CONV: implicit-GEMM gather of the 3x3 window, bias and
// residual in the epilogue); these kernels are the rest: the latent scaling and
// post-quant 1x1 convolution, GroupNorm (statistics and the normalise + affine
// + SiLU pass that writes the next convolution's bf16 operand), the attention's
// row softmax and v transpose, the 3-channel output convolution and the weight
// packing.
//
// Activations are NHWC: [B, P, C] with P = H W pixels per sample, channels
// contiguous, so a GEMM row is a pixel and GroupNorm's groups are runs of C / G
// consecutive channels.
#include <algorithm>

#include "af_internal.h"

namespace af {

namespace {
constexpr int GN_FIN_T = 256;    // threads per (sample, group) in the merge

// Pixels per GroupNorm statistics workgroup: 512, halved (down to 16) until a
// sample has at least 512 chunks, so low-resolution levels still fill the GPU.
// It depends on the sample's size only, not on the batch: a sample's statistics
// are summed in the same order whatever batch it is decoded in.
long gn_chunk_pixels(long P) {
    long pix = 512;
    while (pix > 16 && (P + pix - 1) / pix < 512) pix /= 2;
    return pix;
}
}  // namespace

// ---------------------------------------------------------------------------- latent prep
// z = latents / scaling; y = Wpq z + bpq (the 1x1 post-quant convolution, fp32);
// out[b, p, c] = bf16(y[c]) for c < Cl, 0 for Cl <= c < Cpad. One thread per pixel.
__global__ void k_vae_prep(const float* __restrict__ lat, int B, int Cl, long P, float inv_scale,
                           const float* __restrict__ wpq, const float* __restrict__ bpq, int Cpad,
                           bf16_t* __restrict__ out) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)B * P) return;
    const long b = i / P, p = i % P;
    float z[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) z[c] = c < Cl ? lat[(b * Cl + c) * P + p] * inv_scale : 0.f;
    bf16_t* o = out + i * Cpad;
    for (int c = 0; c < Cpad; ++c) {
        float y = 0.f;
        if (c < Cl) {
            y = bpq[c];
#pragma unroll
            for (int k = 0; k < 32; ++k)
                if (k < Cl) y += wpq[c * Cl + k] * z[k];
        }
        o[c] = f2bf(y);
    }
}

hipError_t vae_prep(const float* lat, int B, int Cl, long P, float scaling, const float* wpq, const float* bpq,
                    int Cpad, bf16_t* out, hipStream_t s) {
    if (Cl > 32 || Cpad < Cl) return hipErrorInvalidValue;
    const long n = (long)B * P;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_vae_prep, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, lat, B, Cl, P, 1.0f / scaling,
                       wpq, bpq, Cpad, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- GroupNorm
// Statistics in two passes over partial results, both in a fixed order (so a
// decode is bit-reproducible). Pass 1: workgroup (chunk, b) covers `pix` pixels
// of sample b; thread t owns float4 column j = t % (C / 4) (four channels of one
// group: C / G is a multiple of 4) and every (256 / (C / 4))-th pixel. It sums
// v - r and (v - r)^2 with r its first value (a shift that keeps the fp32 sums
// well conditioned), turns them into (count, mean, M2), and the eight threads
// of each group are merged in a fixed order with the pairwise update of Chan et
// al. (n = na + nb, delta = mb - ma, mean = ma + delta nb / n, M2 = M2a + M2b +
// delta^2 na nb / n). part[b][chunk][g] = (n, mean, M2, 0).
__global__ __launch_bounds__(256) void k_gn_partial(const float* __restrict__ x, long P, int C, int G, int nchunk,
                                                    long pix, float4* __restrict__ part) {
    const int chunk = blockIdx.x, b = blockIdx.y;
    const int cols = C / 4, lanes = 256 / cols;
    const int t = threadIdx.x, j = t % cols, pl = t / cols;
    const float* xb = x + (long)b * P * C + 4 * j;
    const long p0 = (long)chunk * pix, p1 = min(P, p0 + pix);
    float n = 0.f, ref = 0.f, s1 = 0.f, s2 = 0.f;
    if (pl < lanes && p0 + pl < p1) {
        ref = xb[(p0 + pl) * C];
        for (long p = p0 + pl; p < p1; p += lanes) {
            const float4 v = *reinterpret_cast<const float4*>(xb + p * C);
            const float d0 = v.x - ref, d1 = v.y - ref, d2 = v.z - ref, d3 = v.w - ref;
            s1 += (d0 + d1) + (d2 + d3);
            s2 += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
            n += 4.f;
        }
    }
    __shared__ float sn[256], sm[256], sq[256];
    sn[t] = n;
    sm[t] = n > 0.f ? ref + s1 / n : 0.f;
    sq[t] = n > 0.f ? fmaxf(s2 - s1 * s1 / n, 0.f) : 0.f;
    __syncthreads();
    if (t < G) {
        const int per = C / G / 4;
        float N = 0.f, mu = 0.f, M2 = 0.f;
        for (int l = 0; l < lanes; ++l)
            for (int q = 0; q < per; ++q) {
                const int u = l * cols + t * per + q;
                const float nb = sn[u];
                if (nb == 0.f) continue;
                const float nn = N + nb, dl = sm[u] - mu;
                mu += dl * (nb / nn);
                M2 += sq[u] + dl * dl * (N * nb / nn);
                N = nn;
            }
        part[((long)b * nchunk + chunk) * G + t] = make_float4(N, mu, M2, 0.f);
    }
}

// Pass 2: one workgroup per (b, g). Thread t merges chunks t, t + 256, ... in
// fp64, then a fixed tree merges the 256 results. stats[b G + g] = (mean, rstd).
__global__ __launch_bounds__(GN_FIN_T) void k_gn_finalize(const float4* __restrict__ part, int nchunk, int G,
                                                          float eps, float2* __restrict__ stats) {
    const int bg = blockIdx.x, b = bg / G, g = bg % G, t = threadIdx.x;
    double N = 0.0, mu = 0.0, M2 = 0.0;
    for (int c = t; c < nchunk; c += GN_FIN_T) {
        const float4 v = part[((long)b * nchunk + c) * G + g];
        if (v.x == 0.f) continue;
        const double nb = v.x, nn = N + nb, dl = (double)v.y - mu;
        mu += dl * nb / nn;
        M2 += (double)v.z + dl * dl * N * nb / nn;
        N = nn;
    }
    __shared__ double sN[GN_FIN_T], sM[GN_FIN_T], sQ[GN_FIN_T];
    sN[t] = N;
    sM[t] = mu;
    sQ[t] = M2;
    __syncthreads();
    for (int w = GN_FIN_T / 2; w > 0; w >>= 1) {
        if (t < w) {
            const double na = sN[t], nb = sN[t + w];
            if (nb > 0.0) {
                const double nn = na + nb, dl = sM[t + w] - sM[t];
                sM[t] += dl * nb / nn;
                sQ[t] += sQ[t + w] + dl * dl * na * nb / nn;
                sN[t] = nn;
            }
        }
        __syncthreads();
    }
    if (t == 0) {
        const double var = sN[0] > 0.0 ? sQ[0] / sN[0] : 0.0;
        stats[bg] = make_float2((float)sM[0], (float)(1.0 / sqrt(var + (double)eps)));
    }
}

size_t gn_part_floats(int B, long P, int G) {
    // every P' <= P takes at most this many chunks per sample
    const long most = std::max((P + 511) / 512, 1024L) + 1;
    return (size_t)B * most * G * 4;
}

hipError_t group_norm_stats(const float* x, int B, long P, int C, int G, float eps, float4* part, float2* stats,
                            hipStream_t s) {
    if (C % (4 * G) != 0 || C / 4 > 256 || G > 256) return hipErrorInvalidValue;
    if (B == 0 || P == 0) return hipSuccess;
    const long pix = gn_chunk_pixels(P);
    const int nchunk = (int)((P + pix - 1) / pix);
    hipLaunchKernelGGL(k_gn_partial, dim3(nchunk, B), dim3(256), 0, s, x, P, C, G, nchunk, pix, part);
    hipLaunchKernelGGL(k_gn_finalize, dim3(B * G), dim3(GN_FIN_T), 0, s, (const float4*)part, nchunk, G, eps, stats);
    return hipGetLastError();
}

// y = (x - mean) rstd gamma + beta (then SiLU when silu != 0) -> bf16, eight
// channels per thread (two halves of four, each inside one group).
__global__ void k_gn_apply(const float* __restrict__ x, long P, int C, int G, const float2* __restrict__ stats,
                           const float* __restrict__ gamma, const float* __restrict__ beta, int silu,
                           bf16_t* __restrict__ y, long n8) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    const long e = i * 8;
    const int c = (int)(e % C);
    const long b = e / C / P;
    const int cpg = C / G;
    const float2 st0 = stats[b * G + c / cpg], st1 = stats[b * G + (c + 4) / cpg];
    const float4 v0 = *reinterpret_cast<const float4*>(x + e);
    const float4 v1 = *reinterpret_cast<const float4*>(x + e + 4);
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float r[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = 2 * q + h;
            const float2 st = k < 4 ? st0 : st1;
            float t = (v[k] - st.x) * st.y * gamma[c + k] + beta[c + k];
            if (silu) t = silu_f(t);
            r[h] = t;
        }
        w[q] = (uint32_t)f2bf(r[0]) | ((uint32_t)f2bf(r[1]) << 16);
    }
    *reinterpret_cast<uint4*>(y + e) = make_uint4(w[0], w[1], w[2], w[3]);
}

hipError_t group_norm_apply(const float* x, int B, long P, int C, int G, const float2* stats, const float* gamma,
                            const float* beta, int silu, bf16_t* y, hipStream_t s) {
    if (C % 8 != 0 || (C / G) % 4 != 0) return hipErrorInvalidValue;
    const long n8 = (long)B * P * C / 8;
    if (n8 == 0) return hipSuccess;
    hipLaunchKernelGGL(k_gn_apply, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x, P, C, G, stats, gamma,
                       beta, silu, y, n8);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- attention pieces
// P[r, j] = exp(scale (S[r, j] - max_j S[r, j])) / sum for j < n, 0 for n <= j < ld;
// one workgroup per row, the row read three times (max, sum, write) through L2.
__global__ __launch_bounds__(256) void k_softmax_rows(const float* __restrict__ S, long ld, int n, float scale,
                                                     bf16_t* __restrict__ P) {
    const long r = blockIdx.x;
    const float* row = S + r * ld;
    bf16_t* prow = P + r * ld;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    __shared__ float red[4];
    float m = -INFINITY;
    for (int j = t; j < n; j += 256) m = fmaxf(m, row[j]);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) red[wv] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float sum = 0.f;
    for (int j = t; j < n; j += 256) sum += __expf(scale * (row[j] - m));
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
    if (lane == 0) red[wv] = sum;
    __syncthreads();
    const float inv = 1.0f / ((red[0] + red[1]) + (red[2] + red[3]));
    for (int j = t; j < (int)ld; j += 256) prow[j] = j < n ? f2bf(__expf(scale * (row[j] - m)) * inv) : (bf16_t)0;
}

// The same with the row held in registers (VPT values per thread, n <= 256 VPT):
// one read of S and one write of P.
template <int VPT>
__global__ __launch_bounds__(256) void k_softmax_rows_reg(const float* __restrict__ S, long ld, int n, float scale,
                                                         bf16_t* __restrict__ P) {
    const long r = blockIdx.x;
    const float* row = S + r * ld;
    bf16_t* prow = P + r * ld;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    __shared__ float red[4];
    float v[VPT];
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int j = t + 256 * k;
        v[k] = j < n ? row[j] : -INFINITY;
        m = fmaxf(m, v[k]);
    }
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) red[wv] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        v[k] = (t + 256 * k) < n ? __expf(scale * (v[k] - m)) : 0.f;
        sum += v[k];
    }
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
    if (lane == 0) red[wv] = sum;
    __syncthreads();
    const float inv = 1.0f / ((red[0] + red[1]) + (red[2] + red[3]));
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int j = t + 256 * k;
        if (j < ld) prow[j] = f2bf(v[k] * inv);
    }
    for (long j = 256L * VPT + t; j < ld; j += 256) prow[j] = (bf16_t)0;
}

hipError_t softmax_rows(const float* S, long rows, long ld, int n, float scale, bf16_t* P, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    if (n < 1 || n > ld || rows > 0x7fffffffL) return hipErrorInvalidValue;
    const dim3 g((unsigned)rows), b(256);
    if (n <= 256 * 16) hipLaunchKernelGGL(k_softmax_rows_reg<16>, g, b, 0, s, S, ld, n, scale, P);
    else if (n <= 256 * 32) hipLaunchKernelGGL(k_softmax_rows_reg<32>, g, b, 0, s, S, ld, n, scale, P);
    else if (n <= 256 * 64) hipLaunchKernelGGL(k_softmax_rows_reg<64>, g, b, 0, s, S, ld, n, scale, P);
    else hipLaunchKernelGGL(k_softmax_rows, g, b, 0, s, S, ld, n, scale, P);
    return hipGetLastError();
}

// vt[c, p] = src[p * lds + c] for p < P, 0 for P <= p < Ppad (c < C); 64 x 64 tiles
// through LDS, blockIdx.x over pixel tiles, blockIdx.y over channel tiles.
__global__ __launch_bounds__(256) void k_transpose_cols(const bf16_t* __restrict__ src, long lds, long P, int C,
                                                        long Ppad, bf16_t* __restrict__ vt) {
    __shared__ bf16_t tile[64][66];
    const long p0 = (long)blockIdx.x * 64;
    const int c0 = blockIdx.y * 64, t = threadIdx.x;
    for (int k = t; k < 64 * 64; k += 256) {
        const int pr = k / 64, cc = k % 64;
        const long p = p0 + pr;
        tile[pr][cc] = (p < P && c0 + cc < C) ? src[p * lds + c0 + cc] : (bf16_t)0;
    }
    __syncthreads();
    for (int k = t; k < 64 * 64; k += 256) {
        const int cr = k / 64, pc = k % 64;
        const long p = p0 + pc;
        if (c0 + cr < C && p < Ppad) vt[(long)(c0 + cr) * Ppad + p] = tile[pc][cr];
    }
}

hipError_t transpose_cols(const bf16_t* src, long lds, long P, int C, long Ppad, bf16_t* vt, hipStream_t s) {
    if (Ppad == 0 || C == 0) return hipSuccess;
    hipLaunchKernelGGL(k_transpose_cols, dim3((unsigned)((Ppad + 63) / 64), (unsigned)((C + 63) / 64)), dim3(256), 0, s,
                       src, lds, P, C, Ppad, vt);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- output convolution
// img[b, o, y, x] = bias[o] + sum over taps (dy, dx) and channels c of
// W[o][(3 (dy + 1) + dx + 1) Cin + c] a[b, y + dy, x + dx, c] (zero outside), for
// o < COUT <= 4: the 3x3 convolution to the image channels, too narrow for the
// GEMM's 128-wide tiles. A workgroup computes an 8 x 32 tile of output pixels,
// one per thread. Per 32-channel slice the 10 x 34 input halo is staged in LDS
// (80-byte pixel slots: the 16-byte reads of 16 consecutive pixels hit disjoint
// banks) and each thread takes its 9 taps with v_dot2 on bf16 channel pairs,
// the weights (uniform across the wave) coming from scalar loads.
namespace {
constexpr int CO_TY = 8, CO_TX = 32, CO_HY = CO_TY + 2, CO_HX = CO_TX + 2, CO_PS = 40;
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
}  // namespace

template <int COUT>
__global__ __launch_bounds__(256) void k_conv_out(const bf16_t* __restrict__ a, int H, int W, int Cin,
                                                  const uint32_t* __restrict__ w, const float* __restrict__ bias,
                                                  float* __restrict__ img) {
    __shared__ __attribute__((aligned(16))) bf16_t tile[CO_HY * CO_HX * CO_PS];
    const int tx0 = blockIdx.x * CO_TX, ty0 = blockIdx.y * CO_TY, b = blockIdx.z;
    const int t = threadIdx.x, lx = t % CO_TX, ly = t / CO_TX;
    const int x = tx0 + lx, y = ty0 + ly;
    const int K2 = 9 * Cin / 2;   // bf16 pairs per output channel
    float acc[COUT];
#pragma unroll
    for (int o = 0; o < COUT; ++o) acc[o] = 0.f;
    for (int c0 = 0; c0 < Cin; c0 += 32) {
        __syncthreads();
        for (int k = t; k < CO_HY * CO_HX * 4; k += 256) {
            const int pix = k >> 2, q = k & 3;
            const int sy = ty0 + pix / CO_HX - 1, sx = tx0 + pix % CO_HX - 1;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (sy >= 0 && sy < H && sx >= 0 && sx < W)
                v = *reinterpret_cast<const uint4*>(a + (((long)b * H + sy) * W + sx) * Cin + c0 + q * 8);
            *reinterpret_cast<uint4*>(tile + pix * CO_PS + q * 8) = v;
        }
        __syncthreads();
#pragma unroll
        for (int tap = 0; tap < 9; ++tap) {
            const bf16_t* src = tile + ((ly + tap / 3) * CO_HX + lx + tap % 3) * CO_PS;
            uint32_t u[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 v = *reinterpret_cast<const uint4*>(src + q * 8);
                u[4 * q] = v.x;
                u[4 * q + 1] = v.y;
                u[4 * q + 2] = v.z;
                u[4 * q + 3] = v.w;
            }
            const int wk = (tap * Cin + c0) / 2;
#pragma unroll
            for (int o = 0; o < COUT; ++o)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    acc[o] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, u[j]),
                                                            __builtin_bit_cast(bf16x2v, w[o * K2 + wk + j]), acc[o],
                                                            false);
        }
    }
    if (x < W && y < H) {
        const long HW = (long)H * W;
#pragma unroll
        for (int o = 0; o < COUT; ++o) img[((long)b * COUT + o) * HW + (long)y * W + x] = acc[o] + bias[o];
    }
}

hipError_t conv_out3x3(const bf16_t* a, int B, int H, int W, int Cin, const bf16_t* w, const float* bias, int Cout,
                       float* img, hipStream_t s) {
    if (Cout < 1 || Cout > 4 || Cin % 32 != 0) return hipErrorInvalidValue;
    if ((long)B * H * W == 0) return hipSuccess;
    const dim3 g((unsigned)((W + CO_TX - 1) / CO_TX), (unsigned)((H + CO_TY - 1) / CO_TY), (unsigned)B), blk(256);
    const uint32_t* wp = reinterpret_cast<const uint32_t*>(w);
    switch (Cout) {
        case 1: hipLaunchKernelGGL(k_conv_out<1>, g, blk, 0, s, a, H, W, Cin, wp, bias, img); break;
        case 2: hipLaunchKernelGGL(k_conv_out<2>, g, blk, 0, s, a, H, W, Cin, wp, bias, img); break;
        case 3: hipLaunchKernelGGL(k_conv_out<3>, g, blk, 0, s, a, H, W, Cin, wp, bias, img); break;
        default: hipLaunchKernelGGL(k_conv_out<4>, g, blk, 0, s, a, H, W, Cin, wp, bias, img); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- weight packing
// src[0, n) is a slice of one canonical tensor starting at element `first`.
// mode VAE_PACK_BF16: dst bf16, same order; VAE_PACK_CONV3: a [Cout, Cin, 3, 3]
// kernel to the GEMM's [Cout][9 Cpad] rows, column tap Cpad + c with tap =
// 3 ky + kx (columns of padding channels are left as they are: zero from the
// arena's clear); VAE_PACK_F32R: dst fp32 holding the value's bf16 rounding.
__global__ void k_vae_pack(const float* __restrict__ src, long n, long first, void* __restrict__ dst, int mode,
                           int cin, int cpad) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const long e = first + i;
    const float v = src[i];
    if (mode == VAE_PACK_F32R) {
        ((float*)dst)[e] = bf2f(f2bf(v));
        return;
    }
    long o = e;
    if (mode == VAE_PACK_CONV3) {
        const long per = 9L * cin;
        const long co = e / per, rem = e % per;
        const long c = rem / 9, tap = rem % 9;
        o = co * 9L * cpad + tap * cpad + c;
    }
    ((bf16_t*)dst)[o] = f2bf(v);
}

hipError_t vae_pack(const float* src, long n, long first, void* dst, int mode, int cin, int cpad, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_vae_pack, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, n, first, dst, mode, cin,
                       cpad);
    return hipGetLastError();
}

}  // namespace af

// Kernels of the text encoder (UMT5; configuration in [DEEP] section 2.1
// 文本编码器): token embedding gather, the T5 layer norm, the relative-position
// bias rows and self-attention over 64-channel heads. The matrix products run
// on the bf16 GEMM (STORE, GATED_RESID with a unit gate, GEGLU epilogues).
#include "af_internal.h"

namespace af {

namespace {
constexpr int U_HD = 64;    // channels per head
constexpr int U_QT = 128;   // queries per workgroup: 4 waves x 32

__device__ __forceinline__ int u_swap23(int x) { return (x & ~12) | ((x >> 1) & 4) | ((x << 1) & 8); }

// Bucket of relative position rel = key - query for 32 bidirectional buckets and
// maximum distance 128: 16 per sign (positive distances offset by 16); |rel| < 8
// exact; otherwise 8 + floor(8 log(n / 8) / log 16) = 8 + floor(log2(n^2 / 64)),
// i.e. 8 + bit_length(n^2) - 7, capped at 15 (integer arithmetic, no log).
__device__ __forceinline__ int u_bucket(int rel) {
    const int n = rel < 0 ? -rel : rel;
    const int base = rel > 0 ? 16 : 0;
    if (n < 8) return base + n;
    const unsigned n2 = (unsigned)n * (unsigned)n;
    const int bl = 32 - __clz(n2);
    return base + min(8 + bl - 7, 15);
}
}  // namespace

// ---------------------------------------------------------------------------- embedding
// x[r, :] = E[ids[r], :] (bf16 table -> fp32 rows); an id outside [0, vocab) reads zeros.
// One thread per 8 consecutive values.
__global__ void k_embed_rows(const int32_t* __restrict__ ids, long M, const bf16_t* __restrict__ E, int vocab,
                             int d, float* __restrict__ x) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const int per = d / 8;
    if (i >= M * per) return;
    const long r = i / per;
    const int c = (int)(i % per) * 8;
    const int id = ids[r];
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (id >= 0 && id < vocab) {
        const uint4 u = *reinterpret_cast<const uint4*>(E + (long)id * d + c);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    }
    float* dst = x + r * d + c;
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

hipError_t umt5_embed(const int32_t* ids, long M, const bf16_t* E, int vocab, int d, float* x, hipStream_t s) {
    const long n = M * (d / 8);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_embed_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ids, M, E, vocab, d, x);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- T5 layer norm
// out[r] = x[r] / sqrt(mean(x[r]^2) + eps) * w, fp32 statistics; one wave per row,
// the row held in registers (MAXV float4 per lane).
template <typename OT, int MAXV>
__global__ __launch_bounds__(256) void k_rms_norm(const float* __restrict__ x, int M, int d,
                                                  const float* __restrict__ w, float eps, OT* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const int nv = d / 4;
    const float* xr = x + (long)row * d;
    float4 v[MAXV];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int c4 = lane + 64 * i;
        v[i] = c4 < nv ? reinterpret_cast<const float4*>(xr)[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
        ss += (v[i].x * v[i].x + v[i].y * v[i].y) + (v[i].z * v[i].z + v[i].w * v[i].w);
    }
    const float rs = rsqrtf(wave_sum(ss) / (float)d + eps);
    OT* orow = out + (long)row * d;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int c4 = lane + 64 * i;
        if (c4 < nv) {
            const float4 wv = reinterpret_cast<const float4*>(w)[c4];
            const float a = v[i].x * rs * wv.x, b = v[i].y * rs * wv.y, c = v[i].z * rs * wv.z,
                        e = v[i].w * rs * wv.w;
            if constexpr (sizeof(OT) == 2) {
                *reinterpret_cast<uint2*>(orow + 4 * c4) = make_uint2(pack2bf(a, b), pack2bf(c, e));
            } else {
                *reinterpret_cast<float4*>(orow + 4 * c4) = make_float4(a, b, c, e);
            }
        }
    }
}

hipError_t umt5_rms_norm(const float* x, int M, int d, const float* w, float eps, void* out, bool bf16_out,
                         hipStream_t s) {
    if (M == 0) return hipSuccess;
    const int per_lane = (d / 4 + 63) / 64;
    const dim3 grid((M + 3) / 4), block(256);
#define U_RMS(V)                                                                                           \
    do {                                                                                                   \
        if (bf16_out)                                                                                      \
            hipLaunchKernelGGL((k_rms_norm<bf16_t, V>), grid, block, 0, s, x, M, d, w, eps, (bf16_t*)out); \
        else                                                                                               \
            hipLaunchKernelGGL((k_rms_norm<float, V>), grid, block, 0, s, x, M, d, w, eps, (float*)out);   \
    } while (0)
    if (per_lane <= 4) U_RMS(4);
    else if (per_lane <= 8) U_RMS(8);
    else U_RMS(16);
#undef U_RMS
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- relative-position bias rows
// rows[l][h][rel + T - 1] = rel_bias[l][bucket(rel)][h] for rel in [-(T - 1), T - 1]
// (rel_bias: [L][32][H] fp32, one table per layer).
__global__ void k_rel_bias_rows(const float* __restrict__ rel_bias, int L, int H, int T, float* __restrict__ rows) {
    const long n = (long)L * H * (2 * T - 1);
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int idx = (int)(i % (2 * T - 1));
    const int h = (int)((i / (2 * T - 1)) % H);
    const int l = (int)(i / ((long)(2 * T - 1) * H));
    rows[i] = rel_bias[((long)l * 32 + u_bucket(idx - (T - 1))) * H + h];
}

hipError_t umt5_rel_bias_rows(const float* rel_bias, int L, int H, int T, float* rows, hipStream_t s) {
    const long n = (long)L * H * (2 * T - 1);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_rel_bias_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, rel_bias, L, H, T, rows);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- self-attention, 64-wide heads
// One workgroup = 128 queries of one (sample, head); each wave owns 32 queries
// (one per lane & 31) as MFMA B operands. The sample's keys and values for the
// head are staged once in LDS: K rows [key][64] with 16-byte chunks XOR swizzled
// by key & 7, v^T [64][key] with bits 2 and 3 of the key index swapped inside each
// 16-key group, so that the S^T = K q^T accumulators a lane holds for one 16-key
// step are exactly the 8 keys the P V MFMA takes from it. Per 32-key tile: S^T
// (4 MFMAs over the 64 channels), + relative-position bias + key mask, online
// softmax (running maximum per query; the two lanes holding a query share it
// through one cross-half shuffle), O^T += v^T P^T (4 MFMAs).
template <int TMAX>
__global__ __launch_bounds__(256) void k_umt5_attention(const bf16_t* __restrict__ qkv, int d, int T, int H,
                                                        const float* __restrict__ bias_rows,
                                                        const uint8_t* __restrict__ mask, bf16_t* __restrict__ out) {
    constexpr int VS = TMAX + 8;   // v^T row stride (elements)
    __shared__ __attribute__((aligned(16))) bf16_t sK[TMAX * U_HD];
    __shared__ __attribute__((aligned(16))) bf16_t sV[U_HD * VS];
    __shared__ float sB[2 * TMAX];
    __shared__ float sM[TMAX];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 5, l32 = lane & 31;
    const int nqb = (T + U_QT - 1) / U_QT;
    const int qb = blockIdx.x % nqb, h = (blockIdx.x / nqb) % H, b = blockIdx.x / (nqb * H);
    const int Tp = (T + 31) / 32 * 32;
    const long ld = 3L * d;
    const bf16_t* base = qkv + (long)b * T * ld;

    for (int i = tid; i < Tp * 8; i += 256) {
        const int j = i >> 3, ch = i & 7;   // key, 16-byte chunk of 8 channels
        uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = make_uint4(0u, 0u, 0u, 0u);
        if (j < T) {
            kv = *reinterpret_cast<const uint4*>(base + (long)j * ld + d + h * U_HD + ch * 8);
            vv = *reinterpret_cast<const uint4*>(base + (long)j * ld + 2 * d + h * U_HD + ch * 8);
        }
        *reinterpret_cast<uint4*>(sK + j * U_HD + ((ch ^ (j & 7)) * 8)) = kv;
        const int pos = (j & ~15) | u_swap23(j & 15);
        const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sV[(ch * 8 + 2 * e) * VS + pos] = (bf16_t)(w[e] & 0xffffu);
            sV[(ch * 8 + 2 * e + 1) * VS + pos] = (bf16_t)(w[e] >> 16);
        }
    }
    for (int i = tid; i < 2 * T - 1; i += 256) sB[i] = bias_rows[(long)h * (2 * T - 1) + i];
    for (int j = tid; j < Tp; j += 256) sM[j] = (j < T && (mask == nullptr || mask[(long)b * T + j] != 0)) ? 0.f : -INFINITY;
    __syncthreads();

    // this lane's query (rows past T read row T - 1; their results are not stored)
    const int q = qb * U_QT + wave * 32 + l32;
    const int qr = min(q, T - 1);
    bf16x8 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        qf[ks] = *reinterpret_cast<const bf16x8*>(base + (long)qr * ld + h * U_HD + ks * 16 + grp * 8);

    f32x16 o[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
    float m_run = -INFINITY, l_part = 0.f;
    const int ntile = Tp / 32;
    for (int t = 0; t < ntile; ++t) {
        const int key = t * 32 + l32;
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + key * U_HD + (((2 * ks + grp) ^ (key & 7)) * 8));
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
        }
        // s[r] is key t*32 + 8 (r >> 2) + 4 grp + (r & 3) of query q
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kk = t * 32 + 8 * (r >> 2) + 4 * grp + (r & 3);
            const int bi = min(max(kk - q + T - 1, 0), 2 * T - 2);
            s[r] = s[r] + sB[bi] + sM[kk];
            mt = fmaxf(mt, s[r]);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        const bool none = m_new == -INFINITY;   // every key so far excluded
        const float alpha = none ? 1.f : __expf(m_run - m_new);
        float p[16], ps = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = none ? 0.f : __expf(s[r] - m_new);
            ps += p[r];
        }
        l_part = l_part * alpha + ps;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
        typedef float f32x8 __attribute__((ext_vector_type(8)));
        const f32x8 p0 = {p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]};
        const f32x8 p1 = {p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]};
        const bf16x8 pb[2] = {__builtin_convertvector(p0, bf16x8), __builtin_convertvector(p1, bf16x8)};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = i * 32 + l32;   // channel
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 vf = *reinterpret_cast<const bf16x8*>(sV + row * VS + t * 32 + ks * 16 + grp * 8);
                o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[ks], o[i], 0, 0, 0);
            }
        }
    }
    const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (q < T) {
        // O^T register r of tile i: channel i*32 + 8 (r >> 2) + 4 grp + (r & 3)
        bf16_t* orow = out + ((long)b * T + q) * d + h * U_HD;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int c = i * 32 + 8 * r4 + 4 * grp;
                *reinterpret_cast<uint2*>(orow + c) =
                    make_uint2(pack2bf(o[i][4 * r4] * inv, o[i][4 * r4 + 1] * inv),
                               pack2bf(o[i][4 * r4 + 2] * inv, o[i][4 * r4 + 3] * inv));
            }
    }
}

hipError_t umt5_attention(const bf16_t* qkv, int B, int T, int H, int d, const float* bias_rows,
                          const uint8_t* mask, bf16_t* out, hipStream_t s) {
    if (B == 0 || T == 0) return hipSuccess;
    const dim3 grid((unsigned)(B * H * ((T + U_QT - 1) / U_QT))), block(256);
    if (T <= 256)
        hipLaunchKernelGGL(k_umt5_attention<256>, grid, block, 0, s, qkv, d, T, H, bias_rows, mask, out);
    else if (T <= 512)
        hipLaunchKernelGGL(k_umt5_attention<512>, grid, block, 0, s, qkv, d, T, H, bias_rows, mask, out);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace af

// Joint attention for 256-wide heads on gfx950 (bf16 MFMA, fp32 softmax).
//
// [TRANS] 注意力处理器与 QKV 融合: text and image q/k/v are concatenated (text
// first) and one scaled-dot-product attention runs over the whole sequence, no
// dropout, not causal; the scale is 1/sqrt(head_dim). Keys of padded text
// tokens are excluded through an additive bias (0 or -inf) per key.
//
// Layout: q, k [B, H, S_pad, 256]; v^T [B, H, 256, S_pad] (written transposed by
// the QKV GEMM epilogue so the P V contraction reads keys contiguously);
// output o [M, d] in residual-row order.
//
// One workgroup = 4 waves = 128 queries of one (b, h); each wave owns 32 queries.
// Per 64-key tile:
//   S^T = K Q^T  (A = K from LDS, B = the wave's Q held in registers)
//     -> the accumulator has one query per lane (lane & 31) and 32 keys per lane,
//        so row max / row sum need one cross-half-wave exchange;
//   O^T += V^T P^T (A = v^T from LDS, B = P taken straight from the S^T
//     accumulator registers; the key order inside each 16-key MFMA step is
//     permuted identically on both operands, so P never goes through LDS).
// Online softmax keeps (m, l) per query in fp32; exp via exp2 with log2(e)
// folded into the scale.
#include "af_internal.h"

namespace af {

namespace {
constexpr int HD = 256;
constexpr int QT = 128;  // queries per workgroup
constexpr int KT = 64;   // keys per tile

// K tile: [64 keys][256] bf16, 32 chunks of 16 B per row, chunk ^= row & 15.
__device__ __forceinline__ int kswz(int row) { return row & 15; }
// V^T tile: [256 hd][64 keys] bf16, 8 chunks per row, chunk ^= f(row).
__device__ __forceinline__ int vswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_attention_bf16(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                      const bf16_t* __restrict__ Vt, const float* __restrict__ bias, RowGeom g, int H,
                      int S_pad, bf16_t* __restrict__ O, int d, float scale_log2) {
    __shared__ __attribute__((aligned(16))) bf16_t sK[KT * HD];
    __shared__ __attribute__((aligned(16))) bf16_t sV[HD * KT];
    __shared__ float sBias[KT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.z, h = blockIdx.y;
    const int S = g.S();
    const int q0 = blockIdx.x * QT + wave * 32;
    const long bh = (long)b * H + h;
    const bf16_t* Qbh = Q + bh * S_pad * HD;
    const bf16_t* Kbh = K + bh * S_pad * HD;
    const bf16_t* Vbh = Vt + bh * HD * (long)S_pad;
    const float* biasb = bias + (long)b * S_pad;

    // The wave's 32 queries as MFMA B operands: lane holds query q0 + (lane & 31),
    // head dims [16 s + 8 (lane >> 5), +8) for k-step s.
    bf16x8 qf[16];
    {
        const bf16_t* qrow = Qbh + (long)(q0 + (lane & 31)) * HD + (lane >> 5) * 8;
#pragma unroll
        for (int s = 0; s < 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + s * 16);
    }

    f32x16 o[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int ntiles = (S + KT - 1) / KT;
    for (int kt = 0; kt < ntiles; ++kt) {
        const int k0 = kt * KT;
        // ---- stage K tile and v^T tile in LDS
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            int idx = p * 256 + tid;          // 2048 chunks of 16 B
            int row = idx >> 5, ch = idx & 31;
            uint4 v = *reinterpret_cast<const uint4*>(Kbh + (long)(k0 + row) * HD + ch * 8);
            *reinterpret_cast<uint4*>(sK + row * HD + ((ch ^ kswz(row)) * 8)) = v;
        }
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            int idx = p * 256 + tid;          // 256 rows x 8 chunks
            int row = idx >> 3, ch = idx & 7; // chunk ch holds keys 8 ch .. 8 ch + 7
            uint4 v = *reinterpret_cast<const uint4*>(Vbh + (long)row * S_pad + k0 + ch * 8);
            // key k = 32 t + 8 i + 4 g + j goes to position (2 t + i/2) * 16 + 8 g + 4 (i%2) + j
            int t = ch >> 2, i = ch & 3;
            int base = (2 * t + (i >> 1)) * 16 + 4 * (i & 1);
            int c0 = (base >> 3), off = base & 7;      // 16-byte chunk index and offset (g = 0)
            bf16_t* rowp = sV + row * KT;
            *reinterpret_cast<uint2*>(rowp + ((c0 ^ vswz(row)) * 8) + off) = make_uint2(v.x, v.y);
            *reinterpret_cast<uint2*>(rowp + (((c0 + 1) ^ vswz(row)) * 8) + off) = make_uint2(v.z, v.w);
        }
        if (tid < KT) sBias[tid] = biasb[k0 + tid];
        __syncthreads();

        // ---- S^T = K Q^T for two 32-key sub-tiles
        f32x16 st[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) st[t][r] = 0.f;
            const int row = t * 32 + (lane & 31);
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                int ch = (2 * s + (lane >> 5)) ^ kswz(row);
                bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + row * HD + ch * 8);
                st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], st[t], 0, 0, 0);
            }
        }

        // ---- online softmax (one query per lane, keys spread over regs and the lane^32 partner)
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int key = t * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                float v = st[t][r] * scale_log2 + sBias[key];
                st[t][r] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = exp2f(st[t][r] - m_use);
                st[t][r] = p;
                psum += p;
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[t][r] *= alpha;

        // ---- P as B operands: k-step s4 takes sub-tile t = s4/2, register groups i0 = 2 (s4%2), i0 + 1
        bf16x8 pb[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int t = s4 >> 1, i0 = 2 * (s4 & 1);
            union { uint32_t u[4]; bf16x8 v; } pk;
            pk.u[0] = pack2bf(st[t][i0 * 4 + 0], st[t][i0 * 4 + 1]);
            pk.u[1] = pack2bf(st[t][i0 * 4 + 2], st[t][i0 * 4 + 3]);
            pk.u[2] = pack2bf(st[t][i0 * 4 + 4], st[t][i0 * 4 + 5]);
            pk.u[3] = pack2bf(st[t][i0 * 4 + 6], st[t][i0 * 4 + 7]);
            pb[s4] = pk.v;
        }

        // ---- O^T += V^T P^T
#pragma unroll
        for (int ht = 0; ht < 8; ++ht) {
            const int row = ht * 32 + (lane & 31);
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                int ch = (2 * s4 + (lane >> 5)) ^ vswz(row);
                bf16x8 a = *reinterpret_cast<const bf16x8*>(sV + row * KT + ch * 8);
                o[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s4], o[ht], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---- normalise and store: lane has query q0 + (lane & 31), head dims ht*32 + i*8 + 4 (lane>>5) + j
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.f / l_tot;
    const int q = q0 + (lane & 31);
    if (q < S) {
        bf16_t* orow = O + (long)g.row_of(b, q) * d + h * HD + (lane >> 5) * 4;
#pragma unroll
        for (int ht = 0; ht < 8; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint2 v = make_uint2(pack2bf(o[ht][i * 4 + 0] * inv, o[ht][i * 4 + 1] * inv),
                                     pack2bf(o[ht][i * 4 + 2] * inv, o[ht][i * 4 + 3] * inv));
                *reinterpret_cast<uint2*>(orow + ht * 32 + i * 8) = v;
            }
    }
}

hipError_t attention_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* vt, const float* bias, RowGeom g,
                          int H, int S_pad, bf16_t* o, int d, hipStream_t s) {
    int S = g.S();
    if (g.B == 0 || S == 0) return hipSuccess;
    const float scale_log2 = 1.4426950408889634f / 16.0f;  // log2(e) / sqrt(256)
    dim3 grid((S + QT - 1) / QT, H, g.B);
    hipLaunchKernelGGL(k_attention_bf16, grid, dim3(256), 0, s, q, k, vt, bias, g, H, S_pad, o, d, scale_log2);
    return hipGetLastError();
}

}  // namespace af

// fp32 kernels for the full-precision configuration (any width, head_dim <= 64):
// a tiled GEMM with the residual-stream epilogues and a one-query-per-thread
// attention with online softmax. Same contractions as the bf16 path, without
// bf16 rounding anywhere.
#include "af_internal.h"

namespace af {

namespace {
constexpr int FB = 64;   // block tile (rows and columns)
constexpr int FK = 16;   // k step
}

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmLaunch L) {
    __shared__ float sA[FK][FB + 1];
    __shared__ float sW[FK][FB + 1];
    const int tiles_n = (L.N + FB - 1) / FB;
    int bid = blockIdx.x;
    const int t0 = ((L.g[0].M + FB - 1) / FB) * tiles_n;
    const int gi = bid >= t0 ? 1 : 0;
    if (gi) bid -= t0;
    const float* A = (const float*)(gi ? L.g[1].A : L.g[0].A);
    const long lda = gi ? L.g[1].lda : L.g[0].lda;
    const float* W = (const float*)(gi ? L.g[1].W : L.g[0].W);
    const long ldw = gi ? L.g[1].ldw : L.g[0].ldw;
    const int M = gi ? L.g[1].M : L.g[0].M;
    const int row0 = gi ? L.g[1].row0 : L.g[0].row0;
    const int gate_off = gi ? L.g[1].gate_off : L.g[0].gate_off;
    const int m0 = (bid / tiles_n) * FB, n0 = (bid % tiles_n) * FB;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < L.K; k0 += FK) {
        for (int i = threadIdx.x; i < FB * FK; i += 256) {
            int r = i / FK, kk = i % FK;
            int gm = m0 + r, gn = n0 + r, gk = k0 + kk;
            sA[kk][r] = (gm < M && gk < L.K) ? A[(long)gm * lda + gk] : 0.f;
            sW[kk][r] = (gn < L.N && gk < L.K) ? W[(long)gn * ldw + gk] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < FK; ++kk) {
            float a[4], w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = sW[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * w[j];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int m = m0 + ty * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int n = n0 + tx * 4 + j;
            if (n >= L.N) continue;
            float v = acc[i][j];
            if constexpr (EPI == EPI_STORE) {
                ((float*)L.C)[(long)(row0 + m) * L.ldc + n] = v;
            } else if constexpr (EPI == EPI_STORE_MAPPED) {
                long orow = (long)(m / L.seg_len) * L.seg_stride + L.seg_off + m % L.seg_len;
                L.resid[orow * L.N + n] = v;
            } else if constexpr (EPI == EPI_GATED_RESID) {
                int rr = row0 + m;
                const float* gate = L.mod + (long)L.geom.batch_of(rr) * L.mod_stride + gate_off;
                L.resid[(long)rr * L.N + n] += gate[n] * v;
            }
        }
    }
}

hipError_t gemm_f32(const GemmLaunch& L, hipStream_t s) {
    int tiles_n = (L.N + FB - 1) / FB;
    int total = 0;
    for (int i = 0; i < L.ngroups; ++i) total += ((L.g[i].M + FB - 1) / FB) * tiles_n;
    if (total == 0) return hipSuccess;
    GemmLaunch LL = L;
    if (LL.ngroups < 2) LL.g[1] = LL.g[0], LL.g[1].M = 0;
    if (LL.g[0].M == 0) {
        LL.g[0] = LL.g[1];
        LL.g[1].M = 0;
    }
    dim3 grid(total), block(256);
    switch (L.epi) {
        case EPI_STORE: hipLaunchKernelGGL(k_gemm_f32<EPI_STORE>, grid, block, 0, s, LL); break;
        case EPI_STORE_MAPPED: hipLaunchKernelGGL(k_gemm_f32<EPI_STORE_MAPPED>, grid, block, 0, s, LL); break;
        case EPI_GATED_RESID: hipLaunchKernelGGL(k_gemm_f32<EPI_GATED_RESID>, grid, block, 0, s, LL); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- attention (fp32)
constexpr int FA_MAXHD = 64;
constexpr int FA_KT = 64;

__global__ __launch_bounds__(64) void k_attention_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, const float* __restrict__ bias,
                                                      RowGeom g, int H, int hd, int S_pad,
                                                      float* __restrict__ O, int d, float scale) {
    __shared__ float sK[FA_KT][FA_MAXHD];
    __shared__ float sV[FA_KT][FA_MAXHD];
    __shared__ float sB[FA_KT];
    const int b = blockIdx.z, h = blockIdx.y;
    const int S = g.S();
    const int q = blockIdx.x * 64 + threadIdx.x;
    const long bh = (long)b * H + h;
    float qv[FA_MAXHD], acc[FA_MAXHD];
#pragma unroll
    for (int t = 0; t < FA_MAXHD; ++t) {
        qv[t] = (t < hd && q < S) ? Q[(bh * S_pad + q) * hd + t] : 0.f;
        acc[t] = 0.f;
    }
    float m_run = -INFINITY, l_run = 0.f;
    for (int k0 = 0; k0 < S; k0 += FA_KT) {
        for (int i = threadIdx.x; i < FA_KT * hd; i += 64) {
            int r = i / hd, t = i % hd;
            int key = k0 + r;
            sK[r][t] = key < S ? K[(bh * S_pad + key) * hd + t] : 0.f;
            sV[r][t] = key < S ? V[(bh * S_pad + key) * hd + t] : 0.f;
        }
        sB[threadIdx.x] = (k0 + threadIdx.x < S) ? bias[(long)b * S_pad + k0 + threadIdx.x] : -INFINITY;
        __syncthreads();
        for (int r = 0; r < FA_KT; ++r) {
            if (sB[r] == -INFINITY) continue;
            float sdot = 0.f;
#pragma unroll
            for (int t = 0; t < FA_MAXHD; ++t)
                if (t < hd) sdot += qv[t] * sK[r][t];
            float logit = sdot * scale;
            float m_new = fmaxf(m_run, logit);
            float alpha = expf(m_run - m_new);
            float p = expf(logit - m_new);
            l_run = l_run * alpha + p;
#pragma unroll
            for (int t = 0; t < FA_MAXHD; ++t)
                if (t < hd) acc[t] = acc[t] * alpha + p * sV[r][t];
            m_run = m_new;
        }
        __syncthreads();
    }
    if (q >= S) return;
    float* orow = O + (long)g.row_of(b, q) * d + h * hd;
    for (int t = 0; t < hd; ++t) orow[t] = acc[t] / l_run;
}

hipError_t attention_f32(const float* q, const float* k, const float* v, const float* bias, RowGeom g, int H, int hd,
                         int S_pad, float* o, int d, hipStream_t s) {
    int S = g.S();
    if (g.B == 0 || S == 0) return hipSuccess;
    dim3 grid((S + 63) / 64, H, g.B);
    hipLaunchKernelGGL(k_attention_f32, grid, dim3(64), 0, s, q, k, v, bias, g, H, hd, S_pad, o, d,
                       1.0f / sqrtf((float)hd));
    return hipGetLastError();
}

}  // namespace af

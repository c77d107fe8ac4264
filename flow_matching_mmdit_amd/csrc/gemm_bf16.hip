// bf16 MFMA GEMM for gfx950: C = A W^T, A [M, K] and W [N, K] both K-contiguous,
// fp32 accumulation in v_mfma_f32_32x32x16_bf16, with the transformer's
// epilogues fused into the store:
//   STORE          bf16 C (row row0 + m)
//   STORE_MAPPED   fp32 rows of the residual stream (caption projection)
//   GATED_RESID    residual += gate * acc  (adaLN-Zero gated residual, [TRANS]
//                  核心子模块架构: gate 缩放 after attention and after the FFN)
//   QKV            QK-norm (per-head LayerNorm over the 256 head columns,
//                  [TRANS] 注意力处理器与 QKV 融合) and scatter of q, k to
//                  [B, H, S_pad, 256] and v to v^T [B, H, 256, S_pad]
//   SWIGLU         silu(gate) * up of the interleaved FFN columns
//                  ([PIPE] 深入源码, 前馈网络)
//
// Tiling: 256 x 256 block tile, BK = 64, four waves in a 2 x 2 arrangement, each
// wave owning a 128 x 128 sub-tile (4 x 4 MFMA tiles, 256 fp32 accumulators per
// lane). A and W tiles are staged through LDS with two stages (128 KB); 16-byte
// chunks are XOR-swizzled by row so the MFMA operand reads are bank-conflict
// free. Up to two row groups with different weights share one launch (the joint
// blocks' text and image streams).
#include "af_internal.h"

namespace af {

namespace {
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int TILE_ELEMS = BM * BK;  // bf16 elements of one staged A (or W) tile

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ int tiles_m(int M) { return (M + BM - 1) / BM; }
}  // namespace

template <int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_bf16(GemmLaunch L) {
    __shared__ __attribute__((aligned(16))) bf16_t smem[2 * 2 * TILE_ELEMS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_n = L.N / BN;

    int bid = blockIdx.x;
    const int t0 = tiles_m(L.g[0].M) * tiles_n;
    const int gi = bid >= t0 ? 1 : 0;
    if (gi) bid -= t0;
    const bf16_t* __restrict__ A = (const bf16_t*)(gi ? L.g[1].A : L.g[0].A);
    const long lda = gi ? L.g[1].lda : L.g[0].lda;
    const bf16_t* __restrict__ W = (const bf16_t*)(gi ? L.g[1].W : L.g[0].W);
    const long ldw = gi ? L.g[1].ldw : L.g[0].ldw;
    const int M = gi ? L.g[1].M : L.g[0].M;
    const int row0 = gi ? L.g[1].row0 : L.g[0].row0;
    const int gate_off = gi ? L.g[1].gate_off : L.g[0].gate_off;

    const int tn = bid % tiles_n, tm = bid / tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = L.K;

    uint4 ra[8], rb[8];
    auto gload = [&](int k0) {
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            int r = p * 32 + (tid >> 3);
            int gr = min(m0 + r, M - 1);
            ra[p] = *reinterpret_cast<const uint4*>(A + (long)gr * lda + k0 + (tid & 7) * 8);
            rb[p] = *reinterpret_cast<const uint4*>(W + (long)(n0 + r) * ldw + k0 + (tid & 7) * 8);
        }
    };
    auto sstore = [&](int stage) {
        bf16_t* sA = smem + stage * 2 * TILE_ELEMS;
        bf16_t* sB = sA + TILE_ELEMS;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            int r = p * 32 + (tid >> 3);
            int c = (tid & 7) ^ swz(r);
            *reinterpret_cast<uint4*>(sA + r * BK + c * 8) = ra[p];
            *reinterpret_cast<uint4*>(sB + r * BK + c * 8) = rb[p];
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    auto compute = [&](int stage) {
        const bf16_t* sA = smem + stage * 2 * TILE_ELEMS;
        const bf16_t* sB = sA + TILE_ELEMS;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 a[4], b[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                int r = wm * 128 + mt * 32 + (lane & 31);
                int c = (ks * 2 + (lane >> 5)) ^ swz(r);
                a[mt] = *reinterpret_cast<const bf16x8*>(sA + r * BK + c * 8);
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                int r = wn * 128 + nt * 32 + (lane & 31);
                int c = (ks * 2 + (lane >> 5)) ^ swz(r);
                b[nt] = *reinterpret_cast<const bf16x8*>(sB + r * BK + c * 8);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
        }
    };

    const int KT = K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) gload((kt + 1) * BK);
        compute(kt & 1);
        if (kt + 1 < KT) sstore((kt + 1) & 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogues
    // acc[mt][nt][i*4+j] holds row wm*128 + mt*32 + i*8 + (lane>>5)*4 + j,
    // column wn*128 + nt*32 + (lane&31) of the block tile.
    const int lr_base = wm * 128 + (lane >> 5) * 4;
    const int lc_base = wn * 128 + (lane & 31);

    if constexpr (EPI == EPI_STORE) {
        bf16_t* C = (bf16_t*)L.C;
#pragma unroll 1
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int m = m0 + lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
                if (m >= M) continue;
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) C[(long)(row0 + m) * L.ldc + n0 + lc_base + nt * 32] = f2bf(acc[mt][nt][r]);
            }
    } else if constexpr (EPI == EPI_STORE_MAPPED) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int m = m0 + lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
                if (m >= M) continue;
                long orow = (long)(m / L.seg_len) * L.seg_stride + L.seg_off + m % L.seg_len;
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) L.resid[orow * L.N + n0 + lc_base + nt * 32] = acc[mt][nt][r];
            }
    } else if constexpr (EPI == EPI_GATED_RESID) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int m = m0 + lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
                if (m >= M) continue;
                int rr = row0 + m;
                const float* gate = L.mod + (long)L.geom.batch_of(rr) * L.mod_stride + gate_off;
                float* xrow = L.resid + (long)rr * L.N;
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    int n = n0 + lc_base + nt * 32;
                    xrow[n] += gate[n] * acc[mt][nt][r];
                }
            }
    } else if constexpr (EPI == EPI_SWIGLU) {
        bf16_t* Hout = (bf16_t*)L.C;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int m = m0 + lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
                if (m >= M) continue;
#pragma unroll
                for (int p2 = 0; p2 < 2; ++p2) {
                    float gt = acc[mt][2 * p2][r], up = acc[mt][2 * p2 + 1][r];
                    int f = (n0 + wn * 128 + p2 * 64) / 2 + (lane & 31);
                    Hout[(long)(row0 + m) * L.ldc + f] = f2bf(silu_f(gt) * up);
                }
            }
    } else if constexpr (EPI == EPI_QKV) {
        const int dmodel = L.N / 3;
        const int which = n0 / dmodel;          // 0 q, 1 k, 2 v
        const int head = (n0 % dmodel) / BN;    // one block tile = one 256-wide head
        const int H = L.H, S_pad = L.S_pad;
        if (which < 2) {
            // Per-row LayerNorm over the 256 head columns, split across the two wn
            // waves; row statistics live in LDS (free after the main loop).
            float* rsum = reinterpret_cast<float*>(smem);   // [2][256] partial sums
            float* rsq = rsum + 512;                         // [2][256] partial centred squares
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float s = (acc[mt][0][r] + acc[mt][1][r]) + (acc[mt][2][r] + acc[mt][3][r]);
                    s = half_wave_sum(s);
                    if ((lane & 31) == 0) rsum[wn * 256 + lr_base + mt * 32 + (r >> 2) * 8 + (r & 3)] = s;
                }
            __syncthreads();
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    int lr = lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
                    float mean = (rsum[lr] + rsum[256 + lr]) * (1.f / 256.f);
                    float s = 0.f;
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        float c = acc[mt][nt][r] - mean;
                        s += c * c;
                    }
                    s = half_wave_sum(s);
                    if ((lane & 31) == 0) rsq[wn * 256 + lr] = s;
                }
            __syncthreads();
            bf16_t* dst = (bf16_t*)(which == 0 ? L.q : L.k);
#pragma unroll 1
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    int lr = lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
                    int m = m0 + lr;
                    if (m >= M) continue;
                    float mean = (rsum[lr] + rsum[256 + lr]) * (1.f / 256.f);
                    float rstd = rsqrtf((rsq[lr] + rsq[256 + lr]) * (1.f / 256.f) + L.eps);
                    int rr = row0 + m;
                    int b = L.geom.batch_of(rr), s_ = L.geom.seq_of(rr);
                    bf16_t* drow = dst + (((long)b * H + head) * S_pad + s_) * 256;
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        drow[lc_base + nt * 32] = f2bf((acc[mt][nt][r] - mean) * rstd);
                }
        } else {
            bf16_t* vt = (bf16_t*)L.vt;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    int m = m0 + lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
                    if (m >= M) continue;
                    int rr = row0 + m;
                    int b = L.geom.batch_of(rr), s_ = L.geom.seq_of(rr);
                    bf16_t* base = vt + ((long)b * H + head) * 256 * (long)S_pad + s_;
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        base[(long)(lc_base + nt * 32) * S_pad] = f2bf(acc[mt][nt][r]);
                }
        }
    }
}

hipError_t gemm_bf16(const GemmLaunch& L, hipStream_t s) {
    int tiles_n = L.N / BN;
    int total = 0;
    for (int i = 0; i < L.ngroups; ++i) total += ((L.g[i].M + BM - 1) / BM) * tiles_n;
    if (total == 0) return hipSuccess;
    GemmLaunch LL = L;
    if (LL.ngroups < 2) LL.g[1] = LL.g[0], LL.g[1].M = 0;
    if (LL.g[0].M == 0) {  // keep group 0 non-empty so the tile split is simple
        LL.g[0] = LL.g[1];
        LL.g[1].M = 0;
    }
    dim3 grid(total), block(256);
    switch (L.epi) {
        case EPI_STORE: hipLaunchKernelGGL(k_gemm_bf16<EPI_STORE>, grid, block, 0, s, LL); break;
        case EPI_STORE_MAPPED: hipLaunchKernelGGL(k_gemm_bf16<EPI_STORE_MAPPED>, grid, block, 0, s, LL); break;
        case EPI_GATED_RESID: hipLaunchKernelGGL(k_gemm_bf16<EPI_GATED_RESID>, grid, block, 0, s, LL); break;
        case EPI_QKV: hipLaunchKernelGGL(k_gemm_bf16<EPI_QKV>, grid, block, 0, s, LL); break;
        case EPI_SWIGLU: hipLaunchKernelGGL(k_gemm_bf16<EPI_SWIGLU>, grid, block, 0, s, LL); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace af

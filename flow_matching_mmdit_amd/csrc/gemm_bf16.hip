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
// Tiling: 256 x 256 block tile, BK = 64, eight waves (two per SIMD) in a 4 x 2
// arrangement, each wave owning a 64 x 128 sub-tile (2 x 4 MFMA tiles, 128 fp32
// accumulators per lane). A and W tiles move global -> LDS with the gfx950
// direct loads (global_load_lds_dwordx4: lane i writes LDS bytes [16 i, 16 i + 16)
// of the instruction's 1 KB block), two stages; the XOR swizzle of 16-byte chunks
// is applied by choosing which global chunk each lane fetches, so the MFMA
// operand reads (ds_read_b128) are bank-conflict free. Operand fragments are
// register double-buffered so LDS reads of k-step ks + 1 overlap the MFMAs of ks.
// Blocks are mapped to tiles XCD by XCD (consecutive block ids go to different
// XCDs) and, inside an XCD, in groups of four tile rows so co-resident blocks
// share A and W panels in that XCD's L2. Up to two row groups with different
// weights share one launch (the joint blocks' text and image streams).
// Epilogues that write bf16 stage the tile in LDS and store 16-byte chunks.
#include "af_internal.h"

namespace af {

namespace {
constexpr int BM = 256, BN = 256;
#ifndef GEMM_BK
#define GEMM_BK 64      // k depth of one staged tile (64 or 32)
#endif
#ifndef GEMM_STAGES
#define GEMM_STAGES 2   // LDS stages (prefetch distance STAGES - 1 tiles)
#endif
constexpr int BK = GEMM_BK, STAGES = GEMM_STAGES;
constexpr int CH = BK / 8;             // 16-byte chunks per tile row
constexpr int RPI = 1024 / (BK * 2);   // tile rows per 1 KB direct-load instruction
constexpr int TILE_ELEMS = BM * BK;    // bf16 elements of one staged A (or W) tile
static_assert(2 * STAGES * TILE_ELEMS <= 4 * 64 * 256, "operand stages exceed 128 KB");
constexpr int NXCD = 8;              // MI355X: 8 XCDs, blocks dispatched round-robin
constexpr int GROUP_M = 8;
#ifndef GEMM_WM
#define GEMM_WM 4   // waves along M
#endif
#ifndef GEMM_WN
#define GEMM_WN 2   // waves along N
#endif
constexpr int QS = 264;              // QKV epilogue staging row stride (elements)
constexpr int HS = 136;              // SwiGLU epilogue staging row stride (elements)
constexpr int SMEM_ELEMS = 256 * QS + 2048;   // >= 4 tiles; + [2][256] x 2 fp32 row statistics

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Chunk swizzle per row so the 32 rows one MFMA operand read touches spread over
// all banks (both for 8- and 16-lane LDS issue groups).
__device__ __forceinline__ int swz(int row) {
    if constexpr (BK == 64) return (row & 7) ^ ((row >> 3) & 1);
    else return ((row >> 1) ^ (row >> 3)) & 3;
}
// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
__host__ __device__ __forceinline__ int tiles_m(int M) { return (M + BM - 1) / BM; }

// Issues this wave's share of one 256 x BK tile starting at `tile` (uniform): the
// tile is 256 / RPI blocks of 1 KB (RPI rows each); with NW waves, wave w issues
// blocks cb = w * PER + j. Lane l fills physical chunk l % CH of row
// RPI cb + l / CH with logical chunk (l % CH) ^ swz(row). swz depends on cb only
// through its parity, so two per-lane offsets (off[j & 1]) plus a uniform row
// step cover all of the wave's instructions.
template <int NW>
__device__ __forceinline__ void issue_tile(const bf16_t* tile, const uint32_t* off, long ld, bf16_t* lds_tile,
                                           int wave) {
    constexpr int PER = (BM / RPI) / NW;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const bf16_t* src = tile + (long)(j & ~1) * RPI * ld + off[j & 1];
        __builtin_amdgcn_global_load_lds((glb_void*)src, (lds_void*)(lds_tile + (wave * PER + j) * 512), 16, 0, 0);
    }
}
}  // namespace

// WM x WN waves; each wave owns a (256 / WM) x (256 / WN) sub-tile.
template <int EPI, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4)))
void k_gemm_bf16(GemmLaunch L) {
    constexpr int NW = WM * WN, NTHR = NW * 64;
    constexpr int TM = BM / WM, TN = BN / WN, MT = TM / 32, NT = TN / 32;
    static_assert(SMEM_ELEMS >= 2 * STAGES * TILE_ELEMS, "LDS");
    static_assert(((BM / RPI) / NW) % 2 == 0, "per-wave load count must be even");
    __shared__ __attribute__((aligned(1024))) bf16_t smem[SMEM_ELEMS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int tiles_n = L.N / BN;

    // ---- block -> (group, tile row, tile column)
    const int tm0 = tiles_m(L.g[0].M), tm1 = L.ngroups > 1 ? tiles_m(L.g[1].M) : 0;
    const int T0 = tm0 * tiles_n, T = T0 + tm1 * tiles_n;
    int lid;
    {
        const int b = blockIdx.x, x = b % NXCD, q = T / NXCD, r = T % NXCD;
        lid = x * q + min(x, r) + b / NXCD;
    }
    const int gi = lid >= T0 ? 1 : 0;
    if (gi) lid -= T0;
    const int tmg = gi ? tm1 : tm0;
    int tm, tn;
    {
        const int per = GROUP_M * tiles_n;
        const int gblk = lid / per, idx = lid % per;
        const int gm = min(GROUP_M, tmg - gblk * GROUP_M);
        tm = gblk * GROUP_M + idx % gm;
        tn = idx / gm;
    }
    const bf16_t* __restrict__ A = (const bf16_t*)(gi ? L.g[1].A : L.g[0].A);
    const long lda = gi ? L.g[1].lda : L.g[0].lda;
    const bf16_t* __restrict__ W = (const bf16_t*)(gi ? L.g[1].W : L.g[0].W);
    const long ldw = gi ? L.g[1].ldw : L.g[0].ldw;
    const int M = gi ? L.g[1].M : L.g[0].M;
    const int row0 = gi ? L.g[1].row0 : L.g[0].row0;
    const int gate_off = gi ? L.g[1].gate_off : L.g[0].gate_off;
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = L.K;

    // Per-lane element offsets for the direct loads (logical chunk folded in). Rows
    // past M read the padding rows every activation buffer carries (at least one
    // tile of rows past its last real row); their results are never stored.
    uint32_t aoff[2], woff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = (wave * ((BM / RPI) / NW) + j) * RPI + lane / CH;
        const int c = (lane % CH) ^ swz(r);
        aoff[j] = (uint32_t)(r * lda + c * 8);
        woff[j] = (uint32_t)(r * ldw + c * 8);
    }
    const bf16_t* Atile = A + (long)m0 * lda;
    const bf16_t* Wtile = W + (long)n0 * ldw;

    f32x16 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // MFMA operands for k-step ks come from LDS one step ahead (register double
    // buffer), so the reads of step ks + 1 overlap the MFMAs of step ks.
    auto load_frags = [&](const bf16_t* sA, const bf16_t* sB, int ks, bf16x8* a, bf16x8* b) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            int r = wm * TM + mt * 32 + (lane & 31);
            int c = (ks * 2 + (lane >> 5)) ^ swz(r);
            a[mt] = *reinterpret_cast<const bf16x8*>(sA + r * BK + c * 8);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            int r = wn * TN + nt * 32 + (lane & 31);
            int c = (ks * 2 + (lane >> 5)) ^ swz(r);
            b[nt] = *reinterpret_cast<const bf16x8*>(sB + r * BK + c * 8);
        }
    };
    // `side(ks)` runs at the top of each k-step (used to spread the next tile's loads).
    auto compute = [&](const bf16_t* sA, const bf16_t* sB, auto&& side) {
        bf16x8 a[2][MT], b[2][NT];
        load_frags(sA, sB, 0, a[0], b[0]);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            side(ks);
            if (ks + 1 < BK / 16) load_frags(sA, sB, ks + 1, a[(ks + 1) & 1], b[(ks + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);   // keep the reads of step ks + 1 ahead of these MFMAs
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks & 1][mt], b[ks & 1][nt], acc[mt][nt],
                                                                          0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- main loop: STAGES LDS stages. Tile kt + STAGES - 1 streams into the
    // stage read in iteration kt - 1 while tile kt is multiplied. At the end of an
    // iteration each wave waits until its loads of tile kt + 1 have landed (the
    // loads of later tiles may stay in flight) and the barrier publishes them.
    constexpr int PER2 = 2 * ((BM / RPI) / NW);     // direct loads per wave per tile
    const int KT = K / BK;
    auto stage_ptr = [&](int st) { return smem + st * 2 * TILE_ELEMS; };
    auto issue = [&](int t) {
        bf16_t* dst = stage_ptr(t % STAGES);
        issue_tile<NW>(Atile + t * BK, aoff, lda, dst, wave);
        issue_tile<NW>(Wtile + t * BK, woff, ldw, dst + TILE_ELEMS, wave);
    };
    auto wait_landed = [&](int later) {   // `later` = tiles issued after the one needed
        if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER2));
        else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER2));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_barrier();
    };
    static_assert(STAGES <= 4, "wait_landed covers at most two later tiles");
#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t)
        if (t < KT) issue(t);
    wait_landed(min(STAGES - 2, KT - 1));
    for (int kt = 0; kt < KT; ++kt) {
        // The next tile's direct loads are spread over the k-steps of this tile's
        // MFMAs rather than issued in one burst.
        const int tnext = kt + STAGES - 1;
        const bool more = tnext < KT;
        const bf16_t* cur = stage_ptr(kt % STAGES);
        bf16_t* dst = stage_ptr(tnext % STAGES);
        constexpr int PER = (BM / RPI) / NW;
        constexpr int KS = BK / 16;
        static_assert(PER % KS == 0, "loads per k-step");
        compute(cur, cur + TILE_ELEMS, [&](int ks) {
            if (!more) return;
#pragma unroll
            for (int jj = 0; jj < PER / KS; ++jj) {
                const int j = ks * (PER / KS) + jj;
                __builtin_amdgcn_global_load_lds(
                    (glb_void*)(Atile + tnext * BK + (long)(j & ~1) * RPI * lda + aoff[j & 1]),
                    (lds_void*)(dst + (wave * PER + j) * 512), 16, 0, 0);
                __builtin_amdgcn_global_load_lds(
                    (glb_void*)(Wtile + tnext * BK + (long)(j & ~1) * RPI * ldw + woff[j & 1]),
                    (lds_void*)(dst + TILE_ELEMS + (wave * PER + j) * 512), 16, 0, 0);
            }
        });
        // tiles issued after kt + 1: kt + 2 .. min(kt + STAGES - 1, KT - 1)
        wait_landed(max(0, min(kt + STAGES - 1, KT - 1) - (kt + 1)));
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---------------------------------------------------------------- epilogues
    // acc[mt][nt][i*4+j] holds row wm*128 + mt*32 + i*8 + (lane>>5)*4 + j,
    // column wn*128 + nt*32 + (lane&31) of the block tile. LDS is free here.
    const int lr_base = wm * TM + (lane >> 5) * 4;
    const int lc_base = wn * TN + (lane & 31);

    if constexpr (EPI == EPI_STORE) {
        bf16_t* C = (bf16_t*)L.C;
#pragma unroll 1
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int m = m0 + lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
                if (m >= M) continue;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) C[(long)(row0 + m) * L.ldc + n0 + lc_base + nt * 32] = f2bf(acc[mt][nt][r]);
            }
    } else if constexpr (EPI == EPI_STORE_MAPPED) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int m = m0 + lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
                if (m >= M) continue;
                long orow = (long)(m / L.seg_len) * L.seg_stride + L.seg_off + m % L.seg_len;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) L.resid[orow * L.N + n0 + lc_base + nt * 32] = acc[mt][nt][r];
            }
    } else if constexpr (EPI == EPI_GATED_RESID) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int m = m0 + lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
                if (m >= M) continue;
                int rr = row0 + m;
                const float* gate = L.mod + (long)L.geom.batch_of(rr) * L.mod_stride + gate_off;
                float* xrow = L.resid + (long)rr * L.N;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    int n = n0 + lc_base + nt * 32;
                    xrow[n] += gate[n] * acc[mt][nt][r];
                }
            }
    } else if constexpr (EPI == EPI_SWIGLU) {
        // h tile [256 rows][128 cols] bf16 staged in LDS, then 16-byte row stores.
        bf16_t* st = smem;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int lr = lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
#pragma unroll
                for (int p2 = 0; p2 < NT / 2; ++p2) {
                    float gt = acc[mt][2 * p2][r], up = acc[mt][2 * p2 + 1][r];
                    st[lr * HS + wn * (TN / 2) + p2 * 32 + (lane & 31)] = f2bf(silu_f(gt) * up);
                }
            }
        __syncthreads();
        bf16_t* Hout = (bf16_t*)L.C;
        const int fcol0 = n0 / 2;
#pragma unroll 4
        for (int it = 0; it < 4096 / NTHR; ++it) {
            int idx = it * NTHR + tid;         // 256 rows x 16 chunks
            int lr = idx >> 4, ch = idx & 15;
            int m = m0 + lr;
            if (m < M) {
                uint4 v = *reinterpret_cast<const uint4*>(st + lr * HS + ch * 8);
                *reinterpret_cast<uint4*>(Hout + (long)(row0 + m) * L.ldc + fcol0 + ch * 8) = v;
            }
        }
    } else if constexpr (EPI == EPI_QKV) {
        const int dmodel = L.N / 3;
        const int which = n0 / dmodel;          // 0 q, 1 k, 2 v
        const int head = (n0 % dmodel) / BN;    // one block tile = one 256-wide head
        const int H = L.H, S_pad = L.S_pad;
        // Output tile [256 rows][256 cols] bf16 staged in LDS (row stride QS).
        bf16_t* st = smem;
        float* rsum = reinterpret_cast<float*>(smem + 256 * QS);   // [WN][256]
        float* rsq = rsum + WN * 256;                               // [WN][256]
        if (which < 2) {
            // Per-row LayerNorm over the 256 head columns, split across the two wn waves.
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float s = 0.f;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) s += acc[mt][nt][r];
                    s = half_wave_sum(s);
                    if ((lane & 31) == 0) rsum[wn * 256 + lr_base + mt * 32 + (r >> 2) * 8 + (r & 3)] = s;
                }
            __syncthreads();
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    int lr = lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
                    float tot = 0.f;
#pragma unroll
                    for (int w = 0; w < WN; ++w) tot += rsum[w * 256 + lr];
                    float mean = tot * (1.f / 256.f);
                    float s = 0.f;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        float c = acc[mt][nt][r] - mean;
                        s += c * c;
                    }
                    s = half_wave_sum(s);
                    if ((lane & 31) == 0) rsq[wn * 256 + lr] = s;
                }
            __syncthreads();
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    int lr = lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
                    float tot = 0.f, tsq = 0.f;
#pragma unroll
                    for (int w = 0; w < WN; ++w) tot += rsum[w * 256 + lr], tsq += rsq[w * 256 + lr];
                    float mean = tot * (1.f / 256.f);
                    float rstd = rsqrtf(tsq * (1.f / 256.f) + L.eps);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        st[lr * QS + lc_base + nt * 32] = f2bf((acc[mt][nt][r] - mean) * rstd);
                }
            __syncthreads();
            // rows -> [B, H, S_pad, 256]: 32 chunks of 16 B per row
            bf16_t* dst = (bf16_t*)(which == 0 ? L.q : L.k);
#pragma unroll 4
            for (int it = 0; it < 8192 / NTHR; ++it) {
                int idx = it * NTHR + tid;
                int lr = idx >> 5, ch = idx & 31;
                int m = m0 + lr;
                if (m < M) {
                    int rr = row0 + m;
                    int b = L.geom.batch_of(rr), s_ = L.geom.seq_of(rr);
                    uint4 v = *reinterpret_cast<const uint4*>(st + lr * QS + ch * 8);
                    *reinterpret_cast<uint4*>(dst + (((long)b * H + head) * S_pad + s_) * 256 + ch * 8) = v;
                }
            }
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    int lr = lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) st[lr * QS + lc_base + nt * 32] = f2bf(acc[mt][nt][r]);
                }
            __syncthreads();
            // v^T: for head column c, 8 consecutive tile rows -> 8 consecutive keys (one
            // 16-byte store) when they lie in one sample's segment and start 8-aligned;
            // otherwise element stores.
            bf16_t* vt = (bf16_t*)L.vt;
#pragma unroll 2
            for (int it = 0; it < 8192 / NTHR; ++it) {
                int idx = it * NTHR + tid;             // 256 columns x 32 row-chunks
                int c = idx & 255, rc = idx >> 8;
                int lr0 = rc * 8;
                int m = m0 + lr0;
                if (m >= M) continue;
                int rr = row0 + m;
                int b = L.geom.batch_of(rr), s0 = L.geom.seq_of(rr);
                bool fast = (m + 7 < M) && (s0 % 8 == 0) && L.geom.batch_of(rr + 7) == b &&
                            L.geom.seq_of(rr + 7) == s0 + 7;
                if (fast) {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = (uint32_t)st[(lr0 + 2 * e) * QS + c] | ((uint32_t)st[(lr0 + 2 * e + 1) * QS + c] << 16);
                    bf16_t* base = vt + (((long)b * H + head) * 256 + c) * (long)S_pad;
                    *reinterpret_cast<uint4*>(base + s0) = make_uint4(w[0], w[1], w[2], w[3]);
                } else {
                    for (int e = 0; e < 8 && m + e < M; ++e) {
                        int re = rr + e;
                        int be = L.geom.batch_of(re), se = L.geom.seq_of(re);
                        vt[(((long)be * H + head) * 256 + c) * (long)S_pad + se] = st[(lr0 + e) * QS + c];
                    }
                }
            }
        }
    }
}

hipError_t gemm_bf16(const GemmLaunch& L, hipStream_t s) {
    int tiles_n = L.N / BN;
    GemmLaunch LL = L;
    if (LL.ngroups == 2 && LL.g[0].M == 0) {  // keep group 0 non-empty
        LL.g[0] = LL.g[1];
        LL.ngroups = 1;
    }
    if (LL.ngroups == 2 && LL.g[1].M == 0) LL.ngroups = 1;
    int total = 0;
    for (int i = 0; i < LL.ngroups; ++i) total += tiles_m(LL.g[i].M) * tiles_n;
    if (total == 0) return hipSuccess;
    dim3 grid(total), block(GEMM_WM * GEMM_WN * 64);
    switch (L.epi) {
        case EPI_STORE: hipLaunchKernelGGL((k_gemm_bf16<EPI_STORE, GEMM_WM, GEMM_WN>), grid, block, 0, s, LL); break;
        case EPI_STORE_MAPPED:
            hipLaunchKernelGGL((k_gemm_bf16<EPI_STORE_MAPPED, GEMM_WM, GEMM_WN>), grid, block, 0, s, LL);
            break;
        case EPI_GATED_RESID:
            hipLaunchKernelGGL((k_gemm_bf16<EPI_GATED_RESID, GEMM_WM, GEMM_WN>), grid, block, 0, s, LL);
            break;
        case EPI_QKV: hipLaunchKernelGGL((k_gemm_bf16<EPI_QKV, GEMM_WM, GEMM_WN>), grid, block, 0, s, LL); break;
        case EPI_SWIGLU: hipLaunchKernelGGL((k_gemm_bf16<EPI_SWIGLU, GEMM_WM, GEMM_WN>), grid, block, 0, s, LL); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace af

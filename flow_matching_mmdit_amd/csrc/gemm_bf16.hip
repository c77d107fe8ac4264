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
// Tiling: 256 x 256 block tile, eight waves (two per SIMD) in a 4 x 2
// arrangement, each wave owning a 64 x 128 sub-tile (2 x 4 MFMA tiles, 128 fp32
// accumulators per lane). K is consumed in sub-tiles of 32 (two MFMA k-steps)
// that stream global -> LDS through four slots with buffer_load ... lds (lane i
// writes LDS bytes [16 i, 16 i + 16) of the instruction's 1 KB block; the MUBUF
// form keeps the compiler's LDS-read waits partial, where the FLAT form of the
// same direct load makes every LDS wait a full drain). The XOR swizzle of
// 16-byte chunks is applied by choosing which global chunk each lane fetches, so
// the MFMA operand reads (ds_read_b128) are bank-conflict free. The loop is
// rotated so that no k-step starts on an empty register file: the barrier that
// publishes sub-tile j + 1 sits between the two k-steps of sub-tile j, and the
// second k-step's MFMAs run while the first fragments of sub-tile j + 1 load.
// Blocks are mapped to tiles XCD by XCD (consecutive block ids go to different
// XCDs) and, inside an XCD, in groups of row tiles so co-resident blocks share
// A and W panels in that XCD's L2. Up to two row groups with different weights
// share one launch (the joint blocks' text and image streams).
// Epilogues that write bf16 stage the tile in LDS and store 16-byte chunks.
#include "af_internal.h"

namespace af {

namespace {
constexpr int BM = 256, BN = 256;
constexpr int BK = 32;                 // k depth of one LDS sub-tile (two MFMA k-steps)
constexpr int NS = 4;                  // LDS slots (sub-tiles in flight: NS - 1)
constexpr int CH = BK / 8;             // 16-byte chunks per tile row
constexpr int RPI = 1024 / (BK * 2);   // tile rows per 1 KB direct-load instruction
constexpr int TILE_ELEMS = BM * BK;    // bf16 elements of one staged A (or W) sub-tile
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
constexpr int SMEM_ELEMS = 256 * QS + 2048;   // epilogue staging + [2][256] x 2 fp32 row statistics
static_assert(SMEM_ELEMS >= 2 * NS * TILE_ELEMS, "operand slots exceed the LDS block");

typedef __attribute__((address_space(3))) void lds_void;

// Chunk swizzle per row (4 chunks of 16 B per 64-byte row). Rows r and r + 4
// start on the same bank, so the chunk is XORed with bits 2..3 of the row: the
// MFMA operand reads (ds_read_b128) then run conflict free (measured with the
// LDS bank-conflict counter; an XOR with bits 1 and 3 still gave two-way
// conflicts on gfx950).
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }
// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
__host__ __device__ __forceinline__ int tiles_m(int M) { return (M + BM - 1) / BM; }
// MFMA operand order of a tile: false -> acc = A W^T (a lane holds one column and
// four consecutive rows per 4-register group), true -> acc = (W A^T) = C^T (a lane
// holds one row and four consecutive columns), for epilogues that reduce or store
// along rows.
template <bool T> struct Orient { static constexpr bool value = T; };

// Issues this wave's share of one 256 x BK operand sub-tile: the sub-tile is
// 256 / RPI blocks of 1 KB (RPI rows each); with NW waves, wave w issues blocks
// cb = w * PER + j. Lane l fills physical chunk l % CH of row RPI cb + l / CH
// with logical chunk (l % CH) ^ swz(row). swz depends on the row only within
// its 16-row block, so per-lane byte offsets for two blocks (voff[j & 1]) plus a
// uniform row step (in the scalar offset, with the sub-tile's k offset `sbase`)
// cover all of the wave's instructions.
template <int NW>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rsrc, const uint32_t* voff, int sbase, int ldbytes,
                                           bf16_t* lds_tile, int wave) {
    constexpr int PER = (BM / RPI) / NW;
#pragma unroll
    for (int j = 0; j < PER; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds_tile + (wave * PER + j) * 512), 16, voff[j & 1],
                                                 sbase + (j & ~1) * RPI * ldbytes, 0, 0);
}
}  // namespace

// WM x WN waves; each wave owns a (256 / WM) x (256 / WN) sub-tile.
template <int EPI, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4)))
void k_gemm_bf16(GemmLaunch L) {
    constexpr int NW = WM * WN, NTHR = NW * 64;
    constexpr int TM = BM / WM, TN = BN / WN, MT = TM / 32, NT = TN / 32;
    static_assert(((BM / RPI) / NW) % 2 == 0, "per-wave load count must be even");
    __shared__ __attribute__((aligned(1024))) bf16_t smem[SMEM_ELEMS];

    // wave index in a scalar register: the LDS addresses of the direct loads (M0)
    // are then formed with scalar arithmetic
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    // Per-lane byte offsets for the direct loads (logical chunk folded in). Rows
    // past M read the padding rows every activation buffer carries (at least one
    // tile of rows past its last real row); their results are never stored.
    uint32_t aoff[2], woff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = (wave * ((BM / RPI) / NW) + j) * RPI + lane / CH;
        const int c = (lane % CH) ^ swz(r);
        aoff[j] = (uint32_t)((r * lda + c * 8) * 2);
        woff[j] = (uint32_t)((r * ldw + c * 8) * 2);
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
    auto mfmas = [&](const bf16x8* a, const bf16x8* b, auto orient) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if constexpr (decltype(orient)::value)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[nt], a[mt], acc[mt][nt], 0, 0, 0);
                else
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
            }
    };
    // Issue order inside a k-step: the fragment reads for the next k-step, then
    // the MFMAs with the k-step's direct loads slotted in after the first and the
    // third MFMA.
    static_assert(MT * NT == 8 && (BM / RPI) / NW == 2, "issue pattern is laid out for the 4 x 2 wave grid");
    auto pattern = []() {
        __builtin_amdgcn_sched_group_barrier(0x100, MT + NT, 0);   // DS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);         // VMEM (direct load)
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MT * NT - 3, 0);
    };

    // ---- main loop. Sub-tile t lives in slot t % NS. In iteration j:
    //   k-step 0: W half of sub-tile j + NS - 2 -> its slot (held sub-tile j - 2,
    //             released by barrier j - 1); reads of k-step 1; MFMAs of k-step 0
    //   wait until this wave's loads of sub-tile j + 1 and all its LDS reads of
    //   slot j are done; barrier j (publishes sub-tile j + 1, releases slot j - 1)
    //   k-step 1: A half of sub-tile j + NS - 1 -> slot j - 1; reads of sub-tile
    //             j + 1's k-step 0; MFMAs of k-step 1.
    // Loads past the last sub-tile re-read the last one into a free slot, so the
    // loop body has no branches and the wait counts are the same every iteration.
    constexpr int PER = (BM / RPI) / NW;     // direct loads per wave per operand per sub-tile
    constexpr int PER2 = 2 * PER;
    const int KT = K / BK;
    auto slot_ptr = [&](int st) { return smem + st * 2 * TILE_ELEMS; };
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)Atile, (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc((void*)Wtile, (short)0, 0x7fffffff, 0x00020000);
    const int ldab = (int)lda * 2, ldwb = (int)ldw * 2;
    auto issueA = [&](int t, int st) { issue_tile<NW>(rA, aoff, min(t, KT - 1) * BK * 2, ldab, slot_ptr(st), wave); };
    auto issueW = [&](int t, int st) {
        issue_tile<NW>(rW, woff, min(t, KT - 1) * BK * 2, ldwb, slot_ptr(st) + TILE_ELEMS, wave);
    };
    auto mainloop = [&](auto orient) {
    #pragma unroll
        for (int t = 0; t < NS - 2; ++t) {
            issueA(t, t);
            issueW(t, t);
        }
        issueA(NS - 2, NS - 2);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER2 * (NS - 3) + PER));   // sub-tile 0 landed
        __builtin_amdgcn_s_barrier();
        bf16x8 fa0[MT], fb0[NT], fa1[MT], fb1[NT];
        load_frags(slot_ptr(0), slot_ptr(0) + TILE_ELEMS, 0, fa0, fb0);
        int cs = 0;
        for (int j = 0; j < KT; ++j) {
            const bf16_t* cur = slot_ptr(cs);
            const int ns = cs + 1 == NS ? 0 : cs + 1;      // slot of j + 1
            const int fs = cs == 0 ? NS - 1 : cs - 1;      // slot of j - 1
            const int f2 = fs == 0 ? NS - 1 : fs - 1;      // slot of j - 2
            issueW(j + NS - 2, f2);
            load_frags(cur, cur + TILE_ELEMS, 1, fa1, fb1);
            mfmas(fa0, fb0, orient);
            pattern();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER2 * (NS - 3)) & ~(15 << 8));   // and lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            issueA(j + NS - 1, fs);
            const bf16_t* nxt = slot_ptr(ns);
            load_frags(nxt, nxt + TILE_ELEMS, 0, fa0, fb0);
            mfmas(fa1, fb1, orient);
            pattern();
            __builtin_amdgcn_sched_barrier(0);
            cs = ns;
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    // q and k tiles of the QKV GEMM and the SwiGLU tiles run in the row-major
    // (C^T) orientation; everything else in the column-major one.
    if constexpr (EPI == EPI_SWIGLU) {
        mainloop(Orient<true>{});
    } else if constexpr (EPI == EPI_QKV) {
        if (n0 / (L.N / 3) < 2) mainloop(Orient<true>{});
        else mainloop(Orient<false>{});
    } else {
        mainloop(Orient<false>{});
    }

    // ---------------------------------------------------------------- epilogues
    // Column-major orientation: acc[mt][nt][i*4+j] holds row wm*64 + mt*32 + i*8 +
    // (lane>>5)*4 + j, column wn*128 + nt*32 + (lane&31) of the block tile.
    // Row-major orientation: acc[mt][nt][i*4+j] holds row wm*64 + mt*32 + (lane&31),
    // column wn*128 + nt*32 + i*8 + (lane>>5)*4 + j. LDS is free here.
    const int lr_base = wm * TM + (lane >> 5) * 4;
    const int lc_base = wn * TN + (lane & 31);
    const int rr_row = wm * TM + (lane & 31);           // row-major: row of mt = 0
    const int rr_col = wn * TN + (lane >> 5) * 4;       // row-major: column of nt = i = j = 0

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
        // Rows in groups of four (one r >> 2 of one mt): the residual and gate loads
        // of group g + 1 are issued before group g's read-modify-write stores, so a
        // wave keeps two groups of loads in flight rather than one row's.
        float* __restrict__ resid = L.resid;
        const float* __restrict__ mod = L.mod;
        const int ncol = n0 + lc_base;
        constexpr int NG = MT * 4;
        float xv[2][4][NT], gv[2][4][NT];
        auto grow = [&](int g, int j) { return m0 + lr_base + (g >> 2) * 32 + (g & 3) * 8 + j; };
        auto load = [&](int g, float (*x)[NT], float (*gt)[NT]) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = grow(g, j);
                if (m < M) {
                    const int rr = row0 + m;
                    const float* gate = mod + (long)L.geom.batch_of(rr) * L.mod_stride + gate_off + ncol;
                    const float* xrow = resid + (long)rr * L.N + ncol;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        x[j][nt] = xrow[nt * 32];
                        gt[j][nt] = gate[nt * 32];
                    }
                }
            }
        };
        load(0, xv[0], gv[0]);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (g + 1 < NG) load(g + 1, xv[(g + 1) & 1], gv[(g + 1) & 1]);
            const int mt = g >> 2, i = g & 3;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = grow(g, j);
                if (m < M) {
                    float* xrow = resid + (long)(row0 + m) * L.N + ncol;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        xrow[nt * 32] = xv[g & 1][j][nt] + gv[g & 1][j][nt] * acc[mt][nt][i * 4 + j];
                }
            }
        }
    } else if constexpr (EPI == EPI_SWIGLU) {
        // h tile [256 rows][128 cols] bf16 staged in LDS, then 16-byte row stores.
        // Row-major orientation: gate block nt = 2p and up block 2p + 1 give h
        // columns wn*64 + p*32 + i*8 + grp*4 + j, four of them per 8-byte write.
        bf16_t* st = smem;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int p2 = 0; p2 < NT / 2; ++p2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float h[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) h[j] = silu_f(acc[mt][2 * p2][i * 4 + j]) * acc[mt][2 * p2 + 1][i * 4 + j];
                    *reinterpret_cast<uint2*>(st + (rr_row + mt * 32) * HS + wn * (TN / 2) + p2 * 32 + i * 8 +
                                              (lane >> 5) * 4) = make_uint2(pack2bf(h[0], h[1]), pack2bf(h[2], h[3]));
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
            // Row-major orientation: per-row LayerNorm over the 256 head columns;
            // each lane sums its 64 values of a row, the lane holding the other
            // half-wave's 64 adds in, and the two wn waves meet through LDS.
            float mean[MT], rstd[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                float s1 = 0.f;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s1 += acc[mt][nt][r];
                s1 += __shfl_xor(s1, 32, 64);
                if ((lane >> 5) == 0) rsum[wn * 256 + rr_row + mt * 32] = s1;
            }
            __syncthreads();
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                float tot = 0.f;
#pragma unroll
                for (int w = 0; w < WN; ++w) tot += rsum[w * 256 + rr_row + mt * 32];
                mean[mt] = tot * (1.f / 256.f);
                float s2 = 0.f;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float c = acc[mt][nt][r] - mean[mt];
                        s2 += c * c;
                    }
                s2 += __shfl_xor(s2, 32, 64);
                if ((lane >> 5) == 0) rsq[wn * 256 + rr_row + mt * 32] = s2;
            }
            __syncthreads();
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                float tsq = 0.f;
#pragma unroll
                for (int w = 0; w < WN; ++w) tsq += rsq[w * 256 + rr_row + mt * 32];
                rstd[mt] = rsqrtf(tsq * (1.f / 256.f) + L.eps) * (which == 0 ? L.q_scale : 1.f);
            }
            // normalised tile -> LDS, four consecutive columns per 8-byte write
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float v[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) v[j] = (acc[mt][nt][i * 4 + j] - mean[mt]) * rstd[mt];
                        *reinterpret_cast<uint2*>(st + (rr_row + mt * 32) * QS + rr_col + nt * 32 + i * 8) =
                            make_uint2(pack2bf(v[0], v[1]), pack2bf(v[2], v[3]));
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
            // The tile goes to LDS transposed (head column c -> LDS row c, tile rows
            // along it), four consecutive rows per 8-byte write.
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int lr = lr_base + mt * 32 + i * 8;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        const int c = lc_base + nt * 32;
                        *reinterpret_cast<uint2*>(st + c * QS + lr) =
                            make_uint2(pack2bf(acc[mt][nt][i * 4 + 0], acc[mt][nt][i * 4 + 1]),
                                       pack2bf(acc[mt][nt][i * 4 + 2], acc[mt][nt][i * 4 + 3]));
                    }
                }
            __syncthreads();
            // v^T: 8 consecutive tile rows of head column c -> 8 consecutive keys (one
            // 16-byte store) when they lie in one sample's segment and start 8-aligned;
            // otherwise element stores. Consecutive lanes take consecutive row chunks
            // of one column, so 32 lanes read 512 contiguous LDS bytes and write one
            // 512-byte run of a v^T row.
            bf16_t* vt = (bf16_t*)L.vt;
#pragma unroll 2
            for (int it = 0; it < 8192 / NTHR; ++it) {
                const int idx = it * NTHR + tid;       // 256 columns x 32 row-chunks
                const int rc = idx & 31, c = idx >> 5;
                const int lr0 = rc * 8;
                const int m = m0 + lr0;
                if (m >= M) continue;
                const int rr = row0 + m;
                const int b = L.geom.batch_of(rr), s0 = L.geom.seq_of(rr);
                const bool fast = (m + 7 < M) && (s0 % 8 == 0) && L.geom.batch_of(rr + 7) == b &&
                                  L.geom.seq_of(rr + 7) == s0 + 7;
                if (fast) {
                    const uint4 v = *reinterpret_cast<const uint4*>(st + c * QS + lr0);
                    *reinterpret_cast<uint4*>(vt + (((long)b * H + head) * 256 + c) * (long)S_pad + s0) = v;
                } else {
                    for (int e = 0; e < 8 && m + e < M; ++e) {
                        const int re = rr + e;
                        const int be = L.geom.batch_of(re), se = L.geom.seq_of(re);
                        vt[(((long)be * H + head) * 256 + c) * (long)S_pad + se] = st[c * QS + lr0 + e];
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

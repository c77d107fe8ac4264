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
//   GEGLU          the same with the tanh-form GELU (the text encoder's gated FFN)
//   PARTIAL        fp32 partial sums over one of ksplit K ranges (split-K for
//                  launches with few tiles; splitk_resid adds them in order)
//
// Tiling: 256 x 256 block tile, eight waves (two per SIMD) in a 4 x 2
// arrangement, each wave owning a 64 x 128 sub-tile (2 x 4 MFMA tiles, 128 fp32
// accumulators per lane). K is consumed in sub-tiles of 32 (two MFMA k-steps)
// that stream global -> LDS through four slots with buffer_load ... lds (lane i
// writes LDS bytes [16 i, 16 i + 16) of the instruction's 1 KB block; the MUBUF
// form keeps the compiler's LDS-read waits partial, where the FLAT form of the
// same direct load makes every LDS wait a full drain). The XOR swizzle of
// 16-byte chunks is applied by choosing which global chunk each lane fetches, so
// the MFMA operand reads (ds_read_b128) are bank-conflict free. Two main-loop
// schedules: in the rotated one every wave interleaves its own fragment reads
// and direct loads with its MFMAs, and the barrier that publishes sub-tile j + 1
// sits between the two k-steps of sub-tile j; in the ping-pong one (256 x 256
// tiles) the two waves that share a SIMD run half a sub-tile apart, so one issues
// its 16 MFMAs while the other reads fragments and issues loads.
// Blocks are mapped to tiles XCD by XCD (consecutive block ids go to different
// XCDs) and, inside an XCD, in groups of row tiles so co-resident blocks share
// A and W panels in that XCD's L2. Up to two row groups with different weights
// share one launch (the joint blocks' text and image streams).
// Epilogues that write bf16 stage the tile in LDS and store 16-byte chunks.
#include "gemm_tile.h"

namespace af {

using namespace gemm;

// BM_ x BN_ block tile (square: A and W sub-tiles share one layout), WM x WN
// waves, each owning a (BM_ / WM) x (BN_ / WN) sub-tile. 256 x 256 with 8 waves is
// the main configuration (one workgroup per CU); 128 x 128 with 4 waves (two
// workgroups per CU) serves launches with too few 256 x 256 tiles to fill the GPU.
template <int EPI, int WM, int WN, int BM_ = BM, int BN_ = BN>
__global__ __launch_bounds__(WM * WN * 64)
__attribute__((amdgpu_waves_per_eu(BM_ == 256 ? WM * WN / 4 : 2, BM_ == 256 ? WM * WN / 4 : 2)))
void k_gemm_bf16(GemmLaunch L) {
    constexpr int NW = WM * WN, NTHR = NW * 64;
    constexpr int TM = BM_ / WM, TN = BN_ / WN, MT = TM / 32, NT = TN / 32;
    constexpr int TILE = BM_ * BK;   // bf16 elements of one staged A (or W) sub-tile
    static_assert(BM_ == BN_, "A and W sub-tiles share one layout");
    static_assert(((BM_ / RPI) / NW) % 2 == 0, "per-wave load count must be even");
    static_assert(BM_ != 256 || NW == 8, "the ping-pong schedule pairs waves w and w + 4 on one SIMD");
    static_assert(BM_ == 256 || 2 * NS * TILE >= BM_ * HS, "the gated epilogue's staging fits the operand slots");
    __shared__ __attribute__((aligned(1024))) bf16_t smem[BM_ == 256 ? SMEM_ELEMS : 2 * NS * TILE];

    // wave index in a scalar register: the LDS addresses of the direct loads (M0)
    // are then formed with scalar arithmetic
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // PARTIAL: the launch repeats the tile set once per K range
    int bid = blockIdx.x, split = 0;
    if constexpr (EPI == EPI_PARTIAL) {
        const int T = tiles_m<BM_>(L.g[0].M) * (L.N / BN_);
        split = bid / T;
        bid -= split * T;
    }
    const TileMap tmap = tile_map<BM_, BN_>(L, bid);
    const int gi = tmap.gi;
    const long lda = gi ? L.g[1].lda : L.g[0].lda;
    const long ldw = gi ? L.g[1].ldw : L.g[0].ldw;
    const int K = EPI == EPI_PARTIAL ? L.K / L.ksplit : L.K;
    const bf16_t* __restrict__ A = (const bf16_t*)(gi ? L.g[1].A : L.g[0].A) + (long)split * K;
    const bf16_t* __restrict__ W = (const bf16_t*)(gi ? L.g[1].W : L.g[0].W) + (long)split * K;
    const int M = tmap.M, gate_off = tmap.gate_off;
    const int row0 = EPI == EPI_PARTIAL ? split * M : tmap.row0;
    const int m0 = tmap.m0, n0 = tmap.n0;

    // Per-lane byte offsets for the direct loads (logical chunk folded in). Rows
    // past M read the padding rows every activation buffer carries (at least one
    // tile of rows past its last real row); their results are never stored.
    uint32_t aoff[2], woff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = (wave * ((BM_ / RPI) / NW) + j) * RPI + lane / CH;
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
    static_assert(MT * NT >= 4 && (BM_ / RPI) / NW == 2, "issue pattern: two direct loads among >= 4 MFMAs");
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
    constexpr int PER = (BM_ / RPI) / NW;    // direct loads per wave per operand per sub-tile
    constexpr int PER2 = 2 * PER;
    const int KT = K / BK;
    auto slot_ptr = [&](int st) { return smem + st * 2 * TILE; };
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)Atile, (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc((void*)Wtile, (short)0, 0x7fffffff, 0x00020000);
    const int ldab = (int)lda * 2, ldwb = (int)ldw * 2;
    // Implicit-GEMM 3x3 convolution (EPI_CONV with L.conv != 0): row m of the tile
    // is output pixel (b, y, x), column k = tap Cin + c with tap = 3 (dy + 1) +
    // (dx + 1) reads input pixel (b, y + dy, x + dx) (L.conv == 2: pixel
    // ((y + dy) >> 1, (x + dx) >> 1) of the half-size input, the 2x nearest
    // upsampling). A sub-tile's 32 columns lie in one tap (Cin is a multiple of
    // 32), so each lane gathers its two rows' 16 bytes with per-lane offsets;
    // pixels outside the image and rows past M get an offset past the buffer's
    // end, which the buffer range check reads as zeros (the zero padding).
    int cyy[PER], cxx[PER], cbb[PER];
    uint32_t clc[PER];
    bool conv_on = false;
    __amdgpu_buffer_rsrc_t rAc = rA;
    if constexpr (EPI == EPI_CONV) {
        conv_on = L.conv != 0;
        if (conv_on) {
            const int Ho = L.conv == 2 ? 2 * L.cH : L.cH, Wo = L.conv == 2 ? 2 * L.cW : L.cW;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int r = (wave * PER + j) * RPI + lane / CH;
                const int m = m0 + r;
                const int pb = m / (Ho * Wo), rem = m - pb * (Ho * Wo);
                cbb[j] = pb;
                cyy[j] = m < M ? rem / Wo : -(1 << 20);     // rows past M: never inside the image
                cxx[j] = rem % Wo;
                clc[j] = (uint32_t)(((lane % CH) ^ swz(r)) * 16);
            }
            rAc = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)L.a_bytes, 0x00020000);
        }
    }
    auto issueA_conv = [&](int t, int st) {
        const int k0 = min(t, KT - 1) * BK;
        const int tap = k0 / L.cCin, c0 = k0 - tap * L.cCin;
        const int dy = tap / 3 - 1, dx = tap - 3 * (tap / 3) - 1;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int sy = cyy[j] + dy, sx = cxx[j] + dx;
            uint32_t voff;
            if (L.conv == 2) {
                const bool in = (unsigned)sy < (unsigned)(2 * L.cH) && (unsigned)sx < (unsigned)(2 * L.cW);
                const uint32_t pix = (uint32_t)((cbb[j] * L.cH + (sy >> 1)) * L.cW + (sx >> 1));
                voff = in ? pix * (uint32_t)L.cCin * 2u + clc[j] : 0x80000000u;
            } else {
                const bool in = (unsigned)sy < (unsigned)L.cH && (unsigned)sx < (unsigned)L.cW;
                const uint32_t pix = (uint32_t)((cbb[j] * L.cH + sy) * L.cW + sx);
                voff = in ? pix * (uint32_t)L.cCin * 2u + clc[j] : 0x80000000u;
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rAc, (lds_void*)(slot_ptr(st) + (wave * PER + j) * 512), 16, voff,
                                                     c0 * 2, 0, 0);
        }
    };
    auto issueA = [&](int t, int st) {
        if (conv_on) issueA_conv(t, st);
        else issue_tile<NW, BM_>(rA, aoff, min(t, KT - 1) * BK * 2, ldab, slot_ptr(st), wave);
    };
    auto issueW = [&](int t, int st) {
        issue_tile<NW, BN_>(rW, woff, min(t, KT - 1) * BK * 2, ldwb, slot_ptr(st) + TILE, wave);
    };
    // Ping-pong schedule. Waves w and w + NW / 2 share a SIMD (waves go to SIMDs
    // round-robin); the upper half runs one phase behind the lower half. A wave's
    // iteration j is a memory phase M(j) (read both k-steps' fragments of sub-tile
    // j from its slot, issue the direct loads of sub-tile j + NS - 1 into slot
    // j - 1) and a compute phase C(j) (its 16 MFMAs), each ended by a barrier.
    // Counting barriers from the one after the prologue, the lower half's M(j)
    // lies between barriers 2j - 1 and 2j, the upper half's between 2j and 2j + 1.
    //  - Sub-tile t is first read in the lower half's M(t), after barrier 2t - 1;
    //    every wave arrives there having issued sub-tile t + NS - 2 at most, so
    //    a wait for all but NS - 2 sub-tiles of its loads at each barrier lands t.
    //  - Slot j - 1 is last read in the upper half's M(j - 1), whose reads end
    //    (lgkmcnt 0) before barrier 2j - 1; the first write into it is issued in
    //    the lower half's M(j), after that barrier.
    // Every wave passes the same number of barriers (the upper half one extra at
    // the start, the lower half one at the end).
    auto mainloop_pingpong = [&](auto orient) {
        const bool upper = wave >= NW / 2;
#pragma unroll
        for (int t = 0; t < NS - 1; ++t) {
            issueA(t, t);
            issueW(t, t);
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER2 * (NS - 2)));   // sub-tile 0 landed
        __builtin_amdgcn_s_barrier();
        if (upper) __builtin_amdgcn_s_barrier();
        bf16x8 fa0[MT], fb0[NT], fa1[MT], fb1[NT];
        int cs = 0;
        for (int j = 0; j < KT; ++j) {
            const bf16_t* cur = slot_ptr(cs);
            const int fs = cs == 0 ? NS - 1 : cs - 1;      // slot of j - 1 and of j + NS - 1
            __builtin_amdgcn_sched_barrier(0);
            load_frags(cur, cur + TILE, 0, fa0, fb0);
            load_frags(cur, cur + TILE, 1, fa1, fb1);
            issueA(j + NS - 1, fs);
            issueW(j + NS - 1, fs);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER2 * (NS - 2)) & ~(15 << 8));   // and lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            mfmas(fa0, fb0, orient);
            mfmas(fa1, fb1, orient);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER2 * (NS - 2)));
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            cs = cs + 1 == NS ? 0 : cs + 1;
        }
        if (!upper) __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
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
        load_frags(slot_ptr(0), slot_ptr(0) + TILE, 0, fa0, fb0);
        int cs = 0;
        for (int j = 0; j < KT; ++j) {
            const bf16_t* cur = slot_ptr(cs);
            const int ns = cs + 1 == NS ? 0 : cs + 1;      // slot of j + 1
            const int fs = cs == 0 ? NS - 1 : cs - 1;      // slot of j - 1
            const int f2 = fs == 0 ? NS - 1 : fs - 1;      // slot of j - 2
            issueW(j + NS - 2, f2);
            load_frags(cur, cur + TILE, 1, fa1, fb1);
            mfmas(fa0, fb0, orient);
            pattern();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER2 * (NS - 3)) & ~(15 << 8));   // and lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            issueA(j + NS - 1, fs);
            const bf16_t* nxt = slot_ptr(ns);
            load_frags(nxt, nxt + TILE, 0, fa0, fb0);
            mfmas(fa1, fb1, orient);
            pattern();
            __builtin_amdgcn_sched_barrier(0);
            cs = ns;
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    // q and k tiles of the QKV GEMM and the SwiGLU tiles run in the row-major
    // (C^T) orientation; everything else in the column-major one. The QKV GEMM
    // keeps the rotated schedule (ping-pong measured 0.8% slower there, 0.7-2%
    // faster for the gated-residual and gated-FFN products).
    if constexpr (EPI == EPI_SWIGLU || EPI == EPI_GEGLU) {
        if constexpr (BM_ == 256) mainloop_pingpong(Orient<true>{});
        else mainloop(Orient<true>{});
    } else if constexpr (EPI == EPI_QKV) {
        if (n0 / (L.N / 3) < 2) mainloop(Orient<true>{});
        else mainloop(Orient<false>{});
    } else {
        if constexpr (BM_ == 256) mainloop_pingpong(Orient<false>{});
        else mainloop(Orient<false>{});
    }

    epilogue<EPI, WM, WN, false, BM_, BN_>(L, acc, smem, tid, lane, wm, wn, m0, n0, M, row0, gate_off);
}

hipError_t gemm_bf16(const GemmLaunch& L, hipStream_t s) {
    GemmLaunch LL = L;
    if (LL.ngroups == 2 && LL.g[0].M == 0) {  // keep group 0 non-empty
        LL.g[0] = LL.g[1];
        LL.ngroups = 1;
    }
    if (LL.ngroups == 2 && LL.g[1].M == 0) LL.ngroups = 1;
    int total = 0;
    for (int i = 0; i < LL.ngroups; ++i) total += tiles_m(LL.g[i].M) * ((L.N + BN - 1) / BN);
    if (total == 0) return hipSuccess;
    if (L.epi == EPI_CONV && (LL.ngroups != 1 || L.N % 128 != 0 || L.K % BK != 0 ||
                              (L.conv && (L.cCin % BK != 0 || L.K != 9 * L.cCin || L.a_bytes >= (1L << 31)))))
        return hipErrorInvalidValue;
    if (L.epi == EPI_PARTIAL && (LL.ngroups != 1 || L.ksplit < 1 || L.K % (BK * L.ksplit) != 0))
        return hipErrorInvalidValue;
    const int ks = L.epi == EPI_PARTIAL ? L.ksplit : 1;
    // 128 x 128 tiles (two workgroups per CU) when the 256 x 256 tiles, K ranges
    // included, would occupy at most half of the compute units: one round of the
    // small tiles then takes about half the time of the large tiles' round
    const bool small = (L.n_cu > 0 && 2 * total * ks <= L.n_cu && L.epi != EPI_QKV && L.epi != EPI_STORE_MAPPED) ||
                       (L.epi == EPI_CONV && L.N % BN != 0);
    if (small) {
        int t128 = 0;
        for (int i = 0; i < LL.ngroups; ++i) t128 += tiles_m<128>(LL.g[i].M) * (L.N / 128);
        const dim3 grid(t128 * ks), block(4 * 64);
#define AF_G128(E) hipLaunchKernelGGL((k_gemm_bf16<E, 2, 2, 128, 128>), grid, block, 0, s, LL)
        switch (L.epi) {
            case EPI_STORE: AF_G128(EPI_STORE); break;
            case EPI_GATED_RESID: AF_G128(EPI_GATED_RESID); break;
            case EPI_SWIGLU: AF_G128(EPI_SWIGLU); break;
            case EPI_GEGLU: AF_G128(EPI_GEGLU); break;
            case EPI_PARTIAL: AF_G128(EPI_PARTIAL); break;
            case EPI_CONV: AF_G128(EPI_CONV); break;
            default: return hipErrorInvalidValue;
        }
#undef AF_G128
        return hipGetLastError();
    }
    total *= ks;
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
        case EPI_GEGLU: hipLaunchKernelGGL((k_gemm_bf16<EPI_GEGLU, GEMM_WM, GEMM_WN>), grid, block, 0, s, LL); break;
        case EPI_PARTIAL: hipLaunchKernelGGL((k_gemm_bf16<EPI_PARTIAL, GEMM_WM, GEMM_WN>), grid, block, 0, s, LL); break;
        case EPI_CONV: hipLaunchKernelGGL((k_gemm_bf16<EPI_CONV, GEMM_WM, GEMM_WN>), grid, block, 0, s, LL); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace af

// MXFP8 MFMA GEMM for gfx950: C = A W^T with A [M, K] and W [N, K] stored as
// E4M3 bytes plus one power-of-two scale per 32 consecutive values along K (the
// OCP microscaling block format), multiplied by v_mfma_scale_f32_32x32x64_f8f6f4
// with fp32 accumulation, followed by the epilogues of the bf16 GEMM (QK-norm
// and q/k/v^T scatter, SwiGLU with an MXFP8 output, gated residual update).
//
// Tiling is the bf16 kernel's: 256 x 256 block tile, eight waves in a 4 x 2 grid
// (64 x 128 per wave), operand sub-tiles of 256 rows x 64 bytes (64 fp8 values,
// one MFMA k-step) streamed global -> LDS through four slots with MUBUF direct
// loads and the same 16-byte chunk swizzle. A sub-tile's block scales (256 rows x
// 2 blocks for A and for W, 1 KB) ride along in a 2 KB LDS area per slot: waves
// 0-1 load the A scales and waves 2-3 the W scales (256 bytes each, one direct
// load); waves 4-7 repeat those loads into the area's second half, so that every
// wave has the same number of loads in flight. Scale arrays are stored
// [K/64][rows][2]: the two scales of a row for one sub-tile are adjacent and the
// sub-tile's rows are contiguous.
//
// Operand layout of the scaled MFMA (32 x 32 x 64, fp8): lane l holds row
// l & 31; its VGPRs 0-3 carry 16 values of the first 32-value block and VGPRs
// 4-7 16 values of the second (chunk l >> 5 and chunk 2 + (l >> 5) of the
// 64-byte row); lane l's scale byte is the scale of row l & 31 in block l >> 5.
//
// Loop (one k-step per sub-tile; the fragments of one sub-tile are 48 VGPRs, so
// they are not double-buffered): iteration j reads the A fragments of row block
// 1 of sub-tile j, runs the MFMAs of row block 0, waits for sub-tile j + 1 and
// the barrier, refills slot j with sub-tile j + 4 (nobody reads slot j any
// more), runs the MFMAs of row block 1, then reads sub-tile j + 1's row block 0
// A fragments, all its W fragments and its scales into the registers those
// MFMAs have just consumed.
#include "gemm_tile.h"

namespace af {

using namespace gemm;

namespace {
typedef int i32x8 __attribute__((ext_vector_type(8)));
template <int S> struct Slot { static constexpr int value = S; };
constexpr int MXWM = 4, MXWN = 2;
constexpr int SC_OFF = 2 * NS * TILE_ELEMS;   // bf16-element offset of the scale areas (after the slots)
static_assert(SC_OFF + NS * 1024 <= SMEM_ELEMS, "scale areas exceed the LDS block");
}  // namespace

template <int EPI>
__global__ __launch_bounds__(MXWM * MXWN * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm_mxfp8(GemmLaunch L) {
    constexpr int WM = MXWM, WN = MXWN, NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN, MT = TM / 32, NT = TN / 32;
    static_assert(MT == 2 && NT == 4, "loop is laid out for 64 x 128 wave tiles");
    __shared__ __attribute__((aligned(1024))) bf16_t smem[SMEM_ELEMS];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const TileMap tmap = tile_map(L, blockIdx.x);
    const int gi = tmap.gi;
    const uint8_t* __restrict__ A = (const uint8_t*)(gi ? L.g[1].A : L.g[0].A);
    const long lda = gi ? L.g[1].lda : L.g[0].lda;      // bytes per row
    const uint8_t* __restrict__ W = (const uint8_t*)(gi ? L.g[1].W : L.g[0].W);
    const long ldw = gi ? L.g[1].ldw : L.g[0].ldw;
    const uint8_t* As = gi ? L.g[1].As : L.g[0].As;
    const uint8_t* Ws = gi ? L.g[1].Ws : L.g[0].Ws;
    const int M = tmap.M, row0 = tmap.row0, gate_off = tmap.gate_off;
    const int m0 = tmap.m0, n0 = tmap.n0;
    const int KT = L.K / 64;

    // direct-load byte offsets of the data sub-tiles (as in the bf16 kernel)
    constexpr int PER = (BM / RPI) / NW;      // data loads per wave per operand per sub-tile (2)
    constexpr int PERL = 2 * PER + 1;         // all loads of one sub-tile per wave (data + scales)
    uint32_t aoff[2], woff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = (wave * PER + j) * RPI + lane / CH;
        const int c = (lane % CH) ^ swz(r);
        aoff[j] = (uint32_t)(r * lda + c * 16);
        woff[j] = (uint32_t)(r * ldw + c * 16);
    }
    const __amdgpu_buffer_rsrc_t rA =
        __builtin_amdgcn_make_buffer_rsrc((void*)(A + (long)m0 * lda), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rW =
        __builtin_amdgcn_make_buffer_rsrc((void*)(W + (long)n0 * ldw), (short)0, 0x7fffffff, 0x00020000);
    // scales: wave w < 2 fetches A scale rows m0 + 128 w .. + 127, waves 2-3 W scale
    // rows n0 + 128 (w - 2) .. + 127 (256 bytes); waves 4-7 repeat waves 0-3's
    // loads into a spare area
    const int sw = wave & 3;
    const bool sc_w = sw >= 2;
    const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(sc_w ? Ws + (long)(n0 + 128 * (sw - 2)) * 2 : As + (long)(m0 + 128 * sw) * 2), (short)0, 0x7fffffff,
        0x00020000);
    const int sc_slab = (int)((sc_w ? L.ws_rows : L.as_rows) * 2);   // bytes between sub-tiles' scales

    auto slot_ptr = [&](int st) { return smem + st * 2 * TILE_ELEMS; };
    // per slot 2 KB: A scales [256 rows][2], W scales [256 rows][2], then the
    // 1 KB that waves 4-7 fill with repeats
    auto sc_ptr = [&](int st) { return reinterpret_cast<uint8_t*>(smem + SC_OFF) + st * 2048; };
    auto issue = [&](int t, int st) {
        const int tt = min(t, KT - 1);        // past the end: re-read the last sub-tile into a free slot
        issue_tile<NW>(rA, aoff, tt * 64, (int)lda, slot_ptr(st), wave);
        issue_tile<NW>(rW, woff, tt * 64, (int)ldw, slot_ptr(st) + TILE_ELEMS, wave);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void*)(sc_ptr(st) + 256 * wave), 4, lane * 4, tt * sc_slab, 0, 0);
    };

    f32x16 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int g = lane >> 5;
    // 32 fp8 values of `row` for this lane. The LDS reads are typed as bf16
    // vectors like the bf16 kernel's: with integer-typed reads the compiler
    // assumes they may alias the direct loads in flight and drains them all
    // (vmcnt(0)) before every read; completion is ordered explicitly instead
    // (vmcnt wait + barrier before a slot is read).
    auto frag = [&](const bf16_t* tile, int row) {
        const bf16_t* base = tile + row * 32;
        const bf16x8 lo = *reinterpret_cast<const bf16x8*>(base + ((g ^ swz(row)) * 8));
        const bf16x8 hi = *reinterpret_cast<const bf16x8*>(base + (((2 + g) ^ swz(row)) * 8));
        typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
        return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13,
                                                                 14, 15));
    };
    auto read_a = [&](int st, int mt, i32x8& fa, int* sa) {
        const int row = wm * TM + mt * 32 + (lane & 31);
        fa = frag(slot_ptr(st), row);
        sa[mt] = sc_ptr(st)[row * 2 + g];
    };
    auto read_b = [&](int st, i32x8* fb, int* sb) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int row = wn * TN + nt * 32 + (lane & 31);
            fb[nt] = frag(slot_ptr(st) + TILE_ELEMS, row);
            sb[nt] = sc_ptr(st)[512 + row * 2 + g];
        }
    };
    auto mfmas = [&](int mt, const i32x8& fa, const int* sa, const i32x8* fb, const int* sb, auto orient) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x16& c = acc[mt][nt];
            if constexpr (decltype(orient)::value)
                c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[nt], fa, c, 0, 0, 0, sb[nt], 0, sa[mt]);
            else
                c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb[nt], c, 0, 0, 0, sa[mt], 0, sb[nt]);
        }
    };

    auto mainloop = [&](auto orient) {
#pragma unroll
        for (int t = 0; t < NS; ++t) issue(t, t);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(PERL * (NS - 1)));   // sub-tile 0 landed
        __builtin_amdgcn_s_barrier();
        i32x8 fa0, fa1, fb[NT];
        int sa[MT], sb[NT];
        read_a(0, 0, fa0, sa);
        read_b(0, fb, sb);
        // slots as compile-time constants (the loop is unrolled by NS; K is a
        // multiple of 256), so the compiler can tell the slot being refilled from
        // the slot being read and keeps its LDS-read waits partial
        auto step = [&](int j, auto slot) {
            constexpr int cs = decltype(slot)::value, ns = (cs + 1) % NS;
            read_a(cs, 1, fa1, sa);
            mfmas(0, fa0, sa, fb, sb, orient);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(PERL * (NS - 2)) & ~(15 << 8));   // and lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            issue(j + NS, cs);
            mfmas(1, fa1, sa, fb, sb, orient);
            __builtin_amdgcn_sched_barrier(0);
            read_a(ns, 0, fa0, sa);
            read_b(ns, fb, sb);
        };
        static_assert(NS == 4, "the loop body is unrolled for four slots");
        for (int j = 0; j < KT; j += NS) {
            step(j, Slot<0>{});
            step(j + 1, Slot<1>{});
            step(j + 2, Slot<2>{});
            step(j + 3, Slot<3>{});
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    if constexpr (EPI == EPI_SWIGLU) {
        mainloop(Orient<true>{});
    } else if constexpr (EPI == EPI_QKV) {
        if (n0 / (L.N / 3) < 2) mainloop(Orient<true>{});
        else mainloop(Orient<false>{});
    } else {
        mainloop(Orient<false>{});
    }
    epilogue<EPI, WM, WN, true>(L, acc, smem, tid, lane, wm, wn, m0, n0, M, row0, gate_off);
}

hipError_t gemm_mxfp8(const GemmLaunch& L, hipStream_t s) {
    const int tiles_n = L.N / BN;
    GemmLaunch LL = L;
    if (LL.ngroups == 2 && LL.g[0].M == 0) {
        LL.g[0] = LL.g[1];
        LL.ngroups = 1;
    }
    if (LL.ngroups == 2 && LL.g[1].M == 0) LL.ngroups = 1;
    if (L.K % 256 != 0 || L.N % BN != 0) return hipErrorInvalidValue;
    int total = 0;
    for (int i = 0; i < LL.ngroups; ++i) total += tiles_m(LL.g[i].M) * tiles_n;
    if (total == 0) return hipSuccess;
    dim3 grid(total), block(MXWM * MXWN * 64);
    switch (L.epi) {
        case EPI_QKV: hipLaunchKernelGGL(k_gemm_mxfp8<EPI_QKV>, grid, block, 0, s, LL); break;
        case EPI_SWIGLU: hipLaunchKernelGGL(k_gemm_mxfp8<EPI_SWIGLU>, grid, block, 0, s, LL); break;
        case EPI_GATED_RESID: hipLaunchKernelGGL(k_gemm_mxfp8<EPI_GATED_RESID>, grid, block, 0, s, LL); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace af

// Pieces shared by the bf16 and the MXFP8 MFMA GEMMs: tile geometry, the
// XCD-aware block-to-tile map, the LDS chunk swizzle, the direct-load issue of
// one operand sub-tile and the fused epilogues. Both main loops stage 256-row
// operand sub-tiles of 64 bytes per row (32 bf16 or 64 fp8 values) in the same
// LDS layout, and both leave the same fp32 accumulator layout to the epilogue.
#pragma once
#include "af_internal.h"

namespace af {
namespace gemm {
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
constexpr int HS8 = 144;             // MXFP8 SwiGLU epilogue staging row stride (bytes)
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
template <int BM_ = BM>
__host__ __device__ __forceinline__ int tiles_m(int M) { return (M + BM_ - 1) / BM_; }
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
template <int NW, int ROWS = BM>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rsrc, const uint32_t* voff, int sbase, int ldbytes,
                                           bf16_t* lds_tile, int wave) {
    constexpr int PER = (ROWS / RPI) / NW;
#pragma unroll
    for (int j = 0; j < PER; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds_tile + (wave * PER + j) * 512), 16, voff[j & 1],
                                                 sbase + (j & ~1) * RPI * ldbytes, 0, 0);
}

// Tile of one workgroup: group (text / image rows of a joint block), first row
// and column, rows of the group, residual row of GEMM row 0, gate column.
struct TileMap {
    int gi, m0, n0, M, row0, gate_off;
};

// `b` is the workgroup's index among the launch's tiles (blockIdx.x, or its
// remainder modulo the tile count when a launch repeats the tiles for K ranges).
template <int BM_ = BM, int BN_ = BN>
__device__ __forceinline__ TileMap tile_map(const GemmLaunch& L, int b) {
    const int tiles_n = L.N / BN_;
    const int tm0 = tiles_m<BM_>(L.g[0].M), tm1 = L.ngroups > 1 ? tiles_m<BM_>(L.g[1].M) : 0;
    const int T0 = tm0 * tiles_n, T = T0 + tm1 * tiles_n;
    int lid;
    {
        const int x = b % NXCD, q = T / NXCD, r = T % NXCD;
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
    TileMap t;
    t.gi = gi;
    t.m0 = tm * BM_;
    t.n0 = tn * BN_;
    t.M = gi ? L.g[1].M : L.g[0].M;
    t.row0 = gi ? L.g[1].row0 : L.g[0].row0;
    t.gate_off = gi ? L.g[1].gate_off : L.g[0].gate_off;
    return t;
}

// Fused epilogues on the fp32 accumulators of a 256 x 256 tile. MXOUT: the
// SwiGLU output is MXFP8 (fp8 values + block scales) instead of bf16.
template <int EPI, int WM, int WN, bool MXOUT, int BM_ = BM, int BN_ = BN>
__device__ __forceinline__ void epilogue(const GemmLaunch& L, f32x16 (&acc)[BM_ / WM / 32][BN_ / WN / 32], bf16_t* smem,
                                         int tid, int lane, int wm, int wn, int m0, int n0, int M, int row0,
                                         int gate_off) {
    constexpr int NW = WM * WN, NTHR = NW * 64;
    constexpr int TM = BM_ / WM, TN = BN_ / WN, MT = TM / 32, NT = TN / 32;
    // Column-major orientation: acc[mt][nt][i*4+j] holds row wm*64 + mt*32 + i*8 +
    // (lane>>5)*4 + j, column wn*128 + nt*32 + (lane&31) of the block tile.
    // Row-major orientation: acc[mt][nt][i*4+j] holds row wm*64 + mt*32 + (lane&31),
    // column wn*128 + nt*32 + i*8 + (lane>>5)*4 + j. LDS is free here.
    const int lr_base = wm * TM + (lane >> 5) * 4;
    const int lc_base = wn * TN + (lane & 31);
    const int rr_row = wm * TM + (lane & 31);           // row-major: row of mt = 0
    const int rr_col = wn * TN + (lane >> 5) * 4;       // row-major: column of nt = i = j = 0

    if constexpr (EPI == EPI_PARTIAL) {
        // fp32 partial sums, split slab selected through row0 = split * M
        float* C = (float*)L.C;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int m = m0 + lr_base + mt * 32 + (r >> 2) * 8 + (r & 3);
                if (m >= M) continue;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) C[(long)(row0 + m) * L.N + n0 + lc_base + nt * 32] = acc[mt][nt][r];
            }
    } else if constexpr (EPI == EPI_CONV) {
        // C[m, n] = acc + bias[n] (+ resid[m, n]); half a wave writes 32
        // consecutive columns of one row. resid may be C itself (in place): every
        // element is read and then written by the same lane. The residual loads of
        // an mt block are all issued before its stores (rows past M read row M - 1
        // and discard it, so the loads carry no branch), which keeps 16 NT loads
        // in flight instead of one.
        const float* cb = L.cbias;
        const float* res = L.resid;
        const int ncol = n0 + lc_base;
        float bv[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) bv[nt] = cb ? cb[ncol + nt * 32] : 0.f;
        auto row_of = [&](int mt, int r) { return m0 + lr_base + mt * 32 + (r >> 2) * 8 + (r & 3); };
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float v[16][NT];
#pragma unroll
            for (int r = 0; r < 16; ++r)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) v[r][nt] = acc[mt][nt][r] + bv[nt];
            if (res) {
                float rv[16][NT];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const long ro = (long)(row0 + min(row_of(mt, r), M - 1)) * L.ldc + ncol;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) rv[r][nt] = res[ro + nt * 32];
                }
#pragma unroll
                for (int r = 0; r < 16; ++r)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) v[r][nt] += rv[r][nt];
            }
            if (L.c_bf16) {
                bf16_t* C = (bf16_t*)L.C;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = row_of(mt, r);
                    if (m >= M) continue;
                    const long ro = (long)(row0 + m) * L.ldc + ncol;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) C[ro + nt * 32] = f2bf(v[r][nt]);
                }
            } else {
                float* C = (float*)L.C;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = row_of(mt, r);
                    if (m >= M) continue;
                    const long ro = (long)(row0 + m) * L.ldc + ncol;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) C[ro + nt * 32] = v[r][nt];
                }
            }
        }
    } else if constexpr (EPI == EPI_STORE) {
        bf16_t* C = (bf16_t*)L.C;
#pragma unroll
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
    } else if constexpr (EPI == EPI_SWIGLU && MXOUT) {
        static_assert(BM_ == 256 && BN_ == 256, "the MXFP8 SwiGLU epilogue is laid out for 256 x 256 tiles");
        // h = silu(gate) * up as MXFP8: every 32 h columns of a row share one
        // power-of-two scale 2^e, e = floor(log2(max |h|)) - 8 (at least -127);
        // elements h / 2^e clamped to +-448 and rounded to E4M3. Row-major
        // orientation: the 32 columns wn*64 + p2*32 + [0, 32) of row rr_row + mt*32
        // are held by lanes l and l ^ 32 (16 each). The fp8 tile [256 rows][128 B]
        // is staged in LDS and leaves as 16-byte row chunks; the scale bytes go to
        // the [K/64][rows][2] scale layout directly.
        uint8_t* st8 = reinterpret_cast<uint8_t*>(smem);
        const int fcol0 = n0 / 2;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int p2 = 0; p2 < NT / 2; ++p2) {
                float h[16];
                float amax = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    h[r] = silu_f(acc[mt][2 * p2][r]) * acc[mt][2 * p2 + 1][r];
                    amax = fmaxf(amax, fabsf(h[r]));
                }
                amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
                const int e = mx_scale_exp(amax);
                const float inv = pow2f(-e);
                const int row = rr_row + mt * 32;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<uint32_t*>(st8 + row * HS8 + wn * (TN / 2) + p2 * 32 + i * 8 + (lane >> 5) * 4) =
                        pack4_e4m3(h[i * 4 + 0] * inv, h[i * 4 + 1] * inv, h[i * 4 + 2] * inv, h[i * 4 + 3] * inv);
                const int m = m0 + row;
                if ((lane >> 5) == 0 && m < M) {
                    const int fb = (fcol0 + wn * (TN / 2) + p2 * 32) / 32;
                    L.Cs[(long)(fb >> 1) * L.cs_rows * 2 + (long)(row0 + m) * 2 + (fb & 1)] = (uint8_t)(e + 127);
                }
            }
        __syncthreads();
        uint8_t* Hout = (uint8_t*)L.C;
#pragma unroll 4
        for (int it = 0; it < 2048 / NTHR; ++it) {
            const int idx = it * NTHR + tid;         // 256 rows x 8 chunks of 16 B
            const int lr = idx >> 3, ch = idx & 7;
            const int m = m0 + lr;
            if (m < M) {
                const uint4 v = *reinterpret_cast<const uint4*>(st8 + lr * HS8 + ch * 16);
                *reinterpret_cast<uint4*>(Hout + (long)(row0 + m) * L.ldc + fcol0 + ch * 16) = v;
            }
        }
    } else if constexpr (EPI == EPI_SWIGLU || EPI == EPI_GEGLU) {
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
                    for (int j = 0; j < 4; ++j) {
                        const float g = acc[mt][2 * p2][i * 4 + j];
                        h[j] = (EPI == EPI_GEGLU ? gelu_tanh_f(g) : silu_f(g)) * acc[mt][2 * p2 + 1][i * 4 + j];
                    }
                    *reinterpret_cast<uint2*>(st + (rr_row + mt * 32) * HS + wn * (TN / 2) + p2 * 32 + i * 8 +
                                              (lane >> 5) * 4) = make_uint2(pack2bf(h[0], h[1]), pack2bf(h[2], h[3]));
                }
        __syncthreads();
        bf16_t* Hout = (bf16_t*)L.C;
        const int fcol0 = n0 / 2;
        constexpr int CPR = BN_ / 16;          // 16-byte chunks of h per tile row
#pragma unroll 4
        for (int it = 0; it < BM_ * CPR / NTHR; ++it) {
            int idx = it * NTHR + tid;         // BM_ rows x CPR chunks
            int lr = idx / CPR, ch = idx % CPR;
            int m = m0 + lr;
            if (m < M) {
                uint4 v = *reinterpret_cast<const uint4*>(st + lr * HS + ch * 8);
                *reinterpret_cast<uint4*>(Hout + (long)(row0 + m) * L.ldc + fcol0 + ch * 8) = v;
            }
        }
    } else if constexpr (EPI == EPI_QKV) {
        static_assert(BM_ == 256 && BN_ == 256, "one QKV tile is one 256-wide head");
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

}  // namespace gemm
}  // namespace af

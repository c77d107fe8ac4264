// Joint attention for 256-wide heads on gfx950 (bf16 MFMA, fp32 softmax).
//
// [TRANS] 注意力处理器与 QKV 融合: text and image q/k/v are concatenated (text
// first) and one scaled-dot-product attention runs over the whole sequence, no
// dropout, not causal; the scale is 1/sqrt(head_dim). Keys of padded text
// tokens are excluded through an additive bias per key.
//
// Layout: q, k [B, H, S_pad, 256]; v^T [B, H, 256, S_pad] (written transposed by
// the QKV GEMM epilogue so the P V contraction reads keys contiguously);
// output o [M, d] in residual-row order, bf16, or MXFP8 (E4M3 values plus one
// power-of-two scale per 32 head-dim values) for the MXFP8 out-projection.
//
// Scaled inputs: q arrives multiplied by 1/16 (the QKV epilogue applies it
// before rounding to bf16; a power of two, so it commutes with the rounding) and
// the key bias holds -24 ln 2 for a kept key and -inf for an excluded one, so
// p = exp2((k.q' + bias) log2 e). Softmax reference: QK-norm (LayerNorm over the
// head dim, no affine) gives every normalised q and k a norm of at most
// sqrt(256) = 16, so every logit q.k / 16 lies in [-16, 16]; the kernel
// subtracts the fixed reference 24 ln 2 = 16.64 instead of a running maximum:
// softmax is invariant to the shift, p = e^s 2^-24 stays in [2^-48, 1) (no
// overflow, no denormals), the running-max bookkeeping and the rescaling of O
// disappear, and since the shift is a whole power of two the bf16 rounding of p
// for the P V product is that of e^s. With a fixed reference, partial sums over
// key tiles simply add.
//
// One workgroup = 4 waves = 128 queries of one (b, h); each wave owns 32 queries
// and keeps them in registers as MFMA B operands. Per 64-key tile:
//   S^T = K Q'^T + bias  (A = K rows from LDS) -> one query per lane (lane & 31),
//   P = exp2(S^T log2 e),
//   O^T += V^T P^T (A = v^T from LDS, B = P straight from the S^T registers).
// The K rows each lane feeds to the S^T MFMA are permuted (bits 2 and 3 of the
// row index swapped) so that the accumulator registers a lane holds are, per
// 16-key MFMA step, the 8 consecutive keys the P V MFMA expects; v^T is then used
// in its natural key order.
//
// Software pipeline (one wave per SIMD): iteration t runs the S MFMAs of tile
// t + 1 with the exponentials of tile t's first two key steps interleaved (one
// per MFMA pair), then the P V MFMAs of tile t with the exponentials of its last
// two key steps interleaved into the first half (one per MFMA). K and v^T tiles have two LDS slots each, filled
// by gfx950 direct loads (buffer_load ... lds, 16 bytes per lane; the MUBUF form
// keeps the compiler's LDS-read waits partial) issued one per S MFMA step: in
// iteration t, K and the bias of tile t + 2 and v^T of tile t + 1, so each has
// the whole P V phase to land before the next iteration's wait. One barrier per
// iteration publishes them and frees the slots; the first v^T fragments of a
// P V phase are read during the last S steps. 16-byte chunks are XOR swizzled by
// row so both operand reads are bank-conflict free. The query fragments are
// loaded straight into registers; the output leaves through LDS, whole rows per
// store instruction.
#include "af_internal.h"

namespace af {

namespace {
constexpr int HD = 256;
constexpr int QT = 128;  // queries per workgroup
constexpr int KT = 64;   // keys per tile
constexpr int KTILE = KT * HD;   // bf16 elements of a K (or v^T) tile
// s_waitcnt immediate: vmcnt(17) (bits 3:0 and 15:14), expcnt and lgkmcnt not waited
constexpr int VMCNT_17 = (17 & 15) | ((17 >> 4) << 14) | (7 << 4) | (15 << 8);

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x >> 1) & 4) | ((x << 1) & 8); }
// K tile [64 keys][256]: 32 chunks per row, chunk ^= swap23(row & 15).
__device__ __forceinline__ int kswz(int row) { return swap23(row & 15); }
// v^T tile [256 hd][64 keys]: 8 chunks per row, chunk ^= (row & 7) ^ ((row >> 3) & 1).
__device__ __forceinline__ int vswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_attention_bf16(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                      const bf16_t* __restrict__ Vt, const float* __restrict__ bias, RowGeom g, int H,
                      int S_pad, bf16_t* __restrict__ O, int d, int nqt, int nfull, int kp,
                      float* __restrict__ part, uint8_t* __restrict__ O8, uint8_t* __restrict__ O8s, long sc_rows) {
    // K slot 0, K slot 1, v^T slot 0, v^T slot 1, then per slot and wave a 1 KB
    // bias block (4 copies of 64 fp32 keys)
    __shared__ __attribute__((aligned(1024))) bf16_t smem[4 * KTILE + 2 * 4 * 512];

    // wave index in a scalar register: every LDS address a direct load takes (M0)
    // is then formed with scalar arithmetic
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 5, l32 = lane & 31;
    const int S = g.S();
    const int ntiles = (S + KT - 1) / KT;
    // Work item -> (sample b, head h, query tile qt) and key-tile range [kt0, kt1).
    // Items [0, nfull) are whole query tiles, in (b, h, qt) order with qt fastest,
    // spread so that the items of one XCD (block ids are dispatched round-robin
    // over the 8 XCDs) are consecutive and share K and v^T in that XCD's L2.
    // Items past nfull are pieces: each remaining query tile is split into kp
    // key ranges whose partial sums are added by k_attention_combine.
    int tq, piece = -1, kt0 = 0, kt1 = ntiles;
    {
        const int bid = blockIdx.x;
        if (bid < nfull) {
            const int x = bid % 8, qq = nfull / 8, rr = nfull % 8;
            tq = x * qq + min(x, rr) + bid / 8;
        } else {
            const int j = bid - nfull;
            tq = nfull + j / kp;
            piece = j;
            const int pi = j % kp;
            kt0 = ntiles * pi / kp;
            kt1 = ntiles * (pi + 1) / kp;
        }
    }
    const int qt = tq % nqt, h = (tq / nqt) % H, b = tq / (nqt * H);
    const int nt = kt1 - kt0;   // key tiles of this item
    const int q0 = qt * QT + wave * 32;
    const long bh = (long)b * H + h;
    const bf16_t* Kbh = K + bh * S_pad * HD;
    const bf16_t* Vbh = Vt + bh * HD * (long)S_pad;
    const float* biasb = bias + (long)b * S_pad;
    auto kslot = [&](int i) { return smem + i * KTILE; };
    auto vslot = [&](int i) { return smem + (2 + i) * KTILE; };
    auto bslot = [&](int i) { return reinterpret_cast<const float*>(smem + 4 * KTILE + (i * 4 + wave) * 512); };

    // Direct-load source byte offsets. K: instruction j of this wave fills tile
    // rows 2 cb, 2 cb + 1 (cb = 8 wave + j), lane -> row 2 cb + (lane >> 5),
    // physical chunk lane & 31. v^T: instruction j fills hd rows 8 cb .. 8 cb + 7,
    // lane -> row 8 cb + (lane >> 3), physical chunk lane & 7.
    uint32_t koff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int row = 2 * (wave * 8 + j) + grp;
        int lc = (lane & 31) ^ kswz(row);
        koff[j] = (uint32_t)(row * HD + lc * 8) * 2;
    }
    uint32_t voff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        int row = 8 * (wave * 8 + j) + (lane >> 3);
        int lc = (lane & 7) ^ vswz(row);
        voff[j] = (uint32_t)(row * S_pad + lc * 8) * 2;
    }
    const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc((void*)Kbh, (short)0, S_pad * HD * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc((void*)Vbh, (short)0, S_pad * HD * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void*)biasb, (short)0, S_pad * 4, 0x00020000);
    // one direct load of the item's key tile `tile` (relative to kt0; clamped to
    // its last tile: the loads issued past the end re-read it into a slot nobody
    // reads again)
    auto issue_k = [&](int j, int tile, int slot) {
        const int k0 = (kt0 + min(tile, nt - 1)) * KT;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_void*)(kslot(slot) + (wave * 8 + j) * 512), 16, koff[j],
                                                 k0 * HD * 2, 0, 0);
    };
    auto issue_v = [&](int j, int tile, int slot) {
        const int k0 = (kt0 + min(tile, nt - 1)) * KT;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_void*)(vslot(slot) + (wave * 8 + j) * 512), 16, voff[j & 1],
                                                 k0 * 2 + (j & ~1) * 8 * S_pad * 2, 0, 0);
    };
    auto issue_b = [&](int tile, int slot) {
        const int k0 = (kt0 + min(tile, nt - 1)) * KT;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void*)(smem + 4 * KTILE + (slot * 4 + wave) * 512), 16,
                                                 (lane & 15) * 16, k0 * 4, 0, 0);
    };

    // The wave's 32 queries as MFMA B operands: lane holds query q0 + (lane & 31),
    // head dims [16 s + 8 (lane >> 5), +8) for k-step s, loaded straight into
    // registers. K of tiles 0 and 1, the bias of tile 1 and v^T of tile 0 go out at
    // the same time; the wait before the first barrier covers the queries, the
    // bias of tile 0 and K(0) (the 17 direct loads issued after them may still be
    // in flight).
    bf16x8 qf[16];
    // the bias of tile 0 for the first S tile, in the accumulator order of s_init
    // below, also straight into registers (an LDS read issued behind the direct
    // loads would wait for all of them)
    float4 bias0[8];
    {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                bias0[t * 4 + i] = *reinterpret_cast<const float4*>(biasb + kt0 * KT + t * 32 + (i >> 1) * 16 + grp * 8 +
                                                                    (i & 1) * 4);
        const bf16_t* qsrc = Q + (bh * S_pad + (long)qt * QT) * HD;
        const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc((void*)qsrc, (short)0, QT * HD * 2, 0x00020000);
        const int row = wave * 32 + l32;
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) {
            typedef int i32x4 __attribute__((ext_vector_type(4)));
            const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rQ, (row * HD + (2 * s2 + grp) * 8) * 2, 0, 0);
            qf[s2] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) issue_k(j, 0, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) issue_v(j, 0, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) issue_k(j, 1, 1);
        issue_b(1, 1);
        __builtin_amdgcn_s_waitcnt(VMCNT_17);
        __builtin_amdgcn_s_barrier();
    }

    f32x16 o[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
    float l_run = 0.f;

    // K rows this lane feeds to the S^T MFMA of sub-tile t: t*32 + swap23(lane & 31).
    const int krow0 = swap23(l32);
    constexpr int KD = 3;   // K fragments read KD k-steps ahead
    constexpr int VD = 4;   // v^T fragments read VD MFMAs ahead

    // S^T of the tile in K slot `ks` starts at its bias: register (t, i, j) of a
    // lane holds key t*32 + (i/2)*16 + grp*8 + (i%2)*4 + j.
    auto s_init = [&](f32x16* st, int ks) {
        const float* sB = bslot(ks);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 bv = *reinterpret_cast<const float4*>(sB + t * 32 + (i >> 1) * 16 + grp * 8 + (i & 1) * 4);
                st[t][i * 4 + 0] = bv.x;
                st[t][i * 4 + 1] = bv.y;
                st[t][i * 4 + 2] = bv.z;
                st[t][i * 4 + 3] = bv.w;
            }
    };
    auto kload = [&](const bf16_t* sK, int s, bf16x8* dst) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row = t * 32 + krow0;
            const int ch = (2 * s + grp) ^ kswz(row);
            dst[t] = *reinterpret_cast<const bf16x8*>(sK + row * HD + ch * 8);
        }
    };
    auto pack8 = [&](const float* pf) {
        typedef float f32x8 __attribute__((ext_vector_type(8)));
        const f32x8 v = {pf[0], pf[1], pf[2], pf[3], pf[4], pf[5], pf[6], pf[7]};
        return __builtin_convertvector(v, bf16x8);
    };

    // Prologue: S of tile 0 (K slot 0).
    f32x16 sa[2], sb[2];
    {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sa[t][i * 4 + 0] = bias0[t * 4 + i].x;
                sa[t][i * 4 + 1] = bias0[t * 4 + i].y;
                sa[t][i * 4 + 2] = bias0[t * 4 + i].z;
                sa[t][i * 4 + 3] = bias0[t * 4 + i].w;
            }
        const bf16_t* sK = kslot(0);
        bf16x8 kf[KD + 1][2];
#pragma unroll
        for (int s = 0; s < KD; ++s) kload(sK, s, kf[s]);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            if (s + KD < 16) kload(sK, s + KD, kf[(s + KD) % (KD + 1)]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                sa[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % (KD + 1)][t], qf[s], sa[t], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Iteration t: `cur` holds S of tile t (complete), `nxt` receives S of tile t + 1.
    auto iteration = [&](int t, f32x16* cur, f32x16* nxt) {
        const int c = t & 1, n = c ^ 1;     // slots of tile t and tile t + 1
        // every wave is past iteration t - 1: K slot c, v^T slot n and bias slot
        // c are free; this wave's loads of K(t + 1), bias(t + 1) and v^T(t) landed
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);

        // ---- S(t + 1) = bias + K Q'^T with the exponentials of S(t) interleaved.
        //      The bias is read before this iteration's first direct load is
        //      issued (a read behind an LDS-writing load gets a full vmcnt wait).
        s_init(nxt, n);
        __builtin_amdgcn_sched_barrier(0);
        const bf16_t* sK = kslot(n);
        bf16x8 kf[KD + 1][2];
#pragma unroll
        for (int s = 0; s < KD; ++s) kload(sK, s, kf[s]);
        bf16x8 pb[4];
        float pf[8];
        float psum = 0.f;
        // v^T(t) is in slot c since this iteration's barrier
        const bf16_t* sV = vslot(c);
        bf16x8 vf[VD + 1];
        auto vload = [&](int idx, bf16x8& dst) {      // idx = s4 * 8 + ht
            const int s4 = idx >> 3, ht = idx & 7;
            const int row = ht * 32 + l32;
            const int ch = (2 * s4 + grp) ^ vswz(row);
            dst = *reinterpret_cast<const bf16x8*>(sV + row * KT + ch * 8);
        };
        // p value k (0..31) of S(t): key step s4 = k / 8, element e = k % 8
        auto p_step = [&](int k) {
            const int e = k & 7, s4 = k >> 3;
            const int tt = s4 >> 1, i = 2 * (s4 & 1) + (e >> 2), j = e & 3;
            pf[e] = __builtin_amdgcn_exp2f(cur[tt][i * 4 + j] * ATTN_LOG2E);   // v_exp_f32; argument >= -48 or -inf
            psum += pf[e];
            if (e == 7) pb[s4] = pack8(pf);
        };
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            if (s + KD < 16) kload(sK, s + KD, kf[(s + KD) % (KD + 1)]);
            if (s >= 16 - VD) vload(s - (16 - VD), vf[s - (16 - VD)]);
            // this iteration's direct loads all go out during the S MFMAs, a
            // whole P V phase ahead of the wait at the next iteration's barrier
            if ((s & 1) == 0) issue_k(s >> 1, t + 2, c);
            else issue_v(s >> 1, t + 1, n);
            if (s == 15) issue_b(t + 2, c);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 2; ++u)
                nxt[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % (KD + 1)][u], qf[s], nxt[u], 0, 0, 0);
            p_step(s);   // p values 0..15 (key steps 0, 1) during the S MFMAs
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- O^T += V^T P^T for tile t: 8 independent head-dim chains per key
        //      step, v^T fragments read VD MFMAs ahead (the first VD during the
        //      last S steps)
#pragma unroll
        for (int x = 0; x < 32; ++x) {
            if (x + VD < 32) vload(x + VD, vf[(x + VD) % (VD + 1)]);
            __builtin_amdgcn_sched_barrier(0);
            o[x & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[x % (VD + 1)], pb[x >> 3], o[x & 7], 0, 0, 0);
            if (x < 16) p_step(16 + x);   // p values 16..31 (key steps 2, 3) before their MFMAs
            __builtin_amdgcn_sched_barrier(0);
        }
        l_run += psum;
    };
    int t = 0;
    for (; t + 1 < nt; t += 2) {
        iteration(t, sa, sb);
        iteration(t + 1, sb, sa);
    }
    if (t < nt) iteration(t, sa, sb);
    __builtin_amdgcn_s_waitcnt(0);

    // lane has query q0 + (lane & 31), head dims ht*32 + i*8 + 4 (lane>>5) + j
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    // The outputs leave through LDS: in the accumulator layout a store instruction
    // would write 16 (bf16) or 32 (fp32) bytes per query row; staged, every
    // instruction writes whole rows. Each wave stages and reads back only its own
    // 32 rows, after one barrier that ends every wave's reads of the K and v^T slots.
    if (piece >= 0) {
        // a piece: unnormalised partial O and its sum of p, fp32. Staging: the
        // wave's 32 rows of 1 KB, 16-byte chunk c of row r at c ^ (r & 31).
        __syncthreads();
        float* st = reinterpret_cast<float*>(smem) + wave * 32 * HD;
#pragma unroll
        for (int ht = 0; ht < 8; ++ht)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<float4*>(st + l32 * HD + (((ht * 8 + i * 2 + grp) ^ l32) * 4)) =
                    make_float4(o[ht][i * 4 + 0], o[ht][i * 4 + 1], o[ht][i * 4 + 2], o[ht][i * 4 + 3]);
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's staging writes are done
        __builtin_amdgcn_wave_barrier();
        float* blk = part + (size_t)piece * (QT * HD + QT) + (size_t)(wave * 32) * HD;
#pragma unroll 8
        for (int r = 0; r < 32; ++r)
            *reinterpret_cast<float4*>(blk + r * HD + lane * 4) =
                *reinterpret_cast<const float4*>(st + r * HD + ((lane ^ r) * 4));
        if (grp == 0) part[(size_t)piece * (QT * HD + QT) + QT * HD + wave * 32 + l32] = l_tot;
        return;
    }
    // ---- normalise and store (a query whose keys are all excluded gets zeros)
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int q = q0 + l32;
    if (O8) {
        // MXFP8 output: head-dim block ht (32 values) is held by lanes l and l ^ 32
        const long row = q < S ? g.row_of(b, q) : 0;
#pragma unroll
        for (int ht = 0; ht < 8; ++ht) {
            float amax = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(o[ht][r] * inv));
            amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
            const int e = mx_scale_exp(amax);
            const float sc = inv * pow2f(-e);
            if (q < S) {
                uint8_t* orow = O8 + row * d + h * HD + ht * 32 + grp * 4;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<uint32_t*>(orow + i * 8) =
                        pack4_e4m3(o[ht][i * 4 + 0] * sc, o[ht][i * 4 + 1] * sc, o[ht][i * 4 + 2] * sc, o[ht][i * 4 + 3] * sc);
                if (grp == 0) {
                    const int blk = h * 8 + ht;
                    O8s[((long)(blk >> 1) * sc_rows + row) * 2 + (blk & 1)] = (uint8_t)(e + 127);
                }
            }
        }
        return;
    }
    // bf16 output. Staging: the wave's 32 rows of 512 B, 16-byte chunk c of row r
    // at c ^ (r & 31); a lane's four values are one half of a chunk.
    __syncthreads();
    bf16_t* st = smem + wave * 32 * HD;
#pragma unroll
    for (int ht = 0; ht < 8; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint2*>(st + l32 * HD + (((ht * 4 + i) ^ l32) * 8) + grp * 4) =
                make_uint2(pack2bf(o[ht][i * 4 + 0] * inv, o[ht][i * 4 + 1] * inv),
                           pack2bf(o[ht][i * 4 + 2] * inv, o[ht][i * 4 + 3] * inv));
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's staging writes are done
    __builtin_amdgcn_wave_barrier();
    // one instruction = two rows: lanes 0-31 row 2 k, lanes 32-63 row 2 k + 1,
    // 16 bytes each (logical chunk lane & 31)
#pragma unroll 4
    for (int k = 0; k < 16; ++k) {
        const int r = 2 * k + grp;
        const int qr = q0 + r;
        const uint4 v = *reinterpret_cast<const uint4*>(st + r * HD + ((l32 ^ r) * 8));
        if (qr < S) *reinterpret_cast<uint4*>(O + (long)g.row_of(b, qr) * d + h * HD + l32 * 8) = v;
    }
}

// Sum of the kp partial results of each split query tile, normalised, to O.
// One wave per query: lane l holds head dims [4 l, 4 l + 4).
__global__ __launch_bounds__(256) void k_attention_combine(const float* __restrict__ part, int nfull, int kp,
                                                           int ntail, int nqt, int H, RowGeom g,
                                                           bf16_t* __restrict__ O, int d, uint8_t* __restrict__ O8,
                                                           uint8_t* __restrict__ O8s, long sc_rows) {
    const int lane = threadIdx.x & 63;
    const int w = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (w >= ntail * QT) return;
    const int j = w / QT, ql = w % QT;
    const int tq = nfull + j;
    const int qt = tq % nqt, h = (tq / nqt) % H, b = tq / (nqt * H);
    const int q = qt * QT + ql;
    if (q >= g.S()) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f;
    for (int p = 0; p < kp; ++p) {
        const float* blk = part + (size_t)(j * kp + p) * (QT * HD + QT);
        const float4 v = *reinterpret_cast<const float4*>(blk + ql * HD + lane * 4);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        l += blk[QT * HD + ql];
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const long row = g.row_of(b, q);
    if (O8) {
        // MXFP8 output: one 32-value block = 8 consecutive lanes
        const float y0 = acc.x * inv, y1 = acc.y * inv, y2 = acc.z * inv, y3 = acc.w * inv;
        float amax = fmaxf(fmaxf(fabsf(y0), fabsf(y1)), fmaxf(fabsf(y2), fabsf(y3)));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
        const int e = mx_scale_exp(amax);
        const float sc = pow2f(-e);
        *reinterpret_cast<uint32_t*>(O8 + row * d + h * HD + lane * 4) = pack4_e4m3(y0 * sc, y1 * sc, y2 * sc, y3 * sc);
        if ((lane & 7) == 0) {
            const int blk = h * 8 + (lane >> 3);
            O8s[((long)(blk >> 1) * sc_rows + row) * 2 + (blk & 1)] = (uint8_t)(e + 127);
        }
        return;
    }
    *reinterpret_cast<uint2*>(O + row * d + h * HD + lane * 4) =
        make_uint2(pack2bf(acc.x * inv, acc.y * inv), pack2bf(acc.z * inv, acc.w * inv));
}

size_t attention_bf16_part_floats(int n_cu) { return (size_t)n_cu * (QT * HD + QT); }

hipError_t attention_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* vt, const float* bias, RowGeom g, int H,
                          int S_pad, bf16_t* o, int d, int n_cu, float* part, int part_pieces, uint8_t* o8,
                          uint8_t* o8s, long sc_rows, hipStream_t s) {
    const int S = g.S();
    if (g.B == 0 || S == 0) return hipSuccess;
    const int nqt = (S + QT - 1) / QT, ntiles = (S + KT - 1) / KT;
    const int total = nqt * H * g.B;
    // Wave quantisation: the last `total % n_cu` query tiles would run as a
    // partial round on the n_cu compute units (one workgroup per CU). They are
    // split into kp key ranges each (kp * tail <= n_cu, at least two key tiles
    // per piece) so the partial round is kp times shorter.
    int tail = part && n_cu > 0 ? total % n_cu : 0;
    int kp = tail ? min(min(n_cu, part_pieces) / tail, ntiles / 2) : 1;
    if (kp < 2) tail = 0, kp = 1;
    const int nfull = total - tail;
    hipLaunchKernelGGL(k_attention_bf16, dim3(nfull + tail * kp), dim3(256), 0, s, q, k, vt, bias, g, H, S_pad, o, d,
                       nqt, nfull, kp, part, o8, o8s, sc_rows);
    if (tail) {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_attention_combine, dim3((tail * QT * 64 + 255) / 256), dim3(256), 0, s, part, nfull, kp,
                           tail, nqt, H, g, o, d, o8, o8s, sc_rows);
    }
    return hipGetLastError();
}

}  // namespace af

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
// One workgroup = 4 waves = 128 queries of one (b, h); each wave owns 32 queries
// and keeps them in registers as MFMA B operands. Per 64-key tile:
//   S^T = K Q^T  (A = K rows from LDS) -> one query per lane (lane & 31),
//   P = exp2(S^T * log2(e)/16 - ref + bias),
//   O^T += V^T P^T (A = v^T from LDS, B = P straight from the S^T registers).
// The K rows each lane feeds to the S^T MFMA are permuted (bits 2 and 3 of the
// row index swapped) so that the accumulator registers a lane holds are, per
// 16-key MFMA step, the 8 consecutive keys the P V MFMA expects; v^T is then used
// in its natural key order.
//
// Softmax reference: QK-norm (LayerNorm over the head dim, no affine) gives every
// normalised q and k a norm of at most sqrt(256) = 16, so every logit
// q.k / 16 lies in [-16, 16]. The kernel subtracts a fixed reference of 16.25
// (a margin for bf16 rounding of q and k) instead of a running maximum: softmax
// is invariant to the shift, p stays in [e^-33, 1] (no overflow, no denormals),
// and the running-max bookkeeping and the rescaling of O disappear.
//
// K and v^T tiles move global -> LDS with gfx950 direct loads (buffer_load ...
// lds, 16 bytes per lane; the MUBUF form keeps the compiler's LDS-read waits
// partial), two stages (2 x 64 KB); 16-byte chunks are XOR swizzled by row so
// both operand reads are bank-conflict free. The next tile's loads are spread
// over the MFMAs of the current one (K during S^T, v^T and the bias during
// P V); the last tile re-loads itself into the idle stage so the loop body has
// no branches.
#include "af_internal.h"

namespace af {

namespace {
constexpr int HD = 256;
constexpr int QT = 128;  // queries per workgroup
constexpr int KT = 64;   // keys per tile
constexpr int KTILE = KT * HD;   // bf16 elements of a K (or v^T) tile
constexpr float REF_LOGIT = 16.25f;

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
                      int S_pad, bf16_t* __restrict__ O, int d, float scale_log2) {
    // K0 V0 K1 V1, then per stage and wave a 1 KB bias slot (4 copies of 64 fp32 keys)
    __shared__ __attribute__((aligned(1024))) bf16_t smem[4 * KTILE + 2 * 4 * 512];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 5, l32 = lane & 31;
    const int b = blockIdx.z, h = blockIdx.y;
    const int S = g.S();
    const int q0 = blockIdx.x * QT + wave * 32;
    const long bh = (long)b * H + h;
    const bf16_t* Kbh = K + bh * S_pad * HD;
    const bf16_t* Vbh = Vt + bh * HD * (long)S_pad;
    const float* biasb = bias + (long)b * S_pad;

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
    // one direct load: K rows / v^T rows (instruction j of 8) / bias of the tile at key k0 into `stage`
    auto issue_k = [&](int j, int k0, int stage) {
        bf16_t* sK = smem + stage * 2 * KTILE;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_void*)(sK + (wave * 8 + j) * 512), 16, koff[j], k0 * HD * 2, 0, 0);
    };
    auto issue_v = [&](int j, int k0, int stage) {
        bf16_t* sV = smem + stage * 2 * KTILE + KTILE;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_void*)(sV + (wave * 8 + j) * 512), 16, voff[j & 1],
                                                 k0 * 2 + (j & ~1) * 8 * S_pad * 2, 0, 0);
    };
    auto issue_b = [&](int k0, int stage) {   // 64 fp32 keys, replicated 4x across the 1 KB slot
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void*)(smem + 4 * KTILE + (stage * 4 + wave) * 512), 16,
                                                 (lane & 15) * 16, k0 * 4, 0, 0);
    };

    // The wave's 32 queries as MFMA B operands: lane holds query q0 + (lane & 31),
    // head dims [16 s + 8 (lane >> 5), +8) for k-step s. The workgroup's 128 x 256
    // query tile is staged through the (still idle) second LDS stage so the
    // registers come from LDS reads.
    bf16x8 qf[16];
    {
        bf16_t* sQ = smem + 2 * KTILE;                 // 64 KB: rows of 512 B
        const bf16_t* qsrc = Q + (bh * S_pad + (long)blockIdx.x * QT) * HD;
        const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc((void*)qsrc, (short)0, QT * HD * 2, 0x00020000);
        // 128 rows x 32 chunks = 64 instructions of 1 KB, 16 per wave; lane -> row
        // 2 cb + (lane >> 5), physical chunk lane & 31, logical chunk pc ^ (row & 31).
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            int cb = wave * 16 + j;
            int row = 2 * cb + grp;
            int lc = (lane & 31) ^ (row & 31);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rQ, (lds_void*)(sQ + cb * 512), 16, (row * HD + lc * 8) * 2, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const int row = wave * 32 + l32;
#pragma unroll
        for (int s = 0; s < 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(sQ + row * HD + (((2 * s + grp) ^ (row & 31)) * 8));
        __syncthreads();
    }

    f32x16 o[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
    float l_run = 0.f;
    const float ref = REF_LOGIT * 1.4426950408889634f;

    const int ntiles = (S + KT - 1) / KT;
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_k(j, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_v(j, 0, 0);
    issue_b(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // K rows this lane feeds to the S^T MFMA of sub-tile t: t*32 + swap23(lane & 31).
    const int krow0 = swap23(l32);
    for (int kt = 0; kt < ntiles; ++kt) {
        const int stage = kt & 1;
        const bf16_t* sK = smem + stage * 2 * KTILE;
        const bf16_t* sV = sK + KTILE;
        const float* sB = reinterpret_cast<const float*>(smem + 4 * KTILE + (stage * 4 + wave) * 512);

        // ---- S^T starts at the key bias (0, or -inf for excluded keys); register
        //      (t, i, j) of a lane holds key t*32 + (i/2)*16 + grp*8 + (i%2)*4 + j.
        //      Read before the next tile's loads are issued (they target the other stage).
        f32x16 st[2];
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
        const int knext = min(kt + 1, ntiles - 1) * KT;   // key of the tile loaded during this one

        // ---- S^T += K Q^T: two independent 32-key chains; K fragments read three
        //      k-steps ahead of their MFMAs.
        constexpr int KD = 3;
        bf16x8 kf[KD + 1][2];
        auto kload = [&](int s, bf16x8* dst) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int row = t * 32 + krow0;
                const int ch = (2 * s + grp) ^ kswz(row);
                dst[t] = *reinterpret_cast<const bf16x8*>(sK + row * HD + ch * 8);
            }
        };
#pragma unroll
        for (int s = 0; s < KD; ++s) kload(s, kf[s]);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            if (s + KD < 16) kload(s + KD, kf[(s + KD) % (KD + 1)]);
            if ((s & 1) == 0) issue_k(s >> 1, knext, stage ^ 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % (KD + 1)][t], qf[s], st[t], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- first v^T fragments go out before the exponentials
        constexpr int VD = 4;
        bf16x8 vf[VD + 1];
        auto vload = [&](int idx, bf16x8& dst) {      // idx = s4 * 8 + ht
            const int s4 = idx >> 3, ht = idx & 7;
            const int row = ht * 32 + l32;
            const int ch = (2 * s4 + grp) ^ vswz(row);
            dst = *reinterpret_cast<const bf16x8*>(sV + row * KT + ch * 8);
        };
#pragma unroll
        for (int x = 0; x < VD; ++x) vload(x, vf[x]);

        // ---- P = exp2(S * log2(e)/16 - ref) for key step s4 (16 keys): the lane's
        //      8 values are registers (t, i, j), t = s4/2, i in {2 (s4%2), +1}.
        float psum = 0.f;
        auto p_elem = [&](int s4, int e) {
            const int t = s4 >> 1, i = 2 * (s4 & 1) + (e >> 2), j = e & 3;
            return __builtin_amdgcn_exp2f(st[t][i * 4 + j] * scale_log2 - ref);   // v_exp_f32; argument >= -48 or -inf
        };
        auto pack8 = [&](const float* pf) {
            union { bf16x8 v; uint32_t u[4]; } pk;
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) pk.u[q2] = pack2bf(pf[2 * q2], pf[2 * q2 + 1]);
            return pk.v;
        };
        bf16x8 pb[4];
        {
            float pf[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[e] = p_elem(0, e), psum += pf[e];
            pb[0] = pack8(pf);
        }

        // ---- O^T += V^T P^T: 8 independent head-dim chains per key step, v^T
        //      fragments read four MFMAs ahead; the exponentials of key step
        //      s4 + 1 are computed one per MFMA of step s4.
        float pn[8];
#pragma unroll
        for (int x = 0; x < 32; ++x) {
            const int s4 = x >> 3, sub = x & 7;
            if (x + VD < 32) vload(x + VD, vf[(x + VD) % (VD + 1)]);
            if ((x & 3) == 0) issue_v(x >> 2, knext, stage ^ 1);
            if (x == 2) issue_b(knext, stage ^ 1);
            __builtin_amdgcn_sched_barrier(0);
            o[x & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[x % (VD + 1)], pb[s4], o[x & 7], 0, 0, 0);
            if (s4 + 1 < 4) {
                pn[sub] = p_elem(s4 + 1, sub);
                psum += pn[sub];
                if (sub == 7) pb[s4 + 1] = pack8(pn);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        l_run += psum;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- normalise and store: lane has query q0 + (lane & 31), head dims ht*32 + i*8 + 4 (lane>>5) + j
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.f / l_tot;
    const int q = q0 + l32;
    if (q < S) {
        bf16_t* orow = O + (long)g.row_of(b, q) * d + h * HD + grp * 4;
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

hipError_t attention_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* vt, const float* bias, RowGeom g, int H,
                          int S_pad, bf16_t* o, int d, hipStream_t s) {
    int S = g.S();
    if (g.B == 0 || S == 0) return hipSuccess;
    const float scale_log2 = 1.4426950408889634f / 16.0f;  // log2(e) / sqrt(256)
    dim3 grid((S + QT - 1) / QT, H, g.B);
    hipLaunchKernelGGL(k_attention_bf16, grid, dim3(256), 0, s, q, k, vt, bias, g, H, S_pad, o, d, scale_log2);
    return hipGetLastError();
}

}  // namespace af

// Host-side launch interface between the executor (af_model.hip) and the kernel
// translation units. Every launcher validates nothing: the executor has already
// checked shapes on the host. Each returns the launch's hipError_t.
#pragma once
#include <hip/hip_runtime.h>
#include "af_device.h"
#include "../../include/auraflow.h"

namespace af {

// ------------------------------------------------------------------ GEMM (C = A B^T)
enum GemmEpi {
    EPI_STORE = 0,          // C[m, n] = acc (dtype of the path)
    EPI_STORE_MAPPED = 1,   // resid[map(m), n] = acc (fp32), map = (m/seg_len)*seg_stride + seg_off + m%seg_len
    EPI_GATED_RESID = 2,    // resid[row0 + m, n] += gate[batch(row0 + m), n] * acc
    EPI_QKV = 3,            // bf16 only: per-head LayerNorm of q, k; q, k -> [B,H,S_pad,hd]; v -> v^T [B,H,hd,S_pad]
    EPI_SWIGLU = 4,         // bf16 only: h[m, f] = silu(acc[gate col]) * acc[up col], 32-column interleave
    EPI_GEGLU = 5,          // bf16 only: as SWIGLU with the tanh-form GELU in place of silu (text encoder)
    EPI_PARTIAL = 6,        // bf16 only, one group: split-K partial sums, C = fp32 [ksplit][M][N]; split s
                            // covers K columns [s K/ksplit, (s+1) K/ksplit); splitk_resid adds them up
    EPI_CONV = 7            // bf16 only, one group: C[m, n] = acc + cbias[n] (+ resid[m, n]), fp32 or bf16
                            // (c_bf16), leading dim ldc for C and resid; with conv != 0 the A operand is the
                            // implicit-GEMM gather of a 3x3 convolution (see conv below)
};

struct GemmGroup {
    const void* A; long lda;   // [M, K] row-major (MXFP8: bytes per row)
    const void* W; long ldw;   // [N, K] row-major (weights, y = x W^T)
    const uint8_t* As;         // MXFP8 only: block scales of A, [K/64][as_rows][2] bytes, row 0 of the group
    const uint8_t* Ws;         // MXFP8 only: block scales of W, [K/64][ws_rows][2] bytes
    int M;
    int row0;                  // residual row of GEMM row 0 (GATED_RESID, QKV)
    int gate_off;              // column of gate vector inside a mod row (GATED_RESID)
};

struct GemmLaunch {
    GemmGroup g[2];
    int ngroups;
    int N, K;
    int epi;
    void* C; long ldc;                 // STORE / SWIGLU output (MXFP8 SwiGLU output: fp8, ldc in bytes)
    uint8_t* Cs; long cs_rows;         // MXFP8 SwiGLU output scales, [F/64][cs_rows][2] bytes
    long as_rows, ws_rows;             // MXFP8 operands: rows of one K/64 slab of the scale arrays
    float* resid;                      // MAPPED / GATED_RESID output, leading dim N
    const float* mod; long mod_stride; // gate vectors: mod[b * mod_stride + gate_off + n]
    RowGeom geom;
    int seg_len, seg_stride, seg_off;  // STORE_MAPPED row map
    void* q; void* k; void* vt;        // QKV outputs
    int H, hd, S_pad;
    float eps;
    float q_scale;                     // QKV: factor on the normalised q before rounding (1 = none)
    int ksplit;                        // PARTIAL: number of K ranges (K a multiple of 32 ksplit)
    int n_cu;                          // compute units (0: always 256 x 256 tiles); N a multiple of 256
                                       // (EPI_CONV: a multiple of 128; N % 256 != 0 runs 128 x 128 tiles)
    // EPI_CONV
    const float* cbias;                // [N] or NULL
    int c_bf16;                        // 1: C is bf16, 0: fp32
    // conv = 1: A[m, k] = X[b, y + dy, x + dx, c] for output pixel m = (b, y, x) of an
    // cH x cW image, k = (3 (dy + 1) + dx + 1) cCin + c, X = g[0].A NHWC bf16 with cCin
    // channels (a multiple of 32), zero outside the image (a 3x3 convolution with
    // zero padding, K = 9 cCin); conv = 2: the same on the 2x nearest upsampling of a
    // cH x cW input (the output image is 2cH x 2cW). a_bytes: bytes of X (< 2^31).
    int conv, cH, cW, cCin;
    long a_bytes;
};

hipError_t gemm_bf16(const GemmLaunch& L, hipStream_t s);
// MXFP8 operands (E4M3 values, one power-of-two scale per 32 values along K):
// EPI_QKV, EPI_SWIGLU (MXFP8 output) and EPI_GATED_RESID; K a multiple of 256.
hipError_t gemm_mxfp8(const GemmLaunch& L, hipStream_t s);
hipError_t gemm_f32(const GemmLaunch& L, hipStream_t s);

// ------------------------------------------------------------------ attention
// q, k: [B, H, S_pad, hd]; v^T: [B, H, hd, S_pad] (bf16 path) or v: [B, H, S_pad, hd] (fp32 path);
// bias: [B, S_pad] additive key bias (KEY_KEEP for a kept key, -inf for an
// excluded one); o: [M, d] in residual row order.
// The bf16 kernel uses a fixed softmax reference: it takes q pre-multiplied by
// ATTN_BF16_Q_SCALE = 1/sqrt(256) (a power of two, so the bf16 q it reads is the
// bf16-rounded normalised q, scaled exactly) and the bias with KEY_KEEP =
// ATTN_BF16_KEY_KEEP = -24 ln 2, and forms p = 2^((s + bias) log2 e) = e^s 2^-24
// for the logit s = q.k/16 (QK-norm bounds s to [-16, 16], so p < 1 and no
// denormal). The shift is a whole power of two, so p's bf16 rounding is that
// of e^s. The fp32 kernel takes plain q and KEY_KEEP = 0.
constexpr float ATTN_BF16_Q_SCALE = 1.0f / 16.0f;
constexpr float ATTN_BF16_KEY_KEEP = -24.0f * 0.69314718055994531f;
constexpr float ATTN_LOG2E = 1.4426950408889634f;
// part: scratch for split query tiles, room for part_pieces pieces of
// attention_bf16_part_floats(1) floats each (NULL: no splitting; at most n_cu
// pieces are used); n_cu: compute units of the device. o8 != NULL: the output
// goes to o8 [M, d] as MXFP8 with scales o8s [d/64][sc_rows][2] instead of o.
// A query whose keys are all excluded gets a zero output.
hipError_t attention_bf16(const bf16_t* q, const bf16_t* k, const bf16_t* vt, const float* bias,
                          RowGeom g, int H, int S_pad, bf16_t* o, int d, int n_cu, float* part, int part_pieces,
                          uint8_t* o8, uint8_t* o8s, long sc_rows, hipStream_t s);
size_t attention_bf16_part_floats(int pieces);
hipError_t attention_f32(const float* q, const float* k, const float* v, const float* bias,
                         RowGeom g, int H, int hd, int S_pad, float* o, int d, hipStream_t s);

// ------------------------------------------------------------------ small kernels
hipError_t timestep_features(const float* tau, int B, int half, float tscale, float* e, hipStream_t s);
// y[b, n] = sum_k W[n, k] * act(x[b, k]) + bias[n]   (act = silu when silu_in)
hipError_t gemv(const float* x, int B, int K, const void* W, af_dtype wdt, int N,
                const void* bias, int silu_in, float* y, hipStream_t s);
hipError_t patch_embed(const float* lat, int C, int H, int W, int p, const void* pe_w,
                       const void* pe_b, af_dtype wdt, const float* pos, int G, float* resid,
                       RowGeom g, int d, hipStream_t s);
hipError_t copy_registers(const void* reg, af_dtype wdt, int R, float* resid, RowGeom g, int d,
                          hipStream_t s);
hipError_t f32_to_bf16(const float* src, bf16_t* dst, long n, hipStream_t s);
hipError_t key_bias(const uint8_t* mask, int T, int R, RowGeom g, int S_pad, float keep, float* bias,
                    hipStream_t s);
// out[r] = LN(x[r]) * (1 + scale) + shift; rows r < split use offsets (sh_a, sc_a), others (sh_b, sc_b)
hipError_t ln_modulate(const float* x, int M, int d, RowGeom g, int split, const float* mod,
                       long mod_stride, int sh_a, int sc_a, int sh_b, int sc_b, void* out,
                       af_dtype odt, float eps, hipStream_t s);
// MXFP8 variant: fp8 rows out [M, d] (row stride d bytes) and block scales sc
// [d/64][sc_rows][2]; d a multiple of 256.
hipError_t ln_modulate_mx(const float* x, int M, int d, RowGeom g, int split, const float* mod, long mod_stride,
                          int sh_a, int sc_a, int sh_b, int sc_b, uint8_t* out, uint8_t* sc, long sc_rows, float eps,
                          hipStream_t s);
// bf16 [N, K] -> MXFP8 [N, K] + scales [K/64][N][2].
hipError_t mx_quantize_rows(const bf16_t* src, long N, int K, uint8_t* dst, uint8_t* sc, hipStream_t s);
hipError_t prefinal_project(const float* resid, RowGeom g, int d, const float* mod, long mod_stride,
                            int sc_off, int sh_off, const void* Wout, af_dtype wdt, int Cout, int p,
                            int h, int w, float* out, hipStream_t s);
hipError_t euler_cfg(float* x, const float* v, long n, float dt, float guidance, int cfg_on,
                     hipStream_t s);
// xin = [x; x] (cfg_on) or x, n elements per copy; tau[0 .. (cfg_on ? 2 Bi : Bi)) = sigma
hipError_t cfg_inputs(const float* x, long n, int Bi, int cfg_on, float sigma, float* xin, float* tau,
                      hipStream_t s);
enum PackLayout { PACK_PLAIN = 0, PACK_FFN_GATE = 1, PACK_FFN_UP = 2 };
// Converts src[0, n) (a slice of one canonical tensor starting at element `first`) into dst.
hipError_t pack_weights(const float* src, long n, long first, void* dst, af_dtype ddt, int layout,
                        int cols, hipStream_t s);
hipError_t taps_permute(const float* resid, RowGeom g, int d, float* out, hipStream_t s);
hipError_t qknorm_scatter_f32(const float* raw, int M, RowGeom g, int H, int hd, int S_pad,
                              float eps, float* q, float* k, float* v, int row0, hipStream_t s);
hipError_t swiglu_f32(const float* raw, int M, int F, float* h, hipStream_t s);

// ------------------------------------------------------------------ text encoder (UMT5)
hipError_t umt5_embed(const int32_t* ids, long M, const bf16_t* E, int vocab, int d, float* x, hipStream_t s);
// out = x / sqrt(mean(x^2) + eps) * w per row; bf16 or fp32 output
hipError_t umt5_rms_norm(const float* x, int M, int d, const float* w, float eps, void* out, bool bf16_out,
                         hipStream_t s);
// rows[l][h][rel + T - 1] = rel_bias[l][bucket(rel)][h] (32 buckets, max distance 128)
hipError_t umt5_rel_bias_rows(const float* rel_bias, int L, int H, int T, float* rows, hipStream_t s);
// qkv [B*T (+ padding), 3d] bf16 (q | k | v column blocks, head h at h*64); bias_rows [H][2T-1];
// out [B*T, d] bf16; T <= 512
hipError_t umt5_attention(const bf16_t* qkv, int B, int T, int H, int d, const float* bias_rows,
                          const uint8_t* mask, bf16_t* out, hipStream_t s);

// ------------------------------------------------------------------ VAE decode
// Activations NHWC [B, P, C] (P pixels per sample).
// out[b, p, :Cpad] = bf16(Wpq (lat[b, :, p] / scaling) + bpq), zero past Cl; Cl <= 32.
hipError_t vae_prep(const float* lat, int B, int Cl, long P, float scaling, const float* wpq, const float* bpq,
                    int Cpad, bf16_t* out, hipStream_t s);
// GroupNorm statistics of x [B, P, C] over G groups: stats[b G + g] = (mean, 1/sqrt(var + eps));
// part: scratch of gn_part_floats(B, P, G) floats. C a multiple of 4 G, C <= 1024.
size_t gn_part_floats(int B, long P, int G);
hipError_t group_norm_stats(const float* x, int B, long P, int C, int G, float eps, float4* part, float2* stats,
                            hipStream_t s);
// y = bf16(act((x - mean) rstd gamma + beta)), act = SiLU when silu != 0.
hipError_t group_norm_apply(const float* x, int B, long P, int C, int G, const float2* stats, const float* gamma,
                            const float* beta, int silu, bf16_t* y, hipStream_t s);
// P[r, j] = softmax_j(scale S[r, j]) over j < n, 0 for n <= j < ld; rows x ld, bf16 out.
hipError_t softmax_rows(const float* S, long rows, long ld, int n, float scale, bf16_t* P, hipStream_t s);
// vt[c, p] = src[p lds + c] (p < P), zero for P <= p < Ppad; vt is [C][Ppad].
hipError_t transpose_cols(const bf16_t* src, long lds, long P, int C, long Ppad, bf16_t* vt, hipStream_t s);
// 3x3 convolution (zero padding) of a [B, H, W, Cin] bf16 to Cout <= 4 channels, image NCHW fp32;
// w [Cout][9 Cin] bf16 in the GEMM's column order (tap Cin + c), bias fp32.
hipError_t conv_out3x3(const bf16_t* a, int B, int H, int W, int Cin, const bf16_t* w, const float* bias, int Cout,
                       float* img, hipStream_t s);
enum VaePack { VAE_PACK_BF16 = 0, VAE_PACK_CONV3 = 1, VAE_PACK_F32R = 2 };
hipError_t vae_pack(const float* src, long n, long first, void* dst, int mode, int cin, int cpad, hipStream_t s);

// resid[m, n] += sum over s = 0 .. ks-1, in that order, of part[s][m][n] (the EPI_PARTIAL output)
hipError_t splitk_resid(const float* part, int ks, long M, int N, float* resid, hipStream_t s);

// Records `msg` as this thread's last error (af_last_error) and returns s.
af_status report(af_status s, const char* msg);

}  // namespace af

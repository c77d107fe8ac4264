/*
 * auraflow.h — C ABI of the MI355X (gfx950) AuraFlow transformer library.
 *
 * One denoising forward of the AuraFlow MMDiT/DiT transformer and the
 * flow-matching Euler + classifier-free-guidance latent update, computed by
 * hand-written HIP kernels. Plain pointers and sizes only; no C++ or torch
 * types cross this boundary and nothing throws across it.
 *
 * Sources (the web pages the operations follow):
 *   [PIPE]  "Diffusers 中 AuraFlow 管线实战：从 bitsandbytes 量化到 torch.compile 加速"
 *   [TRANS] "Diffusers 中的 AuraFlowTransformer2DModel：架构解析与源码级使用指南"
 *   [DEEP]  "【深度拆解】AuraFlow从基座到技术实现：开源文生图新范式"
 *
 * Conventions for every call:
 *   - Device pointers are HIP device memory on the model's device; host
 *     pointers are ordinary host memory. Each argument says which.
 *   - The caller owns every buffer it passes; the library owns the weights and
 *     the workspace it allocates in af_create and frees in af_destroy.
 *   - Calls that take a `stream` (a hipStream_t passed as void*; NULL = the
 *     null stream) only enqueue work and return without synchronising.
 *   - Argument and shape errors are detected on the host before anything is
 *     enqueued; the call then returns a non-OK status, af_last_error() gives
 *     a message, and no device memory is touched.
 *   - One model handle must not be used from two streams at once.
 */
#ifndef AURAFLOW_H
#define AURAFLOW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    AF_OK = 0,
    AF_E_INVALID_ARG = 1,   /* null pointer, negative size, bad enum value     */
    AF_E_SHAPE = 2,         /* sizes violate the model's shape rules            */
    AF_E_UNSUPPORTED = 3,   /* valid model, but not a configuration built here  */
    AF_E_OOM = 4,           /* device or host allocation failed                 */
    AF_E_HIP = 5,           /* a HIP runtime call or kernel launch failed       */
    AF_E_STATE = 6          /* call out of order (e.g. forward before weights)  */
} af_status;

typedef enum { AF_F32 = 0, AF_BF16 = 1, AF_MXFP8 = 2 } af_dtype;

/*
 * Model configuration. Field names follow the constructor parameters listed
 * in [TRANS] section 构造参数详解; inner dim d = num_attention_heads *
 * attention_head_dim; FFN width F = find_multiple(int(2/3 * 4d), 256)
 * ([TRANS] 核心子模块架构, FeedForward). pos_embed_max_size must be a
 * perfect square G*G (the table is viewed as a G x G grid).
 *
 * compute_dtype AF_BF16: bf16 weights (the position table stays fp32), fp32
 * accumulation, fp32 norm statistics and residual stream. Requires
 * attention_head_dim == 256, d % 256 == 0 and joint_attention_dim % 64 == 0.
 * compute_dtype AF_MXFP8: the AF_BF16 model with the QKV projection, the
 * out-projection and both FFN products computed on MXFP8 operands (the MI355X
 * counterpart of the 8-bit weight variants in [PIPE] 量化加载：用 bitsandbytes
 * 将模型压到 8-bit): their weights, the LayerNorm + modulate outputs and the
 * attention output feeding them and the SiLU-gated hidden activations are
 * stored as E4M3 values with one power-of-two scale per
 * 32 values along the contraction axis (scale 2^(floor(log2(max |x|)) - 8),
 * values clamped to +-448 and rounded to nearest even), multiplied on the fp8
 * matrix cores with fp32 accumulation. Attention itself and everything else
 * stay as in AF_BF16. The weights are loaded as for AF_BF16;
 * the library quantizes them once the whole list is loaded. Requires, in
 * addition, d % 256 == 0.
 * compute_dtype AF_F32: everything fp32; requires attention_head_dim <= 64
 * and d % 4 == 0.
 * The max_* fields size the workspace; later calls may use any size up to them.
 */
typedef struct {
    int in_channels;              /* latent channels C (4)                         */
    int out_channels;             /* output channels (4)                           */
    int patch_size;               /* p (2)                                         */
    int num_mmdit_layers;         /* joint blocks (4)                              */
    int num_single_dit_layers;    /* single blocks (32)                            */
    int num_attention_heads;      /* H (12)                                        */
    int attention_head_dim;       /* hd (256)                                      */
    int joint_attention_dim;      /* text embedding width (2048)                   */
    int caption_projection_dim;   /* must equal d                                  */
    int pos_embed_max_size;       /* G*G (9216 = 96*96)                            */
    int num_register_tokens;      /* prepended learned tokens (8)                  */
    af_dtype compute_dtype;
    float ln_eps;                 /* LayerNorm / QK-norm epsilon (1e-6)            */
    float timestep_scale;         /* features use u = timestep_scale * tau (1000)  */
    int max_batch;                /* transformer batch upper bound                 */
    int max_latent_h, max_latent_w;
    int max_text_len;             /* T upper bound                                 */
} af_config;

typedef struct af_model af_model;

/* Fills *cfg with the full AuraFlow configuration at bf16, sized for batch 2,
 * 128 x 128 latents and 256 text tokens. Host only. */
af_status af_config_default(af_config* cfg);

/*
 * Host-only validation of a configuration and one call's sizes (no device
 * work, no model needed). B = transformer batch, H x W = latent size,
 * T = text tokens. Mirrors the pipeline's input checks ([PIPE] section
 * AuraFlowPipeline 核心参数详解: resolution must divide evenly, else an
 * error): H and W must be multiples of patch_size; the patch grid must fit
 * the position grid ([TRANS] 核心子模块架构, Patch Embedding); B, H, W, T
 * must not exceed the max_* fields. B == 0 or T == 0 are valid (empty batch,
 * no text tokens).
 */
af_status af_check_shapes(const af_config* cfg, int B, int H, int W, int T);

/*
 * Canonical weight list. The weights are one fp32 blob, tensors in this order
 * (Linear weights are [out, in]; y = x W^T):
 *   t_w1 [d,256] t_b1 [d] t_w2 [d,d] t_b2 [d]         timestep MLP
 *   pe_w [d, C p p] pe_b [d] pos_embed [G*G, d]       patch embed + PE table
 *   ctx_w [d, Dtxt] registers [R, d]                  caption projection (no bias), register tokens
 *   per joint block j, stream img then txt:
 *      ada [6d,d] wq wk wv wo [d,d] ff1 ff2 [F,d] ff3 [d,F]
 *   per single block i: ada wq wk wv wo ff1 ff2 ff3
 *   final_ada [2d,d] proj_out [p p C_out, d]
 * af_weight_count returns the number of tensors and (if total_floats is not
 * NULL) the blob length in floats. af_weight_info describes tensor `index`:
 * its name (NUL-terminated, copied into name[name_cap]), rows, cols (cols = 1
 * for vectors) and blob offset in floats. Host only.
 */
af_status af_weight_count(const af_config* cfg, int* n_tensors, size_t* total_floats);
af_status af_weight_info(const af_config* cfg, int index, char* name, int name_cap,
                         int64_t* rows, int64_t* cols, size_t* offset);

/* Allocates the weight arena and workspace on `device`. *out receives the handle. */
af_status af_create(const af_config* cfg, int device, af_model** out);

/*
 * Loads floats [offset, offset + n_floats) of the canonical blob from host
 * memory `host` (fp32). Slices may be loaded in any order and any size; a
 * forward is allowed once every float has been loaded at least once. With
 * compute_dtype AF_BF16 each value except the position table is rounded to
 * bfloat16 (round to nearest even) on the device. Synchronous with respect to
 * the host buffer: it may be reused when the call returns.
 */
af_status af_load_weights(af_model* m, const float* host, size_t offset, size_t n_floats,
                          void* stream);
/* Whole blob in one call: af_load_weights(m, host_blob, 0, n_floats, stream). */
af_status af_init_weights(af_model* m, const float* host_blob, size_t n_floats, void* stream);

/*
 * One transformer forward ([TRANS] section 前向传播流程): patch embed with the
 * centre-cropped PE, timestep embedding, caption projection with 8 register
 * tokens prepended, num_mmdit_layers joint blocks, num_single_dit_layers
 * single blocks over [registers; text; image], pre-final modulation,
 * projection and unpatchify.
 *   latents     device fp32 [B, C, H, W]
 *   timestep    device fp32 [B]: tau = t / 1000 as the pipeline passes it
 *               ([TRANS] 在 AuraFlowPipeline 中的实际调用); features use 1000 * tau
 *   text_embeds device [B, T, joint_attention_dim], fp32 or bf16 per text_dtype;
 *               fp32 text is rounded to bf16 on the device for AF_BF16 models
 *   text_mask   device uint8 [B, T], 1 = attend, 0 = padding; NULL = all valid.
 *               Padding keys are excluded from every attention; register and
 *               image keys are always valid.
 *   out         device fp32 [B, out_channels, H, W]
 * The workspace is reused; nothing is allocated. Every kernel of the call is
 * launched on `stream`, in order.
 * Reproducibility: two calls with the same inputs give bit-identical outputs.
 * A sample's output does not depend on the other samples' values, but it may
 * depend on the batch size B (and the latent size): the attention splits the
 * key range of its last, partial round of query tiles across workgroups, and
 * which tiles are split depends on the number of tiles, so the fp32 summation
 * order of a sample's attention - and with it the last bits of its output -
 * can change with B (differences at the level of fp32 rounding, far inside
 * the parity bars).
 */
af_status af_transformer_forward(af_model* m, const float* latents, const float* timestep,
                                 const void* text_embeds, af_dtype text_dtype,
                                 const uint8_t* text_mask, int B, int H, int W, int T,
                                 float* out, void* stream);

/*
 * Same inputs as af_transformer_forward, but stops after block
 * `stop_after_block` (0-based over joint then single blocks; -1 = after the
 * embedding stage) and writes the fp32 residual stream to residual_out
 * (device fp32 [B, R + T + N_img, d], tokens in [registers, text, image]
 * order). For parity checks of individual blocks.
 */
af_status af_transformer_forward_taps(af_model* m, const float* latents, const float* timestep,
                                      const void* text_embeds, af_dtype text_dtype,
                                      const uint8_t* text_mask, int B, int H, int W, int T,
                                      int stop_after_block, float* residual_out, void* stream);

/*
 * The attention step of a block on its own ([TRANS] 注意力处理器与 QKV 融合:
 * QK-norm, then one scaled-dot-product attention over the whole sequence,
 * scale 1/sqrt(head_dim), no dropout, not causal), as the transformer forward
 * computes it, for callers that hold their own projections:
 *   q, k, v     device bf16 [B, S, H * head_dim], token-major (head h in
 *               columns [h * head_dim, (h + 1) * head_dim)): the raw q, k, v
 *               projections. q and k are layer-normalised over each head's
 *               head_dim values (fp32 statistics, biased variance, `eps`, no
 *               affine) before the product.
 *   key_mask    device uint8 [B, S]; key j of sample b is excluded iff
 *               key_mask[b * S + j] == 0. NULL = every key valid. A query whose
 *               keys are all excluded gets a zero output.
 *   out         device bf16 [B, S, H * head_dim], same layout as q; must not
 *               overlap the inputs or the workspace.
 *   workspace   device memory of at least
 *               af_attention_workspace_size(B, S, H, head_dim) bytes, owned by
 *               the caller; its prior content does not matter and it holds
 *               scratch values after the call. A smaller workspace of at least
 *               the size for an unsplit launch is accepted and only limits how
 *               many query tiles of the last partial round are split over key
 *               ranges (the result differs from the split one by fp32 summation
 *               order only).
 * Requires head_dim == 256 (else AF_E_UNSUPPORTED) and S <= 2^20. B, S or H
 * equal to 0 is a no-op. The launches (QK-norm pack, v transpose and key bias,
 * attention, combine) are enqueued on `stream`; nothing is allocated.
 * af_attention_workspace_size returns 0 for invalid sizes.
 */
size_t af_attention_workspace_size(int B, int S, int H, int head_dim);
af_status af_attention(const void* q, const void* k, const void* v, const uint8_t* key_mask, int B, int S,
                       int H, int head_dim, float eps, void* out, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * af_attention without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments and result as af_attention, with
 * the scratch taken from a fixed array of af_attention_noalloc_max_bytes()
 * (64 MiB) that the library holds on every device it runs on until the process
 * ends. Nothing is allocated or freed by the call. The device is the calling
 * thread's current HIP device (the one `stream` belongs to).
 * Limit: the packed operands and key bias, 3 * B * H * S_pad * 512 + B * S_pad * 4
 * bytes rounded up per part (S_pad = S rounded up to 128), must fit the 64 MiB
 * (for example B = 2, H = 12, S <= 1792); larger calls return AF_E_SHAPE before
 * anything is enqueued. Whatever room is left holds the partial sums of split
 * query tiles (up to one piece per compute unit), so a call near the limit
 * splits fewer tiles than af_attention would (results then differ from it by
 * fp32 summation order only).
 * Every call on a device shares that device's scratch and leaves its own
 * intermediate values in it; each call writes everything it later reads, so
 * nothing needs clearing between calls. Calls that overlap in time on one device
 * (on different streams, or from different threads) race on the scratch and
 * must be serialised by the caller.
 */
af_status af_attention_noalloc(const void* q, const void* k, const void* v, const uint8_t* key_mask, int B,
                               int S, int H, int head_dim, float eps, void* out, void* stream);
size_t af_attention_noalloc_max_bytes(void);

/*
 * Flow-matching Euler step with classifier-free guidance ([PIPE] section
 * AuraFlowPipeline 核心参数详解: uncond + s (text - uncond), off for s <= 1;
 * [TRANS] 在 AuraFlowPipeline 中的实际调用: outputs split as (uncond, text)):
 *   latents  device fp32 [Bi, C, H, W], updated in place:
 *            x <- x + (sigma_next - sigma) * v_hat
 *   v        device fp32; guidance > 1: [2 Bi, C, H, W] = [uncond; cond],
 *            v_hat = v_u + guidance (v_c - v_u); otherwise [Bi, C, H, W], v_hat = v.
 * Bi == 0 is a no-op.
 */
af_status af_flow_euler_cfg_step(float* latents, const float* v, int Bi, int C, int H, int W,
                                 float sigma, float sigma_next, float guidance, void* stream);

/*
 * Inputs of one CFG denoising step of the sampling loop ([TRANS] 在
 * AuraFlowPipeline 中的实际调用: the latents are duplicated for the (uncond,
 * cond) halves and every sample gets the step's timestep t/1000 = sigma):
 *   latents  device fp32 [Bi, C, H, W] (read only)
 *   x_in     device fp32; cfg_on != 0: [2 Bi, C, H, W] = [latents; latents],
 *            otherwise [Bi, C, H, W] = latents
 *   tau      device fp32 [2 Bi] (cfg_on != 0) or [Bi], every entry = sigma
 * x_in must not overlap latents. Bi == 0 is a no-op. Errors: negative sizes,
 * NULL pointers with Bi > 0, non-finite sigma -> AF_E_INVALID_ARG.
 */
af_status af_flow_cfg_inputs(const float* latents, int Bi, int C, int H, int W, float sigma, int cfg_on,
                             float* x_in, float* tau, void* stream);

/*
 * Flow-matching sigma schedule (host): sigmas_out[i] for i = 0..num_steps,
 * u_i = 1 - i / num_steps mapped through shift * u / (1 + (shift - 1) u)
 * ([DEEP] section 2.3: shift 1.73, 1000 train timesteps). sigmas_out has
 * num_steps + 1 entries; sigma_0 = 1, sigma_N = 0. The transformer's tau for
 * step i is sigma_i.
 */
af_status af_sigma_schedule(int num_steps, double shift, float* sigmas_out);

/*
 * Diagnostics: per-kernel-class timing. While enabled, every kernel launch of
 * af_transformer_forward / _taps is bracketed by a pair of hipEvents recorded
 * on the call's stream. af_profile(m, 1) clears the counters and starts;
 * af_profile(m, 0) stops. af_profile_read waits for the recorded events and
 * returns, for one class, the summed kernel time in milliseconds and the
 * number of launches since the last af_profile(m, 1).
 */
typedef enum {
    AF_K_GEMM_QKV = 0,      /* QKV projection + QK-norm epilogue            */
    AF_K_GEMM_OUT = 1,      /* attention out-projection + gated residual    */
    AF_K_GEMM_FFN_UP = 2,   /* FFN gate/up projection + SiLU gating         */
    AF_K_GEMM_FFN_DOWN = 3, /* FFN down projection + gated residual         */
    AF_K_ATTENTION = 4,     /* joint attention                              */
    AF_K_LN_MOD = 5,        /* LayerNorm + shift/scale modulation           */
    AF_K_ADALN = 6,         /* timestep MLP + all modulation vectors        */
    AF_K_EMBED = 7,         /* patch embed, registers, caption projection   */
    AF_K_FINAL = 8,         /* pre-final modulation + projection            */
    AF_K_COUNT = 9
} af_kernel_class;

af_status af_profile(af_model* m, int enable);
af_status af_profile_read(af_model* m, int kernel_class, double* total_ms, int64_t* launches);

/* Frees the weights and workspace; NULL is ignored. */
void af_destroy(af_model* m);

const char* af_status_string(af_status s);
/* Message of the last non-OK status returned on this thread ("" if none). */
const char* af_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* AURAFLOW_H */

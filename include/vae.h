/*
 * C ABI of the VAE decode: the AutoencoderKL decoder that turns the sampler's
 * latents into images ([PIPE] AuraFlow 模型与管线概述 and [DOCS] the pipeline's
 * `vae` parameter name the AutoencoderKL; [TRANS] 在 AuraFlowPipeline 中的实际调用
 * and [PIPE] VAE 上转精度: the latents are divided by the VAE's scaling factor
 * before the decode, and an fp16 VAE is upcast for it). Built as a random-weight
 * throughput workload beside the transformer; status codes, af_status_string
 * and af_last_error are those of auraflow.h. Source tags as in auraflow.h, plus
 * [DOCS] "AuraFlow", the Diffusers pipeline documentation page.
 *
 * Architecture (the pages name the class only; this is the reading of the
 * published latent-diffusion KL decoder with the AutoencoderKL defaults):
 * z = latents / scaling_factor; z = post_quant(z) (1x1 conv); x = conv_in(z)
 * (3x3); mid: ResNet, self-attention, ResNet; then one up level per entry of
 * block_out_channels, widest first, each of layers_per_block + 1 ResNet blocks,
 * every level but the last followed by a 2x nearest upsampling and a 3x3 conv;
 * GroupNorm + SiLU; conv_out (3x3) to out_channels. ResNet(x) = skip(x) +
 * conv2(SiLU(GN2(conv1(SiLU(GN1(x)))))), skip a 1x1 conv when the width changes.
 * Attention: single head over the pixels of each sample, on GN(x), 1x1 q/k/v/proj
 * with biases, scale 1/sqrt(C), residual. GroupNorm: `norm_groups` groups, biased
 * variance over the group's channels and all pixels, eps `norm_eps`, per-channel
 * affine. Convolutions have zero padding 1 (3x3) and biases.
 *
 * Precision: matrices and kernels stored in bfloat16 (round to nearest even on
 * the device), biases and GroupNorm parameters as the fp32 values of their
 * bfloat16 rounding; convolutions and projections take bf16 operands (the
 * GroupNorm + SiLU outputs, the attention's q, k, v and probabilities) with
 * fp32 accumulation; the residual stream, GroupNorm statistics and the softmax
 * are fp32. bf16 has fp32's exponent range, so the overflow that the fp16
 * upcast avoids does not arise.
 *
 * Built configurations: 4 up levels; every block width a multiple of 128, at most 1024;
 * norm_groups 32; latent_channels <= 32; out_channels <= 4; latent sizes up to
 * max_latent_h x max_latent_w. Others return AF_E_UNSUPPORTED.
 */
#ifndef AF_VAE_H
#define AF_VAE_H

#include <stddef.h>
#include <stdint.h>

#include "auraflow.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int latent_channels;          /* 4 */
    int out_channels;             /* 3 */
    int block_out_channels[4];    /* 128, 256, 512, 512 (encoder order: the decoder runs them reversed) */
    int layers_per_block;         /* 2: the decoder runs 3 ResNet blocks per level */
    int norm_groups;              /* 32 */
    float norm_eps;               /* 1e-6 */
    float scaling_factor;         /* 0.13025 */
    int max_batch;                /* workspace sizing: latents per call */
    int max_latent_h;             /* workspace sizing: latent height (image height / 8) */
    int max_latent_w;             /* workspace sizing: latent width */
} af_vae_config;

typedef struct af_vae af_vae;

/* Fills the defaults above, max_batch 4, max_latent_h = max_latent_w = 128 (1024 x 1024 images). */
af_status af_vae_config_default(af_vae_config* cfg);

/*
 * Canonical weight list (the order of the fp32 blob), names as "<stage>.<part>":
 * post_quant.w [Cl, Cl], .b; conv_in.w [C0, Cl, 3, 3], .b; mid.res0.*; mid.attn.norm.g,
 * .n, q.w [C0, C0], q.b, k.*, v.*, proj.*; mid.res1.*; up<l>.res<r>.* for l = 0..3,
 * r = 0..layers_per_block, then up<l>.upsample.w/.b for l < 3; norm_out.g, .n;
 * conv_out.w [out, C3, 3, 3], .b. A ResNet block: norm1.g, norm1.n, conv1.w, conv1.b,
 * norm2.g, norm2.n, conv2.w, conv2.b, and shortcut.w [Cout, Cin], .b when Cin != Cout.
 * (C0 = block_out_channels[3], C3 = block_out_channels[0]; .g / .n are GroupNorm
 * scale / shift.) A 3x3 kernel [Cout, Cin, 3, 3] is reported as rows Cout, cols
 * 9 Cin, flattened in (Cin, ky, kx) order; a matrix [out, in] as rows out, cols in;
 * a vector as rows n, cols 1. Same contract as af_weight_count / af_weight_info. Host only.
 */
af_status af_vae_weight_count(const af_vae_config* cfg, int* n_tensors, size_t* total_floats);
af_status af_vae_weight_info(const af_vae_config* cfg, int index, char* name, int name_cap, int64_t* rows,
                             int64_t* cols, size_t* offset);

/* Allocates the weight arena and the workspace (sized for max_batch latents of max_latent_h x max_latent_w) on `device`. */
af_status af_vae_create(const af_vae_config* cfg, int device, af_vae** out);

/*
 * Loads floats [offset, offset + n_floats) of the canonical blob from host
 * memory (fp32); any order and slice size; a decode is allowed once every float
 * has been loaded. Synchronous with respect to the host buffer.
 */
af_status af_vae_load_weights(af_vae* m, const float* host, size_t offset, size_t n_floats, void* stream);

/*
 * Decodes B latents. latents: device fp32 [B, latent_channels, h, w] (as the
 * sampler leaves them, before the division by scaling_factor); image: device fp32
 * [B, out_channels, 8h, 8w]. Enqueued on `stream`; B = 0 enqueues nothing.
 * Errors: AF_E_SHAPE for B > max_batch, h > max_latent_h, w > max_latent_w or
 * h, w < 1; AF_E_STATE before the weights are complete.
 */
af_status af_vae_decode(af_vae* m, const float* latents, int B, int h, int w, float* image, void* stream);

/*
 * As af_vae_decode, but stops after stage `stop_after` and writes that stage's
 * fp32 activation in NHWC order to `out`: 0 conv_in ([B, h, w, C0]), 1 the mid
 * block ([B, h, w, C0]), 2 + l the up level l, its upsampling included
 * ([B, H_l, W_l, block_out_channels[3 - l]], H_l = h 2^(l+1) for l < 3, 8h for
 * l = 3). The per-stage parity tap.
 */
af_status af_vae_decode_taps(af_vae* m, const float* latents, int B, int h, int w, int stop_after, float* out,
                             void* stream);

/* Frees everything; NULL is ignored. */
void af_vae_destroy(af_vae* m);

#ifdef __cplusplus
}
#endif

#endif /* AF_VAE_H */

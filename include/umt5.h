/*
 * C ABI of the text encoder: the UMT5 encoder that the AuraFlow pipeline runs on
 * the prompt tokens ([DEEP] section 2.1 文本编码器 gives its configuration: d_model
 * 2048, 32 heads, 24 layers, d_ff 5120, vocabulary 32128, relative-attention
 * maximum distance 128; [DOCS] AuraFlowPipeline parameters and [TRANS] 在
 * AuraFlowPipeline 中的实际调用 name it as the frozen T5-family encoder whose
 * [batch, seq_len, 2048] output is the transformer's text input). Built as a
 * random-weight throughput workload beside the transformer; status codes,
 * af_status_string and af_last_error are those of auraflow.h.
 *
 * Arithmetic (the pages give only the configuration; these are the readings of
 * the published T5 encoder with the UMT5 choices): token embedding lookup; per
 * layer x += SelfAttention(Norm(x)), x += FFN(Norm(x)); final Norm. Norm(x) =
 * x / sqrt(mean(x^2) + eps) * weight. Attention: heads of d_model / num_heads
 * channels, projections without bias, logits q.k without a 1/sqrt(d) factor plus
 * a per-layer, per-head bias of the relative position (key - query) in
 * bidirectional buckets (half per sign, half/2 exact distances, logarithmic steps
 * up to rel_max_distance), padded keys excluded, and a zero output for a query
 * whose sample has no valid token. FFN: wo_ff(gelu_tanh(wi0 x) * wi1 x).
 *
 * Precision: embedding and matrices stored in bfloat16 (round to nearest even
 * on the device), norm weights and relative-position tables in fp32; matrix
 * products take bf16 operands with fp32 accumulation; the residual stream, the
 * norms and the softmax are fp32; attention probabilities enter the P.V product
 * as bf16.
 *
 * Built configurations: d_model / num_heads = 64, d_model a multiple of 256,
 * d_ff a multiple of 128, rel_buckets = 32 with rel_max_distance = 128, at most
 * 512 tokens per sample. Others return AF_E_UNSUPPORTED.
 */
#ifndef AF_UMT5_H
#define AF_UMT5_H

#include <stddef.h>
#include <stdint.h>

#include "auraflow.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int d_model;            /* 2048 */
    int num_heads;          /* 32 */
    int num_layers;         /* 24 */
    int d_ff;               /* 5120 */
    int vocab_size;         /* 32128 */
    int rel_buckets;        /* 32 */
    int rel_max_distance;   /* 128 */
    float eps;              /* 1e-6 */
    int max_batch;          /* workspace sizing: samples per call */
    int max_tokens;         /* workspace sizing: tokens per sample (<= 512) */
} af_umt5_config;

typedef struct af_umt5 af_umt5;

/* Fills the pages' configuration, max_batch 8, max_tokens 256. */
af_status af_umt5_config_default(af_umt5_config* cfg);

/*
 * Canonical weight list (the order of the fp32 blob): embed [vocab, d]; per layer
 * l: ln1 [d], wq [d, d], wk [d, d], wv [d, d], wo [d, d], rel_bias [buckets,
 * heads], ln2 [d], wi0 [d_ff, d], wi1 [d_ff, d], wo_ff [d, d_ff]; final_ln [d].
 * Matrices are [out, in] (y = x W^T). Same contract as af_weight_count /
 * af_weight_info (names "layer<l>.<tensor>"). Host only.
 */
af_status af_umt5_weight_count(const af_umt5_config* cfg, int* n_tensors, size_t* total_floats);
af_status af_umt5_weight_info(const af_umt5_config* cfg, int index, char* name, int name_cap, int64_t* rows,
                              int64_t* cols, size_t* offset);

/* Allocates the weight arena and workspace on `device`. */
af_status af_umt5_create(const af_umt5_config* cfg, int device, af_umt5** out);

/*
 * Loads floats [offset, offset + n_floats) of the canonical blob from host
 * memory (fp32); any order and slice size; an encode is allowed once every float
 * has been loaded. Synchronous with respect to the host buffer.
 */
af_status af_umt5_load_weights(af_umt5* m, const float* host, size_t offset, size_t n_floats, void* stream);

/*
 * Encodes B samples of T tokens. ids: device int32 [B, T] (an id outside
 * [0, vocab_size) reads a zero embedding row); mask: device uint8 [B, T]
 * (nonzero = valid token) or NULL (all valid); out: device fp32 [B, T, d_model],
 * written for every token (padded tokens included). Enqueued on `stream`;
 * B = 0 or T = 0 enqueues nothing. Errors: AF_E_SHAPE for B > max_batch or
 * T > max_tokens, AF_E_STATE before the weights are complete.
 */
af_status af_umt5_encode(af_umt5* m, const int32_t* ids, const uint8_t* mask, int B, int T, float* out,
                         void* stream);

/*
 * As af_umt5_encode, but stops after layer `stop_after_layer` (0-based; -1 = the
 * embedding) and writes the fp32 residual stream [B, T, d_model] before the
 * final norm (the per-layer parity tap).
 */
af_status af_umt5_encode_taps(af_umt5* m, const int32_t* ids, const uint8_t* mask, int B, int T,
                              int stop_after_layer, float* residual_out, void* stream);

/* Frees everything; NULL is ignored. */
void af_umt5_destroy(af_umt5* m);

#ifdef __cplusplus
}
#endif

#endif /* AF_UMT5_H */

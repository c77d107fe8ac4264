// Stand-alone joint attention with QK-norm (af_attention in include/auraflow.h):
// the attention step of a block ([TRANS] 注意力处理器与 QKV 融合: per-head
// LayerNorm of q and k, one scaled-dot-product attention over the whole
// sequence, scale 1/sqrt(head_dim), padded keys excluded) on caller-supplied
// projections in token-major layout.
//
// Three launches on the caller's stream: the QK-norm pack (q and k normalised
// over the head dimension, q pre-scaled by 1/16 for the attention kernel's
// fixed-reference softmax, both scattered to [B, H, S_pad, 256]), the v^T pack
// ([B, H, 256, S_pad] through an LDS transpose) plus the key bias, then the
// attention kernel the transformer forward uses (and its split-tile combine).
// Padding rows and columns of the packed operands are written as zeros on every
// call, so a workspace of any prior content is valid.
#include <algorithm>
#include <cstdio>
#include <mutex>

#include "af_internal.h"

using namespace af;

namespace {

constexpr int HD = 256;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Byte layout of the workspace of one call.
struct AttnWs {
    size_t qk_bytes, bias_off, part_off, total;
    int S_pad;
};

AttnWs attn_ws(int B, int S, int H, int pieces) {
    AttnWs w;
    w.S_pad = (S + 127) / 128 * 128;
    w.qk_bytes = align256((size_t)B * H * w.S_pad * HD * 2);
    w.bias_off = 3 * w.qk_bytes;
    w.part_off = w.bias_off + align256((size_t)B * w.S_pad * 4);
    w.total = w.part_off + (size_t)pieces * attention_bf16_part_floats(1) * 4;
    return w;
}

// One wave per (b, s, h): q and k rows of 256 values, 4 per lane. LayerNorm
// over the head dimension in fp32 (biased variance, no affine), q multiplied by
// q_scale before rounding to bf16. Rows s in [S, S_pad) are written as zeros.
__global__ __launch_bounds__(256) void k_attn_pack_qk(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                      int B, int S, int H, int S_pad, float eps, float q_scale,
                                                      bf16_t* __restrict__ qp, bf16_t* __restrict__ kp) {
    const int lane = threadIdx.x & 63;
    const long w = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if (w >= (long)B * S_pad * H) return;
    const int h = (int)(w % H);
    const long bs = w / H;
    const int s = (int)(bs % S_pad), b = (int)(bs / S_pad);
    const long dst = (((long)b * H + h) * S_pad + s) * HD + lane * 4;
    if (s >= S) {
        *reinterpret_cast<uint2*>(qp + dst) = make_uint2(0u, 0u);
        *reinterpret_cast<uint2*>(kp + dst) = make_uint2(0u, 0u);
        return;
    }
    const long src = ((long)b * S + s) * ((long)H * HD) + (long)h * HD + lane * 4;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const uint2 raw = *reinterpret_cast<const uint2*>((which ? k : q) + src);
        float v[4] = {bf2f((bf16_t)(raw.x & 0xffff)), bf2f((bf16_t)(raw.x >> 16)), bf2f((bf16_t)(raw.y & 0xffff)),
                      bf2f((bf16_t)(raw.y >> 16))};
        const float mean = wave_sum(v[0] + v[1] + v[2] + v[3]) * (1.f / HD);
        float c2 = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] -= mean;
            c2 += v[j] * v[j];
        }
        const float r = rsqrtf(wave_sum(c2) * (1.f / HD) + eps) * (which ? 1.f : q_scale);
        *reinterpret_cast<uint2*>((which ? kp : qp) + dst) =
            make_uint2(pack2bf(v[0] * r, v[1] * r), pack2bf(v[2] * r, v[3] * r));
    }
}

// One workgroup per (b, h, 64-token block): v rows [64][256] through LDS to
// v^T rows [256][64 tokens], each v^T row segment leaving as 128 contiguous
// bytes (eight 16-byte stores by eight consecutive threads). Tokens past S are
// zeros. The workgroup with block index 0 of each (b, h) also writes that
// sample's key bias when h == 0.
__global__ __launch_bounds__(256) void k_attn_pack_vt(const bf16_t* __restrict__ v, const uint8_t* __restrict__ mask,
                                                      int B, int S, int H, int S_pad, float keep,
                                                      bf16_t* __restrict__ vt, float* __restrict__ bias) {
    constexpr int TB = 64, LS = HD + 8;   // tokens per block, LDS row stride (elements)
    __shared__ bf16_t tile[TB * LS];
    const int nblk = S_pad / TB;
    const int blk = blockIdx.x % nblk;
    const int bh = blockIdx.x / nblk;
    const int h = bh % H, b = bh / H;
    const int s0 = blk * TB, tid = threadIdx.x;
    // 64 rows x 32 chunks of 16 B
#pragma unroll
    for (int it = 0; it < TB * 32 / 256; ++it) {
        const int idx = it * 256 + tid;
        const int r = idx >> 5, ch = idx & 31;
        const int s = s0 + r;
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (s < S) val = *reinterpret_cast<const uint4*>(v + ((long)b * S + s) * ((long)H * HD) + (long)h * HD + ch * 8);
        uint32_t* dstp = reinterpret_cast<uint32_t*>(tile + r * LS + ch * 8);
        dstp[0] = val.x; dstp[1] = val.y; dstp[2] = val.z; dstp[3] = val.w;
    }
    __syncthreads();
    // 256 channels x 8 chunks of 8 tokens
#pragma unroll
    for (int it = 0; it < HD * 8 / 256; ++it) {
        const int idx = it * 256 + tid;
        const int c = idx >> 3, ch = idx & 7;
        uint32_t wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            wv[e] = (uint32_t)tile[(ch * 8 + 2 * e) * LS + c] | ((uint32_t)tile[(ch * 8 + 2 * e + 1) * LS + c] << 16);
        *reinterpret_cast<uint4*>(vt + (((long)b * H + h) * HD + c) * (long)S_pad + s0 + ch * 8) =
            make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    if (h == 0 && tid < TB) {
        const int s = s0 + tid;
        const bool valid = s < S && (mask == nullptr || mask[(long)b * S + s] != 0);
        bias[(long)b * S_pad + s] = valid ? keep : -INFINITY;
    }
}

// Scratch of af_attention_noalloc: one fixed array per device, in the code
// object (each GPU the library runs on holds its own copy until the process
// ends). Host code never passes `scratch` itself to a kernel (in host code the
// name is a host-side stand-in, not a device address): its device address is
// looked up once per device with hipGetSymbolAddress and kept in g_scratch.
constexpr size_t NOALLOC_BYTES = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_BYTES];
constexpr int MAX_DEV = 64;
void* g_scratch[MAX_DEV] = {};
std::mutex g_scratch_mu;

int device_cus();

// The current device's scratch address (looked up on the first call on it).
af_status scratch_ptr(char** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return report(AF_E_HIP, hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEV) return report(AF_E_UNSUPPORTED, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return report(AF_E_HIP, "hipGetSymbolAddress of the attention scratch failed");
        g_scratch[dev] = p;
    }
    *out = (char*)g_scratch[dev];
    return AF_OK;
}

int device_cus() {
    static int cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}

af_status check_attn(const void* q, const void* k, const void* v, int B, int S, int H, int hd, float eps,
                     const void* out) {
    if (B < 0 || S < 0 || H < 0) return report(AF_E_INVALID_ARG, "negative size");
    if (hd != HD) return report(AF_E_UNSUPPORTED, "af_attention is built for head_dim 256");
    if (!(eps > 0.f)) return report(AF_E_INVALID_ARG, "eps must be > 0");
    if ((long)B * S * H == 0) return AF_OK;
    if (!q || !k || !v || !out) return report(AF_E_INVALID_ARG, "NULL device pointer");
    if ((long)S > (1L << 20)) return report(AF_E_UNSUPPORTED, "sequence longer than 2^20 tokens");
    return AF_OK;
}

// The three launches of one call on `ws` (layout attn_ws(B, S, H, pieces)).
af_status run_attn(const bf16_t* q, const bf16_t* k, const bf16_t* v, const uint8_t* mask, int B, int S, int H,
                   float eps, bf16_t* out, char* ws, int pieces, hipStream_t s) {
    const AttnWs L = attn_ws(B, S, H, pieces);
    bf16_t* qp = (bf16_t*)ws;
    bf16_t* kp = (bf16_t*)(ws + L.qk_bytes);
    bf16_t* vt = (bf16_t*)(ws + 2 * L.qk_bytes);
    float* bias = (float*)(ws + L.bias_off);
    float* part = pieces > 0 ? (float*)(ws + L.part_off) : nullptr;
    const long rows = (long)B * L.S_pad * H;
    hipLaunchKernelGGL(k_attn_pack_qk, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, q, k, B, S, H, L.S_pad, eps,
                       ATTN_BF16_Q_SCALE, qp, kp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return report(AF_E_HIP, hipGetErrorString(e));
    hipLaunchKernelGGL(k_attn_pack_vt, dim3((unsigned)((long)B * H * (L.S_pad / 64))), dim3(256), 0, s, v, mask, B, S,
                       H, L.S_pad, ATTN_BF16_KEY_KEEP, vt, bias);
    e = hipGetLastError();
    if (e != hipSuccess) return report(AF_E_HIP, hipGetErrorString(e));
    const RowGeom g{B, S, 0};
    e = attention_bf16(qp, kp, vt, bias, g, H, L.S_pad, out, H * HD, device_cus(), part, pieces, nullptr, nullptr, 0,
                       s);
    if (e != hipSuccess) return report(AF_E_HIP, hipGetErrorString(e));
    return AF_OK;
}

}  // namespace

extern "C" {

size_t af_attention_workspace_size(int B, int S, int H, int head_dim) {
    if (B <= 0 || S <= 0 || H <= 0 || head_dim != HD) return 0;
    const int n = device_cus();
    return attn_ws(B, S, H, n > 0 ? n : 256).total;
}

af_status af_attention(const void* q, const void* k, const void* v, const uint8_t* key_mask, int B, int S, int H,
                       int head_dim, float eps, void* out, void* workspace, size_t workspace_bytes, void* stream) {
    af_status st = check_attn(q, k, v, B, S, H, head_dim, eps, out);
    if (st != AF_OK || (long)B * S * H == 0) return st;
    if (!workspace) return report(AF_E_INVALID_ARG, "workspace is NULL");
    // the largest split the workspace has room for (at most one piece per compute unit)
    const AttnWs base = attn_ws(B, S, H, 0);
    if (workspace_bytes < base.total) return report(AF_E_INVALID_ARG, "workspace smaller than af_attention_workspace_size");
    const size_t per = attention_bf16_part_floats(1) * 4;
    const int pieces = (int)std::min<size_t>((workspace_bytes - base.total) / per, (size_t)std::max(device_cus(), 0));
    return run_attn((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, key_mask, B, S, H, eps, (bf16_t*)out,
                    (char*)workspace, pieces, (hipStream_t)stream);
}

af_status af_attention_noalloc(const void* q, const void* k, const void* v, const uint8_t* key_mask, int B, int S,
                               int H, int head_dim, float eps, void* out, void* stream) {
    af_status st = check_attn(q, k, v, B, S, H, head_dim, eps, out);
    if (st != AF_OK || (long)B * S * H == 0) return st;
    const AttnWs base = attn_ws(B, S, H, 0);
    if (base.total > NOALLOC_BYTES) {
        char msg[200];
        snprintf(msg, sizeof msg, "af_attention_noalloc: B * H * S needs %zu bytes of scratch; the fixed scratch holds %zu "
                 "(use af_attention with a workspace)", base.total, NOALLOC_BYTES);
        return report(AF_E_SHAPE, msg);
    }
    char* ws = nullptr;
    st = scratch_ptr(&ws);
    if (st != AF_OK) return st;
    const size_t per = attention_bf16_part_floats(1) * 4;
    const int pieces = (int)std::min<size_t>((NOALLOC_BYTES - base.total) / per, (size_t)std::max(device_cus(), 0));
    return run_attn((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, key_mask, B, S, H, eps, (bf16_t*)out, ws,
                    pieces, (hipStream_t)stream);
}

size_t af_attention_noalloc_max_bytes(void) { return NOALLOC_BYTES; }

}  // extern "C"

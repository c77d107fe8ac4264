// Executor behind include/vae.h: configuration checks, the weight list and its
// packing, the workspace and the launch sequence of one decode (the AutoencoderKL
// decoder of [PIPE] AuraFlow 模型与管线概述, run as a random-weight workload).
//
// Data flow per ResNet block (activations NHWC, one GEMM row per pixel):
//   x (fp32) -> GroupNorm statistics -> normalise + affine + SiLU -> a (bf16)
//   -> 3x3 conv (implicit GEMM, bias in the epilogue) -> h (fp32) -> GroupNorm
//   -> a -> 3x3 conv with the skip added in the epilogue -> new x (fp32).
// The skip is x itself (the epilogue reads and writes it in place) or a 1x1
// convolution of bf16(x) when the width changes. Upsampling is folded into the
// next convolution's gather (each output pixel reads input pixel (y/2, x/2)).
// The mid-block attention runs per sample on the GEMM: S = Q K^T (fp32), a row
// softmax to bf16 probabilities, O = P V with V transposed, then the output
// projection with the residual added in its epilogue.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "af_internal.h"
#include "../../include/vae.h"

using namespace af;

namespace {

#define V_FAIL(st, msg) return af::report((st), (msg))
#define V_HIP(call)                                                                                  \
    do {                                                                                             \
        hipError_t e_ = (call);                                                                      \
        if (e_ != hipSuccess) return af::report(AF_E_HIP, (std::string(#call) + ": " + hipGetErrorString(e_)).c_str()); \
    } while (0)

constexpr int CIN_PAD = 32;    // conv_in's input channels, padded for the GEMM's 32-wide K sub-tiles
constexpr long A_PAD_ROWS = 256;

struct VSlot {
    std::string name;
    int64_t rows, cols;
    size_t offset;     // floats, in the canonical blob
    int buf;           // destination buffer
    size_t dst_elem;   // element offset in the destination
    int mode;          // VaePack
    int cin, cpad;     // VAE_PACK_CONV3
};

struct VRes {
    int cin, cout;
    int n1g, n1n, c1w, c1b, n2g, n2n, c2w, c2b, scw = -1, scb = -1;   // buffer ids
};

af_status check_config(const af_vae_config* c) {
    if (!c) V_FAIL(AF_E_INVALID_ARG, "config is NULL");
    if (c->latent_channels <= 0 || c->out_channels <= 0 || c->layers_per_block < 0 || c->norm_groups <= 0 ||
        c->max_batch < 0 || c->max_latent_h < 0 || c->max_latent_w < 0)
        V_FAIL(AF_E_INVALID_ARG, "config has a negative or zero size");
    for (int i = 0; i < 4; ++i)
        if (c->block_out_channels[i] <= 0) V_FAIL(AF_E_INVALID_ARG, "block_out_channels must be positive");
    if (!(c->norm_eps > 0.f) || !(c->scaling_factor > 0.f) || !std::isfinite(c->scaling_factor))
        V_FAIL(AF_E_INVALID_ARG, "norm_eps and scaling_factor must be positive");
    for (int i = 0; i < 4; ++i)
        if (c->block_out_channels[i] % 128 != 0 || c->block_out_channels[i] > 1024)
            V_FAIL(AF_E_UNSUPPORTED, "block widths must be multiples of 128, at most 1024");
    if (c->norm_groups != 32) V_FAIL(AF_E_UNSUPPORTED, "32 GroupNorm groups are built");
    if (c->latent_channels > CIN_PAD) V_FAIL(AF_E_UNSUPPORTED, "at most 32 latent channels");
    if (c->out_channels > 4) V_FAIL(AF_E_UNSUPPORTED, "at most 4 output channels");
    return AF_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct DevGuard {
    int prev = -1;
    explicit DevGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != dev) (void)hipSetDevice(dev);
    }
    ~DevGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

// Channel width of up level l (widest first).
int up_ch(const af_vae_config& c, int l) { return c.block_out_channels[3 - l]; }

}  // namespace

struct af_vae {
    af_vae_config cfg;
    int device = 0;
    std::vector<VSlot> slots;
    std::vector<size_t> buf_bytes;
    std::vector<void*> bufs;
    size_t total_floats = 0;
    std::map<size_t, size_t> loaded;
    void* arena = nullptr;
    // buffer ids
    int pq_w = -1, pq_b = -1, ci_w = -1, ci_b = -1;
    VRes mid0{}, mid1{};
    int an_g = -1, an_n = -1, a_qkv_w = -1, a_qkv_b = -1, a_pj_w = -1, a_pj_b = -1;
    std::vector<VRes> res[4];
    int ups_w[3] = {-1, -1, -1}, ups_b[3] = {-1, -1, -1};
    int no_g = -1, no_n = -1, co_w = -1, co_b = -1;
    // workspace
    size_t act_floats = 0;       // capacity of X, H, S (fp32) and A (bf16, plus padding rows)
    float* X = nullptr;
    float* Hb = nullptr;
    float* S = nullptr;
    bf16_t* A = nullptr;
    bf16_t* zin = nullptr;       // conv_in operand [B, h, w, CIN_PAD]
    float4* gpart = nullptr;
    float2* gstats = nullptr;
    bf16_t* qkv = nullptr;       // [B hw + pad, 3 C0]
    bf16_t* att_o = nullptr;     // [B hw + pad, C0]
    bf16_t* vt = nullptr;        // [C0, hw_pad]
    float* logits = nullptr;     // [hw, hw_pad]
    bf16_t* probs = nullptr;     // [hw + pad, hw_pad]
    int n_cu = 0;
    float* staging = nullptr;
    size_t staging_floats = 0;
    void* work = nullptr;
};

namespace {

void build_slots(af_vae* m) {
    const af_vae_config& c = m->cfg;
    const int Cl = c.latent_channels, C0 = up_ch(c, 0);
    auto newbuf = [&](size_t bytes) {
        m->buf_bytes.push_back(bytes);
        return (int)m->buf_bytes.size() - 1;
    };
    size_t off = 0;
    auto add = [&](const std::string& name, int64_t rows, int64_t cols, int buf, size_t dst, int mode, int cin,
                   int cpad) {
        m->slots.push_back(VSlot{name, rows, cols, off, buf, dst, mode, cin, cpad});
        off += (size_t)rows * cols;
    };
    // a 3x3 convolution: bf16 [cout][9 cpad] + fp32 bias
    auto conv3 = [&](const std::string& name, int cout, int cin, int cpad, int* wbuf, int* bbuf) {
        *wbuf = newbuf((size_t)cout * 9 * cpad * 2);
        *bbuf = newbuf((size_t)cout * 4);
        add(name + ".w", cout, 9L * cin, *wbuf, 0, VAE_PACK_CONV3, cin, cpad);
        add(name + ".b", cout, 1, *bbuf, 0, VAE_PACK_F32R, 0, 0);
    };
    auto conv1 = [&](const std::string& name, int cout, int cin, int* wbuf, int* bbuf) {
        *wbuf = newbuf((size_t)cout * cin * 2);
        *bbuf = newbuf((size_t)cout * 4);
        add(name + ".w", cout, cin, *wbuf, 0, VAE_PACK_BF16, 0, 0);
        add(name + ".b", cout, 1, *bbuf, 0, VAE_PACK_F32R, 0, 0);
    };
    auto norm = [&](const std::string& name, int ch, int* g, int* n) {
        *g = newbuf((size_t)ch * 4);
        *n = newbuf((size_t)ch * 4);
        add(name + ".g", ch, 1, *g, 0, VAE_PACK_F32R, 0, 0);
        add(name + ".n", ch, 1, *n, 0, VAE_PACK_F32R, 0, 0);
    };
    auto resnet = [&](const std::string& name, int cin, int cout) {
        VRes r;
        r.cin = cin;
        r.cout = cout;
        norm(name + ".norm1", cin, &r.n1g, &r.n1n);
        conv3(name + ".conv1", cout, cin, cin, &r.c1w, &r.c1b);
        norm(name + ".norm2", cout, &r.n2g, &r.n2n);
        conv3(name + ".conv2", cout, cout, cout, &r.c2w, &r.c2b);
        if (cin != cout) conv1(name + ".shortcut", cout, cin, &r.scw, &r.scb);
        return r;
    };
    // post_quant stays fp32 (its 1x1 product runs in the prep kernel)
    m->pq_w = newbuf((size_t)Cl * Cl * 4);
    m->pq_b = newbuf((size_t)Cl * 4);
    add("post_quant.w", Cl, Cl, m->pq_w, 0, VAE_PACK_F32R, 0, 0);
    add("post_quant.b", Cl, 1, m->pq_b, 0, VAE_PACK_F32R, 0, 0);
    conv3("conv_in", C0, Cl, CIN_PAD, &m->ci_w, &m->ci_b);
    m->mid0 = resnet("mid.res0", C0, C0);
    norm("mid.attn.norm", C0, &m->an_g, &m->an_n);
    m->a_qkv_w = newbuf((size_t)3 * C0 * C0 * 2);
    m->a_qkv_b = newbuf((size_t)3 * C0 * 4);
    const char* qkv[3] = {"q", "k", "v"};
    for (int i = 0; i < 3; ++i) {
        add(std::string("mid.attn.") + qkv[i] + ".w", C0, C0, m->a_qkv_w, (size_t)i * C0 * C0, VAE_PACK_BF16, 0, 0);
        add(std::string("mid.attn.") + qkv[i] + ".b", C0, 1, m->a_qkv_b, (size_t)i * C0, VAE_PACK_F32R, 0, 0);
    }
    conv1("mid.attn.proj", C0, C0, &m->a_pj_w, &m->a_pj_b);
    m->mid1 = resnet("mid.res1", C0, C0);
    int cin = C0;
    for (int l = 0; l < 4; ++l) {
        const int cout = up_ch(c, l);
        for (int r = 0; r <= c.layers_per_block; ++r) {
            m->res[l].push_back(resnet("up" + std::to_string(l) + ".res" + std::to_string(r), cin, cout));
            cin = cout;
        }
        if (l < 3) conv3("up" + std::to_string(l) + ".upsample", cout, cout, cout, &m->ups_w[l], &m->ups_b[l]);
    }
    norm("norm_out", cin, &m->no_g, &m->no_n);
    m->co_w = newbuf((size_t)c.out_channels * 9 * cin * 2);
    m->co_b = newbuf((size_t)c.out_channels * 4);
    add("conv_out.w", c.out_channels, 9L * cin, m->co_w, 0, VAE_PACK_CONV3, cin, cin);
    add("conv_out.b", c.out_channels, 1, m->co_b, 0, VAE_PACK_F32R, 0, 0);
    m->total_floats = off;
}

bool complete(const af_vae* m) {
    size_t cur = 0;
    for (auto& iv : m->loaded) {
        if (iv.first > cur) return false;
        cur = std::max(cur, iv.second);
    }
    return cur >= m->total_floats;
}

void mark_loaded(af_vae* m, size_t a, size_t b) {
    auto& L = m->loaded;
    auto it = L.upper_bound(a);
    if (it != L.begin()) {
        auto pv = std::prev(it);
        if (pv->second >= a) {
            a = pv->first;
            b = std::max(b, pv->second);
            it = L.erase(pv);
        }
    }
    while (it != L.end() && it->first <= b) {
        b = std::max(b, it->second);
        it = L.erase(it);
    }
    L[a] = b;
}

// Largest P C (pixels per sample times channels) of any activation the decode
// holds: the stream, the conv1 outputs, the shortcuts and the bf16 operands.
long max_act(const af_vae_config& c, long hw) {
    long mx = hw * std::max(up_ch(c, 0), CIN_PAD);
    long P = hw;
    int cin = up_ch(c, 0);
    for (int l = 0; l < 4; ++l) {
        mx = std::max(mx, P * std::max(cin, up_ch(c, l)));
        cin = up_ch(c, l);
        if (l < 3) {
            P *= 4;
            mx = std::max(mx, P * cin);
        }
    }
    return mx;
}

#define V_K(call)                                                                                           \
    do {                                                                                                    \
        hipError_t e_ = (call);                                                                             \
        if (e_ != hipSuccess) return af::report(AF_E_HIP, (std::string(#call) + ": " + hipGetErrorString(e_)).c_str()); \
    } while (0)

GemmLaunch base_launch(const af_vae* m, const void* A, long lda, const void* W, long ldw, int M, int N, int K) {
    GemmLaunch L;
    memset(&L, 0, sizeof(L));
    L.ngroups = 1;
    L.g[0].A = A;
    L.g[0].lda = lda;
    L.g[0].W = W;
    L.g[0].ldw = ldw;
    L.g[0].M = M;
    L.N = N;
    L.K = K;
    L.epi = EPI_CONV;
    L.n_cu = m->n_cu;
    return L;
}

// out[b, p, :Cout] = bias + conv3x3(a)[b, p] (+ resid[b, p]) for the B samples of
// a [B, Hin, Win, Cin] bf16; up: the convolution runs on the 2x nearest
// upsampling (output 2Hin x 2Win). Launched over as many samples at a time as
// keep the gathered operand under 2 GiB (the buffer offsets are 32-bit).
af_status conv3x3(af_vae* m, const bf16_t* a, int B, int Hin, int Win, int Cin, bool up, const void* W,
                  const float* bias, const float* resid, float* out, int Cout, hipStream_t s) {
    const long in_px = (long)Hin * Win, out_px = up ? 4 * in_px : in_px;
    const long per_bytes = in_px * Cin * 2;
    if (per_bytes >= (1L << 31)) V_FAIL(AF_E_UNSUPPORTED, "one sample's convolution input exceeds 2 GiB");
    const int per = (int)std::max(1L, ((1L << 31) - 1) / per_bytes);
    for (int b0 = 0; b0 < B; b0 += per) {
        const int nb = std::min(per, B - b0);
        GemmLaunch L = base_launch(m, a + (long)b0 * in_px * Cin, Cin, W, 9L * Cin, (int)(nb * out_px), Cout, 9 * Cin);
        L.conv = up ? 2 : 1;
        L.cH = Hin;
        L.cW = Win;
        L.cCin = Cin;
        L.a_bytes = nb * per_bytes;
        L.cbias = bias;
        L.resid = resid ? const_cast<float*>(resid) + (long)b0 * out_px * Cout : nullptr;
        L.C = out + (long)b0 * out_px * Cout;
        L.ldc = Cout;
        V_K(gemm_bf16(L, s));
    }
    return AF_OK;
}

// out[r, :N] = bias + A[r, :K] W^T (fp32, or bf16 when out_bf16) (+ resid[r]), rows r < M.
af_status gemm1x1(af_vae* m, const bf16_t* A, long lda, const void* W, long ldw, int M, int N, int K,
                  const float* bias, const float* resid, void* out, long ldc, bool out_bf16, hipStream_t s) {
    GemmLaunch L = base_launch(m, A, lda, W, ldw, M, N, K);
    L.cbias = bias;
    L.resid = const_cast<float*>(resid);
    L.C = out;
    L.ldc = ldc;
    L.c_bf16 = out_bf16 ? 1 : 0;
    V_K(gemm_bf16(L, s));
    return AF_OK;
}

#define V_TRY(call)                      \
    do {                                 \
        af_status st_ = (call);          \
        if (st_ != AF_OK) return st_;    \
    } while (0)

struct Act {
    int B, H, W, C;
    long px() const { return (long)H * W; }
};

af_status gn(af_vae* m, const float* x, const Act& a, int g, int n, bool silu, bf16_t* y, hipStream_t s) {
    const af_vae_config& c = m->cfg;
    V_K(group_norm_stats(x, a.B, a.px(), a.C, c.norm_groups, c.norm_eps, m->gpart, m->gstats, s));
    V_K(group_norm_apply(x, a.B, a.px(), a.C, c.norm_groups, m->gstats, (const float*)m->bufs[g],
                         (const float*)m->bufs[n], silu ? 1 : 0, y, s));
    return AF_OK;
}

// x <- ResNet(x); x lives in *X (fp32), which may be swapped with S.
af_status resnet(af_vae* m, const VRes& r, Act& a, float*& X, float*& S, hipStream_t s) {
    auto buf = [&](int id) { return m->bufs[id]; };
    const long M = (long)a.B * a.px();
    float* skip = X;
    if (r.scw >= 0) {
        V_K(f32_to_bf16(X, m->A, M * r.cin, s));
        V_TRY(gemm1x1(m, m->A, r.cin, buf(r.scw), r.cin, (int)M, r.cout, r.cin, (const float*)buf(r.scb), nullptr, S,
                      r.cout, false, s));
        skip = S;
    }
    V_TRY(gn(m, X, a, r.n1g, r.n1n, true, m->A, s));
    V_TRY(conv3x3(m, m->A, a.B, a.H, a.W, r.cin, false, buf(r.c1w), (const float*)buf(r.c1b), nullptr, m->Hb, r.cout,
                  s));
    Act h = a;
    h.C = r.cout;
    V_TRY(gn(m, m->Hb, h, r.n2g, r.n2n, true, m->A, s));
    V_TRY(conv3x3(m, m->A, a.B, a.H, a.W, r.cout, false, buf(r.c2w), (const float*)buf(r.c2b), skip, skip, r.cout,
                  s));
    if (skip == S) std::swap(X, S);
    a.C = r.cout;
    return AF_OK;
}

af_status attention(af_vae* m, const Act& a, float* X, hipStream_t s) {
    auto buf = [&](int id) { return m->bufs[id]; };
    const int C = a.C;
    const long hw = a.px(), hwp = (hw + 127) / 128 * 128, M = (long)a.B * hw;
    V_TRY(gn(m, X, a, m->an_g, m->an_n, false, m->A, s));
    V_TRY(gemm1x1(m, m->A, C, buf(m->a_qkv_w), C, (int)M, 3 * C, C, (const float*)buf(m->a_qkv_b), nullptr, m->qkv,
                  3 * C, true, s));
    const float scale = 1.0f / std::sqrt((float)C);
    for (int b = 0; b < a.B; ++b) {
        const bf16_t* qb = m->qkv + (long)b * hw * 3 * C;
        V_TRY(gemm1x1(m, qb, 3 * C, qb + C, 3 * C, (int)hw, (int)hwp, C, nullptr, nullptr, m->logits, hwp, false, s));
        V_K(softmax_rows(m->logits, hw, hwp, (int)hw, scale, m->probs, s));
        V_K(transpose_cols(qb + 2 * C, 3 * C, hw, C, hwp, m->vt, s));
        V_TRY(gemm1x1(m, m->probs, hwp, m->vt, hwp, (int)hw, C, (int)hwp, nullptr, nullptr,
                      m->att_o + (long)b * hw * C, C, true, s));
    }
    V_TRY(gemm1x1(m, m->att_o, C, buf(m->a_pj_w), C, (int)M, C, C, (const float*)buf(m->a_pj_b), X, X, C, false, s));
    return AF_OK;
}

af_status tap_out(const float* X, const Act& a, float* out, hipStream_t s) {
    V_HIP(hipMemcpyAsync(out, X, (size_t)a.B * a.px() * a.C * 4, hipMemcpyDeviceToDevice, s));
    return AF_OK;
}

af_status run_decode(af_vae* m, const float* lat, int B, int h, int w, int stop_after, float* out, hipStream_t s) {
    const af_vae_config& c = m->cfg;
    auto buf = [&](int id) { return m->bufs[id]; };
    float* X = m->X;
    float* S = m->S;
    Act a{B, h, w, up_ch(c, 0)};
    V_K(vae_prep(lat, B, c.latent_channels, (long)h * w, c.scaling_factor, (const float*)buf(m->pq_w),
                 (const float*)buf(m->pq_b), CIN_PAD, m->zin, s));
    V_TRY(conv3x3(m, m->zin, B, h, w, CIN_PAD, false, buf(m->ci_w), (const float*)buf(m->ci_b), nullptr, X, a.C, s));
    if (stop_after == 0) return tap_out(X, a, out, s);
    V_TRY(resnet(m, m->mid0, a, X, S, s));
    V_TRY(attention(m, a, X, s));
    V_TRY(resnet(m, m->mid1, a, X, S, s));
    if (stop_after == 1) return tap_out(X, a, out, s);
    for (int l = 0; l < 4; ++l) {
        for (const VRes& r : m->res[l]) V_TRY(resnet(m, r, a, X, S, s));
        if (l < 3) {
            const long M = (long)a.B * a.px();
            V_K(f32_to_bf16(X, m->A, M * a.C, s));
            V_TRY(conv3x3(m, m->A, a.B, a.H, a.W, a.C, true, buf(m->ups_w[l]), (const float*)buf(m->ups_b[l]), nullptr,
                          S, a.C, s));
            std::swap(X, S);
            a.H *= 2;
            a.W *= 2;
        }
        if (stop_after == 2 + l) return tap_out(X, a, out, s);
    }
    V_TRY(gn(m, X, a, m->no_g, m->no_n, true, m->A, s));
    V_K(conv_out3x3(m->A, a.B, a.H, a.W, a.C, (const bf16_t*)buf(m->co_w), (const float*)buf(m->co_b), c.out_channels,
                    out, s));
    return AF_OK;
}

af_status check_decode(af_vae* m, const float* lat, int B, int h, int w, const void* out) {
    if (!m) V_FAIL(AF_E_INVALID_ARG, "decoder is NULL");
    if (B < 0) V_FAIL(AF_E_INVALID_ARG, "negative batch");
    if (B > m->cfg.max_batch) V_FAIL(AF_E_SHAPE, "batch exceeds max_batch");
    if (B > 0 && (h < 1 || w < 1)) V_FAIL(AF_E_SHAPE, "latent height and width must be >= 1");
    if (h > m->cfg.max_latent_h || w > m->cfg.max_latent_w) V_FAIL(AF_E_SHAPE, "latent exceeds max_latent_h x max_latent_w");
    if (B > 0 && (!lat || !out)) V_FAIL(AF_E_INVALID_ARG, "latents or output pointer is NULL");
    if (!complete(m)) V_FAIL(AF_E_STATE, "weights are not complete");
    return AF_OK;
}

}  // namespace

extern "C" {

af_status af_vae_config_default(af_vae_config* c) {
    if (!c) V_FAIL(AF_E_INVALID_ARG, "config is NULL");
    c->latent_channels = 4;
    c->out_channels = 3;
    c->block_out_channels[0] = 128;
    c->block_out_channels[1] = 256;
    c->block_out_channels[2] = 512;
    c->block_out_channels[3] = 512;
    c->layers_per_block = 2;
    c->norm_groups = 32;
    c->norm_eps = 1e-6f;
    c->scaling_factor = 0.13025f;
    c->max_batch = 4;
    c->max_latent_h = 128;
    c->max_latent_w = 128;
    return AF_OK;
}

af_status af_vae_weight_count(const af_vae_config* c, int* n_tensors, size_t* total_floats) {
    V_TRY(check_config(c));
    if (!n_tensors) V_FAIL(AF_E_INVALID_ARG, "n_tensors is NULL");
    af_vae tmp;
    tmp.cfg = *c;
    build_slots(&tmp);
    *n_tensors = (int)tmp.slots.size();
    if (total_floats) *total_floats = tmp.total_floats;
    return AF_OK;
}

af_status af_vae_weight_info(const af_vae_config* c, int index, char* name, int name_cap, int64_t* rows,
                             int64_t* cols, size_t* offset) {
    V_TRY(check_config(c));
    af_vae tmp;
    tmp.cfg = *c;
    build_slots(&tmp);
    if (index < 0 || index >= (int)tmp.slots.size()) V_FAIL(AF_E_INVALID_ARG, "tensor index out of range");
    const VSlot& S = tmp.slots[index];
    if (name && name_cap > 0) {
        std::strncpy(name, S.name.c_str(), (size_t)name_cap - 1);
        name[name_cap - 1] = 0;
    }
    if (rows) *rows = S.rows;
    if (cols) *cols = S.cols;
    if (offset) *offset = S.offset;
    return AF_OK;
}

af_status af_vae_create(const af_vae_config* c, int device, af_vae** out) {
    if (!out) V_FAIL(AF_E_INVALID_ARG, "out is NULL");
    *out = nullptr;
    V_TRY(check_config(c));
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) V_FAIL(AF_E_INVALID_ARG, "no such device");
    DevGuard guard(device);
    af_vae* m = new af_vae();
    m->cfg = *c;
    m->device = device;
    build_slots(m);
    auto cleanup = [&](af_status st, const char* msg) {
        af_vae_destroy(m);
        return af::report(st, msg);
    };
    size_t total = 0;
    std::vector<size_t> boff(m->buf_bytes.size());
    for (size_t i = 0; i < m->buf_bytes.size(); ++i) {
        boff[i] = total;
        total += align256(m->buf_bytes[i]);
    }
    if (hipMalloc(&m->arena, total) != hipSuccess) return cleanup(AF_E_OOM, "weight arena allocation failed");
    // padding channels of conv_in's packed kernel stay zero
    if (hipMemset(m->arena, 0, total) != hipSuccess) return cleanup(AF_E_HIP, "weight arena clear failed");
    for (size_t i = 0; i < boff.size(); ++i) m->bufs.push_back((char*)m->arena + boff[i]);

    const long Bm = std::max(c->max_batch, 1);
    const long hw = (long)std::max(c->max_latent_h, 1) * std::max(c->max_latent_w, 1);
    const long hwp = (hw + 127) / 128 * 128;
    const long C0 = up_ch(*c, 0);
    m->act_floats = (size_t)(Bm * max_act(*c, hw));
    m->staging_floats = 16u << 20;
    const long cmax = 1024;
    std::vector<std::pair<void**, size_t>> ws = {
        {(void**)&m->X, m->act_floats * 4},
        {(void**)&m->Hb, m->act_floats * 4},
        {(void**)&m->S, m->act_floats * 4},
        {(void**)&m->A, (m->act_floats + (size_t)A_PAD_ROWS * cmax) * 2},
        {(void**)&m->zin, (size_t)Bm * hw * CIN_PAD * 2},
        {(void**)&m->gpart, gn_part_floats((int)Bm, 64 * hw, c->norm_groups) * 4},
        {(void**)&m->gstats, (size_t)Bm * c->norm_groups * 8},
        {(void**)&m->qkv, (size_t)(Bm * hw + A_PAD_ROWS) * 3 * C0 * 2},
        {(void**)&m->att_o, (size_t)(Bm * hw + A_PAD_ROWS) * C0 * 2},
        {(void**)&m->vt, (size_t)C0 * hwp * 2},
        {(void**)&m->logits, (size_t)hw * hwp * 4},
        {(void**)&m->probs, (size_t)(hw + A_PAD_ROWS) * hwp * 2},
        {(void**)&m->staging, m->staging_floats * 4},
    };
    if (hipDeviceGetAttribute(&m->n_cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || m->n_cu <= 0)
        return cleanup(AF_E_HIP, "compute-unit count query failed");
    size_t wtotal = 0;
    for (auto& e : ws) wtotal += align256(e.second);
    if (hipMalloc(&m->work, wtotal) != hipSuccess) return cleanup(AF_E_OOM, "workspace allocation failed");
    // zero once: the padding rows that GEMM tail tiles read hold finite values
    if (hipMemset(m->work, 0, wtotal) != hipSuccess) return cleanup(AF_E_HIP, "workspace clear failed");
    size_t o = 0;
    for (auto& e : ws) {
        *e.first = (char*)m->work + o;
        o += align256(e.second);
    }
    if (hipDeviceSynchronize() != hipSuccess) return cleanup(AF_E_HIP, "device synchronize failed");
    *out = m;
    return AF_OK;
}

af_status af_vae_load_weights(af_vae* m, const float* host, size_t offset, size_t n, void* stream) {
    if (!m) V_FAIL(AF_E_INVALID_ARG, "decoder is NULL");
    if (n == 0) return AF_OK;
    if (!host) V_FAIL(AF_E_INVALID_ARG, "host pointer is NULL");
    if (offset > m->total_floats || n > m->total_floats - offset)
        V_FAIL(AF_E_SHAPE, "slice extends past the end of the weight blob");
    DevGuard guard(m->device);
    hipStream_t s = (hipStream_t)stream;
    const size_t end = offset + n;
    for (const VSlot& S : m->slots) {
        const size_t ts = S.offset, te = S.offset + (size_t)S.rows * S.cols;
        const size_t a = std::max(ts, offset), b = std::min(te, end);
        if (a >= b) continue;
        const size_t esz = S.mode == VAE_PACK_F32R ? 4 : 2;
        void* dst = (char*)m->bufs[S.buf] + S.dst_elem * esz;
        for (size_t c0 = a; c0 < b; c0 += m->staging_floats) {
            const size_t cn = std::min(m->staging_floats, b - c0);
            V_HIP(hipMemcpyAsync(m->staging, host + (c0 - offset), cn * 4, hipMemcpyHostToDevice, s));
            V_K(vae_pack(m->staging, (long)cn, (long)(c0 - ts), dst, S.mode, S.cin, S.cpad, s));
        }
    }
    mark_loaded(m, offset, end);
    V_HIP(hipStreamSynchronize(s));
    return AF_OK;
}

af_status af_vae_decode(af_vae* m, const float* latents, int B, int h, int w, float* image, void* stream) {
    V_TRY(check_decode(m, latents, B, h, w, image));
    if (B == 0) return AF_OK;
    DevGuard guard(m->device);
    return run_decode(m, latents, B, h, w, 1 << 30, image, (hipStream_t)stream);
}

af_status af_vae_decode_taps(af_vae* m, const float* latents, int B, int h, int w, int stop_after, float* out,
                             void* stream) {
    V_TRY(check_decode(m, latents, B, h, w, out));
    if (stop_after < 0 || stop_after > 5) V_FAIL(AF_E_INVALID_ARG, "stop_after out of range (0 .. 5)");
    if (B == 0) return AF_OK;
    DevGuard guard(m->device);
    return run_decode(m, latents, B, h, w, stop_after, out, (hipStream_t)stream);
}

void af_vae_destroy(af_vae* m) {
    if (!m) return;
    {
        DevGuard guard(m->device);
        if (m->arena) (void)hipFree(m->arena);
        if (m->work) (void)hipFree(m->work);
    }
    delete m;
}

}  // extern "C"

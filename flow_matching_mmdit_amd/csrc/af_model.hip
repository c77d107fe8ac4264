// Executor behind include/auraflow.h: configuration checks, the weight arena and
// its packing, the workspace, and the launch sequence of one forward.
//
// Page tags: [PIPE], [TRANS], [DEEP] as listed in include/auraflow.h.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "af_internal.h"

using namespace af;

namespace {

thread_local std::string g_last_error;

af_status fail(af_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

}  // namespace

// Shared with the other executors (the text encoder): records the message read
// back by af_last_error on this thread.
af_status af::report(af_status s, const char* msg) {
    g_last_error = msg;
    return s;
}

namespace {

#define AF_HIP(call)                                                                        \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess)                                                               \
            return fail(AF_E_HIP, std::string(#call) + ": " + hipGetErrorString(e_));        \
    } while (0)

int isqrt_exact(int n) {
    if (n <= 0) return -1;
    int g = (int)std::lround(std::sqrt((double)n));
    for (int c = g - 1; c <= g + 1; ++c)
        if (c > 0 && c * c == n) return c;
    return -1;
}

// FFN width: 2/3 of the 4x hidden width, rounded up to a multiple of 256
// ([TRANS] 核心子模块架构, FeedForward; [PIPE] 深入源码: find_multiple, rounded up).
long ffn_width(long d) {
    long n = (8 * d) / 3;
    return n % 256 == 0 ? n : n + 256 - n % 256;
}

struct Derived {
    int d, F, G, H, hd, R, Lj, Ls, L;
    long mod_cols;  // adaLN rows of all blocks plus the final modulation
};

af_status derive(const af_config* c, Derived* out) {
    if (!c) return fail(AF_E_INVALID_ARG, "config is NULL");
    if (c->in_channels <= 0 || c->out_channels <= 0 || c->patch_size <= 0 || c->num_mmdit_layers < 0 ||
        c->num_single_dit_layers < 0 || c->num_attention_heads <= 0 || c->attention_head_dim <= 0 ||
        c->joint_attention_dim <= 0 || c->caption_projection_dim <= 0 || c->pos_embed_max_size <= 0 ||
        c->num_register_tokens < 0 || c->max_batch < 0 || c->max_latent_h < 0 || c->max_latent_w < 0 ||
        c->max_text_len < 0)
        return fail(AF_E_INVALID_ARG, "config has a negative or zero size");
    if (c->compute_dtype != AF_F32 && c->compute_dtype != AF_BF16 && c->compute_dtype != AF_MXFP8)
        return fail(AF_E_INVALID_ARG, "compute_dtype must be AF_F32, AF_BF16 or AF_MXFP8");
    if (!(c->ln_eps > 0.f) || !std::isfinite(c->timestep_scale))
        return fail(AF_E_INVALID_ARG, "ln_eps must be > 0 and timestep_scale finite");
    Derived d{};
    d.H = c->num_attention_heads;
    d.hd = c->attention_head_dim;
    d.d = d.H * d.hd;
    if (c->caption_projection_dim != d.d)
        return fail(AF_E_SHAPE, "caption_projection_dim must equal num_attention_heads * attention_head_dim");
    d.G = isqrt_exact(c->pos_embed_max_size);
    if (d.G < 0) return fail(AF_E_SHAPE, "pos_embed_max_size must be a perfect square");
    d.F = (int)ffn_width(d.d);
    d.R = c->num_register_tokens;
    d.Lj = c->num_mmdit_layers;
    d.Ls = c->num_single_dit_layers;
    d.L = d.Lj + d.Ls;
    d.mod_cols = (long)(2 * d.Lj + d.Ls) * 6 * d.d + 2L * d.d;
    if (c->in_channels * c->patch_size * c->patch_size > 64 || c->out_channels * c->patch_size * c->patch_size > 64)
        return fail(AF_E_UNSUPPORTED, "patch vectors longer than 64 are not built");
    if (d.d % 4 != 0 || d.d > 4096) return fail(AF_E_UNSUPPORTED, "inner dim must be a multiple of 4 and <= 4096");
    if (c->compute_dtype != AF_F32) {
        if (d.hd != 256) return fail(AF_E_UNSUPPORTED, "bf16 path is built for attention_head_dim 256");
        if (d.d % 256 != 0) return fail(AF_E_UNSUPPORTED, "bf16 path needs inner dim % 256 == 0");
        if (c->out_channels * c->patch_size * c->patch_size > 16)
            return fail(AF_E_UNSUPPORTED, "bf16 path: output patch vectors longer than 16 are not built");
        if (c->joint_attention_dim % 64 != 0)
            return fail(AF_E_UNSUPPORTED, "bf16 path needs joint_attention_dim % 64 == 0");
    } else {
        if (d.hd > 64) return fail(AF_E_UNSUPPORTED, "fp32 path is built for attention_head_dim <= 64");
        if (c->joint_attention_dim % 4 != 0) return fail(AF_E_UNSUPPORTED, "fp32 path needs joint_attention_dim % 4 == 0");
    }
    *out = d;
    return AF_OK;
}

af_status check_call(const af_config* c, const Derived& D, int B, int H, int W, int T) {
    if (B < 0 || H < 0 || W < 0 || T < 0) return fail(AF_E_INVALID_ARG, "negative size");
    if (H % c->patch_size || W % c->patch_size)
        return fail(AF_E_SHAPE, "latent height and width must be multiples of patch_size");
    int h = H / c->patch_size, w = W / c->patch_size;
    if (h > D.G || w > D.G) return fail(AF_E_SHAPE, "patch grid is larger than the position-embedding grid");
    if (B > c->max_batch) return fail(AF_E_SHAPE, "batch exceeds max_batch");
    if (H > c->max_latent_h || W > c->max_latent_w) return fail(AF_E_SHAPE, "latent exceeds max_latent_h/w");
    if (T > c->max_text_len) return fail(AF_E_SHAPE, "text length exceeds max_text_len");
    if (B > 0 && h * w == 0) return fail(AF_E_SHAPE, "latent has no patches");
    return AF_OK;
}

enum Dest { D_PLAIN = 0, D_GATE = 1, D_UP = 2 };

struct Slot {
    std::string name;
    int64_t rows, cols;
    size_t offset;     // in the canonical blob (floats)
    size_t dst_elem;   // element offset inside the destination buffer
    int buf;           // destination buffer id
    int layout;        // PackLayout
    bool keep_f32;     // position table stays fp32
};

struct BlockW {
    void* wqkv;   // [3d, d]
    void* wo;     // [d, d]
    void* ff12;   // [2F, d] gate/up interleaved in 32-row groups
    void* ff3;    // [d, F]
    // MXFP8 models: E4M3 copies of wqkv, wo, ff12, ff3 and their block scales [K/64][N][2]
    uint8_t *wqkv8 = nullptr, *wqkv_s = nullptr, *wo8 = nullptr, *wo_s = nullptr, *ff12_8 = nullptr,
            *ff12_s = nullptr, *ff3_8 = nullptr, *ff3_s = nullptr;
};

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

}  // namespace

struct af_model {
    af_config cfg;
    Derived D;
    int device;
    af_dtype dt;     // storage type of weights and activations: AF_BF16 or AF_F32
    size_t es;       // bytes per compute element (2 bf16, 4 fp32)
    bool mx = false; // AF_MXFP8: QKV, out-projection and FFN products on MXFP8 operands
    bool mx_ready = false;    // the MXFP8 weight copies match the loaded weights
    void* arena8 = nullptr;   // MXFP8 weight copies

    // weights
    std::vector<Slot> slots;
    std::vector<void*> bufs;              // destination buffers (pointers into the arena)
    void* arena = nullptr;
    size_t total_floats = 0;
    std::map<size_t, size_t> loaded;      // merged loaded intervals [a, b)
    void *t_w1, *t_b1, *t_w2, *t_b2, *pe_w, *pe_b, *ctx_w, *reg, *ada, *proj_out;
    float* pos;
    std::vector<BlockW> joint_img, joint_txt, single;

    // workspace
    int M_max = 0, S_pad_max = 0;
    float* resid = nullptr;
    void *nrm = nullptr, *attn = nullptr, *ffh = nullptr, *q = nullptr, *k = nullptr, *v = nullptr;
    float* raw = nullptr;  // fp32 path only
    float *mod = nullptr, *temb = nullptr, *hpre = nullptr, *tfeat = nullptr, *kbias = nullptr;
    bf16_t* text_bf16 = nullptr;
    float* attn_part = nullptr;  // partial sums of split attention query tiles (bf16 path)
    // MXFP8 activations: LN + modulate output [Mp, d], attention output [Mp, d],
    // SwiGLU output [Mp, F] (E4M3) and their block scales [K/64][Mp][2]
    uint8_t *nrm8 = nullptr, *nrm_s = nullptr, *attn8 = nullptr, *attn_s = nullptr, *ffh8 = nullptr,
            *ffh_s = nullptr;
    long Mp = 0;                 // rows of the activation buffers (M_max + one tile of padding)
    int n_cu = 0;                // compute units of the device
    float* staging = nullptr;
    size_t staging_floats = 0;
    void* work = nullptr;

    // per-kernel-class event timing (af_profile)
    bool prof_on = false;
    struct Rec { hipEvent_t a, b; int cls; };
    std::vector<Rec> prof_pool;      // events, reused across reads
    size_t prof_used = 0;
    double prof_ms[AF_K_COUNT] = {};
    int64_t prof_n[AF_K_COUNT] = {};
};

namespace {

// Canonical list ([TRANS] module inventory) with each tensor's destination.
enum BufId {
    B_TW1, B_TB1, B_TW2, B_TB2, B_PEW, B_PEB, B_POS, B_CTX, B_REG, B_ADA, B_PROJ, B_FIXED_COUNT
};

void build_slots(af_model* m) {
    const Derived& D = m->D;
    const af_config& c = m->cfg;
    const long d = D.d, F = D.F;
    std::vector<size_t> bytes;   // per buffer
    auto newbuf = [&](size_t elems, bool f32) {
        bytes.push_back(elems * (f32 ? 4 : m->es));
        return (int)bytes.size() - 1;
    };
    // fixed buffers, in BufId order
    newbuf(d * 256, false); newbuf(d, false); newbuf(d * d, false); newbuf(d, false);
    newbuf(d * (long)c.in_channels * c.patch_size * c.patch_size, false); newbuf(d, false);
    newbuf((size_t)c.pos_embed_max_size * d, true);
    newbuf(d * (long)c.joint_attention_dim, false);
    newbuf((size_t)D.R * d, false);
    newbuf((size_t)D.mod_cols * d, false);
    newbuf((size_t)c.out_channels * c.patch_size * c.patch_size * d, false);

    size_t off = 0;
    auto add = [&](const std::string& name, int64_t rows, int64_t cols, int buf, size_t dst_elem, int layout,
                   bool keep) {
        m->slots.push_back(Slot{name, rows, cols, off, dst_elem, buf, layout, keep});
        off += (size_t)rows * cols;
    };
    add("t_w1", d, 256, B_TW1, 0, PACK_PLAIN, false);
    add("t_b1", d, 1, B_TB1, 0, PACK_PLAIN, false);
    add("t_w2", d, d, B_TW2, 0, PACK_PLAIN, false);
    add("t_b2", d, 1, B_TB2, 0, PACK_PLAIN, false);
    add("pe_w", d, (int64_t)c.in_channels * c.patch_size * c.patch_size, B_PEW, 0, PACK_PLAIN, false);
    add("pe_b", d, 1, B_PEB, 0, PACK_PLAIN, false);
    add("pos_embed", c.pos_embed_max_size, d, B_POS, 0, PACK_PLAIN, true);
    add("ctx_w", d, c.joint_attention_dim, B_CTX, 0, PACK_PLAIN, false);
    add("registers", D.R, d, B_REG, 0, PACK_PLAIN, false);

    long ada_row = 0;
    auto block = [&](const std::string& prefix, std::vector<BlockW>& list) {
        int bq = newbuf(3 * d * d, false), bo = newbuf(d * d, false), bf = newbuf(2 * F * d, false),
            b3 = newbuf(d * F, false);
        list.push_back(BlockW{(void*)(intptr_t)bq, (void*)(intptr_t)bo, (void*)(intptr_t)bf, (void*)(intptr_t)b3});
        add(prefix + "ada", 6 * d, d, B_ADA, (size_t)ada_row * d, PACK_PLAIN, false);
        ada_row += 6 * d;
        add(prefix + "wq", d, d, bq, 0, PACK_PLAIN, false);
        add(prefix + "wk", d, d, bq, d * d, PACK_PLAIN, false);
        add(prefix + "wv", d, d, bq, 2 * d * d, PACK_PLAIN, false);
        add(prefix + "wo", d, d, bo, 0, PACK_PLAIN, false);
        add(prefix + "ff1", F, d, bf, 0, PACK_FFN_GATE, false);
        add(prefix + "ff2", F, d, bf, 0, PACK_FFN_UP, false);
        add(prefix + "ff3", d, F, b3, 0, PACK_PLAIN, false);
    };
    for (int j = 0; j < D.Lj; ++j) {
        block("joint" + std::to_string(j) + ".img.", m->joint_img);
        block("joint" + std::to_string(j) + ".txt.", m->joint_txt);
    }
    for (int i = 0; i < D.Ls; ++i) block("single" + std::to_string(i) + ".", m->single);
    add("final_ada", 2 * d, d, B_ADA, (size_t)ada_row * d, PACK_PLAIN, false);
    add("proj_out", (int64_t)c.out_channels * c.patch_size * c.patch_size, d, B_PROJ, 0, PACK_PLAIN, false);
    m->total_floats = off;

    // buffer offsets inside one arena (filled with real pointers in af_create)
    size_t total = 0;
    std::vector<size_t> boff(bytes.size());
    for (size_t i = 0; i < bytes.size(); ++i) {
        boff[i] = total;
        total += align256(bytes[i]);
    }
    m->bufs.assign(bytes.size(), nullptr);
    for (size_t i = 0; i < bytes.size(); ++i) m->bufs[i] = (void*)(intptr_t)boff[i];
    m->bufs.push_back((void*)(intptr_t)total);  // sentinel: arena size
}

// Host-only weight list for an arbitrary config (af_weight_count / af_weight_info).
struct ListOnly {
    std::vector<Slot> slots;
    size_t total = 0;
};

af_status weight_list(const af_config* c, ListOnly* out) {
    Derived D;
    af_status st = derive(c, &D);
    if (st != AF_OK) return st;
    af_model tmp;
    tmp.cfg = *c;
    tmp.D = D;
    tmp.dt = c->compute_dtype == AF_F32 ? AF_F32 : AF_BF16;
    tmp.es = tmp.dt == AF_BF16 ? 2 : 4;
    build_slots(&tmp);
    out->slots = tmp.slots;
    out->total = tmp.total_floats;
    return AF_OK;
}

bool weights_complete(const af_model* m) {
    size_t cur = 0;
    for (auto& iv : m->loaded) {
        if (iv.first > cur) return false;
        if (iv.second > cur) cur = iv.second;
    }
    return cur >= m->total_floats;
}

void mark_loaded(af_model* m, size_t a, size_t b) {
    auto& L = m->loaded;
    auto it = L.upper_bound(a);
    if (it != L.begin()) {
        auto p = std::prev(it);
        if (p->second >= a) {
            a = p->first;
            b = std::max(b, p->second);
            it = L.erase(p);
        }
    }
    while (it != L.end() && it->first <= b) {
        b = std::max(b, it->second);
        it = L.erase(it);
    }
    L[a] = b;
}

// ---------------------------------------------------------------------------- profiling
// Brackets one launch with two events when profiling is on.
struct ProfScope {
    af_model* m;
    hipStream_t s;
    int idx = -1;
    ProfScope(af_model* m_, int cls, hipStream_t s_) : m(m_), s(s_) {
        if (!m->prof_on) return;
        if (m->prof_used == m->prof_pool.size()) {
            af_model::Rec r{};
            if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) return;
            m->prof_pool.push_back(r);
        }
        idx = (int)m->prof_used++;
        m->prof_pool[idx].cls = cls;
        (void)hipEventRecord(m->prof_pool[idx].a, s);
    }
    void end() {
        if (idx >= 0) (void)hipEventRecord(m->prof_pool[idx].b, s);
        idx = -1;
    }
    ~ProfScope() { end(); }
};

af_status prof_collect(af_model* m) {
    for (size_t i = 0; i < m->prof_used; ++i) {
        auto& r = m->prof_pool[i];
        AF_HIP(hipEventSynchronize(r.b));
        float ms = 0.f;
        AF_HIP(hipEventElapsedTime(&ms, r.a, r.b));
        m->prof_ms[r.cls] += ms;
        m->prof_n[r.cls] += 1;
    }
    m->prof_used = 0;
    return AF_OK;
}

// ---------------------------------------------------------------------------- forward
struct Inputs {
    const float* latents;
    const float* tau;
    const void* text;
    af_dtype text_dtype;
    const uint8_t* mask;
    int B, H, W, T;
};

af_status gemm(af_model* m, GemmLaunch& L, hipStream_t s) {
    hipError_t e = m->dt == AF_BF16 ? gemm_bf16(L, s) : gemm_f32(L, s);
    if (e != hipSuccess) return fail(AF_E_HIP, std::string("gemm launch: ") + hipGetErrorString(e));
    return AF_OK;
}

#define AF_K(call)                                                                                  \
    do {                                                                                            \
        hipError_t e_ = (call);                                                                     \
        if (e_ != hipSuccess) return fail(AF_E_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
    } while (0)
#define AF_TRY(call)                    \
    do {                                \
        af_status s_ = (call);          \
        if (s_ != AF_OK) return s_;     \
    } while (0)

GemmLaunch gemm_base(af_model* m, const float* mod, RowGeom g, int N, int K, int epi) {
    GemmLaunch L;
    memset(&L, 0, sizeof(L));
    L.N = N;
    L.K = K;
    L.epi = epi;
    L.geom = g;
    L.mod = mod;
    L.mod_stride = m->D.mod_cols;
    L.H = m->D.H;
    L.hd = m->D.hd;
    L.eps = m->cfg.ln_eps;
    L.q_scale = 1.f;
    L.n_cu = m->n_cu;   // lets small launches use 128 x 128 tiles
    return L;
}

// The activation buffers of one group of samples [b0, b0 + B): each group keeps
// the whole-batch row layout ([text rows of its samples][image rows of its
// samples]) in its own row range, and its own slices of the per-sample buffers.
struct View {
    float* resid;
    void *nrm, *attn, *ffh, *q, *k, *v;
    float *raw, *kbias, *mod;
    uint8_t *nrm8, *nrm_s, *attn8, *attn_s, *ffh8, *ffh_s;   // MXFP8 models
};

View group_view(af_model* m, int b0, int S, int S_pad) {
    const Derived& D = m->D;
    const size_t es = m->es;
    const long r0 = (long)b0 * S;                                    // first row of the group
    const size_t qkv = (size_t)b0 * D.H * S_pad * D.hd * es;         // bytes before the group's q/k/v
    View V;
    V.resid = m->resid + r0 * D.d;
    V.nrm = (char*)m->nrm + r0 * D.d * es;
    V.attn = (char*)m->attn + r0 * D.d * es;
    V.ffh = (char*)m->ffh + r0 * D.F * es;
    V.q = (char*)m->q + qkv;
    V.k = (char*)m->k + qkv;
    V.v = (char*)m->v + qkv;
    V.raw = m->raw ? m->raw + r0 * std::max(3 * D.d, 2 * D.F) : nullptr;
    V.kbias = m->kbias + (size_t)b0 * S_pad;
    V.mod = m->mod + (size_t)b0 * D.mod_cols;
    V.nrm8 = m->mx ? m->nrm8 + r0 * D.d : nullptr;
    V.nrm_s = m->mx ? m->nrm_s + r0 * 2 : nullptr;
    V.attn8 = m->mx ? m->attn8 + r0 * D.d : nullptr;
    V.attn_s = m->mx ? m->attn_s + r0 * 2 : nullptr;
    V.ffh8 = m->mx ? m->ffh8 + r0 * D.F : nullptr;
    V.ffh_s = m->mx ? m->ffh_s + r0 * 2 : nullptr;
    return V;
}

// One transformer block. Streams: 2 for a joint block (text rows then image
// rows, each with its own weights and modulation), 1 for a single block.
af_status run_block(af_model* m, const View& V, RowGeom g, int S_pad, const BlockW* wt, const BlockW* wi, long off_t,
                    long off_i, hipStream_t s) {
    const Derived& D = m->D;
    const long d = D.d, F = D.F;
    const int M = g.B * g.S();
    const int Mt = g.B * g.Nt;
    const bool joint = wi != nullptr;
    const size_t es = m->es;
    auto grp = [&](GemmLaunch& L, const void* A, long lda, const BlockW* w, int which, int Mrows, int row0,
                   int gate_off) {
        GemmGroup& G = L.g[L.ngroups++];
        G.A = A;
        G.lda = lda;
        G.W = which == 0 ? w->wqkv : which == 1 ? w->wo : which == 2 ? w->ff12 : w->ff3;
        G.ldw = which == 3 ? F : d;
        G.M = Mrows;
        G.row0 = row0;
        G.gate_off = gate_off;
    };
    auto add_groups = [&](GemmLaunch& L, const char* Abase, long lda, size_t row_bytes, int which, long gate_rel) {
        if (joint) {
            grp(L, Abase, lda, wt, which, Mt, 0, (int)(off_t + gate_rel));
            grp(L, Abase + (size_t)Mt * row_bytes, lda, wi, which, M - Mt, Mt, (int)(off_i + gate_rel));
        } else {
            grp(L, Abase, lda, wt, which, M, 0, (int)(off_t + gate_rel));
        }
    };
    const int split = joint ? Mt : M;
    const long off_a = off_t, off_b = joint ? off_i : off_t;

    // MXFP8 operand groups: rows [0, Mt) and [Mt, M) of an fp8 activation buffer
    // (row stride K bytes, scales row-offset by 2 bytes per row) with one weight set each
    auto mx_groups = [&](GemmLaunch& L, const uint8_t* A8, const uint8_t* As, long K, int which) {
        auto one = [&](const BlockW* w, int Mrows, int r0, long gate_rel, long off) {
            GemmGroup& G = L.g[L.ngroups++];
            G.A = A8 + (size_t)r0 * K;
            G.As = As + (size_t)r0 * 2;
            G.lda = K;
            G.W = which == 0 ? w->wqkv8 : which == 1 ? w->wo8 : which == 2 ? w->ff12_8 : w->ff3_8;
            G.Ws = which == 0 ? w->wqkv_s : which == 1 ? w->wo_s : which == 2 ? w->ff12_s : w->ff3_s;
            G.ldw = K;
            G.M = Mrows;
            G.row0 = r0;
            G.gate_off = (int)(off + gate_rel);
        };
        const long gate_rel = which == 3 ? 5 * d : which == 1 ? 2 * d : 0;
        if (joint) {
            one(wt, Mt, 0, gate_rel, off_t);
            one(wi, M - Mt, Mt, gate_rel, off_i);
        } else {
            one(wt, M, 0, gate_rel, off_t);
        }
        L.as_rows = m->Mp;
        L.ws_rows = which == 0 ? 3 * d : which == 2 ? 2 * F : d;   // wo and ff3 have d rows
    };
    auto mx_gemm = [&](GemmLaunch& L) {
        hipError_t e = gemm_mxfp8(L, s);
        if (e != hipSuccess) return fail(AF_E_HIP, std::string("MXFP8 gemm launch: ") + hipGetErrorString(e));
        return AF_OK;
    };

    // 1. LN + modulate(shift1, scale1)
    {
    ProfScope ps(m, AF_K_LN_MOD, s);
    if (m->mx)
        AF_K(ln_modulate_mx(V.resid, M, d, g, split, V.mod, D.mod_cols, off_a, off_a + d, off_b, off_b + d, V.nrm8,
                            V.nrm_s, m->Mp, m->cfg.ln_eps, s));
    else
        AF_K(ln_modulate(V.resid, M, d, g, split, V.mod, D.mod_cols, off_a, off_a + d, off_b, off_b + d, V.nrm, m->dt,
                         m->cfg.ln_eps, s));
    }
    // 2. QKV (+ QK-norm)
    if (m->mx) {
        ProfScope ps(m, AF_K_GEMM_QKV, s);
        GemmLaunch L = gemm_base(m, V.mod, g, 3 * d, d, EPI_QKV);
        L.q = V.q; L.k = V.k; L.vt = V.v; L.S_pad = S_pad;
        L.q_scale = ATTN_BF16_Q_SCALE;
        mx_groups(L, V.nrm8, V.nrm_s, d, 0);
        AF_TRY(mx_gemm(L));
    } else {
        ProfScope ps(m, AF_K_GEMM_QKV, s);
        GemmLaunch L = gemm_base(m, V.mod, g, 3 * d, d, m->dt == AF_BF16 ? EPI_QKV : EPI_STORE);
        L.q = V.q; L.k = V.k; L.vt = V.v; L.S_pad = S_pad;
        L.q_scale = ATTN_BF16_Q_SCALE;
        L.C = V.raw; L.ldc = 3 * d;
        add_groups(L, (const char*)V.nrm, d, d * es, 0, 0);
        AF_TRY(gemm(m, L, s));
        if (m->dt == AF_F32)
            AF_K(qknorm_scatter_f32(V.raw, M, g, D.H, D.hd, S_pad, m->cfg.ln_eps, (float*)V.q, (float*)V.k,
                                    (float*)V.v, 0, s));
    }
    // 3. attention over [registers; text; image]
    {
    ProfScope ps(m, AF_K_ATTENTION, s);
    if (m->dt == AF_BF16)
        AF_K(attention_bf16((const bf16_t*)V.q, (const bf16_t*)V.k, (const bf16_t*)V.v, V.kbias, g, D.H, S_pad,
                            (bf16_t*)V.attn, d, m->n_cu, m->attn_part, m->n_cu, V.attn8, V.attn_s, m->Mp, s));
    else
        AF_K(attention_f32((const float*)V.q, (const float*)V.k, (const float*)V.v, V.kbias, g, D.H, D.hd, S_pad,
                           (float*)V.attn, d, s));
    }
    // 4. out projection, residual += gate1 * (.)
    if (m->mx) {
        ProfScope ps(m, AF_K_GEMM_OUT, s);
        GemmLaunch L = gemm_base(m, V.mod, g, d, d, EPI_GATED_RESID);
        L.resid = V.resid;
        mx_groups(L, V.attn8, V.attn_s, d, 1);
        AF_TRY(mx_gemm(L));
    } else {
        ProfScope ps(m, AF_K_GEMM_OUT, s);
        GemmLaunch L = gemm_base(m, V.mod, g, d, d, EPI_GATED_RESID);
        L.resid = V.resid;
        add_groups(L, (const char*)V.attn, d, d * es, 1, 2 * d);
        AF_TRY(gemm(m, L, s));
    }
    // 5. LN + modulate(shift2, scale2)
    {
    ProfScope ps(m, AF_K_LN_MOD, s);
    if (m->mx)
        AF_K(ln_modulate_mx(V.resid, M, d, g, split, V.mod, D.mod_cols, off_a + 3 * d, off_a + 4 * d, off_b + 3 * d,
                            off_b + 4 * d, V.nrm8, V.nrm_s, m->Mp, m->cfg.ln_eps, s));
    else
        AF_K(ln_modulate(V.resid, M, d, g, split, V.mod, D.mod_cols, off_a + 3 * d, off_a + 4 * d, off_b + 3 * d,
                         off_b + 4 * d, V.nrm, m->dt, m->cfg.ln_eps, s));
    }
    if (m->mx) {
        // 6. FFN up: silu(gate) * up -> MXFP8
        {
            ProfScope ps(m, AF_K_GEMM_FFN_UP, s);
            GemmLaunch L = gemm_base(m, V.mod, g, 2 * F, d, EPI_SWIGLU);
            L.C = V.ffh8; L.ldc = F; L.Cs = V.ffh_s; L.cs_rows = m->Mp;
            mx_groups(L, V.nrm8, V.nrm_s, d, 2);
            AF_TRY(mx_gemm(L));
        }
        // 7. FFN down, residual += gate2 * (.)
        {
            ProfScope ps(m, AF_K_GEMM_FFN_DOWN, s);
            GemmLaunch L = gemm_base(m, V.mod, g, d, F, EPI_GATED_RESID);
            L.resid = V.resid;
            mx_groups(L, V.ffh8, V.ffh_s, F, 3);
            AF_TRY(mx_gemm(L));
        }
        return AF_OK;
    }
    // 6. FFN up: silu(gate) * up
    {
        ProfScope ps(m, AF_K_GEMM_FFN_UP, s);
        GemmLaunch L = gemm_base(m, V.mod, g, 2 * F, d, m->dt == AF_BF16 ? EPI_SWIGLU : EPI_STORE);
        if (m->dt == AF_BF16) { L.C = V.ffh; L.ldc = F; }
        else { L.C = V.raw; L.ldc = 2 * F; }
        add_groups(L, (const char*)V.nrm, d, d * es, 2, 0);
        AF_TRY(gemm(m, L, s));
        if (m->dt == AF_F32) AF_K(swiglu_f32(V.raw, M, F, (float*)V.ffh, s));
    }
    // 7. FFN down, residual += gate2 * (.)
    {
        ProfScope ps(m, AF_K_GEMM_FFN_DOWN, s);
        GemmLaunch L = gemm_base(m, V.mod, g, d, F, EPI_GATED_RESID);
        L.resid = V.resid;
        add_groups(L, (const char*)V.ffh, F, F * es, 3, 5 * d);
        AF_TRY(gemm(m, L, s));
    }
    return AF_OK;
}

// Samples [b0, b0 + Bg) of a forward whose per-sample prologue (key bias,
// modulation vectors, bf16 text) is already on the device: embeddings, the
// blocks and the final layer (or a residual tap) on stream s.
af_status run_group(af_model* m, const Inputs& in, int b0, int Bg, int stop_after, float* resid_out, float* out,
                    hipStream_t s) {
    const Derived& D = m->D;
    const af_config& c = m->cfg;
    const long d = D.d;
    const int p = c.patch_size;
    const int h = in.H / p, w = in.W / p;
    RowGeom g{Bg, D.R + in.T, h * w};
    const int S = g.S();
    const int S_pad = (S + 127) / 128 * 128;
    const View V = group_view(m, b0, S, S_pad);
    const size_t pix = (size_t)in.H * in.W;

    ProfScope ps_embed(m, AF_K_EMBED, s);
    // embeddings: image rows, register rows, caption rows
    AF_K(patch_embed(in.latents + (size_t)b0 * c.in_channels * pix, c.in_channels, in.H, in.W, p, m->pe_w, m->pe_b,
                     m->dt, m->pos, D.G, V.resid, g, d, s));
    AF_K(copy_registers(m->reg, m->dt, D.R, V.resid, g, d, s));
    if (in.T > 0) {
        // bf16 models read the staged bf16 copy; fp32 models take fp32 text
        const size_t first = (size_t)b0 * in.T * c.joint_attention_dim;
        const void* text = m->dt == AF_BF16 ? (const void*)(m->text_bf16 + first)
                                            : (const void*)((const float*)in.text + first);
        GemmLaunch L = gemm_base(m, V.mod, g, d, c.joint_attention_dim, EPI_STORE_MAPPED);
        L.resid = V.resid;
        L.seg_len = in.T;
        L.seg_stride = g.Nt;
        L.seg_off = D.R;
        L.ngroups = 1;
        L.g[0].A = text;
        L.g[0].lda = c.joint_attention_dim;
        L.g[0].W = m->ctx_w;
        L.g[0].ldw = c.joint_attention_dim;
        L.g[0].M = Bg * in.T;
        AF_TRY(gemm(m, L, s));
    }
    ps_embed.end();
    float* tap = resid_out ? resid_out + (size_t)b0 * S * d : nullptr;
    if (stop_after == -1) {
        AF_K(taps_permute(V.resid, g, d, tap, s));
        return AF_OK;
    }
    int bi = 0;
    for (int j = 0; j < D.Lj; ++j, ++bi) {
        AF_TRY(run_block(m, V, g, S_pad, &m->joint_txt[j], &m->joint_img[j], (long)(2 * j + 1) * 6 * d,
                         (long)(2 * j) * 6 * d, s));
        if (stop_after == bi) {
            AF_K(taps_permute(V.resid, g, d, tap, s));
            return AF_OK;
        }
    }
    for (int i = 0; i < D.Ls; ++i, ++bi) {
        AF_TRY(run_block(m, V, g, S_pad, &m->single[i], nullptr, (long)(2 * D.Lj + i) * 6 * d, 0, s));
        if (stop_after == bi) {
            AF_K(taps_permute(V.resid, g, d, tap, s));
            return AF_OK;
        }
    }
    // pre-final modulation (scale, shift) + projection + unpatchify
    const long foff = (long)(2 * D.Lj + D.Ls) * 6 * d;
    ProfScope ps_final(m, AF_K_FINAL, s);
    AF_K(prefinal_project(V.resid, g, d, V.mod, D.mod_cols, foff, foff + d, m->proj_out, m->dt, c.out_channels, p, h,
                          w, out + (size_t)b0 * c.out_channels * pix, s));
    return AF_OK;
}

af_status run_forward(af_model* m, const Inputs& in, int stop_after, float* resid_out, float* out, hipStream_t s) {
    const Derived& D = m->D;
    const af_config& c = m->cfg;
    const long d = D.d;
    const int p = c.patch_size;
    const int h = in.H / p, w = in.W / p;
    RowGeom g{in.B, D.R + in.T, h * w};
    const int S = g.S();
    const int S_pad = (S + 127) / 128 * 128;
    if (in.B == 0) return AF_OK;

    // ---- per-sample prologue for the whole batch, on the caller's stream
    // key-padding bias
    {
    ProfScope ps(m, AF_K_EMBED, s);
    AF_K(key_bias(in.mask, in.T, D.R, g, S_pad, m->dt == AF_BF16 ? ATTN_BF16_KEY_KEEP : 0.f, m->kbias, s));
    }
    // timestep embedding and every block's modulation vectors (one pass over the
    // modulation weights for all samples)
    {
    ProfScope ps(m, AF_K_ADALN, s);
    AF_K(timestep_features(in.tau, in.B, 128, c.timestep_scale, m->tfeat, s));
    AF_K(gemv(m->tfeat, in.B, 256, m->t_w1, m->dt, d, m->t_b1, 0, m->hpre, s));
    AF_K(gemv(m->hpre, in.B, d, m->t_w2, m->dt, d, m->t_b2, 1, m->temb, s));
    AF_K(gemv(m->temb, in.B, d, m->ada, m->dt, (int)D.mod_cols, nullptr, 1, m->mod, s));
    }
    // bf16 models stage the text in the padded internal buffer (rounded to bf16
    // when it arrives as fp32)
    if (in.T > 0 && m->dt == AF_BF16) {
        ProfScope ps(m, AF_K_EMBED, s);
        const long n = (long)in.B * in.T * c.joint_attention_dim;
        if (in.text_dtype == AF_F32) AF_K(f32_to_bf16((const float*)in.text, m->text_bf16, n, s));
        else AF_K(hipMemcpyAsync(m->text_bf16, in.text, (size_t)n * 2, hipMemcpyDeviceToDevice, s));
    }

    // ---- embeddings, the blocks and the final layer for the whole batch
    return run_group(m, in, 0, in.B, stop_after, resid_out, out, s);
}

af_status check_forward_args(af_model* m, const Inputs& in, const void* outp) {
    if (!m) return fail(AF_E_INVALID_ARG, "model is NULL");
    AF_TRY(check_call(&m->cfg, m->D, in.B, in.H, in.W, in.T));
    if (in.text_dtype != AF_F32 && in.text_dtype != AF_BF16) return fail(AF_E_INVALID_ARG, "bad text_dtype");
    if (m->dt == AF_F32 && in.text_dtype != AF_F32)
        return fail(AF_E_UNSUPPORTED, "fp32 models take fp32 text embeddings");
    if (in.B > 0 && (!in.latents || !in.tau || !outp)) return fail(AF_E_INVALID_ARG, "NULL device pointer");
    if (in.B > 0 && in.T > 0 && !in.text) return fail(AF_E_INVALID_ARG, "text_embeds is NULL");
    if (!weights_complete(m)) return fail(AF_E_STATE, "weights not fully loaded");
    if (m->mx && !m->mx_ready) return fail(AF_E_STATE, "MXFP8 weights not quantized");
    return AF_OK;
}

}  // namespace

// ============================================================================ C ABI
extern "C" {

af_status af_config_default(af_config* c) {
    if (!c) return fail(AF_E_INVALID_ARG, "config is NULL");
    c->in_channels = 4;
    c->out_channels = 4;
    c->patch_size = 2;
    c->num_mmdit_layers = 4;
    c->num_single_dit_layers = 32;
    c->num_attention_heads = 12;
    c->attention_head_dim = 256;
    c->joint_attention_dim = 2048;
    c->caption_projection_dim = 3072;
    c->pos_embed_max_size = 9216;
    c->num_register_tokens = 8;
    c->compute_dtype = AF_BF16;
    c->ln_eps = 1e-6f;
    c->timestep_scale = 1000.f;
    c->max_batch = 2;
    c->max_latent_h = 128;
    c->max_latent_w = 128;
    c->max_text_len = 256;
    return AF_OK;
}

af_status af_check_shapes(const af_config* c, int B, int H, int W, int T) {
    Derived D;
    af_status st = derive(c, &D);
    if (st != AF_OK) return st;
    return check_call(c, D, B, H, W, T);
}

af_status af_weight_count(const af_config* c, int* n_tensors, size_t* total_floats) {
    if (!n_tensors) return fail(AF_E_INVALID_ARG, "n_tensors is NULL");
    ListOnly L;
    af_status st = weight_list(c, &L);
    if (st != AF_OK) return st;
    *n_tensors = (int)L.slots.size();
    if (total_floats) *total_floats = L.total;
    return AF_OK;
}

af_status af_weight_info(const af_config* c, int index, char* name, int name_cap, int64_t* rows, int64_t* cols,
                         size_t* offset) {
    ListOnly L;
    af_status st = weight_list(c, &L);
    if (st != AF_OK) return st;
    if (index < 0 || index >= (int)L.slots.size()) return fail(AF_E_INVALID_ARG, "weight index out of range");
    const Slot& S = L.slots[index];
    if (name && name_cap > 0) {
        snprintf(name, (size_t)name_cap, "%s", S.name.c_str());
    }
    if (rows) *rows = S.rows;
    if (cols) *cols = S.cols;
    if (offset) *offset = S.offset;
    return AF_OK;
}

af_status af_create(const af_config* c, int device, af_model** out) {
    if (!out) return fail(AF_E_INVALID_ARG, "out is NULL");
    *out = nullptr;
    Derived D;
    af_status st = derive(c, &D);
    if (st != AF_OK) return st;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev)
        return fail(AF_E_INVALID_ARG, "no such HIP device");
    DevGuard guard(device);
    af_model* m = new af_model();
    m->cfg = *c;
    m->D = D;
    m->device = device;
    m->dt = c->compute_dtype == AF_F32 ? AF_F32 : AF_BF16;
    m->mx = c->compute_dtype == AF_MXFP8;
    m->es = m->dt == AF_BF16 ? 2 : 4;
    build_slots(m);

    auto cleanup = [&](af_status s, const std::string& msg) {
        af_destroy(m);
        return fail(s, msg);
    };
    size_t arena_bytes = (size_t)(intptr_t)m->bufs.back();
    m->bufs.pop_back();
    if (hipMalloc(&m->arena, arena_bytes) != hipSuccess) return cleanup(AF_E_OOM, "weight arena allocation failed");
    for (auto& b : m->bufs) b = (char*)m->arena + (size_t)(intptr_t)b;
    auto bp = [&](int id) { return m->bufs[id]; };
    m->t_w1 = bp(B_TW1); m->t_b1 = bp(B_TB1); m->t_w2 = bp(B_TW2); m->t_b2 = bp(B_TB2);
    m->pe_w = bp(B_PEW); m->pe_b = bp(B_PEB); m->pos = (float*)bp(B_POS); m->ctx_w = bp(B_CTX);
    m->reg = bp(B_REG); m->ada = bp(B_ADA); m->proj_out = bp(B_PROJ);
    for (auto* list : {&m->joint_img, &m->joint_txt, &m->single})
        for (auto& bw : *list) {
            bw.wqkv = bp((int)(intptr_t)bw.wqkv);
            bw.wo = bp((int)(intptr_t)bw.wo);
            bw.ff12 = bp((int)(intptr_t)bw.ff12);
            bw.ff3 = bp((int)(intptr_t)bw.ff3);
        }
    if (m->mx) {
        // E4M3 copies (N x K bytes) and scales (N x K / 32 bytes) of wqkv, wo, ff12, ff3
        const size_t d_ = D.d, F_ = D.F;
        const size_t sizes[4] = {3 * d_ * d_, d_ * d_, 2 * F_ * d_, d_ * F_};
        size_t per = 0;
        for (size_t z : sizes) per += align256(z) + align256(z / 32);
        const size_t nsets = m->joint_img.size() + m->joint_txt.size() + m->single.size();
        if (hipMalloc(&m->arena8, per * nsets) != hipSuccess) return cleanup(AF_E_OOM, "MXFP8 weight allocation failed");
        uint8_t* p8 = (uint8_t*)m->arena8;
        auto take = [&](size_t z) { uint8_t* r = p8; p8 += align256(z); return r; };
        for (auto* list : {&m->joint_img, &m->joint_txt, &m->single})
            for (auto& bw : *list) {
                bw.wqkv8 = take(sizes[0]); bw.wqkv_s = take(sizes[0] / 32);
                bw.wo8 = take(sizes[1]); bw.wo_s = take(sizes[1] / 32);
                bw.ff12_8 = take(sizes[2]); bw.ff12_s = take(sizes[2] / 32);
                bw.ff3_8 = take(sizes[3]); bw.ff3_s = take(sizes[3] / 32);
            }
    }

    // workspace
    const int p = c->patch_size;
    const long hm = c->max_latent_h / p, wm = c->max_latent_w / p;
    const long Smax = D.R + c->max_text_len + hm * wm;
    m->S_pad_max = (int)((Smax + 127) / 128 * 128);
    m->M_max = (int)(c->max_batch * Smax);
    const long Bm = c->max_batch > 0 ? c->max_batch : 1;
    const long Mm = m->M_max > 0 ? m->M_max : 1;
    const long d = D.d, F = D.F;
    // GEMM A operands (nrm, attn, ffh, text) carry one 256-row tile of padding:
    // tail tiles of the bf16 GEMM read past the last row and discard the results.
    const long Mp = Mm + 256;
    const long Tp = Bm * (long)(c->max_text_len > 0 ? c->max_text_len : 1) + 256;
    std::vector<std::pair<void**, size_t>> ws = {
        {(void**)&m->resid, Mm * d * 4},
        {&m->nrm, Mp * d * m->es},
        {&m->attn, Mp * d * m->es},
        {&m->ffh, Mp * F * m->es},
        {&m->q, Bm * D.H * (size_t)m->S_pad_max * D.hd * m->es},
        {&m->k, Bm * D.H * (size_t)m->S_pad_max * D.hd * m->es},
        {&m->v, Bm * D.H * (size_t)m->S_pad_max * D.hd * m->es},
        {(void**)&m->mod, Bm * D.mod_cols * 4},
        {(void**)&m->temb, Bm * d * 4},
        {(void**)&m->hpre, Bm * d * 4},
        {(void**)&m->tfeat, Bm * 256 * 4},
        {(void**)&m->kbias, Bm * (size_t)m->S_pad_max * 4},
        {(void**)&m->text_bf16, (size_t)Tp * c->joint_attention_dim * 2},
    };
    if (m->dt == AF_F32) ws.push_back({(void**)&m->raw, Mm * std::max(3 * d, 2 * F) * 4});
    if (hipDeviceGetAttribute(&m->n_cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || m->n_cu <= 0)
        return cleanup(AF_E_HIP, "compute-unit count query failed");
    if (m->dt == AF_BF16) ws.push_back({(void**)&m->attn_part, attention_bf16_part_floats(m->n_cu) * 4});
    m->Mp = Mp;
    if (m->mx) {
        ws.push_back({(void**)&m->nrm8, (size_t)Mp * d});
        ws.push_back({(void**)&m->nrm_s, (size_t)Mp * d / 32});
        ws.push_back({(void**)&m->attn8, (size_t)Mp * d});
        ws.push_back({(void**)&m->attn_s, (size_t)Mp * d / 32});
        ws.push_back({(void**)&m->ffh8, (size_t)Mp * F});
        ws.push_back({(void**)&m->ffh_s, (size_t)Mp * F / 32});
    }
    m->staging_floats = 16u << 20;
    ws.push_back({(void**)&m->staging, m->staging_floats * 4});
    size_t wtotal = 0;
    for (auto& e : ws) wtotal += align256(e.second);
    if (hipMalloc(&m->work, wtotal) != hipSuccess) return cleanup(AF_E_OOM, "workspace allocation failed");
    // Zero once: padded attention rows/columns must hold finite values.
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

af_status af_load_weights(af_model* m, const float* host, size_t offset, size_t n, void* stream) {
    if (!m) return fail(AF_E_INVALID_ARG, "model is NULL");
    if (n == 0) return AF_OK;
    if (!host) return fail(AF_E_INVALID_ARG, "host pointer is NULL");
    if (offset > m->total_floats || n > m->total_floats - offset)
        return fail(AF_E_SHAPE, "slice extends past the end of the weight blob");
    DevGuard guard(m->device);
    hipStream_t s = (hipStream_t)stream;
    const size_t end = offset + n;
    for (const Slot& S : m->slots) {
        size_t ts = S.offset, te = S.offset + (size_t)S.rows * S.cols;
        size_t a = std::max(ts, offset), b = std::min(te, end);
        if (a >= b) continue;
        void* dst = (char*)m->bufs[S.buf] + S.dst_elem * (S.keep_f32 ? 4 : m->es);
        af_dtype ddt = S.keep_f32 ? AF_F32 : m->dt;
        for (size_t c0 = a; c0 < b; c0 += m->staging_floats) {
            size_t cn = std::min(m->staging_floats, b - c0);
            AF_HIP(hipMemcpyAsync(m->staging, host + (c0 - offset), cn * 4, hipMemcpyHostToDevice, s));
            AF_K(pack_weights(m->staging, (long)cn, (long)(c0 - ts), dst, ddt, S.layout, (int)S.cols, s));
        }
    }
    mark_loaded(m, offset, end);
    if (m->mx) {
        // MXFP8 models: (re)quantize the block GEMM weights once the list is complete
        m->mx_ready = false;
        if (weights_complete(m)) {
            const long d = m->D.d, F = m->D.F;
            for (auto* list : {&m->joint_img, &m->joint_txt, &m->single})
                for (auto& bw : *list) {
                    AF_K(mx_quantize_rows((const bf16_t*)bw.wqkv, 3 * d, (int)d, bw.wqkv8, bw.wqkv_s, s));
                    AF_K(mx_quantize_rows((const bf16_t*)bw.wo, d, (int)d, bw.wo8, bw.wo_s, s));
                    AF_K(mx_quantize_rows((const bf16_t*)bw.ff12, 2 * F, (int)d, bw.ff12_8, bw.ff12_s, s));
                    AF_K(mx_quantize_rows((const bf16_t*)bw.ff3, d, (int)F, bw.ff3_8, bw.ff3_s, s));
                }
            m->mx_ready = true;
        }
    }
    AF_HIP(hipStreamSynchronize(s));
    return AF_OK;
}

af_status af_init_weights(af_model* m, const float* host_blob, size_t n_floats, void* stream) {
    if (!m) return fail(AF_E_INVALID_ARG, "model is NULL");
    if (n_floats != m->total_floats) return fail(AF_E_SHAPE, "blob length does not match the weight list");
    return af_load_weights(m, host_blob, 0, n_floats, stream);
}

af_status af_transformer_forward(af_model* m, const float* latents, const float* timestep, const void* text_embeds,
                                 af_dtype text_dtype, const uint8_t* text_mask, int B, int H, int W, int T,
                                 float* out, void* stream) {
    Inputs in{latents, timestep, text_embeds, text_dtype, text_mask, B, H, W, T};
    AF_TRY(check_forward_args(m, in, out));
    DevGuard guard(m->device);
    return run_forward(m, in, 1 << 30, nullptr, out, (hipStream_t)stream);
}

af_status af_transformer_forward_taps(af_model* m, const float* latents, const float* timestep,
                                      const void* text_embeds, af_dtype text_dtype, const uint8_t* text_mask, int B,
                                      int H, int W, int T, int stop_after_block, float* residual_out, void* stream) {
    Inputs in{latents, timestep, text_embeds, text_dtype, text_mask, B, H, W, T};
    AF_TRY(check_forward_args(m, in, residual_out));
    if (stop_after_block < -1 || stop_after_block >= m->D.L)
        return fail(AF_E_INVALID_ARG, "stop_after_block out of range");
    DevGuard guard(m->device);
    return run_forward(m, in, stop_after_block, residual_out, nullptr, (hipStream_t)stream);
}

af_status af_flow_euler_cfg_step(float* latents, const float* v, int Bi, int C, int H, int W, float sigma,
                                 float sigma_next, float guidance, void* stream) {
    if (Bi < 0 || C < 0 || H < 0 || W < 0) return fail(AF_E_INVALID_ARG, "negative size");
    long n = (long)Bi * C * H * W;
    if (n == 0) return AF_OK;
    if (!latents || !v) return fail(AF_E_INVALID_ARG, "NULL device pointer");
    if (!std::isfinite(sigma) || !std::isfinite(sigma_next) || !std::isfinite(guidance))
        return fail(AF_E_INVALID_ARG, "non-finite sigma or guidance");
    AF_K(euler_cfg(latents, v, n, sigma_next - sigma, guidance, guidance > 1.f ? 1 : 0, (hipStream_t)stream));
    return AF_OK;
}

af_status af_flow_cfg_inputs(const float* latents, int Bi, int C, int H, int W, float sigma, int cfg_on,
                             float* x_in, float* tau, void* stream) {
    if (Bi < 0 || C < 0 || H < 0 || W < 0) return fail(AF_E_INVALID_ARG, "negative size");
    const long n = (long)Bi * C * H * W;
    if (Bi == 0) return AF_OK;
    if (!latents || !x_in || !tau) return fail(AF_E_INVALID_ARG, "NULL device pointer");
    if (!std::isfinite(sigma)) return fail(AF_E_INVALID_ARG, "non-finite sigma");
    const long nin = cfg_on ? 2 * n : n;
    if ((const float*)x_in < latents + n && latents < (const float*)x_in + nin)
        return fail(AF_E_INVALID_ARG, "x_in overlaps latents");
    AF_K(cfg_inputs(latents, n, Bi, cfg_on ? 1 : 0, sigma, x_in, tau, (hipStream_t)stream));
    return AF_OK;
}

af_status af_sigma_schedule(int num_steps, double shift, float* out) {
    if (num_steps <= 0) return fail(AF_E_INVALID_ARG, "num_steps must be positive");
    if (!out) return fail(AF_E_INVALID_ARG, "output is NULL");
    if (!(shift > 0.0) || !std::isfinite(shift)) return fail(AF_E_INVALID_ARG, "shift must be positive");
    for (int i = 0; i <= num_steps; ++i) {
        double u = 1.0 - (double)i / (double)num_steps;
        out[i] = (float)(shift * u / (1.0 + (shift - 1.0) * u));
    }
    return AF_OK;
}

af_status af_profile(af_model* m, int enable) {
    if (!m) return fail(AF_E_INVALID_ARG, "model is NULL");
    DevGuard guard(m->device);
    if (enable) {
        AF_TRY(prof_collect(m));
        for (int i = 0; i < AF_K_COUNT; ++i) m->prof_ms[i] = 0.0, m->prof_n[i] = 0;
    }
    m->prof_on = enable != 0;
    return AF_OK;
}

af_status af_profile_read(af_model* m, int kclass, double* total_ms, int64_t* launches) {
    if (!m) return fail(AF_E_INVALID_ARG, "model is NULL");
    if (kclass < 0 || kclass >= AF_K_COUNT) return fail(AF_E_INVALID_ARG, "bad kernel class");
    DevGuard guard(m->device);
    AF_TRY(prof_collect(m));
    if (total_ms) *total_ms = m->prof_ms[kclass];
    if (launches) *launches = m->prof_n[kclass];
    return AF_OK;
}

void af_destroy(af_model* m) {
    if (!m) return;
    {
        DevGuard guard(m->device);
        for (auto& r : m->prof_pool) {
            (void)hipEventDestroy(r.a);
            (void)hipEventDestroy(r.b);
        }
        if (m->arena) (void)hipFree(m->arena);
        if (m->work) (void)hipFree(m->work);
        if (m->arena8) (void)hipFree(m->arena8);
    }
    delete m;
}

const char* af_status_string(af_status s) {
    switch (s) {
        case AF_OK: return "ok";
        case AF_E_INVALID_ARG: return "invalid argument";
        case AF_E_SHAPE: return "shape error";
        case AF_E_UNSUPPORTED: return "unsupported configuration";
        case AF_E_OOM: return "out of memory";
        case AF_E_HIP: return "HIP error";
        case AF_E_STATE: return "invalid state";
    }
    return "unknown status";
}

const char* af_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

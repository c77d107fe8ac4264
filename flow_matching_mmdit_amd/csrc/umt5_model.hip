// Executor behind include/umt5.h: configuration checks, the weight arena and its
// packing, the workspace and the launch sequence of one encode (the text encoder
// of [DEEP] section 2.1 文本编码器, run as a random-weight workload).
#include <algorithm>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "af_internal.h"
#include "../../include/umt5.h"

using namespace af;

namespace {

#define U_FAIL(st, msg) return af::report((st), (msg))
#define U_HIP(call)                                                                                  \
    do {                                                                                             \
        hipError_t e_ = (call);                                                                      \
        if (e_ != hipSuccess) return af::report(AF_E_HIP, (std::string(#call) + ": " + hipGetErrorString(e_)).c_str()); \
    } while (0)

struct USlot {
    std::string name;
    int64_t rows, cols;
    size_t offset;     // floats, in the canonical blob
    int buf;           // destination buffer
    size_t dst_elem;   // element offset in the destination
    int layout;        // PackLayout
    bool f32;          // stored fp32 (norm weights, relative-position tables)
};

struct ULayer {
    int ln1, wqkv, wo, ln2, wi01, wo_ff;   // buffer ids
};

af_status check_config(const af_umt5_config* c) {
    if (!c) U_FAIL(AF_E_INVALID_ARG, "config is NULL");
    if (c->d_model <= 0 || c->num_heads <= 0 || c->num_layers < 0 || c->d_ff <= 0 || c->vocab_size <= 0 ||
        c->rel_buckets <= 0 || c->rel_max_distance <= 0 || c->max_batch < 0 || c->max_tokens < 0)
        U_FAIL(AF_E_INVALID_ARG, "config has a negative or zero size");
    if (!(c->eps > 0.f)) U_FAIL(AF_E_INVALID_ARG, "eps must be > 0");
    if (c->d_model % c->num_heads != 0 || c->d_model / c->num_heads != 64)
        U_FAIL(AF_E_UNSUPPORTED, "heads of 64 channels (d_model / num_heads = 64) are built");
    if (c->d_model % 256 != 0 || c->d_model > 4096) U_FAIL(AF_E_UNSUPPORTED, "d_model must be a multiple of 256, <= 4096");
    if (c->d_ff % 128 != 0) U_FAIL(AF_E_UNSUPPORTED, "d_ff must be a multiple of 128");
    if (c->rel_buckets != 32 || c->rel_max_distance != 128)
        U_FAIL(AF_E_UNSUPPORTED, "relative-position buckets: 32 buckets with maximum distance 128 are built");
    if (c->max_tokens > 512) U_FAIL(AF_E_UNSUPPORTED, "at most 512 tokens per sample");
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

}  // namespace

struct af_umt5 {
    af_umt5_config cfg;
    int device = 0;
    std::vector<USlot> slots;
    std::vector<size_t> buf_bytes;
    std::vector<void*> bufs;
    std::vector<ULayer> layers;
    int b_embed = -1, b_rel = -1, b_final = -1;
    size_t total_floats = 0;
    std::map<size_t, size_t> loaded;
    void* arena = nullptr;
    // workspace
    long Mmax = 0, Mp = 0;
    float* x = nullptr;          // residual stream [Mmax, d] fp32
    bf16_t* nrm = nullptr;       // norm output [Mp, d]
    bf16_t* qkv = nullptr;       // [Mp, 3d]
    bf16_t* attn = nullptr;      // [Mp, d]
    bf16_t* hbuf = nullptr;      // gated FFN output [Mp, d_ff]
    float* ones = nullptr;       // unit gate [d]
    float* bias_rows = nullptr;  // [L][H][2 Tmax - 1]
    float* part = nullptr;       // split-K partial sums [KSPLIT_MAX][Mmax, d]
    int n_cu = 0;
    float* staging = nullptr;
    size_t staging_floats = 0;
    void* work = nullptr;
};

namespace {

void build_slots(af_umt5* m) {
    const af_umt5_config& c = m->cfg;
    const long d = c.d_model, F = c.d_ff, H = c.num_heads, NB = c.rel_buckets;
    auto newbuf = [&](size_t bytes) {
        m->buf_bytes.push_back(bytes);
        return (int)m->buf_bytes.size() - 1;
    };
    size_t off = 0;
    auto add = [&](const std::string& name, int64_t rows, int64_t cols, int buf, size_t dst, int layout, bool f32) {
        m->slots.push_back(USlot{name, rows, cols, off, buf, dst, layout, f32});
        off += (size_t)rows * cols;
    };
    m->b_embed = newbuf((size_t)c.vocab_size * d * 2);
    m->b_rel = newbuf((size_t)c.num_layers * NB * H * 4);
    add("embed", c.vocab_size, d, m->b_embed, 0, PACK_PLAIN, false);
    for (int l = 0; l < c.num_layers; ++l) {
        const std::string p = "layer" + std::to_string(l) + ".";
        ULayer L;
        L.ln1 = newbuf(d * 4);
        L.wqkv = newbuf(3 * d * d * 2);
        L.wo = newbuf(d * d * 2);
        L.ln2 = newbuf(d * 4);
        L.wi01 = newbuf(2 * F * d * 2);
        L.wo_ff = newbuf(d * F * 2);
        m->layers.push_back(L);
        add(p + "ln1", d, 1, L.ln1, 0, PACK_PLAIN, true);
        add(p + "wq", d, d, L.wqkv, 0, PACK_PLAIN, false);
        add(p + "wk", d, d, L.wqkv, d * d, PACK_PLAIN, false);
        add(p + "wv", d, d, L.wqkv, 2 * d * d, PACK_PLAIN, false);
        add(p + "wo", d, d, L.wo, 0, PACK_PLAIN, false);
        add(p + "rel_bias", NB, H, m->b_rel, (size_t)l * NB * H, PACK_PLAIN, true);
        add(p + "ln2", d, 1, L.ln2, 0, PACK_PLAIN, true);
        add(p + "wi0", F, d, L.wi01, 0, PACK_FFN_GATE, false);
        add(p + "wi1", F, d, L.wi01, 0, PACK_FFN_UP, false);
        add(p + "wo_ff", d, F, L.wo_ff, 0, PACK_PLAIN, false);
    }
    m->b_final = newbuf(d * 4);
    add("final_ln", d, 1, m->b_final, 0, PACK_PLAIN, true);
    m->total_floats = off;
}

bool complete(const af_umt5* m) {
    size_t cur = 0;
    for (auto& iv : m->loaded) {
        if (iv.first > cur) return false;
        cur = std::max(cur, iv.second);
    }
    return cur >= m->total_floats;
}

void mark_loaded(af_umt5* m, size_t a, size_t b) {
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

GemmLaunch gemm_launch(const af_umt5* m, const void* A, long lda, const void* W, long ldw, int M, int N, int K,
                       int epi, int B, int T) {
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
    L.epi = epi;
    L.resid = m->x;
    L.mod = m->ones;        // unit gate: resid += acc
    L.mod_stride = 0;
    L.geom = RowGeom{B, T, 0};
    L.n_cu = m->n_cu;   // lets small launches use 128 x 128 tiles
    return L;
}

constexpr int KSPLIT_MAX = 4;

#define U_K(call)                                                                                           \
    do {                                                                                                    \
        hipError_t e_ = (call);                                                                             \
        if (e_ != hipSuccess) return af::report(AF_E_HIP, (std::string(#call) + ": " + hipGetErrorString(e_)).c_str()); \
    } while (0)

// x += A W^T for the N = d_model products (out-projection, FFN output). With few
// 256 x 256 tiles for the compute units (M = B T rows is small for a text
// encoder) and a long K (the FFN output, K = d_ff), K is cut into up to four
// ranges whose fp32 partial sums are added to x in a fixed order afterwards.
af_status resid_gemm(af_umt5* m, const void* A, long lda, const void* W, int K, int B, int T, hipStream_t s) {
    const int d = m->cfg.d_model, M = B * T;
    const int tiles = ((M + 255) / 256) * (d / 256);
    // each range keeps at least 1280 of K: below that the fixed cost of a tile (pipeline
    // fill, the fp32 partial store) and the extra summing pass outweigh the better fill.
    // Ranges are counted against two 128 x 128-tile workgroups per CU (gemm_bf16 takes
    // that tile size when the 256 x 256 tiles fill at most half the CUs).
    int ks = std::min({KSPLIT_MAX, m->n_cu / std::max(2 * tiles, 1), K / 1280});
    while (ks > 1 && K % (32 * ks) != 0) --ks;
    if (ks < 2) {
        U_K(gemm_bf16(gemm_launch(m, A, lda, W, lda, M, d, K, EPI_GATED_RESID, B, T), s));
        return AF_OK;
    }
    GemmLaunch L = gemm_launch(m, A, lda, W, lda, M, d, K, EPI_PARTIAL, B, T);
    L.C = m->part;
    L.ksplit = ks;
    U_K(gemm_bf16(L, s));
    U_K(splitk_resid(m->part, ks, M, d, m->x, s));
    return AF_OK;
}

af_status run_encode(af_umt5* m, const int32_t* ids, const uint8_t* mask, int B, int T, int stop_after, float* out,
                     hipStream_t s) {
    const af_umt5_config& c = m->cfg;
    const int d = c.d_model, F = c.d_ff, H = c.num_heads;
    const int M = B * T;
    auto buf = [&](int id) { return m->bufs[id]; };
    U_K(umt5_embed(ids, M, (const bf16_t*)buf(m->b_embed), c.vocab_size, d, m->x, s));
    if (stop_after == -1) {
        U_HIP(hipMemcpyAsync(out, m->x, (size_t)M * d * 4, hipMemcpyDeviceToDevice, s));
        return AF_OK;
    }
    U_K(umt5_rel_bias_rows((const float*)buf(m->b_rel), c.num_layers, H, T, m->bias_rows, s));
    for (int l = 0; l < c.num_layers; ++l) {
        const ULayer& Ly = m->layers[l];
        U_K(umt5_rms_norm(m->x, M, d, (const float*)buf(Ly.ln1), c.eps, m->nrm, true, s));
        GemmLaunch Lq = gemm_launch(m, m->nrm, d, buf(Ly.wqkv), d, M, 3 * d, d, EPI_STORE, B, T);
        Lq.C = m->qkv;
        Lq.ldc = 3 * d;
        U_K(gemm_bf16(Lq, s));
        U_K(umt5_attention(m->qkv, B, T, H, d, m->bias_rows + (size_t)l * H * (2 * T - 1), mask, m->attn, s));
        {
            af_status st = resid_gemm(m, m->attn, d, buf(Ly.wo), d, B, T, s);
            if (st != AF_OK) return st;
        }
        U_K(umt5_rms_norm(m->x, M, d, (const float*)buf(Ly.ln2), c.eps, m->nrm, true, s));
        GemmLaunch Lf = gemm_launch(m, m->nrm, d, buf(Ly.wi01), d, M, 2 * F, d, EPI_GEGLU, B, T);
        Lf.C = m->hbuf;
        Lf.ldc = F;
        U_K(gemm_bf16(Lf, s));
        {
            af_status st = resid_gemm(m, m->hbuf, F, buf(Ly.wo_ff), F, B, T, s);
            if (st != AF_OK) return st;
        }
        if (stop_after == l) {
            U_HIP(hipMemcpyAsync(out, m->x, (size_t)M * d * 4, hipMemcpyDeviceToDevice, s));
            return AF_OK;
        }
    }
    U_K(umt5_rms_norm(m->x, M, d, (const float*)buf(m->b_final), c.eps, out, false, s));
    return AF_OK;
}

af_status check_encode(af_umt5* m, const int32_t* ids, int B, int T, const void* out) {
    if (!m) U_FAIL(AF_E_INVALID_ARG, "encoder is NULL");
    if (B < 0 || T < 0) U_FAIL(AF_E_INVALID_ARG, "negative batch or token count");
    if (B > m->cfg.max_batch) U_FAIL(AF_E_SHAPE, "batch exceeds max_batch");
    if (T > m->cfg.max_tokens) U_FAIL(AF_E_SHAPE, "token count exceeds max_tokens");
    if (B > 0 && T > 0 && (!ids || !out)) U_FAIL(AF_E_INVALID_ARG, "ids or output pointer is NULL");
    if (!complete(m)) U_FAIL(AF_E_STATE, "weights are not complete");
    return AF_OK;
}

}  // namespace

extern "C" {

af_status af_umt5_config_default(af_umt5_config* c) {
    if (!c) U_FAIL(AF_E_INVALID_ARG, "config is NULL");
    c->d_model = 2048;
    c->num_heads = 32;
    c->num_layers = 24;
    c->d_ff = 5120;
    c->vocab_size = 32128;
    c->rel_buckets = 32;
    c->rel_max_distance = 128;
    c->eps = 1e-6f;
    c->max_batch = 8;
    c->max_tokens = 256;
    return AF_OK;
}

af_status af_umt5_weight_count(const af_umt5_config* c, int* n_tensors, size_t* total_floats) {
    af_status st = check_config(c);
    if (st != AF_OK) return st;
    if (!n_tensors) U_FAIL(AF_E_INVALID_ARG, "n_tensors is NULL");
    af_umt5 tmp;
    tmp.cfg = *c;
    build_slots(&tmp);
    *n_tensors = (int)tmp.slots.size();
    if (total_floats) *total_floats = tmp.total_floats;
    return AF_OK;
}

af_status af_umt5_weight_info(const af_umt5_config* c, int index, char* name, int name_cap, int64_t* rows,
                              int64_t* cols, size_t* offset) {
    af_status st = check_config(c);
    if (st != AF_OK) return st;
    af_umt5 tmp;
    tmp.cfg = *c;
    build_slots(&tmp);
    if (index < 0 || index >= (int)tmp.slots.size()) U_FAIL(AF_E_INVALID_ARG, "tensor index out of range");
    const USlot& S = tmp.slots[index];
    if (name && name_cap > 0) {
        std::strncpy(name, S.name.c_str(), (size_t)name_cap - 1);
        name[name_cap - 1] = 0;
    }
    if (rows) *rows = S.rows;
    if (cols) *cols = S.cols;
    if (offset) *offset = S.offset;
    return AF_OK;
}

af_status af_umt5_create(const af_umt5_config* c, int device, af_umt5** out) {
    if (!out) U_FAIL(AF_E_INVALID_ARG, "out is NULL");
    *out = nullptr;
    af_status st = check_config(c);
    if (st != AF_OK) return st;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev)
        U_FAIL(AF_E_INVALID_ARG, "no such device");
    DevGuard guard(device);
    af_umt5* m = new af_umt5();
    m->cfg = *c;
    m->device = device;
    build_slots(m);
    auto cleanup = [&](af_status s, const char* msg) {
        af_umt5_destroy(m);
        return af::report(s, msg);
    };
    size_t total = 0;
    std::vector<size_t> boff(m->buf_bytes.size());
    for (size_t i = 0; i < m->buf_bytes.size(); ++i) {
        boff[i] = total;
        total += align256(m->buf_bytes[i]);
    }
    if (hipMalloc(&m->arena, total) != hipSuccess) return cleanup(AF_E_OOM, "weight arena allocation failed");
    for (size_t i = 0; i < boff.size(); ++i) m->bufs.push_back((char*)m->arena + boff[i]);

    const long d = c->d_model, F = c->d_ff, H = c->num_heads;
    const long Bm = std::max(c->max_batch, 1), Tm = std::max(c->max_tokens, 1);
    m->Mmax = Bm * Tm;
    // GEMM A operands carry one 256-row tile of padding (tail tiles read past the last row)
    m->Mp = m->Mmax + 256;
    m->staging_floats = 16u << 20;
    std::vector<std::pair<void**, size_t>> ws = {
        {(void**)&m->x, (size_t)m->Mmax * d * 4},
        {(void**)&m->nrm, (size_t)m->Mp * d * 2},
        {(void**)&m->qkv, (size_t)m->Mp * 3 * d * 2},
        {(void**)&m->attn, (size_t)m->Mp * d * 2},
        {(void**)&m->hbuf, (size_t)m->Mp * F * 2},
        {(void**)&m->ones, (size_t)d * 4},
        {(void**)&m->bias_rows, (size_t)std::max(c->num_layers, 1) * H * (2 * Tm - 1) * 4},
        {(void**)&m->part, (size_t)KSPLIT_MAX * m->Mmax * d * 4},
        {(void**)&m->staging, m->staging_floats * 4},
    };
    if (hipDeviceGetAttribute(&m->n_cu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || m->n_cu <= 0)
        return cleanup(AF_E_HIP, "compute-unit count query failed");
    size_t wtotal = 0;
    for (auto& e : ws) wtotal += align256(e.second);
    if (hipMalloc(&m->work, wtotal) != hipSuccess) return cleanup(AF_E_OOM, "workspace allocation failed");
    // zero once: the padding rows the GEMM tail tiles read hold finite values
    if (hipMemset(m->work, 0, wtotal) != hipSuccess) return cleanup(AF_E_HIP, "workspace clear failed");
    size_t o = 0;
    for (auto& e : ws) {
        *e.first = (char*)m->work + o;
        o += align256(e.second);
    }
    std::vector<float> one((size_t)d, 1.0f);
    if (hipMemcpy(m->ones, one.data(), (size_t)d * 4, hipMemcpyHostToDevice) != hipSuccess)
        return cleanup(AF_E_HIP, "unit gate upload failed");
    if (hipDeviceSynchronize() != hipSuccess) return cleanup(AF_E_HIP, "device synchronize failed");
    *out = m;
    return AF_OK;
}

af_status af_umt5_load_weights(af_umt5* m, const float* host, size_t offset, size_t n, void* stream) {
    if (!m) U_FAIL(AF_E_INVALID_ARG, "encoder is NULL");
    if (n == 0) return AF_OK;
    if (!host) U_FAIL(AF_E_INVALID_ARG, "host pointer is NULL");
    if (offset > m->total_floats || n > m->total_floats - offset)
        U_FAIL(AF_E_SHAPE, "slice extends past the end of the weight blob");
    DevGuard guard(m->device);
    hipStream_t s = (hipStream_t)stream;
    const size_t end = offset + n;
    for (const USlot& S : m->slots) {
        const size_t ts = S.offset, te = S.offset + (size_t)S.rows * S.cols;
        const size_t a = std::max(ts, offset), b = std::min(te, end);
        if (a >= b) continue;
        void* dst = (char*)m->bufs[S.buf] + S.dst_elem * (S.f32 ? 4 : 2);
        for (size_t c0 = a; c0 < b; c0 += m->staging_floats) {
            const size_t cn = std::min(m->staging_floats, b - c0);
            U_HIP(hipMemcpyAsync(m->staging, host + (c0 - offset), cn * 4, hipMemcpyHostToDevice, s));
            U_K(pack_weights(m->staging, (long)cn, (long)(c0 - ts), dst, S.f32 ? AF_F32 : AF_BF16, S.layout,
                             (int)S.cols, s));
        }
    }
    mark_loaded(m, offset, end);
    U_HIP(hipStreamSynchronize(s));
    return AF_OK;
}

af_status af_umt5_encode(af_umt5* m, const int32_t* ids, const uint8_t* mask, int B, int T, float* out,
                         void* stream) {
    af_status st = check_encode(m, ids, B, T, out);
    if (st != AF_OK) return st;
    if (B == 0 || T == 0) return AF_OK;
    DevGuard guard(m->device);
    return run_encode(m, ids, mask, B, T, 1 << 30, out, (hipStream_t)stream);
}

af_status af_umt5_encode_taps(af_umt5* m, const int32_t* ids, const uint8_t* mask, int B, int T,
                              int stop_after_layer, float* residual_out, void* stream) {
    af_status st = check_encode(m, ids, B, T, residual_out);
    if (st != AF_OK) return st;
    if (stop_after_layer < -1 || stop_after_layer >= m->cfg.num_layers)
        U_FAIL(AF_E_INVALID_ARG, "stop_after_layer out of range");
    if (B == 0 || T == 0) return AF_OK;
    DevGuard guard(m->device);
    return run_encode(m, ids, mask, B, T, stop_after_layer, residual_out, (hipStream_t)stream);
}

void af_umt5_destroy(af_umt5* m) {
    if (!m) return;
    {
        DevGuard guard(m->device);
        if (m->arena) (void)hipFree(m->arena);
        if (m->work) (void)hipFree(m->work);
    }
    delete m;
}

}  // extern "C"

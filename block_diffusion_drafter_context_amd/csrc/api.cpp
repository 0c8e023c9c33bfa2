// api.cpp -- the extern "C" surface of libdflash (see include/dflash.h):
// argument checks, context state (length, page table) and launch order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/dflash.h"
#include "host.h"
#include "kernels.h"

using namespace dflash;

struct dflash_ctx {
    DevCtx dev;
    Tracer tracer;
    std::vector<hipEvent_t> events;
    dflash_config cfg;
    int32_t length = 0;
    bool dev_len = false;  // the length lives in the workspace's device word (host length unused)
    int device = 0;
    std::string err;
};

namespace {

dflash_status fail(dflash_ctx* c, dflash_status st, const std::string& msg) {
    if (c) c->err = msg;
    return st;
}

dflash_status hip_fail(dflash_ctx* c, hipError_t e, const char* where) {
    std::string m = std::string(where) + ": " + hipGetErrorString(e);
    return fail(c, DFLASH_ERR_HIP, m);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Check that the current HIP device is the one the context was created on.
dflash_status check_device(dflash_ctx* c) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(c, e, "hipGetDevice");
    if (dev != c->device) return fail(c, DFLASH_ERR_STATE, "current HIP device differs from the context's device");
    return DFLASH_OK;
}

}  // namespace

extern "C" {

const char* dflash_status_str(int st) {
    switch (st) {
        case DFLASH_OK: return "DFLASH_OK";
        case DFLASH_ERR_INVAL: return "DFLASH_ERR_INVAL";
        case DFLASH_ERR_CAPACITY: return "DFLASH_ERR_CAPACITY";
        case DFLASH_ERR_HIP: return "DFLASH_ERR_HIP";
        case DFLASH_ERR_UNSUPPORTED: return "DFLASH_ERR_UNSUPPORTED";
        case DFLASH_ERR_STATE: return "DFLASH_ERR_STATE";
        default: return "DFLASH_ERR_UNKNOWN";
    }
}

const char* dflash_last_error(const dflash_ctx* c) { return c ? c->err.c_str() : ""; }

dflash_status dflash_feature_layers(int32_t target_layers, int32_t* out) {
    if (!out || target_layers < 8) return DFLASH_ERR_INVAL;
    feature_layers(target_layers, out);
    return DFLASH_OK;
}

dflash_status dflash_page_table(const dflash_config* cfg, int32_t* out, int32_t n) {
    Dims d;
    std::string err;
    dflash_status st = validate_config(cfg, &d, &err);
    if (st != DFLASH_OK) return st;
    if (!out || n < d.n_pages) return DFLASH_ERR_INVAL;
    std::vector<int32_t> pt = make_page_table(d.n_pages, cfg->page_seed);
    std::copy(pt.begin(), pt.end(), out);
    return DFLASH_OK;
}

dflash_status dflash_workspace_size(const dflash_config* cfg, size_t* ws, size_t* kv) {
    Dims d;
    std::string err;
    dflash_status st = validate_config(cfg, &d, &err);
    if (st != DFLASH_OK) return st;
    if (!ws || !kv) return DFLASH_ERR_INVAL;
    // sized for the largest device this library targets: 256 compute units
    Layout L = compute_layout(d, 256);
    *ws = L.total;
    *kv = L.kv_total;
    return DFLASH_OK;
}

dflash_status dflash_create(const dflash_config* cfg, const dflash_weights* w, void* workspace, size_t ws_bytes,
                            void* kv_pool, size_t kv_bytes, void* stream, dflash_ctx** out) {
    if (!out) return DFLASH_ERR_INVAL;
    *out = nullptr;
    Dims d;
    std::string err;
    dflash_status st = validate_config(cfg, &d, &err);
    if (st != DFLASH_OK) return st;
    if (!w || !workspace || (!kv_pool && d.max_ctx > 0)) return DFLASH_ERR_INVAL;
    if (!aligned(workspace, 256) || !aligned(kv_pool, 256)) return DFLASH_ERR_INVAL;
    if (!w->fc != !w->fc_norm) return DFLASH_ERR_INVAL;  // fusion weights come as a pair, or not at all
    for (int l = 0; l < d.Ld; ++l)
        if (!w->wk[l] || !w->wv[l]) return DFLASH_ERR_INVAL;

    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DFLASH_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return DFLASH_ERR_HIP;
    cus = std::min(std::max(cus, 1), 256);
    Layout L = compute_layout(d, cus);
    if (ws_bytes < L.total || kv_bytes < L.kv_total) return DFLASH_ERR_CAPACITY;

    // the static scratch of dflash_fuse_context_static: its address on this device
    if (static_scratch_init(dev) != hipSuccess) return DFLASH_ERR_HIP;

    dflash_ctx* c = new (std::nothrow) dflash_ctx();
    if (!c) return DFLASH_ERR_CAPACITY;
    c->cfg = *cfg;
    c->device = dev;
    DevCtx& x = c->dev;
    x.dm = d;
    x.lay = L;
    x.ws = static_cast<char*>(workspace);
    x.kv = static_cast<char*>(kv_pool);
    x.num_cus = cus;
    x.fc = w->fc;
    x.fc_norm = w->fc_norm;
    for (int l = 0; l < DFLASH_MAX_LAYERS; ++l) {
        x.attn_norm[l] = w->attn_norm[l];
        x.wq[l] = w->wq[l];
        x.wk[l] = w->wk[l];
        x.wv[l] = w->wv[l];
        x.wo[l] = w->wo[l];
        x.mlp_norm[l] = w->mlp_norm[l];
        x.wg[l] = w->wg[l];
        x.wu[l] = w->wu[l];
        x.wd[l] = w->wd[l];
    }
    x.final_norm = w->final_norm;
    x.embed = w->embed;
    x.lm_head = w->lm_head;
    x.tracer = &c->tracer;
    for (int l = 0; l < DFLASH_MAX_LAYERS; ++l) {
        const bool in = l < d.Ld;
        x.sw_wq[l] = in ? x.ws + L.sw_wq[l] : nullptr;
        x.sw_wk[l] = in ? x.ws + L.sw_wk[l] : nullptr;
        x.sw_wv[l] = in ? x.ws + L.sw_wv[l] : nullptr;
        x.sw_wo[l] = in ? x.ws + L.sw_wo[l] : nullptr;
        x.sw_wg[l] = in ? x.ws + L.sw_wg[l] : nullptr;
        x.sw_wu[l] = in ? x.ws + L.sw_wu[l] : nullptr;
        x.sw_wd[l] = in ? x.ws + L.sw_wd[l] : nullptr;
    }
    x.sw_lm = x.ws + L.sw_lm;
    x.sw_fc = x.ws + L.sw_fc;

    // rotary table: angle = pos * base^(-2i/d) in fp64, cos/sin stored as fp32
    const int half = d.d / 2;
    std::vector<float> cs((size_t)L.n_rope_pos * half), sn((size_t)L.n_rope_pos * half);
    std::vector<double> inv(half);
    for (int i = 0; i < half; ++i) inv[i] = std::pow(d.rope_base, -2.0 * i / d.d);
    for (int p = 0; p < L.n_rope_pos; ++p)
        for (int i = 0; i < half; ++i) {
            const double a = (double)p * inv[i];
            cs[(size_t)p * half + i] = (float)std::cos(a);
            sn[(size_t)p * half + i] = (float)std::sin(a);
        }
    std::vector<int32_t> pt = make_page_table(d.n_pages, cfg->page_seed);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    // swizzled copies of every streamed weight that was given
    const long long nqd = (long long)d.nq * d.d, nkd = (long long)d.nkv * d.d;
    struct Job { const void* src; long long N, K; const void* dst; };
    std::vector<Job> jobs;
    if (w->fc) jobs.push_back({w->fc, d.H, 5LL * d.H, x.sw_fc});
    if (w->lm_head) jobs.push_back({w->lm_head, d.V, d.H, x.sw_lm});
    for (int l = 0; l < d.Ld; ++l) {
        jobs.push_back({w->wk[l], nkd, d.H, x.sw_wk[l]});
        jobs.push_back({w->wv[l], nkd, d.H, x.sw_wv[l]});
        if (w->wq[l]) jobs.push_back({w->wq[l], nqd, d.H, x.sw_wq[l]});
        if (w->wo[l]) jobs.push_back({w->wo[l], d.H, nqd, x.sw_wo[l]});
        if (w->wg[l]) jobs.push_back({w->wg[l], d.F, d.H, x.sw_wg[l]});
        if (w->wu[l]) jobs.push_back({w->wu[l], d.F, d.H, x.sw_wu[l]});
        if (w->wd[l]) jobs.push_back({w->wd[l], d.H, d.F, x.sw_wd[l]});
    }
    for (const Job& j : jobs) {
        if ((e = launch_swizzle(d.dtype, j.src, (int)j.N, (int)j.K, const_cast<void*>(j.dst), s)) != hipSuccess) {
            delete c;
            return DFLASH_ERR_HIP;
        }
    }
    if ((e = hipMemcpyAsync(x.ws + L.rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, s)) != hipSuccess ||
        (e = hipMemcpyAsync(x.ws + L.rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, s)) != hipSuccess ||
        (pt.size() && (e = hipMemcpyAsync(x.ws + L.page_table, pt.data(), pt.size() * 4, hipMemcpyHostToDevice, s)) !=
                          hipSuccess) ||
        (e = hipMemsetAsync(x.ws + L.tile_cnt, 0, (size_t)L.max_tiles * 4, s)) != hipSuccess ||
        (e = hipMemsetAsync(x.ws + L.counters, 0, 64 * 4, s)) != hipSuccess ||
        (e = hipMemsetAsync(x.ws + L.best, 0, (size_t)kPassRowsMax * 8, s)) != hipSuccess ||
        (e = hipMemsetAsync(x.ws + L.ss_part, 0, (size_t)L.ss_stride * kPassRowsMax * 4 * 2, s)) != hipSuccess ||
        (e = hipStreamSynchronize(s)) != hipSuccess) {
        delete c;
        return DFLASH_ERR_HIP;
    }
    *out = c;
    return DFLASH_OK;
}

static void drop_events(dflash_ctx* c) {
    for (hipEvent_t e : c->events) (void)hipEventDestroy(e);
    c->events.clear();
    c->tracer = Tracer();
}

dflash_status dflash_destroy(dflash_ctx* c) {
    if (c) drop_events(c);
    delete c;
    return DFLASH_OK;
}

int32_t dflash_length(const dflash_ctx* c) { return c && !c->dev_len ? c->length : -1; }

static int* len_word(dflash_ctx* c) { return reinterpret_cast<int*>(c->dev.ws + c->dev.lay.len_dev); }

dflash_status dflash_device_length_enable(dflash_ctx* c, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    if (c->dev_len) return fail(c, DFLASH_ERR_STATE, "the length already lives on the device");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_len_set(len_word(c), c->length, s);
    if (e == hipSuccess) e = launch_len_set(len_word(c) + 1, 0, s);  // capacity-error flag
    if (e != hipSuccess) return hip_fail(c, e, "length word");
    c->dev_len = true;
    return DFLASH_OK;
}

dflash_status dflash_keep_accepted(dflash_ctx* c, const int32_t* result, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    if (!c->dev_len) return fail(c, DFLASH_ERR_STATE, "needs the device-resident length");
    if (!result) return fail(c, DFLASH_ERR_INVAL, "null result");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipError_t e = launch_len_keep(len_word(c), result, c->dev.dm.max_ctx, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(c, e, "keep accepted");
    return DFLASH_OK;
}

dflash_status dflash_set_length_async(dflash_ctx* c, int32_t new_len, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    if (!c->dev_len) return fail(c, DFLASH_ERR_STATE, "needs the device-resident length");
    if (new_len < 0 || new_len > c->dev.dm.max_ctx) return fail(c, DFLASH_ERR_INVAL, "new_len must be in [0, max_ctx]");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipError_t e = launch_len_set(len_word(c), new_len, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(c, e, "set length");
    return DFLASH_OK;
}

dflash_status dflash_read_device_length(dflash_ctx* c, int32_t* out, void* stream) {
    if (!c || !out) return DFLASH_ERR_INVAL;
    if (!c->dev_len) return fail(c, DFLASH_ERR_STATE, "needs the device-resident length");
    if (!aligned(out, 4)) return fail(c, DFLASH_ERR_INVAL, "out misaligned");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipError_t e = launch_len_read(len_word(c), out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(c, e, "read length");
    return DFLASH_OK;
}

dflash_status dflash_fuse_context(dflash_ctx* c, const void* const* layer_hidden, int64_t ld, int32_t M,
                                  void* fused_out, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    const Dims& d = c->dev.dm;
    if (!layer_hidden || !fused_out) return fail(c, DFLASH_ERR_INVAL, "null pointer");
    if (!c->dev.fc) return fail(c, DFLASH_ERR_STATE, "context was created without fusion weights");
    if (M < 1 || M > d.max_rows) return fail(c, DFLASH_ERR_CAPACITY, "M must be in [1, max_rows]");
    if (ld < d.H || ld % (16 / d.elem)) return fail(c, DFLASH_ERR_INVAL, "ld must be >= H and keep rows 16-byte aligned");
    int32_t sel[5];
    feature_layers(d.Lt, sel);
    const void* slabs[5];
    for (int i = 0; i < 5; ++i) {
        slabs[i] = layer_hidden[sel[i]];
        if (!slabs[i] || !aligned(slabs[i], 16)) return fail(c, DFLASH_ERR_INVAL, "selected layer pointer null or misaligned");
    }
    if (!aligned(fused_out, 16)) return fail(c, DFLASH_ERR_INVAL, "fused_out misaligned");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipError_t e = launch_fuse(c->dev, slabs, ld, M, fused_out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(c, e, "fuse launch");
    return DFLASH_OK;
}

dflash_status dflash_fuse_context_static(dflash_ctx* c, const void* const* layer_hidden, int64_t ld, int32_t M,
                                         void* fused_out, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    const Dims& d = c->dev.dm;
    if (!layer_hidden || !fused_out) return fail(c, DFLASH_ERR_INVAL, "null pointer");
    if (!c->dev.fc) return fail(c, DFLASH_ERR_STATE, "context was created without fusion weights");
    if (M < 1 || M > DFLASH_MAX_BLOCK)
        return fail(c, DFLASH_ERR_CAPACITY, "M must be in [1, 16]: the static scratch holds one 16-row fusion");
    if (!static_scratch_fits(c->dev))
        return fail(c, DFLASH_ERR_UNSUPPORTED, "hidden size or CU count beyond the static scratch");
    if (ld < d.H || ld % (16 / d.elem)) return fail(c, DFLASH_ERR_INVAL, "ld must be >= H and keep rows 16-byte aligned");
    int32_t sel[5];
    feature_layers(d.Lt, sel);
    const void* slabs[5];
    for (int i = 0; i < 5; ++i) {
        slabs[i] = layer_hidden[sel[i]];
        if (!slabs[i] || !aligned(slabs[i], 16)) return fail(c, DFLASH_ERR_INVAL, "selected layer pointer null or misaligned");
    }
    if (!aligned(fused_out, 16)) return fail(c, DFLASH_ERR_INVAL, "fused_out misaligned");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipError_t e = launch_fuse_static(c->dev, c->device, slabs, ld, M, fused_out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(c, e, "static fuse launch");
    return DFLASH_OK;
}

dflash_status dflash_inject_kv(dflash_ctx* c, const void* fused, int64_t ld, int32_t M, int32_t pos0, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    const Dims& d = c->dev.dm;
    if (!fused || !aligned(fused, 16)) return fail(c, DFLASH_ERR_INVAL, "fused null or misaligned");
    if (ld < d.H || ld % (16 / d.elem)) return fail(c, DFLASH_ERR_INVAL, "ld must be >= H and keep rows 16-byte aligned");
    if (c->dev_len) {  // rows go to the device length; the length itself is unchanged
        if (pos0 != -1) return fail(c, DFLASH_ERR_INVAL, "with the device-resident length pos0 must be -1");
        if (M < 1 || M > DFLASH_MAX_BLOCK || M > d.max_rows)
            return fail(c, DFLASH_ERR_CAPACITY, "with the device-resident length M must be in [1, 16]");
        dflash_status st = check_device(c);
        if (st != DFLASH_OK) return st;
        hipError_t e = launch_inject(c->dev, fused, ld, M, 0, static_cast<hipStream_t>(stream), len_word(c),
                                     len_word(c) + 1);
        if (e != hipSuccess) return hip_fail(c, e, "inject launch");
        return DFLASH_OK;
    }
    if (M < 1 || M > d.max_rows) return fail(c, DFLASH_ERR_CAPACITY, "M must be in [1, max_rows]");
    if (pos0 != c->length) return fail(c, DFLASH_ERR_STATE, "pos0 must equal the current length");
    if ((long long)pos0 + M > d.max_ctx) return fail(c, DFLASH_ERR_CAPACITY, "injection would exceed max_ctx");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipError_t e = launch_inject(c->dev, fused, ld, M, pos0, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(c, e, "inject launch");
    c->length = pos0 + M;
    return DFLASH_OK;
}

dflash_status dflash_draft_block(dflash_ctx* c, const int32_t* anchor, float* logits_out, int32_t* tokens_out,
                                 void* stream) {
    return dflash_draft_block_ex(c, anchor, logits_out, tokens_out, nullptr, 0, stream);
}

dflash_status dflash_draft_block_ex(dflash_ctx* c, const int32_t* anchor, float* logits_out, int32_t* tokens_out,
                                    void* layer_out, int64_t layer_ld, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    const DevCtx& x = c->dev;
    if (!anchor || !tokens_out) return fail(c, DFLASH_ERR_INVAL, "null anchor or tokens_out");
    if (!x.embed || !x.lm_head || !x.final_norm) return fail(c, DFLASH_ERR_INVAL, "draft needs embed, lm_head, final_norm");
    for (int l = 0; l < x.dm.Ld; ++l)
        if (!x.attn_norm[l] || !x.wq[l] || !x.wo[l] || !x.mlp_norm[l] || !x.wg[l] || !x.wu[l] || !x.wd[l])
            return fail(c, DFLASH_ERR_INVAL, "draft needs every layer's weights");
    if (logits_out && !aligned(logits_out, 4)) return fail(c, DFLASH_ERR_INVAL, "logits_out misaligned");
    if (layer_out && (layer_ld < x.dm.H || !aligned(layer_out, x.dm.elem)))
        return fail(c, DFLASH_ERR_INVAL, "layer_out misaligned or layer_ld < H");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipError_t e = launch_draft_block(x, c->length, anchor, logits_out, tokens_out, layer_out, layer_ld,
                                      c->dev_len ? len_word(c) : nullptr, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(c, e, "draft launch");
    return DFLASH_OK;
}

dflash_status dflash_verify_accept(dflash_ctx* c, const int32_t* draft, const int32_t* target, int32_t* result_out,
                                   void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    if (!draft || !target || !result_out) return fail(c, DFLASH_ERR_INVAL, "null pointer");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipError_t e = launch_accept(c->dev, draft, target, result_out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(c, e, "accept launch");
    return DFLASH_OK;
}

dflash_status dflash_rollback(dflash_ctx* c, int32_t new_len) {
    if (!c) return DFLASH_ERR_INVAL;
    if (c->dev_len) return fail(c, DFLASH_ERR_STATE, "the length lives on the device: use dflash_set_length_async");
    if (new_len < 0 || new_len > c->length) return fail(c, DFLASH_ERR_INVAL, "new_len must be in [0, length]");
    c->length = new_len;
    return DFLASH_OK;
}

}  // extern "C"

namespace {

dflash_status target_forward(dflash_ctx* c, const int32_t* tokens, const int32_t* parent, int32_t M,
                             float* logits_out, int32_t* argmax_out, void* const* capture, int64_t capture_ld,
                             void* stream, void* layer_out = nullptr, int64_t layer_ld = 0) {
    if (!c) return DFLASH_ERR_INVAL;
    if (c->dev_len) return fail(c, DFLASH_ERR_STATE, "not available with the device-resident length");
    const DevCtx& x = c->dev;
    const Dims& d = x.dm;
    if (!tokens || !argmax_out) return fail(c, DFLASH_ERR_INVAL, "null tokens or argmax_out");
    if (!parent && (M < 1 || M > DFLASH_MAX_BLOCK)) return fail(c, DFLASH_ERR_INVAL, "M must be in [1, 16]");
    if (parent && (M < 1 || M > DFLASH_TREE_MAX_NODES)) return fail(c, DFLASH_ERR_INVAL, "tree nodes must be in [1, 32]");
    if (!x.embed || !x.lm_head || !x.final_norm) return fail(c, DFLASH_ERR_INVAL, "needs embed, lm_head, final_norm");
    for (int l = 0; l < d.Ld; ++l)
        if (!x.attn_norm[l] || !x.wq[l] || !x.wo[l] || !x.mlp_norm[l] || !x.wg[l] || !x.wu[l] || !x.wd[l])
            return fail(c, DFLASH_ERR_INVAL, "needs every layer's weights");
    if (logits_out && !aligned(logits_out, 4)) return fail(c, DFLASH_ERR_INVAL, "logits_out misaligned");
    if (capture) {
        if (capture_ld < d.H) return fail(c, DFLASH_ERR_INVAL, "capture_ld must be >= H");
        int32_t sel[DFLASH_NUM_FEATURES];
        feature_layers(d.Lt, sel);
        for (int i = 0; i < DFLASH_NUM_FEATURES; ++i) {
            if (capture[i] && !aligned(capture[i], d.elem)) return fail(c, DFLASH_ERR_INVAL, "capture buffer misaligned");
            if (capture[i] && sel[i] >= d.Ld)
                return fail(c, DFLASH_ERR_INVAL, "capture requested for a layer beyond the context's draft_layers");
        }
    }
    if (layer_out) {
        if (capture) return fail(c, DFLASH_ERR_INVAL, "layer_out and capture are exclusive");
        if (layer_ld < d.H || !aligned(layer_out, d.elem)) return fail(c, DFLASH_ERR_INVAL, "layer_ld must be >= H");
    }
    if ((long long)c->length + M > d.max_ctx) return fail(c, DFLASH_ERR_CAPACITY, "forward would exceed max_ctx");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // a tree of more than 16 nodes: one pass of up to 32 rows where the
    // kernels allow it (each weight is read once for all rows), else two
    // passes, nodes 0..15 then 16..M-1, the second seeing its ancestors among
    // the first pass's nodes in the cache
    const int C0 = c->length;
    const int per_pass = parent && wide_pass_supported(x) ? DFLASH_TREE_MAX_NODES : DFLASH_MAX_BLOCK;
    for (int off = 0; off < M; off += per_pass) {
        const int m = std::min(M - off, per_pass);
        void* cap_off[DFLASH_NUM_FEATURES];
        if (capture)
            for (int i = 0; i < DFLASH_NUM_FEATURES; ++i)
                cap_off[i] = capture[i] ? static_cast<char*>(capture[i]) + (size_t)off * capture_ld * d.elem : nullptr;
        void* lo = layer_out ? static_cast<char*>(layer_out) + (size_t)off * layer_ld * d.elem : nullptr;
        hipError_t e = launch_causal_forward(x, C0 + off, tokens + off, m, logits_out ? logits_out + (size_t)off * d.V : nullptr,
                                             argmax_out + off, capture ? cap_off : nullptr, capture_ld, s, parent,
                                             lo, layer_ld, off, C0, parent ? M : 0, M);
        if (e != hipSuccess) return hip_fail(c, e, "target forward launch");
    }
    c->length += M;
    return DFLASH_OK;
}

}  // namespace

extern "C" {

dflash_status dflash_target_forward(dflash_ctx* c, const int32_t* tokens, int32_t M, float* logits_out,
                                    int32_t* argmax_out, void* const* capture, int64_t capture_ld, void* stream) {
    return target_forward(c, tokens, nullptr, M, logits_out, argmax_out, capture, capture_ld, stream);
}

dflash_status dflash_target_forward_tree(dflash_ctx* c, const int32_t* tokens, const int32_t* parent, int32_t M,
                                         float* logits_out, int32_t* argmax_out, void* const* capture,
                                         int64_t capture_ld, void* stream) {
    if (c && !parent) return fail(c, DFLASH_ERR_INVAL, "null parent");
    return target_forward(c, tokens, parent, M, logits_out, argmax_out, capture, capture_ld, stream);
}

dflash_status dflash_target_forward_ex(dflash_ctx* c, const int32_t* tokens, const int32_t* parent, int32_t M,
                                       float* logits_out, int32_t* argmax_out, void* layer_out, int64_t layer_ld,
                                       void* stream) {
    return target_forward(c, tokens, parent, M, logits_out, argmax_out, nullptr, 0, stream, layer_out, layer_ld);
}

dflash_status dflash_draft_topk(dflash_ctx* c, const float* logits, int64_t ld, int32_t rows, int32_t K,
                                int32_t* ids_out, float* logp_out, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    const Dims& d = c->dev.dm;
    if (!logits || !ids_out || !logp_out) return fail(c, DFLASH_ERR_INVAL, "null pointer");
    if (rows < 1 || rows > DFLASH_MAX_BLOCK) return fail(c, DFLASH_ERR_INVAL, "rows must be in [1, 16]");
    if (K < 1 || K > DFLASH_TREE_MAX_K || K > d.V) return fail(c, DFLASH_ERR_INVAL, "K must be in [1, min(16, V)]");
    if (ld < d.V) return fail(c, DFLASH_ERR_INVAL, "ld must be >= V");
    if (!aligned(logits, 4)) return fail(c, DFLASH_ERR_INVAL, "logits misaligned");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    c->tracer.begin(DFLASH_TRACE_TREE, s);
    hipError_t e = launch_topk(c->dev, logits, ld, rows, K, ids_out, logp_out, s);
    if (e != hipSuccess) return hip_fail(c, e, "top-k launch");
    c->tracer.end(DFLASH_TRACE_TREE, s);
    return DFLASH_OK;
}

dflash_status dflash_build_tree(dflash_ctx* c, const int32_t* anchor, const int32_t* ids, const float* logp,
                                int32_t depths, int32_t K, int32_t budget, int32_t* tokens_out, int32_t* parent_out,
                                void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    if (!anchor || !ids || !logp || !tokens_out || !parent_out) return fail(c, DFLASH_ERR_INVAL, "null pointer");
    if (depths < 1 || depths > DFLASH_MAX_BLOCK - 1) return fail(c, DFLASH_ERR_INVAL, "depths must be in [1, 15]");
    if (K < 1 || K > DFLASH_TREE_MAX_K) return fail(c, DFLASH_ERR_INVAL, "K must be in [1, 16]");
    if (budget < 0 || budget > DFLASH_TREE_MAX_NODES - 1) return fail(c, DFLASH_ERR_INVAL, "budget must be in [0, 31]");
    long long nodes = 0, layer = 1;  // nodes of the full candidate tree (enough once it reaches the budget)
    for (int i = 0; i < depths && nodes < budget; ++i) {
        layer *= K;
        nodes += layer;
    }
    if (nodes < budget) return fail(c, DFLASH_ERR_INVAL, "budget exceeds the candidate tree's size");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    c->tracer.begin(DFLASH_TRACE_TREE, s);
    hipError_t e = launch_tree_build(anchor, c->dev.dm.V, ids, logp, depths, K, budget, tokens_out, parent_out, s);
    if (e != hipSuccess) return hip_fail(c, e, "tree build launch");
    c->tracer.end(DFLASH_TRACE_TREE, s);
    return DFLASH_OK;
}

dflash_status dflash_tree_accept(dflash_ctx* c, const int32_t* tokens, const int32_t* parent, const int32_t* target,
                                 int32_t M, int32_t* result_out, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    if (!tokens || !parent || !target || !result_out) return fail(c, DFLASH_ERR_INVAL, "null pointer");
    if (M < 1 || M > DFLASH_TREE_MAX_NODES) return fail(c, DFLASH_ERR_INVAL, "M must be in [1, 32]");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    c->tracer.begin(DFLASH_TRACE_TREE, s);
    hipError_t e = launch_tree_accept(tokens, parent, target, M, result_out, s);
    if (e != hipSuccess) return hip_fail(c, e, "tree accept launch");
    c->tracer.end(DFLASH_TRACE_TREE, s);
    return DFLASH_OK;
}

dflash_status dflash_sample_tokens(dflash_ctx* c, const float* logits, int64_t ld, int32_t rows, float temperature,
                                   uint64_t seed, int32_t* tokens_out, float* lse_out, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    const Dims& d = c->dev.dm;
    if (!logits || (!tokens_out && !lse_out)) return fail(c, DFLASH_ERR_INVAL, "null pointer");
    if (rows < 1 || rows > DFLASH_MAX_BLOCK) return fail(c, DFLASH_ERR_INVAL, "rows must be in [1, 16]");
    if (!(temperature > 0.f) || !std::isfinite(temperature)) return fail(c, DFLASH_ERR_INVAL, "temperature must be > 0");
    if (ld < d.V || !aligned(logits, 4)) return fail(c, DFLASH_ERR_INVAL, "ld must be >= V and logits aligned");
    if ((tokens_out && !aligned(tokens_out, 4)) || (lse_out && !aligned(lse_out, 4)))
        return fail(c, DFLASH_ERR_INVAL, "tokens_out / lse_out misaligned");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    c->tracer.begin(DFLASH_TRACE_SAMPLE, s);
    hipError_t e = launch_sample_tokens(c->dev, logits, ld, rows, temperature, seed, tokens_out, lse_out, s);
    if (e != hipSuccess) return hip_fail(c, e, "sample launch");
    c->tracer.end(DFLASH_TRACE_SAMPLE, s);
    return DFLASH_OK;
}

dflash_status dflash_verify_sample(dflash_ctx* c, const int32_t* draft, const float* draft_logits,
                                   const float* target_logits, int64_t ld, float temperature, uint64_t seed,
                                   int32_t* result_out, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    const Dims& d = c->dev.dm;
    if (!draft || !draft_logits || !target_logits || !result_out) return fail(c, DFLASH_ERR_INVAL, "null pointer");
    if (!(temperature > 0.f) || !std::isfinite(temperature)) return fail(c, DFLASH_ERR_INVAL, "temperature must be > 0");
    if (ld < d.V || !aligned(draft_logits, 4) || !aligned(target_logits, 4))
        return fail(c, DFLASH_ERR_INVAL, "ld must be >= V and logits aligned");
    if (!aligned(draft, 4) || !aligned(result_out, 4)) return fail(c, DFLASH_ERR_INVAL, "draft / result_out misaligned");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    c->tracer.begin(DFLASH_TRACE_SAMPLE, s);
    hipError_t e = launch_verify_sample(c->dev, draft, draft_logits, target_logits, ld, temperature, seed, result_out, s);
    if (e != hipSuccess) return hip_fail(c, e, "sampled verification launch");
    c->tracer.end(DFLASH_TRACE_SAMPLE, s);
    return DFLASH_OK;
}

dflash_status dflash_tree_commit(dflash_ctx* c, int32_t pos0, int32_t M, const int32_t* result, void* const* capture,
                                 int64_t capture_ld, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    const Dims& d = c->dev.dm;
    if (!result) return fail(c, DFLASH_ERR_INVAL, "null result");
    if (M < 1 || M > DFLASH_TREE_MAX_NODES) return fail(c, DFLASH_ERR_INVAL, "M must be in [1, 32]");
    const long long lim = c->dev_len ? d.max_ctx : c->length;
    if (pos0 < 0 || (long long)pos0 + M > lim) return fail(c, DFLASH_ERR_INVAL, "rows pos0..pos0+M-1 must be inside the context");
    if (capture) {
        if (capture_ld < d.H) return fail(c, DFLASH_ERR_INVAL, "capture_ld must be >= H");
        for (int i = 0; i < DFLASH_NUM_FEATURES; ++i)
            if (capture[i] && !aligned(capture[i], d.elem)) return fail(c, DFLASH_ERR_INVAL, "capture buffer misaligned");
    }
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    c->tracer.begin(DFLASH_TRACE_TREE, s);
    hipError_t e = launch_tree_commit(c->dev, pos0, M, result, capture, capture_ld, s);
    if (e != hipSuccess) return hip_fail(c, e, "tree commit launch");
    c->tracer.end(DFLASH_TRACE_TREE, s);
    return DFLASH_OK;
}

dflash_status dflash_load_kv(dflash_ctx* c, const void* k, const void* v, int32_t M, int32_t pos0, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    if (c->dev_len) return fail(c, DFLASH_ERR_STATE, "not available with the device-resident length");
    const Dims& d = c->dev.dm;
    if (!k || !v) return fail(c, DFLASH_ERR_INVAL, "null pointer");
    if (M < 1) return fail(c, DFLASH_ERR_INVAL, "M must be >= 1");
    if (pos0 != c->length) return fail(c, DFLASH_ERR_STATE, "pos0 must equal the current length");
    if ((long long)pos0 + M > d.max_ctx) return fail(c, DFLASH_ERR_CAPACITY, "load would exceed max_ctx");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipError_t e = launch_kv_copy(c->dev, const_cast<void*>(k), const_cast<void*>(v), M, pos0, true,
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(c, e, "kv copy launch");
    c->length = pos0 + M;
    return DFLASH_OK;
}

dflash_status dflash_read_kv(dflash_ctx* c, int32_t pos0, int32_t M, void* k_out, void* v_out, void* stream) {
    if (!c) return DFLASH_ERR_INVAL;
    if (!k_out || !v_out) return fail(c, DFLASH_ERR_INVAL, "null pointer");
    const long long lim = c->dev_len ? c->dev.dm.max_ctx : c->length;  // device length: the capacity bounds it
    if (M < 1 || pos0 < 0 || (long long)pos0 + M > lim)
        return fail(c, DFLASH_ERR_INVAL, "range must lie inside [0, length)");
    dflash_status st = check_device(c);
    if (st != DFLASH_OK) return st;
    hipError_t e = launch_kv_copy(c->dev, k_out, v_out, M, pos0, false, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(c, e, "kv copy launch");
    return DFLASH_OK;
}

dflash_status dflash_trace_enable(dflash_ctx* c, int32_t kernel_class, int32_t max_launches) {
    if (!c) return DFLASH_ERR_INVAL;
    if (kernel_class < DFLASH_TRACE_OFF || kernel_class > DFLASH_TRACE_SAMPLE || max_launches < 0 ||
        max_launches > (1 << 20))
        return fail(c, DFLASH_ERR_INVAL, "bad trace class or launch count");
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(c, e, "hipDeviceSynchronize");
    drop_events(c);
    if (kernel_class == DFLASH_TRACE_OFF || max_launches == 0) return DFLASH_OK;
    c->events.resize((size_t)2 * max_launches);
    for (size_t i = 0; i < c->events.size(); ++i) {
        if ((e = hipEventCreate(&c->events[i])) != hipSuccess) {
            c->events.resize(i);
            drop_events(c);
            return hip_fail(c, e, "hipEventCreate");
        }
    }
    c->tracer.cls = kernel_class;
    c->tracer.max = max_launches;
    c->tracer.n = 0;
    c->tracer.ev = c->events.data();
    return DFLASH_OK;
}

dflash_status dflash_trace_read(dflash_ctx* c, double* total_ms, int32_t* launches) {
    if (!c || !total_ms || !launches) return DFLASH_ERR_INVAL;
    double tot = 0.0;
    for (int i = 0; i < c->tracer.n; ++i) {
        hipError_t e = hipEventSynchronize(c->events[2 * i + 1]);
        if (e != hipSuccess) return hip_fail(c, e, "hipEventSynchronize");
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, c->events[2 * i], c->events[2 * i + 1]);
        if (e != hipSuccess) return hip_fail(c, e, "hipEventElapsedTime");
        tot += ms;
    }
    *total_ms = tot;
    *launches = c->tracer.n;
    return DFLASH_OK;
}

dflash_status dflash_trace_read_each(dflash_ctx* c, float* durations_ms, int32_t capacity, int32_t* launches) {
    if (!c || !durations_ms || !launches || capacity < 0) return DFLASH_ERR_INVAL;
    const int n = std::min(c->tracer.n, capacity);
    for (int i = 0; i < n; ++i) {
        hipError_t e = hipEventSynchronize(c->events[2 * i + 1]);
        if (e != hipSuccess) return hip_fail(c, e, "hipEventSynchronize");
        e = hipEventElapsedTime(&durations_ms[i], c->events[2 * i], c->events[2 * i + 1]);
        if (e != hipSuccess) return hip_fail(c, e, "hipEventElapsedTime");
    }
    *launches = n;
    return DFLASH_OK;
}

dflash_status dflash_hbm_read_probe(const void* buf, int64_t bytes, void* sink, int64_t* read_bytes, void* stream) {
    if (!buf || !sink || !read_bytes || bytes < 0 || (reinterpret_cast<uintptr_t>(buf) & 15) ||
        (reinterpret_cast<uintptr_t>(sink) & 3))
        return DFLASH_ERR_INVAL;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return DFLASH_ERR_HIP;
    long long rb = 0;
    const hipError_t e = dflash::launch_read_probe(buf, bytes, cus, static_cast<unsigned*>(sink), &rb,
                                                   static_cast<hipStream_t>(stream));
    *read_bytes = rb;
    return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

}  // extern "C"

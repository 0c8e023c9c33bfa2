// host.cpp -- host-only logic of libdflash (see host.h).
#include "host.h"

#include <algorithm>
#include <cstdio>

namespace dflash {

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

void feature_layers(int L, int32_t out[5]) {
    // floor(1 + i(L-3)/4 + 1/2) in integer arithmetic
    for (int i = 0; i < 5; ++i) out[i] = (6 + i * (L - 3)) / 4;
}

dflash_status validate_config(const dflash_config* c, Dims* o, std::string* err) {
    char buf[256];
    auto fail = [&](dflash_status st, const char* msg) {
        if (err) *err = msg;
        return st;
    };
    if (!c) return fail(DFLASH_ERR_INVAL, "config is NULL");
    if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16) return fail(DFLASH_ERR_INVAL, "dtype must be DFLASH_F32 or DFLASH_BF16");
    if (c->hidden <= 0 || c->hidden % 32) return fail(DFLASH_ERR_UNSUPPORTED, "hidden must be a positive multiple of 32");
    if (c->target_layers < 8 || c->target_layers > 1024) return fail(DFLASH_ERR_INVAL, "target_layers must be in [8, 1024]");
    if (c->draft_layers < 1 || c->draft_layers > DFLASH_MAX_LAYERS) return fail(DFLASH_ERR_INVAL, "draft_layers must be in [1, 64]");
    if (c->head_dim != 64 && c->head_dim != 128) return fail(DFLASH_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (c->n_kv_heads <= 0 || c->n_q_heads <= 0 || c->n_q_heads % c->n_kv_heads)
        return fail(DFLASH_ERR_INVAL, "n_q_heads must be a positive multiple of n_kv_heads");
    if (c->n_q_heads / c->n_kv_heads > 8) return fail(DFLASH_ERR_UNSUPPORTED, "at most 8 query heads per kv head");
    if (c->ffn <= 0 || c->ffn % 16) return fail(DFLASH_ERR_UNSUPPORTED, "ffn must be a positive multiple of 16");
    if (c->vocab <= 0 || c->vocab % 16) return fail(DFLASH_ERR_UNSUPPORTED, "vocab must be a positive multiple of 16");
    if (c->block < 2 || c->block > DFLASH_MAX_BLOCK) return fail(DFLASH_ERR_INVAL, "block must be in [2, 16]");
    if (c->mask_id < 0 || c->mask_id >= c->vocab) return fail(DFLASH_ERR_INVAL, "mask_id must be in [0, vocab)");
    if (c->page_size < 64 || c->page_size % 64 || c->page_size > 4096)
        return fail(DFLASH_ERR_UNSUPPORTED, "page_size must be a multiple of 64 in [64, 4096]");
    if (c->max_ctx < 0 || c->max_ctx > (1 << 24)) return fail(DFLASH_ERR_INVAL, "max_ctx must be in [0, 2^24]");
    if (c->max_rows < 1 || c->max_rows > (1 << 20)) return fail(DFLASH_ERR_INVAL, "max_rows must be in [1, 2^20]");
    if (!(c->rope_base > 1.0) || !(c->eps >= 0.0)) return fail(DFLASH_ERR_INVAL, "rope_base must be > 1 and eps >= 0");
    {   // every attention split must touch at most kMaxSplitPages pages
        const long long kps_max = ((long long)c->max_ctx + kMaxSplits - 1) / kMaxSplits + 2LL * kAttnChunk;
        if (std::max<long long>(kps_max, causal_split_keys(c->max_ctx)) / c->page_size + 2 > kMaxSplitPages)
            return fail(DFLASH_ERR_UNSUPPORTED, "max_ctx too large for this page_size");
    }
    const long long nqd = (long long)c->n_q_heads * c->head_dim;
    if (nqd % 32) return fail(DFLASH_ERR_UNSUPPORTED, "n_q_heads*head_dim must be a multiple of 32");
    if ((long long)c->vocab * c->hidden > (1LL << 40)) return fail(DFLASH_ERR_INVAL, "vocab*hidden too large");
    Dims d;
    d.dtype = c->dtype;
    d.H = c->hidden;
    d.Lt = c->target_layers;
    d.Ld = c->draft_layers;
    d.nq = c->n_q_heads;
    d.nkv = c->n_kv_heads;
    d.d = c->head_dim;
    d.F = c->ffn;
    d.V = c->vocab;
    d.B = c->block;
    d.mask_id = c->mask_id;
    d.page = c->page_size;
    d.max_ctx = c->max_ctx;
    d.max_rows = c->max_rows;
    d.n_pages = (c->max_ctx + c->page_size - 1) / c->page_size;
    d.elem = c->dtype == DFLASH_F32 ? 4 : 2;
    d.rope_base = c->rope_base;
    d.eps = c->eps;
    if (o) *o = d;
    (void)buf;
    return DFLASH_OK;
}

Layout compute_layout(const Dims& d, int num_cus) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    const size_t es = (size_t)d.elem;
    L.n_rope_pos = d.max_ctx + DFLASH_MAX_BLOCK;
    L.rope_cos = take((size_t)L.n_rope_pos * (d.d / 2) * 4);
    L.rope_sin = take((size_t)L.n_rope_pos * (d.d / 2) * 4);
    L.page_table = take((size_t)std::max(d.n_pages, 1) * 4);
    // rows of a pass: a 16-row block, or up to 32 verified tree nodes
    const size_t R = kPassRowsMax;
    L.x = take(R * d.H * es);
    L.q = take(R * d.nq * d.d * es);
    L.kblk = take((size_t)16 * d.nkv * d.d * es);
    L.vblkT = take((size_t)16 * d.nkv * d.d * es);
    L.obuf = take(R * d.nq * d.d * es);
    L.hbuf = take(R * d.F * es);
    L.rstd = take(R * 4);
    const int blk = 16 * kSkinnyNT;
    L.max_ss_tiles = (d.H + blk - 1) / blk;
    L.ss_stride = (L.max_ss_tiles + 15) / 16 * 16;
    L.ss_part = take((size_t)L.ss_stride * R * 4 * 2);  // two buffers (see the draft pass)
    // 4 waves per CU: measured best for every skinny-GEMM shape of the draft
    // pass (fewer concurrent weight streams keep DRAM pages open longer)
    L.nwaves = std::max(num_cus, 1) * 4;
    L.partial = take((size_t)L.nwaves * 2 * kSkinnyMaxNT * 256 * 4);
    // tiles of every skinny GEMM: qkv, o, gate/up, down, lm head, fuse, inject
    long long t = 0;
    const long long nqd = (long long)d.nq * d.d, nkd = (long long)d.nkv * d.d;
    t = std::max(t, (nqd + 2 * nkd) / 32);
    t = std::max(t, (long long)(d.H + blk - 1) / blk);
    t = std::max(t, (long long)(d.F + 15) / 16);
    t = std::max(t, (long long)(d.V + blk - 1) / blk);
    t = std::max(t, (long long)d.Ld * 2 * nkd / 32);
    L.max_tiles = (int)t;
    L.tile_cnt = take((size_t)L.max_tiles * 4);
    L.counters = take(64 * 4);
    L.best = take(R * 8);
    const size_t parts = (size_t)(kMaxSplits + 1) * d.nq * R;
    L.attn_o = take(parts * d.d * 4);
    L.attn_ml = take(parts * 2 * 4);
    L.len_dev = take(2 * 4);
    L.tree_info = take(2 * R * 4);
    L.topk_part = take((size_t)16 * kTopKSegs * (2 * kTopKMax + 2) * 4);
    L.sample_draw = take(64 + (size_t)((d.V + 1023) / 1024) * 8);
    const int e = d.elem;
    for (int l = 0; l < d.Ld; ++l) {
        L.sw_wq[l] = take(swizzled_bytes(nqd, d.H, e));
        L.sw_wk[l] = take(swizzled_bytes(nkd, d.H, e));
        L.sw_wv[l] = take(swizzled_bytes(nkd, d.H, e));
        L.sw_wo[l] = take(swizzled_bytes(d.H, nqd, e));
        L.sw_wg[l] = take(swizzled_bytes(d.F, d.H, e));
        L.sw_wu[l] = take(swizzled_bytes(d.F, d.H, e));
        L.sw_wd[l] = take(swizzled_bytes(d.H, d.F, e));
    }
    L.sw_lm = take(swizzled_bytes(d.V, d.H, e));
    L.sw_fc = take(swizzled_bytes(d.H, 5LL * d.H, e));
    L.total = off;
    L.kv_layer_kv = (size_t)d.n_pages * d.nkv * d.page * d.d * es;
    L.kv_total = L.kv_layer_kv * 2 * d.Ld;
    return L;
}

std::vector<int32_t> make_page_table(int n_pages, uint64_t seed) {
    std::vector<int32_t> p(std::max(n_pages, 0));
    for (int i = 0; i < n_pages; ++i) p[i] = i;
    if (seed == 0) return p;
    uint64_t s = seed;
    auto next = [&]() {  // splitmix64
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    };
    for (int i = n_pages - 1; i > 0; --i) {
        int j = (int)(next() % (uint64_t)(i + 1));
        std::swap(p[i], p[j]);
    }
    return p;
}

void attn_split_plan(int C, int nkv, int num_cus, int page, int* kps, int* ns, int wg_per_cu) {
    if (C <= 0) {
        *kps = kAttnChunk;
        *ns = 0;
        return;
    }
    // the splits plus the block's own part fill one round of resident
    // attention workgroups (kAttnWGPerCU per CU, over all kv heads), and every
    // split has at least three chunks (a split's fixed cost -- Q loads,
    // first-chunk latency, partial write and merge read -- is then amortised).
    // On MI355X at 36K keys one round beats 1.5 rounds (3 workgroups per CU) by
    // about 36 us per draft pass; at 4K the three-chunk minimum decides.
    long long target = std::max(1LL, (long long)wg_per_cu * num_cus / std::max(nkv, 1) - 1);
    long long per = (C + target - 1) / target;
    per = ((per + kAttnChunk - 1) / kAttnChunk) * kAttnChunk;
    per = std::max<long long>(per, 3 * kAttnChunk);
    // a split touches at most kMaxSplitPages pages (their ids are staged in LDS)
    const long long per_cap = std::max<long long>(kAttnChunk, ((long long)(kMaxSplitPages - 2) * page) / kAttnChunk * kAttnChunk);
    per = std::min(per, per_cap);
    long long n = (C + per - 1) / per;
    while (n > kMaxSplits) {
        per += kAttnChunk;
        n = (C + per - 1) / per;
    }
    *kps = (int)per;
    *ns = (int)n;
}

int causal_split_keys(int max_ctx) {
    long long per = (std::max(max_ctx, 1) + (long long)kMaxSplits - 1) / kMaxSplits;
    per = ((per + kAttnChunk - 1) / kAttnChunk) * kAttnChunk;
    // at least three chunks per split: at 4K context that gives 22 splits per
    // kv head, and the Qwen3-8B verify pass ran 1 % faster than with four
    return (int)std::max<long long>(per, 3 * kAttnChunk);
}

}  // namespace dflash

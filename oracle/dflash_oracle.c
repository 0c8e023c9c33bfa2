/*
 * dflash_oracle.c -- plain, slow, obviously correct CPU oracle for the DFlash
 * single-pass block-diffusion draft with KV injection and greedy verification.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke entry and the bench's
 * CPU-baseline leg.  It shares nothing with the HIP library.
 *
 * Sources (the web pages this method is described on):
 *  [A] "DFlash 深度解析：块扩散模型如何让 LLM 推理加速 6 倍——2026 投机解码完全指南"
 *      (chenxutan.com/d/2993)
 *  [B] "从 ICML 论文到你的显卡：llama.cpp 吞下 DFlash，本地推理进入 2 倍速时代"
 *      (arex-research.com)
 *  [C] "我在llama.cpp中测试了最新合并的DFlash在Qwen 3.6 27B本地AI上的表现…"
 *      (bittide.aicompass.dev)
 *
 * Arithmetic: every dot product and reduction is accumulated in fp64 in the
 * natural index order.  Results are rounded to the storage type (fp32 or bf16)
 * at the points where the path stores a tensor: GEMM outputs, RMSNorm outputs,
 * rotated q/k, the SwiGLU product, the attention output and the residual stream
 * after every add.  LM-head logits are rounded to fp32 (the precision in which
 * the argmax is taken).  OpenMP only splits independent output elements, so the
 * results do not depend on the thread count.
 */
#include "dflash_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* storage types                                                       */
/* ------------------------------------------------------------------ */

static double ld_elem(const void* p, int32_t dtype, int64_t i)
{
    if (dtype == ORC_F32) return (double)((const float*)p)[i];
    /* bfloat16 is the upper half of an IEEE-754 binary32 pattern */
    uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16 value (8 significant bits, the
 * binary32 exponent range), ties to even.  Written from the format: a value
 * m * 2^e with m in [0.5, 1) keeps 8 bits of m. */
double orc_round_bf16(double v)
{
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    double m = frexp(v, &e);           /* v = m * 2^e, |m| in [0.5, 1) */
    if (e < -125) {                    /* below the normal range: fixed quantum 2^-133 */
        double q = ldexp(1.0, -133);
        return nearbyint(v / q) * q;
    }
    double r = nearbyint(ldexp(m, 8)); /* default rounding mode: nearest, ties to even */
    double out = ldexp(r, e - 8);
    /* beyond the largest finite bfloat16 (0x7F7F) the value overflows to infinity */
    if (fabs(out) > 3.3895313892515355e38) return v > 0 ? INFINITY : -INFINITY;
    return out;
}

double orc_round(double v, int32_t dtype)
{
    return dtype == ORC_F32 ? (double)(float)v : orc_round_bf16(v);
}

void orc_round_array_bf16(const double* in, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) {
        float f = (float)orc_round_bf16(in[i]); /* exact: a bf16 value fits in binary32 */
        uint32_t bits;
        memcpy(&bits, &f, sizeof bits);
        out[i] = (uint16_t)(bits >> 16);
    }
}

/* ------------------------------------------------------------------ */
/* building blocks                                                     */
/* ------------------------------------------------------------------ */

/* Five target layers, spaced uniformly from the second layer (index 1) to the
 * third-from-last layer output, rounded half up: index_i = round(1 + i*(L-3)/4).
 * ([A] §2.2 feature-fusion pseudocode: "[2, mid1, mid2, mid3, len-3]"; the tiny
 * workload fixes {1,2,4,5,6} for 8 target layers, which this reproduces.) */
void orc_feature_layers(int32_t L, int32_t out[5])
{
    for (int i = 0; i < 5; ++i) out[i] = (6 + i * (L - 3)) / 4; /* floor(1 + i(L-3)/4 + 1/2) */
}

/* OpenMP threads of the parallel loops (results do not depend on it: only
 * independent outputs are split).  For timing the oracle on fewer cores. */
void orc_set_threads(int32_t n) { if (n > 0) omp_set_num_threads(n); }
int32_t orc_get_threads(void) { return omp_get_max_threads(); }

/* Accumulator precision of dot products: fp64 (the oracle's definition) unless
 * the fp32 variant is selected.  The fp32 variant exists only to measure how far
 * two correct implementations that differ in accumulation precision drift apart
 * once bf16 storage rounding amplifies it (tolerance calibration). */
static int g_fp32_acc = 0;
void orc_set_fp32_accumulation(int32_t on) { g_fp32_acc = on != 0; }

/* y[r][n] = sum_k W[n][k] * x[r][k]  for a row-major W [N][K] in storage type. */
static void matvec_rows(const void* W, int32_t dtype, int64_t N, int64_t K,
                        const double* x, int32_t R, double* y)
{
    #pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)K);
        #pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k) w[k] = ld_elem(W, dtype, n * K + k);
            for (int32_t r = 0; r < R; ++r) {
                const double* xr = x + (int64_t)r * K;
                if (g_fp32_acc) {
                    float s = 0.0f;
                    for (int64_t k = 0; k < K; ++k) s += (float)(w[k] * xr[k]);
                    y[(int64_t)r * N + n] = s;
                } else {
                    double s = 0.0;
                    for (int64_t k = 0; k < K; ++k) s += w[k] * xr[k];
                    y[(int64_t)r * N + n] = s;
                }
            }
        }
        free(w);
    }
}

/* RMSNorm ([A] §2.2: fusion is "rms_norm(linear(concat(...)))"; the same
 * normalisation is the pre-norm of every decoder layer):
 * out = x * g / sqrt(mean(x^2) + eps) */
void orc_rmsnorm(const double* x, int32_t n, const void* gain, int32_t dtype, double eps, double* out)
{
    double ss = 0.0;
    for (int32_t i = 0; i < n; ++i) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int32_t i = 0; i < n; ++i) out[i] = orc_round(x[i] * inv * ld_elem(gain, dtype, i), dtype);
}

/* Rotary position embedding, rotate-half pairing: component i pairs with i+d/2,
 * frequency theta_i = base^(-2i/d), rotation angle pos*theta_i (fp64). */
void orc_rope(double* v, int32_t d, int64_t pos, double base)
{
    int32_t h = d / 2;
    for (int32_t i = 0; i < h; ++i) {
        double theta = pow(base, -2.0 * (double)i / (double)d);
        double ang = (double)pos * theta;
        double c = cos(ang), s = sin(ang);
        double a = v[i], b = v[i + h];
        v[i] = a * c - b * s;
        v[i + h] = a * s + b * c;
    }
}

static double silu(double a) { return a / (1.0 + exp(-a)); }

/* ------------------------------------------------------------------ */
/* context fusion                                                      */
/* ------------------------------------------------------------------ */

/* [A] §2.2 feature fusion / [B] "KV Injection": the hidden states of five target
 * layers are concatenated (layer order ascending) and fused by a Linear layer
 * (no bias) followed by RMSNorm. */
int orc_fuse_rows(const orc_model* m, const void* const* slabs, int64_t ld,
                  const int64_t* rows, int32_t nrows, double* out)
{
    const int32_t H = m->hidden, dt = m->dtype;
    const int64_t K = 5 * (int64_t)H;
    double* x = (double*)malloc(sizeof(double) * (size_t)(nrows * K));
    double* y = (double*)malloc(sizeof(double) * (size_t)nrows * H);
    if (!x || !y) { free(x); free(y); return -1; }
    for (int32_t r = 0; r < nrows; ++r)
        for (int s = 0; s < 5; ++s)
            for (int32_t k = 0; k < H; ++k)
                x[r * K + (int64_t)s * H + k] = ld_elem(slabs[s], dt, rows[r] * ld + k);
    matvec_rows(m->fc, dt, H, K, x, nrows, y);
    for (int64_t i = 0; i < (int64_t)nrows * H; ++i) y[i] = orc_round(y[i], dt);
    for (int32_t r = 0; r < nrows; ++r)
        orc_rmsnorm(y + (int64_t)r * H, H, m->fc_norm, dt, m->eps, out + (int64_t)r * H);
    free(x);
    free(y);
    return 0;
}

/* ------------------------------------------------------------------ */
/* KV injection                                                        */
/* ------------------------------------------------------------------ */

/* [A] §2.2 kv_injection and §5.2: for every draft layer the fused context
 * feature is projected by that layer's K and V projections and appended to the
 * layer's KV cache.  Context row i sits at position pos0 + i; K is rotated. */
int orc_inject_rows(const orc_model* m, const void* fused, int64_t ld,
                    const int64_t* rows, int32_t nrows, int64_t pos0,
                    double* k_out, double* v_out)
{
    const int32_t H = m->hidden, dt = m->dtype, d = m->head_dim, nkv = m->n_kv_heads;
    const int64_t NK = (int64_t)nkv * d;
    double* c = (double*)malloc(sizeof(double) * (size_t)nrows * H);
    if (!c) return -1;
    for (int32_t r = 0; r < nrows; ++r)
        for (int32_t k = 0; k < H; ++k) c[(int64_t)r * H + k] = ld_elem(fused, dt, rows[r] * ld + k);
    for (int32_t l = 0; l < m->n_layers; ++l) {
        double* kl = k_out + (int64_t)l * nrows * NK;
        double* vl = v_out + (int64_t)l * nrows * NK;
        matvec_rows(m->wk[l], dt, NK, H, c, nrows, kl);
        matvec_rows(m->wv[l], dt, NK, H, c, nrows, vl);
        for (int32_t r = 0; r < nrows; ++r) {
            for (int32_t h = 0; h < nkv; ++h)
                orc_rope(kl + (int64_t)r * NK + (int64_t)h * d, d, pos0 + rows[r], m->rope_base);
            for (int64_t i = 0; i < NK; ++i) {
                kl[(int64_t)r * NK + i] = orc_round(kl[(int64_t)r * NK + i], dt);
                vl[(int64_t)r * NK + i] = orc_round(vl[(int64_t)r * NK + i], dt);
            }
        }
    }
    free(c);
    return 0;
}

/* ------------------------------------------------------------------ */
/* decoder layer                                                       */
/* ------------------------------------------------------------------ */

/* Key/value source for attention: a storage-typed array [n][nkv][d] and/or a
 * double array [n][nkv*d]. */
typedef struct {
    const void* st;  int64_t n_st;   /* storage-typed keys (injected context) */
    const double* db; int64_t n_db;  /* double keys (block rows or a dense cache) */
} kv_src;

static double kv_get(const kv_src* s, int32_t dtype, int64_t t, int64_t off, int64_t NK)
{
    if (t < s->n_st) return ld_elem(s->st, dtype, t * NK + off);
    return s->db[(t - s->n_st) * NK + off];
}

/* One pre-norm decoder layer over R rows held in x[R][H] (updated in place).
 * Rows sit at positions pos[r].  Keys visible to row r, among the concatenation
 * [ksrc.st ; ksrc.db]:
 *   causal == 0: all of them;
 *   causal == 1, tree_vis NULL: keys 0 .. causal_base + r;
 *   causal == 1, tree_vis given: keys 0 .. causal_base - 1, and key
 *     causal_base + i (row i's own key) iff tree_vis[r * R + i] != 0.
 * kv_new_k/v receive the rows' own rotated K and V ([R][nkv*d], rounded) and
 * must already be appended at the end of ksrc.db/vsrc.db by the caller's layout:
 * this function fills them first, then attends. */
static void decoder_layer(const orc_model* m, int32_t l, double* x, int32_t R, const int64_t* pos,
                          kv_src* ks, kv_src* vs, double* kv_new_k, double* kv_new_v,
                          int causal, int64_t causal_base, const unsigned char* tree_vis)
{
    const int32_t H = m->hidden, dt = m->dtype, d = m->head_dim;
    const int32_t nq = m->n_q_heads, nkv = m->n_kv_heads, F = m->ffn;
    const int64_t NQ = (int64_t)nq * d, NK = (int64_t)nkv * d;
    double* u = (double*)malloc(sizeof(double) * (size_t)R * H);
    double* q = (double*)malloc(sizeof(double) * (size_t)R * NQ);
    double* o = (double*)malloc(sizeof(double) * (size_t)R * NQ);
    double* t = (double*)malloc(sizeof(double) * (size_t)R * H);
    double* a = (double*)malloc(sizeof(double) * (size_t)R * F);
    double* b = (double*)malloc(sizeof(double) * (size_t)R * F);

    /* attention block */
    for (int32_t r = 0; r < R; ++r) orc_rmsnorm(x + (int64_t)r * H, H, m->attn_norm[l], dt, m->eps, u + (int64_t)r * H);
    matvec_rows(m->wq[l], dt, NQ, H, u, R, q);
    matvec_rows(m->wk[l], dt, NK, H, u, R, kv_new_k);
    matvec_rows(m->wv[l], dt, NK, H, u, R, kv_new_v);
    for (int32_t r = 0; r < R; ++r) {
        for (int32_t h = 0; h < nq; ++h) orc_rope(q + r * NQ + (int64_t)h * d, d, pos[r], m->rope_base);
        for (int32_t h = 0; h < nkv; ++h) orc_rope(kv_new_k + r * NK + (int64_t)h * d, d, pos[r], m->rope_base);
        for (int64_t i = 0; i < NQ; ++i) q[r * NQ + i] = orc_round(q[r * NQ + i], dt);
        for (int64_t i = 0; i < NK; ++i) {
            kv_new_k[r * NK + i] = orc_round(kv_new_k[r * NK + i], dt);
            kv_new_v[r * NK + i] = orc_round(kv_new_v[r * NK + i], dt);
        }
    }
    const int64_t n_keys = ks->n_st + ks->n_db;
    const int32_t group = nq / nkv;
    const double scale = 1.0 / sqrt((double)d);
    #pragma omp parallel
    {
        double* sc = (double*)malloc(sizeof(double) * (size_t)n_keys);
        #pragma omp for schedule(dynamic, 1) collapse(2)
        for (int32_t r = 0; r < R; ++r)
            for (int32_t h = 0; h < nq; ++h) {
                const int32_t g = h / group;            /* grouped-query: kv head of query head h */
                const int64_t nvis = !causal ? n_keys : (tree_vis ? causal_base + R : causal_base + r + 1);
                /* a key hidden by the tree mask takes no part in the softmax */
#define HIDDEN_KEY(j) (tree_vis && (j) >= causal_base && !tree_vis[(int64_t)r * R + ((j) - causal_base)])
                const double* qh = q + r * NQ + (int64_t)h * d;
                double mx = -INFINITY;
                for (int64_t j = 0; j < nvis; ++j) {
                    if (HIDDEN_KEY(j)) continue;
                    double s = 0.0;
                    for (int32_t i = 0; i < d; ++i) s += qh[i] * kv_get(ks, dt, j, (int64_t)g * d + i, NK);
                    sc[j] = s * scale;
                    if (sc[j] > mx) mx = sc[j];
                }
                double den = 0.0;
                for (int64_t j = 0; j < nvis; ++j) {
                    if (HIDDEN_KEY(j)) continue;
                    sc[j] = exp(sc[j] - mx);
                    den += sc[j];
                }
                double* oh = o + r * NQ + (int64_t)h * d;
                /* o_i = sum_j p_j v_{j,i}: every o_i accumulates over keys in index order */
                double acc[256];
                for (int32_t i = 0; i < d; ++i) acc[i] = 0.0;
                for (int64_t j = 0; j < nvis; ++j) {
                    if (HIDDEN_KEY(j)) continue;
                    for (int32_t i = 0; i < d; ++i) acc[i] += sc[j] * kv_get(vs, dt, j, (int64_t)g * d + i, NK);
                }
#undef HIDDEN_KEY
                for (int32_t i = 0; i < d; ++i) oh[i] = orc_round(acc[i] / den, dt);
            }
        free(sc);
    }
    matvec_rows(m->wo[l], dt, H, NQ, o, R, t);
    for (int64_t i = 0; i < (int64_t)R * H; ++i) x[i] = orc_round(x[i] + orc_round(t[i], dt), dt);

    /* SwiGLU MLP block */
    for (int32_t r = 0; r < R; ++r) orc_rmsnorm(x + (int64_t)r * H, H, m->mlp_norm[l], dt, m->eps, u + (int64_t)r * H);
    matvec_rows(m->wg[l], dt, F, H, u, R, a);
    matvec_rows(m->wu[l], dt, F, H, u, R, b);
    for (int64_t i = 0; i < (int64_t)R * F; ++i) a[i] = orc_round(silu(a[i]) * b[i], dt);
    matvec_rows(m->wd[l], dt, H, F, a, R, t);
    for (int64_t i = 0; i < (int64_t)R * H; ++i) x[i] = orc_round(x[i] + orc_round(t[i], dt), dt);

    free(u); free(q); free(o); free(t); free(a); free(b);
}

/* Final RMSNorm, LM head (shared with the target, [A] §3.3), logits rounded to
 * fp32, argmax with ties to the lowest index and the top-2 gap. */
static void lm_head_argmax(const orc_model* m, const double* x, int32_t R,
                           float* logits, int32_t* tokens, double* gap)
{
    const int32_t H = m->hidden, V = m->vocab, dt = m->dtype;
    double* z = (double*)malloc(sizeof(double) * (size_t)R * H);
    double* lg = (double*)malloc(sizeof(double) * (size_t)R * V);
    for (int32_t r = 0; r < R; ++r) orc_rmsnorm(x + (int64_t)r * H, H, m->final_norm, dt, m->eps, z + (int64_t)r * H);
    matvec_rows(m->lm_head, dt, V, H, z, R, lg);
    for (int32_t r = 0; r < R; ++r) {
        float best = -INFINITY, second = -INFINITY;
        int32_t arg = 0;
        for (int32_t v = 0; v < V; ++v) {
            float f = (float)lg[(int64_t)r * V + v];
            if (logits) logits[(int64_t)r * V + v] = f;
            if (f > best) { second = best; best = f; arg = v; }
            else if (f > second) second = f;
        }
        tokens[r] = arg;
        if (gap) gap[r] = (double)best - (double)second;
    }
    free(z);
    free(lg);
}

/* ------------------------------------------------------------------ */
/* the draft block                                                     */
/* ------------------------------------------------------------------ */

/* One block-diffusion draft forward ([A] §2.2 draft_inference, §5.1; [B]
 * "技术内幕"; [C]: one pass fills the block): rows are the anchor token
 * followed by B-1 mask tokens at positions C..C+B-1, embedded with the
 * target's shared embedding ([A] §3.3).  In every layer each row attends,
 * without any mask (bidirectional inside the block), to all injected context
 * keys of that layer and to all B block keys; then LM head and argmax.  Row j
 * (j >= 1) is the draft for the token at position C + j. */
int orc_draft_block(const orc_model* m, const void* const* ctx_k, const void* const* ctx_v,
                    int64_t C, int32_t anchor, float* logits, int32_t* tokens, double* gap,
                    double* trace)
{
    const int32_t H = m->hidden, B = m->block, dt = m->dtype;
    const int64_t NK = (int64_t)m->n_kv_heads * m->head_dim;
    if (m->head_dim > 256) return -1;
    double* x = (double*)malloc(sizeof(double) * (size_t)B * H);
    double* kb = (double*)malloc(sizeof(double) * (size_t)B * NK);
    double* vb = (double*)malloc(sizeof(double) * (size_t)B * NK);
    int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)B);
    if (!x || !kb || !vb || !pos) return -1;
    for (int32_t j = 0; j < B; ++j) {
        int32_t tok = j == 0 ? anchor : m->mask_id;
        for (int32_t k = 0; k < H; ++k) x[(int64_t)j * H + k] = ld_elem(m->embed, dt, (int64_t)tok * H + k);
        pos[j] = C + j;
    }
    if (trace) memcpy(trace, x, sizeof(double) * (size_t)B * H);
    for (int32_t l = 0; l < m->n_layers; ++l) {
        kv_src ks = { ctx_k ? ctx_k[l] : NULL, C, kb, B };
        kv_src vs = { ctx_v ? ctx_v[l] : NULL, C, vb, B };
        decoder_layer(m, l, x, B, pos, &ks, &vs, kb, vb, 0, 0, NULL);
        if (trace) memcpy(trace + (int64_t)(l + 1) * B * H, x, sizeof(double) * (size_t)B * H);
    }
    lm_head_argmax(m, x, B, logits, tokens, gap);
    free(x); free(kb); free(vb); free(pos);
    return 0;
}

/* The same draft layer on its own: layer l over block rows x_in[B][H]
 * (storage values) at positions C..C+B-1, attending without a mask to the C
 * injected context keys of that layer (ctx_k, ctx_v: [C][nkv][d] storage) and
 * to the block's own keys ([A] §2.2 draft_inference; one repetition of the
 * per-layer step of orc_draft_block).  x_out[B][H] receives the residual
 * stream after the layer.  Used to compare a layer given identical inputs. */
int orc_draft_layer(const orc_model* m, int32_t l, const void* ctx_k, const void* ctx_v, int64_t C,
                    const double* x_in, double* x_out)
{
    const int32_t H = m->hidden, B = m->block;
    const int64_t NK = (int64_t)m->n_kv_heads * m->head_dim;
    if (m->head_dim > 256 || l < 0 || l >= m->n_layers) return -1;
    double* kb = (double*)malloc(sizeof(double) * (size_t)B * NK);
    double* vb = (double*)malloc(sizeof(double) * (size_t)B * NK);
    int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)B);
    if (!kb || !vb || !pos) { free(kb); free(vb); free(pos); return -1; }
    memcpy(x_out, x_in, sizeof(double) * (size_t)B * H);
    for (int32_t j = 0; j < B; ++j) pos[j] = C + j;
    kv_src ks = { C > 0 ? ctx_k : NULL, C, kb, B };
    kv_src vs = { C > 0 ? ctx_v : NULL, C, vb, B };
    decoder_layer(m, l, x_out, B, pos, &ks, &vs, kb, vb, 0, 0, NULL);
    free(kb); free(vb); free(pos);
    return 0;
}

/* The draft's output head on its own: final RMSNorm, shared LM head ([A]
 * §3.3), fp32 logits, argmax (ties: lowest id) and top-2 gap of R rows x[R][H]
 * (storage values). */
int orc_lm_head(const orc_model* m, const double* x, int32_t R, float* logits, int32_t* tokens, double* gap)
{
    if (R < 1) return -1;
    lm_head_argmax(m, x, R, logits, tokens, gap);
    return 0;
}

/* ------------------------------------------------------------------ */
/* greedy verification                                                 */
/* ------------------------------------------------------------------ */

/* [B] "技术内幕" and [A] §1.2 / §8.2 linear verification: drafts are accepted
 * while they equal the target's greedy token at the same position; the first
 * mismatch truncates the block and the target's own token there is emitted.
 * g[j] is the target's prediction for position C+j+1, d[j] the draft for C+j. */
void orc_accept(const int32_t* d, const int32_t* g, int32_t B, int32_t* k, int32_t* bonus)
{
    int32_t n = 0;
    while (n < B - 1 && d[n + 1] == g[n]) ++n;
    *k = n;
    *bonus = g[n];
}

/* ------------------------------------------------------------------ */
/* causal target (toy end-to-end loop)                                 */
/* ------------------------------------------------------------------ */

/* Shared body of the causal and tree forwards: rows at positions pos[j], their
 * K/V stored at cache slots pos0 + j, visibility as in decoder_layer. */
static int target_rows(const orc_model* m, const int32_t* tokens, int32_t n, int64_t pos0, const int64_t* pos,
                       const unsigned char* tree_vis, double* cache_k, double* cache_v, int64_t cap,
                       const int32_t* capture, double* hidden_out,
                       float* logits_out, int32_t* argmax_out, double* gap_out)
{
    const int32_t H = m->hidden, dt = m->dtype;
    const int64_t NK = (int64_t)m->n_kv_heads * m->head_dim;
    double* x = (double*)malloc(sizeof(double) * (size_t)n * H);
    if (!x) return -1;
    for (int32_t j = 0; j < n; ++j)
        for (int32_t k = 0; k < H; ++k) x[(int64_t)j * H + k] = ld_elem(m->embed, dt, (int64_t)tokens[j] * H + k);
    for (int32_t l = 0; l < m->n_layers; ++l) {
        double* ck = cache_k + (int64_t)l * cap * NK;
        double* cv = cache_v + (int64_t)l * cap * NK;
        kv_src ks = { NULL, 0, ck, pos0 + n };
        kv_src vs = { NULL, 0, cv, pos0 + n };
        decoder_layer(m, l, x, n, pos, &ks, &vs, ck + pos0 * NK, cv + pos0 * NK, 1, pos0, tree_vis);
        if (capture && hidden_out)
            for (int s = 0; s < 5; ++s)
                if (capture[s] == l)
                    memcpy(hidden_out + (int64_t)s * n * H, x, sizeof(double) * (size_t)n * H);
    }
    lm_head_argmax(m, x, n, logits_out, argmax_out, gap_out);
    free(x);
    return 0;
}

/* Plain greedy autoregressive model forward ([A] §1.1): causal pre-norm
 * decoder with a dense KV cache; every row's argmax is reported. */
int orc_target_forward(const orc_model* m, const int32_t* tokens, int32_t n, int64_t pos0,
                       double* cache_k, double* cache_v, int64_t cap,
                       const int32_t* capture, double* hidden_out,
                       float* logits_out, int32_t* argmax_out, double* gap_out)
{
    if (pos0 + n > cap || m->head_dim > 256) return -1;
    int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
    if (!pos) return -1;
    for (int32_t j = 0; j < n; ++j) pos[j] = pos0 + j;
    const int rc = target_rows(m, tokens, n, pos0, pos, NULL, cache_k, cache_v, cap, capture, hidden_out,
                               logits_out, argmax_out, gap_out);
    free(pos);
    return rc;
}

/* Tree verification ([A] §8.2, DDTree: several branches checked in one target
 * pass).  Row 0 is the root (parent[0] = -1); row j >= 1 has parent[j] in
 * [0, j).  A row sits at position pos0 + depth(j) (its number of ancestors),
 * its K/V go to cache slot pos0 + j, and it attends to the cache before pos0
 * and to the slots of its ancestors and itself.  Every row therefore computes
 * what a causal forward over its root-to-row path would compute.  -1 when the
 * parent array is not such a tree. */
/* Positions and visibility of tree rows: pos[j] = pos0 + depth(j), vis[j][u]
 * = 1 for u an ancestor of j or j itself.  -1 when parent is not a tree in
 * node order (parent[0] = -1, 0 <= parent[j] < j). */
static int tree_layout(const int32_t* parent, int32_t n, int64_t pos0, int64_t* pos, unsigned char* vis)
{
    if (n < 1 || parent[0] != -1) return -1;
    for (int32_t j = 1; j < n; ++j)
        if (parent[j] < 0 || parent[j] >= j) return -1;
    memset(vis, 0, (size_t)n * n);
    for (int32_t j = 0; j < n; ++j) {
        int64_t depth = 0;
        for (int32_t u = j; u >= 0; u = parent[u]) {  /* walk up to the root */
            vis[(int64_t)j * n + u] = 1;
            if (u != j) ++depth;
        }
        pos[j] = pos0 + depth;
    }
    return 0;
}

int orc_target_forward_tree(const orc_model* m, const int32_t* tokens, const int32_t* parent, int32_t n,
                            int64_t pos0, double* cache_k, double* cache_v, int64_t cap,
                            const int32_t* capture, double* hidden_out,
                            float* logits_out, int32_t* argmax_out, double* gap_out)
{
    if (n < 1 || pos0 + n > cap || m->head_dim > 256) return -1;
    int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
    unsigned char* vis = (unsigned char*)malloc((size_t)n * n);
    int rc = -1;
    if (pos && vis && tree_layout(parent, n, pos0, pos, vis) == 0)
        rc = target_rows(m, tokens, n, pos0, pos, vis, cache_k, cache_v, cap, capture, hidden_out,
                         logits_out, argmax_out, gap_out);
    free(pos); free(vis);
    return rc;
}

/* One layer of the causal (parent NULL) or tree forward on its own: rows
 * x_in[n][H] (storage values, e.g. another implementation's input to layer
 * l) at pos0, with layer l's dense cache cache_k/v [cap][nkv*d] holding the
 * keys before pos0; the rows' K/V are written at pos0.. as in the full
 * forward.  x_out[n][H] receives the residual stream after the layer. */
int orc_target_layer(const orc_model* m, int32_t l, const double* x_in, int32_t n, int64_t pos0,
                     const int32_t* parent, double* cache_k, double* cache_v, int64_t cap, double* x_out)
{
    const int64_t NK = (int64_t)m->n_kv_heads * m->head_dim;
    if (n < 1 || pos0 + n > cap || m->head_dim > 256 || l < 0 || l >= m->n_layers) return -1;
    int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
    unsigned char* vis = parent ? (unsigned char*)malloc((size_t)n * n) : NULL;
    if (!pos || (parent && (!vis || tree_layout(parent, n, pos0, pos, vis) != 0))) {
        free(pos); free(vis);
        return -1;
    }
    if (!parent)
        for (int32_t j = 0; j < n; ++j) pos[j] = pos0 + j;
    memcpy(x_out, x_in, sizeof(double) * (size_t)n * m->hidden);
    kv_src ks = { NULL, 0, cache_k, pos0 + n };
    kv_src vs = { NULL, 0, cache_v, pos0 + n };
    decoder_layer(m, l, x_out, n, pos, &ks, &vs, cache_k + pos0 * NK, cache_v + pos0 * NK, 1, pos0, vis);
    free(pos); free(vis);
    return 0;
}

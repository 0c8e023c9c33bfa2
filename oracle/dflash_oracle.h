/*
 * dflash_oracle.h -- plain CPU oracle for the DFlash draft path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this; only the tests, the smoke entry and the bench's CPU-baseline leg do.
 * It shares no code, header, table or constant generator with the HIP library.
 *
 * Every function computes the plain definition of one step of the method in
 * fp64, rounding to the workload's storage type (fp32 or bf16) exactly where the
 * stored tensors of the path are rounded.  Inputs are raw storage arrays
 * (float for fp32, uint16 bit patterns for bf16).
 */
#ifndef DFLASH_ORACLE_H
#define DFLASH_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_MAX_LAYERS 64
#define ORC_F32 0
#define ORC_BF16 1

typedef struct {
    int32_t dtype;          /* ORC_F32 or ORC_BF16 storage */
    int32_t hidden;         /* H */
    int32_t n_layers;       /* decoder layers of this model */
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t ffn;
    int32_t vocab;
    int32_t block;          /* draft block length B (<= 16) */
    int32_t mask_id;
    double rope_base;
    double eps;
    const void* fc;         /* [H, 5H] fusion weight */
    const void* fc_norm;    /* [H] fusion RMSNorm gain */
    const void* attn_norm[ORC_MAX_LAYERS];
    const void* wq[ORC_MAX_LAYERS];   /* [nq*d, H] */
    const void* wk[ORC_MAX_LAYERS];   /* [nkv*d, H] */
    const void* wv[ORC_MAX_LAYERS];   /* [nkv*d, H] */
    const void* wo[ORC_MAX_LAYERS];   /* [H, nq*d] */
    const void* mlp_norm[ORC_MAX_LAYERS];
    const void* wg[ORC_MAX_LAYERS];   /* [F, H] */
    const void* wu[ORC_MAX_LAYERS];   /* [F, H] */
    const void* wd[ORC_MAX_LAYERS];   /* [H, F] */
    const void* final_norm; /* [H] */
    const void* embed;      /* [V, H] */
    const void* lm_head;    /* [V, H] */
} orc_model;

/* Select fp32 accumulation of the Linear layers' dot products (default fp64).
 * Used only to measure the rounding noise between correct implementations. */
void orc_set_fp32_accumulation(int32_t on);

/* OpenMP threads of the oracle's parallel loops (results are thread-count independent) */
void orc_set_threads(int32_t n);
int32_t orc_get_threads(void);

/* storage rounding */
double orc_round_bf16(double v);
double orc_round(double v, int32_t dtype);
void orc_round_array_bf16(const double* in, int64_t n, uint16_t* out);

/* which 5 target layers feed the fusion */
void orc_feature_layers(int32_t target_layers, int32_t out[5]);

/* RMSNorm of one row (x already in storage precision); out rounded to storage */
void orc_rmsnorm(const double* x, int32_t n, const void* gain, int32_t dtype, double eps, double* out);

/* rotary embedding of one head vector (rotate-half pairing) at integer position */
void orc_rope(double* v, int32_t d, int64_t pos, double base);

/* context fusion of selected rows: out[r][H] = RMSNorm(W_fc . concat(slabs[0..4][row])) */
int orc_fuse_rows(const orc_model* m, const void* const* slabs, int64_t ld,
                  const int64_t* rows, int32_t nrows, double* out);

/* KV injection of selected rows of fused context at positions pos0 + row:
 * k_out, v_out: [n_layers][nrows][nkv*d] (rounded to storage; k rotated) */
int orc_inject_rows(const orc_model* m, const void* fused, int64_t ld,
                    const int64_t* rows, int32_t nrows, int64_t pos0,
                    double* k_out, double* v_out);

/* one draft block over context K/V (ctx_k[l], ctx_v[l]: [C][nkv][d] storage):
 * logits [B][V] (fp32 values, may be NULL), tokens [B], gap [B] top-2 gap (may be NULL),
 * trace [(L+1)][B][H] residual stream after the embedding and each layer (may be NULL) */
int orc_draft_block(const orc_model* m, const void* const* ctx_k, const void* const* ctx_v,
                    int64_t C, int32_t anchor, float* logits, int32_t* tokens, double* gap,
                    double* trace);

/* one draft layer l alone: x_out[B][H] = layer l of the block rows x_in[B][H] at
 * positions C.., over the C context keys ctx_k/ctx_v ([C][nkv][d] storage) and
 * the block's own keys (no mask) */
int orc_draft_layer(const orc_model* m, int32_t l, const void* ctx_k, const void* ctx_v, int64_t C,
                    const double* x_in, double* x_out);

/* final RMSNorm + LM head + argmax of R rows x[R][H]: logits [R][V] fp32 (may be
 * NULL), tokens [R], gap [R] top-2 gap (may be NULL) */
int orc_lm_head(const orc_model* m, const double* x, int32_t R, float* logits, int32_t* tokens, double* gap);

/* greedy block verification: d[1..B-1] drafts, g[0..B-1] target argmax */
void orc_accept(const int32_t* d, const int32_t* g, int32_t B, int32_t* k, int32_t* bonus);

/* Causal (target) forward of n tokens at positions pos0.. with a dense KV cache
 * cache_k/cache_v: [n_layers][cap][nkv*d] doubles holding positions 0..pos0-1 on
 * entry and 0..pos0+n-1 on return.  capture: 5 layer ids (0-based) whose output
 * rows go to hidden_out [5][n][H] (may be NULL).  logits_out [n][V] fp32 (may be
 * NULL), argmax_out [n], gap_out [n]. */
int orc_target_forward(const orc_model* m, const int32_t* tokens, int32_t n, int64_t pos0,
                       double* cache_k, double* cache_v, int64_t cap,
                       const int32_t* capture, double* hidden_out,
                       float* logits_out, int32_t* argmax_out, double* gap_out);
int orc_target_forward_tree(const orc_model* m, const int32_t* tokens, const int32_t* parent, int32_t n,
                            int64_t pos0, double* cache_k, double* cache_v, int64_t cap,
                            const int32_t* capture, double* hidden_out,
                            float* logits_out, int32_t* argmax_out, double* gap_out);
int orc_target_layer(const orc_model* m, int32_t l, const double* x_in, int32_t n, int64_t pos0,
                     const int32_t* parent, double* cache_k, double* cache_v, int64_t cap, double* x_out);

#ifdef __cplusplus
}
#endif
#endif

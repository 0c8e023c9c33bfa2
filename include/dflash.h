/*
 * dflash.h -- C ABI of libdflash: the DFlash single-pass block-diffusion draft
 * with KV injection and greedy block verification, on one AMD MI355X (gfx950).
 *
 * Method sources (web pages):
 *  [A] "DFlash 深度解析：块扩散模型如何让 LLM 推理加速 6 倍——2026 投机解码完全指南"
 *      (chenxutan.com/d/2993): §2.2 feature fusion, KV injection, block draft;
 *      §3.3 shared embedding and LM head; §5.1-5.2; §8.2 linear verification.
 *  [B] "从 ICML 论文到你的显卡：llama.cpp 吞下 DFlash，本地推理进入 2 倍速时代"
 *      (arex-research.com), section 技术内幕: accept up to the first error;
 *      injected K/V live in the draft's KV cache of every layer.
 *  [C] "我在llama.cpp中测试了最新合并的DFlash在Qwen 3.6 27B本地AI上的表现…"
 *      (bittide.aicompass.dev): one pass fills a 15-token block; greedy is lossless.
 *
 * Conventions shared by every call:
 *  - Status: every call returns a dflash_status; 0 is success, negative values
 *    are errors.  On an error nothing is enqueued and the context is unchanged;
 *    dflash_last_error() gives a message.  No call aborts or throws.
 *  - Pointers: "device" pointers are HIP device memory on the context's GPU;
 *    "host" pointers are ordinary host memory.  The caller owns every buffer;
 *    the library borrows them until the work enqueued on `stream` completes.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).  Device work is asynchronous on it; argument checks are host-side
 *    and synchronous.  One context must not be used from two streams at once.
 *  - Layouts: matrices are row-major [out_features, in_features]; activations
 *    are row-major [rows, features] with a row stride `ld` in elements.
 *  - Element type: every floating-point tensor a context touches has the
 *    context's dtype (fp32 or bf16), except logits (always fp32).
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_MAX_LAYERS 64
#define DFLASH_NUM_FEATURES 5
#define DFLASH_MAX_BLOCK 16
#define DFLASH_TREE_MAX_K 16   /* candidates per depth of a verification tree */
#define DFLASH_TREE_MAX_NODES 32  /* nodes of a verification tree, root included */
#define DFLASH_TREE_RESULT 17  /* int32 entries of a tree acceptance result */

typedef enum {
    DFLASH_OK = 0,
    DFLASH_ERR_INVAL = -1,       /* bad argument, shape or pointer */
    DFLASH_ERR_CAPACITY = -2,    /* would exceed max_ctx / max_rows / workspace */
    DFLASH_ERR_HIP = -3,         /* a HIP runtime call failed (message has the HIP string) */
    DFLASH_ERR_UNSUPPORTED = -4, /* shape or dtype outside what the kernels handle */
    DFLASH_ERR_STATE = -5        /* call out of order (e.g. inject at pos0 != length) */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Model and capacity description.  All fields are required. */
typedef struct {
    int32_t dtype;          /* dflash_dtype */
    int32_t hidden;         /* H: target and draft hidden size (multiple of 32) */
    int32_t target_layers;  /* target decoder layers (>= 8); 5 of them feed the fusion */
    int32_t draft_layers;   /* Ld, 1..DFLASH_MAX_LAYERS */
    int32_t n_q_heads;      /* nq, multiple of n_kv_heads, at most 8 per kv head */
    int32_t n_kv_heads;     /* nkv */
    int32_t head_dim;       /* d: 64 or 128 */
    int32_t ffn;            /* F: SwiGLU width (multiple of 16) */
    int32_t vocab;          /* V: shared vocabulary (multiple of 16) */
    int32_t block;          /* B: draft block length, 2..16 (1 anchor + B-1 masks) */
    int32_t mask_id;        /* token id of the mask token, 0 <= mask_id < V */
    int32_t page_size;      /* tokens per KV page: 256 (multiple of 64) */
    int32_t max_ctx;        /* capacity of the draft KV cache in tokens */
    int32_t max_rows;       /* largest M accepted by fuse/inject in one call */
    double rope_base;       /* rotary base theta (e.g. 10000) */
    double eps;             /* RMSNorm epsilon (e.g. 1e-6) */
    uint64_t page_seed;     /* 0: identity page table; else a seeded shuffle of physical pages */
} dflash_config;

/* Device pointers to the weights (borrowed for the context's lifetime).
 * Unused entries may be NULL: a context used only for fuse/inject needs
 * fc, fc_norm, wk and wv; the draft additionally needs the rest.  A context
 * used only as a causal model (dflash_target_forward) may leave fc and fc_norm
 * NULL; dflash_fuse_context then fails with STATE. */
typedef struct {
    const void* fc;          /* [H, 5H] context fusion Linear (no bias) */
    const void* fc_norm;     /* [H] RMSNorm gain after the fusion */
    const void* attn_norm[DFLASH_MAX_LAYERS]; /* [H] pre-attention RMSNorm gain */
    const void* wq[DFLASH_MAX_LAYERS];        /* [nq*d, H] */
    const void* wk[DFLASH_MAX_LAYERS];        /* [nkv*d, H]: block keys AND injected context keys */
    const void* wv[DFLASH_MAX_LAYERS];        /* [nkv*d, H]: block values AND injected values */
    const void* wo[DFLASH_MAX_LAYERS];        /* [H, nq*d] */
    const void* mlp_norm[DFLASH_MAX_LAYERS];  /* [H] pre-MLP RMSNorm gain */
    const void* wg[DFLASH_MAX_LAYERS];        /* [F, H] SwiGLU gate */
    const void* wu[DFLASH_MAX_LAYERS];        /* [F, H] SwiGLU up */
    const void* wd[DFLASH_MAX_LAYERS];        /* [H, F] down */
    const void* final_norm;  /* [H] */
    const void* embed;       /* [V, H] shared with the target ([A] §3.3) */
    const void* lm_head;     /* [V, H] shared with the target ([A] §3.3) */
} dflash_weights;

typedef struct dflash_ctx dflash_ctx;

/* Human-readable name of a status code (static string). */
const char* dflash_status_str(int status);

/* Message of the last failed call on ctx (static empty string if none / ctx NULL). */
const char* dflash_last_error(const dflash_ctx* ctx);

/* The five target layers (0-based decoder-layer outputs, ascending) whose
 * hidden states feed the fusion: spaced uniformly from the second layer to the
 * third-from-last output, rounded half up ([A] §2.2 feature-fusion
 * pseudocode).  out: host int32[5].  INVAL if target_layers < 8. */
dflash_status dflash_feature_layers(int32_t target_layers, int32_t* out);

/* Physical page of each logical page of the draft KV cache (introspection of the
 * cache layout; pure host computation).  out: host int32[n], n >= number of
 * pages = ceil(max_ctx / page_size).  Each (layer, K|V) page array holds pages
 * of page_size positions: K pages are [nkv][page_size][d], V pages
 * [nkv][d][page_size]; the KV pool is [Ld][K,V][pages]. */
dflash_status dflash_page_table(const dflash_config* cfg, int32_t* out, int32_t n);

/* Device memory the caller must provide to dflash_create: `workspace_bytes` of
 * scratch (activations, partial sums, rotary table, page table, counters) and
 * `kv_bytes` for the paged draft KV cache.  Pure host computation; INVAL or
 * UNSUPPORTED if the config is not valid. */
dflash_status dflash_workspace_size(const dflash_config* cfg, size_t* workspace_bytes, size_t* kv_bytes);

/* Create a context.  `workspace` and `kv_pool` are device buffers of at least
 * the sizes above (256-byte aligned); they and the weights stay borrowed until
 * dflash_destroy.  The library never allocates device memory itself.  Fills the
 * rotary table (fp64 angles, fp32 cos/sin) and the page table, zeroes the
 * counters and writes a copy of every streamed weight matrix into the
 * workspace in the matrix-core operand order (so the weights must not change
 * while the context lives), enqueued on `stream`.  Length starts at 0. */
dflash_status dflash_create(const dflash_config* cfg, const dflash_weights* w,
                            void* workspace, size_t workspace_bytes,
                            void* kv_pool, size_t kv_bytes,
                            void* stream, dflash_ctx** out);

/* Destroy a context (host state only; the caller frees its buffers). NULL is a no-op. */
dflash_status dflash_destroy(dflash_ctx* ctx);

/* Current draft-KV length: number of context positions injected and kept. */
int32_t dflash_length(const dflash_ctx* ctx);

/* Context fusion ([A] §2.2 feature fusion; [B] KV Injection):
 *   fused[i] = RMSNorm_fc( W_fc . concat(h_{s0}[i], ..., h_{s4}[i]) ),  i < M
 * where s0..s4 = dflash_feature_layers(target_layers).
 * layer_hidden: host array of target_layers device pointers; entry l points at
 *   target layer l's hidden states [M, H] with row stride ld (elements).  Only
 *   the five selected entries are read; the others may be NULL.
 * fused_out: device [M, H], row stride H.  1 <= M <= max_rows. */
dflash_status dflash_fuse_context(dflash_ctx* ctx, const void* const* layer_hidden, int64_t ld,
                                  int32_t M, void* fused_out, void* stream);

/* dflash_fuse_context for M <= 16 rows (the per-step fusion of the verified
 * rows) that allocates nothing and uses no context scratch: for callers that
 * cannot allocate device memory or change its layout per call (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  The
 * stream-K partial sums and tile counters live in a static array of
 * 8 MiB + 16 KiB per GPU inside the library (held until the process ends;
 * its address is looked up by dflash_create).  Arguments and results are those
 * of dflash_fuse_context, bit for bit.  CAPACITY if M > 16, UNSUPPORTED if the
 * context's hidden size needs more than 4096 32-column tiles.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (two streams,
 * two contexts) race; serialise them. */
dflash_status dflash_fuse_context_static(dflash_ctx* ctx, const void* const* layer_hidden, int64_t ld,
                                         int32_t M, void* fused_out, void* stream);

/* KV injection ([A] §2.2 kv_injection, §5.2; [B] KV Injection): for every draft
 * layer l and row i < M,
 *   K_l[pos0+i] = RoPE(W_k^l . fused[i], pos0+i),  V_l[pos0+i] = W_v^l . fused[i]
 * written into the paged draft KV cache.  fused: device [M, H], row stride ld.
 * Requires pos0 == dflash_length(ctx) (STATE otherwise) and pos0 + M <= max_ctx
 * (CAPACITY otherwise; nothing written).  Afterwards length = pos0 + M. */
dflash_status dflash_inject_kv(dflash_ctx* ctx, const void* fused, int64_t ld,
                               int32_t M, int32_t pos0, void* stream);

/* One block-diffusion draft pass ([A] §2.2 draft_inference, §5.1; [B] 技术内幕; [C]):
 * rows [anchor, mask x (B-1)] at positions C..C+B-1 (C = current length) are
 * embedded with the shared embedding, run through every draft layer attending
 * without a mask to all C injected context keys and all B block keys, then the
 * final RMSNorm, the shared LM head and a per-row argmax (ties: lowest id).
 * anchor: device int32[1] (an id outside [0, V) is clamped into it).  tokens_out: device int32[B]; entry j >= 1 is the
 * draft for position C+j (entry 0 is the anchor row's own argmax, unused by
 * verification).  logits_out: device fp32 [B, V] or NULL.
 * Requires all draft weights; INVAL otherwise.  Context is not modified. */
dflash_status dflash_draft_block(dflash_ctx* ctx, const int32_t* anchor, float* logits_out,
                                 int32_t* tokens_out, void* stream);

/* dflash_draft_block, and in the same launches the residual stream after every
 * draft layer: layer_out (device, [Ld][B][layer_ld] in the context dtype, or
 * NULL) receives row j of layer l's output at layer_out[(l*B + j)*layer_ld].
 * An inspection aid: a caller (a test) can feed layer l's input to another
 * implementation of that one layer.  layer_ld >= H and keeps rows aligned to
 * the element size (INVAL otherwise); tokens and logits are those of
 * dflash_draft_block. */
dflash_status dflash_draft_block_ex(dflash_ctx* ctx, const int32_t* anchor, float* logits_out,
                                    int32_t* tokens_out, void* layer_out, int64_t layer_ld, void* stream);

/* Greedy block verification ([B] 技术内幕; [A] §1.2, §8.2 linear verification):
 *   k = number of leading j in 1..B-1 with draft[j] == target[j-1],  bonus = target[k].
 * draft: device int32[B] (as written by dflash_draft_block); target: device
 * int32[B], target[j] = the target's greedy token for position C+j+1.
 * result_out: device int32[2] = {k, bonus}.  The emitted tokens are
 * draft[1..k] followed by bonus. */
dflash_status dflash_verify_accept(dflash_ctx* ctx, const int32_t* draft, const int32_t* target,
                                   int32_t* result_out, void* stream);

/* Roll the draft KV cache back to new_len tokens (0 <= new_len <= length, INVAL
 * otherwise): after injecting the B verified rows of a step at C, the caller
 * rolls back to C + k + 1 so only the anchor and the accepted drafts remain
 * as context.  Host metadata only: positions from new_len on stop being
 * context and are overwritten by the next injection.  The page table is fixed
 * at creation (logical page i always maps to the same physical page), so no
 * page is released or reassigned. */
dflash_status dflash_rollback(dflash_ctx* ctx, int32_t new_len);

/* Device-resident length: a speculative step without a host round trip
 * ([B] 技术内幕: keep the anchor and the accepted drafts; the next step drafts
 * from there).  After dflash_device_length_enable the context's length lives
 * in a device word (initialised from the host length) for the rest of the
 * context's life, so a whole step -- draft, verification, fusion, injection,
 * keeping the accepted rows -- is stream-ordered device work that can be
 * captured in a HIP graph and replayed:
 *  - dflash_draft_block reads the length from the device word; its attention
 *    is planned for max_ctx (the splits past the length stay empty);
 *  - dflash_inject_kv takes pos0 = -1 and M <= 16 and writes the rows at the
 *    device length without changing it; rows that would pass max_ctx are not
 *    written and the capacity-error word is set instead;
 *  - dflash_keep_accepted adds k + 1 from a dflash_verify_accept result
 *    {k, bonus} (device int32[2]): the anchor and the k accepted drafts of the
 *    rows just injected stay context (k is clamped to [0, 15], the length to
 *    max_ctx);
 *  - dflash_set_length_async sets the length (0 <= new_len <= max_ctx);
 *  - dflash_read_device_length copies {length, capacity-error} to a device
 *    int32[2];
 *  - dflash_rollback, dflash_target_forward and dflash_load_kv return STATE;
 *    dflash_length returns -1; dflash_read_kv checks ranges against max_ctx.
 * STATE if enabled twice, or if the other calls are used without it. */
dflash_status dflash_device_length_enable(dflash_ctx* ctx, void* stream);
dflash_status dflash_keep_accepted(dflash_ctx* ctx, const int32_t* result, void* stream);
dflash_status dflash_set_length_async(dflash_ctx* ctx, int32_t new_len, void* stream);
dflash_status dflash_read_device_length(dflash_ctx* ctx, int32_t* out, void* stream);

/* Causal forward of the context's decoder stack used as the target (verifier)
 * model ([A] §1.1 autoregressive generation, §1.2 parallel verification of a
 * drafted block; [C] greedy verification is lossless): rows tokens[0..M-1] at
 * positions C..C+M-1 (C = current length) are embedded, and in every layer
 * their rotated K and V are appended to the context's paged KV cache before row
 * j attends to keys 0..C+j (causal).  Then the final RMSNorm, the LM head and
 * a per-row argmax (ties: lowest id).  Afterwards length = C + M; a caller
 * that accepts only a prefix rolls back with dflash_rollback.
 * Batch invariant: row j's results are bit-identical whatever M and whatever
 * rows share the call (attention splits sit at fixed key positions; every
 * reduction has a fixed order), so verifying a block of M rows gives exactly
 * the tokens of M one-row calls.
 * tokens: device int32[M], 1 <= M <= 16 (ids outside [0, V) are clamped).
 * argmax_out: device int32[M], argmax_out[j] = greedy token for position C+j+1.
 * logits_out: device fp32 [M, V] or NULL.
 * capture: NULL, or a host array of DFLASH_NUM_FEATURES device pointers (entries
 *   may be NULL); entry i receives the output rows of target layer
 *   dflash_feature_layers(target_layers)[i] (the residual stream after that
 *   layer), [M, H] with row stride capture_ld elements: the hidden states that
 *   dflash_fuse_context of a draft context takes.  A non-NULL entry whose layer
 *   is not below draft_layers (the depth of this context's stack) is INVAL.
 * Requires every layer's weights, final_norm, embed and lm_head (INVAL), and
 * C + M <= max_ctx (CAPACITY; nothing written). */
dflash_status dflash_target_forward(dflash_ctx* ctx, const int32_t* tokens, int32_t M,
                                    float* logits_out, int32_t* argmax_out,
                                    void* const* capture, int64_t capture_ld, void* stream);

/* ---- Tree verification (DDTree) ------------------------------------------
 * [A] §8.2 (DDTree tree verification): instead of one chain of drafts, one
 * target pass checks a tree of candidates under a node budget, so a rejected
 * draft at one depth can still be followed by another branch.  The passage
 * names the idea and the budget, not the construction; the readings taken:
 *  - depth d of the tree holds candidates for position C+d (the anchor is the
 *    root at C): the draft's top-K tokens of block row d with their
 *    log-probabilities (log-softmax of that row's logits);
 *  - a node's score is the sum of the log-probabilities on its root path; the
 *    tree is the `budget` best nodes, ordered by score (descending), then
 *    depth, then rank path (lexicographic).  They always form a tree, and they
 *    maximise the expected number of accepted drafts when positions are taken
 *    as independent.  Scores are fp32 sums, one rounding per edge;
 *  - verification follows, from the root, the child whose token is the
 *    target's greedy token after the current node.
 * Trees have at most DFLASH_TREE_MAX_NODES = 32 nodes (the root and a budget
 * of up to 31), verified in one target pass (bf16 contexts whose projections
 * fit the 32-row kernels; otherwise 17 to 32 nodes take two passes).  Node
 * order: parent[j] < j. */

/* Per row r < rows of logits ([rows][ld] device fp32, ld >= V): the K largest
 * token ids (ties: lower id first) into ids_out (device int32 [rows][K]) and
 * their log-probabilities log_softmax(row)[id] into logp_out (device fp32
 * [rows][K]).  1 <= rows <= 16, 1 <= K <= min(16, V).  For a block drafted by
 * dflash_draft_block, pass the logits from row 1 on (rows = B - 1). */
dflash_status dflash_draft_topk(dflash_ctx* ctx, const float* logits, int64_t ld, int32_t rows, int32_t K,
                                int32_t* ids_out, float* logp_out, void* stream);

/* The verification tree: root = anchor (device int32[1], clamped into
 * [0, V)), and the `budget` best nodes of the candidate tree whose depth d
 * (1..depths) offers ids[d-1][0..K-1] with log-probabilities logp[d-1][..]
 * (device, [depths][K] as written by dflash_draft_topk, entries of a row in
 * descending order).  tokens_out, parent_out: device int32[budget + 1]; node 0
 * is the root (parent -1), node j >= 1 has parent_out[j] < j.  1 <= depths <=
 * 15, 1 <= K <= 16, 0 <= budget <= 31 and no more than the candidate tree
 * holds (INVAL). */
dflash_status dflash_build_tree(dflash_ctx* ctx, const int32_t* anchor, const int32_t* ids, const float* logp,
                                int32_t depths, int32_t K, int32_t budget, int32_t* tokens_out,
                                int32_t* parent_out, void* stream);

/* dflash_target_forward over the M nodes of a tree (parent: device int32[M],
 * parent[0] ignored, an entry outside [0, j) is read as 0, the root): row j
 * is placed at position C + depth(j), its K/V are stored at cache slot C + j,
 * and it attends to the cache before C and to its ancestors and itself, so
 * it computes what a causal forward of its root path computes (up to
 * rounding order).  argmax_out[j] is the target's greedy token after node j.
 * 1 <= M <= 32, in one pass that reads every weight once for all rows; where
 * the context's kernels cannot take more than 16 rows (fp32, or projections
 * whose tiles fill the compute units unevenly), nodes 16..M-1 run as a second
 * pass that finds their ancestors among the first pass's nodes in the cache.
 * Either way row j's results are those of the 16-row arithmetic (a chain of 32
 * nodes gives what two 16-row dflash_target_forward calls give, bit for bit).
 * Afterwards length = C + M; accept
 * with dflash_tree_accept, move the accepted rows with dflash_tree_commit,
 * then dflash_rollback to C + 1 + k.  Otherwise the arguments, errors and
 * capture rules of dflash_target_forward. */
dflash_status dflash_target_forward_tree(dflash_ctx* ctx, const int32_t* tokens, const int32_t* parent, int32_t M,
                                         float* logits_out, int32_t* argmax_out, void* const* capture,
                                         int64_t capture_ld, void* stream);

/* dflash_target_forward (parent NULL) or dflash_target_forward_tree, and in
 * the same launches the residual stream after every layer: layer_out
 * (device, [Ld][M][layer_ld] in the context dtype) receives row j of layer
 * l's output at layer_out[(l*M + j)*layer_ld].  An inspection aid (a test can
 * feed layer l's input to another implementation of that one layer); no
 * feature capture.  layer_ld >= H and keeps rows aligned (INVAL otherwise). */
dflash_status dflash_target_forward_ex(dflash_ctx* ctx, const int32_t* tokens, const int32_t* parent, int32_t M,
                                       float* logits_out, int32_t* argmax_out, void* layer_out, int64_t layer_ld,
                                       void* stream);

/* Greedy acceptance on a verified tree of M nodes (tokens, parent, target:
 * device int32[M]; target[j] = the target's greedy token after node j; a
 * parent outside [0, j) is read as 0; 1 <= M <= 32).  From the root, while a
 * child of the current node carries target[current] (the lowest-index one if
 * several) and fewer than 15 nodes are accepted (a block's draft positions; a
 * tree from dflash_build_tree is no deeper), move to it.  result_out: device int32[DFLASH_TREE_RESULT] = {k, bonus,
 * path[0..14]}: k accepted nodes, the target's token after the last one, and
 * their node indices (path[i] has depth i + 1; unused entries 0).  The prefix
 * {k, bonus} has the layout of a dflash_verify_accept result. */
dflash_status dflash_tree_accept(dflash_ctx* ctx, const int32_t* tokens, const int32_t* parent, const int32_t* target,
                                 int32_t M, int32_t* result_out, void* stream);

/* After dflash_target_forward_tree of M rows at pos0 and dflash_tree_accept:
 * for i < k, copy the K/V of cache slot pos0 + path[i] to slot pos0 + 1 + i in
 * every layer, and row path[i] of each non-NULL capture buffer (host array of
 * DFLASH_NUM_FEATURES device pointers, rows of capture_ld elements, or NULL)
 * to row 1 + i.  Slots and rows then hold the root and the accepted nodes in
 * sequence order, which is what a causal forward of that sequence stores (the
 * nodes were rotated at their depths).  result: device, as written by
 * dflash_tree_accept (k is clamped to [0, min(M-1, 15)], path entries to
 * [1, M-1]); 1 <= M <= 32.
 * Requires pos0 >= 0 and pos0 + M <= length (INVAL); the length is not
 * changed. */
dflash_status dflash_tree_commit(dflash_ctx* ctx, int32_t pos0, int32_t M, const int32_t* result,
                                 void* const* capture, int64_t capture_ld, void* stream);

/* ---- Non-greedy drafting and verification --------------------------------
 * The rebasdaily DFlash2 page (section 先猜几个，再让主模型拍板) ties DFlash2's
 * candidate selection to non-greedy samplers but gives no verification rule
 * for them.  The reading taken is the speculative sampling rule of the
 * literature (Leviathan, Kalman and Matias 2023; Chen et al. 2023), under
 * which the emitted tokens follow the target's own sampling distribution.
 * Random numbers: SplitMix64 as a counter-based generator -- draw n of stream
 * `seed` is its (n + 1)-th output with n = a * 2^32 + b for a draw's
 * coordinates (a, b), and a uniform is the top 24 bits times 2^-24 (plus
 * 2^-25 where a logarithm follows).  A caller gives every step its own seed. */

/* Draw one token per row r < rows of logits ([rows][ld] device fp32, ld >= V)
 * from softmax(row / temperature) by the Gumbel-max method: the id x with
 * the largest row[x] / T - log(-log U), U the draw at coordinates (r, x)
 * (ties: lower id).  tokens_out: device int32[rows] or NULL; lse_out: device
 * fp32[rows] or NULL, the rows' log-sum-exp of row / T (fp64 sums; at least
 * one of the two outputs).  Keys are fp32 with the perturbation good to about
 * 2e-6 absolute.  1 <= rows <= 16, temperature > 0 and finite, every buffer
 * 4-byte aligned (INVAL otherwise, nothing enqueued).  For a drafted block
 * pass the draft's logits from row 1 on: token r is the draft for position
 * C + 1 + r.  Uses the context's workspace: calls on one context are ordered
 * by their stream. */
dflash_status dflash_sample_tokens(dflash_ctx* ctx, const float* logits, int64_t ld, int32_t rows, float temperature,
                                   uint64_t seed, int32_t* tokens_out, float* lse_out, void* stream);

/* Speculative sampling over a drafted block of B (the context's block) rows:
 * draft: device int32[B] (entry j >= 1 is the draft for position C + j);
 * draft_logits, target_logits: device fp32 [B][ld] (draft row j gave draft j;
 * target row i is the target's prediction for position C + i + 1).  Draft j is
 * accepted when U * q < p, U the draw at (2^20 + j, 0), q = softmax(draft
 * row j / T)[d_j], p = softmax(target row j - 1 / T)[d_j]; at the first
 * rejection the next token is drawn from max(0, p - q) of those rows, after B
 * - 1 acceptances the bonus from softmax(target row B - 1 / T), with the draw
 * at (2^20 + 64, 0) (a draw: the first id whose running sum of weights
 * exceeds U * their total).  Probabilities, comparisons and the draw's sums
 * are fp64 (from the fp32 logits): where draft and target nearly agree the
 * residual is a difference of nearly equal probabilities.  result_out: device
 * int32[2] = {k, token}, the layout of a dflash_verify_accept result.
 * temperature > 0 and finite, ld >= V, every buffer 4-byte aligned (INVAL
 * otherwise, nothing enqueued).  Uses the context's workspace: calls on one
 * context are ordered by their stream. */
dflash_status dflash_verify_sample(dflash_ctx* ctx, const int32_t* draft, const float* draft_logits,
                                   const float* target_logits, int64_t ld, float temperature, uint64_t seed,
                                   int32_t* result_out, void* stream);

/* Load already-rotated K and V for positions [pos0, pos0+M) of every layer
 * (restoring a saved cache, or K/V computed elsewhere).  k, v: device
 * [Ld, M, nkv, d] contiguous.  Same pos0/capacity rules as dflash_inject_kv. */
dflash_status dflash_load_kv(dflash_ctx* ctx, const void* k, const void* v,
                             int32_t M, int32_t pos0, void* stream);

/* Read K and V of positions [pos0, pos0+M) (pos0 + M <= length) of every layer
 * into device k_out, v_out [Ld, M, nkv, d] contiguous. */
dflash_status dflash_read_kv(dflash_ctx* ctx, int32_t pos0, int32_t M,
                             void* k_out, void* v_out, void* stream);

/* Kernel classes that can be traced with dflash_trace_enable. */
typedef enum {
    DFLASH_TRACE_OFF = 0,
    DFLASH_TRACE_LM_HEAD = 1,  /* LM head + argmax launch of dflash_draft_block */
    DFLASH_TRACE_GATE_UP = 2,  /* SwiGLU gate/up projection, every layer */
    DFLASH_TRACE_DOWN = 3,     /* down projection + residual, every layer */
    DFLASH_TRACE_QKV = 4,      /* q/k/v projection + rotary, every layer */
    DFLASH_TRACE_O_PROJ = 5,   /* attention output projection + residual, every layer */
    DFLASH_TRACE_ATTN = 6,     /* split-KV attention + merge, every layer */
    DFLASH_TRACE_DRAFT = 7,    /* the whole dflash_draft_block call */
    DFLASH_TRACE_FUSE = 8,     /* fusion GEMM of dflash_fuse_context (without its RMSNorm) */
    DFLASH_TRACE_INJECT = 9,   /* injection of dflash_inject_kv */
    DFLASH_TRACE_TARGET = 10,  /* the whole dflash_target_forward(_tree) call */
    DFLASH_TRACE_TREE = 11,    /* each tree helper call: top-K, tree build, tree accept, tree commit */
    DFLASH_TRACE_SAMPLE = 12   /* each dflash_sample_tokens / dflash_verify_sample call */
} dflash_trace_class;

/* Tracing aid: while enabled, every launch of the given kernel class is
 * bracketed by a pair of HIP events recorded on its stream, for up to
 * max_launches launches (later ones are not timed).  Enabling again (or with
 * DFLASH_TRACE_OFF) discards previous records.  Events are host-side HIP
 * objects; no device memory is allocated. */
dflash_status dflash_trace_enable(dflash_ctx* ctx, int32_t kernel_class, int32_t max_launches);

/* Wait for the recorded events and report the summed duration (ms) of the
 * timed launches and their count.  Host pointers. */
dflash_status dflash_trace_read(dflash_ctx* ctx, double* total_ms, int32_t* launches);

/* The same records one by one: durations_ms (host float[capacity]) receives the
 * duration of each timed launch in launch order, *launches the number written
 * (at most capacity). */
dflash_status dflash_trace_read_each(dflash_ctx* ctx, float* durations_ms, int32_t capacity, int32_t* launches);

/* Measurement aid, not part of the method: one launch of a plain streaming-read
 * kernel over the device buffer buf (bytes long, 16-byte aligned) on the given
 * stream, so a caller can time the chip's practical HBM read rate next to the
 * draft kernels' roofline figures.  Every wave of 4 per CU reads one contiguous
 * range with 16-byte non-temporal loads.  *read_bytes (host) receives the bytes
 * actually read: the largest prefix that divides evenly into the waves' rounds
 * (0 if bytes is below 4 MB per 256 CUs; then nothing is launched).  sink is a
 * 4-byte-aligned device word the kernel may write (never read back).  INVAL on
 * null pointers, a negative size or a misaligned buffer or sink. */
dflash_status dflash_hbm_read_probe(const void* buf, int64_t bytes, void* sink, int64_t* read_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif

// kernels.h -- launch entry points of the libdflash HIP kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include "host.h"

namespace dflash {

// Optional per-launch timing of one kernel class (HIP event pairs).
struct Tracer {
    int cls = 0;
    int max = 0;
    int n = 0;
    hipEvent_t* ev = nullptr;  // 2 * max events
    void begin(int k, hipStream_t s) {
        if (k == cls && n < max) (void)hipEventRecord(ev[2 * n], s);
    }
    void end(int k, hipStream_t s) {
        if (k == cls && n < max) {
            (void)hipEventRecord(ev[2 * n + 1], s);
            ++n;
        }
    }
};

// Everything a launcher needs about one context: dims, layout and the base
// pointers of the caller's buffers.
struct DevCtx {
    Dims dm;
    Layout lay;
    char* ws;   // workspace base
    char* kv;   // KV pool base
    int num_cus;
    const void* fc;
    const void* fc_norm;
    const void* attn_norm[DFLASH_MAX_LAYERS];
    const void* wq[DFLASH_MAX_LAYERS];
    const void* wk[DFLASH_MAX_LAYERS];
    const void* wv[DFLASH_MAX_LAYERS];
    const void* wo[DFLASH_MAX_LAYERS];
    const void* mlp_norm[DFLASH_MAX_LAYERS];
    const void* wg[DFLASH_MAX_LAYERS];
    const void* wu[DFLASH_MAX_LAYERS];
    const void* wd[DFLASH_MAX_LAYERS];
    const void* final_norm;
    const void* embed;
    const void* lm_head;
    // swizzled copies (inside the workspace) of the weights the skinny GEMM streams
    const void* sw_wq[DFLASH_MAX_LAYERS];
    const void* sw_wk[DFLASH_MAX_LAYERS];
    const void* sw_wv[DFLASH_MAX_LAYERS];
    const void* sw_wo[DFLASH_MAX_LAYERS];
    const void* sw_wg[DFLASH_MAX_LAYERS];
    const void* sw_wu[DFLASH_MAX_LAYERS];
    const void* sw_wd[DFLASH_MAX_LAYERS];
    const void* sw_lm;
    const void* sw_fc;
    Tracer* tracer;
};

// Write the swizzled copy of a row-major [N][K] matrix (N % 16 == 0, K % 8 == 0).
hipError_t launch_swizzle(int dtype, const void* W, int N, int K, void* out, hipStream_t s);
// reads the largest whole-round prefix of buf; *read_bytes receives its size
hipError_t launch_read_probe(const void* buf, long long bytes, int num_cus, unsigned* sink, long long* read_bytes,
                             hipStream_t s);

// One draft block over the first C context positions.
// layer_out: optional [Ld][B][layer_ld] copy of the residual stream after every layer.
// len_dev: non-null when the context length lives on the device (C unused).
hipError_t launch_draft_block(const DevCtx& c, int C, const int32_t* anchor, float* logits,
                              int32_t* tokens, void* layer_out, long long layer_ld, const int* len_dev,
                              hipStream_t s);
// Causal forward of M <= 16 tokens at positions C..C+M-1 (K/V appended to the cache),
// or of a tree's 17..32 nodes in one pass when wide_pass_supported(c).
// tree_parent (device int32[tree_n], or null): the rows are nodes tree_off ..
// tree_off + M - 1 of a tree of tree_n <= 32 nodes whose root (node 0) sits at
// tree_base; node u is placed at tree_base + depth(u) and sees the cache before
// tree_base plus its ancestors (K/V of node u at slot tree_base + u, so C must be
// tree_base + tree_off).  layer_out (or null): [Ld][layer_rows][layer_ld]
// residual after every layer (rows of this pass from layer_out on; layer_rows 0:
// M), in place of capture.
hipError_t launch_causal_forward(const DevCtx& c, int C, const int32_t* tokens, int M, float* logits,
                                 int32_t* argmax, void* const* capture, long long capture_ld, hipStream_t s,
                                 const int32_t* tree_parent = nullptr, void* layer_out = nullptr,
                                 long long layer_ld = 0, int tree_off = 0, int tree_base = 0, int tree_n = 0,
                                 int layer_rows = 0);
// Whether a causal pass can take up to 32 rows at once (bf16, and every
// projection on the workgroup-local kernel); otherwise a tree of more than 16
// nodes is verified in passes of 16.
bool wide_pass_supported(const DevCtx& c);
// Tree verification helpers (tree.hip).
// Per row r < rows of logits [rows][ld]: the K <= 16 largest ids (ties: lower
// id first) and their fp32 log-probabilities.
hipError_t launch_topk(const DevCtx& c, const float* logits, long long ld, int rows, int K, int32_t* ids,
                       float* logp, hipStream_t s);
// Best-first candidate tree of `budget` nodes over R depths of K candidates.
hipError_t launch_tree_build(const int32_t* anchor, int V, const int32_t* ids, const float* logp, int R, int K,
                             int budget, int32_t* tokens, int32_t* parent, hipStream_t s);
// Gumbel-max draws at temperature T from each of `rows` logit rows (row r draws
// with generator coordinates (r, id)); tokens and/or the rows' log-sum-exp of z / T.
hipError_t launch_sample_tokens(const DevCtx& c, const float* logits, long long ld, int rows, float T,
                                unsigned long long seed, int32_t* tokens, float* lse, hipStream_t s);
// Speculative sampling over a drafted block: out = {k, token after the accepted drafts}.
hipError_t launch_verify_sample(const DevCtx& c, const int32_t* draft, const float* draft_logits,
                                const float* target_logits, long long ld, float T, unsigned long long seed,
                                int32_t* out, hipStream_t s);
// Accepted path of a verified tree: out = {k, bonus, path[0..14]}.
hipError_t launch_tree_accept(const int32_t* tokens, const int32_t* parent, const int32_t* target, int M,
                              int32_t* out, hipStream_t s);
// Move the accepted rows behind the root: KV slots pos0 + path[i] -> pos0 + 1 + i
// in every layer, and rows path[i] -> 1 + i of each non-null capture buffer.
hipError_t launch_tree_commit(const DevCtx& c, int pos0, int M, const int32_t* result, void* const* capture,
                              long long capture_ld, hipStream_t s);
// Context fusion of M rows (selected slabs given in ascending layer order).
hipError_t launch_fuse(const DevCtx& c, const void* const slabs[5], long long ld, int M, void* out,
                       hipStream_t s);
// The same for M <= 16 rows with the stream-K scratch in the library's static
// per-GPU array (static_scratch_init(device) must have run for that device).
hipError_t launch_fuse_static(const DevCtx& c, int device, const void* const slabs[5], long long ld, int M,
                              void* out, hipStream_t s);
// Look up (once per device, with that device current) the static scratch's address.
hipError_t static_scratch_init(int device);
// Whether a context's 16-row fusion fits the static scratch.
bool static_scratch_fits(const DevCtx& c);
// KV injection of M rows of fused features at positions pos0...
// len_dev non-null: rows go to *len_dev.. (M <= 16; err is set when they do not fit).
hipError_t launch_inject(const DevCtx& c, const void* fused, long long ld, int M, int pos0, hipStream_t s,
                         const int* len_dev = nullptr, int* err = nullptr);
// Device-resident length word: set, add k + 1 from an accept result {k, bonus}, copy {length, error} out.
hipError_t launch_len_set(int* len, int value, hipStream_t s);
hipError_t launch_len_keep(int* len, const int32_t* result, int max_ctx, hipStream_t s);
hipError_t launch_len_read(const int* len, int32_t* out, hipStream_t s);
// Greedy acceptance.
hipError_t launch_accept(const DevCtx& c, const int32_t* draft, const int32_t* target, int32_t* out,
                         hipStream_t s);
// Copy dense [Ld, M, nkv, d] K/V into (to_pages) or out of the pages.
hipError_t launch_kv_copy(const DevCtx& c, void* k, void* v, int M, int pos0, bool to_pages, hipStream_t s);

}  // namespace dflash

// host.h -- host-only logic of libdflash: config validation, workspace layout,
// page table, length bookkeeping.  No HIP dependency, so it is unit-testable on
// a machine without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/dflash.h"

namespace dflash {

// Launch geometry shared by host and device code.
constexpr int kWaveSize = 64;
constexpr int kSkinnyWavesPerWG = 4;     // skinny (M <= 16) GEMM: 256-thread workgroups
constexpr int kSkinnyNT = 2;             // 16-column blocks per skinny tile (most ops)
constexpr int kSkinnyMaxNT = 4;          // the widest skinny tile (LM head)
constexpr int kAttnChunk = 64;           // keys per attention step
constexpr int kMaxSplitPages = 1040;     // KV pages one attention split may touch
constexpr int kAttnStages = 2;           // attention chunks resident in LDS per workgroup (fp32)
constexpr int kAttnStagesBF16 = 2;       // the same for bf16 (its chunks are kAttnChunkBF16 keys)
constexpr int kAttnChunkBF16 = 64;       // keys per bf16 attention chunk
constexpr int kAttnWGPerCU = 2;          // attention workgroups per CU
constexpr int kLDSBytesPerCU = 160 * 1024;
// Attention workgroups that fit a CU: NS stages of CH keys (K rows and V^T rows
// of row_bytes each) plus the staged page ids, at most kAttnWGPerCU.
constexpr int attn_wg_per_cu(int ns, int ch, int row_bytes) {
    return (ns * ch * row_bytes * 2 + kMaxSplitPages * 4 + 64) * kAttnWGPerCU <= kLDSBytesPerCU ? kAttnWGPerCU : 1;
}
template <typename T>
constexpr int attn_stages() { return sizeof(T) == 2 ? kAttnStagesBF16 : kAttnStages; }
template <typename T>
constexpr int attn_chunk() { return sizeof(T) == 2 ? kAttnChunkBF16 : kAttnChunk; }
constexpr int kMaxSplits = 256;          // context splits of the split-KV attention
constexpr int kBigBM = 64, kBigBN = 64;  // large-M GEMM tile
constexpr int kTopKMax = 16;             // candidates per draft position of a tree (the largest useful K)
constexpr int kTopKSegs = 64;            // vocabulary segments of the top-K partial pass (one merge lane each)
constexpr int kPassRowsMax = 32;         // rows of one decoder pass: a 16-row block, or a verified tree of up to 32 nodes

struct Dims {
    int dtype, H, Lt, Ld, nq, nkv, d, F, V, B, mask_id, page, max_ctx, max_rows, n_pages, elem;
    double rope_base, eps;
};

// Byte offsets of every region inside the caller's workspace (256-byte aligned).
// Weights streamed by the skinny GEMM are kept a second time in the MFMA
// operand order ("swizzled"): for W [N][K], block (n/16, k/32) is one
// contiguous group of 64 lanes x 8 elements, lane l holding
// W[16*(n/16) + l%16][32*(k/32) + 8*(l/16) .. +8]; K is zero-padded to a
// multiple of 32.  For fp32 the 8 elements of a lane are split into two
// 16-byte halves stored as two consecutive 1 KB planes.  One wave instruction
// then reads 1 KB of contiguous memory.
inline size_t swizzled_bytes(long long N, long long K, int elem) {
    return (size_t)((N + 15) / 16) * (size_t)((K + 31) / 32) * 512 * (size_t)elem;
}

struct Layout {
    size_t rope_cos, rope_sin, page_table;
    // swizzled weight copies (offsets into the workspace)
    size_t sw_wq[DFLASH_MAX_LAYERS], sw_wk[DFLASH_MAX_LAYERS], sw_wv[DFLASH_MAX_LAYERS], sw_wo[DFLASH_MAX_LAYERS];
    size_t sw_wg[DFLASH_MAX_LAYERS], sw_wu[DFLASH_MAX_LAYERS], sw_wd[DFLASH_MAX_LAYERS];
    size_t sw_lm, sw_fc;
    size_t x, q, kblk, vblkT, obuf, hbuf;
    size_t rstd, ss_part, partial, tile_cnt, counters, best;
    size_t attn_o, attn_ml;
    size_t len_dev;       // device-resident length: {length, capacity-error flag}
    size_t tree_info;     // tree verification: depth[32], then ancestor mask[32]
    size_t topk_part;     // top-K / sampling partials: [16 rows][kTopKSegs] x (K values, K ids, max, sum)
    size_t sample_draw;   // sampled verification: a 64-byte header, then one fp64 weight sum per 1024 ids
    size_t total;
    size_t kv_total;      // bytes of the KV pool
    size_t kv_layer_kv;   // bytes of one (layer, K-or-V) page array
    int nwaves;           // skinny-GEMM waves per launch
    int max_tiles;        // largest tile count of any skinny GEMM
    int max_ss_tiles;     // tiles of an N = H skinny GEMM (row sum-of-squares partials)
    int ss_stride;        // row stride of the partials ([32 rows][ss_stride], zero past the tiles)
    int n_rope_pos;       // positions covered by the rotary table
};

// Validate a config; on failure returns a status and writes a message.
dflash_status validate_config(const dflash_config* cfg, Dims* out, std::string* err);

// Workspace layout for validated dims.  `num_cus` sizes the skinny-GEMM grid.
Layout compute_layout(const Dims& d, int num_cus);

// Physical page of each logical page: identity, or a seeded Fisher-Yates
// shuffle (splitmix64 stream) when seed != 0.
std::vector<int32_t> make_page_table(int n_pages, uint64_t seed);

// The five fused target layers: round_half_up(1 + i*(L-3)/4), i = 0..4.
void feature_layers(int target_layers, int32_t out[5]);

// Attention split plan for a context of C keys: keys per split (multiple of
// kAttnChunk) and number of context splits (the block keys get one more).
void attn_split_plan(int C, int nkv, int num_cus, int page, int* keys_per_split, int* n_splits,
                     int wg_per_cu = kAttnWGPerCU);

// Keys per split of the causal forward: fixed for a context (it depends on
// max_ctx only), so split boundaries sit at the same absolute positions in
// every call.
int causal_split_keys(int max_ctx);

}  // namespace dflash

// tree.hip -- tree verification (DDTree) around the target pass.
//
// "DFlash 深度解析…" §8.2 (DDTree tree verification): one target pass checks a
// tree of candidate drafts under a node budget instead of one chain.  The
// target pass itself is the causal forward with a tree mask (kernels.hip);
// this file holds the small steps around it:
//  - top-K of the draft's logits per block position, with log-probabilities;
//  - the best-first candidate tree: the `budget` nodes with the largest sum of
//    log-probabilities along their root path (ties: shallower, then the
//    lexicographically smaller rank path), scores added in fp32;
//  - the accepted path: from the root, follow the child that carries the
//    target's greedy token after the current node;
//  - the compaction of the accepted rows behind the root (KV slots of every
//    layer, captured feature rows), after which the cache holds exactly the
//    accepted sequence.
// All of them are latency-bound, tiny launches next to the pass they serve.
#include "device_common.h"
#include "kernels.h"
#include "kv_pages.h"

#include <math.h>

#include <algorithm>

namespace dflash {

namespace {

constexpr int kTopKThreads = 256;
constexpr int kPartStride = 2 * kTopKMax + 2;  // floats per (row, segment) record

// (value, id) order of the top-K: larger value first, then lower id
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// (max, sum of exp(x - max)) of two parts, in a fixed operand order
__device__ __forceinline__ void lse_combine(float& m, float& s, float m2, float s2) {
    if (m2 == -INFINITY) return;
    if (m == -INFINITY) {
        m = m2;
        s = s2;
        return;
    }
    const float M = fmaxf(m, m2);
    s = s * __expf(m - M) + s2 * __expf(m2 - M);
    m = M;
}

// One (row, vocabulary segment) per workgroup: every thread keeps a sorted
// list of its K best (value, id) pairs and its own running (max, sum of exp);
// then K rounds of a workgroup-wide best pick the segment's K best in order.
// KM: the list length compiled in (the smallest of 4, 8, 16 that holds K), so
// an insertion costs KM compare-and-moves.
template <int KM>
__global__ __launch_bounds__(kTopKThreads) void topk_partial_kernel(const float* logits, long long ld, int V, int K,
                                                                    float* part) {
    constexpr int W = kTopKThreads / 64;
    __shared__ float w_v[W][kTopKMax];
    __shared__ int w_i[W][kTopKMax];
    __shared__ float s_m[W], s_s[W];
    const int seg = blockIdx.x, r = blockIdx.y, S = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int per = (V + S - 1) / S;
    const int beg = seg * per, end = min(V, beg + per);
    const float* x = logits + (long long)r * ld;

    float tv[KM];
    int ti[KM];
#pragma unroll
    for (int q = 0; q < KM; ++q) {
        tv[q] = -INFINITY;
        ti[q] = 0x7fffffff;
    }
    float thr = -INFINITY;  // the K-th value held (ids scanned in ascending order: ties stay out)
    float m = -INFINITY, sum = 0.f;
    // U loads in flight per thread, then their values in id order
    constexpr int U = 8;
    for (int i0 = beg + tid; i0 < end; i0 += U * kTopKThreads) {
        float vb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kTopKThreads;
            vb[u] = i < end ? x[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
        const int i = i0 + u * kTopKThreads;
        if (i >= end) break;
        const float v = vb[u];
        if (v > m) {
            sum = sum * __expf(m - v) + 1.f;
            m = v;
        } else {
            sum += __expf(v - m);
        }
        if (v > thr) {
            float cv = v;
            int ci = i;
#pragma unroll
            for (int q = 0; q < KM; ++q) {  // insert, shifting the rest down
                const bool take = cv > tv[q];
                const float ov = tv[q];
                const int oi = ti[q];
                tv[q] = take ? cv : ov;
                ti[q] = take ? ci : oi;
                cv = take ? ov : cv;
                ci = take ? oi : ci;
            }
#pragma unroll
            for (int q = 0; q < KM; ++q)
                if (q == K - 1) thr = tv[q];
        }
        }
    }
    float* rec = part + ((long long)r * S + seg) * kPartStride;

    // segment (max, sum): wave butterfly, then the four waves in order
    for (int o = 32; o >= 1; o >>= 1) {
        const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(sum, o, 64);
        // both lanes of a pair combine in the same operand order (lower lane first)
        if (lane & o) {
            float mm = m2, ss = s2;
            lse_combine(mm, ss, m, sum);
            m = mm;
            sum = ss;
        } else {
            lse_combine(m, sum, m2, s2);
        }
    }
    if (lane == 0) {
        s_m[w] = m;
        s_s[w] = sum;
    }
    __syncthreads();
    if (tid == 0) {
        float M = s_m[0], Ssum = s_s[0];
        for (int i = 1; i < kTopKThreads / 64; ++i) lse_combine(M, Ssum, s_m[i], s_s[i]);
        rec[2 * kTopKMax] = M;
        rec[2 * kTopKMax + 1] = Ssum;
    }

    // each wave: K rounds of the best list head over its lanes (no workgroup
    // barrier per round); the owner's list drops its head
    for (int k = 0; k < K; ++k) {
        float bv = tv[0];
        int bi = ti[0];
        for (int o = 32; o >= 1; o >>= 1) {
            const float v2 = __shfl_xor(bv, o, 64);
            const int i2 = __shfl_xor(bi, o, 64);
            if (ranks_before(v2, i2, bv, bi)) {
                bv = v2;
                bi = i2;
            }
        }
        if (lane == 0) {
            w_v[w][k] = bv;
            w_i[w][k] = bi;
        }
        if (ti[0] == bi && tv[0] == bv) {  // the owner (ids are unique among real entries)
#pragma unroll
            for (int q = 0; q + 1 < KM; ++q) {
                tv[q] = tv[q + 1];
                ti[q] = ti[q + 1];
            }
            tv[KM - 1] = -INFINITY;
            ti[KM - 1] = 0x7fffffff;
        }
    }
    __syncthreads();
    // the segment's K best: each of the W*K wave candidates counts those ranked before it
    if (tid < W * K) {
        const float v = w_v[tid / K][tid % K];
        const int id = w_i[tid / K][tid % K];
        int rank = 0;
        for (int u = 0; u < W; ++u)
            for (int q = 0; q < K; ++q) rank += ranks_before(w_v[u][q], w_i[u][q], v, id) ? 1 : 0;
        if (rank < K) {
            rec[rank] = v;
            reinterpret_cast<int*>(rec)[kTopKMax + rank] = id;
        }
    }
}

// One wave per row.  Lane l < S holds segment l's list (its K best in rank
// order, from the partial pass); K rounds of a 64-lane butterfly pick the best
// list head (value descending, id ascending), which the owning lane then
// drops.  The row's log-sum-exp: the segments' largest max, then their sums
// rescaled to it and added over the wave; log-probabilities subtract it.
__global__ __launch_bounds__(64) void topk_merge_kernel(const float* part, int S, int K, int32_t* ids, float* logp) {
    __shared__ float c_v[kTopKSegs * kTopKMax];
    __shared__ int c_i[kTopKSegs * kTopKMax];
    const int r = blockIdx.x, lane = threadIdx.x;
    const float* base = part + (long long)r * S * kPartStride;
    for (int t = lane; t < S * K; t += 64) {
        const float* rec = base + (long long)(t / K) * kPartStride;
        c_v[t] = rec[t % K];
        c_i[t] = reinterpret_cast<const int*>(rec)[kTopKMax + t % K];
    }
    float m = -INFINITY, sm = 0.f;
    if (lane < S) {
        m = base[(long long)lane * kPartStride + 2 * kTopKMax];
        sm = base[(long long)lane * kPartStride + 2 * kTopKMax + 1];
    }
    float M = m;
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float L = m == -INFINITY ? 0.f : sm * __expf(m - M);
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
    const float lse = M + logf(L);
    __syncthreads();
    int head = 0;  // this lane's next unchosen entry
    for (int k = 0; k < K; ++k) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        if (lane < S && head < K) {
            bv = c_v[lane * K + head];
            bi = c_i[lane * K + head];
        }
        const float mv = bv;
        const int mi = bi;
        for (int o = 32; o >= 1; o >>= 1) {
            const float v2 = __shfl_xor(bv, o, 64);
            const int i2 = __shfl_xor(bi, o, 64);
            if (ranks_before(v2, i2, bv, bi)) {
                bv = v2;
                bi = i2;
            }
        }
        if (lane == 0) {
            ids[(long long)r * K + k] = bi;
            logp[(long long)r * K + k] = bv - lse;
        }
        if (lane < S && head < K && mv == bv && mi == bi) ++head;  // the owner (real ids are unique)
    }
}

// Candidate order as one 128-bit key (larger = better), compared branch-free:
//   hi = valid (1 bit) | score mapped to an unsigned order (32 bits) | 31 - depth (5 bits)
//   lo = ~rank path (4 bits per depth, depth 1 in the top bits).
__device__ __forceinline__ unsigned order_bits(float f) {
    const unsigned u = __float_as_uint(f + 0.0f);  // -0 -> +0: equal scores compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long shfl_xor64(unsigned long long v, int o) {
    const unsigned lo = (unsigned)__shfl_xor((int)(unsigned)v, o, 64);
    const unsigned hi = (unsigned)__shfl_xor((int)(unsigned)(v >> 32), o, 64);
    return ((unsigned long long)hi << 32) | lo;
}

// One wave.  Lane u < count holds node u: its score, depth, rank path and the
// rank of its next unchosen child.  Every step the best of the lanes' next
// children (a 32-lane butterfly over the keys above) joins the tree as node
// `count`; a child never beats its parent or an earlier sibling, so the
// chosen nodes are the budget best of the whole candidate tree.
__global__ __launch_bounds__(64) void tree_build_kernel(const int32_t* anchor, int V, const int32_t* ids,
                                                        const float* logp, int R, int K, int budget, int32_t* tokens,
                                                        int32_t* parent) {
    __shared__ float s_lp[15 * kTopKMax];
    __shared__ int s_id[15 * kTopKMax];
    const int lane = threadIdx.x;
    for (int i = lane; i < R * K; i += 64) {
        s_lp[i] = logp[i];
        s_id[i] = ids[i];
    }
    __syncthreads();
    float sc = 0.f;
    int dep = 0, nr = 0, par = -1;
    unsigned long long path = 0ull;
    int tok = lane == 0 ? min(max(anchor[0], 0), V - 1) : 0;
    for (int count = 1; count <= budget; ++count) {
        const bool ok = lane < count && dep < R && nr < K;
        const float cs = sc + s_lp[ok ? dep * K + nr : 0];
        const int cd = min(dep + 1, 15);
        const unsigned long long cp = path | ((unsigned long long)(ok ? nr : 0) << (4 * (15 - min(dep, 14))));
        const unsigned long long hi0 =
            ok ? ((1ull << 37) | ((unsigned long long)order_bits(cs) << 5) | (unsigned)(31 - cd)) : 0ull;
        const unsigned long long lo0 = ~cp;
        unsigned long long hi = hi0, lo = lo0;
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) {
            const unsigned long long h2 = shfl_xor64(hi, o), l2 = shfl_xor64(lo, o);
            const bool take = h2 > hi || (h2 == hi && l2 > lo);
            hi = take ? h2 : hi;
            lo = take ? l2 : lo;
        }
        // lanes 0..31 now hold the winner; its lane is the one whose own key
        // it is (the keys of real candidates differ in their rank paths)
        const unsigned long long own = __ballot(ok && hi0 == hi && lo0 == lo);
        const int wl = own ? __ffsll((long long)own) - 1 : 0;
        const int wd = 31 - (int)(hi & 31ull);
        const unsigned long long wp = ~lo;
        const int rank = (int)((wp >> (4 * (16 - wd))) & 15ull);
        const float ws = __shfl(cs, wl, 64);  // the winner's own fp32 score (all lanes take part)
        if (lane == count) {
            sc = ws;
            dep = wd;
            path = wp;
            nr = 0;
            par = wl;
            tok = s_id[min((wd - 1) * K + rank, R * K - 1)];
        }
        if (lane == wl) ++nr;
    }
    if (lane <= budget) {
        tokens[lane] = tok;
        parent[lane] = par;
    }
}

// One wave: lane j holds node j.  From the root, the child (lowest index
// among equals) whose token is the target's greedy token after the current
// node is accepted, until none is or 15 nodes are (a block's draft
// positions; a tree from the builder is no deeper).  A parent outside
// [0, j) reads as the root.
__global__ __launch_bounds__(64) void tree_accept_kernel(const int32_t* tokens, const int32_t* parent,
                                                         const int32_t* target, int M, int32_t* out) {
    const int lane = threadIdx.x;
    const bool node = lane < M;
    const int tok = node ? tokens[lane] : 0;
    const int p = node ? parent[lane] : 0;
    const int par = (p >= 0 && p < lane) ? p : 0;
    const int tgt = node ? target[lane] : 0;
    int cur = 0, k = 0;
    int path[15];
#pragma unroll
    for (int i = 0; i < 15; ++i) path[i] = 0;
#pragma unroll
    for (int step = 0; step < 15; ++step) {
        const int want = __shfl(tgt, cur, 64);
        const unsigned long long hit = __ballot(node && lane >= 1 && par == cur && tok == want);
        if (hit == 0ull) break;
        cur = __ffsll((long long)hit) - 1;
        path[step] = cur;
        k = step + 1;
    }
    const int bonus = __shfl(tgt, cur, 64);
    if (lane == 0) {
        out[0] = k;
        out[1] = bonus;
#pragma unroll
        for (int i = 0; i < 15; ++i) out[2 + i] = path[i];
    }
}

struct CommitArgs {
    KVPages kv;
    void* cap[5];
    long long cap_ld;
    int H, Ld, pos0, M;
    const int32_t* result;
};

// Blocks [0, Ld*nkv*2): one (layer, kv head, K|V) each, a thread per head
// dimension.  The rest: one (capture buffer, 256-column slice) each.  Every
// thread loads all of its accepted values before storing any, so sources that
// are also destinations (path[i] == 1 + i' for i' > i) are read first.
template <typename T>
__global__ __launch_bounds__(256) void tree_commit_kernel(CommitArgs a) {
    const int M = a.M;
    const int k = min(max(a.result[0], 0), min(M - 1, 15));  // an accepted path holds at most 15 nodes
    int src[15];
#pragma unroll
    for (int i = 0; i < 15; ++i) src[i] = i < k ? min(max(a.result[2 + i], 1), M - 1) : 1;
    const int nkv = a.kv.nkv, d = a.kv.d;
    const int kv_blocks = a.Ld * nkv * 2;
    T val[15];
    if ((int)blockIdx.x < kv_blocks) {
        const int b = blockIdx.x;
        const int isv = b & 1, h = (b >> 1) % nkv, l = (b >> 1) / nkv;
        const int dim = threadIdx.x;
        if (dim >= d) return;
        auto at = [&](int pos) -> T* {
            int slot;
            if (!isv) return a.kv.kpage<T>(l, pos, slot) + ((long long)h * a.kv.page + slot) * d + dim;
            T* pg = a.kv.vpage<T>(l, pos, slot);
            return pg + ((long long)h * d + dim) * a.kv.page + vslot(slot);
        };
#pragma unroll
        for (int i = 0; i < 15; ++i)
            if (i < k) val[i] = *at(a.pos0 + src[i]);
#pragma unroll
        for (int i = 0; i < 15; ++i)
            if (i < k) *at(a.pos0 + 1 + i) = val[i];
        return;
    }
    const int cb = blockIdx.x - kv_blocks;
    const int slices = (a.H + 255) / 256;
    T* buf = reinterpret_cast<T*>(a.cap[cb / slices]);
    const int col = (cb % slices) * 256 + threadIdx.x;
    if (!buf || col >= a.H) return;
#pragma unroll
    for (int i = 0; i < 15; ++i)
        if (i < k) val[i] = buf[(long long)src[i] * a.cap_ld + col];
#pragma unroll
    for (int i = 0; i < 15; ++i)
        if (i < k) buf[(long long)(1 + i) * a.cap_ld + col] = val[i];
}

}  // namespace

hipError_t launch_topk(const DevCtx& c, const float* logits, long long ld, int rows, int K, int32_t* ids, float* logp,
                       hipStream_t s) {
    const int V = c.dm.V;
    // segments of at least 2048 ids: every wave then holds at least K real candidates
    const int S = std::max(1, std::min(kTopKSegs, V / 2048));
    float* part = reinterpret_cast<float*>(c.ws + c.lay.topk_part);
    const dim3 grid(S, rows);
    if (K <= 4) hipLaunchKernelGGL(topk_partial_kernel<4>, grid, dim3(kTopKThreads), 0, s, logits, ld, V, K, part);
    else if (K <= 8) hipLaunchKernelGGL(topk_partial_kernel<8>, grid, dim3(kTopKThreads), 0, s, logits, ld, V, K, part);
    else hipLaunchKernelGGL(topk_partial_kernel<kTopKMax>, grid, dim3(kTopKThreads), 0, s, logits, ld, V, K, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(rows), dim3(64), 0, s, part, S, K, ids, logp);
    return hipGetLastError();
}

hipError_t launch_tree_build(const int32_t* anchor, int V, const int32_t* ids, const float* logp, int R, int K,
                             int budget, int32_t* tokens, int32_t* parent, hipStream_t s) {
    hipLaunchKernelGGL(tree_build_kernel, dim3(1), dim3(64), 0, s, anchor, V, ids, logp, R, K, budget, tokens, parent);
    return hipGetLastError();
}

hipError_t launch_tree_accept(const int32_t* tokens, const int32_t* parent, const int32_t* target, int M,
                              int32_t* out, hipStream_t s) {
    hipLaunchKernelGGL(tree_accept_kernel, dim3(1), dim3(64), 0, s, tokens, parent, target, M, out);
    return hipGetLastError();
}

hipError_t launch_tree_commit(const DevCtx& c, int pos0, int M, const int32_t* result, void* const* capture,
                              long long capture_ld, hipStream_t s) {
    CommitArgs a;
    a.H = c.dm.H;
    a.Ld = c.dm.Ld;
    a.pos0 = pos0;
    a.M = M;
    a.result = result;
    a.cap_ld = capture_ld;
    int n_cap = 0;
    for (int i = 0; i < 5; ++i) {
        a.cap[i] = capture ? capture[i] : nullptr;
        n_cap += a.cap[i] != nullptr;
    }
    const int blocks = c.dm.Ld * c.dm.nkv * 2 + (n_cap ? 5 * ((c.dm.H + 255) / 256) : 0);
    if (c.dm.dtype == DFLASH_F32) {
        a.kv = make_pages<float>(c);
        hipLaunchKernelGGL(tree_commit_kernel<float>, dim3(blocks), dim3(256), 0, s, a);
    } else {
        a.kv = make_pages<bf16_t>(c);
        hipLaunchKernelGGL(tree_commit_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace dflash

// sample.hip -- non-greedy drafting and verification.
//
// The rebasdaily DFlash2 page (section 先猜几个，再让主模型拍板) ties DFlash2's
// candidate selection to non-greedy samplers; the pages give no verification
// rule for them, so this file follows the speculative sampling rule of the
// literature (Leviathan, Kalman and Matias 2023; Chen et al. 2023):
//  - drafting at temperature T draws each block token from softmax(z / T) by
//    the Gumbel-max method, argmax over x of z[x] / T - log(-log U(r, x));
//  - draft d_j is accepted when U_j * q_j(d_j) < p_{j-1}(d_j) (q: the draft's
//    softmax of its row j, p: the target's softmax of its verified row j - 1);
//    at the first rejection the next token is drawn from max(0, p - q), after
//    B - 1 acceptances the bonus is drawn from the target's last row;
//  - a draw from weights w with U: the first id whose running sum exceeds
//    U * sum(w).
// Random numbers come from SplitMix64 used as a counter-based generator (draw
// n of stream `seed` is its (n + 1)-th output, n = a * 2^32 + b for the draw's
// coordinates (a, b)); a uniform keeps the top 24 bits.  Coordinates: the
// Gumbel draw of row r and token x is (r, x); the acceptance draw of draft j
// is (2^20 + j, 0); the rejection / bonus draw is (2^20 + 64, 0).
//
// Precision.  Gumbel keys are fp32, the perturbation good to about 2e-6
// absolute (a draw flips only where two keys lie that close).  The
// verification works in fp64 from the fp32
// logits: where draft and target nearly agree, the residual max(0, p - q)
// is a difference of nearly equal probabilities, and at a 152K vocabulary an
// fp32 log-sum-exp (ulp ~1e-6 at ~12) cannot resolve a residual mass of 1e-5.
//
// Verification launches (B = block rows, S = vocabulary segments):
//   1. lse partials over the B target rows and draft rows 1 .. B-1;
//   2. one workgroup per 1024 ids: merges the row lse values, decides k (every
//      workgroup the same way), sums its ids' weights of the row pair drawn
//      from; workgroup 0 also stores k and the pair's lse for launch 3;
//   3. one workgroup: the draw, by a sequential scan at each level (segment,
//      wave, lane, id), which keeps every running sum non-decreasing; where a
//      level's parts sum past its parent's rounded total the last id of
//      positive weight in the segment is taken.
#include "device_common.h"
#include "kernels.h"

#include <math.h>

#include <algorithm>

namespace dflash {

namespace {

constexpr int kSampleThreads = 256;
constexpr int kDrawSeg = 1024;            // ids per segment of the draw
constexpr int kDrawThreads = 256;         // threads of a draw workgroup (4 ids each)
constexpr int kTagAccept = 1 << 20;
constexpr int kTagResidual = (1 << 20) + 64;
constexpr int kSampleSegs = 64;           // most vocabulary segments of a partial pass

// partial record of one (row, segment): Gumbel key and id, running max and sum of exp
struct SampleRec {
    float key;
    int id;
    double m;
    double sum;
    double pad;
};
static_assert(sizeof(SampleRec) == 32, "record layout");
// the partial records (at most 2 * 16 - 1 rows) live in the top-K partials' workspace
static_assert((2 * 16 - 1) * kSampleSegs * sizeof(SampleRec) <= (size_t)16 * kTopKSegs * (2 * kTopKMax + 2) * 4,
              "sampling partials exceed their workspace");

// header of the draw workspace, written by segment 0 of the weight-sum launch
struct DrawHdr {
    int k;
    int pad;
    double lp, lq;  // log-sum-exp of the target and draft rows drawn from
    double pad2[5];
};
static_assert(sizeof(DrawHdr) == 64, "header layout");

__device__ __forceinline__ unsigned long long splitmix64(unsigned long long seed, unsigned long long n) {
    unsigned long long z = seed + (n + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// top 24 bits of draw (a, b): the uniform is k * 2^-24 in [0, 1), or (k + 0.5) * 2^-24 in (0, 1)
__device__ __forceinline__ unsigned uniform_bits(unsigned long long seed, unsigned a, unsigned b) {
    return (unsigned)(splitmix64(seed, ((unsigned long long)a << 32) | b) >> 40);
}

// Gumbel perturbation -log(-log U) of U = (k + 0.5) * 2^-24, to about 1e-6
// absolute (keys are compared in fp32), from the hardware base-2 logarithm.
// E = -log U: below 1/2 from U itself; above, U is not an fp32 number (it
// needs 25 bits) while c = 1 - U is, and E = -log(1 - c) is taken from the
// series c + c^2/2 + ... for c <= 2^-6 (relative error below 1e-10 with five
// terms) and from log2(1 - c) otherwise (1 - c rounds by at most 2^-25, under
// 2^-19 of E there).  Every input of a logarithm is a normal number.
__device__ __forceinline__ float gumbel(unsigned k) {
    constexpr float kLn2 = 0.693147180559945309f;
    const float U = ((float)k + 0.5f) * 5.9604644775390625e-08f;                           // exact below 1/2
    const float c = ((float)((1u << 24) - 1u - k) + 0.5f) * 5.9604644775390625e-08f;   // exact above 1/2
    float e;
    if (k < (1u << 23))
        e = -kLn2 * __builtin_amdgcn_logf(U);
    else if (c <= 0.015625f)
        e = c * (1.f + c * (0.5f + c * (0.333333333f + c * (0.25f + c * 0.2f))));
    else
        e = -kLn2 * __builtin_amdgcn_logf(1.f - c);
    return -kLn2 * __builtin_amdgcn_logf(e);
}

__device__ __forceinline__ bool key_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// reductions over aligned groups of `width` lanes
__device__ __forceinline__ double group_max(double v, int width) {
    for (int o = width >> 1; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ double group_sum(double v, int width) {
    for (int o = width >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
// a (max, sum of exp(x - max)) record's sum rescaled to a larger max M
__device__ __forceinline__ double rescaled(double m, double s, double M) { return m == -INFINITY ? 0.0 : s * exp(m - M); }

// One (row, vocabulary segment) per workgroup.  Row r < ra is row r of la,
// else row r - ra of lb.  DRAW: the best Gumbel-perturbed fp32 score z / T +
// G of the segment (ties: lower id).  LSE: the segment's fp64 sum of
// exp(z / T - m) for a reference m: each thread keeps its own, moved up only
// where z / T exceeds it by more than 600 (exp(600) and sums of thousands of
// such terms are finite in fp64), so most ids cost one exponential and no
// rescaling; the threads' sums are rescaled to their largest reference.
template <bool DRAW, bool LSE>
__global__ __launch_bounds__(kSampleThreads) void sample_partial_kernel(const float* la, int ra, const float* lb,
                                                                        long long ld, int V, float invT,
                                                                        double invT64, unsigned long long seed,
                                                                        SampleRec* part) {
    __shared__ float s_k[kSampleThreads / 64];
    __shared__ int s_i[kSampleThreads / 64];
    __shared__ double s_m[kSampleThreads / 64], s_s[kSampleThreads / 64];
    const int seg = blockIdx.x, r = blockIdx.y, S = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int per = (V + S - 1) / S;
    const int beg = seg * per, end = min(V, beg + per);
    const float* z = r < ra ? la + (long long)r * ld : lb + (long long)(r - ra) * ld;
    constexpr int U = 8;
    float bk = -INFINITY;
    int bi = 0x7fffffff;
    double m = -INFINITY, sum = 0.0;
    for (int i0 = beg + tid; i0 < end; i0 += U * kSampleThreads) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kSampleThreads;
            v[u] = i < end ? z[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * kSampleThreads;
            if (i >= end) break;
            if (LSE) {
                const double x = (double)v[u] * invT64;
                if (x > m + 600.0) {  // also the thread's first id (m = -inf); -inf logits add nothing
                    sum = sum * exp(m - x) + 1.0;
                    m = x;
                } else if (x > -INFINITY) {
                    sum += exp(x - m);
                }
            }
            if (DRAW) {
                const float key = v[u] * invT + gumbel(uniform_bits(seed, (unsigned)r, (unsigned)i));
                if (key > bk) {  // ids ascend within a thread: an equal key keeps the lower id
                    bk = key;
                    bi = i;
                }
            }
        }
    }
    if (DRAW) {
        for (int o = 32; o >= 1; o >>= 1) {
            const float k2 = __shfl_xor(bk, o, 64);
            const int i2 = __shfl_xor(bi, o, 64);
            if (key_before(k2, i2, bk, bi)) {
                bk = k2;
                bi = i2;
            }
        }
    }
    if (LSE) {
        const double M = group_max(m, 64);
        sum = group_sum(rescaled(m, sum, M), 64);
        m = M;
    }
    if (lane == 0) {
        s_k[w] = bk;
        s_i[w] = bi;
        s_m[w] = m;
        s_s[w] = sum;
    }
    __syncthreads();
    if (tid == 0) {
        for (int q = 1; q < kSampleThreads / 64; ++q) {
            if (key_before(s_k[q], s_i[q], bk, bi)) {
                bk = s_k[q];
                bi = s_i[q];
            }
        }
        double M = -INFINITY, t = 0.0;
        for (int q = 0; q < kSampleThreads / 64; ++q) M = fmax(M, s_m[q]);
        for (int q = 0; q < kSampleThreads / 64; ++q) t += rescaled(s_m[q], s_s[q], M);
        SampleRec rec;
        rec.key = bk;
        rec.id = bi;
        rec.m = M;
        rec.sum = t;
        rec.pad = 0.0;
        part[(long long)r * S + seg] = rec;
    }
}

// A row's S records merged by an aligned group of 8 lanes (lane `sub` takes
// records sub, sub + 8, ...): the draw is the best key (ties: lower id), the
// lse the records' log-sum-exp (the largest max first, then every record's
// sum rescaled to it).
__device__ __forceinline__ void merge_row(const SampleRec* rec, int S, int sub, int& id, double& lse) {
    float bk = -INFINITY;
    int bi = 0x7fffffff;
    double m = -INFINITY;
    for (int sg = sub; sg < S; sg += 8) {
        const SampleRec q = rec[sg];
        if (key_before(q.key, q.id, bk, bi)) {
            bk = q.key;
            bi = q.id;
        }
        m = fmax(m, q.m);
    }
    for (int o = 4; o >= 1; o >>= 1) {
        const float k2 = __shfl_xor(bk, o, 64);
        const int i2 = __shfl_xor(bi, o, 64);
        if (key_before(k2, i2, bk, bi)) {
            bk = k2;
            bi = i2;
        }
    }
    const double M = group_max(m, 8);
    double s = 0.0;
    for (int sg = sub; sg < S; sg += 8) s += rescaled(rec[sg].m, rec[sg].sum, M);
    s = group_sum(s, 8);
    id = bi;
    lse = M + log(s);
}

// 8 rows per workgroup of 64 threads.
__global__ __launch_bounds__(64) void sample_merge_kernel(const SampleRec* part, int S, int R, int32_t* tokens,
                                                          float* lse) {
    const int r = blockIdx.x * 8 + (threadIdx.x >> 3), sub = threadIdx.x & 7;
    if (r >= R) return;  // whole groups of 8 lanes leave together
    int id;
    double l;
    merge_row(part + (long long)r * S, S, sub, id, l);
    if (sub == 0) {
        if (tokens) tokens[r] = id;
        if (lse) lse[r] = (float)l;
    }
}

struct VerifyArgs {
    const int32_t* draft;
    const float* dlog;  // draft logits, row j gave draft j
    const float* tlog;  // target logits, row i predicts position C + i + 1
    long long ld;
    int V, B, S;        // S: lse partial segments per row
    double invT;
    unsigned long long seed;
    const SampleRec* part;  // [B target rows, then draft rows 1 .. B-1][S]
    DrawHdr* hdr;
    double* seg_sum;        // [ceil(V / kDrawSeg)]
    int32_t* out;
};

// weight of id x in the draw: p(x), or max(0, p(x) - q(x)) after a rejection
__device__ __forceinline__ double draw_weight(const float* zp, const float* zq, double invT, double lp, double lq,
                                              bool resid, int x) {
    const double p = exp((double)zp[x] * invT - lp);
    return resid ? fmax(0.0, p - exp((double)zq[x] * invT - lq)) : p;
}

// Launch 2: one workgroup per kDrawSeg ids.
__global__ __launch_bounds__(kDrawThreads) void verify_weights_kernel(VerifyArgs a) {
    __shared__ double s_lse[32];
    __shared__ int s_ok[16];
    __shared__ double s_red[kDrawThreads / 64];
    const int tid = threadIdx.x, B = a.B;
    const int R = 2 * B - 1;
    // the acceptance test's logits, loaded while the row lse values merge
    float zt_j = 0.f, zd_j = 0.f;
    const bool tester = tid >= 1 && tid < B;  // thread j tests draft j
    if (tester) {
        const int dj = min(max(a.draft[tid], 0), a.V - 1);
        zt_j = a.tlog[(long long)(tid - 1) * a.ld + dj];
        zd_j = a.dlog[(long long)tid * a.ld + dj];
    }
    {  // row lse (target rows 0 .. B-1, then draft rows 1 .. B-1): 8 lanes per row
        const int r = tid >> 3, sub = tid & 7;
        if (r < R) {  // whole groups of 8 lanes take the same branch
            int id;
            double l;
            merge_row(a.part + (long long)r * a.S, a.S, sub, id, l);
            if (sub == 0) s_lse[r] = l;
        }
    }
    __syncthreads();
    if (tester) {
        const int j = tid;
        const double p = exp((double)zt_j * a.invT - s_lse[j - 1]);
        const double q = exp((double)zd_j * a.invT - s_lse[B + j - 1]);
        const double u = (double)uniform_bits(a.seed, (unsigned)(kTagAccept + j), 0u) * 5.9604644775390625e-08;
        s_ok[j] = u * q < p;
    }
    __syncthreads();
    int k = B - 1;
    for (int j = 1; j < B; ++j)
        if (!s_ok[j]) {
            k = j - 1;
            break;
        }
    const bool resid = k < B - 1;
    const int prow = resid ? k : B - 1;  // target row of the drawn position
    const float* zp = a.tlog + (long long)prow * a.ld;
    const float* zq = a.dlog + (long long)(resid ? k + 1 : 0) * a.ld;  // draft row k + 1, read only after a rejection
    const double lp = s_lse[prow], lq = resid ? s_lse[B + k] : 0.0;
    const int beg = blockIdx.x * kDrawSeg, end = min(a.V, beg + kDrawSeg);
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < kDrawSeg / kDrawThreads; ++i) {
        const int x = beg + tid + i * kDrawThreads;
        if (x < end) acc += draw_weight(zp, zq, a.invT, lp, lq, resid, x);
    }
    acc = group_sum(acc, 64);
    if ((tid & 63) == 0) s_red[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
        double t = 0.0;
        for (int q = 0; q < kDrawThreads / 64; ++q) t += s_red[q];
        a.seg_sum[blockIdx.x] = t;
        if (blockIdx.x == 0) {
            DrawHdr h{};
            h.k = k;
            h.lp = lp;
            h.lq = lq;
            *a.hdr = h;
        }
    }
}

// lane l's value of a wave-uniform read
__device__ __forceinline__ double readlane_f64(double v, int l) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, l);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), l);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Running sums of the wave's 64 values in lane order, added one at a time
// (so they never decrease): returns this lane's exclusive prefix; total gets
// the sum of all 64.  Every lane computes the same sequence.
__device__ __forceinline__ double wave_prefix_seq(double v, int lane, double& total) {
    double run = 0.0, mine = 0.0;
    for (int l = 0; l < 64; ++l) {
        if (l == lane) mine = run;
        run += readlane_f64(v, l);
    }
    total = run;
    return mine;
}

// lowest lane whose flag is set (-1 if none), and the highest
__device__ __forceinline__ int first_lane(bool f) {
    const unsigned long long m = __ballot(f);
    return m ? __ffsll((long long)m) - 1 : -1;
}
__device__ __forceinline__ int last_lane(bool f) {
    const unsigned long long m = __ballot(f);
    return m ? 63 - __clzll((long long)m) : -1;
}

// Launch 3: the draw, one workgroup.  Every level scans its parts in id order
// with running sums that never decrease: segments (lane l of wave 0 sums its
// run of consecutive segments, the lanes' sums are prefixed in lane order, the
// chosen lane walks its run), then the chosen segment's ids (each thread sums
// its 4 consecutive ids, each wave prefixes its lanes, the 4 waves are
// prefixed in order, the chosen lane walks its 4 ids).  Where rounding leaves
// the target past a level's parts, the last part of positive weight is taken.
__global__ __launch_bounds__(kDrawThreads) void verify_draw_kernel(VerifyArgs a) {
    constexpr int per = kDrawSeg / kDrawThreads;
    __shared__ double s_target;
    __shared__ int s_seg;
    __shared__ double s_wtot[kDrawThreads / 64];
    __shared__ int s_wlast[kDrawThreads / 64];
    __shared__ int s_tok;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const DrawHdr h = *a.hdr;
    const int k = h.k, B = a.B;
    const bool resid = k < B - 1;
    const int nseg = (a.V + kDrawSeg - 1) / kDrawSeg;
    const double u = (double)uniform_bits(a.seed, (unsigned)kTagResidual, 0u) * 5.9604644775390625e-08;
    if (wv == 0) {
        const int c = (nseg + 63) / 64;  // consecutive segments per lane
        const int s0 = min(nseg, lane * c), s1 = min(nseg, s0 + c);
        double v = 0.0;
        for (int sg = s0; sg < s1; ++sg) v += a.seg_sum[sg];
        double total;
        const double pre = wave_prefix_seq(v, lane, total);
        const double target = u * total;
        int L = first_lane(pre + v > target);
        const bool fallback = L < 0;
        if (fallback) L = last_lane(v > 0.0);  // rounding left the target past every lane
        if (L < 0) L = 0;                      // no positive weight anywhere (cannot happen for finite logits)
        if (lane == L) {
            double run = pre, at = pre, at_last = pre;
            int seg = -1, lastpos = -1;
            for (int sg = s0; sg < s1 && seg < 0; ++sg) {
                const double w = a.seg_sum[sg];
                if (w > 0.0) {
                    lastpos = sg;
                    at_last = run;
                }
                if (!fallback && run + w > target) {
                    seg = sg;
                    at = run;
                } else {
                    run += w;
                }
            }
            if (seg < 0) {  // the target lies past the lane's own sums: its last segment of positive weight
                seg = lastpos >= 0 ? lastpos : s0;
                at = lastpos >= 0 ? at_last : pre;
            }
            s_seg = min(max(seg, 0), nseg - 1);
            s_target = target - at;  // measured from the segment's start
        }
    }
    __syncthreads();
    const int prow = resid ? k : B - 1;
    const float* zp = a.tlog + (long long)prow * a.ld;
    const float* zq = a.dlog + (long long)(resid ? k + 1 : 0) * a.ld;
    const int beg = s_seg * kDrawSeg, n = min(a.V - beg, kDrawSeg);
    double w[per];
    double v = 0.0;
    int mylast = -1;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        const int x = tid * per + i;
        w[i] = x < n ? draw_weight(zp, zq, a.invT, h.lp, h.lq, resid, beg + x) : 0.0;
        v += w[i];
        if (w[i] > 0.0) mylast = x;
    }
    double wtot;
    const double pre = wave_prefix_seq(v, lane, wtot);
    int wl = mylast;
    for (int o = 32; o >= 1; o >>= 1) wl = max(wl, __shfl_xor(wl, o, 64));
    if (lane == 0) {
        s_wtot[wv] = wtot;
        s_wlast[wv] = wl;
    }
    __syncthreads();
    // every thread reads the same wave totals: the wave that holds the target
    int seglast = -1;
    for (int q = 0; q < kDrawThreads / 64; ++q) seglast = max(seglast, s_wlast[q]);
    double target = s_target, run = 0.0;
    int W = -1;
    for (int q = 0; q < kDrawThreads / 64; ++q) {
        if (W < 0 && run + s_wtot[q] > target) W = q;
        if (W < 0) run += s_wtot[q];
    }
    if (tid == 0) s_tok = seglast >= 0 ? seglast : 0;
    __syncthreads();
    if (W == wv) {
        const double t = target - run;
        const int L = first_lane(pre + v > t);
        if (lane == L) {
            double r = pre;
            for (int i = 0; i < per; ++i) {
                r += w[i];
                if (r > t) {
                    s_tok = tid * per + i;
                    break;
                }
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        a.out[0] = k;
        a.out[1] = beg + s_tok;
    }
}

}  // namespace

// vocabulary segments of a partial pass: about 2048 ids each, at most kSampleSegs
static int sample_segs(int V) { return std::max(1, std::min(kSampleSegs, V / 2048)); }

hipError_t launch_sample_tokens(const DevCtx& c, const float* logits, long long ld, int rows, float T,
                                unsigned long long seed, int32_t* tokens, float* lse, hipStream_t s) {
    const int V = c.dm.V;
    const int S = sample_segs(V);
    SampleRec* part = reinterpret_cast<SampleRec*>(c.ws + c.lay.topk_part);
    if (tokens && lse)
        hipLaunchKernelGGL((sample_partial_kernel<true, true>), dim3(S, rows), dim3(kSampleThreads), 0, s, logits,
                           rows, logits, ld, V, 1.0f / T, 1.0 / (double)T, seed, part);
    else if (tokens)
        hipLaunchKernelGGL((sample_partial_kernel<true, false>), dim3(S, rows), dim3(kSampleThreads), 0, s, logits,
                           rows, logits, ld, V, 1.0f / T, 1.0 / (double)T, seed, part);
    else
        hipLaunchKernelGGL((sample_partial_kernel<false, true>), dim3(S, rows), dim3(kSampleThreads), 0, s, logits,
                           rows, logits, ld, V, 1.0f / T, 1.0 / (double)T, seed, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sample_merge_kernel, dim3((rows + 7) / 8), dim3(64), 0, s, part, S, rows, tokens, lse);
    return hipGetLastError();
}

hipError_t launch_verify_sample(const DevCtx& c, const int32_t* draft, const float* dlog, const float* tlog,
                                long long ld, float T, unsigned long long seed, int32_t* out, hipStream_t s) {
    VerifyArgs a;
    a.draft = draft;
    a.dlog = dlog;
    a.tlog = tlog;
    a.ld = ld;
    a.V = c.dm.V;
    a.B = c.dm.B;
    a.S = sample_segs(a.V);
    a.invT = 1.0 / (double)T;
    a.seed = seed;
    a.part = reinterpret_cast<const SampleRec*>(c.ws + c.lay.topk_part);
    a.hdr = reinterpret_cast<DrawHdr*>(c.ws + c.lay.sample_draw);
    a.seg_sum = reinterpret_cast<double*>(c.ws + c.lay.sample_draw + sizeof(DrawHdr));
    a.out = out;
    // log-sum-exp partials of the B target rows and of draft rows 1 .. B-1
    hipLaunchKernelGGL((sample_partial_kernel<false, true>), dim3(a.S, 2 * a.B - 1), dim3(kSampleThreads), 0, s,
                       tlog, a.B, dlog + ld, ld, a.V, 1.0f / T, a.invT, seed,
                       reinterpret_cast<SampleRec*>(c.ws + c.lay.topk_part));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nseg = (a.V + kDrawSeg - 1) / kDrawSeg;
    hipLaunchKernelGGL(verify_weights_kernel, dim3(nseg), dim3(kDrawThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(verify_draw_kernel, dim3(1), dim3(kDrawThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace dflash

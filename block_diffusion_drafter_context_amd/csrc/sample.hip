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
// Precision.  Gumbel keys are fp32 (a draw flips only where two keys lie
// within fp32 rounding).  The verification works in fp64 from the fp32
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

// partial record of one (row, segment): Gumbel key and id, running max and sum of exp
struct SampleRec {
    float key;
    int id;
    double m;
    double sum;
    double pad;
};
static_assert(sizeof(SampleRec) == 32, "record layout");

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

__device__ __forceinline__ bool key_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ void lse_add(double& m, double& s, double m2, double s2) {
    if (m2 == -INFINITY) return;
    if (m == -INFINITY) {
        m = m2;
        s = s2;
        return;
    }
    const double M = fmax(m, m2);
    s = s * exp(m - M) + s2 * exp(m2 - M);
    m = M;
}

// One (row, vocabulary segment) per workgroup.  Row r < ra is row r of la,
// else row r - ra of lb.  Every thread scans its ids in ascending order,
// keeping the best Gumbel-perturbed fp32 score (when `draw`) and a running
// fp64 (max, sum of exp) of z / T; the workgroup reduces both.
__global__ __launch_bounds__(kSampleThreads) void sample_partial_kernel(const float* la, int ra, const float* lb,
                                                                        long long ld, int V, float invT,
                                                                        double invT64, unsigned long long seed,
                                                                        int draw, SampleRec* part) {
    __shared__ float s_k[kSampleThreads / 64];
    __shared__ int s_i[kSampleThreads / 64];
    __shared__ double s_m[kSampleThreads / 64], s_s[kSampleThreads / 64];
    const int seg = blockIdx.x, r = blockIdx.y, S = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int per = (V + S - 1) / S;
    const int beg = seg * per, end = min(V, beg + per);
    const float* z = r < ra ? la + (long long)r * ld : lb + (long long)(r - ra) * ld;
    float bk = -INFINITY;
    int bi = 0x7fffffff;
    double m = -INFINITY, sum = 0.0;
    constexpr int U = 8;
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
            const double x = (double)v[u] * invT64;
            if (x > m) {
                sum = sum * exp(m - x) + 1.0;
                m = x;
            } else {
                sum += exp(x - m);
            }
            if (draw) {
                const float uo = ((float)uniform_bits(seed, (unsigned)r, (unsigned)i) + 0.5f) * 5.9604644775390625e-08f;
                const float key = v[u] * invT - logf(-logf(uo));
                if (key > bk) {  // ids ascend within a thread: an equal key keeps the lower id
                    bk = key;
                    bi = i;
                }
            }
        }
    }
    for (int o = 32; o >= 1; o >>= 1) {
        const float k2 = __shfl_xor(bk, o, 64);
        const int i2 = __shfl_xor(bi, o, 64);
        const double m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(sum, o, 64);
        if (key_before(k2, i2, bk, bi)) {
            bk = k2;
            bi = i2;
        }
        // both lanes of a pair combine in the same operand order (lower lane first)
        if (lane & o) {
            double mm = m2, ss = s2;
            lse_add(mm, ss, m, sum);
            m = mm;
            sum = ss;
        } else {
            lse_add(m, sum, m2, s2);
        }
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
            lse_add(m, sum, s_m[q], s_s[q]);
        }
        SampleRec rec;
        rec.key = bk;
        rec.id = bi;
        rec.m = m;
        rec.sum = sum;
        rec.pad = 0.0;
        part[(long long)r * S + seg] = rec;
    }
}

// One thread per row: the segments' records in segment order.
__global__ __launch_bounds__(64) void sample_merge_kernel(const SampleRec* part, int S, int R, int32_t* tokens,
                                                          float* lse) {
    const int r = threadIdx.x;
    if (r >= R) return;
    float bk = -INFINITY;
    int bi = 0x7fffffff;
    double m = -INFINITY, sum = 0.0;
    for (int sg = 0; sg < S; ++sg) {
        const SampleRec q = part[(long long)r * S + sg];
        if (key_before(q.key, q.id, bk, bi)) {
            bk = q.key;
            bi = q.id;
        }
        lse_add(m, sum, q.m, q.sum);
    }
    if (tokens) tokens[r] = bi;
    if (lse) lse[r] = (float)(m + log(sum));
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
    if (tid < R) {  // row lse: target rows 0 .. B-1, then draft rows 1 .. B-1
        double m = -INFINITY, s = 0.0;
        for (int sg = 0; sg < a.S; ++sg) {
            const SampleRec q = a.part[(long long)tid * a.S + sg];
            lse_add(m, s, q.m, q.sum);
        }
        s_lse[tid] = m + log(s);
    }
    __syncthreads();
    if (tid >= 1 && tid < B) {  // the acceptance test of draft j = tid
        const int j = tid;
        const int dj = min(max(a.draft[j], 0), a.V - 1);
        const double p = exp((double)a.tlog[(long long)(j - 1) * a.ld + dj] * a.invT - s_lse[j - 1]);
        const double q = exp((double)a.dlog[(long long)j * a.ld + dj] * a.invT - s_lse[B + j - 1]);
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
    for (int x = beg + tid; x < end; x += kDrawThreads) acc += draw_weight(zp, zq, a.invT, lp, lq, resid, x);
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
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

// Launch 3: the draw.  Levels: segment (thread 0 over the segment sums),
// wave (each thread sums its 4 consecutive ids, lane 0 of each wave its 64
// lanes, thread 0 scans the 4 waves), lane (the chosen wave's lane 0 scans its
// lanes) and id (the same thread walks the chosen lane's 4 ids).
__global__ __launch_bounds__(kDrawThreads) void verify_draw_kernel(VerifyArgs a) {
    __shared__ double s_w[kDrawSeg];
    __shared__ double s_t[kDrawThreads];
    __shared__ double s_wave[kDrawThreads / 64];
    __shared__ double s_target;
    __shared__ int s_seg, s_wv, s_tok;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const DrawHdr h = *a.hdr;
    const int k = h.k, B = a.B;
    const bool resid = k < B - 1;
    const int nseg = (a.V + kDrawSeg - 1) / kDrawSeg;
    const double u = (double)uniform_bits(a.seed, (unsigned)kTagResidual, 0u) * 5.9604644775390625e-08;
    if (tid == 0) {
        double run = 0.0;
        for (int sg = 0; sg < nseg; ++sg) run += a.seg_sum[sg];
        const double target = u * run;
        double pre = 0.0;
        int seg = -1, last = 0;
        for (int sg = 0; sg < nseg; ++sg) {
            const double w = a.seg_sum[sg];
            if (w > 0.0) last = sg;
            if (seg < 0 && pre + w > target) seg = sg;
            if (seg < 0) pre += w;
        }
        if (seg < 0) {  // rounding left the target past every segment: the last one of positive weight
            seg = last;
            pre = 0.0;
            for (int sg = 0; sg < seg; ++sg) pre += a.seg_sum[sg];
        }
        s_seg = seg;
        s_target = target - pre;  // the target measured from the segment's start
    }
    __syncthreads();
    const int prow = resid ? k : B - 1;
    const float* zp = a.tlog + (long long)prow * a.ld;
    const float* zq = a.dlog + (long long)(resid ? k + 1 : 0) * a.ld;
    const int beg = s_seg * kDrawSeg, n = min(a.V - beg, kDrawSeg);
    for (int i = tid; i < kDrawSeg; i += kDrawThreads)
        s_w[i] = i < n ? draw_weight(zp, zq, a.invT, h.lp, h.lq, resid, beg + i) : 0.0;
    __syncthreads();
    constexpr int per = kDrawSeg / kDrawThreads;
    double ts = 0.0;
#pragma unroll
    for (int i = 0; i < per; ++i) ts += s_w[tid * per + i];
    s_t[tid] = ts;
    __syncthreads();
    if (lane == 0) {
        double ws = 0.0;
        for (int l = 0; l < 64; ++l) ws += s_t[wv * 64 + l];
        s_wave[wv] = ws;
    }
    __syncthreads();
    if (tid == 0) {
        // the last id of positive weight in the segment: the answer whenever a
        // level's parts leave the target behind
        int lastid = 0;
        for (int i = n - 1; i >= 0; --i)
            if (s_w[i] > 0.0) {
                lastid = i;
                break;
            }
        s_tok = lastid;
        double pre = 0.0;
        int pick = -1;
        for (int q = 0; q < kDrawThreads / 64; ++q) {
            if (pre + s_wave[q] > s_target) {
                pick = q;
                break;
            }
            pre += s_wave[q];
        }
        s_wv = pick;
        s_target -= pick >= 0 ? pre : 0.0;
    }
    __syncthreads();
    if (s_wv == wv && lane == 0) {
        const double target = s_target;
        double pre = 0.0;
        for (int l = 0; l < 64; ++l) {
            const int t = wv * 64 + l;
            if (pre + s_t[t] > target) {
                double run = pre;
                for (int i = 0; i < per; ++i) {
                    run += s_w[t * per + i];
                    if (run > target) {
                        s_tok = t * per + i;
                        break;
                    }
                }
                break;
            }
            pre += s_t[t];
        }
    }
    __syncthreads();
    if (tid == 0) {
        a.out[0] = k;
        a.out[1] = beg + s_tok;
    }
}

}  // namespace

hipError_t launch_sample_tokens(const DevCtx& c, const float* logits, long long ld, int rows, float T,
                                unsigned long long seed, int32_t* tokens, float* lse, hipStream_t s) {
    const int V = c.dm.V;
    const int S = std::max(1, std::min(kTopKSegs, V / 4096));
    SampleRec* part = reinterpret_cast<SampleRec*>(c.ws + c.lay.topk_part);
    hipLaunchKernelGGL(sample_partial_kernel, dim3(S, rows), dim3(kSampleThreads), 0, s, logits, rows, logits, ld,
                       V, 1.0f / T, 1.0 / (double)T, seed, 1, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sample_merge_kernel, dim3(1), dim3(64), 0, s, part, S, rows, tokens, lse);
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
    a.S = std::max(1, std::min(kTopKSegs, a.V / 4096));
    a.invT = 1.0 / (double)T;
    a.seed = seed;
    a.part = reinterpret_cast<const SampleRec*>(c.ws + c.lay.topk_part);
    a.hdr = reinterpret_cast<DrawHdr*>(c.ws + c.lay.sample_draw);
    a.seg_sum = reinterpret_cast<double*>(c.ws + c.lay.sample_draw + sizeof(DrawHdr));
    a.out = out;
    // log-sum-exp partials of the B target rows and of draft rows 1 .. B-1
    hipLaunchKernelGGL(sample_partial_kernel, dim3(a.S, 2 * a.B - 1), dim3(kSampleThreads), 0, s, tlog, a.B,
                       dlog + ld, ld, a.V, 1.0f / T, a.invT, seed, 0,
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

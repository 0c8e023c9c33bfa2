// device_common.h -- element types, conversions and MFMA fragments for gfx950.
//
// Storage types: float (fp32) and bf16 held as uint16_t bit patterns.
// Matrix-core fragments follow the 16x16 MFMA operand layout of CDNA:
//   A (16 x 32, row m, reduction k):  lane l holds row m = l % 16 and the eight
//                                     reduction slots of lane group g = l / 16;
//   B (32 x 16, reduction k, col n):  lane l holds col n = l % 16, same slots;
//   D (16 x 16 fp32):                 lane l holds rows 4*(l/16) + i, i = 0..3,
//                                     of column l % 16.
// The hardware pairs A and B by (lane group, slot), so any fixed assignment of
// the 32 reduction indices to (group, slot) that both operands share gives the
// full dot product.  We use k = 8*g + slot unless a kernel says otherwise.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// round-to-nearest-even fp32 -> bf16 (the hardware conversion, v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
// two values in one conversion: a in the low half, b in the high half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float to_f32(float v) { return v; }
    __device__ __forceinline__ static float from_f32(float v) { return v; }
    __device__ __forceinline__ static float round(float v) { return v; }
};
template <> struct Elem<bf16_t> {
    __device__ __forceinline__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
    __device__ __forceinline__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
    __device__ __forceinline__ static float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// Eight consecutive reduction elements of one row: one MFMA operand slot set.
template <typename T> struct Frag;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));

template <> struct Frag<bf16_t> {
    uint4 v;
    __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
    // streaming load (non-temporal hint): data read once per pass, e.g. weights
    __device__ __forceinline__ void load_nt(const bf16_t* p) {
        const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        v = make_uint4(t[0], t[1], t[2], t[3]);
    }
    // one lane's slot set of a swizzled 512-element block (see host.h)
    __device__ __forceinline__ void load_sw(const bf16_t* block, int lane) { load_nt(block + lane * 8); }
    // keep (m = ~0u) or clear (m = 0) all elements without a branch
    __device__ __forceinline__ void mask(uint32_t m) {
        v.x &= m;
        v.y &= m;
        v.z &= m;
        v.w &= m;
    }
    __device__ __forceinline__ float get(int i) const {
        uint32_t w = (&v.x)[i >> 1];
        return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
    __device__ __forceinline__ void set8(const float* f) {
        v = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
    }
};
template <> struct Frag<float> {
    float4 a, b;
    __device__ __forceinline__ void zero() { a = make_float4(0, 0, 0, 0); b = a; }
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    __device__ __forceinline__ void load_nt(const float* p) {
        const f32x4v_t x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(p));
        const f32x4v_t y = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(p + 4));
        a = make_float4(x[0], x[1], x[2], x[3]);
        b = make_float4(y[0], y[1], y[2], y[3]);
    }
    __device__ __forceinline__ void load_sw(const float* block, int lane) {
        const f32x4v_t x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(block + lane * 4));
        const f32x4v_t y = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(block + 256 + lane * 4));
        a = make_float4(x[0], x[1], x[2], x[3]);
        b = make_float4(y[0], y[1], y[2], y[3]);
    }
    __device__ __forceinline__ void mask(uint32_t m) {
        a.x = __uint_as_float(__float_as_uint(a.x) & m);
        a.y = __uint_as_float(__float_as_uint(a.y) & m);
        a.z = __uint_as_float(__float_as_uint(a.z) & m);
        a.w = __uint_as_float(__float_as_uint(a.w) & m);
        b.x = __uint_as_float(__float_as_uint(b.x) & m);
        b.y = __uint_as_float(__float_as_uint(b.y) & m);
        b.z = __uint_as_float(__float_as_uint(b.z) & m);
        b.w = __uint_as_float(__float_as_uint(b.w) & m);
    }
    __device__ __forceinline__ float get(int i) const { return i < 4 ? (&a.x)[i] : (&b.x)[i - 4]; }
    __device__ __forceinline__ void set8(const float* f) {
        a = make_float4(f[0], f[1], f[2], f[3]);
        b = make_float4(f[4], f[5], f[6], f[7]);
    }
};

// acc (16x16) += A(16x32) * B(32x16)
__device__ __forceinline__ void mma(f32x4_t& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v), __builtin_bit_cast(bf16x8_t, b.v),
                                                  acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4_t& acc, const Frag<float>& a, const Frag<float>& b) {
    // slot s of every lane group forms one 16x16x4 fp32 product
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.x, b.a.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.y, b.a.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.z, b.a.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.w, b.a.w, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.x, b.b.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.y, b.b.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.z, b.b.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.w, b.b.w, acc, 0, 0, 0);
}

// Device-coherent (agent scope) accesses for data one workgroup hands to
// another inside a kernel.  They carry the scope bits that make the access
// coherent across the XCDs' L2s, so no L2 writeback / invalidate fence is
// needed; wait_vmem() orders them before a following atomic.
__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// sum / max over the 16 lanes that share a lane group (same l / 16)
__device__ __forceinline__ float group16_sum(float v) {
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    v += __shfl_xor(v, 8, 64);
    return v;
}
__device__ __forceinline__ float group16_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 1, 64));
    v = fmaxf(v, __shfl_xor(v, 2, 64));
    v = fmaxf(v, __shfl_xor(v, 4, 64));
    v = fmaxf(v, __shfl_xor(v, 8, 64));
    return v;
}
// reduce across the 4 lane groups (lanes l, l^16, l^32, l^48)
// Workgroup barrier for pipelines that feed LDS with direct global->LDS loads.
// __syncthreads() also fences memory, which drains every outstanding global
// load (vmcnt(0)) and with it the prefetched stages; here the caller has
// already waited (vmcnt) for exactly the loads the next step needs.  This
// wave's LDS reads are complete (lgkmcnt(0)) before it arrives, so a stage
// refilled after the barrier is no longer being read; the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wait states after a run of MFMAs, before control flow can branch away.
// hipcc for gfx950 (ROCm 7.2) pads a read of an MFMA result with the wait
// states the hardware needs (8 for a 16x16x32 bf16 result read by a VALU or
// v_accvgpr_read in straight-line code), but on a path that enters a join
// block through a taken branch it can leave them out when the join block has
// another predecessor whose path is longer: the read then sees the accumulator
// from before the MFMA.  16 explicit wait states cover every MFMA used here,
// so no path leaving the MFMA run depends on the compiler's padding.  (A
// compile-only reproducer is csrc/repro/mfma_join_hazard.hip.)
__device__ __forceinline__ void mfma_settle() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7" ::);
    __builtin_amdgcn_sched_barrier(0);
}

// The pair (lane l, lane l ^ 16) and (lane l, lane l ^ 32) exchanges as VALU
// row swaps (gfx950 v_permlane16_swap / v_permlane32_swap) instead of LDS
// crossbar shuffles: swapping a register with itself leaves, in every lane, the
// lower-row value in the first result and the upper-row value in the second,
// so both lanes of a pair form the same sum (lower + upper) or max.
__device__ __forceinline__ float xor16_pair(float v, bool max_op) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
    return max_op ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float xor32_pair(float v, bool max_op) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
    return max_op ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float cross4_max(float v) { return xor32_pair(xor16_pair(v, true), true); }
__device__ __forceinline__ float cross4_sum(float v) { return xor32_pair(xor16_pair(v, false), false); }

}  // namespace dflash

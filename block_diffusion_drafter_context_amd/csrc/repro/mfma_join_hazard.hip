// mfma_join_hazard.hip -- compile-only reproducer of a missing MFMA wait state
// in hipcc for gfx950 (ROCm 7.2).  Not part of libdflash and never run.
//
//   hipcc --offload-arch=gfx950 -O3 --cuda-device-only -S mfma_join_hazard.hip -o - \
//     | sed -n '/^_Z11branch_last/,/s_endpgm/p'
//
// straight_last: the compiler puts 8 wait states ("s_nop 7") between the MFMA
// that writes a[0:3] and the v_accvgpr_read of a3: what the hardware needs
// before a 16x16x32 bf16 result can be read.
//
// branch_last: the loop's MFMA block branches to a join block (the loop
// latch), which is also reached from the block that stores and clears the
// accumulator.  On the taken-branch path the latch reads a3 with
// v_accvgpr_read only 5 instructions after the MFMA and no s_nop: the padding
// is left out on the short path when the join block has a longer predecessor
// path, so the read can see a3 from before the MFMA.  In libdflash's split-K
// GEMM this pattern (accumulator copies out of AGPRs right after the tile-end
// branch) gave wrong logits; mfma_settle() in device_common.h pads every MFMA
// run explicitly.
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64, 1) void straight_last(const bf16x8* a, const bf16x8* b, float* out) {
    const int l = threadIdx.x;
    f32x4 acc = {0, 0, 0, 0};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[l], b[l], acc, 0, 0, 0);
    out[l] = acc[3] * 3.0f;
}

__global__ __launch_bounds__(64, 1) void branch_last(const bf16x8* a, const bf16x8* b, float* out, int n) {
    const int l = threadIdx.x;
    f32x4 acc = {0, 0, 0, 0};
    for (int i = 0; i < n; ++i) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[l + 64 * i], b[l + 64 * i], acc, 0, 0, 0);
        if (i == n / 2) {
            out[64 + l] = acc[0];
            acc = f32x4{0, 0, 0, 0};
        }
        asm volatile("; use %0" ::"v"(acc[3]));
    }
    out[l] = acc[3];
}

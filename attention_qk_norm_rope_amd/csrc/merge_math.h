// Per-row arithmetic of the two-way out/LSE merge, shared by attn_merge_kernel
// and the merging epilogue of the attention kernel so that both give the same
// bits.  "NPU Wan2.2-I2V模型推理优化实践", Ring Attention Overlap, and
// "feat: support Ascend NPU backend (torch_npu) for Qwen-Image pipelines -
// #274", change list item 2 (update_out_and_lse):
//   M = max(la, lb),  ea = exp(la - M), eb = exp(lb - M),
//   L = M + ln(ea + eb),  out <- (ea out_a + eb out_b) / (ea + eb).
// No contraction into fma: the result does not depend on the caller's code.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace dit {
namespace mg {

// Weights of the two sides and the merged LSE.  Both LSEs -inf: weights 0,
// L = -inf.
__device__ __forceinline__ void weights(float la, float lb, float& wa, float& wb, float& L) {
#pragma clang fp contract(off)
    const float M = fmaxf(la, lb);
    wa = 0.f;
    wb = 0.f;
    L = -INFINITY;
    if (M != -INFINITY) {
        const float ea = expf(la - M), eb = expf(lb - M);
        const float den = ea + eb;
        L = M + logf(den);
        wa = ea / den;
        wb = eb / den;
    }
}

// One element.  A side with weight 0 saw no key: its value is not read into
// the result (it may be anything, even NaN).
__device__ __forceinline__ float combine(float wa, float a, float wb, float b) {
#pragma clang fp contract(off)
    const float ta = wa != 0.f ? wa * a : 0.f;
    const float tb = wb != 0.f ? wb * b : 0.f;
    return ta + tb;
}

}  // namespace mg
}  // namespace dit

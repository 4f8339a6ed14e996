// Per-element arithmetic of the per-head RMSNorm + interleaved rotary, shared
// by qk_norm_rope_kernel and the fused-Q attention kernel so that both give
// the same bits.  Operation: RMSNorm of "Cosmos 昇腾 NPU 多卡并行优化说明" §3.2
// (mean of squares over the head dimension, plus eps, reciprocal square
// root, times the weight) and the interleaved rotary of its §3.3 (adjacent
// pairs, tables taken elementwise).  Every rounding step is written out
// (explicit fma, no contraction left to the compiler).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {
namespace nr {

typedef float nr_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 nr_bf16x2 __attribute__((ext_vector_type(2)));

// The 8 bf16 values of a 16-byte chunk as fp32 (element 2i from the low half
// of dword i).
__device__ __forceinline__ void unpack8(const unsigned (&w)[4], float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
        x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
}

// Sum of squares of one 8-element chunk, in element order.
__device__ __forceinline__ float chunk_sumsq(const float (&x)[8]) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(x[i], x[i], ss);
    return ss;
}

// 1 / sqrt(mean square + eps) from the row's sum of squares.  The chunk
// sums of a row (D/8 of them) are always combined as an xor tree: pairs of
// chunks D/16 apart first, then D/32 apart, ..., then neighbours.
__device__ __forceinline__ float rms_inv(float ss, float inv_d, float eps) {
    return 1.0f / sqrtf(__builtin_fmaf(ss, inv_d, eps));
}

// Normalise, weight and rotate one pair (2i, 2i+1); returns the two results
// packed as bf16 (round to nearest even), element 2i in the low half.
__device__ __forceinline__ unsigned pair(float xa, float xb, float inv_r, float wa, float wb, float ca, float cb,
                                         float sa, float sb) {
    const float ya = (xa * inv_r) * wa;
    const float yb = (xb * inv_r) * wb;
    const float za = __builtin_fmaf(ya, ca, -(yb * sa));
    const float zb = __builtin_fmaf(yb, cb, ya * sb);
    nr_f32x2 f = {za, zb};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, nr_bf16x2));
}

}  // namespace nr
}  // namespace dit

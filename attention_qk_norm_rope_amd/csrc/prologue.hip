// Per-head RMSNorm + interleaved rotary embedding of q and k, in place, for
// gfx950.  HBM-bound: one 16-byte read and one 16-byte write per 8 elements.
//
// Operation: RMSNorm of "Cosmos 昇腾 NPU 多卡并行优化说明" §3.2 and the rms_norm
// section of "NPU Wan2.2-I2V模型推理优化实践" (mean of squares over the head
// dimension, plus eps, reciprocal square root, times the weight), then the
// interleaved rotary of Cosmos §3.3 / the Wan2.2 rotary_mul section (pairs
// (2i, 2i+1), tables taken elementwise).  fp32 arithmetic, one rounding to
// bf16 at the end.
//
// Layout: D/8 consecutive lanes own one (b,h,s) row, 8 elements each, so a
// wave streams 4 (D=128) or 8 (D=64) rows of 256/128 contiguous bytes.  The
// sum of squares is reduced across those lanes with xor shuffles.  The
// weight slice of a lane is loaded once; the cos/sin rows are shared by all
// (b,h) and stay in L2.  blockIdx.y selects q (0) or k (1).
#include "internal.h"

namespace dit {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    f32x2 f = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

template <int D>
__global__ void __launch_bounds__(256)
qk_norm_rope_kernel(uint16_t* __restrict__ q, uint16_t* __restrict__ k, const float* __restrict__ w_q,
                    const float* __restrict__ w_k, const float* __restrict__ cos_t,
                    const float* __restrict__ sin_t, float eps, int64_t rows, int S) {
    constexpr int L = D / 8;               // lanes per row
    constexpr int RPB = 256 / L;           // rows per block per step
    uint16_t* x = blockIdx.y == 0 ? q : k;
    const float* w = blockIdx.y == 0 ? w_q : w_k;
    if (x == nullptr) return;

    const int ch = threadIdx.x % L;
    const int d0 = 8 * ch;
    float wv[8];
    {
        const f32x4 a = *(const f32x4*)(w + d0), b = *(const f32x4*)(w + d0 + 4);
        wv[0] = a[0]; wv[1] = a[1]; wv[2] = a[2]; wv[3] = a[3];
        wv[4] = b[0]; wv[5] = b[1]; wv[6] = b[2]; wv[7] = b[3];
    }
    const float inv_d = 1.0f / (float)D;

    for (int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / L; r < rows; r += (int64_t)gridDim.x * RPB) {
        const int s = (int)(r % S);
        uint16_t* p = x + r * D + d0;
        const u32x4 raw = *(const u32x4*)p;
        float xv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xv[2 * i] = __builtin_bit_cast(float, raw[i] << 16);
            xv[2 * i + 1] = __builtin_bit_cast(float, raw[i] & 0xFFFF0000u);
        }
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(xv[i], xv[i], ss);
#pragma unroll
        for (int m = L / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
        const float inv_r = 1.0f / sqrtf(ss * inv_d + eps);

        const float* cr = cos_t + (int64_t)s * D + d0;
        const float* sr = sin_t + (int64_t)s * D + d0;
        const f32x4 c0 = *(const f32x4*)cr, c1 = *(const f32x4*)(cr + 4);
        const f32x4 s0 = *(const f32x4*)sr, s1 = *(const f32x4*)(sr + 4);
        const float cv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};

        u32x4 res;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ya = xv[2 * i] * inv_r * wv[2 * i];
            const float yb = xv[2 * i + 1] * inv_r * wv[2 * i + 1];
            const float za = ya * cv[2 * i] - yb * sv[2 * i];
            const float zb = yb * cv[2 * i + 1] + ya * sv[2 * i + 1];
            res[i] = pack_bf16(za, zb);
        }
        *(u32x4*)p = res;
    }
}

template <int D>
hipError_t launch(void* q, void* k, const float* w_q, const float* w_k, const float* cos_t,
                  const float* sin_t, float eps, int64_t rows, int S, hipStream_t stream) {
    constexpr int RPB = 256 / (D / 8);
    int64_t blocks = (rows + RPB - 1) / RPB;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL((qk_norm_rope_kernel<D>), dim3((unsigned)blocks, 2), dim3(256), 0, stream,
                       (uint16_t*)q, (uint16_t*)k, w_q, w_k, cos_t, sin_t, eps, rows, S);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_norm_rope(void* q, void* k, const float* w_q, const float* w_k,
                               const float* cos_t, const float* sin_t, float eps, int BH, int S,
                               int D, hipStream_t stream) {
    const int64_t rows = (int64_t)BH * S;
    if (D == 128) return launch<128>(q, k, w_q, w_k, cos_t, sin_t, eps, rows, S, stream);
    return launch<64>(q, k, w_q, w_k, cos_t, sin_t, eps, rows, S, stream);
}

}  // namespace dit

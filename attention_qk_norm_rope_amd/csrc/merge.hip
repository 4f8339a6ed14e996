// Two-way out/LSE merge for gfx950, in place into (out_a, lse_a).  HBM-bound.
//
// Operation: "NPU Wan2.2-I2V模型推理优化实践", Ring Attention Overlap (the
// local-KV and remote-KV attention outputs are combined through their
// log-sum-exp), and "feat: support Ascend NPU backend (torch_npu) for
// Qwen-Image pipelines - #274", change list item 2 (update_out_and_lse):
//   M = max(la, lb),  ea = exp(la - M), eb = exp(lb - M),
//   L = M + ln(ea + eb),  out_a <- (ea out_a + eb out_b) / (ea + eb).
// (ea/(ea+eb) is exp(la - L).)  Both LSEs -inf: out_a = 0, lse_a = -inf.
//
// Layout: D/8 consecutive lanes own one row, 8 elements each (16-byte bf16
// or 32-byte fp32 accesses).  fp32 arithmetic, one rounding when out_a is bf16.
#include "internal.h"
#include "merge_math.h"

#include <math.h>

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

template <bool F32>
__device__ __forceinline__ void load8(const void* base, int64_t off, float (&x)[8]) {
    if constexpr (F32) {
        const f32x4 a = *(const f32x4*)((const float*)base + off);
        const f32x4 b = *(const f32x4*)((const float*)base + off + 4);
        x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
        x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
    } else {
        const u32x4 r = *(const u32x4*)((const uint16_t*)base + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __builtin_bit_cast(float, r[i] << 16);
            x[2 * i + 1] = __builtin_bit_cast(float, r[i] & 0xFFFF0000u);
        }
    }
}

template <int D, bool AF32, bool BF32>
__global__ void __launch_bounds__(256)
attn_merge_kernel(void* __restrict__ out_a, float* __restrict__ lse_a, const void* __restrict__ out_b,
                  const float* __restrict__ lse_b, int64_t rows) {
    constexpr int L = D / 8;
    constexpr int RPB = 256 / L;
    const int d0 = 8 * (threadIdx.x % L);
    for (int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / L; r < rows; r += (int64_t)gridDim.x * RPB) {
        float wa, wb, Lr;
        mg::weights(lse_a[r], lse_b[r], wa, wb, Lr);
        const int64_t off = r * D + d0;
        float a[8], b[8];
        load8<AF32>(out_a, off, a);
        load8<BF32>(out_b, off, b);
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = mg::combine(wa, a[i], wb, b[i]);
        if constexpr (AF32) {
            f32x4 x0 = {o[0], o[1], o[2], o[3]}, x1 = {o[4], o[5], o[6], o[7]};
            *(f32x4*)((float*)out_a + off) = x0;
            *(f32x4*)((float*)out_a + off + 4) = x1;
        } else {
            u32x4 x = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]), pack_bf16(o[4], o[5]), pack_bf16(o[6], o[7])};
            *(u32x4*)((uint16_t*)out_a + off) = x;
        }
        // Every lane of the row has read lse_a[r] above (same wave, in order).
        if (d0 == 0) lse_a[r] = Lr;
    }
}

template <int D, bool AF32, bool BF32>
hipError_t launch(void* out_a, float* lse_a, const void* out_b, const float* lse_b, int64_t rows,
                  hipStream_t stream) {
    constexpr int RPB = 256 / (D / 8);
    int64_t blocks = (rows + RPB - 1) / RPB;
    if (blocks > (1 << 18)) blocks = 1 << 18;   // grid-stride beyond 2^18 blocks
    hipLaunchKernelGGL((attn_merge_kernel<D, AF32, BF32>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       out_a, lse_a, out_b, lse_b, rows);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch(void* out_a, float* lse_a, const void* out_b, const float* lse_b, int64_t rows,
                    bool a_f32, bool b_f32, hipStream_t stream) {
    if (a_f32) {
        return b_f32 ? launch<D, true, true>(out_a, lse_a, out_b, lse_b, rows, stream)
                     : launch<D, true, false>(out_a, lse_a, out_b, lse_b, rows, stream);
    }
    return b_f32 ? launch<D, false, true>(out_a, lse_a, out_b, lse_b, rows, stream)
                 : launch<D, false, false>(out_a, lse_a, out_b, lse_b, rows, stream);
}

}  // namespace

hipError_t launch_attn_merge(void* out_a, float* lse_a, const void* out_b, const float* lse_b,
                             int64_t rows, int D, bool a_f32, bool b_f32, hipStream_t stream) {
    if (D == 128) return dispatch<128>(out_a, lse_a, out_b, lse_b, rows, a_f32, b_f32, stream);
    return dispatch<64>(out_a, lse_a, out_b, lse_b, rows, a_f32, b_f32, stream);
}

}  // namespace dit

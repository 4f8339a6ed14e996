// BSND <-> BNSD with a head slice, for gfx950: the local layout steps on
// either side of the all-to-all of Ulysses sequence parallelism.
//
// Operation: "feat: support Ascend NPU backend (torch_npu) for Qwen-Image
// pipelines - #274", change list item 2 (npu_ulysses_attention: an
// all-to-all that gathers the sequence and splits the heads, the fused
// attention on BNSD, and the all-to-all back), and "NPU Wan2.2-I2V模型推理优化实践"
// (the attention output is produced in BNSD and transposed by the caller).
// After the sequence gather a rank holds every position of its head slice
// [h0, h0+Hs) of the model's [B, S, H, D] activations; the attention wants
// them as [B, Hs, S, D]:
//   to_bnsd:  out[b, h, s, d] = x[b, s, h0 + h, d]
//   to_bsnd:  x[b, s, h0 + h, d] = o[b, h, s, d]   (other heads untouched)
// Pure data movement (bit copies of 2-byte elements), HBM-bound: 2 bytes read
// and 2 bytes written per element of the slice.
//
// Layout: a thread moves one 16-byte chunk (8 elements of d).  Threads are
// ordered chunk-fastest, then head, then position, so the BSND side is read
// (or written) as runs of Hs*D contiguous elements and the BNSD side as runs
// of D; each wave covers 64 chunks.
#include "internal.h"

namespace dit {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool TO_BNSD>
__global__ void __launch_bounds__(256)
layout_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int B, int S, int H, int h0, int Hs,
              int D, int64_t n_chunks) {
    const int cpr = D / 8;                       // chunks per (b, s, h) row
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_chunks; i += (int64_t)gridDim.x * 256) {
        const int c = (int)(i % cpr);
        const int64_t r = i / cpr;               // (b, s, h) with h fastest
        const int h = (int)(r % Hs);
        const int64_t bs = r / Hs;
        const int s = (int)(bs % S);
        const int b = (int)(bs / S);
        const int64_t bsnd = (((int64_t)b * S + s) * H + h0 + h) * D + 8 * c;
        const int64_t bnsd = (((int64_t)b * Hs + h) * S + s) * D + 8 * c;
        // Each chunk is read and written once: non-temporal accesses.
        if constexpr (TO_BNSD)
            __builtin_nontemporal_store(__builtin_nontemporal_load((const u32x4*)(src + bsnd)), (u32x4*)(dst + bnsd));
        else
            __builtin_nontemporal_store(__builtin_nontemporal_load((const u32x4*)(src + bnsd)), (u32x4*)(dst + bsnd));
    }
}

}  // namespace

hipError_t launch_layout(const void* src, void* dst, int B, int S, int H, int h0, int Hs, int D, bool to_bnsd,
                         hipStream_t stream) {
    const int64_t n_chunks = (int64_t)B * S * Hs * (D / 8);
    int64_t blocks = (n_chunks + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;    // grid-stride beyond 2^20 blocks
    if (to_bnsd)
        hipLaunchKernelGGL((layout_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint16_t*)src, (uint16_t*)dst, B, S, H, h0, Hs, D, n_chunks);
    else
        hipLaunchKernelGGL((layout_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint16_t*)src, (uint16_t*)dst, B, S, H, h0, Hs, D, n_chunks);
    return hipGetLastError();
}

}  // namespace dit

// Per-head RMSNorm + interleaved rotary embedding of q and k, in place or
// into separate outputs, for gfx950.  HBM-bound: one 16-byte read and one 16-byte write per 8 elements.
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
// sum of squares is reduced across those lanes with xor shuffles.
#include "internal.h"
#include "norm_rope.h"

namespace dit {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));


// Grid: x = blocks of RPB sequence positions, y = q or k, z = groups of HB
// heads.  A thread loads the cos/sin/weight values of its row slice once and
// applies them to the same position of HB heads (all HB rows in flight), so
// the tables (shared by every (b,h)) are read once per HB heads instead of
// once per row.  HB trades table reads against the number of blocks in
// flight; q and k are read and written once, with non-temporal accesses.
constexpr int HB = 10;       // (b,h) rows per thread
constexpr int UNR = 10;      // rows in flight per thread

template <int D>
__global__ void __launch_bounds__(256)
qk_norm_rope_kernel(const uint16_t* q_src, const uint16_t* k_src, uint16_t* q_dst, uint16_t* k_dst,
                    const float* __restrict__ w_q, const float* __restrict__ w_k, const float* __restrict__ cos_t,
                    const float* __restrict__ sin_t, float eps, int BH, int S) {
    constexpr int L = D / 8;               // lanes per row
    constexpr int RPB = 256 / L;           // sequence positions per block
    // Source and destination are equal for the in-place form (no restrict).
    const uint16_t* x = blockIdx.y == 0 ? q_src : k_src;
    uint16_t* y = blockIdx.y == 0 ? q_dst : k_dst;
    const float* w = blockIdx.y == 0 ? w_q : w_k;
    if (x == nullptr) return;
    // All L lanes of a row share s, so a row group leaves (or stays) as a
    // whole and the xor shuffles below stay inside active lanes.
    const int s = blockIdx.x * RPB + threadIdx.x / L;
    if (s >= S) return;
    const int ch = threadIdx.x % L;
    const int d0 = 8 * ch;

    float wv[8], cv[8], sv[8];
    {
        const f32x4 a = *(const f32x4*)(w + d0), b = *(const f32x4*)(w + d0 + 4);
        const float* cr = cos_t + (int64_t)s * D + d0;
        const float* sr = sin_t + (int64_t)s * D + d0;
        const f32x4 c0 = *(const f32x4*)cr, c1 = *(const f32x4*)(cr + 4);
        const f32x4 s0 = *(const f32x4*)sr, s1 = *(const f32x4*)(sr + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wv[i] = a[i]; wv[i + 4] = b[i];
            cv[i] = c0[i]; cv[i + 4] = c1[i];
            sv[i] = s0[i]; sv[i + 4] = s1[i];
        }
    }
    const float inv_d = 1.0f / (float)D;

    // grid.z is capped at 65535; further head groups are taken in turn.
    for (int64_t g0 = (int64_t)blockIdx.z * HB; g0 < BH; g0 += (int64_t)gridDim.z * HB) {
    const int bh0 = (int)g0, bh1 = (int)min((int64_t)BH, g0 + HB);
    for (int bh = bh0; bh < bh1; bh += UNR) {
        u32x4 raw[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u)
            if (bh + u < bh1) raw[u] = __builtin_nontemporal_load((const u32x4*)(x + ((int64_t)(bh + u) * S + s) * D + d0));
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            if (bh + u >= bh1) break;
            float xv[8];
            const unsigned rw[4] = {raw[u][0], raw[u][1], raw[u][2], raw[u][3]};
            nr::unpack8(rw, xv);
            // Chunk sums combined as an xor tree over the L lanes of the row.
            float ss = nr::chunk_sumsq(xv);
#pragma unroll
            for (int m = L / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
            const float inv_r = nr::rms_inv(ss, inv_d, eps);
            u32x4 res;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                res[i] = nr::pair(xv[2 * i], xv[2 * i + 1], inv_r, wv[2 * i], wv[2 * i + 1], cv[2 * i],
                                  cv[2 * i + 1], sv[2 * i], sv[2 * i + 1]);
            __builtin_nontemporal_store(res, (u32x4*)(y + ((int64_t)(bh + u) * S + s) * D + d0));
        }
    }
    }
}

template <int D>
hipError_t launch(const void* q_src, const void* k_src, void* q, void* k, const float* w_q, const float* w_k,
                  const float* cos_t, const float* sin_t, float eps, int BH, int S, hipStream_t stream) {
    constexpr int RPB = 256 / (D / 8);
    const unsigned gx = (unsigned)((S + RPB - 1) / RPB);
    int64_t gz = ((int64_t)BH + HB - 1) / HB;
    if (gz > 65535) gz = 65535;
    hipLaunchKernelGGL((qk_norm_rope_kernel<D>), dim3(gx, 2, (unsigned)gz), dim3(256), 0, stream,
                       (const uint16_t*)q_src, (const uint16_t*)k_src, (uint16_t*)q, (uint16_t*)k, w_q, w_k, cos_t,
                       sin_t, eps, BH, S);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_norm_rope(const void* q_src, const void* k_src, void* q, void* k, const float* w_q,
                               const float* w_k, const float* cos_t, const float* sin_t, float eps, int BH, int S,
                               int D, hipStream_t stream) {
    if (D == 128) return launch<128>(q_src, k_src, q, k, w_q, w_k, cos_t, sin_t, eps, BH, S, stream);
    return launch<64>(q_src, k_src, q, k, w_q, w_k, cos_t, sin_t, eps, BH, S, stream);
}

}  // namespace dit

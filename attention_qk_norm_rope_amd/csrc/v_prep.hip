// V preparation for attn_fwd_ws on gfx950: each 64-key tile of V (bf16,
// [keys][D] rows) becomes one fp16 V^T tile in exactly the byte order the
// attention kernel keeps in LDS, so the attention kernel copies it with the
// buffer->LDS DMA and does no conversion or transposition itself.
//
// Tile image (64 keys x D rows of 128 bytes): row d holds the 64 keys of
// dimension d as fp16, keys in the order vt_col (bits 2 and 3 of the key
// index swapped, which matches the MFMA accumulator's row order), split in 8
// slots of 16 bytes; slot l is stored at l ^ ((d >> 1) & 7), so the 16 lanes
// that read one slot of 16 consecutive rows hit distinct 16-byte groups of a
// 256-byte LDS bank line.  Keys past Skv are zero.  HBM-bound: reads 2 B and
// writes 2 B per element of V (plus the zero tail of the last tile).
#include "internal.h"

namespace dit {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BN = 64;
constexpr int RSRC_WORD3 = 0x00020000;

__device__ __forceinline__ int vt_col(int key) {
    return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

__device__ __forceinline__ unsigned pack_f16(float a, float b) {
    f32x2 f = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, f16x2));
}

__device__ __forceinline__ unsigned pick_pair_f16(const u32x4& a, const u32x4& b, int e) {
    const unsigned ua = a[e >> 1], ub = b[e >> 1];
    const float fa = __builtin_bit_cast(float, (e & 1) ? (ua & 0xFFFF0000u) : (ua << 16));
    const float fb = __builtin_bit_cast(float, (e & 1) ? (ub & 0xFFFF0000u) : (ub << 16));
    return pack_f16(fa, fb);
}

template <int D>
__global__ void __launch_bounds__(256)
v_prep_kernel(const uint16_t* __restrict__ v, int64_t kv_bh_stride, uint16_t* __restrict__ ws, int BH,
              int Skv, int n_tiles, const int* __restrict__ lkv, int Hkv) {
    constexpr int TILE = BN * D;                 // elements per tile image
    __shared__ __attribute__((aligned(16))) uint16_t img[TILE];
    const int tile = blockIdx.x, tid = threadIdx.x;
    // Thread (kg, dc): keys 4*kg..+3 of the tile, d = 8*dc..+7.
    const int kg = tid & 15, dc = tid >> 4;
    const int col = vt_col(4 * kg);              // multiple of 4: 4 consecutive positions
    const int lslot = col >> 3, sub = col & 7;
    // grid.y is capped at 65535; heads beyond it are taken in turn.
    for (int bh = blockIdx.y; bh < BH; bh += gridDim.y) {
        // Keys past this head's valid length read as zeros.
        const int len = lkv ? min(max(lkv[bh / Hkv], 0), Skv) : Skv;
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(v + (int64_t)bh * kv_bh_stride), (short)0, len * D * 2, RSRC_WORD3);
        if (dc < D / 8) {
            const int key0 = tile * BN + 4 * kg;
            u32x4 r[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                r[kk] = __builtin_amdgcn_raw_buffer_load_b128(rv, ((key0 + kk) * D + 8 * dc) * 2, 0, 0);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = 8 * dc + e;
                const u32x2 w = {pick_pair_f16(r[0], r[1], e), pick_pair_f16(r[2], r[3], e)};
                *(u32x2*)(&img[d * BN + 8 * (lslot ^ ((d >> 1) & 7)) + sub]) = w;
            }
        }
        __syncthreads();
        uint16_t* dst = ws + ((int64_t)bh * n_tiles + tile) * TILE;
#pragma unroll
        for (int r = 0; r < TILE * 2 / 4096; ++r) {
            const int off = r * 2048 + tid * 8;     // elements
            *(u32x4*)(dst + off) = *(const u32x4*)(&img[off]);
        }
        __syncthreads();                         // img is rewritten by the next head
    }
}

template <int D>
hipError_t launch(const void* v, int64_t kv_bh_stride, void* ws, int BH, int Skv, const int* lkv, int Hkv,
                  hipStream_t stream) {
    const int n_tiles = (Skv + BN - 1) / BN;
    const unsigned gy = (unsigned)(BH < 65535 ? BH : 65535);
    hipLaunchKernelGGL((v_prep_kernel<D>), dim3((unsigned)n_tiles, gy), dim3(256), 0, stream,
                       (const uint16_t*)v, kv_bh_stride, (uint16_t*)ws, BH, Skv, n_tiles, lkv, Hkv);
    return hipGetLastError();
}

}  // namespace

int64_t v_prep_bytes(int64_t BH, int Skv, int D) {
    const int64_t n_tiles = (Skv + BN - 1) / BN;
    return BH * n_tiles * BN * D * 2;
}

hipError_t launch_v_prep(const void* v, int64_t kv_bh_stride, void* ws, int BH, int Skv, int D, const int* lkv,
                         int Hkv, hipStream_t stream) {
    if (D == 128) return launch<128>(v, kv_bh_stride, ws, BH, Skv, lkv, Hkv, stream);
    return launch<64>(v, kv_bh_stride, ws, BH, Skv, lkv, Hkv, stream);
}

}  // namespace dit

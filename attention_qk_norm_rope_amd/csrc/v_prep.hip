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
// 256-byte LDS bank line.  Keys past Skv are zero.
//
// fp16 holds magnitudes up to 65504 only, while bf16 V may reach 2^128.  So
// a first pass takes, for every (K/V head, d), the largest |v| over the
// head's keys; a column whose largest |v| is 2^16 or more is scaled by 2^-e
// (which brings it into [2^14, 2^15)) before the conversion, and the
// attention epilogue multiplies O's row d by 2^e.  Both are exact powers of
// two; a column below 2^16 (e = 0) converts exactly as before.
//
// Workspace layout: the tile images of all heads, then fp32-bit maxima
// [K/V head][D] (unsigned, since non-negative floats order like their bits).
// HBM-bound: the column pass reads V once, the conversion reads 2 B and
// writes 2 B per element.
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

// Element e of two key rows, times the column's scale (a power of two, so
// exact), converted to fp16 and packed.
__device__ __forceinline__ unsigned pick_pair_f16(const u32x4& a, const u32x4& b, int e, float sc) {
    const unsigned ua = a[e >> 1], ub = b[e >> 1];
    const float fa = __builtin_bit_cast(float, (e & 1) ? (ua & 0xFFFF0000u) : (ua << 16));
    const float fb = __builtin_bit_cast(float, (e & 1) ? (ub & 0xFFFF0000u) : (ub << 16));
    return pack_f16(fa * sc, fb * sc);
}

__global__ void __launch_bounds__(256) vmax_zero_kernel(unsigned* __restrict__ vmax, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) vmax[i] = 0u;
}

// Largest |v| (as fp32 bits) per (head, d) over keys [x*chunk, (x+1)*chunk)
// of the head's valid keys; blocks of one head combine by atomic max.
template <int D>
__global__ void __launch_bounds__(256)
v_colmax_kernel(const uint16_t* __restrict__ v, int64_t kv_bh_stride, unsigned* __restrict__ vmax, int BH,
                int Skv, int chunk, const int* __restrict__ lkv, int Hkv) {
    constexpr int DC = D / 8;                    // 16-byte chunks of a key row
    constexpr int KR = 256 / DC;                 // key rows per pass
    __shared__ unsigned red[KR][D];
    const int tid = threadIdx.x, dc = tid % DC, kr = tid / DC;
    for (int bh = blockIdx.y; bh < BH; bh += gridDim.y) {
        const int len = lkv ? min(max(lkv[bh / Hkv], 0), Skv) : Skv;
        const int k0 = blockIdx.x * chunk, k1 = min(k0 + chunk, len);
        const uint16_t* vb = v + (int64_t)bh * kv_bh_stride;
        unsigned m[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        for (int key = k0 + kr; key < k1; key += KR) {
            const u32x4 x = *(const u32x4*)(vb + (int64_t)key * D + 8 * dc);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const unsigned w = x[e >> 1];
                const unsigned a = ((e & 1) ? w : (w << 16)) & 0x7FFF0000u;   // |v| as fp32 bits
                m[e] = a > m[e] ? a : m[e];
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) red[kr][8 * dc + e] = m[e];
        __syncthreads();
        if (tid < D) {
            unsigned r = 0u;
#pragma unroll
            for (int i = 0; i < KR; ++i) r = red[i][tid] > r ? red[i][tid] : r;
            if (r) atomicMax(vmax + (int64_t)bh * D + tid, r);
        }
        __syncthreads();                         // red is rewritten for the next head
    }
}

// 2^-e for a column whose largest |v| has fp32 bits `bits`: e is 0 below
// 2^16 (every bf16 value below 2^16 is at most 65280, which fp16 holds),
// else the e that brings the largest value into [2^14, 2^15).
__device__ __forceinline__ float v_col_scale(unsigned bits) {
    const int x = (int)(bits >> 23);
    const int e = x >= 143 ? x - 141 : 0;
    return __builtin_bit_cast(float, (unsigned)(127 - e) << 23);
}

template <int D>
__global__ void __launch_bounds__(256)
v_prep_kernel(const uint16_t* __restrict__ v, int64_t kv_bh_stride, uint16_t* __restrict__ ws,
              const unsigned* __restrict__ vmax, int BH, int Skv, int n_tiles, const int* __restrict__ lkv,
              int Hkv) {
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
            const unsigned* vm = vmax + (int64_t)bh * D + 8 * dc;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = 8 * dc + e;
                const float sc = v_col_scale(vm[e]);
                const u32x2 w = {pick_pair_f16(r[0], r[1], e, sc), pick_pair_f16(r[2], r[3], e, sc)};
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

// Keys per block of the column pass: about 2048 blocks in all (at least 64
// keys, at most 1024 per block), so that small grids still fill the chip.
int colmax_keys(int BH, int Skv, int D) {
    const int rows = 256 / (D / 8);              // key rows one pass of a block covers
    int64_t c = ((int64_t)Skv * BH + 2047) / 2048;
    c = c < 64 ? 64 : c > 1024 ? 1024 : c;
    return (int)((c + rows - 1) / rows * rows);
}

template <int D>
hipError_t launch(const void* v, int64_t kv_bh_stride, void* ws, int BH, int Skv, const int* lkv, int Hkv,
                  hipStream_t stream) {
    const int n_tiles = (Skv + BN - 1) / BN;
    const unsigned gy = (unsigned)(BH < 65535 ? BH : 65535);
    unsigned* vmax = (unsigned*)((char*)ws + v_images_bytes(BH, Skv, D));
    const int64_t n_max = (int64_t)BH * D;
    hipLaunchKernelGGL(vmax_zero_kernel, dim3((unsigned)((n_max + 255) / 256)), dim3(256), 0, stream, vmax,
                       (int)n_max);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ck = colmax_keys(BH, Skv, D);
    hipLaunchKernelGGL((v_colmax_kernel<D>), dim3((unsigned)((Skv + ck - 1) / ck), gy), dim3(256),
                       0, stream, (const uint16_t*)v, kv_bh_stride, vmax, BH, Skv, ck, lkv, Hkv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((v_prep_kernel<D>), dim3((unsigned)n_tiles, gy), dim3(256), 0, stream,
                       (const uint16_t*)v, kv_bh_stride, (uint16_t*)ws, (const unsigned*)vmax, BH, Skv, n_tiles,
                       lkv, Hkv);
    return hipGetLastError();
}

}  // namespace

int64_t v_images_bytes(int64_t BH, int Skv, int D) {
    const int64_t n_tiles = (Skv + BN - 1) / BN;
    return BH * n_tiles * BN * D * 2;
}

int64_t v_prep_bytes(int64_t BH, int Skv, int D) {
    return v_images_bytes(BH, Skv, D) + BH * D * 4;
}

hipError_t launch_v_prep(const void* v, int64_t kv_bh_stride, void* ws, int BH, int Skv, int D, const int* lkv,
                         int Hkv, hipStream_t stream) {
    if (D == 128) return launch<128>(v, kv_bh_stride, ws, BH, Skv, lkv, Hkv, stream);
    return launch<64>(v, kv_bh_stride, ws, BH, Skv, lkv, Hkv, stream);
}

}  // namespace dit

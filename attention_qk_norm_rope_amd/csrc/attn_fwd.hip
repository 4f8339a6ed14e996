// Flash attention forward for gfx950 (CDNA4): softmax(scale * Q K^T) V with a
// per-row log-sum-exp, BNSD layout, MFMA with fp32 accumulation: Q K^T on
// bf16 operands, P V on fp16 operands (see below).
//
// Operation: "Cosmos 昇腾 NPU 多卡并行优化说明" §3.1 and the
// npu_fused_infer_attention_score section of "NPU Wan2.2-I2V模型推理优化实践"
// (BNSD, explicit softmax scale, full or top-left causal attention); the LSE
// is the statistic the Ring Attention Overlap section merges with.
//
// Design (one workgroup = 4 waves = 4 x 32*NQB query rows):
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K fragments (A operand) come from LDS, Q
//    fragments (B operand) stay in registers for the whole loop.  In the
//    32x32 accumulator layout every lane then owns ONE query column and 16
//    keys, so the row max and row sum are in-lane; only one cross-half swap
//    (v_permlane32_swap) per tile is needed for the max.
//  * The probabilities P^T leave the score accumulator already in the B
//    operand layout of the next MFMA, O^T += V^T P^T, provided the key order
//    inside each 16-key step follows the accumulator's row order.  V is
//    therefore written to LDS transposed ([d][key], as fp16) with bits 2 and 3 of the
//    key index swapped, which makes each lane's 8 keys one 16-byte read.
//  * O^T lives in registers with one query per lane, so the online-softmax
//    rescale multiplies by a per-lane scalar.  The running max is only moved
//    when the tile max exceeds it by more than TAU (log2 units); otherwise
//    P is computed against the stale max (values <= 2^TAU, exact after the
//    final division).  Most tiles skip the rescale entirely.  O is
//    normalised by the sum of the bf16-rounded P that entered the MFMA (the
//    applied weights then sum to 1); the LSE uses a separate fp32 sum of P.
//  * K and V^T tiles of BN = 64 keys are double-buffered in LDS; the next
//    tile's global loads are issued before the current tile's MFMAs and
//    written to the other buffer after them, one barrier per tile.
//  * Workgroup ids are remapped so that each XCD (ids are dealt round-robin
//    over 8 XCDs) works on a contiguous range of (b,h, q-tile): the query
//    tiles of one head share that head's K/V through one XCD's L2.
//  * exp is exp2 of fma(s, scale*log2(e), -m); the scale sign is folded into
//    Q (an exact bf16 negation) so the multiplier is always positive.
//  * P V runs on v_mfma_f32_32x32x16_f16 (same rate as bf16): P is rounded
//    to fp16 (11 significant bits instead of 8; P <= 2^TAU fits), and V is
//    converted from bf16 to fp16 while it is transposed into LDS -- exact
//    for |v| in [2^-14, 65504].  With peaked softmax rows (a few dominant
//    keys) bf16 P alone puts errors of ~1e-3 into O; fp16 P makes them 8x
//    smaller.
#include "internal.h"

#include <math.h>

namespace dit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVES = 4;
constexpr int BN = 64;                 // keys per tile
constexpr float LN2 = 0.69314718055994531f;
constexpr float TAU = 8.0f;            // lazy-rescale threshold, log2 units

template <int D>
struct Lds {
    static constexpr int KROW = D + 8;    // K tile row stride, elements (16 B pad)
    static constexpr int VROW = BN + 8;   // V^T tile row stride, elements (16 B pad)
    static constexpr int K_ELEMS = BN * KROW;
    static constexpr int V_ELEMS = D * VROW;
};

// Column of key `key` (0..BN-1) inside a V^T row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_col(int key) {
    return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    f32x2 f = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ unsigned pack_f16(float a, float b) {
    f32x2 f = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, f16x2));
}

// max / sum of a lane's value and the value of the lane 32 away.
__device__ __forceinline__ float pair_max(float x) {
    unsigned u = __builtin_bit_cast(unsigned, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    unsigned u = __builtin_bit_cast(unsigned, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// bf16 element e of two key rows (8 bf16 each), converted to fp16 and packed
// two keys per dword.  The conversion is exact for |v| in [2^-14, 65504].
__device__ __forceinline__ unsigned pick_pair_f16(const u32x4& a, const u32x4& b, int e) {
    const unsigned ua = a[e >> 1], ub = b[e >> 1];
    const float fa = __builtin_bit_cast(float, (e & 1) ? (ua & 0xFFFF0000u) : (ua << 16));
    const float fb = __builtin_bit_cast(float, (e & 1) ? (ub & 0xFFFF0000u) : (ub << 16));
    return pack_f16(fa, fb);
}

template <int D, int NQB, bool OUT_F32>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256)))
__attribute__((amdgpu_waves_per_eu(NQB == 1 ? 2 : 1, NQB == 1 ? 2 : 1)))
attn_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                const uint16_t* __restrict__ v, int64_t kv_bh_stride, void* __restrict__ out,
                float* __restrict__ lse, int Sq, int Skv, float c, unsigned qsign, int causal,
                int n_qtiles) {
    constexpr int QPW = 32 * NQB;       // query rows per wave
    constexpr int BM = WAVES * QPW;     // query rows per workgroup
    constexpr int DT = D / 16;          // MFMA k-steps of Q K^T
    constexpr int DB = D / 32;          // 32-wide d blocks of the output
    constexpr int KB = BN / 32;         // 32-key blocks per tile
    constexpr int KL = BN * D / 8 / 256;  // 16-byte K loads per thread per tile
    constexpr int KROW = Lds<D>::KROW, VROW = Lds<D>::VROW;

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][Lds<D>::K_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][Lds<D>::V_ELEMS];

    // XCD-contiguous remap of the workgroup id.
    const int nblk = gridDim.x, wid = blockIdx.x;
    const int per = nblk >> 3, rem = nblk & 7, xcd = wid & 7;
    const int logical = xcd * per + min(xcd, rem) + (wid >> 3);
    const int bh = logical / n_qtiles;
    int qt = logical - bh * n_qtiles;
    if (causal) qt = n_qtiles - 1 - qt;   // longest rows first
    const int q0 = qt * BM;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, n = lane & 31, hh = lane >> 5;
    const int q0w = q0 + wave * QPW;

    // Q^T fragments: lane holds query (q0w + 32*qb + n), d = 16t + 8hh .. +7.
    bf16x8 qf[NQB][DT];
    {
        const uint16_t* qb_ptr = q + (int64_t)bh * Sq * D;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            const int qi = q0w + 32 * qb + n;
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                u32x4 x = {0u, 0u, 0u, 0u};
                if (qi < Sq) x = *(const u32x4*)(qb_ptr + (int64_t)qi * D + 16 * t + 8 * hh);
                x ^= qsign;
                qf[qb][t] = __builtin_bit_cast(bf16x8, x);
            }
        }
    }

    const uint16_t* kbase = k + (int64_t)bh * kv_bh_stride;
    const uint16_t* vbase = v + (int64_t)bh * kv_bh_stride;
    int n_tiles = (Skv + BN - 1) / BN;
    if (causal) {
        const int qlast = min(q0 + BM, Sq) - 1;
        n_tiles = min(n_tiles, qlast / BN + 1);
    }

    // Staging registers for the next tile.
    u32x4 kst[KL];
    u32x4 vst[4];
    const int v_kg = tid & 15, v_dc = tid >> 4;     // V: keys 4*v_kg.., d 8*v_dc..
    const bool v_active = v_dc < D / 8;

    auto load_tile = [&](int kv0) {
#pragma unroll
        for (int r = 0; r < KL; ++r) {
            const int idx = r * 256 + tid;
            const int key = idx / (D / 8), ch = idx % (D / 8);
            const int gk = kv0 + key;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (gk < Skv) x = *(const u32x4*)(kbase + (int64_t)gk * D + 8 * ch);
            kst[r] = x;
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int gk = kv0 + 4 * v_kg + kk;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (v_active && gk < Skv) x = *(const u32x4*)(vbase + (int64_t)gk * D + 8 * v_dc);
            vst[kk] = x;
        }
    };
    auto store_tile = [&](int b) {
#pragma unroll
        for (int r = 0; r < KL; ++r) {
            const int idx = r * 256 + tid;
            const int key = idx / (D / 8), ch = idx % (D / 8);
            *(u32x4*)(&Ks[b][key * KROW + 8 * ch]) = kst[r];
        }
        if (v_active) {
            const int col = vt_col(4 * v_kg);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u32x2 w2 = {pick_pair_f16(vst[0], vst[1], e), pick_pair_f16(vst[2], vst[3], e)};
                *(u32x2*)(&Vt[b][(8 * v_dc + e) * VROW + col]) = w2;
            }
        }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();

    f32x16 o[NQB][DB];
    // l_run: sum of the bf16-rounded P that multiplied V (normalises O with
    // the same weights the MFMA used); l_lse: exact fp32 sum of P (for LSE).
    float m_run[NQB], l_run[NQB], l_lse[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
        l_lse[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[qb][db][i] = 0.f;
    }
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

    for (int j = 0; j < n_tiles; ++j) {
        const int b = j & 1;
        const int kv0 = j * BN;
        if (j + 1 < n_tiles) load_tile(kv0 + BN);

        // ---- S^T = K Q^T for BN keys x QPW queries ----
        f32x16 s[KB][NQB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][qb][i] = 0.f;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bf16x8 kf = __builtin_bit_cast(
                    bf16x8, *(const u32x4*)(&Ks[b][(32 * kb + n) * KROW + 16 * t + 8 * hh]));
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
                    s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][t], s[kb][qb], 0, 0, 0);
            }
        }

        // ---- masks: ragged key tail, causal diagonal ----
        const bool need_mask = (kv0 + BN > Skv) || (causal && kv0 + BN - 1 > q0w);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    const int qi = q0w + 32 * qb + n;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kv0 + 32 * kb + (i >> 2) * 8 + 4 * hh + (i & 3);
                        if (key >= Skv || (causal && key > qi)) s[kb][qb][i] = -INFINITY;
                    }
                }
        }

        // ---- online softmax (one query per lane) ----
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            float mx = s[0][qb][0];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][qb][i]);
            mx = pair_max(mx);
            const float m_new = mx * c;
            const bool grow = m_new > m_run[qb] + TAU;
            if (__any(grow)) {
                const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[qb] - m_new) : 1.0f;
                m_run[qb] = grow ? m_new : m_run[qb];
                l_run[qb] *= alpha;
                l_lse[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha;
            }
        }

        f16x8 pf[KB][NQB][2];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            const float neg_m = -m_run[qb];
            float lsum = 0.f, esum = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    u32x4 w4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][8 * u + 2 * e], c, neg_m));
                        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][8 * u + 2 * e + 1], c, neg_m));
                        const unsigned pk = pack_f16(p0, p1);
                        w4[e] = pk;
                        esum += p0;
                        esum += p1;
                        lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), ones, lsum, false);
                    }
                    pf[kb][qb][u] = __builtin_bit_cast(f16x8, w4);
                }
            l_run[qb] += lsum;
            l_lse[qb] += esum;
        }

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const f16x8 vf = __builtin_bit_cast(
                        f16x8, *(const u32x4*)(&Vt[b][(32 * db + n) * VROW + 32 * kb + 16 * u + 8 * hh]));
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb)
                        o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[kb][qb][u], o[qb][db], 0, 0, 0);
                }

        if (j + 1 < n_tiles) store_tile(b ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O /= l, LSE = ln2 * (m + log2 l) ----
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const float l = pair_sum(l_run[qb]);
        const float le = pair_sum(l_lse[qb]);
        const float inv = 1.0f / l;
        const int qi = q0w + 32 * qb + n;
        if (qi < Sq) {
            const int64_t row = (int64_t)bh * Sq + qi;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = 32 * db + 8 * g + 4 * hh;
                    const float a0 = o[qb][db][4 * g + 0] * inv, a1 = o[qb][db][4 * g + 1] * inv;
                    const float a2 = o[qb][db][4 * g + 2] * inv, a3 = o[qb][db][4 * g + 3] * inv;
                    if constexpr (OUT_F32) {
                        f32x4 w = {a0, a1, a2, a3};
                        *(f32x4*)((float*)out + row * D + d) = w;
                    } else {
                        u32x2 w = {pack_bf16(a0, a1), pack_bf16(a2, a3)};
                        *(u32x2*)((uint16_t*)out + row * D + d) = w;
                    }
                }
            // v_log_f32 is log2.
            if (lse && hh == 0) lse[row] = (m_run[qb] + __builtin_amdgcn_logf(le)) * LN2;
        }
    }
}

template <int D, int NQB, bool OUT_F32>
hipError_t launch(const void* q, const void* k, const void* v, int64_t kv_bh_stride, void* out,
                  float* lse, int BH, int Sq, int Skv, float c, unsigned qsign, bool causal,
                  hipStream_t stream) {
    constexpr int BM = WAVES * 32 * NQB;
    const int n_qtiles = (Sq + BM - 1) / BM;
    const int64_t nblk = (int64_t)n_qtiles * BH;
    if (nblk > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_fwd_kernel<D, NQB, OUT_F32>), dim3((unsigned)nblk), dim3(256), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, kv_bh_stride, out,
                       lse, Sq, Skv, c, qsign, causal ? 1 : 0, n_qtiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, int64_t kv_bh_stride,
                           void* out, float* lse, int BH, int Sq, int Skv, int D, float scale,
                           bool causal, bool out_f32, hipStream_t stream) {
    // Positive multiplier for exp2; the sign of the scale goes into Q.  A
    // zero (or vanishing) scale keeps a tiny positive multiplier so that
    // masked logits (-inf) still map to probability 0; the logits it yields
    // are below 1e-26 in magnitude, i.e. exactly 0 after exp2 in fp32.
    float c = fabsf(scale) * 1.44269504088896341f;
    if (!(c >= 1e-30f)) c = 1e-30f;
    const unsigned qsign = scale < 0.f ? 0x80008000u : 0u;
    if (D == 128) {
        return out_f32 ? launch<128, 1, true>(q, k, v, kv_bh_stride, out, lse, BH, Sq, Skv, c, qsign, causal, stream)
                       : launch<128, 1, false>(q, k, v, kv_bh_stride, out, lse, BH, Sq, Skv, c, qsign, causal, stream);
    }
    return out_f32 ? launch<64, 1, true>(q, k, v, kv_bh_stride, out, lse, BH, Sq, Skv, c, qsign, causal, stream)
                   : launch<64, 1, false>(q, k, v, kv_bh_stride, out, lse, BH, Sq, Skv, c, qsign, causal, stream);
}

}  // namespace dit

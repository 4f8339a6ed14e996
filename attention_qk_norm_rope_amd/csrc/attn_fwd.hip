// Flash attention forward for gfx950 (CDNA4): softmax(scale * Q K^T) V with a
// per-row log-sum-exp, BNSD layout, MFMA with fp32 accumulation: Q K^T on
// bf16 operands, P V on fp16 operands (see below).
//
// Operation: "Cosmos 昇腾 NPU 多卡并行优化说明" §3.1 and the
// npu_fused_infer_attention_score section of "NPU Wan2.2-I2V模型推理优化实践"
// (BNSD, explicit softmax scale, full or top-left causal attention); the LSE
// is the statistic the Ring Attention Overlap section merges with.
//
// Design (one workgroup = 4 waves; each wave owns 32*NQB query rows):
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K fragments (A operand) come from LDS, Q
//    fragments (B operand) stay in registers for the whole loop.  In the
//    32x32 accumulator layout every lane then owns ONE query column and 16
//    keys, so the row max and row sum are in-lane; only one cross-half swap
//    (v_permlane32_swap) per tile is needed for the max.
//  * The probabilities P^T leave the score accumulator already in the B
//    operand layout of the next MFMA, O^T += V^T P^T, provided the key order
//    inside each 16-key step follows the accumulator's row order.  V is
//    therefore written to LDS transposed ([d][key], as fp16) with bits 2 and
//    3 of the key index swapped, which makes each lane's 8 keys one 16-byte
//    read.
//  * P V runs on v_mfma_f32_32x32x16_f16 (same rate as bf16): P is rounded
//    to fp16 (11 significant bits instead of 8; P <= 2^TAU fits), and V is
//    converted from bf16 to fp16 while it is transposed into LDS -- exact
//    for |v| in [2^-14, 65504].  With peaked softmax rows (a few dominant
//    keys) bf16 P puts errors of ~1e-3 into O; fp16 P makes them 8x smaller.
//  * O^T lives in registers with one query per lane, so the online-softmax
//    rescale multiplies by a per-lane scalar.  The running max only moves
//    when a tile max exceeds it by more than TAU (log2 units); otherwise P is
//    computed against the stale max (values <= 2^TAU, exact after the final
//    division), and most tiles skip the O rescale.  O and the LSE use the sum
//    of the fp16-rounded P that multiplied V: the applied weights sum to 1,
//    and the sum is within 2^-11 relative of the exact one.
//  * Software pipeline, one barrier per 64-key tile: while the softmax of
//    tile j runs on the VALU, the MFMAs of tile j+1's scores are in flight
//    (no branch separates the two in the instruction stream; the masking of
//    a tile's scores is done at the end of the previous iteration).  K is
//    kept one tile ahead of V: iteration j DMAs K_{j+2} straight into LDS
//    (buffer_load ... lds, out-of-range keys read as zero) and loads V_{j+1}
//    through registers for the transposition.  K tiles are stored with a
//    16-byte XOR swizzle so the fragment reads do not conflict in banks.
//  * Workgroup ids are remapped so that each XCD (ids are dealt round-robin
//    over 8 XCDs) works on a contiguous range of (b,h, q-tile): the query
//    tiles of one head share that head's K/V through one XCD's L2.
//  * exp is exp2 of fma(s, scale*log2(e), -m); the scale sign is folded into
//    Q (an exact bf16 negation) so the multiplier is always positive.
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
typedef __attribute__((address_space(3))) void lds_void;

#ifndef ATTN_NQB
#define ATTN_NQB 1                     // 32-row query blocks per wave
#endif
#ifndef ATTN_BN
#define ATTN_BN 64                     // keys per tile
#endif

constexpr int WAVES = 4;
constexpr float LN2 = 0.69314718055994531f;
constexpr float TAU = 8.0f;            // lazy-rescale threshold, log2 units
constexpr int RSRC_WORD3 = 0x00020000; // raw buffer, 32-bit data format (gfx9 family)

template <int D, int BN, bool VPRE>
struct Lds {
    static constexpr int K_ELEMS = BN * D;   // K tile, XOR-swizzled 16-byte slots
    // V^T tile: padded rows when staged through registers, or the prepared
    // image (unpadded rows, XOR-swizzled 16-byte slots) when DMAed.
    static constexpr int VROW = VPRE ? BN : BN + 8;
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

template <int D, int NQB, int BN, bool OUT_F32, bool VPRE>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256)))
__attribute__((amdgpu_waves_per_eu(NQB == 1 ? 2 : 1, NQB == 1 ? 2 : 1)))
attn_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                const uint16_t* __restrict__ v, int64_t kv_bh_stride, void* __restrict__ out,
                float* __restrict__ lse, int Sq, int Skv, float c, unsigned qsign, int causal,
                int n_qtiles, const uint16_t* __restrict__ vws) {
    constexpr int QPW = 32 * NQB;       // query rows per wave
    constexpr int BM = WAVES * QPW;     // query rows per workgroup
    constexpr int DT = D / 16;          // MFMA k-steps of Q K^T
    constexpr int DB = D / 32;          // 32-wide d blocks of the output
    constexpr int KB = BN / 32;         // 32-key blocks per tile
    constexpr int SL = D / 8;           // 16-byte slots per K row
    constexpr int KDMA = BN * D * 2 / 1024 / WAVES;  // 1 KB DMA chunks per wave per tile
    constexpr int VROW = Lds<D, BN, VPRE>::VROW;
    static_assert(!VPRE || BN == 64, "the prepared V image uses 64-key tiles");
    constexpr int VKG = BN / 4;         // 4-key groups per V tile
    static_assert(KDMA >= 1 && BN % 32 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][Lds<D, BN, VPRE>::K_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][Lds<D, BN, VPRE>::V_ELEMS];

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

    // Buffer resources: loads past the end of a (b,h) slab read as zero.
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(q + (int64_t)bh * Sq * D), (short)0, Sq * D * 2, RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(k + (int64_t)bh * kv_bh_stride), (short)0, Skv * D * 2, RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(v + (int64_t)bh * kv_bh_stride), (short)0, Skv * D * 2, RSRC_WORD3);

    // Q^T fragments: lane holds query (q0w + 32*qb + n), d = 16t + 8hh .. +7.
    bf16x8 qf[NQB][DT];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int qi = q0w + 32 * qb + n;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rq, (qi * D + 16 * t + 8 * hh) * 2, 0, 0);
            x ^= qsign;
            qf[qb][t] = __builtin_bit_cast(bf16x8, x);
        }
    }

    int n_tiles = (Skv + BN - 1) / BN;
    if (causal) {
        const int qlast = min(q0 + BM, Sq) - 1;
        n_tiles = min(n_tiles, qlast / BN + 1);
    }

    // K tile j -> Ks[b] by DMA.  Wave w fills 1 KB chunks w*KDMA .. w*KDMA+KDMA-1;
    // lane l of a chunk lands at byte 16*l of it, i.e. linear 16-byte slot
    // s = 64*chunk + l = key*SL + (source slot ^ (key % SL)).
    auto dma_k = [&](int kv0, int b) {
#pragma unroll
        for (int i = 0; i < KDMA; ++i) {
            const int chunk = wave * KDMA + i;
            const int s = chunk * 64 + lane;
            const int key = s / SL;
            const int slot = (s % SL) ^ (key % SL);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(&Ks[b][chunk * 512]), 16,
                                                     ((kv0 + key) * D + 8 * slot) * 2, 0, 0, 0);
        }
    };

    // V tile: thread (v_kg, v_dc) loads keys 4*v_kg..+3, d 8*v_dc..+7, and
    // writes them transposed (fp16) into Vt[b][d][vt_col(key)].
    const int v_kg = tid % VKG, v_dc = tid / VKG;
    const bool v_active = v_dc < D / 8;
    u32x4 vst[4];
    auto load_v = [&](int kv0) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            vst[kk] = __builtin_amdgcn_raw_buffer_load_b128(rv, ((kv0 + 4 * v_kg + kk) * D + 8 * v_dc) * 2, 0, 0);
    };
    auto store_v = [&](int b) {
        if (v_active) {
            const int col = vt_col(4 * v_kg);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u32x2 w2 = {pick_pair_f16(vst[0], vst[1], e), pick_pair_f16(vst[2], vst[3], e)};
                *(u32x2*)(&Vt[b][(8 * v_dc + e) * VROW + col]) = w2;
            }
        }
    };

    // Prepared V: tile j of this (b,h) is the LDS image at vws + (bh*n_vt + j)*BN*D;
    // reads past the last tile return zeros.
    const int n_vt = (Skv + BN - 1) / BN;
    const __amdgpu_buffer_rsrc_t rvw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(VPRE ? vws + (int64_t)bh * n_vt * BN * D : v), (short)0, VPRE ? n_vt * BN * D * 2 : 0, RSRC_WORD3);
    auto dma_v = [&](int kv0, int b) {
#pragma unroll
        for (int i = 0; i < KDMA; ++i) {
            const int chunk = wave * KDMA + i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rvw, (lds_void*)(&Vt[b][chunk * 512]), 16,
                                                     (kv0 * D + chunk * 512 + lane * 8) * 2, 0, 0, 0);
        }
    };

    // S^T = K Q^T for the keys in Ks[b]; K fragments are read one k-step ahead.
    auto kfrag = [&](int b, int kb, int t) {
        const int key = 32 * kb + n;
        const int slot = (2 * t + hh) ^ (key % SL);
        return __builtin_bit_cast(bf16x8, *(const u32x4*)(&Ks[b][key * D + 8 * slot]));
    };
    auto qk = [&](int b, f32x16 (&s)[KB][NQB]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][qb][i] = 0.f;
        bf16x8 kf[2][KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) kf[0][kb] = kfrag(b, kb, 0);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            if (t + 1 < DT) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) kf[(t + 1) & 1][kb] = kfrag(b, kb, t + 1);
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
                    s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t & 1][kb], qf[qb][t], s[kb][qb], 0, 0, 0);
        }
    };

    // Ragged key tail and causal diagonal of the tile starting at kv0.
    auto needs_mask = [&](int kv0) { return (kv0 + BN > Skv) || (causal && kv0 + BN - 1 > q0w); };
    auto mask = [&](int kv0, f32x16 (&s)[KB][NQB]) {
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
    };

    f32x16 o[NQB][DB];
    float m_run[NQB], l_run[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[qb][db][i] = 0.f;
    }
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

    // One pipelined iteration: scores of tile j are in sc; leaves tile j+1's
    // (masked) scores in sn.
    auto step = [&](int j, f32x16 (&sc)[KB][NQB], f32x16 (&sn)[KB][NQB]) {
        const int b = j & 1;
        const int kv0 = j * BN;
        dma_k(kv0 + 2 * BN, b);        // K_{j+2} (zeros past the end)
        if constexpr (VPRE) dma_v(kv0 + BN, b ^ 1);   // V_{j+1} -> the buffer tile j-1 used
        else load_v(kv0 + BN);                         // V_{j+1}
        qk(b ^ 1, sn);                 // S_{j+1}: MFMAs overlap the softmax below

        // ---- online softmax of tile j (one query per lane) ----
        float alpha[NQB];
        bool grow_any = false;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            float mx = sc[0][qb][0];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][qb][i]);
            mx = pair_max(mx);
            const float m_new = mx * c;
            const bool grow = m_new > m_run[qb] + TAU;
            alpha[qb] = grow ? __builtin_amdgcn_exp2f(m_run[qb] - m_new) : 1.0f;
            m_run[qb] = grow ? m_new : m_run[qb];
            grow_any |= grow;
        }
        f16x8 pf[KB][NQB][2];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            const float neg_m = -m_run[qb];
            float lsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    u32x4 w4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][qb][8 * u + 2 * e], c, neg_m));
                        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][qb][8 * u + 2 * e + 1], c, neg_m));
                        // Sum the packed scalar, not w4[e]: a bit_cast of a vector
                        // element lvalue was lowered as element 0.
                        const unsigned pk = pack_f16(p0, p1);
                        w4[e] = pk;
                        lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), ones, lsum, false);
                    }
                    pf[kb][qb][u] = __builtin_bit_cast(f16x8, w4);
                }
            l_run[qb] = __builtin_fmaf(l_run[qb], alpha[qb], lsum);
        }
        // The rescale branch tests a value computed after P (l is never
        // negative), so the compiler keeps it below the softmax instead of
        // splitting the block above it.
        if (__any(grow_any && l_run[0] >= 0.f)) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha[qb];
        }

        // ---- O^T += V^T P^T (V^T fragments read one step ahead) ----
        {
            constexpr int NV = KB * 2 * DB;
            auto vfrag = [&](int idx) {
                const int kb = idx / (2 * DB), u = (idx / DB) % 2, db = idx % DB;
                if constexpr (VPRE) {
                    const int lslot = 4 * kb + 2 * u + hh;
                    return __builtin_bit_cast(
                        f16x8, *(const u32x4*)(&Vt[b][(32 * db + n) * VROW + 8 * (lslot ^ (n & 7))]));
                }
                return __builtin_bit_cast(
                    f16x8, *(const u32x4*)(&Vt[b][(32 * db + n) * VROW + 32 * kb + 16 * u + 8 * hh]));
            };
            f16x8 vf[2];
            vf[0] = vfrag(0);
#pragma unroll
            for (int idx = 0; idx < NV; ++idx) {
                if (idx + 1 < NV) vf[(idx + 1) & 1] = vfrag(idx + 1);
                const int kb = idx / (2 * DB), u = (idx / DB) % 2, db = idx % DB;
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
                    o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[idx & 1], pf[kb][qb][u], o[qb][db], 0, 0, 0);
            }
        }

        if constexpr (!VPRE) store_v(b ^ 1);           // V_{j+1} -> the buffer tile j-1 used
        if (needs_mask(kv0 + BN)) mask(kv0 + BN, sn);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): K_{j+2} has landed in LDS
        __syncthreads();
    };

    // Prologue: K_0, K_1 by DMA, V_0 through registers, scores of tile 0.
    f32x16 sA[KB][NQB], sB[KB][NQB];
    dma_k(0, 0);
    dma_k(BN, 1);
    if constexpr (VPRE) {
        dma_v(0, 0);
    } else {
        load_v(0);
        store_v(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    qk(0, sA);
    if (needs_mask(0)) mask(0, sA);
    __syncthreads();                    // Ks[0] is refilled by iteration 0

    int j = 0;
    for (; j + 1 < n_tiles; j += 2) {
        step(j, sA, sB);
        step(j + 1, sB, sA);
    }
    if (j < n_tiles) step(j, sA, sB);

    // ---- epilogue: O /= l, LSE = ln2 * (m + log2 l) ----
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const float l = pair_sum(l_run[qb]);
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
            if (lse && hh == 0) lse[row] = (m_run[qb] + __builtin_amdgcn_logf(l)) * LN2;
        }
    }
}

template <int D, int NQB, int BN, bool OUT_F32, bool VPRE>
hipError_t launch(const void* q, const void* k, const void* v, int64_t kv_bh_stride, void* out,
                  float* lse, int BH, int Sq, int Skv, float c, unsigned qsign, bool causal,
                  const void* vws, hipStream_t stream) {
    constexpr int BM = WAVES * 32 * NQB;
    const int n_qtiles = (Sq + BM - 1) / BM;
    const int64_t nblk = (int64_t)n_qtiles * BH;
    if (nblk > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_fwd_kernel<D, NQB, BN, OUT_F32, VPRE>), dim3((unsigned)nblk), dim3(256), 0,
                       stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, kv_bh_stride,
                       out, lse, Sq, Skv, c, qsign, causal ? 1 : 0, n_qtiles, (const uint16_t*)vws);
    return hipGetLastError();
}

template <int D, bool OUT_F32>
hipError_t launch_d(const void* q, const void* k, const void* v, int64_t kv_bh_stride, void* out,
                    float* lse, int BH, int Sq, int Skv, float c, unsigned qsign, bool causal,
                    const void* vws, hipStream_t stream) {
    if (vws)
        return launch<D, ATTN_NQB, 64, OUT_F32, true>(q, k, v, kv_bh_stride, out, lse, BH, Sq, Skv, c, qsign,
                                                      causal, vws, stream);
    return launch<D, ATTN_NQB, ATTN_BN, OUT_F32, false>(q, k, v, kv_bh_stride, out, lse, BH, Sq, Skv, c, qsign,
                                                        causal, nullptr, stream);
}

}  // namespace

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, int64_t kv_bh_stride,
                           void* out, float* lse, int BH, int Sq, int Skv, int D, float scale,
                           bool causal, bool out_f32, const void* vws, hipStream_t stream) {
    // Positive multiplier for exp2; the sign of the scale goes into Q.  A
    // zero (or vanishing) scale keeps a tiny positive multiplier so that
    // masked logits (-inf) still map to probability 0; the logits it yields
    // are below 1e-26 in magnitude, i.e. exactly 0 after exp2 in fp32.
    float c = fabsf(scale) * 1.44269504088896341f;
    if (!(c >= 1e-30f)) c = 1e-30f;
    const unsigned qsign = scale < 0.f ? 0x80008000u : 0u;
    if (D == 128) {
        return out_f32 ? launch_d<128, true>(q, k, v, kv_bh_stride, out, lse, BH, Sq, Skv, c, qsign, causal, vws, stream)
                       : launch_d<128, false>(q, k, v, kv_bh_stride, out, lse, BH, Sq, Skv, c, qsign, causal, vws, stream);
    }
    return out_f32 ? launch_d<64, true>(q, k, v, kv_bh_stride, out, lse, BH, Sq, Skv, c, qsign, causal, vws, stream)
                   : launch_d<64, false>(q, k, v, kv_bh_stride, out, lse, BH, Sq, Skv, c, qsign, causal, vws, stream);
}

}  // namespace dit

// Flash attention forward for gfx950 (CDNA4): softmax(scale * Q K^T) V with a
// per-row log-sum-exp, BNSD layout, MFMA with fp32 accumulation: Q K^T on
// bf16 operands, P V on fp16 operands (see below).
//
// Operation: "Cosmos 昇腾 NPU 多卡并行优化说明" §3.1 and the
// npu_fused_infer_attention_score section of "NPU Wan2.2-I2V模型推理优化实践"
// (BNSD, explicit softmax scale, full or top-left causal attention, key/value
// head groups, per-batch valid lengths); the LSE is the statistic the Ring
// Attention Overlap section merges with.
//
// Workgroups of 8 (or 4) waves x 32 query rows share each K/V tile in LDS,
// with two sources of V:
//  * the workspace: v_prep_kernel wrote fp16 V^T tile images into it, and
//    they are copied into LDS by the buffer->LDS DMA like K (attn_fwd_ws);
//  * otherwise (attn_fwd, no workspace) the ping-pong kernel loads each V
//    tile into registers and writes it into LDS in the same image layout.
// Two kernel forms: attn_pp_kernel (8-wave workgroups: two wave groups one
// phase apart, V from the workspace images or staged through registers,
// full or causal attention, and the split launch that deals a partly filled
// last round's key tiles evenly over the CUs) and attn_fwd_kernel (4-wave
// workgroups interleaving scores, softmax and P V within each wave: a
// mostly empty last round, and small causal grids).
//
// Epilogue variants: rows go to BNSD or to a head slice of a BSND tensor
// (a runtime output layout), and MERGE folds each row into a running
// (out, lse) pair of the same queries with the arithmetic of attn_merge
// (merge_math.h), which the ring step of the Wan2.2 page applies per chunk.
//
// Arithmetic design:
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K fragments (A operand) come from LDS, Q
//    fragments (B operand) stay in registers for the whole loop.  In the
//    32x32 accumulator layout every lane then owns ONE query column and 16
//    keys, so the row max and row sum are in-lane; only one cross-half swap
//    (v_permlane32_swap) per tile is needed for the max.
//  * The probabilities P^T leave the score accumulator already in the B
//    operand layout of the next MFMA, O^T += V^T P^T, provided the key order
//    inside each 16-key step follows the accumulator's row order.  V^T tiles
//    in LDS are [d][key] fp16 rows with bits 2 and 3 of the key index
//    swapped, which makes each lane's 8 keys one 16-byte read.
//  * P V runs on v_mfma_f32_32x32x16_f16 (same rate as bf16): P is rounded
//    to fp16 (11 significant bits instead of 8; P <= 2^TAU fits), and V is
//    converted from bf16 to fp16 -- exact for |v| in [2^-14, 65504].  With
//    peaked softmax rows (a few dominant keys) bf16 P puts errors of ~1e-3
//    into O; fp16 P makes them 8x smaller.
//  * O^T lives in registers with one query per lane, so the online-softmax
//    rescale multiplies by a per-lane scalar.  P is first taken against the
//    running max (a stale max is fine: any max gives the same result after
//    the final division, as long as P stays in fp16 range and precision).
//    When every lane of the wave has a tile sum below 2^TAU (so each of its
//    P is at most 2^TAU, log2 units) that P stands and the tile max is not
//    even computed; this is the common case once a row's max is known, and
//    such tiles skip the O rescale.  Otherwise the running max moves up to
//    the tile max wherever that is larger and P is taken again.  O and the
//    LSE use the sum of the fp16-rounded P that multiplied V, so the applied
//    weights sum to 1 (the sum is within 2^-11 relative of the exact one).
//    It is taken with v_fma_mix_f32 (an fp16 half times 1.0 plus the fp32
//    sum: two per packed pair).  The dot-product instructions (v_dot2*)
//    would add a pair in one instruction, but on gfx950 they do not issue
//    while another wave of the SIMD runs MFMAs (about 38 cycles each against
//    8), and the softmax runs beside MFMAs.
//  * exp is exp2 of fma(s, scale*log2(e), -m); the scale sign is folded into
//    Q (an exact bf16 negation) so the multiplier is always positive.
//  * LDS layouts are swizzled in 16-byte slots so that the 16 lanes that
//    read together hit distinct bank groups of a 256-byte line (gfx950 LDS
//    serves 64 banks x 4 bytes per clock).
//  * Each K/V buffer is its own LDS object: the compiler then knows that a
//    DMA into one buffer does not alias reads of the other and does not wait
//    for the DMA before those reads.
//  * Workgroup ids are remapped so that each XCD (ids are dealt round-robin
//    over the device's XCDs) works on a contiguous range of (b,h, q-tile):
//    the query tiles of one head share that head's K/V through one XCD's L2.
#include "internal.h"
#include "merge_math.h"
#include "norm_rope.h"

#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

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
using B0 = std::integral_constant<int, 0>;
using B1 = std::integral_constant<int, 1>;

constexpr int BN = 64;                 // keys per tile
constexpr int QPW = 32;                // query rows per wave
constexpr int WAVES = 8;               // waves per workgroup (4 for small grids, workspace path)
constexpr int SMALL_GRID_ROUNDS = 24;  // causal grids: 4-wave workgroups only below this many 8-wave rounds
constexpr int SK_MIN_ITERS = 16;       // split launch: key tiles per workgroup at least
constexpr int SK_LAUNCH_COST = 40;     // split launch: measured fixed cost, in key tiles of one workgroup
constexpr float LN2 = 0.69314718055994531f;
constexpr float P_SUM_FAST = 256.0f;   // 2^TAU, TAU = 8: a lane's tile sum below it bounds each of its P
constexpr int RSRC_WORD3 = 0x00020000; // raw buffer, 32-bit data format (gfx9 family)
#ifndef DIT_PP_OFFSET
#define DIT_PP_OFFSET 1
#endif
constexpr bool PP_OFFSET = DIT_PP_OFFSET;  // the two wave groups run one phase apart
constexpr bool PP_PRIO = true;         // ping-pong form: raise the wave priority during MFMA phases

// A wave-uniform value moved to a scalar register.
__device__ __forceinline__ int uniform_int(int x) { return __builtin_amdgcn_readfirstlane(x); }

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

// K tile layout: key rows of D bf16, 16-byte slot s of key `key` stored at
// slot s ^ kswz(key): 16 lanes reading one slot of 16 consecutive keys hit
// 16 distinct 16-byte groups of a 256-byte bank line.
template <int D>
__device__ __forceinline__ int kswz(int key) {
    return D == 128 ? (key & 15) : ((key >> 1) & 7);
}

// K/V head of query head bh = b*H + h when G query heads share one K/V head
// (grouped-query attention; G = 1 is plain multi-head attention).
__device__ __forceinline__ int kv_head(int bh, int H, int G) {
    return G == 1 ? bh : (bh / H) * (H / G) + (bh % H) / G;
}

// Workgroup id -> logical tile id, so that each XCD owns a contiguous range
// (the dispatcher deals workgroup ids round-robin over the nx XCDs).
__device__ __forceinline__ int xcd_remap(int wid, int nblk, int nx) {
    if (nx <= 1) return wid;
    const int per = nblk / nx, rem = nblk % nx, xcd = wid % nx;
    return xcd * per + min(xcd, rem) + wid / nx;
}

// Split-key launch (full attention over the workspace).  The query tiles of
// a last, partly filled round of workgroups are cut along the keys into
// `units` equal shares of consecutive (query tile, key tile) iterations, one
// share per workgroup of a launch of its own, so every CU gets the same
// number of key tiles.  A query tile that several shares cover leaves each
// piece's normalised rows and LSE in a slot; a fold launch after it combines
// the pieces of each such tile in share order with the arithmetic of
// attn_merge (merge_math.h).
struct SplitK {
    float* part_l;      // [2 * units][256] LSE of the partial pieces
    float* part_o;      // [2 * units][256][D] their O / l in fp32
    int64_t iters;      // key tiles over all split query tiles (tiles * nkt)
    int units;          // workgroups of the launch (<= SK_MAX_UNITS)
    int nkt;            // key tiles per query tile
};
// Share u covers iterations [u * iters / units, (u + 1) * iters / units).
__device__ __forceinline__ int64_t sk_start(int u, const SplitK& sk) { return (int64_t)u * sk.iters / sk.units; }
// The share that holds iteration x.
__device__ __forceinline__ int sk_unit(int64_t x, const SplitK& sk) {
    return (int)(((x + 1) * sk.units - 1) / sk.iters);
}
// A share has at most two partial pieces: the one it starts with (slot 2u)
// and the one it ends with (slot 2u + 1).
__device__ __forceinline__ int sk_slot(int u, int tl, const SplitK& sk) {
    return 2 * u + (sk_start(u, sk) / sk.nkt != tl ? 1 : 0);
}

// Ragged key tail and causal diagonal of the tile starting at kv0, for the
// query owned by this lane.
template <int KB>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[KB], int kv0, int Skv, bool causal, int qi, int hh) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = kv0 + 32 * kb + (i >> 2) * 8 + 4 * hh + (i & 3);
            if (key >= Skv || (causal && key > qi)) s[kb][i] = -INFINITY;
        }
}

// Row max of a tile's scores (both lane halves) and the running-max update:
// the max moves when the tile max exceeds it by more than tau.
template <int KB>
__device__ __forceinline__ void tile_max(const f32x16 (&s)[KB], float c, float tau, float& m_run, float& alpha,
                                         bool& grow) {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = pair_max(mx);
    const float m_new = mx * c;
    grow = m_new > m_run + tau;
    alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    m_run = grow ? m_new : m_run;
}

// acc + lo + hi of a packed fp16 pair, in fp32 (the conversions are exact):
// v_fma_mix_f32 with a multiplier of 1.0, which the compiler does not form
// from the equivalent C (it emits a conversion and an add per half).
__device__ __forceinline__ float add_f16_pair(unsigned pk, float acc) {
    float lo, hi;
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(lo) : "v"(pk), "v"(acc));
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(hi) : "v"(pk), "v"(lo));
    return hi;
}

// P for unit (kb, u, e) = two scores: exp2(s*c - m), packed to fp16, summed.
__device__ __forceinline__ unsigned p_pair(float s0, float s1, float c, float neg_m, float& lsum) {
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0, c, neg_m));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1, c, neg_m));
    const unsigned pk = pack_f16(p0, p1);
    lsum = add_f16_pair(pk, lsum);
    return pk;
}

// O /= l, store the row (bf16 or fp32) at out + orow*D and LSE[lrow] =
// ln2 * (m + log2 l).  A padding row (pad) and a row that saw no key (l = 0)
// store zeros and LSE = -inf.  MERGE: out/lse already hold a partial
// attention of the same row over other keys; the row is folded into it with
// the arithmetic of attn_merge (this side in fp32, as an fp32 out_b).
//
// vmax (workspace path): per d, the fp32 bits of the largest |v| of this
// K/V head; the prepared V of a column with largest |v| >= 2^16 was scaled
// by 2^-e (see v_prep), and its row of O is multiplied back by 2^e here
// (e = 0, a factor of exactly 1, for every other column).
template <int D, bool OUT_F32, bool MERGE>
__device__ __forceinline__ void store_row(const f32x16 (&o)[D / 32], float m_run, float l_half, int64_t orow,
                                          int64_t lrow, bool valid, bool pad, int hh, void* out, float* lse,
                                          const unsigned* vmax) {
    const float l = pair_sum(l_half);
    const bool empty = pad || !(l > 0.f);
    const float inv = empty ? 0.f : 1.0f / l;
    if (!valid) return;
    // v_log_f32 is log2.
    const float lb = empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l)) * LN2;
    float wa = 0.f, wb = 0.f, lm = lb;
    if constexpr (MERGE) mg::weights(lse[lrow], lb, wa, wb, lm);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = 32 * db + 8 * g + 4 * hh;
            float sc[4] = {1.f, 1.f, 1.f, 1.f};
            if (vmax) {
                const u32x4 mb = *(const u32x4*)(vmax + d);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int x = (int)(mb[i] >> 23);
                    sc[i] = __builtin_bit_cast(float, (unsigned)(127 + (x >= 143 ? x - 141 : 0)) << 23);
                }
            }
            float a[4];
#pragma unroll
            // After the division: o / l is below 2^15 in a scaled column, so
            // the power of two cannot overflow what the output can hold.
            for (int i = 0; i < 4; ++i) a[i] = empty ? 0.f : (o[db][4 * g + i] * inv) * sc[i];   // not 0 * garbage
            if constexpr (MERGE) {
                float x[4];
                if constexpr (OUT_F32) {
                    const f32x4 r = *(const f32x4*)((const float*)out + orow * D + d);
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = r[i];
                } else {
                    const u32x2 r = *(const u32x2*)((const uint16_t*)out + orow * D + d);
                    x[0] = __builtin_bit_cast(float, r[0] << 16);
                    x[1] = __builtin_bit_cast(float, r[0] & 0xFFFF0000u);
                    x[2] = __builtin_bit_cast(float, r[1] << 16);
                    x[3] = __builtin_bit_cast(float, r[1] & 0xFFFF0000u);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = mg::combine(wa, x[i], wb, a[i]);
            }
            if constexpr (OUT_F32) {
                f32x4 w = {a[0], a[1], a[2], a[3]};
                *(f32x4*)((float*)out + orow * D + d) = w;
            } else {
                u32x2 w = {pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3])};
                *(u32x2*)((uint16_t*)out + orow * D + d) = w;
            }
        }
    // Both lanes of the row read lse[lrow] above (same wave, in order).
    if (lse && hh == 0) lse[lrow] = lm;
}

// Fold launch of the split launch: the rows of the split query tiles whose
// keys several shares covered (a tile that one share covered whole was
// stored by it).  D/8 lanes per row, 8 consecutive values each.  The pieces
// (shares u0..u1 of the tile, in that order) are combined with the two-way
// merge of attn_merge, the fp32 result so far as side a and the next piece as
// side b, and the row is stored as store_row stores it (with MERGE, folded
// into the running out/lse).
template <int D, bool OUT_F32, bool MERGE>
__global__ void __launch_bounds__(256)
sk_fold_kernel(SplitK sk, int tile0, int n_qtiles, int Sq, int H, void* __restrict__ out, float* __restrict__ lse,
               int out_heads, int out_h0) {
    constexpr int L = D / 8, RPB = 256 / L, ROWS = WAVES * QPW;
    const int tl = blockIdx.x / (ROWS / RPB);
    const int r = (blockIdx.x % (ROWS / RPB)) * RPB + threadIdx.x / L;
    const int d0 = 8 * (threadIdx.x % L);
    const int64_t x0 = (int64_t)tl * sk.nkt;
    const int u0 = sk_unit(x0, sk), u1 = sk_unit(x0 + sk.nkt - 1, sk);
    if (u0 == u1) return;
    const int logical = tile0 + tl;
    const int bh = logical / n_qtiles;
    const int qi = (logical - bh * n_qtiles) * ROWS + r;
    if (qi >= Sq) return;
    float acc[8];
    float la = -INFINITY;
    for (int u = u0; u <= u1; ++u) {
        const int64_t prow = (int64_t)sk_slot(u, tl, sk) * ROWS + r;
        const float lb = sk.part_l[prow];
        float wa = 0.f, wb = 0.f, lm = lb;
        if (u > u0) mg::weights(la, lb, wa, wb, lm);
        const f32x4 a = *(const f32x4*)(sk.part_o + prow * D + d0);
        const f32x4 b = *(const f32x4*)(sk.part_o + prow * D + d0 + 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = i < 4 ? a[i] : b[i - 4];
            acc[i] = u == u0 ? x : mg::combine(wa, acc[i], wb, x);
        }
        la = lm;
    }
    const int64_t lrow = (int64_t)bh * Sq + qi;
    const int64_t orow = out_heads ? ((int64_t)(bh / H) * Sq + qi) * out_heads + out_h0 + bh % H : lrow;
    float wa = 0.f, wb = 0.f, lm = la;
    if constexpr (MERGE) mg::weights(lse[lrow], la, wa, wb, lm);
    if constexpr (MERGE) {
        float x[8];
        if constexpr (OUT_F32) {
            const f32x4 a = *(const f32x4*)((const float*)out + orow * D + d0);
            const f32x4 b = *(const f32x4*)((const float*)out + orow * D + d0 + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = a[i];
                x[i + 4] = b[i];
            }
        } else {
            const u32x4 rd = *(const u32x4*)((const uint16_t*)out + orow * D + d0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = __builtin_bit_cast(float, rd[i] << 16);
                x[2 * i + 1] = __builtin_bit_cast(float, rd[i] & 0xFFFF0000u);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = mg::combine(wa, x[i], wb, acc[i]);
    }
    if constexpr (OUT_F32) {
        const f32x4 a = {acc[0], acc[1], acc[2], acc[3]}, b = {acc[4], acc[5], acc[6], acc[7]};
        *(f32x4*)((float*)out + orow * D + d0) = a;
        *(f32x4*)((float*)out + orow * D + d0 + 4) = b;
    } else {
        const u32x4 w = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]), pack_bf16(acc[4], acc[5]),
                         pack_bf16(acc[6], acc[7])};
        *(u32x4*)((uint16_t*)out + orow * D + d0) = w;
    }
    // Every lane of the row read lse[lrow] above (same wave, in order).
    if (lse && d0 == 0) lse[lrow] = lm;
}

// Q fragments of query row qi (lane half hh): qf[t] holds elements
// 16t + 8hh .. +7 of the row, the B operand of the score MFMA of k-step t.
// FQ: the row is raw and gets the RMSNorm + rotary of qk_norm_rope on the way
// (same bits): the lane holds the 16-byte chunks ch = 2t + hh of its row, so
// the xor tree of chunk sums (partners D/16 chunks apart first) is a tree
// over t followed by the cross-half pair.  The scale's sign goes into Q.
template <int D, bool FQ>
__device__ __forceinline__ void load_q(const uint16_t* qbh, int Sq, int qi, int hh, unsigned qsign,
                                       const QNormRope& qn, bf16x8 (&qf)[D / 16]) {
    constexpr int DT = D / 16;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)qbh, (short)0, Sq * D * 2,
                                                                        RSRC_WORD3);
    if constexpr (!FQ) {
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rq, (qi * D + 16 * t + 8 * hh) * 2, 0, 0);
            x ^= qsign;
            qf[t] = __builtin_bit_cast(bf16x8, x);
        }
    } else {
        unsigned raw[DT][4];
        float cs[DT];
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rq, (qi * D + 16 * t + 8 * hh) * 2, 0, 0);
            float xv[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) raw[t][i] = x[i];
            nr::unpack8(raw[t], xv);
            cs[t] = nr::chunk_sumsq(xv);
        }
#pragma unroll
        for (int m = DT / 2; m >= 1; m >>= 1)
#pragma unroll
            for (int t = 0; t < m; ++t) cs[t] += cs[t + m];
        const float total = pair_sum(cs[0]);
        const float inv_r = qi < Sq ? nr::rms_inv(total, 1.0f / (float)D, qn.eps) : 0.f;
        // Tables [Sq, D]: rows past Sq read as zeros.
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc((void*)qn.cos_t, (short)0, Sq * D * 4,
                                                                            RSRC_WORD3);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)qn.sin_t, (short)0, Sq * D * 4,
                                                                            RSRC_WORD3);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            const int d0 = 16 * t + 8 * hh;
            const f32x4 w0 = *(const f32x4*)(qn.w + d0), w1 = *(const f32x4*)(qn.w + d0 + 4);
            // Whole-vector bit casts: a bit cast of one element of a vector
            // (an lvalue) is lowered as element 0 by this compiler.
            const f32x4 c0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, (qi * D + d0) * 4, 0, 0));
            const f32x4 c1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, (qi * D + d0 + 4) * 4, 0, 0));
            const f32x4 s0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (qi * D + d0) * 4, 0, 0));
            const f32x4 s1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (qi * D + d0 + 4) * 4, 0, 0));
            const float wv[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
            float cv[8], sv[8], xv[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cv[i] = c0[i];
                cv[i + 4] = c1[i];
                sv[i] = s0[i];
                sv[i + 4] = s1[i];
            }
            nr::unpack8(raw[t], xv);
            u32x4 r;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                r[i] = nr::pair(xv[2 * i], xv[2 * i + 1], inv_r, wv[2 * i], wv[2 * i + 1], cv[2 * i], cv[2 * i + 1],
                                sv[2 * i], sv[2 * i + 1]);
            r ^= qsign;
            qf[t] = __builtin_bit_cast(bf16x8, r);
        }
    }
}

// ---------------------------------------------------------------------------
// Main loop: sub-iteration j issues three independent streams
// of work so that one wave keeps both the MFMA pipe and the VALU busy: the
// scores of tile j+1 (MFMA), the softmax of tile j (VALU) and
// O += P_{j-1} V_{j-1} (MFMA).  The body is cut into DT chunks separated by
// scheduling fences; each chunk issues two score MFMAs, two PV MFMAs, a
// slice of the softmax and the LDS fragment reads of the next chunk.  The
// lazy O rescale of tile j is applied after P_{j-1} V_{j-1}.  One barrier
// per tile; during sub-iteration j the DMAs of K_{j+2} and V_j are in flight.
template <int D, bool OUT_F32, bool FQ, bool MERGE = false, int W = WAVES>
__global__ void __attribute__((amdgpu_flat_work_group_size(W * 64, W * 64)))
__attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                   const uint16_t* __restrict__ vws, const unsigned* __restrict__ vmax, int64_t kv_bh_stride,
                   void* __restrict__ out,
                   float* __restrict__ lse, int Sq, int Skv_all, float c, unsigned qsign, int causal,
                   int n_qtiles, int H, int G, QNormRope qn, const int* __restrict__ lq,
                   const int* __restrict__ lkv, int out_heads, int out_h0, int tile0, int halves, int nxcd,
                   SplitK) {
    constexpr int BM = W * QPW;
    constexpr int DT = D / 16, DB = D / 32, KB = BN / 32, SL = D / 8;
    constexpr int TILE = BN * D;                         // elements of one K or V tile
    constexpr int KDMA = TILE * 2 / 1024 / W;         // 1 KB DMA chunks per wave per tile
    static_assert(KDMA >= 1 && KDMA * W * 1024 == TILE * 2, "tile shape");

    __shared__ __attribute__((aligned(16))) uint16_t Ks0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Ks1[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vt0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vt1[TILE];
    auto Kbuf = [&](auto bc) -> uint16_t* { if constexpr (decltype(bc)::value == 0) return Ks0; else return Ks1; };
    auto Vbuf = [&](auto bc) -> uint16_t* { if constexpr (decltype(bc)::value == 0) return Vt0; else return Vt1; };

    // Tile of this workgroup: logical tile tile0 + id of n_qtiles tiles per
    // head; with halves, two consecutive workgroups split one tile of 2*BM
    // rows (the tail of a grid of larger workgroups).
    int logical = xcd_remap(blockIdx.x, gridDim.x, nxcd);
    int half = 0;
    if (halves) {
        half = logical & 1;
        logical >>= 1;
    }
    logical += tile0;
    const int bh = logical / n_qtiles;
    const int bkv = kv_head(bh, H, G);
    // Per-batch valid lengths (variable-length batches): query rows >= Sq_b
    // are padding, keys >= Skv are masked.  Both clamp to the tensor sizes.
    const int Sq_b = lq ? min(max(lq[bh / H], 0), Sq) : Sq;
    const int Skv = lkv ? min(max(lkv[bh / H], 0), Skv_all) : Skv_all;
    int qt = logical - bh * n_qtiles;
    if (causal) qt = n_qtiles - 1 - qt;
    const int q0 = halves ? (2 * qt + half) * BM : qt * BM;

    const int tid = threadIdx.x;
    // wave is uniform: kept scalar so the DMA's LDS address (M0) needs no VALU.
    const int wave = uniform_int(tid >> 6), lane = tid & 63, n = lane & 31, hh = lane >> 5;
    const int q0w = q0 + wave * QPW;
    const int n_vt = (Skv_all + BN - 1) / BN;     // tiles of the V image

    bf16x8 qf[DT];
    load_q<D, FQ>(q + (int64_t)bh * Sq * D, Sq, q0w + n, hh, qsign, qn, qf);

    int n_tiles = (Skv + BN - 1) / BN;
    if (causal) {
        const int qlast = min(q0 + BM, Sq_b) - 1;
        n_tiles = min(n_tiles, qlast / BN + 1);
    }
    if (q0 >= Sq_b) n_tiles = 0;       // a tile of padding rows only

    // DMA sources: a buffer resource per tile, based at the tile (scalar
    // arithmetic), so every lane's offset is loop-invariant; the resource
    // ends at the last key of this head, and reads past it return zeros.
    const uint16_t* kbh = k + (int64_t)bkv * kv_bh_stride;
    auto dma_k = [&](int kv0, auto b) {
        const int left = Skv - kv0;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(kbh + (int64_t)kv0 * D), (short)0, left > 0 ? left * D * 2 : 0, RSRC_WORD3);
#pragma unroll
        for (int i = 0; i < KDMA; ++i) {
            const int s = (wave * KDMA + i) * 64 + lane;
            const int key = s / SL;
            const int slot = (s % SL) ^ kswz<D>(key);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(Kbuf(b) + (wave * KDMA + i) * 512), 16,
                                                     (key * D + 8 * slot) * 2, 0, 0, 0);
        }
    };
    // V tile `tile` of this head is the image at vbh + tile*TILE (tile < n_vt).
    const uint16_t* vbh = vws + (int64_t)bkv * n_vt * TILE;
    auto dma_v = [&](int tile, auto b) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vbh + (int64_t)tile * TILE), (short)0, TILE * 2, RSRC_WORD3);
#pragma unroll
        for (int i = 0; i < KDMA; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(Vbuf(b) + (wave * KDMA + i) * 512), 16,
                                                     ((wave * KDMA + i) * 64 + lane) * 16, 0, 0, 0);
    };
    auto kfrag = [&](auto b, int kb, int t) {
        const int key = 32 * kb + n;
        const int slot = (2 * t + hh) ^ kswz<D>(key);
        return __builtin_bit_cast(bf16x8, *(const u32x4*)(Kbuf(b) + key * D + 8 * slot));
    };
    // V^T image row d: 64 fp16 keys (128 bytes) in 8 slots, slot l at l ^ ((d>>1)&7).
    auto vfrag = [&](auto b, int kb, int u, int db) {
        const int row = 32 * db + n;
        const int lslot = 4 * kb + 2 * u + hh;
        return __builtin_bit_cast(f16x8, *(const u32x4*)(Vbuf(b) + row * BN + 8 * (lslot ^ ((row >> 1) & 7))));
    };
    auto needs_mask = [&](int kv0) { return (kv0 + BN > Skv) || (causal && kv0 + BN - 1 > q0w); };

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    constexpr int NCH = DT;                  // chunks per sub-iteration
    constexpr int PVC = KB * 2 * DB / NCH;   // PV MFMAs per chunk (2)
    static_assert(PVC * NCH == KB * 2 * DB, "chunking");
    auto pv_idx = [](int idx, int& kb, int& u, int& db) {
        kb = idx / (2 * DB);
        u = (idx / DB) % 2;
        db = idx % DB;
    };

    auto iter = [&](auto b, int j, f32x16 (&sc)[KB], f32x16 (&sn)[KB], const f16x8 (&pp)[KB][2],
                    f16x8 (&pc)[KB][2]) {
        const std::integral_constant<int, 1 - decltype(b)::value> nb{};
        const int kv0 = j * BN;
        dma_k(kv0 + 2 * BN, b);        // K_{j+2} -> the buffer K_j used
        dma_v(j, b);      // V_j -> the buffer V_{j-2} used
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sn[kb][i] = 0.f;

        bf16x8 kf[2][KB];
        f16x8 vf[2][PVC];
        auto load_chunk = [&](int t, bf16x8 (&kfo)[KB], f16x8 (&vfo)[PVC]) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) kfo[kb] = kfrag(nb, kb, t);
#pragma unroll
            for (int i = 0; i < PVC; ++i) {
                int kb, u, db;
                pv_idx(t * PVC + i, kb, u, db);
                vfo[i] = vfrag(nb, kb, u, db);
            }
        };
        load_chunk(0, kf[0], vf[0]);

        float alpha = 1.0f, neg_m = 0.f, lsum = 0.f;
        bool grow = false;
        u32x4 w4[KB][2];
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            if (t + 1 < NCH) load_chunk(t + 1, kf[(t + 1) & 1], vf[(t + 1) & 1]);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t & 1][kb], qf[t], sn[kb], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < PVC; ++i) {
                int kb, u, db;
                pv_idx(t * PVC + i, kb, u, db);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[t & 1][i], pp[kb][u], o[db], 0, 0, 0);
            }
            if (t == 0) {
                neg_m = -m_run;
            } else {
                // 16 units (kb, u, e) of two scores each, spread over chunks 1..NCH-1.
#pragma unroll
                for (int unit = 0; unit < 16; ++unit) {
                    if (1 + unit * (NCH - 1) / 16 != t) continue;
                    const int kb = unit / 8, u = (unit / 4) % 2, e = unit % 4;
                    w4[kb][u][e] = p_pair(sc[kb][8 * u + 2 * e], sc[kb][8 * u + 2 * e + 1], c, neg_m, lsum);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // P was taken against the running max.  Unless every lane's tile sum
        // is below 2^TAU (so each P is at most 2^TAU), the running max moves
        // up to the tile max wherever that is larger, and P is taken again
        // against the new max.
        if (!__all(lsum < P_SUM_FAST)) {
            tile_max(sc, c, 0.f, m_run, alpha, grow);
            if (grow) {
                lsum = 0.f;
                neg_m = -m_run;
#pragma unroll
                for (int unit = 0; unit < 16; ++unit) {
                    const int kb = unit / 8, u = (unit / 4) % 2, e = unit % 4;
                    w4[kb][u][e] = p_pair(sc[kb][8 * u + 2 * e], sc[kb][8 * u + 2 * e + 1], c, neg_m, lsum);
                }
            }
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u) pc[kb][u] = __builtin_bit_cast(f16x8, w4[kb][u]);
        l_run = __builtin_fmaf(l_run, alpha, lsum);
        if (__any(grow && l_run >= 0.f)) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        }
        if (needs_mask(kv0 + BN)) mask_tile(sn, kv0 + BN, Skv, causal, q0w + n, hh);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): K_{j+2}, V_j have landed in LDS
        __syncthreads();
    };

    // Prologue: K_0, K_1 by DMA, zeros in Vt1 (the V_{-1} that P_{-1} = 0
    // multiplies in iteration 0), scores of tile 0.
    f32x16 sA[KB], sB[KB];
    f16x8 pA[KB][2], pB[KB][2];
    dma_k(0, B0{});
    dma_k(BN, B1{});
#pragma unroll
    for (int i = 0; i < TILE / (W * 512); ++i)
        *(u32x4*)(Vt1 + (i * W * 64 + tid) * 8) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) pB[kb][u] = f16x8{};
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sA[kb][i] = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            sA[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(B0{}, kb, t), qf[t], sA[kb], 0, 0, 0);
    if (needs_mask(0)) mask_tile(sA, 0, Skv, causal, q0w + n, hh);
    __syncthreads();                    // Ks0 is refilled by iteration 0

    int j = 0;
    for (; j + 1 < n_tiles; j += 2) {
        iter(B0{}, j, sA, sB, pB, pA);
        iter(B1{}, j + 1, sB, sA, pA, pB);
    }
    // Last P V: V_{n-1} sits in buffer (n-1)&1.
    auto last_pv = [&](auto b, const f16x8 (&pp)[KB][2]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vfrag(b, kb, u, db), pp[kb][u], o[db], 0, 0, 0);
    };
    if (j < n_tiles) {
        iter(B0{}, j, sA, sB, pB, pA);
        last_pv(B0{}, pA);
    } else {
        last_pv(B1{}, pB);
    }

    // Output row: BNSD [B,H,Sq,D], or head out_h0 + h of a BSND [B,Sq,out_heads,D] tensor.
    const int qi = q0w + n;
    const int64_t lrow = (int64_t)bh * Sq + qi;
    const int64_t orow = out_heads ? ((int64_t)(bh / H) * Sq + qi) * out_heads + out_h0 + bh % H : lrow;
    store_row<D, OUT_F32, MERGE>(o, m_run, l_run, orow, lrow, qi < Sq, qi >= Sq_b, hh, out, lse,
                                 vmax ? vmax + (int64_t)bkv * D : nullptr);
}

// ---------------------------------------------------------------------------
// Ping-pong form of the same computation (8-wave workgroups over the
// workspace, full attention).  The waves form two groups of four, and each
// SIMD runs one wave of each group.  A wave alternates two phases per 64-key
// tile j:
//   M(j): the 16 score MFMAs S_j = K_j Q^T and the 16 P V MFMAs
//         O += V_{j-1}^T P_{j-1}^T, with the LDS fragment reads between them;
//   V(j): the softmax of S_j (mask, tile max, lazy rescale, exp2, fp16 P, row
//         sum) and the fragment reads that start M(j+1).
// Group 1 runs one phase behind group 0, and every phase ends at a workgroup
// barrier, so on each SIMD one wave feeds the MFMA pipe while the other keeps
// the VALU busy; the roles swap at each barrier.  Per row, the operations and
// their order are those of attn_fwd_kernel (same bits).
// K and V tiles sit in three LDS buffers each (tile t in buffer t mod 3).
// Each group issues its half of the DMAs of K_{j+2} and V_{j+1} during its
// own M(j), spread over the MFMA steps; each wave waits for its part (vmcnt)
// before the barrier after which they are first read (see tile_step).
template <int D, bool OUT_F32, bool FQ, bool MERGE, bool SK = false, bool VREG = false>
__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512)))
__attribute__((amdgpu_waves_per_eu(2, 2)))
attn_pp_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
               const uint16_t* __restrict__ vws, const unsigned* __restrict__ vmax, int64_t kv_bh_stride,
                   void* __restrict__ out,
               float* __restrict__ lse, int Sq, int Skv_all, float c, unsigned qsign, int causal,
               int n_qtiles, int H, int G, QNormRope qn, const int* __restrict__ lq,
               const int* __restrict__ lkv, int out_heads, int out_h0, int tile0, int halves, int nxcd,
               SplitK sk) {
    constexpr int W = 8;
    constexpr int DT = D / 16, DB = D / 32, KB = BN / 32, SL = D / 8;
    static_assert(!VREG || (!FQ && !MERGE && !SK && PP_OFFSET), "V through registers: the plain call only");
    constexpr int TILE = BN * D;
    constexpr int KDMA = TILE * 2 / 1024 / W;         // 1 KB DMA chunks per wave per tile
    constexpr int NSTEP = KB * DT;                    // score MFMAs per tile = P V MFMAs per tile
    static_assert(KDMA >= 1 && KDMA * W * 1024 == TILE * 2, "tile shape");
    static_assert(NSTEP == KB * 2 * DB, "pairs of one score and one P V MFMA");
    constexpr int SP = NSTEP / (2 * KDMA);            // M-phase steps per DMA chunk issued
    static_assert(SP > 2 && SP * 2 * KDMA == NSTEP, "DMA chunks spread over the steps of a phase");
    constexpr int PF = 2;                             // fragment prefetch distance (steps)
    constexpr int NR = PF + 1;                        // fragment registers in the ring
    // vmcnt that leaves one tile's DMAs (2*KDMA per wave) in flight.
    constexpr int WAIT_ONE_BATCH = 0x0F70 | (2 * KDMA);

    // V buffers first: their LDS offsets (below 48 KB) then fit the 16-bit
    // immediate of ds_write, so staging V through registers needs no
    // per-buffer address registers.
    __shared__ __attribute__((aligned(16))) uint16_t Vt0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vt1[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Vt2[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Ks0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Ks1[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Ks2[TILE];
    auto Kbuf = [&](auto bc) -> uint16_t* {
        constexpr int b = decltype(bc)::value % 3;
        if constexpr (b == 0) return Ks0; else if constexpr (b == 1) return Ks1; else return Ks2;
    };
    auto Vbuf = [&](auto bc) -> uint16_t* {
        constexpr int b = decltype(bc)::value % 3;
        if constexpr (b == 0) return Vt0; else if constexpr (b == 1) return Vt1; else return Vt2;
    };

    const int tid = threadIdx.x;
    const int wave = uniform_int(tid >> 6), lane = tid & 63, n = lane & 31, hh = lane >> 5;
    const int grp = wave >> 2;
    const int n_vt_all = (Skv_all + BN - 1) / BN;

    // One piece of work: query tile `logical` against key tiles [kt0, kt1)
    // (kt1 < 0: all keys of the batch).  slot < 0: the rows go to out;
    // otherwise to partial slot `slot`.
    auto piece = [&](int logical, int kt0, int kt1, int slot) __attribute__((always_inline)) {
        const int bh = logical / n_qtiles;
        const int bkv = kv_head(bh, H, G);
        const int Sq_b = lq ? min(max(lq[bh / H], 0), Sq) : Sq;
        const int Skv_b = lkv ? min(max(lkv[bh / H], 0), Skv_all) : Skv_all;
        // Causal: the longest query tiles of each head first.
        const int qt = logical - bh * n_qtiles;
        const int q0 = (causal ? n_qtiles - 1 - qt : qt) * (W * QPW);
        const int q0w = q0 + wave * QPW;
        const int kt_end = kt1 < 0 ? (Skv_b + BN - 1) / BN : kt1;
        // Keys of the piece, counted from key kt0 * BN, and its V image tiles
        // (those past them read as zeros).
        const int Skv = min(Skv_b, kt_end * BN) - kt0 * BN;
        const int n_vt = kt1 < 0 ? n_vt_all : kt_end - kt0;

        bf16x8 qf[DT];
        load_q<D, FQ>(q + (int64_t)bh * Sq * D, Sq, q0w + n, hh, qsign, qn, qf);

        // Causal: key tiles up to the workgroup's last row only (the split
        // launch, with kt0 > 0, is never causal).
        int n_tiles = q0 >= Sq_b || Skv <= 0 ? 0 : (Skv + BN - 1) / BN;
        if (causal) n_tiles = min(n_tiles, (min(q0 + W * QPW, Sq_b) - 1) / BN + 1);

        // DMA of this wave's 1 KB chunk i of K tile `tile` (keys past the
        // piece read as zeros) or of V image tile `tile` (tiles past the
        // image read as zeros) into buffer b.
        const uint16_t* kbh = k + (int64_t)bkv * kv_bh_stride + (int64_t)kt0 * BN * D;
        auto dma_k1 = [&](int tile, auto b, int i) {
            const int kv0 = tile * BN;
            const int left = Skv - kv0;
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(kbh + (int64_t)kv0 * D), (short)0, left > 0 ? left * D * 2 : 0, RSRC_WORD3);
            const int s = (wave * KDMA + i) * 64 + lane;
            const int key = s / SL;
            const int slot = (s % SL) ^ kswz<D>(key);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(Kbuf(b) + (wave * KDMA + i) * 512), 16,
                                                     (key * D + 8 * slot) * 2, 0, 0, 0);
        };
        const uint16_t* vbh = vws + ((int64_t)bkv * n_vt_all + kt0) * TILE;
        auto dma_v1 = [&](int tile, auto b, int i) {
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(vbh + (int64_t)min(tile, n_vt - 1) * TILE), (short)0, tile < n_vt ? TILE * 2 : 0, RSRC_WORD3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(Vbuf(b) + (wave * KDMA + i) * 512), 16,
                                                     ((wave * KDMA + i) * 64 + lane) * 16, 0, 0, 0);
        };
        auto dma_k = [&](int tile, auto b) {
    #pragma unroll
            for (int i = 0; i < KDMA; ++i) dma_k1(tile, b, i);
        };
        // V through registers (no workspace): thread (kp, dc) loads keys 2kp,
        // 2kp+1 at d-chunk dc (8 elements) of a V tile and writes them, as
        // fp16 key pairs, into that tile's V^T image in LDS (the layout the
        // workspace images have).  With D = 128 each group stages half of
        // the d-chunks; with D = 64 group 0 stages all of them.
        constexpr int VDC = D / 8;                    // d-chunks per key row
        const int v_kp = lane & 31, v_dc = (wave * 64 + lane) >> 5;
        const bool v_on = VREG && uniform_int(wave * 2) < VDC;
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(v + (int64_t)bkv * kv_bh_stride + (int64_t)kt0 * BN * D), (short)0,
            VREG && Skv > 0 ? Skv * D * 2 : 0, RSRC_WORD3);
        u32x4 vst[2];
        auto load_v = [&](int tile) {
            if (v_on) {
    #pragma unroll
                for (int i = 0; i < 2; ++i)
                    vst[i] = __builtin_amdgcn_raw_buffer_load_b128(
                        rv, (int)(((unsigned)(tile * BN + 2 * v_kp + i) * D + 8u * v_dc) * 2u), 0, 0);
            }
        };
        // Row d = 8 dc + e of the image holds this thread's key pair in slot
        // (col >> 3) ^ ((d >> 1) & 7) = sx ^ (e >> 1), sx below.  The element
        // offset is 512 dc + 64 e + 8 slot + (col & 7): the slot's XOR touches
        // bits 3-4 only, so one register, an XOR with 8 (e >> 1) and 64 e as
        // the immediate address all eight rows.
        const int v_col = vt_col(2 * v_kp);           // even: keys 2kp, 2kp+1 stay adjacent
        const int v_sx = (v_col >> 3) ^ ((4 * v_dc) & 7);
        int v_off = 8 * v_dc * BN + 8 * v_sx + (v_col & 7);
        auto store_v1 = [&](auto b, int e) {
            if (v_on) *(unsigned*)(Vbuf(b) + (v_off ^ (8 * (e >> 1))) + e * BN) = pick_pair_f16(vst[0], vst[1], e);
        };
        auto dma_v = [&](int tile, auto b) {
    #pragma unroll
            for (int i = 0; i < KDMA; ++i) dma_v1(tile, b, i);
        };
        auto kfrag = [&](auto b, int kb, int t) {
            const int key = 32 * kb + n;
            const int slot = (2 * t + hh) ^ kswz<D>(key);
            return __builtin_bit_cast(bf16x8, *(const u32x4*)(Kbuf(b) + key * D + 8 * slot));
        };
        auto vfrag = [&](auto b, int kb, int u, int db) {
            const int row = 32 * db + n;
            const int lslot = 4 * kb + 2 * u + hh;
            return __builtin_bit_cast(f16x8, *(const u32x4*)(Vbuf(b) + row * BN + 8 * (lslot ^ ((row >> 1) & 7))));
        };
        // Step i of a phase M: score MFMA (kb = i % KB, k-step i / KB) and
        // P V MFMA (index i = db + DB (u + 2 kb)).
        auto pv_idx = [](int i, int& kb, int& u, int& db) {
            kb = i / (2 * DB);
            u = (i / DB) % 2;
            db = i % DB;
        };
        auto barrier = []() { asm volatile("s_barrier" ::: "memory"); };

        f32x16 o[DB];
    #pragma unroll
        for (int db = 0; db < DB; ++db)
    #pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
        float m_run = -INFINITY, l_run = 0.f;
        f32x16 s[KB];
        f16x8 p[KB][2];
    #pragma unroll
        for (int kb = 0; kb < KB; ++kb)
    #pragma unroll
            for (int u = 0; u < 2; ++u) p[kb][u] = f16x8{};
        bf16x8 kf[NR];
        f16x8 vf[NR];

        // Fragments of step i of phase M(j): K_j in buffer bj, V_{j-1} in bv.
        auto load_step = [&](auto bj, auto bv, int i) {
            int kb, u, db;
            pv_idx(i, kb, u, db);
            kf[i % NR] = kfrag(bj, i % KB, i / KB);
            vf[i % NR] = vfrag(bv, kb, u, db);
        };

        // Prologue: K_0, K_1, V_0 by DMA; zeros in the buffer of V_{-1} (tile -1
        // mod 3 = 2), which P_{-1} = 0 multiplies in M(0).
        dma_k(0, B0{});
        dma_k(1, B1{});
        if constexpr (!VREG) {
            dma_v(0, B0{});
        } else {
            // V_0 into its image now; V_1's rows stay in registers for the
            // second half of M(0).
            load_v(0);
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): V_0 (and K_0, K_1)
    #pragma unroll
            for (int e = 0; e < 8; ++e) store_v1(B0{}, e);
            load_v(1);
        }
    #pragma unroll
        for (int i = 0; i < TILE / (W * 512); ++i)
            *(u32x4*)(Vt2 + (i * W * 64 + tid) * 8) = u32x4{0u, 0u, 0u, 0u};
        if constexpr (!VREG) __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
        else __builtin_amdgcn_s_waitcnt(0xC07F);                   // lgkmcnt(0); V_1's loads stay in flight
        barrier();

        using B2 = std::integral_constant<int, 2>;
    #pragma unroll
        for (int i = 0; i < PF; ++i) load_step(B0{}, B2{}, i);

        // One tile: M(j) then V(j) of group GRP.  b = j mod 3 selects the buffers.
        // Each group runs its own copy of the loop, so the DMAs sit at fixed
        // points of each copy (the compiler then sees which are in flight).
        //
        // DMAs: in its M(j) each group issues its half of K_{j+2} and V_{j+1}
        // (K only when V goes through registers; V_{j+1}'s image is then
        // written in the second half of M(j), see there),
        // one 1 KB chunk every SP steps: a burst of DMA issue stalls the
        // wave behind it, and in the softmax phase that stall would be on
        // the critical path.  Both tiles are first read by the fragment
        // prefetch at the end of group 0's V(j+1), phase 2j+3 (group 0 runs
        // M(j) in phase 2j, group 1 in phase 2j+1).  Group 0 waits for its
        // half at the end of M(j+1) (phase 2j+2, leaving that phase's batch
        // in flight); group 1 at the end of its V(j), also phase 2j+2.
        auto tile_step = [&](auto gc, auto bc, int j) __attribute__((always_inline)) {
            constexpr int GRP = decltype(gc)::value;
            constexpr int b = decltype(bc)::value;
            using BK = std::integral_constant<int, b>;             // K_j
            using BV = std::integral_constant<int, (b + 2) % 3>;   // V_{j-1}
            using BN1 = std::integral_constant<int, (b + 1) % 3>;  // K_{j+1}, V_{j+1}
            using BN2 = std::integral_constant<int, (b + 2) % 3>;  // K_{j+2}
            // ---- M(j)
            if constexpr (GRP == 2) {
                dma_k(j + 2, BN2{});
                dma_v(j + 1, BN1{});
            }
    #pragma unroll
            for (int kb = 0; kb < KB; ++kb)
    #pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
            if constexpr (PP_PRIO) __builtin_amdgcn_s_setprio(1);
            // Step i: the fragment reads of step i + PF, then the two MFMAs of
            // step i (fenced, so the reads stay PF steps ahead).
    #pragma unroll
            for (int i = 0; i < NSTEP; ++i) {
                if (i + PF < NSTEP) load_step(BK{}, BV{}, i + PF);
                int kb, u, db;
                pv_idx(i, kb, u, db);
                s[i % KB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % NR], qf[i / KB], s[i % KB], 0, 0, 0);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[i % NR], p[kb][u], o[db], 0, 0, 0);
                if constexpr (GRP != 2) {
                    if (i % SP == 2) {
                        const int ch = i / SP;
                        if (ch < KDMA) dma_k1(j + 2, BN2{}, ch);
                        else if constexpr (!VREG) dma_v1(j + 1, BN1{}, ch - KDMA);
                    }
                }
                if constexpr (VREG) {
                    // V_{j+1} (its rows loaded at the end of V(j-1)) into its
                    // image, one or two d rows per step of the second half,
                    // beside the MFMAs.  Only this phase's K chunks may still
                    // be in flight.
                    constexpr int HALF = NSTEP / 2, EPS = 8 / HALF;
                    static_assert(EPS * HALF == 8 && 2 < HALF, "V rows spread over the second half");
                    if (i == HALF) {
                        __builtin_amdgcn_s_waitcnt(0x0F70 | KDMA);
                        // Opaque here, so the buffer's row addresses are formed
                        // per conversion instead of living across the loop
                        // (which spilled).
                        asm volatile("" : "+v"(v_off));
                    }
                    if (i >= HALF) {
    #pragma unroll
                        for (int t = 0; t < EPS; ++t) store_v1(BN1{}, (i - HALF) * EPS + t);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (PP_PRIO) __builtin_amdgcn_s_setprio(0);
            // Group 0: its DMAs of the phase pair before have landed (this
            // phase's batch stays in flight).  V through registers: the wait
            // at the middle of the phase covered them; the image rows written
            // in this phase land before the barrier.
            if constexpr (GRP == 0 && !VREG) __builtin_amdgcn_s_waitcnt(WAIT_ONE_BATCH);
            if constexpr (VREG) __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
            if constexpr (GRP != 2) barrier();
            // ---- V(j)
            const int kv0 = j * BN;
            if (kv0 + BN > Skv || (causal && kv0 + BN - 1 > q0w)) mask_tile(s, kv0, Skv, causal, q0w + n, hh);
            // Softmax of the tile (the same rule as attn_fwd_kernel, see there).
            float alpha = 1.0f, lsum = 0.f;
            bool grow = false;
            u32x4 w4[KB][2];
            auto make_p = [&](float neg_m) __attribute__((always_inline)) {
                lsum = 0.f;
    #pragma unroll
                for (int unit = 0; unit < 16; ++unit) {
                    const int kb = unit / 8, u = (unit / 4) % 2, e = unit % 4;
                    w4[kb][u][e] = p_pair(s[kb][8 * u + 2 * e], s[kb][8 * u + 2 * e + 1], c, neg_m, lsum);
                }
            };
            make_p(-m_run);
            if (!__all(lsum < P_SUM_FAST)) {
                tile_max(s, c, 0.f, m_run, alpha, grow);
                if (grow) make_p(-m_run);
            }
    #pragma unroll
            for (int kb = 0; kb < KB; ++kb)
    #pragma unroll
                for (int u = 0; u < 2; ++u) p[kb][u] = __builtin_bit_cast(f16x8, w4[kb][u]);
            l_run = __builtin_fmaf(l_run, alpha, lsum);
            if (__any(grow && l_run >= 0.f)) {
    #pragma unroll
                for (int db = 0; db < DB; ++db)
    #pragma unroll
                    for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
            }
            // V through registers: V_{j+2}'s rows, converted in the middle of
            // M(j+1) (loaded here, after the scores are dead, to keep them out
            // of the softmax's registers).
            if constexpr (VREG) load_v(j + 2);
            // First fragments of M(j+1): K_{j+1}, and V_j (buffer b).
    #pragma unroll
            for (int i = 0; i < PF; ++i) load_step(BN1{}, BK{}, i);
            // Group 1: its DMAs of M(j) have landed (with V through registers,
            // V_{j+2}'s row loads, issued after them in this phase, may stay
            // in flight); one group: this tile's.
            if constexpr (GRP == 1 && VREG) {
                if (v_on) __builtin_amdgcn_s_waitcnt(0x0F70 | 2);
                else __builtin_amdgcn_s_waitcnt(0x0F70);
            } else if constexpr (GRP != 0) {
                __builtin_amdgcn_s_waitcnt(0x0F70);
            }
            barrier();
        };

        // Last P V: O += V_{n-1}^T P_{n-1}^T, V_{n-1} in buffer (n-1) mod 3; its
        // first fragments were loaded at the end of V(n-1) (with the unused K
        // fragments of a tile past the end).
        auto last_pv = [&](auto bv) __attribute__((always_inline)) {
    #pragma unroll
            for (int i = 0; i < NSTEP; ++i) {
                int kb, u, db;
                pv_idx(i, kb, u, db);
                const f16x8 vv = i < PF ? vf[i % NR] : vfrag(bv, kb, u, db);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vv, p[kb][u], o[db], 0, 0, 0);
            }
        };

        auto run = [&](auto gc) __attribute__((always_inline)) {
            constexpr int GRP = decltype(gc)::value;
            if constexpr (GRP == 1) barrier();   // group 1 idles for the first phase
            int j = 0;
            for (; j + 3 <= n_tiles; j += 3) {
                tile_step(gc, B0{}, j);
                tile_step(gc, B1{}, j + 1);
                tile_step(gc, B2{}, j + 2);
            }
            if (j < n_tiles) {
                tile_step(gc, B0{}, j);
                if (++j < n_tiles) tile_step(gc, B1{}, j);
            }
            // Group 1 is one phase behind: its last barrier ended V(n-1); group 0
            // takes the matching barrier after its last P V.  The DMAs of tiles
            // past the end (zeros) are drained before the workgroup can end.
            const int lb = (n_tiles + 2) % 3;       // buffer of tile n-1 (tile -1 when n = 0)
            if (lb == 0) last_pv(B0{});
            else if (lb == 1) last_pv(B1{});
            else last_pv(B2{});
            __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0)
            if constexpr (GRP == 0) barrier();
        };
        if constexpr (!PP_OFFSET) run(std::integral_constant<int, 2>{});
        else if (grp == 0) run(std::integral_constant<int, 0>{});
        else run(std::integral_constant<int, 1>{});

        const int qi = q0w + n;
        const int64_t lrow = (int64_t)bh * Sq + qi;
        const int64_t orow = out_heads ? ((int64_t)(bh / H) * Sq + qi) * out_heads + out_h0 + bh % H : lrow;
        const unsigned* vmax_h = vmax ? vmax + (int64_t)bkv * D : nullptr;
        if (slot < 0) {
            store_row<D, OUT_F32, MERGE>(o, m_run, l_run, orow, lrow, qi < Sq, qi >= Sq_b, hh, out, lse, vmax_h);
            return;
        }
        // Partial piece: its rows (O / l in fp32, with the column scales)
        // and LSE go to the slot, for the fold launch.
        const int64_t prow = (int64_t)slot * (W * QPW) + wave * QPW + n;
        store_row<D, true, false>(o, m_run, l_run, prow, prow, true, qi >= Sq_b, hh, sk.part_o, sk.part_l, vmax_h);
    };

    if constexpr (!SK) {
        piece(xcd_remap(blockIdx.x, gridDim.x, nxcd) + tile0, 0, -1, -1);
    } else {
        // Share u: its iterations, cut at query tile boundaries.
        const int u = xcd_remap(blockIdx.x, gridDim.x, nxcd);
        int64_t it = sk_start(u, sk);
        const int64_t it_end = sk_start(u + 1, sk);
        for (bool first = true; it < it_end; first = false) {
            const int tl = (int)(it / sk.nkt);
            const int kt0 = (int)(it - (int64_t)tl * sk.nkt);
            const int kt1 = (int)min((int64_t)sk.nkt, kt0 + (it_end - it));
            if (!first) __syncthreads();     // every wave is done with the previous piece's LDS
            const bool whole = kt0 == 0 && kt1 == sk.nkt;
            piece(tile0 + tl, kt0, kt1, whole ? -1 : sk_slot(u, tl, sk));
            it += kt1 - kt0;
        }
    }
}

// Compute units and XCDs of the device a stream runs on, looked up once per
// device.
struct DevShape {
    int cus, xcds;
};
constexpr int kMaxDev = 64;
std::atomic<int> g_dev_cus[kMaxDev], g_dev_xcds[kMaxDev];

DevShape dev_shape(hipStream_t stream) {
    int dev = -1;
    if (stream) {
        hipDevice_t d = -1;
        if (hipStreamGetDevice(stream, &d) == hipSuccess) dev = (int)d;
    }
    if (dev < 0 && hipGetDevice(&dev) != hipSuccess) dev = -1;
    if (dev >= 0 && dev < kMaxDev) {
        const int c = g_dev_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) return {c, g_dev_xcds[dev].load(std::memory_order_relaxed)};
    }
    int cus = 0, xcds = 0;
    if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    if (dev < 0 || hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1)
        xcds = 1;
    (void)hipGetLastError();
    if (dev >= 0 && dev < kMaxDev) {
        g_dev_xcds[dev].store(xcds, std::memory_order_relaxed);
        g_dev_cus[dev].store(cus, std::memory_order_relaxed);
    }
    return {cus, xcds};
}

}  // namespace

// Launch form of an attention call.  Full attention over the workspace:
//  * when the last round of 8-wave workgroups (one per CU) is partly filled
//    and a split-launch region is given, the split launch spreads that
//    round's key tiles evenly over up to SK_MAX_UNITS workgroups (at least
//    SK_MIN_ITERS key tiles each); it is taken when its estimated length
//    (its share plus the launch's fixed cost, in key tiles: the second
//    launch, the pipeline fill of its pieces and the fold of the partial
//    rows) beats the form below;
//  * otherwise, when that last round is at most half full, its tiles run as
//    twice as many 4-wave workgroups of 128 query rows in a second launch.
//    Each CU then holds at most one of them, and a lone 4-wave workgroup
//    runs faster than an 8-wave one.  The per-row arithmetic is the same.
// Causal grids, whose tiles differ in cost, use 4-wave workgroups throughout
// when the grid is small.  Without a workspace: one launch of 8-wave
// workgroups.
Plan make_plan(int64_t BH, int Sq, int Skv, bool causal, bool ws, bool sk_region, bool varlen, int cus) {
    Plan p{};
    const int nq8 = (Sq + WAVES * QPW - 1) / (WAVES * QPW);
    const int64_t blk8 = (int64_t)nq8 * BH;
    const int64_t tail8 = blk8 % cus;
    const int64_t nkt = (Skv + BN - 1) / BN;
    p.form = FORM_ONE;
    if (!ws) return p;
    if (causal) {
        if (blk8 < (int64_t)SMALL_GRID_ROUNDS * cus && tail8 > 0 && 2 * tail8 <= cus) p.form = FORM_ALL4;
        return p;
    }
    if (sk_region && !varlen && tail8 > 0 && tail8 <= SK_MAX_UNITS) {
        const int64_t iters = tail8 * nkt;
        const int64_t units = std::min<int64_t>(std::min(cus, SK_MAX_UNITS), iters / SK_MIN_ITERS);
        const int64_t sk_len = units > 0 ? (iters + units - 1) / units + SK_LAUNCH_COST : INT64_MAX;
        const int64_t round_len = 2 * tail8 <= cus ? nkt * 11 / 20 : nkt;
        if (units > tail8 && sk_len < round_len) {
            p.form = FORM_SPLIT;
            p.sk_iters = iters;
            p.sk_units = (int)units;
            return p;
        }
    }
    if (tail8 > 0 && 2 * tail8 <= cus) p.form = FORM_HALVES;
    return p;
}

int plan_attn(int64_t BH, int Sq, int Skv, bool causal, bool ws, bool sk_region, bool varlen, hipStream_t stream) {
    return make_plan(BH, Sq, Skv, causal, ws, sk_region, varlen, dev_shape(stream).cus).form;
}

namespace {

template <int D, bool OUT_F32>
hipError_t launch(const void* q, const void* k, const void* v, int64_t kv_bh_stride, void* out, float* lse,
                  int BH, int H, int G, int Sq, int Skv, float c, unsigned qsign, bool causal, const void* vws,
                  void* sk_ws, const QNormRope* qn, const int* lq, const int* lkv, int out_heads, int out_h0,
                  bool merge, hipStream_t stream) {
    const QNormRope qz{};
    const DevShape dv = dev_shape(stream);
    const int cus = dv.cus;
    // The workspace holds the V images, then the largest |v| per (K/V head, d).
    const unsigned* vmax =
        vws ? (const unsigned*)((const char*)vws + v_images_bytes(BH / G, Skv, D)) : nullptr;
    // One launch of workgroups of w waves over tiles [tile0, tile0 + ntile)
    // of n_qtiles per head; with halves, every tile of 2*w*QPW rows goes to
    // two workgroups; with a split, sk.units workgroups share the key tiles
    // of those query tiles.
    auto go = [&](auto kern, const QNormRope& qa, int w, int n_qtiles, int64_t tile0, int64_t ntile,
                  bool halves, const SplitK& sk) -> hipError_t {
        const int64_t nblk = sk.units ? sk.units : halves ? 2 * ntile : ntile;
        if (nblk > 0x7FFFFFFF || tile0 + ntile > 0x7FFFFFFF) return hipErrorInvalidValue;
        if (nblk == 0) return hipSuccess;
        hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(w * 64), 0, stream, (const uint16_t*)q,
                           (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)vws, vmax, kv_bh_stride, out,
                           lse, Sq,
                           Skv, c, qsign, causal ? 1 : 0, n_qtiles, H, G, qa, lq, lkv, out_heads, out_h0,
                           (int)tile0, halves ? 1 : 0, dv.xcds, sk);
        return hipGetLastError();
    };
    const SplitK none{};
    const int nq8 = (Sq + WAVES * QPW - 1) / (WAVES * QPW);
    const int64_t blk8 = (int64_t)nq8 * BH;
    const int64_t tail8 = blk8 % cus, full8 = blk8 - tail8;
    const Plan pl = make_plan(BH, Sq, Skv, causal, vws != nullptr, sk_ws != nullptr, lq != nullptr, cus);
    SplitK sk{};
    if (pl.form == FORM_SPLIT) {
        char* base = (char*)sk_ws;
        sk.part_l = (float*)base;
        sk.part_o = (float*)(base + (int64_t)2 * SK_MAX_UNITS * WAVES * QPW * 4);
        sk.iters = pl.sk_iters;
        sk.units = pl.sk_units;
        sk.nkt = (Skv + BN - 1) / BN;
    }
    const bool all4 = pl.form == FORM_ALL4, tail_split = pl.form == FORM_HALVES;
    // Full attention over the workspace runs its 8-wave workgroups in the
    // ping-pong form (same bits).
    // The split launch is followed by its fold launch.
    auto fold = [&](auto kf) -> hipError_t {
        constexpr int RPB = 256 / (D / 8);
        hipLaunchKernelGGL(kf, dim3((unsigned)(tail8 * (WAVES * QPW / RPB))), dim3(256), 0, stream, sk, (int)full8,
                           nq8, Sq, H, out, lse, out_heads, out_h0);
        return hipGetLastError();
    };
    auto run = [&](auto k4, auto kpp, auto ksk, auto kf, const QNormRope& qa) -> hipError_t {
        if (all4) return go(k4, qa, 4, (Sq + 4 * QPW - 1) / (4 * QPW), 0, (int64_t)((Sq + 4 * QPW - 1) / (4 * QPW)) * BH,
                            false, none);
        if (pl.form == FORM_SPLIT) {
            hipError_t e = go(kpp, qa, WAVES, nq8, 0, full8, false, none);
            if (e != hipSuccess) return e;
            e = go(ksk, qa, WAVES, nq8, full8, tail8, false, sk);
            if (e != hipSuccess) return e;
            return fold(kf);
        }
        if (!tail_split)
            return go(kpp, qa, WAVES, nq8, 0, blk8, false, none);
        const hipError_t e = go(kpp, qa, WAVES, nq8, 0, full8, false, none);
        if (e != hipSuccess) return e;
        return go(k4, qa, 4, nq8, full8, tail8, true, none);
    };
    if (merge)
        return run(attn_fwd_kernel<D, OUT_F32, false, true, 4>,
                   attn_pp_kernel<D, OUT_F32, false, true>, attn_pp_kernel<D, OUT_F32, false, true, true>,
                   sk_fold_kernel<D, OUT_F32, true>, qz);
    if (vws && qn)
        return run(attn_fwd_kernel<D, OUT_F32, true, false, 4>,
                   attn_pp_kernel<D, OUT_F32, true, false>, attn_pp_kernel<D, OUT_F32, true, false, true>,
                   sk_fold_kernel<D, OUT_F32, false>, *qn);
    if (vws)
        return run(attn_fwd_kernel<D, OUT_F32, false, false, 4>,
                   attn_pp_kernel<D, OUT_F32, false, false>, attn_pp_kernel<D, OUT_F32, false, false, true>,
                   sk_fold_kernel<D, OUT_F32, false>, qz);
    // Without a workspace: the ping-pong form with V staged through registers.
    return go(attn_pp_kernel<D, OUT_F32, false, false, false, true>, qz, WAVES, nq8, 0, blk8, false, none);
}

}  // namespace

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, int64_t kv_bh_stride,
                           void* out, float* lse, int BH, int H, int G, int Sq, int Skv, int D, float scale,
                           bool causal, bool out_f32, const void* vws, void* sk_ws, const QNormRope* qn,
                           const int* lq, const int* lkv, int out_heads, int out_h0, bool merge,
                           hipStream_t stream) {
    // Positive multiplier for exp2; the sign of the scale goes into Q.  A
    // zero (or vanishing) scale keeps a tiny positive multiplier so that
    // masked logits (-inf) still map to probability 0; the logits it yields
    // are below 1e-26 in magnitude, i.e. exactly 0 after exp2 in fp32.
    float c = fabsf(scale) * 1.44269504088896341f;
    if (!(c >= 1e-30f)) c = 1e-30f;
    const unsigned qsign = scale < 0.f ? 0x80008000u : 0u;
    if (D == 128)
        return out_f32 ? launch<128, true>(q, k, v, kv_bh_stride, out, lse, BH, H, G, Sq, Skv, c, qsign, causal, vws, sk_ws, qn, lq, lkv, out_heads, out_h0, merge, stream)
                       : launch<128, false>(q, k, v, kv_bh_stride, out, lse, BH, H, G, Sq, Skv, c, qsign, causal, vws, sk_ws, qn, lq, lkv, out_heads, out_h0, merge, stream);
    return out_f32 ? launch<64, true>(q, k, v, kv_bh_stride, out, lse, BH, H, G, Sq, Skv, c, qsign, causal, vws, sk_ws, qn, lq, lkv, out_heads, out_h0, merge, stream)
                   : launch<64, false>(q, k, v, kv_bh_stride, out, lse, BH, H, G, Sq, Skv, c, qsign, causal, vws, sk_ws, qn, lq, lkv, out_heads, out_h0, merge, stream);
}

}  // namespace dit

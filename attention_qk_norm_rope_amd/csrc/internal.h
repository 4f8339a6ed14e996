// Internal launch interface between the C-ABI layer (dit_attn_api.hip) and the
// gfx950 kernels.  Arguments are already validated when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

// Attention: q [BH,Sq,D] bf16 with BH = B*H query heads; query head
// bh = b*H + h reads K/V head g = b*(H/G) + h/G, rows at k + g*kv_bh_stride
// + j*D (G = 1: g = bh).  With vws != null, V is read from the prepared tiles
// written by launch_v_prep over the B*H/G K/V heads.
// With lq, lkv != null (device int32 [B]), batch b has lq[b] query rows and
// lkv[b] keys (clamped to [0, Sq] and [0, Skv]); padding rows store zeros and
// LSE -inf.  With qn != null (workspace path only), q holds the raw rows and the kernel
// applies the per-head RMSNorm + interleaved rotary of qk_norm_rope to them
// as it loads them (same bits as running qk_norm_rope on q first).
// With out_heads > 0, out is BSND [B, Sq, out_heads, D] and query head h of
// batch b writes head out_h0 + h; otherwise out is BNSD [BH, Sq, D].
// With merge (workspace path, no fused Q), out and lse hold a partial
// attention over other keys and each row is merged into them as attn_merge
// would merge an fp32 out_b.
struct QNormRope {
    const float* w;      // [D]
    const float* cos_t;  // [Sq, D]
    const float* sin_t;  // [Sq, D]
    float eps;
};
// sk_ws (workspace path, may be null): a region of sk_bytes(D) bytes; full
// attention may then run a partly filled last round of query tiles as a
// split launch over their key tiles, followed by a fold launch.
hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, int64_t kv_bh_stride,
                           void* out, float* lse, int BH, int H, int G, int Sq, int Skv, int D, float scale,
                           bool causal, bool out_f32, const void* vws, void* sk_ws, const QNormRope* qn,
                           const int* lq, const int* lkv, int out_heads, int out_h0, bool merge,
                           hipStream_t stream);

// Split-launch region: the LSE and the fp32 O / l of up to 2 * SK_MAX_UNITS
// partial pieces of 256 query rows.
constexpr int SK_MAX_UNITS = 256;
inline int64_t sk_bytes(int D) { return (int64_t)2 * SK_MAX_UNITS * 256 * (D + 1) * 4; }

// Launch form of an attention call (the DIT_FORM_* codes of the header):
// one launch of 8-wave workgroups; 8-wave rounds then the last round as
// 4-wave halves; 8-wave rounds then a split launch of the last round's key
// tiles; 4-wave workgroups throughout (small causal grids).
enum { FORM_ONE = 0, FORM_HALVES = 1, FORM_SPLIT = 2, FORM_ALL4 = 3 };
struct Plan {
    int form;
    int64_t sk_iters;   // FORM_SPLIT: key tiles of the split query tiles
    int sk_units;       // FORM_SPLIT: workgroups of the split launch
};
// BH query heads; ws: V comes from the workspace; sk_region: a split-launch
// region is given; varlen: per-batch lengths.  For the device of `stream`.
int plan_attn(int64_t BH, int Sq, int Skv, bool causal, bool ws, bool sk_region, bool varlen, hipStream_t stream);

// Bytes of prepared V for BH heads of Skv keys; launch_v_prep writes them:
// v_images_bytes of fp16 V^T tile images, then the fp32 bits of the largest
// |v| per (head, d) (BH*D unsigned), from which a column's power-of-two scale
// (applied to the images, undone in the attention epilogue) is derived.
int64_t v_images_bytes(int64_t BH, int Skv, int D);
int64_t v_prep_bytes(int64_t BH, int Skv, int D);
// With lkv != null, head bh (of B*Hkv) keeps keys < lkv[bh / Hkv] and zeros the rest.
hipError_t launch_v_prep(const void* v, int64_t kv_bh_stride, void* ws, int BH, int Skv, int D, const int* lkv,
                         int Hkv, hipStream_t stream);

// RMSNorm + interleaved rotary of q_src/k_src into q/k (equal pointers: in
// place); a tensor whose source is null is skipped.
hipError_t launch_qk_norm_rope(const void* q_src, const void* k_src, void* q, void* k, const float* w_q,
                               const float* w_k, const float* cos_t, const float* sin_t, float eps, int BH, int S,
                               int D, hipStream_t stream);

// BSND [B,S,H,D] head slice [h0, h0+Hs) <-> BNSD [B,Hs,S,D] (2-byte elements).
hipError_t launch_layout(const void* src, void* dst, int B, int S, int H, int h0, int Hs, int D, bool to_bnsd,
                         hipStream_t stream);

// out/LSE merge in place into (out_a, lse_a).
hipError_t launch_attn_merge(void* out_a, float* lse_a, const void* out_b, const float* lse_b,
                             int64_t rows, int D, bool a_f32, bool b_f32, hipStream_t stream);

}  // namespace dit

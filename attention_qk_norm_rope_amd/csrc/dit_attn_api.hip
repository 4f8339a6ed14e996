// C ABI of libdit_attn.so: argument validation, then one launch on the
// caller's stream.  Declarations and the meaning of every argument are in
// include/dit_attn.h.  Nothing here allocates, synchronises or falls back:
// a call either enqueues its kernel or returns a status before launching.
#include "../../include/dit_attn.h"
#include "internal.h"

#include <math.h>
#include <stdint.h>

#include <atomic>

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
    const uintptr_t lo = (uintptr_t)p;
    return Range{lo, lo + (uintptr_t)bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

constexpr int64_t kMaxElems = (int64_t)1 << 46;  // keeps every byte count far from overflow

int hip_status(hipError_t e) { return e == hipSuccess ? DIT_OK : DIT_ERR_HIP; }

// Checks of qk_norm_rope / qk_norm_rope_out; q_in == q (k_in == k) is the
// in-place form.  A destination may coincide exactly with its own source but
// must not overlap anything else it does not own.
int prologue_common(const void* q_in, const void* k_in, void* q, void* k, const float* w_q, const float* w_k,
                    const float* cos_t, const float* sin_t, float eps, int B, int H, int S, int D,
                    hipStream_t stream) {
    if ((!q && !k) || !cos_t || !sin_t) return DIT_ERR_NULL;
    if ((q && !w_q) || (k && !w_k)) return DIT_ERR_NULL;
    if (B < 1 || H < 1 || S < 1 || D < 1) return DIT_ERR_SHAPE;
    if (!(eps >= 0.f) || !isfinite(eps)) return DIT_ERR_SHAPE;
    if (D != 64 && D != 128) return DIT_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)B * H;
    const int64_t elems = BH * S * D;
    if (BH > 0x7FFFFFFF || elems > kMaxElems) return DIT_ERR_SHAPE;
    if ((q && (!aligned(q, 16) || !aligned(q_in, 16))) || (k && (!aligned(k, 16) || !aligned(k_in, 16))) ||
        !aligned(cos_t, 16) || !aligned(sin_t, 16) || (q && !aligned(w_q, 16)) || (k && !aligned(w_k, 16)))
        return DIT_ERR_ALIGN;
    const Range rq = range_of(q, q ? elems * 2 : 0), rk = range_of(k, k ? elems * 2 : 0);
    const Range rqi = range_of(q_in, q ? elems * 2 : 0), rki = range_of(k_in, k ? elems * 2 : 0);
    const Range rc = range_of(cos_t, (int64_t)S * D * 4), rs = range_of(sin_t, (int64_t)S * D * 4);
    const Range rwq = range_of(w_q, q ? (int64_t)D * 4 : 0), rwk = range_of(w_k, k ? (int64_t)D * 4 : 0);
    auto same = [](Range a, Range b) { return a.lo == b.lo && a.hi == b.hi; };
    if (q && k && overlap(rq, rk)) return DIT_ERR_ALIAS;
    const Range outs[2] = {rq, rk}, own[2] = {rqi, rki}, other[2] = {rki, rqi};
    for (int i = 0; i < 2; ++i) {
        const Range out = outs[i];
        if (out.lo == out.hi) continue;
        for (Range in : {rc, rs, rwq, rwk})
            if (in.lo != in.hi && overlap(out, in)) return DIT_ERR_ALIAS;
        if (overlap(out, own[i]) && !same(out, own[i])) return DIT_ERR_ALIAS;
        if (other[i].lo != other[i].hi && overlap(out, other[i])) return DIT_ERR_ALIAS;
    }
    (void)hipGetLastError();  // report only this launch's error
    return hip_status(dit::launch_qk_norm_rope(q ? q_in : nullptr, k ? k_in : nullptr, q, k, q ? w_q : nullptr,
                                               k ? w_k : nullptr, cos_t, sin_t, eps, (int)BH, S, D, stream));
}

}  // namespace

extern "C" {

int qk_norm_rope(void* q, void* k, const float* w_q, const float* w_k, const float* cos_t,
                 const float* sin_t, float eps, int B, int H, int S, int D, hipStream_t stream) {
    return prologue_common(q, k, q, k, w_q, w_k, cos_t, sin_t, eps, B, H, S, D, stream);
}

int qk_norm_rope_out(const void* q_in, const void* k_in, void* q_out, void* k_out, const float* w_q,
                     const float* w_k, const float* cos_t, const float* sin_t, float eps, int B, int H, int S,
                     int D, hipStream_t stream) {
    if ((q_in == nullptr) != (q_out == nullptr) || (k_in == nullptr) != (k_out == nullptr)) return DIT_ERR_NULL;
    return prologue_common(q_in, k_in, q_out, k_out, w_q, w_k, cos_t, sin_t, eps, B, H, S, D, stream);
}

}  // extern "C"

namespace {

// Shared argument checks of the attention entry points; on success fills
// the byte ranges of every tensor for the alias checks.  out_heads > 0 means
// out is BSND [B, Sq, out_heads, D] receiving heads [out_h0, out_h0 + H).
struct AttnRanges {
    Range q, k, v, out, lse;
};

int check_attn(const void* q, const void* k, const void* v, int64_t kv_bh_stride, void* out, float* lse,
               int B, int H, int Hkv, int Sq, int Skv, int D, float scale, int out_dtype, AttnRanges* r,
               int out_heads = 0, int out_h0 = 0) {
    if (!q || !k || !v || !out) return DIT_ERR_NULL;
    if (B < 1 || H < 1 || Sq < 1 || Skv < 1 || D < 1) return DIT_ERR_SHAPE;
    if (Hkv < 1 || Hkv > H || H % Hkv != 0) return DIT_ERR_SHAPE;
    if (!isfinite(scale)) return DIT_ERR_SHAPE;
    if (D != 64 && D != 128) return DIT_ERR_UNSUPPORTED;
    if (out_dtype != DIT_BF16 && out_dtype != DIT_FP32) return DIT_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)B * H;
    const int64_t q_elems = BH * Sq * D;
    if (BH > 0x7FFFFFFF || q_elems > kMaxElems) return DIT_ERR_SHAPE;
    if (out_heads < 0 || (out_heads > 0 && (out_heads < H || out_h0 < 0 || out_h0 > out_heads - H)))
        return DIT_ERR_SHAPE;
    const int64_t out_elems = out_heads > 0 ? (int64_t)B * Sq * out_heads * D : q_elems;
    if (out_elems > kMaxElems) return DIT_ERR_SHAPE;
    // The kernel addresses one (b,h) slab of q/k/v with 32-bit buffer offsets
    // (including up to three tiles of read-ahead past the end).
    if ((int64_t)(Sq + 512) * D * 2 > 0x7FFFFFFF || (int64_t)(Skv + 512) * D * 2 > 0x7FFFFFFF)
        return DIT_ERR_SHAPE;
    if (kv_bh_stride < (int64_t)Skv * D) return DIT_ERR_SHAPE;
    const int64_t BHkv = (int64_t)B * Hkv;
    if (kv_bh_stride > kMaxElems || (BHkv - 1) * kv_bh_stride > kMaxElems) return DIT_ERR_SHAPE;
    if (kv_bh_stride % 8 != 0) return DIT_ERR_ALIGN;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || (lse && !aligned(lse, 4)))
        return DIT_ERR_ALIGN;
    const int64_t kv_elems = (BHkv - 1) * kv_bh_stride + (int64_t)Skv * D;
    r->q = range_of(q, q_elems * 2);
    r->k = range_of(k, kv_elems * 2);
    r->v = range_of(v, kv_elems * 2);
    r->out = range_of(out, out_elems * (out_dtype == DIT_FP32 ? 4 : 2));
    r->lse = range_of(lse, lse ? BH * Sq * 4 : 0);
    if (overlap(r->out, r->q) || overlap(r->out, r->k) || overlap(r->out, r->v)) return DIT_ERR_ALIAS;
    if (lse && (overlap(r->lse, r->q) || overlap(r->lse, r->k) || overlap(r->lse, r->v) || overlap(r->lse, r->out)))
        return DIT_ERR_ALIAS;
    return DIT_OK;
}

// Bytes of prepared V (images and column maxima) for B*Hkv K/V heads; -1 for
// sizes the kernels cannot address.
int64_t v_part_bytes(int B, int Hkv, int Skv, int D) {
    if (B < 1 || Hkv < 1 || Skv < 1 || (D != 64 && D != 128)) return -1;
    const int64_t BH = (int64_t)B * Hkv;
    if (BH > 0x7FFFFFFF || (int64_t)(Skv + 512) * D * 2 > 0x7FFFFFFF) return -1;
    return dit::v_prep_bytes(BH, Skv, D);
}

// Attention launch shared by the entry points: optional workspace (V images),
// optional fused Q prologue (workspace path only), Hkv K/V heads.
int attn_common(const void* q, const void* k, const void* v, int64_t kv_bh_stride, void* workspace,
                int64_t workspace_bytes, void* out, float* lse, int B, int H, int Hkv, int Sq, int Skv, int D,
                float scale, int causal, int out_dtype, const dit::QNormRope* qn, const int* lq, const int* lkv,
                hipStream_t stream, int out_heads = 0, int out_h0 = 0, bool merge = false) {
    AttnRanges r;
    const int st = check_attn(q, k, v, kv_bh_stride, out, lse, B, H, Hkv, Sq, Skv, D, scale, out_dtype, &r,
                              out_heads, out_h0);
    if (st != DIT_OK) return st;
    // The workspace holds the prepared V (required), then the split-launch
    // region (used when the workspace is large enough for it).
    int64_t ws_used = 0;
    bool split = false;
    if (workspace) {
        if (!aligned(workspace, 16)) return DIT_ERR_ALIGN;
        const int64_t need = v_part_bytes(B, Hkv, Skv, D);
        if (need < 0 || workspace_bytes < need) return DIT_ERR_SHAPE;
        split = workspace_bytes - need >= dit::sk_bytes(D);
        ws_used = split ? need + dit::sk_bytes(D) : need;
        const Range rw = range_of(workspace, ws_used);
        if (overlap(rw, r.q) || overlap(rw, r.k) || overlap(rw, r.v) || overlap(rw, r.out) ||
            (lse && overlap(rw, r.lse)))
            return DIT_ERR_ALIAS;
        if (qn) {
            if (!aligned(qn->w, 16) || !aligned(qn->cos_t, 16) || !aligned(qn->sin_t, 16)) return DIT_ERR_ALIGN;
            const int64_t tbytes = (int64_t)Sq * D * 4;
            const Range rt[3] = {range_of(qn->w, (int64_t)D * 4), range_of(qn->cos_t, tbytes),
                                 range_of(qn->sin_t, tbytes)};
            for (const Range& t : rt)
                if (overlap(t, r.out) || overlap(t, rw) || (lse && overlap(t, r.lse))) return DIT_ERR_ALIAS;
        }
    }
    if (lq || lkv) {
        if (!lq || !lkv) return DIT_ERR_NULL;
        if (!aligned(lq, 4) || !aligned(lkv, 4)) return DIT_ERR_ALIGN;
        const Range rl[2] = {range_of(lq, (int64_t)B * 4), range_of(lkv, (int64_t)B * 4)};
        for (const Range& t : rl)
            if (overlap(t, r.out) || (lse && overlap(t, r.lse)) ||
                (workspace && overlap(t, range_of(workspace, ws_used))))
                return DIT_ERR_ALIAS;
    }
    (void)hipGetLastError();
    if (workspace) {
        const hipError_t e = dit::launch_v_prep(v, kv_bh_stride, workspace, B * Hkv, Skv, D, lkv, Hkv, stream);
        if (e != hipSuccess) return DIT_ERR_HIP;
    }
    void* sk_ws = split ? (char*)workspace + v_part_bytes(B, Hkv, Skv, D) : nullptr;
    return hip_status(dit::launch_attn_fwd(q, k, v, kv_bh_stride, out, lse, B * H, H, H / Hkv, Sq, Skv, D, scale,
                                           causal != 0, out_dtype == DIT_FP32, workspace, sk_ws, qn, lq, lkv,
                                           out_heads, out_h0, merge, stream));
}

// Shared checks of the layout entry points: a is the BSND tensor, b the BNSD slice.
int check_layout(const void* a, const void* b, int B, int S, int H, int h0, int Hs, int D) {
    if (!a || !b) return DIT_ERR_NULL;
    if (B < 1 || S < 1 || H < 1 || Hs < 1 || D < 1 || h0 < 0 || h0 > H - Hs) return DIT_ERR_SHAPE;
    if (D % 8 != 0) return DIT_ERR_UNSUPPORTED;
    if ((int64_t)B * S * H * D > kMaxElems) return DIT_ERR_SHAPE;
    if (!aligned(a, 16) || !aligned(b, 16)) return DIT_ERR_ALIGN;
    const Range rs = range_of(a, (int64_t)B * S * H * D * 2);        // the BSND tensor
    const Range rn = range_of(b, (int64_t)B * Hs * S * D * 2);       // the BNSD slice
    if (overlap(rs, rn)) return DIT_ERR_ALIAS;
    return DIT_OK;
}

}  // namespace

extern "C" {

int attn_fwd_kv_strided(const void* q, const void* k, const void* v, int64_t kv_bh_stride, void* out,
                        float* lse, int B, int H, int Sq, int Skv, int D, float scale, int causal,
                        int out_dtype, hipStream_t stream) {
    return attn_fwd_gqa(q, k, v, kv_bh_stride, nullptr, 0, out, lse, B, H, H, Sq, Skv, D, scale, causal,
                        out_dtype, stream);
}

int64_t attn_fwd_workspace_bytes(int B, int H, int Skv, int D) {
    const int64_t v_part = v_part_bytes(B, H, Skv, D);
    return v_part < 0 ? -1 : v_part + dit::sk_bytes(D);
}

int attn_fwd_launch_form(int B, int H, int Hkv, int Sq, int Skv, int D, int causal, int varlen,
                         int64_t workspace_bytes, hipStream_t stream, int* form) {
    if (!form) return DIT_ERR_NULL;
    if (B < 1 || H < 1 || Sq < 1 || Skv < 1 || Hkv < 1 || Hkv > H || H % Hkv != 0) return DIT_ERR_SHAPE;
    if (D != 64 && D != 128) return DIT_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)B * H;
    if (BH > 0x7FFFFFFF || BH * Sq * D > kMaxElems || workspace_bytes < 0) return DIT_ERR_SHAPE;
    const int64_t need = v_part_bytes(B, Hkv, Skv, D);
    if (need < 0 || (workspace_bytes > 0 && workspace_bytes < need)) return DIT_ERR_SHAPE;
    const bool ws = workspace_bytes > 0;
    const bool split = ws && workspace_bytes - need >= dit::sk_bytes(D);
    *form = dit::plan_attn(BH, Sq, Skv, causal != 0, ws, split, varlen != 0, stream);
    return DIT_OK;
}

int attn_fwd_ws(const void* q, const void* k, const void* v, int64_t kv_bh_stride, void* workspace,
                int64_t workspace_bytes, void* out, float* lse, int B, int H, int Sq, int Skv, int D,
                float scale, int causal, int out_dtype, hipStream_t stream) {
    if (!workspace) {
        AttnRanges r;
        const int st = check_attn(q, k, v, kv_bh_stride, out, lse, B, H, H, Sq, Skv, D, scale, out_dtype, &r);
        return st != DIT_OK ? st : DIT_ERR_NULL;
    }
    return attn_fwd_gqa(q, k, v, kv_bh_stride, workspace, workspace_bytes, out, lse, B, H, H, Sq, Skv, D, scale,
                        causal, out_dtype, stream);
}

int attn_fwd_gqa(const void* q, const void* k, const void* v, int64_t kv_bh_stride, void* workspace,
                 int64_t workspace_bytes, void* out, float* lse, int B, int H, int Hkv, int Sq, int Skv, int D,
                 float scale, int causal, int out_dtype, hipStream_t stream) {
    return attn_common(q, k, v, kv_bh_stride, workspace, workspace_bytes, out, lse, B, H, Hkv, Sq, Skv, D, scale,
                       causal, out_dtype, nullptr, nullptr, nullptr, stream);
}

int attn_fwd_ws_fused_q(const void* q, const void* k, const void* v, int64_t kv_bh_stride, void* workspace,
                        int64_t workspace_bytes, void* out, float* lse, const float* w_q, const float* cos_q,
                        const float* sin_q, float eps, int B, int H, int Sq, int Skv, int D, float scale,
                        int causal, int out_dtype, hipStream_t stream) {
    if (!workspace || !w_q || !cos_q || !sin_q) {
        AttnRanges r;
        const int st = check_attn(q, k, v, kv_bh_stride, out, lse, B, H, H, Sq, Skv, D, scale, out_dtype, &r);
        return st != DIT_OK ? st : DIT_ERR_NULL;
    }
    if (!(eps >= 0.f) || !isfinite(eps)) return DIT_ERR_SHAPE;
    // The kernel reads the tables with 32-bit buffer offsets.
    if ((int64_t)Sq * D * 4 > 0x7FFFFFFF) return DIT_ERR_SHAPE;
    const dit::QNormRope qn{w_q, cos_q, sin_q, eps};
    return attn_common(q, k, v, kv_bh_stride, workspace, workspace_bytes, out, lse, B, H, H, Sq, Skv, D, scale,
                       causal, out_dtype, &qn, nullptr, nullptr, stream);
}

int attn_fwd_ws_bsnd(const void* q, const void* k, const void* v, int64_t kv_bh_stride, void* workspace,
                     int64_t workspace_bytes, void* out, float* lse, int B, int H, int Sq, int Skv, int D,
                     float scale, int causal, int out_dtype, int out_heads, int out_h0, hipStream_t stream) {
    if (!workspace) {
        AttnRanges r;
        const int st = check_attn(q, k, v, kv_bh_stride, out, lse, B, H, H, Sq, Skv, D, scale, out_dtype, &r,
                                  out_heads, out_h0);
        return st != DIT_OK ? st : DIT_ERR_NULL;
    }
    if (out_heads < 1) return DIT_ERR_SHAPE;
    return attn_common(q, k, v, kv_bh_stride, workspace, workspace_bytes, out, lse, B, H, H, Sq, Skv, D, scale,
                       causal, out_dtype, nullptr, nullptr, nullptr, stream, out_heads, out_h0);
}

int attn_fwd_ws_merge(const void* q, const void* k, const void* v, int64_t kv_bh_stride, void* workspace,
                      int64_t workspace_bytes, void* out_a, float* lse_a, int B, int H, int Sq, int Skv, int D,
                      float scale, int causal, int a_dtype, hipStream_t stream) {
    if (!workspace || !lse_a) {
        AttnRanges r;
        const int st = check_attn(q, k, v, kv_bh_stride, out_a, lse_a, B, H, H, Sq, Skv, D, scale, a_dtype, &r);
        return st != DIT_OK ? st : DIT_ERR_NULL;
    }
    return attn_common(q, k, v, kv_bh_stride, workspace, workspace_bytes, out_a, lse_a, B, H, H, Sq, Skv, D, scale,
                       causal, a_dtype, nullptr, nullptr, nullptr, stream, 0, 0, true);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* workspace, int64_t workspace_bytes,
                    void* out, float* lse, const int* seqlens_q, const int* seqlens_kv, int B, int H, int Hkv,
                    int Sq, int Skv, int D, float scale, int causal, int out_dtype, hipStream_t stream) {
    if (!seqlens_q || !seqlens_kv) {
        AttnRanges r;
        const int st = check_attn(q, k, v, (int64_t)Skv * D, out, lse, B, H, Hkv, Sq, Skv, D, scale, out_dtype, &r);
        return st != DIT_OK ? st : DIT_ERR_NULL;
    }
    if (Skv < 1 || D < 1) return !q || !k || !v || !out ? DIT_ERR_NULL : DIT_ERR_SHAPE;
    return attn_common(q, k, v, (int64_t)Skv * D, workspace, workspace_bytes, out, lse, B, H, Hkv, Sq, Skv, D,
                       scale, causal, out_dtype, nullptr, seqlens_q, seqlens_kv, stream);
}

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Sq,
             int Skv, int D, float scale, int causal, int out_dtype, hipStream_t stream) {
    if (Skv < 1 || D < 1) return !q || !k || !v || !out ? DIT_ERR_NULL : DIT_ERR_SHAPE;
    return attn_fwd_kv_strided(q, k, v, (int64_t)Skv * D, out, lse, B, H, Sq, Skv, D, scale, causal,
                               out_dtype, stream);
}

int attn_merge(void* out_a, float* lse_a, const void* out_b, const float* lse_b, int B, int H, int Sq,
               int D, int a_dtype, int b_dtype, hipStream_t stream) {
    if (!out_a || !lse_a || !out_b || !lse_b) return DIT_ERR_NULL;
    if (B < 1 || H < 1 || Sq < 1 || D < 1) return DIT_ERR_SHAPE;
    if (D != 64 && D != 128) return DIT_ERR_UNSUPPORTED;
    if ((a_dtype != DIT_BF16 && a_dtype != DIT_FP32) || (b_dtype != DIT_BF16 && b_dtype != DIT_FP32))
        return DIT_ERR_UNSUPPORTED;
    const int64_t rows = (int64_t)B * H * Sq;
    if (rows * D > kMaxElems) return DIT_ERR_SHAPE;
    if (!aligned(out_a, 16) || !aligned(out_b, 16) || !aligned(lse_a, 4) || !aligned(lse_b, 4))
        return DIT_ERR_ALIGN;
    const Range ra = range_of(out_a, rows * D * (a_dtype == DIT_FP32 ? 4 : 2));
    const Range rb = range_of(out_b, rows * D * (b_dtype == DIT_FP32 ? 4 : 2));
    const Range rla = range_of(lse_a, rows * 4), rlb = range_of(lse_b, rows * 4);
    if (overlap(ra, rla) || overlap(rb, ra) || overlap(rb, rla) || overlap(rlb, ra) || overlap(rlb, rla))
        return DIT_ERR_ALIAS;
    (void)hipGetLastError();
    return hip_status(dit::launch_attn_merge(out_a, lse_a, out_b, lse_b, rows, D, a_dtype == DIT_FP32,
                                             b_dtype == DIT_FP32, stream));
}

int bsnd_to_bnsd(const void* x, void* out, int B, int S, int H, int h0, int Hs, int D, hipStream_t stream) {
    const int st = check_layout(x, out, B, S, H, h0, Hs, D);
    if (st != DIT_OK) return st;
    (void)hipGetLastError();
    return hip_status(dit::launch_layout(x, out, B, S, H, h0, Hs, D, true, stream));
}

int bnsd_to_bsnd(const void* o, void* x, int B, int S, int H, int h0, int Hs, int D, hipStream_t stream) {
    const int st = check_layout(x, o, B, S, H, h0, Hs, D);
    if (st != DIT_OK) return st;
    (void)hipGetLastError();
    return hip_status(dit::launch_layout(o, x, B, S, H, h0, Hs, D, false, stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// attn_fwd_noalloc: attn_fwd_ws with its V-image workspace in a static device
// array instead of a caller buffer.  The array lives in this file; host code
// reaches it only through the address hipGetSymbolAddress returns for the
// current device (its name is a host-side stand-in, not a device address).

namespace {

constexpr int64_t kScratchBytes = (int64_t)64 << 20;   // DIT_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == DIT_NOALLOC_SCRATCH_BYTES, "header and library agree on the scratch size");
constexpr int kMaxDevices = 64;

__device__ __align__(256) static unsigned char scratch[kScratchBytes];

// Device address of `scratch` on each device, looked up on the first call
// there (with that device current) and kept until the process ends.
std::atomic<void*> g_scratch_addr[kMaxDevices];

int scratch_address(hipStream_t stream, void** addr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DIT_ERR_HIP;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return DIT_ERR_HIP;
        if ((int)sdev != dev) return DIT_ERR_DEVICE;
    }
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DIT_ERR_HIP;
        g_scratch_addr[dev].store(p, std::memory_order_release);
    }
    *addr = p;
    return DIT_OK;
}

}  // namespace

extern "C" {

int attn_fwd_noalloc(const void* q, const void* k, const void* v, int64_t kv_bh_stride, void* out, float* lse,
                     int B, int H, int Sq, int Skv, int D, float scale, int causal, int out_dtype,
                     hipStream_t stream) {
    AttnRanges r;
    const int st = check_attn(q, k, v, kv_bh_stride, out, lse, B, H, H, Sq, Skv, D, scale, out_dtype, &r);
    if (st != DIT_OK) return st;
    // Heads whose V images fit in the scratch together run as one group;
    // the groups run one after another on the stream.
    const int64_t per_head = dit::v_prep_bytes(1, Skv, D);
    if (per_head > kScratchBytes) return DIT_ERR_SCRATCH;
    const int64_t BH = (int64_t)B * H;
    const int64_t group = BH < kScratchBytes / per_head ? BH : kScratchBytes / per_head;
    void* ws = nullptr;
    const int sa = scratch_address(stream, &ws);
    if (sa != DIT_OK) return sa;
    const int64_t esize = out_dtype == DIT_FP32 ? 4 : 2;
    (void)hipGetLastError();
    for (int64_t h0 = 0; h0 < BH; h0 += group) {
        const int n = (int)(BH - h0 < group ? BH - h0 : group);
        const char* qg = (const char*)q + h0 * Sq * D * 2;
        const char* kg = (const char*)k + h0 * kv_bh_stride * 2;
        const char* vg = (const char*)v + h0 * kv_bh_stride * 2;
        char* og = (char*)out + h0 * Sq * D * esize;
        float* lg = lse ? lse + h0 * Sq : nullptr;
        hipError_t e = dit::launch_v_prep(vg, kv_bh_stride, ws, n, Skv, D, nullptr, n, stream);
        if (e != hipSuccess) return DIT_ERR_HIP;
        e = dit::launch_attn_fwd(qg, kg, vg, kv_bh_stride, og, lg, n, n, 1, Sq, Skv, D, scale, causal != 0,
                                 out_dtype == DIT_FP32, ws, nullptr, nullptr, nullptr, nullptr, 0, 0, false, stream);
        if (e != hipSuccess) return DIT_ERR_HIP;
    }
    return DIT_OK;
}

const char* dit_attn_status_string(int status) {
    switch (status) {
        case DIT_OK: return "ok";
        case DIT_ERR_NULL: return "a required pointer is NULL";
        case DIT_ERR_SHAPE: return "invalid size, stride or scalar argument";
        case DIT_ERR_UNSUPPORTED: return "unsupported head dimension or dtype code";
        case DIT_ERR_ALIGN: return "pointer or stride breaks the alignment rule";
        case DIT_ERR_ALIAS: return "an output overlaps an input it must not overlap";
        case DIT_ERR_HIP: return "the HIP runtime reported a launch error";
        case DIT_ERR_SCRATCH: return "one head's V images exceed the library's static scratch buffer";
        case DIT_ERR_DEVICE: return "the stream belongs to another device than the current one";
        default: return "unknown status";
    }
}

const char* dit_attn_version(void) { return "dit_attn 0.1.0 gfx950"; }

}  // extern "C"

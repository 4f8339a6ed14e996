/*
 * dit_attn.h -- C ABI of libdit_attn.so, the MI355X (gfx950) attention hot
 * path of video and image diffusion transformers:
 *
 *   qk_norm_rope   per-head RMSNorm of q and k, then interleaved rotary, in place
 *   qk_norm_rope_out  the same into separate outputs
 *   attn_fwd       softmax(scale * Q K^T) V with a per-row log-sum-exp (BNSD)
 *   attn_fwd_gqa   the same with Hkv K/V heads shared by H query heads
 *   attn_fwd_varlen  the same over padded batches with per-batch lengths
 *   attn_fwd_ws_fused_q  attention with the query prologue fused into its Q load
 *   attn_fwd_ws_bsnd  attention storing its output into a head slice of a BSND tensor
 *   attn_fwd_ws_merge  attention over one key chunk merged into a running (out, lse)
 *   attn_fwd_noalloc  attn_fwd_ws with its workspace in a static device buffer
 *   attn_merge     fold of two partial attentions over disjoint key sets
 *   bsnd_to_bnsd, bnsd_to_bsnd  head-slice layout change of Ulysses sequence parallelism
 *
 * Sources of the operations (page title, section):
 *   [COSMOS] "Cosmos 昇腾 NPU 多卡并行优化说明": §3.1 fused attention on BNSD
 *            tensors with an explicit scale and a causal switch; §3.2 RMSNorm;
 *            §3.3 rotary embedding.
 *   [WAN]    "NPU Wan2.2-I2V模型推理优化实践": npu_fused_infer_attention_score
 *            section (BNSD, softmax scale, non-causal/causal), rotary_mul
 *            section (interleave mode), rms_norm section, Ring Attention
 *            Overlap (two attention outputs merged through their LSE).
 *   [PR274]  "feat: support Ascend NPU backend (torch_npu) for Qwen-Image
 *            pipelines - #274": change list item 2 (ring attention folds
 *            chunk results with update_out_and_lse).
 *
 * Conventions shared by every call
 *   - Tensors are contiguous row-major device buffers.  BNSD means
 *     q [B,H,Sq,D], k and v [B,H,Skv,D], out [B,H,Sq,D]; lse is fp32 [B,H,Sq].
 *   - bf16 is IEEE bfloat16; conversions to it round to nearest even.
 *   - D must be 64 or 128.  All sizes must be >= 1.  Offsets are 64-bit.
 *   - Tensor pointers must be 16-byte aligned; lse pointers 4-byte aligned.
 *   - The caller owns every buffer.  The library allocates nothing, frees
 *     nothing, never synchronises and prints nothing.  Its only mutable
 *     global state is the static scratch buffer of attn_fwd_noalloc (and the
 *     per-device address of it); every other call is thread-safe and
 *     reentrant.
 *   - Each call validates its arguments, then only enqueues work on
 *     `stream` (NULL = the default stream) and returns.  Buffers must stay
 *     alive until that work completes.  Invalid arguments are reported
 *     before anything is launched; there is no fallback path of any kind.
 *   - Return value: a dit_attn_status code.
 */
#ifndef DIT_ATTN_H
#define DIT_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same declaration as HIP's own; a caller may pass any hipStream_t. */
typedef struct ihipStream_t *hipStream_t;

enum dit_attn_status {
    DIT_OK = 0,
    DIT_ERR_NULL = 1,        /* a required pointer is NULL */
    DIT_ERR_SHAPE = 2,       /* a size is < 1, or sizes are inconsistent/overflow */
    DIT_ERR_UNSUPPORTED = 3, /* D not in {64,128}, or an unknown dtype code */
    DIT_ERR_ALIGN = 4,       /* a pointer or stride breaks the alignment rule */
    DIT_ERR_ALIAS = 5,       /* an output overlaps an input it must not overlap */
    DIT_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
    DIT_ERR_SCRATCH = 7,     /* attn_fwd_noalloc: the shape needs more than its static scratch */
    DIT_ERR_DEVICE = 8       /* attn_fwd_noalloc: the stream is not on the current device */
};

enum dit_attn_dtype {
    DIT_BF16 = 0,
    DIT_FP32 = 1
};

/*
 * Per-head RMSNorm followed by interleaved rotary embedding, in place.
 * [COSMOS] §3.2 and [WAN] rms_norm: for every (b,h,s) row x of q (weight
 * w_q) and of k (weight w_k), y_d = x_d / sqrt(mean_d x_d^2 + eps) * w_d.
 * [COSMOS] §3.3 and [WAN] rotary_mul (interleave): adjacent pairs rotate with
 * the tables taken elementwise at (s, d):
 *   z_{2i}   = y_{2i}   cos[s,2i]   - y_{2i+1} sin[s,2i]
 *   z_{2i+1} = y_{2i+1} cos[s,2i+1] + y_{2i}   sin[s,2i+1]
 * Arithmetic in fp32; one rounding to bf16 at the end.
 *
 *   q, k      bf16 [B,H,S,D], read and overwritten.  Either may be NULL to
 *             leave that tensor alone (not both); they must not overlap.
 *   w_q, w_k  fp32 [D]; required exactly when q (resp. k) is given.
 *   cos, sin  fp32 [S,D], shared by every (b,h) and by q and k.  To rotate a
 *             slice of a longer sequence, pass the table rows of that slice.
 *   eps       added to the mean square (>= 0 and finite).
 */
int qk_norm_rope(void *q, void *k, const float *w_q, const float *w_k,
                 const float *cos, const float *sin, float eps,
                 int B, int H, int S, int D, hipStream_t stream);

/*
 * qk_norm_rope writing its results to separate outputs: q_out <- the
 * normalised, rotated q_in, and k_out <- that of k_in, with the same
 * arithmetic and bits as the in-place form. A model's projections produce
 * fresh q and k every layer, so the in-place form suits them. This form
 * keeps the inputs intact.
 *
 *   q_in, k_in    bf16 [B,H,S,D], read only. q_in and q_out are both NULL
 *                 or both given (same for k); not all four NULL.
 *   q_out, k_out  bf16 [B,H,S,D], written. An output may be exactly its own
 *                 input (the in-place form); otherwise it must not overlap
 *                 either input, the other output, the tables or the weights.
 * Other arguments and errors are as for qk_norm_rope. DIT_ERR_NULL when an
 * input and its output are not both given.
 */
int qk_norm_rope_out(const void *q_in, const void *k_in, void *q_out, void *k_out,
                     const float *w_q, const float *w_k, const float *cos, const float *sin,
                     float eps, int B, int H, int S, int D, hipStream_t stream);

/*
 * Flash attention forward with per-row LSE.  [COSMOS] §3.1 and [WAN]
 * npu_fused_infer_attention_score: for each (b,h) and query row i,
 *   s_j = scale * q_i . k_j,  O_i = sum_j softmax_j(s) v_j,
 *   lse_i = ln sum_j exp(s_j)   (natural log, of the scaled logits)
 * over all keys j < Skv (causal = 0), or over j <= i (causal = 1: top-left
 * aligned, so row i >= Skv sees every key).  Q K^T is a bf16 MFMA product
 * and P V an fp16 MFMA product (P rounded to fp16, V converted from bf16),
 * both with fp32 accumulation; the softmax runs in fp32.
 *
 *   q          bf16 [B,H,Sq,D]
 *   k, v       bf16 [B,H,Skv,D].  Here (no workspace) v must satisfy
 *              |v| <= 65504: its fp16 conversion is exact for |v| in
 *              [2^-14, 65504], smaller magnitudes keep an absolute accuracy
 *              of 2^-25, larger ones overflow: a value of column d beyond
 *              65504 turns column d of the output rows into +-inf or NaN
 *              (the call only enqueues work, so its status cannot report
 *              it; the other columns and the LSE are unaffected).  The
 *              workspace entry points (attn_fwd_ws and the calls built on
 *              it) take any bf16 v.
 *   out        [B,H,Sq,D], bf16 (out_dtype = DIT_BF16) or fp32 (DIT_FP32);
 *              must not overlap q, k, v or lse
 *   lse        fp32 [B,H,Sq], or NULL to skip it
 *   scale      any finite value (typically 1/sqrt(D))
 */
int attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
             int B, int H, int Sq, int Skv, int D, float scale, int causal,
             int out_dtype, hipStream_t stream);

/*
 * attn_fwd over keys that are a window of longer per-head K/V buffers: key j
 * of head (b,h) is read at k + (b*H + h) * kv_bh_stride + j * D (same for v).
 * This is how a key chunk [c0, c1) of a [B,H,S,D] tensor is passed without
 * a copy (k + c0*D, v + c0*D, Skv = c1 - c0, kv_bh_stride = S*D), e.g. the
 * local-chunk / remote-chunks split of [WAN] Ring Attention Overlap.
 * kv_bh_stride >= Skv*D and a multiple of 8 elements.  Otherwise as attn_fwd.
 */
int attn_fwd_kv_strided(const void *q, const void *k, const void *v, int64_t kv_bh_stride,
                        void *out, float *lse, int B, int H, int Sq, int Skv, int D,
                        float scale, int causal, int out_dtype, hipStream_t stream);

/*
 * attn_fwd_kv_strided (same arguments and results) with a caller-provided
 * workspace that lets the kernel stream V without converting it: first
 * launches write each 64-key tile of V once as an fp16, transposed tile image
 * into `workspace`, and the attention launch copies those images straight
 * into LDS.  Faster than attn_fwd on the same inputs.  Any bf16 v is taken:
 * a column (head, d) whose largest |v| is 2^16 or more is scaled by an exact
 * power of two 2^-e into fp16 range before the conversion, and the output's
 * component d is multiplied back by 2^e (values far below the column's
 * largest then keep an absolute accuracy of 2^(e-25)).
 *
 *   workspace        device buffer, 16-byte aligned, overlapping no other
 *                    argument.  Its contents are scratch: overwritten by
 *                    every call, meaningless afterwards.  Calls that share a
 *                    workspace must be ordered on one stream.
 *   workspace_bytes  its size: at least the V part, B*H * (ceil(Skv/64) * 64
 *                    * D * 2 + D * 4) bytes (DIT_ERR_SHAPE when smaller).
 *                    With attn_fwd_workspace_bytes(B, H, Skv, D) bytes (the
 *                    V part plus a split region of fixed size) full
 *                    attention may take the split launch, see below.
 *
 * Launch forms (attn_fwd_launch_form tells which one a call takes).  Query
 * tiles of 256 rows run one per CU.  When the last round of tiles is partly
 * filled:
 *   - with the split region, and when it is estimated to be faster, the key
 *     tiles of that round's query tiles are dealt in equal shares to one
 *     workgroup per CU; a query tile cut between shares is assembled from
 *     its pieces' normalised rows and LSEs with the arithmetic of
 *     attn_merge, in key order, by a fold launch that follows.  The rows of
 *     those tiles then differ from attn_fwd's in rounding only;
 *   - otherwise, when that round is at most half full, it runs as 4-wave
 *     workgroups of 128 rows (same arithmetic).
 * Without the split launch, and for |v| <= 65504, the results are the bits
 * of attn_fwd.
 */
int attn_fwd_ws(const void *q, const void *k, const void *v, int64_t kv_bh_stride,
                void *workspace, int64_t workspace_bytes, void *out, float *lse,
                int B, int H, int Sq, int Skv, int D, float scale, int causal,
                int out_dtype, hipStream_t stream);

/* Workspace bytes for every launch form of attn_fwd_ws: the V part
 * B*H * (ceil(Skv/64) * 64 * D * 2 + D * 4) (the V tile images and the largest
 * |v| of every (head, d)) plus the split region, 512 * 256 * (D + 1) * 4
 * bytes (the LSEs and fp32 rows of up to 512 partial pieces of 256 query
 * rows).  -1 for arguments attn_fwd_ws would reject. */
int64_t attn_fwd_workspace_bytes(int B, int H, int Skv, int D);

/* Launch form codes of attn_fwd_launch_form. */
enum {
    DIT_FORM_ONE = 0,     /* one launch of 8-wave workgroups */
    DIT_FORM_HALVES = 1,  /* full rounds, then the last round as 4-wave halves */
    DIT_FORM_SPLIT = 2,   /* full rounds, then the split launch */
    DIT_FORM_ALL4 = 3     /* 4-wave workgroups throughout (small causal grids) */
};

/* The launch form an attention call with these sizes takes on the device of
 * `stream` (or the current device for the null stream): workspace_bytes = 0
 * for a call without a workspace, Hkv K/V heads, varlen != 0 for
 * attn_fwd_varlen.  Writes a DIT_FORM_* code to *form.  Errors: DIT_ERR_NULL
 * (form), DIT_ERR_SHAPE (sizes an attention call would reject, or a
 * workspace smaller than the V part). */
int attn_fwd_launch_form(int B, int H, int Hkv, int Sq, int Skv, int D, int causal, int varlen,
                         int64_t workspace_bytes, hipStream_t stream, int *form);

/*
 * Grouped-query attention: [WAN] npu_fused_infer_attention_score takes a
 * num_key_value_heads argument, so Hkv K/V heads serve H query heads.
 *
 * Query head (b,h) attends to K/V head (b, h / (H/Hkv)). That K/V head is read
 * at k + (b*Hkv + h/(H/Hkv)) * kv_bh_stride + j*D (same for v). H must be a
 * multiple of Hkv, and Hkv = H is plain multi-head attention. q, out and lse
 * are [B,H,...] as in attn_fwd; k and v hold B*Hkv heads.
 *
 * The workspace is optional:
 *   - NULL: runs the path of attn_fwd_kv_strided.
 *   - non-NULL: runs the path of attn_fwd_ws. It needs at least
 *     attn_fwd_workspace_bytes(B, Hkv, Skv, D) bytes; V is rewritten once per
 *     K/V head.
 * Both paths give identical bits unless the split launch runs (see
 * attn_fwd_ws). Other arguments, results and errors are as for attn_fwd_ws.
 * DIT_ERR_SHAPE when Hkv < 1 or H % Hkv != 0.
 */
int attn_fwd_gqa(const void *q, const void *k, const void *v, int64_t kv_bh_stride,
                 void *workspace, int64_t workspace_bytes, void *out, float *lse,
                 int B, int H, int Hkv, int Sq, int Skv, int D, float scale, int causal,
                 int out_dtype, hipStream_t stream);

/*
 * Variable-length batches: [WAN] npu_fused_infer_attention_score takes
 * actual_seq_lengths and actual_seq_lengths_kv. q, k and v are padded
 * tensors: q [B,H,Sq,D], k and v [B,Hkv,Skv,D] contiguous (Hkv as in
 * attn_fwd_gqa). Batch b holds seqlens_q[b] valid query rows and
 * seqlens_kv[b] valid keys.
 *
 * Valid rows attend to the valid keys only; causal means j <= i as in
 * attn_fwd. Padding rows (i >= seqlens_q[b]) and rows that see no key store
 * out = 0 and lse = -inf, so a later attn_merge ignores them.
 *
 *   seqlens_q, seqlens_kv  device int32 [B], 4-byte aligned, read by the
 *                          kernels on the stream. Values are clamped to
 *                          [0, Sq] and [0, Skv]; they are not checked on the
 *                          host. Neither may overlap out, lse or the workspace.
 *   workspace              optional, as in attn_fwd_gqa.
 *
 * Other arguments and errors are as for attn_fwd_gqa with
 * kv_bh_stride = Skv*D.
 */
int attn_fwd_varlen(const void *q, const void *k, const void *v, void *workspace,
                    int64_t workspace_bytes, void *out, float *lse, const int *seqlens_q,
                    const int *seqlens_kv, int B, int H, int Hkv, int Sq, int Skv, int D,
                    float scale, int causal, int out_dtype, hipStream_t stream);

/*
 * attn_fwd_ws with the query half of qk_norm_rope fused into the attention's
 * query load ([COSMOS] §3.2-§3.3, [WAN] rms_norm and rotary_mul sections).
 * q holds the raw query rows and is only read. Each row is normalised over D,
 * weighted by w_q and rotated with the tables at its own position i, exactly
 * as qk_norm_rope computes it, then rounded to bf16. The results are the bits
 * of qk_norm_rope(q, NULL, w_q, ...) followed by attn_fwd_ws. k must already
 * hold normalised, rotated keys (e.g. qk_norm_rope with q = NULL).
 *
 *   w_q           fp32 [D], 16-byte aligned
 *   cos_q, sin_q  fp32 [Sq, D], 16-byte aligned; row i belongs to query row i
 *   eps           >= 0 and finite
 * Neither the tables nor w_q may overlap out, lse or the workspace. All other
 * arguments and errors are as for attn_fwd_ws.
 */
int attn_fwd_ws_fused_q(const void *q, const void *k, const void *v, int64_t kv_bh_stride,
                        void *workspace, int64_t workspace_bytes, void *out, float *lse,
                        const float *w_q, const float *cos_q, const float *sin_q, float eps,
                        int B, int H, int Sq, int Skv, int D, float scale, int causal,
                        int out_dtype, hipStream_t stream);

/*
 * attn_fwd_ws with the output stored in the model's BSND layout.
 * [WAN] npu_fused_infer_attention_score returns BNSD and the caller
 * transposes it back to [B,S,N,D]. [PR274] item 2 (npu_ulysses_attention)
 * does the same before its all-to-all. Here the attention epilogue writes
 * each row straight to its BSND place:
 *   out[b, i, out_h0 + h, :] = attention row (b, h, i)
 * The other heads of out are not touched. lse stays fp32 [B,H,Sq].
 *
 *   out        [B, Sq, out_heads, D] of out_dtype
 *   out_heads  >= H; out_h0 satisfies 0 <= out_h0 <= out_heads - H
 *
 * The bits are those of attn_fwd_ws followed by bnsd_to_bsnd (for bf16 out).
 * DIT_ERR_SHAPE for a bad out_heads or out_h0. out must not overlap q, k, v,
 * lse or the workspace over its whole BSND extent. All other arguments and
 * errors are as for attn_fwd_ws.
 */
int attn_fwd_ws_bsnd(const void *q, const void *k, const void *v, int64_t kv_bh_stride,
                     void *workspace, int64_t workspace_bytes, void *out, float *lse,
                     int B, int H, int Sq, int Skv, int D, float scale, int causal,
                     int out_dtype, int out_heads, int out_h0, hipStream_t stream);

/*
 * attn_fwd_ws over one key chunk, folded into a running partial result in
 * the same call. [WAN] Ring Attention Overlap merges the attention of each
 * key chunk into the running output through the LSEs; [PR274] item 2 does
 * this with update_out_and_lse. Here the attention epilogue does the merge,
 * so the chunk's output never goes to memory.
 *
 *   out_a  [B,H,Sq,D] of a_dtype (DIT_BF16 or DIT_FP32), read and written.
 *          On entry it holds the attention of the same queries over other
 *          keys (e.g. an attn_fwd_ws result).
 *   lse_a  fp32 [B,H,Sq], read and written; required (NULL: DIT_ERR_NULL).
 *
 * The bits are those of attn_fwd_ws(q, k, v, ..., tmp, tmp_lse) with an fp32
 * tmp, followed by attn_merge(out_a, lse_a, tmp, tmp_lse, ..., a_dtype,
 * DIT_FP32). Other arguments and errors are as for attn_fwd_ws, with out_a
 * in the place of out. As there, causal counts the keys of this chunk from
 * 0 (j <= i); the pages' ring and sequence-parallel attention is non-causal.
 */
int attn_fwd_ws_merge(const void *q, const void *k, const void *v, int64_t kv_bh_stride,
                      void *workspace, int64_t workspace_bytes, void *out_a, float *lse_a,
                      int B, int H, int Sq, int Skv, int D, float scale, int causal,
                      int a_dtype, hipStream_t stream);

/*
 * Merge of two partial attentions over disjoint key sets, in place into
 * (out_a, lse_a).  [WAN] Ring Attention Overlap, [PR274] item 2
 * (update_out_and_lse).  Per row:
 *   M = max(la, lb),  L = M + ln(exp(la - M) + exp(lb - M)),
 *   out_a <- exp(la - L) out_a + exp(lb - L) out_b,  lse_a <- L.
 * A row whose two LSEs are both -inf (no key seen) becomes out_a = 0,
 * lse_a = -inf.  fp32 arithmetic; one rounding per call when out_a is bf16.
 *
 *   out_a   [B,H,Sq,D] of a_dtype (DIT_BF16 or DIT_FP32), read and written
 *   lse_a   fp32 [B,H,Sq], read and written
 *   out_b   [B,H,Sq,D] of b_dtype, read only; must not overlap out_a/lse_a
 *   lse_b   fp32 [B,H,Sq], read only; must not overlap out_a/lse_a
 */
int attn_merge(void *out_a, float *lse_a, const void *out_b, const float *lse_b,
               int B, int H, int Sq, int D, int a_dtype, int b_dtype, hipStream_t stream);

/*
 * Head-slice layout change around the all-to-all of Ulysses sequence
 * parallelism. [PR274] item 2 (npu_ulysses_attention) gathers the sequence
 * and splits the heads, runs the fused attention on BNSD, then does the
 * all-to-all back. [WAN] npu_fused_infer_attention_score produces BNSD that
 * the caller transposes.
 *
 * The model's activations are BSND, x [B,S,H,D]. The attention of the head
 * slice [h0, h0+Hs) wants BNSD, [B,Hs,S,D]:
 *   bsnd_to_bnsd:  out[b,h,s,d] = x[b,s,h0+h,d]
 *   bnsd_to_bsnd:  x[b,s,h0+h,d] = o[b,h,s,d]   (the other heads of x untouched)
 *
 * Elements are 2-byte values (bf16) copied bit for bit.
 *   - D is a multiple of 8.
 *   - 0 <= h0 <= H - Hs.
 *   - The BSND tensor and the BNSD slice must not overlap.
 */
int bsnd_to_bnsd(const void *x, void *out, int B, int S, int H, int h0, int Hs, int D,
                 hipStream_t stream);
int bnsd_to_bsnd(const void *o, void *x, int B, int S, int H, int h0, int Hs, int D,
                 hipStream_t stream);

/*
 * attn_fwd_ws without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the V images that attn_fwd_ws writes into its
 * workspace go to a static device buffer of DIT_NOALLOC_SCRATCH_BYTES inside
 * the library (each GPU the library runs on holds its own copy from the first
 * call until the process ends).  The call allocates nothing.
 *
 * Arguments, layouts and results are those of attn_fwd_ws (the bits of
 * attn_fwd_ws with a workspace of the V part only: no split launch).  The
 * heads are processed in groups whose V images fit in the buffer, one group
 * after another on `stream`.  Limit: one head's share, ceil(Skv/64) * 64 *
 * D * 2 + D * 4 bytes (Skv <= 262080 at D = 128, 524224 at D = 64), must
 * fit, else DIT_ERR_SCRATCH before anything is launched.
 *
 * `stream` must belong to the current device (DIT_ERR_DEVICE otherwise); the
 * first call on a device looks up that device's buffer address.  Every call
 * on a GPU uses that GPU's one buffer: calls that may run at the same time
 * on one GPU (on different streams, or from different threads) race on it
 * and give undefined results; order them on one stream.
 */
#define DIT_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)
int attn_fwd_noalloc(const void *q, const void *k, const void *v, int64_t kv_bh_stride,
                     void *out, float *lse, int B, int H, int Sq, int Skv, int D,
                     float scale, int causal, int out_dtype, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *dit_attn_status_string(int status);

/* Static version string of the library. */
const char *dit_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIT_ATTN_H */

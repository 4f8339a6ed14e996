"""Thin ctypes binding of libdit_attn.so (argument marshalling only).

Every step of the path runs in the library's HIP kernels; this module only
checks tensor metadata, passes ``data_ptr()`` values, sizes and the current
torch stream, and turns a non-zero status into ``DitAttnError``.  There is no
fallback: if the library is missing, the first call raises.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already mapped (both carry the soname libamdhip64.so.7),
and torch's stream handles are valid inside it.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdit_attn.so")

DIT_BF16 = 0
DIT_FP32 = 1

_lib = None


class DitAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m attention_qk_norm_rope_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    p, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.qk_norm_rope.argtypes = [p, p, p, p, p, p, f32, i32, i32, i32, i32, p]
    lib.qk_norm_rope_out.argtypes = [p, p, p, p, p, p, p, p, f32, i32, i32, i32, i32, p]
    lib.attn_fwd.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.attn_fwd_kv_strided.argtypes = [p, p, p, i64, p, p, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.attn_fwd_ws.argtypes = [p, p, p, i64, p, i64, p, p, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.attn_fwd_gqa.argtypes = [p, p, p, i64, p, i64, p, p, i32, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.attn_fwd_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.attn_fwd_workspace_bytes.restype = i64
    lib.attn_fwd_launch_form.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i64, p, ctypes.POINTER(i32)]
    lib.attn_fwd_ws_fused_q.argtypes = [p, p, p, i64, p, i64, p, p, p, p, p, f32, i32, i32, i32, i32, i32, f32, i32,
                                        i32, p]
    lib.attn_fwd_ws_bsnd.argtypes = [p, p, p, i64, p, i64, p, p, i32, i32, i32, i32, i32, f32, i32, i32, i32, i32, p]
    lib.attn_fwd_ws_merge.argtypes = [p, p, p, i64, p, i64, p, p, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.attn_merge.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, i32, p]
    lib.attn_fwd_noalloc.argtypes = [p, p, p, i64, p, p, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.attn_fwd_varlen.argtypes = [p, p, p, p, i64, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.bsnd_to_bnsd.argtypes = [p, p, i32, i32, i32, i32, i32, i32, p]
    lib.bnsd_to_bsnd.argtypes = [p, p, i32, i32, i32, i32, i32, i32, p]
    for name in ("qk_norm_rope", "qk_norm_rope_out", "attn_fwd", "attn_fwd_kv_strided", "attn_fwd_ws", "attn_fwd_gqa", "attn_fwd_ws_fused_q",
                 "attn_fwd_ws_bsnd", "attn_fwd_ws_merge", "attn_fwd_varlen", "attn_merge", "bsnd_to_bnsd", "bnsd_to_bsnd",
                 "attn_fwd_noalloc", "attn_fwd_launch_form"):
        getattr(lib, name).restype = i32
    lib.dit_attn_status_string.argtypes = [i32]
    lib.dit_attn_status_string.restype = ctypes.c_char_p
    lib.dit_attn_version.argtypes = []
    lib.dit_attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def library_path() -> str:
    _load()
    return LIB_PATH


def status_string(status: int) -> str:
    return _load().dit_attn_status_string(int(status)).decode()


def version() -> str:
    return _load().dit_attn_version().decode()


def _check(fn: str, status: int):
    if status != 0:
        raise DitAttnError(fn, status, status_string(status))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _dtype_code(t) -> int:
    if t.dtype == torch.bfloat16:
        return DIT_BF16
    if t.dtype == torch.float32:
        return DIT_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def qk_norm_rope(q, k, w_q, w_k, cos, sin, eps: float):
    """In-place per-head RMSNorm + interleaved RoPE of q and/or k (bf16 BNSD).

    Either q or k may be None.  w_q/w_k: fp32 [D]; cos, sin: fp32 [S, D].
    """
    ref = q if q is not None else k
    if ref is None:
        raise ValueError("q and k are both None")
    dev = ref.device
    B, H, S, D = ref.shape
    for t, name in ((q, "q"), (k, "k")):
        if t is not None:
            _need(t, name, torch.bfloat16, dev)
            if tuple(t.shape) != (B, H, S, D) or not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous [{B},{H},{S},{D}]")
    for t, name, use in ((w_q, "w_q", q is not None), (w_k, "w_k", k is not None)):
        if use:
            _need(t, name, torch.float32, dev)
            if tuple(t.shape) != (D,) or not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous [{D}]")
    for t, name in ((cos, "cos"), (sin, "sin")):
        _need(t, name, torch.float32, dev)
        if tuple(t.shape) != (S, D) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [{S},{D}]")
    st = _load().qk_norm_rope(_ptr(q), _ptr(k), _ptr(w_q if q is not None else None),
                              _ptr(w_k if k is not None else None), _ptr(cos), _ptr(sin),
                              float(eps), B, H, S, D, _stream())
    _check("qk_norm_rope", st)
    return q, k


def qk_norm_rope_out(q, k, q_out, k_out, w_q, w_k, cos, sin, eps: float):
    """qk_norm_rope into separate outputs: q_out <- prologue(q), k_out <-
    prologue(k), inputs left intact (an output may also be its own input).
    Either pair may be None.  Same bits as the in-place form.  Returns
    (q_out, k_out)."""
    ref = q if q is not None else k
    if ref is None:
        raise ValueError("q and k are both None")
    if (q is None) != (q_out is None) or (k is None) != (k_out is None):
        raise ValueError("an input and its output must both be given or both be None")
    dev = ref.device
    B, H, S, D = ref.shape
    for t, name in ((q, "q"), (k, "k"), (q_out, "q_out"), (k_out, "k_out")):
        if t is not None:
            _need(t, name, torch.bfloat16, dev)
            if tuple(t.shape) != (B, H, S, D) or not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous [{B},{H},{S},{D}]")
    for t, name, use in ((w_q, "w_q", q is not None), (w_k, "w_k", k is not None)):
        if use:
            _need(t, name, torch.float32, dev)
            if tuple(t.shape) != (D,) or not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous [{D}]")
    for t, name in ((cos, "cos"), (sin, "sin")):
        _need(t, name, torch.float32, dev)
        if tuple(t.shape) != (S, D) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [{S},{D}]")
    st = _load().qk_norm_rope_out(_ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out),
                                  _ptr(w_q if q is not None else None), _ptr(w_k if k is not None else None),
                                  _ptr(cos), _ptr(sin), float(eps), B, H, S, D, _stream())
    _check("qk_norm_rope_out", st)
    return q_out, k_out


def _kv_bh_stride(t, B, H, S, D) -> int | None:
    """Stride between (b,h) slabs if t is [B,H,S,D] with rows of D contiguous
    elements and the slabs evenly spaced (contiguous, or a window along S)."""
    if tuple(t.shape) != (B, H, S, D):
        return None
    s0, s1, s2, s3 = t.stride()
    if s3 != 1 or s2 != D:
        return None
    if H > 1 and B > 1 and s0 != H * s1:
        return None
    if H == 1:
        s1 = s0 if B > 1 else S * D
    return s1


def _attn_args(q, k, v, out, lse, scale, out_dtype, return_lse, kv_heads=None, bsnd_out=False):
    _need(q, "q", torch.bfloat16, q.device)
    dev = q.device
    _need(k, "k", torch.bfloat16, dev)
    _need(v, "v", torch.bfloat16, dev)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D BNSD")
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    Hkv = H if kv_heads is None else kv_heads
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    sk = _kv_bh_stride(k, B, Hkv, Skv, D)
    sv = _kv_bh_stride(v, B, Hkv, Skv, D)
    if sk is None or sv is None or sk != sv:
        raise ValueError("k and v must be [B,H,Skv,D] with contiguous rows and the same (b,h) stride")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if bsnd_out:
        if (not isinstance(out, torch.Tensor) or out.dim() != 4 or out.shape[0] != B or out.shape[1] != Sq
                or out.shape[3] != D or not out.is_contiguous()):
            raise ValueError(f"out must be a contiguous BSND tensor [{B},{Sq},heads,{D}]")
        if out.device != dev:
            raise ValueError("out is on another device")
    elif out is None:
        out = torch.empty((B, H, Sq, D), dtype=out_dtype, device=dev)
    else:
        if tuple(out.shape) != (B, H, Sq, D) or not out.is_contiguous():
            raise ValueError("out must be contiguous [B,H,Sq,D]")
        if out.device != dev:
            raise ValueError("out is on another device")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev)
        if tuple(lse.shape) != (B, H, Sq) or not lse.is_contiguous():
            raise ValueError("lse must be contiguous fp32 [B,H,Sq]")
    return (B, H, Sq, Skv, D), int(sk), float(scale), out, lse


def attn_fwd(q, k, v, out=None, lse=None, scale: float | None = None, causal: bool = False,
             out_dtype=torch.bfloat16, return_lse: bool = True):
    """softmax(scale * q k^T) v with per-row LSE (natural log), BNSD.

    q: bf16 [B,H,Sq,D] contiguous.  k, v: bf16 [B,H,Skv,D], contiguous or
    windows along S of longer per-head buffers (same strides for k and v).
    Returns (out, lse); lse is None when return_lse is False and no lse given.
    """
    (B, H, Sq, Skv, D), sk, scale, out, lse = _attn_args(q, k, v, out, lse, scale, out_dtype, return_lse)
    code = _dtype_code(out)
    lib = _load()
    if k.is_contiguous() and v.is_contiguous():
        st = lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Sq, Skv, D,
                          scale, 1 if causal else 0, code, _stream())
        _check("attn_fwd", st)
    else:
        st = lib.attn_fwd_kv_strided(_ptr(q), _ptr(k), _ptr(v), sk, _ptr(out), _ptr(lse), B, H,
                                     Sq, Skv, D, scale, 1 if causal else 0, code, _stream())
        _check("attn_fwd_kv_strided", st)
    return out, lse


def attn_fwd_workspace_bytes(B: int, H: int, Skv: int, D: int) -> int:
    """Bytes of device workspace attn_fwd_ws needs for these sizes."""
    n = int(_load().attn_fwd_workspace_bytes(int(B), int(H), int(Skv), int(D)))
    if n < 0:
        raise ValueError(f"no workspace size for B={B} H={H} Skv={Skv} D={D}")
    return n


FORMS = {0: "one", 1: "halves", 2: "split", 3: "all4"}


def attn_fwd_launch_form(B: int, H: int, Sq: int, Skv: int, D: int, causal: bool = False,
                         workspace_bytes: int = 0, Hkv: int | None = None, varlen: bool = False) -> str:
    """Launch form ("one", "halves", "split" or "all4") that an attention call
    with these sizes takes on the current device; workspace_bytes = 0 for a
    call without a workspace."""
    form = ctypes.c_int(-1)
    st = _load().attn_fwd_launch_form(int(B), int(H), int(H if Hkv is None else Hkv), int(Sq), int(Skv), int(D),
                                      1 if causal else 0, 1 if varlen else 0, int(workspace_bytes), _stream(),
                                      ctypes.byref(form))
    _check("attn_fwd_launch_form", st)
    return FORMS[form.value]


def attn_fwd_ws(q, k, v, workspace, out=None, lse=None, scale: float | None = None,
                causal: bool = False, out_dtype=torch.bfloat16, return_lse: bool = True):
    """attn_fwd with a caller-owned device workspace (a contiguous tensor,
    any dtype, of attn_fwd_workspace_bytes(B, H, Skv, D) bytes, or of at least
    the V part B*H*(ceil(Skv/64)*64*D*2 + D*4) bytes, which rules out the split
    launch).  Same results as attn_fwd, faster: V is first rewritten into the
    workspace in the kernel's tile layout.  The workspace holds scratch
    afterwards."""
    (B, H, Sq, Skv, D), sk, scale, out, lse = _attn_args(q, k, v, out, lse, scale, out_dtype, return_lse)
    if not isinstance(workspace, torch.Tensor) or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _load().attn_fwd_ws(_ptr(q), _ptr(k), _ptr(v), sk, _ptr(workspace), ws_bytes, _ptr(out),
                             _ptr(lse), B, H, Sq, Skv, D, scale, 1 if causal else 0, _dtype_code(out),
                             _stream())
    _check("attn_fwd_ws", st)
    return out, lse


def attn_fwd_noalloc(q, k, v, out=None, lse=None, scale: float | None = None, causal: bool = False,
                     out_dtype=torch.bfloat16, return_lse: bool = True):
    """attn_fwd_ws with the library's static scratch buffer in place of a
    workspace: the library call allocates no device memory (pass out and lse
    to allocate nothing here either).  Same bits as attn_fwd_ws.  Calls that
    may overlap on one GPU share that buffer and must be ordered on one
    stream."""
    (B, H, Sq, Skv, D), sk, scale, out, lse = _attn_args(q, k, v, out, lse, scale, out_dtype, return_lse)
    st = _load().attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), sk, _ptr(out), _ptr(lse), B, H, Sq, Skv, D, scale,
                                  1 if causal else 0, _dtype_code(out), _stream())
    _check("attn_fwd_noalloc", st)
    return out, lse


def attn_fwd_gqa(q, k, v, workspace=None, out=None, lse=None, scale: float | None = None,
                 causal: bool = False, out_dtype=torch.bfloat16, return_lse: bool = True):
    """Grouped-query attention: q bf16 [B,H,Sq,D]; k, v bf16 [B,Hkv,Skv,D]
    (contiguous or key windows), H a multiple of Hkv; query head h reads K/V
    head h // (H // Hkv).  With a workspace (at least
    attn_fwd_workspace_bytes(B, Hkv, Skv, D) bytes) the workspace path runs.
    Returns (out, lse)."""
    if k.dim() != 4:
        raise ValueError("k must be 4-D [B,Hkv,Skv,D]")
    Hkv = k.shape[1]
    (B, H, Sq, Skv, D), sk, scale, out, lse = _attn_args(q, k, v, out, lse, scale, out_dtype, return_lse,
                                                         kv_heads=Hkv)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    st = _load().attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), sk, ws_ptr, ws_bytes, _ptr(out), _ptr(lse), B, H, Hkv,
                              Sq, Skv, D, scale, 1 if causal else 0, _dtype_code(out), _stream())
    _check("attn_fwd_gqa", st)
    return out, lse


def attn_fwd_varlen(q, k, v, seqlens_q, seqlens_kv, workspace=None, out=None, lse=None,
                    scale: float | None = None, causal: bool = False, out_dtype=torch.bfloat16,
                    return_lse: bool = True):
    """Attention over padded batches: q bf16 [B,H,Sq,D]; k, v bf16
    [B,Hkv,Skv,D] contiguous; seqlens_q / seqlens_kv int32 [B] device tensors
    (valid query rows / keys per batch).  Padding rows get out = 0 and
    lse = -inf.  Optional workspace as in attn_fwd_gqa.  Returns (out, lse)."""
    if k.dim() != 4 or not k.is_contiguous() or not v.is_contiguous():
        raise ValueError("k and v must be contiguous [B,Hkv,Skv,D]")
    Hkv = k.shape[1]
    (B, H, Sq, Skv, D), sk, scale, out, lse = _attn_args(q, k, v, out, lse, scale, out_dtype, return_lse,
                                                         kv_heads=Hkv)
    for t, name in ((seqlens_q, "seqlens_q"), (seqlens_kv, "seqlens_kv")):
        _need(t, name, torch.int32, q.device)
        if tuple(t.shape) != (B,) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous int32 [{B}]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    st = _load().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), ws_ptr, ws_bytes, _ptr(out), _ptr(lse),
                                 _ptr(seqlens_q), _ptr(seqlens_kv), B, H, Hkv, Sq, Skv, D, scale,
                                 1 if causal else 0, _dtype_code(out), _stream())
    _check("attn_fwd_varlen", st)
    return out, lse


def attn_fwd_ws_fused_q(q, k, v, workspace, w_q, cos_q, sin_q, eps: float, out=None, lse=None,
                        scale: float | None = None, causal: bool = False, out_dtype=torch.bfloat16,
                        return_lse: bool = True):
    """attn_fwd_ws with the query RMSNorm + rotary fused into the Q load: q
    holds raw rows (read only); w_q fp32 [D]; cos_q, sin_q fp32 [Sq, D].  k
    must already be normalised and rotated.  Same bits as
    qk_norm_rope(q, None, w_q, None, cos_q, sin_q, eps) then attn_fwd_ws."""
    (B, H, Sq, Skv, D), sk, scale, out, lse = _attn_args(q, k, v, out, lse, scale, out_dtype, return_lse)
    if not isinstance(workspace, torch.Tensor) or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    _need(w_q, "w_q", torch.float32, q.device)
    if tuple(w_q.shape) != (D,) or not w_q.is_contiguous():
        raise ValueError(f"w_q must be contiguous [{D}]")
    for t, name in ((cos_q, "cos_q"), (sin_q, "sin_q")):
        _need(t, name, torch.float32, q.device)
        if tuple(t.shape) != (Sq, D) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [{Sq},{D}]")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _load().attn_fwd_ws_fused_q(_ptr(q), _ptr(k), _ptr(v), sk, _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse),
                                     _ptr(w_q), _ptr(cos_q), _ptr(sin_q), float(eps), B, H, Sq, Skv, D, scale,
                                     1 if causal else 0, _dtype_code(out), _stream())
    _check("attn_fwd_ws_fused_q", st)
    return out, lse


def attn_fwd_ws_bsnd(q, k, v, workspace, out, out_h0: int = 0, lse=None, scale: float | None = None,
                     causal: bool = False, return_lse: bool = True):
    """attn_fwd_ws whose epilogue stores into the model's BSND layout: out is
    a contiguous bf16 or fp32 tensor [B, Sq, heads, D]; query head h writes
    out[:, :, out_h0 + h, :] and the other heads are left as they are.
    lse stays fp32 [B,H,Sq].  Returns (out, lse)."""
    (B, H, Sq, Skv, D), sk, scale, out, lse = _attn_args(q, k, v, out, lse, scale, None, return_lse,
                                                         bsnd_out=True)
    if not isinstance(workspace, torch.Tensor) or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _load().attn_fwd_ws_bsnd(_ptr(q), _ptr(k), _ptr(v), sk, _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse),
                                  B, H, Sq, Skv, D, scale, 1 if causal else 0, _dtype_code(out),
                                  int(out.shape[2]), int(out_h0), _stream())
    _check("attn_fwd_ws_bsnd", st)
    return out, lse


def attn_fwd_ws_merge(q, k, v, workspace, out_a, lse_a, scale: float | None = None, causal: bool = False):
    """Attention of q over (k, v) merged in place into the running partial
    result (out_a bf16/fp32 [B,H,Sq,D], lse_a fp32 [B,H,Sq]) of the same
    queries over other keys.  Same bits as attn_fwd_ws into an fp32
    temporary followed by attn_merge.  Returns (out_a, lse_a)."""
    if lse_a is None:
        raise ValueError("lse_a is required")
    (B, H, Sq, Skv, D), sk, scale, out_a, lse_a = _attn_args(q, k, v, out_a, lse_a, scale, None, True)
    if not isinstance(workspace, torch.Tensor) or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _load().attn_fwd_ws_merge(_ptr(q), _ptr(k), _ptr(v), sk, _ptr(workspace), ws_bytes, _ptr(out_a),
                                   _ptr(lse_a), B, H, Sq, Skv, D, scale, 1 if causal else 0, _dtype_code(out_a),
                                   _stream())
    _check("attn_fwd_ws_merge", st)
    return out_a, lse_a


def attn_merge(out_a, lse_a, out_b, lse_b):
    """In-place merge of (out_b, lse_b) into (out_a, lse_a).  Returns them."""
    dev = out_a.device
    if out_a.dim() != 4:
        raise ValueError("out_a must be [B,H,Sq,D]")
    B, H, Sq, D = out_a.shape
    for t, name in ((out_a, "out_a"), (out_b, "out_b")):
        if tuple(t.shape) != (B, H, Sq, D) or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be contiguous [{B},{H},{Sq},{D}] on {dev}")
    for t, name in ((lse_a, "lse_a"), (lse_b, "lse_b")):
        _need(t, name, torch.float32, dev)
        if tuple(t.shape) != (B, H, Sq) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous fp32 [{B},{H},{Sq}]")
    st = _load().attn_merge(_ptr(out_a), _ptr(lse_a), _ptr(out_b), _ptr(lse_b), B, H, Sq, D,
                            _dtype_code(out_a), _dtype_code(out_b), _stream())
    _check("attn_merge", st)
    return out_a, lse_a


def attn_fwd_ring_overlap(q, k, v, split: int, ws_local, ws_remote, out_local=None, lse_local=None,
                          out_remote=None, lse_remote=None, scale: float | None = None,
                          side_stream=None):
    """The ring-overlap split on one GPU: attention of q over the keys
    [0, split) ("local") and over [split, Skv) ("remote"), merged through the
    LSE into fp32 (out_local, lse_local), which are returned.

    With a side_stream (a torch.cuda.Stream of default priority) the local
    call runs on it, concurrently with the remote call on the current stream;
    the current stream waits for both before the merge.  Without one, both
    run in order on the current stream.  Each call needs its own workspace
    (attn_fwd_workspace_bytes of its key count) when they run concurrently.
    Non-causal only (a key split has no causal offset).
    """
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if not 0 < split < Skv:
        raise ValueError(f"split must be in (0, {Skv})")
    if side_stream is not None and ws_local.data_ptr() == ws_remote.data_ptr():
        raise ValueError("concurrent calls need two workspaces")
    mk = lambda: torch.empty((B, H, Sq, D), dtype=torch.float32, device=q.device)  # noqa: E731
    ml = lambda: torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)  # noqa: E731
    out_local = mk() if out_local is None else out_local
    lse_local = ml() if lse_local is None else lse_local
    out_remote = mk() if out_remote is None else out_remote
    lse_remote = ml() if lse_remote is None else lse_remote
    main = torch.cuda.current_stream(q.device)
    if side_stream is None:
        attn_fwd_ws(q, k[:, :, :split], v[:, :, :split], ws_local, out=out_local, lse=lse_local, scale=scale)
        attn_fwd_ws(q, k[:, :, split:], v[:, :, split:], ws_remote, out=out_remote, lse=lse_remote, scale=scale)
    else:
        side_stream.wait_stream(main)          # inputs written on the current stream
        with torch.cuda.stream(side_stream):
            attn_fwd_ws(q, k[:, :, :split], v[:, :, :split], ws_local, out=out_local, lse=lse_local, scale=scale)
        attn_fwd_ws(q, k[:, :, split:], v[:, :, split:], ws_remote, out=out_remote, lse=lse_remote, scale=scale)
        main.wait_stream(side_stream)
    attn_merge(out_local, lse_local, out_remote, lse_remote)
    return out_local, lse_local


def _layout_check(x, name):
    if not isinstance(x, torch.Tensor) or x.dim() != 4 or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 4-D tensor")
    if x.element_size() != 2:
        raise TypeError(f"{name} must have 2-byte elements (bf16)")


def bsnd_to_bnsd(x, h0: int = 0, heads: int | None = None, out=None):
    """Head slice [h0, h0+heads) of BSND x [B,S,H,D] as BNSD [B,heads,S,D]."""
    _layout_check(x, "x")
    B, S, H, D = x.shape
    heads = H - h0 if heads is None else heads
    if out is None:
        out = torch.empty((B, heads, S, D), dtype=x.dtype, device=x.device)
    _layout_check(out, "out")
    if tuple(out.shape) != (B, heads, S, D) or out.device != x.device:
        raise ValueError(f"out must be [{B},{heads},{S},{D}] on {x.device}")
    st = _load().bsnd_to_bnsd(_ptr(x), _ptr(out), B, S, H, h0, heads, D, _stream())
    _check("bsnd_to_bnsd", st)
    return out


def bnsd_to_bsnd(o, x, h0: int = 0):
    """Write BNSD o [B,Hs,S,D] into the head slice [h0, h0+Hs) of BSND x
    [B,S,H,D] (other heads untouched).  Returns x."""
    _layout_check(o, "o")
    _layout_check(x, "x")
    B, Hs, S, D = o.shape
    if x.shape[0] != B or x.shape[1] != S or x.shape[3] != D or x.device != o.device:
        raise ValueError("x must be [B,S,H,D] matching o [B,Hs,S,D] on the same device")
    st = _load().bnsd_to_bsnd(_ptr(o), _ptr(x), B, S, x.shape[2], h0, Hs, D, _stream())
    _check("bnsd_to_bsnd", st)
    return x

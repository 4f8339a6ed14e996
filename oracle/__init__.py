"""fp64 CPU oracle for the DiT attention hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it and
has no fallback to it.  The arithmetic lives in ``oracle.c`` (plain C, fp64,
two-pass softmax straight from the definitions); this module only builds that
file with gcc and marshals numpy arrays into it.

Definitions followed (cited by page title and section):
  * attention, LSE -- "Cosmos 昇腾 NPU 多卡并行优化说明" §3.1 (BNSD fused attention,
    explicit scale, causal switch) and "NPU Wan2.2-I2V模型推理优化实践"
    (npu_fused_infer_attention_score section);
  * RMSNorm + interleaved rotary -- Cosmos page §3.2 and §3.3, Wan2.2 page
    (rms_norm and rotary_mul sections, interleave mode);
  * out/LSE merge -- Wan2.2 page, "Ring Attention Overlap", and
    "feat: support Ascend NPU backend ... #274", change list item 2
    (update_out_and_lse);
  * BSND <-> BNSD head-slice layout -- #274 change list item 2
    (npu_ulysses_attention: gather the sequence, split the heads) and the
    Wan2.2 page (attention output in BNSD, transposed by the caller); written
    here with numpy indexing.

Every function is pinned by the CPU tests in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build() -> str:
    """Compile oracle.c with gcc into liboracle.so next to it (always rebuilds)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", _SRC, "-lm", "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # A library older than its source would check against stale arithmetic.
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    p = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_attn.argtypes = [p, p, p, i32, i32, i32, i32, i32, f64, i32, p, i64, p, p, i32]
    lib.oracle_attn.restype = i32
    lib.oracle_qk_norm_rope.argtypes = [p, p, p, p, f64, i32, i32, i32, i32, p, i32]
    lib.oracle_qk_norm_rope.restype = i32
    lib.oracle_merge.argtypes = [p, p, p, p, i64, i32, p, p]
    lib.oracle_merge.restype = i32
    _lib = lib
    return lib


def default_threads() -> int:
    """Host threads for the oracle: every CPU this process may run on, or the
    CPU share that OMP_NUM_THREADS states when it is set (a host with several
    GPUs gives each GPU's jobs a share of its cores)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _bits(a, name):
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name} must hold bf16 bit patterns (uint16), got {a.dtype}")
    return np.ascontiguousarray(a)


def attn(q, k, v, scale: float, causal: bool = False, rows=None, nthreads: int | None = None):
    """Exact attention in fp64.

    q: uint16 bf16 bits [B,H,Sq,D]; k, v: [B,H,Skv,D].  rows: optional flat
    query-row ids ((b*H + h)*Sq + i).  Returns (out [n_rows, D] fp64,
    lse [n_rows] fp64); with rows=None, out is shaped [B,H,Sq,D] and lse
    [B,H,Sq].
    """
    q, k, v = _bits(q, "q"), _bits(k, "k"), _bits(v, "v")
    B, H, Sq, D = q.shape
    Bk, Hk, Skv, Dk = k.shape
    if (Bk, Hk, Dk) != (B, H, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if rows is None:
        n = B * H * Sq
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows_arr.size
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load().oracle_attn(_ptr(q), _ptr(k), _ptr(v), B, H, Sq, Skv, D, float(scale),
                             1 if causal else 0,
                             None if rows_arr is None else _ptr(rows_arr), n,
                             _ptr(out), _ptr(lse), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attn rejected its arguments")
    if rows is None:
        return out.reshape(B, H, Sq, D), lse.reshape(B, H, Sq)
    return out, lse


def qk_norm_rope(x, w, cos, sin, eps: float, nthreads: int | None = None):
    """RMSNorm over D per (b,h,s) row, then interleaved rotary, in fp64.

    x: uint16 bf16 bits [B,H,S,D]; w: fp32 [D]; cos, sin: fp32 [S,D].
    Returns fp64 [B,H,S,D] (unrounded).
    """
    x = _bits(x, "x")
    B, H, S, D = x.shape
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float32))
    cos = np.ascontiguousarray(np.asarray(cos, dtype=np.float32))
    sin = np.ascontiguousarray(np.asarray(sin, dtype=np.float32))
    if w.shape != (D,) or cos.shape != (S, D) or sin.shape != (S, D):
        raise ValueError("w must be [D], cos and sin [S,D]")
    out = np.empty((B, H, S, D), dtype=np.float64)
    rc = _load().oracle_qk_norm_rope(_ptr(x), _ptr(w), _ptr(cos), _ptr(sin), float(eps),
                                     B, H, S, D, _ptr(out), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_qk_norm_rope rejected its arguments")
    return out


def merge(out_a, lse_a, out_b, lse_b):
    """Exact two-way out/LSE merge in fp64.  out_*: [..., D]; lse_*: [...]."""
    oa = np.ascontiguousarray(np.asarray(out_a, dtype=np.float64))
    ob = np.ascontiguousarray(np.asarray(out_b, dtype=np.float64))
    la = np.ascontiguousarray(np.asarray(lse_a, dtype=np.float64))
    lb = np.ascontiguousarray(np.asarray(lse_b, dtype=np.float64))
    if oa.shape != ob.shape or la.shape != lb.shape or oa.shape[:-1] != la.shape:
        raise ValueError("merge operands disagree in shape")
    D = oa.shape[-1]
    rows = la.size
    out = np.empty_like(oa)
    lse = np.empty_like(la)
    rc = _load().oracle_merge(_ptr(oa), _ptr(la), _ptr(ob), _ptr(lb), rows, D, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_merge rejected its arguments")
    return out, lse


def bsnd_to_bnsd(x, h0: int = 0, heads: int | None = None):
    """out[b, h, s, d] = x[b, s, h0 + h, d] for the head slice [h0, h0+heads)
    of a BSND array x [B,S,H,D].  Returns a new contiguous [B,heads,S,D]."""
    x = np.asarray(x)
    B, S, H, D = x.shape
    heads = H - h0 if heads is None else heads
    if not (0 <= h0 and heads >= 1 and h0 + heads <= H):
        raise ValueError("head slice out of range")
    return np.ascontiguousarray(x[:, :, h0:h0 + heads, :].transpose(0, 2, 1, 3))


def bnsd_to_bsnd(o, x, h0: int = 0):
    """x[b, s, h0 + h, d] = o[b, h, s, d]; returns a copy of x [B,S,H,D] with
    that head slice replaced and the other heads as they were."""
    o = np.asarray(o)
    y = np.array(x, copy=True)
    B, Hs, S, D = o.shape
    if y.shape[0] != B or y.shape[1] != S or y.shape[3] != D or not (0 <= h0 and h0 + Hs <= y.shape[2]):
        raise ValueError("shape mismatch")
    y[:, :, h0:h0 + Hs, :] = o.transpose(0, 2, 1, 3)
    return y


def attn_varlen(q, k, v, seqlens_q, seqlens_kv, scale: float, causal: bool = False):
    """Attention over padded batches, from the definition: batch b is full
    attention of its first seqlens_q[b] query rows over its first
    seqlens_kv[b] keys (K/V head h // (H // Hkv) for query head h: H/Hkv
    consecutive query heads share one K/V head, the grouping of the fused
    attention's num_key_value_heads on the Wan2.2 NPU page); padding rows,
    and rows that see no key, are 0 with LSE -inf.  q [B,H,Sq,D], k, v
    [B,Hkv,Skv,D] bf16 bits.  Returns fp64 out [B,H,Sq,D], lse [B,H,Sq]."""
    q, k, v = _bits(q, "q"), _bits(k, "k"), _bits(v, "v")
    B, H, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    out = np.zeros((B, H, Sq, D), dtype=np.float64)
    lse = np.full((B, H, Sq), -np.inf, dtype=np.float64)
    for b in range(B):
        lq = int(min(max(seqlens_q[b], 0), Sq))
        lk = int(min(max(seqlens_kv[b], 0), Skv))
        if lq == 0 or lk == 0:
            continue
        kb = np.repeat(k[b:b + 1, :, :lk], H // Hkv, axis=1)
        vb = np.repeat(v[b:b + 1, :, :lk], H // Hkv, axis=1)
        o, l = attn(np.ascontiguousarray(q[b:b + 1, :, :lq]), np.ascontiguousarray(kb), np.ascontiguousarray(vb),
                    scale, causal)
        out[b, :, :lq] = o[0]
        lse[b, :, :lq] = l[0]
    return out, lse

"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/dit_attn.h declares, and rejects bad arguments with the
documented status before anything is launched.

Every call here is meant to fail validation, so no HIP call is made and no
pointer is dereferenced (fake, suitably aligned addresses are used).  Because
a mistake in one of these cases would launch a kernel on fake addresses, the
module refuses to run where a GPU is visible; the GPU suite covers the same
status codes with real buffers.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit_attn.h")
LIB = os.path.join(ROOT, "attention_qk_norm_rope_amd", "libdit_attn.so")

OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, HIP, SCRATCH, DEVICE = range(9)
BF16, FP32 = 0, 1


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("fake-pointer validation tests run only where no GPU is visible")
    if not os.path.exists(LIB):
        from attention_qk_norm_rope_amd import build
        build.build()
    lib = ctypes.CDLL(LIB)
    p, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.qk_norm_rope.argtypes = [p, p, p, p, p, p, f32, i32, i32, i32, i32, p]
    lib.qk_norm_rope_out.argtypes = [p, p, p, p, p, p, p, p, f32, i32, i32, i32, i32, p]
    lib.attn_fwd.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.attn_fwd_kv_strided.argtypes = [p, p, p, i64, p, p, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.attn_fwd_ws.argtypes = [p, p, p, i64, p, i64, p, p, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.attn_fwd_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.attn_fwd_workspace_bytes.restype = i64
    lib.attn_fwd_gqa.argtypes = [p, p, p, i64, p, i64, p, p, i32, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.attn_fwd_ws_fused_q.argtypes = [p, p, p, i64, p, i64, p, p, p, p, p, f32, i32, i32, i32, i32, i32, f32, i32,
                                        i32, p]
    lib.attn_fwd_ws_bsnd.argtypes = [p, p, p, i64, p, i64, p, p, i32, i32, i32, i32, i32, f32, i32, i32, i32, i32, p]
    lib.attn_fwd_ws_merge.argtypes = [p, p, p, i64, p, i64, p, p, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.attn_merge.argtypes = [p, p, p, p, i32, i32, i32, i32, i32, i32, p]
    lib.attn_fwd_varlen.argtypes = [p, p, p, p, i64, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.bsnd_to_bnsd.argtypes = [p, p, i32, i32, i32, i32, i32, i32, p]
    lib.bnsd_to_bsnd.argtypes = [p, p, i32, i32, i32, i32, i32, i32, p]
    lib.attn_fwd_noalloc.argtypes = [p, p, p, i64, p, p, i32, i32, i32, i32, i32, f32, i32, i32, p]
    lib.attn_fwd_launch_form.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i64, p, ctypes.POINTER(i32)]
    lib.dit_attn_status_string.restype = ctypes.c_char_p
    lib.dit_attn_version.restype = ctypes.c_char_p
    return lib


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert set(names) == {"qk_norm_rope", "qk_norm_rope_out", "attn_fwd", "attn_fwd_kv_strided", "attn_fwd_ws",
                          "attn_fwd_workspace_bytes", "attn_fwd_launch_form", "attn_fwd_gqa", "attn_fwd_ws_fused_q", "attn_fwd_ws_bsnd", "attn_fwd_ws_merge", "attn_fwd_varlen", "attn_fwd_noalloc", "attn_merge", "bsnd_to_bnsd",
                          "bnsd_to_bsnd", "dit_attn_status_string",
                          "dit_attn_version"}, names
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    for s in range(9):
        assert lib.dit_attn_status_string(s) != b"unknown status"
    assert lib.dit_attn_status_string(99) == b"unknown status"
    assert b"gfx950" in lib.dit_attn_version()


# Fake device addresses far apart, 256-byte aligned.
Q, K, V, O, L, W1, W2, C, S_ = (0x10_0000_0000 * (i + 1) for i in range(9))


def attn(lib, q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Sq=256, Skv=256, D=64, scale=0.125, causal=0, dt=BF16):
    return lib.attn_fwd(q, k, v, o, lse, B, H, Sq, Skv, D, scale, causal, dt, None)


def test_attn_fwd_rejections(lib):
    assert attn(lib, q=None) == NULL
    assert attn(lib, o=None) == NULL
    assert attn(lib, Sq=0) == SHAPE
    assert attn(lib, Skv=0) == SHAPE
    assert attn(lib, B=0) == SHAPE
    assert attn(lib, H=-1) == SHAPE
    assert attn(lib, D=96) == UNSUP
    assert attn(lib, D=256) == UNSUP
    assert attn(lib, dt=2) == UNSUP
    assert attn(lib, scale=float("inf")) == SHAPE
    assert attn(lib, scale=float("nan")) == SHAPE
    assert attn(lib, q=Q + 8) == ALIGN
    assert attn(lib, o=O + 4) == ALIGN
    assert attn(lib, lse=L + 2) == ALIGN
    assert attn(lib, o=Q) == ALIAS                       # out on q
    assert attn(lib, o=K + 32 * 1024) == ALIAS           # out inside k (k spans 64 KiB)
    assert attn(lib, lse=O + 1024) == ALIAS              # lse inside out
    assert attn(lib, B=1 << 16, H=1 << 16) == SHAPE      # B*H overflows int


def test_attn_fwd_noalloc_rejections(lib):
    f = lib.attn_fwd_noalloc
    D = 128
    assert f(None, K, V, 256 * D, O, L, 1, 2, 256, 256, D, 0.125, 0, BF16, None) == NULL
    assert f(Q, K, V, 256 * D, O, L, 1, 2, 0, 256, D, 0.125, 0, BF16, None) == SHAPE
    assert f(Q, K, V, 256 * D, O, L, 1, 2, 256, 256, 96, 0.125, 0, BF16, None) == UNSUP
    assert f(Q + 8, K, V, 256 * D, O, L, 1, 2, 256, 256, D, 0.125, 0, BF16, None) == ALIGN
    assert f(Q, K, V, 256 * D, Q, L, 1, 2, 256, 256, D, 0.125, 0, BF16, None) == ALIAS
    # One head's V images and column maxima (ceil(Skv/64)*64*D*2 + D*4 bytes)
    # must fit in the 64 MiB static scratch: 262080 keys fit at D = 128,
    # 262144 do not.
    big = 262144
    assert f(Q, K, V, big * D, O, L, 1, 1, 256, big, D, 0.125, 0, BF16, None) == SCRATCH
    assert f(Q, K, V, 600000 * 64, O, L, 1, 1, 256, 600000, 64, 0.125, 0, FP32, None) == SCRATCH


def test_attn_fwd_kv_strided_rejections(lib):
    f = lib.attn_fwd_kv_strided
    assert f(Q, K, V, 255 * 64, O, L, 1, 2, 256, 256, 64, 0.125, 0, BF16, None) == SHAPE  # stride < Skv*D
    assert f(Q, K, V, 256 * 64 + 4, O, L, 1, 2, 256, 256, 64, 0.125, 0, BF16, None) == ALIGN
    # A long stride makes k span into out.
    assert f(Q, K, V, (O - K) // 2, O, L, 1, 2, 256, 256, 64, 0.125, 0, BF16, None) == ALIAS


def split_region(D):
    """Bytes of the split-launch region: the LSE and fp32 rows of 512 partial
    pieces of 256 query rows."""
    return 512 * 256 * (D + 1) * 4


def test_attn_fwd_workspace_bytes(lib):
    f = lib.attn_fwd_workspace_bytes
    # One fp16 image of 64 keys x D per started 64-key tile and head, then
    # one 4-byte column maximum per (head, d), then the split region.
    assert f(1, 2, 256, 64) == 2 * 4 * 64 * 64 * 2 + 2 * 64 * 4 + split_region(64)
    assert f(1, 1, 1, 128) == 64 * 128 * 2 + 128 * 4 + split_region(128)
    assert f(2, 3, 65, 128) == 6 * 2 * 64 * 128 * 2 + 6 * 128 * 4 + split_region(128)
    assert f(1, 40, 75600, 128) == 40 * 1182 * 64 * 128 * 2 + 40 * 128 * 4 + split_region(128)
    assert f(0, 2, 256, 64) == -1
    assert f(1, 2, 0, 64) == -1
    assert f(1, 2, 256, 96) == -1


WS = 0x10_0000_0000 * 12


def test_attn_fwd_ws_rejections(lib):
    f = lib.attn_fwd_ws
    need = 2 * 4 * 64 * 64 * 2 + 2 * 64 * 4

    def call(ws=WS, nbytes=need, k=K, stride=256 * 64, Skv=256, o=O):
        return f(Q, k, V, stride, ws, nbytes, o, L, 1, 2, 256, Skv, 64, 0.125, 0, BF16, None)

    assert call(ws=None) == NULL
    assert call(ws=WS + 8) == ALIGN
    assert call(nbytes=need - 1) == SHAPE
    assert call(nbytes=0) == SHAPE
    assert call(ws=Q + 4096) == ALIAS                    # workspace inside q
    assert call(ws=O - need + 16) == ALIAS               # workspace runs into out
    # With room for the split region, the region is checked against out too.
    full = need + split_region(64)
    assert call(ws=O - full + 16, nbytes=full) == ALIAS
    assert call(ws=L) == ALIAS                           # workspace on lse
    assert call(o=None) == NULL                          # the attention checks come first
    assert call(stride=255 * 64) == SHAPE


def test_attn_fwd_gqa_rejections(lib):
    f = lib.attn_fwd_gqa
    # B1, H4 query heads over Hkv K/V heads of Skv 256, D64.
    def call(Hkv=2, ws=None, nbytes=0, stride=256 * 64, o=O):
        return f(Q, K, V, stride, ws, nbytes, o, L, 1, 4, Hkv, 256, 256, 64, 0.125, 0, BF16, None)

    assert call(Hkv=0) == SHAPE
    assert call(Hkv=3) == SHAPE                          # 4 % 3 != 0
    assert call(Hkv=8) == SHAPE                          # more K/V heads than query heads
    assert call(o=None) == NULL
    assert call(stride=255 * 64) == SHAPE
    need = 2 * 4 * 64 * 64 * 2 + 2 * 64 * 4              # B*Hkv * (4 tiles * 64 keys * D * 2 B + D * 4 B)
    assert call(ws=WS, nbytes=need - 1) == SHAPE         # sized by Hkv, not H
    assert call(ws=WS + 8, nbytes=need) == ALIGN
    assert call(ws=Q + 4096, nbytes=need) == ALIAS


TAB = 0x20_0000_0000


def test_attn_fwd_ws_fused_q_rejections(lib):
    f = lib.attn_fwd_ws_fused_q
    need = 2 * 4 * 64 * 64 * 2 + 2 * 64 * 4
    tb = 256 * 64 * 4                                    # one [Sq, D] fp32 table

    def call(ws=WS, w=TAB, cq=TAB + 4096, sq=TAB + 4096 + tb, eps=1e-6, o=O):
        return f(Q, K, V, 256 * 64, ws, need, o, L, w, cq, sq, eps, 1, 2, 256, 256, 64, 0.125, 0, BF16, None)

    assert call(ws=None) == NULL
    assert call(w=None) == NULL
    assert call(cq=None) == NULL
    assert call(sq=None) == NULL
    assert call(eps=-1.0) == SHAPE
    assert call(eps=float("nan")) == SHAPE
    assert call(w=TAB + 8) == ALIGN
    assert call(cq=TAB + 4096 + 4) == ALIGN
    assert call(cq=O) == ALIAS                           # a table on the output
    assert call(sq=WS) == ALIAS                          # a table on the workspace
    assert call(o=None) == NULL


def test_attn_fwd_ws_bsnd_rejections(lib):
    f = lib.attn_fwd_ws_bsnd
    need = 2 * 4 * 64 * 64 * 2 + 2 * 64 * 4
    # B1, H2, Sq = Skv = 256, D64 into a BSND output of `heads` heads.

    def call(heads=6, h0=2, ws=WS, o=O, dt=BF16, lse=L):
        return f(Q, K, V, 256 * 64, ws, need, o, lse, 1, 2, 256, 256, 64, 0.125, 0, dt, heads, h0, None)

    assert call(ws=None) == NULL
    assert call(o=None) == NULL
    assert call(heads=0) == SHAPE
    assert call(heads=1) == SHAPE                        # fewer output heads than query heads
    assert call(h0=-1) == SHAPE
    assert call(h0=5) == SHAPE                           # heads 5, 6 do not exist
    assert call(heads=2, h0=0, o=O + 8) == ALIGN
    out_bytes = 256 * 6 * 64 * 2
    assert call(lse=O + out_bytes - 1024) == ALIAS       # lse inside the BSND extent
    assert call(ws=O + out_bytes - need + 16) == ALIAS   # workspace runs into out
    assert call(dt=FP32, ws=O + out_bytes) == ALIAS      # fp32 out is twice as long


def test_attn_fwd_ws_merge_rejections(lib):
    f = lib.attn_fwd_ws_merge
    need = 2 * 4 * 64 * 64 * 2 + 2 * 64 * 4

    def call(ws=WS, o=O, lse=L, dt=FP32, nbytes=need):
        return f(Q, K, V, 256 * 64, ws, nbytes, o, lse, 1, 2, 256, 256, 64, 0.125, 0, dt, None)

    assert call(ws=None) == NULL
    assert call(lse=None) == NULL                        # the running LSE is required
    assert call(o=None) == NULL
    assert call(dt=7) == UNSUP
    assert call(nbytes=need - 1) == SHAPE
    assert call(lse=O + 1024) == ALIAS                   # lse inside out_a
    assert call(ws=L) == ALIAS


def test_qk_norm_rope_out_rejections(lib):
    f = lib.qk_norm_rope_out
    n = 2 * 256 * 64 * 2                                 # bytes of one [1,2,256,64] bf16 tensor
    QO, KO = 0x30_0000_0000, 0x31_0000_0000

    def call(qi=Q, ki=K, qo=QO, ko=KO, wq=W1, wk=W2, c=C, s=S_):
        return f(qi, ki, qo, ko, wq, wk, c, s, 1e-6, 1, 2, 256, 64, None)

    assert call(qo=None) == NULL                         # an input without its output
    assert call(ki=None) == NULL                         # an output without its input
    assert call(qi=None, ki=None, qo=None, ko=None) == NULL
    assert call(qo=QO + 8) == ALIGN
    assert call(ki=K + 8) == ALIGN                       # inputs are checked too
    assert call(qo=Q + 1024) == ALIAS                    # partial overlap with its own input
    assert call(qo=K) == ALIAS                           # onto the other input
    assert call(ko=QO + n - 16) == ALIAS                 # the two outputs overlap
    assert call(qo=C) == ALIAS                           # onto a table
    assert call(ko=W1) == ALIAS                          # onto a weight


def test_qk_norm_rope_rejections(lib):
    f = lib.qk_norm_rope
    args = dict(q=Q, k=K, wq=W1, wk=W2, c=C, s=S_, eps=1e-6, B=1, H=2, S=256, D=64)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["q"], a["k"], a["wq"], a["wk"], a["c"], a["s"], a["eps"], a["B"], a["H"], a["S"], a["D"], None)

    assert call(q=None, k=None) == NULL
    assert call(wq=None) == NULL
    assert call(c=None) == NULL
    assert call(S=0) == SHAPE
    assert call(eps=-1.0) == SHAPE
    assert call(eps=float("nan")) == SHAPE
    assert call(D=32) == UNSUP
    assert call(q=Q + 2) == ALIGN
    assert call(c=C + 4) == ALIGN
    assert call(k=Q + 512) == ALIAS                      # q and k overlap
    assert call(c=Q + 1024) == ALIAS                     # table inside q
    assert call(q=None, wq=None, k=K, c=K) == ALIAS      # table on k


def test_attn_merge_rejections(lib):
    f = lib.attn_merge
    assert f(None, L, V, W1, 1, 2, 256, 64, BF16, BF16, None) == NULL
    assert f(O, L, V, W1, 1, 0, 256, 64, BF16, BF16, None) == SHAPE
    assert f(O, L, V, W1, 1, 2, 256, 64, BF16, 3, None) == UNSUP
    assert f(O, L, V, W1, 1, 2, 256, 48, BF16, BF16, None) == UNSUP
    assert f(O + 8, L, V, W1, 1, 2, 256, 64, BF16, BF16, None) == ALIGN
    assert f(O, L + 1, V, W1, 1, 2, 256, 64, BF16, BF16, None) == ALIGN
    assert f(O, L, O + 4096, W1, 1, 2, 256, 64, BF16, BF16, None) == ALIAS
    assert f(O, O + 1024, V, W1, 1, 2, 256, 64, BF16, BF16, None) == ALIAS
    assert f(O, L, V, L, 1, 2, 256, 64, FP32, BF16, None) == ALIAS


@pytest.mark.parametrize("fn", ["bsnd_to_bnsd", "bnsd_to_bsnd"])
def test_layout_rejections(lib, fn):
    f = getattr(lib, fn)
    X, Y = 0x30_0000_0000, 0x40_0000_0000
    assert f(None, Y, 1, 8, 4, 0, 2, 128, None) == NULL
    assert f(X, None, 1, 8, 4, 0, 2, 128, None) == NULL
    assert f(X, Y, 1, 8, 4, 3, 2, 128, None) == SHAPE        # slice past the last head
    assert f(X, Y, 1, 8, 4, -1, 2, 128, None) == SHAPE
    assert f(X, Y, 1, 8, 4, 0, 0, 128, None) == SHAPE
    assert f(X, Y, 0, 8, 4, 0, 2, 128, None) == SHAPE
    assert f(X, Y, 1, 8, 4, 0, 2, 60, None) == UNSUP         # D not a multiple of 8
    assert f(X + 2, Y, 1, 8, 4, 0, 2, 128, None) == ALIGN
    # the BNSD slice inside the BSND tensor (bsnd_to_bnsd takes the BSND side
    # first, bnsd_to_bsnd second)
    src, dst = (X, X + 4096) if fn == "bsnd_to_bnsd" else (X + 4096, X)
    assert f(src, dst, 1, 8, 4, 0, 2, 128, None) == ALIAS


def test_attn_fwd_varlen_rejections(lib):
    f = lib.attn_fwd_varlen
    LQ, LK = 0x50_0000_0000, 0x50_0000_1000

    def call(lq=LQ, lk=LK, Hkv=2, o=O):
        return f(Q, K, V, None, 0, o, L, lq, lk, 1, 2, Hkv, 256, 256, 64, 0.125, 0, BF16, None)

    assert call(lq=None) == NULL
    assert call(lk=None) == NULL
    assert call(lq=LQ + 2) == ALIGN
    assert call(lk=O) == ALIAS                           # lengths on the output
    assert call(Hkv=3) == SHAPE
    assert call(o=None) == NULL


def test_attn_fwd_launch_form_rejections(lib):
    f = lib.attn_fwd_launch_form
    form = ctypes.c_int(-1)
    D = 128
    need = 4 * (64 * D * 2 + D * 4)                      # B1 H4, one 64-key tile

    def call(B=1, H=4, Hkv=4, Sq=256, Skv=64, D=D, nbytes=0, out=True):
        return f(B, H, Hkv, Sq, Skv, D, 0, 0, nbytes, None, ctypes.byref(form) if out else None)

    assert call(out=False) == NULL
    assert call(Sq=0) == SHAPE
    assert call(Skv=0) == SHAPE
    assert call(Hkv=3) == SHAPE
    assert call(D=96) == UNSUP
    assert call(nbytes=-1) == SHAPE
    assert call(nbytes=need - 1) == SHAPE                # smaller than the V part
    assert form.value == -1                              # untouched by a rejected call

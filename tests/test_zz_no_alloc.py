"""attn_fwd_noalloc through the C ABI: the entry point for callers that
cannot allocate (its V images live in the library's static scratch buffer).
It must give the bits of attn_fwd_ws (the entry point with a caller
workspace) given a workspace of the V part only (so that neither takes the
split launch) and agree with the fp64 oracle, on consecutive calls that reuse
the buffer -- the second with a smaller input -- and when the heads do not
all fit in the buffer at once."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import attn_fwd_workspace_bytes, attn_fwd_ws, binding, inputs
from gpu_common import DEV, dev_bits, host_f64, say

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


def _noalloc(q, k, v, out, lse, scale, causal):
    """Direct C-ABI call on preallocated outputs (nothing is allocated)."""
    lib = binding._load()
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    st = lib.attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), Skv * D, out.data_ptr(), lse.data_ptr(),
                              B, H, Sq, Skv, D, ctypes.c_float(scale), 1 if causal else 0,
                              1 if out.dtype == torch.float32 else 0, torch.cuda.current_stream().cuda_stream)
    return st


def _case(seed, B, H, Sq, Skv, D, causal, out_dtype, check_oracle=True):
    scale = 1 / math.sqrt(D)
    q = inputs.random_bits(seed, (B, H, Sq, D))
    k = inputs.random_bits(seed + 1, (B, H, Skv, D))
    v = inputs.random_bits(seed + 2, (B, H, Skv, D))
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    out = torch.full((B, H, Sq, D), float("nan"), dtype=out_dtype, device=DEV)
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=DEV)
    say(f"[noalloc] B{B} H{H} Sq{Sq} Skv{Skv} D{D} causal={causal} {out_dtype}")
    assert _noalloc(dq, dk, dv, out, lse, scale, causal) == 0
    v_part = B * H * (-(-Skv // 64) * 64 * D * 2 + D * 4)
    assert v_part < attn_fwd_workspace_bytes(B, H, Skv, D)
    ws = torch.empty((v_part,), dtype=torch.uint8, device=DEV)
    ro, rl = attn_fwd_ws(dq, dk, dv, ws, scale=scale, causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(out, ro) and torch.equal(lse, rl), "attn_fwd_noalloc differs from attn_fwd_ws"
    if check_oracle:
        ref_o, ref_l = oracle.attn(q, k, v, scale, causal)
        rep = compare.attn_report(host_f64(out), ref_o, host_f64(lse), ref_l, bf16=out_dtype == torch.bfloat16)
        compare.assert_ok(rep, "attn_fwd_noalloc")


def test_two_calls_second_smaller():
    _case(7100, 2, 3, 700, 1000, 128, False, torch.float32)
    _case(7200, 1, 2, 200, 129, 64, True, torch.bfloat16)


def test_heads_in_groups():
    """One head's V images take 51 MB here, so the 3 heads run as 3 groups,
    one after another through the same buffer."""
    D, Skv = 128, 200000
    per_head = -(-Skv // 64) * 64 * D * 2
    assert SCRATCH // per_head == 1
    _case(7300, 1, 3, 300, Skv, D, False, torch.float32, check_oracle=False)
    # a few rows against the oracle (the full oracle over 200000 keys is slow)
    scale = 1 / math.sqrt(D)
    q = inputs.random_bits(7300, (1, 3, 300, D))
    k = inputs.random_bits(7301, (1, 3, Skv, D))
    v = inputs.random_bits(7302, (1, 3, Skv, D))
    out = torch.empty((1, 3, 300, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((1, 3, 300), dtype=torch.float32, device=DEV)
    assert _noalloc(dev_bits(q), dev_bits(k), dev_bits(v), out, lse, scale, False) == 0
    torch.cuda.synchronize()
    rows = np.array([0, 299, 300, 450, 899], dtype=np.int64)
    ref_o, ref_l = oracle.attn(q, k, v, scale, False, rows=rows)
    rep = compare.attn_report(host_f64(out).reshape(-1, D)[rows], ref_o, host_f64(lse).reshape(-1)[rows], ref_l,
                              bf16=False)
    compare.assert_ok(rep, "attn_fwd_noalloc, heads in groups")


def test_rejects_a_head_larger_than_the_buffer():
    D, Skv = 128, 262208               # ceil(Skv/64)*64*D*2 bytes > 64 MiB
    q = torch.zeros((1, 1, 64, D), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((1, 1, Skv, D), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    out = torch.zeros((1, 1, 64, D), dtype=torch.float32, device=DEV)
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device=DEV)
    assert _noalloc(q, k, v, out, lse, 0.1, False) == 7
    assert torch.count_nonzero(out).item() == 0

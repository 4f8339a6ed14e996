"""attn_fwd_ws_merge: the attention over one key chunk folded into a running
(out, lse) by the attention's own epilogue.  It must give the bits of
attn_fwd_ws into an fp32 temporary followed by attn_merge, agree with the
oracle's attention over the union of the key chunks, and ignore a running
side that has seen no key (lse -inf, out NaN)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import attn_fwd_workspace_bytes, attn_fwd_ws, attn_fwd_ws_merge, attn_merge, inputs
from gpu_common import DEV, dev_bits, host_f64, say

pytestmark = pytest.mark.gpu

CASES = [  # B, H, Sq, keys of the running side, keys of the merged chunk, D, running-side dtype
    (1, 3, 300, 200, 333, 64, torch.float32),
    (2, 2, 257, 64, 129, 128, torch.bfloat16),
    (1, 2, 700, 1000, 65, 128, torch.float32),
    (1, 1, 1, 1, 1, 64, torch.bfloat16),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}q{c[2]}a{c[3]}b{c[4]}D{c[5]}"
                                             f"{'f32' if c[6] == torch.float32 else 'bf16'}" for c in CASES])
def test_ws_merge(case):
    B, H, Sq, Ka, Kb, D, a_dtype = case
    seed = 5000 + Sq + Ka + Kb
    q = inputs.random_bits(seed, (B, H, Sq, D))
    k = inputs.random_bits(seed + 1, (B, H, Ka + Kb, D))
    v = inputs.random_bits(seed + 2, (B, H, Ka + Kb, D))
    scale = 1 / math.sqrt(D)
    say(f"[ws_merge] {case}")
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    ka, va = dk[:, :, :Ka].contiguous(), dv[:, :, :Ka].contiguous()
    kb, vb = dk[:, :, Ka:].contiguous(), dv[:, :, Ka:].contiguous()
    ws = torch.empty((attn_fwd_workspace_bytes(B, H, max(Ka, Kb), D),), dtype=torch.uint8, device=DEV)
    oa, la = attn_fwd_ws(dq, ka, va, ws, scale=scale, out_dtype=a_dtype)
    o2, l2 = oa.clone(), la.clone()
    attn_fwd_ws_merge(dq, kb, vb, ws, oa, la, scale=scale)
    t, tl = attn_fwd_ws(dq, kb, vb, ws, scale=scale, out_dtype=torch.float32)
    attn_merge(o2, l2, t, tl)
    torch.cuda.synchronize()
    assert torch.equal(oa, o2) and torch.equal(la, l2), "fused merge differs from attention + attn_merge"
    ref_o, ref_l = oracle.attn(q, k, v, scale, False)
    rep = compare.attn_report(host_f64(oa), ref_o, host_f64(la), ref_l, bf16=a_dtype == torch.bfloat16)
    compare.assert_ok(rep, f"ws merge {case}")


@pytest.mark.parametrize("a_dtype", [torch.float32, torch.bfloat16])
def test_ws_merge_into_empty_side(a_dtype):
    """A running side that saw no key (lse -inf, out NaN) takes the chunk's
    result exactly."""
    B, H, Sq, Skv, D = 1, 2, 300, 250, 128
    q = inputs.random_bits(61, (B, H, Sq, D))
    k = inputs.random_bits(62, (B, H, Skv, D))
    v = inputs.random_bits(63, (B, H, Skv, D))
    say(f"[ws_merge] empty running side {a_dtype}")
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    ws = torch.empty((attn_fwd_workspace_bytes(B, H, Skv, D),), dtype=torch.uint8, device=DEV)
    oa = torch.full((B, H, Sq, D), float("nan"), dtype=a_dtype, device=DEV)
    la = torch.full((B, H, Sq), float("-inf"), dtype=torch.float32, device=DEV)
    attn_fwd_ws_merge(dq, dk, dv, ws, oa, la)
    o1, l1 = attn_fwd_ws(dq, dk, dv, ws, out_dtype=a_dtype)
    torch.cuda.synchronize()
    # The oracle's merge of an empty running side with this chunk's result.
    rows = B * H * Sq
    ref_o, ref_l = oracle.merge(np.full((rows, D), np.nan), np.full(rows, -np.inf),
                                host_f64(o1).reshape(rows, D), host_f64(l1).reshape(rows))
    assert np.array_equal(host_f64(oa).reshape(rows, D), ref_o) and np.array_equal(host_f64(la).reshape(rows), ref_l)
    assert torch.equal(oa, o1) and torch.equal(la, l1)
    assert np.isfinite(host_f64(oa)).all()
    full_o, full_l = oracle.attn(q, k, v, 1 / math.sqrt(D), False)
    rep = compare.attn_report(host_f64(oa), full_o, host_f64(la), full_l, bf16=a_dtype == torch.bfloat16)
    compare.assert_ok(rep, "ws merge into an empty running side")

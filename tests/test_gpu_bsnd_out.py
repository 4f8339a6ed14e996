"""attn_fwd_ws_bsnd: the attention epilogue stores each output row straight
into a head slice of a BSND [B, Sq, heads, D] tensor.  The written heads must
hold the bits of attn_fwd_ws's BNSD output moved by bnsd_to_bsnd, every other
head must keep its contents, and the result must agree with the oracle's
attention put into BSND by the oracle's layout function."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import attn_fwd_workspace_bytes, attn_fwd_ws, attn_fwd_ws_bsnd, inputs
from gpu_common import DEV, dev_bits, host_bits, host_f64, say

pytestmark = pytest.mark.gpu

CASES = [  # B, H, Sq, Skv, D, causal, out dtype, output heads, first head
    (2, 3, 300, 200, 64, False, torch.bfloat16, 5, 1),
    (1, 4, 257, 333, 128, True, torch.float32, 4, 0),
    (2, 2, 129, 64, 128, False, torch.bfloat16, 7, 5),
    (1, 1, 1, 1, 64, False, torch.float32, 3, 2),
    (1, 10, 4000, 4000, 128, True, torch.bfloat16, 12, 1),   # causal, 160 tiles in one 8-wave launch
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}q{c[2]}k{c[3]}D{c[4]}{'c' if c[5] else 'n'}N{c[7]}h{c[8]}"
                                             for c in CASES])
def test_bsnd_out(case):
    B, H, Sq, Skv, D, causal, out_dtype, heads, h0 = case
    seed = 4000 + Sq + Skv + heads
    q = inputs.random_bits(seed, (B, H, Sq, D))
    k = inputs.random_bits(seed + 1, (B, H, Skv, D))
    v = inputs.random_bits(seed + 2, (B, H, Skv, D))
    scale = 1 / math.sqrt(D)
    say(f"[bsnd_out] {case}")
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    ws = torch.empty((attn_fwd_workspace_bytes(B, H, Skv, D),), dtype=torch.uint8, device=DEV)
    # Sentinel contents in every head; only heads [h0, h0+H) may change.
    out = torch.full((B, Sq, heads, D), 7.25, dtype=out_dtype, device=DEV)
    before = out.clone()
    o_s, l_s = attn_fwd_ws_bsnd(dq, dk, dv, ws, out, out_h0=h0, scale=scale, causal=causal)
    o_n, l_n = attn_fwd_ws(dq, dk, dv, ws, scale=scale, causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert o_s.data_ptr() == out.data_ptr()
    assert torch.equal(out[:, :, h0:h0 + H], o_n.permute(0, 2, 1, 3)), "BSND store differs from the BNSD rows"
    assert torch.equal(l_s, l_n), "LSE differs"
    others = [h for h in range(heads) if not h0 <= h < h0 + H]
    if others:
        assert torch.equal(out[:, :, others], before[:, :, others]), "a head outside the slice was written"
    ref_o, ref_l = oracle.attn(q, k, v, scale, causal)
    ref_bsnd = oracle.bnsd_to_bsnd(ref_o, np.zeros((B, Sq, heads, D)), h0)
    got = host_f64(out)[:, :, h0:h0 + H]
    rep = compare.attn_report(got, ref_bsnd[:, :, h0:h0 + H], host_f64(l_s), ref_l,
                              bf16=out_dtype == torch.bfloat16)
    compare.assert_ok(rep, f"bsnd out {case}")


def test_bsnd_out_matches_layout_kernel():
    """bf16 output: the fused store gives the bits of attn_fwd_ws followed by
    the separate bnsd_to_bsnd layout kernel."""
    from attention_qk_norm_rope_amd import bnsd_to_bsnd
    B, H, Sq, Skv, D, heads, h0 = 1, 4, 700, 500, 128, 10, 3
    q = inputs.random_bits(77, (B, H, Sq, D))
    k = inputs.random_bits(78, (B, H, Skv, D))
    v = inputs.random_bits(79, (B, H, Skv, D))
    say("[bsnd_out] against bnsd_to_bsnd")
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    ws = torch.empty((attn_fwd_workspace_bytes(B, H, Skv, D),), dtype=torch.uint8, device=DEV)
    x1 = torch.zeros((B, Sq, heads, D), dtype=torch.bfloat16, device=DEV)
    x2 = torch.zeros_like(x1)
    attn_fwd_ws_bsnd(dq, dk, dv, ws, x1, out_h0=h0)
    o, _ = attn_fwd_ws(dq, dk, dv, ws)
    bnsd_to_bsnd(o, x2, h0)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(x1), host_bits(x2))

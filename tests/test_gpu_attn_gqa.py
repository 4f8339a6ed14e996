"""Grouped-query attention (attn_fwd_gqa): Hkv K/V heads serve H query heads,
query head h reading K/V head h // (H // Hkv) -- the num_key_value_heads
argument of the Wan2.2 page's npu_fused_infer_attention_score call.  The
reference is the oracle's grouped attention (oracle.attn_varlen at full
lengths), whose K/V head map is pinned on the CPU against torch's SDPA with
enable_gqa and a worked example.  With and without a workspace the bits are
the same, and Hkv = H gives attn_fwd's bits."""
import math

import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import attn_fwd, attn_fwd_gqa, attn_fwd_workspace_bytes, inputs
from gpu_common import DEV, dev_bits, host_f64, say

pytestmark = pytest.mark.gpu

# B, H, Hkv, Sq, Skv, D, causal, out dtype
CASES = [
    (2, 8, 2, 300, 333, 128, False, torch.bfloat16),
    (1, 6, 3, 257, 191, 64, True, torch.float32),
    (1, 4, 1, 129, 700, 128, False, torch.float32),     # one K/V head for all (multi-query)
    (2, 3, 3, 200, 100, 128, True, torch.bfloat16),     # Hkv = H: plain multi-head
    (1, 10, 2, 4000, 4000, 128, True, torch.bfloat16),  # causal, 160 tiles in one 8-wave launch
]


def _ids(c):
    B, H, Hkv, Sq, Skv, D, causal, dt = c
    return f"B{B}H{H}kv{Hkv}q{Sq}k{Skv}D{D}{'c' if causal else 'n'}{'f32' if dt == torch.float32 else 'bf16'}"


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_gqa_matches_oracle(case):
    B, H, Hkv, Sq, Skv, D, causal, out_dtype = case
    scale = 1 / math.sqrt(D)
    seed = 31 * H + 7 * Hkv + Sq
    q = inputs.random_bits(seed, (B, H, Sq, D))
    k = inputs.random_bits(seed + 1, (B, Hkv, Skv, D))
    v = inputs.random_bits(seed + 2, (B, Hkv, Skv, D))
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    say(f"[gqa] {_ids(case)}")
    o0, l0 = attn_fwd_gqa(dq, dk, dv, scale=scale, causal=causal, out_dtype=out_dtype)
    ws = torch.full((attn_fwd_workspace_bytes(B, Hkv, Skv, D),), 0x7E, dtype=torch.uint8, device=DEV)
    o1, l1 = attn_fwd_gqa(dq, dk, dv, workspace=ws, scale=scale, causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    if Hkv == H:
        om, lm = attn_fwd(dq, dk, dv, scale=scale, causal=causal, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(o0, om) and torch.equal(l0, lm)
    ref_o, ref_l = oracle.attn_varlen(q, k, v, [Sq] * B, [Skv] * B, scale, causal)
    rep = compare.attn_report(host_f64(o0), ref_o, host_f64(l0), ref_l, bf16=out_dtype == torch.bfloat16)
    compare.assert_ok(rep, "gqa " + _ids(case))


def test_gqa_equals_mha_on_repeated_kv():
    """The grouped call on Hkv heads gives the same bits as attn_fwd on the
    K/V heads materialised per query head."""
    B, H, Hkv, Sq, Skv, D = 1, 8, 2, 384, 512, 128
    q = dev_bits(inputs.random_bits(5, (B, H, Sq, D)))
    k = dev_bits(inputs.random_bits(6, (B, Hkv, Skv, D)))
    v = dev_bits(inputs.random_bits(7, (B, Hkv, Skv, D)))
    og, lg = attn_fwd_gqa(q, k, v, out_dtype=torch.float32)
    kr = k.repeat_interleave(H // Hkv, dim=1).contiguous()
    vr = v.repeat_interleave(H // Hkv, dim=1).contiguous()
    om, lm = attn_fwd(q, kr, vr, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(og, om) and torch.equal(lg, lm)

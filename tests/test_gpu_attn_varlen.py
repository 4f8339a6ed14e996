"""Variable-length attention (attn_fwd_varlen) on the GPU against the
oracle's definition: padded batches with per-batch valid query rows and keys
(the actual_seq_lengths / actual_seq_lengths_kv of the Wan2.2 page's fused
attention call), padding filled with NaN patterns, with and without a
workspace (same bits), grouped K/V heads, causal, and lengths of 0."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import attn_fwd, attn_fwd_varlen, attn_fwd_workspace_bytes, inputs
from gpu_common import DEV, dev_bits, host_f64, say

pytestmark = pytest.mark.gpu

# B, H, Hkv, Sq, Skv, D, causal, out dtype, seqlens_q, seqlens_kv
CASES = [
    (3, 2, 2, 300, 333, 128, False, torch.bfloat16, [300, 17, 129], [333, 64, 200]),
    (2, 4, 2, 257, 400, 64, True, torch.float32, [257, 100], [1, 400]),
    (3, 2, 1, 128, 128, 128, False, torch.float32, [0, 128, 50], [128, 0, 65]),
    (2, 5, 5, 4000, 4000, 128, True, torch.float32, [4000, 2500], [4000, 3100]),   # causal, one 8-wave launch
]


def _poison(bits, lens, axis_len):
    b = bits.copy()
    for i, n in enumerate(lens):
        b[i, :, n:axis_len] = 0x7FC0      # NaN bit patterns in the padding
    return b


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_varlen_matches_oracle(case):
    B, H, Hkv, Sq, Skv, D, causal, out_dtype, lq, lk = case
    scale = 1 / math.sqrt(D)
    seed = 500 + Sq + Skv
    q = _poison(inputs.random_bits(seed, (B, H, Sq, D)), lq, Sq)
    k = _poison(inputs.random_bits(seed + 1, (B, Hkv, Skv, D)), lk, Skv)
    v = _poison(inputs.random_bits(seed + 2, (B, Hkv, Skv, D)), lk, Skv)
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    slq = torch.tensor(lq, dtype=torch.int32, device=DEV)
    slk = torch.tensor(lk, dtype=torch.int32, device=DEV)
    say(f"[varlen] {case}")
    o0, l0 = attn_fwd_varlen(dq, dk, dv, slq, slk, scale=scale, causal=causal, out_dtype=out_dtype)
    ws = torch.full((attn_fwd_workspace_bytes(B, Hkv, Skv, D),), 0x7E, dtype=torch.uint8, device=DEV)
    o1, l1 = attn_fwd_varlen(dq, dk, dv, slq, slk, workspace=ws, scale=scale, causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert bool(torch.isfinite(o0).all())
    ref_o, ref_l = oracle.attn_varlen(q, k, v, lq, lk, scale, causal)
    got_o, got_l = host_f64(o0), host_f64(l0)
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), empty)
    assert np.all(got_o[empty] == 0)
    rep = compare.attn_report(got_o[~empty], ref_o[~empty], got_l[~empty], ref_l[~empty],
                              bf16=out_dtype == torch.bfloat16)
    compare.assert_ok(rep, f"varlen {case}")


def test_varlen_full_lengths_equal_attn_fwd():
    B, H, S, D = 2, 3, 200, 128
    q = dev_bits(inputs.random_bits(61, (B, H, S, D)))
    k = dev_bits(inputs.random_bits(62, (B, H, S, D)))
    v = dev_bits(inputs.random_bits(63, (B, H, S, D)))
    full = torch.full((B,), S, dtype=torch.int32, device=DEV)
    ov, lv = attn_fwd_varlen(q, k, v, full, full, out_dtype=torch.float32)
    oa, la = attn_fwd(q, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(ov, oa) and torch.equal(lv, la)

"""Seeded random causal shapes over many query tiles: batch, heads, query and
key lengths (1000..6000, ragged last tiles, Sq above and below Skv), D,
output dtype, scale and input spread are drawn per case.  Each case runs
attn_fwd (one 8-wave launch, V through registers), attn_fwd_ws (8-wave, or
4-wave for a small grid whose last round is at most half full) and
attn_fwd_ws_bsnd, which must agree bit for bit, and compares sampled rows
(including both edges of every 256-row tile of the first and last head)
with the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import (attn_fwd, attn_fwd_launch_form, attn_fwd_workspace_bytes, attn_fwd_ws,
                                        attn_fwd_ws_bsnd, inputs)
from gpu_common import DEV, dev_bits, rows_of, say

pytestmark = pytest.mark.gpu

N_CASES = 10


def _cases():
    rng = np.random.default_rng(20261203)
    cases = []
    for i in range(N_CASES):
        D = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 13))
        Sq = int(rng.integers(1000, 6001))
        Skv = int(rng.integers(1000, 6001))
        f32 = bool(rng.random() < 0.5)
        scale = float(rng.uniform(0.5, 2.0)) / math.sqrt(D)
        std = float(rng.uniform(0.5, 2.0))
        cases.append((i, B, H, Sq, Skv, D, f32, scale, std))
    return cases


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}H{c[2]}q{c[3]}k{c[4]}D{c[5]}" for c in CASES])
def test_random_causal(case):
    i, B, H, Sq, Skv, D, f32, scale, std = case
    out_dtype = torch.float32 if f32 else torch.bfloat16
    seed = 9500 + 10 * i
    q = inputs.random_bits(seed, (B, H, Sq, D), std=std)
    k = inputs.random_bits(seed + 1, (B, H, Skv, D), std=std)
    v = inputs.random_bits(seed + 2, (B, H, Skv, D))
    ws_bytes = attn_fwd_workspace_bytes(B, H, Skv, D)
    form = attn_fwd_launch_form(B, H, Sq, Skv, D, True, ws_bytes)
    say(f"[random causal] {case} ws form {form}")
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    ws = torch.full((ws_bytes,), 0x5A, dtype=torch.uint8, device=DEV)
    o0, l0 = attn_fwd(dq, dk, dv, scale=scale, causal=True, out_dtype=out_dtype)
    o1, l1 = attn_fwd_ws(dq, dk, dv, ws, scale=scale, causal=True, out_dtype=out_dtype)
    heads = H + 2
    ob = torch.full((B, Sq, heads, D), 3.5, dtype=out_dtype, device=DEV)
    _, l2 = attn_fwd_ws_bsnd(dq, dk, dv, ws, ob, out_h0=1, scale=scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1), "attn_fwd and attn_fwd_ws differ"
    assert torch.equal(ob[:, :, 1:1 + H], o0.permute(0, 2, 1, 3)) and torch.equal(l2, l0), "BSND store differs"
    assert torch.equal(ob[:, :, 0], torch.full_like(ob[:, :, 0], 3.5)), "a head outside the slice was written"
    edges = [bh * Sq + r for bh in (0, B * H - 1) for t in range(0, Sq, 256) for r in (t, min(t + 255, Sq - 1))]
    rows = inputs.sample_rows(30 + i, B, H, Sq, per_head=24, extra=edges)
    ref_o, ref_l = oracle.attn(q, k, v, scale, True, rows=rows)
    rep = compare.attn_report(rows_of(o0, rows), ref_o, rows_of(l0, rows), ref_l, bf16=not f32)
    say(f"[random causal] {i}: {rep}")
    compare.assert_ok(rep, f"random causal {case}")

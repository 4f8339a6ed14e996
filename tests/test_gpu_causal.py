"""Causal attention over many query tiles, against the fp64 oracle.

Causal calls take the query tiles of each head longest first (in reverse),
and each workgroup stops at the key tile that holds its last row's diagonal;
the tiles crossing the diagonal are masked per wave.  The cases span several
256-row tiles per head with a ragged last tile, Sq below and above Skv
(top-left alignment: row i sees keys 0..i, so rows at or past Skv see every
key), both entry points (attn_fwd, and attn_fwd_ws, whose small causal grids
run in 4-wave workgroups, with the same bits), and the B1 H40 S18900
self-attention at full size on sampled rows over more than eleven rounds of
tiles."""
import math

import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import attn_fwd, attn_fwd_launch_form, attn_fwd_workspace_bytes, attn_fwd_ws, inputs
from gpu_common import DEV, dev_bits, host_f64, rows_of, say

pytestmark = pytest.mark.gpu

# B, H, Sq, Skv, D, out dtype
CASES = [
    (1, 3, 2900, 2900, 128, torch.float32),   # 12 tiles per head, 84-row last tile
    (2, 2, 1000, 3000, 64, torch.bfloat16),   # Sq < Skv: keys past Sq are never seen
    (1, 2, 3000, 1000, 128, torch.float32),   # Sq > Skv: rows >= 1000 see every key
]


def _ids(c):
    B, H, Sq, Skv, D, dt = c
    return f"B{B}H{H}q{Sq}k{Skv}D{D}{'f32' if dt == torch.float32 else 'bf16'}"


def _ws(B, H, Skv, D):
    return torch.full((attn_fwd_workspace_bytes(B, H, Skv, D),), 0x7E, dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_causal_tiles_match_oracle(case):
    B, H, Sq, Skv, D, out_dtype = case
    scale = 1 / math.sqrt(D)
    seed = 9100 + Sq + Skv + D
    q = inputs.random_bits(seed, (B, H, Sq, D))
    k = inputs.random_bits(seed + 1, (B, H, Skv, D))
    v = inputs.random_bits(seed + 2, (B, H, Skv, D))
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    say(f"[causal] {_ids(case)}")
    o0, l0 = attn_fwd(dq, dk, dv, scale=scale, causal=True, out_dtype=out_dtype)
    o1, l1 = attn_fwd_ws(dq, dk, dv, _ws(B, H, Skv, D), scale=scale, causal=True, out_dtype=out_dtype)
    torch.cuda.synchronize()
    # Same per-row arithmetic in both kernel forms.
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    ref_o, ref_l = oracle.attn(q, k, v, scale, True)
    rep = compare.attn_report(host_f64(o0), ref_o, host_f64(l0), ref_l, bf16=out_dtype == torch.bfloat16)
    say(f"[causal] {_ids(case)}: {rep}")
    compare.assert_ok(rep, f"causal {_ids(case)}")


def test_causal_full_size_sampled_rows():
    """B1 H40 S18900 D128 (2,960 tiles, one launch on both entry points):
    sampled rows per head, plus the first and last rows of every 256-row
    tile of two heads, against the oracle; both entry points give the same
    bits."""
    B, H, S, D = 1, 40, 18900, 128
    scale = 1 / math.sqrt(D)
    assert attn_fwd_launch_form(B, H, S, S, D, True, attn_fwd_workspace_bytes(B, H, S, D)) == "one"
    q = inputs.random_bits(9201, (B, H, S, D))
    k = inputs.random_bits(9202, (B, H, S, D))
    v = inputs.random_bits(9203, (B, H, S, D))
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    say("[causal] full size B1 H40 S18900: attn_fwd")
    o0, l0 = attn_fwd(dq, dk, dv, scale=scale, causal=True, out_dtype=torch.float32)
    say("[causal] full size B1 H40 S18900: attn_fwd_ws")
    o1, l1 = attn_fwd_ws(dq, dk, dv, _ws(B, H, S, D), scale=scale, causal=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    edges = [bh * S + i for bh in (0, H - 1) for t in range(0, S, 256) for i in (t, min(t + 255, S - 1))]
    rows = inputs.sample_rows(17, B, H, S, extra=edges)
    say(f"[causal] oracle on {rows.size} rows")
    ref_o, ref_l = oracle.attn(q, k, v, scale, True, rows=rows)
    rep = compare.attn_report(rows_of(o0, rows), ref_o, rows_of(l0, rows), ref_l, bf16=False)
    say(f"[causal] full size: {rep}")
    compare.assert_ok(rep, "causal B1 H40 S18900")

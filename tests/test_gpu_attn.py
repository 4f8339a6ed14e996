"""attn_fwd on the GPU against the fp64 oracle, element by element (all rows).

Shapes span several 128-row query tiles and 64-key tiles with ragged tails on
both, D = 64 and 128, causal and not, Sq != Skv, negative and zero scale, bf16
and fp32 outputs, and the degenerate Sq = 1 / Skv = 1 cases.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import attn_fwd, attn_merge, inputs
from gpu_common import dev_bits, host_bits, host_f64, say

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, Sq, Skv, D, causal, scale, out_dtype
    (1, 2, 256, 256, 64, False, 1 / 8, torch.bfloat16),        # tiny config, non-causal
    (1, 2, 256, 256, 64, True, 1 / 8, torch.bfloat16),         # tiny config, causal
    (1, 1, 1, 1, 128, False, None, torch.bfloat16),
    (1, 1, 1, 300, 128, False, None, torch.bfloat16),
    (2, 3, 129, 65, 128, False, None, torch.bfloat16),
    (1, 2, 300, 513, 64, True, None, torch.bfloat16),
    (1, 2, 700, 130, 128, True, None, torch.bfloat16),         # Sq > Skv, causal
    (1, 2, 130, 700, 128, True, None, torch.bfloat16),         # Sq < Skv, causal
    (1, 1, 33, 1000, 128, False, -0.09, torch.bfloat16),       # negative scale
    (1, 2, 200, 333, 128, False, 0.0, torch.bfloat16),         # zero scale
    (2, 2, 257, 191, 64, False, None, torch.float32),
    (1, 3, 385, 449, 128, True, None, torch.float32),
]


def _ids(c):
    B, H, Sq, Skv, D, causal, scale, dt = c
    return f"B{B}H{H}q{Sq}k{Skv}D{D}{'c' if causal else 'n'}s{scale}{'f32' if dt == torch.float32 else 'bf16'}"


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_attn_matches_oracle(case):
    B, H, Sq, Skv, D, causal, scale, out_dtype = case
    if scale is None:
        scale = 1 / math.sqrt(D)
    seed = Sq * 7 + Skv
    q = inputs.random_bits(seed, (B, H, Sq, D))
    k = inputs.random_bits(seed + 1, (B, H, Skv, D))
    v = inputs.random_bits(seed + 2, (B, H, Skv, D))
    say(f"[attn] {_ids(case)}")
    out, lse = attn_fwd(dev_bits(q), dev_bits(k), dev_bits(v), scale=scale, causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attn(q, k, v, scale, causal)
    rep = compare.attn_report(host_f64(out), ref_o, host_f64(lse), ref_l, bf16=out_dtype == torch.bfloat16)
    compare.assert_ok(rep, _ids(case))


def test_softmax_stability_large_logits():
    """Logit std ~ 8 (Q scaled by 8): the running max moves many times."""
    B, H, Sq, Skv, D = 1, 2, 300, 1200, 128
    q = inputs.random_bits(11, (B, H, Sq, D), std=8.0)
    k = inputs.random_bits(12, (B, H, Skv, D))
    v = inputs.random_bits(13, (B, H, Skv, D))
    out, lse = attn_fwd(dev_bits(q), dev_bits(k), dev_bits(v), out_dtype=torch.float32)
    ref_o, ref_l = oracle.attn(q, k, v, 1 / math.sqrt(D))
    compare.assert_ok(compare.attn_report(host_f64(out), ref_o, host_f64(lse), ref_l, bf16=False), "std-8 logits")


def test_uniform_v_and_single_key_are_exact():
    B, H, Sq, Skv, D = 1, 2, 200, 333, 128
    q = inputs.random_bits(21, (B, H, Sq, D), std=2.0)
    k = inputs.random_bits(22, (B, H, Skv, D), std=2.0)
    row = inputs.random_bits(23, (D,))
    v = np.broadcast_to(row, (B, H, Skv, D)).copy()
    out, _ = attn_fwd(dev_bits(q), dev_bits(k), dev_bits(v), out_dtype=torch.float32)
    err = np.abs(host_f64(out) - inputs.bf16_bits_to_f64(row)).max()
    assert err <= 2e-6 * np.abs(inputs.bf16_bits_to_f64(row)).max(), err
    # One key: the output is that key's value, bit for bit, and lse = scale*q.k.
    k1 = inputs.random_bits(24, (B, H, 1, D))
    v1 = inputs.random_bits(25, (B, H, 1, D))
    out, lse = attn_fwd(dev_bits(q), dev_bits(k1), dev_bits(v1))
    np.testing.assert_array_equal(host_bits(out), np.broadcast_to(v1, (B, H, Sq, D)))
    s = (inputs.bf16_bits_to_f64(q) * inputs.bf16_bits_to_f64(k1)).sum(-1) / math.sqrt(D)
    np.testing.assert_allclose(host_f64(lse), s, atol=1e-4)


def test_causal_row_zero_is_first_value():
    B, H, S, D = 1, 3, 257, 64
    q = inputs.random_bits(31, (B, H, S, D))
    k = inputs.random_bits(32, (B, H, S, D))
    v = inputs.random_bits(33, (B, H, S, D))
    out, lse = attn_fwd(dev_bits(q), dev_bits(k), dev_bits(v), causal=True)
    np.testing.assert_array_equal(host_bits(out)[:, :, 0], v[:, :, 0])


def test_permuting_keys_with_values():
    B, H, Sq, Skv, D = 1, 2, 150, 260, 128
    q = inputs.random_bits(41, (B, H, Sq, D))
    k = inputs.random_bits(42, (B, H, Skv, D))
    v = inputs.random_bits(43, (B, H, Skv, D))
    perm = np.random.default_rng(44).permutation(Skv)
    o1, l1 = attn_fwd(dev_bits(q), dev_bits(k), dev_bits(v), out_dtype=torch.float32)
    o2, l2 = attn_fwd(dev_bits(q), dev_bits(k[:, :, perm].copy()), dev_bits(v[:, :, perm].copy()),
                      out_dtype=torch.float32)
    # Tiles see different key subsets, so P rounds differently: equal within
    # the parity tolerances, not bit for bit.
    assert np.abs(host_f64(o1) - host_f64(o2)).max() <= compare.ATOL
    assert np.abs(host_f64(l1) - host_f64(l2)).max() <= compare.LSE_ATOL


def test_bitwise_deterministic():
    B, H, Sq, Skv, D = 2, 4, 1000, 1500, 128
    q = dev_bits(inputs.random_bits(51, (B, H, Sq, D)))
    k = dev_bits(inputs.random_bits(52, (B, H, Skv, D)))
    v = dev_bits(inputs.random_bits(53, (B, H, Skv, D)))
    o1, l1 = attn_fwd(q, k, v)
    o2, l2 = attn_fwd(q, k, v)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_kv_window_equals_contiguous_chunk():
    """attn_fwd_kv_strided on a key window of a longer tensor equals attn_fwd
    on the same keys copied out, bit for bit."""
    B, H, S, Sq, D = 1, 3, 700, 300, 128
    q = dev_bits(inputs.random_bits(61, (B, H, Sq, D)))
    k = dev_bits(inputs.random_bits(62, (B, H, S, D)))
    v = dev_bits(inputs.random_bits(63, (B, H, S, D)))
    for a, b in ((0, 175), (175, 700), (64, 129)):
        ow, lw = attn_fwd(q, k[:, :, a:b], v[:, :, a:b], out_dtype=torch.float32)
        oc, lc = attn_fwd(q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(), out_dtype=torch.float32)
        assert torch.equal(ow, oc) and torch.equal(lw, lc), (a, b)


def test_split_merge_equals_full_and_differs_from_local_only():
    """The ring bug on the pages returned the local chunk's result unchanged;
    a 2-chunk attn_fwd + attn_merge must instead equal full attention."""
    cfg = inputs.WORKLOADS["tiny"]
    x = inputs.make_inputs(cfg)
    q, k, v = x["q"], x["k"], x["v"]
    kc, vc = inputs.split_kv(k, 2), inputs.split_kv(v, 2)
    dq = dev_bits(q)
    oa, la = attn_fwd(dq, dev_bits(kc[0]), dev_bits(vc[0]), scale=cfg.scale, out_dtype=torch.float32)
    local = host_f64(oa)
    ob, lb = attn_fwd(dq, dev_bits(kc[1]), dev_bits(vc[1]), scale=cfg.scale, out_dtype=torch.float32)
    attn_merge(oa, la, ob, lb)
    ref_o, ref_l = oracle.attn(q, k, v, cfg.scale)
    compare.assert_ok(compare.attn_report(host_f64(oa), ref_o, host_f64(la), ref_l, bf16=False), "2-chunk merge")
    assert np.abs(host_f64(oa) - local).max() > 0.05

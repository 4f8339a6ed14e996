"""Pins of the oracle's grouped-query attention (CPU only).

The fused attention call of the Wan2.2 NPU page takes a key/value head count
(num_key_value_heads) below the query head count.  The oracle maps query head
h to K/V head h // (H/Hkv).  That map is checked here against two things
that do not share the oracle's code:

* a worked example derived by hand (tests/golden/gqa_one_key.json) in which
  an interleaved map (h mod Hkv) gives different outputs and LSEs;
* torch's CPU scaled_dot_product_attention in float64 with enable_gqa=True,
  a library routine that takes K/V with Hkv heads and does its own grouping.
  The LSE comes from the same routine through a sentinel key (a zero key
  whose value is 1 while the others are 0: its weight is 1/(1 + exp(LSE))).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from attention_qk_norm_rope_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(bits):
    return torch.from_numpy(inputs.bf16_bits_to_f64(bits))


def _sdpa_gqa(q, k, v, scale, causal):
    return torch.nn.functional.scaled_dot_product_attention(
        _f64(q), _f64(k), _f64(v), scale=scale, is_causal=causal, enable_gqa=True).numpy()


def _lse_gqa_by_sentinel(q, k, scale, causal):
    B, H, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    kk = torch.cat([torch.zeros(B, Hkv, 1, D, dtype=torch.float64), _f64(k)], dim=2)
    vv = torch.zeros(B, Hkv, Skv + 1, 1, dtype=torch.float64)
    vv[:, :, 0, 0] = 1.0
    mask = torch.ones(Sq, Skv + 1, dtype=torch.bool)
    if causal:
        mask[:, 1:] = torch.ones(Sq, Skv, dtype=torch.bool).tril()
    w = torch.nn.functional.scaled_dot_product_attention(_f64(q), kk, vv, attn_mask=mask, scale=scale,
                                                         enable_gqa=True)[..., 0]
    return torch.log(1.0 / w - 1.0).numpy()


def test_golden_one_key_per_kv_head(oracle):
    g = json.load(open(os.path.join(GOLDEN, "gqa_one_key.json")))
    bits = lambda a: inputs.to_bf16_bits(np.asarray(a, dtype=np.float32))[None]  # noqa: E731
    q, k, v = bits(g["q"]), bits(g["k"]), bits(g["v"])
    assert q.shape[1] == g["H"] and k.shape[1] == g["Hkv"]
    out, lse = oracle.attn_varlen(q, k, v, [1], [1], g["scale"], False)
    np.testing.assert_array_equal(out[0], np.asarray(g["out"]))
    np.testing.assert_allclose(lse[0], np.asarray(g["lse"]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("B,H,Hkv,Sq,Skv,D,scale,causal", [
    (1, 4, 2, 9, 13, 16, 0.25, False),
    (2, 6, 3, 7, 11, 8, 0.4, False),
    (1, 8, 1, 5, 17, 32, 1 / math.sqrt(32), False),   # every query head reads the one K/V head
    (2, 4, 4, 6, 6, 8, 0.3, True),                    # Hkv = H is plain multi-head attention
    (1, 8, 2, 10, 10, 16, 0.25, True),
    (1, 12, 4, 4, 21, 8, -0.5, False),                # negative scale
])
def test_grouping_matches_torch_sdpa_enable_gqa(oracle, B, H, Hkv, Sq, Skv, D, scale, causal):
    q = inputs.random_bits(31, (B, H, Sq, D))
    k = inputs.random_bits(32, (B, Hkv, Skv, D), std=2.0)
    v = inputs.random_bits(33, (B, Hkv, Skv, D))
    out, lse = oracle.attn_varlen(q, k, v, [Sq] * B, [Skv] * B, scale, causal)
    np.testing.assert_allclose(out, _sdpa_gqa(q, k, v, scale, causal), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, _lse_gqa_by_sentinel(q, k, scale, causal), rtol=0, atol=1e-10)


def test_interleaved_map_would_fail(oracle):
    """Guard on the pin itself: with distinct K/V heads, the library's
    grouping differs from the interleaved map h mod Hkv, so a mistake of that
    kind cannot pass the comparison above."""
    q = inputs.random_bits(41, (1, 4, 3, 8))
    k = inputs.random_bits(42, (1, 2, 5, 8), std=2.0)
    v = inputs.random_bits(43, (1, 2, 5, 8))
    ref = _sdpa_gqa(q, k, v, 0.5, False)
    wrong = torch.nn.functional.scaled_dot_product_attention(
        _f64(q), _f64(k)[:, [0, 1, 0, 1]], _f64(v)[:, [0, 1, 0, 1]], scale=0.5).numpy()
    assert np.abs(ref - wrong).max() > 0.1
    out, _ = oracle.attn_varlen(q, k, v, [3], [5], 0.5, False)
    assert np.abs(out - wrong).max() > 0.1

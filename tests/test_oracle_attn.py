"""Pins for the fp64 attention oracle (CPU only).

Each test checks the oracle against something other than itself: a worked
example derived by hand, closed forms, invariants of softmax attention, and
torch's CPU scaled_dot_product_attention in float64 (a library routine the
oracle does not use).  A dropped scale, a transposed operand, a wrong causal
offset, a log2/ln mix-up in the LSE or a wrong row index fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from attention_qk_norm_rope_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(a):
    return inputs.to_bf16_bits(np.asarray(a, dtype=np.float32))


def _f64(bits):
    return torch.from_numpy(inputs.bf16_bits_to_f64(bits))


def _sdpa(q, k, v, scale, causal):
    return torch.nn.functional.scaled_dot_product_attention(
        _f64(q), _f64(k), _f64(v), scale=scale, is_causal=causal).numpy()


def _lse_by_sentinel(q, k, scale, causal):
    """LSE from SDPA alone: append a zero key (logit exactly 0) whose value is
    1 while every other value is 0; its weight w = 1/(1 + exp(LSE))."""
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    kq = _f64(q)
    kk = torch.cat([torch.zeros(B, H, 1, D, dtype=torch.float64), _f64(k)], dim=2)
    vv = torch.zeros(B, H, Skv + 1, 1, dtype=torch.float64)
    vv[:, :, 0, 0] = 1.0
    mask = torch.ones(Sq, Skv + 1, dtype=torch.bool)
    if causal:
        mask[:, 1:] = torch.ones(Sq, Skv, dtype=torch.bool).tril()
    w = torch.nn.functional.scaled_dot_product_attention(kq, kk, vv, attn_mask=mask, scale=scale)[..., 0]
    return torch.log(1.0 / w - 1.0).numpy()


def test_golden_two_keys(oracle):
    g = json.load(open(os.path.join(GOLDEN, "attn_two_keys.json")))
    q = _bits(g["q"])[None, None]
    k = _bits(g["k"])[None, None]
    v = _bits(g["v"])[None, None]
    for mode, causal in (("noncausal", False), ("causal", True)):
        out, lse = oracle.attn(q, k, v, g["scale"], causal)
        np.testing.assert_allclose(out[0, 0], g[mode]["out"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, 0], g[mode]["lse"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("B,H,Sq,Skv,D,scale,causal", [
    (1, 2, 17, 33, 64, 0.125, False),
    (2, 3, 40, 23, 16, 0.3, False),
    (1, 1, 29, 29, 128, 1 / math.sqrt(128), True),
    (2, 2, 31, 45, 8, 0.7, True),      # Sq < Skv, causal: top-left alignment
    (1, 2, 45, 31, 8, 0.7, True),      # Sq > Skv: later rows see every key
    (1, 1, 12, 19, 32, -0.4, False),   # negative scale
])
def test_matches_torch_sdpa(oracle, B, H, Sq, Skv, D, scale, causal):
    q = inputs.random_bits(1, (B, H, Sq, D))
    k = inputs.random_bits(2, (B, H, Skv, D))
    v = inputs.random_bits(3, (B, H, Skv, D))
    out, lse = oracle.attn(q, k, v, scale, causal)
    np.testing.assert_allclose(out, _sdpa(q, k, v, scale, causal), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, _lse_by_sentinel(q, k, scale, causal), rtol=0, atol=1e-10)


def test_lse_is_log_of_softmax_denominator(oracle):
    """torch.logsumexp over the library-computed logit matrix."""
    q = inputs.random_bits(4, (1, 2, 9, 16), std=2.0)
    k = inputs.random_bits(5, (1, 2, 13, 16), std=2.0)
    v = inputs.random_bits(6, (1, 2, 13, 16))
    scale = 0.25
    _, lse = oracle.attn(q, k, v, scale, False)
    logits = torch.matmul(_f64(q), _f64(k).transpose(-1, -2)) * scale
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_uniform_v_gives_constant_output(oracle):
    q = inputs.random_bits(7, (1, 2, 20, 32), std=3.0)
    k = inputs.random_bits(8, (1, 2, 37, 32), std=3.0)
    row = _bits(np.linspace(-2, 2, 32))
    v = np.broadcast_to(row, (1, 2, 37, 32)).copy()
    for causal in (False, True):
        out, _ = oracle.attn(q, k, v, 0.2, causal)
        np.testing.assert_allclose(out, np.broadcast_to(inputs.bf16_bits_to_f64(row), out.shape),
                                   rtol=0, atol=1e-13)


def test_permuting_keys_with_values(oracle):
    q = inputs.random_bits(9, (2, 2, 11, 16))
    k = inputs.random_bits(10, (2, 2, 27, 16))
    v = inputs.random_bits(11, (2, 2, 27, 16))
    perm = np.random.default_rng(12).permutation(27)
    o1, l1 = oracle.attn(q, k, v, 0.3, False)
    o2, l2 = oracle.attn(q, k[:, :, perm].copy(), v[:, :, perm].copy(), 0.3, False)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)
    # Permuting keys alone (values fixed) must change the result.
    o3, _ = oracle.attn(q, k[:, :, perm].copy(), v, 0.3, False)
    assert np.abs(o3 - o1).max() > 1e-3


def test_causal_row_zero_returns_first_value(oracle):
    q = inputs.random_bits(13, (1, 3, 8, 64))
    k = inputs.random_bits(14, (1, 3, 8, 64))
    v = inputs.random_bits(15, (1, 3, 8, 64))
    scale = 0.125
    out, lse = oracle.attn(q, k, v, scale, True)
    np.testing.assert_array_equal(out[:, :, 0], inputs.bf16_bits_to_f64(v[:, :, 0]))
    qk0 = (inputs.bf16_bits_to_f64(q[:, :, 0]) * inputs.bf16_bits_to_f64(k[:, :, 0])).sum(-1)
    np.testing.assert_allclose(lse[:, :, 0], scale * qk0, rtol=0, atol=1e-13)


def test_scale_zero_is_mean_of_values(oracle):
    q = inputs.random_bits(16, (1, 2, 10, 16))
    k = inputs.random_bits(17, (1, 2, 14, 16))
    v = inputs.random_bits(18, (1, 2, 14, 16))
    vf = inputs.bf16_bits_to_f64(v)
    out, lse = oracle.attn(q, k, v, 0.0, False)
    np.testing.assert_allclose(out, np.broadcast_to(vf.mean(axis=2, keepdims=True), out.shape), atol=1e-13)
    np.testing.assert_allclose(lse, np.full(lse.shape, math.log(14)), atol=1e-13)
    out, lse = oracle.attn(q, k, v, 0.0, True)
    for i in range(10):
        n = min(i + 1, 14)
        np.testing.assert_allclose(out[:, :, i], vf[:, :, :n].mean(axis=2), atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i], math.log(n), atol=1e-13)


def test_single_key(oracle):
    q = inputs.random_bits(19, (1, 1, 5, 32))
    k = inputs.random_bits(20, (1, 1, 1, 32))
    v = inputs.random_bits(21, (1, 1, 1, 32))
    out, lse = oracle.attn(q, k, v, 0.5, False)
    np.testing.assert_array_equal(out[0, 0], np.broadcast_to(inputs.bf16_bits_to_f64(v[0, 0, 0]), (5, 32)))
    s = 0.5 * inputs.bf16_bits_to_f64(q[0, 0]) @ inputs.bf16_bits_to_f64(k[0, 0, 0])
    np.testing.assert_allclose(lse[0, 0], s, atol=1e-13)


def test_identical_keys(oracle):
    q = inputs.random_bits(22, (1, 1, 6, 16))
    k = np.broadcast_to(inputs.random_bits(23, (16,)), (1, 1, 9, 16)).copy()
    v = inputs.random_bits(24, (1, 1, 9, 16))
    out, lse = oracle.attn(q, k, v, 0.4, False)
    vf = inputs.bf16_bits_to_f64(v)[0, 0]
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(vf.mean(0), (6, 16)), atol=1e-13)
    s = 0.4 * inputs.bf16_bits_to_f64(q[0, 0]) @ inputs.bf16_bits_to_f64(k[0, 0, 0])
    np.testing.assert_allclose(lse[0, 0], s + math.log(9), atol=1e-12)


@pytest.mark.parametrize("cuts", [(13,), (5, 20, 21)])
def test_merge_of_any_kv_split_equals_full(oracle, cuts):
    q = inputs.random_bits(25, (2, 2, 15, 16), std=2.0)
    k = inputs.random_bits(26, (2, 2, 30, 16), std=2.0)
    v = inputs.random_bits(27, (2, 2, 30, 16))
    full_o, full_l = oracle.attn(q, k, v, 0.35, False)
    bounds = (0,) + cuts + (30,)
    acc_o = acc_l = None
    for a, b in zip(bounds[:-1], bounds[1:]):
        o, l = oracle.attn(q, k[:, :, a:b].copy(), v[:, :, a:b].copy(), 0.35, False)
        if acc_o is None:
            acc_o, acc_l = o, l
        else:
            acc_o, acc_l = oracle.merge(acc_o, acc_l, o, l)
    np.testing.assert_allclose(acc_o, full_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(acc_l, full_l, rtol=0, atol=1e-13)


def test_row_subset_matches_full_rows(oracle):
    q = inputs.random_bits(28, (2, 3, 21, 16))
    k = inputs.random_bits(29, (2, 3, 18, 16))
    v = inputs.random_bits(30, (2, 3, 18, 16))
    full_o, full_l = oracle.attn(q, k, v, 0.25, True)
    rows = inputs.sample_rows(1, 2, 3, 21, per_head=7)
    o, l = oracle.attn(q, k, v, 0.25, True, rows=rows)
    np.testing.assert_array_equal(o, full_o.reshape(-1, 16)[rows])
    np.testing.assert_array_equal(l, full_l.reshape(-1)[rows])


def test_rejects_bad_arguments(oracle):
    q = inputs.random_bits(31, (1, 1, 4, 8))
    with pytest.raises(ValueError):
        oracle.attn(q, q[:, :, :, :4].copy(), q[:, :, :, :4].copy(), 1.0)
    with pytest.raises(ValueError):
        oracle.attn(q, q, q, 1.0, rows=[4])
    with pytest.raises(TypeError):
        oracle.attn(q.astype(np.float32), q, q, 1.0)

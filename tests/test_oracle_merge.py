"""Pins for the fp64 out/LSE merge oracle (CPU only).

Checks: a pair worked by hand; identity when one side saw no key, also
when that side's values are NaN (an empty key set adds no term); the
empty/empty case; commutativity and associativity; equal LSE gives the
average; merged chunk attentions from torch's SDPA (library, float64) equal
torch's full attention; and the negative case of the ring bug on the pages
(a ring that returns only its local chunk): the merge must differ from the
local-only output.
"""
import json
import math
import os

import numpy as np
import torch

from attention_qk_norm_rope_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, rows, D):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, D)), rng.standard_normal(rows) * 3.0


def test_golden_pair(oracle):
    g = json.load(open(os.path.join(GOLDEN, "merge_pair.json")))
    o, l = oracle.merge(np.array([g["out_a"]]), np.array([g["lse_a"]]),
                        np.array([g["out_b"]]), np.array([g["lse_b"]]))
    np.testing.assert_allclose(o[0], g["out"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(l[0], g["lse"], rtol=0, atol=1e-15)


def test_empty_side_is_identity(oracle):
    oa, la = _rand(1, 9, 16)
    ob, _ = _rand(2, 9, 16)
    ninf = np.full(9, -np.inf)
    o, l = oracle.merge(oa, la, ob, ninf)
    np.testing.assert_array_equal(o, oa)
    np.testing.assert_array_equal(l, la)
    o, l = oracle.merge(ob, ninf, oa, la)
    np.testing.assert_array_equal(o, oa)
    np.testing.assert_array_equal(l, la)
    o, l = oracle.merge(oa, ninf, ob, ninf)
    np.testing.assert_array_equal(o, 0.0)
    assert np.all(l == -np.inf)


def test_empty_side_adds_no_term_even_with_nan_values(oracle):
    """The merge is the attention over the union of two key sets.  A side
    with LSE -inf is the attention over an empty key set: it holds no key, so
    whatever its output buffer contains (NaN here) it adds no term."""
    oa, la = _rand(11, 6, 8)
    nan = np.full((6, 8), np.nan)
    ninf = np.full(6, -np.inf)
    o, l = oracle.merge(nan, ninf, oa, la)
    np.testing.assert_array_equal(o, oa)
    np.testing.assert_array_equal(l, la)
    o, l = oracle.merge(oa, la, nan, ninf)
    np.testing.assert_array_equal(o, oa)
    np.testing.assert_array_equal(l, la)
    o, l = oracle.merge(nan, ninf, nan, ninf)
    np.testing.assert_array_equal(o, 0.0)
    assert np.all(l == -np.inf)


def test_commutative_and_associative(oracle):
    a, la = _rand(3, 11, 8)
    b, lb = _rand(4, 11, 8)
    c, lc = _rand(5, 11, 8)
    o1, l1 = oracle.merge(a, la, b, lb)
    o2, l2 = oracle.merge(b, lb, a, la)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-14)
    left = oracle.merge(*oracle.merge(a, la, b, lb), c, lc)
    right = oracle.merge(a, la, *oracle.merge(b, lb, c, lc))
    np.testing.assert_allclose(left[0], right[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(left[1], right[1], rtol=0, atol=1e-13)


def test_equal_lse_averages(oracle):
    a, la = _rand(6, 7, 8)
    b, _ = _rand(7, 7, 8)
    o, l = oracle.merge(a, la, b, la)
    np.testing.assert_allclose(o, (a + b) / 2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(l, la + math.log(2), rtol=0, atol=1e-14)


def _sdpa_with_lse(q, k, v, scale):
    logits = torch.matmul(q, k.transpose(-1, -2)) * scale
    return (torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale),
            torch.logsumexp(logits, dim=-1))


def test_merged_chunks_equal_full_attention_library(oracle):
    torch.manual_seed(0)
    q = torch.randn(2, 3, 10, 16, dtype=torch.float64)
    k = torch.randn(2, 3, 40, 16, dtype=torch.float64) * 2
    v = torch.randn(2, 3, 40, 16, dtype=torch.float64)
    scale = 0.3
    full_o, full_l = _sdpa_with_lse(q, k, v, scale)
    acc = None
    for a, b in ((0, 10), (10, 25), (25, 40)):
        o, l = _sdpa_with_lse(q, k[:, :, a:b], v[:, :, a:b], scale)
        acc = (o.numpy(), l.numpy()) if acc is None else oracle.merge(acc[0], acc[1], o.numpy(), l.numpy())
    np.testing.assert_allclose(acc[0], full_o.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(acc[1], full_l.numpy(), rtol=0, atol=1e-13)


def test_merge_differs_from_local_only_chunk(oracle):
    """The ring bug on the pages returned the local chunk's attention
    unchanged (max error 0 against local-only attention).  A correct merge of
    two chunks must not equal the local-only result."""
    q = inputs.random_bits(8, (1, 2, 16, 64))
    k = inputs.random_bits(9, (1, 2, 64, 64))
    v = inputs.random_bits(10, (1, 2, 64, 64))
    o0, l0 = oracle.attn(q, k[:, :, :32].copy(), v[:, :, :32].copy(), 0.125)
    o1, l1 = oracle.attn(q, k[:, :, 32:].copy(), v[:, :, 32:].copy(), 0.125)
    om, lm = oracle.merge(o0, l0, o1, l1)
    full_o, full_l = oracle.attn(q, k, v, 0.125)
    np.testing.assert_allclose(om, full_o, atol=1e-13)
    assert np.abs(om - o0).max() > 0.05
    assert np.all(lm > l0)

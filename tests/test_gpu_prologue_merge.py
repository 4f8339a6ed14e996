"""qk_norm_rope and attn_merge on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import attn_merge, inputs, qk_norm_rope, qk_norm_rope_out
from gpu_common import dev_bits, dev_f32, host_bits, host_f64, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,S,D,grid", [
    (1, 2, 256, 64, ("line", 256)),
    (2, 3, 61, 128, ("video", 1, 1, 61)),
    (1, 1, 1, 128, ("line", 1)),
    (1, 4, 600, 128, ("video", 2, 15, 20)),
    (3, 29, 37, 64, ("line", 37)),          # 87 (b,h) rows: three groups of 40 heads per thread, the last ragged
    (2, 41, 19, 128, ("line", 19)),         # 82 rows: a group boundary inside a batch
])
def test_prologue_matches_oracle(B, H, S, D, grid):
    q = inputs.random_bits(S + 1, (B, H, S, D), std=1.5)
    k = inputs.random_bits(S + 2, (B, H, S, D))
    rng = np.random.default_rng(S)
    w_q = rng.uniform(0.5, 1.5, D).astype(np.float32)
    w_k = rng.uniform(0.5, 1.5, D).astype(np.float32)
    cos, sin = inputs.rope_tables(inputs.rope_positions(grid), D)
    dq, dk = dev_bits(q), dev_bits(k)
    say(f"[prologue] B{B} H{H} S{S} D{D}")
    qk_norm_rope(dq, dk, dev_f32(w_q), dev_f32(w_k), dev_f32(cos), dev_f32(sin), 1e-6)
    torch.cuda.synchronize()
    for got, x, w in ((dq, q, w_q), (dk, k, w_k)):
        ref = oracle.qk_norm_rope(x, w, cos, sin, 1e-6)
        compare.assert_ok(compare.prologue_report(host_f64(got), ref), "prologue")


def test_prologue_single_tensor_and_table_slice():
    """k alone (q = None), rotated with the table rows of a slice of a longer
    sequence: equals the oracle on those positions; q stays untouched."""
    B, H, S, D = 1, 2, 300, 128
    full_cos, full_sin = inputs.rope_tables(inputs.rope_positions(("line", 1000)), D)
    k = inputs.random_bits(7, (B, H, S, D))
    w = np.random.default_rng(8).uniform(0.5, 1.5, D).astype(np.float32)
    dk = dev_bits(k)
    c, s = dev_f32(full_cos), dev_f32(full_sin)
    qk_norm_rope(None, dk, None, dev_f32(w), c[500:800], s[500:800], 1e-5)
    ref = oracle.qk_norm_rope(k, w, full_cos[500:800], full_sin[500:800], 1e-5)
    compare.assert_ok(compare.prologue_report(host_f64(dk), ref), "k-only prologue")
    q = inputs.random_bits(9, (B, H, S, D))
    dq = dev_bits(q)
    qk_norm_rope(dq, None, dev_f32(w), None, c[:S], s[:S], 1e-5)
    ref = oracle.qk_norm_rope(q, w, full_cos[:S], full_sin[:S], 1e-5)
    compare.assert_ok(compare.prologue_report(host_f64(dq), ref), "q-only prologue")


@pytest.mark.parametrize("B,H,S,D", [(1, 3, 300, 128), (2, 41, 19, 64)])
def test_prologue_out_of_place(B, H, S, D):
    """qk_norm_rope_out gives the bits of the in-place form, leaves its inputs
    untouched, and also accepts an output that is its own input."""
    q = inputs.random_bits(S + 11, (B, H, S, D), std=1.5)
    k = inputs.random_bits(S + 12, (B, H, S, D))
    rng = np.random.default_rng(S + 13)
    w_q = dev_f32(rng.uniform(0.5, 1.5, D).astype(np.float32))
    w_k = dev_f32(rng.uniform(0.5, 1.5, D).astype(np.float32))
    cos, sin = inputs.rope_tables(inputs.rope_positions(("line", S)), D)
    c, s_ = dev_f32(cos), dev_f32(sin)
    say(f"[prologue] out of place B{B} H{H} S{S} D{D}")
    dq, dk = dev_bits(q), dev_bits(k)
    qo, ko = torch.empty_like(dq), torch.empty_like(dk)
    qk_norm_rope_out(dq, dk, qo, ko, w_q, w_k, c, s_, 1e-6)
    qi, ki = dq.clone(), dk.clone()
    qk_norm_rope(qi, ki, w_q, w_k, c, s_, 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dq), q) and np.array_equal(host_bits(dk), k), "an input was modified"
    assert torch.equal(qo, qi) and torch.equal(ko, ki), "out-of-place bits differ from in-place"
    # q in place through the out-of-place entry, k alone skipped
    qk_norm_rope_out(dq, None, dq, None, w_q, None, c, s_, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(dq, qi)
    ref = oracle.qk_norm_rope(k, host_f64(w_k).astype(np.float32), cos, sin, 1e-6)
    compare.assert_ok(compare.prologue_report(host_f64(ko), ref), "out-of-place prologue")


def test_prologue_identity_table_is_rmsnorm_bits():
    """cos = 1, sin = 0, w = 1, eps = 0 on rows that are +-c: every output is
    exactly +-1 (a closed form with no rounding)."""
    B, H, S, D = 1, 1, 8, 128
    signs = np.where(np.random.default_rng(1).random((B, H, S, D)) < 0.5, -1.0, 1.0)
    scales = (2.0 ** np.arange(-3, 5))[None, None, :, None]
    x = inputs.to_bf16_bits((signs * scales).astype(np.float32))
    dx = dev_bits(x)
    qk_norm_rope(dx, None, dev_f32(np.ones(D)), None, dev_f32(np.ones((S, D))), dev_f32(np.zeros((S, D))), 0.0)
    np.testing.assert_array_equal(host_f64(dx), signs)


def _merge_inputs(seed, rows, D, a_f32, b_f32):
    rng = np.random.default_rng(seed)
    oa = rng.standard_normal((rows, D)).astype(np.float32)
    ob = rng.standard_normal((rows, D)).astype(np.float32)
    la = (rng.standard_normal(rows) * 4).astype(np.float32)
    lb = (rng.standard_normal(rows) * 4).astype(np.float32)
    if not a_f32:
        oa = inputs.bf16_bits_to_f32(inputs.to_bf16_bits(oa))
    if not b_f32:
        ob = inputs.bf16_bits_to_f32(inputs.to_bf16_bits(ob))
    return oa, la, ob, lb


def _dev(x, f32, shape):
    if f32:
        return dev_f32(x).reshape(shape)
    return dev_bits(inputs.to_bf16_bits(x)).reshape(shape)


@pytest.mark.parametrize("a_f32,b_f32", [(True, True), (True, False), (False, False), (False, True)])
@pytest.mark.parametrize("D", [64, 128])
def test_merge_matches_oracle(a_f32, b_f32, D):
    B, H, Sq = 2, 3, 333
    rows = B * H * Sq
    oa, la, ob, lb = _merge_inputs(D + a_f32 * 2 + b_f32, rows, D, a_f32, b_f32)
    la[:5] = -np.inf                 # side a saw no key
    lb[5:10] = -np.inf               # side b saw no key
    la[10:12] = -np.inf
    lb[10:12] = -np.inf              # neither side saw a key
    da, db = _dev(oa, a_f32, (B, H, Sq, D)), _dev(ob, b_f32, (B, H, Sq, D))
    dla, dlb = dev_f32(la).reshape(B, H, Sq), dev_f32(lb).reshape(B, H, Sq)
    attn_merge(da, dla, db, dlb)
    ref_o, ref_l = oracle.merge(oa.astype(np.float64), la.astype(np.float64),
                                ob.astype(np.float64), lb.astype(np.float64))
    got_o = host_f64(da).reshape(rows, D)
    got_l = host_f64(dla).reshape(rows)
    np.testing.assert_array_equal(got_o[10:12], 0.0)
    assert np.all(got_l[10:12] == -np.inf)
    fin = np.isfinite(ref_l)
    rep = compare.attn_report(got_o, ref_o, got_l[fin], ref_l[fin], bf16=not a_f32)
    if a_f32:
        assert rep["max_abs"] < 1e-5, rep
    compare.assert_ok(rep, "merge")


def test_merge_ignores_the_empty_side():
    """A side whose LSE is -inf contributes nothing, even if its values are NaN."""
    B, H, Sq, D = 1, 1, 64, 128
    oa = torch.full((B, H, Sq, D), float("nan"), device="cuda", dtype=torch.float32)
    la = torch.full((B, H, Sq), float("-inf"), device="cuda")
    ob = torch.randn(B, H, Sq, D, device="cuda")
    lb = torch.randn(B, H, Sq, device="cuda")
    attn_merge(oa, la, ob, lb)
    ref_o, ref_l = oracle.merge(np.full((Sq, D), np.nan), np.full(Sq, -np.inf), host_f64(ob).reshape(Sq, D),
                                host_f64(lb).reshape(Sq))
    assert np.array_equal(host_f64(oa).reshape(Sq, D), ref_o) and np.array_equal(host_f64(la).reshape(Sq), ref_l)
    assert torch.equal(oa, ob) and torch.equal(la, lb)

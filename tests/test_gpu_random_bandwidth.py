"""Seeded random shapes through the bandwidth-bound kernels against the
oracle: the prologue (in place and into separate outputs, q and/or k, any
position-table slice), the out/LSE merge (every dtype pair, rows where one
or both sides saw no key) and the BSND <-> BNSD head-slice layout (any
multiple of 8 for D, any head slice)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import attn_merge, bnsd_to_bsnd, bsnd_to_bnsd, inputs, qk_norm_rope, qk_norm_rope_out
from gpu_common import DEV, dev_bits, dev_f32, host_bits, host_f64, say

pytestmark = pytest.mark.gpu

N = 24


def _shape(rng):
    return (int(rng.integers(1, 4)), int(rng.integers(1, 50)), int(rng.integers(1, 300)), int(rng.choice([64, 128])))


@pytest.mark.parametrize("i", range(N))
def test_random_prologue(i):
    rng = np.random.default_rng(7000 + i)
    B, H, S, D = _shape(rng)
    which = ["both", "q", "k"][i % 3]
    out_of_place = bool(i % 2)
    off = int(rng.integers(0, 200))                      # the rows' positions start at `off`
    eps = float(rng.choice([0.0, 1e-6, 1e-5]))
    cos, sin = inputs.rope_tables(inputs.rope_positions(("line", off + S)), D)
    cos, sin = cos[off:], sin[off:]
    q = inputs.random_bits(7100 + i, (B, H, S, D), std=float(rng.uniform(0.2, 3.0)))
    k = inputs.random_bits(7200 + i, (B, H, S, D), std=float(rng.uniform(0.2, 3.0)))
    w_q = rng.uniform(0.5, 1.5, D).astype(np.float32)
    w_k = rng.uniform(0.5, 1.5, D).astype(np.float32)
    say(f"[random prologue] {i}: B{B} H{H} S{S} D{D} {which} out_of_place={out_of_place} off={off} eps={eps}")
    dq = dev_bits(q) if which != "k" else None
    dk = dev_bits(k) if which != "q" else None
    wq = dev_f32(w_q) if dq is not None else None
    wk = dev_f32(w_k) if dk is not None else None
    c, s_ = dev_f32(cos), dev_f32(sin)
    if out_of_place:
        qo = torch.empty_like(dq) if dq is not None else None
        ko = torch.empty_like(dk) if dk is not None else None
        qk_norm_rope_out(dq, dk, qo, ko, wq, wk, c, s_, eps)
    else:
        qk_norm_rope(dq, dk, wq, wk, c, s_, eps)
        qo, ko = dq, dk
    torch.cuda.synchronize()
    for got, src, w, name in ((qo, q, w_q, "q"), (ko, k, w_k, "k")):
        if got is None:
            continue
        rep = compare.prologue_report(host_f64(got), oracle.qk_norm_rope(src, w, cos, sin, eps))
        compare.assert_ok(rep, f"random prologue {i} {name}")
    if out_of_place:
        for t, src in ((dq, q), (dk, k)):
            if t is not None:
                assert np.array_equal(host_bits(t), src), "an input of the out-of-place form was modified"


@pytest.mark.parametrize("i", range(N))
def test_random_merge(i):
    rng = np.random.default_rng(7300 + i)
    B, H, S, D = _shape(rng)
    a_f32, b_f32 = bool(i & 1), bool(i & 2)
    rows = B * H * S
    oa = rng.standard_normal((rows, D)).astype(np.float32) * np.float32(rng.uniform(0.1, 4))
    ob = rng.standard_normal((rows, D)).astype(np.float32) * np.float32(rng.uniform(0.1, 4))
    la = (rng.standard_normal(rows) * rng.uniform(0.5, 30)).astype(np.float32)
    lb = (rng.standard_normal(rows) * rng.uniform(0.5, 30)).astype(np.float32)
    for arr in (la, lb):
        arr[rng.random(rows) < 0.05] = -np.inf             # a side that saw no key
    if not a_f32:
        oa = inputs.bf16_bits_to_f32(inputs.to_bf16_bits(oa))
    if not b_f32:
        ob = inputs.bf16_bits_to_f32(inputs.to_bf16_bits(ob))
    say(f"[random merge] {i}: B{B} H{H} S{S} D{D} a_f32={a_f32} b_f32={b_f32}")

    def dev(x, f32):
        t = torch.from_numpy(x.reshape(B, H, S, D)).to(DEV)
        return t if f32 else t.bfloat16()

    da, db = dev(oa, a_f32), dev(ob, b_f32)
    dla, dlb = dev_f32(la).reshape(B, H, S), dev_f32(lb).reshape(B, H, S)
    attn_merge(da, dla, db, dlb)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.merge(oa, la, ob, lb)
    got_o, got_l = host_f64(da).reshape(rows, D), host_f64(dla).reshape(rows)
    none = np.isneginf(la) & np.isneginf(lb)
    assert np.all(got_o[none] == 0) and np.all(np.isneginf(got_l[none]))
    rep = compare.attn_report(got_o[~none], ref_o[~none], got_l[~none], ref_l[~none], bf16=not a_f32)
    compare.assert_ok(rep, f"random merge {i}")


@pytest.mark.parametrize("i", range(N))
def test_random_layout(i):
    rng = np.random.default_rng(7400 + i)
    B, S = int(rng.integers(1, 4)), int(rng.integers(1, 400))
    H = int(rng.integers(1, 12))
    D = 8 * int(rng.integers(1, 33))
    hs = int(rng.integers(1, H + 1))
    h0 = int(rng.integers(0, H - hs + 1))
    x = rng.integers(0, 65536, size=(B, S, H, D), dtype=np.uint16)
    say(f"[random layout] {i}: B{B} S{S} H{H} D{D} h0={h0} heads={hs}")
    dx = dev_bits(x)
    o = bsnd_to_bnsd(dx, h0, hs)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(o), oracle.bsnd_to_bnsd(x, h0, hs))
    p = rng.integers(0, 65536, size=(B, hs, S, D), dtype=np.uint16)
    y = rng.integers(0, 65536, size=(B, S, H, D), dtype=np.uint16)
    dy = dev_bits(y)
    bnsd_to_bsnd(dev_bits(p), dy, h0)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dy), oracle.bnsd_to_bsnd(p, y, h0))

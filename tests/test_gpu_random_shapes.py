"""Seeded random shapes through every attention entry point, against the
fp64 oracle: batch, heads, head groups, query and key lengths (1..520, so
most cases end in a ragged tile), D, causal, output dtype, score scale and
input spread are drawn per case, and the entry point cycles through the
plain, workspace, grouped, variable-length, BSND-output and merging forms."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import (attn_fwd, attn_fwd_gqa, attn_fwd_varlen, attn_fwd_workspace_bytes,
                                        attn_fwd_ws, attn_fwd_ws_bsnd, attn_fwd_ws_merge, inputs)
from gpu_common import DEV, dev_bits, host_f64, say

pytestmark = pytest.mark.gpu

ENTRIES = ["plain", "ws", "gqa", "gqa_ws", "varlen", "bsnd", "merge"]
N_CASES = 70


def _cases():
    rng = np.random.default_rng(20261202)
    cases = []
    for i in range(N_CASES):
        entry = ENTRIES[i % len(ENTRIES)]
        D = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 4))
        Hkv = int(rng.integers(1, 3))
        G = int(rng.choice([1, 2, 3])) if entry in ("gqa", "gqa_ws", "varlen") else 1
        Sq = int(rng.integers(1, 521))
        Skv = int(rng.integers(1 if entry != "merge" else 2, 521))
        causal = bool(rng.random() < 0.3) and entry != "merge"
        f32 = bool(rng.random() < 0.5) or entry == "merge"    # a running merge output is kept in fp32
        scale = float(rng.uniform(0.5, 2.0)) / math.sqrt(D)
        std = float(rng.uniform(0.5, 2.0))
        cases.append((i, entry, B, Hkv * G, Hkv, Sq, Skv, D, causal, f32, scale, std))
    return cases


CASES = _cases()


def _ws(B, Hkv, Skv, D):
    return torch.full((attn_fwd_workspace_bytes(B, Hkv, Skv, D),), 0x5A, dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}" for c in CASES])
def test_random_shape(case):
    i, entry, B, H, Hkv, Sq, Skv, D, causal, f32, scale, std = case
    out_dtype = torch.float32 if f32 else torch.bfloat16
    seed = 9000 + 10 * i
    q = inputs.random_bits(seed, (B, H, Sq, D), std=std)
    k = inputs.random_bits(seed + 1, (B, Hkv, Skv, D), std=std)
    v = inputs.random_bits(seed + 2, (B, Hkv, Skv, D))
    say(f"[random] {case}")
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)

    if entry == "varlen":
        rng = np.random.default_rng(seed)
        lq = [int(x) for x in rng.integers(0, Sq + 1, B)]
        lk = [int(x) for x in rng.integers(0, Skv + 1, B)]
        slq = torch.tensor(lq, dtype=torch.int32, device=DEV)
        slk = torch.tensor(lk, dtype=torch.int32, device=DEV)
        o, l = attn_fwd_varlen(dq, dk, dv, slq, slk, workspace=_ws(B, Hkv, Skv, D), scale=scale, causal=causal,
                               out_dtype=out_dtype)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.attn_varlen(q, k, v, lq, lk, scale, causal)
        got_o, got_l = host_f64(o), host_f64(l)
        empty = np.isneginf(ref_l)
        assert np.array_equal(np.isneginf(got_l), empty)
        assert np.all(got_o[empty] == 0)
        rep = compare.attn_report(got_o[~empty], ref_o[~empty], got_l[~empty], ref_l[~empty], bf16=not f32)
        compare.assert_ok(rep, f"random {case}")
        return

    if entry == "plain":
        o, l = attn_fwd(dq, dk, dv, scale=scale, causal=causal, out_dtype=out_dtype)
    elif entry == "ws":
        o, l = attn_fwd_ws(dq, dk, dv, _ws(B, Hkv, Skv, D), scale=scale, causal=causal, out_dtype=out_dtype)
    elif entry == "gqa":
        o, l = attn_fwd_gqa(dq, dk, dv, scale=scale, causal=causal, out_dtype=out_dtype)
    elif entry == "gqa_ws":
        o, l = attn_fwd_gqa(dq, dk, dv, workspace=_ws(B, Hkv, Skv, D), scale=scale, causal=causal,
                            out_dtype=out_dtype)
    elif entry == "bsnd":
        heads, h0 = H + 2, 1
        x = torch.zeros((B, Sq, heads, D), dtype=out_dtype, device=DEV)
        _, l = attn_fwd_ws_bsnd(dq, dk, dv, _ws(B, Hkv, Skv, D), x, out_h0=h0, scale=scale, causal=causal)
        o = x[:, :, h0:h0 + H].permute(0, 2, 1, 3)
    else:  # merge: the keys split at a random point, the second part merged in the epilogue
        cut = int(np.random.default_rng(seed).integers(1, Skv))
        ws = _ws(B, Hkv, Skv, D)
        o, l = attn_fwd_ws(dq, dk[:, :, :cut], dv[:, :, :cut], ws, scale=scale, out_dtype=out_dtype)
        attn_fwd_ws_merge(dq, dk[:, :, cut:], dv[:, :, cut:], ws, o, l, scale=scale)
    torch.cuda.synchronize()
    # Full lengths: the oracle's grouped attention (its K/V head map is
    # pinned against torch's SDPA with enable_gqa on the CPU).
    ref_o, ref_l = oracle.attn_varlen(q, k, v, [Sq] * B, [Skv] * B, scale, causal)
    got_o, got_l = host_f64(o), host_f64(l)
    empty = np.isneginf(ref_l)               # rows that saw no key: out 0, LSE -inf
    assert np.array_equal(np.isneginf(got_l), empty)
    assert np.all(got_o[empty] == 0)
    rep = compare.attn_report(got_o[~empty], ref_o[~empty], got_l[~empty], ref_l[~empty], bf16=not f32)
    compare.assert_ok(rep, f"random {case}")

"""The calls only enqueue kernels on the given stream (no allocation, memset
or synchronisation inside), so a sequence of them can be captured in a HIP
graph and replayed.  Captured here: a ring step of the Wan2.2 workload at a
small size -- the prologue of q and of k into separate outputs, attention
over the local key window (a partly filled last round in 4-wave halves),
then attention over the remote window (split launch and fold) merged into
the first result in its epilogue.  Every replay must give the bits of the
eager run; the replays alternate with eager work on the same tensors
(outputs overwritten, another call, synchronisations)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import (attn_fwd_launch_form, attn_fwd_workspace_bytes, attn_fwd_ws,
                                        attn_fwd_ws_merge, inputs, qk_norm_rope_out)
from gpu_common import DEV, dev_bits, dev_f32, host_bits, rows_of, say

pytestmark = pytest.mark.gpu


def _tables(seed, S, D):
    ang = np.random.default_rng(seed).uniform(0.0, 2 * math.pi, (S, D // 2))
    ang = np.repeat(ang, 2, axis=1)               # pair-duplicated, as the rotary tables are
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def test_ring_step_in_a_hip_graph():
    B, H, Sq, Skv, D, split = 1, 2, 600, 16000, 128, 4000
    eps, scale = 1e-5, 1 / math.sqrt(D)
    q0 = inputs.random_bits(8801, (B, H, Sq, D))
    k0 = inputs.random_bits(8802, (B, H, Skv, D))
    v = inputs.random_bits(8803, (B, H, Skv, D))
    rng = np.random.default_rng(8804)
    w_q = rng.uniform(0.5, 1.5, D).astype(np.float32)
    w_k = rng.uniform(0.5, 1.5, D).astype(np.float32)
    cq, sq = _tables(8805, Sq, D)
    ck, sk = _tables(8806, Skv, D)
    ws_loc = torch.empty(attn_fwd_workspace_bytes(B, H, split, D), dtype=torch.uint8, device=DEV)
    ws_rem = torch.empty(attn_fwd_workspace_bytes(B, H, Skv - split, D), dtype=torch.uint8, device=DEV)
    assert attn_fwd_launch_form(B, H, Sq, split, D, False, ws_loc.numel()) == "halves"
    assert attn_fwd_launch_form(B, H, Sq, Skv - split, D, False, ws_rem.numel()) == "split"

    dq0, dk0, dv = dev_bits(q0), dev_bits(k0), dev_bits(v)
    wq, wk = dev_f32(w_q), dev_f32(w_k)
    dcq, dsq, dck, dsk = dev_f32(cq), dev_f32(sq), dev_f32(ck), dev_f32(sk)
    dq, dk = torch.empty_like(dq0), torch.empty_like(dk0)
    out = torch.empty((B, H, Sq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)

    def step():
        qk_norm_rope_out(dq0, None, dq, None, wq, None, dcq, dsq, eps)
        qk_norm_rope_out(None, dk0, None, dk, None, wk, dck, dsk, eps)
        attn_fwd_ws(dq, dk[:, :, :split], dv[:, :, :split], ws_loc, out=out, lse=lse, scale=scale)
        attn_fwd_ws_merge(dq, dk[:, :, split:], dv[:, :, split:], ws_rem, out, lse, scale=scale)

    say("[graph] eager ring step")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dq, dk, out, lse)]
    rows = inputs.sample_rows(40, B, H, Sq, per_head=48)
    ref_o, ref_l = oracle.attn(host_bits(dq), host_bits(dk), v, scale, False, rows=rows)
    compare.assert_ok(compare.attn_report(rows_of(out, rows), ref_o, rows_of(lse, rows), ref_l, bf16=False),
                      "eager ring step")

    say("[graph] capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on the capture stream's kind of stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    other_o = torch.empty((B, H, Sq, D), dtype=torch.bfloat16, device=DEV)
    for r in range(3):
        say(f"[graph] replay {r}")
        for t in (dq, dk, out, lse):
            t.fill_(float("nan") if t.dtype == torch.float32 else 0)
        attn_fwd_ws(dq0, dk0, dv, torch.empty(attn_fwd_workspace_bytes(B, H, Skv, D), dtype=torch.uint8,
                                                 device=DEV), out=other_o)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((dq, dk, out, lse), ref, ("q", "k", "out", "lse")):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager run"

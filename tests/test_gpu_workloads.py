"""The five workloads at full size: GPU path against the fp64 oracle.

The prologue is compared on every element.  Attention is compared on a
seeded sample of query rows per (b,h) (rows 0, 127, 128, the ragged tail,
the last row and uniform draws), with the oracle consuming the GPU
prologue's bf16 output, so stage errors do not compound.  The Wan2.2 SP-share workload checks
the 4-chunk ring chain with an fp32 accumulator and with bf16 chunk outputs
and accumulator, and the all-gather path (Skv = 75600 in one call).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import (attn_fwd, attn_fwd_ring_overlap, attn_fwd_workspace_bytes, attn_fwd_ws,
                                        attn_fwd_ws_merge, attn_merge, inputs, qk_norm_rope, qk_norm_rope_out)
from gpu_common import dev_bits, dev_f32, host_bits, host_f64, launch_edge_rows, rows_of, say, workload

pytestmark = pytest.mark.gpu


def _prologue(cfg, x):
    cos, sin = inputs.config_rope_tables(cfg)
    dq, dk = dev_bits(x["q"]), dev_bits(x["k"])
    say(f"[{cfg.name}] prologue")
    qk_norm_rope(dq, dk, dev_f32(x["w_q"]), dev_f32(x["w_k"]), dev_f32(cos), dev_f32(sin), cfg.eps)
    torch.cuda.synchronize()
    return dq, dk, cos, sin


def _check_prologue_heads(cfg, x, dq, dk, cos, sin, heads=None):
    for got, src, w, name in ((dq, x["q"], x["w_q"], "q"), (dk, x["k"], x["w_k"], "k")):
        if heads is None:
            ref = oracle.qk_norm_rope(src, w, cos, sin, cfg.eps)
            out = host_f64(got)
        else:
            ref = oracle.qk_norm_rope(np.ascontiguousarray(src[:, heads]), w, cos, sin, cfg.eps)
            out = host_f64(got[:, heads])
        rep = compare.prologue_report(out, ref)
        say(f"[{cfg.name}] prologue {name}: {rep}")
        compare.assert_ok(rep, f"{cfg.name} prologue {name}")


def _check_attn(cfg, q_bits, k_bits, v_bits, out, lse, tag, extra=()):
    rows = inputs.sample_rows(cfg.index, cfg.B, cfg.H, q_bits.shape[2], extra=extra)
    say(f"[{cfg.name}] oracle on {rows.size} rows ({tag})")
    ref_o, ref_l = oracle.attn(q_bits, k_bits, v_bits, cfg.scale, False, rows=rows)
    rep = compare.attn_report(rows_of(out, rows), ref_o, rows_of(lse, rows), ref_l,
                              bf16=out.dtype == torch.bfloat16)
    say(f"[{cfg.name}] {tag}: {rep}")
    compare.assert_ok(rep, f"{cfg.name} {tag}")


@pytest.mark.parametrize("name", ["qwen", "cosmos"])
def test_prologue_then_attention(name):
    cfg = inputs.WORKLOADS[name]
    x = workload(name)
    dq, dk, cos, sin = _prologue(cfg, x)
    _check_prologue_heads(cfg, x, dq, dk, cos, sin)
    dv = dev_bits(x["v"])
    say(f"[{name}] attn_fwd")
    out, lse = attn_fwd(dq, dk, dv, scale=cfg.scale)
    torch.cuda.synchronize()
    _check_attn(cfg, host_bits(dq), host_bits(dk), x["v"], out, lse, "attention")


@pytest.mark.parametrize("times_four", [False, True], ids=["plain", "q_x4"])
def test_wan_attention(times_four):
    cfg = inputs.WORKLOADS["wan"]
    x = workload("wan")
    qb = inputs.times_four_bits(x["q"]) if times_four else x["q"]
    say(f"[wan] attn_fwd {'q x4' if times_four else 'plain'}")
    out, lse = attn_fwd(dev_bits(qb), dev_bits(x["k"]), dev_bits(x["v"]), scale=cfg.scale)
    torch.cuda.synchronize()
    _check_attn(cfg, qb, x["k"], x["v"], out, lse, "q x4" if times_four else "plain")


@pytest.mark.parametrize("times_four", [False, True], ids=["plain", "q_x4"])
def test_wan_measured_step(times_four):
    """The benchmark's default step at full size, call for call: the
    out-of-place prologue of q and k, attn_fwd_ws over the local quarter of
    the keys into fp32 (out, lse), then attn_fwd_ws_merge over the other
    three quarters, merged into that output in the attention epilogue (one
    workspace for both calls).  The Q x4 variant multiplies the normalised q
    by 4 (exact in bf16) so that the logit std is about 4.  Sampled rows
    include the 32-/128-/256-row block edges and the edges of the last-round
    dispatch; the oracle consumes the GPU prologue's output."""
    cfg = inputs.WORKLOADS["wan"]
    x = workload("wan")
    B, H, S, D = cfg.B, cfg.H, cfg.S, cfg.D
    cos, sin = inputs.config_rope_tables(cfg)
    q0, k0, v = dev_bits(x["q"]), dev_bits(x["k"]), dev_bits(x["v"])
    q, k = torch.empty_like(q0), torch.empty_like(k0)
    say(f"[wan] measured step ({'q x4' if times_four else 'plain'}): prologue")
    qk_norm_rope_out(q0, k0, q, k, dev_f32(x["w_q"]), dev_f32(x["w_k"]), dev_f32(cos), dev_f32(sin), cfg.eps)
    torch.cuda.synchronize()
    del q0, k0
    if times_four:
        q.mul_(4)
    c = S // 4
    ws = torch.empty((attn_fwd_workspace_bytes(B, H, S - c, D),), dtype=torch.uint8, device=q.device)
    out = torch.empty((B, H, S, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    say("[wan] measured step: attn_fwd_ws (local quarter), attn_fwd_ws_merge (remote three quarters)")
    attn_fwd_ws(q, k[:, :, :c], v[:, :, :c], ws, out=out, lse=lse, scale=cfg.scale)
    attn_fwd_ws_merge(q, k[:, :, c:], v[:, :, c:], ws, out, lse, scale=cfg.scale)
    torch.cuda.synchronize()
    del ws
    if not times_four:
        _check_prologue_heads(cfg, x, q, k, cos, sin, heads=[0, 39])
    _check_attn(cfg, host_bits(q), host_bits(k), x["v"], out, lse, "measured step" + (" q x4" if times_four else ""),
                extra=launch_edge_rows(B, H, S))


def test_wan_ring_overlap_step():
    """The measured step: prologue on q and k, attention over the local
    quarter of the keys and over the remaining three quarters (windows of the
    same tensors, through the workspace path with one shared workspace), fp32
    outputs merged through their LSE.  The local window runs with a
    workspace of the V part only (no split launch) and must give the bits of
    attn_fwd; the remote window takes the split launch of its last round."""
    cfg = inputs.WORKLOADS["wan"]
    x = workload("wan")
    dq, dk, cos, sin = _prologue(cfg, x)
    _check_prologue_heads(cfg, x, dq, dk, cos, sin, heads=[0, 17, 39])
    dv = dev_bits(x["v"])
    c = cfg.S // 4
    ws = torch.empty((attn_fwd_workspace_bytes(cfg.B, cfg.H, cfg.S - c, cfg.D),), dtype=torch.uint8,
                     device=dq.device)
    say("[wan] ring-overlap attention (workspace path)")
    v_part = cfg.B * cfg.H * (-(-c // 64) * 64 * cfg.D * 2 + cfg.D * 4)
    oa, la = attn_fwd_ws(dq, dk[:, :, :c], dv[:, :, :c], ws[:v_part], scale=cfg.scale, out_dtype=torch.float32)
    op, lp = attn_fwd(dq, dk[:, :, :c], dv[:, :, :c], scale=cfg.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(oa, op) and torch.equal(la, lp)
    del op, lp
    ob, lb = attn_fwd_ws(dq, dk[:, :, c:], dv[:, :, c:], ws, scale=cfg.scale, out_dtype=torch.float32)
    attn_merge(oa, la, ob, lb)
    torch.cuda.synchronize()
    _check_attn(cfg, host_bits(dq), host_bits(dk), x["v"], oa, la, "ring-overlap step")


@pytest.mark.parametrize("name", ["qwen", "cosmos"])
def test_ring_overlap_two_streams(name):
    """Ring Attention Overlap on one GPU: the local quarter of the keys on a
    side stream, concurrently with the remote three quarters on the current
    stream, then the LSE merge.  Same bits as the one-stream order, and the
    oracle's full attention on sampled rows."""
    cfg = inputs.WORKLOADS[name]
    x = workload(name)
    dq, dk, cos, sin = _prologue(cfg, x)
    dv = dev_bits(x["v"])
    c = cfg.S // 4
    mk_ws = lambda n: torch.empty((attn_fwd_workspace_bytes(cfg.B, cfg.H, n, cfg.D),), dtype=torch.uint8,  # noqa: E731
                                  device=dq.device)
    ws_a, ws_b = mk_ws(c), mk_ws(cfg.S - c)
    say(f"[{name}] ring overlap, one stream")
    o1, l1 = attn_fwd_ring_overlap(dq, dk, dv, c, ws_a, ws_b, scale=cfg.scale)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dq.device)
    say(f"[{name}] ring overlap, two streams")
    o2, l2 = attn_fwd_ring_overlap(dq, dk, dv, c, ws_a, ws_b, scale=cfg.scale, side_stream=side)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    _check_attn(cfg, host_bits(dq), host_bits(dk), x["v"], o2, l2, "ring overlap, two streams")
    with pytest.raises(ValueError):
        attn_fwd_ring_overlap(dq, dk, dv, c, ws_a, ws_a, scale=cfg.scale, side_stream=side)


def test_sp_share_chains():
    cfg = inputs.WORKLOADS["wan_sp"]
    x4 = workload("wan")
    q = np.ascontiguousarray(x4["q"][:, :, : cfg.Sq])
    kc, vc = inputs.split_kv(x4["k"], cfg.chunks), inputs.split_kv(x4["v"], cfg.chunks)
    dq = dev_bits(q)
    results = {}
    for acc_dtype in (torch.float32, torch.bfloat16):
        acc_o = acc_l = None
        for i in range(cfg.chunks):
            say(f"[wan_sp] chunk {i} ({acc_dtype})")
            o, l = attn_fwd(dq, dev_bits(kc[i]), dev_bits(vc[i]), scale=cfg.scale, out_dtype=acc_dtype)
            if acc_o is None:
                acc_o, acc_l = o, l
            else:
                attn_merge(acc_o, acc_l, o, l)
                del o, l
        torch.cuda.synchronize()
        results[acc_dtype] = (acc_o, acc_l)
    say("[wan_sp] gather path (all keys in one call)")
    go, gl = attn_fwd(dq, dev_bits(x4["k"]), dev_bits(x4["v"]), scale=cfg.scale)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(cfg.index, cfg.B, cfg.H, cfg.Sq)
    say(f"[wan_sp] oracle on {rows.size} rows")
    ref_o, ref_l = oracle.attn(q, x4["k"], x4["v"], cfg.scale, False, rows=rows)
    reps = {}
    for name, (o, l) in (("fp32 chain", results[torch.float32]), ("bf16 chain", results[torch.bfloat16]),
                         ("gather", (go, gl))):
        reps[name] = compare.attn_report(rows_of(o, rows), ref_o, rows_of(l, rows), ref_l,
                                         bf16=o.dtype == torch.bfloat16)
        say(f"[wan_sp] {name}: {reps[name]}")
    # The fp32 chain rounded once to bf16 at the end.
    o32 = results[torch.float32][0].to(torch.bfloat16)
    reps["fp32 chain, bf16-rounded"] = compare.attn_report(rows_of(o32, rows), ref_o)
    say(f"[wan_sp] fp32 chain bf16-rounded: {reps['fp32 chain, bf16-rounded']}")
    for name, rep in reps.items():
        compare.assert_ok(rep, f"wan_sp {name}")
    # Rounding every chunk to bf16 costs accuracy, as the pages warn.
    assert reps["bf16 chain"]["max_abs"] >= reps["fp32 chain"]["max_abs"]

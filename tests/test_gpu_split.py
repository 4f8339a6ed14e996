"""The split launch of the workspace path.  When the last round of 256-row
query tiles is partly filled, the key tiles of that round's query tiles are
dealt in equal shares to one workgroup per CU; a query tile cut between
shares is assembled from its pieces with the merge arithmetic by a fold
launch that follows.

Checked here: which launch form a call takes; every row of split tiles
(tiles cut into several pieces, ragged key and query tails) against the
oracle; repeatability (the pieces are folded in key order); rows outside
the split tiles keep the bits of the unsplit form; and the bit relations
between entry points that take the same form (fused Q, BSND store, merging
epilogue, grouped K/V heads)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import (attn_fwd_gqa, attn_fwd_launch_form, attn_fwd_workspace_bytes, attn_fwd_ws,
                                        attn_fwd_ws_bsnd, attn_fwd_ws_fused_q, attn_fwd_ws_merge, attn_merge,
                                        bnsd_to_bsnd, inputs, qk_norm_rope)
from gpu_common import DEV, dev_bits, dev_f32, host_bits, host_f64, rows_of, say

pytestmark = pytest.mark.gpu


def v_part(B, H, Skv, D):
    """Workspace bytes of the prepared V alone (no split region)."""
    return B * H * (((Skv + 63) // 64) * 64 * D * 2 + D * 4)


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def split_rows(B, H, Sq):
    """Flat query rows of the tiles that the split launch covers (the last
    T mod CUs of the T = B*H*ceil(Sq/256) tiles, head-major)."""
    nq = (Sq + 255) // 256
    T = B * H * nq
    rows = []
    for t in range(T - T % cus(), T):
        bh, qt = divmod(t, nq)
        rows.extend(bh * Sq + r for r in range(qt * 256, min(Sq, qt * 256 + 256)))
    return np.asarray(rows, dtype=np.int64)


def full_ws(B, H, Skv, D):
    return torch.full((attn_fwd_workspace_bytes(B, H, Skv, D),), 0x7E, dtype=torch.uint8, device=DEV)


def test_launch_forms():
    """Forms on this device for the Wan2.2 call shapes and small grids."""
    if cus() != 256:
        pytest.skip("the expected forms are those of a 256-CU device")
    B, H, S, D = 1, 40, 75600, 128
    full = attn_fwd_workspace_bytes(B, H, S, D)
    assert attn_fwd_launch_form(B, H, S, S, D, workspace_bytes=full) == "split"
    assert attn_fwd_launch_form(B, H, S, S // 4, D, workspace_bytes=full) == "split"
    assert attn_fwd_launch_form(B, H, S, S, D, workspace_bytes=v_part(B, H, S, D)) == "halves"
    assert attn_fwd_launch_form(B, H, S, S, D) == "one"
    assert attn_fwd_launch_form(B, H, S, S, D, causal=True, workspace_bytes=full) == "one"
    # Few key tiles: a share would cost more than the whole tiles.
    assert attn_fwd_launch_form(1, 3, 1000, 500, D, workspace_bytes=full) == "halves"
    assert attn_fwd_launch_form(1, 3, 1000, 5000, D, workspace_bytes=full) == "halves"
    # Qwen-Image keeps one launch (its last round, 152 tiles of 68 key
    # tiles, costs less whole than split); Cosmos-Predict splits.
    assert attn_fwd_launch_form(1, 24, 4312, 4312, D, workspace_bytes=full) == "one"
    assert attn_fwd_launch_form(2, 16, 12480, 12480, D, workspace_bytes=full) == "split"
    # Grids that fill their last round exactly need no split.
    assert attn_fwd_launch_form(1, 256, 256, 8192, D, workspace_bytes=full) == "one"
    # Per-batch lengths never split.
    assert attn_fwd_launch_form(1, 3, 1000, 13000, D, workspace_bytes=full, varlen=True) == "halves"
    assert attn_fwd_launch_form(1, 3, 1000, 13000, D, workspace_bytes=full) == "split"


CASES = [  # B, H, Sq, Skv, D, out dtype
    (1, 2, 600, 13000, 128, torch.bfloat16),   # 6 tiles of 204 key tiles: ~13 pieces per tile
    (2, 1, 500, 15001, 64, torch.float32),     # ragged query and key tails
    (1, 1, 200, 20000, 128, torch.float32),    # one tile cut into 19 pieces
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}q{c[2]}k{c[3]}D{c[4]}" for c in CASES])
def test_split_matches_oracle(case):
    B, H, Sq, Skv, D, out_dtype = case
    seed = 9000 + Sq + Skv
    q = inputs.random_bits(seed, (B, H, Sq, D))
    k = inputs.random_bits(seed + 1, (B, H, Skv, D))
    v = inputs.random_bits(seed + 2, (B, H, Skv, D))
    scale = 1 / math.sqrt(D)
    full = attn_fwd_workspace_bytes(B, H, Skv, D)
    assert attn_fwd_launch_form(B, H, Sq, Skv, D, workspace_bytes=full) == "split"
    say(f"[split] {case}")
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    ws = full_ws(B, H, Skv, D)
    o1, l1 = attn_fwd_ws(dq, dk, dv, ws, scale=scale, out_dtype=out_dtype)
    o2, l2 = attn_fwd_ws(dq, dk, dv, ws, scale=scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "two identical calls differ"
    ref_o, ref_l = oracle.attn(q, k, v, scale, False)
    rep = compare.attn_report(host_f64(o1), ref_o, host_f64(l1), ref_l, bf16=out_dtype == torch.bfloat16)
    say(f"[split] {case}: {rep}")
    compare.assert_ok(rep, f"split {case}")


def test_split_after_full_rounds():
    """320 tiles on 256 CUs: a full round of whole tiles, then the split
    launch of the other 64 (188 key tiles each, 4 pieces per tile).  Rows of the full round keep the bits of the
    unsplit form (a workspace without the split region); rows of the split
    tiles agree with the oracle and with the unsplit form to rounding."""
    B, H, Sq, Skv, D = 1, 40, 2000, 12000, 128
    if cus() != 256:
        pytest.skip("tile counts are chosen for a 256-CU device")
    q = inputs.random_bits(9101, (B, H, Sq, D))
    k = inputs.random_bits(9102, (B, H, Skv, D))
    v = inputs.random_bits(9103, (B, H, Skv, D))
    full = attn_fwd_workspace_bytes(B, H, Skv, D)
    assert attn_fwd_launch_form(B, H, Sq, Skv, D, workspace_bytes=full) == "split"
    assert attn_fwd_launch_form(B, H, Sq, Skv, D, workspace_bytes=v_part(B, H, Skv, D)) == "halves"
    say("[split] after full rounds")
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    o_s, l_s = attn_fwd_ws(dq, dk, dv, full_ws(B, H, Skv, D), out_dtype=torch.float32)
    ws_v = torch.full((v_part(B, H, Skv, D),), 0x7E, dtype=torch.uint8, device=DEV)
    o_u, l_u = attn_fwd_ws(dq, dk, dv, ws_v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    sr = split_rows(B, H, Sq)
    assert len(sr) == 64 * 256 - 8 * 48          # 64 tiles, the last of each of 8 heads ragged (2000 = 7*256 + 208)
    keep = np.ones(B * H * Sq, dtype=bool)
    keep[sr] = False
    a, b = host_f64(o_s).reshape(-1, D), host_f64(o_u).reshape(-1, D)
    assert np.array_equal(a[keep], b[keep]) and np.array_equal(host_f64(l_s).reshape(-1)[keep],
                                                               host_f64(l_u).reshape(-1)[keep])
    assert float(np.max(np.abs(a[sr] - b[sr]))) <= 1e-4
    rng = np.random.default_rng(9104)
    rows = np.concatenate([sr[:256], rng.choice(sr, 300, replace=False), rng.choice(np.flatnonzero(keep), 100,
                                                                                   replace=False)])
    ref_o, ref_l = oracle.attn(q, k, v, 1 / math.sqrt(D), False, rows=rows)
    rep = compare.attn_report(rows_of(o_s, rows), ref_o, rows_of(l_s, rows), ref_l, bf16=False)
    compare.assert_ok(rep, "split after full rounds")


B4, H4, SQ4, SKV4, D4 = 1, 4, 600, 13000, 128     # 12 tiles of 204 key tiles


def _inputs4(seed):
    return (inputs.random_bits(seed, (B4, H4, SQ4, D4)), inputs.random_bits(seed + 1, (B4, H4, SKV4, D4)),
            inputs.random_bits(seed + 2, (B4, H4, SKV4, D4)))


def test_split_fused_q_and_bsnd():
    """Fused Q prologue and BSND store under the split launch: the bits of
    qk_norm_rope + attn_fwd_ws, and of attn_fwd_ws + bnsd_to_bsnd."""
    assert attn_fwd_launch_form(B4, H4, SQ4, SKV4, D4, workspace_bytes=attn_fwd_workspace_bytes(B4, H4, SKV4, D4)) \
        == "split"
    q, k, v = _inputs4(9201)
    rng = np.random.default_rng(9204)
    w_q = rng.uniform(0.5, 1.5, D4).astype(np.float32)
    cos, sin = inputs.rope_tables(inputs.rope_positions(("line", SQ4)), D4)
    say("[split] fused q and bsnd")
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    wq, cq, sq = dev_f32(w_q), dev_f32(cos), dev_f32(sin)
    ws = full_ws(B4, H4, SKV4, D4)
    of, lf = attn_fwd_ws_fused_q(dq, dk, dv, ws, wq, cq, sq, 1e-6)
    dq2 = dq.clone()
    qk_norm_rope(dq2, None, wq, None, cq, sq, 1e-6)
    ou, lu = attn_fwd_ws(dq2, dk, dv, ws)
    heads, h0 = 7, 2
    x1 = torch.zeros((B4, SQ4, heads, D4), dtype=torch.bfloat16, device=DEV)
    x2 = torch.zeros_like(x1)
    _, lb = attn_fwd_ws_bsnd(dq2, dk, dv, ws, x1, out_h0=h0)
    bnsd_to_bsnd(ou, x2, h0)
    torch.cuda.synchronize()
    assert torch.equal(of, ou) and torch.equal(lf, lu), "fused and unfused results differ"
    assert np.array_equal(host_bits(x1), host_bits(x2)) and torch.equal(lb, lu), "BSND store differs"
    ref_o, ref_l = oracle.attn(host_bits(dq2), k, v, 1 / math.sqrt(D4), False)
    compare.assert_ok(compare.attn_report(host_f64(of), ref_o, host_f64(lf), ref_l), "split fused q")


@pytest.mark.parametrize("a_dtype", [torch.float32, torch.bfloat16])
def test_split_merging_epilogue(a_dtype):
    """attn_fwd_ws_merge under the split launch: the bits of attn_fwd_ws into
    fp32 followed by attn_merge; the union of both key chunks against the
    oracle."""
    q, k, v = _inputs4(9301)
    Ka = 700
    say(f"[split] merging epilogue {a_dtype}")
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    ka, va = dk[:, :, :Ka].contiguous(), dv[:, :, :Ka].contiguous()
    kb, vb = dk[:, :, Ka:].contiguous(), dv[:, :, Ka:].contiguous()
    Kb = SKV4 - Ka
    assert attn_fwd_launch_form(B4, H4, SQ4, Kb, D4, workspace_bytes=attn_fwd_workspace_bytes(B4, H4, Kb, D4)) \
        == "split"
    ws = full_ws(B4, H4, SKV4, D4)
    oa, la = attn_fwd_ws(dq, ka, va, ws, out_dtype=a_dtype)
    o2, l2 = oa.clone(), la.clone()
    attn_fwd_ws_merge(dq, kb, vb, ws, oa, la)
    t, tl = attn_fwd_ws(dq, kb, vb, ws, out_dtype=torch.float32)
    attn_merge(o2, l2, t, tl)
    torch.cuda.synchronize()
    assert torch.equal(oa, o2) and torch.equal(la, l2), "fused merge differs from attention + attn_merge"
    ref_o, ref_l = oracle.attn(q, k, v, 1 / math.sqrt(D4), False)
    rep = compare.attn_report(host_f64(oa), ref_o, host_f64(la), ref_l, bf16=a_dtype == torch.bfloat16)
    compare.assert_ok(rep, f"split merging epilogue {a_dtype}")


def test_split_grouped_kv_heads():
    """Two K/V heads for four query heads under the split launch: the bits of
    attn_fwd_ws on K/V repeated per query head, and the oracle's grouping."""
    q, _, _ = _inputs4(9401)
    k = inputs.random_bits(9402, (B4, 2, SKV4, D4))
    v = inputs.random_bits(9403, (B4, 2, SKV4, D4))
    say("[split] grouped K/V heads")
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    og, lg = attn_fwd_gqa(dq, dk, dv, full_ws(B4, 2, SKV4, D4))
    dk4 = dk.repeat_interleave(2, dim=1).contiguous()
    dv4 = dv.repeat_interleave(2, dim=1).contiguous()
    om, lm = attn_fwd_ws(dq, dk4, dv4, full_ws(B4, H4, SKV4, D4))
    torch.cuda.synchronize()
    assert torch.equal(og, om) and torch.equal(lg, lm)
    ref_o, ref_l = oracle.attn_varlen(q, k, v, np.full(B4, SQ4, np.int32), np.full(B4, SKV4, np.int32),
                                      1 / math.sqrt(D4), False)
    compare.assert_ok(compare.attn_report(host_f64(og), ref_o, host_f64(lg), ref_l), "split gqa")

"""attn_fwd_ws (V rewritten once into a caller workspace, then streamed into
LDS by DMA) on the GPU: the same results as attn_fwd, bit for bit, and the
oracle's within the parity tolerances, on the attention cases of the plain
path plus key windows, D = 64 and a reused workspace."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import attn_fwd, attn_fwd_launch_form, attn_fwd_ws, attn_fwd_workspace_bytes, inputs
from attention_qk_norm_rope_amd.binding import DitAttnError
from gpu_common import DEV, dev_bits, host_f64, say
from test_gpu_attn import CASES, _ids

pytestmark = pytest.mark.gpu


def _ws(B, H, Skv, D, fill=0x7E):
    n = attn_fwd_workspace_bytes(B, H, Skv, D)
    # Filled with garbage (fp16 NaN patterns) so unread-before-written bytes would show.
    return torch.full((n,), fill, dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_ws_matches_plain_and_oracle(case):
    B, H, Sq, Skv, D, causal, scale, out_dtype = case
    if scale is None:
        scale = 1 / math.sqrt(D)
    seed = Sq * 7 + Skv
    q = inputs.random_bits(seed, (B, H, Sq, D))
    k = inputs.random_bits(seed + 1, (B, H, Skv, D))
    v = inputs.random_bits(seed + 2, (B, H, Skv, D))
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    say(f"[attn_ws] {_ids(case)}")
    o1, l1 = attn_fwd_ws(dq, dk, dv, _ws(B, H, Skv, D), scale=scale, causal=causal, out_dtype=out_dtype)
    o0, l0 = attn_fwd(dq, dk, dv, scale=scale, causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    ref_o, ref_l = oracle.attn(q, k, v, scale, causal)
    rep = compare.attn_report(host_f64(o1), ref_o, host_f64(l1), ref_l, bf16=out_dtype == torch.bfloat16)
    compare.assert_ok(rep, "ws " + _ids(case))


def test_ws_on_key_windows_and_reuse():
    """Windows of longer K/V (the strided layout), one workspace reused for
    calls of decreasing size: every call equals attn_fwd bit for bit."""
    B, H, S, Sq, D = 1, 3, 700, 300, 128
    q = dev_bits(inputs.random_bits(71, (B, H, Sq, D)))
    k = dev_bits(inputs.random_bits(72, (B, H, S, D)))
    v = dev_bits(inputs.random_bits(73, (B, H, S, D)))
    ws = _ws(B, H, S, D)
    for a, b in ((0, 700), (175, 700), (64, 129), (0, 1)):
        say(f"[attn_ws] window {a}:{b}")
        ow, lw = attn_fwd_ws(q, k[:, :, a:b], v[:, :, a:b], ws, out_dtype=torch.float32)
        oc, lc = attn_fwd(q, k[:, :, a:b], v[:, :, a:b], out_dtype=torch.float32)
        assert torch.equal(ow, oc) and torch.equal(lw, lc), (a, b)


def test_ws_large_logits_d64():
    B, H, Sq, Skv, D = 2, 2, 333, 1111, 64
    q = inputs.random_bits(81, (B, H, Sq, D), std=8.0)
    k = inputs.random_bits(82, (B, H, Skv, D))
    v = inputs.random_bits(83, (B, H, Skv, D))
    say("[attn_ws] D64 std-8 logits")
    out, lse = attn_fwd_ws(dev_bits(q), dev_bits(k), dev_bits(v), _ws(B, H, Skv, D), out_dtype=torch.float32)
    ref_o, ref_l = oracle.attn(q, k, v, 1 / math.sqrt(D))
    compare.assert_ok(compare.attn_report(host_f64(out), ref_o, host_f64(lse), ref_l, bf16=False), "ws D64")


def test_ws_rejects_small_or_misplaced_workspace():
    """The V part is the minimum; the full size adds the split region, and
    anything in between runs without the split launch."""
    B, H, S, D = 1, 2, 256, 128
    q = dev_bits(inputs.random_bits(91, (B, H, S, D)))
    n = attn_fwd_workspace_bytes(B, H, S, D)
    v_part = B * H * ((S // 64) * 64 * D * 2 + D * 4)
    np.testing.assert_equal(n, v_part + 512 * 256 * (D + 1) * 4)
    small = torch.empty((v_part - 16,), dtype=torch.uint8, device=DEV)
    with pytest.raises(DitAttnError) as e:
        attn_fwd_ws(q, q, q, small)
    assert e.value.status == 2
    with pytest.raises(DitAttnError) as e:            # workspace on top of the output
        out = torch.empty((n // 2,), dtype=torch.bfloat16, device=DEV)
        attn_fwd_ws(q, q, q, out, out=out[: B * H * S * D].view(B, H, S, D))
    assert e.value.status == 5
    o1, l1 = attn_fwd_ws(q, q, q, torch.empty((n - 16,), dtype=torch.uint8, device=DEV))
    o2, l2 = attn_fwd_ws(q, q, q, torch.empty((v_part,), dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("lo,hi", [(-20.0, 100.0), (60.0, 127.0), (15.0, 16.5)])
def test_value_range_of_v_workspace_path(lo, hi):
    """The workspace path takes any bf16 V: magnitudes 2^lo .. 2^hi, beyond
    fp16's 65504, in every column (so columns are scaled by powers of two
    before the fp16 conversion and the output is scaled back).  The error is
    bounded, as below, relative to the largest |v|; with the largest values
    alone (no smaller ones) the output keeps fp16 precision."""
    B, H, Sq, Skv, D = 1, 2, 200, 300, 128
    rng = np.random.default_rng(int(hi))
    mag = np.exp2(rng.uniform(lo, hi, size=(B, H, Skv, D)))
    v = inputs.to_bf16_bits(np.where(rng.random(mag.shape) < 0.5, -mag, mag).astype(np.float32))
    q = inputs.random_bits(98, (B, H, Sq, D))
    k = inputs.random_bits(99, (B, H, Skv, D))
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    say(f"[attn_ws] value range of v 2^{lo} .. 2^{hi}")
    o1, l1 = attn_fwd_ws(dq, dk, dv, _ws(B, H, Skv, D), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attn(q, k, v, 1 / math.sqrt(D), False)
    got = host_f64(o1)
    vmax = float(np.max(np.abs(inputs.bf16_bits_to_f64(v))))
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - ref_o))) <= 2.0 ** -10 * vmax
    assert float(np.max(np.abs(host_f64(l1) - ref_l))) <= 1e-3
    if hi - lo < 2:
        # every value within a factor 4 of its column's largest: fp16 relative precision
        rel = np.abs(got - ref_o) / np.maximum(np.abs(ref_o), 2.0 ** lo)
        assert float(rel.max()) <= 2.0 ** -9


def test_v_beyond_fp16_without_workspace_is_not_finite():
    """Without a workspace a value of V beyond fp16's range (here 2^17 in one
    key of column 5) makes that column of every output row non-finite (+-inf,
    or NaN where the key's P rounds to 0), as the header states, while the
    other columns and the LSE stay correct; the workspace path takes the same
    V and matches the oracle, column 5 relative to its largest |v|."""
    B, H, Sq, Skv, D = 1, 2, 300, 200, 64
    q = inputs.random_bits(90, (B, H, Sq, D))
    k = inputs.random_bits(91, (B, H, Skv, D))
    v = inputs.random_bits(92, (B, H, Skv, D))
    v[:, :, 77, 5] = inputs.to_bf16_bits(np.array([2.0 ** 17], dtype=np.float32))[0]
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    say("[attn] v beyond fp16 without a workspace")
    o0, l0 = attn_fwd(dq, dk, dv, out_dtype=torch.float32)
    o1, l1 = attn_fwd_ws(dq, dk, dv, _ws(B, H, Skv, D), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attn(q, k, v, 1 / math.sqrt(D), False)
    got = host_f64(o0)
    assert not np.isfinite(got[..., 5]).any()
    others = [d for d in range(D) if d != 5]
    rep = compare.attn_report(got[..., others], ref_o[..., others], host_f64(l0), ref_l, bf16=False)
    compare.assert_ok(rep, "columns other than the out-of-range one")
    # Workspace path: column 5 is scaled into fp16 range, so its error is
    # relative to that column's largest |v| (as in the range tests above).
    got1 = host_f64(o1)
    assert np.all(np.isfinite(got1))
    assert float(np.max(np.abs(got1[..., 5] - ref_o[..., 5]))) <= 2.0 ** -10 * 2.0 ** 17
    rep = compare.attn_report(got1[..., others], ref_o[..., others], host_f64(l1), ref_l, bf16=False)
    compare.assert_ok(rep, "workspace path, other columns")


def test_value_range_of_v():
    """V spanning 2^-20 .. 2^15.9 in magnitude (P V runs on fp16 operands):
    within [2^-14, 65504] the bf16 -> fp16 conversion is exact, below it the
    absolute error stays under 2^-25, so the fp32 output tracks the oracle
    to the fp16 rounding of P, relative to the largest |v|."""
    B, H, Sq, Skv, D = 1, 2, 200, 300, 128
    rng = np.random.default_rng(97)
    mag = np.exp2(rng.uniform(-20.0, 15.9, size=(B, H, Skv, D)))
    v = inputs.to_bf16_bits(np.where(rng.random(mag.shape) < 0.5, -mag, mag).astype(np.float32))
    q = inputs.random_bits(98, (B, H, Sq, D))
    k = inputs.random_bits(99, (B, H, Skv, D))
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    say("[attn_ws] value range of v")
    o1, l1 = attn_fwd_ws(dq, dk, dv, _ws(B, H, Skv, D), out_dtype=torch.float32)
    o0, l0 = attn_fwd(dq, dk, dv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    ref_o, ref_l = oracle.attn(q, k, v, 1 / math.sqrt(D), False)
    got = host_f64(o1)
    vmax = float(np.max(np.abs(inputs.bf16_bits_to_f64(v))))
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - ref_o))) <= 2.0 ** -10 * vmax
    assert float(np.max(np.abs(host_f64(l1) - ref_l))) <= 1e-3


@pytest.mark.parametrize("B,H,Sq,causal,form", [
    (1, 129, 256, False, "one"),     # 129 tiles of 256 rows: last round more than half full, one 8-wave launch
    (1, 128, 256, True, "all4"),     # causal, small grid, last round half full: 4-wave workgroups throughout
    (3, 43, 300, False, "halves"),   # 258 tiles = one full round + 2: 8-wave launch, then the 2 tiles as 4 halves
    (1, 96, 256, False, "halves"),   # 96 tiles, no full round: the halves launch alone
    (2, 100, 200, False, "one"),     # 200 tiles: one 8-wave launch
])
def test_ws_workgroup_sizes_match_plain(B, H, Sq, causal, form):
    """The workspace path launches 8-wave workgroups, 4-wave workgroups, or
    8-wave workgroups followed by the last round's tiles as 4-wave halves,
    depending on the grid; every form gives the bits of the path without a
    workspace (one 8-wave launch) and agrees with the oracle on sampled rows."""
    Skv, D = 150, 128
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        # 3 key tiles: a split launch never pays, whatever the workspace.
        assert attn_fwd_launch_form(B, H, Sq, Skv, D, causal, attn_fwd_workspace_bytes(B, H, Skv, D)) == form
    q = inputs.random_bits(B * H + Sq, (B, H, Sq, D))
    k = inputs.random_bits(B * H + Sq + 1, (B, H, Skv, D))
    v = inputs.random_bits(B * H + Sq + 2, (B, H, Skv, D))
    say(f"[ws] workgroup sizes B{B} H{H} Sq{Sq} causal={causal}")
    dq, dk, dv = dev_bits(q), dev_bits(k), dev_bits(v)
    o_ws, l_ws = attn_fwd_ws(dq, dk, dv, _ws(B, H, Skv, D), causal=causal, out_dtype=torch.float32)
    o_pl, l_pl = attn_fwd(dq, dk, dv, causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_ws, o_pl) and torch.equal(l_ws, l_pl)
    rows = np.random.default_rng(Sq).choice(B * H * Sq, 300, replace=False)
    ref_o, ref_l = oracle.attn(q, k, v, 1 / math.sqrt(D), causal, rows=rows)
    got_o = host_f64(o_ws).reshape(-1, D)[rows]
    got_l = host_f64(l_ws).reshape(-1)[rows]
    compare.assert_ok(compare.attn_report(got_o, ref_o, got_l, ref_l, bf16=False), "workgroup sizes")

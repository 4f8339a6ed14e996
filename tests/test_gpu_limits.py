"""Maximum sizes: one (b,h) slab of K/V (or of q) as long as the 32-bit
buffer offsets of the kernels allow -- (S + 512) * D * 2 bytes <= 2^31 - 1,
i.e. 8,388,095 rows at D = 128 -- through the paths with and without a
workspace, checked against the oracle on sampled query rows; and one row
more is rejected before anything is launched."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import attn_fwd, attn_fwd_launch_form, attn_fwd_workspace_bytes, attn_fwd_ws
from attention_qk_norm_rope_amd.binding import DitAttnError
from gpu_common import DEV, host_f64, say

pytestmark = pytest.mark.gpu

D = 128
S_MAX = (2**31 - 1) // (2 * D) - 512        # 8,388,095


def _rand(gen, shape):
    return torch.randn(shape, device=DEV, generator=gen).to(torch.bfloat16)


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def test_longest_key_slab():
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    Sq = 300
    q, k, v = _rand(g, (1, 1, Sq, D)), _rand(g, (1, 1, S_MAX, D)), _rand(g, (1, 1, S_MAX, D))
    scale = 1 / math.sqrt(D)
    say(f"[limits] Skv = {S_MAX}: attn_fwd")
    o0, l0 = attn_fwd(q, k, v, scale=scale, out_dtype=torch.float32)
    # A workspace of the V part only: the bits of attn_fwd.
    say(f"[limits] Skv = {S_MAX}: attn_fwd_ws, V part only")
    v_part = (S_MAX + 63) // 64 * 64 * D * 2 + D * 4
    ws = torch.empty((v_part,), dtype=torch.uint8, device=DEV)
    o1, l1 = attn_fwd_ws(q, k, v, ws, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    del ws, o1, l1
    # The full workspace: the two query tiles' 131072 key tiles are split
    # between one workgroup per CU.
    n = attn_fwd_workspace_bytes(1, 1, S_MAX, D)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert attn_fwd_launch_form(1, 1, Sq, S_MAX, D, workspace_bytes=n) == "split"
    say(f"[limits] Skv = {S_MAX}: attn_fwd_ws, split launch")
    ws = torch.empty((n,), dtype=torch.uint8, device=DEV)
    o2, l2 = attn_fwd_ws(q, k, v, ws, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    del ws
    rows = np.array([0, 1, 127, 128, 255, 256, 299], dtype=np.int64)
    say(f"[limits] oracle on {rows.size} rows x {S_MAX} keys")
    ref_o, ref_l = oracle.attn(_bits(q), _bits(k), _bits(v), scale, False, rows=rows)
    idx = torch.from_numpy(rows).to(DEV)
    for name, o, l in (("attn_fwd", o0, l0), ("split", o2, l2)):
        rep = compare.attn_report(host_f64(o.reshape(-1, D)[idx]), ref_o, host_f64(l.reshape(-1)[idx]), ref_l,
                                  bf16=False)
        say(f"[limits] {name}: {rep}")
        compare.assert_ok(rep, f"longest key slab, {name}")
    # One key more no longer fits the kernels' 32-bit offsets.
    k2 = torch.empty((1, 1, S_MAX + 1, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(DitAttnError):
        attn_fwd(q, k2, k2, scale=scale)


def test_longest_query_slab():
    g = torch.Generator(device=DEV)
    g.manual_seed(12)
    Skv = 77
    q, k, v = _rand(g, (1, 1, S_MAX, D)), _rand(g, (1, 1, Skv, D)), _rand(g, (1, 1, Skv, D))
    ws = torch.empty((attn_fwd_workspace_bytes(1, 1, Skv, D),), dtype=torch.uint8, device=DEV)
    say(f"[limits] Sq = {S_MAX}: attn_fwd_ws, causal")
    o, l = attn_fwd_ws(q, k, v, ws, causal=True)
    torch.cuda.synchronize()
    rows = np.array([0, 76, 77, 5_000_000, S_MAX - 257, S_MAX - 1], dtype=np.int64)
    qr = _bits(q.reshape(-1, D)[torch.from_numpy(rows).to(DEV)].reshape(1, 1, -1, D))
    # Rows past key 76 see every key (top-left causal): compare them as non-causal rows of a small q.
    ref_o, ref_l = oracle.attn(qr, _bits(k), _bits(v), 1 / math.sqrt(D), False)
    got_o = host_f64(o.reshape(-1, D)[torch.from_numpy(rows).to(DEV)])
    got_l = host_f64(l.reshape(-1)[torch.from_numpy(rows).to(DEV)])
    # Row 0 sees key 0 only: its output is v[0] (up to the bf16 rounding of
    # the output) and its LSE the one scaled logit.
    f64 = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    q0, k0, v0 = f64(_bits(q[:, :, :1])[0, 0, 0]), f64(_bits(k)[0, 0, 0]), f64(_bits(v)[0, 0, 0])
    assert np.max(np.abs(got_o[0] - v0)) <= 2.0 ** -8 * np.max(np.abs(v0))
    assert abs(got_l[0] - float(np.dot(q0, k0)) / math.sqrt(D)) <= 1e-3
    far = slice(2, None)
    rep = compare.attn_report(got_o[far], ref_o[0, 0, far], got_l[far], ref_l[0, 0, far])
    say(f"[limits] {rep}")
    compare.assert_ok(rep, "longest query slab")

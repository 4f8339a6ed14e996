"""attn_fwd_ws_fused_q: the query half of the prologue (per-head RMSNorm +
interleaved rotary) applied inside the attention's Q load.  It must give the
bits of qk_norm_rope on q followed by attn_fwd_ws, leave q untouched, and
agree with the oracle's attention of the prologue's output."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import compare
from attention_qk_norm_rope_amd import (attn_fwd_workspace_bytes, attn_fwd_ws, attn_fwd_ws_fused_q, inputs,
                                        qk_norm_rope)
from gpu_common import DEV, dev_bits, dev_f32, host_bits, host_f64, rows_of, say, workload

pytestmark = pytest.mark.gpu


def _run(q_bits, k_bits, v_bits, w_q, w_k, cos, sin, eps, scale, causal, out_dtype):
    B, H, Sq, D = q_bits.shape
    Skv = k_bits.shape[2]
    dq, dk, dv = dev_bits(q_bits), dev_bits(k_bits), dev_bits(v_bits)
    wq, wk = dev_f32(w_q), dev_f32(w_k)
    cq, sq = dev_f32(cos[:Sq]), dev_f32(sin[:Sq])
    ck, sk = dev_f32(cos[:Skv]), dev_f32(sin[:Skv])
    qk_norm_rope(None, dk, None, wk, ck, sk, eps)                  # keys normalised first
    ws = torch.full((attn_fwd_workspace_bytes(B, H, Skv, D),), 0x7E, dtype=torch.uint8, device=DEV)
    of, lf = attn_fwd_ws_fused_q(dq, dk, dv, ws, wq, cq, sq, eps, scale=scale, causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dq), q_bits), "q was modified"
    dq2 = dq.clone()
    qk_norm_rope(dq2, None, wq, None, cq, sq, eps)
    ou, lu = attn_fwd_ws(dq2, dk, dv, ws, scale=scale, causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(of, ou) and torch.equal(lf, lu), "fused and unfused results differ"
    return dq2, dk, of, lf


CASES = [  # B, H, Sq, Skv, D, causal, out dtype, grid
    (1, 3, 600, 700, 128, False, torch.bfloat16),
    (2, 2, 257, 300, 64, True, torch.float32),
    (1, 2, 1, 65, 128, False, torch.float32),
    (1, 10, 4000, 4000, 128, True, torch.bfloat16),   # causal, 160 tiles in one 8-wave launch
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}q{c[2]}k{c[3]}D{c[4]}{'c' if c[5] else 'n'}" for c in CASES])
def test_fused_q_small(case):
    B, H, Sq, Skv, D, causal, out_dtype = case
    seed = 1000 + Sq + Skv
    q = inputs.random_bits(seed, (B, H, Sq, D))
    k = inputs.random_bits(seed + 1, (B, H, Skv, D))
    v = inputs.random_bits(seed + 2, (B, H, Skv, D))
    rng = np.random.default_rng(seed)
    w_q = rng.uniform(0.5, 1.5, D).astype(np.float32)
    w_k = rng.uniform(0.5, 1.5, D).astype(np.float32)
    cos, sin = inputs.rope_tables(inputs.rope_positions(("line", max(Sq, Skv))), D)
    say(f"[fused_q] {case}")
    dq2, dk, o, l = _run(q, k, v, w_q, w_k, cos, sin, 1e-6, 1 / math.sqrt(D), causal, out_dtype)
    ref_o, ref_l = oracle.attn(host_bits(dq2), host_bits(dk), v, 1 / math.sqrt(D), causal)
    rep = compare.attn_report(host_f64(o), ref_o, host_f64(l), ref_l, bf16=out_dtype == torch.bfloat16)
    compare.assert_ok(rep, f"fused q {case}")


def test_fused_q_qwen_workload():
    """The Qwen-Image-shaped workload (B1 H24 S4312 D128, its RoPE grid and
    weights): fused equals unfused, and the oracle agrees on sampled rows."""
    cfg = inputs.WORKLOADS["qwen"]
    x = workload("qwen")
    cos, sin = inputs.config_rope_tables(cfg)
    say("[fused_q] qwen workload")
    dq2, dk, o, l = _run(x["q"], x["k"], x["v"], x["w_q"], x["w_k"], cos, sin, cfg.eps, cfg.scale, False,
                         torch.bfloat16)
    rows = inputs.sample_rows(cfg.index, cfg.B, cfg.H, cfg.Sq)
    ref_o, ref_l = oracle.attn(host_bits(dq2), host_bits(dk), x["v"], cfg.scale, False, rows=rows)
    rep = compare.attn_report(rows_of(o, rows), ref_o, rows_of(l, rows), ref_l)
    say(f"[fused_q] qwen workload: {rep}")
    compare.assert_ok(rep, "fused q qwen workload")

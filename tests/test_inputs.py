"""Host-side input generation: bf16 rounding, seeding, rotary tables, row samples."""
import numpy as np
import torch

from attention_qk_norm_rope_amd import inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, 1e-40], np.float32)])
    # ties: 1 + 2^-8 rounds to even (1.0); 1 + 3*2^-8 rounds up
    ours = inputs.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = inputs.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_times_four_is_exact():
    b = inputs.random_bits(1, (1000,))
    np.testing.assert_array_equal(inputs.bf16_bits_to_f32(inputs.times_four_bits(b)),
                                  inputs.bf16_bits_to_f32(b) * 4)


def test_seeded_inputs_are_deterministic():
    cfg = inputs.WORKLOADS["tiny"]
    a = inputs.make_inputs(cfg)
    b = inputs.make_inputs(cfg)
    for name in a:
        np.testing.assert_array_equal(a[name], b[name])
    assert a["q"].shape == (1, 2, 256, 64) and a["q"].dtype == np.uint16
    assert not np.array_equal(a["q"], a["k"])
    assert np.all((a["w_q"] >= 0.5) & (a["w_q"] <= 1.5))


def test_workload_table_shapes():
    c = inputs.WORKLOADS
    assert (c["qwen"].B, c["qwen"].H, c["qwen"].S, c["qwen"].D) == (1, 24, 4312, 128)
    assert (c["cosmos"].B, c["cosmos"].H, c["cosmos"].S, c["cosmos"].D) == (2, 16, 12480, 128)
    assert (c["wan"].B, c["wan"].H, c["wan"].S, c["wan"].D) == (1, 40, 75600, 128)
    assert (c["wan_sp"].Sq, c["wan_sp"].Skv, c["wan_sp"].chunks) == (18900, 75600, 4)
    assert abs(c["wan"].flops() - 1.17050e14) / 1.17e14 < 1e-3
    for i in ("tiny", "qwen", "cosmos", "wan"):
        assert inputs.rope_positions(c[i].grid).shape[0] == c[i].S


def test_rope_tables():
    pos = inputs.rope_positions(("video", 3, 4, 5))
    assert pos.shape == (60, 3)
    np.testing.assert_array_equal(pos[0], [0, 0, 0])
    np.testing.assert_array_equal(pos[-1], [2, 3, 4])
    np.testing.assert_array_equal(pos[5], [0, 1, 0])
    cos, sin = inputs.rope_tables(pos, 128)
    assert cos.shape == (60, 128) and cos.dtype == np.float32
    np.testing.assert_array_equal(cos[:, 0::2], cos[:, 1::2])
    np.testing.assert_array_equal(sin[:, 0::2], sin[:, 1::2])
    np.testing.assert_allclose(cos.astype(np.float64) ** 2 + sin.astype(np.float64) ** 2, 1.0, atol=2e-7)
    assert inputs.axis_pairs(128, 3) == (22, 21, 21)
    # position 0 on every axis is the identity rotation
    np.testing.assert_array_equal(cos[0], 1.0)
    np.testing.assert_array_equal(sin[0], 0.0)
    q = inputs.rope_positions(("qwen", 78, 52, 256))
    assert q.shape == (4312, 3)
    np.testing.assert_array_equal(q[4056], [0, 78, 78])


def test_sample_rows():
    rows = inputs.sample_rows(2, 1, 3, 300, per_head=64)
    assert rows.size == 3 * 64
    per = rows.reshape(3, 64) - (np.arange(3) * 300)[:, None]
    for r in per:
        assert len(set(r.tolist())) == 64
        assert {0, 31, 32, 127, 128, 255, 256, 299, 284}.issubset(set(r.tolist()))
        assert r.min() >= 0 and r.max() < 300
    np.testing.assert_array_equal(rows, inputs.sample_rows(2, 1, 3, 300, per_head=64))
    small = inputs.sample_rows(1, 1, 1, 10, per_head=64)
    np.testing.assert_array_equal(small, np.arange(10))
    # extra flat rows are added on top, once, in order; out-of-range ids are dropped
    more = inputs.sample_rows(2, 1, 3, 300, per_head=64, extra=[450, 450, 0, 10 ** 6])
    assert set(more.tolist()) == set(rows.tolist()) | {450}
    assert np.all(np.diff(more) > 0)

"""Pins for the fp64 RMSNorm + interleaved-rotary oracle (CPU only).

Checks: a row worked by hand; torch's float64 rms_norm (library) composed
with a complex-number rotation; closed forms (cos=1/sin=0 is a pure RMSNorm,
unit RMS, scale invariance, the constant-row formula with eps); an
asymmetric table that catches a swapped table index; pair norms; and the
relative-position property of the rotation.
"""
import json
import math
import os

import numpy as np
import torch

from attention_qk_norm_rope_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _x(seed, B, H, S, D, std=1.0):
    return inputs.random_bits(seed, (B, H, S, D), std=std)


def test_golden_row(oracle):
    g = json.load(open(os.path.join(GOLDEN, "prologue_pair.json")))
    x = inputs.to_bf16_bits(np.array(g["x"], dtype=np.float32))[None, None, None]
    cos = np.array([g["cos"]], dtype=np.float32)
    sin = np.array([g["sin"]], dtype=np.float32)
    out = oracle.qk_norm_rope(x, np.array(g["w"], np.float32), cos, sin, g["eps"])
    np.testing.assert_allclose(out[0, 0, 0] * math.sqrt(93), g["out_times_sqrt93"], rtol=0, atol=1e-13)


def test_matches_torch_rms_norm_and_complex_rotation(oracle):
    B, H, S, D = 2, 3, 29, 64
    x = _x(1, B, H, S, D, std=2.0)
    w = np.random.default_rng(2).uniform(0.5, 1.5, D).astype(np.float32)
    pos = inputs.rope_positions(("line", S))
    cos, sin = inputs.rope_tables(pos, D)
    eps = 1e-6
    out = oracle.qk_norm_rope(x, w, cos, sin, eps)
    xt = torch.from_numpy(inputs.bf16_bits_to_f64(x))
    y = torch.nn.functional.rms_norm(xt, (D,), weight=torch.from_numpy(w.astype(np.float64)), eps=eps)
    yc = torch.view_as_complex(y.reshape(B, H, S, D // 2, 2).contiguous())
    rot = torch.complex(torch.from_numpy(cos[:, 0::2].astype(np.float64)),
                        torch.from_numpy(sin[:, 0::2].astype(np.float64)))
    ref = torch.view_as_real(yc * rot).reshape(B, H, S, D).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_identity_rotation_is_unit_rms(oracle):
    B, H, S, D = 1, 2, 7, 128
    x = _x(3, B, H, S, D, std=5.0)
    w = np.ones(D, np.float32)
    one = np.ones((S, D), np.float32)
    zero = np.zeros((S, D), np.float32)
    y = oracle.qk_norm_rope(x, w, one, zero, 0.0)
    np.testing.assert_allclose(np.sqrt((y ** 2).mean(-1)), 1.0, rtol=0, atol=1e-14)
    # Same direction as x.
    xf = inputs.bf16_bits_to_f64(x)
    np.testing.assert_allclose(y * np.sqrt((xf ** 2).mean(-1, keepdims=True)), xf, rtol=1e-14, atol=1e-13)
    # Scaling x by a power of two (exact in bf16) leaves y unchanged.
    x8 = inputs.to_bf16_bits(inputs.bf16_bits_to_f32(x) * np.float32(8.0))
    np.testing.assert_allclose(oracle.qk_norm_rope(x8, w, one, zero, 0.0), y, rtol=0, atol=1e-14)


def test_constant_row_with_eps(oracle):
    D = 64
    x = np.full((1, 1, 1, D), inputs.to_bf16_bits(np.float32(0.5)), dtype=np.uint16)
    w = np.linspace(0.5, 1.5, D).astype(np.float32)
    eps = 0.75
    y = oracle.qk_norm_rope(x, w, np.ones((1, D), np.float32), np.zeros((1, D), np.float32), eps)
    expect = 0.5 / math.sqrt(0.25 + eps) * w.astype(np.float64)
    np.testing.assert_allclose(y[0, 0, 0], expect, rtol=0, atol=1e-15)
    # An all-zero row stays zero (no division by zero with eps > 0).
    z = oracle.qk_norm_rope(np.zeros((1, 1, 1, D), np.uint16), w, np.ones((1, D), np.float32),
                            np.zeros((1, D), np.float32), 1e-6)
    np.testing.assert_array_equal(z, 0.0)


def test_table_taken_elementwise(oracle):
    """Distinct values in the even and odd column of each pair pin the index
    of every table read: z_2i = y_2i c_2i - y_2i+1 s_2i, z_2i+1 = y_2i+1 c_2i+1 + y_2i s_2i+1."""
    S, D = 3, 16
    x = _x(4, 1, 1, S, D)
    rng = np.random.default_rng(5)
    cos = rng.uniform(-1, 1, (S, D)).astype(np.float32)
    sin = rng.uniform(-1, 1, (S, D)).astype(np.float32)
    w = np.ones(D, np.float32)
    y = oracle.qk_norm_rope(x, w, np.ones((S, D), np.float32), np.zeros((S, D), np.float32), 0.0)[0, 0]
    z = oracle.qk_norm_rope(x, w, cos, sin, 0.0)[0, 0]
    c, s = cos.astype(np.float64), sin.astype(np.float64)
    np.testing.assert_allclose(z[:, 0::2], y[:, 0::2] * c[:, 0::2] - y[:, 1::2] * s[:, 0::2], atol=1e-14)
    np.testing.assert_allclose(z[:, 1::2], y[:, 1::2] * c[:, 1::2] + y[:, 0::2] * s[:, 1::2], atol=1e-14)
    # Quarter turn: (a, b) -> (-b, a) exactly.
    q = oracle.qk_norm_rope(x, w, np.zeros((S, D), np.float32), np.ones((S, D), np.float32), 0.0)[0, 0]
    np.testing.assert_array_equal(q[:, 0::2], -y[:, 1::2])
    np.testing.assert_array_equal(q[:, 1::2], y[:, 0::2])


def test_rotation_preserves_pair_norms(oracle):
    B, H, S, D = 1, 2, 33, 128
    x = _x(6, B, H, S, D)
    w = np.random.default_rng(7).uniform(0.5, 1.5, D).astype(np.float32)
    cos, sin = inputs.rope_tables(inputs.rope_positions(("line", S)), D)
    y = oracle.qk_norm_rope(x, w, np.ones((S, D), np.float32), np.zeros((S, D), np.float32), 1e-6)
    z = oracle.qk_norm_rope(x, w, cos, sin, 1e-6)
    # cos/sin are fp32-rounded, so cos^2 + sin^2 = 1 only to ~1e-7.
    np.testing.assert_allclose(z[..., 0::2] ** 2 + z[..., 1::2] ** 2,
                               y[..., 0::2] ** 2 + y[..., 1::2] ** 2, rtol=3e-7, atol=1e-12)


def test_relative_position(oracle):
    """q at position m and k at position n: q.k depends on m - n only."""
    D = 64
    q = _x(8, 1, 1, 1, D)
    k = _x(9, 1, 1, 1, D)
    w = np.ones(D, np.float32)

    def at(x, p):
        cos, sin = inputs.rope_tables(np.array([[p]]), D)
        return oracle.qk_norm_rope(x, w, cos, sin, 0.0)[0, 0, 0]

    base = at(q, 5) @ at(k, 2)
    for shift in (1, 17, 250):
        np.testing.assert_allclose(at(q, 5 + shift) @ at(k, 2 + shift), base, rtol=0, atol=2e-5)
    assert abs(at(q, 6) @ at(k, 2) - base) > 1e-3

"""Pins of the oracle's variable-length attention (padded batches with
per-batch valid lengths, the actual_seq_lengths / actual_seq_lengths_kv of
the Wan2.2 page's fused attention call): full lengths are plain attention,
padding contents never matter, empty batches are zeros with LSE -inf, and a
batch equals the same data stored unpadded."""
import math

import numpy as np

import oracle
from attention_qk_norm_rope_amd import inputs


def _data(seed, B, H, Hkv, Sq, Skv, D):
    return (inputs.random_bits(seed, (B, H, Sq, D)), inputs.random_bits(seed + 1, (B, Hkv, Skv, D)),
            inputs.random_bits(seed + 2, (B, Hkv, Skv, D)))


def test_full_lengths_are_plain_attention():
    q, k, v = _data(1, 2, 2, 2, 9, 11, 16)
    o, l = oracle.attn_varlen(q, k, v, [9, 9], [11, 11], 0.25, False)
    ro, rl = oracle.attn(q, k, v, 0.25, False)
    assert np.array_equal(o, ro) and np.array_equal(l, rl)


def test_padding_contents_do_not_matter_and_padding_rows_are_empty():
    q, k, v = _data(2, 2, 2, 1, 8, 10, 16)
    lq, lk = [5, 8], [7, 3]
    o1, l1 = oracle.attn_varlen(q, k, v, lq, lk, 0.3, True)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[0, :, 5:] = 0x7FC0          # NaN patterns in the padding
    k2[0, :, 7:] = 0x7F80
    v2[1, :, 3:] = 0xFF80
    o2, l2 = oracle.attn_varlen(q2, k2, v2, lq, lk, 0.3, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.all(o1[0, :, 5:] == 0) and np.all(np.isneginf(l1[0, :, 5:]))
    assert np.all(np.isfinite(l1[0, :, :5]))


def test_batch_equals_unpadded_data():
    q, k, v = _data(3, 2, 4, 2, 12, 16, 8)
    lq, lk = [12, 6], [16, 9]
    o, l = oracle.attn_varlen(q, k, v, lq, lk, 1 / math.sqrt(8), False)
    b = 1
    kr = np.repeat(k[b:b + 1, :, :9], 2, axis=1)
    vr = np.repeat(v[b:b + 1, :, :9], 2, axis=1)
    ro, rl = oracle.attn(np.ascontiguousarray(q[b:b + 1, :, :6]), np.ascontiguousarray(kr), np.ascontiguousarray(vr),
                         1 / math.sqrt(8), False)
    assert np.array_equal(o[b:b + 1, :, :6], ro) and np.array_equal(l[b:b + 1, :, :6], rl)


def test_zero_lengths_and_clamping():
    q, k, v = _data(4, 3, 1, 1, 4, 4, 8)
    o, l = oracle.attn_varlen(q, k, v, [0, 4, 99], [4, 0, -3], 0.5, False)
    assert np.all(o == 0) and np.all(np.isneginf(l))      # every batch is empty after clamping
    o, l = oracle.attn_varlen(q, k, v, [99, 2, 4], [99, 4, 1], 0.5, False)
    ro, rl = oracle.attn(q, k, v, 0.5, False)
    assert np.array_equal(o[0], ro[0])                    # 99 clamps to the full length
    # one key: the output is that key's value row exactly
    vf = inputs.bf16_bits_to_f64(v)
    assert np.array_equal(o[2], np.broadcast_to(vf[2, :, :1], o[2].shape))

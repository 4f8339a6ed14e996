"""Pins of the oracle's BSND <-> BNSD head-slice layout (the local step on
either side of the Ulysses all-to-all): element-by-element loops on tiny
inputs, a hand-checked position, round trips, and the heads of a P-way split
reassembling the full transpose."""
import numpy as np
import pytest

import oracle


def _iota(shape):
    return np.arange(int(np.prod(shape)), dtype=np.uint16).reshape(shape)


def test_hand_checked_positions():
    # x[b, s, h, d] = ((b*S + s)*H + h)*D + d with B2 S3 H4 D8.
    x = _iota((2, 3, 4, 8))
    out = oracle.bsnd_to_bnsd(x, h0=1, heads=2)
    assert out.shape == (2, 2, 3, 8)
    # out[b=1, h=0, s=2, d=5] is x[1, 2, 1, 5] = ((1*3 + 2)*4 + 1)*8 + 5 = 173
    assert out[1, 0, 2, 5] == 173
    # out[0, 1, 0, 7] is x[0, 0, 2, 7] = 2*8 + 7 = 23
    assert out[0, 1, 0, 7] == 23


@pytest.mark.parametrize("shape,h0,heads", [((1, 5, 3, 8), 0, 3), ((2, 4, 6, 16), 2, 3), ((3, 2, 5, 8), 4, 1)])
def test_matches_loops(shape, h0, heads):
    rng = np.random.default_rng(sum(shape))
    x = rng.integers(0, 65536, size=shape, dtype=np.uint16)
    B, S, H, D = shape
    out = oracle.bsnd_to_bnsd(x, h0, heads)
    for b in range(B):
        for h in range(heads):
            for s in range(S):
                for d in range(D):
                    assert out[b, h, s, d] == x[b, s, h0 + h, d]
    y = rng.integers(0, 65536, size=shape, dtype=np.uint16)
    back = oracle.bnsd_to_bsnd(out, y, h0)
    for b in range(B):
        for s in range(S):
            for h in range(H):
                expect = x[b, s, h, :] if h0 <= h < h0 + heads else y[b, s, h, :]
                assert np.array_equal(back[b, s, h, :], expect)


def test_round_trip_and_split_reassembly():
    rng = np.random.default_rng(7)
    x = rng.integers(0, 65536, size=(2, 9, 8, 16), dtype=np.uint16)
    full = oracle.bsnd_to_bnsd(x)
    assert np.array_equal(full, x.transpose(0, 2, 1, 3))
    # 4-way head split (Ulysses P = 4): the slices tile the full BNSD tensor.
    parts = [oracle.bsnd_to_bnsd(x, 2 * r, 2) for r in range(4)]
    assert np.array_equal(np.concatenate(parts, axis=1), full)
    # Writing every slice back rebuilds x from anything.
    y = np.zeros_like(x)
    for r, p in enumerate(parts):
        y = oracle.bnsd_to_bsnd(p, y, 2 * r)
    assert np.array_equal(y, x)


def test_rejects_bad_slices():
    x = _iota((1, 2, 4, 8))
    with pytest.raises(ValueError):
        oracle.bsnd_to_bnsd(x, 3, 2)
    with pytest.raises(ValueError):
        oracle.bsnd_to_bnsd(x, -1, 1)

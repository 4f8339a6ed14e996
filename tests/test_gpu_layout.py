"""BSND <-> BNSD head-slice layout kernels on the GPU against the oracle's
numpy definition: bit-exact, other heads untouched, ragged sizes, D = 64 and
128 (and any multiple of 8), and one GPU's share of a 4-way Ulysses split at
the Wan2.2 shape."""
import numpy as np
import pytest
import torch

import oracle
from attention_qk_norm_rope_amd import bnsd_to_bsnd, bsnd_to_bnsd
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def _host(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("shape,h0,heads", [
    ((1, 75, 4, 128), 0, 4), ((2, 33, 6, 64), 2, 3), ((1, 1, 3, 128), 1, 1), ((3, 129, 5, 24), 4, 1),
])
def test_layout_matches_oracle(shape, h0, heads):
    rng = np.random.default_rng(sum(shape) + h0)
    x = rng.integers(0, 65536, size=shape, dtype=np.uint16)
    say(f"[layout] {shape} h0={h0} heads={heads}")
    out = bsnd_to_bnsd(_dev(x), h0, heads)
    torch.cuda.synchronize()
    assert np.array_equal(_host(out), oracle.bsnd_to_bnsd(x, h0, heads))
    o = rng.integers(0, 65536, size=out.shape, dtype=np.uint16)
    y = rng.integers(0, 65536, size=shape, dtype=np.uint16)
    dy = _dev(y)
    bnsd_to_bsnd(_dev(o), dy, h0)
    torch.cuda.synchronize()
    assert np.array_equal(_host(dy), oracle.bnsd_to_bsnd(o, y, h0))


def test_ulysses_share_wan_shape():
    """One rank of a 4-way Ulysses split at B1 S75600 H40 D128: its 10 heads
    out of the gathered sequence and back, compared on every element."""
    B, S, H, D, P = 1, 75600, 40, 128, 4
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    x = torch.randint(-32768, 32767, (B, S, H, D), dtype=torch.int16, device=DEV, generator=g).view(torch.bfloat16)
    for r in (0, P - 1):
        h0, hs = r * H // P, H // P
        say(f"[layout] Wan share rank {r}")
        out = bsnd_to_bnsd(x, h0, hs)
        ref = x[:, :, h0:h0 + hs, :].permute(0, 2, 1, 3).contiguous()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        y = torch.zeros_like(x)
        bnsd_to_bsnd(out, y, h0)
        assert torch.equal(y[:, :, h0:h0 + hs, :].view(torch.int16), x[:, :, h0:h0 + hs, :].view(torch.int16))
        assert int(y[:, :, :h0, :].view(torch.int16).abs().sum()) == 0
        assert int(y[:, :, h0 + hs:, :].view(torch.int16).abs().sum()) == 0
        torch.cuda.synchronize()

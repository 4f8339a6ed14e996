"""The C ABI on the GPU: the in-tree library is the one loaded, it shares
torch's HIP runtime, and bad arguments on real buffers return their status
codes without launching."""
import ctypes
import os

import pytest
import torch

import attention_qk_norm_rope_amd as pkg
from attention_qk_norm_rope_amd import binding

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_is_in_tree_and_single_hip_runtime():
    path = pkg.library_path()
    assert os.path.realpath(path).startswith(os.path.realpath(ROOT))
    assert "gfx950" in pkg.version()
    maps = open("/proc/self/maps").read()
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len({os.path.realpath(p) for p in hip}) == 1, hip
    assert os.path.realpath(path) in {os.path.realpath(l.split()[-1]) for l in maps.splitlines() if l.strip()}


def test_status_codes_with_real_buffers():
    lib = binding._load()
    q = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    out = torch.empty_like(q)
    lse = torch.empty(1, 2, 64, dtype=torch.float32, device="cuda")
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)  # noqa: E731
    s = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)  # noqa: E731
    assert lib.attn_fwd(P(q), P(k), P(v), P(out), P(lse), 1, 2, 64, 64, 128, 0.1, 0, 0, s()) == 0
    assert lib.attn_fwd(P(q), P(k), P(v), P(q), P(lse), 1, 2, 64, 64, 128, 0.1, 0, 0, s()) == 5
    assert lib.attn_fwd(P(q), P(k), P(v), P(out, 2), P(lse), 1, 2, 64, 64, 128, 0.1, 0, 0, s()) == 4
    assert lib.attn_fwd(P(q), P(k), P(v), P(out), P(lse), 1, 2, 64, 64, 96, 0.1, 0, 0, s()) == 3
    assert lib.attn_fwd(P(q), P(k), P(v), P(out), P(lse), 1, 2, 0, 64, 128, 0.1, 0, 0, s()) == 2
    assert lib.attn_fwd(None, P(k), P(v), P(out), P(lse), 1, 2, 64, 64, 128, 0.1, 0, 0, s()) == 1
    assert lib.attn_merge(P(out), P(lse), P(out), P(lse), 1, 2, 64, 128, 0, 0, s()) == 5
    torch.cuda.synchronize()
    with pytest.raises(binding.DitAttnError) as e:
        pkg.attn_fwd(q, k, v, out=q)
    assert e.value.status == 5


def test_binding_rejects_bad_tensors():
    q = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):
        pkg.attn_fwd(q.float(), q, q)
    with pytest.raises(ValueError):
        pkg.attn_fwd(q.transpose(2, 3).contiguous().transpose(2, 3), q, q)
    with pytest.raises(ValueError):
        pkg.qk_norm_rope(None, None, None, None, None, None, 1e-6)

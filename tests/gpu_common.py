"""Shared helpers of the GPU tests: host<->device copies of bf16 bit patterns
and a per-session cache of the large seeded workloads."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

from attention_qk_norm_rope_amd import inputs

DEV = "cuda:0"


def say(msg: str):
    """Progress line, flushed before a GPU step so a lost box still names it."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bits(bits: np.ndarray) -> torch.Tensor:
    b = np.ascontiguousarray(bits)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV)


def dev_f32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32))).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rows_of(t: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    """Gather flat rows of a [B,H,S,D] (or [B,H,S]) device tensor to fp64 host."""
    idx = torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(t.device)
    if t.dim() == 4:
        return host_f64(t.reshape(-1, t.shape[-1]).index_select(0, idx))
    return host_f64(t.reshape(-1).index_select(0, idx))


@functools.lru_cache(maxsize=2)
def workload(name: str) -> dict:
    """Host inputs of a config (cached for the session)."""
    say(f"[inputs] generating workload {name}")
    return inputs.make_inputs(inputs.WORKLOADS[name])


def launch_edge_rows(B: int, H: int, Sq: int, cus: int = 256) -> list:
    """Flat query rows of the tiles that the workspace path's second dispatch
    takes when the last round of 256-row tiles is partly filled (4-wave
    halves or the split launch): the rows either side of the first such
    tile's start and middle, the first and last row of every such tile, and
    every 17th row of the first and the last of them."""
    bm = 256
    nq = (Sq + bm - 1) // bm
    blk = nq * B * H
    tail = blk % cus
    rows = set()
    for t in range(blk - tail, blk):
        bh, qt = divmod(t, nq)
        lo, hi = qt * bm, min(Sq, qt * bm + bm)
        picks = [lo, hi - 1]
        if t == blk - tail:
            picks += [lo - 1, lo + bm // 2 - 1, lo + bm // 2]
        if t in (blk - tail, blk - 1):
            picks += list(range(lo, hi, 17))
        rows.update(bh * Sq + r for r in picks if 0 <= r < Sq)
    return sorted(rows)

"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module only *generates inputs*: random tensors, their bf16 bit patterns,
rotary cos/sin tables and row samples.  It holds none of the attention,
normalisation, rotation or merge arithmetic, so neither side of a parity test
borrows the other's maths through it.

The workloads stand in for the models the pages run (Qwen-Image, Cosmos
Predict2.5, Wan2.2), whose weights and data are not available: N(0,1)
tensors in the models' attention shapes.

Recipe (every config): ``numpy.random.SeedSequence(seed).spawn(3*B*H + 1)``
gives one PCG64 stream per [S, D] slab -- stream t*B*H + b*H + h fills slab
(b, h) of tensor t (q = 0, k = 1, v = 2) with ``standard_normal(dtype=float32)``
in C order -- and the last stream draws w_q then w_k ~ U(0.5, 1.5) as float32
[D].  q, k, v are rounded to bf16 (round to nearest even) once.  Independent
streams let the slabs be filled in parallel with a result that does not
depend on the thread count.  The seed is the workload number; the Wan2.2 SP share (5) reuses
the Wan2.2 workload's (4) tensors.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os

import numpy as np


# --------------------------------------------------------------------------
# bf16 bit patterns

def to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    f = np.array(x, dtype=np.float32, copy=True, order="C")
    nan = np.isnan(f)
    u = f.view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    bits = u.astype(np.uint16)
    if nan.any():
        bits[nan] = np.uint16(0x7FC0)
    return bits


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def times_four_bits(bits) -> np.ndarray:
    """bf16 bits of 4*x (exact for every finite x in the generated range)."""
    return to_bf16_bits(bf16_bits_to_f32(bits) * np.float32(4.0))


# --------------------------------------------------------------------------
# Workload table

@dataclasses.dataclass(frozen=True)
class Config:
    index: int                 # workload number: seeds the inputs and the sampled rows
    name: str
    B: int
    H: int
    S: int
    D: int
    seed: int
    eps: float | None          # prologue epsilon (None: no prologue in this config)
    grid: tuple | None         # rotary position grid, see rope_positions()
    sq: int | None = None      # query rows when different from S (the SP share)
    chunks: int = 1            # KV chunks merged with attn_merge

    @property
    def Sq(self) -> int:
        return self.sq if self.sq is not None else self.S

    @property
    def Skv(self) -> int:
        return self.S

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def flops(self, causal: bool = False) -> float:
        f = 4.0 * self.B * self.H * self.Sq * self.Skv * self.D
        return f / 2 if causal else f


WORKLOADS = {
    "tiny": Config(1, "tiny B1 H2 S256 D64", 1, 2, 256, 64, 1, 1e-6, ("line", 256), chunks=2),
    "qwen": Config(2, "Qwen-Image joint B1 H24 S4312 D128", 1, 24, 4312, 128, 2, 1e-6, ("qwen", 78, 52, 256)),
    "cosmos": Config(3, "Cosmos-Predict video B2 H16 S12480 D128", 2, 16, 12480, 128, 3, 1e-6, ("video", 8, 30, 52)),
    "wan": Config(4, "Wan2.2 long video B1 H40 S75600 D128", 1, 40, 75600, 128, 4, 1e-5, ("video", 21, 45, 80)),
    "wan_sp": Config(5, "Wan2.2 4-way SP share Sq18900 Skv75600 H40 D128", 1, 40, 75600, 128, 4, None, None,
              sq=18900, chunks=4),
}


# --------------------------------------------------------------------------
# Random tensors

def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(cfg: Config) -> dict:
    """q, k, v (bf16 bits, [B,H,S,D]) and w_q, w_k (fp32 [D]) for a config.

    For the SP share (5) the returned q is the Wan2.2 workload's q restricted to rows [0, Sq).
    """
    B, H, S, D = cfg.B, cfg.H, cfg.S, cfg.D
    streams = np.random.SeedSequence(cfg.seed).spawn(3 * B * H + 1)
    tensors = [np.empty((B, H, S, D), dtype=np.uint16) for _ in range(3)]

    def fill(job):
        t, bh = job
        rng = np.random.default_rng(streams[t * B * H + bh])
        tensors[t][bh // H, bh % H] = to_bf16_bits(rng.standard_normal((S, D), dtype=np.float32))

    jobs = [(t, bh) for t in range(3) for bh in range(B * H)]
    with concurrent.futures.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, jobs))
    wrng = np.random.default_rng(streams[-1])
    w_q = wrng.uniform(0.5, 1.5, size=D).astype(np.float32)
    w_k = wrng.uniform(0.5, 1.5, size=D).astype(np.float32)
    q, k, v = tensors
    if cfg.sq is not None:
        q = np.ascontiguousarray(q[:, :, : cfg.sq])
    return {"q": q, "k": k, "v": v, "w_q": w_q, "w_k": w_k}


def random_bits(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """Small seeded N(0, std^2) bf16 tensor (tests of arbitrary shapes)."""
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def split_kv(k: np.ndarray, n: int) -> list:
    """Split [B,H,S,D] along S into n contiguous chunk tensors (ring buffers)."""
    S = k.shape[2]
    bounds = [round(i * S / n) for i in range(n + 1)]
    return [np.ascontiguousarray(k[:, :, bounds[i]:bounds[i + 1]]) for i in range(n)]


# --------------------------------------------------------------------------
# Rotary tables (inputs to the prologue; the kernel is table-agnostic)

def axis_pairs(D: int, n_axes: int) -> tuple:
    """Split D/2 rotary pairs over the axes: (t, h, w) = (c - 2*(c//3), c//3, c//3)."""
    c = D // 2
    if n_axes == 1:
        return (c,)
    return (c - 2 * (c // 3), c // 3, c // 3)


def rope_positions(grid) -> np.ndarray:
    """Integer positions [S, n_axes] for a position grid spec.

    ("line", S)        -> one axis, 0..S-1
    ("video", F, Hh, W) -> (t, h, w), t-major over an F x Hh x W latent grid
    ("qwen", Hh, W, T)  -> image tokens (0, r, c) for the Hh x W grid, then T
                           text tokens at (0, Hh + j, Hh + j)
    """
    kind = grid[0]
    if kind == "line":
        return np.arange(grid[1], dtype=np.int64)[:, None]
    if kind == "video":
        F, Hh, W = grid[1:]
        t, h, w = np.meshgrid(np.arange(F), np.arange(Hh), np.arange(W), indexing="ij")
        return np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1).astype(np.int64)
    if kind == "qwen":
        Hh, W, T = grid[1:]
        r, c = np.meshgrid(np.arange(Hh), np.arange(W), indexing="ij")
        img = np.stack([np.zeros(Hh * W, dtype=np.int64), r.ravel(), c.ravel()], axis=1)
        j = np.arange(T)
        txt = np.stack([np.zeros(T, dtype=np.int64), Hh + j, Hh + j], axis=1)
        return np.concatenate([img, txt], axis=0).astype(np.int64)
    raise ValueError(f"unknown grid {grid!r}")


def rope_tables(positions: np.ndarray, D: int, theta: float = 10000.0):
    """Pair-duplicated cos/sin tables, fp32 [S, D].

    Axis a with n_a pairs gives pair j the angle pos_a * theta**(-j / n_a);
    the pairs of the axes are laid side by side in axis order, and each angle
    fills both columns 2p and 2p+1 of its pair p.
    """
    positions = np.asarray(positions, dtype=np.int64)
    S, n_axes = positions.shape
    pairs = axis_pairs(D, n_axes)
    angles = []
    for a, n in enumerate(pairs):
        freq = theta ** (-np.arange(n, dtype=np.float64) / n)
        angles.append(positions[:, a:a + 1].astype(np.float64) * freq[None, :])
    ang = np.concatenate(angles, axis=1)                # [S, D/2]
    ang = np.repeat(ang, 2, axis=1)                     # [S, D]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def config_rope_tables(cfg: Config):
    if cfg.grid is None:
        raise ValueError(f"workload {cfg.name} has no prologue")
    pos = rope_positions(cfg.grid)
    if pos.shape[0] != cfg.S:
        raise ValueError("grid size does not match S")
    return rope_tables(pos, cfg.D)


# --------------------------------------------------------------------------
# Query-row sample for the oracle at large sizes

def sample_rows(cfg_index: int, B: int, H: int, Sq: int, per_head: int = 64, extra=()) -> np.ndarray:
    """Flat query-row ids ((b*H + h)*Sq + i) the oracle evaluates.

    Per (b, h): rows 0, 31, 32, 127, 128, 255, 256 (edges of 32-, 128- and
    256-row query blocks), the last 16 rows (the ragged tail) and Sq - 1,
    topped up to ``per_head`` distinct rows drawn uniformly from
    ``default_rng(100 + cfg_index)``.  ``extra`` flat row ids are added on
    top (sorted, without duplicates).
    """
    rng = np.random.default_rng(100 + cfg_index)
    rows = []
    fixed = sorted({i for i in [0, 31, 32, 127, 128, 255, 256, Sq - 1] + list(range(max(0, Sq - 16), Sq))
                    if 0 <= i < Sq})
    for bh in range(B * H):
        chosen = set(fixed)
        want = min(per_head, Sq)
        while len(chosen) < want:
            chosen.update(int(x) for x in rng.integers(0, Sq, size=want - len(chosen)))
        sel = sorted(chosen)[:want] if len(chosen) > want else sorted(chosen)
        rows.extend(bh * Sq + i for i in sel)
    if len(extra):
        ex = [int(r) for r in extra if 0 <= int(r) < B * H * Sq]
        rows = sorted(set(rows) | set(ex))
    return np.asarray(rows, dtype=np.int64)

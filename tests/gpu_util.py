"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
library through its binding, and compare with the oracle on the CPU."""
from __future__ import annotations

import sys
from typing import List, Sequence, Tuple

import numpy as np

import oracle as O


def torch():
    import torch as t
    return t


def device():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    return t.device("cuda:0")


def banner(msg: str):
    """Name the case before a GPU step, flushed, so a fault can be traced to it."""
    sys.stdout.write(f"[gpu] {msg}\n")
    sys.stdout.flush()


def member_to_device(m):
    """synth.BlockFP8Member -> (uint8 weight, bfloat16 scale grid) on the GPU."""
    t = torch()
    d = device()
    w = t.from_numpy(np.ascontiguousarray(m.codes)).to(d)
    s = t.from_numpy(np.ascontiguousarray(m.scale_bits).view(np.int16)).to(d).view(t.bfloat16)
    return w, s


def raw_member_to_device(codes: np.ndarray, scale: np.ndarray):
    """(uint8 codes, float32 grid) -> device tensors (grid kept as float32)."""
    t = torch()
    d = device()
    return (t.from_numpy(np.ascontiguousarray(codes, np.uint8)).to(d),
            t.from_numpy(np.ascontiguousarray(scale, np.float32)).to(d))


def oracle_members(members) -> List[Tuple[np.ndarray, np.ndarray]]:
    return [(m.codes, m.scale_f32()) for m in members]


def to_np(y) -> np.ndarray:
    """Device output -> float32 numpy (BF16 widened exactly)."""
    t = torch()
    if y.dtype == t.bfloat16:
        return O.bf16_bits_to_f32(y.view(t.int16).cpu().numpy().view(np.uint16))
    return y.float().cpu().numpy()


def assert_within(y_gpu: np.ndarray, y_ref: np.ndarray, abs_sum: np.ndarray, bf16: bool, what: str):
    ok, worst = O.within_bound(y_gpu, y_ref, abs_sum, bf16_out=bf16)
    assert ok, f"{what}: worst err/bound = {worst:.3g}"
    return worst


def sample_rows(n_total: int, members_rows: Sequence[int], k: int, seed: int = 0) -> List[int]:
    """Output rows to check at full size: every member's first/last rows, its
    128-row block edges near the ends, plus random rows."""
    g = np.random.default_rng(seed)
    rows = set()
    r0 = 0
    for n in members_rows:
        for d in (0, 1, 127, 128, 129, n - 129, n - 128, n - 1):
            if 0 <= d < n:
                rows.add(r0 + d)
        r0 += n
    rows.update(int(v) for v in g.integers(0, n_total, k))
    return sorted(rows)

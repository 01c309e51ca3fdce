"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
library through its binding, and compare with the oracle on the CPU."""
from __future__ import annotations

import hashlib
import json
import os
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
    record(what, ok, kind="bound", oracle_sha256=_sha(y_ref), shape=list(np.shape(y_ref)), worst_err_over_bound=worst,
           bf16_out=bool(bf16))
    assert ok, f"{what}: worst err/bound = {worst:.3g}"
    return worst


TILE = 256   # the widest tile any kernel takes over rows or tokens


def sample_rows(n_total: int, members_rows: Sequence[int], k: int, seed: int = 0) -> List[int]:
    """Output rows to check at full size: every member's first/last rows and its
    128-row block edges near the ends, one random row inside every 256-row tile
    of every member (tiles start at each member's row 0, as the kernels lay
    them out), plus ``k`` random rows."""
    g = np.random.default_rng(seed)
    rows = set()
    r0 = 0
    for n in members_rows:
        for d in (0, 1, 127, 128, 129, n - 129, n - 128, n - 1):
            if 0 <= d < n:
                rows.add(r0 + d)
        for t0 in range(0, n, TILE):
            rows.add(r0 + int(g.integers(t0, min(n, t0 + TILE))))
        r0 += n
    rows.update(int(v) for v in g.integers(0, n_total, k))
    return sorted(rows)


def sample_tokens(M: int, k: int = 48, seed: int = 1) -> np.ndarray:
    """Tokens to check: all of them up to 64, else the first and last 8, one
    random token inside every 256-token tile, and ``k`` random ones."""
    if M <= 64:
        return np.arange(M)
    g = np.random.default_rng(seed)
    per_tile = [int(g.integers(t0, min(M, t0 + TILE))) for t0 in range(0, M, TILE)]
    return np.unique(np.concatenate([np.arange(8), np.arange(M - 8, M), per_tile, g.integers(0, M, k)]))


# ------------------------------------------------------------ result records
# Each comparison with the oracle appends one record (test, what was compared,
# sha256 of the fixture's arrays and of the oracle's output, worst err/bound,
# the library's sha256) to parity_records.jsonl in the repository's output
# folder for GPU runs, so the fixture hashes are kept next to the GPU results
# they produced.

_FIXTURE: dict = {}
RECORDS = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out",
                       "parity_records.jsonl")


def _sha(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


def note_fixture(**arrays):
    """Remember the current test's input arrays (weights, scales, activations) for its records."""
    for k, v in arrays.items():
        _FIXTURE[k] = _sha(v)


def clear_fixture():
    _FIXTURE.clear()


_LIB_SHA = None


def _lib_sha() -> str:
    global _LIB_SHA
    if _LIB_SHA is None:
        import block_scaled_fp8_linear_amd as B
        try:
            with open(B.LIB_PATH, "rb") as f:
                _LIB_SHA = hashlib.sha256(f.read()).hexdigest()[:16]
        except OSError:
            _LIB_SHA = "missing"
    return _LIB_SHA


def record(what: str, ok: bool, **fields):
    entry = dict(test=os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], what=what, ok=bool(ok),
                 fixture=dict(_FIXTURE), lib_sha256=_lib_sha())
    entry.update(fields)
    try:
        os.makedirs(os.path.dirname(RECORDS), exist_ok=True)
        with open(RECORDS, "a") as f:
            f.write(json.dumps(entry) + "\n")
    except OSError:
        pass

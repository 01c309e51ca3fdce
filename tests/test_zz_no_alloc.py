"""The no-allocation W8A8 entry point against the one that takes a workspace.

bsf8_linear_w8a8_noalloc runs the same kernels as bsf8_linear_w8a8 but keeps
its split-K partial tiles in the library's fixed per-device scratch array.
Two calls in a row (the second smaller) must give outputs identical to the
workspace entry point's and within the oracle's bound; a call that would need
more partials than the scratch holds is refused before anything runs.
Calls go through the C ABI (ctypes) directly.
"""
import ctypes

import numpy as np
import pytest

import block_scaled_fp8_linear_amd as B
import oracle as O
import synth
from gpu_util import assert_within, banner, device, member_to_device, oracle_members, sample_rows, sample_tokens, torch

pytestmark = pytest.mark.gpu


def _noalloc(w, xq, xs, y):
    L = B.lib()
    return L.bsf8_linear_w8a8_noalloc(w.handle, xq.data_ptr(), xq.stride(0), xs.data_ptr(), xs.stride(0),
                                      xs.stride(1), xq.shape[0], y.data_ptr(), B._dt_of(y), y.stride(0),
                                      B._stream_ptr(xq.device))


CASES = [
    # (name, member rows, K, M): the first needs 63 MB of split-K partials (3 ranges of the
    # [1024, 5120] F32 tile set), the second is smaller and splits too
    ("ffn_down_m1024", (5120,), 17408, 1024),
    ("split_k_512_k8192_m64", (512,), 8192, 64),
]


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    t = torch()
    for name, rows, K, M in CASES:
        ms = [synth.random_code_weight(223, f"noalloc_W{i}_{name}", r, K) for i, r in enumerate(rows)]
        w = B.BlockFP8Weight([member_to_device(m) for m in ms])
        need = w.workspace_size(B.ARM_W8A8, M)
        assert 0 < need <= B.NOALLOC_SCRATCH_BYTES, (name, need)
        x = synth.gaussian_activations(223, f"noalloc_X_{name}", M, K)
        xq, xs = B.quant_act(t.from_numpy(x).to(device()))
        banner(f"noalloc {name}: {w.describe(B.ARM_W8A8, M)} workspace={need}")
        for odt in (t.bfloat16, t.float32):
            y_ref = B.linear_w8a8(w, xq, xs, out_dtype=odt)
            y = t.full((M, w.n_total), 3.0, dtype=odt, device=device())
            st = _noalloc(w, xq, xs, y)
            assert st == 0, (B.status_name(st), B.lib().bsf8_last_error().decode())
            t.cuda.synchronize()
            assert t.equal(y.view(t.int16) if odt == t.bfloat16 else y.view(t.int32),
                           y_ref.view(t.int16) if odt == t.bfloat16 else y_ref.view(t.int32)), (name, odt)
        om = oracle_members(ms)
        q_ref, s_ref = O.quant_act(x)
        rs = sample_rows(w.n_total, list(rows), 32)
        tok = sample_tokens(M)
        yn = y.cpu().numpy()[np.ix_(tok, rs)]
        assert_within(yn, O.linear_w8a8_rows(q_ref[tok], s_ref[tok], om, rs),
                      O.abs_bound_w8a8_rows(q_ref[tok], s_ref[tok], om, rs), False, f"noalloc {name}")
        del w


def test_noalloc_refuses_calls_beyond_its_scratch():
    """A call whose split-K partials exceed the scratch is refused (WORKSPACE) and writes nothing."""
    t = torch()
    N, K, M = 10240, 16384, 1024   # 40 row tiles x 4 token tiles, split 3 ways: 126 MB of partials
    wq = t.zeros((N, K), dtype=t.uint8, device=device())
    sc = t.ones((N // 128, K // 128), dtype=t.bfloat16, device=device())
    w = B.BlockFP8Weight([(wq, sc)])
    need = w.workspace_size(B.ARM_W8A8, M)
    assert need > B.NOALLOC_SCRATCH_BYTES, need
    xq = t.zeros((M, K), dtype=t.uint8, device=device())
    xs = B.scales_kmajor(M, K // 128, device())
    xs.fill_(1.0)
    y = t.full((M, N), 5.0, dtype=t.bfloat16, device=device())
    banner(f"noalloc refusal: needs {need} bytes")
    st = _noalloc(w, xq, xs, y)
    assert B.status_name(st) == "WORKSPACE", B.status_name(st)
    t.cuda.synchronize()
    assert bool((y == 5.0).all())

"""The largest K the streaming and staged kernels take, and the first K past it.

"Qwen checkpoints with block FP8 weights", block-path paragraph: the operator is the
same for every projection, whatever its K.  The kernels stage one row of the scale
grid (or a wave's chunk scales) on chip, which caps K at 1024 blocks of 128
(131072): a wave of the streaming kernels then holds 128 chunk scales, the most its
two scale registers per lane take, and the W8A8 fast GEMM stages 1024 weight
scales per grid row.  Here K = 131072 runs every kernel family at that edge
(one-token ring, few-token kernel with one to three MFMA passes, general W8A16
kernel, W8A8 few-token kernel and fast GEMM, the dynamic call falling back to its
workspace because 128 chunks per wave exceed the in-kernel quantizer's 64), and
K = 131200 (1025 blocks) is refused by the W8A16 arm by name while the W8A8 arm
takes its byte-wise GEMM.  Grouped members of 40 and 24 rows keep the oracle
quick; every output is compared with the oracle within its bound.
"""
import numpy as np
import pytest

import block_scaled_fp8_linear_amd as B
import oracle as O
import synth
from gpu_util import assert_within, banner, device, member_to_device, note_fixture, oracle_members, to_np, torch

pytestmark = pytest.mark.gpu

SEED = 337
K_MAX = 131072


def _weight(K):
    members = [synth.random_code_weight(SEED, f"maxk_W{K}_{i}", r, K) for i, r in enumerate((40, 24))]
    note_fixture(**{f"codes{i}": m.codes for i, m in enumerate(members)},
                 **{f"scale{i}": m.scale_bits for i, m in enumerate(members)})
    return members, B.BlockFP8Weight([member_to_device(m) for m in members])


def _x(K, M):
    return synth.gaussian_activations(SEED, f"maxk_X{K}", 56, K)[:M]


@pytest.mark.parametrize("M,xdt,kernel", [(1, "f32", "w8a16_m1_ring"), (3, "f32", "w8a16_small_m"),
                                          (16, "f32", "w8a16_small_m"), (16, "bf16", "w8a16_small_m"),
                                          (40, "f32", "")])
def test_w8a16_at_the_largest_k(M, xdt, kernel):
    t = torch()
    members, w = _weight(K_MAX)
    om = oracle_members(members)
    x = _x(K_MAX, M)
    if xdt == "bf16":
        x = O.f32_to_bf16(x).astype(np.float32)
    d = w.describe(B.ARM_W8A16, M)
    banner(f"w8a16 K={K_MAX} M={M} x={xdt}: {d}")
    assert kernel in d, d
    xd = t.from_numpy(x).to(device())
    if xdt == "bf16":
        xd = xd.to(t.bfloat16)
    ref, bound = O.linear_w8a16(x, om), O.abs_bound_w8a16(x, om)
    for odt in (t.float32, t.bfloat16):
        y = to_np(B.linear_w8a16(w, xd, out_dtype=odt))
        assert_within(y, ref, bound, odt == t.bfloat16, f"w8a16 K={K_MAX} M={M} {xdt}")


@pytest.mark.parametrize("M,kernel", [(1, "w8a16_m1_ring<e4m3>"), (48, "w8a16_small_m<e4m3>"), (56, "w8a8_gemm_fast")])
def test_w8a8_at_the_largest_k(M, kernel):
    t = torch()
    members, w = _weight(K_MAX)
    om = oracle_members(members)
    x = _x(K_MAX, M)
    xq, xs = O.quant_act(x)
    d = w.describe(B.ARM_W8A8, M)
    banner(f"w8a8 K={K_MAX} M={M}: {d}")
    assert kernel in d, d
    ref, bound = O.linear_w8a8(xq, xs, om), O.abs_bound_w8a8(xq, xs, om)
    for odt in (t.float32, t.bfloat16):
        y = to_np(B.linear_w8a8(w, t.from_numpy(xq).to(device()), t.from_numpy(xs).to(device()), out_dtype=odt))
        assert_within(y, ref, bound, odt == t.bfloat16, f"w8a8 K={K_MAX} M={M}")


def test_dynamic_at_the_largest_k_takes_the_workspace():
    """One token at K = 131072: 128 chunks per wave, beyond what a wave quantizes
    into LDS, so the call quantizes into its workspace; bits equal the two calls."""
    t = torch()
    members, w = _weight(K_MAX)
    x = _x(K_MAX, 1)
    d = w.describe(B.ARM_W8A8_DYNAMIC, 1)
    banner(f"w8a8 dynamic K={K_MAX} M=1: {d}")
    assert "quant_act into the workspace" in d, d
    xd = t.from_numpy(x).to(device())
    y = B.linear_w8a8_dynamic(w, xd, out_dtype=t.float32)
    xq, xs = B.quant_act(xd)
    y2 = B.linear_w8a8(w, xq, xs, out_dtype=t.float32)
    t.cuda.synchronize()
    assert np.array_equal(y.view(t.int32).cpu().numpy(), y2.view(t.int32).cpu().numpy())
    q_ref, s_ref = O.quant_act(x)
    assert np.array_equal(to_np(xq.view(t.uint8)), q_ref) and np.array_equal(to_np(xs), s_ref)


def test_one_block_past_the_largest_k():
    """K = 131200 (1025 blocks): the W8A16 arm refuses it as unsupported; the W8A8 arm
    runs its byte-wise GEMM at one and at 40 tokens."""
    t = torch()
    K = K_MAX + 128
    members, w = _weight(K)
    om = oracle_members(members)
    x = _x(K, 40)
    with pytest.raises(B.BSF8Error, match="UNSUPPORTED"):
        B.linear_w8a16(w, t.from_numpy(x[:1]).to(device()))
    for M in (1, 40):
        d = w.describe(B.ARM_W8A8, M)
        banner(f"w8a8 K={K} M={M}: {d}")
        assert "kernel=w8a8_gemm " in d, d
        xq, xs = O.quant_act(x[:M])
        y = to_np(B.linear_w8a8(w, t.from_numpy(xq).to(device()), t.from_numpy(xs).to(device()),
                                out_dtype=t.float32))
        assert_within(y, O.linear_w8a8(xq, xs, om), O.abs_bound_w8a8(xq, xs, om), False, f"w8a8 K={K} M={M}")

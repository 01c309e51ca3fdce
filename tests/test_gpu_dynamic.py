"""W8A8 with the activations quantized in the same call (bsf8_linear_w8a8_dynamic).

"Module w8a8_prefill", section WHY: activations are quantized per token in 1x128
groups and the FP8 product consumes them.  The dynamic call must give the bits
of bsf8_quant_act followed by bsf8_linear_w8a8 on every path:
* one aligned token is quantized inside the one-token kernels (each wave its K
  range, into LDS; also in their load-ring form for a long K), with F32 or BF16
  activations;
* anything else (more tokens, a K or row pitch that is not 16-byte aligned)
  quantizes into the workspace and runs the W8A8 kernels on it.
Each case is also checked against the oracle (the oracle's quantizer, then its
W8A8 product) within the W8A8 bound.
"""
import numpy as np
import pytest

import block_scaled_fp8_linear_amd as B
import oracle as O
import synth
from gpu_util import assert_within, banner, device, member_to_device, note_fixture, oracle_members, to_np, torch

pytestmark = pytest.mark.gpu

SEED = 311


def _case(name):
    if name == "k1024_640rows":
        return [synth.gaussian_weight(SEED, "d_W1024", 640, 1024)], 1024
    if name == "ragged_k4000":
        return [synth.random_code_weight(SEED, "d_W4000", 300, 4000)], 4000
    if name == "k200_unaligned":
        return [synth.random_code_weight(SEED, "d_W200", 130, 200)], 200
    if name == "grouped_384_136_136":
        return [synth.gaussian_weight(SEED, f"d_qkv{i}", r, 384) for i, r in enumerate([384, 136, 136])], 384
    if name == "long_k17408_ring":
        return [synth.random_code_weight(SEED, "d_W17408", 72, 17408)], 17408
    if name == "long_k40960_ring":   # 40 chunks per wave: two batches of quantization rounds
        return [synth.random_code_weight(SEED, "d_W40960", 40, 40960)], 40960
    if name == "decode_5120":
        return [synth.gaussian_weight(SEED, "d_W5120", 5120, 5120)], 5120
    raise KeyError(name)


# (case, M, x dtype, expected path): "fused" = quantized inside a streaming kernel
CASES = [
    ("k1024_640rows", 1, "f32", "fused"), ("k1024_640rows", 1, "bf16", "fused"),
    ("k1024_640rows", 2, "f32", "two-step"), ("k1024_640rows", 4, "bf16", "two-step"),
    ("k1024_640rows", 5, "f32", "two-step"), ("k1024_640rows", 64, "bf16", "two-step"),
    ("ragged_k4000", 1, "bf16", "fused"), ("ragged_k4000", 1, "f32", "fused"), ("ragged_k4000", 3, "f32", "two-step"),
    ("k200_unaligned", 1, "f32", "two-step"), ("k200_unaligned", 3, "bf16", "two-step"),
    ("grouped_384_136_136", 1, "f32", "fused"), ("grouped_384_136_136", 1, "bf16", "fused"),
    ("grouped_384_136_136", 4, "bf16", "two-step"), ("grouped_384_136_136", 17, "f32", "two-step"),
    ("long_k17408_ring", 1, "f32", "fused"), ("long_k17408_ring", 1, "bf16", "fused"),
    ("long_k17408_ring", 2, "f32", "two-step"),
    ("long_k40960_ring", 1, "f32", "fused"),
    ("decode_5120", 1, "f32", "fused"), ("decode_5120", 4, "f32", "two-step"), ("decode_5120", 8, "bf16", "two-step"),
    ("decode_5120", 40, "f32", "two-step"),
]


def _x(name, M, K, xdt):
    x = synth.gaussian_activations(SEED, f"d_X_{name}_{M}", M, K)
    if M >= 3:
        x[1] = 0.0                                  # an all-zero token: the amax floor
        x[2, : min(K, 300)] *= np.float32(1e30)     # saturating groups
    if xdt == "bf16":
        x = O.f32_to_bf16(x)                        # the BF16 values themselves, widened exactly
    return x.astype(np.float32)


def _bits(y):
    t = torch()
    return (y.view(t.int16) if y.element_size() == 2 else y.view(t.int32)).cpu().numpy()


@pytest.mark.parametrize("name,M,xdt,path", CASES, ids=[f"{c[0]}-M{c[1]}-{c[2]}" for c in CASES])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_dynamic_equals_quantizer_then_w8a8(name, M, xdt, path, out):
    t = torch()
    members, K = _case(name)
    x = _x(name, M, K, xdt)
    note_fixture(**{f"codes{i}": m.codes for i, m in enumerate(members)},
                 **{f"scale{i}": m.scale_bits for i, m in enumerate(members)}, x=x)
    w = B.BlockFP8Weight([member_to_device(m) for m in members])
    d = w.describe(B.ARM_W8A8_DYNAMIC, M)
    banner(f"w8a8 dynamic {name} M={M} x={xdt} out={out} expected={path}: {d}")
    assert ("arm=w8a8-dynamic" in d) == (path == "fused") and ("quant_act into the workspace" in d) == (path != "fused"), d
    xd = t.from_numpy(x).to(device())
    if xdt == "bf16":
        xd = xd.to(t.bfloat16)
    odt = t.float32 if out == "f32" else t.bfloat16
    y = B.linear_w8a8_dynamic(w, xd, out_dtype=odt)
    xq, xs = B.quant_act(xd)
    y2 = B.linear_w8a8(w, xq, xs, out_dtype=odt)
    t.cuda.synchronize()
    assert np.array_equal(_bits(y), _bits(y2)), f"{name} M={M}: dynamic and two calls differ"
    q_ref, s_ref = O.quant_act(x)
    assert np.array_equal(to_np(xq.view(t.uint8)), q_ref) and np.array_equal(to_np(xs), s_ref)
    om = oracle_members(members)
    assert_within(to_np(y), O.linear_w8a8(q_ref, s_ref, om), O.abs_bound_w8a8(q_ref, s_ref, om), out == "bf16",
                  f"dynamic {name} M={M}")


@pytest.mark.parametrize("M", [1, 3])
def test_dynamic_unaligned_pitch_takes_the_workspace(M):
    """x rows one element apart from 16-byte alignment: the call quantizes into the
    workspace (a missing workspace is refused) and still equals the two calls."""
    t = torch()
    members, K = _case("k1024_640rows")
    w = B.BlockFP8Weight([member_to_device(m) for m in members])
    x = _x("pitch", M, K, "f32")
    big = t.zeros((M, K + 1), dtype=t.float32, device=device())
    big[:, :K] = t.from_numpy(x).to(device())
    xv = big[:, :K]                                 # row pitch K + 1 floats
    with pytest.raises(B.BSF8Error, match="WORKSPACE"):
        B.linear_w8a8_dynamic(w, xv, workspace=(None, 0))
    y = B.linear_w8a8_dynamic(w, xv)
    xq, xs = B.quant_act(xv)
    y2 = B.linear_w8a8(w, xq, xs)
    t.cuda.synchronize()
    assert np.array_equal(_bits(y), _bits(y2))


def test_dynamic_fused_needs_no_workspace():
    """One aligned token takes no workspace: calls without one succeed, on a short and a
    long K, and each equals the two-call result."""
    t = torch()
    for case in ("grouped_384_136_136", "long_k17408_ring"):
        members, K = _case(case)
        w = B.BlockFP8Weight([member_to_device(m) for m in members])
        x = t.from_numpy(_x("nows", 1, K, "f32")).to(device())
        y = B.linear_w8a8_dynamic(w, x, workspace=(None, 0))
        xq, xs = B.quant_act(x)
        y2 = B.linear_w8a8(w, xq, xs)
        t.cuda.synchronize()
        assert np.array_equal(_bits(y), _bits(y2)), case

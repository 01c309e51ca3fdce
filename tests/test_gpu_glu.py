"""GPU parity of the gate/up -> activation -> quantization step (bsf8_quant_glu).

("Module w8a8_prefill", preamble and section "WHY (#917 / #928)": the dense
FFN's gate/up/down prefill arm; the down GEMM consumes per-token 1x128 E4M3
activations.  The activation is the gated SiLU, a reading.)

Bar: codes and scales bit-exact against the oracle's glu_quant on seeded
inputs shaped like gate/up outputs (Gaussian with outlier channels), BF16 and
F32, full FFN width and ragged widths, padded strides, and the activation's
tails (zeros, signed zeros, |g| near and past the exp range).
"""
import numpy as np
import pytest

import block_scaled_fp8_linear_amd as B
import oracle as O
import synth
from gpu_util import banner, device, torch

pytestmark = pytest.mark.gpu


def _gate_up(seed, M, F, scale=1.0):
    g = synth.gaussian_activations(seed, f"glu_G{M}x{F}", M, F) * np.float32(scale)
    u = synth.gaussian_activations(seed, f"glu_U{M}x{F}", M, F) * np.float32(scale)
    return np.concatenate([g, u], axis=1).astype(np.float32)


def _run(y_np, F, dtype, ld_pad=0, q_pad=0):
    t = torch()
    M = y_np.shape[0]
    if dtype == "bf16":
        y_np = O.f32_to_bf16(y_np)
        full = np.zeros((M, 2 * F + ld_pad), np.uint16)
        full[:, :2 * F] = O.f32_to_bf16_bits(y_np)
        yd = t.from_numpy(full.view(np.int16)).to(device()).view(t.bfloat16)
    else:
        full = np.zeros((M, 2 * F + ld_pad), np.float32)
        full[:, :2 * F] = y_np
        yd = t.from_numpy(full).to(device())
    Fb = -(-F // 128)
    xq = t.full((M, F + q_pad), 0x5A, dtype=t.uint8, device=device())
    xs = t.full((M, Fb + q_pad), -1.0, dtype=t.float32, device=device())
    banner(f"quant_glu M={M} F={F} {dtype} ldy_pad={ld_pad} q_pad={q_pad}")
    if ld_pad == 0 and q_pad == 0:
        B.quant_glu(yd, xq, xs)            # through the binding
    else:
        _call_strided(yd, F, xq, xs)       # row pitches wider than the data
    q_ref, s_ref = O.glu_quant(y_np, F)
    q = xq.cpu().numpy()
    s = xs.cpu().numpy()
    assert np.array_equal(q[:, :F], q_ref), f"{int(np.count_nonzero(q[:, :F] != q_ref))} codes differ"
    assert np.array_equal(s[:, :Fb].view(np.uint32), s_ref.view(np.uint32)), "scales differ"
    if q_pad:
        assert np.all(q[:, F:] == 0x5A) and np.all(s[:, Fb:] == -1.0)


def _call_strided(yd, F, xq, xs):
    """Call through the C ABI with a row pitch larger than 2F."""
    L = B.lib()
    M = yd.shape[0]
    Fb = -(-F // 128)
    st = L.bsf8_quant_glu(yd.data_ptr(), B._dt_of(yd), M, F, yd.stride(0), xq.data_ptr(), xq.stride(0),
                          xs.data_ptr(), xs.stride(0), xs.stride(1), B._stream_ptr(yd.device))
    assert st == 0, B.status_name(st)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,F", [(1, 17408), (7, 200), (33, 128), (300, 1000), (5, 4)])
def test_quant_glu_bit_exact(M, F, dtype):
    _run(_gate_up(161, M, F, scale=2.0), F, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quant_glu_padded_strides(dtype):
    _run(_gate_up(163, 9, 384), 384, dtype, ld_pad=24, q_pad=8)


def test_quant_glu_ffn_shape_m1024():
    """The dense-FFN shape: the gate/up output [1024, 2 x 17408] in BF16."""
    _run(_gate_up(165, 1024, 17408, scale=0.5), 17408, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quant_glu_tails(dtype):
    """Signed zeros, all-zero groups, large |g| where exp(-|g|) is subnormal or zero,
    and values that saturate the group scale."""
    F = 256
    y = np.zeros((6, 2 * F), np.float32)
    g, u = y[:, :F], y[:, F:]
    g[0] = -0.0
    u[0] = np.linspace(-3, 3, F, dtype=np.float32)                   # h = signed zeros; amax floor
    g[1, :128] = np.linspace(-200, 200, 128, dtype=np.float32)       # exp(-|g|) normal, subnormal and zero
    u[1, :128] = 1.5
    g[2] = np.float32(88.5)
    u[2] = np.linspace(-1e3, 1e3, F, dtype=np.float32)
    g[3] = np.float32(-87.25)
    u[3] = np.float32(-7.0)
    g[4] = np.linspace(-1e4, 1e4, F, dtype=np.float32)
    u[4] = np.float32(1e-3)
    g[5, ::2] = np.float32(3.0)
    u[5, ::2] = np.float32(2.0)                                        # half the channels zero
    _run(y, F, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quant_glu_kmajor_scales_padded(dtype):
    """K-major scale output (token index contiguous) with a row pitch of M + 5: the same
    bits as the oracle's token-major scales, the padding untouched."""
    t = torch()
    M, F = 11, 640
    Fb = F // 128
    y_np = _gate_up(167, M, F)
    if dtype == "bf16":
        y_np = O.f32_to_bf16(y_np)
        yd = t.from_numpy(O.f32_to_bf16_bits(y_np).view(np.int16)).to(device()).view(t.bfloat16)
    else:
        yd = t.from_numpy(y_np).to(device())
    km = t.full((Fb, M + 5), -1.0, dtype=t.float32, device=device())
    banner(f"quant_glu K-major scales {dtype}")
    xq, _ = B.quant_glu(yd, xs=km[:, :M].t())
    q_ref, s_ref = O.glu_quant(y_np, F)
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert np.array_equal(km[:, :M].cpu().numpy().T.view(np.uint32), s_ref.view(np.uint32))
    assert np.all(km[:, M:].cpu().numpy() == -1.0)

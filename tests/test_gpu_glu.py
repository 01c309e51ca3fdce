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


# ----------------------------------------------------- the activation itself

def _glu_act(y_np, F, dtype, ld_pad=0):
    t = torch()
    M = y_np.shape[0]
    if dtype == "bf16":
        y_np = O.f32_to_bf16(y_np)
        yd = t.from_numpy(O.f32_to_bf16_bits(y_np).view(np.int16)).to(device()).view(t.bfloat16)
    else:
        yd = t.from_numpy(np.ascontiguousarray(y_np)).to(device())
    h = t.full((M, F + ld_pad), 7.0, dtype=t.float32, device=device())
    banner(f"glu_act M={M} F={F} {dtype} ldh_pad={ld_pad}")
    B.glu_act(yd, h[:, :F])
    hn = h.cpu().numpy()
    ref = O.silu_glu(y_np[:, :F], y_np[:, F:2 * F])
    differ = int(np.count_nonzero(hn[:, :F].view(np.uint32) != ref.view(np.uint32)))
    assert differ == 0, f"{differ} activations differ"
    if ld_pad:
        assert np.all(hn[:, F:] == 7.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,F", [(1, 17408), (7, 202), (300, 1000)])
def test_glu_act_bit_exact(M, F, dtype):
    """bsf8_glu_act writes the activation bsf8_quant_glu quantizes: bit for bit the oracle's
    silu(g) * u (e = exp(-|g|) correctly rounded to F32), ragged widths and a padded pitch."""
    _glu_act(_gate_up(171, M, F, scale=2.0), F, dtype, ld_pad=3 if F % 2 else 0)


def test_glu_act_over_the_gate_domain():
    """Every 251st float32 gate value with |g| in [2^-26, 104] (both signs; u = 1), plus the
    arguments among a few million whose exp lies within 2^-42 of a float32 rounding
    midpoint, plus values beyond the range (exp rounds to 1 or to 0): the device's
    activation equals the oracle's correctly rounded definition bit for bit.  (Run over
    every value of the domain, 547 356 674 of them, the same comparison finds no
    difference.)"""
    lo = int(np.float32(2.0 ** -26).view(np.uint32))
    hi = int(np.float32(104.0).view(np.uint32))
    bits = np.arange(lo, hi + 1, 251, dtype=np.uint64).astype(np.uint32)
    g = np.concatenate([bits.view(np.float32), -bits.view(np.float32)])
    rng = np.random.default_rng(239)
    cand = (rng.integers(lo, hi, 4_000_000, dtype=np.int64).astype(np.uint32)).view(np.float32)
    e64 = np.exp(-cand.astype(np.float64))
    c32 = e64.astype(np.float32)
    up = (c32.astype(np.float64) + np.nextafter(c32, np.float32(np.inf)).astype(np.float64)) / 2
    dn = (c32.astype(np.float64) + np.nextafter(c32, np.float32(0)).astype(np.float64)) / 2
    hard = cand[np.minimum(np.abs(e64 - up), np.abs(e64 - dn)) <= 2.0 ** -42 * e64]
    extra = np.array([0.0, -0.0, 2.0 ** -30, -2.0 ** -30, 103.9, -103.9, 104.5, -104.5, 1e6, -1e6, 87.3, -87.3],
                     np.float32)
    g = np.concatenate([g, hard, -hard, extra]).astype(np.float32)
    F = 4096
    pad = (-g.size) % F
    gp = np.concatenate([g, np.zeros(pad, np.float32)]).reshape(-1, F)
    y = np.concatenate([gp, np.ones_like(gp)], axis=1)
    banner(f"glu_act gate domain: {g.size} values ({hard.size} near-midpoint)")
    _glu_act(y, F, "f32")

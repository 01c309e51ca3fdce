"""GPU parity of the resident=False arm: the upcast copy and the dense BF16 product.

("th#1803: the consumer half of the layout gate", section "What lands": with
resident=False the loader upcasts ahead of time; section "Proof", item 2: loaded
weights are bit-identical to the reference dequantization.  "FP8 Native
Serving", section "Native FP8 vs dequant-to-BF16".)

Bars:
* the dense copy: bit-exact against the oracle (BF16 and F32 copies, BF16 and
  F32 grids, grouped members, per-tensor scales, ragged K, padded rows);
* the dense product: |y - y_oracle| <= 1e-3 * sum_k |x_k w_k| per element, plus
  half a BF16 ULP for BF16 outputs.  Its weight operand is the oracle's own
  BF16 copy, so no oracle input comes from the GPU.
"""
import zlib

import numpy as np
import pytest

import block_scaled_fp8_linear_amd as B
import oracle as O
import synth
from gpu_util import assert_within, banner, device, member_to_device, oracle_members, sample_rows, to_np, torch

pytestmark = pytest.mark.gpu

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _f32_grid_members(seed, rows, K):
    g = np.random.default_rng(seed)
    out = []
    for r in rows:
        codes = FINITE[g.integers(0, FINITE.size, (r, K))]
        scale = np.exp2(g.uniform(-10, -2, O.scale_grid_shape(r, K))).astype(np.float32)
        out.append((codes, scale))
    return out


def _device_members(om, scale_dtype):
    t = torch()
    dt = t.float32 if scale_dtype == "f32" else t.bfloat16
    return [(t.from_numpy(np.ascontiguousarray(c)).to(device()), t.from_numpy(np.asarray(s, np.float32)).to(device()).to(dt))
            for c, s in om]


def _bits(y):
    t = torch()
    if y.dtype == t.bfloat16:
        return y.view(t.int16).cpu().numpy().view(np.uint16)
    return y.cpu().numpy().view(np.uint32)


def _ref_bits(ref):
    return ref if ref.dtype == np.uint16 else ref.view(np.uint32)


UPCAST_CASES = {
    # name: (member rows, K, grid dtype)
    "grouped_100_28_130_k256_bf16grid": ((100, 28, 130), 256, "bf16"),
    "grouped_130_7_129_k300_f32grid": ((130, 7, 129), 300, "f32"),     # ragged K: the byte-wise path
    "single_257_k512_f32grid": ((257,), 512, "f32"),
    "single_64_k17408_bf16grid": ((64,), 17408, "bf16"),
    "qkv_384_136_136_k384_bf16grid": ((384, 136, 136), 384, "bf16"),
}


@pytest.mark.parametrize("name", list(UPCAST_CASES))
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_upcast_bit_exact(name, out):
    t = torch()
    rows, K, sdt = UPCAST_CASES[name]
    om = _f32_grid_members(zlib.crc32(name.encode()) % 1000, rows, K)
    if sdt == "bf16":
        om = [(c, O.f32_to_bf16(s)) for c, s in om]
    w = B.BlockFP8Weight(_device_members(om, sdt))
    odt = t.bfloat16 if out == "bf16" else t.float32
    ref = _ref_bits(O.upcast_members(om, out))
    banner(f"upcast {name} -> {out}")
    got = _bits(B.upcast(w, out_dtype=odt))
    assert got.shape == ref.shape and np.array_equal(got, ref), \
        f"{int(np.count_nonzero(got != ref))} of {ref.size} differ"
    # padded rows: columns K..ldo-1 untouched
    pad = t.full((w.n_total, K + 24), -3.0, dtype=odt, device=device())
    banner(f"upcast {name} -> {out}, ldo = K + 24")
    B.upcast(w, out_dtype=odt, out=pad)
    p = _bits(pad)
    assert np.array_equal(p[:, :K], ref)
    assert np.all(p[:, K:] == _bits(t.full((1, 1), -3.0, dtype=odt, device=device()))[0, 0])


@pytest.mark.parametrize("K", [384, 300])
def test_upcast_per_tensor(K):
    t = torch()
    g = np.random.default_rng(77 + K)
    codes = [FINITE[g.integers(0, FINITE.size, (r, K))] for r in (130, 300)]
    svals = [np.float32(2.0 ** -7.25), np.float32(3.0 * 2.0 ** -6)]
    dev = [(t.from_numpy(c).to(device()), t.tensor(float(sv), dtype=t.float32, device=device()))
           for c, sv in zip(codes, svals)]
    w = B.BlockFP8Weight(dev, block=(0, 0))
    om = list(zip(codes, svals))
    for out, odt in (("bf16", t.bfloat16), ("f32", t.float32)):
        banner(f"upcast per-tensor K={K} -> {out}")
        assert np.array_equal(_bits(B.upcast(w, out_dtype=odt)), _ref_bits(O.upcast_members(om, out)))


def test_upcast_of_converted_checkpoint_bit_exact():
    """'Proof' item 2: the loaded copy of a converted checkpoint (BF16 N(0, 0.02) source,
    BF16 grid) is bit-identical to the reference dequantization.  (That the reference lands
    within FP8 error of the source is pinned on the oracle.)"""
    t = torch()
    m = synth.gaussian_weight(131, "up_src", 256, 512)
    w = B.BlockFP8Weight([member_to_device(m)])
    ref = O.upcast_members(oracle_members([m]), "bf16")
    banner("upcast of a converted checkpoint")
    got = _bits(B.upcast(w))
    assert np.array_equal(got, ref)


def _bf16_x(seed, M, K):
    return O.f32_to_bf16(synth.gaussian_activations(seed, f"dense_X{M}x{K}", M, K))


def _dense_check(wd_bits, x, out, tag, workspace=None, ldy_pad=0):
    """Run the dense product on the GPU and compare with the oracle on all outputs."""
    t = torch()
    N, K = wd_bits.shape
    M = x.shape[0]
    wd = t.from_numpy(wd_bits.view(np.int16)).to(device()).view(t.bfloat16)
    xd = t.from_numpy(O.f32_to_bf16_bits(x).view(np.int16)).to(device()).view(t.bfloat16)
    odt = t.bfloat16 if out == "bf16" else t.float32
    y = None
    if ldy_pad:
        y = t.full((M, N + ldy_pad), 5.0, dtype=odt, device=device())
    banner(f"dense {tag} N={N} K={K} M={M} out={out}")
    y = B.linear_dense(wd, xd, out_dtype=odt, out=y, workspace=workspace)
    wf = O.bf16_bits_to_f32(wd_bits)
    ref = O.linear_dense(x, wf)
    assert_within(to_np(y)[:, :N], ref, O.abs_bound_dense(x, wf), out == "bf16", tag)
    if ldy_pad:
        assert np.all(to_np(y)[:, N:] == 5.0)
    return y


DENSE_CASES = {
    # name: (member rows, K, M)
    "tiles_n257_m129_k512": ((257,), 512, 129),
    "ragged_k328_n600_m300": ((600,), 328, 300),          # K bytes 656: a partial 128-byte block
    "grouped_384_136_136_m17": ((384, 136, 136), 384, 17),
    "m1_n640_k1024": ((640,), 1024, 1),
    "split_k_n512_k4096_m16": ((512,), 4096, 16),          # one row tile: K is split
    "long_k17408_n64_m3": ((64,), 17408, 3),
}


@pytest.mark.parametrize("name", list(DENSE_CASES))
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dense_parity(name, out):
    rows, K, M = DENSE_CASES[name]
    om = _f32_grid_members(zlib.crc32(name.encode()) % 997, rows, K)
    om = [(c, O.f32_to_bf16(s)) for c, s in om]
    wd_bits = O.upcast_members(om, "bf16")
    x = _bf16_x(141, M, K)
    _dense_check(wd_bits, x, out, name, ldy_pad=8 if name.startswith("tiles") else 0)


def test_dense_split_k_is_deterministic():
    t = torch()
    om = [(c, O.f32_to_bf16(s)) for c, s in _f32_grid_members(5, (512,), 4096)]
    wd_bits = O.upcast_members(om, "bf16")
    x = _bf16_x(143, 16, 4096)
    assert B.dense_workspace_size(512, 4096, 16) > 0
    y1 = _dense_check(wd_bits, x, "f32", "split-K run 1")
    y2 = _dense_check(wd_bits, x, "f32", "split-K run 2")
    assert t.equal(y1, y2)


def test_dense_full_size_qkv_m512_sampled():
    """Grouped QKV [6144|1000|1000, 5120] at M = 512 through the whole arm: the GPU upcast
    is checked bit-exact against the oracle's copy, then the GPU product over that (identical)
    copy is checked against the oracle's product over its own copy, on sampled rows for all
    tokens."""
    t = torch()
    wl = synth.config4(512)
    w = B.BlockFP8Weight([member_to_device(m) for m in wl.members])
    om = oracle_members(wl.members)
    ref_bits = O.upcast_members(om, "bf16")
    banner("full qkv upcast")
    wd = B.upcast(w)
    assert np.array_equal(_bits(wd), ref_bits)
    x = O.f32_to_bf16(wl.x)
    xd = t.from_numpy(O.f32_to_bf16_bits(x).view(np.int16)).to(device()).view(t.bfloat16)
    banner(f"full qkv dense M=512: {w.describe(B.ARM_DENSE, 512)}")
    y = to_np(B.linear_dense(wd, xd, out_dtype=t.bfloat16))
    rows = sample_rows(w.n_total, [m.codes.shape[0] for m in wl.members], 48)
    wf = O.bf16_bits_to_f32(ref_bits[rows])
    assert_within(y[:, rows], O.linear_dense(x, wf), O.abs_bound_dense(x, wf), True, "qkv dense")

"""Pin checks for the oracle: each returns (ok, detail) so that the mutation
tests can show a planted mistake makes the corresponding pin fail.

A pin ties an oracle function to something that is not the oracle: a value
the pages print (tests/golden), a closed form, a library special case
(PyTorch's casts), an invariant of the definition, or brute force.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_facts():
    with open(os.path.join(GOLDEN, "pages_facts.json")) as f:
        return json.load(f)


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            rows.append((parts[0], int(parts[1], 16)))
    return rows


def _parse_float(tok):
    if tok.startswith(("0x", "-0x")):
        return float.fromhex(tok)
    return float(tok)


def e4m3_worked_values():
    return [(_parse_float(v), c) for v, c in _read_table("e4m3_worked_values.txt")]


def bf16_worked_values():
    return [(_parse_float(v), c) for v, c in _read_table("bf16_worked_values.txt")]


# ------------------------------------------------------------------- P1 / P2

def pin_lut_closed_form(O):
    """P1: the table against the pages' facts and the bit-field definition."""
    facts = golden_facts()["e4m3_range"]
    t = O.e4m3_table()
    nan_codes = sorted(int(c) for c in np.nonzero(np.isnan(t))[0])
    if nan_codes != facts["nan_codes"]:
        return False, f"NaN codes {nan_codes}"
    fin = t[~np.isnan(t)]
    if fin.size != 254:
        return False, "finite count"
    if fin.max() != facts["max_finite"] or fin.min() != facts["min_finite"]:
        return False, "range"
    if np.isinf(t).any():
        return False, "inf present"
    if not (t[0x7E] == 448.0 and t[0xFE] == -448.0):
        return False, "448 codes"
    if not (t[0x00] == 0 and not math.copysign(1, t[0x00]) < 0 and math.copysign(1, t[0x80]) < 0):
        return False, "signed zeros"
    if t[0x01] != 2.0 ** -9 or t[0x08] != 2.0 ** -6 or t[0x07] != 7 * 2.0 ** -9:
        return False, "subnormal/normal boundary"
    pos = t[0x00:0x7F]
    if not np.all(np.diff(pos) > 0):
        return False, "not increasing"
    for c in range(0x80):
        if not (np.isnan(t[c]) and np.isnan(t[c | 0x80])) and t[c | 0x80] != -t[c]:
            return False, f"sign symmetry at {c:#x}"
    # exponent/mantissa structure: within each binade 8 equally spaced values
    for e in range(1, 16):
        v = t[(e << 3):(e << 3) + (7 if e == 15 else 8)]
        if not np.allclose(np.diff(v), 2.0 ** (e - 10)):
            return False, f"binade {e}"
    return True, ""


def pin_lut_vs_torch(O):
    """P1 (library special case): table equals PyTorch's float8_e4m3fn -> float32 decode."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    t = O.e4m3_table()
    same = (np.isnan(tv) == np.isnan(t)) & ((tv == t) | np.isnan(t))
    same &= (np.signbit(tv) == np.signbit(t)) | np.isnan(t)
    return bool(same.all()), ""


def pin_roundtrip(O):
    """P2: ENC(dec(c)) == c for all 254 finite codes, -0.0 included."""
    t = O.e4m3_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    back = O.e4m3_encode(t[codes].astype(np.float32))
    bad = codes[back != codes]
    scal = all(O.e4m3_encode_scalar(float(t[c])) == c for c in codes)
    return (bad.size == 0 and scal), f"bad codes {bad[:8]}"


# ------------------------------------------------------------------- P3 / P4

def pin_worked_ties(O):
    """P3: hand-derived encodings in tests/golden/e4m3_worked_values.txt."""
    for v, c in e4m3_worked_values():
        got = int(O.e4m3_encode(np.array([v], np.float32))[0])
        got_s = O.e4m3_encode_scalar(float(np.float32(v)))
        if got != c or got_s != c:
            return False, f"{v!r}: {got:#x}/{got_s:#x} != {c:#x}"
    return True, ""


def _e4m3_boundary_inputs(O):
    t = O.e4m3_table()
    pos = np.sort(t[(~np.isnan(t)) & (t >= 0)])
    mids = (pos[:-1] + pos[1:]) / 2.0
    base = np.concatenate([pos, mids]).astype(np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    dn = np.nextafter(base, np.float32(-np.inf))
    vals = np.concatenate([base, up, dn])
    vals = vals[(vals >= 0) & (vals <= 448)]
    return np.concatenate([vals, -vals]).astype(np.float32)


def pin_encode_vs_torch(O, n_random=2_000_000, seed=7):
    """P4: ENC equals PyTorch's float32 -> float8_e4m3fn cast on [-448, 448].

    Every representable value, every midpoint and their float32 neighbours,
    plus random values spread over all binades (log-uniform magnitudes).
    """
    import torch
    g = np.random.default_rng(seed)
    mag = np.exp2(g.uniform(-14.0, math.log2(448.0), n_random)).astype(np.float32)
    rnd = np.where(g.random(n_random) < 0.5, -mag, mag).astype(np.float32)
    rnd = np.clip(rnd, -448, 448).astype(np.float32)
    vals = np.concatenate([_e4m3_boundary_inputs(O), rnd, np.array([0.0, -0.0], np.float32)])
    ours = O.e4m3_encode(vals)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    return bad.size == 0, (f"{bad.size} mismatches, first {vals[bad[:4]]}" if bad.size else "")


# ------------------------------------------------------------------------ P5

def pin_bf16(O, n_random=1_000_000, seed=11):
    """P5: BF16 RNE against hand-derived values and PyTorch's float32 -> bfloat16 cast."""
    import torch
    for v, c in bf16_worked_values():
        got = int(O.f32_to_bf16_bits(np.array([v], np.float32))[0])
        if got != c:
            return False, f"{v!r}: {got:#x} != {c:#x}"
    g = np.random.default_rng(seed)
    bits = g.integers(0, 2 ** 32, n_random, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[~np.isnan(vals)]
    ours = O.f32_to_bf16_bits(vals)
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(ours != ref)[0]
    # widening is exact and inverts the narrowing on bf16-representable values
    b = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_bits_to_f32(b)
    keep = ~np.isnan(f)
    rt = O.f32_to_bf16_bits(f[keep]) == b[keep]
    return bad.size == 0 and bool(rt.all()), f"{bad.size} mismatches"


# ------------------------------------------------------------------------ P6

def pin_grids(O):
    """P6: the page's [128,256] -> [1,2], the workloads' grids, member-local origins."""
    ex = golden_facts()["grid_example"]
    if list(O.scale_grid_shape(*ex["weight_shape"])) != ex["scale_shape"]:
        return False, "page example"
    want = {(5120, 5120): (40, 40), (5000, 4000): (40, 32), (17408, 5120): (136, 40),
            (5120, 17408): (40, 136), (6144, 5120): (48, 40), (1000, 5120): (8, 40),
            (18432, 7168): (144, 56), (130, 300): (2, 3), (1, 1): (1, 1), (129, 128): (2, 1)}
    for s, g in want.items():
        if O.scale_grid_shape(*s) != g:
            return False, f"{s}"
    rows = [6144, 1000, 1000]
    R, B = O.member_table(rows)
    if R != [0, 6144, 7144] or B != [0, 48, 56]:
        return False, f"member table {R} {B}"
    checks = {0: 0, 6143: 47, 6144: 48, 7143: 55, 7144: 56, 7167: 56, 7271: 56, 7272: 57, 8143: 63}
    for n, r in checks.items():
        if O.stacked_scale_row(n, rows) != r:
            return False, f"row {n}"
    return True, ""


# ------------------------------------------------------------------------ P7

def pin_scale_direction(O, seed=3):
    """P7: the multiply convention lands within FP8 error of the source weights; a divide is far off.

    The source is BF16 N(0,0.02) [128,256], converted the way a checkpoint
    converter does (PyTorch casts, ``synth.convert_checkpoint``).
    """
    import synth
    facts = golden_facts()["scale_direction"]
    g = np.random.default_rng(seed)
    w = synth._bf16_round_torch(g.standard_normal((128, 256)).astype(np.float32) * np.float32(0.02))
    mem = synth.convert_checkpoint(w)
    s = mem.scale_f32()
    wd = O.dequantize_block_scaled(mem.codes, s)
    w64 = w.astype(np.float64)
    normal = np.abs(O.e4m3_decode(mem.codes)) >= 2.0 ** -6
    rel = np.abs(wd - w64)[normal] / np.abs(w64)[normal]
    if not rel.max() <= facts["multiply_rel_error_upper"]:
        return False, f"multiply rel err {rel.max()}"
    frob_mul = np.linalg.norm(wd - w64) / np.linalg.norm(w64)
    s_full = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:128, :256]
    wdiv = O.e4m3_decode(mem.codes) / s_full
    frob_div = np.linalg.norm(wdiv - w64) / np.linalg.norm(w64)
    if not frob_div >= facts["divide_worse_by_at_least"] * frob_mul:
        return False, f"divide not worse: {frob_div} vs {frob_mul}"
    return True, f"mul {frob_mul:.3g} div {frob_div:.3g}"


# ------------------------------------------------------------------------ P8

def pin_quant_invariants(O, seed=5, M=257, K=1000):
    """P8: per-group invariants of the activation quantizer."""
    g = np.random.default_rng(seed)
    x = (g.standard_normal((M, K)) * np.exp(g.uniform(-8, 8, (M, 1)))).astype(np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[2, :130] = 1e-12
    q, s = O.quant_act(x)
    t = O.e4m3_table()
    Kb = -(-K // 128)
    if s.shape != (M, Kb) or q.shape != (M, K):
        return False, "shapes"
    for gi in range(Kb):
        k0, k1 = gi * 128, min(K, gi * 128 + 128)
        xg = x[:, k0:k1].astype(np.float64)
        amax = np.abs(xg).max(axis=1).astype(np.float32)
        want_s = (np.maximum(amax, np.float32(1e-10)) / np.float32(448)).astype(np.float32)
        if not np.array_equal(s[:, gi], want_s):
            return False, "scale formula"
        dec = t[q[:, k0:k1]]
        nz = amax > 1e-10
        if not np.all(np.abs(dec[nz]).max(axis=1) == 448.0):
            return False, "group max code"
        err = np.abs(dec * s[:, gi:gi + 1].astype(np.float64) - xg)
        if not np.all(err <= 2.0 ** -4 * np.abs(xg) + 2.0 ** -10 * s[:, gi:gi + 1]):
            return False, "reconstruction error"
    if not (np.all(q[0] == 0x00) and np.all(q[1] == 0x80)):
        return False, "zero / negative-zero token"
    return True, ""


# ------------------------------------------------------------------- P9-P11

def tiny_case(seed=1, M=5, K=300, rows=(130, 7)):
    g = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    members = []
    for r in rows:
        codes = finite[g.integers(0, finite.size, (r, K))]
        scale = np.exp2(g.uniform(-10, -2, (-(-r // 128), -(-K // 128)))).astype(np.float32)
        members.append((codes, scale))
    x = g.standard_normal((M, K)).astype(np.float32)
    return x, members


def pin_brute_force(O):
    """P9: the NumPy paths equal pure-Python loops on a tiny grouped case with tails."""
    x, members = tiny_case()
    y = O.linear_w8a16(x, members)
    yl = O.linear_w8a16_loops(x, members)
    if not np.allclose(y, yl, rtol=1e-12, atol=1e-300):
        return False, "w8a16"
    xq, xs = O.quant_act(x)
    y8 = O.linear_w8a8(xq, xs, members)
    y8l = O.linear_w8a8_loops(xq, xs, members)
    if not np.allclose(y8, y8l, rtol=1e-12, atol=1e-300):
        return False, "w8a8"
    return True, ""


def pin_per_tensor(O, seed=21):
    """P9c: a per-tensor scale is the degenerate block ([FP8] 'The two FP8 checkpoint
    shapes'): elementwise dec(code) * s by pure-Python loops on a slice, equal to
    the block path with a grid filled with s, through both arms and the row helper."""
    g = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    K = 300
    members = [(finite[g.integers(0, finite.size, (r, K))], np.float32(np.exp2(e)))
               for r, e in ((130, -7.5), (7, 3.25))]
    for codes, sv in members:
        d = O.dequantize_per_tensor(codes, sv)
        for r in sorted({0, 1, min(64, codes.shape[0] - 1), codes.shape[0] - 1}):
            for k in (0, 1, 127, 128, 299):
                c = int(codes[r, k])
                sgn, e, m = -1.0 if c >> 7 else 1.0, (c >> 3) & 15, c & 7
                v = sgn * (m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))   # E4M3 closed form
                if d[r, k] != v * float(sv):
                    return False, f"dequant [{r},{k}]"
        full = np.full(O.scale_grid_shape(*codes.shape), sv, np.float32)
        if not np.array_equal(d, O.dequantize_block_scaled(codes, full)):
            return False, "block path with a constant grid"
        if not np.array_equal(O.dequantize_per_tensor(codes, np.array([sv], np.float32)), d):
            return False, "one-element scale"
    grids = [(c, np.full(O.scale_grid_shape(*c.shape), sv, np.float32)) for c, sv in members]
    x = g.standard_normal((4, K)).astype(np.float32)
    if not np.array_equal(O.linear_w8a16(x, members), O.linear_w8a16(x, grids)):
        return False, "w8a16"
    if not np.allclose(O.linear_w8a16(x, members), O.linear_w8a16_loops(x, grids), rtol=1e-12, atol=1e-300):
        return False, "w8a16 loops"
    xq, xs = O.quant_act(x)
    if not np.array_equal(O.linear_w8a8(xq, xs, members), O.linear_w8a8(xq, xs, grids)):
        return False, "w8a8"
    rows = [0, 129, 130, 136]
    if not np.array_equal(O.dequantize_rows(members, rows), O.dequantize_members(grids)[rows]):
        return False, "rows"
    return True, ""


def pin_sampled_rows(O):
    """P9b: sampled-row helpers equal the corresponding columns of the full computation."""
    x, members = tiny_case(seed=4, M=3, K=300, rows=(130, 7, 129))
    rows = [0, 1, 127, 128, 129, 130, 136, 137, 200, 265]
    # (BLAS may sum in another order for a sub-matrix, hence 1e-13 and not bit equality)
    close = lambda a, b: np.allclose(a, b, rtol=1e-13, atol=0)
    y = O.linear_w8a16(x, members)
    if not close(O.linear_w8a16_rows(x, members, rows), y[:, rows]):
        return False, "w8a16 rows"
    if not np.array_equal(O.dequantize_rows(members, rows), O.dequantize_members(members)[rows]):
        return False, "dequantized rows"
    xq, xs = O.quant_act(x)
    y8 = O.linear_w8a8(xq, xs, members)
    if not close(O.linear_w8a8_rows(xq, xs, members, rows), y8[:, rows]):
        return False, "w8a8 rows"
    if not close(O.abs_bound_w8a8_rows(xq, xs, members, rows), O.abs_bound_w8a8(xq, xs, members)[:, rows]):
        return False, "bound rows"
    try:
        O.dequantize_rows(members, [266])
        return False, "row past the end accepted"
    except IndexError:
        pass
    return True, ""


def pin_int_partials(O, seed=9):
    """P10: float64 block sums of code products equal the exact integer sums."""
    g = np.random.default_rng(seed)
    t = O.e4m3_table()
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    for _ in range(200):
        a = finite[g.integers(0, finite.size, 128)]
        w = finite[g.integers(0, finite.size, 128)]
        exact = O.w8a8_block_partial_int(a, w)
        f = float(np.sum(t[a] * t[w]) * 2.0 ** 18)
        if f != exact:
            return False, f"{f} != {exact}"
    return True, ""


def pin_special_cases(O, seed=13):
    """P11: reductions to plain integer matmul, per-tensor scaling and one-hot rows."""
    g = np.random.default_rng(seed)
    t = O.e4m3_table()
    # (a) unit scales, integer-valued codes, integer X -> exact int64 matmul
    int_codes = np.array([c for c in range(256) if not np.isnan(t[c]) and t[c] == np.round(t[c])
                          and abs(t[c]) <= 16], np.uint8)
    N, K, M = 20, 260, 3
    codes = int_codes[g.integers(0, int_codes.size, (N, K))]
    xi = g.integers(-5, 6, (M, K))
    scale = np.ones(O.scale_grid_shape(N, K), np.float32)
    y = O.linear_w8a16(xi.astype(np.float32), [(codes, scale)])
    yi = xi.astype(np.int64) @ t[codes].astype(np.int64).T
    if not np.array_equal(y, yi.astype(np.float64)):
        return False, "integer matmul"
    # (b) every scale equal to c -> c times the unscaled product (per-tensor degenerate case)
    c = np.float32(0.0078125 * 3)
    y1 = O.linear_w8a16(xi.astype(np.float32), [(codes, scale * c)])
    if not np.array_equal(y1, yi.astype(np.float64) * float(c)):
        return False, "uniform scale"
    # (c) one-hot weight rows: y[m, n] = x[m, k_n] * dec(code) * s
    K2 = 384
    onehot = np.zeros((4, K2), np.uint8)
    ks = [0, 127, 128, 383]
    for n, k in enumerate(ks):
        onehot[n, k] = 0x4B  # 1.375 * 2^2
    sc = np.array([[0.5, 0.25, 2.0 ** -7]], np.float32)
    x = g.standard_normal((2, K2)).astype(np.float32)
    y = O.linear_w8a16(x, [(onehot, sc)])
    for n, k in enumerate(ks):
        want = x[:, k].astype(np.float64) * 5.5 * float(sc[0, k // 128])
        if not np.array_equal(y[:, n], want):
            return False, "one-hot"
    return True, ""


def pin_cross_arm(O):
    """P12: the oracle's own W8A8-vs-W8A16 gate on a reduced decode-like case."""
    import synth
    w = synth.gaussian_weight(2, "pin_cross_arm_W", 512, 1024)
    x = synth.gaussian_activations(2, "pin_cross_arm_X", 16, 1024)
    members = [(w.codes, w.scale_f32())]
    y16 = O.linear_w8a16(x, members)
    xq, xs = O.quant_act(x)
    y8 = O.linear_w8a8(xq, xs, members)
    cos, rel = O.cross_arm_metrics(y8, y16)
    gate = golden_facts()["cross_arm_gate"]
    return (cos >= gate["cosine_min"] and rel <= gate["relative_rms_max"]), f"cos {cos} rel {rel}"


# ------------------------------------------------------------ P8 brute force

def _f32(v: float) -> float:
    import struct
    return struct.unpack("<f", struct.pack("<f", v))[0]


def pin_quant_brute_force(O, seed=17, M=6, K=300):
    """P8b: the vectorised quantizer equals a pure-Python float32 evaluation.

    The pure-Python path divides in double precision and rounds once to
    float32 (``struct``), which is the correctly rounded float32 quotient, so a
    reciprocal-multiply or a missing clamp in the vectorised code shows up.
    """
    g = np.random.default_rng(seed)
    x = (g.standard_normal((M, K)) * np.exp(g.uniform(-6, 6, (M, 1)))).astype(np.float32)
    # Rows built to sit on E4M3 rounding midpoints after the division: each
    # group holds its amax (so s is known) and values mid*s nudged by a few
    # float32 ulps, where a reciprocal-multiply rounds differently.
    t = O.e4m3_table()
    pos = np.sort(t[(~np.isnan(t)) & (t > 0)])
    mids = (pos[:-1] + pos[1:]) / 2.0
    adv = np.zeros((M, K), np.float32)
    for m in range(M):
        for gi in range(-(-K // 128)):
            k0, k1 = gi * 128, min(K, gi * 128 + 128)
            amax = np.float32(np.exp(g.uniform(-5, 5)))
            sc = np.float32(amax / np.float32(448))
            adv[m, k0] = amax
            mu = g.choice(mids, k1 - k0 - 1)
            base = (mu * np.float64(sc)).astype(np.float32)
            nudge = g.integers(-3, 4, k1 - k0 - 1)
            vals = base.view(np.int32) + nudge.astype(np.int32)
            adv[m, k0 + 1:k1] = np.minimum(vals.view(np.float32), amax) * np.where(g.random(k1 - k0 - 1) < 0.5, -1, 1)
    x = np.concatenate([x, adv]).astype(np.float32)
    M = x.shape[0]
    q, s = O.quant_act(x)
    eps = _f32(1e-10)
    for m in range(M):
        for gi in range(-(-K // 128)):
            k0, k1 = gi * 128, min(K, gi * 128 + 128)
            amax = max(abs(float(v)) for v in x[m, k0:k1])
            sc = _f32(max(amax, eps) / 448.0)
            if float(s[m, gi]) != sc:
                return False, f"scale {m},{gi}"
            for k in range(k0, k1):
                f = _f32(float(x[m, k]) / sc)
                f = min(448.0, max(-448.0, f))
                if int(q[m, k]) != O.e4m3_encode_scalar(f):
                    return False, f"code {m},{k}"
    return True, ""


# ------------------------------------------------------------- P13 / P14

def _torch_upcast(members, dtype):
    """The dense copy built with PyTorch's own casts: float8_e4m3fn -> float32,
    an F32 multiply by the expanded grid, then (for BF16) PyTorch's RNE cast."""
    import torch
    parts = []
    for codes, scale in members:
        w = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float32)
        s = torch.from_numpy(np.asarray(scale, np.float32).reshape(-1, np.asarray(scale).shape[-1])
                             if np.asarray(scale).ndim == 2 else np.asarray(scale, np.float32).reshape(1, 1))
        N, K = w.shape
        s_full = s.repeat_interleave(128, 0)[:N].repeat_interleave(128, 1)[:, :K] if s.numel() > 1 else s
        parts.append(w * s_full)
    d = torch.cat(parts, 0)
    if dtype == "f32":
        return d.numpy()
    return d.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def pin_upcast(O, seed=23):
    """P13: the dense copy of the resident=False arm.

    * equals PyTorch's casts (float8_e4m3fn decode, F32 multiply, BF16 RNE cast)
      on grouped members with F32 and with BF16-valued grids and ragged tails;
    * closed form: codes 0x38 (1.0) give the grid itself in every block;
    * with BF16-valued scales the F32 copy is exact (equals the float64 dequantization);
    * the reading 'F32 product, then BF16' is the one taken where it matters:
      products whose F32 rounding lands on a BF16 tie that the exact product
      does not, so one rounding and two differ.
    """
    import torch
    x, members = tiny_case(seed=seed, M=1, K=300, rows=(130, 7, 129))
    bf_members = [(c, O.f32_to_bf16(s)) for c, s in members]
    for mem in (members, bf_members):
        for dt in ("f32", "bf16"):
            ours = O.upcast_members(mem, dt)
            ref = _torch_upcast(mem, dt)
            if ours.shape != ref.shape or not np.array_equal(ours.view(np.uint32 if dt == "f32" else np.uint16),
                                                             ref.view(np.uint32 if dt == "f32" else np.uint16)):
                return False, f"torch casts ({dt})"
    exact = O.upcast_members(bf_members, "f32").astype(np.float64)
    if not np.array_equal(exact, O.dequantize_members(bf_members)):
        return False, "BF16 grid: F32 copy not exact"
    ones = [(np.full_like(c, 0x38), s) for c, s in members]
    d = O.upcast_members(ones, "f32")
    r0 = 0
    for c, s in members:
        N, K = c.shape
        for r in (0, N - 1):
            for k in (0, K - 1):
                if d[r0 + r, k] != s[r // 128, k // 128]:
                    return False, f"closed form [{r0 + r},{k}]"
        r0 += N
    # double rounding: dec = 1.125 (code 0x39); scales near tie/1.125 for BF16 ties T
    cases = 0
    for t in range(1, 256, 2):
        T = 1.0 + t * 2.0 ** -8                      # odd multiple of 2^-8: a BF16 tie in [1, 2)
        s32 = np.float32(T / 1.125)
        for sv in (s32, np.nextafter(s32, np.float32(2)), np.nextafter(s32, np.float32(0))):
            p = 1.125 * float(sv)                     # exact in float64
            f32 = np.float32(p)
            if float(f32) != T or p == T:
                continue
            # one rounding of the exact product to BF16's 8 significant bits, ties to even
            m, e = math.frexp(p)
            once = float(round(m * 256.0)) * 2.0 ** (e - 8)
            twice = torch.tensor([float(f32)], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[0]
            if once == float(O.bf16_bits_to_f32(np.array([twice], np.uint16))[0]):
                continue
            cases += 1
            got = O.upcast_members([(np.array([[0x39]], np.uint8), np.array([[sv]], np.float32))], "bf16")[0, 0]
            if got != twice:
                return False, f"double rounding at T={T}"
    if cases == 0:
        return False, "no double-rounding case found"
    return True, f"{cases} double-rounding cases"


def pin_dense_brute_force(O, seed=29):
    """P14: the dense product equals pure-Python loops on a tiny BF16 case with a ragged K."""
    g = np.random.default_rng(seed)
    x = O.f32_to_bf16(g.standard_normal((3, 70)).astype(np.float32))
    wd = O.f32_to_bf16(g.standard_normal((5, 70)).astype(np.float32) * np.float32(0.02))
    y = O.linear_dense(x, wd)
    if not np.allclose(y, O.linear_dense_loops(x, wd), rtol=1e-12, atol=1e-300):
        return False, "loops"
    if not np.allclose(O.abs_bound_dense(x, wd), O.linear_dense_loops(np.abs(x), np.abs(wd)), rtol=1e-12, atol=1e-300):
        return False, "bound"
    return True, ""


# ------------------------------------------------------------------- P15

def _f32(v: float) -> float:
    import struct
    return struct.unpack("<f", struct.pack("<f", v))[0]


def pin_silu_glu(O, seed=31):
    """P15: the gated activation feeding the down projection.

    * PyTorch's SiLU (float64) times u agrees within 4 float32 ulps where
      exp(-|g|) is a normal float32 (|g| < 80), over values spanning 2^-6..2^6;
    * closed forms: g = 0 gives signed zeros, g = 100 gives g*u exactly,
      g = -200 gives -0 * u (exp(-200) rounds to zero);
    * brute force with the correctly rounded exp of an 80-digit decimal
      evaluation and float32 rounding after each step equals it bit for bit,
      tails included;
    * glu_quant is quant_act of it over the gate/up halves, in that order.
    """
    import math
    import torch
    g = np.random.default_rng(seed)
    gate = (g.standard_normal(4000) * np.exp2(g.uniform(-6, 6, 4000))).astype(np.float32)
    up = (g.standard_normal(4000) * np.exp2(g.uniform(-6, 6, 4000))).astype(np.float32)
    h = O.silu_glu(gate, up)
    ref = (torch.nn.functional.silu(torch.from_numpy(gate).double()) * torch.from_numpy(up).double()).numpy()
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    keep = np.abs(gate) < 80
    if not np.all((np.abs(h.astype(np.float64) - ref) <= 4 * ulp)[keep]):
        return False, "torch silu"
    for gv, uv in ((0.0, 3.0), (0.0, -3.0), (100.0, 1.5), (-200.0, 2.0), (-200.0, -2.0)):
        hv = float(O.silu_glu(np.float32(gv), np.float32(uv)))
        want = {0.0: 0.0 * uv, 100.0: gv * uv, -200.0: -0.0 * uv}[gv]
        if hv != want or math.copysign(1, hv) != math.copysign(1, want):
            return False, f"closed form g={gv} u={uv}: {hv}"
    for gv, uv in list(zip(gate[:300], up[:300])) + [(np.float32(-95.5), np.float32(3.0)),
                                                     (np.float32(-150.25), np.float32(-1.0))]:
        ev = _exp_rn32_decimal(abs(float(gv)))
        tv = _f32(1.0 + ev)
        qv = _f32(float(gv) / tv) if gv >= 0 else _f32(_f32(float(gv) * ev) / tv)
        hv = _f32(qv * float(uv))
        ov = float(O.silu_glu(gv, uv))
        if hv != ov or math.copysign(1, hv) != math.copysign(1, ov):
            return False, f"brute force g={gv} u={uv}"
    M, F = 3, 200
    y = np.concatenate([gate[:M * F].reshape(M, F), up[:M * F].reshape(M, F)], axis=1)
    q, s = O.glu_quant(y, F)
    q2, s2 = O.quant_act(O.silu_glu(y[:, :F], y[:, F:]))
    if not (np.array_equal(q, q2) and np.array_equal(s, s2)):
        return False, "glu_quant composition"
    return True, ""


# ------------------------------------------------------------ P16 - P18
# The helpers every GEMM verdict rests on: the per-element error scale
# sum_k |a_k w_k|, the acceptance test built on it, and the cross-arm metrics
# of "Module w8a8_prefill", section "ACCURACY".

def _dec_py(c: int) -> float:
    """E4M3 value of one finite code from its bit fields (sign, exponent bias 7, 3-bit mantissa)."""
    sgn = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 0xF, c & 7
    return sgn * (m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))


def _abs_sum_loops(a_rows, members, K):
    """sum_k |a[m,k]| * |dec(w[n,k]) * s_i[r//128, k//128]| by plain Python loops.

    ``a_rows`` holds float values (lists of floats) per token; the weights are
    decoded from their bit fields here, so neither the oracle's table nor
    NumPy's matmul is involved."""
    dec = _dec_py
    out = []
    for a in a_rows:
        row = []
        for codes, scale in members:
            for r in range(codes.shape[0]):
                acc = 0.0
                for k in range(K):
                    acc += abs(a[k]) * abs(dec(int(codes[r, k])) * float(scale[r // 128, k // 128]))
                row.append(acc)
        out.append(row)
    return np.array(out, np.float64)


def pin_abs_bounds(O, seed=37):
    """P16: the error scale sum_k |a_k w_k| of both arms and of their row forms.

    * equals pure-Python loops over the dequantized operands, on grouped
      members with ragged rows and a ragged K (W8A16: a_k = x_k; W8A8: a_k =
      dec(q_k) * s_a of the token's group);
    * closed form: with every operand non-negative there is no cancellation,
      so the bound equals the output itself;
    * flipping the sign of activations or weight codes leaves it unchanged,
      while the output changes, so |sum| in place of sum |.| is caught.
    """
    g = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    K = 200
    members = [(finite[g.integers(0, finite.size, (r, K))],
                np.exp2(g.uniform(-9, -3, (-(-r // 128), -(-K // 128)))).astype(np.float32)) for r in (130, 5)]
    x = (g.standard_normal((3, K)) * np.exp2(g.uniform(-3, 3, (3, 1)))).astype(np.float32)
    b16 = O.abs_bound_w8a16(x, members)
    loops16 = _abs_sum_loops([[float(v) for v in row] for row in x], members, K)
    if b16.shape != loops16.shape or not np.allclose(b16, loops16, rtol=1e-12, atol=0):
        return False, "w8a16 bound vs loops"
    xq, xs = O.quant_act(x)
    a = [[_dec_py(int(xq[m, k])) * float(xs[m, k // 128]) for k in range(K)] for m in range(x.shape[0])]
    b8 = O.abs_bound_w8a8(xq, xs, members)
    if not np.allclose(b8, _abs_sum_loops(a, members, K), rtol=1e-12, atol=0):
        return False, "w8a8 bound vs loops"
    rows = [0, 127, 128, 129, 130, 134]
    if not np.allclose(O.abs_bound_w8a16_rows(x, members, rows), loops16[:, rows], rtol=1e-12, atol=0):
        return False, "w8a16 row form"
    if not np.allclose(O.abs_bound_w8a8_rows(xq, xs, members, rows), b8[:, rows], rtol=1e-12, atol=0):
        return False, "w8a8 row form"
    pos = [(c & np.uint8(0x7F), s) for c, s in members]
    xp = np.abs(x)
    if not np.array_equal(O.abs_bound_w8a16(xp, pos), O.linear_w8a16(xp, pos)):
        return False, "non-negative operands: bound != output"
    qp, sp = O.quant_act(xp)
    if not np.array_equal(O.abs_bound_w8a8(qp, sp, pos), O.linear_w8a8(qp, sp, pos)):
        return False, "non-negative operands (w8a8): bound != output"
    flipped = [(c ^ np.uint8(0x80), s) for c, s in members]
    if not np.array_equal(O.abs_bound_w8a16(-x, flipped), b16):
        return False, "sign flips change the bound"
    y = O.linear_w8a16(x, members)
    if not (np.all(b16 >= np.abs(y)) and np.any(b16 > 2 * np.abs(y))):
        return False, "bound does not dominate |y| with room on mixed signs"
    return True, ""


def pin_within_bound(O, seed=41):
    """P17: the acceptance test |y - y_ref| <= 1e-3 * S (+ 2^-8 |y_ref| for BF16).

    * an error of 0.999 x the bound passes and 1.001 x fails, element by
      element, for the F32 form and the BF16 form (whose half-ULP term is
      checked against the F32 form on the same errors);
    * NaN on either side fails; a zero bound with equal outputs passes;
    * the reported worst ratio is max(err / bound) computed by a loop.
    """
    g = np.random.default_rng(seed)
    S = np.exp2(g.uniform(-10, 10, (4, 7)))
    y_ref = g.standard_normal((4, 7)) * S * 0.01
    sign = np.where(g.random((4, 7)) < 0.5, -1.0, 1.0)
    for bf16 in (False, True):
        bound = 1e-3 * S + (2.0 ** -8 * np.abs(y_ref) if bf16 else 0.0)
        ok, worst = O.within_bound(y_ref + sign * 0.999 * bound, y_ref, S, bf16_out=bf16)
        if not ok:
            return False, f"0.999 x bound rejected (bf16={bf16})"
        loop_worst = max(abs((y_ref[i, j] + sign[i, j] * 0.999 * bound[i, j]) - y_ref[i, j]) / bound[i, j]
                         for i in range(4) for j in range(7))
        if abs(worst - loop_worst) > 1e-9:
            return False, f"worst ratio {worst} vs {loop_worst}"
        for i, j in ((0, 0), (3, 6), (2, 3)):
            y = y_ref + sign * 0.5 * bound
            y[i, j] = y_ref[i, j] + sign[i, j] * 1.001 * bound[i, j]
            if O.within_bound(y, y_ref, S, bf16_out=bf16)[0]:
                return False, f"1.001 x bound accepted at {i},{j} (bf16={bf16})"
    # the BF16 form adds exactly half a BF16 ULP's worth: an error between the two bounds
    mid = y_ref + sign * (1e-3 * S + 2.0 ** -9 * np.abs(y_ref))
    if not O.within_bound(mid, y_ref, S, bf16_out=True)[0] or O.within_bound(mid, y_ref, S, bf16_out=False)[0]:
        return False, "BF16 term"
    for bad in (np.nan,):
        y = y_ref.copy()
        y[1, 2] = bad
        if O.within_bound(y, y_ref, S)[0]:
            return False, "NaN output accepted"
        r = y_ref.copy()
        r[1, 2] = bad
        if O.within_bound(y_ref, r, S)[0]:
            return False, "NaN reference accepted"
    z = np.zeros((2, 3))
    if not O.within_bound(z, z, z)[0]:
        return False, "zero bound, equal outputs rejected"
    if O.within_bound(z + 1e-30, z, z)[0]:
        return False, "zero bound, unequal outputs accepted"
    return True, ""


def pin_cross_arm_metrics(O, seed=43):
    """P18: cosine and relative RMS of the W8A8 output against the W8A16 one.

    Closed forms: identical outputs give (1, 0); orthogonal outputs cos 0;
    y8 = 1.01 y16 gives rel 0.01 and y16 = 1.01 y8 gives 0.01/1.01 (the W8A16
    output is the reference, the denominator); y8 = -y16 gives (-1, 2).
    Brute force: sums written out as Python loops over the flattened output,
    on a 2-D case whose rows have very different magnitudes (a per-row mean of
    metrics would differ).
    """
    g = np.random.default_rng(seed)
    y = g.standard_normal((5, 9)) * np.exp2(np.arange(5) * 3.0)[:, None]
    cos, rel = O.cross_arm_metrics(y, y)
    if abs(cos - 1.0) > 1e-15 or rel != 0.0:
        return False, f"identical: {cos} {rel}"
    a = np.array([1.0, 2.0, 0.0, -3.0])
    b = np.array([2.0, -1.0, 5.0, 0.0])
    if abs(O.cross_arm_metrics(a, b)[0]) > 1e-15:
        return False, "orthogonal"
    cos, rel = O.cross_arm_metrics(1.01 * y, y)
    if abs(rel - 0.01) > 1e-12 or abs(cos - 1.0) > 1e-15:
        return False, f"y8 = 1.01 y16: {cos} {rel}"
    if abs(O.cross_arm_metrics(y, 1.01 * y)[1] - 0.01 / 1.01) > 1e-12:
        return False, "denominator is not the W8A16 output"
    cos, rel = O.cross_arm_metrics(-y, y)
    if abs(cos + 1.0) > 1e-15 or abs(rel - 2.0) > 1e-12:
        return False, "opposite"
    y8 = y + g.standard_normal(y.shape) * 0.05 * np.abs(y)
    fa, fb = [float(v) for v in y8.ravel()], [float(v) for v in y.ravel()]
    dot = sum(p * q for p, q in zip(fa, fb))
    na = math.sqrt(sum(p * p for p in fa))
    nb = math.sqrt(sum(q * q for q in fb))
    nd = math.sqrt(sum((p - q) ** 2 for p, q in zip(fa, fb)))
    cos, rel = O.cross_arm_metrics(y8, y)
    if abs(cos - dot / (na * nb)) > 1e-12 or abs(rel - nd / nb) > 1e-12:
        return False, f"loops: {cos} vs {dot / (na * nb)}, {rel} vs {nd / nb}"
    return True, ""


# ------------------------------------------------------------------- P19

def _exp_rn32_decimal(a: float) -> float:
    """exp(-a) correctly rounded to float32, from an 80-digit decimal evaluation
    compared exactly with the float32 midpoints around it."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = 80
        ed = (-Decimal(a)).exp()
        c = np.float32(float(ed))
        for _ in range(2):
            up = np.nextafter(c, np.float32(np.inf))
            dn = np.nextafter(c, np.float32(0.0))
            if ed > (Decimal(float(c)) + Decimal(float(up))) / 2:
                c = up
            elif c > 0 and ed < (Decimal(float(c)) + Decimal(float(dn))) / 2:
                c = dn
    return float(c)


def pin_exp_correctly_rounded(O, seed=47, n_random=20000, n_search=4_000_000):
    """P19: the activation's e = exp(-|g|) is the float32 nearest to the exact value.

    * equals an independent 80-digit decimal evaluation on random float32
      arguments over [0, 110] (both signs of g) and on every argument, among a
      few million random ones, whose exp lies within 2^-42 of a float32 rounding
      midpoint (where a float64 evaluation rounded once more could differ);
    * closed forms: exp(0) = 1; arguments beyond 103.98 round to 0; the value
      stays in [0, 1].
    """
    g = np.random.default_rng(seed)
    x = (g.integers(0, 0x42DC0000, n_random, dtype=np.int64).astype(np.uint32)).view(np.float32)
    x = x * np.where(g.random(n_random) < 0.5, np.float32(-1), np.float32(1))
    e = O.exp_neg_abs_f32(x)
    for xi, ei in zip(x, e):
        if float(ei) != _exp_rn32_decimal(abs(float(xi))):
            return False, f"random argument {float(xi)!r}"
    cand = (g.integers(0, 0x42D00000, n_search, dtype=np.int64).astype(np.uint32)).view(np.float32)
    e64 = np.exp(-cand.astype(np.float64))
    c32 = e64.astype(np.float32)
    mids = [(c32.astype(np.float64) + np.nextafter(c32, np.float32(np.inf)).astype(np.float64)) / 2,
            (c32.astype(np.float64) + np.nextafter(c32, np.float32(0)).astype(np.float64)) / 2]
    dist = np.minimum(np.abs(e64 - mids[0]), np.abs(e64 - mids[1])) / e64
    hard = cand[dist <= 2.0 ** -42]
    if hard.size == 0:
        return False, "no near-midpoint argument found"
    eh = O.exp_neg_abs_f32(hard)
    for xi, ei in zip(hard, eh):
        if float(ei) != _exp_rn32_decimal(float(xi)):
            return False, f"near-midpoint argument {float(xi)!r}"
    edge = O.exp_neg_abs_f32(np.array([0.0, -0.0, 104.0, -200.0, 1e30], np.float32))
    if not (edge[0] == 1.0 and edge[1] == 1.0 and edge[2] == 0.0 and edge[3] == 0.0 and edge[4] == 0.0):
        return False, f"closed forms {edge}"
    if not (np.all(e >= 0) and np.all(e <= 1)):
        return False, "range"
    return True, f"{hard.size} near-midpoint arguments"

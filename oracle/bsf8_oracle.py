"""Plain, slow, obviously correct CPU reference for the block-scaled FP8 linear.

TEST INFRASTRUCTURE ONLY.  Importable by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.  It
shares no code, table or constant generator with the HIP library.

Sources (cited by page title and section; no line numbers):

* [QWEN]   butter docs, "Qwen checkpoints with block FP8 weights":
           layout paragraph, block-path paragraph, operator/grid/refusal paragraph,
           fixture paragraph of the CUDA numerical test.
* [TH1803] python-gen-worker PR, "th#1803: the consumer half of the layout gate":
           sections "What lands", "Why the refusals matter more than the load",
           "Proof (no mocks, CPU, ~9s)".
* [W8A8]   Atlas API docs, "Module w8a8_prefill": sections "WHY (#917 / #928)",
           "ACCURACY".
* [FP8]    Atlas deep dive, "FP8 Native Serving": sections "The two FP8 checkpoint
           shapes", "FP8 E4M3: range and quirks", "Native FP8 vs dequant-to-BF16".

Arithmetic: E4M3 values and BF16/F32 scales are exact in float64, and so is
their product, so dequantized operands are exact; the GEMMs are plain float64
matrix products of those operands.  Activation quantization is done in float32
exactly as stated in ``quant_act`` (the result is a byte pattern, so its
precision is part of the definition).

Readings of points the pages leave open are marked "Reading:" in the docstring
where they are used.  Every function here is pinned (no "parity unpinned").
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "BLOCK", "E4M3_MAX", "ACT_EPS",
    "e4m3_table", "e4m3_decode", "e4m3_encode", "e4m3_encode_scalar",
    "bf16_bits_to_f32", "f32_to_bf16_bits", "f32_to_bf16",
    "scale_grid_shape", "member_table", "stacked_scale_row",
    "dequantize_block_scaled", "dequantize_per_tensor", "dequantize_members", "dequantize_rows",
    "linear_w8a16_rows", "linear_w8a8_rows", "abs_bound_w8a16_rows", "abs_bound_w8a8_rows",
    "linear_w8a16", "quant_act", "dequantize_act", "linear_w8a8",
    "linear_w8a16_loops", "linear_w8a8_loops", "w8a8_block_partial_int",
    "abs_bound_w8a16", "abs_bound_w8a8", "round_output", "within_bound",
    "cross_arm_metrics", "Status", "TensorDesc", "MemberDesc", "validate",
    "upcast_members", "linear_dense", "abs_bound_dense", "linear_dense_loops",
    "exp_neg_abs_f32", "silu_glu", "glu_quant",
]

BLOCK = 128            # weight_block_size [128,128]  [QWEN layout paragraph]
E4M3_MAX = 448.0       # largest finite E4M3 magnitude  [FP8 "FP8 E4M3: range and quirks"]
# Reading: the pages give no floor for an all-zero activation group.  The group
# amax is raised to this float32 value before dividing by 448 (the floor of the
# per-token group quantizer the W8A8 page names), so a zero group quantizes to
# signed zeros with a tiny positive scale.
ACT_EPS = np.float32(1e-10)


# ---------------------------------------------------------------- E4M3 codec

def e4m3_table() -> np.ndarray:
    """256-entry decode table, float64, written from the E4M3 definition.

    [FP8 "FP8 E4M3: range and quirks"]: one sign bit, four exponent bits with
    bias 7, three mantissa bits; no infinities; the two all-ones patterns
    0x7F and 0xFF are NaN; finite range +-448.  Exponent field 0 encodes the
    subnormals m * 2^-9 (definition of the format).
    """
    t = np.empty(256, np.float64)
    for c in range(256):
        sign = -1.0 if (c >> 7) & 1 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = math.nan
        elif e == 0:
            t[c] = sign * m * 2.0 ** -9
        else:
            t[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_E4M3 = e4m3_table()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode uint8 E4M3 codes to float64 through the table."""
    return _E4M3[np.asarray(codes, np.uint8)]


def e4m3_encode_scalar(f: float) -> int:
    """Round-to-nearest-even E4M3 encoding of one float in [-448, 448], pure Python.

    Normal range |f| >= 2^-6: write |f| = t * 2^e with t in [1,2); the mantissa
    field is t's fraction rounded to 3 bits (ties to even); a carry to 8 bumps
    the exponent.  Below 2^-6 the value is a multiple of 2^-9 (subnormal),
    rounded to nearest even; a result of 8 * 2^-9 is the smallest normal 0x08.
    The sign bit is kept for zeros, so -0.0 encodes as 0x80.
    """
    sign = 0x80 if math.copysign(1.0, f) < 0 else 0
    a = abs(float(f))
    if a > E4M3_MAX or a != a:
        raise ValueError("outside the clamped E4M3 domain")
    if a >= 2.0 ** -6:
        mant, exp = math.frexp(a)          # a = mant * 2^exp, mant in [0.5, 1)
        t, e = mant * 2.0, exp - 1
        mq = round((t - 1.0) * 8.0)        # Python round() is ties-to-even
        if mq == 8:
            e, mq = e + 1, 0
        return sign | ((e + 7) << 3) | mq
    mq = round(a * 2.0 ** 9)
    return sign | mq


def e4m3_encode(f: np.ndarray) -> np.ndarray:
    """Vectorised ``e4m3_encode_scalar`` for float32 arrays already clamped to +-448."""
    f = np.asarray(f, np.float32)
    a = np.abs(f.astype(np.float64))
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("outside the clamped E4M3 domain")
    sign = np.where(np.signbit(f), 0x80, 0).astype(np.int64)
    mant, exp = np.frexp(a)
    t, e = mant * 2.0, exp.astype(np.int64) - 1
    mq = np.rint((t - 1.0) * 8.0).astype(np.int64)       # np.rint: ties to even
    carry = mq == 8
    e = np.where(carry, e + 1, e)
    mq = np.where(carry, 0, mq)
    normal_code = ((e + 7) << 3) | mq
    sub_code = np.rint(a * 2.0 ** 9).astype(np.int64)
    code = np.where(a >= 2.0 ** -6, normal_code, sub_code) | sign
    return code.astype(np.uint8)


# ---------------------------------------------------------------- BF16 casts

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """BF16 -> F32 by placing the 16 bits on top of 16 zero bits (exact).

    [QWEN layout paragraph]: BF16 block scales widen exactly to F32.
    """
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """F32 -> BF16 bit patterns, round to nearest, ties to even; NaN -> quiet NaN.

    [FP8 "FP8 E4M3: range and quirks"]: the BF16 cast used when results are
    written back rounds to nearest even.  Written from the definition: keep the
    top 16 bits, round up when the dropped 16 bits exceed half, or equal half
    and the kept part is odd.  A carry may ripple into the exponent (to inf).
    """
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    keep = u >> np.uint64(16)
    rem = u & np.uint64(0xFFFF)
    up = (rem > 0x8000) | ((rem == 0x8000) & ((keep & np.uint64(1)) == 1))
    out = (keep + up.astype(np.uint64)).astype(np.uint32)
    nan = np.isnan(np.asarray(x, np.float32))
    out = np.where(nan, (keep | np.uint64(0x40)).astype(np.uint32), out)
    return out.astype(np.uint16)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """RNE BF16 rounding of float32 values, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ------------------------------------------------------------ grids, members

def scale_grid_shape(n: int, k: int, block: Tuple[int, int] = (BLOCK, BLOCK)) -> Tuple[int, int]:
    """Ceil-divided scale grid [ceil(N/bn), ceil(K/bk)] of an [N,K] weight.

    [QWEN operator paragraph]: partial block rows/columns get their own cell;
    [TH1803 "Proof"]: a [128,256] down_proj has a [1,2] grid.
    """
    return (-(-int(n) // block[0]), -(-int(k) // block[1]))


def member_table(rows: Sequence[int]) -> Tuple[List[int], List[int]]:
    """Origins of grouped members: output-row origin R_i and stacked scale-row origin B_i.

    [QWEN operator paragraph]: grouped tensors keep their own block-row
    origin, so member i's scale rows start at B_i = sum_{j<i} ceil(N_j/128)
    and its output rows at R_i = sum_{j<i} N_j.
    """
    R, B = [0], [0]
    for n in rows:
        R.append(R[-1] + int(n))
        B.append(B[-1] + -(-int(n) // BLOCK))
    return R[:-1], B[:-1]


def stacked_scale_row(n: int, rows: Sequence[int]) -> int:
    """Row of the stacked member grids that holds the scale of output row ``n``."""
    R, B = member_table(rows)
    for i in range(len(rows) - 1, -1, -1):
        if n >= R[i]:
            if n - R[i] >= rows[i]:
                break
            return B[i] + (n - R[i]) // BLOCK
    raise IndexError(n)


# ---------------------------------------------------------------- dequantize

def dequantize_block_scaled(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Wd[r,k] = dec(codes[r,k]) * scale[r//128, k//128], float64 (exact).

    [TH1803 "What lands"]: the grid holds one value per 128x128 block applied
    as a multiplier; [QWEN layout paragraph]: they are dequantization
    multipliers, not reciprocals.  ``scale`` is float32 (BF16 scales are widened
    first with ``bf16_bits_to_f32``).
    """
    codes = np.asarray(codes, np.uint8)
    N, K = codes.shape
    if tuple(scale.shape) != scale_grid_shape(N, K):
        raise ValueError(f"scale grid {scale.shape} != {scale_grid_shape(N, K)}")
    s = np.asarray(scale, np.float32).astype(np.float64)
    s_full = np.repeat(np.repeat(s, BLOCK, axis=0)[:N], BLOCK, axis=1)[:, :K]
    return e4m3_decode(codes) * s_full


def dequantize_per_tensor(codes: np.ndarray, scale) -> np.ndarray:
    """Wd[r,k] = dec(codes[r,k]) * scale, float64 (exact), for one per-tensor scale.

    [FP8 "The two FP8 checkpoint shapes"]: the per-tensor layout pairs the E4M3
    weight with a single weight_scale for the whole tensor, and reads as the
    degenerate block case: one block covering every element.  ``scale`` is a
    float32 scalar (a 0-d or one-element array).
    """
    codes = np.asarray(codes, np.uint8)
    sv = np.asarray(scale, np.float32)
    if sv.size != 1 or sv.ndim > 1:
        raise ValueError(f"per-tensor scale must hold one value, got shape {sv.shape}")
    return e4m3_decode(codes) * float(sv.reshape(()))


def _is_per_tensor(scale) -> bool:
    sv = np.asarray(scale)
    return sv.ndim == 0 or (sv.ndim == 1 and sv.size == 1)


def dequantize_members(members: Iterable[Tuple[np.ndarray, np.ndarray]]) -> np.ndarray:
    """Concatenate the dequantized members along N, each with its own grid (or
    its own per-tensor scale)."""
    return np.concatenate([dequantize_per_tensor(c, s) if _is_per_tensor(s) else dequantize_block_scaled(c, s)
                           for c, s in members], axis=0)


def dequantize_rows(members: Sequence[Tuple[np.ndarray, np.ndarray]], rows: Sequence[int]) -> np.ndarray:
    """Dequantized weight rows for global output indices ``rows`` (float64 [len(rows), K]).

    Row n belongs to the member i with R_i <= n < R_i + N_i and uses row
    (n - R_i) // 128 of that member's own grid (member-local origin).
    """
    sizes = [c.shape[0] for c, _ in members]
    R, _ = member_table(sizes)
    K = members[0][0].shape[1]
    kcol = np.arange(K) // BLOCK
    out = np.empty((len(rows), K), np.float64)
    for j, n in enumerate(rows):
        i = max(ii for ii in range(len(sizes)) if R[ii] <= n)
        r = int(n) - R[i]
        if r >= sizes[i]:
            raise IndexError(n)
        codes, scale = members[i]
        if _is_per_tensor(scale):
            out[j] = e4m3_decode(codes[r]) * float(np.asarray(scale, np.float32).reshape(()))
        else:
            out[j] = e4m3_decode(codes[r]) * np.asarray(scale, np.float32)[r // BLOCK].astype(np.float64)[kcol]
    return out


# ------------------------------------------------------------------ W8A16/F32

def linear_w8a16(x: np.ndarray, members: Sequence[Tuple[np.ndarray, np.ndarray]]) -> np.ndarray:
    """Y = X . Wd^T in float64, X taken as given (float32 or BF16-valued float32).

    [QWEN block-path paragraph]: resident FP8 weights times their block
    multiplier inside the reduction, F32 activations, no requantization of
    either operand.  The exact value of that sum is X . Wd^T.
    """
    x64 = np.asarray(x, np.float32).astype(np.float64)
    return x64 @ dequantize_members(members).T


# ----------------------------------------------- upcast at load (dense arm)

def upcast_members(members: Sequence[Tuple[np.ndarray, np.ndarray]], dtype: str) -> np.ndarray:
    """Dense copy [N_total, K] of a (grouped) weight, as the resident=False arm
    loads it: 'f32' -> float32 values; 'bf16' -> BF16 bit patterns (uint16).

    [TH1803 "What lands"]: with resident=False the loader upcasts the weight
    ahead of time instead of keeping the FP8 bytes; [FP8 "Native FP8 vs
    dequant-to-BF16"]: the dequantized operand the matrix unit then reads is
    BF16.  Members stay in order along N, each with its own grid.
    Reading: an element is dec(q) * s formed as one float32 product (the exact
    float64 product rounded once to float32, which is what an F32 multiply
    returns; exact whenever the scale is BF16, since 4 + 8 significant bits fit
    in 24), and a BF16 copy rounds that float32 value to nearest-even.
    """
    w32 = dequantize_members(members).astype(np.float32)
    if dtype == "f32":
        return w32
    if dtype == "bf16":
        return f32_to_bf16_bits(w32)
    raise ValueError(dtype)


def linear_dense(x: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """Y = X . Wd^T in float64 for dense operands given as float32 values
    (BF16 operands widened with ``bf16_bits_to_f32``).

    [FP8 "Native FP8 vs dequant-to-BF16"]: after the upcast the projection is
    an ordinary BF16 matrix product accumulated in F32, whose exact value is
    this sum.
    """
    return np.asarray(x, np.float32).astype(np.float64) @ np.asarray(wd, np.float32).astype(np.float64).T


def abs_bound_dense(x: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """sum_k |x_k * w_k| per output (float64), the scale of the dense arm's error bound."""
    return np.abs(np.asarray(x, np.float32).astype(np.float64)) @ np.abs(np.asarray(wd, np.float32).astype(np.float64)).T


def linear_dense_loops(x, wd) -> np.ndarray:
    """The dense product by plain Python loops (tiny inputs only)."""
    x = np.asarray(x, np.float32)
    wd = np.asarray(wd, np.float32)
    M, K = x.shape
    N = wd.shape[0]
    y = np.zeros((M, N), np.float64)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(x[m, k]) * float(wd[n, k])
            y[m, n] = acc
    return y


# ------------------------------------------------------- activation quantizer

def quant_act(x: np.ndarray, eps: np.float32 = ACT_EPS) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token 1x128 group quantization of X [M,K] -> (codes uint8 [M,K], scales f32 [M,Kb]).

    [W8A8 "WHY (#917 / #928)"]: per-token FP32 activation scales over groups of
    128 channels.  For token m and group g (channels 128g .. min(128g+128,K)):
      amax = max |x|                       (float32, exact)
      s    = fl32(max(amax, eps) / 448)    (IEEE float32 division)
      f    = fl32(x / s)                   (IEEE float32 division, per element)
      f    = clamp(f, -448, 448)           (saturating; E4M3 has no infinity)
      q    = RNE_E4M3(f)                   (``e4m3_encode``)
    Reading: the stored scale is the dequantization multiplier (x ~ dec(q)*s),
    the same convention as the weight grid; the tail group of a K that is not
    a multiple of 128 takes its amax over its valid channels only.
    """
    x = np.asarray(x, np.float32)
    M, K = x.shape
    Kb = -(-K // BLOCK)
    codes = np.empty((M, K), np.uint8)
    scales = np.empty((M, Kb), np.float32)
    for g in range(Kb):
        k0, k1 = g * BLOCK, min(K, g * BLOCK + BLOCK)
        xg = x[:, k0:k1]
        amax = np.max(np.abs(xg), axis=1) if k1 > k0 else np.zeros(M, np.float32)
        amax = np.maximum(amax, eps).astype(np.float32)
        s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
        f = (xg / s[:, None]).astype(np.float32)
        f = np.clip(f, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
        codes[:, k0:k1] = e4m3_encode(f)
        scales[:, g] = s
    return codes, scales


def exp_neg_abs_f32(g: np.ndarray) -> np.ndarray:
    """e = exp(-|g|) correctly rounded to float32 (nearest, ties to even), for float32 g.

    float64's exp (within a float64 ulp or two) rounded to float32 is the
    correctly rounded value unless exp(-|g|) lies near a float32 rounding
    midpoint; wherever the float64 value is within 2^-45 (relative) of one, the
    value is recomputed with Python's decimal module at 60 digits (its exp is
    correctly rounded at that precision) and compared with the midpoints
    exactly.  exp of a nonzero rational is irrational, so it is never a
    midpoint itself.
    """
    from decimal import Decimal, localcontext
    g = np.asarray(g, np.float32)
    a = np.abs(g.astype(np.float64))
    e64 = np.exp(-a)
    e32 = e64.astype(np.float32)
    up = np.nextafter(e32, np.float32(np.inf))
    dn = np.nextafter(e32, np.float32(0.0))
    m_up = (e32.astype(np.float64) + up.astype(np.float64)) / 2.0   # exact: both are float32
    m_dn = (e32.astype(np.float64) + dn.astype(np.float64)) / 2.0
    tol = 2.0 ** -45 * e64
    near = ((np.abs(e64 - m_up) <= tol) | ((np.abs(e64 - m_dn) <= tol) & (e32 > 0))) & (a > 0)
    if np.any(near):
        e32 = e32.copy()
        flat_a, flat_e = a.reshape(-1), e32.reshape(-1)
        flat_up, flat_dn = up.reshape(-1), dn.reshape(-1)
        with localcontext() as ctx:
            ctx.prec = 60
            for i in np.flatnonzero(near.reshape(-1)):
                ed = (-Decimal(float(flat_a[i]))).exp()
                c = flat_e[i]
                hi = (Decimal(float(c)) + Decimal(float(flat_up[i]))) / 2
                lo = (Decimal(float(c)) + Decimal(float(flat_dn[i]))) / 2
                if ed > hi:
                    flat_e[i] = flat_up[i]
                elif ed < lo and c > 0:
                    flat_e[i] = flat_dn[i]
        e32 = flat_e.reshape(e32.shape)
    return e32


def silu_glu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = silu(g) * u = g * sigmoid(g) * u as float32.

    [W8A8 "Module w8a8_prefill" preamble]: the arm is the dense FFN's
    gate/up/down prefill, in which the gate/up output reaches the down
    projection through the gated activation and the per-token quantizer.
    Reading: the pages do not name the activation; the gated SiLU of the
    Qwen dense FFN is taken.  Its steps are fixed so that the quantized codes
    (decided in float32) are reproducible and single-valued, in the
    overflow-free form: e = exp(-|g|) correctly rounded to float32 (in [0, 1],
    ``exp_neg_abs_f32``), t = 1 + e, then q = g / t for g >= 0 and
    q = (g * e) / t for g < 0, and h = q * u, each an IEEE float32 operation.
    """
    g = np.asarray(g, np.float32)
    u = np.asarray(u, np.float32)
    e = exp_neg_abs_f32(g)
    t = np.float32(1.0) + e
    q = np.where(g >= 0, g / t, (g * e) / t).astype(np.float32)
    return q * u


def glu_quant(y_gu: np.ndarray, F: int, eps: np.float32 = ACT_EPS) -> Tuple[np.ndarray, np.ndarray]:
    """The gate/up -> activation -> quantization step that feeds the down
    projection: y_gu [M, 2F] holds the gate outputs in columns [0, F) and the up
    outputs in [F, 2F) (the fused gate/up weight's member order); returns the
    down projection's quantized input (codes uint8 [M, F], scales f32 [M, ceil(F/128)]).

    [W8A8 "WHY (#917 / #928)"]: the down GEMM consumes per-token 1x128 E4M3
    activations; the activation values are ``silu_glu`` of the two halves.
    """
    y = np.asarray(y_gu, np.float32)
    if y.ndim != 2 or y.shape[1] < 2 * F:
        raise ValueError(f"y_gu {y.shape} does not hold 2F = {2 * F} columns")
    return quant_act(silu_glu(y[:, :F], y[:, F:2 * F]), eps)


def dequantize_act(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """A[m,k] = dec(codes[m,k]) * scales[m, k//128], float64 (exact)."""
    codes = np.asarray(codes, np.uint8)
    M, K = codes.shape
    s = np.repeat(np.asarray(scales, np.float32).astype(np.float64), BLOCK, axis=1)[:, :K]
    return e4m3_decode(codes) * s


# ------------------------------------------------------------------- W8A8

def linear_w8a8(xq: np.ndarray, xs: np.ndarray,
                members: Sequence[Tuple[np.ndarray, np.ndarray]]) -> np.ndarray:
    """Y = A . Wd^T in float64 with A = dequantize_act(xq, xs).

    [W8A8 "WHY (#917 / #928)"]: FP8 x FP8 products accumulated in FP32, each
    128-channel slice rescaled by activation scale x weight scale in an FP32
    epilogue.  Exactly, that sum is sum_kb sa*sw*sum_k dec(a)dec(w) = A . Wd^T.
    """
    return dequantize_act(xq, xs) @ dequantize_members(members).T


def linear_w8a16_rows(x, members, rows) -> np.ndarray:
    """Columns ``rows`` of ``linear_w8a16`` (float64 [M, len(rows)])."""
    return np.asarray(x, np.float32).astype(np.float64) @ dequantize_rows(members, rows).T


def linear_w8a8_rows(xq, xs, members, rows) -> np.ndarray:
    """Columns ``rows`` of ``linear_w8a8`` (float64 [M, len(rows)])."""
    return dequantize_act(xq, xs) @ dequantize_rows(members, rows).T


def abs_bound_w8a16_rows(x, members, rows) -> np.ndarray:
    return np.abs(np.asarray(x, np.float32).astype(np.float64)) @ np.abs(dequantize_rows(members, rows)).T


def abs_bound_w8a8_rows(xq, xs, members, rows) -> np.ndarray:
    return np.abs(dequantize_act(xq, xs)) @ np.abs(dequantize_rows(members, rows)).T


# ---------------------------------------------- brute force (tiny inputs only)

def linear_w8a16_loops(x, members) -> np.ndarray:
    """Pure-Python triple loop of the W8A16 definition, member by member, for tiny inputs."""
    x = np.asarray(x, np.float32)
    M, K = x.shape
    cols = []
    for codes, scale in members:
        N = codes.shape[0]
        for n in range(N):
            col = []
            for m in range(M):
                acc = 0.0
                for kb in range(-(-K // BLOCK)):
                    part = 0.0
                    for k in range(kb * BLOCK, min(K, kb * BLOCK + BLOCK)):
                        part += float(x[m, k]) * e4m3_value_py(int(codes[n, k]))
                    acc += part * float(scale[n // BLOCK, kb])
                col.append(acc)
            cols.append(col)
    return np.array(cols, np.float64).T


def e4m3_value_py(c: int) -> float:
    """E4M3 value of one code, from the bit fields (independent of the table)."""
    s = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 0xF, c & 7
    if e == 15 and m == 7:
        return math.nan
    return s * (m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10))


def w8a8_block_partial_int(a_codes: Sequence[int], w_codes: Sequence[int]) -> int:
    """Exact integer sum of one 128-channel block of code products, times 2^18.

    Each finite E4M3 value times 2^9 is an integer (m or (8+m)*2^(e-1)), so
    sum_k (2^9 dec(a_k)) (2^9 dec(w_k)) is an exact int (|sum| < 2^43 for 128 terms).
    """
    def as_int(c):
        e, m = (c >> 3) & 0xF, c & 7
        v = m if e == 0 else (8 + m) << (e - 1)
        return -v if c & 0x80 else v
    return sum(as_int(int(a)) * as_int(int(w)) for a, w in zip(a_codes, w_codes))


def linear_w8a8_loops(xq, xs, members) -> np.ndarray:
    """W8A8 by loops: exact integer block partials, then sum_kb P * 2^-18 * sa * sw."""
    xq = np.asarray(xq, np.uint8)
    M, K = xq.shape
    cols = []
    for codes, scale in members:
        N = codes.shape[0]
        for n in range(N):
            col = []
            for m in range(M):
                acc = 0.0
                for kb in range(-(-K // BLOCK)):
                    k0, k1 = kb * BLOCK, min(K, kb * BLOCK + BLOCK)
                    p = w8a8_block_partial_int(xq[m, k0:k1], codes[n, k0:k1])
                    acc += p * 2.0 ** -18 * float(xs[m, kb]) * float(scale[n // BLOCK, kb])
                col.append(acc)
            cols.append(col)
    return np.array(cols, np.float64).T


# ------------------------------------------------------- tolerance, metrics

def abs_bound_w8a16(x, members) -> np.ndarray:
    """sum_k |x_k * w_k| per output (float64), the scale of the W8A16 error bound."""
    return np.abs(np.asarray(x, np.float32).astype(np.float64)) @ np.abs(dequantize_members(members)).T


def abs_bound_w8a8(xq, xs, members) -> np.ndarray:
    """sum_k |a_k * w_k| per output with A the dequantized activation (float64)."""
    return np.abs(dequantize_act(xq, xs)) @ np.abs(dequantize_members(members)).T


def round_output(y64: np.ndarray, dtype: str) -> np.ndarray:
    """Output as a kernel writes it: 'f32' -> float32; 'bf16' -> RNE BF16 bits (uint16)."""
    y32 = np.asarray(y64, np.float64).astype(np.float32)
    if dtype == "f32":
        return y32
    if dtype == "bf16":
        return f32_to_bf16_bits(y32)
    raise ValueError(dtype)


def within_bound(y_test: np.ndarray, y_ref: np.ndarray, abs_sum: np.ndarray,
                 rel: float = 1e-3, bf16_out: bool = False) -> Tuple[bool, float]:
    """|y_test - y_ref| <= rel * sum_k|a_k w_k| (+ 2^-8 |y_ref| for BF16 outputs).

    Returns (ok, worst ratio err/bound).  The BF16 term is one half-ULP of a
    BF16 result, which the output rounding alone may spend.
    """
    err = np.abs(np.asarray(y_test, np.float64) - y_ref)
    bound = rel * abs_sum + (2.0 ** -8 * np.abs(y_ref) if bf16_out else 0.0)
    bound = np.maximum(bound, np.finfo(np.float32).tiny)
    ratio = err / bound
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    ok = bool(np.all(err <= bound)) and not np.isnan(err).any()
    return ok, worst


def cross_arm_metrics(y8: np.ndarray, y16: np.ndarray) -> Tuple[float, float]:
    """(cosine, relative RMS) of the W8A8 output against the W8A16 output, float64.

    [W8A8 "ACCURACY"]: the arms are compared by cosine similarity and by the
    relative RMS of their difference over the whole output.
    """
    a = np.asarray(y8, np.float64).ravel()
    b = np.asarray(y16, np.float64).ravel()
    cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
    rel = float(np.linalg.norm(a - b) / np.linalg.norm(b))
    return cos, rel


# ------------------------------------------------------------------ validator

class Status:
    """Refusal names, in precedence order within one member (see ``validate``)."""
    OK = "OK"
    INVALID_ARG = "INVALID_ARG"
    GROUP = "GROUP"
    DECL = "DECL"
    WEIGHT_E5M2 = "WEIGHT_E5M2"
    WEIGHT_DTYPE = "WEIGHT_DTYPE"
    WEIGHT_RANK = "WEIGHT_RANK"
    WEIGHT_EMPTY = "WEIGHT_EMPTY"
    SCALE_MISSING = "SCALE_MISSING"
    SCALE_AMBIGUOUS = "SCALE_AMBIGUOUS"
    SCALE_ROWWISE = "SCALE_ROWWISE"
    SCALE_PER_TENSOR = "SCALE_PER_TENSOR"
    SCALE_RANK = "SCALE_RANK"
    SCALE_DTYPE = "SCALE_DTYPE"
    SCALE_TRANSPOSED = "SCALE_TRANSPOSED"
    SCALE_GRID = "SCALE_GRID"
    ALIGNMENT = "ALIGNMENT"


class TensorDesc:
    """Header-level view of a tensor: dtype name, shape, optional address (int)."""
    def __init__(self, dtype: str, shape: Sequence[int], addr: Optional[int] = None):
        self.dtype, self.shape, self.addr = dtype, tuple(int(s) for s in shape), addr


class MemberDesc:
    """One grouped member: its weight and its two possible scale leaves.

    ``scale_inv`` is the block grid leaf (``weight_scale_inv``); ``scale`` is
    the row-wise / per-tensor leaf (``weight_scale``) of other FP8 layouts.
    """
    def __init__(self, weight: TensorDesc, scale_inv: Optional[TensorDesc] = None,
                 scale: Optional[TensorDesc] = None):
        self.weight, self.scale_inv, self.scale = weight, scale_inv, scale


def validate(quant_method: str, block: Sequence[int], members: Sequence[MemberDesc],
             max_members: int = 8) -> str:
    """Header-only geometry validation; returns the single refusal name (or OK).

    Refusals are the ones the pages list: [QWEN operator paragraph] E5M2
    encodings, ambiguous row/block scales, malformed grids, incompatible
    declarations; [TH1803 "Why the refusals matter"] row-wise trees, transposed
    or mis-blocked grids, FP8 weights without a scale, rank-1 scales, configs
    that disagree with the bytes; [TH1803 "Proof"] dense trees.  Nothing here
    reads tensor data ([TH1803 "What lands"]: headers alone).

    Precedence (so every bad input has exactly one name):
      1. member count outside 1..max_members            -> GROUP
      2. declaration not (fp8, [128,128])               -> DECL
      3. members in index order; within a member:
         WEIGHT_E5M2, WEIGHT_DTYPE (not F8_E4M3), WEIGHT_RANK (not 2),
         WEIGHT_EMPTY (a zero dimension), SCALE_MISSING (no leaf),
         SCALE_AMBIGUOUS (both leaves), SCALE_ROWWISE (a rank-1 leaf),
         SCALE_PER_TENSOR (a rank-0 ``weight_scale``), SCALE_RANK (any other
         rank but 2), SCALE_DTYPE (not BF16/F32), SCALE_TRANSPOSED (shape
         [Kb,Nb] != [Nb,Kb]), SCALE_GRID (any other shape than [Nb,Kb]; also a
         rank-2 leaf under the ``weight_scale`` name, which is not a block grid)
      4. across members: K differs, or scale dtypes differ -> GROUP
      5. a given address not 16-byte aligned (weight) or not aligned to the
         scale element (scale)                           -> ALIGNMENT
    Reading: when Nb == Kb a transposed grid has the right shape and cannot be
    told apart from headers; it is accepted.

    Per-tensor layout ([FP8 "The two FP8 checkpoint shapes"]: E4M3 weight plus
    one weight_scale per tensor, read as the degenerate block case).  Reading:
    the pages do not say how such a checkpoint declares itself; it is taken to
    be quant_method fp8 without a weight_block_size, written block (0, 0).
    Under that declaration each member needs a ``weight_scale`` leaf holding
    one value (rank 0, or rank 1 of shape [1]); a ``weight_scale_inv`` grid
    disagrees with the declaration (DECL), a rank-1 leaf of more than one
    value is row-wise (SCALE_ROWWISE), a higher rank is SCALE_RANK, and the
    dtype must be BF16 or F32.  The weight checks are the same.
    """
    S = Status
    if len(members) < 1 or len(members) > max_members:
        return S.GROUP
    blk = tuple(int(b) for b in block)
    per_tensor = quant_method == "fp8" and blk == (0, 0)
    if quant_method != "fp8" or (blk != (BLOCK, BLOCK) and not per_tensor):
        return S.DECL
    for m in members:
        w = m.weight
        if w.dtype == "F8_E5M2":
            return S.WEIGHT_E5M2
        if w.dtype != "F8_E4M3":
            return S.WEIGHT_DTYPE
        if len(w.shape) != 2:
            return S.WEIGHT_RANK
        if w.shape[0] <= 0 or w.shape[1] <= 0:
            return S.WEIGHT_EMPTY
        if m.scale_inv is None and m.scale is None:
            return S.SCALE_MISSING
        if m.scale_inv is not None and m.scale is not None:
            return S.SCALE_AMBIGUOUS
        leaf = m.scale_inv if m.scale_inv is not None else m.scale
        rank = len(leaf.shape)
        if per_tensor:
            if m.scale_inv is not None:
                return S.DECL
            if rank == 1 and leaf.shape[0] != 1:
                return S.SCALE_ROWWISE
            if rank > 1:
                return S.SCALE_RANK
            if leaf.dtype not in ("BF16", "F32"):
                return S.SCALE_DTYPE
            continue
        if rank == 1:
            return S.SCALE_ROWWISE
        if rank == 0 and m.scale is not None:
            return S.SCALE_PER_TENSOR
        if rank != 2:
            return S.SCALE_RANK
        if leaf.dtype not in ("BF16", "F32"):
            return S.SCALE_DTYPE
        nb, kb = scale_grid_shape(*w.shape)
        if leaf.shape != (nb, kb) and leaf.shape == (kb, nb):
            return S.SCALE_TRANSPOSED
        if leaf.shape != (nb, kb) or m.scale is not None:
            return S.SCALE_GRID
    def leaf_of(m):
        return m.scale_inv if m.scale_inv is not None else m.scale
    k0 = members[0].weight.shape[1]
    dt0 = leaf_of(members[0]).dtype
    for m in members[1:]:
        if m.weight.shape[1] != k0 or leaf_of(m).dtype != dt0:
            return S.GROUP
    for m in members:
        if m.weight.addr is not None and m.weight.addr % 16 != 0:
            return S.ALIGNMENT
        esz = 2 if leaf_of(m).dtype == "BF16" else 4
        if leaf_of(m).addr is not None and leaf_of(m).addr % esz != 0:
            return S.ALIGNMENT
    return S.OK

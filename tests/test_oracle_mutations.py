"""Planted mistakes in the oracle, on the CPU: each must make some pin fail.

This shows the pins are strong enough to catch a dropped term, a wrong sign,
a transposed grid or a wrong rounding rule anywhere in the oracle.
"""
import math

import numpy as np
import pytest

import oracle.bsf8_oracle as OM
import oracle_pins as P


def _fails(pin, O):
    ok, _ = pin(O)
    return not ok


def test_pin_quant_brute_force_passes():
    ok, detail = P.pin_quant_brute_force(OM)
    assert ok, detail


def test_mutation_divide_instead_of_multiply(monkeypatch):
    orig = OM.dequantize_block_scaled

    def divided(codes, scale):
        N, K = codes.shape
        s = np.repeat(np.repeat(np.asarray(scale, np.float64), 128, 0)[:N], 128, 1)[:, :K]
        return OM.e4m3_decode(codes) / s
    monkeypatch.setattr(OM, "dequantize_block_scaled", divided)
    assert _fails(P.pin_scale_direction, OM)
    monkeypatch.setattr(OM, "dequantize_block_scaled", orig)
    assert not _fails(P.pin_scale_direction, OM)


def test_mutation_per_tensor_reciprocal(monkeypatch):
    """A per-tensor scale used as a reciprocal fails the per-tensor pin."""
    orig = OM.dequantize_per_tensor
    monkeypatch.setattr(OM, "dequantize_per_tensor",
                        lambda codes, scale: OM.e4m3_decode(codes) / float(np.asarray(scale, np.float32).reshape(())))
    assert _fails(P.pin_per_tensor, OM)
    monkeypatch.setattr(OM, "dequantize_per_tensor", orig)
    assert not _fails(P.pin_per_tensor, OM)


def test_mutation_wrong_bias(monkeypatch):
    t = OM.e4m3_table() * 2.0
    monkeypatch.setattr(OM, "e4m3_table", lambda: t.copy())
    assert _fails(P.pin_lut_closed_form, OM)


def test_mutation_ties_away_from_zero(monkeypatch):
    def enc(f):
        f = np.asarray(f, np.float32)
        a = np.abs(f.astype(np.float64))
        sign = np.where(np.signbit(f), 0x80, 0)
        mant, exp = np.frexp(a)
        t, e = mant * 2.0, exp - 1
        mq = np.floor((t - 1.0) * 8.0 + 0.5).astype(np.int64)
        e = np.where(mq == 8, e + 1, e)
        mq = np.where(mq == 8, 0, mq)
        sub = np.floor(a * 512 + 0.5).astype(np.int64)
        return (np.where(a >= 2 ** -6, ((e + 7) << 3) | mq, sub) | sign).astype(np.uint8)
    monkeypatch.setattr(OM, "e4m3_encode", enc)
    assert _fails(P.pin_worked_ties, OM)
    assert _fails(P.pin_encode_vs_torch, OM)


def test_mutation_lost_negative_zero(monkeypatch):
    orig = OM.e4m3_encode
    monkeypatch.setattr(OM, "e4m3_encode", lambda f: np.where(np.asarray(f) == 0, 0, orig(f)).astype(np.uint8))
    assert _fails(P.pin_roundtrip, OM)


def test_mutation_reciprocal_multiply_in_quant(monkeypatch):
    def quant(x, eps=OM.ACT_EPS):
        x = np.asarray(x, np.float32)
        M, K = x.shape
        Kb = -(-K // 128)
        q = np.empty((M, K), np.uint8)
        s_all = np.empty((M, Kb), np.float32)
        for g in range(Kb):
            xg = x[:, g * 128:(g + 1) * 128]
            s = (np.maximum(np.abs(xg).max(1), eps) / np.float32(448)).astype(np.float32)
            inv = (np.float32(1) / s).astype(np.float32)
            f = np.clip((xg * inv[:, None]).astype(np.float32), -448, 448)
            q[:, g * 128:(g + 1) * 128] = OM.e4m3_encode(f)
            s_all[:, g] = s
        return q, s_all
    monkeypatch.setattr(OM, "quant_act", quant)
    assert _fails(P.pin_quant_brute_force, OM)


def test_mutation_global_grid_for_grouped_members(monkeypatch):
    def members_global(members):
        codes = np.concatenate([c for c, _ in members])
        scales = np.concatenate([s for _, s in members])
        N, K = codes.shape
        s = np.repeat(np.repeat(scales.astype(np.float64), 128, 0), 128, 1)
        s = s[:N, :K] if s.shape[0] >= N else np.pad(s, ((0, N - s.shape[0]), (0, 0)), mode="edge")[:N, :K]
        return OM.e4m3_decode(codes) * s
    monkeypatch.setattr(OM, "dequantize_members", members_global)
    assert _fails(P.pin_brute_force, OM)


def test_mutation_dropped_tail_block(monkeypatch):
    orig = OM.dequantize_act

    def drop(codes, scales):
        a = orig(codes, scales)
        K = a.shape[1]
        a[:, (K // 128) * 128:] = 0.0
        return a
    monkeypatch.setattr(OM, "dequantize_act", drop)
    assert _fails(P.pin_brute_force, OM)


def test_mutation_transposed_operand(monkeypatch):
    orig = OM.dequantize_block_scaled

    def transposed_scale(codes, scale):
        N, K = codes.shape
        s = np.asarray(scale, np.float64)
        st = np.resize(s.T, s.shape)
        sf = np.repeat(np.repeat(st, 128, 0)[:N], 128, 1)[:, :K]
        return OM.e4m3_decode(codes) * sf
    monkeypatch.setattr(OM, "dequantize_block_scaled", transposed_scale)
    assert _fails(P.pin_brute_force, OM)


def test_mutation_bf16_truncation(monkeypatch):
    monkeypatch.setattr(OM, "f32_to_bf16_bits",
                        lambda x: (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16))
    assert _fails(P.pin_bf16, OM)


def test_mutation_scale_grid_floor(monkeypatch):
    monkeypatch.setattr(OM, "scale_grid_shape", lambda n, k, block=(128, 128): (n // 128, k // 128))
    assert _fails(P.pin_grids, OM)


def test_mutation_upcast_single_rounding(monkeypatch):
    """A BF16 copy rounded once from the exact product fails the upcast pin."""
    orig = OM.upcast_members

    def once(members, dtype):
        if dtype != "bf16":
            return orig(members, dtype)
        m, e = np.frexp(OM.dequantize_members(members))
        v = (np.round(m * 256.0) * np.exp2(e - 8.0)).astype(np.float32)   # exact: 8 significant bits
        return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    monkeypatch.setattr(OM, "upcast_members", once)
    assert _fails(P.pin_upcast, OM)
    monkeypatch.setattr(OM, "upcast_members", orig)
    assert not _fails(P.pin_upcast, OM)


def test_mutation_upcast_member_grid(monkeypatch):
    """A dense copy that scales every member with the first member's grid fails the upcast pin."""
    orig = OM.upcast_members

    def shared(members, dtype):
        s0 = members[0][1]
        fixed = [(c, s0[:-(-c.shape[0] // 128)]) if s0.shape[0] >= -(-c.shape[0] // 128) else (c, s) for c, s in members]
        return orig(fixed, dtype)
    monkeypatch.setattr(OM, "upcast_members", shared)
    assert _fails(P.pin_upcast, OM)


def test_mutation_dense_transposed(monkeypatch):
    """Summing over the wrong weight index fails the dense brute-force pin."""
    monkeypatch.setattr(OM, "linear_dense", lambda x, wd: np.asarray(x, np.float64) @ np.asarray(wd, np.float64)[:, ::-1].T)
    assert _fails(P.pin_dense_brute_force, OM)


def test_mutation_silu_sign_of_exponent(monkeypatch):
    """exp(+|g|) in place of exp(-|g|) fails the activation pin."""
    orig = OM.silu_glu

    def wrong(g, u):
        g = np.asarray(g, np.float32)
        with np.errstate(over="ignore", invalid="ignore"):
            e = np.exp(np.abs(g.astype(np.float64))).astype(np.float32)
            t = np.float32(1) + e
            return np.where(g >= 0, g / t, (g * e) / t).astype(np.float32) * np.asarray(u, np.float32)
    monkeypatch.setattr(OM, "silu_glu", wrong)
    assert _fails(P.pin_silu_glu, OM)
    monkeypatch.setattr(OM, "silu_glu", orig)
    assert not _fails(P.pin_silu_glu, OM)


def test_mutation_silu_negative_branch(monkeypatch):
    """Using g / t for negative g as well (sigmoid of |g|) fails the activation pin."""
    def wrong(g, u):
        g = np.asarray(g, np.float32)
        e = np.exp(-np.abs(g.astype(np.float64))).astype(np.float32)
        return g / (np.float32(1) + e) * np.asarray(u, np.float32)
    monkeypatch.setattr(OM, "silu_glu", wrong)
    assert _fails(P.pin_silu_glu, OM)


def test_mutation_glu_halves_swapped(monkeypatch):
    """The gate taken from the up half (silu applied to the wrong operand) fails the activation pin."""
    orig = OM.silu_glu
    monkeypatch.setattr(OM, "silu_glu", lambda g, u: orig(u, g))
    assert _fails(P.pin_silu_glu, OM)


# ------------------------------------------- tolerance and metric helpers

def test_mutation_bound_abs_of_sum(monkeypatch):
    """|sum_k a_k w_k| in place of sum_k |a_k w_k| fails the bound pin."""
    monkeypatch.setattr(OM, "abs_bound_w8a16", lambda x, members: np.abs(OM.linear_w8a16(x, members)))
    assert _fails(P.pin_abs_bounds, OM)


def test_mutation_bound_missing_activation_abs(monkeypatch):
    """Dropping |.| on the dequantized activation of the W8A8 bound fails the bound pin."""
    monkeypatch.setattr(OM, "abs_bound_w8a8",
                        lambda xq, xs, members: OM.dequantize_act(xq, xs) @ np.abs(OM.dequantize_members(members)).T)
    assert _fails(P.pin_abs_bounds, OM)


def test_mutation_bound_rows_use_global_grid(monkeypatch):
    """A row form that takes the scale row n // 128 of the stacked grids fails the bound pin."""
    def rows_global(xq, xs, members, rows):
        codes = np.concatenate([c for c, _ in members])
        sc = np.concatenate([s for _, s in members])
        K = codes.shape[1]
        w = np.stack([OM.e4m3_decode(codes[n]) * np.repeat(sc[min(n // 128, sc.shape[0] - 1)], 128)[:K] for n in rows])
        return np.abs(OM.dequantize_act(xq, xs)) @ np.abs(w).T
    monkeypatch.setattr(OM, "abs_bound_w8a8_rows", rows_global)
    assert _fails(P.pin_abs_bounds, OM)


def test_mutation_within_bound_loose_factor(monkeypatch):
    """A tolerance of 2e-3 in place of 1e-3 fails the acceptance pin."""
    orig = OM.within_bound
    monkeypatch.setattr(OM, "within_bound", lambda y, r, s, rel=1e-3, bf16_out=False: orig(y, r, s, 2e-3, bf16_out))
    assert _fails(P.pin_within_bound, OM)


def test_mutation_within_bound_full_ulp(monkeypatch):
    """A whole BF16 ULP (2^-7 |y|) in place of half of one fails the acceptance pin."""
    def loose(y_test, y_ref, abs_sum, rel=1e-3, bf16_out=False):
        err = np.abs(np.asarray(y_test, np.float64) - y_ref)
        bound = np.maximum(rel * abs_sum + (2.0 ** -7 * np.abs(y_ref) if bf16_out else 0.0), np.finfo(np.float32).tiny)
        return bool(np.all(err <= bound)) and not np.isnan(err).any(), float(np.nanmax(err / bound))
    monkeypatch.setattr(OM, "within_bound", loose)
    assert _fails(P.pin_within_bound, OM)


def test_mutation_within_bound_ignores_nan(monkeypatch):
    """An acceptance test that skips NaN elements fails the acceptance pin."""
    def nan_blind(y_test, y_ref, abs_sum, rel=1e-3, bf16_out=False):
        err = np.abs(np.asarray(y_test, np.float64) - y_ref)
        bound = np.maximum(rel * abs_sum + (2.0 ** -8 * np.abs(y_ref) if bf16_out else 0.0), np.finfo(np.float32).tiny)
        keep = ~np.isnan(err)
        return bool(np.all(err[keep] <= bound[keep])), float(np.nanmax(err / bound))
    monkeypatch.setattr(OM, "within_bound", nan_blind)
    assert _fails(P.pin_within_bound, OM)


def test_mutation_cross_arm_wrong_denominator(monkeypatch):
    """Relative RMS over the W8A8 output's norm fails the metrics pin."""
    def wrong(y8, y16):
        a, b = np.ravel(y8).astype(np.float64), np.ravel(y16).astype(np.float64)
        return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b))), float(np.linalg.norm(a - b) / np.linalg.norm(a))
    monkeypatch.setattr(OM, "cross_arm_metrics", wrong)
    assert _fails(P.pin_cross_arm_metrics, OM)


def test_mutation_cross_arm_mean_of_rows(monkeypatch):
    """Metrics averaged over rows instead of over the whole output fail the metrics pin."""
    orig = OM.cross_arm_metrics

    def per_row(y8, y16):
        y8, y16 = np.atleast_2d(y8), np.atleast_2d(y16)
        vals = [orig(a, b) for a, b in zip(y8, y16)]
        return float(np.mean([v[0] for v in vals])), float(np.mean([v[1] for v in vals]))
    monkeypatch.setattr(OM, "cross_arm_metrics", per_row)
    assert _fails(P.pin_cross_arm_metrics, OM)


def test_mutation_cross_arm_unnormalised_cosine(monkeypatch):
    """A cosine normalised by the W8A16 norm squared fails the metrics pin."""
    def wrong(y8, y16):
        a, b = np.ravel(y8).astype(np.float64), np.ravel(y16).astype(np.float64)
        return float(a @ b / (b @ b)), float(np.linalg.norm(a - b) / np.linalg.norm(b))
    monkeypatch.setattr(OM, "cross_arm_metrics", wrong)
    assert _fails(P.pin_cross_arm_metrics, OM)


def test_mutation_exp_in_float32(monkeypatch):
    """exp evaluated in float32 (a float32 library exp, not correctly rounded) fails the exp pin."""
    monkeypatch.setattr(OM, "exp_neg_abs_f32", lambda g: np.exp(-np.abs(np.asarray(g, np.float32))))
    assert _fails(P.pin_exp_correctly_rounded, OM)


def test_mutation_exp_rounded_down(monkeypatch):
    """exp rounded toward zero instead of to nearest fails the exp pin."""
    def trunc(g):
        e64 = np.exp(-np.abs(np.asarray(g, np.float32).astype(np.float64)))
        e32 = e64.astype(np.float32)
        return np.where(e32.astype(np.float64) > e64, np.nextafter(e32, np.float32(0)), e32).astype(np.float32)
    monkeypatch.setattr(OM, "exp_neg_abs_f32", trunc)
    assert _fails(P.pin_exp_correctly_rounded, OM)

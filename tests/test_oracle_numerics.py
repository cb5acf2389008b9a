"""Pins for oracle.numerics against what the formats' definitions and independent
library routines fix (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import numerics as nm


def _rand_f32(n, seed=0, scale=3.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(n) * scale).astype(np.float32)


# ----------------------------------------------------------------------------- bf16

def test_bf16_roundtrip_matches_torch():
    x = np.concatenate([_rand_f32(20000, 1), _rand_f32(2000, 2, 1e-30), _rand_f32(2000, 3, 1e30)])
    # exact ties: fp32 patterns whose low 16 bits are exactly 0x8000
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties]).astype(np.float32)
    ours = nm.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = nm.bf16_to_f32(ours)
    ref_back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(back, ref_back)


# ----------------------------------------------------------------------------- INT4 asymmetric

def _bf16_groups(n, seed, scale=1.0, shift=0.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((n, 32)) * scale + shift).astype(np.float32)
    return nm.bf16_to_f32(nm.f32_to_bf16(x))


def test_int4_codes_are_nearest_level_by_exhaustive_search():
    """Brute force: each code must be a level c in 0..15 minimising |x - (s16*c + m16)| in
    exact arithmetic.  At an exact tie between two levels the even code is taken
    (round half to even); away from ties the nearest level is unique and must match."""
    x = _bf16_groups(3000, 10, scale=1.5, shift=0.3)
    codes, s16, m16 = nm.quant_asym(x, 15)
    s = s16.astype(np.float64)[:, None]
    m = m16.astype(np.float64)[:, None]
    levels = s[..., None] * np.arange(16)[None, None, :] + m[..., None]
    err = np.abs(x.astype(np.float64)[..., None] - levels)
    ec = np.take_along_axis(err, codes[..., None].astype(np.int64), -1)[..., 0]
    emin = err.min(-1)
    assert np.all(ec <= emin + 1e-15)
    ties = (np.sort(err, -1)[..., 1] - emin) <= 1e-15
    assert np.all(codes[ties] % 2 == 0)
    assert np.array_equal(codes[~ties], err.argmin(-1)[~ties])


def test_int4_min_max_constant_and_grid():
    x = _bf16_groups(2000, 11, scale=2.0)
    codes, s16, m16 = nm.quant_asym(x, 15)
    assert codes.min() >= 0 and codes.max() <= 15
    rows = np.arange(len(x))
    assert np.all(codes[rows, x.argmin(1)] == 0)
    assert np.all(codes[rows, x.argmax(1)] == 15)
    # a constant group is exact
    c = np.full((4, 32), 0.8125, np.float32)
    cc, cs, cm = nm.quant_asym(c, 15)
    assert np.all(cc == 0) and np.all(cs == 0)
    assert np.array_equal(nm.dequant_asym(cc, cs, cm), c)
    # values on a power-of-two grid come back exactly
    rng = np.random.default_rng(3)
    lv = rng.integers(0, 16, size=(50, 32))
    lv[:, 0], lv[:, 1] = 0, 15
    g = (0.25 * lv - 1.5).astype(np.float32)
    gc, gs, gm = nm.quant_asym(g, 15)
    assert np.array_equal(gc, lv)
    assert np.array_equal(nm.dequant_asym(gc, gs, gm), g)


def test_int4_error_bound_and_scale():
    x = _bf16_groups(3000, 12, scale=0.7, shift=-2.0)
    codes, s16, m16 = nm.quant_asym(x, 15)
    xh = nm.dequant_asym(codes, s16, m16).astype(np.float64)
    s = s16.astype(np.float64)[:, None]
    ulp = np.spacing(np.abs(x)).astype(np.float64)
    assert np.all(np.abs(x - xh) <= s / 2 + 2 * ulp)
    # s16 is within one fp16 rounding of the exact range / 15
    exact = (x.max(1).astype(np.float64) - x.min(1)) / 15
    assert np.all(np.abs(s16.astype(np.float64) - exact) <= np.spacing(s16).astype(np.float64) / 2 + 1e-12 * exact)
    # deterministic
    c2, s2, m2 = nm.quant_asym(x, 15)
    assert np.array_equal(c2, codes) and np.array_equal(s2.view(np.uint16), s16.view(np.uint16))


def test_int4_token_grouping():
    rng = np.random.default_rng(4)
    x = nm.bf16_to_f32(nm.f32_to_bf16(rng.standard_normal((5, 128)).astype(np.float32)))
    c, s, m = nm.quant_int4_token(x)
    assert c.shape == (5, 128) and s.shape == (5, 4)
    for gi in range(4):  # each 32-channel group on its own
        cg, sg, mg = nm.quant_asym(x[:, 32 * gi:32 * gi + 32], 15)
        assert np.array_equal(c[:, 32 * gi:32 * gi + 32], cg)
    xh = nm.dequant_int4_token(c, s, m)
    assert np.max(np.abs(xh - x)) <= np.max(s.astype(np.float32)) / 2 + 1e-6


# ----------------------------------------------------------------------------- INT8 symmetric

def test_int8_sym():
    rng = np.random.default_rng(5)
    x = nm.bf16_to_f32(nm.f32_to_bf16((rng.standard_normal((64, 128)) * 2).astype(np.float32)))
    q, s = nm.quant_int8_sym(x)
    i = np.unravel_index(np.abs(x).argmax(), x.shape)
    assert abs(int(q[i])) == 127 and np.sign(q[i]) == np.sign(x[i])
    assert np.all(np.abs(x - s * q.astype(np.float32)) <= s / 2 * (1 + 1e-6))
    assert np.all(np.abs(q.astype(int)) <= 127)
    z, zs = nm.quant_int8_sym(np.zeros((3, 4), np.float32))
    assert zs == 0 and np.all(z == 0)


# ----------------------------------------------------------------------------- OCP FP8 E4M3

def test_e4m3_table_fixed_points():
    t = nm.e4m3_decode_table()
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0x01] == 2.0 ** -9
    assert t[0x08] == 2.0 ** -6 and t[0x07] == 7 * 2.0 ** -9
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0xB8] == -1.0 and np.nanmax(t) == 448.0
    pos = t[:127]
    assert np.all(np.diff(pos) > 0)  # monotone non-negative codes


def test_e4m3_encode_exhaustive_bf16_vs_torch():
    """All 65,536 bf16 inputs with |x| <= 448 against torch's float8_e4m3fn conversion
    (round to nearest even)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = nm.bf16_to_f32(bits)
    keep = np.isfinite(x) & (np.abs(x) <= 448)
    x = x[keep]
    ours = nm.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of -0 and of negative values that round to zero; so do we
    assert np.array_equal(ours, ref)
    fast = nm.e4m3_round_fast(x)
    slow = nm.e4m3_value(ours)
    assert np.array_equal(fast, slow)


def test_e4m3_ties_and_saturation():
    # midpoint between 1.0 (0x38) and 1.125 (0x39) -> even code 0x38; between 1.125 and 1.25 -> 0x3A
    assert nm.e4m3_encode(np.array([1.0625]))[0] == 0x38
    assert nm.e4m3_encode(np.array([1.1875]))[0] == 0x3A
    assert nm.e4m3_encode(np.array([1e6]))[0] == 0x7E
    assert nm.e4m3_encode(np.array([-1e6]))[0] == 0xFE
    rng = np.random.default_rng(6)
    r = rng.uniform(-460, 460, 20000)
    assert np.array_equal(nm.e4m3_round_fast(r), nm.e4m3_round(r))


# ----------------------------------------------------------------------------- FP4 E2M1 and MX

def test_e2m1_table_is_the_format():
    """E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, exponent 0 subnormal."""
    t = nm.e2m1_decode_table()
    assert list(t[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(t[8:]) == [-v for v in t[:8]]


def test_e2m1_encode_nearest_ties_even_saturating():
    vals = nm.e2m1_decode_table()
    # every code round-trips (the negative zero code included)
    assert np.array_equal(nm.e2m1_encode(vals), np.arange(16, dtype=np.uint8))
    x = np.concatenate([np.arange(-8.0, 8.0, 1.0 / 64), _rand_f32(3000, 11, 2.0)]).astype(np.float32)
    c = nm.e2m1_encode(x)
    v = nm.e2m1_value(c)
    mags = vals[:8]
    for xi, vi, ci in zip(x.astype(np.float64), v, c):
        a = min(abs(xi), 6.0)
        gap = np.abs(mags - a)
        assert abs(abs(vi) - a) == gap.min()          # a nearest magnitude
        if np.count_nonzero(gap == gap.min()) == 2:   # exact midpoint: even mantissa bit
            assert (ci & 1) == 0
        assert (ci >= 8) == bool(np.signbit(xi))      # sign kept
    # monotone in the value
    order = np.argsort(x, kind="stable")
    assert np.all(np.diff(v[order]) >= 0)


def test_mxfp4_block_scale_rule():
    rng = np.random.default_rng(5)
    for trial in range(300):
        x = (rng.standard_normal(32) * 10.0 ** rng.uniform(-6, 6)).astype(np.float32)
        if trial % 50 == 0:
            x[:] = 0.0
        codes, e = nm.mxfp4_quant_block(x)
        amax = float(np.abs(x).max())
        if amax == 0.0:
            assert e == -127 and np.all(codes % 8 == 0)
            continue
        # the block maximum lands in [4, 8) after the division by the shared scale
        assert 4.0 <= amax / 2.0 ** e < 8.0
        # every element is the nearest E2M1 value to x / 2^e (saturating at 6)
        ratio = x.astype(np.float64) / 2.0 ** e
        err = np.abs(nm.e2m1_value(codes) - np.clip(ratio, -6, 6))
        assert np.all(err <= 1.0 + 1e-12)  # half the widest gap (4 -> 6)
    # the vectorised row quantizer is the same rule (a different code path)
    X = (rng.standard_normal((7, 128)) * np.array([1e-5, 1e-2, 1, 3, 100, 1e4, 0])[:, None]).astype(np.float32)
    c, e = nm.mxfp4_quant_rows(X)
    for r in range(7):
        for b in range(4):
            cb, eb = nm.mxfp4_quant_block(X[r, 32 * b:32 * b + 32])
            assert eb == e[r, b] and np.array_equal(cb, c[r, 32 * b:32 * b + 32])


def test_int8_bulk_codes_are_nearest_level_by_exhaustive_search():
    """The 8-bit bulk (255 levels): brute force over the 256 levels, ties to the even code;
    the group minimum maps to 0 and the maximum to 255 (up to the fp16 rounding of s and m)."""
    x = _bf16_groups(1500, 11, scale=2.0, shift=-0.7)
    codes, s16, m16 = nm.quant_int4_token(x, 32, bits=8)
    s = s16.astype(np.float64)[:, 0:1]
    m = m16.astype(np.float64)[:, 0:1]
    levels = s[..., None] * np.arange(256)[None, None, :] + m[..., None]
    err = np.abs(x.astype(np.float64)[..., None] - levels)
    ec = np.take_along_axis(err, codes[..., None].astype(np.int64), -1)[..., 0]
    emin = err.min(-1)
    assert np.all(ec <= emin + 1e-15)
    ties = (np.sort(err, -1)[..., 1] - emin) <= 1e-15
    assert np.all(codes[ties] % 2 == 0)
    assert np.array_equal(codes[~ties], err.argmin(-1)[~ties])
    assert codes.max() == 255 and (codes.min(axis=1) <= 1).all() and (codes.max(axis=1) >= 254).all()
    # the error of the dequantized value is at most half a step, 17x finer than 15 levels
    xh = nm.dequant_asym(codes, s16[:, 0], m16[:, 0]).astype(np.float64)
    assert np.all(np.abs(xh - x) <= 0.5 * s * (1 + 1e-3) + 1e-12)


def test_2bit_codes_are_nearest_level_by_exhaustive_search():
    """The 2-bit bulk (3 levels, the B = 2 of Alg. 3/4's bit-width parameters): brute force
    over the 4 levels, ties to the even code; every group uses both end levels (the minimum
    maps to 0, the maximum to 3, up to the fp16 rounding of s and m)."""
    x = _bf16_groups(2000, 12, scale=0.8, shift=0.2)
    codes, s16, m16 = nm.quant_int4_token(x, 32, bits=2)
    s = s16.astype(np.float64)[:, 0:1]
    m = m16.astype(np.float64)[:, 0:1]
    levels = s[..., None] * np.arange(4)[None, None, :] + m[..., None]
    err = np.abs(x.astype(np.float64)[..., None] - levels)
    ec = np.take_along_axis(err, codes[..., None].astype(np.int64), -1)[..., 0]
    emin = err.min(-1)
    assert np.all(ec <= emin + 1e-15)
    ties = (np.sort(err, -1)[..., 1] - emin) <= 1e-15
    assert np.all(codes[ties] % 2 == 0)
    assert np.array_equal(codes[~ties], err.argmin(-1)[~ties])
    assert codes.max() == 3 and (codes.min(axis=1) == 0).all() and (codes.max(axis=1) >= 2).all()
    xh = nm.dequant_asym(codes, s16[:, 0], m16[:, 0]).astype(np.float64)
    assert np.all(np.abs(xh - x) <= 0.5 * s * (1 + 1e-3) + 1e-12)
    # a hand case: values on the three steps of [0, 3] and a midpoint between codes 1 and 2
    y = np.zeros((1, 32), np.float32)
    y[0, :4] = [0.0, 1.0, 2.0, 3.0]
    y[0, 4] = 1.5
    c, s1, m1 = nm.quant_int4_token(y, 32, bits=2)
    assert float(s1[0, 0]) == 1.0 and float(m1[0, 0]) == 0.0
    assert list(c[0, :5]) == [0, 1, 2, 3, 2]  # 1.5 is a tie: the even code

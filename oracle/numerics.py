"""Number formats and quantizers of the oracle (test infrastructure only).

Citations refer to the HyQuant paper (arXiv page "HyQuant: Hybrid-Precision
Quantization for LLM Attention").

Every quantizer here runs in IEEE fp32 through numpy in the exact operation order
written in its docstring, so that integer codes are a deterministic function of
the input bits.  Where the pages leave the arithmetic open, the docstring states the
reading taken.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

# ----------------------------------------------------------------------------- bf16


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even.

    Written from the definition: keep the top 16 bits of the fp32 pattern and round
    on the 16 discarded bits (above half: up; exactly half: to the even result).
    NaN maps to the canonical quiet NaN 0x7FC0.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    hi = u >> 16
    lo = u & 0xFFFF
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    out = (hi + up.astype(np.uint64)).astype(np.uint16)
    out[np.isnan(x)] = 0x7FC0
    return out


# ----------------------------------------------------------------------------- INT4 / b-bit asymmetric


def quant_asym(x, levels: int = 15):
    """Asymmetric group quantizer over the last axis (one group = the whole last axis).

    HyQuant paper, Alg. 4 (Quant with group size G) and §5.1 (K4V4): the pages fix the
    bit width and that quantization is per group, not the arithmetic.  Reading taken
    (asymmetric min/scale form x ~ s*q + m, 32-channel groups per token):

      1. mn = min(x), mx = max(x)                      (fp32, exact from bf16)
      2. s32 = (mx - mn) / levels                      (IEEE fp32 subtract, divide)
      3. s16 = fp16(s32), m16 = fp16(mn)               (round to nearest even)
      4. if s16 == 0: every code is 0
         else code = clamp(rint((x - m16) / s16), 0, levels)   (fp32 ops, rint = half-even)

    Returns (codes uint8, s16 float16, m16 float16); codes has x's shape, s16/m16 drop
    the last axis.  The dequantized value is ``dequant_asym``.
    """
    x = np.asarray(x, dtype=F32)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    s32 = (mx - mn) / F32(levels)
    s16 = s32.astype(np.float16)
    m16 = mn.astype(np.float16)
    sf = s16.astype(F32)[..., None]
    mf = m16.astype(F32)[..., None]
    diff = x - mf
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = diff / sf
    codes = np.clip(np.rint(qf), 0, levels)
    codes = np.where(sf == 0, F32(0), codes)
    return codes.astype(np.uint8), s16, m16


def dequant_asym(codes, s16, m16) -> np.ndarray:
    """x_hat = fp32(s16) * code + fp32(m16): the product is exact in fp32 (11-bit times
    at most 8-bit significands), the sum is rounded once.  HyQuant paper, Eq. 9."""
    sf = np.asarray(s16).astype(F32)[..., None]
    mf = np.asarray(m16).astype(F32)[..., None]
    return sf * np.asarray(codes).astype(F32) + mf


def quant_int4_token(x_row, group: int = 32, bits: int = 4):
    """Quantize one or more token vectors ``[..., D]`` in contiguous groups of ``group``
    channels with 2^bits - 1 levels (INT4: 15; the bit width is a parameter of the HyQuant
    paper's Alg. 3 and Alg. 4).  Returns codes ``[..., D]`` and s16, m16 ``[..., D/group]``."""
    x = np.asarray(x_row, dtype=F32)
    D = x.shape[-1]
    xg = x.reshape(x.shape[:-1] + (D // group, group))
    c, s, m = quant_asym(xg, (1 << bits) - 1)
    return c.reshape(x.shape), s, m


def dequant_int4_token(codes, s16, m16, group: int = 32) -> np.ndarray:
    c = np.asarray(codes)
    D = c.shape[-1]
    cg = c.reshape(c.shape[:-1] + (D // group, group))
    return dequant_asym(cg, s16, m16).reshape(c.shape)


# ----------------------------------------------------------------------------- INT8 symmetric


def quant_int8_sym(x):
    """Symmetric INT8 over the whole array: HyQuant paper, Alg. 2 Stage 2
    (scale = max|x| / c_B with c_B = 127 for INT8, codes = round(x / scale)).

    Reading: scale in fp32 (max|x| exact, IEEE divide by 127), codes = rint(x / scale)
    (half-even) clamped to [-127, 127]; a zero block gets scale 0 and all-zero codes.
    Returns (codes int8, scale float32).
    """
    x = np.asarray(x, dtype=F32)
    amax = np.abs(x).max() if x.size else F32(0)
    s = F32(amax) / F32(127)
    if s == 0:
        return np.zeros(x.shape, np.int8), F32(0)
    q = np.clip(np.rint(x / s), -127, 127)
    return q.astype(np.int8), F32(s)


# ----------------------------------------------------------------------------- OCP FP8 E4M3


def e4m3_decode_table() -> np.ndarray:
    """Values of all 256 OCP E4M3 (FN) codes, from the format definition: 1 sign bit,
    4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is subnormal
    (m * 2^-9); codes 0x7F / 0xFF are NaN; there are no infinities."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * m * 2.0 ** -9
        else:
            vals[c] = sign * (8 + m) * 2.0 ** (e - 10)
    return vals


_E4M3 = e4m3_decode_table()
_E4M3_POS = _E4M3[:127]  # codes 0x00..0x7E: non-negative finite values, increasing


def e4m3_encode(x) -> np.ndarray:
    """fp32/fp64 -> OCP E4M3 code (uint8): nearest representable value, ties to the even
    code (mantissa LSB 0), saturating at +-448; NaN -> 0x7F.  Brute force over the
    decode table (obviously correct, slow)."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, np.uint8)
    for i, v in enumerate(flat):
        if np.isnan(v):
            out[i] = 0x7F
            continue
        a = min(abs(v), 448.0)
        d = np.abs(_E4M3_POS - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int(best[(best & 1) == 0][0])
        if v < 0 or (v == 0 and np.signbit(v)):
            c |= 0x80
        out[i] = c
    return out.reshape(x.shape)


def e4m3_value(codes) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def e4m3_round(x) -> np.ndarray:
    """Round to the nearest E4M3 value (fp64 result); vectorised via a bf16-exact path is
    not assumed -- this goes through ``e4m3_encode``."""
    return e4m3_value(e4m3_encode(x))


def e4m3_round_fast(x) -> np.ndarray:
    """Same result as ``e4m3_round`` for finite inputs, vectorised with searchsorted over
    the sorted positive value table (used for large prefill emulations; pinned equal
    to ``e4m3_round`` on exhaustive and random inputs)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(_E4M3_POS, a, side="left")
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    vlo, vhi = _E4M3_POS[lo], _E4M3_POS[hi]
    dlo, dhi = a - vlo, vhi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((hi & 1) == 0) & (hi != lo))
    mag = np.where(pick_hi, vhi, vlo)
    mag = np.where(a <= 0, 0.0, mag)
    return np.copysign(mag, x)


# ----------------------------------------------------------------------------- OCP FP4 E2M1, MX


def e2m1_decode_table() -> np.ndarray:
    """Values of the 16 FP4 E2M1 codes, from the format definition: 1 sign bit, 2 exponent
    bits (bias 1), 1 mantissa bit; exponent 0 is subnormal (m * 0.5); no infinity or NaN."""
    vals = np.empty(16, np.float64)
    for c in range(16):
        e = (c >> 1) & 3
        m = c & 1
        v = m * 0.5 if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
        vals[c] = -v if c & 8 else v
    return vals


_E2M1 = e2m1_decode_table()
_E2M1_POS = _E2M1[:8]  # codes 0..7: non-negative values, increasing


def e2m1_encode(x) -> np.ndarray:
    """fp32/fp64 -> FP4 E2M1 code (uint8 0..15): nearest value, ties to the even code
    (mantissa bit 0), saturating at +-6.  Brute force over the 8 magnitudes."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, np.uint8)
    for i, v in enumerate(flat):
        a = min(abs(v), 6.0)
        d = np.abs(_E2M1_POS - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int(best[(best & 1) == 0][0])
        if v < 0 or (v == 0 and np.signbit(v)):
            c |= 8
        out[i] = c
    return out.reshape(x.shape)


def e2m1_value(codes) -> np.ndarray:
    return _E2M1[np.asarray(codes, dtype=np.uint8)]


def mxfp4_quant_block(x):
    """One OCP MX block (32 values) in MXFP4: shared scale X = 2^e with
    e = floor(log2(max|x|)) - 2 (2 = the largest E2M1 exponent), clamped to the E8M0 range
    [-127, 127] (e = -127 for an all-zero block); codes = e2m1(x / X) (the division by a
    power of two is exact in fp32).  Returns (codes uint8 [32], e int)."""
    x = np.asarray(x, dtype=F32)
    amax = float(np.abs(x).max())
    if amax == 0.0:
        e = -127
    else:
        _, ex = np.frexp(amax)  # amax = f * 2^ex with f in [0.5, 1): floor(log2 amax) = ex - 1
        e = int(min(127, max(-127, (int(ex) - 1) - 2)))
    ratio = (x.astype(np.float64) * 2.0 ** (-e)).astype(F32)  # exact (power of two)
    return e2m1_encode(ratio), e


def mxfp4_quant_rows(X, block: int = 32):
    """MXFP4 of every row of X [..., D] in blocks of ``block`` contiguous channels.
    Returns (codes uint8 [..., D], e int16 [..., D / block])."""
    X = np.asarray(X, dtype=F32)
    lead = X.shape[:-1]
    Dm = X.shape[-1]
    flat = X.reshape(-1, Dm // block, block)
    codes = np.empty(flat.shape, np.uint8)
    ex = np.empty(flat.shape[:2], np.int16)
    amax = np.abs(flat).max(axis=2).astype(np.float64)
    with np.errstate(divide="ignore"):
        _, fe = np.frexp(amax)
    e = np.where(amax == 0.0, -127, np.clip(fe.astype(np.int64) - 3, -127, 127))
    ratio = (flat.astype(np.float64) * np.exp2(-e.astype(np.float64))[:, :, None]).astype(F32)
    # vectorised nearest-even E2M1 on the exact ratios (the same rule as e2m1_encode)
    a = np.minimum(np.abs(ratio).astype(np.float64), 6.0)
    hi = np.clip(np.searchsorted(_E2M1_POS, a, side="left"), 0, 7)
    lo = np.clip(hi - 1, 0, 7)
    dlo, dhi = a - _E2M1_POS[lo], _E2M1_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((hi & 1) == 0) & (hi != lo))
    c = np.where(pick_hi, hi, lo).astype(np.uint8)
    c = np.where(np.signbit(ratio), c | 8, c)
    codes[...] = c
    ex[...] = e
    return codes.reshape(lead + (Dm,)), ex.reshape(lead + (Dm // block,))

"""Attention references of the oracle (test infrastructure only).

"HyQuant paper" = the arXiv page "HyQuant: Hybrid-Precision Quantization for LLM
Attention".

* ``decode_ref``      -- exact softmax attention of one step's queries over the cache in
                         its stored precision (the plain definition of Alg. 3's result).
* ``flash_os`` / ``merge_states`` -- FlashAttention-style online-softmax state update and
                         the ReduceSoftmax merge of split partial states (Alg. 3).
* ``uniform_kv``      -- every position quantized with the same b-bit group scheme
                         (uniform-precision comparison points of §2.2 Fig. 2).
* ``prefill_ref``     -- step-by-step emulation of the hybrid prefill operator
                         (Alg. 2; readings listed in its docstring), with an INT8 or an
                         MXFP4 (``prefill_quantize_mx``) bulk Q.K^T.
* ``attention_exact`` -- exact causal softmax attention (fp64) over bf16 inputs.
"""
from __future__ import annotations

import numpy as np

from . import numerics as nm


# ----------------------------------------------------------------------------- decode


def decode_ref(q: np.ndarray, Kh: np.ndarray, Vh: np.ndarray) -> np.ndarray:
    """o_h = sum_j softmax_j(alpha * q_h . k_j) v_j over all positions, alpha = 1/sqrt(D)
    (HyQuant paper §4.3 Eq. 8-9 and Alg. 3: every segment -- quantized prefix, vertical
    lines, staging, window -- enters one softmax).  q: [g][D] fp32; Kh, Vh: [L][D] fp32
    stored-precision values.  Computed in fp64, returned fp32 [g][D]."""
    q = np.asarray(q, np.float64)
    K = np.asarray(Kh, np.float64)
    V = np.asarray(Vh, np.float64)
    alpha = 1.0 / np.sqrt(K.shape[1])
    z = alpha * (q @ K.T)
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return (p @ V).astype(np.float32)


def decode_weights(q: np.ndarray, Kh: np.ndarray) -> np.ndarray:
    """The softmax weights decode_ref applies (fp64), for the convex-combination checks."""
    q = np.asarray(q, np.float64)
    K = np.asarray(Kh, np.float64)
    z = (q @ K.T) / np.sqrt(K.shape[1])
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=1, keepdims=True)


def flash_os(scores: np.ndarray, V: np.ndarray, state):
    """One online-softmax update (FlashOS of Alg. 2/3) in fp64.
    state = (m, l, acc) with m = running max of the scores (natural-log domain)."""
    m, l, acc = state
    scores = np.asarray(scores, np.float64)
    if scores.size == 0:
        return state
    m_new = max(m, float(scores.max()))
    c = 0.0 if m == -np.inf else np.exp(m - m_new)
    p = np.exp(scores - m_new)
    return m_new, l * c + p.sum(), acc * c + p @ np.asarray(V, np.float64)


def merge_states(states):
    """ReduceSoftmax of Alg. 3: m = max m_s, l = sum l_s e^(m_s - m),
    acc = sum acc_s e^(m_s - m).  Returns the merged (m, l, acc)."""
    states = [s for s in states if s[0] != -np.inf]
    m = max(s[0] for s in states)
    l = sum(s[1] * np.exp(s[0] - m) for s in states)
    acc = sum(s[2] * np.exp(s[0] - m) for s in states)
    return m, l, acc


def init_state(D: int):
    return -np.inf, 0.0, np.zeros(D)


# ----------------------------------------------------------------------------- uniform precision


def uniform_kv(K_bits: np.ndarray, V_bits: np.ndarray, bits: int, group: int = 32):
    """Every position quantized with (2^bits - 1)-level asymmetric groups of ``group``
    channels (same operation order as the INT4 quantizer); bits = 16 returns the bf16
    values unchanged.  The uniform 4-bit / 8-bit comparison points of §2.2 Fig. 2."""
    K = nm.bf16_to_f32(K_bits)
    V = nm.bf16_to_f32(V_bits)
    if bits >= 16:
        return K, V
    levels = (1 << bits) - 1
    out = []
    for X in (K, V):
        L, D = X.shape
        Xg = X.reshape(L, D // group, group)
        c, s, m = nm.quant_asym(Xg, levels)
        out.append(nm.dequant_asym(c, s, m).reshape(L, D))
    return out[0], out[1]


# ----------------------------------------------------------------------------- prefill


def attention_exact(Q_bits, K_bits, V_bits) -> np.ndarray:
    """Exact causal softmax attention, fp64, of bf16 inputs.  Q [Hq][N][D], K/V [Hkv][N][D];
    Q head h reads KV head h // (Hq/Hkv).  Returns fp64 [Hq][N][D]."""
    Q = nm.bf16_to_f32(Q_bits).astype(np.float64)
    K = nm.bf16_to_f32(K_bits).astype(np.float64)
    V = nm.bf16_to_f32(V_bits).astype(np.float64)
    Hq, N, D = Q.shape
    g = Hq // K.shape[0]
    out = np.empty_like(Q)
    mask = np.tril(np.ones((N, N), bool))
    for h in range(Hq):
        z = (Q[h] @ K[h // g].T) / np.sqrt(D)
        z = np.where(mask, z, -np.inf)
        z -= z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p /= p.sum(axis=1, keepdims=True)
        out[h] = p @ V[h // g]
    return out


def prefill_quantize(Q_bits, K_bits, V_bits, anchors, BM: int = 64, BN: int = 64):
    """Operand quantization of the hybrid prefill (HyQuant paper Alg. 2 Stage 2, c_B = 127
    for INT8 and 448 for FP8).  Readings:
      * Q: symmetric INT8 per 64-query block per Q head, scale max|Q_blk|/127 (fp32).
      * K: symmetric INT8 per 64-position block per KV head; anchor rows are left out of
        the block maximum (their codes are never used).
      * V: OCP E4M3 with a per-channel fp32 scale s_V[c] = max over the head's non-anchor
        keys of |V[:, c]| / 448; code = e4m3(fp32(V / s_V)).
    Returns dict of codes and scales (numpy)."""
    Q = nm.bf16_to_f32(Q_bits)
    K = nm.bf16_to_f32(K_bits)
    V = nm.bf16_to_f32(V_bits)
    Hq, N, D = Q.shape
    Hkv = K.shape[0]
    nqb = (N + BM - 1) // BM
    nkb = (N + BN - 1) // BN
    q8 = np.zeros(Q.shape, np.int8)
    sq = np.zeros((Hq, nqb), np.float32)
    for h in range(Hq):
        for b in range(nqb):
            q8[h, b * BM:(b + 1) * BM], sq[h, b] = nm.quant_int8_sym(Q[h, b * BM:(b + 1) * BM])
    k8 = np.zeros(K.shape, np.int8)
    sk = np.zeros((Hkv, nkb), np.float32)
    for h in range(Hkv):
        isanc = np.zeros(N, bool)
        isanc[np.asarray(anchors[h], np.int64)] = True
        Kz = np.where(isanc[:, None], np.float32(0), K[h])
        for b in range(nkb):
            k8[h, b * BN:(b + 1) * BN], sk[h, b] = nm.quant_int8_sym(Kz[b * BN:(b + 1) * BN])
    v8, sv = _v_fp8(V, anchors)
    return dict(q8=q8, sq=sq, k8=k8, sk=sk, v8=v8, sv=sv)


def _v_fp8(V, anchors):
    """V of the bulk segment: OCP E4M3 with a per-channel fp32 scale s_V[c] = max over the
    head's non-anchor keys of |V[:, c]| / 448; code = e4m3(fp32(V / s_V)).  V: fp32
    [Hkv][N][D].  Returns (e4m3 code values as numbers, s_V)."""
    Hkv, N, D = V.shape
    v8 = np.zeros(V.shape, np.float64)
    sv = np.zeros((Hkv, D), np.float32)
    for h in range(Hkv):
        isanc = np.zeros(N, bool)
        isanc[np.asarray(anchors[h], np.int64)] = True
        Vz = np.where(isanc[:, None], np.float32(0), V[h])
        amax = np.abs(Vz).max(axis=0).astype(np.float32)
        sv[h] = amax / np.float32(448)
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(sv[h] > 0, Vz / np.where(sv[h] > 0, sv[h], np.float32(1)), np.float32(0))
        v8[h] = nm.e4m3_round_fast(ratio.astype(np.float32))
    return v8, sv


def prefill_quantize_mx(Q_bits, K_bits, V_bits, anchors):
    """Operand quantization of the hybrid prefill with an MXFP4 bulk (the HyQuant paper's
    §4.2 names INT4/FP4 as the lower-precision bulk format on backends that have it).
    Readings:
      * Q and K: OCP MXFP4 per row and per 32-channel block (``mxfp4_quant_rows``): an E8M0
        shared scale and E2M1 codes.  Every key row is quantized (an anchor's codes are
        never used: anchors are masked in the bulk segment).
      * V: as in ``prefill_quantize`` (E4M3, per-channel scale over non-anchor keys): P.V
        stays FP8, only Q.K^T moves to FP4.
    Returns dict(q4, qe, k4, ke, v8, sv): codes uint8, scale exponents int16 [.., 4]."""
    q4, qe = nm.mxfp4_quant_rows(nm.bf16_to_f32(Q_bits))
    k4, ke = nm.mxfp4_quant_rows(nm.bf16_to_f32(K_bits))
    v8, sv = _v_fp8(nm.bf16_to_f32(V_bits), anchors)
    return dict(q4=q4, qe=qe, k4=k4, ke=ke, v8=v8, sv=sv)


def mx_dot(q4, qe, k4, ke) -> np.ndarray:
    """MXFP4 dot products in fp64: sum over blocks of 2^(e_q + e_k) times the sum of the
    E2M1 products.  Every product is a multiple of 2^(e_q + e_k - 2) below 2^6 and a block's
    sum stays below 2^13 of those units, so every partial sum is exact in fp64 -- the result
    is the exact dot -- as long as the block exponents (e_q + e_k) of one (query, key) pair
    span fewer than 40 binades (real activations span a few).
    q4 [M][D], qe [M][D/32], k4 [N][D], ke [N][D/32] -> [M][N]."""
    qv = nm.e2m1_value(q4) * np.exp2(np.repeat(qe.astype(np.float64), 32, axis=-1))
    kv = nm.e2m1_value(k4) * np.exp2(np.repeat(ke.astype(np.float64), 32, axis=-1))
    return qv @ kv.T


MIDPOINT_BAND = 2.0 ** -16


def _count_near_midpoints(stats, p32, valid, seg):
    """Diagnostic of the rounded prefill: how many stored p values another fp32
    implementation could round the other way.  An fp32 value x = 448 p (segment A, E4M3) or
    x = p (segments B and C, bf16) is counted when it lies within MIDPOINT_BAND * x of a
    rounding midpoint of its format; a different but correct fp32 evaluation of the same
    score and exponential (another association, an exp2 with a rescaled argument) moves x
    by far less than that band for scores of the sizes met here, so the count bounds the
    codes that can differ.  stats gets n_A / near_A / n_BC / near_BC and p_near_max_A /
    p_near_max_BC (the largest p among the counted values of each kind)."""
    x = np.asarray(p32, np.float64)
    if seg == "A":
        x = (np.float32(448) * np.asarray(p32, np.float32)).astype(np.float64)
        tab = nm.e4m3_decode_table()[:127]
        hi = np.clip(np.searchsorted(tab, x, side="left"), 1, 126)
        up = np.where(hi < 126, (tab[hi] + tab[np.minimum(hi + 1, 126)]) / 2, np.inf)  # none above 448
        mids = np.stack([(tab[hi - 1] + tab[hi]) / 2, up])
        dist = np.abs(mids - x[None]).min(axis=0)
    else:
        u = np.asarray(p32, np.float32).view(np.uint32).astype(np.int64)
        ulp = np.ldexp(1.0, ((u >> 23) & 0xFF).astype(np.int64) - 127 - 7)  # bf16 spacing at x
        dist = np.abs((u & 0xFFFF) - 0x8000) / 65536.0 * ulp
    near = valid & (x > 0) & (dist <= MIDPOINT_BAND * x)
    key = "A" if seg == "A" else "BC"
    stats["n_" + key] = stats.get("n_" + key, 0) + int(np.count_nonzero(valid))
    stats["near_" + key] = stats.get("near_" + key, 0) + int(np.count_nonzero(near))
    if near.any():
        pm = float(np.asarray(p32, np.float64)[near].max())
        stats["p_near_max_" + key] = max(stats.get("p_near_max_" + key, 0.0), pm)


def prefill_ref(Q_bits, K_bits, V_bits, anchors, W: int = 128, BM: int = 64, BN: int = 64,
                blocks=None, round_p: bool = True, heads=None, qz=None, bulk: str = "int8",
                stats=None):
    """Emulation of the hybrid prefill operator (HyQuant paper §4.2 Eq. 6-7, Alg. 2).

    For query i (causal), keys split three ways (Eq. 1 applied per query):
      window  [max(0, i-W+1), i]             -- bf16 Q.K, bf16 V
      anchors a <= i-W                       -- bf16 Q.K, bf16 V
      the rest j <= i-W                      -- INT8 Q.K (int32 dot * s_Q * s_K * alpha),
                                                FP8 P and FP8 V (per-channel scale)
    One online softmax per row, tiles of BN keys, segment order A (quantized prefix,
    ascending 64-key tiles) -> B (anchors, ascending 64-anchor tiles) -> C (window,
    ascending 64-key tiles) as in Alg. 2 Stage 3.  After each tile's max update
    p = exp(s - m_run); with ``round_p`` p is rounded as the operator stores it:
    segment A: e4m3(448 p) / 448, segments B and C: bf16(p); l sums the rounded values.

    Precision.  With ``round_p`` the values that decide a rounded code -- the score s,
    the running max m and p -- are IEEE fp32 values (the pages fix no precision for them;
    the online softmax of a FlashAttention-style operator keeps fp32 state).  The score
    follows Alg. 2's Segment A line, which multiplies the integer dot by the product of the
    two scales and then by alpha: s = fp32(fp32(dot * fp32(s_Q * s_K)) * alpha) (dot an
    exact integer); bf16 keys: s = fp32(fp32(q.k) * alpha) with q.k exact.  p is the
    correctly rounded fp32 value of exp(fp32(s - m)) (an fp64 exponential rounded once to
    fp32), then 448 p is rounded to fp32 before the E4M3 rounding.  The rescale factors, l
    and the accumulator stay fp64.  Without ``round_p`` everything is fp64 (the exact mixed
    softmax of Eq. 7).  ``blocks`` / ``heads``: optional lists of 64-query blocks and Q heads
    to compute (others are NaN); ``qz``: the ``prefill_quantize`` result, if already at hand.
    ``bulk="mxfp4"``: the quantized segment's Q.K^T uses ``prefill_quantize_mx`` operands,
    s = fp32(exact MX dot) * alpha (the products and their block sums are exact in fp64; the
    operator accumulates them in fp32), everything else unchanged.  ``stats``: an optional
    dict that receives the near-midpoint counts of ``_count_near_midpoints``.
    Returns fp64 [Hq][N][D].
    """
    Qf = nm.bf16_to_f32(Q_bits).astype(np.float64)
    Kf = nm.bf16_to_f32(K_bits).astype(np.float64)
    Vf = nm.bf16_to_f32(V_bits).astype(np.float64)
    Hq, N, D = Qf.shape
    Hkv = Kf.shape[0]
    g = Hq // Hkv
    alpha = 1.0 / np.sqrt(D)

    def bscore(dot64):
        if round_p:
            return dot64.astype(np.float32) * np.float32(alpha)
        return alpha * dot64

    mx = bulk == "mxfp4"
    if qz is None:
        qz = prefill_quantize_mx(Q_bits, K_bits, V_bits, anchors) if mx else \
            prefill_quantize(Q_bits, K_bits, V_bits, anchors, BM, BN)
    nqb = (N + BM - 1) // BM
    if blocks is None:
        blocks = range(nqb)
    out = np.full((Hq, N, D), np.nan)
    for h in (range(Hq) if heads is None else heads):
        hk = h // g
        anc = np.asarray(anchors[hk], np.int64)
        isanc = np.zeros(N, bool)
        isanc[anc] = True
        if not mx:
            k8 = qz["k8"][hk].astype(np.int64)
        vq = qz["v8"][hk] * qz["sv"][hk].astype(np.float64)[None, :]  # dequantized FP8 V
        for b in blocks:
            r0, r1 = b * BM, min(N, (b + 1) * BM)
            rows = np.arange(r0, r1)
            if not mx:
                q8 = qz["q8"][h, r0:r1].astype(np.int64)
                sq = qz["sq"][h, b] if round_p else float(qz["sq"][h, b])
            m = np.full(len(rows), -np.inf, dtype=np.float32 if round_p else np.float64)
            l = np.zeros(len(rows))
            acc = np.zeros((len(rows), D))

            ft = np.float32 if round_p else np.float64

            def step(s, valid, Vt, seg):
                nonlocal m, l, acc
                s = np.where(valid, s, -np.inf).astype(ft)
                tmax = s.max(axis=1)
                m_new = np.maximum(m, tmax)
                live = m_new > -np.inf
                had = m > -np.inf
                c = np.where(live & had, np.exp(np.where(had, m, 0.0).astype(np.float64)
                                                 - np.where(live, m_new, 0.0)), 0.0)
                with np.errstate(invalid="ignore"):
                    z = s - np.where(live, m_new, ft(0))[:, None]  # fp32 difference when rounding
                    p = np.where(valid, np.exp(z.astype(np.float64)).astype(ft), ft(0))
                if round_p:
                    if stats is not None:
                        _count_near_midpoints(stats, p, valid, seg)
                    if seg == "A":
                        p = nm.e4m3_round_fast(np.float32(448) * p) / 448.0
                    else:
                        p = nm.bf16_to_f32(nm.f32_to_bf16(p)).astype(np.float64)
                l = l * c + p.sum(axis=1, dtype=np.float64)
                acc = acc * c[:, None] + p.astype(np.float64) @ Vt
                m = np.where(live, m_new, m)

            # Segment A: quantized prefix tiles.
            last_q = r1 - 1 - W
            if last_q >= 0:
                for t in range(last_q // BN + 1):
                    j = np.arange(t * BN, min(N, (t + 1) * BN))
                    if mx:
                        dot = mx_dot(qz["q4"][h, r0:r1], qz["qe"][h, r0:r1], qz["k4"][hk, j], qz["ke"][hk, j])
                        s = dot.astype(np.float32) * np.float32(alpha) if round_p else dot * alpha
                    else:
                        dot = q8 @ k8[j].T
                        if round_p:
                            ssc = np.float32(sq) * np.float32(qz["sk"][hk, t])  # s_Q s_K (fp32)
                            s = (dot.astype(np.float32) * ssc) * np.float32(alpha)
                        else:
                            s = dot.astype(np.float64) * (sq * float(qz["sk"][hk, t])) * alpha
                    valid = (j[None, :] <= rows[:, None] - W) & ~isanc[j][None, :]
                    step(s, valid, vq[j], "A")
            # Segment B: anchors, ascending tiles of BN anchors.
            for u in range((len(anc) + BN - 1) // BN):
                j = anc[u * BN:(u + 1) * BN]
                s = bscore(Qf[h, r0:r1] @ Kf[hk, j].T)
                valid = j[None, :] <= rows[:, None] - W
                step(s, valid, Vf[hk, j], "B")
            # Segment C: window, ascending aligned tiles.
            t_lo = max(0, r0 - W + 1) // BN
            t_hi = (r1 - 1) // BN
            for t in range(t_lo, t_hi + 1):
                j = np.arange(t * BN, min(N, (t + 1) * BN))
                s = bscore(Qf[h, r0:r1] @ Kf[hk, j].T)
                valid = (j[None, :] <= rows[:, None]) & (j[None, :] >= rows[:, None] - W + 1)
                step(s, valid, Vf[hk, j], "C")
            out[h, r0:r1] = acc / l[:, None]
    return out

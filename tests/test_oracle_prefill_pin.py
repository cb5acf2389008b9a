"""Pins of the oracle's rounded prefill emulation (``oracle.attention.prefill_ref`` with
``round_p=True``) against the HyQuant paper's Alg. 2 Stage 3 (segmented online softmax:
Segment A quantized prefix, Segment B vertical-line tail, Segment C local window, each tile
folded into (m, l, acc) by FlashOS) and the §4.2 implementation note (INT8/FP8 bulk, bf16
vertical-line and window tiles).

The brute force below is written independently of the oracle: one query row at a time,
explicit Python loops over keys and channels, scalar fp32 arithmetic through numpy scalars,
and only codecs pinned elsewhere (``e4m3_encode`` / ``e4m3_value`` exhaustively,
``f32_to_bf16`` against torch, the E2M1 table by its definition).  It takes the quantized
operands from ``prefill_quantize`` / ``prefill_quantize_mx``, whose codes and scales are pinned
by their own tests.  Readings it encodes (the pages fix no precision for these steps):

  * tiles of BN keys; Segment A walks the aligned tiles of the quantized prefix in ascending
    order, Segment B the anchor list in groups of BN, Segment C the aligned window tiles;
  * the running max is updated once per tile, over the tile's visible keys;
  * scores in fp32: Segment A s = fp32(fp32(dot * fp32(s_Q * s_K)) * alpha) (INT8) or
    fp32(exact MX dot) * alpha (MXFP4); Segments B and C s = fp32(fp32(q.k) * alpha);
  * p = fp32(exp(fp32(s - m))) correctly rounded; Segment A stores e4m3(fp32(448 p)) / 448,
    Segments B and C store bf16(p); l sums the stored values, acc the stored values times V.

Each ``mutation`` flag plants one plausible mistake; the tests check that the oracle equals
the correct brute force to 1e-12 and differs from every mutant.
"""
import math

import numpy as np
import pytest

from hybrid_precision_kv_amd import synth
from oracle import attention as att
from oracle import numerics as nm

F32 = np.float32
MUTATIONS = ("trunc_e4m3", "bf16_in_A", "l_unrounded", "per_key_max", "score_order")


def _e4m3_trunc(x):
    """E4M3 rounding toward zero (a planted mistake): the largest code value <= |x|."""
    tab = nm.e4m3_decode_table()[:127]
    a = min(abs(float(x)), 448.0)
    return math.copysign(float(tab[tab <= a].max()), float(x))


def _store_p(p32, seg, mutation):
    """The value the operator keeps for p (fp32) in segment ``seg``."""
    if seg == "A" and mutation != "bf16_in_A":
        x = F32(448) * p32  # fp32 product
        if mutation == "trunc_e4m3":
            return _e4m3_trunc(x) / 448.0
        return float(nm.e4m3_value(nm.e4m3_encode(np.float64(x))).reshape(-1)[0]) / 448.0
    return float(nm.bf16_to_f32(nm.f32_to_bf16(np.float32(p32))).reshape(-1)[0])


def brute_prefill(Q_bits, K_bits, V_bits, anchors, W, BM, BN, bulk="int8", mutation=None):
    """Alg. 2 Stage 3 for every query row with explicit loops.  Returns fp64 [Hq][N][D]."""
    Hq, N, D = Q_bits.shape
    Hkv = K_bits.shape[0]
    g = Hq // Hkv
    alpha = F32(1.0 / math.sqrt(D))
    Qf = nm.bf16_to_f32(Q_bits)
    Kf = nm.bf16_to_f32(K_bits)
    Vf = nm.bf16_to_f32(V_bits)
    if bulk == "mxfp4":
        qz = att.prefill_quantize_mx(Q_bits, K_bits, V_bits, anchors)
        e2m1 = nm.e2m1_decode_table()
    else:
        qz = att.prefill_quantize(Q_bits, K_bits, V_bits, anchors, BM, BN)
    out = np.zeros((Hq, N, D))
    for h in range(Hq):
        hk = h // g
        anc = [int(a) for a in anchors[hk]]
        ancset = set(anc)

        def score_bulk(i, j):
            if bulk == "mxfp4":
                tot = 0.0  # exact in fp64: every product is a small multiple of a power of two
                for c in range(D):
                    b = c // 32
                    tot += float(e2m1[qz["q4"][h, i, c]]) * float(e2m1[qz["k4"][hk, j, c]]) * \
                        2.0 ** (int(qz["qe"][h, i, b]) + int(qz["ke"][hk, j, b]))
                return F32(tot) * alpha
            dot = 0
            for c in range(D):
                dot += int(qz["q8"][h, i, c]) * int(qz["k8"][hk, j, c])
            sq, sk = F32(qz["sq"][h, i // BM]), F32(qz["sk"][hk, j // BN])
            if mutation == "score_order":
                return ((F32(dot) * sq) * sk) * alpha
            return (F32(dot) * (sq * sk)) * alpha

        def score_bf16(i, j):
            dot = 0.0  # bf16 products are exact in fp64 and so is their sum here
            for c in range(D):
                dot += float(Qf[h, i, c]) * float(Kf[hk, j, c])
            return F32(dot) * alpha

        def vq(j):
            return [float(qz["v8"][hk, j, c]) * float(F32(qz["sv"][hk, c])) for c in range(D)]

        def vb(j):
            return [float(Vf[hk, j, c]) for c in range(D)]

        for i in range(N):
            tiles = []  # (segment, [(score fp32, value row)]) in Stage 3 order
            for t in range(N // BN + 1):  # Segment A: aligned tiles of the quantized prefix
                keys = [j for j in range(t * BN, min(N, (t + 1) * BN)) if j <= i - W and j not in ancset]
                if keys:
                    tiles.append(("A", [(score_bulk(i, j), vq(j)) for j in keys]))
            for u in range(0, len(anc), BN):  # Segment B: the anchor list in groups of BN
                keys = [a for a in anc[u:u + BN] if a <= i - W]
                if keys:
                    tiles.append(("B", [(score_bf16(i, j), vb(j)) for j in keys]))
            for t in range(N // BN + 1):  # Segment C: aligned window tiles
                keys = [j for j in range(t * BN, min(N, (t + 1) * BN)) if i - W + 1 <= j <= i]
                if keys:
                    tiles.append(("C", [(score_bf16(i, j), vb(j)) for j in keys]))
            m = None  # running max (fp32); None = no key seen yet
            l = 0.0
            acc = [0.0] * D

            def fold(items, seg):
                nonlocal m, l, acc
                tmax = max(s for s, _ in items)
                m_new = tmax if m is None else max(m, tmax)
                c = 0.0 if m is None else math.exp(float(m) - float(m_new))
                l *= c
                acc = [a * c for a in acc]
                for s, v in items:
                    p32 = F32(math.exp(float(F32(s - m_new))))
                    pt = _store_p(p32, seg, mutation)
                    l += float(p32) if mutation == "l_unrounded" else pt
                    for ch in range(D):
                        acc[ch] += pt * v[ch]
                m = m_new

            for seg, items in tiles:
                if mutation == "per_key_max":  # the max advanced key by key inside a tile
                    for it in items:
                        fold([it], seg)
                else:
                    fold(items, seg)
            out[h, i] = [a / l for a in acc]
    return out


def _case(seed, Hq, Hkv, N, W, n_anc, D):
    """Seeded synthetic inputs at head_dim D (the prefill generator's distribution) and
    n_anc distinct ascending anchors per KV head inside [0, N - W)."""
    d = synth.gen_prefill(seed, Hq, Hkv, N)
    rng = np.random.default_rng(seed + 1)
    P = max(0, N - W)
    A = np.stack([np.sort(rng.choice(P, size=min(n_anc, P), replace=False)) for _ in range(Hkv)]).astype(np.int32) \
        if P else np.zeros((Hkv, 0), np.int32)
    return d["Q"][..., :D].copy(), d["K"][..., :D].copy(), d["V"][..., :D].copy(), A


CASES = [  # (seed, Hq, Hkv, N, W, n_anchor, D, BM, BN)
    (1, 2, 1, 40, 8, 5, 64, 16, 8),
    (2, 2, 2, 33, 4, 3, 32, 8, 4),
    (3, 4, 2, 29, 8, 0, 32, 16, 4),
    (4, 1, 1, 40, 4, 36, 64, 8, 8),  # every candidate an anchor
    (5, 2, 1, 17, 8, 2, 32, 8, 8),
]


@pytest.mark.parametrize("bulk", ["int8", "mxfp4"])
@pytest.mark.parametrize("case", CASES)
def test_prefill_ref_equals_bruteforce(case, bulk):
    seed, Hq, Hkv, N, W, n_anc, D, BM, BN = case
    Q, K, V, A = _case(seed, Hq, Hkv, N, W, n_anc, D)
    ref = att.prefill_ref(Q, K, V, A, W=W, BM=BM, BN=BN, bulk=bulk)
    bf = brute_prefill(Q, K, V, A, W, BM, BN, bulk)
    assert np.abs(ref - bf).max() <= 1e-12


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_bruteforce_tells_each_planted_mistake(mutation):
    """Each plausible mistake changes the rows the brute force returns (so the equality above
    would fail if the oracle made it).  score_order applies to the INT8 bulk only."""
    seed, Hq, Hkv, N, W, n_anc, D, BM, BN = CASES[0]
    Q, K, V, A = _case(seed, Hq, Hkv, N, W, n_anc, D)
    ref = att.prefill_ref(Q, K, V, A, W=W, BM=BM, BN=BN)
    bad = brute_prefill(Q, K, V, A, W, BM, BN, mutation=mutation)
    gap = np.abs(ref - bad).max()
    print(f"{mutation}: max |oracle - mutant| = {gap:.3g}")
    assert gap > 1e-9, mutation


def test_prefill_zero_queries_give_segment_means():
    """Q = 0: every visible score is 0, so after the first tile m = 0 and every p = 1, stored
    exactly in both formats (448 is an E4M3 value, 1 a bf16 value).  Each row's output is the
    plain mean of the values it sees: FP8-dequantized for the quantized prefix, bf16 for
    anchors and window."""
    N, W, BN = 30, 8, 4
    Q, K, V, A = _case(11, 2, 1, N, W, 4, 32)
    Q[:] = 0
    o = att.prefill_ref(Q, K, V, A, W=W, BM=8, BN=BN)
    qz = att.prefill_quantize(Q, K, V, A, 8, BN)
    Vb = nm.bf16_to_f32(V).astype(np.float64)
    vq = qz["v8"][0] * qz["sv"][0].astype(np.float64)
    anc = set(int(a) for a in A[0])
    for i in range(N):
        rows = [Vb[0, j] if (j > i - W or j in anc) else vq[j] for j in range(i + 1)]
        assert np.abs(o[0, i] - np.mean(rows, axis=0)).max() <= 1e-12
        assert np.abs(o[1, i] - np.mean(rows, axis=0)).max() <= 1e-12


def test_prefill_rounding_differs_by_segment():
    """A hand-built row whose two prefix keys and two window keys carry the same pair of
    scores (0 and log 0.3, so p = 1 and 0.3 in one tile): the stored weights are
    e4m3(448 * 0.3) / 448 = 128 / 448 in the quantized segment and bf16(0.3) = 0.30078125 in
    the window, with l summing those.  D = 32, W = 4, BN = 4, no anchors; channel 0 carries
    the scores, channel 1 of V tells the keys apart."""
    D, W, N = 32, 4, 8
    a = math.sqrt(D)
    z = math.log(0.3)
    q = np.zeros((1, N, D), np.float32)
    k = np.zeros((1, N, D), np.float32)
    v = np.zeros((1, N, D), np.float32)
    q[0, N - 1, 0] = 1.0  # only the last row is checked; other rows see their own keys
    # score of key j for the last row = k[j, 0] / sqrt(D); INT8 codes: q8 = 127, s_Q = 1/127,
    # s_K = max|K_blk| / 127 with block max = |z| a, so the prefix scores are exact enough to
    # land p on 1 and about 0.3
    kvals = {0: 0.0, 1: z * a, 4: z * a, 5: 0.0, 6: 0.0, 7: z * a}
    for j, s in kvals.items():
        k[0, j, 0] = s
    for j in range(N):
        v[0, j, 1] = float(j + 1)
    Qb, Kb, Vb = (nm.f32_to_bf16(x) for x in (q, k, v))
    o = att.prefill_ref(Qb, Kb, Vb, np.zeros((1, 0), np.int32), W=W, BM=8, BN=4)
    bf = brute_prefill(Qb, Kb, Vb, np.zeros((1, 0), np.int32), W, 8, 4)
    assert np.abs(o - bf).max() <= 1e-12
    # the prefix tile (keys 0..3, visible 0..3) holds scores 0 and ~log 0.3 (keys 2, 3 at 0 too)
    qz = att.prefill_quantize(Qb, Kb, Vb, np.zeros((1, 0), np.int32), 8, 4)
    vq = qz["v8"][0, :, 1] * float(qz["sv"][0, 1])
    kq = nm.bf16_to_f32(Kb)[0, :, 0].astype(np.float64)
    s_pref = [float(F32(F32(int(qz["q8"][0, N - 1, 0]) * int(qz["k8"][0, j, 0])) *
                        (F32(qz["sq"][0, 0]) * F32(qz["sk"][0, 0]))) * F32(1 / a)) for j in range(4)]
    p_pref = [float(F32(math.exp(float(F32(s - max(s_pref)))))) for s in s_pref]
    w_pref = [float(nm.e4m3_value(nm.e4m3_encode(np.float64(F32(448) * F32(p)))).reshape(-1)[0]) / 448 for p in p_pref]
    assert abs(w_pref[1] - 128 / 448) < 1e-15  # the 0.3 weight is stored as 128/448 = 0.2857
    s_win = [float(F32(kq[j]) * F32(1 / a)) for j in range(4, 8)]
    m = max(max(s_pref), max(s_win))
    p_win = [float(F32(math.exp(float(F32(s - m))))) for s in s_win]
    w_win = [float(nm.bf16_to_f32(nm.f32_to_bf16(np.float32(p))).reshape(-1)[0]) for p in p_win]
    assert abs(w_win[0] - 0.30078125) < 1e-15  # the same ratio stored as bf16
    c = math.exp(max(s_pref) - m)
    num = c * sum(w * vq[j] for j, w in enumerate(w_pref)) + sum(w * (j + 5) for j, w in enumerate(w_win))
    den = c * sum(w_pref) + sum(w_win)
    assert abs(o[0, N - 1, 1] - num / den) <= 1e-12

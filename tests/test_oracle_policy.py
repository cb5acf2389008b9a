"""Pins for oracle.policy: anchor-count rule, vertical-line scores, top-k and the hybrid
cache state machine, against closed forms and brute force on tiny inputs (CPU only)."""
import math

import numpy as np
import pytest

from hybrid_precision_kv_amd import synth
from oracle import numerics as nm
from oracle import policy as pol
from oracle import attention as att


# ----------------------------------------------------------------------------- k rule

def test_k_rule_closed_forms():
    # empty candidate set -> no anchors (Alg. 1: P = max(0, L_K - W), return empty when P = 0)
    assert pol.k_rule(0) == 0 and pol.k_rule(100) == 0 and pol.k_rule(128) == 0
    # at least one anchor once a candidate exists, never more than P
    assert pol.k_rule(129) == 1
    assert pol.k_rule(130, pct_num=100, pct_den=100) == 2
    # ceil of 5% of the context length
    assert pol.k_rule(1024) == 52 and pol.k_rule(4096) == 205
    assert pol.k_rule(16384) == 820 and pol.k_rule(32768) == 1639
    assert pol.k_rule(32768, pct_num=1) == 328 and pol.k_rule(32768, pct_num=10) == 3277
    for L in range(129, 3000, 37):
        k = pol.k_rule(L)
        assert 1 <= k <= L - 128
        assert k == L - 128 or (k >= 0.05 * L - 1e-9 and k < 0.05 * L + 1)


# ----------------------------------------------------------------------------- scores / top-k

def _brute_scores(proxy, keys, n_cand):
    R, D = proxy.shape
    L = keys.shape[0]
    S = [0.0] * n_cand
    for r in range(R):
        z = [sum(float(proxy[r, c]) * float(keys[j, c]) for c in range(D)) / math.sqrt(D) for j in range(L)]
        mx = max(z)
        e = [math.exp(v - mx) for v in z]
        tot = sum(e)
        for j in range(n_cand):
            S[j] += e[j] / tot
    return np.array(S)


def test_vertical_scores_brute_force():
    rng = np.random.default_rng(0)
    for D, L, R, P in [(32, 17, 5, 9), (64, 40, 8, 31), (32, 12, 1, 12)]:
        proxy = rng.standard_normal((R, D)).astype(np.float32)
        keys = rng.standard_normal((L, D)).astype(np.float32) * 1.7
        ours = pol.vertical_scores(proxy, keys, P)
        ref = _brute_scores(proxy, keys, P)
        assert np.allclose(ours, ref, rtol=1e-12, atol=1e-14)


def test_vertical_scores_mass_conservation():
    rng = np.random.default_rng(1)
    proxy = rng.standard_normal((12, 64))
    keys = rng.standard_normal((300, 64)) * 2
    S = pol.vertical_scores(proxy, keys, 300)
    assert abs(S.sum() - 12) < 1e-10  # every proxy row's softmax sums to one
    assert np.all(S >= 0)


def test_topk_brute_force_and_ties():
    rng = np.random.default_rng(2)
    for _ in range(50):
        n = int(rng.integers(1, 60))
        s = rng.integers(0, 6, n).astype(float)  # many ties
        k = int(rng.integers(0, n + 1))
        ref = sorted(sorted(range(n), key=lambda j: (-s[j], j))[:k])
        assert list(pol.topk_lower_index(s, k)) == ref


# ----------------------------------------------------------------------------- cache state machine

class BruteCache:
    """Independent set-based model of the cache rules, for tiny inputs."""

    def __init__(self, W):
        self.W = W
        self.val = {}  # pos -> (kvals, vvals) fp32 as stored
        self.kind = {}

    def _q(self, bits):
        c, s, m = nm.quant_int4_token(nm.bf16_to_f32(bits), 32 if bits.shape[-1] % 32 == 0 else bits.shape[-1])
        return nm.dequant_int4_token(c, s, m, 32 if bits.shape[-1] % 32 == 0 else bits.shape[-1])

    def freeze(self, K, V, A):
        L = len(K)
        self.L = L
        self.bits = {}
        for p in range(L):
            self.bits[p] = (K[p], V[p])
            if p >= L - self.W:
                self.kind[p] = "win"
            elif p in set(A):
                self.kind[p] = "anc"
            else:
                self.kind[p] = "q"
                self.bits[p] = ("q", self._q(K[p]), self._q(V[p]))

    def append(self, k, v):
        if self.L >= self.W:
            self.kind[self.L - self.W] = "stg"
        self.kind[self.L] = "win"
        self.bits[self.L] = (k, v)
        self.L += 1

    def refresh(self, A):
        A = set(int(a) for a in A)
        for p in range(self.L - self.W):
            kd = self.kind[p]
            if p in A:
                if kd == "q":
                    _, kq, vq = self.bits[p]
                    self.bits[p] = (nm.f32_to_bf16(kq), nm.f32_to_bf16(vq))
                self.kind[p] = "anc"
            elif kd in ("anc", "stg"):
                k, v = self.bits[p]
                self.bits[p] = ("q", self._q(k), self._q(v))
                self.kind[p] = "q"

    def values(self):
        Ks, Vs = [], []
        for p in range(self.L):
            b = self.bits[p]
            if self.kind[p] == "q":
                Ks.append(b[1]); Vs.append(b[2])
            else:
                Ks.append(nm.bf16_to_f32(b[0])); Vs.append(nm.bf16_to_f32(b[1]))
        return np.array(Ks), np.array(Vs)


def _brute_attn(q, K, V):
    out = []
    for h in range(q.shape[0]):
        z = [sum(float(q[h, c]) * float(K[j, c]) for c in range(K.shape[1])) / math.sqrt(K.shape[1]) for j in range(len(K))]
        mx = max(z)
        e = [math.exp(t - mx) for t in z]
        tot = sum(e)
        out.append([sum(e[j] * float(V[j, c]) for j in range(len(K))) / tot for c in range(K.shape[1])])
    return np.array(out)


@pytest.mark.parametrize("D,W,L0,steps,seed", [(32, 4, 20, 9, 0), (64, 8, 33, 7, 1), (32, 8, 6, 12, 2)])
def test_cache_state_machine_brute_force(D, W, L0, steps, seed):
    rng = np.random.default_rng(seed)
    g = 2
    bf = lambda a: nm.f32_to_bf16(a.astype(np.float32))
    K = bf(rng.standard_normal((L0, D)) * 1.3)
    V = bf(rng.standard_normal((L0, D)))
    P0 = max(0, L0 - W)
    A0 = np.sort(rng.choice(P0, size=min(3, P0), replace=False)) if P0 else np.zeros(0, np.int64)
    ref = pol.HybridCacheRef(D=D, W=W, group=32, g=g, proxy_cap=4)
    ref.freeze(K, V, A0)
    bc = BruteCache(W)
    bc.freeze(K, V, list(A0))
    for t in range(steps):
        k = bf(rng.standard_normal(D)); v = bf(rng.standard_normal(D)); q = bf(rng.standard_normal((g, D)))
        ref.append(k, v, q)
        bc.append(k, v)
        if t % 4 == 3:
            P = ref.L - W
            A = np.sort(rng.choice(P, size=min(P, 4), replace=False)) if P > 0 else np.zeros(0, np.int64)
            ref.refresh(A)
            bc.refresh(A)
        Kh, Vh = ref.stored_kv()
        Kb, Vb = bc.values()
        assert np.array_equal(Kh, Kb.astype(np.float32)) and np.array_equal(Vh, Vb.astype(np.float32))
        qf = nm.bf16_to_f32(q)
        o = att.decode_ref(qf, Kh, Vh)
        ob = _brute_attn(qf, Kb, Vb)
        assert np.allclose(o, ob, rtol=0, atol=2e-6)
        c = ref.counts()
        assert c["win"] == min(ref.L, W)
        assert c["win"] + c["staged"] + c["anchor"] + c["int4"] == ref.L


def test_cache_counts_follow_closed_form():
    s = synth.HeadStream(5, 600, 4)
    A, _ = pol.select_dense(s.K, s.queries(64))
    c = pol.HybridCacheRef(g=4)
    c.freeze(s.K, s.V, A, s.queries(64))
    k0 = pol.k_rule(600)
    assert c.counts() == dict(L=600, win=128, staged=0, anchor=k0, int4=600 - 128 - k0)
    for t in range(70):
        k, v, q = s.new_tokens(1)
        c.append(k[0], v[0], q[:, 0])
    assert c.counts()["staged"] == 70 and c.proxy.shape[1] == 64
    A2, _ = c.select()
    c.refresh(A2)
    k1 = pol.k_rule(670)
    assert c.counts() == dict(L=670, win=128, staged=0, anchor=k1, int4=670 - 128 - k1)
    assert np.array_equal(c.anchors(), A2)


def test_promoted_positions_carry_bf16_of_dequant():
    s = synth.HeadStream(7, 400, 2)
    c = pol.HybridCacheRef(g=2)
    c.freeze(s.K, s.V, np.array([3, 10]))
    Kh0, Vh0 = c.stored_kv()
    c.refresh(np.array([3, 50]))  # 50 was INT4 -> promoted; 10 demoted
    Kh1, Vh1 = c.stored_kv()
    assert np.array_equal(Kh1[50], nm.bf16_to_f32(nm.f32_to_bf16(Kh0[50])))
    assert np.array_equal(Kh1[3], Kh0[3])
    # a demoted anchor holding its original bf16 gets the same codes Freeze would give
    c2 = pol.HybridCacheRef(g=2)
    c2.freeze(s.K, s.V, np.array([3]))
    assert np.array_equal(c2.stored_kv()[0][10], Kh1[10])


# ----------------------------------------------------------------------------- Alg. 1 literal selector

def test_k_alg1_closed_forms():
    # Alg. 1: k = min(P, max(1, ceil(P r))), on the candidates, not on the context length
    assert pol.k_alg1(0) == 0 and pol.k_alg1(-3) == 0
    assert pol.k_alg1(896) == 45  # ceil(0.05 * 896) = ceil(44.8)
    assert pol.k_alg1(900) == 45 and pol.k_alg1(901) == 46
    assert pol.k_alg1(1) == 1 and pol.k_alg1(19) == 1 and pol.k_alg1(20) == 1 and pol.k_alg1(21) == 2
    assert pol.k_alg1(7, 100, 100) == 7 and pol.k_alg1(7, 1, 1000) == 1
    assert pol.k_alg1(32640, 5, 100) == 1632


def _bits(rng, shape, scale=1.0):
    return nm.f32_to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("LQ", [1, 50, 128, 129, 300])
def test_tail_mean_scores_are_mean_of_tail_logits(LQ):
    """Raw logits are linear in the proxy: qbar . k_j must equal the average over the tail
    queries of q_i . k_j, computed here query by query with explicit loops; the tail is the
    last min(128, L_Q) queries."""
    rng = np.random.default_rng(LQ)
    Hkv, g, L, D = 2, 2, 150, 8
    K = _bits(rng, (Hkv, L, D))
    Q = _bits(rng, (Hkv * g, LQ, D))
    idx, S = pol.select_tail_mean(K, Q, W=128, k=5)
    Kf, Qf = nm.bf16_to_f32(K), nm.bf16_to_f32(Q)
    P = L - 128
    t = min(128, LQ)
    for h in range(Hkv * g):
        for j in range(P):
            tot = 0.0
            for i in range(LQ - t, LQ):
                tot += sum(float(Qf[h, i, d]) * float(Kf[h // g, j, d]) for d in range(D))
            assert abs(S[h, j] - tot / t) <= 1e-12 * (1 + abs(tot))
    # a query outside the tail changes nothing; one inside does
    if LQ > 128:
        Q2 = Q.copy()
        Q2[:, LQ - 129] = _bits(rng, (Hkv * g, D), 10.0)
        assert np.array_equal(pol.select_tail_mean(K, Q2, k=5)[1], S)
    Q3 = Q.copy()
    Q3[:, LQ - 1] = _bits(rng, (Hkv * g, D), 10.0)
    assert not np.array_equal(pol.select_tail_mean(K, Q3, k=5)[1], S)


def test_tail_mean_gqa_form_equals_repeated_kv():
    """Alg. 1's GQA-native branch must give what the H = H_Q branch gives on keys repeated
    per Q head (Q head h reads KV head h // g)."""
    rng = np.random.default_rng(11)
    Hkv, g, L, D = 3, 4, 400, 16
    K = _bits(rng, (Hkv, L, D))
    Q = _bits(rng, (Hkv * g, 200, D))
    idx, S = pol.select_tail_mean(K, Q)
    idx_r, S_r = pol.select_tail_mean(np.repeat(K, g, axis=0), Q)
    assert np.array_equal(S, S_r) and np.array_equal(idx, idx_r)
    assert idx.shape == (Hkv * g, pol.k_alg1(L - 128))


def test_tail_mean_planted_and_degenerate():
    rng = np.random.default_rng(12)
    Hkv, g, L, D = 1, 2, 600, 32
    K = nm.bf16_to_f32(_bits(rng, (Hkv, L, D), 0.1))
    Q = nm.bf16_to_f32(_bits(rng, (Hkv * g, 128, D), 0.1))
    u = np.zeros(D, np.float32)
    u[3] = 1.0
    Q[0] += 2.0 * u  # head 0's tail mean points along u
    planted = [17, 250, 401]
    for j in planted:
        K[0, j] += 3.0 * u
    idx, S = pol.select_tail_mean(nm.f32_to_bf16(K), nm.f32_to_bf16(Q), k=3)
    assert list(idx[0]) == planted
    # the window is never a candidate, and P = 0 selects nothing
    assert S.shape == (2, L - 128)
    idx0, S0 = pol.select_tail_mean(nm.f32_to_bf16(K[:, :128]), nm.f32_to_bf16(Q))
    assert idx0.shape == (2, 0) and S0.shape == (2, 0)


def test_cache_8bit_bulk_is_finer_and_keeps_the_rest():
    """bits = 8 changes only the quantized bulk: windows, anchors and staging keep bf16, the
    quantized positions are the same, and their error is smaller than with INT4."""
    s = synth.HeadStream(91, 700, 4)
    A, _ = pol.select_dense(s.K, s.queries(64))
    c4, c8 = pol.HybridCacheRef(g=4), pol.HybridCacheRef(g=4, bits=8)
    for c in (c4, c8):
        c.freeze(s.K, s.V, A)
    assert c4.counts() == c8.counts() and np.array_equal(c4.anchors(), c8.anchors())
    K4, V4 = c4.stored_kv()
    K8, V8 = c8.stored_kv()
    K, V = nm.bf16_to_f32(s.K), nm.bf16_to_f32(s.V)
    q = c4.kind[:700] == pol.INT4
    assert np.array_equal(K8[~q], K[~q]) and np.array_equal(V8[~q], V[~q])
    assert np.abs(K8[q] - K[q]).mean() < np.abs(K4[q] - K[q]).mean() / 8
    assert c8.kc[:700][q].max() > 15


@pytest.mark.parametrize("bk,bv", [(4, 2), (2, 2)])
def test_cache_2bit_bulk_widths_are_per_operand(bk, bv):
    """bits / bits_v set B_K and B_V separately: K codes follow bits, V codes bits_v; the
    bf16 segments and the quantized positions do not depend on either, and the V error grows
    as B_V drops (3 levels against 15)."""
    s = synth.HeadStream(92, 600, 4)
    A, _ = pol.select_dense(s.K, s.queries(64))
    c44 = pol.HybridCacheRef(g=4)
    cx = pol.HybridCacheRef(g=4, bits=bk, bits_v=bv)
    for c in (c44, cx):
        c.freeze(s.K, s.V, A)
    assert c44.counts() == cx.counts() and np.array_equal(c44.anchors(), cx.anchors())
    q = c44.kind[:600] == pol.INT4
    assert cx.kc[:600][q].max() == (1 << bk) - 1 and cx.vc[:600][q].max() == (1 << bv) - 1
    if bk == 4:
        assert np.array_equal(cx.kc[:600][q], c44.kc[:600][q])  # K unchanged by bits_v
    K, V = nm.bf16_to_f32(s.K), nm.bf16_to_f32(s.V)
    K44, V44 = c44.stored_kv()
    Kx, Vx = cx.stored_kv()
    assert np.array_equal(Vx[~q], V[~q]) and np.array_equal(Kx[~q], K[~q])
    assert np.abs(Vx[q] - V[q]).mean() > 3 * np.abs(V44[q] - V[q]).mean()

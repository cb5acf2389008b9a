"""Precision policy of the oracle: anchor count, vertical-line scores, top-k, and the
hybrid KV-cache state machine (test infrastructure only).

"HyQuant paper" = the arXiv page "HyQuant: Hybrid-Precision Quantization for LLM
Attention"; "techwalker article" = the techwalker.com article summarising it.

Readings of the pages taken here:
  * The window is sliding: the last W positions [L-W, L) of the current length L
    (§4.1 Eq. 2 read with t0 = current length), W = 128 (§5.1, Table 15).
  * Anchors ("vertical lines") are chosen from the non-window prefix [0, L-W)
    (§4.1 Eq. 1, Eq. 3, Eq. 5).
  * Their count is k = min(P, max(1, ceil(rho * L))) with P = L - W candidates,
    and k = 0 when P = 0 (the clamp and the empty case of Alg. 1).  Reading: the ratio
    is applied to the context length L (5% of a 1024-position context = 52 anchors),
    not to P as Alg. 1 writes it.
  * The score of a key is its summed attention probability over the proxy queries
    of all Q heads of its KV group, softmax taken over every cached key (Eq. 4; GQA
    handled per KV head as in Alg. 1's GQA-native form and Alg. 4's per-KV-head
    gather).  Ties in top-k go to the lower position; output is ascending.
  * A token leaving the window waits in bf16 staging (Alg. 3 segment 3; Alg. 4
    staging buffer).  The selector runs every 64 decode tokens (techwalker article,
    design section); at that refresh staged tokens become anchors or INT4.
  * At a refresh a position in the new set keeps/gets bf16: anchors keep theirs,
    staged tokens keep their original bf16, an INT4 position is promoted with
    bf16(dequantized value) -- its original was freed at Freeze (Alg. 4), so no
    precision is recovered.  Anchors and staged tokens not in the new set are
    quantized from the bf16 values they hold.
"""
from __future__ import annotations

import numpy as np

from . import numerics as nm

WIN, STAGED, ANCHOR, INT4 = 0, 1, 2, 3


def k_rule(L: int, W: int = 128, pct_num: int = 5, pct_den: int = 100) -> int:
    """Number of anchors for context length L: k = min(P, max(1, ceil(L*num/den))),
    P = max(0, L - W); P = 0 gives k = 0 (HyQuant paper Alg. 1: P = max(0, L_K - W),
    empty result when P = 0, clamp of k to [1, P]).  Integer arithmetic only."""
    P = max(0, L - W)
    if P == 0:
        return 0
    k = (L * pct_num + pct_den - 1) // pct_den
    return min(P, max(1, k))


def softmax_rows(logits: np.ndarray) -> np.ndarray:
    """Row softmax in fp64 (max-subtracted)."""
    z = np.asarray(logits, dtype=np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def vertical_scores(proxy: np.ndarray, keys: np.ndarray, n_cand: int) -> np.ndarray:
    """S(j) = sum_t a_{t,j} for j < n_cand (HyQuant paper §4.1 Eq. 4).

    proxy: [R][D] fp32 values of the proxy rows (all proxies of all Q heads of the KV
    group); keys: [L][D] fp32 values of every cached key in its stored precision.
    a_{t,.} = softmax(alpha * proxy_t . keys^T) over all L keys, alpha = 1/sqrt(D)
    (Alg. 2/3 scale).  Computed in fp64.
    """
    proxy = np.asarray(proxy, np.float64)
    keys = np.asarray(keys, np.float64)
    if proxy.shape[0] == 0 or keys.shape[0] == 0:
        return np.zeros(n_cand)
    alpha = 1.0 / np.sqrt(keys.shape[1])
    p = softmax_rows(alpha * (proxy @ keys.T))
    return p[:, :n_cand].sum(axis=0)


def topk_lower_index(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, ties to the lower index, returned ascending
    (HyQuant paper Eq. 5 / Alg. 1 TopK; tie rule is a reading)."""
    scores = np.asarray(scores)
    if k <= 0:
        return np.zeros(0, np.int64)
    order = np.lexsort((np.arange(len(scores)), -scores))
    return np.sort(order[:k])


def near_tie_gap(scores: np.ndarray, k: int) -> float:
    """Relative gap between the k-th and (k+1)-th largest score (inf when k covers all)."""
    s = np.sort(np.asarray(scores, np.float64))[::-1]
    if k <= 0 or k >= len(s):
        return np.inf
    return float((s[k - 1] - s[k]) / max(abs(s[k - 1]), 1e-300))


class HybridCacheRef:
    """Hybrid-precision KV cache of one (sequence, KV head), kept per position.

    Four kinds of storage (HyQuant paper Alg. 3 segments / Alg. 4 buffers):
      WIN    -- last W positions, bf16 (local window)
      STAGED -- left the window since the last refresh, bf16 (staging buffer)
      ANCHOR -- vertical-line positions, bf16
      INT4   -- everything else: per token, per 32-channel group asymmetric INT4 with
                fp16 scale and minimum (numerics.quant_asym); ``bits`` sets B_K and
                ``bits_v`` B_V (default: B_K), 2^bits - 1 levels each (the bit widths are
                parameters of Alg. 3 and Alg. 4: 8 gives K8V8, bits=4 with bits_v=2 K4V2)
    The value of a position is its bf16 value, or the dequantized INT4 value.
    """

    def __init__(self, D: int = 128, W: int = 128, group: int = 32, g: int = 4,
                 proxy_cap: int = 64, bits: int = 4, bits_v: int | None = None):
        self.D, self.W, self.group, self.g, self.proxy_cap = D, W, group, g, proxy_cap
        self.bits = bits
        self.bits_v = bits if bits_v is None else bits_v
        self.L = 0
        self.kind = np.zeros(0, np.int8)
        self.kb = np.zeros((0, D), np.uint16)  # bf16 K (valid for WIN/STAGED/ANCHOR)
        self.vb = np.zeros((0, D), np.uint16)
        self.kc = np.zeros((0, D), np.uint8)  # INT4 codes (valid for INT4)
        self.vc = np.zeros((0, D), np.uint8)
        ng = D // group
        self.ks = np.zeros((0, ng), np.float16)
        self.km = np.zeros((0, ng), np.float16)
        self.vs = np.zeros((0, ng), np.float16)
        self.vm = np.zeros((0, ng), np.float16)
        self.proxy = np.zeros((g, 0, D), np.uint16)  # last <= proxy_cap queries per Q head

    # -- storage helpers -----------------------------------------------------------
    def _grow(self, n: int) -> None:
        if n <= len(self.kind):
            return
        extra = n - len(self.kind)
        ng = self.D // self.group
        self.kind = np.concatenate([self.kind, np.zeros(extra, np.int8)])
        self.kb = np.concatenate([self.kb, np.zeros((extra, self.D), np.uint16)])
        self.vb = np.concatenate([self.vb, np.zeros((extra, self.D), np.uint16)])
        self.kc = np.concatenate([self.kc, np.zeros((extra, self.D), np.uint8)])
        self.vc = np.concatenate([self.vc, np.zeros((extra, self.D), np.uint8)])
        for name in ("ks", "km", "vs", "vm"):
            setattr(self, name, np.concatenate([getattr(self, name), np.zeros((extra, ng), np.float16)]))

    def _quantize_positions(self, pos: np.ndarray) -> None:
        """Quantize the bf16 values held at ``pos`` to INT4 (Alg. 4 Quant, G = 32)."""
        if len(pos) == 0:
            return
        c, s, m = nm.quant_int4_token(nm.bf16_to_f32(self.kb[pos]), self.group, self.bits)
        self.kc[pos], self.ks[pos], self.km[pos] = c, s, m
        c, s, m = nm.quant_int4_token(nm.bf16_to_f32(self.vb[pos]), self.group, self.bits_v)
        self.vc[pos], self.vs[pos], self.vm[pos] = c, s, m
        self.kind[pos] = INT4

    def _push_proxy(self, q: np.ndarray) -> None:
        q = np.asarray(q, np.uint16).reshape(self.g, -1, self.D)
        self.proxy = np.concatenate([self.proxy, q], axis=1)[:, -self.proxy_cap:]

    # -- the method ------------------------------------------------------------------
    def freeze(self, K: np.ndarray, V: np.ndarray, anchors, q_tail=None) -> None:
        """Prefill -> decode cache organisation (HyQuant paper Alg. 4): the last W keys
        become the window, ``anchors`` (ascending, inside [0, L-W)) keep bf16, the rest
        of [0, L-W) is quantized.  The staging buffer starts empty.  ``q_tail``
        ([g][n][D]) seeds the proxy-query buffer (at most 64 per head, §5.5)."""
        K = np.asarray(K, np.uint16)
        V = np.asarray(V, np.uint16)
        L = K.shape[0]
        self.L = 0
        self._grow(L)
        self.L = L
        self.kb[:L], self.vb[:L] = K, V
        P = max(0, L - self.W)
        anchors = np.asarray(anchors, np.int64)
        assert np.all(np.diff(anchors) > 0) and (len(anchors) == 0 or (anchors[0] >= 0 and anchors[-1] < P))
        self.kind[P:L] = WIN
        qpos = np.setdiff1d(np.arange(P), anchors)
        self._quantize_positions(qpos)
        self.kind[anchors] = ANCHOR
        self.proxy = np.zeros((self.g, 0, self.D), np.uint16)
        if q_tail is not None:
            self._push_proxy(np.asarray(q_tail, np.uint16))

    def append(self, k: np.ndarray, v: np.ndarray, q: np.ndarray | None = None) -> None:
        """One decode step's cache update: position L enters the window; the position
        that falls out of the window (L - W) goes to staging in bf16 (Alg. 3 segment 3,
        Alg. 4 staging buffer); the step's queries enter the proxy buffer."""
        L = self.L
        self._grow(L + 1)
        if L >= self.W:
            self.kind[L - self.W] = STAGED
        self.kind[L] = WIN
        self.kb[L], self.vb[L] = np.asarray(k, np.uint16), np.asarray(v, np.uint16)
        self.L = L + 1
        if q is not None:
            self._push_proxy(np.asarray(q, np.uint16).reshape(self.g, 1, self.D))

    def refresh(self, new_anchors) -> None:
        """Apply a new vertical-line set (the module docstring gives the reading)."""
        new_anchors = np.asarray(new_anchors, np.int64)
        P = max(0, self.L - self.W)
        assert len(new_anchors) == 0 or (new_anchors[0] >= 0 and new_anchors[-1] < P)
        inset = np.zeros(P, bool)
        inset[new_anchors] = True
        kind = self.kind[:P]
        promote = np.flatnonzero(inset & (kind == INT4))
        if len(promote):
            kh = nm.dequant_int4_token(self.kc[promote], self.ks[promote], self.km[promote], self.group)
            vh = nm.dequant_int4_token(self.vc[promote], self.vs[promote], self.vm[promote], self.group)
            self.kb[promote], self.vb[promote] = nm.f32_to_bf16(kh), nm.f32_to_bf16(vh)
        demote = np.flatnonzero(~inset & ((kind == ANCHOR) | (kind == STAGED)))
        self._quantize_positions(demote)
        self.kind[np.flatnonzero(inset)] = ANCHOR

    # -- views -----------------------------------------------------------------------
    def counts(self) -> dict:
        k = self.kind[:self.L]
        return dict(L=self.L, win=int((k == WIN).sum()), staged=int((k == STAGED).sum()),
                    anchor=int((k == ANCHOR).sum()), int4=int((k == INT4).sum()))

    def anchors(self) -> np.ndarray:
        return np.flatnonzero(self.kind[:self.L] == ANCHOR)

    def stored_kv(self) -> tuple[np.ndarray, np.ndarray]:
        """fp32 K, V of every position in its stored precision (position order)."""
        L = self.L
        Kh = nm.bf16_to_f32(self.kb[:L]).copy()
        Vh = nm.bf16_to_f32(self.vb[:L]).copy()
        qi = np.flatnonzero(self.kind[:L] == INT4)
        if len(qi):
            Kh[qi] = nm.dequant_int4_token(self.kc[qi], self.ks[qi], self.km[qi], self.group)
            Vh[qi] = nm.dequant_int4_token(self.vc[qi], self.vs[qi], self.vm[qi], self.group)
        return Kh, Vh

    def proxy_rows(self) -> np.ndarray:
        """Proxy rows [g * n][D] (fp32), Q head major."""
        return nm.bf16_to_f32(self.proxy.reshape(-1, self.D))

    def select(self, pct_num: int = 5, pct_den: int = 100):
        """Scores of every candidate in [0, L-W) and the new anchor set (Eq. 4-5)."""
        P = max(0, self.L - self.W)
        k = k_rule(self.L, self.W, pct_num, pct_den)
        Kh, _ = self.stored_kv()
        S = vertical_scores(self.proxy_rows(), Kh, P)
        return topk_lower_index(S, k), S


def select_dense(K_bits: np.ndarray, proxy_bits: np.ndarray, W: int = 128, pct_num: int = 5,
                 pct_den: int = 100):
    """Selector at Freeze on the dense bf16 prefix (Alg. 4: the set comes from the prefill tail queries):
    K_bits [L][D]; proxy_bits [g][n][D] (the last prefill queries of the group)."""
    K = nm.bf16_to_f32(K_bits)
    L, D = K.shape
    P = max(0, L - W)
    k = k_rule(L, W, pct_num, pct_den)
    S = vertical_scores(nm.bf16_to_f32(np.asarray(proxy_bits).reshape(-1, D)), K, P)
    return topk_lower_index(S, k), S


# ---------------------------------------------------------------- Alg. 1 taken literally
def k_alg1(P: int, r_num: int = 5, r_den: int = 100) -> int:
    """Anchor count as the HyQuant paper's Alg. 1 writes it: k = min(P, max(1, ceil(P r))) on
    the P = L - W candidates (0 when P = 0), ratio r = r_num / r_den, integers only."""
    if P <= 0:
        return 0
    return min(P, max(1, (P * r_num + r_den - 1) // r_den))


def tail_query_mean(Q_bits: np.ndarray, W: int = 128) -> np.ndarray:
    """The tail-query proxy of HyQuant paper Alg. 1: the mean of the last t = min(W, L_Q)
    queries of each Q head.  Q_bits [H][L_Q][D] bf16 bits -> fp64 [H][D]."""
    Q = nm.bf16_to_f32(Q_bits).astype(np.float64)
    t = min(W, Q.shape[1])
    return Q[:, Q.shape[1] - t:, :].mean(axis=1)


def select_tail_mean(K_bits: np.ndarray, Q_bits: np.ndarray, W: int = 128, r_num: int = 5,
                     r_den: int = 100, k: int | None = None):
    """Vertical-token identification as HyQuant paper Alg. 1 writes it, for one sequence:
    the candidates are the prefix [0, P), P = max(0, L_K - W) (empty when P = 0); each Q head
    h scores them with raw logits S_h(j) = qbar_h . k_j (no softmax, no 1/sqrt(D)) of its
    tail-query mean qbar_h against its KV head h // g (the GQA-native form); the set of each
    Q head is its own top-k (ties to the lower position, ascending).
    K_bits [Hkv][L_K][D], Q_bits [Hq][L_Q][D] (bf16 bits).  k: defaults to ``k_alg1(P)``.
    Returns (idx int64 [Hq][k], S fp64 [Hq][P])."""
    K = nm.bf16_to_f32(K_bits).astype(np.float64)
    Hkv, L, D = K.shape
    Hq = Q_bits.shape[0]
    g = Hq // Hkv
    P = max(0, L - W)
    if k is None:
        k = k_alg1(P, r_num, r_den)
    qbar = tail_query_mean(Q_bits, W)
    S = np.zeros((Hq, P))
    for hk in range(Hkv):
        # the g Q heads of KV head hk against its prefix keys: [g][D] x [D][P]
        S[hk * g:(hk + 1) * g] = qbar[hk * g:(hk + 1) * g] @ K[hk, :P].T
    idx = np.zeros((Hq, k), np.int64)
    for h in range(Hq):
        idx[h] = topk_lower_index(S[h], k)
    return idx, S

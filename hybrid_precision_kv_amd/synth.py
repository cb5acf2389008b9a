"""Seeded synthetic inputs shared by the tests, the bench and the oracle's checks.

This module draws random numbers and rounds them to bf16 storage; it holds none of
the attention method's arithmetic.  Both the HIP path (via the tests and the bench)
and the CPU oracle consume its outputs, which is the only thing they share.

Workload model (the pages evaluate on real long-context prompts; those datasets and
model weights are not available, so this generator stands in for them with their
shapes):

* K, V ~ N(0, 1), rounded to bf16 (round-to-nearest-even).
* Per (sequence, KV head) a random unit vector ``u`` and ``n_planted`` planted
  "vertical-line" keys: position 0 plus ``n_planted - 1`` distinct positions drawn
  uniformly from ``[1, L - window)``; each planted key becomes ``k + 4u``.  This
  mimics the persistent attention anchors described in the HyQuant paper (§2.1,
  Table 1, Fig. 1).
* Queries of that KV head's group (decode queries and proxy queries): ``2u + N(0,1)``.

All arrays are returned as numpy ``uint16`` bf16 bit patterns so that both sides
start from identical bits.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128
WINDOW = 128


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (input preparation only)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> fp32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def seed_for(base: int, b: int, h: int) -> int:
    """Per-(sequence, KV head) seed: ``base + 97*b + h``."""
    return int(base) + 97 * int(b) + int(h)


class HeadStream:
    """Random stream for one (sequence, KV head): prefix K/V, planted anchors, queries."""

    def __init__(self, seed: int, L: int, g: int, D: int = HEAD_DIM, window: int = WINDOW,
                 n_planted: int = 16):
        self.rng = np.random.Generator(np.random.PCG64(seed))
        self.L, self.g, self.D, self.window = L, g, D, window
        u = self.rng.standard_normal(D)
        self.u = (u / np.linalg.norm(u)).astype(np.float32)
        K = self.rng.standard_normal((L, D), dtype=np.float32)
        V = self.rng.standard_normal((L, D), dtype=np.float32)
        cand_hi = L - window
        planted = [0] if L > 0 else []
        if cand_hi > 1 and n_planted > 1:
            n_extra = min(n_planted - 1, cand_hi - 1)
            planted += list(1 + self.rng.choice(cand_hi - 1, size=n_extra, replace=False))
        self.planted = np.array(sorted(planted), dtype=np.int64)
        if len(self.planted):
            K[self.planted] += 4.0 * self.u
        self.K = _to_bf16_bits(K)
        self.V = _to_bf16_bits(V)

    def queries(self, n: int) -> np.ndarray:
        """``n`` query vectors per Q head of the group: uint16 ``[g][n][D]``."""
        q = 2.0 * self.u + self.rng.standard_normal((self.g, n, self.D), dtype=np.float32)
        return _to_bf16_bits(q)

    def new_tokens(self, n: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
        """``n`` decode-time tokens: k ``[n][D]``, v ``[n][D]``, q ``[g][n][D]`` (uint16)."""
        k = _to_bf16_bits(self.rng.standard_normal((n, self.D), dtype=np.float32))
        v = _to_bf16_bits(self.rng.standard_normal((n, self.D), dtype=np.float32))
        return k, v, self.queries(n)


def gen_batch(seed_base: int, B: int, Hkv: int, g: int, L: int, n_proxy: int = 64,
              n_steps: int = 0, D: int = HEAD_DIM, window: int = WINDOW, n_planted: int = 16):
    """Draw a whole batch.

    Returns a dict of uint16 arrays:
      K, V        [B][Hkv][L][D]        prefix keys/values
      proxy       [B][Hkv*g][n_proxy][D] proxy queries (the tail of prefill)
      new_k/new_v [B][Hkv][n_steps][D]  decode-time tokens
      new_q       [B][Hkv*g][n_steps][D] decode-time queries
      planted     list of per-(b,h) planted positions
    Q head ``h_kv*g + j`` belongs to KV head ``h_kv`` (grouped-query layout).
    """
    K = np.empty((B, Hkv, L, D), np.uint16)
    V = np.empty_like(K)
    proxy = np.empty((B, Hkv * g, n_proxy, D), np.uint16)
    nk = np.empty((B, Hkv, n_steps, D), np.uint16)
    nv = np.empty_like(nk)
    nq = np.empty((B, Hkv * g, n_steps, D), np.uint16)
    planted = []
    for b in range(B):
        row = []
        for h in range(Hkv):
            s = HeadStream(seed_for(seed_base, b, h), L, g, D, window, n_planted)
            K[b, h], V[b, h] = s.K, s.V
            proxy[b, h * g:(h + 1) * g] = s.queries(n_proxy)
            if n_steps:
                k, v, q = s.new_tokens(n_steps)
                nk[b, h], nv[b, h] = k, v
                nq[b, h * g:(h + 1) * g] = q
            row.append(s.planted)
        planted.append(row)
    return dict(K=K, V=V, proxy=proxy, new_k=nk, new_v=nv, new_q=nq, planted=planted)


def gen_prefill(seed_base: int, Hq: int, Hkv: int, N: int, D: int = HEAD_DIM,
                window: int = WINDOW, n_planted: int = 16):
    """Prefill inputs for one sequence: Q [Hq][N][D], K, V [Hkv][N][D] (uint16 bf16 bits).

    Queries follow the same planted-direction model as decode queries.
    """
    g = Hq // Hkv
    Q = np.empty((Hq, N, D), np.uint16)
    K = np.empty((Hkv, N, D), np.uint16)
    V = np.empty_like(K)
    planted = []
    for h in range(Hkv):
        s = HeadStream(seed_for(seed_base, 0, h), N, g, D, window, n_planted)
        K[h], V[h] = s.K, s.V
        Q[h * g:(h + 1) * g] = s.queries(N)
        planted.append(s.planted)
    return dict(Q=Q, K=K, V=V, planted=planted)

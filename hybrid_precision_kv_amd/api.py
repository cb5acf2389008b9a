"""Python binding of the C ABI (include/hyq.h): torch tensors in, the same calls out.

Every step of the method runs in the HIP library; this module checks tensor shapes/dtypes,
allocates caller-owned buffers with torch, and passes pointers plus the current HIP stream.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import HyqCache, HyqShape, check

D = 128
WINDOW = 128
PROXY_CAP = 64


def _stream() -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor | None) -> C.c_void_p:
    return C.c_void_p(0 if t is None else t.data_ptr())


def _bf16(t: torch.Tensor, shape: tuple, name: str) -> torch.Tensor:
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name}: expected bfloat16 (or its 16-bit pattern), got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous device tensor")
    return t


def anchor_count(L: int, pct_num: int = 5, pct_den: int = 100, window: int = WINDOW) -> int:
    """k = min(P, max(1, ceil(L * pct))) with P = max(0, L - window); 0 when P = 0."""
    P = max(0, L - window)
    if P == 0:
        return 0
    return min(P, max(1, -(-L * pct_num // pct_den)))


def anchor_count_alg1(L: int, r_num: int = 5, r_den: int = 100, window: int = WINDOW) -> int:
    """Alg. 1's count on the candidates: k = min(P, max(1, ceil(P r))), P = max(0, L - window)."""
    P = max(0, L - window)
    if P == 0:
        return 0
    return min(P, max(1, -(-P * r_num // r_den)))


@dataclass
class Shape:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    int4_cap: int
    anchor_cap: int
    staging_cap: int = 64
    bits: int = 4  # B_K: bits of the quantized bulk's K codes (4, 8 or 2)
    bits_v: int = 0  # B_V: bits of its V codes (0 = B_K; K4V2 is bits=4, bits_v=2)

    def c(self) -> HyqShape:
        return HyqShape(self.batch, self.n_q_heads, self.n_kv_heads, D, 32, WINDOW, PROXY_CAP,
                        self.staging_cap, self.int4_cap, self.anchor_cap, self.bits, self.bits_v)

    @property
    def g(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @staticmethod
    def for_context(batch: int, n_q_heads: int, n_kv_heads: int, max_len: int, pct_num: int = 5,
                    staging_cap: int = 64, bits: int = 4, bits_v: int = 0) -> "Shape":
        """Capacities for contexts up to ``max_len`` with anchors at ``pct_num``%."""
        r32 = lambda x: max(32, -(-x // 32) * 32)
        k = anchor_count(max_len, pct_num)
        return Shape(batch, n_q_heads, n_kv_heads, r32(max(0, max_len - WINDOW)), r32(k), r32(staging_cap), bits,
                     bits_v)


def buffer_bytes(shape: Shape) -> dict:
    lib = _lib.load()
    out = (C.c_size_t * _lib.HYQ_NBUF)()
    s = shape.c()
    check("hyq_cache_buffer_bytes", lib.hyq_cache_buffer_bytes(C.byref(s), C.byref(out)))
    return {name: int(out[i]) for i, name in enumerate(_lib.BUFFERS)}


def workspace_bytes(shape: Shape, op: int, length: int = 0, n_splits: int = 0) -> int:
    lib = _lib.load()
    s = shape.c()
    return int(lib.hyq_workspace_bytes(C.byref(s), op, length, n_splits))


class HybridKVCache:
    """Caller-owned device buffers of the hybrid cache plus the host counters."""

    def __init__(self, shape: Shape, device: str | torch.device = "cuda"):
        self.shape = shape
        self.device = torch.device(device)
        sizes = buffer_bytes(shape)
        self.buffers = {n: torch.empty(max(16, b), dtype=torch.uint8, device=self.device) for n, b in sizes.items()}
        self.c = HyqCache()
        self.c.shape = shape.c()
        for n, t in self.buffers.items():
            setattr(self.c, n, t.data_ptr())

    # counters
    @property
    def len(self) -> int: return self.c.len
    @property
    def n_int4(self) -> int: return self.c.n_int4
    @property
    def n_anchor(self) -> int: return self.c.n_anchor
    @property
    def n_staged(self) -> int: return self.c.n_staged
    @property
    def n_proxy(self) -> int: return self.c.n_proxy

    def counters(self) -> dict:
        return {k: getattr(self.c, k) for k in ("len", "n_int4", "n_anchor", "n_staged", "n_proxy", "proxy_head")}

    def snapshot(self) -> tuple[dict, dict]:
        """Copy of the device buffers and the host counters (checkpoint)."""
        return {n: t.clone() for n, t in self.buffers.items()}, self.counters()

    def restore(self, snap: tuple[dict, dict]) -> None:
        bufs, ctr = snap
        for n, t in bufs.items():
            self.buffers[n].copy_(t)
        for k, v in ctr.items():
            setattr(self.c, k, v)

    def view(self, name: str, dtype: torch.dtype) -> torch.Tensor:
        return self.buffers[name].view(dtype)


def quantize_kv(cache: HybridKVCache, k: torch.Tensor, v: torch.Tensor, anchors: torch.Tensor | None = None,
                q_tail: torch.Tensor | None = None) -> None:
    """Freeze a dense prefill cache into the hybrid layout (hyq_quantize_kv)."""
    s = cache.shape
    L = k.shape[2]
    _bf16(k, (s.batch, s.n_kv_heads, L, D), "k")
    _bf16(v, (s.batch, s.n_kv_heads, L, D), "v")
    n_anchor = 0
    if anchors is not None:
        if anchors.dtype != torch.int32 or not anchors.is_cuda or not anchors.is_contiguous():
            raise TypeError("anchors: contiguous int32 device tensor expected")
        if anchors.dim() != 3 or anchors.shape[:2] != (s.batch, s.n_kv_heads):
            raise ValueError("anchors: shape [B][Hkv][k] expected")
        n_anchor = anchors.shape[2]
    n_tail = 0
    if q_tail is not None:
        n_tail = q_tail.shape[2]
        _bf16(q_tail, (s.batch, s.n_q_heads, n_tail, D), "q_tail")
    lib = _lib.load()
    check("hyq_quantize_kv", lib.hyq_quantize_kv(C.byref(cache.c), _ptr(k), _ptr(v), L,
                                                 _ptr(anchors if n_anchor else None), n_anchor,
                                                 _ptr(q_tail), n_tail, _stream()))


def append_token(cache: HybridKVCache, k_t: torch.Tensor, v_t: torch.Tensor, q_t: torch.Tensor | None = None) -> None:
    s = cache.shape
    _bf16(k_t, (s.batch, s.n_kv_heads, D), "k_t")
    _bf16(v_t, (s.batch, s.n_kv_heads, D), "v_t")
    if q_t is not None:
        _bf16(q_t, (s.batch, s.n_q_heads, D), "q_t")
    lib = _lib.load()
    check("hyq_append_token", lib.hyq_append_token(C.byref(cache.c), _ptr(k_t), _ptr(v_t), _ptr(q_t), _stream()))


class _Workspace:
    def __init__(self):
        self.t = None

    def get(self, nbytes: int, device) -> torch.Tensor:
        if self.t is None or self.t.numel() < nbytes or self.t.device != device:
            self.t = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.t


_ws = _Workspace()
_ws_ragged = _Workspace()


def decode_workspace(shape: Shape, n_splits: int = 0, device="cuda") -> torch.Tensor:
    """A decode workspace for ``n_splits`` splits (0 = automatic)."""
    return torch.empty(max(workspace_bytes(shape, _lib.HYQ_OP_DECODE, 0, n_splits), 256), dtype=torch.uint8,
                       device=device)


def decode_attn(cache: HybridKVCache, q: torch.Tensor, n_splits: int = 0, out: torch.Tensor | None = None,
                ws: torch.Tensor | None = None) -> torch.Tensor:
    """o = softmax(q K^T / sqrt(128)) V over the hybrid cache (hyq_decode_attn); fp32 out.
    ``ws`` (optional) must come from ``decode_workspace``."""
    s = cache.shape
    _bf16(q, (s.batch, s.n_q_heads, D), "q")
    if out is None:
        out = torch.empty((s.batch, s.n_q_heads, D), dtype=torch.float32, device=q.device)
    need = workspace_bytes(s, _lib.HYQ_OP_DECODE, 0, n_splits)
    if ws is None:
        ws = _ws.get(need, q.device)
    lib = _lib.load()
    check("hyq_decode_attn", lib.hyq_decode_attn(C.byref(cache.c), _ptr(q), _ptr(out), n_splits, _ptr(ws),
                                                 ws.numel(), _stream()))
    return out


def decode_attn_noalloc(cache: HybridKVCache, q: torch.Tensor, out: torch.Tensor, n_splits: int = 0) -> torch.Tensor:
    """hyq_decode_attn_noalloc: the decode with its split records in the library's static
    per-GPU scratch (no allocation anywhere; ``out`` is the caller's fp32 [B][Hq][128])."""
    s = cache.shape
    _bf16(q, (s.batch, s.n_q_heads, D), "q")
    if out.dtype != torch.float32 or tuple(out.shape) != (s.batch, s.n_q_heads, D) or not out.is_contiguous():
        raise ValueError("out: contiguous float32 [B][Hq][128]")
    lib = _lib.load()
    check("hyq_decode_attn_noalloc", lib.hyq_decode_attn_noalloc(C.byref(cache.c), _ptr(q), _ptr(out), n_splits,
                                                                 _stream()))
    return out


def decode_ragged_workspace_bytes(shape: Shape, n_seq: int, n_splits: int = 0) -> int:
    lib = _lib.load()
    s = shape.c()
    return int(lib.hyq_decode_ragged_workspace_bytes(C.byref(s), n_seq, n_splits))


def decode_ragged_table_bytes(shape: Shape, n_seq: int, n_splits: int = 0) -> int:
    lib = _lib.load()
    s = shape.c()
    return int(lib.hyq_decode_ragged_table_bytes(C.byref(s), n_seq, n_splits))


def decode_ragged_table(shape: Shape, n_seq: int, n_splits: int = 0) -> torch.Tensor:
    """A page-locked host table for hyq_decode_attn_ragged (uint8)."""
    need = decode_ragged_table_bytes(shape, n_seq, n_splits)
    if need == 0:
        raise ValueError("unsupported ragged batch (sequence count or split count out of range)")
    return torch.empty(need, dtype=torch.uint8, pin_memory=True)


class _TableRing:
    """Page-locked tables used in turn by calls that pass none: a table is written again only
    after the stream has passed the call that last used it (an event per table)."""

    SLOTS = 8

    def __init__(self):
        self.tabs = [None] * self.SLOTS
        self.events = [None] * self.SLOTS
        self.i = 0

    def get(self, nbytes: int):
        i = self.i
        self.i = (i + 1) % self.SLOTS
        if self.events[i] is not None:
            self.events[i].synchronize()
            self.events[i] = None
        if self.tabs[i] is None or self.tabs[i].numel() < nbytes:
            self.tabs[i] = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        return i, self.tabs[i]

    def used(self, i: int) -> None:
        ev = torch.cuda.Event()
        ev.record()
        self.events[i] = ev


_tables = _TableRing()


def _cache_ptrs(caches: list):
    return (C.POINTER(_lib.HyqCache) * len(caches))(*[C.pointer(c.c) for c in caches])


def decode_ragged_plan(caches: list, table: torch.Tensor, n_splits: int = 0) -> int:
    """Rewrite ``table`` for the caches' current counters (hyq_decode_ragged_plan, host only);
    returns the total split count, which must equal the one a captured call recorded."""
    total = C.c_int32(0)
    lib = _lib.load()
    check("hyq_decode_ragged_plan", lib.hyq_decode_ragged_plan(_cache_ptrs(caches), len(caches), n_splits,
                                                               _ptr(table), table.numel(), C.byref(total)))
    return int(total.value)


def decode_attn_ragged(caches: list, q: torch.Tensor, n_splits: int = 0, out: torch.Tensor | None = None,
                       ws: torch.Tensor | None = None, table: torch.Tensor | None = None) -> torch.Tensor:
    """Decode over a variable-length batch (hyq_decode_attn_ragged): ``caches`` are
    single-sequence caches of any lengths with the same heads and bit width; q [n][Hq][128]
    bf16, one row block per cache; fp32 out [n][Hq][128].  ``table``: a page-locked host table
    from ``decode_ragged_table`` that the caller keeps alive and unchanged until the stream has
    passed the call (needed when the call is captured into a graph); without one, the
    binding's own ring of tables is used."""
    n = len(caches)
    s = caches[0].shape
    _bf16(q, (n, s.n_q_heads, D), "q")
    if out is None:
        out = torch.empty((n, s.n_q_heads, D), dtype=torch.float32, device=q.device)
    need = decode_ragged_workspace_bytes(s, n, n_splits)
    if need == 0:
        raise ValueError("unsupported ragged batch (sequence count or split count out of range)")
    if ws is None:
        ws = _ws_ragged.get(need, q.device)
    slot = None
    if table is None:
        slot, table = _tables.get(decode_ragged_table_bytes(s, n, n_splits))
    if table.device.type != "cpu":
        raise ValueError("table: host memory expected")
    lib = _lib.load()
    check("hyq_decode_attn_ragged", lib.hyq_decode_attn_ragged(_cache_ptrs(caches), n, _ptr(q), _ptr(out), n_splits,
                                                               _ptr(table), table.numel(), _ptr(ws), ws.numel(),
                                                               _stream()))
    if slot is not None:
        _tables.used(slot)
    return out


def select_vlines(shape: Shape, k: int, cache: HybridKVCache | None = None, dense_k: torch.Tensor | None = None,
                  proxy: torch.Tensor | None = None, apply: bool = False, scores: bool = False):
    """Vertical-line selector (hyq_select_vlines); returns idx [B][Hkv][k] (and scores)."""
    lib = _lib.load()
    dev = dense_k.device if dense_k is not None else cache.device
    if dense_k is not None:
        L = dense_k.shape[2]
        _bf16(dense_k, (shape.batch, shape.n_kv_heads, L, D), "dense_k")
        n_proxy = proxy.shape[2]
        _bf16(proxy, (shape.batch, shape.n_q_heads, n_proxy, D), "proxy")
    else:
        L, n_proxy = cache.len, cache.n_proxy
    P = max(0, L - WINDOW)
    idx = torch.empty((shape.batch, shape.n_kv_heads, max(k, 1)), dtype=torch.int32, device=dev)
    sc = torch.empty((shape.batch, shape.n_kv_heads, max(P, 1)), dtype=torch.float32, device=dev) if scores else None
    s = shape.c()
    need = int(lib.hyq_workspace_bytes(C.byref(s), _lib.HYQ_OP_SELECT, L, 0))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    check("hyq_select_vlines", lib.hyq_select_vlines(
        C.byref(s), C.byref(cache.c) if cache is not None else None, _ptr(dense_k), L,
        _ptr(proxy), n_proxy, k, int(apply), _ptr(idx), _ptr(sc), _ptr(ws), ws.numel(), _stream()))
    idx = idx[..., :k]
    return (idx, sc) if scores else idx


def select_tail_workspace(shape: Shape, L: int, device=None) -> torch.Tensor:
    """A workspace for hyq_select_vlines_tail at context length L (uint8, on ``device``)."""
    lib = _lib.load()
    s = shape.c()
    need = int(lib.hyq_workspace_bytes(C.byref(s), _lib.HYQ_OP_SELECT_TAIL, L, 0))
    if need == 0:
        raise ValueError(f"select_vlines_tail: unsupported shape or length L={L}")
    return torch.empty(need, dtype=torch.uint8, device=device or "cuda")


def select_vlines_tail(shape: Shape, k: int, dense_k: torch.Tensor, q: torch.Tensor, scores: bool = False,
                       ws: torch.Tensor | None = None):
    """Alg. 1-literal selector (hyq_select_vlines_tail): tail-query mean, raw logits, one set
    per Q head; returns idx [B][Hq][k] (and the logits [B][Hq][P])."""
    lib = _lib.load()
    L = dense_k.shape[2]
    _bf16(dense_k, (shape.batch, shape.n_kv_heads, L, D), "dense_k")
    n_q = q.shape[2]
    _bf16(q, (shape.batch, shape.n_q_heads, n_q, D), "q")
    P = max(0, L - WINDOW)
    dev = dense_k.device
    idx = torch.empty((shape.batch, shape.n_q_heads, max(k, 1)), dtype=torch.int32, device=dev)
    sc = torch.empty((shape.batch, shape.n_q_heads, max(P, 1)), dtype=torch.float32, device=dev) if scores else None
    s = shape.c()
    if ws is None:
        ws = select_tail_workspace(shape, L, dev)
    check("hyq_select_vlines_tail", lib.hyq_select_vlines_tail(
        C.byref(s), _ptr(dense_k), L, _ptr(q), n_q, k, _ptr(idx), _ptr(sc), _ptr(ws), ws.numel(), _stream()))
    idx = idx[..., :k]
    return (idx, sc) if scores else idx


def prefill_workspace(shape: Shape, N: int, device=None) -> torch.Tensor:
    """A workspace for hyq_prefill_attn at sequence length N (uint8, on ``device``)."""
    lib = _lib.load()
    s = shape.c()
    need = int(lib.hyq_workspace_bytes(C.byref(s), _lib.HYQ_OP_PREFILL, N, 0))
    if need == 0:
        raise ValueError(f"prefill: unsupported shape or length N={N}")
    return torch.empty(need, dtype=torch.uint8, device=device or "cuda")


def prefill_attn(shape: Shape, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 anchors: torch.Tensor | None = None, out: torch.Tensor | None = None,
                 ws: torch.Tensor | None = None, bulk: str = "int8") -> torch.Tensor:
    """Hybrid prefill attention for one sequence; fp32 out [Hq][N][128].  ``bulk`` picks the
    bulk Q.K format: "int8" (hyq_prefill_attn) or "mxfp4" (hyq_prefill_attn_mx).
    ``ws`` (from ``prefill_workspace``) receives the quantized operands."""
    if bulk not in ("int8", "mxfp4"):
        raise ValueError(f"bulk: 'int8' or 'mxfp4', not {bulk!r}")
    lib = _lib.load()
    N = q.shape[1]
    _bf16(q, (shape.n_q_heads, N, D), "q")
    _bf16(k, (shape.n_kv_heads, N, D), "k")
    _bf16(v, (shape.n_kv_heads, N, D), "v")
    n_anchor = 0
    if anchors is not None:
        if anchors.dtype != torch.int32 or not anchors.is_contiguous() or anchors.dim() != 2 \
                or anchors.shape[0] != shape.n_kv_heads or anchors.device != q.device:
            raise ValueError("anchors: contiguous int32 [Hkv][n_anchor] on the queries' device")
        n_anchor = anchors.shape[1]
    if out is None:
        out = torch.empty((shape.n_q_heads, N, D), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (shape.n_q_heads, N, D) or not out.is_contiguous():
        raise ValueError("out: contiguous float32 [Hq][N][128]")
    if ws is None:
        ws = prefill_workspace(shape, N, q.device)
    s = shape.c()
    name = "hyq_prefill_attn" if bulk == "int8" else "hyq_prefill_attn_mx"
    check(name, getattr(lib, name)(C.byref(s), _ptr(q), _ptr(k), _ptr(v), N,
                                   _ptr(anchors if n_anchor else None), n_anchor, _ptr(out),
                                   _ptr(ws), ws.numel(), _stream()))
    return out
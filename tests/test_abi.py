"""Host-only checks of the C ABI: the library loads, exports every symbol include/hyq.h
declares, sizes its buffers by the documented closed form, and rejects bad arguments before
enqueuing anything (no GPU needed: every call here fails validation on the host)."""
import ctypes as C
import os
import re

import pytest

from hybrid_precision_kv_amd import _lib
from hybrid_precision_kv_amd._lib import HyqCache, HyqShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from hybrid_precision_kv_amd import build
        build.build_library()
    return _lib.load()


def _shape(**kw):
    d = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, group=32, window=128, proxy_cap=64,
             staging_cap=64, int4_cap=1024, anchor_cap=64)
    d.update(kw)
    return HyqShape(**d)


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "hyq.h")).read()
    declared = sorted(set(re.findall(r"\b(hyq_[a-z_]+)\s*\(", hdr)))
    assert declared == sorted(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_buffer_sizes_closed_form(lib):
    s = _shape()
    out = (C.c_size_t * _lib.HYQ_NBUF)()
    assert lib.hyq_cache_buffer_bytes(C.byref(s), C.byref(out)) == 0
    H = 4
    b = dict(zip(_lib.BUFFERS, list(out)))
    # 160 bytes per INT4 position: 64 + 64 code bytes, 16 + 16 bytes of fp16 (scale, min) x 4 groups
    assert b["int4"] == H * 1024 * 160
    assert b["a_k"] + b["a_v"] == H * 64 * 512 and b["w_k"] + b["w_v"] == H * 128 * 512
    assert b["s_k"] == H * 64 * 256 and b["slot_pos"] == H * 1024 * 4
    assert b["proxy_q"] == 2 * 8 * 64 * 256  # 64 x H_Q x d x 2 bytes per sequence


@pytest.mark.parametrize("kw,status", [(dict(head_dim=64), 2), (dict(group=16), 2), (dict(window=64), 2),
                                       (dict(n_q_heads=24, n_kv_heads=2), 2), (dict(n_q_heads=7), 1),
                                       (dict(int4_cap=1000), 1), (dict(staging_cap=0), 1), (dict(batch=0), 1)])
def test_shape_validation(lib, kw, status):
    s = _shape(**kw)
    out = (C.c_size_t * _lib.HYQ_NBUF)()
    assert lib.hyq_cache_buffer_bytes(C.byref(s), C.byref(out)) == status


def _fake_cache(**counters):
    c = HyqCache()
    c.shape = _shape()
    for i, n in enumerate(_lib.BUFFERS):  # never dereferenced: validation fails first
        setattr(c, n, 0x1000 * (i + 1))
    c.len, c.n_int4, c.n_anchor, c.n_staged, c.n_proxy, c.proxy_head = 1000, 872 - 43, 43, 0, 0, 0
    for k, v in counters.items():
        setattr(c, k, v)
    return c


def test_error_paths_enqueue_nothing(lib):
    c = _fake_cache()
    before = bytes(c)
    # null cache / null tensors
    assert lib.hyq_decode_attn(None, 1, 1, 0, 1, 1 << 20, None) == 1
    assert lib.hyq_decode_attn(C.byref(c), None, 1, 0, 1, 1 << 20, None) == 1
    # workspace too small
    assert lib.hyq_decode_attn(C.byref(c), 0x10, 0x20, 4, 0x30, 16, None) == 4
    assert lib.hyq_decode_attn(C.byref(c), 0x10, 0x20, 4, None, 1 << 30, None) == 4
    # inconsistent counters
    bad = _fake_cache(n_int4=5)
    assert lib.hyq_decode_attn(C.byref(bad), 0x10, 0x20, 4, 0x30, 1 << 30, None) == 1
    # staging full
    full = _fake_cache(len=1000 + 64, n_staged=64)
    assert lib.hyq_append_token(C.byref(full), 0x10, 0x20, None, None) == 3
    # too many anchors for the candidates / capacity
    assert lib.hyq_quantize_kv(C.byref(c), 0x10, 0x20, 200, 0x30, 73, None, 0, None) == 3
    assert lib.hyq_quantize_kv(C.byref(c), 0x10, 0x20, 2000, 0x30, 65, None, 0, None) == 3
    assert lib.hyq_quantize_kv(C.byref(c), 0x10, 0x20, 2000, None, 5, None, 0, None) == 1
    assert bytes(c) == before  # host struct unchanged on error
    assert lib.hyq_status_string(4) == b"workspace missing or too small"


def test_workspace_sizes(lib):
    s = _shape()
    assert lib.hyq_workspace_bytes(C.byref(s), _lib.HYQ_OP_DECODE, 0, 8) == 2 * 8 * 8 * 130 * 4
    bad = _shape(head_dim=64)
    assert lib.hyq_workspace_bytes(C.byref(bad), _lib.HYQ_OP_DECODE, 0, 8) == 0


def test_prefill_workspace_layout_and_errors(lib):
    from tests.gpu_layout import prefill_ws_offsets
    one = _shape(batch=1, n_q_heads=32, n_kv_heads=8)
    for N in (1, 127, 128, 129, 1000, 8192, 32768):
        assert lib.hyq_workspace_bytes(C.byref(one), _lib.HYQ_OP_PREFILL, N, 0) == \
            prefill_ws_offsets(32, 8, N, one.anchor_cap)["total"]
    assert lib.hyq_workspace_bytes(C.byref(one), _lib.HYQ_OP_PREFILL, 0, 0) == 0
    assert lib.hyq_workspace_bytes(C.byref(one), _lib.HYQ_OP_PREFILL, (1 << 20) + 1, 0) == 0
    need = prefill_ws_offsets(32, 8, 1000, one.anchor_cap)["total"]
    f = lib.hyq_prefill_attn
    # batch != 1 -> UNSUPPORTED; null tensors / bad anchor counts -> INVALID; small ws -> WORKSPACE
    assert f(C.byref(_shape(batch=2)), 0x10, 0x20, 0x30, 1000, None, 0, 0x40, 0x50, need, None) == 2
    assert f(C.byref(one), None, 0x20, 0x30, 1000, None, 0, 0x40, 0x50, need, None) == 1
    assert f(C.byref(one), 0x10, 0x20, 0x30, 0, None, 0, 0x40, 0x50, need, None) == 1
    assert f(C.byref(one), 0x10, 0x20, 0x30, 1000, 0x60, 873, 0x40, 0x50, need, None) == 1
    assert f(C.byref(one), 0x10, 0x20, 0x30, 1000, None, 5, 0x40, 0x50, need, None) == 1
    assert f(C.byref(one), 0x10, 0x20, 0x30, 100, 0x60, 1, 0x40, 0x50, need, None) == 1
    assert f(C.byref(one), 0x10, 0x20, 0x30, 1000, None, 0, 0x40, 0x50, need - 1, None) == 4
    assert f(C.byref(one), 0x10, 0x20, 0x30, 1000, None, 0, 0x40, None, need, None) == 4
    assert f(C.byref(one), 0x10, 0x20, 0x30, (1 << 20) + 1, None, 0, 0x40, 0x50, need, None) == 2
    assert f(C.byref(one), 0x10, 0x20, 0x30, 1000, 0x60, one.anchor_cap + 1, 0x40, 0x50, need, None) == 3


def test_prefill_mx_shares_the_prefill_checks(lib):
    one = _shape(batch=1, n_q_heads=32, n_kv_heads=8)
    from tests.gpu_layout import prefill_ws_offsets
    need = prefill_ws_offsets(32, 8, 1000, one.anchor_cap)["total"]
    f = lib.hyq_prefill_attn_mx
    assert f(C.byref(_shape(batch=2)), 0x10, 0x20, 0x30, 1000, None, 0, 0x40, 0x50, need, None) == 2
    assert f(C.byref(one), None, 0x20, 0x30, 1000, None, 0, 0x40, 0x50, need, None) == 1
    assert f(C.byref(one), 0x10, 0x20, 0x30, 1000, 0x60, 873, 0x40, 0x50, need, None) == 1
    assert f(C.byref(one), 0x10, 0x20, 0x30, 1000, None, 0, 0x40, 0x50, need - 1, None) == 4
    assert f(C.byref(one), 0x10, 0x20, 0x30, 1000, 0x60, one.anchor_cap + 1, 0x40, 0x50, need, None) == 3


def test_select_tail_workspace_and_errors(lib):
    s = _shape(batch=2, n_q_heads=8, n_kv_heads=2)
    r256 = lambda x: (x + 255) // 256 * 256
    for L in (1, 128, 129, 1000, 32768):
        P = max(1, L - 128)
        assert lib.hyq_workspace_bytes(C.byref(s), _lib.HYQ_OP_SELECT_TAIL, L, 0) == \
            r256(2 * 8 * 128 * 4) + r256(2 * 8 * P * 4)
    assert lib.hyq_workspace_bytes(C.byref(s), _lib.HYQ_OP_SELECT_TAIL, 0, 0) == 0
    f = lib.hyq_select_vlines_tail
    need = lib.hyq_workspace_bytes(C.byref(s), _lib.HYQ_OP_SELECT_TAIL, 1000, 0)
    # null tensors, bad lengths, k outside [0, P], missing output -> INVALID; small ws -> WORKSPACE
    assert f(C.byref(s), None, 1000, 0x20, 64, 10, 0x30, None, 0x40, need, None) == 1
    assert f(C.byref(s), 0x10, 1000, None, 64, 10, 0x30, None, 0x40, need, None) == 1
    assert f(C.byref(s), 0x10, 0, 0x20, 64, 0, 0x30, None, 0x40, need, None) == 1
    assert f(C.byref(s), 0x10, 1000, 0x20, 0, 10, 0x30, None, 0x40, need, None) == 1
    assert f(C.byref(s), 0x10, 1000, 0x20, 64, 873, 0x30, None, 0x40, need, None) == 1
    assert f(C.byref(s), 0x10, 1000, 0x20, 64, -1, 0x30, None, 0x40, need, None) == 1
    assert f(C.byref(s), 0x10, 1000, 0x20, 64, 10, None, None, 0x40, need, None) == 1
    assert f(C.byref(s), 0x10, 1000, 0x20, 64, 10, 0x30, None, 0x40, need - 1, None) == 4
    assert f(C.byref(s), 0x10, 1000, 0x20, 64, 10, 0x30, None, None, need, None) == 4
    assert f(C.byref(_shape(head_dim=64)), 0x10, 1000, 0x20, 64, 10, 0x30, None, 0x40, need, None) == 2
    # no candidates: k = 0 is accepted and nothing is launched; k = 1 is rejected
    assert f(C.byref(s), 0x10, 128, 0x20, 64, 0, None, None, None, 0, None) == 0
    assert f(C.byref(s), 0x10, 128, 0x20, 64, 1, 0x30, None, 0x40, need, None) == 1


def test_bit_width_field(lib):
    out4 = (C.c_size_t * _lib.HYQ_NBUF)()
    out8 = (C.c_size_t * _lib.HYQ_NBUF)()
    assert lib.hyq_cache_buffer_bytes(C.byref(_shape()), C.byref(out4)) == 0
    assert lib.hyq_cache_buffer_bytes(C.byref(_shape(bits=4)), C.byref(out8)) == 0
    assert list(out4) == list(out8)  # 0 means 4
    assert lib.hyq_cache_buffer_bytes(C.byref(_shape(bits=8)), C.byref(out8)) == 0
    b4, b8 = dict(zip(_lib.BUFFERS, list(out4))), dict(zip(_lib.BUFFERS, list(out8)))
    assert b8["int4"] == 4 * 1024 * 288  # 9216-byte record per 32-slot tile
    assert {k: v for k, v in b8.items() if k != "int4"} == {k: v for k, v in b4.items() if k != "int4"}
    # B_K / B_V pairs: record of 512 (B_K + B_V) + 1024 bytes per 32-slot tile
    for bk, bv, rec in ((4, 2, 4096), (2, 2, 3072), (2, 0, 3072), (8, 0, 9216), (4, 4, 5120), (0, 2, 4096)):
        assert lib.hyq_cache_buffer_bytes(C.byref(_shape(bits=bk, bits_v=bv)), C.byref(out8)) == 0
        assert dict(zip(_lib.BUFFERS, list(out8)))["int4"] == 2 * 2 * 1024 * rec // 32
    for bk, bv in ((3, 0), (16, 0), (-4, 0), (2, 4), (8, 4), (4, 8), (8, 2), (2, 8), (4, 3), (4, -2)):
        assert lib.hyq_cache_buffer_bytes(C.byref(_shape(bits=bk, bits_v=bv)), C.byref(out8)) == 2


def test_ragged_decode_host_checks(lib):
    """hyq_decode_attn_ragged: workspace and table closed forms and every rejection before any
    device work."""
    one = _shape(batch=1)
    r256 = lambda x: -(-x // 256) * 256
    n, S, Hq = 3, 5, one.n_q_heads
    assert lib.hyq_decode_ragged_workspace_bytes(C.byref(one), n, S) == r256(n * 112) + r256(n * S * 4) + \
        n * S * Hq * 130 * 4
    assert lib.hyq_decode_ragged_table_bytes(C.byref(one), n, S) == r256(n * 112) + r256(n * S * 4)
    assert lib.hyq_decode_ragged_workspace_bytes(C.byref(one), 0, S) == 0
    assert lib.hyq_decode_ragged_workspace_bytes(C.byref(one), 1025, S) == 0
    assert lib.hyq_decode_ragged_table_bytes(C.byref(one), 1025, S) == 0
    assert lib.hyq_decode_ragged_workspace_bytes(C.byref(one), n, 0) > 0  # automatic plan: a bound
    caches = [_fake_cache(), _fake_cache(len=300, n_int4=160, n_anchor=12), _fake_cache(len=128, n_int4=0,
                                                                                          n_anchor=0)]
    for c in caches:
        c.shape = one
    arr = lambda cs: (C.POINTER(HyqCache) * len(cs))(*[C.pointer(c) for c in cs])
    big = 1 << 40
    tab = (C.c_uint8 * (1 << 20))()
    tb = C.cast(tab, C.c_void_p)
    T = len(tab)
    assert lib.hyq_decode_attn_ragged(None, 3, 0x10, 0x20, 0, tb, T, 0x30, big, None) == 1
    assert lib.hyq_decode_attn_ragged(arr(caches), 0, 0x10, 0x20, 0, tb, T, 0x30, big, None) == 1
    assert lib.hyq_decode_attn_ragged(arr(caches), 3, None, 0x20, 0, tb, T, 0x30, big, None) == 1
    assert lib.hyq_decode_attn_ragged(arr(caches), 3, 0x10, 0x20, -1, tb, T, 0x30, big, None) == 1
    assert lib.hyq_decode_attn_ragged(arr(caches * 342), 1026, 0x10, 0x20, 0, tb, T, 0x30, big, None) == 3
    nulls = (C.POINTER(HyqCache) * 2)(C.pointer(caches[0]))
    assert lib.hyq_decode_attn_ragged(nulls, 2, 0x10, 0x20, 0, tb, T, 0x30, big, None) == 1
    two = _fake_cache()  # batch 2: not a single-sequence cache
    assert lib.hyq_decode_attn_ragged(arr([caches[0], two]), 2, 0x10, 0x20, 0, tb, T, 0x30, big, None) == 1
    other = _fake_cache()
    other.shape = _shape(batch=1, n_q_heads=16)
    assert lib.hyq_decode_attn_ragged(arr([caches[0], other]), 2, 0x10, 0x20, 0, tb, T, 0x30, big, None) == 1
    wide = _fake_cache()
    wide.shape = _shape(batch=1, bits=8)
    assert lib.hyq_decode_attn_ragged(arr([caches[0], wide]), 2, 0x10, 0x20, 0, tb, T, 0x30, big, None) == 1
    bad = _fake_cache(n_int4=5)
    bad.shape = one
    assert lib.hyq_decode_attn_ragged(arr([caches[0], bad]), 2, 0x10, 0x20, 0, tb, T, 0x30, big, None) == 1
    need = lib.hyq_decode_ragged_workspace_bytes(C.byref(one), 3, S)
    tneed = lib.hyq_decode_ragged_table_bytes(C.byref(one), 3, S)
    assert lib.hyq_decode_attn_ragged(arr(caches), 3, 0x10, 0x20, S, tb, T, 0x30, need - 1, None) == 4
    assert lib.hyq_decode_attn_ragged(arr(caches), 3, 0x10, 0x20, S, tb, T, None, need, None) == 4
    assert lib.hyq_decode_attn_ragged(arr(caches), 3, 0x10, 0x20, S, tb, tneed - 1, 0x30, need, None) == 4
    assert lib.hyq_decode_attn_ragged(arr(caches), 3, 0x10, 0x20, S, None, tneed, 0x30, need, None) == 4
    # more than 16384 splits in all
    assert lib.hyq_decode_attn_ragged(arr(caches * 2), 6, 0x10, 0x20, 4096, tb, T, 0x30, big, None) == 1
    assert [c.len for c in caches] == [1000, 300, 128]  # caches are read only


def test_ragged_plan_writes_the_documented_table(lib):
    """hyq_decode_ragged_plan (host only): one 112-byte descriptor per sequence (slab pointers,
    capacities, counters, split count, first record), then the split map (sequence << 16 |
    split), at a fixed split count and for the automatic plan (every sequence gets at least one
    split, the total is the one reported)."""
    import struct
    one = _shape(batch=1)
    caches = [_fake_cache(), _fake_cache(len=300, n_int4=160, n_anchor=12), _fake_cache(len=128, n_int4=0,
                                                                                          n_anchor=0)]
    for c in caches:
        c.shape = one
    arr = (C.POINTER(HyqCache) * 3)(*[C.pointer(c) for c in caches])
    r256 = lambda x: -(-x // 256) * 256
    for S in (5, 0):
        nb = lib.hyq_decode_ragged_table_bytes(C.byref(one), 3, S)
        tab = (C.c_uint8 * nb)()
        total = C.c_int32(-1)
        assert lib.hyq_decode_ragged_plan(arr, 3, S, C.cast(tab, C.c_void_p), nb, C.byref(total)) == 0
        raw = bytes(tab)
        splits, rec0 = [], 0
        for i, c in enumerate(caches):
            d = struct.unpack_from("<7Q13i", raw, 112 * i)
            assert list(d[:7]) == [c.int4, c.a_k, c.a_v, c.s_k, c.s_v, c.w_k, c.w_v]
            assert list(d[7:14]) == [one.int4_cap, one.anchor_cap, one.staging_cap, c.n_int4, c.n_anchor,
                                     c.n_staged, min(c.len, 128)]
            assert d[15] == rec0 and d[14] >= 1 and (S == 0 or d[14] == S)
            splits.append(d[14])
            rec0 += one.n_q_heads * d[14]
        assert total.value == sum(splits)
        m = struct.unpack_from(f"<{total.value}I", raw, r256(3 * 112))
        assert list(m) == [(i << 16) | j for i in range(3) for j in range(splits[i])]
        if S == 0:  # the longest sequence (most tiles) gets the most splits
            assert splits[0] >= splits[1] >= splits[2]
    assert lib.hyq_decode_ragged_plan(arr, 3, 5, None, 1 << 20, None) == 4
    assert [c.len for c in caches] == [1000, 300, 128]  # caches are read only


def test_noalloc_decode_host_checks(lib):
    """hyq_decode_attn_noalloc rejects a call whose split records exceed the static scratch
    (batch * Hq * splits * 130 * 4 > HYQ_NOALLOC_SCRATCH_BYTES) before any device work, and
    validates like hyq_decode_attn."""
    c = _fake_cache()
    before = bytes(c)
    per_split = c.shape.batch * c.shape.n_q_heads * 130 * 4
    too_many = _lib.HYQ_NOALLOC_SCRATCH_BYTES // per_split + 1
    assert too_many <= 4096
    assert lib.hyq_decode_attn_noalloc(C.byref(c), 0x10, 0x20, too_many, None) == 4
    assert lib.hyq_decode_attn_noalloc(None, 0x10, 0x20, 0, None) == 1
    assert lib.hyq_decode_attn_noalloc(C.byref(c), None, 0x20, 0, None) == 1
    assert lib.hyq_decode_attn_noalloc(C.byref(c), 0x10, 0x20, -1, None) == 1
    assert lib.hyq_decode_attn_noalloc(C.byref(c), 0x10, 0x20, 4097, None) == 1
    bad = _fake_cache(n_int4=5)
    assert lib.hyq_decode_attn_noalloc(C.byref(bad), 0x10, 0x20, 0, None) == 1
    assert bytes(c) == before

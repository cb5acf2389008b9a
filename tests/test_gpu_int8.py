"""GPU parity of the 8-bit quantized bulk (shape.bits = 8: the bit width B_K = B_V of the
HyQuant paper's Alg. 3 and Alg. 4 raised from 4 to 8, 255 levels of the same group quantizer)
against the oracle's cache model with bits = 8, through the C ABI.

Same bar as the INT4 cache: codes, fp16 scale/min, anchor sets and every bf16 store
bit-exact after Freeze, appends and refreshes; decode within 2e-3 max-abs and 1e-3 relative
L2 of the oracle's fp64 decode over the same stored cache; selector sets equal to the
oracle's except near-ties."""
import numpy as np
import pytest

from hybrid_precision_kv_amd import api as hq
from oracle import policy as pol
from tests.test_gpu_decode import Pair
from tests.test_gpu_select import _cache_select_and_refresh, check_set

pytestmark = pytest.mark.gpu


def test_int8_freeze_codes_and_decode():
    p = Pair(8001, 1, 1, 4, 1024, n_steps=1, bits=8)
    p.codes_check()
    assert max(int(r.kc[:1024].max()) for r in p.refs) > 15  # really 8-bit codes
    q = p.append()
    p.codes_check()
    for s in (0, 1, 2, 5):
        p.decode_check(q, n_splits=s)


def test_int8_ragged_multi_tile_gqa_and_splits():
    p = Pair(8077, 2, 2, 4, 3001, n_steps=3, bits=8)
    p.codes_check()
    for _ in range(3):
        q = p.append()
    for s in (1, 3, 7, 0):
        p.decode_check(q, n_splits=s)
    for G in (1, 8):
        p2 = Pair(8100 + G, 1, 2, G, 700, n_steps=1, bits=8)
        p2.decode_check(p2.append())


@pytest.mark.parametrize("L", [1, 127, 129, 161])
def test_int8_edge_lengths(L):
    p = Pair(8200 + L, 1, 2, 4, L, n_steps=2, bits=8)
    p.codes_check()
    q = p.append()
    p.decode_check(q)
    q = p.append()
    p.codes_check()
    p.decode_check(q, n_splits=3)


def test_int8_select_and_refresh_bit_exact():
    """Cache-mode selector over INT8 keys, then refresh: demoted rows quantized to 8 bits,
    promoted slots dequantized from 8 bits, slots moved down -- every stored byte as the
    oracle's."""
    p = Pair(8300, 1, 2, 4, 1000, n_steps=70, bits=8)
    for _ in range(64):  # the staging buffer holds 64 tokens between refreshes
        q = p.append()
    _cache_select_and_refresh(p)
    p.decode_check(q)
    for _ in range(6):
        q = p.append()
    p.decode_check(q)
    # shrink the set (anchors demoted to 8-bit codes), then grow it back to the capacity's 5%
    _cache_select_and_refresh(p, pct=1)
    p.decode_check(q)
    _cache_select_and_refresh(p, pct=5)
    p.decode_check(q)


def test_int8_refresh_every_64_steps():
    p = Pair(8400, 1, 4, 4, 1024, n_steps=128, bits=8)
    flips = 0
    for t in range(128):
        q = p.append()
        if t % 64 == 63:
            k = pol.k_rule(p.cache.len)
            idx = hq.select_vlines(p.cache.shape, k, cache=p.cache).cpu().numpy()
            for h in range(p.Hkv):
                A, S = p.refs[h].select()
                flips += check_set(idx[0, h], S, k, f"int8 step {t} h{h}")
            hq.select_vlines(p.cache.shape, k, cache=p.cache, apply=True)
            for h in range(p.Hkv):
                p.refs[h].refresh(idx[0, h])
        if t % 32 == 31:
            p.decode_check(q)
    p.codes_check()
    print(f"int8: near-tie flips over 2 refreshes: {flips}")


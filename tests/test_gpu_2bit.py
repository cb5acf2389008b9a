"""GPU parity of the 2-bit quantized bulks K4V2 (shape.bits = 4, bits_v = 2) and K2V2 (bits = 2):
B_K and B_V of the HyQuant paper's Alg. 3 and Alg. 4 set separately, 3 levels of the group
quantizer for the 2-bit operand, against the oracle's cache model with the same widths,
through the C ABI.

Same bar as the INT4 cache: codes, fp16 scale/min, anchor sets and every bf16 store
bit-exact after Freeze, appends and refreshes; decode within 2e-3 max-abs and 1e-3 relative
L2 of the oracle's fp64 decode over the same stored cache; selector sets equal to the
oracle's except near-ties."""
import numpy as np
import pytest
import torch

from hybrid_precision_kv_amd import api as hq
from oracle import policy as pol
from tests.test_gpu_decode import Pair, dev
from tests.test_gpu_ragged import ragged_check, same_as_alone
from tests.test_gpu_select import _cache_select_and_refresh, check_set

pytestmark = pytest.mark.gpu

WIDTHS = [(4, 2), (2, 2)]


@pytest.mark.parametrize("bk,bv", WIDTHS)
def test_2bit_freeze_codes_and_decode(bk, bv):
    p = Pair(8501 + bk, 1, 1, 4, 1024, n_steps=1, bits=bk, bits_v=bv)
    p.codes_check()
    assert max(int(r.vc[:1024].max()) for r in p.refs) == 3
    q = p.append()
    p.codes_check()
    for s in (0, 1, 2, 5):
        p.decode_check(q, n_splits=s)


@pytest.mark.parametrize("bk,bv", WIDTHS)
def test_2bit_ragged_multi_tile_gqa_and_splits(bk, bv):
    p = Pair(8577 + bk, 2, 2, 4, 3001, n_steps=3, bits=bk, bits_v=bv)
    p.codes_check()
    for _ in range(3):
        q = p.append()
    for s in (1, 3, 7, 0):
        p.decode_check(q, n_splits=s)
    for G in (1, 8, 16):
        p2 = Pair(8600 + G + bk, 1, 2, G, 700, n_steps=1, bits=bk, bits_v=bv)
        p2.decode_check(p2.append())


@pytest.mark.parametrize("bk,bv", WIDTHS)
@pytest.mark.parametrize("L", [1, 127, 129, 161])
def test_2bit_edge_lengths(bk, bv, L):
    p = Pair(8700 + L + bk, 1, 2, 4, L, n_steps=2, bits=bk, bits_v=bv)
    p.codes_check()
    q = p.append()
    p.decode_check(q)
    q = p.append()
    p.codes_check()
    p.decode_check(q, n_splits=3)


@pytest.mark.parametrize("bk,bv", WIDTHS)
def test_2bit_select_and_refresh_bit_exact(bk, bv):
    """Cache-mode selector over 2-bit or INT4 keys, then refresh: demoted rows quantized to the
    shape's widths, promoted slots dequantized, slots moved down -- every stored byte as the
    oracle's."""
    p = Pair(8800 + bk, 1, 2, 4, 1000, n_steps=70, bits=bk, bits_v=bv)
    for _ in range(64):  # the staging buffer holds 64 tokens between refreshes
        q = p.append()
    _cache_select_and_refresh(p)
    p.decode_check(q)
    for _ in range(6):
        q = p.append()
    p.decode_check(q)
    _cache_select_and_refresh(p, pct=1)
    p.decode_check(q)
    _cache_select_and_refresh(p, pct=5)
    p.decode_check(q)


@pytest.mark.parametrize("bk,bv", WIDTHS)
def test_2bit_refresh_every_64_steps(bk, bv):
    p = Pair(8900 + bk, 1, 4, 4, 1024, n_steps=128, bits=bk, bits_v=bv)
    flips = 0
    for t in range(128):
        q = p.append()
        if t % 64 == 63:
            k = pol.k_rule(p.cache.len)
            idx = hq.select_vlines(p.cache.shape, k, cache=p.cache).cpu().numpy()
            for h in range(p.Hkv):
                A, S = p.refs[h].select()
                flips += check_set(idx[0, h], S, k, f"K{bk}V{bv} step {t} h{h}")
            hq.select_vlines(p.cache.shape, k, cache=p.cache, apply=True)
            for h in range(p.Hkv):
                p.refs[h].refresh(idx[0, h])
        if t % 32 == 31:
            p.decode_check(q)
    p.codes_check()
    print(f"K{bk}V{bv}: near-tie flips over 2 refreshes: {flips}")


@pytest.mark.parametrize("bk,bv", WIDTHS)
def test_2bit_ragged_batch(bk, bv):
    pairs = [Pair(9500 + i + 10 * bk, 1, 2, 4, L, n_steps=1, bits=bk, bits_v=bv)
             for i, L in enumerate([2000, 129, 700, 1])]
    qs = [p.append() for p in pairs]
    ragged_check(pairs, qs)
    o = ragged_check(pairs, qs, n_splits=2)
    same_as_alone(pairs, qs, 2, o)

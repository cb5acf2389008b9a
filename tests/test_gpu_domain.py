"""GPU parity of decode and selection over the edges of their input domain, through the C ABI,
against the oracle (HyQuant paper Alg. 3 with a free split count S, Alg. 4's Quant_B(.; G)).

Domain: K and V below 65504 in magnitude (fp16 scale and min stay finite), q in bf16 with
|q| below 65504.  Cases:
  * V or K groups with ranges of 1e3 to 6e4 (fp16 scales far above 256) at every bulk width;
  * tiny V (scales near the fp16 subnormal range), V mixed over six decades in one head
    (the decode's per-column V weight scale moves in both directions inside a wave), tiny
    and large q;
  * constant groups (scale 0, every code 0) in K and V;
  * the large, mixed and tiny V, large K and constant-group cases at GQA 8 and 16 (two
    column blocks per wave);
  * split counts above 32 (33 to 256) and the automatic plan at 1 KV head x 32K, which takes
    the multi-pass merge; batch 1 x 32K at GQA 8 and 16 (eight waves per workgroup, two
    column blocks per wave);
  * the selector over 65,536 keys (rows longer than the top-k's LDS stage), dense and cache
    mode, with the refresh applied.

Bar: codes and fp16 scale/min bit-exact; decode within 2e-3 max-abs and 1e-3 relative L2,
the max-abs bar taken on o / max|v| when the values are far from unit scale (an fp32
result carries error in proportion to the values it averages); selector sets as in the
selector tests (near-ties reported)."""
import numpy as np
import pytest

from hybrid_precision_kv_amd import api as hq
from hybrid_precision_kv_amd import synth
from oracle import numerics as nm
from oracle import policy as pol
from tests.test_gpu_decode import Pair, dev
from tests.test_gpu_select import _cache_select_and_refresh, check_set

pytestmark = pytest.mark.gpu

WIDTHS = [(4, 4), (8, 8), (4, 2), (2, 2)]


def _rescale(d, names, per_token, seed):
    """Multiply each token row of the named arrays by its own factor from ``per_token(rng, n)``
    (seeded), clipped into the domain, rounded back to bf16."""
    rng = np.random.default_rng(seed)
    for name in names:
        x = nm.bf16_to_f32(d[name]).astype(np.float64)
        f = per_token(rng, x.shape[:-1])[..., None]
        d[name] = nm.f32_to_bf16(np.clip(x * f, -6.0e4, 6.0e4).astype(np.float32))


def large_v(d):
    _rescale(d, ("V", "new_v"), lambda r, n: 10.0 ** r.uniform(3, 4, n), 11)


def large_k(d):
    _rescale(d, ("K", "new_k"), lambda r, n: 10.0 ** r.uniform(3, 4, n), 12)
    _rescale(d, ("proxy", "new_q"), lambda r, n: np.full(n, 1e-3), 13)  # scores stay O(1-10)


def tiny_v(d):
    _rescale(d, ("V", "new_v"), lambda r, n: np.full(n, 1e-4), 14)


def mixed_v(d):
    _rescale(d, ("V", "new_v"), lambda r, n: 10.0 ** r.uniform(-3, 3.5, n), 15)


def tiny_q(d):
    _rescale(d, ("new_q",), lambda r, n: np.full(n, 1e-4), 16)


def large_q(d):
    _rescale(d, ("new_q",), lambda r, n: np.full(n, 300.0), 17)


def constant_groups(d):
    """A quarter of the tokens get one constant 32-channel group in K and in V (scale 0), and
    every 97th token is constant across all 128 channels."""
    rng = np.random.default_rng(18)
    for name in ("K", "V"):
        x = nm.bf16_to_f32(d[name]).copy()
        B, H, L, D = x.shape
        pick = rng.random((B, H, L)) < 0.25
        grp = rng.integers(0, 4, (B, H, L))
        for b, h, t in zip(*np.nonzero(pick)):
            g = grp[b, h, t]
            x[b, h, t, 32 * g:32 * g + 32] = x[b, h, t, 32 * g]
        x[:, :, ::97, :] = x[:, :, ::97, :1]
        d[name] = nm.f32_to_bf16(x)


@pytest.mark.parametrize("bk,bv", WIDTHS)
@pytest.mark.parametrize("transform", [large_v, large_k])
def test_large_ranges_every_width(transform, bk, bv):
    p = Pair(9100 + bk + 10 * bv, 1, 2, 4, 2500, n_steps=1, bits=bk, bits_v=bv, transform=transform)
    p.codes_check()
    q = p.append()
    for s in (0, 3):
        p.decode_check(q, n_splits=s, vnorm=True)


@pytest.mark.parametrize("transform", [tiny_v, mixed_v, tiny_q, large_q])
def test_scales_far_from_unit(transform):
    p = Pair(9200, 2, 2, 4, 3001, n_steps=2, transform=transform)
    p.codes_check()
    p.append()
    q = p.append()
    for s in (0, 1, 7):
        p.decode_check(q, n_splits=s, vnorm=True)


@pytest.mark.parametrize("bk,bv", WIDTHS)
def test_constant_groups(bk, bv):
    p = Pair(9300 + bk, 1, 2, 4, 1500, n_steps=1, bits=bk, bits_v=bv, transform=constant_groups)
    p.codes_check()
    q = p.append()
    p.codes_check()
    p.decode_check(q)


@pytest.mark.parametrize("G", [8, 16])
@pytest.mark.parametrize("transform,bk,bv", [(large_v, 4, 4), (large_v, 2, 2), (mixed_v, 4, 4), (tiny_v, 4, 4),
                                             (large_k, 4, 4), (constant_groups, 4, 2)])
def test_wide_gqa_domain_edges(G, transform, bk, bv):
    """GQA 8 and 16: one wave serves two 4-head column blocks, each with its own softmax state
    and V weight scale; the same domain edges as above over a ragged cache and two split counts."""
    p = Pair(9600 + G, 1, 2, G, 2500, n_steps=1, bits=bk, bits_v=bv, transform=transform)
    p.codes_check()
    q = p.append()
    for s in (0, 5):
        p.decode_check(q, n_splits=s, vnorm=True)


def test_split_counts_above_32():
    """33 to 64 splits (the 64-record one-latency merge), 65 to 256 (the multi-pass merge), and
    more workers than tiles (idle splits carry an empty state)."""
    p = Pair(9400, 1, 2, 4, 3001, n_steps=1)
    q = p.append()
    for s in (33, 48, 64, 65, 100, 256):
        p.decode_check(q, n_splits=s)


def test_auto_splits_one_kv_head_32k():
    """1 KV head x 32K: the automatic plan spreads one head over the chip (the merge then takes
    more than 64 records)."""
    p = Pair(9401, 1, 1, 4, 32768, n_steps=1)
    q = p.append()
    p.decode_check(q)


@pytest.mark.parametrize("G", [8, 16])
def test_auto_splits_batch1_wide_gqa_32k(G):
    """Batch 1 x 32K at GQA 8 and 16 over 2 KV heads: the automatic plan takes 128 and 64
    splits per KV head with eight waves per workgroup, each wave serving two column blocks."""
    p = Pair(9402 + G, 1, 2, G, 32768, n_steps=1)
    q = p.append()
    p.decode_check(q)


def test_selector_65536_keys_dense():
    L, G, pct = 65536, 4, 5
    print(f"[case] dense selector L={L} G={G}", flush=True)
    d = synth.gen_batch(9500, 1, 1, G, L, n_proxy=64)
    k = pol.k_rule(L, pct_num=pct)
    shape = hq.Shape.for_context(1, G, 1, L, pct)
    idx, sc = hq.select_vlines(shape, k, dense_k=dev(d["K"]), proxy=dev(d["proxy"]), scores=True)
    A, S = pol.select_dense(d["K"][0, 0], d["proxy"][0, :G], pct_num=pct)
    assert np.max(np.abs(sc.cpu().numpy()[0, 0, :L - 128] - S)) <= 1e-5 * S.max()
    check_set(idx.cpu().numpy()[0, 0], S, k, "dense L65536")


def test_selector_65536_keys_cache_mode_and_refresh():
    p = Pair(9501, 1, 1, 4, 65536, n_steps=8)
    for _ in range(8):
        p.append()
    _cache_select_and_refresh(p)

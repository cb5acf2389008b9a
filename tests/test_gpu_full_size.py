"""Decode parity at the batched workload's full size and launch configuration: batch 16 x
32768-token contexts, 32 Q / 8 KV heads, 5% anchors, automatic splits (the configuration the
benchmark times), for every built bulk width (K4V4, K8V8, K4V2, K2V2), against the oracle on
sampled (sequence, KV head) pairs.

The whole batch is drawn from the shared seeded generator.  Sampled heads take the oracle's
anchor sets (so both sides freeze the same positions); the other heads take the GPU dense
selector's, which only serve as inputs.  After Freeze and one appended token, each sampled
head's output must meet the decode bar (2e-3 max-abs, 1e-3 relative L2 against the oracle's
fp64 decode over the head's stored cache).  The maintenance step at the same size (64
appends, cache-mode selection, refresh) is checked on the same sampled heads: scores within
1e-5 of the largest, sets equal except near-ties, then decode after the refresh."""
import numpy as np
import pytest
import torch

from hybrid_precision_kv_amd import api as hq
from hybrid_precision_kv_amd import synth
from oracle import attention as att
from oracle import numerics as nm
from oracle import policy as pol
from tests.test_gpu_decode import MAX_ABS, REL_L2, Pair, dev
from tests.test_gpu_select import check_set

pytestmark = pytest.mark.gpu

B, HKV, G, L = 16, 8, 4, 32768
SAMPLE = [(0, 0), (7, 3), (15, 7)]


@pytest.fixture(scope="module")
def batch():
    print(f"[case] full size: generating B={B} Hkv={HKV} G={G} L={L}", flush=True)
    d = synth.gen_batch(12000, B, HKV, G, L, n_proxy=64, n_steps=64)
    print("[case] full size: generated", flush=True)
    k = pol.k_rule(L)
    shape = hq.Shape.for_context(B, HKV * G, HKV, L + 1)
    Kd, Pd = dev(d["K"]), dev(d["proxy"])
    anchors = hq.select_vlines(shape, k, dense_k=Kd, proxy=Pd).cpu().numpy()
    for b, h in SAMPLE:
        A, _ = pol.select_dense(d["K"][b, h], d["proxy"][b, h * G:(h + 1) * G])
        anchors[b, h] = A
    d["anchors"] = anchors
    d["Kd"], d["Vd"], d["Pd"] = Kd, dev(d["V"]), Pd
    return d


@pytest.mark.parametrize("bk,bv", [(4, 4), (8, 8), (4, 2), (2, 2)])
def test_full_size_decode_sampled(batch, bk, bv):
    d = batch
    print(f"[case] full size K{bk}V{bv}", flush=True)
    shape = hq.Shape.for_context(B, HKV * G, HKV, L + 1, bits=bk, bits_v=bv)
    cache = hq.HybridKVCache(shape)
    hq.quantize_kv(cache, d["Kd"], d["Vd"], torch.from_numpy(d["anchors"]).cuda(), d["Pd"])
    hq.append_token(cache, dev(d["new_k"][:, :, 0]), dev(d["new_v"][:, :, 0]), dev(d["new_q"][:, :, 0]))
    q = d["new_q"][:, :, 0]
    o = hq.decode_attn(cache, dev(q), 0).cpu().numpy()
    assert np.all(np.isfinite(o))
    for b, h in SAMPLE:
        r = pol.HybridCacheRef(g=G, bits=bk, bits_v=bv)
        r.freeze(d["K"][b, h], d["V"][b, h], d["anchors"][b, h], d["proxy"][b, h * G:(h + 1) * G])
        r.append(d["new_k"][b, h, 0], d["new_v"][b, h, 0], q[b, h * G:(h + 1) * G])
        Kh, Vh = r.stored_kv()
        ref = att.decode_ref(nm.bf16_to_f32(q[b, h * G:(h + 1) * G]), Kh, Vh)
        got = o[b, h * G:(h + 1) * G]
        err = np.abs(got - ref).max()
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert err <= MAX_ABS and rel <= REL_L2, f"K{bk}V{bv} b{b} h{h}: max-abs {err:.3g} rel-L2 {rel:.3g}"
    del cache
    torch.cuda.empty_cache()


def _check_decode(o, q, refs):
    for (b, h), r in refs.items():
        Kh, Vh = r.stored_kv()
        ref = att.decode_ref(nm.bf16_to_f32(q[b, h * G:(h + 1) * G]), Kh, Vh)
        got = o[b, h * G:(h + 1) * G]
        err = np.abs(got - ref).max()
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert err <= MAX_ABS and rel <= REL_L2, f"b{b} h{h}: max-abs {err:.3g} rel-L2 {rel:.3g}"


def test_full_size_select_and_refresh_sampled(batch):
    """bs16 x 32K, 32/8 heads, K4V4: 64 appends fill the staging buffers, then hyq_select_vlines
    over the cache at the 5% rule and apply (the maintenance step the benchmark times)."""
    d = batch
    print("[case] full size maintenance K4V4", flush=True)
    shape = hq.Shape.for_context(B, HKV * G, HKV, L + 64)
    cache = hq.HybridKVCache(shape)
    hq.quantize_kv(cache, d["Kd"], d["Vd"], torch.from_numpy(d["anchors"]).cuda(), d["Pd"])
    refs = {}
    for b, h in SAMPLE:
        r = pol.HybridCacheRef(g=G)
        r.freeze(d["K"][b, h], d["V"][b, h], d["anchors"][b, h], d["proxy"][b, h * G:(h + 1) * G])
        refs[(b, h)] = r
    for t in range(64):
        hq.append_token(cache, dev(d["new_k"][:, :, t]), dev(d["new_v"][:, :, t]), dev(d["new_q"][:, :, t]))
        for (b, h), r in refs.items():
            r.append(d["new_k"][b, h, t], d["new_v"][b, h, t], d["new_q"][b, h * G:(h + 1) * G, t])
    k = pol.k_rule(cache.len)
    idx, sc = hq.select_vlines(shape, k, cache=cache, scores=True)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    P = cache.len - 128
    flips = 0
    for (b, h), r in refs.items():
        A, S = r.select()
        assert np.max(np.abs(sc[b, h, :P] - S)) <= 1e-5 * S.max(), f"scores b{b} h{h}"
        flips += check_set(idx[b, h], S, k, f"full size b{b} h{h}")
    idx2 = hq.select_vlines(shape, k, cache=cache, apply=True).cpu().numpy()
    assert np.array_equal(idx2, idx)
    for (b, h), r in refs.items():
        r.refresh(idx[b, h])
    assert cache.n_anchor == k and cache.n_staged == 0 and cache.n_int4 == P - k
    q = d["new_q"][:, :, 63]
    _check_decode(hq.decode_attn(cache, dev(q), 0).cpu().numpy(), q, refs)
    print(f"[full size] maintenance: k={k}, near-tie flips {flips}", flush=True)
    del cache
    torch.cuda.empty_cache()


def test_full_size_batch1_decode_all_heads():
    """Batch 1 x 32768 at 32/8 heads with automatic splits (32 per KV head: the latency-bound
    plan the batch-1 benchmark rows time), every head against the oracle."""
    print("[case] full size batch 1", flush=True)
    d = synth.gen_batch(12100, 1, HKV, G, L, n_proxy=64, n_steps=1)
    shape = hq.Shape.for_context(1, HKV * G, HKV, L + 1)
    k = pol.k_rule(L)
    anchors = np.zeros((1, HKV, k), np.int32)
    refs = {}
    for h in range(HKV):
        A, _ = pol.select_dense(d["K"][0, h], d["proxy"][0, h * G:(h + 1) * G])
        anchors[0, h] = A
        r = pol.HybridCacheRef(g=G)
        r.freeze(d["K"][0, h], d["V"][0, h], A, d["proxy"][0, h * G:(h + 1) * G])
        r.append(d["new_k"][0, h, 0], d["new_v"][0, h, 0], d["new_q"][0, h * G:(h + 1) * G, 0])
        refs[(0, h)] = r
    cache = hq.HybridKVCache(shape)
    hq.quantize_kv(cache, dev(d["K"]), dev(d["V"]), torch.from_numpy(anchors).cuda(), dev(d["proxy"]))
    hq.append_token(cache, dev(d["new_k"][:, :, 0]), dev(d["new_v"][:, :, 0]), dev(d["new_q"][:, :, 0]))
    q = d["new_q"][:, :, 0]
    _check_decode(hq.decode_attn(cache, dev(q), 0).cpu().numpy(), q, refs)


def test_full_size_gqa8_decode_sampled():
    """The GQA-8 decode row's workload: 64 Q / 8 KV heads, batch 4 x 32768, 5% anchors,
    automatic splits (one wave per 8 Q heads of a KV head); sampled heads against the oracle."""
    Bs, Gs = 4, 8
    print(f"[case] full size decode B={Bs} G={Gs}", flush=True)
    d = synth.gen_batch(12300, Bs, HKV, Gs, L, n_proxy=64, n_steps=1)
    shape = hq.Shape.for_context(Bs, HKV * Gs, HKV, L + 1)
    k = pol.k_rule(L)
    Kd, Pd = dev(d["K"]), dev(d["proxy"])
    anchors = hq.select_vlines(shape, k, dense_k=Kd, proxy=Pd).cpu().numpy()
    refs = {}
    for b, h in [(0, 0), (2, 5), (3, 7)]:
        A, _ = pol.select_dense(d["K"][b, h], d["proxy"][b, h * Gs:(h + 1) * Gs])
        anchors[b, h] = A
        r = pol.HybridCacheRef(g=Gs)
        r.freeze(d["K"][b, h], d["V"][b, h], A, d["proxy"][b, h * Gs:(h + 1) * Gs])
        r.append(d["new_k"][b, h, 0], d["new_v"][b, h, 0], d["new_q"][b, h * Gs:(h + 1) * Gs, 0])
        refs[(b, h)] = r
    cache = hq.HybridKVCache(shape)
    hq.quantize_kv(cache, Kd, dev(d["V"]), torch.from_numpy(anchors).cuda(), Pd)
    hq.append_token(cache, dev(d["new_k"][:, :, 0]), dev(d["new_v"][:, :, 0]), dev(d["new_q"][:, :, 0]))
    q = d["new_q"][:, :, 0]
    o = hq.decode_attn(cache, dev(q), 0).cpu().numpy()
    assert np.all(np.isfinite(o))
    for (b, h), r in refs.items():
        Kh, Vh = r.stored_kv()
        ref = att.decode_ref(nm.bf16_to_f32(q[b, h * Gs:(h + 1) * Gs]), Kh, Vh)
        got = o[b, h * Gs:(h + 1) * Gs]
        err = np.abs(got - ref).max()
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert err <= MAX_ABS and rel <= REL_L2, f"G8 b{b} h{h}: max-abs {err:.3g} rel-L2 {rel:.3g}"
    del cache
    torch.cuda.empty_cache()


def test_full_size_selector_qwen32b_shape():
    """The selector row's workload: 64 Q / 8 KV heads (GQA 8), batch 4 x 32768, cache-mode
    selection at 1%, 5% and 10% of the context; sampled heads against the oracle (scores
    within 1e-5 of the largest, sets equal except near-ties)."""
    Bs, Gs = 4, 8
    print(f"[case] full size selector B={Bs} G={Gs}", flush=True)
    d = synth.gen_batch(12200, Bs, HKV, Gs, L, n_proxy=64)
    shape = hq.Shape.for_context(Bs, HKV * Gs, HKV, L, 10)
    k5 = pol.k_rule(L)
    anchors = hq.select_vlines(shape, k5, dense_k=dev(d["K"]), proxy=dev(d["proxy"])).cpu().numpy()
    sample = [(0, 0), (3, 7)]
    refs = {}
    for b, h in sample:
        A, _ = pol.select_dense(d["K"][b, h], d["proxy"][b, h * Gs:(h + 1) * Gs])
        anchors[b, h] = A
        r = pol.HybridCacheRef(g=Gs)
        r.freeze(d["K"][b, h], d["V"][b, h], A, d["proxy"][b, h * Gs:(h + 1) * Gs])
        refs[(b, h)] = r
    cache = hq.HybridKVCache(shape)
    hq.quantize_kv(cache, dev(d["K"]), dev(d["V"]), torch.from_numpy(anchors).cuda(), dev(d["proxy"]))
    P = L - 128
    flips = 0
    for pct in (1, 5, 10):
        k = pol.k_rule(L, pct_num=pct)
        idx, sc = hq.select_vlines(shape, k, cache=cache, scores=True)
        idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
        for (b, h), r in refs.items():
            _, S = r.select(pct_num=pct)
            assert np.max(np.abs(sc[b, h, :P] - S)) <= 1e-5 * S.max(), f"scores {pct}% b{b} h{h}"
            flips += check_set(idx[b, h], S, k, f"selector {pct}% b{b} h{h}")
    print(f"[full size] selector: near-tie flips {flips}", flush=True)


def test_full_size_all_bf16_batch1():
    """The all-bf16 comparison row at 32768 tokens (k = P: every candidate an anchor, nothing
    quantized), 32/8 heads, automatic splits, every head against the oracle."""
    p = Pair(12300, 1, HKV, G, L, n_steps=1, pct=100)
    assert p.cache.n_int4 == 0 and p.cache.n_anchor == L - 128
    p.decode_check(p.append())

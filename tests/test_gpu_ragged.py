"""GPU parity of decode over variable-length batches (hyq_decode_attn_ragged): each sequence is
its own single-sequence cache, frozen at its own length, appended to and refreshed on its own
cadence, and one call decodes them all (the HyQuant paper's Alg. 3 per sequence).

Bar: per sequence, the decode bar of the uniform batch (2e-3 max-abs and 1e-3 relative L2
against the oracle's fp64 decode over that sequence's stored cache), and with a fixed split
count, bit-identical outputs to hyq_decode_attn on the sequence's cache alone (same
per-(sequence, KV head) work partition, same arithmetic)."""
import numpy as np
import pytest
import torch

from hybrid_precision_kv_amd import api as hq
from oracle import attention as att
from oracle import numerics as nm
from oracle import policy as pol
from tests.test_gpu_decode import MAX_ABS, REL_L2, Pair, dev
from tests.test_gpu_select import check_set

pytestmark = pytest.mark.gpu


def ragged_check(pairs, qs, n_splits=0, oracle_idx=None):
    """Decode the pairs' caches as one ragged batch; compare sequences with the oracle (all, or
    those in oracle_idx).  Returns the fp32 outputs [n][Hq][128]."""
    q = torch.cat([dev(x) for x in qs], dim=0)
    o = hq.decode_attn_ragged([p.cache for p in pairs], q, n_splits).cpu().numpy()
    assert np.all(np.isfinite(o)), "non-finite output"
    for i, (p, qb) in enumerate(zip(pairs, qs)):
        if oracle_idx is not None and i not in oracle_idx:
            continue
        ref = np.empty_like(o[i])
        for h in range(p.Hkv):
            Kh, Vh = p.refs[h].stored_kv()
            ref[h * p.G:(h + 1) * p.G] = att.decode_ref(nm.bf16_to_f32(qb[0, h * p.G:(h + 1) * p.G]), Kh, Vh)
        err = np.abs(o[i] - ref).max()
        rel = np.linalg.norm(o[i] - ref) / np.linalg.norm(ref)
        assert err <= MAX_ABS and rel <= REL_L2, f"seq {i} (len {p.cache.len}): max-abs {err:.3g} rel-L2 {rel:.3g}"
    return o


def same_as_alone(pairs, qs, n_splits, o):
    for i, (p, qb) in enumerate(zip(pairs, qs)):
        alone = hq.decode_attn(p.cache, dev(qb), n_splits).cpu().numpy()
        assert np.array_equal(alone[0], o[i]), f"seq {i}: ragged and single-cache outputs differ"


@pytest.mark.parametrize("bits", [4, 8])
def test_ragged_lengths_against_oracle_and_single_cache(bits):
    lens = [1000, 3001, 129, 1, 700, 161]
    pairs = [Pair(9000 + i, 1, 2, 4, L, n_steps=2, bits=bits) for i, L in enumerate(lens)]
    qs = [p.append() for p in pairs]
    for s in (0, 1, 3):
        o = ragged_check(pairs, qs, n_splits=s)
        if s:
            same_as_alone(pairs, qs, s, o)


def test_ragged_single_sequence_and_gqa():
    for G in (1, 8, 16):
        p = Pair(9100 + G, 1, 2, G, 900, n_steps=1)
        q = p.append()
        ragged_check([p], [q])
    pairs = [Pair(9120 + i, 1, 1, 8, L, n_steps=1) for i, L in enumerate([2048, 64])]
    ragged_check(pairs, [p.append() for p in pairs], n_splits=2)


@pytest.mark.parametrize("G", [8, 16])
def test_ragged_wide_gqa_matches_single_cache(G):
    """GQA 8 and 16: the variable-length launch takes the uniform batch's two column blocks per
    wave; at a fixed split count every sequence is bit-identical to its single-cache decode."""
    pairs = [Pair(9140 + G + i, 1, 2, G, L, n_steps=1) for i, L in enumerate([3001, 700, 129])]
    qs = [p.append() for p in pairs]
    for s in (0, 3):
        o = ragged_check(pairs, qs, n_splits=s)
        if s:
            same_as_alone(pairs, qs, s, o)


def test_ragged_staggered_refresh():
    """Four sequences of different lengths, 96 steps; sequence i runs select-and-refresh when its
    own staging holds 64 tokens minus 16 i (every sequence on its own cadence), and the batch is
    decoded in one call every 8 steps."""
    lens = [1500, 400, 2600, 200]
    pairs = [Pair(9200 + i, 1, 2, 4, L, n_steps=96) for i, L in enumerate(lens)]
    flips, refreshes = 0, 0
    for t in range(96):
        qs = [p.append() for p in pairs]
        for i, p in enumerate(pairs):
            if p.cache.n_staged >= 64 - 16 * i:
                k = pol.k_rule(p.cache.len)
                idx = hq.select_vlines(p.cache.shape, k, cache=p.cache).cpu().numpy()
                for h in range(p.Hkv):
                    A, S = p.refs[h].select()
                    flips += check_set(idx[0, h], S, k, f"seq {i} step {t} h{h}")
                hq.select_vlines(p.cache.shape, k, cache=p.cache, apply=True)
                for h in range(p.Hkv):
                    p.refs[h].refresh(idx[0, h])
                refreshes += 1
        if t % 8 == 7:
            ragged_check(pairs, qs)
    for p in pairs:
        p.codes_check()
    assert refreshes >= 6
    print(f"staggered: {refreshes} refreshes, {flips} near-tie flips", flush=True)


def test_ragged_full_size_mix():
    """Sixteen sequences at the batched workload's heads (32 Q / 8 KV) with lengths from 1 to
    32768: every output bit-identical to the single-cache call at a fixed split count, five
    sequences (the longest among them) against the oracle, then the automatic plan against the
    oracle on the same five."""
    lens = [32768, 129, 1000, 4096, 16384, 2500, 700, 8192, 24000, 300, 12000, 6000, 1, 20000, 3000, 128]
    pairs = [Pair(9300 + i, 1, 8, 4, L, n_steps=1) for i, L in enumerate(lens)]
    qs = [p.append() for p in pairs]
    sample = {0, 3, 8, 12, 15}
    o = ragged_check(pairs, qs, n_splits=4, oracle_idx=sample)
    same_as_alone(pairs, qs, 4, o)
    ragged_check(pairs, qs, n_splits=0, oracle_idx=sample)


def test_ragged_deterministic_and_workspace_reuse():
    pairs = [Pair(9400 + i, 1, 2, 4, L, n_steps=1) for i, L in enumerate([3000, 500, 129])]
    qs = [p.append() for p in pairs]
    q = torch.cat([dev(x) for x in qs], dim=0)
    ws = torch.empty(hq.decode_ragged_workspace_bytes(pairs[0].cache.shape, 3), dtype=torch.uint8, device="cuda")
    a = hq.decode_attn_ragged([p.cache for p in pairs], q, ws=ws)
    # a different batch through the same workspace in between, then the first again
    hq.decode_attn_ragged([pairs[2].cache, pairs[0].cache], q[[2, 0]].contiguous(), ws=ws)
    b = hq.decode_attn_ragged([p.cache for p in pairs], q, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_ragged_graph_capture_and_replan():
    """The call recorded into a HIP graph with a caller-owned page-locked table: every replay
    (eager work and synchronisations in between) equals the eager call; after appends change
    the counters, hyq_decode_ragged_plan rewrites the table and the replays follow them."""
    pairs = [Pair(9500 + i, 1, 2, 4, L, n_steps=2) for i, L in enumerate([2000, 700, 129])]
    qs = [p.append() for p in pairs]
    q = torch.cat([dev(x) for x in qs], dim=0)
    caches = [p.cache for p in pairs]
    S = 3  # a fixed split count keeps the recorded grid valid when the counters change
    shape = caches[0].shape
    ws = torch.empty(hq.decode_ragged_workspace_bytes(shape, 3, S), dtype=torch.uint8, device="cuda")
    table = hq.decode_ragged_table(shape, 3, S)
    out = torch.empty((3, shape.n_q_heads, 128), dtype=torch.float32, device="cuda")
    eager = hq.decode_attn_ragged(caches, q, S, ws=torch.empty_like(ws)).clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        hq.decode_attn_ragged(caches, q, S, out=out, ws=ws, table=table)
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}"
        hq.decode_attn(caches[0], dev(qs[0]))  # eager work between replays
        torch.cuda.synchronize()
    qs2 = [p.append() for p in pairs]  # the counters move on
    q.copy_(torch.cat([dev(x) for x in qs2], dim=0))
    assert hq.decode_ragged_plan(caches, table, S) == 3 * S
    g.replay()
    torch.cuda.synchronize()
    eager2 = hq.decode_attn_ragged(caches, q, S, ws=torch.empty_like(ws))
    torch.cuda.synchronize()
    assert torch.equal(out, eager2)
    ragged_check(pairs, qs2, n_splits=S)

"""GPU parity of the Alg. 1-literal selector (hyq_select_vlines_tail: tail-query mean, raw
logits, one set per Q head; HyQuant paper appendix A.1, Alg. 1) against
``oracle.policy.select_tail_mean``.

Bar: logits within their fp32 bound of the oracle's fp64 values -- |dS_j| <= 1e-5 *
sum_c |k_jc| * mean_i |q_ic| (the tail sum over <= 128 rows in fp32 and an 8-term dot plus a
16-lane tree add about 140 roundings of 2^-24 to that product); index sets equal to the
oracle's top-k (ties to the lower position) except near-ties, where a position may differ only
if its oracle logit lies within twice that bound of the k-th largest; such flips are
reported."""
import numpy as np
import pytest
import torch

from hybrid_precision_kv_amd import _lib
from hybrid_precision_kv_amd import api as hq
from hybrid_precision_kv_amd import synth
from oracle import numerics as nm
from oracle import policy as pol
from tests.test_gpu_decode import dev

pytestmark = pytest.mark.gpu

REL = 1e-5


def logit_bound(K_bits, Q_bits, g):
    """Per (Q head, prefix key) bound on |fp32 logit - exact logit| (test-side arithmetic)."""
    K = np.abs(nm.bf16_to_f32(K_bits).astype(np.float64))
    Q = nm.bf16_to_f32(Q_bits).astype(np.float64)
    t = min(128, Q.shape[1])
    mabs = np.abs(Q[:, Q.shape[1] - t:]).mean(axis=1)  # [Hq][D]
    P = max(0, K.shape[1] - 128)
    return np.stack([K[h // g, :P] @ mabs[h] for h in range(Q.shape[0])]) * REL


def check_head(got, S, bound, k, label):
    got = np.asarray(got)
    assert len(got) == k
    assert np.all(np.diff(got) > 0), f"{label}: not ascending/distinct"
    ref = pol.topk_lower_index(S, k)
    diff = np.setxor1d(got, ref)
    if len(diff) == 0:
        return 0
    kth = np.sort(S)[::-1][k - 1]
    gap = np.abs(S[diff] - kth)
    assert np.all(gap <= 2 * (bound[diff] + bound.max())), f"{label}: {len(diff)} set differences"
    print(f"[{label}] {len(diff) // 2} near-tie flips", flush=True)
    return len(diff) // 2


def run_case(d, B, Hkv, G, L, k, label):
    print(f"[case] {label} B={B} Hkv={Hkv} G={G} L={L} n_q={d['proxy'].shape[2]} k={k}", flush=True)
    shape = hq.Shape.for_context(B, Hkv * G, Hkv, L)
    idx, sc = hq.select_vlines_tail(shape, k, dev(d["K"]), dev(d["proxy"]), scores=True)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    P = L - 128
    flips = 0
    for b in range(B):
        ref_idx, S = pol.select_tail_mean(d["K"][b], d["proxy"][b], k=k)
        bound = logit_bound(d["K"][b], d["proxy"][b], G)
        err = np.abs(sc[b, :, :P] - S)
        assert np.all(err <= bound), f"{label}: logit error {err.max():.3g} (bound {bound[err > bound].min():.3g})"
        for h in range(Hkv * G):
            flips += check_head(idx[b, h], S[h], bound[h], k, f"{label} b{b} h{h}")
    return flips


@pytest.mark.parametrize("B,Hkv,G,L,n_q,pct", [(1, 1, 4, 1024, 200, 5), (2, 2, 8, 3000, 128, 5),
                                               (1, 2, 1, 700, 50, 10), (1, 1, 16, 2100, 300, 1),
                                               (1, 2, 2, 130, 64, 5), (1, 1, 4, 129, 1, 5),
                                               (1, 4, 2, 1500, 129, 5)])
def test_tail_selector_parity(B, Hkv, G, L, n_q, pct):
    d = synth.gen_batch(7000 + L, B, Hkv, G, L, n_proxy=n_q)
    run_case(d, B, Hkv, G, L, pol.k_alg1(L - 128, pct), f"alg1 pct={pct}")


def test_tail_selector_k_edges_and_zero_logit_ties():
    """k = 1, k = P, k = 0; rows of zero keys (logits +0 / -0, all tied) and duplicated keys."""
    B, Hkv, G, L = 1, 2, 4, 600
    d = synth.gen_batch(7100, B, Hkv, G, L, n_proxy=128)
    zero = nm.f32_to_bf16(np.zeros(128, np.float32))[0]
    d["K"][0, 0, 10:200] = zero
    d["K"][0, 1, 300:310] = d["K"][0, 1, 5]
    P = L - 128
    for k in (1, P, 250):
        run_case(d, B, Hkv, G, L, k, f"k={k}")
    shape = hq.Shape.for_context(B, Hkv * G, Hkv, L)
    idx = hq.select_vlines_tail(shape, 0, dev(d["K"]), dev(d["proxy"]))
    assert idx.shape == (B, Hkv * G, 0)


def test_tail_selector_no_candidates_and_errors():
    d = synth.gen_batch(7200, 1, 1, 2, 128, n_proxy=16)
    shape = hq.Shape.for_context(1, 2, 1, 128)
    idx = hq.select_vlines_tail(shape, 0, dev(d["K"]), dev(d["proxy"]))
    assert idx.shape == (1, 2, 0)
    with pytest.raises(_lib.HyqError):
        hq.select_vlines_tail(shape, 1, dev(d["K"]), dev(d["proxy"]))  # k > P = 0


def test_tail_selector_deterministic():
    d = synth.gen_batch(7300, 2, 2, 4, 2000, n_proxy=128)
    shape = hq.Shape.for_context(2, 8, 2, 2000)
    a = hq.select_vlines_tail(shape, 100, dev(d["K"]), dev(d["proxy"]))
    b = hq.select_vlines_tail(shape, 100, dev(d["K"]), dev(d["proxy"]))
    assert torch.equal(a, b)


def test_tail_selector_full_size():
    """Prefill-boundary shape: 32 Q / 8 KV heads, 32768 keys, 32768 queries (only the last 128
    enter the mean), Alg. 1's 5% of the candidates per Q head."""
    L = 32768
    d = synth.gen_batch(7400, 1, 8, 4, L, n_proxy=128)
    rng = np.random.default_rng(7401)
    filler = nm.f32_to_bf16(rng.standard_normal((1, 32, L - 128, 128), dtype=np.float32) * np.float32(8.0))
    q_full = np.concatenate([filler, d["proxy"]], axis=2)
    shape = hq.Shape.for_context(1, 32, 8, L)
    k = pol.k_alg1(L - 128)
    idx, sc = hq.select_vlines_tail(shape, k, dev(d["K"]), dev(q_full), scores=True)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    ref_idx, S = pol.select_tail_mean(d["K"][0], d["proxy"][0], k=k)  # the tail alone: same mean
    bound = logit_bound(d["K"][0], d["proxy"][0], 4)
    assert np.all(np.abs(sc[0] - S) <= bound)
    flips = sum(check_head(idx[0, h], S[h], bound[h], k, f"full h{h}") for h in range(32))
    print(f"[full] k={k} near-tie flips {flips}")

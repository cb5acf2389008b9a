"""hyq_decode_attn_noalloc (the decode for callers that cannot allocate) through the C ABI:
two calls in a row, the second on a smaller input, each bit-identical to hyq_decode_attn on the
same cache (same kernels and split plan) and within the decode bar of the oracle (2e-3 max-abs,
1e-3 relative L2); a call too large for the static scratch is rejected before any work."""
import numpy as np
import pytest
import torch

from hybrid_precision_kv_amd import api as hq
from hybrid_precision_kv_amd import _lib
from oracle import attention as att
from oracle import numerics as nm
from tests.test_gpu_decode import MAX_ABS, REL_L2, Pair, dev

pytestmark = pytest.mark.gpu


def _oracle(p, q_bits):
    ref = np.empty((p.B, p.Hkv * p.G, 128), np.float32)
    for b in range(p.B):
        for h in range(p.Hkv):
            Kh, Vh = p.refs[b * p.Hkv + h].stored_kv()
            ref[b, h * p.G:(h + 1) * p.G] = att.decode_ref(nm.bf16_to_f32(q_bits[b, h * p.G:(h + 1) * p.G]), Kh, Vh)
    return ref


def _check(p, q_bits, n_splits):
    out = torch.full((p.B, p.Hkv * p.G, 128), float("nan"), dtype=torch.float32, device="cuda")
    hq.decode_attn_noalloc(p.cache, dev(q_bits), out, n_splits)
    with_ws = hq.decode_attn(p.cache, dev(q_bits), n_splits)
    torch.cuda.synchronize()
    assert torch.equal(out, with_ws), "noalloc and workspace calls differ"
    o = out.cpu().numpy()
    ref = _oracle(p, q_bits)
    err = np.abs(o - ref).max()
    rel = np.linalg.norm(o - ref) / np.linalg.norm(ref)
    print(f"  noalloc B={p.B} Hkv={p.Hkv} L={p.cache.len} splits={n_splits}: max-abs {err:.3g} rel-L2 {rel:.3g}")
    assert err <= MAX_ABS and rel <= REL_L2


def test_noalloc_two_calls_second_smaller():
    big = Pair(9600, 2, 2, 4, 3001, n_steps=1)
    small = Pair(9601, 1, 1, 4, 700, n_steps=1)
    qb, qs = big.append(), small.append()
    for s in (0, 7):
        _check(big, qb, s)
        _check(small, qs, s)


def test_noalloc_rejects_more_than_the_scratch():
    p = Pair(9602, 2, 2, 4, 900, n_steps=1)
    q = p.append()
    per_split = p.B * p.Hkv * p.G * 130 * 4
    s = _lib.HYQ_NOALLOC_SCRATCH_BYTES // per_split + 1
    out = torch.zeros((p.B, p.Hkv * p.G, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(_lib.HyqError) as ei:
        hq.decode_attn_noalloc(p.cache, dev(q), out, s)
    assert ei.value.status == 4
    torch.cuda.synchronize()
    assert not out.any()

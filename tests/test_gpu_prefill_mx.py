"""GPU parity of the hybrid prefill with an MXFP4 bulk Q.K^T (hyq_prefill_attn_mx; HyQuant
paper §4.2, the INT4/FP4 option for the bulk operands) against the oracle.

Bar:
  * MXFP4 codes and block exponents of Q and K, E4M3 V codes, s_V and the anchor bitmap
    bit-exact (read back from the documented workspace layout);
  * outputs within 2e-3 max-abs and 1e-3 relative L2 of
    ``oracle.attention.prefill_ref(..., bulk="mxfp4")``, which takes the bulk scores as
    fp32(exact MX dot) * alpha and the P rounding decisions in fp32 like the kernel.
"""
import numpy as np
import pytest
import torch

from hybrid_precision_kv_amd import api as hq
from hybrid_precision_kv_amd import synth
from oracle import attention as att
from oracle import numerics as nm
from tests.gpu_layout import read_prefill_mx, read_prefill_ws
from tests.test_gpu_decode import dev
from tests.test_gpu_prefill import anchors_dense, check_out, report_midpoints

pytestmark = pytest.mark.gpu


def run_gpu_mx(d, A, Hq, Hkv, N):
    shape = hq.Shape(1, Hq, Hkv, int4_cap=32, anchor_cap=max(32, -(-A.shape[1] // 32) * 32))
    ws = hq.prefill_workspace(shape, N)
    anc = torch.from_numpy(np.ascontiguousarray(A)).cuda() if A.shape[1] else None
    o = hq.prefill_attn(shape, dev(d["Q"]), dev(d["K"]), dev(d["V"]), anchors=anc, ws=ws, bulk="mxfp4")
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    w = read_prefill_ws(raw, Hq, Hkv, N, shape.anchor_cap)
    w.update(read_prefill_mx(raw, Hq, Hkv, N, shape.anchor_cap))
    return o.cpu().numpy(), w


def check_operands_mx(w, qz, A, N):
    assert np.array_equal(w["q4"][:, :N], qz["q4"]), "Q codes"
    assert np.array_equal(w["qe"][:, :N], qz["qe"]), "Q block exponents"
    assert not w["q4"][:, N:].any() and (w["qe"][:, N:] == -127).all(), "padded Q rows"
    assert np.array_equal(w["k4"][:, :N], qz["k4"]), "K codes"
    assert np.array_equal(w["ke"][:, :N], qz["ke"]), "K block exponents"
    assert np.array_equal(w["sv"].view(np.uint32), qz["sv"].view(np.uint32)), "s_V"
    assert np.array_equal(nm.e4m3_value(w["v8"][:, :N]), qz["v8"]), "V codes"
    bits = np.zeros(w["abits"].shape, np.uint32)
    for h in range(A.shape[0]):
        for a in A[h]:
            bits[h, a >> 5] |= np.uint32(1 << (int(a) & 31))
    assert np.array_equal(w["abits"], bits), "anchor bitmap"


def parity_mx(d, A, Hq, Hkv, N, label, blocks=None, heads=None):
    print(f"[case] mx {label} Hq={Hq} Hkv={Hkv} N={N} k={A.shape[1]}", flush=True)
    o, w = run_gpu_mx(d, A, Hq, Hkv, N)
    qz = att.prefill_quantize_mx(d["Q"], d["K"], d["V"], A)
    check_operands_mx(w, qz, A, N)
    stats = {}
    ref = att.prefill_ref(d["Q"], d["K"], d["V"], A, blocks=blocks, heads=heads, qz=qz, bulk="mxfp4", stats=stats)
    report_midpoints(stats, "mx " + label)
    check_out(o, ref, "mx " + label)
    return o


@pytest.mark.parametrize("Hq,Hkv,N,pct", [(4, 1, 1000, 5), (8, 2, 1500, 5), (2, 1, 700, 10),
                                          (8, 8, 900, 5)])
def test_prefill_mx_parity(Hq, Hkv, N, pct):
    d = synth.gen_prefill(6000 + N, Hq, Hkv, N)
    parity_mx(d, anchors_dense(d, Hq, Hkv, N, pct), Hq, Hkv, N, f"pct={pct}")


@pytest.mark.parametrize("N", [1, 64, 127, 128, 129, 192, 255, 257, 320])
def test_prefill_mx_edge_lengths(N):
    d = synth.gen_prefill(6100 + N, 2, 1, N)
    parity_mx(d, anchors_dense(d, 2, 1, N), 2, 1, N, f"edge N={N}")


def test_prefill_mx_no_anchors_and_all_anchors():
    d = synth.gen_prefill(6200, 4, 2, 700)
    parity_mx(d, np.zeros((2, 0), np.int32), 4, 2, 700, "no anchors")
    d = synth.gen_prefill(6201, 4, 2, 400)
    A = np.tile(np.arange(400 - 128, dtype=np.int32), (2, 1))
    parity_mx(d, A, 4, 2, 400, "all anchors")


def test_prefill_mx_block_exponents():
    """Blocks of very different magnitude in one row (the per-block shared exponents carry
    them), all-zero blocks and rows (e = -127), values on E2M1 rounding midpoints of their
    block (ties to the even code) and negative zeros."""
    N = 500
    d = synth.gen_prefill(6300, 4, 1, N)
    A = anchors_dense(d, 4, 1, N)
    Q = nm.bf16_to_f32(d["Q"])
    K = nm.bf16_to_f32(d["K"])
    Q[:, :, 32:64] *= np.float32(2.0 ** 3)
    Q[:, :, 64:96] *= np.float32(2.0 ** -6)
    K[0, :, 0:32] *= np.float32(2.0 ** -4)
    K[0, :, 96:128] *= np.float32(2.0 ** 2)
    Q[1, 200:260] = 0.0
    # smallest normal magnitudes: floor(log2 amax) - 2 = -128 is clamped to the E8M0 minimum
    Q[2, 50, 0:32] = np.float32(2.0 ** -126) * np.resize(np.array([1.0, -1.5, 1.75, 0.0], np.float32), 32)
    K[0, 300:310, 32:64] = -0.0
    # row 140 of K: block 0 = amax 4 (e = 0) and E2M1 midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    K[0, 140, 0] = 4.0
    K[0, 140, 1:8] = mids
    K[0, 140, 8:15] = -mids
    d["Q"] = nm.f32_to_bf16(Q)
    d["K"] = nm.f32_to_bf16(K)
    parity_mx(d, A, 4, 1, N, "block exponents")


def test_prefill_mx_deterministic():
    d = synth.gen_prefill(6500, 4, 1, 800)
    A = anchors_dense(d, 4, 1, 800)
    a, _ = run_gpu_mx(d, A, 4, 1, 800)
    b, _ = run_gpu_mx(d, A, 4, 1, 800)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("N,blocks,heads", [(8192, [0, 2, 64, 127], [0, 5, 31]),
                                           (32768, [0, 255, 511], [0, 31])])
def test_prefill_mx_full_size_sampled(N, blocks, heads):
    """Hybrid-prefill workload shapes (32 Q / 8 KV heads, 5% anchors, 8K and 32K tokens, the
    lengths the benchmark times): operands compared in full, outputs on sampled (64-query
    block, head) pairs."""
    d = synth.gen_prefill(6600 + N, 32, 8, N)
    parity_mx(d, anchors_dense(d, 32, 8, N), 32, 8, N, f"full N={N}", blocks=blocks, heads=heads)

#!/usr/bin/env python3
"""Benchmark of hybrid-precision decode attention on one MI355X.

Workload (default): Qwen3-8B-shaped batched decode -- batch 16 x 32768-token context,
32 Q / 8 KV heads, head_dim 128, K4V4 INT4 cache with the top 5% vertical-line anchors
and a 128-token window in bf16, 36 layers of cache resident in HBM; one layer's
hyq_decode_attn is timed per step, rotating over the 36 layers so successive steps never
hit the same 800 MB (far beyond the 256 MB Infinity Cache).

Inputs are seeded and synthetic (planted-anchor keys, see hybrid_precision_kv_amd.synth),
generated on the GPU for the 36 layers; anchors come from hyq_select_vlines when it is
available, else from a torch-side top-k of the same vertical-line score (input preparation
only; the timed step is the library's decode kernel alone).

Prints one JSON line: the headline (metric, value in GB/s of algorithmic bytes per step,
ms_per_step, roofline against the 8 TB/s HBM peak with the stored traffic counters, config),
the other hot-path rows under `rows` (each with its own roofline where one applies), and the
oracle timed on the host under `cpu_baseline`.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "hybrid decode-attn µs/step + achieved HBM GB/s, 32K ctx, bs1/bs16"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_T = 2500.0  # dense f16/bf16 MFMA, TFLOP/s
D, W = 128, 128


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed decode steps right before the timed loop (after the --ramp-steps pre-pass)")
    ap.add_argument("--ramp-steps", type=int, default=1500,
                    help="decode steps run before the warm-up steps, as part of setup: after setup the "
                         "device needs several hundred steps to reach its steady rate (reported as ramp_steps)")
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--ctx", type=int, default=32768)
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--hq", type=int, default=32)
    ap.add_argument("--hkv", type=int, default=8)
    ap.add_argument("--splits", type=int, default=0, help="splits per (b, KV head); 0 = library default")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-heads", type=int, default=32)
    ap.add_argument("--no-cpu-rows", action="store_true",
                    help="time the oracle on the decode sample only (not the selector, refresh and prefill rows)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (PMC byte-counter calibration)")
    ap.add_argument("--seed", type=int, default=3000)
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the other hot-path rows (append, selector/refresh, prefill)")
    ap.add_argument("--prefill-lens", default="8192,32768")
    ap.add_argument("--only-selector", action="store_true",
                    help="run only the selector rows (Eq. 4 selector and cache maintenance, Alg. 1 variant)")
    ap.add_argument("--only-alg1", action="store_true",
                    help="run only the Alg. 1-literal selector row (against the Eq. 4 selector)")
    ap.add_argument("--only-bits", action="store_true",
                    help="run only the bulk bit-width row (K4V4 against K8V8 decode)")
    ap.add_argument("--only-ragged", action="store_true",
                    help="run only the variable-length batch row")
    ap.add_argument("--only-gqa8", action="store_true",
                    help="run only the GQA-8 decode row (64 Q / 8 KV heads, bs4 x 32K)")
    ap.add_argument("--only-prefill", action="store_true",
                    help="run only the hybrid-prefill rows (for profiling the prefill kernels)")
    ap.add_argument("--only-bs1", action="store_true",
                    help="run only the batch-1 decode sweep (for a kernel trace of its launches)")
    ap.add_argument("--bs1-ctxs", default="1024,4096,16384,32768")
    ap.add_argument("--only-freeze", action="store_true",
                    help="run only the Freeze row (bs16 x 32K quantization into the hybrid layout)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of the decode kernel's sources and of its compile flags."""
    from hybrid_precision_kv_amd import build
    h = hashlib.sha256()
    for f in ("decode.hip", "hyq_common.h"):
        with open(os.path.join(ROOT, "hybrid_precision_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(build.COMMON + build.EXTRA["decode.hip"]).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch measured with rocprofv3 PMC counters (profiles/), or None when
    the decode kernel source changed since they were taken."""
    p = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def make_layer(torch, hq, shape, B, Hkv, G, L, gen, device, all_bf16=False, keep=False):
    """One layer: planted-anchor K/V/proxies on the GPU, anchors, Freeze into a hybrid cache.
    all_bf16: every candidate position is an anchor (k = P), so nothing is quantized.
    keep: also return the bf16 K and V the cache was frozen from."""
    Hq = Hkv * G
    H = B * Hkv
    u = torch.randn(H, D, generator=gen, device=device)
    u = u / u.norm(dim=-1, keepdim=True)
    K = torch.randn(H, L, D, generator=gen, device=device, dtype=torch.bfloat16)
    V = torch.randn(B, Hkv, L, D, generator=gen, device=device, dtype=torch.bfloat16)
    n_extra = max(0, min(15, L - W - 1))
    if n_extra:  # planted keys: position 0 plus n_extra distinct positions of [1, L - W)
        extra = 1 + torch.rand(H, L - W - 1, generator=gen, device=device).argsort(dim=1)[:, :n_extra]
        pos = torch.cat([torch.zeros(H, 1, dtype=extra.dtype, device=device), extra], dim=1)
    else:
        pos = torch.zeros(H, 1, dtype=torch.long, device=device)
    rows = torch.arange(H, device=device)[:, None].expand_as(pos)
    K[rows, pos] = (K[rows, pos].float() + 4.0 * u[:, None, :]).to(torch.bfloat16)
    K = K.view(B, Hkv, L, D)
    uq = u.view(B, Hkv, D).repeat_interleave(G, dim=1)  # [B][Hq][D]
    proxy = (2.0 * uq[:, :, None, :] + torch.randn(B, Hq, 64, D, generator=gen, device=device)).to(torch.bfloat16)
    q = (2.0 * uq + torch.randn(B, Hq, D, generator=gen, device=device)).to(torch.bfloat16)
    k = hq.anchor_count(L, 100 if all_bf16 else 5)
    anchors = None
    if k and all_bf16:
        anchors = torch.arange(k, dtype=torch.int32, device=device).expand(B, Hkv, k).contiguous()
    elif k:
        try:
            anchors = hq.select_vlines(shape, k, dense_k=K, proxy=proxy)
        except hq._lib.HyqError:
            anchors = torch_select(torch, K, proxy, G, k)
    cache = hq.HybridKVCache(shape, device)
    hq.quantize_kv(cache, K, V, anchors, proxy)
    if keep:
        return cache, q, K, V
    del K, V
    return cache, q


def torch_select(torch, K, proxy, G, k, chunk=16):
    """Input preparation fallback: top-k of summed softmax probability (fp32 torch ops)."""
    B, Hkv, L, _ = K.shape
    P = L - W
    Kf = K.view(B * Hkv, L, D)
    Pq = proxy.view(B * Hkv, G * proxy.shape[2], D)
    out = torch.empty(B * Hkv, k, dtype=torch.int32, device=K.device)
    for h0 in range(0, B * Hkv, chunk):
        kk = Kf[h0:h0 + chunk].float()
        pt = Pq[h0:h0 + chunk].float().transpose(1, 2).contiguous()
        z = torch.matmul(kk, pt) / math.sqrt(D)  # [h][L][R]
        S = torch.softmax(z, dim=1)[:, :P].sum(dim=2)
        top = torch.topk(S, k, dim=1).indices
        out[h0:h0 + chunk] = torch.sort(top, dim=1).values.to(torch.int32)
    return out.view(B, Hkv, k)


def algorithmic_bytes(cache, B, Hkv, Hq):
    c = cache.counters()
    n_win = min(c["len"], W)
    sh = cache.shape
    slot = (512 * ((sh.bits or 4) + (sh.bits_v or sh.bits or 4)) + 1024) // 32  # codes + fp16 scale/min per token
    per_head = slot * c["n_int4"] + 512 * (c["n_anchor"] + c["n_staged"] + n_win)
    return B * Hkv * per_head + B * Hq * D * (2 + 4)


def settle(torch, fn, ms=40.0):
    """Run fn back to back for about ``ms`` of device time before a timed region: from idle the
    device needs tens of milliseconds of sustained load to reach its steady rate (the first
    100 batched decode steps after an idle second run about 1.6x slower than steady state)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    us = max(a.elapsed_time(b) * 1e3, 1.0)
    for _ in range(int(min(4000, max(4, ms * 1e3 / us)))):
        fn()
    torch.cuda.synchronize()


def timed(torch, fn, reps, warm=2):
    """Mean and min microseconds of fn() over reps launches (events on the current stream)."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) * 1e3 for a, b in evs]
    return sum(t) / len(t), min(t)


def timed_graph(torch, fn, reps):
    """Mean microseconds of fn() replayed from a captured graph (its launches only, no host
    cost per call), and fn's result from the first replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    g.replay()
    torch.cuda.synchronize()
    first = out.clone() if hasattr(out, "clone") else out
    # untimed replays: the first replays of a freshly captured graph run slower than later ones
    # (the first few graphs of a process by up to 20% at bs16 x 32K)
    for _ in range(max(3, reps // 2)):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    del g
    return us, first


def bench_maintenance(torch, hq, cache, B, Hkv, G, L, gen, dev, ws, out, splits):
    """Decode steps with cache maintenance on one layer: per token hyq_append_token +
    hyq_decode_attn, and every 64 tokens hyq_select_vlines(apply=1) at the 5% rule (the
    refresh cadence of the techwalker.com article on HyQuant)."""
    Hq = Hkv * G
    toks = [((torch.randn(B, Hkv, D, generator=gen, device=dev)).to(torch.bfloat16),
             (torch.randn(B, Hkv, D, generator=gen, device=dev)).to(torch.bfloat16),
             (torch.randn(B, Hq, D, generator=gen, device=dev)).to(torch.bfloat16)) for _ in range(64)]
    q = toks[0][2]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    t_app, t_dec = 0.0, 0.0
    for i in range(64):
        k_t, v_t, q_t = toks[i]
        ev[0].record()
        hq.append_token(cache, k_t, v_t, q_t)
        ev[1].record()
        hq.decode_attn(cache, q_t, splits, out, ws)
        ev[2].record()
        torch.cuda.synchronize()
        t_app += ev[0].elapsed_time(ev[1]) * 1e3
        t_dec += ev[1].elapsed_time(ev[2]) * 1e3
    k = hq.anchor_count(cache.len)
    # the selection alone (no state change), then the same selection applied: the difference
    # is the refresh
    ev[0].record()
    idx = hq.select_vlines(cache.shape, k, cache=cache)
    ev[1].record()
    torch.cuda.synchronize()
    t_sel = ev[0].elapsed_time(ev[1]) * 1e3
    model = refresh_bytes(torch, cache, idx)
    ev[0].record()
    hq.select_vlines(cache.shape, k, cache=cache, apply=True)
    ev[1].record()
    torch.cuda.synchronize()
    t_ref = ev[0].elapsed_time(ev[1]) * 1e3
    t_apply = max(t_ref - t_sel, 1e-3)
    # device time of the per-token work from captured graphs (the staging emptied by the
    # refresh above takes the 60 appends the warm-ups and captures make, of its 64 slots; a
    # replay, warm or timed, repeats the recorded appends into the same slots)
    k_t, v_t, q_t = toks[0]
    # the eager select-and-refresh above leaves the device below its steady rate, and at this
    # size the decode keeps speeding up for well over 100 ms of sustained load (152 -> 124 us
    # per call): settle on decodes alone (no state change) for 250 ms before the graphs
    settle(torch, lambda: hq.decode_attn(cache, q_t, splits, out, ws), ms=250.0)

    def app16():  # 16 appends per graph: one replay of a single tiny kernel measures the host
        for _ in range(16):
            hq.append_token(cache, k_t, v_t, q_t)
    us_app_g = timed_graph(torch, app16, 10)[0] / 16

    def step4():  # 4 append + decode steps per graph, so a replay's host launch is shared
        for _ in range(4):
            hq.append_token(cache, k_t, v_t, q_t)
            o = hq.decode_attn(cache, q_t, splits, out, ws)
        return o
    us_step_g = timed_graph(torch, step4, 10)[0] / 4
    return {"append_us": round(us_app_g, 2), "append_us_eager": round(t_app / 64, 2),
            "append_decode_us_graph": round(us_step_g, 2), "decode_us_with_staging": round(t_dec / 64, 2),
            "select_refresh_us": round(t_ref, 1), "select_us": round(t_sel, 1), "refresh_us": round(t_apply, 1),
            "refresh_bytes": model,
            "refresh_roofline": {"bound": "hbm", "achieved_min_bytes": round(model["min_bytes"] / (t_apply * 1e-6) / 1e9, 1),
                                 "achieved_moved_bytes": round(model["moved_bytes"] / (t_apply * 1e-6) / 1e9, 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac_min_bytes": round(model["min_bytes"] / (t_apply * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
            "anchors_after_refresh": k,
            "us_per_token_amortized": round(us_step_g + t_ref / 64, 2),
            "note": f"one layer, bs{B} ctx {L}+64, refresh every 64 tokens; append_us (a graph of 16 appends, per "
                    "append; append_decode_us_graph from a graph of 4 append + decode steps, per step) are device time from "
                    "captured graphs, select_refresh_us one "
                    "eager call; us_per_token_amortized = append_decode_us_graph + select_refresh_us / 64"}


def refresh_bytes(torch, cache, idx):
    """Byte model of one refresh (select with apply=1) that installs the set ``idx`` [B][Hkv][k]
    into ``cache`` as it stands, counted per head from the positions before the refresh.
    min_bytes: what any refresh must move -- the new anchors' sources (bf16 rows of kept anchors
    and staged tokens, quantized slots of promoted positions) and their bf16 rows written, the
    demoted rows read (bf16) and written as slots, the tail slots moved down (read + write), and
    the position arrays.  moved_bytes adds this design's extra traffic: the new anchor rows pass
    through a temporary store (written once, read once more), the V-code dwords of every quad a
    move touches are read and written whole, the plan reads the slot positions and writes its
    bitmaps and move list."""
    s = cache.shape
    c = cache.counters()
    B, Hkv = idx.shape[0], idx.shape[1]
    L = c["len"]
    P = max(0, L - W)
    n_old, n_anc, n_st = c["n_int4"], c["n_anchor"], c["n_staged"]
    bk = s.bits or 4
    bv = s.bits_v or bk
    slot = (512 * (bk + bv) + 1024) // 32
    a_pos = cache.view("a_pos", torch.int32).view(B * Hkv, s.anchor_cap)[:, :n_anc].cpu().numpy()
    s_pos = cache.view("slot_pos", torch.int32).view(B * Hkv, s.int4_cap)[:, :n_old].cpu().numpy()
    new = idx.reshape(B * Hkv, -1).cpu().numpy()
    import numpy as np
    k = new.shape[1]
    tot = {"demoted": 0, "promoted": 0, "kept": 0, "tail_moves": 0, "tiles_touched": 0}
    mn, mv = 0, 0
    for h in range(B * Hkv):
        nset = np.zeros(max(P, 1), dtype=bool)
        nset[new[h]] = True
        kept_a = int(nset[a_pos[h]].sum())
        staged = np.arange(P - n_st, P)
        kept_s = int(nset[staged].sum())
        dele = nset[s_pos[h]]
        p = int(dele.sum())
        e = (n_anc - kept_a) + (n_st - kept_s)
        n_new = n_old - p + e
        tail = int((~dele[n_new:n_old]).sum()) if n_new < n_old else 0
        holes = np.nonzero(dele[:min(n_new, n_old)])[0]
        dst = np.concatenate([holes, np.arange(n_old, max(n_new, n_old))])
        tiles = len(np.unique(dst >> 5))
        quads = len(np.unique((dst >> 5) * 4 + ((dst & 15) >> 2)))
        tot["demoted"] += e
        tot["promoted"] += p
        tot["kept"] += kept_a + kept_s
        tot["tail_moves"] += tail
        tot["tiles_touched"] += tiles
        row = 2 * D * 2  # a bf16 K row and V row
        a_end = (k + 31) // 32 * 32
        m = (kept_a + kept_s) * row + p * slot + k * row  # new anchors: sources read, rows written
        m += e * (row + slot) + tail * 2 * slot + 4 * (k + n_anc + a_end + e + tail)
        mn += m
        vq = 512 * bv // 4  # bytes of one quad's V codes (all channels)
        mv += m + 2 * k * row + 2 * quads * vq + 4 * n_old + 12 * len(dst)
    return {"min_bytes": mn, "moved_bytes": mv, **tot, "heads": B * Hkv, "k": k}


def bench_decode_bs1(torch, hq, gen, dev, ctxs=(1024, 4096, 16384, 32768), Hq=32, Hkv=8, layers=36, steps=100,
                     B=1, all_bf16=False):
    """Llama-3.1-8B-shaped decode at batch 1 (32 Q / 8 KV heads): hyq_decode_attn per step over
    a context sweep, rotating over ``layers`` caches like the batched workload; ``us_per_step`` is
    device time from a captured graph of one rotation, ``us_per_step_eager`` the host-driven
    loop.  With all_bf16
    every position is kept in bf16 (k = P): the full-precision comparison point of the HyQuant
    paper's Table 7, run by the same kernel."""
    G = Hq // Hkv
    out = {}
    for L in ctxs:
        shape = hq.Shape.for_context(B, Hq, Hkv, L + 64, 100 if all_bf16 else 5)
        lay = [make_layer(torch, hq, shape, B, Hkv, G, L, gen, dev, all_bf16) for _ in range(layers)]
        nbytes = algorithmic_bytes(lay[0][0], B, Hkv, Hq)
        ws = hq.decode_workspace(shape, 0, dev)
        o = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
        rot = iter(range(1 << 30))
        settle(torch, lambda: hq.decode_attn(*lay[next(rot) % layers], 0, o, ws))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            c, q = lay[i % layers]
            hq.decode_attn(c, q, 0, o, ws)
        e1.record()
        torch.cuda.synchronize()
        us_eager = e0.elapsed_time(e1) * 1e3 / steps
        ref = o.clone()  # the last layer's output, eager

        # device time: one captured graph of a full rotation over the layers (a batch-1 call
        # is short enough that the binding's host cost would otherwise set the rate)
        def rotation():
            for i in range(steps - layers, steps):
                c, q = lay[i % layers]
                hq.decode_attn(c, q, 0, o, ws)
            return o
        us_rot, got = timed_graph(torch, rotation, 5)
        us = us_rot / layers
        out[str(L)] = {"us_per_step": round(us, 2), "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
                       "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_step": nbytes,
                       "resident_MB": round(layers * nbytes / 1e6, 1), "us_per_step_eager": round(us_eager, 2),
                       "graph_equal": bool(torch.equal(got, ref))}
        if not all_bf16 and B == 1:
            # full step on one layer: append + decode per token (device time from a captured
            # graph of 4 steps) plus one eager select-and-refresh call amortised over 64 tokens
            m = bench_maintenance(torch, hq, lay[0][0], B, Hkv, G, L, gen, dev, ws, o, 0)
            out[str(L)]["full_step_us"] = m["us_per_token_amortized"]
            out[str(L)]["select_refresh_us"] = m["select_refresh_us"]
        del lay, ws
        torch.cuda.empty_cache()
    return out


def bench_decode_bits(torch, hq, gen, dev, B=16, L=32768, Hq=32, Hkv=8, layers=8, n_ref=2):
    """Bit widths of the quantized bulk (B_K, B_V of the HyQuant paper's Alg. 3/4): the batched
    workload's decode with K4V4, K8V8, K4V2 and K2V2 bulks, all with the 5% bf16 anchors and the
    bf16 window.  Per width: time per step (launches rotating over ``layers`` caches), the
    algorithmic bytes (160, 288, 128 or 96 B per quantized token) and the output's relative L2
    error against fp32 attention over the unquantized bf16 K/V of the first ``n_ref`` sequences."""
    G = Hq // Hkv
    out = {}
    for bits, bits_v in ((4, 4), (8, 8), (4, 2), (2, 2)):
        shape = hq.Shape.for_context(B, Hq, Hkv, L + 64, bits=bits, bits_v=bits_v)
        lay = []
        for i in range(layers):
            lay.append(make_layer(torch, hq, shape, B, Hkv, G, L, gen, dev, keep=(i == 0)))
        c0, q0, K, V = lay[0]
        lay[0] = (c0, q0)
        nbytes = algorithmic_bytes(c0, B, Hkv, Hq)
        ws = hq.decode_workspace(shape, 0, dev)
        o = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
        hq.decode_attn(c0, q0, 0, o, ws)
        torch.cuda.synchronize()
        err = []
        for b in range(n_ref):  # fp32 dense attention, right operands made contiguous first
            qf = q0[b].float().view(Hkv, G, D)
            kt = K[b].float().transpose(1, 2).contiguous()
            p = torch.softmax(torch.bmm(qf, kt) / math.sqrt(D), dim=-1)
            ref = torch.bmm(p, V[b].float().contiguous()).view(Hq, D)
            err.append(((o[b] - ref).norm() / ref.norm()).item())
        del K, V

        # back-to-back launches with events only at the ends, as in the headline loop (a batched
        # step is long enough that queued launches hide the binding's host cost)
        steps = 200
        rot = iter(range(1 << 30))
        settle(torch, lambda: hq.decode_attn(*lay[next(rot) % layers], 0, o, ws))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            hq.decode_attn(*lay[i % layers], 0, o, ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        out[f"k{bits}v{bits_v}"] = {"us_per_step": round(us, 2), "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
                                  "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                  "bytes_per_step": nbytes, "rel_l2_vs_fp32_unquantized": round(max(err), 6)}
        del lay, ws
        torch.cuda.empty_cache()
    out["note"] = (f"bs{B} ctx{L} hq{Hq} hkv{Hkv}, {layers} resident layers, hybrid 5% anchors + bf16 window; "
                   f"error over sequences 0..{n_ref - 1} of the first layer")
    return out


def bench_decode_gqa8(torch, hq, gen, dev, B=4, L=32768, Hq=64, Hkv=8, layers=16, steps=100, copy_cal=False):
    """Decode at GQA 8 (the Qwen3-32B shape of the selector workload: 64 Q / 8 KV heads, batch 4,
    32K, 5% anchors): hyq_decode_attn per step rotating over ``layers`` resident caches.  Each
    wave serves the 8 Q heads of its KV head with two 4-head MFMA column blocks, so the slab is
    streamed once; the algorithmic bytes count it once."""
    G = Hq // Hkv
    shape = hq.Shape.for_context(B, Hq, Hkv, L + 64)
    lay = [make_layer(torch, hq, shape, B, Hkv, G, L, gen, dev) for _ in range(layers)]
    torch.cuda.synchronize()
    nbytes = algorithmic_bytes(lay[0][0], B, Hkv, Hq)
    ws = hq.decode_workspace(shape, 0, dev)
    o = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    rot = iter(range(1 << 30))
    settle(torch, lambda: hq.decode_attn(*lay[next(rot) % layers], 0, o, ws))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        hq.decode_attn(lay[i % layers][0], lay[i % layers][1], 0, o, ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    if copy_cal:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b2 = torch.empty_like(a)
        for _ in range(5):
            b2.copy_(a)
        torch.cuda.synchronize()
        del a, b2
    del lay
    torch.cuda.empty_cache()
    return {"workload": f"qwen3-32b-shape decode bs{B} ctx{L} hq{Hq} hkv{Hkv} layers{layers}",
            "us_per_step": round(us, 2), "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_step": nbytes,
            "note": "one wave serves the 8 Q heads of a KV head (two 4-head column blocks); bytes count the slab once"}


def ragged_lengths(n_seq, seed, lo=2048, hi=32768):
    """The variable-length batch's context lengths: seeded, uniform over [lo, hi]."""
    import numpy as np
    return [int(x) for x in np.random.default_rng(seed).integers(lo, hi + 1, size=n_seq)]


def bench_decode_ragged(torch, hq, gen, dev, n_seq=16, Hq=32, Hkv=8, layers=4, seed=77):
    """A variable-length batch: 16 sequences of seeded lengths in [2K, 32K], each its own
    single-sequence cache (5% anchors), decoded by one hyq_decode_attn_ragged call per step,
    rotating over ``layers`` resident batches.  Beside it: the same sequences decoded by one
    hyq_decode_attn call each (device time from a captured graph of the 16 calls, and the
    host-driven time)."""
    G = Hq // Hkv
    lens = ragged_lengths(n_seq, seed)
    lay = []
    for _ in range(layers):
        cs, qs = [], []
        for L in lens:
            shape = hq.Shape.for_context(1, Hq, Hkv, L + 64)
            c, q = make_layer(torch, hq, shape, 1, Hkv, G, L, gen, dev)
            cs.append(c)
            qs.append(q)
        lay.append((cs, torch.cat(qs, dim=0)))
    torch.cuda.synchronize()
    nbytes = sum(algorithmic_bytes(c, 1, Hkv, Hq) for c in lay[0][0])
    ws = torch.empty(hq.decode_ragged_workspace_bytes(lay[0][0][0].shape, n_seq), dtype=torch.uint8, device=dev)
    o = torch.empty(n_seq, Hq, D, dtype=torch.float32, device=dev)
    steps = 200
    rot = iter(range(1 << 30))

    def one():
        i = next(rot) % layers
        hq.decode_attn_ragged(lay[i][0], lay[i][1], 0, o, ws)
    settle(torch, one)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        hq.decode_attn_ragged(lay[i % layers][0], lay[i % layers][1], 0, o, ws)
    e1.record()
    torch.cuda.synchronize()
    us_eager = e0.elapsed_time(e1) * 1e3 / steps
    # device time: one captured graph of a rotation over the resident batches, each call with
    # its own page-locked table (the replay copies the table, then runs the two kernels)
    tables = [hq.decode_ragged_table(lay[0][0][0].shape, n_seq) for _ in range(layers)]

    def rotation():
        for i in range(layers):
            hq.decode_attn_ragged(lay[i][0], lay[i][1], 0, o, ws, table=tables[i])
        return o
    us_rot, ragged_out = timed_graph(torch, rotation, 25)  # output of the last batch
    us = us_rot / layers
    # the same sequences one call each
    wss = [hq.decode_workspace(c.shape, 0, dev) for c in lay[0][0]]
    os1 = [torch.empty(1, Hq, D, dtype=torch.float32, device=dev) for _ in lens]

    def one_by_one(cs, qq):
        for j, c in enumerate(cs):
            hq.decode_attn(c, qq[j:j + 1], 0, os1[j], wss[j])
        return os1[0]
    last = lay[layers - 1]
    one_by_one(*last)
    torch.cuda.synchronize()
    us_sep_eager, _ = timed(torch, lambda: one_by_one(*last), 20)
    graph_us = []
    for cs, qq in lay:
        u, _ = timed_graph(torch, lambda: one_by_one(cs, qq), 10)
        graph_us.append(u)
    us_sep = sum(graph_us) / len(graph_us)
    one_by_one(*last)
    torch.cuda.synchronize()
    # outputs agree up to the split plans (the automatic plans differ between the two forms)
    diff = max(float((os1[j][0] - ragged_out[j]).abs().max()) for j in range(n_seq))
    out = {"lengths": lens, "tokens": sum(lens), "us_per_step": round(us, 2),
           "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
           "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_step": nbytes,
           "us_per_step_eager": round(us_eager, 2),
           "separate_calls_us_graph": round(us_sep, 2), "separate_calls_us_eager": round(us_sep_eager, 2),
           "speedup_vs_separate_graph": round(us_sep / us, 2), "max_abs_diff_vs_separate": diff,
           "note": f"{n_seq} single-sequence caches, hq{Hq} hkv{Hkv}, {layers} resident batches; us_per_step is "
                   "device time from a captured rotation (table copy, split kernel, merge per call); "
                   "us_per_step_eager the host-driven loop"}
    del lay, wss
    torch.cuda.empty_cache()
    return out


def bench_selector(torch, hq, gen, dev, B=4, Hq=64, Hkv=8, L=32768):
    """Selector and cache maintenance at Qwen3-32B shape (64 Q / 8 KV heads, batch 4, 32K):
    hyq_select_vlines scores + top-k at 1% / 5% / 10%; then 64 appends and one select call with
    apply (selector + cache refresh, timed together)."""
    G = Hq // Hkv
    shape = hq.Shape.for_context(B, Hq, Hkv, L + 64, 10)
    cache, _ = make_layer(torch, hq, shape, B, Hkv, G, L, gen, dev)
    res = {"workload": f"qwen3-32b-shape select bs{B} ctx{L} hq{Hq} hkv{Hkv}"}
    settle(torch, lambda: hq.select_vlines(shape, hq.anchor_count(L, 5), cache=cache))
    for pct in (1, 5, 10):
        k = hq.anchor_count(L, pct)
        us, _ = timed(torch, lambda: hq.select_vlines(shape, k, cache=cache), 5)
        res[f"select_{pct}pct_us_eager"] = round(us, 1)
        ref = hq.select_vlines(shape, k, cache=cache)
        us, got = timed_graph(torch, lambda: hq.select_vlines(shape, k, cache=cache), 10)
        res[f"select_{pct}pct_us"] = round(us, 1)
        res[f"select_{pct}pct_graph_equal"] = bool(torch.equal(got, ref))
    # MFMA roofline: the algorithmic work of one selection is one alpha Q K^T over every proxy
    # row and key (2 R L D flops per (b, KV head), R = 64 G rows) at the dense f16/bf16 MFMA
    # peak; the two-pass softmax computes that product twice and takes two exponentials per
    # (row, key) pair, which the achieved figure does not credit
    R = 64 * G
    flops = 2.0 * B * Hkv * R * L * D
    us5 = res["select_5pct_us"]
    res["roofline"] = {"bound": "mfma", "achieved": round(flops / (us5 * 1e-6) / 1e12, 1), "peak": MFMA_BF16_PEAK_T,
                       "unit": "TFLOP/s", "frac": round(flops / (us5 * 1e-6) / 1e12 / MFMA_BF16_PEAK_T, 4),
                       "traffic": None, "flops_per_call": flops, "exps_per_call": 2 * B * Hkv * R * (L - W),
                       "basis": "5% call; one Q.K^T of every proxy row against every key, f16/bf16 dense peak"}
    k_t = torch.randn(B, Hkv, D, generator=gen, device=dev).to(torch.bfloat16)
    q_t = torch.randn(B, Hq, D, generator=gen, device=dev).to(torch.bfloat16)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(64):
        hq.append_token(cache, k_t, k_t, q_t)
    ev[1].record()
    hq.select_vlines(shape, hq.anchor_count(cache.len, 5), cache=cache, apply=True)
    ev[2].record()
    torch.cuda.synchronize()
    res["append_64_us"] = round(ev[0].elapsed_time(ev[1]) * 1e3, 1)
    res["select_and_apply_us"] = round(ev[1].elapsed_time(ev[2]) * 1e3, 1)
    del cache
    return res


def bench_selector_alg1(torch, hq, gen, dev, L=32768, Hq=32, Hkv=8, n_dec=16):
    """Alg. 1-literal selector (tail-query mean, raw logits, one set per Q head) against the
    Eq. 4 selector at the prefill-to-decode boundary (one sequence, 32 Q / 8 KV heads, 32K
    keys, planted vertical keys): time of each call, overlap of the sets, and the relative
    MSE of hybrid decode (anchors bf16, the rest INT4, 128-token window) against exact fp32
    attention for n_dec new queries, with each set as the anchors.  The per-Q-head sets are
    evaluated on a cache with one KV head copy per Q head."""
    G = Hq // Hkv
    P = L - W
    u = torch.randn(Hkv, D, generator=gen, device=dev)
    u = u / u.norm(dim=-1, keepdim=True)
    K = torch.randn(Hkv, L, D, generator=gen, device=dev)
    pos = torch.cat([torch.zeros(Hkv, 1, dtype=torch.long, device=dev),
                     1 + torch.rand(Hkv, P - 1, generator=gen, device=dev).argsort(dim=1)[:, :15]], dim=1)
    K[torch.arange(Hkv, device=dev)[:, None], pos] += 4.0 * u[:, None, :]
    K = K.to(torch.bfloat16)[None].contiguous()
    V = torch.randn(1, Hkv, L, D, generator=gen, device=dev).to(torch.bfloat16)
    uq = u.repeat_interleave(G, dim=0)
    tail = (2.0 * uq[:, None, :] + torch.randn(Hq, W, D, generator=gen, device=dev)).to(torch.bfloat16)[None].contiguous()
    qd = (2.0 * uq[None] + torch.randn(n_dec, Hq, D, generator=gen, device=dev)).to(torch.bfloat16)
    shape = hq.Shape.for_context(1, Hq, Hkv, L)
    k1, k4 = hq.anchor_count_alg1(L), hq.anchor_count(L)
    ws = hq.select_tail_workspace(shape, L, dev)
    proxy = tail[:, :, W - 64:].contiguous()
    us1_eager, _ = timed(torch, lambda: hq.select_vlines_tail(shape, k1, K, tail, ws=ws), 10)
    us4_eager, _ = timed(torch, lambda: hq.select_vlines(shape, k4, dense_k=K, proxy=proxy), 10)
    A1 = hq.select_vlines_tail(shape, k1, K, tail)[0]  # [Hq][k1]
    A4 = hq.select_vlines(shape, k4, dense_k=K, proxy=proxy)  # [1][Hkv][k4]
    # device time: the calls replayed from captured graphs (the replay's sets must match)
    us1, g1 = timed_graph(torch, lambda: hq.select_vlines_tail(shape, k1, K, tail, ws=ws), 20)
    us4, g4 = timed_graph(torch, lambda: hq.select_vlines(shape, k4, dense_k=K, proxy=proxy), 20)
    graph_same = bool(torch.equal(g1[0], A1) and torch.equal(g4, A4))
    ov = []
    for h in range(Hq):
        a, b = A1[h].long(), A4[0, h // G].long()
        ov.append(torch.isin(a, b).sum().item() / min(len(a), len(b)))
    # exact attention (fp32) for the decode queries
    Kf, Vf = K[0].float(), V[0].float()
    Ke, Ve = Kf.repeat_interleave(G, dim=0), Vf.repeat_interleave(G, dim=0)  # [Hq][L][D]
    exact = [torch.softmax(torch.bmm(Ke, qd[i].float()[:, :, None])[:, :, 0] / math.sqrt(D), dim=-1)[:, None, :]
             .bmm(Ve)[:, 0] for i in range(n_dec)]

    def rel_mse(cache):
        num = den = 0.0
        for i in range(n_dec):
            o = hq.decode_attn(cache, qd[i][None].contiguous())[0]
            num += ((o - exact[i]) ** 2).sum().item()
            den += (exact[i] ** 2).sum().item()
        return num / den

    res = {"workload": f"selector at the prefill boundary ctx{L} hq{Hq} hkv{Hkv} (planted vertical keys)",
           "alg1_k": k1, "eq4_k": k4, "alg1_us": round(us1, 1), "eq4_us": round(us4, 1),
           "alg1_us_eager": round(us1_eager, 1), "eq4_us_eager": round(us4_eager, 1), "graph_sets_equal": graph_same,
           "overlap_mean": round(sum(ov) / len(ov), 4), "overlap_min": round(min(ov), 4)}
    c4 = hq.HybridKVCache(shape, dev)
    hq.quantize_kv(c4, K, V, A4.contiguous(), proxy)
    res["eq4_rel_mse"] = float(f"{rel_mse(c4):.4g}")
    c0 = hq.HybridKVCache(shape, dev)
    hq.quantize_kv(c0, K, V, None, proxy)
    res["no_anchor_rel_mse"] = float(f"{rel_mse(c0):.4g}")
    del c4, c0
    shape_e = hq.Shape.for_context(1, Hq, Hq, L)
    ce = hq.HybridKVCache(shape_e, dev)
    hq.quantize_kv(ce, Ke.to(torch.bfloat16)[None].contiguous(), Ve.to(torch.bfloat16)[None].contiguous(),
                   A1[None].contiguous(), proxy)
    res["alg1_rel_mse"] = float(f"{rel_mse(ce):.4g}")
    del ce
    # roofline of the Alg. 1 call: prefix keys once per KV head, the tail queries, the indices
    alg_bytes = Hkv * P * D * 2 + Hq * W * D * 2 + Hq * k1 * 4
    res["roofline"] = {"bound": "hbm", "achieved": round(alg_bytes / (us1 * 1e-6) / 1e9, 1), "peak": 8000.0,
                       "unit": "GB/s", "frac": round(alg_bytes / (us1 * 1e-6) / 8e12, 4), "traffic": None,
                       "bytes": alg_bytes}
    return res


def freeze_bytes(B, Hq, Hkv, L, k, n_proxy, slot_bytes):
    """Algorithmic bytes of one Freeze (HyQuant paper Alg. 4): every K and V row read once as
    bf16, the anchor list and the proxy queries read; written: one quantized slot record
    (codes plus fp16 scale and min) and its position for each of the L - W - k bulk
    positions, a bf16 K and V row and its position for each anchor, the bf16 window, the
    proxy ring.  Clearing the staging store is not counted (the empty set needs no bytes)."""
    n_int4 = L - W - k
    read = B * Hkv * (2 * L * D * 2 + 4 * k) + B * Hq * n_proxy * D * 2
    write = B * Hkv * ((slot_bytes + 4) * n_int4 + (512 + 4) * k + 512 * W) + B * Hq * n_proxy * D * 2
    return read + write


def bench_freeze(torch, hq, gen, dev, B=16, L=32768, Hq=32, Hkv=8, bits=4, reps=20):
    """Freeze at the batched decode workload: bs16 x 32K, 32 Q / 8 KV heads, K4V4 bulk, the 5%
    anchor count at random ascending positions of the candidate prefix, 64 proxy queries.
    Timed per call with events after the device has settled; HBM roofline on the
    algorithmic bytes of freeze_bytes."""
    shape = hq.Shape.for_context(B, Hq, Hkv, L + 64, bits=bits)
    K = torch.randn(B, Hkv, L, D, generator=gen, device=dev, dtype=torch.bfloat16)
    V = torch.randn(B, Hkv, L, D, generator=gen, device=dev, dtype=torch.bfloat16)
    proxy = torch.randn(B, Hq, 64, D, generator=gen, device=dev).to(torch.bfloat16)
    k = hq.anchor_count(L, 5)
    P = L - W
    anchors = torch.rand(B * Hkv, P, generator=gen, device=dev).argsort(dim=1)[:, :k]
    anchors = anchors.sort(dim=1).values.to(torch.int32).view(B, Hkv, k).contiguous()
    cache = hq.HybridKVCache(shape, dev)
    f = lambda: hq.quantize_kv(cache, K, V, anchors, proxy)  # noqa: E731
    settle(torch, f)
    us, us_min = timed(torch, f, reps)
    slot = (512 * 2 * bits + 1024) // 32
    nbytes = freeze_bytes(B, Hq, Hkv, L, k, 64, slot)
    achieved = nbytes / (us * 1e-6) / 1e9
    del K, V, cache
    torch.cuda.empty_cache()
    return {"workload": f"freeze bs{B} ctx{L} hq{Hq} hkv{Hkv} anchors{k} K{bits}V{bits}",
            "us_per_call": round(us, 1), "us_min": round(us_min, 1), "bytes_per_call": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "hyq_quantize_kv (quantized slots, anchor and window stores, staging "
                                   "clear, proxy ring; all launches of the call)"}}


def prefill_ops(anchors_row, N, Hq):
    """Algorithmic MFMA work of the hybrid prefill (per Q head: every (query, key) pair the
    method visits, QK^T and PV at 2 x 128 multiply-adds each): quantized pairs j <= i-128 not
    anchors; bf16 pairs = anchors a <= i-128 plus the window min(i+1, 128)."""
    import numpy as np
    a = np.sort(np.asarray(anchors_row))
    i = np.arange(N)
    n_before = np.maximum(0, i - W + 1)
    n_anc = np.searchsorted(a, i - W, side="right")
    n_win = np.minimum(i + 1, W)
    per_pair = 2 * 2 * D
    ops8 = float((n_before - n_anc).sum()) * Hq * per_pair
    opsb = float((n_anc + n_win).sum()) * Hq * per_pair
    return ops8, opsb


def bench_prefill(torch, hq, gen, dev, N, Hq=32, Hkv=8, bulk="int8"):
    """Hybrid prefill, one sequence of N tokens, 32 Q / 8 KV heads; anchors = the library's
    selector over the last 64 queries (dense keys), 5% rule.  ``bulk``: the bulk Q.K^T format,
    "int8" or "mxfp4" (P.V stays FP8 in both)."""
    G = Hq // Hkv
    u = torch.randn(Hkv, D, generator=gen, device=dev)
    u = u / u.norm(dim=-1, keepdim=True)
    K = torch.randn(Hkv, N, D, generator=gen, device=dev)
    pos = torch.cat([torch.zeros(Hkv, 1, dtype=torch.long, device=dev),
                     1 + torch.rand(Hkv, N - W - 1, generator=gen, device=dev).argsort(dim=1)[:, :15]], dim=1)
    K[torch.arange(Hkv, device=dev)[:, None], pos] += 4.0 * u[:, None, :]
    K = K.to(torch.bfloat16)
    V = torch.randn(Hkv, N, D, generator=gen, device=dev).to(torch.bfloat16)
    Q = (2.0 * u.repeat_interleave(G, dim=0)[:, None, :] + torch.randn(Hq, N, D, generator=gen, device=dev)).to(torch.bfloat16)
    shape = hq.Shape.for_context(1, Hq, Hkv, N)
    k = hq.anchor_count(N)
    anchors = hq.select_vlines(shape, k, dense_k=K[None], proxy=Q[None, :, N - 64:].contiguous())[0].contiguous()
    ws = hq.prefill_workspace(shape, N, dev)
    o = torch.empty(Hq, N, D, dtype=torch.float32, device=dev)
    reps = 10 if N <= 8192 else 3
    call = lambda: hq.prefill_attn(shape, Q, K, V, anchors=anchors, out=o, ws=ws, bulk=bulk)  # noqa: E731
    settle(torch, call)
    us, us_min = timed(torch, call, reps)
    ops8, opsb = prefill_ops(anchors[0].cpu().numpy(), N, Hq)
    if bulk == "mxfp4":  # Q.K^T half of the bulk work at the fp4 peak, P.V half at fp8
        t_roof = 0.5 * ops8 / 10.1e15 + 0.5 * ops8 / 5.0e15 + opsb / 2.5e15
        basis = "fp4 10.1 (bulk Q.K), fp8 5.0 (bulk P.V) and bf16 2.5 PFLOP/s dense, blended by op mix"
    else:
        t_roof = ops8 / 5.0e15 + opsb / 2.5e15
        basis = "int8/fp8 5.0 POP/s and bf16 2.5 PFLOP/s dense, blended by op mix"
    del K, V, Q, o, ws
    return {"workload": f"hybrid prefill N{N} hq{Hq} hkv{Hkv} anchors{k} bulk {bulk}", "us_per_call": round(us, 1),
            "us_min": round(us_min, 1), "tokens_per_s": round(N / (us * 1e-6), 1),
            "roofline": {"bound": "mfma", "achieved": round((ops8 + opsb) / (us * 1e-6) / 1e12, 1),
                         "peak": round((ops8 + opsb) / t_roof / 1e12, 1), "unit": "TFLOP/s",
                         "frac": round(t_roof / (us * 1e-6), 4), "traffic": None,
                         "ops_int8_fp8": ops8, "ops_bf16": opsb,
                         "peak_basis": basis}}


def cpu_baseline(args, G, bytes_per_head):
    """The oracle as it stands, on a bounded sample of the same workload: decode over
    ``cpu-sample-heads`` (sequence, KV head) caches of the same shape."""
    import numpy as np
    from hybrid_precision_kv_amd import synth
    from oracle import attention as att
    from oracle import numerics as nm
    from oracle import policy as pol
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    heads = []
    for i in range(args.cpu_sample_heads):
        s = synth.HeadStream(synth.seed_for(args.seed, i // args.hkv, i % args.hkv), args.ctx, G)
        A, _ = pol.select_dense(s.K, s.queries(64))
        c = pol.HybridCacheRef(g=G)
        c.freeze(s.K, s.V, A)
        heads.append((c, nm.bf16_to_f32(s.queries(1)[:, 0])))
    def run(seconds):  # whole passes over the sample until >= `seconds` of oracle work
        t0 = time.perf_counter()
        passes = 0
        while True:
            for c, q in heads:
                Kh, Vh = c.stored_kv()
                att.decode_ref(q, Kh, Vh)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= seconds or passes >= 200:
                return bytes_per_head * len(heads) * passes / dt / 1e9, passes, dt

    gbs, passes, dt = run(10.0)
    res = {"value": round(gbs, 3), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{passes} passes over {len(heads)} (sequence, KV head) caches of {args.ctx} positions, "
                     f"GQA {G}, one decode step each ({dt:.1f} s; a full step is {args.batch * args.hkv} such heads)",
           "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0))}
    per_head_s = dt / (passes * len(heads))
    res["decode_us_per_step"] = {
        f"bs{args.batch}_{args.ctx}": round(per_head_s * args.batch * args.hkv * 1e6, 1),
        f"bs1_{args.ctx}": round(per_head_s * args.hkv * 1e6, 1),
        "note": "oracle decode time per (sequence, KV head) from the sample above, times the heads of one step"}
    if not args.no_cpu_rows:
        res["rows"] = cpu_rows(args)
    try:  # the same oracle on one thread
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            gbs1, passes1, dt1 = run(3.0)
        res["value_1thread"] = round(gbs1, 3)
        res["sample_1thread"] = f"{passes1} passes, {dt1:.1f} s"
    except Exception as e:  # threadpoolctl missing: report the all-core figure only
        res["value_1thread"] = None
        res["sample_1thread"] = f"not measured ({type(e).__name__})"
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_rows(args):
    """The oracle on bounded samples of the other hot-path rows, extrapolated to one call:
    Freeze, cache-mode selection and refresh at 64 Q / 8 KV heads, 32K (two (sequence, KV head)
    caches, 64 appends each; Freeze scaled to the 128 heads of bs16 x 32K), and the hybrid prefill at 8192 tokens, 32 Q / 8 KV heads (operand
    quantization in full, then six seeded random (64-query block, Q head) pairs)."""
    import numpy as np
    from hybrid_precision_kv_amd import synth
    from oracle import attention as att
    from oracle import policy as pol
    out = {}
    L, G, n_heads_call = 32768, 8, 4 * 8
    t_sel, t_ref, t_frz, n = 0.0, 0.0, 0.0, 2
    for i in range(n):
        s = synth.HeadStream(synth.seed_for(args.seed + 7, i, 0), L, G)
        prox = s.queries(64)
        A, _ = pol.select_dense(s.K, prox)
        c = pol.HybridCacheRef(g=G)
        t0 = time.perf_counter()
        c.freeze(s.K, s.V, A, prox)
        t_frz += time.perf_counter() - t0
        k, v, q = s.new_tokens(64)
        for j in range(64):
            c.append(k[j], v[j], q[:, j])
        t0 = time.perf_counter()
        A2, _ = c.select()
        t1 = time.perf_counter()
        c.refresh(A2)
        t2 = time.perf_counter()
        t_sel += t1 - t0
        t_ref += t2 - t1
    out["selector_5pct"] = {"us_per_call": round(t_sel / n * n_heads_call * 1e6, 1),
                            "sample": f"{n} of the {n_heads_call} (sequence, KV head) caches of bs4 x {L}, "
                                      f"64 Q / 8 KV heads, cache mode after 64 appends ({t_sel:.1f} s)"}
    out["freeze"] = {"us_per_call": round(t_frz / n * 16 * 8 * 1e6, 1),
                     "sample": f"Freeze of {n} (sequence, KV head) caches of {L} positions ({t_frz:.2f} s), "
                               f"times the 128 heads of bs16 x {L} at 8 KV heads"}
    out["refresh"] = {"us_per_call": round(t_ref / n * n_heads_call * 1e6, 1),
                      "sample": f"the same {n} caches, the new set applied ({t_ref:.2f} s)"}
    N, Hq, Hkv = 8192, 32, 8
    d = synth.gen_prefill(args.seed + 8, Hq, Hkv, N)
    anchors = [pol.select_dense(d["K"][h], d["Q"][h * 4:(h + 1) * 4, N - 64:])[0] for h in range(Hkv)]
    t0 = time.perf_counter()
    qz = att.prefill_quantize(d["Q"], d["K"], d["V"], anchors)
    t_q = time.perf_counter() - t0
    rng = np.random.default_rng(args.seed)
    nb, ns = N // 64, 6
    picks = [(int(rng.integers(nb)), int(rng.integers(Hq))) for _ in range(ns)]
    t0 = time.perf_counter()
    for b, h in picks:
        att.prefill_ref(d["Q"], d["K"], d["V"], anchors, blocks=[b], heads=[h], qz=qz)
    t_b = (time.perf_counter() - t0) / ns
    out[f"prefill_{N}"] = {"us_per_call": round((t_q + t_b * nb * Hq) * 1e6, 1),
                           "sample": f"operand quantization in full ({t_q:.1f} s), then {ns} random (64-query block, "
                                     f"Q head) pairs of {nb * Hq} ({t_b:.2f} s each), extrapolated"}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU: --gpus must be 1 (the path shards by "
                                   "sequence or KV head, which no run here launches)"}))
        sys.exit(2)
    import torch
    from hybrid_precision_kv_amd import api as hq
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(3)
    dev = torch.device("cuda:0")
    if args.only_selector:
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        rows = {"selector": bench_selector(torch, hq, gen, dev),
                "selector_alg1": bench_selector_alg1(torch, hq, gen, dev)}
        print(json.dumps({"rows": rows}), flush=True)
        return
    if args.only_alg1:
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        print(json.dumps({"rows": {"selector_alg1": bench_selector_alg1(torch, hq, gen, dev)}}), flush=True)
        return
    if args.only_bits:
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        print(json.dumps({"rows": {"decode_bit_width": bench_decode_bits(torch, hq, gen, dev)}}), flush=True)
        return
    if args.only_ragged:
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        print(json.dumps({"rows": {"decode_ragged": bench_decode_ragged(torch, hq, gen, dev)}}), flush=True)
        return
    if args.only_gqa8:
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        print(json.dumps({"rows": {"decode_gqa8": bench_decode_gqa8(torch, hq, gen, dev,
                                                                     copy_cal=args.copy_calibration)}}), flush=True)
        return
    if args.only_bs1:
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        ctxs = tuple(int(x) for x in args.bs1_ctxs.split(",") if x)
        print(json.dumps({"rows": {"decode_bs1": bench_decode_bs1(torch, hq, gen, dev, ctxs=ctxs)}}), flush=True)
        return
    if args.only_freeze:
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        print(json.dumps({"rows": {"freeze": bench_freeze(torch, hq, gen, dev)}}), flush=True)
        return
    if args.only_prefill:
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        rows = {}
        for n in [int(x) for x in args.prefill_lens.split(",") if x]:
            rows[f"prefill_{n}"] = bench_prefill(torch, hq, gen, dev, n)
            rows[f"prefill_mx_{n}"] = bench_prefill(torch, hq, gen, dev, n, bulk="mxfp4")
        print(json.dumps({"rows": rows}), flush=True)
        return
    B, Hq, Hkv, L = args.batch, args.hq, args.hkv, args.ctx
    G = Hq // Hkv
    shape = hq.Shape.for_context(B, Hq, Hkv, L + 64)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    t_setup = time.perf_counter()
    layers = []
    for li in range(args.layers):
        layers.append(make_layer(torch, hq, shape, B, Hkv, G, L, gen, dev))
        torch.cuda.synchronize()
        if li == 0 or (li + 1) % 12 == 0:
            print(f"[bench] layer {li + 1}/{args.layers} ready ({time.perf_counter() - t_setup:.1f} s)",
                  file=sys.stderr, flush=True)
    nbytes = algorithmic_bytes(layers[0][0], B, Hkv, Hq)
    ws = hq.decode_workspace(shape, args.splits, dev)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    nl = len(layers)
    # context for the peak, taken before the timed region on a loaded device: the read rate a
    # plain streaming reduction reaches (torch's row sums over 4 GiB of fp32 resident in HBM,
    # 4 KB rows; bytes read / time; 50 untimed passes first.  Of the torch reductions tried,
    # row sums read fastest: a full sum reaches about 4 TB/s).  It does not replace the decode
    # warm-up: the decode's own first few hundred steps run slower however busy the device was
    probe = torch.ones(1 << 30, dtype=torch.float32, device=dev).view(1 << 20, 1024)
    for _ in range(50):
        probe.sum(dim=1)
    torch.cuda.synchronize()
    pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pe0.record()
    for _ in range(10):
        probe.sum(dim=1)
    pe1.record()
    torch.cuda.synchronize()
    read_probe = probe.numel() * 4 * 10 / (pe0.elapsed_time(pe1) * 1e-3) / 1e9
    del probe
    # device ramp (setup, untimed): from idle, and after setup, the decode reaches its steady
    # rate only after several hundred steps (the clocks' ramp, then a slower convergence of
    # the nontemporal-load build that settles after about 700 steps); the W warm-up steps
    # follow
    for i in range(args.ramp_steps):
        c, q = layers[i % nl]
        hq.decode_attn(c, q, args.splits, out, ws)
    for i in range(args.warmup):
        c, q = layers[i % nl]
        hq.decode_attn(c, q, args.splits, out, ws)
    torch.cuda.synchronize()
    # timed region: K back-to-back steps, events only at its two ends
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        c, q = layers[i % nl]
        hq.decode_attn(c, q, args.splits, out, ws)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / args.steps
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    # per-launch durations: the same steps again, HIP events (current stream) around each call
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        c, q = layers[i % nl]
        evs[i][0].record()
        hq.decode_attn(c, q, args.splits, out, ws)
        evs[i][1].record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)  # microseconds per launch
    mean_us = sum(per) / len(per)
    achieved = nbytes / (mean_us * 1e-6) / 1e9
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b2 = torch.empty_like(a)
        for _ in range(5):
            b2.copy_(a)
        torch.cuda.synchronize()
    workload = f"qwen3-8b-shape decode bs{B} ctx{L} hq{Hq} hkv{Hkv} layers{nl}"
    traffic = stored_traffic(workload)
    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ramp_steps": args.ramp_steps,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "tokens_per_s_attention_only": round(B / (nl * ms_per_step * 1e-3), 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4+bf16 (f16/bf16 MFMA, fp32 accumulate)",
        "data": "synthetic (seeded planted-anchor K/V/q, generated on device)",
        "config": {"workload": workload, "batch": B, "ctx": L, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                   "layers_resident": nl, "anchors_pct": 5, "window": W,
                   "splits": args.splits or "auto", "bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "hyq_decode_attn (split-K kernel + merge kernel, timed together)",
                     "kernel_us_mean": round(mean_us, 2),
                     "kernel_us_p50": round(per[len(per) // 2], 2), "kernel_us_p90": round(per[int(0.9 * len(per))], 2),
                     "read_probe_GBs": round(read_probe, 1),
                     "read_probe": "torch row sums over 4 GiB resident fp32 (context for the peak, not the peak)"},
        "wall_s_timed": round(wall, 3),
        "tokens_note": f"tokens_per_s_attention_only = batch / ({nl} layers x one layer's decode-attention step): "
                       "the attention share of a decode step, not an end-to-end model rate",
    }
    c0 = layers[0][0]
    cpu_bytes_per_head = 160 * c0.n_int4 + 512 * (c0.n_anchor + min(L, W)) + G * D * 6
    if not args.no_rows:
        rows = {}
        rows["decode_with_maintenance"] = bench_maintenance(torch, hq, layers[0][0], B, Hkv, G, L, gen, dev, ws,
                                                            out, args.splits)
        del layers, c0
        torch.cuda.empty_cache()
        rows["freeze"] = bench_freeze(torch, hq, gen, dev, B=B, L=L, Hq=Hq, Hkv=Hkv)
        print(f"[bench] freeze: {rows['freeze']}", file=sys.stderr, flush=True)
        rows["decode_bs1"] = bench_decode_bs1(torch, hq, gen, dev)
        print(f"[bench] bs1 sweep done", file=sys.stderr, flush=True)
        # the same kernel with every position in bf16 (k = P): what the hybrid layout saves
        allbf = bench_decode_bs1(torch, hq, gen, dev, all_bf16=True)
        allbf[f"bs{B}_{L}"] = bench_decode_bs1(torch, hq, gen, dev, ctxs=(L,), Hq=Hq, Hkv=Hkv, layers=8,
                                               B=B, all_bf16=True)[str(L)]
        for key, r in allbf.items():
            hyb = rows["decode_bs1"].get(key, {}).get("us_per_step") if not key.startswith("bs") else ms_per_step * 1e3
            if hyb:
                r["hybrid_us_per_step"] = round(hyb, 2)
                r["hybrid_speedup"] = round(r["us_per_step"] / hyb, 2)
        rows["decode_all_bf16"] = allbf
        print(f"[bench] all-bf16 sweep done", file=sys.stderr, flush=True)
        rows["decode_bit_width"] = bench_decode_bits(torch, hq, gen, dev, B=B, L=L, Hq=Hq, Hkv=Hkv)
        print(f"[bench] bit widths: {rows['decode_bit_width']}", file=sys.stderr, flush=True)
        rows["decode_gqa8"] = bench_decode_gqa8(torch, hq, gen, dev)
        print(f"[bench] gqa8: {rows['decode_gqa8']}", file=sys.stderr, flush=True)
        rows["decode_ragged"] = bench_decode_ragged(torch, hq, gen, dev, Hq=Hq, Hkv=Hkv)
        print(f"[bench] ragged batch: {rows['decode_ragged']}", file=sys.stderr, flush=True)
        for n in [int(x) for x in args.prefill_lens.split(",") if x]:
            rows[f"prefill_{n}"] = bench_prefill(torch, hq, gen, dev, n)
            print(f"[bench] prefill N={n}: {rows[f'prefill_{n}']['us_per_call']} us", file=sys.stderr, flush=True)
            rows[f"prefill_mx_{n}"] = bench_prefill(torch, hq, gen, dev, n, bulk="mxfp4")
            print(f"[bench] prefill mxfp4 N={n}: {rows[f'prefill_mx_{n}']['us_per_call']} us", file=sys.stderr,
                  flush=True)
        rows["selector"] = bench_selector(torch, hq, gen, dev)
        rows["selector_alg1"] = bench_selector_alg1(torch, hq, gen, dev)
        print(f"[bench] alg1 selector: {rows['selector_alg1']}", file=sys.stderr, flush=True)
        line["rows"] = rows
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, G, cpu_bytes_per_head)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

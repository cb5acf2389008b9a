"""Test-side reader of the documented cache layout (include/hyq.h): turns the device buffers
of a HybridKVCache into per-position arrays that can be compared with the oracle.

This is a host-side decoder of the byte layout only (no method arithmetic beyond unpacking
nibbles and reading fp16 pairs)."""
from __future__ import annotations

import numpy as np

D, W = 128, 128
KSLOT_NIBBLE = np.array([0, 4, 1, 5, 2, 6, 3, 7])
KSLOT_BYTE = np.array([0, 2, 1, 3, 4, 6, 5, 7])  # INT8 V entries (HYQ_V_BYTE_INIT)


def _tile_pos(p):
    p = np.asarray(p)
    q = (p & 15) >> 2
    e = (p & 3) + 4 * (p >> 4)
    return q, e


def read_cache(cache) -> list:
    """Per (b, h_kv): dict with int4 {pos: (kcodes[128], ksm[4,2], vcodes[128], vsm[4,2])} (the
    quantized store, codes of the shape's B_K / B_V bits),
    anchors {pos: (k bf16[128], v bf16[128])}, staged, window (same), in numpy."""
    s = cache.shape
    H = s.batch * s.n_kv_heads
    ctr = cache.counters()
    host = {n: t.cpu().numpy() for n, t in cache.buffers.items()}
    nt = s.int4_cap // 32
    bk = getattr(s, "bits", 4) or 4
    bv = getattr(s, "bits_v", 0) or bk
    CB = 4 * bk                   # bytes of one (slot, group) K chunk
    VC = 512 * bk                 # offset of the V codes in a tile record
    KSM = VC + 512 * bv           # offset of the K (scale, min)
    TB = KSM + 1024
    rec = host["int4"][: H * nt * TB].reshape(H, nt, TB)
    # K codes: [16-slot block][q4][slot in block][CB bytes]
    kc = rec[:, :, :VC].reshape(H, nt, 2, 4, 16, CB)
    kc = kc.transpose(0, 1, 2, 4, 3, 5).reshape(H, s.int4_cap, 4, CB)  # -> [slot][group][CB bytes]
    vraw = np.ascontiguousarray(rec[:, :, VC:KSM])
    if bv == 4:    # u32 [half][quad][channel & 15][r4], channel = 16*(4*half + r4) + i
        vc = vraw.view(np.uint32).reshape(H, nt, 2, 4, 16, 4)
    elif bv == 8:  # [half][quad][i][r4][8 bytes]
        vc = vraw.reshape(H, nt, 2, 4, 16, 4, 8)
    else:          # u32 [quad][i][d4]: channels 16*(2*d4 + h) + i
        vc = vraw.view(np.uint32).reshape(H, nt, 4, 16, 4)
    # (scale, min): [16-slot block][g][slot in block][2]
    ksm = np.ascontiguousarray(rec[:, :, KSM:KSM + 512]).view(np.float16).reshape(H, nt * 2, 4, 16, 2)
    vsm = np.ascontiguousarray(rec[:, :, KSM + 512:TB]).view(np.float16).reshape(H, nt * 2, 4, 16, 2)
    slot_pos = host["slot_pos"][: H * s.int4_cap * 4].view(np.int32).reshape(H, s.int4_cap)

    p32 = np.arange(32)
    q32, e32 = _tile_pos(p32)

    def bf_k(name, cap):
        # tile [16-pos block][chunk tt][quad q4][pos in block][8]
        t = host[name][: H * cap * D * 2].view(np.uint16).reshape(H, cap // 32, 2, 4, 4, 16, 8)
        return t.transpose(0, 1, 2, 5, 4, 3, 6).reshape(H, cap, D)

    def bf_v(name, cap):
        # tile [channel / 16][quad][channel & 15][k-slot]
        t = host[name][: H * cap * D * 2].view(np.uint16).reshape(H, cap // 32, 8, 4, 16, 8)
        out = np.empty((H, cap // 32, 32, D), np.uint16)
        for c in range(D):
            out[:, :, :, c] = t[:, :, c >> 4, q32, c & 15, e32]
        return out.reshape(H, cap, D)

    a_k, a_v = bf_k("a_k", s.anchor_cap), bf_v("a_v", s.anchor_cap)
    s_k, s_v = bf_k("s_k", s.staging_cap), bf_v("s_v", s.staging_cap)
    w_k, w_v = bf_k("w_k", W), bf_v("w_v", W)
    a_pos = host["a_pos"][: H * s.anchor_cap * 4].view(np.int32).reshape(H, s.anchor_cap)

    nsl = s.int4_cap
    sl = np.arange(nsl)
    q, e = _tile_pos(sl & 31)
    vcodes = np.empty((H, nsl, D), np.uint8)
    kcodes = np.empty((H, nsl, D), np.uint8)
    if bv == 4:
        shift = 4 * KSLOT_NIBBLE[e]
        for c in range(D):
            i, r = c & 15, c >> 4
            words = vc[:, sl >> 5, r >> 2, q, i, r & 3]
            vcodes[:, :, c] = (words >> shift) & 0xF
    elif bv == 8:
        byte = KSLOT_BYTE[e]
        for c in range(D):
            i, r = c & 15, c >> 4
            vcodes[:, :, c] = vc[:, sl >> 5, r >> 2, q, i, r & 3, byte]
    else:
        for c in range(D):
            i, r = c & 15, c >> 4
            words = vc[:, sl >> 5, q, i, r >> 1]
            vcodes[:, :, c] = (words >> (2 * (e >> 1) + 16 * (e & 1) + 8 * (r & 1))) & 0x3
    # K: channel 32 g + j at bits bk * j of the group's chunk (little-endian)
    kbits = np.unpackbits(kc, axis=-1, bitorder="little").reshape(H, s.int4_cap, 4, 32, bk)
    kcodes[:] = (kbits.astype(np.uint32) << np.arange(bk, dtype=np.uint32)).sum(-1).reshape(H, s.int4_cap, D)
    ksm_s = ksm.transpose(0, 1, 3, 2, 4)[:, sl >> 4, sl & 15]  # [H][slot][g][2]
    vsm_s = vsm.transpose(0, 1, 3, 2, 4)[:, sl >> 4, sl & 15]

    L, n4, na, ns = ctr["len"], ctr["n_int4"], ctr["n_anchor"], ctr["n_staged"]
    res = []
    for h in range(H):
        d = dict(int4={}, anchors={}, staged={}, window={})
        for t in range(n4):
            d["int4"][int(slot_pos[h, t])] = (kcodes[h, t], ksm_s[h, t], vcodes[h, t], vsm_s[h, t])
        for t in range(na):
            d["anchors"][int(a_pos[h, t])] = (a_k[h, t], a_v[h, t])
        for t in range(ns):
            d["staged"][L - W - ns + t] = (s_k[h, t], s_v[h, t])
        for p in range(max(0, L - W), L):
            d["window"][p] = (w_k[h, p % W], w_v[h, p % W])
        d["a_pos"] = a_pos[h, :na].copy()
        res.append(d)
    return res


# ----------------------------------------------------------------------------- prefill workspace

def _r256(x: int) -> int:
    return (x + 255) // 256 * 256


def prefill_ws_offsets(Hq: int, Hkv: int, N: int, anchor_cap: int) -> dict:
    """Section offsets of the prefill workspace, in the order the header lists them."""
    Np = (N + 127) // 128 * 128
    Ac = (anchor_cap + 63) // 64 * 64
    sizes = [("q8", Hq * Np * D), ("sq", Hq * (Np // 64) * 4), ("k8", Hkv * Np * D),
             ("sk", Hkv * (Np // 64) * 4), ("v8", Hkv * Np * D), ("sv", Hkv * D * 4),
             ("vmax", Hkv * (Np // 64) * D * 4), ("abits", Hkv * (Np // 32) * 4),
             ("vt16", Hkv * Np * D * 2), ("ka16", Hkv * Ac * D * 2), ("va16", Hkv * Ac * D * 2)]
    off, out = 0, {"Np": Np}
    for name, n in sizes:
        out[name] = off
        off += _r256(n)
    out["total"] = off
    return out


def _int8_natural_index() -> np.ndarray:
    """perm[c] = byte of channel c in an operand-order INT8 row: channel 32 (2 s + t) + 8 j + e
    sits at byte 64 s + 16 j + 8 t + e."""
    perm = np.empty(D, np.int64)
    for s in range(2):
        for t in range(2):
            for j in range(4):
                for e in range(8):
                    perm[32 * (2 * s + t) + 8 * j + e] = 64 * s + 16 * j + 8 * t + e
    return perm


def read_prefill_ws(ws: np.ndarray, Hq: int, Hkv: int, N: int, anchor_cap: int) -> dict:
    """Decode the prefill workspace (uint8 numpy) into natural-order arrays:
    q8 int8 [Hq][Np][128], sq f32 [Hq][Np/64], k8 int8 [Hkv][Np][128], sk, v8 uint8 codes
    [Hkv][Np][128], sv f32 [Hkv][128], abits uint32 [Hkv][Np/32]."""
    o = prefill_ws_offsets(Hq, Hkv, N, anchor_cap)
    Np = o["Np"]

    def sec(name, dtype, count):
        start = o[name]
        return ws[start:start + count * np.dtype(dtype).itemsize].view(dtype)

    perm = _int8_natural_index()
    q8 = sec("q8", np.int8, Hq * Np * D).reshape(Hq, Np, D)[:, :, perm]
    # K codes: per 64-key tile, [16-byte chunk 8][key 64][16] of the operand-order rows
    kraw = sec("k8", np.int8, Hkv * Np * D).reshape(Hkv, Np // 64, 8, 64, 16)
    k8 = kraw.transpose(0, 1, 3, 2, 4).reshape(Hkv, Np, D)[:, :, perm]
    # V codes: per 32-key block, [half h][channel][16]; byte b is key 16 (b >> 3) + 8 h + (b & 7)
    raw = sec("v8", np.uint8, Hkv * Np * D).reshape(Hkv, Np // 32, 2, D, 16)
    v8 = np.empty((Hkv, Np, D), np.uint8)
    for h in range(2):
        for b in range(16):
            kk = 16 * (b >> 3) + 8 * h + (b & 7)
            v8[:, kk::32, :] = raw[:, :, h, :, b]
    return dict(Np=Np, q8=q8, k8=k8, v8=v8,
                sq=sec("sq", np.float32, Hq * (Np // 64)).reshape(Hq, Np // 64),
                sk=sec("sk", np.float32, Hkv * (Np // 64)).reshape(Hkv, Np // 64),
                sv=sec("sv", np.float32, Hkv * D).reshape(Hkv, D),
                abits=sec("abits", np.uint32, Hkv * (Np // 32)).reshape(Hkv, Np // 32))


def _nibbles(b: np.ndarray) -> np.ndarray:
    """[..., n] bytes -> [..., 2n] 4-bit codes, the low nibble first."""
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def read_prefill_mx(ws: np.ndarray, Hq: int, Hkv: int, N: int, anchor_cap: int) -> dict:
    """Decode the MXFP4 operands of hyq_prefill_attn_mx from its workspace (uint8 numpy):
    q4 uint8 E2M1 codes [Hq][Np][128], qe int [Hq][Np][4] block exponents (stored e + 127),
    k4 [Hkv][Np][128], ke [Hkv][Np][4]."""
    o = prefill_ws_offsets(Hq, Hkv, N, anchor_cap)
    Np = o["Np"]
    qraw = ws[o["q8"]:o["q8"] + Hq * Np * D].reshape(Hq, Np, D)
    q4 = _nibbles(qraw[:, :, :64])
    qe = qraw[:, :, 64:68].astype(np.int64) - 127
    # K tile of 64 keys: codes [block j][key r][16 B], then scale byte of (j, r) at
    # 4096 + (16 j + (r & 15)) * 4 + (r >> 4)
    kraw = ws[o["k8"]:o["k8"] + Hkv * Np * D].reshape(Hkv, Np // 64, 8192)
    codes = kraw[:, :, :4096].reshape(Hkv, Np // 64, 4, 64, 16).transpose(0, 1, 3, 2, 4)
    k4 = _nibbles(codes.reshape(Hkv, Np // 64, 64, 64)).reshape(Hkv, Np, D)
    sc = kraw[:, :, 4096:4352].reshape(Hkv, Np // 64, 4, 16, 4)  # [j][r & 15][r >> 4]
    ke = sc.transpose(0, 1, 4, 3, 2).reshape(Hkv, Np, 4).astype(np.int64) - 127
    return dict(Np=Np, q4=q4, qe=qe, k4=k4, ke=ke)

// Refresh of the hybrid cache after a new vertical-line set.
//
// The selector runs every 64 decode tokens (techwalker.com article on HyQuant, design section);
// the HyQuant paper ("HyQuant: Hybrid-Precision Quantization for LLM Attention") gives the set
// (§4.1 Eq. 5) and the four storage segments (Alg. 3, Alg. 4) but not how a new set is applied.
// Reading taken (stated in the design notes):
//   * anchors in the new set keep their bf16 values;
//   * staged positions in the new set become anchors with their original bf16 values;
//   * INT4 positions in the new set become anchors holding bf16(dequantized value) -- their
//     original values were freed at Freeze -- and leave the INT4 store;
//   * anchors and staged positions not in the new set are quantized into the INT4 store
//     (same quantizer as Freeze);
//   * staging is emptied.
// INT4 slots are unordered: the slots freed by promotions are refilled first (new entries,
// then -- if the store shrinks -- slots moved down from its tail), so the store stays dense.
//
// Four launches:
//   plan   (one workgroup per head): bitmaps of the new set and of the old anchors with
//          per-word prefix counts (so "which old anchor / which new index is position p" is
//          an O(1) rank), the promoted slots, and the move list (targets, kinds, sources);
//   gather (grid over heads x new anchors): the new anchor rows, bf16, into a temp store;
//   move   (grid over heads x moves): quantize demoted rows into slots / move tail slots;
//   store  (grid over heads x anchor rows): anchor store <- temp, positions.
// Writes of single V codes go through dword atomics (8 slots share each V-code dword).
//
// Built with -ffp-contract=off (the quantizer's operation order is part of its contract).
#include <algorithm>

#include "hyq_common.h"
#include "hyq_launch.h"

namespace hyq {

namespace {

constexpr int PT = 1024;  // threads of the plan workgroup

// block-wide exclusive scan of one int per thread; returns the exclusive prefix, total in *tot
__device__ inline int block_scan(int v, int* sh, int* tot) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < PT; off <<= 1) {
    const int add = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int incl = sh[tid];
  *tot = sh[PT - 1];
  __syncthreads();
  return incl - v;
}

// per-head scratch (4-byte words, then the two bf16 row stores)
struct Scratch {
  uint32_t* inset;   // [inset_words] new-set bitmap over positions
  uint32_t* oldanc;  // [inset_words] old-anchor bitmap over positions
  int32_t* pre_new;  // [inset_words] set bits before word w (new set)
  int32_t* pre_old;  // [inset_words] set bits before word w (old anchors)
  uint32_t* del;     // [del_words] promoted (deleted) INT4 slots
  int32_t* slot_of;  // [anchor_cap] INT4 slot of new anchor i (when it is promoted), else -1
  int32_t* mv_dst;   // [max_moves]
  int32_t* mv_kind;  // [max_moves] 0 old anchor, 1 staged, 2 INT4 slot
  int32_t* mv_src;   // [max_moves]
  int32_t* cnt;      // [4]: moves to execute, n_new, moves listed, promotions
  uint16_t* tk;      // [anchor_cap][128] new anchors K
  uint16_t* tv;      // [anchor_cap][128] new anchors V
};

__device__ inline Scratch scratch(const RefreshParams& p, int hb) {
  Scratch s;
  uint32_t* base = (uint32_t*)(p.ws + hb * p.ws_per_head);
  const int iw = p.inset_words;
  s.inset = base;
  s.oldanc = s.inset + iw;
  s.pre_new = (int32_t*)(s.oldanc + iw);
  s.pre_old = s.pre_new + iw;
  s.del = (uint32_t*)(s.pre_old + iw);
  s.slot_of = (int32_t*)(s.del + p.del_words);
  s.mv_dst = s.slot_of + p.anchor_cap;
  s.mv_kind = s.mv_dst + p.max_moves;
  s.mv_src = s.mv_kind + p.max_moves;
  s.cnt = s.mv_src + p.max_moves;
  s.tk = (uint16_t*)(s.cnt + 4);
  s.tv = s.tk + (size_t)p.anchor_cap * D;
  return s;
}

__device__ inline bool bit_at(const uint32_t* bm, int pos) { return (bm[pos >> 5] >> (pos & 31)) & 1u; }
__device__ inline int rank_at(const uint32_t* bm, const int32_t* pre, int pos) {
  return pre[pos >> 5] + __popc(bm[pos >> 5] & ((1u << (pos & 31)) - 1u));
}

// ------------------------------------------------------------------ plan
__global__ __launch_bounds__(PT) void refresh_plan_kernel(RefreshParams p) {
  __shared__ int sh[PT];
  const int hb = blockIdx.x, tid = threadIdx.x;
  const int P = p.len - WIN;
  const int ps0 = P - p.n_staged;  // first staged position
  const int k_old = p.n_anchor_old, k_new = p.k, n_old = p.n_int4_old, ns = p.n_staged;
  const int32_t* slot_pos = p.slot_pos + hb * (size_t)p.int4_cap;
  const int32_t* a_pos = p.a_pos + hb * (size_t)p.anchor_cap;
  const int32_t* idx = p.idx + hb * (size_t)k_new;
  const Scratch s = scratch(p, hb);
  const int iw = p.inset_words;

  // ---- bitmaps of the new set and of the old anchors, cleared deletion bitmap
  for (int i = tid; i < iw; i += PT) { s.inset[i] = 0u; s.oldanc[i] = 0u; }
  for (int i = tid; i < p.del_words; i += PT) s.del[i] = 0u;
  for (int i = tid; i < k_new && i < p.anchor_cap; i += PT) s.slot_of[i] = -1;
  __syncthreads();
  for (int i = tid; i < k_new; i += PT) {
    const int pos = idx[i];
    if (pos >= 0 && pos < P) atomicOr(&s.inset[pos >> 5], 1u << (pos & 31));
  }
  for (int j = tid; j < k_old; j += PT) {
    const int pos = a_pos[j];
    if (pos >= 0 && pos < P) atomicOr(&s.oldanc[pos >> 5], 1u << (pos & 31));
  }
  __syncthreads();
  // ---- per-word prefix counts (each thread scans a contiguous run of words)
  {
    const int per = (iw + PT - 1) / PT, w0 = min(iw, tid * per), w1 = min(iw, w0 + per);
    int cn = 0, co = 0;
    for (int w = w0; w < w1; ++w) { cn += __popc(s.inset[w]); co += __popc(s.oldanc[w]); }
    int tot;
    int on = block_scan(cn, sh, &tot);
    int oo = block_scan(co, sh, &tot);
    for (int w = w0; w < w1; ++w) {
      s.pre_new[w] = on;
      s.pre_old[w] = oo;
      on += __popc(s.inset[w]);
      oo += __popc(s.oldanc[w]);
    }
  }
  __syncthreads();
  auto in_set = [&](int pos) -> bool { return pos >= 0 && pos < P && bit_at(s.inset, pos); };

  // ---- INT4 slots whose position is in the set are promoted: delete, record the slot
  int npro = 0;
  for (int t = tid; t < n_old; t += PT) {
    const int pos = slot_pos[t];
    if (in_set(pos)) {
      atomicOr(&s.del[t >> 5], 1u << (t & 31));
      const int i = rank_at(s.inset, s.pre_new, pos);
      if (i < k_new && i < p.anchor_cap) s.slot_of[i] = t;
      ++npro;
    }
  }
  __syncthreads();

  // ---- new INT4 entries E (old anchors, then staged tokens, not in the set, ascending),
  // holes (deleted slots), and the move list targets <- sources
  int tot;
  int ca = 0, cs = 0;
  const int per_a = (k_old + PT - 1) / PT, per_s = (ns + PT - 1) / PT;
  for (int j = tid * per_a; j < min(k_old, (tid + 1) * per_a); ++j) ca += !in_set(a_pos[j]);
  for (int j = tid * per_s; j < min(ns, (tid + 1) * per_s); ++j) cs += !in_set(ps0 + j);
  const int off_a = block_scan(ca, sh, &tot);
  const int e_a = tot;
  const int off_s = block_scan(cs, sh, &tot);
  const int e = e_a + tot;
  int pdel_mine = 0;
  for (int w = tid; w < p.del_words; w += PT) pdel_mine += __popc(s.del[w]);
  block_scan(pdel_mine, sh, &tot);
  const int p_del = tot;
  const int n_new = n_old - p_del + e;
  // sources: E entries (indices 0..e-1 of the move list), then alive tail slots [n_new, n_old)
  {
    int o = off_a;
    for (int j = tid * per_a; j < min(k_old, (tid + 1) * per_a); ++j)
      if (!in_set(a_pos[j])) { if (o < p.max_moves) { s.mv_kind[o] = 0; s.mv_src[o] = j; } ++o; }
    o = e_a + off_s;
    for (int j = tid * per_s; j < min(ns, (tid + 1) * per_s); ++j)
      if (!in_set(ps0 + j)) { if (o < p.max_moves) { s.mv_kind[o] = 1; s.mv_src[o] = j; } ++o; }
  }
  // alive tail slots, ascending (words are scanned in order, 32 slots per word)
  const int tail_lo = n_new < n_old ? n_new : n_old;
  const int w_lo = tail_lo >> 5, w_hi = (n_old + 31) >> 5;
  const int per_w = (w_hi - w_lo + PT - 1) / PT;
  int ct = 0;
  for (int w = w_lo + tid * per_w; w < min(w_hi, w_lo + (tid + 1) * per_w); ++w)
    for (int bit = 0; bit < 32; ++bit) {
      const int t = w * 32 + bit;
      if (t >= tail_lo && t < n_old && !((s.del[w] >> bit) & 1u)) ++ct;
    }
  const int off_t = block_scan(ct, sh, &tot);
  {
    int o = e + off_t;
    for (int w = w_lo + tid * per_w; w < min(w_hi, w_lo + (tid + 1) * per_w); ++w)
      for (int bit = 0; bit < 32; ++bit) {
        const int t = w * 32 + bit;
        if (t >= tail_lo && t < n_old && !((s.del[w] >> bit) & 1u)) {
          if (o < p.max_moves) { s.mv_kind[o] = 2; s.mv_src[o] = t; }
          ++o;
        }
      }
  }
  const int n_moves = e + tot;
  // targets: deleted slots below min(n_new, n_old), ascending, then fresh slots [n_old, n_new)
  const int hw = (tail_lo + 31) >> 5;
  const int per_h = (hw + PT - 1) / PT;
  int ch = 0;
  for (int w = tid * per_h; w < min(hw, (tid + 1) * per_h); ++w)
    for (int bit = 0; bit < 32; ++bit) {
      const int t = w * 32 + bit;
      if (t < tail_lo && ((s.del[w] >> bit) & 1u)) ++ch;
    }
  const int off_h = block_scan(ch, sh, &tot);
  const int n_holes = tot;
  {
    int o = off_h;
    for (int w = tid * per_h; w < min(hw, (tid + 1) * per_h); ++w)
      for (int bit = 0; bit < 32; ++bit) {
        const int t = w * 32 + bit;
        if (t < tail_lo && ((s.del[w] >> bit) & 1u)) { if (o < p.max_moves) s.mv_dst[o] = t; ++o; }
      }
  }
  for (int t = n_old + tid; t < n_new; t += PT)
    if (n_holes + (t - n_old) < p.max_moves) s.mv_dst[n_holes + (t - n_old)] = t;
  block_scan(npro, sh, &tot);
  const int n_promo = tot;
  if (tid == 0) {
    // n_new == len - W - k for a valid set (distinct, ascending, inside [0, len - W)); the
    // bound keeps a malformed set from writing outside the store
    s.cnt[0] = min(n_moves, min(p.max_moves, n_holes + max(0, n_new - n_old)));
    s.cnt[1] = n_new;
    s.cnt[2] = n_moves;
    s.cnt[3] = n_promo;
    if (p.status) p.status[hb] = (n_new == P - k_new && n_moves >= 0 && p_del >= 0) ? 0 : 1;
  }
}

// ------------------------------------------------------------------ gather: one wave per new anchor
template <int BK, int BV>
__global__ __launch_bounds__(256) void refresh_gather_kernel(RefreshParams p) {
  const int hb = blockIdx.y, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int k_new = p.k;
  if (i >= k_new || i >= p.anchor_cap) return;
  const int P = p.len - WIN;
  const int ps0 = P - p.n_staged;
  const Scratch s = scratch(p, hb);
  const size_t aslab = (size_t)p.anchor_cap * D, sslab = (size_t)p.staging_cap * D;
  const int pos = p.idx[hb * (size_t)k_new + i];
  uint16_t* tk = s.tk + (size_t)i * D;
  uint16_t* tv = s.tv + (size_t)i * D;
  if (pos < 0 || pos >= P) return;  // malformed set: nothing to gather (status reports it)
  if (pos >= ps0 || bit_at(s.oldanc, pos)) {
    // bf16 already: a staged token or an old anchor
    const uint16_t *sk, *sv;
    int si, cap;
    if (pos >= ps0) { sk = p.s_k + hb * sslab; sv = p.s_v + hb * sslab; si = pos - ps0; cap = p.staging_cap; }
    else { sk = p.a_k + hb * aslab; sv = p.a_v + hb * aslab; si = rank_at(s.oldanc, s.pre_old, pos); cap = p.anchor_cap; }
    if (si >= cap) return;
    for (int c = lane; c < D; c += 64) {
      tk[c] = sk[kbf_index(si, c)];
      tv[c] = sv[vbf_index(si, c)];
    }
    return;
  }
  // a quantized position: dequantize its slot
  const int t = s.slot_of[i];
  if (t < 0 || t >= p.int4_cap) return;
  const uint8_t* slab = p.int4 + hb * (size_t)p.int4_cap * QL<BK, BV>::SLOT;
  for (int c = lane; c < D; c += 64) {
    const int g = c >> 5;
    // K code: channel c & 31 of the chunk at bits BK (c & 31), read from its byte
    const int kbit = BK * (c & 31);
    const uint32_t kc = ((uint32_t)slab[kcode_chunk_b<BK, BV>(t, g) + (kbit >> 3)] >> (kbit & 7)) & ((1u << BK) - 1u);
    size_t voff;
    int vsh;
    vcode_loc<BK, BV>(t, c, voff, vsh);
    const uint32_t vc = (*(const uint32_t*)(slab + voff) >> vsh) & ((1u << BV) - 1u);
    const uint32_t ksm = *(const uint32_t*)(slab + ksm_byte_b<BK, BV>(t, g));
    const uint32_t vsm = *(const uint32_t*)(slab + vsm_byte_b<BK, BV>(t, g));
    // dequantized value = scale * code + min in fp32 (exact product, one rounding), then bf16
    const float kx = __half2float(__ushort_as_half((unsigned short)(ksm & 0xffff))) * (float)kc +
                     __half2float(__ushort_as_half((unsigned short)(ksm >> 16)));
    const float vx = __half2float(__ushort_as_half((unsigned short)(vsm & 0xffff))) * (float)vc +
                     __half2float(__ushort_as_half((unsigned short)(vsm >> 16)));
    tk[c] = f32_to_bf16_bits(kx);
    tv[c] = f32_to_bf16_bits(vx);
  }
}

// ------------------------------------------------------------------ move: one wave per move
// The plan's move count is known only on the device, so a fixed grid of MOVE_BLOCKS workgroups
// per head walks the list (wave w takes moves w, w + waves, ...).
//
// Demoting a bf16 row uses the whole wave: lane = 32 kv + 8 g + sub holds channels
// 32 g + 4 sub + e (e < 4) of K (kv = 0) or V (kv = 1); the group's min and max come from a
// reduction over its 8 lanes, and every code follows the group quantizer's formula.  A V code
// is one nibble of a dword shared by 8 slots: each slot is written by exactly one move, so the
// nibble is replaced with one atomic XOR of (old ^ new), which commutes with the other slots'
// (and is skipped when the nibble already holds the code: the atomics, not the read, bound
// this kernel).  The next move's list entry is loaded while the current move runs.
constexpr int MOVE_BLOCKS = 16;

template <int BK, int BV>
__device__ inline void put_vcode(uint8_t* slab, int slot, int c, uint32_t code) {
  size_t off;
  int sh;
  vcode_loc<BK, BV>(slot, c, off, sh);
  unsigned* dw = (unsigned*)(slab + off);
  const uint32_t delta = (((*dw >> sh) & ((1u << BV) - 1u)) ^ code) << sh;
  if (delta) atomicXor(dw, delta);
}

__device__ inline float group8_min(float v) {
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) v = fminf(v, shfl_xor_f(v, o));
  return v;
}
__device__ inline float group8_max(float v) {
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) v = fmaxf(v, shfl_xor_f(v, o));
  return v;
}

template <int BK, int BV>
__global__ __launch_bounds__(256) void refresh_move_kernel(RefreshParams p) {
  typedef QL<BK, BV> L;
  const int hb = blockIdx.y, lane = threadIdx.x & 63;
  const Scratch s = scratch(p, hb);
  const int n = min(s.cnt[0], p.max_moves), waves = gridDim.x * 4;
  const int P = p.len - WIN;
  const int ps0 = P - p.n_staged;
  uint8_t* slab = p.int4 + hb * (size_t)p.int4_cap * L::SLOT;
  int32_t* slot_pos = p.slot_pos + hb * (size_t)p.int4_cap;
  const size_t aslab = (size_t)p.anchor_cap * D, sslab = (size_t)p.staging_cap * D;
  const int kv = lane >> 5, g = (lane >> 3) & 3, sub = lane & 7;
  int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  int ndst = 0, nkind = 0, nsrc = 0;
  if (t < n) { ndst = s.mv_dst[t]; nkind = s.mv_kind[t]; nsrc = s.mv_src[t]; }
  for (; t < n; t += waves) {
    const int dst = ndst, kind = nkind, src = nsrc;
    if (t + waves < n) { ndst = s.mv_dst[t + waves]; nkind = s.mv_kind[t + waves]; nsrc = s.mv_src[t + waves]; }
    const int src_cap = kind == 0 ? p.anchor_cap : kind == 1 ? p.staging_cap : p.int4_cap;
    if (dst < 0 || dst >= p.int4_cap || src < 0 || src >= src_cap) continue;
    if (kind <= 1) {
      // quantize a bf16 row (old anchor or staged token) into slot dst
      const uint16_t* sk = kind == 0 ? p.a_k + hb * aslab : p.s_k + hb * sslab;
      const uint16_t* sv = kind == 0 ? p.a_v + hb * aslab : p.s_v + hb * sslab;
      const int c0 = 32 * g + 4 * sub;
      float x[4];
      if (kv == 0) {
        const uint2 raw = *(const uint2*)(sk + kbf_index(src, c0));  // channels c0 .. c0+3
        x[0] = bf16_bits_to_f32((uint16_t)raw.x);
        x[1] = bf16_bits_to_f32((uint16_t)(raw.x >> 16));
        x[2] = bf16_bits_to_f32((uint16_t)raw.y);
        x[3] = bf16_bits_to_f32((uint16_t)(raw.y >> 16));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = bf16_bits_to_f32(sv[vbf_index(src, c0 + e)]);
      }
      const float mn = group8_min(fminf(fminf(x[0], x[1]), fminf(x[2], x[3])));
      const float mx = group8_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
      // the group quantizer's scale, minimum and codes (same operations, same order)
      const float LEVELS = kv ? (float)((1 << BV) - 1) : (float)((1 << BK) - 1);
      const __half s16 = __float2half_rn(__fdiv_rn(__fsub_rn(mx, mn), LEVELS));
      const __half m16 = __float2half_rn(mn);
      const float sf = __half2float(s16), mf = __half2float(m16);
      uint32_t code[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float cq = 0.0f;
        if (sf != 0.0f) {
          cq = rintf(__fdiv_rn(__fsub_rn(x[e], mf), sf));
          cq = fminf(fmaxf(cq, 0.0f), LEVELS);
        }
        code[e] = (uint32_t)cq;
      }
      const uint32_t smw = (uint32_t)__half_as_ushort(s16) | ((uint32_t)__half_as_ushort(m16) << 16);
      if (kv == 0) {
        if constexpr (BK == 4) {
          // nibbles 4 sub + e of the group's 32; dword sub / 2 holds lanes sub & ~1 (low) and | 1
          const uint32_t half16 = code[0] | (code[1] << 4) | (code[2] << 8) | (code[3] << 12);
          const uint32_t other = (uint32_t)__float_as_int(shfl_xor_f(__int_as_float((int)half16), 1));
          if ((sub & 1) == 0) *(uint32_t*)(slab + kcode_chunk_b<BK, BV>(dst, g) + 4 * (sub >> 1)) = half16 | (other << 16);
        } else if constexpr (BK == 8) {
          // bytes 4 sub + e of the group's 32: one dword per lane
          *(uint32_t*)(slab + kcode_chunk_b<BK, BV>(dst, g) + 4 * sub) =
              code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
        } else {
          // 2-bit codes 4 sub + e: byte sub & 3 of dword sub / 4, OR-ed over the dword's 4 lanes
          uint32_t w = (code[0] | (code[1] << 2) | (code[2] << 4) | (code[3] << 6)) << (8 * (sub & 3));
          w |= (uint32_t)__float_as_int(shfl_xor_f(__int_as_float((int)w), 1));
          w |= (uint32_t)__float_as_int(shfl_xor_f(__int_as_float((int)w), 2));
          if ((sub & 3) == 0) *(uint32_t*)(slab + kcode_chunk_b<BK, BV>(dst, g) + 4 * (sub >> 2)) = w;
        }
        if (sub == 0) *(uint32_t*)(slab + ksm_byte_b<BK, BV>(dst, g)) = smw;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) put_vcode<BK, BV>(slab, dst, c0 + e, code[e]);
        if (sub == 0) *(uint32_t*)(slab + vsm_byte_b<BK, BV>(dst, g)) = smw;
      }
      if (lane == 0) slot_pos[dst] = kind == 0 ? p.a_pos[hb * (size_t)p.anchor_cap + src] : ps0 + src;
    } else {
      // move a quantized slot: codes, (scale, min), position
      constexpr int KDW = L::CB / 4;  // dwords per (slot, group) K chunk: BK
      if (lane < 4 * KDW) {  // K code chunks as dwords
        const int q4 = lane / KDW, d = lane % KDW;
        *(uint32_t*)(slab + kcode_chunk_b<BK, BV>(dst, q4) + 4 * d) =
            *(const uint32_t*)(slab + kcode_chunk_b<BK, BV>(src, q4) + 4 * d);
      } else if (lane < 4 * KDW + 4) {
        const int q4 = lane - 4 * KDW;
        *(uint32_t*)(slab + ksm_byte_b<BK, BV>(dst, q4)) = *(const uint32_t*)(slab + ksm_byte_b<BK, BV>(src, q4));
        *(uint32_t*)(slab + vsm_byte_b<BK, BV>(dst, q4)) = *(const uint32_t*)(slab + vsm_byte_b<BK, BV>(src, q4));
      }
      for (int c = lane; c < D; c += 64) {
        size_t off;
        int shs;
        vcode_loc<BK, BV>(src, c, off, shs);
        put_vcode<BK, BV>(slab, dst, c, (*(const uint32_t*)(slab + off) >> shs) & ((1u << BV) - 1u));
      }
      if (lane == 0) slot_pos[dst] = slot_pos[src];
    }
  }
}

// ------------------------------------------------------------------ store: one wave per anchor row
// anchor store <- temp (tile layouts), positions, zeroed tail of the last tile
__global__ __launch_bounds__(256) void refresh_store_kernel(RefreshParams p) {
  const int hb = blockIdx.y, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int k_new = p.k;
  const int a_end = min((k_new + 31) & ~31, p.anchor_cap);
  if (i >= a_end) return;
  const Scratch s = scratch(p, hb);
  const size_t aslab = (size_t)p.anchor_cap * D;
  uint16_t* a_k = p.a_k + hb * aslab;
  uint16_t* a_v = p.a_v + hb * aslab;
  for (int c = lane; c < D; c += 64) {
    a_k[kbf_index(i, c)] = i < k_new ? s.tk[(size_t)i * D + c] : (uint16_t)0;
    a_v[vbf_index(i, c)] = i < k_new ? s.tv[(size_t)i * D + c] : (uint16_t)0;
  }
  if (lane == 0) p.a_pos[hb * (size_t)p.anchor_cap + i] = i < k_new ? p.idx[hb * (size_t)k_new + i] : -1;
}

}  // namespace

size_t refresh_scratch_bytes(int inset_words, int del_words, int anchor_cap, int max_moves) {
  return (size_t)4 * (4 * (size_t)inset_words + del_words + anchor_cap + 3 * (size_t)max_moves + 4) +
         (size_t)2 * anchor_cap * D * 2;
}

hipError_t launch_refresh(const RefreshParams& p, hipStream_t stream) {
  const int H = p.B * p.Hkv;
  hipLaunchKernelGGL(refresh_plan_kernel, dim3(H), dim3(PT), 0, stream, p);
  const int ka = min(p.k, p.anchor_cap);
  const dim3 mgrid(std::max(1, std::min((p.max_moves + 3) / 4, MOVE_BLOCKS)), H);
  hipError_t e = with_widths(p.bits, p.bits_v, [&](auto BK, auto BV) {
    constexpr int K = decltype(BK)::value, V = decltype(BV)::value;
    if (ka > 0) hipLaunchKernelGGL((refresh_gather_kernel<K, V>), dim3((ka + 3) / 4, H), dim3(256), 0, stream, p);
    hipLaunchKernelGGL((refresh_move_kernel<K, V>), mgrid, dim3(256), 0, stream, p);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  const int a_end = min((p.k + 31) & ~31, p.anchor_cap);
  if (a_end > 0) hipLaunchKernelGGL(refresh_store_kernel, dim3((a_end + 3) / 4, H), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hyq

// Refresh of the hybrid cache after a new vertical-line set.
//
// The selector runs every 64 decode tokens (techwalker.com article on HyQuant, design section);
// the HyQuant paper ("HyQuant: Hybrid-Precision Quantization for LLM Attention") gives the set
// (§4.1 Eq. 5) and the four storage segments (Alg. 3, Alg. 4) but not how a new set is applied.
// Reading taken:
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
//          an O(1) rank), the promoted slots, each new anchor's source, and the move list
//          (targets, kinds, sources);
//   gather (grid over heads x new anchors): the new anchor rows, bf16, into a temp store;
//   move   (grid over heads x chunks of the move list): quantize demoted rows into slots / move
//          tail slots, each destination tile written by one wave;
//   store  (grid over heads x anchor tiles): anchor store <- temp, positions.
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
  int32_t* src_of;   // [anchor_cap] source of new anchor i: kind << 29 | index (SRC_* kinds)
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
  s.src_of = (int32_t*)(s.del + p.del_words);
  s.mv_dst = s.src_of + p.anchor_cap;
  s.mv_kind = s.mv_dst + p.max_moves;
  s.mv_src = s.mv_kind + p.max_moves;
  s.cnt = s.mv_src + p.max_moves;
  s.tk = (uint16_t*)(s.cnt + 4);
  s.tv = s.tk + (size_t)p.anchor_cap * D;
  return s;
}

// where new anchor i's bf16 row comes from: an old anchor (its rank), a staged token (its
// staging index), a promoted quantized slot (dequantized), or nowhere (a malformed set)
constexpr int SRC_ANCHOR = 0, SRC_STAGED = 1, SRC_SLOT = 2, SRC_NONE = 3;
constexpr int SRC_SHIFT = 29;
__device__ inline int32_t src_code(int kind, int index) { return (kind << SRC_SHIFT) | index; }

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
  for (int i = tid; i < k_new && i < p.anchor_cap; i += PT) s.src_of[i] = src_code(SRC_NONE, 0);
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

  // ---- INT4 slots whose position is in the set are promoted: delete, record the slot.  Eight
  // slots per thread per pass (their loads in flight together); the 64 slots of a wave at one
  // step are consecutive, so each deletion word comes whole from one ballot.
  int npro = 0;
  constexpr int UB = 8;
  const int lane = tid & 63;
  for (int t0 = tid; t0 < n_old; t0 += PT * UB) {
    int pos[UB];
    uint32_t w[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) pos[u] = t0 + u * PT < n_old ? slot_pos[t0 + u * PT] : -1;
#pragma unroll
    for (int u = 0; u < UB; ++u) w[u] = pos[u] >= 0 && pos[u] < P ? s.inset[pos[u] >> 5] : 0u;
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int t = t0 + u * PT;
      const bool hit = (w[u] >> (pos[u] & 31)) & 1u;
      const uint64_t m = __ballot(hit);
      if (t < n_old && (lane & 31) == 0) s.del[t >> 5] = (uint32_t)(m >> (lane & 32));
      if (hit) {
        const int i = s.pre_new[pos[u] >> 5] + __popc(w[u] & ((1u << (pos[u] & 31)) - 1u));
        if (i < k_new && i < p.anchor_cap) s.src_of[i] = src_code(SRC_SLOT, t);
        ++npro;
      }
    }
  }
  __syncthreads();
  // ---- the other new anchors' sources: staged tokens and old anchors (these win over a slot)
  for (int i = tid; i < k_new && i < p.anchor_cap; i += PT) {
    const int pos = idx[i];
    if (pos >= ps0 && pos < P) s.src_of[i] = src_code(SRC_STAGED, pos - ps0);
    else if (pos >= 0 && pos < P && bit_at(s.oldanc, pos)) s.src_of[i] = src_code(SRC_ANCHOR, rank_at(s.oldanc, s.pre_old, pos));
  }

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
  for (int w = w_lo + tid * per_w; w < min(w_hi, w_lo + (tid + 1) * per_w); ++w) {
    const uint32_t dw = s.del[w];
    for (int bit = 0; bit < 32; ++bit) {
      const int t = w * 32 + bit;
      if (t >= tail_lo && t < n_old && !((dw >> bit) & 1u)) ++ct;
    }
  }
  const int off_t = block_scan(ct, sh, &tot);
  {
    int o = e + off_t;
    for (int w = w_lo + tid * per_w; w < min(w_hi, w_lo + (tid + 1) * per_w); ++w) {
      const uint32_t dw = s.del[w];
      for (int bit = 0; bit < 32; ++bit) {
        const int t = w * 32 + bit;
        if (t >= tail_lo && t < n_old && !((dw >> bit) & 1u)) {
          if (o < p.max_moves) { s.mv_kind[o] = 2; s.mv_src[o] = t; }
          ++o;
        }
      }
    }
  }
  const int n_moves = e + tot;
  // targets: deleted slots below min(n_new, n_old), ascending, then fresh slots [n_old, n_new)
  const int hw = (tail_lo + 31) >> 5;
  const int per_h = (hw + PT - 1) / PT;
  int ch = 0;
  for (int w = tid * per_h; w < min(hw, (tid + 1) * per_h); ++w) {
    const uint32_t dw = s.del[w];
    for (int bit = 0; bit < 32; ++bit) {
      const int t = w * 32 + bit;
      if (t < tail_lo && ((dw >> bit) & 1u)) ++ch;
    }
  }
  const int off_h = block_scan(ch, sh, &tot);
  const int n_holes = tot;
  {
    int o = off_h;
    for (int w = tid * per_h; w < min(hw, (tid + 1) * per_h); ++w) {
      const uint32_t dw = s.del[w];
      for (int bit = 0; bit < 32; ++bit) {
        const int t = w * 32 + bit;
        if (t < tail_lo && ((dw >> bit) & 1u)) { if (o < p.max_moves) s.mv_dst[o] = t; ++o; }
      }
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

// ------------------------------------------------------------------ gather: 16 lanes per new anchor
// Lane l = lane & 15 of a row holds channels 8 l .. 8 l + 7 (group l / 4): a 16-byte load of a
// bf16 K row, eight 2-byte loads of a bf16 V row, or the codes and (scale, min) of a quantized
// slot; the row goes to the temp store with two 16-byte stores.
constexpr int GATHER_ROWS = 16;  // rows per workgroup: 4 waves x 4 rows

template <int BK, int BV>
__global__ __launch_bounds__(256) void refresh_gather_kernel(RefreshParams p) {
  const int hb = blockIdx.y, l = threadIdx.x & 15;
  const int i = blockIdx.x * GATHER_ROWS + (threadIdx.x >> 4);
  if (i >= p.k || i >= p.anchor_cap) return;
  const Scratch s = scratch(p, hb);
  const size_t aslab = (size_t)p.anchor_cap * D, sslab = (size_t)p.staging_cap * D;
  const int32_t code = s.src_of[i];
  const int kind = code >> SRC_SHIFT, si = code & ((1 << SRC_SHIFT) - 1);
  const int c0 = 8 * l, g = l >> 2;
  uint32_t ko[4], vo[4];
  if (kind == SRC_ANCHOR || kind == SRC_STAGED) {
    // bf16 already: an old anchor or a staged token
    const bool anc = kind == SRC_ANCHOR;
    if (si >= (anc ? p.anchor_cap : p.staging_cap)) return;
    const uint16_t* sk = anc ? p.a_k + hb * aslab : p.s_k + hb * sslab;
    const uint16_t* sv = anc ? p.a_v + hb * aslab : p.s_v + hb * sslab;
    const u32x4 kr = *(const u32x4*)(sk + kbf_index(si, c0));  // channels c0 .. c0+7
    ko[0] = kr[0]; ko[1] = kr[1]; ko[2] = kr[2]; ko[3] = kr[3];
    uint16_t vr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vr[e] = sv[vbf_index(si, c0 + e)];
#pragma unroll
    for (int e = 0; e < 4; ++e) vo[e] = (uint32_t)vr[2 * e] | ((uint32_t)vr[2 * e + 1] << 16);
  } else if (kind == SRC_SLOT) {
    // a quantized position: dequantize its slot
    if (si >= p.int4_cap) return;
    const uint8_t* slab = p.int4 + hb * (size_t)p.int4_cap * QL<BK, BV>::SLOT;
    // K codes of channels c0 .. c0+7: 8 BK bits from bit 8 BK (l & 3) of the group's chunk
    const int kbit = 8 * BK * (l & 3);
    uint64_t kbits;
    if constexpr (BK == 8) kbits = *(const uint64_t*)(slab + kcode_chunk_b<BK, BV>(si, g) + (kbit >> 3));
    else kbits = *(const uint32_t*)(slab + kcode_chunk_b<BK, BV>(si, g) + 4 * (kbit >> 5)) >> (kbit & 31);
    uint32_t vw[8];
    int vsh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      size_t off;
      vcode_loc<BK, BV>(si, c0 + e, off, vsh[e]);
      vw[e] = *(const uint32_t*)(slab + off);
    }
    const uint32_t ksm = *(const uint32_t*)(slab + ksm_byte_b<BK, BV>(si, g));
    const uint32_t vsm = *(const uint32_t*)(slab + vsm_byte_b<BK, BV>(si, g));
    const float ks = __half2float(__ushort_as_half((unsigned short)(ksm & 0xffff)));
    const float km = __half2float(__ushort_as_half((unsigned short)(ksm >> 16)));
    const float vs = __half2float(__ushort_as_half((unsigned short)(vsm & 0xffff)));
    const float vm = __half2float(__ushort_as_half((unsigned short)(vsm >> 16)));
    uint16_t kx[8], vx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t kc = (uint32_t)(kbits >> (BK * e)) & ((1u << BK) - 1u);
      const uint32_t vc = (vw[e] >> vsh[e]) & ((1u << BV) - 1u);
      // dequantized value = scale * code + min in fp32 (exact product, one rounding), then bf16
      kx[e] = f32_to_bf16_bits(ks * (float)kc + km);
      vx[e] = f32_to_bf16_bits(vs * (float)vc + vm);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ko[e] = (uint32_t)kx[2 * e] | ((uint32_t)kx[2 * e + 1] << 16);
      vo[e] = (uint32_t)vx[2 * e] | ((uint32_t)vx[2 * e + 1] << 16);
    }
  } else {
    return;  // malformed set: nothing to gather (the status reports it)
  }
  *(u32x4*)(s.tk + (size_t)i * D + c0) = (u32x4){ko[0], ko[1], ko[2], ko[3]};
  *(u32x4*)(s.tv + (size_t)i * D + c0) = (u32x4){vo[0], vo[1], vo[2], vo[3]};
}

// ------------------------------------------------------------------ move: tile-owner waves
// The move list is sorted by destination slot (holes ascending, then fresh slots ascending), so
// the moves into one 32-slot tile form a contiguous run of at most 32 entries.  Wave w takes the
// entries [MV_CHUNK w, MV_CHUNK (w + 1)) and owns every tile whose first move lies there; it
// runs past its chunk to finish its last tile.  One 64-lane load of the list from MV_CHUNK w - 1
// covers a chunk plus the longest run, so a wave reads its part of the list once.
//
// A V code shares its dword with the other slots of its quad only (every width), so the owner
// of a tile is the only writer of that tile's V-code dwords: it copies the dwords of the quads
// its moves touch into LDS (lane = 32 + 8 g + sub keeps those of channels 32 g + 4 sub + e,
// e < 4 -- the channels it quantizes -- in a column only it reads and writes, indexed by quad,
// e and half), replaces the codes there, and stores the dwords back -- plain loads and
// stores, no atomics.  Kept codes of slots nobody moves are
// written back unchanged (a tail slot read as a source by another wave keeps its value).  A
// 2-bit dword also spans channels c and c + 16 (lanes sub and sub + 4): those two lanes'
// copies are merged before the store.
//
// Demoting a bf16 row uses the whole wave: lane = 32 kv + 8 g + sub holds channels
// 32 g + 4 sub + e of K (kv = 0) or V (kv = 1); the group's min and max come from a reduction
// over its 8 lanes, and every code follows the group quantizer's formula.  The next move's
// source words are loaded while the current move is processed.
constexpr int MV_CHUNK = 4;
constexpr int MOVE_WAVES = 4;  // waves per workgroup

// min / max over the 8 lanes of a group (lanes 8 k .. 8 k + 7) with DPP, no LDS trip: lane
// swaps within each quad, then the half-row mirror pairs lane i with 7 - i (the other quad)
__device__ inline float dpp_half_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
}
__device__ inline float group8_min(float v) {
  v = fminf(v, dpp_quad_xor1(v));
  v = fminf(v, dpp_quad_xor2(v));
  return fminf(v, dpp_half_mirror(v));
}
__device__ inline float group8_max(float v) {
  v = fmaxf(v, dpp_quad_xor1(v));
  v = fmaxf(v, dpp_quad_xor2(v));
  return fmaxf(v, dpp_half_mirror(v));
}

// source words of one move, per lane (see load_move)
struct MoveSrc {
  uint32_t r[4];
  uint32_t sm;
  int32_t pos;
};

// Offsets inside one head's slab fit 32 bits; computing them as such keeps the address math
// off the 64-bit path.
template <typename T>
__device__ inline const T* at32(const void* base, size_t off) {
  return (const T*)((const uint8_t*)base + (uint32_t)off);
}

template <int BK, int BV>
__device__ inline MoveSrc load_move(const RefreshParams& p, int hb, int kind, int src, int lane, const uint8_t* slab,
                                    const int32_t* slot_pos, int ps0) {
  const int kv = lane >> 5, g = (lane >> 3) & 3, sub = lane & 7, c0 = 32 * g + 4 * sub;
  const size_t aslab = (size_t)p.anchor_cap * D, sslab = (size_t)p.staging_cap * D;
  MoveSrc m = {{0u, 0u, 0u, 0u}, 0u, -1};
  const int src_cap = kind == 0 ? p.anchor_cap : kind == 1 ? p.staging_cap : p.int4_cap;
  if (src < 0 || src >= src_cap) return m;  // not executed (the move loop checks the same bound)
  if (kind <= 1) {
    // bf16 row: K lanes read channels c0 .. c0+3 (8 bytes), V lanes the same channels (4 x 2 bytes)
    const uint16_t* sk = kind == 0 ? p.a_k + hb * aslab : p.s_k + hb * sslab;
    const uint16_t* sv = kind == 0 ? p.a_v + hb * aslab : p.s_v + hb * sslab;
    if (kv == 0) {
      const uint2 raw = *at32<uint2>(sk, 2 * kbf_index(src, c0));
      m.r[0] = raw.x;
      m.r[1] = raw.y;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) m.r[e] = *at32<uint16_t>(sv, 2 * vbf_index(src, c0 + e));
    }
    if (lane == 0) m.pos = kind == 0 ? p.a_pos[hb * (size_t)p.anchor_cap + src] : ps0 + src;
  } else {
    // quantized slot: K lanes sub < BK read dword sub of the group's K chunk, lane sub 0 the
    // group's (scale, min); V lanes read the dwords holding their 4 channels' codes
    if (kv == 0) {
      if (sub < BK) m.r[0] = *at32<uint32_t>(slab, kcode_chunk_b<BK, BV>(src, g) + 4 * sub);
      if (sub == 0) m.sm = *at32<uint32_t>(slab, ksm_byte_b<BK, BV>(src, g));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        size_t off;
        int sh;
        vcode_loc<BK, BV>(src, c0 + e, off, sh);
        m.r[e] = *at32<uint32_t>(slab, off);
      }
      if (sub == 0) m.sm = *at32<uint32_t>(slab, vsm_byte_b<BK, BV>(src, g));
    }
    if (lane == 0) m.pos = slot_pos[src];
  }
  return m;
}

template <int BK, int BV>
__global__ __launch_bounds__(64 * MOVE_WAVES) void refresh_move_kernel(RefreshParams p) {
  constexpr int NH = BV == 8 ? 2 : 1;  // V-code dwords per (quad, channel): INT8 codes take two
  constexpr int NSLOT = 16 * NH;       // owned dwords per V lane: (quad, channel e, half)
  constexpr uint32_t VMASK = (1u << BV) - 1u;
  // the owned V-code dwords, one column per V lane: [slot (quad, e, half)][lane - 32]
  __shared__ uint32_t vbuf[MOVE_WAVES][NSLOT][32];
  const int hb = blockIdx.y, lane = threadIdx.x & 63;
  const Scratch s = scratch(p, hb);
  const int n = min(s.cnt[0], p.max_moves);
  const int lo = (blockIdx.x * MOVE_WAVES + (threadIdx.x >> 6)) * MV_CHUNK;
  if (lo >= n) return;
  const int P = p.len - WIN;
  const int ps0 = P - p.n_staged;
  uint8_t* slab = p.int4 + hb * (size_t)p.int4_cap * QL<BK, BV>::SLOT;
  int32_t* slot_pos = p.slot_pos + hb * (size_t)p.int4_cap;
  const int kv = lane >> 5, g = (lane >> 3) & 3, sub = lane & 7, c0 = 32 * g + 4 * sub;
  const int n_tiles = p.int4_cap >> 5;
  uint32_t* vb = &vbuf[threadIdx.x >> 6][0][lane & 31];
  auto vslot = [](int q, int e, int h) { return ((q * 4 + e) * NH + h) * 32; };

  // the list window: lane i holds entry lo - 1 + i
  const int me = lo - 1 + lane;
  const bool in_list = me >= 0 && me < n;
  const int wdst = in_list ? s.mv_dst[me] : -1, wkind = in_list ? s.mv_kind[me] : 0, wsrc = in_list ? s.mv_src[me] : -1;
  const int wtile = wdst >> 5;
  const int prev_tile = __shfl_up(wtile, 1);
  const bool starts = in_list && lane >= 1 && (me == 0 || wtile != prev_tile);
  const uint64_t start_mask = __ballot(starts);
  // first owned entry: the first tile start at lanes 1 .. MV_CHUNK; the end: the first tile start
  // at lanes > MV_CHUNK, else the end of the list
  const uint64_t own = start_mask & (((1ull << MV_CHUNK) - 1ull) << 1);
  if (own == 0) return;  // the whole chunk continues a tile owned by an earlier wave
  const int j0 = __builtin_ctzll(own);
  const uint64_t later = start_mask & ~((2ull << MV_CHUNK) - 1ull);
  const int j_end = later ? __builtin_ctzll(later) : min(64, n - (lo - 1));

  // list entries are read across lanes with readlane (a uniform lane index, no LDS trip)
  MoveSrc nxt = load_move<BK, BV>(p, hb, __builtin_amdgcn_readlane(wkind, j0), __builtin_amdgcn_readlane(wsrc, j0), lane,
                                  slab, slot_pos, ps0);
  int tile = -1;
  uint32_t qmask = 0;
  for (int j = j0; j < j_end; ++j) {
    const int dst = __builtin_amdgcn_readlane(wdst, j);
    const int kind = __builtin_amdgcn_readlane(wkind, j);
    const int src = __builtin_amdgcn_readlane(wsrc, j);
    const MoveSrc cur = nxt;
    if (j + 1 < j_end)
      nxt = load_move<BK, BV>(p, hb, __builtin_amdgcn_readlane(wkind, j + 1), __builtin_amdgcn_readlane(wsrc, j + 1), lane,
                              slab, slot_pos, ps0);
    if ((dst >> 5) != tile) {
      // a new tile: the quads its moves touch, their V-code dwords into this lane's column
      tile = dst >> 5;
      const bool mine = lane >= j && lane < j_end && wtile == tile && wdst >= 0;
      qmask = 0;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        if (__ballot(mine && tile_quad(wdst & 31) == qq)) qmask |= 1u << qq;
      if (tile < 0 || tile >= n_tiles) qmask = 0;
      if (kv == 1) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          if (qmask >> qq & 1u) {
            uint32_t w[4][NH];
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int hh = 0; hh < NH; ++hh) {
                size_t off;
                int sh;
                vcode_loc<BK, BV>(32 * tile + 4 * qq + 16 * hh, c0 + e, off, sh);
                w[e][hh] = *at32<uint32_t>(slab, off);
              }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int hh = 0; hh < NH; ++hh) vb[vslot(qq, e, hh)] = w[e][hh];
          }
      }
    }
    const int src_cap = kind == 0 ? p.anchor_cap : kind == 1 ? p.staging_cap : p.int4_cap;
    const bool valid = dst >= 0 && dst < p.int4_cap && src >= 0 && src < src_cap;
    if (valid) {
      uint32_t code[4];
      if (kind <= 1) {
        // quantize a bf16 row (old anchor or staged token) into slot dst
        float x[4];
        if (kv == 0) {
          x[0] = bf16_bits_to_f32((uint16_t)cur.r[0]);
          x[1] = bf16_bits_to_f32((uint16_t)(cur.r[0] >> 16));
          x[2] = bf16_bits_to_f32((uint16_t)cur.r[1]);
          x[3] = bf16_bits_to_f32((uint16_t)(cur.r[1] >> 16));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = bf16_bits_to_f32((uint16_t)cur.r[e]);
        }
        const float mn = group8_min(fminf(fminf(x[0], x[1]), fminf(x[2], x[3])));
        const float mx = group8_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        // the group quantizer's scale, minimum and codes (same operations, same order)
        const float LEVELS = kv ? (float)((1 << BV) - 1) : (float)((1 << BK) - 1);
        const __half s16 = __float2half_rn(__fdiv_rn(__fsub_rn(mx, mn), LEVELS));
        const __half m16 = __float2half_rn(mn);
        const float sf = __half2float(s16), mf = __half2float(m16);
        const float rf = sf != 0.0f ? __builtin_amdgcn_rcpf(sf) : 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float cq = 0.0f;
          if (sf != 0.0f) {
            cq = rint_div(__fsub_rn(x[e], mf), sf, rf);  // = rint(IEEE (x - m) / s)
            cq = fminf(fmaxf(cq, 0.0f), LEVELS);
          }
          code[e] = (uint32_t)cq;
        }
        const uint32_t smw = (uint32_t)__half_as_ushort(s16) | ((uint32_t)__half_as_ushort(m16) << 16);
        if (kv == 0) {
          uint32_t* kc = (uint32_t*)(slab + (uint32_t)kcode_chunk_b<BK, BV>(dst, g));
          if constexpr (BK == 4) {
            // nibbles 4 sub + e of the group's 32; dword sub / 2 holds lanes sub & ~1 (low) and | 1
            const uint32_t half16 = code[0] | (code[1] << 4) | (code[2] << 8) | (code[3] << 12);
            const uint32_t other = (uint32_t)__float_as_int(dpp_quad_xor1(__int_as_float((int)half16)));
            if ((sub & 1) == 0) kc[sub >> 1] = half16 | (other << 16);
          } else if constexpr (BK == 8) {
            // bytes 4 sub + e of the group's 32: one dword per lane
            kc[sub] = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
          } else {
            // 2-bit codes 4 sub + e: byte sub & 3 of dword sub / 4, OR-ed over the dword's 4 lanes
            uint32_t w = (code[0] | (code[1] << 2) | (code[2] << 4) | (code[3] << 6)) << (8 * (sub & 3));
            w |= (uint32_t)__float_as_int(dpp_quad_xor1(__int_as_float((int)w)));
            w |= (uint32_t)__float_as_int(dpp_quad_xor2(__int_as_float((int)w)));
            if ((sub & 3) == 0) kc[sub >> 2] = w;
          }
          if (sub == 0) *(uint32_t*)(slab + (uint32_t)ksm_byte_b<BK, BV>(dst, g)) = smw;
        } else if (sub == 0) {
          *(uint32_t*)(slab + (uint32_t)vsm_byte_b<BK, BV>(dst, g)) = smw;
        }
      } else {
        // move a quantized slot: K chunk dwords and (scale, min) as read, V codes re-placed
        if (kv == 0) {
          if (sub < BK) *(uint32_t*)(slab + (uint32_t)(kcode_chunk_b<BK, BV>(dst, g) + 4 * sub)) = cur.r[0];
          if (sub == 0) *(uint32_t*)(slab + (uint32_t)ksm_byte_b<BK, BV>(dst, g)) = cur.sm;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            size_t off;
            int sh;
            vcode_loc<BK, BV>(src, c0 + e, off, sh);
            code[e] = (cur.r[e] >> sh) & VMASK;
          }
          if (sub == 0) *(uint32_t*)(slab + (uint32_t)vsm_byte_b<BK, BV>(dst, g)) = cur.sm;
        }
      }
      if (kv == 1) {
        // replace slot dst's codes in the owned dwords (quad and half are wave-uniform)
        const int q = tile_quad(dst & 31), h = NH == 2 ? (dst & 31) >> 4 : 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          size_t off;
          int sh;
          vcode_loc<BK, BV>(dst, c0 + e, off, sh);
          uint32_t* w = &vb[vslot(q, e, h)];
          *w = (*w & ~(VMASK << sh)) | (code[e] << sh);
        }
      }
      if (lane == 0) slot_pos[dst] = cur.pos;
    }
    // the tile's last move: the owned dwords go back
    if (j + 1 == j_end || (__builtin_amdgcn_readlane(wdst, j + 1) >> 5) != tile) {
      if (kv == 1) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          if (qmask >> qq & 1u) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int hh = 0; hh < NH; ++hh) {
                size_t off;
                int sh;
                vcode_loc<BK, BV>(32 * tile + 4 * qq + 16 * hh, c0 + e, off, sh);
                const uint32_t w = vb[vslot(qq, e, hh)];
                if constexpr (BV == 2) {
                  // a 2-bit dword holds channels c (bytes 0 and 2) and c + 16 (bytes 1 and 3):
                  // lanes sub and sub + 4 edit one each; the merged dword goes out once
                  const uint32_t other = (uint32_t)__shfl_xor((int)w, 4);
                  if (sub < 4) *(uint32_t*)(slab + (uint32_t)off) = (w & 0x00FF00FFu) | (other & 0xFF00FF00u);
                } else {
                  *(uint32_t*)(slab + (uint32_t)off) = w;
                }
              }
          }
      }
    }
  }
}

// ------------------------------------------------------------------ store: one workgroup per anchor tile
// anchor store <- temp (tile layouts), positions, zeroed tail of the last tile.  The tile's 32
// temp rows of K and V (row-major, 16 KB) are staged in LDS with 16-byte loads, then written in
// the tile layouts with 16-byte stores: a K chunk is 8 consecutive channels of one position
// (a permutation of the temp's 16-byte pieces), a V piece one channel at the 8 positions of a
// quad (a transpose, gathered from LDS).
__global__ __launch_bounds__(256) void refresh_store_kernel(RefreshParams p) {
  __shared__ uint16_t sk[32][D], sv[32][D];
  const int hb = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
  const int k_new = p.k;
  const int i0 = tile * 32;
  const Scratch s = scratch(p, hb);
  for (int ch = tid; ch < 1024; ch += 256) {  // 32 rows x 16 pieces, K then V
    const int kv = ch >> 9, row = (ch >> 4) & 31, part = ch & 15;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (i0 + row < k_new) v = *(const u32x4*)((kv ? s.tv : s.tk) + (size_t)(i0 + row) * D + 8 * part);
    *(u32x4*)(kv ? &sv[row][8 * part] : &sk[row][8 * part]) = v;
  }
  __syncthreads();
  const size_t aslab = (size_t)p.anchor_cap * D;
  uint16_t* ak = p.a_k + hb * aslab + (size_t)tile * 4096;
  uint16_t* av = p.a_v + hb * aslab + (size_t)tile * 4096;
  for (int ch = tid; ch < 512; ch += 256) {
    // K chunk ch = ((p16 * 4 + tt) * 4 + q4) * 16 + p15: channels 32 q4 + 8 tt .. + 7 of position 16 p16 + p15
    const int p15 = ch & 15, q4 = (ch >> 4) & 3, tt = (ch >> 6) & 3, p16 = ch >> 8;
    *(u32x4*)(ak + 8 * ch) = *(const u32x4*)&sk[16 * p16 + p15][32 * q4 + 8 * tt];
    // V piece ch = ((c >> 4) * 4 + q) * 16 + (c & 15): channel c at the positions of quad q, k-slot order
    const int ci = ch & 15, q = (ch >> 4) & 3, cb = ch >> 6, c = 16 * cb + ci;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pa = 4 * q + ((2 * e) & 3) + 16 * ((2 * e) >> 2), pb = 4 * q + ((2 * e + 1) & 3) + 16 * ((2 * e + 1) >> 2);
      w[e] = (uint32_t)sv[pa][c] | ((uint32_t)sv[pb][c] << 16);
    }
    *(u32x4*)(av + 8 * ch) = (u32x4){w[0], w[1], w[2], w[3]};
  }
  if (tid < 32) p.a_pos[hb * (size_t)p.anchor_cap + i0 + tid] = i0 + tid < k_new ? p.idx[hb * (size_t)k_new + i0 + tid] : -1;
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
  const int move_waves = (p.max_moves + MV_CHUNK - 1) / MV_CHUNK;
  const dim3 mgrid(std::max(1, (move_waves + MOVE_WAVES - 1) / MOVE_WAVES), H);
  hipError_t e = with_widths(p.bits, p.bits_v, [&](auto BK, auto BV) {
    constexpr int K = decltype(BK)::value, V = decltype(BV)::value;
    if (ka > 0) hipLaunchKernelGGL((refresh_gather_kernel<K, V>), dim3((ka + GATHER_ROWS - 1) / GATHER_ROWS, H), dim3(256), 0, stream, p);
    hipLaunchKernelGGL((refresh_move_kernel<K, V>), mgrid, dim3(64 * MOVE_WAVES), 0, stream, p);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  const int a_end = min((p.k + 31) & ~31, p.anchor_cap);
  if (a_end > 0) hipLaunchKernelGGL(refresh_store_kernel, dim3(a_end / 32, H), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hyq

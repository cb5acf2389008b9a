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

// quantize 32 channels (group g) of a bf16 row and store them into INT4 slot `slot`
__device__ inline void store_int4_group(uint8_t* slab, int slot, int g, bool is_v, const float* x) {
  uint8_t code[32];
  __half s16, m16;
  quant_group32(x, code, s16, m16);
  const uint32_t smw = (uint32_t)__half_as_ushort(s16) | ((uint32_t)__half_as_ushort(m16) << 16);
  if (!is_v) {
    u32x4 packed;
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) {
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) w |= (uint32_t)code[8 * d4 + j] << (4 * j);
      packed[d4] = w;
    }
    *(u32x4*)(slab + kcode_chunk(slot, g)) = packed;
    *(uint32_t*)(slab + ksm_byte(slot, g)) = smw;
  } else {
    const int sh = vcode_shift(slot);
    for (int j = 0; j < 32; ++j) {
      unsigned* dw = (unsigned*)(slab + vcode_byte(slot, 32 * g + j));
      atomicAnd(dw, ~(0xFu << sh));
      atomicOr(dw, (uint32_t)code[j] << sh);
    }
    *(uint32_t*)(slab + vsm_byte(slot, g)) = smw;
  }
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
  // an INT4 position: dequantize its slot
  const int t = s.slot_of[i];
  if (t < 0 || t >= p.int4_cap) return;
  const uint8_t* slab = p.int4 + hb * (size_t)p.int4_cap * 160;
  for (int c = lane; c < D; c += 64) {
    const int g = c >> 5;
    const uint8_t kb = slab[kcode_chunk(t, g) + ((c & 31) >> 1)];
    const uint32_t kc = (c & 1) ? (kb >> 4) : (kb & 15u);
    const uint32_t vw = *(const uint32_t*)(slab + vcode_byte(t, c));
    const uint32_t vc = (vw >> vcode_shift(t)) & 15u;
    const uint32_t ksm = *(const uint32_t*)(slab + ksm_byte(t, g));
    const uint32_t vsm = *(const uint32_t*)(slab + vsm_byte(t, g));
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
__global__ __launch_bounds__(256) void refresh_move_kernel(RefreshParams p) {
  const int hb = blockIdx.y, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const Scratch s = scratch(p, hb);
  if (t >= s.cnt[0]) return;
  const int P = p.len - WIN;
  const int ps0 = P - p.n_staged;
  uint8_t* slab = p.int4 + hb * (size_t)p.int4_cap * 160;
  int32_t* slot_pos = p.slot_pos + hb * (size_t)p.int4_cap;
  const size_t aslab = (size_t)p.anchor_cap * D, sslab = (size_t)p.staging_cap * D;
  const int dst = s.mv_dst[t], kind = s.mv_kind[t], src = s.mv_src[t];
  if (dst < 0 || dst >= p.int4_cap) return;
  if (kind <= 1) {
    // quantize a bf16 row (old anchor or staged token): lanes 0..7 = (K/V, group)
    const uint16_t* sk = kind == 0 ? p.a_k + hb * aslab : p.s_k + hb * sslab;
    const uint16_t* sv = kind == 0 ? p.a_v + hb * aslab : p.s_v + hb * sslab;
    if (lane < 8) {
      const bool is_v = lane >= 4;
      const int g = lane & 3;
      float x[32];
      for (int j = 0; j < 32; ++j) {
        const int c = 32 * g + j;
        x[j] = bf16_bits_to_f32(is_v ? sv[vbf_index(src, c)] : sk[kbf_index(src, c)]);
      }
      store_int4_group(slab, dst, g, is_v, x);
    }
    if (lane == 0) slot_pos[dst] = kind == 0 ? p.a_pos[hb * (size_t)p.anchor_cap + src] : ps0 + src;
  } else {
    // move an INT4 slot: codes, (scale, min), position
    if (lane < 16) {  // K code chunks (4 x 16 B) as 16 dwords
      const int g = lane >> 2, d = lane & 3;
      *(uint32_t*)(slab + kcode_chunk(dst, g) + 4 * d) = *(const uint32_t*)(slab + kcode_chunk(src, g) + 4 * d);
    } else if (lane < 20) {
      const int g = lane - 16;
      *(uint32_t*)(slab + ksm_byte(dst, g)) = *(const uint32_t*)(slab + ksm_byte(src, g));
      *(uint32_t*)(slab + vsm_byte(dst, g)) = *(const uint32_t*)(slab + vsm_byte(src, g));
    }
    const int shs = vcode_shift(src), shd = vcode_shift(dst);
    for (int c = lane; c < D; c += 64) {
      const uint32_t code = (*(const uint32_t*)(slab + vcode_byte(src, c)) >> shs) & 15u;
      unsigned* dw = (unsigned*)(slab + vcode_byte(dst, c));
      atomicAnd(dw, ~(0xFu << shd));
      atomicOr(dw, code << shd);
    }
    if (lane == 0) slot_pos[dst] = slot_pos[src];
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
  if (ka > 0) hipLaunchKernelGGL(refresh_gather_kernel, dim3((ka + 3) / 4, H), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(refresh_move_kernel, dim3((p.max_moves + 3) / 4, H), dim3(256), 0, stream, p);
  const int a_end = min((p.k + 31) & ~31, p.anchor_cap);
  if (a_end > 0) hipLaunchKernelGGL(refresh_store_kernel, dim3((a_end + 3) / 4, H), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hyq

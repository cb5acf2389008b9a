// Refresh of the hybrid cache after a new vertical-line set (one workgroup per head).
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
// Writes of single V codes go through dword atomics (8 slots share each V-code dword).
//
// Built with -ffp-contract=off (the quantizer's operation order is part of its contract).
#include "hyq_common.h"
#include "hyq_launch.h"

namespace hyq {

namespace {

constexpr int RT = 256;  // threads per workgroup

__device__ inline int lower_bound_i32(const int32_t* a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// block-wide exclusive scan of one int per thread; returns the exclusive prefix, total in *tot
__device__ inline int block_scan(int v, int* sh, int* tot) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < RT; off <<= 1) {
    const int add = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int incl = sh[tid];
  *tot = sh[RT - 1];
  __syncthreads();
  return incl - v;
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

__global__ __launch_bounds__(RT) void refresh_apply_kernel(RefreshParams p) {
  __shared__ int sh[RT];
  __shared__ int s_cnt, s_e, s_pdel, s_tail;
  const int hb = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, NWV = RT / 64;
  const int P = p.len - WIN;
  const int ps0 = P - p.n_staged;  // first staged position
  const int k_old = p.n_anchor_old, k_new = p.k, n_old = p.n_int4_old, ns = p.n_staged;
  uint8_t* slab = p.int4 + hb * (size_t)p.int4_cap * 160;
  int32_t* slot_pos = p.slot_pos + hb * (size_t)p.int4_cap;
  const size_t aslab = (size_t)p.anchor_cap * D, sslab = (size_t)p.staging_cap * D;
  uint16_t* a_k = p.a_k + hb * aslab;
  uint16_t* a_v = p.a_v + hb * aslab;
  int32_t* a_pos = p.a_pos + hb * (size_t)p.anchor_cap;
  const uint16_t* s_k = p.s_k + hb * sslab;
  const uint16_t* s_v = p.s_v + hb * sslab;
  const int32_t* idx = p.idx + hb * (size_t)k_new;
  // per-head scratch
  uint8_t* ws = p.ws + hb * p.ws_per_head;
  uint32_t* inset = (uint32_t*)ws;                               // ceil(P/32) words
  uint32_t* del = inset + p.inset_words;                          // ceil(int4_cap/32) words
  uint16_t* tk = (uint16_t*)(del + p.del_words);                  // new anchors K [k][128]
  uint16_t* tv = tk + (size_t)p.anchor_cap * D;                   // new anchors V [k][128]
  int32_t* promo = (int32_t*)(tv + (size_t)p.anchor_cap * D);     // promoted (slot, rank) pairs
  int32_t* mv_dst = promo + 2 * (size_t)p.anchor_cap;             // move targets
  int32_t* mv_kind = mv_dst + p.max_moves;                        // 0 anchor, 1 staged, 2 slot
  int32_t* mv_src = mv_kind + p.max_moves;

  // ---- P0: membership bitmap of the new set, cleared deletion bitmap
  for (int i = tid; i < p.inset_words; i += RT) inset[i] = 0u;
  for (int i = tid; i < p.del_words; i += RT) del[i] = 0u;
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  for (int i = tid; i < k_new; i += RT) atomicOr(&inset[idx[i] >> 5], 1u << (idx[i] & 31));
  __syncthreads();
  auto in_set = [&](int pos) -> bool { return (inset[pos >> 5] >> (pos & 31)) & 1u; };

  // ---- P1: new anchors that already hold bf16 (old anchors, staged tokens) -> temp store
  for (int i = wave; i < k_new; i += NWV) {
    const int pos = idx[i];
    const uint16_t *sk = nullptr, *sv = nullptr;
    int si = -1;
    if (pos >= ps0) { sk = s_k; sv = s_v; si = pos - ps0; }
    else {
      const int j = lower_bound_i32(a_pos, k_old, pos);
      if (j < k_old && a_pos[j] == pos) { sk = a_k; sv = a_v; si = j; }
    }
    if (si < 0) continue;  // an INT4 position: P2
    for (int c = lane; c < D; c += 64) {
      tk[(size_t)i * D + c] = sk[kbf_index(si, c)];
      tv[(size_t)i * D + c] = sv[vbf_index(si, c)];
    }
  }
  // ---- P2: INT4 slots whose position is in the set are promoted
  for (int s = tid; s < n_old; s += RT) {
    const int pos = slot_pos[s];
    if (pos >= 0 && pos < P && in_set(pos)) {
      atomicOr(&del[s >> 5], 1u << (s & 31));
      const int at = atomicAdd(&s_cnt, 1);
      if (at < p.anchor_cap) {
        promo[2 * at] = s;
        promo[2 * at + 1] = lower_bound_i32(idx, k_new, pos);
      }
    }
  }
  __syncthreads();
  const int n_promo = min(s_cnt, p.anchor_cap);
  for (int t = wave; t < n_promo; t += NWV) {
    const int s = promo[2 * t], i = promo[2 * t + 1];
    for (int c = lane; c < D; c += 64) {
      const int g = c >> 5;
      const uint8_t kb = slab[kcode_chunk(s, g) + ((c & 31) >> 1)];
      const uint32_t kc = (c & 1) ? (kb >> 4) : (kb & 15u);
      const uint32_t vw = *(const uint32_t*)(slab + vcode_byte(s, c));
      const uint32_t vc = (vw >> vcode_shift(s)) & 15u;
      const uint32_t ksm = *(const uint32_t*)(slab + ksm_byte(s, g));
      const uint32_t vsm = *(const uint32_t*)(slab + vsm_byte(s, g));
      // dequantized value = scale * code + min in fp32 (exact product, one rounding), then bf16
      const float kx = __half2float(__ushort_as_half((unsigned short)(ksm & 0xffff))) * (float)kc +
                       __half2float(__ushort_as_half((unsigned short)(ksm >> 16)));
      const float vx = __half2float(__ushort_as_half((unsigned short)(vsm & 0xffff))) * (float)vc +
                       __half2float(__ushort_as_half((unsigned short)(vsm >> 16)));
      tk[(size_t)i * D + c] = f32_to_bf16_bits(kx);
      tv[(size_t)i * D + c] = f32_to_bf16_bits(vx);
    }
  }
  __syncthreads();

  // ---- P3: new INT4 entries E (old anchors, then staged tokens, not in the set, ascending),
  // holes (deleted slots), and the move list targets <- sources
  int tot;
  // E from old anchors
  int ca = 0, cs = 0;
  const int per_a = (k_old + RT - 1) / RT, per_s = (ns + RT - 1) / RT;
  for (int j = tid * per_a; j < min(k_old, (tid + 1) * per_a); ++j) ca += !in_set(a_pos[j]);
  for (int j = tid * per_s; j < min(ns, (tid + 1) * per_s); ++j) cs += !in_set(ps0 + j);
  const int off_a = block_scan(ca, sh, &tot);
  const int e_a = tot;
  const int off_s = block_scan(cs, sh, &tot);
  const int e = e_a + tot;
  int pdel_mine = 0;
  for (int w = tid; w < p.del_words; w += RT) pdel_mine += __popc(del[w]);
  block_scan(pdel_mine, sh, &tot);
  const int p_del = tot;
  const int n_new = n_old - p_del + e;
  // sources: E entries (indices 0..e-1 of the move list), then alive tail slots [n_new, n_old)
  {
    int o = off_a;
    for (int j = tid * per_a; j < min(k_old, (tid + 1) * per_a); ++j)
      if (!in_set(a_pos[j])) { if (o < p.max_moves) { mv_kind[o] = 0; mv_src[o] = j; } ++o; }
    o = e_a + off_s;
    for (int j = tid * per_s; j < min(ns, (tid + 1) * per_s); ++j)
      if (!in_set(ps0 + j)) { if (o < p.max_moves) { mv_kind[o] = 1; mv_src[o] = j; } ++o; }
  }
  // alive tail slots, ascending (words are scanned in order, 32 slots per word)
  const int tail_lo = n_new < n_old ? n_new : n_old;
  const int w_lo = tail_lo >> 5, w_hi = (n_old + 31) >> 5;
  const int per_w = (w_hi - w_lo + RT - 1) / RT;
  int ct = 0;
  for (int w = w_lo + tid * per_w; w < min(w_hi, w_lo + (tid + 1) * per_w); ++w)
    for (int bit = 0; bit < 32; ++bit) {
      const int s = w * 32 + bit;
      if (s >= tail_lo && s < n_old && !((del[w] >> bit) & 1u)) ++ct;
    }
  const int off_t = block_scan(ct, sh, &tot);
  {
    int o = e + off_t;
    for (int w = w_lo + tid * per_w; w < min(w_hi, w_lo + (tid + 1) * per_w); ++w)
      for (int bit = 0; bit < 32; ++bit) {
        const int s = w * 32 + bit;
        if (s >= tail_lo && s < n_old && !((del[w] >> bit) & 1u)) {
          if (o < p.max_moves) { mv_kind[o] = 2; mv_src[o] = s; }
          ++o;
        }
      }
  }
  const int n_moves = e + tot;
  // targets: deleted slots below min(n_new, n_old), ascending, then fresh slots [n_old, n_new)
  const int hw = (tail_lo + 31) >> 5;
  const int per_h = (hw + RT - 1) / RT;
  int ch = 0;
  for (int w = tid * per_h; w < min(hw, (tid + 1) * per_h); ++w)
    for (int bit = 0; bit < 32; ++bit) {
      const int s = w * 32 + bit;
      if (s < tail_lo && ((del[w] >> bit) & 1u)) ++ch;
    }
  const int off_h = block_scan(ch, sh, &tot);
  const int n_holes = tot;
  {
    int o = off_h;
    for (int w = tid * per_h; w < min(hw, (tid + 1) * per_h); ++w)
      for (int bit = 0; bit < 32; ++bit) {
        const int s = w * 32 + bit;
        if (s < tail_lo && ((del[w] >> bit) & 1u)) { if (o < p.max_moves) mv_dst[o] = s; ++o; }
      }
  }
  for (int s = n_old + tid; s < n_new; s += RT)
    if (n_holes + (s - n_old) < p.max_moves) mv_dst[n_holes + (s - n_old)] = s;
  __syncthreads();
  if (tid == 0) { s_e = n_moves; s_pdel = p_del; s_tail = n_new; }
  __syncthreads();

  // ---- P4: execute the moves (one wave per move)
  // n_new == len - W - k for a valid set (distinct, ascending, inside [0, len - W)); the guards
  // keep a malformed set from writing outside the store
  const int n_exec = min(n_moves, min(p.max_moves, n_holes + max(0, n_new - n_old)));
  for (int t = wave; t < n_exec; t += NWV) {
    const int dst = mv_dst[t], kind = mv_kind[t], src = mv_src[t];
    if (dst < 0 || dst >= p.int4_cap) continue;
    if (kind <= 1) {
      // quantize a bf16 row (old anchor or staged token): lanes 0..7 = (K/V, group)
      const uint16_t* sk = kind == 0 ? a_k : s_k;
      const uint16_t* sv = kind == 0 ? a_v : s_v;
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
      if (lane == 0) slot_pos[dst] = kind == 0 ? a_pos[src] : ps0 + src;
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
  __syncthreads();

  // ---- P5: anchor store <- temp (tile layouts), positions, zeroed tail of the last tile
  const int a_end = (k_new + 31) & ~31;
  for (int i = wave; i < a_end; i += NWV) {
    for (int c = lane; c < D; c += 64) {
      a_k[kbf_index(i, c)] = i < k_new ? tk[(size_t)i * D + c] : (uint16_t)0;
      a_v[vbf_index(i, c)] = i < k_new ? tv[(size_t)i * D + c] : (uint16_t)0;
    }
    if (lane == 0) a_pos[i] = i < k_new ? idx[i] : -1;
  }
  // report (for the host-side consistency check in tests): n_new must equal len - W - k
  if (tid == 0 && p.status) p.status[hb] = (s_tail == P - k_new && s_e >= 0 && s_pdel >= 0) ? 0 : 1;
}

}  // namespace

hipError_t launch_refresh(const RefreshParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(refresh_apply_kernel, dim3(p.B * p.Hkv), dim3(RT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hyq

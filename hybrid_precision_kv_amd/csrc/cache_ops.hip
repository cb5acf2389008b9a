// Cache maintenance kernels: Freeze (prefill -> decode organisation) and token append.
//
// HyQuant paper ("HyQuant: Hybrid-Precision Quantization for LLM Attention"), Alg. 4: the last
// W keys become the local window, the vertical-line positions keep bf16, every other position
// of the non-window prefix is quantized with group size G (here per token, 32 channels, INT4
// asymmetric with fp16 scale and min); new decode tokens pass through the window and a bf16
// staging buffer (Alg. 3 segment 3).
//
// This file is compiled with -ffp-contract=off: the quantizer's operation order is part of
// its contract (codes are reproducible bit for bit).
#include "hyq_common.h"
#include "hyq_launch.h"

namespace hyq {

namespace {

// Number of anchors a_i (ascending, i = rank) with a_i - i <= s: the INT4 slot s of a Freeze
// holds position s + that count (slots enumerate the non-anchor prefix in order).
__device__ inline int slot_to_pos(const int32_t* anc, int n_anchor, int s) {
  int lo = 0, hi = n_anchor;  // first index with a_i - i > s
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (anc[mid] - mid <= s) lo = mid + 1; else hi = mid;
  }
  return s + lo;
}

// nibble j of a V-code dword -> k-slot e (inverse of kslot_nibble)
__device__ inline int nibble_kslot(int j) { return ((j & 3) << 1) | (j >> 2); }

// ---------------------------------------------------------------- Freeze: quantized slots
constexpr int VROW = 36;  // dwords per slot row of the V-code staging (128 code bytes + 16 pad)
// BK-bit K codes and BV-bit V codes, 2^B - 1 levels each (4/4: the INT4 record; 8/8, 4/2 and
// 2/2: the same record structure)
template <int BK, int BV>
__device__ inline void freeze_q_tile(const CacheView& c, const uint16_t* __restrict__ k,
                                     const uint16_t* __restrict__ v, int len, const int32_t* __restrict__ anchors,
                                     int n_anchor, int n_int4, int tile, int hkv, int b) {
  typedef QL<BK, BV> L;
  // V codes of the tile, one byte each: row = slot, byte = channel (a row of 144 bytes: the
  // 16-byte writes of the four groups of two slots fall on distinct banks)
  __shared__ __align__(16) uint32_t vlds[32][VROW];
  __shared__ int win[64];  // a_i - i for the 64 anchors from c0 on (INT_MAX past the list)
  __shared__ int s_c0, s_ok;
  const size_t hb = (size_t)b * c.Hkv + hkv;
  const int t = threadIdx.x;
  // waves 0-1 quantize K rows and waves 2-3 V rows (kv is uniform in a wave); slot sl, group g
  const int kv = __builtin_amdgcn_readfirstlane(t >> 7), sl = (t >> 2) & 31, g = t & 3;
  const int slot = tile * 32 + sl;
  bool valid = slot < n_int4;
  const int32_t* anc = anchors ? anchors + hb * (size_t)n_anchor : nullptr;
  uint8_t* slab = c.int4 + hb * (size_t)c.int4_cap * L::SLOT;
  // Positions of the tile's 32 slots: slot s holds position s + c(s), c(s) = the number of
  // anchors with a_i - i <= s (a_i - i does not decrease with i).  Wave 0 finds c0 = c(s0) for
  // the tile's first slot with a 64-way search (each round probes 64 indices at once), then
  // stages a_i - i of the next 64 anchors; every slot counts inside that window.  A tile whose
  // range holds more than the window's anchors takes the per-slot binary search.
  const int s0 = tile * 32;
  if (t < 64) {
    int lo = 0, hi = n_anchor;  // c0 in [lo, hi]
    while (lo < hi) {
      const int idx = lo + (int)(((long)(hi - lo) * t) >> 6);
      const bool gt = anc[idx] - idx > s0;
      const uint64_t m = __ballot(gt);
      if (m & 1ull) { hi = lo; break; }  // the first probe (index lo) already exceeds s0
      const int first = m ? __builtin_ctzll(m) : 64;
      const int nlo = lo + (int)(((long)(hi - lo) * (first - 1)) >> 6) + 1;
      const int nhi = first < 64 ? lo + (int)(((long)(hi - lo) * first) >> 6) : hi;
      lo = nlo;
      hi = nhi;
    }
    const int c0 = hi;
    const int i = c0 + t;
    const int w = i < n_anchor ? anc[i] - i : 0x7fffffff;
    win[t] = w;
    const bool covered = __ballot(t == 63 && (w > s0 + 31)) != 0;  // the window reaches past the tile
    if (t == 0) { s_c0 = c0; s_ok = covered; }
  }
  __syncthreads();
  int pos = 0;
  if (valid) {
    if (s_ok) {
      int lo2 = 0, hi2 = 64;  // first window entry above slot
#pragma unroll
      for (int step = 0; step < 7; ++step) {
        if (lo2 < hi2) {
          const int mid = (lo2 + hi2) >> 1;
          if (win[mid] <= slot) lo2 = mid + 1; else hi2 = mid;
        }
      }
      pos = slot + s_c0 + lo2;
    } else {
      pos = slot_to_pos(anc, n_anchor, slot);
    }
  }
  if (pos >= len) { valid = false; pos = 0; }  // anchors outside [0, len - W): contract violation

  __half s16 = __float2half(0.f), m16 = __float2half(0.f);
  uint32_t cb[8];  // the group's 32 codes, one byte each (code j in byte j % 4 of dword j / 4)
#pragma unroll
  for (int d = 0; d < 8; ++d) cb[d] = 0;
  if (valid) {
    const uint16_t* src = (kv ? v : k) + (hb * (size_t)len + pos) * D + 32 * g;
    u32x4 w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = *(const u32x4*)(src + 8 * j);
    // channel j: the bf16 bits of dword j / 2 (low half for even j) as fp32
    auto x = [&](int j) {
      const uint32_t d = w[j >> 3][(j >> 1) & 3];
      return __uint_as_float((j & 1) ? (d & 0xffff0000u) : (d << 16));
    };
    auto fresh = [&]() {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(w[j][e]));
    };
    if constexpr (BK == BV) {
      quant_group32<(1 << BK) - 1, 8>(x, fresh, cb, s16, m16);
    } else {
      if (kv == 0) quant_group32<(1 << BK) - 1, 8>(x, fresh, cb, s16, m16);
      else quant_group32<(1 << BV) - 1, 8>(x, fresh, cb, s16, m16);
    }
  }
  const uint32_t smw = (uint32_t)__half_as_ushort(s16) | ((uint32_t)__half_as_ushort(m16) << 16);
  if (kv == 0) {
    // the slot's group chunk (BK dwords): channel j at bits BK j
    uint32_t kw[BK];
    if constexpr (BK == 8) {
#pragma unroll
      for (int d = 0; d < 8; ++d) kw[d] = cb[d];
    } else if constexpr (BK == 4) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {  // bytes 0 and 2 of b | b >> 4 hold code pairs (4j, 4j + 1), (4j + 2, 4j + 3)
        const uint32_t lo = cb[2 * d] | (cb[2 * d] >> 4), hi = cb[2 * d + 1] | (cb[2 * d + 1] >> 4);
        kw[d] = __builtin_amdgcn_perm(hi, lo, 0x06040200u);
      }
    } else {
#pragma unroll
      for (int d = 0; d < 2; ++d) {  // four dwords of byte codes -> one dword of 2-bit codes
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t b = cb[4 * d + i];
          b |= b >> 6;   // bits 0-3: codes (0, 1); bits 16-19: codes (2, 3)
          b |= b >> 12;  // bits 0-7: codes 0..3
          w |= (b & 0xffu) << (8 * i);
        }
        kw[d] = w;
      }
    }
    uint8_t* chunk = slab + kcode_chunk_b<BK, BV>(slot, g);
    if constexpr (BK == 2) {
      *(uint2*)chunk = make_uint2(kw[0], kw[1]);
    } else {
#pragma unroll
      for (int h = 0; h < BK / 4; ++h)
        *(u32x4*)(chunk + 16 * h) = (u32x4){kw[4 * h], kw[4 * h + 1], kw[4 * h + 2], kw[4 * h + 3]};
    }
    *(uint32_t*)(slab + ksm_byte_b<BK, BV>(slot, g)) = smw;
    if (g == 0) c.slot_pos[hb * (size_t)c.int4_cap + slot] = valid ? pos : -1;
  } else {
    *(uint32_t*)(slab + vsm_byte_b<BK, BV>(slot, g)) = smw;
    *(u32x4*)&vlds[sl][8 * g] = (u32x4){cb[0], cb[1], cb[2], cb[3]};
    *(u32x4*)&vlds[sl][8 * g + 4] = (u32x4){cb[4], cb[5], cb[6], cb[7]};
  }
  __syncthreads();
  const uint8_t* vb = (const uint8_t*)&vlds[0][0];
  auto vcode = [&](int p, int ch) { return (uint32_t)vb[p * (4 * VROW) + ch]; };
  uint32_t* vtile = (uint32_t*)(slab + (size_t)tile * L::TB + L::VC);
  if constexpr (BV == 2) {
    // dword d = (q * 16 + i) * 4 + d4: channel blocks 2 d4 + h at the quad's 8 slots
    {
      const int d = t, d4 = d & 3, i = (d >> 2) & 15, q = d >> 6;
      uint32_t w = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ch = 16 * (2 * d4 + h) + i;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int p = 4 * q + (e & 3) + 16 * (e >> 2);
          w |= vcode(p, ch) << (2 * (e >> 1) + 16 * (e & 1) + 8 * h);
        }
      }
      vtile[d] = w;
    }
  } else if constexpr (BV == 4) {
    for (int d = t; d < 512; d += 256) {  // d = vcode_dword_in_tile(p, ch) for the quad's slots
      const int l = (d & 255) >> 2, q = l >> 4, i = l & 15, r = 4 * (d >> 8) + (d & 3);
      const int ch = 16 * r + i;
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = nibble_kslot(j);
        const int p = 4 * q + (e & 3) + 16 * (e >> 2);
        w |= vcode(p, ch) << (4 * j);
      }
      vtile[d] = w;
    }
  } else {
    // dword d = 2 entry + half8 of entry ((hf * 4 + q) * 16 + i) * 4 + r4: bytes 4 half8 .. + 3
    for (int d = t; d < 1024; d += 256) {
      const int entry = d >> 1, half8 = d & 1;
      const int r4 = entry & 3, i = (entry >> 2) & 15, q = (entry >> 6) & 3, hf = entry >> 8;
      const int ch = 16 * (4 * hf + r4) + i;
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int byte = 4 * half8 + b;  // byte = kslot_byte(e): invert it
        const int e = (byte & 4) | ((byte & 1) << 1) | ((byte >> 1) & 1);
        const int p = 4 * q + (e & 3) + 16 * (e >> 2);
        w |= vcode(p, ch) << (8 * b);
      }
      vtile[d] = w;
    }
  }
}

// ---------------------------------------------------------------- Freeze: bf16 stores
// mode 0: anchor store (tile u holds anchors 32u..32u+31); mode 1: window ring (tile u holds
// ring slots 32u..32u+31).  Positions past the count are written as zeros.
__device__ inline void freeze_bf16_tile(const CacheView& c, const uint16_t* __restrict__ k,
                                        const uint16_t* __restrict__ v, int len,
                                        const int32_t* __restrict__ anchors, int n_anchor, int mode, int tile,
                                        int hkv, int b) {
  __shared__ uint16_t vl[32][D + 8];
  const size_t hb = (size_t)b * c.Hkv + hkv;
  const int t = threadIdx.x;
  uint16_t *dk, *dv;
  size_t slab;
  if (mode == 0) { slab = (size_t)c.anchor_cap * D; dk = c.a_k + hb * slab; dv = c.a_v + hb * slab; }
  else { slab = (size_t)WIN * D; dk = c.w_k + hb * slab; dv = c.w_v + hb * slab; }
  // each thread: one position (t >> 3), 16 channels (t & 7)
  const int pl = t >> 3, cc = (t & 7) * 16;
  const int s = tile * 32 + pl;
  int pos = -1;
  if (mode == 0) {
    if (s < n_anchor) pos = anchors[hb * (size_t)n_anchor + s];
    if (pos >= len) pos = -1;  // contract violation: never read past the prefill buffer
  } else {
    if (len >= WIN) pos = (len - WIN) + ((s - len) % WIN + WIN) % WIN;
    else if (s < len) pos = s;
  }
  u32x4 kw0 = {0, 0, 0, 0}, kw1 = {0, 0, 0, 0}, vw0 = {0, 0, 0, 0}, vw1 = {0, 0, 0, 0};
  if (pos >= 0) {
    const size_t off = (hb * (size_t)len + pos) * D + cc;
    kw0 = *(const u32x4*)(k + off);
    kw1 = *(const u32x4*)(k + off + 8);
    vw0 = *(const u32x4*)(v + off);
    vw1 = *(const u32x4*)(v + off + 8);
  }
  *(u32x4*)(dk + kbf_index(s, cc)) = kw0;
  *(u32x4*)(dk + kbf_index(s, cc + 8)) = kw1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vl[pl][cc + 2 * e] = (uint16_t)(vw0[e] & 0xffff);
    vl[pl][cc + 2 * e + 1] = (uint16_t)(vw0[e] >> 16);
    vl[pl][cc + 8 + 2 * e] = (uint16_t)(vw1[e] & 0xffff);
    vl[pl][cc + 8 + 2 * e + 1] = (uint16_t)(vw1[e] >> 16);
  }
  if (mode == 0 && (t & 7) == 0 && s < c.anchor_cap) c.a_pos[hb * (size_t)c.anchor_cap + s] = pos;
  __syncthreads();
  // tile-transposed V: chunk (r, q, i) = 8 bf16 of channel 16r + i at the quad's 8 positions
  uint16_t* vt = dv + (size_t)tile * 4096;
  for (int ch = t; ch < 512; ch += 256) {
    const int r = ch >> 6, q = (ch >> 4) & 3, i = ch & 15;
    const int chn = 16 * r + i;
    u32x4 w;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const int ea = 2 * e2, eb = 2 * e2 + 1;
      const int pa = 4 * q + (ea & 3) + 16 * (ea >> 2), pb = 4 * q + (eb & 3) + 16 * (eb >> 2);
      w[e2] = (uint32_t)vl[pa][chn] | ((uint32_t)vl[pb][chn] << 16);
    }
    *(u32x4*)(vt + (size_t)ch * 8) = w;
  }
}

// Freeze's stores in one launch: workgroups x < n_at copy anchor tiles, the next WIN / 32 copy
// window tiles, the rest quantize 32-slot tiles.  The copies come first, so their memory
// traffic runs beside the quantizer's arithmetic instead of after it.
template <int BK, int BV>
__global__ __launch_bounds__(256) void freeze_kernel(CacheView c, const uint16_t* __restrict__ k,
                                                     const uint16_t* __restrict__ v, int len,
                                                     const int32_t* __restrict__ anchors, int n_anchor, int n_int4,
                                                     int n_at) {
  const int x = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
  if (x < n_at) freeze_bf16_tile(c, k, v, len, anchors, n_anchor, 0, x, hkv, b);
  else if (x < n_at + WIN / 32) freeze_bf16_tile(c, k, v, len, anchors, n_anchor, 1, x - n_at, hkv, b);
  else freeze_q_tile<BK, BV>(c, k, v, len, anchors, n_anchor, n_int4, x - n_at - WIN / 32, hkv, b);
}

// The rest of Freeze in one launch: workgroups [0, n_clear) clear the K and V staging stores
// (16-byte zero stores), the others fill the proxy ring with the last n queries of q_tail
// (16 threads per 128-channel row, 16 bytes each).
__global__ __launch_bounds__(256) void freeze_aux_kernel(CacheView c, size_t clear_vec, int n_clear,
                                                         const uint16_t* __restrict__ q_tail, int n_tail, int n) {
  const int t = threadIdx.x;
  if ((int)blockIdx.x < n_clear) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (size_t i = (size_t)blockIdx.x * 256 + t; i < clear_vec; i += (size_t)n_clear * 256) {
      ((u32x4*)c.s_k)[i] = z;
      ((u32x4*)c.s_v)[i] = z;
    }
    return;
  }
  const size_t idx = (size_t)(blockIdx.x - n_clear) * 256 + t;
  const size_t rows = (size_t)c.B * c.Hkv * c.G * n;
  const size_t r = idx >> 4;
  const int part = (int)(idx & 15);
  if (r >= rows) return;
  const size_t bh = r / n;  // b * Hq + hq
  const int j = (int)(r % n);
  const u32x4 w = *(const u32x4*)(q_tail + (bh * n_tail + (n_tail - n + j)) * D + 8 * part);
  *(u32x4*)(c.proxy_q + (bh * c.proxy_cap + j) * D + 8 * part) = w;
}

// ---------------------------------------------------------------- append
__global__ __launch_bounds__(128) void append_kernel(CacheView c, const uint16_t* __restrict__ k_t,
                                                     const uint16_t* __restrict__ v_t,
                                                     const uint16_t* __restrict__ q_t, int len, int n_staged,
                                                     int proxy_head) {
  const int hkv = blockIdx.x, b = blockIdx.y, ch = threadIdx.x;
  const size_t hb = (size_t)b * c.Hkv + hkv;
  const int r = len % WIN;
  uint16_t* wk = c.w_k + hb * (size_t)WIN * D;
  uint16_t* wv = c.w_v + hb * (size_t)WIN * D;
  if (len >= WIN) {  // position len - W leaves the window for staging slot n_staged
    uint16_t* sk = c.s_k + hb * (size_t)c.staging_cap * D;
    uint16_t* sv = c.s_v + hb * (size_t)c.staging_cap * D;
    sk[kbf_index(n_staged, ch)] = wk[kbf_index(r, ch)];
    sv[vbf_index(n_staged, ch)] = wv[vbf_index(r, ch)];
  }
  wk[kbf_index(r, ch)] = k_t[hb * D + ch];
  wv[vbf_index(r, ch)] = v_t[hb * D + ch];
  if (q_t) {
    const int Hq = c.Hkv * c.G;
    for (int j = 0; j < c.G; ++j) {
      const int hq = hkv * c.G + j;
      c.proxy_q[(((size_t)b * Hq + hq) * c.proxy_cap + proxy_head) * D + ch] = q_t[((size_t)b * Hq + hq) * D + ch];
    }
  }
}


}  // namespace

hipError_t launch_freeze(const CacheView& c, const uint16_t* k, const uint16_t* v, int len,
                         const int32_t* anchors, int n_anchor, const uint16_t* q_tail, int n_tail,
                         hipStream_t stream) {
  hipError_t e;
  const int P = len > WIN ? len - WIN : 0;
  const int n_int4 = P - n_anchor;
  const int n_at = (n_anchor + 31) / 32;
  {
    dim3 grid(n_at + WIN / 32 + (n_int4 > 0 ? (n_int4 + 31) / 32 : 0), c.Hkv, c.B);
    e = with_widths(c.bits, c.bits_v, [&](auto BK, auto BV) {
      hipLaunchKernelGGL((freeze_kernel<decltype(BK)::value, decltype(BV)::value>), grid, dim3(256), 0, stream, c, k,
                         v, len, anchors, n_anchor, n_int4 > 0 ? n_int4 : 0, n_at);
      return hipGetLastError();
    });
    if (e != hipSuccess) return e;
  }
  // staging bytes per store: a multiple of 16 (staging_cap is a multiple of 32)
  const size_t clear_vec = (size_t)c.B * c.Hkv * c.staging_cap * D * 2 / 16;
  const int n_clear = clear_vec ? (int)((clear_vec + 255) / 256 < 1024 ? (clear_vec + 255) / 256 : 1024) : 0;
  const int n = q_tail && n_tail > 0 ? (n_tail < c.proxy_cap ? n_tail : c.proxy_cap) : 0;
  const size_t proxy_threads = (size_t)c.B * c.Hkv * c.G * n * 16;
  const int n_proxy = (int)((proxy_threads + 255) / 256);
  if (n_clear + n_proxy > 0) {
    hipLaunchKernelGGL(freeze_aux_kernel, dim3(n_clear + n_proxy), dim3(256), 0, stream, c, clear_vec, n_clear,
                       q_tail, n_tail, n);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_append(const CacheView& c, const uint16_t* k_t, const uint16_t* v_t, const uint16_t* q_t,
                         int len, int n_staged, int proxy_head, hipStream_t stream) {
  hipLaunchKernelGGL(append_kernel, dim3(c.Hkv, c.B), dim3(D), 0, stream, c, k_t, v_t, q_t, len, n_staged,
                     proxy_head);
  return hipGetLastError();
}

}  // namespace hyq

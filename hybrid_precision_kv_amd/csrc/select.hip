// Vertical-line selector for gfx950.
//
// HyQuant paper ("HyQuant: Hybrid-Precision Quantization for LLM Attention"), §4.1 Eq. 4-5 and
// Alg. 1: the score of a candidate key is its attention probability summed over the proxy
// queries (here every proxy query of every Q head of the KV group, softmax over every cached
// key), and the anchors are the top-k candidates.
//
// Three passes per call, all keys in their stored precision:
//  1. row statistics: for each proxy row, running max and sum of exp over every key, one
//     partial per 256-key task;
//  2. merge of the partials into each row's max and 1 / normaliser;
//  3. column sums: S(key) = sum over rows of exp(score - max) / normaliser, written by
//     position;
// then a radix select (one workgroup per head) keeps the k largest S, ties to the lower
// position, emitted in ascending position order.
//
// Q.K^T runs on MFMA f32_16x16x32 with 16 keys x 16 proxy rows per instruction group.  INT4 keys
// use one MFMA per 32-channel group (separate accumulators) so each group's scale and min apply
// exactly: q.k = sum_g s_g (q_g . code_g) + m_g sum(q_g); their codes enter as f16 subnormals as
// in the decode kernel.  Proxy rows are staged through LDS one 16-row block at a time, shared by
// the 8 waves of a workgroup.
#include "hyq_common.h"
#include "hyq_launch.h"

namespace hyq {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int SW = 4;             // waves per workgroup
constexpr int KEYS_WG = SW * 32;  // keys per task (one 32-key tile per wave)

__device__ inline f16x8 codes_to_f16(uint32_t x) {
  const uint32_t y = x >> 8;
  u32x4 a;
  a[0] = x & 0x000F000Fu;
  a[1] = x & 0x00F000F0u;
  a[2] = y & 0x000F000Fu;
  a[3] = y & 0x00F000F0u;
  return __builtin_bit_cast(f16x8, a);
}
__device__ inline f16x8 codes8_to_f16(uint32_t x0, uint32_t x1) {  // bytes 0,2 | 1,3 | 4,6 | 5,7
  u32x4 a;
  a[0] = x0 & 0x00FF00FFu;
  a[1] = (x0 >> 8) & 0x00FF00FFu;
  a[2] = x1 & 0x00FF00FFu;
  a[3] = (x1 >> 8) & 0x00FF00FFu;
  return __builtin_bit_cast(f16x8, a);
}
__device__ inline float half_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffff)); }
__device__ inline float half_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

// Key segments of a task list.  Dense mode: one segment of bf16 rows (positions 0..L-1).  Cache
// mode: INT4 slots, anchors, staging, window (in that order); tiles never straddle segments.
struct KeySrc {
  int kind;         // 0 = INT4 tile record, 1 = bf16 tile (cache layout), 2 = dense bf16 rows
  int tile;         // tile index inside the segment (32 keys)
  int count;        // valid keys in the segment
  int seg;          // 0 int4, 1 anchors, 2 staging, 3 window, 4 dense
};

__device__ inline KeySrc key_src(const SelectParams& p, int gt) {
  KeySrc s;
  if (p.dense_k) { s.kind = 2; s.tile = gt; s.count = p.len; s.seg = 4; return s; }
  const int T4 = (p.n_int4 + 31) >> 5, TA = (p.n_anchor + 31) >> 5, TS = (p.n_staged + 31) >> 5;
  if (gt < T4) { s.kind = 0; s.tile = gt; s.count = p.n_int4; s.seg = 0; return s; }
  gt -= T4;
  if (gt < TA) { s.kind = 1; s.tile = gt; s.count = p.n_anchor; s.seg = 1; return s; }
  gt -= TA;
  if (gt < TS) { s.kind = 1; s.tile = gt; s.count = p.n_staged; s.seg = 2; return s; }
  gt -= TS;
  s.kind = 1; s.tile = gt; s.count = p.n_win; s.seg = 3;
  return s;
}

// Proxy row r of head block: (Q head inside the group, proxy index).  Returns the bf16 row.
__device__ inline const uint16_t* proxy_row(const SelectParams& p, int b, int hkv, int r) {
  const int h = r / p.n_proxy, i = r % p.n_proxy;
  const int Hq = p.Hkv * p.G;
  return p.proxy + (((size_t)b * Hq + (size_t)hkv * p.G + h) * p.proxy_stride + i) * D;
}

// Operand prep, once per call: proxy rows in the two B-operand orders of the score MFMAs,
// per 16-row block rb and entry idx = 64 g + 16 q4 + n (row 16 rb + n, channels 32 g + 8 q4 ..
// + 7): pq16 = f16 with the nibble-pair channel order and 1/16 on k-slots 2,3,6,7 (INT4 keys;
// INT8 keys: the byte-pair order, no factor),
// pqbf = bf16 in natural order (bf16 keys).  Rows >= R are zero.  Also the per-row group sums
// qsum[r][g] = 2^-24 sum_{c in g} q[r][c] (fp32 of the f16-rounded q, as the MFMA uses it, in
// the units of the subnormal f16 codes).
__global__ __launch_bounds__(256) void select_prep_kernel(SelectParams p) {
  const int hb = blockIdx.y, b = hb / p.Hkv, hkv = hb % p.Hkv;
  const int R = p.n_proxy * p.G, RB = (R + 15) >> 4;
  f16x8* pq16 = (f16x8*)p.pq16 + (size_t)hb * p.rb_stride * 256;
  bf16x8* pqbf = (bf16x8*)p.pqbf + (size_t)hb * p.rb_stride * 256;
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < RB * 256; t += gridDim.x * blockDim.x) {
    const int rb = t >> 8, idx = t & 255;
    const int g = idx >> 6, ln = idx & 63, n = ln & 15, q4 = ln >> 4;
    const int r = 16 * rb + n;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (r < R) w = *(const u32x4*)(proxy_row(p, b, hkv, r) + 32 * g + 8 * q4);
    f16x8 h;
    if (p.bits == 2) {
      // 2-bit keys: lane quad q4 takes the group's channels 16 (q4 >> 1) + code2_of(q4 & 1, e),
      // times 4^-(e >> 1)
      u32x4 w2[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
      if (r < R) {
        w2[0] = *(const u32x4*)(proxy_row(p, b, hkv, r) + 32 * g + 16 * (q4 >> 1));
        w2[1] = *(const u32x4*)(proxy_row(p, b, hkv, r) + 32 * g + 16 * (q4 >> 1) + 8);
      }
      float f[16];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t x = w2[e >> 2][e & 3];
        f[2 * e] = bf16_bits_to_f32((uint16_t)(x & 0xffff));
        f[2 * e + 1] = bf16_bits_to_f32((uint16_t)(x >> 16));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float fac = (e & 6) == 0 ? 1.0f : (e & 6) == 2 ? 0.25f : (e & 6) == 4 ? 0.0625f : 0.015625f;
        h[e] = (_Float16)(f[code2_of(q4 & 1, e)] * fac);
      }
    } else {
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = bf16_bits_to_f32((uint16_t)(w[e] & 0xffff));
        f[2 * e + 1] = bf16_bits_to_f32((uint16_t)(w[e] >> 16));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        h[e] = p.bits == 8 ? (_Float16)f[kslot_byte(e)] : (_Float16)(f[kslot_nibble(e)] * ((e & 2) ? 0.0625f : 1.0f));
    }
    pq16[t] = h;
    pqbf[t] = __builtin_bit_cast(bf16x8, w);
  }
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < R * 4; idx += gridDim.x * blockDim.x) {
    const int r = idx >> 2, g = idx & 3;
    const uint16_t* row = proxy_row(p, b, hkv, r) + 32 * g;
    float s = 0.f;
    for (int c = 0; c < 32; ++c) s += (float)(_Float16)bf16_bits_to_f32(row[c]);
    p.qsum[(size_t)hb * R * 4 + idx] = s * (1.0f / 16777216.0f);  // in the codes' 2^-24 units
  }
}

// A operands of this wave's 32 keys.  Lane (n, q4): key rows n and 16 + n of the tile; for
// INT4 keys instruction g covers group g (channels 32g + 8q4 + nibble order), the group scales
// of the lane's output keys 4q4 + j are kept in fp32, and the group minima enter one fp32 MFMA
// (A = min of key l%16, group l/16; B = the rows' group sums).
struct KeyOps4 {
  f16x8 a[2][4];     // [block][group]
  float sc[2][4][4]; // scale [block][group][j] of keys 4q4 + j
  float ma[2];       // min of (key lane%16, group lane/16), per block
};
struct KeyOpsB {
  bf16x8 a[2][4];    // [block][8-channel chunk]
};

template <int BK, int BV>
__device__ inline void load_keys4(const SelectParams& p, const KeySrc& ks, size_t hb, int lane, KeyOps4& o) {
  typedef QL<BK, BV> L;
  const int n = lane & 15, q4 = lane >> 4;
  const uint8_t* rec = p.int4 + hb * (size_t)p.int4_cap * L::SLOT + (size_t)ks.tile * L::TB;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // key n, group g: channels 8 q4 .. + 7 (a dword of nibbles, INT4; two of bytes, INT8), or
      // the 2-bit channel set of step q4 (half q4 & 1 of dword q4 >> 1)
      const uint8_t* ch = rec + blk * 64 * L::CB + g * 16 * L::CB + n * L::CB;
      if constexpr (BK == 4) o.a[blk][g] = codes_to_f16(*(const uint32_t*)(ch + 4 * q4));
      else if constexpr (BK == 8) o.a[blk][g] = codes8_to_f16(((const uint32_t*)(ch + 8 * q4))[0], ((const uint32_t*)(ch + 8 * q4))[1]);
      else o.a[blk][g] = codes2_to_f16(*(const uint32_t*)(ch + 4 * (q4 >> 1)), q4 & 1);
    }
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x4 w = *(const u32x4*)(rec + L::KSM + blk * 256 + g * 64 + q4 * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) o.sc[blk][g][j] = half_lo(w[j]);
    }
    o.ma[blk] = half_hi(*(const uint32_t*)(rec + L::KSM + blk * 256 + 4 * lane));
  }
}

__device__ inline void load_keysB(const SelectParams& p, const KeySrc& ks, size_t hb, int lane, KeyOpsB& o) {
  const int n = lane & 15, q4 = lane >> 4;
  if (ks.kind == 1) {
    const uint16_t* base;
    size_t slab;
    if (ks.seg == 1) { slab = (size_t)p.anchor_cap * D; base = p.a_k; }
    else if (ks.seg == 2) { slab = (size_t)p.staging_cap * D; base = p.s_k; }
    else { slab = (size_t)WIN * D; base = p.w_k; }
    const uint16_t* t = base + hb * slab + (size_t)ks.tile * 4096 + lane * 8;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) o.a[blk][tt] = *(const bf16x8*)(t + (blk * 4 + tt) * 512);
  } else {
    // dense rows: key row (tile*32 + 16 blk + n), channels 32 q4 + 8 tt .. +7
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      int key = ks.tile * 32 + 16 * blk + n;
      if (key >= ks.count) key = ks.count - 1;  // masked later; stay inside the buffer
      const uint16_t* row = p.dense_k + (hb * (size_t)p.len + key) * D + 32 * q4;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) o.a[blk][tt] = *(const bf16x8*)(row + 8 * tt);
    }
  }
}

// Raw scores of this lane's 8 (key, row) pairs for one row block -- keys 4q4 + j (block 0) and
// 16 + 4q4 + j (block 1), row r0 + n -- in units where SCALE4 / SCALEB (log2 e / sqrt(128),
// times 2^24 for the INT4 codes) turns them into log2-domain scores.
// INT4: q.k = sum_g s_g (q_g . code_g) + sum_g m_g qsum_g; codes carry 2^-24 and qsb carries
// the rows' group sums times 2^-24 (B operand: group lane/16, row lane%16).
constexpr float SCALE4 = LOG2E * 0.08838834764831845f * 16777216.0f;
constexpr float SCALEB = LOG2E * 0.08838834764831845f;
__device__ inline void scores4(const KeyOps4& o, const f16x8 (&bq)[4], float qsb, float (&sc)[8]) {
  f32x4 v0 = __builtin_amdgcn_mfma_f32_16x16x4f32(o.ma[0], qsb, (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  f32x4 v1 = __builtin_amdgcn_mfma_f32_16x16x4f32(o.ma[1], qsb, (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  f32x4 acc0[4], acc1[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    acc0[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(o.a[0][g], bq[g], (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    acc1[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(o.a[1][g], bq[g], (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      v0[j] = fmaf(o.sc[0][g][j], acc0[g][j], v0[j]);
      v1[j] = fmaf(o.sc[1][g][j], acc1[g][j], v1[j]);
    }
    sc[j] = v0[j];
    sc[4 + j] = v1[j];
  }
}

__device__ inline void scoresB(const KeyOpsB& o, const bf16x8 (&bq)[4], float (&sc)[8]) {
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a[0][tt], bq[tt], a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a[1][tt], bq[tt], a1, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sc[j] = a0[j];
    sc[4 + j] = a1[j];
  }
}

// B operands (and per-row values) of row block rb, loaded one block ahead of their use.
// INT4: entry [group g][lane]; bf16: the lane's rows at channels 32 q4 + 8 tt .. +7 =
// prepared entry [group q4][16 tt + n].
// Every load is unconditional and used as loaded (row indices past R are clamped: those rows
// are masked by the caller), so a block's loads stay in flight while the previous block runs.
template <int PASS, int KIND>
struct RowBlock {
  f16x8 b4[KIND == 0 ? 4 : 1];
  bf16x8 bb[KIND == 0 ? 1 : 4];
  float qsb, M;  // M: the row's max plus log2 of its normaliser (pass 2)
};
template <int PASS, int KIND>
__device__ inline void load_rows(const SelectParams& p, size_t hb, int R, int rb, int lane, RowBlock<PASS, KIND>& x) {
  const int n = lane & 15, q4 = lane >> 4;
  const int r = min(rb * 16 + n, R - 1);
  if constexpr (KIND == 0) {
    const f16x8* pq16 = (const f16x8*)p.pq16 + (hb * p.rb_stride + rb) * 256;
#pragma unroll
    for (int g = 0; g < 4; ++g) x.b4[g] = pq16[g * 64 + lane];
    x.qsb = p.qsum[(hb * R + r) * 4 + q4];  // minima MFMA B operand: row lane%16, group lane/16
  } else {
    const bf16x8* pqbf = (const bf16x8*)p.pqbf + (hb * p.rb_stride + rb) * 256;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) x.bb[tt] = pqbf[q4 * 64 + 16 * tt + n];
  }
  if (PASS == 2) x.M = p.rowstat[(hb * R + r) * 2];
}

// Sweep of the proxy rows for one wave's keys (KIND 0: INT4 tile, 1: bf16 keys).  PASS 1
// writes the wave's per-row (max, sum exp2) partial to red[wave][r]; PASS 2 accumulates the
// column sums of the lane's 8 keys into colsum.
// FULL: all 32 keys of the tile are valid (every tile but a segment's last)
template <int PASS, int KIND, bool FULL, int BK, int BV>
__device__ inline void sweep(const SelectParams& p, const KeySrc& ks, size_t hb, int lane, int wave,
                             const bool (&valid)[8], float* red, float (&colsum)[8]) {
  const int n = lane & 15, q4 = lane >> 4;
  const int R = p.n_proxy * p.G;
  const int RB = (R + 15) >> 4;
  const float c = KIND == 0 ? SCALE4 : SCALEB;
  KeyOps4 k4;
  KeyOpsB kb;
  if (KIND == 0) load_keys4<BK, BV>(p, ks, hb, lane, k4);
  else load_keysB(p, ks, hb, lane, kb);
  auto ok = [&](int j) { return FULL || valid[j]; };
  auto block = [&](const RowBlock<PASS, KIND>& x, int rb) {
    const int r = rb * 16 + n;
    const bool rvalid = r < R;
    float v[8];
    if constexpr (KIND == 0) scores4(k4, x.b4, x.qsb, v);
    else scoresB(kb, x.bb, v);
    if (PASS == 1) {
      float m = -INFINITY;  // max of the raw scores; c > 0, so c * max = max of the scaled ones
#pragma unroll
      for (int j = 0; j < 8; ++j) m = ok(j) ? fmaxf(m, v[j]) : m;
      m = col4_max(m) * c;
      float s = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int j = 0; j < 8; ++j) s += ok(j) ? __builtin_amdgcn_exp2f(fmaf(v[j], c, -m)) : 0.f;
      }
      s = col4_sum(s);
      if (q4 == 0 && rvalid) {
        red[((size_t)wave * R + r) * 2] = m;
        red[((size_t)wave * R + r) * 2 + 1] = s;
      }
    } else if (rvalid) {
#pragma unroll
      for (int j = 0; j < 8; ++j) colsum[j] += ok(j) ? __builtin_amdgcn_exp2f(fmaf(v[j], c, -x.M)) : 0.f;
    }
  };
  // two row blocks in flight: the loads of block rb + 1 are issued before block rb runs.  The
  // loads are unconditional (past the last block they re-read it) so that the compiler can
  // count them and wait only for the block about to run.
  RowBlock<PASS, KIND> b0, b1;
  load_rows(p, hb, R, 0, lane, b0);
  for (int rb = 0; rb < RB; rb += 2) {
    load_rows(p, hb, R, min(rb + 1, RB - 1), lane, b1);
    block(b0, rb);
    if (rb + 1 >= RB) break;
    load_rows(p, hb, R, min(rb + 2, RB - 1), lane, b0);
    block(b1, rb + 1);
  }
}

// One pass over the keys.  A wave owns one 32-key tile and sweeps the proxy rows in 16-row
// blocks, reading the prepared B operands straight from L2 (no LDS staging, no barrier inside
// the sweep).  PASS 1: per-row (max, sum exp2) over the workgroup's keys -- each wave keeps its
// partial of every row in LDS, merged once at the end; PASS 2: column sums by position.
template <int PASS, int BK, int BV>
__global__ __launch_bounds__(SW * 64) __attribute__((amdgpu_waves_per_eu(3))) void select_pass_kernel(SelectParams p) {
  extern __shared__ float red[];  // PASS 1: [SW][R][2]
  const int task = blockIdx.x, hb = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, q4 = lane >> 4;
  const int R = p.n_proxy * p.G;
  const int gt = task * SW + wave;  // this wave's global tile
  const bool has = gt < p.n_tiles;
  KeySrc ks;
  if (has) ks = key_src(p, gt);
  // validity of this lane's 8 keys
  bool valid[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int key = (has ? ks.tile * 32 : 0) + ((j >> 2) << 4) + 4 * q4 + (j & 3);
    valid[j] = has && key < ks.count;
  }
  float colsum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (has) {
    const bool full = (ks.tile + 1) * 32 <= ks.count;
    if (ks.kind == 0) {
      if (full) sweep<PASS, 0, true, BK, BV>(p, ks, hb, lane, wave, valid, red, colsum);
      else sweep<PASS, 0, false, BK, BV>(p, ks, hb, lane, wave, valid, red, colsum);
    } else {
      if (full) sweep<PASS, 1, true, BK, BV>(p, ks, hb, lane, wave, valid, red, colsum);
      else sweep<PASS, 1, false, BK, BV>(p, ks, hb, lane, wave, valid, red, colsum);
    }
  } else if (PASS == 1 && q4 == 0) {
    for (int r = n; r < R; r += 16) {  // no keys: empty partials
      red[((size_t)wave * R + r) * 2] = -INFINITY;
      red[((size_t)wave * R + r) * 2 + 1] = 0.f;
    }
  }
  if (PASS == 1) {
    __syncthreads();
    for (int rr = threadIdx.x; rr < R; rr += blockDim.x) {
      float M = -INFINITY;
      for (int w2 = 0; w2 < SW; ++w2) M = fmaxf(M, red[((size_t)w2 * R + rr) * 2]);
      float S = 0.f;
      if (M != -INFINITY)
        for (int w2 = 0; w2 < SW; ++w2) {
          const float m2 = red[((size_t)w2 * R + rr) * 2];
          if (m2 != -INFINITY) S += red[((size_t)w2 * R + rr) * 2 + 1] * __builtin_amdgcn_exp2f(m2 - M);
        }
      float* dst = p.rowpart + (((size_t)hb * R + rr) * p.n_tasks + task) * 2;  // [H][R][task]
      dst[0] = M;
      dst[1] = S;
    }
  }
  if (PASS == 2 && has) {
    // sum over the 16 rows of each row block held by lanes n = 0..15 (same keys)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = colsum[j];
      v += shfl_xor_f(v, 1);
      v += shfl_xor_f(v, 2);
      v += shfl_xor_f(v, 4);
      v += shfl_xor_f(v, 8);
      colsum[j] = v;
    }
    if (n == 0 && ks.seg != 3) {
      const int P = p.len - WIN > 0 ? p.len - WIN : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (!valid[j]) continue;
        const int key = ks.tile * 32 + ((j >> 2) << 4) + 4 * q4 + (j & 3);
        int pos;
        if (ks.seg == 4) pos = key;
        else if (ks.seg == 0) pos = p.slot_pos[hb * (size_t)p.int4_cap + key];
        else if (ks.seg == 1) pos = p.a_pos[hb * (size_t)p.anchor_cap + key];
        else pos = P - p.n_staged + key;  // staging slot -> position
        if (pos >= 0 && pos < P) p.scores[hb * (size_t)P + pos] = colsum[j];
      }
    }
  }
}

// row partials -> (max + log2 normaliser, 1 / normaliser) per row: one wave per row, lanes
// over the tasks
__global__ __launch_bounds__(256) void select_rowmerge_kernel(SelectParams p) {
  const int hb = blockIdx.y, lane = threadIdx.x & 63;
  const int R = p.n_proxy * p.G;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const float* part = p.rowpart + ((size_t)hb * R + r) * p.n_tasks * 2;  // this row's task partials
  float M = -INFINITY;
  for (int t = lane; t < p.n_tasks; t += 64) M = fmaxf(M, part[(size_t)t * 2]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, shfl_xor_f(M, o));
  float S = 0.f;
  if (M != -INFINITY) {
    for (int t = lane; t < p.n_tasks; t += 64) {
      const float m = part[(size_t)t * 2];
      if (m != -INFINITY) S += part[(size_t)t * 2 + 1] * __builtin_amdgcn_exp2f(m - M);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) S += shfl_xor_f(S, o);
  if (lane == 0) {  // exp2(s - M') = exp2(s - M) / S
    p.rowstat[((size_t)hb * R + r) * 2] = S > 0.f ? M + __log2f(S) : INFINITY;
    p.rowstat[((size_t)hb * R + r) * 2 + 1] = 1.0f / S;
  }
}

// ---------------------------------------------------------------- top-k (radix select)
// One workgroup of 1024 threads per row of P unsigned keys (scores >= 0 as their bit patterns,
// or keys already mapped to an order-preserving unsigned form).  Keeps every key above the
// k-th largest value T and the lowest positions equal to T, written in ascending position order.
//   * Rows of up to 32768 keys are staged once in LDS (one padding word after every 32 keys, so
//     strided and per-thread-contiguous reads are both free of bank conflicts); longer rows are
//     re-read from global memory.
//   * Radix select on digits of 11, 8, 8 and 5 bits.  The first digit is counted over every
//     key; the keys that share the chosen first digit (a few per cent) are copied to a
//     candidate list, and the three later digits scan only that list.
//   * Masked lanes add to per-lane dummy counters and write to per-lane dummy slots, and loads
//     past the row are clamped, so no load or LDS atomic sits behind a branch.
//   * Ordered output: each thread describes its contiguous positions by bit masks of the keys
//     above and equal to T; two block prefix sums give every thread its output offset.
// Every loop is rolled or unrolled by at most 8: the code runs once per workgroup, so its
// size sets the instruction-fetch time.
constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_BATCH = 8 * TK_THREADS;  // keys per batch of the strided passes
constexpr int TK_LDS_KEYS = 32768;        // rows up to this length are staged in LDS
constexpr int TK_BINS = 2048;             // first digit: bits 31..21
constexpr int TK_CAND = 4096;             // keys kept after the first digit
constexpr int TK_TRASH = 64;              // per-lane dummy counters / slots for masked lanes

__device__ inline int wave_scan_incl(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x;
}
__device__ inline int block_scan_excl(int v, int* wtot) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int incl = wave_scan_incl(v);
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  const int t = wave_scan_incl(lane < TK_WAVES ? wtot[lane] : 0);
  const int before = wv ? __builtin_amdgcn_readlane(t, wv - 1) : 0;
  __syncthreads();
  return before + incl - v;
}
__device__ inline int mbcnt64(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
__device__ inline int pad32(int i) { return i + (i >> 5); }
// hist[bin] += 1 for every lane (masked lanes pass their own dummy bin).  The lanes that share
// the first lane's bin are added by one of them, so keys concentrated in a few bins do not
// serialise on one LDS address; the atomic is issued by every lane, without a branch.
__device__ inline void hist_add(int* hist, int bin, int lane) {
  const int b0 = __builtin_amdgcn_readfirstlane(bin);
  const uint64_t same = __builtin_amdgcn_ballot_w64(bin == b0);
  const bool grouped = bin == b0, first = grouped && mbcnt64(same) == 0;
  atomicAdd(&hist[grouped && !first ? TK_BINS + lane : bin], grouped ? (first ? (int)__builtin_popcountll(same) : 0) : 1);
}

template <bool LDS>
__device__ void topk_row(const uint32_t* g, int P, int k, int32_t* out) {
  extern __shared__ uint32_t dyn[];  // LDS: keys of the batches covering P, padded
  __shared__ int hist[TK_BINS + TK_TRASH];
  __shared__ uint32_t cand[TK_CAND + TK_TRASH];
  __shared__ int tsum[TK_WAVES];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_need, s_ncand, s_bin;  // s_bin: keys in the chosen bin of the last digit
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nb = (P + TK_BATCH - 1) / TK_BATCH;
  // key at i for any i of the covered batches: staged zeros past P (LDS) or a clamped read
  // (global; the caller ignores it), so no load sits behind a branch
  auto key = [&](int i) -> uint32_t {
    if constexpr (LDS) return dyn[pad32(i)]; else return g[min(i, P - 1)];
  };
  for (int i = tid; i < TK_BINS + TK_TRASH; i += TK_THREADS) hist[i] = 0;
  if (tid == 0) s_ncand = 0;
  __syncthreads();
  // ---- stage (LDS) and count the first digit, bits 31..21
  for (int b = tid; b < nb * TK_BATCH; b += TK_BATCH) {
    uint32_t x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = g[min(b + u * TK_THREADS, P - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = b + u * TK_THREADS;
      if constexpr (LDS) dyn[pad32(i)] = i < P ? x[u] : 0u;
      hist_add(hist, i < P ? (int)(x[u] >> 21) : TK_BINS + lane, lane);
    }
  }
  __syncthreads();
  {
    const int d0 = TK_BINS - 1 - 2 * tid;  // thread t owns digits d0, d0 - 1
    const int c0 = hist[d0], c1 = hist[d0 - 1];
    const int run = block_scan_excl(c0 + c1, tsum);
    if (tid < 256) hist[tid] = 0;
    if (run < k && run + c0 >= k) {
      s_prefix = (uint32_t)d0 << 21;
      s_need = k - run;
      s_bin = c0;
    } else if (run + c0 < k && (run + c0 + c1 >= k || d0 == 1)) {
      s_prefix = (uint32_t)(d0 - 1) << 21;
      s_need = k - run - c0;
      s_bin = c1;
    }
    if (tid == 0) s_mask = 0xFFE00000u;
    __syncthreads();
  }
  // ---- digits 20..13, 12..5, 4..0 over the keys with the prefix; wave 0 finds each.  As
  // soon as the keys with the current prefix fit the candidate list they are copied there
  // (one LDS atomic per wave and batch) and the remaining digits scan only them.
  bool use_cand = false;
  int ncand = 0;
  for (int pass = 1; pass < 4; ++pass) {
    const int shift = pass == 1 ? 13 : pass == 2 ? 5 : 0;
    const int nbins = pass == 3 ? 32 : 256;
    if (!use_cand && s_bin <= TK_CAND) {
      const uint32_t prefix = s_prefix, mask = s_mask;
      for (int b = tid; b < nb * TK_BATCH; b += TK_BATCH) {
        uint32_t x[8];
        uint64_t m[8];
        int cnt[8], tot = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = b + u * TK_THREADS;
          x[u] = key(i);
          m[u] = __builtin_amdgcn_ballot_w64(i < P && (x[u] & mask) == prefix);
          cnt[u] = tot;
          tot += (int)__builtin_popcountll(m[u]);
        }
        if (tot) {
          int base = 0;
          if (lane == 0) base = atomicAdd(&s_ncand, tot);
          base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const bool mine = (m[u] >> lane) & 1u;
            const int slot = base + cnt[u] + mbcnt64(m[u]);
            cand[mine && slot < TK_CAND ? slot : TK_CAND + lane] = x[u];
          }
        }
      }
      __syncthreads();
      ncand = min(s_ncand, TK_CAND);
      use_cand = true;
    }
    const uint32_t prefix = s_prefix, mask = s_mask;
    if (use_cand) {
      for (int i = tid; i < ncand; i += TK_THREADS) {
        const uint32_t x = cand[i];
        hist_add(hist, (x & mask) == prefix ? (int)((x >> shift) & (nbins - 1)) : TK_BINS + lane, lane);
      }
    } else {
      for (int b = tid; b < nb * TK_BATCH; b += TK_BATCH) {
        uint32_t x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = key(b + u * TK_THREADS);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bool in = b + u * TK_THREADS < P && (x[u] & mask) == prefix;
          hist_add(hist, in ? (int)((x[u] >> shift) & (nbins - 1)) : TK_BINS + lane, lane);
        }
      }
    }
    __syncthreads();
    if (wv == 0) {  // lane l owns digits nbins - 1 - 4 l - r (r < 4); clears them for the next
      const int need = s_need;
      int c4[4], h = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = nbins - 1 - 4 * lane - r;
        c4[r] = d >= 0 ? hist[d] : 0;
        h += c4[r];
        if (d >= 0) hist[d] = 0;
      }
      int run = wave_scan_incl(h) - h;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = nbins - 1 - 4 * lane - r;
        if (d >= 0 && run < need && (run + c4[r] >= need || d == 0)) {
          s_prefix = prefix | ((uint32_t)d << shift);
          s_mask = mask | ((uint32_t)(nbins - 1) << shift);
          s_need = need - run;
          s_bin = c4[r];
        }
        run += c4[r];
      }
    }
    __syncthreads();
  }
  const uint32_t T = s_prefix;
  const int need_eq = s_need;
  // ---- ordered compaction: thread t owns the contiguous positions [lo, hi), in chunks of 32
  // described by bit masks of the keys above T and equal to T
  const int per = (P + TK_THREADS - 1) / TK_THREADS;
  const int lo = min(P, tid * per), hi = min(P, lo + per);
  auto masks = [&](int c, uint32_t& gtm, uint32_t& eqm) {
    const int n = hi - c;
    const uint32_t inm = n >= 32 ? ~0u : ((1u << n) - 1u);
    gtm = 0u;
    eqm = 0u;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const uint32_t x = key(c + e);
      gtm |= x > T ? (1u << e) : 0u;
      eqm |= x == T ? (1u << e) : 0u;
    }
    gtm &= inm;
    eqm &= inm;
  };
  uint32_t gt0 = 0u, eq0 = 0u;  // the first chunk's masks, kept for the output
  int n_gt = 0, n_eq = 0;
  for (int c = lo; c < hi; c += 32) {
    uint32_t gtm, eqm;
    masks(c, gtm, eqm);
    if (c == lo) { gt0 = gtm; eq0 = eqm; }
    n_gt += __builtin_popcount(gtm);
    n_eq += __builtin_popcount(eqm);
  }
  const int eq_before = block_scan_excl(n_eq, tsum);
  int take_eq = need_eq - eq_before;
  take_eq = take_eq < 0 ? 0 : (take_eq > n_eq ? n_eq : take_eq);
  int o = block_scan_excl(n_gt + take_eq, tsum);
  for (int c = lo; c < hi; c += 32) {
    uint32_t gtm = gt0, eqm = eq0;
    if (c != lo) masks(c, gtm, eqm);
    uint32_t sel = gtm;
    while (take_eq > 0 && eqm) {  // the lowest positions equal to T
      sel |= eqm & (0u - eqm);
      eqm &= eqm - 1u;
      --take_eq;
    }
    while (sel) {
      const int e = __builtin_ctz(sel);
      sel &= sel - 1u;
      if (o < k) out[o] = c + e;
      ++o;
    }
  }
}


template <bool LDS>
__global__ __launch_bounds__(TK_THREADS) void topk_kernel(const uint32_t* keys, int P, int k, int32_t* idx) {
  topk_row<LDS>(keys + blockIdx.x * (size_t)P, P, k, idx + blockIdx.x * (size_t)k);
}

}  // namespace

hipError_t launch_select(SelectParams p, hipStream_t stream) {
  const int R = p.n_proxy * p.G;
  const int H = p.B * p.Hkv;
  hipError_t e;
  const int RB = (R + 15) / 16;
  hipLaunchKernelGGL(select_prep_kernel, dim3((RB * 256 + 255) / 256, H), dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 grid(p.n_tasks, H);
  e = with_widths(p.bits, p.bits_v, [&](auto BK, auto BV) {
    hipLaunchKernelGGL((select_pass_kernel<1, decltype(BK)::value, decltype(BV)::value>), grid, dim3(SW * 64),
                       (size_t)SW * R * 2 * sizeof(float), stream, p);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_rowmerge_kernel, dim3((R + 3) / 4, H), dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = with_widths(p.bits, p.bits_v, [&](auto BK, auto BV) {
    hipLaunchKernelGGL((select_pass_kernel<2, decltype(BK)::value, decltype(BV)::value>), grid, dim3(SW * 64), 0,
                       stream, p);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  if (p.k > 0) return launch_topk_keys((const uint32_t*)p.scores, p.len - WIN, p.k, H, p.idx_out, stream);
  return hipSuccess;
}

int select_task_count(int n_tiles) { return (n_tiles + SW - 1) / SW; }

hipError_t launch_topk_keys(const uint32_t* keys, int P, int k, int rows, int32_t* idx_out, hipStream_t stream) {
  if (P <= TK_LDS_KEYS) {
    // staged batches of TK_BATCH keys, one padding word per 32
    const size_t lds = (size_t)((P + TK_BATCH - 1) / TK_BATCH) * TK_BATCH / 32 * 33 * sizeof(uint32_t);
    hipLaunchKernelGGL(topk_kernel<true>, dim3(rows), dim3(TK_THREADS), lds, stream, keys, P, k, idx_out);
  } else {
    hipLaunchKernelGGL(topk_kernel<false>, dim3(rows), dim3(TK_THREADS), 0, stream, keys, P, k, idx_out);
  }
  return hipGetLastError();
}

}  // namespace hyq

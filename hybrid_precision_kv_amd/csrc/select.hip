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
constexpr int SW = 8;             // waves per workgroup
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

// Stage proxy rows [r0, r0+16) into LDS in the two operand orders: f16 with the nibble-pair
// channel order and 1/16 on k-slots 2,3,6,7 (INT4 keys), and bf16 natural order (bf16 keys).
// Layout: [group g][lane = 16*q4 + n][8]: lane (n, q4) of group g holds row r0+n, channels
// 32g + 8q4 .. +7.  Rows >= R are zero.
__device__ inline void stage_rows(const SelectParams& p, int b, int hkv, int r0, int R, f16x8* s16, bf16x8* sbf) {
  for (int idx = threadIdx.x; idx < 4 * 64; idx += blockDim.x) {
    const int g = idx >> 6, ln = idx & 63, n = ln & 15, q4 = ln >> 4;
    const int r = r0 + n;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (r < R) w = *(const u32x4*)(proxy_row(p, b, hkv, r) + 32 * g + 8 * q4);
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_bits_to_f32((uint16_t)(w[e] & 0xffff));
      f[2 * e + 1] = bf16_bits_to_f32((uint16_t)(w[e] >> 16));
    }
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (_Float16)(f[kslot_nibble(e)] * ((e & 2) ? 0.0625f : 1.0f));
    s16[idx] = h;
    sbf[idx] = __builtin_bit_cast(bf16x8, w);
  }
}

// Per-row group sums sum_{c in g} q[r][c] (fp32 of the f16-rounded q, as the MFMA uses it),
// computed once per call into qsum[hb][R][4].
__global__ __launch_bounds__(256) void select_qsum_kernel(SelectParams p) {
  const int hb = blockIdx.y, b = hb / p.Hkv, hkv = hb % p.Hkv;
  const int R = p.n_proxy * p.G;
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < R * 4; idx += gridDim.x * blockDim.x) {
    const int r = idx >> 2, g = idx & 3;
    const uint16_t* row = proxy_row(p, b, hkv, r) + 32 * g;
    float s = 0.f;
    for (int c = 0; c < 32; ++c) s += (float)(_Float16)bf16_bits_to_f32(row[c]);
    p.qsum[(size_t)hb * R * 4 + idx] = s;
  }
}

// A operands and (scale, min) of this wave's 32 keys.  Lane (n, q4): key rows n and 16 + n of
// the tile; for INT4 keys instruction g covers group g (channels 32g + 8q4 + nibble order).
struct KeyOps {
  f16x8 a4[2][4];   // INT4: [block][group]
  bf16x8 ab[2][4];  // bf16: [block][8-channel chunk]
  u32x4 sm0[4], sm1[4];  // INT4: (scale, min) of output rows 4q4..4q4+3, [group], blocks 0 / 1
};

__device__ inline void load_keys(const SelectParams& p, const KeySrc& ks, size_t hb, int lane, KeyOps& o) {
  const int n = lane & 15, q4 = lane >> 4;
  if (ks.kind == 0) {
    const uint8_t* rec = p.int4 + hb * (size_t)p.int4_cap * 160 + (size_t)ks.tile * T4_BYTES;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        o.a4[blk][g] = codes_to_f16(*(const uint32_t*)(rec + blk * 1024 + g * 256 + n * 16 + q4 * 4));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      o.sm0[g] = *(const u32x4*)(rec + T4_KSM + g * 64 + q4 * 16);
      o.sm1[g] = *(const u32x4*)(rec + T4_KSM + 256 + g * 64 + q4 * 16);
    }
  } else if (ks.kind == 1) {
    const uint16_t* base;
    size_t slab;
    if (ks.seg == 1) { slab = (size_t)p.anchor_cap * D; base = p.a_k; }
    else if (ks.seg == 2) { slab = (size_t)p.staging_cap * D; base = p.s_k; }
    else { slab = (size_t)WIN * D; base = p.w_k; }
    const uint16_t* t = base + hb * slab + (size_t)ks.tile * 4096 + lane * 8;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) o.ab[blk][tt] = *(const bf16x8*)(t + (blk * 4 + tt) * 512);
  } else {
    // dense rows: key row (tile*32 + 16 blk + n), channels 32 q4 + 8 tt .. +7
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      int key = ks.tile * 32 + 16 * blk + n;
      if (key >= ks.count) key = ks.count - 1;  // masked later; stay inside the buffer
      const uint16_t* row = p.dense_k + (hb * (size_t)p.len + key) * D + 32 * q4;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) o.ab[blk][tt] = *(const bf16x8*)(row + 8 * tt);
    }
  }
}

// Scores (log2 domain, alpha included) of this lane's 8 (key, row) pairs for one row block:
// keys 4q4 + j (block 0) and 16 + 4q4 + j (block 1), row r0 + n.
__device__ inline void block_scores(const KeySrc& ks, const KeyOps& o, const f16x8* s16, const bf16x8* sbf,
                                    const float* qs, int lane, float (&sc)[8]) {
  const float alpha_log2 = LOG2E * 0.08838834764831845f;
  if (ks.kind == 0) {
    f32x4 acc0[4], acc1[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f16x8 bq = s16[g * 64 + lane];
      acc0[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(o.a4[0][g], bq, (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      acc1[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(o.a4[1][g], bq, (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
    const float c = alpha_log2 * 16777216.0f;  // codes carry 2^-24
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v0 = 0.f, v1 = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        v0 += half_lo(o.sm0[g][j]) * acc0[g][j] + half_hi(o.sm0[g][j]) * qs[g] * (1.0f / 16777216.0f);
        v1 += half_lo(o.sm1[g][j]) * acc1[g][j] + half_hi(o.sm1[g][j]) * qs[g] * (1.0f / 16777216.0f);
      }
      sc[j] = v0 * c;
      sc[4 + j] = v1 * c;
    }
  } else {
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      // B: rows' channels 32q4 + 8tt .. +7 (natural order) = staged chunk (g = q4? no: lane's quad
      // q4 needs channels of group q4 at chunk tt) -> staged entry [q4][16 tt + n]
      const bf16x8 bq = sbf[(lane >> 4) * 64 + 16 * tt + (lane & 15)];
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.ab[0][tt], bq, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.ab[1][tt], bq, a1, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = a0[j] * alpha_log2;
      sc[4 + j] = a1[j] * alpha_log2;
    }
  }
}

template <int PASS>
__global__ __launch_bounds__(512) void select_pass_kernel(SelectParams p) {
  __shared__ f16x8 s16[2][4 * 64];
  __shared__ bf16x8 sbf[2][4 * 64];
  __shared__ float red[SW][16][2];
  const int task = blockIdx.x, hb = blockIdx.y, b = hb / p.Hkv, hkv = hb % p.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, q4 = lane >> 4;
  const int R = p.n_proxy * p.G;
  const int RB = (R + 15) >> 4;
  const int gt = task * SW + wave;  // this wave's global tile
  const bool has = gt < p.n_tiles;
  KeySrc ks;
  KeyOps ko;
  if (has) {
    ks = key_src(p, gt);
    load_keys(p, ks, hb, lane, ko);
  }
  // validity of this lane's 8 keys
  bool valid[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int key = (has ? ks.tile * 32 : 0) + ((j >> 2) << 4) + 4 * q4 + (j & 3);
    valid[j] = has && key < ks.count;
  }
  const float* qsum = p.qsum + (size_t)hb * R * 4;
  float colsum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  stage_rows(p, b, hkv, 0, R, s16[0], sbf[0]);
  __syncthreads();
  for (int rb = 0; rb < RB; ++rb) {
    const int cur = rb & 1;
    if (rb + 1 < RB) stage_rows(p, b, hkv, (rb + 1) * 16, R, s16[cur ^ 1], sbf[cur ^ 1]);
    const int r = rb * 16 + n;
    const bool rvalid = r < R;
    float sc[8];
    if (has) {
      float qs[4] = {0.f, 0.f, 0.f, 0.f};
      if (ks.kind == 0 && rvalid) {
#pragma unroll
        for (int g = 0; g < 4; ++g) qs[g] = qsum[(size_t)r * 4 + g];
      }
      block_scores(ks, ko, s16[cur], sbf[cur], qs, lane, sc);
    }
    if (PASS == 1) {
      // partial (max, sum exp2) of row r over this wave's keys
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = (has && valid[j]) ? fmaxf(m, sc[j]) : m;
      m = fmaxf(m, shfl_xor_f(m, 16));
      m = fmaxf(m, shfl_xor_f(m, 32));
      float s = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int j = 0; j < 8; ++j) s += (has && valid[j]) ? __builtin_amdgcn_exp2f(sc[j] - m) : 0.f;
      }
      s += shfl_xor_f(s, 16);
      s += shfl_xor_f(s, 32);
      if (q4 == 0) { red[wave][n][0] = m; red[wave][n][1] = s; }
      __syncthreads();
      if (threadIdx.x < 16 && rb * 16 + threadIdx.x < R) {
        const int rr = threadIdx.x;
        float M = -INFINITY;
        for (int w2 = 0; w2 < SW; ++w2) M = fmaxf(M, red[w2][rr][0]);
        float S = 0.f;
        if (M != -INFINITY)
          for (int w2 = 0; w2 < SW; ++w2) S += red[w2][rr][1] * __builtin_amdgcn_exp2f(red[w2][rr][0] - M);
        float* dst = p.rowpart + (((size_t)hb * p.n_tasks + task) * R + rb * 16 + rr) * 2;
        dst[0] = M;
        dst[1] = S;
      }
    } else {
      if (has && rvalid) {
        const float M = p.rowstat[((size_t)hb * R + r) * 2];
        const float iz = p.rowstat[((size_t)hb * R + r) * 2 + 1];
#pragma unroll
        for (int j = 0; j < 8; ++j) colsum[j] += valid[j] ? __builtin_amdgcn_exp2f(sc[j] - M) * iz : 0.f;
      }
    }
    __syncthreads();
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

// row partials -> (max, 1 / normaliser) per row
__global__ __launch_bounds__(256) void select_rowmerge_kernel(SelectParams p) {
  const int hb = blockIdx.y;
  const int R = p.n_proxy * p.G;
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < R; r += gridDim.x * blockDim.x) {
    const float* part = p.rowpart + (size_t)hb * p.n_tasks * R * 2;
    float M = -INFINITY;
    for (int t = 0; t < p.n_tasks; ++t) M = fmaxf(M, part[((size_t)t * R + r) * 2]);
    float S = 0.f;
    for (int t = 0; t < p.n_tasks; ++t) {
      const float m = part[((size_t)t * R + r) * 2];
      if (m != -INFINITY) S += part[((size_t)t * R + r) * 2 + 1] * __builtin_amdgcn_exp2f(m - M);
    }
    p.rowstat[((size_t)hb * R + r) * 2] = M;
    p.rowstat[((size_t)hb * R + r) * 2 + 1] = 1.0f / S;
  }
}

// ---------------------------------------------------------------- top-k (radix select)
// One workgroup per head.  Scores are >= 0, so their bit patterns order like the values.
// Keeps every score above the k-th largest value T and the lowest-position scores equal to T,
// written in ascending position order.
constexpr int TK_THREADS = 1024;

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(SelectParams p) {
  __shared__ int hist[256];
  __shared__ int scan_a[TK_THREADS], scan_b[TK_THREADS];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_need;
  const int hb = blockIdx.x, tid = threadIdx.x;
  const int P = p.len - WIN > 0 ? p.len - WIN : 0;
  const uint32_t* sc = (const uint32_t*)(p.scores + hb * (size_t)P);
  int32_t* out = p.idx_out + hb * (size_t)p.k;
  if (tid == 0) { s_prefix = 0u; s_mask = 0u; s_need = p.k; }
  __syncthreads();
  // four 8-bit digits, most significant first: find T and how many of it to keep
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += TK_THREADS) hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix, mask = s_mask;
    for (int i = tid; i < P; i += TK_THREADS) {
      const uint32_t v = sc[i];
      if ((v & mask) == prefix) atomicAdd(&hist[(v >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int need = s_need, d = 255;
      for (; d > 0; --d) {
        if (hist[d] >= need) break;
        need -= hist[d];
      }
      s_prefix = prefix | ((uint32_t)d << shift);
      s_mask = mask | (255u << shift);
      s_need = need;  // how many elements equal to the final prefix must be kept
    }
    __syncthreads();
  }
  const uint32_t T = s_prefix;
  const int need_eq = s_need;
  // ordered compaction: each thread owns a contiguous range of positions
  const int per = (P + TK_THREADS - 1) / TK_THREADS;
  const int lo = tid * per, hi = min(P, lo + per);
  int n_gt = 0, n_eq = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t v = sc[i];
    n_gt += v > T;
    n_eq += v == T;
  }
  scan_a[tid] = n_eq;
  __syncthreads();
  // exclusive scan of the equal counts (Hillis-Steele, ping-pong)
  int* src = scan_a;
  int* dst = scan_b;
  for (int off = 1; off < TK_THREADS; off <<= 1) {
    dst[tid] = src[tid] + (tid >= off ? src[tid - off] : 0);
    __syncthreads();
    int* t = src; src = dst; dst = t;
  }
  const int eq_before = src[tid] - n_eq;
  int take_eq = need_eq - eq_before;
  take_eq = take_eq < 0 ? 0 : (take_eq > n_eq ? n_eq : take_eq);
  const int mine = n_gt + take_eq;
  __syncthreads();
  scan_a[tid] = mine;
  __syncthreads();
  src = scan_a;
  dst = scan_b;
  for (int off = 1; off < TK_THREADS; off <<= 1) {
    dst[tid] = src[tid] + (tid >= off ? src[tid - off] : 0);
    __syncthreads();
    int* t = src; src = dst; dst = t;
  }
  int o = src[tid] - mine;
  int eq_left = take_eq;
  for (int i = lo; i < hi; ++i) {
    const uint32_t v = sc[i];
    if (v > T || (v == T && eq_left > 0)) {
      if (v == T) --eq_left;
      if (o < p.k) out[o] = i;  // exactly k are kept for finite scores; never write past k
      ++o;
    }
  }
}

}  // namespace

hipError_t launch_select(SelectParams p, hipStream_t stream) {
  const int R = p.n_proxy * p.G;
  const int H = p.B * p.Hkv;
  hipError_t e;
  hipLaunchKernelGGL(select_qsum_kernel, dim3((R * 4 + 255) / 256, H), dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 grid(p.n_tasks, H);
  hipLaunchKernelGGL(select_pass_kernel<1>, grid, dim3(SW * 64), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(select_rowmerge_kernel, dim3((R + 255) / 256, H), dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(select_pass_kernel<2>, grid, dim3(SW * 64), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.k > 0) {
    hipLaunchKernelGGL(topk_kernel, dim3(H), dim3(TK_THREADS), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

int select_task_count(int n_tiles) { return (n_tiles + SW - 1) / SW; }

}  // namespace hyq

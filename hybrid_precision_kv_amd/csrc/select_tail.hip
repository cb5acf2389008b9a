// Vertical-token identification as the HyQuant paper's Alg. 1 writes it, for gfx950.
//
// HyQuant paper ("HyQuant: Hybrid-Precision Quantization for LLM Attention"), appendix A.1,
// Alg. 1: the proxy of each Q head is the mean of its last t = min(W, L_Q) queries, every
// prefix key j < P = L_K - W is scored with the raw logit qbar . k_j (no scaling, no softmax),
// the Q heads of a KV group read their KV head's keys in place (the GQA-native form), and each
// Q head keeps its own top-k.
//
// Three launches: the tail means (one workgroup per Q head), the logits (HBM bound: every
// prefix key row is read once, by 16 lanes of 16 bytes, for all G Q heads of its group), and
// the radix top-k of the vertical-line selector, run on order-preserving integer keys of the
// logits.
#include "hyq_common.h"
#include "hyq_launch.h"

namespace hyq {

namespace {

constexpr int TS_WAVES = 4;
constexpr int TS_STEPS = 16;                        // 4-key steps per wave
constexpr int TS_KEYS = TS_WAVES * TS_STEPS * 4;    // keys per workgroup

// qbar[bh][c] = (sum over the t tail rows of q[bh][i][c]) / t in fp32: wave w sums its 32
// consecutive rows (rows t0 + 32 w .. in ascending order), the four partial sums are added in
// wave order, then one IEEE divide.  Lane l holds channels 2l, 2l + 1; every load of a wave is
// issued before the first add.
constexpr int TM_ROWS = 32;
__global__ __launch_bounds__(256) void tail_mean_kernel(TailSelectParams p) {
  __shared__ float part[4][D];
  const int bh = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t0 = p.n_q - p.t;
  const uint32_t* q = (const uint32_t*)(p.q + (size_t)bh * p.n_q * D) + lane;
  uint32_t x[TM_ROWS];
#pragma unroll
  for (int r = 0; r < TM_ROWS; ++r) {
    const int i = TM_ROWS * w + r;
    x[r] = i < p.t ? q[(size_t)(t0 + i) * (D / 2)] : 0u;
  }
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int r = 0; r < TM_ROWS; ++r) {
    s0 += __uint_as_float(x[r] << 16);
    s1 += __uint_as_float(x[r] & 0xffff0000u);
  }
  part[w][2 * lane] = s0;
  part[w][2 * lane + 1] = s1;
  __syncthreads();
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    const float s = ((part[0][c] + part[1][c]) + part[2][c]) + part[3][c];
    p.qbar[(size_t)bh * D + c] = __fdiv_rn(s, (float)p.t);
  }
}

__device__ inline float dpp_row_ror4(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
}
__device__ inline float dpp_row_ror8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}
// sum over the 16 lanes of a DPP row (every lane of the row receives it)
__device__ inline float row16_sum(float v) {
  v += dpp_quad_xor1(v);
  v += dpp_quad_xor2(v);
  v += dpp_row_ror4(v);
  return v + dpp_row_ror8(v);
}

// float -> unsigned key with the same order (both zeros map to one key)
__device__ inline uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  if (f == 0.0f) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Logits of TS_KEYS prefix keys of one (b, KV head) for its G Q heads.  Lane (kk, c) of a
// wave (kk = lane / 16, c = lane % 16) holds channels 8c .. 8c+7 of key 4 s + kk at step s;
// the 16-lane row sums give every lane the full dot, and lane c < G stores Q head c's.
template <int G>
__global__ __launch_bounds__(TS_WAVES * 64) void tail_score_kernel(TailSelectParams p) {
  const int bhk = blockIdx.y;  // b * Hkv + hk
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kk = lane >> 4, c = lane & 15;
  const int P = p.len - WIN;
  const int j0 = blockIdx.x * TS_KEYS + wave * (TS_STEPS * 4);
  const int b = bhk / p.Hkv, hk = bhk % p.Hkv;
  const size_t bh0 = (size_t)b * p.Hkv * G + (size_t)hk * G;  // first Q head of the group
  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const f32x4 a = *(const f32x4*)(p.qbar + (bh0 + h) * D + 8 * c);
    const f32x4 bb = *(const f32x4*)(p.qbar + (bh0 + h) * D + 8 * c + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { qv[h][e] = a[e]; qv[h][4 + e] = bb[e]; }
  }
  const uint16_t* kbase = p.k + (size_t)bhk * p.len * D + 8 * c;
  u32x4 kr[TS_STEPS];
#pragma unroll
  for (int s = 0; s < TS_STEPS; ++s) {
    const int j = j0 + 4 * s + kk;
    kr[s] = j < P ? *(const u32x4*)(kbase + (size_t)j * D) : (u32x4){0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int s = 0; s < TS_STEPS; ++s) {
    const int j = j0 + 4 * s + kk;
    float kf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kf[2 * e] = __uint_as_float(kr[s][e] << 16);
      kf[2 * e + 1] = __uint_as_float(kr[s][e] & 0xffff0000u);
    }
    float mine = 0.0f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d = qv[h][0] * kf[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) d = fmaf(qv[h][e], kf[e], d);
      d = row16_sum(d);
      if (c == h) mine = d;
    }
    if (c < G && j < P) {
      const size_t o = (bh0 + c) * (size_t)P + j;
      p.keys[o] = order_key(mine);
      if (p.scores_out) p.scores_out[o] = mine;
    }
  }
}

}  // namespace

hipError_t launch_select_tail(const TailSelectParams& p, hipStream_t stream) {
  const int P = p.len - WIN;
  hipLaunchKernelGGL(tail_mean_kernel, dim3(p.B * p.Hkv * p.G), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((P + TS_KEYS - 1) / TS_KEYS, p.B * p.Hkv), block(TS_WAVES * 64);
  switch (p.G) {
    case 1: hipLaunchKernelGGL(tail_score_kernel<1>, grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL(tail_score_kernel<2>, grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL(tail_score_kernel<4>, grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL(tail_score_kernel<8>, grid, block, 0, stream, p); break;
    case 16: hipLaunchKernelGGL(tail_score_kernel<16>, grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.k_sel > 0) return launch_topk_keys(p.keys, P, p.k_sel, p.B * p.Hkv * p.G, p.idx_out, stream);
  return hipSuccess;
}

}  // namespace hyq

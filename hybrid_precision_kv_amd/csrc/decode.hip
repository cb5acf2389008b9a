// Split-K hybrid-precision decode attention for gfx950.
//
// HyQuant paper ("HyQuant: Hybrid-Precision Quantization for LLM Attention"), §4.3 Eq. 8-9
// and Alg. 3: every cached position enters one softmax; INT4 positions are dequantized on the
// fly (never materialised), bf16 anchors / staging / window are read directly, the sequence is
// split into chunks whose partial (m, l, acc) states are merged by ReduceSoftmax.
//
// Mapping onto CDNA4 (one wave = one worker, 32-position tiles):
//  * Q.K^T on MFMA f32_16x16x32_f16.  A = 16 cached positions x 32 channels, B = the Q heads of
//    the KV group spread over the 16 MFMA columns as (head, channel group) pairs: column
//    4*h + g carries q[h] restricted to group g, so the MFMA returns per-group partial dots and
//    every lane owns a distinct (head, group).  INT4 codes enter as f16 *subnormals*
//    (bits 0x000c == c * 2^-24, exact), one AND per code pair.  The per-group scale and min are
//    applied in fp32 afterwards: q.k = sum_g s_g * (q_g . code_g) + m_g * sum(q_g).
//  * Sum over the 4 groups with two DPP quad permutes; max across the tile with two lane swaps.
//  * P.V on the same MFMA: A = V codes of 16 channels x 8 positions per lane, read from a
//    tile-transposed layout so one dword is one MFMA operand pair set; B = P' = p * s_V (the
//    MFMA output layout of the K product is exactly the B layout needed here), split into
//    f16 hi + lo parts so the weights keep ~22 bits.  The V min enters as sum p * m_V.
//  * bf16 tiles use the bf16 MFMA with the same softmax state.
//  * 4 waves per workgroup merge their states in LDS; a second tiny kernel merges splits.
#include "hyq_common.h"
#include "hyq_launch.h"

namespace hyq {

namespace {

constexpr int WAVES = 4;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float PSCALE = 256.0f;         // P' = p * s_V * PSCALE keeps f16 weights normal
constexpr float ACC_SCALE = 65536.0f;    // 2^24 / PSCALE: INT4 accumulators -> true scale
constexpr float BF_PSCALE = 1.0f / 65536.0f;  // bf16 tiles feed p * PSCALE * 2^-24
constexpr uint32_t NIB = 0x000F000Fu;

__device__ inline f16x8 codes_to_f16(uint32_t x) {
  u32x4 a;
  a[0] = x & NIB;
  a[1] = (x >> 4) & NIB;
  a[2] = (x >> 8) & NIB;
  a[3] = (x >> 12) & NIB;
  return __builtin_bit_cast(f16x8, a);
}
__device__ inline float half_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffff)); }
__device__ inline float half_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

// maps a cut point of the weighted work sequence (INT4 tiles weigh 5, bf16 tiles 16 --
// their byte ratio) to (INT4 tile index, bf16 tile index)
__device__ inline void work_cut(long x, int T4, int TB, int& i, int& u) {
  const long w4 = 5L * T4;
  if (x <= w4) { i = (int)((x + 2) / 5); u = 0; }
  else { i = T4; u = (int)((x - w4 + 8) / 16); if (u > TB) u = TB; }
  if (i > T4) i = T4;
}

struct WaveState {
  float m, l, mt;
  f32x4 acc[8];
};

// online-softmax update for one tile; sc[8] are log2-domain scores (-inf = masked)
__device__ inline void tile_softmax(WaveState& st, const float (&sc)[8], float (&pv)[8]) {
  float tmax = sc[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, sc[j]);
  tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
  tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
  const float m_new = fmaxf(st.m, tmax);
  if (m_new > st.m) {
    const float c = __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= c;
    st.mt *= c;
#pragma unroll
    for (int r = 0; r < 8; ++r) st.acc[r] *= c;
    st.m = m_new;
  }
  const bool live = st.m != -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j) pv[j] = live ? __builtin_amdgcn_exp2f(sc[j] - st.m) : 0.0f;
  float ls = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ls += pv[j];
  st.l += ls;
}

__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, q4 = lane >> 4;
  const int hh = n >> 2, g = n & 3;
  const int split = blockIdx.x, b = blockIdx.z;
  const int nsub = (p.G + 3) >> 2;
  const int hkv = blockIdx.y / nsub, sub = blockIdx.y % nsub;
  const int head = sub * 4 + hh;  // Q head inside the KV group
  const bool head_ok = head < p.G;
  const size_t hb = (size_t)b * p.Hkv + hkv;
  const int Hq = p.Hkv * p.G;

  // ---- B operands: q restricted to this lane's column group (zero elsewhere)
  f16x8 bq4[4];
  bf16x8 bqb[4];
  float qsum = 0.f;
  {
    const uint16_t* qv = p.q + ((size_t)b * Hq + (size_t)hkv * p.G + (head_ok ? head : 0)) * D;
    const bool use = head_ok && (g == q4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int cp = 32 * q4 + 8 * t + kslot_nibble(e);
        const int cn = 32 * q4 + 8 * t + e;
        const uint16_t bp = use ? qv[cp] : (uint16_t)0;
        const uint16_t bn = use ? qv[cn] : (uint16_t)0;
        bq4[t][e] = (_Float16)bf16_bits_to_f32(bp);
        bqb[t][e] = __builtin_bit_cast(__bf16, bn);
      }
    }
    if (head_ok) {
      for (int c = 0; c < 32; ++c) qsum += (float)(_Float16)bf16_bits_to_f32(qv[32 * g + c]);
    }
  }
  const float qsum24 = qsum * (1.0f / 16777216.0f);
  const float alpha_log2 = LOG2E * 0.08838834764831845f;  // log2(e) / sqrt(128)
  const float c_int4 = alpha_log2 * 16777216.0f;

  WaveState st;
  st.m = -INFINITY; st.l = 0.f; st.mt = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) st.acc[r] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // ---- work range of this worker
  const int NW = p.n_splits * WAVES, w = split * WAVES + wave;
  const int T4 = (p.n_int4 + 31) >> 5;
  const int TA = (p.n_anchor + 31) >> 5, TS = (p.n_staged + 31) >> 5, TWn = (p.n_win + 31) >> 5;
  const int TB = TA + TS + TWn;
  const long Wt = 5L * T4 + 16L * TB;
  int i0, u0, i1, u1;
  work_cut(Wt * w / NW, T4, TB, i0, u0);
  work_cut(Wt * (w + 1) / NW, T4, TB, i1, u1);

  // ---- INT4 tiles
  const uint8_t* kc_head = p.k_codes + hb * (size_t)p.int4_cap * 64;
  const uint32_t* vc_head = p.v_codes + hb * (size_t)(p.int4_cap / 32) * 512;
  const uint32_t* ksm_head = p.k_sm + hb * (size_t)(p.int4_cap / 16) * 64;
  const uint32_t* vsm_head = p.v_sm + hb * (size_t)(p.int4_cap / 16) * 64;
  for (int t = i0; t < i1; ++t) {
    const int base = t * 32;
    const u32x4 kc0 = *(const u32x4*)(kc_head + (size_t)(base + n) * 64 + q4 * 16);
    const u32x4 kc1 = *(const u32x4*)(kc_head + (size_t)(base + 16 + n) * 64 + q4 * 16);
    const u32x4 ks0 = *(const u32x4*)(ksm_head + (size_t)(2 * t) * 64 + g * 16 + q4 * 4);
    const u32x4 ks1 = *(const u32x4*)(ksm_head + (size_t)(2 * t + 1) * 64 + g * 16 + q4 * 4);
    const u32x4 vs0 = *(const u32x4*)(vsm_head + (size_t)(2 * t) * 64 + g * 16 + q4 * 4);
    const u32x4 vs1 = *(const u32x4*)(vsm_head + (size_t)(2 * t + 1) * 64 + g * 16 + q4 * 4);
    const u32x4 vc0 = *(const u32x4*)(vc_head + (size_t)t * 512 + (n * 4 + q4) * 8);
    const u32x4 vc1 = *(const u32x4*)(vc_head + (size_t)t * 512 + (n * 4 + q4) * 8 + 4);

    f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes_to_f16(kc0[tt]), bq4[tt], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes_to_f16(kc1[tt]), bq4[tt], S1, 0, 0, 0);
    }
    float sc[8];
    bool valid[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v0 = fmaf(half_lo(ks0[r]), S0[r], half_hi(ks0[r]) * qsum24);
      float v1 = fmaf(half_lo(ks1[r]), S1[r], half_hi(ks1[r]) * qsum24);
      v0 += dpp_quad_xor1(v0);
      v1 += dpp_quad_xor1(v1);
      v0 += dpp_quad_xor2(v0);
      v1 += dpp_quad_xor2(v1);
      valid[r] = base + 4 * q4 + r < p.n_int4;
      valid[4 + r] = base + 16 + 4 * q4 + r < p.n_int4;
      sc[r] = valid[r] ? v0 * c_int4 : -INFINITY;
      sc[4 + r] = valid[4 + r] ? v1 * c_int4 : -INFINITY;
    }
    float pv[8];
    tile_softmax(st, sc, pv);
    f16x8 bhi, blo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t smv = j < 4 ? vs0[j] : vs1[j - 4];
      const float pj = valid[j] ? pv[j] : 0.f;
      st.mt = valid[j] ? fmaf(pj, half_hi(smv), st.mt) : st.mt;
      const float pp = valid[j] ? pj * half_lo(smv) * PSCALE : 0.f;
      const _Float16 h = (_Float16)pp;
      bhi[j] = h;
      blo[j] = (_Float16)(pp - (float)h);
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const f16x8 a = codes_to_f16(rr < 4 ? vc0[rr] : vc1[rr - 4]);
      st.acc[rr] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bhi, st.acc[rr], 0, 0, 0);
      st.acc[rr] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, blo, st.acc[rr], 0, 0, 0);
    }
  }

  // ---- bf16 tiles (anchors, staging, window)
  const size_t slab_a = (size_t)p.anchor_cap * D, slab_s = (size_t)p.staging_cap * D, slab_w = (size_t)WIN * D;
  for (int u = u0; u < u1; ++u) {
    const uint16_t *kb, *vb;
    int cnt, tl;
    if (u < TA) { kb = p.a_k + hb * slab_a; vb = p.a_v + hb * slab_a; cnt = p.n_anchor; tl = u; }
    else if (u < TA + TS) { kb = p.s_k + hb * slab_s; vb = p.s_v + hb * slab_s; cnt = p.n_staged; tl = u - TA; }
    else { kb = p.w_k + hb * slab_w; vb = p.w_v + hb * slab_w; cnt = p.n_win; tl = u - TA - TS; }
    const int base = tl * 32;
    f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* r0 = kb + (size_t)(base + n) * D + 32 * q4;
    const uint16_t* r1 = kb + (size_t)(base + 16 + n) * D + 32 * q4;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(r0 + 8 * tt), bqb[tt], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(r1 + 8 * tt), bqb[tt], S1, 0, 0, 0);
    }
    float sc[8];
    bool valid[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v0 = S0[r], v1 = S1[r];
      v0 += dpp_quad_xor1(v0);
      v1 += dpp_quad_xor1(v1);
      v0 += dpp_quad_xor2(v0);
      v1 += dpp_quad_xor2(v1);
      valid[r] = base + 4 * q4 + r < cnt;
      valid[4 + r] = base + 16 + 4 * q4 + r < cnt;
      sc[r] = valid[r] ? v0 * alpha_log2 : -INFINITY;
      sc[4 + r] = valid[4 + r] ? v1 * alpha_log2 : -INFINITY;
    }
    float pv[8];
    tile_softmax(st, sc, pv);
    bf16x8 bhi, blo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float pp = valid[j] ? pv[j] * BF_PSCALE : 0.f;
      const __bf16 h = (__bf16)pp;
      bhi[j] = h;
      blo[j] = (__bf16)(pp - (float)h);
    }
    const uint16_t* vt = vb + (size_t)tl * 4096 + (size_t)(n * 4 + q4) * 64;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const bf16x8 a = *(const bf16x8*)(vt + rr * 8);
      st.acc[rr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bhi, st.acc[rr], 0, 0, 0);
      st.acc[rr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, blo, st.acc[rr], 0, 0, 0);
    }
  }

  // ---- per-wave totals, then merge the 4 waves through LDS
  st.l += shfl_xor_f(st.l, 16);
  st.l += shfl_xor_f(st.l, 32);
  st.mt += shfl_xor_f(st.mt, 16);
  st.mt += shfl_xor_f(st.mt, 32);
  __shared__ float red_m[WAVES][4], red_l[WAVES][4];
  __shared__ float red_o[WAVES][4][D];
  if (n == 4 * hh && q4 == 0) {  // one lane per head (g == 0, quad 0)
    red_m[wave][hh] = st.m;
    red_l[wave][hh] = st.l;
  }
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    if ((rr >> 1) == g) {
#pragma unroll
      for (int r = 0; r < 4; ++r) red_o[wave][hh][16 * rr + 4 * q4 + r] = st.acc[rr][r] * ACC_SCALE + st.mt;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 4 * D; idx += 256) {
    const int h2 = idx / D, c = idx % D;
    const int hd = sub * 4 + h2;
    if (hd >= p.G) continue;
    float M = red_m[0][h2];
#pragma unroll
    for (int ww = 1; ww < WAVES; ++ww) M = fmaxf(M, red_m[ww][h2]);
    float O = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) {
        const float f = __builtin_amdgcn_exp2f(red_m[ww][h2] - M);
        O += red_o[ww][h2][c] * f;
        L += red_l[ww][h2] * f;
      }
    }
    float* rec = p.part + (((size_t)b * Hq + (size_t)hkv * p.G + hd) * p.n_splits + split) * (D + 2);
    if (c == 0) { rec[0] = M; rec[1] = L; }
    rec[2 + c] = O;
  }
}

// ReduceSoftmax over splits (HyQuant paper Alg. 3): one workgroup per (b, Q head).
__global__ __launch_bounds__(128) void decode_reduce_kernel(const float* __restrict__ part, float* __restrict__ o,
                                                            int n_splits) {
  const int bh = blockIdx.x, c = threadIdx.x;
  const float* rec = part + (size_t)bh * n_splits * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, rec[(size_t)s * (D + 2)]);
  float O = 0.f, L = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const float* r = rec + (size_t)s * (D + 2);
      const float f = __builtin_amdgcn_exp2f(r[0] - M);
      L += r[1] * f;
      O += r[2 + c] * f;
    }
  }
  o[(size_t)bh * D + c] = O / L;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, float* o, int B, hipStream_t stream) {
  const int nsub = (p.G + 3) >> 2;
  dim3 grid(p.n_splits, p.Hkv * nsub, B);
  hipLaunchKernelGGL(decode_split_kernel, grid, dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3(B * p.Hkv * p.G), dim3(D), 0, stream, p.part, o, p.n_splits);
  return hipGetLastError();
}

}  // namespace hyq

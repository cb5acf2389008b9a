// Hybrid prefill attention for gfx950 (HyQuant paper §4.2 Eq. 6-7, Alg. 2).
//
// Query i attends, causally, to three key sets: the window [i-127, i] and the anchors
// a <= i-128 in bf16, and every other key j <= i-128 through INT8 Q.K and FP8 P.V.  The pass
// is split into operand quantization (Alg. 2 Stage 2: three small kernels writing codes,
// scales, the anchor bitmap and the gathered anchor rows into the caller's workspace) and one
// attention kernel (Alg. 2 Stage 3) that runs a
// single online softmax per query row over 64-key tiles in the order: quantized tiles,
// anchor tiles, window tiles.
//
// Attention kernel design (one workgroup = 128 queries of one Q head, 4 waves x 32 queries):
//  * Scores are computed transposed, S^T = K . Q^T, with 16x16 MFMA tiles: a lane then holds
//    16 keys of ONE query per 16-query block, so row maxima are mostly in-lane.  One
//    v_permlane16_swap per packed word regroups the P codes of both 16-query blocks into the
//    B operand of a 32x32 MFMA (lane l: query l % 32, 32 of the tile's keys), and
//    O^T = V^T . P^T runs on 32x32 tiles: the fp8 32x32x64 MFMA runs at twice the rate of
//    the 16x16x32 one.  The V tile layouts permute the keys the same way.
//  * Quantized tiles: i32 MFMA 16x16x64 on INT8 codes; the mask (anchors, causal edge) enters
//    as the MFMA's C input (-2^28), so interior tiles pay nothing for it; P = E4M3(448 p)
//    feeds the fp8 32x32x64 MFMA against E4M3 V codes; the row sum of the rounded P comes out
//    of 16x16 MFMAs against a row of ones.  After the last quantized tile the accumulator is
//    scaled by the per-channel V scale / 448.
//  * Anchor and window tiles: bf16 MFMA 16x16x32 for the scores with a -inf mask in the C
//    input, P = bf16(p), bf16 32x32x16 MFMA for P.V.
//  * The running max is exact per 64-key tile (no lazy threshold): the P codes depend on it.
//    The accumulator is rescaled only when some row's max moved (wave-uniform branch).
//  * Q is quantized in registers from the bf16 rows (block maximum exchanged through LDS);
//    the codes stay in registers as the QK B operand and are also written to the workspace.
#include "hyq_common.h"
#include "hyq_launch.h"

namespace hyq {
namespace {

constexpr int KBLK = 64;          // quantization block (queries and keys) = softmax key tile
constexpr int WG_ROWS = 128;      // queries per attention workgroup
constexpr int NEG_DOT = -(1 << 28);  // masked INT8 dot (|valid dot| < 2^21)
constexpr float AL2 = 0.08838834764831845f * 1.4426950408889634f;  // alpha * log2(e), alpha = 1/sqrt(128)
constexpr float LOG2_448 = 8.807354922057604f;
constexpr float C2_FAST_MIN = 1e-6f;  // below: masked INT8 scores are zeroed explicitly
constexpr int KB_LD = 272;        // LDS row stride (bytes) of the bf16 K tile
constexpr int LDS_V = 64 * KB_LD; // V tile offset (bf16 tiles)
constexpr int LDS_BF = LDS_V + 16384;
// Quantized tiles rotate through a ring of 4 buffers: buffer b at b * LDS_QBUF holds the K
// codes as [16-byte chunk 8][key 64][16], the V codes at + LDS_QV as stored in the workspace,
// and the per-key mask at + LDS_QBIAS.
constexpr int LDS_QV = 8192;
constexpr int LDS_QBIAS = LDS_QV + 8192;  // per-key MFMA C input: 0, or NEG_DOT for an anchor
constexpr int LDS_QBUF = LDS_QBIAS + 256;
constexpr int RING = 4;
constexpr int LDS_TOTAL = RING * LDS_QBUF > LDS_BF ? RING * LDS_QBUF : LDS_BF;

typedef long i64;

__device__ inline float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ inline float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// reciprocal for int8_code: 0 when s is zero or below the normal range (those take the IEEE
// division)
__device__ inline float int8_rcp(float s) { return s >= 0x1p-120f ? __builtin_amdgcn_rcpf(s) : 0.0f; }
// symmetric INT8 code of x with scale s (s == 0 -> 0) and r = int8_rcp(s): the IEEE quotient
// rounded half-even, clamped to [-127, 127]
__device__ inline int int8_code(float x, float s, float r) {
  if (s == 0.0f) return 0;
  float c = r != 0.0f ? rint_div(x, s, r) : rintf(__fdiv_rn(x, s));
  c = fminf(fmaxf(c, -127.0f), 127.0f);
  return (int)c;
}

// value of lane 0 (bit-exact; tells the compiler the value is wave-uniform)
__device__ inline float uniform_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// Maxima over the 4 lanes l, l^16, l^32, l^48 (one 16x16 MFMA column) of two values at once
// (a: 16-query block 0, b: block 1).  v_permlane32_swap(a, b) leaves block 0's pair
// (l, l+32) on the lower 32 lanes and block 1's pair on the upper ones, v_permlane16_swap
// then folds l^16 in, and a last v_permlane32_swap(y, y) returns block 0's result in its
// first and block 1's in its second output on every lane -- VALU ops, no LDS round trip.
__device__ inline void col4_max2_i(int& a, int& b) {
  const auto x = __builtin_amdgcn_permlane32_swap((unsigned)a, (unsigned)b, false, false);
  int y = max((int)x[0], (int)x[1]);
  const auto z = __builtin_amdgcn_permlane16_swap((unsigned)y, (unsigned)y, false, false);
  y = max((int)z[0], (int)z[1]);
  const auto u = __builtin_amdgcn_permlane32_swap((unsigned)y, (unsigned)y, false, false);
  a = (int)u[0];
  b = (int)u[1];
}
__device__ inline void col4_max2_f(float& a, float& b) {
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  float y = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
  const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  y = fmaxf(__uint_as_float(z[0]), __uint_as_float(z[1]));
  const auto u = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  a = __uint_as_float(u[0]);
  b = __uint_as_float(u[1]);
}

// ------------------------------------------------------------------ operand quantization

// MXFP4 block of 32 values held by one lane: shared exponent e = floor(log2 max|x|) - 2
// (E8M0 range, -127 for a zero block) and E2M1 codes of x * 2^-e (exact scaling; the
// hardware conversion rounds to nearest even and saturates at 6), element i in nibble i of
// the 16 bytes (low nibble first).  Returns e.
__device__ inline int mxfp4_block(const float (&x)[32], u32x4& codes) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  int ex = 0;
  (void)frexpf(amax, &ex);  // amax = f 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
  const int e = amax == 0.0f ? -127 : min(127, max(-127, ex - 3));
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t w = 0;
#define HYQ_FP4_PAIR(SEL)                                                                       \
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __builtin_amdgcn_ldexpf(x[8 * d + 2 * SEL], -e), \
                                               __builtin_amdgcn_ldexpf(x[8 * d + 2 * SEL + 1], -e), 1.0f, SEL)
    HYQ_FP4_PAIR(0);
    HYQ_FP4_PAIR(1);
    HYQ_FP4_PAIR(2);
    HYQ_FP4_PAIR(3);
#undef HYQ_FP4_PAIR
    codes[d] = w;
  }
  return e;
}

// Anchor gather: K rows (list order) and V^T in the bf16 operand order for the 32 list
// entries of tile b (channel c per thread); entries past n_anchor (or outside [0, N)) are zero.
__device__ inline void anchor_gather(const PrefillParams& p, int b, int h, int c) {
  const int32_t* anc = p.anchors + (size_t)h * p.n_anchor;
  const int Ac = p.n_anchor_pad;
  uint32_t raw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) raw[i] = 0;
#pragma unroll
  for (int kk = 0; kk < 32; ++kk) {
    const int idx = 32 * b + kk;
    const int a = idx < p.n_anchor ? anc[idx] : -1;
    uint16_t kb = 0, vb = 0;
    if (a >= 0 && a < p.N) {
      kb = p.k[((size_t)h * p.N + a) * D + c];
      vb = p.v[((size_t)h * p.N + a) * D + c];
    }
    p.ka16[((size_t)h * Ac + idx) * D + c] = kb;
    raw[kk >> 1] |= (uint32_t)vb << (16 * (kk & 1));
  }
  uint16_t* tblk = p.va16 + ((size_t)h * (Ac >> 5) + b) * D * 32;
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *(u32x4*)(tblk + (g * D + c) * 8) = (u32x4){raw[4 * g], raw[4 * g + 1], raw[4 * g + 2], raw[4 * g + 3]};
}

// One launch for the operands that need no global reduction.  Workgroups x < Npad / 64, per
// (KV head, 64-key block):
//   * the block's two words of the anchor bitmap (bit (j & 31) of word j >> 5 set for every
//     listed anchor j; the threads scan the sorted list side by side);
//   * K: symmetric INT8 with the anchors left out of the maximum (BULK 0), or MXFP4 per key
//     and 32-channel block (BULK 1: every row, anchors included);
//   * V: per-channel maximum of |V| over the block's non-anchor keys.
// The first ceil(n_anchor_pad / 64) workgroups of each head gather two 32-entry tiles of the
// anchor list each (first, so that they start in the first round of workgroups).
template <int BULK>
__global__ void __launch_bounds__(256) pf_kquant_kernel(PrefillParams p) {
  __shared__ float red[4];
  __shared__ uint16_t vt[64][130];  // |V| as bf16 bit patterns (ordered as the values: >= 0)
  __shared__ uint32_t bw[2];
  const int h = blockIdx.y;
  const int t = threadIdx.x, row = t >> 2, qd = t & 3;
  const int nw = p.Npad >> 5, nb = p.Npad >> 6;
  const int n_gather = (p.n_anchor_pad / 32 + 1) / 2;
  if ((int)blockIdx.x < n_gather) {  // anchor gather: tiles 2 x and 2 x + 1
    const int b = 2 * blockIdx.x + (t >> 7);
    if (32 * b < p.n_anchor_pad) anchor_gather(p, b, h, t & (D - 1));
    return;
  }
  const int blk = blockIdx.x - n_gather;
  const int key = blk * KBLK + row;
  const bool inside = key < p.N;
  // the block's K and V rows are loaded first (they do not depend on the bitmap)
  u32x4 kr[4], vr[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) { kr[c] = (u32x4){0u, 0u, 0u, 0u}; vr[c] = kr[c]; }
  if (inside) {
    const u32x4* ks = (const u32x4*)(p.k + ((size_t)h * p.N + key) * D + 32 * qd);
    const u32x4* vs = (const u32x4*)(p.v + ((size_t)h * p.N + key) * D + 32 * qd);
#pragma unroll
    for (int c = 0; c < 4; ++c) { kr[c] = ks[c]; vr[c] = vs[c]; }
  }
  if (t < 2) bw[t] = 0u;
  __syncthreads();
  {
    const int32_t* anc = p.anchors + (size_t)h * p.n_anchor;
    const int lo_key = blk * KBLK;
    for (int i0 = t; i0 < p.n_anchor; i0 += 8 * 256) {  // eight entries per thread in flight
      int a[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] = i0 + 256 * u < p.n_anchor ? anc[i0 + 256 * u] : -1;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (a[u] >= lo_key && a[u] < lo_key + KBLK) atomicOr(&bw[(a[u] - lo_key) >> 5], 1u << (a[u] & 31));
    }
  }
  __syncthreads();
  if (t < 2) p.abits[(size_t)h * nw + 2 * blk + t] = bw[t];
  const uint32_t word = bw[row >> 5];
  const bool live = inside && !((word >> (key & 31)) & 1u);
  float kx[32], vx[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kx[8 * c + 2 * e] = bf_lo(kr[c][e]); kx[8 * c + 2 * e + 1] = bf_hi(kr[c][e]);
      vx[8 * c + 2 * e] = live ? bf_lo(vr[c][e]) : 0.0f; vx[8 * c + 2 * e + 1] = live ? bf_hi(vr[c][e]) : 0.0f;
    }
  }
#pragma unroll
  for (int e = 0; e < 32; ++e) vt[row][32 * qd + e] = (uint16_t)(__float_as_uint(fabsf(vx[e])) >> 16);  // exact: bf16
  uint8_t* tile = (uint8_t*)p.k8 + ((size_t)h * nb + blk) * 8192;
  if (BULK == 1) {
    // codes of channel block qd of this key: [block][key][16 B]; scale bytes [block][key%16][key/16]
    u32x4 codes;
    const int e = mxfp4_block(kx, codes);
    *(u32x4*)(tile + (qd * 64 + row) * 16) = codes;
    tile[4096 + (qd * 16 + (row & 15)) * 4 + (row >> 4)] = (uint8_t)(e + 127);
    __syncthreads();
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, live ? fabsf(kx[e]) : 0.0f);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, shfl_xor_f(amax, o));
    if ((t & 63) == 0) red[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = __fdiv_rn(amax, 127.0f);
    const float rs = int8_rcp(s);
    // operand order: dim 32 qd + 8 jj + e  ->  byte 64 (qd >> 1) + 16 jj + 8 (qd & 1) + e, and
    // 16-byte chunk k = 4 (qd >> 1) + jj of the row at [tile][chunk][key in tile][16]
    uint8_t* dst = tile + (4 * (qd >> 1)) * 1024 + row * 16 + 8 * (qd & 1);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0 |= (uint32_t)(int8_code(live ? kx[8 * jj + e] : 0.0f, s, rs) & 0xff) << (8 * e);
        w1 |= (uint32_t)(int8_code(live ? kx[8 * jj + 4 + e] : 0.0f, s, rs) & 0xff) << (8 * e);
      }
      *(uint2*)(dst + 1024 * jj) = make_uint2(w0, w1);
    }
    if (t == 0) p.sk[(size_t)h * nb + blk] = s;
  }
  if (t < D) {
    uint32_t m = 0u;
    for (int r = 0; r < 64; ++r) m = max(m, (uint32_t)vt[r][t]);
    p.vmax[((size_t)h * nb + blk) * D + t] = __uint_as_float(m << 16);
  }
}

// s_V[c] = max over blocks / 448 (IEEE divide).  Block = 8 x 128 threads.
__global__ void __launch_bounds__(1024) pf_vscale_kernel(PrefillParams p) {
  __shared__ float part[8][D];
  const int h = blockIdx.x, c = threadIdx.x & (D - 1), g = threadIdx.x >> 7;
  const int nb = p.Npad >> 6;
  float m = 0.0f;
  for (int b0 = g; b0 < nb; b0 += 64) {  // eight loads in flight per thread
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = b0 + 8 * u < nb ? p.vmax[((size_t)h * nb + b0 + 8 * u) * D + c] : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) m = fmaxf(m, x[u]);
  }
  part[g][c] = m;
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmaxf(m, part[i][c]);
    p.sv[h * D + c] = __fdiv_rn(m, 448.0f);
  }
}

// V -> E4M3(V / s_V[c]) (hardware conversion: round to nearest even).  Per 32-key block:
// [half h][channel][16 bytes], byte e of (h, channel) holding key 16 (e >> 3) + 8 h + (e & 7)
// of the block: two blocks' 16-byte rows of one channel and half are the A operand of the
// 32x32x64 P.V MFMA for the key order the P-code regrouping produces.  The bf16 copy of V
// (window tiles) is [8-key group][channel][8 keys].
__global__ void __launch_bounds__(128) pf_vquant_kernel(PrefillParams p) {
  const int b = blockIdx.x, h = blockIdx.y, c = threadIdx.x;
  const uint32_t word = p.abits[(size_t)h * (p.Npad >> 5) + b];
  const float s = p.sv[h * D + c];
  uint32_t w[8], raw[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) raw[i] = 0;
#pragma unroll
  for (int kk = 0; kk < 32; ++kk) {
    const int key = 32 * b + kk;
    const uint16_t vb = key < p.N ? p.v[((size_t)h * p.N + key) * D + c] : (uint16_t)0;
    raw[kk >> 1] |= (uint32_t)vb << (16 * (kk & 1));
    float x = 0.0f;
    if (key < p.N && !((word >> kk) & 1u)) x = bf16_bits_to_f32(vb);
    uint32_t code = 0;
    if (s != 0.0f) code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(x, s), 0.0f, 0, false) & 0xffu;
    const int byte = 16 * ((kk >> 3) & 1) + 8 * (kk >> 4) + (kk & 7);  // 16 h + e
    w[byte >> 2] |= code << (8 * (byte & 3));
  }
  uint8_t* blk = p.v8 + ((size_t)h * (p.Npad >> 5) + b) * D * 32;
  uint16_t* tblk = p.vt16 + ((size_t)h * (p.Npad >> 5) + b) * D * 32;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
    *(u32x4*)(blk + (hh * D + c) * 16) = (u32x4){w[4 * hh], w[4 * hh + 1], w[4 * hh + 2], w[4 * hh + 3]};
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *(u32x4*)(tblk + (g * D + c) * 8) = (u32x4){raw[4 * g], raw[4 * g + 1], raw[4 * g + 2], raw[4 * g + 3]};
}

// ------------------------------------------------------------------ attention

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

struct RowState {
  float m[2];        // running max, log2 units, of query l16 in each 16-query block
  f32x16 acc[4];     // O^T, 32x32 MFMA layout: element 4 i + r is channel 32 cb + 8 i + 4 hh + r
                     // of query l32
  f32x4 lacc;        // row sum of query l16 of 16-query block hh (all 4 entries equal)
};

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}

struct Ctx {
  int h, hk, r0w, N, Npad, nb64, tid, wave, l16, j, l32, hh, qsel;
  i64 sel8;       // E4M3 row-sum selector: ones on the block-0 bytes for rows 0-7, block-1 bytes for 8-15
  bf16x8 selb;    // the same for bf16 pairs
};

// Max update of both 16-query blocks of the wave from their tile maxima (log2 units, valid =
// the block row has an unmasked key in the tile); rescales the accumulators when some row's
// max moved.  Returns the values to subtract inside exp2 (+inf for rows without a valid key).
__device__ inline void row_update(const Ctx& c, RowState& st, const bool (&valid)[2], const float (&tmax)[2],
                                  float shift, float (&muse)[2]) {
  float resc[2];
  bool moved = false;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float mold = st.m[qb];
    const float mnew = valid[qb] ? fmaxf(mold, tmax[qb]) : mold;
    resc[qb] = (mnew == mold) ? 1.0f : __builtin_amdgcn_exp2f(mold - mnew);
    moved |= resc[qb] != 1.0f;
    st.m[qb] = mnew;
    muse[qb] = valid[qb] ? mnew - shift : INFINITY;
  }
  if (__builtin_amdgcn_ballot_w64(moved)) {  // rare after the first tiles
    const float rs = c.qsel ? resc[1] : resc[0];  // the accumulator row of this lane
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) st.acc[cb] *= rs;
    st.lacc *= c.hh ? resc[1] : resc[0];
  }
}

// Quantized tile t: K codes of keys [64 t, 64 t + 64) as stored (INT8: [chunk][key][16],
// 8 KB; MXFP4: [block][key][16] codes, 4 KB, then 256 scale bytes), the tile's E4M3 V codes
// (as stored) and its anchor words.  fetch: global -> registers (issued ahead of use),
// store: registers -> LDS.
struct TileQRegs {
  u32x4 k[2], v[2];
  uint32_t w0, w1;  // anchor bitmap words of the tile
  float sk;         // K scale of the tile (INT8)
};
template <int BULK>
__device__ inline void fetch_tile_q(const PrefillParams& p, const Ctx& c, int t, TileQRegs& r) {
  const uint32_t* ab = p.abits + (size_t)c.hk * (c.Npad >> 5) + 2 * t;
  r.w0 = ab[0];
  r.w1 = ab[1];
  if (BULK == 0) r.sk = p.sk[(size_t)c.hk * c.nb64 + t];
  const size_t tile = ((size_t)c.hk * c.nb64 + t) * 8192;
  const int8_t* kt = p.k8 + tile;
  const uint8_t* vt = p.v8 + tile;
  r.k[0] = *(const u32x4*)(kt + 16 * c.tid);
  if (BULK == 0) r.k[1] = *(const u32x4*)(kt + 16 * (c.tid + 256));
  else if (c.tid < 16) r.k[1] = *(const u32x4*)(kt + 4096 + 16 * c.tid);
#pragma unroll
  for (int i = 0; i < 2; ++i) r.v[i] = *(const u32x4*)(vt + 16 * (c.tid + 256 * i));
}
template <int BULK>
__device__ inline void store_tile_q(const Ctx& c, uint8_t* lds, const TileQRegs& r) {
  *(u32x4*)(lds + 16 * c.tid) = r.k[0];
  if (BULK == 0) *(u32x4*)(lds + 16 * (c.tid + 256)) = r.k[1];
  else if (c.tid < 16) *(u32x4*)(lds + 4096 + 16 * c.tid) = r.k[1];
#pragma unroll
  for (int i = 0; i < 2; ++i) *(u32x4*)(lds + LDS_QV + 16 * (c.tid + 256 * i)) = r.v[i];
  if (c.tid < 64) {  // anchor mask of key tid, built once per tile for every wave
    const uint32_t word = c.tid < 32 ? r.w0 : r.w1;
    const bool anchor = (word >> (c.tid & 31)) & 1u;
    *(int*)(lds + LDS_QBIAS + 4 * c.tid) = BULK == 0 ? (anchor ? NEG_DOT : 0) : (anchor ? (int)0xff800000u : 0);
  }
}

// bf16 tile: 64 K rows (row stride KB_LD in LDS; rows whose key_of(row) is outside [0, N)
// are zero) and the tile's V (16 KB, copied as stored: [8-key group][channel][8]).
template <typename KeyOf>
__device__ inline void load_tile_bf(const Ctx& c, uint8_t* lds, const uint16_t* krows, int kstride_ok_n,
                                    const uint16_t* vt, KeyOf key_of) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = c.tid + 256 * i, row = ch >> 4, part = ch & 15;
    const int key = key_of(row);
    u32x4 kx = {0u, 0u, 0u, 0u};
    if (key >= 0 && key < kstride_ok_n) kx = *(const u32x4*)(krows + (size_t)key * D + 8 * part);
    *(u32x4*)(lds + row * KB_LD + 16 * part) = kx;
    *(u32x4*)(lds + LDS_V + 16 * ch) = *(const u32x4*)(vt + 8 * ch);
  }
}

// Q operand of the bulk segment, held in registers for the whole segment: INT8 codes
// (qi[qb][s] = bytes 64 s + 16 j of query row 16 qb + l16), or MXFP4 codes of channel block j
// of that row (q4[qb]) with the E8M0 scale bytes of both rows in qs[qb] (byte 0).
struct QOps {
  i32x4 qi[2][2];
  u32x4 q4[2];
  uint32_t qs[2];
};
template <int BULK>
struct BulkT;
template <>
struct BulkT<0> {
  typedef i32x4 S;  // exact INT8 dot products
};
template <>
struct BulkT<1> {
  typedef f32x4 S;  // MX dot products (block scales applied by the MFMA)
};

// Scores of one quantized tile (or of its 16-key block kb) for the wave's 32 queries:
// S^T = K . Q^T on INT8 codes, or on MXFP4 codes with their E8M0 scales, with the masked keys
// (anchors; on an EDGE tile also j > i - 128) pushed to NEG_DOT / -inf through the MFMA's C
// input.
template <int BULK, bool EDGE>
__device__ inline void qk_block_q(const Ctx& c, const uint8_t* buf, const QOps& q, int t, int kb,
                                  typename BulkT<BULK>::S (&S2)[2][4]) {
  typedef typename BulkT<BULK>::S S;
  const S bias = *(const S*)(buf + LDS_QBIAS + 4 * (16 * kb + 4 * c.j));  // keys 16kb+4j+r
  S acc[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    acc[qb] = bias;
    if (EDGE) {
      const int row = c.r0w + 16 * qb + c.l16;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (64 * t + 16 * kb + 4 * c.j + r > row - WIN) acc[qb][r] = BULK == 0 ? NEG_DOT : -INFINITY;
    }
  }
  if constexpr (BULK == 0) {
    const i32x4 kf0 = *(const i32x4*)(buf + (c.j * 64 + 16 * kb + c.l16) * 16);
    const i32x4 kf1 = *(const i32x4*)(buf + ((4 + c.j) * 64 + 16 * kb + c.l16) * 16);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) S2[qb][kb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf0, q.qi[qb][0], acc[qb], 0, 0, 0);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      S2[qb][kb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf1, q.qi[qb][1], S2[qb][kb], 0, 0, 0);
  } else {
    // A: codes of key 16 kb + l16, channel block j; its scale is byte kb of the lane's dword
    const u32x4 kc = *(const u32x4*)(buf + (c.j * 64 + 16 * kb + c.l16) * 16);
    const uint32_t ksc = *(const uint32_t*)(buf + 4096 + (c.j * 16 + c.l16) * 4) >> (8 * kb);
    const i32x8 a = {(int)kc[0], (int)kc[1], (int)kc[2], (int)kc[3], 0, 0, 0, 0};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const i32x8 bq = {(int)q.q4[qb][0], (int)q.q4[qb][1], (int)q.q4[qb][2], (int)q.q4[qb][3], 0, 0, 0, 0};
      S2[qb][kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bq, acc[qb], 4, 4, 0, (int)ksc, 0,
                                                                    (int)q.qs[qb]);
    }
  }
}
template <int BULK, bool EDGE>
__device__ inline void qk_tile_q(const Ctx& c, const uint8_t* buf, const QOps& q, int t,
                                 typename BulkT<BULK>::S (&S2)[2][4]) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) qk_block_q<BULK, EDGE>(c, buf, q, t, kb, S2);
}
template <int BULK>
__device__ inline void qk_tile(const Ctx& c, const uint8_t* buf, const QOps& q, int t,
                               typename BulkT<BULK>::S (&S2)[2][4]) {
  if (64 * t + 63 <= c.r0w - WIN)  // every key of the tile is at least 128 before every row
    qk_tile_q<BULK, false>(c, buf, q, t, S2);
  else
    qk_tile_q<BULK, true>(c, buf, q, t, S2);
}

// Online softmax of one quantized tile's scores: the row-state max update (rescaling the
// accumulators when a max moved), P = E4M3(448 p) codes, their row sums (MFMA against a row
// of ones) and the codes regrouped into the B operand of the 32x32x64 P.V MFMA (pk).  With
// FUSE_QK the scores of the next, interior tile tq (buffer qkbuf) replace S2 block by block
// as the exponentials free them, so its MFMAs run under this softmax's VALU work.
// c2 = s_Q s_K alpha log2(e) (wave-uniform).  Below C2_FAST_MIN a masked score is not
// guaranteed to underflow exp2, so the masked entries are zeroed explicitly.
template <int BULK, bool TINY, bool FUSE_QK = false>
__device__ inline void softmax_tile_q(const Ctx& c, typename BulkT<BULK>::S (&S2)[2][4], float c2, RowState& st,
                                      i32x8& pk, const uint8_t* qkbuf = nullptr, const QOps* q = nullptr,
                                      int tq = 0) {
  bool valid[2];
  float tmax[2], muse[2];
  if constexpr (BULK == 0) {
    int mi[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      mi[qb] = NEG_DOT;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        mi[qb] = max(mi[qb], max(max(S2[qb][kb][0], S2[qb][kb][1]), max(S2[qb][kb][2], S2[qb][kb][3])));
    }
    col4_max2_i(mi[0], mi[1]);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      valid[qb] = mi[qb] > NEG_DOT / 2;
      tmax[qb] = (float)mi[qb] * c2;
    }
  } else {
    float mf[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      mf[qb] = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        mf[qb] = fmaxf(mf[qb], fmaxf(fmaxf(S2[qb][kb][0], S2[qb][kb][1]), fmaxf(S2[qb][kb][2], S2[qb][kb][3])));
    }
    col4_max2_f(mf[0], mf[1]);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      valid[qb] = mf[qb] > -INFINITY;
      tmax[qb] = mf[qb] * c2;
    }
  }
  row_update(c, st, valid, tmax, LOG2_448, muse);
  // w[2 kb + qb]: codes of block qb, keys 16 kb + 4 j + r -- the row-sum B operand as is, and
  // after the in-place swaps of each pair the P.V B operand
  i32x8 w;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)S2[qb][kb][r], c2, -muse[qb]));
        if (BULK == 0 && TINY && S2[qb][kb][r] <= NEG_DOT / 2) pv[r] = 0.0f;
      }
      // the first conversion's high half is overwritten by the second: any old value will do
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], __float_as_int(pv[1]), false);
      w[2 * kb + qb] = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], lo, true);
    }
    // block kb's score registers are free: the next tile's (interior) block kb goes there
    if (FUSE_QK) qk_block_q<BULK, false>(c, qkbuf, *q, tq, kb, S2);
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    st.lacc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
        c.sel8, (i64)(uint32_t)w[2 * kb] | ((i64)(uint32_t)w[2 * kb + 1] << 32), st.lacc, 0, 0, 0);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const auto sw = __builtin_amdgcn_permlane16_swap((uint32_t)w[2 * kb], (uint32_t)w[2 * kb + 1], false, false);
    w[2 * kb] = (int)sw[0];
    w[2 * kb + 1] = (int)sw[1];
  }
  pk = w;
}

// P.V of one quantized tile: 32x32x64 E4M3 MFMA per 32-channel block.  The A operand of lane
// (channel 32 cb + l32, half hh) is the 32 bytes of that channel and half in the tile's two
// 32-key blocks, in the byte order of pk.
__device__ inline void pv_tile_q(const Ctx& c, const uint8_t* buf, const i32x8& pk, RowState& st) {
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const u32x4 a0 = *(const u32x4*)(buf + LDS_QV + ((0 + c.hh) * D + 32 * cb + c.l32) * 16);
    const u32x4 a1 = *(const u32x4*)(buf + LDS_QV + ((2 + c.hh) * D + 32 * cb + c.l32) * 16);
    const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    st.acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pk, st.acc[cb], 0, 0, 0, 127, 0, 127);
  }
}

// One bf16 tile (anchors: ANCHOR = true, keys from the LDS list; window: 64 aligned keys
// from kt0) for the wave's 32 queries.
template <bool ANCHOR>
__device__ inline void compute_tile_bf(const PrefillParams& p, const Ctx& c, const uint8_t* lds,
                                       const int* anc_s, int kt0, RowState& st) {
  int keyv[4][4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      keyv[kb][r] = ANCHOR ? anc_s[16 * kb + 4 * c.j + r] : kt0 + 16 * kb + 4 * c.j + r;
  f32x4 S[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = c.r0w + 16 * qb + c.l16;
    const int rowc = row < c.N ? row : c.N - 1;  // padded rows: any finite query, never stored
    const uint16_t* qrow = p.q + ((size_t)c.h * c.N + rowc) * D + 8 * c.j;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = keyv[kb][r];
        const bool ok = ANCHOR ? (key >= 0 && key <= row - WIN) : (key <= row && key >= row - WIN + 1);
        S[qb][kb][r] = ok ? 0.0f : -INFINITY;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 qfr = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 32 * ks));
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 kfr = *(const bf16x8*)(lds + (16 * kb + c.l16) * KB_LD + 2 * (32 * ks + 8 * c.j));
        S[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfr, qfr, S[qb][kb], 0, 0, 0);
      }
    }
  }
  bool valid[2];
  float tmax[2], muse[2], mt[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    mt[qb] = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      mt[qb] = fmaxf(mt[qb], fmaxf(fmaxf(S[qb][kb][0], S[qb][kb][1]), fmaxf(S[qb][kb][2], S[qb][kb][3])));
  }
  col4_max2_f(mt[0], mt[1]);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    valid[qb] = mt[qb] > -INFINITY;
    tmax[qb] = mt[qb] * AL2;
  }
  row_update(c, st, valid, tmax, 0.0f, muse);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    // bf16 pairs (r 0-1, r 2-3) of keys 16 kb + 4 j + r, block 0 then block 1: the row-sum B
    // operand; the two in-place swaps turn it into the P.V B operand (keys 16 kb + 8 hh + e)
    u32x4 b;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][kb][r], AL2, -muse[qb]));
      b[2 * qb] = pack_bf16x2(pv[0], pv[1]);
      b[2 * qb + 1] = pack_bf16x2(pv[2], pv[3]);
    }
    st.lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.selb, __builtin_bit_cast(bf16x8, b), st.lacc, 0, 0, 0);
    const auto s0 = __builtin_amdgcn_permlane16_swap(b[0], b[2], false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(b[1], b[3], false, false);
    const bf16x8 pb = __builtin_bit_cast(bf16x8, (u32x4){s0[0], s1[0], s0[1], s1[1]});
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const bf16x8 vf = *(const bf16x8*)(lds + LDS_V + ((2 * kb + c.hh) * D + 32 * cb + c.l32) * 16);
      st.acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, st.acc[cb], 0, 0, 0);
    }
  }
}

// Segment A (quantized tiles 0 .. nA-1) for one workgroup.
//
// Software pipeline over a ring of 4 LDS tile buffers, one barrier per tile.  Iteration t:
//   store tile t+3 (fetched into registers during iteration t-1) into buffer (t+3) % 4 --
//   free since the previous barrier, its last reader being P.V(t-1);
//   fetch tile t+4 into registers;
//   P.V(t) (MFMA, codes from the previous iteration), softmax(t+1) (VALU) and, under it,
//   QK^T(t+2) (MFMA; tile t+2 was stored one iteration earlier);
//   barrier (tile t+3 visible to everyone).
// The exact per-tile max update of softmax(t+1) may rescale the accumulator: that multiply
// waits for P.V(t), as the order of Alg. 2 requires.  Tiles past the wave's last row
// (64 t > r0w + 31 - 128) are loaded for the other waves but not computed.  While every step
// is due and QK^T(t+2) is an interior tile the loop runs unrolled by four, so the buffer
// offsets are constants and no step is conditional; the rest runs one conditional step at a
// time.
// exp2 scale of a tile's scores: s_Q s_K alpha log2(e) for INT8 codes, alpha log2(e) for MX
// dots (already scaled)
template <int BULK, bool TINY>
__device__ inline float tile_c2(float sq_u, float sk) {
  if (BULK == 1) return AL2;
  float c2 = uniform_f(sq_u * sk * AL2);
  if (TINY) c2 = c2 > 0.0f ? c2 : 1.0f;  // a zero scale means every valid dot is 0
  return c2;
}

template <int BULK>
struct PipeA {
  TileQRegs pre;      // tile in flight from global memory
  float sk1, sk2, sk3;  // K scales of tiles t+1, t+2, t+3
  typename BulkT<BULK>::S S2[2][4];  // scores of tile t+1
  i32x8 pk;           // P codes of tile t
};

template <int BULK, bool TINY, int PH>
__device__ inline void segment_a_main(const PrefillParams& p, const Ctx& c, uint8_t* lds, const QOps& q,
                                      int nA, float sq_u, int t, PipeA<BULK>& a, RowState& st) {
  store_tile_q<BULK>(c, lds + ((PH + 3) % RING) * LDS_QBUF, a.pre);
  a.sk3 = a.pre.sk;
  fetch_tile_q<BULK>(p, c, min(t + 4, nA - 1), a.pre);  // past the end: loaded, never stored
  pv_tile_q(c, lds + PH * LDS_QBUF, a.pk, st);
  softmax_tile_q<BULK, TINY, true>(c, a.S2, tile_c2<BULK, TINY>(sq_u, a.sk1), st, a.pk,
                                   lds + ((PH + 2) % RING) * LDS_QBUF, &q, t + 2);
  __syncthreads();
  a.sk1 = a.sk2;
  a.sk2 = a.sk3;
}

template <int BULK, bool TINY>
__device__ inline void segment_a_tail(const PrefillParams& p, const Ctx& c, uint8_t* lds, const QOps& q,
                                      int nA, int nAw, float sq_u, int t, PipeA<BULK>& a, RowState& st) {
  if (t + 3 < nA) {
    store_tile_q<BULK>(c, lds + ((t + 3) % RING) * LDS_QBUF, a.pre);
    a.sk3 = a.pre.sk;
  }
  if (t + 4 < nA) fetch_tile_q<BULK>(p, c, t + 4, a.pre);
  if (t < nAw) pv_tile_q(c, lds + (t % RING) * LDS_QBUF, a.pk, st);
  if (t + 1 < nAw) softmax_tile_q<BULK, TINY>(c, a.S2, tile_c2<BULK, TINY>(sq_u, a.sk1), st, a.pk);
  if (t + 2 < nAw) qk_tile<BULK>(c, lds + ((t + 2) % RING) * LDS_QBUF, q, t + 2, a.S2);
  __syncthreads();
  a.sk1 = a.sk2;
  a.sk2 = a.sk3;
}

template <int BULK, bool TINY>
__device__ inline void segment_a(const PrefillParams& p, const Ctx& c, uint8_t* lds, const QOps& q,
                                 int nA, float sq_u, RowState& st) {
  const int nAw = c.r0w + 31 - WIN >= 0 ? ((c.r0w + 31 - WIN) >> 6) + 1 : 0;
  // interior tiles (every key at least 128 before every row of the wave): 64 t + 63 <= r0w - 128
  const int nInt = c.r0w - WIN - 63 >= 0 ? ((c.r0w - WIN - 63) >> 6) + 1 : 0;
  if (nA <= 0) return;
  PipeA<BULK> a;
  float sk0 = 0.0f;
  a.sk1 = a.sk2 = a.sk3 = 0.0f;
  __syncthreads();  // nothing else uses the tile buffers now
  fetch_tile_q<BULK>(p, c, 0, a.pre);
  store_tile_q<BULK>(c, lds, a.pre);
  sk0 = a.pre.sk;
  if (nA > 1) {
    fetch_tile_q<BULK>(p, c, 1, a.pre);
    store_tile_q<BULK>(c, lds + LDS_QBUF, a.pre);
    a.sk1 = a.pre.sk;
  }
  if (nA > 2) {
    fetch_tile_q<BULK>(p, c, 2, a.pre);
    store_tile_q<BULK>(c, lds + 2 * LDS_QBUF, a.pre);
    a.sk2 = a.pre.sk;
  }
  if (nA > 3) fetch_tile_q<BULK>(p, c, 3, a.pre);
  __syncthreads();
  // prologue: scores and P codes of tile 0, scores of tile 1
  if (nAw > 0) {
    qk_tile<BULK>(c, lds, q, 0, a.S2);
    softmax_tile_q<BULK, TINY>(c, a.S2, tile_c2<BULK, TINY>(sq_u, sk0), st, a.pk);
  }
  if (1 < nAw) qk_tile<BULK>(c, lds + LDS_QBUF, q, 1, a.S2);
  int t = 0;
  // group t .. t+3: stores up to tile t+6 < nA, QK^T up to tile t+5 interior (< nInt <= nAw)
  for (; t + 6 < nA && t + 5 < nInt; t += RING) {
    segment_a_main<BULK, TINY, 0>(p, c, lds, q, nA, sq_u, t, a, st);
    segment_a_main<BULK, TINY, 1>(p, c, lds, q, nA, sq_u, t + 1, a, st);
    segment_a_main<BULK, TINY, 2>(p, c, lds, q, nA, sq_u, t + 2, a, st);
    segment_a_main<BULK, TINY, 3>(p, c, lds, q, nA, sq_u, t + 3, a, st);
  }
  for (; t < nA; ++t) segment_a_tail<BULK, TINY>(p, c, lds, q, nA, nAw, sq_u, t, a, st);
}

template <int BULK>
__global__ void __launch_bounds__(256, 2) pf_attn_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_TOTAL];
  __shared__ int anc_s[64];
  __shared__ float qmax[4];
  __shared__ float skmin[4];
  __shared__ int nb_anchor_s;

  // Workgroup -> (query block, Q head), longest rows first.  Workgroups are dispatched to the
  // 8 XCDs round-robin (id % 8); the G Q heads of one KV group read the same K/V tiles in the
  // same order, so they are given consecutive ids on one XCD and share its L2.
  const int nQB = p.Npad / WG_ROWS;
  const int groups = nQB * p.Hkv, bid = (int)blockIdx.x;
  int qblk, hq;
  if (groups % 8 == 0) {
    const int i = bid >> 3, gi = (i / p.G) * 8 + (bid & 7);
    qblk = nQB - 1 - gi / p.Hkv;
    hq = (gi % p.Hkv) * p.G + i % p.G;
  } else {
    qblk = nQB - 1 - bid / p.Hq;
    hq = bid % p.Hq;
  }
  Ctx c;
  c.h = hq;
  c.hk = c.h / p.G;
  const int r0 = qblk * WG_ROWS;
  c.tid = threadIdx.x;
  const int wave = c.tid >> 6, lane = c.tid & 63;
  c.wave = wave;
  c.l16 = lane & 15;
  c.j = lane >> 4;
  c.l32 = lane & 31;
  c.hh = lane >> 5;
  c.qsel = (lane >> 4) & 1;
  {
    const bool lo_rows = (lane & 15) < 8;  // row-sum selector A operand rows 0-7 vs 8-15
    c.sel8 = lo_rows ? (i64)0x38383838L : (i64)0x3838383800000000L;
    const __bf16 one = (__bf16)1.0f, zero = (__bf16)0.0f;
    const __bf16 a = lo_rows ? one : zero, b = lo_rows ? zero : one;
    c.selb = (bf16x8){a, a, a, a, b, b, b, b};
  }
  c.r0w = __builtin_amdgcn_readfirstlane(r0 + 32 * wave);  // wave-uniform: scalar branches
  c.N = p.N;
  c.Npad = p.Npad;
  c.nb64 = p.Npad >> 6;

  // ---- Q: INT8 codes (block maximum over the 64-row block, exchanged through LDS) or MXFP4
  // codes of the lane's channel block; the codes are also stored in the workspace
  QOps qo;
  float sq = 0.0f;
  if (wave == 0) {
    // the number of anchors some row of the workgroup may use (a <= r0 + 127 - 128), by a
    // 64-way search of the sorted list: each round probes 64 entries at once, so up to 4096
    // anchors take two rounds of loads (a binary search by one thread took about ten, and the
    // workgroup's first barrier waited for them)
    const int32_t* anc = p.anchors + (size_t)c.hk * p.n_anchor;
    const int lim = r0 + WG_ROWS - 1 - WIN;
    int lo = 0, hi = p.n_anchor;  // the count lies in [lo, hi]
    while (lo < hi) {
      const int step = (hi - lo + 63) >> 6;
      const int idx = lo + (lane + 1) * step - 1;  // probe l: is the count above idx?
      const bool le = idx < hi && anc[idx] <= lim;
      const int nlo = lo + step * __builtin_popcountll(__ballot(le));
      hi = min(hi, nlo + step - 1);
      lo = nlo;
    }
    if (lane == 0) nb_anchor_s = lo;
  }
  if constexpr (BULK == 1) {
    // lane (qb, l16, j): channels 32 j .. 32 j + 31 of row 16 qb + l16 -- one MX block
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int row = c.r0w + 16 * qb + c.l16;
      float x[32];
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const u32x4 w = row < c.N ? *(const u32x4*)(p.q + ((size_t)c.h * c.N + row) * D + 32 * c.j + 8 * v4)
                                  : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * v4 + 2 * e] = bf_lo(w[e]);
          x[8 * v4 + 2 * e + 1] = bf_hi(w[e]);
        }
      }
      const int e = mxfp4_block(x, qo.q4[qb]);
      qo.qs[qb] = (uint32_t)(e + 127);
      // workspace row: codes of block j at bytes 16 j, scale byte at 64 + j
      int8_t* qrow = p.q8 + ((size_t)c.h * c.Npad + row) * D;
      *(u32x4*)(qrow + 16 * c.j) = qo.q4[qb];
      qrow[64 + c.j] = (int8_t)(e + 127);
    }
    __syncthreads();
  } else {
    u32x4 qf[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int row = c.r0w + 16 * qb + c.l16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qf[qb][ks] = row < c.N ? *(const u32x4*)(p.q + ((size_t)c.h * c.N + row) * D + 32 * ks + 8 * c.j)
                               : (u32x4){0u, 0u, 0u, 0u};
    }
    float amax = 0.0f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          amax = fmaxf(amax, fmaxf(fabsf(bf_lo(qf[qb][ks][e])), fabsf(bf_hi(qf[qb][ks][e]))));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, shfl_xor_f(amax, o));
    if (lane == 0) qmax[wave] = amax;
    __syncthreads();
    sq = __fdiv_rn(fmaxf(qmax[wave], qmax[wave ^ 1]), 127.0f);
    const float rq = int8_rcp(sq);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int s8 = 0; s8 < 2; ++s8) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const u32x4 x = qf[qb][2 * s8 + hh];
          uint32_t w0 = 0, w1 = 0;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            w0 |= (uint32_t)(int8_code(bf_lo(x[e]), sq, rq) & 0xff) << (16 * e);
            w0 |= (uint32_t)(int8_code(bf_hi(x[e]), sq, rq) & 0xff) << (16 * e + 8);
            w1 |= (uint32_t)(int8_code(bf_lo(x[2 + e]), sq, rq) & 0xff) << (16 * e);
            w1 |= (uint32_t)(int8_code(bf_hi(x[2 + e]), sq, rq) & 0xff) << (16 * e + 8);
          }
          qo.qi[qb][s8][2 * hh] = (int)w0;
          qo.qi[qb][s8][2 * hh + 1] = (int)w1;
        }
        const int row = c.r0w + 16 * qb + c.l16;
        *(i32x4*)(p.q8 + ((size_t)c.h * c.Npad + row) * D + 64 * s8 + 16 * c.j) = qo.qi[qb][s8];
      }
    }
    if (lane == 0 && (wave & 1) == 0) p.sq[(size_t)c.h * c.nb64 + (c.r0w >> 6)] = sq;
  }

  RowState st;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) st.m[qb] = -INFINITY;
  st.lacc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) st.acc[cb] = (f32x16){};

  // ---- segment A: quantized tiles
  const int lastA = r0 + WG_ROWS - 1 - WIN;
  const int nA = lastA >= 0 ? (lastA >> 6) + 1 : 0;
  // Masked INT8 scores underflow exp2 only when s_Q s_K is not tiny; the rare wave with a
  // tiny product over its tiles runs the variant that zeroes them explicitly.  MX scores are
  // floats whose masked entries are -inf.
  if constexpr (BULK == 1) {
    segment_a<1, false>(p, c, lds, qo, nA, 0.0f, st);
  } else {
    float m = INFINITY;
    for (int t = c.tid; t < nA; t += 256) m = fminf(m, p.sk[(size_t)c.hk * c.nb64 + t]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fminf(m, shfl_xor_f(m, o));
    if (lane == 0) skmin[wave] = m;
    __syncthreads();
    m = fminf(fminf(skmin[0], skmin[1]), fminf(skmin[2], skmin[3]));
    const float sq_u = uniform_f(sq);
    if (sq_u * m * AL2 >= C2_FAST_MIN)
      segment_a<0, false>(p, c, lds, qo, nA, sq_u, st);
    else
      segment_a<0, true>(p, c, lds, qo, nA, sq_u, st);
  }
  // acc holds sum E4M3(448 p) * code(V): scale to values
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 svc = *(const f32x4*)(p.sv + c.hk * D + 32 * cb + 8 * i + 4 * c.hh) * (1.0f / 448.0f);
#pragma unroll
      for (int r = 0; r < 4; ++r) st.acc[cb][4 * i + r] *= svc[r];
    }
  }
  st.lacc *= (1.0f / 448.0f);

  // ---- segment B: anchor tiles (64 consecutive list entries each)
  const int32_t* anc_g = p.anchors + (size_t)c.hk * p.n_anchor;
  const int nB = (nb_anchor_s + 63) >> 6;
  const int n_anchor = p.n_anchor;
  for (int u = 0; u < nB; ++u) {
    __syncthreads();
    if (c.tid < 64) {
      const int idx = 64 * u + c.tid;
      anc_s[c.tid] = idx < n_anchor ? anc_g[idx] : -1;
    }
    load_tile_bf(c, lds, p.ka16 + ((size_t)c.hk * p.n_anchor_pad + 64 * u) * D, 64,
                 p.va16 + ((size_t)c.hk * (p.n_anchor_pad >> 5) + 2 * u) * D * 32, [&](int row) { return row; });
    __syncthreads();
    const int a0 = anc_s[0];
    if (a0 >= 0 && a0 <= c.r0w + 31 - WIN) compute_tile_bf<true>(p, c, lds, anc_s, 0, st);
  }

  // ---- segment C: window tiles (aligned)
  const int tC0 = max(0, r0 - WIN + 1) >> 6, tC1 = (r0 + WG_ROWS - 1) >> 6;
  for (int t = tC0; t <= tC1; ++t) {
    const int kt0 = 64 * t;
    __syncthreads();
    load_tile_bf(c, lds, p.k + (size_t)c.hk * c.N * D, c.N,
                 p.vt16 + ((size_t)c.hk * (c.Npad >> 5) + 2 * t) * D * 32, [&](int row) { return kt0 + row; });
    __syncthreads();
    if (!(kt0 > c.r0w + 31 || kt0 + 63 < c.r0w - WIN + 1)) compute_tile_bf<false>(p, c, lds, anc_s, kt0, st);
  }

  // ---- epilogue: o = acc / l  (every real row has its own key in the window)
  const int orow = c.r0w + c.l32;
  if (orow < c.N) {
    // row sum of query l32 = block qsel: this lane's when qsel == hh, else lane l ^ 32's
    const auto ls = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.lacc[0]), __float_as_uint(st.lacc[0]), false, false);
    const float other = __uint_as_float(c.hh ? ls[0] : ls[1]);
    const float inv = 1.0f / (c.qsel == c.hh ? st.lacc[0] : other);
    float* dst = p.o + ((size_t)c.h * c.N + orow) * D + 4 * c.hh;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(f32x4*)(dst + 32 * cb + 8 * i) = (f32x4){st.acc[cb][4 * i], st.acc[cb][4 * i + 1], st.acc[cb][4 * i + 2],
                                                   st.acc[cb][4 * i + 3]} * inv;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  const int Hkv = p.Hkv;
  // the anchor gather (two tiles per workgroup), then K quantization and bitmap per 64-key block
  const dim3 g1((p.n_anchor_pad / 32 + 1) / 2 + p.Npad / KBLK, Hkv);
  if (p.bulk == 1)
    hipLaunchKernelGGL(pf_kquant_kernel<1>, g1, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(pf_kquant_kernel<0>, g1, dim3(256), 0, stream, p);
  hipLaunchKernelGGL(pf_vscale_kernel, dim3(Hkv), dim3(1024), 0, stream, p);
  hipLaunchKernelGGL(pf_vquant_kernel, dim3(p.Npad / 32, Hkv), dim3(128), 0, stream, p);
  if (p.bulk == 1)
    hipLaunchKernelGGL(pf_attn_kernel<1>, dim3((p.Npad / WG_ROWS) * p.Hq), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(pf_attn_kernel<0>, dim3((p.Npad / WG_ROWS) * p.Hq), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hyq

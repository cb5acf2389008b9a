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
//    every lane owns a distinct (head, group).  At GQA 8 and 16 a wave holds two such column
//    blocks (8 Q heads) and feeds both from one extraction of the tile's codes.  INT4 codes
//    enter as f16 *subnormals*
//    (bits 0x000c == c * 2^-24, exact): 8 codes become 8 MFMA operands with one shift and four
//    masks (two of the four pairs come out multiplied by 16; the other operand carries 1/16 on
//    those k-slots).  The per-group scale and min are applied in fp32 afterwards:
//    q.k = sum_g s_g * (q_g . code_g) + m_g * sum(q_g).
//  * Sum over the 4 groups with two DPP quad permutes; max across the tile with two lane swaps.
//  * P.V on the same MFMA: A = V codes of 16 channels x 8 positions per lane, B = P' = p * s_V
//    times a power of two 2^e (the MFMA output layout of the K product is exactly the B layout
//    needed here), split into f16 hi + lo parts so the weights keep ~22 bits.  Each MFMA column
//    keeps its own e, chosen so that the largest s_V seen times 2^e stays inside [4, 2^15): P'
//    never overflows f16 and never sinks into its subnormals for any fp16 scale.  When a tile's
//    s_V leave that band, e moves and the accumulator is rescaled by the exact power of two
//    (as the softmax rescales it when the max grows).  The V min enters as sum p * m_V in fp32.
//  * q enters the f16 operands times a power of two per head that puts its largest |q| in
//    [2^13, 2^14), undone in fp32 after the MFMA: no f16 overflow and no subnormal q.
//  * bf16 tiles (anchors, staging, window) use the bf16 MFMA with the same softmax state.
//  * Every load is a coalesced 1 KB read of one 5 KB tile record (layouts in hyq_common.h); the
//    next INT4 tile is loaded while the current one is computed (two register sets).  Worker w
//    of a head takes tiles w, w + NW, ... so the head's workers sweep its records together.
//  * 4 waves per workgroup merge their states in LDS and write one record per split; a second
//    small launch merges the records.
#include <mutex>

#include "hyq_common.h"
#include "hyq_launch.h"

namespace hyq {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
// V weight scale 2^e of an MFMA column: the column's largest s_V times 2^e is kept inside
// [PS_LO, PS_HI); a move puts it in [2^PS_TARGET - 1, 2^PS_TARGET).  The start value 2^8 keeps
// every unit-scale input (s_V below 2^7) inside the band.
constexpr float PS_INIT = 256.0f;
constexpr float PS_HI = 32768.0f;
constexpr float PS_LO = 4.0f;
constexpr int PS_TARGET = 8;
// q scale: the head's largest |q| times 2^sigma lands in [2^(Q_TARGET-1), 2^Q_TARGET)
constexpr int Q_TARGET = 14;

// 8 INT4 codes (one dword) -> 8 f16 MFMA operands (subnormal bit patterns).  Element order:
// nibbles 0,4 | 1,5 (x16) | 2,6 | 3,7 (x16).
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

struct WaveState {
  float m, l, mt;
  float ps, ps_hi, ps_lo;  // V weight scale 2^e of this lane's column, and the band on max s_V
  f32x4 acc[8];
};

// Largest fp16 scale s_V of this lane's 8 positions (low halves of the (scale, min) pairs;
// the scales are >= 0, so the packed f16 max of the low halves is their max).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ inline float max_vscale(const uint32_t (&smv)[8]) {
  f16x2 a[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    a[j] = __builtin_elementwise_max(__builtin_bit_cast(f16x2, smv[2 * j]), __builtin_bit_cast(f16x2, smv[2 * j + 1]));
  const f16x2 b = __builtin_elementwise_max(__builtin_elementwise_max(a[0], a[1]), __builtin_elementwise_max(a[2], a[3]));
  return (float)b[0];
}

// Keeps the column's V weight scale inside its band for a tile whose largest s_V on this lane
// is smax: the four lanes of a column (l, l^16, l^32, l^48) agree on the column maximum, and a
// column that leaves the band moves its scale and rescales its accumulator exactly.  The
// common case is one compare per lane and one wave vote.
__device__ inline void track_vscale(WaveState& st, float smax) {
  const bool out = smax >= st.ps_hi || (smax > 0.f && smax < st.ps_lo);
  if (__builtin_amdgcn_ballot_w64(out) == 0) return;
  const float cm = col4_max(smax);
  if (cm >= st.ps_hi || (cm > 0.f && cm < st.ps_lo)) {
    int ex;
    (void)frexpf(cm, &ex);  // cm = f 2^ex, f in [0.5, 1)
    const float ps = ldexpf(1.0f, PS_TARGET - ex);
    const float f = ps / st.ps;  // a power of two: exact
#pragma unroll
    for (int r = 0; r < 8; ++r) st.acc[r] *= f;
    st.ps = ps;
    st.ps_hi = PS_HI / ps;
    st.ps_lo = PS_LO / ps;
  }
}

// 8 INT8 codes (two dwords) -> 8 f16 MFMA operands (subnormal bit patterns, exact: codes <=
// 255).  Element order: bytes 0,2 | 1,3 | 4,6 | 5,7 (kslot_byte).
__device__ inline f16x8 codes8_to_f16(uint32_t x0, uint32_t x1) {
  u32x4 a;
  a[0] = x0 & 0x00FF00FFu;
  a[1] = (x0 >> 8) & 0x00FF00FFu;
  a[2] = x1 & 0x00FF00FFu;
  a[3] = (x1 >> 8) & 0x00FF00FFu;
  return __builtin_bit_cast(f16x8, a);
}

// one 32-slot tile record of the quantized store for this lane: BK dwords of K codes per
// 16-slot block (the lane's slot and channel group), 2 BV dwords of V codes (the lane's channel
// row at its quad's 8 slots, all 8 channel blocks), and the scale/min quads
template <int BK, int BV>
struct QTile {
  uint32_t kc0[BK], kc1[BK], vc[2 * BV];
  u32x4 ks0, ks1, vs0, vs1;
};

// A load of the streamed cache.  NT: a nontemporal load (the slab is read once per step and
// by one workgroup: a plain streaming read reaches about 6.1 TB/s on gfx950, a nontemporal one
// 6.9).  Head blocks that share a slab through L2 (GQA above 4) keep plain loads.
template <bool NT, typename T>
__device__ inline T ld_stream(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
// n dwords at p (16-byte aligned for n >= 4, 8-byte aligned for n = 2)
template <bool NT, int N>
__device__ inline void load_dw(uint32_t (&d)[N], const uint8_t* p) {
  if constexpr (N == 2) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = ld_stream<NT>((const u32x2*)p);
    d[0] = v[0];
    d[1] = v[1];
  } else {
#pragma unroll
    for (int h = 0; h < N / 4; ++h) {
      const u32x4 v = ld_stream<NT>((const u32x4*)(p + 16 * h));
#pragma unroll
      for (int e = 0; e < 4; ++e) d[4 * h + e] = v[e];
    }
  }
}

// all loads of one tile record for this lane; every one is a coalesced read of the record
template <bool NT, int BK, int BV>
__device__ inline void load_int4_tile(QTile<BK, BV>& x, const uint8_t* slab, int t, uint32_t lane, uint32_t smoff) {
  typedef QL<BK, BV> L;
  const uint8_t* rec = slab + (size_t)t * L::TB;
  load_dw<NT, BK>(x.kc0, rec + lane * L::CB);
  load_dw<NT, BK>(x.kc1, rec + 64 * L::CB + lane * L::CB);
  if constexpr (BV == 2) {
    load_dw<NT, 4>(*(uint32_t(*)[4])x.vc, rec + L::VC + lane * 16);
  } else {  // two halves (channel blocks 0-3, 4-7) of 64 x 4 BV bytes
    load_dw<NT, BV>(*(uint32_t(*)[BV])x.vc, rec + L::VC + lane * 4 * BV);
    load_dw<NT, BV>(*(uint32_t(*)[BV])(x.vc + BV), rec + L::VC + 256 * BV + lane * 4 * BV);
  }
  x.ks0 = ld_stream<NT>((const u32x4*)(rec + L::KSM + smoff));
  x.ks1 = ld_stream<NT>((const u32x4*)(rec + L::KSM + 256 + smoff));
  x.vs0 = ld_stream<NT>((const u32x4*)(rec + L::VSM + smoff));
  x.vs1 = ld_stream<NT>((const u32x4*)(rec + L::VSM + 256 + smoff));
}
// MFMA operand of 8 codes: K step tt of a block's chunk (B = BK), or V channel block rr (B = BV)
template <int B, int N>
__device__ inline f16x8 qcodes(const uint32_t (&c)[N], int i) {
  if constexpr (B == 4) return codes_to_f16(c[i]);
  else if constexpr (B == 8) return codes8_to_f16(c[2 * i], c[2 * i + 1]);
  else return codes2_to_f16(c[i >> 1], i & 1);
}
// factor the other operand carries for element e of a code operand
template <int B>
__device__ inline float code_factor(int e) {
  if constexpr (B == 4) return (e & 2) ? 0.0625f : 1.0f;
  else if constexpr (B == 8) return 1.0f;
  else return (e & 6) == 0 ? 1.0f : (e & 6) == 2 ? 0.25f : (e & 6) == 4 ? 0.0625f : 0.015625f;
}
// channel (inside the 32-channel group) of element e of K step tt
template <int B>
__device__ inline int kstep_channel(int tt, int e) {
  if constexpr (B == 4) return 8 * tt + kslot_nibble(e);
  else if constexpr (B == 8) return 8 * tt + kslot_byte(e);
  else return 16 * (tt >> 1) + code2_of(tt & 1, e);
}

// online-softmax update for one tile; sc[8] are log2-domain scores (-inf = masked)
__device__ inline void tile_softmax(WaveState& st, const float (&sc)[8], float (&pv)[8]) {
  float tmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
  tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
  tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
  if (tmax > st.m) {  // rescale only when the running max grows
    const float c = __builtin_amdgcn_exp2f(st.m - tmax);
    st.l *= c;
    st.mt *= c;
#pragma unroll
    for (int r = 0; r < 8; ++r) st.acc[r] *= c;
    st.m = tmax;
  }
  const float mref = st.m == -INFINITY ? 0.f : st.m;  // all masked so far: every p is 0
#pragma unroll
  for (int j = 0; j < 8; ++j) pv[j] = __builtin_amdgcn_exp2f(sc[j] - mref);
  st.l += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
}

// One INT4 tile for HB column blocks of 4 Q heads each (HB = 2 serves 8 Q heads of one KV head
// from one load of the tile): the code operands are extracted once and feed every block's
// MFMAs; each block keeps its own softmax state.
template <int BK, int BV, bool MASK, int HB>
__device__ inline void int4_tile(WaveState (&st)[HB], const QTile<BK, BV>& x, const f16x8 (&bq)[HB][4],
                                 const float (&qsum24)[HB], const float (&c_int4)[HB], int base, int n_int4,
                                 int q4) {
  f32x4 S0[HB], S1[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    S0[hb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    S1[hb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const f16x8 k0 = qcodes<BK>(x.kc0, tt), k1 = qcodes<BK>(x.kc1, tt);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      S0[hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, bq[hb][tt], S0[hb], 0, 0, 0);
      S1[hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, bq[hb][tt], S1[hb], 0, 0, 0);
    }
  }
  bool valid[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    valid[r] = !MASK || base + 4 * q4 + r < n_int4;
    valid[4 + r] = !MASK || base + 16 + 4 * q4 + r < n_int4;
  }
  float vmax;
  {
    uint32_t smv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      smv[j] = j < 4 ? x.vs0[j] : x.vs1[j - 4];
      if (MASK) smv[j] = valid[j] ? smv[j] : 0u;  // unused slots may hold any bits
    }
    vmax = max_vscale(smv);
  }
  f16x8 bhi[HB], blo[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    float sc[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v0 = fmaf(half_lo(x.ks0[r]), S0[hb][r], half_hi(x.ks0[r]) * qsum24[hb]);
      float v1 = fmaf(half_lo(x.ks1[r]), S1[hb][r], half_hi(x.ks1[r]) * qsum24[hb]);
      v0 += dpp_quad_xor1(v0);
      v1 += dpp_quad_xor1(v1);
      v0 += dpp_quad_xor2(v0);
      v1 += dpp_quad_xor2(v1);
      sc[r] = v0 * c_int4[hb];
      sc[4 + r] = v1 * c_int4[hb];
      if (MASK) {
        sc[r] = valid[r] ? sc[r] : -INFINITY;
        sc[4 + r] = valid[4 + r] ? sc[4 + r] : -INFINITY;
      }
    }
    track_vscale(st[hb], vmax);
    float pv[8];
    tile_softmax(st[hb], sc, pv);
    float mt = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t smv = j < 4 ? x.vs0[j] : x.vs1[j - 4];
      const float pj = pv[j];
      // code operands scaled per k-slot (INT4: x16 on k-slots 2,3,6,7; 2-bit: 4^(j >> 1))
      float pp = pj * half_lo(smv) * (st[hb].ps * code_factor<BV>(j));
      float mm = pj * half_hi(smv);
      if (MASK) {  // unused slots may hold any scale/min bits: keep them out entirely
        pp = valid[j] ? pp : 0.f;
        mm = valid[j] ? mm : 0.f;
      }
      mt += mm;
      const _Float16 h = (_Float16)pp;
      bhi[hb][j] = h;
      blo[hb][j] = (_Float16)(pp - (float)h);
    }
    st[hb].mt += mt;
  }
  f16x8 a[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) a[rr] = qcodes<BV>(x.vc, rr);
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
    for (int rr = 0; rr < 8; ++rr)
      st[hb].acc[rr] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[rr], bhi[hb], st[hb].acc[rr], 0, 0, 0);
#pragma unroll
    for (int rr = 0; rr < 8; ++rr)
      st[hb].acc[rr] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[rr], blo[hb], st[hb].acc[rr], 0, 0, 0);
  }
}

// What one workgroup reads and writes: the slabs of one (sequence, KV head), its counters,
// its split, the q rows of the KV group's Q heads and the group's first partial record.
struct HeadWork {
  const uint8_t* int4;
  const uint16_t *a_k, *a_v, *s_k, *s_v, *w_k, *w_v;
  const uint16_t* q;
  float* rec;
  float* out;  // with a single split: the group's output rows, written directly (no merge launch)
  int n_int4, n_anchor, n_staged, n_win;
  int n_splits, split;
};

// The work of one workgroup: split `split` of KV head `hkv` of sequence `b`, for Q-head block
// `sub` (Q heads H sub .. H sub + H - 1 of the KV group, H = 4 per column block it serves).
struct Unit {
  int split, hkv, sub, b;
};

// Uniform batch: a 1-D grid.  With one head block per KV head (GQA up to 4) the workgroup id
// enumerates (split, KV head, sequence), split fastest.  With several head blocks, the blocks
// of one (split, KV head, sequence) get ids 8 apart: workgroups are dealt to the 8 XCDs in
// turn, so they run on one XCD one after the other and read the same tiles together -- the
// slab is streamed from HBM once and the other blocks' reads hit that XCD's L2.  The id
// space is padded to whole groups of 8; padding workgroups return at once.
__host__ __device__ inline int decode_grid_size(int n_splits, int Hkv, int B, int G) {
  const int nsub = decode_head_blocks(G), units = n_splits * Hkv * B;
  return nsub == 1 ? units : (units + 7) / 8 * 8 * nsub;
}
__device__ inline bool unit_of(const DecodeParams& p, Unit& u) {
  const int nsub = decode_head_blocks(p.G);
  const int L = blockIdx.x;
  int r;  // index over (split, KV head, sequence), split fastest
  if (nsub == 1) {
    r = L;
    u.sub = 0;
  } else {
    const int k = L >> 3;
    u.sub = k % nsub;
    r = (k / nsub) * 8 + (L & 7);
  }
  const int per_b = p.n_splits * p.Hkv;
  if (r >= per_b * p.B) return false;
  u.split = r % p.n_splits;
  u.hkv = (r / p.n_splits) % p.Hkv;
  u.b = r / per_b;
  return true;
}
// variable-length batch: grid (split of the batch, KV head x head block)
__device__ inline bool unit_of(const RaggedDecodeParams& p, Unit& u) {
  const int nsub = decode_head_blocks(p.G);
  u.hkv = blockIdx.y / nsub;
  u.sub = blockIdx.y % nsub;
  u.split = 0;  // from the split map
  u.b = 0;
  return true;
}

// uniform batch: every sequence has the same counters
template <int BK, int BV>
__device__ inline HeadWork head_work(const DecodeParams& p, const Unit& u) {
  const int hkv = u.hkv;
  const size_t hb = (size_t)u.b * p.Hkv + hkv;
  const size_t qh = (size_t)u.b * p.Hkv * p.G + (size_t)hkv * p.G;
  HeadWork h = {};
  h.int4 = p.int4 + hb * (size_t)p.int4_cap * QL<BK, BV>::SLOT;
  h.a_k = p.a_k + hb * (size_t)p.anchor_cap * D;
  h.a_v = p.a_v + hb * (size_t)p.anchor_cap * D;
  h.s_k = p.s_k + hb * (size_t)p.staging_cap * D;
  h.s_v = p.s_v + hb * (size_t)p.staging_cap * D;
  h.w_k = p.w_k + hb * (size_t)WIN * D;
  h.w_v = p.w_v + hb * (size_t)WIN * D;
  h.q = p.q + qh * D;
  h.rec = p.part + qh * p.n_splits * (D + 2);
  h.out = p.n_splits == 1 ? p.o + qh * D : nullptr;
  h.n_int4 = p.n_int4;
  h.n_anchor = p.n_anchor;
  h.n_staged = p.n_staged;
  h.n_win = p.n_win;
  h.n_splits = p.n_splits;
  h.split = u.split;
  return h;
}

// variable-length batch: grid x enumerates the splits of all sequences (split_map), each
// sequence in its own single-sequence cache
template <int BK, int BV>
__device__ inline HeadWork head_work(const RaggedDecodeParams& p, const Unit& u) {
  const int hkv = u.hkv;
  const uint32_t m = p.split_map[blockIdx.x];
  const int seq = (int)(m >> 16);
  const RaggedSeq& d = p.seqs[seq];
  HeadWork h = {};
  h.int4 = d.int4 + (size_t)hkv * d.int4_cap * QL<BK, BV>::SLOT;
  h.a_k = d.a_k + (size_t)hkv * d.anchor_cap * D;
  h.a_v = d.a_v + (size_t)hkv * d.anchor_cap * D;
  h.s_k = d.s_k + (size_t)hkv * d.staging_cap * D;
  h.s_v = d.s_v + (size_t)hkv * d.staging_cap * D;
  h.w_k = d.w_k + (size_t)hkv * WIN * D;
  h.w_v = d.w_v + (size_t)hkv * WIN * D;
  h.q = p.q + ((size_t)seq * p.Hkv * p.G + (size_t)hkv * p.G) * D;
  h.rec = p.part + ((size_t)d.rec0 + (size_t)hkv * p.G * d.n_splits) * (D + 2);
  h.out = nullptr;  // a variable-length batch always merges its records
  h.n_int4 = d.n_int4;
  h.n_anchor = d.n_anchor;
  h.n_staged = d.n_staged;
  h.n_win = d.n_win;
  h.n_splits = d.n_splits;
  h.split = (int)(m & 0xffffu);
  return h;
}

// NWAVES waves per workgroup: 4 when the launch is bandwidth bound (two workgroups per CU), 8
// when it is latency bound (one workgroup per CU: twice the tile loads in flight per CU and
// half the dependent chain per wave).  HB column blocks of 4 Q heads per wave: 1 up to GQA 4,
// 2 for GQA 8 and 16, so that one load of a tile serves 8 Q heads.
template <int BK, int BV, class Params, int NWAVES, bool NT, int HB>
__global__ __launch_bounds__(64 * NWAVES) void decode_split_kernel(Params p) {
  constexpr int WAVES = NWAVES;
  constexpr int HW = 4 * HB;  // Q heads of the workgroup's head block
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, q4 = lane >> 4;
  const int hh = n >> 2, g = n & 3;
  Unit u;
  if (!unit_of(p, u)) return;  // padding of the grid (the whole workgroup)
  const int sub = u.sub;
  const HeadWork hw = head_work<BK, BV>(p, u);

  // ---- q of the head block's Q heads, staged once through LDS
  __shared__ uint32_t q_lds[HW][D / 2];
  for (int idx = threadIdx.x; idx < HW * (D / 2); idx += 64 * WAVES) {
    const int h2 = idx >> 6, cp = idx & 63;  // 2 channels per thread and pass
    const int hd = sub * HW + h2;
    uint32_t v = 0;
    if (hd < p.G) v = *(const uint32_t*)(hw.q + (size_t)hd * D + 2 * cp);
    q_lds[h2][cp] = v;
  }
  __syncthreads();
  // B operand of the quantized path, per column block hb: q[head] restricted to this lane's
  // column group, channels in the order the code extraction produces them, times the inverse
  // of the code operand's per-element factor (INT4: 1/16 on k-slots 2,3,6,7; 2-bit:
  // 4^-(e >> 1)); zero outside the group
  f16x8 bq4[HB][4];
  float qsum24[HB], c_int4[HB];
  bool use[HB];
  const float alpha_log2 = LOG2E * 0.08838834764831845f;  // log2(e) / sqrt(128)
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int hl = 4 * hb + hh;  // this lane's head in the block
    const bool head_ok = sub * HW + hl < p.G;
    use[hb] = head_ok && (g == q4);
    float qs;  // 2^sigma: the head's largest |q| times qs lies in [2^13, 2^14)
    {
      float f[32];  // channels 32 q4 .. 32 q4 + 31
      float amax = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4 w = *(const u32x4*)&q_lds[hl][16 * q4 + 4 * t];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[8 * t + 2 * e] = bf16_bits_to_f32((uint16_t)(w[e] & 0xffff));
          f[8 * t + 2 * e + 1] = bf16_bits_to_f32((uint16_t)(w[e] >> 16));
        }
      }
#pragma unroll
      for (int c = 0; c < 32; ++c) amax = fmaxf(amax, fabsf(f[c]));
      amax = col4_max(amax);  // lanes l, l^16, l^32, l^48: the four channel blocks of the head
      int ex = 0;
      if (amax > 0.f) (void)frexpf(amax, &ex);
      qs = ldexpf(1.0f, min(100, max(-100, Q_TARGET - ex)));
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = f[kstep_channel<BK>(t, e)] * qs * code_factor<BK>(e);
          bq4[hb][t][e] = use[hb] ? (_Float16)v : (_Float16)0.f;
        }
    }
    float qsum = 0.f;
    if (head_ok) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4 w = *(const u32x4*)&q_lds[hl][16 * g + 4 * t];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          qsum += (float)(_Float16)(bf16_bits_to_f32((uint16_t)(w[e] & 0xffff)) * qs) +
                  (float)(_Float16)(bf16_bits_to_f32((uint16_t)(w[e] >> 16)) * qs);
      }
    }
    qsum24[hb] = qsum * (1.0f / 16777216.0f);
    c_int4[hb] = alpha_log2 * 16777216.0f / qs;
  }

  WaveState st[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    st[hb].m = -INFINITY;
    st[hb].l = 0.f;
    st[hb].mt = 0.f;
    st[hb].ps = PS_INIT;
    st[hb].ps_hi = PS_HI / PS_INIT;
    st[hb].ps_lo = PS_LO / PS_INIT;
#pragma unroll
    for (int r = 0; r < 8; ++r) st[hb].acc[r] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  // ---- work of this worker: INT4 tiles w, w + NW, w + 2 NW, ... (the workers of a head sweep
  // the head's records side by side); bf16 tiles go to the workers with the fewest INT4 tiles
  const int NW = hw.n_splits * WAVES, w = hw.split * WAVES + wave;
  const int T4 = (hw.n_int4 + 31) >> 5;
  const int TA = (hw.n_anchor + 31) >> 5, TS = (hw.n_staged + 31) >> 5, TWn = (hw.n_win + 31) >> 5;
  const int TB = TA + TS + TWn;
  const int wr = NW - 1 - w;  // bf16 tiles u with u % NW == wr
  const uint8_t* slab = hw.int4;
  const uint32_t smoff = (uint32_t)(g * 64 + q4 * 16);
  const int full = hw.n_int4 >> 5;  // tiles below this index hold 32 valid slots
  auto tile = [&](const QTile<BK, BV>& x, int t) {
    if (t < full) int4_tile<BK, BV, false, HB>(st, x, bq4, qsum24, c_int4, t * 32, hw.n_int4, q4);
    else int4_tile<BK, BV, true, HB>(st, x, bq4, qsum24, c_int4, t * 32, hw.n_int4, q4);
  };
  // two tiles in flight: the next tile's loads are issued before the current one is computed.
  // The prefetch past the wave's last tile keeps the same loads (so the loop's waits stay
  // exact) but every lane reads the current record's first bytes: one 16-byte chunk per load
  // instead of the 5 KB record (never used).
  auto prefetch = [&](QTile<BK, BV>& x, int t) {
    const bool past = t + NW >= T4;
    load_int4_tile<NT>(x, slab, past ? t : t + NW, past ? 0u : (uint32_t)lane, past ? 0u : smoff);
  };
  if (w < T4) {
    QTile<BK, BV> ta, tb;
    int t = w;
    load_int4_tile<NT>(ta, slab, t, (uint32_t)lane, smoff);
    for (;;) {
      prefetch(tb, t);
      tile(ta, t);
      t += NW;
      if (t >= T4) break;
      prefetch(ta, t);
      tile(tb, t);
      t += NW;
      if (t >= T4) break;
    }
  }

  // ---- bf16 tiles (anchors, staging, window)
  for (int u = wr; u < TB; u += NW) {
    const uint16_t *kb, *vb;
    int cnt, tl;
    if (u < TA) { kb = hw.a_k; vb = hw.a_v; cnt = hw.n_anchor; tl = u; }
    else if (u < TA + TS) { kb = hw.s_k; vb = hw.s_v; cnt = hw.n_staged; tl = u - TA; }
    else { kb = hw.w_k; vb = hw.w_v; cnt = hw.n_win; tl = u - TA - TS; }
    const int base = tl * 32;
    const uint16_t* kt = kb + (size_t)tl * 4096 + lane * 8;
    const uint16_t* vt = vb + (size_t)tl * 4096 + lane * 8;
    bf16x8 ka[8], va[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) ka[j] = __builtin_bit_cast(bf16x8, ld_stream<NT>((const u32x4*)(kt + j * 512)));
#pragma unroll
    for (int j = 0; j < 8; ++j) va[j] = __builtin_bit_cast(bf16x8, ld_stream<NT>((const u32x4*)(vt + j * 512)));
    bool valid[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      valid[r] = base + 4 * q4 + r < cnt;
      valid[4 + r] = base + 16 + 4 * q4 + r < cnt;
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        // B operand: q[head] channels 32q4+8tt .. +7 in natural order, zero outside the group
        u32x4 qw = *(const u32x4*)&q_lds[4 * hb + hh][16 * q4 + 4 * tt];
        if (!use[hb]) qw = (u32x4){0u, 0u, 0u, 0u};
        const bf16x8 bqb = __builtin_bit_cast(bf16x8, qw);
        S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tt], bqb, S0, 0, 0, 0);
        S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[4 + tt], bqb, S1, 0, 0, 0);
      }
      float sc[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v0 = S0[r], v1 = S1[r];
        v0 += dpp_quad_xor1(v0);
        v1 += dpp_quad_xor1(v1);
        v0 += dpp_quad_xor2(v0);
        v1 += dpp_quad_xor2(v1);
        sc[r] = valid[r] ? v0 * alpha_log2 : -INFINITY;
        sc[4 + r] = valid[4 + r] ? v1 * alpha_log2 : -INFINITY;
      }
      float pv[8];
      tile_softmax(st[hb], sc, pv);
      bf16x8 bhi, blo;
      const float bfs = st[hb].ps * (1.0f / 16777216.0f);  // bf16 tiles feed p 2^e 2^-24
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pp = valid[j] ? pv[j] * bfs : 0.f;
        const __bf16 h = (__bf16)pp;
        bhi[j] = h;
        blo[j] = (__bf16)(pp - (float)h);
      }
#pragma unroll
      for (int rr = 0; rr < 8; ++rr)
        st[hb].acc[rr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[rr], bhi, st[hb].acc[rr], 0, 0, 0);
#pragma unroll
      for (int rr = 0; rr < 8; ++rr)
        st[hb].acc[rr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[rr], blo, st[hb].acc[rr], 0, 0, 0);
    }
  }

  // ---- per-wave totals, then merge the waves through LDS
  __shared__ float red_m[WAVES][HW], red_l[WAVES][HW];
  __shared__ float red_o[WAVES][HW][D];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    st[hb].l += shfl_xor_f(st[hb].l, 16);
    st[hb].l += shfl_xor_f(st[hb].l, 32);
    st[hb].mt += shfl_xor_f(st[hb].mt, 16);
    st[hb].mt += shfl_xor_f(st[hb].mt, 32);
    const int hl = 4 * hb + hh;
    if (n == 4 * hh && q4 == 0) {  // one lane per head (g == 0, quad 0)
      red_m[wave][hl] = st[hb].m;
      red_l[wave][hl] = st[hb].l;
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      if ((rr >> 1) == g) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red_o[wave][hl][16 * rr + 4 * q4 + r] = st[hb].acc[rr][r] * (16777216.0f / st[hb].ps) + st[hb].mt;
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < HW * D; idx += 64 * WAVES) {
    const int h2 = idx / D, c = idx % D;
    const int hd = sub * HW + h2;
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
    if (hw.out) {
      // the merge of one record, as the merge computes it (weight exp2(0) = 1)
      hw.out[(size_t)hd * D + c] = __builtin_fmaf(O, 1.0f, 0.0f) / L;
      continue;
    }
    float* rec = hw.rec + ((size_t)hd * hw.n_splits + hw.split) * (D + 2);
    if (c == 0) { rec[0] = M; rec[1] = L; }
    rec[2 + c] = O;
  }
}

// ReduceSoftmax over the split records (HyQuant paper Alg. 3): one workgroup per (b, Q head).
// A separate launch: the kernel boundary makes the records of all XCDs visible without the
// L2 write-back an in-kernel agent-scope release would cost every workgroup.
// Merge of n_splits <= NS records with every load issued before the first is used: lane
// j < n_splits reads split j's (m, l), and every lane its two adjacent channels 2 lane,
// 2 lane + 1 of all records with one 8-byte load each (indices clamped, the surplus weighted
// 0), so the merge costs one memory latency.  Same arithmetic and order per channel as the
// multi-pass merge below.
template <int NS>
__device__ inline void merge_one_latency(const float* rec, int n_splits, float* o, int lane) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const int last = n_splits - 1;
  const f32x2 ml = *(const f32x2*)(rec + (size_t)min(lane, last) * (D + 2));
  const float m = ml[0], l = ml[1];
  f32x2 a[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) a[j] = *(const f32x2*)(rec + (size_t)min(j, last) * (D + 2) + 2 + 2 * lane);
  float M = lane < n_splits ? m : -INFINITY;
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, shfl_xor_f(M, k));
  float w = 0.f, lw = 0.f;
  if (M != -INFINITY && lane < n_splits) {
    w = __builtin_amdgcn_exp2f(m - M);
    lw = l * w;
  }
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) lw += shfl_xor_f(lw, k);
  float O0 = 0.f, O1 = 0.f;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));  // 0 past the last split
    O0 = fmaf(a[j][0], wj, O0);
    O1 = fmaf(a[j][1], wj, O1);
  }
  *(f32x2*)(o + 2 * lane) = (f32x2){O0 / lw, O1 / lw};
}

template <bool RAGGED>
__global__ __launch_bounds__(64) void decode_reduce_kernel(const float* __restrict__ part, float* __restrict__ o,
                                                           int n_splits, const RaggedSeq* __restrict__ seqs, int Hq) {
  // one wave per (b, Q head); lane j holds split j's (m, l) (64 splits per pass), every load of
  // a pass is independent so the whole merge costs about one memory latency per pass
  const int bh = blockIdx.x, lane = threadIdx.x;
  const float* rec;
  if constexpr (RAGGED) {  // a variable-length batch: the sequence's own split count and records
    const RaggedSeq& d = seqs[bh / Hq];
    n_splits = d.n_splits;
    rec = part + ((size_t)d.rec0 + (size_t)(bh % Hq) * n_splits) * (D + 2);
  } else {
    rec = part + (size_t)bh * n_splits * (D + 2);
  }
  if (n_splits <= 4) return merge_one_latency<4>(rec, n_splits, o + (size_t)bh * D, lane);
  if (n_splits <= 8) return merge_one_latency<8>(rec, n_splits, o + (size_t)bh * D, lane);
  if (n_splits <= 16) return merge_one_latency<16>(rec, n_splits, o + (size_t)bh * D, lane);
  if (n_splits <= 32) return merge_one_latency<32>(rec, n_splits, o + (size_t)bh * D, lane);
  if (n_splits <= 64) return merge_one_latency<64>(rec, n_splits, o + (size_t)bh * D, lane);
  float M = -INFINITY;
  for (int s0 = 0; s0 < n_splits; s0 += 64) {
    const int s = s0 + lane;
    float m = s < n_splits ? rec[(size_t)s * (D + 2)] : -INFINITY;
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, shfl_xor_f(m, k));
    M = fmaxf(M, m);
  }
  float L = 0.f, O0 = 0.f, O1 = 0.f;
  if (M != -INFINITY) {
    for (int s0 = 0; s0 < n_splits; s0 += 64) {
      const int s = s0 + lane;
      float w = 0.f, lw = 0.f;
      if (s < n_splits) {
        w = __builtin_amdgcn_exp2f(rec[(size_t)s * (D + 2)] - M);
        lw = rec[(size_t)s * (D + 2) + 1] * w;
      }
#pragma unroll
      for (int k = 32; k >= 1; k >>= 1) lw += shfl_xor_f(lw, k);
      L += lw;
      const int ns = min(64, n_splits - s0);
      for (int j0 = 0; j0 < ns; j0 += 8) {  // 16 independent loads in flight per batch
        float a[8], c[8], wj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = min(j0 + u, ns - 1);
          const float* r = rec + (size_t)(s0 + j) * (D + 2) + 2;
          a[u] = r[lane];
          c[u] = r[lane + 64];
          wj[u] = j0 + u < ns ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j)) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          O0 = fmaf(a[u], wj[u], O0);
          O1 = fmaf(c[u], wj[u], O1);
        }
      }
    }
  }
  o[(size_t)bh * D + lane] = O0 / L;
  o[(size_t)bh * D + lane + 64] = O1 / L;
}

}  // namespace

// Split records of the decode entry point that allocates nothing (for callers that cannot
// allocate: code under graph capture, serving loops that forbid allocation): one array per
// device, held until the process ends.  Host code never uses this name as an address: the
// device address is looked up once per device with hipGetSymbolAddress and kept below.
static __device__ __align__(256) float scratch[HYQ_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::once_flag g_scratch_once[SCRATCH_MAX_DEVICES];
float* g_scratch_ptr[SCRATCH_MAX_DEVICES];
hipError_t g_scratch_err[SCRATCH_MAX_DEVICES];
}  // namespace

hipError_t noalloc_scratch(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {  // runs with `dev` current
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? (float*)p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  if (!g_scratch_ptr[dev]) return hipErrorInvalidSymbol;
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(decode_grid_size(p.n_splits, p.Hkv, p.B, p.G));
  hipError_t e = with_widths(p.bits, p.bits_v, [&](auto BK, auto BV) {
    constexpr int bk = decltype(BK)::value, bv = decltype(BV)::value;
    // nontemporal loads unless the head blocks of a KV head share its slab through L2 (GQA 16)
    const bool nt = decode_head_blocks(p.G) == 1;
    const bool two = decode_heads_per_wave(p.G) == 8;  // two column blocks per wave
    if (p.waves == 8) {
      if (two) {
        if (nt) hipLaunchKernelGGL((decode_split_kernel<bk, bv, DecodeParams, 8, true, 2>), grid, dim3(512), 0, stream, p);
        else hipLaunchKernelGGL((decode_split_kernel<bk, bv, DecodeParams, 8, false, 2>), grid, dim3(512), 0, stream, p);
      } else {
        hipLaunchKernelGGL((decode_split_kernel<bk, bv, DecodeParams, 8, true, 1>), grid, dim3(512), 0, stream, p);
      }
    } else {
      if (two) {
        if (nt) hipLaunchKernelGGL((decode_split_kernel<bk, bv, DecodeParams, 4, true, 2>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((decode_split_kernel<bk, bv, DecodeParams, 4, false, 2>), grid, dim3(256), 0, stream, p);
      } else {
        hipLaunchKernelGGL((decode_split_kernel<bk, bv, DecodeParams, 4, true, 1>), grid, dim3(256), 0, stream, p);
      }
    }
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  if (p.n_splits == 1) return hipSuccess;  // the split kernel wrote the outputs
  hipLaunchKernelGGL(decode_reduce_kernel<false>, dim3(p.B * p.Hkv * p.G), dim3(64), 0, stream, p.part, p.o,
                     p.n_splits, (const RaggedSeq*)nullptr, p.Hkv * p.G);
  return hipGetLastError();
}

hipError_t launch_decode_ragged(const RaggedDecodeParams& p, hipStream_t stream) {
  const int nsub = decode_head_blocks(p.G);
  dim3 grid(p.total_splits, p.Hkv * nsub, 1);
  hipError_t e = with_widths(p.bits, p.bits_v, [&](auto BK, auto BV) {
    constexpr int bk = decltype(BK)::value, bv = decltype(BV)::value;
    if (decode_heads_per_wave(p.G) == 8) {  // two column blocks per wave, as in the uniform batch
      if (nsub == 1)
        hipLaunchKernelGGL((decode_split_kernel<bk, bv, RaggedDecodeParams, 4, true, 2>), grid, dim3(256), 0, stream, p);
      else
        hipLaunchKernelGGL((decode_split_kernel<bk, bv, RaggedDecodeParams, 4, false, 2>), grid, dim3(256), 0, stream, p);
    } else if (nsub == 1) {
      hipLaunchKernelGGL((decode_split_kernel<bk, bv, RaggedDecodeParams, 4, true, 1>), grid, dim3(256), 0, stream, p);
    } else {
      hipLaunchKernelGGL((decode_split_kernel<bk, bv, RaggedDecodeParams, 4, false, 1>), grid, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_reduce_kernel<true>, dim3(p.n_seq * p.Hkv * p.G), dim3(64), 0, stream, p.part, p.o, 0,
                     p.seqs, p.Hkv * p.G);
  return hipGetLastError();
}

}  // namespace hyq

// Shared definitions of the HIP kernels: vector types, cache-layout index helpers and the
// INT4 group quantizer.  gfx950 only.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "../../include/hyq.h"

namespace hyq {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int D = HYQ_HEAD_DIM;
constexpr int TILE = HYQ_TILE;
constexpr int WIN = HYQ_WINDOW;

// ---------------------------------------------------------------- bf16 / fp16 bit helpers
__device__ __host__ inline float bf16_bits_to_f32(uint16_t b) {
  union { uint32_t u; float f; } c;
  c.u = (uint32_t)b << 16;
  return c.f;
}
// fp32 -> bf16, round to nearest even (NaN -> quiet NaN)
__device__ inline uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------- layout helpers
// All per-head stores use 32-position tiles laid out so that each 16-byte piece one lane feeds
// to an MFMA sits at offset 16 * lane of a contiguous 1 KB block (lane = 16 * quad + row), i.e.
// every load instruction of the decode kernel is one fully coalesced 1 KB read.
//
// Position p (0..31) inside a tile -> (quad q, k-slot e):  p = 4q + (e & 3) + 16 (e >> 2)
__device__ __host__ inline int tile_quad(int p) { return (p & 15) >> 2; }
__device__ __host__ inline int tile_kslot(int p) { return (p & 3) + ((p >> 4) << 2); }
// nibble index of k-slot e inside a code dword (pairs (n0,n4),(n1,n5),(n2,n6),(n3,n7) are
// extracted with one mask (and one shared shift) each and feed k-slots (0,1),(2,3),(4,5),(6,7))
__device__ __host__ inline int kslot_nibble(int e) { return ((e & 1) << 2) | (e >> 1); }

// INT4 store: one contiguous 5120-byte record per 32-slot tile (each wave streams one record
// per step): [0, 2048) K codes, [2048, 4096) V codes, [4096, 4608) K (scale, min),
// [4608, 5120) V (scale, min).  Offsets below are bytes inside a head slab.
constexpr int T4_BYTES = 5120, T4_VC = 2048, T4_KSM = 4096, T4_VSM = 4608;
// K codes: 16-byte chunk holding channels 32*q4 .. 32*q4+31 of a slot (even channel in the low
// nibble); code region = [16-slot block][q4][slot in block][16 B].
__device__ __host__ inline size_t kcode_chunk(int slot, int q4) {
  return (size_t)(slot >> 5) * T4_BYTES + (size_t)(((slot >> 4) & 1) * 1024 + q4 * 256 + (slot & 15) * 16);
}
// V codes: dword (inside the V code region of a tile) for (slot, channel): region =
// [half][quad][channel & 15][4]; dword (half, q, i, r4) holds channel 16*(4*half + r4) + i for
// the 8 slots of quad q; the slot with k-slot e sits in nibble kslot_nibble(e).
__device__ __host__ inline int vcode_dword_in_tile(int p, int c) {
  const int i = c & 15, r = c >> 4, q = tile_quad(p);
  return (r >> 2) * 256 + (q * 16 + i) * 4 + (r & 3);
}
__device__ __host__ inline size_t vcode_byte(int slot, int c) {
  return (size_t)(slot >> 5) * T4_BYTES + T4_VC + 4 * (size_t)vcode_dword_in_tile(slot & 31, c);
}
__device__ __host__ inline int vcode_shift(int slot) { return 4 * kslot_nibble(tile_kslot(slot & 31)); }
// (scale, min) half2 for (slot, group): region = [16-slot block][g][slot in block]
__device__ __host__ inline size_t ksm_byte(int slot, int g) {
  return (size_t)(slot >> 5) * T4_BYTES + T4_KSM + 4 * (size_t)(((slot >> 4) & 1) * 64 + g * 16 + (slot & 15));
}
__device__ __host__ inline size_t vsm_byte(int slot, int g) {
  return (size_t)(slot >> 5) * T4_BYTES + T4_VSM + 4 * (size_t)(((slot >> 4) & 1) * 64 + g * 16 + (slot & 15));
}

// Quantized store with BK-bit K codes and BV-bit V codes (4/4: the INT4 record above; 8/8 and
// 2-bit widths: the same structure).  Per 32-slot tile: K codes, V codes, K (scale, min),
// V (scale, min).
template <int BK, int BV = BK>
struct QL {
  static constexpr int CB = 4 * BK;           // bytes of one (slot, 32-channel group) K chunk
  static constexpr int VC = 512 * BK;         // offset of the V codes (after the K codes)
  static constexpr int VCODES = 512 * BV;     // bytes of the V codes of a tile
  static constexpr int KSM = VC + VCODES;     // offset of the K (scale, min)
  static constexpr int VSM = KSM + 512;       // offset of the V (scale, min)
  static constexpr int TB = KSM + 1024;       // bytes per tile: 5120 (4/4), 9216 (8/8), 4096 (4/2), 3072 (2/2)
  static constexpr int SLOT = TB / 32;        // bytes per slot: 160, 288, 128, 96
};
// K codes of (slot, group q4): CB bytes, channel 32 q4 + j at bits BK j .. of the chunk read as
// little-endian dwords (INT4: nibble j, 8 per dword; INT8: byte j; 2-bit: 16 per dword);
// region = [16-slot block][q4][slot in block][CB]
template <int BK, int BV = BK>
__device__ __host__ inline size_t kcode_chunk_b(int slot, int q4) {
  typedef QL<BK, BV> L;
  return (size_t)(slot >> 5) * L::TB + (size_t)(((slot >> 4) & 1) * 64 * L::CB + q4 * 16 * L::CB + (slot & 15) * L::CB);
}
template <int BK, int BV = BK>
__device__ __host__ inline size_t ksm_byte_b(int slot, int g) {
  return (size_t)(slot >> 5) * QL<BK, BV>::TB + QL<BK, BV>::KSM + 4 * (size_t)(((slot >> 4) & 1) * 64 + g * 16 + (slot & 15));
}
template <int BK, int BV = BK>
__device__ __host__ inline size_t vsm_byte_b(int slot, int g) {
  return (size_t)(slot >> 5) * QL<BK, BV>::TB + QL<BK, BV>::VSM + 4 * (size_t)(((slot >> 4) & 1) * 64 + g * 16 + (slot & 15));
}
// 2-bit codes: a dword holds 16 codes, code j at bits 2j.  With h = 0 or 1 (the dword shifted
// right by 8 h), the masks 0x00030003, 0x000C000C, 0x00300030, 0x00C000C0 give the f16 operand
// elements e = 0 .. 7, element e being code code2_of(h, e) multiplied by 4^(e >> 1) (the other
// operand carries 4^-(e >> 1)).
__device__ __host__ inline int code2_of(int h, int e) { return 4 * h + (e >> 1) + 8 * (e & 1); }
__device__ inline f16x8 codes2_to_f16(uint32_t x, int h) {
  const uint32_t y = h ? x >> 8 : x;
  u32x4 a;
  a[0] = y & 0x00030003u;
  a[1] = y & 0x000C000Cu;
  a[2] = y & 0x00300030u;
  a[3] = y & 0x00C000C0u;
  return __builtin_bit_cast(f16x8, a);
}
// INT8 V codes: entry (half, quad, channel & 15, r4) of 8 bytes holds channel 16 (4 half + r4)
// + i for the 8 slots of the quad; the slot with k-slot e sits in byte kslot_byte(e) (bytes
// (0,2), (1,3), (4,6), (5,7) are extracted with one mask each and feed k-slots (0,1) .. (6,7))
__device__ __host__ inline int kslot_byte(int e) { return (e & 4) | ((e & 1) << 1) | ((e >> 1) & 1); }
// 2-bit V codes: dword (quad, channel & 15, d4) holds channels 16 (2 d4 + h) + (c & 15), h = 0, 1,
// at the 8 slots of the quad: the slot with k-slot e at bits 2 (e >> 1) + 16 (e & 1) + 8 h, so
// codes2_to_f16(dword, h) gives channel block 2 d4 + h in k-slot order
// V code of (slot, channel): byte offset of the dword holding it and the code's bit shift
template <int BK, int BV = BK>
__device__ __host__ inline void vcode_loc(int slot, int c, size_t& dword_off, int& shift) {
  const size_t tile = (size_t)(slot >> 5) * QL<BK, BV>::TB + QL<BK, BV>::VC;
  const int p = slot & 31;
  if (BV == 4) {
    dword_off = tile + 4 * (size_t)vcode_dword_in_tile(p, c);
    shift = 4 * kslot_nibble(tile_kslot(p));
  } else if (BV == 2) {
    const int e = tile_kslot(p), rr = c >> 4;
    dword_off = tile + 4 * (size_t)((tile_quad(p) * 16 + (c & 15)) * 4 + (rr >> 1));
    shift = 2 * (e >> 1) + 16 * (e & 1) + 8 * (rr & 1);
  } else {
    const int byte = ((((c >> 6) * 4 + tile_quad(p)) * 16 + (c & 15)) * 4 + ((c >> 4) & 3)) * 8 + kslot_byte(tile_kslot(p));
    dword_off = tile + (size_t)(byte & ~3);
    shift = 8 * (byte & 3);
  }
}
// bytes per slot of the quantized store for (B_K, B_V)
__device__ __host__ inline int qslot_bytes(int bk, int bv) { return (512 * (bk + bv) + 1024) / 32; }

// bf16 K (anchors / staging / window): element index for (pos, channel).  Tile = 4096
// elements: [16-pos block][8-channel chunk tt][quad q4 = channel / 32][pos in block][8].
__device__ __host__ inline size_t kbf_index(int pos, int c) {
  const int t = pos >> 5, p = pos & 31;
  return (size_t)t * 4096 + (size_t)(((((p >> 4) * 4 + ((c & 31) >> 3)) * 4 + (c >> 5)) * 16 + (p & 15)) * 8 + (c & 7));
}
// bf16 V: element index for (pos, channel).  Tile = 4096 elements: [channel / 16][quad]
// [channel & 15][k-slot e]: one 16-byte piece = one channel at the 8 positions of a quad.
__device__ __host__ inline size_t vbf_index(int pos, int c) {
  const int t = pos >> 5, p = pos & 31;
  return (size_t)t * 4096 + (size_t)((((c >> 4) * 4 + tile_quad(p)) * 16 + (c & 15)) * 8 + tile_kslot(p));
}

// ---------------------------------------------------------------- rounded quotient
// rint(fl(a / s)) -- the IEEE-rounded quotient rounded half-even to an integer -- for s > 0
// normal, r = v_rcp_f32(s), where the caller clamps the result to a range within [-255, 255].
// q0 = fl(a r) is within 2^-22 |a / s| of fl(a / s) (the reciprocal is within 1 ulp, the
// product adds half an ulp, the IEEE quotient half an ulp): for |a / s| <= 256 that is below
// 2^-14, so a q0 more than 2^-13 from a half-integer rounds to the integer fl(a / s) rounds
// to.  The rest -- about 2 in 10^4 uniformly placed quotients -- take the IEEE division.  A
// quotient beyond 256 in magnitude clamps to the range's end either way.
__device__ inline float rint_div(float a, float s, float r) {
  const float q0 = __fmul_rn(a, r);
  const float k = rintf(q0);
  if (fabsf(__fsub_rn(q0, k)) > 0.5f - 0x1p-13f) return rintf(__fdiv_rn(a, s));
  return k;
}

// ---------------------------------------------------------------- group quantizer
// One token, 32 contiguous channels, LEVELS = 2^bits - 1 (15 for INT4).  Fixed IEEE fp32
// operation order (the translation units using it are built with -ffp-contract=off):
//   mn = min x, mx = max x; s = fp16((mx - mn) / LEVELS); m = fp16(mn);
//   code = s == 0 ? 0 : clamp(rint((x - m) / s), 0, LEVELS)
// The quotients come from the reciprocal as in rint_div, with the threshold set by the width:
// a quotient that can change a clamped code is at most LEVELS + 1 in magnitude (beyond that
// both roundings clamp to the same end), where q0 is within 2^-22 (LEVELS + 1) of the IEEE
// quotient: 2^-18 for up to 4 bits, 2^-14 for 8 bits.  A q0 further than 2^-16 (2^-13) from a
// half-integer rounds as the IEEE quotient does.  The codes are formed first; a quotient
// inside that band is settled with the IEEE division afterwards.  With bf16 inputs and an fp16
// scale and minimum, exact half-integer quotients are common (about 7 in 10^4 of N(0,1)
// values: most waves of 64 groups hold one), but in a wave they fall on one or two of the 32
// channel positions, so the fast pass records, per position, whether any lane of the wave has
// one (a wave vote), and the exact pass visits only those positions.  With s = 0 the
// reciprocal is taken as 0: every quotient is 0 and every code 0.
// x(j) gives channel j's value.  The codes come out packed: P bits each, code j at bit P j of
// the P dwords of out (P = 2, 4 or 8).
// fresh() runs before the rare exact pass: a caller whose x(j) decodes packed registers can
// mark them rewritten there, so that the compiler decodes them again in that pass instead of
// keeping all 32 differences (x - m) live across the fast pass.
template <int LEVELS, int P, class X, class F>
__device__ inline void quant_group32(X x, F fresh, uint32_t (&out)[P], __half& s16, __half& m16) {
  constexpr float THR = LEVELS <= 15 ? 0.5f - 0x1p-16f : 0.5f - 0x1p-13f;
  constexpr int PER = 32 / P;  // codes per dword
  float mn = x(0), mx = x(0);
#pragma unroll
  for (int j = 1; j < 32; ++j) { mn = fminf(mn, x(j)); mx = fmaxf(mx, x(j)); }
  float s32 = __fdiv_rn(__fsub_rn(mx, mn), (float)LEVELS);
  s16 = __float2half_rn(s32);
  m16 = __float2half_rn(mn);
  const float sf = __half2float(s16), mf = __half2float(m16);
  const float rf = sf != 0.0f ? __builtin_amdgcn_rcpf(sf) : 0.0f;
  uint32_t near = 0;  // bit j: some lane of the wave has its channel-j quotient near a tie
#pragma unroll
  for (int d = 0; d < P; ++d) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const float q0 = __fmul_rn(__fsub_rn(x(PER * d + i), mf), rf);
      const float c = rintf(q0);
      if (__ballot(fabsf(__fsub_rn(q0, c)) > THR)) near |= 1u << (PER * d + i);
      const float cc = fminf(fmaxf(c, 0.0f), (float)LEVELS);
      if constexpr (P == 8) w = __builtin_amdgcn_cvt_pk_u8_f32(cc, i, w);  // byte i of w
      else w |= (uint32_t)cc << (P * i);
    }
    out[d] = w;
  }
  if (near) {
    fresh();
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (!(near & (1u << j))) continue;  // the same on every lane
      const float a = __fsub_rn(x(j), mf);
      const float q0 = __fmul_rn(a, rf);
      if (fabsf(__fsub_rn(q0, rintf(q0))) > THR) {
        const uint32_t c = (uint32_t)fminf(fmaxf(rintf(__fdiv_rn(a, sf)), 0.0f), (float)LEVELS);
        const int sh = P * (j % PER);
        out[j / PER] = (out[j / PER] & ~(((1u << P) - 1u) << sh)) | (c << sh);
      }
    }
  }
}

// ---------------------------------------------------------------- cross-lane helpers
__device__ inline float dpp_quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ inline float dpp_quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
// max / sum over the 4 lanes l, l^16, l^32, l^48 (one MFMA column): v_permlane32_swap(v, v)
// pairs lane l with l^32 and v_permlane16_swap(v, v) pairs l with l^16 (VALU, no LDS trip)
__device__ inline float col4_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float col4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ inline float shfl_xor_f(float v, int m) {
  int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __float_as_int(v)));
}

}  // namespace hyq

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
// Position p (0..31) inside a tile -> (quad q, k-slot e):  p = 4q + (e & 3) + 16 (e >> 2)
__device__ __host__ inline int tile_quad(int p) { return (p & 15) >> 2; }
__device__ __host__ inline int tile_kslot(int p) { return (p & 3) + ((p >> 4) << 2); }
// nibble index of k-slot e inside a V-code dword (pairs (n0,n4),(n1,n5),(n2,n6),(n3,n7) are
// extracted with one shift+mask each and feed k-slots (0,1),(2,3),(4,5),(6,7))
__device__ __host__ inline int kslot_nibble(int e) { return ((e & 1) << 2) | (e >> 1); }

// INT4 V codes: dword index inside a head slab for (slot, channel)
__device__ __host__ inline size_t vcode_dword(int slot, int c) {
  int t = slot >> 5, p = slot & 31;
  int i = c & 15, r = c >> 4, q = tile_quad(p);
  return (size_t)t * 512 + (size_t)((i * 4 + q) * 8 + r);
}
__device__ __host__ inline int vcode_shift(int slot) { return 4 * kslot_nibble(tile_kslot(slot & 31)); }

// bf16 V (anchors / staging / window): element index inside a head slab for (pos, channel)
__device__ __host__ inline size_t vbf_index(int pos, int c) {
  int t = pos >> 5, p = pos & 31;
  int i = c & 15, r = c >> 4, q = tile_quad(p), e = tile_kslot(p);
  return (size_t)t * 4096 + (size_t)((((i * 4 + q) * 8 + r) * 8) + e);
}
// (scale, min) half2 index inside a head slab for (slot, group)
__device__ __host__ inline size_t sm_index(int slot, int g) {
  return (size_t)(slot >> 4) * 64 + (size_t)g * 16 + (slot & 15);
}

// ---------------------------------------------------------------- INT4 group quantizer
// One token, 32 contiguous channels.  Fixed IEEE fp32 operation order (this translation
// unit is built with -ffp-contract=off):
//   mn = min x, mx = max x; s = fp16((mx - mn) / 15); m = fp16(mn);
//   code = s == 0 ? 0 : clamp(rint((x - m) / s), 0, 15)
__device__ inline void quant_group32(const float* x, uint8_t* code, __half& s16, __half& m16) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int j = 1; j < 32; ++j) { mn = fminf(mn, x[j]); mx = fmaxf(mx, x[j]); }
  float s32 = __fdiv_rn(__fsub_rn(mx, mn), 15.0f);
  s16 = __float2half_rn(s32);
  m16 = __float2half_rn(mn);
  float sf = __half2float(s16), mf = __half2float(m16);
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float c = 0.0f;
    if (sf != 0.0f) {
      c = rintf(__fdiv_rn(__fsub_rn(x[j], mf), sf));
      c = fminf(fmaxf(c, 0.0f), 15.0f);
    }
    code[j] = (uint8_t)c;
  }
}

// ---------------------------------------------------------------- cross-lane helpers
__device__ inline float dpp_quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ inline float dpp_quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ inline float shfl_xor_f(float v, int m) {
  int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __float_as_int(v)));
}

}  // namespace hyq

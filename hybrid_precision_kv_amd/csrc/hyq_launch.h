// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hyq {

struct DecodeParams {
  const uint8_t* k_codes;
  const uint32_t* v_codes;
  const uint32_t* k_sm;
  const uint32_t* v_sm;
  const uint16_t *a_k, *a_v, *s_k, *s_v, *w_k, *w_v;
  const uint16_t* q;  // [B][Hq][128]
  float* part;        // [B][Hq][n_splits][130] partial (m, l, acc) records
  int Hkv, G;         // KV heads, Q heads per KV head
  int int4_cap, anchor_cap, staging_cap;
  int n_int4, n_anchor, n_staged, n_win;
  int n_splits;
};
hipError_t launch_decode(const DecodeParams& p, float* o, int B, hipStream_t stream);

struct CacheView {
  uint8_t* k_codes;
  uint32_t* v_codes;
  uint32_t* k_sm;
  uint32_t* v_sm;
  int32_t* slot_pos;
  uint16_t *a_k, *a_v;
  int32_t* a_pos;
  uint16_t *s_k, *s_v, *w_k, *w_v;
  uint16_t* proxy_q;
  int B, Hkv, G;
  int int4_cap, anchor_cap, staging_cap, proxy_cap;
};

// Freeze (prefill -> decode)
hipError_t launch_freeze(const CacheView& c, const uint16_t* k, const uint16_t* v, int len,
                         const int32_t* anchors, int n_anchor, const uint16_t* q_tail, int n_tail,
                         hipStream_t stream);
// One decode token appended to every sequence
hipError_t launch_append(const CacheView& c, const uint16_t* k_t, const uint16_t* v_t, const uint16_t* q_t,
                         int len, int n_staged, int proxy_head, hipStream_t stream);

}  // namespace hyq

// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace hyq {

// Runs f(integral_constant<B_K>, integral_constant<B_V>) for the supported code widths
// (4/4, 8/8, 4/2, 2/2); any other pair is an invalid value.
template <class F>
hipError_t with_widths(int bk, int bv, F&& f) {
  using std::integral_constant;
  if (bk == 4 && bv == 4) return f(integral_constant<int, 4>{}, integral_constant<int, 4>{});
  if (bk == 8 && bv == 8) return f(integral_constant<int, 8>{}, integral_constant<int, 8>{});
  if (bk == 4 && bv == 2) return f(integral_constant<int, 4>{}, integral_constant<int, 2>{});
  if (bk == 2 && bv == 2) return f(integral_constant<int, 2>{}, integral_constant<int, 2>{});
  return hipErrorInvalidValue;
}

struct DecodeParams {
  const uint8_t* int4;  // [hb][int4_cap/32] 5120-byte tile records
  const uint16_t *a_k, *a_v, *s_k, *s_v, *w_k, *w_v;
  const uint16_t* q;  // [B][Hq][128]
  float* part;        // [B][Hq][n_splits][130] partial (m, l, acc) records
  float* o;           // [B][Hq][128]
  int B, Hkv, G;      // sequences, KV heads, Q heads per KV head
  int int4_cap, anchor_cap, staging_cap;
  int n_int4, n_anchor, n_staged, n_win;
  int n_splits;
  int bits, bits_v;  // B_K and B_V of the quantized store: (4, 4), (8, 8), (4, 2) or (2, 2)
  int waves;         // waves per split workgroup: 4, or 8 for latency-bound launches
};
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
// Q heads one decode wave serves in a uniform batch: its 16 MFMA columns are (head, channel
// group) pairs of 4 heads; GQA 8 and 16 take two such column blocks, so that one load of a
// tile serves 8 Q heads.  Head blocks per KV head: ceil(G / that).
__host__ __device__ inline int decode_heads_per_wave(int G) { return G >= 8 ? 8 : 4; }
__host__ __device__ inline int decode_head_blocks(int G) {
  const int h = decode_heads_per_wave(G);
  return (G + h - 1) / h;
}
// Device address of the current device's static decode scratch (HYQ_NOALLOC_SCRATCH_BYTES),
// looked up once per device.
hipError_t noalloc_scratch(float** ptr);

// One sequence of a variable-length batch: its own single-sequence cache (buffers at that
// cache's b = 0) with its own counters and split count.  Built on the host, copied into the
// decode workspace before the launch.
struct RaggedSeq {
  const uint8_t* int4;
  const uint16_t *a_k, *a_v, *s_k, *s_v, *w_k, *w_v;
  int int4_cap, anchor_cap, staging_cap;
  int n_int4, n_anchor, n_staged, n_win;
  int n_splits;  // splits of every KV head of this sequence
  int rec0;      // first partial record of this sequence: records [rec0 + h * n_splits + s]
  int pad[5];
};
static_assert(sizeof(RaggedSeq) == 112, "RaggedSeq layout");

struct RaggedDecodeParams {
  const RaggedSeq* seqs;      // [n_seq] (device)
  const uint32_t* split_map;  // [total_splits] (device): seq << 16 | split within the sequence
  const uint16_t* q;          // [n_seq][Hq][128]
  float* part;                // partial (m, l, acc) records, 130 floats each
  float* o;                   // [n_seq][Hq][128]
  int n_seq, Hkv, G, total_splits;
  int bits, bits_v;  // B_K, B_V
};
hipError_t launch_decode_ragged(const RaggedDecodeParams& p, hipStream_t stream);

struct CacheView {
  uint8_t* int4;
  int32_t* slot_pos;
  uint16_t *a_k, *a_v;
  int32_t* a_pos;
  uint16_t *s_k, *s_v, *w_k, *w_v;
  uint16_t* proxy_q;
  int B, Hkv, G;
  int int4_cap, anchor_cap, staging_cap, proxy_cap;
  int bits, bits_v;  // B_K and B_V of the quantized store: (4, 4), (8, 8), (4, 2) or (2, 2)
};

struct SelectParams {
  const uint16_t* dense_k;  // dense mode: [B][Hkv][len][128]; null in cache mode
  const uint8_t* int4;
  const int32_t* slot_pos;
  const uint16_t *a_k, *s_k, *w_k;
  const int32_t* a_pos;
  const uint16_t* proxy;  // [B][Hq][proxy_stride][128], rows 0..n_proxy-1 valid
  int proxy_stride, n_proxy;
  int B, Hkv, G, len;
  int int4_cap, anchor_cap, staging_cap;
  int n_int4, n_anchor, n_staged, n_win;
  int n_tiles, n_tasks, k;
  float* qsum;     // [H][R][4]
  void* pq16;      // [H][RBmax][256] f16x8: proxy rows, INT4-key operand order
  void* pqbf;      // [H][RBmax][256] bf16x8: proxy rows, bf16-key operand order
  int rb_stride;   // RBmax (16-row blocks per head slot)
  float* rowpart;  // [H][R][n_tasks][2]
  float* rowstat;  // [H][R][2]
  float* scores;   // [H][len - 128] by position
  int32_t* idx_out;  // [H][k]
  int bits, bits_v;  // B_K, B_V of the quantized store (the record layout depends on both)
};
hipError_t launch_select(SelectParams p, hipStream_t stream);
int select_task_count(int n_tiles);
// radix top-k of `rows` rows of P order-preserving keys (largest first, ties to the lower
// position), indices ascending into idx_out [rows][k]
hipError_t launch_topk_keys(const uint32_t* keys, int P, int k, int rows, int32_t* idx_out, hipStream_t stream);

struct TailSelectParams {
  const uint16_t* k;  // [B][Hkv][len][128] dense keys
  const uint16_t* q;  // [B][Hq][n_q][128] queries
  int B, Hkv, G, len, n_q, t, k_sel;
  float* qbar;        // [B][Hq][128] tail-query means
  uint32_t* keys;     // [B][Hq][len - 128] order-preserving keys of the logits
  float* scores_out;  // [B][Hq][len - 128] logits, nullable
  int32_t* idx_out;   // [B][Hq][k_sel]
};
hipError_t launch_select_tail(const TailSelectParams& p, hipStream_t stream);

struct RefreshParams {
  uint8_t* int4;
  int32_t* slot_pos;
  uint16_t *a_k, *a_v;
  int32_t* a_pos;
  const uint16_t *s_k, *s_v;
  const int32_t* idx;  // [H][k] new set, ascending
  int B, Hkv, len, k;
  int int4_cap, anchor_cap, staging_cap;
  int n_int4_old, n_anchor_old, n_staged;
  uint8_t* ws;  // per-head scratch
  size_t ws_per_head;
  int inset_words, del_words, max_moves;
  int* status;  // [H] 0 = counts consistent
  int bits, bits_v;  // B_K, B_V of the quantized store
};
hipError_t launch_refresh(const RefreshParams& p, hipStream_t stream);
// bytes of per-head refresh scratch
size_t refresh_scratch_bytes(int inset_words, int del_words, int anchor_cap, int max_moves);

// Freeze (prefill -> decode)
hipError_t launch_freeze(const CacheView& c, const uint16_t* k, const uint16_t* v, int len,
                         const int32_t* anchors, int n_anchor, const uint16_t* q_tail, int n_tail,
                         hipStream_t stream);
// One decode token appended to every sequence
hipError_t launch_append(const CacheView& c, const uint16_t* k_t, const uint16_t* v_t, const uint16_t* q_t,
                         int len, int n_staged, int proxy_head, hipStream_t stream);

// Hybrid prefill (one sequence).  Workspace sections are described with hyq_prefill_attn.
struct PrefillParams {
  const uint16_t* q;        // [Hq][N][128] bf16
  const uint16_t* k;        // [Hkv][N][128] bf16
  const uint16_t* v;        // [Hkv][N][128] bf16
  const int32_t* anchors;   // [Hkv][n_anchor]
  int n_anchor;
  float* o;                 // [Hq][N][128]
  int N, Npad, Hq, Hkv, G;
  int8_t* q8; float* sq;    // Q codes (operand order) and per-64-query scales
  int8_t* k8; float* sk;    // K codes (operand order) and per-64-key scales
  uint8_t* v8; float* sv;   // V E4M3 codes (operand order) and per-channel scales
  float* vmax;              // per-64-key-block channel maxima of |V| (non-anchor)
  uint32_t* abits;          // anchor bitmap
  uint16_t* vt16;           // V^T bf16 in the bf16 MFMA operand order, all keys
  uint16_t* ka16;           // anchor K rows (list order), bf16
  uint16_t* va16;           // anchor V^T (list order), bf16, operand order
  int n_anchor_pad;         // n_anchor rounded up to 64 (rows of ka16 / va16 written)
  int bulk;                 // bulk Q.K^T format: 0 INT8 codes, 1 MXFP4 (codes in the q8 / k8 sections)
};
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

}  // namespace hyq

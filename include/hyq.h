/*
 * hyq.h -- C ABI of the hybrid-precision KV attention library for AMD MI355X (gfx950).
 *
 * The method is HyQuant (arXiv page "HyQuant: Hybrid-Precision Quantization for LLM
 * Attention", called "the HyQuant paper" below): in decode, most cached positions are held
 * as asymmetric INT4 (K4V4, one fp16 scale and one fp16 minimum per 32-channel group of a
 * token), while a small set of "vertical-line" anchor positions and a sliding window of the
 * most recent 128 positions stay in bf16 (§4.1 Eq. 1-5, §4.3 Eq. 8).  Decode attention
 * dequantizes INT4 inside one online-softmax pass (§4.3 Eq. 9, Alg. 3).  The prefill
 * operator runs the bulk of Q.K^T in INT8 and P.V in FP8 with anchors and the window in
 * bf16, merged in one online softmax (§4.2 Eq. 6-7, Alg. 2).
 *
 * General rules for every entry point
 * -----------------------------------
 *  - Pointers marked "device" are HIP device pointers owned by the caller; the library
 *    never allocates, frees or synchronises.  Its only global state is per device: a cache
 *    of the compute-unit count (a device constant) and, for hyq_decode_attn_noalloc alone,
 *    the static scratch array and its looked-up address.
 *  - Work is enqueued asynchronously on the caller's stream; inputs must stay alive until
 *    the stream has passed the call.  Host structs are read/updated before returning.
 *  - All checks run on the host before anything is enqueued.  On any error nothing is
 *    enqueued and the hyq_cache_t is left unchanged.  Device faults surface at the
 *    caller's next synchronisation.  NaN/Inf inputs are not checked and propagate.
 *  - bf16 tensors are passed as raw 16-bit patterns.  Head dimension is fixed at 128,
 *    the channel group at 32 and the window at 128.
 *  - Q head h belongs to KV head h / (n_q_heads / n_kv_heads) (grouped-query layout).
 *
 * Cache memory layout (per (sequence b, KV head h); "head slab" index hb = b*Hkv + h;
 * every buffer is the concatenation of its head slabs, slab sizes given by
 * hyq_cache_buffer_bytes).  Tiles hold 32 positions.
 *
 *  Inside a tile, position/slot p = 4q + (e & 3) + 16*(e >> 2) with quad q = 0..3 and
 *  k-slot e = 0..7; "lane" below means 16*q + (row within a 16-position block).
 *
 *  int4     u8 [hb][int4_cap/32][5120]  one record per 32-slot INT4 tile (shape.bits 0 or 4):
 *     [0, 2048)    K codes  [16-slot block][q4][slot in block][16 B]: the 16 bytes hold
 *                  channels 32*q4 .. 32*q4+31 of the slot, channel 2j in the low nibble of
 *                  byte j, 2j+1 in its high nibble;
 *     [2048, 4096) V codes  u32 [half][q][i][r4]: channel 16*(4*half + r4) + i of the 8 slots
 *                  of quad q, k-slot e in nibble HYQ_V_NIBBLE[e] (4 bits each, low first);
 *     [4096, 4608) K (scale, min) fp16 pairs [16-slot block][group g][slot in block];
 *     [4608, 5120) V (scale, min), same order.  Dequantized x = scale * code + min.
 *  With shape.bits = 8 the same store holds 8-bit codes (255 levels of the same group
 *  quantizer), one 9216-byte record per 32-slot tile:
 *     [0, 4096)    K codes  [16-slot block][q4][slot in block][32 B]: byte j holds channel
 *                  32*q4 + j of the slot;
 *     [4096, 8192) V codes  [half][q][i][r4][8 B]: channel 16*(4*half + r4) + i of the 8
 *                  slots of quad q, k-slot e in byte HYQ_V_BYTE[e];
 *     [8192, 8704) K (scale, min), [8704, 9216) V (scale, min), as above.
 *  In general a tile record holds, in this order, 512*B_K bytes of K codes, 512*B_V bytes of
 *  V codes and the two 512-byte (scale, min) regions: 5120 (4/4), 9216 (8/8), 4096 (4/2) or
 *  3072 (2/2) bytes.  2-bit codes (3 levels):
 *     K codes  [16-slot block][q4][slot in block][8 B]: channel 32*q4 + j at bits 2*(j & 15)
 *              of little-endian dword j >> 4;
 *     V codes  u32 [q][i][d4]: channels 16*(2*d4 + h) + i (h = 0, 1) of the 8 slots of
 *              quad q, k-slot e at bits 2*(e >> 1) + 16*(e & 1) + 8*h.
 *  slot_pos i32 [hb][int4_cap]          position held by each INT4 slot (-1 for unused).
 *  a_k, s_k, w_k  bf16 [hb][cap/32][4096]  anchor / staging / window K, per tile
 *                  [16-position block][tt][q4][position in block][8]: channels
 *                  32*q4 + 8*tt .. +7 of the position.
 *  a_v, s_v, w_v  bf16 [hb][cap/32][4096]  V per tile [c / 16][q][c & 15][e]: channel c at
 *                  the 8 positions of quad q in k-slot order.
 *  a_pos    i32 [hb][anchor_cap]        anchor positions, ascending.
 *  proxy_q  bf16 [b][n_q_heads][proxy_cap][128]  ring of the last proxy queries.
 *  The window is a ring: position p sits in window slot p % 128.  Staging slot i holds
 *  position len - 128 - n_staged + i.
 */
#ifndef HYQ_H
#define HYQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYQ_HEAD_DIM 128
#define HYQ_GROUP 32
#define HYQ_WINDOW 128
#define HYQ_TILE 32
#define HYQ_PROXY_CAP 64
/* nibble index (0..7, 4 bits each, low first) of k-slot e inside a V-code dword */
#define HYQ_V_NIBBLE_INIT {0, 4, 1, 5, 2, 6, 3, 7}
/* byte index (0..7) of k-slot e inside an 8-byte INT8 V-code entry */
#define HYQ_V_BYTE_INIT {0, 2, 1, 3, 4, 6, 5, 7}

/* status codes */
#define HYQ_OK 0
#define HYQ_ERR_INVALID 1      /* null pointer, bad dimension, inconsistent counters */
#define HYQ_ERR_UNSUPPORTED 2  /* head_dim != 128, group != 32, window != 128, GQA not in {1,2,4,8,16},
                                  an unsupported (bits, bits_v) pair */
#define HYQ_ERR_CAPACITY 3     /* len > capacity, k > anchor_cap or > candidates, staging full */
#define HYQ_ERR_WORKSPACE 4    /* workspace missing or smaller than hyq_workspace_bytes */
#define HYQ_ERR_HIP 5          /* a kernel launch failed (hipGetLastError) */

/* operations for hyq_workspace_bytes */
#define HYQ_OP_DECODE 1
#define HYQ_OP_SELECT 2
#define HYQ_OP_PREFILL 3
#define HYQ_OP_SELECT_TAIL 4

typedef struct {
  int32_t batch;        /* sequences */
  int32_t n_q_heads;    /* Q heads */
  int32_t n_kv_heads;   /* KV heads; n_q_heads / n_kv_heads in {1, 2, 4, 8, 16} */
  int32_t head_dim;     /* must be 128 */
  int32_t group;        /* must be 32 (channels per INT4 scale/min group) */
  int32_t window;       /* must be 128 */
  int32_t proxy_cap;    /* must be 64 (proxy-query buffer, HyQuant paper §5.5) */
  int32_t staging_cap;  /* staging capacity per head, multiple of 32, >= the refresh interval */
  int32_t int4_cap;     /* INT4 slots per head, multiple of 32 */
  int32_t anchor_cap;   /* anchor slots per head, multiple of 32 */
  int32_t bits;         /* B_K, bits of the quantized bulk's K codes (the HyQuant paper's Alg. 3
                           and Alg. 4 take B_K and B_V as parameters): 0 or 4 = INT4, 8, or 2 */
  int32_t bits_v;       /* B_V, bits of its V codes: 0 = same as B_K, else 2, 4 or 8.  Supported
                           (B_K, B_V): (4, 4) the paper's K4V4, (8, 8), (4, 2), (2, 2); any other
                           pair is UNSUPPORTED */
} hyq_shape_t;

typedef struct {
  hyq_shape_t shape;
  /* caller-owned device buffers, layouts above */
  void *int4;
  int32_t *slot_pos;
  void *a_k, *a_v;
  int32_t *a_pos;
  void *s_k, *s_v;
  void *w_k, *w_v;
  void *proxy_q;
  /* host-side counters, identical for every sequence of the batch; updated in place by
     hyq_quantize_kv, hyq_append_token and hyq_select_vlines(apply=1) */
  int32_t len;        /* positions cached */
  int32_t n_int4;     /* INT4 slots in use */
  int32_t n_anchor;   /* anchors held in bf16 */
  int32_t n_staged;   /* staged positions (left the window since the last refresh) */
  int32_t n_proxy;    /* valid proxy queries per Q head (<= proxy_cap) */
  int32_t proxy_head; /* next proxy ring slot to write */
} hyq_cache_t;

/* Buffer indices for hyq_cache_buffer_bytes */
enum {
  HYQ_BUF_INT4 = 0, HYQ_BUF_SLOT_POS,
  HYQ_BUF_A_K, HYQ_BUF_A_V, HYQ_BUF_A_POS, HYQ_BUF_S_K, HYQ_BUF_S_V, HYQ_BUF_W_K,
  HYQ_BUF_W_V, HYQ_BUF_PROXY_Q, HYQ_NBUF
};

/* Human-readable status text (static storage). */
const char* hyq_status_string(int status);

/* Validates a shape; fills bytes[HYQ_NBUF] with the total size in bytes of each cache
   buffer (all head slabs).  Host only, no GPU work. */
int hyq_cache_buffer_bytes(const hyq_shape_t* shape, size_t bytes[HYQ_NBUF]);

/* Workspace bytes an operation needs: op = HYQ_OP_DECODE (len unused; n_splits = the value
   that will be passed, 0 = automatic), HYQ_OP_SELECT and HYQ_OP_SELECT_TAIL (len = context
   length), HYQ_OP_PREFILL (len = sequence length).  Returns 0 for an invalid shape. */
size_t hyq_workspace_bytes(const hyq_shape_t* shape, int op, int32_t len, int32_t n_splits);

/* Freeze: prefill -> decode cache organisation (HyQuant paper Alg. 4).
   k, v: device bf16 [B][Hkv][len][128] dense prefill keys/values.
   anchors: device int32 [B][Hkv][n_anchor], ascending per head, inside [0, len - 128);
            n_anchor may be 0 (pass NULL).  Typically the output of hyq_select_vlines.
   q_tail:  device bf16 [B][Hq][n_tail][128], the last prefill queries; the last
            min(n_tail, 64) seed the proxy ring (nullable, then n_tail must be 0).
   Effect: window ring <- positions [max(0,len-128), len); anchor store <- the anchors (bf16);
   INT4 slots <- every other position of [0, len-128) in ascending order, quantized per
   token and 32-channel group (min/max asymmetric, fp16 scale = fp16((max-min)/15), fp16
   min, codes rint((x-min)/scale) clamped to [0,15]); staging emptied; unused tails zeroed.
   Counters: len, n_int4 = max(0,len-128) - n_anchor, n_anchor, n_staged = 0, proxy.
   Two kernel launches (anchor and window copies with the quantized tiles; staging clear and
   proxy ring).
   Errors: INVALID, UNSUPPORTED, CAPACITY (len-128-n_anchor > int4_cap, n_anchor >
   anchor_cap), HIP. */
int hyq_quantize_kv(hyq_cache_t* cache, const void* k, const void* v, int32_t len,
                    const int32_t* anchors, int32_t n_anchor, const void* q_tail, int32_t n_tail,
                    hipStream_t stream);

/* Append one decode token to every sequence (HyQuant paper Alg. 3 staging segment, Alg. 4
   staging buffer): position len enters window slot len % 128; when len >= 128 the position
   it replaces (len - 128) moves to staging slot n_staged.  q_t (nullable) is pushed into the
   proxy ring.  k_t, v_t: device bf16 [B][Hkv][128]; q_t: device bf16 [B][Hq][128].
   Counters: len += 1, n_staged += (old len >= 128), proxy ring advanced.
   Errors: INVALID, CAPACITY (staging full: call hyq_select_vlines with apply = 1), HIP. */
int hyq_append_token(hyq_cache_t* cache, const void* k_t, const void* v_t, const void* q_t,
                     hipStream_t stream);

/* Vertical-line selector (HyQuant paper §4.1 Eq. 4-5, Alg. 1; cadence: every 64 decode
   tokens per the techwalker.com article on HyQuant).
   For each (b, KV head): rows r = every proxy query of every Q head of the group;
   p_r = softmax(q_r . k_j / sqrt(128)) over all len keys; S(j) = sum_r p_r(j) for candidate
   j in [0, len - 128); idx = the k largest S (ties to the lower position), ascending.
   Dense mode (dense_k != NULL): keys = dense_k, device bf16 [B][Hkv][len][128]; proxy =
     device bf16 [B][Hq][n_proxy][128]; cache may be NULL; apply must be 0.
   Cache mode (dense_k == NULL): keys = the cache in its stored precision, proxy = the cache's
     proxy ring (proxy must be NULL, len and n_proxy are taken from the cache).  With
     apply = 1 the new set is applied: anchors in the set keep bf16; staged positions in the
     set become anchors with their bf16 values; INT4 positions in the set become anchors
     holding bf16(dequantized value); anchors and staged positions not in the set are
     quantized into INT4 slots; staging is emptied.  Counters: n_anchor = k, n_staged = 0,
     n_int4 = len - 128 - k.
   idx_out: device int32 [B][Hkv][k]; scores_out: device f32 [B][Hkv][len - 128] (nullable).
   k must satisfy 0 <= k <= len - 128 (and <= anchor_cap when apply = 1).
   ws: device workspace of at least hyq_workspace_bytes(shape, HYQ_OP_SELECT, len, 0) bytes.
   Errors: INVALID, UNSUPPORTED, CAPACITY, WORKSPACE, HIP. */
int hyq_select_vlines(const hyq_shape_t* shape, hyq_cache_t* cache, const void* dense_k,
                      int32_t len, const void* proxy, int32_t n_proxy, int32_t k, int32_t apply,
                      int32_t* idx_out, float* scores_out, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* Vertical-token identification as the HyQuant paper's Alg. 1 writes it (appendix A.1), the
   literal alternative to hyq_select_vlines' Eq. 4 scores.  For each (b, Q head h):
     qbar_h = mean of the last t = min(128, n_q) query rows (fp32: four partial sums of 32
              consecutive rows each, in ascending row order, added in row order, then an
              IEEE divide by t);
     S_h(j) = qbar_h . k_j for every prefix key j in [0, P), P = len - 128, with the keys of KV
              head h / (Hq / Hkv) (raw logits: no 1/sqrt(128), no softmax; fp32);
     idx_h  = the k largest S_h (ties to the lower position; +0 and -0 tie), ascending.
   One set per Q head: the sets of one KV group may differ, so they are not applied to a cache.
   k: device bf16 [B][Hkv][len][128]; q: device bf16 [B][Hq][n_q][128]; idx_out: device int32
   [B][Hq][k_sel] (nullable when k_sel = 0); scores_out: device f32 [B][Hq][P] (nullable).
   k_sel: 0 <= k_sel <= P (Alg. 1 takes min(P, max(1, ceil(P r))); the caller passes it).
   P = 0 (len <= 128) is accepted with k_sel = 0 and does nothing.
   ws: device workspace of at least hyq_workspace_bytes(shape, HYQ_OP_SELECT_TAIL, len, 0)
   bytes, no initialisation needed; calls sharing one workspace must not overlap in time.
   Three kernel launches (tail means, logits, top-k).  Reads k and q only.
   Errors: INVALID (null pointers, len or n_q <= 0, k_sel outside [0, P]), UNSUPPORTED,
   WORKSPACE, HIP. */
int hyq_select_vlines_tail(const hyq_shape_t* shape, const void* k, int32_t len, const void* q,
                           int32_t n_q, int32_t k_sel, int32_t* idx_out, float* scores_out,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* Decode attention over the hybrid cache (HyQuant paper §4.3 Eq. 8-9, Alg. 3): for every
   (b, Q head), o = sum_j softmax_j(q . k_j / sqrt(128)) v_j over all len cached positions,
   INT4 positions dequantized in registers, bf16 anchors, staging and window in the same
   online softmax; split-K partial states merged by ReduceSoftmax.
   q: device bf16 [B][Hq][128]; o: device f32 [B][Hq][128].  n_splits: splits per (b, KV
   head), 0 = automatic.  ws: >= hyq_workspace_bytes(shape, HYQ_OP_DECODE, 0, n_splits) bytes
   of scratch for the split partial states (no initialisation needed); calls sharing one
   workspace must not overlap in time (same stream is fine).  Two kernel launches (splits,
   then their merge); with one split, one launch that writes o itself.  Reads the cache
   only.  Errors: INVALID, UNSUPPORTED, WORKSPACE, HIP. */
int hyq_decode_attn(const hyq_cache_t* cache, const void* q, float* o, int32_t n_splits,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate (code under graph capture, serving loops or harnesses
   that forbid allocation): hyq_decode_attn with its split records in a static device array of
   HYQ_NOALLOC_SCRATCH_BYTES per GPU (allocated with the library's code object, held until the
   process ends) instead of a caller workspace.  Same arguments, kernels, results and errors as
   hyq_decode_attn, plus WORKSPACE when batch * n_q_heads * splits * 130 * 4 bytes exceed the
   scratch (splits = n_splits, or the automatic count).  Calls no allocating routine.  Every
   call on one GPU uses that GPU's one array: calls that overlap in time on one GPU (two
   streams, two threads) race; calls on one stream are ordered and safe.  No initialisation
   is needed (every record is written before it is read). */
#define HYQ_NOALLOC_SCRATCH_BYTES (8u << 20)
int hyq_decode_attn_noalloc(const hyq_cache_t* cache, const void* q, float* o, int32_t n_splits,
                            hipStream_t stream);

/* Decode attention over a variable-length batch (the HyQuant paper's Alg. 3 for each
   sequence; the paper's batched decode runs sequences of one length).  Each sequence is its
   own single-sequence cache (shape.batch = 1), sized for its own length and maintained on its
   own cadence by hyq_append_token and hyq_select_vlines; this call decodes them together in
   one launch of the split kernel and one of the merge.  Every cache must share n_q_heads,
   n_kv_heads and bits; capacities and counters may differ.
   caches: host array of n_seq pointers (1 <= n_seq <= 1024), read only.
   q: device bf16 [n_seq][Hq][128]; o: device f32 [n_seq][Hq][128].
   n_splits: splits per (sequence, KV head); 0 = automatic (the device's split columns are
   shared in proportion to each sequence's tile count, at least one each).
   table: caller-owned HOST memory of at least hyq_decode_ragged_table_bytes(&caches[0]->shape,
   n_seq, n_splits) bytes.  The call writes into it the caches' pointers and counters and the
   split plan (about 112 bytes per sequence plus 4 per split, the layout of the head of the
   workspace) and enqueues one host-to-device copy of it into `ws` on `stream`, then the two
   kernels.  The caller keeps `table` unchanged until the stream has passed the call (a ring of
   tables, or an event, is the caller's).  Page-locked memory (hipHostMalloc, a pinned torch
   tensor) keeps the copy asynchronous and lets the call be recorded into a graph: a replay
   copies whatever `table` holds at that moment, so after appends or refreshes change the
   counters, rewrite it with hyq_decode_ragged_plan (same caches, same n_splits; the replay is
   valid while the total split count it returns is the one recorded).
   ws: >= hyq_decode_ragged_workspace_bytes(&caches[0]->shape, n_seq, n_splits) bytes of
   device scratch, no initialisation needed.  Calls sharing one workspace must not overlap in
   time (same stream is fine).  Reads the caches only; allocates, frees and waits for nothing.
   Errors: INVALID (null or mismatched cache, batch != 1, len = 0, n_splits > 4096 or more
   than 16384 splits in all), UNSUPPORTED, CAPACITY (n_seq > 1024), WORKSPACE (table or ws
   missing or too small), HIP. */
int hyq_decode_attn_ragged(const hyq_cache_t* const* caches, int32_t n_seq, const void* q, float* o,
                           int32_t n_splits, void* table, size_t table_bytes, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* Host only: writes the table hyq_decode_attn_ragged would write for these caches (same checks
   and errors, no GPU work) and, if total_splits is not NULL, the number of split workgroup
   columns the launch uses. */
int hyq_decode_ragged_plan(const hyq_cache_t* const* caches, int32_t n_seq, int32_t n_splits, void* table,
                           size_t table_bytes, int32_t* total_splits);

/* Workspace bytes of hyq_decode_attn_ragged for n_seq sequences whose heads match `s`
   (s->batch is ignored): an upper bound over any lengths for the automatic plan
   (n_splits = 0), exact for a fixed n_splits.  0 for an invalid shape or n_seq outside
   1..1024. */
size_t hyq_decode_ragged_workspace_bytes(const hyq_shape_t* s, int32_t n_seq, int32_t n_splits);

/* Host table bytes of hyq_decode_attn_ragged (same bound rules as the workspace). */
size_t hyq_decode_ragged_table_bytes(const hyq_shape_t* s, int32_t n_seq, int32_t n_splits);

/* Hybrid prefill attention (HyQuant paper §4.2 Eq. 6-7, Alg. 2), causal, one sequence per
   call (shape->batch must be 1; Q head h reads KV head h / (Hq / Hkv)).
   For query i: keys [i-127, i] and anchors a <= i-128 use bf16 Q.K and bf16 P.V; every
   other key j <= i-128 uses INT8 Q.K and FP8 E4M3 P.V (Alg. 2 Stage 2):
     Q: per 64-query block and Q head, scale s_Q = max|Q_blk| / 127 (fp32, IEEE divide),
        code = clamp(rint(q / s_Q), -127, 127), 0 when s_Q = 0;
     K: per 64-key block and KV head, same rule with the anchor rows left out of the
        maximum (their codes are 0 and never used);
     V: per channel and KV head, s_V[c] = max over non-anchor keys of |V[:,c]| / 448,
        code = E4M3(v / s_V[c]) rounded to nearest even (0 when s_V[c] = 0);
     score = dot_int32 * s_Q * s_K / sqrt(128); P = E4M3(448 p) / 448 on these keys and
     bf16(p) on the bf16 keys, p = exp(score - running max) after the tile's max update.
   One online softmax per row over 64-key tiles in the order: quantized tiles (ascending),
   anchor tiles (64 consecutive entries of the anchor list), window tiles (aligned).
   q: device bf16 [Hq][len][128]; k, v: device bf16 [Hkv][len][128]; anchors: device int32
   [Hkv][n_anchor], ascending and distinct inside [0, len-128) (nullable when n_anchor = 0;
   other contents give unspecified results but no out-of-bounds access);
   o: device f32 [Hq][len][128].
   ws: device workspace of at least hyq_workspace_bytes(shape, HYQ_OP_PREFILL, len, 0)
   bytes, no initialisation needed.  After the call it holds the operands, in this order,
   each section starting at a multiple of 256 bytes (Np = len rounded up to 128):
     q8   int8 [Hq][Np][128]        Q codes, operand order (below), rows >= len zero
     sq   f32  [Hq][Np/64]          s_Q per 64-query block
     k8   int8 [Hkv][Np/64][8][64][16] K codes: 16-byte chunk k of the operand-order row
                                    of key 64 T + r at (tile T, k, r)
     sk   f32  [Hkv][Np/64]         s_K per 64-key block
     v8   u8   [Hkv][Np/32][2][128][16] V codes: byte e of (32-key block b, half h,
                                    channel c) is key 32 b + 16 (e >> 3) + 8 h + (e & 7)
     sv   f32  [Hkv][128]           s_V
     vmax f32  [Hkv][Np/64][128]    per-block max |V| over non-anchor keys
     abits u32 [Hkv][Np/32]         anchor bitmap (bit j & 31 of word j >> 5)
     vt16 bf16 [Hkv][Np/8][128][8]  V (all keys, rows >= len zero): element e of (group g,
                                    channel c) is key 8 g + e
     ka16 bf16 [Hkv][Ap][128]       K rows of the anchors in list order (Ap = n_anchor
                                    rounded up to 64; the section is sized for anchor_cap)
     va16 bf16 [Hkv][Ap/8][128][8]  V of the anchors in list order, layout of vt16
   Operand order of an INT8 row: byte 64 s + 16 j + 8 t + e holds channel
   32 (2 s + t) + 8 j + e (s, t in {0,1}, j < 4, e < 8).
   Calls sharing one workspace must not overlap in time (same stream is fine).
   Four kernel launches (K quantization with the anchor bitmap and gather, V scale, V
   quantization, attention).  Errors: INVALID (null pointers, len <= 0, n_anchor outside
   [0, max(0, len-128)]), CAPACITY (n_anchor > shape->anchor_cap), UNSUPPORTED (batch != 1,
   len > HYQ_PREFILL_MAX_LEN), WORKSPACE, HIP. */
#define HYQ_PREFILL_MAX_LEN (1 << 20)
int hyq_prefill_attn(const hyq_shape_t* shape, const void* q, const void* k, const void* v,
                     int32_t len, const int32_t* anchors, int32_t n_anchor, float* o, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/* Hybrid prefill attention with a 4-bit bulk Q.K (HyQuant paper §4.2, the INT4/FP4 option for
   the bulk operands): as hyq_prefill_attn in every argument, error and key partition, except
   that the bulk Q.K uses MXFP4 (OCP Microscaling) operands instead of INT8:
     Q and K (every row, anchors included), per row and 32-channel block: shared exponent
        e = clamp(floor(log2 max|x|) - 2, -127, 127) (-127 for an all-zero block), codes
        = E2M1(x * 2^-e) rounded to nearest even and saturated at +-6;
     score = fp32(sum over blocks of 2^(eQ + eK) * dot(codes)) / sqrt(128).
   P.V, V codes, s_V and the bf16 keys are as in hyq_prefill_attn.  Workspace sections as there,
   with q8 and k8 reinterpreted and sq, sk left unwritten:
     q8 row (128 bytes): byte 16 j + i/2 holds channel 32 j + i of block j (i even in the low
        nibble), byte 64 + j the biased exponent e + 127 of block j, bytes 68.. unspecified;
     k8 tile of 64 keys (8192 bytes): byte (j 64 + r) 16 + i/2 holds channel 32 j + i of key
        64 T + r; byte 4096 + (j 16 + (r & 15)) 4 + (r >> 4) holds that key's block-j e + 127;
        the rest unspecified. */
int hyq_prefill_attn_mx(const hyq_shape_t* shape, const void* q, const void* k, const void* v,
                        int32_t len, const int32_t* anchors, int32_t n_anchor, float* o, void* ws,
                        size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* HYQ_H */

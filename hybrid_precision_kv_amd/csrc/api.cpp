// C ABI of the hybrid-precision KV attention library: argument validation, host-side cache
// counters, workspace sizing and kernel launches.  Declarations and contracts: include/hyq.h.
#include <atomic>
#include <hip/hip_runtime.h>
#include <queue>
#include <string.h>
#include <vector>

#include "../../include/hyq.h"
#include "hyq_launch.h"

namespace {

constexpr int D = HYQ_HEAD_DIM;
constexpr int W = HYQ_WINDOW;

int check_shape(const hyq_shape_t* s) {
  if (!s) return HYQ_ERR_INVALID;
  if (s->batch <= 0 || s->n_q_heads <= 0 || s->n_kv_heads <= 0) return HYQ_ERR_INVALID;
  if (s->head_dim != D || s->group != HYQ_GROUP || s->window != W || s->proxy_cap != HYQ_PROXY_CAP)
    return HYQ_ERR_UNSUPPORTED;
  if (s->n_q_heads % s->n_kv_heads) return HYQ_ERR_INVALID;
  const int g = s->n_q_heads / s->n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) return HYQ_ERR_UNSUPPORTED;
  if (s->staging_cap <= 0 || s->staging_cap % 32 || s->int4_cap < 0 || s->int4_cap % 32 || s->anchor_cap < 0 ||
      s->anchor_cap % 32)
    return HYQ_ERR_INVALID;
  const int bk = s->bits ? s->bits : 4, bv = s->bits_v ? s->bits_v : bk;
  if (!((bk == 4 && bv == 4) || (bk == 8 && bv == 8) || (bk == 4 && bv == 2) || (bk == 2 && bv == 2)))
    return HYQ_ERR_UNSUPPORTED;
  return HYQ_OK;
}

// B_K and B_V of a (validated) shape
int qbits(const hyq_shape_t* s) { return s->bits ? s->bits : 4; }
int qbits_v(const hyq_shape_t* s) { return s->bits_v ? s->bits_v : qbits(s); }

size_t nheads(const hyq_shape_t* s) { return (size_t)s->batch * s->n_kv_heads; }

int check_cache_ptrs(const hyq_cache_t* c) {
  if (!c->int4 || !c->slot_pos || !c->a_k || !c->a_v || !c->a_pos ||
      !c->s_k || !c->s_v || !c->w_k || !c->w_v || !c->proxy_q)
    return HYQ_ERR_INVALID;
  return HYQ_OK;
}

hyq::CacheView view(const hyq_cache_t* c) {
  hyq::CacheView v;
  v.int4 = (uint8_t*)c->int4;
  v.slot_pos = c->slot_pos;
  v.a_k = (uint16_t*)c->a_k;
  v.a_v = (uint16_t*)c->a_v;
  v.a_pos = c->a_pos;
  v.s_k = (uint16_t*)c->s_k;
  v.s_v = (uint16_t*)c->s_v;
  v.w_k = (uint16_t*)c->w_k;
  v.w_v = (uint16_t*)c->w_v;
  v.proxy_q = (uint16_t*)c->proxy_q;
  v.B = c->shape.batch;
  v.Hkv = c->shape.n_kv_heads;
  v.G = c->shape.n_q_heads / c->shape.n_kv_heads;
  v.int4_cap = c->shape.int4_cap;
  v.anchor_cap = c->shape.anchor_cap;
  v.staging_cap = c->shape.staging_cap;
  v.proxy_cap = c->shape.proxy_cap;
  v.bits = qbits(&c->shape);
  v.bits_v = qbits_v(&c->shape);
  return v;
}

// consistency of the host counters with the method's invariants
int check_counters(const hyq_cache_t* c) {
  const hyq_shape_t& s = c->shape;
  if (c->len < 0 || c->n_int4 < 0 || c->n_anchor < 0 || c->n_staged < 0) return HYQ_ERR_INVALID;
  const int P = c->len > W ? c->len - W : 0;
  if (c->n_int4 + c->n_anchor + c->n_staged != P) return HYQ_ERR_INVALID;
  if (c->n_int4 > s.int4_cap || c->n_anchor > s.anchor_cap || c->n_staged > s.staging_cap) return HYQ_ERR_CAPACITY;
  if (c->n_proxy < 0 || c->n_proxy > s.proxy_cap || c->proxy_head < 0 || c->proxy_head >= s.proxy_cap)
    return HYQ_ERR_INVALID;
  return HYQ_OK;
}

// select workspace layout (all sizes rounded to 256 bytes)
struct SelectWs {
  size_t qsum, pq16, pqbf, rowpart, rowstat, scores, refresh, status, total;
  int rb_max;
  size_t per_head;
  int inset_words, del_words, max_moves, n_tasks;
};
size_t r256(size_t x) { return (x + 255) / 256 * 256; }
SelectWs select_ws(const hyq_shape_t* s, int32_t len) {
  SelectWs w;
  const size_t H = nheads(s);
  const int G = s->n_q_heads / s->n_kv_heads;
  const size_t R = (size_t)s->proxy_cap * G;
  const int P = len > W ? len - W : 0;
  const int n_tiles_max = (len + 31) / 32 + 4;
  w.n_tasks = hyq::select_task_count(n_tiles_max);
  w.inset_words = (P + 31) / 32 + 1;
  w.del_words = (s->int4_cap + 31) / 32 + 1;
  w.max_moves = 2 * s->anchor_cap + s->staging_cap + 32;
  w.per_head = r256(hyq::refresh_scratch_bytes(w.inset_words, w.del_words, s->anchor_cap, w.max_moves));
  w.rb_max = (int)((R + 15) / 16);
  w.qsum = 0;
  w.pq16 = w.qsum + r256(H * R * 4 * 4);
  w.pqbf = w.pq16 + r256(H * (size_t)w.rb_max * 256 * 16);
  w.rowpart = w.pqbf + r256(H * (size_t)w.rb_max * 256 * 16);
  w.rowstat = w.rowpart + r256(H * w.n_tasks * R * 2 * 4);
  w.scores = w.rowstat + r256(H * R * 2 * 4);
  w.refresh = w.scores + r256(H * (size_t)(P > 0 ? P : 1) * 4);
  w.status = w.refresh + H * w.per_head;
  w.total = w.status + r256(H * 4);
  return w;
}

// Alg. 1 selector workspace: tail means [B][Hq][128] f32, then order keys [B][Hq][P] u32
struct TailWs {
  size_t qbar, keys, total;
};
TailWs tail_ws(const hyq_shape_t* s, int32_t len) {
  TailWs w;
  const size_t BH = (size_t)s->batch * s->n_q_heads;
  const size_t P = len > W ? (size_t)(len - W) : 1;
  w.qbar = 0;
  w.keys = r256(BH * D * 4);
  w.total = w.keys + r256(BH * P * 4);
  return w;
}

// prefill workspace layout (sections in this order, each rounded up to 256 bytes)
struct PrefillWs {
  size_t q8, sq, k8, sk, v8, sv, vmax, abits, vt16, ka16, va16, total;
  int Npad;
};
PrefillWs prefill_ws(const hyq_shape_t* s, int32_t len) {
  PrefillWs w;
  const size_t Hq = s->n_q_heads, Hkv = s->n_kv_heads;
  const size_t Np = (size_t)(len + 127) / 128 * 128;
  w.Npad = (int)Np;
  w.q8 = 0;
  w.sq = w.q8 + r256(Hq * Np * D);
  w.k8 = w.sq + r256(Hq * (Np / 64) * 4);
  w.sk = w.k8 + r256(Hkv * Np * D);
  w.v8 = w.sk + r256(Hkv * (Np / 64) * 4);
  w.sv = w.v8 + r256(Hkv * Np * D);
  w.vmax = w.sv + r256(Hkv * D * 4);
  w.abits = w.vmax + r256(Hkv * (Np / 64) * D * 4);
  w.vt16 = w.abits + r256(Hkv * (Np / 32) * 4);
  const size_t Ac = (size_t)(s->anchor_cap + 63) / 64 * 64;
  w.ka16 = w.vt16 + r256(Hkv * Np * D * 2);
  w.va16 = w.ka16 + r256(Hkv * Ac * D * 2);
  w.total = w.va16 + r256(Hkv * Ac * D * 2);
  return w;
}

// compute units of the current device (cached per device; 256 if the query fails)
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Splits per (b, KV head).  Long streams per worker: one full round of two workgroups per CU
// (the register budget fits two) when every wave still gets >= 16 tiles.  Otherwise the call
// is latency bound and one workgroup per CU does better, down to about one tile per wave but
// never fewer than 16 splits (measured at batch 1 with the one-latency merge: 16 and 32 splits
// tie at 1K tokens, 32 is best at 4K, 16K and 32K, 48 and 64 are slower everywhere; at batch
// 16 x 32K, 4 splits = two workgroups per CU).
int auto_splits(const hyq_cache_t* c, int* waves) {
  const int G = c->shape.n_q_heads / c->shape.n_kv_heads;
  const long units = (long)nheads(&c->shape) * hyq::decode_head_blocks(G);
  const long tiles = (c->n_int4 + 31) / 32 + 3 * ((c->n_anchor + 31) / 32 + (c->n_staged + 31) / 32 + 4);
  const long cus = cu_count();
  // K2V2 workgroups fit three per CU and gain from it (6 splits at bs16 x 32K: 96.9 against
  // 100.7 us); K4V2, K4V4 and K8V8 measure best at two
  const long per_cu = qbits(&c->shape) + qbits_v(&c->shape) == 4 ? 3 : 2;
  long s = (per_cu * cus + units - 1) / units;
  *waves = 4;
  if (tiles < 16 * 4 * s) {
    s = (cus + units - 1) / units;
    long by_work = (tiles + 3) / 4;
    if (by_work < 16) by_work = 16;
    if (s > by_work) s = by_work;
    // eight waves per workgroup when every wave still gets a tile (more loads in flight, a
    // shorter chain per wave); with fewer tiles the extra waves idle
    if (tiles >= 8 * s) *waves = 8;
  }
  if (s < 1) s = 1;
  if (s > 256) s = 256;
  return (int)s;
}

// ---- variable-length batches: one decode launch over many single-sequence caches

// Split plan.  Each sequence's work is counted in tiles as in auto_splits.  The chip's budget
// of split columns (two workgroups per CU; one per CU when every wave would get fewer than
// 16 tiles) is dealt out one column at a time to the sequence with the most tiles per split
// (ties to the lower index), starting from one split each: the largest per-split load, which
// sets the launch's time, is as small as whole columns allow.  On the short-batch budget a
// sequence takes at most max(16, tiles / 4) splits (as auto_splits).  The total never exceeds
// ragged_split_bound().
int ragged_columns(int Hkv, int G, bool two_per_cu) {
  const long u1 = (long)Hkv * hyq::decode_head_blocks(G);
  const long cus = cu_count();
  return (int)(((two_per_cu ? 2 : 1) * cus + u1 - 1) / u1);
}
long ragged_split_bound(int n_seq, int Hkv, int G, int n_splits) {
  return n_splits > 0 ? (long)n_seq * n_splits : (long)ragged_columns(Hkv, G, true) + 2L * n_seq;
}
long seq_tiles(const hyq_cache_t* c) {
  return (c->n_int4 + 31) / 32 + 3 * ((c->n_anchor + 31) / 32 + (c->n_staged + 31) / 32 + 4);
}
void ragged_plan(const hyq_cache_t* const* cs, int n, int Hkv, int G, int n_splits, int* out) {
  for (int i = 0; i < n; ++i) out[i] = n_splits > 0 ? n_splits : 1;
  if (n_splits > 0) return;
  long total = 0;
  for (int i = 0; i < n; ++i) total += seq_tiles(cs[i]);
  long C = ragged_columns(Hkv, G, true);
  const bool low = total < 64 * C;
  if (low) C = ragged_columns(Hkv, G, false);
  // max-heap on tiles / splits, compared exactly as t_a * s_b vs t_b * s_a
  struct Item {
    long t;
    int s, i;
  };
  auto less = [](const Item& a, const Item& b) {
    const long l = a.t * b.s, r = b.t * a.s;
    return l != r ? l < r : a.i > b.i;
  };
  std::priority_queue<Item, std::vector<Item>, decltype(less)> heap(less);
  for (int i = 0; i < n; ++i) heap.push({seq_tiles(cs[i]), 1, i});
  for (long left = C - n; left > 0 && !heap.empty(); --left) {
    Item it = heap.top();
    heap.pop();
    const long cap = low ? ((it.t + 3) / 4 > 16 ? (it.t + 3) / 4 : 16) : 1L << 30;
    if (it.s >= cap) {  // this sequence is done; the column goes to the next one
      ++left;
      continue;
    }
    out[it.i] = ++it.s;
    heap.push(it);
  }
}

// workspace of a variable-length decode: descriptors, split map, then the partial records
struct RaggedWs {
  size_t seqs, map, part, total;
};
RaggedWs ragged_ws(int n_seq, int Hq, int Hkv, int n_splits) {
  RaggedWs w;
  const long bound = ragged_split_bound(n_seq, Hkv, Hq / Hkv, n_splits);
  w.seqs = 0;
  w.map = r256((size_t)n_seq * sizeof(hyq::RaggedSeq));
  w.part = w.map + r256((size_t)bound * 4);
  w.total = w.part + (size_t)bound * Hq * (D + 2) * sizeof(float);
  return w;
}

constexpr int RAGGED_MAX_SEQ = 1024;
constexpr long RAGGED_MAX_SPLITS = 16384;

// Checks a variable-length batch and writes its descriptors and split plan into `table` (host
// memory of at least w.part bytes, laid out as the head of the workspace).  Host only.
int ragged_prepare(const hyq_cache_t* const* caches, int32_t n_seq, int32_t n_splits, void* table,
                   size_t table_bytes, RaggedWs& w, long& total) {
  if (!caches || n_seq <= 0 || n_splits < 0 || n_splits > 4096) return HYQ_ERR_INVALID;
  if (n_seq > RAGGED_MAX_SEQ) return HYQ_ERR_CAPACITY;
  int st;
  for (int i = 0; i < n_seq; ++i) {
    const hyq_cache_t* c = caches[i];
    if (!c) return HYQ_ERR_INVALID;
    if ((st = check_shape(&c->shape))) return st;
    if ((st = check_cache_ptrs(c))) return st;
    if ((st = check_counters(c))) return st;
    if (c->shape.batch != 1 || c->len <= 0) return HYQ_ERR_INVALID;
    if (c->shape.n_q_heads != caches[0]->shape.n_q_heads || c->shape.n_kv_heads != caches[0]->shape.n_kv_heads ||
        qbits(&c->shape) != qbits(&caches[0]->shape) || qbits_v(&c->shape) != qbits_v(&caches[0]->shape))
      return HYQ_ERR_INVALID;
  }
  const hyq_shape_t& s0 = caches[0]->shape;
  const int Hq = s0.n_q_heads, Hkv = s0.n_kv_heads, G = Hq / Hkv;
  w = ragged_ws(n_seq, Hq, Hkv, n_splits);
  if (!table || table_bytes < w.part) return HYQ_ERR_WORKSPACE;
  int plan[RAGGED_MAX_SEQ];
  ragged_plan(caches, n_seq, Hkv, G, n_splits, plan);
  total = 0;
  for (int i = 0; i < n_seq; ++i) total += plan[i];
  if (total > ragged_split_bound(n_seq, Hkv, G, n_splits) || total > RAGGED_MAX_SPLITS) return HYQ_ERR_INVALID;
  uint8_t* host = (uint8_t*)table;
  hyq::RaggedSeq* seqs = (hyq::RaggedSeq*)(host + w.seqs);
  uint32_t* map = (uint32_t*)(host + w.map);
  long rec = 0, col = 0;
  for (int i = 0; i < n_seq; ++i) {
    const hyq_cache_t* c = caches[i];
    hyq::RaggedSeq d;
    memset(&d, 0, sizeof d);
    d.int4 = (const uint8_t*)c->int4;
    d.a_k = (const uint16_t*)c->a_k;
    d.a_v = (const uint16_t*)c->a_v;
    d.s_k = (const uint16_t*)c->s_k;
    d.s_v = (const uint16_t*)c->s_v;
    d.w_k = (const uint16_t*)c->w_k;
    d.w_v = (const uint16_t*)c->w_v;
    d.int4_cap = c->shape.int4_cap;
    d.anchor_cap = c->shape.anchor_cap;
    d.staging_cap = c->shape.staging_cap;
    d.n_int4 = c->n_int4;
    d.n_anchor = c->n_anchor;
    d.n_staged = c->n_staged;
    d.n_win = c->len < W ? c->len : W;
    d.n_splits = plan[i];
    d.rec0 = (int)rec;
    memcpy(&seqs[i], &d, sizeof d);
    rec += (long)Hq * plan[i];
    for (int j = 0; j < plan[i]; ++j) map[col++] = ((uint32_t)i << 16) | (uint32_t)j;
  }
  // the gap between the descriptors and the map is padding: keep it defined
  memset(host + w.seqs + (size_t)n_seq * sizeof(hyq::RaggedSeq), 0, w.map - w.seqs - (size_t)n_seq * sizeof(hyq::RaggedSeq));
  memset(host + w.map + (size_t)total * 4, 0, w.part - w.map - (size_t)total * 4);
  return HYQ_OK;
}

}  // namespace

extern "C" {

const char* hyq_status_string(int status) {
  switch (status) {
    case HYQ_OK: return "ok";
    case HYQ_ERR_INVALID: return "invalid argument";
    case HYQ_ERR_UNSUPPORTED: return "unsupported shape";
    case HYQ_ERR_CAPACITY: return "capacity exceeded";
    case HYQ_ERR_WORKSPACE: return "workspace missing or too small";
    case HYQ_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

int hyq_cache_buffer_bytes(const hyq_shape_t* s, size_t bytes[HYQ_NBUF]) {
  int st = check_shape(s);
  if (st) return st;
  if (!bytes) return HYQ_ERR_INVALID;
  const size_t H = nheads(s);
  // per 32-slot tile: 512 (B_K + B_V) code bytes and 1024 bytes of (scale, min)
  bytes[HYQ_BUF_INT4] = H * s->int4_cap * (size_t)((512 * (qbits(s) + qbits_v(s)) + 1024) / 32);
  bytes[HYQ_BUF_SLOT_POS] = H * s->int4_cap * 4;
  bytes[HYQ_BUF_A_K] = H * s->anchor_cap * D * 2;
  bytes[HYQ_BUF_A_V] = H * s->anchor_cap * D * 2;
  bytes[HYQ_BUF_A_POS] = H * s->anchor_cap * 4;
  bytes[HYQ_BUF_S_K] = H * s->staging_cap * D * 2;
  bytes[HYQ_BUF_S_V] = H * s->staging_cap * D * 2;
  bytes[HYQ_BUF_W_K] = H * W * D * 2;
  bytes[HYQ_BUF_W_V] = H * W * D * 2;
  bytes[HYQ_BUF_PROXY_Q] = (size_t)s->batch * s->n_q_heads * s->proxy_cap * D * 2;
  return HYQ_OK;
}

size_t hyq_workspace_bytes(const hyq_shape_t* s, int op, int32_t len, int32_t n_splits) {
  if (check_shape(s)) return 0;
  switch (op) {
    case HYQ_OP_DECODE: {
      const int S = n_splits > 0 ? n_splits : 256;
      return (size_t)s->batch * s->n_q_heads * S * (D + 2) * sizeof(float);
    }
    case HYQ_OP_SELECT: return len > 0 ? select_ws(s, len).total : 0;
    case HYQ_OP_PREFILL: return len > 0 && len <= HYQ_PREFILL_MAX_LEN ? prefill_ws(s, len).total : 0;
    case HYQ_OP_SELECT_TAIL: return len > 0 ? tail_ws(s, len).total : 0;
    default: return 0;
  }
}

int hyq_quantize_kv(hyq_cache_t* c, const void* k, const void* v, int32_t len, const int32_t* anchors,
                    int32_t n_anchor, const void* q_tail, int32_t n_tail, hipStream_t stream) {
  if (!c) return HYQ_ERR_INVALID;
  int st = check_shape(&c->shape);
  if (st) return st;
  if ((st = check_cache_ptrs(c))) return st;
  if (!k || !v || len <= 0 || n_anchor < 0 || n_tail < 0) return HYQ_ERR_INVALID;
  if (n_anchor > 0 && !anchors) return HYQ_ERR_INVALID;
  if (n_tail > 0 && !q_tail) return HYQ_ERR_INVALID;
  const int P = len > W ? len - W : 0;
  if (n_anchor > P) return HYQ_ERR_CAPACITY;
  if (n_anchor > c->shape.anchor_cap || P - n_anchor > c->shape.int4_cap) return HYQ_ERR_CAPACITY;
  hipError_t e = hyq::launch_freeze(view(c), (const uint16_t*)k, (const uint16_t*)v, len, anchors, n_anchor,
                                    (const uint16_t*)q_tail, n_tail, stream);
  if (e != hipSuccess) return HYQ_ERR_HIP;
  c->len = len;
  c->n_anchor = n_anchor;
  c->n_int4 = P - n_anchor;
  c->n_staged = 0;
  const int np = n_tail < c->shape.proxy_cap ? n_tail : c->shape.proxy_cap;
  c->n_proxy = np;
  c->proxy_head = np % c->shape.proxy_cap;
  return HYQ_OK;
}

int hyq_append_token(hyq_cache_t* c, const void* k_t, const void* v_t, const void* q_t, hipStream_t stream) {
  if (!c) return HYQ_ERR_INVALID;
  int st = check_shape(&c->shape);
  if (st) return st;
  if ((st = check_cache_ptrs(c))) return st;
  if ((st = check_counters(c))) return st;
  if (!k_t || !v_t || c->len <= 0) return HYQ_ERR_INVALID;
  const bool leaves = c->len >= W;
  if (leaves && c->n_staged >= c->shape.staging_cap) return HYQ_ERR_CAPACITY;
  hipError_t e = hyq::launch_append(view(c), (const uint16_t*)k_t, (const uint16_t*)v_t, (const uint16_t*)q_t,
                                    c->len, c->n_staged, c->proxy_head, stream);
  if (e != hipSuccess) return HYQ_ERR_HIP;
  c->len += 1;
  if (leaves) c->n_staged += 1;
  if (q_t) {
    c->proxy_head = (c->proxy_head + 1) % c->shape.proxy_cap;
    if (c->n_proxy < c->shape.proxy_cap) c->n_proxy += 1;
  }
  return HYQ_OK;
}

}  // extern "C"

// hyq_decode_attn and hyq_decode_attn_noalloc: checks, split count, launch with `ws` (device
// memory of ws_bytes, or the static scratch when `noalloc`) as the split records
static int decode_common(const hyq_cache_t* c, const void* q, float* o, int32_t n_splits, void* ws, size_t ws_bytes,
                         bool noalloc, hipStream_t stream) {
  if (!c) return HYQ_ERR_INVALID;
  int st = check_shape(&c->shape);
  if (st) return st;
  if ((st = check_cache_ptrs(c))) return st;
  if ((st = check_counters(c))) return st;
  if (!q || !o || c->len <= 0 || n_splits < 0 || n_splits > 4096) return HYQ_ERR_INVALID;
  int waves = 4;
  const int S = n_splits > 0 ? n_splits : auto_splits(c, &waves);
  const size_t need = (size_t)c->shape.batch * c->shape.n_q_heads * S * (D + 2) * sizeof(float);
  if (noalloc) {
    if (need > HYQ_NOALLOC_SCRATCH_BYTES) return HYQ_ERR_WORKSPACE;
    float* p = nullptr;
    if (hyq::noalloc_scratch(&p) != hipSuccess) return HYQ_ERR_HIP;
    ws = p;
    ws_bytes = HYQ_NOALLOC_SCRATCH_BYTES;
  }
  if (!ws || ws_bytes < need) return HYQ_ERR_WORKSPACE;
  hyq::DecodeParams p;
  p.int4 = (const uint8_t*)c->int4;
  p.a_k = (const uint16_t*)c->a_k;
  p.a_v = (const uint16_t*)c->a_v;
  p.s_k = (const uint16_t*)c->s_k;
  p.s_v = (const uint16_t*)c->s_v;
  p.w_k = (const uint16_t*)c->w_k;
  p.w_v = (const uint16_t*)c->w_v;
  p.q = (const uint16_t*)q;
  p.part = (float*)ws;
  p.o = o;
  p.B = c->shape.batch;
  p.Hkv = c->shape.n_kv_heads;
  p.G = c->shape.n_q_heads / c->shape.n_kv_heads;
  p.int4_cap = c->shape.int4_cap;
  p.bits = qbits(&c->shape);
  p.bits_v = qbits_v(&c->shape);
  p.anchor_cap = c->shape.anchor_cap;
  p.staging_cap = c->shape.staging_cap;
  p.n_int4 = c->n_int4;
  p.n_anchor = c->n_anchor;
  p.n_staged = c->n_staged;
  p.n_win = c->len < W ? c->len : W;
  p.n_splits = S;
  p.waves = waves;
  hipError_t e = hyq::launch_decode(p, stream);
  return e == hipSuccess ? HYQ_OK : HYQ_ERR_HIP;
}

extern "C" {

int hyq_decode_attn(const hyq_cache_t* c, const void* q, float* o, int32_t n_splits, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  return decode_common(c, q, o, n_splits, ws, ws_bytes, false, stream);
}

int hyq_decode_attn_noalloc(const hyq_cache_t* c, const void* q, float* o, int32_t n_splits, hipStream_t stream) {
  return decode_common(c, q, o, n_splits, nullptr, 0, true, stream);
}

size_t hyq_decode_ragged_workspace_bytes(const hyq_shape_t* s, int32_t n_seq, int32_t n_splits) {
  if (check_shape(s) || n_seq <= 0 || n_seq > RAGGED_MAX_SEQ || n_splits < 0 || n_splits > 4096) return 0;
  return ragged_ws(n_seq, s->n_q_heads, s->n_kv_heads, n_splits).total;
}

size_t hyq_decode_ragged_table_bytes(const hyq_shape_t* s, int32_t n_seq, int32_t n_splits) {
  if (check_shape(s) || n_seq <= 0 || n_seq > RAGGED_MAX_SEQ || n_splits < 0 || n_splits > 4096) return 0;
  return ragged_ws(n_seq, s->n_q_heads, s->n_kv_heads, n_splits).part;
}

int hyq_decode_ragged_plan(const hyq_cache_t* const* caches, int32_t n_seq, int32_t n_splits, void* table,
                           size_t table_bytes, int32_t* total_splits) {
  RaggedWs w;
  long total = 0;
  const int st = ragged_prepare(caches, n_seq, n_splits, table, table_bytes, w, total);
  if (st) return st;
  if (total_splits) *total_splits = (int32_t)total;
  return HYQ_OK;
}

int hyq_decode_attn_ragged(const hyq_cache_t* const* caches, int32_t n_seq, const void* q, float* o,
                           int32_t n_splits, void* table, size_t table_bytes, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  if (!q || !o) return HYQ_ERR_INVALID;
  RaggedWs w;
  long total = 0;
  int st = ragged_prepare(caches, n_seq, n_splits, table, table_bytes, w, total);
  if (st) return st;
  if (!ws || ws_bytes < w.total) return HYQ_ERR_WORKSPACE;
  // descriptors and map are contiguous in the table as in the workspace: one copy
  if (hipMemcpyAsync(ws, table, w.part, hipMemcpyHostToDevice, stream) != hipSuccess) return HYQ_ERR_HIP;
  const hyq_shape_t& s0 = caches[0]->shape;
  hyq::RaggedDecodeParams p;
  p.seqs = (const hyq::RaggedSeq*)((uint8_t*)ws + w.seqs);
  p.split_map = (const uint32_t*)((uint8_t*)ws + w.map);
  p.q = (const uint16_t*)q;
  p.part = (float*)((uint8_t*)ws + w.part);
  p.o = o;
  p.n_seq = n_seq;
  p.Hkv = s0.n_kv_heads;
  p.G = s0.n_q_heads / s0.n_kv_heads;
  p.total_splits = (int)total;
  p.bits = qbits(&s0);
  p.bits_v = qbits_v(&s0);
  hipError_t e = hyq::launch_decode_ragged(p, stream);
  return e == hipSuccess ? HYQ_OK : HYQ_ERR_HIP;
}

int hyq_select_vlines(const hyq_shape_t* shape, hyq_cache_t* cache, const void* dense_k, int32_t len,
                      const void* proxy, int32_t n_proxy, int32_t k, int32_t apply, int32_t* idx_out,
                      float* scores_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  const bool dense = dense_k != nullptr;
  if (dense) {
    if (!proxy || n_proxy <= 0 || n_proxy > shape->proxy_cap || len <= 0 || apply) return HYQ_ERR_INVALID;
  } else {
    if (!cache || proxy) return HYQ_ERR_INVALID;
    if ((st = check_shape(&cache->shape))) return st;
    if (memcmp(&cache->shape, shape, sizeof(hyq_shape_t))) return HYQ_ERR_INVALID;
    if ((st = check_cache_ptrs(cache))) return st;
    if ((st = check_counters(cache))) return st;
    len = cache->len;
    n_proxy = cache->n_proxy;
    if (len <= 0 || n_proxy <= 0) return HYQ_ERR_INVALID;
  }
  const int P = len > W ? len - W : 0;
  if (k < 0 || k > P) return HYQ_ERR_CAPACITY;
  if (k > 0 && !idx_out) return HYQ_ERR_INVALID;
  if (apply && (k > shape->anchor_cap || P - k > shape->int4_cap)) return HYQ_ERR_CAPACITY;
  const SelectWs w = select_ws(shape, len);
  if (!ws || ws_bytes < w.total) return HYQ_ERR_WORKSPACE;
  char* wb = (char*)ws;
  const int G = shape->n_q_heads / shape->n_kv_heads;
  if (P > 0) {
    hyq::SelectParams p;
    memset(&p, 0, sizeof(p));
    p.dense_k = (const uint16_t*)dense_k;
    p.proxy = dense ? (const uint16_t*)proxy : (const uint16_t*)cache->proxy_q;
    p.proxy_stride = dense ? n_proxy : shape->proxy_cap;
    p.n_proxy = n_proxy;
    p.B = shape->batch;
    p.Hkv = shape->n_kv_heads;
    p.G = G;
    p.len = len;
    p.int4_cap = shape->int4_cap;
    p.bits = qbits(shape);
    p.bits_v = qbits_v(shape);
    p.anchor_cap = shape->anchor_cap;
    p.staging_cap = shape->staging_cap;
    if (dense) {
      p.n_tiles = (len + 31) / 32;
    } else {
      p.int4 = (const uint8_t*)cache->int4;
      p.slot_pos = cache->slot_pos;
      p.a_k = (const uint16_t*)cache->a_k;
      p.s_k = (const uint16_t*)cache->s_k;
      p.w_k = (const uint16_t*)cache->w_k;
      p.a_pos = cache->a_pos;
      p.n_int4 = cache->n_int4;
      p.n_anchor = cache->n_anchor;
      p.n_staged = cache->n_staged;
      p.n_win = len < W ? len : W;
      p.n_tiles = (p.n_int4 + 31) / 32 + (p.n_anchor + 31) / 32 + (p.n_staged + 31) / 32 + (p.n_win + 31) / 32;
    }
    p.n_tasks = hyq::select_task_count(p.n_tiles);
    p.k = k;
    p.qsum = (float*)(wb + w.qsum);
    p.pq16 = wb + w.pq16;
    p.pqbf = wb + w.pqbf;
    p.rb_stride = w.rb_max;
    p.rowpart = (float*)(wb + w.rowpart);
    p.rowstat = (float*)(wb + w.rowstat);
    p.scores = scores_out ? scores_out : (float*)(wb + w.scores);
    p.idx_out = idx_out;
    if (hyq::launch_select(p, stream) != hipSuccess) return HYQ_ERR_HIP;
  }
  if (apply) {
    hyq::RefreshParams r;
    memset(&r, 0, sizeof(r));
    r.int4 = (uint8_t*)cache->int4;
    r.slot_pos = cache->slot_pos;
    r.a_k = (uint16_t*)cache->a_k;
    r.a_v = (uint16_t*)cache->a_v;
    r.a_pos = cache->a_pos;
    r.s_k = (const uint16_t*)cache->s_k;
    r.s_v = (const uint16_t*)cache->s_v;
    r.idx = idx_out;
    r.B = shape->batch;
    r.Hkv = shape->n_kv_heads;
    r.len = len;
    r.k = k;
    r.int4_cap = shape->int4_cap;
    r.bits = qbits(shape);
    r.bits_v = qbits_v(shape);
    r.anchor_cap = shape->anchor_cap;
    r.staging_cap = shape->staging_cap;
    r.n_int4_old = cache->n_int4;
    r.n_anchor_old = cache->n_anchor;
    r.n_staged = cache->n_staged;
    r.ws = (uint8_t*)(wb + w.refresh);
    r.ws_per_head = w.per_head;
    r.inset_words = w.inset_words;
    r.del_words = w.del_words;
    r.max_moves = w.max_moves;
    r.status = (int*)(wb + w.status);
    if (P > 0 && hyq::launch_refresh(r, stream) != hipSuccess) return HYQ_ERR_HIP;
    cache->n_anchor = k;
    cache->n_int4 = P - k;
    cache->n_staged = 0;
  }
  return HYQ_OK;
}

}  // extern "C"

// Both prefill entry points: argument checks, workspace carving, the launch sequence.
static int prefill_common(const hyq_shape_t* shape, const void* q, const void* k, const void* v, int32_t len,
                          const int32_t* anchors, int32_t n_anchor, float* o, void* ws, size_t ws_bytes,
                          hipStream_t stream, int bulk) {
  int st = check_shape(shape);
  if (st) return st;
  if (shape->batch != 1) return HYQ_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o || len <= 0 || n_anchor < 0) return HYQ_ERR_INVALID;
  if (len > HYQ_PREFILL_MAX_LEN) return HYQ_ERR_UNSUPPORTED;
  const int P = len > W ? len - W : 0;
  if (n_anchor > P || (n_anchor > 0 && !anchors)) return HYQ_ERR_INVALID;
  if (n_anchor > shape->anchor_cap) return HYQ_ERR_CAPACITY;
  const PrefillWs w = prefill_ws(shape, len);
  if (!ws || ws_bytes < w.total) return HYQ_ERR_WORKSPACE;
  char* wb = (char*)ws;
  hyq::PrefillParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.anchors = anchors;
  p.n_anchor = n_anchor;
  p.o = o;
  p.N = len;
  p.Npad = w.Npad;
  p.Hq = shape->n_q_heads;
  p.Hkv = shape->n_kv_heads;
  p.G = shape->n_q_heads / shape->n_kv_heads;
  p.q8 = (int8_t*)(wb + w.q8);
  p.sq = (float*)(wb + w.sq);
  p.k8 = (int8_t*)(wb + w.k8);
  p.sk = (float*)(wb + w.sk);
  p.v8 = (uint8_t*)(wb + w.v8);
  p.sv = (float*)(wb + w.sv);
  p.vmax = (float*)(wb + w.vmax);
  p.abits = (uint32_t*)(wb + w.abits);
  p.vt16 = (uint16_t*)(wb + w.vt16);
  p.ka16 = (uint16_t*)(wb + w.ka16);
  p.va16 = (uint16_t*)(wb + w.va16);
  p.n_anchor_pad = (n_anchor + 63) / 64 * 64;
  p.bulk = bulk;
  if (hyq::launch_prefill(p, stream) != hipSuccess) return HYQ_ERR_HIP;
  return HYQ_OK;
}

extern "C" {

int hyq_select_vlines_tail(const hyq_shape_t* shape, const void* k, int32_t len, const void* q, int32_t n_q,
                           int32_t k_sel, int32_t* idx_out, float* scores_out, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  if (!k || !q || len <= 0 || n_q <= 0) return HYQ_ERR_INVALID;
  const int P = len > W ? len - W : 0;
  if (k_sel < 0 || k_sel > P || (k_sel > 0 && !idx_out)) return HYQ_ERR_INVALID;
  if (P == 0) return HYQ_OK;
  const TailWs w = tail_ws(shape, len);
  if (!ws || ws_bytes < w.total) return HYQ_ERR_WORKSPACE;
  hyq::TailSelectParams p;
  p.k = (const uint16_t*)k;
  p.q = (const uint16_t*)q;
  p.B = shape->batch;
  p.Hkv = shape->n_kv_heads;
  p.G = shape->n_q_heads / shape->n_kv_heads;
  p.len = len;
  p.n_q = n_q;
  p.t = n_q < W ? n_q : W;
  p.k_sel = k_sel;
  p.qbar = (float*)((char*)ws + w.qbar);
  p.keys = (uint32_t*)((char*)ws + w.keys);
  p.scores_out = scores_out;
  p.idx_out = idx_out;
  if (hyq::launch_select_tail(p, stream) != hipSuccess) return HYQ_ERR_HIP;
  return HYQ_OK;
}

int hyq_prefill_attn(const hyq_shape_t* shape, const void* q, const void* k, const void* v, int32_t len,
                     const int32_t* anchors, int32_t n_anchor, float* o, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  return prefill_common(shape, q, k, v, len, anchors, n_anchor, o, ws, ws_bytes, stream, 0);
}

int hyq_prefill_attn_mx(const hyq_shape_t* shape, const void* q, const void* k, const void* v, int32_t len,
                        const int32_t* anchors, int32_t n_anchor, float* o, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  return prefill_common(shape, q, k, v, len, anchors, n_anchor, o, ws, ws_bytes, stream, 1);
}

}  // extern "C"

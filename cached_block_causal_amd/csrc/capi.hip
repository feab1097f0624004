// C ABI of libws: argument validation, split planning, kernel launches.
// Every argument is checked before anything is enqueued; on failure nothing
// is launched, caches keep their length, and ws_last_error() says why.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "ws.h"
#include "ws_launch.hpp"

namespace {

thread_local std::string g_last_error;

ws_status fail(ws_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

ws_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return WS_OK;
  return fail(WS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }

ws_status check_cache(const ws_kv_cache* c) {
  if (!c) return fail(WS_ERR_NULL, "cache is NULL");
  if (!head_dim_ok(c->head_dim))
    return fail(WS_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", c->head_dim);
  if (c->heads < 1) return fail(WS_ERR_SHAPE, "cache heads %d < 1", c->heads);
  if (c->capacity < 0 || c->len < 0 || c->len > c->capacity)
    return fail(WS_ERR_SHAPE, "cache len %d / capacity %d invalid", c->len, c->capacity);
  if ((int64_t)c->heads * c->capacity * c->head_dim > ((int64_t)1 << 40))
    return fail(WS_ERR_SHAPE, "cache larger than 2 TiB elements");
  return WS_OK;
}

// Model of the split-KV pass used to pick a split count: each of `slots`
// concurrent workgroups streams ceil(tiles / s) + 2 tiles (the 2 stand for Q
// loads and the epilogue) at ~1.7 us per 128x64 tile at D = 128, in
// ceil(items * s / slots) rounds, plus the partials' round trip through
// memory at ~4 TB/s when s > 1.
constexpr int kSlots = 256 * 2;  // 256 CUs x 2 resident workgroups
// Resident one-wave workgroups of the narrow kernel (32 KB of LDS each):
// measured, four per CU stay resident; the run time steps up once a grid
// exceeds 1024 of them.
constexpr int kNarrowSlots = 256 * 4;
constexpr int kMaxSplits = 256;

int32_t default_splits(int32_t heads, int32_t n_q, int32_t head_dim, int64_t n_keys) {
  if (heads <= 0 || n_q <= 0 || n_keys <= 0 || head_dim <= 0) return 1;
  const int64_t items = (int64_t)heads * (((int64_t)n_q + ws::kAttnBlockM - 1) / ws::kAttnBlockM);
  const bool narrow = ws::attn_narrow(n_q);
  const int64_t tiles = (n_keys + (narrow ? ws::kAttnNarrowN : ws::kAttnBlockN) - 1) /
                        (narrow ? ws::kAttnNarrowN : ws::kAttnBlockN);
  int64_t max_s = tiles / 4;
  if (max_s > kMaxSplits) max_s = kMaxSplits;
  if (max_s < 1) max_s = 1;
  if (narrow) {
    // The narrow kernel streams K/V at the memory's pace, one wave per item:
    // fill one round of resident waves and no more. A second round leaves
    // its few waves streaming alone at the end (40 heads over 244,772 keys:
    // 1,000 waves take 0.83 ms, 1,040 waves 1.01 ms).
    int64_t s = kNarrowSlots / items;
    if (s > max_s) s = max_s;
    return (int32_t)(s < 1 ? 1 : s);
  }
  const double t_tile_us = 1.7 * head_dim / 128.0;
  int32_t best = 1;
  double best_cost = 1e300;
  for (int64_t s = 1; s <= max_s; ++s) {
    const int64_t rounds = (items * s + kSlots - 1) / kSlots;
    const int64_t per = (tiles + s - 1) / s;
    double cost = (double)rounds * (double)(per + 2) * t_tile_us;
    if (s > 1) cost += (double)s * heads * n_q * (head_dim + 1) * 4.0 * 2.0 / 4.0e6;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = (int32_t)s;
    }
  }
  return best;
}

size_t lse_offset(int32_t heads, int32_t n_q, int32_t head_dim, int32_t n_splits) {
  const size_t o = (size_t)n_splits * heads * n_q * head_dim * sizeof(float);
  return (o + 255) & ~(size_t)255;
}

// Workspace: split partials [S][heads][n_q][D] floats and their log2-sum-
// exps [S][heads][n_q] (S > 1), then, for calls of more than WS_MAX_UNITS
// queries, room for a unit table of up to n_q non-empty units
// ([n + 1] row begins, [n] key ends), each region 256-byte aligned.
size_t table_offset(int32_t heads, int32_t n_q, int32_t head_dim, int32_t n_splits) {
  if (n_splits <= 1) return 0;
  const size_t e = lse_offset(heads, n_q, head_dim, n_splits) + (size_t)n_splits * heads * n_q * sizeof(float);
  return (e + 255) & ~(size_t)255;
}

size_t workspace_bytes(int32_t heads, int32_t n_q, int32_t head_dim, int32_t n_splits) {
  if (heads <= 0 || n_q <= 0 || head_dim <= 0 || n_splits <= 0) return 0;
  const size_t table = n_q > WS_MAX_UNITS ? (2 * (size_t)n_q + 1) * sizeof(int32_t) : 0;
  if (n_splits <= 1) return table;
  return table ? table_offset(heads, n_q, head_dim, n_splits) + table
               : lse_offset(heads, n_q, head_dim, n_splits) +
                     (size_t)n_splits * heads * n_q * sizeof(float);
}

// Bytes of workspace a call writes: its split partials, or, when more than
// WS_MAX_UNITS units hold queries, everything up to the end of its unit table.
size_t attn_need_bytes(int32_t heads, int32_t n_q, int32_t head_dim, int32_t splits,
                       int32_t n_live) {
  if (n_live > WS_MAX_UNITS)
    return table_offset(heads, n_q, head_dim, splits) + (2 * (size_t)n_live + 1) * sizeof(int32_t);
  if (splits <= 1) return 0;
  return lse_offset(heads, n_q, head_dim, splits) + (size_t)splits * heads * n_q * sizeof(float);
}

// ---- library-held scratch for callers that cannot allocate
//
// One array per GPU, alive until the process ends. In host code `scratch`
// names a host-side stand-in, never the device memory: its device address
// is looked up once per device (that device current) and only that address
// is passed to kernels.
static __device__ __align__(256) char scratch[WS_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

ws_status scratch_of_current_device(void** out) {
  int dev = -1;
  ws_status st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != WS_OK) return st;
  if (dev < 0 || dev >= kMaxDevices)
    return fail(WS_ERR_UNSUPPORTED, "device %d outside the %d the scratch table tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st != WS_OK) return st;
    if (!p) return fail(WS_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return WS_OK;
}

struct AttnPlan {
  ws::AttnArgs args;
  int32_t splits;
  std::vector<int> table;  // unit table to copy to args.unit_table before the pass
};

// Enqueue the unit-table copy (if any), then the split-KV pass.
ws_status launch_partial(const AttnPlan& plan, int32_t head_dim, hipStream_t s) {
  if (!plan.table.empty()) {
    ws_status st = hip_status(ws::launch_unit_table(const_cast<int*>(plan.args.unit_table),
                                                    plan.table.data(), (int)plan.table.size(), s),
                              "unit table launch");
    if (st != WS_OK) return st;
  }
  return hip_status(ws::launch_attn_partial(plan.args, head_dim, s), "attention launch");
}

// Validate a ws_block_causal_attn / ws_attn_partial call and fill the kernel
// arguments. Returns WS_OK with plan->splits == 0 for a no-op (n_q == 0).
ws_status plan_attn(const ws_kv_cache* cache, const void* q, int32_t n_q, const void* k_self,
                    const void* v_self, int32_t n_self, int32_t n_units,
                    const int32_t* q_unit_begin, const int32_t* unit_kend, float scale,
                    int32_t n_splits, void* out, void* workspace, size_t workspace_bytes_in,
                    AttnPlan* plan) {
  ws_status st = check_cache(cache);
  if (st != WS_OK) return st;
  if (n_q < 0) return fail(WS_ERR_SHAPE, "n_q %d < 0", n_q);
  if (n_self < 0) return fail(WS_ERR_SHAPE, "n_self %d < 0", n_self);
  if (n_units < 1) return fail(WS_ERR_SHAPE, "n_units %d < 1", n_units);
  if (!q_unit_begin || !unit_kend) return fail(WS_ERR_NULL, "unit table is NULL");
  if (q_unit_begin[0] != 0) return fail(WS_ERR_SHAPE, "q_unit_begin[0] = %d != 0", q_unit_begin[0]);
  for (int32_t u = 0; u < n_units; ++u)
    if (q_unit_begin[u + 1] < q_unit_begin[u])
      return fail(WS_ERR_SHAPE, "q_unit_begin decreases at unit %d", u);
  if (q_unit_begin[n_units] != n_q)
    return fail(WS_ERR_SHAPE, "q_unit_begin[%d] = %d != n_q %d", n_units, q_unit_begin[n_units], n_q);
  const int64_t n_keys = (int64_t)cache->len + n_self;
  if (n_keys > 0x7FFFFFFF - ws::kAttnBlockN) return fail(WS_ERR_SHAPE, "too many keys");
  for (int32_t u = 0; u < n_units; ++u) {
    if (unit_kend[u] < 1 || unit_kend[u] > n_keys)
      return fail(WS_ERR_SHAPE, "unit_kend[%d] = %d outside [1, %lld]", u, unit_kend[u],
                  (long long)n_keys);
    if (u > 0 && unit_kend[u] < unit_kend[u - 1])
      return fail(WS_ERR_SHAPE, "unit_kend decreases at unit %d", u);
  }
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(WS_ERR_SHAPE, "scale must be positive and finite");
  if (n_splits < 0 || n_splits > kMaxSplits)
    return fail(WS_ERR_SHAPE, "n_splits %d outside [0, %d]", n_splits, kMaxSplits);
  const int32_t d = cache->head_dim;
  const int32_t splits = n_splits ? n_splits : default_splits(cache->heads, n_q, d, n_keys);
  // units with at least one query row; the others change no row's keys
  int32_t n_live = 0;
  for (int32_t u = 0; u < n_units; ++u) n_live += q_unit_begin[u + 1] > q_unit_begin[u];
  if (n_q == 0) {
    plan->splits = 0;
    return WS_OK;
  }
  if (!q || !out) return fail(WS_ERR_NULL, "q or out is NULL");
  if (cache->len > 0 && (!cache->k || !cache->v)) return fail(WS_ERR_NULL, "cache buffers are NULL");
  if (n_self > 0 && (!k_self || !v_self)) return fail(WS_ERR_NULL, "k_self or v_self is NULL");
  if (!aligned16(q) || !aligned16(out) || !aligned16(cache->k) || !aligned16(cache->v) ||
      !aligned16(k_self) || !aligned16(v_self))
    return fail(WS_ERR_ALIGN, "a device pointer is not 16-byte aligned");
  const int64_t n_qtiles = ((int64_t)n_q + ws::kAttnBlockM - 1) / ws::kAttnBlockM;
  const int64_t items = (int64_t)cache->heads * n_qtiles * splits;
  if (items > 0x7FFFFFF0) return fail(WS_ERR_SHAPE, "too many work items");
  if (splits > 1 || n_live > WS_MAX_UNITS) {
    // what this call writes: the partials, and the unit table if it has one
    const size_t need =
        n_live > WS_MAX_UNITS
            ? table_offset(cache->heads, n_q, d, splits) + (2 * (size_t)n_live + 1) * sizeof(int32_t)
            : lse_offset(cache->heads, n_q, d, splits) + (size_t)splits * cache->heads * n_q * sizeof(float);
    if (!workspace) return fail(WS_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes_in < need)
      return fail(WS_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes_in, need);
    if (!aligned16(workspace)) return fail(WS_ERR_ALIGN, "workspace is not 16-byte aligned");
  }
  ws::AttnArgs& a = plan->args;
  memset(&a, 0, sizeof a);
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint16_t*>(cache->k);
  a.vc = static_cast<const uint16_t*>(cache->v);
  a.ks = static_cast<const uint16_t*>(k_self);
  a.vs = static_cast<const uint16_t*>(v_self);
  a.out = static_cast<uint16_t*>(out);
  if (splits > 1) {
    char* wsb = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<float*>(wsb);
    a.part_lse = reinterpret_cast<float*>(wsb + lse_offset(cache->heads, n_q, d, splits));
  }
  a.cache_head_stride = (int64_t)cache->capacity * d;
  a.heads = cache->heads;
  a.n_q = n_q;
  a.len = cache->len;
  a.n_self = n_self;
  a.n_splits = splits;
  a.n_qtiles = (int)n_qtiles;
  a.n_items = (int)items;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.n_units = n_live;
  plan->table.clear();
  if (n_live <= WS_MAX_UNITS) {
    int32_t i = 0;
    for (int32_t u = 0; u < n_units; ++u) {
      if (q_unit_begin[u + 1] == q_unit_begin[u]) continue;
      a.q_unit_begin[i] = q_unit_begin[u];
      a.unit_kend[i++] = unit_kend[u];
    }
    a.q_unit_begin[n_live] = n_q;
  } else {
    std::vector<int>& t = plan->table;
    t.resize(2 * (size_t)n_live + 1);
    int32_t i = 0;
    for (int32_t u = 0; u < n_units; ++u) {
      if (q_unit_begin[u + 1] == q_unit_begin[u]) continue;
      t[i] = q_unit_begin[u];
      t[n_live + 1 + i++] = unit_kend[u];
    }
    t[n_live] = n_q;
    a.unit_table = reinterpret_cast<const int*>(static_cast<char*>(workspace) +
                                                table_offset(cache->heads, n_q, d, splits));
  }
  plan->splits = splits;
  return WS_OK;
}

}  // namespace

extern "C" {

ws_status ws_kv_append_segments(ws_kv_cache* cache, const ws_kv_segment* segs, int32_t n_segs,
                                 void* stream) {
  g_last_error.clear();
  ws_status st = check_cache(cache);
  if (st != WS_OK) return st;
  if (!segs) return fail(WS_ERR_NULL, "segment table is NULL");
  if (n_segs < 1 || n_segs > WS_MAX_SEGMENTS)
    return fail(WS_ERR_SHAPE, "n_segs %d outside [1, %d]", n_segs, WS_MAX_SEGMENTS);
  int64_t total = 0;
  for (int32_t i = 0; i < n_segs; ++i) {
    const ws_kv_segment& g = segs[i];
    if (g.layout != WS_TOKEN_MAJOR && g.layout != WS_HEAD_MAJOR)
      return fail(WS_ERR_UNSUPPORTED, "segment %d: unknown source layout %d", i, g.layout);
    if (g.n_tok < 0) return fail(WS_ERR_SHAPE, "segment %d: n_tok %d < 0", i, g.n_tok);
    if (g.src_heads < 1 || g.head_begin < 0 || (int64_t)g.head_begin + cache->heads > g.src_heads)
      return fail(WS_ERR_SHAPE, "segment %d: head block [%d, %lld) outside the %d source heads", i,
                  g.head_begin, (long long)g.head_begin + cache->heads, g.src_heads);
    total += g.n_tok;
  }
  if ((int64_t)cache->len + total > cache->capacity)
    return fail(WS_ERR_CAPACITY, "len %d + %lld tokens > capacity %d", cache->len,
                (long long)total, cache->capacity);
  if (total == 0) return WS_OK;
  if (total * (cache->head_dim / 8) > 0x7FFFFFFF || cache->heads > 65535)
    return fail(WS_ERR_SHAPE, "append of %lld tokens x %d heads is too large for one launch",
                (long long)total, cache->heads);
  if (!cache->k || !cache->v) return fail(WS_ERR_NULL, "a cache buffer is NULL");
  if (!aligned16(cache->k) || !aligned16(cache->v))
    return fail(WS_ERR_ALIGN, "a cache buffer is not 16-byte aligned");
  ws::AppendArgs a;
  memset(&a, 0, sizeof a);
  for (int32_t i = 0; i < n_segs; ++i) {
    const ws_kv_segment& g = segs[i];
    if (g.n_tok == 0) continue;
    if (!g.k || !g.v) return fail(WS_ERR_NULL, "segment %d: a buffer is NULL", i);
    if (!aligned16(g.k) || !aligned16(g.v))
      return fail(WS_ERR_ALIGN, "segment %d: a buffer is not 16-byte aligned", i);
    ws::AppendSeg& s = a.seg[a.n_segs++];
    s.k = static_cast<const uint16_t*>(g.k);
    s.v = static_cast<const uint16_t*>(g.v);
    s.n_tok = g.n_tok;
    s.src_heads = g.src_heads;
    s.head_begin = g.head_begin;
    s.layout = g.layout;
    s.row0 = a.total_tok;
    a.total_tok += g.n_tok;
  }
  a.ck = static_cast<uint16_t*>(cache->k);
  a.cv = static_cast<uint16_t*>(cache->v);
  a.cache_head_stride = (int64_t)cache->capacity * cache->head_dim;
  a.len = cache->len;
  a.head_dim = cache->head_dim;
  a.log2_cpr = cache->head_dim == 128 ? 4 : 3;
  st = hip_status(ws::launch_kv_append(a, cache->heads, static_cast<hipStream_t>(stream)),
                  "kv_append launch");
  if (st == WS_OK) cache->len += (int32_t)total;
  return st;
}

ws_status ws_kv_append(ws_kv_cache* cache, const void* k_src, const void* v_src, int32_t n_tok,
                       int32_t src_heads, int32_t head_begin, int32_t layout, void* stream) {
  const ws_kv_segment g = {k_src, v_src, n_tok, src_heads, head_begin, layout};
  return ws_kv_append_segments(cache, &g, 1, stream);
}

int32_t ws_attn_default_splits(int32_t heads, int32_t n_q, int32_t head_dim, int64_t n_keys) {
  return default_splits(heads, n_q, head_dim, n_keys);
}

size_t ws_attn_workspace_bytes(int32_t heads, int32_t n_q, int32_t head_dim, int32_t n_splits) {
  return workspace_bytes(heads, n_q, head_dim, n_splits);
}

ws_status ws_attn_partial(const ws_kv_cache* cache, const void* q, int32_t n_q, const void* k_self,
                          const void* v_self, int32_t n_self, int32_t n_units,
                          const int32_t* q_unit_begin, const int32_t* unit_kend, float scale,
                          int32_t n_splits, void* out, void* workspace, size_t workspace_bytes_in,
                          void* stream) {
  g_last_error.clear();
  AttnPlan plan;
  ws_status st = plan_attn(cache, q, n_q, k_self, v_self, n_self, n_units, q_unit_begin, unit_kend,
                           scale, n_splits, out, workspace, workspace_bytes_in, &plan);
  if (st != WS_OK || plan.splits == 0) return st;
  return launch_partial(plan, cache->head_dim, static_cast<hipStream_t>(stream));
}

ws_status ws_attn_merge(int32_t heads, int32_t n_q, int32_t head_dim, int32_t n_splits,
                        const void* workspace, size_t workspace_bytes_in, void* out, void* stream) {
  g_last_error.clear();
  if (!head_dim_ok(head_dim)) return fail(WS_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", head_dim);
  if (heads < 1 || n_q < 0) return fail(WS_ERR_SHAPE, "heads %d / n_q %d invalid", heads, n_q);
  if (n_splits < 1 || n_splits > kMaxSplits)
    return fail(WS_ERR_SHAPE, "n_splits %d outside [1, %d]", n_splits, kMaxSplits);
  if (n_splits == 1 || n_q == 0) return WS_OK;
  if ((int64_t)heads * n_q > 0x7FFFFFFF) return fail(WS_ERR_SHAPE, "too many rows");
  const size_t need = workspace_bytes(heads, n_q, head_dim, n_splits);
  if (!workspace) return fail(WS_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes_in < need)
    return fail(WS_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes_in, need);
  if (!out) return fail(WS_ERR_NULL, "out is NULL");
  if (!aligned16(out) || !aligned16(workspace))
    return fail(WS_ERR_ALIGN, "a device pointer is not 16-byte aligned");
  const char* wsb = static_cast<const char*>(workspace);
  return hip_status(
      ws::launch_attn_merge(reinterpret_cast<const float*>(wsb),
                            reinterpret_cast<const float*>(wsb + lse_offset(heads, n_q, head_dim, n_splits)),
                            static_cast<uint16_t*>(out), heads, n_q, head_dim, n_splits,
                            static_cast<hipStream_t>(stream)),
      "merge launch");
}

ws_status ws_block_causal_attn(const ws_kv_cache* cache, const void* q, int32_t n_q,
                               const void* k_self, const void* v_self, int32_t n_self,
                               int32_t n_units, const int32_t* q_unit_begin,
                               const int32_t* unit_kend, float scale, int32_t n_splits, void* out,
                               void* workspace, size_t workspace_bytes_in, void* stream) {
  g_last_error.clear();
  AttnPlan plan;
  ws_status st = plan_attn(cache, q, n_q, k_self, v_self, n_self, n_units, q_unit_begin, unit_kend,
                           scale, n_splits, out, workspace, workspace_bytes_in, &plan);
  if (st != WS_OK || plan.splits == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_partial(plan, cache->head_dim, s);
  if (st != WS_OK || plan.splits == 1) return st;
  return hip_status(ws::launch_attn_merge(plan.args.part_o, plan.args.part_lse, plan.args.out,
                                          cache->heads, n_q, cache->head_dim, plan.splits, s),
                    "merge launch");
}

ws_status ws_block_causal_attn_noalloc(const ws_kv_cache* cache, const void* q, int32_t n_q,
                                       const void* k_self, const void* v_self, int32_t n_self,
                                       int32_t n_units, const int32_t* q_unit_begin,
                                       const int32_t* unit_kend, float scale, int32_t n_splits,
                                       void* out, void* stream) {
  g_last_error.clear();
  // Size the call against the scratch before touching the GPU: the default
  // split count is lowered until its partials fit; an explicit one that does
  // not fit is refused.
  int32_t splits = n_splits;
  if (cache && q_unit_begin && n_units >= 1 && n_q > 0 && n_splits >= 0 &&
      head_dim_ok(cache->head_dim) && cache->heads >= 1) {
    int32_t n_live = 0;
    for (int32_t u = 0; u < n_units; ++u) n_live += q_unit_begin[u + 1] > q_unit_begin[u];
    const int64_t n_keys = (int64_t)cache->len + (n_self > 0 ? n_self : 0);
    if (splits == 0) {
      splits = default_splits(cache->heads, n_q, cache->head_dim, n_keys);
      while (splits > 1 &&
             attn_need_bytes(cache->heads, n_q, cache->head_dim, splits, n_live) > WS_SCRATCH_BYTES)
        --splits;
    }
    const size_t need = attn_need_bytes(cache->heads, n_q, cache->head_dim, splits, n_live);
    if (need > WS_SCRATCH_BYTES)
      return fail(WS_ERR_WORKSPACE,
                  "the call needs %zu bytes of scratch; the library holds %zu per GPU "
                  "(use fewer splits or ws_block_causal_attn with a workspace)",
                  need, (size_t)WS_SCRATCH_BYTES);
  }
  AttnPlan plan;
  // validation first (also of the sizes above); the GPU is touched only for
  // a call that will launch
  ws_status st = plan_attn(cache, q, n_q, k_self, v_self, n_self, n_units, q_unit_begin, unit_kend,
                           scale, splits, out, nullptr, 0, &plan);
  if (st == WS_ERR_WORKSPACE) {
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != WS_OK) return st;
    g_last_error.clear();
    st = plan_attn(cache, q, n_q, k_self, v_self, n_self, n_units, q_unit_begin, unit_kend, scale,
                   splits, out, ws, WS_SCRATCH_BYTES, &plan);
  }
  if (st != WS_OK || plan.splits == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_partial(plan, cache->head_dim, s);
  if (st != WS_OK || plan.splits == 1) return st;
  return hip_status(ws::launch_attn_merge(plan.args.part_o, plan.args.part_lse, plan.args.out,
                                          cache->heads, n_q, cache->head_dim, plan.splits, s),
                    "merge launch");
}

ws_status ws_fm_euler_step(float* x, const void* v, int64_t n, float dt, void* stream) {
  g_last_error.clear();
  if (n < 0) return fail(WS_ERR_SHAPE, "n %lld < 0", (long long)n);
  if (!isfinite(dt)) return fail(WS_ERR_SHAPE, "dt is not finite");
  if (n == 0) return WS_OK;
  if (!x || !v) return fail(WS_ERR_NULL, "x or v is NULL");
  if (!aligned16(x) || !aligned16(v)) return fail(WS_ERR_ALIGN, "x or v is not 16-byte aligned");
  return hip_status(ws::launch_fm_euler(x, static_cast<const uint16_t*>(v), n, dt,
                                        static_cast<hipStream_t>(stream)),
                    "euler launch");
}

const char* ws_status_string(ws_status s) {
  // A C caller may pass any int; read the bits as an int so that a value
  // outside the enumerators is handled rather than loaded as the enum.
  static_assert(sizeof(ws_status) == sizeof(int), "ws_status is passed as an int");
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case WS_OK: return "ok";
    case WS_ERR_NULL: return "null pointer";
    case WS_ERR_SHAPE: return "invalid size or table";
    case WS_ERR_CAPACITY: return "cache capacity exceeded";
    case WS_ERR_ALIGN: return "misaligned pointer";
    case WS_ERR_UNSUPPORTED: return "unsupported configuration";
    case WS_ERR_WORKSPACE: return "workspace missing or too small";
    case WS_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* ws_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

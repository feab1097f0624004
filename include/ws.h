/*
 * ws.h -- C ABI of the cached block-causal denoising step for MI355X (gfx950).
 *
 * One performer GPU's hot path for one 160 ms streaming unit: write the
 * thinker's K/V slice into this GPU's pre-sharded cache, then, for every
 * denoise step, run block-causal attention of the unit's latent tokens over
 * the cached history plus the unit's own tokens and apply the flow-matching
 * Euler update.
 *
 * Pages cited (title, then section):
 *   [Summary]   "Wan-Streamer v0.2：更高分辨率，相同延迟 / Wan-Streamer v0.2:
 *               Higher Resolution, Same Latency" (paper.rainbus.top structured
 *               summary): 前置知识 (K/V缓存预分片, Thinker-Performer架构),
 *               核心方法, 方法步骤详情.
 *   [Abstract]  English abstract on chatpaper.ai.
 *   [TechSum]   "Technical Summary: Wan-Streamer v0.2" (gist.science, English):
 *               Methodology, "The Performer".
 *   [News]      "通义实验室发布 Wan-Streamer v0.2…" (remio.ai): section
 *               为什么端到端模型对级联式 AI 智能体构成挑战, and
 *               思考者与执行者的分工掩盖了更高分辨率的成本.
 *
 * Conventions for every call:
 *   - Device pointers are caller-owned, must point to device-accessible
 *     memory, and must be 16-byte aligned; tensors are dense (no strides
 *     other than the stated layouts). bf16 is IEEE binary16-brain (the top 16
 *     bits of a binary32), passed as raw 16-bit words.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on `stream`; none synchronises, none
 *     allocates device memory, and none keeps state between calls.
 *   - All arguments are validated on the host before anything is enqueued;
 *     on any error nothing is enqueued, caches are unchanged, and
 *     ws_last_error() describes the failure. Faults during asynchronous
 *     execution surface at the caller's next synchronisation.
 *   - Calls that write the same memory must be ordered by the caller
 *     (same stream, or events); the library uses no atomics.
 */
#ifndef WS_H
#define WS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ws_status {
  WS_OK = 0,
  WS_ERR_NULL = 1,         /* a required pointer is NULL                         */
  WS_ERR_SHAPE = 2,        /* a size, index or unit table is out of range        */
  WS_ERR_CAPACITY = 3,     /* an append would overflow the cache                 */
  WS_ERR_ALIGN = 4,        /* a device pointer is not 16-byte aligned            */
  WS_ERR_UNSUPPORTED = 5,  /* head_dim not 64/128, or an unknown source layout   */
  WS_ERR_WORKSPACE = 6,    /* workspace missing or smaller than required         */
  WS_ERR_HIP = 7           /* the HIP runtime refused a launch                   */
} ws_status;

/* Source layouts accepted by ws_kv_append. */
enum {
  WS_TOKEN_MAJOR = 0,      /* [n_tok][src_heads][head_dim]: a thinker slice       */
  WS_HEAD_MAJOR = 1        /* [src_heads][n_tok][head_dim]: head-sharded latents  */
};

/* Units with queries whose table travels in the launch arguments. A call with
   more keeps its unit table in the workspace (see ws_attn_workspace_bytes). */
#define WS_MAX_UNITS 64

/*
 * One GPU's pre-sharded, pre-allocated K/V cache ([Summary] 前置知识,
 * K/V缓存预分片; [TechSum] Methodology, "The Performer", K/V handling): the
 * GPU keeps the full history of its own contiguous block of heads, so the
 * cache is head-major. The struct lives in host memory and is owned by the
 * caller; k and v are device buffers of bf16[heads][capacity][head_dim].
 * `len` counts valid rows and is advanced only by a successful ws_kv_append.
 */
typedef struct ws_kv_cache {
  void*   k;
  void*   v;
  int32_t heads;       /* Hr: heads held by this GPU (>= 1)                 */
  int32_t head_dim;    /* D: 64 or 128                                      */
  int32_t capacity;    /* token slots per head (>= 0)                       */
  int32_t len;         /* valid rows, 0 <= len <= capacity                  */
} ws_kv_cache;

/*
 * ws_kv_append -- write this GPU's part of an incoming K/V slice straight into
 * its cache positions ([Summary] 前置知识, K/V缓存预分片 and 方法步骤详情;
 * [Abstract]): a rank stores its own head block of every new slice in a
 * cache that was split and allocated ahead of time, so the write itself
 * moves nothing between GPUs.
 *
 *   For h in [0, cache->heads), t in [0, n_tok):
 *     cache->k[h][cache->len + t][:] = k_src[t][head_begin + h][:]   (WS_TOKEN_MAJOR)
 *                                   = k_src[head_begin + h][t][:]    (WS_HEAD_MAJOR)
 *   and the same for v; then cache->len += n_tok. A bit copy: no rounding.
 *
 *   k_src, v_src: device bf16 buffers in `layout`, src_heads heads.
 *   n_tok >= 0 (0 is a no-op); 0 <= head_begin, head_begin + heads <= src_heads.
 * Errors: WS_ERR_NULL (cache or a buffer NULL while n_tok > 0), WS_ERR_SHAPE
 * (bad heads/head_begin/n_tok/len), WS_ERR_CAPACITY (len + n_tok > capacity),
 * WS_ERR_UNSUPPORTED (head_dim or layout), WS_ERR_ALIGN, WS_ERR_HIP. On error
 * nothing is written and len is unchanged.
 */
ws_status ws_kv_append(ws_kv_cache* cache, const void* k_src, const void* v_src,
                       int32_t n_tok, int32_t src_heads, int32_t head_begin,
                       int32_t layout, void* stream);

/*
 * ws_kv_append_segments -- ws_kv_append of up to WS_MAX_SEGMENTS sources into
 * consecutive cache rows with one launch: segment i's tokens land right after
 * segment i-1's. A unit's end is two such writes ([Summary] 方法步骤详情: the
 * performer keeps what it generated as history, and the thinker's next slice
 * follows it): the unit's committed latents (head-major, already on this GPU)
 * and the next unit's slice (token-major); as one launch they are one
 * 952-token write at the v0.2 sizes instead of a 920- and a 32-token one.
 *   Each segment follows ws_kv_append's rules (layout, n_tok >= 0, head
 *   block inside its src_heads); segments with n_tok == 0 are skipped and may
 *   have NULL buffers. len + sum(n_tok) <= capacity.
 * Errors as ws_kv_append, plus WS_ERR_NULL (segs NULL) and WS_ERR_SHAPE
 * (n_segs outside [1, WS_MAX_SEGMENTS]). All or nothing: on error nothing is
 * written and len is unchanged.
 */
#define WS_MAX_SEGMENTS 4
typedef struct ws_kv_segment {
  const void* k;        /* device bf16 source in `layout`                   */
  const void* v;
  int32_t n_tok;        /* tokens of this segment (>= 0)                    */
  int32_t src_heads;    /* heads in the source                              */
  int32_t head_begin;   /* first source head of this cache's block          */
  int32_t layout;       /* WS_TOKEN_MAJOR or WS_HEAD_MAJOR                  */
} ws_kv_segment;
ws_status ws_kv_append_segments(ws_kv_cache* cache, const ws_kv_segment* segs,
                                int32_t n_segs, void* stream);

/*
 * Split-KV planning. The key range of each query tile is cut into n_splits
 * contiguous chunks processed by separate workgroups and merged by
 * log-sum-exp weights. ws_attn_default_splits returns the library's choice
 * (>= 1) for a call with these sizes; ws_attn_workspace_bytes returns the
 * workspace a call with n_splits needs: the split partials when n_splits >
 * 1, plus, when n_q > WS_MAX_UNITS, room for a unit table of up to n_q units
 * (a call with more than WS_MAX_UNITS units holding queries copies its table
 * there with one small kernel launch per 896 entries). A call with one split
 * and at most WS_MAX_UNITS units with queries needs none. Both are pure host
 * functions. Non-positive sizes give 1 and 0.
 */
int32_t ws_attn_default_splits(int32_t heads, int32_t n_q, int32_t head_dim,
                               int64_t n_keys);
size_t ws_attn_workspace_bytes(int32_t heads, int32_t n_q, int32_t head_dim,
                               int32_t n_splits);

/*
 * ws_block_causal_attn -- block-causal attention of the current unit's latent
 * queries over the cached history plus the unit's own tokens ([News] 为什么
 * 端到端模型…: each streaming block may only use information available when
 * it is produced, so no output depends on later frames; [Summary] 方法步骤详情:
 * each rank attends with its local full-history cache).
 *
 * Keys and values of head h are the concatenation
 *     K_h = cache->k[h][0 : cache->len]  ++  k_self[h][0 : n_self]
 * (likewise V). Query rows are grouped into n_units consecutive units: rows
 * [q_unit_begin[u], q_unit_begin[u+1]) belong to unit u and see exactly the
 * first unit_kend[u] keys of K_h (block-causal: a unit sees every key of its
 * own and earlier units, bidirectionally within its own unit). For each head
 * h and query row i of unit u:
 *     out[h][i] = sum_{j < kend} softmax_j(scale * <q[h][i], K_h[j]>) * V_h[j]
 * with bf16 inputs, fp32 accumulation and softmax, and out rounded to bf16
 * (nearest-even).
 *
 *   q:   device bf16 [heads][n_q][head_dim]   (heads = cache->heads)
 *   k_self, v_self: device bf16 [heads][n_self][head_dim]; may be NULL if n_self == 0
 *   n_units >= 1; q_unit_begin: host int32[n_units + 1],
 *     q_unit_begin[0] == 0, non-decreasing, q_unit_begin[n_units] == n_q;
 *   unit_kend: host int32[n_units], non-decreasing, 1 <= unit_kend[u] <=
 *     cache->len + n_self.
 *   The streaming step is n_units = 1, unit_kend = {len + n_self}.
 *   scale > 0 and finite (normally 1/sqrt(head_dim)).
 *   n_splits: 0 = ws_attn_default_splits(heads, n_q, head_dim, len + n_self);
 *     otherwise 1..256.
 *   out: device bf16 [heads][n_q][head_dim].
 *   workspace: device buffer of >= ws_attn_workspace_bytes(...) bytes when
 *     the split count used is > 1 or more than WS_MAX_UNITS units hold
 *     queries (NULL allowed otherwise); overwritten.
 * Errors: WS_ERR_NULL, WS_ERR_SHAPE, WS_ERR_UNSUPPORTED (head_dim),
 * WS_ERR_WORKSPACE, WS_ERR_ALIGN, WS_ERR_HIP. n_q == 0 is a no-op.
 */
ws_status ws_block_causal_attn(const ws_kv_cache* cache,
                               const void* q, int32_t n_q,
                               const void* k_self, const void* v_self, int32_t n_self,
                               int32_t n_units, const int32_t* q_unit_begin,
                               const int32_t* unit_kend, float scale, int32_t n_splits,
                               void* out, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * The two launches of ws_block_causal_attn, exposed separately so a caller
 * can time or order them (same arguments and rules as above).
 * ws_attn_partial runs the split-KV pass: with one split it writes `out`
 * directly; otherwise it writes per-split partial outputs and log-sum-exps
 * into `workspace`. ws_attn_merge combines the partials of a previous
 * ws_attn_partial with the same heads, n_q, head_dim and n_splits into `out`
 * (a no-op when n_splits == 1). ws_block_causal_attn == partial then merge.
 */
ws_status ws_attn_partial(const ws_kv_cache* cache,
                          const void* q, int32_t n_q,
                          const void* k_self, const void* v_self, int32_t n_self,
                          int32_t n_units, const int32_t* q_unit_begin,
                          const int32_t* unit_kend, float scale, int32_t n_splits,
                          void* out, void* workspace, size_t workspace_bytes,
                          void* stream);
ws_status ws_attn_merge(int32_t heads, int32_t n_q, int32_t head_dim, int32_t n_splits,
                        const void* workspace, size_t workspace_bytes, void* out,
                        void* stream);

/*
 * ws_block_causal_attn_noalloc -- ws_block_causal_attn for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments without the
 * workspace. Its split partials and unit table live in scratch memory the
 * library holds, WS_SCRATCH_BYTES per GPU (a static device array, alive
 * until the process ends); the call allocates nothing.
 *   - n_splits == 0: the default split count, lowered until the partials fit
 *     the scratch; an explicit n_splits whose partials (or unit table) do not
 *     fit is refused with WS_ERR_WORKSPACE before anything is enqueued.
 *   - The scratch of a GPU is shared by every call on it and keeps the last
 *     call's contents: two such calls that can run at the same time on one
 *     GPU (different streams without ordering) race and give wrong results.
 *     Calls on one stream, or ordered by events, are safe.
 *   - The calling thread's current device must be the device of `stream`
 *     (the scratch address is looked up per current device, once).
 * Results equal ws_block_causal_attn's with the same split count.
 */
#define WS_SCRATCH_BYTES (32u << 20)
ws_status ws_block_causal_attn_noalloc(const ws_kv_cache* cache,
                                       const void* q, int32_t n_q,
                                       const void* k_self, const void* v_self, int32_t n_self,
                                       int32_t n_units, const int32_t* q_unit_begin,
                                       const int32_t* unit_kend, float scale, int32_t n_splits,
                                       void* out, void* stream);

/*
 * ws_fm_euler_step -- one explicit Euler step of flow-matching latent
 * generation ([Summary] 核心方法 and Thinker-Performer架构: the performer
 * generates the next unit's latent by flow matching):
 *     x[i] = fp32( x[i] + dt * float(v[i]) ),  i in [0, n)
 * computed as one fused multiply-add (a single rounding to nearest-even).
 *   x: device float32[n], updated in place; v: device bf16[n]; n >= 0;
 *   dt finite.
 * Errors: WS_ERR_NULL, WS_ERR_SHAPE (n < 0 or dt not finite), WS_ERR_ALIGN,
 * WS_ERR_HIP. n == 0 is a no-op.
 */
ws_status ws_fm_euler_step(float* x, const void* v, int64_t n, float dt, void* stream);

/* Static text for a status code ("unknown status" for any other value). */
const char* ws_status_string(ws_status s);

/* Detail of the last failing call on this thread ("" if none). Valid until
   the next library call on the same thread. */
const char* ws_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WS_H */

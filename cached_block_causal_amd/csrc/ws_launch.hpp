// Host-side launchers of the gfx950 kernels (internal to libws).
// Arguments are validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ws.h"

namespace ws {

// Cache append: bit copies of one head block of up to kAppendMaxSegs source
// segments into consecutive cache rows [len, len + total_tok).
constexpr int kAppendMaxSegs = WS_MAX_SEGMENTS;
struct AppendSeg {
  const uint16_t* k;
  const uint16_t* v;
  int n_tok, src_heads, head_begin, layout;
  int row0;                 // first token of this segment within the call
  int blk0;                 // first block of this segment (set by the launcher)
};
struct AppendArgs {
  uint16_t* ck;
  uint16_t* cv;
  int64_t cache_head_stride;  // capacity * D (elements)
  int len, head_dim, log2_cpr, total_tok, n_segs;
  AppendSeg seg[kAppendMaxSegs];
};
hipError_t launch_kv_append(const AppendArgs& a, int heads, hipStream_t stream);

// Euler update x = fma(dt, v, x).
hipError_t launch_fm_euler(float* x, const uint16_t* v, int64_t n, float dt, hipStream_t stream);

// Arguments of the split-KV attention pass (passed by value to the kernel).
struct AttnArgs {
  const uint16_t* q;        // [heads][n_q][D]
  const uint16_t* kc;       // cache K [heads][capacity][D]
  const uint16_t* vc;       // cache V
  const uint16_t* ks;       // own-token K [heads][n_self][D]
  const uint16_t* vs;       // own-token V
  uint16_t* out;            // [heads][n_q][D]              (one split)
  float* part_o;            // [splits][heads][n_q][D]      (several splits)
  float* part_lse;          // [splits][heads][n_q]
  int64_t cache_head_stride;  // capacity * D (elements)
  int heads, n_q, len, n_self;
  int n_splits, n_qtiles, n_items;
  float scale_log2;         // softmax scale * log2(e)
  // Units with at least one query row (empty units change no row's keys).
  // Up to WS_MAX_UNITS of them travel here; a call with more keeps its table
  // in device memory: unit_table = [n_units + 1 row begins][n_units key ends].
  int n_units;
  int q_unit_begin[WS_MAX_UNITS + 1];
  int unit_kend[WS_MAX_UNITS];
  const int* unit_table;
};

// Copy a host int table to device memory with kernel launches whose
// arguments carry the values (no host-side staging buffer, and the same under
// graph capture).
hipError_t launch_unit_table(int* dst, const int* vals, int n, hipStream_t stream);

// Rows of queries one workgroup of the split-KV pass covers.
constexpr int kAttnBlockM = 128;
// Keys per LDS tile.
constexpr int kAttnBlockN = 64;
// Calls whose queries all fit one 32-row block run the narrow kernel: one
// wave per (head, split) over 32-key tiles.
constexpr int kAttnNarrowN = 32;
inline bool attn_narrow(int n_q) { return n_q <= 32; }

hipError_t launch_attn_partial(const AttnArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_attn_merge(const float* part_o, const float* part_lse, uint16_t* out,
                             int heads, int n_q, int head_dim, int n_splits,
                             hipStream_t stream);

}  // namespace ws

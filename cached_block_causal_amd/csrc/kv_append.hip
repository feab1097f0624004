// Cache append: this GPU's head block of an incoming K/V slice is copied
// bit for bit into its pre-allocated, head-major cache rows [len, len + n).
// ("Wan-Streamer v0.2: Higher Resolution, Same Latency" structured summary,
// 前置知识 / K/V缓存预分片: a performer rank writes a new slice straight into
// its own pre-split cache positions; nothing else moves.)
//
// Pure data movement, bound by HBM: 2 * n * heads * D * 2 bytes read and the
// same written per call (K and V). One thread moves one 16-byte chunk; chunks
// are numbered with the D/8 chunks of a row fastest, then tokens, then heads,
// so consecutive lanes write consecutive addresses of a head's cache rows and
// read whole 128/256-byte rows of the source.
#include "ws_device.hpp"
#include "ws_launch.hpp"

namespace ws {

__global__ __launch_bounds__(256) void kv_append_kernel(
    uint16_t* __restrict__ ck, uint16_t* __restrict__ cv,
    const uint16_t* __restrict__ sk, const uint16_t* __restrict__ sv,
    int head_dim, int64_t cache_head_stride, int len, int n_tok, int src_heads,
    int head_begin, int layout, int64_t total_chunks) {
  // blockIdx.y selects K (0) or V (1): one launch moves both.
  uint16_t* __restrict__ dst = blockIdx.y == 0 ? ck : cv;
  const uint16_t* __restrict__ src = blockIdx.y == 0 ? sk : sv;
  const int cpr = head_dim >> 3;  // 16-byte chunks per row
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_chunks; i += stride) {
    const int c = (int)(i % cpr);
    const int64_t rest = i / cpr;
    const int t = (int)(rest % n_tok);
    const int h = (int)(rest / n_tok);
    const int64_t src_row = layout == WS_TOKEN_MAJOR
                                ? (int64_t)t * src_heads + head_begin + h
                                : (int64_t)(head_begin + h) * n_tok + t;
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + src_row * head_dim + c * 8);
    *reinterpret_cast<u32x4*>(dst + h * cache_head_stride + (int64_t)(len + t) * head_dim + c * 8) = v;
  }
}

hipError_t launch_kv_append(uint16_t* ck, uint16_t* cv, const uint16_t* sk, const uint16_t* sv,
                            int heads, int head_dim, int capacity, int len, int n_tok,
                            int src_heads, int head_begin, int layout, hipStream_t stream) {
  const int64_t total = (int64_t)heads * n_tok * (head_dim / 8);
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 8192) blocks = 8192;  // grid-stride beyond ~32 blocks per CU
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks, 2), dim3(threads), 0, stream,
                     ck, cv, sk, sv, head_dim, (int64_t)capacity * head_dim, len, n_tok,
                     src_heads, head_begin, layout, total);
  return hipGetLastError();
}

}  // namespace ws

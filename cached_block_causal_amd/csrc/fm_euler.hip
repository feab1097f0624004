// Flow-matching Euler update x <- x + dt * v ("Wan-Streamer v0.2: Higher
// Resolution, Same Latency" structured summary, 核心方法 and
// Thinker-Performer架构: the performer produces the next unit's latent by
// flow matching; one explicit Euler step per denoise step).
//
// x is the float32 latent share, v the bf16 velocity. Each element is one
// fused multiply-add, so the result is x + dt*v rounded once to nearest-even.
// Bound by HBM: 4 + 4 + 2 = 10 bytes per element. Each thread handles two
// groups of 8 elements per iteration (16-byte accesses, loads issued first),
// all non-temporal: between two steps the attention streams far more than the
// caches hold, so nothing of x or v would still be cached.
#include "ws_device.hpp"
#include "ws_launch.hpp"

namespace ws {

__device__ __forceinline__ void euler8(f32x4& a, f32x4& b, u32x4 w, float dt) {
  a[0] = __builtin_fmaf(dt, bf16_lo(w[0]), a[0]);
  a[1] = __builtin_fmaf(dt, bf16_hi(w[0]), a[1]);
  a[2] = __builtin_fmaf(dt, bf16_lo(w[1]), a[2]);
  a[3] = __builtin_fmaf(dt, bf16_hi(w[1]), a[3]);
  b[0] = __builtin_fmaf(dt, bf16_lo(w[2]), b[0]);
  b[1] = __builtin_fmaf(dt, bf16_hi(w[2]), b[1]);
  b[2] = __builtin_fmaf(dt, bf16_lo(w[3]), b[2]);
  b[3] = __builtin_fmaf(dt, bf16_hi(w[3]), b[3]);
}

constexpr int kEulerUnroll = 2;  // groups of 8 elements in flight per thread

__global__ __launch_bounds__(256) void fm_euler_kernel(float* __restrict__ x,
                                                       const uint16_t* __restrict__ v,
                                                       int64_t n, float dt) {
  const int64_t n8 = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * kEulerUnroll;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x * kEulerUnroll + threadIdx.x; i0 < n8;
       i0 += stride) {
    f32x4 a[kEulerUnroll], b[kEulerUnroll];
    u32x4 w[kEulerUnroll];
#pragma unroll
    for (int j = 0; j < kEulerUnroll; ++j) {  // loads first
      const int64_t i = i0 + (int64_t)j * blockDim.x;
      if (i < n8) {
        const f32x4* xp = reinterpret_cast<const f32x4*>(x + i * 8);
        a[j] = __builtin_nontemporal_load(xp);
        b[j] = __builtin_nontemporal_load(xp + 1);
        w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + i * 8));
      }
    }
#pragma unroll
    for (int j = 0; j < kEulerUnroll; ++j) {
      const int64_t i = i0 + (int64_t)j * blockDim.x;
      if (i < n8) {
        euler8(a[j], b[j], w[j], dt);
        f32x4* xp = reinterpret_cast<f32x4*>(x + i * 8);
        __builtin_nontemporal_store(a[j], xp);
        __builtin_nontemporal_store(b[j], xp + 1);
      }
    }
  }
  // the last n % 8 elements
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t i = (n8 << 3) + threadIdx.x;
    const uint32_t w = v[i];
    x[i] = __builtin_fmaf(dt, bf16_lo(w), x[i]);
  }
}

hipError_t launch_fm_euler(float* x, const uint16_t* v, int64_t n, float dt, hipStream_t stream) {
  const int threads = 256;
  int64_t blocks = ((n >> 3) + threads * kEulerUnroll - 1) / (threads * kEulerUnroll);
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fm_euler_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, x, v, n, dt);
  return hipGetLastError();
}

}  // namespace ws

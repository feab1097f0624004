/*
 * c_abi_demo.c -- the library used from plain C99 through include/ws.h, with
 * the HIP runtime for device memory and no other dependency.
 *
 * It runs the three hand-derived cases of tests/golden/ on the GPU:
 *   1. block-causal attention of two units with scale ln 3, whose softmax
 *      weights are exact rationals ("通义实验室发布 Wan-Streamer v0.2…",
 *      为什么端到端模型对级联式 AI 智能体构成挑战: a unit sees its own and
 *      earlier units' keys);
 *   2. a head-block append of a token-major slice at a non-zero length
 *      ("Wan-Streamer v0.2：更高分辨率，相同延迟", 前置知识 K/V缓存预分片);
 *   3. four flow-matching Euler steps with dt = 1/4 (same page, 核心方法);
 * and one call the library must refuse before launching anything. head_dim is
 * 64, the fixtures' two dimensions padded with zeros. Prints "c_abi_demo ok"
 * and exits 0 when every check holds.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "ws.h"

#define D 64

static uint16_t bf16_exact(float f) { /* the values used are exact in bf16 */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static double from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
      return 1;                                                                \
    }                                                                          \
  } while (0)

#define WS_OK_(x)                                                              \
  do {                                                                         \
    ws_status s_ = (x);                                                        \
    if (s_ != WS_OK) {                                                         \
      fprintf(stderr, "%s: %s (%s)\n", #x, ws_status_string(s_), ws_last_error()); \
      return 1;                                                                \
    }                                                                          \
  } while (0)

static int attention_case(void) {
  enum { NQ = 3, NK = 3, CAP = 8 };
  const float q2[NQ][2] = {{1, 0}, {1, 0}, {0, 1}};
  const float k2[NK][2] = {{0, 1}, {1, 0}, {1, 0}};
  const float v2[NK][2] = {{0.25f, -0.125f}, {0.75f, 0.375f}, {-0.5f, 1.25f}};
  const double want[NQ][2] = {{5.0 / 8, 1.0 / 4}, {1.0 / 7, 19.0 / 28}, {1.0 / 5, 1.0 / 4}};
  uint16_t hq[NQ * D] = {0}, hk[NK * D] = {0}, hv[NK * D] = {0}, hout[NQ * D];
  for (int i = 0; i < NQ; ++i)
    for (int d = 0; d < 2; ++d) hq[i * D + d] = bf16_exact(q2[i][d]);
  for (int j = 0; j < NK; ++j)
    for (int d = 0; d < 2; ++d) {
      hk[j * D + d] = bf16_exact(k2[j][d]);
      hv[j * D + d] = bf16_exact(v2[j][d]);
    }
  void *ck, *cv, *dq, *dk, *dv, *dout, *work;
  const size_t work_bytes = ws_attn_workspace_bytes(1, NQ, D, 2);
  HIP_OK(hipMalloc(&ck, CAP * D * 2));
  HIP_OK(hipMalloc(&cv, CAP * D * 2));
  HIP_OK(hipMalloc(&dq, sizeof hq));
  HIP_OK(hipMalloc(&dk, sizeof hk));
  HIP_OK(hipMalloc(&dv, sizeof hv));
  HIP_OK(hipMalloc(&dout, sizeof hout));
  HIP_OK(hipMalloc(&work, work_bytes));
  HIP_OK(hipMemcpy(dq, hq, sizeof hq, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, hk, sizeof hk, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, hv, sizeof hv, hipMemcpyHostToDevice));
  ws_kv_cache cache = {ck, cv, 1, D, CAP, 0};
  WS_OK_(ws_kv_append(&cache, dk, dv, NK, 1, 0, WS_HEAD_MAJOR, NULL));
  /* unit 0: query row 0 sees keys [0, 2); unit 1: rows 1-2 see keys [0, 3) */
  const int32_t q_unit_begin[3] = {0, 1, 3};
  const int32_t unit_kend[2] = {2, 3};
  for (int32_t splits = 1; splits <= 2; ++splits) {
    WS_OK_(ws_block_causal_attn(&cache, dq, NQ, NULL, NULL, 0, 2, q_unit_begin, unit_kend,
                                logf(3.0f), splits, dout, work, work_bytes, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(hout, dout, sizeof hout, hipMemcpyDeviceToHost));
    for (int i = 0; i < NQ; ++i)
      for (int d = 0; d < D; ++d) {
        const double w = d < 2 ? want[i][d] : 0.0;
        if (fabs(from_bf16(hout[i * D + d]) - w) > 2e-2) {
          fprintf(stderr, "attention, %d splits: out[%d][%d] = %g, want %g\n", (int)splits, i,
                  d, from_bf16(hout[i * D + d]), w);
          return 1;
        }
      }
  }
  /* a unit table whose key ends decrease is refused, and nothing runs */
  const int32_t bad_kend[2] = {3, 2};
  if (ws_block_causal_attn(&cache, dq, NQ, NULL, NULL, 0, 2, q_unit_begin, bad_kend, 1.0f, 1,
                           dout, NULL, 0, NULL) != WS_ERR_SHAPE) {
    fprintf(stderr, "a decreasing unit_kend was not refused\n");
    return 1;
  }
  HIP_OK(hipFree(ck));
  HIP_OK(hipFree(cv));
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(work));
  return 0;
}

static int append_case(void) {
  enum { HS = 3, HR = 2, CAP = 4, N = 2 };
  const float k2[N][HS][2] = {{{1, 2}, {3, 4}, {5, 6}}, {{7, 8}, {-1, -2}, {0.5f, 0.25f}}};
  uint16_t pre[HR * D], slice[N * HS * D] = {0}, got[HR * CAP * D];
  for (int i = 0; i < HR * D; ++i) pre[i] = bf16_exact(9.0f);  /* one sentinel token */
  for (int t = 0; t < N; ++t)
    for (int h = 0; h < HS; ++h)
      for (int d = 0; d < 2; ++d) slice[(t * HS + h) * D + d] = bf16_exact(k2[t][h][d]);
  void *ck, *cv, *dpre, *dsl;
  HIP_OK(hipMalloc(&ck, sizeof got));
  HIP_OK(hipMalloc(&cv, sizeof got));
  HIP_OK(hipMalloc(&dpre, sizeof pre));
  HIP_OK(hipMalloc(&dsl, sizeof slice));
  HIP_OK(hipMemset(ck, 0x41, sizeof got));  /* 0x4141: a finite sentinel pattern */
  HIP_OK(hipMemcpy(dpre, pre, sizeof pre, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dsl, slice, sizeof slice, hipMemcpyHostToDevice));
  ws_kv_cache cache = {ck, cv, HR, D, CAP, 0};
  WS_OK_(ws_kv_append(&cache, dpre, dpre, 1, HR, 0, WS_TOKEN_MAJOR, NULL));
  WS_OK_(ws_kv_append(&cache, dsl, dsl, N, HS, 1, WS_TOKEN_MAJOR, NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(got, ck, sizeof got, hipMemcpyDeviceToHost));
  if (cache.len != 3) {
    fprintf(stderr, "append: len %d, want 3\n", (int)cache.len);
    return 1;
  }
  for (int h = 0; h < HR; ++h)
    for (int r = 0; r < CAP; ++r)
      for (int d = 0; d < D; ++d) {
        uint16_t want;
        if (r == 0) want = bf16_exact(9.0f);
        else if (r <= N) want = d < 2 ? bf16_exact(k2[r - 1][1 + h][d]) : 0;
        else want = 0x4141;
        if (got[(h * CAP + r) * D + d] != want) {
          fprintf(stderr, "append: cache[%d][%d][%d] = 0x%04x, want 0x%04x\n", h, r, d,
                  got[(h * CAP + r) * D + d], want);
          return 1;
        }
      }
  /* one token too many is refused and leaves len unchanged */
  if (ws_kv_append(&cache, dsl, dsl, N, HS, 1, WS_TOKEN_MAJOR, NULL) != WS_ERR_CAPACITY ||
      cache.len != 3) {
    fprintf(stderr, "append past capacity was not refused\n");
    return 1;
  }
  HIP_OK(hipFree(ck));
  HIP_OK(hipFree(cv));
  HIP_OK(hipFree(dpre));
  HIP_OK(hipFree(dsl));
  return 0;
}

static int euler_case(void) {
  float x[4] = {1.0f, 0.5f, -2.0f, 0.0f};
  const float v[4][4] = {{1, -4, 8, 0.25f}, {2, 4, 8, -0.5f}, {-1, -4, 8, 0.75f}, {0.5f, 4, 8, -1}};
  const float want[4] = {1.625f, 0.5f, 6.0f, -0.125f};
  uint16_t hv[4][8] = {{0}};  /* one 16-byte row per step: every v is aligned */
  for (int s = 0; s < 4; ++s)
    for (int i = 0; i < 4; ++i) hv[s][i] = bf16_exact(v[s][i]);
  void *dx, *dv;
  HIP_OK(hipMalloc(&dx, sizeof x));
  HIP_OK(hipMalloc(&dv, sizeof hv));
  HIP_OK(hipMemcpy(dx, x, sizeof x, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, hv, sizeof hv, hipMemcpyHostToDevice));
  for (int s = 0; s < 4; ++s)
    WS_OK_(ws_fm_euler_step((float*)dx, (const uint16_t*)dv + 8 * s, 4, 0.25f, NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(x, dx, sizeof x, hipMemcpyDeviceToHost));
  for (int i = 0; i < 4; ++i)
    if (x[i] != want[i]) {
      fprintf(stderr, "euler: x[%d] = %g, want %g\n", i, x[i], want[i]);
      return 1;
    }
  HIP_OK(hipFree(dx));
  HIP_OK(hipFree(dv));
  return 0;
}

int main(void) {
  if (attention_case() || append_case() || euler_case()) return 1;
  printf("c_abi_demo ok\n");
  return 0;
}

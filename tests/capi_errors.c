/*
 * Host-only exercise of the C ABI's validation and planning code, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_capi_host.py.
 * Every call here is refused before any HIP call (device pointers are fake
 * addresses that are never dereferenced), or is a pure host function. Exits
 * non-zero on the first unexpected status; the sanitizers abort on any
 * invalid memory access or undefined behaviour in the library's host code.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ws.h"

#define FAKE ((void*)(uintptr_t)0x7F0000000000ull)
#define FAKE2 ((void*)(uintptr_t)0x7F0000100000ull)

static int fails = 0;

static void expect(const char* what, ws_status got, ws_status want) {
  if (got != want) {
    fprintf(stderr, "%s: got %d (%s), want %d\n", what, (int)got, ws_last_error(), (int)want);
    ++fails;
  } else if (want != WS_OK && ws_last_error()[0] == '\0') {
    fprintf(stderr, "%s: no error text\n", what);
    ++fails;
  }
}

int main(void) {
  ws_kv_cache c = {FAKE, FAKE2, 2, 128, 100, 10};
  /* append */
  expect("append null cache", ws_kv_append(NULL, FAKE, FAKE, 5, 4, 0, WS_TOKEN_MAJOR, NULL), WS_ERR_NULL);
  expect("append null src", ws_kv_append(&c, NULL, FAKE, 5, 4, 0, WS_TOKEN_MAJOR, NULL), WS_ERR_NULL);
  expect("append overflow", ws_kv_append(&c, FAKE, FAKE, 91, 4, 0, WS_TOKEN_MAJOR, NULL), WS_ERR_CAPACITY);
  expect("append head range", ws_kv_append(&c, FAKE, FAKE, 5, 4, 3, WS_TOKEN_MAJOR, NULL), WS_ERR_SHAPE);
  expect("append layout", ws_kv_append(&c, FAKE, FAKE, 5, 4, 0, 7, NULL), WS_ERR_UNSUPPORTED);
  expect("append align", ws_kv_append(&c, (char*)FAKE + 2, FAKE, 5, 4, 0, WS_TOKEN_MAJOR, NULL), WS_ERR_ALIGN);
  expect("append negative", ws_kv_append(&c, FAKE, FAKE, -1, 4, 0, WS_TOKEN_MAJOR, NULL), WS_ERR_SHAPE);
  if (c.len != 10) { fprintf(stderr, "len changed on error\n"); ++fails; }
  ws_kv_cache bad = c;
  bad.head_dim = 96;
  expect("append head_dim", ws_kv_append(&bad, FAKE, FAKE, 5, 4, 0, WS_TOKEN_MAJOR, NULL), WS_ERR_UNSUPPORTED);
  bad = c;
  bad.len = 101;
  expect("append len > capacity", ws_kv_append(&bad, FAKE, FAKE, 1, 4, 0, WS_TOKEN_MAJOR, NULL), WS_ERR_SHAPE);

  /* attention */
  int32_t qb[WS_MAX_UNITS + 2], ke[WS_MAX_UNITS + 1];
  qb[0] = 0; qb[1] = 8; ke[0] = 12;
  expect("attn null q", ws_block_causal_attn(&c, NULL, 8, FAKE, FAKE, 2, 1, qb, ke, 0.1f, 1, FAKE, NULL, 0, NULL), WS_ERR_NULL);
  expect("attn null table", ws_block_causal_attn(&c, FAKE, 8, FAKE, FAKE, 2, 1, NULL, ke, 0.1f, 1, FAKE, NULL, 0, NULL), WS_ERR_NULL);
  expect("attn units 0", ws_block_causal_attn(&c, FAKE, 8, FAKE, FAKE, 2, 0, qb, ke, 0.1f, 1, FAKE, NULL, 0, NULL), WS_ERR_SHAPE);
  {
    /* more units with queries than the launch arguments hold: the table
       goes to the workspace, which is then required */
    int32_t qb70[71], ke70[70];
    for (int u = 0; u <= 70; ++u) qb70[u] = u;
    for (int u = 0; u < 70; ++u) ke70[u] = 1 + u / 10;
    expect("attn many units, no workspace", ws_block_causal_attn(&c, FAKE, 70, FAKE, FAKE, 2, 70, qb70, ke70, 0.1f, 1, FAKE, NULL, 0, NULL), WS_ERR_WORKSPACE);
    expect("attn many units, short workspace", ws_block_causal_attn(&c, FAKE, 70, FAKE, FAKE, 2, 70, qb70, ke70, 0.1f, 1, FAKE, FAKE2, 16, NULL), WS_ERR_WORKSPACE);
  }
  ke[0] = 13;
  expect("attn kend past keys", ws_block_causal_attn(&c, FAKE, 8, FAKE, FAKE, 2, 1, qb, ke, 0.1f, 1, FAKE, NULL, 0, NULL), WS_ERR_SHAPE);
  ke[0] = 0;
  expect("attn kend 0", ws_block_causal_attn(&c, FAKE, 8, FAKE, FAKE, 2, 1, qb, ke, 0.1f, 1, FAKE, NULL, 0, NULL), WS_ERR_SHAPE);
  ke[0] = 12;
  qb[1] = 7;
  expect("attn table end", ws_block_causal_attn(&c, FAKE, 8, FAKE, FAKE, 2, 1, qb, ke, 0.1f, 1, FAKE, NULL, 0, NULL), WS_ERR_SHAPE);
  qb[1] = 8;
  expect("attn scale", ws_block_causal_attn(&c, FAKE, 8, FAKE, FAKE, 2, 1, qb, ke, -1.0f, 1, FAKE, NULL, 0, NULL), WS_ERR_SHAPE);
  expect("attn splits", ws_block_causal_attn(&c, FAKE, 8, FAKE, FAKE, 2, 1, qb, ke, 0.1f, 257, FAKE, NULL, 0, NULL), WS_ERR_SHAPE);
  expect("attn workspace", ws_block_causal_attn(&c, FAKE, 8, FAKE, FAKE, 2, 1, qb, ke, 0.1f, 4, FAKE, NULL, 0, NULL), WS_ERR_WORKSPACE);
  expect("attn short workspace", ws_block_causal_attn(&c, FAKE, 8, FAKE, FAKE, 2, 1, qb, ke, 0.1f, 4, FAKE, FAKE2, 16, NULL), WS_ERR_WORKSPACE);
  expect("attn align", ws_block_causal_attn(&c, (char*)FAKE + 8, 8, FAKE, FAKE, 2, 1, qb, ke, 0.1f, 1, FAKE, NULL, 0, NULL), WS_ERR_ALIGN);
  expect("attn no-op", ws_block_causal_attn(&c, NULL, 0, NULL, NULL, 0, 1, (int32_t[]){0, 0}, (int32_t[]){10}, 0.1f, 0, NULL, NULL, 0, NULL), WS_OK);
  /* the largest unit table, with one decreasing step at the end */
  for (int u = 0; u <= WS_MAX_UNITS; ++u) qb[u] = u < WS_MAX_UNITS ? u / 8 : 8;
  for (int u = 0; u < WS_MAX_UNITS; ++u) ke[u] = 1 + u / 6;
  qb[WS_MAX_UNITS] = 9;  /* the table ends past n_q */
  expect("attn 64 units, table end", ws_attn_partial(&c, FAKE, 8, FAKE, FAKE, 2, WS_MAX_UNITS, qb, ke, 0.1f, 1, FAKE, NULL, 0, NULL), WS_ERR_SHAPE);
  qb[WS_MAX_UNITS] = 8;
  ke[WS_MAX_UNITS - 1] = 1;
  expect("attn kend decreasing", ws_attn_partial(&c, FAKE, 8, FAKE, FAKE, 2, WS_MAX_UNITS, qb, ke, 0.1f, 1, FAKE, NULL, 0, NULL), WS_ERR_SHAPE);
  expect("merge splits", ws_attn_merge(2, 8, 128, 0, FAKE, 1 << 20, FAKE, NULL), WS_ERR_SHAPE);
  expect("merge workspace", ws_attn_merge(2, 8, 128, 4, FAKE, 16, FAKE, NULL), WS_ERR_WORKSPACE);
  expect("merge one split", ws_attn_merge(2, 8, 128, 1, NULL, 0, FAKE, NULL), WS_OK);

  /* Euler */
  expect("euler null", ws_fm_euler_step(NULL, FAKE, 10, 0.25f, NULL), WS_ERR_NULL);
  expect("euler n", ws_fm_euler_step((float*)FAKE, FAKE, -1, 0.25f, NULL), WS_ERR_SHAPE);
  expect("euler dt", ws_fm_euler_step((float*)FAKE, FAKE, 10, 1.0f / 0.0f, NULL), WS_ERR_SHAPE);
  expect("euler empty", ws_fm_euler_step(NULL, NULL, 0, 0.25f, NULL), WS_OK);

  /* planning: pure host functions over a grid of sizes, extremes included */
  const int32_t hs[] = {0, 1, 10, 40, 1000, 2147483647};
  const int32_t qs[] = {0, 1, 4, 32, 33, 920, 58880, 2147483647};
  const int64_t ks[] = {0, 1, 64, 61880, 244772, 2147483583ll};
  for (unsigned a = 0; a < sizeof hs / sizeof *hs; ++a)
    for (unsigned b = 0; b < sizeof qs / sizeof *qs; ++b)
      for (unsigned d = 0; d < sizeof ks / sizeof *ks; ++d) {
        const int32_t s = ws_attn_default_splits(hs[a], qs[b], 128, ks[d]);
        if (s < 1 || s > 256) { fprintf(stderr, "splits %d\n", (int)s); ++fails; }
        (void)ws_attn_workspace_bytes(hs[a], qs[b] > 65536 ? 65536 : qs[b], 128, s);
      }
  for (int s = 0; s < 9; ++s)
    if (!ws_status_string((ws_status)s)[0]) { fprintf(stderr, "status string %d\n", s); ++fails; }
  if (fails) return 1;
  printf("capi_errors ok\n");
  return 0;
}

/* Drives the C ABI's host-side checks for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer: workspace queries at the extremes of every size argument
 * (integer overflow in the size arithmetic would be undefined behaviour) and calls the
 * library must reject, or accept with nothing to enqueue, before touching the GPU. Device
 * pointers are fake addresses that are never dereferenced. Exits 0 when every status is
 * the documented one. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qmoe.h"

#define FAKE(off) ((void*)(uintptr_t)(0x7f0000000000ull + (off)))

static int failures = 0;

static void expect(const char* what, moe_status got, moe_status want) {
  if (got != want) {
    printf("MISMATCH %s: %s, expected %s\n", what, moe_status_string(got),
           moe_status_string(want));
    ++failures;
  }
}

static moe_qmatrix mat(int rows, int cols, int bits, uintptr_t base) {
  moe_qmatrix m;
  m.codes = (const uint32_t*)FAKE(base);
  m.scale_min = (const uint16_t*)FAKE(base + 0x1000000);
  m.rows = rows;
  m.cols = cols;
  m.bits = bits;
  return m;
}

static moe_layer layer(int d, int f, int E, int k, int bits) {
  moe_layer L;
  memset(&L, 0, sizeof L);
  L.d_model = d;
  L.d_ff = f;
  L.n_experts = E;
  L.top_k = k;
  L.gate = mat(f, d, bits, 0x10000000);
  L.up = mat(f, d, bits, 0x20000000);
  L.down = mat(d, f, bits, 0x30000000);
  return L;
}

int main(void) {
  static const int sizes[] = {INT_MIN, -1, 0, 1, 31, 32, 63, 64, 65, 512, 513, 1024, 1025,
                              4096, 8192, 8193, 65536, 65537, INT_MAX};
  const int ns = (int)(sizeof sizes / sizeof sizes[0]);
  moe_routing r = {(int32_t*)FAKE(0x40000000), (float*)FAKE(0x41000000),
                   (int32_t*)FAKE(0x42000000), (int32_t*)FAKE(0x43000000)};
  size_t acc = 0;

  for (int s = -2; s < 8; ++s) acc += strlen(moe_status_string((moe_status)s));

  /* workspace queries over every combination of extreme sizes */
  for (int a = 0; a < ns; ++a)
    for (int b = 0; b < ns; ++b)
      for (int c = 0; c < ns; ++c) {
        acc += moe_route_workspace_bytes(sizes[a], sizes[b], sizes[c]);
        moe_layer L = layer(sizes[b] > 8192 ? 8192 : sizes[b], 8192, 1024,
                            sizes[c] > 64 ? 64 : sizes[c], 4);
        acc += moe_ffn_workspace_bytes(&L, sizes[a], 0);
        acc += moe_ffn_workspace_bytes(&L, sizes[a], 1);
        L.router_w = (const uint16_t*)FAKE(0x50000000);
        acc += moe_ffn_workspace_bytes(&L, sizes[a], 0);
      }
  acc += moe_ffn_workspace_bytes(NULL, 4, 0);

  /* routing: rejected arguments */
  expect("route no logits", moe_route(NULL, 4, 8, 2, &r, NULL, 0, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("route k > E", moe_route((const float*)FAKE(0), 4, 8, 9, &r, NULL, 0, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("route n > max", moe_route((const float*)FAKE(0), 65537, 8, 2, &r, NULL, 0, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("route no workspace",
         moe_route((const float*)FAKE(0), 8192, 512, 10, &r, NULL, 0, NULL),
         MOE_ERR_WORKSPACE_TOO_SMALL);
  expect("route misaligned workspace",
         moe_route((const float*)FAKE(0), 8192, 512, 10, &r, FAKE(0x60000008), 1 << 30, NULL),
         MOE_ERR_INVALID_ARGUMENT);

  /* decode: rejected arguments */
  moe_layer ok = layer(2048, 768, 512, 10, 4);
  const float* x = (const float*)FAKE(0x70000000);
  float* res = (float*)FAKE(0x71000000);
  void* ws = FAKE(0x80000000);
  const size_t wsb = moe_ffn_workspace_bytes(&ok, 4, 0);
  expect("decode null layer", moe_expert_ffn_decode(NULL, x, 4, &r, res, ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("decode n = 0", moe_expert_ffn_decode(&ok, x, 0, &r, res, ws, wsb, NULL, NULL), MOE_OK);
  expect("decode n < 0", moe_expert_ffn_decode(&ok, x, -1, &r, res, ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("decode n > max", moe_expert_ffn_decode(&ok, x, 513, &r, res, ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("decode workspace too small",
         moe_expert_ffn_decode(&ok, x, 4, &r, res, ws, wsb - 1, NULL, NULL),
         MOE_ERR_WORKSPACE_TOO_SMALL);
  expect("decode misaligned x",
         moe_expert_ffn_decode(&ok, (const float*)FAKE(0x70000004), 4, &r, res, ws, wsb, NULL,
                               NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("decode x overlaps residual",
         moe_expert_ffn_decode(&ok, x, 4, &r, (float*)FAKE(0x70000100), ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("decode workspace overlaps residual",
         moe_expert_ffn_decode(&ok, x, 4, &r, (float*)FAKE(0x80000100), ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("decode stages 0",
         moe_expert_ffn_decode_stages(&ok, x, 4, &r, res, ws, wsb, NULL, 0u, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("decode stages 16",
         moe_expert_ffn_decode_stages(&ok, x, 4, &r, res, ws, wsb, NULL, 16u, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  moe_routing r0 = r;
  r0.pair_index = NULL;
  expect("decode routing without pair index",
         moe_expert_ffn_decode(&ok, x, 4, &r0, res, ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  moe_layer bad = ok;
  bad.d_model = 100;
  expect("decode d not /32", moe_expert_ffn_decode(&bad, x, 4, &r, res, ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  bad = ok;
  bad.d_ff = 8224;
  expect("decode f > 8192", moe_expert_ffn_decode(&bad, x, 4, &r, res, ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  bad = layer(2048, 768, 512, 10, 3);
  expect("decode bits 3", moe_expert_ffn_decode(&bad, x, 4, &r, res, ws, wsb, NULL, NULL),
         MOE_ERR_UNSUPPORTED);
  bad = ok;
  bad.top_k = 513;
  expect("decode k > E", moe_expert_ffn_decode(&bad, x, 4, &r, res, ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  bad = ok;
  bad.n_experts = 1025;
  expect("decode E > max", moe_expert_ffn_decode(&bad, x, 4, &r, res, ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  bad = ok;
  bad.gate.codes = (const uint32_t*)FAKE(0x10000004);
  expect("decode misaligned codes", moe_expert_ffn_decode(&bad, x, 4, &r, res, ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  bad = ok;
  bad.down.rows = 768;
  expect("decode down shape", moe_expert_ffn_decode(&bad, x, 4, &r, res, ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  bad = ok;
  bad.shared_gate = mat(768, 2048, 4, 0x90000000);
  bad.shared_up = mat(768, 2048, 4, 0x91000000);
  bad.shared_down = mat(2048, 768, 4, 0x92000000);
  expect("decode shared expert, 9 tokens",
         moe_expert_ffn_decode(&bad, x, 9, &r, res, ws, moe_ffn_workspace_bytes(&bad, 9, 0),
                               NULL, NULL),
         MOE_ERR_UNSUPPORTED);

  /* the fused layer entry points */
  expect("layer no logits, no router",
         moe_layer_decode(&ok, NULL, x, 4, &r, res, ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("layer n = 0 without prep",
         moe_layer_decode_stages(&ok, (const float*)FAKE(0), x, 0, &r, res, ws, wsb, NULL,
                                 MOE_DECODE_GATE_UP, NULL),
         MOE_OK);
  expect("layer misaligned logits",
         moe_layer_decode(&ok, (const float*)FAKE(2), x, 4, &r, res, ws, wsb, NULL, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("no-alloc beyond its workspace",
         moe_layer_decode_noalloc(&ok, (const float*)FAKE(0), x, 256, &r, res, NULL),
         MOE_ERR_WORKSPACE_TOO_SMALL);
  expect("no-alloc null layer",
         moe_layer_decode_noalloc(NULL, (const float*)FAKE(0), x, 4, &r, res, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("no-alloc n > max",
         moe_layer_decode_noalloc(&ok, (const float*)FAKE(0), x, 513, &r, res, NULL),
         MOE_ERR_INVALID_ARGUMENT);

  /* prefill */
  const uint16_t* xb = (const uint16_t*)FAKE(0xA0000000);
  const size_t pwsb = moe_ffn_workspace_bytes(&ok, 8192, 1);
  expect("prefill n = 0", moe_expert_ffn_prefill(&ok, xb, 0, &r, res, ws, pwsb, NULL), MOE_OK);
  expect("prefill n > max", moe_expert_ffn_prefill(&ok, xb, 8193, &r, res, ws, pwsb, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("prefill workspace too small",
         moe_expert_ffn_prefill(&ok, xb, 8192, &r, res, ws, pwsb - 1, NULL),
         MOE_ERR_WORKSPACE_TOO_SMALL);
  expect("prefill x overlaps residual",
         moe_expert_ffn_prefill(&ok, xb, 16, &r, (float*)FAKE(0xA0000010), ws, pwsb, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("prefill stages 0",
         moe_expert_ffn_prefill_stages(&ok, xb, 16, &r, res, ws, pwsb, 0u, NULL),
         MOE_ERR_INVALID_ARGUMENT);
  expect("prefill shared expert", moe_expert_ffn_prefill(&bad, xb, 16, &r, res, ws, pwsb, NULL),
         MOE_ERR_UNSUPPORTED);

  printf("abi driver: %d mismatches, size sum %zu\n", failures, acc);
  return failures ? 1 : 0;
}

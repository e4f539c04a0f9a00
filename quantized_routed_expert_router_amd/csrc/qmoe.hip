// C ABI of libqmoe: argument validation, workspace sizing and kernel launches.
// Every check runs on the host before anything is enqueued.
#include <algorithm>
#include <mutex>
#include <vector>

#include "qmoe_internal.h"

// Workspace of moe_layer_decode_noalloc: one array per GPU, held by the library's code
// object until the process ends. In host code the name is only a stand-in for the
// symbol: the device address comes from hipGetSymbolAddress, per device (scratch_address
// below), and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace qmoe {

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

namespace {

// Device address of this GPU's scratch array, resolved once per device with that device
// current. Returns nullptr if the runtime cannot resolve it.
void* scratch_address() {
  static std::mutex mu;
  static std::vector<void*> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, nullptr);
  if (!cache[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    cache[dev] = ptr;
  }
  return cache[dev];
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}

moe_status check_matrix(const moe_qmatrix& m, int rows, int cols, int bits) {
  if (!m.codes || !m.scale_min) return MOE_ERR_INVALID_ARGUMENT;
  if (m.rows != rows || m.cols != cols || m.bits != bits) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(m.codes, bits == 4 ? 16 : 8) || !aligned(m.scale_min, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

moe_status check_layer(const moe_layer* L) {
  if (!L) return MOE_ERR_INVALID_ARGUMENT;
  const int d = L->d_model, f = L->d_ff, E = L->n_experts, k = L->top_k;
  if (d <= 0 || f <= 0 || d % 32 || f % 32 || d > 8192 || f > 8192) return MOE_ERR_INVALID_ARGUMENT;
  if (E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOP_K)
    return MOE_ERR_INVALID_ARGUMENT;
  const int bits = L->gate.bits;
  if (bits != 2 && bits != 4) return MOE_ERR_UNSUPPORTED;
  if (L->up.bits != bits || L->down.bits != bits) return MOE_ERR_UNSUPPORTED;
  moe_status s = check_matrix(L->gate, f, d, bits);
  if (s == MOE_OK) s = check_matrix(L->up, f, d, bits);
  if (s == MOE_OK) s = check_matrix(L->down, d, f, bits);
  if (s == MOE_OK && L->router_w && !aligned(L->router_w, 16)) s = MOE_ERR_INVALID_ARGUMENT;
  if (s == MOE_OK && has_shared(*L)) {
    s = check_matrix(L->shared_gate, f, d, bits);
    if (s == MOE_OK) s = check_matrix(L->shared_up, f, d, bits);
    if (s == MOE_OK) s = check_matrix(L->shared_down, d, f, bits);
  }
  return s;
}

// The decode path runs a shared expert on the small-window kernels only: chunks taken
// from the expert ids (n <= 8 tokens, n*k <= 64 pairs) and the token-major down with the
// combine, with one more slot per token.
bool shared_decode_supported(const moe_layer* L, int n, unsigned stages) {
  const int k = L->top_k, nbf = L->d_ff / 32;
  if (n > 8 || (long long)n * k > 64 || k + 1 > 16 || nbf > 32) return false;
  if (((k + 2) / 2) * ((nbf + 7) / 8) > 18) return false;
  const bool down = stages & MOE_DECODE_DOWN, combine = stages & MOE_DECODE_COMBINE;
  return down == combine;
}

moe_status check_routing(const moe_routing* r) {
  if (!r || !r->topk_ids || !r->topk_w || !r->expert_offsets || !r->pair_index)
    return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

moe_status decode_entry(const moe_layer* L, const float* logits, bool project, const float* x,
                        int n_tokens, const moe_routing* r, float* residual, void* ws,
                        size_t ws_bytes, const moe_debug* dbg, unsigned stages, void* stream) {
  if (stages == 0 || (stages & ~MOE_DECODE_ALL)) return MOE_ERR_INVALID_ARGUMENT;
  moe_status s = check_layer(L);
  if (s != MOE_OK) return s;
  if (n_tokens < 0 || n_tokens > MOE_MAX_DECODE_TOKENS) return MOE_ERR_INVALID_ARGUMENT;
  if (n_tokens == 0) return MOE_OK;
  if (check_routing(r) != MOE_OK) return MOE_ERR_INVALID_ARGUMENT;
  if (!x || !residual || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(residual, 4) || !aligned(ws, 256))
    return MOE_ERR_INVALID_ARGUMENT;
  if (has_shared(*L) && !shared_decode_supported(L, n_tokens, stages))
    return MOE_ERR_UNSUPPORTED;
  if (logits && !aligned(logits, 4)) return MOE_ERR_INVALID_ARGUMENT;
  const size_t act_bytes = (size_t)n_tokens * L->d_model * sizeof(float);
  if (x != residual && overlaps(x, act_bytes, residual, act_bytes))
    return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = decode_ws_layout(n_tokens, L->top_k, L->d_model, L->d_ff, has_shared(*L),
                                       L->router_w ? L->n_experts : 0)
                          .total;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (overlaps(ws, need, residual, act_bytes) || overlaps(ws, need, x, act_bytes))
    return MOE_ERR_INVALID_ARGUMENT;
  DecodeDebug dd{};
  if (dbg) {
    dd = DecodeDebug{dbg->xq, dbg->xs, dbg->gate_dots, dbg->up_dots,  dbg->g, dbg->u,
                     dbg->h,  dbg->hq, dbg->hs,        dbg->down_dots, dbg->y, dbg->logits};
  }
  DecodeArgs a{L,        logits, project, x, n_tokens, r, residual, (char*)ws,
               dbg ? &dd : nullptr, (hipStream_t)stream, device_cu_count(), stages};
  const hipError_t err = launch_decode(a);
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace
}  // namespace qmoe

using namespace qmoe;

extern "C" {

const char* moe_status_string(moe_status s) {
  // C callers may pass any int; an enum load of a value outside the enumerators' range is
  // undefined in C++, so the code is read as the int it was passed as
  int code;
  memcpy(&code, &s, sizeof code);
  switch (code) {
    case MOE_OK:
      return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT:
      return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED:
      return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL:
      return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP:
      return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

size_t moe_route_workspace_bytes(int n_tokens, int n_experts, int top_k) {
  if (n_tokens < 0 || n_tokens > MOE_MAX_ROUTE_TOKENS) return 0;
  if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS) return 0;
  if (top_k < 1 || top_k > n_experts || top_k > MOE_MAX_TOP_K) return 0;
  return route_workspace_bytes(n_tokens, n_experts, top_k);
}

moe_status moe_route(const float* logits, int n_tokens, int n_experts, int top_k,
                     const moe_routing* out, void* ws, size_t ws_bytes, void* stream) {
  if (n_tokens < 0 || n_tokens > MOE_MAX_ROUTE_TOKENS) return MOE_ERR_INVALID_ARGUMENT;
  if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARGUMENT;
  if (top_k < 1 || top_k > n_experts || top_k > MOE_MAX_TOP_K) return MOE_ERR_INVALID_ARGUMENT;
  if (!out || !out->expert_offsets) return MOE_ERR_INVALID_ARGUMENT;
  if (n_tokens > 0 && (check_routing(out) != MOE_OK || !logits)) return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = route_workspace_bytes(n_tokens, n_experts, top_k);
  if (need > 0) {
    if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(ws, 256)) return MOE_ERR_INVALID_ARGUMENT;
  }
  const hipError_t err =
      launch_route(logits, n_tokens, n_experts, top_k, out, ws, (hipStream_t)stream);
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

size_t moe_ffn_workspace_bytes(const moe_layer* L, int n_tokens, int prefill) {
  if (!L || n_tokens < 0) return 0;
  const int d = L->d_model, f = L->d_ff, k = L->top_k;
  if (d <= 0 || f <= 0 || k <= 0) return 0;
  if (prefill) {
    if (n_tokens > MOE_MAX_PREFILL_TOKENS) return 0;
    const int E = L->n_experts;
    if (E < 1 || E > MOE_MAX_EXPERTS) return 0;
    return prefill_ws_layout(n_tokens, k, d, f, E).total;
  }
  const int E = L->n_experts;
  if (L->router_w && (E < 1 || E > MOE_MAX_EXPERTS)) return 0;
  return decode_ws_layout(n_tokens, k, d, f, has_shared(*L), L->router_w ? E : 0).total;
}

moe_status moe_expert_ffn_decode(const moe_layer* L, const float* x, int n_tokens,
                                 const moe_routing* r, float* residual, void* ws,
                                 size_t ws_bytes, const moe_debug* dbg, void* stream) {
  return moe_expert_ffn_decode_stages(L, x, n_tokens, r, residual, ws, ws_bytes, dbg,
                                      MOE_DECODE_ALL, stream);
}

moe_status moe_expert_ffn_decode_stages(const moe_layer* L, const float* x, int n_tokens,
                                        const moe_routing* r, float* residual, void* ws,
                                        size_t ws_bytes, const moe_debug* dbg, unsigned stages,
                                        void* stream) {
  return decode_entry(L, nullptr, false, x, n_tokens, r, residual, ws, ws_bytes, dbg, stages,
                      stream);
}

moe_status moe_layer_decode(const moe_layer* L, const float* logits, const float* x,
                            int n_tokens, const moe_routing* r, float* residual, void* ws,
                            size_t ws_bytes, const moe_debug* dbg, void* stream) {
  return moe_layer_decode_stages(L, logits, x, n_tokens, r, residual, ws, ws_bytes, dbg,
                                 MOE_DECODE_ALL, stream);
}

moe_status moe_layer_decode_stages(const moe_layer* L, const float* logits, const float* x,
                                   int n_tokens, const moe_routing* r, float* residual, void* ws,
                                   size_t ws_bytes, const moe_debug* dbg, unsigned stages,
                                   void* stream) {
  // without logits the layer projects its own from the router weights
  const bool project = !logits && L && L->router_w;
  if (n_tokens > 0 && !logits && !project) return MOE_ERR_INVALID_ARGUMENT;
  if (n_tokens == 0) {
    // no tokens: the routing still reports empty expert groups
    moe_status s = check_layer(L);
    if (s != MOE_OK) return s;
    if (stages == 0 || (stages & ~MOE_DECODE_ALL)) return MOE_ERR_INVALID_ARGUMENT;
    if (!(stages & MOE_DECODE_PREP)) return MOE_OK;
    return moe_route(logits, 0, L->n_experts, L->top_k, r, nullptr, 0, stream);
  }
  return decode_entry(L, logits, project, x, n_tokens, r, residual, ws, ws_bytes, dbg, stages,
                      stream);
}

moe_status moe_layer_decode_noalloc(const moe_layer* L, const float* logits, const float* x,
                                    int n_tokens, const moe_routing* r, float* residual,
                                    void* stream) {
  const bool project = !logits && L && L->router_w;
  if (n_tokens > 0 && !logits && !project) return MOE_ERR_INVALID_ARGUMENT;
  if (n_tokens == 0)
    return moe_layer_decode_stages(L, logits, x, 0, r, residual, nullptr, 0, nullptr,
                                   MOE_DECODE_ALL, stream);
  moe_status s = check_layer(L);
  if (s != MOE_OK) return s;
  if (n_tokens < 0 || n_tokens > MOE_MAX_DECODE_TOKENS) return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = decode_ws_layout(n_tokens, L->top_k, L->d_model, L->d_ff, has_shared(*L),
                                       L->router_w ? L->n_experts : 0)
                          .total;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = scratch_address();
  if (!ws) return MOE_ERR_HIP;
  return decode_entry(L, logits, project, x, n_tokens, r, residual, ws,
                      (size_t)MOE_NOALLOC_SCRATCH_BYTES, nullptr, MOE_DECODE_ALL, stream);
}

moe_status moe_expert_ffn_prefill(const moe_layer* L, const uint16_t* x_bf16, int n_tokens,
                                  const moe_routing* r, float* residual, void* ws,
                                  size_t ws_bytes, void* stream) {
  return moe_expert_ffn_prefill_stages(L, x_bf16, n_tokens, r, residual, ws, ws_bytes,
                                       MOE_PREFILL_ALL, stream);
}

moe_status moe_expert_ffn_prefill_stages(const moe_layer* L, const uint16_t* x_bf16,
                                         int n_tokens, const moe_routing* r, float* residual,
                                         void* ws, size_t ws_bytes, unsigned stages,
                                         void* stream) {
  if (stages == 0 || (stages & ~MOE_PREFILL_ALL)) return MOE_ERR_INVALID_ARGUMENT;
  moe_status s = check_layer(L);
  if (s != MOE_OK) return s;
  if (has_shared(*L)) return MOE_ERR_UNSUPPORTED;
  if (n_tokens < 0 || n_tokens > MOE_MAX_PREFILL_TOKENS) return MOE_ERR_INVALID_ARGUMENT;
  if (n_tokens == 0) return MOE_OK;
  if (check_routing(r) != MOE_OK) return MOE_ERR_INVALID_ARGUMENT;
  if (!x_bf16 || !residual || !ws) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x_bf16, 16) || !aligned(residual, 16) || !aligned(ws, 256))
    return MOE_ERR_INVALID_ARGUMENT;
  const size_t x_bytes = (size_t)n_tokens * L->d_model * sizeof(uint16_t);
  const size_t res_bytes = (size_t)n_tokens * L->d_model * sizeof(float);
  if (overlaps(x_bf16, x_bytes, residual, res_bytes)) return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = moe_ffn_workspace_bytes(L, n_tokens, 1);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (overlaps(ws, need, residual, res_bytes) || overlaps(ws, need, x_bf16, x_bytes))
    return MOE_ERR_INVALID_ARGUMENT;
  PrefillArgs a{L, x_bf16, n_tokens, r, residual, (char*)ws, (hipStream_t)stream, stages};
  const hipError_t err = launch_prefill(a);
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"

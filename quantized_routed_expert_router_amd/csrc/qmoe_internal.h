// Internal declarations shared by the translation units of libqmoe.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "qmoe.h"

namespace qmoe {

constexpr int kWave = 64;

// ------------------------------------------------------------------ small device helpers

__device__ __forceinline__ double half_bits_to_double(uint32_t bits16) {
  const uint16_t b = (uint16_t)bits16;
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return (double)(float)h;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  const uint16_t b = (uint16_t)bits16;
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

// Load through the constant address space: a wave-uniform address then becomes a scalar
// load (SGPR result, its own wait counter), used for work-list and pair-list reads of data
// written by an earlier kernel launch.
__device__ __forceinline__ int load_uniform(const int* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return *reinterpret_cast<const __attribute__((address_space(4))) int*>(
      reinterpret_cast<uintptr_t>(p));
#else
  return *p;
#endif
}

__device__ __forceinline__ int4 load_uniform(const int4* p) {
  const int* q = reinterpret_cast<const int*>(p);
  return make_int4(load_uniform(q), load_uniform(q + 1), load_uniform(q + 2), load_uniform(q + 3));
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor word 3). Loads through
// it take one VGPR offset per lane plus a wave-uniform SGPR offset, so the many loads a
// wave keeps in flight share one address register; reads past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Signed 8-bit dot product of 4 byte lanes, accumulated into c (v_dot4c_i32_i8).
__device__ __forceinline__ int dot4_i8(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, false);
}

// Activation bytes are stored permuted so that a masked shift of one packed weight word
// lines up with one 4-byte activation word. For `bits`-bit codes a weight word holds
// per = 32/bits codes; (word >> (bits*s)) & mask leaves in byte m the code s + G*m,
// with G = 8/bits shift groups. Activation word k*G + s therefore holds the codes
// per*k + s + G*m, m = 0..3. Returns the byte position of natural index i (0..31).
template <int BITS>
__host__ __device__ __forceinline__ int act_byte_pos(int i) {
  constexpr int per = 32 / BITS, G = 8 / BITS;
  const int kw = i / per, rem = i % per;
  const int s = rem % G, m = rem / G;
  return 4 * (kw * G + s) + m;
}

template <int BITS>
struct CodeMask;
template <>
struct CodeMask<4> {
  static constexpr uint32_t v = 0x0F0F0F0Fu;
};
template <>
struct CodeMask<2> {
  static constexpr uint32_t v = 0x03030303u;
};

// Exact int32 dot of one packed 32-code block against 8 permuted activation words.
template <int BITS>
__device__ __forceinline__ int block_dot(const uint32_t (&w)[BITS], const int* a) {
  constexpr int G = 8 / BITS;
  int acc = 0;
#pragma unroll
  for (int kw = 0; kw < BITS; ++kw)
#pragma unroll
    for (int s = 0; s < G; ++s)
      acc = dot4_i8((int)((w[kw] >> (BITS * s)) & CodeMask<BITS>::v), a[kw * G + s], acc);
  return acc;
}

// Workgroup barrier that publishes LDS written by global_load_lds: the caller has already
// waited (wait_vmcnt) for its own staging loads, so no release fence (which would also wait
// for the weight loads still in flight) is placed before the barrier.
__device__ __forceinline__ void barrier_after_lds_dma() {
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt with only the vector-memory count limited to `vm` (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ------------------------------------------------------------------ workspace layouts

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Work record of one chunk (up to kMaxChunkPairs pairs of one expert), 128 bytes:
// [0] expert, [1] first pair position in pair_index, [2] pair count np, [3] unused,
// [4..12) pair ids p, [12..20) token ids p / k (entries >= np repeat entry np-1).
constexpr int kMaxChunkPairs = 8;
constexpr int kChunkInts = 32;

// Whether the layer carries a shared expert (moe_layer.shared_*).
inline bool has_shared(const moe_layer& L) { return L.shared_gate.codes != nullptr; }

// Pairs Q = n*k, plus n with a shared expert (token t's shared pair is n*k + t).
struct DecodeWs {
  size_t chunks;   // int [Q][kChunkInts] work records
  size_t nchunks;  // int  [1]
  size_t xq;       // int8 [n][d]  permuted activation codes
  size_t xsc;      // double2 [n][d/32]   (scale, scale*sum of codes)
  size_t hq;       // int8 [Q][f] permuted hidden codes
  size_t hsc;      // double2 [Q][f/32]
  size_t hf;       // float [Q][f] h before quantization (read by the token-major down)
  size_t y;        // double [Q][d]
  size_t logits;   // float [n][E] router logits (a layer with router weights), else empty
  size_t total;
};

// router_E: E for a layer with router weights (its logits are projected into ws), else 0.
inline DecodeWs decode_ws_layout(int n, int k, int d, int f, bool shared, int router_E) {
  DecodeWs L;
  size_t o = 0;
  const size_t P = (size_t)n * k + (shared ? (size_t)n : 0);
  L.chunks = o;
  o = align256(o + sizeof(int) * kChunkInts * (P + 1));
  L.nchunks = o;
  o = align256(o + 16);
  L.xq = o;
  o = align256(o + (size_t)n * d);
  L.xsc = o;
  o = align256(o + 16 * (size_t)n * (d / 32));
  L.hq = o;
  o = align256(o + P * f);
  L.hsc = o;
  o = align256(o + 16 * P * (f / 32));
  L.hf = o;
  o = align256(o + 4 * P * f);
  L.y = o;
  o = align256(o + 4 * P * d);
  L.logits = o;
  o = align256(o + 4 * (size_t)n * (size_t)router_E);
  L.total = o;
  return L;
}

// Prefill workspace. M-tiles hold up to kPrefillBM consecutive grouped pairs of one
// expert; h and y are kept in grouped pair order.
constexpr int kPrefillBM = 256;

struct PrefillWs {
  size_t tiles;     // int4 [max M-tiles] (expert, first grouped position, rows, 0)
  size_t ntiles;    // int  [1]
  size_t tok_of_g;  // int  [n*k] token of grouped position g
  size_t g_of_p;    // int  [n*k] grouped position of pair p = t*k + j
  size_t h;         // bf16 [n*k][f]
  size_t y;         // fp32 [n*k][d]
  size_t total;
};

// Upper bound of the number of M-tiles: sum over experts of ceil(m_e / BM) with
// sum m_e = P and at most min(E, P) non-empty experts.
inline int prefill_max_mtiles(int P, int E) {
  const long long busy = std::min<long long>(E, P);
  return (int)(((long long)P + busy * (kPrefillBM - 1)) / kPrefillBM);
}

inline PrefillWs prefill_ws_layout(int n, int k, int d, int f, int E) {
  PrefillWs L;
  size_t o = 0;
  const size_t P = (size_t)n * k;
  L.tiles = o;
  o = align256(o + 16 * (size_t)(prefill_max_mtiles((int)P, E) + 1));
  L.ntiles = o;
  o = align256(o + 16);
  L.tok_of_g = o;
  o = align256(o + 4 * P);
  L.g_of_p = o;
  o = align256(o + 4 * P);
  L.h = o;
  o = align256(o + 2 * P * f);
  L.y = o;
  o = align256(o + 4 * P * d);
  L.total = o;
  return L;
}

struct PrefillArgs {
  const moe_layer* L;
  const uint16_t* x;
  int n;
  const moe_routing* r;
  float* residual;
  char* ws;
  hipStream_t stream;
  unsigned stages;  // MOE_PREFILL_* bits
};

struct DecodeDebug {
  int8_t* xq;
  float* xs;
  int32_t* gate_dots;
  int32_t* up_dots;
  float* g;
  float* u;
  float* h;
  int8_t* hq;
  float* hs;
  int32_t* down_dots;
  float* y;
  float* logits;
};

struct DecodeArgs {
  const moe_layer* L;
  const float* logits;  // non-null: route inside the prep stage (moe_layer_decode)
  bool project;         // route from logits = x . router_w^T, projected into ws first
  const float* x;
  int n;
  const moe_routing* r;
  float* residual;
  char* ws;
  const DecodeDebug* dbg;  // nullptr: fast instances
  hipStream_t stream;
  int num_cus;
  unsigned stages;  // MOE_DECODE_* bits
};

// ------------------------------------------------------------------ routing workspace

// Grouping of more than kSingleGroupPairs pairs runs over many workgroups, in chunks of
// kChunkPairs pairs, each with its own expert histogram in the routing workspace.
constexpr int kSingleGroupPairs = 4096;
constexpr int kChunkPairs = 2048;
// Up to this many tokens moe_route selects and groups in one workgroup (k_route_fused).
// Above it the selection is spread over many workgroups: at 17-32 tokens the two forms
// take the same time, and from 24 tokens on the spread one is faster.
constexpr int kFusedRouteTokens = 16;

inline size_t route_workspace_bytes(int n, int E, int k) {
  const long long P = (long long)n * k;
  if (n <= 64 || P <= kSingleGroupPairs) return 0;
  const long long nchunks = (P + kChunkPairs - 1) / kChunkPairs;
  return (size_t)(nchunks * E * (long long)sizeof(int));
}

// ------------------------------------------------------------------ launchers

hipError_t launch_route(const float* logits, int n, int E, int k, const moe_routing* out,
                        void* ws, hipStream_t stream);
// The spread top-k alone (one wave a token): expert ids and routing weights, no grouping.
hipError_t launch_route_topk(const float* logits, int n, int E, int k, int32_t* ids, float* w,
                             hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_prefill(const PrefillArgs& a);

int device_cu_count();

}  // namespace qmoe

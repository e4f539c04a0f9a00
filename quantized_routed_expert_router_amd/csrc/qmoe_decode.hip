// Decode-window expert FFN: the hot path of the routed-expert layer for small batches
// (the T <= 5 verify window of speculative decoding, and batches of windows).
//
// The pages' engine computes cached experts for the whole verify window in one grouped
// kernel (Strata engine explainer, m.lqnn.cn/news/264700, section "Expert cache") and
// its CPU kernels quantize each activation vector to int8 once and reuse it over many
// weight rows with 4-wide int8 dot products (section "CPU expert pool"). Kernels here:
//
//   k_router_logits  (optional) logits = x . W_r^T from bf16 router rows, binary64 sums.
//   k_route_prep     top-k routing of up to 16 tokens by one workgroup (one wave per
//                    token), fused with the int8 block quantization of x by the other
//                    workgroups; past the ids path it also groups the pairs and builds
//                    the work list.
//   k_group_prep     wider windows (up to 4096 pairs), after the spread top-k: grouping
//                    and work list in workgroup 0, the quantization of x in the others.
//                    k_prep does the quantization and the work list after a separate
//                    routing call.
//   k_gateup         one workgroup per (chunk of pairs of one expert, 16 or 32 rows of
//                    f): the gate and up rows of the item stream through raw buffer loads
//                    (all blocks of a lane at once), exact int32 block dots with v_dot4
//                    against activation codes staged in LDS, binary64 block terms, then
//                    SwiGLU; 32-row items also quantize their block of h to int8, 16-row
//                    items (small windows) leave h in fp32. For small windows the chunks
//                    come straight from the expert ids and workgroup 0 writes the
//                    routing's grouping.
//   k_down_tok       small windows: the int8 quantization of the token's h, the down
//                    projection by token, and the routing-weighted combine into the
//                    residual (no pair outputs leave the workgroup).
//   k_hquant         the h quantization alone, when a small window's down runs by expert.
//   k_down, k_combine  larger windows: the down projection by expert chunk (fp32 pair
//                    outputs, each a binary64 row sum rounded once), then the slot-order
//                    binary64 combine in a launch of its own. Folding the combine into
//                    k_down through a last-arriver counter needs the pair outputs to cross
//                    XCDs, through device-scope fences (an L2 writeback per workgroup) or
//                    write-through stores and loads, and both put a chain of memory round
//                    trips on the last workgroup that costs more than this small launch.
//
// Block terms (scale*xs)*dot and min*(xs*sum) are exact in binary64, so row sums round
// only in the additions. Every expert's weights are read once per chunk of up to NPC
// pairs; at n <= NPC tokens (the T = 4 window) every touched expert is read exactly once
// per call, and up to 2*NPC tokens at most twice.
#include <algorithm>

#include "qmoe_route_dev.h"

namespace qmoe {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- int8 block quantizer

// Quantize one 32-value block held as v[32]: returns scale; q receives codes. The block
// maximum of |v| is taken over the bit patterns as unsigned integers (which order
// non-negative floats like their values) in a tree, so it is exact and its dependent
// chain is 5 steps instead of 32.
__device__ __forceinline__ float quant_block32(const float (&v)[32], int (&q)[32]) {
  uint32_t m[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t a = __float_as_uint(fabsf(v[2 * i])), b = __float_as_uint(fabsf(v[2 * i + 1]));
    m[i] = a > b ? a : b;
  }
#pragma unroll
  for (int w = 8; w >= 1; w /= 2)
#pragma unroll
    for (int i = 0; i < w; ++i) m[i] = m[i] > m[i + w] ? m[i] : m[i + w];
  const float amax = __uint_as_float(m[0]);
  if (amax == 0.0f) {
#pragma unroll
    for (int i = 0; i < 32; ++i) q[i] = 0;
    return 0.0f;
  }
  const float scale = amax / 127.0f;
  const float inv = 127.0f / amax;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float t = __builtin_rintf(v[i] * inv);
    t = t > 127.0f ? 127.0f : t;
    t = t < -127.0f ? -127.0f : t;
    q[i] = (int)t;
  }
  return scale;
}

// Sum of the 32 codes of a block, in a tree (exact in int32).
__device__ __forceinline__ int code_sum32(const int (&q)[32]) {
  int s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = q[2 * i] + q[2 * i + 1];
#pragma unroll
  for (int w = 8; w >= 1; w /= 2)
#pragma unroll
    for (int i = 0; i < w; ++i) s[i] += s[i + w];
  return s[0];
}

// ---------------------------------------------------------------- prep: x quant + work list

constexpr int kPrepThreads = 1024;  // block 0: one thread per expert (E <= 1024)
constexpr int kPrepWaves = kPrepThreads / kWave;

// One (token, 32-block) of x -> permuted int8 codes, (scale, scale*sum of codes).
template <int BITS>
__device__ __forceinline__ void quant_x_block(const float* __restrict__ x, int d, int t, int b,
                                              int8_t* __restrict__ xq, double2* __restrict__ xsc,
                                              int8_t* __restrict__ dbg_xq,
                                              float* __restrict__ dbg_xs) {
  const int nbd = d / 32;
  float v[32];
  const float4* src = reinterpret_cast<const float4*>(x + (size_t)t * d + 32 * b);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 f4 = src[i];
    v[4 * i] = f4.x;
    v[4 * i + 1] = f4.y;
    v[4 * i + 2] = f4.z;
    v[4 * i + 3] = f4.w;
  }
  int q[32];
  const float scale = quant_block32(v, q);
  const int sum = code_sum32(q);
  uint32_t words[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int pos = act_byte_pos<BITS>(i);
    words[pos / 4] |= ((uint32_t)q[i] & 0xffu) << (8 * (pos % 4));
  }
  uint4* dst = reinterpret_cast<uint4*>(xq + (size_t)t * d + 32 * b);
  dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
  dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
  xsc[(size_t)t * nbd + b] = make_double2((double)scale, (double)scale * (double)sum);
  if (dbg_xq) {
#pragma unroll
    for (int i = 0; i < 32; ++i) dbg_xq[(size_t)t * d + 32 * b + i] = (int8_t)q[i];
  }
  if (dbg_xs) dbg_xs[(size_t)t * nbd + b] = scale;
}

// Work list: expert e (one per thread, E <= blockDim.x = kPrepThreads) with c pairs
// contributes ceil(c/npc) chunk records, in expert order. off/pidx may be LDS or global.
__device__ __forceinline__ void build_work_list(const int32_t* off, const int32_t* pidx, int E,
                                                int k, int npc, int* __restrict__ chunks,
                                                int* __restrict__ nchunks, int* s_wsum) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int e = tid;
  const int beg = e < E ? off[e] : 0;
  const int c = e < E ? off[e + 1] - beg : 0;
  const int cnt = (c + npc - 1) / npc;
  const int incl = wave_inclusive_scan(cnt);
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int base = incl - cnt;
  for (int w = 0; w < wave; ++w) base += s_wsum[w];
  for (int j = 0; j < cnt; ++j) {
    int* rec = chunks + (size_t)(base + j) * kChunkInts;
    const int first = beg + j * npc, np = min(npc, c - j * npc);
    int p[kMaxChunkPairs];
#pragma unroll
    for (int q = 0; q < kMaxChunkPairs; ++q) p[q] = pidx[first + min(q, np - 1)];
    rec[0] = e;
    rec[1] = first;
    rec[2] = np;
    rec[3] = 0;
#pragma unroll
    for (int q = 0; q < kMaxChunkPairs; ++q) {
      rec[4 + q] = p[q];
      rec[4 + kMaxChunkPairs + q] = p[q] / k;
    }
  }
  if (tid == kPrepThreads - 1) *nchunks = base + cnt;
}

// prep after a separate routing call: block 0 builds the work list from the routing in
// global memory, the other blocks quantize x.
template <int BITS>
__global__ __launch_bounds__(kPrepThreads) void k_prep(
    const float* __restrict__ x, int n, int d, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ pair_index, int E, int k, int npc, int* __restrict__ chunks,
    int* __restrict__ nchunks, int8_t* __restrict__ xq,
    double2* __restrict__ xsc, int8_t* __restrict__ dbg_xq, float* __restrict__ dbg_xs) {
  if (blockIdx.x == 0) {
    __shared__ int s_wsum[kPrepWaves];
    build_work_list(offsets, pair_index, E, k, npc, chunks, nchunks, s_wsum);
    return;
  }
  const int nbd = d / 32;
  const int gid = (blockIdx.x - 1) * kPrepThreads + threadIdx.x;
  if (gid >= n * nbd) return;
  quant_x_block<BITS>(x, d, gid / nbd, gid % nbd, xq, xsc, dbg_xq, dbg_xs);
}

// Routing fused with prep for small batches (n <= kFusedMaxTokens): block 0 selects the
// top-k experts of every token (one wavefront per token), groups the pairs by expert and
// builds the work list without leaving LDS, writing the routing outputs on the way; the
// other blocks quantize x meanwhile. Without GROUP, block 0 stops after the top-k: the
// gate/up kernel then takes its chunks from the expert ids and writes the grouping.
constexpr int kFusedMaxTokens = 16;
constexpr int kFusedMaxPairs = kFusedMaxTokens * MOE_MAX_TOP_K;
constexpr int kFusedGroupWaves = 8;

template <int BITS, int KPL, bool GROUP>
__global__ __launch_bounds__(kPrepThreads) void k_route_prep(
    const float* __restrict__ logits, const float* __restrict__ x, int n, int d, int E, int k,
    int npc, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pair_index, int* __restrict__ chunks,
    int* __restrict__ nchunks, int8_t* __restrict__ xq, double2* __restrict__ xsc,
    int8_t* __restrict__ dbg_xq, float* __restrict__ dbg_xs) {
  if (blockIdx.x == 0) {
    __shared__ __attribute__((aligned(16))) int s_ids[kFusedMaxPairs + 4];
    __shared__ int s_pidx[kFusedMaxPairs];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    __shared__ int s_hist[kFusedGroupWaves * MOE_MAX_EXPERTS];
    __shared__ int s_wsum[kPrepWaves];
    __shared__ TopkScratch s_tk[kPrepWaves];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
    const int P = n * k;
    for (int t = wave; t < n; t += kPrepWaves) {
      const int id = wave_topk<KPL>(logits + (size_t)t * E, E, k, topk_ids + (size_t)t * k,
                                    topk_w + (size_t)t * k, &s_tk[wave]);
      if (lane < k) s_ids[t * k + lane] = id;
    }
    if (!GROUP) return;  // the gate/up kernel groups (chunks from ids)
    if (tid < 4 && P + tid < ((P + 3) & ~3)) s_ids[P + tid] = 0x7fffffff;  // group_small pad
    __syncthreads();
    if (P <= kWave)
      group_tiny(s_ids, P, E, s_off, s_pidx);
    else if (P <= kSmallPairs)
      group_small(s_ids, P, E, s_off, s_pidx);
    else
      group_block<kFusedGroupWaves>(s_ids, P, E, s_hist, s_off, s_wsum, s_off, s_pidx);
    __syncthreads();
    for (int e = tid; e <= E; e += kPrepThreads) offsets[e] = s_off[e];
    for (int i = tid; i < P; i += kPrepThreads) pair_index[i] = s_pidx[i];
    build_work_list(s_off, s_pidx, E, k, npc, chunks, nchunks, s_wsum);
    return;
  }
  const int nbd = d / 32;
  const int gid = (blockIdx.x - 1) * kPrepThreads + threadIdx.x;
  if (gid >= n * nbd) return;
  quant_x_block<BITS>(x, d, gid / nbd, gid % nbd, xq, xsc, dbg_xq, dbg_xs);
}

// Prep after the spread top-k, for windows past kFusedMaxTokens with at most
// kSingleGroupPairs pairs: block 0 copies the expert ids into LDS, groups the pairs by
// expert and builds the work list there, writing the grouping outputs on the way (one
// launch and one memory round trip fewer than a separate grouping kernel followed by
// k_prep); the other blocks quantize x.
template <int BITS>
__global__ __launch_bounds__(kPrepThreads) void k_group_prep(
    const float* __restrict__ x, int n, int d, const int32_t* __restrict__ topk_ids, int E,
    int k, int npc, int32_t* __restrict__ offsets, int32_t* __restrict__ pair_index,
    int* __restrict__ chunks, int* __restrict__ nchunks, int8_t* __restrict__ xq,
    double2* __restrict__ xsc, int8_t* __restrict__ dbg_xq, float* __restrict__ dbg_xs) {
  if (blockIdx.x == 0) {
    __shared__ int s_ids[kSingleGroupPairs];
    __shared__ int s_pidx[kSingleGroupPairs];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    __shared__ int s_hist[kFusedGroupWaves * MOE_MAX_EXPERTS];
    __shared__ int s_wsum[kPrepWaves];
    const int tid = threadIdx.x;
    const int P = n * k;
    ids_to_lds<kSingleGroupPairs, kPrepThreads>(topk_ids, P, s_ids);
    __syncthreads();
    group_block<kFusedGroupWaves>(s_ids, P, E, s_hist, s_off, s_wsum, s_off, s_pidx);
    __syncthreads();
    for (int e = tid; e <= E; e += kPrepThreads) offsets[e] = s_off[e];
    for (int i = tid; i < P; i += kPrepThreads) pair_index[i] = s_pidx[i];
    build_work_list(s_off, s_pidx, E, k, npc, chunks, nchunks, s_wsum);
    return;
  }
  const int nbd = d / 32;
  const int gid = (blockIdx.x - 1) * kPrepThreads + threadIdx.x;
  if (gid >= n * nbd) return;
  quant_x_block<BITS>(x, d, gid / nbd, gid % nbd, xq, xsc, dbg_xq, dbg_xs);
}

// ---------------------------------------------------------------- router projection

// logits[t][e] = sum_c x[t][c] * W[e][c], W bf16 [E][d], x fp32 [n][d] (the layer's router;
// the engine explainer keeps it on the GPU, "Architecture overview"). It is a launch of its
// own ahead of k_route_prep: the top-k of a token needs all E logits, which come from many
// workgroups, and a hand-off between workgroups inside one launch needs write-through
// stores, an arrival counter and write-through loads, a chain of memory round trips of
// the order of the 1.5 us kernel boundary.
//
// One workgroup per expert. The reduction axis is cut into passes of 512 columns, and wave
// q of the workgroup takes passes q, q + 4, ...; lane l of a pass owns columns 8l .. 8l+7
// of it and loads them straight from memory (router row and x: no other wave of the
// workgroup needs them). Tokens go in groups of kRtTok, their four sums interleaved.
// Every product (bf16 times fp32) is exact in binary64; a lane sums its columns in
// increasing order, a DPP reduction gathers the 64 lane sums into lane 63, and the four
// waves' sums are added in wave order and rounded to fp32 once.
constexpr int kRtWaves = 4;
constexpr int kRtThreads = kRtWaves * kWave;
constexpr int kRtTok = 4;
constexpr int kRtPass = 8 * kWave;  // columns per pass

// Sum of a binary64 value over the wave, in lane 63: row shifts by 1, 2, 4 and 8 (lanes
// without a source add 0), then row 0's total into row 1 and row 2's into row 3
// (row_bcast:15), then rows 0-1's total into rows 2-3 (row_bcast:31). The order is fixed.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
  uint64_t u;
  __builtin_memcpy(&u, &v, 8);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xF, false);
  u = ((uint64_t)hi << 32) | lo;
  double r;
  __builtin_memcpy(&r, &u, 8);
  return r;
}

__device__ __forceinline__ double wave_sum_f64_to_last(double v) {
  v += dpp_f64<0x111, 0xF>(v);  // row_shr:1
  v += dpp_f64<0x112, 0xF>(v);  // row_shr:2
  v += dpp_f64<0x114, 0xF>(v);  // row_shr:4
  v += dpp_f64<0x118, 0xF>(v);  // row_shr:8
  v += dpp_f64<0x142, 0xA>(v);  // row_bcast:15
  v += dpp_f64<0x143, 0xC>(v);  // row_bcast:31
  return v;
}

__global__ __launch_bounds__(kRtThreads) void k_router_logits(
    const uint16_t* __restrict__ W, const float* __restrict__ x, int n, int d, int E,
    float* __restrict__ logits, float* __restrict__ dbg_logits) {
  __shared__ double red[kRtWaves][kRtTok];
  typedef float v4f __attribute__((ext_vector_type(4)));
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int e = blockIdx.x;
  const uint16_t* __restrict__ wrow = W + (size_t)e * d;
  const int npass = (d + kRtPass - 1) / kRtPass;
  for (int t0 = 0; t0 < n; t0 += kRtTok) {
    double acc[kRtTok];
#pragma unroll
    for (int tt = 0; tt < kRtTok; ++tt) acc[tt] = 0.0;
    for (int p = wave; p < npass; p += kRtWaves) {
      // columns past d: clamped (valid) loads whose terms are dropped by a select
      const int c = p * kRtPass + 8 * lane;
      const bool use = c < d;
      const int cc = min(c, d - 8);
      const v4u wv = *reinterpret_cast<const __attribute__((address_space(1))) v4u*>(
          reinterpret_cast<uintptr_t>(wrow + cc));
      v4f xa[kRtTok], xb[kRtTok];
#pragma unroll
      for (int tt = 0; tt < kRtTok; ++tt) {
        const float* xr = x + (size_t)min(t0 + tt, n - 1) * d + cc;
        xa[tt] = *reinterpret_cast<const __attribute__((address_space(1))) v4f*>(
            reinterpret_cast<uintptr_t>(xr));
        xb[tt] = *reinterpret_cast<const __attribute__((address_space(1))) v4f*>(
            reinterpret_cast<uintptr_t>(xr + 4));
      }
      __builtin_amdgcn_sched_barrier(0);  // all nine requests go out before any arithmetic
      double wd[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wd[2 * i] = (double)__uint_as_float(wv[i] << 16);
        wd[2 * i + 1] = (double)__uint_as_float(wv[i] & 0xffff0000u);
      }
      double s[kRtTok];
#pragma unroll
      for (int tt = 0; tt < kRtTok; ++tt) s[tt] = acc[tt];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int tt = 0; tt < kRtTok; ++tt) {
          const float xv = i < 4 ? xa[tt][i] : xb[tt][i - 4];
          s[tt] = __builtin_fma(wd[i], (double)xv, s[tt]);
        }
      }
#pragma unroll
      for (int tt = 0; tt < kRtTok; ++tt) acc[tt] = use ? s[tt] : acc[tt];
    }
#pragma unroll
    for (int tt = 0; tt < kRtTok; ++tt) {
      const double v = wave_sum_f64_to_last(acc[tt]);
      if (lane == kWave - 1) red[wave][tt] = v;
    }
    __syncthreads();
    if (tid < kRtTok && t0 + tid < n) {
      double v = red[0][tid];
#pragma unroll
      for (int q = 1; q < kRtWaves; ++q) v += red[q][tid];  // wave order
      const float lf = (float)v;
      logits[(size_t)(t0 + tid) * E + e] = lf;
      if (dbg_logits) dbg_logits[(size_t)(t0 + tid) * E + e] = lf;
    }
    __syncthreads();  // red is reused by the next token group
  }
}

// ---------------------------------------------------------------- streaming block loads

// One packed block (16 B at 4 bits, 8 B at 2 bits) through a buffer resource.
// Expert weights and their scale/min words are read once per call: their loads carry the
// non-temporal cache policy (kNt). On the T=4 window this measured 0.5-0.8 us faster in
// the gate/up kernel and about 1 us faster a step.
constexpr int kNt = 2;
template <int BITS>
struct BlockLoad;
template <>
struct BlockLoad<4> {
  __device__ static __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int voff, int soff,
                                              uint32_t (&w)[4]) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kNt);
    w[0] = v[0];
    w[1] = v[1];
    w[2] = v[2];
    w[3] = v[3];
  }
};
template <>
struct BlockLoad<2> {
  __device__ static __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int voff, int soff,
                                              uint32_t (&w)[2]) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, kNt);
    w[0] = v[0];
    w[1] = v[1];
  }
};

// Sum the waves' partial row sums in wave order (deterministic).
template <int NPC, int NW>
__device__ __forceinline__ double reduce_waves(double (*red)[NPC][kWave], int j, int lane) {
  double s = red[0][j][lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) s += red[w][j][lane];
  return s;
}

// All-lane reductions over each 32-lane half of a wave: DPP steps combine lanes within a
// 16-lane row (quad swaps, then the half-row and row mirrors), and one ds_swizzle swaps the
// two rows of the half (xor 16).
template <class Op>
__device__ __forceinline__ uint32_t half_wave_allreduce(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
  // bit-mask swizzle within 32 lanes: and 0x1f, or 0, xor 0x10
  v = op(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (0x10 << 10)));
  return v;
}

// Quantize h over 32-lane halves of a wave (rows 32b .. 32b+31): returns the code; the
// scale and the code sum of the half are returned through scale/sum. |h| is compared as
// unsigned bit patterns, which orders non-negative floats like their values.
__device__ __forceinline__ int quant_half_wave(float h, float& scale, int& sum) {
  const uint32_t abits = half_wave_allreduce(__float_as_uint(fabsf(h)),
                                             [](uint32_t a, uint32_t b) { return a > b ? a : b; });
  const float amax = __uint_as_float(abits);
  int q = 0;
  scale = 0.0f;
  if (amax != 0.0f) {
    scale = amax / 127.0f;
    const float inv = 127.0f / amax;
    float t = __builtin_rintf(h * inv);
    t = t > 127.0f ? 127.0f : t;
    t = t < -127.0f ? -127.0f : t;
    q = (int)t;
  }
  sum = (int)half_wave_allreduce((uint32_t)q, [](uint32_t a, uint32_t b) { return a + b; });
  return q;
}

// ---------------------------------------------------------------- gate/up + SwiGLU + h quant

// A workgroup of WAVES waves takes one item = (chunk of pairs of one expert, ROWS rows of
// f). The first half of the waves streams the gate matrix and the second half the up
// matrix. The reduction axis is cut into parts, 64/ROWS a wave: lane l of wave w owns row
// l%ROWS and part ke = (64/ROWS)*(w % (WAVES/2)) + l/ROWS, and reads blocks ke, ke+kSplit,
// ... in groups of 64 blocks. All loads of a group are issued at once (the whole reduction
// axis at d = 2048), so every weight byte of the item is in flight after one memory
// latency, and the dots of a block start as soon as that block lands. The chunk's
// activation codes and scales are staged in LDS per group and read back with
// half-wave-uniform addresses.
//
// Shapes:
// * ROWS = 16, 4 waves (windows of up to 16 tokens, ahead of the token-major down): 40 KB
//   of weights an item, five workgroups a CU (4-pair chunks), so the ~1000 items of a T=4
//   window run in one round; the 16 rows are half of an h block, so h leaves in fp32 and
//   the down kernel quantizes it. (Reading the same bytes as 1056 workgroups of 40 KB
//   instead of 528 of 80 KB measured 10% faster in a plain read probe.)
// * ROWS = 32 (ahead of the expert-major down): one item is exactly one 32-row block of
//   h, so the int8 quantization of h closes inside the workgroup. Four waves (three
//   workgroups a CU, 16 blocks a lane) serve the batched work list, whose thousands of
//   items run in many rounds: 4-8% faster there than eight waves, which serve the ids
//   path of windows too wide for the token-major down.
template <int V>
struct Int {
  static constexpr int value = V;
};
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));
// The host selects the matrix-core instance of the expert-major down (k_down) when the
// window averages at least this many pairs per busy expert.
constexpr int kMmaMinPairs = 4;
// 2-bit 32-row gate/up work-list items: chunks of at least kGuMmaFull pairs take the
// matrix-core block dots on all eight pair slots, chunks of kGuMmaHalf to 4 pairs the
// half-slot form (k_gateup), smaller chunks the per-chunk-size dot4 variants
constexpr int kGuMmaFull = 5;
constexpr int kGuMmaHalf = 3;
// the same two thresholds in the matrix-core instance of the expert-major down
constexpr int kDnMmaFull = 5;
constexpr int kDnMmaHalf = 3;
template <int BITS, int NPC, int WAVES, int ROWS, bool IDS>
constexpr bool gu_has_mma() {
  return BITS == 2 && NPC == 8 && WAVES == 4 && ROWS == 32 && !IDS;
}
constexpr int kGuRows = 32;   // rows of an h block
constexpr int kGuGroup = 64;  // blocks per group
template <int WAVES, int ROWS>
struct GuShape {
  static constexpr int kThreads = WAVES * kWave;
  static constexpr int kKWaves = WAVES / 2;          // waves per matrix
  static constexpr int kPW = kWave / ROWS;           // reduction-axis parts a wave
  static constexpr int kSplit = kKWaves * kPW;       // reduction-axis parts
  static constexpr int kUnroll = kGuGroup / kSplit;  // blocks per lane per group
};
// register budget (waves a SIMD): five 16-row workgroups a CU where the registers allow
constexpr int gu_waves_per_eu(int waves, int rows, int npc, bool dbg) {
  return rows == 16 ? (npc <= 4 && !dbg ? 5 : 4) : waves == 8 ? 4 : 3;
}

// Activation staging straight into LDS with global_load_lds_dwordx4: each wave-level load
// writes 64 consecutive 16-byte entries of s_act[j][bb][part] (part 0/1: the two halves of
// a block's 32 codes, part 2: (scale, scale*sum)), without passing through registers. The
// loads are issued before the weight loads; since vector loads complete in order, a wave
// then waits for them with vmcnt(number of weight loads issued after them), which leaves
// the weight loads in flight, and a workgroup barrier publishes the staged data.
template <int NPC, int G, int NT>
struct ActLds {
  static constexpr int kTotal = NPC * G * 3;               // 16-byte entries used
  static constexpr int kIter = (kTotal + NT - 1) / NT;     // wave-level loads per wave
  static constexpr int kPadded = kIter * NT;               // entries allocated
};

// Activation row of chunk pair jc (wave-uniform): from the work record in memory, or from
// uniform registers.
template <int N>
struct RowSet {
  int r[N];
};
__device__ __forceinline__ int chunk_row(const int* __restrict__ rows, int jc) {
  return load_uniform(rows + jc);
}
template <int N>
__device__ __forceinline__ int chunk_row(RowSet<N> rows, int jc) {
  int r = rows.r[0];
#pragma unroll
  for (int j = 1; j < N; ++j) r = jc == j ? rows.r[j] : r;
  return r;
}

template <int NPC, int G, int NT, class Rows>
__device__ __forceinline__ void act_load_lds(int4* s_act, const int8_t* __restrict__ act,
                                             const double2* __restrict__ sc, Rows rows, int np,
                                             int g0, int nb, int rowlen, int wave, int lane) {
  constexpr int kTotal = ActLds<NPC, G, NT>::kTotal;
  static_assert((G * 3) % kWave == 0, "a wave-level load stays within one pair's entries");
  // Every wave issues kIter loads with no branch (a branch would make the compiler wait for
  // the first load before issuing the next); loads past kTotal fill the padding.
#pragma unroll
  for (int it = 0; it < ActLds<NPC, G, NT>::kIter; ++it) {
    const int wbase = it * NT + wave * kWave;  // wave-uniform
    const int src_base = min(wbase, kTotal - kWave);
    // the pair is uniform across the wave, and so is its activation row
    const int jc = min(src_base / (G * 3), np - 1);
    const int rj = chunk_row(rows, jc);
    const int rem = src_base % (G * 3) + lane;
    const int bb = rem / 3, part = rem % 3;
    const int b = min(g0 + bb, nb - 1);
    const uintptr_t a_codes =
        reinterpret_cast<uintptr_t>(act + (size_t)rj * rowlen + 32 * b) + 16 * (part & 1);
    const uintptr_t a_scale = reinterpret_cast<uintptr_t>(sc + (size_t)rj * nb + b);
    typedef const __attribute__((address_space(1))) void* gptr_t;
    typedef __attribute__((address_space(3))) void* lptr_t;
    __builtin_amdgcn_global_load_lds((gptr_t)(part < 2 ? a_codes : a_scale),
                                     (lptr_t)(s_act + wbase), 16, 0, 0);
  }
}

// Chunks straight from the routing (IDS): for windows of n <= 2*NPC tokens and P = n*k <=
// 64 pairs, a workgroup derives its item's chunk from the P expert ids instead of reading
// a work list (one wavefront does it). Lane p holds ids[p] and sets bit ids[p] of an expert
// bitset in LDS (a wave's LDS operations complete in order, so no barrier is needed). An
// expert with more than NPC pairs (possible when n > NPC) takes two chunks: its first NPC
// pairs in pair order, then the rest; the lane that arrives as its (NPC+1)-th pair at an
// LDS counter marks it in a second bitset. Chunks are the experts present in ascending id
// order, each followed by its second chunk if marked: a scan of the words' chunk counts
// finds the word holding chunk c and a walk over its bits the expert and part. The
// chunk's pairs are the lanes holding that expert (a ballot). This saves the routing
// kernel its grouping and work list, which sit on the critical path there. With `offsets`
// given, workgroup 0 writes the routing's expert offsets and pair index (the grouping)
// while the other workgroups stream, and item i runs on workgroup i + 1.
constexpr int kExpertWords = MOE_MAX_EXPERTS / 32;
static_assert(kExpertWords <= kWave, "one bitset word per lane");

template <int NPC>
struct IdsChunk {
  int e, np, nch;
  int pid[NPC];
};

// s_bits: 2*kExpertWords words of LDS; s_cnt: MOE_MAX_EXPERTS ints (used when split).
template <int NPC>
__device__ __forceinline__ IdsChunk<NPC> chunk_from_ids(const int32_t* __restrict__ topk_ids,
                                                        int P, int c, int lane, uint32_t* s_bits,
                                                        int* s_cnt, bool split) {
  const int idv = lane < P ? topk_ids[lane] : -1;
  uint32_t* s_two = s_bits + kExpertWords;
  if (lane < kExpertWords) {
    s_bits[lane] = 0u;
    s_two[lane] = 0u;
  }
  if (split && lane < P) s_cnt[idv] = 0;
  if (lane < P) atomicOr(&s_bits[idv >> 5], 1u << (idv & 31));
  if (split && lane < P && atomicAdd(&s_cnt[idv], 1) == NPC)
    atomicOr(&s_two[idv >> 5], 1u << (idv & 31));
  const uint32_t word = lane < kExpertWords ? s_bits[lane] : 0u;
  const uint32_t two = lane < kExpertWords ? s_two[lane] : 0u;
  const int cnt = __popc(word) + __popc(two);  // chunks of the experts in this word
  const int incl = wave_inclusive_scan(cnt);
  IdsChunk<NPC> ch;
  ch.nch = __builtin_amdgcn_readlane(incl, kWave - 1);
  const uint64_t hit = __ballot(incl > c && incl - cnt <= c);  // the word holding chunk c
  const int w = hit ? __builtin_ctzll(hit) : 0;
  uint32_t wb = (uint32_t)__builtin_amdgcn_readlane((int)word, w);
  const uint32_t wb2 = (uint32_t)__builtin_amdgcn_readlane((int)two, w);
  int skip = c - (__builtin_amdgcn_readlane(incl, w) - __builtin_amdgcn_readlane(cnt, w));
  int bit = 0, part = 0;
  while (wb) {  // experts of the word in ascending order, 1 or 2 chunks each
    bit = __builtin_ctz(wb);
    const int take = 1 + (int)((wb2 >> bit) & 1u);
    if (skip < take) {
      part = skip;
      break;
    }
    skip -= take;
    wb &= wb - 1;
  }
  ch.e = 32 * w + bit;  // past the last chunk: some expert present, never used
  uint64_t pm = __ballot(lane < P && idv == ch.e);
  if (part) {
#pragma unroll
    for (int i = 0; i < NPC; ++i) pm &= pm - 1;
  }
  ch.np = min(__popcll(pm), NPC);
#pragma unroll
  for (int j = 0; j < NPC; ++j) {  // slots past np repeat the last pair
    ch.pid[j] = pm ? __builtin_ctzll(pm) : (j ? ch.pid[j - 1] : 0);
    if (j + 1 < ch.np) pm &= pm - 1;
  }
  return ch;
}

template <int BITS, int NPC, int WAVES, int ROWS, bool DBG, bool IDS>
__global__ __launch_bounds__((GuShape<WAVES, ROWS>::kThreads)) __attribute__((
    amdgpu_waves_per_eu(gu_waves_per_eu(WAVES, ROWS, NPC, DBG)))) void k_gateup(
    const uint32_t* __restrict__ gcodes, const uint32_t* __restrict__ gsm,
    const uint32_t* __restrict__ ucodes, const uint32_t* __restrict__ usm, int d, int f,
    const int* __restrict__ chunks, const int* __restrict__ nchunks, const int8_t* __restrict__ xq,
    const double2* __restrict__ xsc, int8_t* __restrict__ hq, double2* __restrict__ hsc,
    const int32_t* __restrict__ topk_ids, int k, int P, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ pair_index, const uint32_t* __restrict__ sgcodes,
    const uint32_t* __restrict__ sgsm, const uint32_t* __restrict__ sucodes,
    const uint32_t* __restrict__ susm, int n, float* __restrict__ hf, DecodeDebug dbg) {
  using S = GuShape<WAVES, ROWS>;
  static_assert(ROWS == 16 || ROWS == 32, "item rows");
  __shared__ double red[WAVES][NPC][ROWS];
  __shared__ int4 s_act_raw[ActLds<NPC, kGuGroup, S::kThreads>::kPadded];
  __shared__ uint32_t s_bits[2 * kExpertWords];
  __shared__ int s_cnt[IDS ? MOE_MAX_EXPERTS : 1];
  int4 (*s_act)[kGuGroup][3] = reinterpret_cast<int4 (*)[kGuGroup][3]>(s_act_raw);
  const int nbd = d / 32, nbf = f / 32;
  const int ntiles = f / ROWS;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int mat = wave / S::kKWaves;  // 0: gate, 1: up
  const int ke = S::kPW * (wave % S::kKWaves) + lane / ROWS;  // reduction-axis part
  const int rl = lane % ROWS;
  // One item per workgroup: the grid covers the largest possible item count and the
  // workgroups past the live count exit. (A loop over items would make the compiler's wait
  // counts conservative at its head: the first weight requests would wait for the
  // activation staging.) Without IDS, scalar loads of a chunk's work record give expert,
  // pair and token ids.
  int e, np, pid[NPC];
  RowSet<NPC> rows;
  int item = blockIdx.x, nch;
  if (IDS) {
    if (offsets) {
      if (blockIdx.x == 0) {  // the grouping of the routing outputs
        int* s_ids = reinterpret_cast<int*>(s_act_raw);
        if (tid < P) s_ids[tid] = topk_ids[tid];
        __syncthreads();
        group_tiny(s_ids, P, E, offsets, pair_index);
        return;
      }
      --item;
    }
    // 16-row items: the two halves of a 32-row block share the 128-byte lines of their
    // scale/min words, so they run on one XCD (one L2): workgroups are dealt to the 8 XCDs
    // in turn, and items 2m and 2m+1 of every 16 go to workgroups 8 apart (a bijection on
    // each run of 16; the grid is a multiple of 16)
    if (ROWS == 16) item = (item & ~15) | ((item & 7) << 1) | ((item >> 3) & 1);
    // wave 0 derives the chunk and hands it to the others through LDS (a derivation in
    // every wave costs more: all waves of all workgroups would read the same ids). The
    // weight pointers are fetched first, during the derivation (a pointer used on one side
    // of a select would be fetched inside a branch, after the barrier).
    // t = p / k as a multiply-high by ceil(2^32 / k), exact while p * k < 2^32 (here p < 72)
    uint32_t kmul = 0xffffffffu / (uint32_t)k + 1u;
    asm volatile("" : "+s"(gcodes), "+s"(gsm), "+s"(ucodes), "+s"(usm), "+s"(sgcodes),
                 "+s"(sgsm), "+s"(sucodes), "+s"(susm), "+s"(xq), "+s"(xsc), "+s"(kmul));
    __shared__ IdsChunk<NPC> s_ch;
    if (wave == 0) {
      IdsChunk<NPC> c0 =
          chunk_from_ids<NPC>(topk_ids, P, item / ntiles, lane, s_bits, s_cnt, n > NPC);
      if (sgcodes) {  // the shared expert: chunks of NPC tokens after the routed ones
        const int ns = (n + NPC - 1) / NPC, sc = item / ntiles - c0.nch;
        if (sc >= 0 && sc < ns) {
          c0.e = -1;
          c0.np = min(NPC, n - sc * NPC);
#pragma unroll
          for (int j = 0; j < NPC; ++j) c0.pid[j] = P + sc * NPC + min(j, c0.np - 1);
        }
        c0.nch += ns;
      }
      if (lane == 0) s_ch = c0;
    }
    __syncthreads();
    IdsChunk<NPC> ch;
    ch.e = __builtin_amdgcn_readfirstlane(s_ch.e);
    ch.np = __builtin_amdgcn_readfirstlane(s_ch.np);
    ch.nch = __builtin_amdgcn_readfirstlane(s_ch.nch);
#pragma unroll
    for (int j = 0; j < NPC; ++j) ch.pid[j] = __builtin_amdgcn_readfirstlane(s_ch.pid[j]);
    e = ch.e;
    np = ch.np;
    nch = ch.nch;
    // activation row: the token of the pair, taken for every pair and pinned, so that the
    // select stays a select (a division feeding one side of it would be moved into a
    // branch of its own ahead of the first weight request)
#pragma unroll
    for (int j = 0; j < NPC; ++j) {
      pid[j] = ch.pid[j];
      int tq = k == 1 ? pid[j] : (int)__umulhi((uint32_t)pid[j], kmul);
      asm volatile("" : "+s"(tq));
      rows.r[j] = pid[j] < P ? tq : pid[j] - P;
    }
  } else {
    // The record, the live chunk count and the weight pointers are fetched together: the
    // empty asm needs all of them, so no load is sunk behind the item test (which would
    // chain two or three round trips before the first weight request). 16-row items are
    // permuted as above; the grid rounded up to 16 may pass the last record, so the index
    // is clamped to the P+1 records of the work list (such items exit below).
    if (ROWS == 16) item = (item & ~15) | ((item & 7) << 1) | ((item >> 3) & 1);
    const int* rec = chunks + (size_t)min(item / ntiles, P) * kChunkInts;
    e = load_uniform(rec);
    np = load_uniform(rec + 2);
#pragma unroll
    for (int j = 0; j < NPC; ++j) {
      pid[j] = load_uniform(rec + 4 + j);
      rows.r[j] = load_uniform(rec + 4 + kMaxChunkPairs + j);
    }
    nch = load_uniform(nchunks);
    asm volatile("" : "+s"(nch) : "s"(e), "s"(np), "s"(gcodes), "s"(gsm), "s"(ucodes), "s"(usm));
  }
  const int nitems = nch * ntiles;
  if (item < nitems) {
    const int tile = item % ntiles;
    const int r = tile * ROWS + rl;
    double acc[NPC];
#pragma unroll
    for (int j = 0; j < NPC; ++j) acc[j] = 0.0;
    // this expert's codes and scale/min of this matrix (e < 0: the shared expert)
    const uint32_t* __restrict__ codes = mat ? ucodes : gcodes;
    const uint32_t* __restrict__ smp = mat ? usm : gsm;
    const uint32_t* cbase = e < 0 ? (mat ? sucodes : sgcodes) : codes + (size_t)e * nbd * f * BITS;
    const uint32_t* sbase = e < 0 ? (mat ? susm : sgsm) : smp + (size_t)e * nbd * f;
    const __amdgpu_buffer_rsrc_t rs_c = buffer_rsrc(cbase, (uint32_t)(nbd * f * BITS * 4));
    const __amdgpu_buffer_rsrc_t rs_s = buffer_rsrc(sbase, (uint32_t)(nbd * f * 4));
    uint32_t w[S::kUnroll][BITS], smw[S::kUnroll];
    for (int g0 = 0; g0 < nbd; g0 += kGuGroup) {
      __syncthreads();  // earlier readers of s_act are done
      act_load_lds<NPC, kGuGroup, S::kThreads>(s_act_raw, xq, xsc, rows, np, g0, nbd, d, wave,
                                              lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < S::kUnroll; ++u) {
        // blocks past the end (partial last group) re-read the last block; never used
        // ke differs between the two halves of the wave, so the whole offset goes into the
        // per-lane offset (a lane-varying scalar offset would split every load in two)
        const int b = min(g0 + ke + S::kSplit * u, nbd - 1);
        BlockLoad<BITS>::load(rs_c, (b * f + r) * BITS * 4, 0, w[u]);
        smw[u] = __builtin_amdgcn_raw_buffer_load_b32(rs_s, (b * f + r) * 4, 0, kNt);
      }
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<2 * S::kUnroll>();  // this wave's staging loads have landed
      barrier_after_lds_dma();
      // the block terms of the chunk's first NP pairs (all of them when NP == np)
      auto blocks = [&](auto np_c) {
        constexpr int NP = decltype(np_c)::value;
#pragma unroll
        for (int u = 0; u < S::kUnroll; ++u) {
          const int bb = ke + S::kSplit * u;
          const int b = g0 + bb;
          if (b < nbd) {
            const double sc_w = half_bits_to_double(smw[u] & 0xffffu);
            const double mn_w = half_bits_to_double(smw[u] >> 16);
#pragma unroll
            for (int j = 0; j < NP; ++j) {
              if (NP == NPC && j >= np) continue;
              const int4 a0 = s_act[j][bb][0], a1 = s_act[j][bb][1], scv = s_act[j][bb][2];
              const int a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
              double2 sc;
              __builtin_memcpy(&sc, &scv, 16);
              const int dt = block_dot<BITS>(w[u], a);
              // both block terms are exact in binary64, so fma rounds exactly like acc + term
              acc[j] = __builtin_fma(sc_w * sc.x, (double)dt, acc[j]);
              acc[j] = __builtin_fma(mn_w, sc.y, acc[j]);
              if (DBG) {
                int32_t* dots = mat ? dbg.up_dots : dbg.gate_dots;
                if (dots) dots[((size_t)pid[j] * f + r) * nbd + b] = dt;
              }
            }
          }
        }
      };
      // The int8 matrix-core form of the block dots (2-bit work-list items of at least
      // kGuMmaFull pairs; chunks of kGuMmaHalf to 4 pairs take the half-slot form below).
      // One v_mfma_i32_32x32x32_i8 computes the exact int32 dots of one block for the 32
      // rows of the wave's matrix (N) and up to 32 pair slots (M; slots past the chunk
      // read a valid slot and are discarded), K = the block's 32 codes. Operand lanes:
      // row (B) or pair (A) lane % 32, codes 16 * (lane / 32) + 0..15;
      // result register i (< 4) of lane l holds pair 4 * (l / 32) + i of row l % 32. The
      // lanes' loads hold the two 16-code words of their own block, lanes 0..31 block b0
      // and lanes 32..63 block b0 + 1; one cross-half swap turns them into the B operands
      // of both blocks (word h of each for the lanes of half h), and another gives every
      // lane the scale/min words of both. The code bytes of a word follow the activation
      // permutation (byte m of (word >> 2s) & 0x03030303 is code 4m + s), so A is the
      // staged activation half as it stands. The binary64 block terms follow as in the
      // dot4 form, for the lane's four pair slots.
      // (a whole group of blocks without a test per block, so that the compiler can issue
      // the next block's matrix-core op ahead of this block's terms; a partial last group
      // tests each block)
      auto mma_blocks = [&](auto partial_c) {
        constexpr bool kPartial = decltype(partial_c)::value != 0;
        const int h = lane >> 5;
        const int am = min(lane & 31, NPC - 1);
        const i32x16_t zero = {};
#pragma unroll
        for (int u = 0; u < S::kUnroll; ++u) {
          const int b0 = g0 + S::kPW * (wave % S::kKWaves) + S::kSplit * u;  // wave-uniform
          const auto cw = __builtin_amdgcn_permlane32_swap(w[u][0], w[u][1], false, false);
          const auto sw = __builtin_amdgcn_permlane32_swap(smw[u], smw[u], false, false);
          // both blocks' matrix-core ops first, then their terms
          i32x16_t dots[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int bb = b0 + q - g0;
            const uint32_t word = q ? cw[1] : cw[0];
            const i32x4_t bop = {(int)(word & 0x03030303u), (int)((word >> 2) & 0x03030303u),
                                 (int)((word >> 4) & 0x03030303u),
                                 (int)((word >> 6) & 0x03030303u)};
            const int4 av = s_act[am][min(bb, kGuGroup - 1)][h];
            const i32x4_t aop = {av.x, av.y, av.z, av.w};
            dots[q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, bop, zero, 0, 0, 0);
          }
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int b = b0 + q;
            if (!kPartial || b < nbd) {
              const int bb = b - g0;
              const uint32_t smq = q ? sw[1] : sw[0];
              const double sc_w = half_bits_to_double(smq & 0xffffu);
              const double mn_w = half_bits_to_double(smq >> 16);
              double2 sc[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int4 scv = s_act[4 * h + i][bb][2];
                __builtin_memcpy(&sc[i], &scv, 16);
              }
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                acc[i] = __builtin_fma(sc_w * sc[i].x, (double)dots[q][i], acc[i]);
                acc[i] = __builtin_fma(mn_w, sc[i].y, acc[i]);
                if (DBG) {
                  int32_t* dd = mat ? dbg.up_dots : dbg.gate_dots;
                  const int j = 4 * h + i;
                  int pj = pid[0];
#pragma unroll
                  for (int j2 = 1; j2 < NPC; ++j2) pj = j == j2 ? pid[j2] : pj;
                  if (dd && j < np) dd[((size_t)pj * f + r) * nbd + b] = dots[q][i];
                }
              }
            }
          }
        }
      };
      // The half-slot form for chunks of at most 4 pairs: only result registers 0..3 of
      // lanes 0..31 (pair slots 0..3) hold pairs, so one cross-half swap per register moves
      // the second block's slots 0..3 into lanes 32..63. Lane l then holds the dots of pair
      // slots 0..3 of its own loaded block b0 + l / 32 (whose scale/min word it read) and
      // row l % 32, and the block terms run once per lane for both blocks; the two halves'
      // sums of a row meet in the final reduction like the dot4 form's parts.
      auto mma_half_blocks = [&](auto partial_c) {
        constexpr bool kPartial = decltype(partial_c)::value != 0;
        const int h = lane >> 5;
        const int am = min(lane & 31, NPC - 1);
        const i32x16_t zero = {};
#pragma unroll
        for (int u = 0; u < S::kUnroll; ++u) {
          const int b0 = g0 + S::kPW * (wave % S::kKWaves) + S::kSplit * u;  // wave-uniform
          const auto cw = __builtin_amdgcn_permlane32_swap(w[u][0], w[u][1], false, false);
          i32x16_t dots[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int bb = b0 + q - g0;
            const uint32_t word = q ? cw[1] : cw[0];
            const i32x4_t bop = {(int)(word & 0x03030303u), (int)((word >> 2) & 0x03030303u),
                                 (int)((word >> 4) & 0x03030303u),
                                 (int)((word >> 6) & 0x03030303u)};
            const int4 av = s_act[am][min(bb, kGuGroup - 1)][h];
            const i32x4_t aop = {av.x, av.y, av.z, av.w};
            dots[q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, bop, zero, 0, 0, 0);
          }
          int dt[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            dt[i] = (int)__builtin_amdgcn_permlane32_swap((uint32_t)dots[0][i],
                                                          (uint32_t)dots[1][i], false, false)[0];
          const int b = b0 + h;  // the lane's own block
          if (!kPartial || b < nbd) {
            const int bb = b - g0;
            const double sc_w = half_bits_to_double(smw[u] & 0xffffu);
            const double mn_w = half_bits_to_double(smw[u] >> 16);
            double2 sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int4 scv = s_act[i][bb][2];
              __builtin_memcpy(&sc[i], &scv, 16);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              acc[i] = __builtin_fma(sc_w * sc[i].x, (double)dt[i], acc[i]);
              acc[i] = __builtin_fma(mn_w, sc[i].y, acc[i]);
              if (DBG) {
                int32_t* dd = mat ? dbg.up_dots : dbg.gate_dots;
                int pj = pid[0];
#pragma unroll
                for (int j2 = 1; j2 < 4; ++j2) pj = i == j2 ? pid[j2] : pj;
                if (dd && i < np) dd[((size_t)pj * f + r) * nbd + b] = dt[i];
              }
            }
          }
        }
      };
      // Other 2-bit 32-row work-list items take one dot4 variant per chunk size, without a
      // branch per pair slot. The 4-bit and the ids-path instances keep the branches: the
      // variants would spill there.
      if constexpr (gu_has_mma<BITS, NPC, WAVES, ROWS, IDS>()) {
        if (np >= kGuMmaFull) {
          if (g0 + kGuGroup <= nbd)
            mma_blocks(Int<0>{});
          else
            mma_blocks(Int<1>{});
        } else if (np >= kGuMmaHalf) {
          if (g0 + kGuGroup <= nbd)
            mma_half_blocks(Int<0>{});
          else
            mma_half_blocks(Int<1>{});
        } else {
          switch (np) {
            case 1: blocks(Int<1>{}); break;
            case 2: blocks(Int<2>{}); break;
            default: blocks(Int<3>{}); break;
          }
        }
      } else {
        blocks(Int<NPC>{});
      }
      // Blocks past the reduction axis leave their loads unused; the empty asm takes every
      // loaded register, so no load is outstanding at the loop's back edge (the compiler
      // would otherwise wait for all loads, the new group's staging included, at the head).
#pragma unroll
      for (int u = 0; u < S::kUnroll; ++u) {
#pragma unroll
        for (int q = 0; q < BITS; ++q) asm volatile("" ::"v"(w[u][q]));
        asm volatile("" ::"v"(smw[u]));
      }
    }
    if (gu_has_mma<BITS, NPC, WAVES, ROWS, IDS>() && np >= kGuMmaFull) {
      // matrix-core form: lane l holds the sums of pair slots 4 * (l / 32) + i of row l % 32
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * (lane >> 5) + i;
        if (j < np) red[wave][j][rl] = acc[i];
      }
    } else {
      // the reduction parts of a row sit in lanes l, l+ROWS, ... (every lane of the row
      // ends with the same sum: fp addition commutes)
#pragma unroll
      for (int j = 0; j < NPC; ++j) {
#pragma unroll
        for (int m = ROWS; m < kWave; m *= 2) {
          const double o = __shfl_xor(acc[j], m);
          acc[j] = (lane & m) ? o + acc[j] : acc[j] + o;
        }
      }
      if (lane < ROWS) {
#pragma unroll
        for (int j = 0; j < NPC; ++j)
          if (j < np) red[wave][j][rl] = acc[j];
      }
    }
    __syncthreads();
    if (ROWS == 16 && wave == 0) {
      // lane l takes pair slots l/16, l/16 + 4, ... at row l%16; h leaves in fp32
      const int js = lane / ROWS;
#pragma unroll
      for (int jj = 0; jj < (NPC + S::kPW - 1) / S::kPW; ++jj) {
        const int j = S::kPW * jj + js;
        if (j < np) {
          // sums over the waves of each matrix, in wave order
          double g = red[0][j][rl], u = red[S::kKWaves][j][rl];
#pragma unroll
          for (int w2 = 1; w2 < S::kKWaves; ++w2) {
            g += red[w2][j][rl];
            u += red[S::kKWaves + w2][j][rl];
          }
          const double silu = g / (1.0 + exp(-g));
          const float h = (float)(silu * u);
          int pj = pid[0];
#pragma unroll
          for (int j2 = 1; j2 < NPC; ++j2) pj = j == j2 ? pid[j2] : pj;
          hf[(size_t)pj * f + r] = h;
          if (DBG) {
            if (dbg.g) dbg.g[(size_t)pj * f + r] = (float)g;
            if (dbg.u) dbg.u[(size_t)pj * f + r] = (float)u;
            if (dbg.h) dbg.h[(size_t)pj * f + r] = h;
          }
        }
      }
    }
    if (ROWS == 32 && wave == 0) {
      // lanes 0..31 take even pair slots, lanes 32..63 odd ones; each half quantizes the
      // 32 rows of its pair (and with hf given also stores h in fp32)
      const int hh = lane / kGuRows;
#pragma unroll
      for (int jj = 0; jj < (NPC + 1) / 2; ++jj) {
        const int j = 2 * jj + hh;
        if (j < np) {
          // sums over the four waves of each matrix, in wave order
          double g = red[0][j][rl], u = red[S::kKWaves][j][rl];
#pragma unroll
          for (int w2 = 1; w2 < S::kKWaves; ++w2) {
            g += red[w2][j][rl];
            u += red[S::kKWaves + w2][j][rl];
          }
          const double silu = g / (1.0 + exp(-g));
          const float h = (float)(silu * u);
          float scale;
          int qsum;
          const int q = quant_half_wave(h, scale, qsum);
          const int p = pid[0];
          int pj = p;
#pragma unroll
          for (int j2 = 1; j2 < NPC; ++j2) pj = j == j2 ? pid[j2] : pj;
          hq[(size_t)pj * f + 32 * tile + act_byte_pos<BITS>(rl)] = (int8_t)q;
          if (hf) hf[(size_t)pj * f + r] = h;
          if (rl == 0) hsc[(size_t)pj * nbf + tile] = make_double2((double)scale, (double)scale * qsum);
          if (DBG) {
            if (dbg.g) dbg.g[(size_t)pj * f + r] = (float)g;
            if (dbg.u) dbg.u[(size_t)pj * f + r] = (float)u;
            if (dbg.h) dbg.h[(size_t)pj * f + r] = h;
            if (dbg.hq) dbg.hq[(size_t)pj * f + r] = (int8_t)q;
            if (dbg.hs && rl == 0) dbg.hs[(size_t)pj * nbf + tile] = scale;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- down projection

constexpr int kDnWaves = 4;
constexpr int kDnThreads = kDnWaves * kWave;
// MMA: the instance with the matrix-core forms (chunks of kDnMmaHalf or more pairs).
// It needs 144 registers a lane (three waves a SIMD against five without), which costs
// the dot4 form of small chunks more than the matrix cores save; the host takes it when
// the window averages kMmaMinPairs or more pairs per busy expert.
template <int BITS, int NPC, bool MMA>
constexpr bool dn_has_mma() {
  return MMA && BITS == 2 && NPC == 8;
}

template <int BITS, int NPC, bool DBG, bool MMA>
__global__ __launch_bounds__(kDnThreads) void k_down(
    const uint32_t* __restrict__ dcodes, const uint32_t* __restrict__ dsm, int d, int f,
    const int* __restrict__ chunks, const int* __restrict__ nchunks, const int8_t* __restrict__ hq,
    const double2* __restrict__ hsc, float* __restrict__ y, DecodeDebug dbg) {
  constexpr int kUnroll = 8;
  constexpr int kDnGroup = kDnWaves * kUnroll;  // blocks per weight-load group
  constexpr int kDnStage = 2 * kDnGroup;        // blocks per activation staging
  __shared__ double red[kDnWaves][NPC][kWave];
  __shared__ int4 s_act_raw[ActLds<NPC, kDnStage, kDnThreads>::kPadded];
  int4 (*s_act)[kDnStage][3] = reinterpret_cast<int4 (*)[kDnStage][3]>(s_act_raw);
  const int nbf = f / 32;
  const int ntiles = (d + kWave - 1) / kWave;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  int item = blockIdx.x;  // first record read with the count: see k_gateup
  const int nitems = load_uniform(nchunks) * ntiles;
  int e, np, pid[NPC];
  const int* rec_rows;  // pair ids of the chunk (rows of hq)
  auto read_record = [&](int it) {
    const int* rec = chunks + (size_t)(it / ntiles) * kChunkInts;
    rec_rows = rec + 4;
    e = load_uniform(rec);
    np = load_uniform(rec + 2);
#pragma unroll
    for (int j = 0; j < NPC; ++j) pid[j] = load_uniform(rec + 4 + j);
  };
  read_record(item);
  for (; item < nitems; item += gridDim.x) {
    if (item != (int)blockIdx.x) read_record(item);
    const int tile = item % ntiles;
    const int r = tile * kWave + lane;
    const bool rvalid = r < d;
    const int rr = rvalid ? r : 0;
    double ay[NPC];
#pragma unroll
    for (int j = 0; j < NPC; ++j) ay[j] = 0.0;
    const __amdgpu_buffer_rsrc_t rs_c =
        buffer_rsrc(dcodes + (size_t)e * nbf * d * BITS, (uint32_t)(nbf * d * BITS * 4));
    const __amdgpu_buffer_rsrc_t rs_s = buffer_rsrc(dsm + (size_t)e * nbf * d, (uint32_t)(nbf * d * 4));
    uint32_t dw[kUnroll][BITS], smw[kUnroll];
    auto load_weights = [&](int g0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int b = min(g0 + wave + kDnWaves * u, nbf - 1);  // see k_gateup
        BlockLoad<BITS>::load(rs_c, rr * BITS * 4, b * d * BITS * 4, dw[u]);
        smw[u] = __builtin_amdgcn_raw_buffer_load_b32(rs_s, rr * 4, b * d * 4, kNt);
      }
    };
    // Matrix-core form of the block dots (2-bit chunks of at least kDnMmaFull pairs; the
    // lane layout of k_gateup's): per block, two v_mfma_i32_32x32x32_i8 give the exact
    // dots of the wave's 64 rows (N: rows 0..31, then 32..63) for the pair slots (M). Every lane holds
    // both code words of its own row; one cross-half swap makes the B operands of the two
    // row halves (word h for the lanes of half h) and another the scale/min words of rows
    // lane % 32 and 32 + lane % 32. Lane l then carries pair slots 4 * (l / 32) + i of
    // those two rows.
    auto compute_mma = [&](int g0, int s0) {
      const int h = lane >> 5;
      const int am = min(lane & 31, NPC - 1);
      const i32x16_t zero = {};
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int b = g0 + wave + kDnWaves * u;  // wave-uniform
        const int bb = b - s0;
        if (b < nbf) {
          const auto cw = __builtin_amdgcn_permlane32_swap(dw[u][0], dw[u][1], false, false);
          const auto sw = __builtin_amdgcn_permlane32_swap(smw[u], smw[u], false, false);
          const int4 av = s_act[am][bb][h];
          const i32x4_t aop = {av.x, av.y, av.z, av.w};
          i32x16_t dots[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint32_t word = q ? cw[1] : cw[0];
            const i32x4_t bop = {(int)(word & 0x03030303u), (int)((word >> 2) & 0x03030303u),
                                 (int)((word >> 4) & 0x03030303u),
                                 (int)((word >> 6) & 0x03030303u)};
            dots[q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, bop, zero, 0, 0, 0);
          }
          double2 sc[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int4 scv = s_act[4 * h + i][bb][2];
            __builtin_memcpy(&sc[i], &scv, 16);
          }
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint32_t smq = q ? sw[1] : sw[0];
            const double s = half_bits_to_double(smq & 0xffffu);
            const double m = half_bits_to_double(smq >> 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              ay[4 * q + i] = __builtin_fma(s * sc[i].x, (double)dots[q][i], ay[4 * q + i]);
              ay[4 * q + i] = __builtin_fma(m, sc[i].y, ay[4 * q + i]);
              if (DBG && dbg.down_dots) {
                const int j = 4 * h + i, rq = tile * kWave + 32 * q + (lane & 31);
                int pj = pid[0];
#pragma unroll
                for (int j2 = 1; j2 < NPC; ++j2) pj = j == j2 ? pid[j2] : pj;
                if (j < np && rq < d) dbg.down_dots[((size_t)pj * d + rq) * nbf + b] = dots[q][i];
              }
            }
          }
        }
      }
    };
    // The half-slot form for chunks of at most 4 pairs: result registers 0..3 of lanes
    // 0..31 (pair slots 0..3) are the only ones holding pairs, so one cross-half swap per
    // register moves those of the second row half into lanes 32..63. Lane l then holds
    // pair slots 0..3 of row l of the tile (the dot4 form's layout) and its own loaded
    // scale/min word, and computes half as many block terms.
    auto compute_mma_half = [&](int g0, int s0) {
      const int h = lane >> 5;
      const int am = min(lane & 31, NPC - 1);
      const i32x16_t zero = {};
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int b = g0 + wave + kDnWaves * u;  // wave-uniform
        const int bb = b - s0;
        if (b < nbf) {
          const auto cw = __builtin_amdgcn_permlane32_swap(dw[u][0], dw[u][1], false, false);
          const int4 av = s_act[am][bb][h];
          const i32x4_t aop = {av.x, av.y, av.z, av.w};
          i32x16_t dots[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint32_t word = q ? cw[1] : cw[0];
            const i32x4_t bop = {(int)(word & 0x03030303u), (int)((word >> 2) & 0x03030303u),
                                 (int)((word >> 4) & 0x03030303u),
                                 (int)((word >> 6) & 0x03030303u)};
            dots[q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, bop, zero, 0, 0, 0);
          }
          const double s = half_bits_to_double(smw[u] & 0xffffu);
          const double m = half_bits_to_double(smw[u] >> 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int dd = (int)__builtin_amdgcn_permlane32_swap((uint32_t)dots[0][i],
                                                                 (uint32_t)dots[1][i], false,
                                                                 false)[0];
            const int4 scv = s_act[i][bb][2];
            double2 sc;
            __builtin_memcpy(&sc, &scv, 16);
            ay[i] = __builtin_fma(s * sc.x, (double)dd, ay[i]);
            ay[i] = __builtin_fma(m, sc.y, ay[i]);
            if (DBG && rvalid && dbg.down_dots && i < np) {
              int pj = pid[0];
#pragma unroll
              for (int j2 = 1; j2 < 4; ++j2) pj = i == j2 ? pid[j2] : pj;
              dbg.down_dots[((size_t)pj * d + r) * nbf + b] = dd;
            }
          }
        }
      }
    };
    auto compute = [&](int g0, int s0) {
      if constexpr (dn_has_mma<BITS, NPC, MMA>()) {
        if (np >= kDnMmaFull) {
          compute_mma(g0, s0);
          return;
        }
        if (np >= kDnMmaHalf) {
          compute_mma_half(g0, s0);
          return;
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int b = g0 + wave + kDnWaves * u;
        const int bb = b - s0;
        if (b < nbf) {
          const double s = half_bits_to_double(smw[u] & 0xffffu);
          const double m = half_bits_to_double(smw[u] >> 16);
#pragma unroll
          for (int j = 0; j < NPC; ++j) {
            if (j < np) {
              const int4 a0 = s_act[j][bb][0], a1 = s_act[j][bb][1], scv = s_act[j][bb][2];
              const int a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
              double2 sc;
              __builtin_memcpy(&sc, &scv, 16);
              const int dd = block_dot<BITS>(dw[u], a);
              ay[j] = __builtin_fma(s * sc.x, (double)dd, ay[j]);  // exact terms: see k_gateup
              ay[j] = __builtin_fma(m, sc.y, ay[j]);
              if (DBG && rvalid && dbg.down_dots)
                dbg.down_dots[((size_t)pid[j] * d + r) * nbf + b] = dd;
            }
          }
        }
      }
    };
    for (int s0 = 0; s0 < nbf; s0 += kDnStage) {
      __syncthreads();  // earlier readers of s_act are done
      act_load_lds<NPC, kDnStage, kDnThreads>(s_act_raw, hq, hsc, rec_rows, np, s0, nbf, f, wave, lane);
      __builtin_amdgcn_sched_barrier(0);  // see k_gateup
      load_weights(s0);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<2 * kUnroll>();
      barrier_after_lds_dma();
      compute(s0, s0);
      for (int g0 = s0 + kDnGroup; g0 < min(nbf, s0 + kDnStage); g0 += kDnGroup) {
        load_weights(g0);
        compute(g0, s0);
      }
    }
    __syncthreads();
    if (dn_has_mma<BITS, NPC, MMA>() && np >= kDnMmaFull) {
      // matrix-core form: slot 4 * (lane / 32) + i of rows lane % 32 and 32 + lane % 32
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * (lane >> 5) + i;
          if (j < np) red[wave][j][32 * q + (lane & 31)] = ay[4 * q + i];
        }
    } else {
#pragma unroll
      for (int j = 0; j < NPC; ++j)
        if (j < np) red[wave][j][lane] = ay[j];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int j = 0; j < NPC; ++j) {
        if (j < np && rvalid) {
          const double v = reduce_waves<NPC, kDnWaves>(red, j, lane);
          y[(size_t)pid[j] * d + r] = (float)v;  // the pair output, rounded once
          if (DBG && dbg.y) dbg.y[(size_t)pid[j] * d + r] = (float)v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- combine

__global__ __launch_bounds__(kThreads) void k_combine(const float* __restrict__ y,
                                                      const float* __restrict__ w, int n, int d,
                                                      int k, float* residual) {
  const int gid = blockIdx.x * kThreads + threadIdx.x;
  if (gid >= n * d) return;
  const int t = gid / d, c = gid % d;
  double acc = 0.0;
  for (int j = 0; j < k; ++j)
    acc += (double)w[(size_t)t * k + j] * (double)y[((size_t)t * k + j) * d + c];
  residual[gid] = (float)((double)residual[gid] + acc);
}

// ---------------------------------------------------------------- down + combine, token-major
//
// For small windows the down projection is organised by token instead of by expert: a
// workgroup owns (token t, R rows of d; R = 32, or 8 and 16 for one and two tokens),
// computes those rows of the down outputs of all k pairs of t and applies the routing-
// weighted combine itself (slot order, binary64), so the pair outputs never leave the
// workgroup and the combine needs no launch of its own. An expert shared by several
// tokens of the window is read once per token; the row tiles are laid out so that all
// tokens of one row tile run on one XCD, whose L2 then serves the repeats. Lane l of wave
// w owns row l%R and the experts j = l/R, l/R + 64/R, ... of the token, for blocks w,
// w+8, ... of f.
//
// Order of requests: the experts of the lane's pairs, the token's residual values and its
// h (fp32) go out first; then all U*I weight blocks of the lane (the whole token at
// f = 768, k = 10), then the routing weights (scalar loads, needed only at the end). The
// wave waits only for the h loads, quantizes h block by block into LDS (every workgroup
// of the token does this for itself, while its weights are in flight) and meets the
// barrier; each block's dots start as soon as that block has landed. The 8 waves' partial
// sums meet in LDS.
constexpr int kDtWaves = 8;
constexpr int kDtThreads = kDtWaves * kWave;
constexpr int kDtMaxK = 16;       // top-k handled by this path
constexpr int kDtMaxBlocks = 32;  // f/32 handled by this path
constexpr int kDtMaxTokens = 16;  // window tokens handled by this path
constexpr int kDtSlots = 16;      // weight blocks in flight per lane
constexpr int kDtSlotsShared = 18;  // the same with one more slot (a shared expert)
constexpr int kDtStage = kDtMaxK * kDtMaxBlocks * 3;  // 16-byte LDS entries of quantized h
static_assert(kDtMaxK * kDtMaxBlocks <= kDtThreads, "one h block per thread");

template <int BITS, int U, int I, bool SH, bool EQ, bool DBG, int R>
__global__ __launch_bounds__(kDtThreads) void k_down_tok(
    const uint32_t* __restrict__ dcodes, const uint32_t* __restrict__ dsm, int d, int f, int k,
    int n, const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_w,
    const float* __restrict__ hf, float* residual, const uint32_t* __restrict__ sdcodes,
    const uint32_t* __restrict__ sdsm, DecodeDebug dbg) {
  // slots j < k: the routed pairs t*k + j; with SH, slot k: the shared expert, pair n*k + t,
  // weight 1. R rows a workgroup; lane group h = lane / R takes slots j = h, h + G, ... (G =
  // 64/R groups, I slots a lane). Without SH every shared-slot select folds away.
  static_assert(R == 8 || R == 16 || R == 32, "row tile");
  constexpr int G = kWave / R;
  const int ke = SH ? k + 1 : k;
  __shared__ int4 s_act[kDtStage];
  __shared__ double red[kDtWaves][kDtMaxK + 1][R];  // slot kDtMaxK: unused pairs
  const int nbf = f / 32, nrt = d / R;
  const int per = (nrt + 7) / 8;  // row tiles per XCD
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int rt = xcd * per + slot / n, t = slot % n;
  if (slot >= per * n || rt >= nrt) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r = lane % R, h = lane / R;
  const int row = rt * R + r;
  const int P = n * k;
  auto pair_of = [&](int j) { return SH && j >= k ? (size_t)P + t : (size_t)t * k + j; };

  // experts of the lane's pairs (-1: the shared expert; slots past ke repeat slot ke-1,
  // never used; the id load is unconditional, its value selected)
  int eid[I];
#pragma unroll
  for (int i = 0; i < I; ++i) {
    const int j = min(h + G * i, ke - 1);
    const int id = topk_ids[(size_t)t * k + min(j, k - 1)];
    eid[i] = SH && j >= k ? -1 : id;
  }
  const bool epi = wave == 0 && lane < R;
  const float res0 = residual[(size_t)t * d + (epi ? row : rt * R)];

  // h of the token in fp32 into registers: thread q takes block q of the token's ke*nbf
  // (<= 512) blocks, slot j = q / nbf and rows 32b .. 32b+31 with b = q % nbf; threads past
  // the end read the last block again, never used. The block is quantized after the
  // weight requests, so the compiler's own wait for it leaves the weight loads in flight.
  const int nblk = ke * nbf;
  typedef float v4f __attribute__((ext_vector_type(4)));
  v4f hv[8];
  {
    const int q = min(tid, nblk - 1);
    const int j = q / nbf, b = q - j * nbf;
    const uintptr_t src = reinterpret_cast<uintptr_t>(hf + pair_of(j) * f + 32 * b);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      hv[i] = reinterpret_cast<const __attribute__((address_space(1))) v4f*>(src)[i];
  }
  // int8 quantization of the thread's block (the arithmetic of the gate/up epilogue of
  // 32-row items, in registers): LDS entry q = the 32 codes at their dot4 byte positions,
  // then (scale, scale*sum). Entries past ke*nbf stay unwritten; the blocks that would read
  // them are dropped below. (Every workgroup of the token quantizes all of its blocks.)
  // With EQ (grids of more workgroups than CUs) it runs before the weight requests, so its
  // registers are free while they are in flight and two workgroups fit a CU; otherwise
  // after them, where its wait for h leaves the weights in flight.
  auto quant_h = [&]() {
    if (tid < nblk) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[4 * i] = hv[i].x;
        v[4 * i + 1] = hv[i].y;
        v[4 * i + 2] = hv[i].z;
        v[4 * i + 3] = hv[i].w;
      }
      int qc[32];
      const float scale = quant_block32(v, qc);
      const int sum = code_sum32(qc);
      uint32_t words[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int pos = act_byte_pos<BITS>(i);
        words[pos / 4] |= ((uint32_t)qc[i] & 0xffu) << (8 * (pos % 4));
      }
      s_act[3 * tid] = make_int4((int)words[0], (int)words[1], (int)words[2], (int)words[3]);
      s_act[3 * tid + 1] = make_int4((int)words[4], (int)words[5], (int)words[6], (int)words[7]);
      reinterpret_cast<double2*>(s_act)[3 * tid + 2] =
          make_double2((double)scale, (double)scale * (double)sum);
      if (DBG && rt == 0) {  // one workgroup per token reports the codes
        const int j = tid / nbf, b = tid - j * nbf;
        if (dbg.hq) {
#pragma unroll
          for (int i = 0; i < 32; ++i) dbg.hq[pair_of(j) * f + 32 * b + i] = (int8_t)qc[i];
        }
        if (dbg.hs) dbg.hs[pair_of(j) * nbf + b] = scale;
      }
    }
  };
  if (EQ) quant_h();
  __builtin_amdgcn_sched_barrier(0);

  // all weight blocks of this lane (past ke or nbf: a valid block, never used)
  uint32_t w[I][U][BITS], smw[I][U];
#pragma unroll
  for (int i = 0; i < I; ++i) {
    const int e = eid[i];
    const uint32_t* cb = SH && e < 0 ? sdcodes : dcodes;
    const uint32_t* sb = SH && e < 0 ? sdsm : dsm;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = min(wave + 8 * u, nbf - 1);
      const size_t blk = ((size_t)(SH && e < 0 ? 0 : e) * nbf + b) * d + row;
      if (BITS == 4) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(cb + blk * 4));
        w[i][u][0] = v.x;
        w[i][u][1] = v.y;
        w[i][u][2 % BITS] = v.z;
        w[i][u][3 % BITS] = v.w;
      } else {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(cb + blk * 2));
        w[i][u][0] = v.x;
        w[i][u][1] = v.y;
      }
      smw[i][u] = __builtin_nontemporal_load(sb + blk);  // read once: see BlockLoad
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // routing weights of the token, for the combine (uniform: scalar loads, needed last)
  float sw[kDtMaxK];
#pragma unroll
  for (int j = 0; j < kDtMaxK; ++j)
    sw[j] = __int_as_float(
        load_uniform(reinterpret_cast<const int*>(topk_w) + (size_t)t * k + min(j, k - 1)));
  if (!EQ) quant_h();
  __syncthreads();

  // Every block is computed and the unused ones (past ke or nbf) are dropped by a select:
  // a weight load feeding only a guarded branch would be sunk into it, behind a full wait.
  // Unused blocks read LDS entries inside s_act (j < kDtMaxK, b < kDtMaxBlocks).
  double acc[I];
#pragma unroll
  for (int i = 0; i < I; ++i) {
    acc[i] = 0.0;
    const int j = h + G * i;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = wave + 8 * u;
      const bool use = j < ke && b < nbf;
      const int4* e3 = s_act + (min(j, kDtMaxK - 1) * nbf + b) * 3;
      const int4 a0 = e3[0], a1 = e3[1], scv = e3[2];
      const int a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      double2 sc;
      __builtin_memcpy(&sc, &scv, 16);
      const int dd = block_dot<BITS>(w[i][u], a);
      const double s = half_bits_to_double(smw[i][u] & 0xffffu);
      const double m = half_bits_to_double(smw[i][u] >> 16);
      // exact terms: see k_gateup
      const double v = __builtin_fma(m, sc.y, __builtin_fma(s * sc.x, (double)dd, acc[i]));
      acc[i] = use ? v : acc[i];
      if (DBG && use && dbg.down_dots) dbg.down_dots[(pair_of(j) * d + row) * nbf + b] = dd;
    }
    red[wave][j < ke ? j : kDtMaxK][r] = acc[i];  // unconditional: see above
  }
  __syncthreads();
  // Each (slot, row) output sums its 8 wave partials in wave order, one per thread
  // (ke*R <= 512: all at once), into LDS over the staged h, which nobody reads any more;
  // then R lanes combine the slots in slot order. (A 32-lane loop over both took 0.9 µs
  // of dependent adds.)
  double(*ys)[R] = reinterpret_cast<double(*)[R]>(s_act);
  static_assert(sizeof(double) * kDtMaxK * R <= sizeof(int4) * kDtStage, "ys fits");
  if (tid < ke * R) {
    const int j = tid / R, rr = tid % R;
    double y = red[0][j][rr];
#pragma unroll
    for (int w2 = 1; w2 < kDtWaves; ++w2) y += red[w2][j][rr];  // wave order
    ys[j][rr] = y;
    if (DBG && dbg.y) dbg.y[pair_of(j) * d + rt * R + rr] = (float)y;
  }
  __syncthreads();
  if (epi) {
    double tot = 0.0;
#pragma unroll
    for (int j = 0; j < kDtMaxK; ++j)  // slot order, the shared expert last
      if (j < ke) tot += (SH && j >= k ? 1.0 : (double)sw[j]) * ys[j][r];
    residual[(size_t)t * d + row] = (float)((double)res0 + tot);
  }
}

// h quantization for the expert-major down after 16-row gate/up items (which leave h in
// fp32 only): one half-wave per (pair, 32-row block), the arithmetic of the gate/up
// epilogue.
constexpr int kHqThreads = 256;
template <int BITS, bool DBG>
__global__ __launch_bounds__(kHqThreads) void k_hquant(const float* __restrict__ hf, int Q, int f,
                                                       int8_t* __restrict__ hq,
                                                       double2* __restrict__ hsc, DecodeDebug dbg) {
  const int nbf = f / 32;
  const int blk = (blockIdx.x * kHqThreads + (int)threadIdx.x) / 32, hl = threadIdx.x % 32;
  if (blk >= Q * nbf) return;  // whole half-waves leave together
  const int p = blk / nbf, b = blk - p * nbf;
  float scale;
  int qsum;
  const int c = quant_half_wave(hf[(size_t)p * f + 32 * b + hl], scale, qsum);
  hq[(size_t)p * f + 32 * b + act_byte_pos<BITS>(hl)] = (int8_t)c;
  if (hl == 0) hsc[(size_t)p * nbf + b] = make_double2((double)scale, (double)scale * qsum);
  if (DBG) {
    if (dbg.hq) dbg.hq[(size_t)p * f + 32 * b + hl] = (int8_t)c;
    if (dbg.hs && hl == 0) dbg.hs[(size_t)p * nbf + b] = scale;
  }
}

// Row tile: 32 rows a workgroup, or 8 and 16 for one- and two-token windows, which would
// otherwise fill only a quarter or half of the CUs (64 and 128 workgroups at d = 2048).
// Slots a lane: with 32 rows, kDtSlots / U weight blocks in flight per lane, or
// kDtSlotsShared / U when the window needs one more slot than that (a shared expert); with
// 16 and 8 rows, 4 and 2 slots (at most 16 slots a token).
inline int down_tok_rows(int n) { return n == 1 ? 8 : n == 2 ? 16 : 32; }

template <int BITS, int U, bool DBG>
hipError_t launch_down_tok_u(const DecodeArgs& a, const float* hf, const DecodeDebug& dbg) {
  const moe_layer& L = *a.L;
  const int d = L.d_model, f = L.d_ff, k = L.top_k, n = a.n;
  const int R = down_tok_rows(n);
  const int per = (d / R + 7) / 8;
  const dim3 grid(8 * per * n), block(kDtThreads);
  const uint32_t* sm = reinterpret_cast<const uint32_t*>(L.down.scale_min);
  const bool shared = has_shared(L);
  const uint32_t* sdc = shared ? L.shared_down.codes : nullptr;
  const uint32_t* sds = shared ? reinterpret_cast<const uint32_t*>(L.shared_down.scale_min) : nullptr;
  constexpr int I1 = kDtSlots / U, I2 = kDtSlotsShared / U;
  const int ke = k + (shared ? 1 : 0);
  // more workgroups than CUs: quantize h early, so that two fit a CU
  const bool eq = (int)grid.x > a.num_cus;
#define QMOE_DT(EQ)                                                                       \
  (R == 8    ? (shared ? k_down_tok<BITS, U, 2, true, EQ, DBG, 8>                          \
                       : k_down_tok<BITS, U, 2, false, EQ, DBG, 8>)                        \
   : R == 16 ? (shared ? k_down_tok<BITS, U, 4, true, EQ, DBG, 16>                         \
                       : k_down_tok<BITS, U, 4, false, EQ, DBG, 16>)                       \
   : shared  ? k_down_tok<BITS, U, I2, true, EQ, DBG, 32>                                  \
   : (ke + 1) / 2 <= I1 ? k_down_tok<BITS, U, I1, false, EQ, DBG, 32>                      \
                        : k_down_tok<BITS, U, I2, false, EQ, DBG, 32>)
  auto kern = eq ? QMOE_DT(true) : QMOE_DT(false);
#undef QMOE_DT
  hipLaunchKernelGGL(kern, grid, block, 0, a.stream, L.down.codes, sm, d, f, k, n,
                     a.r->topk_ids, a.r->topk_w, hf, a.residual, sdc, sds, dbg);
  return hipGetLastError();
}

template <int BITS, bool DBG>
hipError_t launch_down_tok(const DecodeArgs& a, const float* hf, const DecodeDebug& dbg, int U) {
  switch (U) {
    case 1: return launch_down_tok_u<BITS, 1, DBG>(a, hf, dbg);
    case 2: return launch_down_tok_u<BITS, 2, DBG>(a, hf, dbg);
    case 3: return launch_down_tok_u<BITS, 3, DBG>(a, hf, dbg);
    default: return launch_down_tok_u<BITS, 4, DBG>(a, hf, dbg);
  }
}

// ---------------------------------------------------------------- host side

template <int BITS, int NPC, bool DBG>
hipError_t launch_ffn(const DecodeArgs& a) {
  const moe_layer& L = *a.L;
  const int n = a.n, d = L.d_model, f = L.d_ff, k = L.top_k, E = L.n_experts;
  const bool shared = has_shared(L);  // only on the ids path (checked by the entry point)
  const DecodeWs W = decode_ws_layout(n, k, d, f, shared, L.router_w ? E : 0);
  int* chunks = reinterpret_cast<int*>(a.ws + W.chunks);
  int* nchunks = reinterpret_cast<int*>(a.ws + W.nchunks);
  int8_t* xq = reinterpret_cast<int8_t*>(a.ws + W.xq);
  double2* xsc = reinterpret_cast<double2*>(a.ws + W.xsc);
  int8_t* hq = reinterpret_cast<int8_t*>(a.ws + W.hq);
  double2* hsc = reinterpret_cast<double2*>(a.ws + W.hsc);
  float* y = reinterpret_cast<float*>(a.ws + W.y);
  float* hf = reinterpret_cast<float*>(a.ws + W.hf);
  DecodeDebug dbg{};
  if (DBG) dbg = *a.dbg;

  const int nbd = d / 32;
  hipError_t err = hipSuccess;
  // chunks straight from the expert ids (see k_gateup); with logits, the gate/up stage also
  // writes the routing's grouping
  const bool ids = n <= 2 * NPC && (long long)n * k <= kWave;
  // logits to route from: the caller's, or the router projection's in the workspace
  const float* logits = a.project ? reinterpret_cast<const float*>(a.ws + W.logits) : a.logits;
  if (a.stages & MOE_DECODE_PREP) {
    if (a.project) {
      hipLaunchKernelGGL(k_router_logits, dim3(E), dim3(kRtThreads),
                         0, a.stream, L.router_w, a.x, n, d, E,
                         reinterpret_cast<float*>(a.ws + W.logits), DBG ? dbg.logits : nullptr);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    const int prep_blocks = 1 + (n * nbd + kPrepThreads - 1) / kPrepThreads;
    if (logits && n <= kFusedMaxTokens) {
      const int kpl = (E + kWave - 1) / kWave;
#define QMOE_RP(G)                                                                        \
  (kpl <= 1   ? k_route_prep<BITS, 1, G>                                                  \
   : kpl <= 2 ? k_route_prep<BITS, 2, G>                                                  \
   : kpl <= 4 ? k_route_prep<BITS, 4, G>                                                  \
   : kpl <= 8 ? k_route_prep<BITS, 8, G>                                                  \
              : k_route_prep<BITS, 16, G>)
      auto kern = ids ? QMOE_RP(false) : QMOE_RP(true);
#undef QMOE_RP
      hipLaunchKernelGGL(kern, dim3(prep_blocks), dim3(kPrepThreads), 0, a.stream, logits, a.x,
                         n, d, E, k, NPC, a.r->topk_ids, a.r->topk_w, a.r->expert_offsets,
                         a.r->pair_index, chunks, nchunks, xq, xsc, DBG ? dbg.xq : nullptr,
                         DBG ? dbg.xs : nullptr);
    } else if (logits && (long long)n * k <= kSingleGroupPairs) {
      err = launch_route_topk(logits, n, E, k, a.r->topk_ids, a.r->topk_w, a.stream);
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL(k_group_prep<BITS>, dim3(prep_blocks), dim3(kPrepThreads), 0, a.stream,
                         a.x, n, d, a.r->topk_ids, E, k, NPC, a.r->expert_offsets,
                         a.r->pair_index, chunks, nchunks, xq, xsc, DBG ? dbg.xq : nullptr,
                         DBG ? dbg.xs : nullptr);
    } else {
      if (logits) {
        // the histograms of a multi-workgroup grouping live in the pair-output region,
        // which is only written later (fp32 rows of d >= 32: at least 128 bytes per pair;
        // this path runs past 4096 pairs, and the histograms need at most 2 bytes per pair
        // plus 4 KB)
        err = launch_route(logits, n, E, k, a.r, a.ws + W.y, a.stream);
        if (err != hipSuccess) return err;
      }
      hipLaunchKernelGGL(k_prep<BITS>, dim3(prep_blocks), dim3(kPrepThreads), 0, a.stream, a.x,
                         n, d, a.r->expert_offsets, a.r->pair_index, E, k, NPC, chunks, nchunks,
                         xq, xsc, DBG ? dbg.xq : nullptr, DBG ? dbg.xs : nullptr);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }

  // upper bound of chunks: every chunk holds >= 1 pair, an expert holds <= n pairs, and
  // sum_e ceil(c_e / NPC) <= P / NPC + (number of experts with pairs)
  const long long P = (long long)n * k;
  const long long max_chunks = std::min<long long>(
      std::min<long long>(P, (long long)E * ((n + NPC - 1) / NPC)),
      (P + NPC - 1) / NPC + std::min<long long>(E, P));
  // grid cap of the expert-major down, whose workgroups loop over the items past it
  // (16 a CU measured best against 4, 8 and 64 on the 64-sequence batches)
  const int cap = a.num_cus * 16;
  // The token-major down (down and combine in one kernel) takes windows of up to 16 tokens
  // and 16 slots a token, d_ff up to 1024, and as many slots as its lanes hold. It reads h
  // in fp32 and quantizes it itself; the expert-major down reads the codes.
  const int nbf = f / 32, dt_u = (nbf + 7) / 8;
  const int ke = k + (shared ? 1 : 0);  // slots per token
  const bool dt_shape = n <= kDtMaxTokens && ke <= kDtMaxK && nbf <= kDtMaxBlocks &&
                        (ke + 1) / 2 <= kDtSlotsShared / dt_u;
  // 16-row gate/up items for such a window: h leaves in fp32 only, and an expert-major
  // down (down and combine in separate calls) quantizes it first
  const bool h16 = dt_shape;
  if (a.stages & MOE_DECODE_GATE_UP) {
    // one workgroup per item; the shared expert is one more chunk
    const long long gu_items =
        (max_chunks + (shared ? (n + NPC - 1) / NPC : 0)) * (f / (h16 ? 16 : kGuRows));
    const bool group = ids && logits;  // workgroup 0 writes the routing's grouping
    const long long gu_run = h16 ? (gu_items + 15) / 16 * 16 : gu_items;  // see k_gateup
    const int gu_grid = (int)std::max<long long>(1, gu_run + (group ? 1 : 0));
    const uint32_t* gsm = reinterpret_cast<const uint32_t*>(L.gate.scale_min);
    const uint32_t* usm = reinterpret_cast<const uint32_t*>(L.up.scale_min);
    const uint32_t* sgc = shared ? L.shared_gate.codes : nullptr;
    const uint32_t* sgs = shared ? reinterpret_cast<const uint32_t*>(L.shared_gate.scale_min) : nullptr;
    const uint32_t* suc = shared ? L.shared_up.codes : nullptr;
    const uint32_t* sus = shared ? reinterpret_cast<const uint32_t*>(L.shared_up.scale_min) : nullptr;
    if (h16 && ids)
      hipLaunchKernelGGL((k_gateup<BITS, NPC, 4, 16, DBG, true>), dim3(gu_grid),
                         dim3(GuShape<4, 16>::kThreads), 0,
                         a.stream, L.gate.codes, gsm, L.up.codes, usm, d, f, chunks, nchunks, xq,
                         xsc, hq, hsc, a.r->topk_ids, k, n * k, E,
                         group ? a.r->expert_offsets : nullptr, a.r->pair_index, sgc, sgs, suc,
                         sus, n, hf, dbg);
    else if (ids)
      hipLaunchKernelGGL((k_gateup<BITS, NPC, 8, 32, DBG, true>), dim3(gu_grid),
                         dim3(GuShape<8, 32>::kThreads), 0,
                         a.stream, L.gate.codes, gsm, L.up.codes, usm, d, f, chunks, nchunks, xq,
                         xsc, hq, hsc, a.r->topk_ids, k, n * k, E,
                         group ? a.r->expert_offsets : nullptr, a.r->pair_index, sgc, sgs, suc,
                         sus, n, nullptr, dbg);
    else if (h16)
      hipLaunchKernelGGL((k_gateup<BITS, NPC, 4, 16, DBG, false>), dim3(gu_grid),
                         dim3(GuShape<4, 16>::kThreads), 0,
                         a.stream, L.gate.codes, gsm, L.up.codes, usm, d, f, chunks, nchunks, xq,
                         xsc, hq, hsc, a.r->topk_ids, k, n * k, E, nullptr, nullptr, nullptr,
                         nullptr, nullptr, nullptr, n, hf, dbg);
    else
      hipLaunchKernelGGL((k_gateup<BITS, NPC, 4, 32, DBG, false>), dim3(gu_grid),
                         dim3(GuShape<4, 32>::kThreads), 0,
                         a.stream, L.gate.codes, gsm, L.up.codes, usm, d, f, chunks, nchunks, xq,
                         xsc, hq, hsc, a.r->topk_ids, k, n * k, E, nullptr, nullptr, nullptr,
                         nullptr, nullptr, nullptr, n, nullptr, dbg);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // down and combine together for a small window: the token-major kernel does both
  const bool token_major =
      (a.stages & MOE_DECODE_DOWN) && (a.stages & MOE_DECODE_COMBINE) && dt_shape;
  if (token_major) return launch_down_tok<BITS, DBG>(a, hf, dbg, dt_u);
  if (a.stages & MOE_DECODE_DOWN) {
    if (ids && logits) {
      // with logits the ids path builds no work list (gate/up takes its chunks from the
      // expert ids and writes the grouping): the expert-major down builds it from that
      // grouping (block 0 of the prep kernel alone)
      hipLaunchKernelGGL(k_prep<BITS>, dim3(1), dim3(kPrepThreads), 0, a.stream, a.x, n, d,
                         a.r->expert_offsets, a.r->pair_index, E, k, NPC, chunks, nchunks, xq,
                         xsc, nullptr, nullptr);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    if (h16) {
      const long long hblocks = (P + (shared ? n : 0)) * nbf;
      hipLaunchKernelGGL((k_hquant<BITS, DBG>), dim3((int)((hblocks * 32 + kHqThreads - 1) / kHqThreads)),
                         dim3(kHqThreads), 0, a.stream, hf, (int)(P + (shared ? n : 0)), f, hq,
                         hsc, dbg);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    const long long dn_items = max_chunks * ((d + kWave - 1) / kWave);
    const int dn_grid = (int)std::max<long long>(1, std::min<long long>(dn_items, cap));
    // the matrix-core instance when the pairs per busy expert average kMmaMinPairs or more
    auto dn_kernel = k_down<BITS, NPC, DBG, false>;
    if constexpr (dn_has_mma<BITS, NPC, true>()) {
      if (P >= (long long)kMmaMinPairs * std::min<long long>(E, P))
        dn_kernel = k_down<BITS, NPC, DBG, true>;
    }
    hipLaunchKernelGGL(dn_kernel, dim3(dn_grid), dim3(kDnThreads), 0, a.stream, L.down.codes,
                       reinterpret_cast<const uint32_t*>(L.down.scale_min), d, f, chunks, nchunks,
                       hq, hsc, y, dbg);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (a.stages & MOE_DECODE_COMBINE) {
    hipLaunchKernelGGL(k_combine, dim3((n * d + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       a.stream, y, a.r->topk_w, n, d, k, a.residual);
    err = hipGetLastError();
  }
  return err;
}

template <int BITS, bool DBG>
hipError_t launch_bits(const DecodeArgs& a) {
  // chunks of 4 pairs (95 registers: five 16-row gate/up workgroups a CU) up to 8 tokens
  // while the ids path applies (an expert then takes at most two chunks)
  if (a.n <= 4 || (a.n <= 8 && (long long)a.n * a.L->top_k <= kWave))
    return launch_ffn<BITS, 4, DBG>(a);
  return launch_ffn<BITS, 8, DBG>(a);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a) {
  const bool dbg = a.dbg != nullptr;
  if (a.L->gate.bits == 4) return dbg ? launch_bits<4, true>(a) : launch_bits<4, false>(a);
  return dbg ? launch_bits<2, true>(a) : launch_bits<2, false>(a);
}

}  // namespace qmoe

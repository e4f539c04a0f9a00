// Router top-k, routing weights and the grouping of token-expert pairs by expert.
//
// Selection follows the router of the Strata engine explainer (m.lqnn.cn/news/264700,
// "Architecture overview": each token keeps the 10 of 512 experts its router picks);
// the expert ids and routing weights form the hand-over record of the "Doorbell
// handshake" section, and grouping by expert feeds a grouped expert kernel ("Expert
// cache" section).
//
// One wavefront selects for one token: lane l holds the logits of experts l, l+64, ...
// as 64-bit keys (order-preserving bits of the logit, then the complement of the expert
// id so that equal logits favour the lower id); k rounds of a wave max-reduction pick
// the slots in order. Weights are computed in binary64 and summed in slot order.
// Grouping is a stable counting sort done by one workgroup: per-wave histograms in LDS,
// a scan, and an in-order scatter where lanes holding the same expert are ranked with
// ballots over the bits of the expert id.
#include "qmoe_internal.h"

namespace qmoe {

namespace {

constexpr int kGroupWaves = 8;
constexpr int kGroupThreads = kGroupWaves * kWave;

__device__ __forceinline__ uint32_t order_bits(float f) {
  f = f + 0.0f;  // -0 becomes +0, so the two compare equal
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_bits_to_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ uint64_t make_key(float logit, int e) {
  return ((uint64_t)order_bits(logit) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
}

// 64-bit DPP move within a wavefront; lanes whose source is invalid or masked off by
// row_mask keep their own value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const uint32_t lo2 = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi2 = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xF, false);
  return ((uint64_t)hi2 << 32) | lo2;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum of a 64-bit value over the wavefront, returned wave-uniform: DPP steps reduce
// within quads, 8- and 16-lane rows, then across rows (row_bcast15/31) into lane 63.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0xB1, 0xF>(v));   // quad_perm [1,0,3,2]
  v = max_u64(v, dpp_u64<0x4E, 0xF>(v));   // quad_perm [2,3,0,1]
  v = max_u64(v, dpp_u64<0x141, 0xF>(v));  // row_half_mirror
  v = max_u64(v, dpp_u64<0x140, 0xF>(v));  // row_mirror
  v = max_u64(v, dpp_u64<0x142, 0xA>(v));  // row_bcast:15
  v = max_u64(v, dpp_u64<0x143, 0xC>(v));  // row_bcast:31
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, kWave - 1);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), kWave - 1);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  uint64_t u;
  __builtin_memcpy(&u, &v, 8);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), lane);
  u = ((uint64_t)hi << 32) | lo;
  double r;
  __builtin_memcpy(&r, &u, 8);
  return r;
}

// Top-k of one token by one full wavefront; lane j < k writes slot j.
template <int KPL>
__device__ int wave_topk(const float* __restrict__ lrow, int E, int k, int32_t* __restrict__ ids,
                         float* __restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t key[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = lane + kWave * i;
    key[i] = e < E ? make_key(lrow[e], e) : 0ull;
  }
  int my_id = 0;
  float my_l = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < KPL; ++i) best = max_u64(best, key[i]);
    best = wave_max_u64(best);
    const int e = (int)(0xffffffffu - (uint32_t)best);
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (lane + kWave * i == e) key[i] = 0ull;
    if (lane == j) {
      my_id = e;
      my_l = order_bits_to_float((uint32_t)(best >> 32));
    }
  }
  const float l0f = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(my_l)));
  const double ex = lane < k ? exp((double)my_l - (double)l0f) : 0.0;
  double sum = 0.0;
  for (int j = 0; j < k; ++j) sum += readlane_f64(ex, j);  // slot order
  if (lane < k) {
    ids[lane] = my_id;
    w[lane] = (float)(ex / sum);
  }
  return my_id;  // lane j < k: the expert of slot j
}

// Exclusive scan of v[0..n) (n <= 2*kGroupThreads) in LDS by a kGroupThreads block.
__device__ void block_exclusive_scan(int* v, int n, int* wsum) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int a = 2 * tid < n ? v[2 * tid] : 0;
  const int b = 2 * tid + 1 < n ? v[2 * tid + 1] : 0;
  int s = a + b, incl = s;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int wbase = 0;
  for (int i = 0; i < wave; ++i) wbase += wsum[i];
  const int excl = wbase + incl - s;
  __syncthreads();
  if (2 * tid < n) v[2 * tid] = excl;
  if (2 * tid + 1 < n) v[2 * tid + 1] = excl + a;
  __syncthreads();
}

// Stable counting sort of pair ids 0..P-1 by ids[p], by one block of kGroupThreads.
__device__ void group_block(const int32_t* ids, int P, int E, int32_t* __restrict__ offsets,
                            int32_t* __restrict__ pair_index) {
  __shared__ int s_hist[kGroupWaves * MOE_MAX_EXPERTS];  // [wave][E] counts, then bases
  __shared__ int s_off[MOE_MAX_EXPERTS];
  __shared__ int s_wsum[kGroupWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  for (int i = tid; i < kGroupWaves * E; i += kGroupThreads) s_hist[i] = 0;
  __syncthreads();
  const int chunk = (P + kGroupWaves - 1) / kGroupWaves;
  const int beg = min(P, wave * chunk), end = min(P, beg + chunk);
  for (int p = beg + lane; p < end; p += kWave) atomicAdd(&s_hist[wave * E + ids[p]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += kGroupThreads) {
    int run = 0;
    for (int w = 0; w < kGroupWaves; ++w) {
      const int c = s_hist[w * E + e];
      s_hist[w * E + e] = run;
      run += c;
    }
    s_off[e] = run;
  }
  __syncthreads();
  block_exclusive_scan(s_off, E, s_wsum);
  for (int e = tid; e < E; e += kGroupThreads) {
    offsets[e] = s_off[e];
    for (int w = 0; w < kGroupWaves; ++w) s_hist[w * E + e] += s_off[e];
  }
  if (tid == 0) offsets[E] = P;
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  for (int base = beg; base < end; base += kWave) {
    const int p = base + lane;
    const bool valid = p < end;
    const int e = valid ? ids[p] : 0;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {  // experts < 1024
      const bool set = (e >> bit) & 1;
      const uint64_t bal = __ballot(set);
      same &= set ? bal : ~bal;
    }
    const int rank = __popcll(same & below);
    const int cnt = __popcll(same);
    int slot = 0;
    if (valid) slot = s_hist[wave * E + e];
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      pair_index[slot + rank] = p;
      if (rank == cnt - 1) s_hist[wave * E + e] = slot + cnt;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Grouping for small batches (P = n*k <= kSmallPairs): with the pair ids in LDS, thread e
// computes offsets[e] = #{q : ids[q] < e} and pair p lands at
// #{q : ids[q] < ids[p]} + #{q < p : ids[q] == ids[p]}, the position a stable counting sort
// gives it. O(P) LDS broadcasts per thread, no atomics and no scans.
constexpr int kSmallPairs = 256;

__device__ void group_small(const int* s_ids, int P, int E, int32_t* __restrict__ offsets,
                            int32_t* __restrict__ pair_index) {
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += kGroupThreads) {
    int c = 0;
#pragma unroll 8
    for (int q = 0; q < P; ++q) c += s_ids[q] < e;
    offsets[e] = c;
  }
  for (int p = tid; p < P; p += kGroupThreads) {
    const int ep = s_ids[p];
    int pos = 0;
#pragma unroll 8
    for (int q = 0; q < P; ++q) {
      const int eq = s_ids[q];
      pos += (eq < ep) | ((eq == ep) & (q < p));
    }
    pair_index[pos] = p;
  }
}

template <int KPL>
__global__ __launch_bounds__(kGroupThreads) void k_route_fused(
    const float* __restrict__ logits, int n, int E, int k, int32_t* ids, float* __restrict__ w,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pair_index) {
  __shared__ int s_ids[kSmallPairs];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int P = n * k;
  for (int t = wave; t < n; t += kGroupWaves) {
    const int id = wave_topk<KPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k,
                                  w + (size_t)t * k);
    if (P <= kSmallPairs && lane < k) s_ids[t * k + lane] = id;
  }
  __threadfence_block();
  __syncthreads();
  if (P <= kSmallPairs)
    group_small(s_ids, P, E, offsets, pair_index);
  else
    group_block(ids, P, E, offsets, pair_index);
}

template <int KPL>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int n, int E,
                                                    int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int t = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (t >= n) return;
  wave_topk<KPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k);
}

__global__ __launch_bounds__(kGroupThreads) void k_route_group(const int32_t* __restrict__ ids,
                                                               int P, int E,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ pair_index) {
  group_block(ids, P, E, offsets, pair_index);
}

template <int KPL>
hipError_t launch_route_kpl(const float* logits, int n, int E, int k, const moe_routing* out,
                            hipStream_t stream) {
  if (n <= 64) {
    hipLaunchKernelGGL(k_route_fused<KPL>, dim3(1), dim3(kGroupThreads), 0, stream, logits, n, E,
                       k, out->topk_ids, out->topk_w, out->expert_offsets, out->pair_index);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_route_topk<KPL>, dim3((n + 3) / 4), dim3(256), 0, stream, logits, n, E, k,
                     out->topk_ids, out->topk_w);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_route_group, dim3(1), dim3(kGroupThreads), 0, stream, out->topk_ids, n * k,
                     E, out->expert_offsets, out->pair_index);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, int n, int E, int k, const moe_routing* out,
                        hipStream_t stream) {
  const int kpl = (E + kWave - 1) / kWave;
  if (kpl <= 1) return launch_route_kpl<1>(logits, n, E, k, out, stream);
  if (kpl <= 2) return launch_route_kpl<2>(logits, n, E, k, out, stream);
  if (kpl <= 4) return launch_route_kpl<4>(logits, n, E, k, out, stream);
  if (kpl <= 8) return launch_route_kpl<8>(logits, n, E, k, out, stream);
  return launch_route_kpl<16>(logits, n, E, k, out, stream);
}

}  // namespace qmoe

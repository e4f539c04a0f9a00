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
#include "qmoe_route_dev.h"

namespace qmoe {

namespace {

constexpr int kGroupWaves = 8;
constexpr int kGroupThreads = kGroupWaves * kWave;

template <int KPL>
__global__ __launch_bounds__(kGroupThreads) void k_route_fused(
    const float* __restrict__ logits, int n, int E, int k, int32_t* ids, float* __restrict__ w,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pair_index) {
  __shared__ int s_ids[kSmallPairs];
  __shared__ int s_hist[kGroupWaves * MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_wsum[kGroupWaves];
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
    group_block<kGroupWaves>(ids, P, E, s_hist, s_off, s_wsum, offsets, pair_index);
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
  __shared__ int s_hist[kGroupWaves * MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_wsum[kGroupWaves];
  group_block<kGroupWaves>(ids, P, E, s_hist, s_off, s_wsum, offsets, pair_index);
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

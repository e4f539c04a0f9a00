// Router top-k, routing weights and the grouping of token-expert pairs by expert.
//
// Selection follows the router of the Strata engine explainer (m.lqnn.cn/news/264700,
// "Architecture overview": each token keeps the 10 of 512 experts its router picks);
// the expert ids and routing weights form the hand-over record of the "Doorbell
// handshake" section, and grouping by expert feeds a grouped expert kernel ("Expert
// cache" section).
//
// One wavefront selects for one token (wave_topk): lane l holds the logits of experts
// l, l+64, ... as order-preserving bits; a threshold found bit by bit with ballots leaves
// the candidates, which are ranked by (logit desc, id asc) from registers. Weights are
// computed in binary64 and summed in slot order. Grouping is a stable counting sort: by
// one workgroup up to 4096 pairs (per-wave histograms in LDS, a scan, and an in-order
// scatter where lanes holding the same expert are ranked with ballots over the bits of
// the expert id), and beyond that by many workgroups over chunks of 2048 pairs, each
// writing an expert histogram to the workspace.
#include "qmoe_route_dev.h"

namespace qmoe {

namespace {

constexpr int kGroupWaves = 8;
constexpr int kGroupThreads = kGroupWaves * kWave;
// up to this many pairs one workgroup groups them (k_route_group) without a workspace

template <int KPL>
__global__ __launch_bounds__(kGroupThreads) void k_route_fused(
    const float* __restrict__ logits, int n, int E, int k, int32_t* ids, float* __restrict__ w,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pair_index) {
  __shared__ __attribute__((aligned(16))) int s_ids[kSmallPairs + 4];
  __shared__ int s_hist[kGroupWaves * MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_wsum[kGroupWaves];
  __shared__ TopkScratch s_tk[kGroupWaves];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int P = n * k;
  for (int t = wave; t < n; t += kGroupWaves) {
    const int id = wave_topk<KPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k,
                                  w + (size_t)t * k, &s_tk[wave]);
    if (P <= kSmallPairs && lane < k) s_ids[t * k + lane] = id;
  }
  if (P <= kSmallPairs && threadIdx.x < 4 && P + (int)threadIdx.x < ((P + 3) & ~3))
    s_ids[P + threadIdx.x] = 0x7fffffff;  // padding read by group_small
  __threadfence_block();
  __syncthreads();
  if (P <= kWave)
    group_tiny(s_ids, P, E, offsets, pair_index);
  else if (P <= kSmallPairs)
    group_small(s_ids, P, E, offsets, pair_index);
  else
    group_block<kGroupWaves>(ids, P, E, s_hist, s_off, s_wsum, offsets, pair_index);
}

template <int KPL>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int n, int E,
                                                    int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  __shared__ TopkScratch s_tk[256 / kWave];
  const int t = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (t >= n) return;
  wave_topk<KPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k,
                 &s_tk[threadIdx.x / kWave]);
}

__global__ __launch_bounds__(kGroupThreads) void k_route_group(const int32_t* __restrict__ ids,
                                                               int P, int E,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ pair_index) {
  __shared__ int s_ids[kSingleGroupPairs];
  __shared__ int s_hist[kGroupWaves * MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_wsum[kGroupWaves];
  ids_to_lds<kSingleGroupPairs, kGroupThreads>(ids, P, s_ids);
  __syncthreads();
  group_block<kGroupWaves>(s_ids, P, E, s_hist, s_off, s_wsum, offsets, pair_index);
}

// ---- grouping of large batches over many workgroups -------------------------------
//
// Pairs are cut into chunks of kChunkPairs; chunk b is handled by workgroup b of both
// kernels. k_group_count writes each chunk's per-expert histogram to hist[b][E].
// k_group_scatter lets every workgroup derive what it needs from those histograms: the
// expert totals (hence the offsets, by a scan) and the number of pairs of each expert in
// earlier chunks; inside its chunk the scatter is the stable per-wave one of group_block.
constexpr int kScatterThreads = 1024;
constexpr int kScatterWaves = kScatterThreads / kWave;

__global__ __launch_bounds__(kScatterThreads) void k_group_count(const int32_t* __restrict__ ids,
                                                                 int P, int E,
                                                                 int* __restrict__ hist) {
  __shared__ int s_hist[MOE_MAX_EXPERTS];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kScatterThreads) s_hist[e] = 0;
  __syncthreads();
  const int beg = blockIdx.x * kChunkPairs, end = min(P, beg + kChunkPairs);
  for (int p = beg + tid; p < end; p += kScatterThreads) atomicAdd(&s_hist[ids[p]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += kScatterThreads) hist[(size_t)blockIdx.x * E + e] = s_hist[e];
}

__global__ __launch_bounds__(kScatterThreads) void k_group_scatter(
    const int32_t* __restrict__ ids, int P, int E, int nchunks, const int* __restrict__ hist,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pair_index) {
  __shared__ int s_whist[kScatterWaves * MOE_MAX_EXPERTS];  // [wave][E]
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_base[MOE_MAX_EXPERTS];
  __shared__ int s_wsum[kScatterWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int b = blockIdx.x;
  // expert totals and the pairs of each expert in earlier chunks (unrolled, so that several
  // histogram loads are in flight instead of one round trip per chunk)
  for (int e = tid; e < E; e += kScatterThreads) {
    int tot = 0, before = 0;
#pragma unroll 8
    for (int c = 0; c < nchunks; ++c) {
      const int v = hist[(size_t)c * E + e];
      tot += v;
      before += c < b ? v : 0;
    }
    s_off[e] = tot;
    s_base[e] = before;
  }
  for (int i = tid; i < kScatterWaves * E; i += kScatterThreads) s_whist[i] = 0;
  __syncthreads();
  block_exclusive_scan(s_off, E, s_wsum);
  if (b == 0) {
    for (int e = tid; e < E; e += kScatterThreads) offsets[e] = s_off[e];
    if (tid == 0) offsets[E] = P;
  }
  // this chunk: per-wave histograms over contiguous sub-ranges, in pair order
  const int cbeg = b * kChunkPairs, cend = min(P, cbeg + kChunkPairs);
  const int per = (cend - cbeg + kScatterWaves - 1) / kScatterWaves;
  const int wbeg = min(cend, cbeg + wave * per), wend = min(cend, wbeg + per);
  for (int p = wbeg + lane; p < wend; p += kWave) atomicAdd(&s_whist[wave * E + ids[p]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += kScatterThreads) {
    int run = s_off[e] + s_base[e];
    for (int w = 0; w < kScatterWaves; ++w) {
      const int c = s_whist[w * E + e];
      s_whist[w * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  for (int base = wbeg; base < wend; base += kWave) {
    const int p = base + lane;
    const bool valid = p < wend;
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
    if (valid) slot = s_whist[wave * E + e];
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      pair_index[slot + rank] = p;
      if (rank == cnt - 1) s_whist[wave * E + e] = slot + cnt;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int KPL>
hipError_t launch_route_kpl(const float* logits, int n, int E, int k, const moe_routing* out,
                            void* ws, hipStream_t stream) {
  if (n <= kFusedRouteTokens) {
    hipLaunchKernelGGL(k_route_fused<KPL>, dim3(1), dim3(kGroupThreads), 0, stream, logits, n, E,
                       k, out->topk_ids, out->topk_w, out->expert_offsets, out->pair_index);
    return hipGetLastError();
  }
  hipError_t err = launch_route_topk(logits, n, E, k, out->topk_ids, out->topk_w, stream);
  if (err != hipSuccess) return err;
  const int P = n * k;
  if (P <= kSingleGroupPairs) {
    hipLaunchKernelGGL(k_route_group, dim3(1), dim3(kGroupThreads), 0, stream, out->topk_ids, P,
                       E, out->expert_offsets, out->pair_index);
    return hipGetLastError();
  }
  const int nchunks = (P + kChunkPairs - 1) / kChunkPairs;
  int* hist = static_cast<int*>(ws);
  hipLaunchKernelGGL(k_group_count, dim3(nchunks), dim3(kScatterThreads), 0, stream,
                     out->topk_ids, P, E, hist);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_group_scatter, dim3(nchunks), dim3(kScatterThreads), 0, stream,
                     out->topk_ids, P, E, nchunks, hist, out->expert_offsets, out->pair_index);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int n, int E, int k, int32_t* ids, float* w,
                             hipStream_t stream) {
  const int kpl = (E + kWave - 1) / kWave;
  auto kern = kpl <= 1   ? k_route_topk<1>
              : kpl <= 2 ? k_route_topk<2>
              : kpl <= 4 ? k_route_topk<4>
              : kpl <= 8 ? k_route_topk<8>
                         : k_route_topk<16>;
  hipLaunchKernelGGL(kern, dim3((n + 3) / 4), dim3(256), 0, stream, logits, n, E, k, ids, w);
  return hipGetLastError();
}

hipError_t launch_route(const float* logits, int n, int E, int k, const moe_routing* out,
                        void* ws, hipStream_t stream) {
  const int kpl = (E + kWave - 1) / kWave;
  if (kpl <= 1) return launch_route_kpl<1>(logits, n, E, k, out, ws, stream);
  if (kpl <= 2) return launch_route_kpl<2>(logits, n, E, k, out, ws, stream);
  if (kpl <= 4) return launch_route_kpl<4>(logits, n, E, k, out, ws, stream);
  if (kpl <= 8) return launch_route_kpl<8>(logits, n, E, k, out, ws, stream);
  return launch_route_kpl<16>(logits, n, E, k, out, ws, stream);
}

}  // namespace qmoe

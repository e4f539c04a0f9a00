// Device routines of the router: top-k selection with routing weights by one wavefront,
// and the stable grouping of token-expert pairs by expert inside one workgroup.
//
// Selection follows the router of the Strata engine explainer (m.lqnn.cn/news/264700,
// "Architecture overview": each token keeps the 10 of 512 experts its router picks); the
// expert ids and routing weights form the hand-over record of the "Doorbell handshake"
// section, and grouping by expert feeds a grouped expert kernel ("Expert cache" section).
#pragma once

#include "qmoe_internal.h"

namespace qmoe {

// Order-preserving unsigned image of a float; -0 and +0 map to the same value. Finite
// inputs map to values >= 0x00800000, so 0 is free to mark an expert as taken.
__device__ __forceinline__ uint32_t order_bits(float f) {
  f = f + 0.0f;  // -0 becomes +0, so the two compare equal
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_bits_to_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Maximum of a 32-bit value over the wavefront, returned wave-uniform: DPP steps reduce
// within quads, 8- and 16-lane rows, then across rows (row_bcast15/31) into lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1, 0xF>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E, 0xF>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141, 0xF>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140, 0xF>(v));  // row_mirror
  v = max(v, dpp_u32<0x142, 0xA>(v));  // row_bcast:15
  v = max(v, dpp_u32<0x143, 0xC>(v));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// Inclusive prefix sum over the wavefront with DPP: row shifts by 1, 2, 4 and 8 (lanes
// without a source add 0), then row 0's total into row 1 and row 2's into row 3
// (row_bcast:15), then rows 0-1's total into rows 2-3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
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

// Per-wave LDS scratch of the threshold selection in wave_topk.
struct alignas(16) TopkScratch {
  uint32_t key[kWave];  // compacted candidates
  int id[kWave];
  uint32_t slot_key[MOE_MAX_TOP_K];
  int slot_id[MOE_MAX_TOP_K];
};

// Top-k of one token by one full wavefront. Lane l holds the logits of experts l, l+64,
// ... as order bits (ties favour the lower expert id; -0 equals +0).
//
// Selection by threshold: T = the k-th largest of the 64 lane maxima, found bit by bit
// with ballots. At least k experts (those lane maxima) have keys >= T, so every expert
// of the top k has a key >= T, and ranking the candidates (keys >= T) by (key desc, id
// asc) ranks the top k exactly. The candidates are compacted into LDS with ballots and
// each one counts how many candidates precede it. When more than 64 candidates tie at the
// threshold, k rounds of a wave maximum select instead (the lowest id holding the maximum
// is found with one ballot per register slot, since ids grow with the slot first and the
// lane second).
//
// Weights are exp(l_j - l_0) / sum_i exp(l_i - l_0) in binary64, summed in slot order.
// Lane j < k writes slot j and returns its expert id.
template <int KPL>
__device__ __forceinline__ int wave_topk(const float* __restrict__ lrow, int E, int k,
                                         int32_t* __restrict__ ids, float* __restrict__ w,
                                         TopkScratch* sc) {
  const int lane = threadIdx.x & (kWave - 1);
  // All KPL loads are issued unconditionally (clamped index) and pinned by an empty asm
  // that uses every value: a load feeding only a guarded expression is otherwise sunk into
  // a branch of its own with a wait behind it, one memory round trip per slot.
  float lv[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) lv[i] = lrow[min(lane + kWave * i, E - 1)];
#pragma unroll
  for (int i = 0; i < KPL; ++i) asm volatile("" : "+v"(lv[i]));
  uint32_t key[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int e = lane + kWave * i;
    // valid experts never take 0 (only one NaN pattern maps there), so every round finds
    // a maximum held by some untaken expert while j < k <= E
    key[i] = e < E ? max(order_bits(lv[i]), 1u) : 0u;
  }
  uint32_t lmax = key[0];
#pragma unroll
  for (int i = 1; i < KPL; ++i) lmax = max(lmax, key[i]);
  // T: the largest value with at least k lane maxima >= T (at least k lanes hold valid
  // experts, since k <= E and k <= 64)
  uint32_t T = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t t = T | (1u << b);
    if (__popcll(__ballot(lmax >= t)) >= k) T = t;
  }
  // compact the candidates in (slot, lane) order
  const uint64_t below = (1ull << lane) - 1ull;
  int total = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const bool c = key[i] >= T;
    const uint64_t b = __ballot(c);
    const int pos = total + __popcll(b & below);
    if (c && pos < kWave) {
      sc->key[pos] = key[i];
      sc->id[pos] = lane + kWave * i;
    }
    total += __popcll(b);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int my_id = 0;
  uint32_t my_bits = 0;
  if (total <= kWave) {
    // Each candidate is ranked by counting the candidates ahead of it. A candidate's
    // (key desc, id asc) order is the unsigned order of key:~id (ids are below 2^31), and
    // the wave reads the others' packed keys lane by lane from registers.
    const uint32_t mk = lane < total ? sc->key[lane] : 0u;
    const int mi = lane < total ? sc->id[lane] : 0x7fffffff;
    const uint32_t mlo = ~(uint32_t)mi;
    // chunks of 8 lanes (total <= 64 keeps them inside the wave); lanes past total hold
    // key 0, which never ranks ahead of a candidate (candidate keys are >= T >= 1)
    int rank = 0;
    for (int q0 = 0; q0 < total; q0 += 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t qk = (uint32_t)__builtin_amdgcn_readlane((int)mk, q0 + i);
        const uint32_t ql = (uint32_t)__builtin_amdgcn_readlane((int)mlo, q0 + i);
        rank += (qk > mk) | ((qk == mk) & (ql > mlo));
      }
    }
    if (lane < total && rank < k) {
      sc->slot_key[rank] = mk;
      sc->slot_id[rank] = mi;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < k) {
      my_id = sc->slot_id[lane];
      my_bits = sc->slot_key[lane];
    }
  } else {
    for (int j = 0; j < k; ++j) {
      uint32_t best = key[0];
#pragma unroll
      for (int i = 1; i < KPL; ++i) best = max(best, key[i]);
      best = wave_max_u32(best);
      int slot = KPL - 1;
      uint64_t hit = 0;
#pragma unroll
      for (int i = KPL - 1; i >= 0; --i) {
        const uint64_t b = __ballot(key[i] == best);
        if (b) {
          slot = i;
          hit = b;
        }
      }
      const int owner = __builtin_ctzll(hit);
      const int e = owner + kWave * slot;
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if (i == slot && lane == owner) key[i] = 0u;
      if (lane == j) {
        my_id = e;
        my_bits = best;
      }
    }
  }
  const float my_l = order_bits_to_float(my_bits);
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

// Exclusive scan of v[0..n) (n <= 2 * blockDim.x) in LDS; wsum holds one int per wave.
__device__ __forceinline__ void block_exclusive_scan(int* v, int n, int* wsum) {
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

// Copies the P expert ids of a grouping (1 <= P <= MAXP) from global memory into LDS. Every
// thread issues all its loads (clamped indexes, no branch around them) before its first
// store, so the copy costs one memory round trip; the counting and the scatter of
// group_block then read LDS instead of waiting on a load per 64 pairs.
template <int MAXP, int NT>
__device__ __forceinline__ void ids_to_lds(const int32_t* __restrict__ ids, int P, int* s_ids) {
  constexpr int kPer = (MAXP + NT - 1) / NT;
  const int tid = threadIdx.x;
  int v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) v[j] = ids[min(tid + j * NT, P - 1)];
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (tid + j * NT < P) s_ids[tid + j * NT] = v[j];
}

// Stable counting sort of pair ids 0..P-1 by ids[p] (ids may live in LDS or global
// memory), by the first NW waves of the workgroup; the rest of the workgroup only joins
// the barriers. hist: LDS of NW*E ints; s_off: LDS of E+1 ints, which ends up holding the
// offsets too (offsets may be s_off itself). Writes offsets[0..E] and pair_index[0..P).
// Per-wave histograms in LDS, a scan, and an in-order scatter where lanes holding the same
// expert are ranked with ballots over the bits of the expert id.
template <int NW>
__device__ __forceinline__ void group_block(const int32_t* ids, int P, int E, int* hist, int* s_off, int* wsum,
                            int32_t* offsets, int32_t* __restrict__ pair_index) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int nt = blockDim.x;
  for (int i = tid; i < NW * E; i += nt) hist[i] = 0;
  __syncthreads();
  const int chunk = (P + NW - 1) / NW;
  const int beg = min(P, wave * chunk), end = wave < NW ? min(P, beg + chunk) : beg;
  for (int p = beg + lane; p < end; p += kWave) atomicAdd(&hist[wave * E + ids[p]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += nt) {
    int run = 0;
    for (int w = 0; w < NW; ++w) {
      const int c = hist[w * E + e];
      hist[w * E + e] = run;
      run += c;
    }
    s_off[e] = run;
  }
  __syncthreads();
  block_exclusive_scan(s_off, E, wsum);
  for (int e = tid; e < E; e += nt) {
    offsets[e] = s_off[e];
    for (int w = 0; w < NW; ++w) hist[w * E + e] += s_off[e];
  }
  if (tid == 0) {
    offsets[E] = P;
    s_off[E] = P;
  }
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
    if (valid) slot = hist[wave * E + e];
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      pair_index[slot + rank] = p;
      if (rank == cnt - 1) hist[wave * E + e] = slot + cnt;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Grouping for small batches (P = n*k <= kSmallPairs) with the pair ids in LDS: thread e
// computes offsets[e] = #{q : ids[q] < e} and pair p lands at
// #{q : ids[q] < ids[p]} + #{q < p : ids[q] == ids[p]}, the position a stable counting sort
// gives it. O(P) LDS broadcasts per thread, no atomics and no scans.
constexpr int kSmallPairs = 256;

__device__ __forceinline__ void group_small(const int* s_ids, int P, int E, int32_t* __restrict__ offsets,
                                   int32_t* __restrict__ pair_index) {
  // s_ids holds P ids followed by padding up to a multiple of 4 filled with INT_MAX, which
  // is neither below nor equal to any expert id
  const int tid = threadIdx.x, nt = blockDim.x;
  const int4* s4 = reinterpret_cast<const int4*>(s_ids);
  const int P4 = (P + 3) / 4;
  for (int e = tid; e <= E; e += nt) {
    int c = 0;
#pragma unroll 4
    for (int q = 0; q < P4; ++q) {
      const int4 v = s4[q];
      c += (v.x < e) + (v.y < e) + (v.z < e) + (v.w < e);
    }
    offsets[e] = c;
  }
  for (int p = tid; p < P; p += nt) {
    const int ep = s_ids[p];
    int pos = 0;
#pragma unroll 4
    for (int q = 0; q < P4; ++q) {
      const int4 v = s4[q];
      const int q0 = 4 * q;
      pos += (v.x < ep) | ((v.x == ep) & (q0 < p));
      pos += (v.y < ep) | ((v.y == ep) & (q0 + 1 < p));
      pos += (v.z < ep) | ((v.z == ep) & (q0 + 2 < p));
      pos += (v.w < ep) | ((v.w == ep) & (q0 + 3 < p));
    }
    pair_index[pos] = p;
  }
}

// The same stable grouping for P <= 64 pairs, from registers: every wave holds the P ids
// in one register (lane q: ids[q]) and reads them back lane by lane. Thread e counts the
// ids below e (offsets[e]); the last wave ranks the keys id*64 + p, which are distinct
// and order the pairs by (expert, pair index), so pair p lands at its key's rank.
__device__ __forceinline__ void group_tiny(const int* s_ids, int P, int E,
                                           int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ pair_index) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & (kWave - 1);
  const int idv = lane < P ? s_ids[lane] : 0x7fffffff;
  // wave-uniform loop: every lane is active around the lane reads
  for (int e0 = tid - lane; e0 <= E; e0 += nt) {
    const int e = e0 + lane;
    int c = 0;
    for (int q0 = 0; q0 < P; q0 += 8) {  // lanes past P hold INT_MAX: never counted
#pragma unroll
      for (int i = 0; i < 8; ++i) c += __builtin_amdgcn_readlane(idv, q0 + i) < e;
    }
    if (e <= E) offsets[e] = c;
  }
  if (tid >= nt - kWave) {
    const int key = lane < P ? idv * kWave + lane : 0x7fffffff;
    int pos = 0;
    for (int q0 = 0; q0 < P; q0 += 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) pos += __builtin_amdgcn_readlane(key, q0 + i) < key;
    }
    if (lane < P) pair_index[pos] = lane;
  }
}

}  // namespace qmoe

// Decode-window expert FFN: the hot path of the routed-expert layer for T <= 5 tokens.
//
// The pages' engine computes cached experts for the whole verify window in one grouped
// kernel (Strata engine explainer, m.lqnn.cn/news/264700, section "Expert cache") and
// its CPU kernels quantize each activation vector to int8 once and reuse it over many
// weight rows with 4-wide int8 dot products (section "CPU expert pool"). Here:
//
//   k_prep      one lane per (token, 32-block): int8 block quantization of x, stored in
//               a byte order matched to the packed weight nibbles; block 0 of the grid
//               turns the expert offsets into a work list of (expert, pair range) chunks.
//   k_gateup    one lane per weight row, 64 rows per wavefront, the four waves of a
//               workgroup split the reduction blocks. Each lane streams its row's packed
//               codes (16 B per block at 4 bits: one block column of 64 rows is 1 KB
//               contiguous) and scale/min words, and forms exact int32 block dots with
//               v_dot4 against activation words that are wave-uniform (scalar loads).
//               Block terms (scale*xs)*dot and min*(xs*sum) are exact in binary64, so the
//               row sums round only in the additions. The workgroup then applies SwiGLU
//               and quantizes h per 32 rows (two halves of a wave) to int8.
//   k_down      the same streaming scheme over the down projection's d rows.
//   k_combine   residual[t] += sum_j w[t][j] * y[t*k+j] in slot order, binary64.
//
// Every expert's weights are read once per chunk of up to NPC pairs; at n <= NPC tokens
// (the T = 4 window) every touched expert is read exactly once per call.
#include <algorithm>

#include "qmoe_internal.h"

namespace qmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// ---------------------------------------------------------------- int8 block quantizer

// Quantize one 32-value block held as v[32]: returns scale; q receives codes.
__device__ __forceinline__ float quant_block32(const float (&v)[32], int (&q)[32]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float a = fabsf(v[i]);
    amax = a > amax ? a : amax;
  }
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

// ---------------------------------------------------------------- prep: x quant + work list

template <int BITS>
__global__ __launch_bounds__(kThreads) void k_prep(
    const float* __restrict__ x, int n, int d, const int32_t* __restrict__ offsets, int E, int npc,
    int4* __restrict__ chunks, int* __restrict__ nchunks, int8_t* __restrict__ xq,
    double2* __restrict__ xsc, int8_t* __restrict__ dbg_xq, float* __restrict__ dbg_xs) {
  if (blockIdx.x == 0) {
    // work list: expert e with c pairs contributes ceil(c/npc) chunks, in expert order
    __shared__ int s_wsum[kWaves];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    constexpr int per = MOE_MAX_EXPERTS / kThreads;  // experts per thread (4)
    int cnt[per], sum = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int e = tid * per + i;
      const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
      cnt[i] = (c + npc - 1) / npc;
      sum += cnt[i];
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_wsum[w];
    base += incl - sum;
#pragma unroll
    for (int i = 0; i < per; ++i) {
      const int e = tid * per + i;
      if (e < E) {
        const int beg = offsets[e], c = offsets[e + 1] - beg;
        for (int j = 0; j < cnt[i]; ++j)
          chunks[base + j] = make_int4(e, beg + j * npc, min(npc, c - j * npc), 0);
      }
      base += cnt[i];
    }
    if (tid == kThreads - 1) *nchunks = base;
    return;
  }
  const int nbd = d / 32;
  const int gid = (blockIdx.x - 1) * kThreads + threadIdx.x;
  if (gid >= n * nbd) return;
  const int t = gid / nbd, b = gid % nbd;
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
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) sum += q[i];
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

// ---------------------------------------------------------------- streaming block loads

template <int BITS>
struct BlockLoad;
template <>
struct BlockLoad<4> {
  __device__ static __forceinline__ void load(const uint32_t* p, uint32_t (&w)[4]) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
  }
};
template <>
struct BlockLoad<2> {
  __device__ static __forceinline__ void load(const uint32_t* p, uint32_t (&w)[2]) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x;
    w[1] = v.y;
  }
};

// Sum the four waves' partial row sums in wave order (deterministic).
template <int NPC>
__device__ __forceinline__ double reduce_waves(double (*red)[NPC][kWave], int j, int lane) {
  double s = red[0][j][lane];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) s += red[w][j][lane];
  return s;
}

// Quantize h over 32-lane halves of a wave (rows 32b .. 32b+31): returns the code; the
// scale and the code sum of the half are returned through scale/sum.
__device__ __forceinline__ int quant_half_wave(float h, float& scale, int& sum) {
  float amax = fabsf(h);
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    const float o = __shfl_xor(amax, off);
    amax = o > amax ? o : amax;
  }
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
  sum = q;
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) sum += __shfl_xor(sum, off);
  return q;
}

// ---------------------------------------------------------------- gate/up + SwiGLU + h quant

template <int BITS, int NPC, bool DBG>
__global__ __launch_bounds__(kThreads) void k_gateup(
    const uint32_t* __restrict__ gcodes, const uint32_t* __restrict__ gsm,
    const uint32_t* __restrict__ ucodes, const uint32_t* __restrict__ usm, int d, int f, int k,
    const int4* __restrict__ chunks, const int* __restrict__ nchunks,
    const int32_t* __restrict__ pair_index, const int8_t* __restrict__ xq,
    const double2* __restrict__ xsc, int8_t* __restrict__ hq, double2* __restrict__ hsc,
    DecodeDebug dbg) {
  __shared__ double red_g[kWaves][NPC][kWave];
  __shared__ double red_u[kWaves][NPC][kWave];
  const int nbd = d / 32, nbf = f / 32;
  const int ntiles = (f + kWave - 1) / kWave;
  const int nitems = *nchunks * ntiles;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int4 ch = chunks[item / ntiles];
    const int tile = item % ntiles;
    const int e = ch.x, pbeg = ch.y, np = ch.z;
    const int r = tile * kWave + lane;
    const bool rvalid = r < f;
    const int rr = rvalid ? r : 0;
    int pid[NPC], tok[NPC];
#pragma unroll
    for (int j = 0; j < NPC; ++j) {
      pid[j] = j < np ? pair_index[pbeg + j] : 0;
      tok[j] = pid[j] / k;
    }
    double ag[NPC], au[NPC];
#pragma unroll
    for (int j = 0; j < NPC; ++j) ag[j] = au[j] = 0.0;
    for (int b = wave; b < nbd; b += kWaves) {
      const size_t blk = ((size_t)e * nbd + b) * f + rr;
      uint32_t gw[BITS], uw[BITS];
      BlockLoad<BITS>::load(gcodes + blk * BITS, gw);
      BlockLoad<BITS>::load(ucodes + blk * BITS, uw);
      const uint32_t gsmw = gsm[blk], usmw = usm[blk];
      const double gs = half_bits_to_double(gsmw & 0xffffu), gm = half_bits_to_double(gsmw >> 16);
      const double us = half_bits_to_double(usmw & 0xffffu), um = half_bits_to_double(usmw >> 16);
#pragma unroll
      for (int j = 0; j < NPC; ++j) {
        if (j < np) {
          const int* a = reinterpret_cast<const int*>(xq + (size_t)tok[j] * d + 32 * b);
          const double2 sc = xsc[(size_t)tok[j] * nbd + b];
          const int dg = block_dot<BITS>(gw, a);
          const int du = block_dot<BITS>(uw, a);
          ag[j] += (gs * sc.x) * (double)dg;
          ag[j] += gm * sc.y;
          au[j] += (us * sc.x) * (double)du;
          au[j] += um * sc.y;
          if (DBG && rvalid) {
            if (dbg.gate_dots) dbg.gate_dots[((size_t)pid[j] * f + r) * nbd + b] = dg;
            if (dbg.up_dots) dbg.up_dots[((size_t)pid[j] * f + r) * nbd + b] = du;
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NPC; ++j) {
      if (j < np) {
        red_g[wave][j][lane] = ag[j];
        red_u[wave][j][lane] = au[j];
      }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int j = 0; j < NPC; ++j) {
        if (j < np) {
          const double g = reduce_waves<NPC>(red_g, j, lane);
          const double u = reduce_waves<NPC>(red_u, j, lane);
          const double silu = g / (1.0 + exp(-g));
          const float h = rvalid ? (float)(silu * u) : 0.0f;
          float scale;
          int qsum;
          const int q = quant_half_wave(h, scale, qsum);
          const int hb = r / 32;
          if (rvalid) {
            hq[(size_t)pid[j] * f + 32 * hb + act_byte_pos<BITS>(r % 32)] = (int8_t)q;
            if ((lane & 31) == 0)
              hsc[(size_t)pid[j] * nbf + hb] = make_double2((double)scale, (double)scale * qsum);
          }
          if (DBG && rvalid) {
            if (dbg.g) dbg.g[(size_t)pid[j] * f + r] = (float)g;
            if (dbg.u) dbg.u[(size_t)pid[j] * f + r] = (float)u;
            if (dbg.h) dbg.h[(size_t)pid[j] * f + r] = h;
            if (dbg.hq) dbg.hq[(size_t)pid[j] * f + r] = (int8_t)q;
            if (dbg.hs && (lane & 31) == 0) dbg.hs[(size_t)pid[j] * nbf + hb] = scale;
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- down projection

template <int BITS, int NPC, bool DBG>
__global__ __launch_bounds__(kThreads) void k_down(
    const uint32_t* __restrict__ dcodes, const uint32_t* __restrict__ dsm, int d, int f,
    const int4* __restrict__ chunks, const int* __restrict__ nchunks,
    const int32_t* __restrict__ pair_index, const int8_t* __restrict__ hq,
    const double2* __restrict__ hsc, double* __restrict__ y, DecodeDebug dbg) {
  __shared__ double red[kWaves][NPC][kWave];
  const int nbf = f / 32;
  const int ntiles = (d + kWave - 1) / kWave;
  const int nitems = *nchunks * ntiles;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int4 ch = chunks[item / ntiles];
    const int tile = item % ntiles;
    const int e = ch.x, pbeg = ch.y, np = ch.z;
    const int r = tile * kWave + lane;
    const bool rvalid = r < d;
    const int rr = rvalid ? r : 0;
    int pid[NPC];
#pragma unroll
    for (int j = 0; j < NPC; ++j) pid[j] = j < np ? pair_index[pbeg + j] : 0;
    double ay[NPC];
#pragma unroll
    for (int j = 0; j < NPC; ++j) ay[j] = 0.0;
    for (int b = wave; b < nbf; b += kWaves) {
      const size_t blk = ((size_t)e * nbf + b) * d + rr;
      uint32_t dw[BITS];
      BlockLoad<BITS>::load(dcodes + blk * BITS, dw);
      const uint32_t smw = dsm[blk];
      const double s = half_bits_to_double(smw & 0xffffu), m = half_bits_to_double(smw >> 16);
#pragma unroll
      for (int j = 0; j < NPC; ++j) {
        if (j < np) {
          const int* a = reinterpret_cast<const int*>(hq + (size_t)pid[j] * f + 32 * b);
          const double2 sc = hsc[(size_t)pid[j] * nbf + b];
          const int dd = block_dot<BITS>(dw, a);
          ay[j] += (s * sc.x) * (double)dd;
          ay[j] += m * sc.y;
          if (DBG && rvalid && dbg.down_dots)
            dbg.down_dots[((size_t)pid[j] * d + r) * nbf + b] = dd;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NPC; ++j)
      if (j < np) red[wave][j][lane] = ay[j];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int j = 0; j < NPC; ++j) {
        if (j < np && rvalid) {
          const double v = reduce_waves<NPC>(red, j, lane);
          y[(size_t)pid[j] * d + r] = v;
          if (DBG && dbg.y) dbg.y[(size_t)pid[j] * d + r] = (float)v;
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- combine

__global__ __launch_bounds__(kThreads) void k_combine(const double* __restrict__ y,
                                                      const float* __restrict__ w, int n, int d,
                                                      int k, float* residual) {
  const int gid = blockIdx.x * kThreads + threadIdx.x;
  if (gid >= n * d) return;
  const int t = gid / d, c = gid % d;
  double acc = 0.0;
  for (int j = 0; j < k; ++j)
    acc += (double)w[(size_t)t * k + j] * y[((size_t)t * k + j) * d + c];
  residual[gid] = (float)((double)residual[gid] + acc);
}

// ---------------------------------------------------------------- host side

template <int BITS, int NPC, bool DBG>
hipError_t launch_ffn(const DecodeArgs& a) {
  const moe_layer& L = *a.L;
  const int n = a.n, d = L.d_model, f = L.d_ff, k = L.top_k, E = L.n_experts;
  const DecodeWs W = decode_ws_layout(n, k, d, f);
  int4* chunks = reinterpret_cast<int4*>(a.ws + W.chunks);
  int* nchunks = reinterpret_cast<int*>(a.ws + W.nchunks);
  int8_t* xq = reinterpret_cast<int8_t*>(a.ws + W.xq);
  double2* xsc = reinterpret_cast<double2*>(a.ws + W.xsc);
  int8_t* hq = reinterpret_cast<int8_t*>(a.ws + W.hq);
  double2* hsc = reinterpret_cast<double2*>(a.ws + W.hsc);
  double* y = reinterpret_cast<double*>(a.ws + W.y);
  DecodeDebug dbg{};
  if (DBG) dbg = *a.dbg;

  const int nbd = d / 32;
  hipError_t err = hipSuccess;
  if (a.stages & MOE_DECODE_PREP) {
    const int prep_blocks = 1 + (n * nbd + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(k_prep<BITS>, dim3(prep_blocks), dim3(kThreads), 0, a.stream, a.x, n, d,
                       a.r->expert_offsets, E, NPC, chunks, nchunks, xq, xsc,
                       DBG ? dbg.xq : nullptr, DBG ? dbg.xs : nullptr);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }

  // upper bound of chunks: every chunk holds >= 1 pair, and an expert holds <= n pairs
  const long long max_chunks =
      std::min<long long>((long long)n * k, (long long)E * ((n + NPC - 1) / NPC));
  const int cap = a.num_cus * 8;
  if (a.stages & MOE_DECODE_GATE_UP) {
    const long long gu_items = max_chunks * ((f + kWave - 1) / kWave);
    const int gu_grid = (int)std::max<long long>(1, std::min<long long>(gu_items, cap));
    hipLaunchKernelGGL((k_gateup<BITS, NPC, DBG>), dim3(gu_grid), dim3(kThreads), 0, a.stream,
                       L.gate.codes, reinterpret_cast<const uint32_t*>(L.gate.scale_min),
                       L.up.codes, reinterpret_cast<const uint32_t*>(L.up.scale_min), d, f, k,
                       chunks, nchunks, a.r->pair_index, xq, xsc, hq, hsc, dbg);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (a.stages & MOE_DECODE_DOWN) {
    const long long dn_items = max_chunks * ((d + kWave - 1) / kWave);
    const int dn_grid = (int)std::max<long long>(1, std::min<long long>(dn_items, cap));
    hipLaunchKernelGGL((k_down<BITS, NPC, DBG>), dim3(dn_grid), dim3(kThreads), 0, a.stream,
                       L.down.codes, reinterpret_cast<const uint32_t*>(L.down.scale_min), d, f,
                       chunks, nchunks, a.r->pair_index, hq, hsc, y, dbg);
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
  if (a.n <= 4) return launch_ffn<BITS, 4, DBG>(a);
  return launch_ffn<BITS, 8, DBG>(a);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a) {
  const bool dbg = a.dbg != nullptr;
  if (a.L->gate.bits == 4) return dbg ? launch_bits<4, true>(a) : launch_bits<4, false>(a);
  return dbg ? launch_bits<2, true>(a) : launch_bits<2, false>(a);
}

}  // namespace qmoe

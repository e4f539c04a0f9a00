// Prefill-chunk expert FFN on the bf16 matrix cores.
//
// The pages' engine cuts prompts into chunks of at most 8192 tokens and runs the expert
// matrices of a chunk as quantized matrix multiplications (Strata engine explainer,
// m.lqnn.cn/news/264700, "Architecture overview" and "Doorbell handshake"). Here a chunk
// is a grouped GEMM over experts: the token-expert pairs of an expert (contiguous in the
// grouped pair list) form the M dimension of that expert's GEMM.
//
//   k_pf_prep     M-tile work list (expert, first grouped position, rows) and the token
//                 and grouped-position maps of every pair.
//   k_pf_gateup   one workgroup per (M-tile of 128 pairs, 128 rows of f): the gathered bf16
//                 activations and the gate and up weight tiles, dequantized from the packed
//                 codes to bf16 (bf16 of fp32 scale*q + min) straight into LDS, go through
//                 v_mfma_f32_32x32x16_bf16 with fp32 accumulators; the epilogue applies
//                 SwiGLU and writes h = bf16(silu(g) * u) in grouped pair order.
//   k_pf_down     the same GEMM over (M-tile, 128 output columns) with h as the A operand
//                 and the dequantized down tile as B, fp32 outputs y in grouped order.
//   k_pf_combine  residual[t] += sum_j w[t][j] * y[pair (t, j)], slot order, binary64 sum.
//
// The K loop steps over one 32-column quantization block at a time with two LDS buffers:
// the global loads of step k+1 are issued before the matrix-core work of step k.
#include <algorithm>

#include "qmoe_internal.h"

namespace qmoe {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kBM = kPrefillBM;  // pairs per M-tile
constexpr int kBN = 128;         // weight rows (output columns) per N-tile
constexpr int kBK = 32;          // one quantization block of the reduction axis
constexpr int kLdsRow = kBK + 8; // bf16 per LDS row (padding against bank conflicts)
constexpr int kPfThreads = 512;  // 8 waves
constexpr int kPfWaves = kPfThreads / kWave;

// ---------------------------------------------------------------- prep

__global__ __launch_bounds__(1024) void k_pf_prep(const int32_t* __restrict__ offsets,
                                                  const int32_t* __restrict__ pair_index, int E,
                                                  int k, int P, int4* __restrict__ tiles,
                                                  int* __restrict__ ntiles,
                                                  int* __restrict__ tok_of_g,
                                                  int* __restrict__ g_of_p) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    __shared__ int s_wsum[16];
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int e = tid;
    const int beg = e < E ? offsets[e] : 0;
    const int m = e < E ? offsets[e + 1] - beg : 0;
    const int cnt = (m + kBM - 1) / kBM;
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int base = incl - cnt;
    for (int w = 0; w < wave; ++w) base += s_wsum[w];
    for (int i = 0; i < cnt; ++i)
      tiles[base + i] = make_int4(e, beg + i * kBM, min(kBM, m - i * kBM), 0);
    if (tid == 1023) *ntiles = base + cnt;
    return;
  }
  const int g = (blockIdx.x - 1) * 1024 + tid;
  if (g >= P) return;
  const int p = pair_index[g];
  tok_of_g[g] = p / k;
  g_of_p[p] = g;
}

// ---------------------------------------------------------------- dequantization

// 8 consecutive codes (block positions 8*seg .. 8*seg+7) of one packed block -> 8 bf16 of
// fp32(scale*q + min) rounded to nearest even.
template <int BITS>
__device__ __forceinline__ bf16x8 dequant8(const uint32_t (&words)[BITS], int seg, uint32_t sm) {
  constexpr int per = 32 / BITS;
  const int i0 = 8 * seg;
  const uint32_t w = words[i0 / per];
  const int sh0 = BITS * (i0 % per);
  const float s = half_bits_to_float(sm & 0xffffu), mn = half_bits_to_float(sm >> 16);
  bf16x8 out;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t q = (w >> (sh0 + BITS * i)) & ((1u << BITS) - 1u);
    out[i] = (__bf16)__builtin_fmaf(s, (float)q, mn);
  }
  return out;
}

template <int BITS>
struct Words;
template <>
struct Words<4> {
  __device__ static __forceinline__ void load(const uint32_t* p, uint32_t (&w)[4]) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
  }
};
template <>
struct Words<2> {
  __device__ static __forceinline__ void load(const uint32_t* p, uint32_t (&w)[2]) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x;
    w[1] = v.y;
  }
};

// XCD-aware placement. Workgroups are dealt to the 8 XCDs round robin by workgroup id;
// XCD x takes the contiguous item range [x*per, (x+1)*per) of the live items, so that the
// consecutive M-tiles of one expert share that XCD's L2 for the expert's weight tiles.
// The grid is sized for the largest possible item count; returns -1 for idle workgroups.
__device__ __forceinline__ int xcd_item(int nitems) {
  const int per = (nitems + 7) / 8;
  const int slot = (int)(blockIdx.x / 8);
  const int item = (int)(blockIdx.x % 8) * per + slot;
  return (slot < per && item < nitems) ? item : -1;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// ---------------------------------------------------------------- gate/up GEMM

template <int BITS>
__global__ __launch_bounds__(kPfThreads) void k_pf_gateup(
    const uint32_t* __restrict__ gcodes, const uint32_t* __restrict__ gsm,
    const uint32_t* __restrict__ ucodes, const uint32_t* __restrict__ usm, int d, int f,
    const int4* __restrict__ tiles, const int* __restrict__ ntiles,
    const uint16_t* __restrict__ x, const int* __restrict__ tok_of_g, uint16_t* __restrict__ h,
    int) {
  typedef __bf16 Tile[kBM][kLdsRow];
  __shared__ __attribute__((aligned(16))) char smem[6 * sizeof(Tile)];
  Tile* sA = reinterpret_cast<Tile*>(smem);
  Tile* sG = sA + 2;
  Tile* sU = sA + 4;
  const int ntn = (f + kBN - 1) / kBN;
  const int item = xcd_item(load_uniform(ntiles) * ntn);
  if (item < 0) return;
  const int mt = item / ntn, nt = item % ntn;
  const int4 tile = load_uniform(tiles + mt);
  const int e = tile.x, g0 = tile.y, rows = tile.z;
  const int nbd = d / kBK;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

  // load roles: thread -> (tile row lr, 8-column segment seg)
  const int lr = tid / 4, seg = tid % 4;
  const int tok = tok_of_g[g0 + min(lr, rows - 1)];  // padded rows repeat a valid token
  const uint16_t* xrow = x + (size_t)tok * d + 8 * seg;
  const int wrow = min(nt * kBN + lr, f - 1);  // rows past f load row f-1, never stored

  uint4 xa;
  uint32_t gw[BITS], uw[BITS], gs, us;
  auto gload = [&](int kb) {
    xa = *reinterpret_cast<const uint4*>(xrow + kb * kBK);
    const size_t blk = ((size_t)e * nbd + kb) * f + wrow;
    Words<BITS>::load(gcodes + blk * BITS, gw);
    Words<BITS>::load(ucodes + blk * BITS, uw);
    gs = gsm[blk];
    us = usm[blk];
  };
  auto lstore = [&](int buf) {
    *reinterpret_cast<uint4*>(&sA[buf][lr][8 * seg]) = xa;
    *reinterpret_cast<bf16x8*>(&sG[buf][lr][8 * seg]) = dequant8<BITS>(gw, seg, gs);
    *reinterpret_cast<bf16x8*>(&sU[buf][lr][8 * seg]) = dequant8<BITS>(uw, seg, us);
  };

  // wave tile: 32 pairs x 64 weight rows of both matrices
  const int wm = (wave / 2) * 32, wn = (wave % 2) * 64;
  f32x16 accg[2], accu[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) accg[j][i] = accu[j][i] = 0.0f;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kb = 0; kb < nbd; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nbd) gload(kb + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kk = ks * 16 + (lane / 32) * 8;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sA[buf][wm + lane % 32][kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 bg = *reinterpret_cast<const bf16x8*>(&sG[buf][wn + 32 * j + lane % 32][kk]);
        const bf16x8 bu = *reinterpret_cast<const bf16x8*>(&sU[buf][wn + 32 * j + lane % 32][kk]);
        accg[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bg, accg[j], 0, 0, 0);
        accu[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bu, accu[j], 0, 0, 0);
      }
    }
    if (kb + 1 < nbd) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: h = bf16(silu(g) * u), staged per wave in LDS for 16-byte global stores
  __bf16* st = reinterpret_cast<__bf16*>(smem) + wave * (32 * 64);  // 4 KB per wave
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = (i / 4) * 8 + (lane / 32) * 4 + (i % 4);
      const int cc = 32 * j + lane % 32;
      st[rr * 64 + cc] = (__bf16)silu_mul(accg[j][i], accu[j][i]);
    }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = lane + kWave * q;  // 256 chunks of 8 bf16
    const int rr = c / 8, cc = (c % 8) * 8;
    const int col = nt * kBN + wn + cc;
    if (wm + rr < rows && col < f) {
      const uint4 v = *reinterpret_cast<const uint4*>(&st[rr * 64 + cc]);
      *reinterpret_cast<uint4*>(h + (size_t)(g0 + wm + rr) * f + col) = v;
    }
  }
}

// ---------------------------------------------------------------- down GEMM

template <int BITS>
__global__ __launch_bounds__(kPfThreads) void k_pf_down(
    const uint32_t* __restrict__ dcodes, const uint32_t* __restrict__ dsm, int d, int f,
    const int4* __restrict__ tiles, const int* __restrict__ ntiles,
    const uint16_t* __restrict__ h, float* __restrict__ y, int) {
  typedef __bf16 Tile[kBM][kLdsRow];
  __shared__ __attribute__((aligned(16))) char smem[4 * sizeof(Tile)];
  Tile* sA = reinterpret_cast<Tile*>(smem);
  Tile* sW = sA + 2;
  const int ntn = (d + kBN - 1) / kBN;
  const int item = xcd_item(load_uniform(ntiles) * ntn);
  if (item < 0) return;
  const int mt = item / ntn, nt = item % ntn;
  const int4 tile = load_uniform(tiles + mt);
  const int e = tile.x, g0 = tile.y, rows = tile.z;
  const int nbf = f / kBK;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

  const int lr = tid / 4, seg = tid % 4;
  const uint16_t* hrow = h + (size_t)(g0 + min(lr, rows - 1)) * f + 8 * seg;
  const int wrow = min(nt * kBN + lr, d - 1);  // rows past d load row d-1, never stored

  uint4 ha;
  uint32_t dw[BITS], ds;
  auto gload = [&](int kb) {
    ha = *reinterpret_cast<const uint4*>(hrow + kb * kBK);
    const size_t blk = ((size_t)e * nbf + kb) * d + wrow;
    Words<BITS>::load(dcodes + blk * BITS, dw);
    ds = dsm[blk];
  };
  auto lstore = [&](int buf) {
    *reinterpret_cast<uint4*>(&sA[buf][lr][8 * seg]) = ha;
    *reinterpret_cast<bf16x8*>(&sW[buf][lr][8 * seg]) = dequant8<BITS>(dw, seg, ds);
  };

  const int wm = (wave / 2) * 32, wn = (wave % 2) * 64;
  f32x16 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kb = 0; kb < nbf; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nbf) gload(kb + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kk = ks * 16 + (lane / 32) * 8;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sA[buf][wm + lane % 32][kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(&sW[buf][wn + 32 * j + lane % 32][kk]);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
      }
    }
    if (kb + 1 < nbf) lstore(buf ^ 1);
    __syncthreads();
  }
  // y in grouped order: lanes 0..31 of a row write 32 consecutive floats
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = wm + (i / 4) * 8 + (lane / 32) * 4 + (i % 4);
      const int col = nt * kBN + wn + 32 * j + lane % 32;
      if (rr < rows && col < d) y[(size_t)(g0 + rr) * d + col] = acc[j][i];
    }
}

// ---------------------------------------------------------------- combine

// One workgroup per token, 4 columns per thread: the token's k pair-output rows are all
// requested before the first is summed, then residual[t] += sum_j w[t][j] * y[g(t,j)] in
// slot order (binary64, one rounding).
constexpr int kCombineBatch = 16;

__global__ __launch_bounds__(1024) void k_pf_combine(const float* __restrict__ y,
                                                     const int* __restrict__ g_of_p,
                                                     const float* __restrict__ w, int d, int k,
                                                     float* residual) {
  const int t = blockIdx.x;
  for (int c = 4 * threadIdx.x; c < d; c += 4 * blockDim.x) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
      float4 v[kCombineBatch];
      float wj[kCombineBatch];
#pragma unroll
      for (int i = 0; i < kCombineBatch; ++i) {
        if (j0 + i < k) {
          const int g = load_uniform(g_of_p + (size_t)t * k + j0 + i);
          wj[i] = w[(size_t)t * k + j0 + i];
          v[i] = *reinterpret_cast<const float4*>(y + (size_t)g * d + c);
        }
      }
#pragma unroll
      for (int i = 0; i < kCombineBatch; ++i) {
        if (j0 + i < k) {
          const double wd = (double)wj[i];
          acc[0] += wd * (double)v[i].x;
          acc[1] += wd * (double)v[i].y;
          acc[2] += wd * (double)v[i].z;
          acc[3] += wd * (double)v[i].w;
        }
      }
    }
    float4* rp = reinterpret_cast<float4*>(residual + (size_t)t * d + c);
    float4 r = *rp;
    r.x = (float)((double)r.x + acc[0]);
    r.y = (float)((double)r.y + acc[1]);
    r.z = (float)((double)r.z + acc[2]);
    r.w = (float)((double)r.w + acc[3]);
    *rp = r;
  }
}

template <int BITS>
hipError_t launch_prefill_bits(const PrefillArgs& a) {
  const moe_layer& L = *a.L;
  const int n = a.n, d = L.d_model, f = L.d_ff, k = L.top_k, E = L.n_experts;
  const int P = n * k;
  const PrefillWs W = prefill_ws_layout(n, k, d, f, E);
  if (P == 0) return hipSuccess;
  int4* tiles = reinterpret_cast<int4*>(a.ws + W.tiles);
  int* ntiles = reinterpret_cast<int*>(a.ws + W.ntiles);
  int* tok_of_g = reinterpret_cast<int*>(a.ws + W.tok_of_g);
  int* g_of_p = reinterpret_cast<int*>(a.ws + W.g_of_p);
  uint16_t* h = reinterpret_cast<uint16_t*>(a.ws + W.h);
  float* y = reinterpret_cast<float*>(a.ws + W.y);

  hipError_t err = hipSuccess;
  if (a.stages & MOE_PREFILL_PREP) {
    hipLaunchKernelGGL(k_pf_prep, dim3(1 + (P + 1023) / 1024), dim3(1024), 0, a.stream,
                       a.r->expert_offsets, a.r->pair_index, E, k, P, tiles, ntiles, tok_of_g,
                       g_of_p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }

  const int max_mt = prefill_max_mtiles(P, E);
  if (a.stages & MOE_PREFILL_GATE_UP) {
    const int gu_items = ((max_mt * ((f + kBN - 1) / kBN) + 7) / 8) * 8;
    hipLaunchKernelGGL(k_pf_gateup<BITS>, dim3(gu_items), dim3(kPfThreads), 0, a.stream,
                       L.gate.codes, reinterpret_cast<const uint32_t*>(L.gate.scale_min),
                       L.up.codes, reinterpret_cast<const uint32_t*>(L.up.scale_min), d, f, tiles,
                       ntiles, a.x, tok_of_g, h, gu_items);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (a.stages & MOE_PREFILL_DOWN) {
    const int dn_items = ((max_mt * ((d + kBN - 1) / kBN) + 7) / 8) * 8;
    hipLaunchKernelGGL(k_pf_down<BITS>, dim3(dn_items), dim3(kPfThreads), 0, a.stream,
                       L.down.codes, reinterpret_cast<const uint32_t*>(L.down.scale_min), d, f,
                       tiles, ntiles, h, y, dn_items);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (a.stages & MOE_PREFILL_COMBINE) {
    const int threads = std::min(1024, ((d / 4 + kWave - 1) / kWave) * kWave);
    hipLaunchKernelGGL(k_pf_combine, dim3(n), dim3(threads), 0, a.stream, y, g_of_p,
                       a.r->topk_w, d, k, a.residual);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a) {
  if (a.L->gate.bits == 4) return launch_prefill_bits<4>(a);
  return launch_prefill_bits<2>(a);
}

}  // namespace qmoe

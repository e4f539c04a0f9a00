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
//   k_pf_gateup   one workgroup per (M-tile of 256 pairs, 128 rows of f): the gathered bf16
//                 activations and the gate and up weight tiles, dequantized from the packed
//                 codes to bf16 (bf16 of fp32 scale*q + min) straight into LDS, go through
//                 v_mfma_f32_32x32x16_bf16 with fp32 accumulators; the epilogue applies
//                 SwiGLU and writes h = bf16(silu(g) * u) in grouped pair order.
//   k_pf_down     the same GEMM over (M-tile, 128 output columns) with h as the A operand
//                 and the dequantized down tile as B, fp32 outputs y in grouped order.
//   k_pf_combine  residual[t] += sum_j w[t][j] * y[pair (t, j)], slot order, binary64 sum.
//
// The K loop steps over one 32-column quantization block at a time with two LDS buffers
// (see GemmCore below).
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

// Thread (row lr, segment seg) of a K-step dequantizes codes 8*seg .. 8*seg+7 of one
// 32-weight block: one 32-bit code word (4-bit: word seg; 2-bit: half of word seg/2).
template <int BITS>
__device__ __forceinline__ int code_word_index(int seg) {
  return BITS == 4 ? seg : seg / 2;
}

// 8 codes of one word -> 8 bf16 of fp32(scale*q + min) rounded to nearest even (scale*q
// is exact in fp32, so the fma rounds once, like the separate multiply and add).
template <int BITS>
__device__ __forceinline__ bf16x8 dequant_word(uint32_t w, int seg, uint32_t sm) {
  const float s = half_bits_to_float(sm & 0xffffu), mn = half_bits_to_float(sm >> 16);
  float q[8];
  if (BITS == 4) {
    // byte j of lo holds code 2j, byte j of hi code 2j+1 (byte-to-float conversions)
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      q[2 * j] = (float)((lo >> (8 * j)) & 0xffu);
      q[2 * j + 1] = (float)((hi >> (8 * j)) & 0xffu);
    }
  } else {
    const uint32_t v = w >> (16 * (seg & 1));
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = (float)((v >> (2 * i)) & 3u);
  }
  bf16x8 out;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = (__bf16)__builtin_fmaf(s, q[i], mn);
  return out;
}

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

// ---------------------------------------------------------------- grouped GEMM core
//
// One workgroup computes a kBM (256 pairs) x kBN (128 weight rows) tile for NMAT weight
// matrices that share the A operand. 8 waves: wave w covers pairs 64*(w/2) .. +64 and
// weight rows 64*(w%2) .. +64 of every matrix with 2 x 2 x NMAT accumulators of 32x32, so
// each A fragment read from LDS feeds 2*NMAT matrix-core ops and each B fragment 2, and
// each dequantized weight serves 256 pairs. Waves whose pair range lies past the tile's
// rows skip their matrix-core work. Each K-step is one 32-wide quantization block.
// Thread (lr = tid/4, seg = tid%4) brings in 8 consecutive A values of rows lr and lr+128
// and one code word plus the scale/min word of weight row lr of each matrix, and writes
// them (dequantized) into the LDS buffer of its K-step. Raw operands run two K-steps
// ahead in a register ring; step kb dequantizes step kb+1 into the other LDS buffer right
// after issuing its matrix-core work.
//
// (Measured on MI355X: the dequantization and the matrix-core work of a SIMD do not
// overlap, whether they are issued by the same waves or by separate producer and consumer
// waves; the time per tile is their sum, so the 256-pair tile, which halves the
// dequantization per flop against a 128-pair tile, is the one that pays.)
constexpr int kGemmThreads = 512;
static_assert(kBM == 256 && kBN == 128, "tile shape of the grouped GEMM core");

template <int BITS, int NMAT>
struct GemmCore {
  typedef __bf16 ATile[kBM][kLdsRow];
  typedef __bf16 BTile[kBN][kLdsRow];
  static constexpr size_t kLdsBytes = 2 * sizeof(ATile) + (size_t)2 * NMAT * sizeof(BTile);

  struct Raw {
    uint4 a[2];
    uint32_t w[NMAT], sm[NMAT];
  };

  ATile* sA;                    // [2]
  BTile* sB;                    // [NMAT][2]
  const uint16_t* arow[2];      // A rows lr and lr+128 of this thread, at column 8*seg
  const uint32_t* wcol[NMAT];   // code word of weight row lr at K-step 0
  const uint32_t* smcol[NMAT];  // scale/min word at K-step 0
  size_t wstep, smstep;         // stride of one K-step in words
  int lr, seg, lane, wm, wn, nk;
  bool active;                  // this wave's pair range holds rows of the tile
  f32x16 acc[NMAT][2][2];

  __device__ __forceinline__ Raw load(int kb) const {
    Raw R;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      R.a[i] = *reinterpret_cast<const uint4*>(arow[i] + (size_t)kb * kBK);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      R.w[m] = wcol[m][(size_t)kb * wstep];
      R.sm[m] = smcol[m][(size_t)kb * smstep];
    }
    return R;
  }

  __device__ __forceinline__ void stage(const Raw& R, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint4*>(&sA[buf][lr + 128 * i][8 * seg]) = R.a[i];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
      *reinterpret_cast<bf16x8*>(&sB[2 * m + buf][lr][8 * seg]) =
          dequant_word<BITS>(R.w[m], seg, R.sm[m]);
  }

  __device__ __forceinline__ void mma(int buf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kk = ks * 16 + (lane / 32) * 8;
      bf16x8 a[2], b[NMAT][2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&sA[buf][wm + 32 * i + lane % 32][kk]);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          b[m][j] =
              *reinterpret_cast<const bf16x8*>(&sB[2 * m + buf][wn + 32 * j + lane % 32][kk]);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[m][j], acc[m][i][j],
                                                                   0, 0, 0);
    }
  }

  // One K-step: the matrix-core work of step kb (skipped past the last step and by waves
  // with no rows), then step kb+1 dequantized into the other buffer and step kb+3
  // requested into the freed ring slot. Staging and loads run unconditionally (past the
  // end they repeat the last block into a buffer no matrix-core step reads), so the loop
  // has no data-dependent branches around its memory operations and the wait counts stay
  // exact across iterations.
  __device__ __forceinline__ Raw step(int kb, const Raw next) {
    if (active && kb < nk) mma(kb & 1);
    stage(next, (kb + 1) & 1);
    const Raw refill = load(min(kb + 3, nk - 1));
    __syncthreads();
    return refill;
  }

  __device__ __forceinline__ void run() {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[m][i][j][q] = 0.0f;
    Raw r0 = load(0);
    Raw r1 = load(min(1, nk - 1));
    stage(r0, 0);
    r0 = load(min(2, nk - 1));
    __syncthreads();
    for (int kb = 0; kb < nk; kb += 2) {
      r1 = step(kb, r1);
      r0 = step(kb + 1, r0);
    }
  }

  // Set up the LDS views and the wave's tile position.
  __device__ __forceinline__ void init(char* smem, int rows, int nk_) {
    const int tid = threadIdx.x, wave = tid / kWave;
    sA = reinterpret_cast<ATile*>(smem);
    sB = reinterpret_cast<BTile*>(smem + 2 * sizeof(ATile));
    lr = tid / 4;
    seg = tid % 4;
    lane = tid & (kWave - 1);
    wm = (wave / 2) * 64;
    wn = (wave % 2) * 64;
    nk = nk_;
    active = wm < rows;
  }
};

// ---------------------------------------------------------------- gate/up GEMM

template <int BITS>
__global__ __launch_bounds__(kGemmThreads) void k_pf_gateup(
    const uint32_t* __restrict__ gcodes, const uint32_t* __restrict__ gsm,
    const uint32_t* __restrict__ ucodes, const uint32_t* __restrict__ usm, int d, int f,
    const int4* __restrict__ tiles, const int* __restrict__ ntiles,
    const uint16_t* __restrict__ x, const int* __restrict__ tok_of_g, uint16_t* __restrict__ h,
    int) {
  typedef GemmCore<BITS, 2> Core;
  __shared__ __attribute__((aligned(16))) char smem[Core::kLdsBytes];
  const int ntn = (f + kBN - 1) / kBN;
  const int item = xcd_item(load_uniform(ntiles) * ntn);
  if (item < 0) return;
  const int mt = item / ntn, nt = item % ntn;
  const int4 tile = load_uniform(tiles + mt);
  const int e = tile.x, g0 = tile.y, rows = tile.z;
  const int nbd = d / kBK;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;

  Core c;
  c.init(smem, rows, nbd);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int tok = tok_of_g[g0 + min(c.lr + 128 * i, rows - 1)];  // padded rows repeat
    c.arow[i] = x + (size_t)tok * d + 8 * c.seg;                   // a valid token
  }
  const int wrow = min(nt * kBN + c.lr, f - 1);  // rows past f load row f-1, never stored
  const size_t blk0 = (size_t)e * nbd * f + wrow;
  c.wcol[0] = gcodes + blk0 * BITS + code_word_index<BITS>(c.seg);
  c.wcol[1] = ucodes + blk0 * BITS + code_word_index<BITS>(c.seg);
  c.smcol[0] = gsm + blk0;
  c.smcol[1] = usm + blk0;
  c.wstep = (size_t)f * BITS;
  c.smstep = (size_t)f;
  c.run();

  // epilogue: h = bf16(silu(g) * u), staged per wave in LDS (64 x 64 bf16 = 8 KB per wave)
  // for 16-byte global stores
  if (!c.active) return;
  __bf16* st = reinterpret_cast<__bf16*>(smem) + wave * (64 * 64);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rr = 32 * i + (q / 4) * 8 + (lane / 32) * 4 + (q % 4);
        const int cc = 32 * j + lane % 32;
        st[rr * 64 + cc] = (__bf16)silu_mul(c.acc[0][i][j][q], c.acc[1][i][j][q]);
      }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int ch = lane + kWave * q;  // 512 chunks of 8 bf16
    const int rr = ch / 8, cc = (ch % 8) * 8;
    const int col = nt * kBN + c.wn + cc;
    if (c.wm + rr < rows && col < f) {
      const uint4 v = *reinterpret_cast<const uint4*>(&st[rr * 64 + cc]);
      *reinterpret_cast<uint4*>(h + (size_t)(g0 + c.wm + rr) * f + col) = v;
    }
  }
}

// ---------------------------------------------------------------- down GEMM

template <int BITS>
__global__ __launch_bounds__(kGemmThreads) void k_pf_down(
    const uint32_t* __restrict__ dcodes, const uint32_t* __restrict__ dsm, int d, int f,
    const int4* __restrict__ tiles, const int* __restrict__ ntiles,
    const uint16_t* __restrict__ h, float* __restrict__ y, int) {
  typedef GemmCore<BITS, 1> Core;
  __shared__ __attribute__((aligned(16))) char smem[Core::kLdsBytes];
  const int ntn = (d + kBN - 1) / kBN;
  const int item = xcd_item(load_uniform(ntiles) * ntn);
  if (item < 0) return;
  const int mt = item / ntn, nt = item % ntn;
  const int4 tile = load_uniform(tiles + mt);
  const int e = tile.x, g0 = tile.y, rows = tile.z;
  const int nbf = f / kBK;
  const int lane = threadIdx.x & (kWave - 1);

  Core c;
  c.init(smem, rows, nbf);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    c.arow[i] = h + (size_t)(g0 + min(c.lr + 128 * i, rows - 1)) * f + 8 * c.seg;
  const int wrow = min(nt * kBN + c.lr, d - 1);  // rows past d load row d-1, never stored
  const size_t blk0 = (size_t)e * nbf * d + wrow;
  c.wcol[0] = dcodes + blk0 * BITS + code_word_index<BITS>(c.seg);
  c.smcol[0] = dsm + blk0;
  c.wstep = (size_t)d * BITS;
  c.smstep = (size_t)d;
  c.run();
  if (!c.active) return;

  // y in grouped order: lanes 0..31 of a row write 32 consecutive floats
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rr = c.wm + 32 * i + (q / 4) * 8 + (lane / 32) * 4 + (q % 4);
        const int col = nt * kBN + c.wn + 32 * j + lane % 32;
        if (rr < rows && col < d) y[(size_t)(g0 + rr) * d + col] = c.acc[0][i][j][q];
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
    hipLaunchKernelGGL(k_pf_gateup<BITS>, dim3(gu_items), dim3(kGemmThreads), 0, a.stream,
                       L.gate.codes, reinterpret_cast<const uint32_t*>(L.gate.scale_min),
                       L.up.codes, reinterpret_cast<const uint32_t*>(L.up.scale_min), d, f, tiles,
                       ntiles, a.x, tok_of_g, h, gu_items);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (a.stages & MOE_PREFILL_DOWN) {
    const int dn_items = ((max_mt * ((d + kBN - 1) / kBN) + 7) / 8) * 8;
    hipLaunchKernelGGL(k_pf_down<BITS>, dim3(dn_items), dim3(kGemmThreads), 0, a.stream,
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

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
//                 activations and the packed gate and up codes of each K-step arrive in
//                 LDS by direct loads; each wave dequantizes its own matrix-core B operands
//                 (bf16 of fp32 scale*q + min) in registers and runs
//                 v_mfma_f32_32x32x16_bf16 with fp32 accumulators; the epilogue applies
//                 SwiGLU and writes h = bf16(silu(g) * u) in grouped pair order.
//   k_pf_down     the same GEMM over (M-tile, 256 output columns) with h as the A operand
//                 and the down codes as B, fp32 outputs y in grouped order.
//   k_pf_combine  residual[t] += sum_j w[t][j] * y[pair (t, j)], slot order, binary64 sum.
#include <algorithm>

#include "qmoe_internal.h"

namespace qmoe {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kBM = kPrefillBM;  // pairs per M-tile
constexpr int kBK = 32;          // one quantization block of the reduction axis

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

// silu(g) * u in fp32 with the hardware exponential and reciprocal (each within about an
// ulp; h is rounded to bf16 next)
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ---------------------------------------------------------------- grouped GEMM core
//
// One workgroup of 4 waves (one per SIMD) computes kBM (256) pairs x 32 weight rows per B
// operand set of each wave; a wave has two sets (gate/up: the gate and the up rows of the
// same 32 rows, 128 rows a workgroup; down: two groups of 32 output columns, 256 a
// workgroup). Each wave dequantizes its own matrix-core B operands straight into
// registers: lane l needs 8 consecutive reduction-axis codes of weight row l%32 (one 4-bit
// code word, or half a 2-bit word), so no weight passes through LDS as bf16 and none is
// dequantized twice within the tile. Each K-step's operands (the A tile of 256 pairs x 32
// bf16 and each wave's packed code and scale/min words) arrive by direct loads into LDS
// (global_load_lds, no register trip) in a ring of kRbStages stages, each stage its own
// LDS variable so that the compiler can tell the stage being filled from the one being
// read, and registers carry nothing from one loop iteration to the next (which would make
// its wait counts drain the ring). In the A tile, row m's 16-byte segment s sits at
// position s ^ (m/4 % 4), so that the 16 lanes of each quarter-wave read 16 different bank
// groups. The 8 x 2 accumulators of 32x32 of a wave live in the accumulation registers
// (256 a lane). While a K-step's matrix-core ops run, the wave reads and dequantizes the
// next step's operands.
//
// (Measured on MI355X at the 8192-token chunk: the waves spend about half their time
// waiting for the direct loads of the operands; a ring of six stages is 5% faster than
// four. Weights dequantized once per chunk into bf16 for the experts with several M-tiles
// made the gate/up GEMM no faster, and the dequantization pass itself cost 158 us.)
constexpr int kRbThreads = 256;
constexpr int kRbStages = 6;                       // K-steps in flight
constexpr int kRbSlots = kBM * kBK * 2 / 16;       // 16-byte slots of one A tile (1024)
constexpr int kRbDma = kRbSlots / kRbThreads;      // A direct loads a thread a K-step (4)

struct RbStage {
  uint4 a[kRbSlots];          // A tile
  uint4 codes[4][kWave];      // per wave: [set][row] 16 bytes (2-bit: 16 row pairs a set)
  uint32_t sm[4][kWave];      // per wave: [set][row] scale/min word
};

__device__ __forceinline__ int swz(int row, int seg) { return seg ^ ((row >> 2) & 3); }

template <int BITS>
struct RbCore {
  typedef __attribute__((address_space(3))) void* lptr_t;
  typedef const __attribute__((address_space(1))) void* gptr_t;
  static constexpr int kNSet = 2;
  static constexpr int kOps = kRbDma + 2;  // direct loads a thread a K-step

  RbStage* st[kRbStages];
  const char* arow[kRbDma];  // this thread's A segments at K-step 0
  const char* bcode;         // this lane's code bytes at K-step 0
  const char* bsm;           // this lane's scale/min word at K-step 0
  size_t bstep, smstep;      // bytes per K-step of the codes and of the scale/min words
  int lane, wave, nk;
  f32x16 acc[kNSet][8];

  // A tile and this wave's weight words of K-step kb (past the end: the last step again,
  // into a stage no matrix-core step reads).
  template <int S>
  __device__ __forceinline__ void dma(int kb) const {
    const size_t k = (size_t)min(kb, nk - 1);
    const size_t aoff = k * (kBK * 2);
#pragma unroll
    for (int i = 0; i < kRbDma; ++i)
      __builtin_amdgcn_global_load_lds((gptr_t)(arow[i] + aoff),
                                       (lptr_t)(st[S]->a + kRbThreads * i + kWave * wave), 16, 0,
                                       0);
    __builtin_amdgcn_global_load_lds((gptr_t)(bcode + k * bstep), (lptr_t)(st[S]->codes[wave]),
                                     16, 0, 0);
    __builtin_amdgcn_global_load_lds((gptr_t)(bsm + k * smstep), (lptr_t)(st[S]->sm[wave]), 4, 0,
                                     0);
  }

  // Operands of one K-step in registers: the A fragments of both 16-wide halves and the
  // dequantized B operands of both sets.
  struct Ops {
    bf16x8 a[2][8];
    bf16x8 b[2][kNSet];
  };

  // Read K-step operands from stage S; keep = 0 (steps past the last) zeroes the scale and
  // min, hence the B operands.
  template <int S>
  __device__ __forceinline__ Ops read_ops(uint32_t keep) const {
    Ops o;
    const RbStage& sg = *st[S];
    const int r = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int seg = 2 * ks + hi;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int mrow = 32 * i + r;
        const uint4 av = sg.a[4 * mrow + swz(mrow, seg)];
        __builtin_memcpy(&o.a[ks][i], &av, 16);
      }
    }
#pragma unroll
    for (int q = 0; q < kNSet; ++q) {
      const uint32_t smw = sg.sm[wave][32 * q + r] & keep;
      uint32_t w0, w1;  // the code words of the two halves (ks = 0, 1)
      if (BITS == 4) {
        const uint4 c = sg.codes[wave][32 * q + r];
        w0 = hi ? c.y : c.x;
        w1 = hi ? c.w : c.z;
      } else {
        // set q's rows 2i, 2i+1 in slot 16q + i: words (row 2i: 0, 1; row 2i+1: 2, 3)
        const uint4 c = sg.codes[wave][16 * q + r / 2];
        w0 = (r & 1) ? c.z : c.x;
        w1 = (r & 1) ? c.w : c.y;
      }
      o.b[0][q] = dequant_word<BITS>(w0, hi, smw);
      o.b[1][q] = dequant_word<BITS>(w1, 2 + hi, smw);
    }
    return o;
  }

  __device__ __forceinline__ void mma(const Ops& o) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int q = 0; q < kNSet; ++q)
          acc[q][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.a[ks][i], o.b[ks][q], acc[q][i],
                                                              0, 0, 0);
  }

  // One K-step kb (its operands `cur` already in registers, read from stage S): wait for
  // step kb + 1's operands and publish them (this wave's reads of step kb have completed,
  // so after the barrier no wave reads stage S any more), request step kb + kRbStages into
  // stage S, then step kb's matrix-core work with the reads of step kb + 1 placed ahead of
  // it and their dequantization interleaved with the matrix-core ops, which run while it
  // executes. Steps past the last one multiply zero B operands (an AND with a uniform
  // mask, not a branch), so that each step is one basic block in which that order holds.
  template <int S>
  __device__ __forceinline__ Ops step(int kb, const Ops& cur) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
    wait_vmcnt<(kRbStages - 2) * kOps>();
    barrier_after_lds_dma();
    dma<S>(kb + kRbStages);
    __builtin_amdgcn_sched_barrier(0);
    Ops next = read_ops<(S + 1) % kRbStages>(kb + 1 < nk ? 0xffffffffu : 0u);
    mma(cur);
    // the next step's operands are complete within this step
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int q = 0; q < kNSet; ++q) {
        uint4 v;
        __builtin_memcpy(&v, &next.b[ks][q], 16);
        asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
        __builtin_memcpy(&next.b[ks][q], &v, 16);
      }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * 8 + 2 * kNSet, 0);  // LDS reads
#pragma unroll
    for (int i = 0; i < 16 * kNSet; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix-core op
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU instructions
    }
    __builtin_amdgcn_sched_barrier(0);
    return next;
  }

  __device__ __forceinline__ void run() {
#pragma unroll
    for (int q = 0; q < kNSet; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[q][i][e] = 0.0f;
    dma<0>(0);
    dma<1>(1);
    dma<2>(2);
    dma<3>(3);
    dma<4>(4);
    dma<5>(5);
    wait_vmcnt<(kRbStages - 1) * kOps>();
    barrier_after_lds_dma();
    Ops o0 = read_ops<0>(0xffffffffu);
    static_assert(kRbStages == 6, "the loop below is unrolled over the ring");
    for (int kb = 0; kb < nk; kb += kRbStages) {
      const Ops o1 = step<0>(kb, o0);
      const Ops o2 = step<1>(kb + 1, o1);
      const Ops o3 = step<2>(kb + 2, o2);
      const Ops o4 = step<3>(kb + 3, o3);
      const Ops o5 = step<4>(kb + 4, o4);
      o0 = step<5>(kb + 5, o5);
    }
    wait_vmcnt<0>();  // the direct loads past the last step have landed
  }

  __device__ __forceinline__ void init(RbStage* stages, int nk_) {
#pragma unroll
    for (int i = 0; i < kRbStages; ++i) st[i] = stages + i;
    lane = threadIdx.x & (kWave - 1);
    wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    nk = nk_;
  }

  // A row m (0..255) of this thread's slot set i, and the byte offset of its segment
  __device__ __forceinline__ int arow_index(int i) const { return ((int)threadIdx.x >> 2) + 64 * i; }
  __device__ __forceinline__ int aseg_bytes() const {
    const int t = threadIdx.x;
    return 16 * swz(t >> 2, t & 3);
  }

  // The weight row and set whose codes lane l brings in: 4-bit, set l/32 row l%32; 2-bit,
  // set (l%32)/16, rows 2(l%16) and 2(l%16)+1 (16 bytes; lanes 32..63 repeat 0..31). The
  // scale/min word: set l/32, row l%32. row_of(q, r) is the matrix row of set q's row r;
  // past the matrix, a valid row (never stored) is loaded.
  template <class RowOf>
  __device__ __forceinline__ void set_weights(const uint32_t* codes0, const uint32_t* codes1,
                                              const uint32_t* sm0, const uint32_t* sm1,
                                              size_t eoff, int NR, RowOf row_of) {
    const int cq = BITS == 4 ? lane >> 5 : (lane & 31) >> 4;
    const int cr = BITS == 4 ? (lane & 31) : 2 * (lane & 15);
    const int crow = min(row_of(cq, cr), BITS == 4 ? NR - 1 : NR - 2);
    bcode = reinterpret_cast<const char*>((cq ? codes1 : codes0) + (eoff + crow) * BITS);
    bsm = reinterpret_cast<const char*>((lane >> 5 ? sm1 : sm0) + eoff +
                                        min(row_of(lane >> 5, lane & 31), NR - 1));
    bstep = (size_t)NR * BITS * 4;
    smstep = (size_t)NR * 4;
  }
};

// ---------------------------------------------------------------- gate/up GEMM

// h = bf16(silu(g) * u). Lane l holds column 32*wave + l%32 of rows 32i + 8(q/4) +
// 4(l/32) + q%4; the wave's 256 x 32 block goes through LDS (the ring is free by then) so
// that rows leave as 16-byte stores.
template <int BITS>
__global__ __launch_bounds__(kRbThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_pf_gateup(
    const uint32_t* __restrict__ gcodes, const uint32_t* __restrict__ gsm,
    const uint32_t* __restrict__ ucodes, const uint32_t* __restrict__ usm, int d, int f,
    const int4* __restrict__ tiles, const int* __restrict__ ntiles,
    const uint16_t* __restrict__ x, const int* __restrict__ tok_of_g, uint16_t* __restrict__ h) {
  __shared__ RbStage stages[kRbStages];
  constexpr int kN = 4 * 32;  // weight rows a workgroup
  const int ntn = (f + kN - 1) / kN;
  const int item = xcd_item(load_uniform(ntiles) * ntn);
  if (item < 0) return;
  const int mt = item / ntn, nt = item % ntn;
  const int4 tile = load_uniform(tiles + mt);
  const int e = tile.x, g0 = tile.y, rows = tile.z;
  const int nbd = d / kBK;
  RbCore<BITS> c;
  c.init(stages, nbd);
#pragma unroll
  for (int i = 0; i < kRbDma; ++i) {
    const int tok = tok_of_g[g0 + min(c.arow_index(i), rows - 1)];  // padded rows: a valid row
    c.arow[i] = reinterpret_cast<const char*>(x + (size_t)tok * d) + c.aseg_bytes();
  }
  const int n0 = nt * kN + 32 * c.wave;  // this wave's rows n0 + 0..31: gate (set 0), up (set 1)
  c.set_weights(gcodes, ucodes, gsm, usm, (size_t)e * nbd * f, f,
                [&](int, int r) { return n0 + r; });
  c.run();

  __syncthreads();  // every wave is done with the ring before it is reused
  uint16_t* stg = reinterpret_cast<uint16_t*>(stages) + c.wave * (kBM * 32);
  const int lane = c.lane;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int rr = 32 * i + (q / 4) * 8 + (lane / 32) * 4 + (q % 4);
      const __bf16 v = (__bf16)silu_mul(c.acc[0][i][q], c.acc[1][i][q]);
      __builtin_memcpy(&stg[rr * 32 + (lane & 31)], &v, 2);
    }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // 256 rows x 4 chunks of 8 bf16: lane l takes chunk l%4 of rows l/4 + 16p
  const int col0 = n0 + 8 * (lane & 3);
  if (col0 < f) {
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int rr = (lane >> 2) + 16 * p;
      if (rr < rows)
        *reinterpret_cast<uint4*>(h + (size_t)(g0 + rr) * f + col0) =
            *reinterpret_cast<const uint4*>(&stg[rr * 32 + 8 * (lane & 3)]);
    }
  }
}

// ---------------------------------------------------------------- down GEMM

// Lanes l and l+32 hold column 32q + l%32 of rows 32i + 8(e/4) + 4(l/32) + e%4; 32-row
// groups wholly inside the tile store without a per-row test.
template <int BITS>
__global__ __launch_bounds__(kRbThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_pf_down(
    const uint32_t* __restrict__ dcodes, const uint32_t* __restrict__ dsm, int d, int f,
    const int4* __restrict__ tiles, const int* __restrict__ ntiles,
    const uint16_t* __restrict__ h, float* __restrict__ y) {
  __shared__ RbStage stages[kRbStages];
  constexpr int kN = 4 * 64;  // output columns a workgroup
  const int ntn = (d + kN - 1) / kN;
  const int item = xcd_item(load_uniform(ntiles) * ntn);
  if (item < 0) return;
  const int mt = item / ntn, nt = item % ntn;
  const int4 tile = load_uniform(tiles + mt);
  const int e = tile.x, g0 = tile.y, rows = tile.z;
  const int nbf = f / kBK;
  RbCore<BITS> c;
  c.init(stages, nbf);
#pragma unroll
  for (int i = 0; i < kRbDma; ++i)
    c.arow[i] = reinterpret_cast<const char*>(h + (size_t)(g0 + min(c.arow_index(i), rows - 1)) * f) +
                c.aseg_bytes();
  const int c0 = nt * kN + 64 * c.wave;  // set q: output columns c0 + 32q + 0..31
  c.set_weights(dcodes, dcodes, dsm, dsm, (size_t)e * nbf * d, d,
                [&](int q, int r) { return c0 + 32 * q + r; });
  c.run();
  const int lane = c.lane;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int col = c0 + 32 * q + (lane & 31);
    if (col >= d) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float* yb = y + (size_t)(g0 + 32 * i + (lane / 32) * 4) * d + col;
      if (32 * i + 32 <= rows) {
#pragma unroll
        for (int e2 = 0; e2 < 16; ++e2) yb[(size_t)((e2 / 4) * 8 + (e2 % 4)) * d] = c.acc[q][i][e2];
      } else if (32 * i < rows) {
#pragma unroll
        for (int e2 = 0; e2 < 16; ++e2) {
          const int rr = 32 * i + (e2 / 4) * 8 + (lane / 32) * 4 + (e2 % 4);
          if (rr < rows) yb[(size_t)((e2 / 4) * 8 + (e2 % 4)) * d] = c.acc[q][i][e2];
        }
      }
    }
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
    const int gu_items = ((max_mt * ((f + 127) / 128) + 7) / 8) * 8;
    hipLaunchKernelGGL(k_pf_gateup<BITS>, dim3(gu_items), dim3(kRbThreads), 0, a.stream,
                       L.gate.codes, reinterpret_cast<const uint32_t*>(L.gate.scale_min),
                       L.up.codes, reinterpret_cast<const uint32_t*>(L.up.scale_min), d, f, tiles,
                       ntiles, a.x, tok_of_g, h);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (a.stages & MOE_PREFILL_DOWN) {
    const int dn_items = ((max_mt * ((d + 255) / 256) + 7) / 8) * 8;
    hipLaunchKernelGGL(k_pf_down<BITS>, dim3(dn_items), dim3(kRbThreads), 0, a.stream,
                       L.down.codes, reinterpret_cast<const uint32_t*>(L.down.scale_min), d, f,
                       tiles, ntiles, h, y);
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

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
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

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
    // One thread per expert. The M-tiles are listed longest first: every full tile (in
    // expert order), then the last, partly filled tiles grouped by the row groups they
    // compute (8, 4, 2, 1), each group in expert order.
    __shared__ int s_wsum[16];
    __shared__ int s_total;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int e = tid;
    const int beg = e < E ? offsets[e] : 0;
    const int m = e < E ? offsets[e + 1] - beg : 0;
    const int nfull = m / kBM, rem = m - nfull * kBM;
    const int cls = rem == 0 ? -1 : rem > 128 ? 0 : rem > 64 ? 1 : rem > 32 ? 2 : 3;
    int start = 0;  // tiles of the groups listed so far
    // position of this expert's first tile of a group of v tiles an expert
    auto place = [&](int v) {
      int incl = v;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (lane == kWave - 1) s_wsum[wave] = incl;
      __syncthreads();
      int base = incl - v;
      for (int w = 0; w < wave; ++w) base += s_wsum[w];
      if (tid == 1023) s_total = base + v;
      __syncthreads();
      const int pos = start + base;
      start += s_total;
      __syncthreads();  // s_wsum and s_total are rewritten by the next group
      return pos;
    };
    const int fb = place(nfull);
    for (int i = 0; i < nfull; ++i) tiles[fb + i] = make_int4(e, beg + i * kBM, kBM, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int pb = place(cls == c ? 1 : 0);
      if (cls == c) tiles[pb] = make_int4(e, beg + nfull * kBM, rem, 0);
    }
    if (tid == 0) *ntiles = start;
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
// is exact in fp32, so the fma rounds once, like the separate multiply and add). The codes
// are spread one a byte and converted by the byte-to-float conversions (the empty asm keeps
// the compiler from folding the byte masks into a shift and mask per code), and the bf16
// pairs are rounded two at a time.
template <int BITS>
__device__ __forceinline__ bf16x8 dequant_word(uint32_t w, int seg, uint32_t sm) {
  const float s = half_bits_to_float(sm & 0xffffu), mn = half_bits_to_float(sm >> 16);
  float q[8];
  if (BITS == 4) {
    // byte j of lo holds code 2j, byte j of hi code 2j+1
    uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      q[2 * j] = (float)((lo >> (8 * j)) & 0xffu);
      q[2 * j + 1] = (float)((hi >> (8 * j)) & 0xffu);
    }
  } else {
    // codes 0..7 of the half word at bits 2i; byte 0 of t[j] holds code j, byte 1 code j+4
    const uint32_t v = w >> (16 * (seg & 1));
    uint32_t t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) t[j] = (v >> (2 * j)) & 0x0303u;
    asm("" : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      q[j] = (float)(t[j] & 0xffu);
      q[j + 4] = (float)((t[j] >> 8) & 0xffu);
    }
  }
  bf16x8 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x2 v = {__builtin_fmaf(s, q[2 * j], mn), __builtin_fmaf(s, q[2 * j + 1], mn)};
    const bf16x2 r = __builtin_convertvector(v, bf16x2);
    out[2 * j] = r[0];
    out[2 * j + 1] = r[1];
  }
  return out;
}

// XCD-aware placement. Workgroups are dealt to the 8 XCDs round robin by workgroup id. M-tile
// mt goes to XCD mt % 8, whose workgroups take its ntn column tiles one after another (they
// share the A rows in that XCD's L2) and the XCD's M-tiles in list order, longest first, so
// that the XCDs get equal shares of the long and the short tiles and each ends on short
// ones. The grid is sized for the largest possible tile count; returns false for idle
// workgroups.
__device__ __forceinline__ bool xcd_tile(int ntiles, int ntn, int& mt, int& nt) {
  const int slot = (int)(blockIdx.x / 8);
  mt = (int)(blockIdx.x % 8) + 8 * (slot / ntn);
  nt = slot % ntn;
  return mt < ntiles;
}

// Workgroups of a launch over at most max_mt M-tiles of ntn column tiles each
inline int xcd_grid(int max_mt, int ntn) { return ((max_mt + 7) / 8) * 8 * ntn; }

// silu(g) * u in fp32 with the hardware exponential and reciprocal (each within about an
// ulp; h is rounded to bf16 next)
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ---------------------------------------------------------------- grouped GEMM core
//
// One workgroup of 4 waves (one per SIMD) computes up to kBM (256) pairs x 32 weight rows
// per B operand set of each wave; a wave has two sets (gate/up: the gate and the up rows of
// the same 32 rows, 128 rows a workgroup; down: two groups of 32 output columns, 256 a
// workgroup). The pairs are taken in NI groups of 32 (NI = 1, 2, 4 or 8, the smallest that
// holds the M-tile's rows), so that the last, partly filled M-tile of an expert issues
// matrix-core ops and A loads only for the row groups it has. Each wave dequantizes its own
// matrix-core B operands straight into registers: lane l needs 8 consecutive
// reduction-axis codes of weight row l%32 (one 4-bit code word, or half a 2-bit word), so
// no weight passes through LDS as bf16 and none is dequantized twice within the tile.
// Each K-step's operands (the A tile of 32*NI pairs x 32 bf16 and each wave's packed code
// and scale/min words) arrive by direct loads into LDS (global_load_lds, no register trip)
// in a ring of kRbStages slots, each slot its own LDS variable so that the compiler can
// tell the slot being filled from the one being read, and no register written by a global
// load is carried from one loop iteration to the next (which would make its wait counts
// drain the ring). The weight words are read from LDS two steps ahead, so that a step's
// dequantization needs no memory access; the A fragments one step ahead. In the A tile,
// row m's 16-byte segment s sits at position s ^ (m/4 % 4), so that the 16 lanes of each
// quarter-wave read 16 different bank groups. The NI x 2 accumulators of 32x32 of a wave
// live in the accumulation registers (32*NI a lane). A step's LDS reads and dequantization
// are interleaved with its matrix-core ops, one read after each op, so that the reads of
// the four waves do not hold up the issue of their matrix-core ops.
//
// (Measured on MI355X at the 8192-token chunk, gate/up: with every row group computed the
// ragged M-tiles made 31% of the matrix-core ops; the kernel runs near 1.9 GHz, limited by
// power; leaving out the direct loads, the dequantization or the LDS reads each saves
// 100-190 us, and waiting for older data does not, so the loads cost issue slots and power,
// not latency. Weights dequantized once per chunk into bf16 for the experts with several
// M-tiles made the gate/up GEMM no faster, and the dequantization pass itself cost 158 us.
// Tiles of 128 pairs, two workgroups a CU and so two waves a SIMD, measured the same:
// twice the dequantization per flop pays for the latency the second wave hides.)
constexpr int kRbThreads = 256;
constexpr int kRbStages = 4;                       // K-steps in flight
constexpr int kRbSlots = kBM * kBK * 2 / 16;       // 16-byte slots of a full A tile (1024)

struct RbStage {
  uint4 a[kRbSlots];          // A tile
  uint4 codes[4][kWave];      // per wave: [set][row] 16 bytes (2-bit: 16 row pairs a set)
  uint32_t sm[4][kWave];      // per wave: [set][row] scale/min word
};

__device__ __forceinline__ int swz(int row, int seg) { return seg ^ ((row >> 2) & 3); }

// Row groups of 32 computed for an M-tile of `rows` pairs
__device__ __forceinline__ int row_groups(int rows) {
  return rows <= 32 ? 1 : rows <= 64 ? 2 : rows <= 128 ? 4 : 8;
}

template <int BITS, int NI>
struct RbCore {
  typedef __attribute__((address_space(3))) void* lptr_t;
  typedef const __attribute__((address_space(1))) void* gptr_t;
  static constexpr int kNSet = 2;
  // A direct loads a thread a K-step: each covers 64 rows (4 threads a row)
  static constexpr int kDmaA = NI >= 2 ? NI / 2 : 1;
  static constexpr int kOps = kDmaA + 2;  // direct loads a thread a K-step

  RbStage* st[kRbStages];
  const char* arow[kDmaA];   // this thread's A segments at K-step 0
  const char* bcode;         // this lane's code bytes at K-step 0
  const char* bsm;           // this lane's scale/min word at K-step 0
  size_t bstep, smstep;      // bytes per K-step of the codes and of the scale/min words
  int lane, wave, nk;
  f32x16 acc[kNSet][NI];

  // Direct loads of K-step j (past the end: the last step again, into a slot that no
  // matrix-core step reads): the A tile into slot S, and this wave's code and scale/min
  // words into slot S of their own ring (the fields of a slot are filled at different
  // steps: A(j) and the words of j + 1 are requested together).
  template <int S>
  __device__ __forceinline__ void dma_a(int kb) const {
    const size_t aoff = (size_t)min(kb, nk - 1) * (kBK * 2);
#pragma unroll
    for (int i = 0; i < kDmaA; ++i)
      __builtin_amdgcn_global_load_lds((gptr_t)(arow[i] + aoff),
                                       (lptr_t)(st[S]->a + kRbThreads * i + kWave * wave), 16, 0,
                                       0);
  }
  template <int S>
  __device__ __forceinline__ void dma_w(int kb) const {
    const size_t k = (size_t)min(kb, nk - 1);
    __builtin_amdgcn_global_load_lds((gptr_t)(bcode + k * bstep), (lptr_t)(st[S]->codes[wave]),
                                     16, 0, 0);
    __builtin_amdgcn_global_load_lds((gptr_t)(bsm + k * smstep), (lptr_t)(st[S]->sm[wave]), 4, 0,
                                     0);
  }

  // Operands of one K-step in registers: the A fragments of both 16-wide halves and the
  // dequantized B operands of both sets.
  struct Ops {
    bf16x8 a[2][NI];
    bf16x8 b[2][kNSet];
  };
  // This lane's packed weight words of one K-step: per set, the scale/min word and the
  // code words (4-bit: the row's whole 16-byte slot, read without bank conflicts, of which
  // the lane's half uses words hi and 2 + hi; 2-bit: the two words of its row).
  struct Raw {
    uint32_t w[kNSet][BITS == 4 ? 4 : 2];
    uint32_t sm[kNSet];
  };

  template <int S>
  __device__ __forceinline__ void read_a(Ops& o) const {
    const RbStage& sg = *st[S];
    const int r = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int seg = 2 * ks + hi;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int mrow = 32 * i + r;
        const uint4 av = sg.a[4 * mrow + swz(mrow, seg)];
        __builtin_memcpy(&o.a[ks][i], &av, 16);
      }
    }
  }

  template <int S>
  __device__ __forceinline__ Raw read_w() const {
    Raw o;
    const RbStage& sg = *st[S];
    const int r = lane & 31;
#pragma unroll
    for (int q = 0; q < kNSet; ++q) {
      o.sm[q] = sg.sm[wave][32 * q + r];
      if constexpr (BITS == 4) {
        // row r of set q in slot 32q + r
        const uint4 c = sg.codes[wave][32 * q + r];
        o.w[q][0] = c.x;
        o.w[q][1] = c.y;
        o.w[q][2] = c.z;
        o.w[q][3] = c.w;
      } else {
        // rows 2i, 2i+1 of set q in slot 16q + i: words (row 2i: 0, 1; row 2i+1: 2, 3)
        const uint32_t* p =
            reinterpret_cast<const uint32_t*>(sg.codes[wave]) + 4 * (16 * q + r / 2) + 2 * (r & 1);
        o.w[q][0] = p[0];
        o.w[q][1] = p[1];
      }
    }
    return o;
  }

  // keep = 0 (steps past the last) zeroes the scale and min, hence the B operands
  __device__ __forceinline__ void dequant(Ops& o, const Raw& w, uint32_t keep) const {
    const int hi = lane >> 5;
#pragma unroll
    for (int q = 0; q < kNSet; ++q) {
      const uint32_t smw = w.sm[q] & keep;
      uint32_t w0, w1;  // the code words of the two halves (ks = 0, 1)
      if constexpr (BITS == 4) {
        w0 = hi ? w.w[q][1] : w.w[q][0];
        w1 = hi ? w.w[q][3] : w.w[q][2];
      } else {
        w0 = w.w[q][0];
        w1 = w.w[q][1];
      }
      o.b[0][q] = dequant_word<BITS>(w0, hi, smw);
      o.b[1][q] = dequant_word<BITS>(w1, 2 + hi, smw);
    }
  }

  __device__ __forceinline__ void mma(const Ops& o) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int q = 0; q < kNSet; ++q)
          acc[q][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.a[ks][i], o.b[ks][q], acc[q][i],
                                                              0, 0, 0);
  }

  // One K-step kb, S = kb % kRbStages. On entry: step kb's operands `cur` and step kb + 1's
  // weight words `w1` are in registers. Wait for the A tile of kb + 1 and the words of
  // kb + 2 and publish them (this wave's reads of step kb - 1 have completed, so after the
  // barrier no wave reads A slot S or word slot S + 1 any more), request the A tile of
  // kb + 4 into A slot S and the words of kb + 5 into word slot S + 1, then run step kb's
  // matrix-core ops with the reads of the A tile of kb + 1 and of the words of kb + 2, and
  // the dequantization of w1 (no memory access), placed between them. Steps past the last
  // multiply zero B operands (an AND with a uniform mask, not a branch), so that each step
  // is one basic block in which that order holds.
  template <int S>
  __device__ __forceinline__ Ops step(int kb, const Ops& cur, Raw& w1) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
    wait_vmcnt<(kRbStages - 2) * kOps>();
    barrier_after_lds_dma();
    dma_a<S>(kb + kRbStages);
    dma_w<(S + 1) % kRbStages>(kb + kRbStages + 1);
    __builtin_amdgcn_sched_barrier(0);
    Ops next;
    read_a<(S + 1) % kRbStages>(next);
    const Raw w2 = read_w<(S + 2) % kRbStages>();
    dequant(next, w1, kb + 1 < nk ? 0xffffffffu : 0u);
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
    // M matrix-core ops, R LDS reads (A fragments, 2 code words, the scale/min pair)
    constexpr int M = 2 * NI * kNSet, R = 2 * NI + 3;
    constexpr int kRd = (R + M - 1) / M, kValu = NI == 8 ? 3 : 24 / NI;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix-core op
      if (i * kRd + kRd <= R)
        __builtin_amdgcn_sched_group_barrier(0x100, kRd, 0);  // LDS reads
      else if (i * kRd < R)
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU instructions
    }
    __builtin_amdgcn_sched_barrier(0);
    w1 = w2;
    return next;
  }

  // Request order: words(0), then A(j) and words(j + 1) for j < kRbStages; words(4) once
  // words(0) and words(1) have been read (word slot 0 is then free). Every step then
  // requests A(kb + 4) and words(kb + 5) together, so at the top of step kb the batch that
  // holds A(kb + 1) and words(kb + 2) has kRbStages - 2 batches after it. A ring of four
  // steps divides the usual reduction lengths (64 and 24 steps at d = 2048, f = 768), so no
  // step runs past the last one there.
  __device__ __forceinline__ void run() {
#pragma unroll
    for (int q = 0; q < kNSet; ++q)
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[q][i][e] = 0.0f;
    static_assert(kRbStages == 4, "the request order and the loop below are written for four");
    dma_w<0>(0);
    dma_a<0>(0);
    dma_w<1>(1);
    dma_a<1>(1);
    dma_w<2>(2);
    dma_a<2>(2);
    dma_w<3>(3);
    dma_a<3>(3);
    // words(0), A(0), words(1) have landed: after them come A(1..3) and words(2..3)
    wait_vmcnt<3 * kDmaA + 2 * 2>();
    barrier_after_lds_dma();
    Ops o0;
    read_a<0>(o0);
    const Raw w0 = read_w<0>();
    Raw w1 = read_w<1>();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) before word slot 0 is refilled
    dma_w<0>(kRbStages);
    dequant(o0, w0, 0xffffffffu);
    for (int kb = 0; kb < nk; kb += kRbStages) {
      const Ops o1 = step<0>(kb, o0, w1);
      const Ops o2 = step<1>(kb + 1, o1, w1);
      const Ops o3 = step<2>(kb + 2, o2, w1);
      o0 = step<3>(kb + 3, o3, w1);
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

  // A row m of this thread's slot set i (rows 64i .. 64i + 63), and the byte offset of its
  // segment
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
// 4(l/32) + q%4; the wave's 32*NI x 32 block goes through LDS (the ring is free by then) so
// that rows leave as 16-byte stores.
template <int BITS, int NI>
__device__ __forceinline__ void pf_gateup_tile(
    RbStage* stages, const uint32_t* __restrict__ gcodes, const uint32_t* __restrict__ gsm,
    const uint32_t* __restrict__ ucodes, const uint32_t* __restrict__ usm, int d, int f, int e,
    int g0, int rows, int n0w, const uint16_t* __restrict__ x, const int* __restrict__ tok_of_g,
    uint16_t* __restrict__ h) {
  const int nbd = d / kBK;
  RbCore<BITS, NI> c;
  c.init(stages, nbd);
#pragma unroll
  for (int i = 0; i < RbCore<BITS, NI>::kDmaA; ++i) {
    const int tok = tok_of_g[g0 + min(c.arow_index(i), rows - 1)];  // padded rows: a valid row
    c.arow[i] = reinterpret_cast<const char*>(x + (size_t)tok * d) + c.aseg_bytes();
  }
  const int n0 = n0w + 32 * c.wave;  // this wave's rows n0 + 0..31: gate (set 0), up (set 1)
  c.set_weights(gcodes, ucodes, gsm, usm, (size_t)e * nbd * f, f,
                [&](int, int r) { return n0 + r; });
  c.run();

  __syncthreads();  // every wave is done with the ring before it is reused
  uint16_t* stg = reinterpret_cast<uint16_t*>(stages) + c.wave * (kBM * 32);
  const int lane = c.lane;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int rr = 32 * i + (q / 4) * 8 + (lane / 32) * 4 + (q % 4);
      const __bf16 v = (__bf16)silu_mul(c.acc[0][i][q], c.acc[1][i][q]);
      __builtin_memcpy(&stg[rr * 32 + (lane & 31)], &v, 2);
    }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // 32*NI rows x 4 chunks of 8 bf16: lane l takes chunk l%4 of rows l/4 + 16p
  const int col0 = n0 + 8 * (lane & 3);
  if (col0 < f) {
#pragma unroll
    for (int p = 0; p < 2 * NI; ++p) {
      const int rr = (lane >> 2) + 16 * p;
      if (rr < rows)
        *reinterpret_cast<uint4*>(h + (size_t)(g0 + rr) * f + col0) =
            *reinterpret_cast<const uint4*>(&stg[rr * 32 + 8 * (lane & 3)]);
    }
  }
}

template <int BITS>
__global__ __launch_bounds__(kRbThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_pf_gateup(
    const uint32_t* __restrict__ gcodes, const uint32_t* __restrict__ gsm,
    const uint32_t* __restrict__ ucodes, const uint32_t* __restrict__ usm, int d, int f,
    const int4* __restrict__ tiles, const int* __restrict__ ntiles,
    const uint16_t* __restrict__ x, const int* __restrict__ tok_of_g, uint16_t* __restrict__ h) {
  __shared__ RbStage stages[kRbStages];
  constexpr int kN = 4 * 32;  // weight rows a workgroup
  const int ntn = (f + kN - 1) / kN;
  int mt, nt;
  if (!xcd_tile(load_uniform(ntiles), ntn, mt, nt)) return;
  const int4 tile = load_uniform(tiles + mt);
  const int e = tile.x, g0 = tile.y, rows = tile.z;
  switch (row_groups(rows)) {
    case 1:
      pf_gateup_tile<BITS, 1>(stages, gcodes, gsm, ucodes, usm, d, f, e, g0, rows, nt * kN, x,
                              tok_of_g, h);
      break;
    case 2:
      pf_gateup_tile<BITS, 2>(stages, gcodes, gsm, ucodes, usm, d, f, e, g0, rows, nt * kN, x,
                              tok_of_g, h);
      break;
    case 4:
      pf_gateup_tile<BITS, 4>(stages, gcodes, gsm, ucodes, usm, d, f, e, g0, rows, nt * kN, x,
                              tok_of_g, h);
      break;
    default:
      pf_gateup_tile<BITS, 8>(stages, gcodes, gsm, ucodes, usm, d, f, e, g0, rows, nt * kN, x,
                              tok_of_g, h);
  }
}

// ---------------------------------------------------------------- down GEMM

// Lanes l and l+32 hold column 32q + l%32 of rows 32i + 8(e/4) + 4(l/32) + e%4; 32-row
// groups wholly inside the tile store without a per-row test. The fp32 pair outputs
// (671 MB at the 8192-token chunk, more than the 256 MB memory-side cache) are stored
// non-temporally: left dirty in that cache, their write-back competed with the combine's
// reads of them (172 against 146 us for the combine).
template <int BITS, int NI>
__device__ __forceinline__ void pf_down_tile(RbStage* stages, const uint32_t* __restrict__ dcodes,
                                             const uint32_t* __restrict__ dsm, int d, int f,
                                             int e, int g0, int rows, int c0w,
                                             const uint16_t* __restrict__ h,
                                             float* __restrict__ y) {
  const int nbf = f / kBK;
  RbCore<BITS, NI> c;
  c.init(stages, nbf);
#pragma unroll
  for (int i = 0; i < RbCore<BITS, NI>::kDmaA; ++i)
    c.arow[i] = reinterpret_cast<const char*>(h + (size_t)(g0 + min(c.arow_index(i), rows - 1)) * f) +
                c.aseg_bytes();
  const int c0 = c0w + 64 * c.wave;  // set q: output columns c0 + 32q + 0..31
  c.set_weights(dcodes, dcodes, dsm, dsm, (size_t)e * nbf * d, d,
                [&](int q, int r) { return c0 + 32 * q + r; });
  c.run();
  const int lane = c.lane;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int col = c0 + 32 * q + (lane & 31);
    if (col >= d) continue;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float* yb = y + (size_t)(g0 + 32 * i + (lane / 32) * 4) * d + col;
      if (32 * i + 32 <= rows) {
#pragma unroll
        for (int e2 = 0; e2 < 16; ++e2) __builtin_nontemporal_store(c.acc[q][i][e2], &yb[(size_t)((e2 / 4) * 8 + (e2 % 4)) * d]);
      } else if (32 * i < rows) {
#pragma unroll
        for (int e2 = 0; e2 < 16; ++e2) {
          const int rr = 32 * i + (e2 / 4) * 8 + (lane / 32) * 4 + (e2 % 4);
          if (rr < rows) __builtin_nontemporal_store(c.acc[q][i][e2], &yb[(size_t)((e2 / 4) * 8 + (e2 % 4)) * d]);
        }
      }
    }
  }
}

template <int BITS>
__global__ __launch_bounds__(kRbThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_pf_down(
    const uint32_t* __restrict__ dcodes, const uint32_t* __restrict__ dsm, int d, int f,
    const int4* __restrict__ tiles, const int* __restrict__ ntiles,
    const uint16_t* __restrict__ h, float* __restrict__ y) {
  __shared__ RbStage stages[kRbStages];
  constexpr int kN = 4 * 64;  // output columns a workgroup
  const int ntn = (d + kN - 1) / kN;
  int mt, nt;
  if (!xcd_tile(load_uniform(ntiles), ntn, mt, nt)) return;
  const int4 tile = load_uniform(tiles + mt);
  const int e = tile.x, g0 = tile.y, rows = tile.z;
  switch (row_groups(rows)) {
    case 1:
      pf_down_tile<BITS, 1>(stages, dcodes, dsm, d, f, e, g0, rows, nt * kN, h, y);
      break;
    case 2:
      pf_down_tile<BITS, 2>(stages, dcodes, dsm, d, f, e, g0, rows, nt * kN, h, y);
      break;
    case 4:
      pf_down_tile<BITS, 4>(stages, dcodes, dsm, d, f, e, g0, rows, nt * kN, h, y);
      break;
    default:
      pf_down_tile<BITS, 8>(stages, dcodes, dsm, d, f, e, g0, rows, nt * kN, h, y);
  }
}

// ---------------------------------------------------------------- combine

// One workgroup per token, 4 columns per thread: the token's k pair-output rows are all
// requested (non-temporal loads: each is read once) before the first is summed, then
// residual[t] += sum_j w[t][j] * y[g(t,j)] in slot order (binary64, one rounding).
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
          const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + (size_t)g * d + c));
          v[i] = make_float4(t[0], t[1], t[2], t[3]);
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
    const int gu_items = xcd_grid(max_mt, (f + 127) / 128);
    hipLaunchKernelGGL(k_pf_gateup<BITS>, dim3(gu_items), dim3(kRbThreads), 0, a.stream,
                       L.gate.codes, reinterpret_cast<const uint32_t*>(L.gate.scale_min),
                       L.up.codes, reinterpret_cast<const uint32_t*>(L.up.scale_min), d, f, tiles,
                       ntiles, a.x, tok_of_g, h);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (a.stages & MOE_PREFILL_DOWN) {
    const int dn_items = xcd_grid(max_mt, (d + 255) / 256);
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

// Seeded synthetic inputs for the routed-expert MoE layer.
//
// This file draws inputs only: block-quantized expert weights, activations and
// router-logit noise. It holds no step of the MoE computation (no routing, no
// dequantization, no dot products). Both the CPU checker and the GPU library
// consume the bytes it writes; host and device code below produce identical
// bytes for the same (seed, tensor, layer, index), so a large layer can be
// filled directly in device memory while a checker regenerates any expert of it
// on the host.
//
// Recipe:
//   * bits:   lowbias32 (C. Wellons, "hash-prospector") of idx*0x9E3779B9 + key,
//             key derived from (seed, tensor id, layer id) with the same hash;
//   * normal: approximate N(0, sigma) as (sum of the 4 bytes of one hash - 510)
//             * sigma/147.80054 (Irwin-Hall with 4 terms; the byte sum has
//             variance 4*(256^2-1)/12);
//   * weights of expert e, row r, column c use idx = (e*rows + r)*cols + c, so
//             the drawn dense weight does not depend on the packed layout;
//   * quantization of each run of 32 weights along the column (reduction) axis:
//             mn/mx = min/max, scale = fp16_rne((mx-mn)/(2^bits-1)),
//             min = fp16_rne(mn), code = clamp(rne((w-min)/scale), 0, 2^bits-1)
//             (code 0 when scale is 0).
//
// Packed layout written (the layout the library consumes):
//   codes     uint32 [E][cols/32][rows][bits]  (32 codes of `bits` bits per block,
//             code i in word i/(32/bits) at bit offset bits*(i%(32/bits)))
//   scale_min uint16 [E][cols/32][rows][2]     (fp16 scale, fp16 min)
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#pragma clang fp contract(off)

#define QS_HD __host__ __device__ __forceinline__

QS_HD uint32_t qs_hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

QS_HD uint32_t qs_key(uint64_t seed, uint32_t tensor, uint32_t layer) {
  uint32_t k = qs_hash32((uint32_t)seed ^ 0xA511E9B3u);
  k = qs_hash32(k ^ (uint32_t)(seed >> 32));
  k = qs_hash32(k ^ (tensor * 0x9E3779B9u));
  k = qs_hash32(k ^ (layer * 0x85EBCA6Bu + 0x27D4EB2Fu));
  return k;
}

QS_HD uint32_t qs_bits(uint32_t key, uint32_t idx) { return qs_hash32(idx * 0x9E3779B9u + key); }

QS_HD float qs_normal(uint32_t key, uint32_t idx, float scale) {
  uint32_t h = qs_bits(key, idx);
  int s = (int)(h & 255u) + (int)((h >> 8) & 255u) + (int)((h >> 16) & 255u) + (int)(h >> 24) - 510;
  return (float)s * scale;
}

QS_HD uint16_t qs_f16_bits(_Float16 h) {
  uint16_t u;
  memcpy(&u, &h, 2);
  return u;
}

// Draw and quantize one block of 32 weights.
QS_HD void qs_weight_block(uint32_t key, uint32_t base_idx, float scale, int bits,
                           uint32_t* words, uint16_t* sm) {
  float w[32];
  for (int i = 0; i < 32; ++i) w[i] = qs_normal(key, base_idx + (uint32_t)i, scale);
  float mn = w[0], mx = w[0];
  for (int i = 1; i < 32; ++i) {
    mn = w[i] < mn ? w[i] : mn;
    mx = w[i] > mx ? w[i] : mx;
  }
  const int levels = (1 << bits) - 1;
  const _Float16 s16 = (_Float16)((mx - mn) / (float)levels);
  const _Float16 m16 = (_Float16)mn;
  const float s = (float)s16, m = (float)m16;
  const int per_word = 32 / bits;
  uint32_t acc[4] = {0u, 0u, 0u, 0u};
  for (int i = 0; i < 32; ++i) {
    int q = 0;
    if (s != 0.0f) {
      float t = rintf((w[i] - m) / s);
      q = t < 0.0f ? 0 : (t > (float)levels ? levels : (int)t);
    }
    acc[i / per_word] |= (uint32_t)q << (bits * (i % per_word));
  }
  for (int j = 0; j < bits; ++j) words[j] = acc[j];
  sm[0] = qs_f16_bits(s16);
  sm[1] = qs_f16_bits(m16);
}

__global__ void qs_weights_kernel(uint32_t key, int E, int rows, int cols, int bits, float scale,
                                  uint32_t* __restrict__ codes, uint16_t* __restrict__ sm) {
  const int nb = cols / 32;
  const uint64_t nblk = (uint64_t)E * nb * rows;
  for (uint64_t L = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; L < nblk;
       L += (uint64_t)gridDim.x * blockDim.x) {
    const int r = (int)(L % rows);
    const uint64_t t = L / rows;
    const int b = (int)(t % nb);
    const int e = (int)(t / nb);
    const uint32_t base = (uint32_t)(((uint64_t)e * rows + r) * cols + 32u * b);
    qs_weight_block(key, base, scale, bits, codes + L * bits, sm + L * 2);
  }
}

static int qs_hw_threads(int req) {
  if (req > 0) return req;
  unsigned h = std::thread::hardware_concurrency();
  return h == 0 ? 1 : (int)std::min(h, 16u);
}

extern "C" {

uint32_t qs_stream_key(uint64_t seed, uint32_t tensor, uint32_t layer) {
  return qs_key(seed, tensor, layer);
}

// Fill the listed experts (all experts when `experts` is NULL) of a packed matrix in
// host memory. `codes` / `sm` are full-size [E][cols/32][rows][...] buffers.
int qs_weights_host(uint64_t seed, uint32_t tensor, uint32_t layer, int E, int rows, int cols,
                    int bits, float scale, const int32_t* experts, int n_experts, uint32_t* codes,
                    uint16_t* sm, int nthreads) {
  if ((bits != 2 && bits != 4) || cols % 32 != 0 || rows <= 0 || E <= 0) return 1;
  const uint32_t key = qs_key(seed, tensor, layer);
  const int nb = cols / 32;
  std::vector<int> list;
  if (experts) {
    for (int i = 0; i < n_experts; ++i) {
      if (experts[i] < 0 || experts[i] >= E) return 1;
      list.push_back(experts[i]);
    }
  } else {
    for (int e = 0; e < E; ++e) list.push_back(e);
  }
  const int64_t units = (int64_t)list.size() * nb;  // one unit = (expert, block column)
  const int nt = qs_hw_threads(nthreads);
  auto work = [&](int tid) {
    for (int64_t u = tid; u < units; u += nt) {
      const int e = list[u / nb];
      const int b = (int)(u % nb);
      for (int r = 0; r < rows; ++r) {
        const uint64_t L = ((uint64_t)e * nb + b) * rows + r;
        const uint32_t base = (uint32_t)(((uint64_t)e * rows + r) * cols + 32u * b);
        qs_weight_block(key, base, scale, bits, codes + L * bits, sm + L * 2);
      }
    }
  };
  std::vector<std::thread> th;
  for (int t = 1; t < nt; ++t) th.emplace_back(work, t);
  work(0);
  for (auto& t : th) t.join();
  return 0;
}

// Same bytes as qs_weights_host for every expert, written by the GPU.
int qs_weights_device(uint64_t seed, uint32_t tensor, uint32_t layer, int E, int rows, int cols,
                      int bits, float scale, uint32_t* codes, uint16_t* sm, void* stream) {
  if ((bits != 2 && bits != 4) || cols % 32 != 0 || rows <= 0 || E <= 0) return 1;
  const uint32_t key = qs_key(seed, tensor, layer);
  const uint64_t nblk = (uint64_t)E * (cols / 32) * rows;
  const int threads = 256;
  uint64_t blocks = (nblk + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(qs_weights_kernel, dim3((unsigned)blocks), dim3(threads), 0,
                     (hipStream_t)stream, key, E, rows, cols, bits, scale, codes, sm);
  return (int)hipGetLastError();
}

void qs_normal_host(uint64_t seed, uint32_t tensor, uint32_t layer, uint64_t count, float scale,
                    float* out) {
  const uint32_t key = qs_key(seed, tensor, layer);
  for (uint64_t i = 0; i < count; ++i) out[i] = qs_normal(key, (uint32_t)i, scale);
}

void qs_uniform_host(uint64_t seed, uint32_t tensor, uint32_t layer, uint64_t count, float* out) {
  const uint32_t key = qs_key(seed, tensor, layer);
  for (uint64_t i = 0; i < count; ++i)
    out[i] = (float)(qs_bits(key, (uint32_t)i) >> 8) * (1.0f / 16777216.0f);
}

// Fisher-Yates shuffle of 0..n-1 driven by the same hash.
void qs_perm_host(uint64_t seed, uint32_t tensor, uint32_t layer, int n, int32_t* out) {
  const uint32_t key = qs_key(seed, tensor, layer);
  for (int i = 0; i < n; ++i) out[i] = i;
  for (int i = n - 1; i > 0; --i) {
    const int j = (int)(qs_bits(key, (uint32_t)i) % (uint32_t)(i + 1));
    const int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

}  // extern "C"

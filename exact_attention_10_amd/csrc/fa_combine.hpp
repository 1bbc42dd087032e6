// Combine kernel of the split-KV forward pass.
//
// Each split s of a query row's keys produced a normalised partial O_s and its
// log-sum-exp LSE_s over its own keys. The row's result over all keys is the
// rebasing the online softmax already does between key tiles, applied once
// across splits: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s
// ("A09 - Advanced Triton & FlashAttention", section 3, the rescaling update,
// whose identity holds for any partition of the keys; "Building a Verifiable
// FlashAttention Forward from PyTorch to Triton", Part 3, on split-KV needing
// one consistent exponent base). A split that saw no key has LSE_s = -inf and
// weight 0; a row whose splits all saw no key gets O = 0 and LSE = -inf.
#pragma once

#include "fa_kernel.hpp"

namespace fa {

struct CombineParams {
  const float *o_part;     // [n_splits][rows][D]
  const float *lse_part;   // [n_splits][rows]
  void *o;                 // [rows][D] in the input dtype
  float *lse;              // [rows] or null
  int64_t rows;            // B*H*nq
  int n_splits;            // 1 .. kMaxSplits
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// One 64-lane wave per query row; lane s holds split s's LSE, and each lane
// owns D/64 consecutive output elements. 4 rows per 256-thread workgroup.
template <int DT, int D>
__global__ void __launch_bounds__(256) fa_splitkv_combine_kernel(CombineParams p) {
  constexpr int E = D / 64;                      // output elements per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int ns = p.n_splits;
  const float ls = lane < ns ? p.lse_part[(int64_t)lane * p.rows + row] : -INFINITY;
  const float m = wave_max(ls);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float lse_row = -INFINITY;
  if (m != -INFINITY) {
    const float w = lane < ns ? __expf(ls - m) : 0.f;   // exp(-inf) = 0 for empty splits
    const float wsum = wave_sum(w);
    const float inv = 1.0f / wsum;
    lse_row = m + __logf(wsum);
    for (int s = 0; s < ns; ++s) {
      const float ws = __shfl(w, s, 64) * inv;
      if (ws == 0.f) continue;                          // wave-uniform
      const float *src = p.o_part + ((int64_t)s * p.rows + row) * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += ws * src[e];
    }
  }
  if constexpr (DT == DT_FP32) {
    float *dst = (float *)p.o + row * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e] = acc[e];
  } else {
    uint16_t *dst = (uint16_t *)p.o + row * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      const uint32_t pr = pack2<DT>(acc[e], e + 1 < E ? acc[e + 1] : 0.f);
      if (E >= 2) {
        *(uint32_t *)(dst + e) = pr;
      } else {
        dst[e] = (uint16_t)(pr & 0xffffu);
      }
    }
  }
  if (p.lse && lane == 0) p.lse[row] = lse_row;
}

}  // namespace fa

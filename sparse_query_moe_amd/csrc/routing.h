// Device-side routing helpers: float64 widening shared by the prefill router
// and the decode step's router blocks, and the decode step's per-token
// routing (pptc.cn review, section 7: softmax inside the group
// first, then top-k; section 5: every group takes part; hotpaper.ai,
// technical approach: renormalized scoring).  Logits are float64: products of
// bf16/fp32 inputs are exact in float64, so the only rounding is in the sums.
#pragma once

#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace gqe {

// 8 elements of T as raw 16-byte words: one for bf16, two for fp32
template <typename T> struct U4Count { static constexpr int n = sizeof(T) == 2 ? 1 : 2; };

// widen 8 stored elements to float64 (exact)
template <typename T>
__device__ __forceinline__ void widen8(const uint4 (&r)[U4Count<T>::n], double (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = static_cast<double>(__uint_as_float(w[j] << 16));
      v[2 * j + 1] = static_cast<double>(__uint_as_float(w[j] & 0xffff0000u));
    }
  } else {
    const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = static_cast<double>(__uint_as_float(w[j]));
  }
}

// One token per block of 256 threads (the decode step's few tokens): wave w
// forms the logits of experts w, w+4, ...; lane l accumulates model dims
// 8l + 512i in float64 and the wave sums its lanes in a fixed butterfly
// order.  Then one thread per expert takes its rank and exp(r - max); the
// weights divide by the sum over the group's selected experts (all E when
// !renorm) in expert order, the same operations as the prefill router's
// selection.
template <typename T>
__device__ __forceinline__ void route_token_block(const T* __restrict__ x, const T* __restrict__ wr,
                                                  const float* __restrict__ bias,
                                                  int32_t* __restrict__ idx_out,
                                                  float* __restrict__ w_out, int t, int d, int G,
                                                  int E, const GroupK& gk, int renorm) {
  __shared__ double logit[64], ex[64];
  __shared__ int rank_of[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int GE = G * E;
  constexpr int kU4 = U4Count<T>::n;
  const T* xp = x + static_cast<size_t>(t) * d;
  for (int e = wave; e < GE; e += 4) {
    const T* wp = wr + static_cast<size_t>(e) * d;
    double acc = 0.0;
    for (int d0 = 8 * lane; d0 < d; d0 += 512) {
      uint4 rx[kU4], rw[kU4];
#pragma unroll
      for (int q = 0; q < kU4; ++q) {
        rx[q] = reinterpret_cast<const uint4*>(xp + d0)[q];
        rw[q] = reinterpret_cast<const uint4*>(wp + d0)[q];
      }
      double xv[8], wv[8];
      widen8<T>(rx, xv);
      widen8<T>(rw, wv);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = fma(xv[j], wv[j], acc);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) logit[e] = acc + (bias ? static_cast<double>(bias[e]) : 0.0);
  }
  __syncthreads();
  if (tid < GE) {
    const int g = tid / E, e = tid % E;
    const double* r = &logit[g * E];
    double rmax = r[0];
    for (int f = 1; f < E; ++f) rmax = fmax(rmax, r[f]);
    int rank = 0;
    for (int f = 0; f < E; ++f) rank += (r[f] > r[e]) || (r[f] == r[e] && f < e);
    ex[tid] = exp(r[e] - rmax);
    rank_of[tid] = rank;
  }
  __syncthreads();
  if (tid < GE) {
    const int g = tid / E, e = tid % E;
    const int rank = rank_of[tid];
    const int k = gk.kg[g];
    if (rank < k) {
      double z = 0.0;
      for (int f = 0; f < E; ++f)
        if (rank_of[g * E + f] < k || !renorm) z += ex[g * E + f];
      const size_t o = static_cast<size_t>(t) * gk.K + gk.koff[g];  // group g's slots of token t
      idx_out[o + rank] = e;
      w_out[o + rank] = static_cast<float>(ex[tid] / z);
    }
  }
}

}  // namespace gqe

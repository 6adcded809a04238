// K1: router logits, in-group top-k and renormalized weights.
//
// Method (pptc.cn review, section 7: softmax inside the group first, then
// top-k; section 5: the top-k is taken inside every fixed GQA group, so every
// group participates; hotpaper.ai, technical approach: renormalized scoring):
//   r[t, g, e] = x[t] . Wr[g*E+e] + b[g*E+e]
//   idx[t, g, :] = the k experts of group g with the largest r (equivalently
//                  the largest in-group softmax p), best first, ties to the
//                  lower index
//   w[t, g, j]  = exp(r_j - r_0) / sum_j' exp(r_j' - r_0), which equals the
//                  in-group softmax renormalized over the selected k.
//
// The logits are accumulated in float64: products of two bf16 (or two fp32)
// values are exact in float64, so the only rounding is in the sums, far below
// the gaps that decide the selection.
//
// Work split: a block of 256 threads handles 64 tokens; thread (tok, part)
// accumulates the experts e = part + 4m.  x and Wr stream through LDS in
// chunks of 64 model dimensions; the selection then runs one thread per
// (token, group).  HBM traffic is x once plus idx/w: the kernel is bound by
// float64 FMA throughput at about 16 FMAs per loaded x element.
#include "device_common.h"
#include "kernels.h"

namespace gqe {

namespace {

constexpr int kTokPerBlock = 64;
constexpr int kDChunk = 64;
constexpr int kXStride = kDChunk + 1;  // odd float stride: conflict-free row reads

template <typename T>
__global__ __launch_bounds__(256) void router_topk_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ bias,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int n_tokens, int d, int G, int E,
    int k) {
  extern __shared__ __align__(16) char smem[];
  const int GE = G * E;
  float* xs = reinterpret_cast<float*>(smem);                                   // [64][65]
  double* ws = reinterpret_cast<double*>(smem + kTokPerBlock * kXStride * 4 + 16);  // [GE][64]
  double* rl = ws;  // reused after the dot products: [64][GE+1]

  const int tid = threadIdx.x;
  const int tok = tid & 63;
  const int part = tid >> 6;
  const int t0 = blockIdx.x * kTokPerBlock;
  const int ept = (GE + 3) >> 2;  // experts per thread (<= 16)

  double acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = 0.0;

  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  for (int d0 = 0; d0 < d; d0 += kDChunk) {
    const int dn = min(kDChunk, d - d0);
    // x chunk: 64 tokens x 64 dims
    for (int c = tid; c < kTokPerBlock * (kDChunk / EPC); c += 256) {
      const int r = c / (kDChunk / EPC);
      const int cc = c % (kDChunk / EPC);
      const int gt = t0 + r;
      float v[EPC];
      if (gt < n_tokens && cc * EPC < dn) {
        const T* p = x + static_cast<size_t>(gt) * d + d0 + cc * EPC;
        uint4 raw = *reinterpret_cast<const uint4*>(p);
        const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int j = 0; j < EPC; ++j) v[j] = to_f32(e[j]);
      } else {
#pragma unroll
        for (int j = 0; j < EPC; ++j) v[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < EPC; ++j) xs[r * kXStride + cc * EPC + j] = v[j];
    }
    // router weight chunk: GE rows x 64 dims, widened to float64
    for (int c = tid; c < GE * (kDChunk / EPC); c += 256) {
      const int r = c / (kDChunk / EPC);
      const int cc = c % (kDChunk / EPC);
      double v[EPC];
      if (cc * EPC < dn) {
        const T* p = wr + static_cast<size_t>(r) * d + d0 + cc * EPC;
        uint4 raw = *reinterpret_cast<const uint4*>(p);
        const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int j = 0; j < EPC; ++j) v[j] = static_cast<double>(to_f32(e[j]));
      } else {
#pragma unroll
        for (int j = 0; j < EPC; ++j) v[j] = 0.0;
      }
#pragma unroll
      for (int j = 0; j < EPC; ++j) ws[r * kDChunk + cc * EPC + j] = v[j];
    }
    __syncthreads();
    for (int i = 0; i < kDChunk; ++i) {
      const double xv = static_cast<double>(xs[tok * kXStride + i]);
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        if (m < ept) {
          const int e = part + 4 * m;
          if (e < GE) acc[m] = fma(xv, ws[e * kDChunk + i], acc[m]);
        }
      }
    }
    __syncthreads();
  }

  // logits (+ bias) to LDS, one row per token
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int e = part + 4 * m;
    if (m < ept && e < GE) {
      const double b = bias ? static_cast<double>(bias[e]) : 0.0;
      rl[tok * (GE + 1) + e] = acc[m] + b;
    }
  }
  __syncthreads();

  // selection: one thread per (token, group)
  for (int task = tid; task < kTokPerBlock * G; task += 256) {
    const int tt = task % kTokPerBlock;
    const int g = task / kTokPerBlock;
    const int gt = t0 + tt;
    if (gt >= n_tokens) continue;
    const double* r = rl + tt * (GE + 1) + g * E;
    uint32_t taken = 0u;
    double rsel[32];
    int isel[32];
    for (int j = 0; j < k; ++j) {
      int best = -1;
      double bv = 0.0;
      for (int e = 0; e < E; ++e) {
        if (taken & (1u << e)) continue;
        const double v = r[e];
        if (best < 0 || v > bv) {  // strict: equal values keep the lower index
          best = e;
          bv = v;
        }
      }
      taken |= 1u << best;
      rsel[j] = bv;
      isel[j] = best;
    }
    double z = 0.0;
    for (int j = 0; j < k; ++j) z += exp(rsel[j] - rsel[0]);
    const size_t o = (static_cast<size_t>(gt) * G + g) * k;
    for (int j = 0; j < k; ++j) {
      idx_out[o + j] = isel[j];
      w_out[o + j] = static_cast<float>(exp(rsel[j] - rsel[0]) / z);
    }
  }
}

}  // namespace

size_t router_smem_bytes(int G, int E) {
  const int GE = G * E;
  size_t a = static_cast<size_t>(GE) * kDChunk * 8;
  size_t b = static_cast<size_t>(kTokPerBlock) * (GE + 1) * 8;
  return kTokPerBlock * kXStride * 4 + 16 + (a > b ? a : b);
}

template <typename T>
hipError_t launch_router(const T* x, const T* wr, const float* bias, int32_t* idx, float* w,
                         int n_tokens, int d, int G, int E, int k, hipStream_t stream) {
  const int blocks = (n_tokens + kTokPerBlock - 1) / kTokPerBlock;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(router_topk_kernel<T>, dim3(blocks), dim3(256), router_smem_bytes(G, E),
                     stream, x, wr, bias, idx, w, n_tokens, d, G, E, k);
  return hipGetLastError();
}

template hipError_t launch_router<bf16_t>(const bf16_t*, const bf16_t*, const float*, int32_t*,
                                          float*, int, int, int, int, int, hipStream_t);
template hipError_t launch_router<float>(const float*, const float*, const float*, int32_t*,
                                         float*, int, int, int, int, int, hipStream_t);

}  // namespace gqe

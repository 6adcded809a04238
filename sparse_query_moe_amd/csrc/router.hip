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
//                  in-group softmax renormalized over the selected k
//                  (or, for the weighted-concatenation ablation of section
//                  4.3, the in-group softmax p itself: the sum runs over
//                  all E experts).
//
// Two kernels compute the logits.
//
// bf16 layers (router_bf16_kernel): the products of two bf16 values are
// exact in float32, so the bf16 matrix cores (v_mfma_f32_16x16x32_bf16: 16
// tokens x 16 experts x 32 model dims) form every 32-dim partial sum with
// float32 rounding only, and each partial is added into float64
// accumulators.  The result is within
//     31 * 2^-24 * sum_i |x_i| |w_i|  <=  31 * 2^-24 * ||x_t|| * ||w_e||
// of the exact logit (a sequential float32 sum of 32 products at worst,
// then float64 sums).  Wherever a gap that decides the selection or the rank
// order of a (token, group) is within twice that bound, the group's logits
// are recomputed from the products in float64 in a fixed order (the same
// accuracy as the float64 kernel below), so every decision is the one the
// float64 logits make.  A 16-token tile takes all experts, its model
// dimension split over 4 waves (up to 2^19 tokens; from 2^16 tokens each
// wave takes two tiles when one 16-expert tile holds every expert) or held by
// one wave (longer launches); x is read once, W_r once per block (from L2).
//
// fp32 layers, and model widths that are not a multiple of 32
// (router_f64_kernel): the logits are accumulated in float64 on the fp64
// matrix cores (v_mfma_f64_16x16x4: 16 tokens x 16 experts x 4 model dims);
// fp32 inputs are exact in float64, so the only rounding is in the sums.  A
// block of 4 waves takes 16 tokens; each wave accumulates a quarter of the
// model dimension and the four partial 16x16 tiles are added in LDS in a
// fixed order (deterministic).  Every lane loads 8 consecutive elements of x
// and of Wr per 32-dimension step and feeds them to 8 MFMAs; the K index each
// (lane, step) pair covers is the same for both operands, so the products
// pair up correctly.
//
// The selection (both kernels) computes each expert's rank (number of
// experts ahead of it), which needs no per-thread arrays.
#include "device_common.h"
#include "kernels.h"
#include "router_dev.h"
#include "routing.h"

namespace gqe {

namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kTok = 16;

template <typename T>
__global__ __launch_bounds__(256) void router_f64_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ bias,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int n_tokens, int d, int G, int E,
    GroupK gk, int renorm) {
  __shared__ double part[4][kTok][17];
  __shared__ double logit[kTok][65];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, h = lane >> 4;
  const int t0 = blockIdx.x * kTok;
  const int tok = t0 + row;
  const int GE = G * E;
  const int nsteps = (d + 31) >> 5;
  constexpr int kU4 = U4Count<T>::n;
  constexpr int kBatch = sizeof(T) == 2 ? 8 : 4;  // steps whose loads are issued together

  for (int eb = 0; eb < GE; eb += 16) {
    const int e = eb + row;
    const T* xp = x + static_cast<size_t>(tok < n_tokens ? tok : 0) * d;
    const T* wp = wr + static_cast<size_t>(e < GE ? e : 0) * d;
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
    // batches of 8 steps: every load of a batch is issued before its MFMAs,
    // so the wave waits for memory once per batch instead of once per step
    for (int st0 = wave; st0 < nsteps; st0 += 4 * kBatch) {
      uint4 rx[kBatch][kU4], rw[kBatch][kU4];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int d0 = (st0 + 4 * u) * 32 + 8 * h;
        const bool okx = st0 + 4 * u < nsteps && tok < n_tokens && d0 < d;
        const bool okw = st0 + 4 * u < nsteps && e < GE && d0 < d;
#pragma unroll
        for (int q = 0; q < kU4; ++q) {
          rx[u][q] = okx ? reinterpret_cast<const uint4*>(xp + d0)[q] : make_uint4(0, 0, 0, 0);
          rw[u][q] = okw ? reinterpret_cast<const uint4*>(wp + d0)[q] : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        double xv[8], wv[8];
        widen8<T>(rx[u], xv);
        widen8<T>(rw[u], wv);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xv[j], wv[j], acc, 0, 0, 0);
      }
    }
    // accumulator of the f64 16x16 MFMA: value i of lane l is C[4i + l/16][l % 16],
    // i.e. token 4i + h, expert eb + row
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][4 * i + h][row] = acc[i];
    __syncthreads();
    {
      const int tt = tid >> 4, ee = tid & 15;  // 256 threads = 16 tokens x 16 experts
      if (eb + ee < GE) {
        double s = part[0][tt][ee];
        s += part[1][tt][ee];
        s += part[2][tt][ee];
        s += part[3][tt][ee];
        logit[tt][eb + ee] = s + (bias ? static_cast<double>(bias[eb + ee]) : 0.0);
      }
    }
    __syncthreads();
  }

  // selection, one thread per (token, expert): the expert's rank inside its
  // group (experts with a larger logit, or an equal one and a lower index)
  // and exp(r - max) once; then each selected expert's weight divides by the
  // sum over its group's selected experts (all E when !renorm) in expert order
  __shared__ double ex[kTok][65];
  __shared__ int rk[kTok][65];
  for (int task = tid; task < kTok * GE; task += 256) {
    const int tt = task / GE, ge = task % GE, g = ge / E, e = ge % E;
    const double* r = &logit[tt][g * E];
    double rmax = r[0];
    for (int f = 1; f < E; ++f) rmax = fmax(rmax, r[f]);
    int rank = 0;
    for (int f = 0; f < E; ++f) rank += (r[f] > r[e]) || (r[f] == r[e] && f < e);
    ex[tt][ge] = exp(r[e] - rmax);
    rk[tt][ge] = rank;
  }
  __syncthreads();
  for (int task = tid; task < kTok * GE; task += 256) {
    const int tt = task / GE, ge = task % GE, g = ge / E, e = ge % E;
    const int gt = t0 + tt, k = gk.kg[g], rank = rk[tt][ge];
    if (gt >= n_tokens || rank >= k) continue;
    double z = 0.0;
    for (int f = 0; f < E; ++f)
      if (rk[tt][g * E + f] < k || !renorm) z += ex[tt][g * E + f];
    const size_t o = static_cast<size_t>(gt) * gk.K + gk.koff[g];  // group g's slots of token gt
    idx_out[o + rank] = e;
    w_out[o + rank] = static_cast<float>(ex[tt][ge] / z);
  }
}

// The bf16 router kernel: one block body per block index
template <int NE, int KS, int TT>
__global__ __launch_bounds__(256, KS == 1 ? 6 : 2) void router_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, const float* __restrict__ bias,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int n_tokens, int d, int G, int E,
    GroupK gk, int renorm) {
  __shared__ RouterSmem<NE, KS, TT> sm;
  router_bf16_block<NE, KS, TT>(blockIdx.x, sm, x, wr, bias, idx_out, w_out, n_tokens, d, G, E,
                                gk, renorm);
}

// split: 4 waves share each 16-token tile's model dimension; two tiles per
// wave from 2^16 tokens when all experts fit one 16-expert tile
template <int NE>
void launch_router_bf16(bool split, const bf16_t* x, const bf16_t* wr, const float* bias,
                        int32_t* idx, float* w, int n_tokens, int d, int G, int E, const GroupK& gk,
                        int renorm, hipStream_t stream) {
  if constexpr (NE == 1) {
    if (split && n_tokens >= (1 << 16)) {
      const dim3 grid((n_tokens + 31) / 32);
      hipLaunchKernelGGL((router_bf16_kernel<1, 4, 2>), grid, dim3(256), 0, stream, x, wr, bias, idx,
                         w, n_tokens, d, G, E, gk, renorm);
      return;
    }
  }
  const int tb = split ? 16 : 64;  // tokens per block
  const dim3 grid((n_tokens + tb - 1) / tb);
  if (split)
    hipLaunchKernelGGL((router_bf16_kernel<NE, 4, 1>), grid, dim3(256), 0, stream, x, wr, bias, idx,
                       w, n_tokens, d, G, E, gk, renorm);
  else
    hipLaunchKernelGGL((router_bf16_kernel<NE, 1, 1>), grid, dim3(256), 0, stream, x, wr, bias, idx,
                       w, n_tokens, d, G, E, gk, renorm);
}

}  // namespace

template <typename T>
hipError_t launch_router(const T* x, const T* wr, const float* bias, int32_t* idx, float* w,
                         int n_tokens, int d, int G, int E, const GroupK& gk, bool renorm,
                         hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  if constexpr (sizeof(T) == 2) {
    const int GE = G * E;
    if (d % 32 == 0 && GE <= 64) {
      // up to 2^19 tokens, 4 waves split the model dims of every 16-token
      // tile (more blocks, whose load and selection phases then overlap);
      // beyond that, a wave owns 16 tokens and 8 waves share each SIMD
      const bool split = n_tokens <= (1 << 19) && d % 128 == 0;
      const int r = renorm ? 1 : 0;
      switch ((GE + 15) / 16) {
        case 1: launch_router_bf16<1>(split, x, wr, bias, idx, w, n_tokens, d, G, E, gk, r, stream); break;
        case 2: launch_router_bf16<2>(split, x, wr, bias, idx, w, n_tokens, d, G, E, gk, r, stream); break;
        case 3: launch_router_bf16<3>(split, x, wr, bias, idx, w, n_tokens, d, G, E, gk, r, stream); break;
        default: launch_router_bf16<4>(split, x, wr, bias, idx, w, n_tokens, d, G, E, gk, r, stream); break;
      }
      return hipGetLastError();
    }
  }
  const int blocks = (n_tokens + kTok - 1) / kTok;
  hipLaunchKernelGGL(router_f64_kernel<T>, dim3(blocks), dim3(256), 0, stream, x, wr, bias, idx,
                     w, n_tokens, d, G, E, gk, renorm ? 1 : 0);
  return hipGetLastError();
}

template hipError_t launch_router<bf16_t>(const bf16_t*, const bf16_t*, const float*, int32_t*,
                                          float*, int, int, int, int, const GroupK&, bool,
                                          hipStream_t);
template hipError_t launch_router<float>(const float*, const float*, const float*, int32_t*,
                                         float*, int, int, int, int, const GroupK&, bool,
                                         hipStream_t);

}  // namespace gqe

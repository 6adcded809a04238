// The bf16 router's block body (K1: router logits, in-group top-k and
// renormalized weights; pptc.cn review, section 7: softmax inside the group
// first, then top-k; section 5: every group takes part; hotpaper.ai,
// technical approach: renormalized scoring).  It is a device function of the
// block index so that the router kernel and the short-sequence front launch,
// which runs the router's blocks beside the dense projection's tiles, share
// it.  The error bound and the exact recheck of near ties are described in
// router.hip.
#pragma once

#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace gqe {

namespace {

// ---------------------------------------------------------------------------
// bf16 router: 4 waves x 16 tokens; NE tiles of 16 experts
// ---------------------------------------------------------------------------
// the selection of one (token, group) from its E logits r: ranks (larger
// logit first, ties to the lower index), then w = exp(r - max) / z with z the
// sum over the selected experts (all E when !renorm) in expert order.  Returns
// the smallest gap between consecutive ranks that decides the selection or
// its order (ranks 0 .. min(k, E-1)), and writes idx/w when `write`.
__device__ __forceinline__ double select_group(const double* r, int E, int k, int renorm,
                                               int32_t* idx_out, float* w_out, bool write) {
  double rmax = r[0];
  for (int f = 1; f < E; ++f) rmax = fmax(rmax, r[f]);
  const int kk = k < E - 1 ? k : E - 1;
  double z = 0.0, mingap = INFINITY;
  for (int e = 0; e < E; ++e) {
    int rank = 0;
    for (int f = 0; f < E; ++f) rank += (r[f] > r[e]) || (r[f] == r[e] && f < e);
    if (rank < k || !renorm) z += exp(r[e] - rmax);
    if (rank < kk) {  // the gap to the next rank: the largest logit ranked after e
      double nxt = -INFINITY;
      for (int f = 0; f < E; ++f)
        if (r[f] < r[e] || (r[f] == r[e] && f > e)) nxt = fmax(nxt, r[f]);
      mingap = fmin(mingap, r[e] - nxt);
    }
  }
  if (write) {
    for (int e = 0; e < E; ++e) {
      int rank = 0;
      for (int f = 0; f < E; ++f) rank += (r[f] > r[e]) || (r[f] == r[e] && f < e);
      if (rank < k) {
        idx_out[rank] = e;
        w_out[rank] = static_cast<float>(exp(r[e] - rmax) / z);
      }
    }
  }
  return mingap;
}

// KS: waves that split the model dimension of one 16-token tile (4 up to
// 2^19 tokens, so that many blocks exist and their phases overlap; 1 for the
// longest launches, where every wave takes its own tile, W_r is read once
// per 64 tokens and 8 waves share each SIMD).  Their float64 partial sums are
// added in LDS in a fixed order.
// (The long-launch form asks for 6 blocks per compute unit, which holds it to
// 64 VGPRs: 8 waves per SIMD, and enough of x in flight.)
// TT: 16-token tiles per wave (2 on long split launches with one 16-expert
// tile: W_r is then read once per 32 tokens, 7% faster at 2^17 tokens, and
// slower where the halved block count no longer fills the chip).
// The LDS of one router block: a static array of the router kernel, or the
// start of the front launch's dynamic LDS (the router blocks there do not
// touch the GEMM ring, so both share it).  Sized by the expert count, so
// that long launches keep several blocks per compute unit and enough of x in
// flight.
template <int NE, int KS, int TT>
struct RouterSmem {
  static constexpr int TB = 16 * TT * (4 / KS);  // tokens per block
  static constexpr int GEP = 16 * NE;            // experts of all groups, at most
  double logit[TB][GEP + 1];
  double part[KS > 1 ? KS : 1][TB][KS > 1 ? GEP : 1];
  double exs[KS > 1 ? TB : 1][GEP];  // split form: terms of the normalizer (0 outside it)
  float xpart[KS][TB], wpart[KS][GEP];
  float xnorm[TB], wnorm[GEP];
  unsigned char redo[TB * GEP];  // (token, group) pairs recomputed exactly
  unsigned char rkb[KS > 1 ? TB * GEP : 1];  // split form: rank | 0x80 when a deciding gap is too small
};

template <int NE, int KS, int TT>
__device__ __forceinline__ void router_bf16_block(
    int block, RouterSmem<NE, KS, TT>& sm, const bf16_t* __restrict__ x,
    const bf16_t* __restrict__ wr, const float* __restrict__ bias, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, int n_tokens, int d, int G, int E, const GroupK& gk, int renorm) {
  static_assert(KS > 1 || TT == 1, "the long-launch form takes one tile per wave");
  constexpr int TB = RouterSmem<NE, KS, TT>::TB;
  constexpr int GEP = RouterSmem<NE, KS, TT>::GEP;
  auto& logit = sm.logit;
  auto& part = sm.part;
  auto& xpart = sm.xpart;
  auto& wpart = sm.wpart;
  auto& xnorm = sm.xnorm;
  auto& wnorm = sm.wnorm;
  auto& redo = sm.redo;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, kq = lane >> 4;
  const int tile = (wave / KS) * TT, ksp = wave % KS;  // the wave's first tile
  const int blk0 = block * TB;
  const int GE = G * E;
  const int nsteps = d / 32 / KS;  // steps of this wave
  const int kbase = ksp * nsteps * 32;
  const bf16_t* xp[TT];
#pragma unroll
  for (int q = 0; q < TT; ++q) {
    const int tok = blk0 + (tile + q) * 16 + row;
    xp[q] = x + static_cast<size_t>(tok < n_tokens ? tok : 0) * d + kbase + 8 * kq;
  }
  const bf16_t* wp[NE];
#pragma unroll
  for (int n = 0; n < NE; ++n) {
    const int e = 16 * n + row;
    wp[n] = wr + static_cast<size_t>(e < GE ? e : 0) * d + kbase + 8 * kq;
  }
  double acc[TT][NE][4];
  float wsq[NE];
#pragma unroll
  for (int n = 0; n < NE; ++n) {
    wsq[n] = 0.f;
#pragma unroll
    for (int q = 0; q < TT; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[q][n][i] = 0.0;
  }
  float xsq[TT];
#pragma unroll
  for (int q = 0; q < TT; ++q) xsq[q] = 0.f;
  // 32 model dims per MFMA; U steps of loads are issued before their MFMAs
  constexpr int U = (NE <= 2 ? 8 : 4) / TT;
  auto sq8 = [](const bf16x8& v) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s = fmaf(static_cast<float>(v[j]), static_cast<float>(v[j]), s);
    return s;
  };
  for (int st = 0; st < nsteps; st += U) {
    bf16x8 a[TT][U], b[U][NE];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int o = (st + u < nsteps ? st + u : 0) * 32;
#pragma unroll
      for (int q = 0; q < TT; ++q) a[q][u] = load_frag(xp[q] + o);
#pragma unroll
      for (int n = 0; n < NE; ++n) b[u][n] = load_frag(wp[n] + o);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (st + u >= nsteps) break;
#pragma unroll
      for (int q = 0; q < TT; ++q) xsq[q] += sq8(a[q][u]);
#pragma unroll
      for (int n = 0; n < NE; ++n) {
        wsq[n] += sq8(b[u][n]);
#pragma unroll
        for (int q = 0; q < TT; ++q) {
          const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q][u], b[u][n],
                                                                 f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[q][n][i] += static_cast<double>(c[i]);
        }
      }
    }
  }
  // lanes row, row+16, row+32, row+48 hold disjoint dims of token / expert `row`
#pragma unroll
  for (int q = 0; q < TT; ++q) {
    float v = xsq[q];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (kq == 0) xpart[ksp][(tile + q) * 16 + row] = v;
  }
#pragma unroll
  for (int n = 0; n < NE; ++n) {
    float v = wsq[n];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (tile == 0 && kq == 0) wpart[ksp][16 * n + row] = v;
  }
  // accumulator of the 16x16 MFMA: value i of lane l is D[4*(l/16) + i][l % 16],
  // i.e. token 4*kq + i of the wave's tile, expert 16*n + row
#pragma unroll
  for (int n = 0; n < NE; ++n) {
    const int e = 16 * n + row;
    if (e < GE) {
#pragma unroll
      for (int q = 0; q < TT; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tt = (tile + q) * 16 + 4 * kq + i;
          if constexpr (KS == 1)
            logit[tt][e] = acc[q][n][i] + (bias ? static_cast<double>(bias[e]) : 0.0);
          else
            part[ksp][tt][e] = acc[q][n][i];
        }
    }
  }
  __syncthreads();
  if constexpr (KS > 1) {  // the split sums, in a fixed order
    for (int i = tid; i < TB * GE; i += 256) {
      const int tt = i / GE, e = i % GE;
      double v = part[0][tt][e];
#pragma unroll
      for (int k = 1; k < KS; ++k) v += part[k][tt][e];
      logit[tt][e] = v + (bias ? static_cast<double>(bias[e]) : 0.0);
    }
  }
  for (int i = tid; i < TB + GEP; i += 256) {
    float v = 0.f;
    if (i < TB) {
#pragma unroll
      for (int k = 0; k < KS; ++k) v += xpart[k][i];
      xnorm[i] = sqrtf(v);
    } else {
#pragma unroll
      for (int k = 0; k < KS; ++k) v += wpart[k][i - TB];
      wnorm[i - TB] = sqrtf(v);
    }
  }
  __syncthreads();

  // selection, with every (token, group) whose deciding gap is within twice
  // the error bound of its logits flagged for the exact recomputation.
  // Short launches take one lane per (token, expert): the expert's rank in
  // its group (larger logit first, ties to the lower index), its
  // exp(r - max), and whether the gap from it to the best expert ranked after
  // it decides the selection or its order and is too small.
  constexpr float kErr = 32.f * 0x1p-23f;  // per unit of ||x|| ||w||, with margin
  const int tasks = TB * G;
  bool any_fix = false;  // this thread flagged a (token, group)
  if constexpr (KS > 1) {
    constexpr int PER = (TB * GEP + 255) / 256;  // lane-tasks per thread, at most
    auto& rkb = sm.rkb;
    auto& exs = sm.exs;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + 256 * j;
      if (i >= TB * GE) continue;
      const int tt = i / GE, ge = i % GE, g = ge / E, e = ge % E;
      const double* r = &logit[tt][g * E];
      const double re = r[e];
      double rmax = r[0], nxt = -INFINITY;
      int rank = 0;
      for (int f = 0; f < E; ++f) {
        const double rf = r[f];
        rmax = fmax(rmax, rf);
        rank += (rf > re) || (rf == re && f < e);
        if (rf < re || (rf == re && f > e)) nxt = fmax(nxt, rf);
      }
      const int k = gk.kg[g], kk = k < E - 1 ? k : E - 1;
      float wmax = 0.f;
      for (int f = 0; f < E; ++f) wmax = fmaxf(wmax, wnorm[g * E + f]);
      const double tol = 2.0 * static_cast<double>(kErr) * xnorm[tt] * wmax;
      const bool bad = rank < kk && !(re - nxt > tol);
      rkb[i] = static_cast<unsigned char>(rank | (bad ? 0x80 : 0));
      exs[tt][ge] = (rank < k || !renorm) ? exp(re - rmax) : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + 256 * j;
      if (i >= TB * GE) continue;
      const int tt = i / GE, ge = i % GE, g = ge / E, e = ge % E;
      const int rank = rkb[i] & 0x7f, k = gk.kg[g];
      const int gt = blk0 + tt;
      const bool valid = gt < n_tokens;
      bool fix = false;
      for (int f = 0; f < E; ++f) fix = fix || (rkb[tt * GE + g * E + f] & 0x80);
      fix = fix && valid;
      if (rank == 0) redo[tt * G + g] = fix ? 1 : 0;
      any_fix = any_fix || fix;
      if (!valid || fix || rank >= k) continue;
      double z = 0.0;  // in expert order
      for (int f = 0; f < E; ++f) z += exs[tt][g * E + f];
      const size_t o = static_cast<size_t>(gt) * gk.K + gk.koff[g] + rank;
      idx_out[o] = e;
      w_out[o] = static_cast<float>(exs[tt][ge] / z);
    }
  } else {
    // long launches: one thread per (token, group), which keeps the block's
    // barriers few while other blocks stream their tokens
    for (int task = tid; task < tasks; task += 256) {
      const int tt = task / G, g = task % G;
      const int gt = blk0 + tt;
      float wmax = 0.f;
      for (int e = 0; e < E; ++e) wmax = fmaxf(wmax, wnorm[g * E + e]);
      const double tol = 2.0 * static_cast<double>(kErr) * xnorm[tt] * wmax;
      const bool valid = gt < n_tokens;
      const size_t o = static_cast<size_t>(valid ? gt : 0) * gk.K + gk.koff[g];
      const double gap = select_group(&logit[tt][g * E], E, gk.kg[g], renorm, idx_out + o, w_out + o, false);
      const bool fix = valid && !(gap > tol);
      redo[task] = fix ? 1 : 0;
      any_fix = any_fix || fix;
      if (valid && !fix) select_group(&logit[tt][g * E], E, gk.kg[g], renorm, idx_out + o, w_out + o, true);
    }
  }
  // most blocks have no flagged pair and end here
  if (__syncthreads_or(any_fix ? 1 : 0) == 0) return;

  // exact recomputation of the flagged pairs: the block's waves take them in
  // turn (the n-th flagged pair goes to wave n mod 4), one wave per pair, 16
  // lanes per expert (4 experts at a time), each lane 8 dims per 16-byte load
  // at a stride of 128 dims, FB loads of each operand issued before their
  // products; float64 products summed lane-sequentially in dimension order,
  // then over the 16 lanes in a fixed butterfly
  constexpr int FB = KS == 1 ? 2 : 4;  // loads in flight, within the kernels' register budgets
  int nth = 0;
  for (int c0 = 0; c0 < tasks; c0 += 64) {
    uint64_t m = __ballot(c0 + lane < tasks && redo[c0 + lane] != 0);
    while (m) {
      const int task = c0 + __builtin_ctzll(m);
      m &= m - 1;
      if ((nth++ & 3) != wave) continue;
      const int tt = task / G, g = task % G;
      const bf16_t* xr = x + static_cast<size_t>(blk0 + tt) * d;
      const int eg = lane >> 4, sl = lane & 15;
      for (int e0 = 0; e0 < E; e0 += 4) {
        const int e = e0 + eg;
        const bf16_t* wrow = wr + static_cast<size_t>(g * E + (e < E ? e : 0)) * d;
        double sacc = 0.0;
        for (int c0d = 8 * sl; c0d < d; c0d += 128 * FB) {
          bf16x8 xv[FB], wv[FB];
#pragma unroll
          for (int u = 0; u < FB; ++u) {
            const int c = c0d + 128 * u;
            xv[u] = c < d ? load_frag(xr + c) : bf16x8{};
            wv[u] = c < d ? load_frag(wrow + c) : bf16x8{};
          }
#pragma unroll
          for (int u = 0; u < FB; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j)  // zero padding past d adds exact zeros
              sacc = fma(static_cast<double>(static_cast<float>(xv[u][j])),
                         static_cast<double>(static_cast<float>(wv[u][j])), sacc);
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) sacc += __shfl_xor(sacc, off, 64);
        if (e < E && sl == 0)
          logit[tt][g * E + e] = sacc + (bias ? static_cast<double>(bias[g * E + e]) : 0.0);
      }
    }
  }
  __syncthreads();
  for (int task = tid; task < tasks; task += 256) {
    if (!redo[task]) continue;
    const int tt = task / G, g = task % G;
    const size_t o = static_cast<size_t>(blk0 + tt) * gk.K + gk.koff[g];
    select_group(&logit[tt][g * E], E, gk.kg[g], renorm, idx_out + o, w_out + o, true);
  }
}

}  // namespace

}  // namespace gqe

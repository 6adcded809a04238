// Backward pass of the GQE layer (and of dense GQA): the gradients of
// <y, dy> + aux_weight * L_aux with respect to x and every weight.
//
// gist.science, Architectuur en Routing and Training en Loss: the discrete
// top-k choice has no gradient, the language-model loss reaches the router
// through the weighted slot, and a load-balancing auxiliary loss spreads each
// group's tokens over its experts.  The pages give no formula for that loss;
// this implements L_aux = (E / G) * sum_g sum_e f[g, e] * P[g, e], with f the
// fraction of the group's routed slots that chose e (a count: no gradient) and
// P the mean in-group router probability.
//
// The forward pass leaves in its workspace what the backward reads: the
// routing (idx, w, counts), the slot-major queries, K, V^T, the slot vectors
// s and the per-row log-sum-exp of the attention scores.  The pass:
//   1. dS = dy . W_O                      (NT GEMM against W_O^T)
//   2. slot backward: per slot head the attention-output gradient dO (the
//      hard slot's own gradient plus w times the weighted slot's), the row
//      sums D = <dO, O>, and the routing-weight gradient dw
//   3. attention backward, FlashAttention-2 style with P formed again from
//      the saved log-sum-exp:
//        attn_bwd_dkdv_kernel  one wave per 32 keys of a group: for every
//                              slot head of the group and every later query
//                              block, dV^T += dO^T P and dK^T += Q^T dS
//        attn_bwd_dq_kernel    one wave per 32 queries of a slot head: for
//                              every earlier key block, dQ^T += K^T dS^T
//      on 32x32x16 MFMA.  P and dS leave the accumulators as B operands
//      directly: their k order (the accumulator's row order) is the key
//      permutation of the V^T tiles, so Q^T, K^T and dO^T are laid out in the
//      same permuted tiles and every A operand is one 16-byte load.
//   4. router backward: logits again in float64; the routing-weight gradient
//      through the softmax over the selected experts (renormalized weights)
//      or over all E (the weighted-concatenation ablation), plus the
//      auxiliary loss's gradient through the in-group softmax
//   5. the gradients of every projection input are laid side by side in one
//      matrix Gall[token, :] = [dQ by expert head | dK | dV | dr], so that
//        dx = Gall . [W_q; W_k; W_v; W_r]      (NT GEMM against the stacked
//                                              weights transposed)
//        dW = Gall^T . x                      (NT GEMM of transposed copies)
//        dW_O = dy^T . s
//      The routed query gradient sits in the column block of the expert the
//      token chose; the other experts' blocks are zero.
#include <math.h>

#include <algorithm>

#include "debug_check.h"
#include "device_common.h"
#include "kernels.h"
#include "routing.h"

namespace gqe {

namespace {

// column of key position p (< 64) in a permuted tile (keys permuted in
// 16-key groups; the map is its own inverse)
__device__ __forceinline__ int tile_col(int p) {
  return (p & ~15) | (p & 3) | ((p & 4) << 1) | ((p & 8) >> 1);
}

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// layout helpers
// ---------------------------------------------------------------------------
// Rotary embedding backward: the attention backward leaves in Gall the
// gradients of the turned queries and keys; the projections need them turned
// back (the transpose of the rotation) at each row's position.  One thread
// per (row, pair of dims) of the query and key column blocks.
template <typename T>
__global__ __launch_bounds__(256) void rope_back_kernel(T* __restrict__ gall, int rows, int ldg,
                                                        int qcols, int kcol, int kcols, int L,
                                                        int D, RopeTable rope) {
  const int pq = qcols / 2, pairs = pq + kcols / 2;
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<size_t>(rows) * pairs) return;
  const int row = static_cast<int>(i / pairs), pr = static_cast<int>(i % pairs);
  const int c = pr < pq ? 2 * pr : 2 * (pr - pq);  // column inside the block
  const int dim = c % D;
  T* gp = gall + static_cast<size_t>(row) * ldg + (pr < pq ? c : kcol + c);
  const float v0 = to_f32(gp[0]), v1 = to_f32(gp[1]);
  float cs, sn;
  rope_cs(row % L, rope.theta[dim >> 1], cs, sn);
  gp[0] = from_f32<T>(rope_apply(v0, v1, dim, cs, sn, true));
  gp[1] = from_f32<T>(rope_apply(v1, v0, dim + 1, cs, sn, true));
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n16) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// dst[c * ldd + dcol + r] = src[r * lds + c] for r < R, c < C, and zero for
// R <= r < Rpad.  64 x 64 tiles through LDS; grid (ceil(C/64), ceil(Rpad/64)).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, int lds_,
                                                        int R, int C, T* __restrict__ dst,
                                                        int ldd, int dcol, int Rpad) {
  __shared__ T tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i / 64, c = i % 64;
    tile[r][c] = (r0 + r < R && c0 + c < C) ? src[static_cast<size_t>(r0 + r) * lds_ + c0 + c]
                                            : from_f32<T>(0.f);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int c = i / 64, r = i % 64;
    if (c0 + c < C && r0 + r < Rpad) dst[static_cast<size_t>(c0 + c) * ldd + dcol + r0 + r] = tile[r][c];
  }
}

// Row-major slabs [R, D] -> permuted tiles [tiles, D, 64] (zero past R).
// Destination slab s reads source slab (s / dst_heads) * src_heads + s % dst_heads.
// Grid (tiles, slabs).
template <typename T>
__global__ __launch_bounds__(256) void to_tiles_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                       int R, int D, int tiles, int src_heads,
                                                       int dst_heads) {
  extern __shared__ float tsm[];
  T* tile = reinterpret_cast<T*>(tsm);  // [64][D + 1]
  const int j = blockIdx.x, s = blockIdx.y;
  const size_t ss = static_cast<size_t>(s / dst_heads) * src_heads + s % dst_heads;
  const T* sp = src + ss * R * D;
  for (int i = threadIdx.x; i < 64 * D; i += 256) {
    const int r = i / D, d = i % D;
    const int key = 64 * j + r;
    tile[r * (D + 1) + d] = key < R ? sp[static_cast<size_t>(key) * D + d] : from_f32<T>(0.f);
  }
  __syncthreads();
  T* dp = dst + (static_cast<size_t>(s) * tiles + j) * D * 64;
  for (int i = threadIdx.x; i < 64 * D; i += 256) {
    const int d = i / 64, c = i % 64;
    dp[d * 64 + c] = tile[tile_col(c) * (D + 1) + d];
  }
}

// Permuted tiles [tiles, D, 64] -> row-major [R, D].  Grid (tiles, slabs).
template <typename T>
__global__ __launch_bounds__(256) void from_tiles_kernel(const T* __restrict__ src,
                                                         T* __restrict__ dst, int R, int D,
                                                         int tiles) {
  extern __shared__ float tsm[];
  T* tile = reinterpret_cast<T*>(tsm);  // [D][65]
  const int j = blockIdx.x, s = blockIdx.y;
  const T* sp = src + (static_cast<size_t>(s) * tiles + j) * D * 64;
  for (int i = threadIdx.x; i < 64 * D; i += 256) {
    const int d = i / 64, c = i % 64;
    tile[d * 65 + c] = sp[d * 64 + c];
  }
  __syncthreads();
  T* dp = dst + static_cast<size_t>(s) * R * D;
  for (int i = threadIdx.x; i < 64 * D; i += 256) {
    const int r = i / D, d = i % D;
    const int key = 64 * j + r;
    if (key < R) dp[static_cast<size_t>(key) * D + d] = tile[d * 65 + tile_col(r)];
  }
}

// ---------------------------------------------------------------------------
// slot backward: one wave per token
// ---------------------------------------------------------------------------
struct SlotBwdArgs {
  const float* ds;   // [T, Ws] gradient of the slot vectors
  const void* s;     // [T, Ws] slot vectors (forward)
  const float* w;    // [T, n_routed] routing weights (p for the weighted concatenation), or NULL
  void* dO;          // [B, H, L, D]
  float* dsum;       // [B, H, L]
  float* dw;         // [T, n_routed] or NULL
  int B, L, H, D, Ws;
  int n_routed;      // slot heads with a routing weight
  int mode;          // 0 full (weighted slot after the shared one), 1 hard, 2 weighted concat, 3 dense
};

template <typename T>
__global__ __launch_bounds__(256) void slot_bwd_kernel(SlotBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= a.B * a.L) return;
  const int b = tok / a.L, t = tok % a.L;
  const float* ds = a.ds + static_cast<size_t>(tok) * a.Ws;
  const T* s = static_cast<const T*>(a.s) + static_cast<size_t>(tok) * a.Ws;
  const int D = a.D;
  const int d0 = lane, d1 = lane + 64;
  float dsw0 = 0.f, dsw1 = 0.f;  // weighted slot's gradient
  if (a.mode == 0) {
    const int wc = (a.n_routed + 1) * D;
    if (d0 < D) dsw0 = ds[wc + d0];
    if (d1 < D) dsw1 = ds[wc + d1];
  }
  for (int h = 0; h < a.H; ++h) {
    const bool routed = h < a.n_routed && a.mode != 3;
    const float wh = routed && a.w != nullptr ? a.w[static_cast<size_t>(tok) * a.n_routed + h] : 1.f;
    float o0 = 0.f, o1 = 0.f, g0 = 0.f, g1 = 0.f;
    if (d0 < D) {
      o0 = to_f32(s[h * D + d0]);
      g0 = ds[h * D + d0];
    }
    if (d1 < D) {
      o1 = to_f32(s[h * D + d1]);
      g1 = ds[h * D + d1];
    }
    float dwv = 0.f;
    if (routed && a.mode == 0) {
      g0 = fmaf(wh, dsw0, g0);
      g1 = fmaf(wh, dsw1, g1);
      dwv = wsum(dsw0 * o0 + dsw1 * o1);
    } else if (routed && a.mode == 2) {
      // the slot holds p * o: the attention output is s / p
      o0 /= wh;
      o1 /= wh;
      dwv = wsum(g0 * o0 + g1 * o1);
      g0 *= wh;
      g1 *= wh;
    }
    // dO in the storage type; the row sum uses the stored values
    T* dO = static_cast<T*>(a.dO) + ((static_cast<size_t>(b) * a.H + h) * a.L + t) * D;
    const T q0 = from_f32<T>(g0), q1 = from_f32<T>(g1);
    if (d0 < D) dO[d0] = q0;
    if (d1 < D) dO[d1] = q1;
    const float dsum = wsum((d0 < D ? to_f32(q0) * o0 : 0.f) + (d1 < D ? to_f32(q1) * o1 : 0.f));
    if (lane == 0) {
      a.dsum[(static_cast<size_t>(b) * a.H + h) * a.L + t] = dsum;
      if (routed && a.dw != nullptr) a.dw[static_cast<size_t>(tok) * a.n_routed + h] = dwv;
    }
  }
}

// ---------------------------------------------------------------------------
// attention backward
// ---------------------------------------------------------------------------
struct AttnBwdArgs {
  const void* q;       // [B, q_heads, L, D] forward queries (unscaled), slot-major
  int q_heads;
  const void* keys;    // [B, G, L, D]
  const void* vr;      // [B, G, L, D] V row-major
  const void* qt;      // [B, H, tiles, D, 64] Q^T, permuted tiles
  const void* kt;      // [B, G, tiles, D, 64] K^T, permuted tiles
  const void* dO;      // [B, H, L, D]
  const void* dOt;     // [B, H, tiles, D, 64]
  const float* lse;    // [B, H, L] (log2 units of the scaled scores)
  const float* dsum;   // [B, H, L]
  void* gall;          // [T, ldg]
  int ldg, kcol, vcol; // dK and dV column blocks (group g at + g*D)
  const int32_t* idx;  // [B*L, n_grouped] experts by slot, or NULL (dense: head h's dQ at column h*D)
  int E;
  int B, G, L, H, tiles;
  int hbeg[kMaxGroups + 1];  // slot heads hbeg[g] .. hbeg[g+1]-1 read group g (hbeg[G] = n_grouped)
  int n_grouped, extra_group;
  float scale, scale_log2;
  // dK/dV with the query walk split over n_split blocks per key block: float
  // partials [n_split, B, G, L, 2*D] (dK unscaled, then dV), summed afterwards
  int n_split;
  float* dkv_part;
  // dQ with the key walk split over n_qsplit blocks per query block: float
  // partials [n_qsplit, B, H, L, D], already scaled, summed afterwards
  int n_qsplit;
  float* dq_part;
  uint32_t* dbg;       // debug word of a debug build's expert-id checks (else unused)
};

// queries scaled by softmax_scale * log2(e) and rounded to the storage type,
// exactly as the forward kernel forms its scores
__device__ __forceinline__ bf16x8 scaled_frag(const bf16_t* p, float sl) {
  const bf16x8 f = load_frag(p);
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = static_cast<__bf16>(static_cast<float>(f[j]) * sl);
  return r;
}
__device__ __forceinline__ f32x8 scaled_frag(const float* p, float sl) { return load_frag(p) * sl; }

template <typename T>
__device__ __forceinline__ typename Frag<T>::type frag_or_zero(const T* p, bool ok) {
  if (ok) return load_frag(p);
  typename Frag<T>::type f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = 0;
  return f;
}

__device__ __forceinline__ int group_of(const AttnBwdArgs& a, int h) {
  if (h >= a.n_grouped) return a.extra_group;
  int g = 0;
  while (a.hbeg[g + 1] <= h) ++g;
  return g;
}

// 32 rows x D (float) in LDS -> rows of Gall, 16 bytes per store
template <typename T, int D>
__device__ __forceinline__ void store_rows(const float* buf, T* gall, int ldg, int lane,
                                           const int* row_of, const int* col_of) {
  constexpr int EPC = 16 / static_cast<int>(sizeof(T));
  for (int c = lane; c < 32 * (D / EPC); c += 64) {
    const int r = c / (D / EPC), e0 = (c % (D / EPC)) * EPC;
    if (row_of[r] < 0) continue;
    T v[EPC];
#pragma unroll
    for (int j = 0; j < EPC; ++j) v[j] = from_f32<T>(buf[r * (D + 1) + e0 + j]);
    *reinterpret_cast<uint4*>(gall + static_cast<size_t>(row_of[r]) * ldg + col_of[r] + e0) =
        *reinterpret_cast<const uint4*>(v);
  }
}

// grid (ceil(L/128), B*G); wave w of a block takes keys 128x + 32w .. +31
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(AttnBwdArgs a) {
  typedef typename Frag<T>::type F;
  constexpr int NKS = D / 16, NDB = D / 32;
  __shared__ float stat[4][2][32];
  __shared__ float obuf[4][32 * (D + 1)];
  __shared__ int rows[4][32], cols[4][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const int b = blockIdx.y / a.G, g = blockIdx.y % a.G;
  const int key0 = blockIdx.x * 128 + 32 * wave;
  if (key0 >= a.L) return;
  const int L = a.L;
  const int my_key = key0 + (lane & 31);
  const int krow = min(my_key, L - 1);
  const T* Kg = static_cast<const T*>(a.keys) + (static_cast<size_t>(b) * a.G + g) * L * D;
  const T* Vg = static_cast<const T*>(a.vr) + (static_cast<size_t>(b) * a.G + g) * L * D;
  F kf[NKS], vf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kf[ks] = load_frag(Kg + static_cast<size_t>(krow) * D + 16 * ks + 8 * half);
    vf[ks] = load_frag(Vg + static_cast<size_t>(krow) * D + 16 * ks + 8 * half);
  }
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

  const int nh0 = a.hbeg[g + 1] - a.hbeg[g];  // this group's routed (or dense) slot heads
  const int nh = nh0 + (g == a.extra_group && a.n_grouped < a.H ? 1 : 0);
  for (int hi = 0; hi < nh; ++hi) {
    const int h = hi < nh0 ? a.hbeg[g] + hi : a.n_grouped;
    const size_t bh = static_cast<size_t>(b) * a.H + h;
    const T* Q = static_cast<const T*>(a.q) + (static_cast<size_t>(b) * a.q_heads + h) * L * D;
    const T* dO = static_cast<const T*>(a.dO) + bh * L * D;
    const T* Qt = static_cast<const T*>(a.qt) + bh * a.tiles * D * 64;
    const T* dOt = static_cast<const T*>(a.dOt) + bh * a.tiles * D * 64;
    const float* lse = a.lse + bh * L;
    const float* dsm = a.dsum + bh * L;
    for (int q0 = key0; q0 < L; q0 += 32) {
      {
        const int qq = q0 + (lane & 31);
        stat[wave][half][lane & 31] = qq < L ? (half == 0 ? lse[qq] : dsm[qq]) : 0.f;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int my_q = q0 + (lane & 31);
      const bool qok = my_q < L;
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const size_t off = static_cast<size_t>(qok ? my_q : 0) * D + 16 * ks + 8 * half;
        F qa = scaled_frag(Q + off, a.scale_log2);
        if (!qok) qa = frag_or_zero<T>(Q, false);
        mma32(s, qa, kf[ks]);
        mma32(dp, frag_or_zero(dO + off, qok), vf[ks]);
      }
      // rows of s/dp: queries q0 + acc_row(i); column: this lane's key
      f32x16 P, dS;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = acc_row(i, lane);
        const int qq = q0 + r;
        const bool keep = qq < L && my_key <= qq;
        const float pv = keep ? __builtin_amdgcn_exp2f(s[i] - stat[wave][0][r]) : 0.f;
        P[i] = pv;
        dS[i] = pv * (dp[i] - stat[wave][1][r]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const size_t tb = static_cast<size_t>(q0 / 64) * D * 64 + (q0 % 64);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const F bp = FragFromAcc<T>::get(P, 8 * m);
        const F bs = FragFromAcc<T>::get(dS, 8 * m);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const size_t toff = tb + static_cast<size_t>(32 * db + (lane & 31)) * 64 + 16 * m + 8 * half;
          mma32(dv[db], load_frag(dOt + toff), bp);
          mma32(dk[db], load_frag(Qt + toff), bs);
        }
      }
    }
  }
  // dK^T, dV^T accumulators: row = dim 32 db + acc_row(i), column = key -> rows of Gall
  float* buf = obuf[wave];
  if (lane < 32) {
    rows[wave][lane] = key0 + lane < L ? b * L + key0 + lane : -1;
    cols[wave][lane] = a.kcol + g * D;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) buf[(lane & 31) * (D + 1) + 32 * db + acc_row(i, lane)] = dk[db][i] * a.scale;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  store_rows<T, D>(buf, static_cast<T*>(a.gall), a.ldg, lane, rows[wave], cols[wave]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < 32) cols[wave][lane] = a.vcol + g * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) buf[(lane & 31) * (D + 1) + 32 * db + acc_row(i, lane)] = dv[db][i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  store_rows<T, D>(buf, static_cast<T*>(a.gall), a.ldg, lane, rows[wave], cols[wave]);
}

// grid (ceil(L/128), B*H); wave w of a block takes queries 128x + 32w .. +31
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(AttnBwdArgs a) {
  typedef typename Frag<T>::type F;
  constexpr int NKS = D / 16, NDB = D / 32;
  __shared__ float obuf[4][32 * (D + 1)];
  __shared__ int rows[4][32], cols[4][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const int b = blockIdx.y / a.H, h = blockIdx.y % a.H;
  const int q0 = blockIdx.x * 128 + 32 * wave;
  if (q0 >= a.L) return;
  const int L = a.L;
  const int g = group_of(a, h);
  const size_t bh = static_cast<size_t>(b) * a.H + h;
  const int my_q = q0 + (lane & 31);
  const bool qok = my_q < L;
  const T* Q = static_cast<const T*>(a.q) + (static_cast<size_t>(b) * a.q_heads + h) * L * D;
  const T* dO = static_cast<const T*>(a.dO) + bh * L * D;
  const T* Kg = static_cast<const T*>(a.keys) + (static_cast<size_t>(b) * a.G + g) * L * D;
  const T* Vg = static_cast<const T*>(a.vr) + (static_cast<size_t>(b) * a.G + g) * L * D;
  const T* Kt = static_cast<const T*>(a.kt) + (static_cast<size_t>(b) * a.G + g) * a.tiles * D * 64;
  const float lse = qok ? a.lse[bh * L + my_q] : 0.f;
  const float dsm = qok ? a.dsum[bh * L + my_q] : 0.f;
  F qf[NKS], df[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const size_t off = static_cast<size_t>(qok ? my_q : 0) * D + 16 * ks + 8 * half;
    qf[ks] = qok ? scaled_frag(Q + off, a.scale_log2) : frag_or_zero<T>(Q, false);
    df[ks] = frag_or_zero(dO + off, qok);
  }
  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;
  const int q_last = min(q0 + 31, L - 1);
  for (int k0 = 0; k0 <= q_last; k0 += 32) {
    const int krow = min(k0 + (lane & 31), L - 1);
    f32x16 st, dpt;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = dpt[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const size_t off = static_cast<size_t>(krow) * D + 16 * ks + 8 * half;
      mma32(st, load_frag(Kg + off), qf[ks]);
      mma32(dpt, load_frag(Vg + off), df[ks]);
    }
    // rows: keys k0 + acc_row(i); column: this lane's query
    f32x16 dS;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = k0 + acc_row(i, lane);
      const bool keep = qok && kk <= my_q;
      const float pv = keep ? __builtin_amdgcn_exp2f(st[i] - lse) : 0.f;
      dS[i] = pv * (dpt[i] - dsm);
    }
    const size_t tb = static_cast<size_t>(k0 / 64) * D * 64 + (k0 % 64);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const F bs = FragFromAcc<T>::get(dS, 8 * m);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        mma32(dq[db], load_frag(Kt + tb + static_cast<size_t>(32 * db + (lane & 31)) * 64 + 16 * m + 8 * half), bs);
    }
  }
  // dQ^T: row = dim, column = query -> the query's expert column block of Gall
  float* buf = obuf[wave];
  if (lane < 32) {
    const int qq = q0 + lane;
    rows[wave][lane] = qq < L ? b * L + qq : -1;
    int col = h * D;
    if (a.idx != nullptr) {
      if (h < a.n_grouped) {
        const int e = qq < L ? a.idx[(static_cast<size_t>(b) * L + qq) * a.n_grouped + h] : 0;
        if (!dbg_ok(e >= 0 && e < a.E, a.dbg, kDbgExpert)) rows[wave][lane] = -1;
        col = (g * a.E + e) * D;
      } else {
        col = a.G * a.E * D;  // the shared head's own W_q rows follow the routed ones
      }
    }
    cols[wave][lane] = col;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) buf[(lane & 31) * (D + 1) + 32 * db + acc_row(i, lane)] = dq[db][i] * a.scale;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  store_rows<T, D>(buf, static_cast<T*>(a.gall), a.ldg, lane, rows[wave], cols[wave]);
}

// ---------------------------------------------------------------------------
// attention backward, bf16: operand tiles shared by the block through LDS
// ---------------------------------------------------------------------------
// The four waves of a block need the same 64-row tiles (the dK/dV kernel: Q,
// dO, Q^T and dO^T of a query block; the dQ kernel: K, V and K^T of a key
// block).  The tiles go straight from global memory into a two-stage LDS
// ring (global_load_lds_dwordx4, swizzled as in the forward kernel), one
// stage ahead of the MFMAs.
template <int D>
struct BwdTiles {
  static constexpr int ROWB = D * 2;              // bytes per row of a row-major tile
  static constexpr int RT = 64 * ROWB;            // 64 rows
  static constexpr int TT = D * 128;              // a [D][64] permuted tile
  static constexpr int RRUNS = RT / 1024, TRUNS = TT / 1024;
  static_assert(RRUNS % 4 == 0 && TRUNS % 4 == 0, "whole runs per wave");
};

// wave w copies runs w, w + 4, ... of a 64-row row-major tile (rows past
// row_lim repeat the last valid row: their results are masked)
template <int D>
__device__ __forceinline__ void dma_rows(const bf16_t* src, int row_lim, char* lds, int wave,
                                         int lane) {
  typedef BwdTiles<D> S;
#pragma unroll
  for (int i = 0; i < S::RRUNS / 4; ++i) {
    const int run = wave + 4 * i;
    const int off = run * 1024 + 16 * lane;
    const int row = off / S::ROWB, pc = (off % S::ROWB) / 16;
    const int lc = pc ^ swz_xor<S::ROWB>(row);
    dma16(src + static_cast<size_t>(min(row, row_lim - 1)) * D + lc * 8, lds + run * 1024);
  }
}
template <int D>
__device__ __forceinline__ void dma_tile(const bf16_t* src, char* lds, int wave, int lane) {
  typedef BwdTiles<D> S;
#pragma unroll
  for (int i = 0; i < S::TRUNS / 4; ++i) {
    const int run = wave + 4 * i;
    const int off = run * 1024 + 16 * lane;
    const int row = off / 128, pc = (off % 128) / 16;
    const int lc = pc ^ swz_xor<128>(row);
    dma16(src + row * 64 + lc * 8, lds + run * 1024);
  }
}

// The dK/dV kernel's blocks are 8 waves (256 keys; 4 waves at d_h 128, whose
// accumulators need all 256 VGPRs): every query tile a block streams serves
// all of them.  Run r of a stage (1 KB) is copied by wave r % waves.
template <int D> struct DkvWaves { static constexpr int n = D >= 128 ? 4 : 8; };

// grid (ceil(L/256), B*G); wave w owns keys 256x + 32w .. +31.  The block
// walks its 64-query blocks from the last one down, and the group's slot heads
// inside each: concurrent blocks of a group then read the same query tiles at
// the same time, which the caches serve once.
// qs: the queries scaled by softmax_scale*log2(e), rounded to bf16, [B, H, L, D].
template <int D>
__global__ __launch_bounds__(64 * DkvWaves<D>::n, 1) void attn_bwd_dkdv_lds_kernel(
    AttnBwdArgs a, const bf16_t* qs) {
  typedef bf16_t T;
  typedef bf16x8 F;
  typedef BwdTiles<D> S;
  constexpr int NW = DkvWaves<D>::n;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int STAGE = 2 * S::RT + 2 * S::TT;
  constexpr int NRUNS = STAGE / 1024;
  static_assert(NRUNS % NW == 0, "whole runs per wave");
  constexpr int DMA_OPS = NRUNS / NW;  // per wave per stage
  extern __shared__ __align__(16) char smem[];
  __shared__ __align__(16) float stat[NW][2][64];
  __shared__ int rows[NW][32], cols[NW][32];
  const int lane = threadIdx.x & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y / a.G, g = blockIdx.y % a.G;
  const int L = a.L;
  const int kb0 = blockIdx.x * 32 * NW, kw0 = kb0 + 32 * wave;
  const int my_key = kw0 + (lane & 31);
  const int krow = min(my_key, L - 1);
  const T* Kg = static_cast<const T*>(a.keys) + (static_cast<size_t>(b) * a.G + g) * L * D;
  const T* Vg = static_cast<const T*>(a.vr) + (static_cast<size_t>(b) * a.G + g) * L * D;
  F kf[NKS], vf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kf[ks] = load_frag(Kg + static_cast<size_t>(krow) * D + 16 * ks + 8 * half);
    vf[ks] = load_frag(Vg + static_cast<size_t>(krow) * D + 16 * ks + 8 * half);
  }
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

  const int nh0 = a.hbeg[g + 1] - a.hbeg[g];  // this group's routed (or dense) slot heads
  const int nh = nh0 + (g == a.extra_group && a.n_grouped < a.H ? 1 : 0);
  const int q_begin = (kb0 / 64) * 64;
  const int nqb = (L - q_begin + 63) / 64;
  const int last_qb = (L - 1) / 64;
  // this block's part of the walk: stages it_beg .. it_beg + n_iter - 1 of nh*nqb
  const int n_all = nh * nqb;
  const int it_beg = static_cast<int>(static_cast<long long>(n_all) * blockIdx.z / a.n_split);
  const int n_iter = static_cast<int>(static_cast<long long>(n_all) * (blockIdx.z + 1) / a.n_split) - it_beg;
  auto head_of = [&](int hi) { return hi < nh0 ? a.hbeg[g] + hi : a.n_grouped; };
  // stage it: query block last_qb - (it_beg + it) / nh, slot head (it_beg + it) % nh
  auto qblk_of = [&](int it) { return 64 * (last_qb - (it_beg + it) / nh); };
  auto issue = [&](int it) {
    const int h = head_of((it_beg + it) % nh), q0 = qblk_of(it);
    const size_t bh = static_cast<size_t>(b) * a.H + h;
    char* st = smem + (it & 1) * STAGE;
    const T* qsrc = qs + (bh * L + q0) * D;
    const T* dsrc = static_cast<const T*>(a.dO) + (bh * L + q0) * D;
    const size_t tb = (bh * a.tiles + q0 / 64) * D * 64;
    const T* tq = static_cast<const T*>(a.qt) + tb;
    const T* td = static_cast<const T*>(a.dOt) + tb;
#pragma unroll
    for (int i = 0; i < DMA_OPS; ++i) {
      const int run = wave + NW * i;  // wave-uniform
      const int off = run * 1024 + 16 * lane;
      const T* src;
      if (run < 2 * S::RRUNS) {  // Q or dO rows
        const int o = off % S::RT;
        const int row = o / S::ROWB, lc = ((o % S::ROWB) / 16) ^ swz_xor<S::ROWB>(row);
        src = (run < S::RRUNS ? qsrc : dsrc) + static_cast<size_t>(min(row, L - q0 - 1)) * D + lc * 8;
      } else {  // Q^T or dO^T tile
        const int o = (off - 2 * S::RT) % S::TT;
        const int row = o / 128, lc = ((o % 128) / 16) ^ swz_xor<128>(row);
        src = (run < 2 * S::RRUNS + S::TRUNS ? tq : td) + row * 64 + lc * 8;
      }
      dma16(src, st + run * 1024);
    }
  };
  auto load_stats = [&](int it, float& ls, float& ds_) {
    const int h = head_of((it_beg + it) % nh), q = qblk_of(it) + lane;
    const size_t bh = static_cast<size_t>(b) * a.H + h;
    ls = q < L ? a.lse[bh * L + q] : 0.f;
    ds_ = q < L ? a.dsum[bh * L + q] : 0.f;
  };

  float ls_cur = 0.f, ds_cur = 0.f;
  if (n_iter > 0) {
    issue(0);
    load_stats(0, ls_cur, ds_cur);
  }
  for (int it = 0; it < n_iter; ++it) {
    float ls_nxt = 0.f, ds_nxt = 0.f;
    const bool more = it + 1 < n_iter;
    if (more) {
      issue(it + 1);
      load_stats(it + 1, ls_nxt, ds_nxt);
    }
    // this stage's copies and statistics are in; the next stage's are in flight
    wait_vm(more ? DMA_OPS + 2 : 0);
    stat[wave][0][lane] = ls_cur;
    stat[wave][1][lane] = ds_cur;
    __builtin_amdgcn_s_barrier();  // every wave's copies of this stage have landed
    __builtin_amdgcn_sched_barrier(0);
    const char* st = smem + (it & 1) * STAGE;
    const char* sQ = st;
    const char* sdO = st + S::RT;
    const char* sQt = st + 2 * S::RT;
    const char* sdOt = sQt + S::TT;
    const int q0 = qblk_of(it);
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
      const int qs0 = q0 + 32 * m2;
      if (kw0 >= L || qs0 + 31 < kw0 || qs0 >= L) continue;  // wave-uniform: all masked
      f32x16 sc, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = dp[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        mma32(sc, LdsFrag<T, S::ROWB>::get(sQ, 32 * m2 + (lane & 31), 16 * ks + 8 * half), kf[ks]);
        mma32(dp, LdsFrag<T, S::ROWB>::get(sdO, 32 * m2 + (lane & 31), 16 * ks + 8 * half), vf[ks]);
      }
      // the rows' statistics, four consecutive rows per read; P is formed for
      // every entry and the masked ones are selected away afterwards, so the
      // loop has no branches (a masked entry's exp2 may overflow: it is dropped)
      float lsr[16], dsr[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int r0 = 32 * m2 + 8 * q4 + 4 * half;
        const float4 l4 = *reinterpret_cast<const float4*>(&stat[wave][0][r0]);
        const float4 d4 = *reinterpret_cast<const float4*>(&stat[wave][1][r0]);
        lsr[4 * q4 + 0] = l4.x; lsr[4 * q4 + 1] = l4.y; lsr[4 * q4 + 2] = l4.z; lsr[4 * q4 + 3] = l4.w;
        dsr[4 * q4 + 0] = d4.x; dsr[4 * q4 + 1] = d4.y; dsr[4 * q4 + 2] = d4.z; dsr[4 * q4 + 3] = d4.w;
      }
      f32x16 P, dS;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qq = q0 + 32 * m2 + acc_row(i, lane);
        const bool keep = qq < L && my_key <= qq;
        const float pv = __builtin_amdgcn_exp2f(sc[i] - lsr[i]);
        P[i] = keep ? pv : 0.f;
        dS[i] = P[i] * (dp[i] - dsr[i]);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const F bp = FragFromAcc<T>::get(P, 8 * m);
        const F bs = FragFromAcc<T>::get(dS, 8 * m);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int row = 32 * db + (lane & 31), col = 32 * m2 + 16 * m + 8 * half;
          mma32(dv[db], LdsFrag<T, 128>::get(sdOt, row, col), bp);
          mma32(dk[db], LdsFrag<T, 128>::get(sQt, row, col), bs);
        }
      }
    }
    ls_cur = ls_nxt;
    ds_cur = ds_nxt;
    lds_barrier();  // every wave is done with this stage before it is refilled
  }
  if (kw0 >= L) return;
  if (a.n_split > 1) {  // float partials of this part of the walk: key (lane & 31), dims by acc_row
    if (my_key < L) {
      float* pp = a.dkv_part +
                  ((static_cast<size_t>(blockIdx.z) * a.B * a.G + blockIdx.y) * L + my_key) * (2 * D);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pp[32 * db + acc_row(i, lane)] = dk[db][i];
          pp[D + 32 * db + acc_row(i, lane)] = dv[db][i];
        }
    }
    return;
  }
  // dK^T, dV^T: row = dim, column = key -> rows of Gall, through this wave's
  // part of the (now free) ring
  float* buf = reinterpret_cast<float*>(smem) + wave * 32 * (D + 1);
  if (lane < 32) {
    rows[wave][lane] = kw0 + lane < L ? b * L + kw0 + lane : -1;
    cols[wave][lane] = a.kcol + g * D;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) buf[(lane & 31) * (D + 1) + 32 * db + acc_row(i, lane)] = dk[db][i] * a.scale;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  store_rows<T, D>(buf, static_cast<T*>(a.gall), a.ldg, lane, rows[wave], cols[wave]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < 32) cols[wave][lane] = a.vcol + g * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) buf[(lane & 31) * (D + 1) + 32 * db + acc_row(i, lane)] = dv[db][i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  store_rows<T, D>(buf, static_cast<T*>(a.gall), a.ldg, lane, rows[wave], cols[wave]);
}

// dK, dV of the split walk: the n_split float partials of (b, g, key) summed
// in split order, dK scaled, both rounded once into Gall.  One thread per
// 8 consecutive dims of one key.
template <typename T, int D>
__global__ __launch_bounds__(256) void dkv_reduce_kernel(AttnBwdArgs a) {
  constexpr int C8 = 2 * D / 8;  // 8-column chunks of a key's [dK | dV] row
  const size_t n = static_cast<size_t>(a.B) * a.G * a.L * C8;
  const size_t id = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (id >= n) return;
  const int c8 = static_cast<int>(id % C8);
  const size_t bgk = id / C8;  // (b*G + g)*L + key
  const int key = static_cast<int>(bgk % a.L);
  const int bg = static_cast<int>(bgk / a.L);
  const int b = bg / a.G, g = bg % a.G;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  const size_t stride = static_cast<size_t>(a.B) * a.G * a.L * 2 * D;
  const float* src = a.dkv_part + bgk * 2 * D + 8 * c8;
  for (int sp = 0; sp < a.n_split; ++sp) {
    const float4 lo = *reinterpret_cast<const float4*>(src + sp * stride);
    const float4 hi = *reinterpret_cast<const float4*>(src + sp * stride + 4);
    acc[0] += lo.x; acc[1] += lo.y; acc[2] += lo.z; acc[3] += lo.w;
    acc[4] += hi.x; acc[5] += hi.y; acc[6] += hi.z; acc[7] += hi.w;
  }
  const bool is_k = 8 * c8 < D;
  const float f = is_k ? a.scale : 1.f;
  T v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = from_f32<T>(acc[j] * f);
  const int col = (is_k ? a.kcol : a.vcol) + g * D + (8 * c8) % D;
  T* dst = static_cast<T*>(a.gall) + (static_cast<size_t>(b) * a.L + key) * a.ldg + col;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(v);
}

// dQ of the split walk: the n_qsplit float partials of (b, h, query) summed
// in split order and rounded once into the query's column block of Gall.
// One thread per 8 consecutive dims of one query.
template <typename T, int D>
__global__ __launch_bounds__(256) void dq_reduce_kernel(AttnBwdArgs a) {
  constexpr int C8 = D / 8;
  const size_t n = static_cast<size_t>(a.B) * a.H * a.L * C8;
  const size_t id = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (id >= n) return;
  const int c8 = static_cast<int>(id % C8);
  const size_t bhq = id / C8;  // (b*H + h)*L + query
  const int q = static_cast<int>(bhq % a.L);
  const int bh = static_cast<int>(bhq / a.L);
  const int b = bh / a.H, h = bh % a.H;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  const size_t stride = static_cast<size_t>(a.B) * a.H * a.L * D;
  const float* src = a.dq_part + bhq * D + 8 * c8;
  for (int sp = 0; sp < a.n_qsplit; ++sp) {
    const float4 lo = *reinterpret_cast<const float4*>(src + sp * stride);
    const float4 hi = *reinterpret_cast<const float4*>(src + sp * stride + 4);
    acc[0] += lo.x; acc[1] += lo.y; acc[2] += lo.z; acc[3] += lo.w;
    acc[4] += hi.x; acc[5] += hi.y; acc[6] += hi.z; acc[7] += hi.w;
  }
  int col = h * D;  // the dense baseline: head h's own block
  if (a.idx != nullptr) {
    if (h < a.n_grouped) {
      const int e = a.idx[(static_cast<size_t>(b) * a.L + q) * a.n_grouped + h];
      if (!dbg_ok(e >= 0 && e < a.E, a.dbg, kDbgExpert)) return;
      col = (group_of(a, h) * a.E + e) * D;
    } else {
      col = a.G * a.E * D;
    }
  }
  T v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = from_f32<T>(acc[j]);
  T* dst = static_cast<T*>(a.gall) + (static_cast<size_t>(b) * a.L + q) * a.ldg + col + 8 * c8;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(v);
}

// grid (ceil(L/128), B*H, n_qsplit); wave w owns queries 128x + 32w .. +31;
// the block walks (its share of) the 64-key blocks up to its last query.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_lds_kernel(AttnBwdArgs a, const bf16_t* qs) {
  typedef bf16_t T;
  typedef bf16x8 F;
  typedef BwdTiles<D> S;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int STAGE = 2 * S::RT + S::TT;
  constexpr int DMA_OPS = 2 * (S::RRUNS / 4) + S::TRUNS / 4;
  extern __shared__ __align__(16) char smem[];
  __shared__ int rows[4][32], cols[4][32];
  const int lane = threadIdx.x & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y / a.H, h = blockIdx.y % a.H;
  const int L = a.L;
  const int g = group_of(a, h);
  const size_t bh = static_cast<size_t>(b) * a.H + h;
  const int qb0 = blockIdx.x * 128, qw0 = qb0 + 32 * wave;
  const int my_q = qw0 + (lane & 31);
  const bool qok = my_q < L;
  const T* dO = static_cast<const T*>(a.dO) + bh * L * D;
  const T* Kg = static_cast<const T*>(a.keys) + (static_cast<size_t>(b) * a.G + g) * L * D;
  const T* Vg = static_cast<const T*>(a.vr) + (static_cast<size_t>(b) * a.G + g) * L * D;
  const T* Kt = static_cast<const T*>(a.kt) + (static_cast<size_t>(b) * a.G + g) * a.tiles * D * 64;
  const float lse = qok ? a.lse[bh * L + my_q] : 0.f;
  const float dsm = qok ? a.dsum[bh * L + my_q] : 0.f;
  F qf[NKS], df[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const size_t off = static_cast<size_t>(qok ? my_q : 0) * D + 16 * ks + 8 * half;
    qf[ks] = frag_or_zero(qs + bh * L * D + off, qok);
    df[ks] = frag_or_zero(dO + off, qok);
  }
  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;
  // key blocks up to the block's last query; split z of n_qsplit walks its
  // contiguous share of them
  const int n_all = (min(qb0 + 128, L) + 63) / 64;
  const int it_beg = n_all * static_cast<int>(blockIdx.z) / a.n_qsplit;
  const int it_end = n_all * (static_cast<int>(blockIdx.z) + 1) / a.n_qsplit;
  const int w_last = min(qw0 + 31, L - 1);
  auto issue = [&](int it) {
    const int k0 = 64 * it;
    char* st = smem + (it & 1) * STAGE;
    dma_rows<D>(Kg + static_cast<size_t>(k0) * D, L - k0, st, wave, lane);
    dma_rows<D>(Vg + static_cast<size_t>(k0) * D, L - k0, st + S::RT, wave, lane);
    dma_tile<D>(Kt + static_cast<size_t>(it) * D * 64, st + 2 * S::RT, wave, lane);
  };
  if (it_beg < it_end) issue(it_beg);
  for (int it = it_beg; it < it_end; ++it) {
    const bool more = it + 1 < it_end;
    if (more) issue(it + 1);
    dma_barrier(more ? DMA_OPS : 0);
    const char* st = smem + (it & 1) * STAGE;
    const char* sK = st;
    const char* sV = st + S::RT;
    const char* sKt = st + 2 * S::RT;
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
      const int ks0 = 64 * it + 32 * m2;
      if (qw0 >= L || ks0 > w_last) continue;  // wave-uniform: every key after every query
      f32x16 stt, dpt;
#pragma unroll
      for (int i = 0; i < 16; ++i) stt[i] = dpt[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        mma32(stt, LdsFrag<T, S::ROWB>::get(sK, 32 * m2 + (lane & 31), 16 * ks + 8 * half), qf[ks]);
        mma32(dpt, LdsFrag<T, S::ROWB>::get(sV, 32 * m2 + (lane & 31), 16 * ks + 8 * half), df[ks]);
      }
      f32x16 dS;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = ks0 + acc_row(i, lane);
        const bool keep = qok && kk <= my_q;
        const float pv = keep ? __builtin_amdgcn_exp2f(stt[i] - lse) : 0.f;
        dS[i] = pv * (dpt[i] - dsm);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const F bs = FragFromAcc<T>::get(dS, 8 * m);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          mma32(dq[db], LdsFrag<T, 128>::get(sKt, 32 * db + (lane & 31), 32 * m2 + 16 * m + 8 * half), bs);
      }
    }
    lds_barrier();  // every wave is done with this stage before it is refilled
  }
  if (qw0 >= L) return;
  if (a.n_qsplit > 1) {  // float partials: query (lane & 31), 4 consecutive dims per store
    if (!qok) return;
    float* pp = a.dq_part + ((static_cast<size_t>(blockIdx.z) * a.B * a.H + bh) * L + my_q) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 4)
        *reinterpret_cast<float4*>(pp + 32 * db + acc_row(i, lane)) =
            make_float4(dq[db][i] * a.scale, dq[db][i + 1] * a.scale, dq[db][i + 2] * a.scale,
                        dq[db][i + 3] * a.scale);
    return;
  }
  float* buf = reinterpret_cast<float*>(smem) + wave * 32 * (D + 1);
  if (lane < 32) {
    const int qq = qw0 + lane;
    rows[wave][lane] = qq < L ? b * L + qq : -1;
    int col = h * D;
    if (a.idx != nullptr) {
      if (h < a.n_grouped) {
        const int e = qq < L ? a.idx[(static_cast<size_t>(b) * L + qq) * a.n_grouped + h] : 0;
        if (!dbg_ok(e >= 0 && e < a.E, a.dbg, kDbgExpert)) rows[wave][lane] = -1;
        col = (g * a.E + e) * D;
      } else {
        col = a.G * a.E * D;
      }
    }
    cols[wave][lane] = col;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) buf[(lane & 31) * (D + 1) + 32 * db + acc_row(i, lane)] = dq[db][i] * a.scale;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  store_rows<T, D>(buf, static_cast<T*>(a.gall), a.ldg, lane, rows[wave], cols[wave]);
}

// queries scaled by softmax_scale * log2(e), rounded to bf16: dst slab s reads
// source slab (s / H) * q_heads + s % H
__global__ __launch_bounds__(256) void scale_rows_kernel(const bf16_t* __restrict__ src,
                                                         bf16_t* __restrict__ dst, size_t n,
                                                         size_t slab, int H, int q_heads,
                                                         float sl) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * 256) {
    const size_t s = i / slab, e = i % slab;
    const size_t src_s = (s / H) * q_heads + s % H;
    dst[i] = from_f32<bf16_t>(to_f32(src[src_s * slab + e]) * sl);
  }
}

template <int D>
hipError_t launch_attn_bwd_lds(const AttnBwdArgs& a, const bf16_t* qs, hipStream_t stream) {
  typedef BwdTiles<D> S;
  // the ring, or the epilogue's per-wave transposes if they need more
  constexpr int NW = DkvWaves<D>::n;
  constexpr int ring_kv = 2 * (2 * S::RT + 2 * S::TT), tr_kv = NW * 32 * (D + 1) * 4;
  constexpr int lds_kv = ring_kv > tr_kv ? ring_kv : tr_kv;
  constexpr int lds_q = 2 * (2 * S::RT + S::TT);
  static_assert(lds_q >= 4 * 32 * (D + 1) * 4, "the ring holds the epilogue's transposes");
  static_assert(lds_kv <= 160 * 1024 - 8 * 1024, "LDS of one CU");
  static const hipError_t attr1 = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&attn_bwd_dkdv_lds_kernel<D>),
      hipFuncAttributeMaxDynamicSharedMemorySize, lds_kv);
  static const hipError_t attr2 = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&attn_bwd_dq_lds_kernel<D>),
      hipFuncAttributeMaxDynamicSharedMemorySize, lds_q);
  if (attr1 != hipSuccess) return attr1;
  if (attr2 != hipSuccess) return attr2;
  hipLaunchKernelGGL((attn_bwd_dkdv_lds_kernel<D>),
                     dim3((a.L + 32 * NW - 1) / (32 * NW), a.B * a.G, a.n_split), dim3(64 * NW),
                     lds_kv, stream, a, qs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.n_split > 1) {
    const size_t n = static_cast<size_t>(a.B) * a.G * a.L * (2 * D / 8);
    hipLaunchKernelGGL((dkv_reduce_kernel<bf16_t, D>), dim3(static_cast<unsigned>((n + 255) / 256)),
                       dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((attn_bwd_dq_lds_kernel<D>), dim3((a.L + 127) / 128, a.B * a.H, a.n_qsplit),
                     dim3(256), lds_q, stream, a, qs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.n_qsplit > 1) {
    const size_t n = static_cast<size_t>(a.B) * a.H * a.L * (D / 8);
    hipLaunchKernelGGL((dq_reduce_kernel<bf16_t, D>), dim3(static_cast<unsigned>((n + 255) / 256)),
                       dim3(256), 0, stream, a);
    e = hipGetLastError();
  }
  return e;
}

// ---------------------------------------------------------------------------
// router backward: one block per token
// ---------------------------------------------------------------------------
struct RouterBwdArgs {
  const void* x;
  const void* wr;
  const float* bias;
  const int32_t* idx;     // [T, K] experts by slot (group g at koff[g])
  const float* dw;        // [T, K] routing-weight gradient (NULL: none)
  const int32_t* counts;  // [B, G, E] forward dispatch counts
  void* gall;             // dr at columns rcol + g*E + e
  int ldg, rcol;
  float* dr;              // [T, G*E] float copy
  float* p_out;           // [T, G*E] in-group probabilities
  int B, T, d, G, E;
  GroupK gk;              // experts selected per group and their slot offsets
  int mode;               // 0 full (renormalized weights), 1 hard, 2 weighted concatenation
  float aux_weight;
  uint32_t* dbg;          // debug word of a debug build's expert-id checks (else unused)
};

template <typename T>
__global__ __launch_bounds__(256) void router_bwd_kernel(RouterBwdArgs a) {
  __shared__ double logit[64], pr[64], dpv[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;
  const int GE = a.G * a.E;
  constexpr int kU4 = U4Count<T>::n;
  const T* xp = static_cast<const T*>(a.x) + static_cast<size_t>(t) * a.d;
  for (int e = wave; e < GE; e += 4) {
    const T* wp = static_cast<const T*>(a.wr) + static_cast<size_t>(e) * a.d;
    double acc = 0.0;
    for (int d0 = 8 * lane; d0 < a.d; d0 += 512) {
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
    if (lane == 0) logit[e] = acc + (a.bias ? static_cast<double>(a.bias[e]) : 0.0);
  }
  __syncthreads();
  if (tid < GE) {  // in-group softmax p over all E
    const int g = tid / a.E;
    const double* r = &logit[g * a.E];
    double rmax = r[0];
    for (int f = 1; f < a.E; ++f) rmax = fmax(rmax, r[f]);
    double z = 0.0;
    for (int f = 0; f < a.E; ++f) z += exp(r[f] - rmax);
    pr[tid] = exp(logit[tid] - rmax) / z;
    dpv[tid] = 0.0;
  }
  __syncthreads();
  // gradient on p (aux) and on the selected weights
  if (tid < a.G) {
    const int g = tid;
    const int k = a.gk.kg[g];
    const size_t so = static_cast<size_t>(t) * a.gk.K + a.gk.koff[g];  // group g's slots of token t
    const int32_t* id = a.idx + so;
    double* dp = &dpv[g * a.E];
    const double* p = &pr[g * a.E];
    double grad[64];
    for (int e = 0; e < a.E; ++e) grad[e] = 0.0;
    if (a.aux_weight != 0.f) {
      // dL/dp[t, g, e] = aux_weight * (E / G) * f[g, e] / T
      for (int e = 0; e < a.E; ++e) {
        long long c = 0;
        for (int bb = 0; bb < a.B; ++bb) c += a.counts[(static_cast<size_t>(bb) * a.G + g) * a.E + e];
        const double f = static_cast<double>(c) / (static_cast<double>(a.T) * k);
        dp[e] = static_cast<double>(a.aux_weight) * a.E / a.G * f / a.T;
      }
      double sdp = 0.0;
      for (int e = 0; e < a.E; ++e) sdp += p[e] * dp[e];
      for (int e = 0; e < a.E; ++e) grad[e] += p[e] * (dp[e] - sdp);
    }
    bool ids_ok = true;
#ifdef GQE_DEBUG
    for (int j = 0; j < k; ++j) ids_ok = ids_ok && id[j] >= 0 && id[j] < a.E;
    ids_ok = dbg_ok(ids_ok, a.dbg, kDbgExpert);
#endif
    if (a.dw != nullptr && a.mode == 0 && ids_ok) {
      // w = softmax over the selected logits: dr_j = w_j (dw_j - sum w dw)
      double ws[64], z = 0.0, rmax = logit[g * a.E + id[0]];
      for (int j = 0; j < k; ++j) rmax = fmax(rmax, logit[g * a.E + id[j]]);
      for (int j = 0; j < k; ++j) z += (ws[j] = exp(logit[g * a.E + id[j]] - rmax));
      double s = 0.0;
      for (int j = 0; j < k; ++j) {
        ws[j] /= z;
        s += ws[j] * a.dw[so + j];
      }
      for (int j = 0; j < k; ++j) grad[id[j]] += ws[j] * (a.dw[so + j] - s);
    } else if (a.dw != nullptr && a.mode == 2 && ids_ok) {
      // the selected experts' p scale their slots: softmax over all E
      double dps[64];
      for (int e = 0; e < a.E; ++e) dps[e] = 0.0;
      for (int j = 0; j < k; ++j) dps[id[j]] = a.dw[so + j];
      double s = 0.0;
      for (int e = 0; e < a.E; ++e) s += p[e] * dps[e];
      for (int e = 0; e < a.E; ++e) grad[e] += p[e] * (dps[e] - s);
    }
    for (int e = 0; e < a.E; ++e) {
      const size_t o = static_cast<size_t>(t) * GE + g * a.E + e;
      a.dr[o] = static_cast<float>(grad[e]);
      a.p_out[o] = static_cast<float>(p[e]);
      static_cast<T*>(a.gall)[static_cast<size_t>(t) * a.ldg + a.rcol + g * a.E + e] =
          from_f32<T>(static_cast<float>(grad[e]));
    }
  }
}

// Column sums over T rows in a fixed order: block c sums column c of dr (into
// dbr) and of p (into psum, for the auxiliary loss).
__global__ __launch_bounds__(256) void column_sums_kernel(const float* dr, const float* p, int T,
                                                          int C, float* dbr, double* psum) {
  __shared__ double s1[256], s2[256];
  const int c = blockIdx.x;
  double a = 0.0, q = 0.0;
  for (int t = threadIdx.x; t < T; t += 256) {
    a += dr[static_cast<size_t>(t) * C + c];
    q += p[static_cast<size_t>(t) * C + c];
  }
  s1[threadIdx.x] = a;
  s2[threadIdx.x] = q;
  __syncthreads();
  for (int n = 128; n >= 1; n >>= 1) {
    if (threadIdx.x < n) {
      s1[threadIdx.x] += s1[threadIdx.x + n];
      s2[threadIdx.x] += s2[threadIdx.x + n];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    dbr[c] = static_cast<float>(s1[0]);
    psum[c] = s2[0];
  }
}

// L_aux = (E / G) * sum_{g,e} f[g, e] * P[g, e], f[g, e] the share of group
// g's T*k_g routed slots that went to expert e
__global__ void aux_loss_kernel(const double* psum, const int32_t* counts, int B, int T, int G,
                                int E, GroupK gk, float* out) {
  if (threadIdx.x != 0) return;
  double acc = 0.0;
  for (int g = 0; g < G; ++g)
    for (int e = 0; e < E; ++e) {
      long long c = 0;
      for (int bb = 0; bb < B; ++bb) c += counts[(static_cast<size_t>(bb) * G + g) * E + e];
      acc += (static_cast<double>(c) / (static_cast<double>(T) * gk.kg[g])) * (psum[g * E + e] / T);
    }
  *out = static_cast<float>(acc * E / G);
}

template <typename T>
hipError_t launch_transpose(const T* src, int lds_, int R, int C, T* dst, int ldd, int dcol,
                            int Rpad, hipStream_t stream) {
  if (C == 0 || Rpad == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_kernel<T>, dim3((C + 63) / 64, (Rpad + 63) / 64), dim3(256), 0,
                     stream, src, lds_, R, C, dst, ldd, dcol, Rpad);
  return hipGetLastError();
}

hipError_t launch_fill(void* p, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>(std::min<size_t>((n16 + 255) / 256, 8192));
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<uint4*>(p),
                     n16);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_attn_bwd_d(const AttnBwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D>), dim3((a.L + 127) / 128, a.B * a.G), dim3(256),
                     0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D>), dim3((a.L + 127) / 128, a.B * a.H), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

int dkdv_splits(int B, int G, int L, int D) {
  // bf16 dK/dV blocks of 256 keys (128 at d_h 128): below one block per
  // compute unit, the query walk of each key block is split so that the
  // blocks cover the chip
  const int keys = D >= 128 ? 128 : 256;
  const long long blocks = static_cast<long long>((L + keys - 1) / keys) * B * G;
  if (blocks <= 0 || blocks >= cu_count()) return 1;
  return static_cast<int>(std::min<long long>(8, (cu_count() + blocks - 1) / blocks));
}

int dq_splits(int B, int H, int L) {
  // bf16 dQ blocks of 128 queries, two per compute unit: below one block per
  // compute unit, each block's key walk is split so that the blocks fill
  // both slots of every unit (the longest walk, the last query block's,
  // shrinks by the same factor)
  const long long blocks = static_cast<long long>((L + 127) / 128) * B * H;
  if (blocks <= 0 || blocks >= cu_count()) return 1;
  return static_cast<int>(std::max<long long>(1, std::min<long long>(4, 2LL * cu_count() / blocks)));
}

template <typename T>
hipError_t launch_backward(const BwdParams& p, hipStream_t stream) {
  const int B = p.B, L = p.L, T_ = p.B * p.L, d = p.d, G = p.G, E = p.E, D = p.D;
  const int H = p.H;
  hipError_t e;
#define GQE_TRY(x)                     \
  do {                                 \
    if ((e = (x)) != hipSuccess) return e; \
  } while (0)
  const size_t es = sizeof(T);
  // layouts: Gall and the stacked weights transposed (zero outside the
  // blocks), W_O transposed
  GQE_TRY(launch_fill(p.gall, static_cast<size_t>(T_) * p.kpad * es, stream));
  GQE_TRY(launch_fill(p.w_t, static_cast<size_t>(d) * p.kpad * es, stream));
  GQE_TRY(launch_transpose<T>(static_cast<const T*>(p.wq), d, p.qcols, d, static_cast<T*>(p.w_t),
                              p.kpad, 0, p.qcols, stream));
  GQE_TRY(launch_transpose<T>(static_cast<const T*>(p.wk), d, G * D, d, static_cast<T*>(p.w_t),
                              p.kpad, p.kcol, G * D, stream));
  GQE_TRY(launch_transpose<T>(static_cast<const T*>(p.wv), d, G * D, d, static_cast<T*>(p.w_t),
                              p.kpad, p.vcol, G * D, stream));
  if (p.wr != nullptr)
    GQE_TRY(launch_transpose<T>(static_cast<const T*>(p.wr), d, G * E, d, static_cast<T*>(p.w_t),
                                p.kpad, p.rcol, G * E, stream));
  GQE_TRY(launch_transpose<T>(static_cast<const T*>(p.wo), p.ws, d, p.ws, static_cast<T*>(p.wo_t),
                              d, 0, d, stream));

  // 1. dS = dy . W_O
  {
    NtArgs g = {};
    g.a = p.dy;
    g.lda = d;
    g.b = p.wo_t;
    g.ldb = d;
    g.M = T_;
    g.N = p.ws;
    g.K = d;
    g.nseg = 1;
    g.seg[0] = NtSeg{p.ds, 0, T_, p.ws, 0};
    GQE_TRY(launch_nt_gemm<T>(g, stream));
  }
  // 2. slot backward
  {
    SlotBwdArgs s;
    s.ds = p.ds;
    s.s = p.s;
    s.w = p.w;
    s.dO = p.dO;
    s.dsum = p.dsum;
    s.dw = p.dw;
    s.B = B;
    s.L = L;
    s.H = H;
    s.D = D;
    s.Ws = p.ws;
    s.n_routed = p.n_routed;
    s.mode = p.mode;
    hipLaunchKernelGGL(slot_bwd_kernel<T>, dim3((T_ + 3) / 4), dim3(256), 0, stream, s);
    GQE_TRY(hipGetLastError());
  }
  // 3. attention backward
  const int tiles = (L + 63) / 64;
  {
    const size_t tl = 64 * (D + 1) * es;
    hipLaunchKernelGGL(to_tiles_kernel<T>, dim3(tiles, B * H), dim3(256), tl, stream,
                       static_cast<const T*>(p.q), static_cast<T*>(p.qt), L, D, tiles, p.q_heads, H);
    GQE_TRY(hipGetLastError());
    hipLaunchKernelGGL(to_tiles_kernel<T>, dim3(tiles, B * G), dim3(256), tl, stream,
                       static_cast<const T*>(p.keys), static_cast<T*>(p.kt), L, D, tiles, G, G);
    GQE_TRY(hipGetLastError());
    hipLaunchKernelGGL(to_tiles_kernel<T>, dim3(tiles, B * H), dim3(256), tl, stream,
                       static_cast<const T*>(p.dO), static_cast<T*>(p.dOt), L, D, tiles, H, H);
    GQE_TRY(hipGetLastError());
    hipLaunchKernelGGL(from_tiles_kernel<T>, dim3(tiles, B * G), dim3(256), D * 65 * es, stream,
                       static_cast<const T*>(p.vt), static_cast<T*>(p.vr), L, D,
                       static_cast<int>(p.vt_tiles));
    GQE_TRY(hipGetLastError());
    AttnBwdArgs a;
    a.q = p.q;
    a.q_heads = p.q_heads;
    a.keys = p.keys;
    a.vr = p.vr;
    a.qt = p.qt;
    a.kt = p.kt;
    a.dO = p.dO;
    a.dOt = p.dOt;
    a.lse = p.lse;
    a.dsum = p.dsum;
    a.gall = p.gall;
    a.ldg = p.kpad;
    a.kcol = p.kcol;
    a.vcol = p.vcol;
    a.idx = p.idx;
    a.dbg = p.dbg;
    a.E = E;
    a.B = B;
    a.G = G;
    a.L = L;
    a.H = H;
    a.tiles = tiles;
    for (int g = 0; g <= G; ++g) a.hbeg[g] = p.hbeg[g];
    a.n_grouped = p.n_grouped;
    a.n_split = sizeof(T) == 2 ? p.dkv_split : 1;
    a.dkv_part = p.dkv_part;
    a.n_qsplit = sizeof(T) == 2 ? p.dq_split : 1;
    a.dq_part = p.dq_part;
    a.extra_group = p.extra_group;
    a.scale = p.scale;
    a.scale_log2 = p.scale * 1.4426950408889634f;
    if constexpr (sizeof(T) == 2) {
      // queries pre-scaled as the forward kernel scores them
      const size_t n = static_cast<size_t>(B) * H * L * D;
      const unsigned blocks = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 16384));
      hipLaunchKernelGGL(scale_rows_kernel, dim3(blocks), dim3(256), 0, stream,
                         static_cast<const bf16_t*>(p.q), static_cast<bf16_t*>(p.qs), n,
                         static_cast<size_t>(L) * D, H, p.q_heads, a.scale_log2);
      GQE_TRY(hipGetLastError());
      const bf16_t* qs = static_cast<const bf16_t*>(p.qs);
      switch (D) {
        case 32: GQE_TRY(launch_attn_bwd_lds<32>(a, qs, stream)); break;
        case 64: GQE_TRY(launch_attn_bwd_lds<64>(a, qs, stream)); break;
        case 128: GQE_TRY(launch_attn_bwd_lds<128>(a, qs, stream)); break;
        default: return hipErrorInvalidValue;
      }
    } else {
      switch (D) {
        case 32: GQE_TRY((launch_attn_bwd_d<T, 32>(a, stream))); break;
        case 64: GQE_TRY((launch_attn_bwd_d<T, 64>(a, stream))); break;
        case 128: GQE_TRY((launch_attn_bwd_d<T, 128>(a, stream))); break;
        default: return hipErrorInvalidValue;
      }
    }
  }
  // the query and key gradients turned back by position (rotary embedding)
  if (p.rope.on) {
    const size_t n = static_cast<size_t>(T_) * (p.qcols / 2 + G * D / 2);
    hipLaunchKernelGGL(rope_back_kernel<T>, dim3(static_cast<unsigned>((n + 255) / 256)),
                       dim3(256), 0, stream, static_cast<T*>(p.gall), T_, p.kpad, p.qcols, p.kcol,
                       G * D, L, D, p.rope);
    GQE_TRY(hipGetLastError());
  }
  // 4. router backward and the auxiliary loss
  if (p.wr != nullptr) {
    RouterBwdArgs r;
    r.x = p.x;
    r.wr = p.wr;
    r.bias = p.router_bias;
    r.idx = p.idx;
    r.dbg = p.dbg;
    r.dw = p.mode == 1 ? nullptr : p.dw;
    r.counts = p.counts;
    r.gall = p.gall;
    r.ldg = p.kpad;
    r.rcol = p.rcol;
    r.dr = p.dr;
    r.p_out = p.p_all;
    r.B = B;
    r.T = T_;
    r.d = d;
    r.G = G;
    r.E = E;
    r.gk = p.gk;
    r.mode = p.mode;
    r.aux_weight = p.aux_weight;
    hipLaunchKernelGGL(router_bwd_kernel<T>, dim3(T_), dim3(256), 0, stream, r);
    GQE_TRY(hipGetLastError());
    hipLaunchKernelGGL(column_sums_kernel, dim3(G * E), dim3(256), 0, stream, p.dr, p.p_all, T_,
                       G * E, p.dbr, p.psum);
    GQE_TRY(hipGetLastError());
    hipLaunchKernelGGL(aux_loss_kernel, dim3(1), dim3(64), 0, stream, p.psum, p.counts, B, T_, G,
                       E, p.gk, p.aux_loss);
    GQE_TRY(hipGetLastError());
  }
  // 5. transposed copies over tokens (zero past T), then the weight and input gradients
  const int tp = p.tpad;
  GQE_TRY(launch_transpose<T>(static_cast<const T*>(p.gall), p.kpad, T_, p.kpad,
                              static_cast<T*>(p.gall_t), tp, 0, tp, stream));
  GQE_TRY(launch_transpose<T>(static_cast<const T*>(p.x), d, T_, d, static_cast<T*>(p.x_t), tp, 0,
                              tp, stream));
  GQE_TRY(launch_transpose<T>(static_cast<const T*>(p.dy), d, T_, d, static_cast<T*>(p.dy_t), tp, 0,
                              tp, stream));
  GQE_TRY(launch_transpose<T>(static_cast<const T*>(p.s), p.ws, T_, p.ws, static_cast<T*>(p.s_t),
                              tp, 0, tp, stream));
  {
    NtArgs g = {};  // dW_O = dy^T . s
    g.a = p.dy_t;
    g.lda = tp;
    g.b = p.s_t;
    g.ldb = tp;
    g.M = d;
    g.N = p.ws;
    g.K = tp;
    g.nseg = 1;
    g.seg[0] = NtSeg{p.dwo, 0, d, p.ws, 0};
    g.part = p.gemm_part;
    g.splits = p.gemm_part != nullptr ? nt_gemm_splits(g.M, g.N, g.K) : 1;
    GQE_TRY(launch_nt_gemm<T>(g, stream));
  }
  {
    NtArgs g = {};  // dx = Gall . W_all
    g.a = p.gall;
    g.lda = p.kpad;
    g.b = p.w_t;
    g.ldb = p.kpad;
    g.M = T_;
    g.N = d;
    g.K = p.kpad;
    g.nseg = 1;
    g.seg[0] = NtSeg{p.dx, 0, T_, d, 0};
    GQE_TRY(launch_nt_gemm<T>(g, stream));
  }
  {
    NtArgs g = {};  // [dW_q; dW_k; dW_v; dW_r] = Gall^T . x
    g.a = p.gall_t;
    g.lda = tp;
    g.b = p.x_t;
    g.ldb = tp;
    g.M = p.kcols;
    g.N = d;
    g.K = tp;
    g.nseg = p.wr != nullptr ? 4 : 3;
    g.seg[0] = NtSeg{p.dwq, 0, p.qcols, d, 0};
    g.seg[1] = NtSeg{p.dwk, p.kcol, G * D, d, 0};
    g.seg[2] = NtSeg{p.dwv, p.vcol, G * D, d, 0};
    if (p.wr != nullptr) g.seg[3] = NtSeg{p.dwr, p.rcol, G * E, d, 0};
    g.part = p.gemm_part;
    g.splits = p.gemm_part != nullptr ? nt_gemm_splits(g.M, g.N, g.K) : 1;
    GQE_TRY(launch_nt_gemm<T>(g, stream));
  }
#undef GQE_TRY
  return hipSuccess;
}

template hipError_t launch_backward<bf16_t>(const BwdParams&, hipStream_t);
template hipError_t launch_backward<float>(const BwdParams&, hipStream_t);

}  // namespace gqe

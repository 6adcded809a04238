// K2: per-(b, g, e) token compaction ("sparse scheduling" in the pptc.cn
// review, section 6: the fixed cost of routing and dispatch that keeps the
// speed-up small at 2k tokens).
//
// For every list (b, g, e): counts = number of tokens t with e among
// idx[b, t, g, :]; offsets = exclusive prefix sum of counts in (b, g, e)
// row-major order; pos = those t in ascending order; slot = the rank j at
// which t chose e.
//
// Every token picks exactly k_g distinct experts in group g (k_g = k for the
// pages' layer), so the lists of one (b, g) always hold L*k_g entries
// together: they start at b*L*K + koff[g]*L (K = sum of k_g, koff the prefix
// of k_g) whatever the routing, and each (b, g) is dispatched independently of
// the others.  idx[b, t] holds group g's experts at koff[g] .. koff[g]+k_g-1.  The same holds for the tile map of the
// gathered query projection, which is kept per (b, g):
//   tile_off[(b*G+g)*(E+1) + e] = sum over e' < e of ceil(counts / tile_rows).
//
// Order is fixed by construction (wave ballots and prefix sums), never by
// atomics.  Sequences up to 8192 tokens use one block per (b, g) that counts,
// then scatters; longer ones split the tokens into 256-token chunks (count
// kernel, per-(b, g) scan over chunks, scatter kernel).
#include "debug_check.h"
#include "device_common.h"
#include "kernels.h"
#include "dispatch_dev.h"

namespace gqe {

namespace {

constexpr int kChunk = 256;       // tokens per block of the chunked path (4 waves x 64)
// the short-sequence dispatch kernel: one block per (b, g)
__global__ __launch_bounds__(64 * kSmallWaves) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ tile_off, int32_t* __restrict__ pos, int32_t* __restrict__ slot, int L,
    int G, int E, GroupK gk, int tile_rows, int n_lists, uint32_t* dbg) {
  __shared__ DispatchSmem<kSmallWaves> sm;
  dispatch_small_block<kSmallWaves>(blockIdx.x, sm, idx, counts, offsets, tile_off, pos, slot, L,
                                    G, E, gk, tile_rows, n_lists, dbg);
}

// ---------------------------------------------------------------------------
// long sequences: count per chunk, scan per (b, g), scatter per chunk
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ chunk_counts,
                                                             int L, int G, int E, GroupK gk,
                                                             int n_chunks, uint32_t* dbg) {
  __shared__ int cnt[4][64];
  const int c = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = c * kChunk + wave * 64 + lane;
  int32_t ids[32];
  for (int g = 0; g < G; ++g) {
    load_ids(idx, ids, b, t, g, L, gk);
#ifdef GQE_DEBUG
    if (t < L) check_ids(ids, gk.kg[g], E, dbg);
#endif
    for (int e = 0; e < E; ++e) {
      const uint64_t m = __ballot(chosen_rank(ids, gk.kg[g], e) >= 0);
      if (lane == 0) cnt[wave][g * E + e] = popc64(m);
    }
  }
  __syncthreads();
  const int GE = G * E;
  for (int i = threadIdx.x; i < GE; i += 256) {
    const int s = cnt[0][i] + cnt[1][i] + cnt[2][i] + cnt[3][i];
    chunk_counts[(static_cast<size_t>(b) * n_chunks + c) * GE + i] = s;
  }
}

// one block per (b, g), one wave per expert: chunk counts become absolute
// chunk bases in place; counts, offsets and the tile map come out on the way
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    int32_t* __restrict__ chunk_counts, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tile_off, int L, int G, int E, GroupK gk,
    int n_chunks, int tile_rows, int n_lists) {
  __shared__ int total[32];
  __shared__ int base[32];
  const int bg = blockIdx.x, b = bg / G, g = bg % G;
  const int GE = G * E;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n_waves = blockDim.x >> 6;
  for (int e = wave; e < E; e += n_waves) {
    const int gi = g * E + e;
    int runv = 0;
    for (int c0 = 0; c0 < n_chunks; c0 += 64) {
      const int c = c0 + lane;
      const size_t a = (static_cast<size_t>(b) * n_chunks + c) * GE + gi;
      const int v = c < n_chunks ? chunk_counts[a] : 0;
      int wt;
      const int ex = wave_excl_scan(v, lane, &wt);
      if (c < n_chunks) chunk_counts[a] = runv + ex;
      runv += wt;
    }
    if (lane == 0) total[e] = runv;
  }
  __syncthreads();
  if (wave == 0)
    finish_lists(total, counts, offsets, tile_off, bg, E, list_base(gk, b, g, L), L * gk.kg[g],
                 tile_rows, lane, n_lists);
  if (threadIdx.x < 32) {
    int s = list_base(gk, b, g, L);
    for (int e = 0; e < static_cast<int>(threadIdx.x) && e < E; ++e) s += total[e];
    base[threadIdx.x] = s;
  }
  __syncthreads();
  for (int e = wave; e < E; e += n_waves) {
    const int add = base[e];
    for (int c = lane; c < n_chunks; c += 64)
      chunk_counts[(static_cast<size_t>(b) * n_chunks + c) * GE + g * E + e] += add;
  }
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ chunk_base,
    int32_t* __restrict__ pos, int32_t* __restrict__ slot, int L, int G, int E, GroupK gk,
    int n_chunks) {
  __shared__ int cnt[4][64];
  const int c = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = c * kChunk + wave * 64 + lane;
  const int GE = G * E;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t ids[32];
  for (int g = 0; g < G; ++g) {
    load_ids(idx, ids, b, t, g, L, gk);
    for (int e = 0; e < E; ++e) {
      const uint64_t m = __ballot(chosen_rank(ids, gk.kg[g], e) >= 0);
      if (lane == 0) cnt[wave][g * E + e] = popc64(m);
    }
  }
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    load_ids(idx, ids, b, t, g, L, gk);
    for (int e = 0; e < E; ++e) {
      const int r = chosen_rank(ids, gk.kg[g], e);
      const uint64_t m = __ballot(r >= 0);
      if (r >= 0) {
        int wbase = 0;
        for (int w = 0; w < wave; ++w) wbase += cnt[w][g * E + e];
        const int entry = chunk_base[(static_cast<size_t>(b) * n_chunks + c) * GE + g * E + e] +
                          wbase + popc64(m & below);
        pos[entry] = t;
        slot[entry] = r;
      }
    }
  }
}

}  // namespace

int dispatch_chunks(int L) { return (L + kChunk - 1) / kChunk; }

hipError_t launch_dispatch(const int32_t* idx, int32_t* chunk_counts, int32_t* counts,
                           int32_t* offsets, int32_t* tile_off, int32_t* pos, int32_t* slot,
                           int B, int L, int G, int E, const GroupK& gk, int tile_rows,
                           uint32_t* dbg, hipStream_t stream) {
  const int n_lists = B * G * E;
  if (L <= kDispatchSmallMaxL && gk.kmax <= 4) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(B * G), dim3(64 * kSmallWaves), 0, stream, idx,
                       counts, offsets, tile_off, pos, slot, L, G, E, gk, tile_rows, n_lists, dbg);
    return hipGetLastError();
  }
  const int n_chunks = dispatch_chunks(L);
  const dim3 grid(n_chunks, B);
  hipLaunchKernelGGL(dispatch_count_kernel, grid, dim3(256), 0, stream, idx, chunk_counts, L, G,
                     E, gk, n_chunks, dbg);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(B * G), dim3(1024), 0, stream, chunk_counts,
                     counts, offsets, tile_off, L, G, E, gk, n_chunks, tile_rows, n_lists);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scatter_kernel, grid, dim3(256), 0, stream, idx, chunk_counts, pos,
                     slot, L, G, E, gk, n_chunks);
  return hipGetLastError();
}

}  // namespace gqe

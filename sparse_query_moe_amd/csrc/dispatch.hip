// K2: per-(b, g, e) token compaction ("sparse scheduling" in the pptc.cn
// review, section 6: the fixed cost of routing and dispatch that keeps the
// speed-up small at 2k tokens).
//
// For every list (b, g, e): counts = number of tokens t with e among
// idx[b, t, g, :]; offsets = exclusive prefix sum of counts in (b, g, e)
// row-major order; pos = those t in ascending order; slot = the rank j at
// which t chose e.  The order is fixed by construction, never by atomics:
//   1. count   : one block per (b, 256-token chunk); each wave ballots the
//                "chose e" predicate of its 64 tokens per (g, e)
//   2. scan    : one block turns the per-chunk counts into per-chunk list bases
//                (scan over chunks, then over lists) and the tile map of the
//                gathered query projection
//   3. scatter : the same ballots again; a lane's rank inside its wave's
//                ballot plus its wave's and chunk's bases is its list entry.
#include "device_common.h"
#include "kernels.h"

namespace gqe {

namespace {

constexpr int kChunk = 256;  // tokens per block (4 waves x 64)

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// does token t (this lane) choose expert e in group g?  Returns the rank j or -1.
__device__ __forceinline__ int chosen_rank(const int32_t* ids, int k, int e) {
  int r = -1;
  for (int j = 0; j < k; ++j) r = (ids[j] == e) ? j : r;
  return r;
}

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ chunk_counts,
                                                             int L, int G, int E, int k,
                                                             int n_chunks) {
  __shared__ int cnt[4][64];
  const int c = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = c * kChunk + wave * 64 + lane;
  const bool valid = t < L;
  int32_t ids[32];
  for (int g = 0; g < G; ++g) {
    for (int j = 0; j < k; ++j)
      ids[j] = valid ? idx[((static_cast<size_t>(b) * L + t) * G + g) * k + j] : -1;
    for (int e = 0; e < E; ++e) {
      const uint64_t m = __ballot(chosen_rank(ids, k, e) >= 0);
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

// Exclusive scan of 64 values across a wave; returns the exclusive prefix and
// sets *total.
__device__ __forceinline__ int wave_excl_scan(int v, int lane, int* total) {
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  *total = __shfl(incl, 63, 64);
  return incl - v;
}

// One block of 1024 threads.  chunk_counts is rewritten in place into the
// first list entry of every (b, chunk, g, e); counts, offsets and tile_off are
// produced on the way (their global copies double as the block's scratch).
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    int32_t* __restrict__ chunk_counts, int32_t* counts, int32_t* offsets,
    int32_t* __restrict__ tile_off, int B, int G, int E, int n_chunks, int tile_rows) {
  const int GE = G * E;
  const int n_lists = B * GE;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n_waves = blockDim.x >> 6;

  // 1) per list: exclusive scan over its chunks (bases relative to the list)
  for (int li = wave; li < n_lists; li += n_waves) {
    const int b = li / GE, gi = li % GE;
    int run = 0;
    for (int c0 = 0; c0 < n_chunks; c0 += 64) {
      const int c = c0 + lane;
      const size_t a = (static_cast<size_t>(b) * n_chunks + c) * GE + gi;
      const int v = c < n_chunks ? chunk_counts[a] : 0;
      int wt;
      const int ex = wave_excl_scan(v, lane, &wt);
      if (c < n_chunks) chunk_counts[a] = run + ex;
      run += wt;
    }
    if (lane == 0) counts[li] = run;
  }
  __threadfence_block();
  __syncthreads();
  // 2) offsets over lists, and the tile map (tiles of tile_rows rows per list)
  if (wave == 0) {
    int run = 0, trun = 0;
    for (int l0 = 0; l0 < n_lists; l0 += 64) {
      const int li = l0 + lane;
      const int v = li < n_lists ? counts[li] : 0;
      const int tv = (v + tile_rows - 1) / tile_rows;
      int wt, twt;
      const int ex = wave_excl_scan(v, lane, &wt);
      const int tex = wave_excl_scan(tv, lane, &twt);
      if (li < n_lists) {
        offsets[li] = run + ex;
        tile_off[li] = trun + tex;
      }
      run += wt;
      trun += twt;
    }
    if (lane == 0) {
      offsets[n_lists] = run;
      tile_off[n_lists] = trun;
    }
  }
  __threadfence_block();
  __syncthreads();
  // 3) make chunk bases absolute
  for (int li = wave; li < n_lists; li += n_waves) {
    const int b = li / GE, gi = li % GE;
    // written by wave 0 above: read through the vector path, not a scalar load
    const int add = __hip_atomic_load(offsets + li, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    for (int c = lane; c < n_chunks; c += 64)
      chunk_counts[(static_cast<size_t>(b) * n_chunks + c) * GE + gi] += add;
  }
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ chunk_base,
    int32_t* __restrict__ pos, int32_t* __restrict__ slot, int L, int G, int E, int k,
    int n_chunks) {
  __shared__ int cnt[4][64];
  const int c = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = c * kChunk + wave * 64 + lane;
  const bool valid = t < L;
  const int GE = G * E;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t ids[32];
  for (int g = 0; g < G; ++g) {
    for (int j = 0; j < k; ++j)
      ids[j] = valid ? idx[((static_cast<size_t>(b) * L + t) * G + g) * k + j] : -1;
    for (int e = 0; e < E; ++e) {
      const uint64_t m = __ballot(chosen_rank(ids, k, e) >= 0);
      if (lane == 0) cnt[wave][g * E + e] = popc64(m);
    }
  }
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    for (int j = 0; j < k; ++j)
      ids[j] = valid ? idx[((static_cast<size_t>(b) * L + t) * G + g) * k + j] : -1;
    for (int e = 0; e < E; ++e) {
      const int r = chosen_rank(ids, k, e);
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
                           int B, int L, int G, int E, int k, int tile_rows,
                           hipStream_t stream) {
  const int n_chunks = dispatch_chunks(L);
  const dim3 grid(n_chunks, B);
  hipLaunchKernelGGL(dispatch_count_kernel, grid, dim3(256), 0, stream, idx, chunk_counts, L, G,
                     E, k, n_chunks);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, stream, chunk_counts, counts,
                     offsets, tile_off, B, G, E, n_chunks, tile_rows);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scatter_kernel, grid, dim3(256), 0, stream, idx, chunk_counts, pos,
                     slot, L, G, E, k, n_chunks);
  return hipGetLastError();
}

}  // namespace gqe

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
#include "device_common.h"
#include "kernels.h"

namespace gqe {

namespace {

constexpr int kChunk = 256;       // tokens per block of the chunked path (4 waves x 64)
constexpr int kSmallWaves = 16;   // waves of the one-block-per-(b, g) path
constexpr int kSmallRounds = 8;   // 1024-token rounds it covers: L <= 8192

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// rank j at which this lane's token chose expert e, or -1
__device__ __forceinline__ int chosen_rank(const int32_t* ids, int k, int e) {
  int r = -1;
  for (int j = 0; j < k; ++j) r = (ids[j] == e) ? j : r;
  return r;
}

__device__ __forceinline__ void load_ids(const int32_t* idx, int32_t* ids, int b, int t, int g,
                                         int L, const GroupK& gk) {
  const bool valid = t < L;
  const size_t row = (static_cast<size_t>(b) * L + t) * gk.K + gk.koff[g];
  for (int j = 0; j < gk.kg[g]; ++j) ids[j] = valid ? idx[row + j] : -1;
}

// first entry of the lists of (b, g)
__device__ __forceinline__ int list_base(const GroupK& gk, int b, int g, int L) {
  return b * L * gk.K + gk.koff[g] * L;
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

// counts -> offsets and the per-(b, g) tile map for the lists of one (b, g);
// run by all lanes of one wave (lane e < E owns list e)
__device__ __forceinline__ void finish_lists(const int* cnt, int32_t* counts, int32_t* offsets,
                                             int32_t* tile_off, int bg, int E, int base, int rows,
                                             int tile_rows, int lane, int n_lists) {
  const int v = lane < E ? cnt[lane] : 0;
  const int tv = (v + tile_rows - 1) / tile_rows;
  int tot, ttot;
  const int ex = wave_excl_scan(v, lane, &tot);
  const int tex = wave_excl_scan(tv, lane, &ttot);
  if (lane < E) {
    counts[bg * E + lane] = v;
    offsets[bg * E + lane] = base + ex;
    tile_off[bg * (E + 1) + lane] = tex;
  }
  if (lane == 0) {
    tile_off[bg * (E + 1) + E] = ttot;
    if (bg * E + E == n_lists) offsets[n_lists] = base + rows;
  }
}

// ---------------------------------------------------------------------------
// short sequences: one block per (b, g).  Thread (wave w, lane) owns tokens
// t = r*1024 + 64*w + lane for rounds r < kSmallRounds; all their expert ids
// are loaded at once.  Pass 1 ballots every (round, wave, expert) count into
// LDS; one prefix over (expert, round, wave) gives every wave its list bases;
// pass 2 scatters.  Three barriers in all.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ tile_off, int32_t* __restrict__ pos, int32_t* __restrict__ slot, int L,
    int G, int E, GroupK gk, int tile_rows, int n_lists) {
  __shared__ int wcnt[kSmallRounds][kSmallWaves][32];  // count, then offset in the list, per (r, w, e)
  __shared__ int total[32];
  __shared__ int start[32];
  const int bg = blockIdx.x, b = bg / G, g = bg % G;
  const int k = gk.kg[g];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rounds = (L + 64 * kSmallWaves - 1) / (64 * kSmallWaves);

  // expert ids of this thread's tokens, packed 8 bits each (E <= 32, k_g <= 4 here)
  uint32_t packed[kSmallRounds];
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    const int t = r * 64 * kSmallWaves + wave * 64 + lane;
    uint32_t v = 0xffffffffu;
    if (r < rounds && t < L) {
      const int32_t* p = idx + (static_cast<size_t>(b) * L + t) * gk.K + gk.koff[g];
      v = 0u;
      for (int j = 0; j < 4; ++j) v |= static_cast<uint32_t>(j < k ? p[j] : 0xff) << (8 * j);
    }
    packed[r] = v;
  }
  auto rank_of = [&](uint32_t v, int e) {
    int rr = -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) rr = ((v >> (8 * j)) & 0xffu) == static_cast<uint32_t>(e) ? j : rr;
    return rr;
  };

  // pass 1: counts per (round, wave, expert)
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    if (r >= rounds) break;
    for (int e = 0; e < E; ++e) {
      const uint64_t m = __ballot(rank_of(packed[r], e) >= 0);
      if (lane == 0) wcnt[r][wave][e] = __popcll(m);
    }
  }
  __syncthreads();
  // prefix of every expert's counts in (round, wave) order, i.e. tokens
  // ascending: wave e scans list e, each lane owning two consecutive
  // (round, wave) entries; the entries become offsets inside the list
  static_assert(kSmallRounds * kSmallWaves == 128, "two (round, wave) entries per lane");
  for (int e = wave; e < E; e += kSmallWaves) {
    const int n = rounds * kSmallWaves;
    const int i0 = 2 * lane, i1 = 2 * lane + 1;
    int* c0p = &wcnt[i0 / kSmallWaves][i0 % kSmallWaves][e];
    int* c1p = &wcnt[i1 / kSmallWaves][i1 % kSmallWaves][e];
    const int c0 = i0 < n ? *c0p : 0;
    const int c1 = i1 < n ? *c1p : 0;
    int tot;
    const int ex = wave_excl_scan(c0 + c1, lane, &tot);
    if (i0 < n) *c0p = ex;
    if (i1 < n) *c1p = ex + c0;
    if (lane == 0) total[e] = tot;
  }
  __syncthreads();
  if (wave == 0)
    finish_lists(total, counts, offsets, tile_off, bg, E, list_base(gk, b, g, L), L * k, tile_rows,
                 lane, n_lists);
  if (threadIdx.x < 32) {  // first entry of every list
    const int e = threadIdx.x;
    int run = list_base(gk, b, g, L);
    for (int f = 0; f < e && f < E; ++f) run += total[f];
    start[e] = run;
  }
  __syncthreads();
  // pass 2: scatter
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    if (r >= rounds) break;
    const int t = r * 64 * kSmallWaves + wave * 64 + lane;
    for (int e = 0; e < E; ++e) {
      const int rk = rank_of(packed[r], e);
      const uint64_t m = __ballot(rk >= 0);
      if (rk >= 0) {
        const int entry = start[e] + wcnt[r][wave][e] + __popcll(m & below);
        pos[entry] = t;
        slot[entry] = rk;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// long sequences: count per chunk, scan per (b, g), scatter per chunk
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ chunk_counts,
                                                             int L, int G, int E, GroupK gk,
                                                             int n_chunks) {
  __shared__ int cnt[4][64];
  const int c = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = c * kChunk + wave * 64 + lane;
  int32_t ids[32];
  for (int g = 0; g < G; ++g) {
    load_ids(idx, ids, b, t, g, L, gk);
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
                           hipStream_t stream) {
  const int n_lists = B * G * E;
  if (L <= kSmallRounds * 64 * kSmallWaves && gk.kmax <= 4) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(B * G), dim3(64 * kSmallWaves), 0, stream, idx,
                       counts, offsets, tile_off, pos, slot, L, G, E, gk, tile_rows, n_lists);
    return hipGetLastError();
  }
  const int n_chunks = dispatch_chunks(L);
  const dim3 grid(n_chunks, B);
  hipLaunchKernelGGL(dispatch_count_kernel, grid, dim3(256), 0, stream, idx, chunk_counts, L, G,
                     E, gk, n_chunks);
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

// Device side of K2's short-sequence dispatch (per-(b, g, e) token
// compaction, "sparse scheduling" in the pptc.cn review, section 6): the
// helpers shared with the chunked path and the one-block-per-(b, g) body, a
// device function of the (b, g) index and of its block's LDS, so that the
// dispatch kernel and the short-sequence attention launch, which runs these
// blocks first in its grid, share it.  The list layout is described in
// dispatch.hip.
#pragma once

#include "debug_check.h"
#include "device_common.h"
#include "kernels.h"

namespace gqe {

namespace {

constexpr int kSmallWaves = 16;   // waves of the one-block-per-(b, g) kernel

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

// debug builds: the k expert ids of one (token, group) lie in [0, E) and
// differ from each other (a token picks k distinct experts)
__device__ __forceinline__ void check_ids(const int32_t* ids, int k, int E, uint32_t* dbg) {
  bool ok = true;
  for (int j = 0; j < k; ++j) {
    ok = ok && ids[j] >= 0 && ids[j] < E;
    for (int i = 0; i < j; ++i) ok = ok && ids[i] != ids[j];
  }
  dbg_ok(ok, dbg, kDbgExpert);
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
// short sequences: one block per (b, g) of W waves.  Thread (wave w, lane)
// owns tokens t = r*64*W + 64*w + lane for rounds r < 128/W; all their expert ids
// are loaded at once.  Pass 1 ballots every (round, wave, expert) count into
// LDS; one prefix over (expert, round, wave) gives every wave its list bases;
// pass 2 scatters.  Three barriers in all.
// ---------------------------------------------------------------------------
// LDS of one block of W waves (R rounds of 64*W tokens cover 8192): a static
// array of the dispatch kernel, or the start of the attention launch's
// dynamic LDS when the short forward's lists ride in that launch
template <int W>
struct DispatchSmem {
  static constexpr int R = 128 / W;
  static_assert(R * W == 128 && R * 64 * W == kDispatchSmallMaxL, "rounds cover L <= 8192");
  int wcnt[R][W][32];  // count, then offset in the list, per (round, wave, expert)
  int total[32];
  int start[32];
};

template <int W>
__device__ __forceinline__ void dispatch_small_block(
    int bg, DispatchSmem<W>& sm, const int32_t* __restrict__ idx, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tile_off, int32_t* __restrict__ pos,
    int32_t* __restrict__ slot, int L, int G, int E, const GroupK& gk, int tile_rows, int n_lists,
    uint32_t* dbg) {
  constexpr int kSmallWaves = W, kSmallRounds = DispatchSmem<W>::R;
  auto& wcnt = sm.wcnt;
  auto& total = sm.total;
  auto& start = sm.start;
  const int b = bg / G, g = bg % G;
  const int k = gk.kg[g];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rounds = (L + 64 * kSmallWaves - 1) / (64 * kSmallWaves);

  // expert ids of this thread's tokens, packed 8 bits each (E <= 32, k_g <= 4
  // here).  Slot by slot (k_g is the same for the whole block), every round's
  // load is issued before any is used (tokens past the sequence read token
  // 0's ids, inside idx), so the rounds share their load latency.
  const int K = gk.K, ko = gk.koff[g];
  int32_t raw[kSmallRounds][4];
  if (k == 2 && ((K | ko) & 1) == 0) {  // the pair as one 8-byte load per token
#pragma unroll
    for (int r = 0; r < kSmallRounds; ++r) {
      const int t = r * 64 * kSmallWaves + wave * 64 + lane;
      const int2 v = *reinterpret_cast<const int2*>(
          idx + (static_cast<size_t>(b) * L + (t < L ? t : 0)) * K + ko);
      raw[r][0] = v.x;
      raw[r][1] = v.y;
      raw[r][2] = raw[r][3] = 0xff;
    }
  } else {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j < k) {
#pragma unroll
      for (int r = 0; r < kSmallRounds; ++r) {
        const int t = r * 64 * kSmallWaves + wave * 64 + lane;
        raw[r][j] = idx[(static_cast<size_t>(b) * L + (t < L ? t : 0)) * K + ko + j];
      }
    } else {
#pragma unroll
      for (int r = 0; r < kSmallRounds; ++r) raw[r][j] = 0xff;
    }
  }
  }
  uint32_t packed[kSmallRounds];
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    const int t = r * 64 * kSmallWaves + wave * 64 + lane;
    uint32_t v = 0xffffffffu;
    if (r < rounds && t < L) {
#ifdef GQE_DEBUG
      check_ids(raw[r], k, E, dbg);
#endif
      v = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) v |= static_cast<uint32_t>(j < k ? raw[r][j] : 0xff) << (8 * j);
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

}  // namespace

}  // namespace gqe

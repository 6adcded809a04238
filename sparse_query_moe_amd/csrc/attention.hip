// K4: causal flash attention over slot-heads.
//
// Method: every query row a token activates -- one per selected expert of
// every group, plus the always-on shared head -- attends causally to its
// group's dense, unchanged K/V (pptc.cn review, section 5; gist.science,
// Architectuur en Routing).  The routed rows are compacted slot-major: row
// (b, g*k+j, t) holds the query of the j-th expert token t selected in group
// g, so all k*G+1 slot-heads are dense causal sequences and the kernel is the
// same one that runs the dense GQA baseline (G*E heads).  The per-row result
// is exactly softmax_s<=t(scale * q . K_s) V_s.
//
// gfx950 mapping (one block = 4 waves = 128 query rows of one head):
//   S^T = K . Q^T on 32x32x16 MFMA, so lane l owns query l % 32 and 16 of the
//   keys of every 32-key block in its accumulator; the row max needs a single
//   exchange with lane l ^ 32.  The accumulator, converted to bf16, is already
//   the B operand of O^T = V^T . P^T (keys along K), so probabilities never
//   leave registers; V^T comes from the projection in tiles of 64 keys with
//   the keys permuted inside every 16-key group to match that accumulator
//   order, so each V^T tile is one contiguous 8 KB (bf16, d_h 64) read and
//   each V^T fragment one 16-byte LDS read.  O^T again has one query per lane,
//   so the online-softmax rescale is lane-local.
//   K and V^T tiles of 64 keys are double-buffered in LDS (swizzled 16-byte
//   chunks, one barrier per tile).
//
// Softmax without a running maximum (the fast path).  Scores come out of the
// MFMA in log2 units and are exponentiated as they are: the subtraction of a
// maximum only guards the range of exp2, and the same shift cancels between
// numerator and denominator.  A row takes this path when its score against
// key 0 (which every causal row sees) lies in [-60, 60]; the block checks at
// the end that every row's sum stays in [2^-60, 2^100] and its output is
// finite.  Otherwise -- scores far outside the range of ordinary inputs --
// the whole block is recomputed with the running maximum (the fallback):
// the maximum is raised only when a tile exceeds it by more than 2^8, so the
// stale maximum keeps every probability <= 256, and it is subtracted inside
// the score MFMA chain as one more K step: unit key columns against -m split
// exactly into three operand-type parts, so no VALU work is spent on it and
// any float32 maximum is represented exactly.
//   Blocks are issued heaviest query block first to shorten the causal tail.
#include <math.h>

#include <type_traits>

#include "attention.h"
#include "device_common.h"
#include "dispatch_dev.h"
#include "kernels.h"

namespace gqe {

namespace {

constexpr float kRescaleThreshold = 8.0f;  // log2 units

// The running maximum enters the score MFMA of the fallback as one more K
// step: unit key columns against -m in the query's column, so the
// accumulator starts from zero and S^T - m costs no VALU work.  For bf16
// operands -m is split into three bf16 parts whose sum is exactly the
// float32 value (8 + 8 + 8 significant bits), against three unit columns.
template <typename T> struct ShiftOp;
template <> struct ShiftOp<bf16_t> {
  typedef bf16x8 type;
  static __device__ __forceinline__ type unit(int half) {
    type r = {};
    if (half == 0) r[0] = r[1] = r[2] = static_cast<__bf16>(1.f);
    return r;
  }
  static __device__ __forceinline__ type make(float v, int half) {
    type r = {};
    if (half == 0) {
      const __bf16 hi = static_cast<__bf16>(v);
      const float r1 = v - static_cast<float>(hi);  // exact
      const __bf16 mid = static_cast<__bf16>(r1);
      r[0] = hi;
      r[1] = mid;
      r[2] = static_cast<__bf16>(r1 - static_cast<float>(mid));  // exact
    }
    return r;
  }
  static __device__ __forceinline__ f32x16 mma(const type& unit, const type& nm) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(unit, nm, f32x16{}, 0, 0, 0);
  }
};
template <> struct ShiftOp<float> {
  typedef float type;
  static __device__ __forceinline__ type unit(int half) { return half == 0 ? 1.f : 0.f; }
  static __device__ __forceinline__ type make(float v, int half) { return half == 0 ? v : 0.f; }
  static __device__ __forceinline__ f32x16 mma(type unit, type nm) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(unit, nm, f32x16{}, 0, 0, 0);
  }
};

// the fast path's acceptance bounds (log2 units / row sums)
constexpr float kFastScore = 60.f;
constexpr float kFastSumMin = 0x1p-60f, kFastSumMax = 0x1p100f;


// QW query waves of 32*QB rows each share every K/V tile; NS groups of QW
// waves split the key range of the block (tile jt goes to group jt % NS) and
// merge their partial softmax states in LDS at the end.
template <typename T, int D, int QB, int QW, int NS>
struct AttnShape {
  static constexpr int NT = 64 * QW;        // threads of one key group
  static constexpr int THREADS = NT * NS;
  static constexpr int BQ = QW * 32 * QB, BKV = 64;
  static constexpr int EPC = 16 / static_cast<int>(sizeof(T));
  static constexpr int KROW = D * static_cast<int>(sizeof(T));    // bytes per K tile row (a key)
  static constexpr int VROW = BKV * static_cast<int>(sizeof(T));  // bytes per V^T tile row (a dim)
  static constexpr int KT = BKV * KROW, VT = D * VROW;
  static constexpr int STAGE = KT + VT;
  static constexpr int NDB = D / 32;  // 32-row blocks of O^T
  static constexpr int NKS = D / 16;  // K-steps of S^T
  // partial state of one wave in the merge area: o (NDB*16), m, l per lane
  static constexpr int PART = (NDB * 16 + 2) * 64;  // floats
  static constexpr int KV_LDS = NS * 2 * STAGE;
  static constexpr int MERGE_LDS = (NS - 1) * QW * QB * PART * 4;
  static constexpr int LDS = KV_LDS > MERGE_LDS ? KV_LDS : MERGE_LDS;
};

// q . scale * log2(e), rounded back to the storage type: scores come out of the
// MFMA already in log2 units.
__device__ __forceinline__ bf16x8 scale_frag(const bf16x8& f, float c) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = static_cast<__bf16>(static_cast<float>(f[j]) * c);
  return r;
}
__device__ __forceinline__ f32x8 scale_frag(const f32x8& f, float c) { return f * c; }

__device__ __forceinline__ float dot8(const bf16x8& a, const bf16x8& b) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s = fmaf(static_cast<float>(a[j]), static_cast<float>(b[j]), s);
  return s;
}
__device__ __forceinline__ float dot8(const f32x8& a, const f32x8& b) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s = fmaf(a[j], b[j], s);
  return s;
}

// How a launch treats the fallback: inline (a block that needs it runs it
// at once), or split over two launches of the same grid, the first running
// the fast path only and flagging the blocks that need the fallback in
// p.redo, the second running the fallback for the flagged blocks only.  The
// split keeps the fallback's registers out of the fast path's allocation.
enum { kInline = 0, kFastOnly = 1, kFallbackOnly = 2 };

// lists: the short forward's dispatch (one block per (b, g), lists.blocks of
// them) runs as the launch's first blocks, in the K/V stages' LDS; the
// attention's blocks follow.  Only the first launch of a split pair takes it.
template <typename T, int D, int QB, int QW, int NS, int MODE>
__global__ __launch_bounds__(64 * QW * NS, (QW * NS == 4 && D < 128) ? 2 : 1) void attention_kernel(
    AttnParams p, DispatchArgs lists) {
  typedef AttnShape<T, D, QB, QW, NS> S;
  extern __shared__ __align__(16) char smem[];
  int bid = blockIdx.x;
  if constexpr (MODE != kFallbackOnly) {
    constexpr int W = S::THREADS / 64;  // (the launch sizes the LDS for these blocks too)
    if (bid < lists.blocks) {
      dispatch_small_block<W>(bid, *reinterpret_cast<DispatchSmem<W>*>(smem), lists.idx,
                              lists.counts, lists.offsets, lists.tile_off, lists.pos, lists.slot,
                              lists.L, lists.G, lists.E, lists.gk, lists.tile_rows, lists.n_lists,
                              lists.dbg);
      return;
    }
    bid -= lists.blocks;
  }
  if constexpr (MODE == kFallbackOnly) {
    if (p.redo[bid] == 0) return;  // the fast path's result stands
  }
  typedef typename Frag<T>::type F;

  const int lane = threadIdx.x & 63, half = lane >> 5;
  const int grp = NS == 1 ? 0 : (threadIdx.x >> 6) / QW;  // key group
  const int wave = NS == 1 ? (threadIdx.x >> 6) : (threadIdx.x >> 6) % QW;  // query wave
  const int tid = threadIdx.x - grp * S::NT;    // thread inside the group
  char* gsm = smem + grp * 2 * S::STAGE;        // this group's two K/V stages
  const int L = p.L;
  const int nq = (L + S::BQ - 1) / S::BQ;
  const int bh_count = p.B * p.H;
  const int qi = bid / bh_count;
  const int bh = bid % bh_count;
  const int qblk = nq - 1 - qi;  // heaviest first
  const int b = bh / p.H, head = bh % p.H;
  int g = p.extra_group;
  if (head < p.n_grouped) {  // the group whose slot-heads include this one
    g = 0;
    while (p.koff[g + 1] <= head) ++g;
  }

  const T* Q = static_cast<const T*>(p.q) + (static_cast<size_t>(b) * p.q_heads + head) * L * D;
  const T* Kg = static_cast<const T*>(p.k) + (static_cast<size_t>(b) * p.G + g) * L * D;
  const T* Vg = static_cast<const T*>(p.vt) + (static_cast<size_t>(b) * p.G + g) * p.vt_tiles * D * 64;

  const int q0 = qblk * S::BQ;
  const int qw0 = q0 + 32 * QB * wave;                 // first query of this wave
  const int wave_last = min(qw0 + 32 * QB - 1, L - 1);  // last valid query of this wave
  const bool wave_active = qw0 < L;

  const int kv_end = min(q0 + S::BQ, L);
  const int ntiles = (kv_end + S::BKV - 1) / S::BKV;
  // group grp takes tiles grp, grp + NS, grp + 2 NS, ...; every group runs
  // the same number of rounds so that the block-wide barriers pair up
  const int rounds = (ntiles + NS - 1) / NS;
  auto tile_of = [&](int it) { return it * NS + grp; };  // tile of round it

  // K/V^T tiles go straight from global memory to LDS.  Wave w of a group
  // fills the 1 KB runs w, w + QW, ... of each tile (global_load_lds_dwordx4:
  // lane i writes LDS bytes 16i..16i+15 of the run), each lane fetching the
  // chunk that belongs there after the swizzle, so staging costs neither
  // VGPRs nor VALU work.  Keys past the sequence read row 0 of K (their
  // scores are masked) and the zero padding of the last V^T tile.
  constexpr int KPW = S::KT / 1024 / QW, VPW = S::VT / 1024 / QW;  // runs per wave
  static_assert(KPW * QW * 1024 == S::KT && VPW * QW * 1024 == S::VT,
                "direct staging needs whole 1 KB runs per wave");
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  int k_row[KPW], k_src[KPW], v_src[VPW];
#pragma unroll
  for (int i = 0; i < KPW; ++i) {
    const int off = (wave + QW * i) * 1024 + 16 * lane;
    const int row = off / S::KROW, pch = (off % S::KROW) / 16;
    k_row[i] = row;
    k_src[i] = row * D + (pch ^ swz_xor<S::KROW>(row)) * S::EPC;
  }
#pragma unroll
  for (int i = 0; i < VPW; ++i) {
    const int off = (wave + QW * i) * 1024 + 16 * lane;
    const int row = off / S::VROW, pch = (off % S::VROW) / 16;
    v_src[i] = row * 64 + (pch ^ swz_xor<S::VROW>(row)) * S::EPC;
  }
  auto dl_issue = [&](int jt, int buf) {
    const int j0 = jt * S::BKV;
    char* ks_ = gsm + buf * S::STAGE;
    char* vs_ = ks_ + S::KT;
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const size_t src = j0 + k_row[i] < L ? static_cast<size_t>(j0) * D + k_src[i]
                                            : static_cast<size_t>(k_src[i] - k_row[i] * D);
      dma16(Kg + src, ks_ + (swave + QW * i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < VPW; ++i)
      dma16(Vg + static_cast<size_t>(jt) * D * 64 + v_src[i], vs_ + (swave + QW * i) * 1024);
  };

  if (tile_of(0) < ntiles) dl_issue(tile_of(0), 0);

  // queries (pre-scaled) in registers, and each row's score against key 0,
  // which every causal row sees: the fallback's first running maximum, and
  // the test that admits the row to the fast path
  int qrow[QB];
  F qf[QB][S::NKS];
  float m_run[QB], l_run[QB], score0[QB];
  typename ShiftOp<T>::type nm[QB];
  const typename ShiftOp<T>::type unit = ShiftOp<T>::unit(half);
  f32x16 o[QB][S::NDB];
  bool fast = true;
  {
    F k0[S::NKS];
#pragma unroll
    for (int ks = 0; ks < S::NKS; ++ks) k0[ks] = load_frag(Kg + ks * 16 + 8 * half);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      qrow[qb] = qw0 + 32 * qb + (lane & 31);
      // this lane's query row: from q, or through the routing indices
      const T* qsrc = Q + static_cast<size_t>(qrow[qb]) * D;
      if (p.q_idx != nullptr && qrow[qb] < L) {
        int sh = p.q_src_heads - 1;  // the shared head
        if (head < p.n_grouped) {
          const int e = p.q_idx[(static_cast<size_t>(b) * L + qrow[qb]) * p.q_idx_stride + head];
          sh = g * p.q_E + min(max(e, 0), p.q_E - 1);
        }
        qsrc = static_cast<const T*>(p.q_src) +
               ((static_cast<size_t>(b) * p.q_src_heads + sh) * L + qrow[qb]) * D;
      }
      float dot = 0.f;
#pragma unroll
      for (int ks = 0; ks < S::NKS; ++ks) {
        if (qrow[qb] < L) {
          const F raw = load_frag(qsrc + ks * 16 + 8 * half);
          if (p.q_idx != nullptr && grp == 0)  // the slot-major copy of the row
            *reinterpret_cast<F*>(const_cast<T*>(Q) + static_cast<size_t>(qrow[qb]) * D + ks * 16 +
                                  8 * half) = raw;
          qf[qb][ks] = scale_frag(raw, p.scale_log2);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) qf[qb][ks][j] = 0;
        }
        dot += dot8(qf[qb][ks], k0[ks]);
      }
      score0[qb] = dot + __shfl_xor(dot, 32, 64);
      fast = fast && score0[qb] >= -kFastScore && score0[qb] <= kFastScore;
    }
  }
  auto reset = [&](bool shifted) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m_run[qb] = shifted ? score0[qb] : 0.f;
      nm[qb] = ShiftOp<T>::make(-m_run[qb], half);
      l_run[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[qb][db][i] = 0.f;
    }
  };

  // S^T of one query block and one 32-key half of the tile, minus the running
  // maximum when SHIFT (K fragments are read per block: LDS bandwidth is
  // cheaper than the registers that would hold them)
  auto scores = [&](const char* Ks, int j0, int qb, auto shift_tag, auto mask_tag, f32x16 (&sq)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (decltype(shift_tag)::value) {
        sq[kb] = ShiftOp<T>::mma(unit, nm[qb]);
        mma32(sq[kb], LdsFrag<T, S::KROW>::get(Ks, 32 * kb + (lane & 31), 8 * half), qf[qb][0]);
      } else {
        sq[kb] = mma32c(LdsFrag<T, S::KROW>::get(Ks, 32 * kb + (lane & 31), 8 * half), qf[qb][0],
                        f32x16{});
      }
#pragma unroll
      for (int ks = 1; ks < S::NKS; ++ks)
        mma32(sq[kb], LdsFrag<T, S::KROW>::get(Ks, 32 * kb + (lane & 31), ks * 16 + 8 * half),
              qf[qb][ks]);
    }
    if constexpr (decltype(mask_tag)::value) {  // drop keys after the query
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (j0 + 32 * kb + acc_row(i, lane) > qrow[qb]) sq[kb][i] = -INFINITY;
    }
  };
  // probabilities (in place), their lane sum into l_run, and O^T += V^T . P^T
  auto accumulate = [&](const char* Vs, int qb, f32x16 (&sq)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sq[kb][i] = __builtin_amdgcn_exp2f(sq[kb][i]);
    F pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pf[ks] = FragFromAcc<T>::get(sq[ks >> 1], 8 * (ks & 1));
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      l0 += sq[0][i];
      l1 += sq[1][i];
    }
    l_run[qb] += l0 + l1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
        mma32(o[qb][db], LdsFrag<T, S::VROW>::get(Vs, 32 * db + (lane & 31), ks * 16 + 8 * half),
              pf[ks]);
  };

  // one 64-key tile for this wave's QB query blocks: S^T of every block is
  // issued first (the MFMAs run on while the wave moves on), then each
  // block's softmax overlaps the next block's S^T or the previous block's
  // O^T update
  auto tile_fast = [&](const char* Ks, const char* Vs, int j0, auto masked) {
    f32x16 sq[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) scores(Ks, j0, qb, std::false_type{}, masked, sq[qb]);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) accumulate(Vs, qb, sq[qb]);
  };
  // the fallback: the maximum is raised when a tile's (half-row) maximum
  // exceeds it by more than the threshold; the exchange with lane l ^ 32 is
  // only paid then
  auto tile_shifted = [&](const char* Ks, const char* Vs, int j0, auto masked) {
    f32x16 sq[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) scores(Ks, j0, qb, std::true_type{}, masked, sq[qb]);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float v = sq[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) v = fmaxf(v, sq[qb][kb][i]);
      if (__any(v > kRescaleThreshold)) {  // wave-uniform branch
        const float mx = fmaxf(fmaxf(v, __shfl_xor(v, 32, 64)), 0.f);
        const float m_new = m_run[qb] + mx;
        const float sh = m_new - m_run[qb];
        const float alpha = __builtin_amdgcn_exp2f(-sh);
        m_run[qb] = m_new;
        nm[qb] = ShiftOp<T>::make(-m_new, half);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < S::NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sq[qb][kb][i] -= sh;
      }
      accumulate(Vs, qb, sq[qb]);
    }
  };

  // the key walk of this group; the first tile's copy is already in flight
  // on the first walk
  auto walk = [&](auto tilef, bool first_issued) {
    if (!first_issued && tile_of(0) < ntiles) dl_issue(tile_of(0), 0);
    dma_barrier(0);
    for (int it = 0; it < rounds; ++it) {
      const int jt = tile_of(it);
      const int jn = it + 1 < rounds ? tile_of(it + 1) : ntiles;  // next round's tile
      if (jn < ntiles) dl_issue(jn, (it + 1) & 1);
      const char* Ks = gsm + (it & 1) * S::STAGE;
      const char* Vs = Ks + S::KT;
      const int j0 = jt * S::BKV;
      if ((NS == 1 || jt < ntiles) && wave_active && j0 <= wave_last) {
        if (j0 + S::BKV - 1 <= qw0)
          tilef(Ks, Vs, j0, std::false_type{});
        else
          tilef(Ks, Vs, j0, std::true_type{});
      }
      dma_barrier(0);
    }
  };

  // the fast path for the whole block, or the fallback; a block whose fast
  // result fails the range checks is recomputed with the fallback
  if constexpr (MODE == kFallbackOnly) {
    reset(true);
    walk(tile_shifted, true);
  } else if (__syncthreads_or(fast ? 0 : 1) == 0) {
    reset(false);
    walk(tile_fast, true);
    bool ok = true;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
      float os = 0.f;
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) os += o[qb][db][i];
      if (qrow[qb] < L) ok = ok && lt >= kFastSumMin && lt <= kFastSumMax && fabsf(os) <= kFastSumMax;
    }
    const int redo = __syncthreads_or(ok ? 0 : 1);
    if constexpr (MODE == kFastOnly) {
      if (threadIdx.x == 0) p.redo[bid] = redo;
      if (redo) return;
    } else if (redo) {
      reset(true);
      walk(tile_shifted, false);
    }
  } else {
    if constexpr (MODE == kFastOnly) {
      if (threadIdx.x == 0) p.redo[bid] = 1;
      wait_vm(0);  // the first tile's copy lands before the block's LDS is released
      return;
    } else {
      reset(true);
      walk(tile_shifted, true);
    }
  }

  if constexpr (NS > 1) {
    // merge: groups 1.. park (o, m, l) in LDS (the K/V stages are free after
    // the last barrier), group 0 rescales everything to the common maximum
    float* part = reinterpret_cast<float*>(smem);
    auto slot_of = [&](int gsrc, int qb) {
      return part + (((gsrc - 1) * QW + wave) * QB + qb) * S::PART;
    };
    if (grp > 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float* ps = slot_of(grp, qb);
#pragma unroll
        for (int db = 0; db < S::NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) ps[(db * 16 + i) * 64 + lane] = o[qb][db][i];
        ps[S::NDB * 16 * 64 + lane] = m_run[qb];
        ps[(S::NDB * 16 + 1) * 64 + lane] = l_run[qb];
      }
    }
    lds_barrier();
    if (grp > 0) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mmax = m_run[qb];
      for (int gs = 1; gs < NS; ++gs) mmax = fmaxf(mmax, slot_of(gs, qb)[S::NDB * 16 * 64 + lane]);
      const float a0 = __builtin_amdgcn_exp2f(m_run[qb] - mmax);
      m_run[qb] = mmax;
      l_run[qb] *= a0;
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[qb][db][i] *= a0;
      for (int gs = 1; gs < NS; ++gs) {
        const float* ps = slot_of(gs, qb);
        const float a = __builtin_amdgcn_exp2f(ps[S::NDB * 16 * 64 + lane] - mmax);
        l_run[qb] = fmaf(ps[(S::NDB * 16 + 1) * 64 + lane], a, l_run[qb]);
#pragma unroll
        for (int db = 0; db < S::NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[qb][db][i] = fmaf(ps[(db * 16 + i) * 64 + lane], a, o[qb][db][i]);
      }
    }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
    // log-sum-exp of the row's scores (log2 units, as the pre-scaled scores)
    // for the backward pass; both lanes of a row hold the same m_run
    if (p.lse != nullptr && half == 0 && qrow[qb] < L)
      p.lse[(static_cast<size_t>(b) * p.H + head) * L + qrow[qb]] = m_run[qb] + log2f(l_tot);
    if (qrow[qb] < L) {
      float inv = 1.f / l_tot;
      if (p.row_scale != nullptr && head < p.n_grouped)
        inv *= p.row_scale[(static_cast<size_t>(b) * L + qrow[qb]) * p.n_grouped + head];
      T* out = static_cast<T*>(p.o) + (static_cast<size_t>(b) * L + qrow[qb]) * p.ld_o +
               static_cast<size_t>(head) * D;
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d0 = 32 * db + 8 * a + 4 * half;
          T v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = from_f32<T>(o[qb][db][4 * a + r] * inv);
          if constexpr (sizeof(T) == 2)
            *reinterpret_cast<uint2*>(out + d0) = *reinterpret_cast<const uint2*>(v);
          else
            *reinterpret_cast<uint4*>(out + d0) = *reinterpret_cast<const uint4*>(v);
        }
    }
  }
}

template <typename T, int D, int QB, int QW, int NS, int MODE>
hipError_t launch_attention_mode(const AttnParams& p, long long blocks, const DispatchArgs& lists,
                                 hipStream_t stream) {
  typedef AttnShape<T, D, QB, QW, NS> S;
  if (S::LDS > 65536) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&attention_kernel<T, D, QB, QW, NS, MODE>),
        hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS);
    if (attr != hipSuccess) return attr;
  }
  constexpr int lists_lds = static_cast<int>(sizeof(DispatchSmem<S::THREADS / 64>));
  const int lds = lists.blocks > 0 && lists_lds > S::LDS ? lists_lds : S::LDS;
  hipLaunchKernelGGL((attention_kernel<T, D, QB, QW, NS, MODE>),
                     dim3(static_cast<unsigned>(blocks + lists.blocks)), dim3(S::THREADS), lds,
                     stream, p, lists);
  return hipGetLastError();
}

// SPLIT: the fast path and the fallback in two launches (p.redo must hold one
// int per block); otherwise one launch with the fallback inline
template <typename T, int D, int QB, int QW, int NS, bool SPLIT>
hipError_t launch_attention_d(const AttnParams& p, const DispatchArgs& lists, hipStream_t stream) {
  typedef AttnShape<T, D, QB, QW, NS> S;
  const int nq = (p.L + S::BQ - 1) / S::BQ;
  const long long blocks = static_cast<long long>(nq) * p.B * p.H;
  if (blocks == 0 && lists.blocks == 0) return hipSuccess;
  if (!SPLIT || p.redo == nullptr)
    return launch_attention_mode<T, D, QB, QW, NS, kInline>(p, blocks, lists, stream);
  const hipError_t e = launch_attention_mode<T, D, QB, QW, NS, kFastOnly>(p, blocks, lists, stream);
  if (e != hipSuccess) return e;
  DispatchArgs none{};
  return launch_attention_mode<T, D, QB, QW, NS, kFallbackOnly>(p, blocks, none, stream);
}

}  // namespace

// Long launches: 4 query waves per block, two 32-query blocks per wave (half
// the LDS traffic per MFMA).  Short ones, whose blocks would not cover the
// chip, take 64-row blocks whose key range is split over NS groups of waves,
// which shortens the causal critical path NS-fold.
template <typename T>
hipError_t launch_attention(const AttnParams& p, int D, hipStream_t stream,
                            const DispatchArgs* lists_in) {
  DispatchArgs none{};
  const DispatchArgs& lists = lists_in != nullptr ? *lists_in : none;
  if (lists.blocks > 0 && (lists.L > kDispatchSmallMaxL || lists.gk.kmax > 4))
    return hipErrorInvalidValue;
  const bool wide = static_cast<long long>(p.L) * p.B * p.H >= 256LL * 256 * 4;
  if constexpr (sizeof(T) == 2) {
    switch (D) {
      case 32: return wide ? launch_attention_d<T, 32, 2, 4, 1, true>(p, lists, stream)
                           : launch_attention_d<T, 32, 1, 2, 4, false>(p, lists, stream);
      case 64: return wide ? launch_attention_d<T, 64, 2, 4, 1, true>(p, lists, stream)
                           : launch_attention_d<T, 64, 1, 2, 4, false>(p, lists, stream);
      case 128: return wide ? launch_attention_d<T, 128, 1, 4, 1, true>(p, lists, stream)
                            : launch_attention_d<T, 128, 1, 2, 2, false>(p, lists, stream);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (D) {
      case 32: return wide ? launch_attention_d<T, 32, 1, 4, 1, false>(p, lists, stream)
                           : launch_attention_d<T, 32, 1, 2, 4, false>(p, lists, stream);
      case 64: return wide ? launch_attention_d<T, 64, 1, 4, 1, false>(p, lists, stream)
                           : launch_attention_d<T, 64, 1, 2, 2, false>(p, lists, stream);
      case 128: return launch_attention_d<T, 128, 1, 4, 1, false>(p, lists, stream);
      default: return hipErrorInvalidValue;
    }
  }
}

template hipError_t launch_attention<bf16_t>(const AttnParams&, int, hipStream_t,
                                             const DispatchArgs*);
template hipError_t launch_attention<float>(const AttnParams&, int, hipStream_t,
                                            const DispatchArgs*);

}  // namespace gqe

// K3 and K5: the layer's projections on MFMA (bf16 -> fp32 accumulation, or
// fp32 throughout for float32 layers).
//
// Every product here has the "NT" form C[m, n] = sum_k A[m, k] * W[n, k]: the
// activations are row-major with K contiguous and the weights use the
// [out, in] layout, also K contiguous, so both MFMA operands are 16-byte
// vector loads along K.  A block computes a BM x BN tile with 4 waves; K
// streams through a ring of three LDS stages of 128-byte rows (64 bf16 or
// 32 fp32 elements), swizzled per 16-byte chunk.  The stages are filled by
// direct global-to-LDS loads (no register round trip), issued two K steps
// ahead; one barrier per K step, after a wait that counts only the loads of
// the stage about to be read.  The finished tile is staged through LDS so
// that every output row or column is written with 16-byte stores.
//
// The three users differ only in where rows come from and where results go:
//   dense projection  : rows are tokens; output columns are split into
//                       segments (shared-head Q | K | V, or Q | K | V of dense
//                       GQA), each written head-split, V transposed
//                       (gist.science, Architectuur en Routing: dense K/V).
//   gathered Q        : rows are the entries of one dispatch list (b, g, e);
//                       A rows are x[b, pos], W is the d_h rows of head g*E+e,
//                       results land in slot-head g*k+slot at position pos
//                       (only selected experts are computed: the query-side
//                       sparsity of pptc.cn section 5).
//   output projection : slot vectors times W_O (hotpaper.ai: W_O of k*G+2
//                       slots), row-major.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "debug_check.h"
#include "device_common.h"

#include "kernels.h"
#include "router_dev.h"

namespace gqe {

namespace {

// A problem that defines store_acc(row, col, value) (tile-relative) receives
// the float32 accumulators directly instead of a tile staged in LDS as T.
template <class P, class = void> struct HasStoreAcc : std::false_type {};
template <class P>
struct HasStoreAcc<P, std::void_t<decltype(std::declval<const P&>().store_acc(0, 0, 0.f))>>
    : std::true_type {};
// A problem that defines rotating() and rotate(row, col, v, partner) turns its
// float32 results by position before they are stored (the rotary embedding:
// the partner of column c is column c ^ 1, held by lane l ^ 1).
template <class P, class = void> struct HasRotate : std::false_type {};
template <class P>
struct HasRotate<P, std::void_t<decltype(std::declval<const P&>().rotate(0, 0, 0.f, 0.f))>>
    : std::true_type {};
// A problem that defines wslot_k() may form its last K step's A tile in the
// main loop (the output projection's weighted slot, below): wslot_k() hard
// slots of one K step each, then the shared slot, then the weighted slot.
template <class P, class = void> struct HasWslot : std::false_type {};
template <class P>
struct HasWslot<P, std::void_t<decltype(std::declval<const P&>().wslot_k())>> : std::true_type {};
constexpr int kWslotMaxK = 32;  // hard slots the in-loop weighted slot takes

template <typename T, int BM_, int BN_, int WGM_, int WGN_, int NST_ = 2>
struct GemmShape {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, NST = NST_;
  static constexpr int EPC = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte chunk
  static constexpr int BKE = 8 * EPC;                            // K elements per LDS row
  static constexpr int A_CH = BM / 32;                           // A chunks per thread per stage
  static constexpr int B_CH = BN / 32;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int STAGE = (BM + BN) * 128;
  // the finished tile is staged in LDS as T, rows padded by 16 bytes for bf16
  static constexpr int LDC = BN + (sizeof(T) == 2 ? 8 : 0);
  static constexpr int CBYTES = BM * LDC * static_cast<int>(sizeof(T));
  static constexpr int LDS = NST * STAGE > CBYTES ? NST * STAGE : CBYTES;
  static_assert(WGM * WGN == 4, "4 waves");
  static_assert(TM >= 1 && TN >= 1, "wave tile at least 32x32");
  static_assert(NST >= 2 && NST <= 4, "2 to 4 LDS stages");
};

// The main loop: P supplies K (a multiple of S::BKE), a_row(r) and b_row(n)
// (row pointers, or nullptr for rows outside the problem), a_any() (any valid
// row, loaded in place of missing ones: their results are never written) and
// write_tile(staged tile).
//
// K streams through an NST-stage ring of LDS tiles filled by direct
// global-to-LDS loads (global_load_lds_dwordx4): NST-1 stages are in flight
// while one is consumed, without any VGPR staging.  Each wave fills whole
// 1 KB runs of LDS (64 lanes x 16 B); a lane picks the source chunk so that
// the data lands in the swizzled position the fragment reads expect.  One
// barrier per K step, preceded by a wait for this wave's loads of that step
// only (no fence: a fence would also drain the later stages).
template <typename T, class S, class P>
__device__ __forceinline__ void gemm_block(const P& prob, char* smem) {
  typedef typename Frag<T>::type F;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int swave = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform: LDS bases go through M0
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int r0 = tid >> 3;
  const int pc = tid & 7;  // physical 16-byte chunk this lane fills in its row

  const T* ap[S::A_CH];
  const T* bp[S::B_CH];
#pragma unroll
  for (int i = 0; i < S::A_CH; ++i) {
    const int r = r0 + 32 * i;
    const T* p = prob.a_row(r);
    ap[i] = (p != nullptr ? p : prob.a_any()) + ((pc ^ ((r >> 1) & 7)) * S::EPC);
  }
#pragma unroll
  for (int i = 0; i < S::B_CH; ++i) {
    const int r = r0 + 32 * i;
    const T* p = prob.b_row(r);
    bp[i] = (p != nullptr ? p : prob.b_any()) + ((pc ^ ((r >> 1) & 7)) * S::EPC);
  }

  const int nk = prob.K / S::BKE;
  constexpr int per_stage = S::A_CH + S::B_CH;
  // The in-loop weighted slot (bf16, one K step per slot): every thread sums
  // w[row, h] * A[row, chunk] over the hard-slot steps h < wk for the 16-byte
  // chunks it copies itself, in slot order (the weighted-slot kernel's
  // arithmetic), and at the shared step writes the bf16 sums where its copy
  // of the last step's A chunk would land.  The routing weights of the tile's
  // rows come to LDS after the ring, copied before the first stage.
  constexpr bool WSL = HasWslot<P>::value && sizeof(T) == 2;
  int wk = 0;
  float wacc[WSL ? S::A_CH : 1][8];
  if constexpr (WSL) {
    wk = prob.wslot_k();
    if (wk > 0) {
#pragma unroll
      for (int i = 0; i < S::A_CH; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) wacc[i][j] = 0.f;
      // [BM, wk] floats, 16 bytes per lane, runs of 1 KB over the 4 waves
      const char* src = reinterpret_cast<const char*>(prob.wslot_rows());
      const int valid = prob.wslot_valid_rows() * wk * 4;  // bytes inside w
      char* dst = smem + S::NST * S::STAGE;
      const int runs = (S::BM * wk * 4 + 1023) / 1024;
      for (int rr = swave; rr < runs; rr += 4) {
        const int off = rr * 1024 + 16 * lane;
        dma16(src + (off + 16 <= valid ? off : 0), dst + rr * 1024);
      }
    }
  }
  auto issue = [&](int kt) {
    char* st = smem + (kt % S::NST) * S::STAGE;
    const bool own_a = WSL && wk > 0 && kt == nk - 1;  // the weighted slot's A is formed here
#pragma unroll
    for (int i = 0; i < S::A_CH; ++i)
      if (!own_a) dma16(ap[i] + kt * S::BKE, st + (4 * i + swave) * 1024);
#pragma unroll
    for (int i = 0; i < S::B_CH; ++i)
      dma16(bp[i] + kt * S::BKE, st + S::BM * 128 + (4 * i + swave) * 1024);
  };

  f32x16 acc[S::TM][S::TN];
#pragma unroll
  for (int a = 0; a < S::TM; ++a)
#pragma unroll
    for (int b = 0; b < S::TN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  // per K step: wait for this wave's loads of stage kt, barrier (the stage is
  // complete and every wave is done with stage kt-1), refill stage kt-1's
  // buffer with stage kt+NST-1, then read the fragments and multiply
  constexpr int NKS = S::BKE / 16;
#pragma unroll
  for (int st = 0; st < S::NST - 1; ++st)
    if (st < nk) issue(st);
  for (int kt = 0; kt < nk; ++kt) {
    const int later = min(S::NST - 2, nk - 1 - kt);  // stages issued after kt
    // (the last stage copies no A when the weighted slot is formed)
    const bool last_later = WSL && wk > 0 && later > 0 && kt + later == nk - 1;
    wait_vm(later * per_stage - (last_later ? S::A_CH : 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (kt + S::NST - 1 < nk) issue(kt + S::NST - 1);
    const char* sa = smem + (kt % S::NST) * S::STAGE;
    const char* sb = sa + S::BM * 128;
    if constexpr (WSL) {
      if (wk > 0 && kt < wk) {  // hard slot kt: accumulate this thread's chunks
        const float* wt = reinterpret_cast<const float*>(smem + S::NST * S::STAGE);
#pragma unroll
        for (int i = 0; i < S::A_CH; ++i) {
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(sa + (4 * i + swave) * 1024 + 16 * lane);
          const float wv = wt[(r0 + 32 * i) * wk + kt];
#pragma unroll
          for (int j = 0; j < 8; ++j) wacc[i][j] = fmaf(wv, static_cast<float>(v[j]), wacc[i][j]);
        }
      } else if (wk > 0 && kt == wk) {  // the shared step: the weighted slot's A chunks
        char* sw = smem + ((nk - 1) % S::NST) * S::STAGE;
#pragma unroll
        for (int i = 0; i < S::A_CH; ++i) {
          bf16x8 o;
#pragma unroll
          for (int j = 0; j < 8; ++j) o[j] = static_cast<__bf16>(wacc[i][j]);
          *reinterpret_cast<bf16x8*>(sw + (4 * i + swave) * 1024 + 16 * lane) = o;
          const int r = r0 + 32 * i;
          prob.wslot_store(r, pc ^ ((r >> 1) & 7), o);
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int e = ks * 16 + 8 * (lane >> 5);
      F af[S::TM], bf[S::TN];
#pragma unroll
      for (int a = 0; a < S::TM; ++a)
        af[a] = LdsFrag<T, 128>::get(sa, wm * S::WM + 32 * a + (lane & 31), e);
#pragma unroll
      for (int b = 0; b < S::TN; ++b)
        bf[b] = LdsFrag<T, 128>::get(sb, wn * S::WN + 32 * b + (lane & 31), e);
#pragma unroll
      for (int a = 0; a < S::TM; ++a)
#pragma unroll
        for (int b = 0; b < S::TN; ++b) mma32(acc[a][b], af[a], bf[b]);
    }
  }
  if constexpr (HasRotate<P>::value) {
    if (prob.rotating()) {
#pragma unroll
      for (int a = 0; a < S::TM; ++a)
#pragma unroll
        for (int b = 0; b < S::TN; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float v = acc[a][b][i];
            const float partner = __shfl_xor(v, 1, 64);
            acc[a][b][i] = prob.rotate(wm * S::WM + 32 * a + acc_row(i, lane),
                                       wn * S::WN + 32 * b + (lane & 31), v, partner);
          }
    }
  }
  if constexpr (HasStoreAcc<P>::value) {
#pragma unroll
    for (int a = 0; a < S::TM; ++a)
#pragma unroll
      for (int b = 0; b < S::TN; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          prob.store_acc(wm * S::WM + 32 * a + acc_row(i, lane), wn * S::WN + 32 * b + (lane & 31),
                         acc[a][b][i]);
  } else {
    lds_barrier();  // every wave is done reading the ring before it holds the tile

    // epilogue: stage the tile, then the problem writes it out in 8-element chunks
    T* ct = reinterpret_cast<T*>(smem);
#pragma unroll
    for (int a = 0; a < S::TM; ++a)
#pragma unroll
      for (int b = 0; b < S::TN; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          ct[(wm * S::WM + 32 * a + acc_row(i, lane)) * S::LDC + wn * S::WN + 32 * b + (lane & 31)] =
              from_f32<T>(acc[a][b][i]);
    lds_barrier();
    prob.write_tile(ct);
  }
}

// copy 8 contiguous elements (16 B of bf16, 32 B of fp32)
template <typename T>
__device__ __forceinline__ void copy8(T* dst, const T* src) {
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  d4[0] = s4[0];
  if constexpr (sizeof(T) == 4) d4[1] = s4[1];
}

// ---------------------------------------------------------------------------
// dense projection with up to 3 output segments
// ---------------------------------------------------------------------------
struct DenseArgs {
  const void* x;
  int M, K, N, L, D;
  int64_t vt_tiles;
  int nseg;
  ProjSeg seg[3];
  RopeTable rope;
};

template <typename T, class S>
struct DenseProb {
  const DenseArgs& a;
  int m0, n0, K;
  __device__ DenseProb(const DenseArgs& args, int m0_, int n0_) : a(args), m0(m0_), n0(n0_), K(args.K) {}
  // the segment holding output column col, selected field by field (a dynamic
  // index into the argument array would spill it to scratch)
  __device__ __forceinline__ ProjSeg seg_of(int col) const {
    const bool s1 = a.nseg > 1 && col >= a.seg[1].n_begin;
    const bool s2 = a.nseg > 2 && col >= a.seg[2].n_begin;
    ProjSeg r;
    r.w = s2 ? a.seg[2].w : s1 ? a.seg[1].w : a.seg[0].w;
    r.out = s2 ? a.seg[2].out : s1 ? a.seg[1].out : a.seg[0].out;
    r.n_begin = s2 ? a.seg[2].n_begin : s1 ? a.seg[1].n_begin : a.seg[0].n_begin;
    r.n = 0;
    r.heads = s2 ? a.seg[2].heads : s1 ? a.seg[1].heads : a.seg[0].heads;
    r.head_base = s2 ? a.seg[2].head_base : s1 ? a.seg[1].head_base : a.seg[0].head_base;
    r.transposed = s2 ? a.seg[2].transposed : s1 ? a.seg[1].transposed : a.seg[0].transposed;
    r.rope = s2 ? a.seg[2].rope : s1 ? a.seg[1].rope : a.seg[0].rope;
    return r;
  }
  // rows are tokens (position m % L); the rotated segments' columns are
  // head-split, dim (col - n_begin) % D
  __device__ __forceinline__ bool rotating() const { return a.rope.on != 0; }
  __device__ __forceinline__ float rotate(int r, int c, float v, float partner) const {
    const int m = m0 + r, col = n0 + c;
    if (m >= a.M || col >= a.N) return v;
    const ProjSeg sg = seg_of(col);
    if (!sg.rope) return v;
    const int dd = (col - sg.n_begin) % a.D;
    float cs, sn;
    rope_cs(m % a.L, a.rope.theta[dd >> 1], cs, sn);
    return rope_apply(v, partner, dd, cs, sn);
  }
  __device__ __forceinline__ const T* a_any() const { return static_cast<const T*>(a.x); }
  __device__ __forceinline__ const T* b_any() const { return static_cast<const T*>(a.seg[0].w); }
  __device__ __forceinline__ const T* a_row(int r) const {
    const int m = m0 + r;
    return m < a.M ? static_cast<const T*>(a.x) + static_cast<size_t>(m) * a.K : nullptr;
  }
  __device__ __forceinline__ const T* b_row(int n) const {
    const int col = n0 + n;
    if (col >= a.N) return nullptr;
    const ProjSeg sg = seg_of(col);
    return static_cast<const T*>(sg.w) + static_cast<size_t>(col - sg.n_begin) * a.K;
  }
  // head-split outputs: 8 consecutive head dims per chunk; the transposed
  // (V) segment takes 8 consecutive tokens per chunk instead
  __device__ __forceinline__ void write_tile(const T* ct) const {
    constexpr int CW = S::BN / 8;
    for (int c = threadIdx.x; c < S::BM * CW; c += 256) {
      const int r = c / CW, c8 = c % CW;
      const int m = m0 + r, col = n0 + 8 * c8;
      if (m >= a.M || col >= a.N) continue;
      const ProjSeg sg = seg_of(col);
      if (sg.transposed) continue;
      const int cl = col - sg.n_begin;
      const int hh = sg.head_base + cl / a.D, dd = cl % a.D;
      const int b = m / a.L, t = m % a.L;
      T* dst = static_cast<T*>(sg.out) + ((static_cast<size_t>(b) * sg.heads + hh) * a.L + t) * a.D + dd;
      copy8(dst, ct + r * S::LDC + 8 * c8);
    }
    // V^T: one 16-byte chunk = 8 keys of one head dim, in the permuted order
    // (chunk u of a 16-key group holds keys 4u..4u+3 and 8+4u..8+4u+3)
    for (int c = threadIdx.x; c < (S::BM / 8) * S::BN; c += 256) {
      const int nl = c % S::BN, r8 = c / S::BN;
      const int g16 = r8 >> 1, u = r8 & 1;
      const int col = n0 + nl, mg = m0 + 16 * g16;  // first token of the 16-key group
      if (mg >= a.M || col >= a.N) continue;
      const ProjSeg sg = seg_of(col);
      if (!sg.transposed) continue;
      const int cl = col - sg.n_begin;
      const int hh = sg.head_base + cl / a.D, dd = cl % a.D;
      T* out = static_cast<T*>(sg.out);
      auto key_of = [&](int j) { return 16 * g16 + (j < 4 ? 4 * u + j : 8 + 4 * u + (j - 4)); };
      if ((a.L & 15) == 0 && mg + 16 <= a.M) {
        const int b = mg / a.L, t = mg % a.L;  // t is a multiple of 16
        alignas(16) T v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = ct[key_of(j) * S::LDC + nl];
        copy8(out + vt_index(b, sg.heads, hh, dd, t) + 8 * u, v);
      } else {
        for (int j = 0; j < 8; ++j) {
          const int mj = m0 + key_of(j);
          if (mj >= a.M) continue;
          const int bj = mj / a.L, tj = mj % a.L;
          out[vt_index(bj, sg.heads, hh, dd, tj & ~15) + vt_col(tj & 15)] = ct[key_of(j) * S::LDC + nl];
        }
      }
    }
    // the columns of keys L .. 64*tiles-1 of the last tile are written as
    // zeros, so that whole tiles can be staged without masking V
    const int rem = a.L & 63;
    if (rem != 0) {
      const int b_hi = min(a.M - 1, m0 + S::BM - 1) / a.L;
      for (int b = m0 / a.L; b <= b_hi; ++b) {
        const int last = b * a.L + a.L - 1;  // the block holding a sequence's last token pads it
        if (last < m0 || last >= m0 + S::BM || last >= a.M) continue;
        const int t_tile = (a.L - 1) & ~63;
        for (int c = threadIdx.x; c < (64 - rem) * S::BN; c += 256) {
          const int nl = c % S::BN, p = rem + c / S::BN;
          const int col = n0 + nl;
          if (col >= a.N) continue;
          const ProjSeg sg = seg_of(col);
          if (!sg.transposed) continue;
          const int cl = col - sg.n_begin;
          const int hh = sg.head_base + cl / a.D, dd = cl % a.D;
          static_cast<T*>(sg.out)[vt_index(b, sg.heads, hh, dd, t_tile + (p & ~15)) + vt_col(p & 15)] = T(0);
        }
      }
    }
  }
  // element offset of (b, head, dim, 16-aligned key t) in [B, heads, tiles, D, 64]
  __device__ __forceinline__ size_t vt_index(int b, int heads, int hh, int dd, int t) const {
    return ((static_cast<size_t>(b) * heads + hh) * a.vt_tiles + t / 64) * a.D * 64 +
           static_cast<size_t>(dd) * 64 + (t & 63);
  }
  // column of key position p (< 16) inside its 16-key group
  static __device__ __forceinline__ int vt_col(int p) {
    return (p & 3) | ((p & 4) << 1) | ((p & 8) >> 1);
  }
};


// Tile of a 2-D grid of (N tiles) x (M tiles).  Blocks go to the 8 XCDs
// round-robin in launch order; when the row tiles come in whole groups of 8,
// the tiles are renumbered so that every column tile of a row block runs on
// the same XCD and its L2 serves the A rows to all of them.
__device__ __forceinline__ void xcd_tile(int& row_tile, int& col_tile) {
  const int nx = gridDim.x;
  row_tile = blockIdx.y;
  col_tile = blockIdx.x;
  if ((gridDim.y & 7) == 0) {
    const int lin = blockIdx.x + blockIdx.y * nx;
    const int sx = lin >> 3;
    row_tile = (sx / nx) * 8 + (lin & 7);
    col_tile = sx % nx;
  }
}

template <typename T, class S>
__global__ __launch_bounds__(256) void dense_proj_kernel(DenseArgs args) {
  extern __shared__ __align__(16) char smem[];
  int rt, ct;
  xcd_tile(rt, ct);
  DenseProb<T, S> prob(args, rt * S::BM, ct * S::BN);
  gemm_block<T, S>(prob, smem);
}

// ---------------------------------------------------------------------------
// gathered routed-query projection over the dispatch lists
// ---------------------------------------------------------------------------
struct GatherArgs {
  const void* x;
  const void* wq;
  void* q;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* pos;
  const int32_t* slot;
  const int32_t* tile_off;
  int n_lists, L, d, G, E, D, H;
  int koff[kMaxGroups + 1];  // group g's slot-heads start at koff[g]
  RopeTable rope;
  uint32_t* dbg;             // debug word (index checks of debug builds)
};

template <typename T, class S>
struct GatherProb {
  const GatherArgs& a;
  int K, m0, cnt, base, b, g, e;
  __device__ GatherProb(const GatherArgs& args, int tile_in_list, int li)
      : a(args), K(args.d) {
    m0 = tile_in_list * S::BM;
    cnt = args.counts[li];
    base = args.offsets[li];
    const int GE = args.G * args.E;
    b = li / GE;
    g = (li / args.E) % args.G;
    e = li % args.E;
    // the lists of (b, g) fill entries lb .. lb + L*k_g - 1
    const long long lb = (static_cast<long long>(b) * args.koff[args.G] + args.koff[g]) * args.L;
    const long long rows = static_cast<long long>(args.L) * (args.koff[g + 1] - args.koff[g]);
    if (!dbg_ok(m0 >= 0 && cnt >= 0 && cnt <= args.L && base >= lb && base + cnt <= lb + rows,
                args.dbg, kDbgListRange))
      cnt = 0;  // the block computes nothing and writes nothing
  }
  __device__ __forceinline__ const T* a_any() const { return static_cast<const T*>(a.x); }
  __device__ __forceinline__ const T* b_any() const { return static_cast<const T*>(a.wq); }
  __device__ __forceinline__ const T* a_row(int r) const {
    if (m0 + r >= cnt) return nullptr;
    const int t = a.pos[base + m0 + r];
    if (!dbg_ok(t >= 0 && t < a.L, a.dbg, kDbgPos)) return nullptr;
    return static_cast<const T*>(a.x) + (static_cast<size_t>(b) * a.L + t) * a.d;
  }
  __device__ __forceinline__ const T* b_row(int n) const {
    if (n >= a.D) return nullptr;
    return static_cast<const T*>(a.wq) +
           (static_cast<size_t>(g * a.E + e) * a.D + n) * static_cast<size_t>(a.d);
  }
  // a routed row is turned by its position pos; its columns are the head's dims
  __device__ __forceinline__ bool rotating() const { return a.rope.on != 0; }
  __device__ __forceinline__ float rotate(int r, int c, float v, float partner) const {
    if (m0 + r >= cnt || c >= a.D) return v;
    float cs, sn;
    rope_cs(a.pos[base + m0 + r], a.rope.theta[c >> 1], cs, sn);
    return rope_apply(v, partner, c, cs, sn);
  }
  // each routed row lands at (slot-head koff[g] + slot, position pos): 8 dims per chunk
  __device__ __forceinline__ void write_tile(const T* ct) const {
    constexpr int CW = S::BN / 8;
    for (int c = threadIdx.x; c < S::BM * CW; c += 256) {
      const int r = c / CW, c8 = c % CW;
      if (m0 + r >= cnt || 8 * c8 >= a.D) continue;
      const int entry = base + m0 + r;
      const int t = a.pos[entry], j = a.slot[entry];
      if (!dbg_ok(t >= 0 && t < a.L, a.dbg, kDbgPos) ||
          !dbg_ok(j >= 0 && j < a.koff[g + 1] - a.koff[g], a.dbg, kDbgSlot))
        continue;
      T* dst = static_cast<T*>(a.q) + ((static_cast<size_t>(b) * a.H + a.koff[g] + j) * a.L + t) * a.D + 8 * c8;
      copy8(dst, ct + r * S::LDC + 8 * c8);
    }
  }
};

// ---------------------------------------------------------------------------
// the whole GQE projection in one launch: the dense tiles (shared-head Q, K,
// V^T) first, then the gathered routed-query tiles.  Neither depends on the
// other, so one grid covers both and the gathered tiles fill the compute
// units the dense ones leave idle.
//
// Gathered tiles come in one of two orders.  Launches of more blocks than
// the chip holds at once, on sequences up to 2^18 tokens, order them tile
// index first, then list: block i of
// every (b, g, e) list runs at about the same time, and with loads near k/E
// of the tokens the i-th tiles of all lists cover about the same token
// window, so each token's x row, which k*G lists read, is fetched from HBM
// once and found in L2 by the other lists.  Every list then gets
// `per` = ceil(L / rows) slots (a list holds at most L entries); slots past
// its length exit at once.  Other launches pack the tiles of each (b, g)
// one list after another in `per` slots (an upper bound of the (b, g)'s
// total): small ones run all blocks at once anyway, and on the longest
// sequences a skewed expert load puts the lists' i-th tiles far apart, so a
// list read in order is the more local walk over x.
// ---------------------------------------------------------------------------
template <typename T, class SD, class SG>
__global__ __launch_bounds__(256) void project_kernel(DenseArgs dargs, GatherArgs gargs,
                                                      int dense_nx, int dense_blocks, int per,
                                                      int by_tile) {
  extern __shared__ __align__(16) char smem[];
  const int bid = blockIdx.x;
  if (bid < dense_blocks) {
    int rb = bid / dense_nx, c = bid % dense_nx;
    if (by_tile == 2) {  // all column tiles of a row block on one XCD
      const int sx = bid >> 3;
      rb = (sx / dense_nx) * 8 + (bid & 7);
      c = sx % dense_nx;
    }
    DenseProb<T, SD> prob(dargs, rb * SD::BM, c * SD::BN);
    gemm_block<T, SD>(prob, smem);
    return;
  }
  const int gb = bid - dense_blocks;
  int tile, bg, e;
  if (by_tile) {
    tile = gb / gargs.n_lists;
    int li = gb % gargs.n_lists;
    if (by_tile == 2) {  // tile i of every list on XCD i % 8
      const int sx = gb >> 3;
      tile = (sx / gargs.n_lists) * 8 + (gb & 7);
      li = sx % gargs.n_lists;
    }
    bg = li / gargs.E;
    e = li % gargs.E;
    const int* toff = gargs.tile_off + bg * (gargs.E + 1);  // tile map of this (b, g)
    if (tile >= toff[e + 1] - toff[e]) return;              // whole block leaves together
  } else {
    const int slot = gb % per;
    bg = gb / per;
    const int* toff = gargs.tile_off + bg * (gargs.E + 1);
    if (slot >= toff[gargs.E]) return;
    e = 0;  // last e with toff[e] <= slot
    while (e + 1 < gargs.E && toff[e + 1] <= slot) ++e;
    tile = slot - toff[e];
  }
  GatherProb<T, SG> prob(gargs, tile, bg * gargs.E + e);
  gemm_block<T, SG>(prob, smem);
}

// ---------------------------------------------------------------------------
// short sequences: the router's blocks, then the dense projection's tiles, in
// one grid.  The routing and the projection of every query head, K and V^T
// are independent, so the router's latency hides behind the GEMM tiles, and
// the attention that follows reads each slot-head's query row through the
// routing indices.  Tiles run in the XCD-aware order of xcd_tile when the
// router blocks come in whole groups of 8.
// ---------------------------------------------------------------------------
template <class S, int NE>
__global__ __launch_bounds__(256) void front_kernel(RouterArgs r, DenseArgs dargs,
                                                    int router_blocks, int dense_nx,
                                                    int dense_ny) {
  extern __shared__ __align__(16) char smem[];
  const int bid = blockIdx.x;
  if (bid < router_blocks) {  // the router's LDS overlays the GEMM ring's
    router_bf16_block<NE, 4, 1>(bid, *reinterpret_cast<RouterSmem<NE, 4, 1>*>(smem),
                                static_cast<const bf16_t*>(dargs.x), r.wr, r.bias, r.idx, r.w,
                                dargs.M, dargs.K, r.G, r.E, r.gk, r.renorm);
    return;
  }
  const int t = bid - router_blocks;
  int rb = t / dense_nx, c = t % dense_nx;
  if ((dense_ny & 7) == 0 && (router_blocks & 7) == 0) {  // a row block's tiles on one XCD
    const int sx = t >> 3;
    rb = (sx / dense_nx) * 8 + (t & 7);
    c = sx % dense_nx;
  }
  DenseProb<bf16_t, S> prob(dargs, rb * S::BM, c * S::BN);
  gemm_block<bf16_t, S>(prob, smem);
}

// ---------------------------------------------------------------------------
// output projection (row-major)
// ---------------------------------------------------------------------------
struct OutArgs {
  const void* a;
  const void* w;
  void* out;
  int M, N, K;
  // the weighted slot formed in the main loop (bf16, d_h 64), or NULL: the
  // router weights [M, wslot_k] and the slot buffer (a) it is also stored to
  const float* wslot_w;
  int wslot_k;
};

template <typename T, class S>
struct OutProb {
  const OutArgs& a;
  int m0, n0, K;
  __device__ OutProb(const OutArgs& args, int m0_, int n0_) : a(args), m0(m0_), n0(n0_), K(args.K) {}
  __device__ __forceinline__ const T* a_any() const { return static_cast<const T*>(a.a); }
  __device__ __forceinline__ const T* b_any() const { return static_cast<const T*>(a.w); }
  __device__ __forceinline__ const T* a_row(int r) const {
    const int m = m0 + r;
    return m < a.M ? static_cast<const T*>(a.a) + static_cast<size_t>(m) * a.K : nullptr;
  }
  __device__ __forceinline__ const T* b_row(int n) const {
    const int c = n0 + n;
    return c < a.N ? static_cast<const T*>(a.w) + static_cast<size_t>(c) * a.K : nullptr;
  }
  __device__ __forceinline__ void write_tile(const T* ct) const {
    constexpr int CW = S::BN / 8;
    for (int c = threadIdx.x; c < S::BM * CW; c += 256) {
      const int r = c / CW, c8 = c % CW;
      const int m = m0 + r, n = n0 + 8 * c8;
      if (m >= a.M || n >= a.N) continue;
      copy8(static_cast<T*>(a.out) + static_cast<size_t>(m) * a.N + n, ct + r * S::LDC + 8 * c8);
    }
  }
};

template <typename T, class S>
__global__ __launch_bounds__(256) void out_proj_kernel(OutArgs args) {
  extern __shared__ __align__(16) char smem[];
  int rt, ct;
  xcd_tile(rt, ct);
  OutProb<T, S> prob(args, rt * S::BM, ct * S::BN);
  gemm_block<T, S>(prob, smem);
}

// The output projection with the weighted slot formed in its main loop (bf16,
// d_h 64: slot h is K step h).  The slot's A chunks never come from HBM: the
// weighted-slot kernel's pass over the hard slots is folded into the K steps
// that stream them anyway.  The first column tile also stores the slot into
// the slot buffer, so the workspace holds what the separate kernel writes.
template <typename T, class S>
struct OutWsProb : OutProb<T, S> {
  typedef OutProb<T, S> Base;
  __device__ OutWsProb(const OutArgs& args, int m0_, int n0_) : Base(args, m0_, n0_) {}
  // hard slots; the tile's weight rows and how many of them exist
  __device__ __forceinline__ int wslot_k() const { return this->a.wslot_k; }
  __device__ __forceinline__ const float* wslot_rows() const {
    return this->a.wslot_w + static_cast<size_t>(this->m0) * this->a.wslot_k;
  }
  __device__ __forceinline__ int wslot_valid_rows() const { return min(S::BM, this->a.M - this->m0); }
  // one 8-element chunk of tile row r's weighted slot
  __device__ __forceinline__ void wslot_store(int r, int chunk, const bf16x8& v) const {
    const int m = this->m0 + r;
    if (this->n0 != 0 || m >= this->a.M) return;
    *reinterpret_cast<bf16x8*>(static_cast<bf16_t*>(const_cast<void*>(this->a.a)) +
                               static_cast<size_t>(m) * this->a.K + (this->a.wslot_k + 1) * 64 +
                               8 * chunk) = v;
  }
};

template <typename T, class S>
__global__ __launch_bounds__(256) void out_wslot_kernel(OutArgs args) {
  extern __shared__ __align__(16) char smem[];
  int rt, ct;
  xcd_tile(rt, ct);
  OutWsProb<T, S> prob(args, rt * S::BM, ct * S::BN);
  gemm_block<T, S>(prob, smem);
}

// ---------------------------------------------------------------------------
// general NT product with float32 results (the backward pass)
// ---------------------------------------------------------------------------
template <typename T, class S>
struct NtProb {
  const NtArgs& a;
  int m0, n0, K, z, k0;
  __device__ NtProb(const NtArgs& args, int m0_, int n0_, int z_)
      : a(args), m0(m0_), n0(n0_), z(z_), k0(args.splits > 1 ? z_ * args.kchunk : 0) {
    K = args.splits > 1 ? min(args.kchunk, args.K - k0) : args.K;
  }
  __device__ __forceinline__ const T* a_any() const { return static_cast<const T*>(a.a); }
  __device__ __forceinline__ const T* b_any() const { return static_cast<const T*>(a.b); }
  __device__ __forceinline__ const T* a_row(int r) const {
    const int m = m0 + r;
    return m < a.M ? static_cast<const T*>(a.a) + static_cast<size_t>(m) * a.lda + k0 : nullptr;
  }
  __device__ __forceinline__ const T* b_row(int n) const {
    const int c = n0 + n;
    return c < a.N ? static_cast<const T*>(a.b) + static_cast<size_t>(c) * a.ldb + k0 : nullptr;
  }
  __device__ __forceinline__ void store_acc(int r, int c, float v) const {
    const int m = m0 + r, n = n0 + c;
    if (m >= a.M || n >= a.N) return;
    if (a.splits > 1) {
      a.part[(static_cast<size_t>(z) * a.M + m) * a.N + n] = v;
      return;
    }
    for (int i = 0; i < a.nseg; ++i) {
      const NtSeg& sg = a.seg[i];
      if (m >= sg.row_begin && m < sg.row_begin + sg.rows) {
        float* o = sg.out + static_cast<size_t>(m - sg.row_begin) * sg.ldo + n;
        *o = sg.accumulate ? *o + v : v;
        return;
      }
    }
  }
};

template <typename T, class S>
__global__ __launch_bounds__(256) void nt_gemm_kernel(NtArgs args) {
  extern __shared__ __align__(16) char smem[];
  int rt, ct;
  xcd_tile(rt, ct);  // each z layer is a whole number of 8-block rounds when it remaps
  NtProb<T, S> prob(args, rt * S::BM, ct * S::BN, blockIdx.z);
  gemm_block<T, S>(prob, smem);
}

// the split-K partials summed in split order, then stored like store_acc
__global__ __launch_bounds__(256) void nt_split_reduce_kernel(NtArgs a, int zs) {
  const size_t mn = static_cast<size_t>(a.M) * a.N;
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= mn) return;
  float v = a.part[i];
  for (int z = 1; z < zs; ++z) v += a.part[z * mn + i];
  const int m = static_cast<int>(i / a.N), n = static_cast<int>(i % a.N);
  for (int s = 0; s < a.nseg; ++s) {
    const NtSeg& sg = a.seg[s];
    if (m >= sg.row_begin && m < sg.row_begin + sg.rows) {
      float* o = sg.out + static_cast<size_t>(m - sg.row_begin) * sg.ldo + n;
      *o = sg.accumulate ? *o + v : v;
      return;
    }
  }
}

// ---------------------------------------------------------------------------
// weighted slot: s[t, (kG+1)D + c] = sum_{g,j} w[t, g, j] * s[t, (g k + j) D + c]
// (gist.science, Architectuur en Routing: weighted sum of the selected
// experts' outputs with the router weights; a plain sum over groups)
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void weighted_slot_item(size_t gid, T* __restrict__ s,
                                                   const float* __restrict__ w, int n_tokens,
                                                   int K, int D) {
  const int per_tok = D / 4;
  if (gid >= static_cast<size_t>(n_tokens) * per_tok) return;
  const int t = static_cast<int>(gid / per_tok);
  const int c = static_cast<int>(gid % per_tok) * 4;
  const int slots = K;
  T* row = s + static_cast<size_t>(t) * (slots + 2) * D;
  const float* wt = w + static_cast<size_t>(t) * slots;
  float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
  for (int h = 0; h < slots; ++h) {
    const float wh = wt[h];
    const T* src = row + h * D + c;
    acc0 = fmaf(wh, to_f32(src[0]), acc0);
    acc1 = fmaf(wh, to_f32(src[1]), acc1);
    acc2 = fmaf(wh, to_f32(src[2]), acc2);
    acc3 = fmaf(wh, to_f32(src[3]), acc3);
  }
  T* dst = row + (slots + 1) * D + c;
  dst[0] = from_f32<T>(acc0);
  dst[1] = from_f32<T>(acc1);
  dst[2] = from_f32<T>(acc2);
  dst[3] = from_f32<T>(acc3);
}

template <typename T>
__global__ __launch_bounds__(256) void weighted_slot_kernel(T* __restrict__ s,
                                                            const float* __restrict__ w,
                                                            int n_tokens, int K, int D) {
  weighted_slot_item<T>(static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x, s, w,
                        n_tokens, K, D);
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// launch with S::LDS bytes of dynamic LDS (above 64 KB the kernel must opt in once)
template <class S, class Kern, class Args>
static hipError_t launch_gemm(Kern kern, dim3 grid, hipStream_t stream, const Args& a) {
  if (S::LDS > 65536) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS);
    if (attr != hipSuccess) return attr;
  }
  hipLaunchKernelGGL(kern, grid, dim3(256), S::LDS, stream, a);
  return hipGetLastError();
}

// Launches whose blocks all fit on the chip at once get four LDS stages (three
// K steps in flight: latency hiding within the block); larger ones get two
// stages, so that two blocks share a CU and hide each other's prologue and
// epilogue.
int cu_count() {
  static int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    return v;
  }();
  return n;
}
inline bool deep_ring(long long blocks) { return blocks <= cu_count(); }

// Tile shapes of an M x N output: 128 x 128 tiles while they fill the chip;
// below one tile per compute unit, 64-row tiles (twice the blocks; every
// output element still takes the same K steps in the same order, so the
// results are the same).  A launch that fits the chip at once gets the
// four-stage LDS ring.
enum class Tiles { k128, k128Deep, k64, k64Deep };
inline Tiles choose_tiles(int M, int N) {
  const long long b128 = static_cast<long long>((N + 127) / 128) * ((M + 127) / 128);
  if (b128 < cu_count()) {
    const long long b64 = static_cast<long long>((N + 127) / 128) * ((M + 63) / 64);
    return deep_ring(b64) ? Tiles::k64Deep : Tiles::k64;
  }
  return deep_ring(b128) ? Tiles::k128Deep : Tiles::k128;
}
inline dim3 tile_grid(Tiles t, int M, int N) {
  const int bm = (t == Tiles::k64 || t == Tiles::k64Deep) ? 64 : 128;
  return dim3((N + 127) / 128, (M + bm - 1) / bm);
}
#define GQE_LAUNCH_TILED(KERNEL, T, M, N, stream, args) \
  GQE_LAUNCH_TILED_Z(KERNEL, T, M, N, 1, stream, args)
#define GQE_LAUNCH_TILED_Z(KERNEL, T, M, N, Z, stream, args)                                   \
  do {                                                                                       \
    const Tiles t_ = choose_tiles(M, N);                                                     \
    dim3 g_ = tile_grid(t_, M, N);                                                           \
    g_.z = (Z);                                                                              \
    switch (t_) {                                                                            \
      case Tiles::k64: {                                                                     \
        typedef GemmShape<T, 64, 128, 2, 2> S_;                                              \
        return launch_gemm<S_>(KERNEL<T, S_>, g_, stream, args);                             \
      }                                                                                      \
      case Tiles::k64Deep: {                                                                 \
        typedef GemmShape<T, 64, 128, 2, 2, 4> S_;                                           \
        return launch_gemm<S_>(KERNEL<T, S_>, g_, stream, args);                             \
      }                                                                                      \
      case Tiles::k128Deep: {                                                                \
        typedef GemmShape<T, 128, 128, 2, 2, 4> S_;                                          \
        return launch_gemm<S_>(KERNEL<T, S_>, g_, stream, args);                             \
      }                                                                                      \
      default: {                                                                             \
        typedef GemmShape<T, 128, 128, 2, 2> S_;                                             \
        return launch_gemm<S_>(KERNEL<T, S_>, g_, stream, args);                             \
      }                                                                                      \
    }                                                                                        \
  } while (0)

template <typename T>
hipError_t launch_dense_proj(const T* x, int M, int K, int L, int D, int64_t vt_tiles,
                             const ProjSeg* segs, int nseg, const RopeTable& rope,
                             hipStream_t stream) {
  DenseArgs a;
  a.rope = rope;
  a.x = x;
  a.M = M;
  a.K = K;
  a.L = L;
  a.D = D;
  a.vt_tiles = vt_tiles;
  a.nseg = nseg;
  int N = 0;
  for (int i = 0; i < nseg; ++i) {
    a.seg[i] = segs[i];
    N = segs[i].n_begin + segs[i].n;
  }
  a.N = N;
  if (M == 0 || N == 0) return hipSuccess;
  GQE_LAUNCH_TILED(dense_proj_kernel, T, M, N, stream, a);
}

template <typename T, class SD, class SG>
static hipError_t launch_project_s(const DenseArgs& d, const GatherArgs& g, int per,
                                   int by_tile, hipStream_t stream) {
  const int nx = (d.N + SD::BN - 1) / SD::BN;
  const int dense_blocks = d.N == 0 || d.M == 0 ? 0 : nx * ((d.M + SD::BM - 1) / SD::BM);
  const long long blocks =
      dense_blocks + static_cast<long long>(per) * (by_tile ? g.n_lists : g.n_lists / g.E);
  if (blocks == 0) return hipSuccess;
  constexpr int lds = SD::LDS > SG::LDS ? SD::LDS : SG::LDS;
  auto kern = project_kernel<T, SD, SG>;
  if (lds > 65536) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(256), lds, stream, d, g,
                     nx > 0 ? nx : 1, dense_blocks, per, by_tile);
  return hipGetLastError();
}

// Dense tiles: 128 x 128 while the whole launch fills the chip, else 64-row
// tiles (the same K steps in the same order per output element); the
// four-stage ring when every block of the launch is resident at once.
template <typename T, int D>
static hipError_t launch_project_d(const DenseArgs& d, const GatherArgs& g, int kmax,
                                   hipStream_t stream) {
  constexpr int WGM = D >= 128 ? 2 : 4, WGN = D >= 128 ? 2 : 1;
  const int n_bg = g.E == 0 ? 0 : g.n_lists / g.E;
  // packed: a (b, g) has at most L*kmax routed rows, in at most E partial tiles
  const int packed = static_cast<int>((static_cast<long long>(g.L) * kmax + kGatherRows - 1) / kGatherRows) + g.E;
  const int per_list = (g.L + kGatherRows - 1) / kGatherRows;
  const long long nx = (d.N + 127) / 128;
  long long gblocks = static_cast<long long>(packed) * n_bg;
  // tile-index order where the launch exceeds what the chip holds, up to
  // L = 2^18 (beyond that, under a skewed load the lists' i-th tiles lie far
  // apart in the sequence and the packed order reads x more locally)
  const bool by_tile = nx * ((d.M + 127) / 128) + gblocks > 2LL * cu_count() && g.L <= (1 << 18);
  int per = packed;
  if (by_tile) {
    per = per_list;
    gblocks = static_cast<long long>(per_list) * g.n_lists;
  }
  // blocks go to the XCDs round-robin: with whole groups of 8 row blocks and
  // 8 tiles per list, the mapping can keep the blocks that read the same x
  // rows on one XCD's L2
  const int xcd = by_tile && ((d.M + 127) / 128) % 8 == 0 && per_list % 8 == 0 ? 2 : (by_tile ? 1 : 0);
  const long long b128 = nx * ((d.M + 127) / 128) + gblocks;
  const bool small = b128 < cu_count();
  const long long total = small ? nx * ((d.M + 63) / 64) + gblocks : b128;
  if (deep_ring(total)) {
    typedef GemmShape<T, kGatherRows, D, WGM, WGN, 4> SG;
    return small ? launch_project_s<T, GemmShape<T, 64, 128, 2, 2, 4>, SG>(d, g, per, by_tile ? 1 : 0, stream)
                 : launch_project_s<T, GemmShape<T, 128, 128, 2, 2, 4>, SG>(d, g, per, xcd, stream);
  }
  typedef GemmShape<T, kGatherRows, D, WGM, WGN> SG;
  return small ? launch_project_s<T, GemmShape<T, 64, 128, 2, 2>, SG>(d, g, per, by_tile ? 1 : 0, stream)
               : launch_project_s<T, GemmShape<T, 128, 128, 2, 2>, SG>(d, g, per, xcd, stream);
}

template <typename T>
hipError_t launch_project(const T* x, int M, int K, int L, int D, int64_t vt_tiles,
                          const ProjSeg* segs, int nseg, const T* wq, T* q,
                          const int32_t* counts, const int32_t* offsets, const int32_t* pos,
                          const int32_t* slot, const int32_t* tile_off, int B, int G, int E,
                          const GroupK& gk, const RopeTable& rope, uint32_t* dbg,
                          hipStream_t stream) {
  DenseArgs d;
  d.rope = rope;
  d.x = x;
  d.M = M;
  d.K = K;
  d.L = L;
  d.D = D;
  d.vt_tiles = vt_tiles;
  d.nseg = nseg;
  int N = 0;
  for (int i = 0; i < nseg; ++i) {
    d.seg[i] = segs[i];
    N = segs[i].n_begin + segs[i].n;
  }
  d.N = N;
  GatherArgs g;
  g.rope = rope;
  g.x = x;
  g.wq = wq;
  g.q = q;
  g.counts = counts;
  g.offsets = offsets;
  g.pos = pos;
  g.slot = slot;
  g.tile_off = tile_off;
  g.dbg = dbg;
  g.n_lists = B * G * E;
  g.L = L;
  g.d = K;
  g.G = G;
  g.E = E;
  for (int i = 0; i <= G; ++i) g.koff[i] = gk.koff[i];
  g.D = D;
  g.H = gk.K + 1;
  if (B * G == 0) g.n_lists = 0;
  switch (D) {
    case 32: return launch_project_d<T, 32>(d, g, gk.kmax, stream);
    case 64: return launch_project_d<T, 64>(d, g, gk.kmax, stream);
    case 128: return launch_project_d<T, 128>(d, g, gk.kmax, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class S, int NE>
static hipError_t launch_front_s(const RouterArgs& r, const DenseArgs& d, hipStream_t stream) {
  const int router_blocks = (d.M + 15) / 16;
  const int nx = (d.N + S::BN - 1) / S::BN, ny = (d.M + S::BM - 1) / S::BM;
  auto kern = front_kernel<S, NE>;
  constexpr int lds = sizeof(RouterSmem<NE, 4, 1>) > S::LDS ? sizeof(RouterSmem<NE, 4, 1>) : S::LDS;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(router_blocks + nx * ny)), dim3(256), lds,
                     stream, r, d, router_blocks, nx, ny);
  return hipGetLastError();
}

template <int NE>
static hipError_t launch_front_ne(const RouterArgs& r, const DenseArgs& d, hipStream_t stream) {
  switch (choose_tiles(d.M, d.N)) {
    case Tiles::k64: return launch_front_s<GemmShape<bf16_t, 64, 128, 2, 2>, NE>(r, d, stream);
    case Tiles::k64Deep: return launch_front_s<GemmShape<bf16_t, 64, 128, 2, 2, 4>, NE>(r, d, stream);
    case Tiles::k128Deep: return launch_front_s<GemmShape<bf16_t, 128, 128, 2, 2, 4>, NE>(r, d, stream);
    default: return launch_front_s<GemmShape<bf16_t, 128, 128, 2, 2>, NE>(r, d, stream);
  }
}

hipError_t launch_front(const RouterArgs& r, const bf16_t* x, int M, int K, int L, int D,
                        int64_t vt_tiles, const ProjSeg* segs, int nseg, const RopeTable& rope,
                        hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int GE = r.G * r.E;
  if (K % 128 != 0 || GE > 64 || GE <= 0 || M > kFrontMaxTokens) return hipErrorInvalidValue;
  DenseArgs d;
  d.rope = rope;
  d.x = x;
  d.M = M;
  d.K = K;
  d.L = L;
  d.D = D;
  d.vt_tiles = vt_tiles;
  d.nseg = nseg;
  int N = 0;
  for (int i = 0; i < nseg; ++i) {
    d.seg[i] = segs[i];
    N = segs[i].n_begin + segs[i].n;
  }
  d.N = N;
  switch ((GE + 15) / 16) {
    case 1: return launch_front_ne<1>(r, d, stream);
    case 2: return launch_front_ne<2>(r, d, stream);
    case 3: return launch_front_ne<3>(r, d, stream);
    default: return launch_front_ne<4>(r, d, stream);
  }
}

template <typename T>
hipError_t launch_out_proj(const T* a_, const T* wo, T* out, int M, int N, int K,
                           hipStream_t stream) {
  OutArgs a{};
  a.a = a_;
  a.w = wo;
  a.out = out;
  a.M = M;
  a.N = N;
  a.K = K;
  if (M == 0 || N == 0) return hipSuccess;
  GQE_LAUNCH_TILED(out_proj_kernel, T, M, N, stream, a);
}

// dynamic LDS of the in-loop weighted slot: the ring, then the weight rows
template <class S>
static hipError_t launch_out_wslot_s(const OutArgs& a, hipStream_t stream) {
  constexpr int ring = S::NST * S::STAGE;
  constexpr int cap = ring + S::BM * kWslotMaxK * 4 > S::LDS ? ring + S::BM * kWslotMaxK * 4 : S::LDS;
  const int need = ring + S::BM * a.wslot_k * 4;
  const int lds = need > S::LDS ? need : S::LDS;
  auto kern = out_wslot_kernel<bf16_t, S>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, cap);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, tile_grid(choose_tiles(a.M, a.N), a.M, a.N), dim3(256), lds, stream, a);
  return hipGetLastError();
}

bool out_wslot_ok(int K, int D, int hard) {
  return D == 64 && hard > 0 && hard <= kWslotMaxK && hard % 4 == 0 && K == (hard + 2) * D;
}

hipError_t launch_out_proj_wslot(bf16_t* s, const float* w, const bf16_t* wo, bf16_t* out, int M,
                                 int N, int K, int D, int hard, hipStream_t stream) {
  if (!out_wslot_ok(K, D, hard)) return hipErrorInvalidValue;
  OutArgs a{};
  a.a = s;
  a.w = wo;
  a.out = out;
  a.M = M;
  a.N = N;
  a.K = K;
  a.wslot_w = w;
  a.wslot_k = hard;
  if (M == 0 || N == 0) return hipSuccess;
  switch (choose_tiles(M, N)) {
    case Tiles::k64: return launch_out_wslot_s<GemmShape<bf16_t, 64, 128, 2, 2>>(a, stream);
    case Tiles::k64Deep: return launch_out_wslot_s<GemmShape<bf16_t, 64, 128, 2, 2, 4>>(a, stream);
    case Tiles::k128Deep: return launch_out_wslot_s<GemmShape<bf16_t, 128, 128, 2, 2, 4>>(a, stream);
    default: return launch_out_wslot_s<GemmShape<bf16_t, 128, 128, 2, 2>>(a, stream);
  }
}

// The split count s minimizes the rounds of blocks over the compute units per
// unit of work, ceil(tiles * s / cu) / s, plus a small charge per split for
// writing and summing the partials; every split keeps at least 1024 of K.
int nt_gemm_splits(int M, int N, int K) {
  const dim3 g = tile_grid(choose_tiles(M, N), M, N);
  const long long tiles = static_cast<long long>(g.x) * g.y;
  const long long cu = cu_count();
  if (tiles == 0 || tiles >= cu || K < 2048) return 1;
  int best = 1;
  double best_cost = 1.0 + 0.02;
  for (int s = 2; s <= 8 && K / s >= 1024; ++s) {
    const double cost = static_cast<double>((tiles * s + cu - 1) / cu) / s + 0.02 * s;
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

template <typename T>
static hipError_t launch_nt_tiles(const NtArgs& a, int zs, hipStream_t stream) {
  GQE_LAUNCH_TILED_Z(nt_gemm_kernel, T, a.M, a.N, zs, stream, a);
}

// An NT product with float32 results.  With a.splits > 1 (and a.part), K is
// cut into chunks of whole LDS steps, one per grid layer, and a second kernel
// sums the partials in chunk order (deterministic).
template <typename T>
hipError_t launch_nt_gemm(const NtArgs& args, hipStream_t stream) {
  typedef GemmShape<T, 128, 128, 2, 2> S;
  if (args.M == 0 || args.N == 0) return hipSuccess;
  if (args.K % S::BKE != 0 || args.nseg < 1 || args.nseg > 4) return hipErrorInvalidValue;
  NtArgs a = args;
  if (a.splits <= 1 || a.part == nullptr || a.K == 0) {
    a.splits = 1;
    return launch_nt_tiles<T>(a, 1, stream);
  }
  a.kchunk = ((a.K + a.splits - 1) / a.splits + S::BKE - 1) / S::BKE * S::BKE;
  const int zs = (a.K + a.kchunk - 1) / a.kchunk;
  a.splits = zs;
  if (zs <= 1) return launch_nt_tiles<T>(a, 1, stream);
  const hipError_t e = launch_nt_tiles<T>(a, zs, stream);
  if (e != hipSuccess) return e;
  const size_t mn = static_cast<size_t>(a.M) * a.N;
  hipLaunchKernelGGL(nt_split_reduce_kernel, dim3(static_cast<unsigned>((mn + 255) / 256)),
                     dim3(256), 0, stream, a, zs);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_weighted_slot(T* s, const float* w, int n_tokens, int K, int D,
                                hipStream_t stream) {
  const size_t n = static_cast<size_t>(n_tokens) * (D / 4);
  if (n == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  hipLaunchKernelGGL(weighted_slot_kernel<T>, dim3(blocks), dim3(256), 0, stream, s, w, n_tokens,
                     K, D);
  return hipGetLastError();
}

#define GQE_INST(T)                                                                              \
  template hipError_t launch_dense_proj<T>(const T*, int, int, int, int, int64_t, const ProjSeg*, \
                                           int, const RopeTable&, hipStream_t);                  \
  template hipError_t launch_project<T>(const T*, int, int, int, int, int64_t, const ProjSeg*,   \
                                        int, const T*, T*, const int32_t*, const int32_t*,       \
                                        const int32_t*, const int32_t*, const int32_t*, int, int, \
                                        int, const GroupK&, const RopeTable&, uint32_t*,         \
                                        hipStream_t);                                            \
  template hipError_t launch_out_proj<T>(const T*, const T*, T*, int, int, int, hipStream_t);    \
  template hipError_t launch_weighted_slot<T>(T*, const float*, int, int, int, hipStream_t);      \
  template hipError_t launch_nt_gemm<T>(const NtArgs&, hipStream_t);
GQE_INST(bf16_t)
GQE_INST(float)
#undef GQE_INST

}  // namespace gqe

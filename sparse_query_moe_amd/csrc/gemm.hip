// K3 and K5: the layer's projections on MFMA (bf16 -> fp32 accumulation, or
// fp32 throughout for float32 layers).
//
// Every product here has the "NT" form C[m, n] = sum_k A[m, k] * W[n, k]: the
// activations are row-major with K contiguous and the weights use the
// [out, in] layout, also K contiguous, so both MFMA operands are 16-byte
// vector loads along K.  A block computes a BM x BN tile with 4 waves; K
// streams through a double-buffered LDS stage of 128-byte rows (64 bf16 or
// 32 fp32 elements), swizzled per 16-byte chunk.  One barrier per K step: the
// next stage's global loads are issued before the current stage's MFMAs and
// written to the other LDS buffer after them.
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
#include "device_common.h"
#include "kernels.h"

namespace gqe {

namespace {

template <typename T, int BM_, int BN_, int WGM_, int WGN_>
struct GemmShape {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int EPC = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte chunk
  static constexpr int BKE = 8 * EPC;                            // K elements per LDS row
  static constexpr int A_CH = BM / 32;                           // A chunks per thread
  static constexpr int B_CH = BN / 32;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int STAGE = (BM + BN) * 128;
  static constexpr int LDS = 2 * STAGE;
  static_assert(WGM * WGN == 4, "4 waves");
  static_assert(TM >= 1 && TN >= 1, "wave tile at least 32x32");
};

// The main loop: P supplies K, a_row(r), b_row(n) (row pointers or nullptr
// for rows outside the problem, read as zeros) and store(r, n, value).
template <typename T, class S, class P>
__device__ __forceinline__ void gemm_block(const P& prob, char* smem) {
  typedef typename Frag<T>::type F;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int ch = tid & 7;
  const int r0 = tid >> 3;

  const T* ap[S::A_CH];
  const T* bp[S::B_CH];
#pragma unroll
  for (int i = 0; i < S::A_CH; ++i) ap[i] = prob.a_row(r0 + 32 * i);
#pragma unroll
  for (int i = 0; i < S::B_CH; ++i) bp[i] = prob.b_row(r0 + 32 * i);

  uint4 ra[S::A_CH], rb[S::B_CH];
  const int K = prob.K;
  const int nk = (K + S::BKE - 1) / S::BKE;

  auto gload = [&](int kt) {
    const int ke = kt * S::BKE + ch * S::EPC;
#pragma unroll
    for (int i = 0; i < S::A_CH; ++i)
      ra[i] = (ap[i] != nullptr && ke < K) ? *reinterpret_cast<const uint4*>(ap[i] + ke) : zero4();
#pragma unroll
    for (int i = 0; i < S::B_CH; ++i)
      rb[i] = (bp[i] != nullptr && ke < K) ? *reinterpret_cast<const uint4*>(bp[i] + ke) : zero4();
  };
  auto sstore = [&](int buf) {
    char* sa = smem + buf * S::STAGE;
    char* sb = sa + S::BM * 128;
#pragma unroll
    for (int i = 0; i < S::A_CH; ++i)
      *reinterpret_cast<uint4*>(sa + swz<128>(r0 + 32 * i, ch)) = ra[i];
#pragma unroll
    for (int i = 0; i < S::B_CH; ++i)
      *reinterpret_cast<uint4*>(sb + swz<128>(r0 + 32 * i, ch)) = rb[i];
  };

  f32x16 acc[S::TM][S::TN];
#pragma unroll
  for (int a = 0; a < S::TM; ++a)
#pragma unroll
    for (int b = 0; b < S::TN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  gload(0);
  sstore(0);
  lds_barrier();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload(kt + 1);
    const char* sa = smem + (kt & 1) * S::STAGE;
    const char* sb = sa + S::BM * 128;
#pragma unroll
    for (int ks = 0; ks < S::BKE / 16; ++ks) {
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
    if (kt + 1 < nk) sstore((kt + 1) & 1);
    lds_barrier();
  }

#pragma unroll
  for (int a = 0; a < S::TM; ++a)
#pragma unroll
    for (int b = 0; b < S::TN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        prob.store(wm * S::WM + 32 * a + acc_row(i, lane), wn * S::WN + 32 * b + (lane & 31),
                   acc[a][b][i]);
}

// ---------------------------------------------------------------------------
// dense projection with up to 3 output segments
// ---------------------------------------------------------------------------
struct DenseArgs {
  const void* x;
  int M, K, N, L, D;
  int64_t ld_t;
  int nseg;
  ProjSeg seg[3];
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
    return r;
  }
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
  __device__ __forceinline__ void store(int r, int n, float v) const {
    const int m = m0 + r, col = n0 + n;
    if (m >= a.M || col >= a.N) return;
    const ProjSeg sg = seg_of(col);
    const int c = col - sg.n_begin;
    const int hh = sg.head_base + c / a.D, dd = c % a.D;
    const int b = m / a.L, t = m % a.L;
    T* out = static_cast<T*>(sg.out);
    size_t o;
    if (sg.transposed)
      o = (static_cast<size_t>(b) * sg.heads + hh) * a.D * static_cast<size_t>(a.ld_t) +
          static_cast<size_t>(dd) * a.ld_t + t;
    else
      o = ((static_cast<size_t>(b) * sg.heads + hh) * a.L + t) * a.D + dd;
    out[o] = from_f32<T>(v);
  }
};

template <typename T, class S>
__global__ __launch_bounds__(256) void dense_proj_kernel(DenseArgs args) {
  extern __shared__ __align__(16) char smem[];
  DenseProb<T, S> prob(args, blockIdx.y * S::BM, blockIdx.x * S::BN);
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
  int n_lists, L, d, G, E, k, D, H;
};

template <typename T, class S>
struct GatherProb {
  const GatherArgs& a;
  int K, m0, cnt, base, b, g, e;
  __device__ GatherProb(const GatherArgs& args, int tile, int li)
      : a(args), K(args.d) {
    m0 = (tile - args.tile_off[li]) * S::BM;
    cnt = args.counts[li];
    base = args.offsets[li];
    const int GE = args.G * args.E;
    b = li / GE;
    g = (li / args.E) % args.G;
    e = li % args.E;
  }
  __device__ __forceinline__ const T* a_row(int r) const {
    if (m0 + r >= cnt) return nullptr;
    const int t = a.pos[base + m0 + r];
    return static_cast<const T*>(a.x) + (static_cast<size_t>(b) * a.L + t) * a.d;
  }
  __device__ __forceinline__ const T* b_row(int n) const {
    if (n >= a.D) return nullptr;
    return static_cast<const T*>(a.wq) +
           (static_cast<size_t>(g * a.E + e) * a.D + n) * static_cast<size_t>(a.d);
  }
  __device__ __forceinline__ void store(int r, int n, float v) const {
    if (m0 + r >= cnt || n >= a.D) return;
    const int entry = base + m0 + r;
    const int t = a.pos[entry], j = a.slot[entry];
    T* q = static_cast<T*>(a.q);
    q[((static_cast<size_t>(b) * a.H + g * a.k + j) * a.L + t) * a.D + n] = from_f32<T>(v);
  }
};

template <typename T, class S>
__global__ __launch_bounds__(256) void gather_q_kernel(GatherArgs args) {
  extern __shared__ __align__(16) char smem[];
  const int tile = blockIdx.x;
  if (tile >= args.tile_off[args.n_lists]) return;  // whole block leaves together
  int lo = 0, hi = args.n_lists;                     // last li with tile_off[li] <= tile
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (args.tile_off[mid] <= tile) lo = mid; else hi = mid;
  }
  GatherProb<T, S> prob(args, tile, lo);
  gemm_block<T, S>(prob, smem);
}

// ---------------------------------------------------------------------------
// output projection (row-major)
// ---------------------------------------------------------------------------
struct OutArgs {
  const void* a;
  const void* w;
  void* out;
  int M, N, K;
};

template <typename T, class S>
struct OutProb {
  const OutArgs& a;
  int m0, n0, K;
  __device__ OutProb(const OutArgs& args, int m0_, int n0_) : a(args), m0(m0_), n0(n0_), K(args.K) {}
  __device__ __forceinline__ const T* a_row(int r) const {
    const int m = m0 + r;
    return m < a.M ? static_cast<const T*>(a.a) + static_cast<size_t>(m) * a.K : nullptr;
  }
  __device__ __forceinline__ const T* b_row(int n) const {
    const int c = n0 + n;
    return c < a.N ? static_cast<const T*>(a.w) + static_cast<size_t>(c) * a.K : nullptr;
  }
  __device__ __forceinline__ void store(int r, int n, float v) const {
    const int m = m0 + r, c = n0 + n;
    if (m < a.M && c < a.N)
      static_cast<T*>(a.out)[static_cast<size_t>(m) * a.N + c] = from_f32<T>(v);
  }
};

template <typename T, class S>
__global__ __launch_bounds__(256) void out_proj_kernel(OutArgs args) {
  extern __shared__ __align__(16) char smem[];
  OutProb<T, S> prob(args, blockIdx.y * S::BM, blockIdx.x * S::BN);
  gemm_block<T, S>(prob, smem);
}

// ---------------------------------------------------------------------------
// weighted slot: s[t, (kG+1)D + c] = sum_{g,j} w[t, g, j] * s[t, (g k + j) D + c]
// (gist.science, Architectuur en Routing: weighted sum of the selected
// experts' outputs with the router weights; a plain sum over groups)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void weighted_slot_kernel(T* __restrict__ s,
                                                            const float* __restrict__ w,
                                                            int n_tokens, int G, int k, int D) {
  const int per_tok = D / 4;
  const size_t gid = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= static_cast<size_t>(n_tokens) * per_tok) return;
  const int t = static_cast<int>(gid / per_tok);
  const int c = static_cast<int>(gid % per_tok) * 4;
  const int slots = G * k;
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

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T>
hipError_t launch_dense_proj(const T* x, int M, int K, int L, int D, int64_t ld_t,
                             const ProjSeg* segs, int nseg, hipStream_t stream) {
  typedef GemmShape<T, 128, 128, 2, 2> S;
  DenseArgs a;
  a.x = x;
  a.M = M;
  a.K = K;
  a.L = L;
  a.D = D;
  a.ld_t = ld_t;
  a.nseg = nseg;
  int N = 0;
  for (int i = 0; i < nseg; ++i) {
    a.seg[i] = segs[i];
    N = segs[i].n_begin + segs[i].n;
  }
  a.N = N;
  if (M == 0 || N == 0) return hipSuccess;
  const dim3 grid((N + S::BN - 1) / S::BN, (M + S::BM - 1) / S::BM);
  hipLaunchKernelGGL((dense_proj_kernel<T, S>), grid, dim3(256), S::LDS, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_gather_q_d(const GatherArgs& a, int max_tiles, hipStream_t stream) {
  typedef GemmShape<T, kGatherRows, D, (D >= 128 ? 2 : 4), (D >= 128 ? 2 : 1)> S;
  hipLaunchKernelGGL((gather_q_kernel<T, S>), dim3(max_tiles), dim3(256), S::LDS, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gather_q(const T* x, const T* wq, T* q, const int32_t* counts,
                           const int32_t* offsets, const int32_t* pos, const int32_t* slot,
                           const int32_t* tile_off, int B, int L, int d, int G, int E, int k,
                           int D, int max_tiles, hipStream_t stream) {
  GatherArgs a;
  a.x = x;
  a.wq = wq;
  a.q = q;
  a.counts = counts;
  a.offsets = offsets;
  a.pos = pos;
  a.slot = slot;
  a.tile_off = tile_off;
  a.n_lists = B * G * E;
  a.L = L;
  a.d = d;
  a.G = G;
  a.E = E;
  a.k = k;
  a.D = D;
  a.H = G * k + 1;
  if (max_tiles == 0) return hipSuccess;
  switch (D) {
    case 32: return launch_gather_q_d<T, 32>(a, max_tiles, stream);
    case 64: return launch_gather_q_d<T, 64>(a, max_tiles, stream);
    case 128: return launch_gather_q_d<T, 128>(a, max_tiles, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_out_proj(const T* a_, const T* wo, T* out, int M, int N, int K,
                           hipStream_t stream) {
  typedef GemmShape<T, 128, 128, 2, 2> S;
  OutArgs a;
  a.a = a_;
  a.w = wo;
  a.out = out;
  a.M = M;
  a.N = N;
  a.K = K;
  if (M == 0 || N == 0) return hipSuccess;
  const dim3 grid((N + S::BN - 1) / S::BN, (M + S::BM - 1) / S::BM);
  hipLaunchKernelGGL((out_proj_kernel<T, S>), grid, dim3(256), S::LDS, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_weighted_slot(T* s, const float* w, int n_tokens, int G, int k, int D,
                                hipStream_t stream) {
  const size_t n = static_cast<size_t>(n_tokens) * (D / 4);
  if (n == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  hipLaunchKernelGGL(weighted_slot_kernel<T>, dim3(blocks), dim3(256), 0, stream, s, w, n_tokens,
                     G, k, D);
  return hipGetLastError();
}

#define GQE_INST(T)                                                                              \
  template hipError_t launch_dense_proj<T>(const T*, int, int, int, int, int64_t, const ProjSeg*, \
                                           int, hipStream_t);                                    \
  template hipError_t launch_gather_q<T>(const T*, const T*, T*, const int32_t*, const int32_t*, \
                                         const int32_t*, const int32_t*, const int32_t*, int, int, \
                                         int, int, int, int, int, int, hipStream_t);             \
  template hipError_t launch_out_proj<T>(const T*, const T*, T*, int, int, int, hipStream_t);    \
  template hipError_t launch_weighted_slot<T>(T*, const float*, int, int, int, int, hipStream_t);
GQE_INST(bf16_t)
GQE_INST(float)
#undef GQE_INST

}  // namespace gqe

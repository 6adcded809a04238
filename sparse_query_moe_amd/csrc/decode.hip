// Decode: one new token per sequence against a KV cache.
//
// The pages analyse prefill only (pptc.cn review, section 6, lists decode as
// not analysed).  A decode step is the same layer evaluated at one position:
// the token of sequence b at position pos[b] is routed (the prefill router
// kernel, on B tokens), its queries and its K/V are projected (K/V go straight
// into the cache at pos[b]), its query heads attend causally to the cached
// keys 0..pos[b], and the slots go through W_O.
//
// Decode moves the whole cache once per step and does O(1) work per byte, so
// every kernel here is a bandwidth kernel on the VALU, not an MFMA kernel:
//   decode_proj_kernel  one block per (sequence, projected head): the token's
//                       d_model-long row in LDS, one wave per output row at a
//                       time, 16-byte weight loads, a wave reduction.
//   decode_attn_kernel  split-K ("flash decoding"): one block per (sequence,
//                       KV group, chunk of keys); all query heads of the group
//                       share each K row and V^T tile read; a lane owns a key
//                       for the scores and a head dimension for P.V.
//   decode_combine_kernel  merges the chunk partials of one (sequence, head).
//   gemv_kernel         the W_O product of the B slot vectors.
#include <math.h>

#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace gqe {

namespace {

constexpr int kDecThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

// 8 stored elements as floats
__device__ __forceinline__ void load8f(const bf16_t* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(w[j] << 16);
    v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8f(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// row . x for one wave: lane l takes elements 8l + 512i; x is float in LDS
template <typename T>
__device__ __forceinline__ float wave_dot(const T* row, const float* xs, int K, int lane) {
  float acc = 0.f;
  for (int e0 = 8 * lane; e0 < K; e0 += 512) {
    float w[8];
    load8f(row + e0, w);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(w[j], xs[e0 + j], acc);
  }
  return wave_sum(acc);
}

// column of key position p (< 64) in a V^T tile (keys permuted in 16-key groups)
__device__ __forceinline__ int vt_column(int p) {
  return (p & ~15) | (p & 3) | ((p & 4) << 1) | ((p & 8) >> 1);
}

// ---------------------------------------------------------------------------
// projections of the new tokens
// ---------------------------------------------------------------------------
struct DecProjArgs {
  const void* x;          // [B, d]
  const void* wq;         // [(G*E+1)*D, d] (GQE) or [G*E*D, d] (GQA)
  const void* wk;         // [G*D, d]
  const void* wv;
  const int32_t* idx;     // [B, G, k] (GQE), or NULL (GQA: every head)
  const int32_t* pos;     // [B]
  float* q;               // [B, Hq, D] float
  void* k_cache;          // [B, G, Lc, D]
  void* vt_cache;         // [B, G, Lc/64, D, 64]
  int d, G, E, k, D, Hq, Lc, n_routed;  // n_routed: query heads before the shared one
  int shared;             // 1: head n_routed is the shared head (GQE full output)
};

// blockIdx.x: projected head (Hq query heads, then G keys, then G values);
// blockIdx.y: sequence
template <typename T>
__global__ __launch_bounds__(kDecThreads) void decode_proj_kernel(DecProjArgs a) {
  extern __shared__ float xs[];
  const int b = blockIdx.y, slot = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const T* x = static_cast<const T*>(a.x) + static_cast<size_t>(b) * a.d;
  for (int i = threadIdx.x * 8; i < a.d; i += kDecThreads * 8) {
    float v[8];
    load8f(x + i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) xs[i + j] = v[j];
  }
  __syncthreads();
  const size_t dD = static_cast<size_t>(a.D) * a.d;
  const T* w;
  int kind;  // 0 query, 1 key, 2 value
  int g = 0;
  if (slot < a.Hq) {
    kind = 0;
    int head = slot;  // routed head g*k+j uses expert idx[b, g, j] of group g
    if (a.idx != nullptr && slot < a.n_routed) {
      g = slot / a.k;
      head = g * a.E + a.idx[(static_cast<size_t>(b) * a.G + g) * a.k + slot % a.k];
    } else if (a.idx != nullptr) {
      head = a.G * a.E;  // the shared head's rows follow the G*E routed heads
    }
    w = static_cast<const T*>(a.wq) + head * dD;
  } else if (slot < a.Hq + a.G) {
    kind = 1;
    g = slot - a.Hq;
    w = static_cast<const T*>(a.wk) + g * dD;
  } else {
    kind = 2;
    g = slot - a.Hq - a.G;
    w = static_cast<const T*>(a.wv) + g * dD;
  }
  const int t = a.pos[b];
  if (kind != 0 && (t < 0 || t >= a.Lc)) return;  // a position outside the cache writes nothing
  for (int n = wave; n < a.D; n += kDecThreads / 64) {
    const float v = wave_dot(w + static_cast<size_t>(n) * a.d, xs, a.d, lane);
    if (lane != 0) continue;
    if (kind == 0) {
      a.q[(static_cast<size_t>(b) * a.Hq + slot) * a.D + n] = v;
    } else if (kind == 1) {
      static_cast<T*>(a.k_cache)[((static_cast<size_t>(b) * a.G + g) * a.Lc + t) * a.D + n] =
          from_f32<T>(v);
    } else {
      const size_t tiles = (static_cast<size_t>(a.Lc) + 63) / 64;
      static_cast<T*>(a.vt_cache)[((static_cast<size_t>(b) * a.G + g) * tiles + t / 64) * a.D * 64 +
                                  static_cast<size_t>(n) * 64 + vt_column(t & 63)] = from_f32<T>(v);
    }
  }
}

// ---------------------------------------------------------------------------
// split-K attention of the new tokens
// ---------------------------------------------------------------------------
struct DecAttnArgs {
  const float* q;         // [B, Hq, D] (unscaled)
  const void* k_cache;    // [B, G, Lc, D]
  const void* vt_cache;   // [B, G, Lc/64, D, 64]
  const int32_t* pos;     // [B]
  float* part;            // [B, Hq, n_chunks, D + 2]: o (unnormalized), m, l
  int B, G, Lc, D, Hq, chunk, n_chunks;
  int heads_per_group;    // query heads g*hpg .. g*hpg+hpg-1 read group g
  int extra_head;         // a further head (the shared one) or -1
  int extra_group;        // the group it reads
  float scale_log2;
};

// blockIdx.x: chunk of keys; blockIdx.y: b*G + g.  Wave w takes the 64-key
// tiles w, w+4, ... of the chunk; its (m, l, o) state per head is merged with
// the other waves' in LDS at the end.  MAXH bounds the query heads of one
// group (static register indexing); lane l owns head dims l, l+64, ...
template <typename T, int D, int MAXH>
__global__ __launch_bounds__(kDecThreads) void decode_attn_kernel(DecAttnArgs a) {
  constexpr int DPL = (D + 63) / 64;  // head dims per lane
  constexpr int NW = kDecThreads / 64;
  __shared__ float qs[MAXH][D];
  __shared__ float ps[NW][MAXH][64];
  __shared__ float st[NW][MAXH][D + 2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y / a.G, g = blockIdx.y % a.G, c = blockIdx.x;
  const int t = a.pos[b];
  const int kv_end = (t >= 0 && t < a.Lc) ? t + 1 : 0;  // a position outside the cache reads nothing
  const int k0 = c * a.chunk, k1 = min(k0 + a.chunk, kv_end);
  const bool extra = a.extra_head >= 0 && g == a.extra_group;
  const int nh = a.heads_per_group + (extra ? 1 : 0);
  auto head_of = [&](int i) { return i < a.heads_per_group ? g * a.heads_per_group + i : a.extra_head; };
  auto part_of = [&](int i) {
    return a.part + ((static_cast<size_t>(b) * a.Hq + head_of(i)) * a.n_chunks + c) * (D + 2);
  };
  if (k0 >= k1) {  // chunk past this sequence's end: an empty partial
    for (int i = threadIdx.x; i < nh * (D + 2); i += kDecThreads) {
      const int h = i / (D + 2), e = i % (D + 2);
      part_of(h)[e] = e == D ? -INFINITY : 0.f;
    }
    return;
  }
  for (int i = threadIdx.x; i < nh * D; i += kDecThreads)
    qs[i / D][i % D] = a.q[(static_cast<size_t>(b) * a.Hq + head_of(i / D)) * D + i % D] * a.scale_log2;
  __syncthreads();

  const T* Kg = static_cast<const T*>(a.k_cache) + (static_cast<size_t>(b) * a.G + g) * a.Lc * D;
  const size_t tiles = (static_cast<size_t>(a.Lc) + 63) / 64;
  const T* Vg = static_cast<const T*>(a.vt_cache) + (static_cast<size_t>(b) * a.G + g) * tiles * D * 64;
  float m[MAXH], l[MAXH], o[MAXH][DPL];
#pragma unroll
  for (int h = 0; h < MAXH; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int r = 0; r < DPL; ++r) o[h][r] = 0.f;
  }
  for (int j0 = k0 + 64 * wave; j0 < k1; j0 += 64 * NW) {
    // scores: lane owns key j0 + lane
    const int key = j0 + lane;
    const bool valid = key < k1;
    float kr[D];
    {
      const T* kp = Kg + static_cast<size_t>(valid ? key : j0) * D;
#pragma unroll
      for (int e = 0; e < D; e += 8) {
        float v[8];
        load8f(kp + e, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) kr[e + j] = v[j];
      }
    }
#pragma unroll
    for (int h = 0; h < MAXH; ++h) {
      if (h >= nh) break;
      float sc = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) sc = fmaf(qs[h][e], kr[e], sc);
      sc = valid ? sc : -INFINITY;
      const float mn = fmaxf(m[h], wave_max(sc));  // finite: key j0 is valid
      const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
      const float p = __builtin_amdgcn_exp2f(sc - mn);
      l[h] = l[h] * alpha + wave_sum(p);
#pragma unroll
      for (int r = 0; r < DPL; ++r) o[h][r] *= alpha;
      m[h] = mn;
      ps[wave][h][vt_column(lane)] = p;  // by V^T column
    }
    // the other lanes' probabilities are read back below: keep the order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // P . V: lane owns head dims lane + 64 r; V^T rows of the tile, 64 columns
    const int live = k1 - j0;  // keys j0 .. j0+live-1 are valid
#pragma unroll
    for (int r = 0; r < DPL; ++r) {
      const int dim = lane + 64 * r;
      if (dim >= D) continue;
      const T* vp = Vg + (static_cast<size_t>(j0 / 64) * D + dim) * 64;
      for (int c8 = 0; c8 < 64; c8 += 8) {
        float v[8];
        load8f(vp + c8, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = c8 + j;
          const float vv = vt_column(col) < live ? v[j] : 0.f;  // the permutation is an involution
#pragma unroll
          for (int h = 0; h < MAXH; ++h)
            if (h < nh) o[h][r] = fmaf(ps[wave][h][col], vv, o[h][r]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // merge the waves' states, then one partial per head
#pragma unroll
  for (int h = 0; h < MAXH; ++h) {
    if (h >= nh) break;
#pragma unroll
    for (int r = 0; r < DPL; ++r)
      if (lane + 64 * r < D) st[wave][h][lane + 64 * r] = o[h][r];
    if (lane == 0) {
      st[wave][h][D] = m[h];
      st[wave][h][D + 1] = l[h];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nh * D; i += kDecThreads) {
    const int h = i / D, e = i % D;
    float mm = -INFINITY;
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, st[w][h][D]);
    float oo = 0.f, ll = 0.f;
    for (int w = 0; w < NW; ++w) {
      if (st[w][h][D] == -INFINITY) continue;  // a wave that had no tile
      const float s = __builtin_amdgcn_exp2f(st[w][h][D] - mm);
      oo = fmaf(st[w][h][e], s, oo);
      ll = fmaf(st[w][h][D + 1], s, ll);
    }
    float* pp = part_of(h);
    pp[e] = oo;
    if (e == 0) {
      pp[D] = mm;
      pp[D + 1] = ll;
    }
  }
}

struct DecCombineArgs {
  const float* part;      // [B, Hq, n_chunks, D + 2]
  const float* row_scale; // [B, n_scaled] or NULL: output of head h < n_scaled times this
  void* s;                // [B, ld_s] slot vectors; head h at columns h*D
  int Hq, n_chunks, D, ld_s, n_scaled;
};

// one block per (sequence, head): thread = head dim
template <typename T>
__global__ __launch_bounds__(128) void decode_combine_kernel(DecCombineArgs a) {
  const int b = blockIdx.y, h = blockIdx.x, lane = threadIdx.x;
  const float* pp = a.part + (static_cast<size_t>(b) * a.Hq + h) * a.n_chunks * (a.D + 2);
  float mm = -INFINITY;
  for (int c = 0; c < a.n_chunks; ++c) mm = fmaxf(mm, pp[c * (a.D + 2) + a.D]);
  float ll = 0.f, oo = 0.f;
  for (int c = 0; c < a.n_chunks; ++c) {
    const float mc = pp[c * (a.D + 2) + a.D];
    if (mc == -INFINITY) continue;
    const float s = __builtin_amdgcn_exp2f(mc - mm);
    ll = fmaf(pp[c * (a.D + 2) + a.D + 1], s, ll);
    if (lane < a.D) oo = fmaf(pp[c * (a.D + 2) + lane], s, oo);
  }
  if (lane >= a.D) return;
  float v = ll > 0.f ? oo / ll : 0.f;
  if (a.row_scale != nullptr && h < a.n_scaled) v *= a.row_scale[static_cast<size_t>(b) * a.n_scaled + h];
  static_cast<T*>(a.s)[static_cast<size_t>(b) * a.ld_s + static_cast<size_t>(h) * a.D + lane] =
      from_f32<T>(v);
}

// out[b, n] = x[b, :K] . W[n, :K]; blockIdx.y = b, block covers 64 rows
template <typename T>
__global__ __launch_bounds__(kDecThreads) void gemv_kernel(const T* __restrict__ x, int ldx,
                                                           const T* __restrict__ w,
                                                           T* __restrict__ out, int N, int K) {
  extern __shared__ float xs[];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x * 8; i < K; i += kDecThreads * 8) {
    float v[8];
    load8f(x + static_cast<size_t>(b) * ldx + i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) xs[i + j] = v[j];
  }
  __syncthreads();
  const int n0 = blockIdx.x * 64;
  for (int n = n0 + wave; n < min(n0 + 64, N); n += kDecThreads / 64) {
    const float v = wave_dot(w + static_cast<size_t>(n) * K, xs, K, lane);
    if (lane == 0) out[static_cast<size_t>(b) * N + n] = from_f32<T>(v);
  }
}

template <typename T, int D>
hipError_t launch_decode_attn_d(const DecAttnArgs& a, hipStream_t stream) {
  const int nh = a.heads_per_group + (a.extra_head >= 0 ? 1 : 0);
  const dim3 grid(a.n_chunks, a.B * a.G);
  if (nh <= 4)
    hipLaunchKernelGGL((decode_attn_kernel<T, D, 4>), grid, dim3(kDecThreads), 0, stream, a);
  else if (nh <= 8)
    hipLaunchKernelGGL((decode_attn_kernel<T, D, 8>), grid, dim3(kDecThreads), 0, stream, a);
  else if (nh <= kMaxDecodeHeads)
    hipLaunchKernelGGL((decode_attn_kernel<T, D, kMaxDecodeHeads>), grid, dim3(kDecThreads), 0,
                       stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

int decode_chunk(int B, int G, int Lc) {
  // about 2048 attention blocks per step (8 per CU) to keep enough loads in
  // flight; a multiple of 256 keys, one 64-key tile per wave of the block
  constexpr long long kStep = 64LL * (kDecThreads / 64);
  const long long want = static_cast<long long>(Lc) * B * G / 2048;
  return static_cast<int>(kStep * std::max<long long>(1, (want + kStep - 1) / kStep));
}

template <typename T>
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.B == 0) return hipSuccess;
  DecProjArgs pa;
  pa.x = p.x;
  pa.wq = p.wq;
  pa.wk = p.wk;
  pa.wv = p.wv;
  pa.idx = p.idx;
  pa.pos = p.pos;
  pa.q = p.q;
  pa.k_cache = p.k_cache;
  pa.vt_cache = p.vt_cache;
  pa.d = p.d;
  pa.G = p.G;
  pa.E = p.E;
  pa.k = p.k;
  pa.D = p.D;
  pa.Hq = p.Hq;
  pa.Lc = p.Lc;
  pa.n_routed = p.n_routed;
  pa.shared = p.shared_head;
  const size_t xs_bytes = static_cast<size_t>(std::max(p.d, p.K_out)) * sizeof(float);
  hipLaunchKernelGGL(decode_proj_kernel<T>, dim3(p.Hq + 2 * p.G, p.B), dim3(kDecThreads),
                     static_cast<size_t>(p.d) * sizeof(float), stream, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  DecAttnArgs aa;
  aa.q = p.q;
  aa.k_cache = p.k_cache;
  aa.vt_cache = p.vt_cache;
  aa.pos = p.pos;
  aa.part = p.part;
  aa.B = p.B;
  aa.G = p.G;
  aa.Lc = p.Lc;
  aa.D = p.D;
  aa.Hq = p.Hq;
  aa.chunk = p.chunk;
  aa.n_chunks = (p.Lc + p.chunk - 1) / p.chunk;
  aa.heads_per_group = p.heads_per_group;
  aa.extra_head = p.shared_head ? p.n_routed : -1;
  aa.extra_group = p.shared_kv_group;
  aa.scale_log2 = p.scale * kLog2e;
  switch (p.D) {
    case 32: e = launch_decode_attn_d<T, 32>(aa, stream); break;
    case 64: e = launch_decode_attn_d<T, 64>(aa, stream); break;
    case 128: e = launch_decode_attn_d<T, 128>(aa, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;

  DecCombineArgs ca;
  ca.part = p.part;
  ca.row_scale = p.row_scale;
  ca.s = p.s;
  ca.Hq = p.Hq;
  ca.n_chunks = aa.n_chunks;
  ca.D = p.D;
  ca.ld_s = p.ld_s;
  ca.n_scaled = p.n_routed;
  hipLaunchKernelGGL(decode_combine_kernel<T>, dim3(p.Hq, p.B), dim3(p.D > 64 ? 128 : 64), 0,
                     stream, ca);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  if (p.weighted_slot) {
    e = launch_weighted_slot<T>(static_cast<T*>(p.s), p.w, p.B, p.G, p.k, p.D, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(gemv_kernel<T>, dim3((p.d + 63) / 64, p.B), dim3(kDecThreads), xs_bytes,
                     stream, static_cast<const T*>(p.s), p.ld_s, static_cast<const T*>(p.wo),
                     static_cast<T*>(p.out), p.d, p.K_out);
  return hipGetLastError();
}

template hipError_t launch_decode<bf16_t>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode<float>(const DecodeParams&, hipStream_t);

}  // namespace gqe

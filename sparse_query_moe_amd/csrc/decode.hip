// Decode: one new token per sequence against a KV cache.
//
// The pages analyse prefill only (pptc.cn review, section 6, lists decode as
// not analysed).  A decode step is the same layer evaluated at one position:
// the token of sequence b at position pos[b] is routed, its queries and its
// K/V are projected (K/V go straight into the cache at pos[b]), its slot
// heads attend causally to the cached keys 0..pos[b], and the slots go
// through W_O.
//
// Decode moves the whole cache once per step and does O(1) work per byte:
//   decode_front_kernel the projections of the B new tokens, C = A . W^T with
//                       B (a few) rows: 32x32 output tiles on the matrix
//                       cores, the reduction dimension split over 4 waves.
//                       Every query head of every token is projected (the
//                       weight bytes are read once whatever k is); the
//                       epilogue writes K and V^T into the caches.  Further
//                       blocks of the same launch route the tokens.
//   decode_attn_*       split-K attention ("flash decoding"): one block per
//                       (sequence, KV group, chunk of keys); the slot heads of
//                       the group share every K / V^T tile read.
//   decode_combine_kernel  one wave per (sequence, slot head) merges the
//                       chunk partials into the slot vector.
//   rows_gemm_kernel    W_O; its operand loads form the weighted slot.
#include <math.h>

#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "routing.h"

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
// split-K attention of the new tokens
// ---------------------------------------------------------------------------
struct DecAttnArgs {
  const float* q;         // [B, q_heads, D] every query head's projection (unscaled)
  const int32_t* idx;     // [B, K] routed experts by slot, or NULL (slot h uses query head h)
  int E, q_heads;
  const void* k_cache;    // [B, G, Lc, D]
  const void* vt_cache;   // [B, G, Lc/64, D, 64]
  const int32_t* pos;     // [B]
  float* part;            // [B, Hq, n_chunks, D + 2]: o (unnormalized), m, l
  int B, G, Lc, D, Hq, chunk, n_chunks;
  int hbeg[kMaxGroups + 1];  // slot heads hbeg[g] .. hbeg[g+1]-1 read group g
  int max_heads;          // most slot heads of one group, the extra one included
  int extra_head;         // a further head (the shared one) or -1
  int extra_group;        // the group it reads
  float scale_log2;
  // merge of the partials into slot vectors
  const float* row_scale; // [B, n_scaled] or NULL: output of head h < n_scaled times this
  void* s;                // [B, ld_s] slot vectors; head h at columns h*D
  int ld_s, n_scaled;
};

// One wave merges the chunk partials of (sequence b, slot head h): the chunk
// maxima, then the partial outputs weighted by 2^(m_c - max), 64 chunks at a
// time (lane = chunk for the weights, lane = head dimension for the sums);
// sw is the wave's 64-float LDS row.
template <typename T>
__device__ __forceinline__ void combine_head(const DecAttnArgs& a, int b, int h, int lane,
                                             float* sw) {
  const int stride = a.D + 2;
  const float* pp = a.part + (static_cast<size_t>(b) * a.Hq + h) * a.n_chunks * stride;
  float mm = -INFINITY;
  for (int c = lane; c < a.n_chunks; c += 64) mm = fmaxf(mm, pp[c * stride + a.D]);
  mm = wave_max(mm);
  float ll = 0.f, o0 = 0.f, o1 = 0.f;
  for (int c0 = 0; c0 < a.n_chunks; c0 += 64) {
    const int c = c0 + lane;
    float sc = 0.f;
    if (c < a.n_chunks) {
      const float mc = pp[c * stride + a.D];
      if (mc != -INFINITY) {
        sc = __builtin_amdgcn_exp2f(mc - mm);
        ll = fmaf(pp[c * stride + a.D + 1], sc, ll);
      }
    }
    sw[lane] = sc;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int n = min(64, a.n_chunks - c0);
#pragma unroll 8
    for (int j = 0; j < n; ++j) {
      const float* pc = pp + (c0 + j) * stride;
      const float sj = sw[j];
      if (lane < a.D) o0 = fmaf(pc[lane], sj, o0);
      if (lane + 64 < a.D) o1 = fmaf(pc[lane + 64], sj, o1);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  ll = wave_sum(ll);
  float f = ll > 0.f ? 1.f / ll : 0.f;  // no key (position outside the cache): zero output
  if (a.row_scale != nullptr && h < a.n_scaled)
    f *= a.row_scale[static_cast<size_t>(b) * a.n_scaled + h];
  T* out = static_cast<T*>(a.s) + static_cast<size_t>(b) * a.ld_s + static_cast<size_t>(h) * a.D;
  if (lane < a.D) out[lane] = from_f32<T>(o0 * f);
  if (lane + 64 < a.D) out[lane + 64] = from_f32<T>(o1 * f);
}

// One wave per (sequence, slot head).
template <typename T>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecAttnArgs a) {
  __shared__ float sw[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pair = blockIdx.x * 4 + wave;
  if (pair >= a.B * a.Hq) return;
  combine_head<T>(a, pair / a.Hq, pair % a.Hq, lane, sw[wave]);
}

// query head read by slot head h (of group g) of sequence b: routed slot h
// uses expert idx[b, h] of its group (head g*E + e); the next slot is the
// shared head (the last query head); without idx slot h is query head h
__device__ __forceinline__ const float* q_row(const DecAttnArgs& a, int b, int g, int h,
                                             int n_routed, int D) {
  int qh = h;
  if (a.idx != nullptr)
    qh = h < n_routed ? g * a.E + a.idx[static_cast<size_t>(b) * n_routed + h] : a.q_heads - 1;
  return a.q + (static_cast<size_t>(b) * a.q_heads + qh) * D;
}

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
  const int nh0 = a.hbeg[g + 1] - a.hbeg[g];  // this group's routed slot heads
  const int nh = nh0 + (extra ? 1 : 0);
  auto head_of = [&](int i) { return i < nh0 ? a.hbeg[g] + i : a.extra_head; };
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
    qs[i / D][i % D] = q_row(a, b, g, head_of(i / D), a.hbeg[a.G], D)[i % D] * a.scale_log2;
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

// ---- bf16: coalesced K / V^T tiles, packed bf16 dot products --------------
//
// The generic kernel above gives each lane its own key row and V^T row, so a
// wave's 16-byte load touches 64 cache lines.  Here every load instruction of
// a wave reads 1 KB of contiguous cache (16 bytes per lane):
//   K tile [64 keys, D]: load i, lane l holds dims 8*(l % LPK)..+8 of key
//     i*KPI + l / LPK (LPK = D/8 lanes per key, KPI = 64/LPK keys per load);
//     the score partials of the D/8 loads are reduce-scattered over the LPK
//     lanes of a key, after which lane l owns the score of key
//     (l % LPK)*KPI + l / LPK;
//   V^T tile [D, 64]: load j, lane l holds columns 8*(l % 8)..+8 of row
//     8*j + l/8; its P.V partial over those 8 columns stays in a register
//     across the tiles and is summed over the 8 lanes of a row at the end.
// Probabilities go from the lane that owns the key to the lanes that own its
// column through a per-wave LDS row (bf16, by V^T column).  Queries and
// probabilities are bf16, as in the prefill kernel's matrix-core products;
// accumulation is float32.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8 (i ^ 7)
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16 (i ^ 15)

// Sum over the N lanes of a lane group (N in {4, 8, 16}, groups of
// consecutive lanes) of N partials each; lane c of the group returns the
// total of partial c.  Each step pairs lanes that differ in the step's bit
// (and possibly lower ones): a lane keeps the half of the partials whose
// index has its own bit and sends the other half.
// The two-way choices go through v_perm_b32 with a per-lane selector: as
// plain selects the compiler folds them into an indexed array access, which
// it then expands into compare-and-select chains over every partial.
__device__ __forceinline__ float pick(float lo, float hi, uint32_t sel) {
  return __uint_as_float(__builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), sel));
}
constexpr uint32_t kPickLo = 0x03020100u, kPickHi = 0x07060504u;

template <int N>
__device__ __forceinline__ float reduce_scatter(float (&v)[N], int c) {
#pragma unroll
  for (int n = N; n > 1; n >>= 1) {
    const int half = n / 2;
    const bool hi = (c & half) != 0;
    const uint32_t sel_keep = hi ? kPickHi : kPickLo, sel_send = hi ? kPickLo : kPickHi;
#pragma unroll
    for (int j = 0; j < half; ++j) {
      const float keep = pick(v[j], v[j + half], sel_keep);
      const float send = pick(v[j], v[j + half], sel_send);
      float recv;
      if (half == 8) recv = dpp<kDppMirror>(send);
      else if (half == 4) recv = dpp<kDppHalfMirror>(send);
      else if (half == 2) recv = dpp<kDppXor2>(send);
      else recv = dpp<kDppXor1>(send);
      v[j] = keep + recv;
    }
  }
  return v[0];
}

// sum over the 8 lanes l, l^1, ..., l^7 (all lanes of the group get it)
__device__ __forceinline__ float sum8(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  return v + dpp<kDppHalfMirror>(v);
}

// v moved by a row broadcast to the rows in ROW_MASK; the other rows keep old
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_rows(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL,
                                                    ROW_MASK, 0xf, false));
}
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 to rows 2 and 3

// maximum over the wave (all 64 lanes active), without the LDS unit: the
// rows of 16 reduce by lane moves, rows 1 and 3 take in rows 0 and 2, rows 2
// and 3 take in row 1, and lane 63 then holds the maximum of all four rows
__device__ __forceinline__ float wave_max_fast(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  v = fmaxf(v, dpp_rows<kDppRowBcast15, 0xa>(v, v));
  v = fmaxf(v, dpp_rows<kDppRowBcast31, 0xc>(v, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float dot8(const uint4& a, const uint32_t (&b)[4], float c) {
  return dot2(a.w, b[3], dot2(a.z, b[2], dot2(a.y, b[1], dot2(a.x, b[0], c))));
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return static_cast<uint32_t>(from_f32<bf16_t>(lo)) |
         (static_cast<uint32_t>(from_f32<bf16_t>(hi)) << 16);
}

template <int D, int MAXH>
__global__ __launch_bounds__(kDecThreads) void decode_attn_bf16_kernel(DecAttnArgs a) {
  constexpr int LPK = D / 8;      // lanes per key in a K load
  constexpr int KPI = 64 / LPK;   // keys per K load
  constexpr int NL = D / 8;       // loads per tile, for K and for V^T
  constexpr int NW = kDecThreads / 64;
  __shared__ __align__(16) uint16_t ps[NW][MAXH][64];
  __shared__ float st[NW][MAXH][D + 2];
  const int lane = threadIdx.x & 63;
  const int wave = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y / a.G, g = blockIdx.y % a.G, c = blockIdx.x;
  const int t = a.pos[b];
  const int kv_end = (t >= 0 && t < a.Lc) ? t + 1 : 0;
  const int k0 = c * a.chunk, k1 = min(k0 + a.chunk, kv_end);
  const bool extra = a.extra_head >= 0 && g == a.extra_group;
  const int nh0 = a.hbeg[g + 1] - a.hbeg[g];  // this group's routed slot heads
  const int nh = nh0 + (extra ? 1 : 0);
  auto head_of = [&](int i) { return i < nh0 ? a.hbeg[g] + i : a.extra_head; };
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
  const int kc = lane % LPK;              // this lane's dims 8*kc..8*kc+7 in K loads
  const int my_key = kc * KPI + lane / LPK;  // key of the tile whose score this lane owns
  const int my_col = vt_column(my_key);
  const int vc = lane % 8;                // this lane's columns 8*vc..8*vc+7 in V^T loads

  uint32_t qf[MAXH][4];
#pragma unroll
  for (int h = 0; h < MAXH; ++h) {
    if (h < nh) {
      const float* qp = q_row(a, b, g, head_of(h), a.hbeg[a.G], D) + 8 * kc;
      const float4 q0 = reinterpret_cast<const float4*>(qp)[0];
      const float4 q1 = reinterpret_cast<const float4*>(qp)[1];
      const float sl = a.scale_log2;
      qf[h][0] = pack_bf16(q0.x * sl, q0.y * sl);
      qf[h][1] = pack_bf16(q0.z * sl, q0.w * sl);
      qf[h][2] = pack_bf16(q1.x * sl, q1.y * sl);
      qf[h][3] = pack_bf16(q1.z * sl, q1.w * sl);
    }
  }
  float m[MAXH], l[MAXH], acc[MAXH][NL];
#pragma unroll
  for (int h = 0; h < MAXH; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int j = 0; j < NL; ++j) acc[h][j] = 0.f;
  }
  const char* Kg = static_cast<const char*>(a.k_cache) +
                   (static_cast<size_t>(b) * a.G + g) * a.Lc * D * sizeof(bf16_t);
  const size_t tiles = (static_cast<size_t>(a.Lc) + 63) / 64;
  const char* Vg = static_cast<const char*>(a.vt_cache) +
                   (static_cast<size_t>(b) * a.G + g) * tiles * D * 64 * sizeof(bf16_t);

  // 16 bytes per lane per load: the K rows and V^T columns of one tile
  auto load_tile = [&](int j0, uint4 (&kf)[NL], uint4 (&vf)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int key = min(j0 + i * KPI + lane / LPK, a.Lc - 1);  // rows past the cache: any valid row
      kf[i] = *reinterpret_cast<const uint4*>(Kg + (static_cast<size_t>(key) * D + 8 * kc) * 2);
    }
    const char* vt = Vg + static_cast<size_t>(j0 / 64) * D * 64 * sizeof(bf16_t);
#pragma unroll
    for (int j = 0; j < NL; ++j) vf[j] = *reinterpret_cast<const uint4*>(vt + j * 1024 + lane * 16);
  };
  auto do_tile = [&](int j0, uint4 (&kf)[NL], uint4 (&vf)[NL]) {
    const int live = min(64, k1 - j0);  // valid keys of this tile
    if (live < 64) {  // columns of keys past the end may hold anything: zero them
      uint32_t keep[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const bool lo = vt_column(8 * vc + 2 * w) < live, hi = vt_column(8 * vc + 2 * w + 1) < live;
        keep[w] = (lo ? 0x0000ffffu : 0u) | (hi ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        vf[j].x &= keep[0];
        vf[j].y &= keep[1];
        vf[j].z &= keep[2];
        vf[j].w &= keep[3];
      }
    }
#pragma unroll
    for (int h = 0; h < MAXH; ++h) {
      if (h < nh) {
        float part[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) part[i] = dot8(kf[i], qf[h], 0.f);
        float sc = reduce_scatter<NL>(part, kc);
        sc = my_key < live ? sc : -INFINITY;
        const float mn = fmaxf(m[h], wave_max_fast(sc));  // finite: key j0 is valid
        const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
        const float p = __builtin_amdgcn_exp2f(sc - mn);
        m[h] = mn;
        l[h] = fmaf(l[h], alpha, p);
#pragma unroll
        for (int j = 0; j < NL; ++j) acc[h][j] *= alpha;
        ps[wave][h][my_col] = from_f32<bf16_t>(p);
      }
    }
    // the probabilities written above by other lanes are read below
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int h = 0; h < MAXH; ++h) {
      if (h < nh) {
        const uint4 pp = *reinterpret_cast<const uint4*>(&ps[wave][h][8 * vc]);
        const uint32_t pw[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
        for (int j = 0; j < NL; ++j) acc[h][j] = dot8(vf[j], pw, acc[h][j]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // two register buffers: the next tile's loads are in flight while this
  // tile is computed
  constexpr int kStep = 64 * NW;
  uint4 ka[NL], va[NL], kb[NL], vb[NL];
  int j0 = k0 + 64 * wave;
  if (j0 < k1) load_tile(j0, ka, va);
  while (j0 < k1) {
    if (j0 + kStep < k1) load_tile(j0 + kStep, kb, vb);
    do_tile(j0, ka, va);
    j0 += kStep;
    if (j0 >= k1) break;
    if (j0 + kStep < k1) load_tile(j0 + kStep, ka, va);
    do_tile(j0, kb, vb);
    j0 += kStep;
  }
  // this wave's state per head: o over the 8 lanes of a V^T row, l over all lanes
#pragma unroll
  for (int h = 0; h < MAXH; ++h) {
    if (h < nh) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const float o = sum8(acc[h][j]);
        if (vc == 0) st[wave][h][8 * j + lane / 8] = o;
      }
      const float lt = wave_sum(l[h]);
      if (lane == 0) {
        st[wave][h][D] = m[h];
        st[wave][h][D + 1] = lt;
      }
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

// ---------------------------------------------------------------------------
// projections of the new tokens: C[M, N] = A[M, K] . W[N, K]^T
// ---------------------------------------------------------------------------
struct RowsGemmArgs {
  const void* a;          // [M, lda] activations
  int lda;
  const void* w[3];       // the rows of W come from up to three matrices:
  int n_end[3];           // columns [n_end[i-1], n_end[i]) are rows of w[i]
  int M, N, K;
  // plain output
  void* out;              // [M, N] or NULL
  // decode QKV output: columns < nq are query heads (float), then G*D key
  // columns and G*D value columns written into the caches at pos[m]
  float* q;
  int nq;
  void* k_cache;
  void* vt_cache;
  const int32_t* pos;
  int G, D, Lc;
  // weighted slot formed in the A loads: columns [ws_col, ws_col + D) of A
  // are sum_h w[m, h] * A[m, h*D + c] over h < ws_heads, rounded to T
  const float* ws_w;
  int ws_col, ws_heads;
  // rotary embedding of the query and key columns of the decode projection
  RopeTable rope;
};

template <typename T>
__device__ __forceinline__ typename Frag<T>::type weighted_frag(const T* arow, const float* w,
                                                                int heads, int D, int c) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int h = 0; h < heads; ++h) {
    const float wh = w[h];
    float v[8];
    load8f(arow + h * D + c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = fmaf(wh, v[j], acc[j]);
  }
  // the slot is stored in T before the product, as the prefill output stage does
  T r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = from_f32<T>(acc[j]);
  return load_frag(r);
}

// One 32x32 output tile (rows m0.., columns n0..) per block of 4 waves: wave w
// takes the w-th quarter of the K steps (16 elements each); the four partial
// tiles are added in LDS and each wave stores a quarter of the result.
template <typename T>
__device__ __forceinline__ void gemm_tile(const RowsGemmArgs& a, int n0, int m0) {
  constexpr int U = sizeof(T) == 2 ? 8 : 4;  // K steps whose loads are issued together
  __shared__ float red[4][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int seg = 0;
  while (seg < 2 && n0 >= a.n_end[seg]) ++seg;
  const int nb = seg == 0 ? 0 : a.n_end[seg - 1];
  const T* W = static_cast<const T*>(a.w[seg]) + static_cast<size_t>(n0 - nb + lane % 32) * a.K;
  const int m = min(m0 + lane % 32, a.M - 1);  // rows past M: any valid row, not stored
  const T* A = static_cast<const T*>(a.a) + static_cast<size_t>(m) * a.lda;
  const int kh = 8 * (lane / 32);
  const int S = a.K / 16;
  const int per = (S + 3) / 4;
  const int s_beg = wave * per, s_end = min(S, s_beg + per);
  f32x16 acc = splat16(0.f);
  for (int s0 = s_beg; s0 < s_end; s0 += U) {
    typename Frag<T>::type fa[U], fw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < s_end) {
        const int k0 = 16 * (s0 + u) + kh;
        if (a.ws_w != nullptr && k0 >= a.ws_col && k0 < a.ws_col + a.D)
          fa[u] = weighted_frag<T>(A, a.ws_w + static_cast<size_t>(m) * a.ws_heads, a.ws_heads,
                                   a.D, k0 - a.ws_col);
        else
          fa[u] = load_frag(A + k0);
        fw[u] = load_frag(W + k0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + u < s_end) mma32(acc, fa[u], fw[u]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) red[wave][i][lane] = acc[i];
  __syncthreads();
  const int col = n0 + lane % 32;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int i = 4 * wave + ii;
    float v = red[0][i][lane] + red[1][i][lane] + red[2][i][lane] + red[3][i][lane];
    const int row = m0 + acc_row(i, lane);
    if (a.out == nullptr && a.rope.on) {  // queries and keys turn by the token's position
      const float partner = __shfl_xor(v, 1, 64);  // column col ^ 1, the pair partner
      const bool qk = col < a.nq || col - a.nq < a.G * a.D;
      const int t = row < a.M ? a.pos[row] : -1;
      if (qk && t >= 0 && t < a.Lc) {
        const int dim = (col < a.nq ? col : col - a.nq) % a.D;
        float cs, sn;
        rope_cs(t, a.rope.theta[dim >> 1], cs, sn);
        v = rope_apply(v, partner, dim, cs, sn);
      }
    }
    if (row >= a.M) continue;
    if (a.out != nullptr) {
      static_cast<T*>(a.out)[static_cast<size_t>(row) * a.N + col] = from_f32<T>(v);
    } else if (col < a.nq) {
      a.q[static_cast<size_t>(row) * a.nq + col] = v;
    } else {
      const int t = a.pos[row];
      if (t < 0 || t >= a.Lc) continue;  // a position outside the cache writes nothing
      const int GD = a.G * a.D;
      const bool key = col - a.nq < GD;
      const int cc = key ? col - a.nq : col - a.nq - GD;
      const int g = cc / a.D, dim = cc % a.D;
      const size_t bg = static_cast<size_t>(row) * a.G + g;
      if (key) {
        static_cast<T*>(a.k_cache)[(bg * a.Lc + t) * a.D + dim] = from_f32<T>(v);
      } else {
        const size_t tiles = (static_cast<size_t>(a.Lc) + 63) / 64;
        static_cast<T*>(a.vt_cache)[((bg * tiles + t / 64) * a.D + dim) * 64 + vt_column(t & 63)] =
            from_f32<T>(v);
      }
    }
  }
}

// grid (N/32, ceil(M/32))
template <typename T>
__global__ __launch_bounds__(256) void rows_gemm_kernel(RowsGemmArgs a) {
  gemm_tile<T>(a, blockIdx.x * 32, blockIdx.y * 32);
}

struct FrontArgs {
  const void* x;          // [B, d] the new tokens
  const void* wr;         // [G*E, d] router rows, or NULL (no routing)
  const float* bias;      // [G*E] or NULL
  int32_t* idx;           // [B, K]
  float* w;               // [B, K]
  int d, G, E, renorm;
  GroupK gk;              // experts selected per group and their slot offsets
  int n_gemm_blocks, gemm_nbx;
};

// The first launch of a decode step: the projection tiles, then (GQE) one
// routing block per token.
template <typename T>
__global__ __launch_bounds__(256) void decode_front_kernel(RowsGemmArgs g, FrontArgs f) {
  const int id = blockIdx.x;
  if (id < f.n_gemm_blocks)
    gemm_tile<T>(g, (id % f.gemm_nbx) * 32, (id / f.gemm_nbx) * 32);
  else
    route_token_block<T>(static_cast<const T*>(f.x), static_cast<const T*>(f.wr), f.bias, f.idx,
                         f.w, id - f.n_gemm_blocks, f.d, f.G, f.E, f.gk, f.renorm);
}

template <typename T>
hipError_t launch_rows_gemm(const RowsGemmArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (a.N % 32 != 0 || a.K % 16 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rows_gemm_kernel<T>, dim3(a.N / 32, (a.M + 31) / 32), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_attn_d(const DecAttnArgs& a, hipStream_t stream) {
  const int nh = a.max_heads;
  const dim3 grid(a.n_chunks, a.B * a.G);
  if (sizeof(T) == 2) {  // coalesced bf16 kernel while the head accumulators fit
    if (nh <= 4) {
      hipLaunchKernelGGL((decode_attn_bf16_kernel<D, 4>), grid, dim3(kDecThreads), 0, stream, a);
      return hipGetLastError();
    }
    if constexpr (D <= 64) {
      if (nh <= 8) {
        hipLaunchKernelGGL((decode_attn_bf16_kernel<D, 8>), grid, dim3(kDecThreads), 0, stream, a);
        return hipGetLastError();
      }
    }
  }
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
hipError_t launch_decode_front(const DecodeParams& p, hipStream_t stream) {
  RowsGemmArgs ga = {};
  ga.a = p.x;
  ga.lda = p.d;
  ga.w[0] = p.wq;
  ga.w[1] = p.wk;
  ga.w[2] = p.wv;
  const int nq = p.q_heads * p.D, GD = p.G * p.D;
  ga.n_end[0] = nq;
  ga.n_end[1] = nq + GD;
  ga.n_end[2] = nq + 2 * GD;
  ga.M = p.B;
  ga.N = nq + 2 * GD;
  ga.K = p.d;
  ga.q = p.q;
  ga.nq = nq;
  ga.k_cache = p.k_cache;
  ga.vt_cache = p.vt_cache;
  ga.pos = p.pos;
  ga.G = p.G;
  ga.D = p.D;
  ga.Lc = p.Lc;
  ga.rope = p.rope;
  if (ga.N % 32 != 0 || ga.K % 16 != 0) return hipErrorInvalidValue;
  FrontArgs f = {};
  f.x = p.x;
  f.wr = p.wr;
  f.bias = p.router_bias;
  f.idx = const_cast<int32_t*>(p.idx);
  f.w = const_cast<float*>(p.w);
  f.d = p.d;
  f.G = p.G;
  f.E = p.E;
  f.gk = p.gk;
  f.renorm = p.renorm;
  f.gemm_nbx = ga.N / 32;
  f.n_gemm_blocks = f.gemm_nbx * ((p.B + 31) / 32);
  const int blocks = f.n_gemm_blocks + (p.wr != nullptr ? p.B : 0);
  hipLaunchKernelGGL(decode_front_kernel<T>, dim3(blocks), dim3(256), 0, stream, ga, f);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_decode_attend(const DecodeParams& p, hipStream_t stream) {
  DecAttnArgs aa;
  aa.q = p.q;
  aa.idx = p.idx;
  aa.E = p.E;
  aa.q_heads = p.q_heads;
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
  for (int g = 0; g <= p.G; ++g) aa.hbeg[g] = p.hbeg[g];
  aa.max_heads = p.max_heads;
  aa.extra_head = p.shared_head ? p.n_routed : -1;
  aa.extra_group = p.shared_kv_group;
  aa.scale_log2 = p.scale * kLog2e;
  aa.row_scale = p.row_scale;
  aa.s = p.s;
  aa.ld_s = p.ld_s;
  aa.n_scaled = p.n_routed;
  hipError_t e;
  switch (p.D) {
    case 32: e = launch_decode_attn_d<T, 32>(aa, stream); break;
    case 64: e = launch_decode_attn_d<T, 64>(aa, stream); break;
    case 128: e = launch_decode_attn_d<T, 128>(aa, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<T>, dim3((p.B * p.Hq + 3) / 4), dim3(256), 0, stream,
                     aa);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  RowsGemmArgs ga = {};
  ga.a = p.s;
  ga.lda = p.ld_s;
  ga.w[0] = ga.w[1] = ga.w[2] = p.wo;
  ga.n_end[0] = ga.n_end[1] = ga.n_end[2] = p.d;
  ga.M = p.B;
  ga.N = p.d;
  ga.K = p.K_out;
  ga.out = p.out;
  ga.D = p.D;
  if (p.weighted_slot) {  // slot n_routed + 1 = sum_h w[b, h] * slot h over the routed heads
    ga.ws_w = p.w;
    ga.ws_col = (p.n_routed + 1) * p.D;
    ga.ws_heads = p.n_routed;
  }
  return launch_rows_gemm<T>(ga, stream);
}

template hipError_t launch_decode_front<bf16_t>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode_front<float>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode_attend<bf16_t>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode_attend<float>(const DecodeParams&, hipStream_t);

}  // namespace gqe

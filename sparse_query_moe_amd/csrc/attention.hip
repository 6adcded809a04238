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
//   leave registers; V^T tiles are staged in LDS with their keys permuted
//   inside every 16-key group to match that accumulator order, which makes
//   each V^T fragment one 16-byte LDS read.  O^T again has one query per lane,
//   so the online-softmax rescale is lane-local.
//   K and V^T tiles of 64 keys are double-buffered in LDS (swizzled 16-byte
//   chunks, one barrier per tile).  The running maximum is only raised when a
//   tile exceeds it by more than 2^8: the stale maximum keeps every
//   probability <= 256, and since the same maximum scales numerator and
//   denominator the result is unchanged.
//   Blocks are issued heaviest query block first to shorten the causal tail.
#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace gqe {

namespace {

constexpr float kRescaleThreshold = 8.0f;  // log2 units


template <typename T, int D, int QB = 1>
struct AttnShape {
  static constexpr int BQ = 4 * 32 * QB, BKV = 64;  // 4 waves, QB 32-query blocks each
  static constexpr int EPC = 16 / static_cast<int>(sizeof(T));
  static constexpr int KROW = D * static_cast<int>(sizeof(T));    // bytes per K tile row (a key)
  static constexpr int VROW = BKV * static_cast<int>(sizeof(T));  // bytes per V^T tile row (a dim)
  static constexpr int KT = BKV * KROW, VT = D * VROW;
  static constexpr int STAGE = KT + VT;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int K_CPR = KROW / 16, V_CPR = VROW / 16;  // 16-byte chunks per row
  static constexpr int K_CH = BKV * K_CPR / 256, V_CH = D * V_CPR / 256;
  static constexpr int NDB = D / 32;  // 32-row blocks of O^T
  static constexpr int NKS = D / 16;  // K-steps of S^T
  static_assert(K_CH >= 1 && V_CH >= 1, "tile smaller than one chunk per thread");
};

// Where the 16-byte global chunk cc of a V^T row lands in LDS.  Inside each
// 16-key group, logical key 8a + 4u + r (a, u in {0,1}, r < 4) is stored at
// physical position 8u + 4a + r: lane half u then reads its 8 keys contiguously.
template <typename T, int D> struct VStore;
template <int D> struct VStore<bf16_t, D> {
  typedef AttnShape<bf16_t, D> S;
  // a chunk holds keys 8cc..8cc+7 = (a = cc & 1; u = 0 then u = 1): two 8-byte halves
  static __device__ __forceinline__ void put(char* vs, int row, int cc, uint4 v) {
    const int g16 = cc >> 1, a = cc & 1;
    char* p0 = vs + swz<S::VROW>(row, 2 * g16) + 8 * a;
    char* p1 = vs + swz<S::VROW>(row, 2 * g16 + 1) + 8 * a;
    *reinterpret_cast<uint2*>(p0) = make_uint2(v.x, v.y);
    *reinterpret_cast<uint2*>(p1) = make_uint2(v.z, v.w);
  }
};
template <int D> struct VStore<float, D> {
  typedef AttnShape<float, D> S;
  // a chunk holds keys 4cc..4cc+3 = one (a, u) quarter of a 16-key group
  static __device__ __forceinline__ void put(char* vs, int row, int cc, uint4 v) {
    const int g16 = cc >> 2, a = (cc >> 1) & 1, u = cc & 1;
    *reinterpret_cast<uint4*>(vs + swz<S::VROW>(row, 4 * g16 + 2 * u + a)) = v;
  }
};

// zero the elements of a chunk whose keys are >= L (chunk starts at key k0)
template <typename T>
__device__ __forceinline__ uint4 mask_keys(uint4 v, int k0, int L) {
  constexpr int EPC = 16 / static_cast<int>(sizeof(T));
  if (k0 + EPC <= L) return v;
  if (k0 >= L) return zero4();
  T* e = reinterpret_cast<T*>(&v);
#pragma unroll
  for (int j = 0; j < EPC; ++j)
    if (k0 + j >= L) e[j] = T(0);
  return v;
}

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

template <typename T, int D, int QB>
__global__ __launch_bounds__(256, D == 128 ? 1 : 2) void attention_kernel(
    AttnParams p) {
  typedef AttnShape<T, D, QB> S;
  typedef typename Frag<T>::type F;
  extern __shared__ __align__(16) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int L = p.L;
  const int nq = (L + S::BQ - 1) / S::BQ;
  const int bh_count = p.B * p.H;
  const int qi = blockIdx.x / bh_count;
  const int bh = blockIdx.x % bh_count;
  const int qblk = nq - 1 - qi;  // heaviest first
  const int b = bh / p.H, head = bh % p.H;
  const int g = head < p.n_grouped ? head / p.heads_per_group : p.extra_group;

  const T* Q = static_cast<const T*>(p.q) + (static_cast<size_t>(b) * p.H + head) * L * D;
  const T* Kg = static_cast<const T*>(p.k) + (static_cast<size_t>(b) * p.G + g) * L * D;
  const T* Vg = static_cast<const T*>(p.vt) + (static_cast<size_t>(b) * p.G + g) * D * p.vt_ld;

  const int q0 = qblk * S::BQ;
  const int qw0 = q0 + 32 * QB * wave;                 // first query of this wave
  const int wave_last = min(qw0 + 32 * QB - 1, L - 1);  // last valid query of this wave
  const bool wave_active = qw0 < L;

  // queries (pre-scaled) in registers; the running maximum starts at the score
  // against key 0, which every causal row sees, so it is finite from the start
  int qrow[QB];
  F qf[QB][S::NKS];
  float m_run[QB], l_run[QB];
  f32x16 o[QB][S::NDB];
  {
    F k0[S::NKS];
#pragma unroll
    for (int ks = 0; ks < S::NKS; ++ks) k0[ks] = load_frag(Kg + ks * 16 + 8 * half);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      qrow[qb] = qw0 + 32 * qb + (lane & 31);
      float dot = 0.f;
#pragma unroll
      for (int ks = 0; ks < S::NKS; ++ks) {
        if (qrow[qb] < L) {
          qf[qb][ks] = scale_frag(load_frag(Q + static_cast<size_t>(qrow[qb]) * D + ks * 16 + 8 * half),
                                  p.scale_log2);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) qf[qb][ks][j] = 0;
        }
        dot += dot8(qf[qb][ks], k0[ks]);
      }
      m_run[qb] = dot + __shfl_xor(dot, 32, 64);
      l_run[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < S::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[qb][db][i] = 0.f;
    }
  }

  const int kv_end = min(q0 + S::BQ, L);
  const int ntiles = (kv_end + S::BKV - 1) / S::BKV;

  uint4 rk[S::K_CH], rv[S::V_CH];
  auto gload = [&](int jt) {
    const int j0 = jt * S::BKV;
#pragma unroll
    for (int i = 0; i < S::K_CH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / S::K_CPR, cc = c % S::K_CPR;
      const int key = j0 + row;
      rk[i] = key < L ? *reinterpret_cast<const uint4*>(Kg + static_cast<size_t>(key) * D +
                                                         cc * S::EPC)
                      : zero4();
    }
#pragma unroll
    for (int i = 0; i < S::V_CH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / S::V_CPR, cc = c % S::V_CPR;
      const int k0 = j0 + cc * S::EPC;
      uint4 v = zero4();
      if (k0 < L)
        v = mask_keys<T>(*reinterpret_cast<const uint4*>(Vg + static_cast<size_t>(row) * p.vt_ld + k0),
                         k0, L);
      rv[i] = v;
    }
  };
  auto sstore = [&](int buf) {
    char* ks_ = smem + buf * S::STAGE;
    char* vs_ = ks_ + S::KT;
#pragma unroll
    for (int i = 0; i < S::K_CH; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<uint4*>(ks_ + swz<S::KROW>(c / S::K_CPR, c % S::K_CPR)) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < S::V_CH; ++i) {
      const int c = tid + 256 * i;
      VStore<T, D>::put(vs_, c / S::V_CPR, c % S::V_CPR, rv[i]);
    }
  };

  // one 64-key tile for this wave's QB query blocks
  auto tile = [&](const char* Ks, const char* Vs, int j0, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    // S^T - m: the accumulator starts at -m_run, so exp2 applies directly
    f32x16 s[QB][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < S::NKS; ++ks) {
        const F kf = LdsFrag<T, S::KROW>::get(Ks, 32 * kb + (lane & 31), ks * 16 + 8 * half);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (ks == 0) s[qb][kb] = splat16(-m_run[qb]);  // S^T - m: exp2 applies directly
          mma32(s[qb][kb], kf, qf[qb][ks]);
        }
      }
    if constexpr (MASK) {  // drop keys after the query
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (j0 + 32 * kb + acc_row(i, lane) > qrow[qb]) s[qb][kb][i] = -INFINITY;
    }
    float mx[QB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float v = s[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) v = fmaxf(v, s[qb][kb][i]);
      mx[qb] = fmaxf(v, __shfl_xor(v, 32, 64));
      need = need || (mx[qb] > kRescaleThreshold);
    }
    if (__any(need)) {  // raise the running maximum (wave-uniform branch)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float sh = fmaxf(mx[qb], 0.f);
        const float alpha = __builtin_amdgcn_exp2f(-sh);
        m_run[qb] += sh;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < S::NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[qb][kb][i] -= sh;
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(s[qb][kb][i]);
          s[qb][kb][i] = pv;
          ls += pv;
        }
      l_run[qb] += ls;
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      F pf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) pf[qb] = FragFromAcc<T>::get(s[qb][ks >> 1], 8 * (ks & 1));
#pragma unroll
      for (int db = 0; db < S::NDB; ++db) {
        const F vf = LdsFrag<T, S::VROW>::get(Vs, 32 * db + (lane & 31), ks * 16 + 8 * half);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) mma32(o[qb][db], vf, pf[qb]);
      }
    }
  };

  gload(0);
  sstore(0);
  lds_barrier();
  for (int jt = 0; jt < ntiles; ++jt) {
    if (jt + 1 < ntiles) gload(jt + 1);
    const char* Ks = smem + (jt & 1) * S::STAGE;
    const char* Vs = Ks + S::KT;
    const int j0 = jt * S::BKV;
    if (wave_active && j0 <= wave_last) {
      if (j0 + S::BKV - 1 <= qw0)
        tile(Ks, Vs, j0, std::false_type{});
      else
        tile(Ks, Vs, j0, std::true_type{});
    }
    if (jt + 1 < ntiles) sstore((jt + 1) & 1);
    lds_barrier();
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
    if (qrow[qb] < L) {
      const float inv = 1.f / l_tot;
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

template <typename T, int D, int QB>
hipError_t launch_attention_d(const AttnParams& p, hipStream_t stream) {
  typedef AttnShape<T, D, QB> S;
  const int nq = (p.L + S::BQ - 1) / S::BQ;
  const long long blocks = static_cast<long long>(nq) * p.B * p.H;
  if (blocks == 0) return hipSuccess;
  if (S::LDS > 65536) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&attention_kernel<T, D, QB>),
        hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS);
    if (attr != hipSuccess) return attr;
  }
  hipLaunchKernelGGL((attention_kernel<T, D, QB>), dim3(static_cast<unsigned>(blocks)), dim3(256),
                     S::LDS, stream, p);
  return hipGetLastError();
}

}  // namespace

// Two 32-query blocks per wave halve the LDS traffic per MFMA; short
// sequences keep one so that the grid still covers the chip.
template <typename T>
hipError_t launch_attention(const AttnParams& p, int D, hipStream_t stream) {
  if constexpr (sizeof(T) == 2) {
    const bool wide = static_cast<long long>(p.L) * p.B * p.H >= 256LL * 256 * 4;
    switch (D) {
      case 32: return wide ? launch_attention_d<T, 32, 2>(p, stream) : launch_attention_d<T, 32, 1>(p, stream);
      case 64: return wide ? launch_attention_d<T, 64, 2>(p, stream) : launch_attention_d<T, 64, 1>(p, stream);
      case 128: return launch_attention_d<T, 128, 1>(p, stream);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (D) {
      case 32: return launch_attention_d<T, 32, 1>(p, stream);
      case 64: return launch_attention_d<T, 64, 1>(p, stream);
      case 128: return launch_attention_d<T, 128, 1>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
}

template hipError_t launch_attention<bf16_t>(const AttnParams&, int, hipStream_t);
template hipError_t launch_attention<float>(const AttnParams&, int, hipStream_t);

}  // namespace gqe

// Device-side helpers shared by the gfx950 kernels of the GQE layer:
// element types, 8-element MFMA operand fragments, the 32x32 MFMA wrappers and
// the swizzled LDS addressing used by every tiled kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqe {

typedef uint16_t bf16_t;  // bfloat16 storage

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// An MFMA operand fragment: the 8 consecutive K-elements one lane supplies.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ float to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}
__device__ __forceinline__ float to_f32(float v) { return v; }

// float -> storage type, round to nearest even.
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
  __bf16 b = static_cast<__bf16>(v);
  return __builtin_bit_cast(bf16_t, b);
}

// Load / store 8 elements (16 B for bf16, 32 B for fp32) at an aligned address.
__device__ __forceinline__ bf16x8 load_frag(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ f32x8 load_frag(const float* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 a = q[0], b = q[1];
  f32x8 r;
  r[0] = __uint_as_float(a.x); r[1] = __uint_as_float(a.y);
  r[2] = __uint_as_float(a.z); r[3] = __uint_as_float(a.w);
  r[4] = __uint_as_float(b.x); r[5] = __uint_as_float(b.y);
  r[6] = __uint_as_float(b.z); r[7] = __uint_as_float(b.w);
  return r;
}

// acc += A . B for one 32x32 output tile and 16 K-elements.  Lane l supplies
// A[l % 32][k in its half] and B[k in its half][l % 32]; the two operands use
// the same K assignment, so any fixed permutation of K inside a fragment
// leaves the product unchanged.
__device__ __forceinline__ void mma32(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], acc, 0, 0, 0);
}

// A . B + C with a separate accumulator input (C is left unchanged).
__device__ __forceinline__ f32x16 mma32c(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32c(const f32x8& a, const f32x8& b, const f32x16& c) {
  f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
#pragma unroll
  for (int j = 1; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], acc, 0, 0, 0);
  return acc;
}

// A 16-float accumulator with every element v, built with 64-bit moves.
__device__ __forceinline__ f32x16 splat16(float v) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef double f64x8 __attribute__((ext_vector_type(8)));
  const f32x2 pair = {v, v};
  const double d = __builtin_bit_cast(double, pair);
  const f64x8 dv = {d, d, d, d, d, d, d, d};
  return __builtin_bit_cast(f32x16, dv);
}

// Output layout of a 32x32 MFMA accumulator: value i of lane l is
// C[row_of(i, l)][l % 32].
__device__ __forceinline__ int acc_row(int i, int lane) {
  return ((i >> 2) << 3) + ((lane >> 5) << 2) + (i & 3);
}

// Convert 8 float32 values to a fragment of type T.
__device__ __forceinline__ bf16x8 to_frag_bf16(float a0, float a1, float a2, float a3, float a4,
                                               float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = static_cast<__bf16>(a0); r[1] = static_cast<__bf16>(a1);
  r[2] = static_cast<__bf16>(a2); r[3] = static_cast<__bf16>(a3);
  r[4] = static_cast<__bf16>(a4); r[5] = static_cast<__bf16>(a5);
  r[6] = static_cast<__bf16>(a6); r[7] = static_cast<__bf16>(a7);
  return r;
}
template <typename T> struct FragFromAcc;
template <> struct FragFromAcc<bf16_t> {
  static __device__ __forceinline__ bf16x8 get(const f32x16& s, int base) {
    return to_frag_bf16(s[base + 0], s[base + 1], s[base + 2], s[base + 3], s[base + 4],
                        s[base + 5], s[base + 6], s[base + 7]);
  }
};
template <> struct FragFromAcc<float> {
  static __device__ __forceinline__ f32x8 get(const f32x16& s, int base) {
    f32x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = s[base + j];
    return r;
  }
};

// LDS tiles are stored as rows of 16-byte chunks.  gfx950's LDS serves 256
// bytes (64 banks x 4 B) per cycle, i.e. sixteen 16-byte units.  An MFMA
// fragment read has consecutive lanes read the same logical chunk of
// consecutive rows, so the chunk index is XORed with the row's index in units
// of 256 bytes: any 16 consecutive rows then hit 16 different units.
template <int ROWB>
__device__ __forceinline__ int swz_xor(int row) {
  constexpr int CPR = ROWB / 16;                       // chunks per row
  constexpr int RP = ROWB >= 256 ? 1 : 256 / ROWB;     // rows per 256 bytes
  constexpr int mask = CPR < 16 ? CPR - 1 : 15;
  return (row / RP) & mask;
}
template <int ROWB>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * ROWB + ((chunk ^ swz_xor<ROWB>(row)) << 4);
}

// 8 K-elements of row `row`, starting at element `elem`, from a swizzled LDS
// tile with ROWB-byte rows.
template <typename T, int ROWB> struct LdsFrag;
template <int ROWB> struct LdsFrag<bf16_t, ROWB> {
  static __device__ __forceinline__ bf16x8 get(const char* base, int row, int elem) {
    return __builtin_bit_cast(bf16x8,
                              *reinterpret_cast<const uint4*>(base + swz<ROWB>(row, elem >> 3)));
  }
};
template <int ROWB> struct LdsFrag<float, ROWB> {
  static __device__ __forceinline__ f32x8 get(const char* base, int row, int elem) {
    const uint4 a = *reinterpret_cast<const uint4*>(base + swz<ROWB>(row, elem >> 2));
    const uint4 b = *reinterpret_cast<const uint4*>(base + swz<ROWB>(row, (elem >> 2) + 1));
    f32x8 r;
    r[0] = __uint_as_float(a.x); r[1] = __uint_as_float(a.y);
    r[2] = __uint_as_float(a.z); r[3] = __uint_as_float(a.w);
    r[4] = __uint_as_float(b.x); r[5] = __uint_as_float(b.y);
    r[6] = __uint_as_float(b.z); r[7] = __uint_as_float(b.w);
    return r;
  }
};

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Rotary position embedding (RoFormer, Su et al. 2021, interleaved pairs):
// dims (2j, 2j+1) of a query or key head at position t turn by t * theta_j,
// theta_j = base^(-2j/d_h) (float64, from the host; on == 0: no rotation).
// The angle is formed and reduced modulo 2 pi in float64 (positions reach
// 2^20), then its cosine and sine are taken in float32.
struct RopeTable {
  double theta[64];
  int on;
};
__device__ __forceinline__ void rope_cs(int t, double theta, float& c, float& s) {
  const double a = static_cast<double>(t) * theta;
  const double k = rint(a * 0.15915494309189533577);              // a / (2 pi)
  double r = fma(-k, 6.28318530717958623200, a);                   // 2 pi, high part
  r = fma(-k, 2.44929359829470635445e-16, r);                      // 2 pi, low part
  sincosf(static_cast<float>(r), &s, &c);
}
// v (dim d of a head) turned together with its pair partner p (dim d ^ 1);
// inverse turns back (the transpose of the rotation)
__device__ __forceinline__ float rope_apply(float v, float p, int d, float c, float s,
                                            bool inverse = false) {
  const float sn = inverse ? -s : s;
  return (d & 1) ? fmaf(p, sn, v * c) : fmaf(-p, sn, v * c);
}

// an LDS address as the direct-load builtins want it
#define GQE_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Block barrier that orders LDS accesses only.  __syncthreads() is a full
// workgroup fence and also waits for every global load still in flight,
// which would expose the latency of the next tile's prefetch at each
// barrier; the prefetch only targets registers, so the LDS fence suffices.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// wait until at most n of this wave's vector-memory operations are in flight
// (and all its LDS operations are done); n is small and known per call site
__device__ __forceinline__ void wait_vm(int n) {
#define GQE_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4))
  switch (n) {
    case 0: GQE_VM(0); break;
    case 1: GQE_VM(1); break;
    case 2: GQE_VM(2); break;
    case 3: GQE_VM(3); break;
    case 4: GQE_VM(4); break;
    case 5: GQE_VM(5); break;
    case 6: GQE_VM(6); break;
    case 7: GQE_VM(7); break;
    case 8: GQE_VM(8); break;
    case 9: GQE_VM(9); break;
    case 10: GQE_VM(10); break;
    case 11: GQE_VM(11); break;
    case 12: GQE_VM(12); break;
    case 13: GQE_VM(13); break;
    case 14: GQE_VM(14); break;
    case 15: GQE_VM(15); break;
    case 16: GQE_VM(16); break;
    case 17: GQE_VM(17); break;
    case 18: GQE_VM(18); break;
    case 19: GQE_VM(19); break;
    case 20: GQE_VM(20); break;
    case 21: GQE_VM(21); break;
    case 22: GQE_VM(22); break;
    case 23: GQE_VM(23); break;
    case 24: GQE_VM(24); break;
    default: GQE_VM(0); break;
  }
#undef GQE_VM
}

// direct global-to-LDS copy of 16 bytes per lane: lane i's src lands at LDS
// bytes lds + 16 i .. lds + 16 i + 15 (lds must be wave-uniform: it goes
// through M0).  A plain (non-template) device function, so that kernels whose
// bodies use it keep their host-side launch stubs.
__device__ __forceinline__ void dma16(const void* src, char* lds) {
  __builtin_amdgcn_global_load_lds(src, GQE_LDS(lds), 16, 0, 0);
}

// barrier after which every wave's direct global-to-LDS loads issued before
// it have landed (each wave first waits for its own); no fence, which would
// also wait for unrelated loads
__device__ __forceinline__ void dma_barrier(int pending) {
  wait_vm(pending);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace gqe

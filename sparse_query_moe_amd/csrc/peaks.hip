// Measurement probes: the bf16 matrix-core rate and the HBM copy rate this
// device sustains.  Kernel rates are reported against the published peaks,
// which assume the nominal 2.4 GHz clock and 8 TB/s, and also against what
// these two loops reach on the same chip under sustained load.
//
//   mfma_peak_kernel: every wave runs four independent accumulation chains of
//     v_mfma_f32_32x32x16_bf16 (32*32*16*2 = 32768 flop each) and nothing
//     else; a chain is revisited every four MFMAs, which covers the MFMA
//     latency, and two waves per SIMD (all resident at once) keep the matrix
//     core fed.
//   copy_peak_kernel: a one-pass copy in 16-byte non-temporal loads and
//     stores, four in flight per thread (the fastest of the copy forms
//     measured: grid-stride loops, deeper unrolls, plain accesses and the
//     runtime's own copy were 8-28% slower); a buffer larger than the 256 MB
//     last-level cache makes every byte an HBM read and an HBM write.
#include <stdint.h>

#include "../../include/gqe.h"
#include "device_common.h"

namespace gqe {

int cu_count();

namespace {

constexpr int kChains = 4;

__global__ __launch_bounds__(256) void mfma_peak_kernel(float* __restrict__ out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // small multiples of 2^-10: every partial stays far inside float range
    a[j] = static_cast<__bf16>(static_cast<float>((threadIdx.x + j) & 7) * 0x1p-10f);
    b[j] = static_cast<__bf16>(static_cast<float>((threadIdx.x >> 3) & 3) * 0x1p-10f);
  }
  f32x16 c[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) c[i] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += c[i][0] + c[i][15];
  out[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

// one pass: block i copies the 16 KB chunk i, four 16-byte accesses per
// thread, all loads issued before the stores; non-temporal hints keep the
// streams from displacing cached lines
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCopyUnroll = 4;
__global__ __launch_bounds__(256) void copy_peak_kernel(u32x4* __restrict__ dst,
                                                        const u32x4* __restrict__ src, size_t n) {
  const size_t base = static_cast<size_t>(blockIdx.x) * 256 * kCopyUnroll + threadIdx.x;
  u32x4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u)
    if (base + u * 256 < n) v[u] = __builtin_nontemporal_load(src + base + u * 256);
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u)
    if (base + u * 256 < n) __builtin_nontemporal_store(v[u], dst + base + u * 256);
}

}  // namespace
}  // namespace gqe

extern "C" {

int gqe_peak_blocks(void) { return 2 * gqe::cu_count(); }

int gqe_peak_mfma_bf16(float* out, int blocks, int iters, hipStream_t stream) {
  if (out == nullptr || blocks < 1 || iters < 0) return GQE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(gqe::mfma_peak_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, out, iters);
  return hipGetLastError() == hipSuccess ? GQE_OK : GQE_ERR_HIP;
}

int gqe_peak_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return GQE_OK;
  if (dst == nullptr || src == nullptr || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(dst) % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return GQE_ERR_INVALID_ARG;
  const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
  if (d < s + bytes && s < d + bytes) return GQE_ERR_INVALID_ARG;  // overlap
  const size_t n = bytes / 16;
  const size_t blocks = (n + 256 * gqe::kCopyUnroll - 1) / (256 * gqe::kCopyUnroll);
  if (blocks > 0xffffffffu) return GQE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(gqe::copy_peak_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<gqe::u32x4*>(dst), static_cast<const gqe::u32x4*>(src), n);
  return hipGetLastError() == hipSuccess ? GQE_OK : GQE_ERR_HIP;
}

}  // extern "C"

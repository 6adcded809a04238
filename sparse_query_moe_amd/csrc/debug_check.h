// Index checks of debug builds.  A build compiled with -DGQE_DEBUG checks
// every index the kernels take from the routing (expert ids) and from the
// dispatch lists (list extents, positions, slots): a failed check sets its
// bit in the debug word `dbg` (device memory) and the access it guards is
// skipped.  Release builds compile the checks out: dbg_ok is then always true
// and the guarded code is the unchecked code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqe {

enum : uint32_t {
  kDbgExpert = 1u,     // an expert id outside [0, E), or repeated within a group
  kDbgListRange = 2u,  // a list's count or offset outside its (b, g) range
  kDbgPos = 4u,        // a list position outside [0, L)
  kDbgSlot = 8u,       // a list slot outside [0, k_g)
};

__device__ __forceinline__ bool dbg_ok(bool ok, uint32_t* dbg, uint32_t bit) {
#ifdef GQE_DEBUG
  if (!ok && dbg != nullptr) atomicOr(dbg, bit);
  return ok;
#else
  (void)ok;
  (void)dbg;
  (void)bit;
  return true;
#endif
}

}  // namespace gqe

// The causal attention step's launch interface (host side): the parameter
// block the attention kernels read and their launcher.  The attention
// kernel's sources are attention.hip, this header, device_common.h, and the
// headers of the dispatch blocks that can ride in its launch
// (dispatch_dev.h, kernels.h, debug_check.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqe {

// groups (KV heads) a layer may have
constexpr int kMaxGroups = 64;

// ---- K4 attention ------------------------------------------------------------
struct AttnParams {
  const void* q;       // [B, q_heads, L, D]: heads 0 .. H-1 attend
  const void* k;       // [B, G, L, D]
  const void* vt;      // [B, G, vt_tiles, D, 64], keys permuted in 16-key groups
  void* o;             // o[(b*L + t)*ld_o + head*D + d]
  int64_t vt_tiles;
  int64_t ld_o;
  int B, H, G, L;
  int q_heads;          // heads per sequence in q (H, or one more when the shared head is absent)
  int n_grouped;        // heads h < n_grouped read group g with koff[g] <= h < koff[g + 1]
  int koff[kMaxGroups + 1];
  int extra_group;      // heads h >= n_grouped read this group
  float scale_log2;     // softmax scale * log2(e)
  // optional per-row factor of the grouped heads' outputs: o[b, t, h] is
  // multiplied by row_scale[(b*L + t)*n_grouped + h] (h < n_grouped), or NULL
  const float* row_scale;
  // optional [B, H, L]: log2 of each row's softmax normalizer in the units of
  // the scaled scores (max + log2(sum of 2^(s - max))), or NULL
  float* lse;
  // scratch of attention_redo_ints(B, H, L) ints, or NULL: long launches then
  // run the fast path and the fallback as two launches (one flag per block)
  int* redo;
  // optional query gather, or NULL: with it, head h < n_grouped of group g
  // reads row t from head g*q_E + q_idx[(b*L + t)*q_idx_stride + h] of
  // q_src ([B, q_src_heads, L, D]: every expert's query head, then the
  // shared one), any other head from head q_src_heads - 1, and the block
  // stores the rows it read into q at their slot-head and position
  const int32_t* q_idx;
  const void* q_src;
  int q_src_heads, q_E, q_idx_stride;
};
// ints of the per-block flag array of a launch over B x H heads of L rows
inline long long attention_redo_ints(int B, int H, int L) {
  return static_cast<long long>(B) * H * ((L + 31) / 32);
}
// lists: optional (NULL for none): the short forward's dispatch blocks
// (kernels.h, DispatchArgs), run as the launch's first blocks
struct DispatchArgs;
template <typename T>
hipError_t launch_attention(const AttnParams& p, int D, hipStream_t stream,
                            const DispatchArgs* lists = nullptr);

}  // namespace gqe

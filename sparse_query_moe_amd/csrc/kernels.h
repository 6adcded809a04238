// Launchers of the gfx950 kernels (host side).  Every launcher enqueues on
// `stream` and returns the launch status; none synchronizes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attention.h"
#include "device_common.h"

namespace gqe {

typedef uint16_t bf16_t;

// rows of one gathered query-projection tile (the dispatch tile map unit)
constexpr int kGatherRows = 128;

// Experts selected per group: group g owns hard slots koff[g] .. koff[g] +
// kg[g] - 1 of every token, in rank order; K = koff[G] hard slots in all.  A
// uniform top-k is kg[g] = k, koff[g] = g*k (the pages' layer); a per-group k
// is the non-uniform variant the pages list as future work (pptc.cn,
// section 6).  kMaxGroups (attention.h) bounds G.
// compute units of the device (read once)
int cu_count();
struct GroupK {
  int K;
  int kmax;
  int kg[kMaxGroups];
  int koff[kMaxGroups + 1];
};

// ---- K1 router ---------------------------------------------------------------
template <typename T>
// renorm: w = p renormalized over the k selected (the GQE layer); otherwise
// w = p itself, the in-group softmax probability of each selected expert
hipError_t launch_router(const T* x, const T* wr, const float* bias, int32_t* idx, float* w,
                         int n_tokens, int d, int G, int E, const GroupK& gk, bool renorm,
                         hipStream_t stream);

// ---- K2 dispatch -------------------------------------------------------------
// Sequences of at most kDispatchSmallMaxL tokens with every k_g <= 4 are
// dispatched by one block per (b, g).  DispatchArgs carries those blocks into
// another launch (the short forward's attention): `blocks` = B*G of them.
constexpr int kDispatchSmallMaxL = 8192;
struct DispatchArgs {
  const int32_t* idx;
  int32_t *counts, *offsets, *tile_off, *pos, *slot;
  int L, G, E;
  GroupK gk;
  int tile_rows, n_lists, blocks;
  uint32_t* dbg;
};
int dispatch_chunks(int L);
// dbg: the debug word of a debug build's expert-id checks (see launch_project)
hipError_t launch_dispatch(const int32_t* idx, int32_t* chunk_counts, int32_t* counts,
                           int32_t* offsets, int32_t* tile_off, int32_t* pos, int32_t* slot,
                           int B, int L, int G, int E, const GroupK& gk, int tile_rows,
                           uint32_t* dbg, hipStream_t stream);

// ---- K3 projections ----------------------------------------------------------
// One output segment of a dense projection: columns [n_begin, n_begin + n)
// of the concatenated output come from `w` (rows of [out, in] layout) and go
// to head-split tensor `out`, [B, heads, L, D] or, transposed per 64-key tile
// with keys permuted inside 16-key groups, [B, heads, vt_tiles, D, 64].
struct ProjSeg {
  const void* w;
  void* out;
  int n_begin;
  int n;
  int heads;
  int head_base;
  int transposed;
  int rope;        // rotate by position (rope.on): queries and keys
};
// rope: the rotary embedding of the rotated segments (rope.on == 0: none)
template <typename T>
hipError_t launch_dense_proj(const T* x, int M, int K, int L, int D, int64_t vt_tiles,
                             const ProjSeg* segs, int nseg, const RopeTable& rope,
                             hipStream_t stream);

// The dense projection (segments as for launch_dense_proj) and the gathered
// routed-query projection in one launch: for every dispatch list (b, g, e),
// the rows x[b, pos] . Wq[head g*E+e]^T land in slot-head koff[g] + slot at
// their positions.  tile_off is the per-(b, g) tile map written by the
// dispatch.  dbg: the debug word of a debug build's index checks (unused, and
// may be NULL, otherwise).
template <typename T>
hipError_t launch_project(const T* x, int M, int K, int L, int D, int64_t vt_tiles,
                          const ProjSeg* segs, int nseg, const T* wq, T* q,
                          const int32_t* counts, const int32_t* offsets, const int32_t* pos,
                          const int32_t* slot, const int32_t* tile_off, int B, int G, int E,
                          const GroupK& gk, const RopeTable& rope, uint32_t* dbg,
                          hipStream_t stream);

// ---- short sequences: the router beside the dense projection ----------------
// One launch of the bf16 router's blocks (the split form: 16 tokens per block,
// the model dimension over 4 waves) and the dense projection's tiles (segments
// as for launch_dense_proj); neither reads what the other writes.  Requires
// d % 128 == 0, G*E <= 64 and at most kFrontMaxTokens tokens.
constexpr int kFrontMaxTokens = 1 << 15;
struct RouterArgs {
  const bf16_t* wr;
  const float* bias;
  int32_t* idx;
  float* w;
  int G, E;
  GroupK gk;
  int renorm;
};
hipError_t launch_front(const RouterArgs& r, const bf16_t* x, int M, int K, int L, int D,
                        int64_t vt_tiles, const ProjSeg* segs, int nseg, const RopeTable& rope,
                        hipStream_t stream);

// ---- K5 output -----------------------------------------------------------------
// s[t] holds K hard slots, the shared slot and the weighted slot; w is [T, K]
template <typename T>
hipError_t launch_weighted_slot(T* s, const float* w, int n_tokens, int K, int D,
                                hipStream_t stream);
template <typename T>
hipError_t launch_out_proj(const T* a, const T* wo, T* out, int M, int N, int K,
                           hipStream_t stream);
// The weighted slot and the output projection in one launch (bf16, d_h 64,
// `hard` slots, a multiple of 4 and at most 32, then the shared and the
// weighted slot: K = (hard + 2) * 64): the weighted slot is formed from the
// hard slots inside the GEMM's main loop, stored into s (its slot of every
// token), and multiplied with its W_O columns.  out_wslot_ok tells whether a
// shape qualifies; the results equal launch_weighted_slot then
// launch_out_proj bit for bit.
bool out_wslot_ok(int K, int D, int hard);
hipError_t launch_out_proj_wslot(bf16_t* s, const float* w, const bf16_t* wo, bf16_t* out, int M,
                                 int N, int K, int D, int hard, hipStream_t stream);


// ---- backward: C[M, N] = A[M, K] . B[N, K]^T in float32 ------------------------
// Rows of C go to up to four segments: row m in [row_begin, row_begin + rows)
// is stored (or added, when accumulate) at out[(m - row_begin)*ldo + n];
// rows in no segment are dropped.  K must be a multiple of 64 (bf16) or 32
// (fp32) elements.
struct NtSeg {
  float* out;
  int row_begin, rows, ldo, accumulate;
};
struct NtArgs {
  const void* a;
  int lda;
  const void* b;
  int ldb;
  int M, N, K;
  int nseg;
  NtSeg seg[4];
  // split K: with splits > 1, block z multiplies K elements z*kchunk .. and
  // writes float partials part[z][M][N], which are then summed in z order
  // into the segments (launch_nt_gemm sets kchunk)
  float* part;
  int splits, kchunk;
};
// K splits for an NT product whose output tiles alone would leave compute
// units idle (1: no split); part must then hold splits * M * N floats
int nt_gemm_splits(int M, int N, int K);
template <typename T>
hipError_t launch_nt_gemm(const NtArgs& a, hipStream_t stream);

// ---- backward of the layer -----------------------------------------------------
struct BwdParams {
  // inputs of the forward pass and the output gradient
  const void* x;            // [T, d]
  const void* wq;           // query rows, [q_rows, d] (the first qcols are used)
  const void* wk;           // [G*D, d]
  const void* wv;           // [G*D, d]
  const void* wr;           // [G*E, d] or NULL (dense GQA: no router)
  const float* router_bias; // [G*E] or NULL
  const void* wo;           // [d, ws]
  const void* dy;           // [T, d]
  // the forward workspace
  const int32_t* idx;       // [T, K] experts by slot or NULL
  const float* w;           // [T, n_routed] routing weights (p for weighted concatenation) or NULL
  const int32_t* counts;    // [B, G, E] or NULL
  const void* q;            // [B, q_heads, L, D]
  const void* keys;         // [B, G, L, D]
  const void* vt;           // [B, G, vt_tiles, D, 64]
  int64_t vt_tiles;
  const void* s;            // [T, ws]
  const float* lse;         // [B, H, L]
  // gradients (float32, caller-owned)
  float *dx, *dwq, *dwk, *dwv, *dwr, *dbr, *dwo, *aux_loss;
  // scratch
  void *gall, *w_t, *wo_t, *dO, *dOt, *qt, *qs, *kt, *vr, *gall_t, *x_t, *dy_t, *s_t;
  float *ds, *dsum, *dw, *dr, *p_all;
  double* psum;
  // shapes
  int B, L, d, G, E, D;
  GroupK gk;                // experts selected per group and their slot offsets
  int H;                    // attending slot heads
  int q_heads;              // heads allocated in q
  int n_routed;             // slot heads with a routing weight
  int hbeg[kMaxGroups + 1];  // slot heads hbeg[g] .. hbeg[g+1]-1 read group g
  int n_grouped, extra_group;
  int mode;                 // 0 full, 1 hard, 2 weighted concatenation, 3 dense GQA
  int ws;                   // slot width
  int qcols, kcol, vcol, rcol, kcols, kpad;  // column blocks of Gall
  int tpad;                 // tokens rounded up to 64
  int dkv_split;            // dK/dV query-walk splits (dkdv_splits), 1: none
  float* dkv_part;          // [dkv_split, B, G, L, 2*D] float partials when split
  float* gemm_part;         // split-K partials of the weight-gradient products
  int dq_split;             // dQ key-walk splits (dq_splits), 1: none
  float* dq_part;           // [dq_split, B, H, L, D] float partials when split
  float scale, aux_weight;
  RopeTable rope;           // rotary embedding of the forward (on == 0: none)
  uint32_t* dbg;            // debug word of a debug build's expert-id checks (else unused)
};
// dK/dV query-walk splits for a bf16 backward of B x L tokens, G groups, d_h D
int dkdv_splits(int B, int G, int L, int D);
// dQ key-walk splits for a bf16 backward of B x L tokens over H slot heads
int dq_splits(int B, int H, int L);
template <typename T>
hipError_t launch_backward(const BwdParams& p, hipStream_t stream);

// ---- decode: one token per sequence against a KV cache --------------------------
// query heads of one KV group that one decode attention block holds (E <= 32
// dense heads, or k routed heads plus the shared one)
constexpr int kMaxDecodeHeads = 33;

struct DecodeParams {
  const void* x;          // [B, d] the new tokens
  const void* wq;         // query rows, [(G*E + 1)*D, d] (GQE) or [G*E*D, d] (GQA)
  const void* wk;         // [G*D, d]
  const void* wv;         // [G*D, d]
  const void* wo;         // [d, K_out]
  const void* wr;         // [G*E, d] router rows (GQE) or NULL (GQA: no routing)
  const float* router_bias;  // [G*E] or NULL
  int renorm;             // routing weights renormalized over the k selected
  int32_t* idx;           // [B, K] routed experts by slot, or NULL (GQA: every head)
  float* w;               // [B, K] routing weights (GQE) or NULL
  const int32_t* pos;     // [B] position of each new token in its cache
  float* q;               // [B, q_heads, D] scratch: every query head's projection
  void* k_cache;          // [B, G, Lc, D]
  void* vt_cache;         // [B, G, ceil(Lc/64), D, 64], keys permuted in 16-key groups
  float* part;            // [B, Hq, ceil(Lc/chunk), D + 2] scratch
  void* s;                // [B, ld_s] slot vectors (concatenated head outputs)
  const float* row_scale; // [B, n_routed] factor of the routed heads' outputs, or NULL
  void* out;              // [B, d]
  int B, d, G, E, D, Lc;
  GroupK gk;              // GQE: experts per group and their slot offsets
  int q_heads;            // query heads projected per token (G*E, plus the shared head)
  int Hq;                 // slot heads per token (heads that attend)
  int n_routed;           // heads before the shared one (the routed heads)
  int shared_head;        // 1: head n_routed is the shared head
  int shared_kv_group;
  int hbeg[kMaxGroups + 1];  // slot heads hbeg[g] .. hbeg[g+1]-1 read group g (hbeg[G] = n_routed)
  int max_heads;          // most slot heads of one group, the shared one included
  int chunk;              // keys per attention block (decode_chunk)
  float scale;            // softmax scale
  int ld_s, K_out;
  int weighted_slot;      // 1: build the weighted slot after the heads
  RopeTable rope;         // rotary embedding of the new queries and keys (on == 0: none)
};
// keys per decode attention block for B sequences of G groups in a cache of Lc
int decode_chunk(int B, int G, int Lc);
// routing and projections (query heads into q, K and V^T into the caches at
// pos) in one launch ...
template <typename T>
hipError_t launch_decode_front(const DecodeParams& p, hipStream_t stream);
// ... then attention, the merge of its partials into slot vectors, and the
// output projection
template <typename T>
hipError_t launch_decode_attend(const DecodeParams& p, hipStream_t stream);

}  // namespace gqe

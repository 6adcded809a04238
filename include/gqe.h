/*
 * gqe.h -- C ABI of the MI355X (gfx950) Grouped Query Experts prefill layer.
 *
 * The method: "Grouped Query Experts: Mixture-of-Experts on GQA
 * Self-Attention" (arXiv 2606.20945), as described by the pptc.cn review
 * (sections 4.2, 5, 6, 7), the gist.science technical summaries
 * ("Architectuur en Routing" / "Arquitetura e Roteamento") and the
 * hotpaper.ai summary ("core idea", "technical approach").  Inside every
 * grouped-query-attention (GQA) group a per-token router picks k of the E
 * query-head experts; K and V stay dense; the selected heads and one
 * always-on shared head attend causally to their group's K/V; the outputs
 * form k*G hard slots, a shared slot and one renormalized weighted slot,
 * which W_O (k*G+2 slots wide) projects back to d_model.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer is a DEVICE pointer owned by the caller, except `cfg` and
 *    `layout`, which are host pointers read (or written) before the call
 *    returns.  The library never allocates or frees device memory and holds
 *    no global mutable state, except gqe_forward_noalloc's per-device scratch
 *    array (described there) and, in a debug build, the per-device debug
 *    word (below).  Every call is thread-safe; calls that share a
 *    workspace must not overlap.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    default stream), and only on `stream`.  No call synchronizes the host.
 *    An argument error is returned before anything is enqueued.  A call that
 *    returns GQE_ERR_HIP (a launch the runtime rejected) may have enqueued
 *    the stages before the failing launch.  A fault inside a kernel surfaces
 *    at the caller's next synchronization of `stream`.
 *  - Weights use the [out, in] layout of nn.Linear (below), not the [in, out]
 *    layout of a plain x.W product: with it both operands of every projection
 *    are contiguous along the reduction dimension, which is how the matrix
 *    cores take them (16-byte vector loads along K for both).
 *  - Tensors are contiguous and row-major.  Element type `cfg->dtype`:
 *    bfloat16 (GQE_DTYPE_BF16) or float32 (GQE_DTYPE_FP32) for x, every
 *    weight and `out`; router bias and weights w are float32; indices int32.
 *  - Weights use the [out, in] layout of a PyTorch nn.Linear weight:
 *      Wq  [(G*E+1)*d_h, d_model]  head h = g*E+e owns rows h*d_h .. h*d_h+d_h-1;
 *                                  the shared head owns the last d_h rows
 *      Wk, Wv [G*d_h, d_model]     group g owns rows g*d_h .. g*d_h+d_h-1
 *      Wr  [G*E, d_model]          router row of expert e of group g is g*E+e
 *      Wo  [d_model, (k*G+2)*d_h]  input columns: hard slot g*k+j, then the
 *                                  shared slot (k*G), then the weighted slot
 *  - x is [B, L, d_model]; out is [B, L, d_model] and must not alias any
 *    input or the workspace.  Device pointers must be 16-byte aligned
 *    (router_bias: 4-byte).
 *  - B*L == 0 is valid: nothing is launched and GQE_OK is returned.
 *  - Debug build (libgqe_debug.so, compiled with -DGQE_DEBUG): the kernels
 *    check every index they take from the routing (expert ids in [0, E),
 *    distinct within a group) and from the dispatch lists (each list inside
 *    its (b, g) range, positions in [0, L), slots in [0, k_g)), and skip the
 *    access a failed check guards.  gqe_dispatch, gqe_project, gqe_forward,
 *    gqe_forward_noalloc and gqe_backward then synchronize `stream`, read and
 *    clear a per-device debug word, and return GQE_ERR_DEBUG if a check
 *    failed (the outputs are then unspecified).  Release builds compile the
 *    checks out, never synchronize and never return GQE_ERR_DEBUG.
 */
#ifndef GQE_H_
#define GQE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQE_OK = 0,
  GQE_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad size or field  */
  GQE_ERR_UNSUPPORTED = -2,   /* valid but not built: e.g. head_dim 96       */
  GQE_ERR_WORKSPACE = -3,     /* ws_bytes smaller than gqe_workspace_bytes() */
  GQE_ERR_HIP = -4,           /* a launch was rejected by the HIP runtime    */
  GQE_ERR_DEBUG = -5          /* debug builds only: an index check failed    */
} gqe_status;

typedef enum { GQE_DTYPE_BF16 = 0, GQE_DTYPE_FP32 = 1 } gqe_dtype;

/* How the attention outputs become W_O's input (pptc.cn review, section 4.3,
 * Table 1: the output constructions compared in the ablation).
 *   GQE_OUTPUT_FULL             the GQE layer: k*G hard slots, the always-on
 *                               shared head's slot and the renormalized
 *                               weighted slot; W_O [d_model, (k*G+2)*d_h].
 *   GQE_OUTPUT_HARD             hard concatenation only: the k*G hard slots;
 *                               no shared head, no weighted slot;
 *                               W_O [d_model, k*G*d_h].
 *   GQE_OUTPUT_WEIGHTED_CONCAT  the k*G hard slots, each scaled by its
 *                               expert's in-group softmax probability p (not
 *                               renormalized over the k); no shared head, no
 *                               weighted slot; W_O [d_model, k*G*d_h].  ws.w
 *                               then holds p instead of the renormalized w. */
typedef enum {
  GQE_OUTPUT_FULL = 0,
  GQE_OUTPUT_HARD = 1,
  GQE_OUTPUT_WEIGHTED_CONCAT = 2
} gqe_output_mode;

/* Layer shape.  Limits (GQE_ERR_INVALID_ARG when broken): batch, seq_len >= 0;
 * d_model a positive multiple of 8; 1 <= n_groups; 1 <= n_experts <= 32;
 * 1 <= top_k <= n_experts; n_groups*n_experts <= 64;
 * 0 <= shared_kv_group < n_groups; batch*seq_len*n_groups*n_experts < 2^31;
 * output_mode a gqe_output_mode; every group_top_k[g] (when set) in
 * [1, n_experts].  Below, k*G stands for the total K of selected experts
 * (sum of group_top_k, or top_k*G): the hard slots are group-major, group g's
 * k_g slots in rank order, and batch*seq_len*K < 2^31.
 * Built subset (GQE_ERR_UNSUPPORTED otherwise): head_dim in {32, 64, 128};
 * group_top_k on every call (prefill, decode and backward);
 * the projections stream their reduction dimension in 128-byte steps, so
 * d_model, the slot width ((top_k*n_groups+2)*head_dim, or
 * top_k*n_groups*head_dim for the ablation outputs) and
 * n_groups*n_experts*head_dim must be multiples of 64 elements for bf16 and
 * of 32 for fp32. */
typedef struct gqe_config {
  int32_t batch;            /* B                                               */
  int32_t seq_len;          /* L: prefill length, causal, no padding          */
  int32_t d_model;          /* d                                               */
  int32_t n_groups;         /* G: KV heads = GQA groups                        */
  int32_t n_experts;        /* E: routed query-head experts per group          */
  int32_t top_k;            /* k: experts selected per token in every group    */
  int32_t head_dim;         /* d_h                                             */
  int32_t shared_kv_group;  /* KV group read by the always-on shared head      */
  int32_t dtype;            /* gqe_dtype                                       */
  float softmax_scale;      /* attention scale; 0 selects 1/sqrt(head_dim)     */
  const float* router_bias; /* device float32 [G*E] added to the logits, or NULL */
  int32_t output_mode;      /* gqe_output_mode (GQE layer only)                */
  const int32_t* group_top_k; /* host int32 [G]: experts selected in group g (the
                               * non-uniform k the pages list as future work,
                               * pptc.cn section 6), or NULL for top_k in every
                               * group.  Read during each call. */
  float rope_base;          /* rotary position embedding of queries and keys, an
                             * option the pages do not name: 0 = none (the
                             * layer of the pages); b > 0 turns dims (2j, 2j+1)
                             * of every query head and key head at position t
                             * by t * b^(-2j/head_dim) after the projections
                             * (RoFormer's interleaved form); values are never
                             * turned.  Prefill, decode and backward; not with
                             * group_top_k (GQE_ERR_UNSUPPORTED). */
} gqe_config;

/* Byte offsets into the workspace of every intermediate, so that callers can
 * read (or seed) them.  All offsets are 256-byte aligned.
 *   idx     int32 [B, L, G, k]   selected experts, best first (per-group k:
 *                                [B, L, K], group g at its slot offset)
 *   w       float [B, L, G, k]   renormalized router weights (same layout)
 *   counts  int32 [B*G*E]        tokens routed to expert e of (b, g)
 *   offsets int32 [B*G*E+1]      exclusive prefix sum of counts, (b,g,e) order
 *   pos     int32 [B*L*G*k]      list (b,g,e) at offsets[(b*G+g)*E+e]: the
 *   slot    int32 [B*L*G*k]      ascending positions t that chose e, and the
 *                                rank j at which they chose it
 *   q       dtype [B, k*G+1, L, d_h]   queries per slot-head (hard slot g*k+j,
 *                                      then the shared head)
 *   k       dtype [B, G, L, d_h]       keys
 *   vt      dtype [B, G, vt_tiles, d_h, 64]  values, transposed per tile of
 *                                64 keys (vt_tiles = ceil(L/64)); inside
 *                                every 16-key group, key 8a+4u+r (a, u in
 *                                {0,1}, r < 4) sits at column 8u+4a+r, the
 *                                order in which the attention kernel feeds
 *                                keys to the matrix cores; the columns of
 *                                keys >= L in the last tile are zero
 *   s       dtype [B, L, (k*G+2)*d_h]  slot vectors (input of W_O)
 *   lse     float [B, k*G+1, L]  per slot-head row: log2 of the softmax
 *                                normalizer of its scores scaled by
 *                                softmax_scale*log2(e) (max + log2 of the sum
 *                                of 2^(score - max)); read by the backward
 *   the rest is private scratch (dispatch partial counts, tile maps). */
typedef struct gqe_ws_layout {
  size_t idx, w, counts, offsets, pos, slot;
  size_t q, k, vt, s, lse;
  size_t scratch;
  size_t total;
  int64_t vt_tiles;
} gqe_ws_layout;

/* Workspace size in bytes for gqe_forward and its stages (0 when cfg is
 * invalid).  Monotone in B and L. */
size_t gqe_workspace_bytes(const gqe_config* cfg);
int gqe_workspace_layout(const gqe_config* cfg, gqe_ws_layout* layout);

/* Router of every token (pptc.cn section 7: softmax first, then top-k, inside
 * each group; hotpaper.ai technical approach: renormalized scoring; pptc.cn
 * section 5: every group takes part).  Logits r = x . Wr^T + router_bias are
 * accumulated in float64; the k largest of each group are written to
 * ws.idx in rank order (ties to the lower expert index) and their weights,
 * softmax over the selected logits (equal to the in-group softmax
 * renormalized over the k), to ws.w. */
int gqe_route(const gqe_config* cfg, const void* x, const void* Wr,
              void* workspace, size_t ws_bytes, hipStream_t stream);

/* Per-(b, g, e) token lists from ws.idx (pptc.cn section 6: the sparse
 * scheduling cost): ws.counts, ws.offsets, ws.pos, ws.slot as described in
 * gqe_ws_layout.  Deterministic: no atomics decide any order. */
int gqe_dispatch(const gqe_config* cfg, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Projections (gist.science, Architectuur en Routing: the K/V path stays
 * dense and only the query side is sparse).  Dense: K, V (transposed) and the
 * shared head's queries for every token.  Gathered: for every list (b,g,e),
 * the query rows x[pos] . Wq[head g*E+e]^T, written to slot-head g*k+slot at
 * their original positions.  Reads ws.offsets/pos/slot. */
int gqe_project(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                const void* Wv, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Causal attention of every slot-head row against its group's dense K/V
 * (pptc.cn section 5: a token that skips an expert still attends with the
 * experts it chose to that group's KV head; the shared head reads group
 * shared_kv_group).  Writes the hard slots and the shared slot of ws.s. */
int gqe_attention(const gqe_config* cfg, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Output construction (gist.science, Architectuur en Routing: hard
 * concatenation, renormalized weighted sum, always-on shared head;
 * hotpaper.ai: W_O of k*G+2 slots): the weighted slot
 * sum_g sum_j w[t,g,j] * o[t,g,j] is written to ws.s, then out = s . Wo^T
 * with float32 accumulation and one final rounding. */
int gqe_output(const gqe_config* cfg, const void* Wo, void* out, void* workspace,
               size_t ws_bytes, hipStream_t stream);

/* The whole GQE prefill layer: the work of gqe_route, gqe_dispatch,
 * gqe_project, gqe_attention and gqe_output, in that order on `stream` (the
 * dense and the gathered projections share one launch).  Works under HIP
 * graph capture of `stream`, first call included.
 *
 * Short bf16 layers (gqe_forward_is_short) take three launches instead: the
 * router beside one dense projection of every expert's query head (with the
 * shared head, K and V^T), the dispatch lists' blocks beside the attention,
 * which reads each slot-head's query row through the routing indices, and
 * W_O with the weighted slot formed in its main loop (as gqe_output does for
 * every bf16 layer with d_h 64).  The workspace (every view of gqe_ws_layout) and `out` are then
 * bit for bit what the staged calls produce; the workspace also holds the
 * all-heads projection (gqe_workspace_bytes counts it). */
int gqe_forward(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                const void* Wv, const void* Wr, const void* Wo, void* out,
                void* workspace, size_t ws_bytes, hipStream_t stream);

/* 1 when gqe_forward takes the short-layer launches for `cfg`: bf16 storage,
 * d_model a multiple of 128, G*E <= 64, at most 4096 tokens (batch * seq_len)
 * and every k_g <= 4; 0 otherwise; a negative status for an
 * invalid cfg.  Host only: launches nothing. */
int gqe_forward_is_short(const gqe_config* cfg);

/* gqe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * workspace is a library-owned array of GQE_NOALLOC_SCRATCH_BYTES in device
 * memory, one per device, which the device holds from the first use of the
 * library on it until the process ends.  The call allocates and frees
 * nothing.  Every call on a device shares that device's array, so calls that
 * overlap on one device (other streams, other threads) race; the routing
 * and other intermediates of the last call stay in it and are not exposed.
 * Returns GQE_ERR_WORKSPACE when the layer's workspace
 * (gqe_workspace_bytes(cfg)) exceeds GQE_NOALLOC_SCRATCH_BYTES (32 MiB:
 * e.g. B*L <= 8192 tokens of the d_model 1024, G 4, E 4, k 2, d_h 64 layer),
 * and otherwise what gqe_forward returns. */
#define GQE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int gqe_forward_noalloc(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                        const void* Wv, const void* Wr, const void* Wo, void* out,
                        hipStream_t stream);

/* Dense GQA baseline, all G*E query heads active (pptc.cn section 4.2: the
 * all-active comparison model).  Wq [G*E*d_h, d_model], Wo [d_model, G*E*d_h];
 * head h reads KV group h / E.  top_k, shared_kv_group and router_bias are
 * ignored.  Workspace: q [B, G*E, L, d_h], k, vt as above, o [B, L, G*E*d_h]
 * (reported in the layout's `s` field). */
size_t gqa_workspace_bytes(const gqe_config* cfg);
int gqa_workspace_layout(const gqe_config* cfg, gqe_ws_layout* layout);
int gqa_project(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                const void* Wv, void* workspace, size_t ws_bytes, hipStream_t stream);
int gqa_attention(const gqe_config* cfg, void* workspace, size_t ws_bytes, hipStream_t stream);
int gqa_output(const gqe_config* cfg, const void* Wo, void* out, void* workspace,
               size_t ws_bytes, hipStream_t stream);
int gqa_forward(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                const void* Wv, const void* Wo, void* out, void* workspace, size_t ws_bytes,
                hipStream_t stream);

/* ---- Decode: one new token per sequence against a KV cache -----------------
 *
 * The pages analyse prefill only (pptc.cn, section 6: decode is named as not
 * analysed).  A decode step is the same layer evaluated at one position: the
 * row t = pos[b] of the prefill layer over the sequence whose keys and values
 * for positions < t are those in the cache.  For decode, cfg->batch is the
 * number of sequences B (one new token each) and cfg->seq_len the cache
 * capacity Lc >= 1; every other field means what it means for prefill, and
 * the same limits and built subset apply, plus d_model <= 16384
 * (GQE_ERR_UNSUPPORTED otherwise).
 *
 *   x         dtype [B, d_model]              the new tokens
 *   Wq..Wo    as for gqe_forward / gqa_forward
 *   k_cache   dtype [B, G, Lc, d_h]           keys, read for positions
 *                                             <= pos[b]
 *   vt_cache  dtype [B, G, ceil(Lc/64), d_h, 64]  values in the layout of
 *                                             gqe_ws_layout.vt (64-key tiles,
 *                                             keys permuted in 16-key groups);
 *                                             columns past pos[b] are never
 *                                             read (no zero fill needed)
 *   pos       device int32 [B]                position of each new token
 *   out       dtype [B, d_model]
 *
 * The step writes the new token's key and value into both caches at pos[b]
 * (caller-owned, updated in place), routes the tokens as gqe_route does
 * (float64 logits, summed in another fixed order; renormalized weights, or p
 * for GQE_OUTPUT_WEIGHTED_CONCAT), lets
 * every active query head attend to cache positions 0..pos[b] of its group,
 * and projects the slot vectors through Wo as gqe_output does.  pos is read
 * on the device only: a pos[b] outside [0, Lc) touches no cache entry and
 * yields zero head outputs for that sequence (out = 0 . Wo).  The workspace
 * (size from the *_decode_workspace_bytes call, 16-byte aligned) is private
 * scratch; a call may overlap nothing else that uses the same workspace or
 * caches.  Returns GQE_ERR_INVALID_ARG for a NULL or misaligned pointer
 * (16 bytes; 4 for pos), GQE_ERR_WORKSPACE when ws_bytes is too small, and
 * GQE_OK with nothing enqueued when B == 0. */
size_t gqe_decode_workspace_bytes(const gqe_config* cfg);
int gqe_decode(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
               const void* Wv, const void* Wr, const void* Wo, void* k_cache, void* vt_cache,
               const int32_t* pos, void* out, void* workspace, size_t ws_bytes,
               hipStream_t stream);

/* Dense GQA decode step (all G*E heads; head h reads group h / E). */
size_t gqa_decode_workspace_bytes(const gqe_config* cfg);
int gqa_decode(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
               const void* Wv, const void* Wo, void* k_cache, void* vt_cache, const int32_t* pos,
               void* out, void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---- Backward: gradients of <y, dy> + aux_weight * L_aux ----------------------
 *
 * gist.science, Architectuur en Routing and Training en Loss: the top-k choice
 * has no gradient; the loss reaches the router through the weighted slot
 * (through the scaled slots for GQE_OUTPUT_WEIGHTED_CONCAT), and a
 * load-balancing auxiliary loss spreads each group's tokens over its experts.
 * The pages give no formula for that loss; L_aux here is
 *     (E / G) * sum_g sum_e f[g, e] * P[g, e],
 * f[g, e] = (routed slots of group g that chose e) / (B * L * k), which is a
 * count and carries no gradient, and P[g, e] = the mean over all tokens of
 * the in-group softmax p[t, g, e].
 *
 * fwd_workspace is the workspace of a gqe_forward (gqa_forward) call on the
 * same cfg and inputs, unchanged since: the backward reads the routing, the
 * queries, K, V^T, the slot vectors and the per-row log-sum-exp from it.
 * dy has the dtype of the layer, [B, L, d_model].  Every gradient is float32,
 * caller-owned, and overwritten:
 *   dx [B, L, d_model]; dWq, dWk, dWv, dWr, dWo with the shapes of Wq, Wk,
 *   Wv, Wr, Wo; dbr [G*E] (gradient of a router bias, whether or not
 *   cfg->router_bias is set); aux_loss: one float, the value of L_aux.
 * For the ablation outputs the shared head's rows of dWq are zero.  The
 * workspace (size from *_backward_workspace_bytes, 16-byte aligned) is
 * private scratch.  Returns GQE_ERR_INVALID_ARG for a NULL or misaligned
 * pointer (16 bytes; 4 for dbr and aux_loss) or a negative or infinite
 * aux_weight, GQE_ERR_WORKSPACE when either workspace is too small, and
 * GQE_OK with nothing enqueued when B*L == 0. */
size_t gqe_backward_workspace_bytes(const gqe_config* cfg);
int gqe_backward(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                 const void* Wv, const void* Wr, const void* Wo, const void* dy, float aux_weight,
                 const void* fwd_workspace, size_t fwd_ws_bytes, float* dx, float* dWq, float* dWk,
                 float* dWv, float* dWr, float* dbr, float* dWo, float* aux_loss, void* workspace,
                 size_t ws_bytes, hipStream_t stream);

/* Dense GQA backward (gradients of <y, dy>; no router, no auxiliary loss). */
size_t gqa_backward_workspace_bytes(const gqe_config* cfg);
int gqa_backward(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                 const void* Wv, const void* Wo, const void* dy, const void* fwd_workspace,
                 size_t fwd_ws_bytes, float* dx, float* dWq, float* dWk, float* dWv, float* dWo,
                 void* workspace, size_t ws_bytes, hipStream_t stream);

/* Measurement probes (diagnostics, not steps of the layer): what this device
 * sustains, as the second reference beside the published peaks (bf16 matrix
 * cores 2.5166 PFLOP/s at the nominal 2.4 GHz, HBM 8 TB/s).  Both enqueue one
 * kernel on `stream` and return at once; the caller times them.
 *
 * gqe_peak_blocks: the grid gqe_peak_mfma_bf16 should get to load every SIMD
 * with two waves (2 blocks of 256 threads per compute unit, all resident).
 *
 * gqe_peak_mfma_bf16: blocks x 256 threads, each wave running `iters` rounds
 * of four independent v_mfma_f32_32x32x16_bf16 chains and nothing else:
 * blocks * 4 * iters * 4 * 32768 flop in all.  out (device, blocks * 256
 * floats, caller-owned) receives one finite sum per thread.  Returns
 * GQE_ERR_INVALID_ARG for a NULL out, blocks < 1 or iters < 0.
 *
 * gqe_peak_copy: copies `bytes` from src to dst (device, 16-byte aligned,
 * not overlapping, bytes a multiple of 16) in 16-byte loads and stores:
 * `bytes` read and `bytes` written.  Returns GQE_OK with nothing enqueued
 * when bytes == 0 (the pointers are then not looked at), and
 * GQE_ERR_INVALID_ARG for a NULL, misaligned or overlapping pair or a size
 * that is not a multiple of 16. */
int gqe_peak_blocks(void);
int gqe_peak_mfma_bf16(float* out, int blocks, int iters, hipStream_t stream);
int gqe_peak_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

/* Static text for a gqe_status value; never NULL. */
const char* gqe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GQE_H_ */

// C ABI of the GQE prefill layer: argument validation, workspace layout and
// the launch sequence of every stage (declared in include/gqe.h).
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/gqe.h"
#include "kernels.h"

using namespace gqe;

#ifdef GQE_DEBUG
// the debug word of the index checks of a debug build (see debug_check.h)
static __device__ uint32_t debug_word[1];
#endif

namespace {

constexpr int kMaxDevices = 64;

// The device address of a file-scope __device__ array on the device of
// `stream`, resolved with hipGetSymbolAddress once per device (with that
// device current) and kept in `table`.  Host code never uses such a name as
// an address: on the host it stands for a host-side shadow.
int symbol_on_device(const void* symbol, void** table, std::mutex& mu, hipStream_t stream,
                     void** addr) {
  int dev = -1;
  const hipError_t e = stream == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return GQE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GQE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (table[dev] == nullptr) {  // first call on this device (retried after a failure)
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return GQE_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return GQE_ERR_HIP;
    void* p = nullptr;
    const hipError_t ge = hipGetSymbolAddress(&p, symbol);
    if (cur != dev) (void)hipSetDevice(cur);
    if (ge != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return GQE_ERR_HIP;
    }
    table[dev] = p;
  }
  *addr = table[dev];
  return GQE_OK;
}

// Debug builds: the kernels that take indices from the routing or the
// dispatch lists get the device's debug word; after its launches an entry
// point waits for them, reads and clears the word, and returns GQE_ERR_DEBUG
// when a check failed.  Release builds pass NULL and return at once.
#ifdef GQE_DEBUG
std::mutex g_debug_mutex;
void* g_debug_addr[kMaxDevices];
uint32_t* debug_word_of(hipStream_t stream) {
  void* p = nullptr;
  return symbol_on_device(HIP_SYMBOL(debug_word), g_debug_addr, g_debug_mutex, stream, &p) == GQE_OK
             ? static_cast<uint32_t*>(p)
             : nullptr;
}
int debug_collect(hipStream_t stream, int st) {
  if (st != GQE_OK) return st;
  uint32_t* p = debug_word_of(stream);
  if (p == nullptr || hipStreamSynchronize(stream) != hipSuccess) return GQE_ERR_HIP;
  uint32_t v = 0;
  if (hipMemcpy(&v, p, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return GQE_ERR_HIP;
  if (v == 0) return GQE_OK;
  const uint32_t zero = 0;
  if (hipMemcpy(p, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return GQE_ERR_HIP;
  return GQE_ERR_DEBUG;
}
#else
uint32_t* debug_word_of(hipStream_t) { return nullptr; }
int debug_collect(hipStream_t, int st) { return st; }
#endif

constexpr size_t kAlign = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t elem_bytes(const gqe_config* c) { return c->dtype == GQE_DTYPE_BF16 ? 2 : 4; }

bool shape_ok(const gqe_config* c) {
  if (c == nullptr) return false;
  if (c->batch < 0 || c->seq_len < 0) return false;
  if (c->d_model < 8 || c->d_model % 8 != 0) return false;
  if (c->n_groups < 1 || c->n_experts < 1 || c->n_experts > 32) return false;
  if (c->n_groups * c->n_experts > 64) return false;
  if (c->top_k < 1 || c->top_k > c->n_experts) return false;
  if (c->shared_kv_group < 0 || c->shared_kv_group >= c->n_groups) return false;
  if (c->dtype != GQE_DTYPE_BF16 && c->dtype != GQE_DTYPE_FP32) return false;
  if (!(c->softmax_scale >= 0.f) || isinf(c->softmax_scale)) return false;
  if (c->group_top_k != nullptr)  // n_groups <= 64 here
    for (int g = 0; g < c->n_groups; ++g)
      if (c->group_top_k[g] < 1 || c->group_top_k[g] > c->n_experts) return false;
  long long K = 0;
  for (int g = 0; g < c->n_groups; ++g) K += c->group_top_k ? c->group_top_k[g] : c->top_k;
  const long long rows = static_cast<long long>(c->batch) * c->seq_len * K;
  if (rows >= (1LL << 31)) return false;
  if (static_cast<long long>(c->batch) * c->seq_len * c->n_groups * c->n_experts >= (1LL << 31))
    return false;
  if (c->output_mode < GQE_OUTPUT_FULL || c->output_mode > GQE_OUTPUT_WEIGHTED_CONCAT) return false;
  if (!(c->rope_base >= 0.f) || isinf(c->rope_base)) return false;
  return true;
}

// experts selected in group g, and their sum over the groups (the hard slots)
int group_k(const gqe_config* c, int g) { return c->group_top_k ? c->group_top_k[g] : c->top_k; }
int total_k(const gqe_config* c) {
  int K = 0;
  for (int g = 0; g < c->n_groups; ++g) K += group_k(c, g);
  return K;
}
int max_k(const gqe_config* c) {
  int m = 0;
  for (int g = 0; g < c->n_groups; ++g) m = group_k(c, g) > m ? group_k(c, g) : m;
  return m;
}
GroupK make_group_k(const gqe_config* c) {
  GroupK gk{};
  gk.koff[0] = 0;
  for (int g = 0; g < c->n_groups; ++g) {
    gk.kg[g] = group_k(c, g);
    gk.koff[g + 1] = gk.koff[g] + gk.kg[g];
  }
  gk.K = gk.koff[c->n_groups];
  gk.kmax = max_k(c);
  return gk;
}

// the full GQE output has the shared head's slot and the weighted slot after
// the k*G hard slots; the ablation outputs only the hard slots
bool full_output(const gqe_config* c) { return c->output_mode == GQE_OUTPUT_FULL; }
int slot_count(const gqe_config* c) { return total_k(c) + (full_output(c) ? 2 : 0); }

bool head_dim_ok(const gqe_config* c) {
  return c->head_dim == 32 || c->head_dim == 64 || c->head_dim == 128;
}

// The projections stream K in steps of 128 bytes (64 bf16 or 32 fp32
// elements): d_model, the slot width and the dense head width G*E*d_h must be
// multiples of it.
bool k_steps_ok(const gqe_config* c) {
  const int step = c->dtype == GQE_DTYPE_BF16 ? 64 : 32;
  const int D = c->head_dim;
  return c->d_model % step == 0 && (slot_count(c) * D) % step == 0 &&
         (c->n_groups * c->n_experts * D) % step == 0;
}

int check_cfg(const gqe_config* c) {
  if (c == nullptr) return GQE_ERR_INVALID_ARG;
  if (c->head_dim < 1) return GQE_ERR_INVALID_ARG;
  if (!shape_ok(c)) return GQE_ERR_INVALID_ARG;
  if (!head_dim_ok(c) || !k_steps_ok(c)) return GQE_ERR_UNSUPPORTED;
  if (c->rope_base > 0.f && c->group_top_k != nullptr) return GQE_ERR_UNSUPPORTED;
  return GQE_OK;
}

// theta_j = base^(-2j/d_h) of the rotary embedding, in float64
RopeTable make_rope(const gqe_config* c) {
  RopeTable r{};
  r.on = c->rope_base > 0.f ? 1 : 0;
  if (r.on)
    for (int j = 0; j < c->head_dim / 2 && j < 64; ++j)
      r.theta[j] = pow(static_cast<double>(c->rope_base), -2.0 * j / c->head_dim);
  return r;
}

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
  gqe_ws_layout pub;
  size_t chunk_counts, tile_off, redo;
  size_t qall;  // short forward: every expert's query head, then the shared one
};

// Short bf16 layers take the one-pass front (forward_short): at most
// kShortTokens tokens (measured: 68 -> 54 us at 2048 tokens, 110 -> 101 us at
// 4096, and 3% slower than the staged launches at 8192, where the extra
// query heads' projection work no longer hides), sequences the one-block
// dispatch covers, and a router in its split bf16 form.
constexpr long long kShortTokens = 4096;
bool short_forward(const gqe_config* c) {
  return c->dtype == GQE_DTYPE_BF16 && c->d_model % 128 == 0 &&
         c->n_groups * c->n_experts <= 64 &&
         static_cast<long long>(c->batch) * c->seq_len <= kShortTokens &&
         c->seq_len <= kDispatchSmallMaxL && max_k(c) <= 4;
}

// slot-heads that attend: every routed slot and the shared head (full
// output), or all G*E dense heads
int attn_heads(const gqe_config* c, bool dense) {
  return dense ? c->n_groups * c->n_experts
               : total_k(c) + (full_output(c) ? 1 : 0);
}

// Workspace of gqe_forward (dense == false) or gqa_forward (dense == true).
Layout make_layout(const gqe_config* c, bool dense) {
  const size_t B = c->batch, L = c->seq_len, G = c->n_groups, E = c->n_experts;
  const size_t D = c->head_dim, es = elem_bytes(c);
  const size_t vt_tiles = (L + 63) / 64;
  Layout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, kAlign);
    return o;
  };
  if (!dense) {
    const size_t rows = B * L * static_cast<size_t>(total_k(c));
    const size_t lists = B * G * E;
    l.pub.idx = take(rows * 4);
    l.pub.w = take(rows * 4);
    l.pub.counts = take(lists * 4);
    l.pub.offsets = take((lists + 1) * 4);
    l.pub.pos = take(rows * 4);
    l.pub.slot = take(rows * 4);
    l.pub.scratch = off;
    l.chunk_counts = take(B * static_cast<size_t>(dispatch_chunks(static_cast<int>(L))) * G * E * 4);
    l.tile_off = take(B * G * (E + 1) * 4);
    l.pub.q = take(B * (static_cast<size_t>(total_k(c)) + 1) * L * D * es);
    l.pub.s = 0;
  } else {
    l.pub.q = take(B * G * E * L * D * es);
  }
  l.pub.k = take(B * G * L * D * es);
  l.pub.vt = take(B * G * vt_tiles * D * 64 * es);
  l.pub.s = take(B * L * (dense ? G * E : static_cast<size_t>(slot_count(c))) * D * es);
  l.pub.lse = take(B * L * static_cast<size_t>(attn_heads(c, dense)) * 4);
  if (dense) l.pub.scratch = off;
  l.redo = take(static_cast<size_t>(attention_redo_ints(c->batch, attn_heads(c, dense),
                                                        c->seq_len)) * 4);
  if (!dense && short_forward(c)) l.qall = take(B * (G * E + 1) * L * D * es);
  l.pub.total = off;
  l.pub.vt_tiles = static_cast<int64_t>(vt_tiles);
  return l;
}

float softmax_scale(const gqe_config* c) {
  return c->softmax_scale > 0.f ? c->softmax_scale : 1.0f / sqrtf(static_cast<float>(c->head_dim));
}
float scale_log2(const gqe_config* c) { return softmax_scale(c) * 1.4426950408889634f; }

int hip_status(hipError_t e) { return e == hipSuccess ? GQE_OK : GQE_ERR_HIP; }

template <typename T> T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// common entry checks: cfg, workspace.  Returns GQE_OK or an error status.
int check_common(const gqe_config* c, void* ws, size_t ws_bytes, bool dense) {
  int st = check_cfg(c);
  if (st != GQE_OK) return st;
  if (static_cast<long long>(c->batch) * c->seq_len == 0) return GQE_OK;
  if (!aligned16(ws)) return GQE_ERR_INVALID_ARG;
  if (ws_bytes < make_layout(c, dense).pub.total) return GQE_ERR_WORKSPACE;
  return GQE_OK;
}

bool empty(const gqe_config* c) { return static_cast<long long>(c->batch) * c->seq_len == 0; }

// Upper bound of the gathered-projection tiles of one (b, g): its lists hold
// L*k rows in E lists.
template <typename T>
int project_impl(const gqe_config* c, const void* x, const void* wq, const void* wk,
                 const void* wv, void* ws, bool dense, hipStream_t stream) {
  const Layout l = make_layout(c, dense);
  const int B = c->batch, L = c->seq_len, d = c->d_model, G = c->n_groups, E = c->n_experts;
  const int D = c->head_dim;
  ProjSeg seg[3];
  const bool shared = dense || full_output(c);  // the ablation outputs have no shared head
  const int nq_cols = dense ? G * E * D : shared ? D : 0;
  seg[0].w = dense ? wq : static_cast<const void*>(static_cast<const T*>(wq) +
                                                    static_cast<size_t>(G) * E * D * d);
  seg[0].out = at<T>(ws, l.pub.q);
  seg[0].n_begin = 0;
  seg[0].n = nq_cols;
  const int K = total_k(c);
  seg[0].heads = dense ? G * E : K + 1;
  seg[0].head_base = dense ? 0 : K;
  seg[0].transposed = 0;
  seg[0].rope = 1;
  seg[1].w = wk;
  seg[1].out = at<T>(ws, l.pub.k);
  seg[1].n_begin = nq_cols;
  seg[1].n = G * D;
  seg[1].heads = G;
  seg[1].head_base = 0;
  seg[1].transposed = 0;
  seg[1].rope = 1;
  seg[2].w = wv;
  seg[2].out = at<T>(ws, l.pub.vt);
  seg[2].n_begin = nq_cols + G * D;
  seg[2].n = G * D;
  seg[2].heads = G;
  seg[2].head_base = 0;
  seg[2].transposed = 1;
  seg[2].rope = 0;
  if (dense)
    return hip_status(launch_dense_proj<T>(static_cast<const T*>(x), B * L, d, L, D,
                                           l.pub.vt_tiles, seg, 3, make_rope(c), stream));
  // dense tiles and gathered routed-query tiles in one launch
  return hip_status(launch_project<T>(
      static_cast<const T*>(x), B * L, d, L, D, l.pub.vt_tiles, shared ? seg : seg + 1,
      shared ? 3 : 2, static_cast<const T*>(wq), at<T>(ws, l.pub.q), at<int32_t>(ws, l.pub.counts),
      at<int32_t>(ws, l.pub.offsets), at<int32_t>(ws, l.pub.pos), at<int32_t>(ws, l.pub.slot),
      at<int32_t>(ws, l.tile_off), B, G, E, make_group_k(c), make_rope(c), debug_word_of(stream),
      stream));
}

// gather: the short forward's attention, whose slot-heads read their query
// rows from the all-heads projection through the routing indices (and store
// them into q)
template <typename T>
int attention_impl(const gqe_config* c, void* ws, bool dense, hipStream_t stream,
                   bool gather = false, const DispatchArgs* lists = nullptr) {
  const Layout l = make_layout(c, dense);
  const int G = c->n_groups, E = c->n_experts, D = c->head_dim;
  AttnParams p{};
  if (gather) {
    p.q_idx = at<int32_t>(ws, l.pub.idx);
    p.q_src = at<T>(ws, l.qall);
    p.q_src_heads = G * E + 1;
    p.q_E = E;
    p.q_idx_stride = total_k(c);
  }
  p.row_scale = nullptr;
  p.lse = at<float>(ws, l.pub.lse);
  p.redo = at<int>(ws, l.redo);
  p.q = at<T>(ws, l.pub.q);
  p.k = at<T>(ws, l.pub.k);
  p.vt = at<T>(ws, l.pub.vt);
  p.o = at<T>(ws, l.pub.s);
  p.vt_tiles = l.pub.vt_tiles;
  p.B = c->batch;
  p.G = G;
  p.L = c->seq_len;
  if (dense) {
    p.H = G * E;
    p.q_heads = G * E;
    p.n_grouped = G * E;
    for (int g = 0; g <= G; ++g) p.koff[g] = g * E;
    p.extra_group = 0;
    p.ld_o = static_cast<int64_t>(G) * E * D;
  } else {
    const GroupK gk = make_group_k(c);
    p.H = gk.K + (full_output(c) ? 1 : 0);
    p.q_heads = gk.K + 1;  // q always has room for the shared head
    p.n_grouped = gk.K;
    for (int g = 0; g <= G; ++g) p.koff[g] = gk.koff[g];
    p.extra_group = c->shared_kv_group;
    p.ld_o = static_cast<int64_t>(slot_count(c)) * D;
    if (c->output_mode == GQE_OUTPUT_WEIGHTED_CONCAT) p.row_scale = at<float>(ws, l.pub.w);
  }
  p.scale_log2 = scale_log2(c);
  return hip_status(launch_attention<T>(p, D, stream, lists));
}

template <typename T>
int output_impl(const gqe_config* c, const void* wo, void* out, void* ws, bool dense,
                hipStream_t stream);

// Short bf16 layers in three launches: (1) the router's blocks beside one
// dense projection of every expert's query head, the shared head, K and V^T
// (nothing there waits for the routing); (2) the dispatch lists' blocks
// beside the attention, whose slot-heads read their query rows through the
// routing indices; (3) the output stage (W_O, with the weighted slot formed
// in its main loop where d_h is 64).  Every routed query is projected, G*E
// heads instead of the k*G selected (about half again the projection's
// work), which these lengths absorb: their kernels are bound by latency, and
// the router and the dispatch leave the critical path.  The workspace ends up
// as after the staged calls: the same idx, w, lists, q, K, V^T, s and lse.
int forward_short(const gqe_config* c, const void* x, const void* wq, const void* wk,
                  const void* wv, const void* wr, const void* wo, void* out, void* ws,
                  hipStream_t stream) {
  typedef bf16_t T;
  const Layout l = make_layout(c, false);
  const int B = c->batch, L = c->seq_len, G = c->n_groups, E = c->n_experts, D = c->head_dim;
  const GroupK gk = make_group_k(c);
  const bool shared = full_output(c);
  RouterArgs r;
  r.wr = static_cast<const T*>(wr);
  r.bias = c->router_bias;
  r.idx = at<int32_t>(ws, l.pub.idx);
  r.w = at<float>(ws, l.pub.w);
  r.G = G;
  r.E = E;
  r.gk = gk;
  r.renorm = c->output_mode != GQE_OUTPUT_WEIGHTED_CONCAT ? 1 : 0;  // else w = p
  ProjSeg seg[3];
  const int nq = (G * E + (shared ? 1 : 0)) * D;
  seg[0].w = wq;
  seg[0].out = at<T>(ws, l.qall);
  seg[0].n_begin = 0;
  seg[0].n = nq;
  seg[0].heads = G * E + 1;
  seg[0].head_base = 0;
  seg[0].transposed = 0;
  seg[0].rope = 1;
  seg[1].w = wk;
  seg[1].out = at<T>(ws, l.pub.k);
  seg[1].n_begin = nq;
  seg[1].n = G * D;
  seg[1].heads = G;
  seg[1].head_base = 0;
  seg[1].transposed = 0;
  seg[1].rope = 1;
  seg[2].w = wv;
  seg[2].out = at<T>(ws, l.pub.vt);
  seg[2].n_begin = nq + G * D;
  seg[2].n = G * D;
  seg[2].heads = G;
  seg[2].head_base = 0;
  seg[2].transposed = 1;
  seg[2].rope = 0;
  hipError_t e = launch_front(r, static_cast<const T*>(x), B * L, c->d_model, L, D,
                              l.pub.vt_tiles, seg, 3, make_rope(c), stream);
  if (e != hipSuccess) return GQE_ERR_HIP;
  DispatchArgs da;
  da.idx = at<int32_t>(ws, l.pub.idx);
  da.counts = at<int32_t>(ws, l.pub.counts);
  da.offsets = at<int32_t>(ws, l.pub.offsets);
  da.tile_off = at<int32_t>(ws, l.tile_off);
  da.pos = at<int32_t>(ws, l.pub.pos);
  da.slot = at<int32_t>(ws, l.pub.slot);
  da.L = L;
  da.G = G;
  da.E = E;
  da.gk = gk;
  da.tile_rows = kGatherRows;
  da.n_lists = B * G * E;
  da.blocks = B * G;
  da.dbg = debug_word_of(stream);
  const int st = attention_impl<T>(c, ws, false, stream, true, &da);
  if (st != GQE_OK) return st;
  return debug_collect(stream, output_impl<T>(c, wo, out, ws, false, stream));
}

template <typename T>
int output_impl(const gqe_config* c, const void* wo, void* out, void* ws, bool dense,
                hipStream_t stream) {
  const Layout l = make_layout(c, dense);
  const int G = c->n_groups, E = c->n_experts, D = c->head_dim;
  const int M = c->batch * c->seq_len;
  hipError_t e = hipSuccess;
  int K;
  if (!dense) {
    K = slot_count(c) * D;
    if (full_output(c) && sizeof(T) == 2 && out_wslot_ok(K, D, total_k(c)))  // one launch
      return hip_status(launch_out_proj_wslot(
          at<bf16_t>(ws, l.pub.s), at<float>(ws, l.pub.w), static_cast<const bf16_t*>(wo),
          static_cast<bf16_t*>(out), M, c->d_model, K, D, total_k(c), stream));
    if (full_output(c)) {
      e = launch_weighted_slot<T>(at<T>(ws, l.pub.s), at<float>(ws, l.pub.w), M, total_k(c), D,
                                  stream);
      if (e != hipSuccess) return GQE_ERR_HIP;
    }
  } else {
    K = G * E * D;
  }
  e = launch_out_proj<T>(at<T>(ws, l.pub.s), static_cast<const T*>(wo), static_cast<T*>(out), M,
                         c->d_model, K, stream);
  return hip_status(e);
}

}  // namespace

// the workspace of gqe_forward_noalloc (see below)
static __device__ __align__(256) unsigned char scratch[GQE_NOALLOC_SCRATCH_BYTES];

namespace {

// ---- the workspace of gqe_forward_noalloc ------------------------------------
// One array per device, part of the library's code object: it exists from the
// moment the runtime loads that object on a device until the process ends.
// Its device address is resolved once per device (symbol_on_device).
constexpr size_t kNoAllocBytes = GQE_NOALLOC_SCRATCH_BYTES;

std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices];  // device address of `scratch` per device, once resolved

int noalloc_scratch(hipStream_t stream, void** addr) {
  return symbol_on_device(HIP_SYMBOL(scratch), g_scratch_addr, g_scratch_mutex, stream, addr);
}

// ---- decode ------------------------------------------------------------------

// Decode takes batch = B sequences of one new token each and seq_len = the
// cache capacity Lc.  The dynamic LDS of its row products holds d_model floats.
constexpr int kDecodeMaxDModel = 16384;

// query heads projected per token: every routed expert, plus the shared head
// for the full output
int decode_q_heads(const gqe_config* c, bool dense) {
  return c->n_groups * c->n_experts + (!dense && full_output(c) ? 1 : 0);
}
int decode_heads(const gqe_config* c, bool dense) {
  return dense ? c->n_groups * c->n_experts : total_k(c) + (full_output(c) ? 1 : 0);
}
int decode_ld_s(const gqe_config* c, bool dense) {
  return (dense ? c->n_groups * c->n_experts : slot_count(c)) * c->head_dim;
}

struct DecodeLayout {
  size_t idx, w, q, part, s, total;
  int chunk, n_chunks;
};

DecodeLayout make_decode_layout(const gqe_config* c, bool dense) {
  const size_t B = c->batch, K = total_k(c), D = c->head_dim;
  const size_t H = decode_heads(c, dense);
  DecodeLayout l{};
  l.chunk = decode_chunk(c->batch, c->n_groups, c->seq_len);
  l.n_chunks = (c->seq_len + l.chunk - 1) / l.chunk;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, kAlign);
    return o;
  };
  if (!dense) {
    l.idx = take(B * K * 4);
    l.w = take(B * K * 4);
  }
  l.q = take(B * static_cast<size_t>(decode_q_heads(c, dense)) * D * 4);
  l.part = take(B * H * static_cast<size_t>(l.n_chunks) * (D + 2) * 4);
  l.s = take(B * static_cast<size_t>(decode_ld_s(c, dense)) * elem_bytes(c));
  l.total = off;
  return l;
}

int check_decode_cfg(const gqe_config* c) {
  const int st = check_cfg(c);
  if (st != GQE_OK) return st;
  if (c->batch > 0 && c->seq_len < 1) return GQE_ERR_INVALID_ARG;  // no room for the token
  if (c->d_model > kDecodeMaxDModel) return GQE_ERR_UNSUPPORTED;
  return GQE_OK;
}

template <typename T>
int decode_impl(const gqe_config* c, bool dense, const void* x, const void* wq, const void* wk,
                const void* wv, const void* wr, const void* wo, void* k_cache, void* vt_cache,
                const int32_t* pos, void* out, void* ws, hipStream_t stream) {
  const DecodeLayout l = make_decode_layout(c, dense);
  const int G = c->n_groups, E = c->n_experts;
  DecodeParams p;
  p.x = x;
  p.wq = wq;
  p.wk = wk;
  p.wv = wv;
  p.wo = wo;
  p.wr = dense ? nullptr : wr;
  p.router_bias = dense ? nullptr : c->router_bias;
  p.renorm = c->output_mode != GQE_OUTPUT_WEIGHTED_CONCAT;
  p.idx = dense ? nullptr : at<int32_t>(ws, l.idx);
  p.w = dense ? nullptr : at<float>(ws, l.w);
  p.pos = pos;
  p.q = at<float>(ws, l.q);
  p.k_cache = k_cache;
  p.vt_cache = vt_cache;
  p.part = at<float>(ws, l.part);
  p.s = at<T>(ws, l.s);
  p.row_scale = !dense && c->output_mode == GQE_OUTPUT_WEIGHTED_CONCAT ? p.w : nullptr;
  p.out = out;
  p.B = c->batch;
  p.d = c->d_model;
  p.G = G;
  p.E = E;
  p.gk = make_group_k(c);
  p.D = c->head_dim;
  p.Lc = c->seq_len;
  p.q_heads = decode_q_heads(c, dense);
  p.Hq = decode_heads(c, dense);
  p.n_routed = dense ? G * E : p.gk.K;
  p.shared_head = !dense && full_output(c) ? 1 : 0;
  p.shared_kv_group = c->shared_kv_group;
  p.max_heads = 0;
  for (int g = 0; g <= G; ++g) p.hbeg[g] = dense ? g * E : p.gk.koff[g];
  for (int g = 0; g < G; ++g)
    p.max_heads = std::max(p.max_heads, p.hbeg[g + 1] - p.hbeg[g] +
                                            (p.shared_head && g == c->shared_kv_group ? 1 : 0));
  p.chunk = l.chunk;
  p.scale = softmax_scale(c);
  p.ld_s = decode_ld_s(c, dense);
  p.K_out = p.ld_s;
  p.weighted_slot = p.shared_head;
  p.rope = make_rope(c);
  hipError_t e = launch_decode_front<T>(p, stream);
  if (e == hipSuccess) e = launch_decode_attend<T>(p, stream);
  return hip_status(e);
}

int decode_entry(const gqe_config* cfg, bool dense, const void* x, const void* Wq, const void* Wk,
                 const void* Wv, const void* Wr, const void* Wo, void* k_cache, void* vt_cache,
                 const int32_t* pos, void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_decode_cfg(cfg);
  if (st != GQE_OK || cfg->batch == 0) return st;
  if (!aligned16(x) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) || !aligned16(Wo) ||
      !aligned16(k_cache) || !aligned16(vt_cache) || !aligned16(out) || !aligned16(ws) ||
      pos == nullptr || (reinterpret_cast<uintptr_t>(pos) & 3u))
    return GQE_ERR_INVALID_ARG;
  if (!dense && (!aligned16(Wr) ||
                 (cfg->router_bias && (reinterpret_cast<uintptr_t>(cfg->router_bias) & 3u))))
    return GQE_ERR_INVALID_ARG;
  if (ws_bytes < make_decode_layout(cfg, dense).total) return GQE_ERR_WORKSPACE;
  return cfg->dtype == GQE_DTYPE_BF16
             ? decode_impl<bf16_t>(cfg, dense, x, Wq, Wk, Wv, Wr, Wo, k_cache, vt_cache, pos,
                                   out, ws, stream)
             : decode_impl<float>(cfg, dense, x, Wq, Wk, Wv, Wr, Wo, k_cache, vt_cache, pos, out,
                                  ws, stream);
}


}  // namespace

namespace {

// ---- backward ------------------------------------------------------------------

struct BwdLayout {
  size_t gall, w_t, wo_t, ds, dO, dOt, qt, qs, kt, vr, dsum, dw, dr, p_all, psum, gall_t, x_t,
      dy_t, s_t, dkv_part, gemm_part, dq_part, total;
  int tpad, ws, qcols, kcol, vcol, rcol, kcols, kpad, H, q_heads, dkv_split, dq_split;
  bool has_gemm_part;
};

BwdLayout make_bwd_layout(const gqe_config* c, bool dense) {
  const size_t B = c->batch, L = c->seq_len, G = c->n_groups, E = c->n_experts;
  const size_t K = total_k(c);
  const size_t D = c->head_dim, d = c->d_model, es = elem_bytes(c), T = B * L;
  const size_t tiles = (L + 63) / 64;
  BwdLayout l{};
  l.tpad = static_cast<int>((T + 63) / 64 * 64);
  l.H = attn_heads(c, dense);
  l.q_heads = dense ? static_cast<int>(G * E) : static_cast<int>(K + 1);
  l.ws = static_cast<int>((dense ? G * E : static_cast<size_t>(slot_count(c))) * D);
  l.qcols = static_cast<int>((G * E + (dense ? 0 : 1)) * D);
  l.kcol = l.qcols;
  l.vcol = l.kcol + static_cast<int>(G * D);
  l.rcol = l.vcol + static_cast<int>(G * D);
  l.kcols = l.rcol + (dense ? 0 : static_cast<int>(G * E));
  l.kpad = (l.kcols + 63) / 64 * 64;
  const size_t H = l.H, tp = l.tpad, kp = l.kpad, ws = l.ws;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, kAlign);
    return o;
  };
  l.gall = take(T * kp * es);
  l.w_t = take(d * kp * es);
  l.wo_t = take(ws * d * es);
  l.ds = take(T * ws * 4);
  l.dO = take(B * H * L * D * es);
  l.dOt = take(B * H * tiles * D * 64 * es);
  l.qt = take(B * H * tiles * D * 64 * es);
  l.qs = take(B * H * L * D * es);
  l.kt = take(B * G * tiles * D * 64 * es);
  l.vr = take(B * G * L * D * es);
  l.dsum = take(B * H * L * 4);
  l.dw = take(dense ? 0 : T * K * 4);
  l.dr = take(dense ? 0 : T * G * E * 4);
  l.p_all = take(dense ? 0 : T * G * E * 4);
  l.psum = take(dense ? 0 : G * E * 8);
  l.gall_t = take(kp * tp * es);
  l.x_t = take(d * tp * es);
  l.dy_t = take(d * tp * es);
  l.s_t = take(ws * tp * es);
  // float partials of the split dK/dV walk (bf16 short launches only)
  l.dkv_split = c->dtype == GQE_DTYPE_BF16
                    ? dkdv_splits(c->batch, c->n_groups, c->seq_len, c->head_dim)
                    : 1;
  l.dkv_part = take(l.dkv_split > 1 ? static_cast<size_t>(l.dkv_split) * B * G * L * 2 * D * 4 : 0);
  // float partials of the split-K weight-gradient products (dW_O = dy^T s and
  // [dW_q; dW_k; dW_v; dW_r] = Gall^T x), when their tiles alone leave
  // compute units idle
  {
    const int dd = static_cast<int>(d), tpi = l.tpad;
    const int s_o = nt_gemm_splits(dd, l.ws, tpi), s_w = nt_gemm_splits(l.kcols, dd, tpi);
    const size_t part = std::max(s_o > 1 ? static_cast<size_t>(s_o) * d * ws : 0,
                                 s_w > 1 ? static_cast<size_t>(s_w) * l.kcols * d : 0);
    l.gemm_part = part > 0 ? take(part * 4) : 0;
    l.has_gemm_part = part > 0;
  }
  // float partials of the split dQ walk (bf16 short launches only)
  l.dq_split = c->dtype == GQE_DTYPE_BF16 ? dq_splits(c->batch, l.H, c->seq_len) : 1;
  l.dq_part = take(l.dq_split > 1 ? static_cast<size_t>(l.dq_split) * B * H * L * D * 4 : 0);
  l.total = off;
  return l;
}

template <typename T>
int backward_impl(const gqe_config* c, bool dense, const void* x, const void* wq, const void* wk,
                  const void* wv, const void* wr, const void* wo, const void* dy, float aux_weight,
                  const void* fws, float* dx, float* dwq, float* dwk, float* dwv, float* dwr,
                  float* dbr, float* dwo, float* aux_loss, void* ws, hipStream_t stream) {
  const Layout fl = make_layout(c, dense);
  const BwdLayout l = make_bwd_layout(c, dense);
  void* f = const_cast<void*>(fws);
  const int G = c->n_groups, E = c->n_experts;
  BwdParams p;
  p.x = x;
  p.wq = wq;
  p.wk = wk;
  p.wv = wv;
  p.wr = dense ? nullptr : wr;
  p.router_bias = dense ? nullptr : c->router_bias;
  p.wo = wo;
  p.dy = dy;
  p.idx = dense ? nullptr : at<int32_t>(f, fl.pub.idx);
  p.w = dense ? nullptr : at<float>(f, fl.pub.w);
  p.counts = dense ? nullptr : at<int32_t>(f, fl.pub.counts);
  p.q = at<T>(f, fl.pub.q);
  p.keys = at<T>(f, fl.pub.k);
  p.vt = at<T>(f, fl.pub.vt);
  p.vt_tiles = fl.pub.vt_tiles;
  p.s = at<T>(f, fl.pub.s);
  p.lse = at<float>(f, fl.pub.lse);
  p.dx = dx;
  p.dwq = dwq;
  p.dwk = dwk;
  p.dwv = dwv;
  p.dwr = dwr;
  p.dbr = dbr;
  p.dwo = dwo;
  p.aux_loss = aux_loss;
  p.gall = at<T>(ws, l.gall);
  p.w_t = at<T>(ws, l.w_t);
  p.wo_t = at<T>(ws, l.wo_t);
  p.dO = at<T>(ws, l.dO);
  p.dOt = at<T>(ws, l.dOt);
  p.qt = at<T>(ws, l.qt);
  p.qs = at<T>(ws, l.qs);
  p.kt = at<T>(ws, l.kt);
  p.vr = at<T>(ws, l.vr);
  p.gall_t = at<T>(ws, l.gall_t);
  p.x_t = at<T>(ws, l.x_t);
  p.dy_t = at<T>(ws, l.dy_t);
  p.s_t = at<T>(ws, l.s_t);
  p.ds = at<float>(ws, l.ds);
  p.dsum = at<float>(ws, l.dsum);
  p.dw = dense ? nullptr : at<float>(ws, l.dw);
  p.dr = dense ? nullptr : at<float>(ws, l.dr);
  p.p_all = dense ? nullptr : at<float>(ws, l.p_all);
  p.psum = dense ? nullptr : at<double>(ws, l.psum);
  p.B = c->batch;
  p.L = c->seq_len;
  p.d = c->d_model;
  p.G = G;
  p.E = E;
  p.gk = make_group_k(c);
  p.D = c->head_dim;
  p.H = l.H;
  p.q_heads = l.q_heads;
  p.n_routed = dense ? 0 : p.gk.K;
  for (int g = 0; g <= G; ++g) p.hbeg[g] = dense ? g * E : p.gk.koff[g];
  p.n_grouped = p.hbeg[G];
  p.extra_group = c->shared_kv_group;
  p.mode = dense ? 3 : c->output_mode == GQE_OUTPUT_FULL ? 0 : c->output_mode == GQE_OUTPUT_HARD ? 1 : 2;
  p.ws = l.ws;
  p.qcols = l.qcols;
  p.kcol = l.kcol;
  p.vcol = l.vcol;
  p.rcol = l.rcol;
  p.kcols = l.kcols;
  p.kpad = l.kpad;
  p.tpad = l.tpad;
  p.dkv_split = l.dkv_split;
  p.dkv_part = at<float>(ws, l.dkv_part);
  p.gemm_part = l.has_gemm_part ? at<float>(ws, l.gemm_part) : nullptr;
  p.dq_split = l.dq_split;
  p.dq_part = at<float>(ws, l.dq_part);
  p.scale = softmax_scale(c);
  p.aux_weight = dense ? 0.f : aux_weight;
  p.rope = make_rope(c);
  p.dbg = dense ? nullptr : debug_word_of(stream);
  return debug_collect(stream, hip_status(launch_backward<T>(p, stream)));
}

int backward_entry(const gqe_config* cfg, bool dense, const void* x, const void* Wq,
                   const void* Wk, const void* Wv, const void* Wr, const void* Wo, const void* dy,
                   float aux_weight, const void* fws, size_t fws_bytes, float* dx, float* dWq,
                   float* dWk, float* dWv, float* dWr, float* dbr, float* dWo, float* aux_loss,
                   void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_cfg(cfg);
  if (st != GQE_OK || empty(cfg)) return st;
  if (!(aux_weight >= 0.f) || isinf(aux_weight)) return GQE_ERR_INVALID_ARG;
  const void* need[] = {x, Wq, Wk, Wv, Wo, dy, fws, dx, dWq, dWk, dWv, dWo, ws};
  for (const void* q : need)
    if (!aligned16(q)) return GQE_ERR_INVALID_ARG;
  if (!dense && (!aligned16(Wr) || !aligned16(dWr) || dbr == nullptr || aux_loss == nullptr ||
                 (reinterpret_cast<uintptr_t>(dbr) & 3u) || (reinterpret_cast<uintptr_t>(aux_loss) & 3u) ||
                 (cfg->router_bias && (reinterpret_cast<uintptr_t>(cfg->router_bias) & 3u))))
    return GQE_ERR_INVALID_ARG;
  if (fws_bytes < make_layout(cfg, dense).pub.total) return GQE_ERR_WORKSPACE;
  if (ws_bytes < make_bwd_layout(cfg, dense).total) return GQE_ERR_WORKSPACE;
  return cfg->dtype == GQE_DTYPE_BF16
             ? backward_impl<bf16_t>(cfg, dense, x, Wq, Wk, Wv, Wr, Wo, dy, aux_weight, fws, dx,
                                     dWq, dWk, dWv, dWr, dbr, dWo, aux_loss, ws, stream)
             : backward_impl<float>(cfg, dense, x, Wq, Wk, Wv, Wr, Wo, dy, aux_weight, fws, dx,
                                    dWq, dWk, dWv, dWr, dbr, dWo, aux_loss, ws, stream);
}

}  // namespace

extern "C" {

const char* gqe_status_string(int status) {
  switch (status) {
    case GQE_OK: return "GQE_OK";
    case GQE_ERR_INVALID_ARG: return "GQE_ERR_INVALID_ARG: invalid argument";
    case GQE_ERR_UNSUPPORTED: return "GQE_ERR_UNSUPPORTED: configuration not built";
    case GQE_ERR_WORKSPACE: return "GQE_ERR_WORKSPACE: workspace too small";
    case GQE_ERR_HIP: return "GQE_ERR_HIP: the HIP runtime rejected a launch";
    case GQE_ERR_DEBUG: return "GQE_ERR_DEBUG: an index check of the debug build failed";
    default: return "unknown gqe status";
  }
}

size_t gqe_workspace_bytes(const gqe_config* cfg) {
  if (check_cfg(cfg) != GQE_OK) return 0;
  return make_layout(cfg, false).pub.total;
}

int gqe_workspace_layout(const gqe_config* cfg, gqe_ws_layout* layout) {
  const int st = check_cfg(cfg);
  if (st != GQE_OK) return st;
  if (layout == nullptr) return GQE_ERR_INVALID_ARG;
  *layout = make_layout(cfg, false).pub;
  return GQE_OK;
}

size_t gqa_workspace_bytes(const gqe_config* cfg) {
  if (check_cfg(cfg) != GQE_OK) return 0;
  return make_layout(cfg, true).pub.total;
}

int gqa_workspace_layout(const gqe_config* cfg, gqe_ws_layout* layout) {
  const int st = check_cfg(cfg);
  if (st != GQE_OK) return st;
  if (layout == nullptr) return GQE_ERR_INVALID_ARG;
  *layout = make_layout(cfg, true).pub;
  return GQE_OK;
}

int gqe_route(const gqe_config* cfg, const void* x, const void* Wr, void* workspace,
              size_t ws_bytes, hipStream_t stream) {
  int st = check_common(cfg, workspace, ws_bytes, false);
  if (st != GQE_OK || empty(cfg)) return st;
  if (!aligned16(x) || !aligned16(Wr)) return GQE_ERR_INVALID_ARG;
  if (cfg->router_bias && (reinterpret_cast<uintptr_t>(cfg->router_bias) & 3u))
    return GQE_ERR_INVALID_ARG;
  const Layout l = make_layout(cfg, false);
  const bool renorm = cfg->output_mode != GQE_OUTPUT_WEIGHTED_CONCAT;  // else w = p
  hipError_t e;
  if (cfg->dtype == GQE_DTYPE_BF16)
    e = launch_router<bf16_t>(static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(Wr),
                              cfg->router_bias, at<int32_t>(workspace, l.pub.idx),
                              at<float>(workspace, l.pub.w), cfg->batch * cfg->seq_len,
                              cfg->d_model, cfg->n_groups, cfg->n_experts, make_group_k(cfg), renorm,
                              stream);
  else
    e = launch_router<float>(static_cast<const float*>(x), static_cast<const float*>(Wr),
                             cfg->router_bias, at<int32_t>(workspace, l.pub.idx),
                             at<float>(workspace, l.pub.w), cfg->batch * cfg->seq_len,
                             cfg->d_model, cfg->n_groups, cfg->n_experts, make_group_k(cfg), renorm,
                             stream);
  return hip_status(e);
}

int gqe_dispatch(const gqe_config* cfg, void* workspace, size_t ws_bytes, hipStream_t stream) {
  int st = check_common(cfg, workspace, ws_bytes, false);
  if (st != GQE_OK || empty(cfg)) return st;
  const Layout l = make_layout(cfg, false);
  return debug_collect(stream, hip_status(launch_dispatch(
      at<int32_t>(workspace, l.pub.idx), at<int32_t>(workspace, l.chunk_counts),
      at<int32_t>(workspace, l.pub.counts), at<int32_t>(workspace, l.pub.offsets),
      at<int32_t>(workspace, l.tile_off), at<int32_t>(workspace, l.pub.pos),
      at<int32_t>(workspace, l.pub.slot), cfg->batch, cfg->seq_len, cfg->n_groups,
      cfg->n_experts, make_group_k(cfg), kGatherRows, debug_word_of(stream), stream)));
}

int gqe_project(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                const void* Wv, void* workspace, size_t ws_bytes, hipStream_t stream) {
  int st = check_common(cfg, workspace, ws_bytes, false);
  if (st != GQE_OK || empty(cfg)) return st;
  if (!aligned16(x) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv))
    return GQE_ERR_INVALID_ARG;
  return debug_collect(stream, cfg->dtype == GQE_DTYPE_BF16
                                  ? project_impl<bf16_t>(cfg, x, Wq, Wk, Wv, workspace, false, stream)
                                  : project_impl<float>(cfg, x, Wq, Wk, Wv, workspace, false, stream));
}

int gqe_attention(const gqe_config* cfg, void* workspace, size_t ws_bytes, hipStream_t stream) {
  int st = check_common(cfg, workspace, ws_bytes, false);
  if (st != GQE_OK || empty(cfg)) return st;
  return cfg->dtype == GQE_DTYPE_BF16 ? attention_impl<bf16_t>(cfg, workspace, false, stream)
                                      : attention_impl<float>(cfg, workspace, false, stream);
}

int gqe_output(const gqe_config* cfg, const void* Wo, void* out, void* workspace,
               size_t ws_bytes, hipStream_t stream) {
  int st = check_common(cfg, workspace, ws_bytes, false);
  if (st != GQE_OK || empty(cfg)) return st;
  if (!aligned16(Wo) || !aligned16(out)) return GQE_ERR_INVALID_ARG;
  return cfg->dtype == GQE_DTYPE_BF16
             ? output_impl<bf16_t>(cfg, Wo, out, workspace, false, stream)
             : output_impl<float>(cfg, Wo, out, workspace, false, stream);
}

int gqe_forward(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                const void* Wv, const void* Wr, const void* Wo, void* out, void* workspace,
                size_t ws_bytes, hipStream_t stream) {
  int st = check_common(cfg, workspace, ws_bytes, false);
  if (st != GQE_OK || empty(cfg)) return st;
  if (!aligned16(x) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv) || !aligned16(Wr) ||
      !aligned16(Wo) || !aligned16(out))
    return GQE_ERR_INVALID_ARG;
  if (cfg->router_bias && (reinterpret_cast<uintptr_t>(cfg->router_bias) & 3u))
    return GQE_ERR_INVALID_ARG;
  if (short_forward(cfg))
    return forward_short(cfg, x, Wq, Wk, Wv, Wr, Wo, out, workspace, stream);
  if ((st = gqe_route(cfg, x, Wr, workspace, ws_bytes, stream)) != GQE_OK) return st;
  if ((st = gqe_dispatch(cfg, workspace, ws_bytes, stream)) != GQE_OK) return st;
  if ((st = gqe_project(cfg, x, Wq, Wk, Wv, workspace, ws_bytes, stream)) != GQE_OK) return st;
  if ((st = gqe_attention(cfg, workspace, ws_bytes, stream)) != GQE_OK) return st;
  return gqe_output(cfg, Wo, out, workspace, ws_bytes, stream);
}

int gqe_forward_is_short(const gqe_config* cfg) {
  const int st = check_cfg(cfg);
  if (st != GQE_OK) return st;
  return short_forward(cfg) ? 1 : 0;
}

int gqe_forward_noalloc(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                        const void* Wv, const void* Wr, const void* Wo, void* out,
                        hipStream_t stream) {
  int st = check_cfg(cfg);
  if (st != GQE_OK || empty(cfg)) return st;
  if (make_layout(cfg, false).pub.total > kNoAllocBytes) return GQE_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = noalloc_scratch(stream, &ws)) != GQE_OK) return st;
  return gqe_forward(cfg, x, Wq, Wk, Wv, Wr, Wo, out, ws, kNoAllocBytes, stream);
}

int gqa_project(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                const void* Wv, void* workspace, size_t ws_bytes, hipStream_t stream) {
  int st = check_common(cfg, workspace, ws_bytes, true);
  if (st != GQE_OK || empty(cfg)) return st;
  if (!aligned16(x) || !aligned16(Wq) || !aligned16(Wk) || !aligned16(Wv))
    return GQE_ERR_INVALID_ARG;
  return cfg->dtype == GQE_DTYPE_BF16
             ? project_impl<bf16_t>(cfg, x, Wq, Wk, Wv, workspace, true, stream)
             : project_impl<float>(cfg, x, Wq, Wk, Wv, workspace, true, stream);
}

int gqa_attention(const gqe_config* cfg, void* workspace, size_t ws_bytes, hipStream_t stream) {
  int st = check_common(cfg, workspace, ws_bytes, true);
  if (st != GQE_OK || empty(cfg)) return st;
  return cfg->dtype == GQE_DTYPE_BF16 ? attention_impl<bf16_t>(cfg, workspace, true, stream)
                                      : attention_impl<float>(cfg, workspace, true, stream);
}

int gqa_output(const gqe_config* cfg, const void* Wo, void* out, void* workspace,
               size_t ws_bytes, hipStream_t stream) {
  int st = check_common(cfg, workspace, ws_bytes, true);
  if (st != GQE_OK || empty(cfg)) return st;
  if (!aligned16(Wo) || !aligned16(out)) return GQE_ERR_INVALID_ARG;
  return cfg->dtype == GQE_DTYPE_BF16
             ? output_impl<bf16_t>(cfg, Wo, out, workspace, true, stream)
             : output_impl<float>(cfg, Wo, out, workspace, true, stream);
}

int gqa_forward(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                const void* Wv, const void* Wo, void* out, void* workspace, size_t ws_bytes,
                hipStream_t stream) {
  int st = check_common(cfg, workspace, ws_bytes, true);
  if (st != GQE_OK || empty(cfg)) return st;
  if ((st = gqa_project(cfg, x, Wq, Wk, Wv, workspace, ws_bytes, stream)) != GQE_OK) return st;
  if ((st = gqa_attention(cfg, workspace, ws_bytes, stream)) != GQE_OK) return st;
  return gqa_output(cfg, Wo, out, workspace, ws_bytes, stream);
}

size_t gqe_decode_workspace_bytes(const gqe_config* cfg) {
  if (check_decode_cfg(cfg) != GQE_OK) return 0;
  return make_decode_layout(cfg, false).total;
}

size_t gqa_decode_workspace_bytes(const gqe_config* cfg) {
  if (check_decode_cfg(cfg) != GQE_OK) return 0;
  return make_decode_layout(cfg, true).total;
}

int gqe_decode(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
               const void* Wv, const void* Wr, const void* Wo, void* k_cache, void* vt_cache,
               const int32_t* pos, void* out, void* workspace, size_t ws_bytes,
               hipStream_t stream) {
  return decode_entry(cfg, false, x, Wq, Wk, Wv, Wr, Wo, k_cache, vt_cache, pos, out, workspace,
                      ws_bytes, stream);
}

int gqa_decode(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
               const void* Wv, const void* Wo, void* k_cache, void* vt_cache, const int32_t* pos,
               void* out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return decode_entry(cfg, true, x, Wq, Wk, Wv, nullptr, Wo, k_cache, vt_cache, pos, out,
                      workspace, ws_bytes, stream);
}

size_t gqe_backward_workspace_bytes(const gqe_config* cfg) {
  if (check_cfg(cfg) != GQE_OK) return 0;
  return make_bwd_layout(cfg, false).total;
}

size_t gqa_backward_workspace_bytes(const gqe_config* cfg) {
  if (check_cfg(cfg) != GQE_OK) return 0;
  return make_bwd_layout(cfg, true).total;
}

int gqe_backward(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                 const void* Wv, const void* Wr, const void* Wo, const void* dy, float aux_weight,
                 const void* fwd_workspace, size_t fwd_ws_bytes, float* dx, float* dWq, float* dWk,
                 float* dWv, float* dWr, float* dbr, float* dWo, float* aux_loss, void* workspace,
                 size_t ws_bytes, hipStream_t stream) {
  return backward_entry(cfg, false, x, Wq, Wk, Wv, Wr, Wo, dy, aux_weight, fwd_workspace,
                        fwd_ws_bytes, dx, dWq, dWk, dWv, dWr, dbr, dWo, aux_loss, workspace,
                        ws_bytes, stream);
}

int gqa_backward(const gqe_config* cfg, const void* x, const void* Wq, const void* Wk,
                 const void* Wv, const void* Wo, const void* dy, const void* fwd_workspace,
                 size_t fwd_ws_bytes, float* dx, float* dWq, float* dWk, float* dWv, float* dWo,
                 void* workspace, size_t ws_bytes, hipStream_t stream) {
  return backward_entry(cfg, true, x, Wq, Wk, Wv, nullptr, Wo, dy, 0.f, fwd_workspace,
                        fwd_ws_bytes, dx, dWq, dWk, dWv, nullptr, nullptr, dWo, nullptr, workspace,
                        ws_bytes, stream);
}

}  // extern "C"

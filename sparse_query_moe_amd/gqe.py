"""ctypes binding of libgqe.so (include/gqe.h), one Python function per C entry point.

Argument marshalling only: every computation runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU (PyTorch provides device memory
and streams); they are passed as raw device pointers.  The functions raise
GqeError when the library returns an error status, and the import fails
loudly when libgqe.so has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgqe.so")

DTYPE_BF16 = 0
DTYPE_FP32 = 1
_TORCH_DTYPE = {DTYPE_BF16: torch.bfloat16, DTYPE_FP32: torch.float32}

# every entry point include/gqe.h declares
EXPORTS = (
    "gqe_workspace_bytes", "gqe_workspace_layout", "gqe_route", "gqe_dispatch", "gqe_project",
    "gqe_attention", "gqe_output", "gqe_forward", "gqe_forward_is_short", "gqe_forward_noalloc",
    "gqa_workspace_bytes",
    "gqa_workspace_layout",
    "gqa_project", "gqa_attention", "gqa_output", "gqa_forward", "gqe_decode_workspace_bytes",
    "gqe_decode", "gqa_decode_workspace_bytes", "gqa_decode", "gqe_backward_workspace_bytes",
    "gqe_backward", "gqa_backward_workspace_bytes", "gqa_backward", "gqe_peak_blocks",
    "gqe_peak_mfma_bf16", "gqe_peak_copy", "gqe_status_string",
)


class GqeError(RuntimeError):
    pass


class GqeConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("d_model", ctypes.c_int32),
        ("n_groups", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("shared_kv_group", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("router_bias", ctypes.c_void_p), ("output_mode", ctypes.c_int32),
        ("group_top_k", ctypes.c_void_p), ("rope_base", ctypes.c_float),
    ]

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("idx", "w", "counts", "offsets", "pos", "slot", "q", "k", "vt", "s", "lse",
                 "scratch", "total")] + [("vt_tiles", ctypes.c_int64)]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sparse_query_moe_amd.build`")
    lib = ctypes.CDLL(path)
    vp, cfgp, sz = ctypes.c_void_p, ctypes.POINTER(GqeConfig), ctypes.c_size_t
    sig = {
        "gqe_workspace_bytes": (sz, [cfgp]),
        "gqa_workspace_bytes": (sz, [cfgp]),
        "gqe_workspace_layout": (ctypes.c_int, [cfgp, ctypes.POINTER(WsLayout)]),
        "gqa_workspace_layout": (ctypes.c_int, [cfgp, ctypes.POINTER(WsLayout)]),
        "gqe_route": (ctypes.c_int, [cfgp, vp, vp, vp, sz, vp]),
        "gqe_dispatch": (ctypes.c_int, [cfgp, vp, sz, vp]),
        "gqe_project": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, sz, vp]),
        "gqe_attention": (ctypes.c_int, [cfgp, vp, sz, vp]),
        "gqe_output": (ctypes.c_int, [cfgp, vp, vp, vp, sz, vp]),
        "gqe_forward": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "gqe_forward_noalloc": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "gqe_forward_is_short": (ctypes.c_int, [cfgp]),
        "gqa_project": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, sz, vp]),
        "gqa_attention": (ctypes.c_int, [cfgp, vp, sz, vp]),
        "gqa_output": (ctypes.c_int, [cfgp, vp, vp, vp, sz, vp]),
        "gqa_forward": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "gqe_decode_workspace_bytes": (sz, [cfgp]),
        "gqa_decode_workspace_bytes": (sz, [cfgp]),
        "gqe_decode": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "gqa_decode": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "gqe_backward_workspace_bytes": (sz, [cfgp]),
        "gqa_backward_workspace_bytes": (sz, [cfgp]),
        "gqe_backward": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, sz,
                                        vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "gqa_backward": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp,
                                        vp, sz, vp]),
        "gqe_peak_blocks": (ctypes.c_int, []),
        "gqe_peak_mfma_bf16": (ctypes.c_int, [vp, ctypes.c_int, ctypes.c_int, vp]),
        "gqe_peak_copy": (ctypes.c_int, [vp, vp, sz, vp]),
        "gqe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = load_library()


def status_string(status: int) -> str:
    return _lib.gqe_status_string(status).decode()


def _check(status: int, what: str):
    if status != 0:
        raise GqeError(f"{what}: {status_string(status)} ({status})")


OUTPUT_MODES = {"full": 0, "hard": 1, "weighted_concat": 2}  # gqe_output_mode


def make_config(batch, seq_len, d_model, n_groups, n_experts, top_k, head_dim, dtype="bf16",
                shared_kv_group=0, softmax_scale=0.0, router_bias=None,
                output_mode="full", group_top_k=None, rope_base=0.0) -> GqeConfig:
    """Fill a gqe_config.  `router_bias` is a float32 device tensor [G*E] or None;
    the caller keeps it alive while the config is in use.  `output_mode` is
    "full", "hard" or "weighted_concat" (see gqe_output_mode).  `group_top_k`
    is a list of G per-group expert counts or None (top_k in every group).
    `rope_base` > 0 turns queries and keys by position (see gqe_config)."""
    dt = {"bf16": DTYPE_BF16, "fp32": DTYPE_FP32}.get(dtype, dtype)
    gk = None
    if group_top_k is not None:
        gk = (ctypes.c_int32 * len(group_top_k))(*[int(v) for v in group_top_k])
    cfg = GqeConfig(batch, seq_len, d_model, n_groups, n_experts, top_k, head_dim,
                    shared_kv_group, dt, float(softmax_scale),
                    None if router_bias is None else router_bias.data_ptr(),
                    OUTPUT_MODES.get(output_mode, output_mode),
                    None if gk is None else ctypes.cast(gk, ctypes.c_void_p), float(rope_base))
    cfg._group_top_k = gk  # kept alive with the config
    return cfg


def total_k(cfg: GqeConfig) -> int:
    """Hard slots per token: the sum of the per-group expert counts."""
    if cfg.group_top_k:
        arr = ctypes.cast(cfg.group_top_k, ctypes.POINTER(ctypes.c_int32))
        return sum(arr[g] for g in range(cfg.n_groups))
    return cfg.top_k * cfg.n_groups


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def gqe_workspace_bytes(cfg: GqeConfig) -> int:
    return int(_lib.gqe_workspace_bytes(ctypes.byref(cfg)))


def gqa_workspace_bytes(cfg: GqeConfig) -> int:
    return int(_lib.gqa_workspace_bytes(ctypes.byref(cfg)))


def gqe_workspace_layout(cfg: GqeConfig) -> WsLayout:
    lay = WsLayout()
    _check(_lib.gqe_workspace_layout(ctypes.byref(cfg), ctypes.byref(lay)), "gqe_workspace_layout")
    return lay


def gqa_workspace_layout(cfg: GqeConfig) -> WsLayout:
    lay = WsLayout()
    _check(_lib.gqa_workspace_layout(ctypes.byref(cfg), ctypes.byref(lay)), "gqa_workspace_layout")
    return lay


def alloc_workspace(cfg: GqeConfig, dense: bool = False, device="cuda") -> torch.Tensor:
    n = gqa_workspace_bytes(cfg) if dense else gqe_workspace_bytes(cfg)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def gqe_route(cfg, x, wr, ws, stream=None):
    _check(_lib.gqe_route(ctypes.byref(cfg), _ptr(x), _ptr(wr), _ptr(ws), ws.numel(),
                          _stream(stream)), "gqe_route")


def gqe_dispatch(cfg, ws, stream=None):
    _check(_lib.gqe_dispatch(ctypes.byref(cfg), _ptr(ws), ws.numel(), _stream(stream)),
           "gqe_dispatch")


def gqe_project(cfg, x, wq, wk, wv, ws, stream=None):
    _check(_lib.gqe_project(ctypes.byref(cfg), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(ws),
                            ws.numel(), _stream(stream)), "gqe_project")


def gqe_attention(cfg, ws, stream=None):
    _check(_lib.gqe_attention(ctypes.byref(cfg), _ptr(ws), ws.numel(), _stream(stream)),
           "gqe_attention")


def gqe_output(cfg, wo, out, ws, stream=None):
    _check(_lib.gqe_output(ctypes.byref(cfg), _ptr(wo), _ptr(out), _ptr(ws), ws.numel(),
                           _stream(stream)), "gqe_output")


def gqe_forward(cfg, x, wq, wk, wv, wr, wo, out, ws, stream=None):
    _check(_lib.gqe_forward(ctypes.byref(cfg), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wr),
                            _ptr(wo), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)),
           "gqe_forward")


def uses_short_forward(cfg) -> bool:
    """Whether gqe_forward takes the short-layer launches for cfg."""
    r = _lib.gqe_forward_is_short(ctypes.byref(cfg))
    _check(min(r, 0), "gqe_forward_is_short")
    return r == 1


# size of the library-owned workspace of gqe_forward_noalloc (include/gqe.h)
NOALLOC_SCRATCH_BYTES = 32 << 20


def gqe_forward_noalloc(cfg, x, wq, wk, wv, wr, wo, out, stream=None):
    """gqe_forward with the library's per-device workspace array: allocates
    nothing; calls that overlap on one device race."""
    _check(_lib.gqe_forward_noalloc(ctypes.byref(cfg), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv),
                                    _ptr(wr), _ptr(wo), _ptr(out), _stream(stream)),
           "gqe_forward_noalloc")


def gqa_project(cfg, x, wq, wk, wv, ws, stream=None):
    _check(_lib.gqa_project(ctypes.byref(cfg), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(ws),
                            ws.numel(), _stream(stream)), "gqa_project")


def gqa_attention(cfg, ws, stream=None):
    _check(_lib.gqa_attention(ctypes.byref(cfg), _ptr(ws), ws.numel(), _stream(stream)),
           "gqa_attention")


def gqa_output(cfg, wo, out, ws, stream=None):
    _check(_lib.gqa_output(ctypes.byref(cfg), _ptr(wo), _ptr(out), _ptr(ws), ws.numel(),
                           _stream(stream)), "gqa_output")


def gqa_forward(cfg, x, wq, wk, wv, wo, out, ws, stream=None):
    _check(_lib.gqa_forward(ctypes.byref(cfg), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo),
                            _ptr(out), _ptr(ws), ws.numel(), _stream(stream)), "gqa_forward")


def gqe_decode_workspace_bytes(cfg: GqeConfig) -> int:
    return int(_lib.gqe_decode_workspace_bytes(ctypes.byref(cfg)))


def gqa_decode_workspace_bytes(cfg: GqeConfig) -> int:
    return int(_lib.gqa_decode_workspace_bytes(ctypes.byref(cfg)))


def alloc_decode_workspace(cfg: GqeConfig, dense: bool = False, device="cuda") -> torch.Tensor:
    n = gqa_decode_workspace_bytes(cfg) if dense else gqe_decode_workspace_bytes(cfg)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def gqe_decode(cfg, x, wq, wk, wv, wr, wo, k_cache, vt_cache, pos, out, ws, stream=None):
    """One decode step: cfg.batch sequences, cfg.seq_len the cache capacity;
    pos is a device int32 tensor [B]; the caches are updated in place."""
    _check(_lib.gqe_decode(ctypes.byref(cfg), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wr),
                           _ptr(wo), _ptr(k_cache), _ptr(vt_cache), _ptr(pos), _ptr(out),
                           _ptr(ws), ws.numel(), _stream(stream)), "gqe_decode")


def gqa_decode(cfg, x, wq, wk, wv, wo, k_cache, vt_cache, pos, out, ws, stream=None):
    _check(_lib.gqa_decode(ctypes.byref(cfg), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo),
                           _ptr(k_cache), _ptr(vt_cache), _ptr(pos), _ptr(out), _ptr(ws),
                           ws.numel(), _stream(stream)), "gqa_decode")


def gqe_backward_workspace_bytes(cfg: GqeConfig) -> int:
    return int(_lib.gqe_backward_workspace_bytes(ctypes.byref(cfg)))


def gqa_backward_workspace_bytes(cfg: GqeConfig) -> int:
    return int(_lib.gqa_backward_workspace_bytes(ctypes.byref(cfg)))


def alloc_backward_workspace(cfg: GqeConfig, dense: bool = False, device="cuda") -> torch.Tensor:
    n = gqa_backward_workspace_bytes(cfg) if dense else gqe_backward_workspace_bytes(cfg)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def gqe_backward(cfg, x, wq, wk, wv, wr, wo, dy, aux_weight, fwd_ws, dx, dwq, dwk, dwv, dwr, dbr,
                 dwo, aux_loss, ws, stream=None):
    """Gradients of <y, dy> + aux_weight * L_aux (float32 tensors, overwritten);
    fwd_ws is the workspace of a gqe_forward on the same inputs."""
    _check(_lib.gqe_backward(ctypes.byref(cfg), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wr),
                             _ptr(wo), _ptr(dy), float(aux_weight), _ptr(fwd_ws), fwd_ws.numel(),
                             _ptr(dx), _ptr(dwq), _ptr(dwk), _ptr(dwv), _ptr(dwr), _ptr(dbr),
                             _ptr(dwo), _ptr(aux_loss), _ptr(ws), ws.numel(), _stream(stream)),
           "gqe_backward")


def gqa_backward(cfg, x, wq, wk, wv, wo, dy, fwd_ws, dx, dwq, dwk, dwv, dwo, ws, stream=None):
    _check(_lib.gqa_backward(ctypes.byref(cfg), _ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo),
                             _ptr(dy), _ptr(fwd_ws), fwd_ws.numel(), _ptr(dx), _ptr(dwq),
                             _ptr(dwk), _ptr(dwv), _ptr(dwo), _ptr(ws), ws.numel(),
                             _stream(stream)), "gqa_backward")


def peak_blocks() -> int:
    return int(_lib.gqe_peak_blocks())


def peak_mfma_bf16(out, blocks, iters, stream=None):
    """Enqueue the matrix-core probe: blocks*4*iters*4*32768 flop; out holds
    blocks*256 float32 values."""
    _check(_lib.gqe_peak_mfma_bf16(_ptr(out), blocks, iters, _stream(stream)), "gqe_peak_mfma_bf16")


def peak_copy(dst, src, stream=None):
    """Enqueue the HBM copy probe: src's bytes into dst (same size)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise GqeError("gqe_peak_copy: dst and src sizes differ")
    _check(_lib.gqe_peak_copy(_ptr(dst), _ptr(src), n, _stream(stream)), "gqe_peak_copy")


def workspace_views(cfg: GqeConfig, ws: torch.Tensor, dense: bool = False) -> dict:
    """Typed views of the intermediates inside a workspace (see gqe_ws_layout)."""
    lay = gqa_workspace_layout(cfg) if dense else gqe_workspace_layout(cfg)
    B, L, G, E, k, D = (cfg.batch, cfg.seq_len, cfg.n_groups, cfg.n_experts, cfg.top_k,
                        cfg.head_dim)
    dt = cfg.torch_dtype
    es = 2 if dt == torch.bfloat16 else 4

    def view(off, shape, dtype, esize):
        n = 1
        for s in shape:
            n *= s
        return ws[off:off + n * esize].view(dtype).view(*shape)

    out = {}
    if not dense:
        K = total_k(cfg)
        rows = B * L * K
        # [B, L, G, k] for a uniform k, [B, L, K] for per-group counts
        shp = (B, L, G, k) if not cfg.group_top_k else (B, L, K)
        out["idx"] = view(lay.idx, shp, torch.int32, 4)
        out["w"] = view(lay.w, shp, torch.float32, 4)
        out["counts"] = view(lay.counts, (B, G, E), torch.int32, 4)
        out["offsets"] = view(lay.offsets, (B * G * E + 1,), torch.int32, 4)
        out["pos"] = view(lay.pos, (rows,), torch.int32, 4)
        out["slot"] = view(lay.slot, (rows,), torch.int32, 4)
        out["q"] = view(lay.q, (B, K + 1, L, D), dt, es)
        full = cfg.output_mode == OUTPUT_MODES["full"]
        slots = K + (2 if full else 0)
        out["s"] = view(lay.s, (B, L, slots * D), dt, es)
        out["lse"] = view(lay.lse, (B, K + (1 if full else 0), L), torch.float32, 4)
    else:
        out["q"] = view(lay.q, (B, G * E, L, D), dt, es)
        out["s"] = view(lay.s, (B, L, G * E * D), dt, es)
        out["lse"] = view(lay.lse, (B, G * E, L), torch.float32, 4)
    out["k"] = view(lay.k, (B, G, L, D), dt, es)
    # V^T per 64-key tile, keys permuted inside 16-key groups (see include/gqe.h)
    out["vt"] = view(lay.vt, (B, G, int(lay.vt_tiles), D, 64), dt, es)
    return out

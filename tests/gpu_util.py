"""Helpers shared by the GPU tests: moving seeded inputs to the device, reading
results back as exact float64, and the output gates."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import workloads as W


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return W.bf16_bits_to_f32(t.contiguous().view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    return t.double().numpy()


def round_like(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the stored element type (bf16 RNE or fp32); returns stored form."""
    a32 = np.asarray(a, dtype=np.float32)
    return W.f32_to_bf16_bits(a32) if dtype == W.BF16 else a32


# Column of key position p inside its 16-key group in the tiled V^T workspace
# layout (include/gqe.h): key 8a+4u+r sits at column 8u+4a+r.
_VT_COL = np.array([(p & 3) | ((p & 4) << 1) | ((p & 8) >> 1) for p in range(16)])


def vt_encode(v: np.ndarray) -> np.ndarray:
    """V [B, G, L, D] (any dtype) -> tiled V^T [B, G, ceil(L/64), D, 64], zero padded."""
    B, G, L, D = v.shape
    nt = (L + 63) // 64
    pad = np.zeros((B, G, nt * 64, D), dtype=v.dtype)
    pad[:, :, :L] = v
    cols = (np.arange(nt * 64) // 16) * 16 + _VT_COL[np.arange(nt * 64) % 16]
    out = np.zeros_like(pad)
    out[:, :, cols] = pad
    return np.ascontiguousarray(out.reshape(B, G, nt, 64, D).transpose(0, 1, 2, 4, 3))


def vt_decode(vt: np.ndarray, L: int) -> np.ndarray:
    """Tiled V^T [B, G, nt, D, 64] -> V [B, G, L, D]."""
    B, G, nt, D, _ = vt.shape
    flat = vt.transpose(0, 1, 2, 4, 3).reshape(B, G, nt * 64, D)
    cols = (np.arange(nt * 64) // 16) * 16 + _VT_COL[np.arange(nt * 64) % 16]
    return flat[:, :, cols][:, :, :L]


def output_gate(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    """The output tolerances: max-abs 2e-2 and mean-abs 2e-3 for bf16 with fp32
    accumulation; 1e-5 for float32 layers.  Also returns the relative L2 error."""
    err = np.abs(gpu - ref)
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300))
    if dtype == W.BF16:
        assert err.max() <= 2e-2, f"{what}: max-abs {err.max():.3e} > 2e-2 (rel L2 {rel:.2e})"
        assert err.mean() <= 2e-3, f"{what}: mean-abs {err.mean():.3e} > 2e-3 (rel L2 {rel:.2e})"
    else:
        assert err.max() <= 1e-5, f"{what}: max-abs {err.max():.3e} > 1e-5 (rel L2 {rel:.2e})"
    return float(err.max()), float(err.mean()), rel


@functools.lru_cache(maxsize=2)
def inputs(name: str, seq_len: int = 0, batch: int = 0):
    wl = W.WORKLOADS[name]
    if seq_len:
        wl = wl.with_(seq_len=seq_len)
    if batch:
        wl = wl.with_(batch=batch)
    return wl, W.make_inputs(wl, with_gqa=True)


def f64_inputs(wl, I):
    f = lambda a: W.to_f64(a, wl.dtype)  # noqa: E731
    x = W.bf16_bits_to_f32(I["x"]) if wl.dtype == W.BF16 else I["x"]   # exact, float32 storage
    return dict(x=x, wq=f(I["wq"]), wk=f(I["wk"]), wv=f(I["wv"]), wr=f(I["wr"]), wo=f(I["wo"]),
                br=I["br"].astype(np.float64), wq_dense=f(I["wq_dense"]), wo_dense=f(I["wo_dense"]))


# Gates of the bf16 gradients, per tensor: (relative L2, max-abs over the
# tensor's largest magnitude).  Every product takes bf16 operands (dO, P, dS
# and the stacked gradient matrix) with float32 accumulation; the gates sit
# at about twice the largest error measured over the backward tests.  The
# router's gradients sum the logit gradients of every token, with
# cancellation, and carry the largest errors.
BF16_GRAD_GATE = {"dx": (1e-2, 1.5e-2), "dwq": (1e-2, 1.5e-2), "dwk": (1e-2, 1.5e-2),
                  "dwv": (1e-2, 1.5e-2), "dwo": (1e-2, 1.5e-2), "dwr": (2e-2, 3e-2),
                  "dbr": (2e-2, 3e-2)}


def grad_gate(gpu, ref, dtype, what, key):
    """Relative L2 and max-abs (over the largest magnitude) error of one
    gradient tensor against the oracle's, asserted against its gate: the
    bf16 table above, or relative L2 1e-5 for float32 layers."""
    gpu = np.asarray(gpu, dtype=np.float64).reshape(ref.shape)
    scale = max(np.abs(ref).max(), 1e-30)
    rel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.abs(gpu - ref).max() / scale)
    log(f"  {what}: rel-L2 {rel:.2e} max/max {mx:.2e}")
    if dtype == W.BF16:
        g_rel, g_max = BF16_GRAD_GATE[key]
        assert rel <= g_rel and mx <= g_max, f"{what}: rel-L2 {rel:.3e}, max-abs/max {mx:.3e}"
    else:
        assert rel <= 1e-5, f"{what}: rel-L2 {rel:.3e}, max-abs/max {mx:.3e}"
    return rel, mx

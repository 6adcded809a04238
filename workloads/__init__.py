"""Seeded synthetic inputs for the Grouped Query Experts (GQE) prefill layer.

This module only draws numbers: it holds none of the layer's arithmetic.  Both
the CPU oracle's tests and the HIP path's tests and benchmark take their inputs
from here, so that the two sides consume identical bits.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per workload, seed 0):

* draw order: x, W_q, W_k, W_v, W_r, W_O, then the dense-GQA output projection
  W_O^dense; the dense-GQA query projection is the first G*E*d_h rows of W_q.
* every draw is a float64 standard normal times the stated standard deviation,
  cast to float32, then (bf16 workloads) rounded to bfloat16 with
  round-to-nearest-even on the float32 bit pattern.  x is drawn in blocks of
  65 536 rows, which yields the same stream as one draw.
* weights use the [out, in] row-major layout of a PyTorch ``nn.Linear``:
  W_q is [(G*E+1)*d_h, d] (head h = g*E+e owns rows h*d_h..h*d_h+d_h-1, the
  always-on shared head owns the last d_h rows), W_k and W_v are [G*d_h, d],
  W_r is [G*E, d] (expert e of group g is row g*E+e), W_O is [d, (k*G+2)*d_h].
* the router bias is zero except for the load-imbalance workload, where
  b_r[g*E+e] = -s*ln(e+1) (s = 1.2) so that the router prior over the experts
  of every group is a Zipf(s) law.

The pages describe a 250M-parameter model trained on FineWeb-Edu and evaluated
on HellaSwag / ARC-Easy / PIQA; none of that data is used.  These tensors stand
in for it at the layer shapes of the five workloads below.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BF16 = "bf16"
FP32 = "fp32"

_X_BLOCK_ROWS = 65536


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and recipe of one synthetic GQE layer invocation."""

    name: str
    batch: int
    seq_len: int
    d_model: int
    n_groups: int      # G: KV heads
    n_experts: int     # E: routed query-head experts per group
    top_k: int         # k: experts selected per token per group
    head_dim: int      # d_h
    dtype: str         # "bf16" or "fp32"
    x_std: float
    w_std: float
    zipf_s: float = 0.0          # 0 => zero router bias
    sample_rows: int = 0         # 0 => every query row is checked
    description: str = ""

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    @property
    def routed_heads(self) -> int:
        return self.n_groups * self.n_experts

    @property
    def slot_heads(self) -> int:
        """Query rows computed per token: k*G routed + 1 shared."""
        return self.top_k * self.n_groups + 1

    @property
    def slot_width(self) -> int:
        """Width of the concatenated slot vector fed to W_O, (k*G+2)*d_h."""
        return (self.top_k * self.n_groups + 2) * self.head_dim

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload(
        "tiny_fp32", 1, 128, 256, 2, 2, 1, 32, FP32, 1.0, 1.0 / math.sqrt(256.0),
        description="tiny fp32 GQE layer: B1 L128 d256 G2 E2 k1 d_h32"),
    "l2k": Workload(
        "l2k", 1, 2048, 1024, 4, 4, 2, 64, BF16, 1.0, 0.02,
        description="250M-scale GQE layer bf16: B1 L2048 d1024 G4 E4 k2 d_h64"),
    "b4_l8k": Workload(
        "b4_l8k", 4, 8192, 1024, 4, 4, 2, 64, BF16, 1.0, 0.02,
        description="B4 x L8192 bf16, near-uniform expert load, plus dense GQA"),
    "l128k": Workload(
        "l128k", 1, 131072, 1024, 4, 4, 2, 64, BF16, 1.0, 0.02, sample_rows=512,
        description="B1 x L131072 bf16"),
    "l1m_zipf": Workload(
        "l1m_zipf", 1, 1048576, 1024, 4, 4, 2, 64, BF16, 1.0, 0.02, zipf_s=1.2,
        sample_rows=256,
        description="B1 x L1048576 bf16, Zipf(1.2) router prior"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    a = (rng.standard_normal(shape) * std).astype(np.float32)
    return f32_to_bf16_bits(a) if dtype == BF16 else a


def _draw_x(rng, wl: Workload) -> np.ndarray:
    rows = wl.tokens
    out = np.empty((rows, wl.d_model), dtype=np.uint16 if wl.dtype == BF16 else np.float32)
    for r0 in range(0, rows, _X_BLOCK_ROWS):
        r1 = min(rows, r0 + _X_BLOCK_ROWS)
        out[r0:r1] = _draw(rng, (r1 - r0, wl.d_model), wl.x_std, wl.dtype)
    return out.reshape(wl.batch, wl.seq_len, wl.d_model)


def router_bias(wl: Workload) -> np.ndarray:
    """float32 [G*E]: zero, or -s*ln(e+1) per group (a Zipf(s) prior)."""
    b = np.zeros((wl.n_groups, wl.n_experts), dtype=np.float64)
    if wl.zipf_s:
        b[:] = 0.0 - wl.zipf_s * np.log(np.arange(1, wl.n_experts + 1, dtype=np.float64))
    return b.reshape(-1).astype(np.float32)


def make_inputs(wl: Workload, seed: int = 0, with_gqa: bool = False) -> dict:
    """Draw every input of one workload.

    Returns a dict of numpy arrays.  bf16 tensors are uint16 bit patterns,
    fp32 tensors are float32.  Keys: x [B,L,d], wq, wk, wv, wr, wo (layouts in
    the module docstring), br (float32 [G*E]), and with ``with_gqa`` also
    wq_dense ([G*E*d_h, d], a view of W_q's routed rows) and wo_dense
    ([d, G*E*d_h]).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    d, G, E, k, dh = wl.d_model, wl.n_groups, wl.n_experts, wl.top_k, wl.head_dim
    x = _draw_x(rng, wl)
    wq = _draw(rng, ((G * E + 1) * dh, d), wl.w_std, wl.dtype)
    wk = _draw(rng, (G * dh, d), wl.w_std, wl.dtype)
    wv = _draw(rng, (G * dh, d), wl.w_std, wl.dtype)
    wr = _draw(rng, (G * E, d), wl.w_std, wl.dtype)
    wo = _draw(rng, (d, (k * G + 2) * dh), wl.w_std, wl.dtype)
    out = dict(x=x, wq=wq, wk=wk, wv=wv, wr=wr, wo=wo, br=router_bias(wl))
    if with_gqa:
        out["wq_dense"] = wq[: G * E * dh]
        out["wo_dense"] = _draw(rng, (d, G * E * dh), wl.w_std, wl.dtype)
    return out


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored input (bf16 bits or float32)."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def sample_rows(wl: Workload, seed: int = 0) -> np.ndarray:
    """Sorted, distinct positions t at which sampled workloads are checked.

    Always {0, 1, L-1}; the rest are drawn uniformly inside 8 log-spaced
    position bands [L^(i/8)-1, L^((i+1)/8)) so early rows (large outputs) and
    late rows (long causal spans) are both covered.
    """
    L, n = wl.seq_len, wl.sample_rows
    if n == 0 or n >= L:
        return np.arange(L, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    chosen = {0, 1, L - 1}
    edges = [int(round(L ** (i / 8.0))) - 1 for i in range(9)]
    edges[0], edges[-1] = 0, L
    per_band = max(1, (n - 3) // 8)
    for i in range(8):
        lo, hi = edges[i], max(edges[i] + 1, edges[i + 1])
        span = hi - lo
        want = min(per_band, span)
        chosen.update(int(v) for v in lo + rng.choice(span, size=want, replace=False))
    rest = np.setdiff1d(np.arange(L), np.fromiter(chosen, dtype=np.int64))
    need = n - len(chosen)
    if need > 0:
        chosen.update(int(v) for v in rng.choice(rest, size=need, replace=False))
    rows = np.array(sorted(chosen), dtype=np.int64)
    return rows[:n] if len(rows) > n else rows


# ---------------------------------------------------------------------------
# decode: one new token per sequence against a KV cache
# ---------------------------------------------------------------------------

DECODE_WORKLOADS = {
    "dec_tiny_fp32": Workload(
        "dec_tiny_fp32", 3, 200, 256, 2, 2, 1, 32, FP32, 1.0, 1.0 / math.sqrt(256.0),
        description="tiny fp32 decode: 3 sequences, cache 200, d256 G2 E2 k1 d_h32"),
    "dec_b64_c8k": Workload(
        "dec_b64_c8k", 64, 8192, 1024, 4, 4, 2, 64, BF16, 1.0, 0.02,
        description="250M-scale layer decode bf16: 64 sequences, cache 8192"),
}


def make_decode_inputs(wl: Workload, seed: int = 0, with_gqa: bool = False) -> dict:
    """Inputs of one decode step: wl.batch sequences, wl.seq_len the cache capacity.

    Layer weights and the new tokens come from ``make_inputs`` of the same
    shape at one position (x is [B, d]).  A second generator (seed + 2) then
    draws, in order, the key cache and the value cache ([B, G, Lc, d_h], the
    standard deviation of a projection of x, x_std * w_std * sqrt(d)), and the
    positions pos [B] uniform in [0, Lc), after which pos[0] = Lc - 1 (a full
    cache) and, for B > 1, pos[1] = 0 (an empty one).  Entries at positions
    >= pos[b] hold random values that a correct step never reads.
    """
    I = make_inputs(wl.with_(seq_len=1), seed, with_gqa)
    I["x"] = np.ascontiguousarray(I["x"][:, 0])
    rng = np.random.Generator(np.random.PCG64(seed + 2))
    B, G, Lc, dh = wl.batch, wl.n_groups, wl.seq_len, wl.head_dim
    kv_std = wl.x_std * wl.w_std * math.sqrt(wl.d_model)
    I["k_cache"] = _draw(rng, (B, G, Lc, dh), kv_std, wl.dtype)
    I["v_cache"] = _draw(rng, (B, G, Lc, dh), kv_std, wl.dtype)
    pos = rng.integers(0, Lc, size=B).astype(np.int32)
    pos[0] = Lc - 1
    if B > 1:
        pos[1] = 0
    I["pos"] = pos
    return I

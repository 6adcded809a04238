"""The attention step alone (gqe_attention) on queries, keys and values written
straight into the workspace, against causal softmax attention of the
definition in float64 from the same stored values (pptc.cn review, section 5:
every activated query row attends causally to its group's unchanged K/V).
Sampled rows of every slot head: the output row and the saved log-sum-exp.
Needs an MI355X.

The softmax scale is ln 2, so the kernel's pre-scaled queries (q times
scale * log2 e, stored back in the operand type) equal the stored queries and
the log-sum-exp in log2 units is log2 sum_s 2^(q . k_s) exactly."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import workloads as W  # noqa: E402
from gpu_util import log, round_like, to_dev, to_f64, vt_encode  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gqe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_query_moe_amd import gqe as mod
    return mod


# L, B, amplitude of q and k, dtype; 9 slot heads (G4, k2, plus the shared
# head) put L >= 29128 on the long-launch schedule, shorter L on the short one
CASES = [
    (100, 2, 0.6, "bf16"),
    (2048, 1, 0.6, "bf16"),
    (2048, 1, 2.0, "bf16"),
    (33000, 1, 0.6, "bf16"),
    (33000, 1, 2.0, "bf16"),
    (300, 1, 0.6, "fp32"),
]


@pytest.mark.parametrize("L,B,amp,dtype", CASES)
def test_attention_rows_and_logsumexp(gqe, L, B, amp, dtype):
    G, E, k, D = 4, 4, 2, 64
    H = G * k + 1
    log(f"[attention] L={L} B={B} amp={amp} {dtype}")
    cfg = gqe.make_config(B, L, 1024, G, E, k, D, dtype=dtype, softmax_scale=math.log(2.0))
    ws = gqe.alloc_workspace(cfg)
    v = gqe.workspace_views(cfg, ws)
    rng = np.random.Generator(np.random.PCG64(L + int(10 * amp)))
    q = W._draw(rng, (B, H, L, D), amp, dtype)
    kk = W._draw(rng, (B, G, L, D), amp, dtype)
    vv = W._draw(rng, (B, G, L, D), 0.6, dtype)
    v["q"].copy_(to_dev(q, dtype))
    v["k"].copy_(to_dev(kk, dtype))
    v["vt"].copy_(to_dev(vt_encode(vv), dtype))
    gqe.gqe_attention(cfg, ws)
    torch.cuda.synchronize()
    s = to_f64(v["s"])
    lse = v["lse"].cpu().numpy().astype(np.float64)
    qf, kf, vf = (W.to_f64(a, dtype) for a in (q, kk, vv))
    picks = np.unique(np.concatenate([[0, 1, 63, 64, L - 1], rng.integers(0, L, 27)]))
    worst_lse = worst_o = 0.0
    for b in range(B):
        for h in range(H):
            g = h // k if h < G * k else 0
            for t in picks:
                z = kf[b, g, : t + 1] @ qf[b, h, t]          # log2 units at scale ln 2
                m = z.max()
                p = np.exp2(z - m)
                want_lse = m + math.log2(p.sum())
                want_o = (p @ vf[b, g, : t + 1]) / p.sum()
                worst_lse = max(worst_lse, abs(lse[b, h, t] - want_lse))
                worst_o = max(worst_o, np.abs(s[b, t, h * D:(h + 1) * D] - want_o).max())
    log(f"  lse max-abs {worst_lse:.3e}  o max-abs {worst_o:.3e}")
    assert worst_lse <= 2e-5, worst_lse
    assert worst_o <= (1e-2 if dtype == W.BF16 else 1e-5), worst_o


# Scores far outside the range of ordinary inputs.  Keys at a few spike
# positions of group 1 are 40 * u for one unit vector u, and slot head 3 (of
# group 1) adds 4 * u to every query, so its scores against the spikes reach
# about 160 in log2 units (2^160 overflows float32) while its score against
# key 0 stays small: the fast path admits those blocks and must detect the
# overflow after the key walk.  Slot head 0 has queries ten times larger, so
# many of its rows' first scores leave [-60, 60] and its blocks are refused
# at the start.  All other heads stay ordinary, so one launch mixes blocks
# that keep the fast result with blocks recomputed by the fallback.
SPIKE_CASES = [
    (2048, 1, "bf16"),      # short launch: fallback inside the same launch
    (33000, 1, "bf16"),     # long launch: fast launch, then the fallback launch
    (700, 2, "fp32"),
]


@pytest.mark.parametrize("L,B,dtype", SPIKE_CASES)
def test_attention_fallback_paths(gqe, L, B, dtype):
    G, E, k, D = 4, 4, 2, 64
    H = G * k + 1
    log(f"[attention fallback] L={L} B={B} {dtype}")
    cfg = gqe.make_config(B, L, 1024, G, E, k, D, dtype=dtype, softmax_scale=math.log(2.0))
    ws = gqe.alloc_workspace(cfg)
    v = gqe.workspace_views(cfg, ws)
    rng = np.random.Generator(np.random.PCG64(900 + L))
    q = rng.standard_normal((B, H, L, D)) * 0.6
    kk = rng.standard_normal((B, G, L, D)) * 0.6
    vv = rng.standard_normal((B, G, L, D)) * 0.6
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    spikes = [s for s in (100, 1500, 20000) if s < L]
    kk[:, 1, spikes] = 40.0 * u
    q[:, 3] += 4.0 * u
    q[:, 0] *= 10.0
    st = [round_like(a, dtype) for a in (q, kk, vv)]
    v["q"].copy_(to_dev(st[0], dtype))
    v["k"].copy_(to_dev(st[1], dtype))
    v["vt"].copy_(to_dev(vt_encode(st[2]), dtype))
    gqe.gqe_attention(cfg, ws)
    torch.cuda.synchronize()
    s = to_f64(v["s"])
    lse = v["lse"].cpu().numpy().astype(np.float64)
    qf, kf, vf = (W.to_f64(a, dtype) for a in st)
    picks = np.unique(np.concatenate([[0, 1, 99, 100, 101, L - 1], spikes,
                                      rng.integers(0, L, 20)]))
    worst_lse = worst_o = 0.0
    for b in range(B):
        for h in range(H):
            g = h // k if h < G * k else 0
            for t in picks:
                z = kf[b, g, : t + 1] @ qf[b, h, t]
                m = z.max()
                p = np.exp2(z - m)
                want_lse = m + math.log2(p.sum())
                want_o = (p @ vf[b, g, : t + 1]) / p.sum()
                # each score is a float32 sum of D products: its rounding error
                # is at most about D * 2^-24 * sum_i |q_i k_i| (and exact
                # products for bf16 operands), which bounds the error of the
                # log-sum-exp on top of the 2e-5 of ordinary scores
                bound = 2e-5 + D * 2.0 ** -24 * (np.abs(kf[b, g, : t + 1]) @ np.abs(qf[b, h, t])).max()
                worst_lse = max(worst_lse, abs(lse[b, h, t] - want_lse) / bound * 2e-5)
                worst_o = max(worst_o, np.abs(s[b, t, h * D:(h + 1) * D] - want_o).max())
    log(f"  lse max-abs (scaled) {worst_lse:.3e}  o max-abs {worst_o:.3e}")
    assert np.isfinite(s).all() and np.isfinite(lse).all()
    assert worst_lse <= 2e-5, worst_lse
    assert worst_o <= (1e-2 if dtype == W.BF16 else 1e-5), worst_o

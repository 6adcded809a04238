"""Per-group expert counts (the non-uniform k of the pages' future work) on
the GPU against the oracle's per-group layer, through the C ABI (needs an
MI355X).  Routing and dispatch lists bit for bit; outputs to the gates of the
uniform layer (max-abs 2e-2 and mean-abs 2e-3 for bf16, 1e-5 for fp32)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_util import f64_inputs, log, output_gate, to_dev, to_f64  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gqe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_query_moe_amd import gqe as mod
    return mod


CASES = [
    # L, B, d, G, E, ks, D, dtype, mode
    (128, 1, 256, 2, 2, [1, 2], 32, "fp32", "full"),
    (128, 1, 256, 2, 2, [2, 1], 32, "fp32", "hard"),
    (200, 2, 256, 2, 3, [3, 1], 32, "fp32", "weighted_concat"),
    (2048, 1, 1024, 4, 4, [1, 2, 3, 2], 64, "bf16", "full"),
    (2048, 1, 1024, 4, 4, [3, 3, 2, 1], 64, "bf16", "full"),        # K = 9 slots
    (777, 2, 1024, 4, 4, [4, 1, 1, 2], 64, "bf16", "weighted_concat"),
    (9000, 1, 1024, 4, 4, [4, 1, 2, 1], 64, "bf16", "full"),        # chunked dispatch path
]


@pytest.mark.parametrize("L,B,d,G,E,ks,D,dtype,mode", CASES)
def test_group_k_forward(gqe, L, B, d, G, E, ks, D, dtype, mode):
    K = sum(ks)
    wl = W.Workload("group_k", B, L, d, G, E, max(ks), D, dtype, 1.0,
                    0.05 if dtype == W.FP32 else 0.02)
    log(f"[group k] {wl} ks={ks} {mode}")
    I = W.make_inputs(wl, seed=21, with_gqa=True)
    rng = np.random.Generator(np.random.PCG64(22))
    width = (K + (2 if mode == "full" else 0)) * D
    I["wo"] = W._draw(rng, (d, width), wl.w_std, dtype)
    dev = {k: to_dev(v, dtype) for k, v in I.items()}
    cfg = gqe.make_config(B, L, d, G, E, max(ks), D, dtype=dtype, router_bias=dev["br"],
                          output_mode=mode, group_top_k=ks)
    ws = gqe.alloc_workspace(cfg)
    out = torch.empty((B, L, d), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], out, ws)
    torch.cuda.synchronize()
    F = f64_inputs(wl, I)
    ref = oracle.gqe_forward_group_k(F["x"], F["wq"], F["wk"], F["wv"], F["wr"], F["wo"], F["br"],
                                     G, E, ks, D, output_mode=mode)
    v = gqe.workspace_views(cfg, ws)
    assert np.array_equal(v["idx"].cpu().numpy(), ref["idx"]), "idx"
    w_gpu = v["w"].cpu().numpy().astype(np.float64)
    if mode == "weighted_concat":   # the router writes p there
        koff = oracle.group_offsets(ks)
        w_ref = np.concatenate([np.take_along_axis(ref["p"][:, :, g], ref["idx"][:, :, koff[g]:koff[g + 1]]
                                                   .astype(np.int64), axis=-1) for g in range(G)], axis=-1)
    else:
        w_ref = ref["w"]
    assert np.abs(w_gpu - w_ref).max() <= 2e-7
    for key in ("counts", "offsets", "pos", "slot"):
        assert np.array_equal(v[key].cpu().numpy(), ref[key]), key
    mx, mean, rel = output_gate(to_f64(out), ref["y"], dtype, f"group k {ks} y")
    log(f"  y: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e}")


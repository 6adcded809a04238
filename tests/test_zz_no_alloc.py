"""gqe_forward_noalloc (the entry point whose workspace is the library's own
per-device array) against gqe_forward with a caller-allocated workspace,
through the C ABI (needs an MI355X)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import workloads as W  # noqa: E402
from gpu_util import log, output_gate, to_dev, to_f64  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gqe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_query_moe_amd import gqe as mod
    return mod


def _layer(gqe, wl, seed):
    I = W.make_inputs(wl, seed=seed)
    dev = {k: to_dev(v, wl.dtype) for k, v in I.items()}
    cfg = gqe.make_config(wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts, wl.top_k,
                          wl.head_dim, dtype=wl.dtype, router_bias=dev["br"])
    return cfg, dev


def _both(gqe, wl, seed):
    cfg, dev = _layer(gqe, wl, seed)
    args = (dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"])
    shape = (wl.batch, wl.seq_len, wl.d_model)
    y_ref = torch.empty(shape, dtype=cfg.torch_dtype, device="cuda")
    ws = gqe.alloc_workspace(cfg)
    gqe.gqe_forward(cfg, *args, y_ref, ws)
    y = torch.full(shape, float("nan"), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqe_forward_noalloc(cfg, *args, y)
    torch.cuda.synchronize()
    return y, y_ref


def test_noalloc_matches_forward_twice(gqe):
    """Two calls in a row, the second on a smaller layer: each output equals
    gqe_forward's bit for bit (the same kernels on the same inputs)."""
    base = W.WORKLOADS["l2k"]
    for wl, seed in ((base.with_(batch=2), 4), (base.with_(seq_len=777), 5)):
        log(f"[noalloc] B={wl.batch} L={wl.seq_len}")
        y, y_ref = _both(gqe, wl, seed)
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
        output_gate(to_f64(y), to_f64(y_ref), wl.dtype, "noalloc vs forward")


def test_noalloc_fp32_and_limit(gqe):
    """The float32 tiny layer matches too; a layer whose workspace exceeds the
    array is refused with GQE_ERR_WORKSPACE before anything runs."""
    wl = W.WORKLOADS["tiny_fp32"]
    log("[noalloc] tiny fp32")
    y, y_ref = _both(gqe, wl, 0)
    assert torch.equal(y, y_ref)
    big = W.WORKLOADS["l2k"].with_(batch=8, seq_len=8192)
    cfg = gqe.make_config(big.batch, big.seq_len, big.d_model, big.n_groups, big.n_experts,
                          big.top_k, big.head_dim)
    assert gqe.gqe_workspace_bytes(cfg) > gqe.NOALLOC_SCRATCH_BYTES
    t = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gqe.GqeError, match="WORKSPACE"):
        gqe.gqe_forward_noalloc(cfg, t, t, t, t, t, t, t)

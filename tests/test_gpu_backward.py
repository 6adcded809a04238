"""Backward pass on the GPU against the oracle's backward, through the C ABI
(needs an MI355X).

gqe_forward runs first; gqe_backward then reads its workspace.  Every
gradient (dx, dW_q, dW_k, dW_v, dW_r, db_r, dW_O) and the auxiliary loss are
compared with the float64 oracle.  Gate, per gradient tensor (gpu_util's
BF16_GRAD_GATE): for bf16 layers (bf16 operands of every product, float32
accumulation) relative L2 <= 1e-2 and max-abs <= 1.5e-2 of the tensor's
largest magnitude for dx and the projection weights, 2e-2 and 3e-2 for the
router's weight and bias (sums over every token's logit gradient); relative
L2 <= 1e-5 for float32 layers.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_util import f64_inputs, grad_gate, inputs, log, to_dev, to_f64  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gqe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_query_moe_amd import gqe as mod
    return mod


def _cfg(gqe, wl, dev, **kw):
    return gqe.make_config(wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts, wl.top_k,
                           wl.head_dim, dtype=wl.dtype, router_bias=dev["br"], **kw)


def _zeros(*shape):
    return torch.zeros(shape, dtype=torch.float32, device="cuda")


def run_backward(gqe, wl, I, dy, mode="full", aux_weight=0.0, **kw):
    dev = {k: to_dev(v, wl.dtype) for k, v in I.items()}
    cfg = _cfg(gqe, wl, dev, output_mode=mode, **kw)
    fws = gqe.alloc_workspace(cfg)
    y = torch.empty((wl.batch, wl.seq_len, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], y, fws)
    G, E, D, d = wl.n_groups, wl.n_experts, wl.head_dim, wl.d_model
    g = dict(dx=_zeros(wl.batch, wl.seq_len, d), dwq=_zeros(*I["wq"].shape),
             dwk=_zeros(*I["wk"].shape), dwv=_zeros(*I["wv"].shape), dwr=_zeros(G * E, d),
             dbr=_zeros(G * E), dwo=_zeros(*I["wo"].shape), aux=_zeros(1))
    ws = gqe.alloc_backward_workspace(cfg)
    gqe.gqe_backward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"],
                     to_dev(dy, wl.dtype), aux_weight, fws, g["dx"], g["dwq"], g["dwk"], g["dwv"],
                     g["dwr"], g["dbr"], g["dwo"], g["aux"], ws)
    torch.cuda.synchronize()
    return cfg, fws, {k: v.cpu().numpy() for k, v in g.items()}


def draw_dy(wl, seed=12):
    rng = np.random.Generator(np.random.PCG64(seed))
    return W._draw(rng, (wl.batch, wl.seq_len, wl.d_model), 1.0, wl.dtype)


@pytest.mark.parametrize("name", ["tiny_fp32", "l2k"])
def test_forward_saves_row_logsumexp(gqe, name):
    """The forward leaves each slot-head row's log2 softmax normalizer."""
    wl, I = inputs(name)
    dev = {k: to_dev(v, wl.dtype) for k, v in I.items()}
    cfg = _cfg(gqe, wl, dev)
    ws = gqe.alloc_workspace(cfg)
    y = torch.empty((wl.batch, wl.seq_len, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], y, ws)
    torch.cuda.synchronize()
    lse = gqe.workspace_views(cfg, ws)["lse"].cpu().numpy().astype(np.float64)
    F = f64_inputs(wl, I)
    ref = oracle.gqe_forward(F["x"], F["wq"], F["wk"], F["wv"], F["wr"], F["wo"], F["br"],
                             wl.n_groups, wl.n_experts, wl.top_k, wl.head_dim)
    sc = 1.0 / math.sqrt(wl.head_dim)
    L, kG = wl.seq_len, wl.top_k * wl.n_groups
    for b in range(wl.batch):
        for h in range(kG + 1):
            g = h // wl.top_k if h < kG else 0
            s = sc * ref["q"][b, :, h] @ ref["k_"][b, g].T
            s[np.triu_indices(L, 1)] = -np.inf
            m = s.max(axis=1)
            want = (m + np.log(np.exp(s - m[:, None]).sum(axis=1))) / math.log(2.0)
            err = np.abs(lse[b, h] - want).max()
            assert err <= (3e-2 if wl.dtype == W.BF16 else 1e-4), (b, h, err)


BWD_CASES = [
    ("tiny_fp32", "full", 0.0, {}),
    ("tiny_fp32", "full", 0.7, dict(shared_kv_group=1, softmax_scale=0.4)),
    ("tiny_fp32", "hard", 0.0, {}),
    ("tiny_fp32", "weighted_concat", 0.3, {}),
    ("l2k", "full", 0.01, {}),
    ("l2k", "weighted_concat", 0.0, {}),
]


@pytest.mark.parametrize("name,mode,aux,kw", BWD_CASES)
def test_gqe_backward(gqe, name, mode, aux, kw):
    wl, I = inputs(name)
    log(f"[backward] {wl.name} {mode} aux={aux} {kw}")
    J = dict(I)
    if mode != "full":
        J["wo"] = np.ascontiguousarray(I["wo"][:, :wl.top_k * wl.n_groups * wl.head_dim])
    dy = draw_dy(wl)
    cfg, fws, g = run_backward(gqe, wl, J, dy, mode=mode, aux_weight=aux, **kw)
    F = f64_inputs(wl, J)
    okw = {}
    if "shared_kv_group" in kw:
        okw["shared_kv_group"] = kw["shared_kv_group"]
    if "softmax_scale" in kw:
        okw["scale"] = kw["softmax_scale"]
    ref = oracle.gqe_backward(F["x"], F["wq"], F["wk"], F["wv"], F["wr"], F["wo"], F["br"],
                              W.to_f64(dy, wl.dtype), wl.n_groups, wl.n_experts, wl.top_k,
                              wl.head_dim, output_mode=mode, aux_weight=aux, **okw)
    for key, rk in (("dwo", "dwo"), ("dx", "dx"), ("dwq", "dwq"), ("dwk", "dwk"), ("dwv", "dwv"),
                    ("dwr", "dwr"), ("dbr", "dbr")):
        if mode == "hard" and aux == 0.0 and rk in ("dwr", "dbr"):
            assert np.abs(g[key]).max() == 0.0
            continue
        rel, mx = grad_gate(g[key], ref[rk], wl.dtype, f"{name} {mode} {key}", key)
        log(f"  {key}: rel-L2 {rel:.2e} max/max {mx:.2e}")
    assert abs(float(g["aux"][0]) - ref["aux_loss"]) <= 1e-5 * max(1.0, abs(ref["aux_loss"]))


@pytest.mark.parametrize("name", ["tiny_fp32", "l2k"])
def test_gqa_backward(gqe, name):
    wl, I = inputs(name)
    dev = {k: to_dev(v, wl.dtype) for k, v in I.items()}
    cfg = _cfg(gqe, wl, dev)
    fws = gqe.alloc_workspace(cfg, dense=True)
    y = torch.empty((wl.batch, wl.seq_len, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqa_forward(cfg, dev["x"], dev["wq_dense"], dev["wk"], dev["wv"], dev["wo_dense"], y, fws)
    dy = draw_dy(wl, seed=13)
    g = dict(dx=_zeros(wl.batch, wl.seq_len, wl.d_model), dwq=_zeros(*I["wq_dense"].shape),
             dwk=_zeros(*I["wk"].shape), dwv=_zeros(*I["wv"].shape),
             dwo=_zeros(*I["wo_dense"].shape))
    ws = gqe.alloc_backward_workspace(cfg, dense=True)
    gqe.gqa_backward(cfg, dev["x"], dev["wq_dense"], dev["wk"], dev["wv"], dev["wo_dense"],
                     to_dev(dy, wl.dtype), fws, g["dx"], g["dwq"], g["dwk"], g["dwv"], g["dwo"], ws)
    torch.cuda.synchronize()
    F = f64_inputs(wl, I)
    ref = oracle.gqa_backward(F["x"], F["wq_dense"], F["wk"], F["wv"], F["wo_dense"],
                              W.to_f64(dy, wl.dtype), wl.n_groups, wl.n_experts, wl.head_dim)
    for key in ("dwo", "dx", "dwq", "dwk", "dwv"):
        grad_gate(g[key].cpu().numpy(), ref[key], wl.dtype, f"gqa {name} {key}", key)


@pytest.mark.parametrize("L,B,G,E,k,D,dtype", [
    (333, 2, 2, 3, 2, 32, "fp32"),
    (200, 1, 2, 2, 1, 128, "fp32"),
    (97, 2, 4, 4, 2, 64, "bf16"),
    (333, 2, 2, 3, 2, 32, "bf16"),
    (200, 1, 2, 2, 1, 128, "bf16"),
    (600, 1, 4, 4, 2, 64, "bf16"),     # several 256-key blocks, a ragged last one
    # few output tiles and a long token axis: the weight-gradient products
    # split K (dW_O and the stacked projection gradients), and in bf16 the
    # dK/dV query walk and the dQ key walk are split too
    (4100, 1, 2, 2, 1, 32, "fp32"),
    (4100, 1, 2, 2, 1, 32, "bf16"),
])
def test_backward_edge_shapes(gqe, L, B, G, E, k, D, dtype):
    """Ragged lengths (tails of every tile), every head size in both
    precisions, k = 1, and key blocks past the first."""
    wl = W.Workload("edge", B, L, 128, G, E, k, D, dtype, 1.0, 0.05)
    log(f"[backward edge] {wl}")
    I = W.make_inputs(wl, seed=4, with_gqa=True)
    dy = draw_dy(wl, seed=14)
    cfg, fws, g = run_backward(gqe, wl, I, dy, aux_weight=0.2)
    F = f64_inputs(wl, I)
    ref = oracle.gqe_backward(F["x"], F["wq"], F["wk"], F["wv"], F["wr"], F["wo"], F["br"],
                              W.to_f64(dy, wl.dtype), G, E, k, D, aux_weight=0.2)
    for key in ("dwo", "dx", "dwq", "dwk", "dwv", "dwr", "dbr"):
        grad_gate(g[key], ref[key], wl.dtype, f"edge {key}", key)


GROUP_K_BWD_CASES = [
    # L, B, G, E, per-group counts, D, dtype, output mode, aux weight, extra config
    (150, 2, 3, 3, [1, 3, 2], 32, "fp32", "full", 0.3, dict(shared_kv_group=2)),
    (150, 2, 3, 3, [2, 1, 3], 32, "fp32", "hard", 0.0, {}),
    (150, 1, 3, 3, [3, 2, 1], 32, "fp32", "weighted_concat", 0.2, {}),
    (700, 1, 4, 4, [1, 2, 3, 2], 64, "bf16", "full", 0.01, {}),
    (333, 2, 4, 8, [6, 1, 1, 2], 64, "bf16", "full", 0.01, {}),   # 7 slot heads on group 0
]


@pytest.mark.parametrize("L,B,G,E,ks,D,dtype,mode,aux,kw", GROUP_K_BWD_CASES)
def test_gqe_backward_group_k(gqe, L, B, G, E, ks, D, dtype, mode, aux, kw):
    """Per-group expert counts: every gradient and the auxiliary loss against
    the oracle's per-group backward."""
    K = sum(ks)
    wl = W.Workload("bwd_group_k", B, L, 128, G, E, max(ks), D, dtype, 1.0, 0.05)
    log(f"[backward group k] {wl} ks={ks} {mode} aux={aux} {kw}")
    I = W.make_inputs(wl, seed=15, with_gqa=True)
    rng = np.random.Generator(np.random.PCG64(16))
    I["wo"] = W._draw(rng, (wl.d_model, (K + (2 if mode == "full" else 0)) * D), 0.05, dtype)
    dy = draw_dy(wl, seed=17)
    cfg, fws, g = run_backward(gqe, wl, I, dy, mode=mode, aux_weight=aux, group_top_k=ks, **kw)
    F = f64_inputs(wl, I)
    ref = oracle.gqe_backward_group_k(F["x"], F["wq"], F["wk"], F["wv"], F["wr"], F["wo"], F["br"],
                                      W.to_f64(dy, dtype), G, E, ks, D, output_mode=mode,
                                      aux_weight=aux, **kw)
    for key in ("dwo", "dx", "dwq", "dwk", "dwv", "dwr", "dbr"):
        if mode == "hard" and aux == 0.0 and key in ("dwr", "dbr"):
            assert np.abs(g[key]).max() == 0.0
            continue
        rel, mx = grad_gate(g[key], ref[key], dtype, f"group k {ks} {mode} {key}", key)
        log(f"  {key}: rel-L2 {rel:.2e} max/max {mx:.2e}")
    assert abs(float(g["aux"][0]) - ref["aux_loss"]) <= 1e-5 * max(1.0, abs(ref["aux_loss"]))


def test_backward_is_deterministic_and_replays_from_a_graph(gqe):
    """Two gqe_backward calls give the same bits (no atomics anywhere), and so
    does every replay of a HIP graph captured from one, with eager work and
    synchronizations between the replays."""
    wl, I = inputs("l2k")
    dy = draw_dy(wl)
    _, _, g1 = run_backward(gqe, wl, I, dy, aux_weight=0.01)
    _, _, g2 = run_backward(gqe, wl, I, dy, aux_weight=0.01)
    for key in g1:
        assert np.array_equal(g1[key], g2[key]), key

    dev = {k: to_dev(v, wl.dtype) for k, v in I.items()}
    cfg = _cfg(gqe, wl, dev)
    fws = gqe.alloc_workspace(cfg)
    y = torch.empty((wl.batch, wl.seq_len, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], y, fws)
    G, E, d = wl.n_groups, wl.n_experts, wl.d_model
    g = dict(dx=_zeros(wl.batch, wl.seq_len, d), dwq=_zeros(*I["wq"].shape),
             dwk=_zeros(*I["wk"].shape), dwv=_zeros(*I["wv"].shape), dwr=_zeros(G * E, d),
             dbr=_zeros(G * E), dwo=_zeros(*I["wo"].shape), aux=_zeros(1))
    bws = gqe.alloc_backward_workspace(cfg)
    dyd = to_dev(dy, wl.dtype)

    def bwd():
        gqe.gqe_backward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], dyd,
                         0.01, fws, g["dx"], g["dwq"], g["dwk"], g["dwv"], g["dwr"], g["dbr"],
                         g["dwo"], g["aux"], bws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bwd()
    for rep in range(3):
        for t in g.values():
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for key, t in g.items():
            assert np.array_equal(t.cpu().numpy(), g1[key]), f"replay {rep}: {key}"
        # eager work in between
        _, _, _ = run_backward(gqe, wl, I, dy, aux_weight=0.01)
    del graph

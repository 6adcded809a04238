"""HIP path against the CPU oracle, through the C ABI (needs an MI355X).

Stage tests seed each stage with the oracle's inputs so errors do not
compound; layer tests run gqe_forward / gqa_forward end to end.  Routing and
dispatch must match bit for bit; floating outputs must meet max-abs 2e-2 and
mean-abs 2e-3 (bf16 with fp32 accumulation) or 1e-5 (float32 layers).
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_util import (f64_inputs, inputs, log, output_gate, round_like, to_dev, to_f64,  # noqa: E402
                      vt_decode, vt_encode)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gqe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_query_moe_amd import gqe as mod
    return mod


def cfg_for(gqe, wl, bias_dev=None, **kw):
    return gqe.make_config(wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts, wl.top_k,
                           wl.head_dim, dtype=wl.dtype, router_bias=bias_dev, **kw)


def device_inputs(wl, I):
    return {k: to_dev(v, wl.dtype) for k, v in I.items()}


def run_gqe(gqe, wl, I, dev=None, **cfgkw):
    dev = dev or device_inputs(wl, I)
    cfg = cfg_for(gqe, wl, dev["br"], **cfgkw)
    ws = gqe.alloc_workspace(cfg)
    out = torch.empty((wl.batch, wl.seq_len, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], out, ws)
    torch.cuda.synchronize()
    return cfg, ws, out


def oracle_gqe(wl, F, positions=None, **kw):
    return oracle.gqe_forward(F["x"], F["wq"], F["wk"], F["wv"], F["wr"], F["wo"], F["br"],
                              wl.n_groups, wl.n_experts, wl.top_k, wl.head_dim,
                              positions=positions, **kw)


def check_routing(gqe, cfg, ws, ref):
    v = gqe.workspace_views(cfg, ws)
    idx = v["idx"].cpu().numpy()
    assert np.array_equal(idx, ref["idx"]), f"idx mismatches: {(idx != ref['idx']).sum()}"
    w = v["w"].cpu().numpy().astype(np.float64)
    assert np.abs(w - ref["w"]).max() <= 2e-7
    assert np.array_equal(v["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(v["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(v["pos"].cpu().numpy(), ref["pos"])
    assert np.array_equal(v["slot"].cpu().numpy(), ref["slot"])


# ---------------------------------------------------------------------------
# stage parity (tiny fp32 layer, the 2k bf16 layer, and a ragged shape)
# ---------------------------------------------------------------------------

# the last case is long enough (B*L*heads >= 2^18) for the long-launch attention schedule
STAGE_CASES = [("tiny_fp32", 0, 0), ("l2k", 0, 0), ("l2k", 333, 2), ("l2k", 8269, 4)]


@pytest.mark.parametrize("name,L,B", STAGE_CASES)
def test_stage_route_and_dispatch(gqe, name, L, B):
    wl, I = inputs(name, L, B)
    log(f"[route+dispatch] {name} B={wl.batch} L={wl.seq_len}")
    F = f64_inputs(wl, I)
    r, p, idx, w = oracle.route(F["x"].reshape(-1, wl.d_model), F["wr"], F["br"], wl.n_groups,
                                wl.n_experts, wl.top_k)
    idx = idx.reshape(wl.batch, wl.seq_len, wl.n_groups, wl.top_k)
    counts, offsets, pos, slot = oracle.dispatch(idx, wl.n_experts)
    dev = device_inputs(wl, I)
    cfg = cfg_for(gqe, wl, dev["br"])
    ws = gqe.alloc_workspace(cfg)
    gqe.gqe_route(cfg, dev["x"], dev["wr"], ws)
    gqe.gqe_dispatch(cfg, ws)
    torch.cuda.synchronize()
    check_routing(gqe, cfg, ws, dict(idx=idx, w=w.reshape(idx.shape), counts=counts,
                                     offsets=offsets, pos=pos, slot=slot))


@pytest.mark.parametrize("pattern", ["uniform_ties", "one_expert_empty", "all_same", "random"])
@pytest.mark.parametrize("B,L", [(3, 1000), (2, 40000)])
def test_stage_dispatch_patterns(gqe, pattern, B, L):
    """Dispatch alone on seeded idx patterns: ties everywhere, an empty expert,
    every token picking the same pair, and random selections; a short batch
    (one block per (b, g)) and a long one (chunked count / scan / scatter)."""
    G, E, k = 4, 4, 2
    rng = np.random.default_rng(5)
    if pattern == "uniform_ties":
        idx = np.broadcast_to(np.arange(k), (B, L, G, k)).copy()
    elif pattern == "one_expert_empty":
        idx = np.stack([rng.permutation(3)[:k] for _ in range(B * L * G)]).reshape(B, L, G, k)
    elif pattern == "all_same":
        idx = np.broadcast_to(np.array([3, 1]), (B, L, G, k)).copy()
    else:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(B * L * G)]).reshape(B, L, G, k)
    idx = idx.astype(np.int32)
    log(f"[dispatch] pattern={pattern} B={B} L={L}")
    cfg = gqe.make_config(B, L, 64, G, E, k, 64)
    ws = gqe.alloc_workspace(cfg)
    v = gqe.workspace_views(cfg, ws)
    v["idx"].copy_(torch.from_numpy(idx))
    gqe.gqe_dispatch(cfg, ws)
    torch.cuda.synchronize()
    counts, offsets, pos, slot = oracle.dispatch(idx, E)
    assert np.array_equal(v["counts"].cpu().numpy(), counts)
    assert np.array_equal(v["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(v["pos"].cpu().numpy(), pos)
    assert np.array_equal(v["slot"].cpu().numpy(), slot)


@pytest.mark.parametrize("name,L,B", STAGE_CASES)
def test_stage_project(gqe, name, L, B):
    wl, I = inputs(name, L, B)
    log(f"[project] {name} B={wl.batch} L={wl.seq_len}")
    F = f64_inputs(wl, I)
    ref = oracle_gqe(wl, F)
    dev = device_inputs(wl, I)
    cfg = cfg_for(gqe, wl, dev["br"])
    ws = gqe.alloc_workspace(cfg)
    gqe.gqe_route(cfg, dev["x"], dev["wr"], ws)
    gqe.gqe_dispatch(cfg, ws)
    gqe.gqe_project(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], ws)
    torch.cuda.synchronize()
    v = gqe.workspace_views(cfg, ws)
    q = to_f64(v["q"]).transpose(0, 2, 1, 3)            # [B, L, kG+1, D]
    k = to_f64(v["k"])
    vt = vt_decode(to_f64(v["vt"]), wl.seq_len).transpose(0, 1, 3, 2)
    tol = 2.0 ** -8 if wl.dtype == W.BF16 else 1e-6
    for got, want, what in ((q, ref["q"], "q"), (k, ref["k_"], "k"),
                            (vt, ref["v"].transpose(0, 1, 3, 2), "vt")):
        err = np.abs(got - want)
        bound = tol * np.abs(want) + 1e-6 * np.abs(want).max()
        assert (err <= bound).all(), f"{what}: worst {err.max():.3e}"


@pytest.mark.parametrize("name,L,B", STAGE_CASES)
def test_stage_attention(gqe, name, L, B):
    """gqe_attention on oracle Q/K/V rounded to the storage type, against the
    oracle's attention of the same rounded values."""
    wl, I = inputs(name, L, B)
    log(f"[attention] {name} B={wl.batch} L={wl.seq_len}")
    F = f64_inputs(wl, I)
    ref = oracle_gqe(wl, F)
    cfg = cfg_for(gqe, wl)
    ws = gqe.alloc_workspace(cfg)
    v = gqe.workspace_views(cfg, ws)
    q_st = round_like(ref["q"].transpose(0, 2, 1, 3), wl.dtype)      # [B, H, L, D]
    k_st = round_like(ref["k_"], wl.dtype)
    v_st = round_like(ref["v"], wl.dtype)
    v["q"].copy_(to_dev(q_st, wl.dtype))
    v["k"].copy_(to_dev(k_st, wl.dtype))
    v["vt"].copy_(to_dev(vt_encode(v_st), wl.dtype))
    gqe.gqe_attention(cfg, ws)
    torch.cuda.synchronize()
    qf = W.to_f64(q_st, wl.dtype)
    kf, vf = W.to_f64(k_st, wl.dtype), W.to_f64(v_st, wl.dtype)
    H = wl.slot_heads
    s = to_f64(v["s"]).reshape(wl.batch, wl.seq_len, H + 1, wl.head_dim)
    t = np.arange(wl.seq_len)
    scale = 1.0 / math.sqrt(wl.head_dim)
    for b in range(wl.batch):
        for h in range(H):
            g = h // wl.top_k if h < H - 1 else 0
            want = oracle.causal_attention(qf[b, h], t, kf[b, g], vf[b, g], scale)
            output_gate(s[b, :, h], want, wl.dtype, f"attention b={b} h={h}")


# every attention schedule the launcher picks: short launches (key range split
# over wave groups) and long ones (B*L*heads >= 2^18), each head size and type
ATTN_PATH_CASES = [
    ("bf16", 32, 1, 2, 1, 700), ("bf16", 32, 1, 4, 2, 32768), ("bf16", 64, 2, 4, 2, 1500),
    ("bf16", 128, 1, 4, 2, 32768), ("fp32", 32, 1, 4, 2, 32768), ("fp32", 64, 1, 2, 1, 1000),
    ("fp32", 64, 1, 4, 2, 32768),
]


@pytest.mark.parametrize("dtype,D,B,G,k,L", ATTN_PATH_CASES)
def test_attention_paths(gqe, dtype, D, B, G, k, L):
    """gqe_attention on seeded random Q/K/V against the oracle's attention on
    the first 96 rows, the last row and 160 rows drawn at random."""
    log(f"[attention path] {dtype} D={D} B={B} G={G} k={k} L={L}")
    wl = W.Workload("attn", B, L, 128, G, k + 1, k, D, dtype, 1.0, 0.05)
    cfg = cfg_for(gqe, wl)
    ws = gqe.alloc_workspace(cfg)
    v = gqe.workspace_views(cfg, ws)
    H = wl.slot_heads
    rng = np.random.Generator(np.random.PCG64(11))
    q = round_like(rng.standard_normal((B, H, L, D)) * 2.0, dtype)
    kk = round_like(rng.standard_normal((B, G, L, D)), dtype)
    vv = round_like(rng.standard_normal((B, G, L, D)), dtype)
    v["q"].copy_(to_dev(q, dtype))
    v["k"].copy_(to_dev(kk, dtype))
    v["vt"].copy_(to_dev(vt_encode(vv), dtype))
    gqe.gqe_attention(cfg, ws)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(min(L, 96)), [L - 1],
                                     rng.choice(L, size=min(L, 160), replace=False)]))
    s = to_f64(v["s"][:, rows]).reshape(B, len(rows), H + 1, D)
    scale = 1.0 / math.sqrt(D)
    for b in range(B):
        for h in range(H):
            g = h // k if h < H - 1 else 0
            want = oracle.causal_attention(W.to_f64(q[b, h, rows], dtype), rows,
                                           W.to_f64(kk[b, g], dtype), W.to_f64(vv[b, g], dtype),
                                           scale)
            output_gate(s[b, :, h], want, dtype, f"attention b={b} h={h}")


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

LAYER_CASES = ["tiny_fp32", "l2k", "b4_l8k", "l128k", "l1m_zipf"]


@pytest.mark.parametrize("name", LAYER_CASES)
def test_gqe_forward(gqe, name):
    wl, I = inputs(name)
    rows = W.sample_rows(wl)
    log(f"[gqe_forward] {name} B={wl.batch} L={wl.seq_len} rows={len(rows)}")
    cfg, ws, out = run_gqe(gqe, wl, I)
    log("  gpu done; oracle ...")
    F = f64_inputs(wl, I)
    ref = oracle_gqe(wl, F, positions=None if wl.sample_rows == 0 else rows)
    check_routing(gqe, cfg, ws, ref)
    y = to_f64(out[:, rows])
    mx, mean, rel = output_gate(y, ref["y"], wl.dtype, f"{name} y")
    log(f"  y: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e}")
    assert rel <= (2e-2 if wl.dtype == W.BF16 else 1e-5)
    # slot vectors (hard, shared and weighted) too
    s = to_f64(gqe.workspace_views(cfg, ws)["s"][:, rows])
    output_gate(s, ref["s"], wl.dtype, f"{name} s")


@pytest.mark.parametrize("name", ["tiny_fp32", "l2k", "b4_l8k"])
def test_gqa_forward(gqe, name):
    wl, I = inputs(name)
    log(f"[gqa_forward] {name} B={wl.batch} L={wl.seq_len}")
    dev = device_inputs(wl, I)
    cfg = cfg_for(gqe, wl)
    ws = gqe.alloc_workspace(cfg, dense=True)
    out = torch.empty((wl.batch, wl.seq_len, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqa_forward(cfg, dev["x"], dev["wq_dense"].contiguous(), dev["wk"], dev["wv"],
                    dev["wo_dense"], out, ws)
    torch.cuda.synchronize()
    F = f64_inputs(wl, I)
    ref = oracle.gqa_forward(F["x"], F["wq_dense"], F["wk"], F["wv"], F["wo_dense"],
                             wl.n_groups, wl.n_experts, wl.head_dim)
    mx, mean, rel = output_gate(to_f64(out), ref["y"], wl.dtype, f"gqa {name}")
    log(f"  y: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e}")


def test_gqe_with_k_equal_e_matches_gqa_on_gpu(gqe):
    """k=E with a zero router (ties resolve in index order) and the shared and
    weighted W_O rows zeroed is dense GQA: both GPU paths must agree."""
    wl, I = inputs("l2k", 512)
    wl = wl.with_(top_k=wl.n_experts)
    G, E, D, d = wl.n_groups, wl.n_experts, wl.head_dim, wl.d_model
    J = dict(I)
    J["wr"] = np.zeros_like(I["wr"])
    wo = np.zeros((d, (E * G + 2) * D), dtype=np.uint16)
    wo[:, :G * E * D] = I["wo_dense"]
    J["wo"] = wo
    _, _, y_gqe = run_gqe(gqe, wl, J)
    dev = device_inputs(wl, J)
    cfg = cfg_for(gqe, wl)
    ws = gqe.alloc_workspace(cfg, dense=True)
    y_gqa = torch.empty_like(y_gqe)
    gqe.gqa_forward(cfg, dev["x"], dev["wq_dense"].contiguous(), dev["wk"], dev["wv"],
                    dev["wo_dense"], y_gqa, ws)
    torch.cuda.synchronize()
    output_gate(to_f64(y_gqe), to_f64(y_gqa), wl.dtype, "k=E vs gqa")


def test_determinism(gqe):
    wl, I = inputs("l2k")
    dev = device_inputs(wl, I)
    _, ws1, y1 = run_gqe(gqe, wl, I, dev)
    _, ws2, y2 = run_gqe(gqe, wl, I, dev)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    cfg = cfg_for(gqe, wl)
    v1, v2 = gqe.workspace_views(cfg, ws1), gqe.workspace_views(cfg, ws2)
    for key in ("idx", "w", "counts", "offsets", "pos", "slot", "q", "k", "s"):
        assert torch.equal(v1[key].view(torch.uint8), v2[key].view(torch.uint8)), key
    L = wl.seq_len
    assert np.array_equal(vt_decode(v1["vt"].view(torch.int16).cpu().numpy(), L),
                          vt_decode(v2["vt"].view(torch.int16).cpu().numpy(), L))


@pytest.mark.parametrize("name,L,B", [("tiny_fp32", 0, 0), ("l2k", 0, 0), ("l2k", 600, 2)])
@pytest.mark.parametrize("mode", ["hard", "weighted_concat"])
def test_ablation_output_modes(gqe, name, L, B, mode):
    """The two output constructions of the ablation: the k*G hard slots only,
    or each scaled by its in-group probability; no shared head, W_O of k*G*d_h
    inputs (its first k*G*d_h columns here).  Two sequences check that the
    attention steps through the query buffer, which keeps room for the shared
    head, by its own head count."""
    wl, I = inputs(name, L, B)
    log(f"[output mode] {name} {mode}")
    kG, D = wl.top_k * wl.n_groups, wl.head_dim
    J = dict(I)
    J["wo"] = np.ascontiguousarray(I["wo"][:, :kG * D])
    cfg, ws, out = run_gqe(gqe, wl, J, output_mode=mode)
    F = f64_inputs(wl, J)
    ref = oracle_gqe(wl, F, output_mode=mode)
    v = gqe.workspace_views(cfg, ws)
    assert np.array_equal(v["idx"].cpu().numpy(), ref["idx"])
    w_ref = ref["w"] if mode == "hard" else np.take_along_axis(
        ref["p"], ref["idx"].astype(np.int64), axis=-1)
    assert np.abs(v["w"].cpu().numpy().astype(np.float64) - w_ref).max() <= 2e-7
    assert v["s"].shape[-1] == kG * D
    output_gate(to_f64(v["s"]), ref["s"], wl.dtype, f"{name} {mode} s")
    mx, mean, rel = output_gate(to_f64(out), ref["y"], wl.dtype, f"{name} {mode} y")
    log(f"  y: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e}")


def test_forward_equals_stages_and_graph_replay(gqe):
    """gqe_forward gives the same bits as the five stage calls, and so does
    every replay of a HIP graph captured from it, with eager work and
    synchronizations between the replays."""
    wl, I = inputs("l2k")
    dev = device_inputs(wl, I)
    cfg, ws, y_fwd = run_gqe(gqe, wl, I, dev)
    ws2 = gqe.alloc_workspace(cfg)
    y_st = torch.empty_like(y_fwd)
    gqe.gqe_route(cfg, dev["x"], dev["wr"], ws2)
    gqe.gqe_dispatch(cfg, ws2)
    gqe.gqe_project(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], ws2)
    gqe.gqe_attention(cfg, ws2)
    gqe.gqe_output(cfg, dev["wo"], y_st, ws2)
    torch.cuda.synchronize()
    assert torch.equal(y_fwd.view(torch.int16), y_st.view(torch.int16))

    ws3 = gqe.alloc_workspace(cfg)
    y_g = torch.empty_like(y_fwd)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], y_g, ws3)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], y_g, ws3)
    for rep in range(3):
        y_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g.view(torch.int16), y_fwd.view(torch.int16)), f"replay {rep}"
        # eager work in between
        gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], y_st, ws2)
        torch.cuda.synchronize()
    del graph


def test_graph_capture_of_the_first_call():
    """A fresh process whose first gqe_forward calls are made under HIP graph
    capture (short and long launch forms: 2k, 8k x 4, 128k) replays them
    exactly (tests/graph_first_call.py)."""
    import os
    import subprocess
    import sys
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    here = os.path.dirname(os.path.abspath(__file__))
    log("[graph] first calls under capture in a child process: l2k b4_l8k l128k")
    res = subprocess.run([sys.executable, os.path.join(here, "graph_first_call.py"), "l2k", "b4_l8k",
                          "l128k"], capture_output=True, text=True, timeout=300)
    log(res.stdout[-2000:])
    assert res.returncode == 0 and "graph first call ok" in res.stdout, res.stderr[-3000:]


@pytest.mark.parametrize("L,B,G,E,k,D,dtype", [
    (1, 1, 4, 4, 2, 64, "bf16"),
    (65, 2, 4, 4, 2, 64, "bf16"),
    (200, 1, 2, 3, 3, 32, "fp32"),
    (130, 1, 1, 1, 1, 128, "bf16"),
    (97, 2, 3, 5, 2, 128, "fp32"),
    (300, 1, 8, 2, 1, 64, "bf16"),
])
def test_edge_shapes(gqe, L, B, G, E, k, D, dtype):
    """Ragged lengths, a single token, one group / one expert, k = E, every head size."""
    wl = W.Workload("edge", B, L, 128, G, E, k, D, dtype, 1.0, 0.05)
    log(f"[edge] {wl}")
    I = W.make_inputs(wl, seed=3, with_gqa=True)
    cfg, ws, out = run_gqe(gqe, wl, I)
    F = f64_inputs(wl, I)
    ref = oracle_gqe(wl, F)
    check_routing(gqe, cfg, ws, ref)
    output_gate(to_f64(out), ref["y"], wl.dtype, "edge y")


def test_shared_head_group_and_scale(gqe):
    """shared_kv_group and an explicit softmax scale are honoured."""
    wl, I = inputs("l2k", 256)
    cfg, ws, out = run_gqe(gqe, wl, I, shared_kv_group=2, softmax_scale=0.3)
    F = f64_inputs(wl, I)
    ref = oracle_gqe(wl, F, shared_kv_group=2, scale=0.3)
    output_gate(to_f64(out), ref["y"], wl.dtype, "shared group 2 / scale 0.3")


def test_empty_and_errors(gqe):
    wl, I = inputs("l2k", 64)
    dev = device_inputs(wl, I)
    cfg = gqe.make_config(1, 0, wl.d_model, 4, 4, 2, 64)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    out = torch.empty(0, device="cuda", dtype=torch.bfloat16)
    gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], out, ws)
    cfg = cfg_for(gqe, wl)
    small = torch.empty(gqe.gqe_workspace_bytes(cfg) - 256, dtype=torch.uint8, device="cuda")
    out = torch.empty((1, 64, wl.d_model), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gqe.GqeError, match="WORKSPACE"):
        gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], out,
                        small)
    with pytest.raises(gqe.GqeError, match="UNSUPPORTED"):
        gqe.gqe_workspace_layout(gqe.make_config(1, 64, wl.d_model, 4, 4, 2, 80))


# ---------------------------------------------------------------------------
# routing ties against the oracle
# ---------------------------------------------------------------------------

def _route_case(kind, rng):
    """Inputs whose routing hinges on exact ties or on a bias far below any
    rounding of the logits (the tie rule: lower expert index first)."""
    wl = W.WORKLOADS["l2k"].with_(seq_len=512)
    I = dict(W.make_inputs(wl, seed=7, with_gqa=True))
    G, E, d = wl.n_groups, wl.n_experts, wl.d_model
    if kind == "zero_router":            # every logit 0: experts 0 and 1 everywhere
        I["wr"] = np.zeros_like(I["wr"])
    elif kind == "duplicate_rows":       # experts 1 and 3 of every group share a router row
        wr = I["wr"].copy()
        for g in range(G):
            wr[g * E + 3] = wr[g * E + 1]
        I["wr"] = wr
    elif kind == "integer_ties":         # small integers: every sum exact, many exact ties
        x = rng.integers(1, 4, I["x"].shape).astype(np.float32)
        wr = rng.integers(-3, 1, I["wr"].shape).astype(np.float32)
        wr[0 * E + 1] = wr[0 * E + 3] = 2.0
        wr[1 * E + 0] = wr[1 * E + 2] = 1.0
        I["x"] = W.f32_to_bf16_bits(x)
        I["wr"] = W.f32_to_bf16_bits(wr)
    elif kind == "bias_decides":         # identical rows; a 2^-44 bias ranks expert 2 first
        wr = I["wr"].copy()
        for g in range(G):
            wr[g * E + 2] = wr[g * E + 1]
        I["wr"] = wr
        br = np.zeros(G * E, dtype=np.float32)
        br[[g * E + 2 for g in range(G)]] = np.float32(2.0 ** -44)
        I["br"] = br
    return wl, I


@pytest.mark.parametrize("kind", ["zero_router", "duplicate_rows", "integer_ties", "bias_decides"])
def test_routing_ties_match_oracle(gqe, kind):
    """idx (and w, and the dispatch lists) from gqe_route/gqe_dispatch equal
    the oracle's on inputs where the tie rule or a bias of 2^-44 decides."""
    rng = np.random.default_rng(31)
    wl, I = _route_case(kind, rng)
    log(f"[route ties] {kind}")
    F = f64_inputs(wl, I)
    r, p, idx, w = oracle.route(F["x"].reshape(-1, wl.d_model), F["wr"], F["br"], wl.n_groups,
                                wl.n_experts, wl.top_k)
    idx = idx.reshape(wl.batch, wl.seq_len, wl.n_groups, wl.top_k)
    counts, offsets, pos, slot = oracle.dispatch(idx, wl.n_experts)
    dev = device_inputs(wl, I)
    cfg = cfg_for(gqe, wl, dev["br"])
    ws = gqe.alloc_workspace(cfg)
    gqe.gqe_route(cfg, dev["x"], dev["wr"], ws)
    gqe.gqe_dispatch(cfg, ws)
    torch.cuda.synchronize()
    check_routing(gqe, cfg, ws, dict(idx=idx, w=w.reshape(idx.shape), counts=counts,
                                     offsets=offsets, pos=pos, slot=slot))
    if kind == "zero_router":
        assert (idx == np.arange(wl.top_k)).all()
    if kind == "bias_decides":   # expert 2 always beats its twin by 2^-44
        assert (idx[..., 0] != 1).all()


# ---------------------------------------------------------------------------
# negative controls: the gates reject plausible wrong answers
# ---------------------------------------------------------------------------

def test_gates_reject_wrong_layers(gqe):
    """The GPU layer passes the output gate against the oracle, and fails it
    against the oracle's slot vectors rearranged the way plausible mistakes
    would: the two hard slots of every group in index order instead of rank
    order, the weighted slot dropped, the shared and weighted slots swapped,
    and an all-zero output."""
    wl, I = inputs("l2k", 1024)
    cfg, ws, out = run_gqe(gqe, wl, I)
    F = f64_inputs(wl, I)
    ref = oracle_gqe(wl, F)
    y = to_f64(out)

    def layer_gate(got, want, what):   # the gate of test_gqe_forward
        _, _, rel = output_gate(got, want, wl.dtype, what)
        assert rel <= 2e-2, f"{what}: rel-L2 {rel:.3e}"

    layer_gate(y, ref["y"], "the layer")
    G, k, D = wl.n_groups, wl.top_k, wl.head_dim
    s = ref["s"]
    wrong = {}
    s1 = s.copy()                                   # index order within each group
    for g in range(G):
        swap = ref["idx"][..., g, 0] > ref["idx"][..., g, 1]
        a, b = (g * k) * D, (g * k + 1) * D
        s1[swap, a:a + D], s1[swap, b:b + D] = s[swap, b:b + D], s[swap, a:a + D]
    wrong["index-order slots"] = s1
    s2 = s.copy()
    s2[..., (k * G + 1) * D:] = 0.0
    wrong["no weighted slot"] = s2
    s3 = s.copy()
    s3[..., k * G * D:(k * G + 1) * D], s3[..., (k * G + 1) * D:] = (s[..., (k * G + 1) * D:],
                                                                     s[..., k * G * D:(k * G + 1) * D])
    wrong["shared and weighted swapped"] = s3
    for what, sw in wrong.items():
        y_wrong = oracle.output_projection(sw, F["wo"])
        with pytest.raises(AssertionError):
            layer_gate(y, y_wrong, what)
    with pytest.raises(AssertionError):
        layer_gate(np.zeros_like(y), ref["y"], "zero output")

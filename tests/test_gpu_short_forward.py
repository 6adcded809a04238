"""The short-sequence forward against the staged calls, bit for bit (needs an
MI355X).

bf16 layers of up to 4096 tokens run gqe_forward as one front launch (the
router beside a dense projection of every expert's query head), the attention
reading each slot-head's query row through the routing indices with the
dispatch's blocks in its grid, and W_O with the weighted slot formed in its
main loop.  Longer layers, and the stage entry points, run the route /
dispatch / gathered projection / attention / output sequence.
Both compute every value with the same arithmetic in the same order, so the
whole workspace (routing, lists, slot-major queries, K, V^T, slots, row
log-sum-exps) and the output must agree bit for bit; each is also held to the
oracle by the parity tests.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_util import inputs, log, to_dev, vt_decode  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gqe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_query_moe_amd import gqe as mod
    return mod


CASES = [  # (name, L, B, config keywords)
    ("l2k", 0, 0, {}),
    ("l2k", 600, 2, {}),
    ("l2k", 4096, 1, {}),
    ("l2k", 1000, 3, {"rope_base": 10000.0}),
    ("l2k", 777, 1, {"output_mode": "hard"}),
    ("l2k", 777, 1, {"output_mode": "weighted_concat"}),
    ("l2k", 513, 2, {"group_top_k": [1, 2, 3, 2]}),
]


def _bits(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


@pytest.mark.parametrize("name,L,B,kw", CASES)
def test_short_forward_equals_staged(gqe, name, L, B, kw):
    wl, I = inputs(name, L, B)
    log(f"[short forward] {name} B={wl.batch} L={wl.seq_len} {kw}")
    dev = {k: to_dev(v, wl.dtype) for k, v in I.items()}
    wo = dev["wo"]
    if kw.get("output_mode", "full") != "full":  # the ablation's W_O takes the hard slots only
        wo = wo[:, :wl.top_k * wl.n_groups * wl.head_dim].contiguous()
    gk = kw.get("group_top_k")
    cfg = gqe.make_config(wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts, wl.top_k,
                          wl.head_dim, dtype=wl.dtype, router_bias=dev["br"], **kw)
    assert gqe.uses_short_forward(cfg)
    shape = (wl.batch, wl.seq_len, wl.d_model)
    ws1, ws2 = gqe.alloc_workspace(cfg), gqe.alloc_workspace(cfg)
    y1 = torch.empty(shape, dtype=cfg.torch_dtype, device="cuda")
    y2 = torch.empty_like(y1)
    gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], wo, y1, ws1)
    gqe.gqe_route(cfg, dev["x"], dev["wr"], ws2)
    gqe.gqe_dispatch(cfg, ws2)
    gqe.gqe_project(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], ws2)
    gqe.gqe_attention(cfg, ws2)
    gqe.gqe_output(cfg, wo, y2, ws2)
    torch.cuda.synchronize()
    v1, v2 = gqe.workspace_views(cfg, ws1), gqe.workspace_views(cfg, ws2)
    # q keeps room for the shared head; the ablation outputs have none, and
    # that slot is never written
    H = (sum(gk) if gk else wl.top_k * wl.n_groups) + (kw.get("output_mode", "full") == "full")
    for key in ("idx", "w", "counts", "offsets", "pos", "slot", "q", "k", "s", "lse"):
        a, b = v1[key], v2[key]
        if key == "q":
            a, b = a[:, :H], b[:, :H]
        a, b = _bits(a), _bits(b)
        assert np.array_equal(a, b), f"{key}: {(a != b).sum()} bytes differ"
    L_ = wl.seq_len
    assert np.array_equal(vt_decode(v1["vt"].view(torch.int16).cpu().numpy(), L_),
                          vt_decode(v2["vt"].view(torch.int16).cpu().numpy(), L_))
    assert np.array_equal(_bits(y1), _bits(y2))
    if gk is None:
        assert int(v1["counts"].sum()) == wl.batch * wl.seq_len * wl.n_groups * wl.top_k



@pytest.mark.parametrize("name,L,B", [("l2k", 0, 0), ("l2k", 600, 2), ("b4_l8k", 0, 0)])
def test_output_forms_the_weighted_slot_in_its_main_loop(gqe, name, L, B):
    """bf16 layers with d_h 64 form the weighted slot inside the W_O GEMM: the
    slot it stores is sum_h w_h * s_h (float32 in slot order, rounded to bf16:
    within one bf16 step of the float64 sum), and the output is bit for bit
    the plain output GEMM (the dense baseline's, of the same width) over the
    slot vector as stored."""
    wl, I = inputs(name, L, B)
    log(f"[in-loop weighted slot] {name} B={wl.batch} L={wl.seq_len}")
    dev = {k: to_dev(v, wl.dtype) for k, v in I.items()}
    cfg = gqe.make_config(wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts, wl.top_k,
                          wl.head_dim, dtype=wl.dtype, router_bias=dev["br"])
    ws = gqe.alloc_workspace(cfg)
    shape = (wl.batch, wl.seq_len, wl.d_model)
    y = torch.empty(shape, dtype=cfg.torch_dtype, device="cuda")
    gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], y, ws)
    torch.cuda.synchronize()
    v = gqe.workspace_views(cfg, ws)
    kG, D = wl.top_k * wl.n_groups, wl.head_dim
    s = v["s"].double().cpu().numpy()
    hard = s[..., :kG * D].reshape(wl.batch, wl.seq_len, kG, D)
    w = v["w"].double().cpu().numpy().reshape(wl.batch, wl.seq_len, kG)
    ref = np.einsum("blh,blhd->bld", w, hard)
    got = s[..., (kG + 1) * D:]
    mag = np.einsum("blh,blhd->bld", np.abs(w), np.abs(hard))  # float32 sums' scale
    assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + kG * 2.0 ** -23 * mag).all()
    # the plain output GEMM over the same slot vector: a dense layout of width (kG+2)*d_h
    cfg_d = gqe.make_config(wl.batch, wl.seq_len, wl.d_model, 2, (kG + 2) // 2, 1, D,
                            dtype=wl.dtype)
    wsd = gqe.alloc_workspace(cfg_d, dense=True)
    gqe.workspace_views(cfg_d, wsd, dense=True)["s"].copy_(v["s"])
    y2 = torch.empty_like(y)
    gqe.gqa_output(cfg_d, dev["wo"], y2, wsd)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), _bits(y2))

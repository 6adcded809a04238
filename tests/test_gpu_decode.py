"""Decode step (one new token per sequence against a KV cache) on the GPU
against the oracle's decode step, through the C ABI (needs an MI355X).

Checked: the routing of the new tokens (bit for bit), the cache entries the
step writes (and that it writes no other), and the layer output, to the same
gates as prefill: max-abs 2e-2 and mean-abs 2e-3 for bf16, 1e-5 for fp32.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_util import f64_inputs, log, output_gate, to_dev, to_f64, vt_decode, vt_encode  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gqe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_query_moe_amd import gqe as mod
    return mod


def _cfg(gqe, wl, bias=None, **kw):
    return gqe.make_config(wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts, wl.top_k,
                           wl.head_dim, dtype=wl.dtype, router_bias=bias, **kw)


def _device(wl, I):
    dev = {k: to_dev(v, wl.dtype) for k, v in I.items()
           if k not in ("k_cache", "v_cache", "pos")}
    dev["k_cache"] = to_dev(I["k_cache"], wl.dtype)
    dev["vt_cache"] = to_dev(vt_encode(I["v_cache"]), wl.dtype)
    dev["pos"] = torch.from_numpy(I["pos"].astype(np.int32)).cuda()
    return dev


def _run(gqe, wl, dev, dense=False, **kw):
    cfg = _cfg(gqe, wl, None if dense else dev["br"], **kw)
    ws = gqe.alloc_decode_workspace(cfg, dense=dense)
    out = torch.empty((wl.batch, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    if dense:
        gqe.gqa_decode(cfg, dev["x"], dev["wq_dense"], dev["wk"], dev["wv"], dev["wo_dense"],
                       dev["k_cache"], dev["vt_cache"], dev["pos"], out, ws)
    else:
        gqe.gqe_decode(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"],
                       dev["k_cache"], dev["vt_cache"], dev["pos"], out, ws)
    torch.cuda.synchronize()
    return cfg, ws, out


def _oracle(wl, I, F, dense=False, **kw):
    kc, vc = W.to_f64(I["k_cache"], wl.dtype), W.to_f64(I["v_cache"], wl.dtype)
    if dense:
        return oracle.gqa_decode_step(F["x"], kc, vc, I["pos"], F["wq_dense"], F["wk"], F["wv"],
                                      F["wo_dense"], wl.n_groups, wl.n_experts, wl.head_dim)
    return oracle.gqe_decode_step(F["x"], kc, vc, I["pos"], F["wq"], F["wk"], F["wv"], F["wr"],
                                  F["wo"], F["br"], wl.n_groups, wl.n_experts, wl.top_k,
                                  wl.head_dim, **kw)


def _check_caches(wl, I, dev, ref, what):
    """The step writes K and V of the new token at pos[b] and nothing else."""
    B, Lc = wl.batch, wl.seq_len
    kc = to_f64(dev["k_cache"])
    vc = vt_decode(to_f64(dev["vt_cache"]), Lc)
    k0, v0 = W.to_f64(I["k_cache"], wl.dtype), W.to_f64(I["v_cache"], wl.dtype)
    mask = np.ones((B, Lc), dtype=bool)
    for b in range(B):
        t = int(I["pos"][b])
        if 0 <= t < Lc:
            mask[b, t] = False
    assert np.array_equal(kc.transpose(0, 2, 1, 3)[mask], k0.transpose(0, 2, 1, 3)[mask]), \
        f"{what}: key cache written outside pos"
    assert np.array_equal(vc.transpose(0, 2, 1, 3)[mask], v0.transpose(0, 2, 1, 3)[mask]), \
        f"{what}: value cache written outside pos"
    b_idx = np.arange(B)
    t = I["pos"].astype(np.int64)
    output_gate(kc[b_idx, :, t], ref["k_new"], wl.dtype, f"{what} k_new")
    output_gate(vc[b_idx, :, t], ref["v_new"], wl.dtype, f"{what} v_new")


DECODE_CASES = [
    # name, overrides, output mode
    ("dec_tiny_fp32", {}, "full"),
    ("dec_tiny_fp32", {}, "hard"),
    ("dec_tiny_fp32", dict(batch=2, seq_len=64), "full"),           # one tile, one chunk
    ("dec_tiny_fp32", dict(batch=1, seq_len=1), "full"),            # a one-entry cache
    ("dec_tiny_fp32", dict(head_dim=128, n_experts=3, top_k=3, seq_len=333), "full"),  # k = E
    ("dec_b64_c8k", dict(batch=5, seq_len=1000), "full"),           # ragged cache
    ("dec_b64_c8k", dict(batch=5, seq_len=1000), "weighted_concat"),
    ("dec_b64_c8k", dict(batch=3, seq_len=700, n_groups=2, n_experts=16, top_k=16,
                         head_dim=32), "full"),                     # 17 heads on group 0
    ("dec_b64_c8k", {}, "full"),                                    # the benchmark shape
]


@pytest.mark.parametrize("name,over,mode", DECODE_CASES)
def test_gqe_decode(gqe, name, over, mode):
    wl = W.DECODE_WORKLOADS[name].with_(**over)
    log(f"[decode] {wl} {mode}")
    I = W.make_decode_inputs(wl, seed=5, with_gqa=True)
    if mode != "full":
        kG = wl.top_k * wl.n_groups * wl.head_dim
        I["wo"] = np.ascontiguousarray(I["wo"][:, :kG])
    dev = _device(wl, I)
    cfg, ws, out = _run(gqe, wl, dev, output_mode=mode)
    F = f64_inputs(wl, I)
    ref = _oracle(wl, I, F, output_mode=mode)
    # routing of the new tokens, at the front of the workspace
    n = wl.batch * wl.n_groups * wl.top_k
    idx = ws[:4 * n].view(torch.int32).cpu().numpy().reshape(ref["idx"].shape)
    assert np.array_equal(idx, ref["idx"]), f"idx mismatches: {(idx != ref['idx']).sum()}"
    _check_caches(wl, I, dev, ref, name)
    mx, mean, rel = output_gate(to_f64(out), ref["y"], wl.dtype, f"{name} {mode} y")
    log(f"  y: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e}")


@pytest.mark.parametrize("name,over", [
    ("dec_tiny_fp32", {}),
    ("dec_b64_c8k", dict(batch=3, seq_len=700, n_groups=2, n_experts=32, head_dim=32)),  # 32 heads
    ("dec_b64_c8k", {}),
])
def test_gqa_decode(gqe, name, over):
    wl = W.DECODE_WORKLOADS[name].with_(**over)
    log(f"[gqa decode] {wl}")
    I = W.make_decode_inputs(wl, seed=6, with_gqa=True)
    dev = _device(wl, I)
    cfg, ws, out = _run(gqe, wl, dev, dense=True)
    F = f64_inputs(wl, I)
    ref = _oracle(wl, I, F, dense=True)
    _check_caches(wl, I, dev, ref, name)
    output_gate(to_f64(out), ref["y"], wl.dtype, f"{name} gqa y")


def test_decode_two_steps_read_what_the_first_wrote(gqe):
    """Step 2 at pos + 1 attends to the key and value that step 1 wrote."""
    wl = W.DECODE_WORKLOADS["dec_b64_c8k"].with_(batch=4, seq_len=300)
    I = W.make_decode_inputs(wl, seed=7, with_gqa=True)
    I["pos"] = np.array([0, 63, 64, 298], dtype=np.int32)
    dev = _device(wl, I)
    cfg, ws, out1 = _run(gqe, wl, dev)
    F = f64_inputs(wl, I)
    ref1 = _oracle(wl, I, F)
    rng = np.random.Generator(np.random.PCG64(11))
    x2 = W._draw(rng, (wl.batch, wl.d_model), wl.x_std, wl.dtype)
    dev["x"] = to_dev(x2, wl.dtype)
    dev["pos"] += 1
    out2 = torch.empty_like(out1)
    gqe.gqe_decode(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"],
                   dev["k_cache"], dev["vt_cache"], dev["pos"], out2, ws)
    torch.cuda.synchronize()
    F2 = dict(F, x=W.bf16_bits_to_f32(x2))
    ref2 = oracle.gqe_decode_step(F2["x"], ref1["k_cache"], ref1["v_cache"], I["pos"] + 1,
                                  F["wq"], F["wk"], F["wv"], F["wr"], F["wo"], F["br"],
                                  wl.n_groups, wl.n_experts, wl.top_k, wl.head_dim)
    output_gate(to_f64(out1), ref1["y"], wl.dtype, "step 1 y")
    output_gate(to_f64(out2), ref2["y"], wl.dtype, "step 2 y")


def test_decode_position_outside_the_cache(gqe):
    """pos outside [0, Lc): no cache entry changes and the heads give zero."""
    wl = W.DECODE_WORKLOADS["dec_tiny_fp32"].with_(batch=3)
    I = W.make_decode_inputs(wl, seed=8, with_gqa=True)
    I["pos"] = np.array([-1, wl.seq_len, 5], dtype=np.int32)
    dev = _device(wl, I)
    kc0, vt0 = dev["k_cache"].clone(), dev["vt_cache"].clone()
    cfg, ws, out = _run(gqe, wl, dev)
    assert torch.equal(out[:2], torch.zeros_like(out[:2]))
    assert torch.equal(dev["k_cache"][:2], kc0[:2]) and torch.equal(dev["vt_cache"][:2], vt0[:2])
    F = f64_inputs(wl, I)
    one = dict(I, x=I["x"][2:], k_cache=I["k_cache"][2:], v_cache=I["v_cache"][2:],
               pos=I["pos"][2:])
    ref = _oracle(wl.with_(batch=1), one, dict(F, x=F["x"][2:]))
    output_gate(to_f64(out[2:]), ref["y"], wl.dtype, "in-range sequence y")


def test_decode_graph_replay(gqe):
    """A HIP graph of one decode step, replayed with the positions advanced
    between replays (eager work in between), matches eager calls bit for bit."""
    wl = W.DECODE_WORKLOADS["dec_b64_c8k"].with_(batch=4, seq_len=512)
    I = W.make_decode_inputs(wl, seed=9, with_gqa=True)
    I["pos"] = np.array([10, 100, 300, 500], dtype=np.int32)
    dev = _device(wl, I)
    cfg = _cfg(gqe, wl, dev["br"])
    ws_e, ws_g = gqe.alloc_decode_workspace(cfg), gqe.alloc_decode_workspace(cfg)
    kc_e, vt_e = dev["k_cache"].clone(), dev["vt_cache"].clone()
    kc_g, vt_g = dev["k_cache"].clone(), dev["vt_cache"].clone()
    pos_e, pos_g = dev["pos"].clone(), dev["pos"].clone()
    out_e = torch.empty((wl.batch, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    out_g = torch.empty_like(out_e)

    def step(kc, vt, pos, out, ws):
        gqe.gqe_decode(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"],
                       kc, vt, pos, out, ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step(kc_g, vt_g, pos_g, out_g, ws_g)
    for rep in range(3):
        out_g.zero_()
        graph.replay()
        step(kc_e, vt_e, pos_e, out_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), f"replay {rep}"
        assert torch.equal(kc_g.view(torch.int16), kc_e.view(torch.int16))
        assert torch.equal(vt_g.view(torch.int16), vt_e.view(torch.int16))
        pos_g += 1
        pos_e += 1
    del graph


GROUP_K_DECODE_CASES = [
    # name, overrides, per-group counts, output mode
    ("dec_tiny_fp32", dict(n_groups=3, n_experts=3, batch=3), [1, 3, 2], "full"),
    ("dec_tiny_fp32", dict(n_groups=3, n_experts=3, batch=3), [2, 1, 3], "hard"),
    ("dec_tiny_fp32", dict(n_groups=3, n_experts=3, batch=3), [3, 2, 1], "weighted_concat"),
    ("dec_b64_c8k", dict(batch=6, seq_len=1000), [1, 2, 3, 2], "full"),
    ("dec_b64_c8k", dict(batch=4, seq_len=700, n_experts=8), [6, 1, 1, 2], "full"),  # 7 heads on group 0
]


@pytest.mark.parametrize("name,over,ks,mode", GROUP_K_DECODE_CASES)
def test_gqe_decode_group_k(gqe, name, over, ks, mode):
    """Per-group expert counts in decode: routing bit for bit, caches, output."""
    wl = W.DECODE_WORKLOADS[name].with_(**over)
    K = sum(ks)
    log(f"[decode group k] {wl} ks={ks} {mode}")
    I = W.make_decode_inputs(wl.with_(top_k=max(ks)), seed=9, with_gqa=True)
    rng = np.random.Generator(np.random.PCG64(10))
    width = (K + (2 if mode == "full" else 0)) * wl.head_dim
    I["wo"] = W._draw(rng, (wl.d_model, width), wl.w_std, wl.dtype)
    dev = _device(wl, I)
    cfg, ws, out = _run(gqe, wl.with_(top_k=max(ks)), dev, output_mode=mode, group_top_k=ks)
    F = f64_inputs(wl, I)
    kc, vc = W.to_f64(I["k_cache"], wl.dtype), W.to_f64(I["v_cache"], wl.dtype)
    ref = oracle.gqe_decode_step_group_k(F["x"], kc, vc, I["pos"], F["wq"], F["wk"], F["wv"],
                                         F["wr"], F["wo"], F["br"], wl.n_groups, wl.n_experts, ks,
                                         wl.head_dim, output_mode=mode)
    idx = ws[:4 * wl.batch * K].view(torch.int32).cpu().numpy().reshape(ref["idx"].shape)
    assert np.array_equal(idx, ref["idx"]), f"idx mismatches: {(idx != ref['idx']).sum()}"
    _check_caches(wl, I, dev, ref, name)
    mx, mean, rel = output_gate(to_f64(out), ref["y"], wl.dtype, f"{name} {ks} {mode} y")
    log(f"  y: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e}")

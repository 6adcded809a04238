"""The rotary position embedding option (rope_base > 0) on the GPU against the
oracle, through the C ABI (needs an MI355X): prefill (GQE and GQA), decode
(GQE and GQA) and backward (GQE and GQA).

Queries and keys are turned by position after their projections (RoFormer,
section 3.4.2, interleaved pairs of dimensions); values are not.  The gates
are those of the layers without it: routing bit for bit, outputs max-abs
2e-2 / mean-abs 2e-3 for bf16 and 1e-5 for float32, gradients to the
per-tensor gates of the backward tests (gpu_util's BF16_GRAD_GATE) or rel-L2
1e-5 (float32).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_util import (f64_inputs, grad_gate, inputs, log, output_gate, to_dev, to_f64,  # noqa: E402
                      vt_decode, vt_encode)

pytestmark = pytest.mark.gpu

BASE = 10000.0


@pytest.fixture(scope="module")
def gqe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_query_moe_amd import gqe as mod
    return mod


def _cfg(gqe, wl, bias=None, **kw):
    return gqe.make_config(wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts, wl.top_k,
                           wl.head_dim, dtype=wl.dtype, router_bias=bias, **kw)


def _dev(wl, I):
    return {k: to_dev(v, wl.dtype) for k, v in I.items()}


def _zeros(*shape):
    return torch.zeros(shape, dtype=torch.float32, device="cuda")


# name, L override, B override; the last is ragged (L not a tile multiple)
FWD_CASES = [("tiny_fp32", 0, 0), ("l2k", 0, 0), ("l2k", 333, 2)]


@pytest.mark.parametrize("name,L,B", FWD_CASES)
def test_gqe_forward_rope(gqe, name, L, B):
    wl, I = inputs(name, L, B)
    log(f"[rope gqe_forward] {name} B={wl.batch} L={wl.seq_len}")
    dev = _dev(wl, I)
    cfg = _cfg(gqe, wl, dev["br"], rope_base=BASE)
    ws = gqe.alloc_workspace(cfg)
    out = torch.empty((wl.batch, wl.seq_len, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], out, ws)
    torch.cuda.synchronize()
    F = f64_inputs(wl, I)
    ref = oracle.gqe_forward(F["x"], F["wq"], F["wk"], F["wv"], F["wr"], F["wo"], F["br"],
                             wl.n_groups, wl.n_experts, wl.top_k, wl.head_dim, rope_base=BASE)
    v = gqe.workspace_views(cfg, ws)
    assert np.array_equal(v["idx"].cpu().numpy(), ref["idx"])
    # the keys the attention reads are the turned ones
    output_gate(to_f64(v["k"]), ref["k_"], wl.dtype, f"{name} rotated K")
    mx, mean, rel = output_gate(to_f64(out), ref["y"], wl.dtype, f"{name} rope y")
    log(f"  y: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e}")
    output_gate(to_f64(v["s"]), ref["s"], wl.dtype, f"{name} rope s")
    # negative control: the same layer without the rotation is far from it
    plain = oracle.gqe_forward(F["x"], F["wq"], F["wk"], F["wv"], F["wr"], F["wo"], F["br"],
                               wl.n_groups, wl.n_experts, wl.top_k, wl.head_dim)
    assert np.abs(to_f64(out) - plain["y"]).max() > 10 * max(mx, 1e-6)


@pytest.mark.parametrize("name", ["tiny_fp32", "l2k"])
def test_gqa_forward_rope(gqe, name):
    wl, I = inputs(name)
    log(f"[rope gqa_forward] {name}")
    dev = _dev(wl, I)
    cfg = _cfg(gqe, wl, rope_base=BASE)
    ws = gqe.alloc_workspace(cfg, dense=True)
    out = torch.empty((wl.batch, wl.seq_len, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqa_forward(cfg, dev["x"], dev["wq_dense"].contiguous(), dev["wk"], dev["wv"],
                    dev["wo_dense"], out, ws)
    torch.cuda.synchronize()
    F = f64_inputs(wl, I)
    ref = oracle.gqa_forward(F["x"], F["wq_dense"], F["wk"], F["wv"], F["wo_dense"],
                             wl.n_groups, wl.n_experts, wl.head_dim, rope_base=BASE)
    mx, mean, rel = output_gate(to_f64(out), ref["y"], wl.dtype, f"gqa {name} rope y")
    log(f"  y: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e}")


DECODE_CASES = [
    ("dec_tiny_fp32", {}),
    ("dec_b64_c8k", dict(batch=5, seq_len=1000)),
    ("dec_b64_c8k", {}),
]


def _decode_dev(wl, I):
    dev = {k: to_dev(v, wl.dtype) for k, v in I.items() if k not in ("k_cache", "v_cache", "pos")}
    dev["k_cache"] = to_dev(I["k_cache"], wl.dtype)
    dev["vt_cache"] = to_dev(vt_encode(I["v_cache"]), wl.dtype)
    dev["pos"] = torch.from_numpy(I["pos"].astype(np.int32)).cuda()
    return dev


@pytest.mark.parametrize("name,over", DECODE_CASES)
@pytest.mark.parametrize("dense", [False, True])
def test_decode_rope(gqe, name, over, dense):
    wl = W.DECODE_WORKLOADS[name].with_(**over)
    log(f"[rope decode] {wl} dense={dense}")
    I = W.make_decode_inputs(wl, seed=21, with_gqa=True)
    dev = _decode_dev(wl, I)
    cfg = _cfg(gqe, wl, None if dense else dev["br"], rope_base=BASE)
    ws = gqe.alloc_decode_workspace(cfg, dense=dense)
    out = torch.empty((wl.batch, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    if dense:
        gqe.gqa_decode(cfg, dev["x"], dev["wq_dense"], dev["wk"], dev["wv"], dev["wo_dense"],
                       dev["k_cache"], dev["vt_cache"], dev["pos"], out, ws)
    else:
        gqe.gqe_decode(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"],
                       dev["k_cache"], dev["vt_cache"], dev["pos"], out, ws)
    torch.cuda.synchronize()
    F = f64_inputs(wl, I)
    kc, vc = W.to_f64(I["k_cache"], wl.dtype), W.to_f64(I["v_cache"], wl.dtype)
    if dense:
        ref = oracle.gqa_decode_step(F["x"], kc, vc, I["pos"], F["wq_dense"], F["wk"], F["wv"],
                                     F["wo_dense"], wl.n_groups, wl.n_experts, wl.head_dim,
                                     rope_base=BASE)
    else:
        ref = oracle.gqe_decode_step(F["x"], kc, vc, I["pos"], F["wq"], F["wk"], F["wv"],
                                     F["wr"], F["wo"], F["br"], wl.n_groups, wl.n_experts,
                                     wl.top_k, wl.head_dim, rope_base=BASE)
    # the key written into the cache is the turned one
    b = np.arange(wl.batch)
    t = I["pos"].astype(np.int64)
    kc_gpu = to_f64(dev["k_cache"])
    output_gate(kc_gpu[b, :, t], ref["k_new"], wl.dtype, f"{name} rope k_new")
    mx, mean, rel = output_gate(to_f64(out), ref["y"], wl.dtype, f"{name} rope decode y")
    log(f"  y: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e}")


def test_prefill_then_decode_rope(gqe):
    """The caches a rotated prefill leaves, extended by one rotated decode step
    at position L, give the prefill's answer for a sequence of L + 1 tokens."""
    wl, I = inputs("tiny_fp32")
    L = wl.seq_len
    full = wl.with_(seq_len=L + 1)
    rng = np.random.Generator(np.random.PCG64(31))
    x_last = W._draw(rng, (wl.batch, 1, wl.d_model), wl.x_std, wl.dtype)
    J = dict(I, x=np.concatenate([I["x"], x_last], axis=1))
    F = f64_inputs(full, J)
    ref = oracle.gqe_forward(F["x"], F["wq"], F["wk"], F["wv"], F["wr"], F["wo"], F["br"],
                             wl.n_groups, wl.n_experts, wl.top_k, wl.head_dim, rope_base=BASE,
                             positions=[L])
    dev = _dev(full, J)
    # prefill over the first L tokens, on a cache of L + 1 entries
    cfg = _cfg(gqe, wl, dev["br"], rope_base=BASE)
    ws = gqe.alloc_workspace(cfg)
    y = torch.empty((wl.batch, L, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    x0 = dev["x"][:, :L].contiguous()
    gqe.gqe_forward(cfg, x0, dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], y, ws)
    v = gqe.workspace_views(cfg, ws)
    torch.cuda.synchronize()
    B, G, D = wl.batch, wl.n_groups, wl.head_dim
    kc_np = np.zeros((B, G, L + 1, D))
    vc_np = np.zeros((B, G, L + 1, D))
    kc_np[:, :, :L] = to_f64(v["k"])                      # turned keys of the prefill
    vc_np[:, :, :L] = vt_decode(to_f64(v["vt"]), L)
    kc = torch.from_numpy(kc_np).to("cuda", cfg.torch_dtype)
    vt_cache = torch.from_numpy(vt_encode(vc_np)).to("cuda", cfg.torch_dtype)
    dcfg = _cfg(gqe, full, dev["br"], rope_base=BASE)
    dws = gqe.alloc_decode_workspace(dcfg)
    pos = torch.full((wl.batch,), L, dtype=torch.int32, device="cuda")
    out = torch.empty((wl.batch, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqe_decode(dcfg, dev["x"][:, L].contiguous(), dev["wq"], dev["wk"], dev["wv"], dev["wr"],
                   dev["wo"], kc, vt_cache, pos, out, dws)
    torch.cuda.synchronize()
    output_gate(to_f64(out), ref["y"][:, 0], wl.dtype, "decode at L after rotated prefill")


BWD_CASES = [("tiny_fp32", "full", 0.0), ("tiny_fp32", "weighted_concat", 0.3), ("l2k", "full", 0.01)]


@pytest.mark.parametrize("name,mode,aux", BWD_CASES)
def test_gqe_backward_rope(gqe, name, mode, aux):
    wl, I = inputs(name)
    log(f"[rope backward] {name} {mode} aux={aux}")
    J = dict(I)
    if mode != "full":
        J["wo"] = np.ascontiguousarray(I["wo"][:, :wl.top_k * wl.n_groups * wl.head_dim])
    dev = _dev(wl, J)
    cfg = _cfg(gqe, wl, dev["br"], output_mode=mode, rope_base=BASE)
    fws = gqe.alloc_workspace(cfg)
    y = torch.empty((wl.batch, wl.seq_len, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], y, fws)
    rng = np.random.Generator(np.random.PCG64(41))
    dy = W._draw(rng, (wl.batch, wl.seq_len, wl.d_model), 1.0, wl.dtype)
    G, E, d = wl.n_groups, wl.n_experts, wl.d_model
    g = dict(dx=_zeros(wl.batch, wl.seq_len, d), dwq=_zeros(*J["wq"].shape),
             dwk=_zeros(*J["wk"].shape), dwv=_zeros(*J["wv"].shape), dwr=_zeros(G * E, d),
             dbr=_zeros(G * E), dwo=_zeros(*J["wo"].shape), aux=_zeros(1))
    ws = gqe.alloc_backward_workspace(cfg)
    gqe.gqe_backward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"],
                     to_dev(dy, wl.dtype), aux, fws, g["dx"], g["dwq"], g["dwk"], g["dwv"],
                     g["dwr"], g["dbr"], g["dwo"], g["aux"], ws)
    torch.cuda.synchronize()
    F = f64_inputs(wl, J)
    ref = oracle.gqe_backward(F["x"], F["wq"], F["wk"], F["wv"], F["wr"], F["wo"], F["br"],
                              W.to_f64(dy, wl.dtype), G, E, wl.top_k, wl.head_dim,
                              output_mode=mode, aux_weight=aux, rope_base=BASE)
    for key in ("dwo", "dx", "dwq", "dwk", "dwv", "dwr", "dbr"):
        grad_gate(g[key].cpu().numpy(), ref[key], wl.dtype, f"{name} {mode} {key}", key)


@pytest.mark.parametrize("name", ["tiny_fp32", "l2k"])
def test_gqa_backward_rope(gqe, name):
    wl, I = inputs(name)
    log(f"[rope gqa backward] {name}")
    dev = _dev(wl, I)
    cfg = _cfg(gqe, wl, rope_base=BASE)
    fws = gqe.alloc_workspace(cfg, dense=True)
    y = torch.empty((wl.batch, wl.seq_len, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqa_forward(cfg, dev["x"], dev["wq_dense"], dev["wk"], dev["wv"], dev["wo_dense"], y, fws)
    rng = np.random.Generator(np.random.PCG64(43))
    dy = W._draw(rng, (wl.batch, wl.seq_len, wl.d_model), 1.0, wl.dtype)
    g = dict(dx=_zeros(wl.batch, wl.seq_len, wl.d_model), dwq=_zeros(*I["wq_dense"].shape),
             dwk=_zeros(*I["wk"].shape), dwv=_zeros(*I["wv"].shape),
             dwo=_zeros(*I["wo_dense"].shape))
    ws = gqe.alloc_backward_workspace(cfg, dense=True)
    gqe.gqa_backward(cfg, dev["x"], dev["wq_dense"], dev["wk"], dev["wv"], dev["wo_dense"],
                     to_dev(dy, wl.dtype), fws, g["dx"], g["dwq"], g["dwk"], g["dwv"], g["dwo"], ws)
    torch.cuda.synchronize()
    F = f64_inputs(wl, I)
    ref = oracle.gqa_backward(F["x"], F["wq_dense"], F["wk"], F["wv"], F["wo_dense"],
                              W.to_f64(dy, wl.dtype), wl.n_groups, wl.n_experts, wl.head_dim,
                              rope_base=BASE)
    for key in ("dwo", "dx", "dwq", "dwk", "dwv"):
        grad_gate(g[key].cpu().numpy(), ref[key], wl.dtype, f"gqa {name} {key}", key)


def test_rope_rejections(gqe):
    wl, _ = inputs("l2k", 64)
    with pytest.raises(gqe.GqeError, match="INVALID"):
        gqe.gqe_workspace_layout(_cfg(gqe, wl, rope_base=-1.0))
    with pytest.raises(gqe.GqeError, match="UNSUPPORTED"):
        gqe.gqe_workspace_layout(_cfg(gqe, wl, rope_base=BASE, group_top_k=[2, 1, 2, 2]))

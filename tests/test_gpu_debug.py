"""The index-checked debug build (libgqe_debug.so) on the GPU, through the C ABI
(needs an MI355X).

On valid inputs it must give exactly the release library's results: the
checks only observe.  On a workspace whose routing or dispatch lists were
changed from the host between stages, it must catch each planted index
(GQE_ERR_DEBUG) and skip every access that index would have guarded, so the
kernels finish normally.  Only the debug library is handed such lists: in it
every position, slot and list extent the gathered projection takes from the
lists, and every expert id the dispatch and the backward take from the
routing, is checked before it forms an address.
"""
import contextlib
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import workloads as W  # noqa: E402
from gpu_util import log, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu

_LIBS = {}


@pytest.fixture(scope="module")
def gqe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_query_moe_amd import build
    from sparse_query_moe_amd import gqe as mod
    if not os.path.exists(build.DEBUG_LIB):
        pytest.fail(f"{build.DEBUG_LIB} is not built (python -m sparse_query_moe_amd.build --debug)")
    _LIBS["release"] = mod._lib
    _LIBS["debug"] = mod.load_library(build.DEBUG_LIB)
    return mod


@contextlib.contextmanager
def library(gqe, which):
    saved = gqe._lib
    gqe._lib = _LIBS[which]
    try:
        yield
    finally:
        gqe._lib = saved


def _setup(gqe, wl):
    I = W.make_inputs(wl)
    dev = {k: to_dev(v, wl.dtype) for k, v in I.items()}
    cfg = gqe.make_config(wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts, wl.top_k,
                          wl.head_dim, dtype=wl.dtype, router_bias=dev["br"])
    return I, dev, cfg


def _forward(gqe, wl, dev, cfg):
    ws = gqe.alloc_workspace(cfg)
    out = torch.empty((wl.batch, wl.seq_len, wl.d_model), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], out, ws)
    torch.cuda.synchronize()
    return out, ws


def _backward(gqe, wl, I, dev, cfg, fws, dy):
    G, E, d = wl.n_groups, wl.n_experts, wl.d_model
    z = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda")  # noqa: E731
    g = dict(dx=z(wl.batch, wl.seq_len, d), dwq=z(*I["wq"].shape), dwk=z(*I["wk"].shape),
             dwv=z(*I["wv"].shape), dwr=z(G * E, d), dbr=z(G * E), dwo=z(*I["wo"].shape), aux=z(1))
    ws = gqe.alloc_backward_workspace(cfg)
    gqe.gqe_backward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], dy, 0.05,
                     fws, g["dx"], g["dwq"], g["dwk"], g["dwv"], g["dwr"], g["dbr"], g["dwo"],
                     g["aux"], ws)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", ["tiny_fp32", "l2k"])
def test_debug_build_matches_release(gqe, name):
    wl = W.WORKLOADS[name]
    log(f"[debug] {name}: release vs debug forward and backward")
    I, dev, cfg = _setup(gqe, wl)
    dy = torch.randn((wl.batch, wl.seq_len, wl.d_model), generator=torch.Generator().manual_seed(3))
    dy = dy.to(cfg.torch_dtype).to("cuda")
    res = {}
    for which in ("release", "debug"):
        with library(gqe, which):
            out, ws = _forward(gqe, wl, dev, cfg)
            v = gqe.workspace_views(cfg, ws)
            grads = _backward(gqe, wl, I, dev, cfg, ws, dy)
            res[which] = (out, {k: v[k].clone() for k in ("idx", "counts", "offsets", "pos", "slot", "q", "s")},
                          grads)
    (o_r, v_r, g_r), (o_d, v_d, g_d) = res["release"], res["debug"]
    assert torch.equal(o_r, o_d)
    for k in v_r:
        assert torch.equal(v_r[k], v_d[k]), k
    for k in g_r:
        assert torch.equal(g_r[k], g_d[k]), k


def _expect_debug_error(gqe, fn, what):
    with pytest.raises(gqe.GqeError, match="GQE_ERR_DEBUG"):
        fn()
    torch.cuda.synchronize()
    log(f"  caught: {what}")


def test_debug_build_catches_planted_list_indices(gqe):
    """Positions, slots, counts and offsets planted in the dispatch lists
    before the projection; expert ids planted in the routing before the
    dispatch."""
    wl = W.Workload("debug_lists", 1, 300, 256, 2, 4, 2, 64, W.BF16, 1.0, 0.02)
    L = wl.seq_len
    log(f"[debug] planted indices: B1 L{L} d256 G2 E4 k2 d_h64 bf16")
    I, dev, cfg = _setup(gqe, wl)
    ws = gqe.alloc_workspace(cfg)
    with library(gqe, "release"):
        gqe.gqe_route(cfg, dev["x"], dev["wr"], ws)
        gqe.gqe_dispatch(cfg, ws)
        gqe.gqe_project(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], ws)
        torch.cuda.synchronize()
    v = gqe.workspace_views(cfg, ws)
    q_release = v["q"].clone()
    saved = {k: v[k].clone() for k in ("idx", "counts", "offsets", "pos", "slot")}

    def restore():
        for k, t in saved.items():
            v[k].copy_(t)
        torch.cuda.synchronize()

    project = lambda: gqe.gqe_project(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], ws)  # noqa: E731
    plants = [
        ("pos", (0,), L + 7, "a position past the sequence"),
        ("pos", (17,), -1, "a negative position"),
        ("slot", (5,), 2, "a slot past k"),
        ("counts", (0, 0, 0), L + 1, "a count longer than the sequence"),
        ("offsets", (1,), -5, "an offset before its (b, g) range"),
        ("offsets", (4,), 0, "an offset in another group's range"),
    ]
    with library(gqe, "debug"):
        for key, at, val, what in plants:
            v[key][at] = val
            torch.cuda.synchronize()
            _expect_debug_error(gqe, project, f"{key}{list(at)} = {val}: {what}")
            restore()
        project()  # the restored lists pass, with the release library's result
        torch.cuda.synchronize()
        assert torch.equal(v["q"], q_release)

        dispatch = lambda: gqe.gqe_dispatch(cfg, ws)  # noqa: E731
        e0 = int(saved["idx"][0, 0, 0, 0])
        for at, val, what in (((0, 0, 0, 0), 4 + 3, "an expert id past E"),
                              ((0, 9, 1, 1), -2, "a negative expert id"),
                              ((0, 0, 0, 1), e0, "an expert picked twice")):
            v["idx"][at] = val
            torch.cuda.synchronize()
            _expect_debug_error(gqe, dispatch, f"idx{list(at)} = {val}: {what}")
            restore()
        dispatch()
        torch.cuda.synchronize()
        for k in ("counts", "offsets", "pos", "slot"):
            assert torch.equal(v[k], saved[k]), k


def test_debug_build_catches_planted_expert_in_backward(gqe):
    wl = W.WORKLOADS["tiny_fp32"]
    log("[debug] planted expert id before the backward (tiny fp32)")
    I, dev, cfg = _setup(gqe, wl)
    dy = torch.ones((wl.batch, wl.seq_len, wl.d_model), dtype=torch.float32, device="cuda")
    with library(gqe, "debug"):
        _, fws = _forward(gqe, wl, dev, cfg)
        v = gqe.workspace_views(cfg, fws)
        v["idx"][0, 3, 1, 0] = wl.n_experts + 1
        torch.cuda.synchronize()
        _expect_debug_error(gqe, lambda: _backward(gqe, wl, I, dev, cfg, fws, dy),
                            "idx[0, 3, 1, 0] past E before gqe_backward")

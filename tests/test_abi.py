"""The C ABI library: it loads, exports every declared entry point, and rejects
bad arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqe.h")
LIB = os.path.join(ROOT, "sparse_query_moe_amd", "libgqe.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(gq[ae]_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def gqe():
    if not os.path.exists(LIB):
        from sparse_query_moe_amd import build
        build.build()
    from sparse_query_moe_amd import gqe as mod
    # test_asan.py runs this file against the host-ASan build of the library
    other = os.environ.get("GQE_TEST_LIBRARY")
    if other:
        mod._lib = mod.load_library(other)
    return mod


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("gqe_forward", "gqa_forward", "gqe_workspace_bytes", "gqe_workspace_layout",
              "gqe_route", "gqe_dispatch", "gqe_project", "gqe_attention", "gqe_output",
              "gqe_status_string"):
        assert n in names


def test_binding_uses_the_library_under_test(gqe):
    assert gqe._lib._name == os.environ.get("GQE_TEST_LIBRARY", LIB)


def test_library_exports_every_declared_symbol(gqe):
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared_functions()) == set(gqe.EXPORTS)


def _cfg(gqe, **kw):
    base = dict(batch=1, seq_len=2048, d_model=1024, n_groups=4, n_experts=4, top_k=2, head_dim=64)
    base.update(kw)
    return gqe.make_config(**base)


def test_config_validation(gqe):
    assert gqe.gqe_workspace_bytes(_cfg(gqe)) > 0
    bad = [dict(top_k=0), dict(top_k=5), dict(d_model=1020), dict(n_groups=0), dict(seq_len=-1),
           dict(n_experts=33), dict(n_groups=9, n_experts=8), dict(shared_kv_group=4),
           dict(head_dim=0), dict(dtype=7), dict(softmax_scale=-1.0), dict(output_mode=3),
           dict(output_mode=-1)]
    for b in bad:
        assert gqe.gqe_workspace_bytes(_cfg(gqe, **b)) == 0, b
    assert gqe.gqe_workspace_bytes(_cfg(gqe, head_dim=96)) == 0
    lib = gqe._lib
    lay = gqe.WsLayout()
    assert lib.gqe_workspace_layout(ctypes.byref(_cfg(gqe, head_dim=96)), ctypes.byref(lay)) == -2
    assert lib.gqe_workspace_layout(ctypes.byref(_cfg(gqe, top_k=9)), ctypes.byref(lay)) == -1
    # the ablation outputs: k*G*d_h slot columns must fill whole K steps
    assert gqe.gqe_workspace_bytes(_cfg(gqe, output_mode="hard")) > 0
    odd = dict(head_dim=32, n_groups=3, top_k=1, n_experts=2, shared_kv_group=0)
    assert lib.gqe_workspace_layout(ctypes.byref(_cfg(gqe, output_mode="hard", **odd)),
                                    ctypes.byref(lay)) == -2


def test_ablation_outputs_shrink_the_slot_buffer(gqe):
    full = gqe.gqe_workspace_layout(_cfg(gqe))
    hard = gqe.gqe_workspace_layout(_cfg(gqe, output_mode="weighted_concat"))
    assert hard.total < full.total


def test_workspace_monotone_and_aligned(gqe):
    prev = 0
    for L in (1, 63, 64, 65, 2048, 8192, 131072):
        n = gqe.gqe_workspace_bytes(_cfg(gqe, seq_len=L))
        assert n >= prev
        prev = n
        lay = gqe.gqe_workspace_layout(_cfg(gqe, seq_len=L))
        for f in ("idx", "w", "counts", "offsets", "pos", "slot", "q", "k", "vt", "s"):
            assert getattr(lay, f) % 256 == 0
        assert lay.vt_tiles == (L + 63) // 64
    assert gqe.gqe_workspace_bytes(_cfg(gqe, batch=2)) > gqe.gqe_workspace_bytes(_cfg(gqe))


def test_host_errors_before_any_launch(gqe):
    """Invalid arguments return a status on the host; nothing touches a device."""
    lib = gqe._lib
    cfg = _cfg(gqe)
    n = gqe.gqe_workspace_bytes(cfg)
    # null pointers
    st = lib.gqe_forward(ctypes.byref(cfg), None, None, None, None, None, None, None, None, n, None)
    assert st == -1
    # misaligned workspace
    st = lib.gqe_dispatch(ctypes.byref(cfg), ctypes.c_void_p(8), n, None)
    assert st == -1
    # workspace too small
    st = lib.gqe_dispatch(ctypes.byref(cfg), ctypes.c_void_p(256), n - 1, None)
    assert st == -3
    # invalid config
    st = lib.gqe_attention(ctypes.byref(_cfg(gqe, top_k=0)), ctypes.c_void_p(256), n, None)
    assert st == -1
    # empty input: nothing to do
    st = lib.gqe_forward(ctypes.byref(_cfg(gqe, seq_len=0)), None, None, None, None, None, None,
                         None, None, 0, None)
    assert st == 0
    assert gqe.status_string(-3).startswith("GQE_ERR_WORKSPACE")


def test_decode_workspace_and_validation(gqe):
    """Decode: batch = sequences, seq_len = cache capacity."""
    cfg = _cfg(gqe, batch=4, seq_len=8192)
    n = gqe.gqe_decode_workspace_bytes(cfg)
    assert n > 0 and gqe.gqa_decode_workspace_bytes(cfg) > 0
    # split-K partials grow with the cache; the workspace never shrinks
    assert gqe.gqe_decode_workspace_bytes(_cfg(gqe, batch=4, seq_len=65536)) >= n
    assert gqe.gqe_decode_workspace_bytes(_cfg(gqe, batch=8, seq_len=8192)) >= n
    assert gqe.gqe_decode_workspace_bytes(_cfg(gqe, batch=4, seq_len=0)) == 0  # no room
    assert gqe.gqe_decode_workspace_bytes(_cfg(gqe, d_model=32768)) == 0
    assert gqe.gqe_decode_workspace_bytes(_cfg(gqe, top_k=0)) == 0
    # the ablation outputs have fewer heads and slots
    assert gqe.gqe_decode_workspace_bytes(_cfg(gqe, batch=4, seq_len=8192, output_mode="hard")) < n


def test_decode_host_errors_before_any_launch(gqe):
    lib = gqe._lib
    cfg = _cfg(gqe, batch=2, seq_len=4096)
    n = gqe.gqe_decode_workspace_bytes(cfg)
    a = ctypes.c_void_p(256)
    nulls = [None] * 11
    assert lib.gqe_decode(ctypes.byref(cfg), *nulls, n, None) == -1
    assert lib.gqa_decode(ctypes.byref(cfg), *nulls[:10], n, None) == -1
    # misaligned pos
    args = [a] * 11
    args[8] = ctypes.c_void_p(258)
    assert lib.gqe_decode(ctypes.byref(cfg), *args, n, None) == -1
    # workspace too small
    assert lib.gqe_decode(ctypes.byref(cfg), *([a] * 11), n - 1, None) == -3
    m = gqe.gqa_decode_workspace_bytes(cfg)
    assert lib.gqa_decode(ctypes.byref(cfg), *([a] * 10), m - 1, None) == -3
    # unsupported head size
    assert lib.gqe_decode(ctypes.byref(_cfg(gqe, head_dim=96)), *([a] * 11), n, None) == -2
    # no sequences: nothing to do
    assert lib.gqe_decode(ctypes.byref(_cfg(gqe, batch=0)), *nulls, 0, None) == 0


def test_backward_workspace_and_host_errors(gqe):
    lib = gqe._lib
    cfg = _cfg(gqe)
    n = gqe.gqe_backward_workspace_bytes(cfg)
    assert n > 0 and gqe.gqa_backward_workspace_bytes(cfg) > 0
    assert gqe.gqe_backward_workspace_bytes(_cfg(gqe, seq_len=4096)) > n
    assert gqe.gqe_backward_workspace_bytes(_cfg(gqe, top_k=0)) == 0
    f = gqe.gqe_workspace_bytes(cfg)
    a = ctypes.c_void_p(256)
    # null pointers
    st = lib.gqe_backward(ctypes.byref(cfg), *([None] * 7), 0.0, None, f, *([None] * 8), None, n,
                          None)
    assert st == -1
    # negative or infinite auxiliary weight
    for aux in (-1.0, float("inf")):
        st = lib.gqe_backward(ctypes.byref(cfg), *([a] * 7), aux, a, f, *([a] * 8), a, n, None)
        assert st == -1
    # forward workspace or backward workspace too small
    assert lib.gqe_backward(ctypes.byref(cfg), *([a] * 7), 0.0, a, f - 1, *([a] * 8), a, n,
                            None) == -3
    assert lib.gqe_backward(ctypes.byref(cfg), *([a] * 7), 0.0, a, f, *([a] * 8), a, n - 1,
                            None) == -3
    m = gqe.gqa_backward_workspace_bytes(cfg)
    fd = gqe.gqa_workspace_bytes(cfg)
    assert lib.gqa_backward(ctypes.byref(cfg), *([a] * 6), a, fd, *([a] * 5), a, m - 1, None) == -3
    # empty input: nothing to do
    assert lib.gqe_backward(ctypes.byref(_cfg(gqe, seq_len=0)), *([None] * 7), 0.0, None, 0,
                            *([None] * 8), None, 0, None) == 0


def test_group_top_k_validation_and_reach(gqe):
    """Per-group expert counts: validated on the host; every entry point takes
    them (workspaces grow with the total count)."""
    cfg = gqe.make_config(1, 64, 256, 2, 2, 1, 32, dtype="fp32", group_top_k=[1, 2])
    assert gqe.total_k(cfg) == 3
    assert gqe.gqe_workspace_bytes(cfg) > 0
    assert gqe.gqe_workspace_bytes(cfg) > gqe.gqe_workspace_bytes(
        gqe.make_config(1, 64, 256, 2, 2, 1, 32, dtype="fp32"))
    dec = gqe.gqe_decode_workspace_bytes(cfg)
    assert dec > gqe.gqe_decode_workspace_bytes(gqe.make_config(1, 64, 256, 2, 2, 1, 32, dtype="fp32"))
    assert gqe.gqe_backward_workspace_bytes(cfg) > gqe.gqe_backward_workspace_bytes(
        gqe.make_config(1, 64, 256, 2, 2, 1, 32, dtype="fp32"))
    for bad in ([0, 2], [1, 3]):
        assert gqe.gqe_workspace_bytes(
            gqe.make_config(1, 64, 256, 2, 2, 1, 32, dtype="fp32", group_top_k=bad)) == 0


def test_probe_host_errors_before_any_launch(gqe):
    """The measurement probes reject bad arguments on the host."""
    lib = gqe._lib
    assert lib.gqe_peak_mfma_bf16(None, 1, 1, None) == -1
    assert lib.gqe_peak_mfma_bf16(ctypes.c_void_p(256), 0, 1, None) == -1
    assert lib.gqe_peak_mfma_bf16(ctypes.c_void_p(256), 1, -1, None) == -1
    assert lib.gqe_peak_copy(None, ctypes.c_void_p(256), 16, None) == -1
    assert lib.gqe_peak_copy(ctypes.c_void_p(8), ctypes.c_void_p(4096), 16, None) == -1   # misaligned
    assert lib.gqe_peak_copy(ctypes.c_void_p(4096), ctypes.c_void_p(256), 24, None) == -1  # not 16 B steps
    assert lib.gqe_peak_copy(ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 1024), 2048, None) == -1  # overlap
    assert lib.gqe_peak_copy(ctypes.c_void_p(4096), ctypes.c_void_p(256), 0, None) == 0  # nothing to do
    assert lib.gqe_peak_copy(None, None, 0, None) == 0


def test_debug_library_exports_every_declared_symbol():
    """The index-checked debug build has the same boundary."""
    from sparse_query_moe_amd import build
    if not os.path.exists(build.DEBUG_LIB):
        build.build(variant="debug")
    lib = ctypes.CDLL(build.DEBUG_LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings(gqe):
    for st, name in ((0, "GQE_OK"), (-1, "GQE_ERR_INVALID_ARG"), (-2, "GQE_ERR_UNSUPPORTED"),
                     (-3, "GQE_ERR_WORKSPACE"), (-4, "GQE_ERR_HIP"), (-5, "GQE_ERR_DEBUG")):
        assert gqe.status_string(st).startswith(name)


def test_short_forward_predicate(gqe):
    """gqe_forward takes the short-layer launches for bf16 layers of at most
    4096 tokens with k_g <= 4 and d_model a multiple of 128; fp32 layers and
    longer ones take the staged sequence."""
    for kw, want in (({"seq_len": 4096}, True), ({"seq_len": 4097}, False),
                     ({"batch": 2, "seq_len": 2048}, True), ({"batch": 3, "seq_len": 2048}, False),
                     ({"seq_len": 2048, "dtype": "fp32"}, False),
                     ({"seq_len": 2048, "d_model": 1088}, False),
                     ({"seq_len": 2048, "group_top_k": [1, 2, 3, 2]}, True),
                     ({"seq_len": 2048, "n_experts": 8, "top_k": 5}, False)):
        assert gqe.uses_short_forward(_cfg(gqe, **kw)) == want, kw
    # the short forward's workspace also holds the all-heads projection
    assert gqe.gqe_workspace_bytes(_cfg(gqe, seq_len=4096)) > \
        gqe.gqe_workspace_bytes(_cfg(gqe, seq_len=4096, dtype="fp32")) // 2


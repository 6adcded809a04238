"""Seeded random layer shapes on the GPU against the oracle, through the C ABI
(needs an MI355X).

Each case draws a configuration the library accepts -- batch, length, model
width, groups, experts, k, head size, precision, output construction, shared
group, softmax scale, router bias, rotary base -- from a fixed seed (inputs N(0, 1), weights N(0, 0.09/d): outputs of the
benchmark layer's magnitude), and checks gqe_forward against the oracle's
layer: routing and dispatch lists bit
for bit, the output to the output gate (max-abs 2e-2 and mean-abs 2e-3 for
bf16, 1e-5 for float32) and to relative L2 2e-2 (bf16) / 1e-5 (float32).
Configurations the library rejects as unsupported (a width that is not a
whole number of 128-byte steps, for instance) are redrawn, so the cases cover
what the boundary documents as supported.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_util import f64_inputs, log, output_gate, to_dev, to_f64  # noqa: E402

pytestmark = pytest.mark.gpu

N_CASES = 16


@pytest.fixture(scope="module")
def gqe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_query_moe_amd import gqe as mod
    return mod


def _draw_case(gqe, seed):
    rng = np.random.default_rng(1000 + seed)
    while True:
        dtype = "bf16" if rng.random() < 0.6 else "fp32"
        G = int(rng.integers(1, 5))
        E = int(rng.integers(1, 7))
        k = int(rng.integers(1, E + 1))
        D = int(rng.choice([32, 64, 128]))
        d = int(rng.choice([128, 256, 384]))
        B = int(rng.integers(1, 4))
        L = int(rng.choice([1, 2, 63, 64, 65, 127, 200, 257, 511, 700]))
        mode = str(rng.choice(["full", "full", "hard", "weighted_concat"]))
        shared = int(rng.integers(0, G))
        scale = float(rng.choice([0.0, 0.0, 0.3, 1.0 / math.sqrt(D) * 1.7]))
        bias = bool(rng.random() < 0.5)
        rope = float(rng.choice([0.0, 0.0, 1000.0, 10000.0]))
        cfg = gqe.make_config(B, L, d, G, E, k, D, dtype=dtype, shared_kv_group=shared,
                              softmax_scale=scale, output_mode=mode, rope_base=rope)
        try:
            gqe.gqe_workspace_layout(cfg)
        except gqe.GqeError:
            continue
        return dict(dtype=dtype, G=G, E=E, k=k, D=D, d=d, B=B, L=L, mode=mode, shared=shared,
                    scale=scale, bias=bias, rope=rope, rng=rng)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_layer_matches_oracle(gqe, seed):
    c = _draw_case(gqe, seed)
    G, E, k, D, d, B, L = c["G"], c["E"], c["k"], c["D"], c["d"], c["B"], c["L"]
    log(f"[fuzz {seed}] B{B} L{L} d{d} G{G} E{E} k{k} D{D} {c['dtype']} {c['mode']} "
        f"shared{c['shared']} scale{c['scale']:.3f} bias{c['bias']} rope{c['rope']:.0f}")
    # weights of std 0.3/sqrt(d) keep scores, logits and outputs at the
    # magnitudes of the benchmark layer (|y| below about 1), where the
    # absolute output gate is stated
    wl = W.Workload("fuzz", B, L, d, G, E, k, D, c["dtype"], 1.0, 0.3 / math.sqrt(d))
    I = dict(W.make_inputs(wl, seed=seed, with_gqa=True))
    if c["mode"] != "full":
        I["wo"] = np.ascontiguousarray(I["wo"][:, :k * G * D])
    if c["bias"]:
        I["br"] = (c["rng"].standard_normal(G * E) * 0.5).astype(np.float32)
    dev = {key: to_dev(v, wl.dtype) for key, v in I.items()}
    cfg = gqe.make_config(B, L, d, G, E, k, D, dtype=c["dtype"], shared_kv_group=c["shared"],
                          softmax_scale=c["scale"], output_mode=c["mode"], rope_base=c["rope"],
                          router_bias=dev["br"])
    ws = gqe.alloc_workspace(cfg)
    out = torch.empty((B, L, d), dtype=cfg.torch_dtype, device="cuda")
    gqe.gqe_forward(cfg, dev["x"], dev["wq"], dev["wk"], dev["wv"], dev["wr"], dev["wo"], out, ws)
    torch.cuda.synchronize()
    F = f64_inputs(wl, I)
    ref = oracle.gqe_forward(F["x"], F["wq"], F["wk"], F["wv"], F["wr"], F["wo"], F["br"], G, E, k,
                             D, shared_kv_group=c["shared"],
                             scale=None if c["scale"] == 0.0 else c["scale"],
                             output_mode=c["mode"], rope_base=c["rope"])
    v = gqe.workspace_views(cfg, ws)
    for key in ("idx", "counts", "offsets", "pos", "slot"):
        got = v[key].cpu().numpy()
        assert np.array_equal(got, ref[key]), f"{key} differs from the oracle"
    mx, mean, rel = output_gate(to_f64(out), ref["y"], wl.dtype, f"fuzz {seed} y")
    log(f"  y: max-abs {mx:.3e} mean-abs {mean:.3e} rel-L2 {rel:.3e}")
    assert rel <= (2e-2 if wl.dtype == W.BF16 else 1e-5)

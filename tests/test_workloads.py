"""The seeded input generator: determinism and its bf16 rounding (no GPU)."""
import numpy as np

import workloads as W


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is halfway between two bf16 values: ties go to the even one (1.0)
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1e-30, 3.0e38], dtype=np.float32)
    bits = W.f32_to_bf16_bits(vals)
    back = W.bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2.0 ** -6
    assert back[3] == -2.5
    # every value is within half a bf16 ulp
    rel = np.abs(back.astype(np.float64) - vals) / np.abs(vals)
    assert (rel <= 2.0 ** -8).all()


def test_inputs_are_deterministic_and_shaped():
    wl = W.WORKLOADS["tiny_fp32"]
    a = W.make_inputs(wl, with_gqa=True)
    b = W.make_inputs(wl, with_gqa=True)
    for key in a:
        assert np.array_equal(a[key], b[key])
    G, E, k, dh, d = wl.n_groups, wl.n_experts, wl.top_k, wl.head_dim, wl.d_model
    assert a["x"].shape == (1, 128, d)
    assert a["wq"].shape == ((G * E + 1) * dh, d)
    assert a["wo"].shape == (d, (k * G + 2) * dh)
    assert a["wo_dense"].shape == (d, G * E * dh)
    assert abs(a["wq"].std() - 1 / 16) < 0.01


def test_bf16_workload_small_slice():
    wl = W.WORKLOADS["l2k"].with_(seq_len=64)
    a = W.make_inputs(wl)
    assert a["x"].dtype == np.uint16
    x = W.to_f64(a["x"], wl.dtype)
    assert abs(x.std() - 1.0) < 0.05
    assert abs(W.to_f64(a["wq"], wl.dtype).std() - 0.02) < 0.002


def test_zipf_bias_and_sampled_rows():
    wl = W.WORKLOADS["l1m_zipf"]
    br = W.router_bias(wl).reshape(wl.n_groups, wl.n_experts)
    assert np.allclose(np.exp(br[0]) / np.exp(br[0])[0], 1.0 / np.arange(1, 5) ** 1.2, rtol=1e-6)
    rows = W.sample_rows(W.WORKLOADS["l128k"])
    assert len(rows) == 512 and rows[0] == 0 and rows[1] == 1 and rows[-1] == 131071
    assert (np.diff(rows) > 0).all()

#!/usr/bin/env python3
"""Benchmark of the GQE prefill layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload l1m_zipf]

One step = one gqe_forward (router, dispatch, projections, attention, output)
over one batch of synthetic input already resident in HBM.  The headline
workload is the largest one, B1 x L1048576 with a Zipf(1.2) router prior.
The timed region is exactly K back-to-back gqe_forward calls between two
device synchronizations, bracketed by HIP events on the stream.  Separate
passes give the per-stage breakdown (events between the stage calls), the
average duration of the attention kernel over back-to-back launches (the
roofline figure) and, for the short workloads, the same step replayed from a
HIP graph.  The dense-GQA baseline (all G*E query heads) is timed the same
way, giving the GQE-over-GQA prefill speed-up at every length.  The CPU
oracle is timed beside it on the host cores (sampled query rows at the long
workloads, which also check the GPU step).  Rank 0 prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_BF16 = 2516.6e12     # dense bf16 MFMA, FLOP/s
PEAK_FP32_MFMA = 157.3e12
PEAK_HBM = 8.0e12         # bytes/s
METRIC = "GQE prefill tokens/s per layer + speedup vs dense GQA; % bf16 MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def route_bytes(wl):
    """Algorithmic HBM bytes of the router: x and W_r read once, idx and w
    (int32 and float32 per routed slot) written once."""
    T, es = wl.batch * wl.seq_len, 2 if wl.dtype == W.BF16 else 4
    return T * wl.d_model * es + wl.n_groups * wl.n_experts * wl.d_model * es + \
        T * wl.n_groups * wl.top_k * 8


def dispatch_bytes(wl):
    """Algorithmic HBM bytes of the dispatch: idx read once, pos and slot
    (int32 each) written once per routed row."""
    rows = wl.batch * wl.seq_len * wl.n_groups * wl.top_k
    return rows * 4 + rows * 8


def stage_work(wl):
    """Algorithmic work of every stage for one step: (kind, amount) with kind
    'flop' (MFMA) or 'byte' (HBM)."""
    B, L, d, G, E, k, D = (wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts,
                           wl.top_k, wl.head_dim)
    T = B * L
    es = 2 if wl.dtype == W.BF16 else 4
    return {
        "route": ("byte", T * d * es + T * G * k * 8 + G * E * d * es),
        "dispatch": ("byte", T * G * k * 4 + T * G * k * 8),
        "project": ("flop", 2 * T * d * D * (k * G + 2 * G + 1)),
        "attention": ("flop", 2 * 2 * D * (k * G + 1) * B * L * (L + 1) // 2),
        "output": ("flop", 2 * T * (k * G + 2) * D * d),
    }


def gqa_stage_work(wl):
    B, L, d, G, E, D = wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts, wl.head_dim
    T = B * L
    return {
        "project": ("flop", 2 * T * d * D * (G * E + 2 * G)),
        "attention": ("flop", 2 * 2 * D * G * E * B * L * (L + 1) // 2),
        "output": ("flop", 2 * T * G * E * D * d),
    }


class Runner:
    """Device inputs, workspaces and the per-stage call sequence of one workload."""

    def __init__(self, wl, gqe, torch):
        self.wl, self.gqe, self.torch = wl, gqe, torch
        I = W.make_inputs(wl, with_gqa=True)
        dev = {}
        for key, v in I.items():
            if v.dtype == np.uint16:
                dev[key] = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(
                    torch.bfloat16).to("cuda")
            else:
                dev[key] = torch.from_numpy(np.ascontiguousarray(v)).to("cuda")
        self.I, self.dev = I, dev
        self.cfg = gqe.make_config(wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts,
                                   wl.top_k, wl.head_dim, dtype=wl.dtype, router_bias=dev["br"])
        self.ws = gqe.alloc_workspace(self.cfg)
        self.ws_dense = gqe.alloc_workspace(self.cfg, dense=True)
        shape = (wl.batch, wl.seq_len, wl.d_model)
        self.out = torch.empty(shape, dtype=self.cfg.torch_dtype, device="cuda")
        self.out_dense = torch.empty(shape, dtype=self.cfg.torch_dtype, device="cuda")

    def gqe_stages(self):
        g, c, d, ws = self.gqe, self.cfg, self.dev, self.ws
        return [
            ("route", lambda: g.gqe_route(c, d["x"], d["wr"], ws)),
            ("dispatch", lambda: g.gqe_dispatch(c, ws)),
            ("project", lambda: g.gqe_project(c, d["x"], d["wq"], d["wk"], d["wv"], ws)),
            ("attention", lambda: g.gqe_attention(c, ws)),
            ("output", lambda: g.gqe_output(c, d["wo"], self.out, ws)),
        ]

    def gqa_stages(self):
        g, c, d, ws = self.gqe, self.cfg, self.dev, self.ws_dense
        return [
            ("project", lambda: g.gqa_project(c, d["x"], d["wq_dense"], d["wk"], d["wv"], ws)),
            ("attention", lambda: g.gqa_attention(c, ws)),
            ("output", lambda: g.gqa_output(c, d["wo_dense"], self.out_dense, ws)),
        ]

    def gqe_step(self):
        g, d = self.gqe, self.dev
        g.gqe_forward(self.cfg, d["x"], d["wq"], d["wk"], d["wv"], d["wr"], d["wo"], self.out,
                      self.ws)

    def gqa_step(self):
        g, d = self.gqe, self.dev
        g.gqa_forward(self.cfg, d["x"], d["wq_dense"], d["wk"], d["wv"], d["wo_dense"],
                      self.out_dense, self.ws_dense)

    def time_steps(self, step, steps, warmup):
        """Warm up, then time exactly `steps` back-to-back calls between two
        synchronizations; returns ms per call (HIP events on the stream)."""
        torch = self.torch
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            step()
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps

    def time_stages(self, stages, steps):
        """Per-stage breakdown (a separate pass): events between the stage calls."""
        torch = self.torch
        for _, fn in stages:
            fn()
        torch.cuda.synchronize()
        n = len(stages)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
        for s in range(steps):
            ev[s][0].record()
            for i, (_, fn) in enumerate(stages):
                fn()
                ev[s][i + 1].record()
        torch.cuda.synchronize()
        return {name: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps
                for i, (name, _) in enumerate(stages)}

    def time_graph(self, step, steps):
        """The same step captured once in a HIP graph and replayed `steps`
        times; returns (ms per replay, replay output equals the eager one)."""
        torch = self.torch
        out = self.out if step == self.gqe_step else self.out_dense
        step()
        torch.cuda.synchronize()
        eager = out.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        ms = None
        ok = True
        for rep in range(2):
            out.zero_()
            torch.cuda.synchronize()
            start = torch.cuda.Event(enable_timing=True)
            stop = torch.cuda.Event(enable_timing=True)
            start.record()
            for _ in range(steps):
                graph.replay()
            stop.record()
            torch.cuda.synchronize()
            ms = start.elapsed_time(stop) / steps
            ok = ok and bool(torch.equal(out, eager))
        del graph
        return ms, ok


def rate(kind, amount, ms):
    v = amount / (ms * 1e-3)
    return v / 1e12  # TFLOP/s or TB/s


def measure(wl, gqe, torch, steps, warmup, graph=True, side_steps=None):
    """GQE and dense-GQA step times of one workload.  The GQE step is timed
    over exactly `steps` calls after `warmup`; the dense baseline, the
    per-stage breakdown and the attention kernel alone use `side_steps`
    calls (default: `steps`; at least 3)."""
    r = Runner(wl, gqe, torch)
    side = max(3, steps if side_steps is None else side_steps)
    t_gqe = r.time_steps(r.gqe_step, steps, warmup)
    t_gqa = r.time_steps(r.gqa_step, side, min(warmup, 1 if side_steps else warmup))
    st_gqe = r.time_stages(r.gqe_stages(), max(2, side // 2))
    st_gqa = r.time_stages(r.gqa_stages(), max(2, side // 2))
    # the attention kernel alone, launched back to back: its average duration
    k_gqe = r.time_steps(lambda: gqe.gqe_attention(r.cfg, r.ws), side, 1)
    k_gqa = r.time_steps(lambda: gqe.gqa_attention(r.cfg, r.ws_dense), side, 1)
    tokens = wl.batch * wl.seq_len
    work = stage_work(wl)
    gwork = gqa_stage_work(wl)
    peak = PEAK_BF16 if wl.dtype == W.BF16 else PEAK_FP32_MFMA
    att = work["attention"][1] / (k_gqe * 1e-3)
    res = {
        "workload": wl.name,
        "tokens": tokens,
        "gqe_ms": t_gqe,
        "gqa_ms": t_gqa,
        "gqe_tokens_per_s": tokens / (t_gqe * 1e-3),
        "gqa_tokens_per_s": tokens / (t_gqa * 1e-3),
        "speedup_vs_gqa": t_gqa / t_gqe,
        "attention_kernel_ms": k_gqe,
        "gqa_attention_kernel_ms": k_gqa,
        "attention_speedup_vs_gqa": k_gqa / k_gqe,
        "gqe_stage_ms": {k: round(v, 5) for k, v in st_gqe.items()},
        "gqa_stage_ms": {k: round(v, 5) for k, v in st_gqa.items()},
        "attention_tflops": att / 1e12,
        "attention_mfma_frac": att / peak,
        # the routing kernels against HBM: algorithmic bytes / stage time
        "route_hbm_tb_per_s": route_bytes(wl) / (st_gqe["route"] * 1e-3) / 1e12,
        "dispatch_hbm_tb_per_s": dispatch_bytes(wl) / (st_gqe["dispatch"] * 1e-3) / 1e12,
        "gqa_attention_mfma_frac": gwork["attention"][1] / (k_gqa * 1e-3) / peak,
    }
    if graph:
        g_gqe, ok_gqe = r.time_graph(r.gqe_step, steps)
        g_gqa, ok_gqa = r.time_graph(r.gqa_step, steps)
        res.update({"graph_gqe_ms": g_gqe, "graph_gqa_ms": g_gqa,
                    "graph_speedup_vs_gqa": g_gqa / g_gqe,
                    "graph_replay_equals_eager": ok_gqe and ok_gqa})
    return r, res


def measure_decode(gqe, torch, steps, warmup, name="dec_b64_c8k"):
    """One decode step (gqe_decode / gqa_decode): every sequence's new token
    at the last cache position, so each step reads the whole cache.  Returns
    step times, tokens/s and the HBM rate over the algorithmic bytes (the K
    and V^T cache once, every weight once)."""
    wl = W.DECODE_WORKLOADS[name]
    I = W.make_decode_inputs(wl, with_gqa=True)
    I["pos"][:] = wl.seq_len - 1
    B, Lc, d, G, E, k, D = (wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts,
                            wl.top_k, wl.head_dim)
    cfg = gqe.make_config(B, Lc, d, G, E, k, D, dtype=wl.dtype)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to("cuda")
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    # timing only: the V^T cache holds the drawn values in its own tiled shape
    assert Lc % 64 == 0
    vt = I["v_cache"].reshape(B, G, Lc // 64, D, 64)
    x, wq, wk, wv, wr, wo = (dev(I[n]) for n in ("x", "wq", "wk", "wv", "wr", "wo"))
    wqd, wod = dev(I["wq_dense"]), dev(I["wo_dense"])
    kc, vtc = dev(I["k_cache"]), dev(vt)
    pos = torch.from_numpy(I["pos"].astype(np.int32)).cuda()
    out = torch.empty((B, d), dtype=cfg.torch_dtype, device="cuda")
    ws = gqe.alloc_decode_workspace(cfg)
    ws_d = gqe.alloc_decode_workspace(cfg, dense=True)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    t_gqe = timed(lambda: gqe.gqe_decode(cfg, x, wq, wk, wv, wr, wo, kc, vtc, pos, out, ws))
    t_gqa = timed(lambda: gqe.gqa_decode(cfg, x, wqd, wk, wv, wod, kc, vtc, pos, out, ws_d))
    es = 2 if wl.dtype == W.BF16 else 4
    kv = B * G * Lc * D * 2 * es
    w_gqe = ((G * E + 1) * D + 2 * G * D + G * E) * d * es + d * (k * G + 2) * D * es
    w_gqa = (G * E * D + 2 * G * D) * d * es + d * G * E * D * es
    del kc, vtc, ws, ws_d
    torch.cuda.empty_cache()
    return {
        "workload": wl.description, "batch": B, "cache_len": Lc,
        "gqe_step_ms": round(t_gqe, 5), "gqa_step_ms": round(t_gqa, 5),
        "gqe_tokens_per_s": round(B / (t_gqe * 1e-3), 1),
        "gqa_tokens_per_s": round(B / (t_gqa * 1e-3), 1),
        "speedup_vs_gqa": round(t_gqa / t_gqe, 4),
        "gqe_hbm_tb_per_s": round((kv + w_gqe) / (t_gqe * 1e-3) / 1e12, 3),
        "gqa_hbm_tb_per_s": round((kv + w_gqa) / (t_gqa * 1e-3) / 1e12, 3),
        "bytes_per_step": {"kv_cache": kv, "gqe_weights": w_gqe, "gqa_weights": w_gqa},
    }


def measure_training(wl, gqe, torch, steps, warmup):
    """One training step of the layer: gqe_forward then gqe_backward (dy of
    the output's shape, load-balancing weight 0.01), and the same for dense
    GQA; the backward alone is timed too.  Returns ms per step and tokens/s."""
    r = Runner(wl, gqe, torch)
    G, E, D, d = wl.n_groups, wl.n_experts, wl.head_dim, wl.d_model
    f32 = dict(dtype=torch.float32, device="cuda")
    rng = np.random.Generator(np.random.PCG64(12))
    dy = W._draw(rng, (wl.batch, wl.seq_len, d), 1.0, wl.dtype)
    if dy.dtype == np.uint16:
        dy = torch.from_numpy(dy.view(np.int16)).view(torch.bfloat16).to("cuda")
    else:
        dy = torch.from_numpy(dy).to("cuda")
    I = r.I
    g = {k: torch.empty(v, **f32) for k, v in dict(
        dx=(wl.batch, wl.seq_len, d), dwq=I["wq"].shape, dwk=I["wk"].shape, dwv=I["wv"].shape,
        dwr=(G * E, d), dbr=(G * E,), dwo=I["wo"].shape, aux=(1,), dwqd=I["wq_dense"].shape,
        dwod=I["wo_dense"].shape).items()}
    bws = gqe.alloc_backward_workspace(r.cfg)
    bws_d = gqe.alloc_backward_workspace(r.cfg, dense=True)
    dv = r.dev

    def gqe_bwd():
        gqe.gqe_backward(r.cfg, dv["x"], dv["wq"], dv["wk"], dv["wv"], dv["wr"], dv["wo"], dy, 0.01,
                         r.ws, g["dx"], g["dwq"], g["dwk"], g["dwv"], g["dwr"], g["dbr"], g["dwo"],
                         g["aux"], bws)

    def gqa_bwd():
        gqe.gqa_backward(r.cfg, dv["x"], dv["wq_dense"], dv["wk"], dv["wv"], dv["wo_dense"], dy,
                         r.ws_dense, g["dx"], g["dwqd"], g["dwk"], g["dwv"], g["dwod"], bws_d)

    t_gqe = r.time_steps(lambda: (r.gqe_step(), gqe_bwd()), steps, warmup)
    t_gqa = r.time_steps(lambda: (r.gqa_step(), gqa_bwd()), steps, warmup)
    b_gqe = r.time_steps(gqe_bwd, steps, 1)
    b_gqa = r.time_steps(gqa_bwd, steps, 1)
    tokens = wl.batch * wl.seq_len
    del bws, bws_d, g, r
    torch.cuda.empty_cache()
    return {"workload": wl.name, "gqe_step_ms": round(t_gqe, 5), "gqa_step_ms": round(t_gqa, 5),
            "gqe_backward_ms": round(b_gqe, 5), "gqa_backward_ms": round(b_gqa, 5),
            "gqe_tokens_per_s": round(tokens / (t_gqe * 1e-3), 1),
            "gqa_tokens_per_s": round(tokens / (t_gqa * 1e-3), 1),
            "speedup_vs_gqa": round(t_gqa / t_gqe, 4),
            "backward_speedup_vs_gqa": round(b_gqa / b_gqe, 4)}


def measure_sweep(gqe, torch, steps, warmup, batch=4, seq_len=8192):
    """The pages leave two knobs unexplored (pptc.cn section 6): the expert
    pool E per group and a per-group k.  GQE against dense GQA (all G*E heads)
    at B4 x L8192 of the 250M layer for E = 2, 4, 8, 16 with half of each
    group's experts active, and for two per-group splits of k = 8 slots."""
    base = W.WORKLOADS["b4_l8k"].with_(batch=batch, seq_len=seq_len)
    configs = [(E, E // 2, None) for E in (2, 4, 8, 16)] + [(4, 2, [1, 2, 3, 2]),
                                                              (4, 2, [4, 2, 1, 1])]
    out = []
    for E, k, ks in configs:
        wl = base.with_(n_experts=E, top_k=k)
        I = W.make_inputs(wl, with_gqa=True)
        K = sum(ks) if ks else k * wl.n_groups
        if ks:
            rng = np.random.Generator(np.random.PCG64(22))
            I["wo"] = W._draw(rng, (wl.d_model, (K + 2) * wl.head_dim), wl.w_std, wl.dtype)

        def dev(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                    torch.bfloat16).to("cuda")
            return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

        d = {n: dev(v) for n, v in I.items()}
        cfg = gqe.make_config(wl.batch, wl.seq_len, wl.d_model, wl.n_groups, E, k, wl.head_dim,
                              dtype=wl.dtype, router_bias=d["br"], group_top_k=ks)
        ws, ws_d = gqe.alloc_workspace(cfg), gqe.alloc_workspace(cfg, dense=True)
        y = torch.empty((wl.batch, wl.seq_len, wl.d_model), dtype=cfg.torch_dtype, device="cuda")

        def timed(fn):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / steps

        t_gqe = timed(lambda: gqe.gqe_forward(cfg, d["x"], d["wq"], d["wk"], d["wv"], d["wr"],
                                              d["wo"], y, ws))
        t_gqa = timed(lambda: gqe.gqa_forward(cfg, d["x"], d["wq_dense"], d["wk"], d["wv"],
                                              d["wo_dense"], y, ws_d))
        out.append({"n_experts": E, "top_k": k if ks is None else None, "group_top_k": ks,
                    "active_query_heads": f"{K + 1}/{wl.n_groups * E}",
                    "gqe_ms": round(t_gqe, 5), "gqa_ms": round(t_gqa, 5),
                    "speedup_vs_gqa": round(t_gqa / t_gqe, 4)})
        log(f"[bench]   sweep {out[-1]}")
        del ws, ws_d, d, y
        torch.cuda.empty_cache()
    return {"workload": base.description, "points": out}


def measure_ablation(gqe, torch, steps, warmup, name="b4_l8k"):
    """The output constructions of the pages' ablation (pptc.cn section 4.3):
    the full layer, hard concatenation only, and weighted concatenation
    without the renormalized slot, each timed as one gqe_forward against dense
    GQA on the same inputs (W_O of the ablations: its first k*G*d_h input
    columns)."""
    wl = W.WORKLOADS[name]
    I = W.make_inputs(wl, with_gqa=True)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to("cuda")
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    d = {n: dev(v) for n, v in I.items()}
    K = wl.top_k * wl.n_groups
    d["wo_hard"] = dev(np.ascontiguousarray(I["wo"][:, :K * wl.head_dim]))
    y = torch.empty((wl.batch, wl.seq_len, wl.d_model), dtype=torch.bfloat16, device="cuda")

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    out = []
    t_gqa = None
    for mode in ("full", "hard", "weighted_concat"):
        cfg = gqe.make_config(wl.batch, wl.seq_len, wl.d_model, wl.n_groups, wl.n_experts,
                              wl.top_k, wl.head_dim, dtype=wl.dtype, router_bias=d["br"],
                              output_mode=mode)
        ws = gqe.alloc_workspace(cfg)
        wo = d["wo"] if mode == "full" else d["wo_hard"]
        t = timed(lambda: gqe.gqe_forward(cfg, d["x"], d["wq"], d["wk"], d["wv"], d["wr"], wo,
                                          y, ws))
        if t_gqa is None:
            ws_d = gqe.alloc_workspace(cfg, dense=True)
            t_gqa = timed(lambda: gqe.gqa_forward(cfg, d["x"], d["wq_dense"], d["wk"], d["wv"],
                                                  d["wo_dense"], y, ws_d))
            del ws_d
        out.append({"output_mode": mode, "slot_heads": K + (1 if mode == "full" else 0),
                    "gqe_ms": round(t, 5), "gqa_ms": round(t_gqa, 5),
                    "speedup_vs_gqa": round(t_gqa / t, 4)})
        log(f"[bench]   ablation {out[-1]}")
        del ws
    del d, y
    torch.cuda.empty_cache()
    return {"workload": wl.description, "points": out}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_kernel_hbm_traffic.txt")
KERNEL_SOURCES = ("attention.hip", "attention.h", "device_common.h", "dispatch_dev.h", "kernels.h",
                  "debug_check.h")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_query_moe_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(wl_name):
    """HBM bytes per attention launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or None when the
    summary is missing, covers another workload or predates the kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split("=", 1) for line in f if "=" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    key = f"traffic_bytes_per_launch.{wl_name}"
    return float(kv[key]) if key in kv else None


def roofline_for(wl, res, peaks=None):
    """Roofline of the dominant kernel of the step, the causal attention kernel
    (the longest single kernel at every workload), from its average duration
    over back-to-back launches; with `peaks` (measured_peaks) also against the
    matrix-core rate the probe sustains on the same device."""
    kind, amount = stage_work(wl)["attention"]
    ms = res["attention_kernel_ms"]
    peak = (PEAK_BF16 if wl.dtype == W.BF16 else PEAK_FP32_MFMA) / 1e12
    ach = rate(kind, amount, ms)
    out = {"kernel": "attention_kernel", "bound": "mfma", "achieved": round(ach, 3),
           "peak": round(peak, 3), "unit": "TFLOP/s", "frac": round(ach / peak, 4),
           "traffic": measured_traffic(wl.name),
           "per_launch": {"flop": amount, "avg_ms": round(ms, 5)}}
    if peaks is not None and wl.dtype == W.BF16:
        out["peak_measured"] = peaks["mfma_bf16_tflops"]
        out["frac_of_measured"] = round(ach / peaks["mfma_bf16_tflops"], 4)
    return out


def measured_peaks(gqe, torch, mfma_ms=200.0, copy_bytes=2 << 30):
    """What this device sustains, as the second reference beside the published
    peaks: the bf16 matrix-core probe (four independent 32x32x16 MFMA chains
    per wave, two waves per SIMD, nothing else) run for about `mfma_ms` per
    launch, and the HBM copy probe over `copy_bytes` (eight times the 256 MB
    last-level cache), each the best of its timed launches after a warm-up."""
    def time_launch(fn):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    blocks = gqe.peak_blocks()
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    iters = 4000
    time_launch(lambda: gqe.peak_mfma_bf16(out, blocks, iters))
    ms = time_launch(lambda: gqe.peak_mfma_bf16(out, blocks, iters))
    iters = max(iters, int(iters * mfma_ms / max(ms, 1e-3)))
    best = min(time_launch(lambda: gqe.peak_mfma_bf16(out, blocks, iters)) for _ in range(3))
    flop = blocks * 4 * iters * 4 * 32768
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("matrix-core probe produced a non-finite value")
    del out
    src = torch.ones(copy_bytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    time_launch(lambda: gqe.peak_copy(dst, src))
    best_c = min(time_launch(lambda: gqe.peak_copy(dst, src)) for _ in range(5))
    if not bool(torch.equal(dst, src)):
        raise RuntimeError("copy probe result differs from its source")
    del src, dst
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(flop / (best * 1e-3) / 1e12, 1),
            "hbm_copy_tb_per_s": round(2 * copy_bytes / (best_c * 1e-3) / 1e12, 3),
            "mfma_probe": f"{blocks} blocks x 4 waves x {iters} rounds of 4 chained "
                          f"v_mfma_f32_32x32x16_bf16, best of 3 ({best:.1f} ms)",
            "copy_probe": f"{copy_bytes} B read + {copy_bytes} B written, 16 B per access, "
                          f"best of 5 ({best_c:.3f} ms)"}


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        return len(os.sched_getaffinity(0))


def cpu_baseline(wl, budget_s=12.0):
    """The CPU oracle, as it stands, on full layers of the same workload until
    about `budget_s` seconds have passed; tokens/s over the layers it finished."""
    import oracle
    I = W.make_inputs(wl)
    f = lambda a: W.to_f64(a, wl.dtype)  # noqa: E731
    args = (f(I["x"]), f(I["wq"]), f(I["wk"]), f(I["wv"]), f(I["wr"]), f(I["wo"]),
            I["br"].astype(np.float64), wl.n_groups, wl.n_experts, wl.top_k, wl.head_dim)
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.gqe_forward(*args)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(n * wl.tokens / el, 2), "unit": "tokens/s", "cores": int(_oracle_threads()),
            "kind": "oracle",
            "sample": f"{n} full layers of {wl.name} (B={wl.batch}, L={wl.seq_len}) in {el:.1f} s, float64 numpy"}


def cpu_baseline_sampled(wl, runner, gqe):
    """The CPU oracle on the long workloads: routing and dispatch of every
    token, K and V of every position, then the attention and output of the
    workload's sampled query rows only.  Each phase is timed.  The full-layer
    oracle time is extrapolated from the sampled rows (attention in proportion
    to the causal span sum of (t+1), the output projection to the row count)
    and is labelled as such; `value` is tokens / that extrapolated time.

    The same call checks the GPU step that `runner` last ran: the routing and
    dispatch lists bit for bit over all tokens, and the sampled output rows
    against the output gate (max-abs 2e-2, mean-abs 2e-3 for bf16)."""
    import oracle
    I = runner.I
    rows = W.sample_rows(wl)
    f = lambda a: W.to_f64(a, wl.dtype)  # noqa: E731
    x = W.bf16_bits_to_f32(I["x"]) if wl.dtype == W.BF16 else I["x"]
    phases = {}
    t0 = time.perf_counter()
    ref = oracle.gqe_forward(x, f(I["wq"]), f(I["wk"]), f(I["wv"]), f(I["wr"]), f(I["wo"]),
                             I["br"].astype(np.float64), wl.n_groups, wl.n_experts, wl.top_k,
                             wl.head_dim, positions=rows, phase_times=phases)
    el = time.perf_counter() - t0
    L, B = wl.seq_len, wl.batch
    span_all = B * L * (L + 1) / 2.0
    span_sampled = B * float((rows + 1).sum())
    extrap = (phases["route"] + phases["dispatch"] + phases["kv"] +
              phases["attention"] * span_all / span_sampled +
              phases["output"] * (B * L) / (B * len(rows)))
    # the GPU's results of the last timed step
    v = gqe.workspace_views(runner.cfg, runner.ws)
    routing_ok = all(np.array_equal(v[key].cpu().numpy(), ref[key])
                     for key in ("idx", "counts", "offsets", "pos", "slot"))
    sel = runner.torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(runner.out.device)
    y = runner.out[:, sel].float().cpu().double().numpy()
    err = np.abs(y - ref["y"])
    rel = float(np.linalg.norm(y - ref["y"]) / max(np.linalg.norm(ref["y"]), 1e-300))
    tol = (2e-2, 2e-3) if wl.dtype == W.BF16 else (1e-5, 1e-5)
    check = {"rows": int(len(rows)), "routing_bit_exact": bool(routing_ok),
             "max_abs": float(err.max()), "mean_abs": float(err.mean()), "rel_l2": rel,
             "within_gate": bool(routing_ok and err.max() <= tol[0] and err.mean() <= tol[1])}
    return {"value": round(B * L / extrap, 2), "unit": "tokens/s", "cores": int(_oracle_threads()),
            "kind": "oracle",
            "sample": (f"{wl.name}: routing, dispatch and K/V of all {B * L} tokens, then "
                       f"{len(rows)} sampled query rows (seeded, log-spaced position bands) in "
                       f"{el:.1f} s, float64 numpy; value = tokens / extrapolated full-layer "
                       f"oracle time {extrap:.0f} s"),
            "phase_s": {k: round(t, 3) for k, t in phases.items()},
            "sampled_rows_per_s": round(len(rows) * B / (phases["attention"] + phases["output"]), 2),
            "extrapolated_full_layer_s": round(extrap, 1),
            "gpu_check": check}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="l1m_zipf", choices=sorted(W.WORKLOADS))
    ap.add_argument("--lengths", default="l2k,b4_l8k,l128k",
                    help="other workloads timed for the per-length speed-up (comma list, '' = none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step timing")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the expert-pool and per-group-k sweep and the ablation timing")
    ap.add_argument("--training", default="l2k,b4_l8k",
                    help="workloads whose training step (forward + backward) is timed "
                         "(comma list, '' = none)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB three times (the known-size "
                         "kernel that calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_query_moe_amd import gqe

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 x {n} bytes read and written")
        del src, dst

    wl = W.WORKLOADS[args.workload]
    long_step = stage_work(wl)["attention"][1] > 1e14   # a step of 40 ms or more
    log(f"[bench] {wl.description}: warmup {args.warmup}, steps {args.steps}")
    runner, res = measure(wl, gqe, torch, args.steps, args.warmup,
                          graph=not args.no_graph and not long_step,
                          side_steps=3 if long_step else None)
    log(f"[bench] gqe {res['gqe_ms']:.4f} ms  gqa {res['gqa_ms']:.4f} ms  "
        f"speed-up {res['speedup_vs_gqa']:.3f}  attention {res['attention_mfma_frac']:.3f} of peak  "
        f"stages {res['gqe_stage_ms']}")
    cpu = None
    if not args.no_cpu_baseline and wl.sample_rows:
        log("[bench] cpu baseline (oracle, sampled rows) and check of the GPU step ...")
        cpu = cpu_baseline_sampled(wl, runner, gqe)
        log(f"[bench]   {cpu}")
    del runner
    torch.cuda.empty_cache()

    per_length = []
    for name in [n for n in args.lengths.split(",") if n]:
        if name == wl.name:
            continue
        w2 = W.WORKLOADS[name]
        steps = max(2, min(200, int(2e12 / max(1, stage_work(w2)["attention"][1]) + 2)))
        log(f"[bench] per-length {w2.description}: steps {steps}")
        _, r2 = measure(w2, gqe, torch, steps, min(10, steps), graph=not args.no_graph)
        log(f"[bench]   gqe {r2['gqe_ms']:.4f} ms gqa {r2['gqa_ms']:.4f} ms "
            f"speed-up {r2['speedup_vs_gqa']:.3f} attention {r2['attention_mfma_frac']:.3f} of peak")
        per_length.append(r2)
        torch.cuda.empty_cache()
    per_length.append(res)

    log("[bench] measured peaks (matrix-core and HBM copy probes) ...")
    peaks = measured_peaks(gqe, torch)
    log(f"[bench]   {peaks}")

    line = {
        "metric": METRIC,
        "value": round(res["gqe_tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["gqe_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == W.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.description, "name": wl.name, "batch": wl.batch,
                   "seq_len": wl.seq_len, "router_bias": (f"-{wl.zipf_s} ln(e+1) per group"
                                                          if wl.zipf_s else "zero"),
                   "d_model": wl.d_model, "n_groups": wl.n_groups, "n_experts": wl.n_experts,
                   "top_k": wl.top_k, "head_dim": wl.head_dim, "shared_heads": 1,
                   "parallelism": "single GPU"},
        "speedup_vs_gqa": round(res["speedup_vs_gqa"], 4),
        "gqa_tokens_per_s": round(res["gqa_tokens_per_s"], 1),
        "attention_mfma_frac": round(res["attention_mfma_frac"], 4),
        "graph_tokens_per_s": (round(res["tokens"] / (res["graph_gqe_ms"] * 1e-3), 1)
                               if "graph_gqe_ms" in res else None),
        "roofline": roofline_for(wl, res, peaks),
        "measured_peaks": peaks,
        "per_length": [{k: (round(v, 5) if isinstance(v, float) else v) for k, v in r.items()}
                       for r in per_length],
    }
    train = []
    for name in [n for n in args.training.split(",") if n]:
        w2 = W.WORKLOADS[name]
        steps = max(2, min(args.steps, int(2e12 / max(1, stage_work(w2)["attention"][1]) + 2)))
        log(f"[bench] training step {w2.description}: steps {steps}")
        t = measure_training(w2, gqe, torch, steps, 2)
        log(f"[bench]   {t}")
        train.append(t)
    if train:
        line["training"] = train
    if not args.no_sweep:
        log("[bench] expert-pool and per-group-k sweep ...")
        line["sweep"] = measure_sweep(gqe, torch, min(args.steps, 20), 3)
        log("[bench] output constructions of the ablation ...")
        line["ablation"] = measure_ablation(gqe, torch, min(args.steps, 20), 3)
    if not args.no_decode:
        log("[bench] decode step ...")
        line["decode"] = measure_decode(gqe, torch, args.steps, args.warmup)
        log(f"[bench]   decode {line['decode']}")
    if cpu is not None:
        line["cpu_baseline"] = cpu
    elif not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Checks that pin the CPU oracle to facts other than its own code.

Each ``pin_*`` function takes an oracle module and raises AssertionError when
the oracle disagrees with what the pages or the mathematics fix.  They are run
on the real oracle (tests/test_oracle_pins.py) and on copies with planted
mistakes (tests/test_oracle_mutations.py), which each must fail at least one.

Sources: the pages about "Grouped Query Experts: Mixture-of-Experts on GQA
Self-Attention" (arXiv 2606.20945): the pptc.cn review (sections 4.2, 5, 7),
the gist.science technical summaries (Architectuur en Routing / Arquitetura e
Roteamento, Experimentele Resultaten) and the hotpaper.ai summary (core idea,
technical approach).
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_layer(rng, B=2, L=7, d=12, G=2, E=3, k=2, dh=4, w_std=0.5):
    """Random float64 weights of a tiny GQE layer ([out, in] layouts)."""
    return dict(
        x=rng.standard_normal((B, L, d)),
        wq=rng.standard_normal(((G * E + 1) * dh, d)) * w_std,
        wk=rng.standard_normal((G * dh, d)) * w_std,
        wv=rng.standard_normal((G * dh, d)) * w_std,
        wr=rng.standard_normal((G * E, d)) * w_std,
        wo=rng.standard_normal((d, (k * G + 2) * dh)) * w_std,
        br=np.zeros(G * E),
        G=G, E=E, k=k, dh=dh)


def run(orc, t, **kw):
    args = dict(shared_kv_group=0)
    args.update(kw)
    return orc.gqe_forward(t["x"], t["wq"], t["wk"], t["wv"], t["wr"], t["wo"], t["br"],
                           t["G"], t["E"], t["k"], t["dh"], **args)


# ---------------------------------------------------------------------------
# P1: k = E with a uniform router reduces to dense GQA
# ---------------------------------------------------------------------------

def pin_k_equals_e_is_dense_gqa(orc):
    """k=E, W_r=0 (uniform p, ties in index order), shared and weighted rows of
    W_O zeroed  =>  the GQE layer equals dense GQA with W_O^dense = the hard-slot
    columns of W_O (the all-active GQA comparison model, pptc.cn section 4.2)."""
    rng = np.random.default_rng(11)
    for (G, E) in [(2, 3), (3, 2)]:
        t = tiny_layer(rng, G=G, E=E, k=E)
        t["wr"] = np.zeros_like(t["wr"])
        dh = t["dh"]
        wo = t["wo"].copy()
        wo[:, G * E * dh:] = 0.0
        t["wo"] = wo
        y = run(orc, t)["y"]
        ref = orc.gqa_forward(t["x"], t["wq"][:G * E * dh], t["wk"], t["wv"],
                              wo[:, :G * E * dh], G, E, dh)["y"]
        assert np.allclose(y, ref, rtol=0, atol=1e-12), np.abs(y - ref).max()


# ---------------------------------------------------------------------------
# P2, P9, P11: renormalized weights
# ---------------------------------------------------------------------------

def pin_weights_sum_to_one(orc):
    """Per (token, group) the k renormalized weights are >= 0 and sum to 1;
    with k = 1 every weight is exactly 1 (hotpaper.ai: renormalized scoring)."""
    rng = np.random.default_rng(12)
    t = tiny_layer(rng)
    out = run(orc, t)
    w = out["w"]
    assert (w >= 0).all()
    assert np.abs(w.sum(-1) - 1.0).max() <= 1e-15
    # the softmax itself is taken inside each group (pptc.cn section 7)
    assert np.abs(out["p"].sum(-1) - 1.0).max() <= 1e-15
    t1 = tiny_layer(rng, k=1)
    w1 = run(orc, t1)["w"]
    assert (w1 == 1.0).all()


def pin_weights_closed_form(orc):
    """softmax then top-k then renormalize equals a softmax over the selected
    logits alone (the common denominator cancels)."""
    rng = np.random.default_rng(13)
    t = tiny_layer(rng, E=4, k=3)
    out = run(orc, t)
    r, idx, w = out["r"], out["idx"], out["w"]
    rs = np.take_along_axis(r, idx.astype(np.int64), axis=-1)
    e = np.exp(rs - rs.max(-1, keepdims=True))
    assert np.allclose(w, e / e.sum(-1, keepdims=True), rtol=0, atol=1e-15)


def pin_logit_shift_invariance(orc):
    """Adding one constant to every logit of a group (through b_r) changes
    neither the selection nor the weights (softmax inside the group)."""
    rng = np.random.default_rng(14)
    t = tiny_layer(rng, E=4, k=2)
    a = run(orc, t)
    t2 = dict(t)
    shift = np.repeat(rng.standard_normal(t["G"]) * 3.0, t["E"])
    t2["br"] = t["br"] + shift
    b = run(orc, t2)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.allclose(a["w"], b["w"], rtol=0, atol=1e-14)
    assert np.allclose(a["y"], b["y"], rtol=0, atol=1e-12)


def pin_bias_selects(orc):
    """A large router bias on one expert of one group makes it the first
    choice of every token in that group, and only in that group."""
    rng = np.random.default_rng(15)
    t = tiny_layer(rng, G=3, E=4, k=2)
    G, E = t["G"], t["E"]
    br = np.zeros(G * E)
    br[1 * E + 2] = 100.0                        # group 1, expert 2
    t["br"] = br
    out = run(orc, t)
    assert (out["idx"][:, :, 1, 0] == 2).all()
    for g in (0, 2):
        assert not (out["idx"][:, :, g, 0] == 2).all()


# ---------------------------------------------------------------------------
# P3: top-k inside the group
# ---------------------------------------------------------------------------

def pin_topk_brute_force(orc):
    """Against enumeration of every k-subset: the selected set has the
    largest total probability, entries are distinct, in range and in
    descending-p order, and no unselected expert beats a selected one
    (pptc.cn section 5: top-k inside every fixed group)."""
    rng = np.random.default_rng(16)
    t = tiny_layer(rng, B=2, L=9, G=3, E=5, k=2)
    out = run(orc, t)
    p, idx = out["p"], out["idx"]
    B, L, G, E = p.shape
    k = idx.shape[-1]
    for b, l, g in itertools.product(range(B), range(L), range(G)):
        sel = [int(v) for v in idx[b, l, g]]
        assert len(set(sel)) == k and all(0 <= v < E for v in sel)
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(p[b, l, g, list(c)]))
        assert set(best) == set(sel)
        ps = p[b, l, g, sel]
        assert all(ps[i] >= ps[i + 1] for i in range(k - 1))
        rest = [e for e in range(E) if e not in sel]
        assert all(p[b, l, g, e] <= ps.min() for e in rest)


def pin_tie_rule(orc):
    """Exact ties go to the lower expert index: with W_r = 0 every group picks
    experts 0..k-1 in that order; with integer-valued inputs and two equal
    best rows, the lower of the two is ranked first."""
    rng = np.random.default_rng(17)
    t = tiny_layer(rng, G=2, E=4, k=3)
    t["wr"] = np.zeros_like(t["wr"])
    idx = run(orc, t)["idx"]
    assert (idx == np.arange(3)[None, None, None, :]).all()
    # integer-valued: every partial sum is exact in any order
    t = tiny_layer(rng, G=2, E=4, k=2)
    t["x"] = np.abs(rng.integers(1, 4, t["x"].shape)).astype(np.float64)
    wr = rng.integers(-3, 1, t["wr"].shape).astype(np.float64)   # all rows <= 0 ...
    wr[0 * 4 + 3] = 2.0                                            # ... group 0: experts 1 and 3 tie on top
    wr[0 * 4 + 1] = 2.0
    wr[1 * 4 + 0] = 1.0                                            # group 1: experts 0 and 2 tie on top
    wr[1 * 4 + 2] = 1.0
    t["wr"] = wr
    idx = run(orc, t)["idx"]
    assert (idx[:, :, 0, 0] == 1).all() and (idx[:, :, 0, 1] == 3).all()
    assert (idx[:, :, 1, 0] == 0).all() and (idx[:, :, 1, 1] == 2).all()


def pin_exact_logits_keep_the_bias(orc):
    """Near-ties are decided on exactly rounded logits, and those include the
    router bias.  Experts 1 and 2 of group 0 have identical router rows, so
    their products with x tie exactly; a bias of 2^-44 on expert 2 (a gap far
    below the 1e-12 margin that sends the token to the exact path) must rank
    it first, and expert 1 second.  In group 1 the two rows differ by one
    element so that expert 1's dot product is larger by exactly 2^-40, and a
    bias of 2^-39 on expert 2 overturns it.  Inputs are dyadic, so every
    product and every sum here is exact."""
    rng = np.random.default_rng(19)
    t = tiny_layer(rng, B=1, L=5, d=12, G=2, E=4, k=2)
    E = t["E"]
    x = rng.integers(1, 4, t["x"].shape).astype(np.float64)         # positive integers
    wr = rng.integers(-8, -3, t["wr"].shape).astype(np.float64) / 8.0
    wr[0 * E + 1] = wr[0 * E + 2] = 0.5                              # group 0: exact tie
    wr[1 * E + 1] = wr[1 * E + 2] = 0.5                              # group 1 ...
    wr[1 * E + 1, 0] += 2.0 ** -40 / x[0, 0, 0]                      # ... expert 1 ahead by 2^-40 at t=0
    br = np.zeros(t["G"] * E)
    br[0 * E + 2] = 2.0 ** -44
    br[1 * E + 2] = 2.0 ** -39
    t.update(x=x, wr=wr, br=br)
    idx = run(orc, t)["idx"]
    assert (idx[0, :, 0, 0] == 2).all() and (idx[0, :, 0, 1] == 1).all(), idx[0, :, 0]
    assert idx[0, 0, 1, 0] == 2 and idx[0, 0, 1, 1] == 1, idx[0, 0, 1]


# ---------------------------------------------------------------------------
# P5, P10: dispatch lists
# ---------------------------------------------------------------------------

def pin_dispatch_lists(orc):
    """Per (b, g): counts sum to k*L; each list is strictly ascending; offsets
    are the exclusive prefix sum in (b, g, e) order; (pos, slot) rebuild idx."""
    rng = np.random.default_rng(18)
    t = tiny_layer(rng, B=3, L=11, G=2, E=4, k=2)
    out = run(orc, t)
    idx, counts, offsets, pos, slot = (out[n] for n in ("idx", "counts", "offsets", "pos", "slot"))
    B, L, G, k = idx.shape
    E = counts.shape[-1]
    assert (counts.sum(-1) == k * L).all()
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts.reshape(-1))
    rebuilt = np.full_like(idx, -1)
    for b, g, e in itertools.product(range(B), range(G), range(E)):
        li = (b * G + g) * E + e
        ps = pos[offsets[li]:offsets[li + 1]]
        js = slot[offsets[li]:offsets[li + 1]]
        assert (np.diff(ps) > 0).all()
        assert ((0 <= js) & (js < k)).all()
        rebuilt[b, ps, g, js] = e
    assert np.array_equal(rebuilt, idx)


def pin_active_query_ratio(orc):
    """Every routing dispatches exactly k rows per (token, group), so the
    causal attention work over the dispatched rows is sum_t (t+1) per row,
    k*L(L+1)/2 per (b, g); with the always-on head the layer runs k*G+1 query
    heads per token.  The pages' main setting (16 query heads, 8 KV groups,
    k=1, one shared head) gives 9 of 16 active (tests/golden)."""
    with open(os.path.join(GOLDEN, "active_query_heads.json")) as f:
        gold = json.load(f)
    rng = np.random.default_rng(19)
    t = tiny_layer(rng, B=2, L=13, G=2, E=4, k=2)
    t["br"] = np.tile([2.0, 0.0, -1.0, -4.0], 2)           # skewed loads
    out = run(orc, t)
    counts, offsets, pos = out["counts"], out["offsets"], out["pos"]
    B, L, G, k = out["idx"].shape
    E = counts.shape[-1]
    for b, g in itertools.product(range(B), range(G)):
        lo = offsets[(b * G + g) * E]
        hi = offsets[(b * G + g) * E + E]
        assert int((pos[lo:hi] + 1).sum()) == k * L * (L + 1) // 2
    for case in gold["cases"]:
        Gc, Ec, kc = case["kv_groups"], case["query_heads"] // case["kv_groups"], case["top_k"]
        active = kc * Gc + 1
        assert active == case["active_query_heads"]
        assert active * case["ratio"][1] == case["query_heads"] * case["ratio"][0]
        Lc = 4096
        gqe = orc.attention_flops(1, Lc, active, 64)
        gqa = orc.attention_flops(1, Lc, Gc * Ec, 64)
        assert gqe * case["ratio"][1] == gqa * case["ratio"][0]
        assert gqa == 2 * 2 * 64 * Gc * Ec * Lc * (Lc + 1) // 2


# ---------------------------------------------------------------------------
# P4, P7: attention against brute force and a library routine
# ---------------------------------------------------------------------------

def _loop_attention(q, K, V, t, scale):
    """Scalar loops: o = sum_{s<=t} exp(a_s - max a) V_s / sum exp(a_s - max a)."""
    a = [scale * sum(q[i] * K[s, i] for i in range(len(q))) for s in range(t + 1)]
    m = max(a)
    e = [math.exp(v - m) for v in a]
    z = sum(e)
    return np.array([sum(e[s] * V[s, c] for s in range(t + 1)) / z for c in range(V.shape[1])])


def pin_attention_brute_force(orc):
    """Every slot-head row of a tiny layer equals a scalar-loop causal
    attention over its own group's K/V, 1e-12."""
    rng = np.random.default_rng(20)
    t = tiny_layer(rng, B=1, L=6, G=2, E=3, k=2, dh=3)
    out = run(orc, t)
    q, o, K, V = out["q"], out["o"], out["k_"], out["v"]
    G, k, dh = t["G"], t["k"], t["dh"]
    scale = 1.0 / math.sqrt(dh)
    for tt in range(6):
        for g in range(G):
            for j in range(k):
                ref = _loop_attention(q[0, tt, g * k + j], K[0, g], V[0, g], tt, scale)
                assert np.allclose(o[0, tt, g * k + j], ref, rtol=0, atol=1e-12)
        ref = _loop_attention(q[0, tt, G * k], K[0, 0], V[0, 0], tt, scale)
        assert np.allclose(o[0, tt, G * k], ref, rtol=0, atol=1e-12)


def pin_sdpa_cross_check(orc):
    """The dense GQA path, and the GQE slot-heads, equal PyTorch's CPU
    scaled_dot_product_attention in float64 with is_causal=True."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(21)
    t = tiny_layer(rng, B=2, L=9, G=2, E=3, k=2, dh=4)
    G, E, k, dh = t["G"], t["E"], t["k"], t["dh"]
    dense = orc.gqa_forward(t["x"], t["wq"][:G * E * dh], t["wk"], t["wv"],
                            t["wo"][:, :G * E * dh], G, E, dh)
    x = torch.from_numpy(t["x"])
    q = (x @ torch.from_numpy(t["wq"][:G * E * dh]).T).view(2, 9, G * E, dh).transpose(1, 2)
    kk = (x @ torch.from_numpy(t["wk"]).T).view(2, 9, G, dh).transpose(1, 2)
    vv = (x @ torch.from_numpy(t["wv"]).T).view(2, 9, G, dh).transpose(1, 2)
    kk = kk.repeat_interleave(E, dim=1).contiguous()
    vv = vv.repeat_interleave(E, dim=1).contiguous()
    ref = F.scaled_dot_product_attention(q.contiguous(), kk, vv, is_causal=True)
    assert np.allclose(dense["o"], ref.transpose(1, 2).numpy(), rtol=0, atol=1e-12)
    out = run(orc, t, shared_kv_group=1)
    qs = torch.from_numpy(out["q"]).transpose(1, 2).contiguous()        # [B, kG+1, L, dh]
    grp = [g for g in range(G) for _ in range(k)] + [1]
    kg = torch.from_numpy(out["k_"])[:, grp].contiguous()
    vg = torch.from_numpy(out["v"])[:, grp].contiguous()
    ref = F.scaled_dot_product_attention(qs, kg, vg, is_causal=True)
    assert np.allclose(out["o"], ref.transpose(1, 2).numpy(), rtol=0, atol=1e-12)
    assert np.allclose(out["k_"][:, 1], kk[:, E].numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P6: closed form at the first position
# ---------------------------------------------------------------------------

def pin_first_position_closed_form(orc):
    """At t = 0 a token attends only to itself, so every slot is that group's
    V[0]: y[b, 0] = [V_0 (k times), ..., V_{G-1} (k times), V_shared, sum_g V_g] W_O^T,
    whatever W_q and W_r are."""
    rng = np.random.default_rng(22)
    t = tiny_layer(rng, B=2, L=5, G=3, E=3, k=2)
    G, k, dh = t["G"], t["k"], t["dh"]
    for shared in (0, 2):
        y0 = run(orc, t, shared_kv_group=shared)["y"][:, 0]
        for b in range(2):
            v0 = np.array([t["x"][b, 0] @ t["wv"][g * dh:(g + 1) * dh].T for g in range(G)])
            slots = [v0[g] for g in range(G) for _ in range(k)] + [v0[shared], v0.sum(0)]
            ref = np.concatenate(slots) @ t["wo"].T
            assert np.allclose(y0[b], ref, rtol=0, atol=1e-12), np.abs(y0[b] - ref).max()
        t2 = dict(t)
        t2["wq"] = rng.standard_normal(t["wq"].shape)
        t2["wr"] = rng.standard_normal(t["wr"].shape)
        assert np.allclose(run(orc, t2, shared_kv_group=shared)["y"][:, 0], y0, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P8, P12, causality
# ---------------------------------------------------------------------------

def pin_expert_permutation(orc):
    """Relabelling the experts inside a group (their W_q rows, W_r rows and
    b_r entries together) leaves y unchanged when hard slots are in rank
    order; it only renames idx."""
    rng = np.random.default_rng(23)
    t = tiny_layer(rng, B=1, L=8, G=2, E=4, k=2)
    t["br"] = rng.standard_normal(t["br"].shape)
    G, E, dh = t["G"], t["E"], t["dh"]
    a = run(orc, t)
    perm = [rng.permutation(E) for _ in range(G)]
    wq, wr, br = t["wq"].copy(), t["wr"].copy(), t["br"].copy()
    for g in range(G):
        for e in range(E):
            src = g * E + perm[g][e]
            wq[(g * E + e) * dh:(g * E + e + 1) * dh] = t["wq"][src * dh:(src + 1) * dh]
            wr[g * E + e] = t["wr"][src]
            br[g * E + e] = t["br"][src]
    t2 = dict(t, wq=wq, wr=wr, br=br)
    b = run(orc, t2)
    assert np.allclose(a["y"], b["y"], rtol=0, atol=1e-12)
    for g in range(G):                       # new expert e is old expert perm[g][e]
        assert np.array_equal(perm[g][b["idx"][..., g, :]], a["idx"][..., g, :])


def pin_value_scaling(orc):
    """y is linear in W_v: scaling W_v by alpha scales y by alpha."""
    rng = np.random.default_rng(24)
    t = tiny_layer(rng)
    a = run(orc, t)["y"]
    b = run(orc, dict(t, wv=t["wv"] * -2.5))["y"]
    assert np.allclose(b, -2.5 * a, rtol=0, atol=1e-12)


def pin_causality(orc):
    """Changing tokens after position t leaves y at positions <= t unchanged
    (causal prefill), and changing the token at t changes y at t."""
    rng = np.random.default_rng(25)
    t = tiny_layer(rng, B=1, L=9)
    a = run(orc, t)["y"]
    x2 = t["x"].copy()
    x2[:, 5:] = rng.standard_normal(x2[:, 5:].shape)
    b = run(orc, dict(t, x=x2))["y"]
    assert np.allclose(a[:, :5], b[:, :5], rtol=0, atol=1e-12)
    assert not np.allclose(a[:, 5], b[:, 5], rtol=0, atol=1e-6)


def pin_sampled_rows_match_full(orc):
    """Computing only some positions gives the same rows as the full layer."""
    rng = np.random.default_rng(26)
    t = tiny_layer(rng, B=2, L=10)
    full = run(orc, t)
    rows = np.array([0, 3, 4, 9])
    part = run(orc, t, positions=rows)
    assert np.allclose(full["y"][:, rows], part["y"], rtol=0, atol=1e-13)
    assert np.array_equal(full["idx"], part["idx"])



# ---------------------------------------------------------------------------
# Ablation output constructions ([pptc] section 4.3)
# ---------------------------------------------------------------------------

def pin_ablation_constructions(orc):
    """The "hard" construction is the full layer's hard slots alone: with the
    shared and weighted columns of W_O zeroed the full layer gives the same y
    (and the shared head contributes nothing).  With W_r = 0 every in-group
    probability is 1/E, so "weighted_concat" is "hard" divided by E (not by k,
    which renormalized weights would give).  At t = 0 both reduce to each
    group's V[0], scaled by p in "weighted_concat"."""
    rng = np.random.default_rng(31)
    t = tiny_layer(rng, B=2, L=6, G=2, E=3, k=2)
    G, E, k, dh = t["G"], t["E"], t["k"], t["dh"]
    kG = k * G
    wo_hard = t["wo"][:, :kG * dh].copy()
    full_zeroed = dict(t)
    full_zeroed["wo"] = t["wo"].copy()
    full_zeroed["wo"][:, kG * dh:] = 0.0
    y_full = run(orc, full_zeroed)["y"]
    th = dict(t)
    th["wo"] = wo_hard
    hard = run(orc, th, output_mode="hard")
    assert hard["s"].shape[-1] == kG * dh and hard["q"].shape[2] == kG
    assert np.allclose(hard["y"], y_full, rtol=0, atol=1e-12)

    t0 = dict(th)
    t0["wr"] = np.zeros_like(t["wr"])
    t0["br"] = np.zeros_like(t["br"])
    y_h = run(orc, t0, output_mode="hard")["y"]
    y_w = run(orc, t0, output_mode="weighted_concat")["y"]
    assert np.allclose(y_w, y_h / E, rtol=0, atol=1e-12)

    t1 = dict(th)
    t1["br"] = rng.standard_normal(t["br"].shape)
    res = run(orc, t1, output_mode="weighted_concat")
    for b in range(2):
        v0 = [t["x"][b, 0] @ t["wv"][g * dh:(g + 1) * dh].T for g in range(G)]
        r0 = t["x"][b, 0] @ t["wr"].T + t1["br"]
        slots = []
        for g in range(G):
            rg = r0[g * E:(g + 1) * E]
            pg = np.exp(rg - rg.max()) / np.exp(rg - rg.max()).sum()
            order = sorted(range(E), key=lambda e: (-rg[e], e))[:k]
            slots += [pg[e] * v0[g] for e in order]
        ref = np.concatenate(slots) @ wo_hard.T
        assert np.allclose(res["y"][b, 0], ref, rtol=0, atol=1e-12), np.abs(res["y"][b, 0] - ref).max()



# ---------------------------------------------------------------------------
# Decode: one token against a KV cache is the prefill layer's row
# ---------------------------------------------------------------------------

def pin_decode_step_is_prefill_row(orc):
    """With the cache holding K/V of positions < t (anything after t), a decode
    step on x[b, t] gives the prefill layer's y[b, t], its routing, and the
    prefill K/V row t written into the cache; for every output construction
    and for dense GQA."""
    rng = np.random.default_rng(41)
    t_ = tiny_layer(rng, B=2, L=9, G=2, E=3, k=2)
    G, E, k, dh = t_["G"], t_["E"], t_["k"], t_["dh"]
    B, L = t_["x"].shape[:2]
    pos = np.array([8, 3])
    K = np.stack([orc.kv_project(t_["x"][b], t_["wk"], G, dh, L) for b in range(B)])
    V = np.stack([orc.kv_project(t_["x"][b], t_["wv"], G, dh, L) for b in range(B)])
    kc = rng.standard_normal((B, G, 12, dh))
    vc = rng.standard_normal((B, G, 12, dh))
    for b in range(B):
        kc[b, :, :pos[b]] = K[b, :, :pos[b]]
        vc[b, :, :pos[b]] = V[b, :, :pos[b]]
    x_t = np.stack([t_["x"][b, pos[b]] for b in range(B)])
    for mode in ("full", "hard", "weighted_concat"):
        tm = dict(t_)
        if mode != "full":
            tm["wo"] = t_["wo"][:, :k * G * dh]
        pre = run(orc, tm, output_mode=mode)
        dec = orc.gqe_decode_step(x_t, kc, vc, pos, tm["wq"], tm["wk"], tm["wv"], tm["wr"], tm["wo"],
                                  tm["br"], G, E, k, dh, output_mode=mode)
        for b in range(B):
            assert np.array_equal(dec["idx"][b], pre["idx"][b, pos[b]])
            assert np.allclose(dec["y"][b], pre["y"][b, pos[b]], rtol=0, atol=1e-12), mode
            assert np.allclose(dec["k_cache"][b, :, pos[b]], K[b, :, pos[b]], rtol=0, atol=1e-12)
            assert np.allclose(dec["v_cache"][b, :, :pos[b] + 1], V[b, :, :pos[b] + 1], rtol=0, atol=1e-12)
    wq_d = t_["wq"][:G * E * dh]
    wo_d = rng.standard_normal((t_["x"].shape[2], G * E * dh))
    pre = orc.gqa_forward(t_["x"], wq_d, t_["wk"], t_["wv"], wo_d, G, E, dh)
    dec = orc.gqa_decode_step(x_t, kc, vc, pos, wq_d, t_["wk"], t_["wv"], wo_d, G, E, dh)
    for b in range(B):
        assert np.allclose(dec["y"][b], pre["y"][b, pos[b]], rtol=0, atol=1e-12)



# ---------------------------------------------------------------------------
# RoPE option (RoFormer, Su et al. 2021; the pages are silent on positions)
# ---------------------------------------------------------------------------

def pin_rope_closed_forms(orc):
    """The rotation itself: each pair (2i, 2i+1) read as a complex number is
    multiplied by exp(i t theta_i), theta_i = base^(-2i/d_h) (so the first
    pair turns by t radians at any base); it keeps the norm, is the identity
    at t = 0, and the inverse undoes it."""
    rng = np.random.default_rng(81)
    dh, base = 8, 50.0
    v = rng.standard_normal((5, dh))
    t = np.array([0, 1, 7, 1000, 123457])
    got = orc.rope(v, t, base)
    z = (v[:, 0::2] + 1j * v[:, 1::2]) * np.exp(
        1j * t[:, None] * base ** (-np.arange(dh // 2) * 2.0 / dh))
    assert np.allclose(got[:, 0::2], z.real, rtol=0, atol=1e-12)
    assert np.allclose(got[:, 1::2], z.imag, rtol=0, atol=1e-12)
    assert np.allclose(np.linalg.norm(got, axis=1), np.linalg.norm(v, axis=1), rtol=1e-13)
    assert np.array_equal(got[0], v[0])
    assert np.allclose(orc.rope(got, t, base, inverse=True), v, rtol=0, atol=1e-9)
    assert orc.rope(v, t, 0.0) is v


def pin_rope_relative_positions(orc):
    """With RoPE a score depends on positions only through their difference,
    so a layer whose positions all move by the same offset is unchanged: here
    the attention of the shifted rotations equals the original's, and the
    layer at t = 0 (one key, rotated by 0) equals the layer without RoPE."""
    rng = np.random.default_rng(82)
    dh, base = 8, 30.0
    q = rng.standard_normal((6, dh))
    kk = rng.standard_normal((9, dh))
    v = rng.standard_normal((9, dh))
    tq = np.array([0, 2, 3, 5, 8, 8])
    for shift in (1, 17, 4096):
        a = orc.causal_attention(orc.rope(q, tq, base), tq, orc.rope(kk, np.arange(9), base), v, 0.5)
        b = orc.causal_attention(orc.rope(q, tq + shift, base), tq,
                                 orc.rope(kk, np.arange(9) + shift, base), v, 0.5)
        assert np.allclose(a, b, rtol=0, atol=1e-10)
    t = tiny_layer(rng, B=1, L=6, G=2, E=3, k=2)
    plain = run(orc, t)
    rot = run(orc, t, rope_base=30.0)
    assert np.array_equal(plain["idx"], rot["idx"])
    assert np.allclose(rot["y"][:, 0], plain["y"][:, 0], rtol=0, atol=1e-12)
    assert not np.allclose(rot["y"][:, 1:], plain["y"][:, 1:], rtol=0, atol=1e-6)


def pin_rope_layer_reductions(orc):
    """k = E with a uniform router and the extra W_O rows zeroed is dense GQA
    with RoPE too, and a decode step with RoPE is the RoPE prefill row."""
    rng = np.random.default_rng(83)
    base = 25.0
    G, E = 2, 3
    t = tiny_layer(rng, G=G, E=E, k=E)
    t["wr"] = np.zeros_like(t["wr"])
    dh = t["dh"]
    wo = t["wo"].copy()
    wo[:, G * E * dh:] = 0.0
    t["wo"] = wo
    a = run(orc, t, rope_base=base)
    b = orc.gqa_forward(t["x"], t["wq"][:G * E * dh], t["wk"], t["wv"], wo[:, :G * E * dh], G, E,
                        dh, rope_base=base)
    assert np.allclose(a["y"], b["y"], rtol=0, atol=1e-12)
    t_ = tiny_layer(rng, B=2, L=9, G=2, E=3, k=2)
    G, E, k, dh = t_["G"], t_["E"], t_["k"], t_["dh"]
    B, L = t_["x"].shape[:2]
    pos = np.array([8, 3])
    pre = run(orc, t_, rope_base=base)
    K = pre["k_"]
    V = np.stack([orc.kv_project(t_["x"][b], t_["wv"], G, dh, L) for b in range(B)])
    kc = rng.standard_normal((B, G, 12, dh))
    vc = rng.standard_normal((B, G, 12, dh))
    for b in range(B):
        kc[b, :, :pos[b]] = K[b, :, :pos[b]]
        vc[b, :, :pos[b]] = V[b, :, :pos[b]]
    x_t = np.stack([t_["x"][b, pos[b]] for b in range(B)])
    dec = orc.gqe_decode_step(x_t, kc, vc, pos, t_["wq"], t_["wk"], t_["wv"], t_["wr"], t_["wo"],
                              t_["br"], G, E, k, dh, rope_base=base)
    for b in range(B):
        assert np.allclose(dec["y"][b], pre["y"][b, pos[b]], rtol=0, atol=1e-12)
        assert np.allclose(dec["k_cache"][b, :, pos[b]], K[b, :, pos[b]], rtol=0, atol=1e-12)
    wq_d = t_["wq"][:G * E * dh]
    wo_d = rng.standard_normal((t_["x"].shape[2], G * E * dh))
    pre = orc.gqa_forward(t_["x"], wq_d, t_["wk"], t_["wv"], wo_d, G, E, dh, rope_base=base)
    dec = orc.gqa_decode_step(x_t, kc, vc, pos, wq_d, t_["wk"], t_["wv"], wo_d, G, E, dh,
                              rope_base=base)
    for b in range(B):
        assert np.allclose(dec["y"][b], pre["y"][b, pos[b]], rtol=0, atol=1e-12)


def pin_rope_backward_finite_differences(orc):
    """Central differences of <y, dy> + alpha * L_aux agree with the RoPE
    backward on x, W_q and W_k (the inputs the rotation's transpose reaches)
    and W_O, for GQE and dense GQA."""
    rng = np.random.default_rng(84)
    h, base, alpha = 1e-6, 20.0, 0.3
    t = tiny_layer(rng, B=1, L=6, d=6, G=2, E=3, k=2, dh=4)
    t["br"] = rng.standard_normal(t["G"] * t["E"]) * 0.3
    f0 = run(orc, t, rope_base=base)
    srt = -np.sort(-f0["r"], axis=-1)
    assert (srt[..., :-1] - srt[..., 1:]).min() > 1e-3, "seed too close to a routing tie"
    dy = rng.standard_normal(f0["y"].shape)
    g = orc.gqe_backward(t["x"], t["wq"], t["wk"], t["wv"], t["wr"], t["wo"], t["br"], dy,
                         t["G"], t["E"], t["k"], t["dh"], aux_weight=alpha, rope_base=base)
    for name, key in (("x", "dx"), ("wq", "dwq"), ("wk", "dwk"), ("wo", "dwo")):
        flat = t[name].reshape(-1)
        for i in rng.choice(flat.size, size=min(flat.size, 20), replace=False):
            old = flat[i]
            flat[i] = old + h
            lp = _total_loss(orc, t, dy, alpha, rope_base=base)
            flat[i] = old - h
            lm = _total_loss(orc, t, dy, alpha, rope_base=base)
            flat[i] = old
            num = (lp - lm) / (2 * h)
            assert abs(num - g[key].reshape(-1)[i]) <= 1e-6 * (1.0 + abs(num)), (name, i)
    wq_d = t["wq"][:6 * 4].copy()
    wo_d = rng.standard_normal((6, 6 * 4))
    dy = rng.standard_normal((1, 6, 6))
    g = orc.gqa_backward(t["x"], wq_d, t["wk"], t["wv"], wo_d, dy, 2, 3, 4, rope_base=base)
    for arr, key in ((t["x"], "dx"), (wq_d, "dwq"), (t["wk"], "dwk")):
        flat = arr.reshape(-1)
        for i in rng.choice(flat.size, size=min(flat.size, 12), replace=False):
            old = flat[i]
            flat[i] = old + h
            lp = float((orc.gqa_forward(t["x"], wq_d, t["wk"], t["wv"], wo_d, 2, 3, 4,
                                        rope_base=base)["y"] * dy).sum())
            flat[i] = old - h
            lm = float((orc.gqa_forward(t["x"], wq_d, t["wk"], t["wv"], wo_d, 2, 3, 4,
                                        rope_base=base)["y"] * dy).sum())
            flat[i] = old
            num = (lp - lm) / (2 * h)
            assert abs(num - g[key].reshape(-1)[i]) <= 1e-6 * (1.0 + abs(num)), ("gqa", key, i)


# ---------------------------------------------------------------------------
# backward: the gradients are those of the forward (finite differences), and
# they respect the invariances of the layer
# ---------------------------------------------------------------------------

def _total_loss(orc, t, dy, alpha, **kw):
    """<y, dy> + alpha * L_aux, the scalar whose gradients the backward returns."""
    f = run(orc, t, **kw)
    aux = orc.load_balance_loss(f["p"], f["idx"], t["E"])[0]
    return float((f["y"] * dy).sum()) + alpha * aux


def pin_backward_finite_differences(orc):
    """Central differences of <y, dy> + alpha * L_aux agree with the backward on
    every parameter tensor and on x, for every output construction (the
    weighted slot is the router's differentiable path, gist.science Training
    en Loss), with a non-default shared group and scale; and for dense GQA."""
    rng = np.random.default_rng(57)
    h = 1e-6
    for mode, kw in (("full", dict(shared_kv_group=1, scale=0.7)), ("hard", {}),
                     ("weighted_concat", {})):
        t = tiny_layer(rng, B=2, L=5, d=6, G=2, E=3, k=2, dh=4)
        t["br"] = rng.standard_normal(t["G"] * t["E"]) * 0.3
        if mode != "full":
            t["wo"] = np.ascontiguousarray(t["wo"][:, :t["k"] * t["G"] * t["dh"]])
        f0 = run(orc, t, output_mode=mode, **kw)
        srt = -np.sort(-f0["r"], axis=-1)
        assert (srt[..., :-1] - srt[..., 1:]).min() > 1e-3, "seed too close to a routing tie"
        dy = rng.standard_normal(f0["y"].shape)
        alpha = 0.3
        g = orc.gqe_backward(t["x"], t["wq"], t["wk"], t["wv"], t["wr"], t["wo"], t["br"], dy,
                             t["G"], t["E"], t["k"], t["dh"], output_mode=mode,
                             aux_weight=alpha, **kw)
        for name, key in (("x", "dx"), ("wq", "dwq"), ("wk", "dwk"), ("wv", "dwv"),
                          ("wr", "dwr"), ("br", "dbr"), ("wo", "dwo")):
            arr = t[name]
            flat = arr.reshape(-1)
            for i in rng.choice(flat.size, size=min(flat.size, 24), replace=False):
                old = flat[i]
                flat[i] = old + h
                lp = _total_loss(orc, t, dy, alpha, output_mode=mode, **kw)
                flat[i] = old - h
                lm = _total_loss(orc, t, dy, alpha, output_mode=mode, **kw)
                flat[i] = old
                num = (lp - lm) / (2 * h)
                ana = g[key].reshape(-1)[i]
                assert abs(num - ana) <= 1e-6 * (1.0 + abs(num)), (mode, name, i, num, ana)
    # dense GQA
    t = tiny_layer(rng, B=1, L=6, d=6, G=2, E=2, k=1, dh=4)
    wq_d = t["wq"][:4 * 4].copy()
    wo_d = rng.standard_normal((6, 4 * 4))
    dy = rng.standard_normal((1, 6, 6))
    g = orc.gqa_backward(t["x"], wq_d, t["wk"], t["wv"], wo_d, dy, 2, 2, 4)
    for arr, key in ((t["x"], "dx"), (wq_d, "dwq"), (t["wk"], "dwk"), (t["wv"], "dwv"),
                     (wo_d, "dwo")):
        flat = arr.reshape(-1)
        for i in rng.choice(flat.size, size=min(flat.size, 16), replace=False):
            old = flat[i]
            flat[i] = old + h
            lp = float((orc.gqa_forward(t["x"], wq_d, t["wk"], t["wv"], wo_d, 2, 2, 4)["y"] * dy).sum())
            flat[i] = old - h
            lm = float((orc.gqa_forward(t["x"], wq_d, t["wk"], t["wv"], wo_d, 2, 2, 4)["y"] * dy).sum())
            flat[i] = old
            num = (lp - lm) / (2 * h)
            assert abs(num - g[key].reshape(-1)[i]) <= 1e-6 * (1.0 + abs(num)), ("gqa", key, i)


def pin_backward_invariances(orc):
    """Shifting every key of a group by one vector, or every logit of a (token,
    group) by one constant, leaves y unchanged, so the key gradient of each
    group sums to zero over positions and the logit gradient of each (token,
    group) sums to zero over experts.  With dy = 0 and a uniform router
    (ties to the lower index: experts 0..k-1), the auxiliary loss alone gives
    the logit gradient alpha / (G T) * (f_e - 1/E) with f_e = 1/k for e < k."""
    rng = np.random.default_rng(61)
    t = tiny_layer(rng, B=2, L=9, d=8, G=2, E=4, k=2, dh=4)
    f = run(orc, t)
    dy = rng.standard_normal(f["y"].shape)
    g = orc.gqe_backward(t["x"], t["wq"], t["wk"], t["wv"], t["wr"], t["wo"], t["br"], dy,
                         t["G"], t["E"], t["k"], t["dh"], aux_weight=0.2)
    assert np.abs(g["dk"].sum(axis=2)).max() < 1e-9
    assert np.abs(g["dr"].sum(axis=-1)).max() < 1e-12
    assert np.abs(g["dr"]).max() > 1e-3                      # the router does get a gradient
    t["wr"] = np.zeros_like(t["wr"])
    alpha, G, E, k = 0.5, t["G"], t["E"], t["k"]
    T = t["x"].shape[0] * t["x"].shape[1]
    g = orc.gqe_backward(t["x"], t["wq"], t["wk"], t["wv"], t["wr"], t["wo"], t["br"],
                         np.zeros_like(dy), G, E, k, t["dh"], aux_weight=alpha)
    f_e = np.array([1.0 / k if e < k else 0.0 for e in range(E)])
    want = alpha / (G * T) * (f_e - 1.0 / E)
    assert np.allclose(g["dr"], np.broadcast_to(want, g["dr"].shape), rtol=0, atol=1e-15)
    assert abs(g["aux_loss"] - (E / G) * G * sum(f_e / E)) < 1e-12   # = 1 at uniform p


# ---------------------------------------------------------------------------
# non-uniform k per group
# ---------------------------------------------------------------------------

def _run_gk(orc, t, ks, **kw):
    return orc.gqe_forward_group_k(t["x"], t["wq"], t["wk"], t["wv"], t["wr"], t["wo"], t["br"],
                                   t["G"], t["E"], ks, t["dh"], **kw)


def pin_group_k_uniform_is_the_layer(orc):
    """With the same k in every group the per-group layer is the pages' layer:
    routing, dispatch lists and outputs, for every output construction."""
    rng = np.random.default_rng(71)
    for mode in orc.OUTPUT_MODES:
        t = tiny_layer(rng, B=2, L=8, G=3, E=3, k=2)
        if mode != "full":
            t["wo"] = np.ascontiguousarray(t["wo"][:, :t["k"] * t["G"] * t["dh"]])
        a = run(orc, t, output_mode=mode)
        b = _run_gk(orc, t, [t["k"]] * t["G"], output_mode=mode)
        B, L = t["x"].shape[:2]
        assert np.array_equal(b["idx"], a["idx"].reshape(B, L, -1))
        assert np.allclose(b["w"], a["w"].reshape(B, L, -1), rtol=0, atol=1e-15)
        for key in ("counts", "offsets", "pos", "slot"):
            assert np.array_equal(b[key], a[key]), key
        assert np.allclose(b["y"], a["y"], rtol=0, atol=1e-12), mode


def pin_group_k_selection_brute_force(orc):
    """Group g's selection is the best k_g-subset by logit (ties to the lower
    index), in rank order; its weights renormalize over that subset only."""
    rng = np.random.default_rng(73)
    ks = [1, 3, 2]
    t = tiny_layer(rng, B=1, L=6, G=3, E=4, k=2)
    t["wo"] = rng.standard_normal((t["x"].shape[2], (sum(ks) + 2) * t["dh"]))
    f = _run_gk(orc, t, ks)
    koff = [0, 1, 4, 6]
    for tt in range(6):
        for g, kg in enumerate(ks):
            r = f["r"][0, tt, g]
            best = max(itertools.combinations(range(4), kg), key=lambda c: (sum(r[list(c)]), [-i for i in c]))
            got = f["idx"][0, tt, koff[g]:koff[g + 1]]
            assert sorted(got.tolist()) == sorted(best)
            assert all(r[got[i]] >= r[got[i + 1]] for i in range(kg - 1))
            ps = f["p"][0, tt, g][got]
            assert np.allclose(f["w"][0, tt, koff[g]:koff[g + 1]], ps / ps.sum(), rtol=0, atol=1e-15)


def pin_group_k_first_position(orc):
    """At t = 0 every head sees one key: y[0] = [v_g repeated k_g times per
    group | v_shared | sum_g v_g] . W_O^T (the weights of a group sum to 1)."""
    rng = np.random.default_rng(79)
    ks = [3, 1, 2]
    t = tiny_layer(rng, B=1, L=5, G=3, E=3, k=1)
    dh = t["dh"]
    t["wo"] = rng.standard_normal((t["x"].shape[2], (sum(ks) + 2) * dh))
    f = _run_gk(orc, t, ks, shared_kv_group=2)
    x0 = t["x"][0, 0]
    v = (t["wv"] @ x0).reshape(3, dh)
    slots = [v[g] for g in range(3) for _ in range(ks[g])] + [v[2], v.sum(axis=0)]
    want = np.concatenate(slots) @ t["wo"].T
    assert np.allclose(f["y"][0, 0], want, rtol=0, atol=1e-12)

def pin_group_k_decode_step(orc):
    """The per-group decode step is the per-group prefill layer's row t (cache
    holding the prefill K/V of positions < t, anything after), for every output
    construction; with the same k in every group it is the uniform decode step."""
    rng = np.random.default_rng(83)
    ks = [1, 3, 2]
    t_ = tiny_layer(rng, B=2, L=9, G=3, E=3, k=2)
    G, E, dh = t_["G"], t_["E"], t_["dh"]
    B, L, d = t_["x"].shape
    pos = np.array([8, 2])
    K = np.stack([orc.kv_project(t_["x"][b], t_["wk"], G, dh, L) for b in range(B)])
    V = np.stack([orc.kv_project(t_["x"][b], t_["wv"], G, dh, L) for b in range(B)])
    kc = rng.standard_normal((B, G, 12, dh))
    vc = rng.standard_normal((B, G, 12, dh))
    for b in range(B):
        kc[b, :, :pos[b]] = K[b, :, :pos[b]]
        vc[b, :, :pos[b]] = V[b, :, :pos[b]]
    x_t = np.stack([t_["x"][b, pos[b]] for b in range(B)])
    for mode in orc.OUTPUT_MODES:
        width = (sum(ks) + (2 if mode == "full" else 0)) * dh
        wo = rng.standard_normal((d, width))
        pre = orc.gqe_forward_group_k(t_["x"], t_["wq"], t_["wk"], t_["wv"], t_["wr"], wo, t_["br"],
                                      G, E, ks, dh, output_mode=mode)
        dec = orc.gqe_decode_step_group_k(x_t, kc, vc, pos, t_["wq"], t_["wk"], t_["wv"], t_["wr"],
                                          wo, t_["br"], G, E, ks, dh, output_mode=mode)
        for b in range(B):
            assert np.array_equal(dec["idx"][b], pre["idx"][b, pos[b]])
            assert np.allclose(dec["w"][b], pre["w"][b, pos[b]], rtol=0, atol=1e-15)
            assert np.allclose(dec["y"][b], pre["y"][b, pos[b]], rtol=0, atol=1e-12), mode
            assert np.allclose(dec["k_cache"][b, :, pos[b]], K[b, :, pos[b]], rtol=0, atol=1e-12)
    # uniform counts: the pages' decode step
    k = 2
    wo = rng.standard_normal((d, (k * G + 2) * dh))
    a = orc.gqe_decode_step(x_t, kc, vc, pos, t_["wq"], t_["wk"], t_["wv"], t_["wr"], wo, t_["br"],
                            G, E, k, dh)
    g = orc.gqe_decode_step_group_k(x_t, kc, vc, pos, t_["wq"], t_["wk"], t_["wv"], t_["wr"], wo,
                                    t_["br"], G, E, [k] * G, dh)
    assert np.array_equal(g["idx"], a["idx"].reshape(B, -1))
    assert np.allclose(g["y"], a["y"], rtol=0, atol=1e-12)


def pin_group_k_backward(orc):
    """The per-group backward: central differences of <y, dy> + alpha * L_aux
    (f per group over its T*k_g slots) on every parameter tensor and on x, for
    every output construction; with the same k in every group it is the
    pages' backward."""
    rng = np.random.default_rng(89)
    h = 1e-6
    ks = [1, 3, 2]
    for mode, kw in (("full", dict(shared_kv_group=2, scale=0.6)), ("hard", {}),
                     ("weighted_concat", {})):
        t = tiny_layer(rng, B=2, L=5, d=6, G=3, E=3, k=1, dh=4)
        t["br"] = rng.standard_normal(t["G"] * t["E"]) * 0.3
        t["wo"] = rng.standard_normal((6, (sum(ks) + (2 if mode == "full" else 0)) * t["dh"]))
        f0 = _run_gk(orc, t, ks, output_mode=mode, **kw)
        srt = -np.sort(-f0["r"], axis=-1)
        assert (srt[..., :-1] - srt[..., 1:]).min() > 1e-3, "seed too close to a routing tie"
        # f[g] is a share of group g's slots: it sums to one over the experts
        _, fsh, Psh = orc.load_balance_loss_group_k(f0["p"], f0["idx"], t["E"], ks)
        assert np.allclose(fsh.sum(axis=1), 1.0, rtol=0, atol=1e-15)
        assert np.allclose(Psh.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        dy = rng.standard_normal(f0["y"].shape)
        alpha = 0.3
        g = orc.gqe_backward_group_k(t["x"], t["wq"], t["wk"], t["wv"], t["wr"], t["wo"], t["br"],
                                     dy, t["G"], t["E"], ks, t["dh"], output_mode=mode,
                                     aux_weight=alpha, **kw)

        def loss():
            f = _run_gk(orc, t, ks, output_mode=mode, **kw)
            aux = orc.load_balance_loss_group_k(f["p"], f["idx"], t["E"], ks)[0]
            return float((f["y"] * dy).sum()) + alpha * aux
        for name, key in (("x", "dx"), ("wq", "dwq"), ("wk", "dwk"), ("wv", "dwv"),
                          ("wr", "dwr"), ("br", "dbr"), ("wo", "dwo")):
            flat = t[name].reshape(-1)
            for i in rng.choice(flat.size, size=min(flat.size, 16), replace=False):
                old = flat[i]
                flat[i] = old + h
                lp = loss()
                flat[i] = old - h
                lm = loss()
                flat[i] = old
                num = (lp - lm) / (2 * h)
                ana = g[key].reshape(-1)[i]
                assert abs(num - ana) <= 1e-6 * (1.0 + abs(num)), (mode, name, i, num, ana)
    # the same k everywhere: the pages' backward, for every output construction
    for mode in orc.OUTPUT_MODES:
        t = tiny_layer(rng, B=2, L=6, d=6, G=2, E=3, k=2, dh=4)
        if mode != "full":
            t["wo"] = np.ascontiguousarray(t["wo"][:, :t["k"] * t["G"] * t["dh"]])
        dy = rng.standard_normal((2, 6, 6))
        a = orc.gqe_backward(t["x"], t["wq"], t["wk"], t["wv"], t["wr"], t["wo"], t["br"], dy,
                             t["G"], t["E"], t["k"], t["dh"], output_mode=mode, aux_weight=0.2)
        b = orc.gqe_backward_group_k(t["x"], t["wq"], t["wk"], t["wv"], t["wr"], t["wo"], t["br"],
                                     dy, t["G"], t["E"], [t["k"]] * t["G"], t["dh"],
                                     output_mode=mode, aux_weight=0.2)
        for key in ("dx", "dwq", "dwk", "dwv", "dwr", "dbr", "dwo"):
            assert np.allclose(b[key], a[key], rtol=0, atol=1e-12), (mode, key)
        assert abs(b["aux_loss"] - a["aux_loss"]) <= 1e-15


ALL_PINS = [
    pin_k_equals_e_is_dense_gqa,
    pin_weights_sum_to_one,
    pin_weights_closed_form,
    pin_logit_shift_invariance,
    pin_bias_selects,
    pin_topk_brute_force,
    pin_tie_rule,
    pin_exact_logits_keep_the_bias,
    pin_dispatch_lists,
    pin_active_query_ratio,
    pin_attention_brute_force,
    pin_sdpa_cross_check,
    pin_first_position_closed_form,
    pin_expert_permutation,
    pin_value_scaling,
    pin_causality,
    pin_sampled_rows_match_full,
    pin_ablation_constructions,
    pin_decode_step_is_prefill_row,
    pin_rope_closed_forms,
    pin_rope_relative_positions,
    pin_rope_layer_reductions,
    pin_rope_backward_finite_differences,
    pin_backward_finite_differences,
    pin_backward_invariances,
    pin_group_k_uniform_is_the_layer,
    pin_group_k_selection_brute_force,
    pin_group_k_first_position,
    pin_group_k_decode_step,
    pin_group_k_backward,
]

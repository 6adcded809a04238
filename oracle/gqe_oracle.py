"""CPU float64 oracle for the Grouped Query Experts (GQE) attention layer: prefill
forward, decode step and backward.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import or run this module; the product path never does.
It shares no code with the HIP implementation: it is written from the pages
that describe the method, in float64 numpy, plainly and slowly.

Sources (the five pages describe one preprint, arXiv 2606.20945,
"Grouped Query Experts: Mixture-of-Experts on GQA Self-Attention"):

* [pptc]   review on pptc.cn (news/49069): Table 1 and the prefill speed-ups
           (section 4.2), ablation (4.3), related work (5), limitations (6),
           conclusion (7).
* [gist-nl] gist.science/nl technical summary, "Architectuur en Routing",
           "Training en Loss", "Experimentele Resultaten".
* [gist-pt] gist.science/pt technical summary, "Arquitetura e Roteamento".
* [hotpaper] hotpaper.ai summary, "핵심 아이디어" (core idea) and
           "기술적 접근법" (technical approach).

What the layer computes (the plain definition; the method reaches exactly this
result, its sparsity being the routing itself):

1. router logits r[t, g, e] = x[t] . W_r[g*E+e] + b_r[g*E+e]  (a router looks
   at each token and scores the query-head experts of every GQA group;
   [gist-nl] Architectuur en Routing).
2. p[t, g, :] = softmax over the E experts of group g (softmax is taken first,
   inside the group; [pptc] section 7).
3. the k experts with the largest p are selected in every group (top-k within
   each fixed group, every group participates; [pptc] section 5), listed in
   rank order, ties to the lower expert index.
4. w[t, g, j] = p of the j-th selected expert divided by the sum of p over the
   k selected (renormalized scoring; [hotpaper] technical approach).
5. dispatch: for every (b, g, e) the ascending list of positions t that chose
   expert e, with the rank j it was chosen at.
6. K and V are the dense, unchanged GQA projections of group g ([gist-nl]
   Architectuur en Routing: the KV path stays dense).
7. every selected expert (a query head with its own W_q block) attends
   causally to its group's K/V; unselected experts compute nothing ([pptc]
   section 5: a token that skips an expert still attends to that group's KV).
8. one always-on shared head attends for every token ([gist-nl]).
9. the weighted slot is the sum over groups and selected experts of w times
   the expert output ([gist-nl]: a weighted sum of the selected experts'
   outputs using router probabilities).
10. the slot vector [k*G hard slots, shared, weighted] of width (k*G+2)*d_h
    ([hotpaper] core idea: W_O resized to k*G+2 slots) ...
11. ... goes through W_O.

Readings where the pages are silent (each is listed in the design notes):
scale 1/sqrt(d_h); hard slots ordered group-major then by rank; weighted slot
is a plain sum over groups; renormalization is per group; the shared head has
its own W_q rows and reads KV group ``shared_kv_group`` (0); no RoPE, no
projection biases; causal mask s <= t; weights in [out, in] layout.

Ranking on p is done on the logits r: within a group p is proportional to
exp(r), so both orders are the same, and ranking on r avoids ties that
rounding p could create.  Logits whose top-k decision is closer than 1e-12 are
recomputed with an exactly rounded sum (math.fsum of the exact products).
"""
from __future__ import annotations

import math
import time

import numpy as np

# --------------------------------------------------------------------------
# step 1-4: router, in-group softmax, top-k, renormalization
# --------------------------------------------------------------------------


def router_logits(x: np.ndarray, wr: np.ndarray, br: np.ndarray, n_groups: int,
                  n_experts: int) -> np.ndarray:
    """r[T, G, E] = x[T, d] . W_r[G*E, d]^T + b_r  (step 1, [gist-nl])."""
    r = x @ wr.T + br[None, :]
    return r.reshape(x.shape[0], n_groups, n_experts)


def exact_logits(x_row: np.ndarray, wr: np.ndarray, br: np.ndarray) -> np.ndarray:
    """Correctly rounded logits for one token: fsum of the exact products.

    Products of two bf16 or two fp32 values are exact in float64; fsum rounds
    their sum once.
    """
    return np.array([math.fsum(list(x_row * wr[c]) + [float(br[c])])
                     for c in range(wr.shape[0])])


def group_softmax(r: np.ndarray) -> np.ndarray:
    """p = softmax over the experts of each group (step 2, [pptc] section 7)."""
    z = r - r.max(axis=-1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=-1, keepdims=True)


def topk_in_group(r: np.ndarray, top_k: int) -> np.ndarray:
    """idx[..., k]: the k best experts of every group, best first (step 3).

    Order: larger logit first, then lower expert index (a stable sort of the
    negated logits keeps the lower index first among equals).
    """
    order = np.argsort(-r, axis=-1, kind="stable")
    return order[..., :top_k].astype(np.int32)


def renormalize(p: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """w = p[idx] / sum(p[idx]) over the k selected of each group (step 4)."""
    ps = np.take_along_axis(p, idx.astype(np.int64), axis=-1)
    return ps / ps.sum(axis=-1, keepdims=True)


def route(x: np.ndarray, wr: np.ndarray, br: np.ndarray, n_groups: int, n_experts: int,
          top_k: int, exact_margin: float = 1e-12):
    """Steps 1-4 for tokens x[T, d].  Returns (r, p, idx, w), shapes [T,G,E] / [T,G,k].

    Tokens are independent; long inputs are processed in blocks of 65536
    tokens only to bound memory.
    """
    step = 65536
    if x.shape[0] > step:
        parts = [route(x[t0:t0 + step], wr, br, n_groups, n_experts, top_k, exact_margin)
                 for t0 in range(0, x.shape[0], step)]
        return tuple(np.concatenate([prt[i] for prt in parts]) for i in range(4))
    r = router_logits(x, wr, br, n_groups, n_experts)
    # decisions that rounding could flip: recompute those tokens exactly
    srt = -np.sort(-r, axis=-1)
    m = min(top_k, n_experts - 1)                         # rank gaps that decide idx
    gaps = srt[..., :m] - srt[..., 1:m + 1]
    close = (gaps < exact_margin * (1.0 + np.abs(srt[..., :m]))).any(axis=(-1, -2))
    for t in np.nonzero(close)[0]:
        r[t] = exact_logits(x[t], wr, br).reshape(n_groups, n_experts)
    p = group_softmax(r)
    idx = topk_in_group(r, top_k)
    w = renormalize(p, idx)
    return r, p, idx, w


# --------------------------------------------------------------------------
# step 5: dispatch lists
# --------------------------------------------------------------------------


def dispatch(idx: np.ndarray, n_experts: int):
    """Per-(b, g, e) token lists (step 5, [pptc] section 6: sparse scheduling).

    idx is int [B, L, G, k].  Returns counts int32 [B, G, E]; offsets int32
    [B*G*E+1] (exclusive prefix sum of counts in (b, g, e) row-major order);
    pos and slot, int32 [B*L*G*k]: for list (b, g, e), entries
    offsets[(b*G+g)*E+e] onwards hold the positions t that selected e, in
    ascending order, and the rank j at which they selected it.
    """
    B, L, G, k = idx.shape
    counts = np.zeros((B, G, n_experts), dtype=np.int32)
    pos_lists, slot_lists = [], []
    for b in range(B):
        for g in range(G):
            for e in range(n_experts):
                hit = idx[b, :, g, :] == e              # [L, k]
                t_sel, j_sel = np.nonzero(hit)           # row-major: ascending t
                counts[b, g, e] = t_sel.size
                pos_lists.append(t_sel)
                slot_lists.append(j_sel)
    offsets = np.zeros(B * G * n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts.reshape(-1))
    pos = np.concatenate(pos_lists).astype(np.int32)
    slot = np.concatenate(slot_lists).astype(np.int32)
    return counts, offsets.astype(np.int32), pos, slot


# --------------------------------------------------------------------------
# steps 6-8: projections and causal attention
# --------------------------------------------------------------------------


def head_rows(w: np.ndarray, head: int, head_dim: int) -> np.ndarray:
    """The d_h rows of an [out, in] projection that belong to one head."""
    return w[head * head_dim:(head + 1) * head_dim]


def kv_project(x_b: np.ndarray, w: np.ndarray, n_groups: int, head_dim: int,
               upto: int) -> np.ndarray:
    """Dense K (or V) of every group for positions < upto: [G, upto, d_h] (step 6)."""
    out = np.empty((n_groups, upto, head_dim))
    step = 32768
    for t0 in range(0, upto, step):
        t1 = min(upto, t0 + step)
        blk = x_b[t0:t1] @ w.T                           # [n, G*d_h]
        out[:, t0:t1] = blk.reshape(t1 - t0, n_groups, head_dim).transpose(1, 0, 2)
    return out


# Rotary position embedding, an option the pages do not name (they are silent
# on position encoding; a model of this size would normally use one).  The
# form is that of RoFormer (Su et al., 2021) with interleaved pairs: in every
# query head and every key head, the pair of dims (2i, 2i+1) of the vector at
# position t is rotated by the angle t * theta_i, theta_i = base^(-2i/d_h).
# It is applied to the projected queries and keys, never to the values, so
# every score depends on positions only through their difference.  base 0
# means no rotation (the layer of the pages).


def rope(v: np.ndarray, t, base: float, inverse: bool = False) -> np.ndarray:
    """v [..., d_h] at positions t (broadcast against v's leading axes)
    rotated pairwise by t * theta_i; inverse rotates back (the transpose)."""
    if not base:
        return v
    dh = v.shape[-1]
    theta = float(base) ** (-2.0 * np.arange(dh // 2) / dh)
    ang = np.asarray(t, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    if inverse:
        s = -s
    x0, x1 = v[..., 0::2], v[..., 1::2]
    out = np.empty(np.broadcast_shapes(v.shape, c.shape[:-1] + (dh,)))
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def causal_attention(q: np.ndarray, t: np.ndarray, K: np.ndarray, V: np.ndarray,
                     scale: float) -> np.ndarray:
    """o[i] = sum_{s <= t[i]} softmax_s(scale * q[i] . K[s]) V[s]  (step 7).

    Exact two-pass softmax (maximum, then exponentials and their sum), rows
    batched only by sharing the key range [0, max t].
    """
    o = np.empty((q.shape[0], V.shape[1]))
    order = np.argsort(t, kind="stable")
    c0 = 0
    while c0 < len(order):
        # rows per chunk bounded so that a chunk's score matrix stays ~16M entries
        span = int(t[order[min(len(order) - 1, c0 + 255)]]) + 1
        chunk = max(1, min(256, (1 << 24) // span))
        rows = order[c0:c0 + chunk]
        c0 += chunk
        tmax = int(t[rows].max()) + 1
        s = scale * (q[rows] @ K[:tmax].T)               # [n, tmax]
        s[np.arange(tmax)[None, :] > t[rows][:, None]] = -np.inf
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        o[rows] = (e @ V[:tmax]) / e.sum(axis=1, keepdims=True)
    return o


# --------------------------------------------------------------------------
# steps 9-11: output construction
# --------------------------------------------------------------------------


def expert_head(g: int, e: int, n_experts: int) -> int:
    """W_q head index of expert e of group g (the G*E routed heads, group-major)."""
    return g * n_experts + e


def weighted_slot(w_rows: np.ndarray, o_hard: np.ndarray) -> np.ndarray:
    """o_w[n] = sum_g sum_j w[n, g, j] * o[n, g, j]  (step 9, [gist-nl], [gist-pt]).

    w_rows [n, G, k]; o_hard [n, G, k, d_h].  A plain sum over groups.
    """
    return np.einsum("ngj,ngjd->nd", w_rows, o_hard)


def slot_vector(o_hard: np.ndarray, o_sh: np.ndarray, o_w: np.ndarray) -> np.ndarray:
    """[hard slots (group-major, rank-minor) | shared | weighted], width (k*G+2)*d_h (step 10)."""
    n = o_hard.shape[0]
    return np.concatenate([o_hard.reshape(n, -1), o_sh, o_w], axis=1)


def output_projection(s: np.ndarray, wo: np.ndarray) -> np.ndarray:
    """y = s . W_O^T with W_O in [out, in] layout, [d, (k*G+2)*d_h] (step 11)."""
    return s @ wo.T


# Output constructions compared in the ablation of [pptc] section 4.3 (Table 1):
#   "full"            the GQE layer: hard slots, the always-on shared head and the
#                     renormalized weighted slot; W_O has (k*G+2)*d_h inputs.
#   "hard"            hard concatenation only: the k*G selected experts' outputs,
#                     no weighted slot and no shared head (the full layer is
#                     described as this plus the renormalized slot and the shared
#                     head); W_O has k*G*d_h inputs.
#   "weighted_concat" the hard slots, each scaled by its expert's in-group softmax
#                     probability p (not renormalized over the k), and no further
#                     slot or shared head; W_O has k*G*d_h inputs.  (The page says
#                     the weights may be the in-group probabilities; that is the
#                     reading taken.)
OUTPUT_MODES = ("full", "hard", "weighted_concat")


def slot_width(mode: str, n_groups: int, top_k: int, head_dim: int) -> int:
    """Width of the slot vector that W_O projects, per output construction."""
    return (top_k * n_groups + (2 if mode == "full" else 0)) * head_dim


def ablation_slots(mode: str, o_hard: np.ndarray, p_sel: np.ndarray) -> np.ndarray:
    """Slot vector of the "hard" and "weighted_concat" constructions.

    o_hard [n, G, k, d_h]; p_sel [n, G, k] the in-group softmax probability of
    each selected expert.  Group-major, rank-minor, like the full layer's hard
    slots.
    """
    n = o_hard.shape[0]
    if mode == "hard":
        return o_hard.reshape(n, -1)
    if mode == "weighted_concat":
        return (p_sel[..., None] * o_hard).reshape(n, -1)
    raise ValueError(mode)


# --------------------------------------------------------------------------
# full layer
# --------------------------------------------------------------------------


def gqe_forward(x, wq, wk, wv, wr, wo, br, n_groups, n_experts, top_k, head_dim,
                shared_kv_group=0, scale=None, positions=None, output_mode="full",
                phase_times=None, rope_base=0.0):
    """GQE prefill forward (steps 1-11) in float64.

    x: [B, L, d]; wq [(G*E+1)*d_h, d]; wk, wv [G*d_h, d]; wr [G*E, d];
    wo [d, (k*G+2)*d_h]; br [G*E].  All float64 holding the exact input values.
    ``positions`` (sorted ints) restricts the attention/output steps to those
    query positions in every sequence; routing and dispatch always cover
    every token.  Returns a dict with r, p, idx, w ([B,L,G,*]), counts,
    offsets, pos, slot, and for the checked positions: q [B,n,k*G+1,d_h]
    (slot-head order: hard slot g*k+j, then the shared head), k_ and v
    ([B,G,upto,d_h]), o [B,n,k*G+1,d_h] (attention outputs), s
    [B,n,(k*G+2)*d_h] (slot vectors) and y [B,n,d].

    ``output_mode`` picks one of OUTPUT_MODES; the "hard" and "weighted_concat"
    constructions have no shared head (q and o then hold the k*G hard
    slot-heads only) and a W_O of k*G*d_h inputs.

    ``phase_times``, when a dict, receives the wall time in seconds of each
    phase: "route" (steps 1-4), "dispatch" (5), "kv" (6), "attention"
    (7-8, query projections included) and "output" (9-11).  Timing only: it
    changes nothing that is computed.

    ``rope_base`` > 0 rotates every query row and K (``rope``) after the
    projections; q and k_ are then the rotated values.
    """
    if output_mode not in OUTPUT_MODES:
        raise ValueError(output_mode)
    full = output_mode == "full"
    B, L, d = x.shape
    G, E, k, dh = n_groups, n_experts, top_k, head_dim
    scale = 1.0 / math.sqrt(dh) if scale is None else scale
    pos_q = np.arange(L) if positions is None else np.asarray(positions, dtype=np.int64)
    n = len(pos_q)
    upto = int(pos_q.max()) + 1

    clock = [time.perf_counter()]

    def tick(phase):
        now = time.perf_counter()
        if phase_times is not None:
            phase_times[phase] = phase_times.get(phase, 0.0) + now - clock[0]
        clock[0] = now

    r, p, idx, w = route(x.reshape(B * L, d), wr, br, G, E, k)
    r, p = r.reshape(B, L, G, E), p.reshape(B, L, G, E)
    idx, w = idx.reshape(B, L, G, k), w.reshape(B, L, G, k)
    tick("route")
    counts, offsets, pos, slot = dispatch(idx, E)
    tick("dispatch")

    S = k * G + (1 if full else 0)                        # attention slot-heads
    q_all = np.empty((B, n, S, dh))
    o_all = np.empty((B, n, S, dh))
    s_all = np.empty((B, n, slot_width(output_mode, G, k, dh)))
    K_all = np.empty((B, G, upto, dh))
    V_all = np.empty((B, G, upto, dh))
    for b in range(B):
        xb = x[b]
        K_all[b] = rope(kv_project(xb, wk, G, dh, upto), np.arange(upto), rope_base)
        V_all[b] = kv_project(xb, wv, G, dh, upto)
        tick("kv")
        xq = xb[pos_q]                                    # [n, d]
        o_hard = np.empty((n, G, k, dh))
        for g in range(G):
            for j in range(k):
                e_sel = idx[b, pos_q, g, j]               # [n]
                qh = np.empty((n, dh))
                for e in range(E):                        # the selected expert's own W_q rows
                    m = e_sel == e
                    if m.any():
                        qh[m] = xq[m] @ head_rows(wq, expert_head(g, e, E), dh).T
                qh = rope(qh, pos_q, rope_base)
                q_all[b, :, g * k + j] = qh
                o_hard[:, g, j] = causal_attention(qh, pos_q, K_all[b, g], V_all[b, g], scale)
        o_all[b, :, :k * G] = o_hard.reshape(n, G * k, dh)
        if not full:
            tick("attention")
            p_sel = np.take_along_axis(p[b, pos_q], idx[b, pos_q].astype(np.int64), axis=-1)
            s_all[b] = ablation_slots(output_mode, o_hard, p_sel)
            tick("output")
            continue
        q_sh = rope(xq @ head_rows(wq, G * E, dh).T, pos_q, rope_base)  # step 8: shared head
        o_sh = causal_attention(q_sh, pos_q, K_all[b, shared_kv_group],
                                V_all[b, shared_kv_group], scale)
        q_all[b, :, k * G] = q_sh
        o_all[b, :, k * G] = o_sh
        tick("attention")
        o_w = weighted_slot(w[b, pos_q], o_hard)
        s_all[b] = slot_vector(o_hard, o_sh, o_w)
        tick("output")
    y = output_projection(s_all, wo)
    tick("output")
    return dict(r=r, p=p, idx=idx, w=w, counts=counts, offsets=offsets, pos=pos, slot=slot,
                q=q_all, k_=K_all, v=V_all, o=o_all, s=s_all, y=y, positions=pos_q)


def gqa_forward(x, wq_dense, wk, wv, wo_dense, n_groups, n_experts, head_dim, scale=None,
                positions=None, rope_base=0.0):
    """Dense GQA baseline: all G*E query heads active, head h reads KV group h // E.

    wq_dense [G*E*d_h, d]; wo_dense [d, G*E*d_h].  Returns q, o [B,n,G*E,d_h] and
    y [B,n,d] for the checked positions.  ([pptc] section 4.2: the all-active
    GQA comparison model.)
    """
    B, L, d = x.shape
    G, E, dh = n_groups, n_experts, head_dim
    H = G * E
    scale = 1.0 / math.sqrt(dh) if scale is None else scale
    pos_q = np.arange(L) if positions is None else np.asarray(positions, dtype=np.int64)
    n = len(pos_q)
    upto = int(pos_q.max()) + 1
    q_all = np.empty((B, n, H, dh))
    o_all = np.empty((B, n, H, dh))
    for b in range(B):
        K = rope(kv_project(x[b], wk, G, dh, upto), np.arange(upto), rope_base)
        V = kv_project(x[b], wv, G, dh, upto)
        xq = x[b][pos_q]
        for h in range(H):
            qh = rope(xq @ head_rows(wq_dense, h, dh).T, pos_q, rope_base)
            q_all[b, :, h] = qh
            o_all[b, :, h] = causal_attention(qh, pos_q, K[h // E], V[h // E], scale)
    y = output_projection(o_all.reshape(B, n, H * dh), wo_dense)
    return dict(q=q_all, o=o_all, y=y, positions=pos_q)


def attention_flops(batch: int, seq_len: int, heads: int, head_dim: int) -> int:
    """Algorithmic flops of causal attention: QK^T and PV, 2*d_h each per pair s <= t."""
    return 2 * 2 * head_dim * heads * batch * seq_len * (seq_len + 1) // 2


# --------------------------------------------------------------------------
# decode: one new token per sequence against a KV cache
# --------------------------------------------------------------------------
# The pages analyse prefill only ([pptc] section 6 lists decode as not
# analysed).  A decode step is the same layer evaluated at one position: the
# new token of sequence b sits at position pos[b]; it is routed, its K and V
# are appended to the cache at pos[b], and its queries attend causally to the
# cached keys 0..pos[b] (steps 1-11 restricted to that row).


def gqe_decode_step(x_t, k_cache, v_cache, pos, wq, wk, wv, wr, wo, br, n_groups, n_experts,
                    top_k, head_dim, shared_kv_group=0, scale=None, output_mode="full",
                    rope_base=0.0):
    """x_t [B, d]: the new tokens; k_cache, v_cache [B, G, Lc, d_h]: keys and
    values of positions < pos[b] (later entries are never read); pos [B].

    Returns idx, w ([B, G, k]), k_new, v_new ([B, G, d_h]), the updated caches
    (copies), q and o ([B, heads, d_h]: hard slots g*k+j, then the shared head
    for the full output), s (slot vectors) and y [B, d].
    """
    if output_mode not in OUTPUT_MODES:
        raise ValueError(output_mode)
    B, d = x_t.shape
    G, E, k, dh = n_groups, n_experts, top_k, head_dim
    scale = 1.0 / math.sqrt(dh) if scale is None else scale
    full = output_mode == "full"
    r, p, idx, w = route(x_t, wr, br, G, E, k)             # steps 1-4 for the new tokens
    posf = np.asarray(pos, dtype=np.int64)
    k_new = rope((x_t @ wk.T).reshape(B, G, dh), posf[:, None], rope_base)  # step 6
    v_new = (x_t @ wv.T).reshape(B, G, dh)
    kc, vc = k_cache.copy(), v_cache.copy()
    H = k * G + (1 if full else 0)
    q_all = np.empty((B, H, dh))
    o_all = np.empty((B, H, dh))
    s_all = np.empty((B, slot_width(output_mode, G, k, dh)))
    for b in range(B):
        t = int(pos[b])
        kc[b, :, t] = k_new[b]
        vc[b, :, t] = v_new[b]
        tt = np.array([t])
        o_hard = np.empty((1, G, k, dh))
        for g in range(G):
            for j in range(k):                             # step 7: the selected experts
                qh = rope(x_t[b] @ head_rows(wq, expert_head(g, int(idx[b, g, j]), E), dh).T,
                          t, rope_base)
                q_all[b, g * k + j] = qh
                o_hard[0, g, j] = causal_attention(qh[None], tt, kc[b, g], vc[b, g], scale)[0]
        o_all[b, :k * G] = o_hard.reshape(G * k, dh)
        if not full:
            p_sel = np.take_along_axis(p[b][None], idx[b][None].astype(np.int64), axis=-1)
            s_all[b] = ablation_slots(output_mode, o_hard, p_sel)[0]
            continue
        q_sh = rope(x_t[b] @ head_rows(wq, G * E, dh).T, t, rope_base)  # step 8
        o_sh = causal_attention(q_sh[None], tt, kc[b, shared_kv_group], vc[b, shared_kv_group],
                                scale)
        q_all[b, k * G] = q_sh
        o_all[b, k * G] = o_sh[0]
        o_w = weighted_slot(w[b][None], o_hard)             # step 9
        s_all[b] = slot_vector(o_hard, o_sh, o_w)[0]        # step 10
    y = output_projection(s_all, wo)                        # step 11
    return dict(r=r, p=p, idx=idx, w=w, k_new=k_new, v_new=v_new, k_cache=kc, v_cache=vc,
                q=q_all, o=o_all, s=s_all, y=y)


def gqa_decode_step(x_t, k_cache, v_cache, pos, wq_dense, wk, wv, wo_dense, n_groups, n_experts,
                    head_dim, scale=None, rope_base=0.0):
    """Dense GQA decode step: all G*E heads, head h reads KV group h // E."""
    B, d = x_t.shape
    G, E, dh = n_groups, n_experts, head_dim
    H = G * E
    scale = 1.0 / math.sqrt(dh) if scale is None else scale
    posf = np.asarray(pos, dtype=np.int64)
    k_new = rope((x_t @ wk.T).reshape(B, G, dh), posf[:, None], rope_base)
    v_new = (x_t @ wv.T).reshape(B, G, dh)
    kc, vc = k_cache.copy(), v_cache.copy()
    o_all = np.empty((B, H, dh))
    for b in range(B):
        t = int(pos[b])
        kc[b, :, t] = k_new[b]
        vc[b, :, t] = v_new[b]
        for h in range(H):
            qh = rope(x_t[b] @ head_rows(wq_dense, h, dh).T, t, rope_base)
            o_all[b, h] = causal_attention(qh[None], np.array([t]), kc[b, h // E], vc[b, h // E],
                                           scale)[0]
    y = output_projection(o_all.reshape(B, H * dh), wo_dense)
    return dict(k_new=k_new, v_new=v_new, k_cache=kc, v_cache=vc, o=o_all, y=y)


# --------------------------------------------------------------------------
# backward: gradients of  <y, dy> + aux_weight * L_aux
# --------------------------------------------------------------------------
# [gist-nl] "Architectuur en Routing" and "Training en Loss": the discrete
# top-k choice has no gradient; the language-model loss reaches the router
# only through the weighted slot (step 9), and an auxiliary load-balancing
# loss pushes every group's router to spread its tokens over the experts.
# The pages give no formula for that loss.  The reading taken is the usual
# product of the routed fraction and the mean router probability, per group,
# averaged over groups and scaled by E (1 at a perfectly even load):
#     L_aux = (E / G) * sum_g sum_e f[g, e] * P[g, e]
#     f[g, e] = (routed slots of group g that chose e) / (B * L * k)
#     P[g, e] = mean over all tokens of p[t, g, e]
# f is a count and carries no gradient; P carries it through p.


def load_balance_loss(p: np.ndarray, idx: np.ndarray, n_experts: int):
    """L_aux, f [G, E] and P [G, E] from p [..., G, E] and idx [..., G, k]."""
    G, E = p.shape[-2], n_experts
    k = idx.shape[-1]
    pt = p.reshape(-1, G, E)
    it = idx.reshape(-1, G, k)
    T = pt.shape[0]
    f = np.zeros((G, E))
    for g in range(G):
        f[g] = np.bincount(it[:, g, :].reshape(-1), minlength=E)[:E] / (T * k)
    P = pt.mean(axis=0)
    return (E / G) * float((f * P).sum()), f, P


def softmax_backward(prob: np.ndarray, dprob: np.ndarray) -> np.ndarray:
    """Gradient on the logits of prob = softmax(logits) over the last axis."""
    return prob * (dprob - (prob * dprob).sum(axis=-1, keepdims=True))


def attention_backward(q, t, K, V, do, scale):
    """Gradients of o = causal_attention(q, t, K, V, scale) given do.

    q, do [n, d_h] at positions t; K, V [upto, d_h].  Returns dq [n, d_h],
    dK and dV [upto, d_h].  The probabilities P are formed again, exactly;
    with dP = do . V^T, the score gradient is P * (dP - rowsum(dP * P)).
    """
    upto = K.shape[0]
    s = scale * (q @ K.T)
    s[np.arange(upto)[None, :] > t[:, None]] = -np.inf
    P = np.exp(s - s.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    dV = P.T @ do
    dP = do @ V.T
    dS = P * (dP - (dP * P).sum(axis=1, keepdims=True))
    return scale * (dS @ K), scale * (dS.T @ q), dV


def gqe_backward(x, wq, wk, wv, wr, wo, br, dy, n_groups, n_experts, top_k, head_dim,
                 shared_kv_group=0, scale=None, output_mode="full", aux_weight=0.0,
                 rope_base=0.0):
    """Gradients of <y, dy> + aux_weight * L_aux for the GQE layer (float64).

    Returns dx [B, L, d], dwq, dwk, dwv, dwr, dbr, dwo (the shapes of the
    weights), aux_loss, and the intermediates: ds (slot-vector gradient),
    do [B, L, S, d_h] (attention-output gradient per slot-head), dq
    [B, L, S, d_h], dk and dv [B, G, L, d_h], dw [B, L, G, k] (routing-weight
    gradient; the in-group probability of the selected experts for
    "weighted_concat"), dr [B, L, G, E] (logit gradient), and the forward
    dict under "fwd".
    """
    if output_mode not in OUTPUT_MODES:
        raise ValueError(output_mode)
    full = output_mode == "full"
    B, L, d = x.shape
    G, E, k, dh = n_groups, n_experts, top_k, head_dim
    kG = k * G
    sc = 1.0 / math.sqrt(dh) if scale is None else scale
    fwd = gqe_forward(x, wq, wk, wv, wr, wo, br, G, E, k, dh, shared_kv_group=shared_kv_group,
                      scale=scale, output_mode=output_mode, rope_base=rope_base)
    p, idx, w, s_all, o_all = fwd["p"], fwd["idx"], fwd["w"], fwd["s"], fwd["o"]
    Sh = o_all.shape[2]
    dwo = np.einsum("bln,blc->nc", dy, s_all)             # y = s . W_O^T
    ds = dy @ wo
    dx = np.zeros_like(x)
    dwq, dwk, dwv = np.zeros_like(wq), np.zeros_like(wk), np.zeros_like(wv)
    dr = np.zeros((B, L, G, E))
    dw_all = np.zeros((B, L, G, k))
    do_all = np.zeros((B, L, Sh, dh))
    dq_all = np.zeros((B, L, Sh, dh))
    dk_all = np.zeros((B, G, L, dh))
    dv_all = np.zeros((B, G, L, dh))
    tpos = np.arange(L)
    for b in range(B):
        o_hard = o_all[b, :, :kG].reshape(L, G, k, dh)
        ds_h = ds[b, :, :kG * dh].reshape(L, G, k, dh)
        if full:                                          # steps 9-10 backwards
            ds_w = ds[b, :, (kG + 1) * dh:]
            do_hard = ds_h + w[b][..., None] * ds_w[:, None, None, :]
            dw = np.einsum("lgjd,ld->lgj", o_hard, ds_w)
            dr_sel = softmax_backward(w[b], dw)          # w = softmax of the selected logits
            np.put_along_axis(dr[b], idx[b].astype(np.int64), dr_sel, axis=-1)
        elif output_mode == "weighted_concat":
            p_sel = np.take_along_axis(p[b], idx[b].astype(np.int64), axis=-1)
            do_hard = p_sel[..., None] * ds_h
            dw = np.einsum("lgjd,lgjd->lgj", o_hard, ds_h)
            dp = np.zeros((L, G, E))
            np.put_along_axis(dp, idx[b].astype(np.int64), dw, axis=-1)
            dr[b] += softmax_backward(p[b], dp)          # p = softmax over all E
        else:
            do_hard = ds_h
            dw = np.zeros((L, G, k))
        dw_all[b] = dw
        do_all[b, :, :kG] = do_hard.reshape(L, kG, dh)
        xb = x[b]
        K = fwd["k_"][b]
        V = fwd["v"][b]
        heads = [(g * k + j, g) for g in range(G) for j in range(k)]
        if full:
            do_all[b, :, kG] = ds[b, :, kG * dh:(kG + 1) * dh]
            heads.append((kG, shared_kv_group))
        for h, g in heads:
            dq, dKg, dVg = attention_backward(fwd["q"][b, :, h], tpos, K[g], V[g],
                                              do_all[b, :, h], sc)
            dq = rope(dq, tpos, rope_base, inverse=True)  # through the rotation (its transpose)
            dq_all[b, :, h] = dq
            dk_all[b, g] += rope(dKg, tpos, rope_base, inverse=True)
            dv_all[b, g] += dVg
            if h == kG:                                   # the shared head's own W_q rows
                rows = slice(G * E * dh, (G * E + 1) * dh)
                dwq[rows] += dq.T @ xb
                dx[b] += dq @ wq[rows]
                continue
            j = h % k
            for e in range(E):
                m = idx[b, :, g, j] == e
                if m.any():
                    rows = slice(expert_head(g, e, E) * dh, (expert_head(g, e, E) + 1) * dh)
                    dwq[rows] += dq[m].T @ xb[m]
                    dx[b][m] += dq[m] @ wq[rows]
        for g in range(G):                                # K, V = x . W_k^T, x . W_v^T
            rows = slice(g * dh, (g + 1) * dh)
            dwk[rows] += dk_all[b, g].T @ xb
            dwv[rows] += dv_all[b, g].T @ xb
            dx[b] += dk_all[b, g] @ wk[rows] + dv_all[b, g] @ wv[rows]
    aux_loss, f, _ = load_balance_loss(p, idx, E)
    if aux_weight:
        dp_aux = np.broadcast_to(aux_weight * (E / G) * f / (B * L), p.shape)
        dr += softmax_backward(p, dp_aux)
    drf = dr.reshape(B * L, G * E)
    dwr = drf.T @ x.reshape(B * L, d)                     # r = x . W_r^T + b_r
    dbr = drf.sum(axis=0)
    dx += (drf @ wr).reshape(B, L, d)
    return dict(dx=dx, dwq=dwq, dwk=dwk, dwv=dwv, dwr=dwr, dbr=dbr, dwo=dwo, aux_loss=aux_loss,
                ds=ds, do=do_all, dq=dq_all, dk=dk_all, dv=dv_all, dw=dw_all, dr=dr, fwd=fwd)


def gqa_backward(x, wq_dense, wk, wv, wo_dense, dy, n_groups, n_experts, head_dim, scale=None,
                 rope_base=0.0):
    """Gradients of <y, dy> for the dense GQA baseline: dx, dwq, dwk, dwv, dwo."""
    B, L, d = x.shape
    G, E, dh = n_groups, n_experts, head_dim
    H = G * E
    sc = 1.0 / math.sqrt(dh) if scale is None else scale
    fwd = gqa_forward(x, wq_dense, wk, wv, wo_dense, G, E, dh, scale=scale, rope_base=rope_base)
    o = fwd["o"].reshape(B, L, H * dh)
    dwo = np.einsum("bln,blc->nc", dy, o)
    do = (dy @ wo_dense).reshape(B, L, H, dh)
    dx = np.zeros_like(x)
    dwq, dwk, dwv = np.zeros_like(wq_dense), np.zeros_like(wk), np.zeros_like(wv)
    tpos = np.arange(L)
    for b in range(B):
        xb = x[b]
        K = rope(kv_project(xb, wk, G, dh, L), tpos, rope_base)
        V = kv_project(xb, wv, G, dh, L)
        dK = np.zeros((G, L, dh))
        dV = np.zeros((G, L, dh))
        for h in range(H):
            g = h // E
            dq, dKg, dVg = attention_backward(fwd["q"][b, :, h], tpos, K[g], V[g], do[b, :, h], sc)
            dq = rope(dq, tpos, rope_base, inverse=True)
            dKg = rope(dKg, tpos, rope_base, inverse=True)
            dK[g] += dKg
            dV[g] += dVg
            rows = slice(h * dh, (h + 1) * dh)
            dwq[rows] += dq.T @ xb
            dx[b] += dq @ wq_dense[rows]
        for g in range(G):
            rows = slice(g * dh, (g + 1) * dh)
            dwk[rows] += dK[g].T @ xb
            dwv[rows] += dV[g].T @ xb
            dx[b] += dK[g] @ wk[rows] + dV[g] @ wv[rows]
    return dict(dx=dx, dwq=dwq, dwk=dwk, dwv=dwv, dwo=dwo, do=do, fwd=fwd)


# --------------------------------------------------------------------------
# non-uniform k: group g selects k_g experts
# --------------------------------------------------------------------------
# [pptc] section 6 lists a non-uniform k ("each group selects a different
# number of experts") as future work.  Everything else is the layer above:
# the top-k_g of every group by the same rule, weights renormalized over the
# k_g of the group, hard slots group-major (group g's k_g slots in rank
# order), then the shared slot and the weighted slot; W_O has (K+2)*d_h
# inputs with K = sum of k_g.


def group_offsets(group_top_k):
    """koff[g]: first hard slot of group g; koff[G] = K."""
    koff = [0]
    for kg in group_top_k:
        koff.append(koff[-1] + int(kg))
    return koff


def route_group_k(x, wr, br, n_groups, n_experts, group_top_k):
    """Steps 1-4 with k_g experts in group g.  Returns r, p [T, G, E] and idx,
    w [T, K] (group g at koff[g] .. koff[g]+k_g-1, rank order)."""
    r, p, _, _ = route(x, wr, br, n_groups, n_experts, max(group_top_k))
    koff = group_offsets(group_top_k)
    T = x.shape[0]
    idx = np.empty((T, koff[-1]), dtype=np.int32)
    w = np.empty((T, koff[-1]))
    for g, kg in enumerate(group_top_k):
        sel = topk_in_group(r[:, g], kg)                  # [T, k_g]
        idx[:, koff[g]:koff[g + 1]] = sel
        w[:, koff[g]:koff[g + 1]] = renormalize(p[:, g], sel)
    return r, p, idx, w


def dispatch_group_k(idx, n_groups, n_experts, group_top_k):
    """Per-(b, g, e) lists for idx [B, L, K]: counts [B, G, E]; offsets, the
    exclusive prefix of counts in (b, g, e) order; pos and slot (ascending t,
    rank j) per list."""
    B, L, _ = idx.shape
    koff = group_offsets(group_top_k)
    counts = np.zeros((B, n_groups, n_experts), dtype=np.int32)
    pos_l, slot_l = [], []
    for b in range(B):
        for g in range(n_groups):
            ids = idx[b, :, koff[g]:koff[g + 1]]           # [L, k_g]
            for e in range(n_experts):
                t_sel, j_sel = np.nonzero(ids == e)
                counts[b, g, e] = t_sel.size
                pos_l.append(t_sel)
                slot_l.append(j_sel)
    offsets = np.zeros(B * n_groups * n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts.reshape(-1))
    return (counts, offsets.astype(np.int32), np.concatenate(pos_l).astype(np.int32),
            np.concatenate(slot_l).astype(np.int32))


def gqe_forward_group_k(x, wq, wk, wv, wr, wo, br, n_groups, n_experts, group_top_k, head_dim,
                        shared_kv_group=0, scale=None, output_mode="full"):
    """The GQE layer with k_g experts selected in group g (float64).

    Returns r, p [B,L,G,E]; idx, w [B,L,K]; counts, offsets, pos, slot; q, o
    [B,L,S,d_h] (slot-heads: group g's k_g hard slots from koff[g], then the
    shared head for the full output); s [B,L,width]; y [B,L,d].
    """
    if output_mode not in OUTPUT_MODES:
        raise ValueError(output_mode)
    full = output_mode == "full"
    B, L, d = x.shape
    G, E, dh = n_groups, n_experts, head_dim
    koff = group_offsets(group_top_k)
    K = koff[-1]
    scale = 1.0 / math.sqrt(dh) if scale is None else scale
    r, p, idx, w = route_group_k(x.reshape(B * L, d), wr, br, G, E, group_top_k)
    r, p = r.reshape(B, L, G, E), p.reshape(B, L, G, E)
    idx, w = idx.reshape(B, L, K), w.reshape(B, L, K)
    counts, offsets, pos, slot = dispatch_group_k(idx, G, E, group_top_k)
    S = K + (1 if full else 0)
    q_all = np.empty((B, L, S, dh))
    o_all = np.empty((B, L, S, dh))
    s_all = np.empty((B, L, (K + (2 if full else 0)) * dh))
    tpos = np.arange(L)
    for b in range(B):
        K_b = kv_project(x[b], wk, G, dh, L)
        V_b = kv_project(x[b], wv, G, dh, L)
        for g in range(G):
            for j in range(group_top_k[g]):
                h = koff[g] + j
                qh = np.empty((L, dh))
                for e in range(E):
                    m = idx[b, :, h] == e
                    if m.any():
                        qh[m] = x[b][m] @ head_rows(wq, expert_head(g, e, E), dh).T
                q_all[b, :, h] = qh
                o_all[b, :, h] = causal_attention(qh, tpos, K_b[g], V_b[g], scale)
        o_hard = o_all[b, :, :K]                          # [L, K, d_h]
        if output_mode == "hard":
            s_all[b] = o_hard.reshape(L, -1)
            continue
        if output_mode == "weighted_concat":
            p_sel = np.concatenate([np.take_along_axis(p[b, :, g], idx[b, :, koff[g]:koff[g + 1]]
                                                       .astype(np.int64), axis=-1)
                                    for g in range(G)], axis=1)
            s_all[b] = (p_sel[..., None] * o_hard).reshape(L, -1)
            continue
        q_sh = x[b] @ head_rows(wq, G * E, dh).T
        o_sh = causal_attention(q_sh, tpos, K_b[shared_kv_group], V_b[shared_kv_group], scale)
        q_all[b, :, K] = q_sh
        o_all[b, :, K] = o_sh
        o_w = np.einsum("lh,lhd->ld", w[b], o_hard)       # sum over groups and ranks
        s_all[b] = np.concatenate([o_hard.reshape(L, -1), o_sh, o_w], axis=1)
    y = output_projection(s_all, wo)
    return dict(r=r, p=p, idx=idx, w=w, counts=counts, offsets=offsets, pos=pos, slot=slot,
                q=q_all, o=o_all, s=s_all, y=y)


def gqe_decode_step_group_k(x_t, k_cache, v_cache, pos, wq, wk, wv, wr, wo, br, n_groups,
                            n_experts, group_top_k, head_dim, shared_kv_group=0, scale=None,
                            output_mode="full"):
    """One decode step (as gqe_decode_step) with k_g experts selected in group
    g: idx, w [B, K]; q, o [B, S, d_h] with group g's hard slots from koff[g]
    and then the shared head for the full output; s, y as in the prefill layer
    with per-group counts."""
    if output_mode not in OUTPUT_MODES:
        raise ValueError(output_mode)
    B, d = x_t.shape
    G, E, dh = n_groups, n_experts, head_dim
    koff = group_offsets(group_top_k)
    K = koff[-1]
    scale = 1.0 / math.sqrt(dh) if scale is None else scale
    full = output_mode == "full"
    r, p, idx, w = route_group_k(x_t, wr, br, G, E, group_top_k)     # steps 1-4
    k_new = (x_t @ wk.T).reshape(B, G, dh)                            # step 6
    v_new = (x_t @ wv.T).reshape(B, G, dh)
    kc, vc = k_cache.copy(), v_cache.copy()
    S = K + (1 if full else 0)
    q_all = np.empty((B, S, dh))
    o_all = np.empty((B, S, dh))
    s_all = np.empty((B, (K + (2 if full else 0)) * dh))
    for b in range(B):
        t = int(pos[b])
        kc[b, :, t] = k_new[b]
        vc[b, :, t] = v_new[b]
        tt = np.array([t])
        for g in range(G):
            for j in range(group_top_k[g]):                           # step 7
                h = koff[g] + j
                qh = x_t[b] @ head_rows(wq, expert_head(g, int(idx[b, h]), E), dh).T
                q_all[b, h] = qh
                o_all[b, h] = causal_attention(qh[None], tt, kc[b, g], vc[b, g], scale)[0]
        o_hard = o_all[b, :K]
        if output_mode == "hard":
            s_all[b] = o_hard.reshape(-1)
            continue
        if output_mode == "weighted_concat":
            p_sel = np.concatenate([p[b, g, idx[b, koff[g]:koff[g + 1]].astype(np.int64)]
                                    for g in range(G)])
            s_all[b] = (p_sel[:, None] * o_hard).reshape(-1)
            continue
        q_sh = x_t[b] @ head_rows(wq, G * E, dh).T                    # step 8
        o_sh = causal_attention(q_sh[None], tt, kc[b, shared_kv_group], vc[b, shared_kv_group],
                                scale)[0]
        q_all[b, K] = q_sh
        o_all[b, K] = o_sh
        o_w = w[b] @ o_hard                                           # step 9
        s_all[b] = np.concatenate([o_hard.reshape(-1), o_sh, o_w])    # step 10
    y = output_projection(s_all, wo)                                  # step 11
    return dict(r=r, p=p, idx=idx, w=w, k_new=k_new, v_new=v_new, k_cache=kc, v_cache=vc,
                q=q_all, o=o_all, s=s_all, y=y)


def load_balance_loss_group_k(p, idx, n_experts, group_top_k):
    """L_aux, f [G, E] and P [G, E] with k_g experts in group g: f[g, e] is
    expert e's share of group g's T*k_g routed slots (idx [..., K])."""
    G, E = p.shape[-2], n_experts
    koff = group_offsets(group_top_k)
    pt = p.reshape(-1, G, E)
    it = idx.reshape(-1, koff[-1])
    T = pt.shape[0]
    f = np.zeros((G, E))
    for g in range(G):
        f[g] = np.bincount(it[:, koff[g]:koff[g + 1]].reshape(-1), minlength=E)[:E] / (
            T * group_top_k[g])
    P = pt.mean(axis=0)
    return (E / G) * float((f * P).sum()), f, P


def gqe_backward_group_k(x, wq, wk, wv, wr, wo, br, dy, n_groups, n_experts, group_top_k,
                         head_dim, shared_kv_group=0, scale=None, output_mode="full",
                         aux_weight=0.0):
    """Gradients of <y, dy> + aux_weight * L_aux for the layer with k_g experts
    in group g (float64): the same returns as gqe_backward, with dw [B, L, K]
    and the slot-heads of gqe_forward_group_k."""
    if output_mode not in OUTPUT_MODES:
        raise ValueError(output_mode)
    full = output_mode == "full"
    B, L, d = x.shape
    G, E, dh = n_groups, n_experts, head_dim
    koff = group_offsets(group_top_k)
    K = koff[-1]
    sc = 1.0 / math.sqrt(dh) if scale is None else scale
    fwd = gqe_forward_group_k(x, wq, wk, wv, wr, wo, br, G, E, group_top_k, dh,
                              shared_kv_group=shared_kv_group, scale=scale,
                              output_mode=output_mode)
    p, idx, w, s_all, o_all = fwd["p"], fwd["idx"], fwd["w"], fwd["s"], fwd["o"]
    Sh = o_all.shape[2]
    dwo = np.einsum("bln,blc->nc", dy, s_all)             # y = s . W_O^T
    ds = dy @ wo
    dx = np.zeros_like(x)
    dwq, dwk, dwv = np.zeros_like(wq), np.zeros_like(wk), np.zeros_like(wv)
    dr = np.zeros((B, L, G, E))
    dw_all = np.zeros((B, L, K))
    do_all = np.zeros((B, L, Sh, dh))
    dq_all = np.zeros((B, L, Sh, dh))
    dk_all = np.zeros((B, G, L, dh))
    dv_all = np.zeros((B, G, L, dh))
    tpos = np.arange(L)
    for b in range(B):
        o_hard = o_all[b, :, :K]                          # [L, K, d_h]
        ds_h = ds[b, :, :K * dh].reshape(L, K, dh)
        if full:                                          # steps 9-10 backwards
            ds_w = ds[b, :, (K + 1) * dh:]
            do_hard = ds_h + w[b][..., None] * ds_w[:, None, :]
            dw = np.einsum("lhd,ld->lh", o_hard, ds_w)
            for g in range(G):                            # w = softmax of group g's selected logits
                sl = slice(koff[g], koff[g + 1])
                dr_sel = softmax_backward(w[b][:, sl], dw[:, sl])
                np.put_along_axis(dr[b][:, g], idx[b][:, sl].astype(np.int64), dr_sel, axis=-1)
        elif output_mode == "weighted_concat":
            p_sel = np.concatenate([np.take_along_axis(p[b][:, g], idx[b][:, koff[g]:koff[g + 1]]
                                                       .astype(np.int64), axis=-1)
                                    for g in range(G)], axis=1)
            do_hard = p_sel[..., None] * ds_h
            dw = np.einsum("lhd,lhd->lh", o_hard, ds_h)
            for g in range(G):                            # p = softmax over all E
                sl = slice(koff[g], koff[g + 1])
                dp = np.zeros((L, E))
                np.put_along_axis(dp, idx[b][:, sl].astype(np.int64), dw[:, sl], axis=-1)
                dr[b][:, g] += softmax_backward(p[b][:, g], dp)
        else:
            do_hard = ds_h
            dw = np.zeros((L, K))
        dw_all[b] = dw
        do_all[b, :, :K] = do_hard
        xb = x[b]
        K_b = kv_project(xb, wk, G, dh, L)
        V_b = kv_project(xb, wv, G, dh, L)
        heads = [(koff[g] + j, g) for g in range(G) for j in range(group_top_k[g])]
        if full:
            do_all[b, :, K] = ds[b, :, K * dh:(K + 1) * dh]
            heads.append((K, shared_kv_group))
        for h, g in heads:
            dq, dKg, dVg = attention_backward(fwd["q"][b, :, h], tpos, K_b[g], V_b[g],
                                              do_all[b, :, h], sc)
            dq_all[b, :, h] = dq
            dk_all[b, g] += dKg
            dv_all[b, g] += dVg
            if h == K:                                    # the shared head's own W_q rows
                rows = slice(G * E * dh, (G * E + 1) * dh)
                dwq[rows] += dq.T @ xb
                dx[b] += dq @ wq[rows]
                continue
            for e in range(E):
                m = idx[b, :, h] == e
                if m.any():
                    rows = slice(expert_head(g, e, E) * dh, (expert_head(g, e, E) + 1) * dh)
                    dwq[rows] += dq[m].T @ xb[m]
                    dx[b][m] += dq[m] @ wq[rows]
        for g in range(G):                                # K, V = x . W_k^T, x . W_v^T
            rows = slice(g * dh, (g + 1) * dh)
            dwk[rows] += dk_all[b, g].T @ xb
            dwv[rows] += dv_all[b, g].T @ xb
            dx[b] += dk_all[b, g] @ wk[rows] + dv_all[b, g] @ wv[rows]
    aux_loss, f, _ = load_balance_loss_group_k(p, idx, E, group_top_k)
    if aux_weight:
        dp_aux = np.broadcast_to(aux_weight * (E / G) * f / (B * L), p.shape)
        dr += softmax_backward(p, dp_aux)
    drf = dr.reshape(B * L, G * E)
    dwr = drf.T @ x.reshape(B * L, d)                     # r = x . W_r^T + b_r
    dbr = drf.sum(axis=0)
    dx += (drf @ wr).reshape(B, L, d)
    return dict(dx=dx, dwq=dwq, dwk=dwk, dwv=dwv, dwr=dwr, dbr=dbr, dwo=dwo, aux_loss=aux_loss,
                ds=ds, do=do_all, dq=dq_all, dk=dk_all, dv=dv_all, dw=dw_all, dr=dr, fwd=fwd)

"""Plant plausible mistakes in copies of the CPU oracle; the pins must catch each.

Every mutation below is a bug one could make while writing the oracle from
the pages (a dropped term, a wrong sign or index, a transposed operand, a
wrong order).  Each runs on a private copy of the oracle module, on the CPU,
and at least one pin from tests/oracle_pins.py has to fail on it.
"""
import importlib.util
import math
import os

import numpy as np
import pytest

from oracle_pins import ALL_PINS

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "gqe_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("gqe_oracle_mutant", ORACLE_SRC)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _attention_variant(mod, *, scale_mult=1.0, strict=False, no_mask=False, no_max=False):
    def causal_attention(q, t, K, V, scale):
        o = np.empty((q.shape[0], V.shape[1]))
        for i in range(q.shape[0]):
            tmax = int(t.max()) + 1
            s = scale * scale_mult * (K[:tmax] @ q[i])
            if not no_mask:
                keep = np.arange(tmax) < t[i] if strict else np.arange(tmax) <= t[i]
                s = np.where(keep, s, -np.inf)
            m = 0.0 if no_max else s[np.isfinite(s)].max() if np.isfinite(s).any() else 0.0
            e = np.exp(s - m)
            o[i] = (e @ V[:tmax]) / e.sum()
        return o
    mod.causal_attention = causal_attention


def m_no_scale(mod):
    _attention_variant(mod, scale_mult=math.sqrt(4.0))     # drops 1/sqrt(d_h) at d_h = 4


def m_strict_causal(mod):
    _attention_variant(mod, strict=True)


def m_no_causal_mask(mod):
    _attention_variant(mod, no_mask=True)


def m_topk_lowest(mod):
    mod.topk_in_group = lambda r, k: np.argsort(r, axis=-1, kind="stable")[..., :k].astype(np.int32)


def m_tie_to_highest(mod):
    def topk(r, k):
        E = r.shape[-1]
        rev = np.argsort(-r[..., ::-1], axis=-1, kind="stable")[..., :k]
        return (E - 1 - rev).astype(np.int32)
    mod.topk_in_group = topk


def m_index_order_slots(mod):
    orig = mod.topk_in_group
    mod.topk_in_group = lambda r, k: np.sort(orig(r, k), axis=-1)


def m_renorm_over_all_groups(mod):
    def renorm(p, idx):
        ps = np.take_along_axis(p, idx.astype(np.int64), axis=-1)
        return ps / ps.sum(axis=(-1, -2), keepdims=True)
    mod.renormalize = renorm


def m_no_renorm(mod):
    mod.renormalize = lambda p, idx: np.take_along_axis(p, idx.astype(np.int64), axis=-1)


def m_softmax_over_groups(mod):
    def sm(r):
        z = np.exp(r - r.max(axis=(-1, -2), keepdims=True))
        return z / z.sum(axis=(-1, -2), keepdims=True)
    mod.group_softmax = sm


def m_router_group_transposed(mod):
    def logits(x, wr, br, G, E):
        r = x @ wr.T + br[None, :]
        return r.reshape(x.shape[0], E, G).transpose(0, 2, 1).copy()
    mod.router_logits = logits


def m_router_bias_dropped(mod):
    def logits(x, wr, br, G, E):
        return (x @ wr.T).reshape(x.shape[0], G, E)
    mod.router_logits = logits


def m_exact_logits_bias_dropped(mod):
    """the exactly rounded logits of near-tie tokens leave out the router bias."""
    def exact_logits(x_row, wr, br):
        return np.array([math.fsum(list(x_row * wr[c])) for c in range(wr.shape[0])])
    mod.exact_logits = exact_logits


def m_expert_head_transposed(mod):
    mod.expert_head = lambda g, e, E: e * E + g          # group and expert swapped


def m_expert_head_reversed(mod):
    mod.expert_head = lambda g, e, E: g * E + (E - 1 - e)


def m_weighted_mean(mod):
    orig = mod.weighted_slot
    mod.weighted_slot = lambda w_rows, o_hard: orig(w_rows, o_hard) / w_rows.shape[1]


def m_weighted_missing(mod):
    mod.weighted_slot = lambda w_rows, o_hard: np.zeros((o_hard.shape[0], o_hard.shape[-1]))


def m_weighted_unweighted(mod):
    mod.weighted_slot = lambda w_rows, o_hard: o_hard.sum(axis=(1, 2))


def m_slots_rank_major(mod):
    def sv(o_hard, o_sh, o_w):
        n = o_hard.shape[0]
        return np.concatenate([o_hard.transpose(0, 2, 1, 3).reshape(n, -1), o_sh, o_w], axis=1)
    mod.slot_vector = sv


def m_shared_weighted_swapped(mod):
    def sv(o_hard, o_sh, o_w):
        n = o_hard.shape[0]
        return np.concatenate([o_hard.reshape(n, -1), o_w, o_sh], axis=1)
    mod.slot_vector = sv


def m_output_untransposed(mod):
    def proj(s, wo):
        # wrong operand orientation, made to fit: reads W_O column-major
        return s @ wo.reshape(wo.shape[1], wo.shape[0])
    mod.output_projection = proj


def m_dispatch_descending(mod):
    orig = mod.dispatch

    def disp(idx, E):
        counts, offsets, pos, slot = orig(idx, E)
        pos, slot = pos.copy(), slot.copy()
        for i in range(len(offsets) - 1):
            pos[offsets[i]:offsets[i + 1]] = pos[offsets[i]:offsets[i + 1]][::-1]
            slot[offsets[i]:offsets[i + 1]] = slot[offsets[i]:offsets[i + 1]][::-1]
        return counts, offsets, pos, slot
    mod.dispatch = disp


def m_kv_heads_swapped(mod):
    orig = mod.kv_project

    def kvp(x_b, w, G, dh, upto):
        out = orig(x_b, w, G, dh, upto)
        return out[::-1].copy() if G > 1 else out
    mod.kv_project = kvp


def m_head_rows_shifted(mod):
    mod.head_rows = lambda w, head, dh: w[head * dh + 1:(head + 1) * dh + 1] \
        if (head + 1) * dh + 1 <= w.shape[0] else w[head * dh:(head + 1) * dh]


def m_wconcat_renormalized(mod):
    """weighted_concat scales by the renormalized weights instead of p."""
    orig = mod.ablation_slots

    def slots(mode, o_hard, p_sel):
        if mode == "weighted_concat":
            p_sel = p_sel / p_sel.sum(axis=-1, keepdims=True)
        return orig(mode, o_hard, p_sel)
    mod.ablation_slots = slots


def m_wconcat_unscaled(mod):
    """weighted_concat forgets the scaling (same as hard)."""
    orig = mod.ablation_slots
    mod.ablation_slots = lambda mode, o_hard, p_sel: orig("hard", o_hard, p_sel)


def m_hard_rank_reversed(mod):
    """the ablation constructions list the hard slots in reverse rank order."""
    orig = mod.ablation_slots
    mod.ablation_slots = lambda mode, o_hard, p_sel: orig(mode, o_hard[:, :, ::-1], p_sel[:, :, ::-1])


def m_decode_stale_cache(mod):
    """the decode step attends before its own K/V reach the cache."""
    orig = mod.gqe_decode_step

    def step(x_t, k_cache, v_cache, pos, *a, **kw):
        res = orig(x_t, k_cache, v_cache, pos - 1, *a, **kw)
        return res
    mod.gqe_decode_step = step


def _patch_source(mod, old, new):
    """Re-execute the oracle's source with one passage replaced (in place)."""
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, old
    exec(compile(src.replace(old, new), ORACLE_SRC, "exec"), mod.__dict__)


def m_bwd_no_rowsum_term(mod):
    """attention backward without the -rowsum(dP * P) term of the softmax."""
    _patch_source(mod, "dS = P * (dP - (dP * P).sum(axis=1, keepdims=True))", "dS = P * dP")


def m_bwd_dk_unscaled(mod):
    """key gradient without the attention scale."""
    _patch_source(mod, "return scale * (dS @ K), scale * (dS.T @ q), dV",
                  "return scale * (dS @ K), dS.T @ q, dV")


def m_bwd_weighted_slot_dropped(mod):
    """the weighted slot's gradient does not reach the experts' outputs."""
    _patch_source(mod, "do_hard = ds_h + w[b][..., None] * ds_w[:, None, None, :]",
                  "do_hard = ds_h")


def m_bwd_softmax_jacobian_diagonal(mod):
    """the router's softmax backward keeps only the diagonal of the Jacobian."""
    _patch_source(mod, "return prob * (dprob - (prob * dprob).sum(axis=-1, keepdims=True))",
                  "return prob * dprob")


def m_bwd_aux_sign(mod):
    """the load-balancing gradient with the wrong sign."""
    _patch_source(mod, """    aux_loss, f, _ = load_balance_loss(p, idx, E)
    if aux_weight:
        dp_aux = np.broadcast_to(aux_weight * (E / G) * f / (B * L), p.shape)
        dr += softmax_backward(p, dp_aux)""", """    aux_loss, f, _ = load_balance_loss(p, idx, E)
    if aux_weight:
        dp_aux = np.broadcast_to(aux_weight * (E / G) * f / (B * L), p.shape)
        dr -= softmax_backward(p, dp_aux)""")


def m_aux_fraction_per_token(mod):
    """routed fraction counted per token instead of per routed slot."""
    _patch_source(mod, "minlength=E)[:E] / (T * k)", "minlength=E)[:E] / T")


def m_bwd_shared_head_group0(mod):
    """the shared head's gradient goes to group 0 whatever shared_kv_group is."""
    _patch_source(mod, "heads.append((kG, shared_kv_group))", "heads.append((kG, 0))")


def m_group_k_first_groups_k(mod):
    """every group selects as many experts as group 0."""
    _patch_source(mod, "        sel = topk_in_group(r[:, g], kg)                  # [T, k_g]",
                  "        sel = topk_in_group(r[:, g], group_top_k[0])[:, :kg]")


def m_group_k_weights_over_all(mod):
    """per-group weights renormalized over the largest k instead of k_g."""
    _patch_source(mod, "        w[:, koff[g]:koff[g + 1]] = renormalize(p[:, g], sel)",
                  "        w[:, koff[g]:koff[g + 1]] = renormalize(p[:, g], topk_in_group(r[:, g], max(group_top_k)))[:, :kg]")


def m_group_k_decode_group_zero_keys(mod):
    """the per-group decode step's hard slots all read group 0's cache."""
    _patch_source(mod, "                o_all[b, h] = causal_attention(qh[None], tt, kc[b, g], vc[b, g], scale)[0]",
                  "                o_all[b, h] = causal_attention(qh[None], tt, kc[b, 0], vc[b, 0], scale)[0]")


def m_group_k_decode_rank_as_slot(mod):
    """the per-group decode step looks its experts up by rank j, not by slot."""
    _patch_source(mod, "qh = x_t[b] @ head_rows(wq, expert_head(g, int(idx[b, h]), E), dh).T",
                  "qh = x_t[b] @ head_rows(wq, expert_head(g, int(idx[b, j]), E), dh).T")


def m_group_k_aux_over_largest_k(mod):
    """the per-group load fraction divides by the largest k, not by k_g."""
    _patch_source(mod, "            T * group_top_k[g])", "            T * max(group_top_k))")


def m_group_k_bwd_softmax_over_all_slots(mod):
    """the per-group weight gradient treats all K slots as one softmax."""
    _patch_source(mod, "                dr_sel = softmax_backward(w[b][:, sl], dw[:, sl])",
                  "                dr_sel = softmax_backward(w[b], dw)[:, sl]")


def m_rope_on_values(mod):
    """the rotation is applied to V as well."""
    _patch_source(mod, "        V_all[b] = kv_project(xb, wv, G, dh, upto)\n",
                  "        V_all[b] = rope(kv_project(xb, wv, G, dh, upto), np.arange(upto), rope_base)\n")


def m_rope_off_by_one(mod):
    """positions counted from 1."""
    _patch_source(mod, "    ang = np.asarray(t, dtype=np.float64)[..., None] * theta",
                  "    ang = (np.asarray(t, dtype=np.float64)[..., None] + 1.0) * theta")


def m_rope_half_split(mod):
    """dims i and i + d_h/2 paired instead of 2i and 2i+1."""
    _patch_source(mod, "    x0, x1 = v[..., 0::2], v[..., 1::2]",
                  "    x0, x1 = v[..., :dh // 2], v[..., dh // 2:]")


def m_rope_backward_not_inverted(mod):
    """the query gradient is rotated forward instead of back."""
    _patch_source(mod, "            dq = rope(dq, tpos, rope_base, inverse=True)  # through the rotation (its transpose)",
                  "            dq = rope(dq, tpos, rope_base)")


def m_rope_queries_only(mod):
    """keys left unrotated."""
    _patch_source(mod, "        K_all[b] = rope(kv_project(xb, wk, G, dh, upto), np.arange(upto), rope_base)",
                  "        K_all[b] = kv_project(xb, wk, G, dh, upto)")


MUTATIONS = [
    m_rope_on_values, m_rope_off_by_one, m_rope_half_split, m_rope_backward_not_inverted,
    m_rope_queries_only,
    m_no_scale, m_strict_causal, m_no_causal_mask, m_topk_lowest, m_tie_to_highest,
    m_index_order_slots, m_renorm_over_all_groups, m_no_renorm, m_softmax_over_groups,
    m_router_group_transposed, m_router_bias_dropped, m_exact_logits_bias_dropped,
    m_expert_head_transposed,
    m_expert_head_reversed,
    m_weighted_mean, m_weighted_missing, m_weighted_unweighted, m_slots_rank_major,
    m_shared_weighted_swapped, m_output_untransposed, m_dispatch_descending,
    m_kv_heads_swapped, m_head_rows_shifted,
    m_wconcat_renormalized, m_wconcat_unscaled, m_hard_rank_reversed, m_decode_stale_cache,
    m_bwd_no_rowsum_term, m_bwd_dk_unscaled, m_bwd_weighted_slot_dropped,
    m_bwd_softmax_jacobian_diagonal, m_bwd_aux_sign, m_aux_fraction_per_token,
    m_bwd_shared_head_group0, m_group_k_first_groups_k, m_group_k_weights_over_all,
    m_group_k_decode_group_zero_keys, m_group_k_decode_rank_as_slot,
    m_group_k_aux_over_largest_k, m_group_k_bwd_softmax_over_all_slots,
]


@pytest.mark.parametrize("mutate", MUTATIONS, ids=lambda f: f.__name__)
def test_pins_catch_planted_mistake(mutate):
    mod = fresh_oracle()
    mutate(mod)
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            failed.append((pin.__name__, type(exc).__name__))
    assert failed, f"no pin caught {mutate.__name__}"


def test_unmutated_copy_passes_every_pin():
    mod = fresh_oracle()
    for pin in ALL_PINS:
        pin(mod)

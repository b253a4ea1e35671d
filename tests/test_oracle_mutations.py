"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant replaces one oracle function with a plausible wrong version (a
dropped term, a wrong sign, a swapped operand, a wrong tie rule) and runs the
pin tests of tests/test_oracle_pins.py against it; at least one pin must
fail.  The mistakes are planted in the oracle only, on the CPU.
"""
import numpy as np
import pytest

import oracle.coreset as C
import oracle.denoise as D
import oracle.verify as VF
import oracle.head as H
import oracle.moe as M
import oracle.norm as N
import oracle.stack as S
from oracle import bf16
import tests.test_oracle_pins as P


def _silu_sign(z):
    return z / (1.0 + np.exp(z))


def _ffn_swapped(x_row, wg, wu, wd):
    g = bf16.to_f64(wg) @ x_row
    u = bf16.to_f64(wu) @ x_row
    a = bf16.round_f64(M.silu(u) * g)
    return bf16.to_f64(wd) @ a


def _ffn_unrounded(x_row, wg, wu, wd):
    g = bf16.to_f64(wg) @ x_row
    u = bf16.to_f64(wu) @ x_row
    return bf16.to_f64(wd) @ (M.silu(g) * u)


def _topk_high_ties(row, k):
    r = np.array(row, dtype=np.float64)
    out = []
    for _ in range(k):
        j = len(r) - 1 - int(np.argmax(r[::-1]))
        out.append(j)
        r[j] = -np.inf
    return np.array(out)


def _moe_no_shared(orig):
    def f(*a, **kw):
        a = list(a)
        if len(a) > 6:
            a[6:9] = [None, None, None]
        kw.pop("ws_gate", None)
        return orig(*a, **kw)
    return f


def _moe_no_residual(orig):
    def f(*a, **kw):
        kw["residual"] = None
        return orig(*a, **kw)
    return f


def _route_no_renorm(orig):
    def f(x, wr, k, bias=None, renorm=True):
        return orig(x, wr, k, bias, False)
    return f


def _softmax_no_max(l):
    z = np.exp(np.asarray(l, dtype=np.float64))
    return z / z.sum(axis=-1, keepdims=True) * 0.999


def _confidence_mask_kept(l32, mask_id):
    l = np.array(l32, dtype=np.float64)
    a = np.argmax(l, axis=1)
    m = l[np.arange(l.shape[0]), a]
    conf = 1.0 / np.exp(l - m[:, None]).sum(axis=1)
    srt = np.sort(l, axis=1)
    return a, conf, srt[:, -1] - srt[:, -2]


def _unmask_fallback_last(tokens, argmax, conf, mask_id, threshold, fallback=True):
    tokens = np.asarray(tokens, dtype=np.int64)
    c32 = np.asarray(conf, dtype=np.float32)
    masked = tokens == mask_id
    commit = masked & (c32 >= np.float32(threshold))
    if fallback and masked.any() and not commit.any():
        cand = np.where(masked, c32.astype(np.float64), -np.inf)
        commit[len(cand) - 1 - int(np.argmax(cand[::-1]))] = True
    return np.where(commit, argmax, tokens), commit


def _unmask_all_masked(tokens, argmax, conf, mask_id, threshold, fallback=True):
    tokens = np.asarray(tokens, dtype=np.int64)
    commit = np.asarray(conf, np.float32) >= np.float32(threshold)
    return np.where(commit, argmax, tokens), commit


def _rms_no_eps(x_bits, eps=1e-6, gamma=None):
    x = bf16.to_f64(x_bits)
    return bf16.from_f64(x / np.sqrt(np.mean(np.abs(x), axis=-1, keepdims=True)))


def _mass_counts(p, first, E):
    mass = np.zeros(E)
    for t in range(first.shape[0]):
        for e in first[t]:
            mass[e] += 1.0
    return mass


def _cut_one_more(orig):
    return lambda order, mass, top_p: min(len(order), orig(order, mass, top_p) + 1)


def _order_ties_high(mass):
    touched = np.flatnonzero(mass > 0)
    return touched[np.lexsort((-touched, -mass[touched]))]


def _order_ascending(mass):
    touched = np.flatnonzero(mass > 0)
    return touched[np.lexsort((touched, mass[touched]))]


def _step_no_final_norm(tokens, embed_bits, layers, head_bits, k, mask_id, threshold=0.95,
                        eps=1e-6):
    import oracle.stack as S
    tokens = np.asarray(tokens, dtype=np.int64)
    y, near = S.stack_forward(np.asarray(embed_bits)[tokens], layers, k, eps)
    out = H.head_unmask(y, head_bits, tokens, mask_id, threshold)
    out["near_route"] = near.any(axis=0)
    return out


def _stack_ignores_coreset(orig):
    return lambda x, layers, k, eps=1e-6, tokens=None, coreset_top_p=None, block=32: orig(
        x, layers, k, eps, tokens)


def _unmask_whole_call(orig):
    return lambda tokens, argmax, conf, mask_id, threshold, fallback=True, block=None: orig(
        tokens, argmax, conf, mask_id, threshold, fallback)


def _loop_one_step(orig):
    return lambda *a, **kw: orig(*a, **dict(kw, max_steps=1))


def _bound_max(entropy, ratio=0.9, delta=0.6):
    return np.maximum(ratio, delta * np.exp(-np.asarray(entropy, dtype=np.float64)))


def _bound_plus_h(entropy, ratio=0.9, delta=0.6):
    return np.minimum(ratio, delta * np.exp(np.asarray(entropy, dtype=np.float64)))


def _count_all(accept):
    return int(np.sum(accept))


def _stats_bits(l32):
    l = np.asarray(l32, dtype=np.float64)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log2(p), 0.0)
    return np.argmax(l, axis=1).astype(np.int64), p, -plogp.sum(axis=1)


def _verify_bonus_last_row(orig):
    def f(*a, **kw):
        o = orig(*a, **kw)
        o["tokens"][o["n_accepted"]] = o["argmax"][-1]
        return o
    return f


MUTANTS = {
    "verify_bound_max": (VF, "bound", lambda o: _bound_max),
    "verify_bound_sign": (VF, "bound", lambda o: _bound_plus_h),
    "verify_counts_every_accept": (VF, "accept_prefix", lambda o: _count_all),
    "verify_entropy_in_bits": (VF, "stats", lambda o: _stats_bits),
    "verify_bonus_from_last_row": (VF, "verify", _verify_bonus_last_row),
    "denoise_no_final_norm": (D, "denoise_step", lambda o: _step_no_final_norm),
    "denoise_stops_after_one_step": (D, "denoise_block", _loop_one_step),
    "stack_ignores_coreset": (S, "stack_forward", _stack_ignores_coreset),
    "unmask_ignores_blocks": (H, "unmask", _unmask_whole_call),
    "coreset_mass_counts": (C, "expert_mass", lambda o: _mass_counts),
    "coreset_cut_one_more": (C, "cut", _cut_one_more),
    "coreset_mass_ties_high_id": (C, "mass_order", lambda o: _order_ties_high),
    "coreset_order_ascending": (C, "mass_order", lambda o: _order_ascending),
    "silu_sign": (M, "silu", lambda o: _silu_sign),
    "gate_up_swapped": (M, "expert_ffn", lambda o: _ffn_swapped),
    "activation_not_rounded": (M, "expert_ffn", lambda o: _ffn_unrounded),
    "topk_ties_high_id": (M, "select_topk", lambda o: _topk_high_ties),
    "shared_dropped": (M, "moe_block", _moe_no_shared),
    "residual_dropped": (M, "moe_block", _moe_no_residual),
    "no_renormalisation": (M, "route", _route_no_renorm),
    "softmax_scaled": (M, "softmax", lambda o: _softmax_no_max),
    "mask_not_excluded": (H, "confidence", lambda o: _confidence_mask_kept),
    "fallback_last_position": (H, "unmask", lambda o: _unmask_fallback_last),
    "commits_unmasked_rows": (H, "unmask", lambda o: _unmask_all_masked),
    "rmsnorm_wrong": (N, "rmsnorm", lambda o: _rms_no_eps),
}

PINS = [
    P.test_uniform_router_ties_pick_lowest_ids,
    P.test_renormalised_weights_sum_to_one,
    P.test_single_expert_reduces_to_torch_swiglu,
    P.test_identical_experts_make_routing_irrelevant,
    lambda: P.test_route_matches_torch_softmax_topk(True),
    lambda: P.test_route_matches_torch_softmax_topk(False),
    lambda: P.test_moe_matches_dense_brute_force(0, "plain"),
    lambda: P.test_moe_matches_dense_brute_force(1, "residual"),
    lambda: P.test_moe_matches_dense_brute_force(0, "norenorm"),
    P.test_head_closed_form_confidence_and_threshold,
    P.test_head_fallback_commits_exactly_one,
    lambda: P.test_head_matches_dense_brute_force_and_torch(0),
    P.test_rmsnorm_matches_torch_and_unit_rms,
    P.test_stack_tokens_independent_and_matches_chained_brute,
    lambda: P.test_coreset_reproduces_page_simulation(3),
    P.test_coreset_closed_form_identical_tokens,
    P.test_coreset_equal_masses_keep_lower_id,
    P.test_coreset_top_p_one_keeps_routing_and_tiny_top_p_keeps_one,
    P.test_coreset_sets_nest_and_restrict_routing,
    P.test_denoise_loop_terminates_commits_and_never_revisits,
    P.test_denoise_step_is_its_parts_composed,
    P.test_denoise_confident_block_finishes_in_one_step,
    P.test_denoise_with_coreset_selector,
    P.test_unmask_rule_per_block,
    P.test_denoise_multiblock_equals_blocks_alone,
    P.test_verify_bound_matches_page_points,
    P.test_verify_entropy_and_probabilities_closed_form,
    P.test_verify_threshold_decision_and_prefix,
]


def test_unmutated_pins_pass():
    for pin in PINS:
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    mod, attr, make = MUTANTS[name]
    monkeypatch.setattr(mod, attr, make(getattr(mod, attr)))
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception as exc:           # an assertion or a shape error
            caught.append(type(exc).__name__)
    assert caught, f"mutant {name} passed every pin"

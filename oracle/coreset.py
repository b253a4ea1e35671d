"""Block coreset expert selector (test infrastructure only).

The files page, section "The expert selection": for a block, each token's
top-8 routing probabilities are added up per expert, the experts are sorted
by that total, the smallest set whose share of the total reaches top_p (0.9,
and never fewer than the top expert) is kept, and no token of the block may
route outside it.  Section "What Clover is" gives the configuration (the
selector on, top_p 0.9); the selector belongs to the denoising passes.

What is computed here, per block of ``block`` consecutive tokens, in the
pages' order:

1. every token's first-pass picks S_t (the k largest logits, equal logits ->
   lower id) and its routing probabilities p_t = softmax(l_t) over all E;
2. mass_e = sum over the block's tokens t and picks j with S_tj = e of
   p_t[e] (the probabilities themselves, not the renormalised weights);
3. the touched experts sorted by mass, larger first (equal -> lower id);
4. kept = the shortest prefix of that order whose cumulative mass reaches
   top_p times the total mass (at least one expert);
5. every token of the block routes again with the logits of experts outside
   the kept set at -inf: k' = min(k, |kept|) picks (equal -> lower id),
   weights renormalised over the picks (``renorm=False``: the softmax over the
   kept set); slots k'..k-1 hold no expert (id -1, weight 0).

Readings (the pages are silent): the mass adds the plain softmax
probabilities (a simulation cannot tell this apart from the renormalised
weights); ties in the mass order go to the lower id; a block with fewer than
k kept experts gives each token all of them.

Pins (tests/test_oracle_pins.py): the pages' simulation of the selector on
synthetic logits (per-token N(0,1) noise plus a block-wide N(0,1) term of
weight 0..3): union, kept-set size and re-routed slots per token; closed
forms on identical tokens; top_p = 1 keeps every touched expert and changes
no routing; a tiny top_p keeps one expert; kept sets nest as top_p grows.
"""
from __future__ import annotations

import numpy as np

from .moe import GAP_EXCLUDE, select_topk, softmax

CUT_EXCLUDE = 1e-5    # relative closeness of cumulative mass to the cut, or of two masses


def expert_mass(p, first, E: int) -> np.ndarray:
    """Step 2: mass_e = sum over tokens t and picks j with first[t][j] = e of
    p[t][e]."""
    mass = np.zeros(E, dtype=np.float64)
    for t in range(first.shape[0]):
        for e in first[t]:
            mass[e] += p[t, e]
    return mass


def mass_order(mass) -> np.ndarray:
    """Step 3: the touched experts (mass > 0), larger mass first, equal ->
    lower id."""
    touched = np.flatnonzero(mass > 0)
    return touched[np.lexsort((touched, -mass[touched]))]   # last key is primary


def cut(order, mass, top_p: float) -> int:
    """Step 4: the length of the shortest prefix of `order` whose cumulative
    mass reaches top_p times the total (at least 1)."""
    cum = np.cumsum(mass[order])
    thr = top_p * cum[-1]
    n = 1
    while n < len(order) and cum[n - 1] < thr:
        n += 1
    return n


def block_coreset(l32_block, k: int, top_p: float):
    """Steps 1-4 for one block of float32 logits [t][E].  Returns dict:
    kept (expert ids in mass order), order (all touched, mass order), mass
    ([E] float64), first ([t][k] first-pass picks), near (True when the kept
    set is a float-rounding call: a cumulative sum at the cut within
    CUT_EXCLUDE of the threshold, a mass at the cut boundary within
    CUT_EXCLUDE of the next one, or a first-pass near tie)."""
    l32 = np.asarray(l32_block, dtype=np.float32)
    nt, E = l32.shape
    p = softmax(l32)
    first = (np.stack([select_topk(l32[t], k) for t in range(nt)]) if nt
             else np.zeros((0, k), dtype=np.int64))
    near = False
    if k < E:
        for t in range(nt):
            srt = np.sort(l32[t].astype(np.float64))[::-1]
            near |= bool((srt[k - 1] - srt[k]) < GAP_EXCLUDE)
    mass = expert_mass(p, first, E)
    order = mass_order(mass)
    n = cut(order, mass, top_p) if len(order) else 0
    if len(order):
        cum = np.cumsum(mass[order])
        thr = top_p * cum[-1]
        tol = CUT_EXCLUDE * cum[-1]
        near |= bool(abs(cum[n - 1] - thr) < tol)
        if n >= 2:
            near |= bool(abs(cum[n - 2] - thr) < tol)
        if n < len(order):
            a, b = mass[order[n - 1]], mass[order[n]]
            near |= bool(abs(a - b) <= CUT_EXCLUDE * max(a, b))
    return {"kept": order[:n], "order": order, "mass": mass, "first": first, "near": near}


def coreset_route(l32, k: int, top_p: float, block: int = 32, renorm: bool = True):
    """Steps 1-5 for every block of the token rows of l32 ([T][E] float32).

    Returns dict: idx [T][k] (-1 past k'), w [T][k] (0 past k'), kept (list of
    per-block kept arrays), n_kept [nblocks], first [T][k], near_block
    [nblocks], near_tie [T] (restricted selection within GAP_EXCLUDE, or the
    token's block is near), rerouted [T] (first-pass picks outside the kept
    set)."""
    l32 = np.asarray(l32, dtype=np.float32)
    T, E = l32.shape
    nb = (T + block - 1) // block
    idx = np.full((T, k), -1, dtype=np.int64)
    w = np.zeros((T, k), dtype=np.float64)
    near_tok = np.zeros(T, dtype=bool)
    rer = np.zeros(T, dtype=np.int64)
    first = np.zeros((T, k), dtype=np.int64)
    kept_all, n_kept, near_blk = [], np.zeros(nb, dtype=np.int64), np.zeros(nb, dtype=bool)
    for b in range(nb):
        t0, t1 = b * block, min(T, (b + 1) * block)
        c = block_coreset(l32[t0:t1], k, top_p)
        kept = c["kept"]
        kept_all.append(kept)
        n_kept[b] = len(kept)
        near_blk[b] = c["near"]
        allow = np.zeros(E, dtype=bool)
        allow[kept] = True
        kk = min(k, len(kept))
        for t in range(t0, t1):
            first[t] = c["first"][t - t0]
            rer[t] = int(np.sum(~allow[first[t]]))
            lr = np.where(allow, l32[t].astype(np.float64), -np.inf)
            s = select_topk(lr, kk)
            idx[t, :kk] = s
            pr = softmax(np.where(allow, l32[t], -np.inf).astype(np.float32)[None, :])[0]
            ps = pr[s]
            w[t, :kk] = ps / ps.sum() if renorm else ps
            near = c["near"]
            if kk < len(kept):
                srt = np.sort(lr)[::-1]
                near |= bool((srt[kk - 1] - srt[kk]) < GAP_EXCLUDE)
            near_tok[t] = near
    return {"idx": idx, "w": w, "kept": kept_all, "n_kept": n_kept, "first": first,
            "near_block": near_blk, "near_tie": near_tok, "rerouted": rer}


def simulate(weight: float, n_blocks: int, rng, E: int = 256, k: int = 8, block: int = 32,
             top_p: float = 0.9):
    """The pages' experiment: logits = per-token N(0,1) noise + weight times a
    block-wide N(0,1) preference per expert.  Returns the mean union (before
    the selector), mean kept-set size and mean re-routed slots per token."""
    unions, kepts, rers = [], [], []
    for _ in range(n_blocks):
        pref = rng.standard_normal(E)
        l32 = (rng.standard_normal((block, E)) + weight * pref[None, :]).astype(np.float32)
        c = block_coreset(l32, k, top_p)
        unions.append(len(c["order"]))
        kepts.append(len(c["kept"]))
        allow = np.zeros(E, dtype=bool)
        allow[c["kept"]] = True
        rers.append(np.mean([np.sum(~allow[c["first"][t]]) for t in range(block)]))
    return float(np.mean(unions)), float(np.mean(kepts)), float(np.mean(rers))

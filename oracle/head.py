"""Untied output head and the low-confidence unmask rule (test infrastructure only).

What it computes (the files page, "How it writes", steps 2 and 3; "What
Clover is": mask_token_id 151669, denoising_config low_confidence with
threshold 0.95; the head has its own 508,559,360 weights, not the
embedding's, and every step streams all of them):

1. logits l_t = W_head h_t for every vocabulary row, taken to float32;
2. the mask token is excluded (its logit becomes -inf), so no slot can
   predict it;
3. a_t = the most likely token (equal logits: lowest vocabulary id) and
   conf_t = its probability = 1 / sum_v exp(l_t,v - max_v l_t,v);
4. every still-masked slot (tokens[t] == mask_id) whose confidence reaches the
   threshold commits: tokens[t] = a_t.  If none does, the single most
   confident still-masked slot commits (equal confidences: lowest position).
   Slots already committed are never revisited.

Readings where the pages are loose: the page says "above 0.95"; the commit
test here is conf >= threshold, taken on float32 values.  The fallback can be
switched off (``fallback=False``) for the plain threshold rule.

Pins (tests/test_oracle_pins.py): the closed form for one raised logit among
V-2 zeros with the mask excluded, conf = e^b / (e^b + V - 2), on both sides of
its 0.95 crossing b* = ln(19 (V - 2)); a mask column holding the row's largest
logit is never chosen and does not enter conf; all rows below the threshold
commit exactly one slot; committed rows are untouched; an fp64 full-softmax
brute force (``oracle.brute``); torch.softmax on random rows.
"""
from __future__ import annotations

import numpy as np

from . import bf16

GAP_EXCLUDE = 1e-4      # top-2 logit gap / |conf - thr| below this: not compared
REL_GAP_FALLBACK = 1e-4  # relative gap of the top-2 masked confidences


def head_logits(h_bits, w_head_bits, rows_per_chunk: int = 16384) -> np.ndarray:
    """[T][H] x [V][H] bf16 bits -> [T][V] float32 logits.

    The product is formed one slice of vocabulary rows at a time only to bound
    host memory (each logit is still one float64 dot product)."""
    h = bf16.to_f64(h_bits)
    V = w_head_bits.shape[0]
    out = np.empty((h.shape[0], V), dtype=np.float32)
    for v0 in range(0, V, rows_per_chunk):
        v1 = min(V, v0 + rows_per_chunk)
        out[:, v0:v1] = (h @ bf16.to_f64(w_head_bits[v0:v1]).T).astype(np.float32)
    return out


def confidence(l32, mask_id: int):
    """Steps 2-3.  Returns (argmax [T] int, conf [T] float64, top2_gap [T])."""
    l = np.array(l32, dtype=np.float64)
    l[:, mask_id] = -np.inf
    a = np.argmax(l, axis=1)
    m = l[np.arange(l.shape[0]), a]
    conf = 1.0 / np.exp(l - m[:, None]).sum(axis=1)
    srt = np.sort(l, axis=1)
    gap = srt[:, -1] - srt[:, -2]
    return a.astype(np.int64), conf, gap


def unmask(tokens, argmax, conf, mask_id: int, threshold: float, fallback: bool = True,
           block=None):
    """Step 4.  Returns (new tokens [T] int64, committed [T] bool).  With
    ``block``, the rows are several blocks of that many slots and the rule
    (threshold and fallback) applies to each block on its own."""
    tokens = np.asarray(tokens, dtype=np.int64)
    if block and block < len(tokens):
        outs, commits = [], []
        for b0 in range(0, len(tokens), block):
            o, c = unmask(tokens[b0:b0 + block], np.asarray(argmax)[b0:b0 + block],
                          np.asarray(conf)[b0:b0 + block], mask_id, threshold, fallback)
            outs.append(o)
            commits.append(c)
        return np.concatenate(outs), np.concatenate(commits)
    c32 = np.asarray(conf, dtype=np.float32)
    masked = tokens == mask_id
    commit = masked & (c32 >= np.float32(threshold))
    if fallback and masked.any() and not commit.any():
        cand = np.where(masked, c32.astype(np.float64), -np.inf)
        commit[int(np.argmax(cand))] = True      # first (lowest) position on ties
    out = np.where(commit, argmax, tokens)
    return out, commit


def head_unmask(h_bits, w_head_bits, tokens, mask_id: int, threshold: float = 0.95,
                fallback: bool = True, block=None):
    """Steps 1-4 for one block (or, with ``block``, for each block of that many
    rows).  Returns dict with tokens, argmax, conf, committed, n_committed and
    the exclusion masks used by parity tests."""
    l32 = head_logits(h_bits, w_head_bits)
    a, conf, gap = confidence(l32, mask_id)
    new, commit = unmask(tokens, a, conf, mask_id, threshold, fallback, block)
    masked = np.asarray(tokens) == mask_id
    c32 = conf.astype(np.float32).astype(np.float64)
    near_thr = np.abs(c32 - threshold) < GAP_EXCLUDE
    # the fallback pick is a coin toss when the two best masked confidences
    # of a block are within a relative 1e-4 of each other
    fb_tie = False
    B = block if block else len(masked)
    for b0 in range(0, len(masked), B):
        mb, cb = masked[b0:b0 + B], c32[b0:b0 + B]
        if fallback and mb.sum() >= 2 and not (mb & (cb >= threshold)).any():
            mc = np.sort(cb[mb])[::-1]
            fb_tie |= bool(mc[0] - mc[1] < REL_GAP_FALLBACK * mc[0])
    return {
        "tokens": new,
        "argmax": a,
        "conf": conf,
        "committed": commit,
        "n_committed": int(commit.sum()),
        "near_tie": gap < GAP_EXCLUDE,
        "near_threshold": near_thr,
        "fallback_tie": fb_tie,
        "logits": l32,
    }

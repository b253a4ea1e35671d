"""Self-speculative verify epilogue (test infrastructure only).

The files page, section "Two ways to run it": a round previews a block of
candidate tokens with the diffusion pass, runs the same model causally over
them, keeps the longest prefix of candidates the causal pass accepts, and adds
one new token at the boundary, so r accepted candidates give r + 1 tokens.
Two accept tests: "exact" keeps a candidate only if it is the causal pass's
most likely token; "threshold" keeps it if the causal pass gives it a
probability of at least a bound built from the entropy H of the causal
distribution at that position, with defaults ratio 0.9 and delta 0.6.  The
bound's formula is lost in the page text; the prose around it fixes what it
does: with the defaults the ratio never binds, the working bound is
0.6 * e^-H, 0.6 for a certain model and 0.22 at one nat.  The reading taken:

    accept_t  <=>  p_t(c_t) >= min(ratio, delta * exp(-H_t))

What is computed, for T candidates c_0..c_{T-1} and the causal pass's hidden
states h_0..h_T (row t predicts position t; row T the position after the last
candidate):

1. l_t = W_head h_t (float32 logits; the causal pass, no mask exclusion);
2. p_t = softmax(l_t); a_t = argmax (equal: lowest id);
   H_t = -sum_v p_t,v log p_t,v (nats);
3. accept_t by the rule (exact: c_t == a_t);
4. r = the number of leading accepted candidates; the round's tokens are
   c_0 .. c_{r-1} and then a_r (the most likely token at the boundary: the
   greedy reading of the new token).

Parity of the bound's formula is pinned only at what the page fixes (its two
points and the ratio's role); the rest of the formula is the reading above:
parity partly unpinned.

Pins (tests/test_oracle_pins.py): the page's two points of the bound (0.6 at
H = 0, 0.6/e = 0.2207 at H = 1 nat), constructed distributions of known
entropy, the ratio binding only when delta e^-H exceeds it, a uniform
distribution always accepted at the defaults (the page's rubber-stamp
remark), prefix semantics (a rejection hides every later acceptance; all
accepted -> the bonus from row T), exact rule = argmax comparison.
"""
from __future__ import annotations

import numpy as np

from . import head

NEAR = 1e-4     # decisions within this relative distance of the bound are not compared


def bound(entropy, ratio: float = 0.9, delta: float = 0.6):
    """The threshold rule's probability bound min(ratio, delta e^-H)."""
    return np.minimum(ratio, delta * np.exp(-np.asarray(entropy, dtype=np.float64)))


def stats(l32):
    """argmax, probabilities and entropy of float32 logit rows."""
    l = np.asarray(l32, dtype=np.float64)
    a = np.argmax(l, axis=1)
    m = l.max(axis=1, keepdims=True)
    z = np.exp(l - m)
    s = z.sum(axis=1, keepdims=True)
    p = z / s
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(p), 0.0)
    return a.astype(np.int64), p, -plogp.sum(axis=1)


def accept_prefix(accept) -> int:
    """r = the number of leading True entries."""
    r = 0
    for ok in accept:
        if not ok:
            break
        r += 1
    return r


def verify(h_bits, w_head_bits, cand, rule: str = "threshold", ratio: float = 0.9,
           delta: float = 0.6):
    """Steps 1-4.  h_bits [T+1][H] bf16 bits, cand [T] ints.  Returns dict:
    n_accepted, tokens ([T+1]: c_0..c_{r-1}, a_r, then -1), accept [T],
    argmax [T+1], p_cand [T], entropy [T+1], near [T] (a decision within NEAR
    of its bound, or an argmax tie within 1e-4 for the exact rule)."""
    cand = np.asarray(cand, dtype=np.int64)
    T = len(cand)
    l32 = head.head_logits(h_bits, w_head_bits)
    a, p, ent = stats(l32)
    pc = p[np.arange(T), cand]
    srt = np.sort(l32.astype(np.float64), axis=1)
    gap = srt[:, -1] - srt[:, -2]
    if rule == "exact":
        acc = cand == a[:T]
        near = gap[:T] < 1e-4
    elif rule == "threshold":
        b = bound(ent[:T], ratio, delta)
        acc = pc >= b
        near = np.abs(pc - b) < NEAR * b
    else:
        raise ValueError(rule)
    r = accept_prefix(acc)
    tokens = np.full(T + 1, -1, dtype=np.int64)
    tokens[:r] = cand[:r]
    tokens[r] = a[r]
    return {"n_accepted": r, "tokens": tokens, "accept": acc, "argmax": a, "p_cand": pc,
            "entropy": ent, "near": near, "gap": gap, "logits": l32}

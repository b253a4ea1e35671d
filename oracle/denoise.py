"""The denoise loop over one block (test infrastructure only).

The files page, section "How it writes": every slot of a new block holds the
mask token; a step runs the model on all slots together, predicts each slot
(the mask token excluded) with the probability of that prediction, fills the
masked slots whose probability reaches the threshold (the most confident
masked slot alone when none does), and steps repeat until no mask is left;
a filled slot is not rewritten later ([deep] "What DiffuSpace actually
shipped").  Section "What Clover is" fixes block 32, the
mask token 151669 and the threshold 0.95.

What the "model" is here: the expert feed-forward part of the stack only (the
hot path this repository builds), read as a pre-norm residual stack:

1. x = E[tokens]          embedding rows of the current block tokens (bf16);
2. for every layer:  x = bf16(x + MoE(RMSNorm(x)))      (oracle.stack);
3. h = RMSNorm(x)         the final norm before the head;
4. head + unmask rule (oracle.head) -> the block's new tokens.

Readings: the embedding lookup and the final RMSNorm (gamma 1, eps 1e-6) are
the plainest pre-norm reading of a decoder with an untied head; attention and
the Gated DeltaNet layers are not on this path and are left out.  With the
fallback every step commits at least one slot, so a block of T masked slots
needs at most T steps.

Pins (tests/test_oracle_pins.py): at most T steps, every step commits at least
one slot, committed slots never change, nothing masked at the end, an
already-unmasked block takes zero steps, the step equals its parts (stack,
norm, head) composed by hand, and a block whose every slot clears the
threshold finishes in one step.
"""
from __future__ import annotations

import numpy as np

from . import head, norm, stack


def denoise_step(tokens, embed_bits, layers, head_bits, k: int, mask_id: int,
                 threshold: float = 0.95, eps: float = 1e-6, coreset_top_p=None, block=None,
                 picks=None):
    """Steps 1-4 once.  Returns the oracle.head dict (new tokens, argmax, conf,
    n_committed, exclusion masks) plus 'near_route' ([T] any layer's top-k
    near tie, or coreset rounding call) and 'h' (the final normalised hidden
    state, bf16 bits).  ``coreset_top_p``: every layer routes through the
    block coreset selector (the files page, "What Clover is": shipped on at
    0.9) over blocks of min(32, B) slots.  ``block`` = B: the rows are
    several blocks of B slots, each with its own commit rule (one block of
    T slots when None).  ``picks``: per-layer expert ids replacing the
    top-k selection (oracle.stack.stack_forward)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    x = np.asarray(embed_bits)[tokens]
    B = block if block else len(tokens)
    y, near = stack.stack_forward(x, layers, k, eps, coreset_top_p=coreset_top_p,
                                  block=min(32, max(1, B)), picks=picks)
    h = norm.rmsnorm(y, eps)
    out = head.head_unmask(h, head_bits, tokens, mask_id, threshold, block=block)
    out["near_route"] = near.any(axis=0) if len(layers) else np.zeros(len(tokens), bool)
    out["h"] = h
    return out


def denoise_block(tokens, embed_bits, layers, head_bits, k: int, mask_id: int,
                  threshold: float = 0.95, max_steps: int | None = None, eps: float = 1e-6,
                  coreset_top_p=None, block=None):
    """The loop.  Returns (final tokens, commits per step)."""
    tokens = np.asarray(tokens, dtype=np.int64).copy()
    limit = len(tokens) if max_steps is None else max_steps
    commits = []
    while (tokens == mask_id).any() and len(commits) < limit:
        out = denoise_step(tokens, embed_bits, layers, head_bits, k, mask_id, threshold, eps,
                           coreset_top_p, block)
        tokens = out["tokens"]
        commits.append(out["n_committed"])
    return tokens, commits

"""Parameter and byte accounting of the pages (test infrastructure only).

These are the sizes the oracle's tensors must have and the byte model the
measurement uses, derived from shapes and checked against the integers and
figures the pages print (tests/golden/page_counts.json, each with its
citation):

* the files page, "What Clover is": an expert is gate and up at 2,048 by 512
  and down at 512 by 2,048 (3,145,728 parameters, 6.29 MB in BF16); routed
  experts total 32,212,254,720 (92.93%) of 34,661,350,848; a token uses
  1,006,632,960 routed parameters plus 1,940,536,768 others, 2,947,169,728 in
  all (5.89 GB in BF16); the untied head is 508,559,360 parameters, 1.47% of
  the weights and 17% of the active ones;
* the files page, "The expert selection": 32 independently routed tokens hit
  256 (1 - (1 - 8/256)^32) experts on average, about 163, i.e. 41 GB of the
  64 GB of experts per step;
* the files page, "What 680 tokens a second has to be": 4.8 TB/s / 5.89 GB
  gives about 814 tokens/s and 8 TB/s about 1,357; a round at 60% of 4.8 TB/s
  reading the 3.88 GB dense part twice plus 64 preview and 163 verify experts
  per layer is 65 GB and 22.5 ms, so 515 tokens/s needs 11.6 tokens a round.
"""
from __future__ import annotations

from dataclasses import dataclass

BYTES_BF16 = 2


@dataclass(frozen=True)
class ModelDims:
    layers: int = 40
    hidden: int = 2048
    experts: int = 256
    top_k: int = 8
    shared: int = 1
    inter: int = 512
    vocab: int = 248320


def expert_params(d: ModelDims) -> int:
    """gate [I][H] + up [I][H] + down [H][I]."""
    return 3 * d.hidden * d.inter


def routed_params(d: ModelDims) -> int:
    return d.layers * d.experts * expert_params(d)


def head_params(d: ModelDims) -> int:
    """Untied output head [V][H]."""
    return d.vocab * d.hidden


def active_routed_params(d: ModelDims) -> int:
    return d.layers * d.top_k * expert_params(d)


def others_from_total(d: ModelDims, total: int) -> int:
    """Every parameter that is not a routed expert and not the input
    embedding (the embedding is only looked up, one row per token, so a
    token does not 'use' it in the pages' sense; it has the head's shape)."""
    return total - routed_params(d) - head_params(d)


def expected_union(experts: int, k: int, tokens: int) -> float:
    """Mean number of distinct experts hit by ``tokens`` tokens that each pick
    ``k`` of ``experts`` independently and uniformly: each expert is missed by
    one token with probability 1 - k/E, by all with (1 - k/E)^T."""
    return experts * (1.0 - (1.0 - k / experts) ** tokens)


def decode_ceiling_tok_s(bandwidth_Bps: float, bytes_per_token: float) -> float:
    return bandwidth_Bps / bytes_per_token


def round_bytes(d: ModelDims, dense_bytes: float, preview_experts: float,
                verify_experts: float) -> float:
    """One self-speculative round: the dense part read by both passes, plus
    each pass's touched experts in every layer."""
    per_expert = expert_params(d) * BYTES_BF16
    return 2 * dense_bytes + (preview_experts + verify_experts) * d.layers * per_expert


def tokens_per_round_needed(round_B: float, bandwidth_Bps: float, efficiency: float,
                            target_tok_s: float):
    """(round time in s, tokens a round must keep to reach target_tok_s)."""
    t = round_B / (bandwidth_Bps * efficiency)
    return t, target_tok_s * t


def layer_expert_bytes(d: ModelDims, touched_routed: int, shared: bool = True) -> int:
    """Algorithmic HBM bytes of one MoE layer's expert weights for one block:
    every touched routed expert and the shared expert read exactly once."""
    return (touched_routed + (1 if shared else 0)) * expert_params(d) * BYTES_BF16

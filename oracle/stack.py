"""Pre-norm residual stack of MoE layers (test infrastructure only).

The denoise step runs every layer over the whole block (the files page, "How
it writes", step 1: the model is run over the 32 slots).  Only the expert FFN
part of each layer is on this path; between layers the stack workload puts a
residual add and an RMSNorm (eps 1e-6):

    x_{l+1} = bf16( x_l + MoE_l( RMSNorm(x_l) ) )

with the residual add fused into the combine (oracle.moe step 7).  Tokens are
independent through the whole stack, so ``tokens`` may select a subset of the
block's rows to follow (the others are not computed).
"""
import numpy as np

from . import coreset, moe, norm


def stack_forward(x_bits, layers, k, eps=1e-6, tokens=None, coreset_top_p=None, block=32,
                  picks=None):
    """layers: list of dicts with w_router, w_gate, w_up, w_down, ws_gate,
    ws_up, ws_down (and optional router_bias).  With ``coreset_top_p`` every
    layer routes through the block coreset selector (oracle.coreset, blocks of
    ``block`` rows; the files page, "The expert selection") instead of the
    plain top-k.  ``picks``: per layer a [T][k] array of expert ids that
    replaces the top-k selection of that layer (the weights are still those
    of step 4 for these picks, from this stack's own logits) -- for chained
    comparisons whose discrete routing decisions are checked separately.
    Returns (y bits, per-layer near flags [L][T']: a routing near tie, or a
    coreset rounding call)."""
    x = np.asarray(x_bits)
    if tokens is not None:
        if coreset_top_p:
            raise ValueError("the coreset selector needs every row of its block")
        x = x[np.asarray(tokens)]
    near = []
    for li, L in enumerate(layers):
        xn = norm.rmsnorm(x, eps)
        routing = None
        if picks is not None:
            if coreset_top_p:
                raise ValueError("picks replace the plain top-k selection only")
            l32 = moe.router_logits(xn, L["w_router"], L.get("router_bias"))
            idx = np.asarray(picks[li])
            w = np.array([moe.pick_weights(l32[t], idx[t]) for t in range(len(idx))])
            routing = (idx, w, np.zeros(len(idx), dtype=bool))
        elif coreset_top_p:
            l32 = moe.router_logits(xn, L["w_router"], L.get("router_bias"))
            c = coreset.coreset_route(l32, k, coreset_top_p, block=block)
            routing = (c["idx"], c["w"], c["near_tie"])
        r = moe.moe_block(xn, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], k,
                          L.get("ws_gate"), L.get("ws_up"), L.get("ws_down"),
                          residual=x, bias=L.get("router_bias"), routing=routing)
        x = r["y"]
        near.append(r["near_tie"])
    return x, np.array(near)

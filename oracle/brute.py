"""Dense float64 brute force for tiny shapes (test infrastructure only).

A second, differently organised statement of the MoE layer and the head used
to pin ``oracle.moe`` and ``oracle.head``:

* every expert is evaluated for every token (no routing-driven gather), the
  routing becomes a dense [T][E] gate matrix built from a full stable sort of
  the negated logits (ties keep the lower id first), and the layer output is
  one matrix product of the gate matrix with the stacked expert outputs;
* the head forms the whole probability matrix with a full softmax and reads
  the confidence as the largest probability.

It follows the same readings as the oracle (SwiGLU, bf16 storage of the
activation and output, unit-weight shared expert); its value is that a
slip in indexing, ordering or accumulation would have to be made twice, in
two different shapes of code, to go unnoticed.
"""
import numpy as np

from . import bf16


def moe_dense(x_bits, w_router, w_gate, w_up, w_down, k, ws_gate=None, ws_up=None,
              ws_down=None, residual=None, bias=None, renorm=True, round_act=True):
    """Returns (y bits [T][H], gate matrix [T][E], y before rounding)."""
    x = bf16.to_f64(x_bits)
    T, H = x.shape
    Wg = bf16.to_f64(np.asarray(w_gate))    # [E][I][H]
    Wu = bf16.to_f64(np.asarray(w_up))
    Wd = bf16.to_f64(np.asarray(w_down))    # [E][H][I]
    E = Wg.shape[0]
    l = (x @ np.asarray(w_router, np.float64).T)
    if bias is not None:
        l = l + np.asarray(bias, np.float64)
    l = l.astype(np.float32).astype(np.float64)
    order = np.argsort(-l, axis=1, kind="stable")[:, :k]
    ex = np.exp(l - l.max(axis=1, keepdims=True))
    prob = ex / ex.sum(axis=1, keepdims=True)
    G = np.zeros((T, E))
    rows = np.arange(T)[:, None]
    G[rows, order] = prob[rows, order]
    if renorm:
        G = G / G.sum(axis=1, keepdims=True)
    g = np.einsum("eih,th->tei", Wg, x)
    u = np.einsum("eih,th->tei", Wu, x)
    a = g / (1.0 + np.exp(-g)) * u
    if round_act:
        a = bf16.round_f64(a)
    Yall = np.einsum("ehi,tei->teh", Wd, a)          # [T][E][H]
    y = np.einsum("te,teh->th", G, Yall)
    if ws_gate is not None:
        sg = bf16.to_f64(ws_gate) @ x.T                # [I][T]
        su = bf16.to_f64(ws_up) @ x.T
        sa = sg / (1.0 + np.exp(-sg)) * su
        if round_act:
            sa = bf16.round_f64(sa)
        y = y + (bf16.to_f64(ws_down) @ sa).T
    if residual is not None:
        y = y + bf16.to_f64(residual)
    return bf16.from_f64(y), G, y


def head_dense(h_bits, w_head_bits, mask_id):
    """Returns (argmax [T], conf [T]) from the full probability matrix."""
    l = (bf16.to_f64(h_bits) @ bf16.to_f64(w_head_bits).T).astype(np.float32)
    l = l.astype(np.float64)
    keep = np.ones(l.shape[1], dtype=bool)
    keep[mask_id] = False
    z = np.exp(l[:, keep] - l[:, keep].max(axis=1, keepdims=True))
    P = np.zeros_like(l)
    P[:, keep] = z / z.sum(axis=1, keepdims=True)
    # lowest id among the equal largest probabilities
    best = P.max(axis=1)
    a = np.array([int(np.flatnonzero(P[t] == best[t])[0]) for t in range(P.shape[0])])
    return a, best

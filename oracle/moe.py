"""Routed mixture-of-experts layer over one block (test infrastructure only).

What it computes, per token t of the block, independently of every other
token (the files page, "What Clover is": a layer holds 256 routed experts,
sends each token to 8 of them, and a shared expert serves every token; gate
and up map 2,048 to 512, down maps 512 to 2,048; the deep-dive page, "What
DiffuSpace actually shipped": the same top-8 plus shared-expert layout):

1. router logits  l = x_t . W_r^T (+ bias), taken to float32;
2. routing probabilities p = softmax(l) over all E experts;
3. S_t = the k experts with the largest logits (equal logits: lower expert id
   first), listed by decreasing probability;
4. weights w_j = p_{S_j} / sum_{i in S} p_i  (renormalised over the k picks;
   with ``renorm=False`` w_j = p_{S_j});
5. for each pick e = S_j: g = W_g,e x_t, u = W_u,e x_t, a = bf16(silu(g) * u)
   with silu(z) = z / (1 + e^-z), and Y_j = W_d,e a;
6. the shared expert the same way, with weight 1 and no gate;
7. y_t = bf16(r_t + sum_j w_j Y_j + Y_shared), r the residual (or 0).

The pages name neither the activation, nor the router's precision, nor the
renormalisation, nor the shared expert's weighting; the readings above
(SwiGLU, float32 router, renormalised top-k, unit-weight shared expert, bf16
storage of the activation and the output) are the plainest ones consistent
with a bf16-stored, fp32-accumulated SwiGLU MoE.

Pins (tests/test_oracle_pins.py): dense fp64 brute force on tiny shapes
(``oracle.brute``, full sort + dense gate matrix); torch.softmax/torch.topk on
random logits; the E=1, k=1 case against torch.nn.functional.silu-based
SwiGLU; identical experts (y independent of routing); uniform router (ids
0..k-1, weights 1/k); sum w = 1; permutation equivariance; expert relabelling
invariance; the pages' union-of-experts figure for 32 independent tokens.
The shared expert's unit weight is parity unpinned by the pages (only the
brute force, which shares the reading, covers it).
"""
from __future__ import annotations

import numpy as np

from . import bf16

GAP_EXCLUDE = 1e-4   # |l_(k) - l_(k+1)| below this: selection not compared


def router_logits(x_bits, w_router, bias=None) -> np.ndarray:
    """[T][H] bf16 bits x [E][H] fp32 (+ [E] fp32) -> [T][E] float32."""
    x = bf16.to_f64(x_bits)
    l = x @ np.asarray(w_router, dtype=np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l.astype(np.float32)


def softmax(l) -> np.ndarray:
    """Row softmax of float32 logits, computed in float64."""
    l = np.asarray(l, dtype=np.float64)
    m = l.max(axis=-1, keepdims=True)
    z = np.exp(l - m)
    return z / z.sum(axis=-1, keepdims=True)


def select_topk(l32_row, k: int) -> np.ndarray:
    """Indices of the k largest float32 logits of one row, largest first;
    equal logits give the lower expert id first.  Picked one at a time:
    np.argmax returns the first (lowest) index among equal maxima."""
    row = np.array(l32_row, dtype=np.float64)
    out = []
    for _ in range(k):
        j = int(np.argmax(row))
        out.append(j)
        row[j] = -np.inf
    return np.array(out, dtype=np.int64)


def pick_weights(l32_row, picks, renorm: bool = True) -> np.ndarray:
    """Step 4 for one token: the weights of the picked experts (ids, -1 = an
    empty slot with weight 0) from its float32 logits: softmax over all E,
    then renormalised over the picks (``renorm``) or not."""
    p = softmax(np.asarray(l32_row)[None, :])[0]
    picks = np.asarray(picks)
    ps = np.where(picks >= 0, p[np.maximum(picks, 0)], 0.0)
    return ps / ps.sum() if renorm else ps


def route(x_bits, w_router, k: int, bias=None, renorm: bool = True):
    """Steps 1-4.  Returns (idx [T][k] int, w [T][k] float64, logits float32
    [T][E], near_tie [T] bool).  near_tie marks tokens whose k-th and
    (k+1)-th largest float32 logits differ by less than GAP_EXCLUDE; their
    selection is a float-rounding coin toss and is not compared."""
    l32 = router_logits(x_bits, w_router, bias)
    T, E = l32.shape
    idx = np.zeros((T, k), dtype=np.int64)
    w = np.zeros((T, k), dtype=np.float64)
    near = np.zeros(T, dtype=bool)
    for t in range(T):
        s = select_topk(l32[t], k)
        idx[t] = s
        w[t] = pick_weights(l32[t], s, renorm)
        if k < E:
            srt = np.sort(l32[t].astype(np.float64))[::-1]
            near[t] = (srt[k - 1] - srt[k]) < GAP_EXCLUDE
    return idx, w, l32, near


def silu(z):
    return z / (1.0 + np.exp(-z))


def expert_ffn(x_row, w_gate_e, w_up_e, w_down_e) -> np.ndarray:
    """Step 5 for one token and one expert: [H] float64 x bf16 weights ->
    float64 [H].  The activation is stored as bf16 before the down matrix."""
    g = bf16.to_f64(w_gate_e) @ x_row
    u = bf16.to_f64(w_up_e) @ x_row
    a = bf16.round_f64(silu(g) * u)
    return bf16.to_f64(w_down_e) @ a


def moe_block(x_bits, w_router, w_gate, w_up, w_down, k: int, ws_gate=None, ws_up=None,
              ws_down=None, residual=None, bias=None, renorm: bool = True, routing=None):
    """Steps 1-7 for a block.  Weight arguments are indexable by expert id
    (numpy [E][..] uint16 arrays or lazy per-expert views).  ``routing`` =
    (idx, w, near_tie) replaces steps 2-4 (e.g. the block coreset selector's
    routing, oracle.coreset); slots with id -1 hold no expert.

    Returns dict: y (uint16 bf16 bits [T][H]), y_f64 (the value before the
    final rounding), idx, w, logits, near_tie, counts ([E] tokens per expert),
    touched (number of distinct routed experts)."""
    if routing is None:
        idx, w, l32, near = route(x_bits, w_router, k, bias, renorm)
    else:
        idx, w, near = (np.asarray(a) for a in routing)
        l32 = router_logits(x_bits, w_router, bias)
    x = bf16.to_f64(x_bits)
    T, H = x.shape
    E = l32.shape[1]
    out = np.zeros((T, H), dtype=np.float64)
    if residual is not None:
        out += bf16.to_f64(residual)
    for t in range(T):
        acc = np.zeros(H, dtype=np.float64)
        for j in range(k):
            e = int(idx[t, j])
            if e < 0:
                continue
            acc += w[t, j] * expert_ffn(x[t], w_gate[e], w_up[e], w_down[e])
        if ws_gate is not None:
            acc += expert_ffn(x[t], ws_gate, ws_up, ws_down)
        out[t] += acc
    picks = idx.reshape(-1)
    counts = np.bincount(picks[picks >= 0], minlength=E)
    return {
        "y": bf16.from_f64(out),
        "y_f64": out,
        "idx": idx,
        "w": w,
        "logits": l32,
        "near_tie": near,
        "counts": counts,
        "touched": int((counts > 0).sum()),
    }

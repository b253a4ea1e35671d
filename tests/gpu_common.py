"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the oracle on the same tensors."""
import sys

import numpy as np
import torch

import synth
from oracle import bf16, head as ohead, moe as omoe

# Contract tolerance for bf16-stored, fp32-accumulated outputs.
ATOL = 1e-2
RTOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits_to_f64(t: torch.Tensor) -> np.ndarray:
    return bf16.to_f64(synth.bf16_bits(t))


def assert_bf16_close(gpu: torch.Tensor, ref_bits: np.ndarray, rows=None, what="y"):
    g = bits_to_f64(gpu)
    o = bf16.to_f64(ref_bits)
    if rows is not None:
        g, o = g[rows], o[rows]
    err = np.abs(g - o)
    tol = ATOL + RTOL * np.abs(o)
    exact = float(np.mean(g == o)) if g.size else 1.0
    say(f"  {what}: max|err|={err.max() if err.size else 0:.3e} "
        f"max err/tol={np.max(err / tol) if err.size else 0:.3f} bit-exact={exact:.4f}")
    assert np.all(err <= tol), f"{what}: {np.sum(err > tol)} elements beyond tolerance"
    return exact


def packed(lib_mod, t):
    return None if t is None else lib_mod.bdm_pack_weights(t)


def run_moe(lib_mod, inp: synth.MoEInputs, renorm=True, residual=True, shared=True, layout=0):
    """layout 0: row-major weights; 1: the library packs them first (MFMA
    tiles); 2: gate/up packed as pairs (bdm_pack_gate_up), down as tiles."""
    s = inp.shape
    dev = inp.x.device
    W = (inp.w_gate, inp.w_up, inp.w_down, inp.ws_gate, inp.ws_up, inp.ws_down)
    if layout == 1:
        W = tuple(packed(lib_mod, t) for t in W)
    elif layout == 2:
        g, u = lib_mod.bdm_pack_gate_up(inp.w_gate, inp.w_up)
        sg, su = (lib_mod.bdm_pack_gate_up(inp.ws_gate, inp.ws_up) if inp.ws_gate is not None
                  else (None, None))
        W = (g, u, packed(lib_mod, inp.w_down), sg, su, packed(lib_mod, inp.ws_down))
    idx = torch.full((s.T, s.k), -1, dtype=torch.int32, device=dev)
    w = torch.full((s.T, s.k), float("nan"), dtype=torch.float32, device=dev)
    y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device=dev)
    lib_mod.bdm_moe_block_forward(
        inp.x, inp.w_router, W[0], W[1], W[2], s.k,
        router_bias=inp.router_bias,
        ws_gate=W[3] if shared else None, ws_up=W[4] if shared else None,
        ws_down=W[5] if shared else None,
        residual=inp.residual if residual else None, y=y, topk_idx=idx, topk_w=w,
        renorm=renorm)
    torch.cuda.synchronize()
    return y, idx, w


def oracle_moe(inp: synth.MoEInputs, renorm=True, residual=True, shared=True, tokens=None,
               lazy=False):
    h = synth.moe_host(inp, lazy=lazy)
    x = h["x"] if tokens is None else h["x"][tokens]
    r = h["residual"] if (residual and h["residual"] is not None) else None
    if r is not None and tokens is not None:
        r = r[tokens]
    return omoe.moe_block(x, h["w_router"], h["w_gate"], h["w_up"], h["w_down"], h["k"],
                          h["ws_gate"] if shared else None, h["ws_up"] if shared else None,
                          h["ws_down"] if shared else None, residual=r,
                          bias=h["router_bias"], renorm=renorm)


def compare_moe(y, idx, w, o, tokens=None):
    """idx exact and weights close on tokens away from a top-k near tie;
    y within the contract tolerance on the same tokens."""
    T = idx.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    keep = ~o["near_tie"]
    gi = idx.cpu().numpy()[tok]
    gw = w.cpu().numpy()[tok]
    say(f"  tokens compared: {int(keep.sum())}/{len(tok)} (near-tie excluded: {int((~keep).sum())})")
    assert np.array_equal(gi[keep], o["idx"][keep]), "top-k expert indices differ"
    np.testing.assert_allclose(gw[keep], o["w"][keep], rtol=2e-5, atol=1e-6)
    yy = y[torch.as_tensor(tok, device=y.device)] if tokens is not None else y
    return assert_bf16_close(yy, o["y"], rows=np.flatnonzero(keep))


def run_head(lib_mod, blk: synth.HeadInputs, threshold=0.95, fallback=True, layout=0):
    s = blk.shape
    dev = blk.h.device
    w_head = packed(lib_mod, blk.w_head) if layout else blk.w_head
    tokens = blk.tokens.clone().to(dev)
    am = torch.full((s.T,), -1, dtype=torch.int32, device=dev)
    cf = torch.full((s.T,), float("nan"), dtype=torch.float32, device=dev)
    nc = torch.full((1,), -1, dtype=torch.int32, device=dev)
    lib_mod.bdm_lm_head_unmask(blk.h, w_head, s.mask_id, threshold, fallback, tokens,
                               argmax=am, conf=cf, n_committed=nc)
    torch.cuda.synchronize()
    return tokens, am, cf, nc


def oracle_head(blk: synth.HeadInputs, threshold=0.95, fallback=True):
    o = ohead.head_unmask(synth.bf16_bits(blk.h), synth.bf16_bits(blk.w_head),
                          blk.tokens.cpu().numpy(), blk.shape.mask_id, threshold, fallback)
    o["mask_id"] = blk.shape.mask_id
    return o


def compare_head(out, o, tokens_in):
    """argmax exact and conf close on rows away from a tie; commit decisions
    exact unless a row sits within 1e-4 of the threshold or the fallback pick
    is a near tie."""
    tokens, am, cf, nc = [t.cpu().numpy() for t in out]
    excl = o["near_tie"] | o["near_threshold"]
    keep = ~excl
    say(f"  rows compared: {int(keep.sum())}/{len(keep)}; oracle commits {o['n_committed']}, "
        f"gpu commits {int(nc[0])}")
    assert np.array_equal(am[keep], o["argmax"][keep]), "argmax differs"
    np.testing.assert_allclose(cf, o["conf"], rtol=2e-5, atol=1e-9)
    if not excl.any() and not o["fallback_tie"]:
        assert np.array_equal(tokens, o["tokens"]), "unmask decisions differ"
        assert int(nc[0]) == o["n_committed"]
    else:
        # rows away from a threshold/argmax tie must still agree
        assert np.array_equal(tokens[keep], o["tokens"][keep])
    # rows that were already committed never change
    done = np.asarray(tokens_in) != o["mask_id"]
    assert np.array_equal(tokens[done], np.asarray(tokens_in)[done])

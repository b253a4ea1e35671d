"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties an oracle function to a fact it cannot have made up: a figure
printed on the pages (tests/golden/page_counts.json, each with its citation),
a closed form, a special case that reduces to a library routine, an invariant
of the definition, or the dense fp64 brute force (a different algorithm).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import bf16, brute, counts, head, moe, norm, stack

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_counts.json")))


def g(key):
    return GOLD[key]


# --------------------------------------------------------------------------
# bf16 conversions
# --------------------------------------------------------------------------

def test_bf16_roundtrip_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16.to_f64(bits)
    back = bf16.from_f64(vals)
    finite = np.isfinite(vals)
    assert np.array_equal(back[finite], bits[finite])
    assert np.array_equal(back[np.isinf(vals)], bits[np.isinf(vals)])
    assert np.all(np.isnan(bf16.to_f64(back[np.isnan(vals)])))


def test_bf16_ties_to_even_and_torch_agreement():
    # 1 + 2^-8 is exactly half-way between 1 and 1 + 2^-7: ties to even -> 1
    assert bf16.from_f64(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 is half-way between 1+2^-7 (odd) and 1+2^-6 (even) -> 1+2^-6
    assert bf16.to_f64(bf16.from_f64(1.0 + 3 * 2.0 ** -8)) == 1.0 + 2.0 ** -6
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    ours = bf16.from_f64(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


# --------------------------------------------------------------------------
# The pages' integers and figures
# --------------------------------------------------------------------------

D = counts.ModelDims(layers=g("layers")["value"], hidden=g("hidden")["value"],
                     experts=g("experts")["value"], top_k=g("top_k")["value"],
                     vocab=g("vocab")["value"])


def test_page_parameter_counts():
    assert counts.expert_params(D) == g("expert_params")["value"]
    assert round(counts.expert_params(D) * 2 / 1e6, 2) == g("expert_MB_bf16")["value"]
    assert counts.routed_params(D) == g("routed_params")["value"]
    total = g("total_params")["value"]
    assert round(100 * counts.routed_params(D) / total, 2) == g("routed_percent")["value"]
    assert counts.head_params(D) == g("head_params")["value"]
    assert counts.active_routed_params(D) == g("active_routed_params")["value"]
    others = counts.others_from_total(D, total)
    assert others == g("others_params")["value"]
    active = counts.active_routed_params(D) + others
    assert active == g("active_params")["value"]
    assert round(active * 2 / 1e9, 2) == g("active_GB_bf16")["value"]
    assert round(100 * counts.head_params(D) / total, 2) == g("head_percent_of_total")["value"]
    assert round(100 * counts.head_params(D) / active) == g("head_percent_of_active")["value"]


def test_page_union_and_bytes():
    u = counts.expected_union(D.experts, D.top_k, g("block_size")["value"])
    assert round(u) == g("union_32_tokens")["value"]
    assert abs(u - g("union_32_tokens")["simulated"]) < 0.5
    step_B = u * D.layers * counts.expert_params(D) * 2
    assert round(step_B / 1e9) == g("union_GB_per_step")["value"]
    assert round(counts.routed_params(D) * 2 / 1e9) == g("experts_GB_total")["value"]


def test_page_bandwidth_ceilings_and_round_budget():
    per_tok = g("active_params")["value"] * 2
    c1 = counts.decode_ceiling_tok_s(4.8e12, per_tok)
    c2 = counts.decode_ceiling_tok_s(8.0e12, per_tok)
    assert round(c1) == g("ceiling_h200_tok_s")["value"]
    assert round(c2) == g("ceiling_gb300_tok_s")["value"]
    assert round(100 * 515 / c1) == g("share_515")["value"]
    assert round(100 * 680 / c2) == g("share_680")["value"]
    dense = g("dense_GB_bf16")["value"] * 1e9
    rb = counts.round_bytes(D, dense, 64, 163)
    t, need = counts.tokens_per_round_needed(rb, 4.8e12, 0.60, 515)
    ref = g("round_h200_60pct_64_163")
    assert round(rb / 1e9) == ref["GB"]
    assert round(t * 1e3, 1) == ref["ms"]
    assert round(need, 1) == ref["tokens"]
    rb2 = counts.round_bytes(D, dense, 64, 64)
    _, need2 = counts.tokens_per_round_needed(rb2, 4.8e12, 0.60, 515)
    assert round(rb2 / 1e9) == g("round_h200_60pct_64_64")["GB"]
    assert round(need2, 1) == g("round_h200_60pct_64_64")["tokens"]
    rb3 = counts.round_bytes(D, dense, 32, 64)
    _, need3 = counts.tokens_per_round_needed(rb3, 4.8e12, 0.80, 515)
    assert round(need3, 1) == g("round_h200_80pct_32_64")["tokens"]


def test_oracle_tensor_shapes_match_page_counts():
    """The oracle consumes exactly the per-expert and head tensor sizes the
    page counts (gate [I][H] + up [I][H] + down [H][I]; head [V][H])."""
    s = synth.MoEShape(T=1, H=D.hidden, E=1, I=D.inter, k=1)
    per = s.I * s.H + s.I * s.H + s.H * s.I
    assert per == g("expert_params")["value"]
    assert synth.HEAD.V * synth.HEAD.H == g("head_params")["value"]
    assert synth.LAYER.T == g("block_size")["value"]
    assert synth.HEAD.mask_id == g("mask_token_id")["value"]


def test_union_of_routed_experts_matches_page_simulation():
    """The oracle's router on the Clover-shaped layer's router weights and 20
    seeded 32-token blocks touches about 163 experts per block, the page's
    closed form and simulation for independent routing."""
    wr = synth.moe_router(synth.LAYER, 0).numpy()
    us = []
    for b in range(1, 21):
        x, _, _ = synth.moe_tokens(synth.LAYER, b)
        idx, w, l32, near = moe.route(synth.bf16_bits(x), wr, synth.LAYER.k)
        us.append(len(np.unique(idx)))
    assert 160.0 < np.mean(us) < 166.5, us


@pytest.mark.parametrize("nblocks", [2, 4])
def test_union_of_multiblock_batch_matches_closed_form(nblocks):
    """Several 32-token blocks in one call: the union of routed experts grows
    as the page's closed form for independent routing, generalised to T
    tokens, 256 (1 - (248/256)^T): 222.4 at 64 tokens, 251.7 at 128."""
    from oracle import counts
    shape = synth.MoEShape(T=32 * nblocks, H=2048, E=256, I=512, k=8)
    wr = synth.moe_router(shape, 0).numpy()
    us = []
    for b in range(1, 7):
        x, _, _ = synth.moe_tokens(shape, 700 + b)
        idx, _, _, _ = moe.route(synth.bf16_bits(x), wr, shape.k)
        us.append(len(np.unique(idx)))
    ref = counts.expected_union(256, 8, shape.T)
    assert abs(np.mean(us) - ref) < 0.015 * ref, (us, ref)


# --------------------------------------------------------------------------
# Router / top-k
# --------------------------------------------------------------------------

def _identity_router(L):
    """x = identity (exact in bf16), w_router = L^T  ->  logits == L exactly."""
    T, E = L.shape
    x = bf16.from_f64(np.eye(T))
    return x, np.ascontiguousarray(L.T.astype(np.float32))


@pytest.mark.parametrize("renorm", [True, False])
def test_route_matches_torch_softmax_topk(renorm):
    rng = np.random.default_rng(11)
    L = rng.standard_normal((64, 48)).astype(np.float32)
    x, wr = _identity_router(L)
    # the identity trick needs H == T; w_router is [E][H] with H = 64
    idx, w, l32, near = moe.route(x, wr, 6, renorm=renorm)
    assert np.array_equal(l32, L)
    tl = torch.from_numpy(L).double()
    tv, ti = torch.topk(tl, 6, dim=1, largest=True, sorted=True)
    assert np.array_equal(idx, ti.numpy())
    p = torch.softmax(tl, dim=1)
    ref = torch.gather(p, 1, ti)
    if renorm:
        ref = torch.softmax(tv, dim=1)
    np.testing.assert_allclose(w, ref.numpy(), rtol=1e-12, atol=1e-15)


def test_uniform_router_ties_pick_lowest_ids():
    s = synth.TINY
    inp = synth.tiny_inputs()
    h = synth.moe_host(inp)
    idx, w, _, near = moe.route(h["x"], np.zeros((s.E, s.H), np.float32), s.k)
    assert np.all(idx == np.arange(s.k)[None, :])
    np.testing.assert_allclose(w, 1.0 / s.k, rtol=1e-15)
    assert near.all()


def test_renormalised_weights_sum_to_one():
    inp = synth.moe_inputs(synth.MoEShape(T=64, H=64, E=32, I=32, k=5), seed=3)
    h = synth.moe_host(inp)
    _, w, _, _ = moe.route(h["x"], h["w_router"], 5)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)          # listed by decreasing weight
    _, w2, _, _ = moe.route(h["x"], h["w_router"], 5, renorm=False)
    assert np.all(w2.sum(axis=1) < 1.0)


# --------------------------------------------------------------------------
# MoE layer
# --------------------------------------------------------------------------

def _run_oracle(h, **kw):
    return moe.moe_block(h["x"], h["w_router"], h["w_gate"], h["w_up"], h["w_down"], h["k"],
                         h["ws_gate"], h["ws_up"], h["ws_down"], residual=kw.get("residual"),
                         bias=kw.get("bias"), renorm=kw.get("renorm", True))


def _run_brute(h, **kw):
    return brute.moe_dense(h["x"], h["w_router"], h["w_gate"], h["w_up"], h["w_down"], h["k"],
                           h["ws_gate"], h["ws_up"], h["ws_down"], residual=kw.get("residual"),
                           bias=kw.get("bias"), renorm=kw.get("renorm", True))


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("variant", ["plain", "residual", "bias", "norenorm", "noshared"])
def test_moe_matches_dense_brute_force(seed, variant):
    shape = synth.TINY if variant != "noshared" else synth.MoEShape(8, 64, 16, 32, 2, shared=False)
    inp = synth.moe_inputs(shape, seed=seed, block_seed=seed + 1,
                           with_residual=(variant == "residual"),
                           zipf_s=1.1 if variant == "bias" else None)
    h = synth.moe_host(inp)
    kw = {"residual": h["residual"], "bias": h["router_bias"], "renorm": variant != "norenorm"}
    o = _run_oracle(h, **kw)
    yb, G, yf = _run_brute(h, **kw)
    np.testing.assert_allclose(o["y_f64"], yf, rtol=1e-12, atol=1e-12)
    assert np.array_equal(o["y"], yb)
    # the dense gate matrix holds exactly the oracle's (idx, w)
    for t in range(shape.T):
        nz = np.flatnonzero(G[t])
        assert set(nz) == set(o["idx"][t])
        np.testing.assert_allclose(G[t, o["idx"][t]], o["w"][t], rtol=1e-13)


def test_moe_tiny_fp32_originals_bound():
    """The tiny workload is specified in fp32; the bf16-rounded inputs the
    kernels take change the fp32-exact, unrounded result only by bf16-level
    amounts (a sanity bound on the rounding reading)."""
    inp = synth.tiny_inputs()
    h = synth.moe_host(inp)
    o = _run_oracle(h)
    f = inp.fp32
    f32_bits = lambda t: bf16.from_f64(t.double().numpy())  # noqa: E731
    # exact fp64 evaluation on the fp32 originals, no rounding of the activation
    x64 = f["x"].double().numpy()
    _, _, yf = brute.moe_dense(bf16.from_f64(x64), h["w_router"], f32_bits(f["w_gate"]),
                               f32_bits(f["w_up"]), f32_bits(f["w_down"]), h["k"],
                               f32_bits(f["ws_gate"]), f32_bits(f["ws_up"]),
                               f32_bits(f["ws_down"]), round_act=False)
    err = np.abs(o["y_f64"] - yf)
    assert err.max() < 0.05 * max(1.0, np.abs(yf).max())
    _ = f32_bits


def test_single_expert_reduces_to_torch_swiglu():
    """E = 1, k = 1: the layer is the textbook dense SwiGLU FFN plus the shared
    one, y = x + W_d (silu(W_g x) * W_u x) + S(x), here with torch's silu."""
    shape = synth.MoEShape(T=8, H=64, E=1, I=32, k=1)
    inp = synth.moe_inputs(shape, seed=4, with_residual=False)
    h = synth.moe_host(inp)
    o = _run_oracle(h, residual=h["x"])
    F = torch.nn.functional
    x = inp.x.double()

    def ffn(wg, wu, wd):
        a = F.silu(x @ wg.double().T) * (x @ wu.double().T)
        a = a.to(torch.bfloat16).double()
        return a @ wd.double().T

    ref = x + ffn(inp.w_gate[0], inp.w_up[0], inp.w_down[0]) + ffn(inp.ws_gate, inp.ws_up,
                                                                       inp.ws_down)
    np.testing.assert_allclose(o["y_f64"], ref.numpy(), rtol=0, atol=1e-4)
    assert np.all(o["w"] == 1.0)


def test_identical_experts_make_routing_irrelevant():
    """All experts equal: y = x + F(x) + S(x) whatever the router picks and
    however it weighs the picks (the renormalised weights sum to one)."""
    shape = synth.MoEShape(T=8, H=64, E=16, I=32, k=4)
    inp = synth.moe_inputs(shape, seed=6)
    h = synth.moe_host(inp)
    for key in ("w_gate", "w_up", "w_down"):
        h[key] = np.repeat(h[key][:1], shape.E, axis=0)
    o1 = _run_oracle(h)
    h2 = dict(h)
    h2["w_router"] = np.random.default_rng(1).standard_normal(h["w_router"].shape).astype(np.float32)
    o2 = _run_oracle(h2)
    assert not np.array_equal(o1["idx"], o2["idx"])
    np.testing.assert_allclose(o1["y_f64"], o2["y_f64"], rtol=0, atol=1e-12)
    one = synth.MoEShape(T=8, H=64, E=1, I=32, k=1)
    h1 = dict(h, w_gate=h["w_gate"][:1], w_up=h["w_up"][:1], w_down=h["w_down"][:1],
              w_router=h["w_router"][:1], k=1)
    o3 = _run_oracle(h1)
    np.testing.assert_allclose(o1["y_f64"], o3["y_f64"], rtol=0, atol=1e-12)
    _ = one


def test_token_permutation_and_expert_relabelling():
    inp = synth.moe_inputs(synth.TINY, seed=8, block_seed=3)
    h = synth.moe_host(inp)
    o = _run_oracle(h)
    perm = np.random.default_rng(2).permutation(synth.TINY.T)
    hp = dict(h, x=h["x"][perm])
    op = _run_oracle(hp)
    assert np.array_equal(op["y"], o["y"][perm])
    ep = np.random.default_rng(3).permutation(synth.TINY.E)
    he = dict(h, w_router=h["w_router"][ep], w_gate=h["w_gate"][ep], w_up=h["w_up"][ep],
              w_down=h["w_down"][ep])
    oe = _run_oracle(he)
    if not o["near_tie"].any():
        assert np.array_equal(oe["y"], o["y"])
        assert np.array_equal(ep[oe["idx"]], o["idx"])


# --------------------------------------------------------------------------
# Head and unmask rule
# --------------------------------------------------------------------------

def _onehot_head(V, rows):
    """Build h [T][64] and W [V][64] so that row t's logits are exactly
    rows[t] (a dict vocab id -> logit, all others 0): h_t = e_t, W[v][t] = l."""
    T = len(rows)
    H = 64
    h = np.zeros((T, H))
    W = np.zeros((V, H))
    for t, r in enumerate(rows):
        h[t, t] = 1.0
        for v, val in r.items():
            W[v, t] = val
    return bf16.from_f64(h), bf16.from_f64(W)


def test_head_closed_form_confidence_and_threshold():
    V, mask = 512, 0
    bstar = math.log(19 * (V - 2))                 # conf crosses 0.95 here
    assert 9.0 < bstar < 9.5
    rows = [{7: 9.0}, {8: 9.5}, {9: 12.0}, {10: 9.5, mask: 100.0}, {}, {11: 9.5}]
    hb, Wb = _onehot_head(V, rows)
    tokens = np.array([mask, mask, mask, mask, mask, 123])
    r = head.head_unmask(hb, Wb, tokens, mask, 0.95, fallback=True)
    for t, b in ((0, 9.0), (1, 9.5), (2, 12.0), (3, 9.5), (5, 9.5)):
        closed = math.exp(b) / (math.exp(b) + V - 2)
        assert r["conf"][t] == pytest.approx(closed, rel=1e-12)
    assert list(r["argmax"][:4]) == [7, 8, 9, 10]     # mask column (100.0) never chosen
    assert r["conf"][4] == pytest.approx(1.0 / (V - 1), rel=1e-12)
    assert r["argmax"][4] == 1                         # all equal: lowest non-mask id
    assert list(r["committed"]) == [False, True, True, True, False, False]
    assert list(r["tokens"]) == [mask, 8, 9, 10, mask, 123]   # row 5 already committed
    assert r["n_committed"] == 3


def test_head_fallback_commits_exactly_one():
    V, mask = 512, 5
    rows = [{1: 6.0}, {2: 8.0}, {3: 8.0}, {4: 7.0}, {6: 9.0}]
    hb, Wb = _onehot_head(V, rows)
    tokens = np.array([mask, mask, mask, mask, 77])   # the 9.0 row is already committed
    r = head.head_unmask(hb, Wb, tokens, mask, 0.95, fallback=True)
    assert r["n_committed"] == 1
    assert list(r["committed"]) == [False, True, False, False, False]   # tie: lowest position
    assert r["tokens"][1] == 2 and r["tokens"][4] == 77
    r2 = head.head_unmask(hb, Wb, tokens, mask, 0.95, fallback=False)
    assert r2["n_committed"] == 0
    r3 = head.head_unmask(hb, Wb, np.array([9, 9, 9, 9, 9]), mask, 0.95, fallback=True)
    assert r3["n_committed"] == 0                     # nothing masked: no-op


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_head_matches_dense_brute_force_and_torch(seed):
    shape = synth.TINY_HEAD
    W = synth.head_weights(shape, seed)
    blk = synth.head_block(shape, W, block_seed=seed + 1, n_boost=3, mask_boost_rows=2)
    hb, Wb = synth.bf16_bits(blk.h), synth.bf16_bits(W)
    r = head.head_unmask(hb, Wb, blk.tokens.numpy(), shape.mask_id, 0.95)
    a, conf = brute.head_dense(hb, Wb, shape.mask_id)
    assert np.array_equal(a, r["argmax"])
    np.testing.assert_allclose(conf, r["conf"], rtol=1e-12)
    l = torch.from_numpy(r["logits"]).double()
    keep = torch.ones(shape.V, dtype=torch.bool)
    keep[shape.mask_id] = False
    p = torch.softmax(l[:, keep], dim=1)
    np.testing.assert_allclose(p.max(dim=1).values.numpy(), r["conf"], rtol=1e-12)
    ids = torch.arange(shape.V)[keep]
    assert np.array_equal(ids[p.argmax(dim=1)].numpy(), r["argmax"])
    # the boosted rows of the recipe commit, the flat ones do not
    for t in range(shape.T):
        if t in blk.boosted_rows:
            assert r["committed"][t] and r["tokens"][t] == blk.boosted_tokens[
                blk.boosted_rows.index(t)]
        elif t not in blk.mask_boost_rows:
            assert r["conf"][t] < 0.5


# --------------------------------------------------------------------------
# RMSNorm and the stack
# --------------------------------------------------------------------------

def test_rmsnorm_matches_torch_and_unit_rms():
    x = torch.randn(16, 256, generator=torch.Generator().manual_seed(0)) * 3
    xb = synth.bf16_bits(x.to(torch.bfloat16))
    ours = bf16.to_f64(norm.rmsnorm(xb, 1e-6))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(bf16.to_f64(xb)), (256,), eps=1e-6)
    np.testing.assert_allclose(ours, bf16.round_f64(ref.numpy()), rtol=0, atol=0)
    rms = np.sqrt(np.mean(ours ** 2, axis=1))
    np.testing.assert_allclose(rms, 1.0, atol=4e-3)


def test_stack_tokens_independent_and_matches_chained_brute():
    s = synth.TINY
    layers = []
    for l in range(3):
        inp = synth.moe_inputs(s, seed=100 + l)
        h = synth.moe_host(inp)
        layers.append(h)
    x, _, _ = synth.moe_tokens(s, 9)
    xb = synth.bf16_bits(x)
    y, near = stack.stack_forward(xb, layers, s.k)
    ysub, _ = stack.stack_forward(xb, layers, s.k, tokens=[1, 5])
    assert np.array_equal(ysub, y[[1, 5]])
    cur = xb
    for h in layers:
        xn = torch.nn.functional.rms_norm(torch.from_numpy(bf16.to_f64(cur)), (s.H,), eps=1e-6)
        xn = bf16.from_f64(xn.numpy())
        cur, _, _ = brute.moe_dense(xn, h["w_router"], h["w_gate"], h["w_up"], h["w_down"], s.k,
                                    h["ws_gate"], h["ws_up"], h["ws_down"], residual=cur)
    assert np.array_equal(cur, y)


def test_stack_forced_picks():
    """Routing forced to given picks (for chained comparisons): the stack's
    own picks give the plain stack bit for bit; with every expert identical
    the output does not depend on the picks (their weights still sum to 1),
    so arbitrary forced picks give the plain stack too."""
    s = synth.TINY
    layers = [synth.moe_host(synth.moe_inputs(s, seed=110 + l)) for l in range(3)]
    x, _, _ = synth.moe_tokens(s, 4)
    xb = synth.bf16_bits(x)
    y, _ = stack.stack_forward(xb, layers, s.k)
    own, cur = [], xb
    for h in layers:
        xn = norm.rmsnorm(cur, 1e-6)
        r = moe.moe_block(xn, h["w_router"], h["w_gate"], h["w_up"], h["w_down"], s.k,
                          h["ws_gate"], h["ws_up"], h["ws_down"], residual=cur)
        own.append(r["idx"])
        cur = r["y"]
    yf, _ = stack.stack_forward(xb, layers, s.k, picks=own)
    assert np.array_equal(yf, y)
    same = []
    for h in layers:
        g = dict(h)
        for n in ("w_gate", "w_up", "w_down"):
            g[n] = np.repeat(h[n][:1], s.E, axis=0)
        same.append(g)
    rng = np.random.default_rng(3)
    rand = [np.stack([rng.choice(s.E, s.k, replace=False) for _ in range(s.T)]) for _ in same]
    ys, _ = stack.stack_forward(xb, same, s.k)
    yr, _ = stack.stack_forward(xb, same, s.k, picks=rand)
    np.testing.assert_allclose(bf16.to_f64(yr), bf16.to_f64(ys), rtol=0, atol=0.04)
    assert np.mean(yr == ys) > 0.98


# --------------------------------------------------------------------------
# Block coreset expert selector (files page, "The expert selection")
# --------------------------------------------------------------------------

# The page's simulation of the selector at top_p 0.9 on synthetic logits
# (per-token N(0,1) noise plus a block-wide N(0,1) preference of the given
# weight): experts touched before the selector, experts kept, and slots of a
# token's 8 that are re-routed.  (union, kept, rerouted) per weight.
PAGE_CORESET_SIM = {0: (163.4, 126.7, 1.1), 1: (79.0, 45.5, 1.2), 2: (40.8, 16.2, 1.6),
                    3: (27.5, 8.6, 2.5)}


@pytest.mark.parametrize("weight", [0, 1, 2, 3])
def test_coreset_reproduces_page_simulation(weight):
    from oracle import coreset
    rng = np.random.default_rng(100 + weight)
    union, kept, rer = coreset.simulate(weight, 400, rng)
    pu, pk, pr = PAGE_CORESET_SIM[weight]
    # the page's figures carry their own sampling error; 400 blocks here
    assert abs(union - pu) <= (0.02 if weight < 2 else 0.04) * pu, (union, pu)
    assert abs(kept - pk) <= (0.03 if weight < 2 else 0.07) * pk, (kept, pk)
    assert abs(rer - pr) <= (0.12 if weight < 3 else 0.3), (rer, pr)


def _identical_block(T, E, top, k):
    """T identical tokens: logits `top` on experts 0..len(top)-1, -8 elsewhere."""
    l = np.full((T, E), -8.0, dtype=np.float32)
    l[:, :len(top)] = np.asarray(top, dtype=np.float32)
    return l


def test_coreset_closed_form_identical_tokens():
    """Identical tokens with top logits 3, 2, 1, 0 and k = 4: the masses are
    T times the softmax probabilities, so the cumulative shares of the kept
    prefix are e^3, e^3+e^2, ... over e^3+e^2+e+1 (0.644, 0.881, 0.968, 1):
    top_p 0.9 keeps 3 experts, 0.85 keeps 2, 0.5 keeps 1; each token then
    routes to the kept experts with weights softmax over their logits."""
    from oracle import coreset
    E, T, k = 12, 8, 4
    l = _identical_block(T, E, [3, 2, 1, 0], k)
    e = np.exp(np.array([3.0, 2.0, 1.0, 0.0]))
    share = np.cumsum(e) / e.sum()
    assert share[1] < 0.9 <= share[2] and share[0] < 0.85 <= share[1]
    for top_p, n in ((0.9, 3), (0.85, 2), (0.5, 1), (0.99, 4)):
        r = coreset.coreset_route(l, k, top_p, block=T)
        assert r["n_kept"][0] == n
        assert list(r["kept"][0]) == list(range(n))
        for t in range(T):
            assert list(r["idx"][t, :n]) == list(range(n))
            assert np.all(r["idx"][t, n:] == -1) and np.all(r["w"][t, n:] == 0)
            np.testing.assert_allclose(r["w"][t, :n], e[:n] / e[:n].sum(), rtol=1e-6)
        assert np.all(r["rerouted"] == k - n)


def test_coreset_equal_masses_keep_lower_id():
    """Two experts with equal logits in every token have equal masses; a cut
    between them keeps the lower id."""
    from oracle import coreset
    l = _identical_block(4, 10, [1.0, 1.0], 2)
    r = coreset.coreset_route(l, 2, 0.5, block=4)
    assert list(r["kept"][0]) == [0]
    assert np.all(r["idx"][:, 0] == 0) and np.all(r["idx"][:, 1] == -1)
    np.testing.assert_allclose(r["w"][:, 0], 1.0)


def test_coreset_top_p_one_keeps_routing_and_tiny_top_p_keeps_one():
    from oracle import coreset
    rng = np.random.default_rng(7)
    l = rng.standard_normal((32, 64)).astype(np.float32)
    k = 4
    full = coreset.coreset_route(l, k, 1.0)
    first = np.stack([moe.select_topk(l[t], k) for t in range(32)])
    assert full["n_kept"][0] == len(np.unique(first))
    assert np.array_equal(full["idx"], first)
    p = moe.softmax(l)
    for t in range(32):
        ps = p[t, first[t]]
        np.testing.assert_allclose(full["w"][t], ps / ps.sum(), rtol=1e-12)
    assert np.all(full["rerouted"] == 0)
    one = coreset.coreset_route(l, k, 1e-9)
    top = coreset.block_coreset(l, k, 1e-9)["order"][0]
    assert one["n_kept"][0] == 1 and one["kept"][0][0] == top
    assert np.all(one["idx"][:, 0] == top) and np.all(one["idx"][:, 1:] == -1)
    np.testing.assert_allclose(one["w"][:, 0], 1.0)


def test_coreset_sets_nest_and_restrict_routing():
    """Kept sets are prefixes of one mass order, so they nest as top_p
    grows; every token's picks lie in its block's kept set, and a token
    whose first-pass picks were all kept keeps its routing."""
    from oracle import coreset
    rng = np.random.default_rng(11)
    pref = rng.standard_normal(128)
    l = (rng.standard_normal((64, 128)) + 1.0 * pref[None, :]).astype(np.float32)
    k = 8
    prev = None
    for top_p in (0.3, 0.6, 0.9, 0.99):
        r = coreset.coreset_route(l, k, top_p, block=32)
        for b in range(2):
            kept = set(r["kept"][b].tolist())
            if prev is not None:
                assert prev[b] <= kept
            for t in range(32 * b, 32 * b + 32):
                picks = [e for e in r["idx"][t] if e >= 0]
                assert set(picks) <= kept and len(picks) == min(k, len(kept))
                if set(r["first"][t].tolist()) <= kept:
                    assert list(r["idx"][t]) == list(r["first"][t])
        prev = [set(r["kept"][b].tolist()) for b in range(2)]


# --------------------------------------------------------------------------
# The denoise loop (files page, "How it writes")
# --------------------------------------------------------------------------

def _tiny_model(seed=0, L=3, V=96, H=64, E=8, I=32, k=2):
    rng = np.random.default_rng(seed)
    b = lambda *s, sd=0.02: bf16.from_f64(rng.standard_normal(s) * sd)  # noqa: E731
    layers = [{"w_router": (rng.standard_normal((E, H)) * 0.2).astype(np.float32),
               "w_gate": b(E, I, H), "w_up": b(E, I, H), "w_down": b(E, H, I),
               "ws_gate": b(I, H), "ws_up": b(I, H), "ws_down": b(H, I)} for _ in range(L)]
    return layers, b(V, H, sd=1.0), b(V, H, sd=0.3)


def test_denoise_loop_terminates_commits_and_never_revisits():
    from oracle import denoise
    layers, emb, wh = _tiny_model()
    T, mask = 8, 5
    tokens = np.full(T, mask)
    tokens[3] = 17                              # one slot already committed
    final, commits = denoise.denoise_block(tokens, emb, layers, wh, 2, mask, 0.95)
    assert 1 <= len(commits) <= T - 1
    assert all(c >= 1 for c in commits) and sum(commits) == T - 1
    assert not (final == mask).any() and final[3] == 17
    # the same loop one step at a time: each step's commits stay committed
    cur = tokens.copy()
    for c in commits:
        out = denoise.denoise_step(cur, emb, layers, wh, 2, mask, 0.95)
        done = cur != mask
        assert np.array_equal(out["tokens"][done], cur[done])
        assert out["n_committed"] == c
        cur = out["tokens"]
    assert np.array_equal(cur, final)
    # an unmasked block takes no step
    f2, c2 = denoise.denoise_block(final, emb, layers, wh, 2, mask, 0.95)
    assert c2 == [] and np.array_equal(f2, final)


def test_denoise_step_is_its_parts_composed():
    from oracle import denoise
    layers, emb, wh = _tiny_model(seed=1)
    tokens = np.array([5, 5, 9, 5, 5, 40, 5, 5])
    out = denoise.denoise_step(tokens, emb, layers, wh, 2, 5, 0.95)
    x = emb[tokens]
    for lw in layers:
        xn = norm.rmsnorm(x, 1e-6)
        x = moe.moe_block(xn, lw["w_router"], lw["w_gate"], lw["w_up"], lw["w_down"], 2,
                          lw["ws_gate"], lw["ws_up"], lw["ws_down"], residual=x)["y"]
    ref = head.head_unmask(norm.rmsnorm(x, 1e-6), wh, tokens, 5, 0.95)
    assert np.array_equal(out["tokens"], ref["tokens"])
    np.testing.assert_allclose(out["conf"], ref["conf"], rtol=0, atol=0)


def test_denoise_with_coreset_selector():
    """The loop with the block coreset selector on (the files page, "What
    Clover is": shipped at top_p 0.9).  top_p = 1 keeps every touched expert:
    the step is the plain one bit for bit.  A top_p so small that one expert
    is kept per layer: every token of a layer goes to that expert alone with
    weight 1, so the layer is x + FFN_e(xn) + FFN_shared(xn), computed here
    densely with the single-expert FFN."""
    from oracle import coreset as cs, denoise, stack
    layers, emb, wh = _tiny_model(seed=4)
    tokens = np.array([5, 5, 9, 5, 5, 40, 5, 5])
    plain = denoise.denoise_step(tokens, emb, layers, wh, 2, 5, 0.95)
    full = denoise.denoise_step(tokens, emb, layers, wh, 2, 5, 0.95, coreset_top_p=1.0)
    assert np.array_equal(plain["h"], full["h"]) and np.array_equal(plain["tokens"],
                                                                    full["tokens"])
    x = emb[tokens]
    y, _ = stack.stack_forward(x, layers, 2, coreset_top_p=1e-9, block=8)
    ref = x
    for lw in layers:
        xn = norm.rmsnorm(ref, 1e-6)
        l32 = moe.router_logits(xn, lw["w_router"])
        kept = cs.block_coreset(l32, 2, 1e-9)["kept"]
        assert len(kept) == 1
        e = int(kept[0])
        xf, rf = bf16.to_f64(xn), bf16.to_f64(ref)
        out = np.stack([rf[t] + moe.expert_ffn(xf[t], lw["w_gate"][e], lw["w_up"][e],
                                               lw["w_down"][e])
                        + moe.expert_ffn(xf[t], lw["ws_gate"], lw["ws_up"], lw["ws_down"])
                        for t in range(len(tokens))])
        ref = bf16.from_f64(out)
    assert np.array_equal(y, ref)


def test_unmask_rule_per_block():
    """Several blocks in one call: the rule applies to each block on its own.
    Block 0 has a row above the threshold, block 1 none: per block, block 1
    still commits its most confident masked row (the fallback), while the
    rule over the whole call would commit block 0's row only."""
    from oracle import head as oh
    M = 7
    tokens = np.array([M, M, 3, M, M, M, M, M])
    argmax = np.arange(10, 18)
    conf = np.array([0.97, 0.5, 0.99, 0.2, 0.1, 0.6, 0.3, 0.6], dtype=np.float32)
    whole, wc = oh.unmask(tokens, argmax, conf, M, 0.95)
    assert list(np.flatnonzero(wc)) == [0]
    per, pc = oh.unmask(tokens, argmax, conf, M, 0.95, block=4)
    assert list(np.flatnonzero(pc)) == [0, 5]         # equal confidences: lower position
    assert per[5] == 15 and per[7] == M and per[2] == 3


def test_denoise_multiblock_equals_blocks_alone():
    """Three blocks of six slots denoised together: tokens never interact and
    each block has its own rule, so the result is each block's own loop, and
    every step commits at least one slot of every block still masked."""
    from oracle import denoise
    layers, emb, wh = _tiny_model(seed=5)
    rng = np.random.default_rng(8)
    tokens = np.full(18, 5)
    tokens[[1, 8, 15]] = rng.integers(10, 90, 3)
    final, commits = denoise.denoise_block(tokens, emb, layers, wh, 2, 5, 0.95, block=6)
    alone = [denoise.denoise_block(tokens[b:b + 6], emb, layers, wh, 2, 5, 0.95)
             for b in range(0, 18, 6)]
    assert np.array_equal(final, np.concatenate([f for f, _ in alone]))
    assert len(commits) == max(len(c) for _, c in alone)
    for i, c in enumerate(commits):
        assert c == sum(cs[i] for _, cs in alone if i < len(cs))


def test_denoise_confident_block_finishes_in_one_step():
    """A threshold no probability can miss (0 < conf always) commits every
    masked slot in the first step; a threshold above 1 commits one per step."""
    from oracle import denoise
    layers, emb, wh = _tiny_model(seed=2)
    tokens = np.full(6, 3)
    final, commits = denoise.denoise_block(tokens, emb, layers, wh, 2, 3, 0.0)
    assert commits == [6] and not (final == 3).any()
    final, commits = denoise.denoise_block(tokens, emb, layers, wh, 2, 3, 1.5)
    assert commits == [1] * 6


# --------------------------------------------------------------------------
# Self-speculative verify epilogue (files page, "Two ways to run it")
# --------------------------------------------------------------------------

def test_verify_bound_matches_page_points():
    """The page's prose: with the defaults the ratio never binds; the bound is
    0.6 for a certain model (H = 0) and 0.22 at one nat."""
    from oracle import verify
    assert verify.bound(0.0) == pytest.approx(0.6)
    assert verify.bound(1.0) == pytest.approx(0.2207, abs=5e-5)
    assert np.all(verify.bound(np.linspace(0, 10, 101)) <= 0.6)
    # a larger delta lets the ratio bind at low entropy
    assert verify.bound(0.0, delta=3.0) == pytest.approx(0.9)
    assert verify.bound(2.0, delta=3.0) == pytest.approx(3.0 * math.exp(-2.0))


def _rows_with_logits(rows, H=32):
    """bf16 hidden rows e_0 .. and an identity-like head so that the logits of
    row t are exactly rows[t] (vocabulary = H)."""
    V = H
    w = np.zeros((V, H), dtype=np.float64)
    w[np.arange(V), np.arange(V)] = 1.0
    h = np.zeros((len(rows), H), dtype=np.float64)
    for t, r in enumerate(rows):
        h[t, :len(r)] = r
    return bf16.from_f64(h), bf16.from_f64(w)


def test_verify_entropy_and_probabilities_closed_form():
    """Logits with n equal maxima and the rest at -30 (bf16-exact): H = ln n,
    p = 1/n, so at the defaults p >= 0.6/n is always accepted (the page's
    remark that a lenient bound accepts nearly everything); one dominant
    logit gives H ~ 0 and the bound 0.6."""
    from oracle import verify
    rows = [[2.0] * n + [-30.0] * (32 - n) for n in (1, 2, 4, 8)] + [[0.0] * 32]
    hb, wb = _rows_with_logits(rows)
    cand = [0, 1, 3, 7]
    o = verify.verify(hb, wb, cand, "threshold")
    np.testing.assert_allclose(o["entropy"][:4], np.log([1, 2, 4, 8]), atol=1e-9)
    np.testing.assert_allclose(o["p_cand"], [1, 1 / 2, 1 / 4, 1 / 8], rtol=1e-9)
    assert o["n_accepted"] == 4 and o["tokens"][4] == 0      # bonus: argmax of the last row
    # exact rule: only the argmax (lowest id among equal maxima) is kept
    e = verify.verify(hb, wb, cand, "exact")
    assert list(e["accept"]) == [True, False, False, False] and e["n_accepted"] == 1
    assert list(e["tokens"][:2]) == [0, 0] and np.all(e["tokens"][2:] == -1)


def test_verify_threshold_decision_and_prefix():
    """Two-outcome rows with p = sigmoid(d) for the candidate: accepted iff
    p >= 0.6 e^-H(p); a rejection hides every later acceptance."""
    from oracle import verify

    def row(d):
        return [d, 0.0] + [-60.0] * 30

    def rule(p):
        H = -(p * math.log(p) + (1 - p) * math.log(1 - p))
        return p >= 0.6 * math.exp(-H)
    ds = [4.0, 2.0, -1.0, 0.0, 4.0]             # accepted, accepted, rejected, accepted, accepted
    hb, wb = _rows_with_logits([row(d) for d in ds] + [row(3.0)])
    o = verify.verify(hb, wb, [0] * 5, "threshold")
    ps = [1 / (1 + math.exp(-d)) for d in ds]
    np.testing.assert_allclose(o["p_cand"], ps, rtol=1e-6)
    assert [rule(p) for p in ps] == [True, True, False, True, True]
    assert list(o["accept"]) == [True, True, False, True, True]
    assert o["n_accepted"] == 2
    # the boundary token: row 2's most likely token (column 1: d = -1 < 0)
    assert list(o["tokens"]) == [0, 0, 1, -1, -1, -1]

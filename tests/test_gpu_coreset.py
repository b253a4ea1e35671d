"""GPU parity of the block coreset expert selector (files page, "The expert
selection") against oracle.coreset + the MoE oracle fed its routing.

Bar: per block, the kept-set size exact unless the oracle marks the block a
float-rounding call (cumulative mass within 1e-5 of the cut, boundary
masses within 1e-5, or a first-pass near tie); per token away from a
restricted near tie, the expert ids exact (including the empty -1 slots) and
the weights within 2e-5; outputs within 1e-2 + 2e-2 |ref|.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import coreset as ocs, moe as omoe
from tests.conftest import gpu_available
from tests.gpu_common import assert_bf16_close, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def bdm():
    if not gpu_available():
        pytest.skip("no GPU")
    import block_diffusion_moe_amd as b
    b.load()
    return b


def run_gpu(bdm, inp, top_p, block, layout=1, renorm=True, residual=True):
    s = inp.shape
    W = (inp.w_gate, inp.w_up, inp.w_down, inp.ws_gate, inp.ws_up, inp.ws_down)
    if layout == 1:
        W = tuple(bdm.bdm_pack_weights(t) for t in W)
    elif layout == 2:                                   # gate/up packed as pairs
        g, u = bdm.bdm_pack_gate_up(inp.w_gate, inp.w_up)
        sg, su = bdm.bdm_pack_gate_up(inp.ws_gate, inp.ws_up)
        W = (g, u, bdm.bdm_pack_weights(inp.w_down), sg, su, bdm.bdm_pack_weights(inp.ws_down))
    nb = (s.T + block - 1) // block
    idx = torch.full((s.T, s.k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((s.T, s.k), float("nan"), dtype=torch.float32, device=DEV)
    nk = torch.full((nb,), -1, dtype=torch.int32, device=DEV)
    y = bdm.bdm_moe_block_forward(inp.x, inp.w_router, W[0], W[1], W[2], s.k,
                                  router_bias=inp.router_bias, ws_gate=W[3], ws_up=W[4],
                                  ws_down=W[5], residual=inp.residual if residual else None,
                                  topk_idx=idx, topk_w=w, renorm=renorm, coreset_top_p=top_p,
                                  coreset_block=block, n_kept=nk)
    torch.cuda.synchronize()
    return y, idx.cpu().numpy(), w.cpu().numpy(), nk.cpu().numpy()


def oracle_routing(inp, top_p, block, renorm=True):
    h = synth.moe_host(inp, lazy=True)
    l32 = omoe.router_logits(h["x"], h["w_router"], h["router_bias"])
    return h, ocs.coreset_route(l32, inp.shape.k, top_p, block=block, renorm=renorm)


def compare(bdm_out, inp, h, r, tokens=None, residual=True):
    y, gi, gw, nk = bdm_out
    s = inp.shape
    keep_blk = ~r["near_block"]
    say(f"  kept per block (oracle) {r['n_kept'].tolist()}  gpu {nk.tolist()}  "
        f"near blocks {int((~keep_blk).sum())}")
    assert np.array_equal(nk[keep_blk], r["n_kept"][keep_blk]), "kept-set sizes differ"
    ok = ~r["near_tie"]
    assert np.array_equal(gi[ok], r["idx"][ok]), "coreset routing differs"
    np.testing.assert_allclose(gw[ok], r["w"][ok], rtol=2e-5, atol=1e-6)
    # every GPU pick lies in the GPU block's kept set size bound, ids valid
    assert np.all((gi == -1) | ((gi >= 0) & (gi < s.E)))
    tok = np.arange(s.T) if tokens is None else np.asarray(tokens)
    sel = tok[ok[tok]]
    xs = h["x"][sel]
    res = h["residual"][sel] if (residual and h["residual"] is not None) else None
    o = omoe.moe_block(xs, h["w_router"], h["w_gate"], h["w_up"], h["w_down"], s.k, h["ws_gate"],
                       h["ws_up"], h["ws_down"], residual=res, bias=h["router_bias"],
                       routing=(r["idx"][sel], r["w"][sel], r["near_tie"][sel]))
    yy = y[torch.as_tensor(sel, device=y.device)]
    return assert_bf16_close(yy, o["y"])


@pytest.mark.parametrize("layout", [0, 1])
def test_coreset_tiny(bdm, layout):
    say(f"case coreset tiny layout={layout}")
    inp = synth.tiny_inputs(seed=0, block_seed=1, with_residual=True)
    inp = synth.MoEInputs(inp.shape, *(None if t is None else t.to(DEV) for t in
                                       (inp.x, inp.w_router, inp.router_bias, inp.w_gate,
                                        inp.w_up, inp.w_down, inp.ws_gate, inp.ws_up,
                                        inp.ws_down, inp.residual)))
    for top_p, block in ((0.9, 8), (0.5, 4), (0.2, 8)):
        out = run_gpu(bdm, inp, top_p, block, layout=layout)
        h, r = oracle_routing(inp, top_p, block)
        compare(out, inp, h, r)


@pytest.mark.parametrize("bias_w,top_p", [(0.0, 0.9), (2.0, 0.9), (3.0, 0.6)])
def test_coreset_clover_layer(bdm, bias_w, top_p):
    """The Clover-shaped layer, one 32-token block; a block-wide preference
    (router bias = w x logit scale x N(0,1)) shrinks the kept set; at w = 3
    and top_p 0.6 it is below k, so tokens get fewer than k experts."""
    say(f"case coreset clover bias_w={bias_w} top_p={top_p}")
    inp = synth.moe_inputs(synth.LAYER, seed=0, block_seed=4, device=DEV, with_residual=True)
    if bias_w:
        g = torch.Generator(device="cpu")
        g.manual_seed(17)
        scale = 0.02 * np.sqrt(synth.LAYER.H)
        inp.router_bias = (bias_w * scale * torch.randn(synth.LAYER.E, generator=g)).to(DEV)
    out = run_gpu(bdm, inp, top_p, 32)
    h, r = oracle_routing(inp, top_p, 32)
    if bias_w == 3.0:
        assert r["n_kept"][0] < synth.LAYER.k
        assert np.any(out[1] == -1)
    compare(out, inp, h, r)


def test_coreset_eight_blocks_sampled(bdm):
    """T = 256 as eight 32-token blocks (one coreset workgroup each, the last
    one to finish groups the picks): every block's kept set, the routing of
    every token, the outputs of a seeded sample of 24 tokens."""
    say("case coreset eight blocks")
    s = synth.MoEShape(T=256, H=2048, E=256, I=512, k=8)
    inp = synth.moe_inputs(s, seed=1, block_seed=6, device=DEV, with_residual=True)
    out = run_gpu(bdm, inp, 0.9, 32)
    h, r = oracle_routing(inp, 0.9, 32)
    tokens = np.sort(np.random.default_rng(3).choice(256, 24, replace=False))
    compare(out, inp, h, r, tokens=tokens)


@pytest.mark.parametrize("T", [1024, 2048])
def test_coreset_many_blocks_sampled(bdm, T):
    """32 and 64 blocks in one call (the per-block selection, then the
    grouping as its own kernel): every block's kept set, the routing of every
    token, the outputs of a seeded sample of 24 tokens."""
    say(f"case coreset {T // 32} blocks")
    s = synth.MoEShape(T=T, H=2048, E=256, I=512, k=8)
    inp = synth.moe_inputs(s, seed=1, block_seed=T, device=DEV, with_residual=True)
    out = run_gpu(bdm, inp, 0.9, 32)
    h, r = oracle_routing(inp, 0.9, 32)
    tokens = np.sort(np.random.default_rng(T).choice(T, 24, replace=False))
    compare(out, inp, h, r, tokens=tokens)


def test_coreset_ragged_last_block(bdm):
    say("case coreset ragged last block (T=40, block 16)")
    s = synth.MoEShape(T=40, H=512, E=64, I=128, k=4)
    inp = synth.moe_inputs(s, seed=2, block_seed=2, device=DEV, with_residual=True)
    out = run_gpu(bdm, inp, 0.8, 16, layout=0)
    h, r = oracle_routing(inp, 0.8, 16)
    assert len(r["n_kept"]) == 3
    compare(out, inp, h, r)


def test_coreset_top_p_one_is_plain_routing_bitwise(bdm):
    """top_p = 1 keeps every touched expert: the layer is the plain one, bit
    for bit (renormalised weights)."""
    say("case coreset top_p=1 == plain")
    inp = synth.moe_inputs(synth.LAYER, seed=0, block_seed=5, device=DEV, with_residual=True)
    y1, i1, w1, nk = run_gpu(bdm, inp, 1.0, 32, layout=0)
    i0 = torch.empty((32, 8), dtype=torch.int32, device=DEV)
    w0 = torch.empty((32, 8), dtype=torch.float32, device=DEV)
    y0 = bdm.bdm_moe_block_forward(inp.x, inp.w_router, inp.w_gate, inp.w_up, inp.w_down, 8,
                                   ws_gate=inp.ws_gate, ws_up=inp.ws_up, ws_down=inp.ws_down,
                                   residual=inp.residual, topk_idx=i0, topk_w=w0)
    torch.cuda.synchronize()
    assert nk[0] == len(np.unique(i0.cpu().numpy()))
    assert np.array_equal(i1, i0.cpu().numpy())
    assert np.array_equal(w1.view(np.int32), w0.cpu().numpy().view(np.int32))
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))


def test_coreset_repeatable_and_renorm_off(bdm):
    say("case coreset repeatability + renorm=0")
    inp = synth.moe_inputs(synth.LAYER, seed=3, block_seed=1, device=DEV, with_residual=True)
    a = run_gpu(bdm, inp, 0.9, 32, renorm=False)
    b = run_gpu(bdm, inp, 0.9, 32, renorm=False)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2].view(np.int32), b[2].view(np.int32))
    h, r = oracle_routing(inp, 0.9, 32, renorm=False)
    compare(a, inp, h, r)


@pytest.mark.parametrize("T,block", [(32, 32), (256, 32)])
def test_coreset_gate_up_pair_layout_bitwise(bdm, T, block):
    """The coreset path with gate/up packed as pairs equals the tile layout
    bit for bit (one block; eight blocks on the many-token kernels)."""
    say(f"case coreset gate/up pair layout T={T}")
    shp = synth.MoEShape(T=T, H=2048, E=256, I=512, k=8)
    inp = synth.moe_inputs(shp, seed=4, block_seed=T, device=DEV, with_residual=True)
    a = run_gpu(bdm, inp, 0.9, block, layout=1)
    b = run_gpu(bdm, inp, 0.9, block, layout=2)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2].view(np.int32), b[2].view(np.int32))
    assert np.array_equal(a[3], b[3])

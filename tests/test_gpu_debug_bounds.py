"""The bounds-checked build (libbdmoe_debug.so) on the GPU.

Every index a kernel reads from memory or derives from what it read (slot
table entries, pair rows, picks, re-route candidates and ranks, token ids,
head row groups, partial indices) passes a device-side check in that build;
a failed check sets a bit of a violation word and clamps the index.  Here
the debug build runs the MoE layer (few-token and many-token kernels, the
coreset selector, ragged shapes, NaN rows, a poisoned workspace), the head
with its commit rule, the verify epilogue and the denoise loop: every call
gives the release build's outputs bit for bit and leaves no violation.  An
out-of-vocabulary token id handed to the loop's embedding gather (which
both builds clamp) is reported as such.

Setting BDM_LIBRARY to the debug library runs the whole GPU suite on it;
tests/conftest.py then checks the violation word after every GPU test.
"""
import contextlib

import numpy as np
import pytest
import torch

import synth
from tests.conftest import gpu_available
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CHK_TOKEN_ID = 5          # bit of an out-of-vocabulary id at the embedding gather


@pytest.fixture(scope="module")
def bdm():
    if not gpu_available():
        pytest.skip("no GPU")
    import block_diffusion_moe_amd as b
    b.load()
    return b


@contextlib.contextmanager
def using(path):
    """Route the binding's calls to the library at `path`, then back."""
    from block_diffusion_moe_amd import binding
    prev = binding._lib
    binding._lib = None
    try:
        binding.load(path)
        yield
    finally:
        binding._lib = prev


def both(bdm, fn):
    """fn() under the release and the debug library; the debug run's
    violation word (read after it)."""
    with using(bdm.LIB_PATH):
        rel = fn()
        torch.cuda.synchronize()
    with using(bdm.DEBUG_LIB_PATH):
        bdm.bdm_debug_bounds()                       # start from a clear word
        dbg = fn()
        torch.cuda.synchronize()
        word = bdm.bdm_debug_bounds()
    return rel, dbg, word


def same_bits(a, b):
    for x, y in zip(a, b):
        if x is None:
            assert y is None
            continue
        if isinstance(x, (int, float)):
            assert x == y
            continue
        assert x.shape == y.shape and x.dtype == y.dtype
        xv = x.view(torch.int16) if x.dtype == torch.bfloat16 else (
            x.view(torch.int32) if x.dtype == torch.float32 else x)
        yv = y.view(torch.int16) if y.dtype == torch.bfloat16 else (
            y.view(torch.int32) if y.dtype == torch.float32 else y)
        assert torch.equal(xv, yv)


def _moe_weights(bdm, inp, layout):
    W = (inp.w_gate, inp.w_up, inp.w_down, inp.ws_gate, inp.ws_up, inp.ws_down)
    if layout == 2:
        g, u = bdm.bdm_pack_gate_up(inp.w_gate, inp.w_up)
        sg, su = bdm.bdm_pack_gate_up(inp.ws_gate, inp.ws_up)
        return (g, u, bdm.bdm_pack_weights(inp.w_down), sg, su, bdm.bdm_pack_weights(inp.ws_down))
    return W


MOE_CASES = [
    # (name, shape, layout, coreset top_p, router offset, NaN rows, poisoned workspace)
    ("clover32_pairs", synth.LAYER, 2, None, False, False, False),
    ("clover32_coreset", synth.LAYER, 2, 0.9, False, False, False),
    ("clover32_rowmajor_nan_poison", synth.LAYER, 0, None, False, True, True),
    ("skew256_pairs", synth.MoEShape(T=256, H=2048, E=256, I=512, k=8), 2, None, True, False,
     False),
    ("multi512_pairs", synth.MoEShape(T=512, H=2048, E=256, I=512, k=8), 2, None, False, False,
     True),
    ("coreset_4_blocks", synth.MoEShape(T=128, H=2048, E=256, I=512, k=8), 2, 0.5, False,
     False, False),
    ("ragged_T17", synth.MoEShape(T=17, H=256, E=64, I=96, k=4), 0, None, False, False, False),
    ("ragged_T7_E1024", synth.MoEShape(T=7, H=2048, E=1024, I=64, k=3), 0, None, False, False,
     False),
    ("ragged_T40_k16", synth.MoEShape(T=40, H=512, E=128, I=128, k=16), 0, None, False, False,
     False),
]


@pytest.mark.parametrize("case", MOE_CASES, ids=[c[0] for c in MOE_CASES])
def test_moe_layer_debug_build(bdm, case):
    name, s, layout, top_p, skew, nan_rows, poison = case
    say(f"case debug-build MoE layer {name} T={s.T} H={s.H} E={s.E} I={s.I} k={s.k} "
        f"layout={layout} top_p={top_p}")
    inp = synth.moe_inputs(s, seed=3, block_seed=s.T, device=DEV, with_residual=True,
                           zipf_s=1.1 if skew else None)
    W = _moe_weights(bdm, inp, layout)
    x = inp.x.clone()
    if nan_rows:
        x[[1, s.T // 2]] = float("nan")
    nbytes = bdm.bdm_moe_workspace_bytes(s.T, s.H, s.I, s.E, s.k, True)

    def run():
        ws = bdm.workspace(nbytes, DEV)
        if poison:
            ws.view(torch.uint8).fill_(0xA5)
        y = torch.empty_like(x)
        idx = torch.full((s.T, s.k), -7, dtype=torch.int32, device=DEV)
        w = torch.full((s.T, s.k), -7.0, dtype=torch.float32, device=DEV)
        kw = dict(router_bias=inp.router_bias, ws_gate=W[3], ws_up=W[4], ws_down=W[5],
                  residual=inp.residual, y=y, topk_idx=idx, topk_w=w, ws=ws)
        if top_p is not None:
            nk = torch.zeros(((s.T + 31) // 32,), dtype=torch.int32, device=DEV)
            bdm.bdm_moe_block_forward(x, inp.w_router, W[0], W[1], W[2], s.k,
                                      coreset_top_p=top_p, coreset_block=32, n_kept=nk, **kw)
            return y, idx, w, nk
        bdm.bdm_moe_block_forward(x, inp.w_router, W[0], W[1], W[2], s.k, **kw)
        return y, idx, w, None

    rel, dbg, word = both(bdm, run)
    same_bits(rel, dbg)
    assert word == 0, f"bounds violations {word:#x}"
    say(f"  same bits as the release build, no violation")


@pytest.mark.parametrize("V,T,layout", [(248320, 32, 1), (70001, 33, 0), (4099, 512, 1)])
def test_head_rule_debug_build(bdm, V, T, layout):
    say(f"case debug-build head + rule V={V} T={T} layout={layout}")
    hs = synth.HeadShape(T=T, H=2048 if V > 5000 else 256, V=V, mask_id=V // 3)
    W = synth.head_weights(hs, 7, device=DEV)
    blk = synth.head_block(hs, W, block_seed=4, n_boost=T // 2, committed_rows=3)
    Wl = bdm.bdm_pack_weights(W) if layout else W
    h = blk.h.clone()
    h[[0, T - 1]] = float("nan")

    def run():
        tok = blk.tokens.clone()
        am = torch.empty((T,), dtype=torch.int32, device=DEV)
        cf = torch.empty((T,), dtype=torch.float32, device=DEV)
        nc = torch.empty((1,), dtype=torch.int32, device=DEV)
        bdm.bdm_lm_head_unmask(h, Wl, hs.mask_id, 0.95, True, tok, argmax=am, conf=cf,
                               n_committed=nc, block_tokens=min(T, 32))
        return tok, am, cf, nc

    rel, dbg, word = both(bdm, run)
    same_bits(rel, dbg)
    assert word == 0, f"bounds violations {word:#x}"


def test_verify_debug_build(bdm):
    say("case debug-build verify epilogue")
    hs = synth.HeadShape(T=33, H=2048, V=248320, mask_id=0)
    W = synth.head_weights(hs, 8, device=DEV)
    blk = synth.head_block(hs, W, block_seed=6, boost=12.0, boost_all=True)
    cand = torch.tensor(blk.boosted_tokens[:32], dtype=torch.int32, device=DEV)
    cand[20] = (cand[20] + 1) % hs.V

    def run():
        acc = torch.empty(32, dtype=torch.int32, device=DEV)
        am = torch.empty(33, dtype=torch.int32, device=DEV)
        tok, na = bdm.bdm_lm_head_verify(blk.h, W, cand, "threshold", 0.9, 0.6, accept=acc,
                                         argmax=am)
        return tok, na, acc, am

    rel, dbg, word = both(bdm, run)
    same_bits(rel, dbg)
    assert word == 0, f"bounds violations {word:#x}"


def _tiny_loop(bdm):
    s = synth.MoEShape(T=8, H=64, E=16, I=32, k=2)
    V = 512
    layers = []
    for sd in (11, 12):
        wr, wg, wu, wd, sg, su, sdn, _ = synth.moe_weights(s, sd, DEV)
        layers.append({"w_router": wr, "w_gate": wg, "w_up": wu, "w_down": wd, "ws_gate": sg,
                       "ws_up": su, "ws_down": sdn})
    g = torch.Generator(device=DEV)
    g.manual_seed(901)
    emb = torch.randn((V, s.H), generator=g, device=DEV).to(torch.bfloat16)
    w_head = synth.head_weights(synth.HeadShape(T=8, H=64, V=V, mask_id=0), 5, device=DEV)
    w_head = (w_head.float() * 30.0).to(torch.bfloat16)
    return s, V, layers, emb, w_head


@pytest.mark.parametrize("top_p", [None, 0.9])
def test_denoise_loop_debug_build(bdm, top_p):
    say(f"case debug-build denoise loop top_p={top_p}")
    s, V, layers, emb, w_head = _tiny_loop(bdm)
    tok0 = torch.zeros((s.T,), dtype=torch.int32, device=DEV)
    tok0[2] = 7

    def run():
        cur = tok0.clone()
        steps, commits = bdm.bdm_denoise_block(cur, emb, layers, w_head, s.k, 0, 0.95,
                                               coreset_top_p=top_p)
        return cur, steps, tuple(commits)

    rel, dbg, word = both(bdm, run)
    assert torch.equal(rel[0], dbg[0]) and rel[1] == dbg[1] and rel[2] == dbg[2]
    assert word == 0, f"bounds violations {word:#x}"


def test_out_of_vocabulary_token_reported(bdm):
    """A committed slot holding an id past the vocabulary: both builds read
    the nearest embedding row and finish the loop with the same tokens; the
    debug build reports the id (and nothing else)."""
    say("case debug-build out-of-vocabulary token id at the embedding gather")
    s, V, layers, emb, w_head = _tiny_loop(bdm)
    tok0 = torch.zeros((s.T,), dtype=torch.int32, device=DEV)
    tok0[3] = V + 5

    def run():
        cur = tok0.clone()
        steps, _ = bdm.bdm_denoise_block(cur, emb, layers, w_head, s.k, 0, 0.95)
        return cur, steps

    rel, dbg, word = both(bdm, run)
    assert torch.equal(rel[0], dbg[0]) and rel[1] == dbg[1]
    assert int(dbg[0][3]) == V + 5 and not bool((dbg[0] == 0).any())
    assert word == 1 << CHK_TOKEN_ID, f"violation word {word:#x}"
    with using(bdm.DEBUG_LIB_PATH):
        assert bdm.bdm_debug_bounds() == 0            # read clears it
    say("  reported as an out-of-vocabulary token id; outputs equal the release build's")

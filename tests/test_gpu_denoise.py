"""GPU parity of the denoise loop (bdm_denoise_block) against oracle.denoise.

Tiny model: every step of the GPU loop is checked against the oracle step on
the GPU's own current tokens (teacher forcing; decisions exact away from a
routing near tie, an argmax near tie, a threshold near call or a fallback
near tie), and the whole loop equals those single steps bit for bit.  The
40-layer Clover-shaped stack with the full head: the loop's invariants (at
most T steps, at least one commit per step, committed slots unchanged,
nothing masked at the end), and its first step equals the library's single
calls composed by hand, bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import denoise as oden
from tests.conftest import gpu_available
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def bdm():
    if not gpu_available():
        pytest.skip("no GPU")
    import block_diffusion_moe_amd as b
    b.load()
    return b


def _layers(shape, seeds, device):
    out = []
    for sd in seeds:
        wr, wg, wu, wd, sg, su, sdn, _ = synth.moe_weights(shape, sd, device)
        out.append({"w_router": wr, "w_gate": wg, "w_up": wu, "w_down": wd, "ws_gate": sg,
                    "ws_up": su, "ws_down": sdn})
    return out


def _host_layers(layers):
    return [{"w_router": lw["w_router"].cpu().numpy(),
             **{n: synth.bf16_bits(lw[n]) for n in ("w_gate", "w_up", "w_down", "ws_gate",
                                                     "ws_up", "ws_down")}} for lw in layers]


def _embed(V, H, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(900 + seed)
    return torch.randn((V, H), generator=g, device=device).to(torch.bfloat16)


@pytest.mark.parametrize("threshold,top_p", [(0.95, None), (0.0, None), (0.02, None),
                                             (0.95, 0.9), (0.02, 0.5)])
def test_denoise_tiny_teacher_forced(bdm, threshold, top_p):
    """With top_p, every layer routes through the block coreset selector."""
    say(f"case denoise tiny threshold={threshold} coreset_top_p={top_p}")
    s = synth.MoEShape(T=8, H=64, E=16, I=32, k=2)
    V, mask = 512, 0
    layers = _layers(s, (11, 12, 13), DEV)
    emb = _embed(V, s.H, 1, DEV)
    w_head = synth.head_weights(synth.HeadShape(T=8, H=64, V=V, mask_id=mask), 5, device=DEV)
    w_head = (w_head.float() * 30.0).to(torch.bfloat16)      # sharper rows: some commit
    hl, eb, hb = _host_layers(layers), synth.bf16_bits(emb), synth.bf16_bits(w_head)
    tok0 = torch.full((s.T,), mask, dtype=torch.int32, device=DEV)
    tok0[2] = 7
    cur = tok0.clone()
    history = []
    while (cur == mask).any():
        before = cur.cpu().numpy().astype(np.int64)
        steps, commits = bdm.bdm_denoise_block(cur, emb, layers, w_head, s.k, mask, threshold,
                                               max_steps=1, coreset_top_p=top_p)
        torch.cuda.synchronize()
        after = cur.cpu().numpy().astype(np.int64)
        o = oden.denoise_step(before, eb, hl, hb, s.k, mask, threshold, coreset_top_p=top_p)
        assert steps == 1 and commits[0] >= 1
        excl = o["near_route"] | o["near_tie"] | o["near_threshold"]
        keep = ~excl
        assert np.array_equal(after[before != mask], before[before != mask])
        if not excl.any() and not o["fallback_tie"]:
            assert np.array_equal(after, o["tokens"]), (after, o["tokens"])
            assert commits[0] == o["n_committed"]
        else:
            assert np.array_equal(after[keep], o["tokens"][keep])
        history.append(commits[0])
        assert len(history) <= s.T
    say(f"  commits per step {history}")
    # the whole loop at once gives the same block, bit for bit
    full = tok0.clone()
    steps, commits = bdm.bdm_denoise_block(full, emb, layers, w_head, s.k, mask, threshold,
                                           coreset_top_p=top_p)
    torch.cuda.synchronize()
    assert commits == history and steps == len(history)
    assert torch.equal(full, cur)
    if threshold == 0.0:
        assert history == [s.T - 1]


@pytest.mark.parametrize("T", [24, 20], ids=["3x8", "8+8+4"])
@pytest.mark.parametrize("top_p", [None, 0.9])
def test_denoise_multiblock_tiny(bdm, top_p, T):
    """Blocks of 8 slots in one loop (each its own commit rule; 20 slots: a
    ragged last block of 4): every step against the oracle's (teacher-forced,
    near calls excluded), and the final tokens equal each block denoised
    alone, bit for bit."""
    say(f"case denoise multi-block tiny T={T} coreset_top_p={top_p}")
    s = synth.MoEShape(T=T, H=64, E=16, I=32, k=2)
    V, mask, B = 512, 0, 8
    layers = _layers(s, (21, 22), DEV)
    emb = _embed(V, s.H, 3, DEV)
    w_head = synth.head_weights(synth.HeadShape(T=24, H=64, V=V, mask_id=mask), 6, device=DEV)
    w_head = (w_head.float() * 30.0).to(torch.bfloat16)
    hl, eb, hb = _host_layers(layers), synth.bf16_bits(emb), synth.bf16_bits(w_head)
    tok0 = torch.full((s.T,), mask, dtype=torch.int32, device=DEV)
    tok0[[2, 11, T - 1]] = torch.tensor([7, 8, 9], dtype=torch.int32, device=DEV)
    cur = tok0.clone()
    while (cur == mask).any():
        before = cur.cpu().numpy().astype(np.int64)
        steps, commits = bdm.bdm_denoise_block(cur, emb, layers, w_head, s.k, mask, 0.95,
                                               max_steps=1, coreset_top_p=top_p, block_tokens=B)
        torch.cuda.synchronize()
        after = cur.cpu().numpy().astype(np.int64)
        o = oden.denoise_step(before, eb, hl, hb, s.k, mask, 0.95, coreset_top_p=top_p,
                              block=B)
        excl = o["near_route"] | o["near_tie"] | o["near_threshold"]
        if not excl.any() and not o["fallback_tie"]:
            assert np.array_equal(after, o["tokens"]), (after, o["tokens"])
            assert commits[0] == o["n_committed"]
        else:
            assert np.array_equal(after[~excl], o["tokens"][~excl])
        for b in range(0, s.T, B):              # every block still masked commits
            if (before[b:b + B] == mask).any():
                assert (after[b:b + B] != before[b:b + B]).any()
    full = tok0.clone()
    bdm.bdm_denoise_block(full, emb, layers, w_head, s.k, mask, 0.95, coreset_top_p=top_p,
                          block_tokens=B)
    for b in range(0, s.T, B):
        one = tok0[b:b + B].clone()
        bdm.bdm_denoise_block(one, emb, layers, w_head, s.k, mask, 0.95, coreset_top_p=top_p)
        torch.cuda.synchronize()
        assert torch.equal(one, full[b:b + B]), b


@pytest.mark.parametrize("top_p", [None, 0.9])
def test_denoise_layouts_agree(bdm, top_p):
    """The whole tiny loop with row-major, tile-packed and pair-packed
    (gate/up through bdm_pack_gate_up) weights gives the same tokens."""
    say(f"case denoise layouts coreset_top_p={top_p}")
    s = synth.MoEShape(T=16, H=64, E=16, I=32, k=2)
    V, mask = 512, 0
    layers = _layers(s, (31, 32), DEV)
    emb = _embed(V, s.H, 4, DEV)
    w_head = synth.head_weights(synth.HeadShape(T=16, H=64, V=V, mask_id=mask), 7, device=DEV)
    w_head = (w_head.float() * 30.0).to(torch.bfloat16)
    pk = bdm.bdm_pack_weights
    tiles = [{**lw, **{n: pk(lw[n]) for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up",
                                               "ws_down")}} for lw in layers]
    pairs = []
    for lw in layers:
        g, u = bdm.bdm_pack_gate_up(lw["w_gate"], lw["w_up"])
        sg, su = bdm.bdm_pack_gate_up(lw["ws_gate"], lw["ws_up"])
        pairs.append({**lw, "w_gate": g, "w_up": u, "w_down": pk(lw["w_down"]), "ws_gate": sg,
                      "ws_up": su, "ws_down": pk(lw["ws_down"])})
    tok0 = torch.full((s.T,), mask, dtype=torch.int32, device=DEV)
    tok0[5] = 9
    outs = []
    for lay, wh in ((layers, w_head), (tiles, pk(w_head)), (pairs, pk(w_head))):
        t = tok0.clone()
        steps, commits = bdm.bdm_denoise_block(t, emb, lay, wh, s.k, mask, 0.95,
                                               coreset_top_p=top_p)
        torch.cuda.synchronize()
        outs.append((t.cpu(), steps, commits))
    for o in outs[1:]:
        assert torch.equal(o[0], outs[0][0]) and o[1:] == outs[0][1:]


@pytest.mark.parametrize("top_p", [None, 0.9])
def test_denoise_clover_stack_invariants_and_first_step(bdm, top_p):
    """40 Clover-shaped layers, the 248,320-row head, packed weights; plain
    routing, and the coreset selector at the shipped top_p 0.9."""
    s = synth.LAYER
    HS = synth.HEAD
    say(f"case denoise 40-layer stack + head coreset_top_p={top_p}")
    layers = _layers(s, range(100, 100 + synth.STACK_LAYERS), DEV)
    pk = bdm.bdm_pack_weights
    players = [{**{n: lw[n] for n in ("w_router",)},
                **{n: pk(lw[n]) for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up",
                                          "ws_down")}} for lw in layers]
    del layers
    torch.cuda.empty_cache()
    emb = _embed(HS.V, s.H, 2, DEV)
    w_head = pk(synth.head_weights(HS, 0, device=DEV))
    torch.cuda.synchronize()
    say("  weights ready")
    tok0 = torch.full((s.T,), HS.mask_id, dtype=torch.int32, device=DEV)
    tok0[[0, 9, 20]] = torch.tensor([11, 12, 13], dtype=torch.int32, device=DEV)
    # first step by hand from the single calls
    x = emb[tok0.long()].contiguous()
    xn = torch.empty_like(x)
    ws = bdm.workspace(bdm.bdm_moe_workspace_bytes(s.T, s.H, s.I, s.E, s.k, True), DEV)
    for lw in players:
        bdm.bdm_rmsnorm(x, xn, eps=1e-6)
        kw = {} if top_p is None else {"coreset_top_p": top_p, "coreset_block": s.T}
        bdm.bdm_moe_block_forward(xn, lw["w_router"], lw["w_gate"], lw["w_up"], lw["w_down"],
                                  s.k, ws_gate=lw["ws_gate"], ws_up=lw["ws_up"],
                                  ws_down=lw["ws_down"], residual=x, y=x, ws=ws, **kw)
    bdm.bdm_rmsnorm(x, xn, eps=1e-6)
    ref = tok0.clone()
    nc = torch.zeros(1, dtype=torch.int32, device=DEV)
    bdm.bdm_lm_head_unmask(xn, w_head, HS.mask_id, 0.95, True, ref, n_committed=nc)
    one = tok0.clone()
    steps, commits = bdm.bdm_denoise_block(one, emb, players, w_head, s.k, HS.mask_id, 0.95,
                                           max_steps=1, coreset_top_p=top_p)
    torch.cuda.synchronize()
    assert steps == 1 and commits == [int(nc.item())]
    assert torch.equal(one, ref)
    # the whole loop (layers marshalled once: the same results as the list)
    tok = tok0.clone()
    steps, commits = bdm.bdm_denoise_block(tok, emb, bdm.MoeStack(players), w_head, s.k,
                                           HS.mask_id, 0.95, coreset_top_p=top_p)
    torch.cuda.synchronize()
    say(f"  {steps} steps, commits {commits}")
    masked0 = int((tok0 == HS.mask_id).sum())
    assert 1 <= steps <= masked0 and all(c >= 1 for c in commits) and sum(commits) == masked0
    assert not (tok == HS.mask_id).any()
    done = tok0 != HS.mask_id
    assert torch.equal(tok[done], tok0[done])
    assert int(tok.min()) >= 0 and int(tok.max()) < HS.V
    del players, w_head, emb
    torch.cuda.empty_cache()


def test_denoise_clover_stack_two_blocks_gate_up_pairs(bdm):
    """40 Clover-shaped layers with gate/up packed as pairs, two 32-slot
    blocks in one call: the first step equals the single calls composed (the
    head's rule per block), the loop ends with both blocks unmasked, and
    each block's tokens equal that block denoised alone."""
    s = synth.LAYER
    HS = synth.HEAD
    say("case denoise 40-layer stack, two blocks, gate/up pairs")
    layers = _layers(s, range(200, 200 + synth.STACK_LAYERS), DEV)
    pk = bdm.bdm_pack_weights
    players = []
    for lw in layers:
        g, u = bdm.bdm_pack_gate_up(lw["w_gate"], lw["w_up"])
        sg, su = bdm.bdm_pack_gate_up(lw["ws_gate"], lw["ws_up"])
        players.append({"w_router": lw["w_router"], "w_gate": g, "w_up": u,
                        "w_down": pk(lw["w_down"]), "ws_gate": sg, "ws_up": su,
                        "ws_down": pk(lw["ws_down"])})
    del layers
    torch.cuda.empty_cache()
    stack = bdm.MoeStack(players)
    emb = _embed(HS.V, s.H, 5, DEV)
    w_head = pk(synth.head_weights(HS, 1, device=DEV))
    torch.cuda.synchronize()
    say("  weights ready")
    T = 2 * s.T
    tok0 = torch.full((T,), HS.mask_id, dtype=torch.int32, device=DEV)
    tok0[[3, 17, 40, 41, 60]] = torch.tensor([21, 22, 23, 24, 25], dtype=torch.int32, device=DEV)
    # first step by hand
    x = emb[tok0.long()].contiguous()
    xn = torch.empty_like(x)
    ws = bdm.workspace(bdm.bdm_moe_workspace_bytes(T, s.H, s.I, s.E, s.k, True), DEV)
    for lw in players:
        bdm.bdm_rmsnorm(x, xn, eps=1e-6)
        bdm.bdm_moe_block_forward(xn, lw["w_router"], lw["w_gate"], lw["w_up"], lw["w_down"],
                                  s.k, ws_gate=lw["ws_gate"], ws_up=lw["ws_up"],
                                  ws_down=lw["ws_down"], residual=x, y=x, ws=ws)
    bdm.bdm_rmsnorm(x, xn, eps=1e-6)
    ref = tok0.clone()
    nc = torch.zeros(1, dtype=torch.int32, device=DEV)
    bdm.bdm_lm_head_unmask(xn, w_head, HS.mask_id, 0.95, True, ref, n_committed=nc,
                           block_tokens=s.T)
    one = tok0.clone()
    steps, commits = bdm.bdm_denoise_block(one, emb, stack, w_head, s.k, HS.mask_id, 0.95,
                                           max_steps=1, block_tokens=s.T)
    torch.cuda.synchronize()
    assert steps == 1 and commits == [int(nc.item())] and commits[0] >= 2
    assert torch.equal(one, ref)
    # the whole loop, and each block alone
    tok = tok0.clone()
    steps, commits = bdm.bdm_denoise_block(tok, emb, stack, w_head, s.k, HS.mask_id, 0.95,
                                           block_tokens=s.T)
    torch.cuda.synchronize()
    say(f"  {steps} steps, commits {commits}")
    assert steps <= s.T and not (tok == HS.mask_id).any()
    done = tok0 != HS.mask_id
    assert torch.equal(tok[done], tok0[done])
    for b in range(2):
        alone = tok0[b * s.T:(b + 1) * s.T].clone()
        bdm.bdm_denoise_block(alone, emb, stack, w_head, s.k, HS.mask_id, 0.95)
        torch.cuda.synchronize()
        assert torch.equal(alone, tok[b * s.T:(b + 1) * s.T]), b
    del players, stack, w_head, emb
    torch.cuda.empty_cache()


def test_denoise_degenerate_calls(bdm):
    """max_steps = 0 does nothing; a block with nothing masked takes one
    step that commits nothing and leaves it as it was; with several blocks,
    a block that starts unmasked is never written while the others are
    denoised, and they end as when run alone."""
    say("case denoise degenerate calls")
    s = synth.MoEShape(T=16, H=64, E=16, I=32, k=2)
    V, mask, B = 512, 0, 8
    layers = _layers(s, (41, 42), DEV)
    stack = bdm.MoeStack(layers)
    emb = _embed(V, s.H, 7, DEV)
    w_head = synth.head_weights(synth.HeadShape(T=16, H=64, V=V, mask_id=mask), 8, device=DEV)
    tok = torch.full((s.T,), mask, dtype=torch.int32, device=DEV)
    steps, commits = bdm.bdm_denoise_block(tok, emb, stack, w_head, s.k, mask, 0.95,
                                           max_steps=0)
    torch.cuda.synchronize()
    assert (steps, commits) == (0, []) and bool((tok == mask).all())
    full = torch.arange(1, s.T + 1, dtype=torch.int32, device=DEV)
    tok = full.clone()
    steps, commits = bdm.bdm_denoise_block(tok, emb, stack, w_head, s.k, mask, 0.95)
    torch.cuda.synchronize()
    assert (steps, commits) == (1, [0]) and torch.equal(tok, full)
    # block 0 unmasked from the start, block 1 all masked
    tok0 = torch.cat([full[:B], torch.full((B,), mask, dtype=torch.int32, device=DEV)])
    tok = tok0.clone()
    steps, commits = bdm.bdm_denoise_block(tok, emb, stack, w_head, s.k, mask, 0.95,
                                           block_tokens=B)
    alone = tok0[B:].clone()
    steps1, commits1 = bdm.bdm_denoise_block(alone, emb, stack, w_head, s.k, mask, 0.95)
    torch.cuda.synchronize()
    assert torch.equal(tok[:B], full[:B]) and torch.equal(tok[B:], alone)
    assert (steps, commits) == (steps1, commits1) and sum(commits) == B
    assert not (tok == mask).any()

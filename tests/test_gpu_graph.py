"""The denoise step captured into a HIP graph (through torch.cuda.graph) and
replayed: every replay, with eager work and synchronisations between the
replays, gives the eager result bit for bit.  The step is the one bench.py
times (RMSNorm, the Clover-shaped MoE layer, the head statistics and the
unmask rule); none of its calls allocates, synchronises or records a memset.
"""
import pytest
import torch

import synth
from tests.conftest import gpu_available
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


@pytest.fixture(scope="module")
def bdm():
    if not gpu_available():
        pytest.skip("no GPU")
    import block_diffusion_moe_amd as b
    b.load()
    return b


def test_step_graph_replays_equal_eager(bdm):
    L, HS = synth.LAYER, synth.HEAD
    say("case denoise step graph replay")
    inp = synth.moe_inputs(L, seed=3, block_seed=4, device=DEV, with_residual=False)
    pk = bdm.bdm_pack_weights
    W = [pk(t) for t in (inp.w_gate, inp.w_up, inp.w_down, inp.ws_gate, inp.ws_up, inp.ws_down)]
    wh = synth.head_weights(HS, 3, device=DEV)
    blk = synth.head_block(HS, wh, block_seed=4, n_boost=10)
    w_head = pk(wh)
    del wh
    tok0 = blk.tokens.clone()
    T, H = L.T, L.H
    ws = bdm.workspace(bdm.bdm_moe_workspace_bytes(T, H, L.I, L.E, L.k, True), DEV)
    P = bdm.bdm_head_stat_parts()
    xn = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    y = torch.empty_like(xn)
    sm = torch.empty((T, P), dtype=torch.float32, device=DEV)
    ss = torch.empty_like(sm)
    sa = torch.empty((T, P), dtype=torch.int32, device=DEV)
    tok = tok0.clone()
    nc = torch.empty((1,), dtype=torch.int32, device=DEV)

    def step():
        bdm.bdm_rmsnorm(inp.x, xn, eps=1e-6)
        bdm.bdm_moe_block_forward(xn, inp.w_router, W[0], W[1], W[2], L.k, ws_gate=W[3],
                                  ws_up=W[4], ws_down=W[5], residual=inp.x, y=y, ws=ws)
        bdm.bdm_lm_head_stats(y, w_head, HS.mask_id, sm, ss, sa)
        bdm.bdm_unmask_from_stats(sm, ss, sa, HS.mask_id, 0.95, True, tok, n_committed=nc)

    step()                                      # eager (also the one-time set-up)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y, sm, ss, sa, tok, nc)]
    g = torch.cuda.CUDAGraph()
    tok.copy_(tok0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        tok.copy_(tok0)                         # eager work between replays
        y.zero_()
        sm.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((y, sm, ss, sa, tok, nc), ref):
            assert torch.equal(_bits(a), _bits(b)), rep
        say(f"  replay {rep} == eager")
    del g
    torch.cuda.empty_cache()


def test_multiblock_step_graph_replays_equal_eager(bdm):
    """The same for 16 blocks (512 slots) in one call: the many-token expert
    kernels, the head over 512 rows in one launch and the rule per block."""
    L, HS = synth.LAYER, synth.HEAD
    say("case multi-block step graph replay")
    T = 16 * L.T
    shp = synth.MoEShape(T=T, H=L.H, E=L.E, I=L.I, k=L.k)
    inp = synth.moe_inputs(shp, seed=5, block_seed=6, device=DEV, with_residual=False)
    pk = bdm.bdm_pack_weights
    W = [pk(t) for t in (inp.w_gate, inp.w_up, inp.w_down, inp.ws_gate, inp.ws_up, inp.ws_down)]
    w_head = pk(synth.head_weights(HS, 4, device=DEV))
    g_tok = torch.Generator().manual_seed(11)
    tok0 = torch.full((T,), HS.mask_id, dtype=torch.int32)
    keep = torch.rand((T,), generator=g_tok) < 0.5
    tok0[keep] = torch.randint(0, HS.mask_id, (int(keep.sum()),), generator=g_tok,
                               dtype=torch.int32)
    tok0 = tok0.to(DEV)
    H = L.H
    ws = bdm.workspace(bdm.bdm_moe_workspace_bytes(T, H, L.I, L.E, L.k, True), DEV)
    P = bdm.bdm_head_stat_parts()
    xn = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    y = torch.empty_like(xn)
    sm = torch.empty((T, P), dtype=torch.float32, device=DEV)
    ss = torch.empty_like(sm)
    sa = torch.empty((T, P), dtype=torch.int32, device=DEV)
    tok = tok0.clone()
    nc = torch.empty((1,), dtype=torch.int32, device=DEV)

    def step():
        bdm.bdm_rmsnorm(inp.x, xn, eps=1e-6)
        bdm.bdm_moe_block_forward(xn, inp.w_router, W[0], W[1], W[2], L.k, ws_gate=W[3],
                                  ws_up=W[4], ws_down=W[5], residual=inp.x, y=y, ws=ws)
        bdm.bdm_lm_head_stats(y, w_head, HS.mask_id, sm, ss, sa)
        bdm.bdm_unmask_from_stats(sm, ss, sa, HS.mask_id, 0.95, True, tok, n_committed=nc,
                                  block_tokens=L.T)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y, sm, ss, sa, tok, nc)]
    assert int(nc.item()) >= 16                # every block commits at least one slot
    g = torch.cuda.CUDAGraph()
    tok.copy_(tok0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        tok.copy_(tok0)
        y.zero_()
        sm.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((y, sm, ss, sa, tok, nc), ref):
            assert torch.equal(_bits(a), _bits(b)), rep
        say(f"  replay {rep} == eager")
    del g
    torch.cuda.empty_cache()

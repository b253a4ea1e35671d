"""The allocation-free MoE entry point (bdm_moe_block_forward_noalloc) against
bdm_moe_block_forward with a workspace: the same kernels, so the same bits,
on two calls in a row, the second with a smaller input (the static buffer
keeps the first call's contents)."""
import pytest
import torch

import synth
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


def _both(bdm, inp, W, k, residual):
    s = inp.shape
    outs = []
    for fn in (bdm.bdm_moe_block_forward, bdm.bdm_moe_block_forward_noalloc):
        y = torch.empty((s.T, s.H), dtype=torch.bfloat16, device=DEV)
        yn = torch.empty_like(y)
        idx = torch.full((s.T, k), -1, dtype=torch.int32, device=DEV)
        w = torch.full((s.T, k), float("nan"), dtype=torch.float32, device=DEV)
        fn(inp.x, inp.w_router, W[0], W[1], W[2], k, router_bias=inp.router_bias,
           ws_gate=W[3], ws_up=W[4], ws_down=W[5], residual=residual, y=y, y_norm=yn,
           topk_idx=idx, topk_w=w)
        torch.cuda.synchronize()
        outs.append((y, yn, idx, w))
    (y0, n0, i0, w0), (y1, n1, i1, w1) = outs
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(n0.view(torch.int16), n1.view(torch.int16))
    assert torch.equal(i0, i1) and torch.equal(w0.view(torch.int32), w1.view(torch.int32))


def test_noalloc_equals_workspace_call_twice(bdm):
    """The load-skew batch (256 tokens, many-token kernels), then one 32-token
    block (few-token kernels) with gate/up pairs: each equal bit for bit to
    the call with a workspace."""
    say("case no-alloc entry point: T=256 skew, then T=32")
    big = synth.skew_inputs(seed=3, block_seed=2, device=DEV)
    pk = bdm.bdm_pack_weights
    g, u = bdm.bdm_pack_gate_up(big.w_gate, big.w_up)
    sg, su = bdm.bdm_pack_gate_up(big.ws_gate, big.ws_up)
    W = (g, u, pk(big.w_down), sg, su, pk(big.ws_down))
    _both(bdm, big, W, 8, None)
    # the same layer weights, a smaller block (no router offset)
    x, res, _ = synth.moe_tokens(synth.LAYER, block_seed=4, device=DEV, with_residual=True)
    small = synth.MoEInputs(synth.LAYER, x, big.w_router, None, big.w_gate, big.w_up,
                            big.w_down, big.ws_gate, big.ws_up, big.ws_down, res)
    _both(bdm, small, W, 8, res)
    say("  both calls equal the workspace calls bit for bit")


def test_noalloc_rejects_oversized(bdm):
    """A size whose workspace exceeds the static buffer returns
    BDM_ERR_WORKSPACE_TOO_SMALL and writes nothing."""
    say("case no-alloc entry point: oversized call rejected")
    s = synth.MoEShape(T=2048, H=2048, E=256, I=512, k=8)
    x = torch.zeros((s.T, s.H), dtype=torch.bfloat16, device=DEV)
    wr = torch.zeros((s.E, s.H), dtype=torch.float32, device=DEV)
    wg = torch.zeros((s.E, s.I, s.H), dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros((s.E, s.H, s.I), dtype=torch.bfloat16, device=DEV)
    y = torch.full((s.T, s.H), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(bdm.BdmError) as e:
        bdm.bdm_moe_block_forward_noalloc(x, wr, wg, wg, wd, s.k, y=y)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())

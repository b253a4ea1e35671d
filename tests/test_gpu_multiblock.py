"""GPU parity of multi-block batching: many 32-slot blocks through one MoE
layer call, sharing one pass over the touched experts' weights.

A routed expert of a many-block batch, and always the shared expert, serves
more tokens than one work item takes (64), so its group is split into
several work items; these tests cover that path.  Bar: every token's
routing against the oracle router (top-k ids exact away from a near tie,
weights within 2e-5 relative), the outputs of a seeded token sample within
the bf16 contract tolerance of the oracle, and -- since every token's
result is computed on its own -- each block's rows bit-identical to the
same block run as a call of its own.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import moe as omoe
from tests.conftest import gpu_available
from tests.gpu_common import compare_moe, oracle_moe, run_moe, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LAYOUTS = pytest.mark.parametrize("layout", [0, 1], ids=["rowmajor", "packed"])


@pytest.fixture(scope="module")
def bdm():
    if not gpu_available():
        pytest.skip("no GPU")
    import block_diffusion_moe_amd as b
    b.load()
    return b


def _clover(T, block_seed, zipf=None):
    s = synth.MoEShape(T=T, H=2048, E=256, I=512, k=8)
    return synth.moe_inputs(s, seed=0, block_seed=block_seed, device=DEV, with_residual=True,
                            zipf_s=zipf)


def _check_routing(inp, idx, w):
    h = synth.moe_host(inp, lazy=True)
    oi, ow, _, near = omoe.route(h["x"], h["w_router"], inp.shape.k, h["router_bias"])
    keep = ~near
    gi, gw = idx.cpu().numpy(), w.cpu().numpy()
    say(f"  routing compared on {int(keep.sum())}/{len(keep)} tokens")
    assert np.array_equal(gi[keep], oi[keep])
    np.testing.assert_allclose(gw[keep], ow[keep], rtol=2e-5, atol=1e-6)
    counts = np.bincount(gi.reshape(-1), minlength=inp.shape.E)
    return counts


def _block(inp, b, B=32):
    sl = slice(b * B, (b + 1) * B)
    return dataclasses.replace(inp, shape=dataclasses.replace(inp.shape, T=B),
                               x=inp.x[sl].contiguous(), residual=inp.residual[sl].contiguous())


@LAYOUTS
@pytest.mark.parametrize("T", [512, 1024, 2048])
def test_multiblock_clover_sampled(bdm, T, layout):
    """T/32 Clover-shaped blocks in one call: all routing, 24 sampled outputs."""
    say(f"case multiblock clover T={T} layout={layout}")
    inp = _clover(T, block_seed=40 + T)
    y, idx, w = run_moe(bdm, inp, layout=layout)
    counts = _check_routing(inp, idx, w)
    say(f"  touched {int((counts > 0).sum())} experts, busiest {int(counts.max())} tokens")
    if T >= 2048:
        assert counts.max() > 64            # routed groups split over several work items
    tokens = np.sort(np.random.default_rng(T).choice(T, 24, replace=False))
    o = oracle_moe(inp, tokens=tokens, lazy=True)
    compare_moe(y, idx, w, o, tokens=tokens)


@pytest.mark.parametrize("T,zipf", [(1024, None), (2048, None), (1024, 1.1)],
                         ids=["T1024", "T2048", "T1024_skew"])
def test_multiblock_rows_equal_single_block_calls(bdm, T, zipf):
    """Each sampled block's rows of the batched call equal the block run on
    its own, bit for bit (outputs, ids, weights); the skewed router sends
    hundreds of tokens to its hottest experts."""
    say(f"case multiblock block independence T={T} zipf={zipf}")
    inp = _clover(T, block_seed=90 + T, zipf=zipf)
    y, idx, w = run_moe(bdm, inp, layout=1)
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=256)
    say(f"  busiest expert {int(counts.max())} tokens")
    nb = T // 32
    for b in sorted({0, 5, nb // 2, nb - 1}):
        sub = _block(inp, b)
        yb, ib, wb = run_moe(bdm, sub, layout=1)
        sl = slice(b * 32, (b + 1) * 32)
        assert torch.equal(yb.view(torch.int16), y[sl].view(torch.int16)), b
        assert torch.equal(ib, idx[sl]) and torch.equal(wb.view(torch.int32),
                                                         w[sl].view(torch.int32)), b


@LAYOUTS
@pytest.mark.parametrize("shape", [(65, 256, 16, 64, 2), (200, 256, 4, 64, 2),
                                   (130, 512, 2, 32, 1), (300, 128, 8, 96, 3),
                                   (450, 512, 8, 96, 3), (400, 256, 16, 32, 2),
                                   (400, 1024, 6, 128, 2), (390, 2048, 4, 64, 1),
                                   (400, 256, 512, 1024, 4), (512, 512, 1024, 64, 8)],
                         ids=lambda s: "T%d_H%d_E%d_I%d_k%d" % s)
def test_multiblock_small_full(bdm, shape, layout):
    """Small shapes whose groups exceed one work item (shared 65 = 64 + 1;
    routed groups of ~100-130 tokens), on both the few-token kernels and
    (T >= 256, H of 256, 512, 1024 or 2048) the many-token ones, with partial
    column runs (I = 96) and guarded k-steps: every output against the
    oracle."""
    T, H, E, I, k = shape
    say(f"case multiblock small T={T} H={H} E={E} I={I} k={k} layout={layout}")
    s = synth.MoEShape(T=T, H=H, E=E, I=I, k=k)
    inp = synth.moe_inputs(s, seed=T, block_seed=E, device=DEV, with_residual=True)
    y, idx, w = run_moe(bdm, inp, layout=layout)
    o = oracle_moe(inp)
    compare_moe(y, idx, w, o)

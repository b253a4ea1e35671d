"""Rows with no finite logit (a NaN hidden row) through the head and the rule.

A hidden row of NaNs makes every logit of that row NaN; its online-softmax
statistics then hold no finite maximum.  Such a row has no prediction: its
argmax is -1 and its conf 0, the commit rule never fills it (neither by the
threshold nor as the progress fallback), it stays masked and n_committed
does not count it.  Every other row is decided exactly as the oracle decides
the block without the NaN rows (page "Clover-35B-A3B: how a diffusion model
gets to 680 tokens a second, read from its files", section "How it writes",
steps 2-3: only a slot's prediction can fill it).  The kernels' indexing does
not depend on the values, so these inputs stay inside every buffer.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import head as ohead
from tests.conftest import gpu_available
from tests.gpu_common import compare_head, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def bdm():
    if not gpu_available():
        pytest.skip("no GPU")
    import block_diffusion_moe_amd as b
    b.load()
    return b


def _run(bdm, h, W, tokens, mask_id, layout, block_tokens=0):
    T = h.shape[0]
    Wl = bdm.bdm_pack_weights(W) if layout else W
    tok = tokens.clone()
    am = torch.full((T,), -7, dtype=torch.int32, device=DEV)
    cf = torch.full((T,), -7.0, dtype=torch.float32, device=DEV)
    nc = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    bdm.bdm_lm_head_unmask(h, Wl, mask_id, 0.95, True, tok, argmax=am, conf=cf, n_committed=nc,
                           block_tokens=block_tokens)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), am.cpu().numpy(), cf.cpu().numpy(), int(nc.item())


@pytest.mark.parametrize("layout", [0, 1], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("V,T,boost", [(512, 8, 12.0), (70001, 32, 20.0), (70001, 32, 2.0)])
def test_nan_rows_never_commit(bdm, V, T, boost, layout):
    """Two NaN rows among masked ones (boost 2: no row reaches the threshold,
    so the fallback decides among the finite rows only)."""
    say(f"case NaN rows V={V} T={T} boost={boost} layout={layout}")
    s = synth.HeadShape(T=T, H=256 if V > 512 else 64, V=V, mask_id=V // 5)
    W = synth.head_weights(s, 11, device=DEV)
    blk = synth.head_block(s, W, block_seed=3, n_boost=T // 2, boost=boost, committed_rows=2)
    bad = [r for r in range(T) if int(blk.tokens[r]) == s.mask_id][:2]
    h = blk.h.clone()
    h[bad] = float("nan")
    tok, am, cf, nc = _run(bdm, h, W, blk.tokens, s.mask_id, layout)
    good = np.array([r for r in range(T) if r not in bad])
    assert np.all(am[bad] == -1) and np.all(cf[bad] == 0.0)
    assert np.all(tok[bad] == s.mask_id)
    o = ohead.head_unmask(synth.bf16_bits(blk.h)[good], synth.bf16_bits(W),
                          blk.tokens.cpu().numpy()[good], s.mask_id, 0.95)
    o["mask_id"] = s.mask_id
    sub = tuple(torch.as_tensor(v) for v in (tok[good], am[good], cf[good], np.array([nc])))
    compare_head(sub, o, blk.tokens.cpu().numpy()[good])
    say(f"  NaN rows {bad} stay masked; {nc} commits among the finite rows, as the oracle")


@pytest.mark.parametrize("layout", [0, 1], ids=["rowmajor", "packed"])
def test_all_masked_rows_nan(bdm, layout):
    """Every masked row NaN: nothing commits, tokens unchanged; with two blocks
    the block with finite rows still commits on its own."""
    say(f"case every masked row NaN layout={layout}")
    s = synth.HeadShape(T=16, H=64, V=512, mask_id=0)
    W = synth.head_weights(s, 12, device=DEV)
    blk = synth.head_block(s, W, block_seed=4, n_boost=8, committed_rows=3)
    h = blk.h.clone()
    masked = (blk.tokens == s.mask_id).cpu().numpy()
    h[torch.as_tensor(masked, device=DEV)] = float("nan")
    tok, am, cf, nc = _run(bdm, h, W, blk.tokens, s.mask_id, layout)
    assert nc == 0 and np.array_equal(tok, blk.tokens.cpu().numpy())
    assert np.all(am[masked] == -1) and np.all(cf[masked] == 0.0)
    # block 0 (rows 0..7) NaN, block 1 finite: block 1 alone decides as the oracle
    h2 = blk.h.clone()
    h2[:8] = float("nan")
    tok2, am2, _, nc2 = _run(bdm, h2, W, blk.tokens, s.mask_id, layout, block_tokens=8)
    o = ohead.head_unmask(synth.bf16_bits(blk.h)[8:], synth.bf16_bits(W),
                          blk.tokens.cpu().numpy()[8:], s.mask_id, 0.95)
    assert np.array_equal(tok2[:8], blk.tokens.cpu().numpy()[:8]) and np.all(am2[:8] == -1)
    assert np.array_equal(tok2[8:], o["tokens"]) and nc2 == o["n_committed"] >= 1


def test_unmask_from_stats_empty_row(bdm):
    """Phase 2 given triples with no element (max -inf, sum 0, id INT32_MAX)
    for one row: that row has no prediction and is not committed."""
    say("case unmask from stats, a row with empty triples")
    T, P = 4, 8
    m = torch.full((T, P), -1.0, dtype=torch.float32, device=DEV)
    s_ = torch.full((T, P), 2.0, dtype=torch.float32, device=DEV)
    a = torch.arange(T * P, dtype=torch.int32, device=DEV).view(T, P) + 10
    m[1] = float("-inf")
    s_[1] = 0.0
    a[1] = 2**31 - 1
    tok = torch.full((T,), 5, dtype=torch.int32, device=DEV)
    am = torch.empty(T, dtype=torch.int32, device=DEV)
    cf = torch.empty(T, dtype=torch.float32, device=DEV)
    nc = torch.empty(1, dtype=torch.int32, device=DEV)
    bdm.bdm_unmask_from_stats(m, s_, a, 5, 0.95, True, tok, argmax=am, conf=cf, n_committed=nc)
    torch.cuda.synchronize()
    # finite rows: max -1 in all 8 parts, sum 8 * 2 = 16 -> conf 1/16, the
    # lowest id of the equal maxima; none reaches 0.95, the fallback takes
    # row 0 (equal confidences: lowest position)
    assert int(am[1]) == -1 and float(cf[1]) == 0.0
    assert [int(v) for v in am[[0, 2, 3]]] == [10, 26, 34]
    assert torch.all(cf[[0, 2, 3]] == 1.0 / 16)
    assert int(nc.item()) == 1 and tok.tolist() == [10, 5, 5, 5]


def test_verify_nan_row_rejected(bdm):
    """Verify epilogue: a NaN causal row has no prediction (argmax -1) and
    rejects its candidate, which ends the accepted prefix there."""
    say("case verify with a NaN row")
    s = synth.HeadShape(T=9, H=256, V=4096, mask_id=0)
    W = synth.head_weights(s, 13, device=DEV)
    blk = synth.head_block(s, W, block_seed=5, boost=12.0, boost_all=True)
    cand = torch.tensor(blk.boosted_tokens[:8], dtype=torch.int32, device=DEV)
    h = blk.h.clone()
    h[3] = float("nan")
    acc = torch.empty(8, dtype=torch.int32, device=DEV)
    am = torch.empty(9, dtype=torch.int32, device=DEV)
    for rule in ("exact", "threshold"):
        tok, na = bdm.bdm_lm_head_verify(h, W, cand, rule, 0.9, 0.6, accept=acc, argmax=am)
        torch.cuda.synchronize()
        assert int(am[3]) == -1 and int(acc[3]) == 0
        assert int(na.item()) <= 3
        r = int(na.item())
        assert tok[:r].tolist() == cand[:r].tolist() and int(tok[r]) == int(am[r])


@pytest.mark.parametrize("T", [8, 32, 256])
def test_moe_layer_nan_rows_stay_in_bounds(bdm, T):
    """NaN rows in the MoE layer's input (the header: undefined values, never
    an out-of-bounds access): their expert ids stay in [0, E) and every other
    row is bit for bit what the call without the NaN rows gives (tokens are
    independent through the layer); few-token kernels at 8 and 32 tokens,
    many-token kernels at 256."""
    say(f"case MoE layer with NaN rows T={T}")
    s = synth.MoEShape(T=T, H=2048, E=256, I=512, k=8)
    inp = synth.moe_inputs(s, seed=21, block_seed=T, device=DEV, with_residual=True)
    outs = []
    for poison in (False, True):
        x = inp.x.clone()
        if poison:
            x[[1, T // 2]] = float("nan")
        y = torch.empty_like(x)
        idx = torch.full((T, s.k), -7, dtype=torch.int32, device=DEV)
        w = torch.empty((T, s.k), dtype=torch.float32, device=DEV)
        bdm.bdm_moe_block_forward(x, inp.w_router, inp.w_gate, inp.w_up, inp.w_down, s.k,
                                  ws_gate=inp.ws_gate, ws_up=inp.ws_up, ws_down=inp.ws_down,
                                  residual=inp.residual, y=y, topk_idx=idx, topk_w=w)
        torch.cuda.synchronize()
        outs.append((y, idx, w))
    (y0, i0, w0), (y1, i1, w1) = outs
    bad = torch.zeros(T, dtype=torch.bool, device=DEV)
    bad[[1, T // 2]] = True
    assert int(i1.min()) >= 0 and int(i1.max()) < s.E
    assert torch.equal(y1[~bad].view(torch.int16), y0[~bad].view(torch.int16))
    assert torch.equal(i1[~bad], i0[~bad])
    assert torch.equal(w1[~bad].view(torch.int32), w0[~bad].view(torch.int32))
